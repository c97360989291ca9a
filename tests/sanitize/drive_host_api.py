"""Valid calls of every host entry point of libkvq against the host-only
stub build (tests/sanitize/host_stubs.cpp), run under AddressSanitizer and
UndefinedBehaviorSanitizer by tests/test_host_sanitized.py.

Pointers are fake aligned addresses: the stub launchers check the argument
blocks the API built and launch nothing.  Refuses to run against a library
without the stub marker.

    python tests/sanitize/drive_host_api.py LIB.so
"""

import ctypes
import itertools
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from quantized_paged_kv_02_amd import kvq  # noqa: E402

FAKE = 0x100000   # 256-byte aligned, never dereferenced by the stubs


def main(path):
    lib = kvq._load(path, strict=False)
    if not hasattr(lib, "kvq_host_stub_build"):
        raise SystemExit(f"{path} is not the host stub build; refusing to pass fake pointers")
    calls = 0
    rng = np.random.default_rng(0)
    formats = [("int8", "token", "token"), ("int8", "channel", "head"), ("fp8", "tensor", "tensor"),
               ("fp8", "head", "token"), ("fp8e5m2", "channel", "channel"), ("fp16", "none", "none"),
               ("int4", "channel", "token"), ("int4-affine", "channel", "token"),
               ("int2-affine", "channel", "token")]
    for (dt, kg, vg), (hq, hkv), batch, max_len, split, part in itertools.product(
            formats, [(8, 8), (32, 8), (64, 8), (4, 4)], [1, 3, 64, 256], [1, 17, 2048, 32768],
            [0, 64, 4096], ["per-row", "balanced"]):
        kivi = dt in ("int4", "int4-affine", "int2-affine")
        if kivi and (part == "balanced" or (dt == "int2-affine" and hq // hkv > 4)):
            continue
        mbs = (max_len + 15) // 16
        lay = kvq.make_layout(dt, kg, vg, hq, hkv, batch * mbs, mbs, split, partition=part)
        cache = kvq.Cache(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, batch)
        assert lib.kvq_validate(ctypes.byref(lay), ctypes.byref(cache), batch, max_len) == 0
        ws = lib.kvq_decode_workspace_bytes(ctypes.byref(lay), batch, max_len)
        st = lib.kvq_paged_decode(ctypes.byref(lay), ctypes.byref(cache), FAKE, FAKE, FAKE, batch,
                                  max_len, 0.1, FAKE, FAKE if ws else None, ws, None)
        assert st == 0, (dt, kg, vg, hq, hkv, batch, max_len, split, part, st)
        st = lib.kvq_write_decode(ctypes.byref(lay), ctypes.byref(cache), FAKE, FAKE, FAKE, FAKE,
                                  FAKE, batch, max_len, 0.1, FAKE, FAKE if ws else None, ws, None)
        assert st == 0, ("write_decode", dt, batch, max_len, split, part, st)
        nq = 2 if (hq // hkv) * 2 <= 16 and dt != "int2-affine" else 1
        wq = lib.kvq_paged_decode_mq_workspace_bytes(ctypes.byref(lay), nq, batch, max_len)
        st = lib.kvq_paged_decode_mq(ctypes.byref(lay), ctypes.byref(cache), FAKE, nq, FAKE, FAKE,
                                     batch, max_len, 0.1, FAKE, FAKE if wq else None, wq, None)
        assert st == 0, ("mq", dt, batch, max_len, split, part, st)
        st = lib.kvq_write(ctypes.byref(lay), ctypes.byref(cache), FAKE, FAKE, FAKE, FAKE, FAKE,
                           batch, batch * max_len, max_len, None)
        assert st == 0, ("write", dt, batch, max_len, st)
        if dt in ("int8", "fp8", "fp8e5m2"):
            n_tok = batch * max_len
            cw = lib.kvq_calibrate_workspace_bytes(ctypes.byref(lay), n_tok)
            st = lib.kvq_calibrate(ctypes.byref(lay), FAKE, FAKE, n_tok, FAKE, FAKE, 1, FAKE, cw,
                                   None)
            assert st == 0, ("calibrate", dt, st)
        # host plans and the table checker on host arrays
        lens = rng.integers(0, max_len + 1, size=batch).astype(np.int32)
        lens[0] = max_len
        split_t = lib.kvq_plan_split_tokens(ctypes.byref(lay), lens.ctypes.data, batch)
        assert split_t > 0
        pm = lib.kvq_plan_partition(ctypes.byref(lay), lens.ctypes.data, batch)
        assert pm in (0, 1)
        table = (np.arange(batch)[:, None] * mbs + np.arange(mbs)[None]).astype(np.int32)
        bad = ctypes.c_int32(7)
        assert lib.kvq_check_tables(ctypes.byref(lay), table.ctypes.data, lens.ctypes.data, batch,
                                    max_len, ctypes.byref(bad)) == 0 and bad.value == -1
        calls += 9
    print(f"{calls} valid host calls through the stub launchers")


if __name__ == "__main__":
    main(sys.argv[1])
