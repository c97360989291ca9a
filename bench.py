"""Decode-step benchmark of libkvq on one MI355X.

One step = for every layer: quantize-on-write of each row's new token and
split-K paged decode attention over the whole cache, as one
kvq_write_decode call (``--separate``: kvq_write then kvq_paged_decode).
The cache is prefilled once, untimed; every step rewrites the same
position with the same token, so all steps do identical work.  The step is
captured once into a HIP graph and replayed (``--eager`` launches it from
Python instead).

Prints ONE JSON line: KV read GB/s of the step (algorithmic decode bytes /
step time) as ``value``, decode tokens/s, the decode launch's roofline
figures (per-launch algorithmic bytes / its HIP-event-timed duration, also
against the read rate a loads-only probe reaches, and the rocprofv3
durations of its decode and merge kernels when profiles/ holds them for
these sources), on KIVI caches the step that flushes a group, and the CPU
oracle's rate on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--eager]
                    [--no-cpu-baseline] [--no-probe] [--probe]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from quantized_paged_kv_02_amd import inputs, metrics  # noqa: E402
from quantized_paged_kv_02_amd.profile_summary import kernel_source_hash  # noqa: E402

METRIC = ("quantized paged-decode KV read GB/s (% of HBM peak) + decode tokens/s, 1 GPU")
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, vendor figure
# The KIVI-style INT4 shape (batch 16, 32/8 heads, 32768 tokens, 32 layers):
# the configuration the decode bandwidth target (>= 70 % of HBM peak) is set
# on.  Every other workload runs with --workload.
DEFAULT_WORKLOAD = "kivi-int4"
KIVI = ("int4", "int4-affine", "int2-affine")
PROBE_LIB = os.path.join(ROOT, "quantized_paged_kv_02_amd", "libkvq_probe.so")
TIMES_FILE = os.path.join(ROOT, "profiles", "decode_kernel_times.json")


def decode_kernel_label(dtype: str, n_query: int) -> str:
    """The kernels one decode launch runs, as rocprofv3 names them."""
    entry = "kvq_paged_decode_mq" if n_query else "kvq_paged_decode"
    kern = ("kvq_paged_decode_int4_kernel" if dtype in ("int4", "int4-affine", "int2-affine")
            else "kvq_paged_decode_kernel")
    return (f"{entry} launch: {kern} + kvq_partition_reduce_kernel (the reduce is skipped "
            "when one partition covers every row)")


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of (layer, row) units
# ---------------------------------------------------------------------------

def _cpu_unit(args):
    """Quantize one (layer, row) cache with the oracle (untimed), then time
    the oracle's decode step for it: the write (quantize the new token;
    INT4: the 64-token group that leaves the fp16 window) and the attention
    (dequantize the row's cache, fp64 attention for all query heads).
    Returns (write seconds, attention seconds)."""
    name, layer, row, seq = args
    from threadpoolctl import threadpool_limits
    import torch
    torch.set_num_threads(1)
    import oracle
    w = inputs.WORKLOADS[name]
    k, v = inputs.gen_kv(w, layer, row, seq, "cpu", 0)
    # bf16 inputs (a BF16 cache) as float32, exactly; numpy has no bf16
    k = k.float().numpy() if k.dtype == torch.bfloat16 else k.numpy()
    v = v.float().numpy() if v.dtype == torch.bfloat16 else v.numpy()
    q = inputs.gen_q(w, layer, "cpu", 0)[row].float().numpy().astype(np.float64)
    scale = 1.0 / math.sqrt(inputs.HEAD_DIM)
    with threadpool_limits(limits=1):
        if w.dtype in ("int4", "int4-affine", "int2-affine"):
            affine = w.dtype != "int4"
            bits = 2 if w.dtype == "int2-affine" else 4
            qmax = (1 << bits) - 1
            full = oracle.kivi_quantize(k, v, residual=w.residual_len, affine=affine, bits=bits)
            nq_old = oracle.kivi_quantized_len(seq - 1, w.residual_len)
            t0 = time.perf_counter()
            for g0 in range(nq_old, full["nq"], 64):
                for h in range(w.num_kv_heads):
                    if affine:
                        oracle.kivi_affine_quantize_k_group(k[g0:g0 + 64, h], qmax=qmax)
                        oracle.kivi_affine_quantize_v_tokens(v[g0:g0 + 64, h], qmax=qmax)
                    else:
                        oracle.kivi_quantize_k_group(k[g0:g0 + 64, h])
                        oracle.kivi_quantize_v_tokens(v[g0:g0 + 64, h])
            t1 = time.perf_counter()
            k_hat, v_hat = oracle.kivi_dequantize(full)
            oracle.decode_attention(q, k_hat, v_hat, scale)
            return t1 - t0, time.perf_counter() - t1
        if w.dtype in ("fp16", "bf16"):
            # unquantized cache: the new token is stored as is
            t0 = time.perf_counter()
            oracle.decode_attention(q, k, v, scale)
            return 0.0, time.perf_counter() - t0
        if w.k_gran == "token":
            kc, ks = oracle.quantize_per_token(k, w.dtype)
            vc, vs = oracle.quantize_per_token(v, w.dtype)
            t0 = time.perf_counter()
            oracle.quantize_per_token(k[seq - 1:], w.dtype)
            oracle.quantize_per_token(v[seq - 1:], w.dtype)
            t1 = time.perf_counter()
            k_hat = oracle.dequantize(kc, ks[..., None], w.dtype)
            v_hat = oracle.dequantize(vc, vs[..., None], w.dtype)
        else:
            sk = oracle.calibrate_scales(k[:seq - 1], w.k_gran, w.dtype)
            sv = oracle.calibrate_scales(v[:seq - 1], w.v_gran, w.dtype)
            kc = oracle.quantize_static(k, sk, w.k_gran, w.dtype)
            vc = oracle.quantize_static(v, sv, w.v_gran, w.dtype)
            shp = (1, 1, 1) if w.k_gran == "tensor" else (1, -1, 1)
            t0 = time.perf_counter()
            oracle.quantize_static(k[seq - 1:], sk, w.k_gran, w.dtype)
            oracle.quantize_static(v[seq - 1:], sv, w.v_gran, w.dtype)
            t1 = time.perf_counter()
            k_hat = oracle.dequantize(kc, sk.reshape(shp), w.dtype)
            v_hat = oracle.dequantize(vc, sv.reshape(shp), w.dtype)
        oracle.decode_attention(q, k_hat, v_hat, scale)
        return t1 - t0, time.perf_counter() - t1


def _host_cpu():
    """(logical CPUs of the host, CPUs this process may run on, CPU model)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        allowed = len(os.sched_getaffinity(0))
    except AttributeError:
        allowed = os.cpu_count() or 1
    return os.cpu_count() or 1, allowed, model


def cpu_baseline(w, lens, workers: int, target_cpu_s: float = 20.0):
    """Time the oracle over a bounded sample of (layer, row) units: first
    one unit alone in one process (the single-thread figure), then units on
    ``workers`` host processes at once (one BLAS thread each) until about
    ``target_cpu_s`` seconds of CPU work (never more than the whole step).
    Write (quantize the new token) and attention are timed separately."""
    import concurrent.futures as cf
    import multiprocessing as mp
    all_units = [(w.name, layer, row, int(lens[row]))
                 for layer in range(w.layers) for row in range(w.batch)]
    ctx = mp.get_context("spawn")

    def unit_bytes(units):
        return sum(metrics.decode_bytes(w.dtype, w.k_gran, w.v_gran, [u[3]], w.num_q_heads,
                                        w.num_kv_heads, w.residual_len) for u in units)

    # single thread: one process, nothing else running
    with cf.ProcessPoolExecutor(max_workers=1, mp_context=ctx) as ex:
        tw1, ta1 = ex.submit(_cpu_unit, all_units[-1]).result()
    single = {"GBps": round(unit_bytes(all_units[-1:]) / (tw1 + ta1) / 1e9, 4),
              "tokens_per_s": round(1.0 / ((tw1 + ta1) * w.layers), 4),
              "write_s": round(tw1, 5), "attention_s": round(ta1, 4),
              "note": "one (layer, row) unit in one process; tokens/s for one row "
                      "through all layers"}
    with cf.ProcessPoolExecutor(max_workers=workers, mp_context=ctx) as ex:
        first = all_units[:min(workers, len(all_units))]
        secs = list(ex.map(_cpu_unit, first))
        per_unit = sum(a + b for a, b in secs) / len(secs)
        more = int(max(0.0, target_cpu_s - sum(a + b for a, b in secs)) / max(per_unit, 1e-6))
        rest = all_units[len(first):len(first) + more]
        if rest:
            secs += list(ex.map(_cpu_unit, rest))
    units = all_units[:len(secs)]
    n = len(units)
    cores = min(workers, n)
    tw = sum(a for a, _ in secs)
    ta = sum(b for _, b in secs)
    # units ran concurrently on `cores` processes
    wall = (tw + ta) / cores
    gbs = unit_bytes(units) / wall / 1e9
    step_s = (tw + ta) / n * w.layers * w.batch / cores
    nproc, allowed, model = _host_cpu()
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "tokens_per_s": round(w.batch / step_s, 4),
            "write_s_per_unit": round(tw / n, 5), "attention_s_per_unit": round(ta / n, 4),
            "single_thread": single, "nproc": nproc, "cpus_allowed": allowed,
            "cpu_model": model,
            "sample": (f"{n} of {len(all_units)} (layer, row) units of {w.name}; each: "
                       f"quantize the new token (write), dequantize the row's cache and fp64 "
                       f"attention (attention); numpy oracle, 1 BLAS thread per process, "
                       f"{cores} processes at once (a 16-CPU share of the host's "
                       f"{nproc} logical CPUs); {tw + ta:.1f} s of CPU work; K/V drawn on "
                       f"the CPU by the same recipe")}


# ---------------------------------------------------------------------------
# Achievable read bandwidth: the probe of libkvq_probe.so
# ---------------------------------------------------------------------------

def bandwidth_probe(gib: float = 4, reps: int = 5, grids=(128, 256, 512, 1024, 2048),
                    threads: int = 256, orders=(0, 1)):
    """Read ``gib`` GiB (a power of two) per launch in 1 KiB chunks (one
    16-byte buffer load per lane, the decode's granule and cache policy)
    with several grid sizes, in wavefront-strided and in scattered chunk
    order; each configuration is launched back to back ``reps`` times
    between one HIP event pair, each launch on another slice of a buffer of
    at least 2 GiB (so a launch smaller than the 256 MB Infinity Cache does
    not read what the previous one left there, as the decode's layers do
    not).  Returns the best rate (GB/s, 1e9 bytes) and every
    configuration's."""
    import ctypes
    import torch
    if not os.path.exists(PROBE_LIB):
        raise SystemExit(f"{PROBE_LIB} is missing: build it with "
                         "`python -m quantized_paged_kv_02_amd.build`")
    lib = ctypes.CDLL(PROBE_LIB)
    lib.kvq_probe_read.restype = ctypes.c_int
    lib.kvq_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    nbytes = int(gib * (1 << 30))
    slices = max(1, (2 << 30) // nbytes)
    reps = max(reps, min(slices, 64))
    buf = torch.empty(nbytes * slices, dtype=torch.uint8, device="cuda")
    buf.fill_(0x5A)          # every dword xors to 0: the sink is never written
    sink = torch.zeros(max(grids), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)

    def launch(wgs, order, i=0):
        rc = lib.kvq_probe_read(buf.data_ptr() + (i % slices) * nbytes, nbytes, wgs, threads,
                                order, sink.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise SystemExit(f"kvq_probe_read failed ({rc})")

    rows = []
    for order, name in ((0, "strided"), (1, "scattered")):
        if order not in orders:
            continue
        for wgs in grids:
            launch(wgs, order, reps - 1)
            e0.record()
            for i in range(reps):
                launch(wgs, order, i)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            rows.append({"order": name, "workgroups": wgs, "threads": threads,
                         "us": round(ms * 1e3, 1),
                         "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1)})
    del buf
    best = max(rows, key=lambda r: r["GBps"])
    return {"GBps": best["GBps"], "best": best, "bytes_per_launch": nbytes, "slices": slices,
            "chunk_bytes": 1024, "all": rows,
            "kernel": "kvq_probe_read_kernel (libkvq_probe.so): loads only, 8 chunks in "
                      "flight per wavefront"}


def write_probe(read_bytes: int, reps: int = 5, grids=(256, 512, 1024, 2048, 4096),
                threads: int = 256):
    """The read-and-write probe of libkvq_probe.so: read ``read_bytes`` (a
    power of two) in 1 KiB chunks and write half as many bytes in 512-byte
    runs, the bulk write's 2 : 1 mix of fp16 in and one-byte codes out, at
    several grid sizes, each launch on fresh source and destination slices.
    Returns the best rate over the bytes read plus written (GB/s)."""
    import ctypes
    import torch
    if not os.path.exists(PROBE_LIB):
        raise SystemExit(f"{PROBE_LIB} is missing: build it with "
                         "`python -m quantized_paged_kv_02_amd.build`")
    lib = ctypes.CDLL(PROBE_LIB)
    lib.kvq_probe_rw.restype = ctypes.c_int
    lib.kvq_probe_rw.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                 ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    slices = max(2, (2 << 30) // read_bytes)
    src = torch.empty(read_bytes * slices, dtype=torch.uint8, device="cuda")
    dst = torch.empty(read_bytes // 2 * slices, dtype=torch.uint8, device="cuda")
    src.fill_(0x3C)
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)

    def launch(wgs, i):
        rc = lib.kvq_probe_rw(src.data_ptr() + (i % slices) * read_bytes, read_bytes,
                              dst.data_ptr() + (i % slices) * (read_bytes // 2), wgs, threads,
                              stream.cuda_stream)
        if rc != 0:
            raise SystemExit(f"kvq_probe_rw failed ({rc})")

    rows = []
    for wgs in grids:
        launch(wgs, reps - 1)
        e0.record()
        for i in range(reps):
            launch(wgs, i)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        moved = read_bytes + read_bytes // 2
        rows.append({"workgroups": wgs, "threads": threads, "us": round(ms * 1e3, 1),
                     "GBps": round(moved / (ms * 1e-3) / 1e9, 1)})
    del src, dst
    best = max(rows, key=lambda r: r["GBps"])
    return {"GBps": best["GBps"], "frac_of_peak": round(best["GBps"] / HBM_PEAK_GBS, 4),
            "bytes_read": read_bytes, "bytes_written": read_bytes // 2, "best": best,
            "all": rows,
            "kernel": "kvq_probe_rw_kernel (libkvq_probe.so): 16-byte loads, 8-byte "
                      "stores, 8 chunks in flight per wavefront"}


def launch_floor(layer_bytes: int):
    """The loads-only probe at the size of one decode launch (the largest
    power of two not above its bytes, fresh data each launch): how long a
    kernel that only reads that much takes, the floor of the launch."""
    p2 = 1 << (int(layer_bytes).bit_length() - 1)
    if p2 < (1 << 20) or p2 > (1 << 30):
        return None
    r = bandwidth_probe(p2 / (1 << 30), reps=32)
    best = r["best"]
    return {"bytes": p2, "us": best["us"], "GBps": best["GBps"],
            "frac_of_peak": round(best["GBps"] / HBM_PEAK_GBS, 4),
            "launch_floor_us": round(layer_bytes / (best["GBps"] * 1e9) * 1e6, 2),
            "config": {k: best[k] for k in ("order", "workgroups", "threads")}}


# ---------------------------------------------------------------------------
# GPU setup
# ---------------------------------------------------------------------------

class Bench:
    def __init__(self, w: inputs.Workload, device="cuda", n_query: int = 0,
                 partition: str = "auto", with_probe: bool = True, prefill_calls: int = 10,
                 prefill_warm: int = 30):
        import torch
        from quantized_paged_kv_02_amd import kvq
        self.torch, self.kvq, self.w = torch, kvq, w
        self.n_query = n_query
        lens = inputs.seq_lens(w)
        self.lens = lens
        table, nb = inputs.block_tables(w, lens)
        self.table = torch.as_tensor(table, device=device)
        self.lens_t = torch.as_tensor(lens, device=device)
        self.max_len = int(lens.max())
        self.layout = kvq.make_layout(w.dtype, w.k_gran, w.v_gran, w.num_q_heads,
                                      w.num_kv_heads, nb, table.shape[1], 0, w.residual_len)
        # the partition length for the rows' real lengths (known here, as
        # in a serving scheduler); several queries per row take the automatic
        # plan, which counts the queries
        if not n_query:
            self.layout.split_tokens = kvq.plan_split_tokens(self.layout, lens)
        if partition == "auto":
            self.layout.partition = kvq.plan_partition(self.layout, lens)
        else:
            self.layout.partition = kvq.PARTITIONS[partition]
        b = w.batch
        self.calibrate = None
        self.prefill_write = None
        self.ones_cu = torch.arange(b + 1, dtype=torch.int32, device=device)
        self.caches, self.k_new, self.v_new, self.q, self.out = [], [], [], [], []
        self.k_prev, self.v_prev = [], []
        for layer in range(w.layers):
            kk, vv = [], []
            for r in range(b):
                k, v = inputs.gen_kv(w, layer, r, int(lens[r]), device, 0)
                kk.append(k)
                vv.append(v)
            pre_k = [k[:-1] for k in kk]
            pre_v = [v[:-1] for v in vv]
            cache = kvq.alloc_cache(self.layout, ring_rows=b, device=device)
            # static scales calibrated by the library from the prefill tokens
            static = ("tensor", "head", "channel")
            if w.dtype in ("int8", "fp8", "fp8e5m2") and (w.k_gran in static or
                                                          w.v_gran in static):
                ks_ok, vs_ok = w.k_gran in static, w.v_gran in static
                ck = torch.cat(pre_k) if ks_ok else None
                cv = torch.cat(pre_v) if vs_ok else None
                cks = cache.k_scales if ks_ok else None
                cvs = cache.v_scales if vs_ok else None
                kvq.calibrate(self.layout, ck, cv, cks, cvs)
                if layer == 0:
                    # time the calibration of one layer's prefill: repeated
                    # accumulating calls leave the scales as they are
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record()
                    for _ in range(3):
                        kvq.calibrate(self.layout, ck, cv, cks, cvs, accumulate=True)
                    e1.record()
                    torch.cuda.synchronize()
                    n_tok = int((ck if ck is not None else cv).shape[0])
                    nbytes = n_tok * w.num_kv_heads * 128 * 2 * (int(ks_ok) + int(vs_ok))
                    us = e0.elapsed_time(e1) * 1e3 / 3
                    self.calibrate = {
                        "call": "kvq_calibrate of one layer's prefill K/V", "tokens": n_tok,
                        "bytes_read": nbytes, "us": round(us, 2),
                        "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                        "frac_of_hbm_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
                del ck, cv
            n = (lens - 1).astype(np.int32)
            cu = torch.as_tensor(np.concatenate([[0], np.cumsum(n)]).astype(np.int32),
                                 device=device)
            kpre, vpre = torch.cat(pre_k).contiguous(), torch.cat(pre_v).contiguous()
            n_t = torch.as_tensor(n, device=device)
            kvq.write(cache, kpre, vpre, cu, self.table, n_t, int(n.max()))
            if layer == 0:
                # time the prefill write of one layer: rewriting the same
                # tokens stores the same codes, scales and ring values.  Every
                # kernel of the call is timed (a KIVI write is the flush and
                # the fp16-window append).  The engine clock dips for a few
                # milliseconds once back-to-back write kernels start (to ~1.6
                # GHz around the 3rd-10th call, back above 2 GHz by the
                # 20th), so prefill_warm untimed calls come first, then
                # prefill_calls timed back to back, each between its own
                # events; us is their median
                for _ in range(prefill_warm):
                    kvq.write(cache, kpre, vpre, cu, self.table, n_t, int(n.max()))
                ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                      for _ in range(max(1, prefill_calls))]
                for e0, e1 in ev:
                    e0.record()
                    kvq.write(cache, kpre, vpre, cu, self.table, n_t, int(n.max()))
                    e1.record()
                torch.cuda.synchronize()
                calls = [e0.elapsed_time(e1) * 1e3 for e0, e1 in ev]
                us = float(np.median(calls))
                us_mean = float(np.mean(calls))
                if w.dtype in KIVI:
                    nbytes = metrics.kivi_write_bytes(w.dtype, n, w.num_kv_heads, w.residual_len)
                else:
                    nbytes = metrics.write_bytes(w.dtype, w.k_gran, w.v_gran, int(n.sum()),
                                                 w.num_kv_heads)
                self.prefill_write = {
                    "call": "kvq_write of one layer's prefill (S - 1 tokens per row): median "
                            "of back-to-back calls after untimed ones",
                    "warm_calls": prefill_warm,
                    "tokens": int(n.sum()), "bytes": nbytes, "us": round(us, 2),
                    "us_mean": round(us_mean, 2), "calls": len(calls),
                    "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                    "frac_of_hbm_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
                if with_probe:
                    # the read-and-write probe at the prefill's read size
                    # (largest power of two): the achievable 2 : 1 rate
                    rd = int(n.sum()) * w.num_kv_heads * 128 * 2 * 2
                    p2 = 1 << (rd.bit_length() - 1)
                    if (1 << 20) <= p2 <= (1 << 30):
                        wp = write_probe(p2)
                        self.prefill_write["write_probe_GBps"] = wp["GBps"]
                        self.prefill_write["frac_of_write_probe"] = round(
                            nbytes / (us * 1e-6) / 1e9 / wp["GBps"], 4)
            del kpre, vpre
            self.caches.append(cache)
            nq = max(n_query, 1)   # new tokens per row and step
            self.k_new.append(torch.cat([k[-nq:] for k in kk]).contiguous())
            self.v_new.append(torch.cat([v[-nq:] for v in vv]).contiguous())
            if not n_query and w.dtype in KIVI and int(lens.min()) >= 2:
                # the token before the last: a step at length S - 1 rewrites
                # it (the same values the prefill stored) and flushes the
                # group that leaves the fp16 window at S
                self.k_prev.append(torch.cat([k[-2:-1] for k in kk]).contiguous())
                self.v_prev.append(torch.cat([v[-2:-1] for v in vv]).contiguous())
            if n_query:
                self.q.append(inputs.gen_q(w, layer, device, 0, batch=b * n_query).reshape(
                    b, n_query, w.num_q_heads, 128).contiguous())
                self.out.append(torch.empty((b, n_query, w.num_q_heads, 128),
                                            dtype=torch.float32, device=device))
            else:
                self.q.append(inputs.gen_q(w, layer, device, 0))
                self.out.append(torch.empty((b, w.num_q_heads, 128), dtype=torch.float32,
                                            device=device))
            del kk, vv, pre_k, pre_v
        if n_query:
            self.cu_nq = torch.arange(b + 1, dtype=torch.int32, device=device) * n_query
            nbytes = kvq.paged_decode_mq_workspace_bytes(self.layout, n_query, b, self.max_len)
            self.ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        else:
            self.ws = kvq.alloc_workspace(self.layout, b, self.max_len, device)
        self.scale = 1.0 / math.sqrt(128)
        if self.k_prev:
            self.lens_prev_t = torch.as_tensor(lens - 1, device=device)
            self.out_prev = [torch.empty_like(o) for o in self.out]
        torch.cuda.synchronize()

    def flush_step(self):
        """A KIVI decode step at length S - 1 over all layers
        (kvq_write_decode): it rewrites token S - 2 with the values the
        prefill stored and flushes the group [nq(S) - 64, nq(S)) that leaves
        the fp16 window at S, which the prefill already flushed with the same
        codes, so the cache is unchanged.  Every 64th step of a row flushes
        so; the other steps are the plain step."""
        for layer in range(self.w.layers):
            self.kvq.write_decode(self.caches[layer], self.k_prev[layer], self.v_prev[layer],
                                  self.q[layer], self.table, self.lens_prev_t,
                                  self.max_len - 1, self.scale, self.out_prev[layer], self.ws)

    def step(self, write=True, fused=True):
        """One decode step over all layers: append each row's new token and
        decode.  fused: one kvq_write_decode call per layer, else kvq_write
        then kvq_paged_decode; write=False: the decode launches alone."""
        kvq = self.kvq
        if self.n_query:
            # several query tokens per row: rewrite the rows' last n_query
            # tokens (the draft tokens' K/V), then attend with all of them
            for layer in range(self.w.layers):
                if write:
                    kvq.write(self.caches[layer], self.k_new[layer], self.v_new[layer],
                              self.cu_nq, self.table, self.lens_t, self.n_query)
                kvq.paged_decode_mq(self.caches[layer], self.q[layer], self.table, self.lens_t,
                                    self.max_len, self.scale, self.out[layer], self.ws)
            return
        for layer in range(self.w.layers):
            if write and fused:
                kvq.write_decode(self.caches[layer], self.k_new[layer], self.v_new[layer],
                                 self.q[layer], self.table, self.lens_t, self.max_len,
                                 self.scale, self.out[layer], self.ws)
                continue
            if write:
                kvq.write(self.caches[layer], self.k_new[layer], self.v_new[layer],
                          self.ones_cu, self.table, self.lens_t, 1)
            kvq.paged_decode(self.caches[layer], self.q[layer], self.table, self.lens_t,
                             self.max_len, self.scale, self.out[layer], self.ws)


def run(args):
    import torch
    w = inputs.WORKLOADS[args.workload]
    cpu = None
    if not args.no_cpu_baseline:
        # before the GPU is touched: the oracle runs in fresh worker processes
        cpu = cpu_baseline(w, inputs.seq_lens(w), workers=args.cpu_workers)
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU (torch.cuda.is_available() is False)")
    bench = Bench(w, n_query=args.n_query, partition=args.partition,
                  with_probe=not args.no_probe, prefill_calls=args.prefill_calls,
                  prefill_warm=args.prefill_warm)
    b = w.batch
    L = w.layers
    layer_bytes = metrics.decode_bytes(w.dtype, w.k_gran, w.v_gran, bench.lens,
                                       w.num_q_heads, w.num_kv_heads, w.residual_len)
    step_bytes = layer_bytes * L

    # eager reference pass, then the graph
    fused = not args.separate
    bench.step(fused=fused)
    torch.cuda.synchronize()
    ref = [o.clone() for o in bench.out]
    graph = None
    if not args.eager:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            bench.step(fused=fused)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            bench.step(fused=fused)
        torch.cuda.synchronize()

    def one():
        if graph is not None:
            graph.replay()
        else:
            bench.step(fused=fused)

    for _ in range(args.warmup):
        one()
    torch.cuda.synchronize()
    for o, r in zip(bench.out, ref):
        if not torch.equal(o, r):
            raise SystemExit("replayed step output differs from the eager step")

    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        one()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps

    # KIVI: the step that flushes a group (one in 64), timed the same way
    flush = None
    if bench.k_prev and not args.separate:
        fgraph = None
        if not args.eager:
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                bench.flush_step()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            fgraph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(fgraph):
                bench.flush_step()
        for _ in range(max(args.warmup, 1)):
            fgraph.replay() if fgraph is not None else bench.flush_step()
        torch.cuda.synchronize()
        start.record()
        for _ in range(args.steps):
            fgraph.replay() if fgraph is not None else bench.flush_step()
        stop.record()
        torch.cuda.synchronize()
        fms = start.elapsed_time(stop) / args.steps
        # the flush step attends over S - 1 tokens (other outputs) and leaves
        # the cache as it was: the plain step still gives the reference outputs
        if any(torch.equal(a, b) for a, b in zip(bench.out_prev, ref)):
            raise SystemExit("the flush step gave the plain step's outputs")
        one()
        torch.cuda.synchronize()
        for o, r in zip(bench.out, ref):
            if not torch.equal(o, r):
                raise SystemExit("the flush step changed the cache")
        flush = {"length": int(bench.max_len) - 1, "ms_per_step": round(fms, 5),
                 "cycle_ms_per_step": round((63 * ms + fms) / 64, 5),
                 "note": "kvq_write_decode at length S - 1 flushes the 64-token group "
                         "leaving the fp16 window (one step in 64 does); cycle = 63 plain "
                         "steps and one flush step, averaged"}

    # Decode-launch duration: one HIP event pair, on the stream the launches
    # run on, around the L decode launches of a step (one per layer, back to
    # back, the write launches left out), elapsed / L.  They run as the timed
    # step runs them: from a HIP graph of those launches (eagerly with
    # --eager, each queued behind a spin kernel so no host latency falls
    # inside).  No marker sits between launches.
    dgraph = None
    if not args.eager:
        dgraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(dgraph):
            bench.step(write=False)
        dgraph.replay()
        torch.cuda.synchronize()
    k0 = torch.cuda.Event(enable_timing=True)
    k1 = torch.cuda.Event(enable_timing=True)
    durs = []
    for _ in range(max(1, args.kernel_samples)):
        if dgraph is not None:
            # an untimed replay first: the timed one is queued while it runs,
            # and the GPU is as busy as in the timed steps when it starts
            dgraph.replay()
            k0.record()
            dgraph.replay()
        else:
            torch.cuda._sleep(int(2e7))
            k0.record()
            bench.step(write=False)
        k1.record()
        torch.cuda.synchronize()
        durs.append(k0.elapsed_time(k1) / L)
    kernel_timing = ("HIP events around the step's decode launches (one per layer, back to "
                     "back, " + ("launched eagerly behind a spin kernel" if dgraph is None
                                 else "replayed from a HIP graph") + "), elapsed / launches")
    kern_ms = float(np.mean(durs))

    copy_probe = None
    if args.copy_probe_mib > 0:
        # a plain device-to-device copy of known size: the yardstick that
        # converts profiler byte counters into bytes
        nbytes = args.copy_probe_mib << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        dst.copy_(src)
        torch.cuda.synchronize()
        c0.record()
        for _ in range(3):
            dst.copy_(src)
        c1.record()
        torch.cuda.synchronize()
        cms = c0.elapsed_time(c1) / 3
        copy_probe = {"bytes_read": nbytes, "bytes_written": nbytes, "ms": round(cms, 4),
                      "GBps_read_plus_write": round(2 * nbytes / (cms * 1e-3) / 1e9, 1)}
        del src, dst
    achieved = layer_bytes / (kern_ms * 1e-3) / 1e9
    probe = None if args.no_probe else bandwidth_probe(args.probe_gib)
    floor = None if args.no_probe else launch_floor(layer_bytes)

    part_name = "balanced" if bench.layout.partition else "per-row"
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        ent = t.get(w.name) if not args.n_query else None   # decode launches only
        # counters taken with other kernels or another partition length
        # describe other launches
        if (ent and t.get("kernel_source_hash") == kernel_source_hash()
                and ent.get("split_tokens") == int(bench.layout.split_tokens)
                and ent.get("partition", "per-row") == part_name):
            traffic = ent.get("bytes_per_launch")

    # rocprofv3 durations of this workload's decode and merge kernels
    # (profiles/, taken under the same kernel sources and partition length)
    profiled = None
    if os.path.exists(TIMES_FILE) and not args.n_query:
        with open(TIMES_FILE) as f:
            t = json.load(f)
        ent = t.get(w.name)
        if (ent and t.get("kernel_source_hash") == kernel_source_hash()
                and ent.get("split_tokens") == int(bench.layout.split_tokens)
                and ent.get("partition", "per-row") == part_name):
            dec, mer = ent["decode_us"], ent.get("merge_us", 0.0)
            profiled = {"decode_us": dec, "merge_us": mer,
                        "frac_decode": round(layer_bytes / (dec * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                        "frac_decode_plus_merge": round(
                            layer_bytes / ((dec + mer) * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                        "launch_span_us": ent.get("launch_span_us"),
                        "source": os.path.relpath(TIMES_FILE, ROOT),
                        "command": ent.get("command")}

    step_gbs = step_bytes / (ms * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(step_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the matrix products' operand type (fp32 accumulation and softmax)
        "dtype": "bf16" if w.dtype == "bf16" else "f16",
        "data": "synthetic",
        "tokens_per_s": round(b * max(args.n_query, 1) / (ms * 1e-3), 2),
        "hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4),
        "config": {
            "workload": w.name, "description": w.description, "layers": L, "batch": b,
            "seq_len": int(w.max_seq) if not isinstance(w.seq, tuple) else list(w.seq),
            "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
            "kv_dtype": w.dtype, "k_granularity": w.k_gran, "v_granularity": w.v_gran,
            "block_tables": w.table, "n_query": max(args.n_query, 1),
            "step": (f"per layer: kvq_write of the last {args.n_query} tokens/row + "
                     f"kvq_paged_decode_mq ({args.n_query} causal queries/row)" if args.n_query
                     else "per layer: kvq_write of 1 token/row + kvq_paged_decode"
                     if args.separate
                     else "per layer: kvq_write_decode (1 token/row appended, then decoded)"),
            "launch": "hip graph" if graph is not None else "eager",
            "split_tokens": int(bench.layout.split_tokens),
            "partition": "balanced" if bench.layout.partition else "per-row",
            "algorithmic_bytes_per_step": step_bytes,
        },
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": decode_kernel_label(w.dtype, args.n_query),
            "bytes_per_launch": layer_bytes,
            "avg_launch_us": round(kern_ms * 1e3, 3), "launches_timed": len(durs) * L,
            "timing": kernel_timing,
            "probe_GBps": probe["GBps"] if probe else None,
            "frac_of_probe": round(achieved / probe["GBps"], 4) if probe else None,
            "launch_size_probe": floor,
            "profiled": profiled,
        },
        "cpu_baseline": cpu,
    }
    if copy_probe is not None:
        result["copy_probe"] = copy_probe
    if probe is not None:
        result["probe"] = probe
    if flush is not None:
        result["flush_step"] = flush
    if bench.calibrate is not None:
        result["calibrate"] = bench.calibrate
    if bench.prefill_write is not None:
        result["prefill_write"] = bench.prefill_write
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(inputs.WORKLOADS))
    ap.add_argument("--eager", action="store_true", help="launch from Python, no HIP graph")
    ap.add_argument("--separate", action="store_true",
                    help="step with kvq_write + kvq_paged_decode instead of kvq_write_decode")
    ap.add_argument("--n-query", type=int, default=0,
                    help="query tokens per row and step (kvq_paged_decode_mq); 0: decode")
    ap.add_argument("--kernel-samples", type=int, default=10,
                    help="extra synchronised replays for the per-launch timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-calls", type=int, default=10,
                    help="back-to-back prefill writes timed for prefill_write")
    ap.add_argument("--prefill-warm", type=int, default=30,
                    help="untimed back-to-back prefill writes before them")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also time a device copy of this many MiB (profiler yardstick)")
    ap.add_argument("--cpu-workers", type=int, default=min(16, os.cpu_count() or 1),
                    help="oracle processes (default: 16, the host CPU share a GPU job gets)")
    ap.add_argument("--partition", default="auto", choices=["auto", "per-row", "balanced"],
                    help="decode partitions: the host plan's choice (auto) or a forced mode")
    ap.add_argument("--no-probe", action="store_true",
                    help="skip the read-bandwidth probe")
    ap.add_argument("--probe-gib", type=float, default=4,
                    help="bytes the bandwidth probe reads per launch (GiB, a power of two)")
    ap.add_argument("--probe-threads", type=int, default=256,
                    help="threads per workgroup of the probe (--probe)")
    ap.add_argument("--probe", action="store_true",
                    help="run only the read-bandwidth probe and print its JSON")
    ap.add_argument("--probe-grids", default="",
                    help="workgroup counts of the probe (--probe), comma-separated")
    ap.add_argument("--probe-order", default="both", choices=["strided", "scattered", "both"],
                    help="chunk order of the probe (--probe)")
    ap.add_argument("--probe-reps", type=int, default=5,
                    help="launches per probe configuration (--probe; at least the buffer's "
                         "slices)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the decode "
              "path has no multi-GPU mode in this library", file=sys.stderr)
        raise SystemExit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs as a single process on one GPU", file=sys.stderr)
        raise SystemExit(2)
    if args.probe:
        grids = tuple(int(g) for g in args.probe_grids.split(",")) if args.probe_grids else (
            128, 256, 512, 1024, 2048)
        orders = {"strided": (0,), "scattered": (1,), "both": (0, 1)}[args.probe_order]
        print(json.dumps(bandwidth_probe(args.probe_gib, reps=args.probe_reps, grids=grids,
                                         threads=args.probe_threads, orders=orders)),
              flush=True)
        return
    run(args)


if __name__ == "__main__":
    main()
