"""Shared driver for the GPU parity tests: build a cache through the C ABI,
run one decode step, read everything back and compare with the oracle.

Only the tests import this.  Inputs come from quantized_paged_kv_02_amd.inputs
(seeded); expected values come from ``oracle`` alone.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

import oracle
from quantized_paged_kv_02_amd import inputs
from tests import layout_view as lv

ATOL = 2e-3
RTOL = 1e-2
KIVI = ("int4", "int4-affine", "int2-affine")   # KIVI-grouped caches


@dataclass
class CaseResult:
    w: inputs.Workload
    lens: np.ndarray
    table: np.ndarray
    k: list            # per row fp16 [S, H, 128] (host numpy)
    v: list
    q: np.ndarray      # [B, Hq, 128] fp16
    out: np.ndarray    # [B, Hq, 128] fp32
    pools: dict        # host copies of the cache tensors
    k_static: np.ndarray | None
    v_static: np.ndarray | None
    softmax_scale: float


def _np(t):
    """A tensor on the host as numpy; bf16 (which numpy lacks) as float32,
    an exact conversion."""
    t = t.cpu()
    return t.float().numpy() if t.dtype == torch.bfloat16 else t.numpy()


def _static(w, gran, tensors, dtype):
    """Static scales from the rows' prefill tokens, by the oracle's
    calibration (rows folded in one at a time)."""
    if dtype in ("fp16", "bf16") or gran not in ("tensor", "head", "channel"):
        return None
    s = None
    for t in tensors:
        s = oracle.calibrate_scales(t.cpu().numpy(), gran, dtype, previous=s)
    return s


def fill_garbage(cache):
    """Poison every pool byte so reads of unwritten slots would show."""
    if cache.layout.dtype in (4, 8):   # FP16 / BF16 values
        cache.k_codes.fill_(float("nan"))
        cache.v_codes.fill_(float("nan"))
        return
    cache.k_codes.fill_(0x7F)          # E4M3 NaN pattern
    cache.v_codes.fill_(0xFF)
    if cache.k_resid is not None:
        cache.k_resid.fill_(float("nan"))
        cache.v_resid.fill_(float("nan"))
    int4 = cache.layout.dtype in (3, 5, 7)
    if int4 or cache.layout.k_gran == 3:
        cache.k_scales.fill_(float("nan"))
    if int4 or cache.layout.v_gran == 3:
        cache.v_scales.fill_(float("nan"))


def run_case(w: inputs.Workload, lens, seed=0, layer=0, split_tokens=0, chunks=None,
             table=None, garbage=True, decode_twice=False, fused=False, repeats=0,
             n_query=0, host_plan=False, partition="per-row", device="cuda", kv=None, q=None,
             compact_pools=False):
    """Write rows of lengths ``lens`` (prefill of S-1 tokens in ``chunks``
    calls, then one decode token) and run one decode step.  ``fused``: the
    decode token is written by kvq_write_decode together with the decode
    step instead of by kvq_write before kvq_paged_decode.  ``host_plan``:
    partition as bench.py does, from the rows' lengths on the host
    (kvq_plan_split_tokens), instead of ``split_tokens``.  ``kv``: the rows'
    (K, V) device tensors [S, H, 128] instead of the workload's draws; ``q``:
    the queries [B, Hq, 128] likewise.  ``compact_pools``: copy to the host
    only the blocks the table names (gathered on the device, the table
    renumbered to match), for pools too large to copy whole."""
    from quantized_paged_kv_02_amd import kvq
    lens = np.asarray(lens, np.int32)
    b = len(lens)
    if table is None:
        table, nb = inputs.block_tables(w, np.maximum(lens, 1), seed)
    else:
        nb = int(table.max()) + 1
    mbs = table.shape[1]
    layout = kvq.make_layout(w.dtype, w.k_gran, w.v_gran, w.num_q_heads, w.num_kv_heads,
                             nb, mbs, split_tokens, w.residual_len, partition=partition)
    if host_plan:
        layout.split_tokens = kvq.plan_split_tokens(layout, lens)
        layout.partition = kvq.plan_partition(layout, lens)
    ks, vs = [], []
    for r in range(b):
        k, v = kv[r] if kv is not None else inputs.gen_kv(w, layer, r, int(lens[r]), device, seed)
        ks.append(k)
        vs.append(v)
    prefill_k = [k[:max(int(s) - 1, 0)] for k, s in zip(ks, lens)]
    prefill_v = [v[:max(int(s) - 1, 0)] for v, s in zip(vs, lens)]
    k_static = v_static = None
    if w.dtype not in KIVI:
        k_static = _static(w, w.k_gran, [t for t in prefill_k if len(t)] or ks, w.dtype)
        v_static = _static(w, w.v_gran, [t for t in prefill_v if len(t)] or vs, w.dtype)
    cache = kvq.alloc_cache(layout, ring_rows=b, device=device,
                            k_static=k_static, v_static=v_static)
    if garbage:
        fill_garbage(cache)
    table_t = torch.as_tensor(table, device=device)

    # prefill in `chunks` calls: chunk c writes tokens [cut_c, cut_{c+1}) of each row
    pre = np.maximum(lens - 1, 0)
    n_chunks = chunks or 1
    cuts = [np.floor(pre * c / n_chunks).astype(np.int64) for c in range(n_chunks + 1)]
    for c in range(n_chunks):
        lo, hi = cuts[c], cuts[c + 1]
        n = (hi - lo).astype(np.int32)
        if n.sum() == 0:
            continue
        kn = torch.cat([ks[r][lo[r]:hi[r]] for r in range(b)]).contiguous()
        vn = torch.cat([vs[r][lo[r]:hi[r]] for r in range(b)]).contiguous()
        cu = torch.as_tensor(np.concatenate([[0], np.cumsum(n)]).astype(np.int32), device=device)
        sl = torch.as_tensor(hi.astype(np.int32), device=device)
        kvq.write(cache, kn, vn, cu, table_t, sl, int(n.max()))
    # decode token (rows with S >= 1)
    n = (lens >= 1).astype(np.int32)
    if n.sum() and not fused:
        kn = torch.cat([ks[r][lens[r] - 1:lens[r]] for r in range(b) if lens[r] >= 1]).contiguous()
        vn = torch.cat([vs[r][lens[r] - 1:lens[r]] for r in range(b) if lens[r] >= 1]).contiguous()
        cu = torch.as_tensor(np.concatenate([[0], np.cumsum(n)]).astype(np.int32), device=device)
        kvq.write(cache, kn, vn, cu, table_t, torch.as_tensor(lens, device=device), 1)

    max_len = int(lens.max()) if b else 0
    scale = 1.0 / math.sqrt(128)
    lens_t = torch.as_tensor(lens, device=device)
    if n_query:
        # several query tokens per row: the last n_query positions (cached)
        q = inputs.gen_q(w, layer, device, seed, batch=b * n_query).reshape(
            b, n_query, w.num_q_heads, 128).contiguous()
        out = torch.full((b, n_query, w.num_q_heads, 128), float("nan"), dtype=torch.float32,
                         device=device)
        nbytes = kvq.paged_decode_mq_workspace_bytes(layout, n_query, b, max_len)
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
    else:
        if q is None:
            q = inputs.gen_q(w, layer, device, seed, batch=b)
        out = torch.full((b, w.num_q_heads, 128), float("nan"), dtype=torch.float32,
                         device=device)
        ws = kvq.alloc_workspace(layout, b, max_len, device)
    if n_query:
        kvq.paged_decode_mq(cache, q, table_t, lens_t, max_len, scale, out, ws)
    elif fused:
        # entry r is row r's decode token; rows of length 0 keep zeros (unread)
        kn = torch.zeros((b, w.num_kv_heads, 128), dtype=kvq.act_dtype(layout), device=device)
        vn = torch.zeros_like(kn)
        for r in range(b):
            if lens[r] >= 1:
                kn[r] = ks[r][lens[r] - 1]
                vn[r] = vs[r][lens[r] - 1]
        kvq.write_decode(cache, kn, vn, q, table_t, lens_t, max_len, scale, out, ws)
    else:
        kvq.paged_decode(cache, q, table_t, lens_t, max_len, scale, out, ws)
    out2 = None
    if decode_twice:
        out2 = torch.full_like(out, float("nan"))
        if n_query:
            kvq.paged_decode_mq(cache, q, table_t, lens_t, max_len, scale, out2, ws)
        else:
            kvq.paged_decode(cache, q, table_t, lens_t, max_len, scale, out2, ws)
    # further launches on the same workspace (`repeats` of them)
    rep_outs = []
    for _ in range(repeats):
        o = torch.full_like(out, float("nan"))
        kvq.paged_decode(cache, q, table_t, lens_t, max_len, scale, o, ws)
        rep_outs.append(o)
    torch.cuda.synchronize()
    if compact_pools:
        # block-major arrays: codes always, scales when per token or KIVI
        used = np.unique(table)
        idx = torch.as_tensor(used.astype(np.int64), device=device)
        major = {"k_codes": True, "v_codes": True,
                 "k_scales": w.dtype in KIVI or w.k_gran == "token",
                 "v_scales": w.dtype in KIVI or w.v_gran == "token"}
        pools = {name: _np(getattr(cache, name).index_select(0, idx) if bm
                           else getattr(cache, name))
                 for name, bm in major.items() if getattr(cache, name) is not None}
        table = np.searchsorted(used, table).astype(np.int32)
    else:
        pools = {name: _np(getattr(cache, name))
                 for name in ("k_codes", "v_codes", "k_scales", "v_scales")
                 if getattr(cache, name) is not None}
    if cache.k_resid is not None:
        pools["k_resid"] = cache.k_resid.cpu().numpy()
        pools["v_resid"] = cache.v_resid.cpu().numpy()
    res = CaseResult(w, lens, table, [_np(k) for k in ks], [_np(v) for v in vs],
                     _np(q), out.cpu().numpy(), pools, k_static, v_static, scale)
    if decode_twice:
        res.out2 = out2.cpu().numpy()
    res.repeat_outs = [o.cpu().numpy() for o in rep_outs]
    res.n_query = n_query
    return res


def oracle_row(res: CaseResult, r: int, check_codes=True):
    """Compare row r's cache bit-exactly with the oracle and return the
    oracle's fp64 attention output for the row."""
    w = res.w
    s = int(res.lens[r])
    kb, vb = res.k[r], res.v[r]
    row = res.table[r]
    p = res.pools
    if w.dtype in KIVI:
        affine = w.dtype != "int4"
        bits = 2 if w.dtype == "int2-affine" else 4
        kv = oracle.kivi_quantize(kb, vb, residual=w.residual_len, affine=affine, bits=bits)
        nq = kv["nq"]
        if check_codes:
            # A row of length S also holds, quantized, the group that leaves
            # the window at length S + 1 (flushed one write early); its tokens
            # are all older than S, so a repeated last token stands in for
            # token S.
            kq = oracle.kivi_quantize(np.concatenate([kb, kb[-1:]]),
                                      np.concatenate([vb, vb[-1:]]),
                                      residual=w.residual_len, affine=affine, bits=bits)
            nq1 = kq["nq"]
            assert np.array_equal(lv.logical_codes(p["k_codes"], row, nq1, "k", w.dtype),
                                  kq["k_codes"]), f"row {r}: INT4 K codes"
            assert np.array_equal(lv.logical_codes(p["v_codes"], row, nq1, "v", w.dtype),
                                  kq["v_codes"]), f"row {r}: INT4 V codes"
            if affine:
                assert np.array_equal(lv.int4_k_zero_points(p["k_scales"], row, nq1 // 64),
                                      kq["k_zp"]), f"row {r}: INT4 K zero points"
                assert np.array_equal(lv.int4_v_zero_points(p["v_scales"], row, nq1),
                                      kq["v_zp"]), f"row {r}: INT4 V zero points"
            gks = lv.int4_k_scales(p["k_scales"], row, nq1 // 64)
            assert np.array_equal(gks.view(np.uint32), kq["k_scales"].view(np.uint32)), \
                f"row {r}: INT4 K scales"
            gvs = lv.int4_v_scales(p["v_scales"], row, nq1)
            assert np.array_equal(gvs.view(np.uint32), kq["v_scales"].view(np.uint32)), \
                f"row {r}: INT4 V scales"
            ring = w.residual_len + 64
            rk, rv = lv.ring_tokens(p["k_resid"], p["v_resid"], r, np.arange(nq, s), ring)
            assert np.array_equal(rk.view(np.uint16), kv["k_resid"].view(np.uint16)), \
                f"row {r}: ring K"
            assert np.array_equal(rv.view(np.uint16), kv["v_resid"].view(np.uint16)), \
                f"row {r}: ring V"
        k_hat, v_hat = oracle.kivi_dequantize(kv)
    elif w.dtype in ("fp16", "bf16"):
        # unquantized: the cache holds the inputs' 16-bit values, attended as
        # such (bf16 arrays arrive as float32, converted exactly)
        if check_codes:
            for which, x in (("k", kb), ("v", vb)):
                g = lv.logical_codes(p[f"{which}_codes"], row, s, which, w.dtype)
                bits = np.uint32 if x.dtype == np.float32 else np.uint16
                assert np.array_equal(g.view(bits), x.view(bits)), \
                    f"row {r}: {w.dtype} {which} values differ"
        k_hat, v_hat = kb, vb
    else:
        out = []
        for which, x, gran, static in (("k", kb, w.k_gran, res.k_static),
                                      ("v", vb, w.v_gran, res.v_static)):
            pool = p[f"{which}_codes"]
            if gran == "token":
                codes, sc = oracle.quantize_per_token(x, w.dtype)
                if check_codes:
                    gsc = lv.logical_token_scales(p[f"{which}_scales"], row, s)
                    assert np.array_equal(gsc.view(np.uint32), sc.view(np.uint32)), \
                        f"row {r}: {which} per-token scales"
                scb = sc[..., None]
            else:
                codes = oracle.quantize_static(x, static, gran, w.dtype)
                st_ = np.asarray(static)
                if gran == "tensor":
                    scb = st_.reshape(1, 1, 1)
                elif gran == "head":
                    scb = st_.reshape(1, -1, 1)
                else:
                    scb = st_[None]
            if check_codes:
                g = lv.logical_codes(pool, row, s, which, w.dtype)
                want = codes.view(np.uint8)
                bad = np.argwhere(g != want)
                assert bad.size == 0, (f"row {r}: {which} codes differ at {len(bad)} places, "
                                       f"first {bad[:3].tolist()}")
            out.append(oracle.dequantize(codes, scb, w.dtype))
        k_hat, v_hat = out
    if getattr(res, "n_query", 0):
        return oracle.multi_query_attention(res.q[r].astype(np.float64), k_hat, v_hat,
                                            res.softmax_scale)
    return oracle.decode_attention(res.q[r].astype(np.float64), k_hat, v_hat, res.softmax_scale)


def check_rows(res: CaseResult, rows=None, check_codes=True):
    """Check rows against the oracle; returns the largest absolute error and
    leaves in ``res.tol_ratio`` the largest error as a fraction of its
    tolerance, max |got - want| / (ATOL + RTOL |want|) (1.0 = at the bound)."""
    rows = range(len(res.lens)) if rows is None else rows
    worst = 0.0
    ratio = 0.0
    for r in rows:
        want = oracle_row(res, r, check_codes)
        got = res.out[r].astype(np.float64)
        assert np.all(np.isfinite(got)), f"row {r}: non-finite output"
        err = np.abs(got - want)
        worst = max(worst, float(err.max()))
        bound = ATOL + RTOL * np.abs(want)
        ratio = max(ratio, float((err / bound).max()))
        ok = err <= bound
        assert ok.all(), (f"row {r}: {int((~ok).sum())} outputs out of tolerance, "
                          f"max abs err {err.max():.3e}, "
                          f"max err / tolerance {float((err / bound).max()):.3f}")
    res.tol_ratio = ratio
    return worst
