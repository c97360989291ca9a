"""Seeded synthetic inputs for the five decode workloads.

This module only draws data (K, V, Q, sequence lengths, block tables) and
holds the workload table; it contains none of the quantization or attention
arithmetic.  Both the HIP path and the CPU oracle receive the same tensors
from here.  The recipes are stated in the design notes:

* K, V, Q ~ N(0, 1) in fp32, then outliers, then rounded to fp16.
* Channel outliers: one seeded set of channel indices per workload, shared
  by every layer, head and token, scaled by the given factor.
* Element outliers: each element independently (seeded Bernoulli) scaled.
* Static scales (per head / per tensor) are calibrated from the layer's own
  prefill K (or V): max |x| over the extent divided by 448, in fp32.
* Block tables are the identity (row b owns blocks b*MBS ...) or a seeded
  permutation of all the blocks the rows need.
"""

from __future__ import annotations

import hashlib
from dataclasses import dataclass, field, replace

import numpy as np
import torch

HEAD_DIM = 128
BLOCK = 16


@dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    seq: int | tuple            # fixed length, or (lo, hi) uniform inclusive
    dtype: str                  # "int8" | "fp8" | "fp8e5m2" | "int4" | "int4-affine" |
                                # "int2-affine" | "fp16" | "bf16"
    k_gran: str                 # "tensor" | "head" | "channel" | "token" ("none": fp16, bf16)
    v_gran: str
    table: str = "identity"     # "identity" | "shuffled"
    channel_outliers: tuple = ()    # (count, factor, tensors) e.g. (4, 10.0, "kvq")
    element_outliers: tuple = ()    # (prob, factor, tensors)
    shift: tuple = ()               # (offset, tensors): mean added before fp16 rounding
    residual_len: int = 128
    description: str = field(default="", compare=False)

    @property
    def max_seq(self) -> int:
        return self.seq[1] if isinstance(self.seq, tuple) else self.seq


WORKLOADS = {
    "tiny": Workload(
        "tiny", 1, 1, 4, 2, 256, "int8", "token", "token",
        channel_outliers=(4, 10.0, "kvq"),
        description="1 layer, batch 1, 4 q / 2 KV heads, seq 256, INT8 per-token"),
    "llama2-7b": Workload(
        "llama2-7b", 32, 4, 32, 32, 2048, "int8", "token", "token",
        element_outliers=(0.01, 8.0, "kv"),
        description="Llama-2-7B shape: 32 layers, 32/32 heads, batch 4, seq 2048, INT8 per-token"),
    "llama3-8b-gqa": Workload(
        "llama3-8b-gqa", 32, 32, 32, 8, (1024, 16384), "fp8", "head", "head",
        table="shuffled",
        description="Llama-3-8B GQA: 32 layers, 32/8 heads, batch 32, seq U[1024,16384], "
                    "shuffled tables, FP8 E4M3 per-head static scales"),
    "kivi-int4": Workload(
        "kivi-int4", 32, 16, 32, 8, 32768, "int4", "channel", "token",
        channel_outliers=(8, 10.0, "k"),
        description="KIVI INT4: 32 layers, 32/8 heads, batch 16, seq 32768, K per-channel, "
                    "V per-token, group 64, fp16 residual 128"),
    "llama3-70b-int8": Workload(
        "llama3-70b-int8", 80, 24, 64, 8, 16384, "int8", "token", "token",
        description="Llama-3-70B shape: 80 layers, 64/8 heads, batch 24, seq 16384, INT8 per-token"),
    "llama3-70b-fp8": Workload(
        "llama3-70b-fp8", 80, 24, 64, 8, 16384, "fp8", "tensor", "tensor",
        description="Llama-3-70B shape: 80 layers, 64/8 heads, batch 24, seq 16384, FP8 per-tensor"),
    # the 70B FP8 workload with the pages' other FP8 format
    "llama3-70b-fp8e5m2": Workload(
        "llama3-70b-fp8e5m2", 80, 24, 64, 8, 16384, "fp8e5m2", "tensor", "tensor",
        description="Llama-3-70B shape: 80 layers, 64/8 heads, batch 24, seq 16384, "
                    "FP8 E5M2 per-tensor"),
    # the KIVI workload with asymmetric (affine) groups; V shifted off zero
    # so the zero points matter
    "kivi-int4-affine": Workload(
        "kivi-int4-affine", 32, 16, 32, 8, 32768, "int4-affine", "channel", "token",
        channel_outliers=(8, 10.0, "k"), shift=(0.5, "v"),
        description="KIVI INT4 affine: 32 layers, 32/8 heads, batch 16, seq 32768, K per-channel, "
                    "V per-token, group 64, zero points, fp16 residual 128; V ~ N(0.5, 1)"),
    # the same with 2-bit codes
    "kivi-int2-affine": Workload(
        "kivi-int2-affine", 32, 16, 32, 8, 32768, "int2-affine", "channel", "token",
        channel_outliers=(8, 10.0, "k"), shift=(0.5, "v"),
        description="KIVI 2-bit affine: 32 layers, 32/8 heads, batch 16, seq 32768, K "
                    "per-channel, V per-token, group 64, zero points, fp16 residual 128"),
    # unquantized baselines of the INT8 comparison ([intelli] §5): the INT8
    # workloads' shapes and inputs with an FP16 cache
    "llama2-7b-fp16": Workload(
        "llama2-7b-fp16", 32, 4, 32, 32, 2048, "fp16", "none", "none",
        element_outliers=(0.01, 8.0, "kv"),
        description="Llama-2-7B shape: 32 layers, 32/32 heads, batch 4, seq 2048, FP16 cache"),
    "llama3-70b-fp16": Workload(
        "llama3-70b-fp16", 80, 24, 64, 8, 16384, "fp16", "none", "none",
        description="Llama-3-70B shape: 80 layers, 64/8 heads, batch 24, seq 16384, FP16 cache"),
    # the same baselines for models that run in bf16: cache, queries and new
    # tokens in bf16
    "llama2-7b-bf16": Workload(
        "llama2-7b-bf16", 32, 4, 32, 32, 2048, "bf16", "none", "none",
        element_outliers=(0.01, 8.0, "kv"),
        description="Llama-2-7B shape: 32 layers, 32/32 heads, batch 4, seq 2048, BF16 cache"),
    "llama3-70b-bf16": Workload(
        "llama3-70b-bf16", 80, 24, 64, 8, 16384, "bf16", "none", "none",
        description="Llama-3-70B shape: 80 layers, 64/8 heads, batch 24, seq 16384, BF16 cache"),
}


def derive_seed(*parts) -> int:
    """Stable 63-bit seed from any tuple of ints/strings."""
    h = hashlib.sha256(repr(parts).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def seq_lens(w: Workload, seed: int = 0) -> np.ndarray:
    if isinstance(w.seq, tuple):
        rng = np.random.default_rng(derive_seed(seed, w.name, "lens"))
        return rng.integers(w.seq[0], w.seq[1] + 1, size=w.batch).astype(np.int32)
    return np.full(w.batch, w.seq, dtype=np.int32)


def block_tables(w: Workload, lens: np.ndarray, seed: int = 0, spare_blocks: int = 0):
    """(table int32 [B][MBS], num_blocks).  Identity: row b owns blocks
    b*MBS .. b*MBS + MBS - 1.  Shuffled: a seeded permutation of the
    sum_b ceil(S_b/16) blocks the rows need (+ spare_blocks unused ones);
    unused table entries are 0."""
    mbs = (int(np.max(lens)) + BLOCK - 1) // BLOCK if len(lens) else 1
    mbs = max(mbs, 1)
    b = len(lens)
    if w.table == "identity":
        table = (np.arange(b, dtype=np.int64)[:, None] * mbs
                 + np.arange(mbs, dtype=np.int64)[None, :]).astype(np.int32)
        return table, b * mbs + spare_blocks
    need = [(int(s) + BLOCK - 1) // BLOCK for s in lens]
    total = sum(need) + spare_blocks
    rng = np.random.default_rng(derive_seed(seed, w.name, "table"))
    perm = rng.permutation(total).astype(np.int32)
    table = np.zeros((b, mbs), np.int32)
    pos = 0
    for i, n in enumerate(need):
        table[i, :n] = perm[pos:pos + n]
        pos += n
    return table, max(total, 1)


def _channels(w: Workload, seed: int) -> np.ndarray:
    count = w.channel_outliers[0]
    rng = np.random.default_rng(derive_seed(seed, w.name, "outlier-channels"))
    return np.sort(rng.choice(HEAD_DIM, size=count, replace=False))


def _draw(w: Workload, shape, tensor: str, seed: int, layer: int, row: int, device,
          offset: int = 0):
    g = torch.Generator(device=device)
    g.manual_seed(derive_seed(seed, w.name, layer, row, tensor, offset))
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if w.channel_outliers and tensor in w.channel_outliers[2]:
        ch = torch.as_tensor(_channels(w, seed), device=device)
        x[..., ch] *= w.channel_outliers[1]
    if w.element_outliers and tensor in w.element_outliers[2]:
        prob, factor = w.element_outliers[0], w.element_outliers[1]
        u = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
        x = torch.where(u < prob, x * factor, x)
    if w.shift and tensor in w.shift[1]:
        x = x + w.shift[0]
    return x.to(torch.bfloat16 if w.dtype == "bf16" else torch.float16)


def gen_kv(w: Workload, layer: int, row: int, n_tokens: int, device="cpu", seed: int = 0,
           offset: int = 0):
    """fp16 (bf16 for a BF16 cache) K and V of one row, tokens
    offset .. offset+n_tokens-1, shape
    [n_tokens, Hkv, 128].  Tokens are drawn per (row, layer); ``offset`` only
    selects an independent stream for tokens written later."""
    shape = (n_tokens, w.num_kv_heads, HEAD_DIM)
    return (_draw(w, shape, "k", seed, layer, row, device, offset),
            _draw(w, shape, "v", seed, layer, row, device, offset))


def gen_q(w: Workload, layer: int, device="cpu", seed: int = 0, batch: int | None = None):
    b = w.batch if batch is None else batch
    return _draw(w, (b, w.num_q_heads, HEAD_DIM), "q", seed, layer, -1, device)


def scaled_down(w: Workload, **kw) -> Workload:
    """Same recipe with some fields replaced (small parity cases)."""
    return replace(w, **kw)
