"""Seeded synthetic inputs for MLA decode over a paged latent KV cache.

This module only draws random numbers and lays out storage: it rounds draws to
the storage formats (bf16 bit patterns; OCP FP8 E4M3FN codes with one fp32
scale per token), builds the page pool and the block table, and poisons unused
page slots. It holds none of the attention arithmetic. Both the CPU oracle and
the GPU path consume exactly the bytes it returns.

Shapes (all row-major, contiguous):
  q_bits       uint16 [B, s, H, 576]   bf16 bit patterns (512 latent + 64 rope), or
               uint16 [T, H, 576]      with a per-sequence q_len: the query
                                       tokens of sequence b are rows
                                       cu_q[b] .. cu_q[b+1] (cu_q int32 [B+1])
  cache        uint16 [P, 64, 576]     bf16 bit patterns, or
               uint8  [P, 64, 576]     E4M3FN codes
  kv_scale     float32 [P, 64]         per-token dequant scale (fp8 only)
  block_table  int32  [B, max_pages]   page ids, -1 past each sequence's pages
  seqlens      int32  [B]

Draw order for one workload (one numpy PCG64 stream): sequence lengths, the
page permutation, the per-sequence query counts (if drawn), q, then the
latent cache page by page.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

PAGE_TOKENS = 64
D_QK = 576      # latent (512) + rope (64)
D_V = 512
D_ROPE = 64
E4M3_MAX = 448.0
BF16_NAN = 0x7FC0
E4M3_NAN = 0x7F
DEFAULT_SCALE = 1.0 / math.sqrt(192.0)


@dataclass
class Workload:
    name: str
    q_bits: np.ndarray
    cache: np.ndarray
    kv_scale: Optional[np.ndarray]
    block_table: np.ndarray
    seqlens: np.ndarray
    softmax_scale: float
    kv_dtype: str                      # "bf16" or "fp8_e4m3"
    meta: dict = field(default_factory=dict)
    cu_q: Optional[np.ndarray] = None  # int32 [B+1] when q_len varies per sequence

    @property
    def varlen(self):
        return self.cu_q is not None

    @property
    def batch(self):
        return int(self.seqlens.shape[0])

    @property
    def q_lens(self):
        if self.varlen:
            return np.diff(self.cu_q).astype(np.int32)
        return np.full(self.batch, self.q_bits.shape[1], dtype=np.int32)

    @property
    def q_len(self):
        """Query tokens per sequence (the largest one for a per-sequence q_len)."""
        if self.varlen:
            return int(self.q_lens.max()) if self.batch else 0
        return int(self.q_bits.shape[1])

    @property
    def num_heads(self):
        return int(self.q_bits.shape[-2])

    @property
    def num_pages(self):
        return int(self.cache.shape[0])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest, ties to even); finite inputs."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _e4m3_encode(x: np.ndarray) -> np.ndarray:
    """float32 -> E4M3FN codes, round to nearest even, |x| <= 448 assumed."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def pages_for(seqlens: np.ndarray) -> np.ndarray:
    return (np.asarray(seqlens, dtype=np.int64) + PAGE_TOKENS - 1) // PAGE_TOKENS


def make_workload(name: str, batch: int, num_heads: int, q_len: int, seqlens,
                  kv_dtype: str = "bf16", seed: int = 0, table: str = "shuffled",
                  softmax_scale: float = DEFAULT_SCALE, poison_tail: bool = True,
                  rng: Optional[np.random.Generator] = None,
                  page_chunk: int = 512, q_lens=None) -> Workload:
    """Build one workload. `seqlens` is an int array or a callable(rng) -> array.

    q_lens (optional): per-sequence query counts (an int array or a
    callable(rng) -> array); q is then drawn as [sum(q_lens), H, 576] with
    offsets cu_q, and `q_len` is ignored.

    table: "identity" (pages laid out in (sequence, tile) order) or "shuffled"
    (a random permutation of the pool assigned in (sequence, tile) order).
    """
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(seed))
    if callable(seqlens):
        seqlens = seqlens(rng)
    seqlens = np.asarray(seqlens, dtype=np.int32).reshape(batch)
    npg = pages_for(seqlens)
    total_pages = int(npg.sum())
    max_pages = max(int(npg.max()) if batch else 0, 1)
    if table == "identity":
        perm = np.arange(total_pages, dtype=np.int64)
    elif table == "shuffled":
        perm = rng.permutation(total_pages)
    else:
        raise ValueError(table)
    block_table = np.full((batch, max_pages), -1, dtype=np.int32)
    pos = 0
    for b in range(batch):
        n = int(npg[b])
        block_table[b, :n] = perm[pos:pos + n]
        pos += n

    cu_q = None
    if q_lens is not None:
        if callable(q_lens):
            q_lens = q_lens(rng)
        q_lens = np.asarray(q_lens, dtype=np.int32).reshape(batch)
        cu_q = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
        q32 = rng.standard_normal((int(cu_q[-1]), num_heads, D_QK), dtype=np.float32)
    else:
        q32 = rng.standard_normal((batch, q_len, num_heads, D_QK), dtype=np.float32)
    q_bits = f32_to_bf16_bits(q32)
    del q32

    P = max(total_pages, 1)
    if kv_dtype == "bf16":
        cache = np.zeros((P, PAGE_TOKENS, D_QK), dtype=np.uint16)
        kv_scale = None
    elif kv_dtype == "fp8_e4m3":
        cache = np.zeros((P, PAGE_TOKENS, D_QK), dtype=np.uint8)
        kv_scale = np.ones((P, PAGE_TOKENS), dtype=np.float32)
    else:
        raise ValueError(kv_dtype)
    for p0 in range(0, total_pages, page_chunk):
        p1 = min(total_pages, p0 + page_chunk)
        x = rng.standard_normal((p1 - p0, PAGE_TOKENS, D_QK), dtype=np.float32)
        if kv_dtype == "bf16":
            cache[p0:p1] = f32_to_bf16_bits(x)
        else:
            # one scale per token: absmax over its 576 dims / 448; an all-zero
            # token keeps scale 1 (any scale encodes it as zero codes)
            amax = np.abs(x).max(axis=2)
            sc = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
            y = np.clip(x / sc[:, :, None], -E4M3_MAX, E4M3_MAX)
            cache[p0:p1] = _e4m3_encode(y)
            kv_scale[p0:p1] = sc
        del x

    if poison_tail:
        # slots past L_b on each sequence's last page hold NaN: a correct
        # kernel never lets them reach the output
        for b in range(batch):
            L = int(seqlens[b])
            if L % PAGE_TOKENS:
                last = block_table[b, L // PAGE_TOKENS]
                cache[last, L % PAGE_TOKENS:, :] = BF16_NAN if kv_dtype == "bf16" else E4M3_NAN
                if kv_scale is not None:
                    kv_scale[last, L % PAGE_TOKENS:] = np.nan

    return Workload(name=name, q_bits=q_bits, cache=cache, kv_scale=kv_scale,
                    block_table=block_table, seqlens=seqlens,
                    softmax_scale=float(softmax_scale), kv_dtype=kv_dtype,
                    meta={"seed": seed, "table": table, "total_pages": total_pages}, cu_q=cu_q)


# ---------------------------------------------------------------------------
# The five workloads the measurements are quoted on, and scaled-down variants
# with the same structure for parity tests the CPU oracle finishes in seconds.
# ---------------------------------------------------------------------------

def _uniform_lengths(lo, hi, n):
    return lambda rng: rng.integers(lo, hi + 1, size=n, dtype=np.int64).astype(np.int32)


def _ragged_lengths(n_short, lo, hi, long_len):
    def draw(rng):
        u = rng.uniform(math.log(lo), math.log(hi), size=n_short)
        short = np.floor(np.exp(u)).astype(np.int64)
        idx = int(rng.integers(0, n_short + 1))
        out = np.insert(short, idx, long_len)
        return out.astype(np.int32)
    return draw


CONFIGS = {
    # name: (batch, heads, q_len, seqlens, kv dtype, table)
    "tiny": dict(batch=1, num_heads=16, q_len=1, seqlens=[256], kv_dtype="bf16", table="identity"),
    "share16": dict(batch=64, num_heads=16, q_len=1, seqlens=_uniform_lengths(1024, 4096, 64),
                    kv_dtype="bf16", table="shuffled"),
    # the same batch over an fp8 cache (the 16-row fp8 kernel)
    "share16_fp8": dict(batch=64, num_heads=16, q_len=1, seqlens=_uniform_lengths(1024, 4096, 64),
                        kv_dtype="fp8_e4m3", table="shuffled"),
    "mtp": dict(batch=128, num_heads=128, q_len=2, seqlens=[4096] * 128, kv_dtype="bf16", table="shuffled"),
    "ragged": dict(batch=32, num_heads=128, q_len=1, seqlens=_ragged_lengths(31, 512, 16384, 65536),
                   kv_dtype="bf16", table="shuffled"),
    "fp8": dict(batch=128, num_heads=128, q_len=2, seqlens=[8192] * 128, kv_dtype="fp8_e4m3",
                table="shuffled"),
    # per-sequence q_len: each sequence verifies 1 + its own number of draft tokens
    "varlen": dict(batch=128, num_heads=128, q_len=6, q_lens=_uniform_lengths(1, 6, 128),
                   seqlens=[4096] * 128, kv_dtype="bf16", table="shuffled"),
}

CONFIG_TEXT = {
    "tiny": "batch 1, H=16, q_len=1, seqlen 256, bf16, identity block table",
    "share16": "batch 64, H=16, q_len=1, seqlens U[1024,4096], bf16, permuted block table",
    "share16_fp8": "batch 64, H=16, q_len=1, seqlens U[1024,4096], fp8 e4m3 cache + per-token fp32 scale, "
                   "permuted block table",
    "mtp": "batch 128, H=128, q_len=2 causal, seqlen 4096, bf16, shuffled block table",
    "ragged": "batch 32, H=128, q_len=1, 31 log-uniform seqlens in [512,16384] + one 65536, bf16",
    "fp8": "batch 128, H=128, q_len=2 causal, seqlen 8192, fp8 e4m3 cache + per-token fp32 scale",
    "varlen": "batch 128, H=128, per-sequence q_len U{1..6} causal, seqlen 4096, bf16, shuffled block table",
}

# Same structure, fewer sequences / shorter contexts.
SMALL = {
    "tiny": dict(CONFIGS["tiny"]),
    "share16": dict(batch=6, num_heads=16, q_len=1, seqlens=_uniform_lengths(1024, 4096, 6),
                    kv_dtype="bf16", table="shuffled"),
    "share16_fp8": dict(batch=6, num_heads=16, q_len=1, seqlens=_uniform_lengths(1024, 4096, 6),
                        kv_dtype="fp8_e4m3", table="shuffled"),
    "mtp": dict(batch=3, num_heads=128, q_len=2, seqlens=[4096, 1000, 130], kv_dtype="bf16",
                table="shuffled"),
    "ragged": dict(batch=5, num_heads=128, q_len=1, seqlens=_ragged_lengths(4, 512, 4000, 16384),
                   kv_dtype="bf16", table="shuffled"),
    "fp8": dict(batch=3, num_heads=128, q_len=2, seqlens=[8192, 777, 65], kv_dtype="fp8_e4m3",
                table="shuffled"),
    "varlen": dict(batch=5, num_heads=128, q_len=6, q_lens=[1, 6, 3, 2, 5], seqlens=[4096, 700, 65, 6, 1300],
                   kv_dtype="bf16", table="shuffled"),
}


def config(name: str, seed: int = 0, small: bool = False, **overrides) -> Workload:
    spec = dict((SMALL if small else CONFIGS)[name])
    spec.update(overrides)
    return make_workload(name + ("-small" if small else ""), seed=seed, **spec)


# ---------------------------------------------------------------------------
# Second workload: prefill / extend in the un-absorbed form. Packed,
# contiguous tensors (no pages): q [Tq, H, 192], k_nope [Tk, H, 128],
# k_rope [Tk, 64] (shared by the heads), v [Tk, H, 128], bf16 bits; sequence b
# owns queries cu_q[b]..cu_q[b+1] and keys cu_k[b]..cu_k[b+1]. Draw order: q,
# k_nope, k_rope, v (one PCG64 stream).
# ---------------------------------------------------------------------------
D_NOPE = 128
D_ROPE = 64
D_QK_PREFILL = D_NOPE + D_ROPE
D_V_PREFILL = 128


@dataclass
class PrefillWorkload:
    name: str
    q_bits: np.ndarray
    k_nope_bits: np.ndarray
    k_rope_bits: np.ndarray
    v_bits: np.ndarray
    cu_q: np.ndarray
    cu_k: np.ndarray
    softmax_scale: float
    meta: dict = field(default_factory=dict)

    @property
    def batch(self):
        return int(self.cu_q.shape[0] - 1)

    @property
    def num_heads(self):
        return int(self.q_bits.shape[1])

    @property
    def q_lens(self):
        return np.diff(self.cu_q).astype(np.int64)

    @property
    def k_lens(self):
        return np.diff(self.cu_k).astype(np.int64)


def make_prefill_workload(name: str, q_lens, k_lens, num_heads: int, seed: int = 0,
                          softmax_scale: float = DEFAULT_SCALE) -> PrefillWorkload:
    """q_lens[b] new tokens at the end of k_lens[b] tokens (q_lens <= k_lens)."""
    q_lens = np.asarray(q_lens, dtype=np.int64)
    k_lens = np.asarray(k_lens, dtype=np.int64)
    if np.any(q_lens > k_lens) or np.any(q_lens < 0):
        raise ValueError("need 0 <= q_len <= k_len per sequence")
    rng = np.random.Generator(np.random.PCG64(seed))
    cu_q = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(k_lens)]).astype(np.int32)
    Tq, Tk, H = int(cu_q[-1]), int(cu_k[-1]), num_heads
    q = f32_to_bf16_bits(rng.standard_normal((max(Tq, 1), H, D_QK_PREFILL), dtype=np.float32))[:Tq]
    kn = f32_to_bf16_bits(rng.standard_normal((max(Tk, 1), H, D_NOPE), dtype=np.float32))[:Tk]
    kr = f32_to_bf16_bits(rng.standard_normal((max(Tk, 1), D_ROPE), dtype=np.float32))[:Tk]
    v = f32_to_bf16_bits(rng.standard_normal((max(Tk, 1), H, D_V_PREFILL), dtype=np.float32))[:Tk]
    return PrefillWorkload(name=name, q_bits=np.ascontiguousarray(q), k_nope_bits=np.ascontiguousarray(kn),
                           k_rope_bits=np.ascontiguousarray(kr), v_bits=np.ascontiguousarray(v),
                           cu_q=cu_q, cu_k=cu_k, softmax_scale=float(softmax_scale),
                           meta={"seed": seed})


# DeepSeek-V3 attention on one GPU's share of a TP8 deployment (128 / 8 = 16
# heads): a long prefill, and extends of 1024 new tokens after an 8K prefix.
PREFILL_CONFIGS = {
    "prefill": dict(q_lens=[8192, 8192], k_lens=[8192, 8192], num_heads=16),
    "extend": dict(q_lens=[1024] * 4, k_lens=[9216] * 4, num_heads=16),
}
PREFILL_TEXT = {
    "prefill": "un-absorbed MLA prefill, 2 sequences x 8192 tokens, H=16, head dim 192 (128 nope + 64 rope), v 128, causal",
    "extend": "un-absorbed MLA extend, 4 sequences x 1024 new tokens after 8192 cached, H=16, head dim 192, v 128",
}
PREFILL_SMALL = {
    "prefill": dict(q_lens=[300, 129, 64, 1], k_lens=[300, 129, 64, 1], num_heads=16),
    "extend": dict(q_lens=[100, 64, 3], k_lens=[400, 64, 700], num_heads=16),
}


def prefill_config(name: str, seed: int = 0, small: bool = False) -> PrefillWorkload:
    spec = (PREFILL_SMALL if small else PREFILL_CONFIGS)[name]
    return make_prefill_workload(name + ("-small" if small else ""), spec["q_lens"], spec["k_lens"],
                                 spec["num_heads"], seed=seed)
