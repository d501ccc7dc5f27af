"""Plain float64 MLA decode (test infrastructure only; see the package docstring).

Readings of the pages used here (the pages fix none of these numbers; the
workload descriptions do, and where both are silent the plainest reading is
taken):
  * one latent row of 576 values per cached token, shared by all heads; the key
    is the whole row, the value is its first 512 entries (the absorbed form of
    MLA that the pages switch on with matrix absorption for DeepSeek decode --
    mhpq.cn article on PaddleNLP inference flags, section on speculative
    decoding parameters);
  * q_len > 1 query tokens per sequence (PaddleNLP issue #10157, MLA operator
    overview: decode with more than one token per request; MTP section: the
    verification batch keeps its size). Query i of s sees keys j <= L - s + i;
  * pages of 64 tokens reached through a block table;
  * LSE is the natural-log log-sum-exp of the scaled scores;
  * a row with no visible key gives O = 0 and LSE = -inf.
"""
from __future__ import annotations

import math

import numpy as np

PAGE_TOKENS = 64
D_QK = 576
D_V = 512


# --------------------------------------------------------------------------
# Storage formats, decoded exactly to float64.
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64. A bf16 value is the top half of a float32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):      # NaN patterns stay NaN
        return u.view(np.float32).astype(np.float64)


def e4m3fn_value(code: int) -> float:
    """Value of one OCP FP8 E4M3FN code, from the format definition.

    sign 1 bit, exponent 4 bits (bias 7), mantissa 3 bits. Exponent field 0
    encodes subnormals m/8 * 2^-6. S.1111.111 is NaN; there is no infinity, so
    S.1111.110 = 448 is the largest finite magnitude.
    """
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** -6
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


E4M3FN_TABLE = np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    return E4M3FN_TABLE[np.asarray(codes, dtype=np.uint8)]


# --------------------------------------------------------------------------
# Paged gather and the causal rule.
# --------------------------------------------------------------------------

def sequence_rows(cache: np.ndarray, block_table_row: np.ndarray, n: int,
                  kv_dtype: str = "bf16", kv_scale: np.ndarray | None = None) -> np.ndarray:
    """The first n latent rows of one sequence, float64 [n, 576].

    Token j lives in page block_table_row[j // 64], slot j % 64. For the fp8
    cache the row is the decoded code times that token's fp32 scale (the
    product is exact in float64).
    """
    j = np.arange(n)
    pages = np.asarray(block_table_row)[j // PAGE_TOKENS].astype(np.int64)
    slots = j % PAGE_TOKENS
    raw = cache[pages, slots]
    if kv_dtype == "bf16":
        return bf16_bits_to_f64(raw)
    if kv_dtype == "fp8_e4m3":
        return decode_e4m3fn(raw) * kv_scale[pages, slots].astype(np.float64)[:, None]
    raise ValueError(kv_dtype)


def visible_counts(seqlen: int, q_len: int, num_heads: int) -> np.ndarray:
    """Keys visible to each of the q_len*num_heads rows (row = i*H + h).

    Query i sees keys 0 .. L - s + i, i.e. L - s + i + 1 keys, clipped to
    [0, L]; every head of one query token sees the same keys.
    """
    i = np.arange(q_len * num_heads) // num_heads
    return np.clip(seqlen - q_len + i + 1, 0, seqlen).astype(np.int64)


# --------------------------------------------------------------------------
# Attention, plain definition.
# --------------------------------------------------------------------------

def attend(q_rows: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
           visible: np.ndarray):
    """O[r] = sum_j p_rj V_j, LSE[r] = log sum_j exp(z_rj) over j < visible[r].

    z = scale * q_r . K_j; p_r = softmax of z_r over the visible keys. The full
    score matrix [R, n] is materialised. Returns (O [R, Dv], lse [R]) float64.
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    R, n = q_rows.shape[0], K.shape[0]
    O = np.zeros((R, V.shape[1]), dtype=np.float64)
    lse = np.full(R, -np.inf, dtype=np.float64)
    if n == 0:
        return O, lse
    Z = float(scale) * (q_rows @ K.T)
    mask = np.arange(n)[None, :] < np.asarray(visible)[:, None]
    Z = np.where(mask, Z, -np.inf)
    live = np.asarray(visible) > 0
    if not live.any():
        return O, lse
    Zl = Z[live]
    m = Zl.max(axis=1)
    E = np.exp(Zl - m[:, None])
    l = E.sum(axis=1)
    P = E / l[:, None]
    O[live] = P @ V
    lse[live] = m + np.log(l)
    return O, lse


def attend_partials(q_rows, K, V, scale, visible, cuts):
    """Attention restricted to key chunks [cuts[k], cuts[k+1]), one partial each.

    Each partial is (O_k, LSE_k) of the keys in the chunk that are visible to
    the row; a chunk with no visible key gives O_k = 0, LSE_k = -inf.
    """
    parts = []
    visible = np.asarray(visible)
    for a, b in zip(cuts[:-1], cuts[1:]):
        vis = np.clip(visible - a, 0, b - a)
        parts.append(attend(q_rows, K[a:b], V[a:b], scale, vis))
    return parts


def lse_merge(outs, lses):
    """Merge partials of disjoint key sets.

    LSE = M + log sum_k exp(LSE_k - M), M = max_k LSE_k;
    O = sum_k exp(LSE_k - LSE) O_k. Partials with LSE_k = -inf weigh 0; if all
    are -inf the result is O = 0, LSE = -inf.
    """
    outs = np.asarray(outs, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    M = lses.max(axis=0)
    finite = np.isfinite(M)
    Ms = np.where(finite, M, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - Ms[None]), 0.0)
    tot = w.sum(axis=0)
    lse = np.where(finite, Ms + np.log(np.where(finite, tot, 1.0)), -np.inf)
    coef = np.where(finite[None], w / np.where(finite, tot, 1.0)[None], 0.0)
    O = np.einsum("kr,krd->rd", coef, outs)
    return O, lse


def mla_decode_sequence(q_bits_b, cache, block_table_row, seqlen, softmax_scale,
                        kv_dtype="bf16", kv_scale=None, q_values=None):
    """One sequence: q_bits_b uint16 [s, H, 576] -> (O [s, H, 512], lse [s, H]).

    q_values (optional, float64 [s, H, 576]) replaces the decoded q_bits, e.g.
    the E4M3 image of the queries from quantize_query_rows_e4m3."""
    s, H, _ = q_bits_b.shape
    if q_values is None:
        q_rows = bf16_bits_to_f64(q_bits_b).reshape(s * H, D_QK)
    else:
        q_rows = np.asarray(q_values, dtype=np.float64).reshape(s * H, D_QK)
    L = int(seqlen)
    rows = sequence_rows(cache, block_table_row, L, kv_dtype, kv_scale)
    O, lse = attend(q_rows, rows, rows[:, :D_V], softmax_scale, visible_counts(L, s, H))
    return O.reshape(s, H, D_V), lse.reshape(s, H)


def mla_decode_varlen(q_bits, cu_q, cache, block_table, seqlens, softmax_scale, kv_dtype="bf16",
                      kv_scale=None, batch_indices=None):
    """Per-sequence q_len (the MTP verification of PaddleNLP issue #10157: each
    request checks 1 + its own number of draft tokens). q_bits uint16 [T, H, 576];
    the s_b = cu_q[b+1] - cu_q[b] query tokens of sequence b are rows
    cu_q[b]..cu_q[b+1], and query i of them sees keys j <= L_b - s_b + i.
    Returns out [T, H, 512], lse [T, H] float64 (rows of sequences not listed in
    batch_indices stay 0 / -inf)."""
    T, H, _ = q_bits.shape
    out = np.zeros((T, H, D_V), dtype=np.float64)
    lse = np.full((T, H), -np.inf, dtype=np.float64)
    idx = range(len(seqlens)) if batch_indices is None else list(batch_indices)
    for b in idx:
        r0, r1 = int(cu_q[b]), int(cu_q[b + 1])
        if r1 == r0:
            continue
        out[r0:r1], lse[r0:r1] = mla_decode_sequence(q_bits[r0:r1], cache, block_table[b], seqlens[b],
                                                      softmax_scale, kv_dtype, kv_scale)
    return out, lse


def mla_decode(q_bits, cache, block_table, seqlens, softmax_scale, kv_dtype="bf16",
               kv_scale=None, batch_indices=None, q_values=None):
    """Whole batch (or the listed sequences): out [B, s, H, 512], lse [B, s, H] float64.

    q_values (optional, float64 [B, s, H, 576]) replaces the decoded q_bits."""
    B, s, H, _ = q_bits.shape
    idx = range(B) if batch_indices is None else list(batch_indices)
    out = np.zeros((len(idx), s, H, D_V), dtype=np.float64)
    lse = np.zeros((len(idx), s, H), dtype=np.float64)
    for k, b in enumerate(idx):
        out[k], lse[k] = mla_decode_sequence(q_bits[b], cache, block_table[b], seqlens[b],
                                              softmax_scale, kv_dtype, kv_scale,
                                              None if q_values is None else q_values[b])
    return out, lse


# --------------------------------------------------------------------------
# Appending new tokens' latent rows to the cache (the step before attention
# in a decode step; cache quantisation C8 of PaddleNLP issue #10157's
# overview, read as OCP E4M3FN codes with one fp32 scale per token).
# --------------------------------------------------------------------------

E4M3FN_MAX = 448.0


def encode_e4m3fn(x) -> np.ndarray:
    """Nearest OCP E4M3FN code to each value, ties to the code with the even
    mantissa (round to nearest even), read off the format's value table.

    Only |x| <= 448 is accepted (callers clamp first). The sign of x is kept,
    so values that round to zero give 0x00 or 0x80.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.abs(x) <= E4M3FN_MAX):
        raise ValueError("encode_e4m3fn takes |x| <= 448")
    pos = E4M3FN_TABLE[:0x7F]                       # codes 0x00..0x7E, ascending 0..448
    a = np.abs(x)
    hi = np.clip(np.searchsorted(pos, a, side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo = a - pos[lo]
    d_hi = pos[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo).astype(np.uint8)
    return code | (np.signbit(x).astype(np.uint8) << np.uint8(7))


def quantize_token_e4m3(x_f32) -> tuple[np.ndarray, np.float32]:
    """One token's row -> (E4M3FN codes, fp32 scale).

    scale = max|x| / 448 in fp32 (1 for an all-zero row); code = nearest-even
    E4M3FN of clamp(x / scale, -448, 448), the division done in fp32. Every
    fp32 operation here is a single correctly rounded IEEE operation.
    """
    x = np.asarray(x_f32, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x)))
    scale = np.float32(amax / np.float32(E4M3FN_MAX)) if amax > 0 else np.float32(1.0)
    y = np.clip((x / scale).astype(np.float32), -E4M3FN_MAX, E4M3FN_MAX)
    return encode_e4m3fn(y), scale


def append_kv(latent_bits, block_table, seqlens, cache, kv_scale=None, kv_dtype="bf16"):
    """Store each sequence's newest latent rows in their pages; returns new
    (cache, kv_scale) arrays (inputs are not modified).

    latent_bits: bf16 bits [B, s, 576]; seqlens include the new tokens, so
    token i of sequence b is position j = L_b - s + i, stored at page
    block_table[b][j // 64], slot j % 64. Positions j < 0 are skipped.
    bf16 cache: the bits are copied. fp8 cache: quantize_token_e4m3 of the
    row's exact fp32 values.
    """
    latent_bits = np.asarray(latent_bits, dtype=np.uint16)
    B, s, _ = latent_bits.shape
    cache = np.array(cache, copy=True)
    kv_scale = None if kv_scale is None else np.array(kv_scale, copy=True)
    for b in range(B):
        L = int(seqlens[b])
        for i in range(s):
            j = L - s + i
            if j < 0:
                continue
            page = int(block_table[b][j // PAGE_TOKENS])
            slot = j % PAGE_TOKENS
            if kv_dtype == "bf16":
                cache[page, slot] = latent_bits[b, i]
            else:
                x = bf16_bits_to_f64(latent_bits[b, i]).astype(np.float32)   # exact
                codes, sc = quantize_token_e4m3(x)
                cache[page, slot] = codes
                kv_scale[page, slot] = sc
    return cache, kv_scale


def query_row_exponent(amax) -> int:
    """The exponent k of a query row's power-of-two scale: the smallest
    integer with max|row| <= 448 * 2^k, never below -126 (rows whose maximum
    lies under 448 * 2^-127 keep k = -126)."""
    amax = float(amax)
    if amax <= 0.0:
        return 0
    m, e = np.frexp(amax)                 # amax = m * 2^e, m in [0.5, 1)
    k = int(e) - 1 - 8                    # 2^(e-1) <= amax < 2^e; 448 = 1.75 * 2^8
    while amax > E4M3FN_MAX * 2.0 ** k:
        k += 1
    while k > -126 and amax <= E4M3FN_MAX * 2.0 ** (k - 1):
        k -= 1
    return max(k, -126)


def quantize_query_rows_e4m3(q_bits) -> np.ndarray:
    """E4M3 image of the query rows for a decode that runs the contractions on
    FP8 operands (PaddleNLP issue #10157, quantization section: SageAttention2
    quantises the attention operands dynamically, one scale per block of
    values, and dequantises the products once; the form of the scale is left
    open there). Each row of 576 values gets a power-of-two scale 2^k, k from
    query_row_exponent (the E8M0 form of the fp8 matrix cores' block scales),
    and nearest-even E4M3FN codes of x * 2^-k (exact products, |x| 2^-k <= 448);
    returns 2^k * value(code) as float64, shape of q_bits (bf16 bits)."""
    x = bf16_bits_to_f64(q_bits)
    flat = x.reshape(-1, x.shape[-1])
    out = np.empty(flat.shape, dtype=np.float64)
    for r in range(flat.shape[0]):
        k = query_row_exponent(np.max(np.abs(flat[r])))
        codes = encode_e4m3fn(flat[r] * 2.0 ** -k)
        out[r] = decode_e4m3fn(codes) * 2.0 ** k
    return out.reshape(x.shape)


# --------------------------------------------------------------------------
# Prefill / extend, the un-absorbed form (the second workload): per head the
# key is [k_nope_h (128), k_rope (64, shared by the heads)], head dim 192 (the
# DeepSeek head dim of PaddleNLP issue #10157, quantization section,
# SageAttention), and the value is v_h (128).
# --------------------------------------------------------------------------
D_NOPE = 128
D_ROPE = 64
D_QK_PREFILL = D_NOPE + D_ROPE
D_V_PREFILL = 128


def mla_prefill(q_bits, k_nope_bits, k_rope_bits, v_bits, cu_q, cu_k, softmax_scale, batch_indices=None):
    """Causal attention of new tokens over their sequence's keys.

    q [Tq, H, 192], k_nope [Tk, H, 128], k_rope [Tk, 64], v [Tk, H, 128], all
    bf16 bits. Sequence b owns queries cu_q[b]..cu_q[b+1] (N_b of them) and
    keys cu_k[b]..cu_k[b+1] (L_b >= N_b); its N_b queries are the last N_b of
    its L_b tokens, so query i sees keys j <= L_b - N_b + i (prefill: N_b = L_b;
    extend: a cached prefix of L_b - N_b tokens). Returns out [Tq, H, 128] and
    lse [Tq, H] float64 (natural log); rows of unlisted sequences stay 0 / -inf.
    """
    Tq, H, _ = q_bits.shape
    out = np.zeros((Tq, H, D_V_PREFILL), dtype=np.float64)
    lse = np.full((Tq, H), -np.inf, dtype=np.float64)
    idx = range(len(cu_q) - 1) if batch_indices is None else list(batch_indices)
    for b in idx:
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        k0, k1 = int(cu_k[b]), int(cu_k[b + 1])
        N, L = q1 - q0, k1 - k0
        if N == 0:
            continue
        vis = visible_counts(L, N, 1)
        rope = bf16_bits_to_f64(k_rope_bits[k0:k1])
        for h in range(H):
            K = np.concatenate([bf16_bits_to_f64(k_nope_bits[k0:k1, h]), rope], axis=1)
            V = bf16_bits_to_f64(v_bits[k0:k1, h])
            out[q0:q1, h], lse[q0:q1, h] = attend(bf16_bits_to_f64(q_bits[q0:q1, h]), K, V, softmax_scale, vis)
    return out, lse
