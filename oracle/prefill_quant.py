"""Quantised prefill attention, the method's steps in float64 (test
infrastructure only: the tests, the smoke check and the benchmark's CPU leg
use it; the HIP library never does).

The method (PaddleNLP issue #10157, quantization section "SageAttention
quantization", and the Paddle 3.0 article's section on SageAttention dynamic
quantization for DeepSeek, head dim 192): Q and K are quantised on the fly to
INT8 and V to FP8; the INT32 products Q.K^T are turned into FP32 and
dequantised, an online softmax runs over them, its output P is quantised to
FP8 and multiplied with the FP8 V, and the product is dequantised once to give
O.

The pages fix none of the block sizes, scale rules or roundings. The readings
taken here (each listed with its reason in the design notes):
  * Q: one INT8 block per (query token, head) over its 192 features;
  * K: one INT8 block per (sequence, 64-key tile from the sequence's first key,
    head) over the tile's valid keys x 192 features;
  * INT8 block: scale = max|x| / 127 and inv = 127 / max|x| in fp32 (scale 1,
    codes 0 for an all-zero block); code = clamp(rint(fp32(x * inv)), +-127);
  * V: E4M3FN codes per (sequence, 32-key block, head, feature) with a
    power-of-two scale 2^e, e the smallest integer with max|v| <= 448 * 2^e
    (clamped to [-127, 127], 0 for an all-zero block); code = nearest-even
    E4M3FN of v * 2^-e (exact in fp32);
  * online softmax over 64-key tiles, the running max always raised to the
    tile's max (so every P <= 1); P is quantised as the E4M3FN code of
    P * 2^8 (<= 256, inside the format's range) and counts 2^-8 times its
    value in P.V; the row sum l accumulates the unquantised P.
Scores are dequantised as S = (q8 . k8) * s_q * s_k * softmax_scale; LSE is
the natural-log log-sum-exp of S over the visible keys; a row with no visible
key gives O = 0, LSE = -inf (as in the unquantised oracle).
"""
from __future__ import annotations

import numpy as np

from .mla_oracle import bf16_bits_to_f64, decode_e4m3fn, encode_e4m3fn, E4M3FN_MAX

K_TILE = 64        # keys per K block and per online-softmax step
V_BLOCK = 32       # keys per V scale block
P_SHIFT = 8        # P is stored as P * 2^8
INT8_MAX = 127


def quantize_int8(x_f32, axis=None) -> tuple[np.ndarray, np.ndarray]:
    """Symmetric INT8 codes of blocks of fp32 values: (codes int8, scales fp32).

    A block is the whole array (axis=None) or every slice along the given
    axes. amax = max|x| over the block; scale = fp32(amax / 127) and
    inv = fp32(127 / amax) (scale 1 and all codes 0 when amax = 0);
    code = clamp(rint(fp32(x * inv)), -127, 127). Each fp32 operation is one
    correctly rounded IEEE operation.
    """
    x = np.asarray(x_f32, dtype=np.float32)
    amax = np.max(np.abs(x), axis=axis, keepdims=True).astype(np.float32)
    zero = amax == 0
    safe = np.where(zero, np.float32(1), amax).astype(np.float32)
    scale = np.where(zero, np.float32(1), (safe / np.float32(INT8_MAX)).astype(np.float32)).astype(np.float32)
    inv = np.where(zero, np.float32(0), (np.float32(INT8_MAX) / safe).astype(np.float32)).astype(np.float32)
    codes = np.clip(np.rint((x * inv).astype(np.float32)), -INT8_MAX, INT8_MAX).astype(np.int8)
    scale = scale.reshape(()) if axis is None else np.squeeze(scale, axis=axis)
    return codes, scale


def e8m0_exponent(amax) -> np.ndarray:
    """Smallest integer e with amax <= 448 * 2^e, clamped to [-127, 127]; 0
    for amax = 0 (elementwise). With amax = m * 2^E (m in [0.5, 1)) and
    448 = 0.875 * 2^9, e = E - 9 when m <= 0.875 and E - 8 otherwise."""
    a = np.asarray(amax, dtype=np.float64)
    m, E = np.frexp(a)
    e = np.where(m <= 0.875, E - 9, E - 8)
    return np.where(a == 0, 0, np.clip(e, -127, 127)).astype(np.int64)


def quantize_e4m3_pow2(x_f32, e) -> np.ndarray:
    """E4M3FN codes of x * 2^-e (exact), nearest even, clamped to +-448 (e broadcasts)."""
    y = np.ldexp(np.asarray(x_f32, dtype=np.float32).astype(np.float64), -np.asarray(e))
    return encode_e4m3fn(np.clip(y, -E4M3FN_MAX, E4M3FN_MAX))


def quantize_query(q_bits):
    """q bf16 bits [Tq, H, 192] -> (codes int8 [Tq, H, 192], scales fp32 [Tq, H]),
    one INT8 block per (token, head)."""
    q = bf16_bits_to_f64(np.asarray(q_bits, dtype=np.uint16)).astype(np.float32)
    return quantize_int8(q, axis=2)


def quantize_kv(k_nope_bits, k_rope_bits, v_bits, cu_k):
    """Per sequence b, its quantised keys and values:
      k_codes int8 [L, H, 192]  (features: the head's 128 k_nope, then the 64 shared k_rope)
      k_scale fp32 [ceil(L/64), H]
      v_codes uint8 [L, H, 128] (E4M3FN)
      v_exp   int   [ceil(L/32), H, 128]
    """
    kn = bf16_bits_to_f64(np.asarray(k_nope_bits, dtype=np.uint16)).astype(np.float32)
    kr = bf16_bits_to_f64(np.asarray(k_rope_bits, dtype=np.uint16)).astype(np.float32)
    v = bf16_bits_to_f64(np.asarray(v_bits, dtype=np.uint16)).astype(np.float32)
    H, Dv = kn.shape[1], v.shape[2]
    seqs = []
    for b in range(len(cu_k) - 1):
        k0, k1 = int(cu_k[b]), int(cu_k[b + 1])
        L = k1 - k0
        K = np.concatenate([kn[k0:k1], np.broadcast_to(kr[k0:k1, None, :], (L, H, kr.shape[1]))], axis=2)
        nt, ng = -(-L // K_TILE), -(-L // V_BLOCK)
        k_codes = np.zeros((L, H, K.shape[2]), dtype=np.int8)
        k_scale = np.ones((nt, H), dtype=np.float32)
        for t in range(nt):
            a, z = t * K_TILE, min(L, (t + 1) * K_TILE)
            k_codes[a:z], k_scale[t] = quantize_int8(K[a:z], axis=(0, 2))   # one block per head
        v_codes = np.zeros((L, H, Dv), dtype=np.uint8)
        v_exp = np.zeros((ng, H, Dv), dtype=np.int64)
        for g in range(ng):
            a, z = g * V_BLOCK, min(L, (g + 1) * V_BLOCK)
            blk = v[k0 + a:k0 + z]                                   # [keys, H, Dv]
            v_exp[g] = e8m0_exponent(np.max(np.abs(blk), axis=0))    # one block per (head, feature)
            v_codes[a:z] = quantize_e4m3_pow2(blk, v_exp[g][None])
        seqs.append(dict(k_codes=k_codes, k_scale=k_scale, v_codes=v_codes, v_exp=v_exp))
    return seqs


# P codes whose input lies within this relative distance of a rounding tie
# may come out either way in an fp32 evaluation of the same steps.
TIE_WINDOW = 2.0 ** -14


def prefill_quant(q_bits, k_nope_bits, k_rope_bits, v_bits, cu_q, cu_k, softmax_scale,
                  batch_indices=None, rows=None, return_slack=False, tile_dot_rel=0.0):
    """Quantised causal prefill / extend. Shapes and visibility as the
    unquantised prefill: sequence b owns queries cu_q[b]..cu_q[b+1] (N_b, the
    last N_b of its L_b tokens) and keys cu_k[b]..cu_k[b+1]; query i sees keys
    j <= L_b - N_b + i. Returns out [Tq, H, 128], lse [Tq, H] float64 (rows of
    unlisted sequences stay 0 / -inf). rows: optional {b: query indices} to
    compute only those rows of sequence b.

    return_slack: also return slack [Tq, H, 128], a bound on how far out may
    move when P codes whose input P * 2^8 lies within TIE_WINDOW (relative)
    of a rounding tie take the other of their two candidate codes -- the
    codes an fp32 evaluation of these steps may legitimately pick -- plus,
    when tile_dot_rel > 0, an error of up to tile_dot_rel times the largest
    |P8_j V8_jd| term in each tile's P.V sum (for arithmetic that rounds
    those sums more coarsely than the exact products).
    """
    q_codes, q_scale = quantize_query(q_bits)
    kv = quantize_kv(k_nope_bits, k_rope_bits, v_bits, cu_k)
    Tq, H, _ = q_codes.shape
    Dv = kv[0]["v_codes"].shape[2] if kv else 128
    out = np.zeros((Tq, H, Dv), dtype=np.float64)
    lse = np.full((Tq, H), -np.inf, dtype=np.float64)
    slack = np.zeros((Tq, H, Dv), dtype=np.float64)
    idx = range(len(cu_q) - 1) if batch_indices is None else list(batch_indices)
    for b in idx:
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        N, L = q1 - q0, int(cu_k[b + 1]) - int(cu_k[b])
        if N == 0:
            continue
        sel = np.arange(N) if rows is None or b not in rows else np.asarray(rows[b], dtype=np.int64)
        last_key = (L - N) + sel                       # row i sees keys 0..L-N+i
        s = kv[b]
        vvals = decode_e4m3fn(s["v_codes"])            # [L, H, Dv]
        vscale = np.ldexp(1.0, np.repeat(s["v_exp"], V_BLOCK, axis=0)[:L])  # [L, H, Dv]
        for h in range(H):
            qc = q_codes[q0 + sel, h].astype(np.float64)           # exact small integers
            sq = q_scale[q0 + sel, h].astype(np.float64)
            m = np.full(len(sel), -np.inf)
            l = np.zeros(len(sel))
            o = np.zeros((len(sel), Dv))
            sl = np.zeros((len(sel), Dv))
            for t in range(-(-L // K_TILE)):
                a, z = t * K_TILE, min(L, (t + 1) * K_TILE)
                keys = np.arange(a, z)
                vis = keys[None, :] <= last_key[:, None]
                if not vis.any():
                    continue
                dots = qc @ s["k_codes"][a:z, h].astype(np.float64).T          # exact integers
                S = dots * sq[:, None] * np.float64(s["k_scale"][t, h]) * float(softmax_scale)
                S = np.where(vis, S, -np.inf)
                m_new = np.maximum(m, S.max(axis=1))
                live = m_new > -np.inf
                alpha = np.where(live & (m > -np.inf), np.exp(np.where(live, m - m_new, 0.0)), 0.0)
                P = np.where(vis, np.exp(S - np.where(live, m_new, 0.0)[:, None]), 0.0)
                y = np.ldexp(P, P_SHIFT)
                P8 = decode_e4m3fn(encode_e4m3fn(y)) * 2.0 ** -P_SHIFT
                V8 = vvals[a:z, h] * vscale[a:z, h]
                l = l * alpha + P.sum(axis=1)
                o = o * alpha[:, None] + P8 @ V8
                if return_slack:
                    lo = decode_e4m3fn(encode_e4m3fn(y * (1 - TIE_WINDOW)))
                    hi = decode_e4m3fn(encode_e4m3fn(np.minimum(y * (1 + TIE_WINDOW), E4M3FN_MAX)))
                    sl = sl * alpha[:, None] + ((hi - lo) * 2.0 ** -P_SHIFT) @ np.abs(V8)
                    if tile_dot_rel > 0:
                        sl += tile_dot_rel * (P8[:, :, None] * np.abs(V8)[None]).max(axis=1)
                m = np.where(live, m_new, m)
            live = l > 0
            rows_out = q0 + sel
            out[rows_out, h] = np.where(live[:, None], o / np.where(live, l, 1.0)[:, None], 0.0)
            lse[rows_out, h] = np.where(live, m + np.log(np.where(live, l, 1.0)), -np.inf)
            slack[rows_out, h] = np.where(live[:, None], sl / np.where(live, l, 1.0)[:, None], 0.0)
    return (out, lse, slack) if return_slack else (out, lse)
