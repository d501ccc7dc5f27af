"""Per-element error budget of the quantised prefill against exact attention.

Derived from the rounding steps of the method (INT8 Q and K with per-block
scales, FP8 E4M3 V with power-of-two scales per 32-key block and feature, FP8
P), not from any implementation of it: each rounding error is modelled as
independent and uniform over its rounding step (standard deviation
step / sqrt(12)), and the error of a row's output is the first-order
propagation of those errors through the softmax and the weighted sum:

  dS_j   = softmax_scale * sum_e (q_e dk_je + k_je dq_e)           (INT8 codes)
  dO_d   = sum_j p_j [ dS_j (V_jd - O_d) + dV_jd + V_jd dP_j / P_j ]
  dLSE   = sum_j p_j dS_j

with p the exact softmax and O the exact output. The query's rounding errors
dq_e are shared by all keys of the row, so their part of the variance is
taken over the sums they multiply (sum_j p_j (V_jd - O_d) k_je for O,
sum_j p_j k_je for LSE); the others are independent. The budget is six standard
deviations of that sum plus an fp32 floor. Every input of the computation is
taken from the bf16 inputs directly (scales recomputed here from the block
maxima), so a mistake in a quantiser shows up as a violation.
"""
from __future__ import annotations

import numpy as np

SIGMAS = 6.0


def _bf16(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _e4m3_step(y):
    """Rounding step of E4M3FN at |y| (y in [0, 448]): 2^(floor(log2 y) - 3) for
    normal values (y >= 2^-6), 2^-9 below."""
    y = np.maximum(np.abs(y), 2.0 ** -6)
    return np.ldexp(1.0, np.floor(np.log2(y)).astype(np.int64) - 3)


def budget(q_bits, k_nope_bits, k_rope_bits, v_bits, cu_q, cu_k, softmax_scale, rows=None):
    """Returns (o_budget [Tq, H, 128], lse_budget [Tq, H]); rows: optional
    {b: query indices} (other rows get budget 0)."""
    q, kn, kr, v = _bf16(q_bits), _bf16(k_nope_bits), _bf16(k_rope_bits), _bf16(v_bits)
    Tq, H, _ = q.shape
    Dv = v.shape[2]
    ob = np.zeros((Tq, H, Dv))
    lb = np.zeros((Tq, H))
    for b in range(len(cu_q) - 1):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        k0, k1 = int(cu_k[b]), int(cu_k[b + 1])
        N, L = q1 - q0, k1 - k0
        if N == 0:
            continue
        sel = np.arange(N) if rows is None or b not in rows else np.asarray(rows[b])
        keys = np.arange(L)
        vis = keys[None, :] <= (L - N + sel)[:, None]
        for h in range(H):
            Q = q[q0 + sel, h]                                          # [n, 192]
            K = np.concatenate([kn[k0:k1, h], kr[k0:k1]], axis=1)       # [L, 192]
            V = v[k0:k1, h]                                             # [L, 128]
            sq = np.abs(Q).max(axis=1) / 127.0                          # per-row INT8 step
            sk = np.array([np.abs(K[a:a + 64]).max() / 127.0 for a in range(0, L, 64)])
            sk = np.repeat(sk, 64)[:L]                                  # per-key INT8 step of its tile
            S = softmax_scale * (Q @ K.T)
            S = np.where(vis, S, -np.inf)
            mx = S.max(axis=1, keepdims=True)
            e = np.exp(S - mx)
            p = e / e.sum(axis=1, keepdims=True)
            O = p @ V
            # key rounding (independent per key and feature): variance of its part of dS_j
            varSk = softmax_scale ** 2 * (Q ** 2).sum(axis=1)[:, None] * (sk ** 2 / 12.0)[None, :]
            # query rounding (shared by the row's keys): sum_e var(dq_e) C_e^2
            vq = softmax_scale ** 2 * sq ** 2 / 12.0                    # [n]
            C = np.matmul((p[:, :, None] * V[None]).transpose(0, 2, 1), K) - O[:, :, None] * (p @ K)[:, None, :]
            # V rounding: power-of-two scale per 32-key block and feature
            amax = np.stack([np.abs(V[a:a + 32]).max(axis=0) for a in range(0, L, 32)])   # [G, 128]
            with np.errstate(divide="ignore"):
                ev = np.where(amax > 0, np.ceil(np.log2(np.where(amax > 0, amax, 1.0) / 448.0)), 0.0)
            scale_v = np.repeat(np.ldexp(1.0, ev.astype(np.int64)), 32, axis=0)[:L]        # [L, 128]
            varV = (_e4m3_step(V / scale_v) * scale_v) ** 2 / 12.0
            # P rounding: E4M3 of P * 2^8 with P = exp(S - running max) <= 1;
            # relative step bounded by the step at P itself
            P256 = np.ldexp(np.where(vis, e, 0.0), 8)
            varPrel = np.where(P256 > 0, (_e4m3_step(P256) / np.where(P256 > 0, P256, 1.0)) ** 2 / 12.0, 0.0)
            p2 = p ** 2
            a = p2 * varSk
            varO = (a @ V ** 2 - 2 * O * (a @ V) + O ** 2 * a.sum(axis=1, keepdims=True)
                    + vq[:, None] * (C ** 2).sum(axis=2)
                    + p2 @ varV + (p2 * varPrel) @ V ** 2)
            varL = a.sum(axis=1) + vq * ((p @ K) ** 2).sum(axis=1)
            ob[q0 + sel, h] = SIGMAS * np.sqrt(np.maximum(varO, 0.0)) + 1e-6 * np.abs(O).max()
            lb[q0 + sel, h] = SIGMAS * np.sqrt(varL) + 1e-5
    return ob, lb
