"""The fp8-MFMA decode (mla_decode_fwd_fp8mma: queries and P quantised to E4M3,
both contractions on fp8 matrix cores) against the fp64 oracle.

Two references:
  * the oracle on the E4M3 image of the queries (oracle.quantize_query_rows_e4m3,
    the rule the kernel applies): the only remaining approximation is P' =
    P_j * s_j in E4M3 with a power-of-two scale per (row, 32-key block). Round
    to nearest keeps a relative error <= 2^-4 for normal codes and an
    absolute one <= 2^-10 * 2^e <= 2^-17 * (block max) below them, so per
    element |O - O_q| <= 2^-4 * sum_j p_j |V_jd| + 2^-17 * sum_j bmax_j |v8_jd| / l
    (checked with a small allowance for fp32 accumulation); the LSE uses the
    unquantised P, so it matches the reference to fp32 accuracy;
  * the exact oracle: the query rounding moves each score by ~0.06 (natural
    log) on the normally distributed test data; O must stay within 15% of
    max|O| there (the measured error is ~6%).
"""
import numpy as np
import pytest
import torch

import oracle
import mla_decode_attention_amd as mla
from workloads import config, make_workload
from _gpu_util import to_device, reference

pytestmark = pytest.mark.gpu

O_TOL_EXACT = 0.15      # max|O - O_ref| / max|O_ref| against the exact oracle
LSE_TOL_Q = 2e-3        # |LSE - LSE_q| against the oracle on the quantised queries
SLACK = 1e-4            # fp32 accumulation allowance, relative to max|O_q|


def run_q8(w, split=True, num_units=None, min_tiles=0):
    d = to_device(w)
    plan = None
    if split:
        plan = mla.get_split_metadata(d["seqlens"], w.q_len, w.num_heads, num_units=num_units,
                                      min_tiles_per_unit=min_tiles)
    out, lse = mla.decode(d["q"], d["kv"], d["block_table"], d["seqlens"], w.softmax_scale,
                          kv_scale=d["kv_scale"], plan=plan, fp8_mma=True)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def _o_bound(w, q_vals):
    """Per-element bound on |O - O_q| from the E4M3 rounding of P' (see the
    module docstring), [B, s, H, 512]."""
    B, s, H, _ = w.q_bits.shape
    bound = np.zeros((B, s, H, 512))
    for b in range(B):
        L = int(w.seqlens[b])
        if L == 0:
            continue
        rows = oracle.sequence_rows(w.cache, w.block_table[b], L, w.kv_dtype, w.kv_scale)
        sc = np.array([w.kv_scale[w.block_table[b][j // 64], j % 64] for j in range(L)], np.float64)
        v8 = np.abs(rows[:, :512] / sc[:, None])
        qr = q_vals[b].reshape(s * H, 576)
        vis = oracle.visible_counts(L, s, H)
        z = w.softmax_scale * (qr @ rows.T)
        z = np.where(np.arange(L)[None, :] < vis[:, None], z, -np.inf)
        m = np.max(z, axis=1, keepdims=True)
        m = np.where(np.isfinite(m), m, 0.0)
        pw = np.exp(z - m)
        l = pw.sum(axis=1, keepdims=True)
        l = np.where(l > 0, l, 1.0)
        pp = pw * sc[None, :]                         # P' up to the common factor
        nb = (L + 31) // 32
        bm = np.zeros_like(pp)
        for k in range(nb):
            bm[:, 32 * k:32 * k + 32] = pp[:, 32 * k:32 * k + 32].max(axis=1, keepdims=True)
        bound[b] = ((2.0 ** -4 * pp @ v8 + 2.0 ** -17 * bm @ v8) / l).reshape(s, H, 512)
    return bound


def check(w, out, lse, what):
    q_vals = oracle.quantize_query_rows_e4m3(w.q_bits)
    qo, ql = oracle.mla_decode(w.q_bits, w.cache, w.block_table, w.seqlens, w.softmax_scale, w.kv_dtype,
                               w.kv_scale, q_values=q_vals)
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    neg = np.isneginf(ql)
    assert np.array_equal(np.isneginf(lse), neg), f"{what}: -inf LSE pattern differs"
    live = ~neg
    if not live.any():
        assert np.all(out == 0)
        return
    lerr = float(np.max(np.abs(lse[live] - ql[live])))
    assert lerr <= LSE_TOL_Q, f"{what}: LSE err {lerr:.3e} vs the quantised-query oracle"
    bound = _o_bound(w, q_vals) + SLACK * float(np.max(np.abs(qo)))
    excess = np.abs(out - qo) - bound
    assert np.all(excess <= 0), f"{what}: O off the rounding bound by {float(excess.max()):.3e}"
    ref_out, _ = reference(w)
    err = float(np.max(np.abs(out - ref_out)))
    scale = float(np.max(np.abs(ref_out)))
    assert err <= O_TOL_EXACT * scale, f"{what}: O err {err:.3e} vs max|O| {scale:.3e} (exact oracle)"


@pytest.mark.parametrize("split", [False, True])
def test_fp8_config_small(split):
    w = config("fp8", small=True, seed=1)
    out, lse = run_q8(w, split=split)
    check(w, out, lse, f"fp8 small split={split}")


@pytest.mark.parametrize("H,s", [(16, 1), (16, 2), (64, 3), (128, 1), (128, 2)])
@pytest.mark.parametrize("split", [False, True])
def test_shapes_and_tails(H, s, split):
    """Row counts below, at and above one 64-row block; lengths with ragged
    last pages (NaN-poisoned slots past each sequence), one-key sequences."""
    lens = [1, 63, 64, 65, 300, 1000]
    lens = [L for L in lens if L >= s] + [s]
    w = make_workload("q8", len(lens), H, s, lens, kv_dtype="fp8_e4m3", seed=40 + H + s)
    out, lse = run_q8(w, split=split, num_units=9, min_tiles=1)
    check(w, out, lse, f"H={H} s={s} split={split}")


def test_empty_sequences():
    lens = [0, 300, 0, 5]
    w = make_workload("q8-empty", len(lens), 128, 2, lens, kv_dtype="fp8_e4m3", seed=8)
    for split in (False, True):
        out, lse = run_q8(w, split=split, num_units=5, min_tiles=1)
        check(w, out, lse, f"empty split={split}")


@pytest.mark.parametrize("H,s", [(16, 2), (128, 2)])
def test_rising_scores(H, s):
    """Scores climbing through the sequence: the running max moves mid-unit."""
    from test_gpu_parity import _ramp_cache
    lens = [1000, 700, 130, 64]
    w = _ramp_cache(make_workload("q8-ramp", len(lens), H, s, lens, kv_dtype="fp8_e4m3", seed=3 + H), 6.0, 5)
    out, lse = run_q8(w, split=True, num_units=7, min_tiles=1)
    check(w, out, lse, f"ramp H={H} s={s}")


def test_close_to_exact_path():
    """The fp8-MFMA output against the exact fp8 path on the same inputs."""
    w = config("fp8", small=True, seed=2)
    d = to_device(w)
    plan = mla.get_split_metadata(d["seqlens"], w.q_len, w.num_heads)
    exact, le = mla.decode(d["q"], d["kv"], d["block_table"], d["seqlens"], w.softmax_scale,
                           kv_scale=d["kv_scale"], plan=plan)
    q8, lq = mla.decode(d["q"], d["kv"], d["block_table"], d["seqlens"], w.softmax_scale,
                        kv_scale=d["kv_scale"], plan=plan, fp8_mma=True)
    torch.cuda.synchronize()
    exact, q8 = exact.cpu().numpy(), q8.cpu().numpy()
    rms = np.linalg.norm(q8 - exact) / np.linalg.norm(exact)
    assert rms <= 0.08, rms
    assert float((lq - le).abs().max()) <= 0.3


def test_bf16_cache_rejected():
    w = make_workload("q8-bf16", 2, 16, 1, [100, 64], kv_dtype="bf16", seed=1)
    d = to_device(w)
    with pytest.raises(mla.MLAError):
        mla.decode(d["q"], d["kv"], d["block_table"], d["seqlens"], w.softmax_scale, fp8_mma=True)
