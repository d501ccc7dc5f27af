"""Parity of the quantised prefill (INT8 Q.K^T, FP8 P.V) through the C-ABI.

  * The K/V quantiser is integer work: its INT8 and E4M3 codes, E8M0 bytes and
    fp32 K scales must equal the oracle's bit for bit.
  * The attention follows the same steps as the oracle's quantised prefill;
    the two differ by fp32 against fp64 arithmetic, and where that moves a P
    value across an E4M3 rounding tie the code may differ; and the FP8 MFMA
    sums its 64 products of a tile more coarsely than fp32 (measured on
    gfx950: within 2^-11 of the largest product's magnitude for operands over
    the whole E4M3 range). The tolerance is an fp32 floor plus the oracle's
    slack for tie flips and for a tile sum error of TILE_DOT_REL times its
    largest term; test_tile_sum_rounding_bound checks that bound on inputs
    where it is the only source of error.
  * Against exact attention (the unquantised oracle) every element must stay
    within the error budget derived from the rounding steps.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import prefill_quant as pq
import mla_decode_attention_amd as mla
from workloads import make_prefill_workload, prefill_config
from _prefill_quant_budget import budget

pytestmark = pytest.mark.gpu

O_FLOOR = 2e-5        # of max|O| of the row: fp32 accumulation over the keys
LSE_TOL = 1e-4
TILE_DOT_REL = 2.0 ** -10   # FP8 MFMA sum of a tile, relative to its largest term


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _inputs(w):
    return (_dev(w.q_bits), _dev(w.k_nope_bits), _dev(w.k_rope_bits), _dev(w.v_bits),
            torch.from_numpy(w.cu_q).cuda(), torch.from_numpy(w.cu_k).cuda())


def run(w, qkv=None):
    q, kn, kr, v, cq, ck = _inputs(w)
    out, lse = mla.prefill_quant(q, kn, kr, v, cq, ck, int(max(1, w.q_lens.max())), w.softmax_scale, qkv=qkv)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


# ----------------------------------------------------- quantised K/V layout
def _layout_index():
    f, l, i = np.meshgrid(np.arange(12), np.arange(64), np.arange(16), indexing="ij")
    k_key, k_feat = 32 * (f // 6) + l % 32, 32 * (f % 6) + 16 * (l // 32) + i
    g, l2, i2 = np.meshgrid(np.arange(8), np.arange(64), np.arange(16), indexing="ij")
    q = g % 2
    v_key, v_feat = 32 * q + 8 * (i2 // 4) + 4 * (l2 // 32) + i2 % 4, 32 * (g // 2) + l2 % 32
    return k_key, k_feat, v_key, v_feat


def unpack_qkv(buf, cu_k, H):
    """The quantised buffer (layout of include/mla_decode.h) -> per sequence
    k_codes [L, H, 192] int8, k_scale [T, H] f32, v_codes [L, H, 128] u8,
    v_exp [G, H, 128]."""
    B = len(cu_k) - 1
    Tk = int(cu_k[-1])
    n = (Tk // 64 + B) * H
    r256 = lambda x: (x + 255) // 256 * 256
    o_v8 = r256(n * 12288)
    o_vs = o_v8 + r256(n * 8192)
    o_ks = o_vs + r256(n * 256)
    k8 = buf[:n * 12288].view(np.int8).reshape(n, 12, 64, 16)
    v8 = buf[o_v8:o_v8 + n * 8192].reshape(n, 8, 64, 16)
    vs = buf[o_vs:o_vs + n * 256].reshape(n, 64, 4)
    ks = buf[o_ks:o_ks + n * 4].view(np.float32)
    k_key, k_feat, v_key, v_feat = _layout_index()
    seqs = []
    for b in range(B):
        L = int(cu_k[b + 1] - cu_k[b])
        nt = -(-L // 64)
        base = int(cu_k[b]) // 64 + b
        kc = np.zeros((nt * 64, H, 192), np.int8)
        vc = np.zeros((nt * 64, H, 128), np.uint8)
        kscale = np.zeros((nt, H), np.float32)
        vexp = np.zeros((2 * nt, H, 128), np.int64)
        for t in range(nt):
            for h in range(H):
                rec = (base + t) * H + h
                kc[64 * t + k_key, h, k_feat] = k8[rec]
                vc[64 * t + v_key, h, v_feat] = v8[rec]
                kscale[t, h] = ks[rec]
                for g in range(4):
                    vexp[2 * t + np.arange(64) // 32, h, 32 * g + np.arange(64) % 32] = vs[rec, :, g].astype(np.int64) - 127
        seqs.append(dict(k_codes=kc, k_scale=kscale, v_codes=vc, v_exp=vexp, L=L))
    return seqs


def check_codes(w, H):
    q, kn, kr, v, cq, ck = _inputs(w)
    buf = mla.prefill_quantize_kv(kn, kr, v, ck)
    torch.cuda.synchronize()
    got = unpack_qkv(buf.cpu().numpy(), w.cu_k, H)
    ref = pq.quantize_kv(w.k_nope_bits, w.k_rope_bits, w.v_bits, w.cu_k)
    for b, (g, r) in enumerate(zip(got, ref)):
        L = g["L"]
        assert np.array_equal(g["k_codes"][:L], r["k_codes"]), f"seq {b}: INT8 K codes"
        assert np.all(g["k_codes"][L:] == 0), f"seq {b}: K tail codes"
        assert np.array_equal(g["k_scale"].view(np.uint32), r["k_scale"].view(np.uint32)), f"seq {b}: K scales"
        assert np.array_equal(g["v_codes"][:L], r["v_codes"]), f"seq {b}: E4M3 V codes"
        assert np.all(g["v_codes"][L:] == 0), f"seq {b}: V tail codes"
        G = r["v_exp"].shape[0]
        assert np.array_equal(g["v_exp"][:G], r["v_exp"]), f"seq {b}: V exponents"
        assert np.all(g["v_exp"][G:] == 0), f"seq {b}: exponents of empty blocks"
    return buf


@pytest.mark.parametrize("q_lens,k_lens,H", [([300, 129, 64, 1], [300, 129, 64, 1], 16),
                                             ([40, 100, 3], [200, 100, 33], 4),
                                             ([1, 65, 64], [1, 65, 128], 2)])
def test_quantised_kv_matches_oracle_bitwise(q_lens, k_lens, H):
    w = make_prefill_workload("qkv", q_lens, k_lens, H, seed=sum(k_lens))
    check_codes(w, H)


# ----------------------------------------------------------------- attention
def check_vs_quant_oracle(out, lse, w, rows=None, what=""):
    args = (w.q_bits, w.k_nope_bits, w.k_rope_bits, w.v_bits, w.cu_q, w.cu_k, w.softmax_scale)
    ro, rl, slack = pq.prefill_quant(*args, rows=rows, return_slack=True, tile_dot_rel=TILE_DOT_REL)
    sel = np.zeros(ro.shape[0], bool)
    if rows is None:
        sel[:] = True
    else:
        for b, r in rows.items():
            sel[int(w.cu_q[b]) + np.asarray(r)] = True
    o, l = out[sel], lse[sel]
    ro, rl, slack = ro[sel], rl[sel], slack[sel]
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    tol = O_FLOOR * np.abs(ro).max(axis=2, keepdims=True) + 1.01 * slack + 1e-30
    bad = np.abs(o - ro) > tol
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements off; worst excess "
                           f"{float(np.max(np.abs(o - ro) - tol)):.3e}")
    neg = np.isneginf(rl)
    assert np.array_equal(np.isneginf(l), neg), f"{what}: -inf LSE pattern differs"
    if (~neg).any():
        assert float(np.max(np.abs(l[~neg] - rl[~neg]))) <= LSE_TOL, f"{what}: LSE"
    return float(np.max(np.abs(o - ro) / np.maximum(np.abs(ro).max(axis=2, keepdims=True), 1e-30)))


@pytest.mark.parametrize("q_lens,k_lens,H", [([300, 129, 64, 1], [300, 129, 64, 1], 16),
                                             ([1, 127, 128, 129, 200, 3, 64], [1, 127, 128, 129, 333, 70, 64], 8),
                                             ([40, 100], [200, 100], 128)])
def test_matches_quant_oracle_and_budget(q_lens, k_lens, H):
    w = make_prefill_workload("pq", q_lens, k_lens, H, seed=H + len(q_lens))
    out, lse = run(w)
    check_vs_quant_oracle(out, lse, w, what=f"H={H}")
    args = (w.q_bits, w.k_nope_bits, w.k_rope_bits, w.v_bits, w.cu_q, w.cu_k, w.softmax_scale)
    ro, rl = oracle.mla_prefill(*args)
    ob, lb = budget(*args)
    assert np.all(np.abs(out - ro) <= ob), "outside the error budget against exact attention"
    assert np.all(np.abs(lse - rl) <= lb), "LSE outside its budget against exact attention"


def test_tile_sum_rounding_bound():
    """Inputs the quantised formats hold exactly, with power-of-two softmax
    weights (the oracle pins' construction) and V over a wide range of
    magnitudes: the quantised steps then reproduce exact attention, and all
    that separates the kernel from it is the rounding of its FP8 tile sums,
    which must stay within TILE_DOT_REL of each tile's largest term."""
    from test_oracle_prefill_quant import _representable_case
    seqs = [(150, 150), (40, 100), (1, 1), (70, 200)]
    H = 4
    q, kn, kr, v, cu_q, cu_k, scale = _representable_case(seqs, H, seed=11)
    w = make_prefill_workload("rep", [N for N, _ in seqs], [L for _, L in seqs], H, seed=0)
    w.q_bits[...], w.k_nope_bits[...], w.k_rope_bits[...], w.v_bits[...] = q, kn, kr, v
    w.softmax_scale = scale
    out, lse = run(w)
    ro, rl = oracle.mla_prefill(q, kn, kr, v, cu_q, cu_k, scale)
    _, _, slack = pq.prefill_quant(q, kn, kr, v, cu_q, cu_k, scale, return_slack=True, tile_dot_rel=TILE_DOT_REL)
    tol = 1e-6 * np.abs(ro).max(axis=2, keepdims=True) + slack
    assert np.all(np.abs(out - ro) <= tol)
    assert np.max(np.abs(lse - rl)) <= LSE_TOL


@pytest.mark.parametrize("name", ["prefill", "extend"])
def test_small_configs(name):
    w = prefill_config(name, small=True, seed=2)
    out, lse = run(w)
    check_vs_quant_oracle(out, lse, w, what=name)


def test_empty_sequence_rows_untouched():
    w = make_prefill_workload("empty", [5, 0, 7], [9, 4, 7], 4, seed=3)
    q, kn, kr, v, cq, ck = _inputs(w)
    out = torch.full((12, 4, 128), 7.0, device="cuda")
    lse = torch.full((12, 4), 7.0, device="cuda")
    mla.prefill_quant(q, kn, kr, v, cq, ck, 7, w.softmax_scale, out=out, lse=lse)
    torch.cuda.synchronize()
    check_vs_quant_oracle(out.cpu().numpy(), lse.cpu().numpy(), w, what="empty sequence")


def test_reuse_quantised_kv_and_run_to_run_bitwise():
    w = prefill_config("extend", small=True, seed=4)
    q, kn, kr, v, cq, ck = _inputs(w)
    qkv = mla.prefill_quantize_kv(kn, kr, v, ck)
    mq = int(w.q_lens.max())
    o1, l1 = mla.prefill_quant(q, kn, kr, v, cq, ck, mq, w.softmax_scale, qkv=qkv, quantize=False)
    o2, l2 = mla.prefill_quant(q, kn, kr, v, cq, ck, mq, w.softmax_scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_short_buffer_rejected():
    w = make_prefill_workload("short", [4], [4], 2, seed=5)
    q, kn, kr, v, cq, ck = _inputs(w)
    small = torch.empty(mla.prefill_quant_kv_bytes(1, 4, 2) - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(mla.MLAError, match="WORKSPACE"):
        mla.prefill_quantize_kv(kn, kr, v, ck, qkv=small)


def test_full_size_sampled_rows():
    """The benchmark's workload (2 x 8192 tokens, H = 16): every quantised code
    bit for bit, and sampled rows of every query block region against the
    oracle's quantised steps."""
    w = prefill_config("prefill", seed=0)
    H = w.num_heads
    print(f"[full-size quantised prefill] q_lens={list(w.q_lens)} H={H}", flush=True)
    buf = check_codes(w, H)
    out, lse = run(w, qkv=buf)
    rng = np.random.default_rng(0)
    rows = {}
    for b, N in enumerate(w.q_lens):
        N = int(N)
        pick = {0, 1, 63, 64, 127, 128, 129, N // 2, N - 2, N - 1}
        pick |= set(int(x) for x in rng.integers(0, N, 6))
        rows[b] = sorted(x for x in pick if 0 <= x < N)
    check_vs_quant_oracle(out, lse, w, rows=rows, what="full size")


def test_negative_softmax_scale():
    """A negative scale enters as negated query codes (the INT8 rule is odd),
    so the result matches the oracle's steps with the scale as given."""
    w = make_prefill_workload("neg", [1, 127, 129, 40], [1, 127, 129, 200], 4, seed=6)
    w.softmax_scale = -0.11
    out, lse = run(w)
    check_vs_quant_oracle(out, lse, w, what="negative scale")
