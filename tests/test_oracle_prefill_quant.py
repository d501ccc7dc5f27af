"""Pins of the quantised prefill oracle (INT8 Q.K^T, FP8 P.V): each test
checks it against something other than itself -- properties the quantisers
must have by definition, a brute-force minimum, the FP8 cast of torch, exact
agreement with the unquantised oracle on inputs the formats represent
exactly, a one-key closed form, and the error budget derived from the
rounding steps."""
import math

import numpy as np
import pytest

import oracle
from oracle import prefill_quant as pq
from workloads import make_prefill_workload
from _prefill_quant_budget import budget


def _bits(x):
    """float -> bf16 bits (inputs here are exact bf16 values)."""
    f = np.asarray(x, dtype=np.float32)
    b = f.view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "value not exactly representable in bf16"
    return (b >> 16).astype(np.uint16)


# ----------------------------------------------------------------- INT8 blocks
def test_int8_block_properties():
    rng = np.random.default_rng(1)
    for _ in range(200):
        n = int(rng.integers(1, 300))
        x = (rng.standard_normal(n) * 10.0 ** rng.uniform(-30, 30)).astype(np.float32)
        codes, s = pq.quantize_int8(x)
        amax = np.abs(x).max()
        assert s.dtype == np.float32 and codes.dtype == np.int8
        assert np.all(np.abs(codes.astype(np.int64)) <= 127)
        # the largest magnitude maps to +-127, with its sign
        i = int(np.argmax(np.abs(x)))
        assert codes[i] == (127 if x[i] > 0 else -127)
        # every code is the nearest multiple of the step (half a step, plus the
        # fp32 rounding of amax / 127 and 127 / amax)
        err = np.abs(x.astype(np.float64) - codes.astype(np.float64) * np.float64(s))
        assert np.all(err <= 0.5 * float(s) * (1 + 1e-5) + 1e-6 * float(s))
        assert math.isclose(float(s), float(amax) / 127, rel_tol=1e-6)


def test_int8_zero_block_and_axes():
    codes, s = pq.quantize_int8(np.zeros(7, np.float32))
    assert np.all(codes == 0) and s == np.float32(1)
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 3, 9)).astype(np.float32)
    x[2, 1] = 0
    codes, s = pq.quantize_int8(x, axis=2)
    assert s.shape == (5, 3)
    for i in range(5):
        for j in range(3):
            c1, s1 = pq.quantize_int8(x[i, j])
            assert np.array_equal(codes[i, j], c1) and s[i, j] == s1
    codes, s = pq.quantize_int8(x, axis=(0, 2))
    assert s.shape == (3,)
    for j in range(3):
        c1, s1 = pq.quantize_int8(x[:, j])
        assert np.array_equal(codes[:, j], c1) and s[j] == s1


# ------------------------------------------------------ E8M0 exponent, FP8 V
def test_e8m0_exponent_is_the_smallest_power_that_fits():
    rng = np.random.default_rng(3)
    vals = list(rng.uniform(0, 1, 2000) * 10.0 ** rng.integers(-40, 39, 2000))
    vals += [448.0 * 2.0 ** k for k in range(-20, 20)]
    vals += [np.nextafter(448.0 * 2.0 ** k, np.inf) for k in range(-20, 20)]
    vals += [np.nextafter(448.0 * 2.0 ** k, 0) for k in range(-20, 20)]
    vals += [2.0 ** -133, 1e-40, 3.0e38]
    e = pq.e8m0_exponent(np.array(vals))
    for a, k in zip(vals, e):
        k = int(k)
        assert -127 <= k <= 127
        if a == 0:
            assert k == 0
            continue
        if k > -127:
            assert a <= 448.0 * 2.0 ** k and not (a <= 448.0 * 2.0 ** (k - 1)), (a, k)
        else:
            assert a <= 448.0 * 2.0 ** k
    assert int(pq.e8m0_exponent(0.0)) == 0


def test_pow2_e4m3_matches_torch_cast():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(4)
    x = (rng.standard_normal(5000) * 3).astype(np.float32)
    x[:10] = [0, -0.0, 28, -28, 27.99, 1e-6, -1e-6, 0.0009765625, 3.5, -3.25]
    e = int(pq.e8m0_exponent(np.abs(x).max()))
    codes = pq.quantize_e4m3_pow2(x, e)
    y = np.ldexp(x.astype(np.float64), -e)
    ref = torch.from_numpy(y.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)
    back = oracle.decode_e4m3fn(codes) * 2.0 ** e
    step = np.ldexp(1.0, np.floor(np.log2(np.maximum(np.abs(y), 2.0 ** -6))).astype(int) - 3) * 2.0 ** e
    assert np.all(np.abs(back - x) <= 0.5 * step + 1e-30)


# ----------------------------------------------- exact when the formats are
def _representable_case(seqs, H, seed):
    """Inputs the quantised formats hold exactly and whose softmax weights are
    powers of two: q has 127/128 in feature 0 (so its INT8 step is 2^-7),
    every key has 127/128 in rope feature 63 (the tile steps are 2^-7) and an
    integer multiple of 2^-7 in its head's feature 0, so the score of key j is
    c_j * ln 2 for softmax_scale = 2^14 ln 2 / 127, and P = 2^(c_j - max) is an
    E4M3 value. V entries are E4M3 values times 2^-4 with one 28 = 448 * 2^-4
    per 32-key block and feature, so the V scale is 2^-4 and the codes exact."""
    rng = np.random.default_rng(seed)
    Tk = sum(L for _, L in seqs)
    Tq = sum(N for N, _ in seqs)
    q = np.zeros((Tq, H, 192), np.float32)
    q[:, :, 0] = 127 / 128
    kn = np.zeros((Tk, H, 128), np.float32)
    kr = np.zeros((Tk, 64), np.float32)
    kr[:, 63] = 127 / 128
    v = np.zeros((Tk, H, 128), np.float32)
    e4 = oracle.decode_e4m3fn(np.arange(0x78, dtype=np.uint8))      # 0 .. 240, all finite
    off = 0
    for N, L in seqs:
        # scores rise along the sequence (the running max moves up across
        # tiles) with noise, all within 16 of the final max
        c = np.clip(np.floor(np.arange(L) * 12 / max(L, 1)) - rng.integers(0, 5, (H, L)), -4, 12) - 4
        kn[off:off + L, :, 0] = (c.T / 128).astype(np.float32)
        vals = e4[rng.integers(0, len(e4), (L, H, 128))] * rng.choice([-1, 1], (L, H, 128)) / 16
        vals[::32] = 28.0 * rng.choice([-1, 1], vals[::32].shape)
        v[off:off + L] = vals
        off += L
    cu_q = np.concatenate([[0], np.cumsum([N for N, _ in seqs])]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum([L for _, L in seqs])]).astype(np.int32)
    scale = 2.0 ** 14 * math.log(2) / 127
    return _bits(q), _bits(kn), _bits(kr), _bits(v), cu_q, cu_k, scale


@pytest.mark.parametrize("seqs", [[(150, 150), (40, 100)], [(1, 1), (70, 200), (33, 33)]])
def test_exact_on_representable_inputs(seqs):
    q, kn, kr, v, cu_q, cu_k, scale = _representable_case(seqs, 2, seed=len(seqs))
    o, l = pq.prefill_quant(q, kn, kr, v, cu_q, cu_k, scale)
    oe, le = oracle.mla_prefill(q, kn, kr, v, cu_q, cu_k, scale)
    assert np.allclose(o, oe, rtol=1e-12, atol=1e-12 * np.abs(oe).max())
    assert np.allclose(l, le, rtol=0, atol=1e-9)
    # and the quantised keys / values are exactly the inputs
    kv = pq.quantize_kv(kn, kr, v, cu_k)
    assert all(np.all(s["k_scale"] == np.float32(2.0 ** -7)) for s in kv)
    assert all(np.all(s["v_exp"] == -4) for s in kv)


def test_one_visible_key_closed_form():
    """A row that sees one key has P = 1 (code 2^8 exactly): O is the
    dequantised V row and LSE is its dequantised score."""
    w = make_prefill_workload("one", [1, 3], [1, 5], 4, seed=7)
    o, l = pq.prefill_quant(w.q_bits, w.k_nope_bits, w.k_rope_bits, w.v_bits, w.cu_q, w.cu_k, w.softmax_scale)
    qc, qs = pq.quantize_query(w.q_bits)
    kv = pq.quantize_kv(w.k_nope_bits, w.k_rope_bits, w.v_bits, w.cu_k)
    s, row = kv[0], 0                    # sequence 0: one query over one key
    for h in range(4):
        vdeq = oracle.decode_e4m3fn(s["v_codes"][0, h]) * np.ldexp(1.0, s["v_exp"][0, h])
        assert np.array_equal(o[row, h], vdeq)
        dot = float(np.dot(qc[row, h].astype(np.int64), s["k_codes"][0, h].astype(np.int64)))
        z = dot * float(qs[row, h]) * float(s["k_scale"][0, h]) * w.softmax_scale
        assert math.isclose(l[row, h], z, rel_tol=1e-12, abs_tol=1e-12)


def test_empty_rows_and_sequences():
    w = make_prefill_workload("e", [0, 2], [5, 2], 2, seed=8)
    o, l = pq.prefill_quant(w.q_bits, w.k_nope_bits, w.k_rope_bits, w.v_bits, w.cu_q, w.cu_k, w.softmax_scale)
    assert o.shape == (2, 2, 128) and np.all(np.isfinite(o))


# --------------------------------------------------------- error budget
@pytest.mark.parametrize("seed,q_lens,k_lens", [(3, [300, 129, 64, 1], [300, 129, 64, 1]),
                                                (5, [40, 100], [200, 100])])
def test_within_error_budget_of_exact_attention(seed, q_lens, k_lens):
    w = make_prefill_workload("b", q_lens, k_lens, 16, seed=seed)
    args = (w.q_bits, w.k_nope_bits, w.k_rope_bits, w.v_bits, w.cu_q, w.cu_k, w.softmax_scale)
    oe, le = oracle.mla_prefill(*args)
    o, l = pq.prefill_quant(*args)
    ob, lb = budget(*args)
    assert np.all(np.abs(o - oe) <= ob)
    assert np.all(np.abs(l - le) <= lb)
    # and the quantisation is really there (not the unquantised path)
    assert np.abs(o - oe).max() > 1e-3 * np.abs(oe).max()


def test_slack_marks_only_near_ties():
    w = make_prefill_workload("s", [64], [64], 2, seed=9)
    args = (w.q_bits, w.k_nope_bits, w.k_rope_bits, w.v_bits, w.cu_q, w.cu_k, w.softmax_scale)
    o, l, slack = pq.prefill_quant(*args, return_slack=True)
    o2, l2 = pq.prefill_quant(*args)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)
    assert np.all(slack >= 0) and slack.max() < 0.1 * np.abs(o).max()
    assert slack[0].max() == 0          # row 0: P = 1 exactly, no tie
