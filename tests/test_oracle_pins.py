"""Pins for the CPU oracle, each independent of the oracle's own code.

Closed forms, invariants, a pure-Python brute force, library cross-checks and
hand-worked fixtures (tests/golden). No GPU needed.
"""
import json
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from workloads import make_workload, f32_to_bf16_bits, PAGE_TOKENS, config

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
D_QK, D_V = 576, 512


# ----------------------------------------------------------------- helpers

def _bits(x):
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _py_bf16(bits):
    """bf16 bits -> float via struct (independent of the oracle's numpy path)."""
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def _py_e4m3(code):
    """E4M3FN via math.ldexp, written independently of the oracle's table."""
    code = int(code)
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 15
    m = code & 7
    if e == 15 and m == 7:
        return math.nan
    if e == 0:
        return s * math.ldexp(m, -9)
    return s * math.ldexp(8 + m, e - 10)


def brute_force(w, scale=None):
    """Pure-Python loops + math.fsum: the definition, one output at a time."""
    scale = w.softmax_scale if scale is None else scale
    B, s, H, _ = w.q_bits.shape
    out = np.zeros((B, s, H, D_V))
    lse = np.zeros((B, s, H))
    for b in range(B):
        L = int(w.seqlens[b])
        rows = []
        for j in range(L):
            page = int(w.block_table[b][j // 64])
            slot = j % 64
            if w.kv_dtype == "bf16":
                rows.append([_py_bf16(v) for v in w.cache[page, slot]])
            else:
                sc = float(w.kv_scale[page, slot])
                rows.append([_py_e4m3(v) * sc for v in w.cache[page, slot]])
        for i in range(s):
            n = max(0, min(L, L - s + i + 1))
            for h in range(H):
                q = [_py_bf16(v) for v in w.q_bits[b, i, h]]
                if n == 0:
                    lse[b, i, h] = -math.inf
                    continue
                z = [scale * math.fsum(q[d] * rows[j][d] for d in range(D_QK)) for j in range(n)]
                m = max(z)
                e = [math.exp(x - m) for x in z]
                tot = math.fsum(e)
                for d in range(D_V):
                    out[b, i, h, d] = math.fsum(e[j] * rows[j][d] for j in range(n)) / tot
                lse[b, i, h] = m + math.log(tot)
    return out, lse


def run_oracle(w, **kw):
    return oracle.mla_decode(w.q_bits, w.cache, w.block_table, w.seqlens,
                             kw.get("scale", w.softmax_scale), w.kv_dtype, w.kv_scale)


def _tiny(seed, B=2, H=3, s=2, seqlens=(7, 3), kv="bf16", table="shuffled"):
    return make_workload("tiny-bf", B, H, s, list(seqlens), kv_dtype=kv, seed=seed, table=table)


# ----------------------------------------------------------------- formats

def test_bf16_decode_all_codes_vs_torch():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_bits_to_f64(codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_e4m3_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode_e4m3fn(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_e4m3_golden_codes():
    with open(os.path.join(GOLDEN, "e4m3fn_codes.json")) as f:
        g = json.load(f)["codes"]
    for code, text in g.items():
        v = oracle.e4m3fn_value(int(code, 16))
        if text == "nan":
            assert math.isnan(v)
            continue
        sign = -1.0 if text.startswith("-") else 1.0
        t = text.lstrip("-")
        if "*" in t:
            a, b = t.split("*")
            exp = float(a) * 2.0 ** int(b.split("^")[1])
        elif "^" in t:
            exp = 2.0 ** int(t.split("^")[1])
        else:
            exp = float(t)
        assert v == sign * exp and math.copysign(1.0, v) == sign, code


# ----------------------------------------------------------------- closed forms

def test_golden_causal_worked_example():
    with open(os.path.join(GOLDEN, "causal_worked_example.json")) as f:
        g = json.load(f)
    cache = np.full((g["num_pages"], 64, D_QK), 0x7FC0, dtype=np.uint16)   # NaN everywhere
    L = g["seqlens"][0]
    page = g["block_table"][0][0]
    cache[page, :L, :] = 0
    for j, d, v in g["latent_nonzero"]:
        cache[page, j, d] = _bits([v])[0]
    q = np.zeros((1, 2, 1, D_QK), dtype=np.uint16)
    for i, d, v in g["q_nonzero"]:
        q[0, i, 0, d] = _bits([v])[0]
    out, lse = oracle.mla_decode(q, cache, np.array(g["block_table"], np.int32),
                                 np.array(g["seqlens"], np.int32), math.log(2.0))
    exp_out = np.zeros((2, D_V))
    for i, d, frac in g["expected"]["out_nonzero"]:
        exp_out[i, d] = float(Fraction(frac))
    assert np.allclose(out[0, :, 0, :], exp_out, rtol=0, atol=1e-14)
    assert abs(lse[0, 0, 0] - math.log(4)) < 1e-14
    assert abs(lse[0, 1, 0] - math.log(9)) < 1e-14


def test_softmax_rows_sum_to_one():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((6, 576))
    K = rng.standard_normal((37, 576))
    vis = np.array([37, 1, 5, 36, 20, 2])
    O, _ = oracle.attend(q, K, np.ones((37, 1)), 0.3, vis)
    assert np.all(np.abs(O[:, 0] - 1.0) <= 1e-12)


def test_seqlen_one_returns_that_row():
    w = _tiny(2, B=1, H=4, s=1, seqlens=(1,))
    out, lse = run_oracle(w)
    row = oracle.bf16_bits_to_f64(w.cache[w.block_table[0, 0], 0])
    for h in range(4):
        assert np.array_equal(out[0, 0, h], row[:D_V])
        q = [_py_bf16(v) for v in w.q_bits[0, 0, h]]
        z = w.softmax_scale * math.fsum(q[d] * row[d] for d in range(D_QK))
        assert abs(lse[0, 0, h] - z) <= 1e-12 * max(1.0, abs(z))


def test_identical_keys_give_mean_of_values():
    # (a) the core attention with identical keys and free values
    rng = np.random.default_rng(3)
    k = rng.standard_normal(576)
    K = np.tile(k, (9, 1))
    V = rng.standard_normal((9, 512))
    q = rng.standard_normal((4, 576))
    O, lse = oracle.attend(q, K, V, 0.25, np.array([9, 9, 3, 1]))
    for r, n in enumerate([9, 9, 3, 1]):
        assert np.allclose(O[r], V[:n].mean(axis=0), rtol=0, atol=1e-13)
        z = 0.25 * float(q[r] @ k)
        assert abs(lse[r] - (z + math.log(n))) < 1e-12
    # (b) MLA form: latent part of q is zero and the rope dims are identical
    # across tokens, so scores tie while the value rows differ
    w = _tiny(4, B=1, H=2, s=1, seqlens=(70,))
    w.q_bits[..., :512] = 0
    for j in range(70):
        w.cache[w.block_table[0, j // 64], j % 64, 512:] = w.cache[w.block_table[0, 0], 0, 512:]
    out, lse = run_oracle(w)
    rows = np.array([[_py_bf16(v) for v in w.cache[w.block_table[0, j // 64], j % 64]] for j in range(70)])
    for h in range(2):
        assert np.allclose(out[0, 0, h], rows[:, :512].mean(axis=0), rtol=0, atol=1e-12)
        q = [_py_bf16(v) for v in w.q_bits[0, 0, h]]
        z = w.softmax_scale * math.fsum(q[d] * rows[0][d] for d in range(576))
        assert abs(lse[0, 0, h] - (z + math.log(70))) < 1e-12


def test_zero_scale_gives_visible_mean_and_log_count():
    w = _tiny(5, B=1, H=2, s=3, seqlens=(11,))
    out, lse = run_oracle(w, scale=0.0)
    rows = np.array([[_py_bf16(v) for v in w.cache[w.block_table[0, j // 64], j % 64]] for j in range(11)])
    for i in range(3):
        n = 11 - 3 + i + 1
        for h in range(2):
            assert np.allclose(out[0, i, h], rows[:n, :512].mean(axis=0), rtol=0, atol=1e-13)
            assert abs(lse[0, i, h] - math.log(n)) < 1e-14


def test_one_dominant_key_is_stable():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 576))
    K = np.zeros((5, 576))
    K[3] = 1000.0 * q[0] / float(q[0] @ q[0])
    V = rng.standard_normal((5, 512))
    O, lse = oracle.attend(q, K, V, 1.0, np.array([5]))
    assert np.all(np.isfinite(O))
    assert np.max(np.abs(O[0] - V[3])) <= 1e-12
    assert abs(lse[0] - 1000.0) < 1e-9


def test_empty_rows_are_zero_and_minus_inf():
    w = _tiny(7, B=2, H=2, s=3, seqlens=(2, 0))
    out, lse = run_oracle(w)
    # sequence 0 has L=2 < s=3: token 0 sees no key
    assert np.all(out[0, 0] == 0) and np.all(np.isneginf(lse[0, 0]))
    assert np.all(np.isfinite(lse[0, 1:]))
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))


# ----------------------------------------------------------------- brute force

@pytest.mark.parametrize("seed,kv,seqlens,s,H", [
    (10, "bf16", (7, 3), 2, 3),
    (11, "bf16", (10, 1), 3, 2),
    (12, "fp8_e4m3", (9, 4), 2, 3),
    (13, "fp8_e4m3", (1, 10), 1, 2),
    (14, "bf16", (2, 5), 3, 1),
])
def test_brute_force_agreement(seed, kv, seqlens, s, H):
    w = _tiny(seed, B=2, H=H, s=s, seqlens=seqlens, kv=kv)
    out, lse = run_oracle(w)
    bo, bl = brute_force(w)
    fin = np.isfinite(bl)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.max(np.abs(out - bo)) <= 1e-12 * max(1.0, np.max(np.abs(bo)))
    assert np.max(np.abs(lse[fin] - bl[fin])) <= 1e-12 * max(1.0, np.max(np.abs(bl[fin])))


def test_brute_force_multi_page():
    # crosses a page boundary (L > 64) through a shuffled table
    w = _tiny(15, B=1, H=1, s=2, seqlens=(130,))
    out, lse = run_oracle(w)
    bo, bl = brute_force(w)
    assert np.max(np.abs(out - bo)) <= 1e-12 * np.max(np.abs(bo))
    assert np.max(np.abs(lse - bl)) <= 1e-12 * np.max(np.abs(bl))


# ----------------------------------------------------------------- invariants

@pytest.mark.parametrize("seed", [20, 21, 22])
def test_split_merge_equals_unsplit(seed):
    rng = np.random.default_rng(seed)
    n = 150
    q = rng.standard_normal((8, 576))
    K = rng.standard_normal((n, 576))
    V = K[:, :512]
    vis = rng.integers(0, n + 1, size=8)
    vis[0] = n
    full_O, full_lse = oracle.attend(q, K, V, 0.07, vis)
    inner = sorted(set(rng.integers(0, n + 1, size=6).tolist()) | {0, 1, 64, 64, n})
    cuts = sorted(set([0] + inner + [n]))
    cuts = cuts[:2] + [cuts[1]] + cuts[2:]   # include an empty chunk
    parts = oracle.attend_partials(q, K, V, 0.07, vis, cuts)
    O, lse = oracle.lse_merge([p[0] for p in parts], [p[1] for p in parts])
    live = vis > 0
    assert np.max(np.abs(O - full_O)) <= 1e-12 * np.max(np.abs(full_O))
    assert np.max(np.abs(lse[live] - full_lse[live])) <= 1e-12 * np.max(np.abs(full_lse[live]))
    assert np.array_equal(np.isneginf(lse), np.isneginf(full_lse))


def test_lse_merge_closed_forms():
    O1 = np.full((1, 3), 2.0)
    O2 = np.full((1, 3), 5.0)
    O, lse = oracle.lse_merge([O1, O2], [np.array([math.log(1.0)]), np.array([math.log(3.0)])])
    assert abs(lse[0] - math.log(4.0)) < 1e-15
    assert np.allclose(O, (1 * 2.0 + 3 * 5.0) / 4.0, atol=1e-15)
    O, lse = oracle.lse_merge([O1, O2], [np.array([-np.inf]), np.array([0.5])])
    assert lse[0] == 0.5 and np.all(O == 5.0)
    O, lse = oracle.lse_merge([O1, O2], [np.array([-np.inf]), np.array([-np.inf])])
    assert np.isneginf(lse[0]) and np.all(O == 0)


def test_causal_prefix_consistency():
    w = _tiny(30, B=1, H=2, s=3, seqlens=(75,))
    out, lse = run_oracle(w)
    for i in range(3):
        n = 75 - 3 + i + 1
        w1 = make_workload("x", 1, 2, 1, [n], seed=0)
        w1.q_bits[0, 0] = w.q_bits[0, i]
        w1.cache, w1.block_table = w.cache, w.block_table
        o1, l1 = run_oracle(w1)
        assert np.array_equal(o1[0, 0], out[0, i]) and np.array_equal(l1[0, 0], lse[0, i])


def test_paging_invariance_exact():
    w = _tiny(31, B=2, H=2, s=2, seqlens=(150, 64), table="shuffled")
    out, lse = run_oracle(w)
    # re-lay the same tokens contiguously (identity table) and compare bit for bit
    cache2 = np.zeros_like(w.cache)
    bt2 = np.full_like(w.block_table, -1)
    p = 0
    for b in range(2):
        for t in range(-(-int(w.seqlens[b]) // 64)):
            cache2[p] = w.cache[w.block_table[b, t]]
            bt2[b, t] = p
            p += 1
    o2, l2 = oracle.mla_decode(w.q_bits, cache2, bt2, w.seqlens, w.softmax_scale)
    assert np.array_equal(out, o2) and np.array_equal(lse, l2)


def test_torch_sdpa_float64_cross_check():
    w = _tiny(40, B=2, H=4, s=3, seqlens=(200, 70))
    out, lse = run_oracle(w)
    for b in range(2):
        L = int(w.seqlens[b])
        rows = torch.from_numpy(w.cache[w.block_table[b, np.arange(L) // 64], np.arange(L) % 64]
                                .astype(np.int16)).view(torch.bfloat16).to(torch.float64)
        q = torch.from_numpy(w.q_bits[b].astype(np.int16)).view(torch.bfloat16).to(torch.float64)
        q = q.reshape(3 * 4, 576)
        mask = torch.zeros(12, L, dtype=torch.bool)
        for r in range(12):
            mask[r, : L - 3 + r // 4 + 1] = True
        o = torch.nn.functional.scaled_dot_product_attention(
            q[None, None], rows[None, None], rows[None, None, :, :512].contiguous(),
            attn_mask=mask[None, None], scale=w.softmax_scale)[0, 0]
        z = (q @ rows.T) * w.softmax_scale
        l = torch.logsumexp(z.masked_fill(~mask, -float("inf")), dim=1)
        assert np.max(np.abs(o.numpy().reshape(3, 4, 512) - out[b])) < 1e-10
        assert np.max(np.abs(l.numpy().reshape(3, 4) - lse[b])) < 1e-10


def test_fp8_rows_match_torch_dequant():
    w = _tiny(41, B=1, H=2, s=1, seqlens=(100,), kv="fp8_e4m3")
    rows = oracle.sequence_rows(w.cache, w.block_table[0], 100, "fp8_e4m3", w.kv_scale)
    j = np.arange(100)
    pg, sl = w.block_table[0, j // 64], j % 64
    ref = (torch.from_numpy(w.cache[pg, sl]).view(torch.float8_e4m3fn).to(torch.float64)
           * torch.from_numpy(w.kv_scale[pg, sl]).to(torch.float64)[:, None]).numpy()
    assert np.array_equal(rows, ref)


def test_workload_generators_are_seeded_and_shaped():
    a = config("share16", small=True, seed=3)
    b = config("share16", small=True, seed=3)
    assert np.array_equal(a.q_bits, b.q_bits) and np.array_equal(a.cache, b.cache)
    assert a.q_bits.shape == (6, 1, 16, 576) and a.cache.shape[1:] == (64, 576)
    assert np.all((a.seqlens >= 1024) & (a.seqlens <= 4096))
    f = config("fp8", small=True)
    assert f.cache.dtype == np.uint8 and f.kv_scale.shape == f.cache.shape[:2]
    # scale is absmax/448 over the token's 576 dims: the largest |code| is 448
    L = int(f.seqlens[0])
    pg = f.block_table[0, 0]
    vals = oracle.decode_e4m3fn(f.cache[pg, :min(64, L)])
    assert np.all(np.max(np.abs(vals), axis=1) == 448.0)


# ----------------------------------------------------------------- cache append (E4M3FN encode)

def _finite_codes():
    return [c for c in range(256) if (c & 0x7F) != 0x7F]


def test_e4m3_encode_round_trips_every_code():
    # every finite code's value encodes back to that code (the format definition)
    codes = np.array(_finite_codes(), dtype=np.uint8)
    vals = np.array([oracle.e4m3fn_value(int(c)) for c in codes])
    assert np.array_equal(oracle.encode_e4m3fn(vals), codes)


def test_e4m3_encode_ties_go_to_even_and_neighbours_to_nearest():
    pos = [oracle.e4m3fn_value(c) for c in range(0x7F)]   # 0 .. 448
    for c in range(0x7E):
        lo, hi = pos[c], pos[c + 1]
        mid = (lo + hi) / 2            # exact in float64
        even = c if c % 2 == 0 else c + 1
        assert oracle.encode_e4m3fn([mid])[0] == even
        assert oracle.encode_e4m3fn([-mid])[0] == even | 0x80
        step = (hi - lo) * 1e-6
        assert oracle.encode_e4m3fn([mid - step])[0] == c
        assert oracle.encode_e4m3fn([mid + step])[0] == c + 1


def test_e4m3_encode_matches_torch_on_random_values():
    # library cross-check: torch's float32 -> float8_e4m3fn (round to nearest even)
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.uniform(-448, 448, 20000), rng.normal(0, 1, 20000),
                        rng.normal(0, 2.0 ** -8, 20000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.encode_e4m3fn(x.astype(np.float64)), ref)


def test_quantize_token_closed_forms():
    rng = np.random.default_rng(8)
    x = rng.normal(0, 3, 576).astype(np.float32)
    codes, sc = oracle.quantize_token_e4m3(x)
    assert sc == np.float32(np.abs(x).max() / np.float32(448))
    k = int(np.argmax(np.abs(x)))
    assert codes[k] == (0x7E if x[k] > 0 else 0xFE)           # the largest entry maps to +-448
    back = oracle.decode_e4m3fn(codes) * np.float64(sc)
    # relative error of E4M3 (3 mantissa bits) is at most 2^-4 for normal codes;
    # absolute error below the smallest normal is at most half a subnormal step
    err = np.abs(back - x.astype(np.float64))
    assert np.all(err <= np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * float(sc)) + 1e-12)
    z_codes, z_sc = oracle.quantize_token_e4m3(np.zeros(576, np.float32))
    assert z_sc == 1.0 and np.all(z_codes == 0)


def test_append_kv_places_rows_and_skips_negative_positions():
    rng = np.random.default_rng(9)
    B, s = 3, 2
    seqlens = np.array([130, 1, 64], dtype=np.int32)     # 1 < s: position -1 is skipped
    bt = np.array([[5, 2, 7], [0, -1, -1], [3, -1, -1]], dtype=np.int32)
    lat = f32_to_bf16_bits(rng.normal(size=(B, s, 576)).astype(np.float32))
    cache = np.zeros((8, 64, 576), np.uint16)
    new, _ = oracle.append_kv(lat, bt, seqlens, cache)
    expect = np.zeros_like(cache)
    expect[7, 0] = lat[0, 0]; expect[7, 1] = lat[0, 1]       # positions 128, 129 -> page bt[0][2]
    expect[0, 0] = lat[1, 1]                                  # position 0 (token 1); token 0 skipped
    expect[3, 62] = lat[2, 0]; expect[3, 63] = lat[2, 1]     # positions 62, 63
    assert np.array_equal(new, expect)
    c8 = np.zeros((8, 64, 576), np.uint8)
    s8 = np.ones((8, 64), np.float32)
    n8, ns = oracle.append_kv(lat, bt, seqlens, c8, s8, "fp8_e4m3")
    x = oracle.bf16_bits_to_f64(lat[0, 1]).astype(np.float32)
    codes, sc = oracle.quantize_token_e4m3(x)
    assert np.array_equal(n8[7, 1], codes) and ns[7, 1] == sc
    assert np.count_nonzero(ns != 1) == 5


# ----------------------------------------------------------------- per-sequence q_len

@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_varlen_brute_force_agreement(kv):
    # each sequence's rows against the pure-Python definition with its own q_len
    w = make_workload("vl", 4, 2, 1, [5, 9, 4, 2], kv_dtype=kv, seed=31, q_lens=[1, 3, 0, 3])
    out, lse = oracle.mla_decode_varlen(w.q_bits, w.cu_q, w.cache, w.block_table, w.seqlens,
                                        w.softmax_scale, w.kv_dtype, w.kv_scale)
    assert out.shape == (7, 2, D_V) and lse.shape == (7, 2)
    for b in range(4):
        r0, r1 = int(w.cu_q[b]), int(w.cu_q[b + 1])
        if r1 == r0:
            continue
        one = make_workload("vl1", 1, 2, r1 - r0, [int(w.seqlens[b])], kv_dtype=kv, seed=0)
        one.q_bits = w.q_bits[r0:r1][None]
        one.cache, one.kv_scale, one.block_table = w.cache, w.kv_scale, w.block_table[b:b + 1]
        bo, bl = brute_force(one)
        fin = np.isfinite(bl[0])
        assert np.array_equal(fin, np.isfinite(lse[r0:r1]))
        assert np.max(np.abs(out[r0:r1] - bo[0])) <= 1e-12 * max(1.0, np.max(np.abs(bo)))
        assert np.max(np.abs(lse[r0:r1][fin] - bl[0][fin])) <= 1e-12 * max(1.0, np.max(np.abs(bl[0][fin])))
    # sequence 3 (q_len 3 > L 2): its first query sees no key
    assert np.all(np.isneginf(lse[4])) and np.all(out[4] == 0)


def test_varlen_uniform_q_len_equals_batched_call():
    w = make_workload("vu", 3, 4, 2, [70, 3, 200], seed=32)
    flat = w.q_bits.reshape(-1, 4, 576)
    cu = np.arange(0, 7, 2, dtype=np.int32)
    o1, l1 = oracle.mla_decode_varlen(flat, cu, w.cache, w.block_table, w.seqlens, w.softmax_scale)
    o2, l2 = run_oracle(w)
    assert np.array_equal(o1, o2.reshape(-1, 4, D_V)) and np.array_equal(l1, l2.reshape(-1, 4))


# ------------------------------------------- E4M3 image of the query rows

def test_query_quantisation_worked_example():
    """Row max 1.0: the smallest 2^k with 1.0 <= 448 * 2^k is 2^-8 (448 * 2^-9
    = 0.875 is too small); bf16(0.3) = 0.30078125 scales to 77.0, between the
    E4M3 codes 72 and 80 (spacing 8 in [64, 128)), so it maps to 80 * 2^-8;
    -1.0 maps to -256 * 2^-8 exactly; 0 stays 0. A row max of 1.875 (mantissa
    above 1.75) needs 2^-7: 1.875 * 2^7 = 240 is a code, 1.875 * 2^8 = 480
    exceeds 448; bf16(0.1) * 2^7 = 12.8125 rounds to 13."""
    row = np.zeros(576, dtype=np.float32)
    row[0], row[1], row[2] = 1.0, 0.3, -1.0
    got = oracle.quantize_query_rows_e4m3(_bits(row)[None])[0]
    assert got[0] == 1.0 and got[2] == -1.0
    assert got[1] == 80 / 256
    assert np.all(got[3:] == 0)
    assert oracle.query_row_exponent(1.0) == -8
    row2 = np.zeros(576, dtype=np.float32)
    row2[5], row2[6] = 1.875, 0.1
    got2 = oracle.quantize_query_rows_e4m3(_bits(row2)[None])[0]
    assert oracle.query_row_exponent(1.875) == -7
    assert got2[5] == 1.875 and got2[6] == 13 / 128
    # 448 * 2^k itself keeps k; anything above moves to k + 1
    assert oracle.query_row_exponent(448.0) == 0 and oracle.query_row_exponent(448.0 * (1 + 2 ** -7)) == 1
    # the floor: tiny rows keep k = -126
    assert oracle.query_row_exponent(1e-40) == -126


def test_query_quantisation_against_torch_float8():
    """Random rows (with a spread of magnitudes) against torch's own
    float8_e4m3fn rounding (round to nearest even) of x * 2^-k, k from the
    exact condition 448 * 2^(k-1) < max|x| <= 448 * 2^k (above the -126 floor)."""
    import math
    import torch
    rng = np.random.default_rng(5)
    q = rng.standard_normal((3, 4, 576)) * np.exp(rng.uniform(-20, 20, (3, 4, 1)))
    qb = _bits(q.astype(np.float32))
    x = oracle.bf16_bits_to_f64(qb)
    got = oracle.quantize_query_rows_e4m3(qb)
    assert got.shape == x.shape
    for idx in np.ndindex(x.shape[:-1]):
        row = x[idx]
        amax = float(np.max(np.abs(row)))
        k = math.ceil(math.log2(amax / 448.0))
        k += 1 if amax > 448.0 * 2.0 ** k else 0
        k -= 1 if amax <= 448.0 * 2.0 ** (k - 1) else 0
        assert 448.0 * 2.0 ** (k - 1) < amax <= 448.0 * 2.0 ** k
        ref = torch.from_numpy(row * 2.0 ** -k).to(torch.float32).to(torch.float8_e4m3fn).to(torch.float64)
        assert np.array_equal(got[idx], ref.numpy() * 2.0 ** k), idx
        # nearest: relative error <= 2^-4 for normal codes, absolute <= 2^-10 * 2^k below
        err = np.abs(got[idx] - row)
        assert np.all(err <= np.maximum(np.abs(row) * 2.0 ** -4, 2.0 ** -10 * 2.0 ** k))
        # the largest code lands in [224, 448]
        assert 224.0 <= np.max(np.abs(got[idx])) * 2.0 ** -k <= 448.0
    z = np.zeros((1, 576), dtype=np.float32)
    assert np.all(oracle.quantize_query_rows_e4m3(_bits(z)) == 0)


def test_decode_with_query_values_matches_bits():
    """q_values equal to the decoded q_bits reproduce the default result."""
    w = make_workload("qv", 2, 16, 2, [70, 130], seed=4)
    o1, l1 = oracle.mla_decode(w.q_bits, w.cache, w.block_table, w.seqlens, w.softmax_scale)
    o2, l2 = oracle.mla_decode(w.q_bits, w.cache, w.block_table, w.seqlens, w.softmax_scale,
                               q_values=oracle.bf16_bits_to_f64(w.q_bits))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ------------------------------------------------ prefill / extend (un-absorbed)

def test_prefill_brute_force():
    """Pure-Python loops: per sequence, head and query, the scores over the
    visible keys (query i of N sees keys j <= L - N + i), then softmax and the
    weighted sum; the key is k_nope of that head followed by the shared rope."""
    from workloads import make_prefill_workload
    w = make_prefill_workload("bf", [3, 2, 1], [5, 2, 4], 2, seed=11)
    out, lse = oracle.mla_prefill(w.q_bits, w.k_nope_bits, w.k_rope_bits, w.v_bits, w.cu_q, w.cu_k,
                                  w.softmax_scale)
    q = oracle.bf16_bits_to_f64(w.q_bits)
    kn = oracle.bf16_bits_to_f64(w.k_nope_bits)
    kr = oracle.bf16_bits_to_f64(w.k_rope_bits)
    v = oracle.bf16_bits_to_f64(w.v_bits)
    for b in range(3):
        q0, q1, k0, k1 = int(w.cu_q[b]), int(w.cu_q[b + 1]), int(w.cu_k[b]), int(w.cu_k[b + 1])
        N, L = q1 - q0, k1 - k0
        for h in range(2):
            for i in range(N):
                z = []
                for j in range(L - N + i + 1):
                    acc = 0.0
                    for d in range(128):
                        acc += q[q0 + i, h, d] * kn[k0 + j, h, d]
                    for d in range(64):
                        acc += q[q0 + i, h, 128 + d] * kr[k0 + j, d]
                    z.append(acc * w.softmax_scale)
                m = max(z)
                e = [math.exp(x - m) for x in z]
                tot = sum(e)
                assert abs(lse[q0 + i, h] - (m + math.log(tot))) < 1e-12
                for d in range(0, 128, 17):
                    ref = sum(e[j] * v[k0 + j, h, d] for j in range(len(z))) / tot
                    assert abs(out[q0 + i, h, d] - ref) < 1e-12


def test_prefill_absorption_identity():
    """The un-absorbed form against the absorbed decode oracle on the same
    attention: with latent rows c_j (entries in {-1,0,1}), a 0/1 map W_uk that
    sends each latent dim to one of the 128 nope dims (and W_uv likewise),
    k_nope = W_uk^T c, v = W_uv^T c and q_latent = W_uk q_nope, every value is
    an exact bf16 integer, the scores agree, and O_prefill = W_uv^T O_decode."""
    rng = np.random.default_rng(3)
    L, s, H = 70, 2, 3
    c = rng.integers(-1, 2, size=(L, 512)).astype(np.float32)
    r = rng.integers(-1, 2, size=(L, 64)).astype(np.float32)
    Wuk = np.zeros((H, 512, 128), np.float32)
    Wuv = np.zeros((H, 512, 128), np.float32)
    for h in range(H):
        Wuk[h, np.arange(512), rng.integers(0, 128, 512)] = 1
        Wuv[h, np.arange(512), rng.integers(0, 128, 512)] = 1
    qn = rng.integers(-1, 2, size=(s, H, 128)).astype(np.float32)
    qr = rng.integers(-1, 2, size=(s, H, 64)).astype(np.float32)
    kn = np.einsum("ld,hdk->lhk", c, Wuk)
    v = np.einsum("ld,hdk->lhk", c, Wuv)
    qlat = np.einsum("hdk,shk->shd", Wuk, qn)
    assert np.abs(kn).max() <= 256 and np.abs(qlat).max() <= 256   # exact in bf16
    scale = 0.05
    # un-absorbed: s new tokens at the end of L
    po, pl = oracle.mla_prefill(_bits(np.concatenate([qn, qr], -1)), _bits(kn), _bits(r), _bits(v),
                                np.array([0, s], np.int32), np.array([0, L], np.int32), scale)
    # absorbed: one sequence in pages of 64, q = [W_uk q_nope, q_rope]
    pages = (L + 63) // 64
    cache = np.zeros((pages, 64, 576), np.uint16)
    rows = _bits(np.concatenate([c, r], -1))
    for j in range(L):
        cache[j // 64, j % 64] = rows[j]
    bt = np.arange(pages, dtype=np.int32)[None]
    do, dl = oracle.mla_decode(_bits(np.concatenate([qlat, qr], -1))[None], cache, bt,
                               np.array([L], np.int32), scale)
    assert np.allclose(pl, dl[0], rtol=0, atol=1e-12)
    assert np.allclose(po, np.einsum("shd,hdk->shk", do[0], Wuv), rtol=0, atol=1e-10)


def test_prefill_extend_equals_prefill_rows():
    """An extend of the last N tokens returns the last N rows of the full
    prefill of the same L tokens (same keys, same visibility), up to the
    summation order of the BLAS product."""
    from workloads import make_prefill_workload
    w = make_prefill_workload("full", [90], [90], 4, seed=2)
    full_o, full_l = oracle.mla_prefill(w.q_bits, w.k_nope_bits, w.k_rope_bits, w.v_bits, w.cu_q, w.cu_k,
                                        w.softmax_scale)
    N = 25
    ext_o, ext_l = oracle.mla_prefill(w.q_bits[-N:], w.k_nope_bits, w.k_rope_bits, w.v_bits,
                                      np.array([0, N], np.int32), w.cu_k, w.softmax_scale)
    assert np.allclose(ext_o, full_o[-N:], rtol=0, atol=1e-12)
    assert np.allclose(ext_l, full_l[-N:], rtol=0, atol=1e-12)
