"""Parity of the HIP path (through the C ABI) with the CPU fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import mla_decode_attention_amd as mla
from workloads import config, make_workload, PAGE_TOKENS
from _gpu_util import to_device, run_gpu, reference, assert_parity
from _split_contract import check_metadata, schedule_words

pytestmark = pytest.mark.gpu


# ----------------------------------------------------------------- small configs

@pytest.mark.parametrize("name", ["tiny", "share16", "share16_fp8", "mtp", "ragged", "fp8"])
@pytest.mark.parametrize("split", [False, True])
def test_small_config_parity(name, split):
    w = config(name, small=True, seed=1)
    out, lse, _ = run_gpu(w, split=split)
    ref_out, ref_lse = reference(w)
    assert_parity(w, out, lse, ref_out, ref_lse, f"{name} split={split}")


@pytest.mark.parametrize("H,s", [(16, 1), (16, 2), (128, 1), (128, 2), (64, 3)])
@pytest.mark.parametrize("split", [False, True])
def test_edge_lengths(H, s, split):
    lens = [1, 2, 63, 64, 65, 127, 129, 4097]
    lens = [L for L in lens if L >= s] + [s]
    w = make_workload("edges", len(lens), H, s, lens, seed=5)
    out, lse, _ = run_gpu(w, split=split, num_units=13, min_tiles=1)
    ref_out, ref_lse = reference(w)
    assert_parity(w, out, lse, ref_out, ref_lse, f"H={H} s={s} split={split}")


@pytest.mark.parametrize("H", [16, 32, 48, 64, 128])
@pytest.mark.parametrize("s", [1, 2, 4, 6])
def test_heads_and_query_tokens(H, s):
    w = make_workload("hs", 3, H, s, [300, 64, 1000], seed=H * 10 + s)
    out, lse, _ = run_gpu(w, split=True, num_units=7, min_tiles=1)
    ref_out, ref_lse = reference(w)
    assert_parity(w, out, lse, ref_out, ref_lse, f"H={H} s={s}")


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("split", [False, True])
def test_max_rows_per_sequence(kv_dtype, split):
    # q_len * H = 4096 rows per sequence, the library's limit: 64 row blocks,
    # causal over 32 query tokens, a sequence shorter than them
    lens = [200, 32, 65]
    w = make_workload("maxrows", len(lens), 128, 32, lens, kv_dtype=kv_dtype, seed=41)
    out, lse, _ = run_gpu(w, split=split, num_units=5, min_tiles=1)
    ref_out, ref_lse = reference(w)
    assert_parity(w, out, lse, ref_out, ref_lse, f"max rows {kv_dtype} split={split}")


@pytest.mark.parametrize("H,s", [(16, 1), (16, 3), (64, 2), (128, 2)])
@pytest.mark.parametrize("split", [False, True])
def test_fp8_cache_shapes(H, s, split):
    """fp8 e4m3 cache with per-token scales across the three kernel variants,
    ragged tails (NaN-poisoned codes and scales past each sequence)."""
    lens = [1, 63, 64, 65, 300, 1000]
    lens = [L for L in lens if L >= s] + [s]
    w = make_workload("fp8-shapes", len(lens), H, s, lens, kv_dtype="fp8_e4m3", seed=17 + H + s)
    out, lse, _ = run_gpu(w, split=split, num_units=9, min_tiles=1)
    ref_out, ref_lse = reference(w)
    assert_parity(w, out, lse, ref_out, ref_lse, f"fp8 H={H} s={s} split={split}")


@pytest.mark.parametrize("split", [False, True])
def test_empty_sequences_and_rows(split):
    # L = 0 sequences and sequences shorter than q_len (rows with no visible key)
    w = make_workload("empty", 5, 16, 3, [0, 1, 2, 70, 0], seed=9)
    out, lse, _ = run_gpu(w, split=split, num_units=3, min_tiles=1)
    ref_out, ref_lse = reference(w)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.all(out[4] == 0) and np.all(np.isneginf(lse[4]))
    assert_parity(w, out, lse, ref_out, ref_lse, f"empty split={split}")


# ----------------------------------------------------------------- invariants

def _relayout_identity(w):
    cache2 = np.zeros_like(w.cache)
    bt2 = np.full_like(w.block_table, -1)
    p = 0
    for b in range(w.batch):
        for t in range(-(-int(w.seqlens[b]) // PAGE_TOKENS)):
            cache2[p] = w.cache[w.block_table[b, t]]
            bt2[b, t] = p
            p += 1
    return cache2, bt2


@pytest.mark.parametrize("H,s", [(16, 1), (128, 2)])
def test_paging_invariance_bitwise(H, s):
    w = make_workload("pg", 4, H, s, [700, 64, 1, 300], seed=11)
    out1, lse1, _ = run_gpu(w, split=True, num_units=5, min_tiles=1)
    w.cache, w.block_table = _relayout_identity(w)
    out2, lse2, _ = run_gpu(w, split=True, num_units=5, min_tiles=1)
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)


def test_run_to_run_bitwise():
    w = config("ragged", small=True, seed=2)
    d = to_device(w)
    a = run_gpu(w, d, split=True)
    b = run_gpu(w, d, split=True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_split_and_unsplit_agree():
    w = config("mtp", small=True, seed=3)
    d = to_device(w)
    o1, l1, _ = run_gpu(w, d, split=False)
    o2, l2, _ = run_gpu(w, d, split=True, num_units=11, min_tiles=1)
    ref_out, ref_lse = reference(w)
    assert_parity(w, o1, l1, ref_out, ref_lse, "unsplit")
    assert_parity(w, o2, l2, ref_out, ref_lse, "split")
    assert np.max(np.abs(o1 - o2)) <= 1e-2 * np.max(np.abs(ref_out))


# ----------------------------------------------------------------- scheduler + combine

METADATA_CASES = [
    ([256], 256, 0), ([4096] * 7, 16, 0), ([1, 63, 64, 65, 0, 700], 5, 1), ([0, 0], 4, 8),
    ([65536, 512, 3000, 70], 64, 0), ([130] * 3, 1000, 1), (list(range(0, 5000, 37)), 250, 0),
    # a large batch: 8000 sequences over 400 units, several sequences per thread
    ([int(x) for x in np.random.default_rng(5).integers(0, 3000, 8000)], 400, 0),
]


def _device_metadata(lens, units, mt, q_len, heads):
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    plan = mla.get_split_metadata(sl, q_len, heads, num_units=units, min_tiles_per_unit=mt)
    return plan.metadata.cpu().numpy()


@pytest.mark.parametrize("lens,units,mt", METADATA_CASES)
@pytest.mark.parametrize("q_len,heads,cost", [(1, 16, 1), (2, 128, 3)])
def test_metadata_is_a_valid_schedule(lens, units, mt, q_len, heads, cost):
    """Properties every valid split schedule has, whatever its balance rule:
    each tile in exactly one unit, contiguous unit ranges, consecutive units
    per sequence, offsets and first units that agree with the ranges, and
    every unit's cost within one sequence start of an even share."""
    md = _device_metadata(lens, units, mt, q_len, heads)
    check_metadata(md, lens, units, mt if mt else 8, cost)


def test_metadata_is_valid_on_random_batches():
    rng = np.random.default_rng(123)
    for _ in range(24):
        B = int(rng.choice([1, 3, 32, 129, 1000]))
        kind = rng.integers(0, 3)
        if kind == 0:
            lens = rng.integers(0, 5000, B)
        elif kind == 1:
            lens = np.exp(rng.uniform(np.log(1), np.log(70000), B)).astype(int)
        else:
            lens = rng.choice([0, 1, 64, 65, 4096], B)
        lens = [int(x) for x in lens]
        units = int(rng.choice([1, 7, 64, 256, 1024]))
        mt = int(rng.choice([0, 1, 3, 8, 100]))
        q_len, heads, cost = [(1, 16, 1), (2, 128, 3)][int(rng.integers(0, 2))]
        md = _device_metadata(lens, units, mt, q_len, heads)
        check_metadata(md, lens, units, mt if mt else 8, cost)


@pytest.mark.parametrize("lens,units,mt", METADATA_CASES)
@pytest.mark.parametrize("q_len,heads,cost", [(1, 16, 1), (2, 128, 3)])
def test_metadata_matches_header_definition(lens, units, mt, q_len, heads, cost):
    """The device metadata is word for word the rule include/mla_decode.h
    states (the library's own contract; not part of what the method computes)."""
    md = _device_metadata(lens, units, mt, q_len, heads)
    want = schedule_words(lens, units, mt if mt else 8, cost)
    assert [int(x) for x in md[:len(want)]] == want


@pytest.mark.parametrize("R", [16, 256])
def test_combine_matches_oracle_merge(R):
    rng = np.random.default_rng(R)
    counts = [3, 1, 0, 5, 2]
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    N = int(offs[-1])
    po = rng.standard_normal((N, R, 512)).astype(np.float32)
    pl = (rng.standard_normal((N, R)) * 3).astype(np.float32)
    pl[0, :5] = -np.inf                      # some partials saw no visible key
    pl[3:8, 7] = -np.inf                     # a row with only -inf partials in sequence 3
    po_gpu = po.copy()
    po_gpu[np.isneginf(pl)] = np.nan         # values of -inf partials are never read into the result
    out, lse = mla.combine(torch.from_numpy(po_gpu).cuda(), torch.from_numpy(pl).cuda(),
                           torch.from_numpy(offs).cuda())
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    for b in range(len(counts)):
        k0, k1 = offs[b], offs[b + 1]
        if k1 == k0:
            assert np.all(out[b] == 0) and np.all(np.isneginf(lse[b]))
            continue
        ro, rl = oracle.lse_merge(po[k0:k1].astype(np.float64), pl[k0:k1].astype(np.float64))
        assert np.max(np.abs(out[b] - ro)) <= 1e-5 * max(1.0, np.max(np.abs(ro)))
        fin = np.isfinite(rl)
        assert np.array_equal(np.isneginf(lse[b]), ~fin)
        assert np.max(np.abs(lse[b][fin] - rl[fin])) <= 1e-5


# ----------------------------------------------------------------- full sizes, sampled

# every sequence of the smaller workloads; at least 16 of the two largest
FULL_SIZE_SAMPLE = {"tiny": None, "share16": None, "share16_fp8": None, "ragged": None, "mtp": 16, "fp8": 16}


@pytest.mark.parametrize("name", ["tiny", "share16", "share16_fp8", "mtp", "ragged", "fp8"])
def test_full_size(name):
    """Whole-batch run in the launch configuration the benchmark times (default
    split plan), compared with the oracle on every sequence of tiny, share16,
    share16_fp8 and ragged, and on 16 sequences (the first, the last and 14 drawn) of mtp
    and fp8."""
    w = config(name, seed=0)
    out, lse, _ = run_gpu(w, split=True)
    B = w.batch
    k = FULL_SIZE_SAMPLE[name]
    if k is None:
        sample = list(range(B))
    else:
        rng = np.random.default_rng(99)
        sample = sorted({0, B - 1} | set(int(x) for x in rng.choice(np.arange(1, B - 1), k - 2, replace=False)))
    ref_out, ref_lse = reference(w, batch_indices=sample)
    assert_parity(w, out[sample], lse[sample], ref_out, ref_lse, f"{name} full, {len(sample)} sequences")


# ------------------------------------------------------- lazy-rescale coverage

def _ramp_cache(w, amp, seed):
    """Rewrite every live key j of sequence b as noise + amp * (j / L_b) * v,
    with one shared random direction v: rows whose query leans on v see their
    scores climb through the sequence, so the running max moves many times
    (well past the lazy-rescale threshold) and on tiles in the middle of a
    split unit; the other rows see falling scores."""
    from workloads import f32_to_bf16_bits, _e4m3_encode, E4M3_MAX
    rng = np.random.default_rng(seed)
    v = rng.standard_normal(w.cache.shape[-1]).astype(np.float32)
    for b, L in enumerate(w.seqlens):
        L = int(L)
        if L == 0:
            continue
        j = np.arange(L)
        x = (0.3 * rng.standard_normal((L, v.size)) + amp * (j / L)[:, None] * v[None, :]).astype(np.float32)
        pages = w.block_table[b, j // PAGE_TOKENS]
        if w.kv_dtype == "bf16":
            w.cache[pages, j % PAGE_TOKENS] = f32_to_bf16_bits(x)
        else:
            amax = np.abs(x).max(axis=1)
            sc = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
            w.cache[pages, j % PAGE_TOKENS] = _e4m3_encode(np.clip(x / sc[:, None], -E4M3_MAX, E4M3_MAX))
            w.kv_scale[pages, j % PAGE_TOKENS] = sc
    return w


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("H,s", [(16, 1), (16, 2), (128, 2)])
@pytest.mark.parametrize("split", [False, True])
def test_rising_scores_rescale(kv_dtype, H, s, split):
    lens = [1000, 700, 130, 64]
    w = _ramp_cache(make_workload("ramp", len(lens), H, s, lens, kv_dtype=kv_dtype, seed=31 + H + s), 6.0, 5)
    out, lse, _ = run_gpu(w, split=split, num_units=7, min_tiles=1)
    ref_out, ref_lse = reference(w)
    # the ramp really moves the running max: the largest score of many rows
    # sits far above their first tile's
    assert float(np.max(ref_lse)) > 20.0
    assert_parity(w, out, lse, ref_out, ref_lse, f"ramp {kv_dtype} H={H} s={s} split={split}")


@pytest.mark.parametrize("kv_dtype,H,s", [("bf16", 16, 1), ("bf16", 128, 2), ("fp8_e4m3", 128, 2)])
def test_negative_softmax_scale(kv_dtype, H, s):
    """Any finite scale is accepted; a negative one turns the row max into the
    most negative dot product (every decode kernel scales before its max)."""
    w = make_workload("neg", 3, H, s, np.array([1, 200, 700]), kv_dtype=kv_dtype, seed=9, softmax_scale=-0.05)
    for split in (False, True):
        out, lse, _ = run_gpu(w, split=split)
        assert_parity(w, out, lse, *reference(w), what=f"negative scale split={split}")
