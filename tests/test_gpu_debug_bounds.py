"""The page-id bounds build (libmla_decode_debug.so, MLA_DEBUG_BOUNDS).

With valid block tables it counts nothing and computes bit for bit what the
release library computes; with page ids outside the pool, or tables narrower
than a sequence's pages, it counts the bad uses and reads page 0 instead, so
the run completes (the release library trusts the table: these inputs are
given to the checking build only)."""
import numpy as np
import pytest
import torch

import mla_decode_attention_amd as mla
from workloads import make_workload
from _gpu_util import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture
def release_then_debug():
    mla.use_debug_library(False)
    yield
    mla.use_debug_library(False)


def _run(w, d, split, block_table=None):
    bt = d["block_table"] if block_table is None else block_table
    plan = None
    if split:
        plan = mla.get_split_metadata(d["seqlens"], w.q_len, w.num_heads)
    out, lse = mla.decode(d["q"], d["kv"], bt, d["seqlens"], w.softmax_scale, kv_scale=d["kv_scale"], plan=plan)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


CASES = [("narrow", 6, 16, 1, [1, 63, 64, 65, 700, 2000], "bf16"),
         ("wide", 4, 128, 2, [2, 130, 900, 1500], "bf16"),
         ("wide_fp8", 3, 128, 2, [70, 640, 1100], "fp8_e4m3"),
         ("narrow_fp8", 3, 16, 1, [70, 640, 1100], "fp8_e4m3")]


@pytest.mark.parametrize("name,B,H,s,lens,kv", CASES)
def test_valid_tables_count_nothing_and_match_release(release_then_debug, name, B, H, s, lens, kv):
    w = make_workload(name, B, H, s, np.array(lens), kv_dtype=kv, seed=B + H)
    d = to_device(w)
    ref = [_run(w, d, split) for split in (False, True)]
    mla.use_debug_library(True)
    mla.debug_page_violations(reset=True)
    for split, (ro, rl) in zip((False, True), ref):
        o, l = _run(w, d, split)
        assert np.array_equal(o, ro) and np.array_equal(l, rl), f"{name} split={split}"
    assert mla.debug_page_violations() == 0


@pytest.mark.parametrize("name,B,H,s,lens,kv", CASES)
def test_page_ids_outside_the_pool_are_counted(release_then_debug, name, B, H, s, lens, kv):
    w = make_workload(name, B, H, s, np.array(lens), kv_dtype=kv, seed=3)
    d = to_device(w)
    num_pages = d["kv"].shape[0]
    bt = d["block_table"].clone()
    bt[B - 1, 0] = num_pages + 7         # past the pool
    bt[B - 2, (lens[B - 2] - 1) // 64] = -2   # negative, on that sequence's last page
    mla.use_debug_library(True)
    mla.debug_page_violations(reset=True)
    for split in (False, True):
        o, l = _run(w, d, split, block_table=bt)
        assert np.all(np.isfinite(o[: B - 2])), "rows of untouched sequences"
    assert mla.debug_page_violations() > 0
    assert mla.debug_page_violations() == 0   # the read above reset the counters


def test_table_narrower_than_a_sequence(release_then_debug):
    """Pages past the table's row (max_pages_per_seq) are not read."""
    w = make_workload("narrowtab", 2, 16, 1, np.array([300, 100]), seed=4)
    d = to_device(w)
    bt = d["block_table"][:, :2].contiguous()   # 2 ids per row; sequence 0 has 5 pages
    mla.use_debug_library(True)
    mla.debug_page_violations(reset=True)
    _run(w, d, split=False, block_table=bt)
    assert mla.debug_page_violations() > 0


def test_release_library_has_no_counters(release_then_debug):
    with pytest.raises(mla.MLAError, match="UNSUPPORTED"):
        mla.debug_page_violations()
