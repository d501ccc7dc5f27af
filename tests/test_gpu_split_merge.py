"""Split-KV decode details: sequences without tiles in split mode (16-row and
64-row kernels), one metadata buffer reused by several calls, and metadata
that does not match the call (checked on the device: nothing is written)."""
import numpy as np
import pytest
import torch

import mla_decode_attention_amd as mla
from workloads import config, make_workload
from _gpu_util import to_device, run_gpu, reference, assert_parity

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("H,s", [(16, 1), (128, 2)])
@pytest.mark.parametrize("lens,units", [
    ([0, 0, 130, 0, 64, 0, 4000, 0, 0], 7),        # empties first, between, at unit edges, last
    ([0, 0, 0], 4),                                # nothing to compute
    ([0] * 20 + [700], 3),                         # more empty sequences than units
    ([65, 0, 1, 0, 2000], 64),                     # more units than tiles
])
def test_empty_sequences_split(H, s, lens, units):
    lens = [L if L == 0 else max(L, s) for L in lens]
    w = make_workload("empty-split", len(lens), H, s, lens, seed=21)
    out, lse, _ = run_gpu(w, split=True, num_units=units, min_tiles=1)
    ref_out, ref_lse = reference(w)
    for b, L in enumerate(lens):
        if L == 0:
            assert np.all(out[b] == 0) and np.all(np.isneginf(lse[b])), f"sequence {b}"
    assert_parity(w, out, lse, ref_out, ref_lse, f"H={H} s={s} lens={lens}")


@pytest.mark.parametrize("name", ["share16", "mtp"])
def test_metadata_reused_by_several_calls(name):
    """One metadata buffer and workspace for several calls (as for the layers
    of a decode step): identical bits every time."""
    w = config(name, small=True, seed=4)
    d = to_device(w)
    plan = mla.get_split_metadata(d["seqlens"], w.q_len, w.num_heads, num_units=13, min_tiles_per_unit=1)
    results = []
    for _ in range(3):
        o, l = mla.decode(d["q"], d["kv"], d["block_table"], d["seqlens"], w.softmax_scale, plan=plan)
        torch.cuda.synchronize()
        results.append((o.cpu().numpy(), l.cpu().numpy()))
    for o, l in results[1:]:
        assert np.array_equal(o, results[0][0]) and np.array_equal(l, results[0][1])
    ref_out, ref_lse = reference(w)
    assert_parity(w, results[0][0], results[0][1], ref_out, ref_lse, "reused metadata")


@pytest.mark.parametrize("H,s", [(16, 1), (128, 2)])
@pytest.mark.parametrize("units_call", [5, 9])
def test_mismatched_metadata_writes_nothing(H, s, units_call):
    """Metadata built for 6 units, call made with another unit count: the
    decode kernels and the merge check the header and leave out / lse as
    they were."""
    w = make_workload("md-mismatch", 3, H, s, [500, 70, 1300], seed=5)
    d = to_device(w)
    plan = mla.get_split_metadata(d["seqlens"], s, H, num_units=6, min_tiles_per_unit=1)
    plan.num_units = units_call
    if units_call > 6:   # the workspace must still pass the host-side size check
        plan.workspace = torch.empty(mla.workspace_bytes(3, s, H, units_call), dtype=torch.uint8, device="cuda")
    out = torch.full((3, s, H, 512), 7.0, dtype=torch.float32, device="cuda")
    lse = torch.full((3, s, H), 7.0, dtype=torch.float32, device="cuda")
    mla.decode(d["q"], d["kv"], d["block_table"], d["seqlens"], w.softmax_scale, plan=plan, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0) and torch.all(lse == 7.0)


@pytest.mark.parametrize("batch,q_len,heads", [(64, 1, 16), (128, 2, 128), (128, 3, 64), (128, 3, 128),
                                               (128, 6, 128), (32, 1, 128), (1, 32, 128), (1000, 5, 64)])
def test_default_unit_counts_fill_whole_rounds(batch, q_len, heads):
    """Default unit counts: a multiple of the 8 XCDs, and each XCD's units x
    row blocks fill whole rounds of its CUs (row blocks of a unit share an
    XCD); the varlen default also gives about one unit per sequence."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    per_xcd = cus // 8
    rows = q_len * heads
    rb = 1 if rows <= 16 else (rows + 63) // 64
    for varlen in (False, True):
        u = mla.default_num_units(batch, q_len, heads, varlen=varlen)
        assert u > 0 and u % 8 == 0, (u, varlen)
        k = u // 8
        assert (k * rb) % per_xcd == 0, (u, rb, varlen)
        assert k >= max(1, per_xcd // rb)
        if varlen:
            assert u >= batch
        # and a plan with that many units runs (metadata sized for it)
        sl = torch.full((batch,), 300, dtype=torch.int32, device="cuda")
        plan = mla.get_split_metadata(sl, q_len, heads, varlen=varlen)
        assert plan.num_units == u
