"""mla_decode_fwd_noalloc (schedule and partials in the library's static
device buffer) against mla_decode_fwd with a plan of the same unit count:
bit for bit, on two calls in a row, the second with a smaller input, and
within the oracle bar. Called through the C ABI via the binding."""
import numpy as np
import pytest
import torch

import mla_decode_attention_amd as mla
from workloads import make_workload
from _gpu_util import to_device, reference, assert_parity

pytestmark = pytest.mark.gpu


def _both(w, units, min_tiles=1):
    d = to_device(w)
    plan = mla.get_split_metadata(d["seqlens"], w.q_len, w.num_heads, num_units=units, min_tiles_per_unit=min_tiles)
    o1, l1 = mla.decode(d["q"], d["kv"], d["block_table"], d["seqlens"], w.softmax_scale, kv_scale=d["kv_scale"],
                        plan=plan)
    o2, l2 = mla.decode_noalloc(d["q"], d["kv"], d["block_table"], d["seqlens"], w.softmax_scale,
                                kv_scale=d["kv_scale"], num_units=units, min_tiles_per_unit=min_tiles)
    torch.cuda.synchronize()
    return (o1.cpu().numpy(), l1.cpu().numpy()), (o2.cpu().numpy(), l2.cpu().numpy())


@pytest.mark.parametrize("H,s,kv", [(16, 1, "bf16"), (128, 2, "bf16"), (128, 2, "fp8_e4m3")])
def test_noalloc_matches_the_planned_call_twice(H, s, kv):
    big = make_workload("noalloc-a", 6, H, s, [3000, 65, 1, 700, 4096, 129], kv_dtype=kv, seed=51)
    small = make_workload("noalloc-b", 2, H, s, [300, 64], kv_dtype=kv, seed=52)
    for w, units in ((big, 13), (small, 3)):
        (o1, l1), (o2, l2) = _both(w, units)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2), f"{w.name}"
        ref_out, ref_lse = reference(w)
        assert_parity(w, o2, l2, ref_out, ref_lse, f"noalloc {w.name}")


def test_noalloc_default_units_and_empty_sequences():
    w = make_workload("noalloc-c", 5, 128, 2, [0, 130, 2, 0, 900], seed=53)
    d = to_device(w)
    o, l = mla.decode_noalloc(d["q"], d["kv"], d["block_table"], d["seqlens"], w.softmax_scale)
    torch.cuda.synchronize()
    o, l = o.cpu().numpy(), l.cpu().numpy()
    ref_out, ref_lse = reference(w)
    assert np.all(o[0] == 0) and np.all(np.isneginf(l[0]))
    assert_parity(w, o, l, ref_out, ref_lse, "noalloc default units")


def test_noalloc_rejects_shapes_past_the_scratch():
    lib = mla.load_library()
    assert lib.mla_noalloc_scratch_need(128, 2, 128, 64) <= 128 << 20
    w = make_workload("noalloc-d", 2, 128, 2, [100, 100], seed=54)
    d = to_device(w)
    with pytest.raises(mla.MLAError, match="MLA_ERR_WORKSPACE"):
        mla.decode_noalloc(d["q"], d["kv"], d["block_table"], d["seqlens"], w.softmax_scale, num_units=4096)
