"""A decode step (split schedule, attention, merge) captured in a HIP graph and
replayed: every replay, with eager work and synchronisation between replays,
gives the eager result bit for bit (the schedule is fixed, so the kernels are
deterministic), and the eager result meets the oracle bar."""
import numpy as np
import pytest
import torch

import mla_decode_attention_amd as mla
from workloads import config, make_workload
from _gpu_util import to_device, reference, assert_parity

pytestmark = pytest.mark.gpu


def _step(w, d, plan, out, lse, fp8_mma=False):
    mla.get_split_metadata(d["seqlens"], w.q_len, w.num_heads, num_units=plan.num_units,
                           metadata=plan.metadata, workspace=plan.workspace)
    mla.decode(d["q"], d["kv"], d["block_table"], d["seqlens"], w.softmax_scale, kv_scale=d["kv_scale"],
               plan=plan, out=out, lse=lse, fp8_mma=fp8_mma)


@pytest.mark.parametrize("name", ["share16", "share16_fp8", "mtp", "ragged", "fp8"])
def test_graph_replay_matches_eager(name):
    w = config(name, small=True, seed=4)
    d = to_device(w)
    plan = mla.get_split_metadata(d["seqlens"], w.q_len, w.num_heads, num_units=24, min_tiles_per_unit=1)
    shape = (w.batch, w.q_len, w.num_heads)
    out_e = torch.empty(shape + (512,), dtype=torch.float32, device="cuda")
    lse_e = torch.empty(shape, dtype=torch.float32, device="cuda")
    _step(w, d, plan, out_e, lse_e)
    torch.cuda.synchronize()
    ref_out, ref_lse = reference(w)
    assert_parity(w, out_e.cpu().numpy(), lse_e.cpu().numpy(), ref_out, ref_lse, f"{name} eager")

    out_g = torch.empty_like(out_e)
    lse_g = torch.empty_like(lse_e)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(w, d, plan, out_g, lse_g)
    torch.cuda.synchronize()
    for rep in range(3):
        # eager work between the replays: poison the outputs and the metadata
        out_g.fill_(float("nan"))
        lse_g.fill_(float("nan"))
        plan.metadata.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), f"{name}: replay {rep} output differs from eager"
        assert torch.equal(lse_g, lse_e), f"{name}: replay {rep} LSE differs from eager"


def test_graph_replay_follows_new_lengths():
    # the captured step reads cache_seqlens on the device at every replay:
    # new lengths written in place between replays give that step's result
    # (each within the pages its sequence was built with)
    lens_a = [1000, 700, 1000, 300]
    w = make_workload("graph-lens", 4, 128, 2, lens_a, seed=8)
    d = to_device(w)
    plan = mla.get_split_metadata(d["seqlens"], w.q_len, w.num_heads, num_units=6, min_tiles_per_unit=1)
    out = torch.empty((4, 2, 128, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((4, 2, 128), dtype=torch.float32, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(w, d, plan, out, lse)
    for lens in (lens_a, [64, 65, 999, 2], [1000, 3, 17, 300]):
        assert all(n <= cap for n, cap in zip(lens, lens_a))
        d["seqlens"].copy_(torch.tensor(lens, dtype=torch.int32))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        w.seqlens = np.array(lens, dtype=np.int32)
        ref_out, ref_lse = reference(w)
        assert_parity(w, out.cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse, f"lens={lens}")


def test_profile_hook_records_every_kernel_kind():
    """The measurement hook gives one dispatch-timed interval per launch of
    each kernel kind (attention, metadata, merge), in launch order."""
    w = config("share16", small=True, seed=8)
    d = to_device(w)
    plan = mla.get_split_metadata(d["seqlens"], w.q_len, w.num_heads, num_units=5, min_tiles_per_unit=1)
    torch.cuda.synchronize()
    mla.profile_enable(True)
    for k in (mla.PROFILE_ATTENTION, mla.PROFILE_METADATA, mla.PROFILE_COMBINE):
        mla.profile_read_launches(k, capacity=0)
    for _ in range(3):
        mla.get_split_metadata(d["seqlens"], w.q_len, w.num_heads, num_units=5, min_tiles_per_unit=1,
                               metadata=plan.metadata, workspace=plan.workspace)
        mla.decode(d["q"], d["kv"], d["block_table"], d["seqlens"], w.softmax_scale, plan=plan)
    mla.profile_enable(False)
    att = mla.profile_read_launches(mla.PROFILE_ATTENTION)
    md = mla.profile_read_launches(mla.PROFILE_METADATA)
    cb = mla.profile_read_launches(mla.PROFILE_COMBINE)
    assert len(att) == 3 and len(md) == 3 and len(cb) == 3
    assert all(0.0 < t < 100.0 for t in att + md + cb)
    assert mla.profile_read_launches(mla.PROFILE_ATTENTION) == []
