"""Per-sequence q_len (mla_decode_fwd_varlen) against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import mla_decode_attention_amd as mla
from workloads import config, make_workload
from _gpu_util import to_device, assert_parity

pytestmark = pytest.mark.gpu


def run_varlen(w, split=True, num_units=None, min_tiles=0, out=None, lse=None):
    d = to_device(w)
    q = torch.from_numpy(w.q_bits.view(np.int16)).cuda().view(torch.bfloat16)
    cu = torch.from_numpy(w.cu_q).cuda()
    plan = None
    if split:
        # (default unit count: the varlen one, as the benchmark launches it)
        plan = mla.get_split_metadata(d["seqlens"], w.q_len, w.num_heads, num_units=num_units,
                                      min_tiles_per_unit=min_tiles, varlen=True)
    o, l = mla.decode_varlen(q, cu, w.q_len, d["kv"], d["block_table"], d["seqlens"], w.softmax_scale,
                             kv_scale=d["kv_scale"], plan=plan, out=out, lse=lse)
    torch.cuda.synchronize()
    return o.cpu().numpy(), l.cpu().numpy()


def reference(w, batch_indices=None):
    return oracle.mla_decode_varlen(w.q_bits, w.cu_q, w.cache, w.block_table, w.seqlens, w.softmax_scale,
                                    w.kv_dtype, w.kv_scale, batch_indices=batch_indices)


@pytest.mark.parametrize("split", [False, True])
def test_small_varlen_config(split):
    w = config("varlen", small=True, seed=1)
    out, lse = run_varlen(w, split=split)
    ref_out, ref_lse = reference(w)
    assert_parity(w, out, lse, ref_out, ref_lse, f"varlen split={split}")


@pytest.mark.parametrize("H", [16, 64, 128])
@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_varlen_mixed_counts(H, kv):
    # q_len 1..6, a sequence with none, one with q_len > L, lengths around page edges
    lens = [64, 65, 3, 129, 700, 1, 300]
    qls = [1, 6, 4, 0, 3, 2, 5]
    w = make_workload("vl", len(lens), H, 1, lens, kv_dtype=kv, seed=H + 3, q_lens=qls)
    out, lse = run_varlen(w, split=True, num_units=9, min_tiles=1)
    ref_out, ref_lse = reference(w)
    assert_parity(w, out, lse, ref_out, ref_lse, f"varlen H={H} {kv}")


def test_varlen_leaves_foreign_rows_alone():
    # rows past cu[B] (here 3 spare rows) are not written
    w = make_workload("vl", 3, 16, 1, [100, 64, 5], seed=5, q_lens=[2, 0, 1])
    T = int(w.cu_q[-1])
    q_bits = np.concatenate([w.q_bits, np.zeros((3, 16, 576), np.uint16)])
    w.q_bits = q_bits
    out0 = torch.full((T + 3, 16, 512), 7.0, device="cuda")
    lse0 = torch.full((T + 3, 16), 7.0, device="cuda")
    out, lse = run_varlen(w, split=True, num_units=3, min_tiles=1, out=out0, lse=lse0)
    assert np.all(out[T:] == 7.0) and np.all(lse[T:] == 7.0)
    ref_out, ref_lse = reference(w)
    assert_parity(w, out[:T], lse[:T], ref_out[:T], ref_lse[:T], "varlen rows")


@pytest.mark.parametrize("H,s", [(16, 1), (16, 3), (128, 2)])
def test_varlen_with_equal_counts_matches_the_batched_call(H, s):
    """Uniform counts through the varlen entry: the batched call and the varlen
    call run the same kernel on the same schedule (the 16-row kernel up to 16
    rows, the score/output-wave kernel above), so they agree bit for bit; both
    meet the oracle bar."""
    w = make_workload("eq", 4, H, s, [300, 64, 1, 1000], seed=6)
    d = to_device(w)
    plan = mla.get_split_metadata(d["seqlens"], s, H, num_units=5, min_tiles_per_unit=1)
    o1, l1 = mla.decode(d["q"], d["kv"], d["block_table"], d["seqlens"], w.softmax_scale, plan=plan)
    cu = torch.arange(0, 4 * s + 1, s, dtype=torch.int32, device="cuda")
    o2, l2 = mla.decode_varlen(d["q"].reshape(4 * s, H, 576), cu, s, d["kv"], d["block_table"], d["seqlens"],
                               w.softmax_scale, plan=plan)
    torch.cuda.synchronize()
    o1, l1 = o1.reshape(4 * s, H, 512), l1.reshape(4 * s, H)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    ref_out, ref_lse = oracle.mla_decode(w.q_bits, w.cache, w.block_table, w.seqlens, w.softmax_scale)
    ref_out, ref_lse = ref_out.reshape(4 * s, H, 512), ref_lse.reshape(4 * s, H)
    assert_parity(w, o2.cpu().numpy(), l2.cpu().numpy(), ref_out, ref_lse, "varlen")


def test_full_size_varlen_sampled():
    w = config("varlen", seed=0)
    out, lse = run_varlen(w, split=True)
    B = w.batch
    sample = sorted({0, B - 1, B // 2, int(np.argmax(w.q_lens))})
    ref_out, ref_lse = reference(w, batch_indices=sample)
    rows = np.concatenate([np.arange(w.cu_q[b], w.cu_q[b + 1]) for b in sample])
    assert_parity(w, out[rows], lse[rows], ref_out[rows], ref_lse[rows], f"varlen full, sample {sample}")
