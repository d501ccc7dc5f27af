"""The Python binding rejects buffers of the wrong shape, dtype or device
before any call into the library (a wrong-shape output would otherwise be
written past its end)."""
import numpy as np
import pytest
import torch

import mla_decode_attention_amd as mla
from workloads import make_workload
from _gpu_util import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def small():
    w = make_workload("binding", 2, 16, 2, [100, 70], seed=3)
    return w, to_device(w)


def _decode(w, d, **kw):
    return mla.decode(d["q"], d["kv"], d["block_table"], d["seqlens"], w.softmax_scale, **kw)


def test_wrong_output_shapes_are_rejected(small):
    w, d = small
    B, s, H = w.batch, w.q_len, w.num_heads
    with pytest.raises(ValueError):
        _decode(w, d, out=torch.empty((B, s, H, 256), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        _decode(w, d, out=torch.empty((B, 1, H, 512), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        _decode(w, d, lse=torch.empty((B, s, 2 * H), dtype=torch.float32, device="cuda"))


def test_plan_buffers_are_checked(small):
    w, d = small
    plan = mla.get_split_metadata(d["seqlens"], w.q_len, w.num_heads, num_units=4, min_tiles_per_unit=1)
    with pytest.raises(TypeError):
        mla.get_split_metadata(d["seqlens"], w.q_len, w.num_heads, num_units=4,
                               metadata=torch.empty(4096, dtype=torch.uint8, device="cuda"))
    plan.workspace = plan.workspace.view(torch.float32)
    with pytest.raises(TypeError):
        _decode(w, d, plan=plan)


def test_fp8_scales_shape_is_checked():
    w = make_workload("binding-fp8", 2, 16, 1, [100, 70], kv_dtype="fp8_e4m3", seed=4)
    d = to_device(w)
    bad = d["kv_scale"][:, :32].contiguous()
    with pytest.raises(ValueError):
        mla.decode(d["q"], d["kv"], d["block_table"], d["seqlens"], w.softmax_scale, kv_scale=bad)


def test_combine_output_shapes_are_checked():
    po = torch.zeros((3, 16, 512), dtype=torch.float32, device="cuda")
    pl = torch.zeros((3, 16), dtype=torch.float32, device="cuda")
    offs = torch.tensor([0, 1, 3], dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        mla.combine(po, pl, offs, out=torch.empty((2, 8, 512), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        mla.combine(po, pl[:2].contiguous(), offs)
    out, lse = mla.combine(po, pl, offs)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (2, 16, 512) and np.allclose(lse.cpu().numpy()[1], np.log(2.0))
