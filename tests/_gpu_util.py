"""Shared helpers for the GPU tests: move a workload to the device, run the
HIP path through the binding, compare with the oracle at the stated bar."""
import math

import numpy as np
import torch

import oracle
import mla_decode_attention_amd as mla

# Tolerances of the parity bar: max|O_gpu - O_ref| <= 1e-2 * max|O_ref| over the
# whole output; |LSE_gpu - LSE_ref| <= 1e-3 (bf16 cache) or 3e-2 (fp8 cache).
O_REL_TOL = 1e-2
LSE_TOL = {"bf16": 1e-3, "fp8_e4m3": 3e-2}


def to_device(w, device="cuda"):
    q = torch.from_numpy(w.q_bits.view(np.int16)).to(device).view(torch.bfloat16)
    if w.kv_dtype == "bf16":
        kv = torch.from_numpy(w.cache.view(np.int16)).to(device).view(torch.bfloat16)
        sc = None
    else:
        kv = torch.from_numpy(w.cache).to(device)
        sc = torch.from_numpy(w.kv_scale).to(device)
    bt = torch.from_numpy(w.block_table).to(device)
    sl = torch.from_numpy(w.seqlens).to(device)
    return dict(q=q, kv=kv, kv_scale=sc, block_table=bt, seqlens=sl)


def run_gpu(w, d=None, split=True, num_units=None, min_tiles=0):
    d = d or to_device(w)
    plan = None
    if split:
        plan = mla.get_split_metadata(d["seqlens"], w.q_len, w.num_heads, num_units=num_units,
                                      min_tiles_per_unit=min_tiles)
    out, lse = mla.decode(d["q"], d["kv"], d["block_table"], d["seqlens"], w.softmax_scale,
                          kv_scale=d["kv_scale"], plan=plan)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), plan


def reference(w, batch_indices=None):
    return oracle.mla_decode(w.q_bits, w.cache, w.block_table, w.seqlens, w.softmax_scale,
                             w.kv_dtype, w.kv_scale, batch_indices=batch_indices)


def assert_parity(w, out, lse, ref_out, ref_lse, what=""):
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    o_err = float(np.max(np.abs(out - ref_out))) if out.size else 0.0
    o_scale = float(np.max(np.abs(ref_out))) if out.size else 0.0
    assert o_err <= O_REL_TOL * max(o_scale, 1e-30), f"{what}: O err {o_err:.3e} vs scale {o_scale:.3e}"
    neg = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), neg), f"{what}: -inf LSE pattern differs"
    if (~neg).any():
        l_err = float(np.max(np.abs(lse[~neg] - ref_lse[~neg])))
        assert l_err <= LSE_TOL[w.kv_dtype], f"{what}: LSE err {l_err:.3e}"
    return o_err / max(o_scale, 1e-30)
