"""Cache append (mla_append_kv) against the oracle, bit for bit, and a decode
step on the appended cache against the oracle at the parity bar."""
import numpy as np
import pytest
import torch

import oracle
import mla_decode_attention_amd as mla
from workloads import make_workload, f32_to_bf16_bits, PAGE_TOKENS
from _gpu_util import to_device, run_gpu, assert_parity

pytestmark = pytest.mark.gpu


def _bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _latents(rng, B, s, kind):
    x = rng.normal(size=(B, s, 576)).astype(np.float32)
    if kind == "mixed":
        x[0, 0] = 0.0                                    # all-zero row: scale 1, zero codes
        if s > 1:
            x[0, 1] *= 2.0 ** -12                        # tiny row
        x[-1, -1] *= 1.0e4                               # large row
        x[1 % B, 0, ::7] *= 2.0 ** -10                   # subnormal codes inside a normal row
    return f32_to_bf16_bits(x)


def _grid_row():
    """One latent row whose scale is exactly 1 (max 448) and whose other values
    are every finite E4M3FN value and every midpoint between neighbours, both
    signs: the conversion's rounding is then checked on every code and tie."""
    pos = [oracle.e4m3fn_value(c) for c in range(0x7F)]
    vals = [448.0] + pos[:-1] + [(pos[k] + pos[k + 1]) / 2 for k in range(0x7E)]
    vals += [-v for v in vals[1:]]
    row = np.zeros(576, np.float32)
    row[:len(vals)] = np.array(vals, np.float32)
    bits = f32_to_bf16_bits(row)
    assert np.array_equal(oracle.bf16_bits_to_f64(bits), row.astype(np.float64))   # all exact in bf16
    return bits


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("s", [1, 3])
def test_append_matches_oracle_bitwise(kv_dtype, s):
    rng = np.random.default_rng(40 + s)
    lens = [1, 2, 63, 64, 65, 300, 1000]
    w = make_workload("append", len(lens), 16, 1, lens, kv_dtype=kv_dtype, seed=11 + s, poison_tail=False)
    lat = _latents(rng, len(lens), s, "mixed")
    if kv_dtype == "fp8_e4m3":
        lat[2, 0] = _grid_row()
    ref_cache, ref_scale = oracle.append_kv(lat, w.block_table, w.seqlens, w.cache, w.kv_scale, kv_dtype)
    d = to_device(w)
    mla.append_kv(_bf16_dev(lat), d["block_table"], d["seqlens"], d["kv"], d["kv_scale"])
    torch.cuda.synchronize()
    got = d["kv"].cpu()
    got = got.view(torch.int16).numpy().view(np.uint16) if kv_dtype == "bf16" else got.numpy()
    assert np.array_equal(got, ref_cache), "cache bytes differ"
    if kv_dtype == "fp8_e4m3":
        assert np.array_equal(d["kv_scale"].cpu().numpy().view(np.uint32), ref_scale.view(np.uint32))


def test_append_skips_invalid_positions_and_pages():
    # position < 0 (L < new_tokens), a page id past the pool and -1: nothing is written
    B, s = 3, 2
    seqlens = np.array([1, 70, 64], np.int32)
    bt = np.array([[0, -1], [1, 99], [-1, 2]], np.int32)     # seq 1 pos 68,69 -> page 99 (invalid); seq 2 pos 62,63 -> page -1
    pool = np.full((3, 64, 576), 0x1234, np.uint16)
    lat = f32_to_bf16_bits(np.random.default_rng(3).normal(size=(B, s, 576)).astype(np.float32))
    kv = _bf16_dev(pool)
    mla.append_kv(_bf16_dev(lat), torch.from_numpy(bt).cuda(), torch.from_numpy(seqlens).cuda(), kv)
    torch.cuda.synchronize()
    got = kv.cpu().view(torch.int16).numpy().view(np.uint16)
    expect = pool.copy()
    expect[0, 0] = lat[0, 1]                                    # only seq 0 token 1 (position 0) lands
    assert np.array_equal(got, expect)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
def test_decode_step_after_append(kv_dtype):
    """One decode step: append the q_len new tokens' latents, then attend with the
    same cache_seqlens; compared with the oracle on the oracle-appended cache."""
    rng = np.random.default_rng(77)
    lens = [2, 65, 300, 129]
    w = make_workload("step", len(lens), 16, 2, lens, kv_dtype=kv_dtype, seed=21, poison_tail=False)
    lat = _latents(rng, len(lens), 2, "normal")
    w.cache, w.kv_scale = oracle.append_kv(lat, w.block_table, w.seqlens, w.cache, w.kv_scale, kv_dtype)
    ref_out, ref_lse = oracle.mla_decode(w.q_bits, w.cache, w.block_table, w.seqlens, w.softmax_scale,
                                         w.kv_dtype, w.kv_scale)
    w2 = make_workload("step", len(lens), 16, 2, lens, kv_dtype=kv_dtype, seed=21, poison_tail=False)
    d = to_device(w2)                        # cache before the append
    mla.append_kv(_bf16_dev(lat), d["block_table"], d["seqlens"], d["kv"], d["kv_scale"])
    out, lse, _ = run_gpu(w, d, split=True, num_units=5, min_tiles=1)
    assert_parity(w, out, lse, ref_out, ref_lse, f"append+decode {kv_dtype}")
