"""Parity of the prefill / extend kernel (mla_prefill_fwd, un-absorbed MLA,
head dim 192 = 128 + 64 shared rope, v 128) with the fp64 oracle, at the bar
of the bf16 decode: max|O - O_ref| <= 1e-2 * max|O_ref|, |LSE - LSE_ref| <= 1e-3."""
import numpy as np
import pytest
import torch

import oracle
import mla_decode_attention_amd as mla
from workloads import make_prefill_workload, prefill_config

pytestmark = pytest.mark.gpu

O_REL_TOL = 1e-2
LSE_TOL = 1e-3


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def run(w):
    q, kn, kr, v = _dev(w.q_bits), _dev(w.k_nope_bits), _dev(w.k_rope_bits), _dev(w.v_bits)
    cq = torch.from_numpy(w.cu_q).cuda()
    ck = torch.from_numpy(w.cu_k).cuda()
    out, lse = mla.prefill(q, kn, kr, v, cq, ck, int(w.q_lens.max()), w.softmax_scale)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def check(out, lse, ref_o, ref_l, what):
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    err = float(np.max(np.abs(out - ref_o)))
    scale = float(np.max(np.abs(ref_o)))
    assert err <= O_REL_TOL * scale, f"{what}: O err {err:.3e} vs max|O| {scale:.3e}"
    lerr = float(np.max(np.abs(lse - ref_l)))
    assert lerr <= LSE_TOL, f"{what}: LSE err {lerr:.3e}"


def reference(w):
    return oracle.mla_prefill(w.q_bits, w.k_nope_bits, w.k_rope_bits, w.v_bits, w.cu_q, w.cu_k,
                              w.softmax_scale)


@pytest.mark.parametrize("name", ["prefill", "extend"])
def test_small_configs(name):
    w = prefill_config(name, small=True, seed=1)
    out, lse = run(w)
    check(out, lse, *reference(w), name)


@pytest.mark.parametrize("H", [1, 16, 128])
def test_lengths_and_heads(H):
    """Query blocks of 128 with ragged ends, one-token sequences, extends
    whose prefix is not a multiple of the 64-key tile."""
    q_lens = [1, 127, 128, 129, 200, 3, 64]
    k_lens = [1, 127, 128, 129, 333, 70, 64]
    w = make_prefill_workload("shapes", q_lens, k_lens, H, seed=H)
    out, lse = run(w)
    check(out, lse, *reference(w), f"H={H}")


def test_batch_with_an_empty_sequence():
    w = make_prefill_workload("empty", [5, 0, 7], [9, 4, 7], 4, seed=3)
    q, kn, kr, v = _dev(w.q_bits), _dev(w.k_nope_bits), _dev(w.k_rope_bits), _dev(w.v_bits)
    out = torch.full((12, 4, 128), 7.0, device="cuda")
    lse = torch.full((12, 4), 7.0, device="cuda")
    mla.prefill(q, kn, kr, v, torch.from_numpy(w.cu_q).cuda(), torch.from_numpy(w.cu_k).cuda(), 7,
                w.softmax_scale, out=out, lse=lse)
    torch.cuda.synchronize()
    ref_o, ref_l = reference(w)
    check(out.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, "with an empty sequence")


def test_run_to_run_bitwise():
    w = prefill_config("extend", small=True, seed=4)
    o1, l1 = run(w)
    o2, l2 = run(w)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("name", ["prefill", "extend"])
def test_full_size_sampled(name):
    """The full workload in the launch configuration the bench times; sampled
    rows checked one by one (a single query at position p sees keys 0..p)."""
    w = prefill_config(name, seed=0)
    out, lse = run(w)
    rng = np.random.default_rng(9)
    for b in range(w.batch):
        q0, q1 = int(w.cu_q[b]), int(w.cu_q[b + 1])
        k0, k1 = int(w.cu_k[b]), int(w.cu_k[b + 1])
        N, L = q1 - q0, k1 - k0
        for i in sorted(set([0, N - 1, N // 2] + list(rng.integers(0, N, 3)))):
            p = L - N + i
            ro, rl = oracle.mla_prefill(w.q_bits[q0 + i:q0 + i + 1], w.k_nope_bits[k0:k0 + p + 1],
                                        w.k_rope_bits[k0:k0 + p + 1], w.v_bits[k0:k0 + p + 1],
                                        np.array([0, 1], np.int32), np.array([0, p + 1], np.int32),
                                        w.softmax_scale)
            check(out[q0 + i:q0 + i + 1], lse[q0 + i:q0 + i + 1], ro, rl, f"{name} b={b} i={i}")


def test_negative_softmax_scale():
    """The API takes any finite scale: with a negative one the row max is the
    most negative dot product, which the kernel handles by negating q."""
    w = make_prefill_workload("neg", [1, 127, 129, 40], [1, 127, 129, 200], 4, seed=6)
    w.softmax_scale = -0.11
    out, lse = run(w)
    check(out, lse, *reference(w), "negative scale")
