"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments from the host before touching any device (runs without a GPU)."""
import ctypes
import os
import re

import pytest

import mla_decode_attention_amd as mla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_decode.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = ctypes.c_void_p(0x10000)        # never dereferenced: calls must fail first
FAKE_ODD = ctypes.c_void_p(0x10008)    # 8-byte aligned, not 16


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return mla.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert "mla_decode_fwd" in names and "mla_get_split_metadata" in names and "mla_combine" in names
    for n in names:
        assert hasattr(lib, n), n


def test_bounds_checking_build_exports_the_same_symbols():
    path = os.path.join(os.path.dirname(mla.library_path()), "libmla_decode_debug.so")
    if not os.path.exists(path):
        pytest.skip("libmla_decode_debug.so not built")
    dbg = ctypes.CDLL(path)
    for n in declared_functions():
        assert hasattr(dbg, n), n


def test_abi_and_status_strings(lib):
    assert lib.mla_abi_version() == 2
    assert lib.mla_status_string(0) == b"MLA_OK"
    assert lib.mla_status_string(3) == b"MLA_ERR_WORKSPACE"
    assert lib.mla_status_string(99) == b"MLA_ERR_UNKNOWN"


def test_sizes(lib):
    assert lib.mla_metadata_bytes(64, 256) == 4 * (8 + 2 * 65 + 256 + 257 + 64)
    # (B + units) partial slots x rows x (512 + 1) fp32
    assert lib.mla_workspace_bytes(64, 1, 16, 256) == 320 * 16 * 512 * 4 + ((320 * 16 * 4 + 255) // 256) * 256
    assert lib.mla_metadata_bytes(0, 4) == 0
    assert lib.mla_workspace_bytes(1, 0, 16, 4) == 0


def _decode(lib, **kw):
    a = dict(q=FAKE, kv=FAKE, scale=None, dtype=0, pages=4, bt=FAKE, maxp=4, sl=FAKE, B=1, s=1, H=16,
             sm=0.072, out=FAKE, lse=FAKE, md=None, units=0, ws=None, wsb=0)
    a.update(kw)
    return lib.mla_decode_fwd(a["q"], a["kv"], a["scale"], a["dtype"], a["pages"], a["bt"], a["maxp"],
                              a["sl"], a["B"], a["s"], a["H"], a["sm"], a["out"], a["lse"], a["md"],
                              a["units"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), INVALID),
    (dict(kv=None), INVALID),
    (dict(out=None), INVALID),
    (dict(B=0), INVALID),
    (dict(s=0), INVALID),
    (dict(H=0), INVALID),
    (dict(s=6, H=1024), INVALID),            # rows over the limit
    (dict(s=1, H=4097), INVALID),            # one row over the limit (4096 rows per sequence)
    (dict(pages=0), INVALID),
    (dict(maxp=0), INVALID),
    (dict(sm=float("nan")), INVALID),
    (dict(sm=float("inf")), INVALID),
    (dict(q=FAKE_ODD), INVALID),
    (dict(out=FAKE_ODD), INVALID),
    (dict(dtype=7), UNSUPPORTED),
    (dict(dtype=1), INVALID),                # fp8 without scales
    (dict(md=FAKE, units=0, ws=FAKE, wsb=1 << 30), INVALID),
    (dict(md=FAKE, units=8, ws=None), INVALID),
    (dict(md=FAKE, units=8, ws=FAKE, wsb=1024), WORKSPACE),
])
def test_decode_argument_errors(lib, kw, expect):
    st = _decode(lib, **kw)
    assert st == expect, (st, lib.mla_last_error())
    assert lib.mla_last_error() != b""


def test_metadata_argument_errors(lib):
    f = lib.mla_get_split_metadata
    assert f(None, 4, 1, 16, 8, 0, FAKE, 1 << 20, None) == INVALID
    assert f(FAKE, 0, 1, 16, 8, 0, FAKE, 1 << 20, None) == INVALID
    assert f(FAKE, 4, 0, 16, 8, 0, FAKE, 1 << 20, None) == INVALID
    assert f(FAKE, 4, 1, 0, 8, 0, FAKE, 1 << 20, None) == INVALID
    assert f(FAKE, 4, 1, 16, 0, 0, FAKE, 1 << 20, None) == INVALID
    assert f(FAKE, 4, 1, 16, 8, -1, FAKE, 1 << 20, None) == INVALID
    assert f(FAKE, 4, 1, 16, 8, 0, FAKE, 16, None) == WORKSPACE


def test_combine_argument_errors(lib):
    f = lib.mla_combine
    assert f(None, FAKE, FAKE, 2, 16, FAKE, FAKE, None) == INVALID
    assert f(FAKE, FAKE, FAKE, 0, 16, FAKE, FAKE, None) == INVALID
    assert f(FAKE, FAKE, FAKE, 2, 0, FAKE, FAKE, None) == INVALID
    assert f(FAKE, FAKE, FAKE, 2, 5000, FAKE, FAKE, None) == INVALID
    assert f(FAKE_ODD, FAKE, FAKE, 2, 16, FAKE, FAKE, None) == INVALID


def test_append_argument_errors(lib):
    f = lib.mla_append_kv
    ok_args = dict(lat=FAKE, B=2, s=1, bt=FAKE, maxp=4, sl=FAKE, kv=FAKE, sc=None, dt=0, P=8)
    def call(**kw):
        a = dict(ok_args, **kw)
        return f(a["lat"], a["B"], a["s"], a["bt"], a["maxp"], a["sl"], a["kv"], a["sc"], a["dt"], a["P"], None)
    assert call(lat=None) == INVALID
    assert call(B=0) == INVALID
    assert call(s=0) == INVALID
    assert call(P=0) == INVALID
    assert call(dt=7) == UNSUPPORTED
    assert call(dt=1, sc=None) == INVALID           # fp8 needs scales
    assert call(dt=0, sc=FAKE) == INVALID           # bf16 takes none
    assert call(lat=FAKE_ODD) == INVALID
    assert call(kv=FAKE_ODD) == INVALID


def test_varlen_argument_errors(lib):
    f = lib.mla_decode_fwd_varlen
    def call(cu=FAKE, T=4, mq=2, H=16):
        return f(FAKE, cu, T, mq, FAKE, None, 0, 4, FAKE, 4, FAKE, 2, H, ctypes.c_float(0.072), FAKE, FAKE,
                 None, 0, None, 0, None)
    assert call(cu=None) == INVALID
    assert call(T=0) == INVALID
    assert call(mq=0) == INVALID
    assert call(mq=300, H=16) == INVALID      # rows over the limit


def test_fp8mma_argument_errors(lib):
    f = lib.mla_decode_fwd_fp8mma
    def call(dtype=1, scale=FAKE, q=FAKE, s=1):
        return f(q, FAKE, scale, dtype, 4, FAKE, 4, FAKE, 1, s, 16, ctypes.c_float(0.072), FAKE, FAKE,
                 None, 0, None, 0, None)
    assert call(dtype=0, scale=None) == UNSUPPORTED   # bf16 cache: no fp8 contraction path
    assert call(dtype=1, scale=None) == INVALID       # fp8 needs scales
    assert call(q=None) == INVALID
    assert call(s=0) == INVALID
    assert lib.mla_last_error() != b""


def test_prefill_argument_errors(lib):
    f = lib.mla_prefill_fwd
    def call(q=FAKE, cu=FAKE, B=2, mq=128, H=16, sm=0.072, out=FAKE):
        return f(q, FAKE, FAKE, FAKE, cu, FAKE, B, mq, H, ctypes.c_float(sm), out, FAKE, None)
    assert call(q=None) == INVALID
    assert call(cu=None) == INVALID
    assert call(B=0) == INVALID
    assert call(mq=0) == INVALID
    assert call(H=0) == INVALID
    assert call(H=70000) == INVALID
    # (query blocks x sequences x heads) past the 32-bit workgroup index
    assert call(B=40000, mq=1 << 15, H=256) == INVALID
    assert call(sm=float("nan")) == INVALID
    assert call(q=FAKE_ODD) == INVALID
    assert call(out=FAKE_ODD) == INVALID


def test_binding_rejects_host_tensors():
    import torch
    q = torch.zeros(1, 1, 16, 576, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mla.decode(q, q, q, q, 0.1)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import importlib
    monkeypatch.setattr(mla, "_lib", None)
    monkeypatch.setattr(mla, "library_path", lambda: str(tmp_path / "missing.so"))
    with pytest.raises(mla.MLAError):
        mla.load_library()
