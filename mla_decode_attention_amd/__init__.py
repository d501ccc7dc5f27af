"""MLA decode over a paged latent KV cache on MI355X (gfx950).

Thin Python binding of libmla_decode.so (C ABI in include/mla_decode.h):
argument checking of tensor types/shapes and marshalling of device pointers
and the current HIP stream. Every step of the computation runs in the HIP
kernels of the library; there is no fallback: if the library is not built or
cannot be loaded, every call raises.

    append_kv(latent, block_table, cache_seqlens, kv_cache)          # new tokens' rows
    plan = get_split_metadata(cache_seqlens, q_len, num_heads)     # once per step
    out, lse = decode(q, kv_cache, block_table, cache_seqlens, scale, plan=plan)
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

__all__ = ["load_library", "library_path", "abi_version", "default_num_units", "metadata_bytes",
           "workspace_bytes", "SplitPlan", "profile_enable", "profile_read", "profile_read_launches",
           "PROFILE_ATTENTION", "PROFILE_METADATA", "PROFILE_COMBINE", "get_split_metadata", "decode",
           "decode_varlen", "decode_noalloc", "combine", "append_kv", "prefill", "PROFILE_QUANTIZE",
           "prefill_quant_kv_bytes", "prefill_quantize_kv", "prefill_quant",
           "use_debug_library", "debug_page_violations",
           "MLAError", "KV_BF16", "KV_FP8_E4M3", "PAGE_TOKENS", "D_QK", "D_V"]

PAGE_TOKENS = 64
D_QK = 576
D_V = 512
KV_BF16 = 0
KV_FP8_E4M3 = 1
_LIB_NAME = "libmla_decode.so"
_DEBUG_LIB_NAME = "libmla_decode_debug.so"
_lib = None
_use_debug = False


class MLAError(RuntimeError):
    pass


def library_path() -> str:
    name = _DEBUG_LIB_NAME if _use_debug else _LIB_NAME
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), name)


def use_debug_library(enable: bool) -> None:
    """Route every later call through libmla_decode_debug.so (built with
    MLA_DEBUG_BOUNDS: page ids checked against the pool) or back through the
    release library."""
    global _lib, _use_debug
    if bool(enable) != _use_debug:
        _use_debug = bool(enable)
        _lib = None


def load_library():
    """Load libmla_decode.so (built in-tree by mla_decode_attention_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise MLAError(f"{path} is missing: build it with `python -m mla_decode_attention_amd.build`")
    lib = ctypes.CDLL(path)
    c_int, c_size, vp = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
    sigs = {
        "mla_abi_version": (c_int, []),
        "mla_status_string": (ctypes.c_char_p, [c_int]),
        "mla_last_error": (ctypes.c_char_p, []),
        "mla_default_num_units": (c_int, [c_int, c_int, c_int]),
        "mla_default_num_units_varlen": (c_int, [c_int, c_int, c_int]),
        "mla_metadata_bytes": (c_size, [c_int, c_int]),
        "mla_workspace_bytes": (c_size, [c_int, c_int, c_int, c_int]),
        "mla_get_split_metadata": (c_int, [vp, c_int, c_int, c_int, c_int, c_int, vp, c_size, vp]),
        "mla_decode_fwd": (c_int, [vp, vp, vp, c_int, c_int, vp, c_int, vp, c_int, c_int, c_int,
                                   ctypes.c_float, vp, vp, vp, c_int, vp, c_size, vp]),
        "mla_decode_fwd_fp8mma": (c_int, [vp, vp, vp, c_int, c_int, vp, c_int, vp, c_int, c_int, c_int,
                                          ctypes.c_float, vp, vp, vp, c_int, vp, c_size, vp]),
        "mla_combine": (c_int, [vp, vp, vp, c_int, c_int, vp, vp, vp]),
        "mla_prefill_fwd": (c_int, [vp, vp, vp, vp, vp, vp, c_int, c_int, c_int, ctypes.c_float, vp, vp, vp]),
        "mla_prefill_quant_kv_bytes": (c_size, [c_int, ctypes.c_int64, c_int]),
        "mla_prefill_quantize_kv": (c_int, [vp, vp, vp, vp, c_int, ctypes.c_int64, c_int, vp, c_size, vp]),
        "mla_prefill_quant_fwd": (c_int, [vp, vp, c_size, vp, vp, c_int, c_int, ctypes.c_int64, c_int,
                                          ctypes.c_float, vp, vp, vp]),
        "mla_append_kv": (c_int, [vp, c_int, c_int, vp, c_int, vp, vp, vp, c_int, c_int, vp]),
        "mla_decode_fwd_varlen": (c_int, [vp, vp, c_int, c_int, vp, vp, c_int, c_int, vp, c_int, vp, c_int,
                                          c_int, ctypes.c_float, vp, vp, vp, c_int, vp, c_size, vp]),
        "mla_decode_fwd_noalloc": (c_int, [vp, vp, vp, c_int, c_int, vp, c_int, vp, c_int, c_int, c_int,
                                           ctypes.c_float, vp, vp, c_int, c_int, vp]),
        "mla_noalloc_scratch_need": (c_size, [c_int, c_int, c_int, c_int]),
        "mla_debug_page_violations": (c_int, [c_int, ctypes.POINTER(ctypes.c_uint64)]),
        "mla_profile_enable": (c_int, [c_int]),
        "mla_profile_read": (c_int, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(c_int)]),
        "mla_profile_read_launches": (c_int, [c_int, ctypes.POINTER(ctypes.c_float), c_int,
                                              ctypes.POINTER(c_int)]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int, what: str):
    if status != 0:
        lib = load_library()
        raise MLAError(f"{what}: {lib.mla_status_string(status).decode()}: "
                       f"{lib.mla_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t: torch.Tensor, name: str, dtypes, ndim=None, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the other tensors on {device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _plan_buffers(plan, dev):
    """(metadata, workspace, num_units, workspace bytes) of a plan, checked."""
    _need(plan.metadata, "plan.metadata", (torch.int32,), 1, device=dev)
    _need(plan.workspace, "plan.workspace", (torch.uint8,), 1, device=dev)
    return plan.metadata, plan.workspace, plan.num_units, _nbytes(plan.workspace)


def _check_cache(kv_cache, kv_scale, dev):
    """(kv_dtype, num_pages) of a [P, 64, 576] cache, with its scales checked."""
    fp8_types = (torch.uint8,) + ((torch.float8_e4m3fn,) if hasattr(torch, "float8_e4m3fn") else ())
    _need(kv_cache, "kv_cache", (torch.bfloat16,) + fp8_types, 3, device=dev)
    if tuple(kv_cache.shape[1:]) != (PAGE_TOKENS, D_QK):
        raise ValueError(f"kv_cache must be [pages, {PAGE_TOKENS}, {D_QK}]")
    P = kv_cache.shape[0]
    kv_dtype = KV_BF16 if kv_cache.dtype == torch.bfloat16 else KV_FP8_E4M3
    if kv_dtype == KV_FP8_E4M3:
        if kv_scale is None:
            raise ValueError("fp8 cache needs kv_scale")
        _need(kv_scale, "kv_scale", (torch.float32,), 2, shape=(P, PAGE_TOKENS), device=dev)
    elif kv_scale is not None:
        raise ValueError("kv_scale is only for an fp8 cache")
    return kv_dtype, P


def abi_version() -> int:
    return load_library().mla_abi_version()


def default_num_units(batch: int, q_len: int, num_heads: int, varlen: bool = False) -> int:
    """Library default unit count (varlen: for decode_varlen, q_len = max_q_len)."""
    lib = load_library()
    f = lib.mla_default_num_units_varlen if varlen else lib.mla_default_num_units
    return f(batch, q_len, num_heads)


def metadata_bytes(batch: int, num_units: int) -> int:
    return load_library().mla_metadata_bytes(batch, num_units)


def workspace_bytes(batch: int, q_len: int, num_heads: int, num_units: int) -> int:
    return load_library().mla_workspace_bytes(batch, q_len, num_heads, num_units)


@dataclass
class SplitPlan:
    """Split schedule on the device plus the partials workspace it needs."""
    metadata: torch.Tensor     # int32, device
    num_units: int
    batch: int
    q_len: int
    num_heads: int
    workspace: torch.Tensor    # uint8, device


def get_split_metadata(cache_seqlens: torch.Tensor, q_len: int, num_heads: int,
                       num_units: Optional[int] = None, min_tiles_per_unit: int = 0,
                       metadata: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None, varlen: bool = False) -> SplitPlan:
    """Build the split-KV schedule for one decode step (reusable across layers).

    varlen: the plan is for decode_varlen (q_len = max_q_len); only changes
    the default unit count."""
    lib = load_library()
    _need(cache_seqlens, "cache_seqlens", (torch.int32,), 1)
    batch = cache_seqlens.shape[0]
    if num_units is None:
        num_units = (lib.mla_default_num_units_varlen if varlen else lib.mla_default_num_units)(
            batch, q_len, num_heads)
        if num_units < 1:
            raise MLAError(f"mla_default_num_units failed: {lib.mla_last_error().decode()}")
    dev = cache_seqlens.device
    nbytes = lib.mla_metadata_bytes(batch, num_units)
    if metadata is None:
        metadata = torch.empty((nbytes + 3) // 4, dtype=torch.int32, device=dev)
    _need(metadata, "metadata", (torch.int32,), 1, device=dev)
    wbytes = lib.mla_workspace_bytes(batch, q_len, num_heads, num_units)
    if workspace is None:
        workspace = torch.empty(wbytes, dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", (torch.uint8,), 1, device=dev)
    _check(lib.mla_get_split_metadata(_ptr(cache_seqlens), batch, q_len, num_heads, num_units,
                                      min_tiles_per_unit, _ptr(metadata), _nbytes(metadata), _stream()),
           "mla_get_split_metadata")
    return SplitPlan(metadata, num_units, batch, q_len, num_heads, workspace)


def decode(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
           cache_seqlens: torch.Tensor, softmax_scale: float, kv_scale: Optional[torch.Tensor] = None,
           plan: Optional[SplitPlan] = None, out: Optional[torch.Tensor] = None,
           lse: Optional[torch.Tensor] = None, fp8_mma: bool = False):
    """MLA decode attention. Returns (out fp32 [B,s,H,512], lse fp32 [B,s,H]).

    q bf16 [B, s, H, 576]; kv_cache [P, 64, 576] bf16 (or uint8 / float8_e4m3fn
    codes with kv_scale fp32 [P, 64]); block_table int32 [B, max_pages];
    cache_seqlens int32 [B]. plan=None runs one work unit per sequence.
    fp8_mma=True (fp8 cache only) runs mla_decode_fwd_fp8mma: queries and P
    quantised to E4M3, an approximation of the default path.
    """
    lib = load_library()
    _need(q, "q", (torch.bfloat16,), 4)
    dev = q.device
    B, s, H, d = q.shape
    if d != D_QK:
        raise ValueError(f"q last dim must be {D_QK}")
    kv_dtype, P = _check_cache(kv_cache, kv_scale, dev)
    _need(block_table, "block_table", (torch.int32,), 2, device=dev)
    _need(cache_seqlens, "cache_seqlens", (torch.int32,), 1, shape=(B,), device=dev)
    if block_table.shape[0] != B:
        raise ValueError("block_table / cache_seqlens batch mismatch")
    if out is None:
        out = torch.empty((B, s, H, D_V), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, s, H), dtype=torch.float32, device=dev)
    _need(out, "out", (torch.float32,), 4, shape=(B, s, H, D_V), device=dev)
    _need(lse, "lse", (torch.float32,), 3, shape=(B, s, H), device=dev)
    md = ws = None
    units, wbytes = 0, 0
    if plan is not None:
        if (plan.batch, plan.q_len, plan.num_heads) != (B, s, H):
            raise ValueError("plan was built for another shape")
        md, ws, units, wbytes = _plan_buffers(plan, dev)
    name = "mla_decode_fwd_fp8mma" if fp8_mma else "mla_decode_fwd"
    _check(getattr(lib, name)(_ptr(q), _ptr(kv_cache), _ptr(kv_scale), kv_dtype, P,
                              _ptr(block_table), block_table.shape[1], _ptr(cache_seqlens), B, s, H,
                              float(softmax_scale), _ptr(out), _ptr(lse), _ptr(md), units, _ptr(ws),
                              wbytes, _stream()), name)
    return out, lse


def decode_noalloc(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
                   cache_seqlens: torch.Tensor, softmax_scale: float, kv_scale: Optional[torch.Tensor] = None,
                   num_units: int = 0, min_tiles_per_unit: int = 0, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None):
    """Split decode whose schedule and partials live in the library's static
    device buffer (mla_decode_fwd_noalloc): no workspace, no allocation in the
    library (out / lse are allocated here only when not given)."""
    lib = load_library()
    _need(q, "q", (torch.bfloat16,), 4)
    dev = q.device
    B, s, H, d = q.shape
    if d != D_QK:
        raise ValueError(f"q last dim must be {D_QK}")
    kv_dtype, P = _check_cache(kv_cache, kv_scale, dev)
    _need(block_table, "block_table", (torch.int32,), 2, device=dev)
    _need(cache_seqlens, "cache_seqlens", (torch.int32,), 1, shape=(B,), device=dev)
    if block_table.shape[0] != B:
        raise ValueError("block_table / cache_seqlens batch mismatch")
    if out is None:
        out = torch.empty((B, s, H, D_V), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, s, H), dtype=torch.float32, device=dev)
    _need(out, "out", (torch.float32,), 4, shape=(B, s, H, D_V), device=dev)
    _need(lse, "lse", (torch.float32,), 3, shape=(B, s, H), device=dev)
    _check(lib.mla_decode_fwd_noalloc(_ptr(q), _ptr(kv_cache), _ptr(kv_scale), kv_dtype, P, _ptr(block_table),
                                      block_table.shape[1], _ptr(cache_seqlens), B, s, H, float(softmax_scale),
                                      _ptr(out), _ptr(lse), int(num_units), int(min_tiles_per_unit), _stream()),
           "mla_decode_fwd_noalloc")
    return out, lse


def prefill(q: torch.Tensor, k_nope: torch.Tensor, k_rope: torch.Tensor, v: torch.Tensor,
            cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor, max_q_len: int, softmax_scale: float,
            out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """Prefill / extend attention, un-absorbed MLA. Returns (out fp32 [Tq,H,128], lse fp32 [Tq,H]).

    q bf16 [Tq, H, 192]; k_nope bf16 [Tk, H, 128]; k_rope bf16 [Tk, 64]; v bf16
    [Tk, H, 128]; cu_seqlens_q / cu_seqlens_k int32 [B+1]. Sequence b's
    queries are the last N_b of its L_b tokens (causal).
    """
    lib = load_library()
    _need(q, "q", (torch.bfloat16,), 3)
    Tq, H, d = q.shape
    if d != 192:
        raise ValueError("q last dim must be 192")
    dev = q.device
    _need(k_nope, "k_nope", (torch.bfloat16,), 3, device=dev)
    _need(k_rope, "k_rope", (torch.bfloat16,), 2, device=dev)
    _need(v, "v", (torch.bfloat16,), 3, device=dev)
    Tk = k_nope.shape[0]
    if tuple(k_nope.shape) != (Tk, H, 128) or tuple(k_rope.shape) != (Tk, 64) or tuple(v.shape) != (Tk, H, 128):
        raise ValueError("k_nope [Tk,H,128], k_rope [Tk,64], v [Tk,H,128] expected")
    _need(cu_seqlens_q, "cu_seqlens_q", (torch.int32,), 1, device=dev)
    _need(cu_seqlens_k, "cu_seqlens_k", (torch.int32,), 1, device=dev)
    B = cu_seqlens_q.shape[0] - 1
    if B < 1 or cu_seqlens_k.shape[0] != B + 1:
        raise ValueError("cu_seqlens_q / cu_seqlens_k must both have batch + 1 entries")
    if out is None:
        out = torch.empty((Tq, H, 128), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((Tq, H), dtype=torch.float32, device=dev)
    _need(out, "out", (torch.float32,), 3, shape=(Tq, H, 128), device=dev)
    _need(lse, "lse", (torch.float32,), 2, shape=(Tq, H), device=dev)
    _check(lib.mla_prefill_fwd(_ptr(q), _ptr(k_nope), _ptr(k_rope), _ptr(v), _ptr(cu_seqlens_q),
                               _ptr(cu_seqlens_k), B, int(max_q_len), H, float(softmax_scale), _ptr(out),
                               _ptr(lse), _stream()), "mla_prefill_fwd")
    return out, lse


def _prefill_kv_args(k_nope, k_rope, v, cu_seqlens_k, H=None):
    dev = k_nope.device
    _need(k_nope, "k_nope", (torch.bfloat16,), 3)
    Tk = k_nope.shape[0]
    H = k_nope.shape[1] if H is None else H
    _need(k_nope, "k_nope", (torch.bfloat16,), 3, shape=(Tk, H, 128), device=dev)
    _need(k_rope, "k_rope", (torch.bfloat16,), 2, shape=(Tk, 64), device=dev)
    _need(v, "v", (torch.bfloat16,), 3, shape=(Tk, H, 128), device=dev)
    _need(cu_seqlens_k, "cu_seqlens_k", (torch.int32,), 1, device=dev)
    B = cu_seqlens_k.shape[0] - 1
    if B < 1:
        raise ValueError("cu_seqlens_k must have batch + 1 >= 2 entries")
    return Tk, H, B


def prefill_quant_kv_bytes(batch: int, total_k: int, num_heads: int) -> int:
    """Bytes of the quantised K/V buffer of prefill_quantize_kv."""
    return int(load_library().mla_prefill_quant_kv_bytes(int(batch), int(total_k), int(num_heads)))


def prefill_quantize_kv(k_nope: torch.Tensor, k_rope: torch.Tensor, v: torch.Tensor, cu_seqlens_k: torch.Tensor,
                        qkv: Optional[torch.Tensor] = None) -> torch.Tensor:
    """K to INT8 and V to FP8 for prefill_quant (layout in include/mla_decode.h).
    Returns the uint8 buffer (allocated when qkv is None)."""
    lib = load_library()
    Tk, H, B = _prefill_kv_args(k_nope, k_rope, v, cu_seqlens_k)
    nbytes = prefill_quant_kv_bytes(B, Tk, H)
    if qkv is None:
        qkv = torch.empty(nbytes, dtype=torch.uint8, device=k_nope.device)
    _need(qkv, "qkv", (torch.uint8,), 1, device=k_nope.device)
    _check(lib.mla_prefill_quantize_kv(_ptr(k_nope), _ptr(k_rope), _ptr(v), _ptr(cu_seqlens_k), B, Tk, H,
                                       _ptr(qkv), _nbytes(qkv), _stream()), "mla_prefill_quantize_kv")
    return qkv


def prefill_quant(q: torch.Tensor, k_nope: torch.Tensor, k_rope: torch.Tensor, v: torch.Tensor,
                  cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor, max_q_len: int, softmax_scale: float,
                  out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                  qkv: Optional[torch.Tensor] = None, quantize: bool = True):
    """Quantised prefill / extend (INT8 Q.K^T, FP8 P.V). Arguments as prefill();
    K and V are quantised into qkv first (skipped with quantize=False, for a
    qkv that prefill_quantize_kv already filled from the same K, V and
    cu_seqlens_k). Returns (out fp32 [Tq,H,128], lse fp32 [Tq,H])."""
    lib = load_library()
    _need(q, "q", (torch.bfloat16,), 3)
    Tq, H, d = q.shape
    if d != 192:
        raise ValueError("q last dim must be 192")
    dev = q.device
    Tk, _, B = _prefill_kv_args(k_nope, k_rope, v, cu_seqlens_k, H)
    _need(cu_seqlens_q, "cu_seqlens_q", (torch.int32,), 1, shape=(B + 1,), device=dev)
    if quantize:
        qkv = prefill_quantize_kv(k_nope, k_rope, v, cu_seqlens_k, qkv)
    elif qkv is None:
        raise ValueError("quantize=False needs a filled qkv")
    _need(qkv, "qkv", (torch.uint8,), 1, device=dev)
    if out is None:
        out = torch.empty((Tq, H, 128), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((Tq, H), dtype=torch.float32, device=dev)
    _need(out, "out", (torch.float32,), 3, shape=(Tq, H, 128), device=dev)
    _need(lse, "lse", (torch.float32,), 2, shape=(Tq, H), device=dev)
    _check(lib.mla_prefill_quant_fwd(_ptr(q), _ptr(qkv), _nbytes(qkv), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), B,
                                     int(max_q_len), Tk, H, float(softmax_scale), _ptr(out), _ptr(lse), _stream()),
           "mla_prefill_quant_fwd")
    return out, lse


def decode_varlen(q: torch.Tensor, cu_seqlens_q: torch.Tensor, max_q_len: int, kv_cache: torch.Tensor,
                  block_table: torch.Tensor, cache_seqlens: torch.Tensor, softmax_scale: float,
                  kv_scale: Optional[torch.Tensor] = None, plan: Optional[SplitPlan] = None,
                  out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """MLA decode with a query count per sequence. Returns (out fp32 [T,H,512], lse fp32 [T,H]).

    q bf16 [T, H, 576]; cu_seqlens_q int32 [B+1] (sequence b owns q rows
    cu[b]..cu[b+1], at most max_q_len of them); other arguments as decode().
    A plan comes from get_split_metadata(cache_seqlens, max_q_len, H).
    """
    lib = load_library()
    _need(q, "q", (torch.bfloat16,), 3)
    T, H, d = q.shape
    if d != D_QK:
        raise ValueError(f"q last dim must be {D_QK}")
    dev = q.device
    _need(cu_seqlens_q, "cu_seqlens_q", (torch.int32,), 1, device=dev)
    B = cu_seqlens_q.shape[0] - 1
    kv_dtype, P = _check_cache(kv_cache, kv_scale, dev)
    _need(block_table, "block_table", (torch.int32,), 2, device=dev)
    _need(cache_seqlens, "cache_seqlens", (torch.int32,), 1, shape=(B,), device=dev)
    if block_table.shape[0] != B:
        raise ValueError("block_table / cache_seqlens batch mismatch")
    if out is None:
        out = torch.empty((T, H, D_V), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    _need(out, "out", (torch.float32,), 3, shape=(T, H, D_V), device=dev)
    _need(lse, "lse", (torch.float32,), 2, shape=(T, H), device=dev)
    md = ws = None
    units, wbytes = 0, 0
    if plan is not None:
        if (plan.batch, plan.q_len, plan.num_heads) != (B, max_q_len, H):
            raise ValueError("plan was built for another shape")
        md, ws, units, wbytes = _plan_buffers(plan, dev)
    _check(lib.mla_decode_fwd_varlen(_ptr(q), _ptr(cu_seqlens_q), T, int(max_q_len), _ptr(kv_cache),
                                     _ptr(kv_scale), kv_dtype, P, _ptr(block_table),
                                     block_table.shape[1], _ptr(cache_seqlens), B, H, float(softmax_scale),
                                     _ptr(out), _ptr(lse), _ptr(md), units, _ptr(ws), wbytes, _stream()),
           "mla_decode_fwd_varlen")
    return out, lse


def profile_enable(enable: bool = True):
    """Record a HIP event pair around every main decode-kernel launch."""
    _check(load_library().mla_profile_enable(1 if enable else 0), "mla_profile_enable")


def profile_read():
    """(total_ms, launches) of the recorded main-kernel launches; clears the record."""
    ms, n = ctypes.c_double(0.0), ctypes.c_int(0)
    _check(load_library().mla_profile_read(ctypes.byref(ms), ctypes.byref(n)), "mla_profile_read")
    return ms.value, n.value


PROFILE_ATTENTION, PROFILE_METADATA, PROFILE_COMBINE, PROFILE_QUANTIZE = 0, 1, 2, 3


def debug_page_violations(reset: bool = True) -> int:
    """Page ids outside the pool seen by the decode kernels since the last
    reset (libmla_decode_debug.so only; MLAError otherwise). Waits for the
    device."""
    lib = load_library()
    torch.cuda.synchronize()
    n = ctypes.c_uint64(0)
    _check(lib.mla_debug_page_violations(1 if reset else 0, ctypes.byref(n)), "mla_debug_page_violations")
    return int(n.value)


def profile_read_launches(kernel: int = PROFILE_ATTENTION, capacity: int = 4096):
    """Elapsed ms of each recorded launch of one kernel kind (attention,
    metadata or combine), in launch order; clears that kind's record."""
    lib = load_library()
    n = ctypes.c_int(0)
    buf = (ctypes.c_float * capacity)()
    _check(lib.mla_profile_read_launches(int(kernel), buf, capacity, ctypes.byref(n)), "mla_profile_read_launches")
    return [float(buf[i]) for i in range(min(n.value, capacity))]


def combine(part_out: torch.Tensor, part_lse: torch.Tensor, seq_part_offsets: torch.Tensor,
            out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """LSE-merge partials: part_out [N, R, 512], part_lse [N, R], offsets int32 [B+1]."""
    lib = load_library()
    _need(part_out, "part_out", (torch.float32,), 3)
    dev = part_out.device
    N, R = part_out.shape[0], part_out.shape[1]
    if part_out.shape[2] != D_V:
        raise ValueError(f"part_out must be [partials, rows, {D_V}]")
    _need(part_lse, "part_lse", (torch.float32,), 2, shape=(N, R), device=dev)
    _need(seq_part_offsets, "seq_part_offsets", (torch.int32,), 1, device=dev)
    B = seq_part_offsets.shape[0] - 1
    if B < 1:
        raise ValueError("seq_part_offsets must have batch + 1 >= 2 entries")
    if out is None:
        out = torch.empty((B, R, D_V), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, R), dtype=torch.float32, device=dev)
    _need(out, "out", (torch.float32,), 3, shape=(B, R, D_V), device=dev)
    _need(lse, "lse", (torch.float32,), 2, shape=(B, R), device=dev)
    _check(lib.mla_combine(_ptr(part_out), _ptr(part_lse), _ptr(seq_part_offsets), B, R, _ptr(out),
                           _ptr(lse), _stream()), "mla_combine")
    return out, lse


def append_kv(latent: torch.Tensor, block_table: torch.Tensor, cache_seqlens: torch.Tensor,
              kv_cache: torch.Tensor, kv_scale: Optional[torch.Tensor] = None):
    """Store each sequence's newest latent rows in their pages (in place).

    latent bf16 [B, new_tokens, 576]; cache_seqlens int32 [B] already count the
    new tokens (token i goes to position L_b - new_tokens + i); kv_cache
    [P, 64, 576] bf16, or uint8 / float8_e4m3fn codes with kv_scale fp32
    [P, 64] (per-token E4M3FN quantisation).
    """
    lib = load_library()
    _need(latent, "latent", (torch.bfloat16,), 3)
    dev = latent.device
    B, s, d = latent.shape
    if d != D_QK:
        raise ValueError(f"latent last dim must be {D_QK}")
    kv_dtype, P = _check_cache(kv_cache, kv_scale, dev)
    _need(block_table, "block_table", (torch.int32,), 2, device=dev)
    _need(cache_seqlens, "cache_seqlens", (torch.int32,), 1, shape=(B,), device=dev)
    if block_table.shape[0] != B:
        raise ValueError("block_table / cache_seqlens batch mismatch")
    _check(lib.mla_append_kv(_ptr(latent), B, s, _ptr(block_table), block_table.shape[1], _ptr(cache_seqlens),
                             _ptr(kv_cache), _ptr(kv_scale), kv_dtype, P, _stream()),
           "mla_append_kv")
    return kv_cache, kv_scale
