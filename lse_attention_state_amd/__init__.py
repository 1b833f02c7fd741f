"""Python binding for libmi.so: attention-state merging and split-KV decode on MI355X.

The functions below only marshal arguments: they check tensor dtypes, shapes,
devices and contiguity, allocate missing outputs with torch (device memory is
plumbing), and call the C ABI declared in ``include/mi.h`` on the current
torch stream. Every step of the computation runs in the HIP kernels of
libmi.so. There is no CPU fallback: if the library is missing or fails to
load, every call raises.

Conventions (see ``include/mi.h``): an attention state is (v, s) with s the
base-2 log-sum-exp, empty = (0, -inf); s / lse tensors are float32.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmi.so")

MI_F16, MI_BF16, MI_F32 = 0, 1, 2
_DT = {torch.float16: MI_F16, torch.bfloat16: MI_BF16, torch.float32: MI_F32}

STATUS = {0: "MI_OK", 1: "MI_ERR_NULL", 2: "MI_ERR_SHAPE", 3: "MI_ERR_DTYPE",
          4: "MI_ERR_UNSUPPORTED", 5: "MI_ERR_HIP", 6: "MI_ERR_ALIAS", 7: "MI_ERR_SCRATCH"}

# Largest B * Hq * num_splits that split_kv_decode_noalloc accepts (include/mi.h).
NOALLOC_MAX_PARTIAL_ROWS = 32768

# (name, argtypes) of every exported entry point; the list mirrors include/mi.h.
_P, _I32, _I64, _F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
SIGNATURES = {
    "mi_status_string": [ctypes.c_int],
    "mi_merge_state": [_P, _P, _P, _P, _P, _P, _I64, _I32, _I32, ctypes.c_int, ctypes.c_int, _P],
    "mi_merge_states": [_P, _P, _P, _P, _I64, _I32, _I32, _I32, ctypes.c_int, ctypes.c_int, _P],
    "mi_plan_splits": [_I32, _I32, _P, _I32, _I32, _P],
    "mi_split_range": [_I32, _I32, _I32, _I32, _P, _P],
    "mi_split_kv_partial": [_P, _P, _P, _P, _I32, _P, _I32, _I32, _I32, _I32, _I32, _I64, _I32,
                            _F, ctypes.c_int, _P, _P, _P],
    "mi_split_kv_decode": [_P, _P, _P, _P, _I32, _P, _I32, _I32, _I32, _I32, _I32, _I64, _I32, _F,
                           ctypes.c_int, _P, _P, _P, _P, ctypes.c_int, _P],
    "mi_split_kv_decode_fused": [_P, _P, _P, _P, _I32, _P, _I32, _I32, _I32, _I32, _I32, _I64,
                                 _I32, _F, ctypes.c_int, _P, _P, _P, _P, _P, ctypes.c_int, _P],
    "mi_prefix_attention": [_P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _I64, _F,
                            ctypes.c_int, _P, ctypes.c_size_t, _P, _P, ctypes.c_int, _P],
    "mi_prefix_attention_workspace": [_I32, _I32, _I32, _I32, _I32, _P],
    "mi_cascade_decode": [_P, _P, _P, _P, _I32, _P, _I32, _P, _I32, _I32, _I32, _I32, _I32, _I64,
                          _I32, _F, ctypes.c_int, _P, ctypes.c_size_t, _P, _P, _P, _P, _P,
                          ctypes.c_int, _P],
    "mi_merge_state_in_place": [_P, _P, _P, _P, _P, _I64, _I32, _I32, ctypes.c_int, _P],
    "mi_merge_states_two_level": [_P, _P, _P, _P, _I64, _I32, _I32, _I32, ctypes.c_int,
                                  ctypes.c_int, _P, ctypes.c_size_t, _P],
    "mi_merge_states_workspace": [_I64, _I32, _I32, _I32, _P],
    "mi_merge_sink": [_P, _P, _P, _P, _P, _I64, _I32, _I32, ctypes.c_int, ctypes.c_int, _P],
    "mi_merge_states_varlen": [_P, _P, _P, _I64, _P, _P, _I64, _I32, _I32, ctypes.c_int,
                               ctypes.c_int, _P],
    "mi_plan_splits_varlen": [_I32, _I32, _P, _I32, _I32, _P],
    "mi_split_kv_decode_varlen": [_P, _P, _P, _P, _I32, _P, _I32, _I32, _I32, _I32, _I32, _I64,
                                  _P, _I32, _F, ctypes.c_int, _P, _P, _P, _P, _P, ctypes.c_int,
                                  _P],
    "mi_stream_read": [_P, _I64, _P, _P],
    "mi_split_kv_decode_noalloc": [_P, _P, _P, _P, _I32, _P, _I32, _I32, _I32, _I32, _I32, _I64,
                                   _I32, _F, ctypes.c_int, _P, _P, ctypes.c_int, _P],
}


class MiError(RuntimeError):
    def __init__(self, name: str, status: int):
        super().__init__(f"{name} failed: {STATUS.get(status, status)}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libmi.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m lse_attention_state_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, argtypes in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = argtypes
            fn.restype = ctypes.c_char_p if name == "mi_status_string" else ctypes.c_int
        _lib = handle
    return _lib


def _call(name: str, *args):
    rc = getattr(lib(), name)(*args)
    if rc != 0:
        raise MiError(name, rc)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _check_cuda(*ts):
    """Every given tensor is a contiguous GPU tensor on the first one's device."""
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("tensors must all be on one GPU")


def _expect(t, name, shape=None, dtype=None, numel_at_least=None):
    """Shape / dtype / size checks of an optional tensor (None passes)."""
    if t is None:
        return
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel_at_least is not None and t.numel() < numel_at_least:
        raise ValueError(f"{name} must have at least {numel_at_least} elements, got {t.numel()}")


def _out_dtype_ok(t, name):
    if t is not None and t.dtype not in _DT:
        raise TypeError(f"{name}: unsupported dtype {t.dtype}")


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def _f32(t, name):
    if t is not None and t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32")


# ----------------------------------------------------------------------------- merges

def merge_state(v_a, s_a, v_b, s_b, out_dtype=None, v_out=None, s_out=None, return_s=True):
    """Merge two states: v_* [..., D], s_* [...] (float32, base 2). Returns (v, s).

    ``v_out`` may be ``v_a`` or ``v_b`` (in place) when dtypes match; ``s_out``
    may be ``s_a`` or ``s_b``."""
    _f32(s_a, "s_a"), _f32(s_b, "s_b"), _f32(s_out, "s_out")
    _dt(v_a)
    if v_b.dtype != v_a.dtype:
        raise TypeError("merge_state: v_a and v_b must share one dtype")
    if v_a.shape != v_b.shape or s_a.shape != s_b.shape or v_a.shape[:-1] != s_a.shape:
        raise ValueError("merge_state: shapes must be v [..., D] and s [...] for both states")
    _out_dtype_ok(v_out, "v_out")
    _expect(v_out, "v_out", v_a.shape)
    _expect(s_out, "s_out", s_a.shape)
    out_dtype = out_dtype or (v_out.dtype if v_out is not None else v_a.dtype)
    if v_out is not None and v_out.dtype != out_dtype:
        raise TypeError("merge_state: v_out's dtype differs from out_dtype")
    _check_cuda(v_a, s_a, v_b, s_b, v_out, s_out)
    if v_out is None:
        v_out = torch.empty(v_a.shape, dtype=out_dtype, device=v_a.device)
    if s_out is None and return_s:
        s_out = torch.empty(s_a.shape, dtype=torch.float32, device=v_a.device)
    D = v_a.shape[-1]
    rows = s_a.numel()
    _call("mi_merge_state", _ptr(v_a), _ptr(s_a), _ptr(v_b), _ptr(s_b), _ptr(v_out), _ptr(s_out),
          rows, 1, D, _dt(v_a), _dt(v_out), _stream(v_a))
    return v_out, s_out


def merge_states(v, s, out_dtype=None, v_out=None, s_out=None, return_s=True):
    """Merge N states: v [S, N, H, D], s [S, N, H] -> (v [S, H, D], s [S, H])."""
    _f32(s, "s"), _f32(s_out, "s_out")
    _dt(v)
    if v.dim() != 4 or s.shape != v.shape[:3]:
        raise ValueError("merge_states: v must be [S, N, H, D] and s [S, N, H]")
    S, N, H, D = v.shape
    _out_dtype_ok(v_out, "v_out")
    _expect(v_out, "v_out", (S, H, D))
    _expect(s_out, "s_out", (S, H))
    out_dtype = out_dtype or (v_out.dtype if v_out is not None else v.dtype)
    if v_out is not None and v_out.dtype != out_dtype:
        raise TypeError("merge_states: v_out's dtype differs from out_dtype")
    _check_cuda(v, s, v_out, s_out)
    if v_out is None:
        v_out = torch.empty((S, H, D), dtype=out_dtype, device=v.device)
    if s_out is None and return_s:
        s_out = torch.empty((S, H), dtype=torch.float32, device=v.device)
    _call("mi_merge_states", _ptr(v), _ptr(s), _ptr(v_out), _ptr(s_out), S, N, H, D, _dt(v),
          _dt(v_out), _stream(v))
    return v_out, s_out


def merge_states_workspace_bytes(S: int, N: int, H: int, D: int) -> int:
    out = ctypes.c_size_t()
    _call("mi_merge_states_workspace", S, N, H, D, ctypes.byref(out))
    return out.value


def merge_states_two_level(v, s, out_dtype=None, v_out=None, s_out=None, workspace=None,
                           return_s=True):
    """N-state merge over two levels (few positions, many states):
    v [S, N, H, D], s [S, N, H] -> (v [S, H, D], s [S, H])."""
    _f32(s, "s"), _f32(s_out, "s_out"), _f32(workspace, "workspace")
    _dt(v)
    if v.dim() != 4 or s.shape != v.shape[:3]:
        raise ValueError("merge_states_two_level: v must be [S, N, H, D] and s [S, N, H]")
    S, N, H, D = v.shape
    _out_dtype_ok(v_out, "v_out")
    _expect(v_out, "v_out", (S, H, D))
    _expect(s_out, "s_out", (S, H))
    need = merge_states_workspace_bytes(S, N, H, D)
    if workspace is not None and workspace.numel() * 4 < need:
        raise ValueError(f"merge_states_two_level: workspace holds {workspace.numel() * 4} bytes, "
                         f"{need} needed")
    out_dtype = out_dtype or (v_out.dtype if v_out is not None else v.dtype)
    if v_out is not None and v_out.dtype != out_dtype:
        raise TypeError("merge_states_two_level: v_out's dtype differs from out_dtype")
    _check_cuda(v, s, v_out, s_out, workspace)
    if v_out is None:
        v_out = torch.empty((S, H, D), dtype=out_dtype, device=v.device)
    if s_out is None and return_s:
        s_out = torch.empty((S, H), dtype=torch.float32, device=v.device)
    if workspace is None and need > 0:
        workspace = torch.empty(need // 4, dtype=torch.float32, device=v.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * 4
    _call("mi_merge_states_two_level", _ptr(v), _ptr(s), _ptr(v_out), _ptr(s_out), S, N, H, D,
          _dt(v), _dt(v_out), _ptr(workspace), ws_bytes, _stream(v))
    return v_out, s_out


def merge_state_in_place(v, s, v_other, s_other, mask=None):
    """v, s <- merge((v, s), (v_other, s_other)) where mask [S] (bool / uint8) is set;
    positions with a zero mask byte are left untouched. v [S, H, D] or [S, D]."""
    _f32(s, "s"), _f32(s_other, "s_other")
    _dt(v)
    if v.shape != v_other.shape or s.shape != s_other.shape or v.shape[:-1] != s.shape:
        raise ValueError("merge_state_in_place: v [S, (H,) D] and s [S, (H)] for both states")
    if v.dtype != v_other.dtype:
        raise TypeError("merge_state_in_place: v and v_other must share one dtype")
    S = s.shape[0] if s.dim() > 0 else 1
    H = s.numel() // S if S > 0 else 1
    D = v.shape[-1]
    if mask is not None:
        if mask.dtype == torch.bool:
            mask = mask.view(torch.uint8)
        if mask.dtype != torch.uint8 or mask.shape != (S,):
            raise ValueError("mask must be bool or uint8 of shape [S]")
    _check_cuda(v, s, v_other, s_other, mask)
    _call("mi_merge_state_in_place", _ptr(v), _ptr(s), _ptr(v_other), _ptr(s_other), _ptr(mask),
          S, max(H, 1), D, _dt(v), _stream(v))
    return v, s


def merge_sink(v, s, sink, out_dtype=None, v_out=None, s_out=None, return_s=True):
    """Fold an attention sink (natural-log logit per head, sink [H] float32) into
    states v [S, H, D], s [S, H] -> (v, s). v_out / s_out may be v / s."""
    _f32(s, "s"), _f32(sink, "sink"), _f32(s_out, "s_out")
    _dt(v)
    if v.dim() != 3 or s.shape != v.shape[:2] or sink.shape != (v.shape[1],):
        raise ValueError("merge_sink: v [S, H, D], s [S, H], sink [H]")
    S, H, D = v.shape
    _out_dtype_ok(v_out, "v_out")
    _expect(v_out, "v_out", v.shape)
    _expect(s_out, "s_out", s.shape)
    out_dtype = out_dtype or (v_out.dtype if v_out is not None else v.dtype)
    if v_out is not None and v_out.dtype != out_dtype:
        raise TypeError("merge_sink: v_out's dtype differs from out_dtype")
    _check_cuda(v, s, sink, v_out, s_out)
    if v_out is None:
        v_out = torch.empty(v.shape, dtype=out_dtype, device=v.device)
    if s_out is None and return_s:
        s_out = torch.empty(s.shape, dtype=torch.float32, device=v.device)
    _call("mi_merge_sink", _ptr(v), _ptr(s), _ptr(sink), _ptr(v_out), _ptr(s_out), S, H, D,
          _dt(v), _dt(v_out), _stream(v))
    return v_out, s_out


def merge_states_varlen(v, s, indptr, out_dtype=None, v_out=None, s_out=None, return_s=True):
    """Merge variable-length index sets: v [total, H, D], s [total, H], indptr [S+1]
    int32 (device) -> (v [S, H, D], s [S, H])."""
    _f32(s, "s"), _f32(s_out, "s_out")
    _dt(v)
    if indptr.dtype != torch.int32:
        raise TypeError("merge_states_varlen: indptr must be int32")
    if v.dim() != 3 or s.shape != v.shape[:2] or indptr.dim() != 1 or indptr.shape[0] < 1:
        raise ValueError("merge_states_varlen: v [total, H, D], s [total, H], indptr int32 [S+1]")
    total, H, D = v.shape
    S = indptr.shape[0] - 1
    _out_dtype_ok(v_out, "v_out")
    _expect(v_out, "v_out", (S, H, D))
    _expect(s_out, "s_out", (S, H))
    out_dtype = out_dtype or (v_out.dtype if v_out is not None else v.dtype)
    if v_out is not None and v_out.dtype != out_dtype:
        raise TypeError("merge_states_varlen: v_out's dtype differs from out_dtype")
    _check_cuda(v, s, indptr, v_out, s_out)
    if v_out is None:
        v_out = torch.empty((S, H, D), dtype=out_dtype, device=v.device)
    if s_out is None and return_s:
        s_out = torch.empty((S, H), dtype=torch.float32, device=v.device)
    _call("mi_merge_states_varlen", _ptr(v), _ptr(s), _ptr(indptr), total, _ptr(v_out),
          _ptr(s_out), S, H, D, _dt(v), _dt(v_out), _stream(v))
    return v_out, s_out


# ----------------------------------------------------------------------------- planning

def plan_splits(ctx_lens, Hkv: int, page_size: int = 16, num_cus: int = 0) -> int:
    """Split count for a decode step; ``ctx_lens`` is host data (list / numpy / CPU tensor)."""
    import numpy as np
    ctx = np.ascontiguousarray(np.asarray(ctx_lens.cpu() if isinstance(ctx_lens, torch.Tensor)
                                          else ctx_lens, dtype=np.int32))
    out = ctypes.c_int32()
    _call("mi_plan_splits", len(ctx), Hkv, ctx.ctypes.data_as(ctypes.c_void_p), page_size,
          num_cus, ctypes.byref(out))
    return out.value


def plan_splits_varlen(ctx_lens, Hkv: int, page_size: int = 16, num_cus: int = 0):
    """Per-sequence split counts -> split_indptr (numpy int32 [B+1], host)."""
    import numpy as np
    ctx = np.ascontiguousarray(np.asarray(ctx_lens.cpu() if isinstance(ctx_lens, torch.Tensor)
                                          else ctx_lens, dtype=np.int32))
    out = np.empty(len(ctx) + 1, np.int32)
    _call("mi_plan_splits_varlen", len(ctx), Hkv, ctx.ctypes.data_as(ctypes.c_void_p), page_size,
          num_cus, out.ctypes.data_as(ctypes.c_void_p))
    return out


def split_range(ctx: int, page_size: int, num_splits: int, split: int):
    a, b = ctypes.c_int32(), ctypes.c_int32()
    _call("mi_split_range", ctx, page_size, num_splits, split, ctypes.byref(a), ctypes.byref(b))
    return a.value, b.value


# ----------------------------------------------------------------------------- decode

def _decode_args(q, k_cache, v_cache, page_table, ctx_lens):
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q must be [B, Hq, D] and k/v caches [pages, Hkv, PAGE, D]")
    if q.dtype != k_cache.dtype or k_cache.dtype != v_cache.dtype:
        raise TypeError("q, k_cache and v_cache must share one dtype")
    if page_table.dtype != torch.int32 or ctx_lens.dtype != torch.int32:
        raise TypeError("page_table and ctx_lens must be int32")
    B, Hq, D = q.shape
    P, Hkv, page, Dk = k_cache.shape
    if Dk != D or page_table.dim() != 2 or page_table.shape[0] != B or ctx_lens.shape != (B,):
        raise ValueError("inconsistent decode shapes")
    return B, Hq, Hkv, D, page, P


def _decode_outputs(B, Hq, Hkv, D, parts, o_part, lse_part, out=None, lse=None, counters=None):
    """Checks of caller-given decode outputs and workspaces: parts is the shape
    prefix of the partials ((B, Hq, splits) or (total, Hq))."""
    _expect(o_part, "o_part", (*parts, D), torch.float32)
    _expect(lse_part, "lse_part", parts, torch.float32)
    _out_dtype_ok(out, "out")
    _expect(out, "out", (B, Hq, D))
    _expect(lse, "lse", (B, Hq), torch.float32)
    _expect(counters, "counters", None, torch.int32, B * Hkv)


def split_kv_partial(q, k_cache, v_cache, page_table, ctx_lens, num_splits: int, sm_scale: float,
                     o_part=None, lse_part=None):
    """Pass 1 only -> (o_part [B, Hq, splits, D] f32, lse_part [B, Hq, splits] f32)."""
    B, Hq, Hkv, D, page, P = _decode_args(q, k_cache, v_cache, page_table, ctx_lens)
    _decode_outputs(B, Hq, Hkv, D, (B, Hq, num_splits), o_part, lse_part)
    _check_cuda(q, k_cache, v_cache, page_table, ctx_lens, o_part, lse_part)
    if o_part is None:
        o_part = torch.empty((B, Hq, num_splits, D), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((B, Hq, num_splits), dtype=torch.float32, device=q.device)
    _call("mi_split_kv_partial", _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
          page_table.shape[1], _ptr(ctx_lens), B, Hq, Hkv, D, page, P, num_splits,
          float(sm_scale), _dt(q), _ptr(o_part), _ptr(lse_part), _stream(q))
    return o_part, lse_part


def split_kv_decode(q, k_cache, v_cache, page_table, ctx_lens, num_splits: int, sm_scale: float,
                    out_dtype=None, o_part=None, lse_part=None, out=None, lse=None,
                    return_lse=True, return_partials=False):
    """Both passes -> (o [B, Hq, D], lse [B, Hq] f32 base 2[, o_part, lse_part])."""
    B, Hq, Hkv, D, page, P = _decode_args(q, k_cache, v_cache, page_table, ctx_lens)
    _decode_outputs(B, Hq, Hkv, D, (B, Hq, num_splits), o_part, lse_part, out, lse)
    _check_cuda(q, k_cache, v_cache, page_table, ctx_lens, o_part, lse_part, out, lse)
    out_dtype = out_dtype or (out.dtype if out is not None else q.dtype)
    if o_part is None:
        o_part = torch.empty((B, Hq, num_splits, D), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((B, Hq, num_splits), dtype=torch.float32, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _call("mi_split_kv_decode", _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
          page_table.shape[1], _ptr(ctx_lens), B, Hq, Hkv, D, page, P, num_splits,
          float(sm_scale), _dt(q), _ptr(o_part), _ptr(lse_part), _ptr(out), _ptr(lse),
          _dt(out), _stream(q))
    if return_partials:
        return out, lse, o_part, lse_part
    return out, lse


def split_kv_decode_fused(q, k_cache, v_cache, page_table, ctx_lens, num_splits: int,
                          sm_scale: float, counters=None, out_dtype=None, o_part=None,
                          lse_part=None, out=None, lse=None, return_lse=True,
                          return_partials=False):
    """Single-launch decode -> (o [B, Hq, D], lse [B, Hq][, o_part, lse_part]).

    ``counters`` is an int32 [B, Hkv] device workspace that must be zero before
    the first call; each call leaves it zero. It is allocated (zeroed) when not
    given."""
    B, Hq, Hkv, D, page, P = _decode_args(q, k_cache, v_cache, page_table, ctx_lens)
    _decode_outputs(B, Hq, Hkv, D, (B, Hq, num_splits), o_part, lse_part, out, lse, counters)
    _check_cuda(q, k_cache, v_cache, page_table, ctx_lens, o_part, lse_part, out, lse, counters)
    out_dtype = out_dtype or (out.dtype if out is not None else q.dtype)
    if counters is None:
        counters = torch.zeros((B, Hkv), dtype=torch.int32, device=q.device)
    if o_part is None:
        o_part = torch.empty((B, Hq, num_splits, D), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((B, Hq, num_splits), dtype=torch.float32, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _call("mi_split_kv_decode_fused", _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
          page_table.shape[1], _ptr(ctx_lens), B, Hq, Hkv, D, page, P, num_splits,
          float(sm_scale), _dt(q), _ptr(o_part), _ptr(lse_part), _ptr(counters), _ptr(out),
          _ptr(lse), _dt(out), _stream(q))
    if return_partials:
        return out, lse, o_part, lse_part
    return out, lse


def split_kv_decode_varlen(q, k_cache, v_cache, page_table, ctx_lens, split_indptr,
                           sm_scale: float, fused: bool = True, counters=None, out_dtype=None,
                           o_part=None, lse_part=None, out=None, lse=None, return_lse=True,
                           return_partials=False):
    """Decode with per-sequence split counts. ``split_indptr`` is int32 [B+1] on the
    device (from ``plan_splits_varlen``); its last entry (the total) is read from the
    host copy when given as numpy, else fetched once. -> (o, lse[, o_part [total, Hq, D],
    lse_part [total, Hq]])."""
    import numpy as np
    B, Hq, Hkv, D, page, P = _decode_args(q, k_cache, v_cache, page_table, ctx_lens)
    if isinstance(split_indptr, np.ndarray):
        if split_indptr.shape != (B + 1,):
            raise ValueError("split_indptr must be int32 [B + 1]")
        total = int(split_indptr[-1])
    else:
        if split_indptr.dtype != torch.int32 or split_indptr.shape != (B + 1,):
            raise ValueError("split_indptr must be int32 [B + 1]")
        total = None
    if not fused:
        counters = None
    if total is not None:
        _decode_outputs(B, Hq, Hkv, D, (total, Hq), o_part, lse_part, out, lse, counters)
    else:
        _decode_outputs(B, Hq, Hkv, D, (B, Hq), None, None, out, lse, counters)
    _check_cuda(q, k_cache, v_cache, page_table, ctx_lens, o_part, lse_part, out, lse, counters,
                None if total is not None else split_indptr)
    if total is None:
        total = int(split_indptr[-1].item())
        _decode_outputs(B, Hq, Hkv, D, (total, Hq), o_part, lse_part)
    else:
        split_indptr = torch.from_numpy(np.ascontiguousarray(split_indptr, np.int32)).to(q.device)
    out_dtype = out_dtype or (out.dtype if out is not None else q.dtype)
    if fused and counters is None:
        counters = torch.zeros((B, Hkv), dtype=torch.int32, device=q.device)
    if o_part is None:
        o_part = torch.empty((total, Hq, D), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((total, Hq), dtype=torch.float32, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _call("mi_split_kv_decode_varlen", _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
          page_table.shape[1], _ptr(ctx_lens), B, Hq, Hkv, D, page, P, _ptr(split_indptr), total,
          float(sm_scale), _dt(q), _ptr(o_part), _ptr(lse_part), _ptr(counters), _ptr(out),
          _ptr(lse), _dt(out), _stream(q))
    if return_partials:
        return out, lse, o_part, lse_part
    return out, lse


def split_kv_decode_noalloc(q, k_cache, v_cache, page_table, ctx_lens, num_splits: int,
                            sm_scale: float, out, lse=None):
    """Two-launch decode whose partials live in the library's static device
    scratch (the C entry point allocates nothing; ``out`` [B, Hq, D] and the
    optional ``lse`` [B, Hq] f32 are the caller's) -> (out, lse). Calls that
    overlap on one GPU race on the scratch."""
    B, Hq, Hkv, D, page, P = _decode_args(q, k_cache, v_cache, page_table, ctx_lens)
    if out is None:
        raise ValueError("split_kv_decode_noalloc: out must be given")
    _decode_outputs(B, Hq, Hkv, D, (B, Hq, num_splits), None, None, out, lse)
    if B * Hq * num_splits > NOALLOC_MAX_PARTIAL_ROWS:
        raise ValueError(f"split_kv_decode_noalloc: B * Hq * num_splits = {B * Hq * num_splits} "
                         f"exceeds {NOALLOC_MAX_PARTIAL_ROWS}")
    _check_cuda(q, k_cache, v_cache, page_table, ctx_lens, out, lse)
    _call("mi_split_kv_decode_noalloc", _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
          page_table.shape[1], _ptr(ctx_lens), B, Hq, Hkv, D, page, P, num_splits,
          float(sm_scale), _dt(q), _ptr(out), _ptr(lse), _dt(out), _stream(q))
    return out, lse


# ----------------------------------------------------------------------------- cascade

def prefix_attention_workspace_bytes(R: int, Hq: int, Hkv: int, D: int, prefix_len: int) -> int:
    out = ctypes.c_size_t()
    _call("mi_prefix_attention_workspace", R, Hq, Hkv, D, prefix_len, ctypes.byref(out))
    return out.value


def prefix_attention(q, k_cache, v_cache, prefix_pages, prefix_len: int, sm_scale: float,
                     out_dtype=torch.float32, workspace=None, v_out=None, s_out=None):
    """Cascade level 0: every (request, head) of q [R, Hq, D] against the shared
    prefix pages -> (v [R, Hq, D] out_dtype, s [R, Hq] f32 base 2)."""
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q must be [R, Hq, D] and k/v caches [pages, Hkv, PAGE, D]")
    if q.dtype != k_cache.dtype or k_cache.dtype != v_cache.dtype:
        raise TypeError("q, k_cache and v_cache must share one dtype")
    if prefix_pages.dtype != torch.int32:
        raise TypeError("prefix_pages must be int32")
    R, Hq, D = q.shape
    P, Hkv, page, _ = k_cache.shape
    if prefix_len < 0 or k_cache.shape[3] != D:
        raise ValueError("prefix_attention: prefix_len must be >= 0 and q's D the caches' D")
    _expect(prefix_pages, "prefix_pages", None, None, -(-prefix_len // page))
    need = prefix_attention_workspace_bytes(R, Hq, Hkv, D, prefix_len)
    _expect(workspace, "workspace", None, torch.float32, (need + 3) // 4)
    _out_dtype_ok(v_out, "v_out")
    _expect(v_out, "v_out", (R, Hq, D))
    _expect(s_out, "s_out", (R, Hq), torch.float32)
    _check_cuda(q, k_cache, v_cache, prefix_pages, v_out, s_out, workspace)
    if v_out is not None:
        out_dtype = v_out.dtype
    if workspace is None:
        workspace = torch.empty(max(need // 4, 1), dtype=torch.float32, device=q.device)
    if v_out is None:
        v_out = torch.empty((R, Hq, D), dtype=out_dtype, device=q.device)
    if s_out is None:
        s_out = torch.empty((R, Hq), dtype=torch.float32, device=q.device)
    _call("mi_prefix_attention", _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(prefix_pages),
          prefix_len, R, Hq, Hkv, D, page, P, float(sm_scale), _dt(q), _ptr(workspace),
          workspace.numel() * 4, _ptr(v_out), _ptr(s_out), _dt(v_out), _stream(q))
    return v_out, s_out


def cascade_decode(q, k_cache, v_cache, prefix_pages, prefix_len: int, suffix_table,
                   suffix_lens, sm_scale: float, suffix_splits: int = 1, out_dtype=None):
    """Two-level cascade decode: the shared prefix level (matrix cores), each
    request's own suffix (split-KV decode), then the merge of the two states.
    Returns (o [R, Hq, D], lse [R, Hq]) and the per-level states."""
    out_dtype = out_dtype or q.dtype
    vp, sp = prefix_attention(q, k_cache, v_cache, prefix_pages, prefix_len, sm_scale)
    vs, ss = split_kv_decode_fused(q, k_cache, v_cache, suffix_table, suffix_lens, suffix_splits,
                                   sm_scale, out_dtype=torch.float32)
    o, lse = merge_state(vp, sp, vs, ss, out_dtype=out_dtype)
    return o, lse, (vp, sp), (vs, ss)


def cascade_decode_fused(q, k_cache, v_cache, prefix_pages, prefix_len: int, suffix_table,
                         suffix_lens, sm_scale: float, suffix_splits: int = 1, out_dtype=None,
                         workspace=None, o_part=None, lse_part=None, counters=None, out=None,
                         lse=None, return_lse=True):
    """Two-level cascade decode in two launches (prefix level on the matrix cores,
    then the suffix decode whose combine also merges the prefix chunk states)
    -> (o [R, Hq, D], lse [R, Hq])."""
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q must be [R, Hq, D] and k/v caches [pages, Hkv, PAGE, D]")
    if q.dtype != k_cache.dtype or k_cache.dtype != v_cache.dtype:
        raise TypeError("q, k_cache and v_cache must share one dtype")
    if prefix_pages.dtype != torch.int32 or suffix_table.dtype != torch.int32 or \
            suffix_lens.dtype != torch.int32:
        raise TypeError("page lists, tables and lengths must be int32")
    R, Hq, D = q.shape
    P, Hkv, page, _ = k_cache.shape
    if prefix_len < 0 or k_cache.shape[3] != D:
        raise ValueError("cascade_decode_fused: prefix_len must be >= 0 and q's D the caches' D")
    if suffix_table.dim() != 2 or suffix_table.shape[0] != R or suffix_lens.shape != (R,):
        raise ValueError("cascade_decode_fused: suffix_table must be [R, stride] and "
                         "suffix_lens [R]")
    _expect(prefix_pages, "prefix_pages", None, None, -(-prefix_len // page))
    need = prefix_attention_workspace_bytes(R, Hq, Hkv, D, prefix_len)
    _expect(workspace, "workspace", None, torch.float32, (need + 3) // 4)
    _decode_outputs(R, Hq, Hkv, D, (R, Hq, suffix_splits), o_part, lse_part, out, lse, counters)
    _check_cuda(q, k_cache, v_cache, prefix_pages, suffix_table, suffix_lens, workspace, o_part,
                lse_part, counters, out, lse)
    out_dtype = out_dtype or (out.dtype if out is not None else q.dtype)
    if workspace is None:
        workspace = torch.empty(max(need // 4, 1), dtype=torch.float32, device=q.device)
    if o_part is None:
        o_part = torch.empty((R, Hq, suffix_splits, D), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((R, Hq, suffix_splits), dtype=torch.float32, device=q.device)
    if counters is None:
        counters = torch.zeros((R, Hkv), dtype=torch.int32, device=q.device)
    if out is None:
        out = torch.empty((R, Hq, D), dtype=out_dtype, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((R, Hq), dtype=torch.float32, device=q.device)
    _call("mi_cascade_decode", _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(prefix_pages),
          prefix_len, _ptr(suffix_table), suffix_table.shape[1], _ptr(suffix_lens), R, Hq, Hkv,
          D, page, P, suffix_splits, float(sm_scale), _dt(q), _ptr(workspace),
          workspace.numel() * 4, _ptr(o_part), _ptr(lse_part), _ptr(counters), _ptr(out),
          _ptr(lse), _dt(out), _stream(q))
    return out, lse


# ----------------------------------------------------------------------------- measurement

def stream_read(x, xor_out=None):
    """One plain streaming read of the contiguous device tensor x (its byte size
    a multiple of 16): the practical HBM read rate's probe. Returns the uint32
    XOR of all its 32-bit words as a one-element int32 device tensor, or XOR-s it
    into the given ``xor_out``."""
    _expect(xor_out, "xor_out", None, torch.int32, 1)
    _check_cuda(x, xor_out)
    if xor_out is None:
        xor_out = torch.zeros(1, dtype=torch.int32, device=x.device)
    _call("mi_stream_read", _ptr(x), x.numel() * x.element_size(), _ptr(xor_out), _stream(x))
    return xor_out
