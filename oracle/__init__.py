"""ctypes wrapper around the plain fp64 CPU oracle (``oracle/oracle.cpp``).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. It never imports
the product package and the product never imports it.

Inputs are host numpy arrays holding the raw bytes that are also handed to the
GPU path: fp16/bf16 tensors as ``uint16`` bit patterns, fp32 as ``float32``.
The oracle decodes them itself and computes in double precision; outputs are
``float64`` numpy arrays.

Definitions followed (see the header of ``oracle.cpp`` for the full list):
merge of two / N states, "F2 hints: merge_state, base-2 LSE merge",
sections 3-5; LSE sanitising, "FlashAttention's empty-row LSE", section 2.2;
softmax attention, same page, section 0; split page ranges, empty splits and
the split-count rules, "L3 hints: split-KV decode and LSE merge", sections 2, 4
and 6; the attention sink, "FlashAttention's empty-row LSE", sections 0.1 and 1;
the masked in-place and variable-length merges, "F2 hints", section 7.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "oracle.cpp")

F16, BF16, F32 = 0, 1, 2
_DTYPE_CODES = {"f16": F16, "bf16": BF16, "f32": F32}


def build(force: bool = True) -> str:
    """Compile ``liboracle.so`` with g++ (host only, no GPU code)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread",
               "-fno-fast-math", SRC_PATH, "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(LIB_PATH)
        P, I, I64, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.or_decode_f16.argtypes = [P, P, I64]
        lib.or_decode_bf16.argtypes = [P, P, I64]
        lib.or_merge_state.argtypes = [P, P, P, P, I, I64, I, P, P, I]
        lib.or_merge_states.argtypes = [P, P, I, I64, I, I, I, P, P, I]
        lib.or_split_range.argtypes = [I, I, I, I, P, P]
        lib.or_plan_splits.argtypes = [I, I, P, I, I]
        lib.or_attention.argtypes = [P, I, P, P, I, P, I, P, I, I, I, I, I, D, P, P, I]
        lib.or_split_partials.argtypes = [P, I, P, P, I, P, I, P, I, I, I, I, I, D, I, P, P, I]
        lib.or_merge_sink.argtypes = [P, P, I, I64, I, I, P, P, P, I]
        lib.or_merge_state_masked.argtypes = [P, P, P, P, I, I64, I, I, P, P, P, I]
        lib.or_merge_states_varlen.argtypes = [P, P, I, P, I64, I, I, P, P, I]
        lib.or_plan_splits_varlen.argtypes = [I, I, P, I, I, P]
        lib.or_split_partials_varlen.argtypes = [P, I, P, P, I, P, I, P, I, I, I, I, I, D, P, P,
                                                 P, I]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _code(dtype: str) -> int:
    return _DTYPE_CODES[dtype]


def _check(rc: int, name: str):
    if rc != 0:
        raise ValueError(f"oracle {name} rejected its arguments (rc={rc})")


def decode_f16(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, np.float64)
    _load().or_decode_f16(_ptr(bits), _ptr(out), bits.size)
    return out


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, np.float64)
    _load().or_decode_bf16(_ptr(bits), _ptr(out), bits.size)
    return out


def merge_state(va, sa, vb, sb, dtype: str, threads: int = 0):
    """Two states v[S,H,D] (or [rows, D]), s[S,H] -> (v fp64, s fp64)."""
    va, vb = np.ascontiguousarray(va), np.ascontiguousarray(vb)
    sa = np.ascontiguousarray(sa, dtype=np.float32)
    sb = np.ascontiguousarray(sb, dtype=np.float32)
    D = va.shape[-1]
    rows = sa.size
    assert va.size == rows * D and vb.size == rows * D and sb.size == rows
    v_out = np.empty(va.shape, np.float64)
    s_out = np.empty(sa.shape, np.float64)
    rc = _load().or_merge_state(_ptr(va), _ptr(sa), _ptr(vb), _ptr(sb), _code(dtype), rows, D,
                                _ptr(v_out), _ptr(s_out), threads)
    _check(rc, "merge_state")
    return v_out, s_out


def merge_states(v, s, dtype: str, threads: int = 0):
    """N states v[S,N,H,D], s[S,N,H] -> (v[S,H,D] fp64, s[S,H] fp64)."""
    v = np.ascontiguousarray(v)
    s = np.ascontiguousarray(s, dtype=np.float32)
    S, N, H, D = v.shape
    assert s.shape == (S, N, H)
    v_out = np.empty((S, H, D), np.float64)
    s_out = np.empty((S, H), np.float64)
    rc = _load().or_merge_states(_ptr(v), _ptr(s), _code(dtype), S, N, H, D, _ptr(v_out),
                                 _ptr(s_out), threads)
    _check(rc, "merge_states")
    return v_out, s_out


def split_range(ctx: int, page: int, splits: int, k: int):
    p0, p1 = ctypes.c_int(), ctypes.c_int()
    rc = _load().or_split_range(ctx, page, splits, k, ctypes.byref(p0), ctypes.byref(p1))
    _check(rc, "split_range")
    return p0.value, p1.value


def plan_splits(B: int, Hkv: int, ctx_lens, page: int, num_cus: int) -> int:
    ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    r = _load().or_plan_splits(B, Hkv, _ptr(ctx), page, num_cus)
    if r < 0:
        raise ValueError("oracle plan_splits rejected its arguments")
    return r


def _decode_common(q, k_cache, v_cache, page_table, ctx_lens, q_dtype, kv_dtype):
    q = np.ascontiguousarray(q)
    k_cache = np.ascontiguousarray(k_cache)
    v_cache = np.ascontiguousarray(v_cache)
    page_table = np.ascontiguousarray(page_table, dtype=np.int32)
    ctx_lens = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    B, Hq, D = q.shape
    _, Hkv, page, Dk = k_cache.shape
    assert Dk == D and v_cache.shape == k_cache.shape
    assert page_table.ndim == 2 and page_table.shape[0] == B and ctx_lens.shape == (B,)
    return q, k_cache, v_cache, page_table, ctx_lens, B, Hq, Hkv, D, page


def attention(q, k_cache, v_cache, page_table, ctx_lens, sm_scale: float, q_dtype: str,
              kv_dtype: str, threads: int = 0):
    """Unsplit decode attention -> (o[B,Hq,D] fp64, s[B,Hq] fp64 base-2 LSE).

    q [B,Hq,D]; k_cache, v_cache [pages, Hkv, PAGE, D]; page_table [B, stride]
    int32 (logical page -> physical page); ctx_lens [B] int32.
    """
    q, k_cache, v_cache, pt, ctx, B, Hq, Hkv, D, page = _decode_common(
        q, k_cache, v_cache, page_table, ctx_lens, q_dtype, kv_dtype)
    o = np.empty((B, Hq, D), np.float64)
    s = np.empty((B, Hq), np.float64)
    rc = _load().or_attention(_ptr(q), _code(q_dtype), _ptr(k_cache), _ptr(v_cache),
                              _code(kv_dtype), _ptr(pt), pt.shape[1], _ptr(ctx), B, Hq, Hkv, D,
                              page, float(sm_scale), _ptr(o), _ptr(s), threads)
    _check(rc, "attention")
    return o, s


def split_partials(q, k_cache, v_cache, page_table, ctx_lens, sm_scale: float, splits: int,
                   q_dtype: str, kv_dtype: str, threads: int = 0):
    """Per-split partial states -> (o_part[B,Hq,splits,D], lse_part[B,Hq,splits]) fp64."""
    q, k_cache, v_cache, pt, ctx, B, Hq, Hkv, D, page = _decode_common(
        q, k_cache, v_cache, page_table, ctx_lens, q_dtype, kv_dtype)
    o = np.empty((B, Hq, splits, D), np.float64)
    s = np.empty((B, Hq, splits), np.float64)
    rc = _load().or_split_partials(_ptr(q), _code(q_dtype), _ptr(k_cache), _ptr(v_cache),
                                   _code(kv_dtype), _ptr(pt), pt.shape[1], _ptr(ctx), B, Hq, Hkv,
                                   D, page, float(sm_scale), splits, _ptr(o), _ptr(s), threads)
    _check(rc, "split_partials")
    return o, s


def merge_sink(v, s, sink, dtype: str, threads: int = 0):
    """State v[S,H,D], s[S,H] merged with the sink of each head (logit sink[H],
    natural units, value 0) -> (v fp64, s fp64)."""
    v = np.ascontiguousarray(v)
    s = np.ascontiguousarray(s, dtype=np.float32)
    sink = np.ascontiguousarray(sink, dtype=np.float32)
    H, D = s.shape[-1], v.shape[-1]
    assert sink.shape == (H,) and v.size == s.size * D
    v_out = np.empty(v.shape, np.float64)
    s_out = np.empty(s.shape, np.float64)
    rc = _load().or_merge_sink(_ptr(v), _ptr(s), _code(dtype), s.size, H, D, _ptr(sink),
                               _ptr(v_out), _ptr(s_out), threads)
    _check(rc, "merge_sink")
    return v_out, s_out


def merge_state_masked(va, sa, vb, sb, mask, dtype: str, threads: int = 0):
    """Two states v[S,H,D], s[S,H]; positions with mask[S] == 0 keep state a."""
    va, vb = np.ascontiguousarray(va), np.ascontiguousarray(vb)
    sa = np.ascontiguousarray(sa, dtype=np.float32)
    sb = np.ascontiguousarray(sb, dtype=np.float32)
    S, H, D = va.shape
    m = None if mask is None else np.ascontiguousarray(mask, dtype=np.uint8)
    assert m is None or m.shape == (S,)
    v_out = np.empty(va.shape, np.float64)
    s_out = np.empty(sa.shape, np.float64)
    rc = _load().or_merge_state_masked(_ptr(va), _ptr(sa), _ptr(vb), _ptr(sb), _code(dtype), S,
                                       H, D, None if m is None else _ptr(m), _ptr(v_out),
                                       _ptr(s_out), threads)
    _check(rc, "merge_state_masked")
    return v_out, s_out


def merge_states_varlen(v, s, indptr, dtype: str, threads: int = 0):
    """States v[total,H,D], s[total,H]; segment i = states indptr[i]..indptr[i+1]-1
    -> (v[S,H,D] fp64, s[S,H] fp64) with S = len(indptr) - 1."""
    v = np.ascontiguousarray(v)
    s = np.ascontiguousarray(s, dtype=np.float32)
    indptr = np.ascontiguousarray(indptr, dtype=np.int32)
    S = indptr.size - 1
    _, H, D = v.shape
    v_out = np.empty((S, H, D), np.float64)
    s_out = np.empty((S, H), np.float64)
    rc = _load().or_merge_states_varlen(_ptr(v), _ptr(s), _code(dtype), _ptr(indptr), S, H, D,
                                        _ptr(v_out), _ptr(s_out), threads)
    _check(rc, "merge_states_varlen")
    return v_out, s_out


def plan_splits_varlen(B: int, Hkv: int, ctx_lens, page: int, num_cus: int):
    """-> (pages per split c, split counts [B] int32)."""
    ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    counts = np.empty(B, np.int32)
    c = _load().or_plan_splits_varlen(B, Hkv, _ptr(ctx), page, num_cus, _ptr(counts))
    if c < 0:
        raise ValueError("oracle plan_splits_varlen rejected its arguments")
    return c, counts


def split_partials_varlen(q, k_cache, v_cache, page_table, ctx_lens, sm_scale: float, indptr,
                          q_dtype: str, kv_dtype: str, threads: int = 0):
    """Partials with per-sequence splits (sequence b has indptr[b+1] - indptr[b] >= 1 splits,
    each with the page-range formula) -> (o_part[total,Hq,D], lse_part[total,Hq]) fp64."""
    q, k_cache, v_cache, pt, ctx, B, Hq, Hkv, D, page = _decode_common(
        q, k_cache, v_cache, page_table, ctx_lens, q_dtype, kv_dtype)
    indptr = np.ascontiguousarray(indptr, dtype=np.int32)
    assert indptr.shape == (B + 1,)
    total = int(indptr[-1])
    o = np.empty((total, Hq, D), np.float64)
    s = np.empty((total, Hq), np.float64)
    rc = _load().or_split_partials_varlen(_ptr(q), _code(q_dtype), _ptr(k_cache),
                                          _ptr(v_cache), _code(kv_dtype), _ptr(pt), pt.shape[1],
                                          _ptr(ctx), B, Hq, Hkv, D, page, float(sm_scale),
                                          _ptr(indptr), _ptr(o), _ptr(s), threads)
    _check(rc, "split_partials_varlen")
    return o, s
