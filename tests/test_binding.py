"""The Python binding rejects inconsistent arguments before anything reaches the C ABI.

Every case here fails on a dtype, shape or size check that the binding runs before it
looks at devices, so the tests run on the CPU with CPU tensors and no kernel is ever
launched. A call with consistent CPU tensors must fail only at the device check.
"""
import numpy as np
import pytest
import torch

import lse_attention_state_amd as mi

F16, BF16, F32 = torch.float16, torch.bfloat16, torch.float32


def _t(shape, dtype=F32):
    return torch.zeros(shape, dtype=dtype)


def _gpu_only(fn, *a, **k):
    with pytest.raises(ValueError, match="GPU"):
        fn(*a, **k)


def test_merge_state_checks():
    va, vb, sa, sb = _t((4, 2, 8), F16), _t((4, 2, 8), F16), _t((4, 2)), _t((4, 2))
    with pytest.raises(TypeError):
        mi.merge_state(va, sa, _t((4, 2, 8), BF16), sb)
    with pytest.raises(ValueError):
        mi.merge_state(va, sa, vb, sb, v_out=_t((4, 2, 16), F16))
    with pytest.raises(ValueError):
        mi.merge_state(va, sa, vb, sb, s_out=_t((4, 3)))
    with pytest.raises(TypeError):
        mi.merge_state(va, sa, vb, sb, s_out=_t((4, 2), torch.float64))
    with pytest.raises(TypeError):
        mi.merge_state(va, sa, vb, sb, v_out=_t((4, 2, 8), torch.float64))
    with pytest.raises(TypeError):
        mi.merge_state(va, sa, vb, sb, out_dtype=F32, v_out=_t((4, 2, 8), F16))
    _gpu_only(mi.merge_state, va, sa, vb, sb)


def test_merge_states_checks():
    v, s = _t((3, 4, 2, 8), F16), _t((3, 4, 2))
    with pytest.raises(ValueError):
        mi.merge_states(v, s, v_out=_t((3, 4, 8), F16))
    with pytest.raises(ValueError):
        mi.merge_states(v, s, s_out=_t((3, 4)))
    with pytest.raises(TypeError):
        mi.merge_states(_t((3, 4, 2, 8), torch.int32), s)
    _gpu_only(mi.merge_states, v, s)


def test_merge_states_two_level_checks():
    v, s = _t((2, 1024, 1, 8)), _t((2, 1024, 1))
    need = mi.merge_states_workspace_bytes(2, 1024, 1, 8)
    assert need > 0
    with pytest.raises(ValueError, match="workspace"):
        mi.merge_states_two_level(v, s, workspace=_t((need // 4 - 1,)))
    with pytest.raises(ValueError):
        mi.merge_states_two_level(v, s, v_out=_t((2, 2, 8)))
    _gpu_only(mi.merge_states_two_level, v, s, workspace=_t((need // 4,)))


def test_merge_sink_and_in_place_checks():
    v, s, sink = _t((4, 2, 8), BF16), _t((4, 2)), _t((2,))
    with pytest.raises(ValueError):
        mi.merge_sink(v, s, sink, v_out=_t((4, 2, 4), BF16))
    with pytest.raises(ValueError):
        mi.merge_sink(v, s, sink, s_out=_t((2, 4)))
    with pytest.raises(ValueError):
        mi.merge_sink(v, s, _t((3,)))
    with pytest.raises(TypeError):
        mi.merge_state_in_place(v, s, _t((4, 2, 8), F16), s)
    with pytest.raises(ValueError):
        mi.merge_state_in_place(v, s, v, s, mask=torch.zeros(5, dtype=torch.uint8))
    _gpu_only(mi.merge_sink, v, s, sink)
    _gpu_only(mi.merge_state_in_place, v, s, v.clone(), s.clone())


def test_merge_states_varlen_checks():
    v, s = _t((10, 2, 8), F16), _t((10, 2))
    indptr = torch.tensor([0, 4, 10], dtype=torch.int32)
    with pytest.raises(TypeError):
        mi.merge_states_varlen(v, s, indptr.long())
    with pytest.raises(ValueError):
        mi.merge_states_varlen(v, s, indptr, v_out=_t((3, 2, 8), F16))
    with pytest.raises(ValueError):
        mi.merge_states_varlen(v, s, indptr, s_out=_t((2, 3)))
    _gpu_only(mi.merge_states_varlen, v, s, indptr)


def _decode_case(B=2, Hq=8, Hkv=2, pages=6, dtype=F16):
    q = _t((B, Hq, 128), dtype)
    k = _t((pages, Hkv, 16, 128), dtype)
    v = _t((pages, Hkv, 16, 128), dtype)
    pt = torch.zeros((B, 3), dtype=torch.int32)
    ctx = torch.tensor([20, 33][:B], dtype=torch.int32)
    return q, k, v, pt, ctx


def test_decode_input_checks():
    q, k, v, pt, ctx = _decode_case()
    with pytest.raises(TypeError):
        mi.split_kv_partial(q, k.to(BF16), v, pt, ctx, 4, 0.1)
    with pytest.raises(TypeError):
        mi.split_kv_partial(q, k, v, pt.long(), ctx, 4, 0.1)
    with pytest.raises(ValueError):
        mi.split_kv_partial(q, k, v, pt[:1], ctx, 4, 0.1)
    with pytest.raises(ValueError):
        mi.split_kv_partial(q, k, v, pt, ctx[:1], 4, 0.1)


def test_decode_output_checks():
    q, k, v, pt, ctx = _decode_case()
    B, Hq, Hkv = 2, 8, 2
    with pytest.raises(ValueError):
        mi.split_kv_partial(q, k, v, pt, ctx, 4, 0.1, o_part=_t((B, Hq, 3, 128)))
    with pytest.raises(TypeError):
        mi.split_kv_partial(q, k, v, pt, ctx, 4, 0.1, o_part=_t((B, Hq, 4, 128), F16))
    with pytest.raises(ValueError):
        mi.split_kv_partial(q, k, v, pt, ctx, 4, 0.1, lse_part=_t((B, Hq, 5)))
    with pytest.raises(ValueError):
        mi.split_kv_decode(q, k, v, pt, ctx, 4, 0.1, out=_t((B, Hq, 64), F16))
    with pytest.raises(TypeError):
        mi.split_kv_decode(q, k, v, pt, ctx, 4, 0.1, lse=_t((B, Hq), F16))
    with pytest.raises(ValueError):
        mi.split_kv_decode_fused(q, k, v, pt, ctx, 4, 0.1,
                                 counters=torch.zeros(B * Hkv - 1, dtype=torch.int32))
    with pytest.raises(TypeError):
        mi.split_kv_decode_fused(q, k, v, pt, ctx, 4, 0.1,
                                 counters=torch.zeros(B * Hkv, dtype=torch.int64))
    _gpu_only(mi.split_kv_partial, q, k, v, pt, ctx, 4, 0.1)
    _gpu_only(mi.split_kv_decode, q, k, v, pt, ctx, 4, 0.1)
    _gpu_only(mi.split_kv_decode_fused, q, k, v, pt, ctx, 4, 0.1)


def test_decode_varlen_checks():
    q, k, v, pt, ctx = _decode_case()
    indptr = np.array([0, 2, 5], np.int32)
    with pytest.raises(ValueError):
        mi.split_kv_decode_varlen(q, k, v, pt, ctx, np.array([0, 2], np.int32), 0.1)
    with pytest.raises(ValueError):
        mi.split_kv_decode_varlen(q, k, v, pt, ctx, indptr, 0.1, o_part=_t((4, 8, 128)))
    with pytest.raises(ValueError):
        mi.split_kv_decode_varlen(q, k, v, pt, ctx, indptr, 0.1, lse_part=_t((5, 7)))
    with pytest.raises(ValueError):
        mi.split_kv_decode_varlen(q, k, v, pt, ctx, torch.tensor([0, 2], dtype=torch.int32), 0.1)
    _gpu_only(mi.split_kv_decode_varlen, q, k, v, pt, ctx, indptr, 0.1)


def test_prefix_and_cascade_checks():
    R, Hq, Hkv = 4, 8, 2
    q = _t((R, Hq, 128), BF16)
    k = _t((10, Hkv, 16, 128), BF16)
    v = _t((10, Hkv, 16, 128), BF16)
    pages = torch.zeros(4, dtype=torch.int32)        # 4 pages: up to 64 prefix tokens
    st = torch.zeros((R, 2), dtype=torch.int32)
    sl = torch.full((R,), 20, dtype=torch.int32)
    with pytest.raises(TypeError):
        mi.prefix_attention(q.to(F16), k, v, pages, 64, 0.1)
    with pytest.raises(ValueError):
        mi.prefix_attention(q, k, v, pages, 65, 0.1)
    need = mi.prefix_attention_workspace_bytes(R, Hq, Hkv, 128, 64)
    with pytest.raises(ValueError):
        mi.prefix_attention(q, k, v, pages, 64, 0.1, workspace=_t((need // 4 - 1,)))
    with pytest.raises(ValueError):
        mi.prefix_attention(q, k, v, pages, 64, 0.1, v_out=_t((R, Hq, 64)))
    with pytest.raises(TypeError):
        mi.cascade_decode_fused(q, k.to(F16), v, pages, 64, st, sl, 0.1)
    with pytest.raises(ValueError):
        mi.cascade_decode_fused(q, k, v, pages, 65, st, sl, 0.1)
    with pytest.raises(ValueError):
        mi.cascade_decode_fused(q, k, v, pages, 64, st[:3], sl, 0.1)
    with pytest.raises(ValueError):
        mi.cascade_decode_fused(q, k, v, pages, 64, st, sl[:3], 0.1)
    with pytest.raises(ValueError):
        mi.cascade_decode_fused(q, k, v, pages, 64, st, sl, 0.1, o_part=_t((R, Hq, 2, 128)))
    with pytest.raises(ValueError):
        mi.cascade_decode_fused(q, k, v, pages, 64, st, sl, 0.1,
                                counters=torch.zeros(R * Hkv - 1, dtype=torch.int32))
    _gpu_only(mi.prefix_attention, q, k, v, pages, 64, 0.1)
    _gpu_only(mi.cascade_decode_fused, q, k, v, pages, 64, st, sl, 0.1)


def test_stream_read_checks():
    with pytest.raises(TypeError):
        mi.stream_read(_t((16,)), xor_out=torch.zeros(1, dtype=torch.int64))
    _gpu_only(mi.stream_read, _t((16,)))
