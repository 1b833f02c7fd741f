"""The decode entry point that allocates nothing (partials in the library's
static device scratch) against the two-launch decode with caller workspaces,
through the C ABI: two calls in a row, the second smaller, both bit-identical
to mi_split_kv_decode (same kernels, same arithmetic) and within tolerance of
the oracle; work beyond the scratch is refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import lse_attention_state_amd as mi
import oracle
from lse_attention_state_amd import inputs
from parity import check_lse, check_values, to_device

pytestmark = pytest.mark.gpu


def _dev(case):
    dt = case["dtype"]
    return (to_device(case["q"], dt), to_device(case["k"], dt), to_device(case["v"], dt),
            torch.from_numpy(case["page_table"]).cuda(), torch.from_numpy(case["ctx_lens"]).cuda())


@pytest.mark.parametrize("order", ["large_then_small", "small_then_large"])
def test_noalloc_decode_matches_two_launch_decode(order):
    runs = [(np.array([37, 5000, 1, 900, 0, 2048], np.int32), 16, "f16", 32, 8),
            (np.array([300], np.int32), 4, "bf16", 8, 2)]
    if order == "small_then_large":
        runs = runs[::-1]
    for i, (ctx, splits, dt, Hq, Hkv) in enumerate(runs):
        print("noalloc decode", order, i, ctx.tolist(), splits, dt, flush=True)
        case = inputs.paged_kv_case(900 + i, ctx, Hq, Hkv, 128, 16, dtype=dt)
        q, k, v, pt, cl = _dev(case)
        B = len(ctx)
        o_ref, lse_ref = mi.split_kv_decode(q, k, v, pt, cl, splits, case["sm_scale"])
        out = torch.full((B, Hq, 128), float("nan"), dtype=q.dtype, device="cuda")
        lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
        mi.split_kv_decode_noalloc(q, k, v, pt, cl, splits, case["sm_scale"], out, lse)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), o_ref.view(torch.int16))
        assert torch.equal(lse.view(torch.int32), lse_ref.view(torch.int32))
        args = (case["q"], case["k"], case["v"], case["page_table"], case["ctx_lens"],
                case["sm_scale"])
        o, s = oracle.attention(*args, dt, dt)
        check_values(out, o)
        check_lse(lse, s)


def test_noalloc_decode_refuses_work_beyond_the_scratch():
    ctx = np.array([64, 64], np.int32)
    case = inputs.paged_kv_case(950, ctx, 32, 8, 128, 16, dtype="f16")
    q, k, v, pt, cl = _dev(case)
    out = torch.zeros((2, 32, 128), dtype=torch.float16, device="cuda")
    splits = mi.NOALLOC_MAX_PARTIAL_ROWS // 64 + 1          # 2 * 32 * splits > the maximum
    assert splits <= 1024
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = mi.lib().mi_split_kv_decode_noalloc(p(q), p(k), p(v), p(pt), pt.shape[1], p(cl), 2, 32,
                                            8, 128, 16, k.shape[0], splits,
                                            ctypes.c_float(case["sm_scale"]), mi.MI_F16, p(out),
                                            None, mi.MI_F16, st)
    assert rc == 7   # MI_ERR_SCRATCH
    with pytest.raises(ValueError):
        mi.split_kv_decode_noalloc(q, k, v, pt, cl, splits, case["sm_scale"], out)


def test_noalloc_decode_under_graph_capture():
    """Graph capture is one of the uses this entry point is for: one call is
    captured, then replayed with new queries copied into the captured buffers
    (eager work in between); every replay equals the two-launch decode with
    workspaces on the same inputs, bit for bit."""
    ctx = np.array([700, 33, 4096], np.int32)
    case = inputs.paged_kv_case(960, ctx, 32, 8, 128, 16, dtype="f16")
    q, k, v, pt, cl = _dev(case)
    splits = 8
    out = torch.empty((3, 32, 128), dtype=torch.float16, device="cuda")
    lse = torch.empty((3, 32), dtype=torch.float32, device="cuda")

    def work():
        mi.split_kv_decode_noalloc(q, k, v, pt, cl, splits, case["sm_scale"], out, lse)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work()                                     # first call on the device: outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work()
    torch.cuda.synchronize()
    g = torch.Generator(device="cpu").manual_seed(961)
    for rep in range(3):
        print("noalloc graph replay", rep, flush=True)
        q.copy_(torch.randn(q.shape, generator=g).half().cuda())
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got_o, got_s = out.clone(), lse.clone()
        _ = (torch.randn(1024, device="cuda") * 2).sum()
        o_ref, s_ref = mi.split_kv_decode(q, k, v, pt, cl, splits, case["sm_scale"])
        torch.cuda.synchronize()
        assert torch.equal(got_o.view(torch.int16), o_ref.view(torch.int16))
        assert torch.equal(got_s.view(torch.int32), s_ref.view(torch.int32))
