"""HIP-graph capture of the library's calls: the single-launch decode, the
two-launch cascade and a merge are captured once, then replayed several times
with new inputs copied into the captured buffers and eager work in between;
every replay must equal the eager result for the same inputs, and the decode
counters must be zero after each replay (the kernels reset them themselves --
nothing in the captured work is a memset)."""
import numpy as np
import pytest
import torch

import lse_attention_state_amd as mi
from lse_attention_state_amd import inputs
from parity import to_device

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def test_graph_replays_decode_cascade_and_merge():
    _say("graph capture")
    dev = torch.device("cuda")
    # decode: B=4 mixed lengths, Hq=32, Hkv=8, 4 splits, fp16
    ctx = np.array([37, 1000, 4096, 1], np.int32)
    case = inputs.paged_kv_case(71, ctx, 32, 8, 128, 16, dtype="f16")
    q = to_device(case["q"], "f16")
    k, v = to_device(case["k"], "f16"), to_device(case["v"], "f16")
    pt = torch.from_numpy(case["page_table"]).cuda()
    cl = torch.from_numpy(ctx).cuda()
    splits = 4
    o_part = torch.empty((4, 32, splits, 128), dtype=torch.float32, device=dev)
    lse_part = torch.empty((4, 32, splits), dtype=torch.float32, device=dev)
    counters = torch.zeros((4, 8), dtype=torch.int32, device=dev)
    o = torch.empty((4, 32, 128), dtype=torch.float16, device=dev)
    lse = torch.empty((4, 32), dtype=torch.float32, device=dev)
    # cascade: 6 requests share a 256-token prefix, 48-token suffixes, bf16
    cas = inputs.cascade_case(72, R=6, prefix_len=256, suffix_len=48, Hq=8, Hkv=2)
    cq = to_device(cas["q"], "bf16")
    ck, cv = to_device(cas["k"], "bf16"), to_device(cas["v"], "bf16")
    cpages = torch.from_numpy(cas["prefix_pages"]).cuda()
    ctab = torch.from_numpy(cas["suffix_table"]).cuda()
    clen = torch.from_numpy(cas["suffix_lens"]).cuda()
    ws = torch.empty(mi.prefix_attention_workspace_bytes(6, 8, 2, 128, 256) // 4,
                     dtype=torch.float32, device=dev)
    c_op = torch.empty((6, 8, 1, 128), dtype=torch.float32, device=dev)
    c_lp = torch.empty((6, 8, 1), dtype=torch.float32, device=dev)
    c_cnt = torch.zeros((6, 2), dtype=torch.int32, device=dev)
    c_o = torch.empty((6, 8, 128), dtype=torch.bfloat16, device=dev)
    c_lse = torch.empty((6, 8), dtype=torch.float32, device=dev)
    # merge: the decode output merged with a second state
    vb = torch.randn((4, 32, 128), device=dev).half()
    sb = torch.randn((4, 32), device=dev) * 4
    m_v = torch.empty((4, 32, 128), dtype=torch.float16, device=dev)
    m_s = torch.empty((4, 32), dtype=torch.float32, device=dev)

    def work():
        mi.split_kv_decode_fused(q, k, v, pt, cl, splits, case["sm_scale"], counters=counters,
                                 o_part=o_part, lse_part=lse_part, out=o, lse=lse)
        mi.cascade_decode_fused(cq, ck, cv, cpages, 256, ctab, clen, cas["sm_scale"],
                                workspace=ws, o_part=c_op, lse_part=c_lp, counters=c_cnt,
                                out=c_o, lse=c_lse)
        mi.merge_state(o, lse, vb, sb, v_out=m_v, s_out=m_s)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work()                                     # warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work()
    torch.cuda.synchronize()

    g = torch.Generator(device="cpu").manual_seed(73)
    for rep in range(4):
        # new inputs in the captured buffers
        q.copy_(torch.randn(q.shape, generator=g).half().to(dev))
        cq.copy_(torch.randn(cq.shape, generator=g).bfloat16().to(dev))
        sb.copy_((torch.randn(sb.shape, generator=g) * 4).to(dev))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (o, lse, c_o, c_lse, m_v, m_s)]
        assert not counters.any() and not c_cnt.any(), "counters must be zero after a replay"
        # eager work in between, then the eager result for the same inputs
        _ = (torch.randn(1024, device=dev) * 2).sum()
        work()
        torch.cuda.synchronize()
        want = (o, lse, c_o, c_lse, m_v, m_s)
        for a, b in zip(got, want):
            assert torch.equal(a, b), f"replay {rep} differs from the eager result"
        _say("replay", rep, "ok")
