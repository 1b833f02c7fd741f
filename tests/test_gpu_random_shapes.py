"""Seeded random shapes against the oracle: the N-state, variable-length and
two-level merges (including fp32 rows read in halves, adaptive batch sizes and
every team-size regime of the segmented kernel) and the decode entry points
(uniform and per-sequence plans, both launch forms). Shapes are drawn from a
fixed generator, so every run checks the same cases."""
import numpy as np
import pytest
import torch

import lse_attention_state_amd as mi
import oracle
from lse_attention_state_amd import inputs
from parity import TORCH_DT, check_lse, check_values, to_device

pytestmark = pytest.mark.gpu

_DTS = ["f16", "bf16", "f32"]


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("case_id", range(12))
def test_random_merges(case_id):
    g = np.random.default_rng(4000 + case_id)
    D = int(g.choice([8, 64, 96, 128, 136, 256, 512]))
    H = int(g.integers(1, 9))
    dt_in = str(g.choice(_DTS))
    dt_out = str(g.choice(_DTS))
    S = int(g.integers(1, 300))
    N = int(g.choice([1, 2, 3, 5, 8, 17, 64, 200]))
    _say("random merges", case_id, dict(S=S, N=N, H=H, D=D, dt_in=dt_in, dt_out=dt_out))
    c = inputs.merge_states_case(4100 + case_id, S=S, N=N, H=H, D=D, dtype=dt_in,
                                 s_lo=-40, s_hi=40)
    v_dev = to_device(c["v"], dt_in)
    s_dev = torch.from_numpy(c["s"]).cuda()
    rv, rs = oracle.merge_states(c["v"], c["s"], dt_in)
    odt = TORCH_DT[dt_out]
    # N-state entry (the segmented kernel below 2048 rows)
    vo, so = mi.merge_states(v_dev, s_dev, out_dtype=odt)
    torch.cuda.synchronize()
    check_values(vo, rv)
    check_lse(so, rs)
    # the same sets through an index pointer array
    indptr = (np.arange(S + 1) * N).astype(np.int32)
    vo2, so2 = mi.merge_states_varlen(v_dev.reshape(S * N, H, D), s_dev.reshape(S * N, H),
                                      torch.from_numpy(indptr).cuda(), out_dtype=odt)
    torch.cuda.synchronize()
    check_values(vo2, rv)
    check_lse(so2, rs)
    # two levels through an fp32 workspace
    need = mi.merge_states_workspace_bytes(S, N, H, D)
    ws = (torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda")
          if need else None)
    vo3, so3 = mi.merge_states_two_level(v_dev, s_dev, out_dtype=odt, workspace=ws)
    torch.cuda.synchronize()
    check_values(vo3, rv)
    check_lse(so3, rs)


@pytest.mark.parametrize("case_id", range(6))
def test_random_varlen_sets(case_id):
    g = np.random.default_rng(4200 + case_id)
    D = int(g.choice([64, 128, 256]))
    H = int(g.integers(1, 9))
    dt_in = str(g.choice(_DTS))
    S = int(g.integers(1, 2000))
    max_len = int(g.choice([2, 8, 40, 300]))
    _say("random varlen", case_id, dict(S=S, max_len=max_len, H=H, D=D, dt_in=dt_in))
    indptr = inputs.segment_indptr(4300 + case_id, S, max_len)
    total = int(indptr[-1])
    c = inputs.merge_states_case(4400 + case_id, S=1, N=max(total, 1), H=H, D=D, dtype=dt_in)
    v = np.ascontiguousarray(c["v"].reshape(-1, H, D)[:max(total, 1)])
    s = np.ascontiguousarray(c["s"].reshape(-1, H)[:max(total, 1)])
    vo, so = mi.merge_states_varlen(to_device(v, dt_in), torch.from_numpy(s).cuda(),
                                    torch.from_numpy(indptr).cuda(), out_dtype=torch.float16)
    torch.cuda.synchronize()
    rv, rs = oracle.merge_states_varlen(v, s, indptr, dt_in)
    check_values(vo, rv)
    check_lse(so, rs)


@pytest.mark.parametrize("case_id", range(8))
def test_random_decode(case_id):
    g = np.random.default_rng(4500 + case_id)
    G = int(g.choice([1, 2, 4, 8]))
    Hkv = int(g.choice([1, 2, 8]))
    Hq = G * Hkv
    B = int(g.integers(1, 9))
    ctx = g.integers(0, 5000, size=B).astype(np.int32)
    dt = str(g.choice(["f16", "bf16"]))
    splits = int(g.choice([1, 3, 7, 16, 64]))
    _say("random decode", case_id, dict(B=B, Hq=Hq, Hkv=Hkv, splits=splits, dt=dt,
                                        ctx=ctx.tolist()))
    case = inputs.paged_kv_case(4600 + case_id, ctx, Hq, Hkv, 128, 16, dtype=dt)
    q, k, v = (to_device(case["q"], dt), to_device(case["k"], dt), to_device(case["v"], dt))
    pt = torch.from_numpy(case["page_table"]).cuda()
    cl = torch.from_numpy(ctx).cuda()
    ro, rs = oracle.attention(case["q"], case["k"], case["v"], case["page_table"], ctx,
                              case["sm_scale"], dt, dt)
    o1, s1 = mi.split_kv_decode(q, k, v, pt, cl, splits, case["sm_scale"])
    o2, s2 = mi.split_kv_decode_fused(q, k, v, pt, cl, splits, case["sm_scale"])
    indptr = mi.plan_splits_varlen(ctx, Hkv, 16)
    o3, s3 = mi.split_kv_decode_varlen(q, k, v, pt, cl, indptr, case["sm_scale"])
    torch.cuda.synchronize()
    for o, s in ((o1, s1), (o2, s2), (o3, s3)):
        check_values(o, ro)
        check_lse(s, rs)
