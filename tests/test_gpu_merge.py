"""GPU parity of the merge kernels against the fp64 oracle (through the C ABI).

Workloads: the two-state merge at bf16 S=32768, H=32, D=128 (1% of rows with
both states empty; every row), the N-state merge at fp16 S=64, N=4, H=8, D=128
(10% of states empty) and at S=65536 (sampled), and smaller cases spanning several
workgroups with ragged tails, every dtype pair and the special LSE values.
"""
import numpy as np
import pytest
import torch

import lse_attention_state_amd as mi
import oracle
from lse_attention_state_amd import inputs
from parity import TORCH_DT, check_lse, check_values, host64, to_device

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _run_merge_state(case, out_dtype=None, prefill_nan=True):
    dt = case["dtype"]
    va, vb = to_device(case["va"], dt), to_device(case["vb"], dt)
    sa, sb = torch.from_numpy(case["sa"]).cuda(), torch.from_numpy(case["sb"]).cuda()
    odt = TORCH_DT[out_dtype or dt]
    v_out = torch.full(va.shape, float("nan"), dtype=odt, device="cuda") if prefill_nan else None
    s_out = torch.full(sa.shape, float("nan"), dtype=torch.float32, device="cuda")
    v, s = mi.merge_state(va, sa, vb, sb, v_out=v_out, s_out=s_out, out_dtype=odt)
    torch.cuda.synchronize()
    return v, s


@pytest.mark.parametrize("dt_in,dt_out", [("f16", "f16"), ("bf16", "bf16"), ("f32", "f32"),
                                          ("f16", "f32"), ("bf16", "f16"), ("f32", "bf16")])
@pytest.mark.parametrize("D", [8, 64, 128, 136, 512])
def test_merge_state_small(dt_in, dt_out, D):
    _say("merge_state", dt_in, dt_out, D)
    case = inputs.merge_state_case(31 + D, S=37, H=7, D=D, dtype=dt_in, s_lo=-30, s_hi=30,
                                   empty_row_frac=0.05)
    v, s = _run_merge_state(case, dt_out)
    rv, rs = oracle.merge_state(case["va"], case["sa"], case["vb"], case["sb"], dt_in)
    check_values(v, rv)
    check_lse(s, rs)


def test_merge_state_full_size():
    """bf16 S=32768, H=32, D=128: every one of the 1,048,576 rows against the
    oracle (in slices of 131072 rows), every empty row exactly (0, -inf)."""
    _say("merge_state full size")
    case = inputs.merge_state_case(1002, S=32768, H=32, D=128, dtype="bf16")
    v, s = _run_merge_state(case)
    vh, sh = v.view(-1, 128), s.view(-1)
    assert not torch.isnan(vh).any() and not torch.isnan(sh).any()
    empty = np.flatnonzero(case["empty_rows"].reshape(-1))
    assert empty.size > 0
    e_idx = torch.from_numpy(empty).cuda()
    assert torch.all(sh[e_idx] == float("-inf")) and torch.all(vh[e_idx] == 0)
    va, vb = case["va"].reshape(-1, 128), case["vb"].reshape(-1, 128)
    sa, sb = case["sa"].reshape(-1), case["sb"].reshape(-1)
    rows = va.shape[0]
    step = 131072
    max_abs, ulp_only = 0.0, 0
    for r0 in range(0, rows, step):
        sl = slice(r0, min(rows, r0 + step))
        rv, rs = oracle.merge_state(np.ascontiguousarray(va[sl]), np.ascontiguousarray(sa[sl]),
                                    np.ascontiguousarray(vb[sl]), np.ascontiguousarray(sb[sl]),
                                    "bf16")
        st = check_values(vh[sl], rv)
        check_lse(sh[sl], rs)
        max_abs = max(max_abs, st["max_abs"])
        ulp_only += st["ulp_only"]
    _say(f"merge_state full size: {rows} rows, max |dv| {max_abs:.3e}, "
         f"{ulp_only} elements pass only by the rounding term")


def test_merge_state_special_values():
    _say("merge_state special values")
    inf, nan = np.inf, np.nan
    # rows: (s_a, s_b): both empty, +inf vs finite, NaN vs finite, finite vs -inf, equal
    sa = np.array([-inf, 1.0, 2.5, 3.0, 10.0, inf, nan], np.float32)
    sb = np.array([-inf, inf, nan, -inf, 10.0, inf, -inf], np.float32)
    D = 16
    g = np.random.default_rng(1)
    va = g.standard_normal((7, D)).astype(np.float32)
    vb = g.standard_normal((7, D)).astype(np.float32)
    va[0] = 0
    vb[0] = np.nan          # an empty state's v is skipped whatever it holds
    vb[1] = np.nan          # +inf LSE is sanitised: v_b must not leak
    vb[2] = np.nan
    vb[3] = np.nan
    va[5] = np.nan
    case = {"va": va, "vb": vb, "sa": sa, "sb": sb, "dtype": "f32"}
    v, s = _run_merge_state(case)
    got_v, got_s = host64(v), host64(s)
    assert got_s[0] == -np.inf and np.all(got_v[0] == 0)
    for r in (1, 2, 3):
        assert np.allclose(got_v[r], va[r].astype(np.float64), rtol=1e-6, atol=0)
        assert got_s[r] == pytest.approx(float(sa[r]), abs=1e-6)
    assert got_s[4] == pytest.approx(11.0, abs=1e-6)
    assert np.allclose(got_v[4], (va[4].astype(np.float64) + vb[4]) / 2, rtol=1e-6, atol=1e-6)
    assert got_s[5] == -np.inf and np.all(got_v[5] == 0)     # both sanitised to empty
    assert got_s[6] == -np.inf and np.all(got_v[6] == 0)
    rv, rs = oracle.merge_state(va, sa, vb, sb, "f32")
    check_values(v, rv)
    check_lse(s, rs)


def test_merge_state_commutes_bit_exactly_and_in_place():
    _say("merge_state commutativity / in place")
    case = inputs.merge_state_case(77, S=300, H=8, D=128, dtype="f16", s_lo=-10, s_hi=10)
    va, vb = to_device(case["va"], "f16"), to_device(case["vb"], "f16")
    sa, sb = torch.from_numpy(case["sa"]).cuda(), torch.from_numpy(case["sb"]).cuda()
    v1, s1 = mi.merge_state(va, sa, vb, sb)
    v2, s2 = mi.merge_state(vb, sb, va, sa)
    torch.cuda.synchronize()
    assert torch.equal(v1.view(torch.int16), v2.view(torch.int16))
    assert torch.equal(s1.view(torch.int32), s2.view(torch.int32))
    va2, sa2 = va.clone(), sa.clone()
    mi.merge_state(va2, sa2, vb, sb, v_out=va2, s_out=sa2)
    torch.cuda.synchronize()
    assert torch.equal(va2.view(torch.int16), v1.view(torch.int16))
    assert torch.equal(sa2.view(torch.int32), s1.view(torch.int32))


@pytest.mark.parametrize("N,H,dt_in,dt_out", [(4, 8, "f16", "f16"), (1, 3, "bf16", "bf16"),
                                              (2, 1, "f32", "f32"), (3, 5, "bf16", "f32"),
                                              (7, 2, "f16", "bf16"), (64, 1, "f32", "f16"),
                                              (100, 2, "f32", "f32")])
def test_merge_states(N, H, dt_in, dt_out):
    _say("merge_states", N, H, dt_in, dt_out)
    for S, D in ((64, 128), (13, 64), (5, 136)):
        case = inputs.merge_states_case(500 + N * 7 + S, S=S, N=N, H=H, D=D, dtype=dt_in)
        v_dev = to_device(case["v"], dt_in)
        s_dev = torch.from_numpy(case["s"]).cuda()
        v_out = torch.full((S, H, D), float("nan"), dtype=TORCH_DT[dt_out], device="cuda")
        s_out = torch.full((S, H), float("nan"), dtype=torch.float32, device="cuda")
        mi.merge_states(v_dev, s_dev, v_out=v_out, s_out=s_out)
        torch.cuda.synchronize()
        rv, rs = oracle.merge_states(case["v"], case["s"], dt_in)
        check_values(v_out, rv)
        check_lse(s_out, rs)


def test_merge_states_config_shape_with_all_empty_rows_and_special_lse():
    """fp16 S=64, N=4, H=8, D=128 with 10% empty states, then the same input with
    some rows made all-empty and some LSEs set to +inf / NaN."""
    _say("merge_states special")
    case = inputs.merge_states_case(1001, S=64, N=4, H=8, D=128, dtype="f16")
    s = case["s"].copy()
    v = case["v"].copy()
    s[3, :, 2] = -np.inf
    v[3, :, 2] = 0
    s[5, 1, 0] = np.inf
    s[6, 2, 7] = np.nan
    v[6, 2, 7] = 0x7E00   # NaN payload in a state whose LSE is NaN: must be skipped
    for arr_s, arr_v in ((case["s"], case["v"]), (s, v)):
        vo, so = mi.merge_states(to_device(arr_v, "f16"), torch.from_numpy(arr_s).cuda())
        torch.cuda.synchronize()
        rv, rs = oracle.merge_states(arr_v, arr_s, "f16")
        check_values(vo, rv)
        check_lse(so, rs)
    assert host64(so)[3, 2] == -np.inf and np.all(host64(vo)[3, 2] == 0)


def test_merge_states_streaming_size_sampled():
    """fp16 S=65536, N=4, H=8, D=128 (the size that streams HBM, same inputs and
    launch as the measured step): every all-empty row checked, 4096 sampled
    (position, head) rows against the oracle, plus global no-NaN."""
    _say("merge_states streaming size")
    S, N, H, D = 65536, 4, 8, 128
    case = inputs.merge_states_case(1001, S=S, N=N, H=H, D=D, dtype="f16")
    vo = torch.full((S, H, D), float("nan"), dtype=torch.float16, device="cuda")
    so = torch.full((S, H), float("nan"), dtype=torch.float32, device="cuda")
    mi.merge_states(to_device(case["v"], "f16"), torch.from_numpy(case["s"]).cuda(),
                    v_out=vo, s_out=so)
    torch.cuda.synchronize()
    vh, sh = vo.view(-1, D), so.view(-1)
    assert not torch.isnan(vh).any() and not torch.isnan(sh).any()
    g = np.random.default_rng(1)
    rows = np.sort(g.choice(S * H, size=4096, replace=False))
    pos, head = rows // H, rows % H
    rv, rs = oracle.merge_states(case["v"][pos, :, head][:, :, None, :],
                                 case["s"][pos, :, head][:, :, None], "f16")
    idx = torch.from_numpy(rows).cuda()
    stats = check_values(vh[idx], rv.reshape(-1, D))
    check_lse(sh[idx], rs.reshape(-1))
    # all-empty (position, head) rows give exactly (0, -inf)
    empty = np.flatnonzero(np.all(np.isneginf(case["s"]), axis=1).reshape(-1))
    if empty.size:
        e_idx = torch.from_numpy(empty).cuda()
        assert torch.all(sh[e_idx] == float("-inf")) and torch.all(vh[e_idx] == 0)
    _say("merge_states streaming size stats", stats)


def test_merge_states_matches_pairwise_merge_state():
    """N = 2 through merge_states equals merge_state on the two slices (same kernel math)."""
    _say("merge_states vs merge_state")
    case = inputs.merge_states_case(9, S=128, N=2, H=4, D=128, dtype="bf16")
    v = to_device(case["v"], "bf16")
    s = torch.from_numpy(case["s"]).cuda()
    vo, so = mi.merge_states(v, s)
    va, vb = v[:, 0].contiguous(), v[:, 1].contiguous()
    sa, sb = s[:, 0].contiguous(), s[:, 1].contiguous()
    v2, s2 = mi.merge_state(va, sa, vb, sb)
    torch.cuda.synchronize()
    rv, rs = oracle.merge_states(case["v"], case["s"], "bf16")
    check_values(vo, rv)
    check_values(v2, rv)
    check_lse(so, rs)
    check_lse(s2, rs)
