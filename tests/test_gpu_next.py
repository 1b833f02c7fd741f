"""GPU parity, through the C ABI, of the entry points beyond the core path:
the attention-sink fold, the masked in-place merge, the variable-length
(and many-state) merge, and split-KV decode with per-sequence split counts,
each against the fp64 oracle.

Workloads: states at bf16 S=32768, H=32, D=128 (sampled) and small ragged
cases over dtypes and head dims; segments of 0..3000 states; the mixed decode
batch B=32, ctx ~ U[1, 8192] with forced short sequences, Hq=32, Hkv=8, fp16,
split counts from the per-sequence planner (checked in full, single launch and
two launches); B=1, ctx=32768 (the planner gives 64 splits of 32 pages); and
small ragged decode cases over group sizes and both 16-bit dtypes.
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


def _states(seed, S, H, D, dtype, lo=-20.0, hi=40.0, empty_frac=0.1):
    c = inputs.merge_states_case(seed, S=S, N=1, H=H, D=D, dtype=dtype, s_lo=lo, s_hi=hi,
                                 empty_frac=0.0)
    v, s = c["v"][:, 0], c["s"][:, 0]
    g = np.random.default_rng(seed + 7)
    e = g.random((S, H)) < empty_frac
    s[e] = -np.inf
    v[e] = 0
    return np.ascontiguousarray(v), np.ascontiguousarray(s)


# ----------------------------------------------------------------------------- sink

@pytest.mark.parametrize("dt_in,dt_out", [("f16", "f16"), ("bf16", "bf16"), ("f32", "f32"),
                                          ("f32", "bf16"), ("bf16", "f32")])
@pytest.mark.parametrize("D", [8, 128, 520 - 8])
def test_sink_small(dt_in, dt_out, D):
    _say("sink", dt_in, dt_out, D)
    S, H = 45, 6
    v, s = _states(70 + D, S, H, D, dt_in, lo=-12, hi=12)
    sink = inputs.sink_logits(71 + D, H)
    sink[1], sink[2], sink[3] = -np.inf, np.nan, np.inf     # no sink; sanitised to no sink
    s[0, 0], s[1, 1] = np.nan, np.inf                        # sanitised to empty
    vd, sd = to_device(v, dt_in), torch.from_numpy(s).cuda()
    odt = TORCH_DT[dt_out]
    vo = torch.full(vd.shape, float("nan"), dtype=odt, device="cuda")
    so = torch.full(sd.shape, float("nan"), dtype=torch.float32, device="cuda")
    mi.merge_sink(vd, sd, torch.from_numpy(sink).cuda(), v_out=vo, s_out=so)
    torch.cuda.synchronize()
    rv, rs = oracle.merge_sink(v, s, sink, dt_in)
    check_values(vo, rv)
    check_lse(so, rs)


def test_sink_in_place_full_size_sampled():
    """bf16 S=32768, H=32, D=128 in place: 4096 sampled rows against the oracle."""
    _say("sink full size in place")
    c = inputs.merge_state_case(1102, S=32768, H=32, D=128, dtype="bf16")
    sink = inputs.sink_logits(1103, 32, lo=0.0, hi=60.0 * 0.6931)
    v = to_device(c["va"], "bf16")
    s = torch.from_numpy(c["sa"]).cuda()
    mi.merge_sink(v, s, torch.from_numpy(sink).cuda(), v_out=v, s_out=s)
    torch.cuda.synchronize()
    vh, sh = v.view(-1, 128), s.view(-1)
    assert not torch.isnan(vh).any() and not torch.isnan(sh).any()
    rows = np.sort(np.random.default_rng(2).choice(32768 * 32, 4096, replace=False))
    rv, rs = _sink_rows(c, sink, rows)
    idx = torch.from_numpy(rows).cuda()
    check_values(vh[idx], rv)
    check_lse(sh[idx], rs)


def _sink_rows(c, sink, rows):
    # the oracle over the sampled rows, each with its own head's sink
    out_v, out_s = [], []
    for h in range(32):
        sel = rows[rows % 32 == h]
        vv, ss = oracle.merge_sink(c["va"].reshape(-1, 1, 128)[sel], c["sa"].reshape(-1, 1)[sel],
                                   sink[h:h + 1], "bf16")
        out_v.append((sel, vv[:, 0]))
        out_s.append((sel, ss[:, 0]))
    order = np.argsort(np.concatenate([a for a, _ in out_v]))
    return (np.concatenate([b for _, b in out_v])[order],
            np.concatenate([b for _, b in out_s])[order])


# ----------------------------------------------------------------------------- masked in place

@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("D", [16, 128, 256])
def test_merge_state_in_place_masked(dtype, D):
    _say("in place masked", dtype, D)
    S, H = 67, 5
    va, sa = _states(80 + D, S, H, D, dtype)
    vb, sb = _states(81 + D, S, H, D, dtype)
    mask = inputs.position_mask(82 + D, S)
    sa[np.flatnonzero(mask == 0)[:2], 0] = np.nan          # kept as is (not sanitised)
    sa[np.flatnonzero(mask == 1)[:2], 1] = np.nan          # sanitised where merged
    v, s = to_device(va, dtype), torch.from_numpy(sa).cuda()
    mi.merge_state_in_place(v, s, to_device(vb, dtype), torch.from_numpy(sb).cuda(),
                            torch.from_numpy(mask).cuda())
    torch.cuda.synchronize()
    rv, rs = oracle.merge_state_masked(va, sa, vb, sb, mask, dtype)
    off = mask == 0
    # untouched positions: bit-identical to the input, v and s alike
    bits = np.uint32 if dtype == "f32" else np.uint16
    got_v = (v.cpu().numpy() if dtype == "f32" else v.cpu().view(torch.int16).numpy()).view(bits)
    assert np.array_equal(got_v[off], np.asarray(va).view(bits)[off])
    assert np.array_equal(s.cpu().numpy()[off].view(np.uint32), sa[off].view(np.uint32))
    on = torch.from_numpy(mask == 1).cuda()
    check_values(v[on], rv[mask == 1])
    check_lse(s[on], rs[mask == 1])


def test_merge_state_in_place_without_mask_is_merge_state():
    _say("in place no mask")
    c = inputs.merge_state_case(90, S=300, H=8, D=128, dtype="bf16")
    v, s = to_device(c["va"], "bf16"), torch.from_numpy(c["sa"]).cuda()
    vb, sb = to_device(c["vb"], "bf16"), torch.from_numpy(c["sb"]).cuda()
    ref_v, ref_s = mi.merge_state(v, s, vb, sb)
    mi.merge_state_in_place(v, s, vb, sb, None)
    torch.cuda.synchronize()
    assert torch.equal(v.view(torch.int16), ref_v.view(torch.int16))
    assert torch.equal(s, ref_s)


def test_merge_state_in_place_full_size_sampled():
    """bf16 S=32768, H=32, D=128, half the positions masked out."""
    _say("in place full size")
    c = inputs.merge_state_case(1002, S=32768, H=32, D=128, dtype="bf16")
    mask = inputs.position_mask(1010, 32768)
    v, s = to_device(c["va"], "bf16"), torch.from_numpy(c["sa"]).cuda()
    mi.merge_state_in_place(v, s, to_device(c["vb"], "bf16"), torch.from_numpy(c["sb"]).cuda(),
                            torch.from_numpy(mask).cuda().bool())
    torch.cuda.synchronize()
    pos = np.sort(np.random.default_rng(3).choice(32768, 256, replace=False))
    rv, rs = oracle.merge_state_masked(c["va"][pos], c["sa"][pos], c["vb"][pos], c["sb"][pos],
                                       mask[pos], "bf16")
    idx = torch.from_numpy(pos).cuda()
    check_values(v[idx], rv)
    check_lse(s[idx], rs)


# ----------------------------------------------------------------------------- variable-length merge

@pytest.mark.parametrize("dt_in,dt_out", [("f32", "f16"), ("f16", "f16"), ("bf16", "f32")])
@pytest.mark.parametrize("D,H", [(128, 1), (128, 8), (64, 3), (512, 2), (8, 4)])
def test_merge_states_varlen(dt_in, dt_out, D, H):
    _say("varlen merge", dt_in, dt_out, D, H)
    indptr = inputs.segment_indptr(100 + D + H, 41, max_len=70)
    total = int(indptr[-1])
    v, s = _states(101 + D, total, H, D, dt_in)
    odt = TORCH_DT[dt_out]
    vo = torch.full((41, H, D), float("nan"), dtype=odt, device="cuda")
    so = torch.full((41, H), float("nan"), dtype=torch.float32, device="cuda")
    mi.merge_states_varlen(to_device(v, dt_in), torch.from_numpy(s).cuda(),
                           torch.from_numpy(indptr).cuda(), v_out=vo, s_out=so)
    torch.cuda.synchronize()
    rv, rs = oracle.merge_states_varlen(v, s, indptr, dt_in)
    check_values(vo, rv)
    check_lse(so, rs)


@pytest.mark.parametrize("S,N", [(32, 64), (4, 3000), (1, 1), (256, 16), (3, 1000)])
def test_merge_states_many_states(S, N):
    """Uniform segments given as an index pointer array; checked against the
    oracle's N-state merge ([S, N, H, D] is the same memory)."""
    _say("many states", S, N)
    c = inputs.merge_states_case(110 + N, S=S, N=N, H=1, D=128, dtype="f32", s_lo=-40, s_hi=40)
    indptr = (np.arange(S + 1) * N).astype(np.int32)
    vo, so = mi.merge_states_varlen(torch.from_numpy(c["v"].reshape(S * N, 1, 128)).cuda(),
                                    torch.from_numpy(c["s"].reshape(S * N, 1)).cuda(),
                                    torch.from_numpy(indptr).cuda(), out_dtype=torch.float16)
    torch.cuda.synchronize()
    rv, rs = oracle.merge_states(c["v"], c["s"], "f32")
    check_values(vo, rv)
    check_lse(so, rs)


def test_merge_states_varlen_clamps_bad_indptr():
    """Entries outside [0, total] or decreasing are clamped: such sets are empty
    or cut at total, and nothing is read outside the states."""
    _say("varlen clamp")
    v, s = _states(120, 10, 2, 16, "f32", empty_frac=0.0)
    indptr = np.array([0, 4, -3, 2, 50, 10], np.int32)
    vo, so = mi.merge_states_varlen(torch.from_numpy(v).cuda(), torch.from_numpy(s).cuda(),
                                    torch.from_numpy(indptr).cuda())
    torch.cuda.synchronize()
    # clamped: [0,4), [4,0)->empty, [0,2), [2,10) (50 cut at total), [10,10)
    seg_ref = [(0, 4), (0, 0), (0, 2), (2, 10), (10, 10)]
    for p, (a, b) in enumerate(seg_ref):
        if b <= a:
            assert host64(so)[p].tolist() == [-np.inf, -np.inf] and not host64(vo)[p].any()
        else:
            rv, rs = oracle.merge_states(v[a:b][None].copy(), s[a:b][None].copy(), "f32")
            check_values(vo[p], rv[0])
            check_lse(so[p], rs[0])


# ----------------------------------------------------------------------------- per-sequence split decode

def _dev(case):
    dt = case["dtype"]
    return (to_device(case["q"], dt), to_device(case["k"], dt), to_device(case["v"], dt),
            torch.from_numpy(case["page_table"]).cuda(), torch.from_numpy(case["ctx_lens"]).cuda())


def _varlen_decode(case, indptr, fused, out_dtype=None):
    q, k, v, pt, ctx = _dev(case)
    B, Hq, D = q.shape
    total = int(indptr[-1])
    nan = float("nan")
    o_part = torch.full((total, Hq, D), nan, dtype=torch.float32, device="cuda")
    lse_part = torch.full((total, Hq), nan, dtype=torch.float32, device="cuda")
    out = torch.full((B, Hq, D), nan, dtype=out_dtype or q.dtype, device="cuda")
    lse = torch.full((B, Hq), nan, dtype=torch.float32, device="cuda")
    counters = torch.zeros((B, case["Hkv"]), dtype=torch.int32, device="cuda") if fused else None
    mi.split_kv_decode_varlen(q, k, v, pt, ctx, indptr, case["sm_scale"], fused=fused,
                              counters=counters, o_part=o_part, lse_part=lse_part, out=out,
                              lse=lse)
    torch.cuda.synchronize()
    if fused:
        assert not counters.any(), "counters must be left zero"
    return out, lse, o_part, lse_part


def _check_varlen(case, indptr, fused, out_dtype=None):
    out, lse, o_part, lse_part = _varlen_decode(case, indptr, fused, out_dtype)
    args = (case["q"], case["k"], case["v"], case["page_table"], case["ctx_lens"], case["sm_scale"])
    op, sp = oracle.split_partials_varlen(*args, indptr, case["dtype"], case["dtype"])
    o, s = oracle.attention(*args, case["dtype"], case["dtype"])
    st = check_values(o_part, op, "o_part")
    check_lse(lse_part, sp, "lse_part")
    st2 = check_values(out, o, "o")
    check_lse(lse, s, "lse")
    return st, st2


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("Hq,Hkv", [(4, 1), (32, 8), (16, 2), (8, 8)])
def test_varlen_decode_small_ragged(fused, dtype, Hq, Hkv):
    _say("varlen decode small", fused, dtype, Hq, Hkv)
    ctx = np.array([1, 16, 17, 37, 100, 0, 250, 1000, 129], np.int32)
    case = inputs.paged_kv_case(400 + Hq, ctx, Hq, Hkv, 128, 16, dtype=dtype, extra_pages=3)
    counts = np.array([1, 2, 3, 4, 1, 2, 5, 9, 1], np.int32)   # includes empty splits
    indptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    _check_varlen(case, indptr, fused)


@pytest.mark.parametrize("fused", [True, False])
def test_varlen_decode_mixed_batch_planned(fused):
    """B=32, ctx ~ U[1,8192] with forced short sequences, Hq=32, Hkv=8, fp16;
    split counts from the per-sequence planner; every output checked."""
    _say("varlen decode mixed batch", fused)
    ctx = inputs.mixed_ctx_lens(1004, 32)
    case = inputs.paged_kv_case(1004, ctx, 32, 8, 128, 16, dtype="f16")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    indptr = mi.plan_splits_varlen(ctx, 8, 16)
    _, counts = oracle.plan_splits_varlen(32, 8, ctx, 16, cus)
    assert np.array_equal(np.diff(indptr), counts)
    st = _check_varlen(case, indptr, fused)
    _say("total splits", int(indptr[-1]), "stats", st)


def test_varlen_decode_long_context_b1():
    """B=1, ctx=32768: the per-sequence plan equals the uniform plan (64 splits)."""
    _say("varlen decode B=1 ctx=32768")
    ctx = np.array([32768], np.int32)
    case = inputs.paged_kv_case(1003, ctx, 32, 8, 128, 16, dtype="f16")
    indptr = mi.plan_splits_varlen(ctx, 8, 16, 256)
    assert indptr.tolist() == [0, 64]
    _check_varlen(case, indptr, True)


def test_varlen_decode_matches_uniform_partials():
    """Equal split counts: the per-sequence partials are the uniform ones
    (same kernel arithmetic, another layout) -- bit-identical."""
    _say("varlen vs uniform partials")
    ctx = np.array([37, 1000, 1, 300, 0], np.int32)
    case = inputs.paged_kv_case(130, ctx, 32, 8, 128, 16, dtype="bf16")
    q, k, v, pt, ctxd = _dev(case)
    op_u, lp_u = mi.split_kv_partial(q, k, v, pt, ctxd, 4, case["sm_scale"])
    indptr = np.arange(0, 21, 4, dtype=np.int32)
    _, _, op_v, lp_v = _varlen_decode(case, indptr, False)
    assert torch.equal(op_v.view(5, 4, 32, 128).permute(0, 2, 1, 3), op_u)
    assert torch.equal(lp_v.view(5, 4, 32).permute(0, 2, 1), lp_u)


def test_varlen_decode_repeated_calls_reuse_counters():
    _say("varlen decode repeated")
    ctx = inputs.mixed_ctx_lens(140, 12, hi=3000)
    case = inputs.paged_kv_case(140, ctx, 32, 8, 128, 16, dtype="f16")
    indptr = mi.plan_splits_varlen(ctx, 8, 16)
    q, k, v, pt, ctxd = _dev(case)
    counters = torch.zeros((12, 8), dtype=torch.int32, device="cuda")
    first = None
    for _ in range(3):
        o, lse = mi.split_kv_decode_varlen(q, k, v, pt, ctxd, indptr, case["sm_scale"],
                                           counters=counters)
        torch.cuda.synchronize()
        assert not counters.any()
        if first is None:
            first = (o.clone(), lse.clone())
        else:
            assert torch.equal(o, first[0]) and torch.equal(lse, first[1])


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("B", [63, 64, 300, 4031])
def test_varlen_decode_many_sequences(fused, B):
    """Batches past one 64-entry search round (B >= 64 takes the second round;
    4031 is the largest supported), short random lengths including 0, and
    random split counts 1..4 per sequence (so that segment boundaries fall
    everywhere in the index array)."""
    _say("varlen decode many sequences", B, fused)
    g = np.random.default_rng(500 + B)
    ctx = g.integers(0, 120, size=B).astype(np.int32)
    ctx[g.random(B) < 0.05] = 0
    Hq, Hkv = (8, 8) if B > 1000 else (16, 4)
    case = inputs.paged_kv_case(501 + B, ctx, Hq, Hkv, 128, 16, dtype="bf16")
    counts = g.integers(1, 5, size=B).astype(np.int32)
    indptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    _say("total splits", int(indptr[-1]))
    _check_varlen(case, indptr, fused)


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_varlen_decode_sequences_without_splits(fused, dtype):
    """Sequences given no split (equal consecutive split_indptr entries) at the
    start, in the middle and at the end of the batch come out as the empty
    state (0, -inf) in both launch forms, with every output pre-filled with
    NaN; the other sequences' partials and outputs match the oracle."""
    _say("varlen decode, sequences without splits", fused, dtype)
    ctx = np.array([40, 300, 17, 1000, 5, 64, 33], np.int32)
    case = inputs.paged_kv_case(610, ctx, 16, 4, 128, 16, dtype=dtype)
    counts = np.array([0, 2, 0, 3, 1, 0, 0], np.int32)
    indptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    out, lse, o_part, lse_part = _varlen_decode(case, indptr, fused)
    args = (case["q"], case["k"], case["v"], case["page_table"], case["ctx_lens"], case["sm_scale"])
    o, s = oracle.attention(*args, dtype, dtype)
    empty = counts == 0
    o[empty] = 0.0
    s[empty] = -np.inf
    check_values(out, o, "o")
    check_lse(lse, s, "lse")
    keep = np.flatnonzero(~empty)
    sub = (np.ascontiguousarray(case["q"][keep]), case["k"], case["v"],
           np.ascontiguousarray(case["page_table"][keep]), np.ascontiguousarray(ctx[keep]),
           case["sm_scale"])
    sub_indptr = np.concatenate([[0], np.cumsum(counts[keep])]).astype(np.int32)
    op, sp = oracle.split_partials_varlen(*sub, sub_indptr, dtype, dtype)
    check_values(o_part, op, "o_part")
    check_lse(lse_part, sp, "lse_part")


def test_varlen_decode_items_past_the_index_array():
    """total_splits larger than split_indptr[B] (inconsistent device data): the
    extra work items write empty partial rows and leave the counters alone, so
    the counters come back zero, the outputs match the consistent call, and a
    second call gives the same result."""
    import ctypes
    _say("varlen decode, items past the index array")
    ctx = np.array([100, 33, 700], np.int32)
    case = inputs.paged_kv_case(620, ctx, 32, 8, 128, 16, dtype="f16")
    q, k, v, pt, ctxd = _dev(case)
    B, Hq, D = q.shape
    counts = np.array([2, 1, 4], np.int32)
    indptr_h = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    indptr = torch.from_numpy(indptr_h).cuda()
    total = int(indptr_h[-1]) + 3
    nan = float("nan")
    counters = torch.zeros((B, 8), dtype=torch.int32, device="cuda")
    res = []
    for _ in range(2):
        o_part = torch.full((total, Hq, D), nan, dtype=torch.float32, device="cuda")
        lse_part = torch.full((total, Hq), nan, dtype=torch.float32, device="cuda")
        out = torch.full((B, Hq, D), nan, dtype=torch.float16, device="cuda")
        lse = torch.full((B, Hq), nan, dtype=torch.float32, device="cuda")
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        p = lambda t: ctypes.c_void_p(t.data_ptr())
        rc = mi.lib().mi_split_kv_decode_varlen(
            p(q), p(k), p(v), p(pt), pt.shape[1], p(ctxd), B, Hq, 8, D, 16, k.shape[0], p(indptr),
            total, ctypes.c_float(case["sm_scale"]), mi.MI_F16, p(o_part), p(lse_part),
            p(counters), p(out), p(lse), mi.MI_F16, st)
        assert rc == 0
        torch.cuda.synchronize()
        assert not counters.any(), "counters must be left zero"
        extra_o, extra_s = host64(o_part[total - 3:]), host64(lse_part[total - 3:])
        assert np.all(extra_o == 0) and np.all(np.isneginf(extra_s))
        res.append((out.clone(), lse.clone()))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])
    args = (case["q"], case["k"], case["v"], case["page_table"], case["ctx_lens"], case["sm_scale"])
    o, s = oracle.attention(*args, "f16", "f16")
    check_values(res[0][0], o, "o")
    check_lse(res[0][1], s, "lse")


@pytest.mark.parametrize("S,N,H,dt", [(64, 1024, 1, "f32"), (4, 3000, 2, "f16"), (1, 5000, 1, "bf16"),
                                      (32, 64, 1, "f32"), (8, 200, 3, "f32")])
def test_merge_states_two_level(S, N, H, dt):
    """Few positions with many states, merged over two levels through an fp32
    workspace; checked against the oracle's N-state merge."""
    _say("two-level merge", S, N, H, dt)
    c = inputs.merge_states_case(150 + N, S=S, N=N, H=H, D=128, dtype=dt, s_lo=-40, s_hi=40)
    need = mi.merge_states_workspace_bytes(S, N, H, 128)
    ws = (torch.full((max(need // 4, 1),), float("nan"), dtype=torch.float32, device="cuda")
          if need else None)
    vo, so = mi.merge_states_two_level(to_device(c["v"], dt), torch.from_numpy(c["s"]).cuda(),
                                       out_dtype=torch.float16, workspace=ws)
    torch.cuda.synchronize()
    rv, rs = oracle.merge_states(c["v"], c["s"], dt)
    check_values(vo, rv)
    check_lse(so, rs)


def test_merge_states_two_level_streaming_size():
    """The sweep's streaming size: fp32 S=64, N=16384, H=1 (32 slices of 512 states,
    teams of 256 lanes over several batches), every row against the oracle."""
    _say("two-level merge, streaming size")
    S, N = 64, 16384
    c = inputs.merge_states_case(2100 + N, S=S, N=N, H=1, D=128, dtype="f32")
    need = mi.merge_states_workspace_bytes(S, N, 1, 128)
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda")
    vo, so = mi.merge_states_two_level(torch.from_numpy(c["v"]).cuda(),
                                       torch.from_numpy(c["s"]).cuda(),
                                       out_dtype=torch.float16, workspace=ws)
    torch.cuda.synchronize()
    rv, rs = oracle.merge_states(c["v"], c["s"], "f32")
    check_values(vo, rv)
    check_lse(so, rs)


def test_merge_states_varlen_streaming_size():
    """The sweep's streaming size: 65536 sets of U[0..8] fp16 states, H=8 (adaptive
    batches in waves whose rows share one set), every row against the oracle."""
    _say("varlen merge, streaming size")
    indptr = inputs.segment_indptr(2202, 65536, 8)
    total = int(indptr[-1])
    c = inputs.merge_states_case(2203, S=1, N=total, H=8, D=128, dtype="f16")
    v = np.ascontiguousarray(c["v"].reshape(total, 8, 128))
    s = np.ascontiguousarray(c["s"].reshape(total, 8))
    vo = torch.full((65536, 8, 128), float("nan"), dtype=torch.float16, device="cuda")
    so = torch.full((65536, 8), float("nan"), dtype=torch.float32, device="cuda")
    mi.merge_states_varlen(to_device(v, "f16"), torch.from_numpy(s).cuda(),
                           torch.from_numpy(indptr).cuda(), v_out=vo, s_out=so)
    torch.cuda.synchronize()
    rv, rs = oracle.merge_states_varlen(v, s, indptr, "f16")
    check_values(vo, rv)
    check_lse(so, rs)
