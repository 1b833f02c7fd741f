"""Pins for the oracle functions behind the next rows of the path: the
attention-sink merge, merge_state with a per-position mask, the
variable-length merge, per-sequence split counts and their partials. No GPU.

Each check is against something other than the oracle's own formulas: a value
a page prints (tests/golden), a closed form written another way (the sink's
sigmoid / log1p form in natural units), the already-pinned two-state and
N-state merges, brute force over the planner's defining conditions, or the
q = 0 closed form (mean of V, log2 of the token count).
"""
import math

import numpy as np
import pytest

import oracle
from golden import keyed
from lse_attention_state_amd import inputs

LN2 = math.log(2.0)


# ----------------------------------------------------------------------------- attention sink

def _states(seed, S, H, D, lo=-20.0, hi=40.0):
    g = np.random.default_rng(seed)
    v = g.standard_normal((S, H, D)).astype(np.float32)
    s = g.uniform(lo, hi, (S, H)).astype(np.float32)
    return v, s


def test_sink_minus_inf_nan_and_plus_inf_leave_the_state_alone():
    v, s = _states(1, 4, 3, 8)
    for bad in (-np.inf, np.nan, np.inf):
        vo, so = oracle.merge_sink(v, s, np.full(3, bad, np.float32), "f32")
        assert np.array_equal(vo, v.astype(np.float64))
        assert np.array_equal(so, s.astype(np.float64))


def test_sink_matches_the_rescale_form_in_natural_units():
    # The page's form: o' = o * e^L / (e^L + e^sink), L' = log(e^L + e^sink),
    # written here as a sigmoid and a log1p in natural units.
    v, s = _states(2, 16, 4, 8, lo=-10, hi=10)
    sink = np.random.default_rng(3).uniform(-12, 12, 4).astype(np.float32)
    vo, so = oracle.merge_sink(v, s, sink, "f32")
    L = s.astype(np.float64) * LN2
    d = sink.astype(np.float64)[None, :] - L
    scale = 1.0 / (1.0 + np.exp(d))
    L2 = L + np.log1p(np.exp(d))
    assert np.allclose(vo, v * scale[..., None], rtol=1e-12, atol=1e-15)
    assert np.allclose(so, L2 / LN2, rtol=0, atol=1e-12)


def test_sink_printed_shard_weight():
    # "FlashAttention's empty-row LSE", section 0.2: LSEs 1 and 0 (natural)
    # carry weights 0.731 and 0.269; a sink at 0 against a state at L = 1
    # leaves the state 0.731 of its weight.
    g = keyed("self_tests.txt")
    (l1, l0), (w1, w0) = g["w_lse_nat"], g["w_weights"]
    v = np.ones((1, 1, 2), np.float32)
    s = np.array([[l1 / LN2]], np.float32)
    vo, so = oracle.merge_sink(v, s, np.array([l0], np.float32), "f32")
    assert vo[0, 0, 0] == pytest.approx(w1, abs=w1.tol)
    assert 1.0 - vo[0, 0, 0] == pytest.approx(w0, abs=w0.tol)


def test_sink_on_an_empty_state_gives_the_sink_lse():
    v = np.zeros((2, 2, 8), np.float32)
    s = np.full((2, 2), -np.inf, np.float32)
    s[1, 1] = np.nan  # sanitised to empty as well
    sink = np.array([0.5, -3.0], np.float32)
    vo, so = oracle.merge_sink(v, s, sink, "f32")
    assert not vo.any()
    assert np.array_equal(so, np.broadcast_to(sink.astype(np.float64) / LN2, (2, 2)))


def test_sink_equal_weight_halves_v_and_adds_one():
    v, s = _states(4, 3, 1, 16, lo=-5, hi=5)
    for i in range(3):
        sink = np.array([float(s[i, 0]) * LN2], np.float32)
        vo, so = oracle.merge_sink(v[i:i + 1], s[i:i + 1], sink, "f32")
        w = 2.0 ** (float(sink[0]) / LN2 - float(s[i, 0]))   # 1 up to the fp32 rounding of sink
        assert w == pytest.approx(1.0, abs=1e-6)
        assert np.allclose(vo[0, 0], v[i, 0].astype(np.float64) / (1.0 + w), rtol=1e-13, atol=0)
        assert so[0, 0] == pytest.approx(float(s[i, 0]) + math.log2(1.0 + w), abs=1e-12)


# ----------------------------------------------------------------------------- masked merge

def test_masked_merge_is_merge_state_where_set_and_a_elsewhere():
    va, sa = _states(5, 6, 3, 8)
    vb, sb = _states(6, 6, 3, 8)
    sa[2, 1] = np.nan  # kept as is where the mask is 0
    full_v, full_s = oracle.merge_state(va, sa, vb, sb, "f32")
    v1, s1 = oracle.merge_state_masked(va, sa, vb, sb, None, "f32")
    assert np.array_equal(v1, full_v) and np.array_equal(s1, full_s)
    v0, s0 = oracle.merge_state_masked(va, sa, vb, sb, np.zeros(6, np.uint8), "f32")
    assert np.array_equal(v0, va.astype(np.float64))
    assert np.array_equal(np.isnan(s0), np.isnan(sa)) and np.array_equal(s0[~np.isnan(s0)], sa[~np.isnan(sa)])
    mask = np.array([1, 0, 1, 1, 0, 0], np.uint8)
    vm, sm = oracle.merge_state_masked(va, sa, vb, sb, mask, "f32")
    on = mask.astype(bool)
    assert np.array_equal(vm[on], full_v[on]) and np.array_equal(sm[on], full_s[on])
    assert np.array_equal(vm[~on], va[~on].astype(np.float64))


# ----------------------------------------------------------------------------- variable-length merge

def test_varlen_with_equal_lengths_is_merge_states():
    case = inputs.merge_states_case(7, S=5, N=4, H=3, D=16, dtype="f16")
    v, s = case["v"], case["s"]                      # [S,N,H,D], [S,N,H]
    ref_v, ref_s = oracle.merge_states(v, s, "f16")
    indptr = np.arange(0, 5 * 4 + 1, 4, dtype=np.int32)
    got_v, got_s = oracle.merge_states_varlen(v.reshape(20, 3, 16), s.reshape(20, 3), indptr, "f16")
    assert np.array_equal(got_v, ref_v) and np.array_equal(got_s, ref_s)


def test_varlen_empty_single_and_permuted_segments():
    g = np.random.default_rng(8)
    v = g.standard_normal((9, 2, 8)).astype(np.float32)
    s = g.uniform(-5, 5, (9, 2)).astype(np.float32)
    s[4, 0] = np.inf      # sanitised: no weight
    indptr = np.array([0, 0, 1, 6, 9], np.int32)
    vo, so = oracle.merge_states_varlen(v, s, indptr, "f32")
    assert not vo[0].any() and np.all(so[0] == -np.inf)              # empty segment
    assert np.array_equal(vo[1], v[0].astype(np.float64)) and np.array_equal(so[1], s[0])
    for seg, (a, b) in ((2, (1, 6)), (3, (6, 9))):                  # = pinned N-state merge
        rv, rs = oracle.merge_states(v[a:b][None].copy(), s[a:b][None].copy(), "f32")
        assert np.array_equal(vo[seg], rv[0]) and np.array_equal(so[seg], rs[0])
    perm = np.array([0, 5, 3, 1, 4, 2, 8, 6, 7])
    vp, sp = oracle.merge_states_varlen(v[perm], s[perm], indptr, "f32")
    assert np.allclose(vp, vo, rtol=1e-14, atol=1e-14) and np.allclose(sp, so, rtol=0, atol=1e-13)


# ----------------------------------------------------------------------------- per-sequence split plan

def _np(ctx, page):
    return [-(-int(c) // page) for c in ctx]


def _items(nps, c, Hkv):
    return Hkv * sum(max(1, -(-n // c)) for n in nps)


@pytest.mark.parametrize("seed", range(12))
def test_varlen_plan_meets_its_defining_conditions(seed):
    # c: the largest pages-per-split (at most the longest sequence, at least 8)
    # whose work items still reach twice the CU count.
    g = np.random.default_rng(seed)
    B = int(g.integers(1, 65))
    Hkv = int(g.choice([1, 2, 8]))
    cus = int(g.choice([64, 170, 256]))
    ctx = g.integers(0, 20000, B).astype(np.int32)
    c, counts = oracle.plan_splits_varlen(B, Hkv, ctx, 16, cus)
    nps = _np(ctx, 16)
    cap = 2 * cus
    if max(nps) <= 8:
        assert c == 8
    else:
        assert 8 <= c <= max(nps)
        assert c == 8 or _items(nps, c, Hkv) >= cap
        assert c == max(nps) or _items(nps, c + 1, Hkv) < cap   # nothing larger qualifies
    assert list(counts) == [max(1, -(-n // c)) for n in nps]


def test_varlen_plan_examples():
    # "L3 hints", section 6 table, first row: one 32K sequence, Hkv = 8 -> the
    # uniform plan's 64 splits of 32 pages.
    c, counts = oracle.plan_splits_varlen(1, 8, np.array([32768]), 16, 256)
    assert (c, list(counts)) == (32, [64])
    c, counts = oracle.plan_splits_varlen(2, 8, np.array([32768, 100]), 16, 256)
    assert (c, list(counts)) == (33, [63, 1])         # the short sequence is not split
    c, counts = oracle.plan_splits_varlen(4, 8, np.array([0, 0, 0, 0]), 16, 256)
    assert c == 8 and list(counts) == [1, 1, 1, 1]
    # third row: B*Hkv = 512 already twice the CUs -> no split.
    c, counts = oracle.plan_splits_varlen(64, 8, np.full(64, 1024), 16, 256)
    assert c == 64 and set(counts) == {1}
    # second row (8 x 4096, 170 CUs as on the page's GPU): 16 splits of 16 pages
    # reach 1024 >= 340 items; the largest such c gives ceil(256/c) = 6 splits.
    c, counts = oracle.plan_splits_varlen(8, 8, np.full(8, 4096), 16, 170)
    assert (c, set(counts)) == (51, {6})
    # empty sequences still cost one work item each (their outputs are written):
    # 299 empty + one of 2048 pages, Hkv = 1, target 512 -> 299 + ceil(2048/c) >= 512
    # holds up to c = 9 (228 splits), not c = 10 (205).
    c, counts = oracle.plan_splits_varlen(300, 1, np.array([0] * 299 + [32768]), 16, 256)
    assert c == 9 and counts[-1] == 228 and set(counts[:-1]) == {1}
    # a batch too small to reach the target bottoms out at 8 pages per split:
    # 100 pages -> 13 splits.
    c, counts = oracle.plan_splits_varlen(1, 1, np.array([1600]), 16, 256)
    assert (c, list(counts)) == (8, [13])
    # equal lengths reduce to the largest c that the uniform rule's target allows
    for B, n in ((1, 2048), (8, 256), (3, 1000)):
        c, counts = oracle.plan_splits_varlen(B, 8, np.full(B, n * 16), 16, 256)
        k = -(-n // c)
        assert B * 8 * k >= 512 or c == 8
        assert B * 8 * -(-n // (c + 1)) < 512 or c == n


# ----------------------------------------------------------------------------- per-sequence partials

def test_varlen_partials_zero_query_closed_form():
    ctx = np.array([37, 1000, 1, 0, 300], np.int32)
    case = inputs.paged_kv_case(12, ctx, 4, 2, 16, 16, dtype="f16")
    case["q"][:] = 0
    counts = np.array([4, 7, 2, 3, 1], np.int32)
    indptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    o, s = oracle.split_partials_varlen(case["q"], case["k"], case["v"], case["page_table"], ctx,
                                        case["sm_scale"], indptr, "f16", "f16")
    vdec = oracle.decode_f16(case["v"])
    for b, n in enumerate(ctx):
        covered = 0
        for k in range(counts[b]):
            p0, p1 = oracle.split_range(int(n), 16, int(counts[b]), k)   # pinned page ranges
            t0, t1 = p0 * 16, min(p1 * 16, int(n))
            i = indptr[b] + k
            if t1 <= t0:
                assert np.all(s[i] == -np.inf) and not o[i].any()
                continue
            t = np.arange(t0, t1)
            mean = vdec[case["page_table"][b][t // 16], :, t % 16, :].mean(axis=0)
            for h in range(4):
                assert np.allclose(o[i, h], mean[h // 2], rtol=1e-13, atol=1e-13)
                assert s[i, h] == pytest.approx(math.log2(t1 - t0), abs=1e-13)
            covered += t1 - t0
        assert covered == n


def test_varlen_partials_with_uniform_counts_are_the_uniform_partials():
    ctx = np.array([37, 1000, 1, 300], np.int32)
    case = inputs.paged_kv_case(14, ctx, 4, 2, 16, 16, dtype="bf16")
    args = (case["q"], case["k"], case["v"], case["page_table"], ctx, case["sm_scale"])
    ou, su = oracle.split_partials(*args, 4, "bf16", "bf16")         # [B, Hq, 4, D]
    indptr = np.arange(0, 17, 4, dtype=np.int32)
    ov, sv = oracle.split_partials_varlen(*args, indptr, "bf16", "bf16")
    assert np.array_equal(ov.reshape(4, 4, 4, 16).transpose(0, 2, 1, 3), ou)
    assert np.array_equal(sv.reshape(4, 4, 4).transpose(0, 2, 1), su)


def test_varlen_partials_merge_to_unsplit_attention():
    ctx = inputs.mixed_ctx_lens(13, 12, hi=3000)
    case = inputs.paged_kv_case(13, ctx, 8, 2, 32, 16, dtype="bf16")
    args = (case["q"], case["k"], case["v"], case["page_table"], ctx, case["sm_scale"])
    c, counts = oracle.plan_splits_varlen(12, 2, ctx, 16, 64)
    indptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    assert counts.max() > 1 and counts.min() == 1
    op, sp = oracle.split_partials_varlen(*args, indptr, "bf16", "bf16")
    mo, ms = oracle.merge_states_varlen(op.astype(np.float32), sp.astype(np.float32), indptr, "f32")
    o, s = oracle.attention(*args, "bf16", "bf16")
    assert np.allclose(mo, o, rtol=1e-5, atol=1e-6)
    assert np.allclose(ms, s, rtol=0, atol=1e-5)
