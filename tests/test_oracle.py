"""Pins for the CPU oracle: values the pages print, closed forms, invariants,
library special cases and brute force. No GPU is used here.

Every check below is against something other than the oracle's own formulas:
a number a page prints (tests/golden), a closed form, an algebraic invariant,
an independent library routine (numpy's float16 decoder, torch's bfloat16
conversion, torch's float64 scaled-dot-product attention and logsumexp), or a
brute-force enumeration.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
from golden import keyed, rows
from lse_attention_state_amd import inputs

LN2 = math.log(2.0)
NEG_INF = -math.inf


# ----------------------------------------------------------------------------- codecs

def test_f16_codec_matches_numpy_for_every_bit_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode_f16(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_bf16_codec_matches_torch_for_every_bit_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


# ----------------------------------------------------------------------------- helpers

def _f32(*xs):
    return np.array(xs, dtype=np.float32)


def _merge2(va, sa, vb, sb):
    va = np.asarray(va, np.float32).reshape(1, -1)
    vb = np.asarray(vb, np.float32).reshape(1, -1)
    v, s = oracle.merge_state(va, _f32(sa), vb, _f32(sb), "f32")
    return v[0], s[0]


def _tiny_decode(scores, values, page, splits=None, scale=1.0, permute=True):
    """One query with D = 1: q = [1], k_t = score_t, v_t = value_t, so the
    attention scores are exactly ``scale * scores``. Pages are placed at
    permuted physical positions to exercise the page table."""
    n = len(scores)
    n_pages = -(-n // page)
    phys = np.arange(n_pages, dtype=np.int32)[::-1].copy() if permute else np.arange(n_pages, dtype=np.int32)
    k = np.full((n_pages, 1, page, 1), np.nan, np.float32)
    v = np.full((n_pages, 1, page, 1), np.nan, np.float32)
    for t in range(n):
        k[phys[t // page], 0, t % page, 0] = scores[t]
        v[phys[t // page], 0, t % page, 0] = values[t]
    q = np.ones((1, 1, 1), np.float32)
    table = phys.reshape(1, -1)
    ctx = np.array([n], np.int32)
    if splits is None:
        return oracle.attention(q, k, v, table, ctx, scale, "f32", "f32")
    return oracle.split_partials(q, k, v, table, ctx, scale, splits, "f32", "f32")


# ----------------------------------------------------------------------------- worked example

def test_worked_example_partials_and_merge():
    g = keyed("worked_example.txt")
    scores = [float(x) for x in g["scores"]]
    values = [float(x) for x in g["values"]]
    o_part, s_part = _tiny_decode(scores, values, page=2, splits=2)
    for i in range(2):
        assert abs(o_part[0, 0, i, 0] - g["split_o"][i]) <= g["split_o"][i].tol
        assert abs(s_part[0, 0, i] - g["split_s_base2"][i]) <= g["split_s_base2"][i].tol
        assert abs(s_part[0, 0, i] * LN2 - g["split_lse_nat"][i]) <= g["split_lse_nat"][i].tol
    w_a = 2.0 ** (s_part[0, 0, 0] - s_part[0, 0, 1])
    assert abs(w_a - g["weight_A"][0]) <= g["weight_A"][0].tol
    # merging the two partial states
    v, s = _merge2(o_part[0, 0, 0], s_part[0, 0, 0], o_part[0, 0, 1], s_part[0, 0, 1])
    assert abs(v[0] - g["merged_v"][0]) <= g["merged_v"][0].tol
    assert abs(s - g["merged_s_base2"][0]) <= g["merged_s_base2"][0].tol
    assert abs(s * LN2 - g["merged_lse_nat"][0]) <= g["merged_lse_nat"][0].tol
    assert abs(2.0 ** s - g["merged_Z"][0]) <= g["merged_Z"][0].tol
    # the unsplit computation gives the same state
    o, s_un = _tiny_decode(scores, values, page=2)
    assert abs(o[0, 0, 0] - g["merged_v"][0]) <= g["merged_v"][0].tol
    assert abs(s_un[0, 0] - g["merged_s_base2"][0]) <= g["merged_s_base2"][0].tol


def test_worked_example_full_precision_closed_form():
    # The same example in closed form: Z = e^1 + e^2 + e^3 + e^0, v = sum e^x v / Z.
    e = [math.exp(x) for x in (1, 2, 3, 0)]
    Z = sum(e)
    v_ref = sum(w * x for w, x in zip(e, (10, 20, 30, 40))) / Z
    o, s = _tiny_decode([1, 2, 3, 0], [10, 20, 30, 40], page=2)
    assert o[0, 0, 0] == pytest.approx(v_ref, rel=1e-14)
    assert s[0, 0] == pytest.approx(math.log2(Z), rel=1e-14)


# ----------------------------------------------------------------------------- self tests

def test_self_test_equal_states():
    g = keyed("self_tests.txt")
    v, s = _merge2(g["st1_va"], g["st1_sa"][0], g["st1_vb"], g["st1_sb"][0])
    assert list(v) == [float(x) for x in g["st1_v"]]
    assert s == float(g["st1_s"][0])


def test_self_test_natural_to_base2():
    g = keyed("self_tests.txt")
    # a single key whose score is the natural LSE itself
    _, s = _tiny_decode([float(g["st2_lse_nat"][0])], [1.0], page=16)
    assert abs(s[0, 0] - g["st2_s_base2"][0]) <= g["st2_s_base2"][0].tol


def test_shard_weights_for_lse_1_and_0():
    g = keyed("self_tests.txt")
    l1, l0 = (float(x) for x in g["w_lse_nat"])
    v, _ = _merge2([1, 0], l1 / LN2, [0, 1], l0 / LN2)
    for got, want in zip(v, g["w_weights"]):
        assert abs(got - want) <= want.tol


def test_self_test_two_splits_lse_0_and_10():
    g = keyed("self_tests.txt")
    l0, l1 = (float(x) for x in g["st3_lse_nat"])
    v, _ = _merge2(g["st3_same_v"], l0 / LN2, g["st3_same_v"], l1 / LN2)
    assert list(v) == [float(x) for x in g["st3_same_out"]]
    v, _ = _merge2(g["st3_va"], l0 / LN2, g["st3_vb"], l1 / LN2)
    for got, want in zip(v, g["st3_out"]):
        assert abs(got - want) <= want.tol


@pytest.mark.parametrize("bad", [math.inf, math.nan])
def test_sanitised_lse_leaves_first_state_alone(bad):
    g = keyed("self_tests.txt")
    s_first = float(g["inf_lse"][0])
    v, s = _merge2([1.5, -2.0], s_first, [3.0, 4.0], bad)
    assert list(v) == [1.5, -2.0] and s == np.float32(s_first)
    v, s = _merge2([3.0, 4.0], bad, [1.5, -2.0], s_first)
    assert list(v) == [1.5, -2.0] and s == np.float32(s_first)


def test_merge_states_offsets_example():
    g = keyed("self_tests.txt")
    S, N, H = (int(x) for x in g["offsets_shape"])
    pid = int(g["offsets_pid"][0])
    want = [int(x) for x in g["offsets_read"]]
    D = 4
    # Only the flat s offsets the page lists are non-empty; each gets a distinct
    # value and a one-hot v, so the output row for pid shows which offsets it read.
    s = np.full((S, N, H), -np.inf, np.float32)
    v = np.zeros((S, N, H, D), np.float32)
    flat_s = s.reshape(-1)
    flat_v = v.reshape(-1, D)
    for j, off in enumerate(want):
        flat_s[off] = 5.0
        flat_v[off, j] = 1.0
    v_out, s_out = oracle.merge_states(v, s, "f32")
    pos, h = divmod(pid, H)
    assert np.allclose(v_out[pos, h, :3], [1 / 3] * 3, rtol=0, atol=1e-15)
    assert s_out[pos, h] == pytest.approx(5.0 + math.log2(3), abs=1e-15)
    others = [(p, hh) for p in range(S) for hh in range(H) if (p, hh) != (pos, h)]
    for p, hh in others:
        assert s_out[p, hh] == NEG_INF and not v_out[p, hh].any()


# ----------------------------------------------------------------------------- empties & closed forms

def test_empty_merges():
    # empty + empty = empty (no NaN); empty + x = x exactly, even if the empty v is NaN
    v, s = _merge2([0, 0], -np.inf, [0, 0], -np.inf)
    assert s == NEG_INF and list(v) == [0.0, 0.0]
    v, s = _merge2([np.nan, np.nan], -np.inf, [0.25, -7.5], 3.0)
    assert list(v) == [0.25, -7.5] and s == 3.0


def test_identical_states_add_log2_n():
    g = np.random.default_rng(1)
    for N in (1, 2, 3, 7, 64):
        row = g.standard_normal(16).astype(np.float32)
        v = np.broadcast_to(row, (1, N, 1, 16)).copy()
        s = np.full((1, N, 1), 2.75, np.float32)
        vo, so = oracle.merge_states(v, s, "f32")
        assert np.allclose(vo[0, 0], row.astype(np.float64), rtol=1e-15, atol=0)
        assert so[0, 0] == pytest.approx(2.75 + math.log2(N), abs=1e-14)


def test_one_nonempty_among_empties_is_exact():
    g = np.random.default_rng(2)
    v = g.standard_normal((3, 5, 2, 8)).astype(np.float32)
    s = np.full((3, 5, 2), -np.inf, np.float32)
    s[:, 3, :] = g.uniform(-10, 10, (3, 2)).astype(np.float32)
    vo, so = oracle.merge_states(v, s, "f32")
    assert np.array_equal(vo, v[:, 3].astype(np.float64))
    assert np.array_equal(so, s[:, 3].astype(np.float64))


def test_commutative_and_associative():
    g = np.random.default_rng(3)
    D = 32
    vs = [g.standard_normal(D).astype(np.float32) for _ in range(3)]
    ss = [float(x) for x in g.uniform(-5, 30, 3).astype(np.float32)]
    ab = _merge2(vs[0], ss[0], vs[1], ss[1])
    ba = _merge2(vs[1], ss[1], vs[0], ss[0])
    assert np.array_equal(ab[0], ba[0]) and ab[1] == ba[1]
    # associativity: (a+b)+c, a+(b+c) and the 3-state merge agree (intermediates
    # pass through fp32 inputs, hence the fp32-level tolerance)
    v3 = np.stack(vs)[None, :, None, :]
    s3 = np.array(ss, np.float32)[None, :, None]
    vo, so = oracle.merge_states(v3, s3, "f32")
    left = _merge2(*_merge2(vs[0], ss[0], vs[1], ss[1]), vs[2], ss[2])
    right = _merge2(vs[0], ss[0], *_merge2(vs[1], ss[1], vs[2], ss[2]))
    for v, s in (left, right):
        assert np.allclose(v, vo[0, 0], rtol=1e-6, atol=1e-6)
        assert s == pytest.approx(so[0, 0], abs=1e-5)
    # and a permuted 3-state merge is the same state
    vp, sp = oracle.merge_states(v3[:, ::-1].copy(), s3[:, ::-1].copy(), "f32")
    assert np.allclose(vp, vo, rtol=1e-15, atol=1e-15) and sp[0, 0] == pytest.approx(so[0, 0], abs=1e-14)


# ----------------------------------------------------------------------------- split ranges

def test_split_ranges_printed_examples():
    for ctx, page, splits, k, p0, p1, ntok in rows("split_ranges.txt"):
        assert oracle.split_range(ctx, page, splits, k) == (p0, p1)
        t0, t1 = p0 * page, min(p1 * page, ctx)
        assert max(0, t1 - t0) == ntok


@pytest.mark.parametrize("splits", [1, 2, 3, 4, 5, 16, 64])
def test_split_ranges_tile_pages_brute_force(splits):
    page = 16
    for ctx in range(0, 2049):
        num_pages = -(-ctx // page)
        covered = []
        sizes = []
        for k in range(splits):
            p0, p1 = oracle.split_range(ctx, page, splits, k)
            if p1 > p0:
                covered.extend(range(p0, p1))
                sizes.append(p1 - p0)
        # contiguous, ordered, disjoint tiling of all pages
        assert covered == list(range(num_pages))
        # every non-empty split but the last holds the same (maximal) count, the
        # empties come last, and the count is the smallest that fits in `splits`
        if sizes:
            per = sizes[0]
            assert all(x == per for x in sizes[:-1]) and sizes[-1] <= per
            assert per == min(c for c in range(1, num_pages + 1) if c * splits >= num_pages)


# ----------------------------------------------------------------------------- plan

def test_plan_matches_pages_table():
    for B, ctx, Hkv, page, cus, want in rows("plan_table.txt"):
        assert oracle.plan_splits(B, Hkv, [ctx] * B, page, cus) == want


def test_plan_steps_down_for_short_contexts():
    # Reading of "at least several pages per split": a split keeps >= 8 pages.
    # Worked by hand at 256 CUs, Hkv = 8, PAGE = 16:
    #   ctx 1024 -> 64 pages: 64 splits (1 page) -> 16 (4 pages) -> 4 (16 pages): 4
    #   ctx 100  -> 7 pages: 64 -> 16 -> 4 (2 pages) -> 1: 1
    #   ctx 2048 -> 128 pages: 64 (2 pages) -> 16 (8 pages): 16
    #   ctx 0    -> no pages: 1
    assert oracle.plan_splits(1, 8, [1024], 16, 256) == 4
    assert oracle.plan_splits(1, 8, [100], 16, 256) == 1
    assert oracle.plan_splits(1, 8, [2048], 16, 256) == 16
    assert oracle.plan_splits(1, 8, [0], 16, 256) == 1
    # the longest sequence decides: one long sequence keeps the split count up
    assert oracle.plan_splits(2, 8, [100, 32768], 16, 256) == 64


def test_plan_on_mi355x_workloads():
    assert oracle.plan_splits(1, 8, [32768], 16, 256) == 64          # B=1, ctx=32K
    assert oracle.plan_splits(64, 8, [512] * 64, 16, 256) == 1        # cascade suffixes
    ctx = inputs.mixed_ctx_lens(1004, 32)
    assert oracle.plan_splits(32, 8, ctx, 16, 256) == 4               # mixed batch


# ----------------------------------------------------------------------------- decode

def _dense_reference(case):
    """Library special case: torch float64 scaled-dot-product attention and
    logsumexp on the gathered (unpaged) K/V of each sequence."""
    dt = case["dtype"]
    dec = oracle.decode_f16 if dt == "f16" else oracle.decode_bf16
    q = torch.from_numpy(dec(case["q"]))
    k = torch.from_numpy(dec(case["k"]))
    v = torch.from_numpy(dec(case["v"]))
    B, Hq, D = q.shape
    G = Hq // case["Hkv"]
    page = case["page"]
    outs, lses = [], []
    for b in range(B):
        n = int(case["ctx_lens"][b])
        if n == 0:
            outs.append(torch.zeros(Hq, D, dtype=torch.float64))
            lses.append(torch.full((Hq,), -math.inf, dtype=torch.float64))
            continue
        t = torch.arange(n)
        phys = torch.from_numpy(case["page_table"][b]).long()[t // page]
        kb = k[phys, :, t % page, :].permute(1, 0, 2)       # [Hkv, n, D]
        vb = v[phys, :, t % page, :].permute(1, 0, 2)
        qb = q[b].unsqueeze(1)                              # [Hq, 1, D]
        o = torch.nn.functional.scaled_dot_product_attention(
            qb.unsqueeze(0), kb.unsqueeze(0), vb.unsqueeze(0), scale=case["sm_scale"],
            enable_gqa=True)[0, :, 0, :]
        kk = kb.repeat_interleave(G, dim=0)
        x = (qb @ kk.transpose(1, 2))[:, 0, :] * case["sm_scale"]
        outs.append(o)
        lses.append(torch.logsumexp(x, dim=-1) / LN2)
    return torch.stack(outs).numpy(), torch.stack(lses).numpy()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("Hq,Hkv", [(4, 1), (8, 2), (6, 3)])
def test_attention_matches_torch_sdpa(dtype, Hq, Hkv):
    ctx = np.array([1, 16, 17, 37, 100, 0, 250], np.int32)
    case = inputs.paged_kv_case(7, ctx, Hq, Hkv, 32, 16, dtype=dtype, extra_pages=3)
    o, s = oracle.attention(case["q"], case["k"], case["v"], case["page_table"], case["ctx_lens"],
                            case["sm_scale"], dtype, dtype)
    o_ref, s_ref = _dense_reference(case)
    assert np.allclose(o, o_ref, rtol=1e-12, atol=1e-12)
    finite = np.isfinite(s_ref)
    assert np.array_equal(finite, np.isfinite(s))
    assert np.allclose(s[finite], s_ref[finite], rtol=0, atol=1e-12)
    assert np.all(s[~finite] == -np.inf) and not np.isnan(o).any()


def test_zero_query_gives_mean_and_log2_count():
    ctx = np.array([37, 100, 1, 64], np.int32)
    case = inputs.paged_kv_case(11, ctx, 4, 2, 16, 16, dtype="f16")
    case["q"][:] = 0
    o, s = oracle.attention(case["q"], case["k"], case["v"], case["page_table"], ctx,
                            case["sm_scale"], "f16", "f16")
    vdec = oracle.decode_f16(case["v"])
    for b, n in enumerate(ctx):
        t = np.arange(n)
        rows_ = vdec[case["page_table"][b][t // 16], :, t % 16, :]     # [n, Hkv, D]
        mean = rows_.mean(axis=0)
        for h in range(4):
            assert np.allclose(o[b, h], mean[h // 2], rtol=1e-13, atol=1e-13)
            assert s[b, h] == pytest.approx(math.log2(n), abs=1e-13)
    # per split: mean over the split's tokens, log2 of its token count, (0, -inf) if empty
    o_p, s_p = oracle.split_partials(case["q"], case["k"], case["v"], case["page_table"], ctx,
                                     case["sm_scale"], 4, "f16", "f16")
    for b, n in enumerate(ctx):
        for k in range(4):
            p0, p1 = oracle.split_range(int(n), 16, 4, k)
            t0, t1 = p0 * 16, min(p1 * 16, int(n))
            if p1 <= p0:
                assert s_p[b, 0, k] == -np.inf and not o_p[b, :, k].any()
                continue
            assert s_p[b, 1, k] == pytest.approx(math.log2(t1 - t0), abs=1e-13)


@pytest.mark.parametrize("splits", [1, 2, 4, 16, 64])
def test_merging_all_splits_equals_unsplit(splits):
    ctx = np.array([1, 16, 17, 37, 300, 1000, 0], np.int32)
    case = inputs.paged_kv_case(21, ctx, 8, 2, 32, 16, dtype="bf16")
    args = (case["q"], case["k"], case["v"], case["page_table"], ctx, case["sm_scale"])
    o, s = oracle.attention(*args, "bf16", "bf16")
    o_p, s_p = oracle.split_partials(*args, splits, "bf16", "bf16")
    B, Hq, D = o.shape
    vo, so = oracle.merge_states(o_p.reshape(B * Hq, splits, 1, D).astype(np.float32),
                                 s_p.reshape(B * Hq, splits, 1).astype(np.float32), "f32")
    # partials were rounded to fp32 for the merge input: compare at fp32 resolution
    assert np.allclose(vo.reshape(B, Hq, D), o, rtol=1e-6, atol=1e-6)
    fin = np.isfinite(s)
    assert np.allclose(so.reshape(B, Hq)[fin], s[fin], rtol=0, atol=1e-6)
    assert np.all(so.reshape(B, Hq)[~fin] == -np.inf)


def test_brute_force_every_merge_order_tiny():
    # ctx <= 64 tokens, 4 splits: merging the partials in every order, pairwise,
    # reproduces the unsplit state.
    for n in (1, 5, 16, 33, 64):
        ctx = np.array([n], np.int32)
        case = inputs.paged_kv_case(100 + n, ctx, 2, 1, 8, 16, dtype="f16")
        args = (case["q"], case["k"], case["v"], case["page_table"], ctx, case["sm_scale"])
        o, s = oracle.attention(*args, "f16", "f16")
        o_p, s_p = oracle.split_partials(*args, 4, "f16", "f16")
        for perm in itertools.permutations(range(4)):
            acc_v = np.zeros(8, np.float32)
            acc_s = -np.inf
            for k in perm:
                acc_v, acc_s = _merge2(acc_v, acc_s, o_p[0, 0, k].astype(np.float32), s_p[0, 0, k])
                acc_v = acc_v.astype(np.float32)
            assert np.allclose(acc_v, o[0, 0], rtol=1e-5, atol=1e-6)
            assert acc_s == pytest.approx(s[0, 0], abs=1e-5)


def test_nan_tail_slots_are_never_read():
    ctx = np.array([5, 21, 37], np.int32)
    case = inputs.paged_kv_case(5, ctx, 4, 1, 16, 16, dtype="f16")
    o, s = oracle.attention(case["q"], case["k"], case["v"], case["page_table"], ctx,
                            case["sm_scale"], "f16", "f16")
    assert not np.isnan(o).any() and not np.isnan(s).any()
