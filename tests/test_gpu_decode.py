"""GPU parity of split-KV paged decode (pass 1 partials and the combine) against
the fp64 oracle, through the C ABI.

Workloads: B=1, ctx=32768, Hq=32, Hkv=8, D=128, PAGE=16, 64 splits, fp16, page
table a random permutation (checked in full); the mixed batch B=32 with
ctx ~ U[1, 8192] including short sequences that leave empty splits, split count
from the planner (checked in full); and small ragged cases over group sizes,
split counts and both 16-bit dtypes. Unused tail slots hold NaN throughout.
"""
import numpy as np
import pytest
import torch

import lse_attention_state_amd as mi
import oracle
from lse_attention_state_amd import inputs
from parity import check_lse, check_values, host64, to_device

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _dev(case):
    dt = case["dtype"]
    return (to_device(case["q"], dt), to_device(case["k"], dt), to_device(case["v"], dt),
            torch.from_numpy(case["page_table"]).cuda(), torch.from_numpy(case["ctx_lens"]).cuda())


def _decode(case, splits, out_dtype=None):
    q, k, v, pt, ctx = _dev(case)
    B, Hq, D = q.shape
    nan = float("nan")
    o_part = torch.full((B, Hq, splits, D), nan, dtype=torch.float32, device="cuda")
    lse_part = torch.full((B, Hq, splits), nan, dtype=torch.float32, device="cuda")
    odt = out_dtype or q.dtype
    out = torch.full((B, Hq, D), nan, dtype=odt, device="cuda")
    lse = torch.full((B, Hq), nan, dtype=torch.float32, device="cuda")
    mi.split_kv_decode(q, k, v, pt, ctx, splits, case["sm_scale"], o_part=o_part,
                       lse_part=lse_part, out=out, lse=lse)
    torch.cuda.synchronize()
    return out, lse, o_part, lse_part


def _oracle(case, splits):
    args = (case["q"], case["k"], case["v"], case["page_table"], case["ctx_lens"], case["sm_scale"])
    o, s = oracle.attention(*args, case["dtype"], case["dtype"])
    op, sp = oracle.split_partials(*args, splits, case["dtype"], case["dtype"])
    return o, s, op, sp


def _check_all(case, splits, out_dtype=None):
    out, lse, o_part, lse_part = _decode(case, splits, out_dtype)
    o, s, op, sp = _oracle(case, splits)
    st = check_values(o_part, op, "o_part")
    check_lse(lse_part, sp, "lse_part")
    st2 = check_values(out, o, "o")
    check_lse(lse, s, "lse")
    return st, st2


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("Hq,Hkv", [(4, 1), (8, 2), (32, 8), (8, 8), (16, 2)])
@pytest.mark.parametrize("splits", [1, 3, 4, 16, 64])
def test_decode_small_ragged(dtype, Hq, Hkv, splits):
    _say("decode small", dtype, Hq, Hkv, splits)
    ctx = np.array([1, 16, 17, 37, 100, 0, 250, 1000, 129], np.int32)
    case = inputs.paged_kv_case(300 + Hq + splits, ctx, Hq, Hkv, 128, 16, dtype=dtype,
                                extra_pages=5)
    _check_all(case, splits)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_decode_output_dtypes(out_dtype):
    _say("decode out dtype", out_dtype)
    ctx = np.array([33, 700], np.int32)
    case = inputs.paged_kv_case(41, ctx, 8, 2, 128, 16, dtype="f16")
    _check_all(case, 4, out_dtype)


def test_decode_long_context_b1_64_splits():
    """B=1, ctx=32768, Hq=32, Hkv=8, D=128, PAGE=16, 64 splits, fp16: all outputs."""
    _say("decode B=1 ctx=32768 64 splits")
    ctx = np.array([32768], np.int32)
    case = inputs.paged_kv_case(1003, ctx, 32, 8, 128, 16, dtype="f16")
    assert sorted(case["page_table"][0].tolist()) == list(range(2048))
    st = _check_all(case, 64)
    _say("stats", st)


def test_decode_mixed_batch_planned_splits():
    """B=32, ctx ~ U[1,8192] with forced short sequences; splits from the planner."""
    _say("decode mixed batch")
    ctx = inputs.mixed_ctx_lens(1004, 32)
    case = inputs.paged_kv_case(1004, ctx, 32, 8, 128, 16, dtype="f16")
    splits = mi.plan_splits(ctx, 8, 16)
    assert splits == oracle.plan_splits(32, 8, ctx, 16, torch.cuda.get_device_properties(0).multi_processor_count)
    st = _check_all(case, splits)
    _say("splits", splits, "stats", st)
    # the short sequences leave empty splits: exactly (0, -inf)
    _, _, o_part, lse_part = _decode(case, splits)
    for b in range(4):
        for k in range(splits):
            p0, p1 = mi.split_range(int(ctx[b]), 16, splits, k)
            if p1 <= p0:
                assert host64(lse_part)[b, :, k].tolist() == [-np.inf] * 32
                assert not host64(o_part)[b, :, k].any()


def test_decode_zero_context_and_bad_page_ids():
    """ctx = 0 gives (0, -inf); a negative ctx counts as 0; a page id outside the
    pool contributes no tokens (here the last page, so the expected state is the
    attention over the pages before it)."""
    _say("decode ctx=0 / bad page ids")
    ctx = np.array([0, 48, 48, 48], np.int32)
    case = inputs.paged_kv_case(51, ctx, 8, 2, 128, 16, dtype="f16", extra_pages=2)
    P = case["k"].shape[0]
    bad = case.copy()
    bad["page_table"] = case["page_table"].copy()
    bad["ctx_lens"] = case["ctx_lens"].copy()
    bad["page_table"][1, 2] = -1
    bad["page_table"][2, 2] = P
    bad["page_table"][3, 2] = P + 1000
    bad["ctx_lens"][0] = -5
    out, lse, _, _ = _decode(bad, 4)
    ref = case.copy()
    ref["ctx_lens"] = np.array([0, 32, 32, 32], np.int32)
    o, s, _, _ = _oracle(ref, 4)
    check_values(out, o)
    check_lse(lse, s)


def test_decode_is_deterministic():
    _say("decode determinism")
    ctx = np.array([4000, 77, 1], np.int32)
    case = inputs.paged_kv_case(61, ctx, 32, 8, 128, 16, dtype="bf16")
    a = _decode(case, 16)
    b = _decode(case, 16)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int8), y.view(torch.int8))


def test_split_count_invariance():
    """Merging all splits equals the unsplit result, for every split count."""
    _say("decode split invariance")
    ctx = np.array([3000, 17], np.int32)
    case = inputs.paged_kv_case(71, ctx, 8, 2, 128, 16, dtype="f16")
    o, s, _, _ = _oracle(case, 1)
    for splits in (1, 2, 4, 8, 16, 64, 200):
        out, lse, _, _ = _decode(case, splits, torch.float32)
        check_values(out, o)
        check_lse(lse, s)


# ----------------------------------------------------------------------------- single launch

def _decode_fused(case, splits, out_dtype=None, counters=None):
    q, k, v, pt, ctx = _dev(case)
    B, Hq, D = q.shape
    Hkv = case["Hkv"]
    nan = float("nan")
    if counters is None:
        counters = torch.zeros((B, Hkv), dtype=torch.int32, device="cuda")
    o_part = torch.full((B, Hq, splits, D), nan, dtype=torch.float32, device="cuda")
    lse_part = torch.full((B, Hq, splits), nan, dtype=torch.float32, device="cuda")
    odt = out_dtype or q.dtype
    out = torch.full((B, Hq, D), nan, dtype=odt, device="cuda")
    lse = torch.full((B, Hq), nan, dtype=torch.float32, device="cuda")
    mi.split_kv_decode_fused(q, k, v, pt, ctx, splits, case["sm_scale"], counters=counters,
                             o_part=o_part, lse_part=lse_part, out=out, lse=lse)
    torch.cuda.synchronize()
    assert int(counters.abs().sum()) == 0, "counters must be left at zero"
    return out, lse, o_part, lse_part


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("Hq,Hkv", [(4, 1), (32, 8), (16, 2), (8, 8)])
@pytest.mark.parametrize("splits", [1, 4, 64, 100])
def test_fused_decode_small_ragged(dtype, Hq, Hkv, splits):
    _say("fused decode small", dtype, Hq, Hkv, splits)
    ctx = np.array([1, 16, 17, 37, 100, 0, 250, 1000, 129], np.int32)
    case = inputs.paged_kv_case(400 + Hq + splits, ctx, Hq, Hkv, 128, 16, dtype=dtype,
                                extra_pages=5)
    out, lse, o_part, lse_part = _decode_fused(case, splits)
    o, s, op, sp = _oracle(case, splits)
    check_values(o_part, op, "o_part")
    check_lse(lse_part, sp, "lse_part")
    check_values(out, o, "o")
    check_lse(lse, s, "lse")


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_fused_decode_output_dtypes(out_dtype):
    _say("fused decode out dtype", out_dtype)
    ctx = np.array([33, 700, 4], np.int32)
    case = inputs.paged_kv_case(43, ctx, 8, 2, 128, 16, dtype="f16")
    out, lse, _, _ = _decode_fused(case, 4, out_dtype)
    o, s, _, _ = _oracle(case, 4)
    check_values(out, o)
    check_lse(lse, s)


def test_fused_decode_long_context_and_mixed_batch():
    """The B=1 ctx=32768 64-split case and the mixed batch through the single
    launch; repeated calls reuse the counters and give the same bits."""
    _say("fused decode long + mixed")
    ctx = np.array([32768], np.int32)
    case = inputs.paged_kv_case(1003, ctx, 32, 8, 128, 16, dtype="f16")
    counters = torch.zeros((1, 8), dtype=torch.int32, device="cuda")
    out1, lse1, _, _ = _decode_fused(case, 64, counters=counters)
    out2, lse2, _, _ = _decode_fused(case, 64, counters=counters)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse1.view(torch.int32), lse2.view(torch.int32))
    o, s, _, _ = _oracle(case, 64)
    check_values(out1, o)
    check_lse(lse1, s)
    ctx = inputs.mixed_ctx_lens(1004, 32)
    case = inputs.paged_kv_case(1004, ctx, 32, 8, 128, 16, dtype="f16")
    splits = mi.plan_splits(ctx, 8, 16)
    out, lse, _, _ = _decode_fused(case, splits)
    o, s, _, _ = _oracle(case, splits)
    check_values(out, o)
    check_lse(lse, s)


def test_fused_matches_two_launch_decode():
    _say("fused vs two-launch")
    ctx = np.array([5000, 3, 64, 999], np.int32)
    case = inputs.paged_kv_case(81, ctx, 32, 8, 128, 16, dtype="bf16")
    a = _decode(case, 16, torch.float32)
    b = _decode_fused(case, 16, torch.float32)
    # identical pass 1; the two combines differ only in summation order
    assert torch.equal(a[2].view(torch.int32), b[2].view(torch.int32))
    assert torch.equal(a[3].view(torch.int32), b[3].view(torch.int32))
    assert torch.allclose(a[0], b[0], rtol=1e-5, atol=1e-6)
    assert torch.allclose(a[1], b[1], rtol=0, atol=1e-5)


@pytest.mark.parametrize("fused", [True, False])
def test_decode_maximum_split_count(fused):
    """1024 splits (the largest supported): a 16385-token sequence gets one or
    two pages per split and empty splits at the end; a short one is almost all
    empty splits. Partials and outputs checked in full."""
    _say("decode 1024 splits", fused)
    ctx = np.array([16385, 33], np.int32)
    case = inputs.paged_kv_case(61, ctx, 8, 2, 128, 16, dtype="bf16")
    if fused:
        out, lse, o_part, lse_part = _decode_fused(case, 1024)
    else:
        out, lse, o_part, lse_part = _decode(case, 1024)
    o, s, op, sp = _oracle(case, 1024)
    check_values(o_part, op, "o_part")
    check_lse(lse_part, sp, "lse_part")
    check_values(out, o, "o")
    check_lse(lse, s, "lse")


@pytest.mark.parametrize("splits", [100, 500])
def test_fused_decode_many_splits_single_launch(splits):
    """Few work items but many splits (B=1, Hkv=1, Hq=4): the single launch is
    used and its last workgroup merges more than 64 splits per row, in several
    passes."""
    _say("fused decode many splits, one launch", splits)
    ctx = np.array([16000], np.int32)
    case = inputs.paged_kv_case(70 + splits, ctx, 4, 1, 128, 16, dtype="f16")
    out, lse, o_part, lse_part = _decode_fused(case, splits)
    o, s, op, sp = _oracle(case, splits)
    check_values(o_part, op, "o_part")
    check_lse(lse_part, sp, "lse_part")
    check_values(out, o, "o")
    check_lse(lse, s, "lse")


_SWEEP_CACHE = {}


def _sweep_case(name):
    """The L3 page's 8 x 4096 and 64 x 1024 workloads (Hq=32, Hkv=8, fp16,
    random page permutation), as the split sweep times them."""
    if name not in _SWEEP_CACHE:
        B, ctx_len = {"8x4096": (8, 4096), "64x1024": (64, 1024)}[name]
        ctx = np.full(B, ctx_len, np.int32)
        case = inputs.paged_kv_case(2000 + B, ctx, 32, 8, 128, 16, dtype="f16")
        args = (case["q"], case["k"], case["v"], case["page_table"], case["ctx_lens"],
                case["sm_scale"])
        _SWEEP_CACHE[name] = (case, oracle.attention(*args, "f16", "f16"))
    return _SWEEP_CACHE[name]


@pytest.mark.parametrize("name", ["8x4096", "64x1024"])
@pytest.mark.parametrize("splits", [1, 4, 16, 64])
def test_decode_sweep_workloads(name, splits):
    """The split sweep's own workloads at every split count it times, in both
    launch forms: partials in full against the oracle's per-split partials,
    outputs in full against unsplit attention."""
    _say("decode sweep workload", name, splits)
    case, (o, s) = _sweep_case(name)
    args = (case["q"], case["k"], case["v"], case["page_table"], case["ctx_lens"], case["sm_scale"])
    op, sp = oracle.split_partials(*args, splits, "f16", "f16")
    for fused in (False, True):
        out, lse, o_part, lse_part = (_decode_fused if fused else _decode)(case, splits)
        check_values(o_part, op, "o_part")
        check_lse(lse_part, sp, "lse_part")
        check_values(out, o, "o")
        check_lse(lse, s, "lse")
