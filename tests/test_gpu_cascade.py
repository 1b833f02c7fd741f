"""GPU parity of the cascade (shared-prefix) path against the fp64 oracle.

Workload: 64 requests share an 8192-token prefix and each has its own
512-token suffix, Hq=32, Hkv=8, D=128, PAGE=16, bf16, one shuffled page pool.
The prefix level runs on the matrix cores, the suffixes through split-KV
decode, and merge_state joins the levels; the result must equal unsplit
attention over prefix + suffix. Smaller cases cover ragged prefix lengths,
row counts that leave a partial row block, fp16, and the empty prefix.
"""
import numpy as np
import pytest
import torch

import lse_attention_state_amd as mi
import oracle
from lse_attention_state_amd import inputs
from parity import check_lse, check_values, to_device

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _prefix_oracle(case, prefix_len):
    R = case["R"]
    n_pre = -(-prefix_len // case["page"])
    table = np.ascontiguousarray(np.broadcast_to(case["prefix_pages"][:n_pre], (R, n_pre)))
    if n_pre == 0:
        table = np.zeros((R, 1), np.int32)
    lens = np.full(R, prefix_len, np.int32)
    return oracle.attention(case["q"], case["k"], case["v"], table, lens, case["sm_scale"],
                            case["dtype"], case["dtype"])


def _dev(case):
    dt = case["dtype"]
    return to_device(case["q"], dt), to_device(case["k"], dt), to_device(case["v"], dt)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("R,Hq,Hkv,prefix_len", [(3, 8, 2, 100), (16, 32, 8, 1024),
                                                 (5, 4, 1, 37), (20, 16, 2, 530),
                                                 (7, 8, 8, 16)])
def test_prefix_attention_small(dtype, R, Hq, Hkv, prefix_len):
    _say("prefix small", dtype, R, Hq, Hkv, prefix_len)
    case = inputs.cascade_case(900 + R + prefix_len, R=R, prefix_len=-(-prefix_len // 16) * 16,
                               suffix_len=16, Hq=Hq, Hkv=Hkv, dtype=dtype)
    q, k, v = _dev(case)
    pages = torch.from_numpy(case["prefix_pages"]).cuda()
    v_out = torch.full((R, Hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    s_out = torch.full((R, Hq), float("nan"), dtype=torch.float32, device="cuda")
    mi.prefix_attention(q, k, v, pages, prefix_len, case["sm_scale"], v_out=v_out, s_out=s_out)
    torch.cuda.synchronize()
    o, s = _prefix_oracle(case, prefix_len)
    check_values(v_out, o)
    check_lse(s_out, s)


def test_prefix_attention_empty_prefix():
    _say("prefix empty")
    case = inputs.cascade_case(5, R=4, prefix_len=16, suffix_len=16, Hq=8, Hkv=2, dtype="bf16")
    q, k, v = _dev(case)
    pages = torch.from_numpy(case["prefix_pages"]).cuda()
    vo, so = mi.prefix_attention(q, k, v, pages, 0, case["sm_scale"])
    torch.cuda.synchronize()
    assert torch.all(vo == 0) and torch.all(so == float("-inf"))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("R,Hq,Hkv,n_full,tail", [(5, 8, 2, 40, 7), (20, 16, 2, 300, 5)])
def test_prefix_attention_absent_pages_and_nan_tail(dtype, R, Hq, Hkv, n_full, tail):
    """Prefix page ids outside [0, pages) contribute no tokens, and whatever the
    slots past the prefix end of its last page hold (NaN here, in K and V)
    never reaches the result: equal to the oracle over the prefix with those
    pages left out."""
    _say("prefix absent pages / NaN tail", dtype, R, Hq, Hkv, n_full, tail)
    prefix_len = 16 * n_full + tail
    case = inputs.cascade_case(970 + R + n_full, R=R, prefix_len=16 * (n_full + 1), suffix_len=16,
                               Hq=Hq, Hkv=Hkv, dtype=dtype)
    nan_bits = 0x7FC0 if dtype == "bf16" else 0x7E00
    last = case["prefix_pages"][n_full]
    case["k"][last, :, tail:, :] = nan_bits
    case["v"][last, :, tail:, :] = nan_bits
    P = case["k"].shape[0]
    absent = [3, n_full // 2]
    pages_dev = case["prefix_pages"].copy()
    pages_dev[absent[0]] = -1
    pages_dev[absent[1]] = P
    keep = np.array([i for i in range(n_full + 1) if i not in absent], np.int32)
    q, k, v = _dev(case)
    v_out = torch.full((R, Hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    s_out = torch.full((R, Hq), float("nan"), dtype=torch.float32, device="cuda")
    mi.prefix_attention(q, k, v, torch.from_numpy(pages_dev).cuda(), prefix_len, case["sm_scale"],
                        v_out=v_out, s_out=s_out)
    torch.cuda.synchronize()
    table = np.ascontiguousarray(np.broadcast_to(case["prefix_pages"][keep], (R, len(keep))))
    lens = np.full(R, prefix_len - 16 * len(absent), np.int32)
    o, s = oracle.attention(case["q"], case["k"], case["v"], table, lens, case["sm_scale"],
                            dtype, dtype)
    check_values(v_out, o)
    check_lse(s_out, s)


def test_cascade_64_requests_8k_prefix_512_suffix():
    _say("cascade full")
    case = inputs.cascade_case(1005)
    q, k, v = _dev(case)
    pages = torch.from_numpy(case["prefix_pages"]).cuda()
    st = torch.from_numpy(case["suffix_table"]).cuda()
    sl = torch.from_numpy(case["suffix_lens"]).cuda()
    splits = mi.plan_splits(case["suffix_lens"], 8, 16)
    o, lse, (vp, sp), (vs, ss) = mi.cascade_decode(q, k, v, pages, case["prefix_len"], st, sl,
                                                   case["sm_scale"], suffix_splits=splits)
    torch.cuda.synchronize()
    # the final result against unsplit attention over prefix + suffix
    ro, rs = oracle.attention(case["q"], case["k"], case["v"], case["full_table"],
                              case["full_lens"], case["sm_scale"], "bf16", "bf16")
    stats = check_values(o, ro)
    check_lse(lse, rs)
    # each level against its own definition
    po, ps = _prefix_oracle(case, case["prefix_len"])
    check_values(vp, po, "prefix v")
    check_lse(sp, ps, "prefix s")
    so_, ss_ = oracle.attention(case["q"], case["k"], case["v"], case["suffix_table"],
                                case["suffix_lens"], case["sm_scale"], "bf16", "bf16")
    check_values(vs, so_, "suffix v")
    check_lse(ss, ss_, "suffix s")
    _say("cascade stats", stats, "suffix splits", splits)


def _fused(case, prefix_len, suffix_lens, splits, out_dtype=None):
    q, k, v = _dev(case)
    pages = torch.from_numpy(case["prefix_pages"]).cuda()
    st = torch.from_numpy(case["suffix_table"]).cuda()
    sl = torch.from_numpy(np.ascontiguousarray(suffix_lens, np.int32)).cuda()
    R, Hq, Hkv = case["R"], case["Hq"], case["Hkv"]
    nan = float("nan")
    out = torch.full((R, Hq, 128), nan, dtype=out_dtype or q.dtype, device="cuda")
    lse = torch.full((R, Hq), nan, dtype=torch.float32, device="cuda")
    counters = torch.zeros((R, Hkv), dtype=torch.int32, device="cuda")
    mi.cascade_decode_fused(q, k, v, pages, prefix_len, st, sl, case["sm_scale"],
                            suffix_splits=splits, counters=counters, out=out, lse=lse)
    torch.cuda.synchronize()
    assert not counters.any(), "counters must be left zero"
    return out, lse


@pytest.mark.parametrize("splits", [1, 4])
def test_cascade_decode_fused_64_requests(splits):
    """64 requests x (8192 shared + 512 own), two launches: equals unsplit
    attention over prefix + suffix."""
    _say("cascade fused full", splits)
    case = inputs.cascade_case(1005)
    o, lse = _fused(case, case["prefix_len"], case["suffix_lens"], splits)
    ro, rs = oracle.attention(case["q"], case["k"], case["v"], case["full_table"],
                              case["full_lens"], case["sm_scale"], "bf16", "bf16")
    stats = check_values(o, ro)
    check_lse(lse, rs)
    _say("stats", stats)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("R,Hq,Hkv,prefix_len,splits", [(3, 8, 2, 100, 1), (5, 4, 1, 37, 3),
                                                        (20, 16, 2, 530, 4), (7, 8, 8, 0, 2),
                                                        (16, 32, 8, 1024, 1)])
def test_cascade_decode_fused_ragged(dtype, R, Hq, Hkv, prefix_len, splits):
    """Ragged prefix lengths (including none) and per-request suffix lengths
    (including 0): the result is the merge of the prefix-only and suffix-only
    oracle states (disjoint key sets merge exactly)."""
    _say("cascade fused ragged", dtype, R, Hq, Hkv, prefix_len, splits)
    case = inputs.cascade_case(950 + R + prefix_len, R=R, prefix_len=max(16, -(-prefix_len // 16) * 16),
                               suffix_len=80, Hq=Hq, Hkv=Hkv, dtype=dtype)
    suffix_lens = np.random.default_rng(951 + R).integers(0, 81, size=R).astype(np.int32)
    suffix_lens[0] = 0
    o, lse = _fused(case, prefix_len, suffix_lens, splits, out_dtype=torch.float32)
    po, ps = _prefix_oracle(case, prefix_len)
    so_, ss_ = oracle.attention(case["q"], case["k"], case["v"], case["suffix_table"],
                                suffix_lens, case["sm_scale"], dtype, dtype)
    ro, rs = oracle.merge_state(po.astype(np.float32), ps.astype(np.float32),
                                so_.astype(np.float32), ss_.astype(np.float32), "f32")
    check_values(o, ro)
    check_lse(lse, rs)
