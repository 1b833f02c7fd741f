"""Address arithmetic past 32 bits, and the largest sizes.

The decode and cascade kernels must address K/V pages at any offset of the
cache: the same small seeded case is run on its own caches and again with its
pages moved past 4 GiB of a large cache (page ids shifted), and every output
must be bit-identical, since only the addresses differ. The merge kernels must
index tensors of more than 2^31 elements: a two-state merge and an N-state merge
whose inputs cross that element count, checked against the oracle on the rows on
both sides of it and at the start. And the decode at its largest batch.
"""
import numpy as np
import pytest
import torch

import lse_attention_state_amd as mi
import oracle
from lse_attention_state_amd import inputs
from parity import check_lse, check_values, to_device

pytestmark = pytest.mark.gpu

# 32 KiB per page (8 kv heads x 16 tokens x 128 x 2 bytes): page ids from here
# on start past 4 GiB of the cache.
SHIFT = (1 << 32) // (8 * 16 * 128 * 2) + 3901


def _say(*a):
    print(*a, flush=True)


def _moved(cache: torch.Tensor) -> torch.Tensor:
    big = torch.empty((SHIFT + cache.shape[0],) + tuple(cache.shape[1:]), dtype=cache.dtype,
                      device=cache.device)
    big[SHIFT:] = cache
    return big


def _shift(table: torch.Tensor) -> torch.Tensor:
    return torch.where(table >= 0, table + SHIFT, table)


def _same(a: torch.Tensor, b: torch.Tensor):
    assert a.shape == b.shape and a.dtype == b.dtype
    iv = torch.int16 if a.element_size() == 2 else torch.int32
    assert torch.equal(a.view(iv), b.view(iv))


def _release():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_decode_pages_past_4gib():
    ctx = np.array([1000, 37, 4096, 300], np.int32)
    _say("decode with pages past 4 GiB", ctx.tolist())
    case = inputs.paged_kv_case(1201, ctx, 32, 8, 128, 16, dtype="f16")
    q, k, v = (to_device(case[n], "f16") for n in ("q", "k", "v"))
    pt = torch.from_numpy(case["page_table"]).cuda()
    cl = torch.from_numpy(case["ctx_lens"]).cuda()
    kb, vb, ptb = _moved(k), _moved(v), _shift(pt)
    assert kb.numel() * kb.element_size() > (1 << 32) + (1 << 20)
    sc = case["sm_scale"]
    for splits in (1, 8):
        a = mi.split_kv_decode(q, k, v, pt, cl, splits, sc, return_partials=True)
        b = mi.split_kv_decode(q, kb, vb, ptb, cl, splits, sc, return_partials=True)
        for x, y in zip(a, b):
            _same(x, y)
        a = mi.split_kv_decode_fused(q, k, v, pt, cl, splits, sc)
        b = mi.split_kv_decode_fused(q, kb, vb, ptb, cl, splits, sc)
        for x, y in zip(a, b):
            _same(x, y)
    indptr = mi.plan_splits_varlen(case["ctx_lens"], 8)
    ip = torch.from_numpy(indptr).cuda()
    a = mi.split_kv_decode_varlen(q, k, v, pt, cl, ip, sc)
    b = mi.split_kv_decode_varlen(q, kb, vb, ptb, cl, ip, sc)
    for x, y in zip(a, b):
        _same(x, y)
    o = torch.empty((4, 32, 128), dtype=torch.float16, device="cuda")
    s = torch.empty((4, 32), dtype=torch.float32, device="cuda")
    mi.split_kv_decode_noalloc(q, kb, vb, ptb, cl, 8, sc, o, s)
    ref_o, ref_s = mi.split_kv_decode(q, k, v, pt, cl, 8, sc)
    torch.cuda.synchronize()
    _same(o, ref_o)
    _same(s, ref_s)
    # And the moved case against the oracle.
    ro, rs = oracle.attention(case["q"], case["k"], case["v"], case["page_table"],
                              case["ctx_lens"], sc, "f16", "f16")
    check_values(b[0], ro)
    check_lse(b[1], rs)
    del kb, vb
    _release()


def test_cascade_pages_past_4gib():
    _say("cascade with pages past 4 GiB")
    cas = inputs.cascade_case(1202, R=8, prefix_len=1024, suffix_len=72)
    q, k, v = (to_device(cas[n], "bf16") for n in ("q", "k", "v"))
    pp = torch.from_numpy(cas["prefix_pages"]).cuda()
    st = torch.from_numpy(cas["suffix_table"]).cuda()
    sl = torch.from_numpy(cas["suffix_lens"]).cuda()
    kb, vb = _moved(k), _moved(v)
    a = mi.cascade_decode_fused(q, k, v, pp, cas["prefix_len"], st, sl, cas["sm_scale"])
    b = mi.cascade_decode_fused(q, kb, vb, _shift(pp), cas["prefix_len"], _shift(st), sl,
                                cas["sm_scale"])
    for x, y in zip(a, b):
        _same(x, y)
    ro, rs = oracle.attention(cas["q"], cas["k"], cas["v"], cas["full_table"], cas["full_lens"],
                              cas["sm_scale"], "bf16", "bf16")
    check_values(b[0], ro)
    check_lse(b[1], rs)
    del kb, vb
    _release()


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def test_merge_state_past_2g_elements():
    rows = (1 << 24) + 64          # rows * 128 elements cross 2^31 at row 2^24
    _say("merge_state over", rows, "rows of 128 bf16")
    g = torch.Generator(device="cuda").manual_seed(1203)
    va = torch.randn((rows, 128), generator=g, device="cuda").to(torch.bfloat16)
    vb = torch.randn((rows, 128), generator=g, device="cuda").to(torch.bfloat16)
    sa = torch.rand(rows, generator=g, device="cuda") * 40 - 20
    sb = torch.rand(rows, generator=g, device="cuda") * 40 - 20
    vo, so = mi.merge_state(va, sa, vb, sb)
    torch.cuda.synchronize()
    for r0, r1 in ((0, 32), ((1 << 24) - 32, rows)):
        rv, rs = oracle.merge_state(_bits(va[r0:r1]), sa[r0:r1].cpu().numpy(),
                                    _bits(vb[r0:r1]), sb[r0:r1].cpu().numpy(), "bf16")
        check_values(vo[r0:r1], rv)
        check_lse(so[r0:r1], rs)
    del va, vb, vo
    _release()


def test_merge_states_past_2g_elements():
    S, N = (1 << 22) + 32, 4       # (pos * N + n) * 128 crosses 2^31 at pos 2^22
    _say("merge_states over", S, "positions x", N, "states of 128 f16")
    g = torch.Generator(device="cuda").manual_seed(1204)
    v = torch.randn((S, N, 1, 128), generator=g, device="cuda").to(torch.float16)
    s = torch.rand((S, N, 1), generator=g, device="cuda") * 40 - 20
    vo, so = mi.merge_states(v, s)
    torch.cuda.synchronize()
    for p0, p1 in ((0, 16), ((1 << 22) - 16, S)):
        rv, rs = oracle.merge_states(_bits(v[p0:p1]), s[p0:p1].cpu().numpy(), "f16")
        check_values(vo[p0:p1], rv)
        check_lse(so[p0:p1], rs)
    del v, vo
    _release()


def test_decode_largest_batch():
    """B = 65535 (the largest the decode accepts), one kv head, lengths U[0, 48]
    (some empty, most with empty splits at 3 splits): every output against the
    oracle, in both launch forms. The sequences draw their pages, with repeats,
    from a pool of 2048 physical pages (shared pages are a valid layout), so the
    inputs stay small; no page holds NaN tails here."""
    g = inputs.rng(1205)
    B, P = 65535, 2048
    ctx = g.integers(0, 49, B).astype(np.int32)
    n_pages = -(-ctx // 16)
    table = g.integers(0, P, (B, 3)).astype(np.int32)
    table[np.arange(3)[None, :] >= n_pages[:, None]] = -1
    qb = inputs.normal_bits(g, (B, 1, 128), "bf16")
    kb = inputs.normal_bits(g, (P, 1, 16, 128), "bf16")
    vb = inputs.normal_bits(g, (P, 1, 16, 128), "bf16")
    _say("decode B=65535", int(ctx.sum()), "tokens")
    q, k, v = (to_device(x, "bf16") for x in (qb, kb, vb))
    pt = torch.from_numpy(table).cuda()
    cl = torch.from_numpy(ctx).cuda()
    sc = 1.0 / np.sqrt(128.0)
    ro, rs = oracle.attention(qb, kb, vb, table, ctx, sc, "bf16", "bf16")
    assert np.isneginf(rs).sum() == (ctx == 0).sum() > 0
    for fused in (False, True):
        f = mi.split_kv_decode_fused if fused else mi.split_kv_decode
        o, s = f(q, k, v, pt, cl, 3, sc)
        torch.cuda.synchronize()
        check_values(o, ro)
        check_lse(s, rs)
    _release()


@pytest.mark.parametrize("R,Hq,Hkv,prefix_len,dtype", [
    (4, 4, 1, 65536, "bf16"),    # one row block, 512 chunks of 128 tokens
    (2, 8, 8, 65552, "f16"),     # chunks at their 1024-token cap: 65 of them
])
def test_cascade_long_prefix(R, Hq, Hkv, prefix_len, dtype):
    """A long shared prefix: many chunk states per row, merged by the suffix
    kernel's combine from memory, or chunks at the cap of 64 pages."""
    _say("cascade long prefix", R, Hq, Hkv, prefix_len, dtype)
    cas = inputs.cascade_case(1206 + Hkv, R=R, prefix_len=prefix_len, suffix_len=40, Hq=Hq,
                              Hkv=Hkv, dtype=dtype)
    q, k, v = (to_device(cas[n], dtype) for n in ("q", "k", "v"))
    pp = torch.from_numpy(cas["prefix_pages"]).cuda()
    st = torch.from_numpy(cas["suffix_table"]).cuda()
    sl = torch.from_numpy(cas["suffix_lens"]).cuda()
    o, s = mi.cascade_decode_fused(q, k, v, pp, prefix_len, st, sl, cas["sm_scale"])
    torch.cuda.synchronize()
    ro, rs = oracle.attention(cas["q"], cas["k"], cas["v"], cas["full_table"], cas["full_lens"],
                              cas["sm_scale"], dtype, dtype)
    check_values(o, ro)
    check_lse(s, rs)
    _release()


@pytest.mark.parametrize("dt_in", ["f32", "f16"])
def test_merge_states_varlen_one_huge_set(dt_in):
    """Index sets of 0-8 states with one set of 200,000 among them: the launch
    sizes its lane teams for the short sets, so the long one is folded by one
    team in batches; every row against the oracle."""
    _say("varlen merge with one set of 200000 states", dt_in)
    g = inputs.rng(1207)
    lens = g.integers(0, 9, 3000)
    lens[1234] = 200_000
    indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total, S, H, D = int(indptr[-1]), 3000, 2, 128
    c = inputs.merge_states_case(1208, S=total, N=1, H=H, D=D, dtype=dt_in, s_lo=-30, s_hi=30)
    v, s = np.ascontiguousarray(c["v"][:, 0]), np.ascontiguousarray(c["s"][:, 0])
    vo, so = mi.merge_states_varlen(to_device(v, dt_in), torch.from_numpy(s).cuda(),
                                    torch.from_numpy(indptr).cuda(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    rv, rs = oracle.merge_states_varlen(v, s, indptr, dt_in)
    check_values(vo, rv)
    check_lse(so, rs)
    _release()
