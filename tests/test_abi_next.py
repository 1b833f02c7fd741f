"""CPU-only checks of the entry points for per-sequence splits, the attention
sink, the masked in-place merge, the variable-length merge and the streaming
read used for measurement: the host-side
planner agrees bit-exactly with the oracle's, and argument validation refuses
bad calls before anything is launched (fake device addresses, never touched).
"""
import ctypes

import numpy as np
import pytest

import lse_attention_state_amd as mi
import oracle

OK, ENULL, ESHAPE, EDTYPE, EUNSUP, EHIP, EALIAS = range(7)
F16, BF16, F32 = 0, 1, 2
FAKE = 1 << 40
NULL = ctypes.c_void_p(0)


def P(off=0):
    return ctypes.c_void_p(FAKE + off)


def test_varlen_plan_bit_exact_with_oracle():
    g = np.random.default_rng(21)
    for _ in range(400):
        B = int(g.integers(1, 100))
        Hkv = int(g.choice([1, 2, 4, 8, 16]))
        hi = int(g.choice([1, 64, 1024, 8192, 65536]))
        ctx = g.integers(0, hi + 1, size=B).astype(np.int32)
        if g.random() < 0.3:   # a long/short mix like the mixed-length decode workload
            ctx[: B // 2] = g.integers(1, 64, size=B // 2)
        cus = int(g.choice([80, 170, 256, 304]))
        indptr = mi.plan_splits_varlen(ctx, Hkv, 16, cus)
        _, counts = oracle.plan_splits_varlen(B, Hkv, ctx, 16, cus)
        assert indptr[0] == 0
        assert np.array_equal(np.diff(indptr), counts)


def test_varlen_plan_validation():
    lib = mi.lib()
    ctx = (ctypes.c_int32 * 2)(5, 7)
    out = (ctypes.c_int32 * 3)()
    assert lib.mi_plan_splits_varlen(2, 8, None, 16, 256, out) == ENULL
    assert lib.mi_plan_splits_varlen(2, 8, ctx, 16, 256, None) == ENULL
    assert lib.mi_plan_splits_varlen(0, 8, ctx, 16, 256, out) == ESHAPE
    assert lib.mi_plan_splits_varlen(2, 0, ctx, 16, 256, out) == ESHAPE
    bad = (ctypes.c_int32 * 2)(5, -7)
    assert lib.mi_plan_splits_varlen(2, 8, bad, 16, 256, out) == ESHAPE
    assert lib.mi_plan_splits_varlen(2, 8, ctx, 16, 256, out) == OK
    assert list(out) == [0, 1, 2]


def _sink(**kw):
    a = dict(v=P(0), s=P(1 << 30), sink=P(2 << 30), vo=P(3 << 30), so=P(4 << 30), S=8, H=4,
             D=128, dti=F16, dto=F16)
    a.update(kw)
    return mi.lib().mi_merge_sink(a["v"], a["s"], a["sink"], a["vo"], a["so"], a["S"], a["H"],
                                  a["D"], a["dti"], a["dto"], NULL)


def test_merge_sink_validation():
    assert _sink(sink=NULL) == ENULL
    assert _sink(vo=NULL) == ENULL
    assert _sink(S=-1) == ESHAPE
    assert _sink(H=0) == ESHAPE
    assert _sink(dto=3) == EDTYPE
    assert _sink(D=12) == EUNSUP
    assert _sink(sink=P((2 << 30) + 2)) == EUNSUP          # misaligned
    assert _sink(vo=P(0), so=P(1 << 30), S=0) == OK        # exact in place is allowed
    assert _sink(vo=P(0), dto=F32, S=1) == EALIAS           # in place needs the same dtype
    assert _sink(vo=P(64), S=1) == EALIAS                   # partial overlap
    assert _sink(so=P(1 << 30), vo=P(3 << 30), S=0) == OK   # s in place, nothing to do
    assert _sink(sink=P(3 << 30), S=1) == EALIAS            # output over the sink
    assert _sink(S=0) == OK


def _inplace(**kw):
    a = dict(v=P(0), s=P(1 << 30), vo=P(2 << 30), so=P(3 << 30), mask=P(4 << 30), S=8, H=4,
             D=128, dt=BF16)
    a.update(kw)
    return mi.lib().mi_merge_state_in_place(a["v"], a["s"], a["vo"], a["so"], a["mask"], a["S"],
                                            a["H"], a["D"], a["dt"], NULL)


def test_merge_state_in_place_validation():
    assert _inplace(v=NULL) == ENULL
    assert _inplace(so=NULL) == ENULL
    assert _inplace(S=-2) == ESHAPE
    assert _inplace(dt=9) == EDTYPE
    assert _inplace(D=1024) == EUNSUP
    assert _inplace(vo=P(0)) == EALIAS          # the other state is the state itself
    assert _inplace(mask=P(4)) == EALIAS        # mask inside v
    assert _inplace(s=P(16)) == EALIAS          # s inside v
    assert _inplace(S=0) == OK


def _varlen_merge(**kw):
    a = dict(v=P(0), s=P(1 << 30), ip=P(2 << 30), total=40, vo=P(3 << 30), so=P(4 << 30), S=8,
             H=4, D=128, dti=F32, dto=F16)
    a.update(kw)
    return mi.lib().mi_merge_states_varlen(a["v"], a["s"], a["ip"], a["total"], a["vo"], a["so"],
                                           a["S"], a["H"], a["D"], a["dti"], a["dto"], NULL)


def test_merge_states_varlen_validation():
    assert _varlen_merge(ip=NULL) == ENULL
    assert _varlen_merge(total=-1) == ESHAPE
    assert _varlen_merge(S=-1) == ESHAPE
    assert _varlen_merge(dti=4) == EDTYPE
    assert _varlen_merge(D=4) == EUNSUP
    assert _varlen_merge(ip=P((2 << 30) + 2)) == EUNSUP
    assert _varlen_merge(vo=P(64)) == EALIAS             # output inside the states
    assert _varlen_merge(so=P((2 << 30) + 4)) == EALIAS  # output over indptr
    assert _varlen_merge(S=0) == OK


def _vdec(**kw):
    a = dict(q=P(0), k=P(1 << 30), v=P(2 << 30), pt=P(3 << 30), ctx=P(4 << 30),
             ip=P(10 << 30), total=12, op=P(5 << 30), lp=P(6 << 30), cnt=P(9 << 30),
             o=P(7 << 30), lse=P(8 << 30), dto=F16, B=4, Hq=32, Hkv=8, dt=F16)
    a.update(kw)
    return mi.lib().mi_split_kv_decode_varlen(
        a["q"], a["k"], a["v"], a["pt"], 64, a["ctx"], a["B"], a["Hq"], a["Hkv"], 128, 16, 1024,
        a["ip"], a["total"], ctypes.c_float(0.1), a["dt"], a["op"], a["lp"], a["cnt"], a["o"],
        a["lse"], a["dto"], NULL)


def test_split_kv_decode_varlen_validation():
    assert _vdec(ip=NULL) == ENULL
    assert _vdec(o=NULL) == ENULL
    assert _vdec(op=NULL) == ENULL
    assert _vdec(total=-1) == ESHAPE
    assert _vdec(B=-1) == ESHAPE
    assert _vdec(B=5000, total=5000) == EUNSUP     # beyond the segment search
    assert _vdec(total=70000) == EUNSUP            # beyond the grid height
    assert _vdec(dt=F32) == EDTYPE
    assert _vdec(Hq=48, Hkv=3) == EUNSUP
    assert _vdec(ip=P((10 << 30) + 2)) == EUNSUP   # misaligned
    assert _vdec(ip=P(5 << 30)) == EALIAS          # indptr inside o_part
    assert _vdec(cnt=P((7 << 30) + 64)) == EALIAS  # counters inside o
    assert _vdec(op=P((1 << 30) + 64)) == EALIAS   # o_part inside the K cache
    assert _vdec(B=0, total=0) == OK


def test_merge_states_workspace_and_two_level_validation():
    lib = mi.lib()
    out = ctypes.c_size_t()
    assert lib.mi_merge_states_workspace(64, 1024, 1, 128, None) == ENULL
    assert lib.mi_merge_states_workspace(-1, 4, 1, 128, ctypes.byref(out)) == ESHAPE
    assert lib.mi_merge_states_workspace(64, 1024, 1, 128, ctypes.byref(out)) == OK
    assert out.value == 64 * 16 * 1 * 129 * 4          # 16 slices of 64 states per position
    assert lib.mi_merge_states_workspace(65536, 4, 8, 128, ctypes.byref(out)) == OK
    assert out.value == 0                                # many rows: one level

    def call(**kw):
        a = dict(v=P(0), s=P(1 << 30), vo=P(2 << 30), so=P(3 << 30), S=64, N=1024, H=1, D=128,
                 dti=F32, dto=F16, ws=P(4 << 30), wsb=64 * 16 * 129 * 4)
        a.update(kw)
        return lib.mi_merge_states_two_level(a["v"], a["s"], a["vo"], a["so"], a["S"], a["N"],
                                             a["H"], a["D"], a["dti"], a["dto"], a["ws"],
                                             ctypes.c_size_t(a["wsb"]), NULL)
    assert call(ws=NULL) == ENULL                       # needed and missing
    assert call(wsb=100) == ESHAPE                      # too small
    assert call(ws=P((4 << 30) + 4)) == EUNSUP          # misaligned
    assert call(ws=P(64)) == EALIAS                     # workspace inside the states
    assert call(ws=P((2 << 30) + 16)) == EALIAS         # workspace over the output
    assert call(N=0) == ESHAPE
    assert call(S=0) == OK


def test_stream_read_validation():
    lib = mi.lib()

    def call(x=P(0), nbytes=1 << 20, out=P(1 << 30)):
        return lib.mi_stream_read(x, ctypes.c_int64(nbytes), out, NULL)
    assert call(nbytes=-16) == ESHAPE
    assert call(nbytes=24) == ESHAPE                     # not a multiple of 16
    assert call(x=NULL, out=NULL, nbytes=0) == OK        # nothing to read: nothing enqueued
    assert call(x=NULL) == ENULL
    assert call(out=NULL) == ENULL
    assert call(x=P(8)) == EUNSUP                        # 16-byte alignment
    assert call(out=P((1 << 30) + 2)) == EUNSUP
    assert call(out=P(4096)) == EALIAS                   # the result word inside the buffer
