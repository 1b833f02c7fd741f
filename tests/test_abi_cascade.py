"""CPU-only argument validation of the cascade entry points and of the decode
that allocates nothing. Every device pointer is a fake address that is never
dereferenced, and every call is one that validation must refuse (or a size-0
no-op), so nothing reaches a launch."""
import ctypes

import lse_attention_state_amd as mi

OK, ENULL, ESHAPE, EDTYPE, EUNSUP, EHIP, EALIAS, ESCRATCH = range(8)
F16, BF16, F32 = 0, 1, 2
FAKE = 1 << 40
NULL = ctypes.c_void_p(0)


def P(off=0):
    return ctypes.c_void_p(FAKE + off)


def test_prefix_workspace_validation():
    lib = mi.lib()
    n = ctypes.c_size_t()
    assert lib.mi_prefix_attention_workspace(4, 8, 2, 128, 64, None) == ENULL
    assert lib.mi_prefix_attention_workspace(-1, 8, 2, 128, 64, ctypes.byref(n)) == ESHAPE
    assert lib.mi_prefix_attention_workspace(4, 8, 3, 128, 64, ctypes.byref(n)) == ESHAPE
    assert lib.mi_prefix_attention_workspace(4, 8, 2, 128, -5, ctypes.byref(n)) == ESHAPE
    assert lib.mi_prefix_attention_workspace(4, 8, 2, 64, 64, ctypes.byref(n)) == EUNSUP
    assert lib.mi_prefix_attention_workspace(4, 8, 2, 128, 64, ctypes.byref(n)) == OK
    assert n.value > 0


def _ws(R=4, Hq=8, Hkv=2, L=64):
    n = ctypes.c_size_t()
    assert mi.lib().mi_prefix_attention_workspace(R, Hq, Hkv, 128, L, ctypes.byref(n)) == OK
    return n.value


def _prefix(**kw):
    a = dict(q=P(0), k=P(1 << 30), v=P(2 << 30), pages=P(3 << 30), L=64, R=4, Hq=8, Hkv=2,
             D=128, page=16, Pn=100, dt=BF16, ws=P(4 << 30), wsb=None, vo=P(5 << 30),
             so=P(6 << 30), dto=F32)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = _ws(a["R"] if a["R"] >= 0 else 0, 8, 2, max(a["L"], 0))
    return mi.lib().mi_prefix_attention(a["q"], a["k"], a["v"], a["pages"], a["L"], a["R"],
                                        a["Hq"], a["Hkv"], a["D"], a["page"], a["Pn"],
                                        ctypes.c_float(0.1), a["dt"], a["ws"], a["wsb"], a["vo"],
                                        a["so"], a["dto"], NULL)


def test_prefix_attention_validation():
    assert _prefix(q=NULL) == ENULL
    assert _prefix(ws=NULL) == ENULL
    assert _prefix(vo=NULL) == ENULL
    assert _prefix(pages=NULL) == ENULL          # a non-empty prefix needs its page list
    assert _prefix(R=-1) == ESHAPE
    assert _prefix(Hq=7) == ESHAPE               # not a multiple of Hkv
    assert _prefix(Pn=0) == ESHAPE
    assert _prefix(dt=F32) == EDTYPE             # K/V must be 16-bit
    assert _prefix(dto=9) == EDTYPE
    assert _prefix(D=64) == EUNSUP
    assert _prefix(page=32) == EUNSUP
    assert _prefix(q=P(2)) == EUNSUP             # misaligned
    assert _prefix(wsb=_ws() - 4) == ESHAPE      # workspace too small
    assert _prefix(ws=P((1 << 30) + 64)) == EALIAS   # workspace inside the K cache
    assert _prefix(vo=P(4 << 30)) == EALIAS      # output on top of the workspace
    assert _prefix(R=0) == OK                    # nothing to do, nothing launched


def _cascade(**kw):
    a = dict(q=P(0), k=P(1 << 30), v=P(2 << 30), pages=P(3 << 30), L=64, tab=P(7 << 30),
             stride=8, lens=P(8 << 30), R=4, Hq=8, Hkv=2, D=128, page=16, Pn=100, splits=1,
             dt=BF16, ws=P(4 << 30), wsb=None, op=P(9 << 30), lp=P(10 << 30), cnt=P(11 << 30),
             o=P(5 << 30), lse=P(6 << 30), dto=BF16)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = _ws(a["R"] if a["R"] >= 0 else 0, 8, 2, max(a["L"], 0))
    return mi.lib().mi_cascade_decode(a["q"], a["k"], a["v"], a["pages"], a["L"], a["tab"],
                                      a["stride"], a["lens"], a["R"], a["Hq"], a["Hkv"], a["D"],
                                      a["page"], a["Pn"], a["splits"], ctypes.c_float(0.1),
                                      a["dt"], a["ws"], a["wsb"], a["op"], a["lp"], a["cnt"],
                                      a["o"], a["lse"], a["dto"], NULL)


def test_cascade_decode_validation():
    assert _cascade(o=NULL) == ENULL
    assert _cascade(cnt=NULL) == ENULL
    assert _cascade(ws=NULL) == ENULL
    assert _cascade(pages=NULL) == ENULL
    assert _cascade(tab=NULL) == ENULL
    assert _cascade(L=-1) == ESHAPE
    assert _cascade(splits=0) == ESHAPE
    assert _cascade(Hq=6, Hkv=4) == ESHAPE
    assert _cascade(dt=F32) == EDTYPE
    assert _cascade(D=64) == EUNSUP
    assert _cascade(wsb=_ws() - 4) == ESHAPE
    assert _cascade(ws=P((4 << 30) + 2)) == EUNSUP   # misaligned workspace
    assert _cascade(ws=P(1 << 30)) == EALIAS     # workspace inside the K cache
    assert _cascade(pages=P(4 << 30)) == EALIAS  # page list inside the workspace
    assert _cascade(R=0) == OK


def _noalloc(**kw):
    a = dict(q=P(0), k=P(1 << 30), v=P(2 << 30), pt=P(3 << 30), pts=64, ctx=P(4 << 30), B=2,
             Hq=32, Hkv=8, D=128, page=16, Pn=100, splits=4, dt=F16, o=P(5 << 30),
             lse=P(6 << 30), dto=F16)
    a.update(kw)
    return mi.lib().mi_split_kv_decode_noalloc(a["q"], a["k"], a["v"], a["pt"], a["pts"],
                                               a["ctx"], a["B"], a["Hq"], a["Hkv"], a["D"],
                                               a["page"], a["Pn"], a["splits"],
                                               ctypes.c_float(0.1), a["dt"], a["o"], a["lse"],
                                               a["dto"], NULL)


def test_noalloc_decode_validation():
    assert _noalloc(q=NULL) == ENULL
    assert _noalloc(o=NULL) == ENULL
    assert _noalloc(B=-1) == ESHAPE
    assert _noalloc(splits=0) == ESHAPE
    assert _noalloc(Hq=30) == ESHAPE
    assert _noalloc(dt=F32) == EDTYPE
    assert _noalloc(dto=9) == EDTYPE
    assert _noalloc(D=64) == EUNSUP
    assert _noalloc(splits=2048) == EUNSUP
    assert _noalloc(q=P(2)) == EUNSUP
    assert _noalloc(o=P(1 << 30)) == EALIAS      # output inside the K cache
    assert _noalloc(lse=P(5 << 30)) == EALIAS    # lse on top of o
    # B * Hq * splits beyond the fixed array: refused before any device call
    assert _noalloc(B=64, splits=64) == ESCRATCH
    assert mi.NOALLOC_MAX_PARTIAL_ROWS == 32768
    assert _noalloc(B=0) == OK
