"""Seeded synthetic inputs for attention-state merging and split-KV decode.

This module only draws and lays out data; it holds none of the method's
arithmetic. Both the GPU path and the CPU oracle receive the very same host
bytes produced here: fp16 and bf16 tensors are returned as ``uint16`` bit
patterns, fp32 as ``float32``, indices as ``int32``.

Workload recipes (sizes are arguments; the named cases below use the sizes of
the workloads the merge and decode pages discuss):
  * merge of N states: v ~ N(0,1), s ~ U(lo, hi) base 2, a fraction of states
    empty (s = -inf, v = 0), at least one non-empty state per (pos, h).
  * merge of two states: v ~ N(0,1), s ~ U(lo, hi), a fraction of rows where
    both states are empty.
  * paged decode: q, K, V ~ N(0,1); physical pages drawn from a shuffled pool;
    page_table entries past a sequence's last page are -1 and never read; the
    slots of the last page past ctx are filled with NaN.
"""
from __future__ import annotations

import math

import numpy as np

F16_NAN = np.uint16(0x7E00)
BF16_NAN = np.uint16(0x7FC0)


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bfloat16 (round to nearest even), as bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def normal_bits(g: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0,1) values encoded as ``dtype`` ('f16', 'bf16' -> uint16 bits; 'f32' -> float32)."""
    x = g.standard_normal(size=shape, dtype=np.float32)
    if dtype == "f16":
        return f32_to_f16_bits(x)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f32":
        return x
    raise ValueError(dtype)


def zeros_bits(shape, dtype: str) -> np.ndarray:
    return np.zeros(shape, np.float32 if dtype == "f32" else np.uint16)


def nan_bits(dtype: str):
    return {"f16": F16_NAN, "bf16": BF16_NAN, "f32": np.float32(np.nan)}[dtype]


# ----------------------------------------------------------------------------- merges

def merge_states_case(seed: int, S: int, N: int, H: int, D: int, dtype: str = "f16",
                      s_lo: float = -20.0, s_hi: float = 40.0, empty_frac: float = 0.10):
    """v [S,N,H,D], s [S,N,H] fp32 base 2; ``empty_frac`` of states empty,
    and for every (pos, h) at least one non-empty state (n = 0 is un-emptied)."""
    g = rng(seed)
    v = normal_bits(g, (S, N, H, D), dtype)
    s = g.uniform(s_lo, s_hi, size=(S, N, H)).astype(np.float32)
    empty = g.random((S, N, H)) < empty_frac
    all_empty = empty.all(axis=1)                        # [S, H]
    empty[:, 0, :] &= ~all_empty
    s[empty] = -np.inf
    v[empty] = 0
    return {"v": v, "s": s, "S": S, "N": N, "H": H, "D": D, "dtype": dtype}


def merge_state_case(seed: int, S: int, H: int, D: int, dtype: str = "bf16",
                     s_lo: float = 0.0, s_hi: float = 60.0, empty_row_frac: float = 0.01):
    """v_a, v_b [S,H,D]; s_a, s_b [S,H]; ``empty_row_frac`` of (pos, h) rows have
    both states empty (s = -inf, v = 0); no other state is empty."""
    g = rng(seed)
    va = normal_bits(g, (S, H, D), dtype)
    vb = normal_bits(g, (S, H, D), dtype)
    sa = g.uniform(s_lo, s_hi, size=(S, H)).astype(np.float32)
    sb = g.uniform(s_lo, s_hi, size=(S, H)).astype(np.float32)
    empty = g.random((S, H)) < empty_row_frac
    sa[empty] = -np.inf
    sb[empty] = -np.inf
    va[empty] = 0
    vb[empty] = 0
    return {"va": va, "sa": sa, "vb": vb, "sb": sb, "S": S, "H": H, "D": D,
            "dtype": dtype, "empty_rows": empty}


# ----------------------------------------------------------------------------- decode

def mixed_ctx_lens(seed: int, B: int, hi: int = 8192, forced=(1, 16, 17, 37)) -> np.ndarray:
    """ctx ~ U[1, hi] with the first entries forced to short lengths that leave
    empty splits (and partial last pages)."""
    g = rng(seed)
    ctx = g.integers(1, hi + 1, size=B, dtype=np.int64).astype(np.int32)
    for i, c in enumerate(forced[:B]):
        ctx[i] = c
    return ctx


def paged_kv_case(seed: int, ctx_lens, Hq: int, Hkv: int, D: int, page: int,
                  dtype: str = "f16", extra_pages: int = 0, nan_tail: bool = True):
    """q [B,Hq,D]; K, V [P,Hkv,page,D]; page_table [B, max_pages] int32; ctx [B].

    Each sequence's pages are a disjoint draw from a shuffled pool of
    P = sum(ceil(ctx/page)) + extra_pages physical pages. Entries past a
    sequence's last page are -1. Slots of the last page past ctx hold NaN."""
    g = rng(seed)
    ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    B = ctx.shape[0]
    n_pages = [-(-int(c) // page) for c in ctx]
    P = max(1, sum(n_pages) + extra_pages)
    max_pages = max(1, max(n_pages) if n_pages else 1)
    pool = g.permutation(P).astype(np.int32)
    table = np.full((B, max_pages), -1, np.int32)
    at = 0
    for b in range(B):
        table[b, :n_pages[b]] = pool[at:at + n_pages[b]]
        at += n_pages[b]
    q = normal_bits(g, (B, Hq, D), dtype)
    k = normal_bits(g, (P, Hkv, page, D), dtype)
    v = normal_bits(g, (P, Hkv, page, D), dtype)
    if nan_tail:
        nan = nan_bits(dtype)
        for b in range(B):
            c = int(ctx[b])
            if c % page and n_pages[b]:
                last = table[b, n_pages[b] - 1]
                k[last, :, c % page:, :] = nan
                v[last, :, c % page:, :] = nan
    return {"q": q, "k": k, "v": v, "page_table": table, "ctx_lens": ctx, "B": B, "Hq": Hq,
            "Hkv": Hkv, "D": D, "page": page, "dtype": dtype, "sm_scale": 1.0 / math.sqrt(D)}


def cascade_case(seed: int, R: int = 64, prefix_len: int = 8192, suffix_len: int = 512,
                 Hq: int = 32, Hkv: int = 8, D: int = 128, page: int = 16, dtype: str = "bf16"):
    """R requests sharing one prefix, each with its own suffix, in one shuffled
    page pool. Returns q [R,Hq,D], K/V pools, the shared prefix page list,
    per-request suffix page tables, and the per-request full page tables
    (prefix pages followed by suffix pages) for the unsplit check."""
    assert prefix_len % page == 0, "the shared prefix covers whole pages"
    g = rng(seed)
    n_pre = prefix_len // page
    n_suf = -(-suffix_len // page)
    P = n_pre + R * n_suf
    pool = g.permutation(P).astype(np.int32)
    prefix_pages = pool[:n_pre].copy()
    suffix_table = pool[n_pre:].reshape(R, n_suf).copy()
    full_table = np.concatenate([np.broadcast_to(prefix_pages, (R, n_pre)), suffix_table], axis=1)
    q = normal_bits(g, (R, Hq, D), dtype)
    k = normal_bits(g, (P, Hkv, page, D), dtype)
    v = normal_bits(g, (P, Hkv, page, D), dtype)
    return {"q": q, "k": k, "v": v, "prefix_pages": prefix_pages, "prefix_len": prefix_len,
            "suffix_table": np.ascontiguousarray(suffix_table),
            "suffix_lens": np.full(R, suffix_len, np.int32),
            "full_table": np.ascontiguousarray(full_table),
            "full_lens": np.full(R, prefix_len + suffix_len, np.int32),
            "R": R, "Hq": Hq, "Hkv": Hkv, "D": D, "page": page, "dtype": dtype,
            "sm_scale": 1.0 / math.sqrt(D)}


# ----------------------------------------------------------------------------- sink, mask, segments

def sink_logits(seed: int, H: int, lo: float = -8.0, hi: float = 8.0) -> np.ndarray:
    """One attention-sink logit per head (natural-log units), fp32 [H]."""
    return rng(seed).uniform(lo, hi, size=H).astype(np.float32)


def position_mask(seed: int, S: int, frac_on: float = 0.5) -> np.ndarray:
    """uint8 [S]: 1 where a position is merged, 0 where it is left alone."""
    return (rng(seed).random(S) < frac_on).astype(np.uint8)


def segment_indptr(seed: int, S: int, max_len: int, empty_frac: float = 0.1) -> np.ndarray:
    """int32 [S+1] running sums of segment lengths ~ U[1, max_len], with
    ``empty_frac`` of the segments empty."""
    g = rng(seed)
    lens = g.integers(1, max_len + 1, size=S)
    lens[g.random(S) < empty_frac] = 0
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
