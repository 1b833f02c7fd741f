"""Benchmark: one step = one pass of the attention-state hot path on one GPU.

A step runs, on synthetic data resident in HBM:
  1. merge_state   bf16 S=32768, H=32, D=128 (1% of rows with both states empty)
  2. merge_states  fp16 S=65536, N=4, H=8, D=128, 10% empty states (the N-state
                   layout of the S=64 parity case at a size that streams HBM)
  3. split-KV decode fp16 B=1, ctx=32768, Hq=32, Hkv=8, D=128, PAGE=16: the
                   planner picks the split count (64), then pass 1 and the
                   combine in one launch (mi_split_kv_decode_fused)
  4. cascade bf16: 64 requests share an 8192-token prefix (matrix-core level),
                   each has a 512-token suffix (split-KV decode) whose combine also
                   merges the prefix chunk states (mi_cascade_decode, two launches)
Inputs are rotated across copies so that consecutive uses of one buffer are
separated by far more traffic than the 256 MB Infinity Cache holds.

Output: one JSON line. value = the N-state merge's algorithmic HBM bytes / its
launch time inside the step (GB/s, 1e9), with frac_of_peak against 8 TB/s;
decode_us is the split-KV decode at B=1, ctx=32768 (both passes, back to back)
and the whole step's rate is under "step". Per-kernel durations come from HIP
events recorded on the stream the kernels run on; the roofline object
describes the kernel that takes the most time in a step, "rooflines" the two
kernels of the metric. cpu_baseline times the fp64 CPU oracle on a bounded
sample of the same inputs.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "HBM GB/s (% of peak) for merge_states + split-KV decode µs at B=1 ctx=32K"
COUNTERS_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--ceiling", action="store_true",
                    help=("run only the plain streaming read (mi_stream_read over 1 GiB and "
                          "128 MiB) and a 1 GiB device copy: the practical HBM rates the "
                          "roofline fractions are read against"))
    ap.add_argument("--configs", action="store_true",
                    help=("instead of the step: one JSON line per workload (the two merges, "
                          "decode at B=1 and on the mixed batch, the cascade) with median / "
                          "p10 / p90 times, GB/s, and the fp64 oracle timed and compared beside "
                          "it"))
    ap.add_argument("--sweep", action="store_true",
                    help=("instead of the step: split-count sweep over the page's three decode "
                          "workloads and the mixed batch (uniform and per-sequence plans), "
                          "plus the merge variants; prints a markdown report"))
    return ap.parse_args()


def to_dev(bits, dt, torch):
    if dt == "f32":
        return torch.from_numpy(np.ascontiguousarray(bits, np.float32)).cuda()
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[dt]
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdt).cuda()


class Raw:
    """A C-ABI entry point bound to precomputed arguments: one ctypes call per
    launch, so the host enqueues far faster than the GPU drains."""

    def __init__(self, mi, name, *args):
        import ctypes
        self.fn = getattr(mi.lib(), name)
        conv = []
        for a in args:
            if hasattr(a, "data_ptr"):
                conv.append(ctypes.c_void_p(a.data_ptr()))
            elif isinstance(a, float):
                conv.append(ctypes.c_float(a))
            else:
                conv.append(a)
        self.args = conv
        self.name = name

    def __call__(self):
        rc = self.fn(*self.args)
        if rc != 0:
            raise RuntimeError(f"{self.name} returned {rc}")


class Timer:
    """Pairs of HIP events on the current stream, averaged per label."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}

    def start(self, label):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs.setdefault(label, []).append([e, None])

    def stop(self, label):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs[label][-1][1] = e

    def mean_us(self, label):
        ps = self.pairs[label]
        return 1000.0 * sum(a.elapsed_time(b) for a, b in ps) / len(ps)

    def reset(self):
        self.pairs = {}


def counter_traffic(name):
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE passes,
    or None when there are none for this kernel or its sources have changed
    since the counters were taken (a stored hash of the sources decides)."""
    import hashlib
    if not os.path.exists(COUNTERS_FILE):
        return None
    with open(COUNTERS_FILE) as f:
        tr = json.load(f).get(name)
    if tr is None:
        return None
    h = hashlib.sha256()
    for src in tr["sources"]:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if h.hexdigest()[:16] != tr["sources_sha256_16"]:
        return None
    return tr["bytes_per_launch"]


def build_workload(torch, mi, inputs):
    """Device buffers, algorithmic bytes and launch closures for one step."""
    parts = []

    # 1. merge_state, bf16 [32768, 32, 128]
    ms = inputs.merge_state_case(1002, S=32768, H=32, D=128, dtype="bf16")
    rows = 32768 * 32
    ms_copies = []
    for c in range(2):
        va = to_dev(ms["va"], "bf16", torch) if c == 0 else ms_copies[0][0].roll(1, 0)
        vb = to_dev(ms["vb"], "bf16", torch) if c == 0 else ms_copies[0][2].roll(1, 0)
        sa = torch.from_numpy(ms["sa"]).cuda() if c == 0 else ms_copies[0][1].roll(1, 0)
        sb = torch.from_numpy(ms["sb"]).cuda() if c == 0 else ms_copies[0][3].roll(1, 0)
        ms_copies.append((va, sa, vb, sb))
    ms_out = torch.empty_like(ms_copies[0][0])
    ms_sout = torch.empty_like(ms_copies[0][1])
    ms_bytes = rows * (3 * 128 * 2 + 3 * 4)

    stream = torch.cuda.current_stream().cuda_stream
    import ctypes
    st = ctypes.c_void_p(stream)
    ms_calls = [Raw(mi, "mi_merge_state", va, sa, vb, sb, ms_out, ms_sout, rows, 1, 128,
                    mi.MI_BF16, mi.MI_BF16, st) for (va, sa, vb, sb) in ms_copies]

    def run_ms(i):
        ms_calls[i % 2]()

    parts.append(dict(name="merge_state", kernel="merge_state_kernel", bytes=ms_bytes, run=run_ms,
                      shape="bf16 S=32768 H=32 D=128"))

    # 2. merge_states, fp16 [65536, 4, 8, 128]
    mss = inputs.merge_states_case(1001, S=65536, N=4, H=8, D=128, dtype="f16")
    mss_v = to_dev(mss["v"], "f16", torch)
    mss_s = torch.from_numpy(mss["s"]).cuda()
    mss_vo = torch.empty((65536, 8, 128), dtype=torch.float16, device="cuda")
    mss_so = torch.empty((65536, 8), dtype=torch.float32, device="cuda")
    mss_bytes = 65536 * 8 * (4 * 128 * 2 + 4 * 4 + 128 * 2 + 4)

    mss_call = Raw(mi, "mi_merge_states", mss_v, mss_s, mss_vo, mss_so, 65536, 4, 8, 128,
                   mi.MI_F16, mi.MI_F16, st)

    def run_mss(i):
        mss_call()

    parts.append(dict(name="merge_states", kernel="merge_states_kernel", bytes=mss_bytes,
                      run=run_mss, shape="f16 S=65536 N=4 H=8 D=128"))

    # 3. split-KV decode, fp16 B=1 ctx=32768 Hq=32 Hkv=8 D=128 PAGE=16
    ctx_host = np.array([32768], np.int32)
    dec = inputs.paged_kv_case(1003, ctx_host, 32, 8, 128, 16, dtype="f16")
    q = to_dev(dec["q"], "f16", torch)
    kv_copies = []
    k0, v0 = to_dev(dec["k"], "f16", torch), to_dev(dec["v"], "f16", torch)
    for c in range(4):
        kv_copies.append((k0, v0) if c == 0 else (k0.clone(), v0.clone()))
    pt = torch.from_numpy(dec["page_table"]).cuda()
    ctx = torch.from_numpy(dec["ctx_lens"]).cuda()
    splits = mi.plan_splits(ctx_host, 8, 16)
    o_part = torch.empty((1, 32, splits, 128), dtype=torch.float32, device="cuda")
    lse_part = torch.empty((1, 32, splits), dtype=torch.float32, device="cuda")
    o = torch.empty((1, 32, 128), dtype=torch.float16, device="cuda")
    lse = torch.empty((1, 32), dtype=torch.float32, device="cuda")
    kv_bytes = 2 * 32768 * 8 * 128 * 2
    part_bytes = 32 * splits * (128 + 1) * 4
    dec_partial_bytes = kv_bytes + q.numel() * 2 + pt.numel() * 4 + 4 + part_bytes
    dec_combine_bytes = part_bytes + 32 * (128 * 2 + 4)

    def plan(i):
        assert mi.plan_splits(ctx_host, 8, 16) == splits

    scale = float(dec["sm_scale"])
    partial_calls = [Raw(mi, "mi_split_kv_partial", q, k, v, pt, 2048, ctx, 1, 32, 8, 128, 16,
                         2048, splits, scale, mi.MI_F16, o_part, lse_part, st)
                     for (k, v) in kv_copies]
    combine_call = Raw(mi, "mi_merge_states", o_part, lse_part, o, lse, 32, splits, 1, 128,
                       mi.MI_F32, mi.MI_F16, st)
    decode_calls = [Raw(mi, "mi_split_kv_decode", q, k, v, pt, 2048, ctx, 1, 32, 8, 128, 16, 2048,
                        splits, scale, mi.MI_F16, o_part, lse_part, o, lse, mi.MI_F16, st)
                    for (k, v) in kv_copies]
    counters = torch.zeros((1, 8), dtype=torch.int32, device="cuda")
    fused_calls = [Raw(mi, "mi_split_kv_decode_fused", q, k, v, pt, 2048, ctx, 1, 32, 8, 128, 16,
                       2048, splits, scale, mi.MI_F16, o_part, lse_part, counters, o, lse,
                       mi.MI_F16, st)
                   for (k, v) in kv_copies]

    def run_decode(i):
        fused_calls[i % 4]()

    parts.append(dict(name="split_kv_decode", kernel="split_kv_partial_kernel",
                      bytes=dec_partial_bytes + dec_combine_bytes, run=run_decode, host=plan,
                      shape=(f"f16 B=1 ctx=32768 Hq=32 Hkv=8 D=128 PAGE=16 splits={splits}, "
                             "pass 1 and combine in one launch")))
    # 4. cascade, bf16: 64 requests share an 8192-token prefix, 512-token suffixes
    cas = inputs.cascade_case(1005)
    R, cHq, cHkv = cas["R"], cas["Hq"], cas["Hkv"]
    cq = to_dev(cas["q"], "bf16", torch)
    ck, cv = to_dev(cas["k"], "bf16", torch), to_dev(cas["v"], "bf16", torch)
    cpages = torch.from_numpy(cas["prefix_pages"]).cuda()
    ctab = torch.from_numpy(cas["suffix_table"]).cuda()
    clen = torch.from_numpy(cas["suffix_lens"]).cuda()
    cP = cas["k"].shape[0]
    c_splits = mi.plan_splits(cas["suffix_lens"], cHkv, 16)
    ws_bytes = mi.prefix_attention_workspace_bytes(R, cHq, cHkv, 128, cas["prefix_len"])
    c_ws = torch.empty(ws_bytes // 4, dtype=torch.float32, device="cuda")
    vp = torch.empty((R, cHq, 128), dtype=torch.float32, device="cuda")
    sp = torch.empty((R, cHq), dtype=torch.float32, device="cuda")
    vs = torch.empty_like(vp)
    ss = torch.empty_like(sp)
    c_op = torch.empty((R, cHq, c_splits, 128), dtype=torch.float32, device="cuda")
    c_lp = torch.empty((R, cHq, c_splits), dtype=torch.float32, device="cuda")
    c_cnt = torch.zeros((R, cHkv), dtype=torch.int32, device="cuda")
    c_o = torch.empty((R, cHq, 128), dtype=torch.bfloat16, device="cuda")
    c_lse = torch.empty((R, cHq), dtype=torch.float32, device="cuda")
    cscale = float(cas["sm_scale"])
    prefix_call = Raw(mi, "mi_prefix_attention", cq, ck, cv, cpages, cas["prefix_len"], R, cHq,
                      cHkv, 128, 16, cP, cscale, mi.MI_BF16, c_ws, ws_bytes, vp, sp, mi.MI_F32, st)
    suffix_call = Raw(mi, "mi_split_kv_decode_fused", cq, ck, cv, ctab, ctab.shape[1], clen, R,
                      cHq, cHkv, 128, 16, cP, c_splits, cscale, mi.MI_BF16, c_op, c_lp, c_cnt, vs,
                      ss, mi.MI_F32, st)
    level_merge = Raw(mi, "mi_merge_state", vp, sp, vs, ss, c_o, c_lse, R * cHq, 1, 128,
                      mi.MI_F32, mi.MI_BF16, st)
    n_ch = ws_bytes // (R * cHq * 129 * 4)
    rows_s = R * cHq
    prefix_bytes = (cas["prefix_len"] * cHkv * 128 * 2 * 2 + cq.numel() * 2 + cpages.numel() * 4
                    + 2 * rows_s * n_ch * 129 * 4 + rows_s * 129 * 4)
    suffix_bytes = (R * 512 * cHkv * 128 * 2 * 2 + cq.numel() * 2 + ctab.numel() * 4 + R * 4
                    + 2 * rows_s * c_splits * 129 * 4 + rows_s * 129 * 4)
    merge_bytes = 2 * rows_s * 129 * 4 + rows_s * (128 * 2 + 4)
    prefix_flops = 4 * R * cHq * cas["prefix_len"] * 128

    # The cascade in the step: mi_cascade_decode, two launches (the prefix
    # chunk states, then the suffix decode whose combine also merges them).
    f_o = torch.empty((R, cHq, 128), dtype=torch.bfloat16, device="cuda")
    f_lse = torch.empty((R, cHq), dtype=torch.float32, device="cuda")
    f_cnt = torch.zeros((R, cHkv), dtype=torch.int32, device="cuda")
    cascade_call = Raw(mi, "mi_cascade_decode", cq, ck, cv, cpages, cas["prefix_len"], ctab,
                       ctab.shape[1], clen, R, cHq, cHkv, 128, 16, cP, c_splits, cscale,
                       mi.MI_BF16, c_ws, ws_bytes, c_op, c_lp, f_cnt, f_o, f_lse, mi.MI_BF16, st)
    cascade_bytes = (cas["prefix_len"] * cHkv * 128 * 2 * 2 + R * 512 * cHkv * 128 * 2 * 2
                     + 2 * cq.numel() * 2 + cpages.numel() * 4 + ctab.numel() * 4 + R * 4
                     + 2 * rows_s * n_ch * 129 * 4
                     + (2 if c_splits > 1 else 1) * rows_s * c_splits * 129 * 4
                     + rows_s * (128 * 2 + 4))
    parts.append(dict(name="cascade", kernel="prefix_attention_kernel", bytes=cascade_bytes,
                      flops=prefix_flops, run=lambda i: cascade_call(),
                      shape=(f"bf16 64 requests x (8192 shared + 512 own), Hq=32 Hkv=8 D=128: "
                             f"prefix level on MFMA ({n_ch} chunks), suffix decode "
                             f"(splits={c_splits}) whose combine merges the prefix chunks")))
    host = dict(ms=ms, mss=mss, dec=dec, cas=cas, cascade_bytes=cascade_bytes, splits=splits,
                mss_call=mss_call, ms_calls=ms_calls,
                decode_calls=decode_calls,
                prefix_call=prefix_call, prefix_flops=prefix_flops, prefix_bytes=prefix_bytes,
                four_launch=[prefix_call, suffix_call, level_merge], cascade_call=cascade_call,
                fused_calls=fused_calls, partial_calls=partial_calls, combine_call=combine_call,
                plan=plan)
    return parts, host


def cpu_baseline(host, oracle, min_seconds=10.0, max_reps=40):
    """Time the oracle on the step's own inputs: one pass is every part of the
    step (merge_state over all rows, merge_states over all positions, unsplit
    decode attention at ctx=32768, unsplit cascade attention over prefix and
    suffix), repeated until at least `min_seconds` of wall time have passed
    (at most `max_reps` passes). GB/s counts the same algorithmic bytes per
    pass as the GPU step."""
    threads = len(os.sched_getaffinity(0))
    ms, mss, dec, cas = host["ms"], host["mss"], host["dec"], host["cas"]
    rows = 32768 * 32
    pass_bytes = (rows * (3 * 128 * 2 + 3 * 4) + 65536 * 8 * (4 * 128 * 2 + 4 * 4 + 128 * 2 + 4)
                  + 2 * 32768 * 8 * 128 * 2 + host["cascade_bytes"])
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.merge_state(ms["va"].reshape(-1, 128), ms["sa"].reshape(-1),
                           ms["vb"].reshape(-1, 128), ms["sb"].reshape(-1), "bf16", threads)
        oracle.merge_states(mss["v"], mss["s"], "f16", threads)
        oracle.attention(dec["q"], dec["k"], dec["v"], dec["page_table"], dec["ctx_lens"],
                         dec["sm_scale"], "f16", "f16", threads)
        oracle.attention(cas["q"], cas["k"], cas["v"], cas["full_table"], cas["full_lens"],
                         cas["sm_scale"], "bf16", "bf16", threads)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or reps >= max_reps:
            break
    return {"value": round(reps * pass_bytes / dt / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"fp64 oracle over the step's whole workload (merge_state all rows, "
                       f"merge_states all positions, unsplit decode at ctx=32768, unsplit "
                       f"cascade attention), {reps} passes in {dt:.2f} s wall; GB/s counts "
                       f"the same algorithmic bytes per pass as the GPU step")}


def _loop_us(torch, fn, iters, warmup=5):
    """Mean time per call (µs) over `iters` calls enqueued back to back, with
    one HIP event pair around the loop on the current stream (events between
    calls would add their own gaps to kernels of a few microseconds)."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(iters):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return 1000.0 * a.elapsed_time(b) / iters


def sweep(torch, mi, inputs, iters, with_cpu=True):
    """Split-count sweep ("L3 hints", section 6 table: 1 x 32768, 8 x 4096,
    64 x 1024 with 1/4/16/64 splits) plus the mixed batch, under the uniform and
    the per-sequence plans, and the merge variants. K/V are rotated over 4
    copies (512 MiB) so every call streams from HBM."""
    import ctypes
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    Hq, Hkv, D, PAGE = 32, 8, 128, 16
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = ["# Split-count sweep and merge variants (fp16 decode, Hq=32, Hkv=8, D=128, PAGE=16)",
           "", f"Device compute units: {cus}. Mean per call over {iters} calls enqueued back to "
           "back (one HIP event pair around the loop), inputs rotated over copies (K/V over 4). "
           "GB/s counts valid K/V tokens once plus the partials written and read.",
           ""]
    workloads = [("1 x 32768", np.array([32768], np.int32)),
                 ("8 x 4096", np.full(8, 4096, np.int32)),
                 ("64 x 1024", np.full(64, 1024, np.int32)),
                 ("mixed 32 x U[1,8192]", inputs.mixed_ctx_lens(1004, 32))]
    out += ["The fused entry points (mi_split_kv_decode_fused, mi_split_kv_decode_varlen with "
            "counters) run one launch while the work items (B * Hkv * splits) are at most twice "
            "the compute units, else pass 1 and the combine as two launches; the form column "
            "says which.", "",
            "| workload | plan | splits (total) | two launches µs | fused entry µs | form | "
            "fused GB/s |", "|---|---|---:|---:|---:|---|---:|"]
    for wi, (name, ctx) in enumerate(workloads):
        case = inputs.paged_kv_case(2000 + wi, ctx, Hq, Hkv, D, PAGE, dtype="f16")
        B = len(ctx)
        q = to_dev(case["q"], "f16", torch)
        k0, v0 = to_dev(case["k"], "f16", torch), to_dev(case["v"], "f16", torch)
        kv = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(3)]
        pt = torch.from_numpy(case["page_table"]).cuda()
        ctxd = torch.from_numpy(ctx).cuda()
        P = case["k"].shape[0]
        scale = float(case["sm_scale"])
        kv_bytes = int(ctx.astype(np.int64).sum()) * Hkv * D * 2 * 2
        o = torch.empty((B, Hq, D), dtype=torch.float16, device="cuda")
        lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
        cnt = torch.zeros((B, Hkv), dtype=torch.int32, device="cuda")
        pick = mi.plan_splits(ctx, Hkv, PAGE)
        rows = []
        for n in (1, 4, 16, 64):
            op = torch.empty((B, Hq, n, D), dtype=torch.float32, device="cuda")
            lp = torch.empty((B, Hq, n), dtype=torch.float32, device="cuda")
            two = [Raw(mi, "mi_split_kv_decode", q, k, v, pt, pt.shape[1], ctxd, B, Hq, Hkv, D,
                       PAGE, P, n, scale, mi.MI_F16, op, lp, o, lse, mi.MI_F16, st) for k, v in kv]
            one = [Raw(mi, "mi_split_kv_decode_fused", q, k, v, pt, pt.shape[1], ctxd, B, Hq, Hkv,
                       D, PAGE, P, n, scale, mi.MI_F16, op, lp, cnt, o, lse, mi.MI_F16, st)
                   for k, v in kv]
            t2 = _loop_us(torch, lambda i: two[i % 4](), iters)
            t1 = _loop_us(torch, lambda i: one[i % 4](), iters)
            part = B * Hq * n * (D + 1) * 4 * 2 if n > 1 else 0
            label = "uniform" + (" (planner's pick)" if n == pick else "")
            form = "one" if n == 1 or B * Hkv * n <= 2 * cus else "two"
            rows.append(f"| {name} | {label} | {n} | {t2:.1f} | {t1:.1f} | {form} | "
                        f"{(kv_bytes + part) / (t1 * 1e-6) / 1e9:.0f} |")
        indptr = mi.plan_splits_varlen(ctx, Hkv, PAGE)
        total = int(indptr[-1])
        ipd = torch.from_numpy(indptr).cuda()
        op = torch.empty((total, Hq, D), dtype=torch.float32, device="cuda")
        lp = torch.empty((total, Hq), dtype=torch.float32, device="cuda")
        vtwo = [Raw(mi, "mi_split_kv_decode_varlen", q, k, v, pt, pt.shape[1], ctxd, B, Hq, Hkv, D,
                    PAGE, P, ipd, total, scale, mi.MI_F16, op, lp, None, o, lse, mi.MI_F16, st)
                for k, v in kv]
        vone = [Raw(mi, "mi_split_kv_decode_varlen", q, k, v, pt, pt.shape[1], ctxd, B, Hq, Hkv, D,
                    PAGE, P, ipd, total, scale, mi.MI_F16, op, lp, cnt, o, lse, mi.MI_F16, st)
                for k, v in kv]
        t2 = _loop_us(torch, lambda i: vtwo[i % 4](), iters)
        t1 = _loop_us(torch, lambda i: vone[i % 4](), iters)
        counts = np.diff(indptr)
        part = Hq * total * (D + 1) * 4 * 2 if total > B else 0
        form = "one" if total * Hkv <= 2 * cus else "two"
        rows.append(f"| {name} | per-sequence (counts {counts.min()}..{counts.max()}) | "
                    f"({total}) | {t2:.1f} | {t1:.1f} | {form} | "
                    f"{(kv_bytes + part) / (t1 * 1e-6) / 1e9:.0f} |")
        out += rows
        del kv, k0, v0
        torch.cuda.empty_cache()

    # Merges: mi_merge_states (N-state kernel; segmented kernel below 2048 rows)
    # against mi_merge_states_varlen (always the segmented kernel) on the same data.
    out += ["", "| merge | shape | mi_merge_states µs | mi_merge_states_varlen µs | "
            "mi_merge_states_two_level µs |", "|---|---|---:|---:|---:|"]
    two_level_rows = []
    for S, N, H, dt in ((32, 64, 1, "f32"), (1024, 16, 1, "f32"), (2048, 16, 1, "f32"),
                        (4096, 16, 1, "f32"), (4096, 4, 8, "f16"), (512, 64, 8, "f16"),
                        (64, 1024, 1, "f32"), (64, 16384, 1, "f32")):
        c = inputs.merge_states_case(2100 + N, S=S, N=N, H=H, D=D, dtype=dt)
        cop = [(to_dev(c["v"], dt, torch), torch.from_numpy(c["s"]).cuda()) for _ in range(4)]
        vo = torch.empty((S, H, D), dtype=torch.float16, device="cuda")
        so = torch.empty((S, H), dtype=torch.float32, device="cuda")
        ipd = torch.from_numpy((np.arange(S + 1) * N).astype(np.int32)).cuda()
        code = {"f16": mi.MI_F16, "bf16": mi.MI_BF16, "f32": mi.MI_F32}[dt]
        a = [Raw(mi, "mi_merge_states", v, s, vo, so, S, N, H, D, code, mi.MI_F16, st)
             for v, s in cop]
        b = [Raw(mi, "mi_merge_states_varlen", v, s, ipd, S * N, vo, so, S, H, D, code, mi.MI_F16,
                 st) for v, s in cop]
        need = mi.merge_states_workspace_bytes(S, N, H, D)
        ws = torch.empty(max(need // 4, 1), dtype=torch.float32, device="cuda")
        w = [Raw(mi, "mi_merge_states_two_level", v, s, vo, so, S, N, H, D, code, mi.MI_F16, ws,
                 need, st) for v, s in cop]
        ta = _loop_us(torch, lambda i: a[i % 4](), iters)
        tb = _loop_us(torch, lambda i: b[i % 4](), iters)
        tw = _loop_us(torch, lambda i: w[i % 4](), iters)
        out.append(f"| merge_states {dt}->f16 | S={S} N={N} H={H} D={D} | {ta:.1f} | {tb:.1f} | "
                   f"{tw:.1f} |")
        if N >= 1024:
            by = S * N * H * (D * 4 + 4) + S * H * (D * 2 + 4)
            two_level_rows.append(
                f"| merge_states_two_level (two launches) | f32->f16 S={S} N={N} H={H} D={D} | "
                f"{tw:.1f} | {by} | {by / (tw * 1e-6) / 1e9:.0f} | {by / (tw * 1e-6) / 8e12 * 100:.1f} |")
        del cop
        torch.cuda.empty_cache()

    # Sink and masked in-place merges at the two-state size (bf16 S=32768 H=32 D=128).
    ms = inputs.merge_state_case(1002, S=32768, H=32, D=128, dtype="bf16")
    rows_ = 32768 * 32
    va = [to_dev(ms["va"], "bf16", torch) for _ in range(2)]
    sa = [torch.from_numpy(ms["sa"]).cuda() for _ in range(2)]
    vb = to_dev(ms["vb"], "bf16", torch)
    sb = torch.from_numpy(ms["sb"]).cuda()
    sink = torch.from_numpy(inputs.sink_logits(1103, 32)).cuda()
    mask = torch.from_numpy(inputs.position_mask(1010, 32768)).cuda()
    ones = torch.ones(32768, dtype=torch.uint8, device="cuda")
    out += ["", "| kernel | shape | µs | algorithmic bytes | GB/s | % of 8 TB/s |",
            "|---|---|---:|---:|---:|---:|"]
    # The two core merges back to back (inputs rotated), for comparison with
    # their once-per-step times in the default run.
    msv = [(to_dev(ms["va"], "bf16", torch), torch.from_numpy(ms["sa"]).cuda(),
            to_dev(ms["vb"], "bf16", torch), torch.from_numpy(ms["sb"]).cuda()) for _ in range(2)]
    mvo, mso = torch.empty_like(msv[0][0]), torch.empty_like(msv[0][1])
    calls = [Raw(mi, "mi_merge_state", a, b, c_, d, mvo, mso, rows_, 1, 128, mi.MI_BF16,
                 mi.MI_BF16, st) for a, b, c_, d in msv]
    t = _loop_us(torch, lambda i: calls[i % 2](), iters)
    by = rows_ * (3 * 256 + 3 * 4)
    out.append(f"| merge_state, back to back | bf16 S=32768 H=32 D=128 | {t:.1f} | {by} | "
               f"{by / (t * 1e-6) / 1e9:.0f} | {by / (t * 1e-6) / 8e12 * 100:.1f} |")
    del msv, mvo, mso, calls
    mss = inputs.merge_states_case(1001, S=65536, N=4, H=8, D=128, dtype="f16")
    mv = [to_dev(mss["v"], "f16", torch) for _ in range(2)]
    msd = torch.from_numpy(mss["s"]).cuda()
    mvo = torch.empty((65536, 8, 128), dtype=torch.float16, device="cuda")
    mso = torch.empty((65536, 8), dtype=torch.float32, device="cuda")
    calls = [Raw(mi, "mi_merge_states", v_, msd, mvo, mso, 65536, 4, 8, 128, mi.MI_F16,
                 mi.MI_F16, st) for v_ in mv]
    t = _loop_us(torch, lambda i: calls[i % 2](), iters)
    by = 65536 * 8 * (4 * 128 * 2 + 4 * 4 + 128 * 2 + 4)
    out.append(f"| merge_states, back to back | f16 S=65536 N=4 H=8 D=128 | {t:.1f} | {by} | "
               f"{by / (t * 1e-6) / 1e9:.0f} | {by / (t * 1e-6) / 8e12 * 100:.1f} |")
    del mv, mvo, mso, calls
    torch.cuda.empty_cache()
    sink_calls = [Raw(mi, "mi_merge_sink", va[i], sa[i], sink, va[i], sa[i], 32768, 32, 128,
                      mi.MI_BF16, mi.MI_BF16, st) for i in range(2)]
    t = _loop_us(torch, lambda i: sink_calls[i % 2](), iters)
    by = rows_ * (2 * 256 + 2 * 4) + 32 * 4
    out.append(f"| merge_sink (in place) | bf16 S=32768 H=32 D=128 | {t:.1f} | {by} | "
               f"{by / (t * 1e-6) / 1e9:.0f} | {by / (t * 1e-6) / 8e12 * 100:.1f} |")
    for label, m, frac in (("all set", ones, 1.0), ("half set", mask, float(mask.float().mean()))):
        calls = [Raw(mi, "mi_merge_state_in_place", va[i], sa[i], vb, sb, m, 32768, 32, 128,
                     mi.MI_BF16, st) for i in range(2)]
        t = _loop_us(torch, lambda i: calls[i % 2](), iters)
        by = int(rows_ * frac) * (3 * 256 + 3 * 4) + 32768
        out.append(f"| merge_state_in_place, mask {label} | bf16 S=32768 H=32 D=128 | {t:.1f} | "
                   f"{by} | {by / (t * 1e-6) / 1e9:.0f} | {by / (t * 1e-6) / 8e12 * 100:.1f} |")
    # Variable-length merges: 8192 and 65536 sets of 0..8 fp16 states, H=8.
    for n_sets, seeds in ((65536, (2202, 2203)), (8192, (2200, 2201))):
        indptr_ = inputs.segment_indptr(seeds[0], n_sets, 8)
        total = int(indptr_[-1])
        c_ = inputs.merge_states_case(seeds[1], S=1, N=total, H=8, D=128, dtype="f16")
        ncp = 4 if n_sets <= 8192 else 2
        vv = [to_dev(c_["v"].reshape(total, 8, 128), "f16", torch) for _ in range(ncp)]
        ss = torch.from_numpy(c_["s"].reshape(total, 8)).cuda()
        ipd = torch.from_numpy(indptr_).cuda()
        vo = torch.empty((n_sets, 8, 128), dtype=torch.float16, device="cuda")
        so = torch.empty((n_sets, 8), dtype=torch.float32, device="cuda")
        calls = [Raw(mi, "mi_merge_states_varlen", vv[i], ss, ipd, total, vo, so, n_sets, 8, 128,
                     mi.MI_F16, mi.MI_F16, st) for i in range(ncp)]
        t = _loop_us(torch, lambda i: calls[i % ncp](), iters)
        by = total * 8 * (256 + 4) + (n_sets + 1) * 4 + n_sets * 8 * (256 + 4)
        out.append(f"| merge_states_varlen | f16 {n_sets} sets x U[0..8] states ({total}), H=8 D=128 | "
                   f"{t:.1f} | {by} | {by / (t * 1e-6) / 1e9:.0f} | {by / (t * 1e-6) / 8e12 * 100:.1f} |")
        if n_sets == 8192:
            indptr, c = indptr_, c_
        del vv, ss, vo, so, calls
        torch.cuda.empty_cache()
    out += two_level_rows
    if with_cpu:
        import oracle
        out += [""] + cpu_baseline_sweep(oracle, inputs, ms, sink.cpu().numpy(), indptr, c)
    print("\n".join(out))


def ceiling(torch, mi, iters):
    """Practical HBM rates, printed as JSON lines: the library's plain streaming
    read (mi_stream_read: 16-byte non-temporal loads, nothing else) over 1 GiB
    and over 128 MiB (the decode's K/V size), and torch's 1 GiB device copy.
    They are the context for the kernels' fractions of the 8 TB/s peak. Buffers
    are rotated so that the 256 MB Infinity Cache holds none of the next call's
    input."""
    import ctypes
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    xo = torch.zeros(1, dtype=torch.int32, device="cuda")
    for nbytes, copies in ((1 << 30, 2), (128 << 20, 4)):
        bufs = [torch.ones(nbytes // 4, dtype=torch.int32, device="cuda") for _ in range(copies)]
        calls = [Raw(mi, "mi_stream_read", b, nbytes, xo, st) for b in bufs]
        t = _loop_us(torch, lambda i: calls[i % copies](), iters)
        print(json.dumps({"kernel": "mi_stream_read (plain 16-byte streaming read)",
                          "bytes": nbytes, "us": round(t, 2),
                          "GB/s": round(nbytes / (t * 1e-6) / 1e9, 1),
                          "frac_of_8TBs": round(nbytes / (t * 1e-6) / 8e12, 4)}))
        del bufs, calls
    a = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    t = _loop_us(torch, lambda i: b.copy_(a), iters)
    moved = 2 * a.numel() * 4
    print(json.dumps({"kernel": "torch device copy: 1 GiB read + 1 GiB written", "bytes": moved,
                      "us": round(t, 2), "GB/s": round(moved / (t * 1e-6) / 1e9, 1),
                      "frac_of_8TBs": round(moved / (t * 1e-6) / 8e12, 4)}))
    del a, b
    # The two-state merge's read:write mix (2:1) in a plain elementwise kernel:
    # torch's add of two bf16 tensors of 256 MiB into a third, inputs rotated.
    n = 1 << 27
    xs = [torch.ones(n, dtype=torch.bfloat16, device="cuda") for _ in range(4)]
    y = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    t = _loop_us(torch, lambda i: torch.add(xs[(2 * i) % 4], xs[(2 * i + 1) % 4], out=y), iters)
    moved = 3 * n * 2
    print(json.dumps({"kernel": "torch add, two 256 MiB bf16 inputs into a third (2:1 read:write)",
                      "bytes": moved, "us": round(t, 2), "GB/s": round(moved / (t * 1e-6) / 1e9, 1),
                      "frac_of_8TBs": round(moved / (t * 1e-6) / 8e12, 4)}))
    del xs, y
    # The N-state merge's mix at N = 4 (4:1): torch's sum over the first axis of a
    # [4, n] fp16 tensor (four 128 MiB rows into one), inputs rotated.
    n = 1 << 26
    xs = [torch.ones((4, n), dtype=torch.float16, device="cuda") for _ in range(2)]
    y = torch.empty(n, dtype=torch.float16, device="cuda")
    t = _loop_us(torch, lambda i: torch.sum(xs[i % 2], dim=0, out=y), iters)
    moved = 5 * n * 2
    print(json.dumps({"kernel": "torch sum over 4 rows of 128 MiB fp16 into one (4:1 read:write)",
                      "bytes": moved, "us": round(t, 2), "GB/s": round(moved / (t * 1e-6) / 1e9, 1),
                      "frac_of_8TBs": round(moved / (t * 1e-6) / 8e12, 4)}))


def cpu_baseline_sweep(oracle, inputs, ms, sink, indptr, vs_case):
    """The fp64 oracle timed beside the sweep's kernels, on bounded samples of
    the same inputs (cpu_baseline leg of --sweep). GB/s counts the same
    algorithmic bytes per row as the GPU lines."""
    threads = len(os.sched_getaffinity(0))
    L = [f"Oracle (fp64 CPU, {threads} threads) on bounded samples of the same inputs:", "",
         "| path | sample | s | algorithmic GB/s |", "|---|---|---:|---:|"]
    n = 32768 * 32 // 4                       # a quarter of the two-state rows
    va, sa = ms["va"].reshape(-1, 1, 128)[:n], ms["sa"].reshape(-1, 1)[:n]
    vb, sb = ms["vb"].reshape(-1, 1, 128)[:n], ms["sb"].reshape(-1, 1)[:n]
    t0 = time.perf_counter()
    oracle.merge_sink(va, sa, sink[:1], "bf16", threads)
    dt = time.perf_counter() - t0
    L.append(f"| merge_sink | {n} rows (one head's sink) | {dt:.2f} | {n * 520 / dt / 1e9:.3f} |")
    mask = np.ones(n, np.uint8)
    t0 = time.perf_counter()
    oracle.merge_state_masked(va, sa, vb, sb, mask, "bf16", threads)
    dt = time.perf_counter() - t0
    L.append(f"| merge_state_in_place (mask all set) | {n} rows | {dt:.2f} | {n * 780 / dt / 1e9:.3f} |")
    S2 = len(indptr) - 1                      # every set
    ip = indptr
    tot = int(ip[-1])
    t0 = time.perf_counter()
    oracle.merge_states_varlen(vs_case["v"].reshape(-1, 8, 128)[:tot], vs_case["s"].reshape(-1, 8)[:tot],
                               ip, "f16", threads)
    dt = time.perf_counter() - t0
    L.append(f"| merge_states_varlen | all {S2} sets ({tot} states), H=8 | {dt:.2f} | "
             f"{(tot + S2) * 8 * 260 / dt / 1e9:.3f} |")
    ctx = inputs.mixed_ctx_lens(1004, 32)
    case = inputs.paged_kv_case(2003, ctx, 32, 8, 128, 16, dtype="f16")
    args = (case["q"], case["k"], case["v"], case["page_table"], ctx, case["sm_scale"])
    pages = -(-ctx.astype(np.int64) // 16)
    counts = np.maximum(1, -(-pages // 64))             # splits of at most 64 pages
    ipd = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    t0 = time.perf_counter()
    oracle.split_partials_varlen(*args, ipd, "f16", "f16", threads)
    dt = time.perf_counter() - t0
    kvb = int(ctx.astype(np.int64).sum()) * 8 * 128 * 4
    L.append(f"| per-sequence decode partials | the 32-sequence mixed batch "
             f"({int(ctx.sum())} tokens) | {dt:.2f} | {kvb / dt / 1e9:.3f} |")
    return L


def _times_us(torch, fn, iters, warmup=10):
    """Per-call HIP-event durations (µs) on the current stream."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    ev = []
    for i in range(iters):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn(i)
        b.record()
        ev.append((a, b))
    torch.cuda.synchronize()
    return np.array([1000.0 * a.elapsed_time(b) for a, b in ev])


_MANT = {"f16": 10, "bf16": 7, "f32": 23}
_MIN_EXP = {"f16": -14, "bf16": -126, "f32": -126}


def _agreement(got, ref, out_dt, got_s=None, ref_s=None):
    """GPU output against the oracle's: max abs / rel error, how many elements
    pass the 2e-3 + 2e-3|ref| rule only by the rounding term (half an ulp of the
    output type plus 2^-16 |ref|, the allowance of the parity tests), NaNs,
    and the largest LSE difference (-inf must match -inf)."""
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref)
    stated = 2e-3 + 2e-3 * np.abs(ref)
    a = np.abs(ref)
    e = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), _MIN_EXP[out_dt])
    rounding = 0.5 * np.exp2(e - _MANT[out_dt]) + 2.0 ** -16 * a
    r = {"max_abs_err": float(err.max(initial=0.0)),
         "max_rel_err": float((err / np.maximum(a, 1e-30)).max(initial=0.0)),
         "outside_tolerance": int((err > np.maximum(stated, rounding)).sum()),
         "pass_by_ulp_only": int(((err > stated) & (err <= rounding)).sum()),
         "nan": int(np.isnan(got).sum())}
    if got_s is not None:
        gs = np.asarray(got_s, np.float64)
        fin = ~np.isneginf(ref_s)
        r["lse_inf_pattern_equal"] = bool(np.array_equal(np.isneginf(gs), ~fin))
        r["max_lse_err"] = float(np.abs(gs[fin] - ref_s[fin]).max(initial=0.0))
        r["lse_nan"] = int(np.isnan(gs).sum())
    return r


def configs_report(torch, mi, inputs, iters, with_cpu):
    """One JSON line per workload ("configs"): GPU times over `iters` calls
    (median, p10, p90), algorithmic GB/s, and -- the cpu_baseline leg -- the
    fp64 oracle on the same inputs, timed, with its outputs compared."""
    import ctypes
    import platform
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    threads = len(os.sched_getaffinity(0))
    cpu = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    oracle = None
    if with_cpu:
        import oracle

    def emit(name, shape, seed, by, ts, extra, oracle_run=None):
        med = float(np.median(ts))
        line = {"config": name, "shape": shape, "seed": seed, "algorithmic_bytes": by,
                "us_median": round(med, 2), "us_p10": round(float(np.percentile(ts, 10)), 2),
                "us_p90": round(float(np.percentile(ts, 90)), 2),
                "GB/s": round(by / (med * 1e-6) / 1e9, 1),
                "frac_of_8TB/s": round(by / (med * 1e-6) / 8e12, 4)}
        line.update(extra)
        if oracle_run is not None:
            t0 = time.perf_counter()
            cmp = oracle_run()
            line["oracle"] = {"seconds": round(time.perf_counter() - t0, 3), "threads": threads,
                              "cpu": cpu, "vs_gpu": cmp}
        print(json.dumps(line), flush=True)

    # 1. merge_states fp16 S=64 N=4 H=8 D=128
    c1 = inputs.merge_states_case(1001, S=64, N=4, H=8, D=128, dtype="f16")
    v1, s1 = to_dev(c1["v"], "f16", torch), torch.from_numpy(c1["s"]).cuda()
    vo1 = torch.empty((64, 8, 128), dtype=torch.float16, device="cuda")
    so1 = torch.empty((64, 8), dtype=torch.float32, device="cuda")
    call = Raw(mi, "mi_merge_states", v1, s1, vo1, so1, 64, 4, 8, 128, mi.MI_F16, mi.MI_F16, st)
    ts = _times_us(torch, lambda i: call(), iters)
    def cmp1():
        rv, rs = oracle.merge_states(c1["v"], c1["s"], "f16", threads)
        return _agreement(vo1.float().cpu().numpy(), rv, "f16", so1.cpu().numpy(), rs)
    emit("merge_states", "f16 S=64 N=4 H=8 D=128 (10% empty states)", 1001,
         64 * 8 * (4 * 256 + 16 + 256 + 4), ts, {}, cmp1 if oracle else None)

    # The per-call floor of this timing: one near-empty launch (a 4 KiB plain
    # read), for scale beside the small workload above.
    fl = torch.zeros(1024, dtype=torch.int32, device="cuda")
    flx = torch.zeros(1, dtype=torch.int32, device="cuda")
    fcall = Raw(mi, "mi_stream_read", fl, 4096, flx, st)
    ts = _times_us(torch, lambda i: fcall(), iters)
    print(json.dumps({"config": "launch_floor", "shape": "mi_stream_read over 4 KiB (one launch, "
                      "no work to speak of): the per-call floor of this timing",
                      "us_median": round(float(np.median(ts)), 2),
                      "us_p10": round(float(np.percentile(ts, 10)), 2),
                      "us_p90": round(float(np.percentile(ts, 90)), 2)}), flush=True)

    # 2. merge_state bf16 S=32768 H=32 D=128, inputs rotated over two copies
    c2 = inputs.merge_state_case(1002, S=32768, H=32, D=128, dtype="bf16")
    cp = [(to_dev(c2["va"], "bf16", torch), torch.from_numpy(c2["sa"]).cuda(),
           to_dev(c2["vb"], "bf16", torch), torch.from_numpy(c2["sb"]).cuda()) for _ in range(2)]
    vo2 = torch.empty_like(cp[0][0])
    so2 = torch.empty_like(cp[0][1])
    calls = [Raw(mi, "mi_merge_state", a, b, c_, d, vo2, so2, 32768 * 32, 1, 128, mi.MI_BF16,
                 mi.MI_BF16, st) for a, b, c_, d in cp]
    ts = _times_us(torch, lambda i: calls[i % 2](), iters)

    def cmp2():
        rv, rs = oracle.merge_state(c2["va"], c2["sa"], c2["vb"], c2["sb"], "bf16", threads)
        return _agreement(vo2.float().cpu().numpy(), rv, "bf16", so2.cpu().numpy(), rs)
    emit("merge_state", "bf16 S=32768 H=32 D=128 (1% of rows empty)", 1002,
         32768 * 32 * (3 * 256 + 12), ts, {}, cmp2 if oracle else None)
    del cp, calls, vo2, so2
    torch.cuda.empty_cache()

    def decode_case(name, seed, ctx, plan, per_sequence=False):
        case = inputs.paged_kv_case(seed, ctx, 32, 8, 128, 16, dtype="f16")
        B = len(ctx)
        q = to_dev(case["q"], "f16", torch)
        k0, v0 = to_dev(case["k"], "f16", torch), to_dev(case["v"], "f16", torch)
        kv = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(3)]
        pt = torch.from_numpy(case["page_table"]).cuda()
        cl = torch.from_numpy(ctx).cuda()
        P = case["k"].shape[0]
        scale = float(case["sm_scale"])
        o = torch.empty((B, 32, 128), dtype=torch.float16, device="cuda")
        lse = torch.empty((B, 32), dtype=torch.float32, device="cuda")
        cnt = torch.zeros((B, 8), dtype=torch.int32, device="cuda")
        if per_sequence:
            indptr = mi.plan_splits_varlen(ctx, 8, 16)
            total = int(indptr[-1])
            ipd = torch.from_numpy(indptr).cuda()
            op = torch.empty((total, 32, 128), dtype=torch.float32, device="cuda")
            lp = torch.empty((total, 32), dtype=torch.float32, device="cuda")
            calls = [Raw(mi, "mi_split_kv_decode_varlen", q, k, v, pt, pt.shape[1], cl, B, 32, 8,
                         128, 16, P, ipd, total, scale, mi.MI_F16, op, lp, cnt, o, lse, mi.MI_F16,
                         st) for k, v in kv]
            splits, parts_rows = f"per sequence, total {total}", total
        else:
            n = mi.plan_splits(ctx, 8, 16)
            op = torch.empty((B, 32, n, 128), dtype=torch.float32, device="cuda")
            lp = torch.empty((B, 32, n), dtype=torch.float32, device="cuda")
            calls = [Raw(mi, "mi_split_kv_decode_fused", q, k, v, pt, pt.shape[1], cl, B, 32, 8,
                         128, 16, P, n, scale, mi.MI_F16, op, lp, cnt, o, lse, mi.MI_F16, st)
                     for k, v in kv]
            splits, parts_rows = n, B * n
        t0 = time.perf_counter()
        for _ in range(100):
            plan()
        plan_us = (time.perf_counter() - t0) * 1e4      # host µs per plan (outside the events)
        ts = _times_us(torch, lambda i: calls[i % 4](), iters)
        by = (int(ctx.astype(np.int64).sum()) * 8 * 128 * 2 * 2 + q.numel() * 2
              + pt.numel() * 4 + B * 4 + (2 * parts_rows * 32 * 129 * 4 if parts_rows > B else 0)
              + B * 32 * (256 + 4))

        def cmp():
            ro, rs = oracle.attention(case["q"], case["k"], case["v"], case["page_table"], ctx,
                                      case["sm_scale"], "f16", "f16", threads)
            return _agreement(o.float().cpu().numpy(), ro, "f16", lse.cpu().numpy(), rs)
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        form = "one launch" if parts_rows * 8 <= 2 * cus else "two launches"
        emit(name, f"f16 B={B} Hq=32 Hkv=8 D=128 PAGE=16, fused entry ({form})", seed, by, ts,
             {"num_splits": splits, "host_plan_us": round(plan_us, 2)}, cmp if oracle else None)

    # 3. decode B=1 ctx=32768 (64 splits); 4. the mixed batch (uniform and per-sequence plans)
    ctx3 = np.array([32768], np.int32)
    decode_case("split_kv_decode_b1_32k", 1003, ctx3, lambda: mi.plan_splits(ctx3, 8, 16))
    ctx4 = inputs.mixed_ctx_lens(1004, 32)
    decode_case("split_kv_decode_mixed_b32", 1004, ctx4, lambda: mi.plan_splits(ctx4, 8, 16))
    decode_case("split_kv_decode_mixed_b32_per_sequence", 1004, ctx4,
                lambda: mi.plan_splits_varlen(ctx4, 8, 16), per_sequence=True)
    torch.cuda.empty_cache()

    # 5. cascade: 64 requests x (8192 shared + 512 own), two launches
    cas = inputs.cascade_case(1005)
    R, Hq, Hkv = cas["R"], cas["Hq"], cas["Hkv"]
    cq = to_dev(cas["q"], "bf16", torch)
    k0, v0 = to_dev(cas["k"], "bf16", torch), to_dev(cas["v"], "bf16", torch)
    kv = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(3)]
    pages = torch.from_numpy(cas["prefix_pages"]).cuda()
    tab = torch.from_numpy(cas["suffix_table"]).cuda()
    lens = torch.from_numpy(cas["suffix_lens"]).cuda()
    n = mi.plan_splits(cas["suffix_lens"], Hkv, 16)
    wsb = mi.prefix_attention_workspace_bytes(R, Hq, Hkv, 128, cas["prefix_len"])
    ws = torch.empty(wsb // 4, dtype=torch.float32, device="cuda")
    op = torch.empty((R, Hq, n, 128), dtype=torch.float32, device="cuda")
    lp = torch.empty((R, Hq, n), dtype=torch.float32, device="cuda")
    cnt = torch.zeros((R, Hkv), dtype=torch.int32, device="cuda")
    o = torch.empty((R, Hq, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((R, Hq), dtype=torch.float32, device="cuda")
    calls = [Raw(mi, "mi_cascade_decode", cq, k, v, pages, cas["prefix_len"], tab, tab.shape[1],
                 lens, R, Hq, Hkv, 128, 16, cas["k"].shape[0], n, float(cas["sm_scale"]),
                 mi.MI_BF16, ws, wsb, op, lp, cnt, o, lse, mi.MI_BF16, st) for k, v in kv]
    ts = _times_us(torch, lambda i: calls[i % 4](), iters)
    n_ch = wsb // (R * Hq * 129 * 4)
    rows = R * Hq
    by = (cas["prefix_len"] * Hkv * 128 * 2 * 2 + R * 512 * Hkv * 128 * 2 * 2 + 2 * cq.numel() * 2
          + pages.numel() * 4 + tab.numel() * 4 + R * 4 + 2 * rows * n_ch * 129 * 4
          + (2 if n > 1 else 1) * rows * n * 129 * 4 + rows * (256 + 4))

    def cmp5():
        ro, rs = oracle.attention(cas["q"], cas["k"], cas["v"], cas["full_table"], cas["full_lens"],
                                  cas["sm_scale"], "bf16", "bf16", threads)
        return _agreement(o.float().cpu().numpy(), ro, "bf16", lse.cpu().numpy(), rs)
    emit("cascade", "bf16 64 x (8192 shared + 512 own) Hq=32 Hkv=8 D=128, two launches", 1005,
         by, ts, {"prefix_chunks": n_ch, "suffix_splits": n}, cmp5 if oracle else None)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import torch

    import lse_attention_state_amd as mi
    from lse_attention_state_amd import inputs

    if args.copy_calibration:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "launches": 5}))
        return

    if args.ceiling:
        ceiling(torch, mi, max(args.steps, 20))
        return

    if args.configs:
        configs_report(torch, mi, inputs, max(args.steps, 100), not args.no_cpu_baseline)
        return

    if args.sweep:
        sweep(torch, mi, inputs, max(args.steps, 20), with_cpu=not args.no_cpu_baseline)
        return

    parts, host = build_workload(torch, mi, inputs)
    timer = Timer(torch)

    def step(i, timed):
        for p in parts:
            if "host" in p:
                p["host"](i)        # host-side planning, outside the event brackets
            if timed:
                timer.start(p["name"])
            p["run"](i)
            if timed:
                timer.stop(p["name"])

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    # Timed region 1: the steps alone (no events between kernels).
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        step(i, False)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = 1000.0 * wall / args.steps
    gpu_ms_per_step = e0.elapsed_time(e1) / args.steps

    # Timed region 2: the same steps with an event pair around every kernel.
    for i in range(args.steps):
        step(i, True)
    torch.cuda.synchronize()

    # Back-to-back loops timed with one event pair around the whole loop (mean
    # per call), so the GPU never waits for the host between launches.
    def loop_us(fn, n):
        fn(0)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(n):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return 1000.0 * a.elapsed_time(b) / n

    host["plan"](0)
    extra = {
        # decode end to end with rotated K/V copies: single launch, two launches
        "decode": loop_us(lambda i: host["fused_calls"][i % 4](), args.steps),
        "decode_two_launch": loop_us(lambda i: host["decode_calls"][i % 4](), args.steps),
        "split_kv_partial": loop_us(lambda i: host["partial_calls"][i % 4](), args.steps),
        "combine": loop_us(lambda i: host["combine_call"](), args.steps),
        # the cascade's prefix level alone (MFMA contraction + chunk merge), and
        # the cascade as four launches (prefix, chunk merge, suffix, level merge)
        "cascade_prefix_level": loop_us(lambda i: host["prefix_call"](), args.steps),
        "cascade_four_launch": loop_us(lambda i: [c_() for c_ in host["four_launch"]], args.steps),
        "cascade": loop_us(lambda i: host["cascade_call"](), args.steps),
        "merge_states": loop_us(lambda i: host["mss_call"](), args.steps),
        "merge_state": loop_us(lambda i: host["ms_calls"][i % 2](), args.steps),
    }
    # The practical read rate in the same run: the plain streaming read over
    # 1 GiB (two buffers rotated), as context for the fractions of the peak.
    rd = [torch.ones(1 << 28, dtype=torch.int32, device="cuda") for _ in range(2)]
    rd_x = torch.zeros(1, dtype=torch.int32, device="cuda")
    import ctypes
    st_ = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rd_calls = [Raw(mi, "mi_stream_read", b, 1 << 30, rd_x, st_) for b in rd]
    read_gbs = (1 << 30) / (loop_us(lambda i: rd_calls[i % 2](), 20) * 1e-6) / 1e9
    del rd, rd_calls
    torch.cuda.empty_cache()

    step_bytes = sum(p["bytes"] for p in parts)
    step_gbs = step_bytes / (ms_per_step / 1000.0) / 1e9
    per = []
    for p in parts:
        us = timer.mean_us(p["name"])
        gbs = p["bytes"] / (us * 1e-6) / 1e9
        entry = {"kernel": p["name"], "shape": p["shape"], "us": round(us, 2),
                 "bytes": p["bytes"], "GB/s": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)}
        if "flops" in p:
            tf = p["flops"] / (us * 1e-6) / 1e12
            entry.update({"TFLOP/s": round(tf, 1), "mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)})
        per.append(entry)
    by_name = {e["kernel"]: e for e in per}

    def roofline_of(entry):
        return {"bound": "hbm", "achieved": entry["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": entry["frac"], "traffic": counter_traffic(entry["kernel"]),
                "kernel": entry["kernel"]}

    # The headline: the N-state merge at its streaming size, event-timed per
    # launch inside the steps; beside it the decode at B=1, ctx=32768.
    mss = by_name["merge_states"]
    dom = max(per, key=lambda r: r["us"])
    decode_us = extra["decode"]
    dec_bytes = by_name["split_kv_decode"]["bytes"]
    line = {
        "metric": METRIC, "value": mss["GB/s"], "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "storage_dtypes": {"merge_states": "f16", "merge_state": "bf16",
                           "split_kv_decode": "f16", "cascade": "bf16"},
        "data": "synthetic",
        "config": {"workload": ("value: merge_states f16 S=65536 N=4 H=8 D=128 (10% empty "
                                "states), per launch inside the step; step: merge_state bf16 "
                                "S=32768 H=32 D=128 + merge_states + split-KV decode f16 B=1 "
                                f"ctx=32768 Hq=32 Hkv=8 D=128 PAGE=16 splits={host['splits']} + "
                                "cascade bf16 64 x (8192 shared + 512) Hq=32 Hkv=8 D=128"),
                   "step_bytes": step_bytes},
        "frac_of_peak": mss["frac"],
        "merge_states_us": mss["us"],
        "decode_us": round(decode_us, 2),
        "decode_GBs": round(dec_bytes / (decode_us * 1e-6) / 1e9, 1),
        "decode_frac": round(dec_bytes / (decode_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "decode_us_in_step": by_name["split_kv_decode"]["us"],
        "decode_two_launch_us": round(extra["decode_two_launch"], 2),
        "decode_pass1_us": round(extra["split_kv_partial"], 2),
        "decode_combine_us": round(extra["combine"], 2),
        "merge_states_back_to_back_us": round(extra["merge_states"], 2),
        "merge_state_back_to_back_us": round(extra["merge_state"], 2),
        "cascade_prefix_level_us": round(extra["cascade_prefix_level"], 2),
        "cascade_prefix_level_TFLOPs": round(host["prefix_flops"] / (extra["cascade_prefix_level"] * 1e-6) / 1e12, 1),
        "cascade_four_launch_us": round(extra["cascade_four_launch"], 2),
        "cascade_two_launch_us": round(extra["cascade"], 2),
        "step": {"bytes": step_bytes, "GB/s": round(step_gbs, 1),
                 "frac": round(step_gbs / HBM_PEAK_GBS, 4),
                 "gpu_ms_per_step": round(gpu_ms_per_step, 4)},
        "kernels": per,
        "roofline": roofline_of(dom),
        "rooflines": {"merge_states": roofline_of(mss),
                      "split_kv_decode": roofline_of(by_name["split_kv_decode"])},
        "practical_read": {"kernel": "mi_stream_read", "bytes": 1 << 30,
                           "GB/s": round(read_gbs, 1), "frac": round(read_gbs / HBM_PEAK_GBS, 4),
                           "roofline_achieved_over_it": round(dom["GB/s"] / read_gbs, 4)},
    }
    if not args.no_cpu_baseline:
        import oracle
        line["cpu_baseline"] = cpu_baseline(host, oracle)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
