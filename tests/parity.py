"""Comparison rules for GPU results against the fp64 oracle.

Floating point outputs (v / o in fp16, bf16 or fp32):
    |gpu - ref| <= max(ATOL + RTOL * |ref|, ulp_out(ref) / 2 + SLACK * |ref|)
with ATOL = RTOL = 2e-3. The second term is one correct rounding of the
result into the output type (half an ulp) plus the error of the fp32
arithmetic before that rounding (SLACK = 2^-16 relative). It only matters
for bf16 with |ref| >= 2, where half an ulp (2^-9 to 2^-8 relative) already exceeds
the stated tolerance; for fp16 and fp32 the first term always dominates at
these magnitudes. A result rounded to the wrong neighbour fails it. Elements
that pass only by the rounding term are counted and reported.

LSE (fp32, base 2): |gpu - ref| <= 1e-4, and -inf must match -inf exactly.
No output may hold NaN.
"""
import math

import numpy as np
import torch

ATOL = 2e-3
RTOL = 2e-3
LSE_TOL = 1e-4
SLACK = 2.0 ** -16

_MANT = {torch.float16: 10, torch.bfloat16: 7, torch.float32: 23}
_MIN_EXP = {torch.float16: -14, torch.bfloat16: -126, torch.float32: -126}

TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def to_device(bits: np.ndarray, dtype: str, device="cuda"):
    """Host bits (uint16 for 16-bit types, float32 for f32) -> device tensor of that dtype."""
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.float32)).to(device)
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(TORCH_DT[dtype]).to(device)


def host64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def ulp(ref: np.ndarray, dtype) -> np.ndarray:
    a = np.abs(ref)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, _MIN_EXP[dtype])
    return np.exp2(e - _MANT[dtype])


def check_values(gpu: torch.Tensor, ref: np.ndarray, what: str = "v"):
    got = host64(gpu)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert not np.isnan(got).any(), f"{what}: NaN in GPU output"
    assert not np.isnan(ref).any(), f"{what}: NaN in oracle output"
    err = np.abs(got - ref)
    stated = ATOL + RTOL * np.abs(ref)
    bound = np.maximum(stated, 0.5 * ulp(ref, gpu.dtype) + SLACK * np.abs(ref))
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} / {err.size} outside tolerance; worst at {i}: "
                             f"gpu={got[i]!r} ref={ref[i]!r} err={err[i]:.3e} bound={bound[i]:.3e}")
    return {"max_abs": float(err.max(initial=0.0)), "ulp_only": int((err > stated).sum())}


def check_lse(gpu: torch.Tensor, ref: np.ndarray, what: str = "s"):
    got = host64(gpu)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert not np.isnan(got).any(), f"{what}: NaN in GPU LSE"
    ninf_ref = np.isneginf(ref)
    ninf_got = np.isneginf(got)
    assert np.array_equal(ninf_ref, ninf_got), f"{what}: -inf pattern differs"
    fin = ~ninf_ref
    if fin.any():
        err = np.abs(got[fin] - ref[fin])
        assert err.max() <= LSE_TOL, f"{what}: max |ds| = {err.max():.3e} > {LSE_TOL}"
        return float(err.max())
    return 0.0


def sm_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)
