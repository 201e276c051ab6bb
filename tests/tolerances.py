"""Error metrics and bounds used by the parity tests.

fp32 outputs: max |gpu - ref| / max |ref| over the tensor (per row for
logits) <= 1e-4 -- elementwise relative error is undefined where the
reference cancels to ~0.

bf16 outputs (identical bf16 inputs on both sides; the reference is the fp64
value): |gpu - ref| <= 2e-2, except where one bf16 step at |ref| is itself
wider than that (|ref| >= 8), where the bound is one bf16 step of |ref|:
rounding a correct fp32 result to bf16 alone moves it by up to half a step.
"""
import numpy as np

F32_REL = 1e-4
BF16_ABS = 2e-2


def bf16_step(r):
    """Spacing of bf16 numbers at |r| (2^(e - 7) for |r| in [2^e, 2^(e+1)))."""
    r = np.abs(np.asarray(r, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(r, 1e-30)))
    return np.exp2(e - 7)


def check_f32(gpu, ref, rel=F32_REL, axis=None, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.isfinite(gpu).all(), f"{what}: non-finite GPU output"
    num = np.max(np.abs(gpu - ref), axis=axis)
    den = np.max(np.abs(ref), axis=axis)
    err = np.max(num / np.maximum(den, 1e-30))
    assert err <= rel, f"{what}: max rel err {err:.3e} > {rel:.1e}"
    return float(err)


def check_bf16(gpu, ref, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.isfinite(gpu).all(), f"{what}: non-finite GPU output"
    err = np.abs(gpu - ref)
    bound = np.maximum(BF16_ABS, bf16_step(ref))
    worst = float(np.max(err / bound))
    assert worst <= 1.0, f"{what}: max abs err {err.max():.3e} exceeds its bound (ratio {worst:.2f})"
    return float(err.max())
