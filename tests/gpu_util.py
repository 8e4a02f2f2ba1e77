"""Shared helpers of the GPU parity tests: tolerances and error metrics."""
import numpy as np

import oracle

# bf16 outputs vs the fp64 oracle: max |err| <= 1e-2 and L1 ratio sum|err|/sum|ref| <= 2e-3.
# FP8 paths (the oracle dequantises the same bytes): max |err| <= 3e-2, and the same L1
# ratio bound is also enforced.
BF16_MAX_ABS, BF16_L1 = 1e-2, 2e-3
FP8_MAX_ABS, FP8_L1 = 3e-2, 2e-3
LSE_ABS = 2e-3


def errors(got: np.ndarray, ref: np.ndarray):
    d = np.abs(got.astype(np.float64) - ref)
    return float(d.max()), float(d.sum() / max(np.abs(ref).sum(), 1e-300))


def assert_close(got, ref, max_abs, l1, what=""):
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    mx, r = errors(got, ref)
    print(f"{what}: max_abs={mx:.3e} l1_ratio={r:.3e}", flush=True)
    assert mx <= max_abs and r <= l1, f"{what}: max_abs={mx:.3e} (<= {max_abs}) l1={r:.3e} (<= {l1})"


def assert_close_stress(got, ref, max_abs, l1, what=""):
    """Stress cases with peaked softmax have outputs up to ~5 in magnitude, where the final
    rounding of a correct result to bf16 alone moves it by up to half an ulp (0.0156 at
    [4, 8)), more than 1e-2.  So the max-abs bound applies to the kernel's error before that
    rounding: |got - ref| - ulp/2 <= max_abs, with the bf16 ulp of max(|got|, |ref|) (the
    larger binade, in case the rounding crossed a power of two).  The L1 ratio is taken
    against the exact fp64 result."""
    a = np.maximum(np.abs(ref), np.abs(got))
    half_ulp = np.exp2(np.floor(np.log2(np.maximum(a, 2.0 ** -126))) - 8)
    excess = float(np.max(np.abs(got - ref) - half_ulp))
    _, r = errors(got, ref)
    print(f"{what}: max error beyond half a bf16 ulp={excess:.3e} l1_ratio={r:.3e}", flush=True)
    assert np.isfinite(got).all() and excess <= max_abs and r <= l1, what


def bf16_out(t) -> np.ndarray:
    """Device bf16 tensor -> float64 host array (exact)."""
    import torch
    return oracle.bf16_to_f64(t.detach().view(torch.int16).cpu().numpy().view(np.uint16))
