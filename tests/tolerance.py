"""Parity bar between a GPU product and the oracle.

Per element, with both results read exactly as BF16 values:

    |C - C_ref| <= 2^-7 * |C_ref| + 2^-10 * sqrt(K) * sigma

sigma = 1 for BF16 operands drawn from [-1, 1] (the bound as stated for the
workloads). For block-scaled FP4 operands the absolute term is taken for the
problem normalised to the same second moment: sigma = sigma_A * sigma_B with
sigma_X = sqrt(3) * rms(decoded X), which is 1 for uniform[-1, 1] data.
Why the bound holds for a correct FP32-accumulating kernel: the relative term
covers the final BF16 rounding (half an ulp is 2^-8 relative; rounding the FP32
sum that was itself rounded can cost up to one ulp, 2^-7); the absolute term
covers FP32 accumulation error, which grows like sqrt(K) * 2^-24 * (scale of
the products), far below 2^-10 * sqrt(K) * sigma.

NaN or infinity anywhere in C fails the check.
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def sigma_of(decoded: np.ndarray) -> float:
    """sqrt(3) * rms of a decoded operand (1 for uniform[-1, 1])."""
    d = np.asarray(decoded, dtype=np.float64)
    return float(np.sqrt(3.0 * np.mean(d * d))) if d.size else 1.0


def bound(c_ref: np.ndarray, K: int, sigma: float = 1.0) -> np.ndarray:
    return 2.0 ** -7 * np.abs(c_ref) + 2.0 ** -10 * np.sqrt(max(K, 0)) * sigma


class ParityResult:
    def __init__(self, ok, n_bad, worst_ratio, first_bad, max_abs_err):
        self.ok = ok
        self.n_bad = n_bad
        self.worst_ratio = worst_ratio  # max |err| / bound; <= 1 passes
        self.first_bad = first_bad
        self.max_abs_err = max_abs_err

    def __bool__(self):
        return bool(self.ok)

    def __repr__(self):
        return ("ParityResult(ok=%s, n_bad=%d, worst_ratio=%.4g, first_bad=%s, max_abs_err=%.4g)"
                % (self.ok, self.n_bad, self.worst_ratio, self.first_bad, self.max_abs_err))


def check(c_bits, c_ref_bits, K: int, sigma: float = 1.0) -> ParityResult:
    c = bf16_bits_to_f64(c_bits)
    r = bf16_bits_to_f64(c_ref_bits)
    if c.shape != r.shape:
        raise ValueError("shape mismatch %s vs %s" % (c.shape, r.shape))
    if c.size == 0:
        return ParityResult(True, 0, 0.0, None, 0.0)
    err = np.abs(c - r)
    b = bound(r, K, sigma)
    finite = np.isfinite(c)
    bad = (~finite) | (err > b)
    n_bad = int(bad.sum())
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(finite, err / b, np.inf)
    first = None
    if n_bad:
        first = tuple(int(i) for i in np.argwhere(bad)[0])
    return ParityResult(n_bad == 0, n_bad, float(np.max(ratio)), first,
                        float(np.max(np.where(finite, err, np.inf))))
