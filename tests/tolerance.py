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


# ---- fused epilogue (bias, activation) ------------------------------------
#
# y = act(z), z = sum + bias. With y_ref the oracle's BF16 result and z_ref its
# binary64 pre-activation value:
#
#   |y - y_ref| <= 2^-7 |y_ref| + L (2^-10 sqrt(K) sigma + 2^-20 |z_ref|) + e_act
#
# 2^-7 |y_ref| covers the two output roundings (GPU and oracle, half an ulp
# each); L, the activation's largest slope (1 for the identity and ReLU, below
# 1.13 for the tanh-form GELU), carries the sum's FP32 error (the plain bound's
# absolute term) and the FP32 rounding of the bias addition through the
# activation; e_act = 2^-18 (1 + |z_ref|) for the GELU, whose FP32 evaluation
# (exponential and division) errs by a few units in the last place.
LIPSCHITZ = {0: 1.0, 1: 1.0, 2: 1.13}


def fused_bound(y_ref: np.ndarray, z_ref: np.ndarray, K: int, act: int, sigma: float = 1.0) -> np.ndarray:
    z = np.abs(np.asarray(z_ref, dtype=np.float64))
    b = 2.0 ** -7 * np.abs(y_ref) + LIPSCHITZ[act] * (2.0 ** -10 * np.sqrt(max(K, 0)) * sigma + 2.0 ** -20 * z)
    if act == 2:
        b = b + 2.0 ** -18 * (1.0 + z)
    return b


def check_fused(c_bits, y_ref_bits, z_ref, K: int, act: int, sigma: float = 1.0) -> ParityResult:
    c = bf16_bits_to_f64(c_bits)
    r = bf16_bits_to_f64(y_ref_bits)
    z = np.asarray(z_ref, dtype=np.float64)
    if c.shape != r.shape or z.shape != r.shape:
        raise ValueError("shape mismatch %s vs %s vs %s" % (c.shape, r.shape, z.shape))
    if c.size == 0:
        return ParityResult(True, 0, 0.0, None, 0.0)
    err = np.abs(c - r)
    b = fused_bound(r, z, K, act, sigma)
    finite = np.isfinite(c)
    bad = (~finite) | (err > b)
    n_bad = int(bad.sum())
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(finite, err / np.maximum(b, 1e-300), np.inf)
    first = tuple(int(i) for i in np.argwhere(bad)[0]) if n_bad else None
    return ParityResult(n_bad == 0, n_bad, float(np.max(ratio)), first,
                        float(np.max(np.where(finite, err, np.inf))))
