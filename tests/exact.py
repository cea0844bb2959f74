"""Exact rational arithmetic used to pin the oracle (CPU, test-only).

Independent of the oracle's C code: values are decoded with torch's own dtypes
(bfloat16, float8_e4m3fn) or with the E2M1 value list of the FP4 page, summed
as ``fractions.Fraction`` and rounded to BF16 by the definition of round to
nearest, ties to even.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import torch

# E2M1 magnitudes by the low three code bits, as listed in "NVFP4 GEMM on
# Blackwell", section "NVFP4 Datatype"; bit 3 is the sign.
E2M1_MAGNITUDE = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2),
                  Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def e2m1_fraction(code: int) -> Fraction:
    v = E2M1_MAGNITUDE[code & 7]
    return -v if code & 8 else v


def bf16_bits_to_fractions(bits) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    vals = t.view(torch.bfloat16).to(torch.float64).numpy()
    return np.vectorize(lambda v: Fraction(float(v)), otypes=[object])(vals)


def e4m3_fraction(byte: int) -> Fraction:
    v = torch.tensor([byte], dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).item()
    return Fraction(v)


def rne_bf16(q: Fraction) -> int:
    """Exact value -> BF16 bit pattern, round to nearest, ties to even.

    BF16 has 8 significant bits and binary32's exponent range: for
    2^e <= |q| < 2^(e+1) the spacing is 2^(e-7), never below 2^-133.
    """
    sign = 0x8000 if q < 0 else 0
    a = abs(q)
    if a == 0:
        return sign
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    spacing = Fraction(2) ** max(e - 7, -133)
    n = a / spacing
    lo = n.numerator // n.denominator
    rem = n - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    value = lo * spacing
    if value >= Fraction(2) ** 128:
        return sign | 0x7F80
    f = torch.tensor([float(value)], dtype=torch.float32)  # exact: value is a BF16 value
    return sign | (int(f.to(torch.bfloat16).view(torch.int16).item()) & 0x7FFF)


def gemm_exact_bits(Af: np.ndarray, Bf: np.ndarray) -> np.ndarray:
    """C = rne_bf16(A @ B^T) with A, B object arrays of Fractions."""
    M, K = Af.shape
    N = Bf.shape[0]
    out = np.empty((M, N), dtype=np.uint16)
    for m in range(M):
        for n in range(N):
            s = Fraction(0)
            for k in range(K):
                s += Af[m, k] * Bf[n, k]
            out[m, n] = rne_bf16(s)
    return out


def fp4_fractions(Q: np.ndarray, SF: np.ndarray, K: int) -> np.ndarray:
    rows = Q.shape[0]
    out = np.empty((rows, K), dtype=object)
    scale_cache = {}
    for r in range(rows):
        for k in range(K):
            byte = int(Q[r, k // 2])
            code = (byte >> 4) if (k & 1) else (byte & 15)
            sb = int(SF[r, k // 16])
            if sb not in scale_cache:
                scale_cache[sb] = e4m3_fraction(sb)
            out[r, k] = e2m1_fraction(code) * scale_cache[sb]
    return out
