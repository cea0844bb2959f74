"""Seeded synthetic operands shared by the tests, the smoke check and the bench.

This module only draws inputs. It holds none of the product's arithmetic: no
decoding, no multiply, no accumulation and no output rounding. Its one
conversion, float32 -> BF16 for the *inputs*, is torch's own cast (round to
nearest even), as the workloads prescribe ("i.i.d. uniform[-1,1] from a seed
then rounded to BF16").

Every array is returned as raw bits in numpy: BF16 as ``uint16``; packed E2M1
codes (two per byte, even k in the low nibble) and E4M3 scale bytes as
``uint8``. Generators are ``numpy.random.Generator(PCG64(seed))``.

Workload recipes
  * BF16: i.i.d. uniform[-1, 1) float32 -> BF16.
  * FP4 codes: every byte uniform over 0..255, i.e. both nibbles uniform over
    the 16 E2M1 codes (including -0).
  * FP4 scales: one byte per 16 consecutive K of a row, ``((u + 7) << 3) | m``
    with integer u uniform in [-4, 4] and m uniform in 0..7, i.e. the E4M3
    value 2^u * (1 + m/8).
  * MXFP4 (microscaled FP4): the same codes; one E8M0 byte per 32
    consecutive K of a row, 127 + u with integer u uniform in [-4, 4].
  * Rotation sets: seed = 1000 * config_index + set_index.
"""
from __future__ import annotations

import numpy as np
import torch


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def to_bf16_bits(x) -> np.ndarray:
    """float array -> BF16 bit patterns via torch's round-to-nearest-even cast."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_uniform(rows: int, cols: int, seed: int, lo: float = -1.0, hi: float = 1.0) -> np.ndarray:
    """(rows, cols) BF16 bits, i.i.d. uniform[lo, hi) rounded to BF16."""
    x = rng(seed).uniform(lo, hi, size=(rows, cols)).astype(np.float32)
    return to_bf16_bits(x)


def bf16_sixteenths(rows: int, cols: int, seed: int, jmax: int = 16) -> np.ndarray:
    """(rows, cols) BF16 bits holding j/16 with integer j uniform in [-jmax, jmax].

    With jmax <= 16 every product is a multiple of 2^-8 with magnitude <= 1, so
    every partial sum of up to 2^15 terms is exact in binary32.
    """
    j = rng(seed).integers(-jmax, jmax + 1, size=(rows, cols))
    return to_bf16_bits(j.astype(np.float32) / 16.0)


def bf16_sixteenths_large(rows: int, cols: int, seed: int) -> np.ndarray:
    """(rows, cols) BF16 bits holding j/16, integer j uniform in [-16, 15], for
    arrays of billions of elements: byte draws mapped through a 32-entry table
    of BF16 bit patterns (torch's cast of j/16), in slices, without float
    temporaries. Products of such values are exact as for ``bf16_sixteenths``."""
    table = to_bf16_bits(np.arange(-16, 16, dtype=np.float32) / 16.0)
    g = rng(seed)
    out = np.empty(rows * cols, dtype=np.uint16)
    step = 1 << 24
    for i in range(0, out.size, step):
        n = min(step, out.size - i)
        j = np.frombuffer(g.bytes(n), dtype=np.uint8) & 31
        out[i:i + n] = table[j]
    return out.reshape(rows, cols)


def bf16_identity(n: int) -> np.ndarray:
    return to_bf16_bits(np.eye(n, dtype=np.float32))


def permutation(n: int, seed: int) -> np.ndarray:
    return rng(seed).permutation(n)


def bf16_permutation_matrix(perm: np.ndarray) -> np.ndarray:
    """P with P[n, perm[n]] = 1, so (A @ P^T)[:, n] = A[:, perm[n]]."""
    n = perm.size
    P = np.zeros((n, n), dtype=np.float32)
    P[np.arange(n), perm] = 1.0
    return to_bf16_bits(P)


def fp4_codes(rows: int, K: int, seed: int) -> np.ndarray:
    """(rows, K/2) bytes, both nibbles uniform over the 16 E2M1 codes."""
    if K % 2:
        raise ValueError("K must be even")
    return rng(seed).integers(0, 256, size=(rows, K // 2), dtype=np.uint8)


def e4m3_scales(rows: int, K: int, seed: int, u_lo: int = -4, u_hi: int = 4,
                m_lo: int = 0, m_hi: int = 7) -> np.ndarray:
    """(rows, K/16) E4M3 bytes ((u + 7) << 3) | m, u in [u_lo, u_hi], m in [m_lo, m_hi]."""
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    g = rng(seed)
    u = g.integers(u_lo, u_hi + 1, size=(rows, K // 16))
    m = g.integers(m_lo, m_hi + 1, size=(rows, K // 16))
    return (((u + 7) << 3) | m).astype(np.uint8)


def fp4_operand(rows: int, K: int, seed: int):
    """(codes, scales) for one block-scaled FP4 operand of the workload recipe."""
    return fp4_codes(rows, K, seed), e4m3_scales(rows, K, seed + 7919)


def e8m0_scales(rows: int, K: int, seed: int, u_lo: int = -4, u_hi: int = 4) -> np.ndarray:
    """(rows, K/32) E8M0 bytes 127 + u with integer u uniform in [u_lo, u_hi],
    i.e. the power-of-two scale 2^u of each 32-element block."""
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    return (127 + rng(seed).integers(u_lo, u_hi + 1, size=(rows, K // 32))).astype(np.uint8)


def mxfp4_operand(rows: int, K: int, seed: int):
    """(codes, scales) for one microscaled FP4 operand: the FP4 workload's codes
    with an E8M0 scale 2^u, u uniform in [-4, 4], per 32 elements."""
    return fp4_codes(rows, K, seed), e8m0_scales(rows, K, seed + 7919)


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """(rows, K) codes 0..15 -> (rows, K/2) bytes, even k in the low nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    if codes.shape[1] % 2:
        raise ValueError("K must be even")
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def seed_for(config_index: int, set_index: int) -> int:
    return 1000 * config_index + set_index
