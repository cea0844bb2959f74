"""Pins of the oracle's microscaled FP4 (MXFP4) product: E8M0 decoding against
torch's float8_e8m0fnu for all 256 bytes, exact rational brute force on tiny
shapes, and the identity with the NVFP4 product when every scale is one (the
same codes and nibble order). CPU only.

The format is not defined by the pages (their FP4 variant carries an E4M3
scale per 16 elements, "NVFP4 GEMM on Blackwell", "NVFP4 Datatype"); it is the
microscaling convention the gfx950 matrix cores apply in hardware.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from tests import exact


def test_e8m0_all_bytes_match_torch():
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    ours = np.array([oracle.e8m0_to_double(b) for b in range(256)])
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert np.array_equal(ours[:255], ref[:255])


def _mx_fractions(Q, S, K):
    rows = Q.shape[0]
    out = np.empty((rows, K), dtype=object)
    for r in range(rows):
        for k in range(K):
            byte = int(Q[r, k // 2])
            code = (byte >> 4) if k & 1 else (byte & 15)
            out[r, k] = exact.e2m1_fraction(code) * Fraction(2) ** (int(S[r, k // 32]) - 127)
    return out


@pytest.mark.parametrize("M,N,K", [(3, 5, 32), (4, 2, 64), (5, 3, 96), (1, 7, 32), (2, 2, 128)])
def test_mx_brute_force_exact(M, N, K):
    Aq, SA = syn.mxfp4_operand(M, K, seed=M + 10 * K)
    Bq, SB = syn.mxfp4_operand(N, K, seed=N + 10 * K + 3)
    ref = exact.gemm_exact_bits(_mx_fractions(Aq, SA, K), _mx_fractions(Bq, SB, K))
    assert np.array_equal(oracle.gemm_mxfp4_nt(Aq, SA, Bq, SB, K), ref)


def test_unit_scales_equal_the_nvfp4_product_with_unit_scales():
    M, N, K = 9, 11, 256
    Aq = syn.fp4_codes(M, K, seed=1)
    Bq = syn.fp4_codes(N, K, seed=2)
    one_mx = lambda r: np.full((r, K // 32), 127, np.uint8)
    one_nv = lambda r: np.full((r, K // 16), 0x38, np.uint8)   # E4M3 1.0
    assert np.array_equal(oracle.gemm_mxfp4_nt(Aq, one_mx(M), Bq, one_mx(N), K),
                          oracle.gemm_nvfp4_nt(Aq, one_nv(M), Bq, one_nv(N), K))


def test_one_block_scale_scales_one_block():
    # doubling one 32-element block's scale doubles exactly that block's part
    M, N, K = 4, 6, 128
    Aq, SA = syn.mxfp4_operand(M, K, seed=7)
    Bq, SB = syn.mxfp4_operand(N, K, seed=8)
    ms, ns = (x.ravel() for x in np.meshgrid(np.arange(M), np.arange(N), indexing="ij"))
    _, s0 = oracle.gemm_mxfp4_nt_at(Aq, SA, Bq, SB, K, ms, ns, with_sum=True)
    SA2 = SA.copy()
    SA2[:, 2] += 1
    _, s1 = oracle.gemm_mxfp4_nt_at(Aq, SA2, Bq, SB, K, ms, ns, with_sum=True)
    # the block's own contribution, from the sums over K = 32 with the other blocks' codes zeroed
    keep = np.zeros_like(Aq)
    keep[:, 32:48] = Aq[:, 32:48]
    _, blk = oracle.gemm_mxfp4_nt_at(keep, SA, Bq, SB, K, ms, ns, with_sum=True)
    assert np.array_equal(s1, s0 + blk)
    assert np.any(blk != 0)


def test_sampled_elements_match_whole_product():
    M, N, K = 20, 24, 160
    Aq, SA = syn.mxfp4_operand(M, K, seed=11)
    Bq, SB = syn.mxfp4_operand(N, K, seed=12)
    whole = oracle.gemm_mxfp4_nt(Aq, SA, Bq, SB, K)
    ms, ns = (x.ravel() for x in np.meshgrid(np.arange(M), np.arange(N), indexing="ij"))
    assert np.array_equal(oracle.gemm_mxfp4_nt_at(Aq, SA, Bq, SB, K, ms, ns).reshape(M, N), whole)


def test_mx_fused_oracle_rejects_bad_arguments():
    # K not a multiple of 32, an unknown activation, an index out of range
    Aq, SA = syn.mxfp4_operand(2, 64, seed=301)
    Bq, SB = syn.mxfp4_operand(3, 64, seed=302)
    ms, ns = np.array([0, 1]), np.array([2, 0])
    for act in (-1, 3):
        with pytest.raises(ValueError):
            oracle.gemm_mxfp4_nt_bias_act_at(Aq, SA, Bq, SB, 64, None, act, ms, ns)
    with pytest.raises(ValueError):
        oracle.gemm_mxfp4_nt_bias_act_at(Aq, SA, Bq, SB, 64, None, oracle.ACT_NONE, np.array([2]), np.array([0]))
    with pytest.raises(ValueError):
        oracle.gemm_mxfp4_nt_bias_act_at(Aq[:, :8], SA[:, :1], Bq[:, :8], SB[:, :1], 16, None, oracle.ACT_NONE, ms, ns)


def test_mx_equals_decode_then_bf16_path():
    # with the workload's scales (2^u, u in -4..4) every decoded element is
    # e2m1 * 2^u, at most 2 significant bits: exact in BF16, so the
    # microscaled product is the BF16 product of the decoded operands
    K = 256
    Aq, SA = syn.mxfp4_operand(33, K, seed=30)
    Bq, SB = syn.mxfp4_operand(17, K, seed=31)
    e2 = np.array([oracle.e2m1_to_double(c) for c in range(16)])
    e8 = np.array([oracle.e8m0_to_double(b) for b in range(255)] + [np.nan])
    dec = lambda Q, S: e2[np.stack([Q & 15, Q >> 4], -1).reshape(Q.shape[0], -1)] * np.repeat(e8[S], 32, axis=1)
    Ad, Bd = dec(Aq, SA), dec(Bq, SB)
    Ab, Bb = oracle.bf16_from_double(Ad), oracle.bf16_from_double(Bd)
    assert np.array_equal(oracle.bf16_to_double(Ab), Ad)
    assert np.array_equal(oracle.gemm_mxfp4_nt(Aq, SA, Bq, SB, K), oracle.gemm_bf16_nt(Ab, Bb))
