"""Parity of the HIP microscaled FP4 path (gemm_mxfp4_nt through the C ABI)
with the oracle: E2M1 codes with one E8M0 power-of-two scale per 32 elements,
taken undecoded by the matrix cores' scaled instructions.

Ragged shapes (partial tiles, scale blocks of four K steps with an odd number
of blocks) element by element within the sigma-scaled bound; exactly summable
inputs bitwise, including the 8192^3 workload on every element; the decoded
identity; K = 0; guard bands around C throughout.

Reference: "NVFP4 GEMM on Blackwell", "NVFP4 Datatype" (block-scaled FP4 whose
scales the MMA applies inside the instruction); the E8M0 scale per 32 is the
hardware's format, not the page's E4M3 per 16.
"""
import numpy as np
import pytest
import torch

import dense_gemm_14_amd as g
import oracle
import synthetic as syn
from tests import tolerance
from tests.gpu_util import GuardedC, need_gpu, sample_positions, to_dev

pytestmark = pytest.mark.gpu

_E2M1 = np.array([oracle.e2m1_to_double(c) for c in range(16)])
_E8M0 = np.array([oracle.e8m0_to_double(b) if b != 0xFF else np.nan for b in range(256)])


def decode(Q, S):
    """Decoded operand in binary64, from the oracle's per-code and per-scale values."""
    codes = np.stack([Q & 15, Q >> 4], -1).reshape(Q.shape[0], -1)
    return _E2M1[codes] * np.repeat(_E8M0[S], 32, axis=1)


def run_mx(Aq, SA, Bq, SB, M, N, K):
    C = GuardedC(M, N)
    g.gemm_mxfp4_nt(M, N, K, to_dev(Aq), to_dev(SA), to_dev(Bq), to_dev(SB), C.view)
    torch.cuda.synchronize()
    assert C.guards_intact(), "write outside C"
    return C.bits()


def _sigma(Q, S):
    return tolerance.sigma_of(decode(Q[:512], S[:512]))


@pytest.mark.parametrize("M,N,K", [(256, 256, 512), (1, 8, 512), (65, 72, 512), (257, 264, 1024),
                                   (513, 520, 1536), (300, 8, 2560), (128, 1024, 512), (520, 256, 4608)])
def test_ragged_shapes_match_oracle(M, N, K):
    need_gpu()
    print("mx ragged", M, N, K, flush=True)
    Aq, SA = syn.mxfp4_operand(M, K, seed=M + 5 * N + K)
    Bq, SB = syn.mxfp4_operand(N, K, seed=M + 5 * N + K + 1)
    C = run_mx(Aq, SA, Bq, SB, M, N, K)
    ref = oracle.gemm_mxfp4_nt(Aq, SA, Bq, SB, K)
    res = tolerance.check(C, ref, K, _sigma(Aq, SA) * _sigma(Bq, SB))
    assert res, res


def test_wide_scale_range_matches_oracle():
    # scales 2^-20 .. 2^20: a scale taken from the wrong 32-block, step or
    # row changes the sum by orders of magnitude
    need_gpu()
    M, N, K = 264, 256, 2048
    Aq, Bq = syn.fp4_codes(M, K, seed=31), syn.fp4_codes(N, K, seed=32)
    SA = syn.e8m0_scales(M, K, seed=33, u_lo=-20, u_hi=20)
    SB = syn.e8m0_scales(N, K, seed=34, u_lo=-20, u_hi=20)
    C = run_mx(Aq, SA, Bq, SB, M, N, K)
    ms, ns = (x.ravel() for x in np.meshgrid(np.arange(M), np.arange(N), indexing="ij"))
    ref, s = oracle.gemm_mxfp4_nt_at(Aq, SA, Bq, SB, K, ms, ns, with_sum=True)
    # per element: a term of the sum can be 2^40 times another, so the bound
    # is the deterministic one of FP32 summation, K 2^-24 times the sum of
    # magnitudes |a| |b| over k; a scale from the wrong block moves a term by
    # a power of two and the sum by about that term
    Ad, Bd = decode(Aq, SA), decode(Bq, SB)
    mag = (np.abs(Ad) @ np.abs(Bd).T).ravel()
    got = tolerance.bf16_bits_to_f64(C).ravel()
    want = tolerance.bf16_bits_to_f64(ref)
    excess = np.abs(got - want) - 2.0 ** -7 * np.abs(want) - K * 2.0 ** -24 * mag
    assert np.all(excess <= 0), (np.argmax(excess), excess.max())


@pytest.mark.parametrize("M,N,K", [(264, 520, 512), (513, 256, 1024)])
def test_exact_unit_scales_bitwise(M, N, K):
    # scales 2^0, all 16 codes, K <= 1024: every partial sum is a multiple of
    # 2^-2 below 2^16, exact in FP32, so the result is unique
    need_gpu()
    Aq, Bq = syn.fp4_codes(M, K, seed=61), syn.fp4_codes(N, K, seed=62)
    SA = syn.e8m0_scales(M, K, seed=63, u_lo=0, u_hi=0)
    SB = syn.e8m0_scales(N, K, seed=64, u_lo=0, u_hi=0)
    assert np.array_equal(run_mx(Aq, SA, Bq, SB, M, N, K), oracle.gemm_mxfp4_nt(Aq, SA, Bq, SB, K))


def test_decoded_identity_reproduces_A():
    # B = I (code 2 = 1.0 on the diagonal, scales 2^0): C = dec(A)
    need_gpu()
    M, K = 300, 512
    Aq, SA = syn.mxfp4_operand(M, K, seed=65)
    codes = np.zeros((K, K), np.uint8)
    codes[np.arange(K), np.arange(K)] = 2
    Bq = syn.pack_nibbles(codes)
    SB = np.full((K, K // 32), 127, np.uint8)
    C = run_mx(Aq, SA, Bq, SB, M, K, K)
    want = syn.to_bf16_bits(decode(Aq, SA))
    # compared as values: code 8 is -0, and a zero sum's sign is not specified
    assert np.array_equal(tolerance.bf16_bits_to_f64(C), tolerance.bf16_bits_to_f64(want))


def test_empty_sum_is_zero():
    need_gpu()
    M, N = 70, 72
    C = GuardedC(M, N)
    g.gemm_mxfp4_nt(M, N, 0, None, None, None, None, C.view)
    torch.cuda.synchronize()
    assert C.guards_intact()
    assert np.all(tolerance.bf16_bits_to_f64(C.bits()) == 0.0)


def test_mx_workload_sampled_against_oracle():
    need_gpu()
    M = N = K = 8192
    print("mx workload", M, N, K, flush=True)
    Aq, SA = syn.mxfp4_operand(M, K, seed=171)
    Bq, SB = syn.mxfp4_operand(N, K, seed=172)
    C = run_mx(Aq, SA, Bq, SB, M, N, K)
    ms, ns = sample_positions(M, N, 3000, seed=173)
    ref = oracle.gemm_mxfp4_nt_at(Aq, SA, Bq, SB, K, ms, ns)
    res = tolerance.check(C[ms, ns], ref, K, _sigma(Aq, SA) * _sigma(Bq, SB))
    assert res, res
    assert np.all(np.isfinite(tolerance.bf16_bits_to_f64(C)))


def test_mx_workload_exactly_summable_every_element():
    # scales in {2^-1, 2^0}, all 16 codes, K = 8192: every partial sum is a
    # multiple of 2^-4 below 2^19, exact in FP32; the whole product in binary64
    need_gpu()
    M = N = K = 8192
    print("mx workload exact", M, N, K, flush=True)
    Aq, Bq = syn.fp4_codes(M, K, seed=181), syn.fp4_codes(N, K, seed=182)
    SA = syn.e8m0_scales(M, K, seed=183, u_lo=-1, u_hi=0)
    SB = syn.e8m0_scales(N, K, seed=184, u_lo=-1, u_hi=0)
    C = run_mx(Aq, SA, Bq, SB, M, N, K)
    want = oracle.bf16_from_double(decode(Aq, SA) @ decode(Bq, SB).T)
    ms, ns = sample_positions(M, N, 300, seed=185)
    assert np.array_equal(oracle.gemm_mxfp4_nt_at(Aq, SA, Bq, SB, K, ms, ns), want[ms, ns])
    bad = np.argwhere(C != want)
    assert bad.size == 0, "first mismatches %s" % bad[:5].tolist()


def test_multi_round_ragged_tiles_exact_every_element():
    # 17 x 17 = 289 tiles of 256 x 256 on a grid of at most 256 workgroups:
    # some workgroups take a second (ragged) tile, whose first steps the ring
    # fetched during the first tile's last ones, others stop after one.
    # Unit scales and K = 1024: every partial sum is a multiple of 2^-2 below
    # 2^16, exact in FP32, so every element is compared bitwise.
    need_gpu()
    M, N, K = 4100, 4104, 1024
    print("mx multi-round ragged", M, N, K, flush=True)
    Aq, Bq = syn.fp4_codes(M, K, seed=191), syn.fp4_codes(N, K, seed=192)
    SA = syn.e8m0_scales(M, K, seed=193, u_lo=0, u_hi=0)
    SB = syn.e8m0_scales(N, K, seed=194, u_lo=0, u_hi=0)
    C = run_mx(Aq, SA, Bq, SB, M, N, K)
    want = oracle.bf16_from_double(decode(Aq, SA) @ decode(Bq, SB).T)
    ms, ns = sample_positions(M, N, 300, seed=195)
    assert np.array_equal(oracle.gemm_mxfp4_nt_at(Aq, SA, Bq, SB, K, ms, ns), want[ms, ns])
    bad = np.argwhere(C != want)
    assert bad.size == 0, "first mismatches %s" % bad[:5].tolist()
