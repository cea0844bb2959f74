"""Parity of the HIP BF16 path (gemm_bf16_nt through the C ABI) with the oracle.

Small and ragged shapes are compared element by element with the oracle's
whole product; the workload shapes (4096^3, 8192^3, 8000^3, 128 x 8192 x 8192)
are compared on sampled elements, including every tile-boundary row and
column, plus properties that hold at any size: B = I gives C = A and A = I
gives C = B^T bitwise, and exactly summable inputs (multiples of 1/16) have a
unique correctly rounded answer, checked bitwise for every element.
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


def run_bf16(A_bits, B_bits, M, N, K, stream=None):
    A = to_dev(A_bits) if A_bits is not None else None
    B = to_dev(B_bits) if B_bits is not None else None
    C = GuardedC(M, N)
    g.gemm_bf16_nt(M, N, K, A, B, C.view, stream=stream)
    torch.cuda.synchronize()
    assert C.guards_intact(), "write outside C"
    return C.bits()


RAGGED = [
    (256, 256, 256),      # the small workload
    (1, 8, 8), (7, 16, 24), (65, 72, 40), (255, 256, 264), (257, 264, 136),
    (513, 520, 264), (300, 8, 1000), (128, 1024, 512), (1000, 1000, 64),
    (31, 40, 8), (520, 264, 72), (64, 64, 4104),
]


@pytest.mark.parametrize("M,N,K", RAGGED)
def test_ragged_shapes_match_oracle(M, N, K):
    need_gpu()
    A = syn.bf16_uniform(M, K, seed=M + 3 * N + 7 * K)
    B = syn.bf16_uniform(N, K, seed=M + 3 * N + 7 * K + 1)
    C = run_bf16(A, B, M, N, K)
    ref = oracle.gemm_bf16_nt(A, B)
    res = tolerance.check(C, ref, K)
    assert res, res


@pytest.mark.parametrize("M,N,K", [(513, 520, 264), (256, 256, 256), (1024, 1024, 1024), (72, 1032, 2056)])
def test_exactly_summable_inputs_are_bitwise(M, N, K):
    need_gpu()
    A = syn.bf16_sixteenths(M, K, seed=11 + K)
    B = syn.bf16_sixteenths(N, K, seed=12 + K)
    C = run_bf16(A, B, M, N, K)
    assert np.array_equal(C, oracle.gemm_bf16_nt(A, B))


def test_k_zero_writes_zeros_and_empty_output_writes_nothing():
    need_gpu()
    C = run_bf16(None, None, 40, 48, 0)
    assert np.array_equal(C, np.zeros((40, 48), np.uint16))
    c = GuardedC(8, 8)
    g.gemm_bf16_nt(0, 8, 64, None, None, c.view)
    torch.cuda.synchronize()
    assert np.all(c.bits() == 0x7FC1) and c.guards_intact()


def test_side_stream_and_determinism():
    need_gpu()
    M = N = 512
    K = 1024
    A = syn.bf16_uniform(M, K, seed=21)
    B = syn.bf16_uniform(N, K, seed=22)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        first = run_bf16(A, B, M, N, K, stream=s)
    second = run_bf16(A, B, M, N, K)
    assert np.array_equal(first, second)
    assert tolerance.check(first, oracle.gemm_bf16_nt(A, B), K)


def test_transpose_identity():
    need_gpu()
    M, N, K = 264, 520, 328
    A = syn.bf16_uniform(M, K, seed=31)
    B = syn.bf16_uniform(N, K, seed=32)
    C = run_bf16(A, B, M, N, K)
    Ct = run_bf16(B, A, N, M, K)
    assert tolerance.check(Ct, C.T.copy(), K)
    A = syn.bf16_sixteenths(M, K, seed=33)
    B = syn.bf16_sixteenths(N, K, seed=34)
    assert np.array_equal(run_bf16(B, A, N, M, K), run_bf16(A, B, M, N, K).T)


# ---- the workload shapes ------------------------------------------------------

WORKLOADS = [
    ("4096^3", 4096, 4096, 4096),
    ("8192^3", 8192, 8192, 8192),
    ("8000^3", 8000, 8000, 8000),
    ("skinny 128 x 8192 x 8192", 128, 8192, 8192),
]


@pytest.mark.parametrize("name,M,N,K", WORKLOADS)
def test_workload_sampled_against_oracle(name, M, N, K):
    need_gpu()
    A = syn.bf16_uniform(M, K, seed=syn.seed_for(2, 0) + M)
    B = syn.bf16_uniform(N, K, seed=syn.seed_for(2, 0) + M + 1)
    C = run_bf16(A, B, M, N, K)
    ms, ns = sample_positions(M, N, 3000, seed=M + N)
    ref = oracle.gemm_bf16_nt_at(A, B, ms, ns)
    res = tolerance.check(C[ms, ns], ref, K)
    assert res, (name, res)
    assert np.all(np.isfinite(tolerance.bf16_bits_to_f64(C)))


@pytest.mark.parametrize("name,M,N,K", [w for w in WORKLOADS if w[2] == w[3]])
def test_workload_identity_right_is_exact(name, M, N, K):
    # B = I (N = K): every element of C must equal A bitwise.
    need_gpu()
    A = syn.bf16_uniform(M, K, seed=41 + M)
    C = run_bf16(A, syn.bf16_identity(K), M, N, K)
    assert np.array_equal(C, A), name


def test_identity_left_gives_B_transposed():
    need_gpu()
    N, K = 520, 1000
    B = syn.bf16_uniform(N, K, seed=43)
    assert np.array_equal(run_bf16(syn.bf16_identity(K), B, K, N, K), B.T)


def test_permutation_moves_columns():
    need_gpu()
    M, K = 300, 1032
    A = syn.bf16_uniform(M, K, seed=44)
    perm = syn.permutation(K, seed=45)
    C = run_bf16(A, syn.bf16_permutation_matrix(perm), M, K, K)
    assert np.array_equal(C, A[:, perm])


@pytest.mark.parametrize("M,N,K", [(8192, 8192, 8192), (8000, 8000, 8000), (128, 8192, 8192)])
def test_workload_exactly_summable_every_element(M, N, K):
    # Multiples of 1/16 with |j| <= 16: every partial sum is exact in FP32, so the
    # correctly rounded result is unique. The exact sums are formed in float64
    # (any order is exact here) and rounded once by the oracle's BF16 rounding;
    # the oracle itself is compared on a sample.
    # Several launches: a missing wait between the copies into LDS and their
    # readers shows up only now and then (a late copy at the start of a
    # workgroup's first tile once made about one launch in thirty wrong).
    need_gpu()
    A = syn.bf16_sixteenths(M, K, seed=51 + M)
    B = syn.bf16_sixteenths(N, K, seed=52 + M)
    Af = tolerance.bf16_bits_to_f64(A)
    Bf = tolerance.bf16_bits_to_f64(B)
    want = oracle.bf16_from_double(Af @ Bf.T)
    ms, ns = sample_positions(M, N, 500, seed=7)
    assert np.array_equal(oracle.gemm_bf16_nt_at(A, B, ms, ns), want[ms, ns])
    dA, dB = to_dev(A), to_dev(B)
    for launch in range(8):
        C = GuardedC(M, N)
        g.gemm_bf16_nt(M, N, K, dA, dB, C.view)
        torch.cuda.synchronize()
        assert C.guards_intact(), "write outside C"
        bad = np.argwhere(C.bits() != want)
        assert bad.size == 0, "launch %d: %d mismatches, first %s" % (launch, len(bad), bad[:5].tolist())
