"""Pins for the oracle's GEMM loops (CPU only).

The oracle is checked against exact rational brute force on tiny shapes,
closed forms (identity, permutation, rank-1), the transpose identity
C^T = B A^T ("NVFP4 GEMM on Blackwell", section "Production Kernel", "Swap
AB"), the FP4 = decode-then-BF16 identity, and the parity bar's own
sensitivity to planted mistakes.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from tests import exact, tolerance

TINY = [1, 2, 3, 5, 8, 16, 17, 31, 33]


def _tiny_shapes(count, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    combos = list(itertools.product(TINY, TINY, TINY))
    idx = g.choice(len(combos), size=count, replace=False)
    return [combos[i] for i in idx]


@pytest.mark.parametrize("M,N,K", _tiny_shapes(14, 1) + [(1, 1, 1), (33, 33, 33)])
def test_bf16_brute_force_exact(M, N, K):
    A = syn.bf16_uniform(M, K, seed=M * 100 + K)
    B = syn.bf16_uniform(N, K, seed=N * 100 + K + 1)
    ref = exact.gemm_exact_bits(exact.bf16_bits_to_fractions(A), exact.bf16_bits_to_fractions(B))
    assert np.array_equal(oracle.gemm_bf16_nt(A, B), ref)


@pytest.mark.parametrize("M,N,K", [(3, 5, 16), (4, 2, 32), (5, 3, 48), (1, 7, 16)])
def test_fp4_brute_force_exact(M, N, K):
    Aq, SFA = syn.fp4_operand(M, K, seed=M + 10 * K)
    Bq, SFB = syn.fp4_operand(N, K, seed=N + 10 * K + 3)
    ref = exact.gemm_exact_bits(exact.fp4_fractions(Aq, SFA, K), exact.fp4_fractions(Bq, SFB, K))
    assert np.array_equal(oracle.gemm_nvfp4_nt(Aq, SFA, Bq, SFB, K), ref)


def test_identity_right_gives_A():
    M, K = 40, 72
    A = syn.bf16_uniform(M, K, seed=3)
    C = oracle.gemm_bf16_nt(A, syn.bf16_identity(K))
    assert np.array_equal(C, A)


def test_identity_left_gives_B_transposed():
    N, K = 24, 56
    B = syn.bf16_uniform(N, K, seed=4)
    C = oracle.gemm_bf16_nt(syn.bf16_identity(K), B)
    assert np.array_equal(C, B.T)


def test_permutation_moves_columns():
    M, K = 16, 48
    A = syn.bf16_uniform(M, K, seed=5)
    perm = syn.permutation(K, seed=6)
    C = oracle.gemm_bf16_nt(A, syn.bf16_permutation_matrix(perm))
    assert np.array_equal(C, A[:, perm])


def test_rank1_closed_form_exact():
    # A = u 1^T, B = v 1^T with u, v multiples of 1/16: C[m, n] = K u_m v_n
    # exactly (at most 8 significant bits, so representable in BF16).
    M, N, K = 20, 28, 64
    g = np.random.Generator(np.random.PCG64(7))
    u = g.integers(-16, 17, size=M) / 16.0
    v = g.integers(-16, 17, size=N) / 16.0
    A = syn.to_bf16_bits(np.repeat(u[:, None], K, axis=1))
    B = syn.to_bf16_bits(np.repeat(v[:, None], K, axis=1))
    want = syn.to_bf16_bits(K * np.outer(u, v))
    # compared as values: the sign of a zero result is not part of the contract
    assert np.array_equal(tolerance.bf16_bits_to_f64(oracle.gemm_bf16_nt(A, B)),
                          tolerance.bf16_bits_to_f64(want))


def test_rank1_with_random_B_matches_exact_sum():
    M, N, K = 6, 9, 64
    g = np.random.Generator(np.random.PCG64(8))
    u = g.integers(-16, 17, size=M) / 16.0
    A = syn.to_bf16_bits(np.repeat(u[:, None], K, axis=1))
    B = syn.bf16_uniform(N, K, seed=9)
    Bf = exact.bf16_bits_to_fractions(B)
    ms, ns = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    out, sums = oracle.gemm_bf16_nt_at(A, B, ms.ravel(), ns.ravel(), with_sum=True)
    from fractions import Fraction
    for i, (m, n) in enumerate(zip(ms.ravel(), ns.ravel())):
        s = Fraction(float(u[m])) * sum(Bf[n, :], Fraction(0))
        assert out[i] == exact.rne_bf16(s)
        assert Fraction(float(sums[i])) == s  # these sums are exact in binary64


def test_sum_is_rounded_once_at_the_end():
    # 1 + 2^-8 + 2^-30 lies just above a BF16 tie: the exact sum rounds up to
    # 1 + 2^-7. Accumulating in binary32 (or rounding twice) would drop 2^-30
    # and round the tie to even, 1.0.
    A = syn.to_bf16_bits(np.array([[1.0, 2.0 ** -8, 2.0 ** -30]]))
    B = syn.to_bf16_bits(np.ones((1, 3)))
    assert int(oracle.gemm_bf16_nt(A, B)[0, 0]) == 0x3F81
    assert int(oracle.gemm_bf16_nt(A[:, ::-1].copy(), B)[0, 0]) == 0x3F81


def test_transpose_identity_bitwise():
    A = syn.bf16_uniform(37, 80, seed=10)
    B = syn.bf16_uniform(29, 80, seed=11)
    assert np.array_equal(oracle.gemm_bf16_nt(B, A), oracle.gemm_bf16_nt(A, B).T)


def test_thread_count_does_not_change_bits():
    A = syn.bf16_uniform(64, 256, seed=12)
    B = syn.bf16_uniform(48, 256, seed=13)
    n0 = oracle.max_threads()
    try:
        oracle.set_threads(1)
        one = oracle.gemm_bf16_nt(A, B)
        oracle.set_threads(max(2, n0))
        many = oracle.gemm_bf16_nt(A, B)
    finally:
        oracle.set_threads(n0)
    assert np.array_equal(one, many)


def test_sampled_elements_match_full_product():
    A = syn.bf16_uniform(50, 96, seed=14)
    B = syn.bf16_uniform(70, 96, seed=15)
    full = oracle.gemm_bf16_nt(A, B)
    g = np.random.Generator(np.random.PCG64(16))
    ms = g.integers(0, 50, 300)
    ns = g.integers(0, 70, 300)
    assert np.array_equal(oracle.gemm_bf16_nt_at(A, B, ms, ns), full[ms, ns])
    Aq, SFA = syn.fp4_operand(50, 96, seed=17)
    Bq, SFB = syn.fp4_operand(70, 96, seed=18)
    full4 = oracle.gemm_nvfp4_nt(Aq, SFA, Bq, SFB, 96)
    assert np.array_equal(oracle.gemm_nvfp4_nt_at(Aq, SFA, Bq, SFB, 96, ms, ns), full4[ms, ns])


def test_empty_and_degenerate_shapes():
    A = syn.bf16_uniform(0, 16, seed=1)
    B = syn.bf16_uniform(5, 16, seed=2)
    assert oracle.gemm_bf16_nt(A, B).shape == (0, 5)
    # K = 0: the empty sum is +0
    C = oracle.gemm_bf16_nt(np.zeros((3, 0), np.uint16), np.zeros((4, 0), np.uint16))
    assert np.array_equal(C, np.zeros((3, 4), np.uint16))


def test_fp4_equals_decode_then_bf16_path():
    K = 128
    Aq, SFA = syn.fp4_operand(33, K, seed=20)
    Bq, SFB = syn.fp4_operand(17, K, seed=21)
    Ad = oracle.decode_nvfp4(Aq, SFA, K)
    Bd = oracle.decode_nvfp4(Bq, SFB, K)
    # decoded elements need at most 6 significant bits: exact in BF16
    Ab = syn.to_bf16_bits(Ad)
    assert np.array_equal(tolerance.bf16_bits_to_f64(Ab), Ad)
    assert np.array_equal(oracle.gemm_nvfp4_nt(Aq, SFA, Bq, SFB, K),
                          oracle.gemm_bf16_nt(Ab, syn.to_bf16_bits(Bd)))


def test_fp4_decode_matches_page_table_and_torch_scales():
    K = 64
    Q, SF = syn.fp4_operand(9, K, seed=22)
    ours = oracle.decode_nvfp4(Q, SF, K)
    ref = exact.fp4_fractions(Q, SF, K)
    assert all(ours[r, k] == float(ref[r, k]) for r in range(9) for k in range(K))


def test_fp4_nibble_order_low_nibble_is_even_k():
    # Reading: even k in the low nibble. Byte 0x21: k=0 -> code 1 (0.5),
    # k=1 -> code 2 (1.0). Unit scales (0x38 = 1.0).
    K = 16
    Aq = np.zeros((1, K // 2), np.uint8)
    Aq[0, 0] = 0x21
    SF = np.full((1, 1), 0x38, np.uint8)
    Bq = np.zeros((2, K // 2), np.uint8)
    Bq[0, 0] = 0x02   # b(0, 0) = 1
    Bq[1, 0] = 0x20   # b(1, 1) = 1
    C = tolerance.bf16_bits_to_f64(oracle.gemm_nvfp4_nt(Aq, SF, Bq, np.full((2, 1), 0x38, np.uint8), K))
    assert C.tolist() == [[0.5, 1.0]]


def test_fp4_unit_scales_reduce_to_plain_e2m1_product():
    K = 32
    Aq = syn.fp4_codes(5, K, seed=23)
    Bq = syn.fp4_codes(6, K, seed=24)
    ones_a = np.full((5, K // 16), 0x38, np.uint8)
    ones_b = np.full((6, K // 16), 0x38, np.uint8)
    Ad = exact.fp4_fractions(Aq, ones_a, K)
    Bd = exact.fp4_fractions(Bq, ones_b, K)
    assert np.array_equal(oracle.gemm_nvfp4_nt(Aq, ones_a, Bq, ones_b, K), exact.gemm_exact_bits(Ad, Bd))


# ---- the parity bar catches planted mistakes ------------------------------

def _problem(seed=30, M=64, N=64, K=256):
    A = syn.bf16_uniform(M, K, seed=seed)
    B = syn.bf16_uniform(N, K, seed=seed + 1)
    return A, B, oracle.gemm_bf16_nt(A, B)


def test_bar_accepts_oracle_and_one_ulp():
    A, B, C = _problem()
    assert tolerance.check(C, C, 256)
    bumped = C.copy()
    bumped[3, 7] = np.uint16(int(bumped[3, 7]) + 1)
    assert tolerance.check(bumped, C, 256)


def test_bar_rejects_dropped_k_block():
    A, B, C = _problem()
    A2 = A.copy()
    A2[:, 64:80] = 0
    assert not tolerance.check(oracle.gemm_bf16_nt(A2, B), C, 256)


def test_bar_rejects_swapped_rows_and_nan():
    A, B, C = _problem()
    assert not tolerance.check(C[[1, 0] + list(range(2, 64))], C, 256)
    D = C.copy()
    D[5, 5] = 0x7FC0
    assert not tolerance.check(D, C, 256)


def test_bar_rejects_one_wrong_scale_byte():
    K = 512
    Aq, SFA = syn.fp4_operand(32, K, seed=40)
    Bq, SFB = syn.fp4_operand(32, K, seed=41)
    C = oracle.gemm_nvfp4_nt(Aq, SFA, Bq, SFB, K)
    sigma = tolerance.sigma_of(oracle.decode_nvfp4(Aq, SFA, K)) * tolerance.sigma_of(oracle.decode_nvfp4(Bq, SFB, K))
    assert tolerance.check(C, C, K, sigma)
    bad = SFA.copy()
    bad[4, 3] = bad[4, 3] + 8 if bad[4, 3] < 0x58 else bad[4, 3] - 8  # one scale off by 2x
    assert not tolerance.check(oracle.gemm_nvfp4_nt(Aq, bad, Bq, SFB, K), C, K, sigma)
