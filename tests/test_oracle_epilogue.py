"""Pins of the oracle's fused epilogue (bias, activation) against what does
not come from the oracle itself: exact rational sums rounded by the definition
of round-to-nearest-even, a library routine for the GELU (torch's tanh-form
GELU in binary64), closed forms of the activations, and planted mistakes that
the fused parity bound must catch. CPU only.

Reference: "NVFP4 GEMM on Blackwell", "Kernel 1", "Epilogue Warps" (per-element
work on the sums belongs in the epilogue);
the operation itself (bias per output column, then ReLU or the tanh-form GELU)
is this library's reading, since the page names none.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from tests import exact, tolerance

ACTS = [oracle.ACT_NONE, oracle.ACT_RELU, oracle.ACT_GELU_TANH]


def _gelu_torch(z: np.ndarray) -> np.ndarray:
    return torch.nn.functional.gelu(torch.from_numpy(np.asarray(z, dtype=np.float64)), approximate="tanh").numpy()


def test_gelu_matches_torch_tanh_gelu_in_binary64():
    z = np.concatenate([np.linspace(-12, 12, 4801), [-1e-300, 0.0, 1e-300, 37.0, -37.0]])
    ours = np.array([oracle.activate(v, oracle.ACT_GELU_TANH) for v in z])
    ref = _gelu_torch(z)
    # relative agreement; below z = -7 both evaluations of 1 + tanh(u) cancel
    # to within a few 1e-16 of zero (absolute)
    assert np.allclose(ours, ref, rtol=4e-15, atol=1e-15)


def test_activation_closed_forms():
    g = lambda v: oracle.activate(v, oracle.ACT_GELU_TANH)
    assert g(0.0) == 0.0
    # gelu(z) - gelu(-z) = z (the tanh terms cancel)
    for v in (0.25, 1.0, 2.5, 7.0):
        assert abs(g(v) - g(-v) - v) <= 1e-15 * max(1.0, v)
    # large |z|: the identity above, and zero
    assert g(20.0) == 20.0 and g(-20.0) == 0.0
    # GELU(1) with the tanh form: 0.5 (1 + tanh(sqrt(2/pi) * 1.044715))
    assert abs(g(1.0) - 0.8411919906082768) < 1e-15
    for v in (-3.0, -0.0, 0.0, 0.5, 4.0):
        assert oracle.activate(v, oracle.ACT_RELU) == max(v, 0.0)
        assert oracle.activate(v, oracle.ACT_NONE) == v


@pytest.mark.parametrize("M,N,K", [(3, 5, 7), (5, 3, 16), (1, 9, 33), (4, 4, 1)])
@pytest.mark.parametrize("act", [oracle.ACT_NONE, oracle.ACT_RELU])
def test_bias_relu_exact_against_fractions(M, N, K, act):
    # exact rational z = sum + bias[n] (bias differs per column, so a bias
    # taken per row or from the neighbouring column fails); ReLU is exact
    A = syn.bf16_uniform(M, K, seed=M + 7 * K)
    B = syn.bf16_uniform(N, K, seed=N + 7 * K + 1)
    bias = syn.bf16_uniform(1, N, seed=99 + N, lo=-4.0, hi=4.0)[0]
    Af, Bf = exact.bf16_bits_to_fractions(A), exact.bf16_bits_to_fractions(B)
    bf = exact.bf16_bits_to_fractions(bias[None, :])[0]
    want = np.empty((M, N), dtype=np.uint16)
    for m in range(M):
        for n in range(N):
            z = sum((Af[m, k] * Bf[n, k] for k in range(K)), Fraction(0)) + bf[n]
            if act == oracle.ACT_RELU and z < 0:
                z = Fraction(0)
            want[m, n] = exact.rne_bf16(z)
    assert np.array_equal(oracle.gemm_bf16_nt_bias_act(A, B, bias, act), want)


def test_no_bias_and_identity_activation_is_the_plain_product():
    A = syn.bf16_uniform(17, 40, seed=5)
    B = syn.bf16_uniform(9, 40, seed=6)
    assert np.array_equal(oracle.gemm_bf16_nt_bias_act(A, B, None, oracle.ACT_NONE), oracle.gemm_bf16_nt(A, B))


@pytest.mark.parametrize("act", ACTS)
def test_empty_sum_gives_activation_of_bias(act):
    N = 24
    bias = syn.bf16_uniform(1, N, seed=3, lo=-3.0, hi=3.0)[0]
    A = np.zeros((5, 0), np.uint16)
    B = np.zeros((N, 0), np.uint16)
    got = oracle.gemm_bf16_nt_bias_act(A, B, bias, act)
    b = tolerance.bf16_bits_to_f64(bias)
    if act == oracle.ACT_GELU_TANH:
        y = _gelu_torch(b)
    elif act == oracle.ACT_RELU:
        y = np.maximum(b, 0.0)
    else:
        y = b
    assert np.array_equal(got, np.broadcast_to(oracle.bf16_from_double(y), (5, N)))


@pytest.mark.parametrize("act", ACTS)
def test_identity_operand_gives_elementwise_activation(act):
    # B = I: z = A + bias exactly (one product per element), then the
    # activation evaluated by torch (GELU) or by hand
    K = 48
    A = syn.bf16_uniform(7, K, seed=21, lo=-3.0, hi=3.0)
    bias = syn.bf16_uniform(1, K, seed=22)[0]
    z = tolerance.bf16_bits_to_f64(A) + tolerance.bf16_bits_to_f64(bias)[None, :]
    y = _gelu_torch(z) if act == oracle.ACT_GELU_TANH else (np.maximum(z, 0.0) if act == oracle.ACT_RELU else z)
    assert np.array_equal(oracle.gemm_bf16_nt_bias_act(A, syn.bf16_identity(K), bias, act), oracle.bf16_from_double(y))


@pytest.mark.parametrize("act", ACTS)
def test_sampled_elements_match_whole_product(act):
    A = syn.bf16_uniform(30, 64, seed=31)
    B = syn.bf16_uniform(26, 64, seed=32)
    bias = syn.bf16_uniform(1, 26, seed=33)[0]
    whole = oracle.gemm_bf16_nt_bias_act(A, B, bias, act)
    ms, ns = np.meshgrid(np.arange(30), np.arange(26), indexing="ij")
    got, z = oracle.gemm_bf16_nt_bias_act_at(A, B, bias, act, ms.ravel(), ns.ravel(), with_z=True)
    assert np.array_equal(got.reshape(30, 26), whole)
    plain, s = oracle.gemm_bf16_nt_at(A, B, ms.ravel(), ns.ravel(), with_sum=True)
    assert np.array_equal(z, s + tolerance.bf16_bits_to_f64(bias)[ns.ravel()])


def test_fused_bound_accepts_one_ulp_and_rejects_planted_mistakes():
    # planted in a copy of the oracle's result on the CPU: a bias shifted by one
    # column, the activation left out, ReLU instead of GELU, one K step dropped
    M, N, K = 40, 48, 64
    A = syn.bf16_uniform(M, K, seed=41)
    B = syn.bf16_uniform(N, K, seed=42)
    bias = syn.bf16_uniform(1, N, seed=43)[0]
    ms, ns = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    for act in ACTS:
        ref, z = oracle.gemm_bf16_nt_bias_act_at(A, B, bias, act, ms.ravel(), ns.ravel(), with_z=True)
        ref, z = ref.reshape(M, N), z.reshape(M, N)
        assert tolerance.check_fused(ref, ref, z, K, act)
        nudged = ref.copy()
        nudged[3, 5] += 1   # one BF16 ulp
        assert tolerance.check_fused(nudged, ref, z, K, act)
        shifted = oracle.gemm_bf16_nt_bias_act(A, B, np.roll(bias, 1), act)
        assert not tolerance.check_fused(shifted, ref, z, K, act)
        dropped = oracle.gemm_bf16_nt_bias_act(A[:, :-1], B[:, :-1], bias, act)
        assert not tolerance.check_fused(dropped, ref, z, K, act)
    ref, z = oracle.gemm_bf16_nt_bias_act_at(A, B, bias, oracle.ACT_GELU_TANH, ms.ravel(), ns.ravel(), with_z=True)
    ref, z = ref.reshape(M, N), z.reshape(M, N)
    for wrong in (oracle.ACT_NONE, oracle.ACT_RELU):
        assert not tolerance.check_fused(oracle.gemm_bf16_nt_bias_act(A, B, bias, wrong), ref, z, K,
                                         oracle.ACT_GELU_TANH)


@pytest.mark.parametrize("act", ACTS)
def test_fp4_fused_is_activation_of_plain_fp4_sum_plus_bias(act):
    # the FP4 form: z must be the plain FP4 oracle's binary64 sum plus the
    # bias of the column (bias from one column to the left fails), and the
    # output the activation of z evaluated independently (torch for the GELU)
    M, N, K = 9, 24, 96
    Aq, SFA = syn.fp4_operand(M, K, seed=131)
    Bq, SFB = syn.fp4_operand(N, K, seed=132)
    bias = syn.bf16_uniform(1, N, seed=133, lo=-64.0, hi=64.0)[0]
    ms, ns = (x.ravel() for x in np.meshgrid(np.arange(M), np.arange(N), indexing="ij"))
    got, z = oracle.gemm_nvfp4_nt_bias_act_at(Aq, SFA, Bq, SFB, K, bias, act, ms, ns, with_z=True)
    _, s = oracle.gemm_nvfp4_nt_at(Aq, SFA, Bq, SFB, K, ms, ns, with_sum=True)
    b = tolerance.bf16_bits_to_f64(bias)
    assert np.array_equal(z, s + b[ns])
    assert not np.array_equal(z, s + np.roll(b, 1)[ns])
    y = _gelu_torch(z) if act == oracle.ACT_GELU_TANH else (np.maximum(z, 0.0) if act == oracle.ACT_RELU else z)
    assert np.array_equal(got, oracle.bf16_from_double(y))
    if act == oracle.ACT_NONE:
        assert np.array_equal(oracle.gemm_nvfp4_nt_bias_act_at(Aq, SFA, Bq, SFB, K, None, act, ms, ns),
                              oracle.gemm_nvfp4_nt(Aq, SFA, Bq, SFB, K).ravel())


@pytest.mark.parametrize("act", ACTS)
def test_mx_fused_is_activation_of_plain_mx_sum_plus_bias(act):
    # the microscaled form: z must be the plain microscaled oracle's binary64
    # sum plus the column's bias (a bias one column to the left fails), and
    # the output the activation of z evaluated independently (torch: GELU)
    M, N, K = 9, 24, 128
    Aq, SA = syn.mxfp4_operand(M, K, seed=231)
    Bq, SB = syn.mxfp4_operand(N, K, seed=232)
    bias = syn.bf16_uniform(1, N, seed=233, lo=-64.0, hi=64.0)[0]
    ms, ns = (x.ravel() for x in np.meshgrid(np.arange(M), np.arange(N), indexing="ij"))
    got, z = oracle.gemm_mxfp4_nt_bias_act_at(Aq, SA, Bq, SB, K, bias, act, ms, ns, with_z=True)
    _, s = oracle.gemm_mxfp4_nt_at(Aq, SA, Bq, SB, K, ms, ns, with_sum=True)
    b = tolerance.bf16_bits_to_f64(bias)
    assert np.array_equal(z, s + b[ns])
    assert not np.array_equal(z, s + np.roll(b, 1)[ns])
    y = _gelu_torch(z) if act == oracle.ACT_GELU_TANH else (np.maximum(z, 0.0) if act == oracle.ACT_RELU else z)
    assert np.array_equal(got, oracle.bf16_from_double(y))
    if act == oracle.ACT_NONE:
        assert np.array_equal(oracle.gemm_mxfp4_nt_bias_act_at(Aq, SA, Bq, SB, K, None, act, ms, ns),
                              oracle.gemm_mxfp4_nt(Aq, SA, Bq, SB, K).ravel())
