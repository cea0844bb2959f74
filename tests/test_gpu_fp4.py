"""Parity of the HIP block-scaled FP4 path (gemm_nvfp4_nt through the C ABI)
with the oracle.

The tolerance's absolute term is scaled by sigma_A * sigma_B (sqrt(3) times
the rms of each decoded operand), the stated bound for [-1, 1] data
transferred to the FP4 workload's second moment. Exactly summable scale
choices have a unique answer and are checked bitwise.
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


def run_fp4(Aq, SFA, Bq, SFB, M, N, K):
    C = GuardedC(M, N)
    g.gemm_nvfp4_nt(M, N, K, to_dev(Aq), to_dev(SFA), to_dev(Bq), to_dev(SFB), C.view)
    torch.cuda.synchronize()
    assert C.guards_intact(), "write outside C"
    return C.bits()


def _sigma(Q, SF, K):
    return tolerance.sigma_of(oracle.decode_nvfp4(Q, SF, K))


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (1, 8, 64), (65, 72, 128), (257, 264, 192),
                                   (513, 520, 320), (300, 8, 1024), (128, 1024, 512)])
def test_ragged_shapes_match_oracle(M, N, K):
    need_gpu()
    Aq, SFA = syn.fp4_operand(M, K, seed=M + 5 * N + K)
    Bq, SFB = syn.fp4_operand(N, K, seed=M + 5 * N + K + 1)
    C = run_fp4(Aq, SFA, Bq, SFB, M, N, K)
    ref = oracle.gemm_nvfp4_nt(Aq, SFA, Bq, SFB, K)
    res = tolerance.check(C, ref, K, _sigma(Aq, SFA, K) * _sigma(Bq, SFB, K))
    assert res, res


@pytest.mark.parametrize("M,N,K", [(264, 520, 512), (513, 256, 448)])
def test_exact_unit_exponent_scales_bitwise(M, N, K):
    # scales 2^0 * (1 + m/8), all 16 codes, K <= 512: sums exact in FP32
    need_gpu()
    Aq = syn.fp4_codes(M, K, seed=61)
    Bq = syn.fp4_codes(N, K, seed=62)
    SFA = syn.e4m3_scales(M, K, seed=63, u_lo=0, u_hi=0)
    SFB = syn.e4m3_scales(N, K, seed=64, u_lo=0, u_hi=0)
    C = run_fp4(Aq, SFA, Bq, SFB, M, N, K)
    assert np.array_equal(C, oracle.gemm_nvfp4_nt(Aq, SFA, Bq, SFB, K))


def test_decoded_identity_reproduces_A():
    # B = I as FP4 (code 2 = 1.0 on the diagonal, unit scales 0x38): C = dec(A).
    need_gpu()
    M, K = 300, 512
    Aq, SFA = syn.fp4_operand(M, K, seed=65)
    codes = np.zeros((K, K), np.uint8)
    codes[np.arange(K), np.arange(K)] = 2
    Bq = syn.pack_nibbles(codes)
    SFB = np.full((K, K // 16), 0x38, np.uint8)
    C = run_fp4(Aq, SFA, Bq, SFB, M, K, K)
    # compared as values: code 8 decodes to -0, and the sign of a zero sum is
    # not part of the contract
    want = syn.to_bf16_bits(oracle.decode_nvfp4(Aq, SFA, K))
    assert np.array_equal(tolerance.bf16_bits_to_f64(C), tolerance.bf16_bits_to_f64(want))


def test_fp4_workload_sampled_against_oracle():
    need_gpu()
    M = N = K = 8192
    Aq, SFA = syn.fp4_operand(M, K, seed=syn.seed_for(5, 0))
    Bq, SFB = syn.fp4_operand(N, K, seed=syn.seed_for(5, 0) + 1)
    C = run_fp4(Aq, SFA, Bq, SFB, M, N, K)
    ms, ns = sample_positions(M, N, 3000, seed=5)
    ref = oracle.gemm_nvfp4_nt_at(Aq, SFA, Bq, SFB, K, ms, ns)
    sig = _sigma(Aq[:512], SFA[:512], K) * _sigma(Bq[:512], SFB[:512], K)
    res = tolerance.check(C[ms, ns], ref, K, sig)
    assert res, res
    assert np.all(np.isfinite(tolerance.bf16_bits_to_f64(C)))


def test_fp4_workload_exactly_summable_every_element():
    # scales in {2^-1, 2^0}, all 16 codes, K = 8192: sums exact in FP32.
    need_gpu()
    M = N = K = 8192
    Aq = syn.fp4_codes(M, K, seed=71)
    Bq = syn.fp4_codes(N, K, seed=72)
    SFA = syn.e4m3_scales(M, K, seed=73, u_lo=-1, u_hi=0, m_lo=0, m_hi=0)
    SFB = syn.e4m3_scales(N, K, seed=74, u_lo=-1, u_hi=0, m_lo=0, m_hi=0)
    C = run_fp4(Aq, SFA, Bq, SFB, M, N, K)
    Ad = oracle.decode_nvfp4(Aq, SFA, K)
    Bd = oracle.decode_nvfp4(Bq, SFB, K)
    want = oracle.bf16_from_double(Ad @ Bd.T)
    ms, ns = sample_positions(M, N, 300, seed=8)
    assert np.array_equal(oracle.gemm_nvfp4_nt_at(Aq, SFA, Bq, SFB, K, ms, ns), want[ms, ns])
    bad = np.argwhere(C != want)
    assert bad.size == 0, "first mismatches %s" % bad[:5].tolist()


# ---- K % 64 == 32: the last K step is half past K -----------------------------
# Rows are contiguous, so the upper half of the last step, read as it stands,
# would fetch the first codes and scales of the next row; the kernel must read
# zeros there instead. Random codes in every row make any such leak visible.

@pytest.mark.parametrize("M,N,K", [(257, 264, 32), (300, 520, 96), (65, 264, 8160), (4352, 4104, 96),
                                   (8, 8, 32)])
def test_k_half_step_tail_matches_oracle(M, N, K):
    need_gpu()
    print("fp4 K tail", M, N, K, flush=True)
    Aq, SFA = syn.fp4_operand(M, K, seed=M + 7 * N + K)
    Bq, SFB = syn.fp4_operand(N, K, seed=M + 7 * N + K + 1)
    C = run_fp4(Aq, SFA, Bq, SFB, M, N, K)
    sig = _sigma(Aq[:512], SFA[:512], K) * _sigma(Bq[:512], SFB[:512], K)
    if M * N <= 300 * 520:
        res = tolerance.check(C, oracle.gemm_nvfp4_nt(Aq, SFA, Bq, SFB, K), K, sig)
    else:   # two rounds of tiles per workgroup: sampled, every tile edge included
        ms, ns = sample_positions(M, N, 4000, seed=K)
        res = tolerance.check(C[ms, ns], oracle.gemm_nvfp4_nt_at(Aq, SFA, Bq, SFB, K, ms, ns), K, sig)
    assert res, res


@pytest.mark.parametrize("M,N,K", [(264, 520, 480), (513, 256, 96), (4352, 4104, 32)])
def test_k_half_step_tail_exact_bitwise(M, N, K):
    # scales 2^0 * (1 + m/8), all 16 codes, K <= 512: every partial sum is
    # exact in FP32, so the answer is unique and a leaked half step would show
    need_gpu()
    print("fp4 K tail exact", M, N, K, flush=True)
    Aq = syn.fp4_codes(M, K, seed=K + 61)
    Bq = syn.fp4_codes(N, K, seed=K + 62)
    SFA = syn.e4m3_scales(M, K, seed=K + 63, u_lo=0, u_hi=0)
    SFB = syn.e4m3_scales(N, K, seed=K + 64, u_lo=0, u_hi=0)
    C = run_fp4(Aq, SFA, Bq, SFB, M, N, K)
    Ad, Bd = oracle.decode_nvfp4(Aq, SFA, K), oracle.decode_nvfp4(Bq, SFB, K)
    want = oracle.bf16_from_double(Ad @ Bd.T)
    ms, ns = sample_positions(M, N, 300, seed=K)
    assert np.array_equal(oracle.gemm_nvfp4_nt_at(Aq, SFA, Bq, SFB, K, ms, ns), want[ms, ns])
    bad = np.argwhere(C != want)
    assert bad.size == 0, "first mismatches %s" % bad[:5].tolist()


def test_k_half_step_tail_decoded_identity():
    # B = I (code 2 on the diagonal, unit scales) at K = 480: C = dec(A)
    need_gpu()
    M, K = 300, 480
    Aq, SFA = syn.fp4_operand(M, K, seed=66)
    codes = np.zeros((K, K), np.uint8)
    codes[np.arange(K), np.arange(K)] = 2
    Bq = syn.pack_nibbles(codes)
    SFB = np.full((K, K // 16), 0x38, np.uint8)
    C = run_fp4(Aq, SFA, Bq, SFB, M, K, K)
    want = syn.to_bf16_bits(oracle.decode_nvfp4(Aq, SFA, K))
    assert np.array_equal(tolerance.bf16_bits_to_f64(C), tolerance.bf16_bits_to_f64(want))


def test_k_half_step_tail_fused_epilogue():
    need_gpu()
    M, N, K = 300, 264, 96
    Aq, SFA = syn.fp4_operand(M, K, seed=67)
    Bq, SFB = syn.fp4_operand(N, K, seed=68)
    bias = syn.bf16_uniform(1, N, seed=69, lo=-64.0, hi=64.0)[0]
    C = GuardedC(M, N)
    g.gemm_nvfp4_nt_bias_act(M, N, K, *(to_dev(x) for x in (Aq, SFA, Bq, SFB)), to_dev(bias), g.ACT_GELU_TANH,
                             C.view)
    torch.cuda.synchronize()
    assert C.guards_intact(), "write outside C"
    ms, ns = (x.ravel() for x in np.meshgrid(np.arange(M), np.arange(N), indexing="ij"))
    ref, z = oracle.gemm_nvfp4_nt_bias_act_at(Aq, SFA, Bq, SFB, K, bias, g.ACT_GELU_TANH, ms, ns, with_z=True)
    sig = _sigma(Aq, SFA, K) * _sigma(Bq, SFB, K)
    res = tolerance.check_fused(C.bits(), ref.reshape(M, N), z.reshape(M, N), K, g.ACT_GELU_TANH, sig)
    assert res, res


# ---- dynamic tile order (gemm355_force_schedule) ------------------------------

@pytest.mark.parametrize("M,N,K", [(8192, 8192, 1024), (4352, 4104, 1024), (520, 776, 512), (2304, 2304, 256),
                                   (300, 264, 256)])
def test_dynamic_order_gives_the_static_result(M, N, K):
    # Every tile is computed the same way whichever workgroup takes it, so
    # the dynamic order must reproduce the static result bitwise. 4352 x 4104
    # has 289 tiles: the second round's 33 tiles all sit on one XCD's share,
    # so the other XCDs' workgroups take them from its counter. 520 x 776
    # (12 tiles, a grid of 8) and 300 x 264 (4 tiles, a grid of 4: one
    # counter) cover the small grids. Three dynamic launches in a row: a
    # counter left uncleared would make later launches skip tiles (their C
    # would keep the canary values).
    need_gpu()
    print("fp4 dynamic order", M, N, K, flush=True)
    Aq, SFA = syn.fp4_operand(M, K, seed=M + N + 3)
    Bq, SFB = syn.fp4_operand(N, K, seed=M + N + 4)
    want = run_fp4(Aq, SFA, Bq, SFB, M, N, K)
    try:
        g.force_schedule(g.SCHEDULE_DYNAMIC)
        for launch in range(3):
            got = run_fp4(Aq, SFA, Bq, SFB, M, N, K)
            bad = np.argwhere(got != want)
            assert bad.size == 0, "launch %d: %d differ, first %s" % (launch, len(bad), bad[:5].tolist())
    finally:
        g.force_schedule(g.SCHEDULE_STATIC)
    ms, ns = sample_positions(M, N, 500, seed=M)
    sig = _sigma(Aq[:512], SFA[:512], K) * _sigma(Bq[:512], SFB[:512], K)
    res = tolerance.check(want[ms, ns], oracle.gemm_nvfp4_nt_at(Aq, SFA, Bq, SFB, K, ms, ns), K, sig)
    assert res, res


def test_dynamic_order_leaves_other_calls_static():
    # the fused and the K % 64 == 32 instances keep the static order: results
    # with the option set equal those without it
    need_gpu()
    M, N, K = 520, 264, 96
    Aq, SFA = syn.fp4_operand(M, K, seed=91)
    Bq, SFB = syn.fp4_operand(N, K, seed=92)
    want = run_fp4(Aq, SFA, Bq, SFB, M, N, K)
    try:
        g.force_schedule(g.SCHEDULE_DYNAMIC)
        got = run_fp4(Aq, SFA, Bq, SFB, M, N, K)
    finally:
        g.force_schedule(g.SCHEDULE_STATIC)
    assert np.array_equal(got, want)
