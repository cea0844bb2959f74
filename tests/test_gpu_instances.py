"""The three BF16 kernel instances (256 x 256 output tiles, 64 x 64 tiles, and
128 x 128 tiles -- through gemm_bf16_nt with one split storing C directly,
through gemm_bf16_nt_ws with K split over workgroups, FP32 partials in the
caller's workspace and a reduction), each forced through
gemm355_force_instance, against the oracle: ragged shapes element by element,
exactly summable inputs bitwise, K = 0, and B = I bitwise. The automatic
choice routes small and skinny problems away from the 256 x 256 instance, so
without forcing it would only see the large workload shapes."""
import numpy as np
import pytest
import torch

import dense_gemm_14_amd as g
import oracle
import synthetic as syn
from tests import tolerance
from tests.gpu_util import (GuardedC, need_gpu, sample_positions, to_dev, workspace_for,
                            workspace_tail_intact)

pytestmark = pytest.mark.gpu

# (instance, through gemm_bf16_nt_ws with a workspace)
INSTANCES = [(g.INSTANCE_LARGE, False), (g.INSTANCE_SMALL, False), (g.INSTANCE_SPLITK, False),
             (g.INSTANCE_SPLITK, True)]
IDS = ["large", "small", "splitk_1", "splitk_ws"]


@pytest.fixture
def forced(request):
    need_gpu()
    g.force_instance(request.param[0])
    yield request.param
    g.force_instance(g.INSTANCE_AUTO)


def run_bf16(A_bits, B_bits, M, N, K, ws=False):
    A = to_dev(A_bits) if A_bits is not None else None
    B = to_dev(B_bits) if B_bits is not None else None
    C = GuardedC(M, N)
    if ws:
        buf, nbytes = workspace_for(M, N, K)
        g.gemm_bf16_nt_ws(M, N, K, A, B, C.view, buf, nbytes)
    else:
        g.gemm_bf16_nt(M, N, K, A, B, C.view)
    torch.cuda.synchronize()
    assert C.guards_intact(), "write outside C"
    if ws:
        assert workspace_tail_intact(buf, nbytes), "write past the workspace"
    return C.bits()


SHAPES = [(1, 8, 8), (63, 72, 40), (65, 64, 136), (257, 264, 520), (300, 8, 1000), (128, 1032, 4104),
          (520, 264, 72)]


@pytest.mark.parametrize("forced", INSTANCES, indirect=True, ids=IDS)
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_forced_instance_matches_oracle(forced, M, N, K):
    A = syn.bf16_uniform(M, K, seed=5 * M + N + 3 * K)
    B = syn.bf16_uniform(N, K, seed=5 * M + N + 3 * K + 1)
    C = run_bf16(A, B, M, N, K, forced[1])
    res = tolerance.check(C, oracle.gemm_bf16_nt(A, B), K)
    assert res, res


@pytest.mark.parametrize("forced", INSTANCES, indirect=True, ids=IDS)
@pytest.mark.parametrize("M,N,K", [(200, 136, 2056), (64, 64, 64), (513, 520, 264)])
def test_forced_instance_exact_sums_bitwise(forced, M, N, K):
    A = syn.bf16_sixteenths(M, K, seed=31 + K)
    B = syn.bf16_sixteenths(N, K, seed=32 + K)
    assert np.array_equal(run_bf16(A, B, M, N, K, forced[1]), oracle.gemm_bf16_nt(A, B))


@pytest.mark.parametrize("forced", INSTANCES, indirect=True, ids=IDS)
def test_forced_instance_k_zero(forced):
    assert np.array_equal(run_bf16(None, None, 70, 72, 0, forced[1]), np.zeros((70, 72), np.uint16))


@pytest.mark.parametrize("forced", INSTANCES, indirect=True, ids=IDS)
def test_forced_instance_identity(forced):
    M, K = 96, 520
    A = syn.bf16_uniform(M, K, seed=77)
    B = syn.bf16_identity(K)
    assert np.array_equal(run_bf16(A, B, M, K, K, forced[1]), A)


def test_instances_agree_within_bound_at_a_medium_shape():
    need_gpu()
    M, N, K = 1024, 1024, 1024   # 16 tiles of 256 x 256: the automatic choice is 64 x 64
    A = syn.bf16_uniform(M, K, seed=91)
    B = syn.bf16_uniform(N, K, seed=92)
    ref = oracle.gemm_bf16_nt(A, B)
    try:
        for inst, ws in [(g.INSTANCE_AUTO, False), (g.INSTANCE_AUTO, True)] + INSTANCES:
            g.force_instance(inst)
            res = tolerance.check(run_bf16(A, B, M, N, K, ws), ref, K)
            assert res, (inst, ws, res)
    finally:
        g.force_instance(g.INSTANCE_AUTO)


# Shapes with more 256 x 256 tiles than workgroups, so workgroups run several
# tiles back to back (the next tile's first units are copied during the
# previous tile's last steps): ragged M and N, K tails, K just above the
# 192 that the 256 x 256 instance needs (four steps, the last one partial).
MULTI_TILE = [(4352, 4104, 520), (4400, 4400, 200), (4360, 4352, 1000)]


@pytest.mark.parametrize("M,N,K", MULTI_TILE)
def test_large_instance_multi_tile_sampled(M, N, K):
    need_gpu()
    A = syn.bf16_uniform(M, K, seed=M + 2 * K)
    B = syn.bf16_uniform(N, K, seed=N + 2 * K + 1)
    try:
        g.force_instance(g.INSTANCE_LARGE)
        C = run_bf16(A, B, M, N, K)
    finally:
        g.force_instance(g.INSTANCE_AUTO)
    ms, ns = sample_positions(M, N, 3000, seed=M + N + K)
    res = tolerance.check(C[ms, ns], oracle.gemm_bf16_nt_at(A, B, ms, ns), K)
    assert res, res


def test_large_instance_multi_tile_exact_every_element():
    # Multiples of 1/16: every partial sum is exact in FP32, so the answer is
    # unique; the exact sums are formed in float64 and rounded once by the
    # oracle's BF16 rounding, and the oracle itself is compared on a sample.
    need_gpu()
    M, N, K = 4352, 4104, 1032
    A = syn.bf16_sixteenths(M, K, seed=61)
    B = syn.bf16_sixteenths(N, K, seed=62)
    try:
        g.force_instance(g.INSTANCE_LARGE)
        C = run_bf16(A, B, M, N, K)
    finally:
        g.force_instance(g.INSTANCE_AUTO)
    want = oracle.bf16_from_double(tolerance.bf16_bits_to_f64(A) @ tolerance.bf16_bits_to_f64(B).T)
    ms, ns = sample_positions(M, N, 300, seed=9)
    assert np.array_equal(oracle.gemm_bf16_nt_at(A, B, ms, ns), want[ms, ns])
    bad = np.argwhere(C != want)
    assert bad.size == 0, "first mismatches %s" % bad[:5].tolist()


def test_splitk_many_splits_exact_every_element():
    # 2 x 9 tiles of 128 x 128 and 65 K steps: the automatic plan with a
    # workspace splits K eight ways (the last split has two steps, the last
    # step a K tail). With multiples of 1/16 every partial sum and the sum of
    # the partials is exact in FP32, so every element must match the
    # correctly rounded sum.
    need_gpu()
    M, N, K = 136, 1032, 4104
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert g.bf16_plan(M, N, K, cus, with_workspace=True) == (g.INSTANCE_SPLITK, 8)
    A = syn.bf16_sixteenths(M, K, seed=71)
    B = syn.bf16_sixteenths(N, K, seed=72)
    C = run_bf16(A, B, M, N, K, ws=True)
    want = oracle.bf16_from_double(tolerance.bf16_bits_to_f64(A) @ tolerance.bf16_bits_to_f64(B).T)
    assert np.array_equal(oracle.gemm_bf16_nt(A[:3], B), want[:3])
    bad = np.argwhere(C != want)
    assert bad.size == 0, "first mismatches %s" % bad[:5].tolist()


@pytest.mark.parametrize("M,N,K", [(2048, 2048, 2048), (1992, 2040, 2056)])
def test_single_split_direct_store_exact_every_element(M, N, K):
    # A quarter of the units' worth of 256 x 256 tiles: the automatic plan
    # runs one round of 128 x 128 tiles with one split each, which store C
    # directly (no partials, no reduction). Ragged M and N at the second shape;
    # multiples of 1/16 make the answer unique, so every element is compared.
    need_gpu()
    g.force_instance(g.INSTANCE_AUTO)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert g.bf16_plan(M, N, K, cus) == (g.INSTANCE_SPLITK, 1)
    A = syn.bf16_sixteenths(M, K, seed=M + 7)
    B = syn.bf16_sixteenths(N, K, seed=N + 8)
    C = run_bf16(A, B, M, N, K)
    want = oracle.bf16_from_double(tolerance.bf16_bits_to_f64(A) @ tolerance.bf16_bits_to_f64(B).T)
    assert np.array_equal(oracle.gemm_bf16_nt(A[:2], B), want[:2])
    bad = np.argwhere(C != want)
    assert bad.size == 0, "first mismatches %s" % bad[:5].tolist()


def test_splitk_streams_and_determinism():
    # The same split product on a side stream and on the default stream, each
    # with its own workspace, and twice in a row: bitwise equal (splits are
    # added in a fixed order) and within the bound of the oracle; the product
    # without a workspace (no split) is within the bound too.
    need_gpu()
    M, N, K = 128, 2048, 4096
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert g.bf16_plan(M, N, K, cus, with_workspace=True)[1] > 1
    A = syn.bf16_uniform(M, K, seed=81)
    B = syn.bf16_uniform(N, K, seed=82)
    s = torch.cuda.Stream()
    dA, dB = to_dev(A), to_dev(B)
    outs = []
    torch.cuda.synchronize()
    for stream in (s, None, None):
        if stream is None:
            C = GuardedC(M, N)
            buf, nbytes = workspace_for(M, N, K)
            g.gemm_bf16_nt_ws(M, N, K, dA, dB, C.view, buf, nbytes)
        else:
            with torch.cuda.stream(stream):
                C = GuardedC(M, N)
                buf, nbytes = workspace_for(M, N, K)
                g.gemm_bf16_nt_ws(M, N, K, dA, dB, C.view, buf, nbytes, stream=stream)
        torch.cuda.synchronize()
        assert C.guards_intact(), "write outside C"
        outs.append(C.bits())
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2])
    ref = oracle.gemm_bf16_nt(A, B)
    res = tolerance.check(outs[0], ref, K)
    assert res, res
    res = tolerance.check(run_bf16(A, B, M, N, K), ref, K)
    assert res, res


def test_workspace_too_small_is_rejected_without_launching():
    need_gpu()
    M, N, K = 128, 2048, 4096
    nbytes = g.workspace_size(M, N, K)
    assert nbytes > 0
    buf = torch.zeros(nbytes // 2, dtype=torch.int16, device="cuda")
    C = GuardedC(M, N)
    with pytest.raises(g.Gemm355Error) as e:
        g.gemm_bf16_nt_ws(M, N, K, to_dev(syn.bf16_uniform(M, K, 1)), to_dev(syn.bf16_uniform(N, K, 2)), C.view,
                          buf, nbytes - 16)
    assert e.value.status == g.ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert np.all(C.bits() == 0x7FC1), "C written by a rejected call"


# ---- the 64 x 64 instance's long-K staging (B in 512-byte row segments) -------
# Taken when K >= 4096 and the 64 x 64 tiles number at least half the compute
# units: ragged M and N, and K tails that end inside the last 4-step B unit.
LONG_SHAPES = [(520, 1040, 4104), (136, 8200, 4160), (128, 8192, 8192), (264, 2056, 4352)]


@pytest.mark.parametrize("M,N,K", LONG_SHAPES)
def test_small_instance_long_k_matches_oracle(M, N, K):
    need_gpu()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert K >= 4096 and 2 * (-(-M // 64)) * (-(-N // 64)) >= cus
    print("small long-K", M, N, K, flush=True)
    A = syn.bf16_uniform(M, K, seed=M + 5 * K)
    B = syn.bf16_uniform(N, K, seed=N + 5 * K + 1)
    try:
        g.force_instance(g.INSTANCE_SMALL)
        C = run_bf16(A, B, M, N, K)
    finally:
        g.force_instance(g.INSTANCE_AUTO)
    ms, ns = sample_positions(M, N, 4000, seed=M + N, tile=64)
    res = tolerance.check(C[ms, ns], oracle.gemm_bf16_nt_at(A, B, ms, ns), K)
    assert res, res


@pytest.mark.parametrize("M,N,K", [(520, 1040, 4104), (136, 8200, 4160)])
def test_small_instance_long_k_exact_every_element(M, N, K):
    need_gpu()
    A = syn.bf16_sixteenths(M, K, seed=M + 11)
    B = syn.bf16_sixteenths(N, K, seed=N + 12)
    try:
        g.force_instance(g.INSTANCE_SMALL)
        C = run_bf16(A, B, M, N, K)
    finally:
        g.force_instance(g.INSTANCE_AUTO)
    want = oracle.bf16_from_double(tolerance.bf16_bits_to_f64(A) @ tolerance.bf16_bits_to_f64(B).T)
    assert np.array_equal(oracle.gemm_bf16_nt(A[:2], B), want[:2])
    bad = np.argwhere(C != want)
    assert bad.size == 0, "first mismatches %s" % bad[:5].tolist()


def test_small_instance_long_k_fused_epilogue():
    need_gpu()
    M, N, K = 264, 2056, 4352
    A = syn.bf16_uniform(M, K, seed=21)
    B = syn.bf16_uniform(N, K, seed=22)
    bias = syn.bf16_uniform(1, N, seed=23, lo=-8.0, hi=8.0)[0]
    C = GuardedC(M, N)
    try:
        g.force_instance(g.INSTANCE_SMALL)
        g.gemm_bf16_nt_bias_act(M, N, K, to_dev(A), to_dev(B), to_dev(bias), g.ACT_GELU_TANH, C.view)
        torch.cuda.synchronize()
    finally:
        g.force_instance(g.INSTANCE_AUTO)
    assert C.guards_intact()
    ms, ns = sample_positions(M, N, 3000, seed=24, tile=64)
    ref, z = oracle.gemm_bf16_nt_bias_act_at(A, B, bias, g.ACT_GELU_TANH, ms, ns, with_z=True)
    res = tolerance.check_fused(C.bits()[ms, ns], ref, z, K, g.ACT_GELU_TANH)
    assert res, res


# The split instance on one row of 128 x 128 tiles (M <= 128), with and without
# a workspace, ragged N and K tails. Multiples of 1/16 make every partial sum
# exact, so every element must equal the correctly rounded sum whatever the
# split.
@pytest.mark.parametrize("M,N,K,ws", [(100, 1032, 4104, True), (128, 264, 8200, True), (7, 136, 1544, True),
                                      (128, 1032, 4104, False), (33, 72, 72, True)])
def test_one_tile_row_split_exact_every_element(M, N, K, ws):
    need_gpu()
    g.force_instance(g.INSTANCE_SPLITK)
    try:
        A = syn.bf16_sixteenths(M, K, seed=M + K)
        B = syn.bf16_sixteenths(N, K, seed=N + K)
        C = run_bf16(A, B, M, N, K, ws=ws)
    finally:
        g.force_instance(g.INSTANCE_AUTO)
    want = oracle.bf16_from_double(tolerance.bf16_bits_to_f64(A) @ tolerance.bf16_bits_to_f64(B).T)
    assert np.array_equal(oracle.gemm_bf16_nt(A[:2], B), want[:2])
    bad = np.argwhere(C != want)
    assert bad.size == 0, "first mismatches %s" % bad[:5].tolist()


def test_one_tile_row_split_workload_every_element():
    # The skinny workload shape, 128 x 8192 x 8192, through the split instance
    # with a workspace (four splits of 32 K steps): all of C against the oracle
    # on uniform inputs (about 1.5 s of oracle time).
    need_gpu()
    M, N, K = 128, 8192, 8192
    A = syn.bf16_uniform(M, K, seed=syn.seed_for(3, 0) + 21)
    B = syn.bf16_uniform(N, K, seed=syn.seed_for(3, 0) + 22)
    g.force_instance(g.INSTANCE_SPLITK)
    try:
        C = run_bf16(A, B, M, N, K, ws=True)
    finally:
        g.force_instance(g.INSTANCE_AUTO)
    res = tolerance.check(C, oracle.gemm_bf16_nt(A, B), K)
    assert res and res.n_bad == 0, res
