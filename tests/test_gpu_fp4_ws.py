"""Parity of gemm_nvfp4_nt_ws and gemm_nvfp4_nt_bias_act_ws, the NVFP4
products with a caller-owned workspace, through the C ABI. Its decode-first path decodes each operand once
into BF16 rows in the workspace and runs the BF16 kernels on them; it is forced
(gemm355_force_fp4_path) at ragged and K-tail shapes so that small problems
exercise it too, and taken by shape at 8192^3. Checks: the oracle within the
FP4 parity bound (absolute term scaled by sigma_A sigma_B), exactly summable
inputs bitwise, the staging path equal to gemm_nvfp4_nt bitwise, a workspace
guard band that stays intact, and a too-small workspace rejected before any
work is enqueued."""
import numpy as np
import pytest
import torch

import dense_gemm_14_amd as g
import oracle
import synthetic as syn
from tests import tolerance
from tests.gpu_util import GUARD, CANARY, GuardedC, need_gpu, sample_positions, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture
def path(request):
    need_gpu()
    g.force_fp4_path(request.param)
    yield request.param
    g.force_fp4_path(g.FP4_PATH_AUTO)


def run_ws(Aq, SFA, Bq, SFB, M, N, K):
    nbytes = g.nvfp4_workspace_size(M, N, K)
    ws = torch.full((nbytes // 2 + GUARD,), CANARY, dtype=torch.int16, device="cuda") if nbytes else None
    C = GuardedC(M, N)
    g.gemm_nvfp4_nt_ws(M, N, K, to_dev(Aq), to_dev(SFA), to_dev(Bq), to_dev(SFB), C.view, ws, nbytes)
    torch.cuda.synchronize()
    assert C.guards_intact(), "write outside C"
    if ws is not None:
        tail = ws[nbytes // 2:].cpu().numpy()
        assert np.all(tail == CANARY), "write past the workspace"
    return C.bits()


def _sigma(Q, SF, K):
    return tolerance.sigma_of(oracle.decode_nvfp4(Q, SF, K))


@pytest.mark.parametrize("path", [g.FP4_PATH_DECODE_FIRST], indirect=True)
@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (1, 8, 64), (65, 72, 128), (257, 264, 192), (300, 8, 1024),
                                   (128, 1024, 512), (257, 264, 32), (300, 520, 96), (65, 264, 8160),
                                   # more rows than the decode grid's 8192 waves: waves walk several rows,
                                   # some across the boundary from A's rows to B's
                                   (8200, 304, 64), (304, 8200, 96)])
def test_decode_first_matches_oracle(path, M, N, K):
    Aq, SFA = syn.fp4_operand(M, K, seed=M + 7 * N + K)
    Bq, SFB = syn.fp4_operand(N, K, seed=M + 7 * N + K + 1)
    assert g.nvfp4_workspace_size(M, N, K) > 0
    C = run_ws(Aq, SFA, Bq, SFB, M, N, K)
    ref = oracle.gemm_nvfp4_nt(Aq, SFA, Bq, SFB, K)
    res = tolerance.check(C, ref, K, _sigma(Aq, SFA, K) * _sigma(Bq, SFB, K))
    assert res, res


@pytest.mark.parametrize("path", [g.FP4_PATH_DECODE_FIRST], indirect=True)
@pytest.mark.parametrize("M,N,K", [(264, 520, 512), (513, 256, 448), (100, 136, 96)])
def test_decode_first_exact_sums_bitwise(path, M, N, K):
    # scales 2^0 * (1 + m/8), all 16 codes, K <= 512: sums exact in FP32
    Aq = syn.fp4_codes(M, K, seed=81)
    Bq = syn.fp4_codes(N, K, seed=82)
    SFA = syn.e4m3_scales(M, K, seed=83, u_lo=0, u_hi=0)
    SFB = syn.e4m3_scales(N, K, seed=84, u_lo=0, u_hi=0)
    C = run_ws(Aq, SFA, Bq, SFB, M, N, K)
    assert np.array_equal(C, oracle.gemm_nvfp4_nt(Aq, SFA, Bq, SFB, K))


@pytest.mark.parametrize("path", [g.FP4_PATH_STAGING], indirect=True)
def test_staging_path_equals_gemm_nvfp4_nt(path):
    M, N, K = 520, 264, 1056
    Aq, SFA = syn.fp4_operand(M, K, seed=91)
    Bq, SFB = syn.fp4_operand(N, K, seed=92)
    assert g.nvfp4_workspace_size(M, N, K) == 0
    C = run_ws(Aq, SFA, Bq, SFB, M, N, K)
    D = GuardedC(M, N)
    g.gemm_nvfp4_nt(M, N, K, to_dev(Aq), to_dev(SFA), to_dev(Bq), to_dev(SFB), D.view)
    torch.cuda.synchronize()
    assert np.array_equal(C, D.bits())


def test_workload_decodes_first_and_is_exact_every_element():
    # 8192^3 on 256 units is four rounds of tiles: the shape rule decodes
    # first. Scales in {2^-1, 2^0} with all 16 codes keep every sum exact.
    need_gpu()
    M = N = K = 8192
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if cus <= 256:
        assert g.nvfp4_plan(M, N, K, cus) == (True, 4 * M * K)
    Aq = syn.fp4_codes(M, K, seed=101)
    Bq = syn.fp4_codes(N, K, seed=102)
    SFA = syn.e4m3_scales(M, K, seed=103, u_lo=-1, u_hi=0, m_lo=0, m_hi=0)
    SFB = syn.e4m3_scales(N, K, seed=104, u_lo=-1, u_hi=0, m_lo=0, m_hi=0)
    C = run_ws(Aq, SFA, Bq, SFB, M, N, K)
    want = oracle.bf16_from_double(oracle.decode_nvfp4(Aq, SFA, K) @ oracle.decode_nvfp4(Bq, SFB, K).T)
    ms, ns = sample_positions(M, N, 200, seed=9)
    assert np.array_equal(oracle.gemm_nvfp4_nt_at(Aq, SFA, Bq, SFB, K, ms, ns), want[ms, ns])
    bad = np.argwhere(C != want)
    assert bad.size == 0, "first mismatches %s" % bad[:5].tolist()


def test_workload_sampled_against_oracle():
    need_gpu()
    M = N = K = 8192
    Aq, SFA = syn.fp4_operand(M, K, seed=syn.seed_for(5, 0) + 40)
    Bq, SFB = syn.fp4_operand(N, K, seed=syn.seed_for(5, 0) + 41)
    C = run_ws(Aq, SFA, Bq, SFB, M, N, K)
    ms, ns = sample_positions(M, N, 3000, seed=15)
    ref = oracle.gemm_nvfp4_nt_at(Aq, SFA, Bq, SFB, K, ms, ns)
    sig = _sigma(Aq[:512], SFA[:512], K) * _sigma(Bq[:512], SFB[:512], K)
    res = tolerance.check(C[ms, ns], ref, K, sig)
    assert res, res
    assert np.all(np.isfinite(tolerance.bf16_bits_to_f64(C)))


@pytest.mark.parametrize("path", [g.FP4_PATH_DECODE_FIRST], indirect=True)
def test_small_workspace_is_rejected_without_launching(path):
    M, N, K = 72, 64, 96
    Aq, SFA = syn.fp4_operand(M, K, seed=111)
    Bq, SFB = syn.fp4_operand(N, K, seed=112)
    nbytes = g.nvfp4_workspace_size(M, N, K)
    assert nbytes == -(-2 * M * K // 256) * 256 + 2 * N * K
    ws = torch.full((nbytes // 2,), CANARY, dtype=torch.int16, device="cuda")
    C = GuardedC(M, N)
    with pytest.raises(g.Gemm355Error) as e:
        g.gemm_nvfp4_nt_ws(M, N, K, to_dev(Aq), to_dev(SFA), to_dev(Bq), to_dev(SFB), C.view, ws, nbytes - 16)
    assert e.value.status == g.ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert np.all(C.bits() == CANARY) and bool(torch.all(ws == CANARY))


# ---- the fused epilogue through the workspace (gemm_nvfp4_nt_bias_act_ws) -----

ACTS = [g.ACT_NONE, g.ACT_RELU, g.ACT_GELU_TANH]


def run_ws_fused(Aq, SFA, Bq, SFB, bias, act, M, N, K):
    nbytes = g.nvfp4_workspace_size(M, N, K)
    ws = torch.full((nbytes // 2 + GUARD,), CANARY, dtype=torch.int16, device="cuda") if nbytes else None
    C = GuardedC(M, N)
    g.gemm_nvfp4_nt_bias_act_ws(M, N, K, to_dev(Aq), to_dev(SFA), to_dev(Bq), to_dev(SFB),
                                to_dev(bias) if bias is not None else None, act, C.view, ws, nbytes)
    torch.cuda.synchronize()
    assert C.guards_intact(), "write outside C"
    if ws is not None:
        assert np.all(ws[nbytes // 2:].cpu().numpy() == CANARY), "write past the workspace"
    return C.bits()


@pytest.mark.parametrize("path", [g.FP4_PATH_DECODE_FIRST], indirect=True)
@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("M,N,K", [(300, 264, 512), (65, 72, 96)])
def test_fused_decode_first_matches_oracle(path, act, M, N, K):
    Aq, SFA = syn.fp4_operand(M, K, seed=M + K + 3 * act)
    Bq, SFB = syn.fp4_operand(N, K, seed=N + K + 1)
    sigma = _sigma(Aq, SFA, K) * _sigma(Bq, SFB, K)
    # bias on the scale of the sums, so the activations' bend is exercised
    bias = syn.bf16_uniform(1, N, seed=N + 9, lo=-sigma * K ** 0.5, hi=sigma * K ** 0.5)[0]
    got = run_ws_fused(Aq, SFA, Bq, SFB, bias, act, M, N, K)
    ms, ns = (x.ravel() for x in np.meshgrid(np.arange(M), np.arange(N), indexing="ij"))
    ref, z = oracle.gemm_nvfp4_nt_bias_act_at(Aq, SFA, Bq, SFB, K, bias, act, ms, ns, with_z=True)
    res = tolerance.check_fused(got, ref.reshape(M, N), z.reshape(M, N), K, act, sigma)
    assert res, res


@pytest.mark.parametrize("path", [g.FP4_PATH_DECODE_FIRST], indirect=True)
@pytest.mark.parametrize("act", [g.ACT_NONE, g.ACT_RELU])
def test_fused_decode_first_exact_inputs_bitwise(path, act):
    # unit-exponent scales (1 + m/8) with K = 256: every partial sum is a
    # multiple of 2^-8 below 2^15, exact in FP32, and so is the bias sum
    M, N, K = 264, 256, 256
    Aq, Bq = syn.fp4_codes(M, K, seed=241), syn.fp4_codes(N, K, seed=242)
    SFA = syn.e4m3_scales(M, K, seed=243, u_lo=0, u_hi=0)
    SFB = syn.e4m3_scales(N, K, seed=244, u_lo=0, u_hi=0)
    bias = syn.bf16_sixteenths(1, N, seed=245, jmax=64)[0]
    got = run_ws_fused(Aq, SFA, Bq, SFB, bias, act, M, N, K)
    ms, ns = (x.ravel() for x in np.meshgrid(np.arange(M), np.arange(N), indexing="ij"))
    assert np.array_equal(got, oracle.gemm_nvfp4_nt_bias_act_at(Aq, SFA, Bq, SFB, K, bias, act, ms, ns).reshape(M, N))


@pytest.mark.parametrize("path", [g.FP4_PATH_STAGING], indirect=True)
def test_fused_staging_path_equals_gemm_nvfp4_nt_bias_act(path):
    M, N, K = 520, 264, 1056
    Aq, SFA = syn.fp4_operand(M, K, seed=251)
    Bq, SFB = syn.fp4_operand(N, K, seed=252)
    bias = syn.bf16_uniform(1, N, seed=253, lo=-50.0, hi=50.0)[0]
    assert g.nvfp4_workspace_size(M, N, K) == 0
    C = run_ws_fused(Aq, SFA, Bq, SFB, bias, g.ACT_GELU_TANH, M, N, K)
    D = GuardedC(M, N)
    g.gemm_nvfp4_nt_bias_act(M, N, K, to_dev(Aq), to_dev(SFA), to_dev(Bq), to_dev(SFB), to_dev(bias),
                             g.ACT_GELU_TANH, D.view)
    torch.cuda.synchronize()
    assert np.array_equal(C, D.bits())
