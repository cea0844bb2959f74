"""Products at the largest sizes the boundary accepts, through the C ABI.

Operand extents, padded to whole 256-row tiles, must stay below 2^31 bytes
(the kernels address with 32-bit offsets and rely on the buffer range to turn
rows past M or N into zeros). These tests sit just inside that limit:

  * K at the limit with M = 3, N = 16: the offsets the kernels form for the
    padded rows 3 .. 255 reach 2^31 - 4 KiB and must all fall outside A's
    range; every BF16 instance forced in turn (split K through the workspace
    entry point), the FP4 kernel, and the
    microscaled FP4 kernel at K = 2^24 - 512;
  * C (and A) at the limit with M = 2^27 - 300, N = K = 8: the store offsets
    reach 2^31 - 8 KiB; sampled rows, including the last tile's, compared
    bitwise (K = 8 sixteenths: the sums are exact).
"""
import numpy as np
import pytest
import torch

import dense_gemm_14_amd as g
import oracle
import synthetic as syn
from tests import tolerance
from tests.gpu_util import GuardedC, need_gpu, to_dev, workspace_for, workspace_tail_intact

pytestmark = pytest.mark.gpu

K_BF16 = (1 << 22) - 8       # 256 padded rows x K x 2 bytes = 2^31 - 4096
K_FP4 = (1 << 24) - 64       # 256 padded rows x K / 2 bytes = 2^31 - 8192
K_MX = (1 << 24) - 512       # the same for the microscaled product (K % 512 == 0)


@pytest.mark.parametrize("instance,ws", [(g.INSTANCE_LARGE, False), (g.INSTANCE_SMALL, False),
                                         (g.INSTANCE_SPLITK, False), (g.INSTANCE_SPLITK, True),
                                         (g.INSTANCE_AUTO, False), (g.INSTANCE_AUTO, True)])
def test_bf16_k_at_extent_limit(instance, ws):
    need_gpu()
    M, N, K = 3, 16, K_BF16
    print("bf16 K limit", instance, ws, M, N, K, flush=True)
    A = syn.bf16_uniform(M, K, seed=101)
    B = syn.bf16_uniform(N, K, seed=102)
    C = GuardedC(M, N)
    try:
        g.force_instance(instance)
        if ws:   # one 128 x 128 tile: K is split eight ways
            buf, nbytes = workspace_for(M, N, K)
            assert instance == g.INSTANCE_AUTO or nbytes == 8 * 65536
            g.gemm_bf16_nt_ws(M, N, K, to_dev(A), to_dev(B), C.view, buf, nbytes)
        else:
            g.gemm_bf16_nt(M, N, K, to_dev(A), to_dev(B), C.view)
        torch.cuda.synchronize()
    finally:
        g.force_instance(g.INSTANCE_AUTO)
    assert C.guards_intact(), "write outside C"
    if ws:
        assert workspace_tail_intact(buf, nbytes), "write past the workspace"
    res = tolerance.check(C.bits(), oracle.gemm_bf16_nt(A, B), K)
    assert res, res


def test_fp4_k_at_extent_limit():
    need_gpu()
    M, N, K = 3, 16, K_FP4
    print("fp4 K limit", M, N, K, flush=True)
    Aq, SFA = syn.fp4_operand(M, K, seed=111)
    Bq, SFB = syn.fp4_operand(N, K, seed=112)
    C = GuardedC(M, N)
    g.gemm_nvfp4_nt(M, N, K, *(to_dev(x) for x in (Aq, SFA, Bq, SFB)), C.view)
    torch.cuda.synchronize()
    assert C.guards_intact(), "write outside C"
    sigma = (tolerance.sigma_of(oracle.decode_nvfp4(Aq[:, :1 << 16], SFA[:, :1 << 13], 1 << 17)) *
             tolerance.sigma_of(oracle.decode_nvfp4(Bq[:, :1 << 16], SFB[:, :1 << 13], 1 << 17)))
    ms, ns = (x.ravel() for x in np.meshgrid(np.arange(M), np.arange(N), indexing="ij"))
    want = oracle.gemm_nvfp4_nt_at(Aq, SFA, Bq, SFB, K, ms, ns).reshape(M, N)   # threads over elements
    res = tolerance.check(C.bits(), want, K, sigma)
    assert res, res


def test_mx_k_at_extent_limit():
    need_gpu()
    M, N, K = 3, 16, K_MX
    print("mx K limit", M, N, K, flush=True)
    Aq, SA = syn.mxfp4_operand(M, K, seed=113)
    Bq, SB = syn.mxfp4_operand(N, K, seed=114)
    C = GuardedC(M, N)
    g.gemm_mxfp4_nt(M, N, K, *(to_dev(x) for x in (Aq, SA, Bq, SB)), C.view)
    torch.cuda.synchronize()
    assert C.guards_intact(), "write outside C"
    ms, ns = (x.ravel() for x in np.meshgrid(np.arange(M), np.arange(N), indexing="ij"))
    want = oracle.gemm_mxfp4_nt_at(Aq, SA, Bq, SB, K, ms, ns).reshape(M, N)
    # sigma from the first 2^17 elements of each row, decoded from the
    # oracle's per-code and per-scale values
    e2 = np.array([oracle.e2m1_to_double(c) for c in range(16)])
    e8 = np.array([oracle.e8m0_to_double(b) if b != 0xFF else np.nan for b in range(256)])
    def dec(Q, S):
        Q, S = Q[:, :1 << 16], S[:, :1 << 12]
        return e2[np.stack([Q & 15, Q >> 4], -1).reshape(Q.shape[0], -1)] * np.repeat(e8[S], 32, axis=1)
    sigma = tolerance.sigma_of(dec(Aq, SA)) * tolerance.sigma_of(dec(Bq, SB))
    res = tolerance.check(C.bits(), want, K, sigma)
    assert res, res


def test_bf16_c_at_extent_limit():
    need_gpu()
    M, N, K = (1 << 27) - 300, 8, 8
    print("bf16 C limit", M, N, K, flush=True)
    A = syn.bf16_sixteenths_large(M, K, seed=121)
    B = syn.bf16_sixteenths(N, K, seed=122)
    dA = to_dev(A)
    C = torch.full((M * N + 64,), 0x7FC1, dtype=torch.int16, device="cuda")
    g.gemm_bf16_nt(M, N, K, dA, to_dev(B), C)
    torch.cuda.synchronize()
    del dA
    assert bool((C[M * N:] == 0x7FC1).all()), "write past C"
    rng = np.random.Generator(np.random.PCG64(123))
    rows = np.unique(np.concatenate([rng.integers(0, M, 3000), np.arange(M - 600, M), np.arange(0, 300)]))
    got = C[:M * N].view(M, N)[torch.from_numpy(rows).cuda()].cpu().numpy().view(np.uint16)
    want = oracle.gemm_bf16_nt(A[rows], B)
    assert np.array_equal(got, want)
