"""Every element of the workload products on uniformly random data against
the oracle, through the C ABI (the sampled workload tests elsewhere check a
few thousand elements; these check all of C, or whole output tiles).

  * BF16 4096^3 and 128 x 8192 x 8192: all of C, i.i.d. uniform[-1, 1) inputs
    rounded to BF16, against oracle.gemm_bf16_nt (about 11 s and 1.4 s of
    oracle time on 16 host threads).
  * BF16 8192^3 and 8000^3: whole 256 x 256 tiles -- the tile that each of
    the first and the last workgroup of every XCD computes in every round of
    the persistent grid (every wave, lane and epilogue position of those
    tiles), plus the last row, last column and corner tiles, which are ragged
    at 8000.
  * NVFP4 and microscaled FP4 at 4096^3: all of C, with the workload's codes
    and scales. The oracle side decodes each operand with the oracle's own
    codecs (every decoded value is exact in BF16) and runs the oracle's BF16
    product: the identity the oracle tests pin for both formats.

Tolerance: |C - C_ref| <= 2^-7 |C_ref| + 2^-10 sqrt(K) (sigma_A sigma_B for
FP4), as for every other parity test.
"""
import numpy as np
import pytest
import torch

import dense_gemm_14_amd as g
import oracle
import synthetic as syn
from tests import tolerance
from tests.gpu_util import GuardedC, need_gpu, to_dev

pytestmark = pytest.mark.gpu

TILE = 256


def _run(launch, M, N):
    C = GuardedC(M, N)
    launch(C.view)
    torch.cuda.synchronize()
    assert C.guards_intact(), "write outside C"
    return C.bits()


def _check_all(got, ref, K, sigma=1.0, what=""):
    res = tolerance.check(got, ref, K, sigma)
    assert res, (what, res)
    assert res.n_bad == 0


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 4096), (128, 8192, 8192)])
def test_bf16_every_element(M, N, K):
    need_gpu()
    print("bf16 every element", M, N, K, flush=True)
    cfg = 1 if M == 4096 else 3
    A = syn.bf16_uniform(M, K, seed=syn.seed_for(cfg, 0))
    B = syn.bf16_uniform(N, K, seed=syn.seed_for(cfg, 0) + 1)
    got = _run(lambda c: g.gemm_bf16_nt(M, N, K, to_dev(A), to_dev(B), c), M, N)
    _check_all(got, oracle.gemm_bf16_nt(A, B), K, what=(M, N, K))


def _checked_tiles(M, N, K, cus):
    """(tm, tn) of the tiles computed by the first and last workgroup of each
    XCD in every round, plus the last row, last column and corner tiles."""
    tm_n, tn_n = -(-M // TILE), -(-N // TILE)
    tiles = tm_n * tn_n
    grid = min(tiles, cus) & ~7
    order_m, order_n = g.tile_order(tm_n, tn_n, g.supergroup(tn_n, K))
    slots = g.schedule(tiles, grid)
    picked = set()
    for x in range(8):
        for w in (x, grid - 8 + x):          # first and last workgroup of XCD x
            for pos in slots[w]:
                if pos >= 0:
                    picked.add((order_m[pos], order_n[pos]))
    for t in range(0, max(tm_n, tn_n), 7):
        picked.add((min(t, tm_n - 1), tn_n - 1))
        picked.add((tm_n - 1, min(t, tn_n - 1)))
    picked.add((tm_n - 1, tn_n - 1))
    return sorted(picked)


@pytest.mark.parametrize("M,N,K", [(8192, 8192, 8192), (8000, 8000, 8000)])
def test_bf16_whole_tiles(M, N, K):
    need_gpu()
    print("bf16 whole tiles", M, N, K, flush=True)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    cfg = 2 if M == 8192 else 3
    A = syn.bf16_uniform(M, K, seed=syn.seed_for(cfg, 0) + 2)
    B = syn.bf16_uniform(N, K, seed=syn.seed_for(cfg, 0) + 3)
    got = _run(lambda c: g.gemm_bf16_nt(M, N, K, to_dev(A), to_dev(B), c), M, N)
    tiles = _checked_tiles(M, N, K, cus)
    assert len(tiles) >= 64
    ms, ns = [], []
    for tm, tn in tiles:
        r = np.arange(tm * TILE, min(M, tm * TILE + TILE), dtype=np.int32)
        c = np.arange(tn * TILE, min(N, tn * TILE + TILE), dtype=np.int32)
        mm, nn = np.meshgrid(r, c, indexing="ij")
        ms.append(mm.ravel())
        ns.append(nn.ravel())
    ms, ns = np.concatenate(ms), np.concatenate(ns)
    _check_all(got[ms, ns], oracle.gemm_bf16_nt_at(A, B, ms, ns), K, what=(M, N, K, len(tiles)))
    assert np.all(np.isfinite(tolerance.bf16_bits_to_f64(got)))


def _e2m1_table():
    return np.array([oracle.e2m1_to_double(c) for c in range(16)])


def _unpack(Q):
    return np.stack([Q & 15, Q >> 4], -1).reshape(Q.shape[0], -1)


def test_nvfp4_every_element_4096():
    need_gpu()
    M = N = K = 4096
    print("nvfp4 every element", M, N, K, flush=True)
    Aq, SFA = syn.fp4_operand(M, K, seed=syn.seed_for(4, 0) + 7)
    Bq, SFB = syn.fp4_operand(N, K, seed=syn.seed_for(4, 0) + 8)
    got = _run(lambda c: g.gemm_nvfp4_nt(M, N, K, *(to_dev(x) for x in (Aq, SFA, Bq, SFB)), c), M, N)
    Ad, Bd = oracle.decode_nvfp4(Aq, SFA, K), oracle.decode_nvfp4(Bq, SFB, K)
    Ab, Bb = oracle.bf16_from_double(Ad), oracle.bf16_from_double(Bd)
    assert np.array_equal(oracle.bf16_to_double(Ab), Ad)   # the decode is exact in BF16
    ref = oracle.gemm_bf16_nt(Ab, Bb)
    _check_all(got, ref, K, tolerance.sigma_of(Ad) * tolerance.sigma_of(Bd), what="nvfp4")


def test_mxfp4_every_element_4096():
    need_gpu()
    M = N = K = 4096
    print("mxfp4 every element", M, N, K, flush=True)
    Aq, SA = syn.mxfp4_operand(M, K, seed=syn.seed_for(4, 0) + 9)
    Bq, SB = syn.mxfp4_operand(N, K, seed=syn.seed_for(4, 0) + 10)
    got = _run(lambda c: g.gemm_mxfp4_nt(M, N, K, *(to_dev(x) for x in (Aq, SA, Bq, SB)), c), M, N)
    e2 = _e2m1_table()
    e8 = np.array([oracle.e8m0_to_double(b) if b != 0xFF else np.nan for b in range(256)])
    Ad = e2[_unpack(Aq)] * np.repeat(e8[SA], 32, axis=1)
    Bd = e2[_unpack(Bq)] * np.repeat(e8[SB], 32, axis=1)
    Ab, Bb = oracle.bf16_from_double(Ad), oracle.bf16_from_double(Bd)
    assert np.array_equal(oracle.bf16_to_double(Ab), Ad)
    # the decoded product is the oracle's microscaled product (checked here on rows)
    rows = np.arange(0, M, 512)
    assert np.array_equal(oracle.gemm_bf16_nt(Ab[rows], Bb), oracle.gemm_mxfp4_nt(Aq[rows], SA[rows], Bq, SB, K))
    ref = oracle.gemm_bf16_nt(Ab, Bb)
    _check_all(got, ref, K, tolerance.sigma_of(Ad) * tolerance.sigma_of(Bd), what="mxfp4")
