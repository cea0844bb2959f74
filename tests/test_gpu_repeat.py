"""Repeated launches of the persistent 256 x 256 kernels give bitwise the same C.

Their workgroups take several output tiles in turn (four each at M = N = 8192
on 256 compute units), and the BF16 and microscaled kernels carry their LDS
copy ring from one tile into the next, behind the previous tile's epilogue
stores. Each product here is launched once for its reference, then again and
again, alternating with launches on a second input set so that every tile
boundary carries the other set's data through the ring, and every repeat must
equal the reference bitwise. An ordering mistake between copies, LDS reads
and stores shows up as a result that changes from launch to launch. The
values themselves are checked against the oracle by the parity tests; this
file checks only that they repeat.
"""
import pytest
import torch

import dense_gemm_14_amd as g
import synthetic as syn
from tests.gpu_util import need_gpu, to_dev

pytestmark = pytest.mark.gpu

REPEATS = 24


def _repeats_bitwise(name, launch, M, N):
    """launch(set_index, C) runs the product on input set 0 or 1 into C."""
    print("repeat", name, flush=True)
    c0 = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    c1 = torch.empty_like(c0)
    launch(0, c0)
    torch.cuda.synchronize()
    ref = c0.view(torch.int16).clone()
    wrong = []
    for r in range(REPEATS):
        launch(1, c1)
        c0.fill_(float("nan"))
        launch(0, c0)
        if r % 4 == 3:
            torch.cuda.synchronize()
        if not torch.equal(c0.view(torch.int16), ref):
            wrong.append(r)
    torch.cuda.synchronize()
    assert not wrong, "%s: repeats %s differ from the first launch" % (name, wrong)


@pytest.mark.parametrize("K", [1024, 1000])   # whole K steps; a K tail (the range-checked copy form)
def test_bf16_repeats(K):
    need_gpu()
    M = N = 8192
    A = [to_dev(syn.bf16_uniform(M, K, seed=901 + 2 * s)) for s in range(2)]
    B = [to_dev(syn.bf16_uniform(N, K, seed=902 + 2 * s)) for s in range(2)]
    _repeats_bitwise("bf16 %dx%dx%d" % (M, N, K), lambda s, c: g.gemm_bf16_nt(M, N, K, A[s], B[s], c), M, N)


def test_mxfp4_repeats():
    need_gpu()
    M = N = 8192
    K = 1024
    ops = [[syn.mxfp4_operand(rows, K, seed=911 + 2 * s + t) for t, rows in enumerate((M, N))] for s in range(2)]
    dev = [[(to_dev(q), to_dev(sc)) for q, sc in pair] for pair in ops]

    def launch(s, c):
        (aq, sa), (bq, sb) = dev[s]
        g.gemm_mxfp4_nt(M, N, K, aq, sa, bq, sb, c)

    _repeats_bitwise("mxfp4 %dx%dx%d" % (M, N, K), launch, M, N)


def test_nvfp4_repeats():
    need_gpu()
    M = N = 8192
    K = 1024
    ops = [[syn.fp4_operand(rows, K, seed=921 + 2 * s + t) for t, rows in enumerate((M, N))] for s in range(2)]
    dev = [[(to_dev(q), to_dev(sc)) for q, sc in pair] for pair in ops]

    def launch(s, c):
        (aq, sa), (bq, sb) = dev[s]
        g.gemm_nvfp4_nt(M, N, K, aq, sa, bq, sb, c)

    _repeats_bitwise("nvfp4 %dx%dx%d" % (M, N, K), launch, M, N)
