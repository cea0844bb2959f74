"""gemm_bf16_nt_noalloc (the BF16 product for callers that cannot allocate:
split-K partials in the library's fixed per-device scratch array) against
gemm_bf16_nt_ws with a caller workspace, through the C ABI: bitwise equal on
two calls in a row, the second smaller (the scratch still holds the first
call's partials), plus a shape that does not split K and the oracle's bound.
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


def _pair(M, N, K, seed):
    A = syn.bf16_uniform(M, K, seed=seed)
    B = syn.bf16_uniform(N, K, seed=seed + 1)
    dA, dB = to_dev(A), to_dev(B)
    ref_c = GuardedC(M, N)
    buf, nbytes = workspace_for(M, N, K)
    g.gemm_bf16_nt_ws(M, N, K, dA, dB, ref_c.view, buf, nbytes)
    c = GuardedC(M, N)
    g.gemm_bf16_nt_noalloc(M, N, K, dA, dB, c.view)
    torch.cuda.synchronize()
    assert ref_c.guards_intact() and c.guards_intact(), "write outside C"
    assert workspace_tail_intact(buf, nbytes), "write past the workspace"
    return A, B, ref_c.bits(), c.bits(), nbytes


def test_noalloc_matches_the_workspace_entry_point_twice_then_smaller():
    need_gpu()
    g.force_instance(g.INSTANCE_AUTO)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    # each call needs less scratch than the one before: the whole 16 MiB
    # (eight splits of 32 tiles), 9 MiB, then 1.9 MiB (six splits, ragged)
    shapes = [(64, 4096, 8192, 5), (136, 1032, 4104, 11), (72, 640, 3080, 21)]
    sizes = []
    for M, N, K, seed in shapes:
        print("noalloc", M, N, K, flush=True)
        assert g.bf16_plan(M, N, K, cus, with_workspace=True)[1] > 1
        A, B, want, got, nbytes = _pair(M, N, K, seed)
        sizes.append(nbytes)
        assert np.array_equal(got, want), "first mismatches %s" % np.argwhere(got != want)[:5].tolist()
        res = tolerance.check(got, oracle.gemm_bf16_nt(A, B), K)
        assert res, res
    assert sizes[0] == 16 << 20 and sizes[2] < sizes[1] < sizes[0], sizes


def test_noalloc_without_split_equals_the_plain_product():
    need_gpu()
    M, N, K = 300, 264, 520
    print("noalloc no split", M, N, K, flush=True)
    A = syn.bf16_uniform(M, K, seed=31)
    B = syn.bf16_uniform(N, K, seed=32)
    dA, dB = to_dev(A), to_dev(B)
    c0, c1 = GuardedC(M, N), GuardedC(M, N)
    g.gemm_bf16_nt(M, N, K, dA, dB, c0.view)
    g.gemm_bf16_nt_noalloc(M, N, K, dA, dB, c1.view)
    torch.cuda.synchronize()
    assert c1.guards_intact()
    assert np.array_equal(c0.bits(), c1.bits())
