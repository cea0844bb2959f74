"""Graph capture. Every product enqueues only kernel launches on the caller's
stream (no allocation, no memset, no synchronisation, no query that capture
forbids once the compute-unit count is cached), so a call can be captured into
a HIP graph. Each product below is captured once on a side stream (default
priority), and the graph is replayed three times with eager work that
overwrites C and a device synchronisation between replays; every replay's C
must equal the eager call's bitwise (the kernels are deterministic).

Covered: the 64 x 64, 128 x 128 (one split) and 256 x 256 BF16 instances
through gemm_bf16_nt, a split product with its reduction through
gemm_bf16_nt_ws, gemm_bf16_nt_noalloc (its static scratch), the fused
epilogue, the NVFP4 and microscaled FP4 products, and the decode-first NVFP4
path (the decode launch and the BF16 product in one graph)."""
import numpy as np
import pytest
import torch

import dense_gemm_14_amd as g
import synthetic as syn
from tests.gpu_util import need_gpu, to_dev, workspace_for

pytestmark = pytest.mark.gpu


def _capture_and_replay(launch, C, reps=3):
    launch()
    torch.cuda.synchronize()
    ref = C.clone()
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    C.fill_(-1)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        launch()
    torch.cuda.synchronize()
    for r in range(reps):
        C.fill_(-1)                 # eager work on the default stream between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(C, ref), "replay %d differs from the eager result" % r
    del graph


def _bf16(M, N, K, seed):
    A = to_dev(syn.bf16_uniform(M, K, seed=seed))
    B = to_dev(syn.bf16_uniform(N, K, seed=seed + 1))
    C = torch.empty(M * N, dtype=torch.int16, device="cuda")
    return A, B, C


@pytest.mark.parametrize("M,N,K", [(1024, 1024, 1024), (2048, 2048, 2048), (4096, 4096, 1024)])
def test_bf16_plain_replays(M, N, K):
    need_gpu()
    A, B, C = _bf16(M, N, K, seed=M + K)
    print("graph bf16", M, N, K, g.bf16_plan(M, N, K, torch.cuda.get_device_properties(0).multi_processor_count),
          flush=True)
    _capture_and_replay(lambda: g.gemm_bf16_nt(M, N, K, A, B, C), C)


def test_bf16_split_with_workspace_replays():
    need_gpu()
    M, N, K = 136, 1032, 4104
    A, B, C = _bf16(M, N, K, seed=9)
    ws, nbytes = workspace_for(M, N, K)
    assert nbytes > 0
    _capture_and_replay(lambda: g.gemm_bf16_nt_ws(M, N, K, A, B, C, ws, nbytes), C)


def test_bf16_noalloc_replays():
    need_gpu()
    M, N, K = 64, 4096, 8192
    A, B, C = _bf16(M, N, K, seed=10)
    _capture_and_replay(lambda: g.gemm_bf16_nt_noalloc(M, N, K, A, B, C), C)


def test_bf16_fused_epilogue_replays():
    need_gpu()
    M, N, K = 1024, 2048, 512
    A, B, C = _bf16(M, N, K, seed=11)
    bias = to_dev(syn.bf16_uniform(1, N, seed=12, lo=-4.0, hi=4.0)[0])
    _capture_and_replay(lambda: g.gemm_bf16_nt_bias_act(M, N, K, A, B, bias, g.ACT_GELU_TANH, C), C)


@pytest.mark.parametrize("kind", ["nvfp4", "mx"])
def test_fp4_replays(kind):
    need_gpu()
    M, N, K = 1024, 1024, 1024
    op = syn.mxfp4_operand if kind == "mx" else syn.fp4_operand
    Aq, SA = op(M, K, seed=13)
    Bq, SB = op(N, K, seed=14)
    ops = [to_dev(x) for x in (Aq, SA, Bq, SB)]
    C = torch.empty(M * N, dtype=torch.int16, device="cuda")
    f = g.gemm_mxfp4_nt if kind == "mx" else g.gemm_nvfp4_nt
    _capture_and_replay(lambda: f(M, N, K, *ops, C), C)


def test_fp4_decode_first_replays():
    need_gpu()
    M, N, K = 1024, 1024, 1024
    Aq, SA = syn.fp4_operand(M, K, seed=15)
    Bq, SB = syn.fp4_operand(N, K, seed=16)
    ops = [to_dev(x) for x in (Aq, SA, Bq, SB)]
    C = torch.empty(M * N, dtype=torch.int16, device="cuda")
    g.force_fp4_path(g.FP4_PATH_DECODE_FIRST)
    try:
        nbytes = g.nvfp4_workspace_size(M, N, K)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        _capture_and_replay(lambda: g.gemm_nvfp4_nt_ws(M, N, K, *ops, C, ws, nbytes), C)
    finally:
        g.force_fp4_path(g.FP4_PATH_AUTO)
