"""Helpers for the GPU parity tests: device buffers with guard bands, sampled
output positions, and a skip when no GPU is present (the tests still fail
loudly when a GPU is present but the HIP library is not)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

GUARD = 4096          # elements of canary on each side of C
CANARY = 0x7FC1       # a BF16 NaN pattern no finite result can produce


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this host")


def to_dev(bits: np.ndarray) -> torch.Tensor:
    """numpy bits (uint16 or uint8) -> contiguous device tensor of the same bytes."""
    a = np.ascontiguousarray(bits)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda()
    if a.dtype == np.uint8:
        return torch.from_numpy(a).cuda()
    raise TypeError(a.dtype)


class GuardedC:
    """A BF16 output of M x N elements inside a canary-filled buffer."""

    def __init__(self, M: int, N: int):
        self.M, self.N = M, N
        self.buf = torch.full((M * N + 2 * GUARD,), CANARY, dtype=torch.int16, device="cuda")
        self.view = self.buf[GUARD:GUARD + M * N]

    def bits(self) -> np.ndarray:
        return self.view.cpu().numpy().view(np.uint16).reshape(self.M, self.N)

    def guards_intact(self) -> bool:
        host = self.buf.cpu().numpy().view(np.uint16)
        return bool(np.all(host[:GUARD] == CANARY) and np.all(host[GUARD + self.M * self.N:] == CANARY))


def workspace_for(M: int, N: int, K: int):
    """A device workspace for gemm_bf16_nt_ws at this shape (None when the
    plan needs none), with a canary tail that the product must not touch."""
    import dense_gemm_14_amd as g
    nbytes = g.workspace_size(M, N, K)
    if nbytes == 0:
        return None, 0
    buf = torch.full((nbytes // 2 + GUARD,), CANARY, dtype=torch.int16, device="cuda")
    return buf, nbytes


def workspace_tail_intact(buf, nbytes) -> bool:
    if buf is None:
        return True
    return bool(np.all(buf[nbytes // 2:].cpu().numpy().view(np.uint16) == CANARY))


def sample_positions(M: int, N: int, count: int, seed: int, tile: int = 256):
    """Random (m, n) plus every combination of tile-boundary rows and columns."""
    g = np.random.Generator(np.random.PCG64(seed))
    ms = list(g.integers(0, M, count))
    ns = list(g.integers(0, N, count))
    edge_m = sorted({x for t in range(0, M, tile) for x in (t, t + tile - 1) if x < M} | {M - 1})
    edge_n = sorted({x for t in range(0, N, tile) for x in (t, t + tile - 1) if x < N} | {N - 1})
    # every boundary row against a few columns, and every boundary column against a few rows
    pick_n = list(g.integers(0, N, 4)) + [0, N - 1]
    pick_m = list(g.integers(0, M, 4)) + [0, M - 1]
    for m in edge_m:
        for n in pick_n:
            ms.append(m)
            ns.append(n)
    for n in edge_n:
        for m in pick_m:
            ms.append(m)
            ns.append(n)
    return np.array(ms, dtype=np.int32), np.array(ns, dtype=np.int32)
