"""The C ABI without a GPU: the library loads, exports what its header
declares, rejects bad arguments before any HIP call, and its host-side tile
schedule is a bijection with the documented order. No compute is launched.
"""
import ctypes
import os

import numpy as np
import pytest

import dense_gemm_14_amd as g

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

FAKE = 0x10000  # a 16-byte-aligned address that is never dereferenced


def test_library_exports_every_declared_function():
    lib = g.load()
    names = g.declared_functions()
    assert set(names) >= {"gemm_bf16_nt", "gemm_bf16_nt_bias_act", "gemm_nvfp4_nt", "gemm_nvfp4_nt_bias_act",
                          "gemm_mxfp4_nt", "gemm355_status_string", "gemm_bf16_nt_ws", "gemm_bf16_nt_bias_act_ws",
                          "gemm_bf16_nt_workspace_size",
                          "gemm355_tile_order", "gemm355_schedule"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for s in range(5):
        assert g.status_string(s)
    assert g.status_string(99) == "unknown status"


def _bf16(M, N, K, a=FAKE, b=FAKE + 0x100000, c=FAKE + 0x200000):
    return g.load().gemm_bf16_nt(M, N, K, a, b, c, None)


def _fp4(M, N, K, aq=FAKE, sfa=FAKE + 0x100000, bq=FAKE + 0x200000, sfb=FAKE + 0x300000, c=FAKE + 0x400000):
    return g.load().gemm_nvfp4_nt(M, N, K, aq, sfa, bq, sfb, c, None)


def _mx(M, N, K, aq=FAKE, sa=FAKE + 0x100000, bq=FAKE + 0x200000, sb=FAKE + 0x300000, c=FAKE + 0x400000):
    return g.load().gemm_mxfp4_nt(M, N, K, aq, sa, bq, sb, c, None)


@pytest.mark.parametrize("fn,K", [(_bf16, 64), (_fp4, 64), (_mx, 512)])
def test_rejections_happen_before_any_device_call(fn, K):
    assert fn(-1, 8, K) == g.ERR_INVALID_ARG
    assert fn(8, -8, K) == g.ERR_INVALID_ARG
    assert fn(8, 8, -K) == g.ERR_INVALID_ARG
    # empty output: nothing to do, even with NULL pointers
    assert fn(0, 8, K, None, None, None) == g.OK if fn is _bf16 else fn(0, 8, K, None, None, None, None, None) == g.OK
    assert fn(8, 8, K, c=None) == g.ERR_INVALID_ARG
    assert fn(8, 12, K) == g.ERR_UNSUPPORTED          # N % 8
    assert fn(8, 8, K, c=FAKE + 0x900008) == g.ERR_UNSUPPORTED  # C not 16-byte aligned


def test_bf16_specific_rejections():
    assert _bf16(8, 8, 64, a=None) == g.ERR_INVALID_ARG
    assert _bf16(8, 8, 12) == g.ERR_UNSUPPORTED                   # K % 8
    assert _bf16(8, 8, 64, a=FAKE + 2) == g.ERR_UNSUPPORTED
    assert _bf16(1 << 16, 8, 1 << 15, b=1 << 40, c=1 << 41) == g.ERR_UNSUPPORTED  # A spans 4 GiB
    # C overlapping A
    assert _bf16(8, 8, 64, a=FAKE, c=FAKE + 64) == g.ERR_INVALID_ARG


def _fused(M, N, K, act=0, bias=FAKE + 0x300000, a=FAKE, b=FAKE + 0x100000, c=FAKE + 0x200000):
    return g.load().gemm_bf16_nt_bias_act(M, N, K, a, b, bias, act, c, None)


def test_fused_epilogue_rejections():
    # the plain product's rules, then the activation and the bias
    assert _fused(-1, 8, 64) == g.ERR_INVALID_ARG
    assert _fused(8, 12, 64) == g.ERR_UNSUPPORTED                  # N % 8
    assert _fused(8, 8, 64, c=None) == g.ERR_INVALID_ARG
    for bad_act in (-1, 3, 99):
        assert _fused(8, 8, 64, act=bad_act) == g.ERR_INVALID_ARG
        assert _fused(0, 8, 64, act=bad_act) == g.ERR_INVALID_ARG   # checked even with nothing to do
    assert _fused(8, 8, 64, bias=FAKE + 0x300008) == g.ERR_UNSUPPORTED   # bias not 16-byte aligned
    assert _fused(8, 8, 64, bias=FAKE + 0x200000 + 64) == g.ERR_INVALID_ARG  # bias inside C
    # empty output with a valid activation: nothing to do
    assert _fused(0, 8, 64, act=g.ACT_GELU_TANH, a=None, b=None, bias=None, c=None) == g.OK


def _fused4(M, N, K, act=0, bias=FAKE + 0x500000, c=FAKE + 0x400000):
    return g.load().gemm_nvfp4_nt_bias_act(M, N, K, FAKE, FAKE + 0x100000, FAKE + 0x200000, FAKE + 0x300000,
                                           bias, act, c, None)


def test_fp4_fused_epilogue_rejections():
    assert _fused4(8, 8, 48) == g.ERR_UNSUPPORTED                  # K % 32
    for bad_act in (-1, 3):
        assert _fused4(8, 8, 64, act=bad_act) == g.ERR_INVALID_ARG
    assert _fused4(8, 8, 64, bias=FAKE + 0x500004) == g.ERR_UNSUPPORTED
    assert _fused4(8, 8, 64, bias=FAKE + 0x400000 + 16) == g.ERR_INVALID_ARG   # bias inside C
    assert _fused4(0, 8, 64, act=g.ACT_RELU, bias=None, c=None) == g.OK


def _fused_mx(M, N, K, act=0, bias=FAKE + 0x500000, c=FAKE + 0x400000):
    return g.load().gemm_mxfp4_nt_bias_act(M, N, K, FAKE, FAKE + 0x100000, FAKE + 0x200000, FAKE + 0x300000,
                                           bias, act, c, None)


def test_mx_fused_epilogue_rejections():
    assert _fused_mx(8, 8, 256) == g.ERR_UNSUPPORTED                # K % 512
    for bad_act in (-1, 3):
        assert _fused_mx(8, 8, 512, act=bad_act) == g.ERR_INVALID_ARG
    assert _fused_mx(8, 8, 512, bias=FAKE + 0x500004) == g.ERR_UNSUPPORTED   # bias 16-byte aligned
    assert _fused_mx(8, 8, 512, bias=FAKE + 0x400000 + 16) == g.ERR_INVALID_ARG   # bias inside C
    assert _fused_mx(8, 12, 512) == g.ERR_UNSUPPORTED               # N % 8
    assert _fused_mx(0, 8, 512, act=g.ACT_GELU_TANH, bias=None, c=None) == g.OK


def test_extent_limits_are_exact():
    # Operand extents, padded to whole 256-row tiles, must stay below 2^31
    # bytes. Just inside, validation passes and the call stops at the missing
    # device (NO_DEVICE here); at the limit it is UNSUPPORTED. The calls just
    # inside carry fake addresses, so they run only where there is no device.
    import torch
    if torch.cuda.is_available():
        pytest.skip("calls with fake device addresses need a host without a GPU")
    lib = g.load()
    big = [FAKE, 1 << 40, 1 << 41, 1 << 42, 1 << 43]
    assert lib.gemm_bf16_nt(3, 16, (1 << 22) - 8, big[0], big[1], big[2], None) == g.ERR_NO_DEVICE
    assert lib.gemm_bf16_nt(3, 16, 1 << 22, big[0], big[1], big[2], None) == g.ERR_UNSUPPORTED
    assert lib.gemm_nvfp4_nt(3, 16, (1 << 24) - 64, *big, None) == g.ERR_NO_DEVICE
    assert lib.gemm_nvfp4_nt(3, 16, 1 << 24, *big, None) == g.ERR_UNSUPPORTED
    # K % 32 == 0 is accepted (here the call then stops at the missing device)
    for K in (32, 96, 8160):
        assert lib.gemm_nvfp4_nt(3, 16, K, *big, None) == g.ERR_NO_DEVICE, K
        assert lib.gemm_nvfp4_nt_bias_act(3, 16, K, *big[:4], None, 2, big[4], None) == g.ERR_NO_DEVICE, K
    assert lib.gemm_bf16_nt((1 << 27) - 300, 8, 8, big[0], big[1], big[2], None) == g.ERR_NO_DEVICE   # C, A
    assert lib.gemm_bf16_nt(1 << 27, 8, 8, big[0], big[1], big[2], None) == g.ERR_UNSUPPORTED


def test_fp4_specific_rejections():
    assert _fp4(8, 8, 64, sfa=None) == g.ERR_INVALID_ARG
    assert _fp4(8, 8, 48) == g.ERR_UNSUPPORTED                    # K % 32
    assert _fp4(8, 8, 16) == g.ERR_UNSUPPORTED
    assert _fp4(8, 8, 64, sfb=FAKE + 0x300002) == g.ERR_UNSUPPORTED  # scales need 4-byte alignment
    assert _fp4(8, 8, 64, aq=FAKE + 8) == g.ERR_UNSUPPORTED


def test_mx_specific_rejections():
    assert _mx(8, 8, 512, sa=None) == g.ERR_INVALID_ARG
    assert _mx(8, 8, 512, bq=None) == g.ERR_INVALID_ARG
    for K in (32, 256, 768):                                     # K % 512 (scales move 16 bytes per row)
        assert _mx(8, 8, K) == g.ERR_UNSUPPORTED
    assert _mx(8, 8, 512, sb=FAKE + 0x300004) == g.ERR_UNSUPPORTED   # scales need 16-byte alignment
    assert _mx(8, 8, 512, aq=FAKE + 8) == g.ERR_UNSUPPORTED
    assert _mx(8, 8, 512, aq=FAKE, c=FAKE + 512) == g.ERR_INVALID_ARG   # C overlaps the A codes
    import torch
    if torch.cuda.is_available():
        return
    lib = g.load()
    big = [FAKE, 1 << 40, 1 << 41, 1 << 42, 1 << 43]
    # codes of 256 padded rows: K / 2 bytes each, below 2^31 in all
    assert lib.gemm_mxfp4_nt(3, 16, (1 << 24) - 512, *big, None) == g.ERR_NO_DEVICE
    assert lib.gemm_mxfp4_nt(3, 16, 1 << 24, *big, None) == g.ERR_UNSUPPORTED
    assert _mx(8, 8, 0, None, None, None, None) == g.ERR_NO_DEVICE   # K = 0: zeros, no operand read


def test_binding_checks_tensor_sizes_before_calling():
    import torch
    with pytest.raises(ValueError):
        g.gemm_bf16_nt(4, 8, 8, torch.zeros(4, 8, dtype=torch.bfloat16), FAKE, FAKE)  # CPU tensor


def _golden_order():
    pairs = []
    for line in open(os.path.join(GOLDEN, "supergroup4_order.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            m, n = line.split()
            pairs.append((int(m), int(n)))
    return pairs


def test_tile_order_matches_the_pages_supergroup_example():
    tm, tn = g.tile_order(2, 8, 4)
    assert list(zip(tm, tn)) == _golden_order()


@pytest.mark.parametrize("tiles_m,tiles_n,sg", [(32, 32, 8), (32, 32, 4), (1, 32, 8), (5, 7, 3),
                                                 (32, 32, 1), (3, 2, 8), (31, 33, 8)])
def test_tile_order_is_a_bijection(tiles_m, tiles_n, sg):
    tm, tn = g.tile_order(tiles_m, tiles_n, sg)
    assert sorted(zip(tm, tn)) == [(m, n) for m in range(tiles_m) for n in range(tiles_n)]


@pytest.mark.parametrize("tiles,grid", [(1024, 256), (256, 256), (32, 32), (1, 1), (7, 7), (1000, 248), (12, 8)])
def test_schedule_covers_every_tile_once(tiles, grid):
    slots = g.schedule(tiles, grid)
    got = sorted(p for w in slots for p in w if p >= 0)
    assert got == list(range(tiles))


def test_schedule_keeps_an_xcds_tiles_compact():
    # 8192^3 with 256 x 256 tiles: 32 x 32 tiles on 256 workgroups. In each
    # round the 32 workgroups of one XCD (w % 8 equal) must cover a 4 x 8
    # block of tiles: 4 A row strips and 8 B row strips per L2.
    slots = g.schedule(1024, 256)
    tm, tn = g.tile_order(32, 32, 8)
    for r in range(4):
        for x in range(8):
            pos = [slots[w][r] for w in range(256) if w % 8 == x]
            ms = {tm[p] for p in pos}
            ns = {tn[p] for p in pos}
            assert len(ms) == 4 and len(ns) == 8, (r, x, ms, ns)


def test_force_instance_accepts_only_known_instances():
    lib = g.load()
    for bad in (-1, 4, 99):
        assert lib.gemm355_force_instance(bad) == g.ERR_INVALID_ARG
    for ok in (g.INSTANCE_LARGE, g.INSTANCE_SMALL, g.INSTANCE_SPLITK, g.INSTANCE_AUTO):
        assert lib.gemm355_force_instance(ok) == g.OK


def test_force_schedule_accepts_only_known_modes():
    lib = g.load()
    for bad in (-1, 2, 7):
        assert lib.gemm355_force_schedule(bad) == g.ERR_INVALID_ARG
    for ok in (g.SCHEDULE_DYNAMIC, g.SCHEDULE_STATIC):
        assert lib.gemm355_force_schedule(ok) == g.OK


def test_supergroup_rule():
    # 16 only for short K loops with many tiles across N, where the ablations
    # measured it faster; 8 everywhere else
    for k in (g.KERNEL_BF16, g.KERNEL_MXFP4):
        assert g.supergroup(64, 1024, k) == 16 and g.supergroup(128, 256, k) == 16
        assert g.supergroup(63, 1024, k) == 8 and g.supergroup(64, 1032, k) == 8
        assert g.supergroup(32, 8192, k) == 8 and g.supergroup(1, 0, k) == 8
    nv = g.KERNEL_NVFP4
    assert g.supergroup(32, 2048, nv) == 16 and g.supergroup(64, 512, nv) == 16
    assert g.supergroup(31, 1024, nv) == 8 and g.supergroup(32, 2080, nv) == 8 and g.supergroup(32, 8192, nv) == 8
    assert g.supergroup(4096, 64, g.KERNEL_BF16_SMALL) == 8
    lib = g.load()
    assert lib.gemm355_supergroup(0, 0, 8) == -g.ERR_INVALID_ARG
    assert lib.gemm355_supergroup(0, 8, -1) == -g.ERR_INVALID_ARG
    assert lib.gemm355_supergroup(4, 8, 8) == -g.ERR_INVALID_ARG
    assert lib.gemm355_supergroup(-1, 8, 8) == -g.ERR_INVALID_ARG


def test_force_supergroup_range():
    lib = g.load()
    for bad in (-1, 4097):
        assert lib.gemm355_force_supergroup(bad) == g.ERR_INVALID_ARG
    for ok in (1, 4, 4096, 0):
        assert lib.gemm355_force_supergroup(ok) == g.OK


def test_bf16_plan_for_the_workload_shapes():
    # 256 compute units: the square workloads take 256 x 256 tiles, the small
    # one 64 x 64 tiles; the skinny one (M = 128) has exactly one round of 256
    # tiles of 64 x 64, where that instance beats splitting K (measured).
    g.force_instance(g.INSTANCE_AUTO)
    g.force_supergroup(0)
    for ws in (False, True):
        assert g.bf16_plan(8192, 8192, 8192, 256, ws) == (g.INSTANCE_LARGE, 1)
        assert g.bf16_plan(8000, 8000, 8000, 256, ws) == (g.INSTANCE_LARGE, 1)
        assert g.bf16_plan(4096, 4096, 4096, 256, ws) == (g.INSTANCE_LARGE, 1)
        assert g.bf16_plan(256, 256, 256, 256, ws) == (g.INSTANCE_SMALL, 1)
        assert g.bf16_plan(128, 8192, 8192, 256, ws) == (g.INSTANCE_SMALL, 1)
        # short K: nothing to split
        assert g.bf16_plan(128, 8192, 2048, 256, ws) == (g.INSTANCE_SMALL, 1)
        # mid shapes with a quarter of the units' worth of 256 x 256 tiles: one
        # round of 128 x 128 tiles, stored directly (measured 27 us against 42 us
        # for 64 x 64 tiles and 46 us for 256 x 256 ones at 2048^3)
        assert g.bf16_plan(2048, 2048, 2048, 256, ws) == (g.INSTANCE_SPLITK, 1)
        assert g.bf16_plan(1024, 4096, 8192, 256, ws) == (g.INSTANCE_SPLITK, 1)
        assert g.bf16_plan(1024, 1024, 1024, 256, ws) == (g.INSTANCE_SMALL, 1)
        # half the units' worth of 256 x 256 tiles or more: that instance
        assert g.bf16_plan(1024, 8192, 1024, 256, ws) == (g.INSTANCE_LARGE, 1)
        assert g.bf16_plan(3072, 3072, 3072, 256, ws) == (g.INSTANCE_LARGE, 1)
        # K too short for the 256 x 256 instance's four kinds of step
        assert g.bf16_plan(4096, 4096, 192, 256, ws) == (g.INSTANCE_SMALL, 1)
        assert g.bf16_plan(4096, 4096, 200, 256, ws)[0] == g.INSTANCE_LARGE
    # fewer 64 x 64 tiles than compute units, or two rounds of them: split K,
    # when a workspace is given; without one, the 64 x 64 instance
    assert g.bf16_plan(64, 4096, 8192, 256, True) == (g.INSTANCE_SPLITK, 8)
    assert g.bf16_plan(512, 4096, 8192, 256, True) == (g.INSTANCE_SPLITK, 2)
    assert g.bf16_plan(1024, 1024, 16384, 256, True) == (g.INSTANCE_SPLITK, 4)
    for shape in [(64, 4096, 8192), (512, 4096, 8192), (1024, 1024, 16384)]:
        assert g.bf16_plan(*shape, 256) == (g.INSTANCE_SMALL, 1)
    # splitting never makes a split shorter than 8 steps of 64, or empty
    for M, N, K in [(128, 1032, 4104), (64, 64, 4104), (512, 4096, 8192), (128, 2048, 520), (2048, 2048, 2048)]:
        inst, splits = g.bf16_plan(M, N, K, 256, True)
        if inst == g.INSTANCE_SPLITK and splits > 1:
            steps = -(-K // 64)
            per = -(-steps // splits)
            assert splits <= 8 and per >= 8 and (splits - 1) * per < steps, (M, N, K, splits)


def test_bf16_plan_workspace_bytes():
    # 64 KiB of FP32 partials per 128 x 128 tile and split; none without a split
    g.force_instance(g.INSTANCE_AUTO)
    assert g.bf16_plan_workspace_bytes(8192, 8192, 8192, 256) == 0
    assert g.bf16_plan_workspace_bytes(128, 8192, 8192, 256) == 0
    assert g.bf16_plan_workspace_bytes(64, 4096, 8192, 256) == 32 * 8 * 65536
    assert g.bf16_plan_workspace_bytes(136, 1032, 4104, 256) == 2 * 9 * 8 * 65536
    # splits are chosen so that work items do not outnumber the units: the
    # workspace never exceeds 64 KiB per compute unit, even when forced
    rng = np.random.Generator(np.random.PCG64(5))
    try:
        for forced in (g.INSTANCE_AUTO, g.INSTANCE_SPLITK):
            g.force_instance(forced)
            for _ in range(300):
                M, N = (int(x) for x in rng.integers(1, 4096, 2))
                K = int(rng.integers(0, 32768))
                cus = int(rng.choice([80, 104, 256, 304]))
                inst, splits = g.bf16_plan(M, N, K, cus, True)
                nb = g.bf16_plan_workspace_bytes(M, N, K, cus)
                tiles = -(-M // 128) * -(-N // 128)
                assert nb == (tiles * splits * 65536 if splits > 1 else 0), (M, N, K, cus)
                assert nb <= cus * 65536, (M, N, K, cus)
                assert g.bf16_plan(M, N, K, cus)[1] == 1
    finally:
        g.force_instance(g.INSTANCE_AUTO)


def _ws(M, N, K, w, nbytes, a=FAKE, b=FAKE + 0x100000, c=FAKE + 0x200000):
    return g.load().gemm_bf16_nt_ws(M, N, K, a, b, c, w, nbytes, None)


def test_workspace_rejections_happen_before_any_device_call():
    lib = g.load()
    assert _ws(-1, 8, 64, None, 0) == g.ERR_INVALID_ARG
    assert _ws(0, 8, 64, None, 0) == g.OK                             # empty: nothing to do
    assert _ws(8, 8, 64, None, 4096) == g.ERR_INVALID_ARG             # NULL with bytes
    assert _ws(8, 8, 64, FAKE + 0x300008, 4096) == g.ERR_UNSUPPORTED  # not 16-byte aligned
    assert _ws(8, 8, 64, FAKE + 0x200000, 4096) == g.ERR_INVALID_ARG  # overlaps C
    assert _ws(8, 8, 64, FAKE, 4096) == g.ERR_INVALID_ARG             # overlaps A
    assert _ws(8, 8, 64, FAKE + 0x100010, 4096) == g.ERR_INVALID_ARG  # overlaps B
    assert lib.gemm_bf16_nt_bias_act_ws(8, 8, 64, FAKE, FAKE + 0x100000, FAKE + 0x300000, 2, FAKE + 0x200000,
                                        FAKE + 0x300000, 4096, None) == g.ERR_INVALID_ARG   # overlaps the bias
    assert lib.gemm_bf16_nt_bias_act_ws(8, 8, 64, FAKE, FAKE + 0x100000, None, 7, FAKE + 0x200000,
                                        None, 0, None) == g.ERR_INVALID_ARG                 # unknown activation
    out = ctypes.c_size_t(99)
    assert lib.gemm_bf16_nt_workspace_size(-1, 8, 8, ctypes.byref(out)) == g.ERR_INVALID_ARG
    assert lib.gemm_bf16_nt_workspace_size(8, 8, 8, None) == g.ERR_INVALID_ARG
    assert lib.gemm_bf16_nt_workspace_size(0, 8, 8, ctypes.byref(out)) == g.OK and out.value == 0


def test_noalloc_rejections_happen_before_any_device_call():
    lib = g.load()
    f = lambda M, N, K, a=FAKE, b=FAKE + 0x100000, c=FAKE + 0x200000: lib.gemm_bf16_nt_noalloc(M, N, K, a, b, c, None)
    assert f(-1, 8, 64) == g.ERR_INVALID_ARG
    assert f(0, 8, 64, None, None, None) == g.OK
    assert f(8, 8, 64, c=None) == g.ERR_INVALID_ARG
    assert f(8, 8, 64, a=None) == g.ERR_INVALID_ARG
    assert f(8, 8, 12) == g.ERR_UNSUPPORTED                      # K % 8
    assert f(8, 8, 64, c=FAKE + 0x900008) == g.ERR_UNSUPPORTED   # C not 16-byte aligned
    assert f(8, 8, 64, c=FAKE + 0x100010) == g.ERR_INVALID_ARG   # C overlaps B


def test_no_allocation_reachable_from_the_library():
    # the library allocates nothing: no allocation call appears in its host source
    src = open(os.path.join(os.path.dirname(g.__file__), "csrc", "gemm355.hip")).read()
    for call in ("hipMalloc", "hipFree", "hipMemPool", "hipHostMalloc", "hipExtMalloc", "malloc(", "new "):
        assert call not in src, call


def test_bf16_plan_follows_the_forced_instance_and_checks_arguments():
    lib = g.load()
    try:
        g.force_instance(g.INSTANCE_SMALL)
        assert g.bf16_plan(8192, 8192, 8192, 256) == (g.INSTANCE_SMALL, 1)
        g.force_instance(g.INSTANCE_SPLITK)
        inst, splits = g.bf16_plan(8192, 8192, 8192, 256, True)
        assert inst == g.INSTANCE_SPLITK and splits >= 1
        assert g.bf16_plan(128, 1032, 4104, 256) == (g.INSTANCE_SPLITK, 1)
        g.force_instance(g.INSTANCE_LARGE)
        assert g.bf16_plan(8192, 8192, 128, 256) == (g.INSTANCE_SMALL, 1)
    finally:
        g.force_instance(g.INSTANCE_AUTO)
    out = (ctypes.c_int * 2)()
    nb = ctypes.c_size_t(0)
    for bad in [(0, 8, 8, 256), (8, -1, 8, 256), (8, 8, -8, 256), (8, 8, 8, 0)]:
        assert lib.gemm355_bf16_plan(*bad, 1, ctypes.byref(out, 0), ctypes.byref(out, 4),
                                     ctypes.byref(nb)) == g.ERR_INVALID_ARG
    assert lib.gemm355_bf16_plan(8, 8, 8, 256, 0, None, ctypes.byref(out, 4), ctypes.byref(nb)) == g.ERR_INVALID_ARG
    assert lib.gemm355_bf16_plan(8, 8, 8, 256, 0, ctypes.byref(out, 0), ctypes.byref(out, 4),
                                 None) == g.ERR_INVALID_ARG


def test_nvfp4_ws_plan_and_rejections_before_any_device_call():
    lib = g.load()
    # the shape rule: decode first from two rounds of 256 x 256 tiles on, once
    # the rounds times 7000 exceed M + N (the sides of the measured balance)
    assert g.nvfp4_plan(8192, 8192, 8192, 256) == (True, 4 * 8192 * 8192)   # 4 rounds, 16384
    assert g.nvfp4_plan(8192, 8192, 8192, 304) == (True, 4 * 8192 * 8192)   # ceil(1024 / 304) = 4
    assert g.nvfp4_plan(8192, 8192, 8192, 512) == (False, 0)                # 2 rounds, 14000 < 16384
    assert g.nvfp4_plan(4096, 4096, 8192, 256) == (False, 0)                # 1 round
    assert g.nvfp4_plan(3072, 3072, 8192, 256) == (False, 0)                # 1 round, 144 tiles
    assert g.nvfp4_plan(8192, 8192, 0, 256) == (False, 0)                   # K = 0: nothing to decode
    assert g.nvfp4_plan(6144, 6144, 6144, 256)[0]                            # 3 rounds, 12288
    assert g.nvfp4_plan(7168, 7168, 64, 256)[0]                              # 784 tiles: 4 rounds
    assert g.nvfp4_plan(5120, 5120, 5120, 256)[0]                            # 2 rounds, 10240
    assert g.nvfp4_plan(4096, 8192, 8192, 256)[0]                            # 2 rounds, 12288
    assert g.nvfp4_plan(4096, 16384, 1024, 256)[0]                           # 4 rounds, 20480
    assert not g.nvfp4_plan(2048, 16384, 8192, 256)[0]                       # 2 rounds, 18432
    assert g.nvfp4_plan(12288, 12288, 4096, 256)[0]                          # 9 rounds, 24576
    # workspace: 2 M K rounded up to 256 bytes, then 2 N K
    try:
        g.force_fp4_path(g.FP4_PATH_DECODE_FIRST)
        assert g.nvfp4_plan(3, 8, 32, 256) == (True, 256 + 2 * 8 * 32)
        assert g.nvfp4_plan(8, 3, 64, 256) == (True, 1024 + 2 * 3 * 64)
        g.force_fp4_path(g.FP4_PATH_STAGING)
        assert g.nvfp4_plan(8192, 8192, 8192, 256) == (False, 0)
    finally:
        g.force_fp4_path(g.FP4_PATH_AUTO)
    assert lib.gemm355_force_fp4_path(3) == g.ERR_INVALID_ARG
    d, nb = ctypes.c_int(0), ctypes.c_size_t(0)
    assert lib.gemm355_nvfp4_plan(0, 8, 8, 256, ctypes.byref(d), ctypes.byref(nb)) == g.ERR_INVALID_ARG
    assert lib.gemm355_nvfp4_plan(8, 8, 8, 0, ctypes.byref(d), ctypes.byref(nb)) == g.ERR_INVALID_ARG
    out = ctypes.c_size_t(99)
    assert lib.gemm_nvfp4_nt_workspace_size(-1, 8, 64, ctypes.byref(out)) == g.ERR_INVALID_ARG
    assert lib.gemm_nvfp4_nt_workspace_size(8, 8, 64, None) == g.ERR_INVALID_ARG
    assert lib.gemm_nvfp4_nt_workspace_size(0, 8, 64, ctypes.byref(out)) == g.OK and out.value == 0
    assert lib.gemm_nvfp4_nt_workspace_size(8, 8, 0, ctypes.byref(out)) == g.OK and out.value == 0

    def ws(M, N, K, w, nb, aq=FAKE, sfa=FAKE + 0x100000, bq=FAKE + 0x200000, sfb=FAKE + 0x300000, c=FAKE + 0x400000):
        return lib.gemm_nvfp4_nt_ws(M, N, K, aq, sfa, bq, sfb, c, w, nb, None)
    assert ws(-1, 8, 64, None, 0) == g.ERR_INVALID_ARG
    assert ws(0, 8, 64, None, 0) == g.OK                                # empty: nothing to do
    assert ws(8, 8, 48, FAKE + 0x500000, 4096) == g.ERR_UNSUPPORTED      # K % 32, as gemm_nvfp4_nt
    assert ws(8, 8, 64, None, 4096) == g.ERR_INVALID_ARG                 # NULL with bytes
    assert ws(8, 8, 64, FAKE + 0x500008, 4096) == g.ERR_UNSUPPORTED      # not 16-byte aligned
    assert ws(8, 8, 64, FAKE + 0x400000, 4096) == g.ERR_INVALID_ARG      # overlaps C
    assert ws(8, 8, 64, FAKE, 4096) == g.ERR_INVALID_ARG                 # overlaps Aq
    assert ws(8, 8, 64, FAKE + 0x300000, 4096) == g.ERR_INVALID_ARG      # overlaps SFB
    assert ws(8, 8, 64, FAKE + 0x500000, 4096) == g.ERR_NO_DEVICE        # valid: reaches the device query

    # the fused form: the same checks, plus the epilogue's
    def wsf(M, N, K, w, nb, bias=FAKE + 0x600000, act=g.ACT_GELU_TANH):
        return lib.gemm_nvfp4_nt_bias_act_ws(M, N, K, FAKE, FAKE + 0x100000, FAKE + 0x200000, FAKE + 0x300000,
                                             bias, act, FAKE + 0x400000, w, nb, None)
    assert wsf(0, 8, 64, None, 0) == g.OK                               # empty: nothing to do
    assert wsf(8, 8, 64, FAKE + 0x500000, 4096, act=7) == g.ERR_INVALID_ARG    # unknown activation
    assert wsf(8, 8, 64, FAKE + 0x500000, 4096, bias=FAKE + 0x600008) == g.ERR_UNSUPPORTED   # bias alignment
    assert wsf(8, 8, 64, FAKE + 0x500000, 4096, bias=FAKE + 0x400000) == g.ERR_INVALID_ARG   # bias inside C
    assert wsf(8, 8, 64, FAKE + 0x5FFF00, 4096) == g.ERR_INVALID_ARG    # workspace overlaps the bias
    assert wsf(8, 8, 64, FAKE + 0x500000, 4096) == g.ERR_NO_DEVICE      # valid: reaches the device query
    assert wsf(8, 8, 64, FAKE + 0x500000, 4096, bias=None) == g.ERR_NO_DEVICE   # no bias: zeros
