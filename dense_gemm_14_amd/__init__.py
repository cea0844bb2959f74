"""Python binding of libgemm355 (gfx950 HIP kernels behind a C ABI).

Argument marshalling only: every step of the product runs in the HIP kernels
of ``libgemm355.so``. There is no CPU path and no fallback -- if the library
cannot be loaded, every call raises.

The functions mirror the C entry points declared in ``include/gemm355.h``:

    gemm_bf16_nt(M, N, K, A, B, C, stream=None)
    gemm_bf16_nt_bias_act(M, N, K, A, B, bias, activation, C, stream=None)
    gemm_bf16_nt_ws(M, N, K, A, B, C, workspace, workspace_bytes=None, stream=None)
    gemm_bf16_nt_bias_act_ws(M, N, K, A, B, bias, activation, C, workspace, workspace_bytes=None, stream=None)
    workspace_size(M, N, K)           # bytes the *_ws calls need on the current device
    gemm_bf16_nt_noalloc(M, N, K, A, B, C, stream=None)   # *_ws plan, library's fixed scratch
    gemm_nvfp4_nt(M, N, K, Aq, SFA, Bq, SFB, C, stream=None)
    gemm_nvfp4_nt_bias_act(M, N, K, Aq, SFA, Bq, SFB, bias, activation, C, stream=None)
    gemm_nvfp4_nt_ws(M, N, K, Aq, SFA, Bq, SFB, C, workspace, workspace_bytes=None, stream=None)
    gemm_nvfp4_nt_bias_act_ws(M, N, K, Aq, SFA, Bq, SFB, bias, activation, C, workspace,
                              workspace_bytes=None, stream=None)
    nvfp4_workspace_size(M, N, K)     # bytes the NVFP4 *_ws calls need on the current device
    nvfp4_plan(M, N, K, compute_units)  # (decode_first, workspace_bytes) of those calls
    force_fp4_path(path)              # their path for the process (diagnostic)
    gemm_mxfp4_nt(M, N, K, Aq, SA, Bq, SB, C, stream=None)
    gemm_mxfp4_nt_bias_act(M, N, K, Aq, SA, Bq, SB, bias, activation, C, stream=None)
    force_instance(instance)          # BF16 instance override (diagnostic)
    force_supergroup(width)           # band width of the tile order (diagnostic)
    supergroup(tiles_n, K, kernel)    # the default band width of a kernel's visiting order
    force_schedule(mode)              # static or dynamic tile order of the NVFP4 kernel (diagnostic)
    bf16_plan(M, N, K, compute_units, with_workspace=False)  # (instance, splits) a BF16 call would run
    bf16_plan_workspace_bytes(M, N, K, compute_units)  # workspace bytes of the *_ws plan

Operands may be torch tensors on a ROCm device (their storage is checked
against the sizes before the call, since the C side cannot see it) or raw
device addresses as ints (unchecked). ``stream`` is a ``torch.cuda.Stream``,
a raw hipStream_t as int, or None for torch's current stream.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_PATH = os.path.join(HERE, "libgemm355.so")
HEADER = os.path.join(ROOT, "include", "gemm355.h")

OK = 0
ERR_INVALID_ARG = 1
ERR_UNSUPPORTED = 2
ERR_NO_DEVICE = 3
ERR_LAUNCH = 4

ACT_NONE = 0         # fused epilogue activations (gemm_bf16_nt_bias_act)
ACT_RELU = 1
ACT_GELU_TANH = 2

INSTANCE_AUTO = 0    # gemm_bf16_nt picks the instance by shape
INSTANCE_LARGE = 1   # 256 x 256 output tiles
INSTANCE_SMALL = 2   # 64 x 64 output tiles
KERNEL_BF16 = 0     # kernels of the supergroup rule (gemm355_supergroup)
KERNEL_NVFP4 = 1
KERNEL_MXFP4 = 2
KERNEL_BF16_SMALL = 3
FP4_PATH_AUTO = 0    # gemm_nvfp4_nt_ws: decode first by shape (gemm355_force_fp4_path)
FP4_PATH_STAGING = 1  # always the kernel that decodes while staging
FP4_PATH_DECODE_FIRST = 2  # always decode into the workspace, then the BF16 product
SCHEDULE_STATIC = 0  # the NVFP4 kernel's tile order (gemm355_force_schedule)
SCHEDULE_DYNAMIC = 1
INSTANCE_SPLITK = 3  # 128 x 128 output tiles; with a workspace (the *_ws calls) K split over workgroups

_lib = None


class Gemm355Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (what, status_string(status), status))


def load() -> ctypes.CDLL:
    """Load libgemm355.so, building it first if (and only if) none is built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _build
        _build.build()
    try:
        lib = ctypes.CDLL(LIB_PATH)
    except OSError as e:  # no silent fallback: the HIP library is the product
        raise RuntimeError("libgemm355.so could not be loaded from %s: %s" % (LIB_PATH, e)) from e
    p, i = ctypes.c_void_p, ctypes.c_int
    lib.gemm_bf16_nt.argtypes = [i, i, i, p, p, p, p]
    lib.gemm_bf16_nt.restype = i
    lib.gemm_bf16_nt_bias_act.argtypes = [i, i, i, p, p, p, i, p, p]
    lib.gemm_bf16_nt_bias_act.restype = i
    sz = ctypes.c_size_t
    lib.gemm_bf16_nt_ws.argtypes = [i, i, i, p, p, p, p, sz, p]
    lib.gemm_bf16_nt_ws.restype = i
    lib.gemm_bf16_nt_bias_act_ws.argtypes = [i, i, i, p, p, p, i, p, p, sz, p]
    lib.gemm_bf16_nt_bias_act_ws.restype = i
    lib.gemm_bf16_nt_noalloc.argtypes = [i, i, i, p, p, p, p]
    lib.gemm_bf16_nt_noalloc.restype = i
    lib.gemm_bf16_nt_workspace_size.argtypes = [i, i, i, ctypes.POINTER(sz)]
    lib.gemm_bf16_nt_workspace_size.restype = i
    lib.gemm_nvfp4_nt.argtypes = [i, i, i, p, p, p, p, p, p]
    lib.gemm_nvfp4_nt.restype = i
    lib.gemm_nvfp4_nt_bias_act.argtypes = [i, i, i, p, p, p, p, p, i, p, p]
    lib.gemm_nvfp4_nt_bias_act.restype = i
    lib.gemm_nvfp4_nt_ws.argtypes = [i, i, i, p, p, p, p, p, p, sz, p]
    lib.gemm_nvfp4_nt_ws.restype = i
    lib.gemm_nvfp4_nt_bias_act_ws.argtypes = [i, i, i, p, p, p, p, p, i, p, p, sz, p]
    lib.gemm_nvfp4_nt_bias_act_ws.restype = i
    lib.gemm_nvfp4_nt_workspace_size.argtypes = [i, i, i, ctypes.POINTER(sz)]
    lib.gemm_nvfp4_nt_workspace_size.restype = i
    lib.gemm355_nvfp4_plan.argtypes = [i, i, i, i, p, p]
    lib.gemm355_nvfp4_plan.restype = i
    lib.gemm355_force_fp4_path.argtypes = [i]
    lib.gemm355_force_fp4_path.restype = i
    lib.gemm_mxfp4_nt.argtypes = [i, i, i, p, p, p, p, p, p]
    lib.gemm_mxfp4_nt.restype = i
    lib.gemm_mxfp4_nt_bias_act.argtypes = [i, i, i, p, p, p, p, p, i, p, p]
    lib.gemm_mxfp4_nt_bias_act.restype = i
    lib.gemm355_status_string.argtypes = [i]
    lib.gemm355_status_string.restype = ctypes.c_char_p
    lib.gemm355_tile_order.argtypes = [i, i, i, p, p]
    lib.gemm355_tile_order.restype = i
    lib.gemm355_schedule.argtypes = [i, i, p, i]
    lib.gemm355_schedule.restype = i
    lib.gemm355_force_instance.argtypes = [i]
    lib.gemm355_force_instance.restype = i
    lib.gemm355_force_schedule.argtypes = [i]
    lib.gemm355_force_schedule.restype = i
    lib.gemm355_supergroup.argtypes = [i, i, i]
    lib.gemm355_supergroup.restype = i
    lib.gemm355_force_supergroup.argtypes = [i]
    lib.gemm355_force_supergroup.restype = i
    lib.gemm355_bf16_plan.argtypes = [i, i, i, i, i, p, p, p]
    lib.gemm355_bf16_plan.restype = i
    _lib = lib
    return lib


def declared_functions() -> list:
    """Names of the functions declared in include/gemm355.h."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)


def status_string(status: int) -> str:
    return load().gemm355_status_string(int(status)).decode()


# ---- marshalling -----------------------------------------------------------

def _addr(x, need_bytes: int, what: str):
    """Device address of a tensor (checked) or a raw int address (unchecked)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    import torch
    if not isinstance(x, torch.Tensor):
        raise TypeError("%s: expected a torch tensor or an int address, got %r" % (what, type(x)))
    if x.device.type != "cuda":
        raise ValueError("%s must be on the GPU, got device %s" % (what, x.device))
    if not x.is_contiguous():
        raise ValueError("%s must be contiguous" % what)
    have = x.numel() * x.element_size()
    if have < need_bytes:
        raise ValueError("%s holds %d bytes, the sizes need %d" % (what, have, need_bytes))
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, what: str):
    if status != OK:
        raise Gemm355Error(status, what)


# ---- entry points ------------------------------------------------------------

def gemm_bf16_nt(M: int, N: int, K: int, A, B, C, stream=None) -> None:
    """C (M x N, BF16) = A (M x K, BF16) @ B (N x K, BF16)^T, FP32 sums."""
    lib = load()
    M, N, K = int(M), int(N), int(K)
    nz = M > 0 and N > 0
    a = _addr(A, M * K * 2 if nz else 0, "A")
    b = _addr(B, N * K * 2 if nz else 0, "B")
    c = _addr(C, M * N * 2 if nz else 0, "C")
    _check(lib.gemm_bf16_nt(M, N, K, a, b, c, _stream(stream)), "gemm_bf16_nt")


def gemm_bf16_nt_bias_act(M: int, N: int, K: int, A, B, bias, activation: int, C, stream=None) -> None:
    """C = act(A @ B^T + bias), bias (N BF16 values, or None) and activation
    (ACT_NONE, ACT_RELU, ACT_GELU_TANH) applied in the kernels' epilogue."""
    lib = load()
    M, N, K = int(M), int(N), int(K)
    nz = M > 0 and N > 0
    a = _addr(A, M * K * 2 if nz else 0, "A")
    b = _addr(B, N * K * 2 if nz else 0, "B")
    bb = _addr(bias, N * 2 if nz else 0, "bias")
    c = _addr(C, M * N * 2 if nz else 0, "C")
    _check(lib.gemm_bf16_nt_bias_act(M, N, K, a, b, bb, int(activation), c, _stream(stream)),
           "gemm_bf16_nt_bias_act")


def _workspace(ws, nbytes):
    """(address, bytes) of a workspace tensor, int address or None."""
    if ws is None:
        return None, 0 if nbytes is None else int(nbytes)
    if isinstance(ws, int):
        if nbytes is None:
            raise ValueError("workspace_bytes is needed with a raw workspace address")
        return ws, int(nbytes)
    have = ws.numel() * ws.element_size()
    nb = have if nbytes is None else int(nbytes)
    if nb > have:
        raise ValueError("workspace holds %d bytes, workspace_bytes says %d" % (have, nb))
    return _addr(ws, nb, "workspace"), nb


def gemm_bf16_nt_ws(M: int, N: int, K: int, A, B, C, workspace, workspace_bytes=None, stream=None) -> None:
    """gemm_bf16_nt with a caller-owned workspace (a device tensor of at least
    workspace_size(M, N, K) bytes, or None when that is 0), which lets the
    128 x 128 instance split K."""
    lib = load()
    M, N, K = int(M), int(N), int(K)
    nz = M > 0 and N > 0
    a = _addr(A, M * K * 2 if nz else 0, "A")
    b = _addr(B, N * K * 2 if nz else 0, "B")
    c = _addr(C, M * N * 2 if nz else 0, "C")
    w, nb = _workspace(workspace, workspace_bytes)
    _check(lib.gemm_bf16_nt_ws(M, N, K, a, b, c, w, nb, _stream(stream)), "gemm_bf16_nt_ws")


def gemm_bf16_nt_bias_act_ws(M: int, N: int, K: int, A, B, bias, activation: int, C, workspace,
                             workspace_bytes=None, stream=None) -> None:
    """gemm_bf16_nt_bias_act with a caller-owned workspace (see gemm_bf16_nt_ws)."""
    lib = load()
    M, N, K = int(M), int(N), int(K)
    nz = M > 0 and N > 0
    a = _addr(A, M * K * 2 if nz else 0, "A")
    b = _addr(B, N * K * 2 if nz else 0, "B")
    bb = _addr(bias, N * 2 if nz else 0, "bias")
    c = _addr(C, M * N * 2 if nz else 0, "C")
    w, nb = _workspace(workspace, workspace_bytes)
    _check(lib.gemm_bf16_nt_bias_act_ws(M, N, K, a, b, bb, int(activation), c, w, nb, _stream(stream)),
           "gemm_bf16_nt_bias_act_ws")


def gemm_bf16_nt_noalloc(M: int, N: int, K: int, A, B, C, stream=None) -> None:
    """gemm_bf16_nt_ws's product with the library's fixed scratch array as
    the workspace: allocates nothing (for graph capture and the like); calls
    overlapping on one GPU race on the scratch."""
    lib = load()
    M, N, K = int(M), int(N), int(K)
    nz = M > 0 and N > 0
    a = _addr(A, M * K * 2 if nz else 0, "A")
    b = _addr(B, N * K * 2 if nz else 0, "B")
    c = _addr(C, M * N * 2 if nz else 0, "C")
    _check(lib.gemm_bf16_nt_noalloc(M, N, K, a, b, c, _stream(stream)), "gemm_bf16_nt_noalloc")


def workspace_size(M: int, N: int, K: int) -> int:
    """Bytes of workspace gemm_bf16_nt_ws / gemm_bf16_nt_bias_act_ws need for
    this shape on the current device (0: no split, no workspace)."""
    out = ctypes.c_size_t(0)
    _check(load().gemm_bf16_nt_workspace_size(int(M), int(N), int(K), ctypes.byref(out)),
           "gemm_bf16_nt_workspace_size")
    return out.value


def gemm_nvfp4_nt(M: int, N: int, K: int, Aq, SFA, Bq, SFB, C, stream=None) -> None:
    """C (M x N, BF16) = dec(Aq, SFA) @ dec(Bq, SFB)^T for E2M1 codes + E4M3 scales."""
    lib = load()
    M, N, K = int(M), int(N), int(K)
    nz = M > 0 and N > 0
    aq = _addr(Aq, M * K // 2 if nz else 0, "Aq")
    sfa = _addr(SFA, M * K // 16 if nz else 0, "SFA")
    bq = _addr(Bq, N * K // 2 if nz else 0, "Bq")
    sfb = _addr(SFB, N * K // 16 if nz else 0, "SFB")
    c = _addr(C, M * N * 2 if nz else 0, "C")
    _check(lib.gemm_nvfp4_nt(M, N, K, aq, sfa, bq, sfb, c, _stream(stream)), "gemm_nvfp4_nt")


def gemm_nvfp4_nt_ws(M: int, N: int, K: int, Aq, SFA, Bq, SFB, C, workspace, workspace_bytes=None,
                     stream=None) -> None:
    """gemm_nvfp4_nt with a caller-owned workspace (a device tensor of at least
    nvfp4_workspace_size(M, N, K) bytes, or None when that is 0): large
    products decode each operand once into BF16 there and run the BF16 core."""
    lib = load()
    M, N, K = int(M), int(N), int(K)
    nz = M > 0 and N > 0
    aq = _addr(Aq, M * K // 2 if nz else 0, "Aq")
    sfa = _addr(SFA, M * K // 16 if nz else 0, "SFA")
    bq = _addr(Bq, N * K // 2 if nz else 0, "Bq")
    sfb = _addr(SFB, N * K // 16 if nz else 0, "SFB")
    c = _addr(C, M * N * 2 if nz else 0, "C")
    w, nb = _workspace(workspace, workspace_bytes)
    _check(lib.gemm_nvfp4_nt_ws(M, N, K, aq, sfa, bq, sfb, c, w, nb, _stream(stream)), "gemm_nvfp4_nt_ws")


def nvfp4_workspace_size(M: int, N: int, K: int) -> int:
    """Workspace bytes gemm_nvfp4_nt_ws uses for this shape on the current device."""
    out = ctypes.c_size_t(0)
    _check(load().gemm_nvfp4_nt_workspace_size(int(M), int(N), int(K), ctypes.byref(out)),
           "gemm_nvfp4_nt_workspace_size")
    return out.value


def nvfp4_plan(M: int, N: int, K: int, compute_units: int):
    """(decode_first, workspace_bytes) of gemm_nvfp4_nt_ws on a device with
    `compute_units` compute units; host only."""
    d = ctypes.c_int(0)
    nb = ctypes.c_size_t(0)
    _check(load().gemm355_nvfp4_plan(int(M), int(N), int(K), int(compute_units), ctypes.byref(d), ctypes.byref(nb)),
           "gemm355_nvfp4_plan")
    return bool(d.value), nb.value


def force_fp4_path(path: int) -> None:
    """gemm_nvfp4_nt_ws's path for the whole process: FP4_PATH_AUTO (default),
    FP4_PATH_STAGING or FP4_PATH_DECODE_FIRST (a diagnostic)."""
    _check(load().gemm355_force_fp4_path(int(path)), "gemm355_force_fp4_path")


def gemm_nvfp4_nt_bias_act(M: int, N: int, K: int, Aq, SFA, Bq, SFB, bias, activation: int, C,
                           stream=None) -> None:
    """C = act(dec(Aq, SFA) @ dec(Bq, SFB)^T + bias) with the fused epilogue."""
    lib = load()
    M, N, K = int(M), int(N), int(K)
    nz = M > 0 and N > 0
    aq = _addr(Aq, M * K // 2 if nz else 0, "Aq")
    sfa = _addr(SFA, M * K // 16 if nz else 0, "SFA")
    bq = _addr(Bq, N * K // 2 if nz else 0, "Bq")
    sfb = _addr(SFB, N * K // 16 if nz else 0, "SFB")
    bb = _addr(bias, N * 2 if nz else 0, "bias")
    c = _addr(C, M * N * 2 if nz else 0, "C")
    _check(lib.gemm_nvfp4_nt_bias_act(M, N, K, aq, sfa, bq, sfb, bb, int(activation), c, _stream(stream)),
           "gemm_nvfp4_nt_bias_act")


def gemm_nvfp4_nt_bias_act_ws(M: int, N: int, K: int, Aq, SFA, Bq, SFB, bias, activation: int, C, workspace,
                              workspace_bytes=None, stream=None) -> None:
    """gemm_nvfp4_nt_bias_act with a caller-owned workspace, sized and used as
    for gemm_nvfp4_nt_ws."""
    lib = load()
    M, N, K = int(M), int(N), int(K)
    nz = M > 0 and N > 0
    aq = _addr(Aq, M * K // 2 if nz else 0, "Aq")
    sfa = _addr(SFA, M * K // 16 if nz else 0, "SFA")
    bq = _addr(Bq, N * K // 2 if nz else 0, "Bq")
    sfb = _addr(SFB, N * K // 16 if nz else 0, "SFB")
    bb = _addr(bias, N * 2 if nz else 0, "bias")
    c = _addr(C, M * N * 2 if nz else 0, "C")
    w, nb = _workspace(workspace, workspace_bytes)
    _check(lib.gemm_nvfp4_nt_bias_act_ws(M, N, K, aq, sfa, bq, sfb, bb, int(activation), c, w, nb, _stream(stream)),
           "gemm_nvfp4_nt_bias_act_ws")


def gemm_mxfp4_nt(M: int, N: int, K: int, Aq, SA, Bq, SB, C, stream=None) -> None:
    """C (M x N, BF16) = dec(Aq, SA) @ dec(Bq, SB)^T for E2M1 codes with one
    E8M0 scale per 32 elements (microscaled FP4)."""
    lib = load()
    M, N, K = int(M), int(N), int(K)
    nz = M > 0 and N > 0
    aq = _addr(Aq, M * K // 2 if nz else 0, "Aq")
    sa = _addr(SA, M * K // 32 if nz else 0, "SA")
    bq = _addr(Bq, N * K // 2 if nz else 0, "Bq")
    sb = _addr(SB, N * K // 32 if nz else 0, "SB")
    c = _addr(C, M * N * 2 if nz else 0, "C")
    _check(lib.gemm_mxfp4_nt(M, N, K, aq, sa, bq, sb, c, _stream(stream)), "gemm_mxfp4_nt")


def gemm_mxfp4_nt_bias_act(M: int, N: int, K: int, Aq, SA, Bq, SB, bias, activation: int, C, stream=None) -> None:
    """C = act(dec(Aq, SA) @ dec(Bq, SB)^T + bias), microscaled FP4 with the
    fused epilogue."""
    lib = load()
    M, N, K = int(M), int(N), int(K)
    nz = M > 0 and N > 0
    aq = _addr(Aq, M * K // 2 if nz else 0, "Aq")
    sa = _addr(SA, M * K // 32 if nz else 0, "SA")
    bq = _addr(Bq, N * K // 2 if nz else 0, "Bq")
    sb = _addr(SB, N * K // 32 if nz else 0, "SB")
    bb = _addr(bias, N * 2 if nz else 0, "bias")
    c = _addr(C, M * N * 2 if nz else 0, "C")
    _check(lib.gemm_mxfp4_nt_bias_act(M, N, K, aq, sa, bq, sb, bb, int(activation), c, _stream(stream)),
           "gemm_mxfp4_nt_bias_act")


def force_instance(instance: int) -> None:
    """Force gemm_bf16_nt's kernel instance for the whole process
    (INSTANCE_AUTO, INSTANCE_LARGE, INSTANCE_SMALL or INSTANCE_SPLITK)."""
    _check(load().gemm355_force_instance(instance), "gemm355_force_instance")


def force_supergroup(width: int) -> None:
    """Force the band width of the persistent kernels' supergroup tile order
    for the whole process (0 = the default)."""
    _check(load().gemm355_force_supergroup(width), "gemm355_force_supergroup")


def _plan(M, N, K, compute_units, with_workspace):
    inst = ctypes.c_int(0)
    splits = ctypes.c_int(0)
    nbytes = ctypes.c_size_t(0)
    _check(load().gemm355_bf16_plan(M, N, K, compute_units, int(bool(with_workspace)), ctypes.byref(inst),
                                    ctypes.byref(splits), ctypes.byref(nbytes)), "gemm355_bf16_plan")
    return inst.value, splits.value, nbytes.value


def force_schedule(mode: int) -> None:
    """Tile order of the NVFP4 kernel for the whole process: SCHEDULE_STATIC
    (default) or SCHEDULE_DYNAMIC (a measurement option)."""
    _check(load().gemm355_force_schedule(mode), "gemm355_force_schedule")


def supergroup(tiles_n: int, K: int, kernel: int = 0) -> int:
    """Default band width of the visiting order (kernel: KERNEL_BF16,
    KERNEL_NVFP4, KERNEL_MXFP4 or KERNEL_BF16_SMALL); host only."""
    r = load().gemm355_supergroup(int(kernel), int(tiles_n), int(K))
    if r < 0:
        raise Gemm355Error(-r, "gemm355_supergroup")
    return r


def bf16_plan(M: int, N: int, K: int, compute_units: int, with_workspace: bool = False):
    """(instance, splits) that gemm_bf16_nt (or, with_workspace, gemm_bf16_nt_ws)
    runs for this shape on a device with `compute_units` compute units; host only."""
    return _plan(M, N, K, compute_units, with_workspace)[:2]


def bf16_plan_workspace_bytes(M: int, N: int, K: int, compute_units: int) -> int:
    """Workspace bytes of gemm_bf16_nt_ws's plan on such a device; host only."""
    return _plan(M, N, K, compute_units, True)[2]


def tile_order(tiles_m: int, tiles_n: int, supergroup: int):
    """Visiting order of output tiles as two lists (tm, tn); host only."""
    lib = load()
    n = tiles_m * tiles_n
    tm = (ctypes.c_int * max(n, 1))()
    tn = (ctypes.c_int * max(n, 1))()
    _check(lib.gemm355_tile_order(tiles_m, tiles_n, supergroup, tm, tn), "gemm355_tile_order")
    return list(tm[:n]), list(tn[:n])


def schedule(tiles: int, grid: int):
    """slot[w][r] = visiting-order position of workgroup w in round r (-1: none)."""
    lib = load()
    rounds = -(-tiles // grid) if tiles > 0 and grid > 0 else 1
    buf = (ctypes.c_int * max(rounds * max(grid, 1), 1))()
    r = lib.gemm355_schedule(tiles, grid, buf, len(buf))
    if r < 0:
        raise Gemm355Error(-r, "gemm355_schedule")
    return [list(buf[w * r:(w + 1) * r]) for w in range(grid)]
