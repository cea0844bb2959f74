"""Plain CPU reference ("oracle") for the dense NT GEMM -- test infrastructure.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The GPU product
path (``dense_gemm_14_amd`` and ``libgemm355.so``) never imports it, and the two
share no source.

The arithmetic lives in ``oracle355.c`` (plain C, built with gcc, summed in
binary64, k ascending); this module only builds it and marshals numpy arrays.
Operands are passed as their raw bit patterns: BF16 as ``uint16``, packed E2M1
codes and E4M3 scales as ``uint8``.

What is computed (cited passages):
  * C = A @ B^T, A (M x K) and B (N x K) row-major, BF16 in and out
    ("Achieve cuBLAS Performance on NVIDIA GB300 for HGEMM", opening paragraph);
  * output rounding to nearest, ties to even ("Optimized B200 Matrix
    Multiplication", section 5 "The Epilogue");
  * block-scaled FP4: E2M1 values with one FP8 scale per 16 elements
    ("NVFP4 GEMM on Blackwell", section "NVFP4 Datatype");
  * a fused epilogue, bias and activation applied to the sum before rounding
    ("NVFP4 GEMM on Blackwell", "Kernel 1", "Epilogue Warps").
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle355.c")
_SRC = SOURCE
LIB_PATH = os.path.join(_HERE, "liboracle355.so")

_lib = None


GCC_FLAGS = ["-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
             "-fno-fast-math", "-Wall", "-Wextra"]


def compile_source(src: str, out: str) -> str:
    """gcc one C source into a shared library at ``out``."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *GCC_FLAGS, "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


SANITIZE_DRIVER = os.path.join(_HERE, "sanitize_driver.c")
SANITIZED_PATH = os.path.join(_HERE, "oracle355_sanitized")
SANITIZE_FLAGS = ["-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
                  "-fno-omit-frame-pointer", "-fsanitize=address,undefined,float-cast-overflow",
                  "-fno-sanitize-recover=all"]


def build_sanitized() -> str:
    """gcc oracle355.c with sanitize_driver.c into one executable built with
    AddressSanitizer and UndefinedBehaviorSanitizer (CPU tests only)."""
    tmp = SANITIZED_PATH + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *SANITIZE_FLAGS, "-o", tmp, _SRC, SANITIZE_DRIVER, "-lm"], check=True)
    os.replace(tmp, SANITIZED_PATH)
    return SANITIZED_PATH


def build(force: bool = True) -> str:
    """Compile ``liboracle355.so`` with gcc (no HIP, no GPU headers), and the
    sanitizer build of the same source used by the CPU tests."""
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    build_sanitized()
    return compile_source(_SRC, LIB_PATH)


def _bind(lib):
    p = ctypes.c_void_p
    i = ctypes.c_int
    lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_double.restype = ctypes.c_double
    lib.oracle_bf16_from_double.argtypes = [ctypes.c_double]
    lib.oracle_bf16_from_double.restype = ctypes.c_uint16
    lib.oracle_e2m1_to_double.argtypes = [ctypes.c_uint]
    lib.oracle_e2m1_to_double.restype = ctypes.c_double
    lib.oracle_e4m3_to_double.argtypes = [ctypes.c_uint]
    lib.oracle_e4m3_to_double.restype = ctypes.c_double
    lib.oracle_bf16_to_double_n.argtypes = [p, p, ctypes.c_long]
    lib.oracle_bf16_to_double_n.restype = None
    lib.oracle_bf16_from_double_n.argtypes = [p, p, ctypes.c_long]
    lib.oracle_bf16_from_double_n.restype = None
    lib.oracle_gemm_bf16_nt.argtypes = [i, i, i, p, p, p]
    lib.oracle_gemm_bf16_nt.restype = i
    lib.oracle_gemm_nvfp4_nt.argtypes = [i, i, i, p, p, p, p, p]
    lib.oracle_gemm_nvfp4_nt.restype = i
    lib.oracle_gemm_bf16_nt_at.argtypes = [i, i, i, p, p, ctypes.c_long, p, p, p, p]
    lib.oracle_gemm_bf16_nt_at.restype = i
    lib.oracle_gemm_nvfp4_nt_at.argtypes = [i, i, i, p, p, p, p, ctypes.c_long, p, p, p, p]
    lib.oracle_gemm_nvfp4_nt_at.restype = i
    lib.oracle_activate.argtypes = [ctypes.c_double, i]
    lib.oracle_activate.restype = ctypes.c_double
    lib.oracle_gemm_bf16_nt_bias_act.argtypes = [i, i, i, p, p, p, i, p]
    lib.oracle_gemm_bf16_nt_bias_act.restype = i
    lib.oracle_gemm_bf16_nt_bias_act_at.argtypes = [i, i, i, p, p, p, i, ctypes.c_long, p, p, p, p]
    lib.oracle_gemm_bf16_nt_bias_act_at.restype = i
    lib.oracle_gemm_nvfp4_nt_bias_act_at.argtypes = [i, i, i, p, p, p, p, p, i, ctypes.c_long, p, p, p, p]
    lib.oracle_gemm_nvfp4_nt_bias_act_at.restype = i
    lib.oracle_e8m0_to_double.argtypes = [ctypes.c_uint]
    lib.oracle_e8m0_to_double.restype = ctypes.c_double
    lib.oracle_gemm_mxfp4_nt.argtypes = [i, i, i, p, p, p, p, p]
    lib.oracle_gemm_mxfp4_nt.restype = i
    lib.oracle_gemm_mxfp4_nt_at.argtypes = [i, i, i, p, p, p, p, ctypes.c_long, p, p, p, p]
    lib.oracle_gemm_mxfp4_nt_at.restype = i
    lib.oracle_gemm_mxfp4_nt_bias_act_at.argtypes = [i, i, i, p, p, p, p, p, i, ctypes.c_long, p, p, p, p]
    lib.oracle_gemm_mxfp4_nt_bias_act_at.restype = i
    lib.oracle_decode_nvfp4.argtypes = [i, i, p, p, p]
    lib.oracle_decode_nvfp4.restype = i
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = i
    lib.oracle_set_threads.argtypes = [i]
    lib.oracle_set_threads.restype = None
    return lib


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(_SRC):
        build()
    _lib = _bind(ctypes.CDLL(LIB_PATH))
    return _lib


@contextlib.contextmanager
def using_library(path: str):
    """Temporarily route every call through another build of oracle355.c.

    Used by the mutation tests, which compile deliberately broken copies of the
    source on the CPU to show that the pins catch each planted mistake.
    """
    global _lib
    saved = _load()
    _lib = _bind(ctypes.CDLL(path))
    try:
        yield
    finally:
        _lib = saved


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data) if a.size else ctypes.c_void_p(0)


def _c(a, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError("expected %s array, got %s" % (np.dtype(dtype), a.dtype))
    return a


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError("%s: oracle rejected the arguments (code %d)" % (what, rc))


# ---- scalar codecs -------------------------------------------------------

def bf16_to_double(bits) -> np.ndarray:
    """BF16 bit patterns -> float64 (elementwise, through the C codec)."""
    lib = _load()
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.float64)
    lib.oracle_bf16_to_double_n(_ptr(bits), _ptr(out), bits.size)
    return out


def bf16_from_double(x) -> np.ndarray:
    """float64 -> BF16 bit patterns, round to nearest even in one step."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    lib.oracle_bf16_from_double_n(_ptr(x), _ptr(out), x.size)
    return out


def e2m1_to_double(code: int) -> float:
    return _load().oracle_e2m1_to_double(int(code))


def e4m3_to_double(byte: int) -> float:
    return _load().oracle_e4m3_to_double(int(byte))


# ---- products --------------------------------------------------------------

def gemm_bf16_nt(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """C = bf16(A @ B^T) for BF16 bit arrays A (M, K) and B (N, K)."""
    lib = _load()
    A = _c(A, np.uint16)
    B = _c(B, np.uint16)
    M, K = A.shape
    N, K2 = B.shape
    if K != K2:
        raise ValueError("K mismatch")
    C = np.empty((M, N), dtype=np.uint16)
    _check(lib.oracle_gemm_bf16_nt(M, N, K, _ptr(A), _ptr(B), _ptr(C)), "gemm_bf16_nt")
    return C


def gemm_nvfp4_nt(Aq, SFA, Bq, SFB, K: int) -> np.ndarray:
    """C = bf16(dec(A) @ dec(B)^T) for packed E2M1 codes and E4M3 scales.

    Aq (M, K/2) uint8, SFA (M, K/16) uint8, Bq (N, K/2), SFB (N, K/16).
    """
    lib = _load()
    Aq, SFA, Bq, SFB = (_c(x, np.uint8) for x in (Aq, SFA, Bq, SFB))
    M, N = Aq.shape[0], Bq.shape[0]
    _shape_fp4(Aq, SFA, M, K)
    _shape_fp4(Bq, SFB, N, K)
    C = np.empty((M, N), dtype=np.uint16)
    _check(lib.oracle_gemm_nvfp4_nt(M, N, K, _ptr(Aq), _ptr(SFA), _ptr(Bq), _ptr(SFB), _ptr(C)),
           "gemm_nvfp4_nt")
    return C


ACT_NONE, ACT_RELU, ACT_GELU_TANH = 0, 1, 2


def activate(z: float, act: int) -> float:
    """The fused epilogue's activation of one binary64 value."""
    return _load().oracle_activate(float(z), int(act))


def _bias(bias, N):
    if bias is None:
        return None
    bias = _c(bias, np.uint16)
    if bias.shape != (N,):
        raise ValueError("bias must hold N = %d BF16 values" % N)
    return bias


def gemm_bf16_nt_bias_act(A: np.ndarray, B: np.ndarray, bias, act: int) -> np.ndarray:
    """C = bf16(act(A @ B^T + bias)) for BF16 bit arrays; bias (N,) or None."""
    lib = _load()
    A = _c(A, np.uint16)
    B = _c(B, np.uint16)
    M, K = A.shape
    N, K2 = B.shape
    if K != K2:
        raise ValueError("K mismatch")
    bias = _bias(bias, N)
    C = np.empty((M, N), dtype=np.uint16)
    _check(lib.oracle_gemm_bf16_nt_bias_act(M, N, K, _ptr(A), _ptr(B), _ptr(bias) if bias is not None else None,
                                            int(act), _ptr(C)), "gemm_bf16_nt_bias_act")
    return C


def gemm_bf16_nt_bias_act_at(A, B, bias, act: int, ms, ns, with_z: bool = False):
    """Only the elements C[ms[i], ns[i]] (and optionally z before the activation)."""
    lib = _load()
    A = _c(A, np.uint16)
    B = _c(B, np.uint16)
    M, K = A.shape
    N = B.shape[0]
    bias = _bias(bias, N)
    ms, ns = _idx(ms, ns)
    out = np.empty(ms.size, dtype=np.uint16)
    zs = np.empty(ms.size, dtype=np.float64)
    _check(lib.oracle_gemm_bf16_nt_bias_act_at(M, N, K, _ptr(A), _ptr(B),
                                               _ptr(bias) if bias is not None else None, int(act), ms.size,
                                               _ptr(ms), _ptr(ns), _ptr(out), _ptr(zs)),
           "gemm_bf16_nt_bias_act_at")
    return (out, zs) if with_z else out


def gemm_nvfp4_nt_bias_act_at(Aq, SFA, Bq, SFB, K: int, bias, act: int, ms, ns, with_z: bool = False):
    """Elements C[ms[i], ns[i]] of bf16(act(dec(A) @ dec(B)^T + bias))
    (and optionally z before the activation)."""
    lib = _load()
    Aq, SFA, Bq, SFB = (_c(x, np.uint8) for x in (Aq, SFA, Bq, SFB))
    M, N = Aq.shape[0], Bq.shape[0]
    _shape_fp4(Aq, SFA, M, K)
    _shape_fp4(Bq, SFB, N, K)
    bias = _bias(bias, N)
    ms, ns = _idx(ms, ns)
    out = np.empty(ms.size, dtype=np.uint16)
    zs = np.empty(ms.size, dtype=np.float64)
    _check(lib.oracle_gemm_nvfp4_nt_bias_act_at(M, N, K, _ptr(Aq), _ptr(SFA), _ptr(Bq), _ptr(SFB),
                                                _ptr(bias) if bias is not None else None, int(act), ms.size,
                                                _ptr(ms), _ptr(ns), _ptr(out), _ptr(zs)),
           "gemm_nvfp4_nt_bias_act_at")
    return (out, zs) if with_z else out


def e8m0_to_double(byte: int) -> float:
    return _load().oracle_e8m0_to_double(int(byte))


def _shape_mx(Q, S, rows, K):
    if K % 32:
        raise ValueError("K must be a multiple of 32 for one scale per 32 elements")
    if Q.shape != (rows, K // 2) or S.shape != (rows, K // 32):
        raise ValueError("MXFP4 operand shapes do not match K=%d: codes %s, scales %s" % (K, Q.shape, S.shape))


def gemm_mxfp4_nt(Aq, SA, Bq, SB, K: int) -> np.ndarray:
    """C = bf16(dec(A) @ dec(B)^T) for E2M1 codes with one E8M0 scale per 32
    elements: Aq (M, K/2), SA (M, K/32), Bq (N, K/2), SB (N, K/32), uint8."""
    lib = _load()
    Aq, SA, Bq, SB = (_c(x, np.uint8) for x in (Aq, SA, Bq, SB))
    M, N = Aq.shape[0], Bq.shape[0]
    _shape_mx(Aq, SA, M, K)
    _shape_mx(Bq, SB, N, K)
    C = np.empty((M, N), dtype=np.uint16)
    _check(lib.oracle_gemm_mxfp4_nt(M, N, K, _ptr(Aq), _ptr(SA), _ptr(Bq), _ptr(SB), _ptr(C)), "gemm_mxfp4_nt")
    return C


def gemm_mxfp4_nt_at(Aq, SA, Bq, SB, K: int, ms, ns, with_sum: bool = False):
    lib = _load()
    Aq, SA, Bq, SB = (_c(x, np.uint8) for x in (Aq, SA, Bq, SB))
    M, N = Aq.shape[0], Bq.shape[0]
    _shape_mx(Aq, SA, M, K)
    _shape_mx(Bq, SB, N, K)
    ms, ns = _idx(ms, ns)
    out = np.empty(ms.size, dtype=np.uint16)
    sums = np.empty(ms.size, dtype=np.float64)
    _check(lib.oracle_gemm_mxfp4_nt_at(M, N, K, _ptr(Aq), _ptr(SA), _ptr(Bq), _ptr(SB), ms.size, _ptr(ms), _ptr(ns),
                                       _ptr(out), _ptr(sums)), "gemm_mxfp4_nt_at")
    return (out, sums) if with_sum else out


def gemm_mxfp4_nt_bias_act_at(Aq, SA, Bq, SB, K: int, bias, act: int, ms, ns, with_z: bool = False):
    """Elements C[ms[i], ns[i]] of bf16(act(dec(A) @ dec(B)^T + bias)) for
    microscaled FP4 operands (and optionally z before the activation)."""
    lib = _load()
    Aq, SA, Bq, SB = (_c(x, np.uint8) for x in (Aq, SA, Bq, SB))
    M, N = Aq.shape[0], Bq.shape[0]
    _shape_mx(Aq, SA, M, K)
    _shape_mx(Bq, SB, N, K)
    bias = _bias(bias, N)
    ms, ns = _idx(ms, ns)
    out = np.empty(ms.size, dtype=np.uint16)
    zs = np.empty(ms.size, dtype=np.float64)
    _check(lib.oracle_gemm_mxfp4_nt_bias_act_at(M, N, K, _ptr(Aq), _ptr(SA), _ptr(Bq), _ptr(SB),
                                                _ptr(bias) if bias is not None else None, int(act), ms.size,
                                                _ptr(ms), _ptr(ns), _ptr(out), _ptr(zs)),
           "gemm_mxfp4_nt_bias_act_at")
    return (out, zs) if with_z else out


def _shape_fp4(Q, SF, rows, K):
    if K % 16:
        raise ValueError("K must be a multiple of 16 for one scale per 16 elements")
    if Q.shape != (rows, K // 2) or SF.shape != (rows, K // 16):
        raise ValueError("FP4 operand shapes do not match K=%d: codes %s, scales %s"
                         % (K, Q.shape, SF.shape))


def _idx(ms, ns):
    ms = np.ascontiguousarray(ms, dtype=np.int32)
    ns = np.ascontiguousarray(ns, dtype=np.int32)
    if ms.shape != ns.shape or ms.ndim != 1:
        raise ValueError("ms and ns must be 1-D and the same length")
    return ms, ns


def gemm_bf16_nt_at(A, B, ms, ns, with_sum: bool = False):
    """Only the elements C[ms[i], ns[i]] (and optionally their binary64 sums)."""
    lib = _load()
    A = _c(A, np.uint16)
    B = _c(B, np.uint16)
    M, K = A.shape
    N = B.shape[0]
    ms, ns = _idx(ms, ns)
    out = np.empty(ms.size, dtype=np.uint16)
    sums = np.empty(ms.size, dtype=np.float64)
    _check(lib.oracle_gemm_bf16_nt_at(M, N, K, _ptr(A), _ptr(B), ms.size, _ptr(ms), _ptr(ns),
                                      _ptr(out), _ptr(sums)), "gemm_bf16_nt_at")
    return (out, sums) if with_sum else out


def gemm_nvfp4_nt_at(Aq, SFA, Bq, SFB, K: int, ms, ns, with_sum: bool = False):
    lib = _load()
    Aq, SFA, Bq, SFB = (_c(x, np.uint8) for x in (Aq, SFA, Bq, SFB))
    M, N = Aq.shape[0], Bq.shape[0]
    _shape_fp4(Aq, SFA, M, K)
    _shape_fp4(Bq, SFB, N, K)
    ms, ns = _idx(ms, ns)
    out = np.empty(ms.size, dtype=np.uint16)
    sums = np.empty(ms.size, dtype=np.float64)
    _check(lib.oracle_gemm_nvfp4_nt_at(M, N, K, _ptr(Aq), _ptr(SFA), _ptr(Bq), _ptr(SFB), ms.size,
                                       _ptr(ms), _ptr(ns), _ptr(out), _ptr(sums)),
           "gemm_nvfp4_nt_at")
    return (out, sums) if with_sum else out


def decode_nvfp4(Q, SF, K: int) -> np.ndarray:
    """Decoded block-scaled FP4 operand as float64 (rows, K)."""
    lib = _load()
    Q = _c(Q, np.uint8)
    SF = _c(SF, np.uint8)
    rows = Q.shape[0]
    _shape_fp4(Q, SF, rows, K)
    out = np.empty((rows, K), dtype=np.float64)
    _check(lib.oracle_decode_nvfp4(rows, K, _ptr(Q), _ptr(SF), _ptr(out)), "decode_nvfp4")
    return out


def max_threads() -> int:
    return _load().oracle_max_threads()


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))
