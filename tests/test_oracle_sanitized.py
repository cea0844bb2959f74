"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

oracle355.c is compiled a second time, together with a small driver
(oracle/sanitize_driver.c), into one executable built with
-fsanitize=address,undefined,float-cast-overflow and no recovery: any
out-of-bounds access, use after free, leak, signed overflow, bad shift or
out-of-range float-to-integer conversion aborts it. Each case runs every
entry point of one kind (full product, sampled elements with their binary64
sums, fused bias + activation, the FP4 decode, the codecs) on tiny ragged
shapes, each operand in a heap block of exactly its size, and the results
must be bitwise those of the regular build, which the other oracle tests pin.
"""
import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
import synthetic as syn

_EXE = None


def _exe():
    global _EXE
    if _EXE is None:
        _EXE = oracle.build_sanitized()
    return _EXE


def _run(header, arrays, out_sizes):
    """Write a case, run the sanitized driver on it, split its result file."""
    with tempfile.TemporaryDirectory() as d:
        case, res = os.path.join(d, "case.bin"), os.path.join(d, "res.bin")
        with open(case, "wb") as f:
            f.write(np.array(list(header) + [0] * (8 - len(header)), dtype="<i4").tobytes())
            for a in arrays:
                f.write(np.ascontiguousarray(a).tobytes())
        env = dict(os.environ, OMP_NUM_THREADS="3",
                   ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        p = subprocess.run([_exe(), case, res], capture_output=True, text=True, env=env, timeout=120)
        assert p.returncode == 0, p.stderr[-3000:]
        assert "runtime error" not in p.stderr and "Sanitizer" not in p.stderr, p.stderr[-3000:]
        raw = open(res, "rb").read()
    out, pos = [], 0
    for dtype, n in out_sizes:
        nbytes = np.dtype(dtype).itemsize * n
        out.append(np.frombuffer(raw[pos:pos + nbytes], dtype=dtype))
        pos += nbytes
    assert pos == len(raw)
    return out


def _all_positions(M, N, seed):
    ms, ns = (x.ravel().astype(np.int32) for x in np.meshgrid(np.arange(M), np.arange(N), indexing="ij"))
    g = np.random.Generator(np.random.PCG64(seed))
    extra = g.integers(0, M * N, 5)   # some positions twice
    return np.concatenate([ms, ms[extra]]), np.concatenate([ns, ns[extra]])


def _same(a, b):
    return np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))


@pytest.mark.parametrize("M,N,K,act", [(1, 1, 1, 0), (3, 5, 8, 1), (17, 16, 33, 2), (33, 31, 17, 2),
                                       (5, 8, 0, 1)])
def test_bf16_entry_points_clean_and_equal(M, N, K, act):
    A = syn.bf16_uniform(M, K, seed=M + 7 * K) if K else np.zeros((M, 0), np.uint16)
    B = syn.bf16_uniform(N, K, seed=N + 7 * K + 1) if K else np.zeros((N, 0), np.uint16)
    bias = syn.bf16_uniform(1, N, seed=N + 3, lo=-4.0, hi=4.0)[0]
    ms, ns = _all_positions(M, N, M + N)
    n = ms.size
    C, at, s, Cb, atb, z = _run((1, M, N, K, act, n), [A, B, bias, ms, ns],
                                [("<u2", M * N), ("<u2", n), ("<f8", n), ("<u2", M * N), ("<u2", n), ("<f8", n)])
    assert _same(C.reshape(M, N), oracle.gemm_bf16_nt(A, B))
    want_at, want_s = oracle.gemm_bf16_nt_at(A, B, ms, ns, with_sum=True)
    assert _same(at, want_at) and _same(s, want_s)
    assert _same(Cb.reshape(M, N), oracle.gemm_bf16_nt_bias_act(A, B, bias, act))
    want_b, want_z = oracle.gemm_bf16_nt_bias_act_at(A, B, bias, act, ms, ns, with_z=True)
    assert _same(atb, want_b) and _same(z, want_z)


@pytest.mark.parametrize("M,N,K,act", [(1, 1, 16, 0), (3, 5, 32, 1), (17, 16, 48, 2), (2, 33, 64, 2)])
def test_nvfp4_entry_points_clean_and_equal(M, N, K, act):
    Aq, SFA = syn.fp4_operand(M, K, seed=M + K)
    Bq, SFB = syn.fp4_operand(N, K, seed=N + K + 1)
    bias = syn.bf16_uniform(1, N, seed=N + 5, lo=-64.0, hi=64.0)[0]
    ms, ns = _all_positions(M, N, M * N)
    n = ms.size
    C, at, s, atb, z, dec = _run((2, M, N, K, act, n), [Aq, SFA, Bq, SFB, bias, ms, ns],
                                 [("<u2", M * N), ("<u2", n), ("<f8", n), ("<u2", n), ("<f8", n), ("<f8", M * K)])
    assert _same(C.reshape(M, N), oracle.gemm_nvfp4_nt(Aq, SFA, Bq, SFB, K))
    want_at, want_s = oracle.gemm_nvfp4_nt_at(Aq, SFA, Bq, SFB, K, ms, ns, with_sum=True)
    assert _same(at, want_at) and _same(s, want_s)
    want_b, want_z = oracle.gemm_nvfp4_nt_bias_act_at(Aq, SFA, Bq, SFB, K, bias, act, ms, ns, with_z=True)
    assert _same(atb, want_b) and _same(z, want_z)
    assert _same(dec.reshape(M, K), oracle.decode_nvfp4(Aq, SFA, K))


@pytest.mark.parametrize("M,N,K,act", [(1, 1, 32, 0), (3, 5, 32, 1), (17, 16, 64, 2), (2, 33, 96, 1)])
def test_mxfp4_entry_points_clean_and_equal(M, N, K, act):
    Aq, SA = syn.mxfp4_operand(M, K, seed=M + K)
    Bq, SB = syn.mxfp4_operand(N, K, seed=N + K + 1)
    bias = syn.bf16_uniform(1, N, seed=N + 9, lo=-16.0, hi=16.0)[0]
    ms, ns = _all_positions(M, N, M * N + 1)
    n = ms.size
    C, at, s, atb, z = _run((3, M, N, K, act, n), [Aq, SA, Bq, SB, bias, ms, ns],
                            [("<u2", M * N), ("<u2", n), ("<f8", n), ("<u2", n), ("<f8", n)])
    assert _same(C.reshape(M, N), oracle.gemm_mxfp4_nt(Aq, SA, Bq, SB, K))
    want_at, want_s = oracle.gemm_mxfp4_nt_at(Aq, SA, Bq, SB, K, ms, ns, with_sum=True)
    assert _same(at, want_at) and _same(s, want_s)
    want_b, want_z = oracle.gemm_mxfp4_nt_bias_act_at(Aq, SA, Bq, SB, K, bias, act, ms, ns, with_z=True)
    assert _same(atb, want_b) and _same(z, want_z)


def test_codecs_clean_and_equal():
    g = np.random.Generator(np.random.PCG64(77))
    # ties, near-ties, subnormals, the overflow edge, zeros and a wide spread
    x = np.concatenate([
        np.array([0.0, -0.0, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 2 - 2.0 ** -9, 2.0 ** -133, 3 * 2.0 ** -134,
                  -(2.0 ** -140), 3.3895313892515355e38, 3.39e38, -1e-45, 1e30, -7.25]),
        g.standard_normal(2000) * np.exp2(g.integers(-140, 127, 2000)),
    ])
    n = x.size
    dec, e2, e4, e8, r, rn, back = _run((4, 0, 0, 0, 0, n), [x.astype("<f8")],
                                        [("<f8", 65536), ("<f8", 16), ("<f8", 256), ("<f8", 256), ("<u2", n),
                                         ("<u2", n), ("<f8", n)])
    assert _same(dec, oracle.bf16_to_double(np.arange(65536, dtype=np.uint16)))
    assert _same(e2, np.array([oracle.e2m1_to_double(c) for c in range(16)]))
    e4_want = np.array([oracle.e4m3_to_double(b) for b in range(256)])
    assert np.array_equal(np.isnan(e4), np.isnan(e4_want)) and _same(e4[~np.isnan(e4)], e4_want[~np.isnan(e4_want)])
    e8_want = np.array([oracle.e8m0_to_double(b) for b in range(256)])
    assert np.array_equal(np.isnan(e8), np.isnan(e8_want)) and _same(e8[~np.isnan(e8)], e8_want[~np.isnan(e8_want)])
    want = oracle.bf16_from_double(x)
    assert _same(r, want) and _same(rn, want)
    assert _same(back, oracle.bf16_to_double(want))


def test_the_sanitizers_are_live():
    # a copy of the oracle whose BF16 sum reads one element past each row:
    # the sanitized build must abort on the case above (the last row of B
    # reads past its heap block)
    src = open(oracle.SOURCE).read()
    old = "for (long k = 0; k < K; ++k)\n        s += bf16_elem"
    assert old in src
    with tempfile.TemporaryDirectory() as d:
        bad_src = os.path.join(d, "oracle355.c")
        open(bad_src, "w").write(src.replace(old, "for (long k = 0; k <= K; ++k)\n        s += bf16_elem"))
        exe = os.path.join(d, "bad")
        subprocess.run(["gcc", *oracle.SANITIZE_FLAGS, "-o", exe, bad_src, oracle.SANITIZE_DRIVER, "-lm"],
                       check=True)
        M, N, K = 3, 5, 8
        case, res = os.path.join(d, "case.bin"), os.path.join(d, "res.bin")
        with open(case, "wb") as f:
            f.write(np.array([1, M, N, K, 0, 1, 0, 0], dtype="<i4").tobytes())
            for a in (syn.bf16_uniform(M, K, 1), syn.bf16_uniform(N, K, 2), np.zeros(N, np.uint16),
                      np.zeros(1, np.int32), np.zeros(1, np.int32)):
                f.write(a.tobytes())
        p = subprocess.run([exe, case, res], capture_output=True, text=True, timeout=120,
                           env=dict(os.environ, OMP_NUM_THREADS="1"))
        assert p.returncode != 0 and "AddressSanitizer" in p.stderr, (p.returncode, p.stderr[-2000:])
