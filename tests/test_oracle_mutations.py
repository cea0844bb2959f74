"""Planted mistakes in the oracle are caught by its pins (CPU only).

Each case compiles a copy of the oracle's C source with one plausible mistake
(a dropped term, a wrong sign, bias or index, a swapped nibble, a wrong
rounding rule, a narrower accumulator) into a temporary library, runs a quick
subset of the pins against it, and requires at least one pin to fail.
"""
import os
import tempfile
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synthetic as syn
from tests import exact

MUTATIONS = {
    "dropped_first_term": ("for (long k = 0; k < K; ++k)\n        s += bf16_elem",
                           "for (long k = 1; k < K; ++k)\n        s += bf16_elem"),
    "dropped_last_fp4_term": ("for (long k = 0; k < K; ++k)\n        s += fp4_elem",
                              "for (long k = 0; k < K - 1; ++k)\n        s += fp4_elem"),
    "e2m1_sign_lost": ("ldexp(1.0 + 0.5 * (double)m, (int)e - 1);\n    return s ? -mag : mag;",
                       "ldexp(1.0 + 0.5 * (double)m, (int)e - 1);\n    return mag;"),
    "e2m1_bias": ("(int)e - 1);", "(int)e - 2);"),
    "e2m1_subnormal": ("? 0.5 * (double)m", "? 1.0 * (double)m"),
    "e4m3_bias": ("(int)e - 7);", "(int)e - 8);"),
    "nibble_order": ("(k & 1) ? (unsigned)(byte >> 4) : (unsigned)(byte & 15u);\n    return oracle_e2m1_to_double(code) * oracle_e4m3",
                     "(k & 1) ? (unsigned)(byte & 15u) : (unsigned)(byte >> 4);\n    return oracle_e2m1_to_double(code) * oracle_e4m3"),
    # (the nibble order of the microscaled product has no mutant: swapping it
    # relabels k and k ^ 1 in both operands alike, and both lie in one scale
    # block, so every product is unchanged)
    "mx_scale_row": ("S[row * (K / 32) + k / 32]", "S[(row / 2) * (K / 32) + k / 32]"),
    "mx_scale_block_64": ("S[row * (K / 32) + k / 32]", "S[row * (K / 32) + (k / 64) * 2]"),
    "e8m0_bias": ("ldexp(1.0, (int)byte - 127)", "ldexp(1.0, (int)byte - 128)"),
    "scale_block_32": ("SF[row * (K / 16) + k / 16]", "SF[row * (K / 16) + k / 32]"),
    "scale_row": ("SF[row * (K / 16) + k / 16]", "SF[(row / 2) * (K / 16) + k / 16]"),
    "ties_away": ("if (frac > 0.5)", "if (frac >= 0.5)"),
    "ties_to_odd": ("fmod(lower, 2.0) != 0.0", "fmod(lower, 2.0) == 0.0"),
    "truncate": ("if (frac > 0.5)\n        q = lower + 1.0;", "if (frac > 2.0)\n        q = lower + 1.0;"),
    "float_accumulator": ("static double dot_bf16(const uint16_t *A, const uint16_t *B, long K, long m, long n)\n{\n    double s = 0.0;",
                          "static double dot_bf16(const uint16_t *A, const uint16_t *B, long K, long m, long n)\n{\n    float s = 0.0f;"),
    "subnormal_quantum": ("if (qexp < -133)\n        qexp = -133;", "if (qexp < -126)\n        qexp = -126;"),
    "same_operand_twice": ("bf16_elem(A, K, m, k) * bf16_elem(B, K, n, k)",
                           "bf16_elem(A, K, m, k) * bf16_elem(A, K, m, k)"),
    "b_row_for_a": ("bf16_elem(A, K, m, k) * bf16_elem(B, K, n, k)",
                    "bf16_elem(A, K, n % 1, k) * bf16_elem(B, K, n, k)"),
    "output_transposed": ("C[m * (long)N + n] = oracle_bf16_from_double(dot_bf16(A, B, K, m, n));",
                          "C[m * (long)N + n] = oracle_bf16_from_double(dot_bf16(A, B, K, n % M, m % N));"),
}


def _pins_pass() -> bool:
    """A quick subset of the pins; True only if every one of them holds."""
    checks = []
    # codecs
    xs = [1 + 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -40, 2 - 2.0 ** -8, 2.0 ** -133, 3 * 2.0 ** -134, 1.3]
    got = oracle.bf16_from_double(np.array(xs))
    checks.append(all(int(g) == exact.rne_bf16(Fraction(x)) for g, x in zip(got, xs)))
    checks.append(all(oracle.e2m1_to_double(c) == float(exact.e2m1_fraction(c)) for c in range(16)))
    checks.append(all(oracle.e4m3_to_double(b) == float(exact.e4m3_fraction(b)) for b in range(0, 120)))
    # BF16 brute force, identity, transpose
    for (M, N, K) in [(3, 5, 17), (5, 3, 33), (2, 2, 8)]:
        A = syn.bf16_uniform(M, K, seed=M * 7 + K)
        B = syn.bf16_uniform(N, K, seed=N * 7 + K + 1)
        ref = exact.gemm_exact_bits(exact.bf16_bits_to_fractions(A), exact.bf16_bits_to_fractions(B))
        checks.append(np.array_equal(oracle.gemm_bf16_nt(A, B), ref))
    A = syn.bf16_uniform(6, 16, seed=3)
    checks.append(np.array_equal(oracle.gemm_bf16_nt(A, syn.bf16_identity(16)), A))
    # a sum whose low bits decide the final rounding
    tie = syn.to_bf16_bits(np.array([[1.0, 2.0 ** -8, 2.0 ** -30]]))
    checks.append(int(oracle.gemm_bf16_nt(tie, syn.to_bf16_bits(np.ones((1, 3))))[0, 0]) == 0x3F81)
    # FP4 brute force
    for (M, N, K) in [(3, 4, 32), (4, 3, 48)]:
        Aq, SFA = syn.fp4_operand(M, K, seed=M + K)
        Bq, SFB = syn.fp4_operand(N, K, seed=N + K + 5)
        ref = exact.gemm_exact_bits(exact.fp4_fractions(Aq, SFA, K), exact.fp4_fractions(Bq, SFB, K))
        checks.append(np.array_equal(oracle.gemm_nvfp4_nt(Aq, SFA, Bq, SFB, K), ref))
    # element decode (the nibble order is invisible in a product whose two
    # operands follow the same convention, but not in the decoded operand)
    Q, SF = syn.fp4_operand(2, 32, seed=9)
    dec = oracle.decode_nvfp4(Q, SF, 32)
    ref = exact.fp4_fractions(Q, SF, 32)
    checks.append(all(dec[r, k] == float(ref[r, k]) for r in range(2) for k in range(32)))
    # microscaled FP4: E8M0 values, and A against an identity B coded as
    # 1.0 (code 2) with unit scales, whose product is A decoded by hand
    checks.append(all(oracle.e8m0_to_double(b) == 2.0 ** (b - 127) for b in range(255)))
    K = 128
    Q, S = syn.mxfp4_operand(3, K, seed=11)
    codes = np.zeros((K, K), np.uint8)
    codes[np.arange(K), np.arange(K)] = 2
    got = oracle.gemm_mxfp4_nt(Q, S, syn.pack_nibbles(codes), np.full((K, K // 32), 127, np.uint8), K)
    nib = lambda r, k: (int(Q[r, k // 2]) >> (4 * (k & 1))) & 15
    want = [[exact.rne_bf16(exact.e2m1_fraction(nib(r, k)) * Fraction(2) ** (int(S[r, k // 32]) - 127))
             for k in range(K)] for r in range(3)]
    # compared as values: code 8 is -0
    checks.append(all(exact.rne_bf16(Fraction(oracle.bf16_to_double(np.array([got[r, k]]))[0].item())) == want[r][k]
                      for r in range(3) for k in range(K)))
    return all(checks)


def test_unmutated_source_passes_the_quick_pins():
    assert _pins_pass()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    old, new = MUTATIONS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, "mutation anchor for %s not found exactly once" % name
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "mutant.c")
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        lib = oracle.compile_source(path, os.path.join(d, "libmutant.so"))
        with oracle.using_library(lib):
            assert not _pins_pass(), "planted mistake %r went unnoticed" % name
