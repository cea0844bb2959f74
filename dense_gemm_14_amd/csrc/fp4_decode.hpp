// fp4_decode.hpp -- block-scaled FP4 operands ("NVFP4 GEMM on Blackwell",
// section "NVFP4 Datatype") decoded once into BF16 rows, for the decode-first
// path of gemm_nvfp4_nt_ws: the BF16 product then runs on the decoded
// operands.
//
// Why a second path beside the kernel that decodes while staging: there every
// 256 x 256 tile decodes its own A and B strips, so at M = N = K = 8192 each
// operand element is decoded 32 times, and the decode's vector work and LDS
// writes hold that kernel at the board power limit at a lower clock than the
// BF16 kernel. Decoding once costs a read of the codes and a write and re-read
// of 2 (M + N) K bytes of BF16 in HBM instead.
//
// A thread decodes 32 consecutive elements of one row: 16 code bytes, the two
// E4M3 scales of their 16-element blocks, 64 bytes of BF16 out. The decode is
// the staging kernel's (decode8, exact to FP16); FP16 -> BF16 is then exact as
// well (every decoded value has at most 6 significant bits and lies in
// [2^-10, 2688]), by way of FP32 and its top 16 bits.
#pragma once

#include "gemm_fp4.hpp"

namespace gemm355 {
namespace fp4 {

constexpr int DECODE_THREADS = 256;
constexpr int DECODE_MAX_BLOCKS = 8192;

// Two FP16 values -> two BF16 values (exact for the decoded set), packed.
__device__ inline unsigned bf16_pair(_Float16 lo, _Float16 hi)
{
    return (__builtin_bit_cast(unsigned, (float)lo) >> 16) | (__builtin_bit_cast(unsigned, (float)hi) & 0xFFFF0000u);
}

// rows x K operand (codes: rows x K/2 bytes, scales: rows x K/16 bytes, both
// row-major) -> rows x K BF16, row-major. K % 32 == 0; 16-byte aligned codes
// and output, 2-byte aligned scales.
struct DecodeArgs {
    const uint8_t *q, *sf;
    uint16_t *out;
    int rows, K;
};

__global__ __launch_bounds__(DECODE_THREADS) void decode_nvfp4_bf16_kernel(DecodeArgs a)
{
    const uint8_t *q = a.q, *sf = a.sf;
    uint16_t *out = a.out;
    const int rows = a.rows, K = a.K;
    const int per_row = K / 32;
    const long long total = (long long)rows * per_row;
    for (long long c = (long long)blockIdx.x * DECODE_THREADS + threadIdx.x; c < total;
         c += (long long)gridDim.x * DECODE_THREADS) {
        const int row = (int)(c / per_row), j = (int)(c - (long long)row * per_row);
        const u32x4 codes = *reinterpret_cast<const u32x4 *>(q + (size_t)row * (K / 2) + 16 * j);
        const unsigned s = *reinterpret_cast<const uint16_t *>(sf + (size_t)row * (K / 16) + 2 * j);
        const f16x2 sc = scales2(s);
        u32x4 *o = reinterpret_cast<u32x4 *>(out + (size_t)row * K + 32 * j);
        static_for<4>([&](auto dc) {
            constexpr int d = decltype(dc)::value;
            const f16x8 v = decode8(codes[d], scale2<d / 2>(sc));
            o[d] = u32x4{bf16_pair(v[0], v[1]), bf16_pair(v[2], v[3]), bf16_pair(v[4], v[5]), bf16_pair(v[6], v[7])};
        });
    }
}

} // namespace fp4
} // namespace gemm355
