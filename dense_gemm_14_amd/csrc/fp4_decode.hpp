// fp4_decode.hpp -- block-scaled FP4 operands ("NVFP4 GEMM on Blackwell",
// section "NVFP4 Datatype") decoded once into BF16 rows, for the decode-first
// path of gemm_nvfp4_nt_ws: the BF16 product then runs on the decoded
// operands.
//
// Why a second path beside the kernel that decodes while staging: there every
// 256 x 256 tile decodes its own A and B strips, so at M = N = K = 8192 each
// operand element is decoded 32 times, and writing the decoded values to LDS
// (64 KiB per workgroup and K step, beside 192 KiB of fragment reads) costs
// that kernel matrix-busy cycles the BF16 kernel, whose copies bypass the
// vector registers, does not lose. Decoding once costs a read of the codes and
// a write and re-read of 2 (M + N) K bytes of BF16 in HBM instead.
//
// Work is split into units of 512 consecutive elements of one row (256 code
// bytes, 32 scale bytes, 1 KiB of BF16): lane l of a wave decodes elements
// 8 l .. 8 l + 7 of a unit -- one code dword, its block's scale byte -- into
// 16 bytes at byte 16 l of the unit's output, so every load and store
// instruction of a wave covers one contiguous range (256, 32 and 1024 bytes).
// A wave takes whole rows (A's rows, then B's, as one sequence; one launch
// decodes both operands) and walks each row's units DECODE_UNROLL at a time,
// loads first, so no index division is needed. The decode is the staging
// kernel's (decode8, exact to FP16); FP16 -> BF16 is then exact as well
// (every decoded value has at most 6 significant bits and lies in
// [2^-10, 2688]), by way of FP32 and its top 16 bits. A row's last unit may
// be partial (K % 512 != 0): lanes past K neither load nor store.
#pragma once

#include "gemm_fp4.hpp"

namespace gemm355 {
namespace fp4 {

constexpr int DECODE_THREADS = 256;
constexpr int DECODE_WAVES = DECODE_THREADS / 64;
constexpr int DECODE_UNROLL = 4;
constexpr int DECODE_MAX_BLOCKS = 2048;

// Two FP16 values -> two BF16 values (exact for the decoded set), packed.
__device__ inline unsigned bf16_pair(_Float16 lo, _Float16 hi)
{
    return (__builtin_bit_cast(unsigned, (float)lo) >> 16) | (__builtin_bit_cast(unsigned, (float)hi) & 0xFFFF0000u);
}

// Operand o (0 = A, 1 = B): rows x K codes (rows x K/2 bytes) and scales
// (rows x K/16 bytes), row-major, into rows x K BF16, row-major. K % 32 == 0;
// codes 4-byte aligned, output 16-byte aligned.
struct DecodeArgs {
    const uint8_t *q[2], *sf[2];
    uint16_t *out[2];
    int rows[2];
    int K;
};

__global__ __launch_bounds__(DECODE_THREADS) void decode_nvfp4_bf16_kernel(DecodeArgs a)
{
    const int K = a.K;
    const int lane = threadIdx.x & 63;
    const int rows = a.rows[0] + a.rows[1];
    const int waves = (int)gridDim.x * DECODE_WAVES;
    const int first = (int)blockIdx.x * DECODE_WAVES + __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    for (int r = first; r < rows; r += waves) {
        const int o = r < a.rows[0] ? 0 : 1;
        const int row = o ? r - a.rows[0] : r;
        const uint8_t *q = a.q[o] + (size_t)row * (K / 2);
        const uint8_t *sf = a.sf[o] + (size_t)row * (K / 16);
        uint16_t *out = a.out[o] + (size_t)row * K;
        for (int e = 8 * lane; e - 8 * lane < K; e += DECODE_UNROLL * 512) {
            unsigned codes[DECODE_UNROLL], sfb[DECODE_UNROLL];
#pragma unroll
            for (int j = 0; j < DECODE_UNROLL; ++j) {
                const int e0 = e + 512 * j;
                if (e0 < K) {
                    codes[j] = *reinterpret_cast<const unsigned *>(q + e0 / 2);
                    sfb[j] = sf[e0 / 16];
                }
            }
#pragma unroll
            for (int j = 0; j < DECODE_UNROLL; ++j) {
                const int e0 = e + 512 * j;
                if (e0 < K) {
                    const f16x8 v = decode8(codes[j], scale2<0>(scales2(sfb[j])));
                    *reinterpret_cast<u32x4 *>(out + e0) =
                        u32x4{bf16_pair(v[0], v[1]), bf16_pair(v[2], v[3]), bf16_pair(v[4], v[5]), bf16_pair(v[6], v[7])};
                }
            }
        }
    }
}

} // namespace fp4
} // namespace gemm355
