// gemm_bf16_splitk.hpp -- BF16 NT GEMM for gfx950 on skinny problems (few
// output tiles, long K, e.g. M = 128 against N = K = 8192), as two kernels:
// 128 x 128 output tiles whose K range is split over several workgroups, each
// writing an FP32 partial tile, then a reduction that adds the partials of
// every output element in split order and rounds once to BF16.
//
// Why: such a problem is bound by operand traffic. With one workgroup per
// 64 x 64 tile every compute unit streams 64 rows of A and 64 rows of B over
// the whole K (2 MiB at M = 128, N = K = 8192), which is the per-unit copy
// engine's limit, not the memory's. A 128 x 128 tile over a quarter of K moves
// half as much per unit (128 + 128 rows x K / 4) for the same multiply-adds;
// the partials cost 64 KiB per workgroup.
//
//   * 8 waves in 2 x 4 (two per SIMD), each wave 64 x 32 = 4 x 2 blocks of
//     v_mfma_f32_16x16x32_bf16 (32 accumulation registers per lane). Eight
//     waves rather than four because the transfer is the bound and more
//     waves issuing copies move more: a probe streaming these tiles' operand
//     traffic alone (LDS-DMA, split 4 of 128 x 8192 x 8192) takes 34.2 us
//     with 4 waves and 28.5 us with 8.
//   * K advances 64 per step; a unit is the A tile or the B tile of one step
//     (128 rows of 128 bytes, same chunk swizzle as the other BF16 kernels,
//     16 KiB). LDS holds a ring of 3 A units and a ring of 7 B units. Waves 0
//     to 3 copy A rows 32 w .. 32 w + 31, waves 4 to 7 the same rows of B
//     (four 1 KiB LDS-DMA copies per wave and step under one m0, through the
//     instruction offset), so B, which streams from HBM, is requested five
//     steps ahead and A, which stays in L2, one step ahead.
//   * Step s: copy step s + stages - 1 of the wave's operand into the slot of
//     step s - 1 (read by every wave before the previous barrier), wait until
//     this wave's copies of step s + 1 have landed, one barrier, then the 16
//     matrix instructions of step s on fragments read during step s - 1, with
//     the 12 fragment reads of step s + 1 interleaved.
//   * The result is deterministic: each split sums its K range in a fixed
//     order and the reduction adds the splits in index order.
#pragma once

#include "common.hpp"

#include <utility>

namespace gemm355 {
namespace bf16_splitk {

constexpr int TM = 128;                      // output tile rows
constexpr int TN = 128;                      // output tile columns
constexpr int BK = 64;                       // K elements per step
constexpr int ROW_BYTES = BK * 2;            // 128-byte LDS rows
constexpr int A_UNIT = TM * ROW_BYTES;       // A tile of one step: 16 KiB
constexpr int B_UNIT = TN * ROW_BYTES;       // B tile of one step: 16 KiB
constexpr int A_STAGES = 3;                  // A ring (its rows come from L2): one step ahead
constexpr int B_STAGES = 7;                  // B ring (its rows stream from HBM): five steps ahead
constexpr int LDS_BYTES = A_STAGES * A_UNIT + B_STAGES * B_UNIT;
constexpr int COPIES = 4;                    // 1 KiB copies per wave per step
constexpr int THREADS_SK = 512;              // 8 waves, two per SIMD
constexpr int TILE_FLOATS = TM * TN;         // one partial tile
constexpr int MAX_SPLITS = 8;
constexpr int REDUCE_THREADS = 256;

static_assert(LDS_BYTES <= 163840, "LDS rings exceed the 160 KiB of a gfx950 workgroup");
static_assert(TM == 128 && TN == 128 && THREADS_SK == 512, "the copy map assumes 128 x 128 tiles and 8 waves");
static_assert(COPIES * (B_STAGES - 1) <= 63, "vmcnt counts at most 63 outstanding operations");

// Kernel arguments. Work item w = tile * splits + split; tile = tm * tiles_n + tn.
struct SplitProblem {
    const void *a, *b;
    float *ws;          // partial tiles, [tiles][splits][TM][TN] FP32, row-major (unused with one split)
    void *c;
    const void *bias;   // fused epilogue only: N BF16 values, or NULL (zeros)
    int M, N, K;
    int tiles_m, tiles_n;
    int splits;
    int steps_per_split;   // K steps of 64 per split (the last split may have fewer)
};

__device__ inline int swizzle(int r, int c) { return c ^ ((r >> 1) & 7); }

typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ inline i32x4 rsrc_words(const void *p, unsigned bytes)
{
    const unsigned long long a = reinterpret_cast<unsigned long long>(p);
    return i32x4{(int)(unsigned)a, (int)(unsigned)(a >> 32), (int)bytes, (int)RSRC_WORD3};
}

// The instruction offset of a copy moves both its global address and its LDS
// destination; the resources start SHIFT bytes early so the per-lane offset
// (global offset + SHIFT - instruction offset) is never negative, and
// OOB_SHIFTED stays past every range after any instruction offset.
constexpr int SHIFT = 3072;
constexpr unsigned OOB_SHIFTED = 0xFFFF0000u;

// Four 1 KiB global -> LDS copies under one m0: lane i's 16 bytes at buffer
// offset v_t + 1024 t land at LDS byte lds_addr + 1024 t + 16 i. Inline
// assembly so that the compiler does not order every later LDS read after the
// in-flight LDS writes; the kernel orders them with vmcnt waits and barriers.
// The s_nop: on gfx9 an LDS-DMA instruction must not directly follow a scalar
// write of m0 (one wait state).
__device__ inline void copy_four(const i32x4 &rsrc, unsigned lds_addr, unsigned v0, unsigned v1, unsigned v2,
                                 unsigned v3)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\t"
                 "buffer_load_dwordx4 %1, %5, 0 offen offset:0 lds\n\t"
                 "buffer_load_dwordx4 %2, %5, 0 offen offset:1024 lds\n\t"
                 "buffer_load_dwordx4 %3, %5, 0 offen offset:2048 lds\n\t"
                 "buffer_load_dwordx4 %4, %5, 0 offen offset:3072 lds"
                 :
                 : "s"(lds_addr), "v"(v0), "v"(v1), "v"(v2), "v"(v3), "s"(rsrc)
                 : "memory", "m0");
}

__device__ inline void wait_all_copies() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
template <int N>
__device__ inline void wait_copies_le() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }
__device__ inline void wait_reads() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Copy duty is split by operand: waves 0 to 3 copy the A tile (32 rows each)
// through a short ring, since the few A rows of a skinny problem stay in L2;
// waves 4 to 7 copy the B tile through a deep ring, since B streams from
// HBM, whose loaded latency is several microseconds: a wave's copies
// complete in issue order, so a wave copying both operands would wait for its
// older B copies whenever it waits for A, and B's prefetch depth would shrink
// to A's. LDS: A ring, then B ring; row r of a unit at byte 128 r.
// EPI: EPI_PLAIN, or the activation of the fused epilogue, applied here with
// one split (with several, by the reduction).
template <int EPI>
__global__ __attribute__((amdgpu_flat_work_group_size(THREADS_SK, THREADS_SK), amdgpu_waves_per_eu(2, 2)))
void gemm_bf16_nt_splitk_kernel(SplitProblem p)
{
    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];
    constexpr bool FUSED = EPI != EPI_PLAIN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1;   // 64-row half of the tile (A rows)
    const int wn = wave >> 1;  // 32-column quarter (B rows)
    const int l16 = lane & 15;
    const int grp = lane >> 4;
    const int K = p.K;
    const bool copies_b = wave >= 4;              // uniform per wave
    const int quarter = wave & 3;                 // which 32 rows of its operand this wave copies

    const int item = blockIdx.x;
    const int tile = item / p.splits;
    const int split = item - tile * p.splits;
    const int tm = tile / p.tiles_n;
    const int tn = tile - tm * p.tiles_n;
    const int nk = (K + BK - 1) / BK;
    const int k_first = split * p.steps_per_split;   // first global K step of this split
    const int rest = nk - k_first;
    const int steps = rest < p.steps_per_split ? (rest > 0 ? rest : 0) : p.steps_per_split;

    // Fragment of a 16-row block: row l16, logical chunk grp (first half of
    // the step) or 4 + grp (second half); blocks start at multiples of 16 rows.
    const int kofs[2] = {swizzle(l16, grp) << 4, swizzle(l16, 4 + grp) << 4};
    const int a_frag = (64 * wm + l16) * ROW_BYTES;
    const int b_frag = A_STAGES * A_UNIT + (32 * wn + l16) * ROW_BYTES;
    const int copy_row = lane >> 3;

    const unsigned lds_base = (unsigned)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)lds;
    const i32x4 rsrc = copies_b
        ? rsrc_words(static_cast<const uint8_t *>(p.b) - SHIFT, (unsigned)p.N * (unsigned)K * 2u + SHIFT)
        : rsrc_words(static_cast<const uint8_t *>(p.a) - SHIFT, (unsigned)p.M * (unsigned)K * 2u + SHIFT);
    const int stages = copies_b ? B_STAGES : A_STAGES;
    const unsigned ring = lds_base + (unsigned)(copies_b ? A_STAGES * A_UNIT : 0) + (unsigned)(quarter * 4096);

    // Copy t (0..3): rows 32 quarter + 8 t .. + 7 of this wave's operand tile;
    // lane i fills position i & 7 of row i / 8.
    unsigned off[COPIES];
    int chunk_k[2];
#pragma unroll
    for (int t = 0; t < COPIES; ++t) {
        const int row = 32 * quarter + 8 * t + copy_row;
        const int c = swizzle(row, lane & 7);
        if (t < 2)
            chunk_k[t] = 8 * c;   // depends on the block's parity only
        off[t] = (unsigned)((((copies_b ? tn * TN : tm * TM) + row) * K + 8 * c) * 2 + SHIFT - 1024 * (t & 3));
    }
    // This wave's eight copies of local step ls into its ring slot ls % stages;
    // steps past the split (or past K) and the K tail read as zeros, rows past
    // M or N fall outside the buffer and do too.
    auto copy_step = [&](int ls) {
        const int k0 = (k_first + ls) * BK;
        const bool in = ls < steps;
        const unsigned slot = ring + (unsigned)((ls % stages) * (copies_b ? B_UNIT : A_UNIT));
        unsigned v[COPIES];
#pragma unroll
        for (int t = 0; t < COPIES; ++t)
            v[t] = in && k0 + chunk_k[t & 1] < K ? off[t] + (unsigned)(k0 * 2) : OOB_SHIFTED;
        copy_four(rsrc, __builtin_amdgcn_readfirstlane(slot), v[0], v[1], v[2], v[3]);
    };
    // This wave's copies of the next step to be read have landed.
    auto wait_next = [&]() {
        if (copies_b)
            wait_copies_le<COPIES * (B_STAGES - 2)>();
        else
            wait_copies_le<COPIES * (A_STAGES - 2)>();
    };

    // fused epilogue with one split: bias[n .. n + 3] of this lane's columns
    // in block column j (requested before any copy, so landed by the first
    // step's wait; zeros past N and without a bias)
    u32x2 bias_w[2];
    if constexpr (FUSED) {
        const __amdgpu_buffer_rsrc_t rbias = make_rsrc(p.bias, p.bias && p.splits == 1 ? (unsigned)p.N * 2u : 0u);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = tn * TN + 32 * wn + 16 * j + 4 * grp;
            bias_w[j] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rbias, n < p.N ? n * 2 : OOB, 0, 0));
        }
    }

    f32x4 acc[4][2];
    bf16x8 fa[2][2][4], fb[2][2][2];   // [buffer][half][block]
    // Read q (0..11) of local step ls: half q / 6; A block q % 6 for q % 6 < 4,
    // else B block q % 6 - 4.
    auto read = [&](int ls, int buf, int q) {
        const int h = q / 6, r = q % 6, blk = r & 3;
        if (r < 4)
            fa[buf][h][blk] = *reinterpret_cast<const bf16x8 *>(lds + (ls % A_STAGES) * A_UNIT + a_frag +
                                                                blk * 16 * ROW_BYTES + kofs[h]);
        else
            fb[buf][h][r - 4] = *reinterpret_cast<const bf16x8 *>(lds + (ls % B_STAGES) * B_UNIT + b_frag +
                                                                  (r - 4) * 16 * ROW_BYTES + kofs[h]);
    };
    // Matrix instruction t (0..15): half t / 8, block ((t / 2) % 4, t % 2).
    // B rows are the first operand, so each 16 x 16 result arrives transposed
    // (lane (l16, grp) holds C[16 i + l16][16 j + 4 grp .. + 3]).
    auto mma = [&](int buf, int t, bool first) {
        const int h = t >> 3, i = (t >> 1) & 3, j = t & 1;
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[buf][h][j], fa[buf][h][i],
                                                           (first && h == 0) ? f32x4{} : acc[i][j], 0, 0, 0);
    };

    // Prologue: each copying wave fills all but one slot of its ring.
    for (int ls = 0; ls < stages - 1; ++ls)
        copy_step(ls);
    wait_next();
    lds_barrier();
#pragma unroll
    for (int q = 0; q < 12; ++q)
        read(0, 0, q);

    auto step = [&](int ls, auto buf_c, bool first) {
        constexpr int buf = decltype(buf_c)::value;
        // step ls + stages - 1 goes into the slot of step ls - 1, which every
        // wave finished reading before the previous barrier
        copy_step(ls + stages - 1);
        // this wave's reads of step ls and its copies of step ls + 1 are done
        wait_reads();
        wait_next();
        lds_barrier();
        SCHED_FENCE();
        static_for<16>([&](auto tc) {
            constexpr int t = decltype(tc)::value;
            mma(buf, t, first);
            if constexpr (t < 12)
                read(ls + 1, buf ^ 1, t);
            SCHED_VALU_ONLY();
        });
    };

    if (steps == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = f32x4{};
    } else {
        step(0, Int<0>{}, true);
        int ls = 1;
        for (; ls + 1 < steps; ls += 2) {
            step(ls, Int<1>{}, false);
            step(ls + 1, Int<0>{}, false);
        }
        if (ls < steps)
            step(ls, Int<1>{}, false);
    }

    // Lane (l16, grp) of block (i, j) holds row 64 wm + 16 i + l16, columns
    // 32 wn + 16 j + 4 grp .. + 3 of the tile.
    if (p.splits == 1) {
        // One split: the tile is final; round to BF16 and store it into C
        // (8 bytes per lane and block; rows past M and columns past N masked,
        // N % 8 == 0 so a lane's 4 columns are all inside or all outside).
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.c, (unsigned)p.M * (unsigned)p.N * 2u);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int m = tm * TM + 64 * wm + 16 * i + l16, n = tn * TN + 32 * wn + 16 * j + 4 * grp;
                const int off = (m < p.M && n < p.N) ? (m * p.N + n) * 2 : OOB;
                f32x4 x = acc[i][j];
                if constexpr (FUSED)
                    x = epilogue4<EPI>(x, bias_w[j]);
                const u32x2 v = {pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])};
                __builtin_amdgcn_raw_buffer_store_b64(v, rc, off, 0, 0);
            }
    } else {
        const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.ws + (size_t)item * TILE_FLOATS, TILE_FLOATS * 4u);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int r = 64 * wm + 16 * i + l16, c = 32 * wn + 16 * j + 4 * grp;
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[i][j]), rw, (r * TN + c) * 4, 0, 0);
            }
    }
    wait_reads();
    wait_all_copies(); // no copy may still be writing LDS when the workgroup ends
}

// C[m][n .. n + 7] = bf16_rne(sum over splits z = 0, 1, ... of the partials),
// one thread per 8 consecutive outputs of a row (N % 8 == 0); with the fused
// epilogue (EPI an activation) applied to the sum before rounding.
template <int EPI>
__global__ __launch_bounds__(REDUCE_THREADS) void splitk_reduce_kernel(SplitProblem p)
{
    const int per_row = p.N / 8;
    const long long g = (long long)blockIdx.x * REDUCE_THREADS + threadIdx.x;
    if (g >= (long long)p.M * per_row)
        return;
    const int m = (int)(g / per_row);
    const int n = (int)(g - (long long)m * per_row) * 8;
    const int tile = (m / TM) * p.tiles_n + n / TN;
    const float *src = p.ws + (size_t)tile * p.splits * TILE_FLOATS + (m % TM) * TN + n % TN;
    f32x4 lo = {}, hi = {};
    for (int z = 0; z < p.splits; ++z) {
        lo += *reinterpret_cast<const f32x4 *>(src + (size_t)z * TILE_FLOATS);
        hi += *reinterpret_cast<const f32x4 *>(src + (size_t)z * TILE_FLOATS + 4);
    }
    if constexpr (EPI != EPI_PLAIN) {
        u32x4 b = {};
        if (p.bias)
            b = *reinterpret_cast<const u32x4 *>(static_cast<const uint8_t *>(p.bias) + (size_t)n * 2);
        lo = epilogue4<EPI>(lo, u32x2{b[0], b[1]});
        hi = epilogue4<EPI>(hi, u32x2{b[2], b[3]});
    }
    const u32x4 out = {pack_bf16(lo[0], lo[1]), pack_bf16(lo[2], lo[3]), pack_bf16(hi[0], hi[1]), pack_bf16(hi[2], hi[3])};
    *reinterpret_cast<u32x4 *>(static_cast<uint8_t *>(p.c) + ((size_t)m * p.N + n) * 2) = out;
}

} // namespace bf16_splitk
} // namespace gemm355
