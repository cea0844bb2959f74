// gemm_fp4.hpp -- persistent block-scaled FP4 NT GEMM for gfx950.
//
// The operands are E2M1 codes (two per byte, even k in the low nibble) with
// one E4M3 scale per 16 consecutive K elements of a row ("NVFP4 GEMM on
// Blackwell", section "NVFP4 Datatype"). They are decoded exactly to FP16
// while being staged into LDS, so the matrix-core loop is the ordinary FP16
// one (v_mfma_f32_32x32x16_f16, same rate as BF16).
//
// Work decomposition
//   * Output tile 256 x 256 per workgroup, 4 waves in a 2 x 2 layout, each
//     wave owning a 128 x 128 block = 4 x 4 MFMA blocks of 32 x 32 whose FP32
//     accumulators (256 per lane) live in the accumulation registers.
//   * K advances 64 at a time through a 2-stage LDS ring (2 x 64 KiB): while
//     the matrix cores work on stage s, the next K slice sitting in registers
//     (codes and scales, 18 registers per lane) is decoded and written into
//     stage s^1, and the slice after it is requested from memory. One
//     workgroup barrier per K step separates reuse of a stage.
//   * LDS rows are 128 bytes (64 FP16 values); the 16-byte chunk c of row r is
//     stored at chunk position c ^ ((r >> 1) & 7). gfx950's LDS serves a
//     ds_read_b128 16 lanes (256 bytes, 64 banks of 4 bytes) per cycle; the 16
//     consecutive rows one such group reads at the same logical chunk then
//     cover all 16 bank groups (row parity picks the 128-byte half of the bank
//     space, (r >> 1) & 7 the chunk within it), so the reads are conflict-free.
#pragma once

#include "common.hpp"

namespace gemm355 {
namespace fp4 {

constexpr int BK = 64;                       // K elements per pipeline step
constexpr int ROW_BYTES = BK * 2;            // one LDS tile row: 64 x FP16
constexpr int TILE_BYTES = BM * ROW_BYTES;   // 32 KiB per operand per stage
constexpr int STAGE_BYTES = 2 * TILE_BYTES;  // A tile then B tile
constexpr int STAGES = 2;
constexpr int LDS_BYTES = STAGES * STAGE_BYTES;

// Physical 16-byte chunk position of logical chunk `chunk` in LDS tile row `row`.
__device__ inline int swizzle(int row, int chunk)
{
    return chunk ^ ((row >> 1) & 7);
}

// ---- block-scaled FP4 operands ---------------------------------------------
//
// Thread t stages row t of the A tile and row t of the B tile: per K step of
// 64 elements that is 32 bytes of packed codes and 4 scale bytes per row.
// Decoding ("NVFP4 GEMM on Blackwell", section "NVFP4 Datatype"): each code
// pair converts to two FP16 E2M1 values (v_cvt_scalef32_pk_f16_fp4 with a unit
// scale), then one packed FP16 multiply applies the E4M3 scale of its 16-element
// block. Both steps are exact: an E4M3 value and every product e2m1 * e4m3
// lie in FP16's normal range with at most 6 significant bits. (gfx950's scaled
// FP4 conversion applies only the exponent of its scale operand, which is why
// the E4M3 mantissa goes through the multiply, and FP16 rather than BF16 is
// used because gfx950 has a packed FP16 multiply but no packed BF16 one; the
// FP16 and BF16 matrix instructions have the same rate.)
struct Fp4Staging {
    typedef f16x8 frag;
    __amdgpu_buffer_rsrc_t ra, rb, rsa, rsb;
    int a_code_off, b_code_off, a_sf_off, b_sf_off;
    int lds_off;
    int K;
    u32x4 a_code[2], b_code[2];
    unsigned a_sf, b_sf;

    __device__ void init(const Problem &p, int tm, int tn, int tid)
    {
        const unsigned kc = (unsigned)p.K / 2, ks = (unsigned)p.K / 16;
        K = p.K;
        ra = make_rsrc(p.a, (unsigned)p.M * kc);
        rb = make_rsrc(p.b, (unsigned)p.N * kc);
        rsa = make_rsrc(p.sfa, (unsigned)p.M * ks);
        rsb = make_rsrc(p.sfb, (unsigned)p.N * ks);
        a_code_off = (tm * BM + tid) * (int)kc;
        b_code_off = (tn * BN + tid) * (int)kc;
        a_sf_off = (tm * BM + tid) * (int)ks;
        b_sf_off = (tn * BN + tid) * (int)ks;
        lds_off = tid * ROW_BYTES;
    }

    __device__ void load(int k0)
    {
        // K % 64 == 0: every step is whole; a step at or past K reads zeros
        const bool valid = k0 < K;
        const int oc = k0 / 2, os = k0 / 16;
        const int ac = valid ? a_code_off + oc : OOB, bc = valid ? b_code_off + oc : OOB;
        a_code[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, ac, 0, 0));
        a_code[1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, ac + 16, 0, 0));
        b_code[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, bc, 0, 0));
        b_code[1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, bc + 16, 0, 0));
        a_sf = __builtin_amdgcn_raw_buffer_load_b32(rsa, valid ? a_sf_off + os : OOB, 0, 0);
        b_sf = __builtin_amdgcn_raw_buffer_load_b32(rsb, valid ? b_sf_off + os : OOB, 0, 0);
    }

    // 8 codes (one dword) scaled by `s` -> 8 FP16 values.
    static __device__ f16x8 decode8(unsigned codes, f16x2 s)
    {
        f16x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * s;
        f16x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * s;
        f16x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * s;
        f16x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * s;
        f16x8 r = {v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
        return r;
    }

    // Scale block BLK (elements 16 BLK .. 16 BLK + 15 of the step) of one row.
    template <int BLK>
    static __device__ void decode_block(uint8_t *row_base, int row, const u32x4 *code, unsigned sf)
    {
        const _Float16 s = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)sf, BLK); // exact
        const f16x2 s2 = {s, s};
#pragma unroll
        for (int h = 0; h < 2; ++h) {                    // two dwords = 16 elements
            const int d = BLK * 2 + h;                   // 16-byte chunk d of the row
            const unsigned codes = code[d >> 2][d & 3];
            *reinterpret_cast<f16x8 *>(row_base + (swizzle(row, d) << 4)) = decode8(codes, s2);
        }
    }

    static __device__ void decode_row(uint8_t *row_base, int row, const u32x4 *code, unsigned sf)
    {
        decode_block<0>(row_base, row, code, sf);
        decode_block<1>(row_base, row, code, sf);
        decode_block<2>(row_base, row, code, sf);
        decode_block<3>(row_base, row, code, sf);
    }

    __device__ void commit(uint8_t *stage)
    {
        const int row = lds_off / ROW_BYTES;
        decode_row(stage + lds_off, row, a_code, a_sf);
        decode_row(stage + TILE_BYTES + lds_off, row, b_code, b_sf);
    }

    static __device__ f32x16 mma(frag s0, frag s1, f32x16 acc)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(s0, s1, acc, 0, 0, 0);
    }

    // Sub-step 1: 16 matrix instructions, 8 fragment reads, the decode
    // (vector ALU) and 16 LDS writes of the next slice.
    static __device__ void schedule_commit()
    {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            SCHED(SG_MFMA, 1);
            SCHED(SG_DS_READ, 1);
            SCHED(SG_VALU, 9);
            SCHED(SG_DS_WRITE, 1);
            SCHED(SG_MFMA, 1);
            SCHED(SG_VALU, 9);
            SCHED(SG_DS_WRITE, 1);
        }
    }

    // Sub-step 2: 16 matrix instructions, 8 fragment reads, the 6 global
    // reads of the slice after next.
    static __device__ void schedule_load()
    {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            SCHED(SG_MFMA, 1);
            SCHED(SG_DS_READ, 1);
            SCHED(SG_VMEM_READ, 1);
            SCHED(SG_MFMA, 1);
        }
    }
};

// ---- the persistent kernel --------------------------------------------------

__global__ __attribute__((amdgpu_flat_work_group_size(THREADS, THREADS), amdgpu_waves_per_eu(1, 1)))
void gemm_nvfp4_nt_kernel(Problem p)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
    typedef Fp4Staging Staging;
    typedef Staging::frag frag;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave & 1;   // wave's 128-row half of the tile (A rows)
    const int wn = wave >> 1;  // wave's 128-column half (B rows)
    const int l32 = lane & 31;
    const int half = lane >> 5;

    // Per-lane LDS fragment addresses: row (l32 + 32 i) of the wave's block,
    // logical chunk (2 kk + half) for K sub-step kk of 16 elements.
    const int a_row = (wm * 128 + l32) * ROW_BYTES;
    const int b_row = TILE_BYTES + (wn * 128 + l32) * ROW_BYTES;
    int kofs[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        kofs[kk] = swizzle(l32, 2 * kk + half) << 4;   // rows differ from l32 by multiples of 32

    const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.c, (unsigned)p.M * (unsigned)p.N * 2u);
    const int nk = (p.K + BK - 1) / BK;

    auto read_frags = [&](const uint8_t *stage, int kk, frag *fa, frag *fb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            fa[i] = *reinterpret_cast<const frag *>(stage + a_row + i * 32 * ROW_BYTES + kofs[kk]);
            fb[i] = *reinterpret_cast<const frag *>(stage + b_row + i * 32 * ROW_BYTES + kofs[kk]);
        }
    };

    for (int round = 0;; ++round) {
        const int pos = schedule_position(blockIdx.x, round, p.grid);
        if (pos >= p.tiles)
            break;
        int tm, tn;
        supergroup_tile(pos, p.tiles_m, p.tiles_n, p.supergroup, tm, tn);

        f32x16 acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = f32x16{};

        auto mma_all = [&](const frag *fa, const frag *fb) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = Staging::mma(fb[j], fa[i], acc[i][j]);
        };

        Staging st;
        st.init(p, tm, tn, tid);
        frag fa0[4], fb0[4], fa1[4], fb1[4];
        st.load(0);
        lds_barrier();            // every wave is done with the previous tile's stages
        st.commit(lds);
        st.load(BK);
        lds_barrier();
        read_frags(lds, 0, fa0, fb0);

        // Software pipeline over K steps. Step kt computes on LDS stage kt & 1
        // in four sub-steps of 16; each sub-step's fragments were read from LDS
        // during the previous sub-step's matrix instructions. Along the way the
        // step writes the registers holding slice kt + 1 into the other stage,
        // requests slice kt + 2 from memory, and -- after the step's single
        // barrier -- reads the first fragments of the other stage. The body has
        // no branches, so the compiler can interleave all of it with the matrix
        // instructions; slices at or past K load as zeros and are never used.
        for (int kt = 0; kt < nk; ++kt) {
            const uint8_t *cur = lds + (kt & 1) * STAGE_BYTES;
            uint8_t *nxt = lds + ((kt + 1) & 1) * STAGE_BYTES;

            read_frags(cur, 1, fa1, fb1);
            mma_all(fa0, fb0);
            schedule_reads_with_mma();
            SCHED_FENCE();

            read_frags(cur, 2, fa0, fb0);
            st.commit(nxt);
            mma_all(fa1, fb1);
            Staging::schedule_commit();
            SCHED_FENCE();

            read_frags(cur, 3, fa1, fb1);
            st.load((kt + 2) * BK);
            mma_all(fa0, fb0);
            Staging::schedule_load();
            SCHED_FENCE();

            // every wave is done reading stage `nxt` (last step) and writing it (this step)
            lds_barrier();
            SCHED_FENCE();
            read_frags(nxt, 0, fa0, fb0);
            mma_all(fa1, fb1);
            schedule_reads_with_mma();
            SCHED_FENCE();
        }

        store_tile(acc, rc, p.M, p.N, tm * BM + wm * 128, tn * BN + wn * 128, l32, half);
    }
}

} // namespace fp4
} // namespace gemm355
