// gemm355.hip -- host side of libgemm355: argument checks, grid sizing and
// launches of the gfx950 kernels in gemm_bf16.hpp and gemm_fp4.hpp. The C ABI
// is declared in include/gemm355.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <stdint.h>

#include "gemm355.h"
#include "gemm_bf16.hpp"
#include "gemm_bf16_small.hpp"
#include "gemm_fp4.hpp"
#include "schedule.hpp"

namespace {

using gemm355::BM;
using gemm355::BN;
using gemm355::Problem;

constexpr int kMaxDevices = 64;
constexpr int kSupergroup = 8; // adjacent N tiles per band of the visiting order

// BF16 kernel instance: 0 = chosen by shape, 1 = 256 x 256 tiles, 2 = 64 x 64
// tiles (set through gemm355_force_instance, for tests and measurements).
std::atomic<int> g_bf16_instance{0};

// The 256 x 256 kernel needs enough tiles to occupy the compute units; below
// half of them (128 tiles) the 64 x 64 kernel streams the operands faster.
constexpr int64_t kSmallTileThreshold = 128;

std::mutex g_cu_lock;
int g_cu_count[kMaxDevices];   // 0 = not queried yet

// Compute units of the current device, queried once per device.
int compute_units(int *cus)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return GEMM355_ERR_NO_DEVICE;
    std::lock_guard<std::mutex> guard(g_cu_lock);
    if (g_cu_count[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            return GEMM355_ERR_NO_DEVICE;
        g_cu_count[dev] = n;
    }
    *cus = g_cu_count[dev];
    return GEMM355_OK;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlaps(const void *p, size_t pn, const void *q, size_t qn)
{
    if (!p || !q || pn == 0 || qn == 0)
        return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
    return a < b + qn && b < a + pn;
}

// Byte extent of `rows` rows (rounded up to whole 256-row tiles) of `row_bytes`
// each must stay below 2^31: the kernels address operands with 32-bit offsets.
bool extent_ok(int64_t rows, int64_t row_bytes)
{
    const int64_t padded = (rows + 255) / 256 * 256;
    return padded * row_bytes < (int64_t(1) << 31);
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

template <class Kernel>
int launch(Kernel kernel, Problem p, void *stream, int tile_m = BM, int tile_n = BN)
{
    int cus = 0;
    const int rc = compute_units(&cus);
    if (rc != GEMM355_OK)
        return rc;
    p.tiles_m = (int)ceil_div(p.M, tile_m);
    p.tiles_n = (int)ceil_div(p.N, tile_n);
    p.tiles = p.tiles_m * p.tiles_n;
    p.supergroup = kSupergroup;
    p.grid = gemm355::persistent_grid(p.tiles, cus);
    (void)hipGetLastError(); // clear a stale error so the check below is ours
    hipLaunchKernelGGL(kernel, dim3(p.grid), dim3(gemm355::THREADS), 0, static_cast<hipStream_t>(stream), p);
    return hipGetLastError() == hipSuccess ? GEMM355_OK : GEMM355_ERR_LAUNCH;
}

} // namespace

extern "C" int gemm_bf16_nt(int M, int N, int K, const void *A, const void *B, void *C, void *stream)
{
    if (M < 0 || N < 0 || K < 0)
        return GEMM355_ERR_INVALID_ARG;
    if (M == 0 || N == 0)
        return GEMM355_OK;
    if (!C || (K > 0 && (!A || !B)))
        return GEMM355_ERR_INVALID_ARG;
    const size_t c_bytes = size_t(M) * size_t(N) * 2;
    if (K > 0 && (overlaps(C, c_bytes, A, size_t(M) * K * 2) || overlaps(C, c_bytes, B, size_t(N) * K * 2)))
        return GEMM355_ERR_INVALID_ARG;
    if (!aligned(A, 16) || !aligned(B, 16) || !aligned(C, 16))
        return GEMM355_ERR_UNSUPPORTED;
    if (K % 8 != 0 || N % 8 != 0)
        return GEMM355_ERR_UNSUPPORTED;
    if (!extent_ok(M, int64_t(K) * 2) || !extent_ok(N, int64_t(K) * 2) || !extent_ok(M, int64_t(N) * 2))
        return GEMM355_ERR_UNSUPPORTED;

    Problem p = {};
    p.a = A;
    p.b = B;
    p.c = C;
    p.M = M;
    p.N = N;
    p.K = K;
    int instance = g_bf16_instance.load(std::memory_order_relaxed);
    if (instance == 0)
        instance = ceil_div(M, BM) * ceil_div(N, BN) < kSmallTileThreshold ? 2 : 1;
    if (K <= 3 * gemm355::bf16::BK)
        instance = 2;   // the 256 x 256 kernel runs its tiles back to back and needs K > 192
    if (instance == 2)
        return launch(gemm355::bf16_small::gemm_bf16_nt_small_kernel, p, stream, gemm355::bf16_small::TM,
                      gemm355::bf16_small::TN);
    return launch(gemm355::bf16::gemm_bf16_nt_kernel, p, stream);
}

extern "C" int gemm355_force_instance(int instance)
{
    if (instance < 0 || instance > 2)
        return GEMM355_ERR_INVALID_ARG;
    g_bf16_instance.store(instance, std::memory_order_relaxed);
    return GEMM355_OK;
}

extern "C" int gemm_nvfp4_nt(int M, int N, int K, const void *Aq, const void *SFA, const void *Bq,
                             const void *SFB, void *C, void *stream)
{
    if (M < 0 || N < 0 || K < 0)
        return GEMM355_ERR_INVALID_ARG;
    if (M == 0 || N == 0)
        return GEMM355_OK;
    if (!C || (K > 0 && (!Aq || !SFA || !Bq || !SFB)))
        return GEMM355_ERR_INVALID_ARG;
    const size_t c_bytes = size_t(M) * size_t(N) * 2;
    if (K > 0 && (overlaps(C, c_bytes, Aq, size_t(M) * K / 2) || overlaps(C, c_bytes, Bq, size_t(N) * K / 2) ||
                  overlaps(C, c_bytes, SFA, size_t(M) * K / 16) || overlaps(C, c_bytes, SFB, size_t(N) * K / 16)))
        return GEMM355_ERR_INVALID_ARG;
    if (!aligned(Aq, 16) || !aligned(Bq, 16) || !aligned(C, 16) || !aligned(SFA, 4) || !aligned(SFB, 4))
        return GEMM355_ERR_UNSUPPORTED;
    if (K % 64 != 0 || N % 8 != 0)
        return GEMM355_ERR_UNSUPPORTED;
    if (!extent_ok(M, int64_t(K) / 2) || !extent_ok(N, int64_t(K) / 2) || !extent_ok(M, int64_t(N) * 2))
        return GEMM355_ERR_UNSUPPORTED;

    Problem p = {};
    p.a = Aq;
    p.b = Bq;
    p.sfa = SFA;
    p.sfb = SFB;
    p.c = C;
    p.M = M;
    p.N = N;
    p.K = K;
    return launch(gemm355::fp4::gemm_nvfp4_nt_kernel, p, stream);
}

extern "C" const char *gemm355_status_string(int status)
{
    switch (status) {
    case GEMM355_OK:
        return "ok";
    case GEMM355_ERR_INVALID_ARG:
        return "invalid argument (negative size, NULL pointer or overlapping output)";
    case GEMM355_ERR_UNSUPPORTED:
        return "unsupported (alignment, K or N granularity, or operand extent)";
    case GEMM355_ERR_NO_DEVICE:
        return "no usable HIP device";
    case GEMM355_ERR_LAUNCH:
        return "kernel launch failed";
    default:
        return "unknown status";
    }
}

extern "C" int gemm355_tile_order(int tiles_m, int tiles_n, int supergroup, int *tm, int *tn)
{
    if (tiles_m <= 0 || tiles_n <= 0 || supergroup <= 0 || !tm || !tn)
        return GEMM355_ERR_INVALID_ARG;
    const int64_t total = int64_t(tiles_m) * tiles_n;
    if (total > (int64_t(1) << 30))
        return GEMM355_ERR_INVALID_ARG;
    for (int pos = 0; pos < (int)total; ++pos)
        gemm355::supergroup_tile(pos, tiles_m, tiles_n, supergroup, tm[pos], tn[pos]);
    return GEMM355_OK;
}

extern "C" int gemm355_schedule(int tiles, int grid, int *slot, int slot_len)
{
    if (tiles <= 0 || grid <= 0 || !slot)
        return -GEMM355_ERR_INVALID_ARG;
    const int rounds = (int)ceil_div(tiles, grid);
    if (int64_t(rounds) * grid > slot_len)
        return -GEMM355_ERR_INVALID_ARG;
    for (int w = 0; w < grid; ++w)
        for (int r = 0; r < rounds; ++r) {
            const int pos = gemm355::schedule_position(w, r, grid);
            slot[w * rounds + r] = pos < tiles ? pos : -1;
        }
    return rounds;
}
