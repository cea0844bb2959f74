// gemm355.hip -- host side of libgemm355: argument checks, instance plans,
// grid sizing and launches of the gfx950 kernels (gemm_bf16*.hpp,
// gemm_fp4.hpp, gemm_mxfp4.hpp). The C ABI is declared in include/gemm355.h.
// Nothing here allocates memory: the split-K partials live in a workspace the
// caller passes to the *_ws entry points.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <stdint.h>

#include "gemm355.h"
#include "gemm_bf16.hpp"
#include "gemm_bf16_small.hpp"
#include "gemm_bf16_small_long.hpp"
#include "gemm_bf16_splitk.hpp"
#include "gemm_mxfp4.hpp"
#include "gemm_fp4.hpp"
#include "fp4_decode.hpp"
#include "schedule.hpp"

// Scratch of gemm_bf16_nt_noalloc: the split-K partials of the largest plan
// on a 256-unit device (64 KiB per compute unit). Every GPU the library runs
// on holds its own copy until the process ends. In host code `scratch` names
// a host-side stand-in, never the device memory: the device address comes
// from hipGetSymbolAddress, once per device, and only that address is used.
static constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

namespace {

using gemm355::BM;
using gemm355::BN;
using gemm355::Problem;

constexpr int kMaxDevices = 64;
// Band width of the supergroup visiting order ("NVFP4 GEMM on Blackwell",
// "Production Kernel", "Supergroup Size"). One XCD's L2 (4 MB) serves the
// grid / 8 = 32 tiles its workgroups compute at once; a band of w adjacent N
// tiles makes those tiles a (32 / w) x w block, whose A and B strips number
// 32 / w + w: fewest (12) at w = 4 or 8, and the K steps of a strip are what
// each L2 re-serves. That decides whenever the tile's K loop is long. When it
// is short (K <= 1024: at most 16 steps) the C writes weigh as much as the
// operands, all of which fit in the 256 MB last-level cache, and a wide band
// keeps w tiles of the same C rows in flight, so C is written in runs of
// w x 512 bytes. Measured (256 x 256 tiles, min of round-robin passes):
//  * BF16 (27 shapes, M, N in {4096, 8192, 16384}, K in {1024, 4096, 16384})
//    and microscaled FP4: w = 16 is 4-6 % (BF16) and 6-16 % (FP4) faster than
//    8 when K <= 1024 with at least 64 tiles across N; elsewhere 8 is best or
//    within noise;
//  * NVFP4 (decode-bound, a prologue per tile): w = 16 is 3-15 % faster from
//    32 tiles across N when K <= 2048, and 1-2 % slower at 16 tiles.
enum Kernel { KERNEL_BF16 = 0, KERNEL_NVFP4 = 1, KERNEL_MXFP4 = 2, KERNEL_BF16_SMALL = 3 };
int supergroup_for(int kernel, int tiles_n, int K)
{
    if (kernel == KERNEL_NVFP4)
        return (K <= 2048 && tiles_n >= 32) ? 16 : 8;
    if (kernel == KERNEL_BF16 || kernel == KERNEL_MXFP4)
        return (K <= 1024 && tiles_n >= 64) ? 16 : 8;
    return 8;   // the 64 x 64 instance (few tiles; not ablated)
}

// Band width override for measurements (0 = supergroup_for); set through
// gemm355_force_supergroup.
std::atomic<int> g_supergroup{0};

// Tile order of the NVFP4 kernel: 0 static, 1 dynamic (a measurement option;
// set through gemm355_force_schedule).
std::atomic<int> g_schedule{0};
// gemm_nvfp4_nt_ws's path: 0 by shape, 1 always the staging-decode kernel,
// 2 always decode first (set through gemm355_force_fp4_path).
std::atomic<int> g_fp4_path{0};

// BF16 kernel instance: 0 = chosen by shape, 1 = 256 x 256 tiles, 2 = 64 x 64
// tiles, 3 = 128 x 128 tiles with split K (set through gemm355_force_instance,
// for tests and measurements).
std::atomic<int> g_bf16_instance{0};

// Instance choice for problems with fewer 256 x 256 tiles than half the
// compute units (with more, the 256 x 256 kernel was the fastest at every
// shape measured). The smaller instances are compared by an estimate of
// their time in microseconds: the busiest compute unit's K steps at the
// measured time of one step of its tile on a busy MI355X, or the operands
// (plus the split's partials) at a loaded HBM rate, whichever is longer, plus
// fixed costs, plus the split's reduction. The constants come from an
// ablation over M, N, K in {1024, 2048, 4096, 8192, 16384} and skinny shapes
// (M = 64 .. 512, N = 1024 .. 8192, K = 2048 .. 8192); only their ratios
// decide.
constexpr double kStep64 = 0.27;        // one K step of a 64 x 64 tile
constexpr double kStep128 = 0.56;       // one K step of a 128 x 128 tile (8 waves)
constexpr double kLaunchFixed = 3.0;    // prologue, epilogue, launch
constexpr double kReduceFixed = 3.0;    // the reduction's own launch
constexpr double kHbmBytesPerUs = 4.5e6;

std::mutex g_cu_lock;
int g_cu_count[kMaxDevices];   // 0 = not queried yet

void *g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device; guarded by g_cu_lock

// The device address of the current device's scratch array, looked up on the
// first call on that device (with that device current).
int scratch_address(void **ptr)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return GEMM355_ERR_NO_DEVICE;
    std::lock_guard<std::mutex> guard(g_cu_lock);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return GEMM355_ERR_NO_DEVICE;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return GEMM355_OK;
}

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

// One kernel launch on `stream`. The launch's own return code is the status:
// the thread's pending HIP error is neither read nor cleared, so an error the
// caller has not collected yet stays theirs.
template <class Kernel, class Args>
int launch_kernel(Kernel kernel, unsigned blocks, unsigned threads, Args &args, hipStream_t stream)
{
    void *argv[] = {&args};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(kernel), dim3(blocks), dim3(threads), argv,
                                         0, stream);
    return e == hipSuccess ? GEMM355_OK : GEMM355_ERR_LAUNCH;
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

// One launch of a persistent kernel on `stream`: tile counts for tile_m x
// tile_n output tiles, the supergroup width, a grid of at most one workgroup
// per compute unit, `threads` work-items per workgroup.
template <class KernelFn>
int launch(KernelFn kernel, int which, Problem p, void *stream, int tile_m = BM, int tile_n = BN,
           int threads = gemm355::THREADS)
{
    int cus = 0;
    const int rc = compute_units(&cus);
    if (rc != GEMM355_OK)
        return rc;
    p.tiles_m = (int)ceil_div(p.M, tile_m);
    p.tiles_n = (int)ceil_div(p.N, tile_n);
    p.tiles = p.tiles_m * p.tiles_n;
    const int sg = g_supergroup.load(std::memory_order_relaxed);
    p.supergroup = sg > 0 ? sg : supergroup_for(which, p.tiles_n, p.K);
    p.grid = gemm355::persistent_grid(p.tiles, cus);
    return launch_kernel(kernel, (unsigned)p.grid, (unsigned)threads, p, static_cast<hipStream_t>(stream));
}

// Split-K plan for 128 x 128 tiles: enough splits to give every compute unit a
// work item (at most max_splits), each split at least 8 K steps long.
void splitk_plan(int M, int N, int K, int cus, int max_splits, int *tiles_m, int *tiles_n, int *splits,
                 int *steps_per_split)
{
    namespace sk = gemm355::bf16_splitk;
    *tiles_m = (int)ceil_div(M, sk::TM);
    *tiles_n = (int)ceil_div(N, sk::TN);
    const int64_t tiles = int64_t(*tiles_m) * *tiles_n;
    const int nk = (int)ceil_div(K, sk::BK);
    int s = (int)std::max<int64_t>(1, cus / std::max<int64_t>(1, tiles));
    s = std::min(s, max_splits);
    s = std::max(1, std::min(s, nk / 8));
    const int per = (int)std::max<int64_t>(1, ceil_div(nk, s));
    *steps_per_split = per;
    *splits = std::max(1, (int)ceil_div(nk, per));   // no empty split
}

// Estimated time of the 64 x 64 instance (persistent, one workgroup per unit).
double estimate_small(int M, int N, int K, int cus)
{
    const int64_t tiles = ceil_div(M, 64) * ceil_div(N, 64);
    const int64_t grid = gemm355::persistent_grid((int)std::min<int64_t>(tiles, 1 << 30), cus);
    const double steps = double(ceil_div(tiles, grid)) * double(ceil_div(K, 64));
    const double operands = 2.0 * (double(M) * K + double(N) * K + double(M) * N);
    return std::max(steps * kStep64, operands / kHbmBytesPerUs) + kLaunchFixed;
}

// Estimated time of the 128 x 128 split-K instance (one workgroup per work
// item and unit), its reduction included when there is more than one split.
double estimate_split(int M, int N, int K, int cus, int tiles_m, int tiles_n, int splits, int per)
{
    const int64_t items = int64_t(tiles_m) * tiles_n * splits;
    const double steps = double(ceil_div(items, cus)) * per;
    const double operands = 2.0 * (double(M) * K + double(N) * K + double(M) * N);
    const double partials = splits > 1 ? 4.0 * double(M) * N * splits : 0.0;
    double t = std::max(steps * kStep128, (operands + partials) / kHbmBytesPerUs) + kLaunchFixed;
    if (splits > 1)
        t += kReduceFixed + (partials + 2.0 * double(M) * N) / kHbmBytesPerUs;
    return t;
}

// What a BF16 product runs: the instance (1 = 256 x 256, 2 = 64 x 64, 3 =
// 128 x 128 tiles with split K), the K splits of instance 3 and the workspace
// bytes its FP32 partials need (0 with one split).
struct Bf16Plan {
    int instance;
    int splits;
    size_t workspace_bytes;
};

// The plan for a problem (forced: 0 = by shape, else 1..3). Without a
// workspace (the entry points that take none) K is never split. Pure host
// arithmetic.
Bf16Plan plan_bf16(int M, int N, int K, int cus, int forced, bool with_workspace)
{
    namespace sk = gemm355::bf16_splitk;
    int tmn = 0, tnn = 0, per = 0, splits = 1;
    splitk_plan(M, N, K, cus, with_workspace ? sk::MAX_SPLITS : 1, &tmn, &tnn, &splits, &per);
    int instance = forced;
    if (instance == 0) {
        instance = 1;
        if (2 * ceil_div(M, BM) * ceil_div(N, BN) < cus)
            instance = estimate_small(M, N, K, cus) <= estimate_split(M, N, K, cus, tmn, tnn, splits, per) ? 2 : 3;
    }
    if (instance == 1 && K <= 3 * gemm355::bf16::BK)
        instance = 2;   // the 256 x 256 kernel runs its tiles back to back and needs K > 192
    if (instance != 3)
        splits = 1;
    const size_t ws = splits > 1 ? size_t(tmn) * size_t(tnn) * size_t(splits) * sk::TILE_FLOATS * sizeof(float) : 0;
    return {instance, splits, ws};
}

// Split-K instance: partial tiles into the caller's workspace, then the
// reduction into C, both on `stream`; with one split the tiles go straight to
// C and neither the workspace nor the reduction is used.
template <int EPI>
int launch_splitk(const Problem &p, const Bf16Plan &plan, void *workspace, void *stream)
{
    namespace sk = gemm355::bf16_splitk;
    int cus = 0;
    const int rc = compute_units(&cus);
    if (rc != GEMM355_OK)
        return rc;
    sk::SplitProblem sp = {};
    sp.a = p.a;
    sp.b = p.b;
    sp.c = p.c;
    sp.bias = p.bias;
    sp.M = p.M;
    sp.N = p.N;
    sp.K = p.K;
    splitk_plan(p.M, p.N, p.K, cus, plan.splits, &sp.tiles_m, &sp.tiles_n, &sp.splits, &sp.steps_per_split);
    const int64_t items = int64_t(sp.tiles_m) * sp.tiles_n * sp.splits;
    if (items > (int64_t(1) << 30))
        return GEMM355_ERR_UNSUPPORTED;
    if (sp.splits > 1)
        sp.ws = static_cast<float *>(workspace);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    int st = launch_kernel(sk::gemm_bf16_nt_splitk_kernel<EPI>, (unsigned)items, (unsigned)sk::THREADS_SK, sp, s);
    if (st == GEMM355_OK && sp.splits > 1) {   // one split stores C itself
        const int64_t outs = int64_t(p.M) * (p.N / 8);
        st = launch_kernel(sk::splitk_reduce_kernel<EPI>, (unsigned)ceil_div(outs, sk::REDUCE_THREADS),
                           (unsigned)sk::REDUCE_THREADS, sp, s);
    }
    return st;
}

// The 64 x 64 instance's B staging: 512-byte row segments (the _long kernel)
// for K >= 4096 with at least half the compute units' worth of tiles.
bool small_long_variant(int M, int N, int K, int cus)
{
    return K >= 4096 && 2 * ceil_div(M, 64) * ceil_div(N, 64) >= cus;
}

// The planned instance's kernels with epilogue EPI.
template <int EPI>
int launch_instance(const Bf16Plan &plan, const Problem &p, void *workspace, void *stream)
{
    int cus = 0;
    const int rc = compute_units(&cus);
    if (rc != GEMM355_OK)
        return rc;
    if (plan.instance == 3)
        return launch_splitk<EPI>(p, plan, workspace, stream);
    if (plan.instance == 2) {
        // B in 512-byte row segments where HBM streaming decides: long K and
        // at least half the units' worth of tiles (measured: 128 x 8192 x 8192
        // 42.2 -> 38.7 us; with 64 tiles or K <= 2048 the per-step kernel is
        // 3-10 % faster)
        if (small_long_variant(p.M, p.N, p.K, cus))
            return launch(gemm355::bf16_small_long::gemm_bf16_nt_small_long_kernel<EPI, 4>, KERNEL_BF16_SMALL, p,
                          stream, gemm355::bf16_small_long::TM, gemm355::bf16_small_long::TN);
        return launch(gemm355::bf16_small::gemm_bf16_nt_small_kernel<EPI>, KERNEL_BF16_SMALL, p, stream,
                      gemm355::bf16_small::TM, gemm355::bf16_small::TN);
    }
    if (p.K % gemm355::bf16::BK != 0)
        return launch(gemm355::bf16::gemm_bf16_nt_kernel<EPI, true>, KERNEL_BF16, p, stream);
    return launch(gemm355::bf16::gemm_bf16_nt_kernel<EPI, false>, KERNEL_BF16, p, stream);
}

// Shared by the BF16 entry points: validation, plan, launch. FUSED selects
// the kernels with the fused epilogue; WS the entry points that take a
// workspace (K may then be split; NULL with workspace_bytes 0 is allowed and
// rules splitting out only if the plan needs none); SCRATCH (with WS) uses
// the library's fixed scratch array as the workspace instead of the caller's.
template <bool FUSED, bool WS, bool SCRATCH = false>
int bf16_product(int M, int N, int K, const void *A, const void *B, const void *bias, int act, void *C,
                 void *workspace, size_t workspace_bytes, void *stream)
{
    if (M < 0 || N < 0 || K < 0)
        return GEMM355_ERR_INVALID_ARG;
    if (FUSED && (act < GEMM355_ACT_NONE || act > GEMM355_ACT_GELU_TANH))
        return GEMM355_ERR_INVALID_ARG;
    if (M == 0 || N == 0)
        return GEMM355_OK;
    if (!C || (K > 0 && (!A || !B)))
        return GEMM355_ERR_INVALID_ARG;
    const size_t c_bytes = size_t(M) * size_t(N) * 2;
    if (K > 0 && (overlaps(C, c_bytes, A, size_t(M) * K * 2) || overlaps(C, c_bytes, B, size_t(N) * K * 2)))
        return GEMM355_ERR_INVALID_ARG;
    if (FUSED && overlaps(C, c_bytes, bias, size_t(N) * 2))
        return GEMM355_ERR_INVALID_ARG;
    if (WS && workspace_bytes > 0 && !workspace)
        return GEMM355_ERR_INVALID_ARG;
    if (WS && (overlaps(workspace, workspace_bytes, C, c_bytes) ||
               (K > 0 && (overlaps(workspace, workspace_bytes, A, size_t(M) * K * 2) ||
                          overlaps(workspace, workspace_bytes, B, size_t(N) * K * 2))) ||
               (FUSED && overlaps(workspace, workspace_bytes, bias, size_t(N) * 2))))
        return GEMM355_ERR_INVALID_ARG;
    if (!aligned(A, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(bias, 16) || !aligned(workspace, 16))
        return GEMM355_ERR_UNSUPPORTED;
    if (K % 8 != 0 || N % 8 != 0)
        return GEMM355_ERR_UNSUPPORTED;
    if (!extent_ok(M, int64_t(K) * 2) || !extent_ok(N, int64_t(K) * 2) || !extent_ok(M, int64_t(N) * 2))
        return GEMM355_ERR_UNSUPPORTED;

    Problem p = {};
    p.a = A;
    p.b = B;
    p.c = C;
    p.bias = FUSED ? bias : nullptr;
    p.M = M;
    p.N = N;
    p.K = K;
    int cus = 0;
    const int rc = compute_units(&cus);
    if (rc != GEMM355_OK)
        return rc;
    const Bf16Plan plan = plan_bf16(M, N, K, cus, g_bf16_instance.load(std::memory_order_relaxed), WS);
    if (SCRATCH && plan.workspace_bytes > 0) {
        if (plan.workspace_bytes > kScratchBytes)
            return GEMM355_ERR_UNSUPPORTED;   // the plan's partials exceed the fixed scratch
        const int sr = scratch_address(&workspace);
        if (sr != GEMM355_OK)
            return sr;
        workspace_bytes = kScratchBytes;
    }
    if (plan.workspace_bytes > workspace_bytes)
        return GEMM355_ERR_UNSUPPORTED;   // the caller's workspace is smaller than the plan needs
    if (!FUSED)
        return launch_instance<gemm355::EPI_PLAIN>(plan, p, workspace, stream);
    if (act == GEMM355_ACT_RELU)
        return launch_instance<gemm355::ACT_RELU>(plan, p, workspace, stream);
    if (act == GEMM355_ACT_GELU_TANH)
        return launch_instance<gemm355::ACT_GELU_TANH>(plan, p, workspace, stream);
    return launch_instance<gemm355::ACT_NONE>(plan, p, workspace, stream);
}

} // namespace

extern "C" int gemm_bf16_nt(int M, int N, int K, const void *A, const void *B, void *C, void *stream)
{
    return bf16_product<false, false>(M, N, K, A, B, nullptr, GEMM355_ACT_NONE, C, nullptr, 0, stream);
}

extern "C" int gemm_bf16_nt_bias_act(int M, int N, int K, const void *A, const void *B, const void *bias,
                                     int activation, void *C, void *stream)
{
    return bf16_product<true, false>(M, N, K, A, B, bias, activation, C, nullptr, 0, stream);
}

extern "C" int gemm_bf16_nt_ws(int M, int N, int K, const void *A, const void *B, void *C, void *workspace,
                               size_t workspace_bytes, void *stream)
{
    return bf16_product<false, true>(M, N, K, A, B, nullptr, GEMM355_ACT_NONE, C, workspace, workspace_bytes,
                                     stream);
}

extern "C" int gemm_bf16_nt_bias_act_ws(int M, int N, int K, const void *A, const void *B, const void *bias,
                                        int activation, void *C, void *workspace, size_t workspace_bytes,
                                        void *stream)
{
    return bf16_product<true, true>(M, N, K, A, B, bias, activation, C, workspace, workspace_bytes, stream);
}

extern "C" int gemm_bf16_nt_noalloc(int M, int N, int K, const void *A, const void *B, void *C, void *stream)
{
    return bf16_product<false, true, true>(M, N, K, A, B, nullptr, GEMM355_ACT_NONE, C, nullptr, 0, stream);
}

extern "C" int gemm_bf16_nt_workspace_size(int M, int N, int K, size_t *bytes)
{
    if (M < 0 || N < 0 || K < 0 || !bytes)
        return GEMM355_ERR_INVALID_ARG;
    if (M == 0 || N == 0) {
        *bytes = 0;
        return GEMM355_OK;
    }
    int cus = 0;
    const int rc = compute_units(&cus);
    if (rc != GEMM355_OK)
        return rc;
    *bytes = plan_bf16(M, N, K, cus, g_bf16_instance.load(std::memory_order_relaxed), true).workspace_bytes;
    return GEMM355_OK;
}

extern "C" int gemm355_bf16_plan(int M, int N, int K, int compute_units, int with_workspace, int *instance,
                                 int *splits, size_t *workspace_bytes)
{
    if (M <= 0 || N <= 0 || K < 0 || compute_units <= 0 || !instance || !splits || !workspace_bytes)
        return GEMM355_ERR_INVALID_ARG;
    const Bf16Plan plan =
        plan_bf16(M, N, K, compute_units, g_bf16_instance.load(std::memory_order_relaxed), with_workspace != 0);
    *instance = plan.instance;
    *splits = plan.splits;
    *workspace_bytes = plan.workspace_bytes;
    return GEMM355_OK;
}

extern "C" int gemm355_force_instance(int instance)
{
    if (instance < 0 || instance > 3)
        return GEMM355_ERR_INVALID_ARG;
    g_bf16_instance.store(instance, std::memory_order_relaxed);
    return GEMM355_OK;
}

extern "C" int gemm355_force_schedule(int mode)
{
    if (mode < 0 || mode > 1)
        return GEMM355_ERR_INVALID_ARG;
    g_schedule.store(mode, std::memory_order_relaxed);
    return GEMM355_OK;
}

extern "C" int gemm355_supergroup(int kernel, int tiles_n, int K)
{
    if (kernel < KERNEL_BF16 || kernel > KERNEL_BF16_SMALL || tiles_n <= 0 || K < 0)
        return -GEMM355_ERR_INVALID_ARG;
    return supergroup_for(kernel, tiles_n, K);
}

extern "C" int gemm355_force_supergroup(int supergroup)
{
    if (supergroup < 0 || supergroup > 4096)
        return GEMM355_ERR_INVALID_ARG;
    g_supergroup.store(supergroup, std::memory_order_relaxed);
    return GEMM355_OK;
}

namespace {

// The NVFP4 kernel for the epilogue and the K granularity (KTAIL: K % 64 == 32).
template <bool FUSED, bool KTAIL>
int fp4_launch(const Problem &p, int act, void *stream)
{
    using namespace gemm355;
    if (!FUSED && !KTAIL && g_schedule.load(std::memory_order_relaxed) == 1)
        return launch(fp4::gemm_nvfp4_nt_kernel<EPI_PLAIN, false, true>, KERNEL_NVFP4, p, stream, BM, BN, fp4::THREADS_FP4);
    if (!FUSED)
        return launch(fp4::gemm_nvfp4_nt_kernel<EPI_PLAIN, KTAIL>, KERNEL_NVFP4, p, stream, BM, BN, fp4::THREADS_FP4);
    if (act == GEMM355_ACT_RELU)
        return launch(fp4::gemm_nvfp4_nt_kernel<ACT_RELU, KTAIL>, KERNEL_NVFP4, p, stream, BM, BN, fp4::THREADS_FP4);
    if (act == GEMM355_ACT_GELU_TANH)
        return launch(fp4::gemm_nvfp4_nt_kernel<ACT_GELU_TANH, KTAIL>, KERNEL_NVFP4, p, stream, BM, BN, fp4::THREADS_FP4);
    return launch(fp4::gemm_nvfp4_nt_kernel<ACT_NONE, KTAIL>, KERNEL_NVFP4, p, stream, BM, BN, fp4::THREADS_FP4);
}

// Argument checks of the NVFP4 products (GEMM355_OK: valid and not empty;
// GEMM355_OK with *empty set: nothing to do).
template <bool FUSED>
int fp4_validate(int M, int N, int K, const void *Aq, const void *SFA, const void *Bq, const void *SFB,
                 const void *bias, int act, const void *C, bool *empty)
{
    *empty = false;
    if (M < 0 || N < 0 || K < 0)
        return GEMM355_ERR_INVALID_ARG;
    if (FUSED && (act < GEMM355_ACT_NONE || act > GEMM355_ACT_GELU_TANH))
        return GEMM355_ERR_INVALID_ARG;
    if (M == 0 || N == 0) {
        *empty = true;
        return GEMM355_OK;
    }
    if (!C || (K > 0 && (!Aq || !SFA || !Bq || !SFB)))
        return GEMM355_ERR_INVALID_ARG;
    const size_t c_bytes = size_t(M) * size_t(N) * 2;
    if (K > 0 && (overlaps(C, c_bytes, Aq, size_t(M) * K / 2) || overlaps(C, c_bytes, Bq, size_t(N) * K / 2) ||
                  overlaps(C, c_bytes, SFA, size_t(M) * K / 16) || overlaps(C, c_bytes, SFB, size_t(N) * K / 16)))
        return GEMM355_ERR_INVALID_ARG;
    if (FUSED && overlaps(C, c_bytes, bias, size_t(N) * 2))
        return GEMM355_ERR_INVALID_ARG;
    if (!aligned(Aq, 16) || !aligned(Bq, 16) || !aligned(C, 16) || !aligned(SFA, 4) || !aligned(SFB, 4) ||
        !aligned(bias, 16))
        return GEMM355_ERR_UNSUPPORTED;
    if (K % 32 != 0 || N % 8 != 0)
        return GEMM355_ERR_UNSUPPORTED;
    if (!extent_ok(M, int64_t(K) / 2) || !extent_ok(N, int64_t(K) / 2) || !extent_ok(M, int64_t(N) * 2))
        return GEMM355_ERR_UNSUPPORTED;
    return GEMM355_OK;
}

// Shared by gemm_nvfp4_nt and gemm_nvfp4_nt_bias_act: validation, launch.
template <bool FUSED>
int fp4_product(int M, int N, int K, const void *Aq, const void *SFA, const void *Bq, const void *SFB,
                const void *bias, int act, void *C, void *stream)
{
    bool empty = false;
    const int v = fp4_validate<FUSED>(M, N, K, Aq, SFA, Bq, SFB, bias, act, C, &empty);
    if (v != GEMM355_OK || empty)
        return v;

    Problem p = {};
    p.a = Aq;
    p.b = Bq;
    p.sfa = SFA;
    p.sfb = SFB;
    p.c = C;
    p.bias = FUSED ? bias : nullptr;
    p.M = M;
    p.N = N;
    p.K = K;
    if (K % 64 != 0)
        return fp4_launch<FUSED, true>(p, act, stream);
    return fp4_launch<FUSED, false>(p, act, stream);
}

} // namespace

extern "C" int gemm_nvfp4_nt(int M, int N, int K, const void *Aq, const void *SFA, const void *Bq,
                             const void *SFB, void *C, void *stream)
{
    return fp4_product<false>(M, N, K, Aq, SFA, Bq, SFB, nullptr, GEMM355_ACT_NONE, C, stream);
}

extern "C" int gemm_nvfp4_nt_bias_act(int M, int N, int K, const void *Aq, const void *SFA, const void *Bq,
                                      const void *SFB, const void *bias, int activation, void *C, void *stream)
{
    return fp4_product<true>(M, N, K, Aq, SFA, Bq, SFB, bias, activation, C, stream);
}

namespace {

// gemm_nvfp4_nt_ws's plan: decode first, or the staging-decode kernel. Both
// run 256 x 256 tiles on the same persistent grid; a K step of the BF16
// kernel on decoded operands is shorter than one of the staging kernel,
// which decodes every A strip once per tile of its row and every B strip once
// per tile of its column, so decoding first saves time in proportion to the
// grid's rounds and the number of K steps, and costs time in proportion to
// (M + N) K, the elements decoded, plus a second launch. Measured on MI355X
// (14 shapes from 3072^2 x 8192 to 12288^2 x 4096, both paths alternating):
// with one round the staging kernel was faster at every shape, and from two
// rounds on the two balance at about kFp4RowsPerRound rows of M + N per
// round, whatever K. Forced by gemm355_force_fp4_path.
constexpr int64_t kFp4RowsPerRound = 7000;
bool fp4_decode_first(int M, int N, int K, int cus)
{
    const int forced = g_fp4_path.load(std::memory_order_relaxed);
    if (K == 0 || forced == 1)
        return false;
    if (forced == 2)
        return true;
    const int64_t tiles = ceil_div(M, BM) * ceil_div(N, BN);
    const int64_t grid = gemm355::persistent_grid((int)std::min<int64_t>(tiles, 1 << 30), cus);
    const int64_t rounds = ceil_div(tiles, grid);
    return rounds >= 2 && rounds * kFp4RowsPerRound > int64_t(M) + N;
}

constexpr size_t kFp4WsAlign = 256;
size_t fp4_ws_a_bytes(int M, int K) { return (size_t(M) * size_t(K) * 2 + kFp4WsAlign - 1) / kFp4WsAlign * kFp4WsAlign; }
size_t fp4_ws_bytes(int M, int N, int K) { return fp4_ws_a_bytes(M, K) + size_t(N) * size_t(K) * 2; }

// Both operands decoded into BF16 rows by one launch.
int launch_decode(const void *Aq, const void *SFA, void *a16, int M, const void *Bq, const void *SFB, void *b16,
                  int N, int K, void *stream)
{
    namespace f = gemm355::fp4;
    f::DecodeArgs d = {};
    d.q[0] = static_cast<const uint8_t *>(Aq);
    d.sf[0] = static_cast<const uint8_t *>(SFA);
    d.out[0] = static_cast<uint16_t *>(a16);
    d.rows[0] = M;
    d.q[1] = static_cast<const uint8_t *>(Bq);
    d.sf[1] = static_cast<const uint8_t *>(SFB);
    d.out[1] = static_cast<uint16_t *>(b16);
    d.rows[1] = N;
    d.K = K;
    // one wave per row until the grid is full; a wave walks its rows' units
    const unsigned blocks = (unsigned)std::max<int64_t>(1, std::min<int64_t>(ceil_div(int64_t(M) + N, f::DECODE_WAVES),
                                                                             f::DECODE_MAX_BLOCKS));
    return launch_kernel(f::decode_nvfp4_bf16_kernel, blocks, (unsigned)f::DECODE_THREADS, d,
                         static_cast<hipStream_t>(stream));
}

} // namespace

extern "C" int gemm_nvfp4_nt_workspace_size(int M, int N, int K, size_t *bytes)
{
    if (M < 0 || N < 0 || K < 0 || !bytes)
        return GEMM355_ERR_INVALID_ARG;
    *bytes = 0;
    if (M == 0 || N == 0 || K == 0)
        return GEMM355_OK;
    int cus = 0;
    const int rc = compute_units(&cus);
    if (rc != GEMM355_OK)
        return rc;
    if (fp4_decode_first(M, N, K, cus))
        *bytes = fp4_ws_bytes(M, N, K);
    return GEMM355_OK;
}

namespace {

// Shared by gemm_nvfp4_nt_ws and gemm_nvfp4_nt_bias_act_ws: validation (all
// before any HIP call), then the staging kernel or decode-first by the shape
// rule (fp4_decode_first); FUSED adds the bias and activation in the epilogue
// of whichever kernel writes C.
template <bool FUSED>
int fp4_ws_product(int M, int N, int K, const void *Aq, const void *SFA, const void *Bq, const void *SFB,
                   const void *bias, int act, void *C, void *workspace, size_t workspace_bytes, void *stream)
{
    bool empty = false;
    const int v = fp4_validate<FUSED>(M, N, K, Aq, SFA, Bq, SFB, bias, act, C, &empty);
    if (v != GEMM355_OK || empty)
        return v;
    if (workspace_bytes > 0 && !workspace)
        return GEMM355_ERR_INVALID_ARG;
    if (workspace_bytes > 0) {   // checks of the workspace itself, before any HIP call
        if (!aligned(workspace, 16))
            return GEMM355_ERR_UNSUPPORTED;
        if (overlaps(workspace, workspace_bytes, C, size_t(M) * size_t(N) * 2) ||
            overlaps(workspace, workspace_bytes, Aq, size_t(M) * K / 2) ||
            overlaps(workspace, workspace_bytes, Bq, size_t(N) * K / 2) ||
            overlaps(workspace, workspace_bytes, SFA, size_t(M) * K / 16) ||
            overlaps(workspace, workspace_bytes, SFB, size_t(N) * K / 16) ||
            (FUSED && overlaps(workspace, workspace_bytes, bias, size_t(N) * 2)))
            return GEMM355_ERR_INVALID_ARG;
    }
    int cus = 0;
    const int rc = compute_units(&cus);
    if (rc != GEMM355_OK)
        return rc;
    if (!fp4_decode_first(M, N, K, cus))
        return fp4_product<FUSED>(M, N, K, Aq, SFA, Bq, SFB, bias, act, C, stream);
    if (workspace_bytes < fp4_ws_bytes(M, N, K))
        return GEMM355_ERR_UNSUPPORTED;
    if (!extent_ok(M, int64_t(K) * 2) || !extent_ok(N, int64_t(K) * 2))
        return GEMM355_ERR_UNSUPPORTED;   // the decoded operands' extents, as for gemm_bf16_nt
    uint8_t *a16 = static_cast<uint8_t *>(workspace);
    uint8_t *b16 = a16 + fp4_ws_a_bytes(M, K);
    const int st = launch_decode(Aq, SFA, a16, M, Bq, SFB, b16, N, K, stream);
    if (st != GEMM355_OK)
        return st;
    return bf16_product<FUSED, false>(M, N, K, a16, b16, bias, act, C, nullptr, 0, stream);
}

} // namespace

extern "C" int gemm_nvfp4_nt_ws(int M, int N, int K, const void *Aq, const void *SFA, const void *Bq,
                                const void *SFB, void *C, void *workspace, size_t workspace_bytes, void *stream)
{
    return fp4_ws_product<false>(M, N, K, Aq, SFA, Bq, SFB, nullptr, GEMM355_ACT_NONE, C, workspace,
                                 workspace_bytes, stream);
}

extern "C" int gemm_nvfp4_nt_bias_act_ws(int M, int N, int K, const void *Aq, const void *SFA, const void *Bq,
                                         const void *SFB, const void *bias, int activation, void *C,
                                         void *workspace, size_t workspace_bytes, void *stream)
{
    return fp4_ws_product<true>(M, N, K, Aq, SFA, Bq, SFB, bias, activation, C, workspace, workspace_bytes,
                                stream);
}

extern "C" int gemm355_nvfp4_plan(int M, int N, int K, int compute_units, int *decode_first, size_t *workspace_bytes)
{
    if (M <= 0 || N <= 0 || K < 0 || compute_units <= 0 || !decode_first || !workspace_bytes)
        return GEMM355_ERR_INVALID_ARG;
    const bool d = fp4_decode_first(M, N, K, compute_units);
    *decode_first = d ? 1 : 0;
    *workspace_bytes = d ? fp4_ws_bytes(M, N, K) : 0;
    return GEMM355_OK;
}

extern "C" int gemm355_force_fp4_path(int path)
{
    if (path < 0 || path > 2)
        return GEMM355_ERR_INVALID_ARG;
    g_fp4_path.store(path, std::memory_order_relaxed);
    return GEMM355_OK;
}

namespace {

template <bool FUSED>
int mx_product(int M, int N, int K, const void *Aq, const void *SA, const void *Bq, const void *SB, const void *bias,
               int act, void *C, void *stream)
{
    if (M < 0 || N < 0 || K < 0)
        return GEMM355_ERR_INVALID_ARG;
    if (FUSED && (act < GEMM355_ACT_NONE || act > GEMM355_ACT_GELU_TANH))
        return GEMM355_ERR_INVALID_ARG;
    if (M == 0 || N == 0)
        return GEMM355_OK;
    if (!C || (K > 0 && (!Aq || !SA || !Bq || !SB)))
        return GEMM355_ERR_INVALID_ARG;
    const size_t c_bytes = size_t(M) * size_t(N) * 2;
    if (K > 0 && (overlaps(C, c_bytes, Aq, size_t(M) * K / 2) || overlaps(C, c_bytes, Bq, size_t(N) * K / 2) ||
                  overlaps(C, c_bytes, SA, size_t(M) * K / 32) || overlaps(C, c_bytes, SB, size_t(N) * K / 32)))
        return GEMM355_ERR_INVALID_ARG;
    if (FUSED && overlaps(C, c_bytes, bias, size_t(N) * 2))
        return GEMM355_ERR_INVALID_ARG;
    if (!aligned(Aq, 16) || !aligned(Bq, 16) || !aligned(C, 16) || !aligned(SA, 16) || !aligned(SB, 16) ||
        !aligned(bias, 16))
        return GEMM355_ERR_UNSUPPORTED;
    if (K % 512 != 0 || N % 8 != 0)
        return GEMM355_ERR_UNSUPPORTED;
    if (!extent_ok(M, int64_t(K) / 2) || !extent_ok(N, int64_t(K) / 2) || !extent_ok(M, int64_t(N) * 2))
        return GEMM355_ERR_UNSUPPORTED;

    Problem p = {};
    p.a = Aq;
    p.b = Bq;
    p.sfa = SA;
    p.sfb = SB;
    p.c = C;
    p.bias = FUSED ? bias : nullptr;
    p.M = M;
    p.N = N;
    p.K = K;
    using namespace gemm355;
    if (!FUSED)
        return launch(mx::gemm_mxfp4_nt_kernel<EPI_PLAIN>, KERNEL_MXFP4, p, stream, mx::TM, mx::TN, mx::THREADS_MX);
    if (act == GEMM355_ACT_RELU)
        return launch(mx::gemm_mxfp4_nt_kernel<ACT_RELU>, KERNEL_MXFP4, p, stream, mx::TM, mx::TN, mx::THREADS_MX);
    if (act == GEMM355_ACT_GELU_TANH)
        return launch(mx::gemm_mxfp4_nt_kernel<ACT_GELU_TANH>, KERNEL_MXFP4, p, stream, mx::TM, mx::TN, mx::THREADS_MX);
    return launch(mx::gemm_mxfp4_nt_kernel<ACT_NONE>, KERNEL_MXFP4, p, stream, mx::TM, mx::TN, mx::THREADS_MX);
}

} // namespace

extern "C" int gemm_mxfp4_nt(int M, int N, int K, const void *Aq, const void *SA, const void *Bq, const void *SB,
                             void *C, void *stream)
{
    return mx_product<false>(M, N, K, Aq, SA, Bq, SB, nullptr, GEMM355_ACT_NONE, C, stream);
}

extern "C" int gemm_mxfp4_nt_bias_act(int M, int N, int K, const void *Aq, const void *SA, const void *Bq,
                                      const void *SB, const void *bias, int activation, void *C, void *stream)
{
    return mx_product<true>(M, N, K, Aq, SA, Bq, SB, bias, activation, C, stream);
}

extern "C" const char *gemm355_status_string(int status)
{
    switch (status) {
    case GEMM355_OK:
        return "ok";
    case GEMM355_ERR_INVALID_ARG:
        return "invalid argument (negative size, NULL pointer or overlapping output)";
    case GEMM355_ERR_UNSUPPORTED:
        return "unsupported (alignment, K or N granularity, operand extent, or a workspace smaller than the plan "
               "needs)";
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
