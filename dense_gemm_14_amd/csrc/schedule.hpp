// schedule.hpp -- which output tile each workgroup of the persistent grid
// computes, and in which order. Compiled for both host and device: the kernels
// use it on the GPU and the library exports a host-only view for tests.
#pragma once

#include <hip/hip_runtime.h>

namespace gemm355 {

// Position `pos` of the visiting order -> output tile (tm, tn).
//
// "Supergroup" order ("NVFP4 GEMM on Blackwell", section "Kernel 5",
// "Redesign"): the N tiles are cut into bands of `sg` adjacent tiles; a band
// is walked one M tile at a time, covering the band's N tiles for that M tile
// before moving to the next M tile; then the next band. The last band may be
// narrower than `sg`.
__host__ __device__ inline void supergroup_tile(int pos, int tiles_m, int tiles_n, int sg,
                                                int &tm, int &tn)
{
    const int band_tiles = sg * tiles_m;
    const int band = pos / band_tiles;
    const int n0 = band * sg;
    const int rest = tiles_n - n0;
    const int width = rest < sg ? rest : sg;
    const int r = pos - band * band_tiles;
    tm = r / width;
    tn = n0 + r % width;
}

// Visiting-order position that workgroup `wg` of a `grid`-wide persistent
// launch computes in round `round` (may be >= tiles, meaning: nothing left).
//
// Workgroups are dispatched to the 8 XCDs round-robin (wg % 8), each XCD with
// its own L2. When the grid is a multiple of 8, the grid/8 workgroups that
// share an XCD take consecutive positions of each round, so the tiles an L2
// serves at the same time form one compact block of the supergroup order and
// share their A rows and B rows.
__host__ __device__ inline int schedule_position(int wg, int round, int grid)
{
    const int base = round * grid;
    if (grid % 8 != 0)
        return base + wg;
    return base + (wg % 8) * (grid / 8) + wg / 8;
}

// Grid size for `tiles` output tiles on `cus` compute units, one resident
// workgroup per compute unit: a multiple of 8 whenever there are at least 8
// tiles, so that the XCD-aware dealing above is a bijection in every round.
__host__ __device__ inline int persistent_grid(int tiles, int cus)
{
    if (tiles < 8)
        return tiles;
    int g = tiles < cus ? tiles : cus;
    g &= ~7;
    return g < 8 ? 8 : g;
}

} // namespace gemm355
