// Shared pieces of the 128 x 128 tile kernels (the products with the
// weights as stored and the floating-point tiled product): the
// workgroup-to-tile mapping, a barrier that leaves global loads in flight,
// and the double-buffered K loop of the weights-as-stored kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

namespace nqk {

// Tile of workgroup b in a grid of tiles_m x tiles_n output tiles, for
// kernels launched with 8 * ceil(tiles_m * tiles_n / 8) workgroups.
// Workgroups are dealt to the 8 XCDs round-robin (b on XCD b % 8), and XCD x
// takes the x-th eighth of a tile list that runs through panels of 4 tile
// rows, column by column inside a panel: the tiles one XCD holds at once
// then share 4 row tiles of the activations and a band of weight columns in
// that XCD's L2, instead of every XCD reading every activation row.  False
// for the workgroups past the last tile.
__device__ __forceinline__ bool xcd_panel_tile(int b, int tiles_m, int tiles_n, int &tm, int &tn)
{
    const int total = tiles_m * tiles_n, per_xcd = (total + 7) / 8;
    const int t = (b % 8) * per_xcd + b / 8;
    if (t >= total) return false;
    const int per_panel = 4 * tiles_n, p0 = t / per_panel * 4, in_panel = t % per_panel;
    const int h = min(4, tiles_m - p0);
    tm = p0 + in_panel % h;
    tn = in_panel / h;
    return true;
}

// Workgroup barrier that waits only for this wave's LDS accesses (and
// scalar loads), leaving its global loads in flight: __syncthreads() would
// also wait for every outstanding global load.  s_waitcnt fields on gfx9:
// vmcnt in bits 3:0 and 15:14 (all ones: no wait), expcnt in bits 6:4 (7: no
// wait), lgkmcnt in bits 11:8 (0).  The empty asm statements keep the
// compiler from moving memory accesses across the barrier, and the
// scheduling barriers any other instruction: arithmetic on data of a later
// step stays after it, so that its wait for that data does too.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// The K loop of the 128 x 128 tile kernels, for `steps` K steps.  The
// kernel supplies load(j, ld) (issue step j's global loads into registers),
// stage(ld, buffer) (convert them and write the x and weight tiles into LDS
// buffer 0 or 1, a std::integral_constant) and mfmas(buffer) (the step's
// matrix-core work on that buffer).  Step j's data sits in ld[j % 2]: it is
// loaded two steps before its MFMAs and staged one step before them, into
// buffer j % 2.  At step j the MFMAs read buffer j % 2, staged before the
// previous barrier; then step j + 1 is staged into the other buffer, whose
// last reader, step j - 1, every wave finished before that barrier.  One
// barrier per step, waiting for LDS accesses only, so the loads of the next
// two steps stay in flight across it.  Inside the loop every load and stage
// is unconditional, with step indices past the last clamped to it (the last
// step read again, staged into a buffer nothing reads any more): the same
// loads are then in flight at every step, and the compiler's waits count
// only the step being staged.
template <typename Ld, typename LoadF, typename StageF, typename MfmaF>
__device__ __forceinline__ void tile_pipeline(int steps, LoadF &&load, StageF &&stage, MfmaF &&mfmas)
{
    if (steps <= 0) return;
    const int last = steps - 1;
    Ld ld[2];
    auto step = [&](int j, auto parc) {
        constexpr int B = decltype(parc)::value;
        mfmas(parc);
        stage(ld[B ^ 1], std::integral_constant<int, B ^ 1>{});
        load(min(j + 3, last), ld[B ^ 1]);
        lds_barrier();
    };
    load(0, ld[0]);
    load(min(1, last), ld[1]);
    stage(ld[0], std::integral_constant<int, 0>{});
    load(min(2, last), ld[0]);
    lds_barrier();
    int j = 0;
    for (; j + 1 < steps; j += 2) {
        step(j, std::integral_constant<int, 0>{});
        step(j + 1, std::integral_constant<int, 1>{});
    }
    if (j < steps) mfmas(std::integral_constant<int, 0>{});   // an odd last step, staged in buffer 0
    __builtin_amdgcn_s_waitcnt(0);                            // the clamped prefetches
}

// Workgroups to launch for `tiles` tiles (a multiple of 8), or 0 when the
// tile count does not fit the 32-bit index arithmetic.
inline unsigned xcd_panel_blocks(int64_t tiles)
{
    return tiles >= ((int64_t)1 << 31) - 8 ? 0u : (unsigned)((tiles + 7) / 8 * 8);
}

}  // namespace nqk
