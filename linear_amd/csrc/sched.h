// sched.h -- workgroup-to-tile mapping and instruction-order helpers shared by
// the MFMA kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>

namespace lin {

// Tile (tm, tn) of workgroup bid in a tiles_m x tiles_n grid.  Consecutive
// workgroup ids are dealt round-robin over the device's 2^xcd_shift XCDs (8 on
// a whole MI355X; the host reads the count from the device), so each XCD is
// given a contiguous run of tiles, walked in groups of 4 tile-rows: tiles running
// together on one XCD share operand panels in its L2.  With 32 tiles at a time
// per XCD that is 4 x panels and 8 weight panels; x panels cost more L2 misses
// per panel, and 4 rows measured faster than 2, 8 or 16.
__device__ inline void tile_coords(int bid, int tiles_m, int tiles_n, int xcd_shift, int& tm, int& tn) {
    const int G = tiles_m * tiles_n;
    const int xmask = (1 << xcd_shift) - 1;
    const int xcd = bid & xmask, idx = bid >> xcd_shift;
    const int q = G >> xcd_shift, r = G & xmask;
    const int t = (xcd < r) ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
    constexpr int GROUP = 4;
    const int per_group = GROUP * tiles_n;
    const int g = t / per_group;
    const int first_m = g * GROUP;
    const int gm = min(tiles_m - first_m, GROUP);
    const int rem = t - g * per_group;
    tm = first_m + rem % gm;
    tn = rem / gm;
}

// Calls f.template operator()<I>() for I = B .. N-1 (compile-time loop).
template <int B, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < N) {
        f.template operator()<B>();
        static_for<B + 1, N>(f);
    }
}

// Instruction order of one K step of the streaming GEMM: its first MFMA, the
// NREAD fragment reads of the next step, then the other NMFMA - 1 MFMAs with ND
// loads spaced evenly between them.
template <int NMFMA, int NREAD, int ND>
__device__ __forceinline__ void order_step() {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (NREAD > 0) __builtin_amdgcn_sched_group_barrier(0x100, NREAD, 0);
    constexpr int q = (NMFMA - 1) / (ND + 1);
    static_for<0, ND>([&]<int d>() {
        if constexpr (q > 0) __builtin_amdgcn_sched_group_barrier(0x008, q, 0);
        __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
    });
    if constexpr (NMFMA - 1 - q * ND > 0) __builtin_amdgcn_sched_group_barrier(0x008, NMFMA - 1 - q * ND, 0);
    __builtin_amdgcn_sched_barrier(0);
}

// Instruction order of one K step of the 16 x 16 x 32 streaming loop: its first
// MFMA, the FN A-fragment reads of the next step, the rest of B fragment 0's
// MFMAs, then for each B fragment j its next-step read, one of the ND loads while
// any are left, and fragment j + 1's FN MFMAs.
template <int FN, int FM, int ND>
__device__ __forceinline__ void order_step16() {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, FN, 0);
    if constexpr (FN > 1) __builtin_amdgcn_sched_group_barrier(0x008, FN - 1, 0);
    static_for<0, FM>([&]<int j>() {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if constexpr (j < ND) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
        if constexpr (j + 1 < FM) __builtin_amdgcn_sched_group_barrier(0x008, FN, 0);
    });
    if constexpr (ND > FM) __builtin_amdgcn_sched_group_barrier(0x010, ND - FM, 0);
    __builtin_amdgcn_sched_barrier(0);
}

}  // namespace lin
