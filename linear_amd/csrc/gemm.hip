// gemm.hip -- MFMA tiled GEMM for the FP16 linear layer on gfx950.
//
// Computes the projection tile C[n, m] = sum_k weight[n, k] * x[m, k] with
// v_mfma_f32_32x32x16_f16 (exact FP16 products, FP32 accumulation), then the
// contract's epilogue in registers: round to FP16, and with a bias widen, add
// b[n] in FP32 and round again ("tensor programs, part 1", section "One Program
// and One Numerical Contract"; the Inductor capture's cast sequence).
//
// Layout choices:
//  - The weight tile is the MFMA A operand and the x tile the B operand, so the
//    accumulator rows are output columns n: each lane ends up holding four
//    consecutive n of one output row m and stores them as one 8-byte write.
//  - Both operands are K-contiguous in HBM and are read in place ([N, K] weight,
//    no transpose copy, as the poot op table's dense contraction requires):
//    each thread moves 16-byte chunks along K; a wave covers 8 full 128-byte
//    rows per load instruction.
//  - K-slices of BK = 64 are staged through LDS, double buffered: the loads of
//    slice t+1 are issued before the MFMAs of slice t, written to the other LDS
//    buffer after them, one barrier per slice.
//  - LDS rows are 128 bytes; the 16-byte chunk c of row r is stored at chunk
//    c ^ (r & 7) so that the ds_read_b128 of 8 consecutive rows at one K offset
//    touches 8 different bank groups.
//  - Ragged M, N and K need no special tiles: loads go through buffer
//    resources whose range ends at the matrix's last valid element, so rows past
//    M or N and K chunks past K read as zero; stores are masked.
//  - Workgroup ids are remapped so that each XCD (consecutive ids are dealt
//    round-robin over the 8 XCDs) owns a contiguous run of tiles, walked in
//    groups of 8 tile-rows, so tiles running together share x and weight panels
//    in that XCD's L2.
#include "common.h"
#include "kernels.h"

namespace lin {

__device__ inline void tile_coords(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int G = tiles_m * tiles_n;
    const int xcd = bid & 7, idx = bid >> 3;
    const int q = G >> 3, r = G & 7;
    const int t = (xcd < r) ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
    constexpr int GROUP = 8;
    const int per_group = GROUP * tiles_n;
    const int g = t / per_group;
    const int first_m = g * GROUP;
    const int gm = min(tiles_m - first_m, GROUP);
    const int rem = t - g * per_group;
    tm = first_m + rem % gm;
    tn = rem / gm;
}

template <int BM, int BN, int WM, int WN, bool VEC, bool BIAS>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_f16_kernel(LinearArgs a) {
    constexpr int BK = 64;
    constexpr int NT = WM * WN * 64;
    constexpr int TM = BM / WM, TN = BN / WN;   // one wave's output tile (m x n)
    constexpr int FM = TM / 32, FN = TN / 32;   // 32x32 MFMA blocks per wave
    constexpr int RSTEP = NT / 8;               // rows covered by one pass of the block
    constexpr int CW = BN / RSTEP, CX = BM / RSTEP;
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");
    static_assert(CW * RSTEP == BN && CX * RSTEP == BM, "tile rows must be a multiple of NT/8");
    static_assert(RSTEP % 8 == 0, "swizzle assumes rows of one thread share r & 7");
    constexpr int STAGE = (BN + BM) * BK;       // halves per LDS stage
    __shared__ __attribute__((aligned(16))) f16 smem[2 * STAGE];

    int tm, tn;
    tile_coords(blockIdx.x, a.tiles_m, a.tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int K = a.K;

    const __amdgpu_buffer_rsrc_t rw = matrix_rsrc(a.w, n0, a.N, a.ldw, K);
    const __amdgpu_buffer_rsrc_t rx = matrix_rsrc(a.x, m0, a.M, a.ldx, K);

    const int tid = threadIdx.x;
    const int kc = tid & 7;          // this thread's 16-byte chunk within a BK slice
    const int r0 = tid >> 3;         // first tile row it loads; then r0 + i * RSTEP
    const int swz = (kc ^ (r0 & 7)) << 3;

    uint32_t woff[CW], xoff[CX];
#pragma unroll
    for (int i = 0; i < CW; ++i) woff[i] = (uint32_t)(((int64_t)(r0 + i * RSTEP) * a.ldw + kc * 8) * 2);
#pragma unroll
    for (int i = 0; i < CX; ++i) xoff[i] = (uint32_t)(((int64_t)(r0 + i * RSTEP) * a.ldx + kc * 8) * 2);

    u32x4 wreg[CW], xreg[CX];

    auto gload = [&](int k0) {
        if (VEC) {
            const bool kin = k0 + kc * 8 < K;
            const uint32_t kb = (uint32_t)k0 * 2u;
#pragma unroll
            for (int i = 0; i < CW; ++i) wreg[i] = load16(rw, kin ? woff[i] + kb : kOOB);
#pragma unroll
            for (int i = 0; i < CX; ++i) xreg[i] = load16(rx, kin ? xoff[i] + kb : kOOB);
        } else {
            const uint32_t kb = (uint32_t)k0 * 2u;
#pragma unroll
            for (int i = 0; i < CW; ++i) wreg[i] = load8_masked(rw, woff[i] + kb, k0 + kc * 8, K, true);
#pragma unroll
            for (int i = 0; i < CX; ++i) xreg[i] = load8_masked(rx, xoff[i] + kb, k0 + kc * 8, K, true);
        }
    };
    auto lds_store = [&](int s) {
        f16* sw = smem + s * STAGE;
        f16* sx = sw + BN * BK;
#pragma unroll
        for (int i = 0; i < CW; ++i) *(u32x4*)(sw + (r0 + i * RSTEP) * BK + swz) = wreg[i];
#pragma unroll
        for (int i = 0; i < CX; ++i) *(u32x4*)(sx + (r0 + i * RSTEP) * BK + swz) = xreg[i];
    };

    const int lane = tid & 63, wave = tid >> 6;
    const int wn = wave % WN, wm = wave / WN;
    const int lr = lane & 31, lh = lane >> 5;

    f32x16 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = (f32x16){};

    const int nk = (K + BK - 1) / BK;
    gload(0);
    lds_store(0);
    __syncthreads();

    for (int t = 0; t < nk; ++t) {
        const int cur = t & 1;
        if (t + 1 < nk) gload((t + 1) * BK);
        const f16* sw = smem + cur * STAGE;
        const f16* sx = sw + BN * BK;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int ch = ((ks * 2 + lh) ^ (lr & 7)) << 3;
            f16x8 av[FN], bv[FM];
#pragma unroll
            for (int i = 0; i < FN; ++i) av[i] = *(const f16x8*)(sw + (wn * TN + i * 32 + lr) * BK + ch);
#pragma unroll
            for (int j = 0; j < FM; ++j) bv[j] = *(const f16x8*)(sx + (wm * TM + j * 32 + lr) * BK + ch);
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
        }
        if (t + 1 < nk) lds_store(cur ^ 1);
        __syncthreads();
    }

    // Epilogue.  Accumulator element v of block (i, j) sits at
    //   n = n0 + wn*TN + 32 i + 8 (v / 4) + 4 lh + (v % 4),   m = m0 + wm*TM + 32 j + lr.
#pragma unroll
    for (int i = 0; i < FN; ++i) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int nb = n0 + wn * TN + i * 32 + g * 8 + lh * 4;
            float bias[4] = {0.f, 0.f, 0.f, 0.f};
            if (BIAS) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (nb + e < a.N) bias[e] = (float)bits_to_f16(a.b[nb + e]);
            }
#pragma unroll
            for (int j = 0; j < FM; ++j) {
                const int m = m0 + wm * TM + j * 32 + lr;
                if (m >= a.M) continue;
                uint16_t o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = finish<BIAS>(acc[i][j][g * 4 + e], bias[e]);
                uint16_t* dst = a.y + (int64_t)m * a.ldy + nb;
                if (a.vec_store && nb + 3 < a.N) {
                    uint2 v;
                    v.x = (uint32_t)o[0] | ((uint32_t)o[1] << 16);
                    v.y = (uint32_t)o[2] | ((uint32_t)o[3] << 16);
                    *(uint2*)dst = v;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (nb + e < a.N) dst[e] = o[e];
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Host-side launchers: one per tile configuration.

template <int BM, int BN, int WM, int WN>
static hipError_t launch_cfg(const LinearArgs& a, bool vec, bool bias, hipStream_t stream) {
    const dim3 grid((unsigned)(a.tiles_m * a.tiles_n));
    const dim3 block(WM * WN * 64);
    LinearArgs args = a;
    void* params[] = {&args};
    const void* fn;
    if (vec) fn = bias ? (const void*)gemm_f16_kernel<BM, BN, WM, WN, true, true>
                       : (const void*)gemm_f16_kernel<BM, BN, WM, WN, true, false>;
    else fn = bias ? (const void*)gemm_f16_kernel<BM, BN, WM, WN, false, true>
                   : (const void*)gemm_f16_kernel<BM, BN, WM, WN, false, false>;
    return hipLaunchKernel(fn, grid, block, params, 0, stream);
}

const GemmConfig kGemmConfigs[kNumGemmConfigs] = {
    // BM, BN, WM, WN
    {256, 256, 2, 2},
    {256, 128, 2, 2},
    {128, 256, 2, 2},
    {128, 128, 2, 2},
    {64, 64, 2, 2},
};

hipError_t launch_gemm(int cfg, const LinearArgs& a, bool vec, bool bias, hipStream_t stream) {
    switch (cfg) {
        case 0: return launch_cfg<256, 256, 2, 2>(a, vec, bias, stream);
        case 1: return launch_cfg<256, 128, 2, 2>(a, vec, bias, stream);
        case 2: return launch_cfg<128, 256, 2, 2>(a, vec, bias, stream);
        case 3: return launch_cfg<128, 128, 2, 2>(a, vec, bias, stream);
        case 4: return launch_cfg<64, 64, 2, 2>(a, vec, bias, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace lin
