// indexed.hip -- the indexed contraction on gfx950 ("The Graph IR", op table:
// IndexedMatMul).  x [M, K] against expert tables W [E, K, N] read in place:
// row m contracts against expert idx[m], y[m, n] = sum_k x[m, k] * W[idx[m], k, n],
// FP32 accumulation, the result rounded to the element type (or the FP32 sums).
//
// One workgroup per (expert, 64 output columns).  It first collects, in index
// order, the rows whose idx names its expert: the 256 threads test 256 entries
// of idx at a time and place the hits with wave ballots and per-wave counts, so
// the row list is deterministic and needs no workspace.  The rows are then
// contracted 16 at a time with v_mfma_f32_16x16x32 (expert columns as the A
// operand, x rows as B), K split over the 4 waves and the partial tiles added in
// FP32 through LDS in wave order.  Each expert's table is therefore read once
// per 16 of its rows, and an expert no row selects costs one scan of idx.
//
// The expert table is stored k-major ([K, N], n contiguous) while an MFMA
// operand holds 8 consecutive k of one n per lane, so the A fragments are
// gathered column-wise: lane l takes W[k .. k+7][n0 + l % 16].  x rows are
// K-contiguous and load as 16-byte fragments when aligned.
#include "common.h"
#include "kernels.h"

namespace lin {

template <int E, int MODE>
__device__ inline void indexed_store4(const IndexedArgs& a, int m, int nb, f32x4 v) {
    if (MODE == kOutF32) {
        float* dst = (float*)a.y + (int64_t)m * a.ldy + nb;
        if (a.vec_store && nb + 3 < a.N) {
            *(f32x4*)dst = v;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (nb + e < a.N) dst[e] = v[e];
        }
        return;
    }
    uint16_t* dst = (uint16_t*)a.y + (int64_t)m * a.ldy + nb;
    uint16_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = narrow<E>(v[e]);
    if (a.vec_store && nb + 3 < a.N) {
        uint2 u;
        u.x = (uint32_t)o[0] | ((uint32_t)o[1] << 16);
        u.y = (uint32_t)o[2] | ((uint32_t)o[3] << 16);
        *(uint2*)dst = u;
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (nb + e < a.N) dst[e] = o[e];
    }
}

template <int E, int MODE>
__global__ void __launch_bounds__(kIdxWaves * 64)
indexed_kernel(IndexedArgs a) {
    constexpr int NT = kIdxWaves * 64;
    __shared__ int rows[kIdxCap];
    __shared__ int wcount[kIdxWaves];
    __shared__ f32x4 red[kIdxWaves][4][64];

    const int expert = blockIdx.y;
    const int n0 = blockIdx.x * kIdxCols;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, grp = lane >> 4;
    const uint16_t* we = a.w + (int64_t)expert * a.sw;
    const int U = (a.K + 31) / 32;
    const int ub = wave * U / kIdxWaves, ue = (wave + 1) * U / kIdxWaves;

    int cursor = 0;
    for (;;) {
        // collect up to kIdxCap rows of this expert, in index order
        int count = 0;
        while (cursor < a.M && count <= kIdxCap - NT) {
            const int m = cursor + (int)threadIdx.x;
            const bool hit = m < a.M && a.idx[m] == expert;
            const uint64_t mask = __ballot(hit);
            if (lane == 0) wcount[wave] = __popcll(mask);
            __syncthreads();
            int base = count, total = 0;
#pragma unroll
            for (int w = 0; w < kIdxWaves; ++w) {
                if (w < wave) base += wcount[w];
                total += wcount[w];
            }
            if (hit) rows[base + __popcll(mask & ((uint64_t(1) << lane) - 1))] = m;
            __syncthreads();
            count += total;
            cursor += NT;
        }
        for (int rc = 0; rc < count; rc += 16) {
            const int nrow = min(16, count - rc);
            const int m = r < nrow ? rows[rc + r] : -1;
            f32x4 acc[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[b] = (f32x4){};
            for (int u = ub; u < ue; ++u) {
                const int k = u * 32 + grp * 8;          // this lane's 8 K values: k .. k+7
                u32x4 xb = (u32x4){0u, 0u, 0u, 0u};
                if (m >= 0) {
                    const uint16_t* xr = a.x + (int64_t)m * a.ldx + k;
                    if (a.vec_x && k + 7 < a.K) {
                        xb = *(const u32x4*)xr;
                    } else {
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            if (k + j < a.K) xb[j >> 1] |= (uint32_t)xr[j] << (16 * (j & 1));
                    }
                }
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int n = n0 + 16 * b + r;
                    u32x4 wa = (u32x4){0u, 0u, 0u, 0u};
                    if (n < a.N) {
                        const uint16_t* wc = we + (int64_t)k * a.ldw + n;
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            if (k + j < a.K) wa[j >> 1] |= (uint32_t)wc[(int64_t)j * a.ldw] << (16 * (j & 1));
                    }
                    acc[b] = mfma16x16x32<E>(wa, xb, acc[b]);
                }
            }
#pragma unroll
            for (int b = 0; b < 4; ++b) red[wave][b][lane] = acc[b];
            __syncthreads();
            if (wave == 0 && m >= 0) {
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    f32x4 s = red[0][b][lane];
#pragma unroll
                    for (int w = 1; w < kIdxWaves; ++w) s += red[w][b][lane];
                    // lane l holds x row l % 16 and expert columns 4 (l / 16) .. +3 of block b
                    indexed_store4<E, MODE>(a, m, n0 + 16 * b + 4 * grp, s);
                }
            }
            __syncthreads();
        }
        if (cursor >= a.M) break;
    }
}

template <int E>
static const void* indexed_fn(int mode) {
    return mode == kOutF32 ? (const void*)indexed_kernel<E, kOutF32> : (const void*)indexed_kernel<E, kOutRound>;
}

hipError_t launch_indexed(int elem, const IndexedArgs& a, int mode, hipStream_t stream) {
    const void* fn = elem == kBF16 ? indexed_fn<kBF16>(mode) : indexed_fn<kF16>(mode);
    IndexedArgs args = a;
    void* params[] = {&args};
    const dim3 grid((unsigned)((a.N + kIdxCols - 1) / kIdxCols), (unsigned)a.E);
    return hipLaunchKernel(fn, grid, dim3(kIdxWaves * 64), params, 0, stream);
}

}  // namespace lin
