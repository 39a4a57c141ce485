// skinny.hip -- the small-M (decode) path of the linear layer on gfx950
// (binary16 or bfloat16 operands; rounded, biased or FP32 output, as the GEMM).
//
// For M <= 16 the layer is a weight stream: every weight element is used by at
// most 16 rows of x, so the time is the time to read weight[N, K] once from HBM.
// One workgroup owns 16 weight rows (16 output columns n) and up to 16 rows of x;
// its waves split K into contiguous ranges, so all of the block's weight bytes
// are in flight at once.  Each wave contracts its range with
// v_mfma_f32_16x16x32_f16 (weight rows as the A operand, x rows as B; rows of x
// past M read as zero through the buffer resource, costing no memory traffic),
// keeping FP32 partial sums in registers.  The partial tiles are then added in
// FP32 through LDS in a fixed wave order (deterministic), and only that full-K
// sum is rounded to FP16, followed by the bias epilogue ("tensor programs, part
// 1", section "One Program and One Numerical Contract").
//
// Within one MFMA step of 32 K values, lane l supplies weight row (l % 16) and
// x row (l % 16) over the same 8 K values, chunk 4u + l/16 of the row: the four
// lanes of one row read 64 contiguous bytes, and A and B always pair the same K.
//
// Two variants:
//  - skinny_stream (16-byte aligned layouts): per pass of up to 16 MFMA steps
//    a wave first copies the rows of x it needs straight into its own LDS region
//    (one contiguous 1 KB direct-to-LDS load per x row, so at M = 1 a single
//    instruction instead of one per step), then issues all of its weight loads
//    back to back (a scheduling barrier keeps the compiler from interleaving them
//    with the MFMAs, so every load is in flight at once), and consumes each weight
//    fragment as it arrives.
//  - skinny_kernel (any layout): element-wise masked loads of both operands.
// Both request the bias words of the finishing wave before the main loop.
//
// A third kernel, gemv_stream, takes M = 1 (16-byte aligned, ungrouped, no
// epilogue program, K up to kGemvMaxK).  There x is a single row, so nothing is
// gained by sharing it between weight rows through an MFMA, and the weight can be
// streamed the way a plain read streams a buffer fastest on this part: many
// small workgroups, each wave one weight row with all of its loads in flight.
// Wave w of workgroup g owns row n = kGemvRows g + w; segment s of the row (K
// values [512 s, 512 s + 512), 16 bytes per lane) is one 1 KB load.  The
// workgroup first copies x into LDS; each lane multiplies its 8 weight values of
// a segment by the matching x values in FP32 (exact products: 11-bit or 8-bit
// significands) and adds them in K order into one of 8 sums (segment s into sum
// s mod 8, which keeps the dependent FMA chains short); the 8 sums are added in
// order, then the 64 lanes' (DPP exchanges within each row of 16 lanes, then the
// four row sums in row order), and lane 0 rounds the full-K sum and runs the
// bias step.  A fixed order throughout: deterministic.
#include "common.h"
#include "kernels.h"

namespace lin {

template <int WAVES, int E, int MODE>
__global__ void __launch_bounds__(WAVES * 64)
skinny_stream(LinearArgs a) {
    enter_group<MODE>(a);
    constexpr int PU = 16;                    // MFMA steps (32 K values each) per pass
    constexpr int XPITCH = PU * 64 + 16;      // bytes per LDS row of x: 512 halves + pad
    __shared__ __attribute__((aligned(16))) unsigned char xs[WAVES * 16 * XPITCH];
    __shared__ f32x4 red[WAVES][64];

    const int n0 = blockIdx.x * 16, m0 = blockIdx.y * 16;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row = lane & 15, grp = lane >> 4;
    const int K = a.K;
    const int mv = min(16, a.M - m0);         // valid x rows in this block

    const __amdgpu_buffer_rsrc_t rw = matrix_rsrc(a.w, n0, a.N, a.ldw, K);
    const __amdgpu_buffer_rsrc_t rx = matrix_rsrc(a.x, m0, a.M, a.ldx, K);
    const uint32_t wrow = (uint32_t)((int64_t)row * a.ldw * 2);
    unsigned char* xreg = xs + wave * 16 * XPITCH;

    const int U = (K + 31) / 32;
    const int ub = (int)((int64_t)wave * U / WAVES);
    const int ue = (int)((int64_t)(wave + 1) * U / WAVES);
    const int kend = min(ue * 32, K);

    // wave 0 finishes the block: its bias words are requested now, ahead of the
    // weight stream, so their latency is not added after the last weight byte lands
    const int m = m0 + (lane & 15);
    const int nb = n0 + (lane >> 4) * 4;
    f32x4 bias = (f32x4){};
    if (MODE == kOutBias && wave == 0) bias = load_bias4<E>(a, nb);
    Extras4 ex{};
    if (MODE == kOutEpi && wave == 0) ex = epi_prefetch4(a, m, nb);
    __builtin_amdgcn_sched_barrier(0);

    f32x4 acc = (f32x4){};
    for (int u0 = ub; u0 < ue; u0 += PU) {
        // x rows j < mv: halves [32 u0 + 8 lane, +8) of each row, zero past kend
        const int kx = u0 * 32 + lane * 8;
        for (int j = 0; j < mv; ++j) {
            const uint32_t off = kx < kend ? (uint32_t)(((int64_t)j * a.ldx + kx) * 2) : kOOB;
            lds_dma16(rx, xreg + j * XPITCH, off);
        }
        u32x4 wa[PU];
#pragma unroll
        for (int s = 0; s < PU; ++s) {
            const int k = ((u0 + s) * 4 + grp) * 8;
            wa[s] = load16(rw, k < kend ? wrow + 2u * (uint32_t)k : kOOB);
        }
        __builtin_amdgcn_sched_barrier(0);
        // the x copies were issued before the PU weight loads: wait for them alone
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PU) : "memory");
#pragma unroll
        for (int s = 0; s < PU; ++s) {
            const int k = ((u0 + s) * 4 + grp) * 8;
            // rows past M and K past the range contribute zero (masked, not branched)
            const uint32_t keep = (row < mv && k < kend) ? 0xffffffffu : 0u;
            u32x4 xv = *(const u32x4*)(xreg + row * XPITCH + (s * 4 + grp) * 16);
            xv &= (u32x4){keep, keep, keep, keep};
            acc = mfma16x16x32<E>(wa[s], xv, acc);
        }
        // every LDS read of this pass has been consumed by an MFMA above, so the
        // next pass may overwrite the region
    }

    red[wave][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
    f32x4 s = red[0][lane];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) s += red[w][lane];

    // Accumulator layout: lane l holds column m = l % 16 and rows n = 4 (l / 16) + e.
    if constexpr (MODE == kOutEpi) {
        uint16_t o[4] = {narrow<E>(s[0]), narrow<E>(s[1]), narrow<E>(s[2]), narrow<E>(s[3])};
        epi_apply4<E>(a.epi, o, ex);
        if (m < a.M) store4_words(a, m, nb, o);
    } else {
        if (m < a.M) store4<E, MODE>(a, m, nb, s[0], s[1], s[2], s[3], bias);
    }
}

template <int WAVES, int E, int MODE>
__global__ void __launch_bounds__(WAVES * 64)
skinny_kernel(LinearArgs a) {
    enter_group<MODE>(a);
    constexpr int UNROLL = 8;
    const int n0 = blockIdx.x * 16, m0 = blockIdx.y * 16;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row = lane & 15, grp = lane >> 4;
    const int K = a.K;

    const __amdgpu_buffer_rsrc_t rw = matrix_rsrc(a.w, n0, a.N, a.ldw, K);
    const __amdgpu_buffer_rsrc_t rx = matrix_rsrc(a.x, m0, a.M, a.ldx, K);
    const uint32_t wrow = (uint32_t)((int64_t)row * a.ldw * 2);
    const uint32_t xrow = (uint32_t)((int64_t)row * a.ldx * 2);
    const bool w_ok = n0 + row < a.N, x_ok = m0 + row < a.M;

    const int U = (K + 31) / 32;
    const int ub = (int)((int64_t)wave * U / WAVES);
    const int ue = (int)((int64_t)(wave + 1) * U / WAVES);

    const int m = m0 + (lane & 15);
    const int nb = n0 + (lane >> 4) * 4;
    f32x4 bias = (f32x4){};
    if (MODE == kOutBias && wave == 0) bias = load_bias4<E>(a, nb);
    Extras4 ex{};
    if (MODE == kOutEpi && wave == 0) ex = epi_prefetch4(a, m, nb);

    f32x4 acc = (f32x4){};
    for (int u = ub; u < ue; u += UNROLL) {
        u32x4 wa[UNROLL], xb[UNROLL];
#pragma unroll
        for (int s = 0; s < UNROLL; ++s) {
            const int k = ((u + s) * 4 + grp) * 8;   // first K of this lane's chunk
            const bool in = (u + s) < ue;
            wa[s] = load8_masked(rw, wrow + 2u * (uint32_t)k, k, in ? K : 0, w_ok);
            xb[s] = load8_masked(rx, xrow + 2u * (uint32_t)k, k, in ? K : 0, x_ok);
        }
#pragma unroll
        for (int s = 0; s < UNROLL; ++s)
            acc = mfma16x16x32<E>(wa[s], xb[s], acc);
    }

    __shared__ f32x4 red[WAVES][64];
    red[wave][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
    f32x4 s = red[0][lane];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) s += red[w][lane];

    // Accumulator layout: lane l holds column m = l % 16 and rows n = 4 (l / 16) + e.
    if constexpr (MODE == kOutEpi) {
        uint16_t o[4] = {narrow<E>(s[0]), narrow<E>(s[1]), narrow<E>(s[2]), narrow<E>(s[3])};
        epi_apply4<E>(a.epi, o, ex);
        if (m < a.M) store4_words(a, m, nb, o);
    } else {
        if (m < a.M) store4<E, MODE>(a, m, nb, s[0], s[1], s[2], s[3], bias);
    }
}

// v + (v of lane CTRL's source) on every lane, by a DPP operand (no LDS trip).
template <int CTRL>
__device__ inline float dpp_add(float v) {
    return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf,
                                                                    false));
}

__device__ inline float lane_value(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// The sum of v over the wave's 64 lanes, in one fixed order of FP32 additions:
// pairs, then quads (quad permutations), then the two halves of each row of 8
// and the two halves of each row of 16 (mirrors), then the four row sums in
// order.  Each step adds a lane's value to a partner's, and FP32 addition is
// commutative, so every lane of a group ends with the same bits.  Against the
// butterfly through LDS permutes (six round trips) this takes 0.2 us off the
// M = 1 decode launch.
__device__ inline float wave_sum(float v) {
    v = dpp_add<0xB1>(v);     // quad_perm [1, 0, 3, 2]
    v = dpp_add<0x4E>(v);     // quad_perm [2, 3, 0, 1]
    v = dpp_add<0x141>(v);    // row_half_mirror
    v = dpp_add<0x140>(v);    // row_mirror
    return ((lane_value(v, 0) + lane_value(v, 16)) + lane_value(v, 32)) + lane_value(v, 48);
}

template <int E, int MODE>
__global__ void __launch_bounds__(kGemvRows * 64)
gemv_stream(LinearArgs a) {
    constexpr int U = 8;                      // segments (1 KB loads per wave) in flight per pass
    extern __shared__ __attribute__((aligned(16))) unsigned char xs_row[];   // x: K * 2 bytes
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);        // uniform
    const int n = blockIdx.x * kGemvRows + wave;
    const int K = a.K;
    const int S = (K + kGemvSeg - 1) / kGemvSeg;
    const __amdgpu_buffer_rsrc_t rx = matrix_rsrc(a.x, 0, 1, a.ldx, K);
    const __amdgpu_buffer_rsrc_t rw = matrix_rsrc(a.w, n < a.N ? n : a.N, a.N, a.ldw, K);   // empty past N
    // the bias word, requested first and widened only at the end (zero past N)
    uint32_t bword = 0;
    if constexpr (MODE == kOutBias) {
        const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc((void*)a.b, (short)0, a.N * 2, kRsrcWord3);
        bword = __builtin_amdgcn_raw_buffer_load_b16(rb, (uint32_t)n * 2u, 0, 0);
    }
    // x into LDS, segment s by wave s % kGemvRows
    for (int s = wave; s < S; s += kGemvRows) {
        const int k = s * kGemvSeg + lane * 8;
        lds_dma16(rx, xs_row + s * 1024, k < K ? (uint32_t)k * 2u : kOOB);
    }
    float sums[U] = {};
    for (int p = 0; p < S; p += U) {
        u32x4 wv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = (p + u) * kGemvSeg + lane * 8;
            wv[u] = load16(rw, (p + u < S && k < K) ? (uint32_t)k * 2u : kOOB);
        }
        __builtin_amdgcn_sched_barrier(0);    // every load of the pass in flight before any use
        if (p == 0) {
            // this wave's x copies were issued before the weight loads: wait for
            // them alone, then for every wave's
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(U) : "memory");
            lds_barrier();
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = p + u;
            // a segment past K has zero weights (out-of-range loads): any x will do
            const u32x4 xv = *(const u32x4*)(xs_row + (s < S ? s : S - 1) * 1024 + lane * 16);
            float acc = sums[u];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc = __builtin_fmaf(widen<E>((uint16_t)wv[u][q]), widen<E>((uint16_t)xv[q]), acc);
                acc = __builtin_fmaf(widen<E>((uint16_t)(wv[u][q] >> 16)), widen<E>((uint16_t)(xv[q] >> 16)), acc);
            }
            sums[u] = acc;
        }
    }
    float acc = sums[0];
#pragma unroll
    for (int u = 1; u < U; ++u) acc += sums[u];
    acc = wave_sum(acc);
    if (lane != 0 || n >= a.N) return;
    if constexpr (MODE == kOutF32) {
        ((float*)a.y)[n] = acc;
    } else {
        uint16_t t = narrow<E>(acc);
        if constexpr (MODE == kOutBias) t = narrow<E>(widen<E>(t) + widen<E>((uint16_t)bword));
        ((uint16_t*)a.y)[n] = t;
    }
}

template <int E>
static const void* gemv_fn(int mode) {
    if (mode == kOutBias) return (const void*)gemv_stream<E, kOutBias>;
    if (mode == kOutRound) return (const void*)gemv_stream<E, kOutRound>;
    return (const void*)gemv_stream<E, kOutF32>;
}

hipError_t launch_gemv(int elem, const LinearArgs& a, int mode, hipStream_t stream) {
    if (a.M != 1 || a.groups > 1 || mode == kOutEpi || a.K > kGemvMaxK) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((a.N + kGemvRows - 1) / kGemvRows)), block(kGemvRows * 64);
    LinearArgs args = a;
    void* params[] = {&args};
    const void* fn = elem == kBF16 ? gemv_fn<kBF16>(mode) : gemv_fn<kF16>(mode);
    const size_t lds = (size_t)((a.K + kGemvSeg - 1) / kGemvSeg) * 1024;
    return hipLaunchKernel(fn, grid, block, params, lds, stream);
}

template <int E>
static const void* skinny_fn(bool vec, int mode) {
    if (vec) {
        if (mode == kOutBias) return (const void*)skinny_stream<kSkinnyWaves, E, kOutBias>;
        if (mode == kOutRound) return (const void*)skinny_stream<kSkinnyWaves, E, kOutRound>;
        if (mode == kOutEpi) return (const void*)skinny_stream<kSkinnyWaves, E, kOutEpi>;
        return (const void*)skinny_stream<kSkinnyWaves, E, kOutF32>;
    }
    if (mode == kOutBias) return (const void*)skinny_kernel<kSkinnyWaves, E, kOutBias>;
    if (mode == kOutRound) return (const void*)skinny_kernel<kSkinnyWaves, E, kOutRound>;
    if (mode == kOutEpi) return (const void*)skinny_kernel<kSkinnyWaves, E, kOutEpi>;
    return (const void*)skinny_kernel<kSkinnyWaves, E, kOutF32>;
}

hipError_t launch_skinny(int elem, const LinearArgs& a, bool vec, int mode, hipStream_t stream) {
    const dim3 grid((unsigned)((a.N + 15) / 16), (unsigned)((a.M + 15) / 16), (unsigned)a.groups);
    const dim3 block(kSkinnyWaves * 64);
    LinearArgs args = a;
    void* params[] = {&args};
    const void* fn = elem == kBF16 ? skinny_fn<kBF16>(vec, mode) : skinny_fn<kF16>(vec, mode);
    return hipLaunchKernel(fn, grid, block, params, 0, stream);
}

}  // namespace lin
