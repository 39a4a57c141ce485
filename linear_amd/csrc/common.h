// common.h -- types and small device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lin {

typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// The steps of a multi-step contraction epilogue, applied in order to the
// rounded projection, each result rounded to the element type.
constexpr int kEpiMaxSteps = 8;
enum : int { kEpiBias = 1, kEpiResidual = 2, kEpiMul = 3, kEpiSilu = 4, kEpiGeluTanh = 5, kEpiGeluErf = 6 };
constexpr int kActWords = 65536;   // one table entry per 16-bit input word

struct EpiArgs {
    const uint16_t* bias;   // [N]
    const uint16_t* res;    // [M, N], row stride ldr
    const uint16_t* mul;    // [M, N], row stride ldm
    const uint16_t* act;    // this element type's tables: SiLU, tanh GeLU, erf GeLU (3 x kActWords)
    int64_t ldr, ldm;
    int nsteps;
    uint64_t ops;           // step s in byte s (packed: a kernel indexes no array of its arguments,
                            // which would move a modified argument copy to scratch memory)
    int vec16;              // bits: 1 y, 2 bias, 4 res, 8 mul allow 16-byte (8-word) accesses
};

__host__ __device__ inline int epi_op(const EpiArgs& ep, int s) { return (int)((ep.ops >> (8 * s)) & 0xff); }

// Arguments of one linear-layer launch.  Pointers are device pointers to 16-bit
// words (binary16 or bfloat16, per the kernel's element type); y holds 16-bit
// words or, in the FP32-output mode, floats.  Strides in elements.
struct LinearArgs {
    const uint16_t* x;   // [M, K], row stride ldx
    const uint16_t* w;   // [N, K], row stride ldw
    const uint16_t* b;   // [N] or nullptr
    void* y;             // [M, N], row stride ldy
    int64_t ldx, ldw, ldy;
    int M, N, K;
    int tiles_m, tiles_n;
    int vec_store;       // 1: y aligned for 4-element vector stores and ldy % 4 == 0
    EpiArgs epi;         // the epilogue program (kOutEpi only)
    int64_t gsx, gsy;    // grouped calls (gridDim.z groups): x and y group strides in elements
    int groups;          // gridDim.z (1 for ungrouped calls)
    int xcd_shift;       // log2 of the device's XCD count (workgroup ids are dealt round-robin over them)
};


// Element types of x, weight, b and (rounded) y.
enum : int { kF16 = 0, kBF16 = 1 };

// Output modes: round the FP32 sum to the element type and add the bias (then
// round again); round only; store the FP32 sum itself; or round and run the
// epilogue program of a.epi.
enum : int { kOutBias = 0, kOutRound = 1, kOutF32 = 2, kOutEpi = 3 };

// Grouped contraction: group g is the activation slice x + g * gsx, the weight
// block of rows g * N .. g * N + N - 1, y + g * gsy and the bias words g * N ..
template <int MODE>
__device__ inline void enter_group_at(LinearArgs& a, int64_t g) {
    if (g == 0) return;
    a.x += g * a.gsx;
    a.w += g * (int64_t)a.N * a.ldw;
    a.y = (void*)((char*)a.y + g * a.gsy * (MODE == kOutF32 ? 4 : 2));
    if (a.b) a.b += g * (int64_t)a.N;
}

// Workgroup z handles group z (no-op for ungrouped launches, gridDim.z == 1).
template <int MODE>
__device__ inline void enter_group(LinearArgs& a) {
    enter_group_at<MODE>(a, blockIdx.z);
}

// Word 3 of a gfx9 buffer resource: 32-bit data format, no swizzle, no stride.
constexpr uint32_t kRsrcWord3 = 0x00020000u;
// A byte offset that is never inside a resource: every resource built here has
// num_records <= 0x7fffffff, so a load at this offset returns zero.
constexpr uint32_t kOOB = 0x80000000u;

// Buffer resource over the rows [row0, rows) of a row-major binary16 matrix with
// row stride ld and K valid columns; rows at or past `rows` read as zero.
__device__ inline __amdgpu_buffer_rsrc_t matrix_rsrc(const uint16_t* base, int64_t row0, int64_t rows,
                                                     int64_t ld, int64_t K) {
    int64_t left = rows - row0;
    int64_t bytes = left > 0 ? ((left - 1) * ld + K) * 2 : 0;
    if (bytes > 0x7fffffff) bytes = 0x7fffffff;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + row0 * ld), (short)0, (int)bytes, kRsrcWord3);
}

__device__ inline u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

typedef __attribute__((address_space(3))) void lds_void;

// Direct-to-LDS load: each lane's 16 bytes at byte offset `off` of the resource
// land at lds + 16 * lane (lds must be the same for the whole wave).  Out-of-range
// offsets deliver zeros.  Kept out of lambdas: inside one, the host compilation
// pass drops the enclosing kernel's launch stub.
__device__ inline void lds_dma16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, off, 0, 0, 0);
}

// Workgroup barrier for slices handed over in LDS by direct-to-LDS loads.
// __syncthreads() orders every earlier LDS write before the barrier, and direct
// loads count as LDS writes, so the compiler puts a wait for all of them (vmcnt
// 0) in front of it, including loads of later slices.  Here each wave has already
// waited for the loads the next slice needs (an explicit vmcnt), so only its own
// LDS reads are drained (lgkmcnt 0: a slot may be refilled after the barrier);
// the memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Eight consecutive binary16 elements starting at byte offset `off`, element e
// replaced by zero when k0 + e >= K (element-wise loader for unaligned layouts).
__device__ inline u32x4 load8_masked(__amdgpu_buffer_rsrc_t r, uint32_t off, int k0, int K, bool row_ok) {
    uint16_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        uint32_t o = (row_ok && k0 + e < K) ? off + 2u * e : kOOB;
        h[e] = __builtin_amdgcn_raw_buffer_load_b16(r, o, 0, 0);
    }
    u32x4 v;
    v.x = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
    v.y = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
    v.z = (uint32_t)h[4] | ((uint32_t)h[5] << 16);
    v.w = (uint32_t)h[6] | ((uint32_t)h[7] << 16);
    return v;
}

__device__ inline f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }

__device__ inline f16 bits_to_f16(uint16_t u) { return __builtin_bit_cast(f16, u); }
__device__ inline uint16_t f16_to_bits(f16 h) { return __builtin_bit_cast(uint16_t, h); }

// Exact widening of a 16-bit word of element type E to FP32.
template <int E>
__device__ inline float widen(uint16_t u) {
    if (E == kF16) return (float)bits_to_f16(u);
    return __builtin_bit_cast(float, (uint32_t)u << 16);
}

// Round an FP32 value to element type E, round to nearest even (v_cvt_f16_f32 /
// v_cvt_pk_bf16_f32 under the default rounding mode, subnormals kept).
template <int E>
__device__ inline uint16_t narrow(float v) {
    if (E == kF16) return f16_to_bits((f16)v);
    return __builtin_bit_cast(uint16_t, (__bf16)v);
}

// One MFMA step on raw 16-byte operand fragments: FP32 accumulation of exact
// products (binary16 x binary16 and bfloat16 x bfloat16 products are exact in FP32).
template <int E>
__device__ inline f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
    if (E == kF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <int E>
__device__ inline f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    if (E == kF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// The epilogue of the contract for four consecutive output columns nb..nb+3 of
// row m, and the store.  Rounded modes: round each FP32 sum to E (round to
// nearest even); with a bias, widen the rounded value and b[n] to FP32, add, and
// round the sum to E.  FP32 mode: store the sums unrounded.  Columns past N are
// skipped; rows are checked by the caller.
// The epilogue program on one rounded projection word t at (m, n).  Additions and
// the multiply run in FP32 on exactly widened operands and round to E once: FP32
// carries at least 2p + 2 significant bits for p = 11 (binary16) and 8
// (bfloat16), so that equals rounding the exact sum or product.  An activation
// step reads its table: the library's correctly rounded composition for every
// input word.
template <int E>
__device__ inline uint16_t epi_apply(const EpiArgs& ep, uint16_t t, int m, int n) {
    for (int s = 0; s < ep.nsteps; ++s) {
        const int op = epi_op(ep, s);
        if (op == kEpiBias) t = narrow<E>(widen<E>(t) + widen<E>(ep.bias[n]));
        else if (op == kEpiResidual) t = narrow<E>(widen<E>(t) + widen<E>(ep.res[(int64_t)m * ep.ldr + n]));
        else if (op == kEpiMul) t = narrow<E>(widen<E>(t) * widen<E>(ep.mul[(int64_t)m * ep.ldm + n]));
        else t = ep.act[(op - kEpiSilu) * kActWords + t];
    }
    return t;
}

// Word-wise on 8 packed words: a binary step (R(W(x) + W(y)) or R(W(x) * W(y)))
// or a table lookup.
template <int E, bool MUL>
__device__ inline u32x4 binop8(u32x4 x, u32x4 y) {
    u32x4 r;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint32_t out = 0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float a = widen<E>((uint16_t)(x[q] >> (16 * h))), b = widen<E>((uint16_t)(y[q] >> (16 * h)));
            out |= (uint32_t)narrow<E>(MUL ? a * b : a + b) << (16 * h);
        }
        r[q] = out;
    }
    return r;
}

// The activation-table window that the GEMM epilogue copies into LDS: for each
// sign, the 8192 consecutive words from exponent field kActWinExp<E> on, i.e.
// |x| in [2^-7, 2) for binary16 and [2^-40, 2^24) for bfloat16, 32 KB in all.
// Entry (x >> 15) * 8192 + (x & 0x7fff) - (kActWinExp << mantissa bits) holds
// the table's word for x; other words are read from the table in global memory.
constexpr int kActWinWords = 16384;
template <int E> constexpr int kActWinExp = E == kF16 ? 8 : 87;
template <int E> constexpr uint32_t kActWinBase = (uint32_t)kActWinExp<E> << (E == kF16 ? 10 : 7);

typedef __attribute__((address_space(3))) const uint16_t lds_u16;

// Buffer resource over one activation table (kActWords words).
__device__ inline __amdgpu_buffer_rsrc_t table_rsrc(const uint16_t* tab) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)tab, (short)0, kActWords * 2, kRsrcWord3);
}

// Lookups through the window: the table's word for x comes from the LDS window
// when the window holds x, else from the table in global memory.  Both reads
// are issued for every word and neither is branched: the LDS read at its sign's
// first entry when the window misses, the buffer load at an out-of-range offset
// (zero, no memory traffic) when it hits.  (A select of the two addresses as
// one generic pointer had the compiler wait after every two lookups.)
// The table's words for CH chunks of 8 packed words: every read issued first,
// then (past a scheduling barrier) the selects, so that the compiler cannot
// consume each lookup as it goes.  win: the LDS window, or null for none (all
// words from the table in global memory).
template <int E, int CH>
__device__ inline void lookup_chunks(lds_u16* win, __amdgpu_buffer_rsrc_t rt, u32x4 (&t)[CH]) {
    uint32_t w[CH][8], g[CH][8];
#pragma unroll
    for (int k = 0; k < CH; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t x = (t[k][e >> 1] >> (16 * (e & 1))) & 0xffffu;
            if (win) {
                const uint32_t d = (x & 0x7fffu) - kActWinBase<E>;
                const bool in = d < 8192u;
                w[k][e] = win[((x >> 15) << 13) | (in ? d : 0u)];
                g[k][e] = __builtin_amdgcn_raw_buffer_load_b16(rt, in ? kOOB : 2u * x, 0, 0);
            } else {
                g[k][e] = __builtin_amdgcn_raw_buffer_load_b16(rt, 2u * x, 0, 0);
            }
        }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < CH; ++k)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t v[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int e = 2 * q + h;
                const uint32_t x = (t[k][q] >> (16 * h)) & 0xffffu;
                const bool in = win && ((x & 0x7fffu) - kActWinBase<E>) < 8192u;
                v[h] = in ? w[k][e] : g[k][e];
            }
            t[k][q] = v[0] | (v[1] << 16);
        }
}

// 8 consecutive words src[0..7] of a row, the valid ones only (col + e < N,
// row valid); 16-byte load when allowed.
__device__ inline u32x4 load8(const uint16_t* src, bool row_ok, int col, int N, bool vec) {
    if (row_ok && vec && col + 7 < N) return *(const u32x4*)src;
    u32x4 r = (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e)
        if (row_ok && col + e < N) r[e >> 1] |= (uint32_t)src[e] << (16 * (e & 1));
    return r;
}

__device__ inline void store8(uint16_t* dst, bool row_ok, int col, int N, bool vec, u32x4 v) {
    if (!row_ok) return;
    if (vec && col + 7 < N) {
        *(u32x4*)dst = v;
        return;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
        if (col + e < N) dst[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
}

// The epilogue inputs of four consecutive outputs (m, nb..nb+3), for kernels that
// request them before their main loop (only those the program reads; zero for
// outputs past M or N).
struct Extras4 {
    uint16_t b[4], r[4], u[4];
};

__device__ inline Extras4 epi_prefetch4(const LinearArgs& a, int m, int nb) {
    const EpiArgs& ep = a.epi;
    bool ub = false, ur = false, uu = false;
    for (int s = 0; s < ep.nsteps; ++s) {
        ub |= epi_op(ep, s) == kEpiBias;
        ur |= epi_op(ep, s) == kEpiResidual;
        uu |= epi_op(ep, s) == kEpiMul;
    }
    Extras4 x;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const bool col = nb + e < a.N, ok = col && m < a.M;
        x.b[e] = (ub && col) ? ep.bias[nb + e] : 0;
        x.r[e] = (ur && ok) ? ep.res[(int64_t)m * ep.ldr + nb + e] : 0;
        x.u[e] = (uu && ok) ? ep.mul[(int64_t)m * ep.ldm + nb + e] : 0;
    }
    return x;
}

// The program on four words with their inputs already loaded: the table lookups
// of an activation step are the only memory accesses, issued together.
template <int E>
__device__ inline void epi_apply4(const EpiArgs& ep, uint16_t t[4], const Extras4& x) {
    for (int s = 0; s < ep.nsteps; ++s) {
        const int op = epi_op(ep, s);
        if (op >= kEpiSilu) {
            const __amdgpu_buffer_rsrc_t rt = table_rsrc(ep.act + (op - kEpiSilu) * kActWords);
#pragma unroll
            for (int e = 0; e < 4; ++e) t[e] = __builtin_amdgcn_raw_buffer_load_b16(rt, 2u * t[e], 0, 0);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float v = widen<E>(t[e]);
                if (op == kEpiBias) t[e] = narrow<E>(v + widen<E>(x.b[e]));
                else if (op == kEpiResidual) t[e] = narrow<E>(v + widen<E>(x.r[e]));
                else t[e] = narrow<E>(v * widen<E>(x.u[e]));
            }
        }
    }
}

// Store four rounded words at (m, nb..nb+3), skipping columns past N.
__device__ inline void store4_words(const LinearArgs& a, int m, int nb, const uint16_t o[4]) {
    uint16_t* dst = (uint16_t*)a.y + (int64_t)m * a.ldy + nb;
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

// The bias words b[nb..nb+3] widened to FP32 (0 past N), for callers that load
// them before their main loop so the load latency is off the kernel's tail.
template <int E>
__device__ inline f32x4 load_bias4(const LinearArgs& a, int nb) {
    f32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = (nb + e < a.N) ? widen<E>(a.b[nb + e]) : 0.f;
    return r;
}

template <int E, int MODE>
__device__ inline void store4(const LinearArgs& a, int m, int nb, float v0, float v1, float v2, float v3,
                              f32x4 bias);

template <int E, int MODE>
__device__ inline void store4(const LinearArgs& a, int m, int nb, float v0, float v1, float v2, float v3) {
    f32x4 bias = (f32x4){};
    if (MODE == kOutBias) bias = load_bias4<E>(a, nb);
    store4<E, MODE>(a, m, nb, v0, v1, v2, v3, bias);
}

// As above with the widened bias words already loaded (ignored unless MODE is kOutBias).
template <int E, int MODE>
__device__ inline void store4(const LinearArgs& a, int m, int nb, float v0, float v1, float v2, float v3,
                              f32x4 bias) {
    const float v[4] = {v0, v1, v2, v3};
    if (MODE == kOutF32) {
        float* dst = (float*)a.y + (int64_t)m * a.ldy + nb;
        if (a.vec_store && nb + 3 < a.N) {
            *(f32x4*)dst = (f32x4){v0, v1, v2, v3};
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (nb + e < a.N) dst[e] = v[e];
        }
        return;
    }
    uint16_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        uint16_t p = narrow<E>(v[e]);
        if (MODE == kOutBias) p = narrow<E>(widen<E>(p) + bias[e]);
        if (MODE == kOutEpi) p = (nb + e < a.N) ? epi_apply<E>(a.epi, p, m, nb + e) : p;
        o[e] = p;
    }
    uint16_t* dst = (uint16_t*)a.y + (int64_t)m * a.ldy + nb;
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

}  // namespace lin
