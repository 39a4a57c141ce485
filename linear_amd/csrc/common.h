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

// Arguments of one linear-layer launch.  Pointers are device pointers to binary16
// words; strides in elements.
struct LinearArgs {
    const uint16_t* x;   // [M, K], row stride ldx
    const uint16_t* w;   // [N, K], row stride ldw
    const uint16_t* b;   // [N] or nullptr
    uint16_t* y;         // [M, N], row stride ldy
    int64_t ldx, ldw, ldy;
    int M, N, K;
    int tiles_m, tiles_n;
    int vec_store;       // 1: y 8-byte aligned and ldy % 4 == 0
};

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

// The epilogue of the contract for one accumulator value: round the FP32 sum to
// FP16 (round to nearest even), then, with a bias, widen both to FP32, add, and
// round the sum to FP16.
template <bool BIAS>
__device__ inline uint16_t finish(float acc, float bias) {
    f16 p = (f16)acc;
    if (BIAS) {
        f16 yv = (f16)((float)p + bias);
        return f16_to_bits(yv);
    }
    return f16_to_bits(p);
}

}  // namespace lin
