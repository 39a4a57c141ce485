// probe.hip -- measurement kernels for the benchmark's ceilings (not part of the
// linear-layer ABI; built into liblinear_probe.so, loaded only by bench.py).
//
//  - probe_read: a plain streaming read of a buffer with the decode kernel's grid
//    (workgroups x 512 threads, 16-byte loads, every load of a thread in flight at
//    once), the bytes per second that any kernel reading that buffer can reach.
//  - probe_empty: a kernel that does nothing, on the same grid: the per-launch
//    floor inside a HIP graph.
//  - probe_mfma: v_mfma_f32_32x32x16_f16 on register operands only (no memory
//    traffic inside the loop), the matrix-core rate this part sustains on real
//    data at its power-limited clock.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 512;
constexpr int kUnroll = 16;   // loads per thread in flight at once

// Workgroup g reads 16-byte chunks [g * per, (g + 1) * per); thread t reads
// chunks t, t + 512, ... of that range, kUnroll at a time.  per is a multiple of
// 512 * kUnroll (checked on the host).  The XOR of everything read goes to
// sink[g] so the loads cannot be removed.
__global__ void __launch_bounds__(kThreads) probe_read_kernel(const u32x4* src, int64_t per, uint32_t* sink) {
    const u32x4* p = src + (int64_t)blockIdx.x * per + threadIdx.x;
    u32x4 acc = (u32x4){0u, 0u, 0u, 0u};
    for (int64_t i = 0; i < per; i += (int64_t)kThreads * kUnroll) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = p[i + (int64_t)u * kThreads];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
    }
    const uint32_t r = acc.x ^ acc.y ^ acc.z ^ acc.w;
    __shared__ uint32_t red[kThreads / 64];
    uint32_t w = r;
    for (int o = 32; o > 0; o >>= 1) w ^= __shfl_xor(w, o);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = w;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t s = 0;
        for (int i = 0; i < kThreads / 64; ++i) s ^= red[i];
        sink[blockIdx.x] = s;
    }
}

__global__ void __launch_bounds__(kThreads) probe_empty_kernel() {}

// Each wave keeps 4 independent accumulators and runs `iters` rounds of 8 MFMAs
// on operands loaded once from `ops` (random binary16 data: the matrix unit's
// power, hence the clock, depends on the operand bits).  Writes its accumulators
// to out (16 floats x 4 per lane).
__global__ void __launch_bounds__(256) probe_mfma_kernel(const u32x4* ops, int iters, float* out) {
    const int lane = threadIdx.x & 63;
    const int64_t gw = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6));
    u32x4 a0 = ops[(gw * 4 + 0) % 4096 * 64 + lane];
    u32x4 a1 = ops[(gw * 4 + 1) % 4096 * 64 + lane];
    u32x4 b0 = ops[(gw * 4 + 2) % 4096 * 64 + lane];
    u32x4 b1 = ops[(gw * 4 + 3) % 4096 * 64 + lane];
    f32x16 c0 = (f32x16){}, c1 = (f32x16){}, c2 = (f32x16){}, c3 = (f32x16){};
    const f16x8 A0 = __builtin_bit_cast(f16x8, a0), A1 = __builtin_bit_cast(f16x8, a1);
    const f16x8 B0 = __builtin_bit_cast(f16x8, b0), B1 = __builtin_bit_cast(f16x8, b1);
    for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(A0, B0, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(A0, B1, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(A1, B0, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(A1, B1, c3, 0, 0, 0);
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(A1, B1, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(A1, B0, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(A0, B1, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(A0, B0, c3, 0, 0, 0);
    }
    float* o = out + (gw * 64 + lane) * 64;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        o[e] = c0[e];
        o[16 + e] = c1[e];
        o[32 + e] = c2[e];
        o[48 + e] = c3[e];
    }
}

}  // namespace

extern "C" {

// Bytes read per call: grid * per * 16.  Returns 0, or -1 for a shape the kernel
// does not take (bytes not a multiple of grid * 512 * 16 * kUnroll), or the HIP error.
int32_t probe_read(const void* src, int64_t bytes, int32_t grid, uint32_t* sink, void* stream) {
    const int64_t unit = (int64_t)grid * kThreads * kUnroll * 16;
    if (!src || !sink || grid <= 0 || bytes <= 0 || bytes % unit != 0) return -1;
    hipLaunchKernelGGL(probe_read_kernel, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                       (const u32x4*)src, bytes / 16 / grid, sink);
    return (int32_t)hipGetLastError();
}

int32_t probe_empty(int32_t grid, void* stream) {
    if (grid <= 0) return -1;
    hipLaunchKernelGGL(probe_empty_kernel, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream);
    return (int32_t)hipGetLastError();
}

// ops: 4096 * 64 16-byte words (4 MiB) of operand data; out: grid * 4 * 64 * 64
// floats.  FLOPs per call: grid * 4 waves * iters * 8 MFMAs * 32768.
int32_t probe_mfma(const void* ops, int32_t grid, int32_t iters, float* out, void* stream) {
    if (!ops || !out || grid <= 0 || iters <= 0) return -1;
    hipLaunchKernelGGL(probe_mfma_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const u32x4*)ops,
                       iters, out);
    return (int32_t)hipGetLastError();
}

}  // extern "C"
