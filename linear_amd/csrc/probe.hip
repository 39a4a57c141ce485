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
//  - probe_loads: the streaming GEMM's operand loads alone (its tile, its ring of
//    64-wide K slices, its direct-to-LDS loads, waits, barriers and XCD tile walk,
//    no fragment reads and no MFMAs): how fast the operands of a tile reach a CU.
//  - probe_mfma_lds: the 256 x 256 tile's MFMAs fed from LDS with no operand loads
//    from memory: 8 waves of 128 x 64, each 32-wide K step's 12 fragments read
//    from a two-slot ring of 64-wide slices (filled once with random binary16
//    data, the streaming GEMM's swizzle, so the reads are free of bank conflicts)
//    while the previous step's 32 v_mfma_f32_16x16x32_f16 run, and a barrier per
//    slice: what the tile's matrix work costs once its operands are in LDS.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

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

// Tile t of a tiles_m x tiles_n grid for workgroup bid: workgroups are dealt
// round-robin over 2^xcd_shift XCDs, each XCD takes a contiguous run of tiles,
// walked 4 tile-rows at a time (the streaming GEMM's order).
__device__ inline void probe_tile(int bid, int tiles_m, int tiles_n, int xcd_shift, int& tm, int& tn) {
    const int G = tiles_m * tiles_n, xmask = (1 << xcd_shift) - 1;
    const int xcd = bid & xmask, idx = bid >> xcd_shift;
    const int q = G >> xcd_shift, r = G & xmask;
    const int t = (xcd < r) ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
    const int per_group = 4 * tiles_n, g = t / per_group, first_m = g * 4;
    const int gm = min(tiles_m - first_m, 4), rem = t - g * per_group;
    tm = first_m + rem % gm;
    tn = rem / gm;
}

typedef __attribute__((address_space(3))) void lds_void;

// The operand loads of a BM x BN tile over all of K (a multiple of 64): slice s
// (64 K values, 128 bytes of each of the tile's BN weight rows and BM x rows) goes
// into LDS slot s % STAGES as (BM + BN) / 8 direct loads of 8 rows x 128 bytes.
// Slices 0 .. STAGES-1 are requested at once; slot s - 1 is refilled with slice
// s - 1 + STAGES once slice s has landed in every wave (wait, then barrier), as
// the GEMM refills a slot after the barrier that follows its last reads.  Only
// slices that exist are requested.  One LDS word per workgroup goes to sink.
template <int BM, int BN, int NW, int STAGES>
__global__ void __launch_bounds__(NW * 64) probe_loads_kernel(const uint16_t* x, const uint16_t* w, int M, int N,
                                                              int K, int xcd_shift, uint32_t* sink) {
    constexpr int SLICE = (BM + BN) * 128, GPW = (BM + BN) / 8 / NW;
    static_assert((BM + BN) / 8 % NW == 0 && STAGES * SLICE <= 160 * 1024, "probe tile");
    __shared__ __attribute__((aligned(1024))) unsigned char smem[STAGES * SLICE];
    int tm, tn;
    probe_tile(blockIdx.x, M / BM, N / BN, xcd_shift, tm, tn);
    const int64_t bytes_w = (int64_t)BN * K * 2, bytes_x = (int64_t)BM * K * 2;
    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc((void*)(w + (int64_t)tn * BN * K), (short)0, (int)bytes_w, 0x00020000);
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc((void*)(x + (int64_t)tm * BM * K), (short)0, (int)bytes_x, 0x00020000);
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nk = K / 64;
    auto issue = [&](int s) {
        unsigned char* slot = smem + (s % STAGES) * SLICE;
#pragma unroll
        for (int j = 0; j < GPW; ++j) {
            const int g = wave * GPW + j;
            const bool isw = g < BN / 8;
            const int r = (isw ? g : g - BN / 8) * 8 + lane / 8;
            const uint32_t off = (uint32_t)(((int64_t)r * K + s * 64 + (lane % 8) * 8) * 2);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(isw ? rw : rx, (lds_void*)(slot + g * 1024), 16, off, 0, 0, 0);
        }
    };
    // at most c (< STAGES) slices' loads left in flight
    auto wait_behind = [&](int c) {
        if (c <= 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        else if (c == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(GPW) : "memory");
        else if (c == 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * GPW) : "memory");
        else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * GPW) : "memory");
    };
    static_assert(STAGES <= 4 && 3 * GPW < 64, "waits cover rings of up to 4 slots");
    const int pro = nk < STAGES ? nk : STAGES;
    for (int s = 0; s < pro; ++s) issue(s);
    wait_behind(pro - 1);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    for (int t = 1; t < nk; ++t) {
        wait_behind(min(STAGES - 2, nk - 1 - t));
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (t - 1 + STAGES < nk) issue(t - 1 + STAGES);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = *(const uint32_t*)(smem + ((nk - 1) % STAGES) * SLICE);
}

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


// One 256 x 256 tile's K loop with its operands already in LDS.  LDS holds two
// slots of a 64-wide K slice: 256 weight rows then 256 x rows of 128 bytes, the
// 16-byte chunk c of row r at chunk c ^ ((r / 2) % 8).  Wave (wm, wn) of the 2 x 4
// grid owns x rows wm * 128 .. +128 and weight rows wn * 64 .. +64: per 32-wide K
// step it reads 4 weight and 8 x fragments (lane l: row l % 16, chunk 4 step +
// l / 16) and runs 32 v_mfma_f32_16x16x32_f16, as the layer's 256 x 256 tile
// does; the next step's fragments are read while this step's MFMAs run.  nk
// slices, a barrier after each.  Each lane's accumulators are added into
// out[blockIdx.x * 512 + threadIdx.x].
__global__ void __launch_bounds__(512) probe_mfma_lds_kernel(const u32x4* ops, int nk, float* out) {
    constexpr int SLICE = 512 * 128;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * SLICE];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = wave & 3, wm = wave >> 2;
    // fill both slots: 8192 chunks of 16 bytes, 16 per thread
    for (int i = 0; i < 16; ++i) {
        const int q = tid * 16 + i;
        *(u32x4*)(smem + q * 16) = ops[((int64_t)blockIdx.x * 8192 + q) % (4096 * 64)];
    }
    __syncthreads();
    auto frag = [&](int slot, int row, int step) -> f16x8 {
        const int c = 4 * step + (lane >> 4);
        const int r = row + (lane & 15);
        return __builtin_bit_cast(f16x8, *(const u32x4*)(smem + slot * SLICE + r * 128 + ((c ^ ((r >> 1) & 7)) << 4)));
    };
    f32x4 acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = (f32x4){};
    f16x8 a[2][4], b[2][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[0][i] = frag(0, wn * 64 + i * 16, 0);
#pragma unroll
    for (int j = 0; j < 8; ++j) b[0][j] = frag(0, 256 + wm * 128 + j * 16, 0);
    for (int t = 0; t < nk; ++t) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int cur = ks & 1, nxt = cur ^ 1;
            // the next step's fragments (the next slice's first step after the last)
            const int nslot = ks < 1 ? (t & 1) : ((t + 1) & 1);
            const int nstep = (ks + 1) & 1;
#pragma unroll
            for (int i = 0; i < 4; ++i) a[nxt][i] = frag(nslot, wn * 64 + i * 16, nstep);
#pragma unroll
            for (int j = 0; j < 8; ++j) b[nxt][j] = frag(nslot, 256 + wm * 128 + j * 16, nstep);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[cur][i], b[cur][j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) sum += acc[i][j][e];
    out[(int64_t)blockIdx.x * 512 + tid] = sum;
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

// The operand loads of the streaming GEMM's tile over x [M, K] and weight [N, K]
// (both row-major, 16-byte aligned, row stride K): tile 0 is 256 x 256 (8 waves,
// 2 slots), tile 1 is 64 x 64 (4 waves, 4 slots).  M and N must be multiples of
// the tile, K a positive multiple of 64 with 256 K * 2 bytes below 2 GiB; sink
// holds one word per tile.  The tile walk takes the current device's XCD count,
// as the library does.  Returns 0, -1 for a shape it does not take, or the HIP
// error.
int32_t probe_loads(const void* x, const void* w, int32_t M, int32_t N, int32_t K, int32_t tile, uint32_t* sink,
                    void* stream) {
    if (!x || !w || !sink || K <= 0 || K % 64 != 0 || (int64_t)256 * K * 2 >= ((int64_t)1 << 31)) return -1;
    int dev = 0, xcds = 1, xcd_shift = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    if (hipDeviceGetAttribute(&xcds, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || xcds < 1) xcds = 1;
    while ((2 << xcd_shift) <= xcds) ++xcd_shift;
    if ((1 << xcd_shift) != xcds) xcd_shift = 0;
    if (tile == 0) {
        if (M <= 0 || N <= 0 || M % 256 != 0 || N % 256 != 0) return -1;
        hipLaunchKernelGGL((probe_loads_kernel<256, 256, 8, 2>), dim3((M / 256) * (N / 256)), dim3(512), 0,
                           (hipStream_t)stream, (const uint16_t*)x, (const uint16_t*)w, M, N, K, xcd_shift, sink);
    } else if (tile == 1) {
        if (M <= 0 || N <= 0 || M % 64 != 0 || N % 64 != 0) return -1;
        hipLaunchKernelGGL((probe_loads_kernel<64, 64, 4, 4>), dim3((M / 64) * (N / 64)), dim3(256), 0,
                           (hipStream_t)stream, (const uint16_t*)x, (const uint16_t*)w, M, N, K, xcd_shift, sink);
    } else {
        return -1;
    }
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

// ops: 4096 * 64 16-byte words (4 MiB) of operand data; out: grid * 512 floats.
// FLOPs per call: grid * 8 waves * nk slices * 2 steps * 32 MFMAs * 16384, i.e. a
// 256 x 256 x 64 nk tile per workgroup.
int32_t probe_mfma_lds(const void* ops, int32_t grid, int32_t nk, float* out, void* stream) {
    if (!ops || !out || grid <= 0 || nk <= 0) return -1;
    hipLaunchKernelGGL(probe_mfma_lds_kernel, dim3(grid), dim3(512), 0, (hipStream_t)stream, (const u32x4*)ops, nk,
                       out);
    return (int32_t)hipGetLastError();
}

}  // extern "C"
