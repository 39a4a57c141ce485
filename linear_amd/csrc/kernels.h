// kernels.h -- internal launch interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace lin {

struct GemmConfig {
    int bm, bn, wm, wn;   // tile rows (m), tile columns (n), waves along m and n
    int stages;           // LDS ring depth
    int bk;               // K elements per slice
};

// Streaming MFMA GEMM (16-byte aligned layouts), direct-to-LDS K-slice ring.
constexpr int kNumStreamConfigs = 5;
inline constexpr GemmConfig kStreamConfigs[kNumStreamConfigs] = {
    {256, 256, 2, 4, 2, 64},
    {256, 128, 4, 2, 3, 64},
    {128, 256, 2, 4, 4, 32},
    {128, 128, 2, 2, 4, 64},
    {64, 64, 2, 2, 4, 64},
};

// Register-staged MFMA GEMM with element-wise loads (any layout).
constexpr int kNumGemmConfigs = 2;
inline constexpr GemmConfig kGemmConfigs[kNumGemmConfigs] = {
    {128, 128, 2, 2, 2, 64},
    {64, 64, 2, 2, 2, 64},
};

// a.tiles_m / a.tiles_n must match the chosen configuration; mode is kOut*.
template <int E> hipError_t launch_gemm_t(int cfg, const LinearArgs& a, int mode, hipStream_t stream);
template <int E> hipError_t launch_gemm_stream_t(int cfg, const LinearArgs& a, int mode, hipStream_t stream);

inline hipError_t launch_gemm(int elem, int cfg, const LinearArgs& a, int mode, hipStream_t stream) {
    return elem == kBF16 ? launch_gemm_t<kBF16>(cfg, a, mode, stream) : launch_gemm_t<kF16>(cfg, a, mode, stream);
}
inline hipError_t launch_gemm_stream(int elem, int cfg, const LinearArgs& a, int mode, hipStream_t stream) {
    return elem == kBF16 ? launch_gemm_stream_t<kBF16>(cfg, a, mode, stream)
                         : launch_gemm_stream_t<kF16>(cfg, a, mode, stream);
}

// Skinny weight-streaming kernel: 16 output columns (n) by 16 rows (m) per
// workgroup, K split over the workgroup's waves.
constexpr int kSkinnyWaves = 8;
constexpr int kSkinnyTile = 16;
constexpr int kSkinnyKStep = 32;
hipError_t launch_skinny(int elem, const LinearArgs& a, bool vec, int mode, hipStream_t stream);

// Indexed contraction (x [M, K] against expert tables W [E, K, N], row m against
// expert idx[m]): one workgroup per (expert, kIdxCols output columns).
struct IndexedArgs {
    const uint16_t* x;      // [M, K], row stride ldx
    const uint16_t* w;      // [E, K, N]: k-row stride ldw, expert stride sw
    const int32_t* idx;     // [M]
    void* y;                // [M, N], row stride ldy (16-bit words or floats)
    int64_t ldx, ldw, sw, ldy;
    int E, M, N, K;
    int vec_x;              // x rows load as 16-byte fragments
    int vec_store;          // y takes 4-element vector stores
};
constexpr int kIdxWaves = 4;
constexpr int kIdxCols = 64;
constexpr int kIdxCap = 320;   // rows collected per batch
hipError_t launch_indexed(int elem, const IndexedArgs& a, int mode, hipStream_t stream);

// The activation tables of element type elem on `device` (3 x kActWords words:
// SiLU, tanh GeLU, erf GeLU), built on `stream` by the first call and waited for
// there; that first call fails with hipErrorStreamCaptureUnsupported under
// stream capture.
hipError_t act_tables(int elem, int device, hipStream_t stream, const uint16_t** tables);

}  // namespace lin
