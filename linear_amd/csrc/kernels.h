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

// The activation tables of element type elem on `device` (3 x kActWords words:
// SiLU, tanh GeLU, erf GeLU), built on `stream` by the first call and waited for
// there; that first call fails with hipErrorStreamCaptureUnsupported under
// stream capture.
hipError_t act_tables(int elem, int device, hipStream_t stream, const uint16_t** tables);

}  // namespace lin
