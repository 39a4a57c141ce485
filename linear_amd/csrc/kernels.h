// kernels.h -- internal launch interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace lin {

struct GemmConfig {
    int bm, bn, wm, wn;   // tile rows (m), tile columns (n), waves along m and n
    int stages;           // LDS ring depth (streaming kernel); 2 for the register-staged one
    int bk;               // K elements per slice
};

// Register-staged MFMA GEMM (any layout).
constexpr int kNumGemmConfigs = 5;
extern const GemmConfig kGemmConfigs[kNumGemmConfigs];

// Streaming MFMA GEMM (16-byte aligned layouts), direct-to-LDS K-slice ring.
constexpr int kNumStreamConfigs = 10;
extern const GemmConfig kStreamConfigs[kNumStreamConfigs];

// a.tiles_m / a.tiles_n must match the chosen configuration.
// vec: 16-byte loader (aligned layouts only).
hipError_t launch_gemm(int cfg, const LinearArgs& a, bool vec, bool bias, hipStream_t stream);
hipError_t launch_gemm_stream(int cfg, const LinearArgs& a, bool bias, hipStream_t stream);

// Skinny weight-streaming kernel: 16 output columns (n) by 16 rows (m) per
// workgroup, K split over the workgroup's waves.
constexpr int kSkinnyWaves = 8;
constexpr int kSkinnyTile = 16;
constexpr int kSkinnyKStep = 32;
hipError_t launch_skinny(const LinearArgs& a, bool vec, bool bias, hipStream_t stream);

}  // namespace lin
