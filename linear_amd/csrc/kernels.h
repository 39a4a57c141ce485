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

// One-row kernel of the skinny path (M = 1, 16-byte aligned layouts, ungrouped,
// no epilogue program, K <= kGemvMaxK): one wave per weight row, kGemvRows rows
// per workgroup, x staged in LDS (K * 2 bytes of dynamic shared memory).
constexpr int kGemvRows = 4;
constexpr int kGemvSeg = 512;      // K values per 1 KB wave load (64 lanes x 8)
constexpr int kGemvMaxK = 32768;   // 64 KB of x in LDS
hipError_t launch_gemv(int elem, const LinearArgs& a, int mode, hipStream_t stream);

// Indexed contraction (x [M, K] against expert tables W [E, K, N], row m against
// expert idx[m]).
struct IndexedArgs {
    const uint16_t* x;      // [M, K], row stride ldx
    const uint16_t* w;      // [E, K, N]: k-row stride ldw, expert stride sw
    const int32_t* idx;     // [M]
    void* y;                // [M, N], row stride ldy (16-bit words or floats)
    int32_t* ws;            // workspace (routed path): tile count, row list, tile table
    int64_t ldx, ldw, sw, ldy;
    int E, M, N, K;
    int vec_x;              // x rows load as 16-byte fragments
    int vec_store;          // y takes 4-element vector stores
    int slots;              // routed path: row-tile slots in the grid (>= tiles used)
    int cus;                // compute units of the device (the routing pass's round size)
    int xcd_shift;          // log2 of the device's XCD count (workgroup ids are dealt round-robin over them)
};

// Row-scan kernel (any layout): one workgroup per (expert, kIdxCols columns).
constexpr int kIdxWaves = 4;
constexpr int kIdxCols = 64;
constexpr int kIdxCap = 320;   // rows collected per batch

// Routed kernels (16-byte aligned layouts): a one-workgroup routing pass bins
// the rows by expert into the workspace, then an MFMA kernel runs one
// workgroup per (row tile of one expert, column tile).
constexpr int kIdxMaxExperts = 4096;     // experts the routing pass can bin
constexpr int kIdxMinRows = 16;          // smallest row tile
constexpr int64_t kIdxHeaderWords = 64;  // workspace: word 0 = tile count
// Workspace words before the tile table: header, then the M-entry row list.
__host__ __device__ inline int64_t idx_ws_tiles(int64_t M) { return (kIdxHeaderWords + M + 3) & ~int64_t(3); }
// Workspace bytes for up to E experts and M rows (any row tile >= kIdxMinRows).
inline int64_t idx_ws_bytes(int64_t E, int64_t M) {
    return (idx_ws_tiles(M) + 4 * ((M + kIdxMinRows - 1) / kIdxMinRows + E)) * 4;
}
// Routed configurations: 0 decode (16 x 128 tiles, waves split K), 1 prefill
// (256 x 256 tiles), 2 decode with the routing done by every workgroup itself
// (no routing pass; for M <= kIdxSelfRouteRows and a grid at most two
// workgroups deep per CU, since every workgroup repeats the routing).
constexpr int kNumIdxConfigs = 3;
inline constexpr GemmConfig kIdxConfigs[kNumIdxConfigs] = {
    {16, 128, 1, 4, 4, 32},
    {256, 256, 2, 4, 2, 64},
    {16, 128, 1, 4, 4, 32},
};
constexpr int kIdxSelfRouteRows = 4096;
// Rows past 256 that a prefill tile can take in (the routing pass's absorbed
// leftover rows of an expert).
constexpr int kIdxExtraRows = 32;
hipError_t launch_indexed(int elem, const IndexedArgs& a, int mode, hipStream_t stream);
hipError_t launch_indexed_routed(int elem, int cfg, const IndexedArgs& a, int mode, hipStream_t stream);

// The activation tables of element type elem on `device` (3 x kActWords words:
// SiLU, tanh GeLU, erf GeLU), built on `stream` by the first call and waited for
// there; that first call fails with hipErrorStreamCaptureUnsupported under
// stream capture.
hipError_t act_tables(int elem, int device, hipStream_t stream, const uint16_t** tables);

}  // namespace lin
