// linear_abi.hip -- the C ABI: argument validation, path and tile choice, launch.
//
// All shape, stride, alias and path checks run on the host before anything is
// enqueued, and kernel choice is a host decision made from the static shapes
// ("The Graph IR", section "Host-side shape inference", and the op table's MatMul
// row: shapes are known on the host and GEMV versus GEMM is chosen when the call
// is planned, not inside a kernel).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>

#include "../../include/linear_amd.h"
#include "kernels.h"

namespace {

thread_local int32_t g_last_hip_error = 0;

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxLdIn = (int64_t(1) << 22) - 1;
constexpr int64_t kMaxLdOut = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxGridX = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxGridY = 65535;
constexpr int kSkinnyMaxM = 16;   // AUTO sends M <= 16 to the skinny path

// The compute units and XCDs of the device a call runs on, read from the device
// (a partitioned part has fewer).  Plans made without a usable device (the
// pure-host linear_f16_plan) assume a whole MI355X: 256 CUs in 8 XCDs.
struct DevInfo {
    int cus;
    int xcd_shift;   // log2 of the XCD count; 0 (no XCD-aware remap) when not a power of two
};
constexpr DevInfo kWholeMI355X{256, 3};

struct Extent {
    uintptr_t lo, hi;  // [lo, hi) in bytes; hi == lo when empty
};

Extent extent(const void* p, int64_t rows, int64_t ld, int64_t cols, int64_t elem_bytes = 2) {
    Extent e{(uintptr_t)p, (uintptr_t)p};
    if (p && rows > 0 && cols > 0) e.hi = e.lo + (uintptr_t)(((rows - 1) * ld + cols) * elem_bytes);
    return e;
}

bool overlaps(Extent a, Extent b) { return a.lo < b.hi && b.lo < a.hi; }

struct Request {
    const uint16_t* x;
    int64_t ldx;
    const uint16_t* w;
    int64_t ldw;
    const uint16_t* b;
    void* y;
    int64_t ldy;
    int64_t M, N, K;
    int32_t path;
    bool need_bias;  // the bias entry point: b must be present
    int elem;        // lin::kF16 or lin::kBF16
    bool f32_out;    // y holds the unrounded FP32 sums
    const linear_epilogue* epi = nullptr;   // the epilogue entry points: the program
    int64_t G = 1, sx = 0, sy = 0;           // grouped calls: groups, x and y group strides
};

// The byte range of G groups of a [rows, cols] matrix (row stride ld, group stride s).
Extent extent_g(const void* p, int64_t G, int64_t s, int64_t rows, int64_t ld, int64_t cols, int64_t eb = 2) {
    Extent e{(uintptr_t)p, (uintptr_t)p};
    if (p && G > 0 && rows > 0 && cols > 0) e.hi = e.lo + (uintptr_t)(((G - 1) * s + (rows - 1) * ld + cols) * eb);
    return e;
}

bool epi_uses(const linear_epilogue* ep, int32_t op) {
    for (int s = 0; s < ep->nsteps; ++s)
        if (ep->op[s] == op) return true;
    return false;
}

// The program's own checks: step count and codes, the extra inputs its steps
// read, their strides, and overlaps with y (y may be the residual itself, with
// the same row stride: each element is read before it is written, by the same
// thread).
int32_t validate_epilogue(const Request& r) {
    const linear_epilogue* ep = r.epi;
    if (!ep) return LINEAR_E_NULL;
    if (ep->nsteps < 0 || ep->nsteps > LINEAR_EPI_MAX_STEPS) return LINEAR_E_EPILOGUE;
    for (int s = 0; s < ep->nsteps; ++s)
        if (ep->op[s] < LINEAR_EPI_BIAS || ep->op[s] > LINEAR_EPI_GELU_ERF) return LINEAR_E_EPILOGUE;
    if (r.M == 0 || r.N == 0) return LINEAR_OK;
    const Extent ey = extent(r.y, r.M, r.ldy, r.N);
    if (epi_uses(ep, LINEAR_EPI_BIAS)) {
        if (!ep->bias) return LINEAR_E_NULL;
        if (overlaps(ey, extent(ep->bias, 1, r.N, r.N))) return LINEAR_E_ALIAS;
    }
    if (epi_uses(ep, LINEAR_EPI_RESIDUAL)) {
        if (!ep->residual) return LINEAR_E_NULL;
        if (ep->ldr < r.N || ep->ldr > kMaxLdOut) return LINEAR_E_STRIDE;
        const bool in_place = (const void*)ep->residual == r.y && ep->ldr == r.ldy;
        if (!in_place && overlaps(ey, extent(ep->residual, r.M, ep->ldr, r.N))) return LINEAR_E_ALIAS;
    }
    if (epi_uses(ep, LINEAR_EPI_MUL)) {
        if (!ep->mul) return LINEAR_E_NULL;
        if (ep->ldm < r.N || ep->ldm > kMaxLdOut) return LINEAR_E_STRIDE;
        if (overlaps(ey, extent(ep->mul, r.M, ep->ldm, r.N))) return LINEAR_E_ALIAS;
    }
    return LINEAR_OK;
}

// Shape, pointer, stride, alias and path checks.  Pure host logic.
int32_t validate(const Request& r) {
    if (r.M < 0 || r.N < 0 || r.K < 0 || r.G < 0) return LINEAR_E_SHAPE;
    if (r.M > kMaxDim || r.N > kMaxDim || r.K > kMaxDim || r.G > kMaxGridY) return LINEAR_E_SHAPE;
    if (r.G > 1 && r.N * r.G > kMaxDim) return LINEAR_E_SHAPE;
    if (r.path != LINEAR_PATH_AUTO && r.path != LINEAR_PATH_GEMM && r.path != LINEAR_PATH_SKINNY)
        return LINEAR_E_PATH;
    if (r.M == 0 || r.N == 0 || r.G == 0) return LINEAR_OK;  // nothing to write
    if (!r.y) return LINEAR_E_NULL;
    if (r.K > 0 && (!r.x || !r.w)) return LINEAR_E_NULL;
    if (r.need_bias && !r.b) return LINEAR_E_NULL;
    if (r.ldx < r.K || r.ldw < r.K || r.ldy < r.N) return LINEAR_E_STRIDE;
    if (r.ldx > kMaxLdIn || r.ldw > kMaxLdIn || r.ldy > kMaxLdOut) return LINEAR_E_STRIDE;
    if (r.G > 1) {
        // groups read their activation slices anywhere, but write disjoint outputs
        if (r.sx < 0 || r.sx > kMaxLdOut * 1024) return LINEAR_E_STRIDE;
        if (r.sy < (r.M - 1) * r.ldy + r.N || r.sy > kMaxLdOut * 1024) return LINEAR_E_STRIDE;
    }
    const int64_t eb = r.f32_out ? 4 : 2;
    const Extent ey = extent_g(r.y, r.G, r.sy, r.M, r.ldy, r.N, eb);
    if (overlaps(ey, extent_g(r.x, r.G, r.sx, r.M, r.ldx, r.K))) return LINEAR_E_ALIAS;
    if (overlaps(ey, extent(r.w, r.N * r.G, r.ldw, r.K))) return LINEAR_E_ALIAS;
    if (r.b && overlaps(ey, extent(r.b, 1, r.N * r.G, r.N * r.G))) return LINEAR_E_ALIAS;
    return LINEAR_OK;
}

int32_t validate_all(const Request& r) {
    const int32_t st = validate(r);
    if (st != LINEAR_OK || !r.epi) return st;
    return validate_epilogue(r);
}

bool vector_loads_ok(const Request& r) {
    return ((uintptr_t)r.x % 16 == 0) && ((uintptr_t)r.w % 16 == 0) && (r.ldx % 8 == 0) &&
           (r.ldw % 8 == 0) && (r.K % 8 == 0) && (r.G <= 1 || r.sx % 8 == 0);
}

// The skinny path's one-row kernel: a single x row, 16-byte loads, one group,
// no epilogue program, x small enough to stage in LDS.
bool one_row_kernel(const Request& r) {
    return r.M == 1 && r.G <= 1 && !r.epi && r.K <= lin::kGemvMaxK && vector_loads_ok(r);
}

bool vector_store_ok(const Request& r) {
    return ((uintptr_t)r.y % (r.f32_out ? 16 : 8) == 0) && (r.ldy % 4 == 0) && (r.G <= 1 || r.sy % 4 == 0);
}

// Tile choice for the register-staged kernel (unaligned layouts, not tuned): the
// larger tile when it still gives every CU a tile.  Tiles count over all G groups.
int choose_gemm_config(int64_t M, int64_t N, int64_t G, int cus) {
    const lin::GemmConfig& g = lin::kGemmConfigs[0];
    const int64_t tiles = ((M + g.bm - 1) / g.bm) * ((N + g.bn - 1) / g.bn) * G;
    return tiles >= cus ? 0 : 1;
}

// Tile choice for the streaming kernel (aligned layouts).  Measured on MI355X, a
// 256x256 tile sustains the highest rate, and a partial last wave of large tiles
// costs little, so: the largest tile that still gives every CU at least one tile;
// when no tile size does, the one that keeps the most CUs busy at its rate.
// Tiles count over all G groups of a grouped call.
struct StreamChoice {
    int cfg;
    double rate;   // sustained throughput relative to the 256x256 tile
};
// kStreamConfigs in order: 256x256, 256x128, 128x256, 128x128, 64x64
const StreamChoice kStreamOrder[] = {{0, 1.00}, {1, 0.94}, {2, 0.85}, {3, 0.80}, {4, 0.57}};

int choose_stream_config(int64_t M, int64_t N, int64_t G, int cus) {
    int best = 4;
    double best_score = -1.0;
    for (const StreamChoice& c : kStreamOrder) {
        const lin::GemmConfig& g = lin::kStreamConfigs[c.cfg];
        const int64_t per_group = ((M + g.bm - 1) / g.bm) * ((N + g.bn - 1) / g.bn);
        if (per_group > kMaxGridX / 64) continue;
        const int64_t tiles = per_group * G;
        if (tiles >= cus) return c.cfg;
        const double score = (double)tiles * c.rate;
        if (score > best_score) {
            best_score = score;
            best = c.cfg;
        }
    }
    return best;
}

// Column split of a streaming GEMM call whose last wave of tiles would be at
// most half full: columns [0, n0) run in whole waves of configuration cfg's
// tiles and [n0, N) as a second launch with the tile chosen for it alone (the
// idle half of the chip in a half-empty wave costs more than a second launch:
// measured on mlp_up, 4096 x 14336 x 4096, 417-418 us against 433).  n0 = 0:
// one launch.  Only single-group calls of the 256 x 256 tile are split; the
// columns offset every [., N] operand, so each launch is a layer of its own and
// the results are those of one launch bit for bit.
struct ColumnSplit {
    int64_t n0;
    int cfg2;
};

ColumnSplit column_split(int64_t M, int64_t N, int64_t G, int cfg, int cus) {
    ColumnSplit sp{0, 0};
    if (G != 1 || cfg != 0) return sp;
    const lin::GemmConfig& g = lin::kStreamConfigs[cfg];
    const int64_t tm = (M + g.bm - 1) / g.bm, tn = (N + g.bn - 1) / g.bn;
    const int64_t tiles = tm * tn, last = tiles % cus;
    if (tiles <= cus || last == 0 || last > cus / 2) return sp;
    // the most column tiles short of tn that make whole waves
    for (int64_t t = tn - 1; t > 0; --t) {
        if ((tm * t) % cus == 0) {
            sp.n0 = t * g.bn;
            sp.cfg2 = choose_stream_config(M, N - sp.n0, 1, cus);
            return sp;
        }
    }
    return sp;
}

int32_t plan(const Request& r, linear_plan* p, int cus) {
    memset(p, 0, sizeof *p);
    int32_t path = r.path;
    if (path == LINEAR_PATH_AUTO) path = (r.M <= kSkinnyMaxM) ? LINEAR_PATH_SKINNY : LINEAR_PATH_GEMM;
    p->path = path;
    p->vector_io = vector_loads_ok(r) ? 1 : 0;
    if (path == LINEAR_PATH_SKINNY && one_row_kernel(r)) {
        p->tile_m = 1;
        p->tile_n = lin::kGemvRows;
        p->tile_k = lin::kGemvSeg;
        p->threads = lin::kGemvRows * 64;
        p->grid = (r.N + lin::kGemvRows - 1) / lin::kGemvRows;
        if (p->grid > kMaxGridX) return LINEAR_E_SHAPE;
    } else if (path == LINEAR_PATH_SKINNY) {
        p->tile_m = lin::kSkinnyTile;
        p->tile_n = lin::kSkinnyTile;
        p->tile_k = lin::kSkinnyKStep;
        p->threads = lin::kSkinnyWaves * 64;
        const int64_t gx = (r.N + 15) / 16, gy = (r.M + 15) / 16;
        if (gx > kMaxGridX || gy > kMaxGridY) return LINEAR_E_SHAPE;
        p->grid = gx * gy * r.G;
    } else {
        const bool stream = p->vector_io != 0;
        const int c = stream ? choose_stream_config(r.M, r.N, r.G, cus) : choose_gemm_config(r.M, r.N, r.G, cus);
        const lin::GemmConfig& g = stream ? lin::kStreamConfigs[c] : lin::kGemmConfigs[c];
        p->tile_m = g.bm;
        p->tile_n = g.bn;
        p->tile_k = g.bk;
        p->stages = g.stages;
        p->threads = g.wm * g.wn * 64;
        p->grid = ((r.M + g.bm - 1) / g.bm) * ((r.N + g.bn - 1) / g.bn);
        if (p->grid > kMaxGridX / 64) return LINEAR_E_SHAPE;
        p->grid *= r.G;
        if (stream) {
            const ColumnSplit sp = column_split(r.M, r.N, r.G, c, cus);
            if (sp.n0 > 0) {
                const lin::GemmConfig& g2 = lin::kStreamConfigs[sp.cfg2];
                p->grid = ((r.M + g.bm - 1) / g.bm) * (sp.n0 / g.bn);
                p->split_n = sp.n0;
                p->tile_m2 = g2.bm;
                p->tile_n2 = g2.bn;
                p->grid2 = ((r.M + g2.bm - 1) / g2.bm) * ((r.N - sp.n0 + g2.bn - 1) / g2.bn);
            }
        }
    }
    return LINEAR_OK;
}

// Device check, cached per device: the current device must be a gfx950.  Also
// caches its compute units and XCDs for the tile rules and the tile remap.
int32_t check_device(int* dev_out, DevInfo* info = nullptr) {
    // per device: 0 unknown, 1 gfx950, 2 other (callers may be on several threads);
    // the CU and XCD figures are stored before the state is published
    static std::atomic<int> cached[64];
    static std::atomic<int> cus[64], xcd_shift[64];
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0) {
        g_last_hip_error = (int32_t)e;
        return LINEAR_E_DEVICE;
    }
    if (dev < 64 && cached[dev] == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) {
            g_last_hip_error = (int32_t)e;
            return LINEAR_E_DEVICE;
        }
        int xcds = 1;
        if (hipDeviceGetAttribute(&xcds, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || xcds < 1) xcds = 1;
        int shift = 0;
        while ((2 << shift) <= xcds) ++shift;
        if ((1 << shift) != xcds) shift = 0;   // not a power of two: no XCD-aware remap
        cus[dev] = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : kWholeMI355X.cus;
        xcd_shift[dev] = shift;
        cached[dev] = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    }
    if (dev >= 64 || cached[dev] != 1) return LINEAR_E_DEVICE;
    *dev_out = dev;
    if (info) *info = DevInfo{cus[dev], xcd_shift[dev]};
    return LINEAR_OK;
}

// The current device's figures when a usable device is current, else a whole
// MI355X's (leaves the thread's last HIP error as it was).
DevInfo current_device_or_whole_part() {
    const int32_t saved = g_last_hip_error;
    int dev = 0;
    DevInfo info = kWholeMI355X;
    if (check_device(&dev, &info) != LINEAR_OK) info = kWholeMI355X;
    g_last_hip_error = saved;
    return info;
}

int32_t run(const Request& r, void* stream) {
    int32_t st = validate_all(r);
    if (st != LINEAR_OK) return st;
    if (r.M == 0 || r.N == 0 || r.G == 0) return LINEAR_OK;
    linear_plan p;
    st = plan(r, &p, kWholeMI355X.cus);   // shape errors come before device errors
    if (st != LINEAR_OK) return st;
    int dev = 0;
    DevInfo di = kWholeMI355X;
    st = check_device(&dev, &di);
    if (st != LINEAR_OK) return st;
    if (di.cus != kWholeMI355X.cus) {
        st = plan(r, &p, di.cus);
        if (st != LINEAR_OK) return st;
    }

    lin::LinearArgs a;
    a.x = r.x;
    a.w = r.w;
    a.b = r.b;
    a.y = r.y;
    a.ldx = r.ldx;
    a.ldw = r.ldw;
    a.ldy = r.ldy;
    a.M = (int)r.M;
    a.N = (int)r.N;
    a.K = (int)r.K;
    a.vec_store = vector_store_ok(r) ? 1 : 0;
    a.groups = (int)r.G;
    a.xcd_shift = di.xcd_shift;
    a.gsx = r.sx;
    a.gsy = r.sy;
    memset(&a.epi, 0, sizeof a.epi);
    auto al16 = [](const void* q, int64_t ld) { return ((uintptr_t)q % 16 == 0) && (ld % 8 == 0); };
    // 16-byte row accesses of the staged epilogue: y and the bias (the program's inputs below)
    a.epi.vec16 = (al16(r.y, r.ldy) && (r.G <= 1 || r.sy % 8 == 0) ? 1 : 0) |
                  (al16(r.b, 8) && (r.G <= 1 || r.N % 8 == 0) ? 2 : 0);
    int mode = r.f32_out ? lin::kOutF32 : (r.b != nullptr ? lin::kOutBias : lin::kOutRound);
    if (r.epi) {
        mode = lin::kOutEpi;
        const linear_epilogue* ep = r.epi;
        a.epi.bias = ep->bias;
        a.epi.res = ep->residual;
        a.epi.mul = ep->mul;
        a.epi.ldr = ep->ldr;
        a.epi.ldm = ep->ldm;
        a.epi.nsteps = ep->nsteps;
        a.epi.vec16 = (al16(r.y, r.ldy) ? 1 : 0) | (al16(ep->bias, 8) ? 2 : 0) |
                      (al16(ep->residual, ep->ldr) ? 4 : 0) | (al16(ep->mul, ep->ldm) ? 8 : 0);
        for (int s = 0; s < ep->nsteps; ++s) a.epi.ops |= (uint64_t)(uint8_t)ep->op[s] << (8 * s);
        if (epi_uses(ep, LINEAR_EPI_SILU) || epi_uses(ep, LINEAR_EPI_GELU_TANH) || epi_uses(ep, LINEAR_EPI_GELU_ERF)) {
            hipError_t te = lin::act_tables(r.elem, dev, (hipStream_t)stream, &a.epi.act);
            if (te == hipErrorStreamCaptureUnsupported) {
                g_last_hip_error = (int32_t)te;
                return LINEAR_E_CAPTURE;
            }
            if (te != hipSuccess) {
                g_last_hip_error = (int32_t)te;
                return LINEAR_E_DEVICE;
            }
        }
    }
    const bool vec = p.vector_io != 0;
    hipError_t e;
    if (p.path == LINEAR_PATH_SKINNY) {
        a.tiles_m = (int)((r.M + 15) / 16);
        a.tiles_n = (int)((r.N + 15) / 16);
        e = one_row_kernel(r) ? lin::launch_gemv(r.elem, a, mode, (hipStream_t)stream)
                              : lin::launch_skinny(r.elem, a, vec, mode, (hipStream_t)stream);
    } else if (vec) {
        const int c = choose_stream_config(r.M, r.N, r.G, di.cus);
        const lin::GemmConfig& g = lin::kStreamConfigs[c];
        a.tiles_m = (int)((r.M + g.bm - 1) / g.bm);
        a.tiles_n = (int)((r.N + g.bn - 1) / g.bn);
        const ColumnSplit sp = column_split(r.M, r.N, r.G, c, di.cus);
        if (sp.n0 == 0) {
            e = lin::launch_gemm_stream(r.elem, c, a, mode, (hipStream_t)stream);
        } else {
            lin::LinearArgs a1 = a;
            a1.N = (int)sp.n0;
            a1.tiles_n = (int)(sp.n0 / g.bn);
            e = lin::launch_gemm_stream(r.elem, c, a1, mode, (hipStream_t)stream);
            if (e == hipSuccess) {
                // the second launch sees columns [n0, N) as a layer of its own
                const lin::GemmConfig& g2 = lin::kStreamConfigs[sp.cfg2];
                const int64_t nr = r.N - sp.n0;
                lin::LinearArgs a2 = a;
                a2.N = (int)nr;
                a2.w = r.w + sp.n0 * r.ldw;
                if (a2.b) a2.b += sp.n0;
                a2.y = (unsigned char*)r.y + sp.n0 * (r.f32_out ? 4 : 2);
                if (a2.epi.bias) a2.epi.bias += sp.n0;
                if (a2.epi.res) a2.epi.res += sp.n0;
                if (a2.epi.mul) a2.epi.mul += sp.n0;
                a2.tiles_m = (int)((r.M + g2.bm - 1) / g2.bm);
                a2.tiles_n = (int)((nr + g2.bn - 1) / g2.bn);
                e = lin::launch_gemm_stream(r.elem, sp.cfg2, a2, mode, (hipStream_t)stream);
            }
        }
    } else {
        const int c = choose_gemm_config(r.M, r.N, r.G, di.cus);
        const lin::GemmConfig& g = lin::kGemmConfigs[c];
        a.tiles_m = (int)((r.M + g.bm - 1) / g.bm);
        a.tiles_n = (int)((r.N + g.bn - 1) / g.bn);
        e = lin::launch_gemm(r.elem, c, a, mode, (hipStream_t)stream);
    }
    if (e != hipSuccess) {
        g_last_hip_error = (int32_t)e;
        return LINEAR_E_LAUNCH;
    }
    return LINEAR_OK;
}

// The routed indexed kernels need 16-byte chunks of x rows and of table rows,
// 32-bit byte offsets within x and within one table, and few enough experts
// for the routing pass.
bool indexed_routed_ok(const uint16_t* x, int64_t ldx, const uint16_t* w, int64_t ldw, int64_t sw, int64_t E,
                       int64_t M, int64_t N, int64_t K) {
    return E <= lin::kIdxMaxExperts && (uintptr_t)x % 16 == 0 && (uintptr_t)w % 16 == 0 && ldx % 8 == 0 &&
           ldw % 8 == 0 && sw % 8 == 0 && K % 8 == 0 && N % 8 == 0 &&
           ((M - 1) * ldx + K) * 2 < (int64_t(1) << 31) && (K * ldw + N) * 2 < (int64_t(1) << 31);
}

// The indexed contraction: checks, then the launches.
int32_t run_indexed(int elem, bool f32_out, const uint16_t* x, int64_t ldx, const uint16_t* w, int64_t ldw,
                    int64_t sw, const int32_t* idx, void* y, int64_t ldy, int64_t E, int64_t M, int64_t N,
                    int64_t K, void* ws, int64_t ws_bytes, void* stream) {
    if (M < 0 || N < 0 || K < 0 || E < 0) return LINEAR_E_SHAPE;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim || E > kMaxGridY) return LINEAR_E_SHAPE;
    if (M == 0 || N == 0 || E == 0) return LINEAR_OK;   // no row has an expert: nothing to write
    if (!y || !idx || !ws) return LINEAR_E_NULL;
    if (K > 0 && (!x || !w)) return LINEAR_E_NULL;
    if (ldx < K || ldw < N || ldy < N || sw < K * ldw) return LINEAR_E_STRIDE;
    if (ldx > kMaxLdOut || ldw > kMaxLdOut || ldy > kMaxLdOut) return LINEAR_E_STRIDE;
    const int64_t need = lin::idx_ws_bytes(E, M);
    if (ws_bytes < need || (uintptr_t)ws % 16 != 0) return LINEAR_E_WORKSPACE;
    const int64_t eb = f32_out ? 4 : 2;
    const Extent ey = extent(y, M, ldy, N, eb);
    const Extent ew = extent(ws, 1, need, need, 1);
    if (overlaps(ey, extent(x, M, ldx, K))) return LINEAR_E_ALIAS;
    if (K > 0 && overlaps(ey, extent_g(w, E, sw, K, ldw, N))) return LINEAR_E_ALIAS;
    if (overlaps(ey, extent(idx, 1, M, M, 4))) return LINEAR_E_ALIAS;
    if (overlaps(ew, ey) || overlaps(ew, extent(x, M, ldx, K)) || overlaps(ew, extent(idx, 1, M, M, 4)) ||
        (K > 0 && overlaps(ew, extent_g(w, E, sw, K, ldw, N))))
        return LINEAR_E_ALIAS;
    int dev = 0;
    DevInfo di = kWholeMI355X;
    int32_t st = check_device(&dev, &di);
    if (st != LINEAR_OK) return st;
    lin::IndexedArgs a;
    a.x = x;
    a.w = w;
    a.idx = idx;
    a.y = y;
    a.ws = (int32_t*)ws;
    a.ldx = ldx;
    a.ldw = ldw;
    a.sw = sw;
    a.ldy = ldy;
    a.E = (int)E;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.vec_x = ((uintptr_t)x % 16 == 0) && (ldx % 8 == 0) ? 1 : 0;
    a.vec_store = ((uintptr_t)y % (f32_out ? 16 : 8) == 0) && (ldy % 4 == 0) ? 1 : 0;
    a.slots = 0;
    a.cus = di.cus;
    a.xcd_shift = di.xcd_shift;
    const int mode = f32_out ? lin::kOutF32 : lin::kOutRound;
    hipError_t e;
    if (indexed_routed_ok(x, ldx, w, ldw, sw, E, M, N, K)) {
        // rows per expert on average decide the row tile; decode tiles route
        // themselves (no routing pass) when every workgroup's routing, which all
        // of them repeat, runs at most two workgroups deep per CU
        int cfg = M > 16 * E ? 1 : 0;
        const lin::GemmConfig& g0 = lin::kIdxConfigs[cfg];
        // every expert with rows ends at most one partial tile
        a.slots = (int)((M + g0.bm - 1) / g0.bm + std::min(E, M));
        const int64_t grid = (int64_t)a.slots * ((N + g0.bn - 1) / g0.bn);
        if (grid > kMaxGridX) return LINEAR_E_SHAPE;
        if (cfg == 0 && M <= lin::kIdxSelfRouteRows && grid <= 2 * di.cus) cfg = 2;
        e = lin::launch_indexed_routed(elem, cfg, a, mode, (hipStream_t)stream);
    } else {
        e = lin::launch_indexed(elem, a, mode, (hipStream_t)stream);
    }
    if (e != hipSuccess) {
        g_last_hip_error = (int32_t)e;
        return LINEAR_E_LAUNCH;
    }
    return LINEAR_OK;
}

// The no-allocation indexed entry point's routing scratch: one array per GPU,
// held from the library's load until the process ends.  In host code the name
// `scratch` is only a stand-in for the symbol, never a device address: kernels
// get the address that hipGetSymbolAddress returns for the current device,
// looked up once per device at that device's first such call.
constexpr int64_t kNoAllocScratchBytes = LINEAR_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
static_assert(kNoAllocScratchBytes % 16 == 0, "the workspace must stay 16-byte sized");

// This device's address of `scratch` (dev current), or null with the HIP error kept.
void* scratch_address(int dev) {
    static std::atomic<void*> addr[64];   // per device; calls may come from several host threads
    if (dev < 0 || dev >= 64) return nullptr;
    void* p = addr[dev].load();
    if (p) return p;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
        g_last_hip_error = (int32_t)e;
        return nullptr;
    }
    addr[dev].store(p);
    return p;
}

}  // namespace

extern "C" {

int32_t linear_f16_indexed_noalloc(const uint16_t* x, int64_t ldx, const uint16_t* w, int64_t ldw, int64_t sw,
                                   const int32_t* idx, uint16_t* y, int64_t ldy, int64_t E, int64_t M, int64_t N,
                                   int64_t K, void* stream) {
    // the workspace call's own checks decide shapes and no-ops; only a call that
    // would launch needs the scratch, and it must fit
    if (M < 0 || N < 0 || K < 0 || E < 0) return LINEAR_E_SHAPE;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim || E > kMaxGridY) return LINEAR_E_SHAPE;
    if (M == 0 || N == 0 || E == 0) return LINEAR_OK;
    if (lin::idx_ws_bytes(E, M) > kNoAllocScratchBytes) return LINEAR_E_SCRATCH;
    int dev = 0;
    const int32_t st = check_device(&dev);
    if (st != LINEAR_OK) return st;
    void* ws = scratch_address(dev);
    if (!ws) return LINEAR_E_DEVICE;
    return run_indexed(lin::kF16, false, x, ldx, w, ldw, sw, idx, y, ldy, E, M, N, K, ws, kNoAllocScratchBytes,
                       stream);
}

int64_t linear_indexed_workspace_bytes(int64_t E, int64_t M) {
    if (E < 0 || M < 0 || E > kMaxGridY || M > kMaxDim) return -1;
    return lin::idx_ws_bytes(E, M);
}

int32_t linear_f16_indexed(const uint16_t* x, int64_t ldx, const uint16_t* w, int64_t ldw, int64_t sw,
                           const int32_t* idx, uint16_t* y, int64_t ldy, int64_t E, int64_t M, int64_t N, int64_t K,
                           void* workspace, int64_t workspace_bytes, void* stream) {
    return run_indexed(lin::kF16, false, x, ldx, w, ldw, sw, idx, y, ldy, E, M, N, K, workspace, workspace_bytes,
                       stream);
}

int32_t linear_bf16_indexed(const uint16_t* x, int64_t ldx, const uint16_t* w, int64_t ldw, int64_t sw,
                            const int32_t* idx, uint16_t* y, int64_t ldy, int64_t E, int64_t M, int64_t N, int64_t K,
                            void* workspace, int64_t workspace_bytes, void* stream) {
    return run_indexed(lin::kBF16, false, x, ldx, w, ldw, sw, idx, y, ldy, E, M, N, K, workspace, workspace_bytes,
                       stream);
}

int32_t linear_f16_indexed_f32out(const uint16_t* x, int64_t ldx, const uint16_t* w, int64_t ldw, int64_t sw,
                                  const int32_t* idx, float* y, int64_t ldy, int64_t E, int64_t M, int64_t N, int64_t K,
                                  void* workspace, int64_t workspace_bytes, void* stream) {
    return run_indexed(lin::kF16, true, x, ldx, w, ldw, sw, idx, y, ldy, E, M, N, K, workspace, workspace_bytes,
                       stream);
}

int32_t linear_bf16_indexed_f32out(const uint16_t* x, int64_t ldx, const uint16_t* w, int64_t ldw, int64_t sw,
                                   const int32_t* idx, float* y, int64_t ldy, int64_t E, int64_t M, int64_t N, int64_t K,
                                   void* workspace, int64_t workspace_bytes, void* stream) {
    return run_indexed(lin::kBF16, true, x, ldx, w, ldw, sw, idx, y, ldy, E, M, N, K, workspace, workspace_bytes,
                       stream);
}

int32_t linear_f16(const uint16_t* x, int64_t ldx, const uint16_t* weight, int64_t ldw,
                   const uint16_t* b, uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                   void* stream) {
    Request r{x, ldx, weight, ldw, b, y, ldy, M, N, K, LINEAR_PATH_AUTO, true, lin::kF16, false};
    return run(r, stream);
}

int32_t linear_f16_nobias(const uint16_t* x, int64_t ldx, const uint16_t* weight, int64_t ldw,
                          uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K, void* stream) {
    Request r{x, ldx, weight, ldw, nullptr, y, ldy, M, N, K, LINEAR_PATH_AUTO, false, lin::kF16, false};
    return run(r, stream);
}

int32_t linear_f16_ex(const uint16_t* x, int64_t ldx, const uint16_t* weight, int64_t ldw,
                      const uint16_t* b, uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                      int32_t path, void* stream) {
    Request r{x, ldx, weight, ldw, b, y, ldy, M, N, K, path, false, lin::kF16, false};
    return run(r, stream);
}

int32_t linear_f16_f32out(const uint16_t* x, int64_t ldx, const uint16_t* weight, int64_t ldw,
                          float* y, int64_t ldy, int64_t M, int64_t N, int64_t K, int32_t path,
                          void* stream) {
    Request r{x, ldx, weight, ldw, nullptr, y, ldy, M, N, K, path, false, lin::kF16, true};
    return run(r, stream);
}

int32_t linear_bf16(const uint16_t* x, int64_t ldx, const uint16_t* weight, int64_t ldw,
                    const uint16_t* b, uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                    void* stream) {
    Request r{x, ldx, weight, ldw, b, y, ldy, M, N, K, LINEAR_PATH_AUTO, true, lin::kBF16, false};
    return run(r, stream);
}

int32_t linear_bf16_nobias(const uint16_t* x, int64_t ldx, const uint16_t* weight, int64_t ldw,
                           uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K, void* stream) {
    Request r{x, ldx, weight, ldw, nullptr, y, ldy, M, N, K, LINEAR_PATH_AUTO, false, lin::kBF16, false};
    return run(r, stream);
}

int32_t linear_bf16_ex(const uint16_t* x, int64_t ldx, const uint16_t* weight, int64_t ldw,
                       const uint16_t* b, uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                       int32_t path, void* stream) {
    Request r{x, ldx, weight, ldw, b, y, ldy, M, N, K, path, false, lin::kBF16, false};
    return run(r, stream);
}

int32_t linear_bf16_f32out(const uint16_t* x, int64_t ldx, const uint16_t* weight, int64_t ldw,
                           float* y, int64_t ldy, int64_t M, int64_t N, int64_t K, int32_t path,
                           void* stream) {
    Request r{x, ldx, weight, ldw, nullptr, y, ldy, M, N, K, path, false, lin::kBF16, true};
    return run(r, stream);
}

int32_t linear_f16_epilogue(const uint16_t* x, int64_t ldx, const uint16_t* weight, int64_t ldw,
                            const linear_epilogue* epilogue, uint16_t* y, int64_t ldy, int64_t M, int64_t N,
                            int64_t K, int32_t path, void* stream) {
    if (!epilogue) return LINEAR_E_NULL;
    Request r{x, ldx, weight, ldw, nullptr, y, ldy, M, N, K, path, false, lin::kF16, false, epilogue};
    return run(r, stream);
}

int32_t linear_bf16_epilogue(const uint16_t* x, int64_t ldx, const uint16_t* weight, int64_t ldw,
                             const linear_epilogue* epilogue, uint16_t* y, int64_t ldy, int64_t M, int64_t N,
                             int64_t K, int32_t path, void* stream) {
    if (!epilogue) return LINEAR_E_NULL;
    Request r{x, ldx, weight, ldw, nullptr, y, ldy, M, N, K, path, false, lin::kBF16, false, epilogue};
    return run(r, stream);
}

int32_t linear_f16_grouped(const uint16_t* x, int64_t ldx, int64_t sx, const uint16_t* weight, int64_t ldw,
                           const uint16_t* b, uint16_t* y, int64_t ldy, int64_t sy, int64_t G, int64_t M,
                           int64_t N, int64_t K, int32_t path, void* stream) {
    Request r{x, ldx, weight, ldw, b, y, ldy, M, N, K, path, false, lin::kF16, false, nullptr, G, sx, sy};
    return run(r, stream);
}

int32_t linear_bf16_grouped(const uint16_t* x, int64_t ldx, int64_t sx, const uint16_t* weight, int64_t ldw,
                            const uint16_t* b, uint16_t* y, int64_t ldy, int64_t sy, int64_t G, int64_t M,
                            int64_t N, int64_t K, int32_t path, void* stream) {
    Request r{x, ldx, weight, ldw, b, y, ldy, M, N, K, path, false, lin::kBF16, false, nullptr, G, sx, sy};
    return run(r, stream);
}

int32_t linear_f16_grouped_f32out(const uint16_t* x, int64_t ldx, int64_t sx, const uint16_t* weight, int64_t ldw,
                                  float* y, int64_t ldy, int64_t sy, int64_t G, int64_t M, int64_t N, int64_t K,
                                  int32_t path, void* stream) {
    Request r{x, ldx, weight, ldw, nullptr, y, ldy, M, N, K, path, false, lin::kF16, true, nullptr, G, sx, sy};
    return run(r, stream);
}

int32_t linear_bf16_grouped_f32out(const uint16_t* x, int64_t ldx, int64_t sx, const uint16_t* weight,
                                   int64_t ldw, float* y, int64_t ldy, int64_t sy, int64_t G, int64_t M, int64_t N,
                                   int64_t K, int32_t path, void* stream) {
    Request r{x, ldx, weight, ldw, nullptr, y, ldy, M, N, K, path, false, lin::kBF16, true, nullptr, G, sx, sy};
    return run(r, stream);
}

int32_t linear_f16_plan(const uint16_t* x, int64_t ldx, const uint16_t* weight, int64_t ldw,
                        const uint16_t* b, uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                        int32_t path, linear_plan* out) {
    if (!out) return LINEAR_E_NULL;
    Request r{x, ldx, weight, ldw, b, y, ldy, M, N, K, path, false, lin::kF16, false};
    int32_t st = validate(r);
    if (st != LINEAR_OK) return st;
    if (M == 0 || N == 0) {
        memset(out, 0, sizeof *out);
        out->path = path == LINEAR_PATH_AUTO ? LINEAR_PATH_SKINNY : path;
        return LINEAR_OK;
    }
    return plan(r, out, current_device_or_whole_part().cus);
}

const char* linear_status_string(int32_t status) {
    switch (status) {
        case LINEAR_OK: return "ok";
        case LINEAR_E_NULL: return "a required pointer is NULL";
        case LINEAR_E_SHAPE: return "invalid shape: M, N or K negative or too large";
        case LINEAR_E_STRIDE: return "invalid row stride: ldx/ldw < K, ldy < N, or beyond the stride limit";
        case LINEAR_E_ALIAS: return "y overlaps x, weight, b or an epilogue input";
        case LINEAR_E_PATH: return "unknown path selector";
        case LINEAR_E_DEVICE: return "no usable gfx950 device is current";
        case LINEAR_E_LAUNCH: return "kernel launch failed";
        case LINEAR_E_EPILOGUE: return "invalid epilogue program: step count or step code";
        case LINEAR_E_CAPTURE: return "the first activation epilogue on a device cannot run under stream capture";
        case LINEAR_E_WORKSPACE: return "workspace not 16-byte aligned or smaller than linear_indexed_workspace_bytes";
        case LINEAR_E_SCRATCH: return "the call needs more routing scratch than LINEAR_NOALLOC_SCRATCH_BYTES";
        default: return "unknown status";
    }
}

int32_t linear_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
