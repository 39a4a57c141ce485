// indexed.hip -- the indexed contraction on gfx950 ("The Graph IR", op table:
// IndexedMatMul).  x [M, K] against expert tables W [E, K, N] read in place:
// row m contracts against expert idx[m], y[m, n] = sum_k x[m, k] * W[idx[m], k, n],
// FP32 accumulation, the result rounded to the element type (or the FP32 sums).
//
// Two paths.
//
// Routed (16-byte aligned layouts).  A routing pass (one workgroup) counts the
// rows of each expert, lays out the row list expert by expert and cuts it into
// row tiles of at most BM rows (the 256-row tiles take up to 32 leftover rows of
// their expert when that saves a round of workgroups): the tile table.  The
// contraction kernel then runs
// one workgroup per (tile, BN output columns), a GEMM over the tile's gathered x
// rows and the expert's [K, BN] column panel, streamed through an LDS ring by
// direct-to-LDS loads, 64 k per slice.  The table is k-major ([K, N], n
// contiguous) while an MFMA operand holds 8 consecutive k per lane, so the
// panel is read out of LDS with the transposing read ds_read_b64_tr_b16: within
// each 16-lane group it hands lane i the 4 elements that lanes 4j + i/4 (j = 0..3)
// address at their offset i % 4, so when the lanes address 4 k-rows x 16 columns
// in 8-byte pieces, lane i receives 4 consecutive k of column i.  The output rows
// are independent, so the order of rows inside a tile (set by the routing pass's
// atomic slots) does not change any result.
//
// Row scan (any other layout).  One workgroup per (expert, 64 output columns)
// collects, in index order, the rows whose idx names its expert (ballots and
// per-wave counts) and contracts them 16 at a time with v_mfma_f32_16x16x32,
// the A fragments gathered column-wise from the table, K split over the 4 waves
// and the partial tiles added in FP32 through LDS in wave order.
#include "common.h"
#include "kernels.h"
#include "sched.h"

namespace lin {

template <int E, int MODE>
__device__ inline void indexed_store4(const IndexedArgs& a, int m, int nb, f32x4 v) {
    if (MODE == kOutF32) {
        float* dst = (float*)a.y + (int64_t)m * a.ldy + nb;
        if (a.vec_store && nb + 3 < a.N) {
            *(f32x4*)dst = v;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (nb + e < a.N) dst[e] = v[e];
        }
        return;
    }
    uint16_t* dst = (uint16_t*)a.y + (int64_t)m * a.ldy + nb;
    uint16_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = narrow<E>(v[e]);
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

template <int E, int MODE>
__global__ void __launch_bounds__(kIdxWaves * 64)
indexed_kernel(IndexedArgs a) {
    constexpr int NT = kIdxWaves * 64;
    __shared__ int rows[kIdxCap];
    __shared__ int wcount[kIdxWaves];
    __shared__ f32x4 red[kIdxWaves][4][64];

    const int expert = blockIdx.y;
    const int n0 = blockIdx.x * kIdxCols;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, grp = lane >> 4;
    const uint16_t* we = a.w + (int64_t)expert * a.sw;
    const int U = (a.K + 31) / 32;
    const int ub = wave * U / kIdxWaves, ue = (wave + 1) * U / kIdxWaves;

    int cursor = 0;
    for (;;) {
        // collect up to kIdxCap rows of this expert, in index order
        int count = 0;
        while (cursor < a.M && count <= kIdxCap - NT) {
            const int m = cursor + (int)threadIdx.x;
            const bool hit = m < a.M && a.idx[m] == expert;
            const uint64_t mask = __ballot(hit);
            if (lane == 0) wcount[wave] = __popcll(mask);
            __syncthreads();
            int base = count, total = 0;
#pragma unroll
            for (int w = 0; w < kIdxWaves; ++w) {
                if (w < wave) base += wcount[w];
                total += wcount[w];
            }
            if (hit) rows[base + __popcll(mask & ((uint64_t(1) << lane) - 1))] = m;
            __syncthreads();
            count += total;
            cursor += NT;
        }
        for (int rc = 0; rc < count; rc += 16) {
            const int nrow = min(16, count - rc);
            const int m = r < nrow ? rows[rc + r] : -1;
            f32x4 acc[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[b] = (f32x4){};
            for (int u = ub; u < ue; ++u) {
                const int k = u * 32 + grp * 8;          // this lane's 8 K values: k .. k+7
                u32x4 xb = (u32x4){0u, 0u, 0u, 0u};
                if (m >= 0) {
                    const uint16_t* xr = a.x + (int64_t)m * a.ldx + k;
                    if (a.vec_x && k + 7 < a.K) {
                        xb = *(const u32x4*)xr;
                    } else {
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            if (k + j < a.K) xb[j >> 1] |= (uint32_t)xr[j] << (16 * (j & 1));
                    }
                }
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int n = n0 + 16 * b + r;
                    u32x4 wa = (u32x4){0u, 0u, 0u, 0u};
                    if (n < a.N) {
                        const uint16_t* wc = we + (int64_t)k * a.ldw + n;
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            if (k + j < a.K) wa[j >> 1] |= (uint32_t)wc[(int64_t)j * a.ldw] << (16 * (j & 1));
                    }
                    acc[b] = mfma16x16x32<E>(wa, xb, acc[b]);
                }
            }
#pragma unroll
            for (int b = 0; b < 4; ++b) red[wave][b][lane] = acc[b];
            __syncthreads();
            if (wave == 0 && m >= 0) {
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    f32x4 s = red[0][b][lane];
#pragma unroll
                    for (int w = 1; w < kIdxWaves; ++w) s += red[w][b][lane];
                    // lane l holds x row l % 16 and expert columns 4 (l / 16) .. +3 of block b
                    indexed_store4<E, MODE>(a, m, n0 + 16 * b + 4 * grp, s);
                }
            }
            __syncthreads();
        }
        if (cursor >= a.M) break;
    }
}

// ---------------------------------------------------------------------------
// Routed path

// Exclusive prefix sums of a and b over the 1024 threads (both in the same
// shuffles and barriers); *ta and *tb get the sums.  Uses wsum (66 words) and
// ends with a barrier.
__device__ inline int2 block_scan2_1024(int a, int b, int* wsum, int* ta, int* tb) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int ia = a, ib = b;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int xa = __shfl_up(ia, o, 64), xb = __shfl_up(ib, o, 64);
        if (lane >= o) {
            ia += xa;
            ib += xb;
        }
    }
    if (lane == 63) {
        wsum[wave] = ia;
        wsum[16 + wave] = ib;
    }
    __syncthreads();
    if (wave == 0) {
        const int sa = lane < 16 ? wsum[lane] : 0, sb = lane < 16 ? wsum[16 + lane] : 0;
        int ja = sa, jb = sb;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
            const int xa = __shfl_up(ja, o, 64), xb = __shfl_up(jb, o, 64);
            if (lane >= o) {
                ja += xa;
                jb += xb;
            }
        }
        if (lane < 16) {
            wsum[32 + lane] = ja - sa;                // exclusive wave offsets
            wsum[48 + lane] = jb - sb;
        }
        if (lane == 15) {
            wsum[64] = ja;
            wsum[65] = jb;
        }
    }
    __syncthreads();
    const int2 r = make_int2(wsum[32 + wave] + ia - a, wsum[48 + wave] + ib - b);
    *ta = wsum[64];
    *tb = wsum[65];
    __syncthreads();
    return r;
}

// Row tiles of an expert with c rows: ceil(c / BM), or, when absorbing, only its
// f = c / BM full tiles if the r = c mod BM rows left over fit xr more into each
// of them (0 < r <= xr f).
__device__ inline int expert_tiles(int c, int BM, int xr, bool absorb) {
    const int f = c / BM, r = c - f * BM;
    return f + (r > 0 && !(absorb && f > 0 && r <= xr * f));
}

// The routing pass: tile count, row list and tile table into the workspace.
// Row list: the rows of expert 0, then expert 1, ...; tile v = {first list
// position, expert, rows}.  Tiles hold at most BM rows, except that when the
// leftover rows of the experts would need another round of workgroups (tiles x
// tiles_n over cus), an expert's leftover rows are spread over its full tiles
// instead, up to xr more rows each, wherever they fit (tiles of BM + r / f rows,
// the first r mod f of them one more).
__global__ void __launch_bounds__(1024) indexed_route(const int32_t* __restrict__ idx, int M, int E, int BM, int xr,
                                                      int tiles_n, int cus, int32_t* __restrict__ ws) {
    __shared__ int cnt[kIdxMaxExperts];
    __shared__ int cur[kIdxMaxExperts];
    __shared__ int tbase[kIdxMaxExperts];
    __shared__ int wsum[66];
    const int tid = threadIdx.x;
    int32_t* perm = ws + kIdxHeaderWords;
    int4* tiles = (int4*)(ws + idx_ws_tiles(M));

    for (int e = tid; e < E; e += 1024) cnt[e] = 0;
    __syncthreads();
    if (tid == 0) wsum[64] = wsum[65] = 0;
    // idx is read 4 rows per thread at a time, the loads issued together; the
    // first 4096 rows' values stay in registers for the row list below
    auto load4 = [&](int m0, int (&e)[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int m = m0 + 1024 * j + tid;
            const int v = idx[min(m, M - 1)];         // unconditional: the four loads go out together
            e[j] = m < M ? v : -1;
        }
    };
    int e0[4];
    load4(0, e0);
    for (int m0 = 0; m0 < M; m0 += 4096) {
        int e[4];
        if (m0 == 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) e[j] = e0[j];
        } else {
            load4(m0, e);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if ((unsigned)e[j] < (unsigned)E) atomicAdd(&cnt[e[j]], 1);
    }
    __syncthreads();

    // prefix sums over the experts of rows and of tiles: thread t owns experts 4t .. 4t+3
    int c[4], rs = 0, ts = 0, ta = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = 4 * tid + j;
        c[j] = e < E ? cnt[e] : 0;
        rs += c[j];
        ts += expert_tiles(c[j], BM, xr, false);
        ta += expert_tiles(c[j], BM, xr, true);
    }
    // absorb only when it saves a round of workgroups on the CUs
    if (ts) atomicAdd(&wsum[64], ts);
    if (ta) atomicAdd(&wsum[65], ta);
    __syncthreads();
    const int tplain = wsum[64], tabs = wsum[65];
    const int64_t cap = (int64_t)cus;
    const bool absorb = (tabs * (int64_t)tiles_n + cap - 1) / cap < (tplain * (int64_t)tiles_n + cap - 1) / cap;
    int rtot, ttot;
    const int2 st = block_scan2_1024(rs, absorb ? ta : ts, wsum, &rtot, &ttot);
    int r0 = st.x, t0 = st.y;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = 4 * tid + j;
        if (e < E) {
            cur[e] = r0;
            tbase[e] = t0;
        }
        r0 += c[j];
        t0 += expert_tiles(c[j], BM, xr, absorb);
    }
    if (tid == 0) ws[0] = ttot;
    __syncthreads();

    // tile table: tile v belongs to the last expert whose first tile is <= v
    for (int v = tid; v < ttot; v += 1024) {
        int lo = 0, hi = E - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (tbase[mid] <= v) lo = mid;
            else hi = mid - 1;
        }
        const int t = v - tbase[lo], ce = cnt[lo];
        const int f = ce / BM, r = ce - f * BM;
        if (absorb && f > 0 && r > 0 && r <= xr * f) {
            const int q = r / f, rm = r - q * f;
            tiles[v] = make_int4(cur[lo] + t * (BM + q) + min(t, rm), lo, BM + q + (t < rm ? 1 : 0), 0);
        } else {
            tiles[v] = make_int4(cur[lo] + t * BM, lo, min(BM, ce - t * BM), 0);
        }
    }
    __syncthreads();

    // row list: each row takes the next free slot of its expert
    for (int m0 = 0; m0 < M; m0 += 4096) {
        int e[4];
        if (m0 == 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) e[j] = e0[j];
        } else {
            load4(m0, e);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if ((unsigned)e[j] < (unsigned)E) perm[atomicAdd(&cur[e[j]], 1)] = m0 + 1024 * j + tid;
    }
}

// LDS byte address of a pointer into the workgroup's LDS.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// The transposing LDS read (ds_read_b64_tr_b16) at LDS byte address addr + OFF,
// as inline assembly.  The compiler cannot tell which LDS bytes the builtin form
// reads, so before each one it makes the wave wait for every direct-to-LDS load
// in flight (vmcnt 0), the loads of the slices ahead included: a ring would then
// never overlap its loads with the MFMAs.  The wait insertion does not look into
// inline assembly, so the caller waits for the result itself (lds_ready) before
// any use; LDS operations of a wave complete in issue order.
template <int OFF>
__device__ __forceinline__ uint2 lds_tr16(uint32_t addr) {
    static_assert(OFF >= 0 && OFF < 65536, "the ds offset field is 16 bits");
    uint2 v;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF));
    return v;
}

// The same read of 16 bytes (ds_read_b128) for operands whose wait goes with the
// transposing reads around them.
template <int OFF>
__device__ __forceinline__ u32x4 lds_b128(uint32_t addr) {
    static_assert(OFF >= 0 && OFF < 65536, "the ds offset field is 16 bits");
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF));
    return v;
}

// Wait until at most N of the wave's LDS operations are outstanding, with the
// registers of a and b as operands, so that no use of them moves above the wait.
template <int N, typename A>
__device__ __forceinline__ void lds_ready(A& a) {
    static_assert(N >= 0 && N < 16, "lgkmcnt is 4 bits");
    asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a) : "n"(N));
}
template <int N, typename A, typename B>
__device__ __forceinline__ void lds_ready(A& a, B& b) {
    static_assert(N >= 0 && N < 16, "lgkmcnt is 4 bits");
    asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "n"(N));
}
template <int N, typename A, typename B, typename C>
__device__ __forceinline__ void lds_ready(A& a, B& b, C& c) {
    static_assert(N >= 0 && N < 16, "lgkmcnt is 4 bits");
    asm volatile("s_waitcnt lgkmcnt(%3)" : "+v"(a), "+v"(b), "+v"(c) : "n"(N));
}

// Swizzle of the panel rows: the 32-byte column pair u of k-row kr sits at pair
// u ^ pair_swz(kr).  The LDS serves a 64-lane 8-byte read 32 lanes at a time, and
// those 32 lanes of a transposing read fetch eight 32-byte pieces: the four
// k-rows 4i .. 4i + 3 in two adjacent pairs (32 x 32 fragments), or those four
// rows and the four rows 8 further on in one pair (16 x 16 fragments), with
// 4i mod 16 equal to 0 or 4.  pair_swz(kr) = 2 (kr mod 4) + (kr / 8) mod 2 sends
// the eight pieces to eight different 32-byte bank groups: no conflicts.
__host__ __device__ constexpr int pair_swz(int kr) { return 2 * (kr & 3) | ((kr >> 3) & 1); }

// Workgroup (tile v, column tile tn): y[rows of v, n0 .. n0 + BN) for tile v's
// expert.  Waves WM x WN; a wave owns TM = BM / WM rows and TN = BN / WN columns
// as (TN / 32) x (TM / 32) blocks of v_mfma_f32_32x32x16 (panel columns as the
// A operand, x rows as B).
//
// A tile may hold up to XR rows more than BM (the routing pass's absorbed
// leftover rows): rows BM .. BM + XR - 1 form one more 32-row block, of which
// wave (wm, wn) multiplies the 32 columns wn TN + 32 wm against the same panel
// fragments.
//
// LDS slot of one 64-k slice: the panel, 64 k-rows of BN columns (2 BN bytes,
// pair-swizzled as above), then XS >= BM + XR x rows of 64 k (128 bytes, 16-byte
// chunk c of row r at c ^ ((r >> 1) & 7), as in the dense kernel; rows past the
// tile's load as zero).  Each direct load fills 1 KB of the slot; lane l lands
// at byte 16 l of it and fetches the chunk that the swizzle places there.
template <int BM, int BN, int WM, int WN, int STAGES, int XR, int E, int MODE>
__global__ void __launch_bounds__(WM * WN * 64)
indexed_routed(IndexedArgs a) {
    constexpr int BK = 64, KS = BK / 16;
    constexpr int NW = WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int PROW = 2 * BN;                      // bytes per panel k-row
    constexpr int PBYTES = BK * PROW;
    constexpr int XS = (BM + XR + 8 * NW - 1) / (8 * NW) * (8 * NW);   // x rows per slot: whole loads per wave
    constexpr int XBYTES = XS * BK * 2;
    constexpr int SLICE = PBYTES + XBYTES;
    constexpr int GP = PBYTES / 1024, GX = XBYTES / 1024;
    constexpr int GPP = GP / NW, GPX = GX / NW;       // panel and x loads per wave per slice
    constexpr int GPW = GPP + GPX;
    static_assert(BN == 128 || BN == 256, "panel width must be 128 or 256 columns");
    static_assert(BM % 32 == 0 && TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");
    static_assert(GP % NW == 0 && GX % NW == 0, "direct loads must divide evenly over the waves");
    static_assert(STAGES >= 2 && STAGES * SLICE <= 160 * 1024, "LDS ring too large");
    static_assert(XR == 0 || (XR == 32 && FN == WM), "one extra 32-row block, a column block per wave row");
    __shared__ __attribute__((aligned(1024))) unsigned char smem[STAGES * SLICE];

    const int tiles_n = (a.N + BN - 1) / BN;
    // the used (tile, column tile) pairs are the first workgroup ids; the rest
    // exit.  Each XCD (ids are dealt round-robin over them) takes a contiguous
    // run of the pairs, walked 4 row tiles at a time as in the dense kernel:
    // the tiles running together on an XCD share x and panel reads in its L2.
    const int ntiles = a.ws[0];
    if ((int)blockIdx.x >= ntiles * tiles_n) return;  // an unused slot (uniform)
    int tv, tn;
    tile_coords(blockIdx.x, ntiles, tiles_n, a.xcd_shift, tv, tn);
    const int4 tile = ((const int4*)(a.ws + idx_ws_tiles(a.M)))[tv];
    const int32_t* list = a.ws + kIdxHeaderWords + tile.x;
    const int expert = tile.y, rows = tile.z;
    const int n0 = tn * BN;
    const int K = a.K;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // the expert's table: K rows, the last one ending at column N
    const __amdgpu_buffer_rsrc_t rp = matrix_rsrc(a.w + (int64_t)expert * a.sw, 0, K, a.ldw, a.N);
    // all of x: M rows of K
    const __amdgpu_buffer_rsrc_t rx = matrix_rsrc(a.x, 0, a.M, a.ldx, K);

    // This wave's direct loads, per slice: panel groups wave * GPP + j (j < GPP),
    // then x groups wave * GPX + j - GPP.
    uint32_t goff[GPW];
    int gk[GPW];                                      // k of the fetched chunk within a slice
#pragma unroll
    for (int j = 0; j < GPW; ++j) {
        if (j < GPP) {
            const int byte = (wave * GPP + j) * 1024 + 16 * lane;
            const int kr = byte / PROW;
            const int c = ((byte % PROW) / 16) ^ (2 * pair_swz(kr));
            const int n = n0 + 8 * c;
            gk[j] = kr;
            goff[j] = n < a.N ? (uint32_t)(((int64_t)kr * a.ldw + n) * 2) : kOOB;
        } else {
            const int xr = (wave * GPX + j - GPP) * 8 + lane / 8;
            const int c = (lane % 8) ^ ((xr >> 1) & 7);
            gk[j] = 8 * c;
            goff[j] = xr < rows ? (uint32_t)(((int64_t)list[xr] * a.ldx + 8 * c) * 2) : kOOB;
        }
    }
    const uint32_t pstep = (uint32_t)(BK * a.ldw * 2), xstep = (uint32_t)(BK * 2);
    const int nk = (K + BK - 1) / BK;

    const int wn = wave % WN, wm = wave / WN;
    // transposing reads: lane (q = lane / 16, s = lane % 16) addresses k-row
    // kq + 4 h + 16 ks with kq = 8 (q / 2) + s / 4, and the 8-byte piece at column
    // nb + 16 (q % 2) + 4 (s % 4) of its fragment; the row's pair swizzle is
    // pair_swz(kq) for every h and ks
    const int q = lane >> 4, s = lane & 15;
    const int kq = 8 * (q >> 1) + (s >> 2);
    const int sw = pair_swz(kq);
    uint32_t aoff[FN];
#pragma unroll
    for (int i = 0; i < FN; ++i) {
        const int n = wn * TN + i * 32 + 16 * (q & 1) + 4 * (s & 3);
        aoff[i] = kq * PROW + (((n >> 3) ^ (2 * sw)) << 4) + 8 * ((n >> 2) & 1);
    }
    // x fragment j of K step ks: row r = wm TM + 32 j + lr at r * 128 within the x
    // part, chunk (2 ks + lh) ^ ((r >> 1) & 7); 32 j + wm TM is a multiple of 16, so
    // the chunk does not depend on j and 32 j rows go into the constant offset
    static_assert(TM % 16 == 0, "x fragment rows keep their swizzle across blocks");
    const int lr = lane & 31, lh = lane >> 5;
    uint32_t boff[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) boff[ks] = (wm * TM + lr) * 128 + (((ks * 2 + lh) ^ ((lr >> 1) & 7)) << 4);
    // the extra block's x fragment: row BM + lr, at boff + xdelta
    const uint32_t xdelta = (uint32_t)((BM - wm * TM) * 128);

#define LIN_IDX_ISSUE(t_, j_)                                                                    \
    do {                                                                                         \
        const int t__ = (t_);                                                                    \
        unsigned char* slot__ = smem + (t__ % STAGES) * SLICE;                                   \
        const bool kin__ = goff[(j_)] != kOOB && t__ * BK + gk[(j_)] < K;                        \
        if ((j_) < GPP)                                                                          \
            lds_dma16(rp, slot__ + (wave * GPP + (j_)) * 1024, kin__ ? goff[(j_)] + (uint32_t)t__ * pstep : kOOB); \
        else                                                                                     \
            lds_dma16(rx, slot__ + PBYTES + (wave * GPX + (j_) - GPP) * 1024,                    \
                      kin__ ? goff[(j_)] + (uint32_t)t__ * xstep : kOOB);                        \
    } while (0)

    f32x16 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = (f32x16){};
    f32x16 accx = (f32x16){};                         // the extra rows' block (XR > 0)

    if (nk > 0) {
        // as in the dense streaming kernel: loads past the last slice carry
        // out-of-range offsets, so every wait below is static
#pragma unroll
        for (int t = 0; t < STAGES - 1; ++t)
#pragma unroll
            for (int j = 0; j < GPW; ++j) LIN_IDX_ISSUE(t, j);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((STAGES - 2) * GPW) : "memory");
        __syncthreads();

        // The wave's work scales with the tile's rows: FA of its FM row blocks
        // hold rows, and the reads and MFMAs of the others are skipped (one copy
        // of the pipeline per FA; every copy issues the same loads and barriers).
        // Fragment reads are inline assembly (lds_tr16, lds_b128): the reads of
        // one K step go into buffer BUF while the MFMAs of the other buffer run,
        // and the MFMAs of BUF first wait until only the reads of the following
        // step (2 FN + FA + XA) are outstanding.  XA: the tile has extra rows.
        auto pipeline = [&]<int FA, bool XA>() {
            constexpr int NR = 2 * FN + FA + (XA ? 1 : 0);   // reads per K step
            uint2 alo[2][FN], ahi[2][FN];
            u32x4 bf[2][FM], bx[2];
            auto read_frags = [&]<int KS_, int BUF>(uint32_t slot) {
                if constexpr (FA > 0) {
                    static_for<0, FN>([&]<int i>() {
                        alo[BUF][i] = lds_tr16<(16 * KS_) * PROW>(slot + aoff[i]);
                        ahi[BUF][i] = lds_tr16<(16 * KS_ + 4) * PROW>(slot + aoff[i]);
                    });
                    static_for<0, FA>([&]<int j>() { bf[BUF][j] = lds_b128<PBYTES + 32 * 128 * j>(slot + boff[KS_]); });
                    if constexpr (XA) bx[BUF] = lds_b128<PBYTES>(slot + boff[KS_] + xdelta);
                }
            };
            auto mfmas = [&]<int BUF>() {
                if constexpr (FA > 0) {
                    static_for<0, FN>([&]<int i>() { lds_ready<NR>(alo[BUF][i], ahi[BUF][i]); });
                    static_for<0, FA>([&]<int j>() { lds_ready<NR>(bf[BUF][j]); });
                    u32x4 af[FN];
#pragma unroll
                    for (int i = 0; i < FN; ++i) {
                        af[i] = (u32x4){alo[BUF][i].x, alo[BUF][i].y, ahi[BUF][i].x, ahi[BUF][i].y};
#pragma unroll
                        for (int j = 0; j < FA; ++j) acc[i][j] = mfma32x32x16<E>(af[i], bf[BUF][j], acc[i][j]);
                    }
                    if constexpr (XA) {
                        lds_ready<NR>(bx[BUF]);
                        accx = mfma32x32x16<E>(wm ? af[1] : af[0], bx[BUF], accx);
                    }
                }
            };
            const uint32_t base = lds_addr(smem);
            read_frags.template operator()<0, 0>(base);

            for (int t = 0; t < nk; ++t) {
                // slice t + STAGES - 1 goes into the slot released by the barrier
                // that ended slice t - 1
#pragma unroll
                for (int j = 0; j < GPW; ++j) LIN_IDX_ISSUE(t + STAGES - 1, j);
                const uint32_t slot = base + (t % STAGES) * SLICE;
                static_for<0, KS - 1>([&]<int ks>() {
                    read_frags.template operator()<ks + 1, (ks + 1) & 1>(slot);
                    mfmas.template operator()<ks & 1>();
                    __builtin_amdgcn_sched_barrier(0);
                });
                // slice t + 1 has landed once only the later slices' loads are
                // outstanding; the barrier also drains every wave's reads of slot t
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"((STAGES - 2) * GPW) : "memory");
                lds_barrier();
                if (t + 1 < nk) read_frags.template operator()<0, KS & 1>(base + ((t + 1) % STAGES) * SLICE);
                mfmas.template operator()<(KS - 1) & 1>();
            }
        };
        const int active = min(FM, max(0, (rows - wm * TM + 31) / 32));   // uniform
        if (XR > 0 && rows > BM) {
            if constexpr (XR > 0) pipeline.template operator()<FM, true>();
        } else {
            static_for<0, FM + 1>([&]<int fa>() {
                if (active == fa) pipeline.template operator()<fa, false>();
            });
        }
        // the zero-fill loads past the end must land before the LDS is released
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
#undef LIN_IDX_ISSUE

    // The tile goes out in row order through the freed ring, as in the dense
    // kernel: each lane stages its accumulators (element 4 b + r of (i, j) is tile
    // column wn TN + 32 i + 8 b + 4 (lane / 32) + r of tile row wm TM + 32 j +
    // lane % 32) with 16-byte chunk c of a staged row at c ^ (row mod chunks per
    // row), then every thread stores whole 16-byte chunks of the gathered rows.
    // FP32 sums, twice the bytes of the ring, go out in two bands of rows; the
    // extra rows of an absorbing tile in a band of their own.
    {
        constexpr int NT = NW * 64;
        constexpr int EB = MODE == kOutF32 ? 4 : 2;            // output bytes per element
        constexpr int EPC = 16 / EB;                          // elements per chunk
        constexpr int CPR = BN / EPC;                         // chunks per tile row
        constexpr int PASSES = (BM * BN * EB + STAGES * SLICE - 1) / (STAGES * SLICE);
        constexpr int RPP = BM / PASSES;                      // tile rows per band
        static_assert(BM % PASSES == 0 && RPP % 32 == 0, "bands must hold whole 32-row fragment blocks");
        static_assert((RPP * CPR) % NT == 0 && (32 * CPR) % NT == 0, "chunks must divide evenly over the threads");
        const bool vec = a.vec_store && ((uintptr_t)a.y % 16 == 0) && (a.ldy % EPC == 0);
        // accumulator v (4 consecutive columns from nl) into staged row ml
        auto stage = [&](int ml, int nl, const f32x4& v) {
            if constexpr (MODE == kOutF32) {
                *(f32x4*)(smem + (ml * CPR + ((nl / 4) ^ (ml % CPR))) * 16) = v;
            } else {
                uint2 u;
                u.x = (uint32_t)narrow<E>(v[0]) | ((uint32_t)narrow<E>(v[1]) << 16);
                u.y = (uint32_t)narrow<E>(v[2]) | ((uint32_t)narrow<E>(v[3]) << 16);
                *(uint2*)(smem + (ml * CPR + ((nl / 8) ^ (ml % CPR))) * 16 + ((nl / 4) & 1) * 8) = u;
            }
        };
        // the staged band of RB rows, tile rows row0 .. row0 + RB - 1, to y
        auto store_band = [&]<int RB>(int row0) {
#pragma unroll
            for (int k = 0; k < RB * CPR / NT; ++k) {
                const int c = (int)threadIdx.x + k * NT, r = c / CPR, cc = c % CPR;
                const int tr = row0 + r, n = n0 + cc * EPC;
                if (tr >= rows || n >= a.N) continue;
                const u32x4 v = *(const u32x4*)(smem + (r * CPR + (cc ^ (r % CPR))) * 16);
                const int64_t m = list[tr];
                unsigned char* dst = (unsigned char*)a.y + (m * a.ldy + n) * EB;
                if (vec && n + EPC <= a.N) {
                    *(u32x4*)dst = v;
                } else if constexpr (MODE == kOutF32) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < a.N) ((uint32_t*)dst)[e] = v[e];
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (n + e < a.N) ((uint16_t*)dst)[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
                }
            }
        };
#pragma unroll
        for (int pass = 0; pass < PASSES; ++pass) {
            __syncthreads();                                  // the ring, or the last band, is free
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int nl = wn * TN + i * 32 + 8 * b + 4 * lh;
#pragma unroll
                    for (int j = 0; j < FM; ++j) {
                        const int ml = wm * TM + j * 32 + lr - pass * RPP;
                        if (ml < 0 || ml >= RPP) continue;
                        stage(ml, nl, (f32x4){acc[i][j][4 * b], acc[i][j][4 * b + 1], acc[i][j][4 * b + 2],
                                              acc[i][j][4 * b + 3]});
                    }
                }
            __syncthreads();
            store_band.template operator()<RPP>(pass * RPP);
        }
        if constexpr (XR > 0) {
            if (rows > BM) {                                  // uniform
                __syncthreads();
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    stage(lr, wn * TN + wm * 32 + 8 * b + 4 * lh,
                          (f32x4){accx[4 * b], accx[4 * b + 1], accx[4 * b + 2], accx[4 * b + 3]});
                __syncthreads();
                store_band.template operator()<32>(BM);
            }
        }
    }
}

// Exclusive prefix sum of v over the 256 threads; *total gets the sum.  Uses
// wsum (8 words) and ends with a barrier.
__device__ inline int block_scan_256(int v, int* wsum, int* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int before = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) before += w < wave ? wsum[w] : 0;
    *total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
    return before + incl - v;
}

// Routing inside the workgroup, for small M: find tile v of the tile table the
// routing pass would build (rows of each expert in index order, cut into tiles
// of 16) and collect its rows into list[0 .. 16).  cnt: E words of scratch LDS.
// Returns false when tile v does not exist.  Uniform; ends with a barrier.
__device__ inline bool route_tile16(const int32_t* __restrict__ idx, int M, int E, int v, int* cnt, int* list,
                                    int* info, int* wsum) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int e = tid; e < E; e += 256) cnt[e] = 0;
    __syncthreads();
    for (int m = tid; m < M; m += 256) {
        const int e = idx[m];
        if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    // tiles per expert over contiguous ranges of experts, then the scan
    const int per = (E + 255) / 256, e0 = min(E, tid * per), e1 = min(E, e0 + per);
    int mine = 0;
    for (int e = e0; e < e1; ++e) mine += (cnt[e] + 15) / 16;
    int total;
    int t0 = block_scan_256(mine, wsum, &total);
    if (v >= total) return false;
    if (v >= t0 && v < t0 + mine) {
        for (int e = e0; e < e1; ++e) {
            const int nt = (cnt[e] + 15) / 16;
            if (v < t0 + nt) {
                info[0] = e;
                info[1] = v - t0;
                info[2] = min(16, cnt[e] - 16 * (v - t0));
                break;
            }
            t0 += nt;
        }
    }
    __syncthreads();
    const int e = info[0], first = 16 * info[1], last = first + info[2];
    // ranks of the expert's rows in index order: wave ballots, waves in order
    int seen = 0;
    for (int base = 0; base < M && seen < last; base += 256) {
        const int m = base + tid;
        const bool hit = m < M && idx[m] == e;
        const uint64_t mask = __ballot(hit);
        if (lane == 0) wsum[wave] = __popcll(mask);
        __syncthreads();
        int before = seen, add = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            before += w < wave ? wsum[w] : 0;
            add += wsum[w];
        }
        const int rank = before + __popcll(mask & ((uint64_t(1) << lane) - 1));
        if (hit && rank >= first && rank < last) list[rank - first] = m;
        seen += add;
        __syncthreads();
    }
    return true;
}

// Decode-shaped tiles (at most 16 rows): the contraction is the streaming of the
// panel.  Workgroup (tile v, 128 columns); its 4 waves split K, wave w taking
// the 32-k slices t = w, w + 4, ...: each streams its slices of the panel (32
// k-rows x 256 bytes, 8 direct loads of four whole 256-byte row pieces) and of
// the tile's x rows (16 rows x 64 bytes, 1 direct load) through a private ring
// of S slots and waits only for its own loads, so the loop has no barrier.
// SELF: the workgroup finds its tile itself (route_tile16) instead of reading
// the routing pass's table.
// v_mfma_f32_16x16x32: panel columns as A (two transposing reads per 16
// columns), x rows as B.  At the end the 4 partial tiles are added in wave
// order through LDS.
//
// Panel slot: k-row kr, 32-byte column pair u at pair u ^ pair_swz(kr).
// x slot: row r (64 bytes), 16-byte chunk c at chunk c ^ ((r >> 2) & 3).
template <int S, int E, int MODE, bool SELF>
__global__ void __launch_bounds__(256)
indexed_decode(IndexedArgs a) {
    constexpr int BK = 32;
    constexpr int PB = BK * 256;                      // panel bytes per slice
    constexpr int XB = 16 * BK * 2;                   // x bytes per slice
    constexpr int WSLOT = PB + XB;
    constexpr int L = PB / 1024 + XB / 1024;          // direct loads per slice
    static_assert(4 * S * WSLOT <= 160 * 1024 - 256 && 4 * S * WSLOT >= 4 * 8 * 64 * 16 &&
                  4 * S * WSLOT >= kIdxMaxExperts * 4, "LDS ring size");
    __shared__ __attribute__((aligned(1024))) unsigned char smem[4 * S * WSLOT];
    __shared__ int lrows[16], linfo[4], lsum[8];

    const int tiles_n = (a.N + 127) / 128;
    const int tv = blockIdx.x / tiles_n, tn = blockIdx.x - tv * tiles_n;
    const int32_t* list;
    int expert, rows;
    if constexpr (SELF) {
        // the ring is free until the first load below
        if (!route_tile16(a.idx, a.M, a.E, tv, (int*)smem, lrows, linfo, lsum)) return;
        list = lrows;
        expert = linfo[0];
        rows = linfo[2];
    } else {
        if (tv >= a.ws[0]) return;                    // an unused slot (uniform)
        const int4 tile = ((const int4*)(a.ws + idx_ws_tiles(a.M)))[tv];
        list = a.ws + kIdxHeaderWords + tile.x;
        expert = tile.y;
        rows = tile.z;
    }
    const int K = a.K;
    const int n0 = tn * 128;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    unsigned char* ring = smem + wave * S * WSLOT;

    const __amdgpu_buffer_rsrc_t rp = matrix_rsrc(a.w + (int64_t)expert * a.sw, 0, K, a.ldw, a.N);
    const __amdgpu_buffer_rsrc_t rx = matrix_rsrc(a.x, 0, a.M, a.ldx, K);

    // panel load j: k-row 4 j + lane / 16, stored chunk lane % 16
    uint32_t poff[PB / 1024];
    int pk[PB / 1024];
#pragma unroll
    for (int j = 0; j < PB / 1024; ++j) {
        const int kr = 4 * j + lane / 16;
        const int c = (lane % 16) ^ (2 * pair_swz(kr));
        const int n = n0 + 8 * c;
        pk[j] = kr;
        poff[j] = n < a.N ? (uint32_t)(((int64_t)kr * a.ldw + n) * 2) : kOOB;
    }
    // x load: row lane / 4, stored chunk lane % 4
    const int xr = lane / 4;
    const int xc = (lane % 4) ^ ((xr >> 2) & 3);
    const int xk = 8 * xc;
    const uint32_t xoff = xr < rows ? (uint32_t)(((int64_t)list[xr] * a.ldx + xk) * 2) : kOOB;
    const uint32_t pstep = (uint32_t)(BK * a.ldw * 2);
    const int nk = (K + BK - 1) / BK;
    const int mine = nk > wave ? (nk - wave + 3) / 4 : 0;   // this wave's slices

    // i-th slice of this wave: global slice wave + 4 i
    auto issue = [&](int i) {
        const int t = wave + 4 * i;
        unsigned char* slot = ring + (i % S) * WSLOT;
#pragma unroll
        for (int j = 0; j < PB / 1024; ++j) {
            const bool in = i < mine && poff[j] != kOOB && t * BK + pk[j] < K;
            lds_dma16(rp, slot + j * 1024, in ? poff[j] + (uint32_t)t * pstep : kOOB);
        }
        const bool in = i < mine && xoff != kOOB && t * BK + xk < K;
        lds_dma16(rx, slot + PB, in ? xoff + (uint32_t)t * (BK * 2) : kOOB);
    };

    // transposing reads: lane (q = lane / 16, s = lane % 16) addresses k-row
    // 8 q + 4 h + s / 4 and the 8-byte piece at column 16 b + 4 (s % 4); the
    // row's pair swizzle is pair_swz(8 q + s / 4) for both h
    const int q = lane >> 4, s = lane & 15;
    const int psw = pair_swz(8 * q + (s >> 2));
    const uint32_t abase = (8 * q + (s >> 2)) * 256 + 8 * (s & 1);
    uint32_t aoff[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) aoff[b] = abase + ((2 * (b ^ psw) + ((s & 3) >> 1)) << 4);
    // x read (B operand): row s, chunk q, at PB + boff
    const uint32_t boff = s * 64 + ((q ^ ((s >> 2) & 3)) << 4);

    f32x4 acc[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[b] = (f32x4){};
    for (int i = 0; i < S - 1; ++i) issue(i);
    const uint32_t rbase = lds_addr(ring);
    for (int i = 0; i < mine; ++i) {
        // slot (i - 1) % S: this wave's reads of it finished before its last MFMA
        issue(i + S - 1);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((S - 1) * L) : "memory");
        const uint32_t slot = rbase + (i % S) * WSLOT;
        // all 17 reads of the slice at once (inline assembly, see lds_tr16), then
        // each MFMA waits for its own: 2 (7 - b) reads follow block b's
        u32x4 xb = lds_b128<PB>(slot + boff);
        uint2 lo[8], hi[8];
        static_for<0, 8>([&]<int b>() {
            lo[b] = lds_tr16<0>(slot + aoff[b]);
            hi[b] = lds_tr16<4 * 256>(slot + aoff[b]);
        });
        static_for<0, 8>([&]<int b>() {
            if constexpr (b == 0) lds_ready<14>(xb, lo[0], hi[0]);
            else lds_ready<14 - 2 * b>(lo[b], hi[b]);
            acc[b] = mfma16x16x32<E>((u32x4){lo[b].x, lo[b].y, hi[b].x, hi[b].y}, xb, acc[b]);
        });
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // add the 4 partial tiles in wave order; wave w finishes blocks 2 w, 2 w + 1
    __syncthreads();
    f32x4* red = (f32x4*)smem;                        // [wave][block][lane]
#pragma unroll
    for (int b = 0; b < 8; ++b) red[(wave * 8 + b) * 64 + lane] = acc[b];
    __syncthreads();
    if (s < rows) {
        const int m = list[s];
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
            const int b = 2 * wave + bb;
            f32x4 v = red[b * 64 + lane];
#pragma unroll
            for (int w = 1; w < 4; ++w) v += red[(w * 8 + b) * 64 + lane];
            // element r: column n0 + 16 b + 4 (lane / 16) + r, tile row lane % 16
            const int n = n0 + 16 * b + 4 * q;
            if (n < a.N) indexed_store4<E, MODE>(a, m, n, v);
        }
    }
}

template <int E>
static const void* routed_fn(int cfg, int mode) {
    if (cfg == 0)
        return mode == kOutF32 ? (const void*)indexed_decode<4, E, kOutF32, false>
                               : (const void*)indexed_decode<4, E, kOutRound, false>;
    if (cfg == 2)
        return mode == kOutF32 ? (const void*)indexed_decode<4, E, kOutF32, true>
                               : (const void*)indexed_decode<4, E, kOutRound, true>;
    return mode == kOutF32 ? (const void*)indexed_routed<256, 256, 2, 4, 2, kIdxExtraRows, E, kOutF32>
                           : (const void*)indexed_routed<256, 256, 2, 4, 2, kIdxExtraRows, E, kOutRound>;
}

hipError_t launch_indexed_routed(int elem, int cfg, const IndexedArgs& a, int mode, hipStream_t stream) {
    const GemmConfig& g = kIdxConfigs[cfg];
    if (cfg != 2) {
        const int tiles_n = (int)((a.N + g.bn - 1) / g.bn);
        hipLaunchKernelGGL(indexed_route, dim3(1), dim3(1024), 0, stream, a.idx, a.M, a.E, g.bm,
                           cfg == 1 ? kIdxExtraRows : 0, tiles_n, a.cus, a.ws);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const void* fn = elem == kBF16 ? routed_fn<kBF16>(cfg, mode) : routed_fn<kF16>(cfg, mode);
    IndexedArgs args = a;
    void* params[] = {&args};
    const int64_t tiles_n = (a.N + g.bn - 1) / g.bn;
    return hipLaunchKernel(fn, dim3((unsigned)(tiles_n * a.slots)), dim3(g.wm * g.wn * 64), params, 0, stream);
}

template <int E>
static const void* indexed_fn(int mode) {
    return mode == kOutF32 ? (const void*)indexed_kernel<E, kOutF32> : (const void*)indexed_kernel<E, kOutRound>;
}

hipError_t launch_indexed(int elem, const IndexedArgs& a, int mode, hipStream_t stream) {
    const void* fn = elem == kBF16 ? indexed_fn<kBF16>(mode) : indexed_fn<kF16>(mode);
    IndexedArgs args = a;
    void* params[] = {&args};
    const dim3 grid((unsigned)((a.N + kIdxCols - 1) / kIdxCols), (unsigned)a.E);
    return hipLaunchKernel(fn, grid, dim3(kIdxWaves * 64), params, 0, stream);
}

}  // namespace lin
