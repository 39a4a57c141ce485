// gemm_impl.h -- MFMA tiled GEMM for the linear layer on gfx950 (templates).
//
// Computes the projection tile C[n, m] = sum_k weight[n, k] * x[m, k] with
// v_mfma_f32_32x32x16_f16 / _bf16, or v_mfma_f32_16x16x32_f16 / _bf16 on the
// 256 x 256 streaming tile (exact products, FP32 accumulation), then the
// contract's epilogue: round to the element type, and with a bias widen, add b[n]
// in FP32 and round again ("tensor programs, part 1", section "One Program and One
// Numerical Contract"; the Inductor capture's cast sequence; for bfloat16, "The
// Graph IR", op table, ContractionEpilogue: a BF16 head rounds to BF16 before the
// first epilogue step), or an epilogue program of several such steps.  The
// FP32-output mode stores the sums unrounded (the op table's DenseContraction
// produces f32).
//
// Layout choices (both kernels):
//  - The weight tile is the MFMA A operand and the x tile the B operand, so the
//    accumulator rows are output columns n: each lane holds four consecutive n of
//    one output row m.
//  - Both operands are K-contiguous in HBM and are read in place ([N, K] weight,
//    no transpose copy, as the op table's dense contraction requires).
//  - Every tile feeds each output the same sequence of 16-wide k chunks into one
//    accumulator, so the tile choice never changes a result.
//  - Ragged M, N and K need no special tiles: loads go through buffer
//    resources whose range ends at the matrix's last valid element, so rows past
//    M or N and K chunks past K read as zero; stores are masked.
//  - Workgroup ids are remapped so that each XCD (consecutive ids are dealt
//    round-robin over the device's XCDs) owns a contiguous run of tiles, walked in
//    groups of 4 tile-rows, so tiles running together share x and weight panels
//    in that XCD's L2.
// The streaming kernel (aligned layouts) and the register-staged one (any
// layout) are described where they are defined below.
#pragma once

#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "sched.h"

namespace lin {


// Register-staged variant for layouts the streaming kernel cannot take (K, ldx or
// ldw not a multiple of 8, or x / weight not 16-byte aligned): every element is
// loaded with its own masked 2-byte buffer load, staged through registers into
// double-buffered LDS tiles (the loads of slice t + 1 are issued before the MFMAs
// of slice t and written to the other buffer after them; one barrier per slice).
// LDS rows are 128 bytes, 16-byte chunk c of row r at chunk c ^ ((r >> 1) & 7): the
// LDS serves a 16-byte-per-lane read 16 lanes (256 bytes) at a time, and the 16
// consecutive rows such a group reads at one K offset then fall in 16 different
// 16-byte bank groups.  The epilogue runs in registers: each lane finishes its
// four consecutive columns of one row and stores them with one 8-byte write.
template <int BM, int BN, int WM, int WN, int E, int MODE>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_kernel(LinearArgs a) {
    enter_group<MODE>(a);
    constexpr int BK = 64;
    constexpr int NT = WM * WN * 64;
    constexpr int TM = BM / WM, TN = BN / WN;   // one wave's output tile (m x n)
    constexpr int FM = TM / 32, FN = TN / 32;   // 32x32 MFMA blocks per wave
    constexpr int RSTEP = NT / 8;               // rows covered by one pass of the block
    constexpr int CW = BN / RSTEP, CX = BM / RSTEP;
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");
    static_assert(CW * RSTEP == BN && CX * RSTEP == BM, "tile rows must be a multiple of NT/8");
    static_assert(RSTEP % 16 == 0, "swizzle assumes rows of one thread share (r >> 1) & 7");
    constexpr int STAGE = (BN + BM) * BK;       // halves per LDS stage
    __shared__ __attribute__((aligned(16))) f16 smem[2 * STAGE];

    int tm, tn;
    tile_coords(blockIdx.x, a.tiles_m, a.tiles_n, a.xcd_shift, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int K = a.K;

    const __amdgpu_buffer_rsrc_t rw = matrix_rsrc(a.w, n0, a.N, a.ldw, K);
    const __amdgpu_buffer_rsrc_t rx = matrix_rsrc(a.x, m0, a.M, a.ldx, K);

    const int tid = threadIdx.x;
    const int kc = tid & 7;          // this thread's 16-byte chunk within a BK slice
    const int r0 = tid >> 3;         // first tile row it loads; then r0 + i * RSTEP
    const int swz = (kc ^ ((r0 >> 1) & 7)) << 3;

    uint32_t woff[CW], xoff[CX];
#pragma unroll
    for (int i = 0; i < CW; ++i) woff[i] = (uint32_t)(((int64_t)(r0 + i * RSTEP) * a.ldw + kc * 8) * 2);
#pragma unroll
    for (int i = 0; i < CX; ++i) xoff[i] = (uint32_t)(((int64_t)(r0 + i * RSTEP) * a.ldx + kc * 8) * 2);

    u32x4 wreg[CW], xreg[CX];

    auto gload = [&](int k0) {
        const uint32_t kb = (uint32_t)k0 * 2u;
#pragma unroll
        for (int i = 0; i < CW; ++i) wreg[i] = load8_masked(rw, woff[i] + kb, k0 + kc * 8, K, true);
#pragma unroll
        for (int i = 0; i < CX; ++i) xreg[i] = load8_masked(rx, xoff[i] + kb, k0 + kc * 8, K, true);
    };
    auto lds_store = [&](int s) {
        f16* sw = smem + s * STAGE;
        f16* sx = sw + BN * BK;
#pragma unroll
        for (int i = 0; i < CW; ++i) *(u32x4*)(sw + (r0 + i * RSTEP) * BK + swz) = wreg[i];
#pragma unroll
        for (int i = 0; i < CX; ++i) *(u32x4*)(sx + (r0 + i * RSTEP) * BK + swz) = xreg[i];
    };

    const int lane = tid & 63, wave = tid >> 6;
    const int wn = wave % WN, wm = wave / WN;
    const int lr = lane & 31, lh = lane >> 5;

    f32x16 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = (f32x16){};

    const int nk = (K + BK - 1) / BK;
    gload(0);
    lds_store(0);
    __syncthreads();

    for (int t = 0; t < nk; ++t) {
        const int cur = t & 1;
        if (t + 1 < nk) gload((t + 1) * BK);
        const f16* sw = smem + cur * STAGE;
        const f16* sx = sw + BN * BK;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int ch = ((ks * 2 + lh) ^ ((lr >> 1) & 7)) << 3;
            u32x4 av[FN], bv[FM];
#pragma unroll
            for (int i = 0; i < FN; ++i) av[i] = *(const u32x4*)(sw + (wn * TN + i * 32 + lr) * BK + ch);
#pragma unroll
            for (int j = 0; j < FM; ++j) bv[j] = *(const u32x4*)(sx + (wm * TM + j * 32 + lr) * BK + ch);
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j) acc[i][j] = mfma32x32x16<E>(av[i], bv[j], acc[i][j]);
        }
        if (t + 1 < nk) lds_store(cur ^ 1);
        __syncthreads();
    }

    // Epilogue.  Accumulator element v of block (i, j) sits at
    //   n = n0 + wn*TN + 32 i + 8 (v / 4) + 4 lh + (v % 4),   m = m0 + wm*TM + 32 j + lr.
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int nb = n0 + wn * TN + i * 32 + g * 8 + lh * 4;
#pragma unroll
            for (int j = 0; j < FM; ++j) {
                const int m = m0 + wm * TM + j * 32 + lr;
                if (m < a.M)
                    store4<E, MODE>(a, m, nb, acc[i][j][g * 4], acc[i][j][g * 4 + 1], acc[i][j][g * 4 + 2],
                                    acc[i][j][g * 4 + 3]);
            }
        }
}


// The epilogue program over a tile of rounded projection words staged in LDS.
// Layout: row r of the BM x BN tile holds CPR = BN / 8 chunks of 16 bytes, chunk
// c stored at position c ^ (r % CPR), so that the accumulator-order writes (32
// rows at one column per instruction) and the row-order reads below both spread
// over the banks.  Thread tid of NT takes chunks tid, tid + NT, ... (8
// consecutive columns of one row each) and runs the program step by step over
// up to 8 of them at a time: each step issues every load it needs before using
// any, and the extra inputs and y move as 16-byte row accesses where aligned.
// win: the LDS copy of activation step win_op's table window (or none when
// win_op is 0); other activation steps read their tables from global memory.
template <int BM, int BN, int NT, int E, int MODE>
__device__ inline void epi_tile(const LinearArgs& a, const unsigned char* tile, int m0, int n0, int tid,
                                lds_u16* win = nullptr, int win_op = 0, const u32x4* bias8 = nullptr) {
    constexpr int CPR = BN / 8;
    constexpr int CHT = BM * CPR / NT;               // chunks per thread
    constexpr int CH = CHT < 8 ? CHT : 8;            // chunks per pass (bounds register use)
    static_assert((BM * CPR) % NT == 0 && CHT % CH == 0, "chunks must divide evenly over the threads");
    const EpiArgs& ep = a.epi;
    for (int pass = 0; pass < CHT / CH; ++pass) {
        u32x4 t[CH];
        int rr[CH], cc[CH];
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            const int c = tid + (pass * CH + k) * NT, r = c / CPR, c8 = c % CPR;
            t[k] = *(const u32x4*)(tile + (r * CPR + (c8 ^ (r % CPR))) * 16);
            rr[k] = m0 + r;
            cc[k] = n0 + c8 * 8;
        }
        if constexpr (MODE == kOutBias) {       // the layer's own epilogue: one bias step
            u32x4 v[CH];
#pragma unroll
            for (int k = 0; k < CH; ++k) v[k] = bias8 ? *bias8 : load8(a.b + cc[k], true, cc[k], a.N, ep.vec16 & 2);
#pragma unroll
            for (int k = 0; k < CH; ++k) t[k] = binop8<E, false>(t[k], v[k]);
        }
        for (int s = 0; MODE == kOutEpi && s < ep.nsteps; ++s) {
            const int op = epi_op(ep, s);
            if (op >= kEpiSilu) {
                const __amdgpu_buffer_rsrc_t rt = table_rsrc(ep.act + (op - kEpiSilu) * kActWords);
                if (op == win_op) lookup_chunks<E, CH>(win, rt, t);
                else lookup_chunks<E, CH>(nullptr, rt, t);
                continue;
            }
            u32x4 v[CH];
            if (op == kEpiBias) {
#pragma unroll
                for (int k = 0; k < CH; ++k) v[k] = load8(ep.bias + cc[k], true, cc[k], a.N, ep.vec16 & 2);
            } else if (op == kEpiResidual) {
#pragma unroll
                for (int k = 0; k < CH; ++k)
                    v[k] = load8(ep.res + (int64_t)rr[k] * ep.ldr + cc[k], rr[k] < a.M, cc[k], a.N, ep.vec16 & 4);
            } else {
#pragma unroll
                for (int k = 0; k < CH; ++k)
                    v[k] = load8(ep.mul + (int64_t)rr[k] * ep.ldm + cc[k], rr[k] < a.M, cc[k], a.N, ep.vec16 & 8);
            }
            if (op == kEpiMul) {
#pragma unroll
                for (int k = 0; k < CH; ++k) t[k] = binop8<E, true>(t[k], v[k]);
            } else {
#pragma unroll
                for (int k = 0; k < CH; ++k) t[k] = binop8<E, false>(t[k], v[k]);
            }
        }
#pragma unroll
        for (int k = 0; k < CH; ++k)
            store8((uint16_t*)a.y + (int64_t)rr[k] * a.ldy + cc[k], rr[k] < a.M, cc[k], a.N, ep.vec16 & 1, t[k]);
    }
}

// The end of a streaming tile, after its last MFMA: the accumulators acc[i][j]
// (R x R blocks of wave (wm, wn), R = 32 or 16; four consecutive output columns
// n of one row m per lane and register group) leave through the LDS the ring used (RINGB
// bytes, free again), in row order.  FP32 mode: the sums, staged as floats in
// row bands when the tile is larger than the ring, 16-byte row stores.  Rounded
// modes: the rounded tile staged as 16-bit words, then epi_tile (the bias or the
// epilogue program, 16-byte row stores), with an epilogue program's first
// activation table window copied into LDS behind the tile.
template <int BM, int BN, int WM, int WN, int RINGB, int E, int MODE, int R, typename AccT>
__device__ __forceinline__ void finish_tile(const LinearArgs& a, unsigned char* smem,
                                            AccT (&acc)[BN / WN / R][BM / WM / R], int m0, int n0, int wave,
                                            int lane, const u32x4* bias8 = nullptr) {
    constexpr int NW = WM * WN, NT = NW * 64;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / R, FN = TN / R;
    constexpr int G = R * R / 256;                   // groups of 4 consecutive n per lane and block
    constexpr int TILEB = BM * BN * 2;
    const int wn = wave % WN, wm = wave / WN;
    const int lr = lane % R, lh = lane / R;
    if constexpr (MODE == kOutF32) {
        // the FP32 sums go out the same way, staged as floats in the freed ring
        // (in row bands when the whole tile does not fit): row r of a band holds
        // BN / 4 chunks of 16 bytes, chunk c at position c ^ (r % (BN / 4))
        constexpr int CPR4 = BN / 4;
        constexpr int PASSES = (BM * BN * 4 + RINGB - 1) / (RINGB);
        constexpr int RPP = BM / PASSES;                   // rows per band
        static_assert(BM % PASSES == 0 && RPP % R == 0, "bands must hold whole fragment blocks");
        constexpr int CHT = RPP * CPR4 / NT;
        static_assert((RPP * CPR4) % NT == 0, "chunks must divide evenly over the threads");
#pragma unroll
        for (int pass = 0; pass < PASSES; ++pass) {
            __syncthreads();
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const int nl = wn * TN + i * R + g * 8 + lh * 4;
#pragma unroll
                    for (int j = 0; j < FM; ++j) {
                        const int ml = wm * TM + j * R + lr - pass * RPP;
                        if (ml >= 0 && ml < RPP) {
                            const f32x4 v = (f32x4){acc[i][j][g * 4], acc[i][j][g * 4 + 1], acc[i][j][g * 4 + 2],
                                                    acc[i][j][g * 4 + 3]};
                            *(f32x4*)(smem + (ml * CPR4 + ((nl / 4) ^ (ml % CPR4))) * 16) = v;
                        }
                    }
                }
            __syncthreads();
            const bool vec = a.vec_store && ((uintptr_t)a.y % 16 == 0);
#pragma unroll
            for (int k = 0; k < CHT; ++k) {
                const int c = (int)threadIdx.x + k * NT, r = c / CPR4, c4 = c % CPR4;
                const f32x4 v = *(const f32x4*)(smem + (r * CPR4 + (c4 ^ (r % CPR4))) * 16);
                const int m = m0 + pass * RPP + r, n = n0 + c4 * 4;
                if (m >= a.M) continue;
                float* dst = (float*)a.y + (int64_t)m * a.ldy + n;
                if (vec && n + 3 < a.N) {
                    *(f32x4*)dst = v;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < a.N) dst[e] = v[e];
                }
            }
        }
        return;
    }

    if constexpr (MODE != kOutF32) {
        // stage the rounded tile in the (now free) ring, then finish it in row order:
        // the bias or the epilogue program, and 16-byte stores of whole row chunks
        static_assert(BM * BN * 2 <= RINGB, "the rounded tile must fit in the ring");
        constexpr int CPR = BN / 8;
        __syncthreads();
        // an epilogue program's first activation: its table window goes into LDS
        // behind the tile (32 direct loads of 1 KB: for each sign 8192 words from
        // kActWinBase on), landing while the tile is staged
        int win_op = 0;
        if constexpr (MODE == kOutEpi) {
            for (int s = 0; s < a.epi.nsteps; ++s)
                if (win_op == 0 && epi_op(a.epi, s) >= kEpiSilu) win_op = epi_op(a.epi, s);
            if (win_op != 0) {
                const __amdgpu_buffer_rsrc_t rt = __builtin_amdgcn_make_buffer_rsrc(
                    (void*)(a.epi.act + (win_op - kEpiSilu) * kActWords), (short)0, kActWords * 2, kRsrcWord3);
                constexpr int PW = 32 / NW;
                static_assert(32 % NW == 0, "window loads must divide evenly over the waves");
#pragma unroll
                for (int q = 0; q < PW; ++q) {
                    const int j = wave * PW + q, h = j >> 4, piece = j & 15;
                    const uint32_t word = ((uint32_t)h << 15) + kActWinBase<E> + (uint32_t)piece * 512u;
                    lds_dma16(rt, smem + TILEB + j * 1024, word * 2u + 16u * (uint32_t)lane);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int nl = wn * TN + i * R + g * 8 + lh * 4;
#pragma unroll
                for (int j = 0; j < FM; ++j) {
                    const int ml = wm * TM + j * R + lr;
                    uint2 u;
                    u.x = (uint32_t)narrow<E>(acc[i][j][g * 4]) | ((uint32_t)narrow<E>(acc[i][j][g * 4 + 1]) << 16);
                    u.y = (uint32_t)narrow<E>(acc[i][j][g * 4 + 2]) | ((uint32_t)narrow<E>(acc[i][j][g * 4 + 3]) << 16);
                    const int c8 = nl / 8;
                    *(uint2*)(smem + (ml * CPR + (c8 ^ (ml % CPR))) * 16 + ((nl / 4) & 1) * 8) = u;
                }
            }
        if constexpr (MODE == kOutEpi) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        epi_tile<BM, BN, NT, E, MODE>(a, smem, m0, n0, threadIdx.x, (lds_u16*)(smem + TILEB), win_op, bias8);
        return;
    }
}

// Tile (tm, tn) of this workgroup, with its group entered.  One group: the XCD
// walk of tile_coords over blockIdx.x.  Several groups (grid z): the groups' row
// tiles are stacked into one column of G x tiles_m row tiles and walked as one
// grid in the order workgroups are dispatched (x fastest, then z), so the run of
// tiles an XCD holds spans as few groups, and so as few panels, as it can.
template <int MODE>
__device__ inline void stream_tile(LinearArgs& a, int& tm, int& tn) {
    if (gridDim.z == 1) {
        tile_coords(blockIdx.x, a.tiles_m, a.tiles_n, a.xcd_shift, tm, tn);
        return;
    }
    const int tiles = a.tiles_m * a.tiles_n;
    int row;
    tile_coords(blockIdx.x + tiles * blockIdx.z, gridDim.z * a.tiles_m, a.tiles_n, a.xcd_shift, row, tn);
    const int g = row / a.tiles_m;
    tm = row - g * a.tiles_m;
    enter_group_at<MODE>(a, g);
}

// ---------------------------------------------------------------------------
// Streaming variant for 16-byte aligned layouts (x, weight 16-byte aligned, ldx,
// ldw and K multiples of 8).
//
// K-slices of BK (32 or 64) move from HBM straight into LDS with direct-to-LDS
// buffer loads (no register staging, no LDS write instructions), through a ring
// of STAGES slots: slice t + STAGES is requested as soon as slot t is retired, so
// each load has STAGES - 1 slices of MFMA work to arrive in.
//
// The fragment reads are software pipelined by hand: the fragments of the next
// K step are read while the MFMAs of the current one run, and the one barrier
// per slice sits between the last fragment reads of slice t and its last MFMAs,
// so the barrier, the next request and the first reads of slice t + 1 overlap
// MFMA work already queued.  Scheduling-group barriers pin that order.
//
// LDS layout of a slice: tile rows of 2 BK bytes (CPR = BK / 8 chunks of 8
// halves), chunk c of row r stored at chunk c ^ ((r / RP) % CPR), RP = 256 / (2 BK)
// rows per 256-byte span.  The LDS serves 16 lanes (256 bytes) of a 16-byte read
// per cycle; an MFMA fragment read (32 consecutive rows, one logical chunk) then
// touches 16 distinct 16-byte bank groups in each group of 16 lanes.  A direct
// load fills 1 KB = 1024 / (2 BK) consecutive rows; lane l lands at byte 16 l,
// i.e. row l / CPR, stored chunk l % CPR, so it fetches the logical chunk that the
// swizzle puts there.  With BK = 64 every load instruction covers whole 128-byte
// rows.
//
// WHOLE (tiles with one MFMA per wave and K step): a K step's fragment reads
// would have a single MFMA to hide behind, so each slice's fragments are read at
// once and its MFMAs run as they land; and only slices that exist are requested,
// the wait for slice t choosing at run time how many later slices may still be
// in flight (no zero-fill requests past K).
template <int BM, int BN, int WM, int WN, int STAGES, int BK, int E, int MODE, int SPREAD = 1, bool WHOLE = false,
          bool M16 = false>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_stream(LinearArgs a) {
    constexpr int R = M16 ? 16 : 32;                  // MFMA block rows and columns
    constexpr int KSTEP = M16 ? 32 : 16;              // k values per MFMA
    constexpr int KS = BK / KSTEP;                    // MFMA K steps per slice
    constexpr int NW = WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / R, FN = TN / R;
    using AccT = std::conditional_t<M16, f32x4, f32x16>;
    constexpr int ROWB = BK * 2;                      // bytes per LDS tile row
    constexpr int CPR = BK / 8;                       // 16-byte chunks per row
    constexpr int RP = 256 / ROWB;                    // rows per 256-byte span
    constexpr int RPL = 1024 / ROWB;                  // rows per direct load
    constexpr int SLICE = (BN + BM) * ROWB;           // bytes per slot (weight rows first)
    constexpr int GROUPS = (BN + BM) / RPL;           // direct loads per slice
    constexpr int GPW = GROUPS / NW;                  // loads per wave per slice
    static_assert(BK == 32 || BK == 64, "BK must be 32 or 64");
    static_assert(GROUPS % NW == 0, "row groups must divide evenly over the waves");
    static_assert(BN % RPL == 0, "weight rows must fill whole direct loads");
    static_assert(TM % R == 0 && TN % R == 0, "wave tile must be a multiple of the MFMA block");
    static_assert(WHOLE || KS % 2 == 0, "the pipelined loop alternates two fragment buffers per slice");
    static_assert(STAGES >= 2 && STAGES * SLICE <= 160 * 1024, "LDS ring too large");
    // after the main loop the ring holds the rounded tile (BM x BN words) and, for
    // an epilogue program, the LDS window of its first activation's table behind it
    constexpr int TILEB = BM * BN * 2;
    constexpr int LDSB = MODE == kOutEpi && TILEB + 2 * kActWinWords > STAGES * SLICE ? TILEB + 2 * kActWinWords
                                                                                      : STAGES * SLICE;
    static_assert(LDSB <= 160 * 1024, "LDS too large");
    __shared__ __attribute__((aligned(1024))) unsigned char smem[LDSB];

    int tm, tn;
    stream_tile<MODE>(a, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int K = a.K;
    const __amdgpu_buffer_rsrc_t rw = matrix_rsrc(a.w, n0, a.N, a.ldw, K);
    const __amdgpu_buffer_rsrc_t rx = matrix_rsrc(a.x, m0, a.M, a.ldx, K);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform

    // The bias chunk this thread adds in the epilogue, requested now so that its
    // latency is off the tile's tail: the epilogue gives thread t the row chunks
    // t, t + NT, ..., all at column n0 + 8 (t % (BN / 8)) since NT is a multiple
    // of BN / 8 (on the toy layer a bias load after the main loop cost ~1.3 us).
    // The 16 x 16 x 32 loop has no registers to hold it through the K loop and
    // requests it before its last slice instead.
    static_assert((NW * 64) % (BN / 8) == 0, "a thread's epilogue chunks must share their columns");
    u32x4 bias8 = (u32x4){0u, 0u, 0u, 0u};
    auto request_bias = [&]() {
        const int c = n0 + 8 * ((int)threadIdx.x % (BN / 8));
        bias8 = load8(a.b + c, true, c, a.N, a.epi.vec16 & 2);
    };
    constexpr bool LATE_BIAS = M16 && !WHOLE;        // requested after the K loop instead
    if constexpr (MODE == kOutBias && !LATE_BIAS) request_bias();

    // This wave's loads: groups g = wave * GPW + j; group g < BN / RPL holds weight
    // rows RPL g .., the others x rows.  Lane l fetches row l / CPR of the group,
    // logical chunk (l % CPR) ^ ((row / RP) % CPR).  (The whole offset stays in
    // the lane's register: the range check that zero-fills rows past M or N
    // looks at that part of the offset.)
    // The chunk a lane fetches repeats every GPER groups (a wave's first group
    // starts that period), so its first K element is kept once per phase.
    constexpr int GPER = CPR / ((RPL / RP) < CPR ? (RPL / RP) : CPR);
    static_assert((GPW * (RPL / RP)) % CPR == 0, "a wave's first group must start the swizzle's period");
    uint32_t goff[GPW];
    int gk[GPER];                                  // first K element this lane fetches, per phase
#pragma unroll
    for (int j = 0; j < GPW; ++j) {
        const int g = wave * GPW + j;
        const bool isw = g < BN / RPL;
        const int tr = g * RPL + lane / CPR;       // row within the slot (weight rows first)
        const int r = isw ? tr : tr - BN;          // row within its matrix tile
        const int c = (lane % CPR) ^ ((tr / RP) % CPR);
        if (j < GPER) gk[j] = c * 8;
        goff[j] = (uint32_t)(((int64_t)r * (isw ? a.ldw : a.ldx) + c * 8) * 2);
    }

    const int nk = (K + BK - 1) / BK;
    // One direct load: group j of this wave for slice t_ (j_ a compile-time index).
#define LIN_ISSUE_ONE(t_, j_)                                                            \
    do {                                                                                 \
        const int t__ = (t_);                                                            \
        unsigned char* slot__ = smem + (t__ % STAGES) * SLICE;                           \
        const uint32_t kb__ = (uint32_t)(t__ * BK) * 2u;                                 \
        const int g__ = wave * GPW + (j_);                                               \
        const bool kin__ = t__ * BK + gk[(j_) % GPER] < K;                               \
        lds_dma16(g__ < BN / RPL ? rw : rx, slot__ + g__ * 1024, kin__ ? goff[(j_)] + kb__ : kOOB); \
    } while (0)

    // The loads of slice t + STAGES go into the slot that the barrier after slice
    // t releases.  They are spread over a window of 1 + SP K steps (the last
    // step of slice t and the first SP steps of slice t + 1), DPS per step, so
    // that the CU's load requests trickle in between MFMAs instead of reaching the
    // texture addresser as one burst that stalls every wave's instruction issue.
    // (the window ends at least one K step before the barrier that waits for
    // these loads: SPREAD is capped at KS - 2)
    static_assert(SPREAD >= 0, "SPREAD counts K steps");
    constexpr int SP = SPREAD < KS - 2 ? SPREAD : (KS > 2 ? KS - 2 : 0);
    constexpr int DPS = (GPW + SP) / (1 + SP);

    const int wn = wave % WN, wm = wave / WN;
    // lane l of a fragment holds row l % R and the 8 k values of chunk l / R of its K step
    const int lr = lane % R, lh = lane / R;
    // byte offsets of this lane's first A and B fragment rows within a slot, per
    // K step.  Fragment i sits R i rows further down and R / RP is a multiple of
    // CPR, so the swizzle term (r / RP) % CPR is the same for every fragment: the
    // others are the first one's offset plus a constant (the read's immediate)
    static_assert((R / RP) % CPR == 0, "fragment blocks must keep their rows' swizzle");
    uint32_t aoff[KS], boff[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int ra = wn * TN + lr, rb = BN + wm * TM + lr;
        aoff[ks] = ra * ROWB + (((ks * (KSTEP / 8) + lh) ^ ((ra / RP) % CPR)) << 4);
        boff[ks] = rb * ROWB + (((ks * (KSTEP / 8) + lh) ^ ((rb / RP) % CPR)) << 4);
    }
    constexpr uint32_t FRAGB = R * ROWB;              // bytes between a wave's fragment blocks
    auto mma = [](u32x4 x, u32x4 y, AccT c) {
        if constexpr (M16) return mfma16x16x32<E>(x, y, c);
        else return mfma32x32x16<E>(x, y, c);
    };

    AccT acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = (AccT){};

    if constexpr (WHOLE) {
        // at most c (< STAGES, uniform) slices' requests left in flight
        auto wait_behind = [&](int c) {
            static_for<0, STAGES>([&]<int k>() {
                if (c == k) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(k * GPW) : "memory");
            });
        };
        if (nk > 0) {
            const int pro = nk < STAGES ? nk : STAGES;
            for (int t = 0; t < pro; ++t) static_for<0, GPW>([&]<int j>() { LIN_ISSUE_ONE(t, j); });
            wait_behind(pro - 1);
            lds_barrier();
        }
        for (int t = 0; t < nk; ++t) {
            // slot t - 1 is refilled once the barrier shows that slice t has
            // landed and that every wave has read slice t - 1
            if (t > 0) {
                wait_behind(min(STAGES - 2, nk - 1 - t));
                lds_barrier();
            }
            const unsigned char* slot = smem + (t % STAGES) * SLICE;
            u32x4 fa[KS][FN], fb[KS][FM];
            static_for<0, KS>([&]<int ks>() {
#pragma unroll
                for (int i = 0; i < FN; ++i) fa[ks][i] = *(const u32x4*)(slot + aoff[ks] + i * FRAGB);
#pragma unroll
                for (int j = 0; j < FM; ++j) fb[ks][j] = *(const u32x4*)(slot + boff[ks] + j * FRAGB);
            });
            __builtin_amdgcn_sched_barrier(0);   // every read issued before the refill and the MFMAs
            if (t > 0 && t - 1 + STAGES < nk) static_for<0, GPW>([&]<int j>() { LIN_ISSUE_ONE(t - 1 + STAGES, j); });
            __builtin_amdgcn_sched_barrier(0);
            static_for<0, KS>([&]<int ks>() {
#pragma unroll
                for (int i = 0; i < FN; ++i)
#pragma unroll
                    for (int j = 0; j < FM; ++j) acc[i][j] = mma(fa[ks][i], fb[ks][j], acc[i][j]);
            });
        }
    } else if (nk > 0) {
        // Requests past the last slice carry out-of-range offsets (zero fill, no
        // memory traffic), so the number of requests behind any slice is fixed and
        // every wait below is static.  The prologue issues slices 0 .. STAGES-2 and
        // the first DPS loads of slice STAGES-1, as the steady state would have.
#pragma unroll
        for (int t = 0; t < STAGES; ++t)
#pragma unroll
            for (int j = 0; j < GPW; ++j)
                if (t + 1 < STAGES || j < DPS) LIN_ISSUE_ONE(t, j);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((STAGES - 2) * GPW + DPS) : "memory");
        lds_barrier();   // slice 0 only: __syncthreads() would also wait for every later slice

        if constexpr (M16) {
        // 16 x 16 x 32 MFMAs (two K steps per 64-wide slice).  A wave's FN A
        // fragments are double buffered and its FM B fragments single: each step
        // runs its MFMAs B-fragment-major and reads the next step's B fragment j
        // right after the FN MFMAs that use fragment j have been issued (the
        // registers allow no second B buffer next to 128 accumulators).
        static_assert(KS == 2, "the 16 x 16 x 32 loop takes 64-wide slices");
        u32x4 a2[2][FN], b1[FM];
#pragma unroll
        for (int i = 0; i < FN; ++i) a2[0][i] = *(const u32x4*)(smem + aoff[0] + i * FRAGB);
#pragma unroll
        for (int j = 0; j < FM; ++j) b1[j] = *(const u32x4*)(smem + boff[0] + j * FRAGB);
        // the MFMAs of the step held in buffer CUR while the step NKS of nslot is read
        auto step = [&]<int CUR, int NKS>(const unsigned char* nslot) {
#pragma unroll
            for (int i = 0; i < FN; ++i) a2[CUR ^ 1][i] = *(const u32x4*)(nslot + aoff[NKS] + i * FRAGB);
#pragma unroll
            for (int j = 0; j < FM; ++j) {
#pragma unroll
                for (int i = 0; i < FN; ++i) acc[i][j] = mma(a2[CUR][i], b1[j], acc[i][j]);
                b1[j] = *(const u32x4*)(nslot + boff[NKS] + j * FRAGB);
            }
        };
        for (int t = 0; t + 1 < nk; ++t) {
            step.template operator()<0, 1>(smem + (t % STAGES) * SLICE);
            order_step16<FN, FM, 0>();
            // slice t + 1 has landed and every wave has read slot t's last step
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"((STAGES - 2) * GPW) : "memory");
            lds_barrier();
            step.template operator()<1, 0>(smem + ((t + 1) % STAGES) * SLICE);
            static_for<0, GPW>([&]<int j>() { LIN_ISSUE_ONE(t + STAGES, j); });
            order_step16<FN, FM, GPW>();
        }
        if constexpr (MODE == kOutBias) request_bias();
        step.template operator()<0, 1>(smem + ((nk - 1) % STAGES) * SLICE);
        order_step16<FN, FM, 0>();
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int i = 0; i < FN; ++i) acc[i][j] = mma(a2[1][i], b1[j], acc[i][j]);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        } else {
        u32x4 af[2][FN], bf[2][FM];
#pragma unroll
        for (int i = 0; i < FN; ++i) af[0][i] = *(const u32x4*)(smem + aoff[0] + i * FRAGB);
#pragma unroll
        for (int j = 0; j < FM; ++j) bf[0][j] = *(const u32x4*)(smem + boff[0] + j * FRAGB);

        auto read_frags = [&](const unsigned char* slot, int ks, int buf) {
#pragma unroll
            for (int i = 0; i < FN; ++i) af[buf][i] = *(const u32x4*)(slot + aoff[ks] + i * FRAGB);
#pragma unroll
            for (int j = 0; j < FM; ++j) bf[buf][j] = *(const u32x4*)(slot + boff[ks] + j * FRAGB);
        };
        auto mfmas = [&](int buf) {
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j)
                    acc[i][j] = mma(af[buf][i], bf[buf][j], acc[i][j]);
        };
        // K steps 0 .. KS-2 of slice t: read the next step while this one
        // multiplies; the first SP steps also issue the deferred loads of
        // slice t - 1 + STAGES
        auto inner_steps = [&](int t) {
            const unsigned char* slot = smem + (t % STAGES) * SLICE;
            static_for<0, KS - 1>([&]<int ks>() {
                read_frags(slot, ks + 1, (ks + 1) & 1);
                mfmas(ks & 1);
                constexpr int j0 = ks < SP ? DPS * (ks + 1) : GPW;
                constexpr int j1 = ks < SP ? (DPS * (ks + 2) < GPW ? DPS * (ks + 2) : GPW) : GPW;
                static_for<j0, j1>([&]<int j>() { LIN_ISSUE_ONE(t - 1 + STAGES, j); });
                order_step<FN * FM, FN + FM, (j1 > j0 ? j1 - j0 : 0)>();
            });
        };

        for (int t = 0; t + 1 < nk; ++t) {
            inner_steps(t);
            // slice t + 1 has landed once only the later slices' requests are
            // outstanding; the barrier also waits for every wave's last reads of
            // slot t, which the refill below overwrites
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"((STAGES - 2) * GPW) : "memory");
            lds_barrier();
            read_frags(smem + ((t + 1) % STAGES) * SLICE, 0, KS & 1);
            mfmas((KS - 1) & 1);
            constexpr int D0 = DPS < GPW ? DPS : GPW;
            static_for<0, D0>([&]<int j>() { LIN_ISSUE_ONE(t + STAGES, j); });
            order_step<FN * FM, FN + FM, D0>();
        }
        inner_steps(nk - 1);
        mfmas((KS - 1) & 1);
        // the zero-fill requests past the end must land before the LDS is released
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
    }
#undef LIN_ISSUE_ONE
    // with no K slice at all the 16 x 16 x 32 loop did not run: the bias chunk still goes in
    if constexpr (MODE == kOutBias && LATE_BIAS) {
        if (nk == 0) request_bias();
    }
    finish_tile<BM, BN, WM, WN, STAGES * SLICE, E, MODE, R>(a, smem, acc, m0, n0, wave, lane,
                                                           MODE == kOutBias ? &bias8 : nullptr);
}

// ---------------------------------------------------------------------------
// Launchers (instantiated once per element type in gemm_f16.hip / gemm_bf16.hip).

template <int BM, int BN, int WM, int WN, int E>
static const void* regstaged_fn(int mode) {
    if (mode == kOutBias) return (const void*)gemm_kernel<BM, BN, WM, WN, E, kOutBias>;
    if (mode == kOutRound) return (const void*)gemm_kernel<BM, BN, WM, WN, E, kOutRound>;
    if (mode == kOutEpi) return (const void*)gemm_kernel<BM, BN, WM, WN, E, kOutEpi>;
    return (const void*)gemm_kernel<BM, BN, WM, WN, E, kOutF32>;
}

template <int BM, int BN, int WM, int WN, int STAGES, int BK, int E, int SPREAD, bool WHOLE = false, bool M16 = false>
static const void* stream_fn(int mode) {
    if (mode == kOutBias)
        return (const void*)gemm_stream<BM, BN, WM, WN, STAGES, BK, E, kOutBias, SPREAD, WHOLE, M16>;
    if (mode == kOutRound)
        return (const void*)gemm_stream<BM, BN, WM, WN, STAGES, BK, E, kOutRound, SPREAD, WHOLE, M16>;
    if (mode == kOutEpi) return (const void*)gemm_stream<BM, BN, WM, WN, STAGES, BK, E, kOutEpi, SPREAD, WHOLE, M16>;
    return (const void*)gemm_stream<BM, BN, WM, WN, STAGES, BK, E, kOutF32, SPREAD, WHOLE, M16>;
}

static hipError_t launch(const void* fn, const LinearArgs& a, int threads, hipStream_t stream) {
    LinearArgs args = a;
    void* params[] = {&args};
    return hipLaunchKernel(fn, dim3((unsigned)(a.tiles_m * a.tiles_n), 1, (unsigned)a.groups), dim3(threads), params,
                           0, stream);
}

template <int E>
hipError_t launch_gemm_t(int cfg, const LinearArgs& a, int mode, hipStream_t stream) {
    switch (cfg) {
        case 0: return launch(regstaged_fn<128, 128, 2, 2, E>(mode), a, 256, stream);
        case 1: return launch(regstaged_fn<64, 64, 2, 2, E>(mode), a, 256, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int E>
hipError_t launch_gemm_stream_t(int cfg, const LinearArgs& a, int mode, hipStream_t stream) {
    switch (cfg) {
        // load spread (K steps a slice's refill is spread over), measured per tile
        // with the ring's own barriers: 256 x 256 best at 1, 256 x 128 and 128 x 128
        // at 2 (down 241 -> 222 us); 128 x 256 (32-wide slices) has no step to
        // spare.  64 x 64 reads whole slices (toy layer: 6.94 us per call against
        // 7.17 pipelined; rings of 3, 5 or 6 slots 7.6-8.1).  The 256 x 256 tile
        // multiplies with 16 x 16 x 32 MFMAs (attn 232 -> 226 us, mlp_up 408 ->
        // 400); the smaller tiles measured slower with them (down +4%, 128 x 128
        // +15%) and keep 32 x 32 x 16
        case 0: return launch(stream_fn<256, 256, 2, 4, 2, 64, E, 1, false, true>(mode), a, 512, stream);
        case 1: return launch(stream_fn<256, 128, 4, 2, 3, 64, E, 2>(mode), a, 512, stream);
        case 2: return launch(stream_fn<128, 256, 2, 4, 4, 32, E, 0>(mode), a, 512, stream);
        case 3: return launch(stream_fn<128, 128, 2, 2, 4, 64, E, 2>(mode), a, 256, stream);
        case 4: return launch(stream_fn<64, 64, 2, 2, 4, 64, E, 0, true>(mode), a, 256, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace lin
