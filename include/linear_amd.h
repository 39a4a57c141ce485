/*
 * linear_amd.h -- C ABI of the MI355X (gfx950) FP16 linear layer.
 *
 *     proj[m,n] = FP16( sum_k x[m,k] * weight[n,k] )     products exact, FP32 accumulation
 *     y[m,n]    = FP16( FP32(proj[m,n]) + FP32(b[n]) )
 *
 * This is the computation and numerical contract of "tensor programs, part 1":
 * the PyTorch line y = torch.matmul(x, weight.T) + b and Figure 1.1 (the weight
 * transpose is a view, the projection is rounded before the bias add), the
 * contraction formula of section "One Program and One Numerical Contract" and its
 * two requirements (FP32 accumulation of unrounded products in any order; the
 * projection rounded to FP16 before the bias addition, output FP16), and the
 * Inductor capture's epilogue (both operands widened to f32, added, rounded to
 * f16).  The weight is contracted in its stored [N, K] order with no transposed or
 * widened copy, as "The Graph IR" op table describes a dense contraction
 * (DenseContraction).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Binary16 values are passed as uint16_t words (their IEEE 754 bit patterns).
 *  - x is [M, K] with row stride ldx >= K, weight is [N, K] with row stride
 *    ldw >= K (the [out_features, in_features] layout), y is [M, N] with row
 *    stride ldy >= N; strides are in elements, the inner stride is 1.  b is [N],
 *    contiguous.
 *  - All data pointers are DEVICE pointers owned by the caller.  The library
 *    neither allocates, frees nor keeps them after the call returns.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL means the default stream)
 *    and the call returns without synchronising.  Results are visible after the
 *    stream is synchronised.  A call enqueues kernel launches only (one, or two:
 *    a column split of a large GEMM, see linear_plan, and the indexed call's
 *    routing pass), no allocation, copy or memset, so it can be captured into a
 *    HIP graph (the first activation call on a device excepted, see below).
 *  - Only y[m, n] for m < M, n < N is written; stride padding is never touched.
 *  - Rounding is IEEE round-to-nearest-even with subnormals kept (no flush to
 *    zero) and overflow to infinity; the empty sum (K == 0) is +0.
 *  - For given shapes, the bias call and the bias-less call use the same
 *    summation order, so y of the bias call equals FP16(FP32(p) + FP32(b)) where
 *    p is the bias-less result, bit for bit.  Reruns are bit-identical.
 *  - Every argument error is detected on the host before anything is enqueued;
 *    y is then untouched.  No exception or abort crosses this ABI.
 *  - Limits: M, N, K < 2^31; ldx, ldw < 2^22 and ldy < 2^31 elements.
 *  - Fast path: x and weight 16-byte aligned, ldx, ldw and K multiples of 8.
 *    Any other layout is accepted and runs a slower element-wise loader.
 */
#ifndef LINEAR_AMD_H
#define LINEAR_AMD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Status codes.  Every entry point returns one: a call the library cannot run is
 * refused with a typed error before anything is enqueued, never a crash or an
 * abort, as the pages' builder refuses ill-formed ops with a typed error rather
 * than a panic ("Tracing a Model", section "The Builder and Traced handles";
 * "The Graph IR", section "Graph structure": shapes and dtypes are checked when
 * an op is added).
 */
#define LINEAR_OK         0
#define LINEAR_E_NULL     1  /* a required pointer is NULL (only when the output is non-empty) */
#define LINEAR_E_SHAPE    2  /* M, N or K negative, or beyond the limits above */
#define LINEAR_E_STRIDE   3  /* ldx < K, ldw < K, ldy < N, or a stride beyond its limit */
#define LINEAR_E_ALIAS    4  /* y's byte range overlaps x, weight or b */
#define LINEAR_E_PATH     5  /* unknown path selector */
#define LINEAR_E_DEVICE   6  /* no usable gfx950 device current, or a HIP query failed */
#define LINEAR_E_LAUNCH   7  /* a kernel launch failed; linear_last_hip_error() has the HIP code */
#define LINEAR_E_EPILOGUE 8  /* epilogue program: step count outside 0..LINEAR_EPI_MAX_STEPS or an unknown step */
#define LINEAR_E_CAPTURE  9  /* the first activation epilogue on a device was called under stream capture */
#define LINEAR_E_WORKSPACE 10 /* indexed contraction: workspace misaligned or below linear_indexed_workspace_bytes */
#define LINEAR_E_SCRATCH  11  /* linear_f16_indexed_noalloc: the call needs more than LINEAR_NOALLOC_SCRATCH_BYTES */

/*
 * Path selectors for linear_f16_ex / linear_f16_plan.  The path and the tile are
 * chosen on the host from the static shapes before any launch: the op table
 * treats GEMV and GEMM as one MatMul op specialised when the call is planned, and
 * shapes are inferred on the host ("The Graph IR", op table, MatMul row, and
 * section "Host-side shape inference").  AUTO is that specialisation; the forced
 * paths give results within the same contract.
 */
#define LINEAR_PATH_AUTO   0  /* M <= 16: skinny path; otherwise the MFMA tiled GEMM */
#define LINEAR_PATH_GEMM   1  /* force the MFMA tiled GEMM (any M) */
#define LINEAR_PATH_SKINNY 2  /* force the weight-streaming skinny path (any M, 16 rows per block;
                                 at M == 1 with the fast-path layout, no epilogue program, one group
                                 and K <= 32768: one wave per weight row, 4 rows per block) */

/*
 * y = FP16(FP16(x . weight^T) + b).  See the conventions above.
 * M == 0 or N == 0 is a successful no-op (pointers may then be NULL).
 * Returns LINEAR_OK or one of the LINEAR_E_* codes.
 */
int32_t linear_f16(const uint16_t* x, int64_t ldx,
                   const uint16_t* weight, int64_t ldw,
                   const uint16_t* b,
                   uint16_t* y, int64_t ldy,
                   int64_t M, int64_t N, int64_t K,
                   void* stream);

/*
 * The projection alone: y = FP16(x . weight^T), no bias.  Same conventions.
 */
int32_t linear_f16_nobias(const uint16_t* x, int64_t ldx,
                          const uint16_t* weight, int64_t ldw,
                          uint16_t* y, int64_t ldy,
                          int64_t M, int64_t N, int64_t K,
                          void* stream);

/*
 * linear_f16 with an explicit path (LINEAR_PATH_*) and an optional bias
 * (b == NULL computes the projection alone).  Every path gives results within
 * the same contract; forcing one lets tests exercise both on every shape.
 */
int32_t linear_f16_ex(const uint16_t* x, int64_t ldx,
                      const uint16_t* weight, int64_t ldw,
                      const uint16_t* b,
                      uint16_t* y, int64_t ldy,
                      int64_t M, int64_t N, int64_t K,
                      int32_t path, void* stream);

/*
 * The unrounded FP32 sums: y[m,n] = sum_k x[m,k] * weight[n,k] accumulated in FP32
 * (products exact), stored as float with row stride ldy (elements).  No rounding,
 * no bias.  This is the op table's DenseContraction with an f32 output ("The
 * Graph IR", op table) and the rank-local partial product that a K-split tensor
 * parallel layer all-reduces before rounding and adding the bias ("Model and
 * Distributed IR", section "Boundary between the layers"; rounding per rank would
 * break the projection-rounding requirement).  Same conventions otherwise; path
 * as in linear_f16_ex.  Fast path additionally needs y 16-byte aligned.
 */
int32_t linear_f16_f32out(const uint16_t* x, int64_t ldx,
                          const uint16_t* weight, int64_t ldw,
                          float* y, int64_t ldy,
                          int64_t M, int64_t N, int64_t K,
                          int32_t path, void* stream);

/*
 * The same layer with bfloat16 x, weight, b and y (words are the upper halves of
 * binary32): FP32 accumulation, the projection rounded to bfloat16 (round to
 * nearest even) before the bias, then y = BF16(FP32(proj) + FP32(b[n])).  This
 * is the BF16 form of the contraction epilogue ("The Graph IR", op table:
 * ContractionEpilogue, a BF16 head rounds to BF16 before the first epilogue step;
 * Cast to bf16 rounds to bf16 precision).  bfloat16 x bfloat16 products are exact
 * in FP32 unless they leave its normal range.  Conventions, status codes, paths
 * and limits as for the binary16 entry points.
 */
int32_t linear_bf16(const uint16_t* x, int64_t ldx,
                    const uint16_t* weight, int64_t ldw,
                    const uint16_t* b,
                    uint16_t* y, int64_t ldy,
                    int64_t M, int64_t N, int64_t K,
                    void* stream);

int32_t linear_bf16_nobias(const uint16_t* x, int64_t ldx,
                           const uint16_t* weight, int64_t ldw,
                           uint16_t* y, int64_t ldy,
                           int64_t M, int64_t N, int64_t K,
                           void* stream);

int32_t linear_bf16_ex(const uint16_t* x, int64_t ldx,
                       const uint16_t* weight, int64_t ldw,
                       const uint16_t* b,
                       uint16_t* y, int64_t ldy,
                       int64_t M, int64_t N, int64_t K,
                       int32_t path, void* stream);

/* The unrounded FP32 sums for bfloat16 operands (see linear_f16_f32out). */
int32_t linear_bf16_f32out(const uint16_t* x, int64_t ldx,
                           const uint16_t* weight, int64_t ldw,
                           float* y, int64_t ldy,
                           int64_t M, int64_t N, int64_t K,
                           int32_t path, void* stream);

/*
 * Multi-step contraction epilogue ("The Graph IR", op table: ContractionEpilogue,
 * whose extra inputs are the bias, a residual and so on: the head contraction's
 * result keeps its dtype and every step rounds through it), with the activation
 * compositions of "Tracing a Model" (the gated feed-forward section: SiLU as
 * x / (1 + exp(-x)) over Neg, Exp, Add and Div; the tanh GeLU in the same
 * sigmoid form, x / (1 + exp(-2 sqrt(2/pi) (x + 0.044715 x^3))); the exact GeLU
 * (x (1 + erf(x / sqrt 2))) * 0.5 on the Erf primitive).
 *
 *     t = RNE_E( sum_k x[m,k] * weight[n,k] )          the projection, as linear_*_nobias
 *     for each step s: t = step_s(t)                    each result rounded to E
 *     y[m,n] = t
 *
 * Steps (op[s]):
 *   LINEAR_EPI_BIAS       t + bias[n]
 *   LINEAR_EPI_RESIDUAL   t + residual[m * ldr + n]
 *   LINEAR_EPI_MUL        t * mul[m * ldm + n]     (the gate product of a gated feed-forward)
 *   LINEAR_EPI_SILU, LINEAR_EPI_GELU_TANH, LINEAR_EPI_GELU_ERF
 * Every primitive of a step (each Add, Mul, Div, Neg, Exp, Erf of a composition,
 * left to right, x^3 as (x*x)*x) returns its exact result rounded to E, round to
 * nearest even; the constants 1, 0.5, 0.044715, -2 sqrt(2/pi) and 1/sqrt 2 are
 * E values (their real value rounded to E).  IEEE special values propagate
 * (e.g. SiLU of -inf is NaN: -inf / inf).
 *
 * bias, residual and mul are device words of the call's element type, caller
 * owned; each is read only by the steps that name it and may be NULL otherwise.
 * y may be the residual itself (same pointer, ldr == ldy: y = ... + y in place);
 * any other overlap of y with an input is LINEAR_E_ALIAS.  The program is read
 * when the call is made (the struct may be reused right after the call returns).
 * The activation steps use tables the library builds on the device at the first
 * such call per device and element type: that call waits for the build on
 * `stream`, and made under stream capture it returns LINEAR_E_CAPTURE with
 * nothing enqueued.  With no steps the call is linear_*_nobias; with the single
 * step LINEAR_EPI_BIAS it gives the bits of linear_*.
 */
#define LINEAR_EPI_MAX_STEPS 8
#define LINEAR_EPI_BIAS      1
#define LINEAR_EPI_RESIDUAL  2
#define LINEAR_EPI_MUL       3
#define LINEAR_EPI_SILU      4
#define LINEAR_EPI_GELU_TANH 5
#define LINEAR_EPI_GELU_ERF  6

typedef struct linear_epilogue {
    int32_t nsteps;                        /* 0 .. LINEAR_EPI_MAX_STEPS */
    int32_t op[LINEAR_EPI_MAX_STEPS];      /* LINEAR_EPI_*, applied in index order */
    const uint16_t* bias;                  /* [N] */
    const uint16_t* residual;              /* [M, N], row stride ldr >= N */
    int64_t ldr;
    const uint16_t* mul;                   /* [M, N], row stride ldm >= N */
    int64_t ldm;
} linear_epilogue;

int32_t linear_f16_epilogue(const uint16_t* x, int64_t ldx,
                            const uint16_t* weight, int64_t ldw,
                            const linear_epilogue* epilogue,
                            uint16_t* y, int64_t ldy,
                            int64_t M, int64_t N, int64_t K,
                            int32_t path, void* stream);

/* The same with bfloat16 x, weight, epilogue inputs and y. */
int32_t linear_bf16_epilogue(const uint16_t* x, int64_t ldx,
                             const uint16_t* weight, int64_t ldw,
                             const linear_epilogue* epilogue,
                             uint16_t* y, int64_t ldy,
                             int64_t M, int64_t N, int64_t K,
                             int32_t path, void* stream);

/*
 * Grouped contraction ("The Graph IR", op table: GroupedDenseContraction): a
 * [G*N, K] weight read in place as G blocks of N rows against a [G, M, K]
 * activation, giving [G, M, N]:
 *
 *     y[g, m, n] = RNE_E( sum_k x[g, m, k] * weight[g*N + n, k] )   (+ b[g*N + n] as in linear_*)
 *
 * x: group g at x + g * sx, rows with stride ldx (sx in elements, >= 0; slices may
 * overlap, they are only read); weight: [G*N, K] with row stride ldw; b: [G*N] or
 * NULL (NULL: the projection alone); y: group g at y + g * sy, row stride ldy,
 * sy >= (M-1)*ldy + N so that groups write disjoint outputs.  Element type,
 * rounding, bias epilogue, paths, reruns and errors as for linear_f16_ex (G up to
 * 65535); each group is exactly linear_f16_ex on its slices.  The _f32out forms
 * return the unrounded FP32 sums (the op table gives this contraction an f32
 * output).  The op table's f32 activation is read here in the weight's element
 * type: the MFMA path multiplies 16-bit operands.
 */
int32_t linear_f16_grouped(const uint16_t* x, int64_t ldx, int64_t sx,
                           const uint16_t* weight, int64_t ldw,
                           const uint16_t* b,
                           uint16_t* y, int64_t ldy, int64_t sy,
                           int64_t G, int64_t M, int64_t N, int64_t K,
                           int32_t path, void* stream);
int32_t linear_bf16_grouped(const uint16_t* x, int64_t ldx, int64_t sx,
                            const uint16_t* weight, int64_t ldw,
                            const uint16_t* b,
                            uint16_t* y, int64_t ldy, int64_t sy,
                            int64_t G, int64_t M, int64_t N, int64_t K,
                            int32_t path, void* stream);
int32_t linear_f16_grouped_f32out(const uint16_t* x, int64_t ldx, int64_t sx,
                                  const uint16_t* weight, int64_t ldw,
                                  float* y, int64_t ldy, int64_t sy,
                                  int64_t G, int64_t M, int64_t N, int64_t K,
                                  int32_t path, void* stream);
int32_t linear_bf16_grouped_f32out(const uint16_t* x, int64_t ldx, int64_t sx,
                                   const uint16_t* weight, int64_t ldw,
                                   float* y, int64_t ldy, int64_t sy,
                                   int64_t G, int64_t M, int64_t N, int64_t K,
                                   int32_t path, void* stream);

/*
 * Indexed contraction ("The Graph IR", op table: IndexedMatMul; "Tracing a
 * Model", section "Mixture-of-experts routing": each row contracts against its
 * own expert, the expert tables read in place):
 *
 *     y[m, n] = RNE_E( sum_k x[m, k] * w[idx[m], k, n] )      (FP32 accumulation)
 *
 * x: [M, K], row stride ldx >= K.  w: E expert tables of [K, N] (k first, n
 * contiguous): element (e, k, n) at w[e * sw + k * ldw + n], ldw >= N,
 * sw >= K * ldw.  idx: [M] device int32.  y: [M, N], row stride ldy >= N.  A row
 * whose idx lies outside [0, E) has no expert and its outputs are left untouched.
 * Only rows m < M and columns n < N are written; reruns are bit-identical.
 * E up to 65535; M, N, K < 2^31.  The _f32out forms store the unrounded sums.
 *
 * workspace: device memory of at least linear_indexed_workspace_bytes(E, M)
 * bytes, 16-byte aligned, owned by the caller, overwritten by the call (it holds
 * the row-to-expert binning) and free again once the call's work on `stream`
 * has finished; two calls in flight at once need two workspaces.
 *
 * Errors as for linear_f16_ex (y or the workspace overlapping x, w, idx or each
 * other is LINEAR_E_ALIAS; a NULL workspace is LINEAR_E_NULL, a short or
 * misaligned one LINEAR_E_WORKSPACE); E == 0, M == 0 or N == 0 is a successful
 * no-op that touches nothing.
 */
int64_t linear_indexed_workspace_bytes(int64_t E, int64_t M);   /* -1 if E or M is out of range */
int32_t linear_f16_indexed(const uint16_t* x, int64_t ldx,
                           const uint16_t* w, int64_t ldw, int64_t sw,
                           const int32_t* idx,
                           uint16_t* y, int64_t ldy,
                           int64_t E, int64_t M, int64_t N, int64_t K,
                           void* workspace, int64_t workspace_bytes, void* stream);
int32_t linear_bf16_indexed(const uint16_t* x, int64_t ldx,
                            const uint16_t* w, int64_t ldw, int64_t sw,
                            const int32_t* idx,
                            uint16_t* y, int64_t ldy,
                            int64_t E, int64_t M, int64_t N, int64_t K,
                            void* workspace, int64_t workspace_bytes, void* stream);
int32_t linear_f16_indexed_f32out(const uint16_t* x, int64_t ldx,
                                  const uint16_t* w, int64_t ldw, int64_t sw,
                                  const int32_t* idx,
                                  float* y, int64_t ldy,
                                  int64_t E, int64_t M, int64_t N, int64_t K,
                                  void* workspace, int64_t workspace_bytes, void* stream);
int32_t linear_bf16_indexed_f32out(const uint16_t* x, int64_t ldx,
                                   const uint16_t* w, int64_t ldw, int64_t sw,
                                   const int32_t* idx,
                                   float* y, int64_t ldy,
                                   int64_t E, int64_t M, int64_t N, int64_t K,
                                   void* workspace, int64_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): linear_f16_indexed
 * without the workspace argument.  Same arguments otherwise, same kernels, same
 * results bit for bit, same errors, except that the row-to-expert binning goes
 * into a scratch array of LINEAR_NOALLOC_SCRATCH_BYTES that the library holds in
 * device memory (one per GPU, from the first such call on that GPU until the
 * process ends).  A call whose binning needs more, i.e.
 * linear_indexed_workspace_bytes(E, M) > LINEAR_NOALLOC_SCRATCH_BYTES (about
 * 200,000 rows at a few experts), returns LINEAR_E_SCRATCH with nothing
 * enqueued.  The call allocates nothing and frees nothing; nothing in the
 * scratch array needs clearing between calls (each call's routing pass writes
 * every word its kernels read).  All such calls on one GPU share that GPU's
 * array: two of them in flight at once on that GPU (on different streams, or
 * captured graphs replayed concurrently) race and may give wrong results; calls
 * in one stream's order are safe.
 */
#define LINEAR_NOALLOC_SCRATCH_BYTES (1 << 20)
int32_t linear_f16_indexed_noalloc(const uint16_t* x, int64_t ldx,
                                   const uint16_t* w, int64_t ldw, int64_t sw,
                                   const int32_t* idx,
                                   uint16_t* y, int64_t ldy,
                                   int64_t E, int64_t M, int64_t N, int64_t K,
                                   void* stream);

/* Which kernels a call would launch: the host-side plan of "The Graph IR" (op
 * table, MatMul row: GEMV versus GEMM chosen at plan time; section "Host-side
 * shape inference").  Enqueues nothing and touches no device memory; the tile
 * rules count the compute units of the current device when a gfx950 is current
 * (a partitioned part has fewer), else those of a whole MI355X (256).
 * A GEMM call whose largest tiles would leave a last wave of workgroups at most
 * half full over the GPU's CUs is split by output columns into two launches of
 * the same kernel family: columns [0, split_n) in whole waves of the first tile,
 * columns [split_n, N) with the tile chosen for that part alone. */
typedef struct linear_plan {
    int32_t path;       /* LINEAR_PATH_GEMM or LINEAR_PATH_SKINNY */
    int32_t tile_m;     /* output rows (m) per workgroup */
    int32_t tile_n;     /* output columns (n) per workgroup */
    int32_t tile_k;     /* K elements per main-loop stage (GEMM), per wave step (skinny) or per wave
                           load (skinny at M == 1: tile_m 1, tile_n 4) */
    int32_t threads;    /* threads per workgroup */
    int32_t vector_io;  /* 1: 16-byte loads; 0: element-wise loader */
    int64_t grid;       /* workgroups launched (the first launch when split) */
    int64_t split_n;    /* 0: one launch; else the first column of the second launch */
    int32_t tile_m2;    /* the second launch's tile (0 when not split) */
    int32_t tile_n2;
    int64_t grid2;      /* the second launch's workgroups (0 when not split) */
    int32_t stages;     /* GEMM: slices of tile_k K in its LDS ring (0 for the skinny path) */
} linear_plan;

/*
 * Fill *plan for a call with these shapes, strides, alignments and path, after
 * the same validation as linear_f16_ex (device pointers are only inspected for
 * alignment, never dereferenced).  Returns LINEAR_OK or a LINEAR_E_* code.
 */
int32_t linear_f16_plan(const uint16_t* x, int64_t ldx,
                        const uint16_t* weight, int64_t ldw,
                        const uint16_t* b,
                        uint16_t* y, int64_t ldy,
                        int64_t M, int64_t N, int64_t K,
                        int32_t path, linear_plan* plan);

/* Static English text for a status code (never NULL). */
const char* linear_status_string(int32_t status);

/* The hipError_t of the last LINEAR_E_DEVICE / LINEAR_E_LAUNCH on this thread (0 if none). */
int32_t linear_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LINEAR_AMD_H */
