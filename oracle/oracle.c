/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * The plain, slow, obviously correct CPU definition of the FP16 linear layer
 *
 *     proj[m,n] = FP16( sum_k x[m,k] * weight[n,k] )      (FP32 accumulation)
 *     y[m,n]    = FP16( FP32(proj[m,n]) + FP32(b[n]) )
 *
 * as fixed by "tensor programs, part 1", section "One Program and One Numerical
 * Contract" (the contraction formula and its two numbered requirements: FP32
 * matrix arithmetic with products not rounded to FP16, any summation order;
 * the projection rounded to FP16 before the bias is added, output FP16) and by
 * the Inductor capture in section "Inductor Retains MatMul and Explicit Casts"
 * (the rounded mm result and the bias are both widened to f32, added in f32,
 * and the sum is converted back to f16).
 *
 * Nothing on the GPU path calls, links or includes this file.  Only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg load it.  It
 * shares no source with the HIP library: every conversion below is written out
 * from the IEEE 754 binary16 / binary32 encodings, not taken from a compiler
 * intrinsic or a library.
 *
 * The same definition with bfloat16 operands ("The Graph IR", op table: a Cast
 * to bf16 rounds to bf16 precision; ContractionEpilogue: a BF16 head rounds to
 * BF16 before the first epilogue step reads it) and the unrounded FP32 sum (the op
 * table's DenseContraction produces f32) are provided too, and so is the
 * multi-step contraction epilogue (bias, residual, multiply, SiLU and GeLU
 * compositions, each primitive rounding through the element type; at the end of
 * this file).
 *
 * Readings where the pages are silent (all listed in the design notes):
 *   - "rounded to FP16" is IEEE roundTiesToEven, with gradual underflow
 *     (subnormals kept) and overflow to infinity;
 *   - of the many summation orders the contract allows, the oracle takes the
 *     plain sequential one, k = 0, 1, ..., K-1, starting from +0;
 *   - K == 0 is the empty sum (+0).
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC
 * (no reassociation; an FMA would give the same bits anyway because every
 * product of two binary16 values is exact in binary32).
 */
#include <stdint.h>
#include <string.h>
#include <math.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------------------
 * binary16 -> binary32, from the encoding: 1 sign bit, 5 exponent bits (bias
 * 15), 10 fraction bits.  Exponent field 0 is zero/subnormal (value
 * fraction * 2^-24), field 31 is infinity/NaN.  Every binary16 value is exactly
 * representable in binary32, so this is exact.
 * ------------------------------------------------------------------------- */
static float f32_from_bits(uint32_t u) {
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint32_t bits_from_f32(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

float oracle_f16_to_f32(uint16_t h) {
    uint32_t sign = (uint32_t)(h >> 15) & 1u;
    uint32_t e = (uint32_t)(h >> 10) & 0x1fu;
    uint32_t frac = (uint32_t)h & 0x3ffu;
    float mag;
    if (e == 0u) {
        /* zero or subnormal: frac * 2^-24; frac < 2^10 so the product is exact */
        mag = ldexpf((float)frac, -24);
    } else if (e == 31u) {
        if (frac == 0u) {
            mag = f32_from_bits(0x7f800000u);                       /* infinity */
        } else {
            /* NaN: keep it quiet, carry the fraction into the top bits */
            mag = f32_from_bits(0x7fc00000u | (frac << 13));
        }
    } else {
        /* normal: (1024 + frac) * 2^(e - 25) */
        mag = ldexpf((float)(1024u + frac), (int)e - 25);
    }
    return sign ? -mag : mag;
}

/* ---------------------------------------------------------------------------
 * binary32 -> binary16, round to nearest, ties to even.
 *
 * A finite non-zero binary32 value is s * 2^(e-23) with s a 24-bit integer in
 * [2^23, 2^24) (normal) -- binary32 subnormals are below 2^-126, far under half
 * of the smallest binary16 subnormal (2^-25), so they round to zero.  The
 * binary16 grid has spacing 2^(e-10) for e >= -14 and 2^-24 below that.  We
 * express the value in units of the target spacing, split off the integer part
 * q and the discarded remainder, and round: up if the remainder is more than
 * half a unit, or exactly half and q is odd.
 * ------------------------------------------------------------------------- */
uint16_t oracle_f32_to_f16(float f) {
    uint32_t u = bits_from_f32(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t be = (u >> 23) & 0xffu;
    uint32_t frac = u & 0x7fffffu;

    if (be == 0xffu) {
        if (frac == 0u) return (uint16_t)(sign | 0x7c00u);          /* +-inf */
        return (uint16_t)(sign | 0x7e00u | (frac >> 13));            /* quiet NaN */
    }
    if (be == 0u) return sign;                   /* +-0 and binary32 subnormals */

    int e = (int)be - 127;                       /* value = s * 2^(e-23) */
    uint32_t s = frac | 0x800000u;
    if (e >= 16) return (uint16_t)(sign | 0x7c00u);   /* >= 2^16: overflow */

    int shift;        /* number of low bits of s below the target spacing */
    int normal = (e >= -14);
    if (normal) {
        shift = 13;                              /* spacing 2^(e-10) = 2^13 units of 2^(e-23) */
    } else {
        shift = -e - 1;                          /* spacing 2^-24: 2^(-24-(e-23)) = 2^(-e-1) */
        if (shift >= 25) return sign;            /* value < 2^-25 ... strictly below half: 0 */
    }
    uint32_t q = s >> shift;
    uint32_t rem = s & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1u))) q += 1u;

    if (normal) {
        /* q in [1024, 2048]; 2048 means the significand carried into the next binade */
        if (q == 2048u) { q = 1024u; e += 1; }
        if (e >= 16) return (uint16_t)(sign | 0x7c00u);
        return (uint16_t)(sign | (uint16_t)(((uint32_t)(e + 15) << 10) | (q - 1024u)));
    }
    /* subnormal: q in [0, 1024]; q == 1024 is exactly the smallest normal, whose
       encoding (exponent field 1, fraction 0) is the integer 1024 itself */
    return (uint16_t)(sign | (uint16_t)q);
}

/* ---------------------------------------------------------------------------
 * bfloat16: by definition the upper 16 bits of a binary32 (1 sign, 8 exponent,
 * 7 fraction bits), so widening places the word in the upper half (exact), and
 * rounding keeps the upper half, rounded to nearest, ties to even, on the
 * discarded lower 16 bits.  A NaN stays a (quiet) NaN; rounding up past the
 * largest finite value carries into the exponent and gives infinity, as IEEE
 * rounding does.
 * ------------------------------------------------------------------------- */
float oracle_bf16_to_f32(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }

uint16_t oracle_f32_to_bf16(float f) {
    uint32_t u = bits_from_f32(f);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0u)
        return (uint16_t)((u >> 16) | 0x0040u);                    /* quiet NaN */
    uint32_t q = u >> 16;
    uint32_t rem = u & 0xffffu;
    if (rem > 0x8000u || (rem == 0x8000u && (q & 1u))) q += 1u;   /* may carry into the exponent */
    return (uint16_t)q;
}

/* Element-type dispatch: 0 = binary16, 1 = bfloat16. */
static float widen16(int elem, uint16_t h) { return elem ? oracle_bf16_to_f32(h) : oracle_f16_to_f32(h); }
static uint16_t narrow16(int elem, float f) { return elem ? oracle_f32_to_bf16(f) : oracle_f32_to_f16(f); }

void oracle_bf16_to_f32_array(const uint16_t* h, float* out, int64_t n) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_to_f32(h[i]);
}

void oracle_f32_to_bf16_array(const float* f, uint16_t* out, int64_t n) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_bf16(f[i]);
}

void oracle_f16_to_f32_array(const uint16_t* h, float* out, int64_t n) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_to_f32(h[i]);
}

void oracle_f32_to_f16_array(const float* f, uint16_t* out, int64_t n) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_f16(f[i]);
}

/* The bias epilogue, one element: widen the rounded projection and the bias to
   FP32, add in FP32, round the sum to FP16 (Inductor capture's cast sequence). */
uint16_t oracle_bias_epilogue(uint16_t proj16, uint16_t b16) {
    float s = oracle_f16_to_f32(proj16) + oracle_f16_to_f32(b16);
    return oracle_f32_to_f16(s);
}

void oracle_bias_epilogue_array(const uint16_t* p, const uint16_t* b, uint16_t* out, int64_t n) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bias_epilogue(p[i], b[i]);
}

/* The bias epilogue for either element type. */
static uint16_t bias_epilogue16(int elem, uint16_t proj16, uint16_t b16) {
    return narrow16(elem, widen16(elem, proj16) + widen16(elem, b16));
}

void oracle_bias_epilogue_elem_array(int elem, const uint16_t* p, const uint16_t* b, uint16_t* out, int64_t n) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = bias_epilogue16(elem, p[i], b[i]);
}

/* The FP32 accumulation for one output element: sequential k order from +0.
   Each product of two binary16 values is exact in binary32 (11 + 11 significand
   bits, exponents within range), so only the additions round. */
static float dot_f32(const float* xr, const float* wr, int64_t K) {
    float acc = 0.0f;
    for (int64_t k = 0; k < K; ++k) acc = acc + xr[k] * wr[k];
    return acc;
}

/* Widen a row-major [rows, cols] binary16 matrix with row stride ld to a dense
   FP32 copy (test-side only; the GPU path never widens). */
static float* widen(int elem, const uint16_t* src, int64_t ld, int64_t rows, int64_t cols) {
    float* dst = (float*)malloc((size_t)(rows > 0 ? rows : 1) * (size_t)(cols > 0 ? cols : 1) * sizeof(float));
    if (!dst) return NULL;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) dst[r * cols + c] = widen16(elem, src[r * ld + c]);
    return dst;
}

/*
 * Full oracle.  x: [M,K] row stride ldx; w: [N,K] row stride ldw (the
 * [out_features, in_features] weight, contracted over its second axis, i.e. the
 * transposed weight is a view); b: [N] or NULL; outputs y and proj: [M,N] row
 * stride ldy (either may be NULL).  With b == NULL, y = proj.  elem: 0 binary16,
 * 1 bfloat16.  y32 (may be NULL): the unrounded FP32 sums, row stride ldy.
 * nthreads <= 0 uses the OpenMP default.  Returns 0, or -1 on allocation failure.
 */
int oracle_linear(int elem, const uint16_t* x, int64_t ldx, const uint16_t* w, int64_t ldw,
                  const uint16_t* b, uint16_t* y, uint16_t* proj, float* y32, int64_t ldy,
                  int64_t M, int64_t N, int64_t K, int nthreads) {
    if (M <= 0 || N <= 0) return 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    float* xf = widen(elem, x, ldx, M, K);
    float* wf = widen(elem, w, ldw, N, K);
    if (!xf || !wf) { free(xf); free(wf); return -1; }
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            float acc = dot_f32(xf + m * K, wf + n * K, K);
            if (y32) y32[m * ldy + n] = acc;
            uint16_t p16 = narrow16(elem, acc);
            if (proj) proj[m * ldy + n] = p16;
            if (y) y[m * ldy + n] = b ? bias_epilogue16(elem, p16, b[n]) : p16;
        }
    }
    free(xf);
    free(wf);
    return 0;
}

int oracle_linear_f16(const uint16_t* x, int64_t ldx, const uint16_t* w, int64_t ldw,
                      const uint16_t* b, uint16_t* y, uint16_t* proj, int64_t ldy,
                      int64_t M, int64_t N, int64_t K, int nthreads) {
    return oracle_linear(0, x, ldx, w, ldw, b, y, proj, NULL, ldy, M, N, K, nthreads);
}

/*
 * The same definition evaluated at a list of output coordinates (ms[i], ns[i]),
 * for full-size problems where the whole triple loop would take minutes.  Any of
 * the outputs may be NULL.  S and A are the FP64 band data: S = sum_k x*w and
 * A = sum_k |x*w|, each product exact in FP64 (used by the tolerance rule).
 */
void oracle_linear_points(int elem, const uint16_t* x, int64_t ldx, const uint16_t* w, int64_t ldw,
                          const uint16_t* b, int64_t K, const int64_t* ms, const int64_t* ns,
                          int64_t count, uint16_t* y_out, uint16_t* proj_out, float* y32_out,
                          double* S_out, double* A_out, int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < count; ++i) {
        const uint16_t* xr = x + ms[i] * ldx;
        const uint16_t* wr = w + ns[i] * ldw;
        float acc = 0.0f;
        double S = 0.0, A = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            float xv = widen16(elem, xr[k]);
            float wv = widen16(elem, wr[k]);
            acc = acc + xv * wv;
            double pd = (double)xv * (double)wv;
            S += pd;
            A += fabs(pd);
        }
        uint16_t p16 = narrow16(elem, acc);
        if (proj_out) proj_out[i] = p16;
        if (y_out) y_out[i] = b ? bias_epilogue16(elem, p16, b[ns[i]]) : p16;
        if (y32_out) y32_out[i] = acc;
        if (S_out) S_out[i] = S;
        if (A_out) A_out[i] = A;
    }
}

void oracle_linear_f16_points(const uint16_t* x, int64_t ldx, const uint16_t* w, int64_t ldw,
                              const uint16_t* b, int64_t K, const int64_t* ms, const int64_t* ns,
                              int64_t count, uint16_t* y_out, uint16_t* proj_out,
                              double* S_out, double* A_out, int nthreads) {
    oracle_linear_points(0, x, ldx, w, ldw, b, K, ms, ns, count, y_out, proj_out, NULL, S_out, A_out, nthreads);
}

/* FP64 band data for a whole [M,N] output (small problems only). */
int oracle_band(int elem, const uint16_t* x, int64_t ldx, const uint16_t* w, int64_t ldw,
                int64_t M, int64_t N, int64_t K, double* S, double* A, int nthreads) {
    if (M <= 0 || N <= 0) return 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    float* xf = widen(elem, x, ldx, M, K);
    float* wf = widen(elem, w, ldw, N, K);
    if (!xf || !wf) { free(xf); free(wf); return -1; }
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0, a = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double pd = (double)xf[m * K + k] * (double)wf[n * K + k];
                s += pd;
                a += fabs(pd);
            }
            S[m * N + n] = s;
            A[m * N + n] = a;
        }
    }
    free(xf);
    free(wf);
    return 0;
}

int oracle_band_f64(const uint16_t* x, int64_t ldx, const uint16_t* w, int64_t ldw,
                    int64_t M, int64_t N, int64_t K, double* S, double* A, int nthreads) {
    return oracle_band(0, x, ldx, w, ldw, M, N, K, S, A, nthreads);
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------------------
 * Multi-step contraction epilogue ("The Graph IR", op table: ContractionEpilogue).
 *
 * The head contraction's result keeps the head dtype (binary16 or bfloat16: the
 * projection is rounded to it first) and every epilogue step rounds through
 * that dtype.  The steps are pointwise primitives of the op table (Binary Add /
 * Mul / Div, Unary Neg / Exp / Erf) over the element type; the activations are
 * the compositions the "Tracing a Model" page describes for the feed-forward:
 *
 *   SiLU        x / (1 + exp(-x))                    over Neg, Exp, Add, Div
 *   GeLU, tanh  x / (1 + exp(-2 sqrt(2/pi) (x + 0.044715 x^3)))   the same
 *               sigmoid form over Mul, Add, Exp and Div
 *   GeLU, erf   (x (1 + erf(x / sqrt 2))) * 0.5       over Mul, Erf, Add
 *
 * Readings (the pages name the primitives, not their precision):
 *   - each primitive returns its exact result rounded to the element type
 *     (round to nearest, ties to even): the operands are widened exactly to
 *     double, the operation is carried out in double, and the double is rounded
 *     to the element type.  For +, -, *, / double has more than 2p+2 bits, so
 *     rounding through double equals one correct rounding; for exp and erf the
 *     double result is within an ulp of double, far inside the element type's
 *     grid (the pins check every element-type input against a high-precision
 *     evaluation);
 *   - constants (1, 0.5, 0.044715, -2 sqrt(2/pi), 1/sqrt 2) are element-type
 *     values: their real value rounded to the element type;
 *   - the evaluation order inside a composition is the one written above, left
 *     to right (x^3 as (x*x)*x, the constant multiplied last).
 * ------------------------------------------------------------------------- */
#define ORACLE_EPI_BIAS 1       /* t + b[n]                 */
#define ORACLE_EPI_RESIDUAL 2   /* t + r[m, n]              */
#define ORACLE_EPI_MUL 3        /* t * u[m, n]              */
#define ORACLE_EPI_SILU 4
#define ORACLE_EPI_GELU_TANH 5
#define ORACLE_EPI_GELU_ERF 6

/* Round a double to the element type, ties to even: snap to the type's grid at
   the value's binade with nearbyint (default rounding mode), then encode the
   now exactly representable value through the FP32 encoders above. */
uint16_t oracle_f64_to_elem(int elem, double v) {
    if (isnan(v)) return elem ? 0x7fc0u : 0x7e00u;
    if (isinf(v)) return (uint16_t)((v < 0 ? 0x8000u : 0u) | (elem ? 0x7f80u : 0x7c00u));
    const int p = elem ? 8 : 11;                 /* significand bits */
    const int emin = elem ? -126 : -14;          /* smallest normal exponent */
    const double maxv = elem ? ldexp(2.0 - ldexp(1.0, -7), 127) : 65504.0;
    double a = fabs(v);
    double r;
    if (a == 0.0) {
        r = 0.0;
    } else {
        int e;
        frexp(a, &e);                            /* a = f * 2^e, f in [0.5, 1) */
        e -= 1;                                  /* a in [2^e, 2^(e+1)) */
        if (e < emin) e = emin;                  /* subnormal grid */
        const double q = ldexp(1.0, e - (p - 1));
        r = nearbyint(a / q) * q;
    }
    uint16_t bits;
    if (r > maxv) bits = elem ? 0x7f80u : 0x7c00u;
    else bits = elem ? oracle_f32_to_bf16((float)r) : oracle_f32_to_f16((float)r);
    if (signbit(v)) bits |= 0x8000u;
    return bits;
}

static double wd(int elem, uint16_t h) { return (double)widen16(elem, h); }
static uint16_t rd(int elem, double v) { return oracle_f64_to_elem(elem, v); }

/* Element-type constants, rounded from their real values. */
static uint16_t cst(int elem, double v) { return rd(elem, v); }

uint16_t oracle_epi_silu(int elem, uint16_t x) {
    uint16_t n = rd(elem, -wd(elem, x));
    uint16_t e = rd(elem, exp(wd(elem, n)));
    uint16_t d = rd(elem, wd(elem, cst(elem, 1.0)) + wd(elem, e));
    return rd(elem, wd(elem, x) / wd(elem, d));
}

uint16_t oracle_epi_gelu_tanh(int elem, uint16_t x) {
    const uint16_t c1 = cst(elem, 0.044715);
    const uint16_t c2 = cst(elem, -2.0 * sqrt(2.0 / 3.14159265358979323846));
    uint16_t a = rd(elem, wd(elem, x) * wd(elem, x));
    uint16_t b = rd(elem, wd(elem, a) * wd(elem, x));
    uint16_t c = rd(elem, wd(elem, b) * wd(elem, c1));
    uint16_t d = rd(elem, wd(elem, x) + wd(elem, c));
    uint16_t z = rd(elem, wd(elem, d) * wd(elem, c2));
    uint16_t e = rd(elem, exp(wd(elem, z)));
    uint16_t f = rd(elem, wd(elem, cst(elem, 1.0)) + wd(elem, e));
    return rd(elem, wd(elem, x) / wd(elem, f));
}

uint16_t oracle_epi_gelu_erf(int elem, uint16_t x) {
    const uint16_t c3 = cst(elem, 0.70710678118654752440);
    uint16_t s = rd(elem, wd(elem, x) * wd(elem, c3));
    uint16_t f = rd(elem, erf(wd(elem, s)));
    uint16_t g = rd(elem, wd(elem, cst(elem, 1.0)) + wd(elem, f));
    uint16_t h = rd(elem, wd(elem, x) * wd(elem, g));
    return rd(elem, wd(elem, h) * wd(elem, cst(elem, 0.5)));
}

/* Unary primitives rounded to the element type (pinned one by one). */
uint16_t oracle_epi_exp(int elem, uint16_t x) { return rd(elem, exp(wd(elem, x))); }
uint16_t oracle_epi_erf(int elem, uint16_t x) { return rd(elem, erf(wd(elem, x))); }

/* One step applied to t (an element-type word). */
static uint16_t epi_step(int elem, int op, uint16_t t, uint16_t bias, uint16_t res, uint16_t mul) {
    switch (op) {
        case ORACLE_EPI_BIAS: return rd(elem, wd(elem, t) + wd(elem, bias));
        case ORACLE_EPI_RESIDUAL: return rd(elem, wd(elem, t) + wd(elem, res));
        case ORACLE_EPI_MUL: return rd(elem, wd(elem, t) * wd(elem, mul));
        case ORACLE_EPI_SILU: return oracle_epi_silu(elem, t);
        case ORACLE_EPI_GELU_TANH: return oracle_epi_gelu_tanh(elem, t);
        case ORACLE_EPI_GELU_ERF: return oracle_epi_gelu_erf(elem, t);
        default: return t;
    }
}

/*
 * The epilogue over element-type words t[i] (i < count): out[i] = the steps
 * ops[0 .. nsteps-1] applied in order to t[i], with the extra inputs of element
 * i at bias[i], res[i], mul[i] (arrays of count words; NULL when no step reads
 * them).  Callers gather the broadcast bias and the [M, N] inputs per element.
 */
void oracle_epilogue(int elem, const int32_t* ops, int nsteps, const uint16_t* t, const uint16_t* bias,
                     const uint16_t* res, const uint16_t* mul, uint16_t* out, int64_t count) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        uint16_t v = t[i];
        for (int s = 0; s < nsteps; ++s)
            v = epi_step(elem, ops[s], v, bias ? bias[i] : 0, res ? res[i] : 0, mul ? mul[i] : 0);
        out[i] = v;
    }
}

/* Element-wise unary primitive over an array (op: ORACLE_EPI_SILU .. GELU_ERF, or
   7 = exp, 8 = erf). */
void oracle_unary_array(int elem, int op, const uint16_t* x, uint16_t* out, int64_t n) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        if (op == 7) out[i] = oracle_epi_exp(elem, x[i]);
        else if (op == 8) out[i] = oracle_epi_erf(elem, x[i]);
        else out[i] = epi_step(elem, op, x[i], 0, 0, 0);
    }
}

/* ---------------------------------------------------------------------------
 * Grouped and indexed contractions ("The Graph IR", op table).
 *
 * GroupedDenseContraction: a [G*N, K] weight read as G blocks of N rows against
 * a [G, M, K] activation, giving [G, M, N]: group g contracts activation slice
 * g with weight rows g*N .. g*N+N-1, each block read in place.
 *
 * IndexedMatMul: x [M, K], W [E, K, N], idx [M] -> [M, N]: row m contracts
 * against expert idx[m], y[m, n] = sum_k x[m, k] * W[idx[m], k, n]; the expert
 * tables are read in place (note the [K, N] order of each expert: the weight
 * is indexed by k first).
 *
 * Readings: operands are element-type words (binary16 or bfloat16) as for the
 * layer; accumulation is FP32 in sequential k from +0; the result is rounded to
 * the element type, or returned as the FP32 sums; a grouped call may add a
 * [G*N] bias as the layer does.  A row whose idx lies outside [0, E) has no
 * expert: the oracle leaves its outputs untouched (the kernels do the same).
 * ------------------------------------------------------------------------- */

/* x: [G, M, K] with row stride ldx and group stride sx; w: [G*N, K] row stride
   ldw; b: [G*N] or NULL; y/proj: [G, M, N] row stride ldy, group stride sy;
   y32: FP32 sums, same layout (each may be NULL). */
int oracle_grouped(int elem, const uint16_t* x, int64_t ldx, int64_t sx, const uint16_t* w, int64_t ldw,
                   const uint16_t* b, uint16_t* y, uint16_t* proj, float* y32, int64_t ldy, int64_t sy,
                   int64_t G, int64_t M, int64_t N, int64_t K, int nthreads) {
    for (int64_t g = 0; g < G; ++g) {
        int rc = oracle_linear(elem, x + g * sx, ldx, w + g * N * ldw, ldw, b ? b + g * N : NULL,
                               y ? y + g * sy : NULL, proj ? proj + g * sy : NULL, y32 ? y32 + g * sy : NULL,
                               ldy, M, N, K, nthreads);
        if (rc != 0) return rc;
    }
    return 0;
}

/* x: [M, K] row stride ldx; w: [E, K, N] with row stride ldw (>= N, between k
   rows) and expert stride sw (>= K*ldw); idx: [M]; y: [M, N] row stride ldy
   (rounded), y32: FP32 sums (each may be NULL). */
void oracle_indexed(int elem, const uint16_t* x, int64_t ldx, const uint16_t* w, int64_t ldw, int64_t sw,
                    const int32_t* idx, uint16_t* y, float* y32, int64_t ldy, int64_t E, int64_t M, int64_t N,
                    int64_t K, int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m) {
        const int64_t e = idx[m];
        if (e < 0 || e >= E) continue;
        const uint16_t* we = w + e * sw;
        for (int64_t n = 0; n < N; ++n) {
            float acc = 0.0f;
            for (int64_t k = 0; k < K; ++k) acc = acc + widen16(elem, x[m * ldx + k]) * widen16(elem, we[k * ldw + n]);
            if (y32) y32[m * ldy + n] = acc;
            if (y) y[m * ldy + n] = narrow16(elem, acc);
        }
    }
}

/* FP64 band data S = sum x*w and A = sum |x*w| of the indexed contraction
   (rows without an expert get 0). */
void oracle_indexed_band(int elem, const uint16_t* x, int64_t ldx, const uint16_t* w, int64_t ldw, int64_t sw,
                         const int32_t* idx, double* S, double* A, int64_t E, int64_t M, int64_t N, int64_t K) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m) {
        const int64_t e = idx[m];
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0, a = 0.0;
            if (e >= 0 && e < E) {
                const uint16_t* we = w + e * sw;
                for (int64_t k = 0; k < K; ++k) {
                    const double pd = (double)widen16(elem, x[m * ldx + k]) * (double)widen16(elem, we[k * ldw + n]);
                    s += pd;
                    a += fabs(pd);
                }
            }
            S[m * N + n] = s;
            A[m * N + n] = a;
        }
    }
}
