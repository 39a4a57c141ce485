// epilogue.hip -- the activation tables of the multi-step contraction epilogue.
//
// The epilogue ("The Graph IR", op table: ContractionEpilogue) rounds every step
// through the element type, and the activations are compositions of pointwise
// primitives ("Tracing a Model", the gated feed-forward: SiLU as
// x / (1 + exp(-x)) over Neg, Exp, Add, Div; the tanh GeLU in the same sigmoid
// form over Mul, Add, Exp, Div; the erf GeLU on Erf).  Each primitive's result
// is the exact operation rounded once to the element type (round to nearest,
// ties to even), constants are element-type values, and a composition
// evaluates left to right.
//
// An activation is then a function of one 16-bit word, so the library evaluates
// it once for all 65536 words per element type and the GEMM and skinny
// epilogues look the result up: one load per element instead of dozens of
// instructions after the MFMA loop.  The tables are built here on the device:
// exp and erf in double precision (far finer than either element type's grid),
// every intermediate rounded by round_to<E>, an integer rounding of the double's
// bits.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "kernels.h"

namespace lin {

// Tables per element type (binary16, bfloat16): SiLU, tanh GeLU, erf GeLU.
static __device__ uint16_t g_act_tables[2][3][kActWords];

// Round a double to element type E, ties to even, from its bits: keep the top
// P significant bits (fewer below the normal range), round on the rest, carry,
// and encode.  Overflow gives infinity, NaN a quiet NaN.
template <int E>
__device__ uint16_t round_to(double v) {
    constexpr int P = E == kF16 ? 11 : 8;           // significant bits
    constexpr int EMIN = E == kF16 ? -14 : -126;    // smallest normal exponent
    constexpr int EMAX = E == kF16 ? 15 : 127;
    constexpr int BIAS = E == kF16 ? 15 : 127;
    constexpr uint16_t INF = E == kF16 ? 0x7c00 : 0x7f80;
    constexpr uint16_t QNAN = E == kF16 ? 0x7e00 : 0x7fc0;
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
    const int bexp = (int)((u >> 52) & 0x7ff);
    const uint64_t frac = u & ((uint64_t(1) << 52) - 1);
    if (bexp == 0x7ff) return frac ? QNAN : (uint16_t)(sign | INF);
    if (bexp == 0) return sign;                     // zero, or a double subnormal: far below the type
    const int e = bexp - 1023;
    const uint64_t sig = frac | (uint64_t(1) << 52);
    const int drop = (53 - P) + (e < EMIN ? EMIN - e : 0);   // low bits that do not fit
    if (drop >= 54) return sign;                    // below half the smallest subnormal
    uint64_t k = sig >> drop;
    const uint64_t low = sig & ((uint64_t(1) << drop) - 1);
    const uint64_t half = uint64_t(1) << (drop - 1);
    if (low > half || (low == half && (k & 1))) ++k;
    int qe = (e < EMIN ? EMIN : e) - (P - 1);       // value = k * 2^qe
    if (k == (uint64_t(1) << P)) {                  // rounding carried into the next binade
        k >>= 1;
        ++qe;
    }
    if (k < (uint64_t(1) << (P - 1))) return (uint16_t)(sign | k);   // subnormal
    const int ue = qe + P - 1;
    if (ue > EMAX) return (uint16_t)(sign | INF);
    return (uint16_t)(sign | ((uint32_t)(ue + BIAS) << (P - 1)) | (uint32_t)(k - (uint64_t(1) << (P - 1))));
}

template <int E>
__device__ inline double wide(uint16_t w) { return (double)widen<E>(w); }

// y = x / (1 + exp(-x)), each primitive rounded to E
template <int E>
__device__ uint16_t silu_word(uint16_t x) {
    const double one = wide<E>(round_to<E>(1.0));
    const uint16_t nx = round_to<E>(-wide<E>(x));
    const uint16_t ex = round_to<E>(exp(wide<E>(nx)));
    const uint16_t den = round_to<E>(one + wide<E>(ex));
    return round_to<E>(wide<E>(x) / wide<E>(den));
}

// y = x / (1 + exp(c2 * (x + c1 * (x * x) * x))), c1 = 0.044715, c2 = -2 sqrt(2/pi)
template <int E>
__device__ uint16_t gelu_tanh_word(uint16_t x) {
    const double one = wide<E>(round_to<E>(1.0));
    const double c1 = wide<E>(round_to<E>(0.044715));
    const double c2 = wide<E>(round_to<E>(-1.5957691216057307117597842397375));
    const double xv = wide<E>(x);
    const uint16_t sq = round_to<E>(xv * xv);
    const uint16_t cube = round_to<E>(wide<E>(sq) * xv);
    const uint16_t term = round_to<E>(wide<E>(cube) * c1);
    const uint16_t inner = round_to<E>(xv + wide<E>(term));
    const uint16_t z = round_to<E>(wide<E>(inner) * c2);
    const uint16_t ez = round_to<E>(exp(wide<E>(z)));
    const uint16_t den = round_to<E>(one + wide<E>(ez));
    return round_to<E>(xv / wide<E>(den));
}

// y = (x * (1 + erf(x * c3))) * 0.5, c3 = 1 / sqrt 2
template <int E>
__device__ uint16_t gelu_erf_word(uint16_t x) {
    const double one = wide<E>(round_to<E>(1.0));
    const double c3 = wide<E>(round_to<E>(0.70710678118654752440084436210485));
    const double xv = wide<E>(x);
    const uint16_t s = round_to<E>(xv * c3);
    const uint16_t ef = round_to<E>(erf(wide<E>(s)));
    const uint16_t g = round_to<E>(one + wide<E>(ef));
    const uint16_t h = round_to<E>(xv * wide<E>(g));
    return round_to<E>(wide<E>(h) * 0.5);
}

template <int E>
__global__ void __launch_bounds__(256) build_act_tables(uint16_t* t) {
    const int w = blockIdx.x * 256 + threadIdx.x;
    if (w >= kActWords) return;
    t[w] = silu_word<E>((uint16_t)w);
    t[kActWords + w] = gelu_tanh_word<E>((uint16_t)w);
    t[2 * kActWords + w] = gelu_erf_word<E>((uint16_t)w);
}

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
std::atomic<uint16_t*> g_base[kMaxDevices][2];   // per device and element type, once built

}  // namespace

hipError_t act_tables(int elem, int device, hipStream_t stream, const uint16_t** tables) {
    if (device < 0 || device >= kMaxDevices || (elem != kF16 && elem != kBF16)) return hipErrorInvalidValue;
    uint16_t* base = g_base[device][elem].load(std::memory_order_acquire);
    if (base) {
        *tables = base;
        return hipSuccess;
    }
    std::lock_guard<std::mutex> lock(g_mu);
    base = g_base[device][elem].load(std::memory_order_relaxed);
    if (!base) {
        // the first call on this device builds the tables and waits for them, so
        // it cannot be made under stream capture
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        hipError_t e = hipStreamIsCapturing(stream, &cap);
        if (e != hipSuccess) return e;
        if (cap != hipStreamCaptureStatusNone) return hipErrorStreamCaptureUnsupported;
        void* sym = nullptr;
        e = hipGetSymbolAddress(&sym, HIP_SYMBOL(g_act_tables));
        if (e != hipSuccess) return e;
        uint16_t* t = (uint16_t*)sym + (size_t)elem * 3 * kActWords;
        if (elem == kBF16) hipLaunchKernelGGL(build_act_tables<kBF16>, dim3(kActWords / 256), dim3(256), 0, stream, t);
        else hipLaunchKernelGGL(build_act_tables<kF16>, dim3(kActWords / 256), dim3(256), 0, stream, t);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        e = hipStreamSynchronize(stream);
        if (e != hipSuccess) return e;
        base = t;
        g_base[device][elem].store(base, std::memory_order_release);
    }
    *tables = base;
    return hipSuccess;
}

}  // namespace lin
