// gemm_bf16.hip -- the GEMM kernels instantiated for bfloat16 operands.
#include "gemm_impl.h"

namespace lin {
template hipError_t launch_gemm_t<kBF16>(int, const LinearArgs&, int, hipStream_t);
template hipError_t launch_gemm_stream_t<kBF16>(int, const LinearArgs&, int, hipStream_t);
}  // namespace lin
