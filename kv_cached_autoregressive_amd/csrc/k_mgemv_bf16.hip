// MFMA skinny GEMM kernels for bf16 weights (all variants but the prologue ones).
#include "k_mgemv_impl.h"

namespace wd {
hipError_t mrun_bf16(const MGemvParams& p, hipStream_t st) { return mrun<bf16_t>(p, st); }
}  // namespace wd
