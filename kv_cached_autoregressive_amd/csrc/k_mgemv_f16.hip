// MFMA skinny GEMM kernels for f16 weights (all variants but the prologue ones).
#include "k_mgemv_impl.h"

namespace wd {
hipError_t mrun_f16(const MGemvParams& p, hipStream_t st) { return mrun<f16_t>(p, st); }
}  // namespace wd
