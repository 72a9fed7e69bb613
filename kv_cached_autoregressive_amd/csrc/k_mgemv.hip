// Public launchers of the MFMA skinny GEMM (kernels and shape policy in k_mgemv_impl.h).
#define WD_MG_MAIN
#include "k_mgemv_impl.h"
