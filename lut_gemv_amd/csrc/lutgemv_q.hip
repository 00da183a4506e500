// One translation unit per plane count: compiled with -DLUTGEMM_Q=q (1..8), it
// instantiates every kernel of that q (see lutgemv_kernel.h and
// sign_mfma_kernel.h).
#include "lutgemv_kernel.h"
#include "sign_mfma_kernel.h"

#ifndef LUTGEMM_Q
#error "compile with -DLUTGEMM_Q=<plane count 1..8>"
#endif

namespace lutgemm {
template KernelFn kernels_of_q<LUTGEMM_Q>(int, int, bool, bool, int, int, bool, int, bool, bool);
template KernelFn nibble_kernel_of_q<LUTGEMM_Q>(bool, int, int);
template KernelFn sign_mfma_kernel_of_q<LUTGEMM_Q>(int, bool, int, bool, bool);
}  // namespace lutgemm
