// prefill_prep_raw.hip -- the chunk prep kernel of the bf16 MFMA prefill for
// raw gate projections: log g = -exp(A_log) softplus(a + dt_bias) and
// beta = sigmoid(b) are formed where the kernel fetches the gates ("Qwen3.5
// Gated Delta Net NKI Kernel for AWS Neuron", section "Correctness Contract",
// for the decay law).  Same body as chunk_prep_kernel (prefill_prep.inc); a
// translation unit of its own so that each prep kernel is register-allocated
// on its own.
#include "prefill_mfma_common.h"

namespace gdn {
namespace mfma_prefill {

#define PREP_KERNEL chunk_prep_raw_kernel
#define PREP_RAW true
#include "prefill_prep.inc"
#undef PREP_KERNEL
#undef PREP_RAW

hipError_t launch_prep_raw(const PrefillArgs& a, int NRc, unsigned char* ws, int c_first,
                          int n_chunks, hipStream_t stream) {
    const int blocks = a.B * a.Hk * n_chunks;
    hipLaunchKernelGGL(chunk_prep_raw_kernel, dim3(blocks), dim3(NT), 0, stream,
                       static_cast<const bf16_t*>(a.q), static_cast<const bf16_t*>(a.k), a.log_g,
                       a.beta, a.A_log, a.dt_bias, ws, a.T, NRc, a.Hk, a.Hv, a.l2norm, a.cu,
                       a.total, c_first, n_chunks);
    return hipGetLastError();
}

}  // namespace mfma_prefill
}  // namespace gdn
