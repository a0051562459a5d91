// cap.hip — dlm_cap_select: one workgroup per sequence (the device code is in
// cap_impl.h) and host validation.
#include "checks.h"
#include "cap_impl.h"

namespace {

template <bool BF16>
__global__ __launch_bounds__(kCapNT) void k_cap(
    const void* __restrict__ logits, int64_t ld, int64_t vocab,
    const int64_t* __restrict__ row_index,
    const int32_t* __restrict__ seq_offsets, const float* __restrict__ conf,
    const int32_t* __restrict__ argmax, const float* __restrict__ lse,
    const uint8_t* __restrict__ eligible, float tau_low, float tau_high, float gamma, int k_max,
    uint8_t* __restrict__ commit, int32_t* __restrict__ n_commit, int32_t* __restrict__ cand_out,
    float* __restrict__ dmat_out) {
  __shared__ CapSmem sm;
  cap_seq<BF16>(blockIdx.x, logits, ld, vocab, row_index, seq_offsets, conf, argmax, lse,
                eligible, tau_low, tau_high, gamma, k_max, commit, n_commit, cand_out, dmat_out,
                sm);
}

}  // namespace

extern "C" int dlm_cap_select(const void* logits, int dtype, int64_t vocab, int64_t ld,
                              const int64_t* row_index, const int32_t* seq_offsets,
                              int32_t n_seq, const float* conf, const int32_t* argmax,
                              const float* lse, const uint8_t* eligible, float tau_low,
                              float tau_high, float gamma, int32_t k_max, uint8_t* commit,
                              int32_t* n_commit, int32_t* cand, float* dmat, void* stream) {
  const int rc = dlmh::check_cap(logits, dtype, vocab, ld, row_index, seq_offsets, n_seq, conf,
                                 argmax, lse, tau_low, tau_high, gamma, k_max, commit, n_commit);
  if (rc != DLM_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == DLM_BF16)
    hipLaunchKernelGGL(k_cap<true>, dim3(n_seq), dim3(kCapNT), 0, s, logits, ld, vocab, row_index,
                       seq_offsets, conf, argmax, lse, eligible, tau_low, tau_high, gamma,
                       k_max, commit, n_commit, cand, dmat);
  else
    hipLaunchKernelGGL(k_cap<false>, dim3(n_seq), dim3(kCapNT), 0, s, logits, ld, vocab, row_index,
                       seq_offsets, conf, argmax, lse, eligible, tau_low, tau_high, gamma,
                       k_max, commit, n_commit, cand, dmat);
  DLM_CHECK_LAUNCH();
  return DLM_OK;
}
