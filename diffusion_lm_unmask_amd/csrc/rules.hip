// rules.hip — dlm_fastdllm_select and dlm_depcap_boundary: one workgroup per
// sequence (the device code is in rules_impl.h), host validation, and the
// status strings.
#include "checks.h"
#include "rules_impl.h"

namespace {

__global__ __launch_bounds__(kRuleNT) void k_fastdllm(const float* __restrict__ conf,
                                                  const uint8_t* __restrict__ eligible,
                                                  const int32_t* __restrict__ seq_offsets,
                                                  float tau, uint8_t* __restrict__ commit,
                                                  int32_t* __restrict__ n_commit) {
  fastdllm_seq(blockIdx.x, conf, eligible, seq_offsets, tau, commit, n_commit);
}

__global__ __launch_bounds__(kRuleNT) void k_depcap(const float* __restrict__ kl,
                                                const float* __restrict__ ent,
                                                const int32_t* __restrict__ seq_offsets,
                                                const uint8_t* __restrict__ has_prev,
                                                double lambda, int l_min, int l_max, int R,
                                                double eps, int32_t* __restrict__ block_len,
                                                double* __restrict__ score) {
  __shared__ DepSmem sm;
  depcap_seq(blockIdx.x, kl, ent, seq_offsets, has_prev, lambda, l_min, l_max, R, eps, block_len,
             score, sm);
}

}  // namespace

extern "C" int dlm_fastdllm_select(const float* conf, const uint8_t* eligible,
                                   const int32_t* seq_offsets, int32_t n_seq, float tau,
                                   uint8_t* commit, int32_t* n_commit, void* stream) {
  const int rc = dlmh::check_fastdllm(conf, seq_offsets, n_seq, tau, commit, n_commit);
  if (rc != DLM_OK) return rc;
  hipLaunchKernelGGL(k_fastdllm, dim3(n_seq), dim3(kRuleNT), 0, static_cast<hipStream_t>(stream),
                     conf, eligible, seq_offsets, tau, commit, n_commit);
  DLM_CHECK_LAUNCH();
  return DLM_OK;
}

extern "C" int dlm_depcap_boundary(const float* kl, const float* entropy,
                                   const int32_t* seq_offsets, int32_t n_seq,
                                   const uint8_t* has_prev, double lambda, int32_t l_min,
                                   int32_t l_max, int32_t smooth_radius, double eps,
                                   int32_t* block_len, double* score, void* stream) {
  const int rc = dlmh::check_depcap(kl, entropy, seq_offsets, n_seq, lambda, l_min, l_max,
                                    smooth_radius, eps, block_len);
  if (rc != DLM_OK) return rc;
  hipLaunchKernelGGL(k_depcap, dim3(n_seq), dim3(kRuleNT), 0, static_cast<hipStream_t>(stream), kl,
                     entropy, seq_offsets, has_prev, lambda, l_min, l_max, smooth_radius, eps,
                     block_len, score);
  DLM_CHECK_LAUNCH();
  return DLM_OK;
}

extern "C" const char* dlm_status_string(int status) {
  switch (status) {
    case DLM_OK:
      return "ok";
    case DLM_ERR_ARG:
      return "invalid argument";
    case DLM_ERR_UNSUPPORTED:
      return "unsupported dtype or size above a documented limit";
    case DLM_ERR_HIP:
      return "HIP kernel launch failed";
    default:
      return "unknown status";
  }
}
