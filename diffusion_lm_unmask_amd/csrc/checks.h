// checks.h — host-side argument checks shared by the individual entry points
// and dlm_decide_step, so that both reject exactly the same calls.  Each
// returns DLM_OK or the error code the entry point documents.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "../../include/dlm.h"

namespace dlmh {

// row_index may be NULL (row r itself); its values are not read on the host.
inline int check_stats(const void* logits, const void* prev, int dtype, int64_t vocab,
                       int64_t ld, [[maybe_unused]] const int64_t* row_index, int64_t n_rows,
                       const void* conf,
                       const void* argmax, const void* entropy, const void* kl, const void* lse) {
  if (!logits || !conf || !argmax || !entropy || !lse) return DLM_ERR_ARG;
  if ((prev == nullptr) != (kl == nullptr)) return DLM_ERR_ARG;
  if (dtype != DLM_BF16 && dtype != DLM_F32) return DLM_ERR_UNSUPPORTED;
  if (vocab <= 0 || n_rows <= 0 || ld < vocab) return DLM_ERR_ARG;
  if (vocab > DLM_MAX_VOCAB || n_rows > 2147483647LL) return DLM_ERR_UNSUPPORTED;
  const int es = dtype == DLM_BF16 ? 2 : 4;
  if (reinterpret_cast<uintptr_t>(logits) % es || reinterpret_cast<uintptr_t>(prev) % es)
    return DLM_ERR_ARG;
  return DLM_OK;
}

inline int check_fastdllm(const void* conf, const void* seq_offsets, int32_t n_seq, float tau,
                          const void* commit, const void* n_commit) {
  if (!conf || !seq_offsets || !commit || !n_commit || n_seq <= 0 || tau != tau)
    return DLM_ERR_ARG;
  return DLM_OK;
}

inline int check_depcap(const void* kl, const void* entropy, const void* seq_offsets,
                        int32_t n_seq, double lambda, int32_t l_min, int32_t l_max,
                        int32_t radius, double eps, const void* block_len) {
  if (!kl || !entropy || !seq_offsets || !block_len || n_seq <= 0) return DLM_ERR_ARG;
  if (lambda != lambda || eps != eps || eps < 0.0 || radius < 0 || l_min < 0 || l_max <= 0 ||
      l_min > l_max)
    return DLM_ERR_ARG;
  if (l_max > DLM_MAX_WINDOW) return DLM_ERR_UNSUPPORTED;
  return DLM_OK;
}

inline int check_cap(const void* logits, int dtype, int64_t vocab, int64_t ld,
                     [[maybe_unused]] const void* row_index, const void* seq_offsets,
                     int32_t n_seq,
                     const void* conf, const void* argmax, const void* lse, float tau_low,
                     float tau_high, float gamma, int32_t k_max, const void* commit,
                     const void* n_commit) {
  if (!logits || !seq_offsets || !conf || !argmax || !lse || !commit || !n_commit)
    return DLM_ERR_ARG;
  if (n_seq <= 0 || vocab <= 0 || ld < vocab || k_max <= 0) return DLM_ERR_ARG;
  if (tau_low != tau_low || tau_high != tau_high || gamma != gamma) return DLM_ERR_ARG;
  if (dtype != DLM_BF16 && dtype != DLM_F32) return DLM_ERR_UNSUPPORTED;
  if (k_max > DLM_MAX_KMAX || vocab > DLM_MAX_VOCAB) return DLM_ERR_UNSUPPORTED;
  const int es = dtype == DLM_BF16 ? 2 : 4;
  if (reinterpret_cast<uintptr_t>(logits) % es) return DLM_ERR_ARG;
  return DLM_OK;
}

inline int check_dapd(const void* attn, int dtype, int32_t n_lh, int64_t S, int64_t batch_stride,
                      const void* masked_pos, const void* seq_offsets, int32_t n_seq,
                      int32_t m_max, const void* conf, float tau, float late_frac,
                      float late_tau, const void* commit, const void* n_commit,
                      const void* workspace, size_t workspace_bytes) {
  if (!attn || !masked_pos || !seq_offsets || !conf || !commit || !n_commit || !workspace)
    return DLM_ERR_ARG;
  if (n_lh <= 0 || S <= 0 || n_seq <= 0 || m_max <= 0 || tau != tau) return DLM_ERR_ARG;
  if (late_frac != late_frac || late_tau != late_tau) return DLM_ERR_ARG;
  if (dtype != DLM_BF16 && dtype != DLM_F32) return DLM_ERR_UNSUPPORTED;
  if (m_max > DLM_MAX_SEQ_ROWS || S > 2147483647LL) return DLM_ERR_UNSUPPORTED;
  if (S > INT64_MAX / S / n_lh) return DLM_ERR_UNSUPPORTED;  // n_lh * S * S elements overflow
  const int64_t maps = static_cast<int64_t>(n_lh) * S * S;
  if (n_seq > 1 && batch_stride < maps) return DLM_ERR_ARG;
  const int es = dtype == DLM_BF16 ? 2 : 4;
  if (reinterpret_cast<uintptr_t>(attn) % es) return DLM_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(workspace) % 16) return DLM_ERR_ARG;
  if (workspace_bytes < dlm_dapd_workspace_bytes(n_seq, m_max)) return DLM_ERR_ARG;
  return DLM_OK;
}

}  // namespace dlmh
