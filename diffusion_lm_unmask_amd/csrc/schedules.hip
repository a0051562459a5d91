// schedules.hip — fixed top-K, factor decoding and fixed-block eligibility:
// the baseline and adaptive commit schedules that sit beside the threshold
// rule.
//
//  * top-K: LLaDA's default schedule commits the K most confident masked
//    tokens per step (Fast-dLLM review, Prior limitations; Comparison).
//  * factor decoding: the largest n with (n+1)(1 - c(n)) < f over the
//    confidences in descending order (Fast-dLLM review, Method), with
//    Theorem 1's certificate (n+1)(1 - min committed c) <= 1 (Key idea).
//  * fixed-block eligibility: confidence decoding in fixed 16/32/64-token
//    blocks (DepCap summary, Experiments): the masked rows of the earliest
//    block that still holds a mask.
//
// k_rank_select: one workgroup (1024 threads) per sequence, one row per
// thread.  A row's rank in (conf desc, row asc) order among the eligible
// non-NaN rows is counted against the sequence's confidences held in LDS
// (broadcast reads, four per ds_read_b128).  Both rules then follow from the
// ranks; factor decoding takes the largest admissible rank (a max
// reduction), so it equals "the largest n" for any input, monotone or not.
// The factor test runs in fp64 on the fp32 confidences, where it is exact.
#include <math.h>

#include "dlm_device.h"

namespace {

constexpr int kRankNT = DLM_MAX_SEQ_ROWS;  // one thread per row
constexpr int kBlockNT = 256;

enum Mode { kTopK = 0, kFactor = 1 };

template <int MODE>
__global__ __launch_bounds__(kRankNT) void k_rank_select(
    const float* __restrict__ conf, const uint8_t* __restrict__ eligible,
    const int32_t* __restrict__ seq_offsets, int k, float f, uint8_t* __restrict__ commit,
    int32_t* __restrict__ n_commit, uint8_t* __restrict__ certificate) {
  __shared__ __align__(16) float cs[kRankNT];  // confidence, NaN when not a candidate
  __shared__ int shi[kRankNT / DLM_WAVE];
  const int b = blockIdx.x, i = threadIdx.x;
  const int lo = seq_offsets[b], M = seq_offsets[b + 1] - lo;
  if (M > kRankNT || M < 0) {  // over-long sequence: nothing committed, reported as -1
    for (int r = i; r < M; r += kRankNT) commit[lo + r] = 0;
    if (i == 0) {
      n_commit[b] = -1;
      if (MODE == kFactor && certificate) certificate[b] = 0;
    }
    return;
  }
  float c = NAN;
  if (i < M && (!eligible || eligible[lo + i])) c = conf[lo + i];
  const bool ok = c == c;
  cs[i] = c;  // rows >= M hold NaN
  __syncthreads();

  // rank = candidates before this row: higher confidence, or equal and lower row
  int rank = 0;
  if (ok) {
    const float4* c4 = reinterpret_cast<const float4*>(cs);
    const int n4 = (M + 3) / 4;
    for (int q = 0; q < n4; ++q) {
      const float4 v = c4[q];
      const int j = 4 * q;
      rank += (v.x > c) | ((v.x == c) & (j + 0 < i));
      rank += (v.y > c) | ((v.y == c) & (j + 1 < i));
      rank += (v.z > c) | ((v.z == c) & (j + 2 < i));
      rank += (v.w > c) | ((v.w == c) & (j + 3 < i));
    }
  }
  const int n_ok = dlm::block_sum<kRankNT>(ok ? 1 : 0, shi);
  int n;
  if constexpr (MODE == kTopK) {
    n = min(k, n_ok);
  } else {
    const bool adm =
        ok && static_cast<double>(rank + 2) * (1.0 - static_cast<double>(c)) <
                  static_cast<double>(f);
    n = dlm::block_max_i<kRankNT>(adm ? rank + 1 : 0, shi);
    if (n == 0 && n_ok > 0) n = 1;  // progress: the most confident row
    if (certificate) {
      if (n == 0) {
        if (i == 0) certificate[b] = 0;
      } else if (ok && rank == n - 1) {
        certificate[b] = static_cast<uint8_t>(static_cast<double>(n + 1) *
                                                  (1.0 - static_cast<double>(c)) <=
                                              1.0);
      }
    }
  }
  if (i < M) commit[lo + i] = static_cast<uint8_t>(ok && rank < n);
  if (i == 0) n_commit[b] = n;
}

__global__ __launch_bounds__(kBlockNT) void k_fixed_block(const int32_t* __restrict__ masked_pos,
                                                          const int32_t* __restrict__ seq_offsets,
                                                          const int32_t* __restrict__ gen_start,
                                                          int block_len,
                                                          uint8_t* __restrict__ eligible) {
  __shared__ int shi[kBlockNT / DLM_WAVE];
  const int b = blockIdx.x;
  const int lo = seq_offsets[b], hi = seq_offsets[b + 1];
  const int64_t g0 = gen_start ? gen_start[b] : 0;
  int first = INT32_MAX;
  for (int r = lo + threadIdx.x; r < hi; r += kBlockNT) {
    const int64_t rel = static_cast<int64_t>(masked_pos[r]) - g0;
    if (rel >= 0) first = min(first, static_cast<int>(rel / block_len));
  }
  first = dlm::block_min_i<kBlockNT>(first, shi);
  for (int r = lo + threadIdx.x; r < hi; r += kBlockNT) {
    const int64_t rel = static_cast<int64_t>(masked_pos[r]) - g0;
    eligible[r] = static_cast<uint8_t>(rel >= 0 && first != INT32_MAX && rel / block_len == first);
  }
}

}  // namespace

extern "C" int dlm_topk_select(const float* conf, const uint8_t* eligible,
                               const int32_t* seq_offsets, int32_t n_seq, int32_t k,
                               uint8_t* commit, int32_t* n_commit, void* stream) {
  if (!conf || !seq_offsets || !commit || !n_commit || n_seq <= 0 || k < 1) return DLM_ERR_ARG;
  hipLaunchKernelGGL(k_rank_select<kTopK>, dim3(n_seq), dim3(kRankNT), 0,
                     static_cast<hipStream_t>(stream), conf, eligible, seq_offsets, k, 0.f,
                     commit, n_commit, nullptr);
  DLM_CHECK_LAUNCH();
  return DLM_OK;
}

extern "C" int dlm_factor_select(const float* conf, const uint8_t* eligible,
                                 const int32_t* seq_offsets, int32_t n_seq, float f,
                                 uint8_t* commit, int32_t* n_commit, uint8_t* certificate,
                                 void* stream) {
  if (!conf || !seq_offsets || !commit || !n_commit || n_seq <= 0 || f != f) return DLM_ERR_ARG;
  hipLaunchKernelGGL(k_rank_select<kFactor>, dim3(n_seq), dim3(kRankNT), 0,
                     static_cast<hipStream_t>(stream), conf, eligible, seq_offsets, 0, f, commit,
                     n_commit, certificate);
  DLM_CHECK_LAUNCH();
  return DLM_OK;
}

extern "C" int dlm_fixed_block_eligible(const int32_t* masked_pos, const int32_t* seq_offsets,
                                        int32_t n_seq, const int32_t* gen_start,
                                        int32_t block_len, uint8_t* eligible, void* stream) {
  if (!masked_pos || !seq_offsets || !eligible || n_seq <= 0 || block_len < 1)
    return DLM_ERR_ARG;
  hipLaunchKernelGGL(k_fixed_block, dim3(n_seq), dim3(kBlockNT), 0,
                     static_cast<hipStream_t>(stream), masked_pos, seq_offsets, gen_start,
                     block_len, eligible);
  DLM_CHECK_LAUNCH();
  return DLM_OK;
}
