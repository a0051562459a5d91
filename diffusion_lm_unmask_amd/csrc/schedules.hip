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
// k_rank_select: one workgroup (256 threads) per sequence.  The eligible
// non-NaN rows are keyed (confidence descending, row ascending), gathered
// into LDS (slot order is irrelevant: the sort decides) and sorted: up to 64
// keys by one wave in registers (bitonic network, no barriers); more as runs
// of 64 sorted in registers, each key placed at its rank (its lane plus
// binary searches in the other runs).  Position t of the sorted keys is the row of rank
// t.  Top-K takes positions < K; factor decoding tests (t+2)(1 - c) < f at
// every position and takes the largest admissible one (a max reduction, so
// it equals "the largest n" for any input, monotone or not).  The test runs
// in fp64 on the fp32 confidences, where it is exact.
#include <math.h>

#include "dlm_device.h"

namespace {

constexpr int kRankNT = 256;
constexpr int kRankMax = DLM_MAX_SEQ_ROWS;  // rows per sequence
constexpr int kBlockNT = 256;

enum Mode { kTopK = 0, kFactor = 1 };

template <int MODE>
__global__ __launch_bounds__(kRankNT) void k_rank_select(
    const float* __restrict__ conf, const uint8_t* __restrict__ eligible,
    const int32_t* __restrict__ seq_offsets, int k, float f, uint8_t* __restrict__ commit,
    int32_t* __restrict__ n_commit, uint8_t* __restrict__ certificate) {
  __shared__ uint64_t keys[kRankMax];  // candidates' (desc conf, row), then sorted runs
  __shared__ uint64_t sorted[kRankMax];  // keys in order (more than 64 keys)
  __shared__ float cs[kRankMax];       // confidence by row
  __shared__ uint8_t take[kRankMax];   // selected, by row
  __shared__ int shi[kRankNT / DLM_WAVE];
  __shared__ int cnt;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int lo = seq_offsets[b], M = seq_offsets[b + 1] - lo;
  if (M > kRankMax || M < 0) {  // over-long sequence: nothing committed, reported as -1
    for (int r = tid; r < M; r += kRankNT) commit[lo + r] = 0;
    if (tid == 0) {
      n_commit[b] = -1;
      if (MODE == kFactor && certificate) certificate[b] = 0;
    }
    return;
  }
  if (tid == 0) cnt = 0;
  __syncthreads();
  for (int r = tid; r < M; r += kRankNT) {
    float c = NAN;
    if (!eligible || eligible[lo + r]) c = conf[lo + r];
    cs[r] = c;
    take[r] = 0;
    if (c == c) {
      const int slot = atomicAdd(&cnt, 1);
      keys[slot] = (static_cast<uint64_t>(dlm::desc_bits(c)) << 32) | static_cast<uint32_t>(r);
    }
  }
  __syncthreads();
  const int n_ok = cnt;
  int n2 = 1;
  while (n2 < n_ok) n2 <<= 1;
  const uint64_t* order = keys;  // position t holds the key of rank t
  if (n2 <= DLM_WAVE) {
    if (tid < DLM_WAVE) {  // one wave, in registers: lane l holds key l
      const uint64_t v = dlm::wave_sort_asc(tid < n_ok ? keys[tid] : ~0ull, n2);
      if (tid < n_ok) keys[tid] = v;
    }
    __syncthreads();
  } else {  // runs of 64 sorted in registers, placed by rank
    dlm::sort_runs<kRankNT>(keys, sorted, n_ok, n_ok);
    order = sorted;
  }
  int n;
  if constexpr (MODE == kTopK) {
    n = min(k, n_ok);
  } else {
    int adm = 0;  // largest admissible position + 1 among this thread's positions
    for (int t = tid; t < n_ok; t += kRankNT) {
      const float ct = cs[order[t] & 0xffffffffu];
      if (static_cast<double>(t + 2) * (1.0 - static_cast<double>(ct)) < static_cast<double>(f))
        adm = t + 1;
    }
    n = dlm::block_max_i<kRankNT>(adm, shi);
    if (n == 0 && n_ok > 0) n = 1;  // progress: the most confident row
    if (certificate) {
      if (n == 0) {
        if (tid == 0) certificate[b] = 0;
      } else if ((n - 1) % kRankNT == tid) {
        const float ct = cs[order[n - 1] & 0xffffffffu];
        certificate[b] = static_cast<uint8_t>(static_cast<double>(n + 1) *
                                                  (1.0 - static_cast<double>(ct)) <=
                                              1.0);
      }
    }
  }
  for (int t = tid; t < n; t += kRankNT) take[order[t] & 0xffffffffu] = 1;
  __syncthreads();
  for (int r = tid; r < M; r += kRankNT) commit[lo + r] = take[r];
  if (tid == 0) n_commit[b] = n;
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
