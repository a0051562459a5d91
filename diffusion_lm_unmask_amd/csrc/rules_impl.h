// rules_impl.h — device code of the two per-sequence scans that need only
// per-row statistics:
//   dlm_fastdllm_select  (Fast-dLLM review, Method; Fast-dLLM notes, Key ideas)
//   dlm_depcap_boundary  (DepCap summary, Methodology bullets 1-3;
//                         Technical Contribution)
// One workgroup of kRuleNT threads per sequence (b); everything stays in
// registers/LDS.
#include <math.h>

#pragma once
#include "dlm_device.h"

namespace {

constexpr int kRuleNT = 256;

// Fast-dLLM: commit conf > tau inside the eligible set; if nothing passes,
// commit the top-1 eligible row (lowest row on ties; NaN never commits).
__device__ __forceinline__ void fastdllm_seq(int b, const float* __restrict__ conf,
                                             const uint8_t* __restrict__ eligible,
                                             const int32_t* __restrict__ seq_offsets,
                                             float tau, uint8_t* __restrict__ commit,
                                             int32_t* __restrict__ n_commit) {
  __shared__ float shf[kRuleNT / DLM_WAVE];
  __shared__ int shi[kRuleNT / DLM_WAVE];
  const int lo = seq_offsets[b], hi = seq_offsets[b + 1];
  int cnt = 0;
  float best = -INFINITY;
  int bidx = INT32_MAX;
  for (int r = lo + threadIdx.x; r < hi; r += kRuleNT) {
    const float c = conf[r];
    const bool el = eligible ? eligible[r] != 0 : true;
    const bool take = el && c > tau;
    commit[r] = take;
    cnt += take;
    if (el && c == c && (bidx == INT32_MAX || c > best)) {
      best = c;
      bidx = r;
    }
  }
  const int total = dlm::block_sum<kRuleNT>(cnt, shi);
  const int top = dlm::block_argmax<kRuleNT>(bidx == INT32_MAX ? NAN : best, bidx, shf, shi);
  if (threadIdx.x == 0) {
    int n = total;
    if (n == 0 && top != INT32_MAX) {
      commit[top] = 1;
      n = 1;
    }
    n_commit[b] = n;
  }
}

// DepCap's LDS, declared by the caller (__shared__) so that a kernel running
// other roles in other workgroups can overlay their LDS on it.
struct DepSmem {
  double sI[DLM_MAX_WINDOW];
  double sH[DLM_MAX_WINDOW];
  double shd[kRuleNT / DLM_WAVE];
  int shi[kRuleNT / DLM_WAVE];
};

// DepGA-Block boundary.  Window W = min(l_max, rows); box smoothing of
// radius R clipped to the window, division by the window mean (+eps),
// S_k = I~_k - lambda*H~_k in fp64, stored in fp64; k* = first S_k < 0.
__device__ __forceinline__ void depcap_seq(int b, const float* __restrict__ kl,
                                           const float* __restrict__ ent,
                                           const int32_t* __restrict__ seq_offsets,
                                           const uint8_t* __restrict__ has_prev,
                                           double lambda, int l_min, int l_max, int R,
                                           double eps, int32_t* __restrict__ block_len,
                                           double* __restrict__ score, DepSmem& sm) {
  auto& sI = sm.sI;
  auto& sH = sm.sH;
  auto& shd = sm.shd;
  auto& shi = sm.shi;
  const int lo = seq_offsets[b], n = seq_offsets[b + 1] - lo;
  const int W = max(0, min(l_max, n));
  const bool warm = has_prev ? has_prev[b] != 0 : true;
  R = min(R, W);  // a wider box covers the whole window anyway (and k + R stays in range)
  if (score)
    for (int k = W + threadIdx.x; k < n; k += kRuleNT) score[lo + k] = NAN;
  if (!warm || W == 0) {
    if (score)
      for (int k = threadIdx.x; k < W; k += kRuleNT) score[lo + k] = NAN;
    if (threadIdx.x == 0) block_len[b] = min(l_min, W);
    return;
  }
  for (int k = threadIdx.x; k < W; k += kRuleNT) {
    sI[k] = static_cast<double>(kl[lo + k]);
    sH[k] = static_cast<double>(ent[lo + k]);
  }
  __syncthreads();
  // smoothed values, kept in registers (each thread owns k = tid + j*kRuleNT)
  constexpr int KPT = DLM_MAX_WINDOW / kRuleNT;
  double ib[KPT], hb[KPT];
  double si = 0.0, sh = 0.0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int k = threadIdx.x + j * kRuleNT;
    ib[j] = hb[j] = 0.0;
    if (k < W) {
      const int j0 = max(0, k - R), j1 = min(W - 1, k + R);
      double a = 0.0, h = 0.0;
      for (int t = j0; t <= j1; ++t) {
        a += sI[t];
        h += sH[t];
      }
      ib[j] = a / static_cast<double>(j1 - j0 + 1);
      hb[j] = h / static_cast<double>(j1 - j0 + 1);
      si += ib[j];
      sh += hb[j];
    }
  }
  const double mi = dlm::block_sum<kRuleNT>(si, shd) / static_cast<double>(W);
  const double mh = dlm::block_sum<kRuleNT>(sh, shd) / static_cast<double>(W);
  int first = INT32_MAX;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int k = threadIdx.x + j * kRuleNT;
    if (k < W) {
      const double s = ib[j] / (mi + eps) - lambda * (hb[j] / (mh + eps));
      if (score) score[lo + k] = s;
      if (s < 0.0) first = min(first, k);
    }
  }
  const int ks = dlm::block_min_i<kRuleNT>(first, shi);
  if (threadIdx.x == 0) {
    const int kstar = ks == INT32_MAX ? W : ks;
    block_len[b] = min(max(kstar, l_min), W);
  }
}

}  // namespace
