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
// One wave does it (the other waves of the workgroup return at once): the
// eligible set is an active block of a few rows, and a wave's DPP reductions
// need no workgroup barrier (the 256-thread version spent six barriers).
__device__ __forceinline__ void fastdllm_seq(int b, const float* __restrict__ conf,
                                             const uint8_t* __restrict__ eligible,
                                             const int32_t* __restrict__ seq_offsets,
                                             float tau, uint8_t* __restrict__ commit,
                                             int32_t* __restrict__ n_commit) {
  if (threadIdx.x >= DLM_WAVE) return;
  const int lane = threadIdx.x;
  const int lo = seq_offsets[b], hi = seq_offsets[b + 1];
  int cnt = 0;
  float best = -INFINITY;
  int bidx = INT32_MAX;
  for (int r = lo + lane; r < hi; r += DLM_WAVE) {
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
  const int total = dlm::wave_reduce(cnt, dlm::OpAdd{});
  const float m = dlm::wave_reduce(bidx == INT32_MAX ? -INFINITY : best, dlm::OpMaxF{});
  const int top =
      dlm::wave_reduce((bidx != INT32_MAX && best == m) ? bidx : INT32_MAX, dlm::OpMinI{});
  const bool fallback = total == 0 && top != INT32_MAX;
  // the lane that wrote the top row's 0 overwrites it (same thread, program order)
  if (fallback && (top - lo) % DLM_WAVE == lane) commit[top] = 1;
  if (lane == 0) n_commit[b] = fallback ? 1 : total;
}

// DepCap's LDS, declared by the caller (__shared__) so that a kernel running
// other roles in other workgroups can overlay their LDS on it.
struct DepSmem {
  double sI[DLM_MAX_WINDOW];
  double sH[DLM_MAX_WINDOW];
  double shd[kRuleNT / DLM_WAVE];
  int shi[kRuleNT / DLM_WAVE];
};

// Windows of up to kDepWaveRows positions: one wave computes the boundary
// (the other waves of the workgroup return at once), lane l owning positions
// l, l + 64, ...  The window is staged in LDS for the box filter; only this
// wave writes and reads it, and a wave's LDS operations execute in order, so
// the wavefront-scope fences (which keep the compiler from moving the reads
// above the writes) replace a workgroup barrier.  The sums are DPP
// reductions: the 256-thread version spent seven barriers on a 128-row window.
constexpr int kDepWaveRows = 4 * DLM_WAVE;
__device__ __forceinline__ void depcap_window_wave(int lo, int W, int R,
                                                   const float* __restrict__ kl,
                                                   const float* __restrict__ ent, double lambda,
                                                   int l_min, double eps,
                                                   int32_t* __restrict__ block_len,
                                                   double* __restrict__ score, DepSmem& sm) {
  if (threadIdx.x >= DLM_WAVE) return;
  const int lane = threadIdx.x;
  constexpr int KPT = kDepWaveRows / DLM_WAVE;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int k = lane + j * DLM_WAVE;
    if (k < W) {
      sm.sI[k] = static_cast<double>(kl[lo + k]);
      sm.sH[k] = static_cast<double>(ent[lo + k]);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  double ib[KPT], hb[KPT];
  double si = 0.0, sh = 0.0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int k = lane + j * DLM_WAVE;
    ib[j] = hb[j] = 0.0;
    if (k < W) {
      const int j0 = max(0, k - R), j1 = min(W - 1, k + R);
      double a = 0.0, h = 0.0;
      for (int t = j0; t <= j1; ++t) {
        a += sm.sI[t];
        h += sm.sH[t];
      }
      ib[j] = a / static_cast<double>(j1 - j0 + 1);
      hb[j] = h / static_cast<double>(j1 - j0 + 1);
      si += ib[j];
      sh += hb[j];
    }
  }
  const double mi = dlm::wave_sum(si) / static_cast<double>(W);
  const double mh = dlm::wave_sum(sh) / static_cast<double>(W);
  int first = INT32_MAX;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int k = lane + j * DLM_WAVE;
    if (k < W) {
      const double s = ib[j] / (mi + eps) - lambda * (hb[j] / (mh + eps));
      if (score) score[lo + k] = s;
      if (s < 0.0) first = min(first, k);
    }
  }
  const int ks = dlm::wave_reduce(first, dlm::OpMinI{});
  if (lane == 0) {
    const int kstar = ks == INT32_MAX ? W : ks;
    *block_len = min(max(kstar, l_min), W);
  }
}

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
  if (W <= kDepWaveRows) {
    depcap_window_wave(lo, W, R, kl, ent, lambda, l_min, eps, block_len + b, score, sm);
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
