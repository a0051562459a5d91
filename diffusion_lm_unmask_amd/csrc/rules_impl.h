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

// The fused step knows the statistics' row count (n_rows >= 1).  When every
// sequence has the same number of rows (len), sequence b's rows are guessed
// as b * len .. before its offsets arrive, and read in the same trip to
// memory as the offsets; a guess that the offsets contradict is read again.
// With GUESS the first rows are read whatever the guess (from row 0 when
// len = 0), so that the loads carry no branch: a branch made the compiler
// wait for them before the offsets' load.  Rows at or above n_rows are never
// read.  The entry points do without (GUESS false).
struct RowGuess {
  int len;
  int64_t n_rows;
};

// Fast-dLLM: commit conf > tau inside the eligible set; if nothing passes,
// commit the top-1 eligible row (lowest row on ties; NaN never commits).
// One wave does it (the other waves of the workgroup return at once): the
// eligible set is an active block of a few rows, and a wave's DPP reductions
// need no workgroup barrier (the 256-thread version spent six barriers).
// Rows go in batches of four per lane, each lane in row order.
template <bool GUESS = false>
__device__ __forceinline__ void fastdllm_seq(int b, const float* __restrict__ conf,
                                             const uint8_t* __restrict__ eligible,
                                             const int32_t* __restrict__ seq_offsets,
                                             float tau, uint8_t* __restrict__ commit,
                                             int32_t* __restrict__ n_commit,
                                             RowGuess gs = {0, 1}) {
  if (threadIdx.x >= DLM_WAVE) return;
  constexpr int U = 4;
  const int lane = threadIdx.x;
  float c[U];
  uint8_t e[U];  // compared where used, so that no load waits for its value early
  // without an eligible set, bytes of conf (rows < n_rows, unused): the
  // loads carry no branch
  const uint8_t* ep = eligible ? eligible : reinterpret_cast<const uint8_t*>(conf);
  // rows base + lane + 64u, clamped below lim (lim > base); branch-free
  auto load = [&](int64_t base, int64_t lim) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t r = min(base + lane + u * DLM_WAVE, lim - 1);
      c[u] = conf[r];
      e[u] = ep[r];
    }
  };
  const int64_t g0 = static_cast<int64_t>(b) * gs.len;
  const bool guess = GUESS && gs.len > 0 && g0 < gs.n_rows;
  if constexpr (GUESS) load(guess ? g0 : 0, gs.n_rows);
  const int lo = seq_offsets[b], hi = seq_offsets[b + 1];  // in flight with the guess
  // both arrive here: keeps the compiler from moving the guessed loads into
  // the loop, behind the wait for the offsets
  if constexpr (GUESS)
    asm volatile("" ::"v"(c[0]), "v"(c[1]), "v"(c[2]), "v"(c[3]), "v"(uint32_t{e[0]}),
                 "v"(uint32_t{e[1]}), "v"(uint32_t{e[2]}), "v"(uint32_t{e[3]}), "v"(lo), "v"(hi));
  int cnt = 0;
  float best = -INFINITY;
  int bidx = INT32_MAX;
  bool held = guess && lo == g0 && hi <= gs.n_rows;  // the first batch is already here
  for (int base = lo; base < hi; base += U * DLM_WAVE) {
    if (!held) load(base, hi);
    held = false;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = base + lane + u * DLM_WAVE;
      if (r < hi) {
        const bool el = !eligible || e[u] != 0;
        const bool take = el && c[u] > tau;
        commit[r] = take;
        cnt += take;
        if (el && c[u] == c[u] && (bidx == INT32_MAX || c[u] > best)) {
          best = c[u];
          bidx = r;
        }
      }
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
constexpr int kDepKPT = kDepWaveRows / DLM_WAVE;

// Box sums of I and H over window positions j0 .. j1 (from +0.0, in position
// order).  For a radius of at most 1 the three reads are issued together,
// from clamped positions, and a neighbour outside the window adds +0.0: the
// running sums start at +0.0 and so are never -0.0, which makes that add
// exact, and the sums are bitwise those of the loop.  (The loop's reads wait
// for one another: 0.55 us of the one-wave path at radius 1.)
__device__ __forceinline__ void box_sums(const double* sI, const double* sH, int k, int W, int R,
                                         int j0, int j1, double& a, double& h) {
  a = 0.0;
  h = 0.0;
  if (R <= 1) {
    const int kl = max(k - 1, 0), kr = min(k + 1, W - 1);
    const double il = sI[kl], ic = sI[k], ir = sI[kr];
    const double hl = sH[kl], hc = sH[k], hr = sH[kr];
    const bool l = j0 < k, r = j1 > k;
    a = ((a + (l ? il : 0.0)) + ic) + (r ? ir : 0.0);
    h = ((h + (l ? hl : 0.0)) + hc) + (r ? hr : 0.0);
    return;
  }
  for (int t = j0; t <= j1; ++t) {
    a += sI[t];
    h += sH[t];
  }
}
__device__ __forceinline__ void depcap_window_wave(int lo, int W, int R,
                                                   const float* __restrict__ kl,
                                                   const float* __restrict__ ent, double lambda,
                                                   int l_min, double eps,
                                                   int32_t* __restrict__ block_len,
                                                   double* __restrict__ score, DepSmem& sm,
                                                   const float* gI, const float* gH, bool held) {
  if (threadIdx.x >= DLM_WAVE) return;
  const int lane = threadIdx.x;
  constexpr int KPT = kDepKPT;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int k = lane + j * DLM_WAVE;
    if (k < W) {
      sm.sI[k] = static_cast<double>(held ? gI[j] : kl[lo + k]);
      sm.sH[k] = static_cast<double>(held ? gH[j] : ent[lo + k]);
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
      double a, h;
      box_sums(sm.sI, sm.sH, k, W, R, j0, j1, a, h);
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
template <bool GUESS = false>
__device__ __forceinline__ void depcap_seq(int b, const float* __restrict__ kl,
                                           const float* __restrict__ ent,
                                           const int32_t* __restrict__ seq_offsets,
                                           const uint8_t* __restrict__ has_prev,
                                           double lambda, int l_min, int l_max, int R,
                                           double eps, int32_t* __restrict__ block_len,
                                           double* __restrict__ score, DepSmem& sm,
                                           RowGuess gs = {0, 1}) {
  auto& sI = sm.sI;
  auto& sH = sm.sH;
  auto& shd = sm.shd;
  auto& shi = sm.shi;
  // the guessed window (when it fits the one-wave path), read with the
  // offsets by every wave, so that the loads carry no branch
  const int64_t g0 = static_cast<int64_t>(b) * gs.len;
  const int gw = max(0, min(l_max, gs.len));
  const bool guess =
      GUESS && gs.len > 0 && gw > 0 && gw <= kDepWaveRows && g0 + gw <= gs.n_rows;
  float gI[kDepKPT], gH[kDepKPT];
  if constexpr (GUESS) {
    const int64_t base = guess ? g0 : 0;
    const int lim = guess ? gw : 1;
#pragma unroll
    for (int j = 0; j < kDepKPT; ++j) {
      const int64_t r = base + min(static_cast<int>(threadIdx.x % DLM_WAVE) + j * DLM_WAVE, lim - 1);
      gI[j] = kl[r];
      gH[j] = ent[r];
    }
  }
  const uint8_t* hpp = has_prev ? has_prev + b : reinterpret_cast<const uint8_t*>(seq_offsets);
  const uint8_t hraw = *hpp;  // has_prev in the same trip (no branch: without has_prev, a
                              // byte of the offsets, unused)
  const int lo = seq_offsets[b], n = seq_offsets[b + 1] - lo;  // in flight with the guess
  const int W = max(0, min(l_max, n));
  const bool warm = has_prev ? hraw != 0 : true;
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
    depcap_window_wave(lo, W, R, kl, ent, lambda, l_min, eps, block_len + b, score, sm, gI, gH,
                       guess && lo == g0 && W == gw);
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
      double a, h;
      box_sums(sI, sH, k, W, R, j0, j1, a, h);
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
