// rules.hip — the two per-sequence scans that need only per-row statistics:
//   dlm_fastdllm_select  (Fast-dLLM review, Method; Fast-dLLM notes, Key ideas)
//   dlm_depcap_boundary  (DepCap summary, Methodology bullets 1-3;
//                         Technical Contribution)
// One workgroup per sequence; everything stays in registers/LDS.
#include <math.h>

#include "dlm_device.h"

namespace {

constexpr int kNT = 256;

// Fast-dLLM: commit conf > tau inside the eligible set; if nothing passes,
// commit the top-1 eligible row (lowest row on ties; NaN never commits).
__global__ __launch_bounds__(kNT) void k_fastdllm(const float* __restrict__ conf,
                                                  const uint8_t* __restrict__ eligible,
                                                  const int32_t* __restrict__ seq_offsets,
                                                  float tau, uint8_t* __restrict__ commit,
                                                  int32_t* __restrict__ n_commit) {
  __shared__ float shf[kNT / DLM_WAVE];
  __shared__ int shi[kNT / DLM_WAVE];
  const int b = blockIdx.x;
  const int lo = seq_offsets[b], hi = seq_offsets[b + 1];
  int cnt = 0;
  float best = -INFINITY;
  int bidx = INT32_MAX;
  for (int r = lo + threadIdx.x; r < hi; r += kNT) {
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
  const int total = dlm::block_sum<kNT>(cnt, shi);
  const int top = dlm::block_argmax<kNT>(bidx == INT32_MAX ? NAN : best, bidx, shf, shi);
  if (threadIdx.x == 0) {
    int n = total;
    if (n == 0 && top != INT32_MAX) {
      commit[top] = 1;
      n = 1;
    }
    n_commit[b] = n;
  }
}

// DepGA-Block boundary.  Window W = min(l_max, rows); box smoothing of
// radius R clipped to the window, division by the window mean (+eps),
// S_k = I~_k - lambda*H~_k in fp64 rounded to f32; k* = first f32 S_k < 0.
__global__ __launch_bounds__(kNT) void k_depcap(const float* __restrict__ kl,
                                                const float* __restrict__ ent,
                                                const int32_t* __restrict__ seq_offsets,
                                                const uint8_t* __restrict__ has_prev,
                                                double lambda, int l_min, int l_max, int R,
                                                double eps, int32_t* __restrict__ block_len,
                                                float* __restrict__ score) {
  __shared__ double sI[DLM_MAX_WINDOW];
  __shared__ double sH[DLM_MAX_WINDOW];
  __shared__ double shd[kNT / DLM_WAVE];
  __shared__ int shi[kNT / DLM_WAVE];
  const int b = blockIdx.x;
  const int lo = seq_offsets[b], n = seq_offsets[b + 1] - lo;
  const int W = max(0, min(l_max, n));
  const bool warm = has_prev ? has_prev[b] != 0 : true;
  if (score)
    for (int k = W + threadIdx.x; k < n; k += kNT) score[lo + k] = NAN;
  if (!warm || W == 0) {
    if (score)
      for (int k = threadIdx.x; k < W; k += kNT) score[lo + k] = NAN;
    if (threadIdx.x == 0) block_len[b] = min(l_min, W);
    return;
  }
  for (int k = threadIdx.x; k < W; k += kNT) {
    sI[k] = static_cast<double>(kl[lo + k]);
    sH[k] = static_cast<double>(ent[lo + k]);
  }
  __syncthreads();
  // smoothed values, kept in registers (each thread owns k = tid + j*kNT)
  constexpr int KPT = DLM_MAX_WINDOW / kNT;
  double ib[KPT], hb[KPT];
  double si = 0.0, sh = 0.0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int k = threadIdx.x + j * kNT;
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
  const double mi = dlm::block_sum<kNT>(si, shd) / static_cast<double>(W);
  const double mh = dlm::block_sum<kNT>(sh, shd) / static_cast<double>(W);
  int first = INT32_MAX;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int k = threadIdx.x + j * kNT;
    if (k < W) {
      const float s = static_cast<float>(ib[j] / (mi + eps) - lambda * (hb[j] / (mh + eps)));
      if (score) score[lo + k] = s;
      if (s < 0.f) first = min(first, k);
    }
  }
  const int ks = dlm::block_min_i<kNT>(first, shi);
  if (threadIdx.x == 0) {
    const int kstar = ks == INT32_MAX ? W : ks;
    block_len[b] = min(max(kstar, l_min), W);
  }
}

}  // namespace

extern "C" int dlm_fastdllm_select(const float* conf, const uint8_t* eligible,
                                   const int32_t* seq_offsets, int32_t n_seq, float tau,
                                   uint8_t* commit, int32_t* n_commit, void* stream) {
  if (!conf || !seq_offsets || !commit || !n_commit || n_seq <= 0 || tau != tau)
    return DLM_ERR_ARG;
  hipLaunchKernelGGL(k_fastdllm, dim3(n_seq), dim3(kNT), 0, static_cast<hipStream_t>(stream),
                     conf, eligible, seq_offsets, tau, commit, n_commit);
  DLM_CHECK_LAUNCH();
  return DLM_OK;
}

extern "C" int dlm_depcap_boundary(const float* kl, const float* entropy,
                                   const int32_t* seq_offsets, int32_t n_seq,
                                   const uint8_t* has_prev, double lambda, int32_t l_min,
                                   int32_t l_max, int32_t smooth_radius, double eps,
                                   int32_t* block_len, float* score, void* stream) {
  if (!kl || !entropy || !seq_offsets || !block_len || n_seq <= 0) return DLM_ERR_ARG;
  if (lambda != lambda || eps != eps || eps < 0.0 || smooth_radius < 0 || l_min < 0 ||
      l_max <= 0 || l_min > l_max)
    return DLM_ERR_ARG;
  if (l_max > DLM_MAX_WINDOW) return DLM_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(k_depcap, dim3(n_seq), dim3(kNT), 0, static_cast<hipStream_t>(stream), kl,
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
