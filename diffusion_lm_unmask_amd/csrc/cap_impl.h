// cap_impl.h — device code of dlm_cap_select: CAP-Decoding (DepCap summary,
// Methodology bullets 4-6; Technical Contribution; AI Executive Summary).
//
// One workgroup per sequence:
//   1. pool = eligible rows with conf >= tau_low, as 64-bit keys
//      (conf descending, row ascending) in LDS, sorted (one wave in registers
//      up to 64 keys, else the LDS bitonic sort).  Each row's argmax, lse and
//      row offset are read in the same pass as its confidence, so the
//      candidates need no second dependent trip to memory;
//   2. the first k_max become candidates; empty pool -> top-1 eligible row;
//   3. G[a][b] = logit_a[yhat_b] - lse_a gathered from HBM into LDS
//      (k_max^2 two-byte gathers), D_ab = G[a][b] + G[b][a] (bit-symmetric),
//      conflict bits (D_ab > gamma) as two 64-bit words per candidate;
//   4. the greedy in candidate order on one wave (readlane of each
//      candidate's conflict words): tau_high members unconditionally, the
//      rest when their conflict words do not meet the chosen set.
#include <math.h>

#pragma once
#include "dlm_device.h"

namespace {

constexpr int kCapNT = 256;
constexpr int kMaxRows = DLM_MAX_SEQ_ROWS;
constexpr int kKM = DLM_MAX_KMAX;

template <bool BF16>
__device__ __forceinline__ float gather(const void* logits, int64_t idx) {
  if constexpr (BF16) return dlm::bf16_at(static_cast<const uint16_t*>(logits), idx);
  return static_cast<const float*>(logits)[idx];
}

template <bool BF16>
__device__ __forceinline__ void cap_seq(int b, const void* __restrict__ logits, int64_t ld,
    int64_t vocab, const int64_t* __restrict__ row_index, const int32_t* __restrict__ seq_offsets,
    const float* __restrict__ conf, const int32_t* __restrict__ argmax,
    const float* __restrict__ lse, const uint8_t* __restrict__ eligible, float tau_low,
    float tau_high, float gamma, int k_max, uint8_t* __restrict__ commit,
    int32_t* __restrict__ n_commit, int32_t* __restrict__ cand_out, float* __restrict__ dmat_out) {
  __shared__ uint64_t keys[kMaxRows];
  __shared__ float rc[kMaxRows];      // by local row (pool rows only): conf
  __shared__ int32_t ry[kMaxRows];    // argmax
  __shared__ float rlse[kMaxRows];    // lse
  __shared__ int64_t rri[kMaxRows];   // row_index
  __shared__ float G[kKM][kKM + 1];
  __shared__ uint64_t cw[kKM][2];
  __shared__ int64_t coff[kKM];
  __shared__ int crow[kKM], cy[kKM];
  __shared__ float cconf[kKM], clse[kKM];
  __shared__ uint32_t sel[kMaxRows / 32];
  __shared__ float shf[kCapNT / DLM_WAVE];
  __shared__ int shi[kCapNT / DLM_WAVE];
  __shared__ int npool, bad;

  const int tid = threadIdx.x;
  const int lo = seq_offsets[b], n = seq_offsets[b + 1] - lo;
  const int64_t dbase = static_cast<int64_t>(b) * k_max * k_max;

  // a violated device-side precondition: commit nothing, report -1
  auto report = [&]() {
    for (int r = tid; r < n; r += kCapNT) commit[lo + r] = 0;
    if (cand_out)
      for (int a = tid; a < k_max; a += kCapNT) cand_out[b * k_max + a] = -1;
    if (dmat_out)
      for (int e = tid; e < k_max * k_max; e += kCapNT) dmat_out[dbase + e] = NAN;
    if (tid == 0) n_commit[b] = -1;
  };
  if (n > kMaxRows || n < 0) {  // device-side limit
    report();
    return;
  }
  if (tid == 0) {
    npool = 0;
    bad = 0;
  }
  for (int w = tid; w < kMaxRows / 32; w += kCapNT) sel[w] = 0u;
  __syncthreads();

  // 1. pool (arrival order is irrelevant: the sort makes it deterministic).
  // The per-row reads do not depend on each other (one trip to memory).
  float best = 0.f;
  int bidx = INT32_MAX;
  for (int r = tid; r < n; r += kCapNT) {
    const float c = conf[lo + r];
    const bool el = eligible ? eligible[lo + r] != 0 : true;
    const int32_t y = argmax[lo + r];
    const float l = lse[lo + r];
    const int64_t ri = row_index[lo + r];
    if (!el || c != c) continue;
    if (bidx == INT32_MAX || c > best) {
      best = c;
      bidx = r;
    }
    if (c >= tau_low) {
      const int slot = atomicAdd(&npool, 1);
      keys[slot] = (static_cast<uint64_t>(dlm::desc_bits(c)) << 32) | static_cast<uint32_t>(r);
      rc[r] = c;
      ry[r] = y;
      rlse[r] = l;
      rri[r] = ri;
    }
  }
  __syncthreads();
  const int P = npool;
  int n2 = 1;
  while (n2 < P) n2 <<= 1;
  if (n2 <= DLM_WAVE) {
    if (tid < DLM_WAVE && P > 1) {  // one wave, in registers: lane l holds key l
      const uint64_t v = dlm::wave_sort_asc(tid < P ? keys[tid] : ~0ull, n2);
      if (tid < P) keys[tid] = v;
    }
    __syncthreads();
  } else {
    for (int i = P + tid; i < n2; i += kCapNT) keys[i] = ~0ull;
    __syncthreads();
    dlm::bitonic_sort<kCapNT>(keys, n2);
  }
  const int K = min(P, k_max);

  if (K == 0) {  // 2. no candidate: top-1 eligible row
    const int top = dlm::block_argmax<kCapNT>(bidx == INT32_MAX ? NAN : best, bidx, shf, shi);
    for (int r = tid; r < n; r += kCapNT) commit[lo + r] = (r == top);
    if (cand_out)
      for (int a = tid; a < k_max; a += kCapNT) cand_out[b * k_max + a] = -1;
    if (dmat_out)
      for (int e = tid; e < k_max * k_max; e += kCapNT) dmat_out[dbase + e] = NAN;
    if (tid == 0) n_commit[b] = top == INT32_MAX ? 0 : 1;
    return;
  }

  for (int a = tid; a < K; a += kCapNT) {
    const int r = static_cast<int>(keys[a] & 0xffffffffu);
    crow[a] = lo + r;
    cconf[a] = rc[r];
    cy[a] = ry[r];
    clse[a] = rlse[r];
    coff[a] = rri[r] * ld;
    // every gather below is at coff[.] + cy[.]: check the indices first
    if (ry[r] < 0 || ry[r] >= vocab || rri[r] < 0) bad = 1;
  }
  __syncthreads();
  if (bad) {  // an argmax outside [0, vocab) or a negative row index
    report();
    return;
  }

  // 3. gathers G[a][b] = log p_a(yhat_b), eight in flight per lane
  const int KK = K * K;
  for (int base = tid; base < KK; base += 8 * kCapNT) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int p = base + u * kCapNT;
      v[u] = 0.f;
      if (p < KK) {
        const int a = p / K, e = p - a * K;
        v[u] = gather<BF16>(logits, coff[a] + cy[e]);
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int p = base + u * kCapNT;
      if (p < KK) {
        const int a = p / K, e = p - a * K;
        G[a][e] = v[u] - clse[a];
      }
    }
  }
  __syncthreads();

  // conflict words: wave w handles candidates a = w, w + 4, ...
  const int wv = tid / DLM_WAVE, ln = tid % DLM_WAVE;
  for (int a = wv; a < K; a += kCapNT / DLM_WAVE) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = h * DLM_WAVE + ln;
      bool c = false;
      if (e < K && e != a) c = (G[a][e] + G[e][a]) > gamma;
      const uint64_t bits = __ballot(c);
      if (ln == 0) cw[a][h] = bits;
    }
  }
  if (dmat_out) {
    for (int idx = tid; idx < k_max * k_max; idx += kCapNT) {
      const int a = idx / k_max, e = idx - a * k_max;
      float d = NAN;
      if (a < K && e < K && a != e) d = G[a][e] + G[e][a];
      dmat_out[dbase + idx] = d;
    }
  }
  __syncthreads();

  // 4. greedy pick on wave 0: lane l holds the conflict words of candidates
  // l and l + 64, and the scan reads them with readlane (no memory trip per
  // step).  s0 / s1 are the chosen candidates as a bitset.
  if (tid < DLM_WAVE) {
    uint64_t w00 = 0, w01 = 0, w10 = 0, w11 = 0;
    bool f0 = false, f1 = false;  // forced: conf > tau_high
    if (tid < K) {
      w00 = cw[tid][0];
      w01 = cw[tid][1];
      f0 = cconf[tid] > tau_high;
    }
    if (tid + DLM_WAVE < K) {
      w10 = cw[tid + DLM_WAVE][0];
      w11 = cw[tid + DLM_WAVE][1];
      f1 = cconf[tid + DLM_WAVE] > tau_high;
    }
    const uint64_t forced0 = __ballot(f0), forced1 = __ballot(f1);
    uint64_t s0 = 0, s1 = 0;
    for (int a = 0; a < K; ++a) {
      const int l = a & (DLM_WAVE - 1);
      const bool hi = a >= DLM_WAVE;
      const uint64_t c0 = dlm::rdlane64(hi ? w10 : w00, l);
      const uint64_t c1 = dlm::rdlane64(hi ? w11 : w01, l);
      const bool forced = (((hi ? forced1 : forced0) >> l) & 1ull) != 0;
      if (forced || ((c0 & s0) == 0 && (c1 & s1) == 0)) {
        if (hi) s1 |= 1ull << l;
        else s0 |= 1ull << l;
      }
    }
    if ((s0 >> tid) & 1ull) {
      const int lr = crow[tid] - lo;
      atomicOr(&sel[lr >> 5], 1u << (lr & 31));
    }
    if ((s1 >> tid) & 1ull) {
      const int lr = crow[tid + DLM_WAVE] - lo;
      atomicOr(&sel[lr >> 5], 1u << (lr & 31));
    }
    if (tid == 0) n_commit[b] = __popcll(s0) + __popcll(s1);
  }
  __syncthreads();
  for (int r = tid; r < n; r += kCapNT) commit[lo + r] = (sel[r >> 5] >> (r & 31)) & 1u;
  if (cand_out)
    for (int a = tid; a < k_max; a += kCapNT) cand_out[b * k_max + a] = a < K ? crow[a] : -1;
}

}  // namespace
