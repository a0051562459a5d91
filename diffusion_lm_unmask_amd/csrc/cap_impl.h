// cap_impl.h — device code of dlm_cap_select: CAP-Decoding (DepCap summary,
// Methodology bullets 4-6; Technical Contribution; AI Executive Summary).
//
// One workgroup per sequence:
//   1. pool = eligible rows with conf >= tau_low, as 64-bit keys
//      (conf descending, row ascending) in LDS, ordered (one wave in
//      registers up to 64 keys; else runs of 64 sorted in registers and
//      ranked by binary search, keeping the first k_max).  Each row's argmax, lse and
//      row offset are read in the same pass as its confidence, so the
//      candidates need no second dependent trip to memory;
//   2. the first k_max become candidates; empty pool -> top-1 eligible row;
//   3. G[a][b] = logit_a[yhat_b] - lse_a gathered from HBM into LDS
//      (k_max^2 two-byte gathers), D_ab = G[a][b] + G[b][a] (bit-symmetric),
//      conflict bits (D_ab > gamma) as two 64-bit words per candidate;
//   4. the greedy in candidate order, in rounds on one wave (lane l holds
//      candidates l and l + 64): tau_high members unconditionally, the rest
//      when no earlier candidate they conflict with is chosen.
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

// G[a][b] = logit_a[yhat_b] - lse_a for a, b < K, kGU loads in flight per
// lane.  The loads carry no branch: an index past the end gathers the lane's
// own first pair again (tid < K*K inside the loop; unused, and a different
// address in every lane).  Guarded loads each ended in a wait for every load.
template <int kGU, bool BF16>
__device__ __forceinline__ void cap_gathers(const void* __restrict__ logits,
                                            const int64_t* coff, const int32_t* cy,
                                            const float* clse, float (*G)[kKM + 1], int K,
                                            int tid) {
  const int KK = K * K;
  for (int base = tid; base < KK; base += kGU * kCapNT) {
    float v[kGU];
#pragma unroll
    for (int u = 0; u < kGU; ++u) {
      const int p = base + u * kCapNT < KK ? base + u * kCapNT : tid;
      const int a = p / K, e = p - a * K;
      v[u] = gather<BF16>(logits, coff[a] + cy[e]);
    }
#pragma unroll
    for (int u = 0; u < kGU; ++u) {
      const int p = base + u * kCapNT;
      if (p < KK) {
        const int a = p / K, e = p - a * K;
        G[a][e] = v[u] - clse[a];
      }
    }
  }
}

// The workgroup's LDS.  The caller declares it (__shared__), so that a kernel
// running other roles in other workgroups can overlay their LDS on it.
struct CapSmem {
  uint64_t keys[kMaxRows];
  uint64_t top[kKM];       // the first k_max keys in order (runs path)
  float rc[kMaxRows];      // by local row (pool rows only): conf
  int32_t ry[kMaxRows];    // argmax
  float rlse[kMaxRows];    // lse
  int64_t rri[kMaxRows];   // row_index
  float G[kKM][kKM + 1];
  uint64_t cw[kKM][2];
  int64_t coff[kKM];
  int crow[kKM], cy[kKM];
  float cconf[kKM], clse[kKM];
  uint32_t sel[kMaxRows / 32];
  float shf[kCapNT / DLM_WAVE];
  int shi[kCapNT / DLM_WAVE];
  int npool, bad;
};

template <bool BF16>
__device__ __forceinline__ void cap_seq(int b, const void* __restrict__ logits, int64_t ld,
    int64_t vocab, const int64_t* __restrict__ row_index, const int32_t* __restrict__ seq_offsets,
    const float* __restrict__ conf, const int32_t* __restrict__ argmax,
    const float* __restrict__ lse, const uint8_t* __restrict__ eligible, float tau_low,
    float tau_high, float gamma, int k_max, uint8_t* __restrict__ commit,
    int32_t* __restrict__ n_commit, int32_t* __restrict__ cand_out, float* __restrict__ dmat_out,
    CapSmem& sm) {
  auto& keys = sm.keys;
  auto& top = sm.top;
  auto& rc = sm.rc;
  auto& ry = sm.ry;
  auto& rlse = sm.rlse;
  auto& rri = sm.rri;
  auto& G = sm.G;
  auto& cw = sm.cw;
  auto& coff = sm.coff;
  auto& crow = sm.crow;
  auto& cy = sm.cy;
  auto& cconf = sm.cconf;
  auto& clse = sm.clse;
  auto& sel = sm.sel;
  auto& shf = sm.shf;
  auto& shi = sm.shi;
  int& npool = sm.npool;
  int& bad = sm.bad;

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
    const int64_t ri = row_index ? row_index[lo + r] : static_cast<int64_t>(lo + r);
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
  const int K = min(P, k_max);
  int n2 = 1;
  while (n2 < P) n2 <<= 1;
  const uint64_t* order = keys;  // the candidates' keys in order
  if (n2 <= DLM_WAVE) {
    if (tid < DLM_WAVE && P > 1) {  // one wave, in registers: lane l holds key l
      const uint64_t v = dlm::wave_sort_asc(tid < P ? keys[tid] : ~0ull, n2);
      if (tid < P) keys[tid] = v;
    }
    __syncthreads();
  } else {
    // runs of 64 keys sorted in registers, ranks by binary search; only the
    // k_max first ranks are kept, in top
    dlm::sort_runs<kCapNT>(keys, top, P, K);
    order = top;
  }

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
    const int r = static_cast<int>(order[a] & 0xffffffffu);
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

  // 3. gathers G[a][b] = log p_a(yhat_b): eight in flight per lane, or four
  // when the K*K gathers fit in four per lane (an eight-wide batch would then
  // be half filler loads)
  if (K * K <= 4 * kCapNT)
    cap_gathers<4, BF16>(logits, coff, cy, clse, G, K, tid);
  else
    cap_gathers<8, BF16>(logits, coff, cy, clse, G, K, tid);
  __syncthreads();

  // conflict words.  Up to 32 candidates: wave w builds the words of
  // candidates w, w + 4, ... with one ballot per word (lane e tests pair
  // (a, e)).  More: item (a, h, q) sets bits 16q .. 16q + 15 of word h of
  // candidate a (e = 64h + 16q + i), stored as one 16-bit piece, which keeps
  // more reads in flight (measured: 0.5 against 0.9 us at K = 32, 2.8
  // against 1.7 us at K = 64).
  if (K <= 32) {
    const int wv = tid / DLM_WAVE, ln = tid % DLM_WAVE;
    for (int a = wv; a < K; a += kCapNT / DLM_WAVE) {
      bool c = false;
      if (ln < K && ln != a) c = (G[a][ln] + G[ln][a]) > gamma;
      const uint64_t bits = __ballot(c);
      if (ln == 0) {
        cw[a][0] = bits;
        cw[a][1] = 0ull;
      }
    }
  }
  for (int item = tid; K > 32 && item < K * 8; item += kCapNT) {
    const int a = item >> 3, h = (item >> 2) & 1, q = item & 3;
    const int e0 = h * DLM_WAVE + q * 16;
    uint32_t piece = 0u;
    if (e0 < K) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int e = e0 + i;
        const int ec = min(e, K - 1);  // read unconditionally: the 32 reads overlap
        const float d = G[a][ec] + G[ec][a];
        if (e < K && e != a && d > gamma) piece |= 1u << i;
      }
    }
    reinterpret_cast<uint16_t*>(&cw[a][h])[q] = static_cast<uint16_t>(piece);
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

  // 4. greedy on wave 0, in rounds: lane l holds candidates l and l + 64
  // (their conflict words and forced flags, conf > tau_high).  A forced
  // candidate is taken at once; any other is out as soon as an earlier
  // candidate it conflicts with is taken, and taken once all of those have
  // decided and none was taken.  The lowest undecided candidate always
  // decides, and each decision is the candidate-order scan's.  s0 / s1:
  // chosen candidates 0..63 / 64..127 as bitsets.
  if (tid < DLM_WAVE) {
    uint64_t w00 = 0, w10 = 0, w11 = 0;
    bool f0 = false, f1 = false;
    if (tid < K) {
      w00 = cw[tid][0];
      f0 = cconf[tid] > tau_high;
    }
    if (tid + DLM_WAVE < K) {
      w10 = cw[tid + DLM_WAVE][0];
      w11 = cw[tid + DLM_WAVE][1];
      f1 = cconf[tid + DLM_WAVE] > tau_high;
    }
    const uint64_t below = (1ull << tid) - 1ull;
    const uint64_t e0 = w00 & below;  // candidate l: earlier conflicts (all in word 0)
    const uint64_t e1 = w11 & below;  // candidate 64 + l: earlier conflicts in word 1 (plus w10)
    uint64_t open0 = K >= DLM_WAVE ? ~0ull : (1ull << K) - 1ull;
    uint64_t open1 = K <= DLM_WAVE ? 0ull : (K >= 2 * DLM_WAVE ? ~0ull : (1ull << (K - DLM_WAVE)) - 1ull);
    uint64_t s0 = 0, s1 = 0;
    while (K <= DLM_WAVE && open0) {  // one word: half the ballots per round
      const bool m0 = (open0 >> tid) & 1ull;
      const bool x0 = m0 && !f0 && (e0 & s0) != 0ull;
      const bool t0 = m0 && !x0 && (f0 || (e0 & open0) == 0ull);
      s0 |= __ballot(t0);
      open0 &= ~__ballot(t0 || x0);
    }
    while (open0 | open1) {
      const bool m0 = (open0 >> tid) & 1ull, m1 = (open1 >> tid) & 1ull;
      const bool x0 = m0 && !f0 && (e0 & s0) != 0ull;
      const bool x1 = m1 && !f1 && ((w10 & s0) | (e1 & s1)) != 0ull;
      const bool t0 = m0 && !x0 && (f0 || (e0 & open0) == 0ull);
      const bool t1 = m1 && !x1 && (f1 || ((w10 & open0) | (e1 & open1)) == 0ull);
      s0 |= __ballot(t0);
      s1 |= __ballot(t1);
      open0 &= ~__ballot(t0 || x0);
      open1 &= ~__ballot(t1 || x1);
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
