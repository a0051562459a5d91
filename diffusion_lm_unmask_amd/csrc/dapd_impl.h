// dapd_impl.h — device code of dlm_dapd_select and dlm_dapd_step: DAPD
// dependency graph and Welsh-Powell-ordered independent set (DAPD paper note: overall framework; key design 1
// (s_ij = (a_ij + a_ji)/2, edge iff s_ij > tau); key design 2 (proxy degree,
// order by degree x confidence, maximal independent set)).
//
// Three kernels:
//  k_dapd_avg    grid-wide, HBM-bound.  Streams only the masked x masked
//                sub-blocks of the n_lh attention maps (fp32 accumulation) and
//                writes a to the workspace.  A workgroup owns 32 (row, 8-column
//                chunk) items = one row x 256 columns, so each wave reads whole
//                512-byte row segments of two maps; its 512 lanes are 16 map
//                groups x 32 items (the statistics kernel's workgroup size, so
//                the fused step can run both in one launch), and a single
//                sequence already fills every CU.  A lane streams its maps
//                in double-buffered batches of DLM_DAPD_UNR_BF16 (more in
//                flight only queue up behind the memory system).  Map groups
//                are summed in LDS in a fixed order.
//  k_dapd_sym    grid-wide: s = (a + aT)/2 for 4 rows per workgroup (one
//                wave), one 16-lane team per row, lane l taking the 16
//                consecutive columns 16l .. 16l+15 of each 256 (four 16-byte
//                row loads), whose edge bits are its own 16-bit adjacency
//                piece; the transposed half a[j][i] is read from a itself
//                (the four teams of a wave read neighbouring columns of the
//                same rows), so no transposed copy is written; fp64 proxy
//                degree and the ordering key.
//  k_dapd_select one workgroup (1024 threads) per sequence (the fused step
//                runs it at 256 threads, in the sequence's last scores
//                workgroup; see dapd_scores_select; up to 64 rows, one wave
//                decides, see dapd_select_wave and dapd_small_select):
//                1. the adjacency bitset and keys into LDS;
//                2. order by the 64-bit keys (key desc, position asc): each
//                   wave sorts a run of 64 in registers, and a key's rank is
//                   its lane plus a binary search in every other run;
//                3. greedy over blocks of 64 nodes in that order: a node is
//                   blocked by an earlier block's chosen node (bitset AND) or by
//                   an earlier node of its own block (ballots), which gives the
//                   same set as the one-node-at-a-time scan.
//
// dlm_dapd_step adds the full step policy (DAPD note, key design 3): a
// sequence whose masked rows fell below late_frac of its generation length
// skips the graph (no attention read, no adjacency) and commits conf >
// late_tau with a top-1 fallback; rows with conf exactly 1.0 may be
// committed in either stage (pre-unmask).  Every kernel evaluates the same
// stage test, in fp64: M < late_frac * gen_len.
#include <math.h>

#pragma once
#include "dlm_device.h"

namespace {

// Tuning (build flags): map groups per averaging workgroup (a divisor of
// 512; the rest of the 512 lanes are 8-column items) and bf16 maps a lane
// keeps in flight in the averaging call.
#ifndef DLM_DAPD_GROUPS
#define DLM_DAPD_GROUPS 16
#endif
#ifndef DLM_DAPD_UNR_BF16
#define DLM_DAPD_UNR_BF16 4
#endif
constexpr int kGroups = DLM_DAPD_GROUPS;  // map groups per workgroup
constexpr int kAvgNT = 512;
constexpr int kItems = kAvgNT / kGroups;  // (row, 8-column chunk) items per workgroup
static_assert(kAvgNT % kGroups == 0 && kItems * 8 <= kAvgNT,
              "each of a tile's kItems * 8 outputs is finished by one thread");
constexpr int kTileRows = 1;
constexpr int kTileChunks = kItems / kTileRows;  // 8-column chunks per tile
constexpr int kSelNT = 1024;
constexpr int kMaxM = DLM_MAX_SEQ_ROWS;
constexpr int kWords = kMaxM / 64;

// Row stride (floats) of the workspace matrices: 16-float aligned rows.
__host__ __device__ inline int ws_ld(int m_max) { return (m_max + 15) & ~15; }

// The full-step policy; gen_len == nullptr and pre_unmask == 0 give the plain
// DAPD selection.
struct Policy {
  const int32_t* gen_len;  // [n_seq] generation length per sequence, or null
  float late_frac, late_tau;
  int pre_unmask;
  uint8_t* stage;          // [n_seq] 1 = late stage, or null
};
__device__ __forceinline__ bool late_stage(const Policy& P, int b, int M) {
  return P.gen_len != nullptr &&
         static_cast<double>(M) < static_cast<double>(P.late_frac) * static_cast<double>(P.gen_len[b]);
}

template <bool BF16>
__device__ __forceinline__ float ld1(const void* base, int64_t idx) {
  if constexpr (BF16) return dlm::bf16_at(static_cast<const uint16_t*>(base), idx);
  return static_cast<const float*>(base)[idx];
}

// UNR_BF16: bf16 maps per batch; PIPE: two batches in flight (else one).
// Neither changes the summation order (each lane adds its maps in map order),
// only how hard one tile presses on the memory system.
template <bool BF16, int UNR_BF16 = DLM_DAPD_UNR_BF16, bool PIPE = true>
__device__ __forceinline__ void dapd_avg_tile(int b, int tile, const void* __restrict__ attn,
    int n_lh, int64_t S, int64_t batch_stride, const int32_t* __restrict__ masked_pos,
    const int32_t* __restrict__ seq_offsets, int m_max, int n_tc, int vec_ok,
    float* __restrict__ ws_a, Policy P) {
  __shared__ float red[kGroups][kItems][9];
  const int lo = seq_offsets[b], M = seq_offsets[b + 1] - lo;
  if (M > m_max || M <= 0 || late_stage(P, b, M)) return;  // late stage: no graph
  const int ti = tile / n_tc, tc = tile % n_tc;
  const int i0 = ti * kTileRows, c0 = tc * kTileChunks;
  if (i0 >= M || c0 * 8 >= M) return;  // whole workgroup idle (uniform)
  const int g = threadIdx.x / kItems, it = threadIdx.x % kItems;
  const int i = i0 + it / kTileChunks, c = c0 + it % kTileChunks;
  const int j0 = c * 8;
  const int* pos = masked_pos + lo;
  // positions outside [0, S) are never dereferenced (k_dapd_select reports
  // the sequence)
  const bool item_ok = i < M && j0 < M && pos[i] >= 0 && pos[i] < S;

  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.f;

  if (item_ok) {
    const int64_t prow = static_cast<int64_t>(pos[i]) * S;
    int pj[8];
    bool contig = vec_ok && (j0 + 8 <= M);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      pj[k] = (j0 + k < M) ? pos[j0 + k] : -1;
      if (pj[k] >= S) pj[k] = -1;
      contig = contig && (pj[k] >= 0) && (pj[k] == pj[0] + k);
    }
    contig = contig && (pj[0] % (BF16 ? 8 : 4) == 0);
    const char* base = static_cast<const char*>(attn) +
                       static_cast<int64_t>(b) * batch_stride * (BF16 ? 2 : 4);
    const int64_t map_stride = S * S;
    if (contig) {
      // Lane maps g, g + kGroups, ... in batches of UNR.  PIPE: double-
      // buffered, the loads of batch k+1 issued before batch k is added, so
      // loads stay in flight while the lane adds; else one batch at a time.
      // Either way each lane adds its maps in map order.  Loads are
      // branch-free (an index past the last map reads the last map, and its
      // add is skipped by a select), which keeps the compiler's waits per
      // load rather than per loop trip.
      constexpr int UNR = BF16 ? UNR_BF16 : 2;
      constexpr int NQ = BF16 ? 1 : 2;  // 16-byte loads per map row piece
      constexpr int ES = BF16 ? 2 : 4;
      const char* rowp = base + (prow + pj[0]) * ES;
      const int64_t mbytes = map_stride * ES;
      const int last = n_lh - 1;
      auto load = [&](uint4 (&q)[UNR][NQ], int m0) {
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          const char* p = rowp + min(g + kGroups * (m0 + u), last) * mbytes;
#pragma unroll
          for (int h = 0; h < NQ; ++h) q[u][h] = *reinterpret_cast<const uint4*>(p + 16 * h);
        }
      };
      auto add = [&](const uint4 (&q)[UNR][NQ], int m0) {
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          const bool on = g + kGroups * (m0 + u) < n_lh;
          float v[8];
          if constexpr (BF16) {
            v[0] = dlm::bf16_lo(q[u][0].x);
            v[1] = dlm::bf16_hi(q[u][0].x);
            v[2] = dlm::bf16_lo(q[u][0].y);
            v[3] = dlm::bf16_hi(q[u][0].y);
            v[4] = dlm::bf16_lo(q[u][0].z);
            v[5] = dlm::bf16_hi(q[u][0].z);
            v[6] = dlm::bf16_lo(q[u][0].w);
            v[7] = dlm::bf16_hi(q[u][0].w);
          } else {
            v[0] = __uint_as_float(q[u][0].x);
            v[1] = __uint_as_float(q[u][0].y);
            v[2] = __uint_as_float(q[u][0].z);
            v[3] = __uint_as_float(q[u][0].w);
            v[4] = __uint_as_float(q[u][1].x);
            v[5] = __uint_as_float(q[u][1].y);
            v[6] = __uint_as_float(q[u][1].z);
            v[7] = __uint_as_float(q[u][1].w);
          }
#pragma unroll
          for (int k = 0; k < 8; ++k) acc[k] = on ? acc[k] + v[k] : acc[k];
        }
      };
      const int nm = (n_lh + kGroups - 1) / kGroups;  // maps of the fullest group
      const int nb = (nm + UNR - 1) / UNR;
      uint4 qa[UNR][NQ], qb[UNR][NQ];
      // the scheduling barriers keep each batch's loads ahead of the adds
      // that are meant to overlap them
      if constexpr (PIPE) {
        load(qa, 0);
        __builtin_amdgcn_sched_barrier(0);
        int k = 0;
        // the last trip is peeled, so every trip of the loop enters with the
        // same loads outstanding and the waits stay per load
        for (; k + 2 < nb; k += 2) {
          load(qb, (k + 1) * UNR);
          __builtin_amdgcn_sched_barrier(0);
          add(qa, k * UNR);
          load(qa, (k + 2) * UNR);
          __builtin_amdgcn_sched_barrier(0);
          add(qb, (k + 1) * UNR);
        }
        if (k + 1 < nb) {
          load(qb, (k + 1) * UNR);
          __builtin_amdgcn_sched_barrier(0);
          add(qa, k * UNR);
          add(qb, (k + 1) * UNR);
        } else {
          add(qa, k * UNR);
        }
      } else {
        for (int k = 0; k < nb; ++k) {
          load(qa, k * UNR);
          __builtin_amdgcn_sched_barrier(0);
          add(qa, k * UNR);
        }
      }
    } else {
      for (int lh = g; lh < n_lh; lh += kGroups) {
        const int64_t e = static_cast<int64_t>(lh) * map_stride + prow;
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (pj[k] >= 0) acc[k] += ld1<BF16>(base, e + pj[k]);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) red[g][it][k] = acc[k];
  __syncthreads();
  // 32 items x 8 columns = 256 outputs; thread t < 256 finishes one
  if (threadIdx.x < kItems * 8) {
    const int oi = threadIdx.x / 8, k = threadIdx.x % 8;
    const int ri = i0 + oi / kTileChunks, rj = (c0 + oi % kTileChunks) * 8 + k;
    if (ri < M && rj < M) {
      float s = red[0][oi][k];
#pragma unroll
      for (int q = 1; q < kGroups; ++q) s += red[q][oi][k];  // fixed order
      const float a = s / static_cast<float>(n_lh);
      const int ld = ws_ld(m_max);
      ws_a[(static_cast<int64_t>(b) * m_max + ri) * ld + rj] = a;
    }
  }
}

// Workspace layout (every region 256-byte aligned), for n_seq x m_max:
//   a          f32 [n_seq][m_max][ws_ld]     averaged maps
//   adj        u64 [n_seq][m_max][words]     adjacency bitsets, words = ceil(m_max/64)
//   keys       u64 [n_seq][m_max]            (order key, position)
//   has_edge   u8  [n_seq][m_max]            bit 0: an edge; bit 1: position out of range
//   tally      u64 [n_seq]                   the fused step's per-sequence counters
struct Layout {
  size_t a, adj, keys, has_edge, tally, total;
  int ld, words;
};
__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
__host__ __device__ inline Layout layout(int n_seq, int m_max) {
  Layout L;
  L.ld = ws_ld(m_max);
  L.words = (m_max + 63) / 64;
  const size_t nm = static_cast<size_t>(n_seq) * m_max;
  L.a = 0;
  L.adj = align256(nm * L.ld * sizeof(float));
  L.keys = L.adj + align256(nm * L.words * sizeof(uint64_t));
  L.has_edge = L.keys + align256(nm * sizeof(uint64_t));
  L.tally = L.has_edge + align256(nm);
  L.total = L.tally + align256(static_cast<size_t>(n_seq) * sizeof(uint64_t));
  return L;
}

// Rows per k_dapd_sym workgroup: one wave of four 16-lane teams, one row
// each.  (Sixteen rows per workgroup, four waves, measured 6.4 against 5.1
// us on the step; 32-lane teams, half the steps per wave but twice the waves
// and cache lines, made the fused LLaDA step 0.6 us slower.)
constexpr int kTeam = 16;
constexpr int kSymRows = DLM_WAVE / kTeam;
constexpr int kSymNT = DLM_WAVE;

// A row's part of its sequence's tally (the fused step adds them up): bits
// 16-31 count commits as an edgeless graph makes them, 32-47 rows with an
// edge, 48-63 rows whose position is out of range (or a sequence longer than
// m_max).  Bits 0-15 count blocks of kSymRows rows.  Each field stays below
// 2^16 (at most 1024 rows, at most 512 blocks per sequence).
constexpr uint64_t kTallyWG = 1ull, kTallyCommit = 1ull << 16, kTallyEdge = 1ull << 32,
                   kTallyBad = 1ull << 48;

// s = (a + aT)/2 for kSymRows rows per workgroup: adjacency bits (each lane's
// own 16-column piece), fp64 proxy degree (fixed-pattern reduction over the
// team), ordering key.  Each
// row's masked position is checked here too: has_edge carries bit 1 for a
// position outside [0, S), which the selection reports.  With `commit`, each
// row also gets the commit an edgeless graph gives it (a key that is not NaN,
// or pre-unmasked).  Returns the row's tally on its team's lane 0, else 0.
__device__ __forceinline__ uint64_t dapd_sym_rows(int b, int rb,
    const int32_t* __restrict__ seq_offsets, const int32_t* __restrict__ masked_pos, int64_t S,
    int m_max, const float* __restrict__ conf, float tau,
    const char* __restrict__ ws, Layout L, float* __restrict__ degree, float* __restrict__ sym,
    float* __restrict__ key_out, Policy P, uint8_t* __restrict__ commit) {
  const int lo = seq_offsets[b], M = seq_offsets[b + 1] - lo;
  const int team = (threadIdx.x % DLM_WAVE) / kTeam, tl = threadIdx.x % kTeam;  // this wave's teams
  const int i = rb * kSymRows + team;
  const int64_t sbase = static_cast<int64_t>(b) * m_max * m_max;
  if (M > m_max || M < 0) return tl == 0 ? kTallyBad : 0ull;  // over-long: the selection reports
  if (i >= m_max) return 0ull;
  if (i >= M || late_stage(P, b, M)) {  // pad rows, or no graph: NaN in the optional outputs
    if (i < M && tl == 0) {
      if (degree) degree[lo + i] = NAN;
      if (key_out) key_out[lo + i] = NAN;
    }
    if (sym)
      for (int j = tl; j < m_max; j += 16) sym[sbase + static_cast<int64_t>(i) * m_max + j] = NAN;
    return 0ull;
  }
  // read now, used at the end: their latency hides behind the row reads
  const int pos_i = masked_pos[lo + i];
  const float conf_i = conf[lo + i];
  const float* A = reinterpret_cast<const float*>(ws + L.a) + static_cast<int64_t>(b) * m_max * L.ld;
  const float* ar = A + static_cast<int64_t>(i) * L.ld;
  // the row's adjacency words, as 16-bit pieces: piece q = columns 16q .. 16q+15
  uint16_t* adjp = reinterpret_cast<uint16_t*>(
      const_cast<char*>(ws) + L.adj + (static_cast<int64_t>(b) * m_max + i) * L.words * 8);
  const int nw = (M + 63) / 64;
  float* so = sym ? sym + sbase + static_cast<int64_t>(i) * m_max : nullptr;
  double dsum = 0.0;
  bool any = false;
  for (int c0 = 0; c0 < 64 * nw; c0 += 256) {
    // lane tl takes the 16 consecutive columns j0 .. j0 + 15 of its piece
    // c0/16 + tl, so its edge bits are its own piece (no ballots).  Its row
    // part is four 16-byte loads: from column j0, or, past the row's stride
    // (columns that are all >= M, read and masked), from its last 16
    // columns.  a[j][i] (the transposed half) is read straight from a, with
    // columns past M reading column M - 1 (i < M, so M >= 1); every load is
    // in range and none is branched.
    const int j0 = c0 + 16 * tl;
    float va[16], vt[16];
    const float4* rp = reinterpret_cast<const float4*>(ar + min(j0, L.ld - 16));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 f = rp[q];
      va[4 * q] = f.x;
      va[4 * q + 1] = f.y;
      va[4 * q + 2] = f.z;
      va[4 * q + 3] = f.w;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int jc = min(j0 + e, M - 1);
      vt[e] = A[static_cast<int64_t>(jc) * L.ld + i];
    }
    // off-diagonal columns below M as a 16-bit lane mask; a masked column
    // adds +0.0 to the degree (the same sum as skipping it: the terms are
    // never negative) and sets no edge
    const int lim = M - j0, di = i - j0;
    uint32_t valid = lim >= 16 ? 0xffffu : (lim <= 0 ? 0u : (1u << lim) - 1u);
    if (di >= 0 && di < 16) valid &= ~(1u << di);
    float sv[16];
    uint32_t gt = 0u;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      sv[e] = 0.5f * (va[e] + vt[e]);
      gt |= static_cast<uint32_t>(sv[e] > tau) << e;
      dsum += static_cast<double>(((valid >> e) & 1u) ? sv[e] : 0.0f);
    }
    const uint32_t mine = gt & valid;
    if (so) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int j = j0 + e;
        if (j < m_max) so[j] = j < M ? sv[e] : NAN;
      }
    }
    if (j0 < 64 * nw) adjp[c0 / 16 + tl] = static_cast<uint16_t>(mine);  // zero past M
    any = any || mine != 0u;
  }
  if (so)
    for (int j = 64 * nw + tl; j < m_max; j += 16) so[j] = NAN;
  // over the team's 16 lanes (a DPP row), in a fixed pattern
  dsum += dlm::xor_val<8>(dsum);
  dsum += dlm::xor_val<4>(dsum);
  dsum += dlm::xor_val<2>(dsum);
  dsum += dlm::xor_val<1>(dsum);
  uint32_t anyb = any ? 1u : 0u;
  anyb |= dlm::xor_val<8>(anyb);
  anyb |= dlm::xor_val<4>(anyb);
  anyb |= dlm::xor_val<2>(anyb);
  anyb |= dlm::xor_val<1>(anyb);
  if (tl == 0) {
    const float df = static_cast<float>(dsum);
    const float kk = df * conf_i;
    if (degree) degree[lo + i] = df;
    if (key_out) key_out[lo + i] = kk;
    const uint64_t hi = (kk != kk) ? 0xffffffffull : static_cast<uint64_t>(dlm::desc_bits(kk));
    // NaN keys sort last; every other key maps below 0xffffffff
    reinterpret_cast<uint64_t*>(const_cast<char*>(ws) + L.keys)[static_cast<int64_t>(b) * m_max + i] =
        (hi << 32) | static_cast<uint32_t>(i);
    const uint32_t bad = pos_i < 0 || pos_i >= S;
    reinterpret_cast<uint8_t*>(const_cast<char*>(ws) + L.has_edge)[static_cast<int64_t>(b) * m_max + i] =
        static_cast<uint8_t>(anyb | (bad << 1));
    const uint32_t c = (kk == kk) | (P.pre_unmask && conf_i == 1.0f);
    if (commit) commit[lo + i] = static_cast<uint8_t>(c);
    return c * kTallyCommit + anyb * kTallyEdge + bad * kTallyBad;
  }
  return 0ull;
}

// The greedy's LDS for NT threads, declared by the caller (__shared__) so
// that a kernel running other roles in other workgroups can overlay their LDS
// on it.
template <int NT>
struct SelSmem {
  uint64_t adj[kMaxM][kWords];   // 128 KiB; row i = neighbours of node i
  uint64_t keys[kMaxM];          // by node, then sorted runs of 64
  uint64_t chosen[kWords];
  uint64_t bmk[kWords][kWords];  // block k (ranks 64k..64k+63): its nodes as a bitset
  uint64_t lmask[kMaxM];         // by rank: lanes of the earlier neighbours in its block
  uint64_t tally;                // the fused step: the sequence's totals
  uint64_t part[NT / DLM_WAVE];  // the fused step: each wave's tally
  int16_t order[kMaxM];          // node of rank t (-1 - node: NaN key)
  int16_t rank_of[kMaxM];        // rank of each node
  uint8_t has_edge[kMaxM];
  int shi[NT / DLM_WAVE];
  float shf[NT / DLM_WAVE];
  int last;                      // the fused step: this workgroup counted in last
};

// Exclusive OR scan over the wave: lane l gets the OR of lanes 0 .. l-1.
// An xor butterfly: at distance d, a lane in the upper half of its aligned
// 2d-lane segment takes the lower half's total, and both halves' totals
// merge.
template <int D>
__device__ __forceinline__ void or_scan_step(uint64_t& seg, uint64_t& below, int l) {
  const uint64_t o = dlm::xor_lane64<D>(seg);
  if (l & D) below |= o;
  seg |= o;
}
__device__ __forceinline__ uint64_t wave_or_scan_excl(uint64_t v, int l) {
  uint64_t below = 0ull;
  or_scan_step<1>(v, below, l);
  or_scan_step<2>(v, below, l);
  or_scan_step<4>(v, below, l);
  or_scan_step<8>(v, below, l);
  or_scan_step<16>(v, below, l);
  or_scan_step<32>(v, below, l);
  return below;
}

// A sequence of at most 64 masked positions outside the late stage, on one
// wave, node r on lane r.  The keys sort in registers (rank t on lane t); an
// OR scan over the ranks gives each rank the nodes ordered before it, which
// goes back to that rank's node lane, where it masks the node's adjacency
// word into its earlier neighbours.  The greedy then runs in rounds on node
// bits, so the chosen set is the one the order defines.  No LDS and no
// barrier.
// The decision itself, given node ln's key, edge flags (bit 0: an edge, bit
// 1: position out of range) and adjacency word on lane ln (lanes >= M:
// anything).
__device__ __forceinline__ void dapd_decide_wave(int b, int lo, int M, int m_max, uint64_t kk,
    uint32_t he, uint64_t adj, const float* __restrict__ conf, uint8_t* __restrict__ commit,
    int32_t* __restrict__ n_commit, float* __restrict__ degree, float* __restrict__ sym,
    float* __restrict__ key_out, Policy P) {
  const int ln = threadIdx.x % DLM_WAVE;
  const bool in = ln < M;
  const float cf = (P.pre_unmask && in) ? conf[lo + ln] : 0.f;  // an empty last sequence has lo = rows
  if (!in) {
    kk = ~0ull;  // padding keys sort after every node
    he = 0u;
    adj = 0ull;
  }
  if (__ballot(in && (he & 2u))) {  // a position out of range: report
    if (in) {
      commit[lo + ln] = 0;
      if (degree) degree[lo + ln] = NAN;
      if (key_out) key_out[lo + ln] = NAN;
    }
    if (sym)
      for (int64_t e = ln; e < static_cast<int64_t>(m_max) * m_max; e += DLM_WAVE)
        sym[static_cast<int64_t>(b) * m_max * m_max + e] = NAN;
    if (ln == 0) {
      n_commit[b] = -1;
      if (P.stage) P.stage[b] = 0;
    }
    return;
  }
  if (ln == 0 && P.stage) P.stage[b] = 0;
  uint64_t take;  // chosen nodes, as node bits
  if (__ballot(in && (he & 1u)) == 0ull) {
    take = __ballot(in && (kk >> 32) != 0xffffffffull);  // no edge: every node with a key
  } else {
    // lane t: the key of rank t (a power-of-two run of at least M lanes; the
    // padding keys above it sort among themselves)
    const int n = M <= 16 ? 16 : M <= 32 ? 32 : DLM_WAVE;
    const uint64_t sk = dlm::wave_sort_asc(kk, n);
    const bool valid = ln < M;
    const int v = static_cast<int>(sk & 0xffffffffu);
    // the nodes of the ranks below t
    const uint64_t below = wave_or_scan_excl(valid ? 1ull << v : 0ull, ln);
    // back to node lanes: rank t sends its set to lane v (the padding ranks,
    // t >= M, to themselves, so every lane receives exactly one)
    const int dst = (valid ? v : ln) << 2;
    const uint32_t blo = static_cast<uint32_t>(
        __builtin_amdgcn_ds_permute(dst, static_cast<int>(below)));
    const uint32_t bhi = static_cast<uint32_t>(
        __builtin_amdgcn_ds_permute(dst, static_cast<int>(below >> 32)));
    // node ln's earlier neighbours, as node bits
    const uint64_t E = in ? adj & ((static_cast<uint64_t>(bhi) << 32) | blo) : 0ull;
    // rounds: a node with a chosen earlier neighbour is out at once; one whose
    // earlier neighbours have all decided, none chosen, is chosen.  The
    // lowest undecided node always decides, and every decision is the one
    // the node-by-node scan in key order makes.  A NaN key is never chosen.
    uint64_t sel = 0ull, open = __ballot(in && (kk >> 32) != 0xffffffffull);
    while (open) {
      const bool mine = (open >> ln) & 1ull;
      const bool out = mine && (E & sel) != 0ull;
      const bool pick = mine && !out && (E & open) == 0ull;
      sel |= __ballot(pick);
      open &= ~__ballot(pick || out);
    }
    take = sel;
  }
  const bool c = in && (((take >> ln) & 1ull) || (P.pre_unmask && cf == 1.0f));
  if (in) commit[lo + ln] = static_cast<uint8_t>(c);
  const uint64_t cb = __ballot(c);
  if (ln == 0) n_commit[b] = __popcll(cb);
}
__device__ __forceinline__ void dapd_select_wave(int b, int lo, int M, int m_max,
    const char* __restrict__ ws, Layout L, const float* __restrict__ conf,
    uint8_t* __restrict__ commit, int32_t* __restrict__ n_commit, float* __restrict__ degree,
    float* __restrict__ sym, float* __restrict__ key_out, Policy P) {
  const int ln = threadIdx.x % DLM_WAVE;
  const int r = ln < M ? ln : 0;  // lanes past the sequence read its first entry (unused)
  const int64_t row = static_cast<int64_t>(b) * m_max;
  const uint64_t kk = reinterpret_cast<const uint64_t*>(ws + L.keys)[row + r];
  const uint32_t he = reinterpret_cast<const uint8_t*>(ws + L.has_edge)[row + r];
  const uint64_t adj = reinterpret_cast<const uint64_t*>(ws + L.adj)[(row + r) * L.words];
  dapd_decide_wave(b, lo, M, m_max, kk, he, adj, conf, commit, n_commit, degree, sym, key_out, P);
}

// Per sequence: load the graph into LDS, order the nodes, run the greedy
// (NT threads).  The result does not depend on NT.
template <int NT>
__device__ __forceinline__ void dapd_select_seq(int b, const int32_t* __restrict__ masked_pos,
    int64_t S, const int32_t* __restrict__ seq_offsets, int m_max, const char* __restrict__ ws,
    Layout L, const float* __restrict__ conf, uint8_t* __restrict__ commit,
    int32_t* __restrict__ n_commit, float* __restrict__ degree, float* __restrict__ sym,
    float* __restrict__ key_out, Policy P, SelSmem<NT>& sm) {
  constexpr int NW = NT / DLM_WAVE;
  auto& adj = sm.adj;
  auto& keys = sm.keys;
  auto& order = sm.order;
  auto& chosen = sm.chosen;
  auto& rank_of = sm.rank_of;
  auto& bmk = sm.bmk;
  auto& lmask = sm.lmask;
  auto& has_edge = sm.has_edge;
  auto& shi = sm.shi;
  auto& shf = sm.shf;
  const int tid = threadIdx.x;
  const int wv = tid / DLM_WAVE, ln = tid % DLM_WAVE;
  const int lo = seq_offsets[b], M = seq_offsets[b + 1] - lo;
  const int64_t sbase = static_cast<int64_t>(b) * m_max * m_max;

  auto report = [&]() {  // nothing committed, n_commit = -1
    for (int r = tid; r < M; r += NT) {
      commit[lo + r] = 0;
      if (degree) degree[lo + r] = NAN;
      if (key_out) key_out[lo + r] = NAN;
    }
    if (sym)
      for (int64_t e = tid; e < static_cast<int64_t>(m_max) * m_max; e += NT)
        sym[sbase + e] = NAN;
    if (tid == 0) {
      n_commit[b] = -1;
      if (P.stage) P.stage[b] = 0;
    }
  };
  if (M > m_max || M < 0) {  // over-long sequence
    report();
    return;
  }
  const bool late = late_stage(P, b, M);  // uniform over the workgroup
  if (M <= DLM_WAVE && !late) {  // uniform: one wave decides, the others leave
    if (wv == 0)
      dapd_select_wave(b, lo, M, m_max, ws, L, conf, commit, n_commit, degree, sym, key_out, P);
    return;
  }
  // a masked position outside [0, S) reports the sequence.  In the graph
  // stage the scores kernel has checked every row (bit 1 of has_edge), so
  // the graph's loads below are the only trip to memory before the check.
  int bad_pos = 0, any_edge = 0;
  const int nw = (M + 63) / 64;  // adjacency words in use
  if (late) {
    for (int r = tid; r < M; r += NT) {
      const int p = masked_pos[lo + r];
      bad_pos |= p < 0 || p >= S;
    }
  } else {
    const uint64_t* gadj = reinterpret_cast<const uint64_t*>(ws + L.adj) +
                           static_cast<int64_t>(b) * m_max * L.words;
    const uint64_t* gkeys = reinterpret_cast<const uint64_t*>(ws + L.keys) +
                            static_cast<int64_t>(b) * m_max;
    const uint8_t* gedge = reinterpret_cast<const uint8_t*>(ws + L.has_edge) +
                           static_cast<int64_t>(b) * m_max;
    // every load of a batch is issued before its LDS stores, so a thread
    // with several words (fewer threads, longer sequences) waits for memory
    // once per batch rather than once per word
    constexpr int kAU = 8, kKU = 4;
    const int n_adj = M * nw;
    for (int e0 = tid; e0 < n_adj; e0 += kAU * NT) {
      uint64_t v[kAU];
#pragma unroll
      for (int u = 0; u < kAU; ++u) {
        const int e = e0 + u * NT;
        if (e < n_adj) {
          const int i = e / nw, w = e - i * nw;
          v[u] = gadj[static_cast<int64_t>(i) * L.words + w];
        }
      }
#pragma unroll
      for (int u = 0; u < kAU; ++u) {
        const int e = e0 + u * NT;
        if (e < n_adj) {
          const int i = e / nw, w = e - i * nw;
          adj[i][w] = v[u];
        }
      }
    }
    for (int e0 = tid; e0 < M; e0 += kKU * NT) {
      uint64_t kv[kKU];
      uint8_t he[kKU];
#pragma unroll
      for (int u = 0; u < kKU; ++u) {
        const int e = e0 + u * NT;
        if (e < M) {
          kv[u] = gkeys[e];
          he[u] = gedge[e];
        }
      }
#pragma unroll
      for (int u = 0; u < kKU; ++u) {
        const int e = e0 + u * NT;
        if (e < M) {
          keys[e] = kv[u];
          has_edge[e] = he[u] & 1u;
          any_edge |= he[u] & 1u;
          bad_pos |= he[u] >> 1;
        }
      }
    }
    if (tid < kWords) chosen[tid] = 0ull;
    for (int e = tid; e < kWords * kWords; e += NT) bmk[e / kWords][e % kWords] = 0ull;
    for (int t = tid; t < M; t += NT) lmask[t] = 0ull;
  }
  const int flags = dlm::block_or_i<NT>(bad_pos | (any_edge << 1), shi);  // ends with a barrier
  if (flags & 1) {
    report();
    return;
  }
  if (tid == 0 && P.stage) P.stage[b] = static_cast<uint8_t>(late);
  if (late) {  // no graph: conf > late_tau, else the most confident row
    int above = 0, bi = INT32_MAX;
    float bv = -INFINITY;
    for (int r = tid; r < M; r += NT) {
      const float cf = conf[lo + r];
      above += cf > P.late_tau;
      if (cf == cf && (bi == INT32_MAX || cf > bv)) {
        bv = cf;
        bi = r;
      }
    }
    above = dlm::block_sum<NT>(above, shi);
    const int fb = above == 0 ? dlm::block_argmax<NT>(bv, bi, shf, shi) : INT32_MAX;
    int cnt = 0;
    for (int r = tid; r < M; r += NT) {
      const float cf = conf[lo + r];
      const int c = (cf > P.late_tau) || r == fb || (P.pre_unmask && cf == 1.0f);
      commit[lo + r] = static_cast<uint8_t>(c);
      cnt += c;
    }
    cnt = dlm::block_sum<NT>(cnt, shi);
    if (tid == 0) n_commit[b] = cnt;
    return;
  }

  if (!(flags & 2)) {
    // no edge anywhere: the independent set is every node whatever the
    // order, except a NaN key (never chosen)
    int cnt = 0;
    for (int r = tid; r < M; r += NT) {
      const int c = static_cast<int>((keys[r] >> 32) != 0xffffffffull) |
                    (P.pre_unmask && conf[lo + r] == 1.0f);  // pre-unmask
      commit[lo + r] = static_cast<uint8_t>(c);
      cnt += c;
    }
    cnt = dlm::block_sum<NT>(cnt, shi);
    if (tid == 0) n_commit[b] = cnt;
    return;
  }

  // ---- order the nodes (keys are unique: they carry the node).  Wave w
  // sorts runs w, w + NW, ... (keys 64r .. 64r+63 of run r) in registers; a
  // key's rank is its lane plus, for every other sorted run, the number of
  // keys below it (binary searches, four runs side by side).  Padding keys
  // (~0) sort after every node and get no rank.
  const int n_runs = (M + 63) / 64;
  for (int run = wv; run < n_runs; run += NW) {  // whole waves: every lane takes part
    const int i = run * 64 + ln;
    keys[i] = dlm::wave_sort_asc(i < M ? keys[i] : ~0ull, 64);  // a wave rewrites only its run
  }
  __syncthreads();
  for (int run = wv; run < n_runs; run += NW) {
    const uint64_t v = keys[run * 64 + ln];
    if (v == ~0ull) continue;
    const int rank = ln + dlm::count_below_in_runs(keys, n_runs, run, v);
    // a NaN key (it sorts after every finite key) is stored as -1 - node:
    // such a node is never chosen
    const int node = static_cast<int>(v & 0xffffffffu);
    order[rank] = static_cast<int16_t>((v >> 32) == 0xffffffffull ? -1 - node : node);
    rank_of[node] = static_cast<int16_t>(rank);
    atomicOr(reinterpret_cast<unsigned long long*>(&bmk[rank >> 6][node >> 6]), 1ull << (node & 63));
  }
  __syncthreads();

  // ---- each node's earlier neighbours inside its block of 64 ranks, as lane
  // bits.  They do not depend on what earlier blocks chose, so every node is
  // done at once here rather than inside the sequential greedy: one
  // (node, adjacency word) pair per thread, ORed into the node's mask
  // (zeroed with the loads).
  for (int e = tid; e < M * nw; e += NT) {
    const int v = e / nw, w = e - v * nw;
    if (!has_edge[v]) continue;
    const int t = rank_of[v], k = t >> 6;
    uint64_t m = adj[v][w] & bmk[k][w];
    uint64_t loc = 0ull;
    while (m) {
      const int ru = rank_of[w * 64 + __builtin_ctzll(m)];
      m &= m - 1;
      if (ru < t) loc |= 1ull << (ru & 63);
    }
    if (loc) atomicOr(reinterpret_cast<unsigned long long*>(&lmask[t]), loc);
  }
  __syncthreads();

  // ---- greedy on wave 0, 64 nodes of the order at a time.  A block's inputs
  // (its nodes, their in-block masks, edge flags and adjacency rows) do not
  // depend on what earlier blocks chose, so block k+1's are read from LDS
  // while block k decides; only the chosen set is read on the sequential path.
  if (wv == 0) {
    constexpr int kPW = 4;  // adjacency words held in registers (256 nodes)
    auto fetch = [&](int base, int& v, uint64_t& local, bool& he, uint64_t* av) {
      const int t = base + ln;
      v = -1;
      local = 0ull;
      he = false;
      if (t < M) {
        const int cand = order[t];
        if (cand >= 0) v = cand;  // NaN keys never chosen
        local = lmask[t];
      }
      if (v >= 0) {
        he = has_edge[v] != 0;
#pragma unroll
        for (int w = 0; w < kPW; ++w) av[w] = w < nw ? adj[v][w] : 0ull;
      }
    };
    int nv;
    uint64_t nlocal, nav[kPW];
    bool nhe;
    fetch(0, nv, nlocal, nhe, nav);
    for (int base = 0; base < M; base += 64) {
      const int v = nv;
      const uint64_t local = nlocal;  // earlier neighbours in this block (lane bits)
      const bool he = nhe;
      uint64_t av[kPW];
#pragma unroll
      for (int w = 0; w < kPW; ++w) av[w] = nav[w];
      if (base + 64 < M) fetch(base + 64, nv, nlocal, nhe, nav);
      uint64_t sel;
      if (__ballot(v >= 0 && he) == 0ull) {
        sel = __ballot(v >= 0);  // no node of this block has an edge: all chosen
      } else {
        // blocked by a node chosen in an earlier block
        bool blocked = false;
        if (v >= 0) {
#pragma unroll
          for (int w = 0; w < kPW; ++w) blocked |= (av[w] & chosen[w]) != 0ull;
          for (int w = kPW; w < nw; ++w) blocked |= (adj[v][w] & chosen[w]) != 0ull;
        }
        const uint64_t cand = __ballot(v >= 0 && !blocked);
        if (__ballot(local != 0ull) == 0ull) {
          sel = cand;  // no conflicts inside the block
        } else {
          // in rounds: a candidate with a chosen earlier in-block neighbour
          // is out at once; one whose earlier in-block neighbours have all
          // decided, none chosen, is chosen.  The lowest undecided candidate
          // always decides, and each decision is the one the node-by-node
          // scan makes.
          sel = 0ull;
          uint64_t open = cand;
          while (open) {
            const bool mine = (open >> ln) & 1ull;
            const bool out = mine && (local & sel) != 0ull;
            const bool pick = mine && !out && (local & open) == 0ull;
            sel |= __ballot(pick);
            open &= ~__ballot(pick || out);
          }
        }
      }
      if ((sel >> ln) & 1ull)
        atomicOr(reinterpret_cast<unsigned long long*>(&chosen[v >> 6]), 1ull << (v & 63));
    }
  }
  __syncthreads();
  int cnt = 0;
  for (int r = tid; r < M; r += NT) {
    const int c = static_cast<int>((chosen[r >> 6] >> (r & 63)) & 1ull) |
                  (P.pre_unmask && conf[lo + r] == 1.0f);  // pre-unmask
    commit[lo + r] = static_cast<uint8_t>(c);
    cnt += c;
  }
  cnt = dlm::block_sum<NT>(cnt, shi);
  if (tid == 0) n_commit[b] = cnt;
}

// The fused step's DAPD part, on NT-thread workgroups: `waves` waves of the
// workgroup each score one block of kSymRows rows of sequence b (blocks
// waves*wg .. of the sequence's `blocks` blocks; dapd_sym_rows), writing each
// row's commit as an edgeless graph has it; the workgroup then adds its
// tally to the sequence's counter, which the launch before zeroed.  The
// workgroup whose count completes the sequence holds the totals and goes on.
// Without an edge, a bad position, an over-long sequence or the late stage,
// the commits written are the greedy's (every node whose key is not NaN, and
// the pre-unmasked rows), so it only writes n_commit.  Otherwise it runs the
// greedy, which rewrites every commit.  The outputs are those of k_dapd_sym
// then k_dapd_select.
template <int NT>
__device__ __forceinline__ void dapd_scores_select(int b, int wg, int waves, int blocks,
    const int32_t* __restrict__ seq_offsets, const int32_t* __restrict__ masked_pos, int64_t S,
    int m_max, const float* __restrict__ conf, float tau, const char* __restrict__ ws, Layout L,
    uint8_t* __restrict__ commit, int32_t* __restrict__ n_commit, Policy P, SelSmem<NT>& sm) {
  static_assert(kSymNT == DLM_WAVE && NT >= DLM_WAVE, "a block of rows is one wave's");
  const int wv = threadIdx.x / DLM_WAVE, rb = wg * waves + wv;
  if (threadIdx.x == 0) sm.last = 0;
  __syncthreads();
  const bool scores = wv < waves && rb < blocks;
  uint64_t t = 0;
  if (scores) {
    t = dapd_sym_rows(b, rb, seq_offsets, masked_pos, S, m_max, conf, tau, ws, L, nullptr,
                      nullptr, nullptr, P, commit);
    t += dlm::xor_lane64<16>(t);  // the teams' lane 0
    t += dlm::xor_lane64<32>(t);
    t += kTallyWG;
  }
  // count in: the workgroup's tally in one atomic, after one agent-scope
  // release.  With several scoring waves, each first waits until its stores
  // are complete, and the workgroup barrier orders them before wave 0's
  // release (one release and one atomic per workgroup, not per wave: on the
  // 8-sequence shape the per-wave releases cost 4.6 us).
  unsigned long long* ctr = reinterpret_cast<unsigned long long*>(const_cast<char*>(ws) + L.tally) + b;
  if (waves > 1) {
    __builtin_amdgcn_s_waitcnt(0);
    if (threadIdx.x % DLM_WAVE == 0) sm.part[wv] = t;
    __syncthreads();
    if (wv == 0) {
      t = 0;
#pragma unroll
      for (int w = 0; w < NT / DLM_WAVE; ++w) t += w < waves ? sm.part[w] : 0ull;
    }
  }
  if (wv == 0 && t != 0ull) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");  // the rows, before counting in
    if (threadIdx.x == 0) {
      const uint64_t tot = atomicAdd(ctr, static_cast<unsigned long long>(t)) + t;
      if ((tot & 0xffffull) == static_cast<uint64_t>(blocks)) {  // one workgroup per sequence
        sm.tally = tot;
        sm.last = 1;
      }
    }
  }
  __syncthreads();
  if (!sm.last) return;  // uniform over the workgroup
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // the other workgroups' rows
  const uint64_t tot = sm.tally;
  // no edge, bad position or over-long sequence, and not the late stage (no
  // trip to memory for the stage test when there is no stage policy)
  if (tot < kTallyEdge &&
      (P.gen_len == nullptr || !late_stage(P, b, seq_offsets[b + 1] - seq_offsets[b]))) {
    if (threadIdx.x == 0) {
      n_commit[b] = static_cast<int32_t>((tot >> 16) & 0xffffull);
      if (P.stage) P.stage[b] = 0;
    }
    return;
  }
  dapd_select_seq<NT>(b, masked_pos, S, seq_offsets, m_max, ws, L, conf, commit, n_commit,
                      nullptr, nullptr, nullptr, P, sm);
}

// The fused step's DAPD part for sequences of at most 64 rows (m_max <= 64):
// one 256-thread workgroup scores every row of sequence b and decides it, so
// the graph passes through LDS, with no workspace round trip and no tally.
// Rows take 4-lane teams (16 rows per wave); lane tl of a team takes
// columns 16tl .. 16tl+15 with the loads, masks and fixed-order fp64 sum of
// dapd_sym_rows.  There the other twelve lanes of a 16-lane team hold
// columns >= 64 >= M and add exactly +0.0, so the degrees, keys and
// adjacency words are bitwise the same, and so is the decision
// (dapd_decide_wave, as in the selection call).  Over-long sequences and the
// late stage go to dapd_select_seq, which reads no graph for them.
template <int NT>
__device__ __forceinline__ void dapd_small_select(int b, const int32_t* __restrict__ seq_offsets,
    const int32_t* __restrict__ masked_pos, int64_t S, int m_max, const float* __restrict__ conf,
    float tau, const char* __restrict__ ws, Layout L, uint8_t* __restrict__ commit,
    int32_t* __restrict__ n_commit, Policy P, SelSmem<NT>& sm) {
  constexpr int kSmallTeam = 4, kRowsPerWave = DLM_WAVE / kSmallTeam;
  static_assert(NT / DLM_WAVE * kRowsPerWave == DLM_WAVE, "one row per team, 64 rows");
  const int lo = seq_offsets[b], M = seq_offsets[b + 1] - lo;
  if (M > m_max || M < 0 || late_stage(P, b, M)) {  // uniform over the workgroup
    dapd_select_seq<NT>(b, masked_pos, S, seq_offsets, m_max, ws, L, conf, commit, n_commit,
                        nullptr, nullptr, nullptr, P, sm);
    return;
  }
  const int wv = threadIdx.x / DLM_WAVE, ln = threadIdx.x % DLM_WAVE;
  const int tl = ln % kSmallTeam, i = wv * kRowsPerWave + ln / kSmallTeam;
  if (i < M) {  // whole teams
    const int pos_i = masked_pos[lo + i];
    const float conf_i = conf[lo + i];
    const float* A =
        reinterpret_cast<const float*>(ws + L.a) + static_cast<int64_t>(b) * m_max * L.ld;
    const int j0 = 16 * tl;
    float va[16], vt[16];
    const float4* rp = reinterpret_cast<const float4*>(A + static_cast<int64_t>(i) * L.ld +
                                                       min(j0, L.ld - 16));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 f = rp[q];
      va[4 * q] = f.x;
      va[4 * q + 1] = f.y;
      va[4 * q + 2] = f.z;
      va[4 * q + 3] = f.w;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) vt[e] = A[static_cast<int64_t>(min(j0 + e, M - 1)) * L.ld + i];
    const int lim = M - j0, di = i - j0;
    uint32_t valid = lim >= 16 ? 0xffffu : (lim <= 0 ? 0u : (1u << lim) - 1u);
    if (di >= 0 && di < 16) valid &= ~(1u << di);
    double dsum = 0.0;
    uint32_t gt = 0u;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float sv = 0.5f * (va[e] + vt[e]);
      gt |= static_cast<uint32_t>(sv > tau) << e;
      dsum += static_cast<double>(((valid >> e) & 1u) ? sv : 0.0f);
    }
    const uint32_t mine = gt & valid;
    reinterpret_cast<uint16_t*>(&sm.adj[i][0])[tl] = static_cast<uint16_t>(mine);
    dsum += dlm::xor_val<2>(dsum);
    dsum += dlm::xor_val<1>(dsum);
    uint32_t anyb = mine != 0u ? 1u : 0u;
    anyb |= dlm::xor_val<2>(anyb);
    anyb |= dlm::xor_val<1>(anyb);
    if (tl == 0) {
      const float kk = static_cast<float>(dsum) * conf_i;
      const uint64_t hi = (kk != kk) ? 0xffffffffull : static_cast<uint64_t>(dlm::desc_bits(kk));
      sm.keys[i] = (hi << 32) | static_cast<uint32_t>(i);
      sm.has_edge[i] = static_cast<uint8_t>(anyb | (static_cast<uint32_t>(pos_i < 0 || pos_i >= S) << 1));
    }
  }
  __syncthreads();
  if (wv != 0) return;
  const int r = ln < M ? ln : 0;
  dapd_decide_wave(b, lo, M, m_max, sm.keys[r], sm.has_edge[r], sm.adj[r][0], conf, commit,
                   n_commit, nullptr, nullptr, nullptr, P);
}

}  // namespace
