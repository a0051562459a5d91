// dapd.hip — dlm_dapd_select: DAPD dependency graph and Welsh-Powell-ordered
// independent set (DAPD paper note: overall framework; key design 1
// (s_ij = (a_ij + a_ji)/2, edge iff s_ij > tau); key design 2 (proxy degree,
// order by degree x confidence, maximal independent set)).
//
// Two kernels:
//  k_dapd_avg   grid-wide, HBM-bound.  Streams only the masked x masked
//               sub-blocks of the n_lh attention maps (fp32 accumulation) and
//               writes a and its transpose to the workspace.  A workgroup owns a
//               tile of 8 rows x 64 columns; its 4 waves take every 4th map and
//               are summed in LDS in a fixed order.  The 8-row tile makes the
//               transposed writes 32-byte runs.
//  k_dapd_select one workgroup (1024 threads) per sequence: s = (a + aT)/2
//               (computed once per unordered pair value, so bit-symmetric),
//               adjacency bitset in LDS, fp64 proxy degree, key, bitonic sort,
//               and the sequential greedy on one wave with the chosen-set
//               bitset spread over its lanes.
#include <math.h>

#include "dlm_device.h"

namespace {

constexpr int kAvgNT = 256;  // 4 waves = 4 map groups
constexpr int kTileRows = 8;
constexpr int kTileChunks = 8;  // 8 chunks of 8 columns = 64 columns
constexpr int kSelNT = 1024;
constexpr int kMaxM = DLM_MAX_SEQ_ROWS;
constexpr int kWords = kMaxM / 64;

template <bool BF16>
__device__ __forceinline__ float ld1(const void* base, int64_t idx) {
  if constexpr (BF16) return dlm::bf16_at(static_cast<const uint16_t*>(base), idx);
  return static_cast<const float*>(base)[idx];
}

template <bool BF16>
__global__ __launch_bounds__(kAvgNT) void k_dapd_avg(const void* __restrict__ attn, int n_lh,
                                                     int64_t S, int64_t batch_stride,
                                                     const int32_t* __restrict__ masked_pos,
                                                     const int32_t* __restrict__ seq_offsets,
                                                     int m_max, int n_tc, int vec_ok,
                                                     float* __restrict__ ws_a,
                                                     float* __restrict__ ws_at) {
  __shared__ float red[4][64][9];
  const int b = blockIdx.y;
  const int lo = seq_offsets[b], M = seq_offsets[b + 1] - lo;
  if (M > m_max || M <= 0) return;
  const int ti = blockIdx.x / n_tc, tc = blockIdx.x % n_tc;
  const int i0 = ti * kTileRows, c0 = tc * kTileChunks;
  if (i0 >= M || c0 * 8 >= M) return;  // whole workgroup idle (uniform)
  const int wv = threadIdx.x / DLM_WAVE, ln = threadIdx.x % DLM_WAVE;
  const int i = i0 + ln / kTileChunks, c = c0 + ln % kTileChunks;
  const int j0 = c * 8;
  const bool row_ok = i < M;
  const int* pos = masked_pos + lo;

  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.f;

  if (row_ok && j0 < M) {
    const int64_t prow = static_cast<int64_t>(pos[i]) * S;
    int pj[8];
    bool contig = vec_ok && (j0 + 8 <= M);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      pj[k] = (j0 + k < M) ? pos[j0 + k] : -1;
      contig = contig && (pj[k] == pj[0] + k);
    }
    contig = contig && (pj[0] % (BF16 ? 8 : 4) == 0);
    const char* base = static_cast<const char*>(attn) +
                       static_cast<int64_t>(b) * batch_stride * (BF16 ? 2 : 4);
    const int64_t map_stride = S * S;
    if (contig) {
      constexpr int UNR = 4;
      int lh = wv;
      for (; lh + 4 * (UNR - 1) < n_lh; lh += 4 * UNR) {
        uint4 q[UNR][BF16 ? 1 : 2];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          const int64_t e = static_cast<int64_t>(lh + 4 * u) * map_stride + prow + pj[0];
          if constexpr (BF16) {
            q[u][0] = *reinterpret_cast<const uint4*>(base + e * 2);
          } else {
            q[u][0] = *reinterpret_cast<const uint4*>(base + e * 4);
            q[u][1] = *reinterpret_cast<const uint4*>(base + e * 4 + 16);
          }
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          if constexpr (BF16) {
            acc[0] += dlm::bf16_lo(q[u][0].x);
            acc[1] += dlm::bf16_hi(q[u][0].x);
            acc[2] += dlm::bf16_lo(q[u][0].y);
            acc[3] += dlm::bf16_hi(q[u][0].y);
            acc[4] += dlm::bf16_lo(q[u][0].z);
            acc[5] += dlm::bf16_hi(q[u][0].z);
            acc[6] += dlm::bf16_lo(q[u][0].w);
            acc[7] += dlm::bf16_hi(q[u][0].w);
          } else {
            acc[0] += __uint_as_float(q[u][0].x);
            acc[1] += __uint_as_float(q[u][0].y);
            acc[2] += __uint_as_float(q[u][0].z);
            acc[3] += __uint_as_float(q[u][0].w);
            acc[4] += __uint_as_float(q[u][1].x);
            acc[5] += __uint_as_float(q[u][1].y);
            acc[6] += __uint_as_float(q[u][1].z);
            acc[7] += __uint_as_float(q[u][1].w);
          }
        }
      }
      for (; lh < n_lh; lh += 4) {
        const int64_t e = static_cast<int64_t>(lh) * map_stride + prow + pj[0];
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] += ld1<BF16>(base, e + k);
      }
    } else {
      for (int lh = wv; lh < n_lh; lh += 4) {
        const int64_t e = static_cast<int64_t>(lh) * map_stride + prow;
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (pj[k] >= 0) acc[k] += ld1<BF16>(base, e + pj[k]);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) red[wv][ln][k] = acc[k];
  __syncthreads();
  if (wv == 0 && row_ok && j0 < M) {
    const float fn = static_cast<float>(n_lh);
    float* arow = ws_a + (static_cast<int64_t>(b) * m_max + i) * m_max;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int j = j0 + k;
      if (j < M) {
        const float s = ((red[0][ln][k] + red[1][ln][k]) + red[2][ln][k]) + red[3][ln][k];
        const float a = s / fn;
        arow[j] = a;
        ws_at[(static_cast<int64_t>(b) * m_max + j) * m_max + i] = a;
      }
    }
  }
}

__device__ __forceinline__ uint32_t desc_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~asc;
}

__global__ __launch_bounds__(kSelNT) void k_dapd_select(
    const int32_t* __restrict__ seq_offsets, int m_max, const float* __restrict__ conf,
    float tau, const float* __restrict__ ws_a, const float* __restrict__ ws_at,
    uint8_t* __restrict__ commit, int32_t* __restrict__ n_commit, float* __restrict__ degree,
    float* __restrict__ sym, float* __restrict__ key_out) {
  __shared__ uint64_t adj[kMaxM][kWords];  // 128 KiB
  __shared__ uint64_t keys[kMaxM];
  __shared__ uint64_t chosen[kWords];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int wv = tid / DLM_WAVE, ln = tid % DLM_WAVE;
  constexpr int NW = kSelNT / DLM_WAVE;
  const int lo = seq_offsets[b], M = seq_offsets[b + 1] - lo;
  const int64_t sbase = static_cast<int64_t>(b) * m_max * m_max;

  if (M > m_max || M < 0) {
    for (int r = tid; r < M; r += kSelNT) {
      commit[lo + r] = 0;
      if (degree) degree[lo + r] = NAN;
      if (key_out) key_out[lo + r] = NAN;
    }
    if (sym)
      for (int64_t e = tid; e < static_cast<int64_t>(m_max) * m_max; e += kSelNT)
        sym[sbase + e] = NAN;
    if (tid == 0) n_commit[b] = -1;
    return;
  }
  const int nw = (M + 63) / 64;       // adjacency words in use
  const int wm = (m_max + 63) / 64;   // words spanned by a sym row

  // phase 1: s, adjacency words, proxy degree, key.  Wave w owns rows w, w+16, ...
  for (int i = wv; i < m_max; i += NW) {
    if (i >= M) {  // pad rows of the optional sym output
      if (sym)
        for (int j = ln; j < m_max; j += DLM_WAVE) sym[sbase + static_cast<int64_t>(i) * m_max + j] = NAN;
      continue;
    }
    const float* ar = ws_a + sbase + static_cast<int64_t>(i) * m_max;
    const float* tr = ws_at + sbase + static_cast<int64_t>(i) * m_max;
    double dsum = 0.0;
    for (int w = 0; w < wm; ++w) {
      const int j = w * 64 + ln;
      bool edge = false;
      float s = NAN;
      if (j < M) {
        s = 0.5f * (ar[j] + tr[j]);
        if (j != i) {
          dsum += static_cast<double>(s);
          edge = s > tau;
        }
      }
      if (sym && j < m_max) sym[sbase + static_cast<int64_t>(i) * m_max + j] = s;
      if (w < nw) {  // w is wave-uniform
        const uint64_t bits = __ballot(edge);
        if (ln == 0) adj[i][w] = bits;
      }
    }
    dsum = dlm::wave_sum(dsum);
    if (ln == 0) {
      const float d = static_cast<float>(dsum);
      const float kk = d * conf[lo + i];
      if (degree) degree[lo + i] = d;
      if (key_out) key_out[lo + i] = kk;
      const uint64_t hi = (kk != kk) ? 0xffffffffull : static_cast<uint64_t>(desc_bits(kk));
      // NaN keys sort last; every finite key maps below 0xffffffff
      keys[i] = (hi << 32) | static_cast<uint32_t>(i);
    }
  }
  int n2 = 1;
  while (n2 < M) n2 <<= 1;
  for (int i = M + tid; i < n2; i += kSelNT) keys[i] = ~0ull;
  if (tid < kWords) chosen[tid] = 0ull;
  __syncthreads();

  // phase 2: order by (key desc, position asc)
  for (int k = 2; k <= n2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int t = tid; t < n2 / 2; t += kSelNT) {
        const int i = 2 * j * (t / j) + (t % j);
        const int p = i + j;
        const bool up = (i & k) == 0;
        const uint64_t x = keys[i], y = keys[p];
        if ((x > y) == up) {
          keys[i] = y;
          keys[p] = x;
        }
      }
      __syncthreads();
    }
  }

  // phase 3: greedy on wave 0; lane w < nw holds word w of the excluded set
  if (wv == 0) {
    uint64_t excl = 0ull, mine = 0ull;
    for (int t = 0; t < M; ++t) {
      const uint64_t kv = keys[t];
      if ((kv >> 32) == 0xffffffffull) break;  // NaN keys: never chosen
      const int v = static_cast<int>(kv & 0xffffffffu);
      const uint64_t word = __shfl(excl, v >> 6, DLM_WAVE);
      if (((word >> (v & 63)) & 1ull) == 0ull) {
        if (ln < nw) excl |= adj[v][ln];
        if (ln == (v >> 6)) mine |= 1ull << (v & 63);
      }
    }
    if (ln < kWords) chosen[ln] = mine;
  }
  __syncthreads();
  int cnt = 0;
  for (int r = tid; r < M; r += kSelNT) {
    const int c = static_cast<int>((chosen[r >> 6] >> (r & 63)) & 1ull);
    commit[lo + r] = static_cast<uint8_t>(c);
    cnt += c;
  }
  __shared__ int shi[NW];
  cnt = dlm::block_sum<kSelNT>(cnt, shi);
  if (tid == 0) n_commit[b] = cnt;
}

}  // namespace

extern "C" size_t dlm_dapd_workspace_bytes(int32_t n_seq, int32_t m_max) {
  if (n_seq <= 0 || m_max <= 0 || m_max > DLM_MAX_SEQ_ROWS) return 0;
  return static_cast<size_t>(2) * static_cast<size_t>(n_seq) * static_cast<size_t>(m_max) *
         static_cast<size_t>(m_max) * sizeof(float);
}

extern "C" int dlm_dapd_select(const void* attn, int dtype, int32_t n_lh, int64_t S,
                               int64_t batch_stride, const int32_t* masked_pos,
                               const int32_t* seq_offsets, int32_t n_seq, int32_t m_max,
                               const float* conf, float tau, uint8_t* commit,
                               int32_t* n_commit, float* degree, float* sym, float* key,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (!attn || !masked_pos || !seq_offsets || !conf || !commit || !n_commit || !workspace)
    return DLM_ERR_ARG;
  if (n_lh <= 0 || S <= 0 || n_seq <= 0 || m_max <= 0 || tau != tau) return DLM_ERR_ARG;
  if (dtype != DLM_BF16 && dtype != DLM_F32) return DLM_ERR_UNSUPPORTED;
  if (m_max > DLM_MAX_SEQ_ROWS || S > 2147483647LL) return DLM_ERR_UNSUPPORTED;
  const int64_t maps = static_cast<int64_t>(n_lh) * S * S;
  if (n_seq > 1 && batch_stride < maps) return DLM_ERR_ARG;
  const int es = dtype == DLM_BF16 ? 2 : 4;
  const uintptr_t ab = reinterpret_cast<uintptr_t>(attn);
  if (ab % es) return DLM_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(workspace) % 16) return DLM_ERR_ARG;
  if (workspace_bytes < dlm_dapd_workspace_bytes(n_seq, m_max)) return DLM_ERR_ARG;
  const int vec_ok = (ab % 16 == 0) && (S % 8 == 0) && (batch_stride % 8 == 0);
  float* ws_a = static_cast<float*>(workspace);
  float* ws_at = ws_a + static_cast<size_t>(n_seq) * m_max * m_max;
  const int n_ti = (m_max + kTileRows - 1) / kTileRows;
  const int n_tc = (m_max + 8 * kTileChunks - 1) / (8 * kTileChunks);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(n_ti * n_tc, n_seq);
  if (dtype == DLM_BF16)
    hipLaunchKernelGGL(k_dapd_avg<true>, grid, dim3(kAvgNT), 0, s, attn, n_lh, S, batch_stride,
                       masked_pos, seq_offsets, m_max, n_tc, vec_ok, ws_a, ws_at);
  else
    hipLaunchKernelGGL(k_dapd_avg<false>, grid, dim3(kAvgNT), 0, s, attn, n_lh, S, batch_stride,
                       masked_pos, seq_offsets, m_max, n_tc, vec_ok, ws_a, ws_at);
  DLM_CHECK_LAUNCH();
  hipLaunchKernelGGL(k_dapd_select, dim3(n_seq), dim3(kSelNT), 0, s, seq_offsets, m_max, conf,
                     tau, ws_a, ws_at, commit, n_commit, degree, sym, key);
  DLM_CHECK_LAUNCH();
  return DLM_OK;
}
