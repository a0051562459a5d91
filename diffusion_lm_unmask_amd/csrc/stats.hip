// stats.hip — dlm_step_stats: one streaming pass over each logits row (and
// the previous step's row) computing confidence, argmax, entropy, KL and
// log-normaliser.
//
// Definitions: DepCap summary, Methodology (H_k = H(p_curr^k),
// I_k = KL(p_curr^k || p_prev^k), c_i = max_v p_i(v)); Fast-dLLM review,
// Method (max-softmax confidence and argmax commit).
//
// Design (gfx950):
//  * one workgroup per row; each lane owns 16-byte chunks tid, tid+NT, ...
//    so every wave load is a contiguous 1 KiB (global_load_dwordx4);
//  * a lane processes U chunks per segment: segment maxima first, then one
//    exp2 per element, t = x*log2(e) - h, with the lane reference
//    h = ceil(max*log2(e)) an integer, so a rescale of the running sums when
//    the max grows is an exact power of two (ldexp) and adds no rounding;
//  * sums are fp32 per segment and per lane; lanes are combined exactly
//    (ldexp) in fp64 relative to the row's integer reference, and the
//    fractional offset between that reference and the row max is applied
//    once, in fp64, when the statistics are formed;
//  * the argmax costs one compare per chunk in the hot loop: a lane records
//    the first chunk where its running max strictly grew; only lanes whose
//    max equals the row max re-read that one chunk to find the element;
//  * any non-finite total (NaN/inf entries, -inf logits, empty rows) sends
//    the row to an element-wise path that applies the definitions'
//    conventions exactly (0 log 0 = 0, q = 0 with p > 0 gives KL = +inf).
#include "dlm_device.h"

namespace {

constexpr float kL2E = 1.4426950408889634f;  // log2(e) in fp32
constexpr double kL2Ed = static_cast<double>(kL2E);  // the same value, widened
constexpr double kLN2 = 0.6931471805599453;
constexpr float kLow = -1e30f;  // running-max sentinel: no finite data seen yet

__device__ __forceinline__ float ex2(float t) { return __builtin_amdgcn_exp2f(t); }

template <bool BF16>
__device__ __forceinline__ void unpack(const uint4 q, float* x) {
  if constexpr (BF16) {
    x[0] = dlm::bf16_lo(q.x);
    x[1] = dlm::bf16_hi(q.x);
    x[2] = dlm::bf16_lo(q.y);
    x[3] = dlm::bf16_hi(q.y);
    x[4] = dlm::bf16_lo(q.z);
    x[5] = dlm::bf16_hi(q.z);
    x[6] = dlm::bf16_lo(q.w);
    x[7] = dlm::bf16_hi(q.w);
  } else {
    x[0] = __uint_as_float(q.x);
    x[1] = __uint_as_float(q.y);
    x[2] = __uint_as_float(q.z);
    x[3] = __uint_as_float(q.w);
  }
}

template <bool BF16>
__device__ __forceinline__ float load_elem(const char* row, int64_t v) {
  if constexpr (BF16) return dlm::bf16_at(reinterpret_cast<const uint16_t*>(row), v);
  return reinterpret_cast<const float*>(row)[v];
}

// Per-lane running state for the current (cur) and previous (prv) rows.
struct CurState {
  float m, h, Z, A, B;  // max, ceil(m*log2e), sum e, sum e*t (log2 units), sum e*(x-y)
  int64_t best;         // first element index of the chunk holding the lane max
  int bestw;            // width of that chunk (VEC, or 1 for a tail element)
};
struct PrvState {
  float m, h, Z;
};

// Fold a block of N values (x: current, y: previous) into the lane state.
// `valid` masks whole sub-blocks of W values (chunks); start[u] is the
// element index of sub-block u (for the argmax record).
template <int NSUB, int W, bool PREV>
__device__ __forceinline__ void fold(CurState& c, PrvState& p, const float (*x)[W],
                                     const float (*y)[W], const bool* valid,
                                     const int64_t* start) {
  // segment maxima and the first-strict-increase chunk record
  float mr = c.m;
#pragma unroll
  for (int u = 0; u < NSUB; ++u) {
    float cm = x[u][0];
#pragma unroll
    for (int k = 1; k < W; ++k) cm = fmaxf(cm, x[u][k]);
    if (valid[u]) {
      if (cm > mr) {
        c.best = start[u];
        c.bestw = W;
      }
      mr = fmaxf(mr, cm);
    }
  }
  {  // rescale running sums to the new integer reference (exact: a power of two)
    const float hn = ceilf(mr * kL2E);
    const float dh = c.h - hn;  // integer <= 0 (or a huge negative from the sentinel)
    const int di = static_cast<int>(fmaxf(dh, -256.f));
    c.A = ldexpf(fmaf(dh, c.Z, c.A), di);
    c.Z = ldexpf(c.Z, di);
    if constexpr (PREV) c.B = ldexpf(c.B, di);
    c.h = hn;
    c.m = mr;
  }
  float z = 0.f, a = 0.f, b = 0.f;
#pragma unroll
  for (int u = 0; u < NSUB; ++u) {
    if (!valid[u]) continue;
#pragma unroll
    for (int k = 0; k < W; ++k) {
      const float t = fmaf(x[u][k], kL2E, -c.h);
      const float e = ex2(t);
      z += e;
      a = fmaf(e, t, a);
      if constexpr (PREV) b = fmaf(e, x[u][k] - y[u][k], b);
    }
  }
  c.Z += z;
  c.A += a;
  if constexpr (PREV) {
    c.B += b;
    float mq = p.m;
#pragma unroll
    for (int u = 0; u < NSUB; ++u) {
      if (!valid[u]) continue;
#pragma unroll
      for (int k = 0; k < W; ++k) mq = fmaxf(mq, y[u][k]);
    }
    const float hn = ceilf(mq * kL2E);
    p.Z = ldexpf(p.Z, static_cast<int>(fmaxf(p.h - hn, -256.f)));
    p.h = hn;
    p.m = mq;
    float z2 = 0.f;
#pragma unroll
    for (int u = 0; u < NSUB; ++u) {
      if (!valid[u]) continue;
#pragma unroll
      for (int k = 0; k < W; ++k) z2 += ex2(fmaf(y[u][k], kL2E, -p.h));
    }
    p.Z += z2;
  }
}

// Sum four doubles over the workgroup in a fixed order.
template <int NT>
__device__ __forceinline__ void block_sum4(double& a, double& b, double& c, double& d,
                                           double (*sh)[NT / DLM_WAVE]) {
  constexpr int NW = NT / DLM_WAVE;
  a = dlm::wave_sum(a);
  b = dlm::wave_sum(b);
  c = dlm::wave_sum(c);
  d = dlm::wave_sum(d);
  const int w = threadIdx.x / DLM_WAVE, l = threadIdx.x % DLM_WAVE;
  __syncthreads();
  if (l == 0) {
    sh[0][w] = a;
    sh[1][w] = b;
    sh[2][w] = c;
    sh[3][w] = d;
  }
  __syncthreads();
  a = sh[0][0];
  b = sh[1][0];
  c = sh[2][0];
  d = sh[3][0];
#pragma unroll
  for (int i = 1; i < NW; ++i) {
    a += sh[0][i];
    b += sh[1][i];
    c += sh[2][i];
    d += sh[3][i];
  }
}

template <int NT>
struct Shared {
  float f[NT / DLM_WAVE];
  int i[NT / DLM_WAVE];
  double d[4][NT / DLM_WAVE];
  int flag;
};

// Element-wise path with the definitions' conventions applied term by term.
template <int NT, bool BF16, bool PREV>
__device__ void careful_row(const char* cur, const char* prv, int64_t V, Shared<NT>& sh,
                            int64_t r, float* conf, int32_t* argmax, float* ent, float* kl,
                            float* lse) {
  const int tid = threadIdx.x;
  // pass 1: maxima over non-NaN entries, lowest index, NaN presence
  float m = -INFINITY, m2 = -INFINITY;
  int idx = INT32_MAX, nan1 = 0, nan2 = 0;
  for (int64_t v = tid; v < V; v += NT) {
    const float x = load_elem<BF16>(cur, v);
    if (x != x) {
      nan1 = 1;
    } else if (idx == INT32_MAX || x > m) {
      m = x;
      idx = static_cast<int>(v);
    }
    if constexpr (PREV) {
      const float y = load_elem<BF16>(prv, v);
      if (y != y) nan2 = 1;
      else m2 = fmaxf(m2, y);
    }
  }
  const float M = dlm::block_max<NT>(m, sh.f);
  const int cidx = (idx != INT32_MAX && m == M) ? idx : INT32_MAX;
  int yhat = dlm::block_min_i<NT>(cidx, sh.i);
  if (yhat == INT32_MAX) yhat = 0;
  const int any_nan1 = dlm::block_max_i<NT>(nan1, sh.i);
  float M2 = 0.f;
  int any_nan2 = 0;
  if constexpr (PREV) {
    M2 = dlm::block_max<NT>(m2, sh.f);
    any_nan2 = dlm::block_max_i<NT>(nan2, sh.i);
  }
  const bool ok1 = !any_nan1 && isfinite(M);
  const bool ok2 = !any_nan2 && isfinite(M2);
  if (!ok1) {
    if (tid == 0) {
      argmax[r] = yhat;
      conf[r] = ent[r] = lse[r] = NAN;
      if constexpr (PREV) kl[r] = NAN;
    }
    return;
  }
  // pass 2: sums, skipping zero-probability terms
  float z = 0.f, a = 0.f, b = 0.f, z2 = 0.f;
  int inf_kl = 0;
  for (int64_t v = tid; v < V; v += NT) {
    const float x = load_elem<BF16>(cur, v);
    float y = 0.f;
    if constexpr (PREV) {
      y = load_elem<BF16>(prv, v);
      if (ok2 && y != -INFINITY) z2 += expf(y - M2);
    }
    if (x == -INFINITY) continue;
    const float d = x - M;
    const float e = expf(d);
    z += e;
    a = fmaf(e, d, a);
    if constexpr (PREV) {
      if (y == -INFINITY) inf_kl = 1;
      else b = fmaf(e, x - y, b);
    }
  }
  double Z = z, A = a, B = b, Z2 = z2;
  block_sum4<NT>(Z, A, B, Z2, sh.d);
  if constexpr (PREV) inf_kl = dlm::block_max_i<NT>(inf_kl, sh.i);
  if (tid == 0) {
    const double lz = log(Z);
    argmax[r] = yhat;
    lse[r] = static_cast<float>(static_cast<double>(M) + lz);
    conf[r] = static_cast<float>(1.0 / Z);
    ent[r] = static_cast<float>(lz - A / Z);
    if constexpr (PREV) {
      double k;
      if (!ok2) k = NAN;
      else if (inf_kl) k = INFINITY;
      else k = B / Z + (static_cast<double>(M2) - static_cast<double>(M)) + log(Z2) - lz;
      kl[r] = static_cast<float>(k);
    }
  }
}

template <int NT, bool BF16, bool PREV>
__global__ __launch_bounds__(NT) void k_stats(const void* __restrict__ logits,
                                              const void* __restrict__ prev, int64_t V,
                                              int64_t ld, const int64_t* __restrict__ row_index,
                                              float* __restrict__ conf,
                                              int32_t* __restrict__ argmax,
                                              float* __restrict__ ent, float* __restrict__ kl,
                                              float* __restrict__ lse, int aligned) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int VEC = 16 / ES;          // elements per 16-byte chunk
  constexpr int U = BF16 ? 2 : 4;       // chunks per lane per segment
  __shared__ Shared<NT> sh;

  const int64_t r = blockIdx.x;
  const int64_t off = row_index[r] * ld;
  const char* cur = static_cast<const char*>(logits) + off * ES;
  const char* prv = PREV ? static_cast<const char*>(prev) + off * ES : nullptr;
  const int tid = threadIdx.x;

  if (!aligned) {
    careful_row<NT, BF16, PREV>(cur, prv, V, sh, r, conf, argmax, ent, kl, lse);
    return;
  }

  const uint4* cur4 = reinterpret_cast<const uint4*>(cur);
  const uint4* prv4 = reinterpret_cast<const uint4*>(prv);
  const int64_t nC = V / VEC;
  const int tail = static_cast<int>(V - nC * VEC);
  constexpr int64_t SEG = static_cast<int64_t>(U) * NT;
  const int64_t n_full = nC / SEG;

  CurState c{kLow, kLow * kL2E, 0.f, 0.f, 0.f, -1, VEC};  // h sentinel: integral
  PrvState p{kLow, kLow * kL2E, 0.f};
  bool allv[U];
#pragma unroll
  for (int u = 0; u < U; ++u) allv[u] = true;

  // software-pipelined full segments: loads of segment it+1 are issued
  // before segment it is folded
  uint4 qc[U], qp[U];
  if (n_full > 0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      qc[u] = cur4[u * NT + tid];
      if constexpr (PREV) qp[u] = prv4[u * NT + tid];
    }
  }
  for (int64_t it = 0; it < n_full; ++it) {
    float x[U][VEC], y[U][VEC];
    int64_t st[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      unpack<BF16>(qc[u], x[u]);
      if constexpr (PREV) unpack<BF16>(qp[u], y[u]);
      st[u] = (it * SEG + u * NT + tid) * VEC;
    }
    if (it + 1 < n_full) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t ch = (it + 1) * SEG + u * NT + tid;
        qc[u] = cur4[ch];
        if constexpr (PREV) qp[u] = prv4[ch];
      }
    }
    fold<U, VEC, PREV>(c, p, x, y, allv, st);
  }
  // last, partial segment
  if (n_full * SEG < nC) {
    float x[U][VEC], y[U][VEC];
    int64_t st[U];
    bool val[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t ch = n_full * SEG + u * NT + tid;
      val[u] = ch < nC;
      uint4 a = make_uint4(0u, 0u, 0u, 0u), b = a;
      if (val[u]) {
        a = cur4[ch];
        if constexpr (PREV) b = prv4[ch];
      }
      unpack<BF16>(a, x[u]);
      if constexpr (PREV) unpack<BF16>(b, y[u]);
      st[u] = ch * VEC;
    }
    fold<U, VEC, PREV>(c, p, x, y, val, st);
  }
  // scalar tail elements (vocab not a multiple of the chunk width)
  if (tid < tail) {
    const int64_t v = nC * VEC + tid;
    float x[1][1], y[1][1];
    x[0][0] = load_elem<BF16>(cur, v);
    y[0][0] = PREV ? load_elem<BF16>(prv, v) : 0.f;
    const bool val[1] = {true};
    const int64_t st[1] = {v};
    fold<1, 1, PREV>(c, p, x, y, val, st);
    if (c.best == v) c.bestw = 1;
  }

  // ---- combine lanes
  const float M = dlm::block_max<NT>(c.m, sh.f);
  float M2 = 0.f;
  if constexpr (PREV) M2 = dlm::block_max<NT>(p.m, sh.f);
  int cand = INT32_MAX;
  if (c.m == M && c.best >= 0) {
    if (c.bestw == 1) {
      cand = static_cast<int>(c.best);
    } else {
      float x[VEC];
      unpack<BF16>(cur4[c.best / VEC], x);
#pragma unroll
      for (int k = VEC - 1; k >= 0; --k)
        if (x[k] == M) cand = static_cast<int>(c.best + k);
    }
  }
  const int yhat = dlm::block_min_i<NT>(cand, sh.i);

  // Lane sums relative to the row's integer reference hM = ceil(M*log2e):
  // exact power-of-two scaling.  Sentinel lanes (no finite data) scale to 0.
  const float hM = ceilf(M * kL2E);
  const int di = static_cast<int>(fmaxf(c.h - hM, -1100.f));
  double Z = ldexp(static_cast<double>(c.Z), di);
  double A = ldexp(static_cast<double>(c.A) + static_cast<double>(c.h - hM) *
                                                 static_cast<double>(c.Z), di);
  double B = 0.0, Z2 = 0.0;
  float hM2 = 0.f;
  if constexpr (PREV) {
    B = ldexp(static_cast<double>(c.B), di);
    hM2 = ceilf(M2 * kL2E);
    Z2 = ldexp(static_cast<double>(p.Z), static_cast<int>(fmaxf(p.h - hM2, -1100.f)));
  }
  block_sum4<NT>(Z, A, B, Z2, sh.d);
  if (tid == 0) {
    bool ok = isfinite(Z) && Z > 0.0 && isfinite(A) && M > kLow && isfinite(M) && yhat >= 0 &&
              yhat != INT32_MAX;
    if constexpr (PREV)
      ok = ok && isfinite(B) && isfinite(Z2) && Z2 > 0.0 && M2 > kLow && isfinite(M2);
    sh.flag = ok;
    if (ok) {
      // Z_true = Z * 2^cM with cM = hM - M*log2e in [0, 1]: conf and lse need
      // it; entropy does not (it cancels); KL needs cM2 - cM.
      const double cM = static_cast<double>(hM) - static_cast<double>(M) * kL2Ed;
      const double lz = log(Z);
      argmax[r] = yhat;
      lse[r] = static_cast<float>(static_cast<double>(M) + lz + kLN2 * cM);
      conf[r] = static_cast<float>(exp2(-cM) / Z);
      ent[r] = static_cast<float>(lz - kLN2 * (A / Z));
      if constexpr (PREV) {
        const double cM2 = static_cast<double>(hM2) - static_cast<double>(M2) * kL2Ed;
        kl[r] = static_cast<float>(B / Z + (static_cast<double>(M2) - static_cast<double>(M)) +
                                   log(Z2 / Z) + kLN2 * (cM2 - cM));
      }
    }
  }
  __syncthreads();
  if (!sh.flag) careful_row<NT, BF16, PREV>(cur, prv, V, sh, r, conf, argmax, ent, kl, lse);
}

template <int NT, bool BF16>
hipError_t launch_nt(const void* logits, const void* prev, int64_t V, int64_t ld,
                     const int64_t* row_index, int64_t n_rows, float* conf, int32_t* argmax,
                     float* ent, float* kl, float* lse, int aligned, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(n_rows));
  if (prev)
    hipLaunchKernelGGL((k_stats<NT, BF16, true>), grid, dim3(NT), 0, s, logits, prev, V, ld,
                       row_index, conf, argmax, ent, kl, lse, aligned);
  else
    hipLaunchKernelGGL((k_stats<NT, BF16, false>), grid, dim3(NT), 0, s, logits, prev, V, ld,
                       row_index, conf, argmax, ent, kl, lse, aligned);
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch_dt(int nt, const void* logits, const void* prev, int64_t V, int64_t ld,
                     const int64_t* row_index, int64_t n_rows, float* conf, int32_t* argmax,
                     float* ent, float* kl, float* lse, int aligned, hipStream_t s) {
  switch (nt) {
    case 256:
      return launch_nt<256, BF16>(logits, prev, V, ld, row_index, n_rows, conf, argmax, ent,
                                  kl, lse, aligned, s);
    case 512:
      return launch_nt<512, BF16>(logits, prev, V, ld, row_index, n_rows, conf, argmax, ent,
                                  kl, lse, aligned, s);
    default:
      return launch_nt<1024, BF16>(logits, prev, V, ld, row_index, n_rows, conf, argmax, ent,
                                   kl, lse, aligned, s);
  }
}

// Threads per row: enough waves in flight to cover HBM latency.  Few rows
// (one step of one sequence) get the widest workgroups; many rows get
// narrower ones so several rows share a CU.
int threads_per_row(int64_t n_rows) {
  static int forced = -1;
  if (forced < 0) {
    const char* e = getenv("DLM_STATS_THREADS");
    const int v = e ? atoi(e) : 0;
    forced = (v == 256 || v == 512 || v == 1024) ? v : 0;
  }
  if (forced) return forced;
  if (n_rows >= 4096) return 256;
  if (n_rows >= 1024) return 512;
  return 1024;
}

}  // namespace

extern "C" int dlm_step_stats(const void* logits, const void* prev_logits, int dtype,
                              int64_t vocab, int64_t ld, const int64_t* row_index,
                              int64_t n_rows, float* conf, int32_t* argmax, float* entropy,
                              float* kl, float* lse, void* stream) {
  if (!logits || !row_index || !conf || !argmax || !entropy || !lse) return DLM_ERR_ARG;
  if ((prev_logits == nullptr) != (kl == nullptr)) return DLM_ERR_ARG;
  if (dtype != DLM_BF16 && dtype != DLM_F32) return DLM_ERR_UNSUPPORTED;
  if (vocab <= 0 || n_rows <= 0 || ld < vocab) return DLM_ERR_ARG;
  if (vocab > DLM_MAX_VOCAB || n_rows > 2147483647LL) return DLM_ERR_UNSUPPORTED;
  const int es = dtype == DLM_BF16 ? 2 : 4;
  const uintptr_t a = reinterpret_cast<uintptr_t>(logits);
  const uintptr_t b = reinterpret_cast<uintptr_t>(prev_logits);
  if (a % es || b % es) return DLM_ERR_ARG;
  const int aligned = (a % 16 == 0) && (b % 16 == 0) && ((ld * es) % 16 == 0);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int nt = threads_per_row(n_rows);
  hipError_t err;
  if (dtype == DLM_BF16)
    err = launch_dt<true>(nt, logits, prev_logits, vocab, ld, row_index, n_rows, conf, argmax,
                          entropy, kl, lse, aligned, s);
  else
    err = launch_dt<false>(nt, logits, prev_logits, vocab, ld, row_index, n_rows, conf, argmax,
                           entropy, kl, lse, aligned, s);
  return err == hipSuccess ? DLM_OK : DLM_ERR_HIP;
}
