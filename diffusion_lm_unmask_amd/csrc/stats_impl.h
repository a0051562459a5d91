// stats_impl.h — device code of dlm_step_stats: one streaming pass over each
// logits row (and the previous step's row) computing confidence, argmax,
// entropy, KL and log-normaliser.
//
// Definitions: DepCap summary, Methodology (H_k = H(p_curr^k),
// I_k = KL(p_curr^k || p_prev^k), c_i = max_v p_i(v)); Fast-dLLM review,
// Method (max-softmax confidence and argmax commit).
//
// Design (gfx950):
//  * one workgroup per row; each lane owns 16-byte chunks tid, tid+NT, ...
//    so every wave load is a contiguous 1 KiB (global_load_dwordx4);
//  * a lane processes U chunks per segment: segment maxima first, then one
//    exp2 per element, t = x*log2(e) - h, with the lane reference h an
//    integer (ceil(max*log2(e)) when it is set), so a rescale of the running
//    sums is an exact power of two (ldexp) and adds no rounding; the
//    reference trails the max and moves only once the max passes it by a
//    margin, so most chunks skip the rescale;
//  * the previous step's row is summed against the same reference, so KL
//    needs no second maximum: KL = ln 2 * (B/Z + log2(Z2/Z));
//  * sums are fp32 per segment and per lane; lanes are combined exactly
//    (ldexp) in fp64 relative to the row's integer reference, and the
//    fractional offset between that reference and the row max is applied
//    once, in fp64, when the statistics are formed;
//  * the argmax costs one compare and a register copy per chunk in the hot
//    loop: a lane keeps the raw bits of the first chunk where its running max
//    strictly grew, and finds the element in it after the stream, without a
//    second memory access;
//  * lanes are merged per wave on the DPP crossbar, waves through one LDS
//    record each and a single barrier;
//  * any non-finite total (NaN/inf entries, -inf logits, empty rows) sends
//    the row to an element-wise path that applies the definitions'
//    conventions exactly (0 log 0 = 0, q = 0 with p > 0 gives KL = +inf).
#pragma once
#include "dlm_device.h"

namespace {

constexpr float kL2E = 1.4426950408889634f;  // log2(e) in fp32
constexpr double kL2Ed = static_cast<double>(kL2E);  // the same value, widened
constexpr double kLN2 = 0.6931471805599453;
constexpr float kLow = -1e30f;  // running-max sentinel: no finite data seen yet

__device__ __forceinline__ float ex2(float t) { return __builtin_amdgcn_exp2f(t); }

// Tuning: 16-byte chunks per lane per segment (512-thread workgroups, and the
// 256-thread ones of very many rows), and whether row loads carry the
// non-temporal hint (streamed once, not worth caching).  Same-process A/B of
// back-to-back statistics calls: 2 chunks at 512 threads (256 rows: 25.0 us
// against 25.5 with 3 and 26.6 with 4; 2048 rows: even); 3 at 256 threads
// (4096 x 151936: 190.9 us against 196.0 with 2 and 192.1 with 4; 65536
// rows: 4846 against 4868 us).
#ifndef DLM_STATS_U_BF16
#define DLM_STATS_U_BF16 2
#endif
#ifndef DLM_STATS_U_BF16_256
#define DLM_STATS_U_BF16_256 3
#endif
#ifndef DLM_STATS_NT_LOADS
#define DLM_STATS_NT_LOADS 1
#endif
// Chunks per lane per segment for 768-thread workgroups.
#ifndef DLM_STATS_U_BF16_768
#define DLM_STATS_U_BF16_768 1
#endif
// Threads of a row's workgroup.  Many rows (from DLM_STATS_NT256_ROWS): 256,
// more workgroups per compute unit.  bf16 rows with a previous row, at most
// one per compute unit: 768 (12 waves, three per SIMD), whose extra waves
// overlap the fold's arithmetic (two exponentials per element pair) with the
// loads better when each compute unit streams a single row; same-process A/B,
// 256 x 126464 with prev: 21.9 against 22.5 us at 512 threads (and 832
// threads, which leave no partial segment at this vocabulary, lose to the
// uneven split of 13 waves over four SIMDs); without prev,
// or with two or more rows per compute unit, 512 stays ahead (256 rows
// without prev: 15.2 against 17.1 us).  Otherwise 512.  The statistics call
// and the fused step's statistics-only launch share this rule, so their
// results are bitwise equal.
#ifndef DLM_STATS_NT256_ROWS
#define DLM_STATS_NT256_ROWS 4096
#endif
__host__ __device__ constexpr int stats_threads(int64_t n_rows, bool prev, bool bf16, int cus) {
  return n_rows >= DLM_STATS_NT256_ROWS ? 256 : (prev && bf16 && n_rows <= cus) ? 768 : 512;
}
// bf16 chunks per lane per segment for a workgroup of NT threads.
template <int NT>
constexpr int stats_unroll() {
  return NT == 256 ? DLM_STATS_U_BF16_256 : NT == 768 ? DLM_STATS_U_BF16_768 : DLM_STATS_U_BF16;
}
// Whether a workgroup of NT threads keeps two segments in flight (the
// statistics block's PING form): bf16 rows outside the 768-thread shape.
#ifndef DLM_STATS_PING_768
#define DLM_STATS_PING_768 0
#endif
template <int NT, bool BF16>
constexpr bool stats_ping() {
  return BF16 && (NT != 768 || DLM_STATS_PING_768);
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load16(const uint4* p) {
#if DLM_STATS_NT_LOADS
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
#else
  return *p;
#endif
}

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

// Element k of a 16-byte chunk (k is a compile-time constant after unrolling).
template <bool BF16>
__device__ __forceinline__ float elem_of(const uint4 q, int k) {
  if constexpr (BF16) {
    const uint32_t w = (k >> 1) == 0 ? q.x : (k >> 1) == 1 ? q.y : (k >> 1) == 2 ? q.z : q.w;
    return (k & 1) ? dlm::bf16_hi(w) : dlm::bf16_lo(w);
  } else {
    return __uint_as_float(k == 0 ? q.x : k == 1 ? q.y : k == 2 ? q.z : q.w);
  }
}

// Per-lane running state.  Both rows' sums use the current row's integer
// reference h (at most ceil(m * log2 e), m the lane's running max of the
// current row): the previous row only needs sum 2^(t_y), t_y = y*log2e - h,
// and KL = ln 2 * (B/Z + log2(Z2/Z)) then involves no reference at all.  A
// previous row far above or below the current one overflows or underflows Z2
// and is sent to the element-wise path.
struct LaneState {
  float m, h;       // running max of the current row, integer reference
  float thr;        // the reference moves once the max passes this value
  float Z, A, B;    // sum e, sum e*t, sum e*(t - t_y) (log2 units)
  float Z2;         // sum 2^(t_y)
  int best;         // first element index of the chunk holding the lane max
  int bestw;        // width of that chunk (VEC, or 1 for a tail element)
  uint4 bq;         // raw bits of that chunk (VEC > 1)
};

// The reference trails the running max: it is moved to ceil(m * log2 e) only
// once the max exceeds it by more than kSlack (log2 units), so every term has
// t = x*log2e - h <= kSlack (2^t at most 2^kSlack: no overflow) while the
// rescale, which costs ten instructions, is skipped on almost every chunk.
constexpr float kSlack = 8.f;
constexpr float kLn2f = 0.69314718f;  // ln 2 in fp32

// Fold NSUB sub-blocks of W values into the lane state, in two parts.
// fold_head: the sub-blocks' maxima, the first-strict-increase chunk record
// (qc holds the raw chunks, unused for W == 1) and, once the max has passed
// the reference by more than kSlack, the exact power-of-two rescale of the
// running sums to a new integer reference.  fold_tail: the
// sums; the previous row's values come from yf (unpacked), else ys (one
// value per sub-block), else the raw chunks qp.  `valid` masks whole
// sub-blocks; start[u] is the element index of sub-block u.
template <int NSUB, int W, bool BF16, bool PREV>
__device__ __forceinline__ void fold_head(LaneState& c, const float (*x)[W], const uint4* qc,
                                          const bool* valid, const int* start) {
  float mr = c.m;
#pragma unroll
  for (int u = 0; u < NSUB; ++u) {
    if (!valid[u]) continue;
    float mn = mr;
#pragma unroll
    for (int k = 0; k < W; ++k) mn = fmaxf(mn, x[u][k]);
    if (mn > mr) {  // the running max grew strictly in this sub-block
      c.best = start[u];
      c.bestw = W;
      if constexpr (W > 1) c.bq = qc[u];
    }
    mr = mn;
  }
  c.m = mr;
  // Move the reference when the max has passed it by more than kSlack: an
  // exact power-of-two rescale of the running sums.  The wave takes the
  // branch together (a lane that does not need it rescales to its own
  // ceil(m * log2e), which is as exact).
  if (__builtin_amdgcn_ballot_w64(mr > c.thr) != 0) {
    const float hn = ceilf(mr * kL2E);
    const float dh = c.h - hn;  // integer <= 0 (or a huge negative from the sentinel)
    const int di = static_cast<int>(fmaxf(dh, -256.f));
    c.A = ldexpf(fmaf(dh, c.Z, c.A), di);
    c.Z = ldexpf(c.Z, di);
    if constexpr (PREV) {
      c.B = ldexpf(c.B, di);
      c.Z2 = ldexpf(c.Z2, di);
    }
    c.h = hn;
    c.thr = (hn + kSlack) * kLn2f;
  }
}
template <int NSUB, int W, bool BF16, bool PREV>
__device__ __forceinline__ void fold_tail(LaneState& c, const float (*x)[W],
                                          const float (*yf)[W], const uint4* qp,
                                          const float* ys, const bool* valid) {
  // sum e*(t - t_y) is taken as sum e*t - sum e*t_y per call: t_y is needed
  // for the previous row's exponential anyway, and equal rows give bitwise
  // equal sums (B = 0 exactly).  The sums start at -0.0, the identity of the
  // addition, so the first term needs no add.
  float z = -0.f, a = -0.f, ay = -0.f, z2 = -0.f;
#pragma unroll
  for (int u = 0; u < NSUB; ++u) {
    if (!valid[u]) continue;
#pragma unroll
    for (int k = 0; k < W; ++k) {
      const float t = fmaf(x[u][k], kL2E, -c.h);
      const float e = ex2(t);
      z += e;
      a = fmaf(e, t, a);
      if constexpr (PREV) {
        const float y = yf ? yf[u][k] : ys ? ys[u * W + k] : elem_of<BF16>(qp[u], k);
        const float ty = fmaf(y, kL2E, -c.h);
        ay = fmaf(e, ty, ay);
        z2 += ex2(ty);
      }
    }
  }
  c.Z += z;
  c.A += a;
  if constexpr (PREV) {
    c.B += a - ay;
    c.Z2 += z2;
  }
}
template <int NSUB, int W, bool BF16, bool PREV>
__device__ __forceinline__ void fold(LaneState& c, const float (*x)[W], const uint4* qc,
                                     const uint4* qp, const float* ys, const bool* valid,
                                     const int* start) {
  fold_head<NSUB, W, BF16, PREV>(c, x, qc, valid, start);
  fold_tail<NSUB, W, BF16, PREV>(c, x, nullptr, qp, ys, valid);
}

// Sum four doubles over the workgroup in a fixed order.  Only thread 0
// receives the totals (the only consumer); its loop over the per-wave
// partials is kept rolled so the other waves' partials are not all held in
// registers at once.
template <int NT>
__device__ __forceinline__ void block_sum4_to0(double& a, double& b, double& c, double& d,
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
  if (threadIdx.x == 0) {
    a = sh[0][0];
    b = sh[1][0];
    c = sh[2][0];
    d = sh[3][0];
#pragma unroll 1
    for (int i = 1; i < NW; ++i) {
      a += sh[0][i];
      b += sh[1][i];
      c += sh[2][i];
      d += sh[3][i];
    }
  }
}

// Partial statistics of one wave, workgroup or split of a row: its max m,
// the lowest index holding m, and sums relative to its integer reference
// h = ceil(m * log2 e).
struct Partial {
  double Z, A, B, Z2;
  float m, h;
  int cand, pad;
};

template <int NT>
struct Shared {
  float f[NT / DLM_WAVE];
  int i[NT / DLM_WAVE];
  double d[4][NT / DLM_WAVE];
  Partial rec[NT / DLM_WAVE];
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
  block_sum4_to0<NT>(Z, A, B, Z2, sh.d);
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

struct StatsArgs {
  const void* logits;
  const void* prev;
  int64_t V, ld;
  const int64_t* row_index;
  float *conf, *ent, *kl, *lse;
  int32_t* argmax;
  int aligned, splits;
  int* counters;     // [rows], zero between calls
  Partial* parts;    // [rows][splits]
};

// Sums taken relative to the integer reference h, moved to the reference
// hn >= h: an exact power-of-two scaling (terms that fall below the double
// range, such as those of lanes that saw no finite data, become zero).
__device__ __forceinline__ void rebase(double& Z, double& A, double& B, double& Z2, float h,
                                       float hn) {
  const double d = static_cast<double>(h) - static_cast<double>(hn);  // integer <= 0
  const int di = static_cast<int>(fmax(d, -1100.0));
  A = ldexp(fma(d, Z, A), di);
  Z = ldexp(Z, di);
  B = ldexp(B, di);
  Z2 = ldexp(Z2, di);
}

// Merge n partial records (got in index order 0..n-1, a fixed order) into
// one: the max, the lowest index among records holding it, and the sums
// relative to the max's integer reference.
template <bool PREV, typename Get>
__device__ __forceinline__ Partial merge(int n, Get get) {
  Partial t;
  t.m = kLow;
  for (int k = 0; k < n; ++k) t.m = fmaxf(t.m, get(k).m);
  t.h = ceilf(t.m * kL2E);
  t.cand = INT32_MAX;
  t.Z = t.A = t.B = t.Z2 = 0.0;
  for (int k = 0; k < n; ++k) {
    const Partial q = get(k);
    double Z = q.Z, A = q.A, B = q.B, Z2 = q.Z2;
    rebase(Z, A, B, Z2, q.h, t.h);
    t.Z += Z;
    t.A += A;
    if constexpr (PREV) {
      t.B += B;
      t.Z2 += Z2;
    }
    if (q.m == t.m && q.cand < t.cand) t.cand = q.cand;
  }
  return t;
}

template <int J>
__device__ __forceinline__ double xor_lane_d(double v) {
  return __longlong_as_double(static_cast<long long>(
      dlm::xor_lane64<J>(static_cast<uint64_t>(__double_as_longlong(v)))));
}

// Merge the NW per-wave records on one wave (lane k < NW holds record k)
// with a fixed butterfly over lane distances 1, 2, 4, ...: the max, the
// lowest index holding it, and the sums moved to the max's integer
// reference.  Every lane ends with the same total.  Call with the whole wave.
template <int NW, bool PREV>
__device__ __forceinline__ Partial merge_lanes(Partial q) {
  const int l = threadIdx.x % DLM_WAVE;
  const bool real = l < NW;
  float m = real ? q.m : kLow;
  if constexpr (NW > 1) m = fmaxf(m, __int_as_float(dlm::xor_lane<1>(__float_as_int(m))));
  if constexpr (NW > 2) m = fmaxf(m, __int_as_float(dlm::xor_lane<2>(__float_as_int(m))));
  if constexpr (NW > 4) m = fmaxf(m, __int_as_float(dlm::xor_lane<4>(__float_as_int(m))));
  if constexpr (NW > 8) m = fmaxf(m, __int_as_float(dlm::xor_lane<8>(__float_as_int(m))));
  Partial t;
  t.m = m;
  t.h = ceilf(m * kL2E);
  double Z = 0.0, A = 0.0, B = 0.0, Z2 = 0.0;
  int cand = INT32_MAX;
  if (real) {
    Z = q.Z;
    A = q.A;
    B = q.B;
    Z2 = q.Z2;
    rebase(Z, A, B, Z2, q.h, t.h);
    if (q.m == m) cand = q.cand;
  }
#define DLM_MERGE_STEP(J)                                                 \
  Z += xor_lane_d<J>(Z);                                                  \
  A += xor_lane_d<J>(A);                                                  \
  if constexpr (PREV) {                                                   \
    B += xor_lane_d<J>(B);                                                \
    Z2 += xor_lane_d<J>(Z2);                                              \
  }                                                                       \
  cand = min(cand, dlm::xor_lane<J>(cand));
  if constexpr (NW > 1) { DLM_MERGE_STEP(1) }
  if constexpr (NW > 2) { DLM_MERGE_STEP(2) }
  if constexpr (NW > 4) { DLM_MERGE_STEP(4) }
  if constexpr (NW > 8) { DLM_MERGE_STEP(8) }
#undef DLM_MERGE_STEP
  t.Z = Z;
  t.A = A;
  t.B = PREV ? B : 0.0;
  t.Z2 = PREV ? Z2 : 0.0;
  t.cand = cand;
  return t;
}

// log2 of a positive finite double: exact exponent plus an fp32 log2 of the
// mantissa in [0.5, 1) (absolute error about 1e-7).
__device__ __forceinline__ double log2_split(double v) {
  int e;
  const double f = frexp(v, &e);
  return static_cast<double>(e) + static_cast<double>(log2f(static_cast<float>(f)));
}

// Turn row totals (relative to the integer reference t.h) into the outputs.
// Returns false when a total is not finite (or the previous row's mass is out
// of the reference's range): the caller then runs the element-wise path.
template <bool PREV>
__device__ __forceinline__ bool finalize(const StatsArgs& p, int64_t r, const Partial& t) {
  const float M = t.m;
  bool ok = isfinite(t.Z) && t.Z > 0.0 && isfinite(t.A) && M > kLow && isfinite(M) &&
            t.cand >= 0 && t.cand != INT32_MAX;
  // Z2 below 2^-60 would mean the previous row's mass sits far below the
  // current row's reference, where fp32 terms lose precision: exact path.
  if constexpr (PREV) ok = ok && isfinite(t.B) && isfinite(t.Z2) && t.Z2 >= 0x1p-60;
  if (!ok) return false;
  // Z_true = Z * 2^cM with cM = h - M*log2e in [0, 1]: conf and lse need it;
  // entropy does not (it cancels) and KL uses a common reference.
  const double cM = static_cast<double>(t.h) - static_cast<double>(M) * kL2Ed;
  const double iz = 1.0 / t.Z;
  const double l2z = log2_split(t.Z);
  p.argmax[r] = t.cand;
  p.lse[r] = static_cast<float>(static_cast<double>(M) + kLN2 * (l2z + cM));
  p.conf[r] = static_cast<float>(static_cast<double>(exp2f(static_cast<float>(-cM))) * iz);
  p.ent[r] = static_cast<float>(kLN2 * (l2z - t.A * iz));
  if constexpr (PREV) p.kl[r] = static_cast<float>(kLN2 * (t.B * iz + log2_split(t.Z2 * iz)));
  return true;
}

template <typename T>
__device__ __forceinline__ void st_agent(T* a, T v) {
  __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_agent(T* a) {
  return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The work of one workgroup of NT threads: row r, split s of p.splits.  With
// one split the workgroup owns the whole row.  Otherwise each split streams a contiguous range of the row's
// chunks and publishes a Partial; the row's last-arriving workgroup (atomic
// counter) merges the partials in split order — the same order whichever
// workgroup arrives last — and resets the counter to zero.
// UB: 16-byte chunks per lane per segment for bf16 rows (fp32 rows use 4).
// More chunks keep more bytes in flight per workgroup at the cost of
// registers; the value changes the summation order, not the definitions.
template <int NT, bool BF16, bool PREV, int UB = DLM_STATS_U_BF16, bool PING = false>
__device__ __forceinline__ void stats_block(const StatsArgs& p, int64_t r, int s) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int VEC = 16 / ES;          // elements per 16-byte chunk
  constexpr int U = BF16 ? UB : 4;      // chunks per lane per segment
  __shared__ Shared<NT> sh;

  const int S = p.splits;
  const int64_t V = p.V;
  // no index array: row r itself (no dependent load before the stream starts)
  const int64_t off = (p.row_index ? p.row_index[r] : r) * p.ld;
  const char* cur = static_cast<const char*>(p.logits) + off * ES;
  const char* prv = PREV ? static_cast<const char*>(p.prev) + off * ES : nullptr;
  const int tid = threadIdx.x;

  if (!p.aligned) {  // the host never splits unaligned rows
    careful_row<NT, BF16, PREV>(cur, prv, V, sh, r, p.conf, p.argmax, p.ent, p.kl, p.lse);
    return;
  }

  const uint4* cur4 = reinterpret_cast<const uint4*>(cur);
  const uint4* prv4 = reinterpret_cast<const uint4*>(prv);
  const int64_t nC = V / VEC;
  const int tail = static_cast<int>(V - nC * VEC);
  const int64_t c_lo = nC * s / S, c_hi = nC * (s + 1) / S;  // this split's chunks
  const int64_t n_c = c_hi - c_lo;
  constexpr int64_t SEG = static_cast<int64_t>(U) * NT;
  const int64_t n_full = n_c / SEG;

  // (the sentinel's h is integral; any finite max passes thr and sets h)
  LaneState c{kLow, kLow * kL2E, kLow, 0.f, 0.f, 0.f, 0.f, -1, VEC, make_uint4(0u, 0u, 0u, 0u)};
  bool allv[U];
#pragma unroll
  for (int u = 0; u < U; ++u) allv[u] = true;

  // software-pipelined full segments: the loads of segment it+1 are issued
  // before segment it is folded
  uint4 qc[U], qp[U];
  if (!PING && n_full > 0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      qc[u] = load16(cur4 + c_lo + u * NT + tid);
      if constexpr (PREV) qp[u] = load16(prv4 + c_lo + u * NT + tid);
    }
  }
  if constexpr (PING) {
    // two segments in flight: segment it+1 is issued into the other
    // register set before segment it is folded, and the last trip is peeled,
    // so every trip of the loop enters with one set outstanding.  The empty
    // asm statements fix where values exist: the unpacked rows right after
    // unpacking (the compiler would otherwise rederive them from the raw
    // chunk after the next loads were issued into it, and then copy the
    // loaded registers at the loop's end behind a full wait), and the
    // running sums before the next issue (else the folds sink below the
    // waits).  Same-process A/B, bitwise-equal outputs: 2048 x 126464
    // without prev 78.1 against 80.5 us, 4096 x 151936 184.2 against 185.9,
    // 65536 x 126464 with prev 4786 against 4817, 1024 with prev 81.4
    // against 82.5.  The 768-thread rows keep the single buffer: there
    // every form with a second segment in flight per wave measured slower
    // (this one 22.5 against 21.8 us).
    uint4 ca[U], pa[U], cb[U], pb[U];
    auto issue = [&](uint4 (&qc2)[U], uint4 (&qp2)[U], int64_t it) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t ch = c_lo + it * SEG + u * NT + tid;
        qc2[u] = load16(cur4 + ch);
        if constexpr (PREV) qp2[u] = load16(prv4 + ch);
      }
    };
    auto consume = [&](const uint4 (&qc2)[U], const uint4 (&qp2)[U], int64_t it) {
      float x[U][VEC], y[U][VEC];
      int st[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        unpack<BF16>(qc2[u], x[u]);
        if constexpr (PREV) unpack<BF16>(qp2[u], y[u]);
        st[u] = static_cast<int>((c_lo + it * SEG + u * NT + tid) * VEC);
        // the unpacked values exist from here on: the compiler may not
        // rederive them from the raw chunk later, so the chunk's registers
        // are free for the next loads once the head has read them
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
          asm volatile("" : "+v"(x[u][k]));
          if constexpr (PREV) asm volatile("" : "+v"(y[u][k]));
        }
      }
      fold_head<U, VEC, BF16, PREV>(c, x, qc2, allv, st);
      fold_tail<U, VEC, BF16, PREV>(c, x, PREV ? y : nullptr, nullptr, nullptr, allv);
      // the sums are complete here, before the next loads are issued
      asm volatile("" : "+v"(c.Z), "+v"(c.A));
      if constexpr (PREV) asm volatile("" : "+v"(c.B), "+v"(c.Z2));
    };
    int64_t it = 0;
    if (n_full > 0) issue(ca, pa, 0);
    __builtin_amdgcn_sched_barrier(0);
    for (; it + 2 < n_full; it += 2) {
      issue(cb, pb, it + 1);
      __builtin_amdgcn_sched_barrier(0);
      consume(ca, pa, it);
      __builtin_amdgcn_sched_barrier(0);
      issue(ca, pa, it + 2);
      __builtin_amdgcn_sched_barrier(0);
      consume(cb, pb, it + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (it + 1 < n_full) {
      issue(cb, pb, it + 1);
      __builtin_amdgcn_sched_barrier(0);
      consume(ca, pa, it);
      consume(cb, pb, it + 1);
    } else if (it < n_full) {
      consume(ca, pa, it);
    }
  } else
  for (int64_t it = 0; it < n_full; ++it) {
    float x[U][VEC];
    uint4 xq[U], yq[U];
    int st[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      unpack<BF16>(qc[u], x[u]);
      xq[u] = qc[u];
      if constexpr (PREV) yq[u] = qp[u];
      st[u] = static_cast<int>((c_lo + it * SEG + u * NT + tid) * VEC);
    }
    if (it + 1 < n_full) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t ch = c_lo + (it + 1) * SEG + u * NT + tid;
        qc[u] = load16(cur4 + ch);
        if constexpr (PREV) qp[u] = load16(prv4 + ch);
      }
      __builtin_amdgcn_s_setprio(0);
    }
    fold<U, VEC, BF16, PREV>(c, x, xq, yq, nullptr, allv, st);
    // 768-thread rows: from the end of the fold until the next loads are
    // issued the wave runs at a raised priority, so when its segment arrives
    // it moves the chunk and issues the next loads ahead of the other waves'
    // folds on its SIMD (the memory stream waits less).  Same-process A/B,
    // bitwise-equal outputs: 22.20-22.27 against 22.30-22.48 us.
    if constexpr (NT == 768) __builtin_amdgcn_s_setprio(3);
  }
  __builtin_amdgcn_s_setprio(0);
  // last, partial segment of this split
  if (n_full * SEG < n_c) {
    float x[U][VEC];
    uint4 xq[U], yq[U];
    int st[U];
    bool val[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t ch = c_lo + n_full * SEG + u * NT + tid;
      val[u] = ch < c_hi;
      uint4 a = make_uint4(0u, 0u, 0u, 0u), b = a;
      if (val[u]) {
        a = load16(cur4 + ch);
        if constexpr (PREV) b = load16(prv4 + ch);
      }
      unpack<BF16>(a, x[u]);
      xq[u] = a;
      yq[u] = b;
      st[u] = static_cast<int>(ch * VEC);
    }
    fold<U, VEC, BF16, PREV>(c, x, xq, yq, nullptr, val, st);
  }
  // scalar tail elements (vocab not a multiple of the chunk width): last split
  if (s == S - 1 && tid < tail) {
    const int64_t v = nC * VEC + tid;
    float x[1][1];
    x[0][0] = load_elem<BF16>(cur, v);
    const float y = PREV ? load_elem<BF16>(prv, v) : 0.f;
    const bool val[1] = {true};
    const int st[1] = {static_cast<int>(v)};
    fold<1, 1, BF16, PREV>(c, x, nullptr, nullptr, &y, val, st);
  }

  // ---- this lane's argmax candidate, from the chunk kept in registers
  int cand = INT32_MAX;
  if (c.best >= 0) {
    if (c.bestw == 1) {
      cand = c.best;
    } else {
#pragma unroll
      for (int k = VEC - 1; k >= 0; --k)
        if (elem_of<BF16>(c.bq, k) == c.m) cand = c.best + k;
    }
  }

  // ---- wave merge (DPP): max, lowest index holding it, and the sums moved
  // to the wave's integer reference hw = ceil(Mw*log2e)
  Partial w;
  w.m = dlm::wave_reduce(c.m, dlm::OpMaxF{});
  w.cand = dlm::wave_reduce(c.m == w.m ? cand : INT32_MAX, dlm::OpMinI{});
  w.h = ceilf(w.m * kL2E);
  {
    double Z = c.Z, A = c.A, B = c.B, Z2 = c.Z2;
    rebase(Z, A, B, Z2, c.h, w.h);
    w.Z = dlm::wave_reduce(Z, dlm::OpAdd{});
    w.A = dlm::wave_reduce(A, dlm::OpAdd{});
    if constexpr (PREV) {
      w.B = dlm::wave_reduce(B, dlm::OpAdd{});
      w.Z2 = dlm::wave_reduce(Z2, dlm::OpAdd{});
    } else {
      w.B = w.Z2 = 0.0;
    }
  }
  // ---- workgroup merge: one record per wave, one barrier, wave 0 merges
  // the records across its lanes and thread 0 finalizes
  if (tid % DLM_WAVE == 0) sh.rec[tid / DLM_WAVE] = w;
  __syncthreads();
  Partial t;
  if (tid < DLM_WAVE) {
    Partial q{};
    if (tid < NT / DLM_WAVE) q = sh.rec[tid];
    t = merge_lanes<NT / DLM_WAVE, PREV>(q);
  }

  if (S == 1) {
    if (tid == 0) sh.flag = finalize<PREV>(p, r, t);
    __syncthreads();
    if (!sh.flag)
      careful_row<NT, BF16, PREV>(cur, prv, V, sh, r, p.conf, p.argmax, p.ent, p.kl, p.lse);
    return;
  }

  // ---- publish this split; the last workgroup of the row merges
  if (tid == 0) {
    Partial* mine = p.parts + r * S + s;
    st_agent(&mine->Z, t.Z);
    st_agent(&mine->A, t.A);
    st_agent(&mine->B, t.B);
    st_agent(&mine->Z2, t.Z2);
    st_agent(&mine->m, t.m);
    st_agent(&mine->h, t.h);
    st_agent(&mine->cand, t.cand);
    __threadfence();  // release the partial before counting in
    const int arrived = atomicAdd(p.counters + r, 1);
    sh.flag = arrived == S - 1 ? 1 : 0;
  }
  __syncthreads();
  if (!sh.flag) return;  // not the last split of this row (uniform)
  if (tid == 0) {
    __threadfence();  // acquire the other splits' partials
    Partial* row = p.parts + r * S;
    const Partial u = merge<PREV>(S, [&](int k) {  // split order: deterministic
      Partial q;
      q.Z = ld_agent(&row[k].Z);
      q.A = ld_agent(&row[k].A);
      q.B = ld_agent(&row[k].B);
      q.Z2 = ld_agent(&row[k].Z2);
      q.m = ld_agent(&row[k].m);
      q.h = ld_agent(&row[k].h);
      q.cand = ld_agent(&row[k].cand);
      return q;
    });
    st_agent(p.counters + r, 0);  // ready for the next call
    sh.flag = finalize<PREV>(p, r, u);
  }
  __syncthreads();
  if (!sh.flag)
    careful_row<NT, BF16, PREV>(cur, prv, V, sh, r, p.conf, p.argmax, p.ent, p.kl, p.lse);
}

}  // namespace
