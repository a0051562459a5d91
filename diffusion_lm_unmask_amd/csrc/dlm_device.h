// dlm_device.h — small device helpers shared by the library's kernels:
// bf16 unpacking, 64-wide wavefront reductions (shuffle and DPP), sort keys,
// register sorts of 64-key runs with rank placement, and workgroup
// reductions.
// gfx950 only (wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dlm.h"

#define DLM_WAVE 64

namespace dlm {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_at(const uint16_t* p, int64_t i) {
  return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}

// Wave reductions on the DPP crossbar (no LDS traffic).  Inside each row of
// 16 lanes, four steps pair every lane with one lane of the other half of its
// current group: quad swaps (xor 1, xor 2), then the half-row mirror (i with
// 7-i) and the row mirror (i with 15-i).  Each lane then holds its row's
// total, bitwise equal across the row because + , max and min are
// commutative.  The four row totals (lanes 0, 16, 32, 48) are combined in a
// fixed order and returned to every lane.  Call with all 64 lanes active.
// Every control used here (quad permutations, row and half-row mirrors)
// reads a lane of the same row for every lane, so all lanes are written and
// no old value is needed (v_mov_dpp without an initialising move).
template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(dpp<CTRL>(__float_as_int(v)));
}
template <int CTRL>
__device__ __forceinline__ double dpp(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = dpp<CTRL>(static_cast<int>(b));
  const int hi = dpp<CTRL>(static_cast<int>(b >> 32));
  return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned>(lo));
}
__device__ __forceinline__ int rdlane(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ float rdlane(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ double rdlane(double v, int l) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane(static_cast<int>(b), l);
  const int hi = __builtin_amdgcn_readlane(static_cast<int>(b >> 32), l);
  return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned>(lo));
}
__device__ __forceinline__ uint64_t rdlane64(uint64_t v, int l) {
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), l));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v >> 32), l));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T v, Op op) {
  v = op(v, dpp<0xB1>(v));   // quad_perm [1,0,3,2]
  v = op(v, dpp<0x4E>(v));   // quad_perm [2,3,0,1]
  v = op(v, dpp<0x141>(v));  // row_half_mirror
  v = op(v, dpp<0x140>(v));  // row_mirror
  return op(op(rdlane(v, 0), rdlane(v, 16)), op(rdlane(v, 32), rdlane(v, 48)));
}
struct OpAdd {
  template <typename T>
  __device__ T operator()(T a, T b) const { return a + b; }
};
struct OpMaxF {
  __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct OpMinI {
  __device__ int operator()(int a, int b) const { return min(a, b); }
};
struct OpMaxI {
  __device__ int operator()(int a, int b) const { return max(a, b); }
};
struct OpOrI {
  __device__ int operator()(int a, int b) const { return a | b; }
};

// Order-preserving key of a float for a descending sort: a larger value gives
// a smaller key (NaN is the caller's to exclude); -0 and +0 share a key, so
// equal values tie and a secondary key (a row in the low bits) decides.
__device__ __forceinline__ uint32_t desc_bits(float f) {
  const uint32_t u = f == 0.f ? 0u : __float_as_uint(f);
  const uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~asc;
}

// The value of lane (l xor J) for every lane l, on the VALU (no LDS
// crossbar).  Inside a row of 16 lanes it is DPP: xor 1 and xor 2 are quad
// permutations; xor 4 is the half-row mirror (xor 7) followed by the quad
// reversal (xor 3); xor 8 is the row mirror (xor 15) followed by the half-row
// mirror (xor 7).  Across rows it is gfx950's lane swaps, given the value
// twice: v_permlane16_swap exchanges rows 1 and 3 of its first operand with
// rows 0 and 2 of its second, so the second result holds each even row's
// partner and the first each odd row's; v_permlane32_swap does the same for
// the two halves of the wave.
template <int J>
__device__ __forceinline__ int xor_lane(int v) {
  static_assert(J == 1 || J == 2 || J == 4 || J == 8 || J == 16 || J == 32, "a lane of the wave");
  if constexpr (J == 1) return dpp<0xB1>(v);                  // quad_perm [1,0,3,2]
  else if constexpr (J == 2) return dpp<0x4E>(v);             // quad_perm [2,3,0,1]
  else if constexpr (J == 4) return dpp<0x1B>(dpp<0x141>(v));  // quad_perm [3,2,1,0]
  else if constexpr (J == 8) return dpp<0x141>(dpp<0x140>(v));
  else if constexpr (J == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return static_cast<int>((__lane_id() & 16) ? r[0] : r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return static_cast<int>((__lane_id() & 32) ? r[0] : r[1]);
  }
}
template <int J>
__device__ __forceinline__ uint64_t xor_lane64(uint64_t v) {
  const uint32_t lo = static_cast<uint32_t>(xor_lane<J>(static_cast<int>(v)));
  const uint32_t hi = static_cast<uint32_t>(xor_lane<J>(static_cast<int>(v >> 32)));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
// xor_lane for any 4- or 8-byte value (the bits move unchanged).
template <int J, typename T>
__device__ __forceinline__ T xor_val(T v) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "a 32- or 64-bit value");
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, xor_lane<J>(__builtin_bit_cast(int, v)));
  } else {
    return __builtin_bit_cast(T, xor_lane64<J>(__builtin_bit_cast(uint64_t, v)));
  }
}

// Butterfly sum over the wave (xor 32, 16, ..., 1): every lane ends with the
// total, in one fixed order of additions.
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
  v += xor_val<32>(v);
  v += xor_val<16>(v);
  v += xor_val<8>(v);
  v += xor_val<4>(v);
  v += xor_val<2>(v);
  v += xor_val<1>(v);
  return v;
}

// One compare-exchange step of the bitonic network (pair distance J, merge
// size k) on one wave's registers.
template <int J>
__device__ __forceinline__ uint64_t bitonic_step(uint64_t v, int k, int l) {
  const uint64_t o = xor_lane64<J>(v);
  // the lower lane of a pair keeps the min in an ascending run: one compare
  // picks it (equal keys are interchangeable)
  const bool keep_min = ((l & J) == 0) == ((l & k) == 0);
  return (v < o) == keep_min ? v : o;
}

// Ascending bitonic sort of the first n (a power of two <= 64) lanes' keys
// of one wave, in registers: lane l ends with the key of rank l.  Lanes >= n
// must hold keys no smaller than any of the first n (they sort among
// themselves).  Call with all 64 lanes active (n wave-uniform).
__device__ __forceinline__ uint64_t wave_sort_asc(uint64_t v, int n) {
  const int l = threadIdx.x % DLM_WAVE;
  if (n >= 2) v = bitonic_step<1>(v, 2, l);
  if (n >= 4) {
    v = bitonic_step<2>(v, 4, l);
    v = bitonic_step<1>(v, 4, l);
  }
  if (n >= 8) {
    v = bitonic_step<4>(v, 8, l);
    v = bitonic_step<2>(v, 8, l);
    v = bitonic_step<1>(v, 8, l);
  }
  if (n >= 16) {
    v = bitonic_step<8>(v, 16, l);
    v = bitonic_step<4>(v, 16, l);
    v = bitonic_step<2>(v, 16, l);
    v = bitonic_step<1>(v, 16, l);
  }
  if (n >= 32) {
    v = bitonic_step<16>(v, 32, l);
    v = bitonic_step<8>(v, 32, l);
    v = bitonic_step<4>(v, 32, l);
    v = bitonic_step<2>(v, 32, l);
    v = bitonic_step<1>(v, 32, l);
  }
  if (n >= 64) {
    v = bitonic_step<32>(v, 64, l);
    v = bitonic_step<16>(v, 64, l);
    v = bitonic_step<8>(v, 64, l);
    v = bitonic_step<4>(v, 64, l);
    v = bitonic_step<2>(v, 64, l);
    v = bitonic_step<1>(v, 64, l);
  }
  return v;
}

// Number of keys below v in the sorted runs of 64 keys at runs + 64 r,
// r < n_runs, other than run `mine` (a key's own run gives its lane).  Four
// runs are searched side by side, without branches (a run that is `mine`
// or past the last is searched as run `mine` and not counted).
__device__ __forceinline__ int count_below_in_runs(const uint64_t* runs, int n_runs, int mine,
                                                   uint64_t v) {
  int rank = 0;
  for (int r0 = 0; r0 < n_runs; r0 += 4) {
    const uint64_t* run[4];
    bool use[4];
    int c[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = r0 + q;
      use[q] = r < n_runs && r != mine;
      run[q] = runs + (use[q] ? r : mine) * DLM_WAVE;
      c[q] = 0;
    }
#pragma unroll
    for (int step = 32; step > 0; step >>= 1) {
#pragma unroll
      for (int q = 0; q < 4; ++q) c[q] += run[q][c[q] + step - 1] < v ? step : 0;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      c[q] += run[q][c[q]] < v ? 1 : 0;  // c <= 63 before: 0..64 after
      rank += use[q] ? c[q] : 0;
    }
  }
  return rank;
}

// Sorts the first n (<= 1024) keys of `keys` (LDS) ascending: wave w of the
// NT-thread workgroup sorts the runs of 64 keys w, w + NT/64, ... in
// registers and writes them back in place (a wave touches only its own
// runs); then every key of rank below `limit` is stored at out[rank], its
// rank being its lane plus the keys below it in the other runs.  Keys must be
// unique; slots n .. 64*ceil(n/64) - 1 of `keys` are overwritten with ~0.
// Every thread of the workgroup must call it (it contains two barriers).
template <int NT>
__device__ __forceinline__ void sort_runs(uint64_t* keys, uint64_t* out, int n, int limit) {
  constexpr int NW = NT / DLM_WAVE;
  constexpr int kRunsPerWave = (1024 / DLM_WAVE + NW - 1) / NW;
  const int wv = threadIdx.x / DLM_WAVE, ln = threadIdx.x % DLM_WAVE;
  const int n_runs = (n + DLM_WAVE - 1) / DLM_WAVE;
  uint64_t v[kRunsPerWave];
#pragma unroll
  for (int q = 0; q < kRunsPerWave; ++q) {
    const int r = wv + q * NW;
    v[q] = ~0ull;
    if (r < n_runs) {  // wave-uniform: whole waves sort
      const int i = r * DLM_WAVE + ln;
      v[q] = wave_sort_asc(i < n ? keys[i] : ~0ull, DLM_WAVE);
    }
  }
#pragma unroll
  for (int q = 0; q < kRunsPerWave; ++q) {
    const int r = wv + q * NW;
    if (r < n_runs) keys[r * DLM_WAVE + ln] = v[q];
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kRunsPerWave; ++q) {
    const int r = wv + q * NW;
    if (r < n_runs && v[q] != ~0ull) {
      const int rank = ln + count_below_in_runs(keys, n_runs, r, v[q]);
      if (rank < limit) out[rank] = v[q];
    }
  }
  __syncthreads();
}

// Workgroup reductions (every thread of the workgroup must call them, so each
// wave is whole). `sh` must hold NT/64 elements; every thread gets the
// result.  Each call ends with a barrier-protected read, so `sh` may be
// reused by the next call after it returns (the leading barrier covers it).
template <int NT, typename T>
__device__ __forceinline__ T block_sum(T v, T* sh) {
  constexpr int NW = NT / DLM_WAVE;
  if constexpr (__is_integral(T)) v = wave_reduce(v, OpAdd{});  // exact: DPP
  else v = wave_sum(v);  // floating point: the shuffle tree's fixed order
  const int w = threadIdx.x / DLM_WAVE, l = threadIdx.x % DLM_WAVE;
  __syncthreads();
  if (l == 0) sh[w] = v;
  __syncthreads();
  T r = sh[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r += sh[i];  // fixed order: deterministic
  return r;
}
template <int NT>
__device__ __forceinline__ float block_max(float v, float* sh) {
  constexpr int NW = NT / DLM_WAVE;
  v = wave_reduce(v, OpMaxF{});
  const int w = threadIdx.x / DLM_WAVE, l = threadIdx.x % DLM_WAVE;
  __syncthreads();
  if (l == 0) sh[w] = v;
  __syncthreads();
  float r = sh[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = fmaxf(r, sh[i]);
  return r;
}
template <int NT>
__device__ __forceinline__ int block_min_i(int v, int* sh) {
  constexpr int NW = NT / DLM_WAVE;
  v = wave_reduce(v, OpMinI{});
  const int w = threadIdx.x / DLM_WAVE, l = threadIdx.x % DLM_WAVE;
  __syncthreads();
  if (l == 0) sh[w] = v;
  __syncthreads();
  int r = sh[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = min(r, sh[i]);
  return r;
}
template <int NT>
__device__ __forceinline__ int block_max_i(int v, int* sh) {
  constexpr int NW = NT / DLM_WAVE;
  v = wave_reduce(v, OpMaxI{});
  const int w = threadIdx.x / DLM_WAVE, l = threadIdx.x % DLM_WAVE;
  __syncthreads();
  if (l == 0) sh[w] = v;
  __syncthreads();
  int r = sh[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = max(r, sh[i]);
  return r;
}

// Bitwise OR over a workgroup (DPP within each wave); every thread must call
// it, and every thread gets the result.  `sh` holds NT/64 ints and may be
// reused once it returns.
template <int NT>
__device__ __forceinline__ int block_or_i(int v, int* sh) {
  constexpr int NW = NT / DLM_WAVE;
  v = wave_reduce(v, OpOrI{});
  const int w = threadIdx.x / DLM_WAVE, l = threadIdx.x % DLM_WAVE;
  __syncthreads();
  if (l == 0) sh[w] = v;
  __syncthreads();
  int r = sh[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r |= sh[i];
  return r;
}

// (value, index) arg-max over a workgroup: largest value, lowest index among
// equal values; NaN values never win.  Returns the index (or INT32_MAX).
template <int NT>
__device__ __forceinline__ int block_argmax(float v, int idx, float* shv, int* shi) {
  if (v != v) idx = INT32_MAX;  // NaN
  const float m = block_max<NT>(v != v ? -INFINITY : v, shv);
  int cand = (v == m && idx != INT32_MAX) ? idx : INT32_MAX;
  return block_min_i<NT>(cand, shi);
}

}  // namespace dlm

#define DLM_CHECK_LAUNCH()                                   \
  do {                                                       \
    if (hipGetLastError() != hipSuccess) return DLM_ERR_HIP; \
  } while (0)
