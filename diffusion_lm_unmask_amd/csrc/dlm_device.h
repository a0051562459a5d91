// dlm_device.h — small device helpers shared by the library's kernels:
// bf16 unpacking, 64-wide wavefront reductions and workgroup reductions.
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

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, DLM_WAVE);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, DLM_WAVE));
  return v;
}
__device__ __forceinline__ int wave_min_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, DLM_WAVE));
  return v;
}
__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, DLM_WAVE));
  return v;
}

// Workgroup reductions. `sh` must hold NT/64 elements; every thread gets the
// result.  Each call ends with a barrier-protected read, so `sh` may be
// reused by the next call after it returns (the leading barrier covers it).
template <int NT, typename T>
__device__ __forceinline__ T block_sum(T v, T* sh) {
  constexpr int NW = NT / DLM_WAVE;
  v = wave_sum(v);
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
  v = wave_max(v);
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
  v = wave_min_i(v);
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
  v = wave_max_i(v);
  const int w = threadIdx.x / DLM_WAVE, l = threadIdx.x % DLM_WAVE;
  __syncthreads();
  if (l == 0) sh[w] = v;
  __syncthreads();
  int r = sh[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = max(r, sh[i]);
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
