// dapd.hip — dlm_dapd_select and dlm_dapd_step: the three kernels (device
// code and design notes in dapd_impl.h), the workspace size and the host
// entry points.
#include <atomic>
#include <mutex>

#include "checks.h"
#include "dapd_impl.h"

namespace {

template <bool BF16>
__global__ __launch_bounds__(kAvgNT) void k_dapd_avg(
    const void* __restrict__ attn, int n_lh, int64_t S, int64_t batch_stride,
    const int32_t* __restrict__ masked_pos, const int32_t* __restrict__ seq_offsets, int m_max,
    int n_tc, int vec_ok, float* __restrict__ ws_a, Policy P) {
  dapd_avg_tile<BF16>(blockIdx.y, blockIdx.x, attn, n_lh, S, batch_stride, masked_pos,
                      seq_offsets, m_max, n_tc, vec_ok, ws_a, P);
}

__global__ __launch_bounds__(kSymNT) void k_dapd_sym(
    const int32_t* __restrict__ seq_offsets, const int32_t* __restrict__ masked_pos, int64_t S,
    int m_max, const float* __restrict__ conf, float tau, const char* __restrict__ ws, Layout L,
    float* __restrict__ degree, float* __restrict__ sym, float* __restrict__ key_out, Policy P) {
  dapd_sym_rows(blockIdx.y, blockIdx.x, seq_offsets, masked_pos, S, m_max, conf, tau, ws, L,
                degree, sym, key_out, P, nullptr);
}

__global__ __launch_bounds__(kSelNT) void k_dapd_select(
    const int32_t* __restrict__ masked_pos, int64_t S, const int32_t* __restrict__ seq_offsets,
    int m_max, const char* __restrict__ ws, Layout L, const float* __restrict__ conf,
    uint8_t* __restrict__ commit, int32_t* __restrict__ n_commit, float* __restrict__ degree,
    float* __restrict__ sym, float* __restrict__ key_out, Policy P) {
  __shared__ SelSmem<kSelNT> sm;
  dapd_select_seq<kSelNT>(blockIdx.x, masked_pos, S, seq_offsets, m_max, ws, L, conf, commit,
                          n_commit, degree, sym, key_out, P, sm);
}

}  // namespace

extern "C" size_t dlm_dapd_workspace_bytes(int32_t n_seq, int32_t m_max) {
  if (n_seq <= 0 || m_max <= 0 || m_max > DLM_MAX_SEQ_ROWS) return 0;
  return layout(n_seq, m_max).total;
}

namespace {

int dapd_run(const void* attn, int dtype, int32_t n_lh, int64_t S, int64_t batch_stride,
             const int32_t* masked_pos, const int32_t* seq_offsets, int32_t n_seq, int32_t m_max,
             const float* conf, float tau, const Policy& P, uint8_t* commit, int32_t* n_commit,
             float* degree, float* sym, float* key, void* workspace, size_t workspace_bytes,
             void* stream) {
  const int rc = dlmh::check_dapd(attn, dtype, n_lh, S, batch_stride, masked_pos, seq_offsets, n_seq,
                                  m_max, conf, tau, P.late_frac, P.late_tau, commit, n_commit,
                                  workspace, workspace_bytes);
  if (rc != DLM_OK) return rc;
  const uintptr_t ab = reinterpret_cast<uintptr_t>(attn);
  const int vec_ok = (ab % 16 == 0) && (S % 8 == 0) && (batch_stride % 8 == 0);
  const Layout L = layout(n_seq, m_max);
  char* ws = static_cast<char*>(workspace);
  float* ws_a = reinterpret_cast<float*>(ws + L.a);
  const int n_ti = (m_max + kTileRows - 1) / kTileRows;
  const int n_tc = (m_max + 8 * kTileChunks - 1) / (8 * kTileChunks);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(n_ti * n_tc, n_seq);
  if (dtype == DLM_BF16)
    hipLaunchKernelGGL(k_dapd_avg<true>, grid, dim3(kAvgNT), 0, s, attn, n_lh, S, batch_stride,
                       masked_pos, seq_offsets, m_max, n_tc, vec_ok, ws_a, P);
  else
    hipLaunchKernelGGL(k_dapd_avg<false>, grid, dim3(kAvgNT), 0, s, attn, n_lh, S, batch_stride,
                       masked_pos, seq_offsets, m_max, n_tc, vec_ok, ws_a, P);
  DLM_CHECK_LAUNCH();
  hipLaunchKernelGGL(k_dapd_sym, dim3((m_max + kSymRows - 1) / kSymRows, n_seq), dim3(kSymNT), 0,
                     s, seq_offsets, masked_pos, S, m_max, conf, tau, ws, L, degree, sym, key, P);
  DLM_CHECK_LAUNCH();
  hipLaunchKernelGGL(k_dapd_select, dim3(n_seq), dim3(kSelNT), 0, s, masked_pos, S, seq_offsets,
                     m_max, ws, L, conf, commit, n_commit, degree, sym, key, P);
  DLM_CHECK_LAUNCH();
  return DLM_OK;
}

}  // namespace

extern "C" int dlm_dapd_select(const void* attn, int dtype, int32_t n_lh, int64_t S,
                               int64_t batch_stride, const int32_t* masked_pos,
                               const int32_t* seq_offsets, int32_t n_seq, int32_t m_max,
                               const float* conf, float tau, uint8_t* commit,
                               int32_t* n_commit, float* degree, float* sym, float* key,
                               void* workspace, size_t workspace_bytes, void* stream) {
  const Policy P{nullptr, 0.f, 0.f, 0, nullptr};
  return dapd_run(attn, dtype, n_lh, S, batch_stride, masked_pos, seq_offsets, n_seq, m_max, conf,
                  tau, P, commit, n_commit, degree, sym, key, workspace, workspace_bytes, stream);
}

extern "C" int dlm_dapd_step(const void* attn, int dtype, int32_t n_lh, int64_t S,
                             int64_t batch_stride, const int32_t* masked_pos,
                             const int32_t* seq_offsets, int32_t n_seq, int32_t m_max,
                             const float* conf, float tau, const int32_t* gen_len, float late_frac,
                             float late_tau, int32_t pre_unmask, uint8_t* commit,
                             int32_t* n_commit, uint8_t* stage, float* degree, float* sym,
                             float* key, void* workspace, size_t workspace_bytes, void* stream) {
  const Policy P{gen_len, late_frac, late_tau, pre_unmask != 0 ? 1 : 0, stage};
  return dapd_run(attn, dtype, n_lh, S, batch_stride, masked_pos, seq_offsets, n_seq, m_max, conf,
                  tau, P, commit, n_commit, degree, sym, key, workspace, workspace_bytes, stream);
}

// ---- dlm_dapd_select_static: the same selection with its workspace in a
// file-scope device array instead of caller memory, for callers that cannot
// allocate.  Each device holds its own copy of the array from the library's
// load until the process ends.  In host code `scratch` names a host-side
// stand-in, never the device memory: the device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// only that address is handed to kernels.
static __device__ __align__(256) char scratch[DLM_DAPD_STATIC_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch array, or nullptr on a HIP
// error (or a device ordinal beyond the table).
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (!p) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr)
      return nullptr;
    g_scratch[dev].store(q, std::memory_order_release);
    p = q;
  }
  return p;
}

}  // namespace

extern "C" int dlm_dapd_select_static(const void* attn, int dtype, int32_t n_lh, int64_t S,
                                      int64_t batch_stride, const int32_t* masked_pos,
                                      const int32_t* seq_offsets, int32_t n_seq, int32_t m_max,
                                      const float* conf, float tau, uint8_t* commit,
                                      int32_t* n_commit, float* degree, float* sym, float* key,
                                      void* stream) {
  // validate everything else first (with a stand-in workspace of the right
  // size), so that a bad call returns the same code as dlm_dapd_select's
  const size_t need = dlm_dapd_workspace_bytes(n_seq, m_max);
  int rc = dlmh::check_dapd(attn, dtype, n_lh, S, batch_stride, masked_pos, seq_offsets, n_seq,
                            m_max, conf, tau, 0.f, 0.f, commit, n_commit,
                            reinterpret_cast<void*>(uintptr_t{256}), need);
  if (rc != DLM_OK) return rc;
  if (need > static_cast<size_t>(DLM_DAPD_STATIC_BYTES)) return DLM_ERR_UNSUPPORTED;
  void* ws = scratch_ptr();
  if (!ws) return DLM_ERR_HIP;
  const Policy P{nullptr, 0.f, 0.f, 0, nullptr};
  return dapd_run(attn, dtype, n_lh, S, batch_stride, masked_pos, seq_offsets, n_seq, m_max, conf,
                  tau, P, commit, n_commit, degree, sym, key, ws,
                  static_cast<size_t>(DLM_DAPD_STATIC_BYTES), stream);
}
