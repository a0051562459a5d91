// stats.hip — dlm_step_stats: the kernel (one workgroup per row or row split;
// the device code and its design notes are in stats_impl.h) and the host
// entry points: launch shape, split-row workspace, validation.
#include "checks.h"
#include "devinfo.h"
#include "stats_impl.h"

namespace {

template <int NT, bool BF16, bool PREV>
__global__ __launch_bounds__(NT) void k_stats(const StatsArgs p) {
  stats_block<NT, BF16, PREV, stats_unroll<NT>(), stats_ping<NT, BF16>()>(
      p, blockIdx.x / p.splits, static_cast<int>(blockIdx.x % p.splits));
}

template <int NT, bool BF16>
hipError_t launch_nt(const StatsArgs& a, int64_t n_rows, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(n_rows * a.splits));
  if (a.prev)
    hipLaunchKernelGGL((k_stats<NT, BF16, true>), grid, dim3(NT), 0, s, a);
  else
    hipLaunchKernelGGL((k_stats<NT, BF16, false>), grid, dim3(NT), 0, s, a);
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch_dt(int nt, const StatsArgs& a, int64_t n_rows, hipStream_t s) {
  switch (nt) {
    case 256:
      return launch_nt<256, BF16>(a, n_rows, s);
    case 768:
      return launch_nt<768, BF16>(a, n_rows, s);
    default:
      return launch_nt<512, BF16>(a, n_rows, s);
  }
}

constexpr int kMaxSplits = 8;
constexpr size_t kCounterAlign = 256;

size_t counters_bytes(int64_t n_rows) {
  const size_t b = static_cast<size_t>(n_rows) * sizeof(int);
  return (b + kCounterAlign - 1) / kCounterAlign * kCounterAlign;
}
size_t bytes_for(int64_t rows) {
  return counters_bytes(rows) + static_cast<size_t>(rows) * kMaxSplits * sizeof(Partial);
}
// Rows a workspace of `bytes` serves.  The layout (counters, then partials)
// depends on the workspace size only, never on the call's row count, so calls
// with different row counts can share one zero-filled buffer.
int64_t workspace_rows(size_t bytes) {
  int64_t c = static_cast<int64_t>(bytes / (sizeof(int) + kMaxSplits * sizeof(Partial)));
  while (c > 0 && bytes_for(c) > bytes) --c;
  return c;
}

// Threads per row (stats_threads) and splits per row.  Very few rows (<= 64)
// with a workspace: split each row so that the launch has about one
// workgroup per CU.  Splitting more rows than that costs more than it gains:
// each split's agent-scope release/acquire writes back / invalidates its
// XCD's L2 while the other workgroups stream through it.
void launch_shape(int64_t n_rows, int64_t n_chunks, bool can_split, bool prev, bool bf16, int cus,
                  int* nt, int* splits) {
  *nt = stats_threads(n_rows, prev, bf16, cus);
  int sp = 1;
  if (can_split && n_rows <= 64) {
    *nt = 512;  // split rows: the cap below assumes 512-thread splits
    sp = static_cast<int>((256 + n_rows - 1) / n_rows);
    if (sp > kMaxSplits) sp = kMaxSplits;
    // each split should keep every lane busy for at least two segments
    const int64_t cap = n_chunks / (2 * 2 * 512);
    if (sp > cap) sp = static_cast<int>(cap < 1 ? 1 : cap);
  }
  *splits = sp;
}

}  // namespace

extern "C" size_t dlm_step_stats_workspace_bytes(int64_t n_rows) {
  if (n_rows <= 0 || n_rows > 2147483647LL) return 0;
  return bytes_for(n_rows);
}

extern "C" int dlm_step_stats(const void* logits, const void* prev_logits, int dtype,
                              int64_t vocab, int64_t ld, const int64_t* row_index,
                              int64_t n_rows, float* conf, int32_t* argmax, float* entropy,
                              float* kl, float* lse, void* workspace, size_t workspace_bytes,
                              void* stream) {
  const int rc = dlmh::check_stats(logits, prev_logits, dtype, vocab, ld, row_index, n_rows, conf,
                                   argmax, entropy, kl, lse);
  if (rc != DLM_OK) return rc;
  const int es = dtype == DLM_BF16 ? 2 : 4;
  const uintptr_t a = reinterpret_cast<uintptr_t>(logits);
  const uintptr_t b = reinterpret_cast<uintptr_t>(prev_logits);
  if (workspace) {
    if (reinterpret_cast<uintptr_t>(workspace) % 16) return DLM_ERR_ARG;
    if (workspace_bytes < dlm_step_stats_workspace_bytes(n_rows)) return DLM_ERR_ARG;
  }
  const int aligned = (a % 16 == 0) && (b % 16 == 0) && ((ld * es) % 16 == 0);
  int cus = 0;
  const int rc2 = dlmh::cu_count(&cus);
  if (rc2 != DLM_OK) return rc2;
  int nt, splits;
  launch_shape(n_rows, vocab / (16 / es), workspace != nullptr && aligned,
               prev_logits != nullptr, dtype == DLM_BF16, cus, &nt, &splits);
  StatsArgs args{logits, prev_logits, vocab, ld, row_index, conf, entropy, kl, lse, argmax,
                 aligned, splits, static_cast<int*>(workspace),
                 workspace ? reinterpret_cast<Partial*>(
                                 static_cast<char*>(workspace) +
                                 counters_bytes(workspace_rows(workspace_bytes)))
                           : nullptr};
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t err = dtype == DLM_BF16 ? launch_dt<true>(nt, args, n_rows, s)
                                           : launch_dt<false>(nt, args, n_rows, s);
  return err == hipSuccess ? DLM_OK : DLM_ERR_HIP;
}
