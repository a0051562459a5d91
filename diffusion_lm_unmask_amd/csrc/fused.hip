// fused.hip — dlm_decide_step: the small-batch decision step in two
// launches, built from the same device code as the individual entry points
// (stats_impl.h, rules_impl.h, cap_impl.h, dapd_impl.h).  The statistics run
// with four 16-byte chunks per lane and segment (the statistics call uses
// two), so they may differ from that call's in the last bits; every rule's
// outputs are bitwise those of its entry point on these statistics.
//
//  launch 1  k_step_stream: workgroups [0, n_rows) each stream one row's
//            statistics; the rest average one DAPD attention tile.  Both are
//            HBM streams with the same 512-thread workgroup, so one grid
//            keeps the memory system busy through each other's ramp-up and
//            tail instead of paying two.  Without DAPD, launch 1 is
//            k_step_rows: the statistics call's own kernel and launch shape
//            (bitwise its results).
//  launch 2  k_step_rules: Fast-dLLM, DepCap and CAP one workgroup per
//            sequence each, and the DAPD scores four rows per wave (one to
//            four waves per workgroup), side by side.  The workgroup that
//            finishes a sequence's last block of scores (an atomic tally per
//            sequence) runs that sequence's greedy (dapd_scores_select).
//            With at most 64 rows per sequence, one workgroup per sequence
//            scores every row and decides (dapd_small_select).
//
// No workgroup waits for another: the statistics reach the rules through
// the launch boundary, and the scores reach the greedy through the tally's
// release/acquire, in the one workgroup that sees every other one done.
#include <hip/hip_ext.h>

#include <algorithm>
#include <atomic>

#include "cap_impl.h"
#include "checks.h"
#include "dapd_impl.h"
#include "devinfo.h"
#include "rules_impl.h"
#include "stats_impl.h"

// Launch 1's balance between a compute unit's statistics row and its
// attention tile (same-process A/B on the 256-row step, launch 1 alone):
// four 16-byte chunks per lane for the row (two: 31.2 us, three: 30.7, four:
// 30.0; five and more exceed the registers for two workgroups per compute
// unit) and two maps in flight per lane for the tile (five: 30.0 us, two:
// 28.9, one: 29.3).  A tile that streams less greedily leaves the row more of
// the compute unit's bandwidth, and the row is the long pole.
#ifndef DLM_STEP_STATS_U
#define DLM_STEP_STATS_U 4
#endif
#ifndef DLM_STEP_TILE_UNR
#define DLM_STEP_TILE_UNR 2
#endif
// The tile's maps one batch at a time (0) or double-buffered (1), as the
// averaging call streams them; the summation order is the same.
#ifndef DLM_STEP_TILE_PIPE
#define DLM_STEP_TILE_PIPE 0
#endif

namespace {

constexpr int kStepNT = 512;

static_assert(kAvgNT == kStepNT, "an attention tile must use the statistics workgroup size");
static_assert(kRuleNT == 256 && kCapNT == 256 && kSymNT <= 256, "rules run with 256 threads");
constexpr int kRulesNT = 256;

struct StreamArgs {
  StatsArgs st;
  int64_t n_rows;
  const void* attn;
  int n_lh, m_max, n_tc, vec_ok, tiles_per_seq;
  int64_t S, batch_stride;
  const int32_t* masked_pos;
  const int32_t* seq_offsets;
  float* ws_a;
  uint64_t* tally;  // [n_seq], zeroed here for launch 2
  Policy P;
};

// Launch 1 without attention tiles: exactly the statistics call's kernel and
// launch shape (one workgroup per row, stats_threads threads), so
// these statistics are bitwise those of dlm_step_stats without a workspace.
template <int NT, bool BF16, bool PREV>
__global__ __launch_bounds__(NT) void k_step_rows(const StatsArgs p) {
  stats_block<NT, BF16, PREV, stats_unroll<NT>(), stats_ping<NT, BF16>()>(p, blockIdx.x, 0);
}

template <bool BF16, bool PREV, bool ABF16>
__global__ __launch_bounds__(kStepNT) void k_step_stream(const StreamArgs a) {
  const int64_t g = blockIdx.x;
  if (g < a.n_rows) {
    stats_block<kStepNT, BF16, PREV, DLM_STEP_STATS_U>(a.st, g, 0);
    return;
  }
  const int64_t t = g - a.n_rows;
  if (threadIdx.x == 0 && t % a.tiles_per_seq == 0) a.tally[t / a.tiles_per_seq] = 0ull;
  dapd_avg_tile<ABF16, DLM_STEP_TILE_UNR, DLM_STEP_TILE_PIPE != 0>(
      static_cast<int>(t / a.tiles_per_seq), static_cast<int>(t % a.tiles_per_seq), a.attn, a.n_lh,
      a.S, a.batch_stride, a.masked_pos, a.seq_offsets, a.m_max, a.n_tc, a.vec_ok, a.ws_a, a.P);
}

struct RulesArgs {
  const int32_t* seq_offsets;
  RowGuess guess;  // equal-length sequences: each one's rows read with its offsets
  const float *conf, *ent, *kl, *lse;
  const int32_t* argmax;
  int nf, nd, nc, ns;  // workgroups of each part (0 = off)
  // Fast-dLLM
  const uint8_t* f_el;
  float f_tau;
  uint8_t* f_commit;
  int32_t* f_n;
  // DepCap
  const uint8_t* d_has_prev;
  double d_lambda, d_eps;
  int d_lmin, d_lmax, d_radius;
  int32_t* d_block_len;
  double* d_score;
  // CAP
  const void* logits;
  int64_t ld, vocab;
  const int64_t* row_index;
  const uint8_t* c_el;
  float c_tau_low, c_tau_high, c_gamma;
  int c_kmax;
  uint8_t* c_commit;
  int32_t* c_n;
  // DAPD scores and greedy
  const int32_t* masked_pos;
  int64_t S;
  int m_max, blocks, waves, wg_per_seq;  // row blocks per sequence, blocks per workgroup
  int small;                             // m_max <= 64: one workgroup per sequence
  float tau;
  const char* ws;
  Layout L;
  Policy P;
  uint8_t* p_commit;
  int32_t* p_n;
};

// The roles' LDS share one allocation: a workgroup runs one role.
union RulesSmem {
  CapSmem cap;
  DepSmem dep;
  SelSmem<kRulesNT> sel;
};

template <bool BF16>
__global__ __launch_bounds__(kRulesNT) void k_step_rules(const RulesArgs a) {
  __shared__ RulesSmem sm;
  int g = blockIdx.x;
  if (g < a.nf) {
    fastdllm_seq<true>(g, a.conf, a.f_el, a.seq_offsets, a.f_tau, a.f_commit, a.f_n, a.guess);
    return;
  }
  g -= a.nf;
  if (g < a.nd) {
    depcap_seq<true>(g, a.kl, a.ent, a.seq_offsets, a.d_has_prev, a.d_lambda, a.d_lmin, a.d_lmax,
               a.d_radius, a.d_eps, a.d_block_len, a.d_score, sm.dep, a.guess);
    return;
  }
  g -= a.nd;
  if (g < a.nc) {
    cap_seq<BF16>(g, a.logits, a.ld, a.vocab, a.row_index, a.seq_offsets, a.conf, a.argmax,
                  a.lse, a.c_el, a.c_tau_low, a.c_tau_high, a.c_gamma, a.c_kmax, a.c_commit,
                  a.c_n, nullptr, nullptr, sm.cap);
    return;
  }
  g -= a.nc;
  if (a.small)
    dapd_small_select<kRulesNT>(g, a.seq_offsets, a.masked_pos, a.S, a.m_max, a.conf, a.tau, a.ws,
                                a.L, a.p_commit, a.p_n, a.P, sm.sel);
  else
    dapd_scores_select<kRulesNT>(g / a.wg_per_seq, g % a.wg_per_seq, a.waves, a.blocks,
                                 a.seq_offsets, a.masked_pos, a.S, a.m_max, a.conf, a.tau, a.ws,
                                 a.L, a.p_commit, a.p_n, a.P, sm.sel);
}

// With events, the launch itself sets them to the kernel's start and end
// (hipExtLaunchKernel), so they time the kernel and not the queue around it.
template <bool BF16, bool PREV, bool ABF16>
void launch_stream_k(dim3 grid, hipStream_t s, const StreamArgs& a, hipEvent_t e0, hipEvent_t e1) {
  if (e0 || e1)
    hipExtLaunchKernelGGL((k_step_stream<BF16, PREV, ABF16>), grid, dim3(kStepNT), 0, s, e0, e1,
                          0, a);
  else
    hipLaunchKernelGGL((k_step_stream<BF16, PREV, ABF16>), grid, dim3(kStepNT), 0, s, a);
}
template <int NT, bool BF16, bool PREV>
void launch_rows_k(int64_t n_rows, hipStream_t s, const StatsArgs& a, hipEvent_t e0,
                   hipEvent_t e1) {
  const dim3 grid(static_cast<unsigned>(n_rows));
  if (e0 || e1)
    hipExtLaunchKernelGGL((k_step_rows<NT, BF16, PREV>), grid, dim3(NT), 0, s, e0, e1, 0, a);
  else
    hipLaunchKernelGGL((k_step_rows<NT, BF16, PREV>), grid, dim3(NT), 0, s, a);
}
template <bool BF16, bool PREV>
void launch_rows(int64_t n_rows, int cus, hipStream_t s, const StatsArgs& a, hipEvent_t e0,
                 hipEvent_t e1) {
  switch (stats_threads(n_rows, PREV, BF16, cus)) {
    case 256:
      launch_rows_k<256, BF16, PREV>(n_rows, s, a, e0, e1);
      break;
    case 768:
      launch_rows_k<768, BF16, PREV>(n_rows, s, a, e0, e1);
      break;
    default:
      launch_rows_k<512, BF16, PREV>(n_rows, s, a, e0, e1);
  }
}
template <bool BF16, bool PREV>
void launch_stream(bool abf16, dim3 grid, hipStream_t s, const StreamArgs& a, hipEvent_t e0,
                   hipEvent_t e1) {
  if (abf16) launch_stream_k<BF16, PREV, true>(grid, s, a, e0, e1);
  else launch_stream_k<BF16, PREV, false>(grid, s, a, e0, e1);
}

}  // namespace

extern "C" int dlm_decide_step(const dlm_step_desc* d, void* stream) {
  if (!d) return DLM_ERR_ARG;
  int rc = dlmh::check_stats(d->logits, d->prev_logits, d->dtype, d->vocab, d->ld, d->row_index,
                             d->n_rows, d->conf, d->argmax, d->entropy, d->kl, d->lse);
  if (rc != DLM_OK) return rc;
  const bool fast = d->fast_commit != nullptr, dep = d->depcap_block_len != nullptr;
  const bool cap = d->cap_commit != nullptr, dapd = d->dapd_commit != nullptr;
  if ((fast || dep || cap || dapd) && (!d->seq_offsets || d->n_seq <= 0)) return DLM_ERR_ARG;
  if (fast &&
      (rc = dlmh::check_fastdllm(d->conf, d->seq_offsets, d->n_seq, d->fast_tau, d->fast_commit,
                                 d->fast_n_commit)) != DLM_OK)
    return rc;
  if (dep && (rc = dlmh::check_depcap(d->kl, d->entropy, d->seq_offsets, d->n_seq,
                                      d->depcap_lambda, d->depcap_l_min, d->depcap_l_max,
                                      d->depcap_radius, d->depcap_eps, d->depcap_block_len)) !=
                 DLM_OK)
    return rc;
  if (cap && (rc = dlmh::check_cap(d->logits, d->dtype, d->vocab, d->ld, d->row_index,
                                   d->seq_offsets, d->n_seq, d->conf, d->argmax, d->lse,
                                   d->cap_tau_low, d->cap_tau_high, d->cap_gamma, d->cap_k_max,
                                   d->cap_commit, d->cap_n_commit)) != DLM_OK)
    return rc;
  if (dapd && (rc = dlmh::check_dapd(d->attn, d->attn_dtype, d->n_lh, d->S, d->batch_stride,
                                     d->masked_pos, d->seq_offsets, d->n_seq, d->m_max, d->conf,
                                     d->dapd_tau, 0.f, 0.f, d->dapd_commit, d->dapd_n_commit,
                                     d->dapd_workspace, d->dapd_workspace_bytes)) != DLM_OK)
    return rc;

  int cus = 0;
  if ((rc = dlmh::cu_count(&cus)) != DLM_OK) return rc;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf16 = d->dtype == DLM_BF16, prev = d->prev_logits != nullptr;
  const int es = bf16 ? 2 : 4;
  const uintptr_t la = reinterpret_cast<uintptr_t>(d->logits);
  const uintptr_t lb = reinterpret_cast<uintptr_t>(d->prev_logits);
  const int aligned = (la % 16 == 0) && (lb % 16 == 0) && ((d->ld * es) % 16 == 0);
  const Policy P{nullptr, 0.f, 0.f, 0, nullptr};

  // ---- launch 1: statistics rows, then attention tiles
  StreamArgs sa{};
  sa.st = StatsArgs{d->logits, d->prev_logits, d->vocab, d->ld, d->row_index, d->conf, d->entropy,
                    d->kl, d->lse, d->argmax, aligned, 1, nullptr, nullptr};
  sa.n_rows = d->n_rows;
  sa.P = P;
  int64_t n_tiles = 0;
  Layout L{};
  char* ws = nullptr;
  if (dapd) {
    L = layout(d->n_seq, d->m_max);
    ws = static_cast<char*>(d->dapd_workspace);
    const uintptr_t ab = reinterpret_cast<uintptr_t>(d->attn);
    sa.attn = d->attn;
    sa.n_lh = d->n_lh;
    sa.m_max = d->m_max;
    sa.n_tc = (d->m_max + 8 * kTileChunks - 1) / (8 * kTileChunks);
    sa.vec_ok = (ab % 16 == 0) && (d->S % 8 == 0) && (d->batch_stride % 8 == 0);
    sa.tiles_per_seq = ((d->m_max + kTileRows - 1) / kTileRows) * sa.n_tc;
    sa.S = d->S;
    sa.batch_stride = d->batch_stride;
    sa.masked_pos = d->masked_pos;
    sa.seq_offsets = d->seq_offsets;
    sa.ws_a = reinterpret_cast<float*>(ws + L.a);
    sa.tally = reinterpret_cast<uint64_t*>(ws + L.tally);
    n_tiles = static_cast<int64_t>(sa.tiles_per_seq) * d->n_seq;
  }
  const int64_t g1 = d->n_rows + n_tiles;
  if (g1 > 2147483647LL) return DLM_ERR_UNSUPPORTED;
  const dim3 grid1(static_cast<unsigned>(g1));
  const bool abf16 = !dapd || d->attn_dtype == DLM_BF16;
  const hipEvent_t e0 = static_cast<hipEvent_t>(d->launch1_begin_event);
  const hipEvent_t e1 = static_cast<hipEvent_t>(d->launch1_end_event);
  if (!dapd) {  // statistics only: the statistics call's own kernel and shape
    if (bf16) {
      if (prev) launch_rows<true, true>(d->n_rows, cus, s, sa.st, e0, e1);
      else launch_rows<true, false>(d->n_rows, cus, s, sa.st, e0, e1);
    } else {
      if (prev) launch_rows<false, true>(d->n_rows, cus, s, sa.st, e0, e1);
      else launch_rows<false, false>(d->n_rows, cus, s, sa.st, e0, e1);
    }
  } else if (bf16) {
    if (prev) launch_stream<true, true>(abf16, grid1, s, sa, e0, e1);
    else launch_stream<true, false>(abf16, grid1, s, sa, e0, e1);
  } else {
    if (prev) launch_stream<false, true>(abf16, grid1, s, sa, e0, e1);
    else launch_stream<false, false>(abf16, grid1, s, sa, e0, e1);
  }
  DLM_CHECK_LAUNCH();

  // ---- launch 2: the per-sequence rules, the DAPD scores and greedy
  RulesArgs ra{};
  ra.seq_offsets = d->seq_offsets;
  ra.guess = RowGuess{0, d->n_rows};  // n_rows >= 1 (checked)
  if (d->n_seq > 0 && d->n_rows % d->n_seq == 0 && d->n_rows / d->n_seq <= 2147483647LL)
    ra.guess.len = static_cast<int>(d->n_rows / d->n_seq);
  ra.conf = d->conf;
  ra.ent = d->entropy;
  ra.kl = d->kl;
  ra.lse = d->lse;
  ra.argmax = d->argmax;
  ra.nf = fast ? d->n_seq : 0;
  ra.nd = dep ? d->n_seq : 0;
  ra.nc = cap ? d->n_seq : 0;
  if (dapd && d->m_max <= DLM_WAVE) {
    ra.small = 1;  // one workgroup per sequence: scores and decision
    ra.ns = d->n_seq;
  } else if (dapd) {
    // one block of kSymRows rows per wave; with more blocks than free compute
    // units (every launch-2 workgroup takes a whole compute unit's LDS), a
    // workgroup scores up to four blocks, so that the scores finish in one
    // round of workgroups
    ra.blocks = (d->m_max + kSymRows - 1) / kSymRows;
    const int64_t total = static_cast<int64_t>(ra.blocks) * d->n_seq;
    const int64_t free_cus = std::max<int64_t>(1, cus - (ra.nf + ra.nd + ra.nc));
    ra.waves = static_cast<int>(
        std::min<int64_t>(kRulesNT / DLM_WAVE, std::max<int64_t>(1, (total + free_cus - 1) / free_cus)));
    ra.wg_per_seq = (ra.blocks + ra.waves - 1) / ra.waves;
    ra.ns = ra.wg_per_seq * d->n_seq;
  }
  ra.f_el = d->fast_eligible;
  ra.f_tau = d->fast_tau;
  ra.f_commit = d->fast_commit;
  ra.f_n = d->fast_n_commit;
  ra.d_has_prev = d->depcap_has_prev;
  ra.d_lambda = d->depcap_lambda;
  ra.d_eps = d->depcap_eps;
  ra.d_lmin = d->depcap_l_min;
  ra.d_lmax = d->depcap_l_max;
  ra.d_radius = d->depcap_radius;
  ra.d_block_len = d->depcap_block_len;
  ra.d_score = d->depcap_score;
  ra.logits = d->logits;
  ra.ld = d->ld;
  ra.vocab = d->vocab;
  ra.row_index = d->row_index;
  ra.c_el = d->cap_eligible;
  ra.c_tau_low = d->cap_tau_low;
  ra.c_tau_high = d->cap_tau_high;
  ra.c_gamma = d->cap_gamma;
  ra.c_kmax = d->cap_k_max;
  ra.c_commit = d->cap_commit;
  ra.c_n = d->cap_n_commit;
  ra.masked_pos = d->masked_pos;
  ra.S = d->S;
  ra.m_max = d->m_max;
  ra.tau = d->dapd_tau;
  ra.ws = ws;
  ra.L = L;
  ra.P = P;
  ra.p_commit = d->dapd_commit;
  ra.p_n = d->dapd_n_commit;
  const int64_t g2 = static_cast<int64_t>(ra.nf) + ra.nd + ra.nc + ra.ns;
  if (g2 > 0) {
    if (bf16)
      hipLaunchKernelGGL(k_step_rules<true>, dim3(static_cast<unsigned>(g2)), dim3(kRulesNT), 0, s,
                         ra);
    else
      hipLaunchKernelGGL(k_step_rules<false>, dim3(static_cast<unsigned>(g2)), dim3(kRulesNT), 0,
                         s, ra);
    DLM_CHECK_LAUNCH();
  }

  return DLM_OK;
}
