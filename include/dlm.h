/*
 * dlm.h — C ABI of the MI355X (gfx950) library for the per-denoising-step
 * unmask decision of masked diffusion language models.
 *
 * One step of a masked diffusion LM produces a logits row for every masked
 * position.  This library decides which of those positions to commit:
 *   1. dlm_step_stats      — per-row confidence, argmax, entropy, KL to the
 *                            previous step's row, log-normaliser (one pass
 *                            over the vocabulary);
 *   2. dlm_fastdllm_select — Fast-dLLM confidence threshold + top-1 fallback;
 *   3. dlm_depcap_boundary — DepCap DepGA-Block boundary scan;
 *   4. dlm_cap_select      — DepCap CAP-Decoding conflict-aware pick;
 *   5. dlm_dapd_select     — DAPD attention graph + Welsh-Powell independent set.
 * and the schedules around them:
 *   6. dlm_dapd_step       — DAPD's full step: late-stage threshold switch and
 *                            pre-unmask of certain rows;
 *   7. dlm_factor_select   — Fast-dLLM factor decoding (+ Theorem-1 certificate);
 *   8. dlm_topk_select     — LLaDA's fixed top-K per step;
 *   9. dlm_fixed_block_eligible — active block of fixed-length block decoding.
 *
 * Conventions for every entry point
 *   - Pointers marked (device) are device pointers owned by the caller; the
 *     library never allocates, frees or retains memory and keeps no global
 *     mutable state, so calls from several host threads are safe.
 *   - Arguments are validated on the host before any HIP call.  On an
 *     invalid argument nothing is enqueued and DLM_ERR_ARG or
 *     DLM_ERR_UNSUPPORTED is returned.  Device-side data (offsets, indices)
 *     cannot be read by the host; a violated device-side precondition is
 *     reported per sequence where stated (n_commit[b] = -1), never by an
 *     out-of-bounds access when the documented bounds are respected.
 *   - Kernels are enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream) and the call returns without synchronising.  Asynchronous
 *     device faults surface at the caller's next synchronisation.
 *   - Outputs are fully overwritten (rows that are not eligible get 0).
 *   - Rows of a sequence are given in CSR form by seq_offsets (device int32,
 *     n_seq+1 entries, non-decreasing, seq_offsets[0] = 0), in position order.
 *   - A NULL `eligible` means every row is eligible.
 *
 * Sources (page title, section) are cited per entry point:
 *   [DepCap] "DepCap: Adaptive Block-Wise Parallel Decoding for Efficient
 *            Diffusion LM Inference" (summary of arXiv 2604.15750);
 *   [DAPD]   "DAPD: Dependency-Aware Parallel Decoding via Attention for
 *            Diffusion LLMs" (ICML 2026 paper note);
 *   [FastR]  "Fast-dLLM: Training-Free Acceleration of Diffusion LLMs via KV
 *            Cache and Parallel Decoding" (review);
 *   [FastN]  "Fast-dLLM: Training-free Acceleration of Diffusion LLM by
 *            Enabling KV Cache and Parallel Decoding" (notes).
 */
#ifndef DLM_H
#define DLM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define DLM_OK 0
#define DLM_ERR_ARG 1         /* NULL required pointer, size <= 0, NaN threshold, ...   */
#define DLM_ERR_UNSUPPORTED 2 /* unknown dtype, a size above a documented limit         */
#define DLM_ERR_HIP 3         /* a kernel launch failed (hipGetLastError)               */

/* logits / attention element types */
#define DLM_BF16 0
#define DLM_F32 1

/* limits */
#define DLM_MAX_VOCAB 2147483647LL /* vocab < 2^31                                       */
#define DLM_MAX_WINDOW 1024        /* DepCap l_max                                        */
#define DLM_MAX_SEQ_ROWS 1024      /* CAP, top-K and factor rows per sequence; DAPD m_max */
#define DLM_MAX_KMAX 128           /* CAP candidate cap                                   */

/* default parameters quoted by the pages */
#define DLM_FASTDLLM_TAU 0.9f      /* [FastR, Method]: default threshold                   */
#define DLM_FASTDLLM_BLOCK 32      /* [FastN, Technical details]: block size               */
#define DLM_DEPCAP_LAMBDA 1.2      /* [DepCap, Experiments]: defaults                      */
#define DLM_DEPCAP_L_MIN 8
#define DLM_DEPCAP_L_MAX 128
#define DLM_DEPCAP_RADIUS 1        /* smoothing radius (a reading: the pages give none)   */
#define DLM_DEPCAP_EPS 1e-12       /* normalisation guard (a reading)                     */
#define DLM_CAP_TAU_LOW 0.8f       /* [DepCap, Experiments; AI Executive Summary]          */
#define DLM_CAP_TAU_HIGH 0.95f
#define DLM_CAP_GAMMA (-16.0f)
#define DLM_DAPD_LAYER_FRAC 0.3    /* [DAPD, overall framework]: last ~30% of layers       */
#define DLM_DAPD_LATE_FRAC 0.5     /* [DAPD, key design 3]: late-stage switch point       */
#define DLM_DAPD_LATE_TAU 0.9f     /* [DAPD, key design 3]: late-stage threshold          */
#define DLM_FACTOR_F 1.0f          /* [FastR, Method; Key idea]: f = Theorem 1's bound (a
                                      reading: the pages give no value)                    */

/*
 * dlm_step_stats — [DepCap, Methodology] H_k = H(p_curr^k) and
 * I_k = KL(p_curr^k || p_prev^k); [DepCap, Methodology] and [FastR, Method]
 * confidence c = max_v p(v) and the argmax token.
 *
 * For r in [0, n_rows): row = logits + row_index[r]*ld elements (and the
 * same offset into prev_logits).  With p = softmax(row) (natural log,
 * temperature 1):
 *   argmax[r]  = lowest index attaining the maximum over non-NaN entries
 *                (0 if the row has none)
 *   lse[r]     = log sum_v exp(row_v)
 *   conf[r]    = max_v p_v = exp(max - lse)
 *   entropy[r] = -sum_v p_v log p_v                       (0 log 0 = 0)
 *   kl[r]      = sum_v p_v (log p_v - log q_v), q = softmax(prev row);
 *                +inf if some p_v > 0 has q_v = 0.
 * A row with a NaN or +inf entry, or with every entry -inf, gives NaN conf,
 * entropy, kl and lse.
 *
 * logits, prev_logits (device): dtype elements (DLM_BF16 or DLM_F32), base
 *   aligned to the element size; prev_logits may be NULL (then kl must be
 *   NULL too).  Rows are streamed at full speed when both bases are 16-byte
 *   aligned and ld*element_size is a multiple of 16; otherwise a slower
 *   element-wise path is used.
 * vocab: 1 <= vocab < 2^31; ld >= vocab.
 * row_index (device int64 [n_rows], or NULL); n_rows >= 1.  Each entry must
 *   name a row of logits (and of prev_logits): 0 <= row_index[r] and the
 *   row's vocab elements inside the caller's allocation, which the library
 *   cannot see.  NULL means row_index[r] = r (the first n_rows rows, in
 *   order), with no index read.
 * conf, entropy, kl, lse (device f32 [n_rows]); argmax (device int32 [n_rows]).
 * workspace (device, optional): NULL, or at least
 *   dlm_step_stats_workspace_bytes(n_rows) bytes, 16-byte aligned and
 *   zero-filled before its first use; every call leaves its counters zero
 *   again.  Its layout depends on workspace_bytes only, so one buffer (always
 *   passed with the same size) serves calls with any row count it covers.
 *   With a workspace, launches of few rows split each row over several
 *   workgroups (the last one merges, always in the same order, so results do
 *   not depend on which finishes first); without one, one workgroup per row.
 *   Calls that overlap in time must not share a workspace.
 * Floating point: fp32 element arithmetic with fp64 cross-lane combination.
 */
int dlm_step_stats(const void* logits, const void* prev_logits, int dtype, int64_t vocab,
                   int64_t ld, const int64_t* row_index, int64_t n_rows, float* conf,
                   int32_t* argmax, float* entropy, float* kl, float* lse, void* workspace,
                   size_t workspace_bytes, void* stream);

/* Workspace bytes dlm_step_stats may use for n_rows rows (0 if n_rows is invalid). */
size_t dlm_step_stats_workspace_bytes(int64_t n_rows);

/*
 * dlm_fastdllm_select — [FastR, Method]; [FastN, Key ideas, Technical details]:
 * commit every eligible row whose confidence exceeds tau; if none does,
 * commit the single highest-confidence eligible row (progress guarantee).
 *   commit[r] = eligible[r] && conf[r] > tau   (strict; NaN never commits)
 *   fallback ties go to the lowest row of the sequence.
 * conf (device f32 [rows]); eligible (device u8 [rows] or NULL);
 * seq_offsets (device int32 [n_seq+1]); n_seq >= 1; tau not NaN.
 * commit (device u8 [rows]); n_commit (device int32 [n_seq]).
 */
int dlm_fastdllm_select(const float* conf, const uint8_t* eligible, const int32_t* seq_offsets,
                        int32_t n_seq, float tau, uint8_t* commit, int32_t* n_commit,
                        void* stream);

/*
 * dlm_depcap_boundary — [DepCap, Methodology bullets 1-3; Technical
 * Contribution]: over the window W_b = min(l_max, rows of sequence b) of
 * future positions right after the last decoded block, smooth and locally
 * normalise I_k (= kl) and H_k (= entropy), form S_k = I~_k - lambda*H~_k,
 * stop before the first S_k < 0 and clip the length to [l_min, W_b]; use
 * l_min (clipped to W_b) on cold start (has_prev[b] == 0).
 * Readings (the pages give no formula): I-bar_k = mean of I_j over
 * j in [k-r, k+r] clipped to the window; I~_k = I-bar_k / (mean_k I-bar + eps);
 * the same for H.  S_k is computed, returned and compared with 0 in fp64
 * (NaN is not negative), so the returned score is the value decided on.
 * kl, entropy (device f32 [rows]); seq_offsets (device int32 [n_seq+1]);
 * has_prev (device u8 [n_seq] or NULL = all warm); 0 <= l_min <= l_max <= 1024;
 * smooth_radius >= 0; eps >= 0; lambda, eps not NaN.
 * block_len (device int32 [n_seq]); score (device f64 [rows] or NULL):
 * S_k for the first W_b rows of a warm sequence, NaN elsewhere.
 */
int dlm_depcap_boundary(const float* kl, const float* entropy, const int32_t* seq_offsets,
                        int32_t n_seq, const uint8_t* has_prev, double lambda, int32_t l_min,
                        int32_t l_max, int32_t smooth_radius, double eps, int32_t* block_len,
                        double* score, void* stream);

/*
 * dlm_cap_select — [DepCap, Methodology bullets 4-6; Technical Contribution;
 * AI Executive Summary]: candidate pool P = {eligible rows with conf >= tau_low},
 * kept to the first k_max in (conf desc, row asc) order; if P is empty commit
 * the top-1 eligible row.  Otherwise
 *   D_ab = (logit_a[yhat_b] - lse_a) + (logit_b[yhat_a] - lse_b)
 * (log p_a(yhat_b) + log p_b(yhat_a)), a conflict is D_ab > gamma (a reading);
 * rows with conf > tau_high are committed first, then the rest in priority
 * order are added when they conflict with nothing chosen.
 * logits (device, dtype, same layout as dlm_step_stats) and row_index (as
 * there; NULL is row r itself): only gathered at (candidate row, candidate
 * argmax).  conf, argmax, lse: the
 * outputs of dlm_step_stats for the same rows.
 * Limits: rows per sequence <= 1024 (else n_commit[b] = -1 and no commit);
 * 1 <= k_max <= 128.  Before any gather, every candidate's argmax is checked
 * to lie in [0, vocab) and its row_index to be >= 0; a sequence failing the
 * check gets n_commit[b] = -1 and no commit (row_index values past the end
 * of the logits cannot be checked: the caller keeps them in range).
 * commit (device u8 [rows]); n_commit (device int32 [n_seq]);
 * cand (device int32 [n_seq*k_max] or NULL): candidate rows in priority
 * order, -1 pad; dmat (device f32 [n_seq*k_max*k_max] or NULL): D in
 * candidate order, NaN on the diagonal and pad.
 */
int dlm_cap_select(const void* logits, int dtype, int64_t vocab, int64_t ld,
                   const int64_t* row_index, const int32_t* seq_offsets, int32_t n_seq,
                   const float* conf, const int32_t* argmax, const float* lse,
                   const uint8_t* eligible, float tau_low, float tau_high, float gamma,
                   int32_t k_max, uint8_t* commit, int32_t* n_commit, int32_t* cand,
                   float* dmat, void* stream);

/*
 * dlm_dapd_workspace_bytes — device workspace that dlm_dapd_select needs for
 * n_seq sequences of at most m_max masked positions (per sequence: the fp32
 * m_max x m_max attention average, the adjacency bitsets, the ordering keys
 * and one counter that dlm_decide_step uses).  Returns 0 for invalid sizes.
 */
size_t dlm_dapd_workspace_bytes(int32_t n_seq, int32_t m_max);

/*
 * dlm_dapd_select — [DAPD, overall framework; key designs 1-2]:
 *   a_ij   = mean over the n_lh maps of attn[b][lh][pos_i][pos_j]
 *            (the caller passes the maps of the last ~30% of layers, all heads;
 *            probabilities used as given, no renormalisation)
 *   s_ij   = (a_ij + a_ji)/2 ; edge (i,j) iff i != j and s_ij > tau
 *   d~_i   = sum_{j != i} s_ij ; key_i = f32(f32(d~_i) * conf_i)
 *   scan nodes by (key desc, position asc) and add each node with no edge
 *   into the chosen set (Welsh-Powell order); NaN keys are never chosen.
 * attn (device, dtype): sequence b's maps start at attn + b*batch_stride
 * elements; map lh is the S x S row-major matrix at offset lh*S*S.
 * masked_pos (device int32 [rows], CSR by seq_offsets): positions in [0, S);
 * a sequence holding a position outside it is never read and gets
 * n_commit = -1.  conf (device f32 [rows]) in the same row order.
 * 1 <= m_max <= 1024 bounds the masked positions per sequence (a longer
 * sequence gets n_commit = -1).
 * workspace (device, >= dlm_dapd_workspace_bytes(n_seq, m_max) bytes, 16-byte
 * aligned, else DLM_ERR_ARG): scratch, overwritten; calls that overlap in
 * time (including dlm_decide_step's DAPD part) must not share one.
 * commit (device u8 [rows]); n_commit (device int32 [n_seq]); degree, key
 * (device f32 [rows] or NULL); sym (device f32 [n_seq*m_max*m_max] or NULL):
 * s_ij, NaN pad.
 */
int dlm_dapd_select(const void* attn, int dtype, int32_t n_lh, int64_t S, int64_t batch_stride,
                    const int32_t* masked_pos, const int32_t* seq_offsets, int32_t n_seq,
                    int32_t m_max, const float* conf, float tau, uint8_t* commit,
                    int32_t* n_commit, float* degree, float* sym, float* key, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * dlm_dapd_select_static — dlm_dapd_select without a caller workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  The workspace is a
 * static device array of DLM_DAPD_STATIC_BYTES in the library, one per GPU,
 * held from the library's load until the process ends; the call allocates
 * nothing.  Every argument, output and error is that of dlm_dapd_select,
 * plus DLM_ERR_UNSUPPORTED when dlm_dapd_workspace_bytes(n_seq, m_max)
 * exceeds DLM_DAPD_STATIC_BYTES (16 MiB: up to 32 sequences of 256 masked
 * positions, or 3 of 1024, fit; 64 of 1024 do not), and DLM_ERR_HIP when the array's device address
 * cannot be obtained.  All calls on one GPU share that GPU's array: calls
 * that overlap in time on one GPU (any streams, any threads) race and must
 * be serialised by the caller.  Nothing in the array needs to start zeroed;
 * each call overwrites what it reads.
 */
#define DLM_DAPD_STATIC_BYTES (16 << 20)
int dlm_dapd_select_static(const void* attn, int dtype, int32_t n_lh, int64_t S,
                           int64_t batch_stride, const int32_t* masked_pos,
                           const int32_t* seq_offsets, int32_t n_seq, int32_t m_max,
                           const float* conf, float tau, uint8_t* commit, int32_t* n_commit,
                           float* degree, float* sym, float* key, void* stream);

/*
 * dlm_dapd_step — [DAPD, overall framework; key design 3]: dlm_dapd_select
 * with the full step policy.  For sequence b with M_b masked rows:
 *   - late stage iff gen_len != NULL and M_b < late_frac * gen_len[b]
 *     (evaluated in double; DLM_DAPD_LATE_FRAC = 0.5, "below 50%"): the graph
 *     is skipped (no attention read) and the rows with conf > late_tau
 *     (DLM_DAPD_LATE_TAU) are committed, or the most confident row (lowest
 *     row on ties, NaN never) when none is (a reading: the page gives no
 *     fallback);
 *   - otherwise the graph stage of dlm_dapd_select;
 *   - with pre_unmask != 0, every row whose conf is exactly 1.0f is also
 *     committed in either stage (the graph is still built over all rows).
 * gen_len (device int32 [n_seq]) or NULL (never late).  stage (device u8
 * [n_seq] or NULL): 1 for a late-stage sequence.  degree and key are NaN for
 * late-stage rows and sym is NaN for late-stage sequences.  Every other
 * argument, and the errors, are those of dlm_dapd_select; late_frac or
 * late_tau NaN gives DLM_ERR_ARG.
 */
int dlm_dapd_step(const void* attn, int dtype, int32_t n_lh, int64_t S, int64_t batch_stride,
                  const int32_t* masked_pos, const int32_t* seq_offsets, int32_t n_seq,
                  int32_t m_max, const float* conf, float tau, const int32_t* gen_len,
                  float late_frac, float late_tau, int32_t pre_unmask, uint8_t* commit,
                  int32_t* n_commit, uint8_t* stage, float* degree, float* sym, float* key,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * dlm_factor_select — [FastR, Method] factor decoding; [FastR, Key idea]
 * Theorem 1.  Per sequence, with c(1) >= c(2) >= ... the confidences of the
 * eligible rows (NaN excluded; ties by lower row), commit the n most
 * confident rows for the largest n with (n+1)(1 - c(n)) < f, evaluated in
 * double on the fp32 values (exact).  At least one row is committed when any
 * is eligible (a reading).  DLM_FACTOR_F = 1 is the theorem's bound.
 * conf (device f32 [rows]); eligible (device u8 [rows] or NULL = all);
 * commit (device u8 [rows]); n_commit (device int32 [n_seq]); certificate
 * (device u8 [n_seq] or NULL): 1 iff n >= 1 and (n+1)(1 - c(n)) <= 1, the
 * theorem's sufficient condition for the parallel commit to equal greedy
 * one-token decoding.  A sequence with more than DLM_MAX_SEQ_ROWS rows gets
 * n_commit = -1 and nothing committed.  f NaN, n_seq <= 0 or a NULL
 * required pointer: DLM_ERR_ARG.
 */
int dlm_factor_select(const float* conf, const uint8_t* eligible, const int32_t* seq_offsets,
                      int32_t n_seq, float f, uint8_t* commit, int32_t* n_commit,
                      uint8_t* certificate, void* stream);

/*
 * dlm_topk_select — [FastR, Prior limitations; Comparison]: LLaDA's default
 * schedule, the k most confident eligible rows of each sequence whatever
 * their confidence (ties by lower row; NaN never; all of them when fewer
 * than k are eligible).  Arguments, limits and errors as dlm_factor_select,
 * with k >= 1 (else DLM_ERR_ARG).
 */
int dlm_topk_select(const float* conf, const uint8_t* eligible, const int32_t* seq_offsets,
                    int32_t n_seq, int32_t k, uint8_t* commit, int32_t* n_commit, void* stream);

/*
 * dlm_fixed_block_eligible — [DepCap, Experiments]: confidence decoding with
 * fixed 16/32/64-token blocks.  Blocks of block_len tile the generation from
 * its first position gen_start[b] (device int32 [n_seq], values >= 0, or NULL
 * = 0); eligible[r] = 1 iff masked_pos[r] lies in the earliest block that
 * still holds a masked position of the sequence (a position before gen_start
 * is never eligible).  Pass the result to dlm_fastdllm_select as `eligible`.
 * masked_pos (device int32 [rows], CSR by seq_offsets); eligible (device u8
 * [rows]).  block_len < 1, n_seq <= 0 or a NULL required pointer:
 * DLM_ERR_ARG.
 */
int dlm_fixed_block_eligible(const int32_t* masked_pos, const int32_t* seq_offsets,
                             int32_t n_seq, const int32_t* gen_start, int32_t block_len,
                             uint8_t* eligible, void* stream);

/*
 * dlm_decide_step — the whole small-batch decision step in two launches
 * (Fast-dLLM review, Limitations: the gains are small-batch; DepCap summary,
 * Applications: profile the decision for large batches).
 *   launch 1: the statistics of every row and, when DAPD is on, the
 *             attention average, side by side in one grid;
 *   launch 2: Fast-dLLM, the DepCap boundary, CAP and the DAPD scores, each
 *             part in its own workgroups; the last scores workgroup of a
 *             sequence to finish (a per-sequence counter in the DAPD
 *             workspace, zeroed by launch 1) runs its DAPD selection.  With
 *             m_max <= 64, one workgroup per sequence scores and selects.
 * Each part computes what its own entry point computes.  The statistics are
 * those of dlm_step_stats to its stated accuracy (argmax identical; the
 * streaming order differs, so the floats may differ in the last bits), and
 * the outputs of each rule are bitwise those of dlm_fastdllm_select,
 * dlm_depcap_boundary, dlm_cap_select and dlm_dapd_select called on these
 * statistics with the same arguments.  A part is
 * skipped when its output pointer below is NULL.  The statistics part is
 * required.  Rows are the statistics rows in seq_offsets order (the same
 * CSR for every part, n_rows = seq_offsets[n_seq] by the caller's contract).
 * Arguments, limits and errors are those of the individual entry points;
 * the first invalid part makes the call return its error before any launch.
 */
typedef struct dlm_step_desc {
  /* statistics (dlm_step_stats) */
  const void* logits;
  const void* prev_logits; /* NULL: no KL */
  int32_t dtype;
  int64_t vocab, ld;
  const int64_t* row_index; /* NULL: rows 0..n_rows-1 in order */
  int64_t n_rows;
  float* conf;
  int32_t* argmax;
  float* entropy;
  float* kl; /* NULL iff prev_logits is NULL */
  float* lse;
  const int32_t* seq_offsets;
  int32_t n_seq;
  /* Fast-dLLM (dlm_fastdllm_select); skipped when fast_commit is NULL */
  const uint8_t* fast_eligible;
  float fast_tau;
  uint8_t* fast_commit;
  int32_t* fast_n_commit;
  /* DepGA-Block boundary (dlm_depcap_boundary); skipped when depcap_block_len is NULL */
  const uint8_t* depcap_has_prev;
  double depcap_lambda;
  int32_t depcap_l_min, depcap_l_max, depcap_radius;
  double depcap_eps;
  int32_t* depcap_block_len;
  double* depcap_score;
  /* CAP (dlm_cap_select); skipped when cap_commit is NULL */
  const uint8_t* cap_eligible;
  float cap_tau_low, cap_tau_high, cap_gamma;
  int32_t cap_k_max;
  uint8_t* cap_commit;
  int32_t* cap_n_commit;
  /* DAPD (dlm_dapd_select); skipped when dapd_commit is NULL */
  const void* attn;
  int32_t attn_dtype, n_lh;
  int64_t S, batch_stride;
  const int32_t* masked_pos;
  int32_t m_max;
  float dapd_tau;
  uint8_t* dapd_commit;
  int32_t* dapd_n_commit;
  void* dapd_workspace;        /* as dlm_dapd_select's; its per-sequence counters are
                                  zeroed by launch 1 and counted up in launch 2 */
  size_t dapd_workspace_bytes;
  /* optional hipEvent_t handles (created, timing enabled) that launch 1 sets
   * to its own start and end (hipExtLaunchKernel's start and stop events), to
   * time it; NULL: not set.  A failed launch returns DLM_ERR_HIP. */
  void* launch1_begin_event;
  void* launch1_end_event;
} dlm_step_desc;

int dlm_decide_step(const dlm_step_desc* desc, void* stream);

/* Human-readable text for a status code (static storage). */
const char* dlm_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* DLM_H */
