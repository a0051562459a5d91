/*
 * dlm_oracle.h — plain, slow fp64 CPU oracle for the per-step unmask decision
 * of masked diffusion language models.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no source,
 * header, table or helper with the HIP library; neither includes the other.
 *
 * Every function computes the plain definition from the pages (cited per
 * function in dlm_oracle.c) in IEEE double precision, with plain
 * left-to-right summation in index order.  Inputs in bf16 are widened
 * exactly (every bf16 value is a double).  Outputs are doubles.
 *
 * Conventions shared by all functions:
 *   - rows of a sequence are given in CSR form: seq_offsets[b] .. seq_offsets[b+1]-1
 *     index the per-row arrays (conf, argmax, ...), in position order;
 *   - a NULL `eligible` means every row is eligible;
 *   - return value 0 = ok, 1 = bad argument (nothing written).
 */
#ifndef DLM_ORACLE_H
#define DLM_ORACLE_H
#include <stdint.h>

#define DLMO_BF16 0
#define DLMO_F32 1

#ifdef __cplusplus
extern "C" {
#endif

/* Step statistics per logits row: conf, argmax, entropy (nats), KL(cur||prev)
 * (nats; only if prev != NULL, else kl may be NULL), lse.  Rows are
 * logits + row_index[r]*ld (elements).  n_threads <= 0 means 1. */
int dlmo_step_stats(const void* logits, const void* prev, int dtype, int64_t vocab,
                    int64_t ld, const int64_t* row_index, int64_t n_rows, double* conf,
                    int32_t* argmax, double* entropy, double* kl, double* lse, int n_threads);

/* Fast-dLLM confidence-threshold commit with top-1 fallback. */
int dlmo_fastdllm_select(const double* conf, const uint8_t* eligible,
                         const int32_t* seq_offsets, int32_t n_seq, double tau,
                         uint8_t* commit, int32_t* n_commit);

/* DepGA-Block scores S_k over each sequence's window W = min(l_max, rows).
 * score[] gets NaN outside the window and for cold-start sequences. */
int dlmo_depcap_scores(const double* kl, const double* entropy, const int32_t* seq_offsets,
                       int32_t n_seq, int32_t l_max, const uint8_t* has_prev, double lambda,
                       int32_t radius, double eps, double* score);
/* Boundary decision from given scores (oracle's own or externally supplied). */
int dlmo_depcap_decide(const double* score, const int32_t* seq_offsets, int32_t n_seq,
                       int32_t l_max, const uint8_t* has_prev, int32_t l_min,
                       int32_t* block_len);

/* CAP-Decoding, split into its three steps for one sequence of n rows.
 * pool: candidates sorted by (conf desc, local index asc), at most k_max,
 *       cand[] = local row indices; *fallback = local index of the top-1
 *       eligible row when the pool is empty (else -1; -1 also when nothing
 *       is eligible). */
int dlmo_cap_pool(const double* conf, const uint8_t* eligible, int32_t n, double tau_low,
                  int32_t k_max, int32_t* cand, int32_t* n_cand, int32_t* fallback);
/* D[a*ldd+b] = log p_a(yhat_b) + log p_b(yhat_a) over candidate rows
 * (row_index/argmax/lse indexed by the candidates' row numbers). Diagonal = NaN. */
int dlmo_cap_dmatrix(const void* logits, int dtype, int64_t vocab, int64_t ld,
                     const int64_t* row_index, const int32_t* argmax, const double* lse,
                     const int32_t* cand_rows, int32_t n_cand, double* D, int32_t ldd);
/* Greedy pick: cand_conf in candidate order, D with leading dimension ldd. */
int dlmo_cap_greedy(const double* cand_conf, const double* D, int32_t ldd, int32_t n_cand,
                    double tau_high, double gamma, uint8_t* take);
/* Whole CAP step over CSR sequences (pool + D + greedy + fallback).
 * cand_out [n_seq*k_max] global row numbers (-1 pad) and dmat_out
 * [n_seq*k_max*k_max] (NaN pad/diagonal) are optional. */
int dlmo_cap_select(const void* logits, int dtype, int64_t vocab, int64_t ld,
                    const int64_t* row_index, const int32_t* seq_offsets, int32_t n_seq,
                    const double* conf, const int32_t* argmax, const double* lse,
                    const uint8_t* eligible, double tau_low, double tau_high, double gamma,
                    int32_t k_max, uint8_t* commit, int32_t* n_commit, int32_t* cand_out,
                    double* dmat_out, int n_threads);

/* DAPD attention average for one sequence: a[i*M+j] = mean over the n_lh maps
 * of attn[lh][pos[i]][pos[j]] (maps are S x S, contiguous, map stride S*S). */
int dlmo_dapd_average(const void* attn, int dtype, int32_t n_lh, int64_t S,
                      const int32_t* pos, int32_t M, double* a);
/* Symmetrised scores s, proxy degree and ordering key for one sequence. */
int dlmo_dapd_graph(const double* a, int32_t M, const double* conf, double* s,
                    double* degree, double* key);
/* Welsh-Powell-ordered greedy independent set from s (ld_s) and key. */
int dlmo_dapd_greedy(const double* s, int32_t M, int64_t ld_s, double tau, const double* key,
                     uint8_t* take);
/* Whole DAPD step over CSR sequences.  attn points at sequence 0; sequence b
 * starts at attn + b*batch_stride elements.  degree/key are per row (CSR),
 * sym is [n_seq*m_max*m_max] (NaN pad); all three optional. */
int dlmo_dapd_select(const void* attn, int dtype, int32_t n_lh, int64_t S, int64_t batch_stride,
                     const int32_t* masked_pos, const int32_t* seq_offsets, int32_t n_seq,
                     const double* conf, double tau, uint8_t* commit, int32_t* n_commit,
                     double* degree, double* sym, int32_t m_max, double* key, int n_threads);

/* Fixed top-K per step (LLaDA's default schedule). */
int dlmo_topk_select(const double* conf, const uint8_t* eligible, const int32_t* seq_offsets,
                     int32_t n_seq, int32_t k, uint8_t* commit, int32_t* n_commit);
/* Factor decoding: largest n with (n+1)(1 - c(n)) < f; certificate optional. */
int dlmo_factor_select(const double* conf, const uint8_t* eligible, const int32_t* seq_offsets,
                       int32_t n_seq, double f, uint8_t* commit, int32_t* n_commit,
                       uint8_t* certificate);
/* Eligible rows of fixed-length block decoding: the earliest block with a mask. */
int dlmo_fixed_block_eligible(const int32_t* masked_pos, const int32_t* seq_offsets,
                              int32_t n_seq, const int32_t* gen_start, int32_t block_len,
                              uint8_t* eligible);
/* Full DAPD step: late-stage threshold switch and conf == 1 pre-unmask. */
int dlmo_dapd_step(const void* attn, int dtype, int32_t n_lh, int64_t S, int64_t batch_stride,
                   const int32_t* masked_pos, const int32_t* seq_offsets, int32_t n_seq,
                   const double* conf, double tau, const int32_t* gen_len, double late_frac,
                   double late_tau, int pre_unmask, uint8_t* commit, int32_t* n_commit,
                   uint8_t* stage, int n_threads);

#ifdef __cplusplus
}
#endif
#endif

