/*
 * CPU oracle of the MISA routed indexer -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, obviously-correct host code in double precision.  It exists to
 * check the GPU library; only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load it.  It shares no source with the
 * GPU library and the GPU library never calls it.
 *
 * What it computes (per query row n, independently):
 *   L_n = q_pos[n] + 1 visible keys of sequence q_seq[n] (causal, inclusive).
 *   Block pooling: M_n = ceil(L_n / B) blocks; block b is the mean of the
 *     visible keys b*B .. min((b+1)*B, L_n) - 1 (a partial last block is the
 *     mean of its visible keys only).
 *     [MISA technical summary, gist.science, "Methodology" item 1: the prefix
 *      is split into M = ceil(L/B) blocks summarised by mean-pooled index keys]
 *   Router: r_j = |w_j| * sum_b ReLU(q_j . kbar_b); the routed set is the first
 *     h heads under (r desc, head index asc), returned in ascending order.
 *     [same page, "Methodology" item 1: per-head affinities against pooled
 *      keys, aggregated into a head importance, top-h kept; the exact
 *      affinity/aggregation is not printed on the pages -- this reading takes
 *      the indexer's own ReLU term at block granularity, weighted by |w_j|]
 *   Routed score: I(s) = sum_{j in routed, ascending} w_j * ReLU(q_j . k_s),
 *     s < L_n.  [DSA token-wise indexer score, named in the MISA abstract on the
 *     HF Daily Papers digest; "Methodology" item 2: only the routed heads score
 *     every prefix token]
 *   Top-k: the min(k, L_n) tokens first under (I desc, index asc).
 *   MISA-dagger rerank: candidates (a coarse top-k') are re-scored with all H_I
 *     heads and the top-k kept under (I_full desc, index asc).
 *     [same page, "Hierarchical variant (MISA-dagger)": coarse stage k' (e.g.
 *      8192), fine stage re-scores only the candidates with the full indexer]
 *   Dense DSA: routed score with every head (h = H_I).
 *
 * Inputs are decoded exactly: bf16 bit patterns widen to double; e4m3 codes
 * follow the OCP 8-bit floating point definition (bias 7, 3 mantissa bits,
 * subnormals, 0x7F/0xFF NaN) and are multiplied by their token's fp32 scale.
 *
 * All pointers are host pointers to C-contiguous arrays:
 *   q [N,H_I,d] (dt 0 = f32, 1 = bf16 bits, 2 = e4m3 codes), q_scale [N,H_I]
 *   f32 (e4m3 only, else NULL: head j of row n is q_scale[n,j] times its
 *   codes), w [N,H_I] f32,
 *   k [S,L,d] (dt 0 = f32, 1 = bf16 bits, 2 = e4m3 codes), k_scale [S,L] f32
 *   (e4m3 only, else NULL), q_seq [N], q_pos [N] int32.
 * Every function returns 0 on success, 1 for a NULL pointer, 2 for a shape or
 * range error (including q_pos/q_seq/cand out of range), 3 for an unsupported
 * dtype.  The MAC counters mac[4] are ADDED to (router MACs, scoring MACs,
 * rerank MACs, pooling adds); pass NULL to skip them.
 */
#ifndef MISA_REF_H
#define MISA_REF_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Decode rows*d stored values (dt 0/1/2) to double; scale[rows] is applied to
 * e4m3 rows (may be NULL for f32/bf16). */
int misa_ref_decode(const void* src, const float* scale, int dt, int64_t rows, int d,
                    double* out);

/* kbar[s,b,:] = mean of k[s, b*B .. min((b+1)*B, L)-1, :], table [S, ceil(L/B), d]. */
int misa_ref_pool_keys(const void* k, const float* k_scale, int k_dt, int S, int L, int d,
                       int B, double* kbar, uint64_t* mac);

/* heads [N,h] ascending; head_score [N,H_I] = r_j (may be NULL). */
int misa_ref_route_heads(const void* q, int q_dt, const float* q_scale, const float* w, const void* k,
                         const float* k_scale, int k_dt, const int32_t* q_seq,
                         const int32_t* q_pos, int N, int S, int L, int d, int B, int H_I,
                         int h, int32_t* heads, double* head_score, uint64_t* mac);

/* scores [N,L]: I(s) for s < L_n with the given heads [N,h] (heads == NULL means
 * all H_I heads, h ignored); -inf for s >= L_n. */
int misa_ref_scores(const void* q, int q_dt, const float* q_scale, const float* w, const void* k,
                    const float* k_scale, int k_dt, const int32_t* q_seq, const int32_t* q_pos,
                    const int32_t* heads, int N, int S, int L, int d, int H_I, int h,
                    double* scores, uint64_t* mac);

/* Top-k of the routed score: idx [N,topk] in (score desc, index asc) order,
 * score [N,topk]; slots past min(topk, L_n) hold -1 / -inf.  kth [N] is the
 * score of the last selected token (may be NULL). */
int misa_ref_score_topk(const void* q, int q_dt, const float* q_scale, const float* w, const void* k,
                        const float* k_scale, int k_dt, const int32_t* q_seq,
                        const int32_t* q_pos, const int32_t* heads, int N, int S, int L, int d,
                        int H_I, int h, int topk, int32_t* idx, double* score, double* kth,
                        uint64_t* mac);

/* Dense DSA indexer: misa_ref_score_topk with every head. */
int dsa_ref_score_topk(const void* q, int q_dt, const float* q_scale, const float* w, const void* k,
                       const float* k_scale, int k_dt, const int32_t* q_seq,
                       const int32_t* q_pos, int N, int S, int L, int d, int H_I, int topk,
                       int32_t* idx, double* score, double* kth, uint64_t* mac);

/* MISA-dagger fine stage: cand [N,k_prime] token indices (-1 = empty slot;
 * valid entries distinct and < L_n) re-scored with all H_I heads; top-k as
 * above. */
int misa_ref_rerank(const void* q, int q_dt, const float* q_scale, const float* w, const void* k,
                    const float* k_scale, int k_dt, const int32_t* q_seq, const int32_t* q_pos,
                    const int32_t* cand, int N, int S, int L, int d, int H_I, int k_prime,
                    int topk, int32_t* idx, double* score, double* kth, uint64_t* mac);

/* Routed scoring with a block prefilter: head routing composed with a
 * token-axis hierarchy (the MISA pages call head-axis routing complementary
 * to token-axis hierarchies, technical summary "Key contributions"; HISA,
 * gonzo_ML TL;DR: a coarse block-level filter, then token-level refinement
 * that keeps the exact top-k output).  For row n with routed heads
 * heads[n,:]:
 *   block b (b < M_n = ceil(L_n / B)) has the key mean of the row's visible
 *   keys b*B .. min((b+1)*B, L_n) - 1 and the score
 *   I_blk(b) = sum_{j routed} w_j ReLU(q_j . mean_b);
 *   the m_blocks blocks first under (I_blk desc, block asc) are kept and
 *   listed ascending in blocks [N, m_blocks] (-1 padding);
 *   the top-k (score desc, index asc) of the routed token scores over the
 *   kept blocks' visible tokens goes to idx/score [N, topk] (-1 / -inf pad). */
int misa_ref_score_topk_blocks(const void* q, int q_dt, const float* q_scale, const float* w,
                               const void* k, const float* k_scale, int k_dt,
                               const int32_t* q_seq, const int32_t* q_pos, const int32_t* heads,
                               int N, int S, int L, int d, int B, int H_I, int h, int m_blocks,
                               int topk, int32_t* blocks, int32_t* idx, double* score);

/* Sparse attention over the selected tokens (the consumer of the top-k: the
 * indexer picks the tokens the main attention reads [MISA abstract, HF Daily
 * Papers digest; technical summary, "Problem statement"]; the attention
 * itself is ordinary softmax attention, not specified by the pages).
 * For row n, head h and the valid tokens T_n = {idx[n,i] >= 0} (distinct,
 * < L) of sequence q_seq[n]:
 *   s_t = scale * q[n,h,:] . kv[q_seq[n], t, 0:d_qk]
 *   out[n,h,:] = sum_t exp(s_t - m) kv[q_seq[n], t, 0:d_v] / sum_t exp(s_t - m),
 *   m = max_t s_t,   lse[n,h] = m + log(sum_t exp(s_t - m))
 * Value rows are the first d_v elements of the same cache rows (latent
 * attention's shared key/value rows).  q [N,H,d_qk], kv [S,L,d_qk] (dt 0 =
 * f32, 1 = bf16 bits); out [N,H,d_v], lse [N,H] doubles.  A row without a
 * valid token gets out = 0, lse = -inf. */
int misa_ref_sparse_attention(const void* q, int q_dt, const void* kv, int kv_dt,
                              const int32_t* q_seq, const int32_t* idx, int N, int S, int L,
                              int H, int d_qk, int d_v, int topk, double scale, double* out,
                              double* lse);

/* Threads the OpenMP runtime will use. */
int misa_ref_max_threads(void);

/* Threads for the calling thread's later calls (n > 0; timing of the
 * one-thread baseline). */
void misa_ref_set_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
