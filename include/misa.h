/*
 * misa.h -- C ABI of the MISA routed indexer for AMD MI355X (gfx950).
 *
 * MISA (Mixture of Indexer Sparse Attention) is a drop-in replacement for the
 * token indexer of DeepSeek Sparse Attention (DSA).  DSA's indexer scores every
 * prefix token with all H_I indexer heads and keeps one shared top-k token set
 * for the main attention (MISA abstract, HF Daily Papers digest).  MISA keeps
 * only h of the H_I heads per query, chosen by a light router over
 * block-pooled keys, so the per-query cost drops from O(H_I L) to
 * O(h L + H_I M) with M = ceil(L/B) (MISA technical summary, gist.science,
 * "Methodology" items 1-2).  MISA-dagger re-scores a wider routed candidate
 * set of k' tokens with all H_I heads to recover the final top-k
 * ("Hierarchical variant (MISA-dagger)").
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - All array pointers are DEVICE pointers to C-contiguous row-major memory
 *    owned by the caller.  The library allocates and frees no device memory;
 *    scratch space is the caller's workspace `ws` of `ws_bytes` bytes
 *    (size it with misa_workspace_bytes; it needs no initialisation and is
 *    overwritten).  The library keeps no pointer after a call returns.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    asynchronously; outputs are valid once the stream has synchronised.
 *  - Layouts:
 *      q       [N, H_I, d]  dtype q_dt (MISA_F32, MISA_BF16 or MISA_FP8_E4M3)
 *      q_scale [N, H_I]     float32 per-head scale, required iff q_dt is fp8
 *                           (head j of row n = q_scale[n,j] * its e4m3
 *                           values; scale > 0), else ignored (may be NULL)
 *      w       [N, H_I]     float32 head weights
 *      k       [S, L, d]    dtype k_dt (MISA_F32, MISA_BF16 or MISA_FP8_E4M3)
 *      k_scale [S, L]       float32 per-token scale, required iff k_dt is fp8
 *                           (key value = scale * e4m3 value; scale > 0)
 *    Paged keys (every entry point that reads k takes block_table, page_size
 *    right after k_dt): page_size 0 means the contiguous layout above and
 *    block_table must be NULL.  Otherwise keys live in a page pool
 *      k       [P, page_size, d], k_scale [P, page_size] (fp8)
 *      block_table [S, ceil(L / page_size)] int32: physical page of each
 *                  logical page of each sequence; token t of sequence s is
 *                  row t % page_size of page block_table[s][t / page_size]
 *    with page_size a power of two in [16, 65536] and L the per-sequence
 *    capacity in tokens.  Entries are read only for pages that hold tokens a
 *    call can see (t <= q_pos[n], or the tokens being pooled); they must be
 *    valid page numbers of the pool (device-resident: not checked).  Many
 *    rows over one paged sequence take the per-row scoring kernels (the
 *    prefill GEMM reads contiguous keys only).
 *      q_seq   [N]  int32   key sequence of query row n, 0 <= q_seq[n] < S
 *      q_pos   [N]  int32   position of query row n, 0 <= q_pos[n] < L;
 *                           row n sees keys 0..q_pos[n] (L_n = q_pos[n] + 1)
 *    Supported (q_dt, k_dt): (F32, F32), (BF16, BF16), (BF16, FP8_E4M3),
 *    (FP8_E4M3, FP8_E4M3) (e4m3 as in the OCP 8-bit floating point format:
 *    bias 7, max 448, no infinities); d in {64, 128}; 1 <= h <= H_I <= 64; 1 <= B <= 1024;
 *    1 <= topk <= 65536; 1 <= N <= 65535; 1 <= S <= 65535; 1 <= L <= 2^27.
 *  - Index-score: I(s) = sum over heads j of w[n,j] * ReLU(q[n,j,:] . key_s),
 *    accumulated in fp32 from exact bf16 (or fp8-dequantised) products.
 *    Exception: fp8 queries on the many-rows path (S = 1, N >= 128,
 *    d = 128) are scored by the e4m3 matrix cores
 *    (v_mfma_f32_16x16x128_f8f6f4), which sum each group of 8 consecutive
 *    products after truncating every product toward zero to a multiple of
 *    2^(E - 13), E the group's largest exponent sum e(q) + e(k) of the codes
 *    (measured on gfx950).  Those scores carry that rounding on top of fp32;
 *    fp8 queries on every other path are scored exactly like bf16 ones.
 *  - Top-k outputs idx [N, topk] int32 and score [N, topk] float32 hold the
 *    min(topk, L_n) tokens first under (score desc, token index asc), listed
 *    in ASCENDING TOKEN INDEX order, followed by -1 / -inf padding.
 *  - Errors: host-checkable arguments are validated before anything is
 *    enqueued; a failed check returns its status and launches nothing.  A HIP
 *    launch failure returns MISA_ERR_HIP (see misa_last_hip_error).
 *    Device-resident values (q_seq, q_pos, heads, cand, idx of the attention,
 *    len_old / len_new) are preconditions and are NOT read on the host in
 *    normal use: out-of-range values there are undefined behaviour.
 *  - Debug validation: with the environment variable MISA_DEBUG_SYNC set to
 *    "1" (read at every call), each entry point first synchronises `stream`,
 *    copies those device-resident arguments to the host and checks them:
 *    0 <= q_seq[n] < S, 0 <= q_pos[n] < L; heads distinct in [0, H_I);
 *    cand entries -1 or in [0, L_n) with the valid ones strictly ascending;
 *    attention idx entries -1 or distinct in [0, L); 0 <= len_old[s] <=
 *    len_new[s] <= L with len_new - len_old <= max_new.  A violation returns
 *    MISA_ERR_SHAPE before anything is launched (outputs untouched).
 *    Block-table entries are never checked (the pool size is not an
 *    argument).  The synchronisation makes this a debugging aid only.
 *  - The library keeps no state between calls except the kernel-timing
 *    records of misa_profile_begin/end, which belong to the calling host
 *    thread; calls from several threads on different streams are safe.
 */
#ifndef MISA_H
#define MISA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MISA_F32 = 0, MISA_BF16 = 1, MISA_FP8_E4M3 = 2 } misa_dtype;

typedef enum {
  MISA_OK = 0,
  MISA_ERR_NULL = 1,        /* a required pointer is NULL */
  MISA_ERR_SHAPE = 2,       /* a size or size relation is out of range */
  MISA_ERR_UNSUPPORTED = 3, /* dtype combination or d not supported */
  MISA_ERR_WORKSPACE = 4,   /* ws_bytes smaller than misa_workspace_bytes */
  MISA_ERR_HIP = 5          /* the HIP runtime reported an error */
} misa_status;

typedef enum {
  MISA_OP_ROUTE = 0,        /* misa_route_heads */
  MISA_OP_SCORE_TOPK = 1,   /* misa_score_topk (also dsa_score_topk) */
  MISA_OP_RERANK = 2,       /* misa_rerank */
  MISA_OP_ATTENTION = 3,    /* misa_sparse_attention (d = d_v, H_I = heads) */
  MISA_OP_BLOCKS = 4,       /* misa_score_topk_blocks (k_prime = m_blocks) */
  MISA_OP_ROUTE_SCORE_TOPK = 5  /* misa_route_score_topk */
} misa_op;

/*
 * Block pooling (MISA technical summary, "Methodology" item 1: the prefix is
 * split into M = ceil(L/B) blocks summarised by mean-pooled index keys).
 *   kbar[s, b, :] = mean of key rows b*B .. min((b+1)*B, L) - 1 of sequence s
 * Output kbar [S, ceil(L/B), d] float32 (fp32 accumulation).  The last block
 * may be partial.  The table is causal only for rows that see all L keys;
 * misa_route_heads handles each row's own partial block.
 */
int32_t misa_pool_keys(const void* k, const float* k_scale, int32_t k_dt,
                       const int32_t* block_table, int32_t page_size, int32_t S, int32_t L,
                       int32_t d, int32_t B, float* kbar, void* stream);

/*
 * Incremental block pooling for a decode loop that appends tokens to its key
 * cache (same page, "Methodology" item 1: the router works on block means, at
 * O(H_I M) per query).  The router reads only the blocks a row sees
 * completely and computes the row's partial last block from k itself, so a
 * cached table needs only complete blocks.  For every sequence s this writes
 * kbar[s, b] (as misa_pool_keys would) for exactly the blocks b completed by
 * the tokens len_old[s] .. len_new[s]-1, i.e. those with
 * len_old[s] < (b+1)*B <= len_new[s]; other rows of kbar are not touched.
 * len_old, len_new: [S] int32 device arrays with 0 <= len_old <= len_new <= L;
 * max_new >= len_new[s] - len_old[s] for every s (host bound that sizes the
 * launch; 0 = nothing to do).  Cost: O(B d) per completed block.
 */
int32_t misa_pool_update(const void* k, const float* k_scale, int32_t k_dt,
                         const int32_t* block_table, int32_t page_size, int32_t S, int32_t L,
                         int32_t d, int32_t B, const int32_t* len_old, const int32_t* len_new,
                         int32_t max_new, float* kbar, void* stream);

/*
 * Head router (same page, "Methodology" item 1: per-head affinities against
 * the pooled keys, aggregated into a head importance, top-h heads kept; the
 * router costs O(H_I M)).  The pages do not print the affinity formula; this
 * library takes the indexer's own term at block granularity:
 *   r[n, j] = |w[n,j]| * sum_{b < M_n} ReLU(q[n,j,:] . kbar_n[b])
 * with M_n = ceil(L_n / B); blocks fully visible to row n come from the
 * pooled table kbar [S, ceil(L/B), d] (from misa_pool_keys); a partial last
 * block is the mean of row n's visible keys of that block only, read from k.
 * heads [N, h] receives the first h heads under (r desc, head index asc),
 * sorted ascending; head_score [N, H_I] receives r (may be NULL).
 * Workspace: misa_workspace_bytes(MISA_OP_ROUTE, ...).
 */
int32_t misa_route_heads(const void* q, int32_t q_dt, const float* q_scale, const float* w,
                         const float* kbar, const void* k, const float* k_scale, int32_t k_dt,
                         const int32_t* block_table, int32_t page_size, const int32_t* q_seq,
                         const int32_t* q_pos, int32_t N, int32_t S, int32_t L, int32_t d,
                         int32_t B, int32_t H_I, int32_t h, int32_t* heads, float* head_score,
                         void* ws, size_t ws_bytes, void* stream);

/*
 * Routed token scoring + top-k (same page, "Methodology" item 2: only the h
 * routed heads score every prefix token; the top-k tokens are taken from
 * these reduced scores).  heads [N, h] are head indices in [0, H_I) (any
 * order, distinct), normally the output of misa_route_heads.
 *   I_n(s) = sum_{j in heads[n]} w[n,j] * ReLU(q[n,j,:] . key_{q_seq[n]}(s)),
 *   s = 0 .. q_pos[n]
 * Outputs idx/score as described in the conventions (score may be NULL).
 * Workspace: misa_workspace_bytes(MISA_OP_SCORE_TOPK, ...).
 */
int32_t misa_score_topk(const void* q, int32_t q_dt, const float* q_scale, const float* w,
                        const void* k, const float* k_scale, int32_t k_dt,
                        const int32_t* block_table, int32_t page_size, const int32_t* q_seq,
                        const int32_t* q_pos, const int32_t* heads, int32_t N, int32_t S,
                        int32_t L, int32_t d, int32_t H_I, int32_t h, int32_t topk,
                        int32_t* idx, float* score, void* ws, size_t ws_bytes, void* stream);

/*
 * Head router + routed token scoring + top-k in one call (the two steps of
 * the same page's "Methodology", items 1 and 2): the same results as
 * misa_route_heads followed by misa_score_topk, bit for bit.  heads [N, h]
 * (required) and head_score [N, H_I] (may be NULL) receive the router's
 * outputs; idx/score the top-k.  For decode rows with bf16 queries and bf16 or
 * e4m3 keys (not one sequence with N >= 128) the selection of the heads runs
 * at the start of the scoring kernel, so the step launches two kernels fewer;
 * otherwise the two calls run in turn.  All other arguments, layouts and
 * errors are those of the two calls.
 * Workspace: misa_workspace_bytes(MISA_OP_ROUTE_SCORE_TOPK, q_dt, N, L, d, H_I,
 * B, topk, 0).
 */
int32_t misa_route_score_topk(const void* q, int32_t q_dt, const float* q_scale, const float* w,
                              const float* kbar, const void* k, const float* k_scale,
                              int32_t k_dt, const int32_t* block_table, int32_t page_size,
                              const int32_t* q_seq, const int32_t* q_pos, int32_t N, int32_t S,
                              int32_t L, int32_t d, int32_t B, int32_t H_I, int32_t h,
                              int32_t topk, int32_t* heads, float* head_score, int32_t* idx,
                              float* score, void* ws, size_t ws_bytes, void* stream);

/*
 * One decode serving step (the same page, "Methodology" items 1 and 2): the
 * incremental pooling of misa_pool_update (kbar [S, ceil(L/B), d], read and
 * written: the blocks completed by tokens len_old[s] .. len_new[s] - 1),
 * then misa_route_score_topk on the updated table, with the same results bit
 * for bit, the written kbar entries included.  For the decode rows that
 * misa_route_score_topk fuses (bf16 queries, bf16 or e4m3 keys, not one
 * sequence with N >= 128) the pooling runs inside the router's launch: the
 * router's workgroups that need a block completed by this call pool it
 * themselves with the pooling kernel's arithmetic, and further workgroups of
 * the same launch write the table, so the step has no separate pooling
 * launch; otherwise the calls run in turn.  Arguments, layouts, errors and
 * the workspace (misa_workspace_bytes(MISA_OP_ROUTE_SCORE_TOPK, ...)) are
 * those of the two calls; nothing runs if any check of either fails.
 */
int32_t misa_pool_route_score_topk(const void* q, int32_t q_dt, const float* q_scale,
                                   const float* w, float* kbar, const void* k,
                                   const float* k_scale, int32_t k_dt, const int32_t* block_table,
                                   int32_t page_size, const int32_t* q_seq, const int32_t* q_pos,
                                   const int32_t* len_old, const int32_t* len_new, int32_t max_new,
                                   int32_t N, int32_t S, int32_t L, int32_t d, int32_t B,
                                   int32_t H_I, int32_t h, int32_t topk, int32_t* heads,
                                   float* head_score, int32_t* idx, float* score, void* ws,
                                   size_t ws_bytes, void* stream);

/*
 * misa_pool_route_score_topk for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments, results and errors, without ws/ws_bytes.
 * Its scratch is a 32 MiB array the library holds on every GPU it runs on
 * (until the process ends); a call whose workspace
 * (misa_workspace_bytes(MISA_OP_ROUTE_SCORE_TOPK, ...)) exceeds 32 MiB
 * returns MISA_ERR_WORKSPACE and launches nothing.  It calls no allocation
 * routine (MISA_DEBUG_SYNC=1 copies its checks' inputs to host memory).
 * Every call on one GPU uses that GPU's array: calls that overlap on one GPU
 * (concurrent streams, several host threads) race and must be serialised by
 * the caller.
 */
int32_t misa_pool_route_score_topk_scratch(
    const void* q, int32_t q_dt, const float* q_scale, const float* w, float* kbar, const void* k,
    const float* k_scale, int32_t k_dt, const int32_t* block_table, int32_t page_size,
    const int32_t* q_seq, const int32_t* q_pos, const int32_t* len_old, const int32_t* len_new,
    int32_t max_new, int32_t N, int32_t S, int32_t L, int32_t d, int32_t B, int32_t H_I,
    int32_t h, int32_t topk, int32_t* heads, float* head_score, int32_t* idx, float* score,
    void* stream);

/*
 * Dense DSA indexer (the baseline MISA replaces: every one of the H_I heads
 * scores every prefix token, MISA abstract and "Problem statement"):
 * misa_score_topk with all H_I heads.
 */
int32_t dsa_score_topk(const void* q, int32_t q_dt, const float* q_scale, const float* w,
                       const void* k, const float* k_scale, int32_t k_dt,
                       const int32_t* block_table, int32_t page_size, const int32_t* q_seq,
                       const int32_t* q_pos, int32_t N, int32_t S, int32_t L, int32_t d,
                       int32_t H_I, int32_t topk, int32_t* idx, float* score, void* ws,
                       size_t ws_bytes, void* stream);

/*
 * MISA-dagger fine stage (same page, "Hierarchical variant (MISA-dagger)":
 * the routed pass keeps a wider candidate set of k' tokens, e.g. 8192, and the
 * original DSA indexer with all H_I heads re-scores only those candidates to
 * recover the final top-k).
 * cand [N, k_prime] int32: candidate token indices of row n, each < L_n, the
 * valid ones strictly ascending, -1 marking empty slots (the idx output of
 * misa_score_topk with topk = k_prime has exactly this form).
 * Outputs idx/score [N, topk] as in the conventions, over the valid
 * candidates, ranked by the all-head score.  Requires topk <= k_prime.
 * Workspace: misa_workspace_bytes(MISA_OP_RERANK, ...).
 */
int32_t misa_rerank(const void* q, int32_t q_dt, const float* q_scale, const float* w,
                    const void* k, const float* k_scale, int32_t k_dt, const int32_t* block_table,
                    int32_t page_size, const int32_t* q_seq, const int32_t* q_pos,
                    const int32_t* cand, int32_t N, int32_t S, int32_t L, int32_t d, int32_t H_I,
                    int32_t k_prime, int32_t topk, int32_t* idx, float* score, void* ws,
                    size_t ws_bytes, void* stream);

/*
 * Routed scoring behind a block prefilter: head routing composed with a
 * token-axis hierarchy (the MISA pages call head-axis routing complementary
 * to token-axis hierarchies, technical summary "Key contributions"; HISA,
 * gonzo_ML TL;DR: a coarse block-level filter, then token-level refinement
 * that keeps the exact top-k output).  For row n with routed heads heads[n,:]:
 *   block b < M_n = ceil(L_n / B) has key kbar (complete blocks: the pooled
 *   table from misa_pool_keys / misa_pool_update; a partial last block: the
 *   mean of the row's visible keys of that block, read from k) and score
 *   I_blk(b) = sum_{j routed} w[n,j] * ReLU(q[n,j,:] . kbar_b);
 *   the m_blocks blocks first under (I_blk desc, block asc) are kept; blocks
 *   [N, m_blocks] (may be NULL) receives them ascending, -1 padded;
 *   idx/score [N, topk] receive the routed top-k (as misa_score_topk) over the
 *   kept blocks' visible tokens.
 * m_blocks >= M_n gives exactly misa_score_topk's result.  Requires
 * m_blocks * B <= 65536 and 1 <= topk <= m_blocks * B.  Cost per row:
 * O(h M d) for the block scores plus O(h m_blocks B d) token scoring, instead
 * of O(h L d).  Workspace: misa_workspace_bytes(MISA_OP_BLOCKS, q_dt, N, L, d,
 * H_I, B, topk, m_blocks).
 */
int32_t misa_score_topk_blocks(const void* q, int32_t q_dt, const float* q_scale, const float* w,
                               const float* kbar, const void* k, const float* k_scale,
                               int32_t k_dt, const int32_t* block_table, int32_t page_size,
                               const int32_t* q_seq, const int32_t* q_pos, const int32_t* heads,
                               int32_t N, int32_t S, int32_t L, int32_t d, int32_t B,
                               int32_t H_I, int32_t h, int32_t m_blocks, int32_t topk,
                               int32_t* blocks, int32_t* idx, float* score, void* ws,
                               size_t ws_bytes, void* stream);

/*
 * Sparse attention over the selected tokens: the consumer of the top-k (the
 * indexer picks the tokens the main attention reads, MISA abstract and
 * "Problem statement"; the attention itself is ordinary softmax attention,
 * which the pages do not specify).  For row n, head h and the valid entries
 * t of idx[n, :] (-1 = empty; distinct tokens of sequence q_seq[n]):
 *   s_t = scale * q[n,h,:] . kv_t[0:d_qk],  m = max_t s_t,
 *   out[n,h,:] = sum_t exp(s_t - m) kv_t[0:d_v] / sum_t exp(s_t - m),
 *   lse[n,h] = m + log(sum_t exp(s_t - m))   (natural log)
 * Values are the first d_v elements of the same cache rows (multi-head latent
 * attention's shared key/value cache).  A row without a valid entry gets
 * out = 0 and lse = -inf.
 *   q   [N, H, d_qk] bf16 (q_dt = MISA_BF16); kv: cache rows of d_qk bf16
 *       (kv_dt = MISA_BF16), contiguous [S, L, d_qk] or paged through
 *       block_table/page_size exactly like keys (see the conventions)
 *   idx [N, topk] int32 (e.g. the idx output of misa_score_topk)
 *   out [N, H, d_v] float32, lse [N, H] float32; scale > 0
 *   d_qk in {64, 128, 256, 576}; d_v a multiple of 32, 32 <= d_v <= min(512, d_qk);
 *   1 <= H <= 1024.  Entries of idx are device-resident: not checked.
 * Accuracy: fp32 dot products of exact bf16 products; the probabilities are
 * carried as bf16 hi + lo pairs into the value products (~2^-17 relative).
 * Workspace: misa_workspace_bytes(MISA_OP_ATTENTION, q_dt, N, L, d_v, H, 0,
 * topk, 0).
 */
int32_t misa_sparse_attention(const void* q, int32_t q_dt, const void* kv, int32_t kv_dt,
                              const int32_t* block_table, int32_t page_size,
                              const int32_t* q_seq, const int32_t* idx, int32_t N, int32_t S,
                              int32_t L, int32_t H, int32_t d_qk, int32_t d_v, int32_t topk,
                              float scale, float* out, float* lse, void* ws, size_t ws_bytes,
                              void* stream);

/*
 * Workspace bytes for `op` at these sizes with queries of dtype q_dt (0 for
 * invalid sizes or dtype).  Arguments an op does not use are ignored
 * (k_prime only matters for MISA_OP_RERANK, B only for MISA_OP_ROUTE).  For
 * MISA_OP_SCORE_TOPK with many rows over one long sequence (N >= 128,
 * L >= 32768, topk <= 2048) the size includes the region of the
 * sampled-threshold candidate path; for bf16 queries a workspace that only
 * covers the full path (the size for topk > 2048) is accepted too, and then
 * that path runs.  fp8 queries add N * H_I * (2d + 4) bytes (rounded up) for
 * their bf16 copies and folded weights on the paths that read bf16 queries.
 */
size_t misa_workspace_bytes(int32_t op, int32_t q_dt, int32_t N, int32_t L, int32_t d,
                            int32_t H_I, int32_t B, int32_t topk, int32_t k_prime);

/*
 * Diagnostic of the prefill candidate path (rows sharing one contiguous key
 * sequence with N >= 128, L >= 32768, topk <= 2048, see
 * misa_workspace_bytes): a misa_score_topk or dsa_score_topk call that takes
 * it leaves one uint32 flag per row in its workspace, at this byte offset:
 * 1 when the row's sampled threshold could not prove its top-k and the row
 * was re-scored in full, else 0.  Returns -1 when calls at these sizes do not
 * take that path.
 */
int64_t misa_candidate_flags_offset(int32_t N, int32_t L, int32_t topk);

/* Static description of a status code. */
const char* misa_status_string(int32_t status);

/* hipError_t of the last MISA_ERR_HIP on the calling thread (0 if none). */
int32_t misa_last_hip_error(void);

/*
 * Kernel timing for benchmarks.  misa_profile_begin(capacity) creates
 * `capacity` pairs of HIP events (host-side allocation happens here, not in
 * the timed calls) and from then on launches every kernel of the library
 * with an event pair (hipExtLaunchKernelGGL) that the runtime stamps with the
 * kernel's own start and end on its stream, until capacity is used up or
 * misa_profile_end is called.  misa_profile_end
 * synchronises the recorded events and writes up to `max` records:
 * kernel_id[i] (see misa_kernel_name) and ms[i], the elapsed time between the
 * pair.  It returns the number of records written (negative on error) and
 * frees the events.  The profiling state belongs to the calling host
 * thread: only launches made by that thread are timed.
 */
int32_t misa_profile_begin(int32_t capacity);
int32_t misa_profile_end(int32_t* kernel_id, float* ms, int32_t max);
const char* misa_kernel_name(int32_t kernel_id);

#ifdef __cplusplus
}
#endif
#endif /* MISA_H */
