// Host-side launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.hpp"

namespace misa {

enum KernelId : int {
  K_POOL = 0,
  K_ROUTE_PARTIAL,
  K_ROUTE_SELECT,
  K_CLEAR,
  K_SCORE_MFMA,
  K_SCORE_F32,
  K_SCORE_PREFILL,
  K_TOPK_COLLECT,
  K_TOPK_FINAL,
  K_TOPK_ROW,
  K_PREFILL_SAMPLE,
  K_PREFILL_FULL,
  K_TOPK_TAU,
  K_TOPK_CAND,
  K_ROUTE_SPLIT,
  K_Q8_PREP,
  K_POOL_UPDATE,
  K_ATTN_SPLIT,
  K_ATTN_COMBINE,
  K_BLOCK_SCORE,
  K_EXPAND_BLOCKS,
  K_COUNT_IDS
};

// Kernel timing (only while misa_profile_begin is active): the launch goes
// through hipExtLaunchKernelGGL with a start/stop event pair, which the
// runtime stamps with the kernel's own start and end.
bool prof_events(int kernel_id, hipEvent_t* start, hipEvent_t* stop);

#define MISA_LAUNCH(kid, kernel, grid, block, lds, st, ...)                                  \
  do {                                                                                     \
    hipEvent_t misa_ev0_, misa_ev1_;                                                       \
    if (::misa::prof_events((kid), &misa_ev0_, &misa_ev1_))                                \
      hipExtLaunchKernelGGL((kernel), (grid), (block), (lds), (st), misa_ev0_, misa_ev1_, 0, \
                            __VA_ARGS__);                                                  \
    else                                                                                   \
      hipLaunchKernelGGL((kernel), (grid), (block), (lds), (st), __VA_ARGS__);             \
  } while (0)

// ---------------------------------------------------------------- pooling
struct PoolArgs {
  const void* k;
  const float* k_scale;
  int k_dt, S, L, d, B;
  float* kbar;
  KeyIndex kidx;
  // incremental mode (len_new != NULL): for each sequence s, only the blocks
  // completed by tokens len_old[s] .. len_new[s]-1 are written; at most
  // max_new tokens were appended to any sequence
  const int32_t* len_old = nullptr;
  const int32_t* len_new = nullptr;
  int max_new = 0;
};
hipError_t launch_pool(const PoolArgs& a, hipStream_t st);

// ---------------------------------------------------------------- router
struct RouteArgs {
  const void* q;
  int q_dt;
  const float* q_scale;  // e4m3 q: per-head scale [N, H_I] (folded into |w|), else NULL
  const float* w;
  const float* kbar;
  const void* k;
  const float* k_scale;
  int k_dt;
  const int32_t* q_seq;
  const int32_t* q_pos;
  int N, S, L, d, B, H_I, h;
  int32_t* heads;
  float* head_score;
  float* partial;        // workspace [N, nchunks, H_I]
  int nchunks;           // chunks of full blocks per row
  uint16_t* kb_split;    // workspace [2, M, d] bf16: pooled keys as hi + lo (one-sequence GEMM)
  KeyIndex kidx;         // where the keys of the partial block live
  // routed decode step (heads picked by the scoring kernel): only partials
  // [N, nchunks + 1, H_I] with the partial-block term in slot nchunks, no
  // selection kernel; hist0 (if not NULL), the scoring kernel's level-0
  // histogram [N, kHistWords], is cleared on the way.
  bool partials_only = false;
  uint32_t* hist0 = nullptr;
  // with partials_only: also pool the blocks completed by tokens
  // len_old[s] .. len_new[s] - 1 into kbar_out (= kbar), max_new bounding
  // len_new - len_old; the chunks pool such blocks for themselves
  const int32_t* len_old = nullptr;
  const int32_t* len_new = nullptr;
  int max_new = 0;
  float* kbar_out = nullptr;
};
int route_blocks_per_chunk();
bool route_uses_mfma(const RouteArgs& a);
hipError_t launch_route(const RouteArgs& a, hipStream_t st);

// ---------------------------------------------------------------- scoring
struct ScoreArgs {
  const void* q;
  int q_dt;
  const float* w;
  const void* k;
  const float* k_scale;
  int k_dt;
  const int32_t* q_seq;
  const int32_t* q_pos;     // row length L_n = q_pos[n] + 1 (NULL with cand)
  const int32_t* heads;     // [N, h] or NULL = all H_I heads
  const int32_t* cand;      // [N, ncols] token per element, -1 = empty; NULL = identity
  int N, S, L, d, H_I, h;
  int ncols;                // elements per row with cand
  uint32_t* u;              // [N, u_stride] order keys
  int u_stride;
  uint32_t* hist0;          // [N, kHistWords] level-0 histogram (NULL = skip)
  KeyIndex kidx;
  // routed decode step: the kernel picks each row's h heads itself from the
  // router's partials [N, route_nchunks + 1, H_I] (slot route_nchunks = the
  // partial-block term) before scoring, and workgroup 0 of each row writes
  // them to heads_out [N, h] (and r to head_score_out [N, H_I] if not NULL).
  // heads must be NULL then.  NULL route_partial: heads come from `heads`.
  const float* route_partial = nullptr;
  int route_nchunks = 0, B = 0;
  int32_t* heads_out = nullptr;
  float* head_score_out = nullptr;
};
hipError_t launch_score(const ScoreArgs& a, hipStream_t st);

// ---------------------------------------------------------------- fp8 queries
// e4m3 query heads -> exact bf16 copies qb [rows, d], and wq = w * q_scale
// [rows] (rows = N * H_I).  A positive head scale s gives
// w * ReLU(s * x) = (w * s) * ReLU(x) and |w| * s = |w * s|, so the kernels
// that read bf16 queries compute the fp8 problem from (qb, wq).
struct Q8PrepArgs {
  const uint8_t* q;
  const float* q_scale;
  const float* w;
  int64_t rows;
  int d;
  uint16_t* qb;
  float* wq;
};
hipError_t launch_q8_prep(const Q8PrepArgs& a, hipStream_t st);

// ---------------------------------------------------------------- prefill scoring
// Rows that all read one key sequence (bf16 q and keys, or e4m3 q and keys
// with their scales and d = 128): MFMA GEMM over the gathered routed head
// rows.
//  plain mode (cand_out NULL): writes order keys u[t, s] for s <= q_pos[t];
//    with key_step > 1 it scores only keys key_step*s' (s' <= q_pos[t] >>
//    pos_shift) and writes them to u[t, s'].  With block_flag, row blocks
//    whose flag is 0 are skipped.
//  candidate mode: writes no u; every visible (t, s) with score >= tau[t]
//    is appended as (score bits, s) to cand_out[(t * splits + split) * cap + slot]
//    (slots past cap are dropped) and cnt_out[t * splits + split] receives
//    the number of such keys (which may exceed cap).
struct PrefillArgs {
  const void* q;
  const float* w;
  const void* k;            // the key sequence [L, d] bf16
  const int32_t* q_pos;
  const int32_t* heads;     // [N, h] or NULL = all H_I heads
  int N, L, d, H_I, h;
  uint32_t* u;
  int u_stride;
  int key_step = 1;
  int pos_shift = 0;
  const uint32_t* block_flag = nullptr;
  const float* tau = nullptr;
  uint32_t* cnt_out = nullptr;
  uint2* cand_out = nullptr;
  int cap = 0;
  int kernel_id = K_SCORE_PREFILL;
  bool fp8 = false;                 // e4m3 q [N, H_I, d] and k [L, d] (d = 128)
  const float* q_scale = nullptr;   // fp8: [N, H_I]
  const float* k_scale = nullptr;   // fp8: [L]
};
int prefill_rows_per_block(int h_eff);
// key-range splits of the candidate-mode GEMM (the layout of cnt_out / cand_out)
int prefill_cand_splits(int N, int L, int h_eff, int d, bool fp8);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st);

// ---------------------------------------------------------------- top-k
struct TopkArgs {
  const uint32_t* u;
  int u_stride;
  const int32_t* q_pos;     // row length = q_pos[n] + 1, or fixed_len if NULL
  int fixed_len;
  int N, topk;
  bool one_row_per_block;
  uint32_t* hist;           // few-rows layout: [N, kHistWords] | bitmap | candidates
  const int32_t* cand;      // output index map (NULL = element index)
  int cand_stride;
  int32_t* idx;
  float* score;
  const uint32_t* row_flag = nullptr;   // one-row mode: rows whose flag is 0 are skipped
};
int topk_chunk();
// Rows of at most this many elements are selected by one workgroup holding
// the whole row in registers.
int topk_small_row();
size_t topk_few_rows_bytes(int N, int u_stride);
hipError_t launch_topk(const TopkArgs& a, hipStream_t st);
hipError_t launch_clear(uint32_t* p, size_t n_words, hipStream_t st);

// Sampled threshold per row (prefill candidate path): from the sample order
// keys us[n, 0 .. (q_pos[n] >> sample_shift)], a score tau[n] such that about
// 2 * min(topk, L_n) of the row's scores are expected at or above it.  Also
// clears block_flag[n / rows_per_block].
struct TauArgs {
  const uint32_t* us;
  int us_stride;
  const int32_t* q_pos;
  int N, topk, sample_shift, rows_per_block;
  float* tau;
  uint32_t* block_flag;
};
hipError_t launch_tau(const TauArgs& a, hipStream_t st);

// Exact top-k of each row from its candidate list (the scores >= tau[n]).  A row
// whose candidates cannot prove the result (a split list overflowed, fewer
// than min(topk, L_n) candidates, or more than the per-row capacity) is
// flagged in row_flag[n] and block_flag[n / rows_per_block] and left to the
// full path; other rows get idx/score written and row_flag[n] = 0.
struct CandTopkArgs {
  const uint32_t* cnt;
  const uint2* cand;
  int splits, cap;
  const int32_t* q_pos;
  int N, topk, rows_per_block;
  uint32_t* row_flag;
  uint32_t* block_flag;
  int32_t* idx;
  float* score;
};
int cand_topk_capacity();
hipError_t launch_cand_topk(const CandTopkArgs& a, hipStream_t st);

// ---------------------------------------------------------------- block prefilter
// Block scores of each row under its routed heads (complete blocks from the
// pooled table, a partial last block averaged from the keys) as order keys
// ub [N, ub_stride], and last_block[n] = ceil(L_n / B) - 1.
struct BlockScoreArgs {
  const void* q;
  int q_dt;
  const float* w;
  const float* kbar;
  const void* k;
  const float* k_scale;
  int k_dt;
  KeyIndex kidx;
  const int32_t* q_seq;
  const int32_t* q_pos;
  const int32_t* heads;
  int N, L, d, B, H_I, h;
  uint32_t* ub;
  int ub_stride;
  int32_t* last_block;
};
hipError_t launch_block_scores(const BlockScoreArgs& a, hipStream_t st);
// cand[n, i*B + t] = blocks[n, i] * B + t when that token is visible, else -1
hipError_t launch_expand_blocks(const int32_t* blocks, const int32_t* q_pos, int N, int m, int B,
                                int32_t* cand, hipStream_t st);

// ---------------------------------------------------------------- sparse attention
// Softmax attention of every head of each row over its selected tokens
// (idx [N, topk], -1 = empty); cache rows [.., d_qk] bf16 addressed through
// kidx, values = the first d_v elements of each row.  Splits of 64 selected
// tokens write partials (o_part [N, H, splits, d_v], ml_part [N, H, splits]
// float2) that a second kernel merges into out [N, H, d_v] and lse [N, H].
struct AttnArgs {
  const void* q;
  const void* kv;
  KeyIndex kidx;
  const int32_t* q_seq;
  const int32_t* idx;
  int N, H, d_qk, d_v, topk;
  float scale;
  float* o_part;
  void* ml_part;
  float* out;
  float* lse;
};
int attn_splits(int topk);
int attn_chunks_per_split(int topk);
hipError_t launch_attention(const AttnArgs& a, hipStream_t st);

}  // namespace misa
