// C ABI of the MISA indexer library: argument validation, workspace layout,
// dispatch to the gfx950 kernels, kernel timing.  See include/misa.h for the
// contract of every entry point.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <mutex>
#include <utility>
#include <vector>

#include "common.hpp"
#include "kernels.hpp"
#include "misa.h"

namespace {

thread_local int32_t g_last_hip = 0;

constexpr int kMaxN = 65535;          // grid y limit
constexpr int kMaxL = 1 << 27;
constexpr int kMaxTopk = 65536;
constexpr int kOneRowMinN = 128;      // rows at which one workgroup per row fills the chip
// prefill candidate path: sampled threshold from every 32nd key
constexpr int kSampleShift = 5;
constexpr int kCandMinL = 32768;      // shorter sequences keep the full path
constexpr int kCandMaxTopk = 2048;    // about 2 topk candidates must fit the LDS select
constexpr int kCandRegion = 16384;    // candidate slots per row, shared evenly by the splits
constexpr int kMaxSplits = 256;
constexpr int kMaxAttnHeads = 1024;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int32_t hip_status(hipError_t e) {
  if (e == hipSuccess) return MISA_OK;
  g_last_hip = static_cast<int32_t>(e);
  return MISA_ERR_HIP;
}

int32_t check_dtypes(int32_t q_dt, int32_t k_dt, const float* q_scale, const float* k_scale) {
  const bool ok = (q_dt == MISA_F32 && k_dt == MISA_F32) ||
                  (q_dt == MISA_BF16 && k_dt == MISA_BF16) ||
                  (q_dt == MISA_BF16 && k_dt == MISA_FP8_E4M3) ||
                  (q_dt == MISA_FP8_E4M3 && k_dt == MISA_FP8_E4M3);
  if (!ok) return MISA_ERR_UNSUPPORTED;
  if (k_dt == MISA_FP8_E4M3 && !k_scale) return MISA_ERR_NULL;
  if (q_dt == MISA_FP8_E4M3 && !q_scale) return MISA_ERR_NULL;
  return MISA_OK;
}

int32_t check_sizes(int32_t N, int32_t S, int32_t L, int32_t d, int32_t H_I) {
  if (d != 64 && d != 128) return MISA_ERR_UNSUPPORTED;
  if (N < 1 || N > kMaxN || S < 1 || S > kMaxN || L < 1 || L > kMaxL) return MISA_ERR_SHAPE;
  if (H_I < 1 || H_I > 64) return MISA_ERR_SHAPE;
  return MISA_OK;
}

// Key storage: page_size 0 = contiguous [S, L, d] (block_table must be NULL);
// otherwise pages of page_size tokens (a power of two, 16 .. 65536) listed
// per sequence by block_table [S, ceil(L / page_size)].
int32_t key_index(const int32_t* block_table, int32_t page_size, int32_t L, misa::KeyIndex& ki) {
  ki = misa::KeyIndex{nullptr, L, 0, 0};
  if (page_size == 0) return block_table ? MISA_ERR_SHAPE : MISA_OK;
  if (!block_table) return MISA_ERR_NULL;
  if (page_size < 16 || page_size > 65536 || (page_size & (page_size - 1))) return MISA_ERR_SHAPE;
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  ki = misa::KeyIndex{block_table, L, shift, (L + page_size - 1) >> shift};
  return MISA_OK;
}

int32_t check_pool(const void* k, const float* k_scale, int32_t k_dt, int32_t S, int32_t L,
                   int32_t d, int32_t B, const float* kbar) {
  if (!k || !kbar) return MISA_ERR_NULL;
  if (k_dt != MISA_F32 && k_dt != MISA_BF16 && k_dt != MISA_FP8_E4M3) return MISA_ERR_UNSUPPORTED;
  if (k_dt == MISA_FP8_E4M3 && !k_scale) return MISA_ERR_NULL;
  if (d != 64 && d != 128) return MISA_ERR_UNSUPPORTED;
  if (S < 1 || S > kMaxN || L < 1 || L > kMaxL || B < 1 || B > 1024) return MISA_ERR_SHAPE;
  if (!aligned16(k)) return MISA_ERR_SHAPE;
  return MISA_OK;
}

// ---------------------------------------------------------------- workspace layouts
struct TopkLayout {
  bool one_row = false;
  int u_stride = 0;
  size_t off_hist = 0, bytes = 0;
};

TopkLayout topk_layout(int N, int len_max) {
  TopkLayout t;
  const int chunk = misa::topk_chunk();
  t.u_stride = static_cast<int>(align_up(static_cast<size_t>(len_max), chunk));
  // many rows, or rows short enough for one workgroup's registers
  t.one_row = N >= kOneRowMinN || t.u_stride <= misa::topk_small_row();
  size_t off = align_up(static_cast<size_t>(N) * t.u_stride * 4, 256);
  if (!t.one_row) {
    t.off_hist = off;
    off = align_up(off + misa::topk_few_rows_bytes(N, t.u_stride), 256);
  }
  t.bytes = off;
  return t;
}

// Candidate path region, placed after the full-path layout.
struct CandLayout {
  int us_stride = 0;
  size_t off_us = 0, off_tau = 0, off_cnt = 0, off_cand = 0, off_rflag = 0, off_bflag = 0;
  size_t bytes = 0;   // end offset
};

bool cand_eligible(int N, int L, int topk) {
  return N >= kOneRowMinN && L >= kCandMinL && topk <= kCandMaxTopk;
}

CandLayout cand_layout(size_t start, int N, int L) {
  CandLayout c;
  c.us_stride = static_cast<int>(align_up(static_cast<size_t>((L + (1 << kSampleShift) - 1) >>
                                                              kSampleShift), 64));
  size_t off = align_up(start, 256);
  c.off_us = off;
  off = align_up(off + static_cast<size_t>(N) * c.us_stride * 4, 256);
  c.off_tau = off;
  off = align_up(off + static_cast<size_t>(N) * 4, 256);
  c.off_cnt = off;
  off = align_up(off + static_cast<size_t>(N) * kMaxSplits * 4, 256);
  c.off_cand = off;
  off = align_up(off + static_cast<size_t>(N) * kCandRegion * 8, 256);
  c.off_rflag = off;
  off = align_up(off + static_cast<size_t>(N) * 4, 256);
  c.off_bflag = off;
  off = align_up(off + static_cast<size_t>(N) * 4, 256);
  c.bytes = off;
  return c;
}

size_t score_topk_bytes(int N, int L, int topk) {
  const TopkLayout t = topk_layout(N, L);
  if (!cand_eligible(N, L, topk)) return t.bytes;
  return cand_layout(t.bytes, N, L).bytes;
}

// sparse attention: per-split partial outputs, then (max, sum) pairs
size_t attention_bytes(int N, int H, int d_v, int topk) {
  const size_t parts = static_cast<size_t>(N) * H * misa::attn_splits(topk);
  return align_up(parts * d_v * 4, 256) + align_up(parts * 8, 256);
}

// block prefilter: block keys, row lengths, kept blocks, candidate tokens,
// candidate order keys
struct BlocksLayout {
  int ub_stride = 0, u_stride = 0;
  size_t off_last = 0, off_blocks = 0, off_cand = 0, off_u = 0, bytes = 0;
};

BlocksLayout blocks_layout(int N, int L, int B, int m) {
  BlocksLayout b;
  const int mmax = (L + B - 1) / B;
  b.ub_stride = topk_layout(kOneRowMinN, mmax).u_stride;
  b.u_stride = topk_layout(kOneRowMinN, m * B).u_stride;
  size_t off = align_up(static_cast<size_t>(N) * b.ub_stride * 4, 256);
  b.off_last = off;
  off = align_up(off + static_cast<size_t>(N) * 4, 256);
  b.off_blocks = off;
  off = align_up(off + static_cast<size_t>(N) * m * 4, 256);
  b.off_cand = off;
  off = align_up(off + static_cast<size_t>(N) * m * B * 4, 256);
  b.off_u = off;
  b.bytes = align_up(off + static_cast<size_t>(N) * b.u_stride * 4, 256);
  return b;
}

size_t rerank_bytes(int N, int k_prime) {
  const TopkLayout t = topk_layout(kOneRowMinN, k_prime);   // always one row per workgroup
  return align_up(static_cast<size_t>(N) * t.u_stride * 4, 256);
}

int route_chunks(int L, int B) {
  const int mf = L / B;
  const int per = misa::route_blocks_per_chunk();
  const int c = (mf + per - 1) / per;
  return c > 0 ? c : 1;
}

size_t route_partial_bytes(int N, int L, int B, int H_I) {
  return align_up(static_cast<size_t>(N) * route_chunks(L, B) * H_I * 4, 256);
}

// partial sums, then the pooled table split into bf16 hi / lo halves (d <= 128)
size_t route_bytes(int N, int L, int B, int H_I) {
  const size_t M = (static_cast<size_t>(L) + B - 1) / B;
  return route_partial_bytes(N, L, B, H_I) + align_up(M * 128 * 2 * 2, 256);
}

// fp8 queries: bf16 copies of the codes [N, H_I, d] and the folded weights
// w * q_scale [N, H_I], placed after an op's own workspace.
size_t q8_bytes(int N, int H_I, int d) {
  const size_t rows = static_cast<size_t>(N) * H_I;
  return align_up(rows * d * 2, 256) + align_up(rows * 4, 256);
}

// routed decode step: router region (partials with one more slot per row for
// the partial-block term), then the scoring workspace
size_t route_score_route_bytes(int q_dt, int N, int L, int d, int B, int H_I) {
  return route_bytes(N, L, B, H_I) + align_up(static_cast<size_t>(N) * H_I * 4, 256) +
         (q_dt == MISA_FP8_E4M3 ? q8_bytes(N, H_I, d) : 0);
}

// Converts fp8 queries into `region` and points (q, q_dt, w) at the bf16
// problem with the same scores (see launch_q8_prep).
hipError_t prep_fp8_queries(const void*& q, int32_t& q_dt, const float*& w, const float* q_scale,
                            int N, int H_I, int d, uint8_t* region, hipStream_t st) {
  const size_t rows = static_cast<size_t>(N) * H_I;
  uint16_t* qb = reinterpret_cast<uint16_t*>(region);
  float* wq = reinterpret_cast<float*>(region + align_up(rows * d * 2, 256));
  misa::Q8PrepArgs a{static_cast<const uint8_t*>(q), q_scale, w, static_cast<int64_t>(rows), d,
                     qb, wq};
  const hipError_t e = misa::launch_q8_prep(a, st);
  q = qb;
  q_dt = MISA_BF16;
  w = wq;
  return e;
}

// ---------------------------------------------------------------- kernel timing
// Per host thread: a thread's misa_profile_begin times the launches that
// thread makes, so threads calling the library never share this state.
struct Profiler {
  bool on = false;
  int cap = 0, used = 0;
  std::vector<hipEvent_t> ev0, ev1;
  std::vector<int> ids;
};
thread_local Profiler g_prof;

void profiler_release(Profiler& pr) {
  for (size_t i = 0; i < pr.ev0.size(); ++i) {
    if (pr.ev0[i]) (void)hipEventDestroy(pr.ev0[i]);
    if (pr.ev1[i]) (void)hipEventDestroy(pr.ev1[i]);
  }
  pr = Profiler();
}

// ---------------------------------------------------------------- debug validation
// With MISA_DEBUG_SYNC=1 in the environment (read at every call) each entry
// point synchronises the caller's stream, copies the device-resident index
// arguments to the host and checks them before it launches anything; an
// out-of-range value returns MISA_ERR_SHAPE.  Release use leaves it unset.
bool debug_sync() {
  const char* v = getenv("MISA_DEBUG_SYNC");
  return v && v[0] == '1' && v[1] == '\0';
}

// Copies n int32 values from the device after the stream's earlier work.
int32_t fetch_i32(const int32_t* dev, size_t n, hipStream_t st, std::vector<int32_t>& out) {
  out.assign(n, 0);
  if (n == 0) return MISA_OK;
  hipError_t e = hipStreamSynchronize(st);
  if (e == hipSuccess) e = hipMemcpy(out.data(), dev, n * sizeof(int32_t), hipMemcpyDeviceToHost);
  return hip_status(e);
}

// Rows: 0 <= q_seq[n] < S, 0 <= q_pos[n] < L.
int32_t debug_rows(const int32_t* q_seq, const int32_t* q_pos, int N, int S, int L,
                   hipStream_t st, std::vector<int32_t>* pos_out = nullptr) {
  std::vector<int32_t> seq, pos;
  int32_t rc = fetch_i32(q_seq, N, st, seq);
  if (!rc && q_pos) rc = fetch_i32(q_pos, N, st, pos);
  if (rc) return rc;
  for (int n = 0; n < N; ++n) {
    if (seq[n] < 0 || seq[n] >= S) return MISA_ERR_SHAPE;
    if (q_pos && (pos[n] < 0 || pos[n] >= L)) return MISA_ERR_SHAPE;
  }
  if (pos_out) *pos_out = std::move(pos);
  return MISA_OK;
}

// Heads: every row lists h distinct heads in [0, H_I).
int32_t debug_heads(const int32_t* heads, int N, int h, int H_I, hipStream_t st) {
  std::vector<int32_t> hd;
  int32_t rc = fetch_i32(heads, static_cast<size_t>(N) * h, st, hd);
  if (rc) return rc;
  for (int n = 0; n < N; ++n) {
    uint64_t seen = 0;
    for (int i = 0; i < h; ++i) {
      const int32_t j = hd[static_cast<size_t>(n) * h + i];
      if (j < 0 || j >= H_I || ((seen >> j) & 1u)) return MISA_ERR_SHAPE;
      seen |= uint64_t{1} << j;
    }
  }
  return MISA_OK;
}

// Token lists (MISA-dagger candidates, attention selections): entries are -1
// or tokens below the row's bound; valid ones strictly ascending when
// `ascending`, else distinct.
int32_t debug_tokens(const int32_t* tok, int N, int stride, const std::vector<int32_t>& bound,
                     int L, bool ascending, hipStream_t st) {
  std::vector<int32_t> t;
  int32_t rc = fetch_i32(tok, static_cast<size_t>(N) * stride, st, t);
  if (rc) return rc;
  std::vector<uint8_t> seen;
  for (int n = 0; n < N; ++n) {
    const int32_t lim = bound.empty() ? L : bound[n] + 1;
    int32_t last = -1;
    if (!ascending) seen.assign(static_cast<size_t>(L), 0);
    for (int i = 0; i < stride; ++i) {
      const int32_t x = t[static_cast<size_t>(n) * stride + i];
      if (x == -1) continue;
      if (x < 0 || x >= lim) return MISA_ERR_SHAPE;
      if (ascending) {
        if (x <= last) return MISA_ERR_SHAPE;
        last = x;
      } else {
        if (seen[x]) return MISA_ERR_SHAPE;
        seen[x] = 1;
      }
    }
  }
  return MISA_OK;
}

// Appended lengths: 0 <= len_old[s] <= len_new[s] <= L, len_new - len_old <= max_new.
int32_t debug_lens(const int32_t* len_old, const int32_t* len_new, int S, int L, int max_new,
                   hipStream_t st) {
  std::vector<int32_t> a, b;
  int32_t rc = fetch_i32(len_old, S, st, a);
  if (!rc) rc = fetch_i32(len_new, S, st, b);
  if (rc) return rc;
  for (int s = 0; s < S; ++s)
    if (a[s] < 0 || a[s] > b[s] || b[s] > L || b[s] - a[s] > max_new) return MISA_ERR_SHAPE;
  return MISA_OK;
}

// The routed decode step's scoring launch picks the heads itself from the
// router partials (see misa_route_score_topk); its histogram was cleared by
// the router partials kernel.
struct FusedRoute {
  const float* partial;
  int nchunks, B;
  int32_t* heads_out;
  float* head_score_out;
};

int32_t score_topk_impl(const void* q, int32_t q_dt, const float* q_scale, const float* w,
                        const void* k, const float* k_scale, int32_t k_dt,
                        const int32_t* block_table, int32_t page_size, const int32_t* q_seq,
                        const int32_t* q_pos, const int32_t* heads, int32_t N, int32_t S,
                        int32_t L, int32_t d, int32_t H_I, int32_t h, int32_t topk,
                        int32_t* idx, float* score, void* ws, size_t ws_bytes, void* stream,
                        const FusedRoute* fr = nullptr) {
  if (!q || !w || !k || !q_seq || !q_pos || !idx) return MISA_ERR_NULL;
  int32_t rc = check_dtypes(q_dt, k_dt, q_scale, k_scale);
  if (rc) return rc;
  if ((rc = check_sizes(N, S, L, d, H_I))) return rc;
  misa::KeyIndex ki;
  if ((rc = key_index(block_table, page_size, L, ki))) return rc;
  if (h < 1 || h > H_I || topk < 1 || topk > kMaxTopk) return MISA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k)) return MISA_ERR_SHAPE;
  const bool f8 = q_dt == MISA_FP8_E4M3;
  const TopkLayout lay = topk_layout(N, L);
  const size_t q8_off = score_topk_bytes(N, L, topk);
  if (!ws) return MISA_ERR_NULL;
  if (ws_bytes < (f8 ? q8_off + q8_bytes(N, H_I, d) : lay.bytes)) return MISA_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (!fr && debug_sync()) {
    if ((rc = debug_rows(q_seq, q_pos, N, S, L, st))) return rc;
    if (heads && (rc = debug_heads(heads, N, h, H_I, st))) return rc;
  }
  uint8_t* base = static_cast<uint8_t*>(ws);
  uint32_t* u = reinterpret_cast<uint32_t*>(base);
  uint32_t* hist = lay.one_row ? nullptr : reinterpret_cast<uint32_t*>(base + lay.off_hist);
  hipError_t e = hipSuccess;
  if (hist && !fr) e = misa::launch_clear(hist, static_cast<size_t>(N) * misa::kHistWords, st);
  if (e != hipSuccess) return hip_status(e);
  // many rows over one contiguous sequence: GEMM over the gathered head rows
  // (bf16, or e4m3 straight from the codes)
  const bool gemm = S == 1 && !block_table && lay.one_row && N >= kOneRowMinN &&
                    ((q_dt == MISA_BF16 && k_dt == MISA_BF16) || (f8 && d == 128)) &&
                    static_cast<size_t>(L) * d * (f8 ? 1 : 2) < (size_t{1} << 32);
  if (f8 && !gemm) {
    e = prep_fp8_queries(q, q_dt, w, q_scale, N, H_I, d, base + q8_off, st);
    if (e != hipSuccess) return hip_status(e);
  }
  auto prefill_args = [&](uint32_t* uu, int u_stride) {
    misa::PrefillArgs a{q, w, k, q_pos, heads, N, L, d, H_I, h, uu, u_stride};
    a.fp8 = f8;
    a.q_scale = q_scale;
    a.k_scale = k_scale;
    return a;
  };
  if (gemm && cand_eligible(N, L, topk) && ws_bytes >= cand_layout(lay.bytes, N, L).bytes) {
    // many rows over one sequence, candidate path: sampled thresholds, GEMM
    // keeping only the keys above them, exact select; unproven rows redo the
    // full path
    const CandLayout cl = cand_layout(lay.bytes, N, L);
    const int h_eff = heads ? h : H_I;
    const int qb = misa::prefill_rows_per_block(h_eff);
    const int splits = misa::prefill_cand_splits(N, L, h_eff, d, f8);
    const int cap = kCandRegion / splits;
    uint32_t* us = reinterpret_cast<uint32_t*>(base + cl.off_us);
    float* tau = reinterpret_cast<float*>(base + cl.off_tau);
    uint32_t* cnt = reinterpret_cast<uint32_t*>(base + cl.off_cnt);
    uint2* cand = reinterpret_cast<uint2*>(base + cl.off_cand);
    uint32_t* rflag = reinterpret_cast<uint32_t*>(base + cl.off_rflag);
    uint32_t* bflag = reinterpret_cast<uint32_t*>(base + cl.off_bflag);
    misa::PrefillArgs sp = prefill_args(us, cl.us_stride);
    sp.key_step = 1 << kSampleShift;
    sp.pos_shift = kSampleShift;
    sp.kernel_id = misa::K_PREFILL_SAMPLE;
    if ((e = misa::launch_prefill(sp, st)) != hipSuccess) return hip_status(e);
    misa::TauArgs ta{us, cl.us_stride, q_pos, N, topk, kSampleShift, qb, tau, bflag};
    if ((e = misa::launch_tau(ta, st)) != hipSuccess) return hip_status(e);
    misa::PrefillArgs mp = prefill_args(nullptr, 0);
    mp.tau = tau;
    mp.cnt_out = cnt;
    mp.cand_out = cand;
    mp.cap = cap;
    if ((e = misa::launch_prefill(mp, st)) != hipSuccess) return hip_status(e);
    misa::CandTopkArgs ca{cnt, cand, splits, cap, q_pos, N, topk, qb, rflag, bflag, idx, score};
    if ((e = misa::launch_cand_topk(ca, st)) != hipSuccess) return hip_status(e);
    misa::PrefillArgs fp = prefill_args(u, lay.u_stride);
    fp.block_flag = bflag;
    fp.kernel_id = misa::K_PREFILL_FULL;
    if ((e = misa::launch_prefill(fp, st)) != hipSuccess) return hip_status(e);
    misa::TopkArgs ft{u, lay.u_stride, q_pos, 0, N, topk, true, nullptr, nullptr, 0, idx, score};
    ft.row_flag = rflag;
    return hip_status(misa::launch_topk(ft, st));
  }
  if (gemm) {
    e = misa::launch_prefill(prefill_args(u, lay.u_stride), st);
  } else {
    misa::ScoreArgs sa{q, q_dt, w, k, k_scale, k_dt, q_seq, q_pos, heads, nullptr,
                       N, S, L, d, H_I, h, 0, u, lay.u_stride, hist, ki};
    if (fr) {
      sa.route_partial = fr->partial;
      sa.route_nchunks = fr->nchunks;
      sa.B = fr->B;
      sa.heads_out = fr->heads_out;
      sa.head_score_out = fr->head_score_out;
    }
    e = misa::launch_score(sa, st);
  }
  if (e != hipSuccess) return hip_status(e);
  misa::TopkArgs ta{u, lay.u_stride, q_pos, 0, N, topk, lay.one_row, hist,
                    nullptr, 0, idx, score};
  return hip_status(misa::launch_topk(ta, st));
}

// Host checks of misa_pool_route_score_topk (every argument but the
// workspace): the key index and the route / score workspace parts on success.
int32_t check_pool_route_score_topk(const void* q, int32_t q_dt, const float* q_scale,
                                    const float* w, const float* kbar, const void* k,
                                    const float* k_scale, int32_t k_dt,
                                    const int32_t* block_table, int32_t page_size,
                                    const int32_t* q_seq, const int32_t* q_pos,
                                    const int32_t* len_old, const int32_t* len_new,
                                    int32_t max_new, int32_t N, int32_t S, int32_t L, int32_t d,
                                    int32_t B, int32_t H_I, int32_t h, int32_t topk,
                                    const int32_t* heads, const int32_t* idx,
                                    misa::KeyIndex* ki, size_t* rb, size_t* sb) {
  int32_t rc = check_pool(k, k_scale, k_dt, S, L, d, B, kbar);
  if (rc) return rc;
  if (!len_old || !len_new) return MISA_ERR_NULL;
  if (max_new < 0 || max_new > L) return MISA_ERR_SHAPE;
  if (!q || !w || !q_seq || !q_pos || !heads || !idx) return MISA_ERR_NULL;
  if ((rc = check_dtypes(q_dt, k_dt, q_scale, k_scale))) return rc;
  if ((rc = check_sizes(N, S, L, d, H_I))) return rc;
  if ((rc = key_index(block_table, page_size, L, *ki))) return rc;
  if (h < 1 || h > H_I || topk < 1 || topk > kMaxTopk) return MISA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k)) return MISA_ERR_SHAPE;
  *rb = route_score_route_bytes(q_dt, N, L, d, B, H_I);
  *sb = score_topk_bytes(N, L, topk) + (q_dt == MISA_FP8_E4M3 ? q8_bytes(N, H_I, d) : 0);
  return MISA_OK;
}

// ---------------------------------------------------------------- static scratch
// Device scratch of misa_pool_route_score_topk_scratch, for callers that
// cannot allocate: one array per GPU the library runs on, held until the
// process ends.  Host code never uses the array's name as an address: each
// device's address comes from hipGetSymbolAddress, taken once per device with
// that device current.
constexpr size_t kScratchBytes = size_t{32} << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int32_t scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return MISA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (!p) return MISA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MISA_OK;
}

}  // namespace

namespace misa {

bool prof_events(int kernel_id, hipEvent_t* start, hipEvent_t* stop) {
  if (!g_prof.on || g_prof.used >= g_prof.cap) return false;
  *start = g_prof.ev0[g_prof.used];
  *stop = g_prof.ev1[g_prof.used];
  g_prof.ids[g_prof.used] = kernel_id;
  ++g_prof.used;
  return true;
}

}  // namespace misa

extern "C" {

const char* misa_status_string(int32_t status) {
  switch (status) {
    case MISA_OK: return "ok";
    case MISA_ERR_NULL: return "a required pointer is NULL";
    case MISA_ERR_SHAPE: return "size or alignment out of range";
    case MISA_ERR_UNSUPPORTED: return "unsupported dtype combination or head dimension";
    case MISA_ERR_WORKSPACE: return "workspace too small";
    case MISA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int32_t misa_last_hip_error(void) { return g_last_hip; }

size_t misa_workspace_bytes(int32_t op, int32_t q_dt, int32_t N, int32_t L, int32_t d,
                            int32_t H_I, int32_t B, int32_t topk, int32_t k_prime) {
  if (op == MISA_OP_ATTENTION) {     // d = d_v, H_I = attention heads
    if (N < 1 || N > kMaxN || L < 1 || L > kMaxL || H_I < 1 || H_I > kMaxAttnHeads) return 0;
    if (d < 32 || d > 512 || d % 32 || topk < 1 || topk > kMaxTopk) return 0;
    return attention_bytes(N, H_I, d, topk);
  }
  if (N < 1 || N > kMaxN || L < 1 || L > kMaxL || H_I < 1 || H_I > 64) return 0;
  if (d != 64 && d != 128) return 0;
  if (q_dt != MISA_F32 && q_dt != MISA_BF16 && q_dt != MISA_FP8_E4M3) return 0;
  const size_t extra = q_dt == MISA_FP8_E4M3 ? q8_bytes(N, H_I, d) : 0;
  switch (op) {
    case MISA_OP_ROUTE:
      if (B < 1 || B > 1024) return 0;
      return route_bytes(N, L, B, H_I) + extra;
    case MISA_OP_SCORE_TOPK:
      if (topk < 1 || topk > kMaxTopk) return 0;
      return score_topk_bytes(N, L, topk) + extra;
    case MISA_OP_RERANK:
      if (k_prime < 1 || k_prime > kMaxTopk) return 0;
      return rerank_bytes(N, k_prime) + extra;
    case MISA_OP_ROUTE_SCORE_TOPK:
      if (B < 1 || B > 1024 || topk < 1 || topk > kMaxTopk) return 0;
      return route_score_route_bytes(q_dt, N, L, d, B, H_I) + score_topk_bytes(N, L, topk) +
             extra;
    case MISA_OP_BLOCKS:            // k_prime = m_blocks
      if (B < 1 || B > 1024 || k_prime < 1 || static_cast<int64_t>(k_prime) * B > kMaxTopk)
        return 0;
      if (topk < 1 || topk > k_prime * B) return 0;
      return blocks_layout(N, L, B, k_prime).bytes + extra;
    default:
      return 0;
  }
}

int64_t misa_candidate_flags_offset(int32_t N, int32_t L, int32_t topk) {
  if (N < 1 || N > kMaxN || L < 1 || L > kMaxL || topk < 1 || topk > kMaxTopk) return -1;
  if (!cand_eligible(N, L, topk)) return -1;
  const TopkLayout t = topk_layout(N, L);
  return static_cast<int64_t>(cand_layout(t.bytes, N, L).off_rflag);
}

int32_t misa_pool_keys(const void* k, const float* k_scale, int32_t k_dt,
                       const int32_t* block_table, int32_t page_size, int32_t S, int32_t L,
                       int32_t d, int32_t B, float* kbar, void* stream) {
  int32_t rc = check_pool(k, k_scale, k_dt, S, L, d, B, kbar);
  if (rc) return rc;
  misa::KeyIndex ki;
  if ((rc = key_index(block_table, page_size, L, ki))) return rc;
  misa::PoolArgs a{k, k_scale, k_dt, S, L, d, B, kbar, ki};
  return hip_status(misa::launch_pool(a, static_cast<hipStream_t>(stream)));
}

int32_t misa_pool_update(const void* k, const float* k_scale, int32_t k_dt,
                         const int32_t* block_table, int32_t page_size, int32_t S, int32_t L,
                         int32_t d, int32_t B, const int32_t* len_old, const int32_t* len_new,
                         int32_t max_new, float* kbar, void* stream) {
  int32_t rc = check_pool(k, k_scale, k_dt, S, L, d, B, kbar);
  if (rc) return rc;
  if (!len_old || !len_new) return MISA_ERR_NULL;
  if (max_new < 0 || max_new > L) return MISA_ERR_SHAPE;
  misa::KeyIndex ki;
  if ((rc = key_index(block_table, page_size, L, ki))) return rc;
  if (debug_sync() && (rc = debug_lens(len_old, len_new, S, L, max_new,
                                        static_cast<hipStream_t>(stream))))
    return rc;
  if (max_new == 0) return MISA_OK;
  misa::PoolArgs a{k, k_scale, k_dt, S, L, d, B, kbar, ki, len_old, len_new, max_new};
  return hip_status(misa::launch_pool(a, static_cast<hipStream_t>(stream)));
}

int32_t misa_route_heads(const void* q, int32_t q_dt, const float* q_scale, const float* w,
                         const float* kbar, const void* k, const float* k_scale, int32_t k_dt,
                         const int32_t* block_table, int32_t page_size, const int32_t* q_seq,
                         const int32_t* q_pos, int32_t N, int32_t S, int32_t L, int32_t d,
                         int32_t B, int32_t H_I, int32_t h, int32_t* heads, float* head_score,
                         void* ws, size_t ws_bytes, void* stream) {
  if (!q || !w || !kbar || !k || !q_seq || !q_pos || !heads) return MISA_ERR_NULL;
  int32_t rc = check_dtypes(q_dt, k_dt, q_scale, k_scale);
  if (rc) return rc;
  if ((rc = check_sizes(N, S, L, d, H_I))) return rc;
  misa::KeyIndex ki;
  if ((rc = key_index(block_table, page_size, L, ki))) return rc;
  if (B < 1 || B > 1024 || h < 1 || h > H_I) return MISA_ERR_SHAPE;
  const bool f8 = q_dt == MISA_FP8_E4M3;
  if (f8 && !aligned16(q)) return MISA_ERR_SHAPE;
  const size_t own = route_bytes(N, L, B, H_I);
  if (!ws) return MISA_ERR_NULL;
  if (ws_bytes < own + (f8 ? q8_bytes(N, H_I, d) : 0)) return MISA_ERR_WORKSPACE;
  if (debug_sync() &&
      (rc = debug_rows(q_seq, q_pos, N, S, L, static_cast<hipStream_t>(stream))))
    return rc;
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  misa::RouteArgs a{q, q_dt, f8 ? q_scale : nullptr, w, kbar, k, k_scale, k_dt, q_seq, q_pos, N,
                    S, L, d, B, H_I, h, heads, head_score, reinterpret_cast<float*>(wsb),
                    route_chunks(L, B),
                    reinterpret_cast<uint16_t*>(wsb + route_partial_bytes(N, L, B, H_I)), ki};
  // the GEMM router widens e4m3 queries itself; the per-row kernels take
  // them converted to bf16 (scale folded into the weight)
  if (f8 && !misa::route_uses_mfma(a)) {
    const hipError_t e = prep_fp8_queries(a.q, a.q_dt, a.w, q_scale, N, H_I, d, wsb + own,
                                          static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_status(e);
    a.q_scale = nullptr;
  }
  return hip_status(misa::launch_route(a, static_cast<hipStream_t>(stream)));
}

int32_t misa_score_topk(const void* q, int32_t q_dt, const float* q_scale, const float* w,
                        const void* k, const float* k_scale, int32_t k_dt,
                        const int32_t* block_table, int32_t page_size, const int32_t* q_seq,
                        const int32_t* q_pos, const int32_t* heads, int32_t N, int32_t S,
                        int32_t L, int32_t d, int32_t H_I, int32_t h, int32_t topk,
                        int32_t* idx, float* score, void* ws, size_t ws_bytes, void* stream) {
  if (!heads) return MISA_ERR_NULL;
  return score_topk_impl(q, q_dt, q_scale, w, k, k_scale, k_dt, block_table, page_size, q_seq,
                         q_pos, heads, N, S, L, d, H_I, h, topk, idx, score, ws, ws_bytes,
                         stream);
}

int32_t dsa_score_topk(const void* q, int32_t q_dt, const float* q_scale, const float* w,
                       const void* k, const float* k_scale, int32_t k_dt,
                       const int32_t* block_table, int32_t page_size, const int32_t* q_seq,
                       const int32_t* q_pos, int32_t N, int32_t S, int32_t L, int32_t d,
                       int32_t H_I, int32_t topk, int32_t* idx, float* score, void* ws,
                       size_t ws_bytes, void* stream) {
  return score_topk_impl(q, q_dt, q_scale, w, k, k_scale, k_dt, block_table, page_size, q_seq,
                         q_pos, nullptr, N, S, L, d, H_I, H_I, topk, idx, score, ws, ws_bytes,
                         stream);
}

int32_t misa_route_score_topk(const void* q, int32_t q_dt, const float* q_scale, const float* w,
                              const float* kbar, const void* k, const float* k_scale,
                              int32_t k_dt, const int32_t* block_table, int32_t page_size,
                              const int32_t* q_seq, const int32_t* q_pos, int32_t N, int32_t S,
                              int32_t L, int32_t d, int32_t B, int32_t H_I, int32_t h,
                              int32_t topk, int32_t* heads, float* head_score, int32_t* idx,
                              float* score, void* ws, size_t ws_bytes, void* stream) {
  if (!q || !w || !kbar || !k || !q_seq || !q_pos || !heads || !idx) return MISA_ERR_NULL;
  int32_t rc = check_dtypes(q_dt, k_dt, q_scale, k_scale);
  if (rc) return rc;
  if ((rc = check_sizes(N, S, L, d, H_I))) return rc;
  misa::KeyIndex ki;
  if ((rc = key_index(block_table, page_size, L, ki))) return rc;
  if (B < 1 || B > 1024 || h < 1 || h > H_I || topk < 1 || topk > kMaxTopk) return MISA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k)) return MISA_ERR_SHAPE;
  const size_t rb = route_score_route_bytes(q_dt, N, L, d, B, H_I);
  const size_t sb = score_topk_bytes(N, L, topk) +
                    (q_dt == MISA_FP8_E4M3 ? q8_bytes(N, H_I, d) : 0);
  if (!ws) return MISA_ERR_NULL;
  if (ws_bytes < rb + sb) return MISA_ERR_WORKSPACE;
  if (debug_sync() &&
      (rc = debug_rows(q_seq, q_pos, N, S, L, static_cast<hipStream_t>(stream))))
    return rc;
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  // the fused form: decode rows (not the one-sequence GEMM shapes), bf16
  // queries, bf16 or e4m3 keys; otherwise the two calls in turn
  const bool fused = q_dt == MISA_BF16 && k_dt != MISA_F32 && !(S == 1 && N >= kOneRowMinN);
  if (!fused) {
    rc = misa_route_heads(q, q_dt, q_scale, w, kbar, k, k_scale, k_dt, block_table, page_size,
                          q_seq, q_pos, N, S, L, d, B, H_I, h, heads, head_score, wsb, rb,
                          stream);
    if (rc) return rc;
    return misa_score_topk(q, q_dt, q_scale, w, k, k_scale, k_dt, block_table, page_size, q_seq,
                           q_pos, heads, N, S, L, d, H_I, h, topk, idx, score, wsb + rb, sb,
                           stream);
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  const TopkLayout lay = topk_layout(N, L);
  uint32_t* hist = lay.one_row ? nullptr : reinterpret_cast<uint32_t*>(wsb + rb + lay.off_hist);
  const int nchunks = route_chunks(L, B);
  float* partial = reinterpret_cast<float*>(wsb);
  misa::RouteArgs a{q, q_dt, nullptr, w, kbar, k, k_scale, k_dt, q_seq, q_pos, N, S, L, d, B,
                    H_I, h, heads, head_score, partial, nchunks, nullptr, ki};
  a.partials_only = true;
  a.hist0 = hist;
  const hipError_t e = misa::launch_route(a, st);
  if (e != hipSuccess) return hip_status(e);
  const FusedRoute fr{partial, nchunks, B, heads, head_score};
  return score_topk_impl(q, q_dt, q_scale, w, k, k_scale, k_dt, block_table, page_size, q_seq,
                         q_pos, nullptr, N, S, L, d, H_I, h, topk, idx, score, wsb + rb, sb,
                         stream, &fr);
}

int32_t misa_pool_route_score_topk(const void* q, int32_t q_dt, const float* q_scale,
                                   const float* w, float* kbar, const void* k,
                                   const float* k_scale, int32_t k_dt, const int32_t* block_table,
                                   int32_t page_size, const int32_t* q_seq, const int32_t* q_pos,
                                   const int32_t* len_old, const int32_t* len_new, int32_t max_new,
                                   int32_t N, int32_t S, int32_t L, int32_t d, int32_t B,
                                   int32_t H_I, int32_t h, int32_t topk, int32_t* heads,
                                   float* head_score, int32_t* idx, float* score, void* ws,
                                   size_t ws_bytes, void* stream) {
  // the checks of both calls, before anything runs
  misa::KeyIndex ki;
  size_t rb = 0, sb = 0;
  int32_t rc = check_pool_route_score_topk(q, q_dt, q_scale, w, kbar, k, k_scale, k_dt,
                                           block_table, page_size, q_seq, q_pos, len_old,
                                           len_new, max_new, N, S, L, d, B, H_I, h, topk, heads,
                                           idx, &ki, &rb, &sb);
  if (rc) return rc;
  if (!ws) return MISA_ERR_NULL;
  if (ws_bytes < rb + sb) return MISA_ERR_WORKSPACE;
  if (debug_sync()) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((rc = debug_lens(len_old, len_new, S, L, max_new, st))) return rc;
    if ((rc = debug_rows(q_seq, q_pos, N, S, L, st))) return rc;
  }
  const bool fused = q_dt == MISA_BF16 && k_dt != MISA_F32 && !(S == 1 && N >= kOneRowMinN);
  if (!fused || max_new == 0) {
    rc = misa_pool_update(k, k_scale, k_dt, block_table, page_size, S, L, d, B, len_old, len_new,
                          max_new, kbar, stream);
    if (rc) return rc;
    return misa_route_score_topk(q, q_dt, q_scale, w, kbar, k, k_scale, k_dt, block_table,
                                 page_size, q_seq, q_pos, N, S, L, d, B, H_I, h, topk, heads,
                                 head_score, idx, score, ws, ws_bytes, stream);
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  const TopkLayout lay = topk_layout(N, L);
  uint32_t* hist = lay.one_row ? nullptr : reinterpret_cast<uint32_t*>(wsb + rb + lay.off_hist);
  const int nchunks = route_chunks(L, B);
  float* partial = reinterpret_cast<float*>(wsb);
  misa::RouteArgs a{q, q_dt, nullptr, w, kbar, k, k_scale, k_dt, q_seq, q_pos, N, S, L, d, B,
                    H_I, h, heads, head_score, partial, nchunks, nullptr, ki};
  a.partials_only = true;
  a.hist0 = hist;
  a.len_old = len_old;
  a.len_new = len_new;
  a.max_new = max_new;
  a.kbar_out = kbar;
  const hipError_t e = misa::launch_route(a, st);
  if (e != hipSuccess) return hip_status(e);
  const FusedRoute fr{partial, nchunks, B, heads, head_score};
  return score_topk_impl(q, q_dt, q_scale, w, k, k_scale, k_dt, block_table, page_size, q_seq,
                         q_pos, nullptr, N, S, L, d, H_I, h, topk, idx, score, wsb + rb, sb,
                         stream, &fr);
}

int32_t misa_pool_route_score_topk_scratch(
    const void* q, int32_t q_dt, const float* q_scale, const float* w, float* kbar, const void* k,
    const float* k_scale, int32_t k_dt, const int32_t* block_table, int32_t page_size,
    const int32_t* q_seq, const int32_t* q_pos, const int32_t* len_old, const int32_t* len_new,
    int32_t max_new, int32_t N, int32_t S, int32_t L, int32_t d, int32_t B, int32_t H_I,
    int32_t h, int32_t topk, int32_t* heads, float* head_score, int32_t* idx, float* score,
    void* stream) {
  // the workspace call's own checks, then its workspace size against the
  // scratch array's
  misa::KeyIndex ki;
  size_t rb = 0, sb = 0;
  int32_t rc = check_pool_route_score_topk(q, q_dt, q_scale, w, kbar, k, k_scale, k_dt,
                                           block_table, page_size, q_seq, q_pos, len_old,
                                           len_new, max_new, N, S, L, d, B, H_I, h, topk, heads,
                                           idx, &ki, &rb, &sb);
  if (rc) return rc;
  if (rb + sb > kScratchBytes) return MISA_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((rc = scratch_of_current_device(&ws))) return rc;
  return misa_pool_route_score_topk(q, q_dt, q_scale, w, kbar, k, k_scale, k_dt, block_table,
                                    page_size, q_seq, q_pos, len_old, len_new, max_new, N, S, L,
                                    d, B, H_I, h, topk, heads, head_score, idx, score, ws,
                                    kScratchBytes, stream);
}

int32_t misa_rerank(const void* q, int32_t q_dt, const float* q_scale, const float* w,
                    const void* k, const float* k_scale, int32_t k_dt, const int32_t* block_table,
                    int32_t page_size, const int32_t* q_seq, const int32_t* q_pos,
                    const int32_t* cand, int32_t N, int32_t S, int32_t L, int32_t d, int32_t H_I,
                    int32_t k_prime, int32_t topk, int32_t* idx, float* score, void* ws,
                    size_t ws_bytes, void* stream) {
  if (!q || !w || !k || !q_seq || !q_pos || !cand || !idx) return MISA_ERR_NULL;
  int32_t rc = check_dtypes(q_dt, k_dt, q_scale, k_scale);
  if (rc) return rc;
  if ((rc = check_sizes(N, S, L, d, H_I))) return rc;
  misa::KeyIndex ki;
  if ((rc = key_index(block_table, page_size, L, ki))) return rc;
  if (topk < 1 || k_prime < topk || k_prime > kMaxTopk) return MISA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k)) return MISA_ERR_SHAPE;
  const bool f8 = q_dt == MISA_FP8_E4M3;
  const size_t own = rerank_bytes(N, k_prime);
  if (!ws) return MISA_ERR_NULL;
  if (ws_bytes < own + (f8 ? q8_bytes(N, H_I, d) : 0)) return MISA_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (debug_sync()) {
    std::vector<int32_t> pos;
    if ((rc = debug_rows(q_seq, q_pos, N, S, L, st, &pos))) return rc;
    if ((rc = debug_tokens(cand, N, k_prime, pos, L, true, st))) return rc;
  }
  if (f8) {
    const hipError_t e =
        prep_fp8_queries(q, q_dt, w, q_scale, N, H_I, d, static_cast<uint8_t*>(ws) + own, st);
    if (e != hipSuccess) return hip_status(e);
  }
  const int u_stride = topk_layout(kOneRowMinN, k_prime).u_stride;
  uint32_t* u = static_cast<uint32_t*>(ws);
  misa::ScoreArgs sa{q, q_dt, w, k, k_scale, k_dt, q_seq, q_pos, nullptr, cand,
                     N, S, L, d, H_I, H_I, k_prime, u, u_stride, nullptr, ki};
  hipError_t e = misa::launch_score(sa, st);
  if (e != hipSuccess) return hip_status(e);
  misa::TopkArgs ta{u, u_stride, nullptr, k_prime, N, topk, true, nullptr,
                    cand, k_prime, idx, score};
  return hip_status(misa::launch_topk(ta, st));
}

int32_t misa_score_topk_blocks(const void* q, int32_t q_dt, const float* q_scale, const float* w,
                               const float* kbar, const void* k, const float* k_scale,
                               int32_t k_dt, const int32_t* block_table, int32_t page_size,
                               const int32_t* q_seq, const int32_t* q_pos, const int32_t* heads,
                               int32_t N, int32_t S, int32_t L, int32_t d, int32_t B,
                               int32_t H_I, int32_t h, int32_t m_blocks, int32_t topk,
                               int32_t* blocks, int32_t* idx, float* score, void* ws,
                               size_t ws_bytes, void* stream) {
  if (!q || !w || !kbar || !k || !q_seq || !q_pos || !heads || !idx) return MISA_ERR_NULL;
  int32_t rc = check_dtypes(q_dt, k_dt, q_scale, k_scale);
  if (rc) return rc;
  if ((rc = check_sizes(N, S, L, d, H_I))) return rc;
  misa::KeyIndex ki;
  if ((rc = key_index(block_table, page_size, L, ki))) return rc;
  if (B < 1 || B > 1024 || h < 1 || h > H_I || m_blocks < 1) return MISA_ERR_SHAPE;
  if (static_cast<int64_t>(m_blocks) * B > kMaxTopk || topk < 1 || topk > m_blocks * B)
    return MISA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k)) return MISA_ERR_SHAPE;
  const bool f8 = q_dt == MISA_FP8_E4M3;
  const BlocksLayout bl = blocks_layout(N, L, B, m_blocks);
  if (!ws) return MISA_ERR_NULL;
  if (ws_bytes < bl.bytes + (f8 ? q8_bytes(N, H_I, d) : 0)) return MISA_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (debug_sync()) {
    if ((rc = debug_rows(q_seq, q_pos, N, S, L, st))) return rc;
    if ((rc = debug_heads(heads, N, h, H_I, st))) return rc;
  }
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  hipError_t e = hipSuccess;
  if (f8) {
    e = prep_fp8_queries(q, q_dt, w, q_scale, N, H_I, d, wsb + bl.bytes, st);
    if (e != hipSuccess) return hip_status(e);
  }
  uint32_t* ub = reinterpret_cast<uint32_t*>(wsb);
  int32_t* last = reinterpret_cast<int32_t*>(wsb + bl.off_last);
  int32_t* kept = blocks ? blocks : reinterpret_cast<int32_t*>(wsb + bl.off_blocks);
  int32_t* cand = reinterpret_cast<int32_t*>(wsb + bl.off_cand);
  uint32_t* u = reinterpret_cast<uint32_t*>(wsb + bl.off_u);
  misa::BlockScoreArgs ba{q, q_dt, w, kbar, k, k_scale, k_dt, ki, q_seq, q_pos, heads,
                          N, L, d, B, H_I, h, ub, bl.ub_stride, last};
  if ((e = misa::launch_block_scores(ba, st)) != hipSuccess) return hip_status(e);
  misa::TopkArgs tb{ub, bl.ub_stride, last, 0, N, m_blocks, true, nullptr, nullptr, 0, kept,
                    nullptr};
  if ((e = misa::launch_topk(tb, st)) != hipSuccess) return hip_status(e);
  if ((e = misa::launch_expand_blocks(kept, q_pos, N, m_blocks, B, cand, st)) != hipSuccess)
    return hip_status(e);
  const int ncols = m_blocks * B;
  misa::ScoreArgs sa{q, q_dt, w, k, k_scale, k_dt, q_seq, q_pos, heads, cand,
                     N, S, L, d, H_I, h, ncols, u, bl.u_stride, nullptr, ki};
  if ((e = misa::launch_score(sa, st)) != hipSuccess) return hip_status(e);
  misa::TopkArgs ta{u, bl.u_stride, nullptr, ncols, N, topk, true, nullptr, cand, ncols, idx,
                    score};
  return hip_status(misa::launch_topk(ta, st));
}

int32_t misa_sparse_attention(const void* q, int32_t q_dt, const void* kv, int32_t kv_dt,
                              const int32_t* block_table, int32_t page_size,
                              const int32_t* q_seq, const int32_t* idx, int32_t N, int32_t S,
                              int32_t L, int32_t H, int32_t d_qk, int32_t d_v, int32_t topk,
                              float scale, float* out, float* lse, void* ws, size_t ws_bytes,
                              void* stream) {
  if (!q || !kv || !q_seq || !idx || !out || !lse) return MISA_ERR_NULL;
  if (q_dt != MISA_BF16 || kv_dt != MISA_BF16) return MISA_ERR_UNSUPPORTED;
  if (d_qk != 64 && d_qk != 128 && d_qk != 256 && d_qk != 576) return MISA_ERR_UNSUPPORTED;
  if (d_v < 32 || d_v > 512 || d_v % 32 || d_v > d_qk) return MISA_ERR_SHAPE;
  if (N < 1 || N > kMaxN || S < 1 || S > kMaxN || L < 1 || L > kMaxL) return MISA_ERR_SHAPE;
  if (H < 1 || H > kMaxAttnHeads || topk < 1 || topk > kMaxTopk) return MISA_ERR_SHAPE;
  if (!(scale > 0.f) || scale > 1e30f) return MISA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(kv) || !aligned16(out)) return MISA_ERR_SHAPE;
  misa::KeyIndex ki;
  int32_t rc = key_index(block_table, page_size, L, ki);
  if (rc) return rc;
  const size_t need = attention_bytes(N, H, d_v, topk);
  if (!ws) return MISA_ERR_NULL;
  if (ws_bytes < need) return MISA_ERR_WORKSPACE;
  if (debug_sync()) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((rc = debug_rows(q_seq, nullptr, N, S, L, st))) return rc;
    if ((rc = debug_tokens(idx, N, topk, {}, L, false, st))) return rc;
  }
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  const size_t parts = static_cast<size_t>(N) * H * misa::attn_splits(topk);
  misa::AttnArgs a{q, kv, ki, q_seq, idx, N, H, d_qk, d_v, topk, scale,
                   reinterpret_cast<float*>(wsb), wsb + align_up(parts * d_v * 4, 256), out, lse};
  return hip_status(misa::launch_attention(a, static_cast<hipStream_t>(stream)));
}

int32_t misa_profile_begin(int32_t capacity) {
  if (capacity < 1) return MISA_ERR_SHAPE;
  profiler_release(g_prof);
  g_prof.ev0.assign(capacity, nullptr);
  g_prof.ev1.assign(capacity, nullptr);
  g_prof.ids.assign(capacity, -1);
  for (int i = 0; i < capacity; ++i) {
    hipError_t e = hipEventCreate(&g_prof.ev0[i]);
    if (e == hipSuccess) e = hipEventCreate(&g_prof.ev1[i]);
    if (e != hipSuccess) {
      profiler_release(g_prof);           // the events created so far
      return hip_status(e);
    }
  }
  g_prof.cap = capacity;
  g_prof.used = 0;
  g_prof.on = true;
  return MISA_OK;
}

int32_t misa_profile_end(int32_t* kernel_id, float* ms, int32_t max) {
  int32_t written = 0;
  for (int i = 0; i < g_prof.used; ++i) {
    if (i < max && kernel_id && ms) {
      float t = 0.f;
      (void)hipEventSynchronize(g_prof.ev1[i]);
      if (hipEventElapsedTime(&t, g_prof.ev0[i], g_prof.ev1[i]) != hipSuccess) t = -1.f;
      kernel_id[i] = g_prof.ids[i];
      ms[i] = t;
      ++written;
    }
  }
  profiler_release(g_prof);
  return written;
}

const char* misa_kernel_name(int32_t kernel_id) {
  static const char* names[misa::K_COUNT_IDS] = {
      "pool_kernel",       "route_partial_kernel", "route_select_kernel", "topk_clear_kernel",
      "score_mfma_kernel", "score_f32_kernel",     "score_prefill_kernel",
      "topk_collect_kernel", "topk_final_kernel",   "topk_row_kernel",
      "score_prefill_sample", "score_prefill_full", "topk_tau_kernel", "topk_cand_kernel",
      "route_split_kernel", "q8_prep_kernel", "pool_update_kernel", "attn_split_kernel",
      "attn_combine_kernel", "block_score_kernel", "expand_blocks_kernel"};
  if (kernel_id < 0 || kernel_id >= misa::K_COUNT_IDS) return "unknown";
  return names[kernel_id];
}

}  // extern "C"
