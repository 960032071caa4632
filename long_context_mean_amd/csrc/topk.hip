// Exact top-k selection over fp32 index scores, gfx950.
//
// Scores arrive as 32-bit order keys (order_key: larger score <-> larger key,
// -0 == +0, key 0 = empty slot).  The wanted set is the min(k, valid) keys
// first under (key desc, index asc).  With T the k-th largest key and K2 the
// number of key == T elements that make the cut, the set is {key > T} plus
// the K2 lowest-index elements with key == T.  T is found by radix select on
// 12 + 12 + 8 bit digits; outputs are written in ascending index order, so
// results are deterministic.
//
// Few long rows (decode): the scoring kernel has already built each row's
// level-0 histogram (top 12 key bits).
//  topk_collect (grid: 4096-element chunks x rows) finds the bin d0 holding
//    the k-th key; elements above it are certain winners and are recorded in
//    a bitmap (each chunk writes its own words, no atomics); elements in bin
//    d0 are appended to a short candidate list.
//  topk_final (grid: 32768-element slices x rows, 1024 threads) loads the
//    candidates into LDS and resolves the exact threshold among them with two
//    more radix levels (every workgroup of a row finds the same one), counts
//    the winners before its slice (bitmap words and candidates), marks the
//    candidate winners inside it and emits the slice's winners in index
//    order, a bitmap word per thread.  When the candidates do not fit in LDS
//    (heavily tied scores, or rows of millions of tokens) or the row is longer
//    than 2^24 tokens, the row's first workgroup falls back to a full radix
//    select over the row.
// Many rows or short rows (prefill, rerank): topk_row, one 1024-thread
//    workgroup per row with every histogram in LDS.
#include "common.hpp"
#include "kernels.hpp"

namespace misa {
namespace {

constexpr int kChunk = 4096;          // elements per collect workgroup
constexpr int kPerThread = 16;        // contiguous elements per thread per tile
constexpr int kCandCap = 8192;        // candidates resolved in LDS
constexpr int kBitmapWords = 8192;    // 262144 elements: the one-row select's LDS bitmap of a row
constexpr int kFinalThreads = 1024;   // threads of the few-rows final selection

// Finds the bin of a histogram (NBINS bins, bin NBINS-1 = largest keys) that
// holds the K-th largest element.  With clamp_total, K = min(K, total) first.
// All NT threads call it; results in `res`: [0] digit, [1] rank inside the
// digit's bin (1-based), [2] K, [3] total.  K == 0 leaves digit/rank 0.
template <int NT, int NBINS>
__device__ __forceinline__ void find_digit(const uint32_t* hist, uint32_t K, bool clamp_total, uint32_t* sm,
                           uint32_t* res) {
  constexpr int PER = NBINS >= NT ? NBINS / NT : 1;
  const int t = static_cast<int>(threadIdx.x);
  const bool owner = NBINS >= NT || t < NBINS;
  const int lo = NBINS - (t + 1) * PER;                 // this thread's lowest bin
  uint32_t v[PER];
  if (owner) {
    if constexpr (PER % 4 == 0) {
      const uint4* p4 = reinterpret_cast<const uint4*>(hist + lo);
#pragma unroll
      for (int q = 0; q < PER / 4; ++q) {
        const uint4 x = p4[q];
        v[4 * q] = x.x;
        v[4 * q + 1] = x.y;
        v[4 * q + 2] = x.z;
        v[4 * q + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int q = 0; q < PER; ++q) v[q] = hist[lo + q];
    }
  } else {
#pragma unroll
    for (int q = 0; q < PER; ++q) v[q] = 0u;
  }
  uint32_t c = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) c += v[q];
  uint32_t total;
  const uint32_t above = block_excl_scan<NT>(c, sm, total);
  if (clamp_total && K > total) K = total;
  if (t == 0) {
    res[0] = 0;
    res[1] = 0;
    res[2] = K;
    res[3] = total;
  }
  __syncthreads();
  if (K > 0 && above < K && K <= above + c) {
    uint32_t acc = above;
#pragma unroll
    for (int q = PER - 1; q >= 0; --q) {
      if (acc < K && acc + v[q] >= K) {
        res[0] = static_cast<uint32_t>(lo + q);
        res[1] = K - acc;
      }
      acc += v[q];
    }
  }
  __syncthreads();
}

// Ties at the threshold: among the n_eq candidates whose key equals T, the K2
// lowest token indices win (K2 <= n_eq).  Returns the largest winning index.
// Radix select on the indices in hA (4096 words) and hB (64 words): indices
// below 2^18 take bits 6..17, then 0..5; with `big` (indices below 2^24)
// bits 12..23, then 6..11, then 0..5.  Every thread calls it.
template <int NT>
__device__ __forceinline__ uint32_t tie_cut(const uint32_t* cu, const uint32_t* ci, int total,
                                            uint32_t T, uint32_t K2, uint32_t n_eq, bool big,
                                            uint32_t* hA, uint32_t* hB, uint32_t* sm,
                                            uint32_t* res) {
  const int sA = big ? 12 : 6;
  for (int b = threadIdx.x; b < 4096; b += NT) hA[b] = 0u;
  if (threadIdx.x < 64) hB[threadIdx.x] = 0u;
  __syncthreads();
  for (int i = threadIdx.x; i < total; i += NT)
    if (cu[i] == T) atomicAdd(&hA[ci[i] >> sA], 1u);
  __syncthreads();
  // the K2-th smallest index is the (n_eq - K2 + 1)-th largest
  find_digit<NT, 4096>(hA, n_eq - K2 + 1u, false, sm, res);
  uint32_t pre = res[0], r = res[1];                 // index bits [sA, ..) decided
  if (big) {
    for (int i = threadIdx.x; i < total; i += NT)
      if (cu[i] == T && (ci[i] >> 12) == pre) atomicAdd(&hB[(ci[i] >> 6) & 63u], 1u);
    __syncthreads();
    find_digit<NT, 64>(hB, r, false, sm, res);
    pre = (pre << 6) | res[0];                       // bits [6, ..) decided
    r = res[1];
    if (threadIdx.x < 64) hB[threadIdx.x] = 0u;
    __syncthreads();
  }
  for (int i = threadIdx.x; i < total; i += NT)
    if (cu[i] == T && (ci[i] >> 6) == pre) atomicAdd(&hB[ci[i] & 63u], 1u);
  __syncthreads();
  find_digit<NT, 64>(hB, r, false, sm, res);
  const uint32_t cut = (pre << 6) | res[0];
  __syncthreads();
  return cut;
}

struct Threshold {
  uint32_t T;     // exact k-th largest key
  uint32_t K2;    // number of key == T elements to take (lowest indices)
  uint32_t K;     // number selected = min(topk, valid elements)
};

__device__ __forceinline__ int row_len(const int32_t* q_pos, int fixed_len, int n) {
  return q_pos ? q_pos[n] + 1 : fixed_len;
}

// 16 consecutive keys from element i0 (buffers are padded to whole chunks, so
// the loads stay in bounds); keys at or past `len` read as 0 (empty).
__device__ __forceinline__ void load16(const uint32_t* row, int i0, int len, uint32_t (&v)[16]) {
  const uint4* p = reinterpret_cast<const uint4*>(row + i0);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint4 x = p[j];
    v[4 * j + 0] = x.x;
    v[4 * j + 1] = x.y;
    v[4 * j + 2] = x.z;
    v[4 * j + 3] = x.w;
  }
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (i0 + j >= len) v[j] = 0u;
}

// LDS histogram of digit LEVEL over the row's elements [0, span) whose higher
// digits equal `prefix` (NT threads).
template <int NT, int LEVEL>
__device__ __forceinline__ void hist_range(const uint32_t* row, int span, int len, uint32_t prefix,
                           uint32_t* lh) {
  for (int i0 = static_cast<int>(threadIdx.x) * kPerThread; i0 < span; i0 += NT * kPerThread) {
    uint32_t v[16];
    load16(row, i0, len, v);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t u = v[j];
      if (u == 0u) continue;
      if (LEVEL == 0) {
        atomicAdd(&lh[u >> kShift0], 1u);
      } else if (LEVEL == 1) {
        if ((u >> kShift0) == prefix) atomicAdd(&lh[(u >> kShift1) & (kBins1 - 1)], 1u);
      } else {
        if ((u >> kShift1) == prefix) atomicAdd(&lh[u & (kBins2 - 1)], 1u);
      }
    }
  }
}

// Ordered compaction of the row's elements [0, span) against threshold th:
// writes the selected elements, in index order, to idx_row/score_row.
template <int NT>
__device__ __forceinline__ void compact_row(const uint32_t* row, int span, int len, Threshold th,
                            const int32_t* cand_row, int32_t* idx_row, float* score_row,
                            uint32_t* sm) {
  uint32_t offset = 0, eq_before = 0;
  for (int t0 = 0; t0 < span; t0 += NT * kPerThread) {
    const int i0 = t0 + static_cast<int>(threadIdx.x) * kPerThread;
    uint32_t v[16];
    if (i0 < span) {
      load16(row, i0, len, v);
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = 0u;
    }
    uint32_t n_eq = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) n_eq += (v[j] == th.T) ? 1u : 0u;
    uint32_t eq_tot;
    const uint32_t eq_rank = eq_before + block_excl_scan<NT>(n_eq, sm, eq_tot);
    uint32_t sel_mask = 0, n_sel = 0;
    {
      uint32_t r = eq_rank;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const bool gt = v[j] > th.T;
        const bool eq = v[j] == th.T;
        const bool sel = gt || (eq && r < th.K2);
        r += eq ? 1u : 0u;
        sel_mask |= sel ? (1u << j) : 0u;
        n_sel += sel ? 1u : 0u;
      }
    }
    uint32_t sel_tot;
    uint32_t pos = offset + block_excl_scan<NT>(n_sel, sm, sel_tot);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if ((sel_mask & (1u << j)) && pos < th.K) {
        const int i = i0 + j;
        idx_row[pos] = cand_row ? cand_row[i] : i;
        if (score_row) score_row[pos] = key_score(v[j]);
        ++pos;
      }
    }
    offset += sel_tot;
    eq_before += eq_tot;
  }
}

// Full single-workgroup selection over one row (three LDS histogram levels
// and an ordered compaction).  h0 may already hold the level-0 histogram
// (have_h0); h0/h1 hold 4096 words, h2 256 words, all in LDS.
template <int NT>
__device__ __forceinline__ void row_select(const uint32_t* row, int len, int topk, const int32_t* cand_row,
                           int32_t* idx_row, float* score_row, uint32_t* h0, uint32_t* h1,
                           uint32_t* h2, bool have_h0, uint32_t* sm, uint32_t* res) {
  const int span = (len + kPerThread - 1) / kPerThread * kPerThread;
  for (int b = threadIdx.x; b < kBins0; b += NT) {
    if (!have_h0) h0[b] = 0u;
    h1[b] = 0u;
  }
  for (int b = threadIdx.x; b < kBins2; b += NT) h2[b] = 0u;
  __syncthreads();
  if (!have_h0) {
    hist_range<NT, 0>(row, span, len, 0u, h0);
    __syncthreads();
  }
  find_digit<NT, kBins0>(h0, static_cast<uint32_t>(topk), true, sm, res);
  const uint32_t K = res[2], d0 = res[0], r0 = res[1];
  __syncthreads();
  for (int i = static_cast<int>(K) + threadIdx.x; i < topk; i += NT) {
    idx_row[i] = -1;
    if (score_row) score_row[i] = -__builtin_inff();
  }
  if (K == 0) return;
  // a bin taken whole (rank inside it == its count) ends the search: its
  // lower edge is the threshold and every key equal to it wins, so the
  // remaining sweeps over the row are skipped
  Threshold th;
  th.K = K;
  th.K2 = 0xFFFFFFFFu;
  if (r0 == h0[d0]) {
    th.T = d0 << kShift0;
  } else {
    hist_range<NT, 1>(row, span, len, d0, h1);
    __syncthreads();
    find_digit<NT, kBins1>(h1, r0, false, sm, res);
    const uint32_t d1 = res[0], r1 = res[1];
    const bool whole = r1 == h1[d1];
    __syncthreads();
    th.T = (d0 << kShift0) | (d1 << kShift1);
    if (!whole) {
      hist_range<NT, 2>(row, span, len, (d0 << kDigit1Bits) | d1, h2);
      __syncthreads();
      find_digit<NT, kBins2>(h2, r1, false, sm, res);
      th.T |= res[0];
      th.K2 = res[1];
      __syncthreads();
    }
  }
  compact_row<NT>(row, span, len, th, cand_row, idx_row, score_row, sm);
}

// ---------------------------------------------------------------- few long rows
__global__ __launch_bounds__(256) void topk_collect_kernel(
    const uint32_t* __restrict__ u, int u_stride, const int32_t* __restrict__ q_pos,
    int fixed_len, uint32_t* hist, uint32_t* __restrict__ bitmap, uint2* __restrict__ clist,
    int topk) {
  __shared__ uint32_t sm[4];
  __shared__ uint32_t res[4];
  __shared__ uint32_t base_slot;
  const int n = blockIdx.y;
  const int len = row_len(q_pos, fixed_len, n);
  const int base = blockIdx.x * kChunk;
  if (base >= len) return;
  uint32_t* h0 = hist + static_cast<size_t>(n) * kHistWords;
  // the chunk's keys do not depend on the threshold digit: their loads go
  // out first, so they and the histogram's share one round trip
  const uint32_t* row = u + static_cast<size_t>(n) * u_stride;
  const int i0 = base + threadIdx.x * kPerThread;
  uint32_t v[16];
  load16(row, i0, len, v);
  find_digit<256, kBins0>(h0, static_cast<uint32_t>(topk), true, sm, res);
  const uint32_t K = res[2], d0 = res[0];
  // the final workgroups read the digit, its rank and K instead of scanning
  // the histogram again
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    h0[kMetaOffset] = d0;
    h0[kMetaOffset + 1] = res[1];
    h0[kMetaOffset + 2] = K;
  }
  if (K == 0) return;
  uint32_t sure = 0, n_cand = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint32_t dg = v[j] >> kShift0;
    sure |= (v[j] != 0u && dg > d0) ? (1u << j) : 0u;
    n_cand += (v[j] != 0u && dg == d0) ? 1u : 0u;
  }
  // bitmap word = 32 elements = this thread's 16 bits and its odd neighbour's
  const uint32_t other = __shfl_xor(sure, 1, 64);
  if ((threadIdx.x & 1) == 0)
    bitmap[static_cast<size_t>(n) * (u_stride / 32) + (i0 >> 5)] = sure | (other << 16);
  uint32_t tot;
  uint32_t off = block_excl_scan<256>(n_cand, sm, tot);
  if (threadIdx.x == 0) base_slot = tot ? atomicAdd(&h0[kCandCountOffset], tot) : 0u;
  __syncthreads();
  off += base_slot;
  uint2* cl = clist + static_cast<size_t>(n) * kCandCap;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (v[j] != 0u && (v[j] >> kShift0) == d0) {
      if (off < kCandCap) cl[off] = make_uint2(v[j], static_cast<uint32_t>(i0 + j));
      ++off;
    }
  }
}

template <int NT>
__global__ __launch_bounds__(NT) void topk_final_kernel(
    const uint32_t* __restrict__ u, int u_stride, const int32_t* __restrict__ q_pos,
    int fixed_len, const uint32_t* hist, const uint32_t* __restrict__ bitmap,
    const uint2* __restrict__ clist, int topk, int32_t* __restrict__ idx,
    float* __restrict__ score) {
  constexpr int kSlice = 32 * NT;                       // elements per workgroup, a word per thread
  static_assert(kBitmapWords == 8 * NT, "two 16-byte bitmap loads per thread cover 2^18 tokens");
  __shared__ __align__(16) uint32_t bm[NT];             // the slice's winners, one bit per element
  __shared__ __align__(16) uint32_t cu[kCandCap];       // candidate order key
  __shared__ __align__(16) uint32_t ci[kCandCap];       // candidate element index
  __shared__ __align__(16) uint32_t hA[kBins0];
  __shared__ __align__(16) uint32_t hB[kBins2];
  __shared__ uint32_t sm[16];
  __shared__ uint32_t res[4];
  __shared__ uint32_t wcnt[NT / 64];                    // winners before the slice, per wavefront
  const int n = blockIdx.y, slice = blockIdx.x;
  const int len = row_len(q_pos, fixed_len, n);
  const int s0 = slice * kSlice;
  if (slice > 0 && s0 >= len) return;
  const uint32_t* row = u + static_cast<size_t>(n) * u_stride;
  const uint32_t* h0g = hist + static_cast<size_t>(n) * kHistWords;
  int32_t* idx_row = idx + static_cast<size_t>(n) * topk;
  float* score_row = score ? score + static_cast<size_t>(n) * topk : nullptr;
  const int nwords = (len + 31) / 32;
  const int w0 = s0 / 32;                               // the slice's first bitmap word
  const int t = static_cast<int>(threadIdx.x);

  // one round trip: the candidate count with the collect's digit, rank and K;
  // the certain-winner words before the slice (counted) and the slice's own
  // word; every thread's first candidate (the list holds kCandCap >= NT
  // entries, so the read stays inside it)
  // (every read unconditional, at an address inside the row's regions, and
  // the value dropped where it does not apply: a guarded read would wait
  // on its own)
  const uint32_t* bmg = bitmap + static_cast<size_t>(n) * (u_stride / 32);
  const uint4 meta_r = *reinterpret_cast<const uint4*>(h0g + kCandCountOffset);
  uint4 pw[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int w = 4 * (t + q * NT);
    pw[q] = *reinterpret_cast<const uint4*>(bmg + (w < w0 ? w : 0));
  }
  const uint32_t wd_r = bmg[w0 + t < nwords ? w0 + t : 0];
  const uint2* cl = clist + static_cast<size_t>(n) * kCandCap;
  static_assert(kCandCap >= NT, "one speculative candidate per thread");
  const uint2 e_first = cl[t];
  const uint4 meta = len > 0 ? meta_r : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
  for (int q = 0; q < 2; ++q)
    if (4 * (t + q * NT) >= w0) pw[q] = make_uint4(0u, 0u, 0u, 0u);
  const uint32_t wd = w0 + t < nwords ? wd_r : 0u;
  const uint32_t c = meta.x, d0 = meta.y, r0 = meta.z, K = meta.w;
  // (rows past 2^24 tokens would need a fourth index level in the tie cut)
  const bool fallback = c > static_cast<uint32_t>(kCandCap) || len > (1 << 24);
  if (fallback) {
    if (slice > 0) return;
    for (int b = t; b < kBins0; b += NT) hA[b] = h0g[b];
    __syncthreads();
    row_select<NT>(row, len, topk, nullptr, idx_row, score_row, hA, cu, hB, true, sm, res);
    return;
  }
  if (slice == 0) {
    for (int i = static_cast<int>(K) + t; i < topk; i += NT) {
      idx_row[i] = -1;
      if (score_row) score_row[i] = -__builtin_inff();
    }
  }
  if (K == 0) return;

  // the slice's certain winners and the candidates of bin d0 into LDS
  bm[t] = wd;
  {
    uint32_t pre = 0;
#pragma unroll
    for (int q = 0; q < 2; ++q)
      pre += __popc(pw[q].x) + __popc(pw[q].y) + __popc(pw[q].z) + __popc(pw[q].w);
    // rows past 2^18 tokens: the words before the slice beyond the first
    // kBitmapWords (w0 is a multiple of 4, so no load reaches the slice)
    for (int w = 4 * (t + 2 * NT); w < w0; w += 4 * NT) {
      const uint4 x = *reinterpret_cast<const uint4*>(bmg + w);
      pre += __popc(x.x) + __popc(x.y) + __popc(x.z) + __popc(x.w);
    }
    pre = wave_sum(pre);
    if ((t & 63) == 0) wcnt[t >> 6] = pre;
  }
  for (int i = t; i < static_cast<int>(c); i += NT) {
    const uint2 e = i < NT ? e_first : cl[i];
    cu[i] = e.x;
    ci[i] = e.y;
  }
  for (int b = t; b < kBins1; b += NT) hA[b] = 0u;
  if (t < kBins2) hB[t] = 0u;
  __syncthreads();
  // exact threshold among the candidates: digits 1 and 2 (rank r0); every
  // workgroup of the row finds the same one
  for (int i = t; i < static_cast<int>(c); i += NT)
    atomicAdd(&hA[(cu[i] >> kShift1) & (kBins1 - 1)], 1u);
  __syncthreads();
  find_digit<NT, kBins1>(hA, r0, false, sm, res);
  const uint32_t d1 = res[0], r1 = res[1];
  // a digit-1 bin taken whole (rank inside it == its count): every candidate
  // at or above its lower edge wins, so that edge is T with every tie winning
  // and the last level is skipped (the same for every thread: LDS counts)
  const bool whole = r1 == hA[d1];
  __syncthreads();
  uint32_t T = (d0 << kShift0) | (d1 << kShift1), K2 = 0, n_eq = 0;
  if (!whole) {
    const uint32_t pre = (d0 << kDigit1Bits) | d1;
    for (int i = t; i < static_cast<int>(c); i += NT)
      if ((cu[i] >> kShift1) == pre) atomicAdd(&hB[cu[i] & (kBins2 - 1)], 1u);
    __syncthreads();
    find_digit<NT, kBins2>(hB, r1, false, sm, res);
    T |= res[0];
    K2 = res[1];
    n_eq = hB[res[0]];                                 // candidates whose key equals T
    __syncthreads();
  }

  // candidate winners (key > T, or key == T among the K2 lowest indices; all
  // ties win when n_eq == K2, the usual case): marked when in the slice,
  // counted when before it
  const uint32_t cut = n_eq == K2 ? 0xFFFFFFFFu
                                  : tie_cut<NT>(cu, ci, static_cast<int>(c), T, K2, n_eq,
                                                len > (1 << 18), hA, hB, sm, res);
  uint32_t cb = 0;
  for (int i = t; i < static_cast<int>(c); i += NT) {
    const uint32_t kv = cu[i], e = ci[i];
    if (kv > T || (kv == T && e <= cut)) {
      const int r = static_cast<int>(e) - s0;
      if (r >= 0 && r < kSlice)
        atomicOr(&bm[r >> 5], 1u << (r & 31));
      else if (r < 0)
        ++cb;
    }
  }
  cb = wave_sum(cb);
  if ((t & 63) == 0) wcnt[t >> 6] += cb;
  __syncthreads();
  uint32_t before = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) before += wcnt[i];

  // ordered emit of the slice: word t holds elements s0 + 32t .. s0 + 32t + 31
  uint32_t bits = bm[t];
  uint32_t tot;
  uint32_t pos = before + block_excl_scan<NT>(__popc(bits), sm, tot);
  while (bits) {
    const int b = __ffs(bits) - 1;
    bits &= bits - 1u;
    const int e = s0 + 32 * t + b;
    if (pos < K) {
      idx_row[pos] = e;
      if (score_row) score_row[pos] = key_score(row[e]);
    }
    ++pos;
  }
}

// ---------------------------------------------------------------- short rows in registers
// Rows of at most kSmallRow elements (MISA-dagger's rerank, the block
// prefilter's selects, short decode rows): one workgroup per row, of 256, 512
// or 1024 threads (as few as hold the row); thread t holds elements
// 16t .. 16t+15 in registers for every pass.  The
// keys of such a row are often close together (re-scored candidates, block
// scores), so the radix digits are taken on key - min over the row's key
// range (digits [sA, 32), [sB, sA), [0, sB) with (max - min) >> sA < 4096),
// which spreads the histogram's LDS atomics; a row whose range fits 12 bits
// needs one level.  Ties at the threshold T go to the lowest indices: a
// thread's elements are contiguous, so a block prefix of the per-thread tie
// counts ranks them (skipped when every tie wins).  Outputs in index order
// from a block prefix of the per-thread winner counts.
constexpr int kSmallRow = 1024 * kPerThread;

// Block prefix with one barrier: exclusive prefix of v over the threads in
// index order and the total.  `sm` (NT/64 words) must not be in use by a
// previous call that some thread may still be reading.
template <int NT>
__device__ __forceinline__ uint32_t block_prefix1(uint32_t v, uint32_t* sm, uint32_t& total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan(v);
  if (lane == 63) sm[wid] = incl;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const uint32_t s = sm[i];
    before += (i < wid) ? s : 0u;
    tot += s;
  }
  total = tot;
  return before + incl - v;
}

// The bin of an NBINS-bin histogram (bin NBINS-1 = largest keys) holding the
// K-th largest element, 1 <= K <= its total, with two barriers (the
// histogram's updates must be complete, i.e. a barrier between them and this
// call).  res[0] = bin, res[1] = rank of the element inside the bin (1-based).
template <int NT, int NBINS>
__device__ __forceinline__ void locate_bin(const uint32_t* hist, uint32_t K, uint32_t* sm,
                                           uint32_t* res) {
  constexpr int PER = NBINS >= NT ? NBINS / NT : 1;
  const int t = static_cast<int>(threadIdx.x);
  const bool owner = NBINS >= NT || t < NBINS;
  const int lo = NBINS - (t + 1) * PER;
  uint32_t vb[PER];
  uint32_t c = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    vb[q] = owner ? hist[lo + q] : 0u;
    c += vb[q];
  }
  uint32_t total;
  const uint32_t above = block_prefix1<NT>(c, sm, total);
  if (owner && above < K && K <= above + c) {
    uint32_t acc = above;
#pragma unroll
    for (int q = PER - 1; q >= 0; --q) {
      if (acc < K && acc + vb[q] >= K) {
        res[0] = static_cast<uint32_t>(lo + q);
        res[1] = K - acc;
      }
      acc += vb[q];
    }
  }
  __syncthreads();
}

// The selection of one row whose elements sit in registers: thread t holds
// elements PT*t .. PT*t+PT-1 (in index order, PT <= 32) as order keys v (0 = empty) and
// their output indices ct; the min(topk, valid) first under (key desc, index
// asc) are written in index order to idx_row / score_row, then the padding.
// NT threads; LDS: two 4096-word histograms and a 256-word one, sm
// [4][NT/64], res [3][4], wmin / wmax [NT/64].
template <int NT, int PT>
__device__ __forceinline__ void select_in_registers(const uint32_t (&v)[PT],
                                                    const int32_t (&ct)[PT], int topk,
                                                    int32_t* idx_row, float* score_row,
                                                    uint32_t* hA, uint32_t* hA2, uint32_t* hB,
                                                    uint32_t (*sm)[NT / 64], uint32_t (*res)[4],
                                                    uint32_t* wmin, uint32_t* wmax) {
  static_assert(NT >= kBins2, "one thread per level-2 bin clears the histogram");
  const int tid = static_cast<int>(threadIdx.x);
  for (int b = tid; b < kBins0; b += NT) {
    hA[b] = 0u;
    hA2[b] = 0u;
  }
  if (tid < kBins2) hB[tid] = 0u;
  uint32_t lo = 0xFFFFFFFFu, hi = 0u, nv = 0;
#pragma unroll
  for (int j = 0; j < PT; ++j) {
    if (v[j] != 0u) {
      lo = min(lo, v[j]);
      hi = max(hi, v[j]);
      ++nv;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    lo = min(lo, static_cast<uint32_t>(__shfl_xor(static_cast<int>(lo), o, 64)));
    hi = max(hi, static_cast<uint32_t>(__shfl_xor(static_cast<int>(hi), o, 64)));
  }
  if ((tid & 63) == 0) {
    wmin[tid >> 6] = lo;
    wmax[tid >> 6] = hi;
  }
  uint32_t nv_tot;
  (void)block_prefix1<NT>(nv, sm[0], nv_tot);   // (its barrier also publishes wmin / wmax)
  const uint32_t K = min(static_cast<uint32_t>(topk), nv_tot);
  uint32_t T = 0, K2 = 0, n_eq = 0;
  if (K > 0) {
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
      kmin = min(kmin, wmin[w]);
      kmax = max(kmax, wmax[w]);
    }
    const uint32_t base = kmin, range = kmax - kmin;
    int sA = 0;
    while ((range >> sA) >= static_cast<uint32_t>(kBins0)) ++sA;
    const int sB = sA > 12 ? sA - 12 : 0;
#pragma unroll
    for (int j = 0; j < PT; ++j)
      if (v[j] != 0u) atomicAdd(&hA[(v[j] - base) >> sA], 1u);
    __syncthreads();
    locate_bin<NT, kBins0>(hA, K, sm[1], res[0]);
    const uint32_t dA = res[0][0];
    uint32_t r = res[0][1], dB = 0, dC = 0;
    n_eq = hA[dA];
    // a threshold bin taken whole (rank inside it == its count) ends the
    // search: every key at or above its lower edge wins and no tie straddles
    // the cut (the same for every thread: the counts are in LDS)
    bool whole = r == n_eq;
    if (sA > 0 && !whole) {
      const uint32_t mB = (1u << (sA - sB)) - 1u;
#pragma unroll
      for (int j = 0; j < PT; ++j)
        if (v[j] != 0u && ((v[j] - base) >> sA) == dA)
          atomicAdd(&hA2[((v[j] - base) >> sB) & mB], 1u);
      __syncthreads();
      locate_bin<NT, kBins0>(hA2, r, sm[2], res[1]);
      dB = res[1][0];
      r = res[1][1];
      n_eq = hA2[dB];
      whole = r == n_eq;
      if (sB > 0 && !whole) {                 // sB <= 8
        const uint32_t preB = (dA << (sA - sB)) | dB;
#pragma unroll
        for (int j = 0; j < PT; ++j)
          if (v[j] != 0u && ((v[j] - base) >> sB) == preB)
            atomicAdd(&hB[(v[j] - base) & ((1u << sB) - 1u)], 1u);
        __syncthreads();
        locate_bin<NT, kBins2>(hB, r, sm[3], res[2]);
        dC = res[2][0];
        r = res[2][1];
        n_eq = hB[dC];
      }
    }
    if (whole) {
      // winners: keys >= the bin's lower edge (>= base >= 1, so T >= 0 and
      // empty slots, key 0, never win)
      T = base + ((dA << sA) | (dB << sB)) - 1u;
      K2 = 0;
      n_eq = 0;
    } else {
      T = base + ((dA << sA) | (dB << sB) | dC);
      K2 = r;                                 // ties at T that win: the K2 lowest indices
    }
  }
  // this thread's winners: keys above T, and ties ranked by index (every tie
  // wins when K2 == n_eq, the usual case: no ranking needed)
  uint32_t tie_rank = 0;
  if (K2 != n_eq) {
    uint32_t ties = 0;
#pragma unroll
    for (int j = 0; j < PT; ++j) ties += (v[j] == T) ? 1u : 0u;
    uint32_t tie_tot;
    __syncthreads();                          // sm[0] is free again
    tie_rank = block_prefix1<NT>(ties, sm[0], tie_tot);
  }
  uint32_t sel = 0, nsel = 0;
#pragma unroll
  for (int j = 0; j < PT; ++j) {
    const bool eq = K > 0 && v[j] == T;
    const bool win = (K > 0 && v[j] > T) || (eq && tie_rank < K2);
    tie_rank += eq ? 1u : 0u;
    sel |= win ? (1u << j) : 0u;
    nsel += win ? 1u : 0u;
  }
  uint32_t tot;
  // (sm[1]'s readers in the first level's locate_bin passed its closing barrier)
  uint32_t pos = block_prefix1<NT>(nsel, sm[1], tot);
#pragma unroll
  for (int j = 0; j < PT; ++j) {
    if ((sel >> j) & 1u) {
      idx_row[pos] = ct[j];
      if (score_row) score_row[pos] = key_score(v[j]);
      ++pos;
    }
  }
  for (int i = static_cast<int>(K) + tid; i < topk; i += NT) {
    idx_row[i] = -1;
    if (score_row) score_row[i] = -__builtin_inff();
  }
}


template <int NT>
__global__ __launch_bounds__(NT) void topk_small_kernel(
    const uint32_t* __restrict__ u, int u_stride, const int32_t* __restrict__ q_pos,
    int fixed_len, int topk, const int32_t* __restrict__ cand, int cand_stride,
    int32_t* __restrict__ idx, float* __restrict__ score) {
  __shared__ __align__(16) uint32_t hA[kBins0];
  __shared__ __align__(16) uint32_t hA2[kBins0];
  __shared__ __align__(16) uint32_t hB[kBins2];
  __shared__ uint32_t sm[4][NT / 64];
  __shared__ uint32_t res[3][4];
  __shared__ uint32_t wmin[NT / 64], wmax[NT / 64];
  const int n = blockIdx.x, tid = threadIdx.x;
  const int len = row_len(q_pos, fixed_len, n);
  const uint32_t* row = u + static_cast<size_t>(n) * u_stride;
  const int32_t* cand_row = cand ? cand + static_cast<size_t>(n) * cand_stride : nullptr;
  int32_t* idx_row = idx + static_cast<size_t>(n) * topk;
  float* score_row = score ? score + static_cast<size_t>(n) * topk : nullptr;
  const int i0 = tid * kPerThread;
  uint32_t v[kPerThread];
  int32_t ct[kPerThread];                     // the elements' output indices
  if (i0 < len) {
    load16(row, i0, len, v);                  // in bounds: rows are padded to whole chunks
  } else {
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) v[j] = 0u;
  }
#pragma unroll
  for (int j = 0; j < kPerThread; ++j)
    ct[j] = cand_row ? (i0 + j < len ? cand_row[i0 + j] : -1) : i0 + j;
  select_in_registers<NT, kPerThread>(v, ct, topk, idx_row, score_row, hA, hA2, hB, sm, res,
                                      wmin, wmax);
}

__global__ void topk_clear_kernel(uint32_t* __restrict__ p, size_t n_words) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n_words;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

// ---------------------------------------------------------------- one row per workgroup
// Two sweeps over the row: (1) level-0 histogram; (2) certain winners into an
// LDS bitmap, candidates of the threshold bin into an LDS list.  The
// candidates are resolved and the winners emitted exactly as in topk_final.
// Rows longer than the LDS bitmap, or with more threshold-bin candidates than
// fit in LDS, take the full radix path (row_select).
__global__ __launch_bounds__(1024) void topk_row_kernel(
    const uint32_t* __restrict__ u, int u_stride, const int32_t* q_pos, int fixed_len, int topk,
    const int32_t* __restrict__ cand, int cand_stride, int32_t* __restrict__ idx,
    float* __restrict__ score, const uint32_t* __restrict__ row_flag) {
  __shared__ __align__(16) uint32_t bm[kBitmapWords];
  __shared__ __align__(16) uint32_t cu[kCandCap];
  __shared__ __align__(16) uint32_t ci[kCandCap];
  __shared__ __align__(16) uint32_t hA[kBins0];
  __shared__ __align__(16) uint32_t hB[kBins2];
  __shared__ uint32_t sm[16];
  __shared__ uint32_t res[4];
  __shared__ uint32_t n_cand;
  const int n = blockIdx.x;
  if (row_flag && row_flag[n] == 0u) return;
  const int len = row_len(q_pos, fixed_len, n);
  const uint32_t* row = u + static_cast<size_t>(n) * u_stride;
  const int32_t* cand_row = cand ? cand + static_cast<size_t>(n) * cand_stride : nullptr;
  int32_t* idx_row = idx + static_cast<size_t>(n) * topk;
  float* score_row = score ? score + static_cast<size_t>(n) * topk : nullptr;
  const int span = (len + kPerThread - 1) / kPerThread * kPerThread;
  const int nwords = (len + 31) / 32;
  if (nwords > kBitmapWords) {
    row_select<1024>(row, len, topk, cand_row, idx_row, score_row, hA, cu, hB, false, sm, res);
    return;
  }
  for (int b = threadIdx.x; b < kBins0; b += 1024) hA[b] = 0u;
  if (threadIdx.x < kBins2) hB[threadIdx.x] = 0u;
  if (threadIdx.x == 0) n_cand = 0u;
  __syncthreads();
  hist_range<1024, 0>(row, span, len, 0u, hA);
  __syncthreads();
  find_digit<1024, kBins0>(hA, static_cast<uint32_t>(topk), true, sm, res);
  const uint32_t K = res[2], d0 = res[0], r0 = res[1];
  __syncthreads();
  for (int i = static_cast<int>(K) + threadIdx.x; i < topk; i += 1024) {
    idx_row[i] = -1;
    if (score_row) score_row[i] = -__builtin_inff();
  }
  if (K == 0) return;
  // sweep 2: bitmap of certain winners, candidate list of bin d0
  for (int i0 = static_cast<int>(threadIdx.x) * kPerThread; i0 < ((span + 31) / 32) * 32;
       i0 += 1024 * kPerThread) {
    uint32_t v[16];
    if (i0 < span) {
      load16(row, i0, len, v);
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = 0u;
    }
    uint32_t sure = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t dg = v[j] >> kShift0;
      sure |= (v[j] != 0u && dg > d0) ? (1u << j) : 0u;
      if (v[j] != 0u && dg == d0) {
        const uint32_t slot = atomicAdd(&n_cand, 1u);
        if (slot < static_cast<uint32_t>(kCandCap)) {
          cu[slot] = v[j];
          ci[slot] = static_cast<uint32_t>(i0 + j);
        }
      }
    }
    const uint32_t other = __shfl_xor(sure, 1, 64);
    if ((threadIdx.x & 1) == 0 && (i0 >> 5) < nwords) bm[i0 >> 5] = sure | (other << 16);
  }
  for (int b = threadIdx.x; b < kBins1; b += 1024) hA[b] = 0u;
  __syncthreads();
  const uint32_t c = n_cand;
  if (c > static_cast<uint32_t>(kCandCap)) {
    __syncthreads();
    row_select<1024>(row, len, topk, cand_row, idx_row, score_row, hA, cu, hB, false, sm, res);
    return;
  }
  // exact threshold among the candidates: digits 1 and 2 (rank r0)
  for (int i = threadIdx.x; i < static_cast<int>(c); i += 1024)
    atomicAdd(&hA[(cu[i] >> kShift1) & (kBins1 - 1)], 1u);
  __syncthreads();
  find_digit<1024, kBins1>(hA, r0, false, sm, res);
  const uint32_t d1 = res[0], r1 = res[1];
  // a digit-1 bin taken whole: its lower edge is T, every tie wins, and the
  // last level is skipped
  const bool whole = r1 == hA[d1];
  __syncthreads();
  uint32_t T = (d0 << kShift0) | (d1 << kShift1), K2 = 0, n_eq = 0;
  if (!whole) {
    const uint32_t pre = (d0 << kDigit1Bits) | d1;
    for (int i = threadIdx.x; i < static_cast<int>(c); i += 1024)
      if ((cu[i] >> kShift1) == pre) atomicAdd(&hB[cu[i] & (kBins2 - 1)], 1u);
    __syncthreads();
    find_digit<1024, kBins2>(hB, r1, false, sm, res);
    T |= res[0];
    K2 = res[1];
    n_eq = hB[res[0]];
    __syncthreads();
  }
  // mark the candidate winners: key > T, or key == T among the K2 lowest
  // indices (all ties win when n_eq == K2, the usual case)
  const uint32_t cut = n_eq == K2 ? 0xFFFFFFFFu
                                  : tie_cut<1024>(cu, ci, static_cast<int>(c), T, K2, n_eq, false,
                                                  hA, hB, sm, res);
  for (int i = threadIdx.x; i < static_cast<int>(c); i += 1024) {
    const uint32_t kv = cu[i], e = ci[i];
    if (kv > T || (kv == T && e <= cut)) atomicOr(&bm[e >> 5], 1u << (e & 31));
  }
  __syncthreads();
  // ordered emit of every marked element
  uint32_t base_pos = 0;
  for (int w0 = 0; w0 < nwords; w0 += 4 * 1024) {
    const int w = w0 + 4 * threadIdx.x;
    uint32_t wd[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) wd[q] = (w + q < nwords) ? bm[w + q] : 0u;
    const uint32_t cnt = __popc(wd[0]) + __popc(wd[1]) + __popc(wd[2]) + __popc(wd[3]);
    uint32_t tot;
    uint32_t pos = base_pos + block_excl_scan<1024>(cnt, sm, tot);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t bits = wd[q];
      while (bits) {
        const int b = __ffs(bits) - 1;
        bits &= bits - 1u;
        const uint32_t e = static_cast<uint32_t>(32 * (w + q) + b);
        if (pos < K) {
          idx_row[pos] = cand_row ? cand_row[e] : static_cast<int32_t>(e);
          if (score_row) score_row[pos] = key_score(row[e]);
        }
        ++pos;
      }
    }
    base_pos += tot;
  }
}


// ---------------------------------------------------------------- prefill candidate path
// A row's exact top-k only needs the keys at or above any threshold that at
// least min(k, L_n) keys reach.  topk_tau picks such a threshold per row from
// a strided sample of the row's scores (aiming at about twice the wanted
// count), the scoring GEMM keeps only the keys at or above it, and
// topk_cand selects exactly among them.  Whether the threshold was low enough
// is checked exactly (the candidate count), so a poor sample only costs time:
// such rows are flagged and take the full path.

constexpr int kCandRow = 8192;        // candidates per row resolved in LDS

__global__ __launch_bounds__(256) void topk_tau_kernel(const uint32_t* __restrict__ us,
                                                       int us_stride,
                                                       const int32_t* __restrict__ q_pos,
                                                       int topk, int shift, int rows_per_block,
                                                       float* __restrict__ tau,
                                                       uint32_t* __restrict__ block_flag) {
  __shared__ __align__(16) uint32_t hA[kBins0];
  __shared__ uint32_t sm[4];
  __shared__ uint32_t res[4];
  const int n = blockIdx.x;
  if (threadIdx.x == 0 && n % rows_per_block == 0) block_flag[n / rows_per_block] = 0u;
  const int pos = q_pos[n];
  const int len = pos + 1;
  const int m = (pos >> shift) + 1;                    // visible samples
  const int K = min(topk, len);
  // sample rank whose key about 1.75 K of the row's keys reach (the k-th
  // score lies below it unless the sample overstates the top keys by ~6
  // standard deviations at L = 64K, k = 2048); at least min(K, 32), since the
  // sampled keys are row keys themselves
  long long r = (7LL * K * m + 4LL * len - 1) / (4LL * len);
  r = max(r, static_cast<long long>(min(K, 32)));
  r = min(r, static_cast<long long>(m));
  const uint32_t* row = us + static_cast<size_t>(n) * us_stride;
  // the sample keys in batches of 16 per thread, all loads of a batch issued
  // before the first histogram update (one round trip per batch, not one per
  // key); out-of-range slots reread key 0 and are skipped
  constexpr int PB = 16;
  // a row of at most one batch (4096 samples: L <= 128K at a stride of 32)
  // keeps its batch in registers for the second level instead of reading
  // it again
  const bool one = m <= 256 * PB;
  bool held = false;                                   // vb holds the row's one batch
  uint32_t vb[PB];
  auto sweep = [&](auto&& use) {
    for (int i0 = 0; i0 < m; i0 += 256 * PB) {
      if (!held) {
#pragma unroll
        for (int u = 0; u < PB; ++u) {
          const int i = i0 + static_cast<int>(threadIdx.x) + 256 * u;
          vb[u] = row[i < m ? i : 0];
        }
        held = one;
      }
#pragma unroll
      for (int u = 0; u < PB; ++u)
        if (i0 + static_cast<int>(threadIdx.x) + 256 * u < m) use(vb[u]);
    }
  };
  for (int b = threadIdx.x; b < kBins0; b += 256) hA[b] = 0u;
  __syncthreads();
  sweep([&](uint32_t v) { atomicAdd(&hA[v >> kShift0], 1u); });
  __syncthreads();
  find_digit<256, kBins0>(hA, static_cast<uint32_t>(r), true, sm, res);
  const uint32_t d0 = res[0], r0 = res[1];
  for (int b = threadIdx.x; b < kBins1; b += 256) hA[b] = 0u;
  __syncthreads();
  sweep([&](uint32_t v) {
    if ((v >> kShift0) == d0) atomicAdd(&hA[(v >> kShift1) & (kBins1 - 1)], 1u);
  });
  __syncthreads();
  find_digit<256, kBins1>(hA, r0, false, sm, res);
  if (threadIdx.x == 0) {
    // lower end of the sample's 24-bit key bin, at least the key of -FLT_MAX
    // (every finite score's key is), as a score
    const uint32_t t = (d0 << kShift0) | (res[0] << kShift1);
    tau[n] = key_score(t > 0x00800000u ? t : 0x00800000u);
  }
}

// One 512-thread workgroup per row.  The row's candidate lists, concatenated
// split after split, are in ascending token order (each list in key order,
// the splits in key-range order), so thread t takes the concatenated
// candidates 16t .. 16t+15 into registers and the row is selected like a
// short row (select_in_registers): a row of up to kCandRow candidates, its
// outputs already in token order.  (Measured: 3 of these workgroups per CU
// beat 2 of 1024 threads with 8 candidates each, and 4 capped at 64 VGPRs,
// which spill.)
constexpr int kCandThreads = 512;
constexpr int kCandPer = kPerThread;     // candidates per thread
constexpr int kCandMaxK = kBins0 / 2;    // selected per row at most
static_assert(kCandThreads * kCandPer >= kCandRow, "a row's candidates fit the registers");

__global__ __launch_bounds__(kCandThreads) void topk_cand_kernel(
    const uint32_t* __restrict__ cnt, const uint2* __restrict__ cand, int splits, int cap,
    const int32_t* __restrict__ q_pos, int topk, int rows_per_block,
    uint32_t* __restrict__ row_flag, uint32_t* __restrict__ block_flag,
    int32_t* __restrict__ idx, float* __restrict__ score) {
  constexpr int NT = kCandThreads;
  __shared__ __align__(16) uint32_t hA[kBins0];
  __shared__ __align__(16) uint32_t hA2[kBins0];
  __shared__ __align__(16) uint32_t hB[kBins2];
  __shared__ uint32_t spre[257];
  __shared__ uint32_t sm[4][NT / 64];
  __shared__ uint32_t res[3][4];
  __shared__ uint32_t wmin[NT / 64], wmax[NT / 64];
  __shared__ uint32_t bad;
  const int n = blockIdx.x;
  const int tid = threadIdx.x;
  const int len = q_pos[n] + 1;
  const uint32_t K = static_cast<uint32_t>(min(topk, len));
  // split counts -> offsets; overflow check
  uint32_t cs = 0;
  if (tid < splits) cs = cnt[static_cast<size_t>(n) * splits + tid];
  if (tid == 0) bad = 0u;
  __syncthreads();
  if (cs > static_cast<uint32_t>(cap)) bad = 1u;
  uint32_t total;
  const uint32_t before = block_excl_scan<NT>(cs, sm[0], total);
  if (tid < splits) spre[tid] = before;
  if (tid == 0) spre[splits] = total;
  __syncthreads();
  const bool flag = bad != 0u || total < K || total > static_cast<uint32_t>(kCandRow);
  if (flag) {
    if (tid == 0) {
      row_flag[n] = 1u;
      atomicOr(&block_flag[n / rows_per_block], 1u);
    }
    return;
  }
  // this thread's candidates p0 .. p0+15 (positions past the total read the
  // last candidate and are marked empty): the list holding each position is
  // the last split s with spre[s] <= p, found by bisection for the first and
  // by stepping for the rest; then the 16 loads, all in flight together
  const int p0 = tid * kCandPer;
  const int last = static_cast<int>(total) - 1;
  int sp;
  {
    const uint32_t p = static_cast<uint32_t>(min(p0, last));
    int lo = 0, hi = splits - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (spre[mid] <= p) lo = mid; else hi = mid - 1;
    }
    sp = lo;
  }
  uint32_t off[kCandPer];
#pragma unroll
  for (int j = 0; j < kCandPer; ++j) {
    const uint32_t p = static_cast<uint32_t>(min(p0 + j, last));
    while (spre[sp + 1] <= p) ++sp;
    off[j] = static_cast<uint32_t>(sp) * static_cast<uint32_t>(cap) + (p - spre[sp]);
  }
  const uint2* crow = cand + static_cast<size_t>(n) * splits * cap;
  uint32_t v[kCandPer];
  int32_t ct[kCandPer];
#pragma unroll
  for (int j = 0; j < kCandPer; ++j) {
    const uint2 e = crow[off[j]];
    v[j] = e.x;
    ct[j] = static_cast<int32_t>(e.y);
  }
#pragma unroll
  for (int j = 0; j < kCandPer; ++j) {
    const bool ok = p0 + j <= last;
    v[j] = ok ? order_key(__uint_as_float(v[j])) : 0u;
    ct[j] = ok ? ct[j] : -1;
  }
  if (tid == 0) row_flag[n] = 0u;
  int32_t* idx_row = idx + static_cast<size_t>(n) * topk;
  float* score_row = score ? score + static_cast<size_t>(n) * topk : nullptr;
  select_in_registers<NT, kCandPer>(v, ct, topk, idx_row, score_row, hA, hA2, hB, sm, res, wmin,
                                    wmax);
}

}  // namespace

size_t topk_few_rows_bytes(int N, int u_stride) {
  // hist | bitmap | candidate list, each 256-byte aligned
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  return al(static_cast<size_t>(N) * kHistWords * 4) + al(static_cast<size_t>(N) * u_stride / 8) +
         al(static_cast<size_t>(N) * kCandCap * 8);
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  if (a.one_row_per_block && !a.row_flag && a.u_stride <= kSmallRow) {
    // as few threads as hold the row (16 elements each): fewer wavefronts
    // in every barrier of the select
    if (a.u_stride <= 256 * kPerThread)
      MISA_LAUNCH(K_TOPK_ROW, topk_small_kernel<256>, dim3(a.N), dim3(256), 0, st, a.u,
                  a.u_stride, a.q_pos, a.fixed_len, a.topk, a.cand, a.cand_stride, a.idx, a.score);
    else if (a.u_stride <= 512 * kPerThread)
      MISA_LAUNCH(K_TOPK_ROW, topk_small_kernel<512>, dim3(a.N), dim3(512), 0, st, a.u,
                  a.u_stride, a.q_pos, a.fixed_len, a.topk, a.cand, a.cand_stride, a.idx, a.score);
    else
      MISA_LAUNCH(K_TOPK_ROW, topk_small_kernel<1024>, dim3(a.N), dim3(1024), 0, st, a.u,
                  a.u_stride, a.q_pos, a.fixed_len, a.topk, a.cand, a.cand_stride, a.idx, a.score);
    return hipGetLastError();
  }
  if (a.one_row_per_block) {
    MISA_LAUNCH(K_TOPK_ROW, topk_row_kernel, dim3(a.N), dim3(1024), 0, st, a.u, a.u_stride,
                a.q_pos, a.fixed_len, a.topk, a.cand, a.cand_stride, a.idx, a.score, a.row_flag);
    return hipGetLastError();
  }
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  uint8_t* base = reinterpret_cast<uint8_t*>(a.hist);
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(base + al(static_cast<size_t>(a.N) * kHistWords * 4));
  uint2* clist = reinterpret_cast<uint2*>(reinterpret_cast<uint8_t*>(bitmap) +
                                          al(static_cast<size_t>(a.N) * a.u_stride / 8));
  const int nchunks = a.u_stride / kChunk;
  MISA_LAUNCH(K_TOPK_COLLECT, topk_collect_kernel, dim3(nchunks, a.N), dim3(256), 0, st, a.u,
              a.u_stride, a.q_pos, a.fixed_len, a.hist, bitmap, clist, a.topk);
  const int nslices = (a.u_stride + 32 * kFinalThreads - 1) / (32 * kFinalThreads);
  MISA_LAUNCH(K_TOPK_FINAL, topk_final_kernel<kFinalThreads>, dim3(nslices, a.N),
              dim3(kFinalThreads), 0, st, a.u, a.u_stride,
              a.q_pos, a.fixed_len, a.hist, bitmap, clist, a.topk, a.idx, a.score);
  return hipGetLastError();
}

hipError_t launch_clear(uint32_t* p, size_t n_words, hipStream_t st) {
  if (n_words == 0) return hipSuccess;
  size_t blocks = (n_words + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  MISA_LAUNCH(K_CLEAR, topk_clear_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st,
              p, n_words);
  return hipGetLastError();
}

int topk_chunk() { return kChunk; }

int topk_small_row() { return kSmallRow; }

int cand_topk_capacity() { return kCandRow; }

hipError_t launch_tau(const TauArgs& a, hipStream_t st) {
  MISA_LAUNCH(K_TOPK_TAU, topk_tau_kernel, dim3(a.N), dim3(256), 0, st, a.us, a.us_stride,
              a.q_pos, a.topk, a.sample_shift, a.rows_per_block, a.tau, a.block_flag);
  return hipGetLastError();
}

hipError_t launch_cand_topk(const CandTopkArgs& a, hipStream_t st) {
  if (a.splits < 1 || a.splits > 256 || a.topk > kCandMaxK) return hipErrorInvalidValue;
  MISA_LAUNCH(K_TOPK_CAND, topk_cand_kernel, dim3(a.N), dim3(kCandThreads), 0, st, a.cnt, a.cand,
              a.splits, a.cap, a.q_pos, a.topk, a.rows_per_block, a.row_flag, a.block_flag, a.idx,
              a.score);
  return hipGetLastError();
}

}  // namespace misa
