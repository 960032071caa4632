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
//  topk_final (one 1024-thread workgroup per row) loads the bitmap and the
//    candidates into LDS, resolves the exact threshold among the candidates
//    with two more radix levels, marks the candidate winners in the bitmap
//    and emits every marked element in index order.  When the candidates do
//    not fit in LDS (heavily tied scores) or the row is very long, the same
//    workgroup falls back to a full radix select over the row.
// Many rows or short rows (prefill, rerank): topk_row, one 1024-thread
//    workgroup per row with every histogram in LDS.
#include "common.hpp"
#include "kernels.hpp"

namespace misa {
namespace {

constexpr int kChunk = 4096;          // elements per collect workgroup
constexpr int kPerThread = 16;        // contiguous elements per thread per tile
constexpr int kCandCap = 8192;        // candidates resolved in LDS
constexpr int kBitmapWords = 8192;    // rows up to 262144 elements use the LDS bitmap

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
// Radix select on the indices (< 2^18: bits 6..17, then 0..5) in hA (4096
// words) and hB (64 words); every thread calls it.
template <int NT>
__device__ __forceinline__ uint32_t tie_cut(const uint32_t* cu, const uint32_t* ci, int total,
                                            uint32_t T, uint32_t K2, uint32_t n_eq, uint32_t* hA,
                                            uint32_t* hB, uint32_t* sm, uint32_t* res) {
  for (int b = threadIdx.x; b < 4096; b += NT) hA[b] = 0u;
  if (threadIdx.x < 64) hB[threadIdx.x] = 0u;
  __syncthreads();
  for (int i = threadIdx.x; i < total; i += NT)
    if (cu[i] == T) atomicAdd(&hA[ci[i] >> 6], 1u);
  __syncthreads();
  // the K2-th smallest index is the (n_eq - K2 + 1)-th largest
  find_digit<NT, 4096>(hA, n_eq - K2 + 1u, false, sm, res);
  const uint32_t dA = res[0], rA = res[1];
  for (int i = threadIdx.x; i < total; i += NT)
    if (cu[i] == T && (ci[i] >> 6) == dA) atomicAdd(&hB[ci[i] & 63u], 1u);
  __syncthreads();
  find_digit<NT, 64>(hB, rA, false, sm, res);
  const uint32_t cut = (dA << 6) | res[0];
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
  hist_range<NT, 1>(row, span, len, d0, h1);
  __syncthreads();
  find_digit<NT, kBins1>(h1, r0, false, sm, res);
  const uint32_t d1 = res[0], r1 = res[1];
  __syncthreads();
  hist_range<NT, 2>(row, span, len, (d0 << kDigit1Bits) | d1, h2);
  __syncthreads();
  find_digit<NT, kBins2>(h2, r1, false, sm, res);
  Threshold th;
  th.K = K;
  th.T = (d0 << kShift0) | (d1 << kShift1) | res[0];
  th.K2 = res[1];
  __syncthreads();
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

__global__ __launch_bounds__(1024) void topk_final_kernel(
    const uint32_t* __restrict__ u, int u_stride, const int32_t* __restrict__ q_pos,
    int fixed_len, const uint32_t* hist, const uint32_t* __restrict__ bitmap,
    const uint2* __restrict__ clist, int topk, int32_t* __restrict__ idx,
    float* __restrict__ score) {
  __shared__ __align__(16) uint32_t bm[kBitmapWords];   // winners, one bit per element
  __shared__ __align__(16) uint32_t cu[kCandCap];       // candidate order key
  __shared__ __align__(16) uint32_t ci[kCandCap];       // candidate element index
  __shared__ __align__(16) uint32_t hA[kBins0];
  __shared__ __align__(16) uint32_t hB[kBins2];
  __shared__ uint32_t sm[16];
  __shared__ uint32_t res[4];
  const int n = blockIdx.x;
  const int len = row_len(q_pos, fixed_len, n);
  const uint32_t* row = u + static_cast<size_t>(n) * u_stride;
  const uint32_t* h0g = hist + static_cast<size_t>(n) * kHistWords;
  int32_t* idx_row = idx + static_cast<size_t>(n) * topk;
  float* score_row = score ? score + static_cast<size_t>(n) * topk : nullptr;
  const int nwords = (len + 31) / 32;

  // the bitmap words (certain winners) and the candidate count are read in
  // the same round trip as the level-0 histogram
  const uint32_t* bmg = bitmap + static_cast<size_t>(n) * (u_stride / 32);
  uint4 bw[kBitmapWords / 4096];
#pragma unroll
  for (int q = 0; q < kBitmapWords / 4096; ++q) {
    const int w = 4 * (threadIdx.x + q * 1024);
    bw[q] = w + 3 < nwords ? *reinterpret_cast<const uint4*>(bmg + w) : make_uint4(0u, 0u, 0u, 0u);
    if (w < nwords && w + 3 >= nwords) {          // ragged last words
      bw[q].x = bmg[w];
      if (w + 1 < nwords) bw[q].y = bmg[w + 1];
      if (w + 2 < nwords) bw[q].z = bmg[w + 2];
    }
  }
  const uint32_t c = h0g[kCandCountOffset];
  // the first candidate of every thread, read before the count is known (the
  // list holds kCandCap >= 1024 entries, so the read stays inside it)
  const uint2* cl = clist + static_cast<size_t>(n) * kCandCap;
  static_assert(kCandCap >= 1024, "one speculative candidate per thread");
  const uint2 e_first = cl[threadIdx.x];
  find_digit<1024, kBins0>(h0g, static_cast<uint32_t>(topk), true, sm, res);
  const uint32_t K = res[2], d0 = res[0], r0 = res[1];
  __syncthreads();
  bool fallback = c > static_cast<uint32_t>(kCandCap) || nwords > kBitmapWords;
  uint32_t T = 0, K2 = 0, n_eq = 0;
  if (!fallback && K > 0) {
    // certain winners (bitmap) and the candidates of bin d0 into LDS
#pragma unroll
    for (int q = 0; q < kBitmapWords / 4096; ++q)
      *reinterpret_cast<uint4*>(&bm[4 * (threadIdx.x + q * 1024)]) = bw[q];
    for (int i = threadIdx.x; i < static_cast<int>(c); i += 1024) {
      const uint2 e = i < 1024 ? e_first : cl[i];
      cu[i] = e.x;
      ci[i] = e.y;
    }
    for (int b = threadIdx.x; b < kBins1; b += 1024) hA[b] = 0u;
    if (threadIdx.x < kBins2) hB[threadIdx.x] = 0u;
    __syncthreads();
    // exact threshold among the candidates: digits 1 and 2 (rank r0)
    for (int i = threadIdx.x; i < static_cast<int>(c); i += 1024)
      atomicAdd(&hA[(cu[i] >> kShift1) & (kBins1 - 1)], 1u);
    __syncthreads();
    find_digit<1024, kBins1>(hA, r0, false, sm, res);
    const uint32_t d1 = res[0], r1 = res[1];
    __syncthreads();
    const uint32_t pre = (d0 << kDigit1Bits) | d1;
    for (int i = threadIdx.x; i < static_cast<int>(c); i += 1024)
      if ((cu[i] >> kShift1) == pre) atomicAdd(&hB[cu[i] & (kBins2 - 1)], 1u);
    __syncthreads();
    find_digit<1024, kBins2>(hB, r1, false, sm, res);
    T = (d0 << kShift0) | (d1 << kShift1) | res[0];
    K2 = res[1];
    n_eq = hB[res[0]];                    // candidates whose key equals T
    __syncthreads();
  }
  if (fallback) {
    for (int b = threadIdx.x; b < kBins0; b += 1024) hA[b] = h0g[b];
    __syncthreads();
    row_select<1024>(row, len, topk, nullptr, idx_row, score_row, hA, cu, hB, true, sm, res);
    return;
  }
  for (int i = static_cast<int>(K) + threadIdx.x; i < topk; i += 1024) {
    idx_row[i] = -1;
    if (score_row) score_row[i] = -__builtin_inff();
  }
  if (K == 0) return;

  // mark the candidate winners: key > T, or key == T among the K2 lowest
  // indices (all ties win when n_eq == K2, the usual case)
  const uint32_t cut = n_eq == K2 ? 0xFFFFFFFFu
                                  : tie_cut<1024>(cu, ci, static_cast<int>(c), T, K2, n_eq, hA,
                                                  hB, sm, res);
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
          idx_row[pos] = static_cast<int32_t>(e);
          if (score_row) score_row[pos] = key_score(row[e]);
        }
        ++pos;
      }
    }
    base_pos += tot;
  }
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
  __syncthreads();
  const uint32_t pre = (d0 << kDigit1Bits) | d1;
  for (int i = threadIdx.x; i < static_cast<int>(c); i += 1024)
    if ((cu[i] >> kShift1) == pre) atomicAdd(&hB[cu[i] & (kBins2 - 1)], 1u);
  __syncthreads();
  find_digit<1024, kBins2>(hB, r1, false, sm, res);
  const uint32_t T = (d0 << kShift0) | (d1 << kShift1) | res[0];
  const uint32_t K2 = res[1];
  const uint32_t n_eq = hB[res[0]];
  __syncthreads();
  // mark the candidate winners: key > T, or key == T among the K2 lowest
  // indices (all ties win when n_eq == K2, the usual case)
  const uint32_t cut = n_eq == K2 ? 0xFFFFFFFFu
                                  : tie_cut<1024>(cu, ci, static_cast<int>(c), T, K2, n_eq, hA,
                                                  hB, sm, res);
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
  auto sweep = [&](auto&& use) {
    for (int i0 = 0; i0 < m; i0 += 256 * PB) {
      uint32_t v[PB];
#pragma unroll
      for (int u = 0; u < PB; ++u) {
        const int i = i0 + static_cast<int>(threadIdx.x) + 256 * u;
        v[u] = row[i < m ? i : 0];
      }
#pragma unroll
      for (int u = 0; u < PB; ++u)
        if (i0 + static_cast<int>(threadIdx.x) + 256 * u < m) use(v[u]);
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

// One 512-thread workgroup per row; each thread keeps up to kCandPer
// candidates in registers.  Dynamic LDS: the row's winner bitmap (nwords_max
// words) and a 16-bit per-word prefix of marked bits.
constexpr int kCandThreads = 512;
constexpr int kCandMaxK = kBins0 / 2;    // selected per row (outputs staged in hA)
constexpr int kCandPer = kCandRow / kCandThreads;

__global__ __launch_bounds__(kCandThreads, 8) void topk_cand_kernel(
    const uint32_t* __restrict__ cnt, const uint2* __restrict__ cand, int splits, int cap,
    const int32_t* __restrict__ q_pos, int topk, int rows_per_block, int nwords_max,
    uint32_t* __restrict__ row_flag, uint32_t* __restrict__ block_flag,
    int32_t* __restrict__ idx, float* __restrict__ score) {
  extern __shared__ __align__(16) uint32_t dyn[];
  __shared__ __align__(16) uint32_t hA[kBins0];
  __shared__ __align__(16) uint32_t hB[kBins2];
  __shared__ uint32_t spre[257];
  __shared__ uint32_t tpre[kCandThreads];
  __shared__ uint16_t bsplit[kCandRow / 32];
  __shared__ uint32_t sm[kCandThreads / 64];
  __shared__ uint32_t res[4];
  __shared__ uint32_t bad;
  constexpr int NT = kCandThreads;
  uint32_t* bm = dyn;
  uint16_t* wpre = reinterpret_cast<uint16_t*>(dyn + nwords_max);
  const int n = blockIdx.x;
  const int tid = threadIdx.x;
  const int len = q_pos[n] + 1;
  const uint32_t K = static_cast<uint32_t>(min(topk, len));
  const int nwords = (len + 31) / 32;
  // split counts -> offsets; overflow check
  uint32_t cs = 0;
  if (tid < splits) cs = cnt[static_cast<size_t>(n) * splits + tid];
  if (tid == 0) bad = 0u;
  __syncthreads();
  if (cs > static_cast<uint32_t>(cap)) bad = 1u;
  uint32_t total;
  const uint32_t before = block_excl_scan<NT>(cs, sm, total);
  if (tid < splits) spre[tid] = before;
  if (tid == 0) spre[splits] = total;
  __syncthreads();
  const bool flag = bad != 0u || total < K || total > static_cast<uint32_t>(kCandRow) ||
                    nwords > nwords_max;
  if (flag) {
    if (tid == 0) {
      row_flag[n] = 1u;
      atomicOr(&block_flag[n / rows_per_block], 1u);
    }
    return;
  }
  // register slots holding candidates (a uniform bound: slots past it are
  // skipped by the whole workgroup)
  const int nsl = __builtin_amdgcn_readfirstlane(static_cast<int>((total + NT - 1) / NT));
  // split of every 32nd element (element j lives in split s with
  // spre[s] <= j < spre[s + 1]; empty splits have spre[s] == spre[s + 1])
  if (tid < kCandRow / 32 && 32 * tid < static_cast<int>(total)) {
    const uint32_t j = 32u * tid;
    int lo = 0, hi = splits - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (spre[mid] <= j) lo = mid; else hi = mid - 1;
    }
    bsplit[tid] = static_cast<uint16_t>(lo);
  }
  __syncthreads();
  // candidates into registers: element j = tid + NT * i, its split found from
  // the one of element 32 * (j / 32) forward; key 0 marks an empty slot
  uint32_t ck[kCandPer], cx[kCandPer];
#pragma unroll
  for (int i = 0; i < kCandPer && i < nsl; ++i) {
    const int j = tid + NT * i;
    ck[i] = 0u;
    cx[i] = 0u;
    if (j < static_cast<int>(total)) {
      int lo = bsplit[j >> 5];
      while (spre[lo + 1] <= static_cast<uint32_t>(j)) ++lo;
      const uint2 e = cand[(static_cast<size_t>(n) * splits + lo) * cap + (j - spre[lo])];
      ck[i] = order_key(__uint_as_float(e.x));
      cx[i] = e.y;
    }
  }
  for (int b = tid; b < kBins0; b += NT) hA[b] = 0u;
  if (tid < kBins2) hB[tid] = 0u;
  __syncthreads();
  // exact threshold: three radix levels over the candidates
#pragma unroll
  for (int i = 0; i < kCandPer && i < nsl; ++i)
    if (ck[i] != 0u) atomicAdd(&hA[ck[i] >> kShift0], 1u);
  __syncthreads();
  find_digit<NT, kBins0>(hA, K, false, sm, res);
  const uint32_t d0 = res[0], r0 = res[1];
  for (int b = tid; b < kBins1; b += NT) hA[b] = 0u;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kCandPer && i < nsl; ++i)
    if (ck[i] != 0u && (ck[i] >> kShift0) == d0) atomicAdd(&hA[(ck[i] >> kShift1) & (kBins1 - 1)], 1u);
  __syncthreads();
  find_digit<NT, kBins1>(hA, r0, false, sm, res);
  const uint32_t d1 = res[0], r1 = res[1];
  const uint32_t pre = (d0 << kDigit1Bits) | d1;
#pragma unroll
  for (int i = 0; i < kCandPer && i < nsl; ++i)
    if (ck[i] != 0u && (ck[i] >> kShift1) == pre) atomicAdd(&hB[ck[i] & (kBins2 - 1)], 1u);
  __syncthreads();
  find_digit<NT, kBins2>(hB, r1, false, sm, res);
  const uint32_t T = (d0 << kShift0) | (d1 << kShift1) | res[0];
  const uint32_t K2 = res[1];
  const uint32_t n_eq = hB[res[0]];
  __syncthreads();
  // ties at T: the K2 lowest token indices win (radix select on the indices,
  // which are < 2^18 here: bits 6..17, then 0..5)
  uint32_t cut = 0xFFFFFFFFu;
  if (n_eq != K2) {
    for (int b = tid; b < kBins0; b += NT) hA[b] = 0u;
    if (tid < 64) hB[tid] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kCandPer && i < nsl; ++i)
      if (ck[i] == T) atomicAdd(&hA[cx[i] >> 6], 1u);
    __syncthreads();
    find_digit<NT, kBins0>(hA, n_eq - K2 + 1u, false, sm, res);
    const uint32_t dA = res[0], rA = res[1];
#pragma unroll
    for (int i = 0; i < kCandPer && i < nsl; ++i)
      if (ck[i] == T && (cx[i] >> 6) == dA) atomicAdd(&hB[cx[i] & 63u], 1u);
    __syncthreads();
    find_digit<NT, 64>(hB, rA, false, sm, res);
    cut = (dA << 6) | res[0];
  }
  if (tid == 0) row_flag[n] = 0u;
  for (int w = tid; w < nwords; w += NT) bm[w] = 0u;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kCandPer && i < nsl; ++i)
    if (ck[i] > T || (ck[i] == T && ck[i] != 0u && cx[i] <= cut))
      atomicOr(&bm[cx[i] >> 5], 1u << (cx[i] & 31));
  __syncthreads();
  // output position of a winner = marked bits before it: thread prefix over
  // wpt consecutive words, plus a 16-bit prefix inside the thread's words
  const int wpt = (nwords + NT - 1) / NT;
  uint32_t mine = 0;
  for (int q = 0; q < wpt; ++q) {
    const int w = tid * wpt + q;
    if (w < nwords) {
      wpre[w] = static_cast<uint16_t>(mine);
      mine += __popc(bm[w]);
    }
  }
  uint32_t tot;
  tpre[tid] = block_excl_scan<NT>(mine, sm, tot);
  __syncthreads();
  // winners to their output slots in LDS (hA: indices, then keys), then out
  // in order with contiguous stores
  uint32_t* oidx = hA;
  uint32_t* okey = hA + kCandMaxK;
#pragma unroll
  for (int i = 0; i < kCandPer && i < nsl; ++i) {
    const uint32_t e = cx[i];
    if (ck[i] == 0u) continue;
    const int w = static_cast<int>(e >> 5);
    const uint32_t word = bm[w];
    if (!((word >> (e & 31)) & 1u)) continue;
    const uint32_t pos = tpre[w / wpt] + wpre[w] + __popc(word & ((1u << (e & 31)) - 1u));
    oidx[pos] = e;
    okey[pos] = ck[i];
  }
  __syncthreads();
  int32_t* idx_row = idx + static_cast<size_t>(n) * topk;
  float* score_row = score ? score + static_cast<size_t>(n) * topk : nullptr;
  for (int i = tid; i < topk; i += NT) {
    const bool sel = i < static_cast<int>(K);
    idx_row[i] = sel ? static_cast<int32_t>(oidx[i]) : -1;
    if (score_row) score_row[i] = sel ? key_score(okey[i]) : -__builtin_inff();
  }
}

}  // namespace

size_t topk_few_rows_bytes(int N, int u_stride) {
  // hist | bitmap | candidate list, each 256-byte aligned
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  return al(static_cast<size_t>(N) * kHistWords * 4) + al(static_cast<size_t>(N) * u_stride / 8) +
         al(static_cast<size_t>(N) * kCandCap * 8);
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
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
  MISA_LAUNCH(K_TOPK_FINAL, topk_final_kernel, dim3(a.N), dim3(1024), 0, st, a.u, a.u_stride,
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

int cand_topk_capacity() { return kCandRow; }

hipError_t launch_tau(const TauArgs& a, hipStream_t st) {
  MISA_LAUNCH(K_TOPK_TAU, topk_tau_kernel, dim3(a.N), dim3(256), 0, st, a.us, a.us_stride,
              a.q_pos, a.topk, a.sample_shift, a.rows_per_block, a.tau, a.block_flag);
  return hipGetLastError();
}

hipError_t launch_cand_topk(const CandTopkArgs& a, hipStream_t st) {
  if (a.splits < 1 || a.splits > 256 || a.topk > kCandMaxK) return hipErrorInvalidValue;
  // bitmap + 16-bit word prefix for the longest row (longer rows are flagged)
  const int nwords_max = min((a.L + 31) / 32, kBitmapWords);
  const size_t lds = static_cast<size_t>(nwords_max) * 4 + (static_cast<size_t>(nwords_max) * 2 + 15) / 16 * 16;
  MISA_LAUNCH(K_TOPK_CAND, topk_cand_kernel, dim3(a.N), dim3(kCandThreads), lds, st, a.cnt,
              a.cand, a.splits, a.cap, a.q_pos, a.topk, a.rows_per_block, nwords_max, a.row_flag,
              a.block_flag, a.idx, a.score);
  return hipGetLastError();
}

}  // namespace misa
