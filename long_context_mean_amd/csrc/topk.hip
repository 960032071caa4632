// Exact top-k selection over fp32 index scores, gfx950.
//
// Scores arrive as 32-bit order keys (order_key: larger score <-> larger key,
// -0 == +0, key 0 = empty slot).  The k-th largest key T is found by a
// three-level radix select (12 + 12 + 8 bit digits) over per-row histograms;
// the selected set is {key > T} plus the first K2 tokens (lowest index) with
// key == T, which realises the order (score desc, token index asc) exactly.
// Results are written in ascending index order by an ordered compaction
// (per-thread runs + workgroup scans), so outputs are deterministic.
//
// Two layouts share the device code:
//  - few long rows (decode): a grid of 4096-element chunks per row; the
//    level-0 histogram comes from the scoring kernel, levels 1-2 and the
//    per-chunk counts go through global memory;
//  - many rows, or short rows (prefill, rerank): one 1024-thread workgroup
//    per row keeps every histogram in LDS.
#include "common.hpp"
#include "kernels.hpp"

namespace misa {
namespace {

constexpr int kChunk = 4096;          // elements per workgroup (few-rows layout)
constexpr int kPerThread = 16;        // contiguous elements per thread per tile

struct Digit {
  uint32_t digit, rank;   // rank (1-based) of the wanted key inside the digit's bin
};

// Scans histogram `hist` (nbins bins, highest bin first) and finds the bin that
// holds the K-th largest element.  With clamp_total, K = min(K, total count)
// first.  Must be called by all NT threads; results in LDS `res` ([0] digit,
// [1] rank, [2] K, [3] total).  K == 0 leaves digit/rank at 0.
template <int NT>
__device__ void find_digit(const uint32_t* hist, int nbins, uint32_t K, bool clamp_total,
                           uint32_t* sm, uint32_t* res) {
  const int per = (nbins + NT - 1) / NT;
  const int hi = nbins - static_cast<int>(threadIdx.x) * per;
  const int lo = hi - per > 0 ? hi - per : 0;
  uint32_t c = 0;
  for (int b = hi - 1; b >= lo; --b) c += hist[b];
  uint32_t total;
  const uint32_t above = block_excl_scan<NT>(c, sm, total);
  if (clamp_total && K > total) K = total;
  if (threadIdx.x == 0) {
    res[0] = 0;
    res[1] = 0;
    res[2] = K;
    res[3] = total;
  }
  __syncthreads();
  if (K > 0 && above < K && K <= above + c) {
    uint32_t acc = above;
    for (int b = hi - 1; b >= lo; --b) {
      const uint32_t hb = hist[b];
      if (acc + hb >= K) {
        res[0] = static_cast<uint32_t>(b);
        res[1] = K - acc;
        break;
      }
      acc += hb;
    }
  }
  __syncthreads();
}

struct Threshold {
  uint32_t T;     // exact k-th largest key
  uint32_t K2;    // number of key == T elements to take (lowest indices)
  uint32_t K;     // number selected = min(topk, valid elements)
};

// Derives the threshold from the three histogram levels (all NT threads).
template <int NT>
__device__ Threshold derive_threshold(const uint32_t* h0, const uint32_t* h1, const uint32_t* h2,
                                      uint32_t topk, uint32_t* sm, uint32_t* res) {
  Threshold th;
  find_digit<NT>(h0, kBins0, topk, true, sm, res);
  th.K = res[2];
  const uint32_t d0 = res[0], r0 = res[1];
  __syncthreads();
  if (th.K == 0) {
    th.T = 0xFFFFFFFFu;
    th.K2 = 0;
    return th;
  }
  find_digit<NT>(h1, kBins1, r0, false, sm, res);
  const uint32_t d1 = res[0], r1 = res[1];
  __syncthreads();
  find_digit<NT>(h2, kBins2, r1, false, sm, res);
  const uint32_t d2 = res[0], r2 = res[1];
  __syncthreads();
  th.T = (d0 << kShift0) | (d1 << kShift1) | d2;
  th.K2 = r2;
  return th;
}

__device__ __forceinline__ int row_len(const int32_t* q_pos, int fixed_len, int n) {
  return q_pos ? q_pos[n] + 1 : fixed_len;
}

// Loads 16 consecutive keys starting at element i0 (row stride is a multiple
// of the chunk size, so the loads stay inside the buffer); keys at or past
// `len` read as 0 (empty).
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

// Histogram of digit `level` over elements [i_begin, i_end) of a row that
// match the higher digits in `prefix`, accumulated into LDS `lh` (NT threads).
template <int NT, int LEVEL>
__device__ void hist_range(const uint32_t* row, int i_begin, int i_end, int len, uint32_t prefix,
                           uint32_t* lh) {
  for (int i0 = i_begin + static_cast<int>(threadIdx.x) * kPerThread; i0 < i_end;
       i0 += NT * kPerThread) {
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

// Ordered compaction of elements [i_begin, i_end): writes the selected
// elements to out positions starting at `offset`, in index order.  eq_before
// is the number of key == T elements before i_begin in the row.
template <int NT>
__device__ void compact_range(const uint32_t* row, int i_begin, int i_end, int len, Threshold th,
                              uint32_t offset, uint32_t eq_before, const int32_t* cand_row,
                              int32_t* idx_row, float* score_row, uint32_t* sm) {
  for (int t0 = i_begin; t0 < i_end; t0 += NT * kPerThread) {
    const int i0 = t0 + static_cast<int>(threadIdx.x) * kPerThread;
    uint32_t v[16];
    if (i0 < i_end) {
      load16(row, i0, len, v);
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = 0u;
    }
    uint32_t n_eq = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) n_eq += (v[j] == th.T) ? 1u : 0u;
    uint32_t eq_tot;
    uint32_t eq_rank = eq_before + block_excl_scan<NT>(n_eq, sm, eq_tot);
    uint32_t sel_mask = 0, n_sel = 0;
    {
      uint32_t r = eq_rank;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const bool gt = v[j] > th.T && v[j] != 0u;
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

// ---------------------------------------------------------------- few rows
__global__ __launch_bounds__(256) void topk_hist_kernel(const uint32_t* __restrict__ u,
                                                        int u_stride, const int32_t* q_pos,
                                                        int fixed_len, uint32_t* hist,
                                                        int topk, int level) {
  __shared__ uint32_t lh[kBins1];
  __shared__ uint32_t sm[4];
  __shared__ uint32_t res[4];
  const int n = blockIdx.y;
  const int len = row_len(q_pos, fixed_len, n);
  const int base = blockIdx.x * kChunk;
  if (base >= len) return;
  uint32_t* h0 = hist + static_cast<size_t>(n) * kHistWords;
  uint32_t* h1 = h0 + kBins0;
  uint32_t* h2 = h1 + kBins1;
  find_digit<256>(h0, kBins0, static_cast<uint32_t>(topk), true, sm, res);
  const uint32_t K = res[2], d0 = res[0], r0 = res[1];
  __syncthreads();
  if (K == 0) return;
  uint32_t prefix = d0;
  const int nb = level == 1 ? kBins1 : kBins2;
  if (level == 2) {
    find_digit<256>(h1, kBins1, r0, false, sm, res);
    prefix = (d0 << kDigit1Bits) | res[0];
  }
  for (int b = threadIdx.x; b < nb; b += 256) lh[b] = 0u;
  __syncthreads();
  const uint32_t* row = u + static_cast<size_t>(n) * u_stride;
  const int end = base + kChunk;
  if (level == 1)
    hist_range<256, 1>(row, base, end, len, prefix, lh);
  else
    hist_range<256, 2>(row, base, end, len, prefix, lh);
  __syncthreads();
  uint32_t* dst = level == 1 ? h1 : h2;
  for (int b = threadIdx.x; b < nb; b += 256) {
    const uint32_t c = lh[b];
    if (c) atomicAdd(&dst[b], c);
  }
}

__global__ __launch_bounds__(256) void topk_count_kernel(const uint32_t* __restrict__ u,
                                                         int u_stride, const int32_t* q_pos,
                                                         int fixed_len, const uint32_t* hist,
                                                         uint32_t* cnt, int nchunks, int topk) {
  __shared__ uint32_t sm[4];
  __shared__ uint32_t res[4];
  const int n = blockIdx.y;
  const int len = row_len(q_pos, fixed_len, n);
  const int base = blockIdx.x * kChunk;
  uint32_t* my = cnt + (static_cast<size_t>(n) * nchunks + blockIdx.x) * 2;
  if (base >= len) {
    if (threadIdx.x == 0) my[0] = my[1] = 0u;
    return;
  }
  const uint32_t* h0 = hist + static_cast<size_t>(n) * kHistWords;
  const Threshold th = derive_threshold<256>(h0, h0 + kBins0, h0 + kBins0 + kBins1,
                                             static_cast<uint32_t>(topk), sm, res);
  const uint32_t* row = u + static_cast<size_t>(n) * u_stride;
  uint32_t gt = 0, eq = 0;
  const int i0 = base + threadIdx.x * kPerThread;
  if (th.K > 0) {
    uint32_t v[16];
    load16(row, i0, len, v);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      gt += (v[j] > th.T && v[j] != 0u) ? 1u : 0u;
      eq += (v[j] == th.T) ? 1u : 0u;
    }
  }
  gt = block_sum<256>(gt, sm);
  eq = block_sum<256>(eq, sm);
  if (threadIdx.x == 0) {
    my[0] = gt;
    my[1] = eq;
  }
}

__global__ __launch_bounds__(256) void topk_write_kernel(
    const uint32_t* __restrict__ u, int u_stride, const int32_t* q_pos, int fixed_len,
    const uint32_t* hist, const uint32_t* cnt, int nchunks, int topk,
    const int32_t* __restrict__ cand, int cand_stride, int32_t* __restrict__ idx,
    float* __restrict__ score) {
  __shared__ uint32_t sm[4];
  __shared__ uint32_t res[4];
  const int n = blockIdx.y;
  const int c = blockIdx.x;
  const int len = row_len(q_pos, fixed_len, n);
  const int base = c * kChunk;
  const uint32_t* h0 = hist + static_cast<size_t>(n) * kHistWords;
  const Threshold th = derive_threshold<256>(h0, h0 + kBins0, h0 + kBins0 + kBins1,
                                             static_cast<uint32_t>(topk), sm, res);
  int32_t* idx_row = idx + static_cast<size_t>(n) * topk;
  float* score_row = score ? score + static_cast<size_t>(n) * topk : nullptr;
  if (c == 0) {
    for (int i = static_cast<int>(th.K) + threadIdx.x; i < topk; i += 256) {
      idx_row[i] = -1;
      if (score_row) score_row[i] = -__builtin_inff();
    }
  }
  if (base >= len || th.K == 0) return;
  uint32_t gt_b = 0, eq_b = 0;
  const uint32_t* my = cnt + static_cast<size_t>(n) * nchunks * 2;
  for (int j = threadIdx.x; j < c; j += 256) {
    gt_b += my[2 * j];
    eq_b += my[2 * j + 1];
  }
  gt_b = block_sum<256>(gt_b, sm);
  eq_b = block_sum<256>(eq_b, sm);
  const uint32_t offset = gt_b + (eq_b < th.K2 ? eq_b : th.K2);
  const uint32_t* row = u + static_cast<size_t>(n) * u_stride;
  const int32_t* cand_row = cand ? cand + static_cast<size_t>(n) * cand_stride : nullptr;
  compact_range<256>(row, base, base + kChunk, len, th, offset, eq_b, cand_row, idx_row,
                     score_row, sm);
}

__global__ void topk_clear_kernel(uint32_t* __restrict__ p, size_t n_words) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n_words;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

// ---------------------------------------------------------------- one row per workgroup
__global__ __launch_bounds__(1024) void topk_row_kernel(
    const uint32_t* __restrict__ u, int u_stride, const int32_t* q_pos, int fixed_len, int topk,
    const int32_t* __restrict__ cand, int cand_stride, int32_t* __restrict__ idx,
    float* __restrict__ score) {
  __shared__ uint32_t h0[kBins0];
  __shared__ uint32_t h1[kBins1];
  __shared__ uint32_t h2[kBins2];
  __shared__ uint32_t sm[16];
  __shared__ uint32_t res[4];
  const int n = blockIdx.x;
  const int len = row_len(q_pos, fixed_len, n);
  const int span = (len + kPerThread - 1) / kPerThread * kPerThread;
  const uint32_t* row = u + static_cast<size_t>(n) * u_stride;
  for (int b = threadIdx.x; b < kBins0; b += 1024) {
    h0[b] = 0u;
    h1[b] = 0u;
  }
  if (threadIdx.x < kBins2) h2[threadIdx.x] = 0u;
  __syncthreads();
  hist_range<1024, 0>(row, 0, span, len, 0u, h0);
  __syncthreads();
  find_digit<1024>(h0, kBins0, static_cast<uint32_t>(topk), true, sm, res);
  const uint32_t K = res[2], d0 = res[0], r0 = res[1];
  __syncthreads();
  Threshold th;
  th.K = K;
  th.T = 0xFFFFFFFFu;
  th.K2 = 0;
  if (K > 0) {
    hist_range<1024, 1>(row, 0, span, len, d0, h1);
    __syncthreads();
    find_digit<1024>(h1, kBins1, r0, false, sm, res);
    const uint32_t d1 = res[0], r1 = res[1];
    __syncthreads();
    hist_range<1024, 2>(row, 0, span, len, (d0 << kDigit1Bits) | d1, h2);
    __syncthreads();
    find_digit<1024>(h2, kBins2, r1, false, sm, res);
    th.T = (d0 << kShift0) | (d1 << kShift1) | res[0];
    th.K2 = res[1];
    __syncthreads();
  }
  int32_t* idx_row = idx + static_cast<size_t>(n) * topk;
  float* score_row = score ? score + static_cast<size_t>(n) * topk : nullptr;
  for (int i = static_cast<int>(K) + threadIdx.x; i < topk; i += 1024) {
    idx_row[i] = -1;
    if (score_row) score_row[i] = -__builtin_inff();
  }
  if (K == 0) return;
  const int32_t* cand_row = cand ? cand + static_cast<size_t>(n) * cand_stride : nullptr;
  compact_range<1024>(row, 0, span, len, th, 0u, 0u, cand_row, idx_row, score_row, sm);
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  if (a.one_row_per_block) {
    MISA_LAUNCH(K_TOPK_ROW, topk_row_kernel, dim3(a.N), dim3(1024), 0, st, a.u, a.u_stride,
                a.q_pos, a.fixed_len, a.topk, a.cand, a.cand_stride, a.idx, a.score);
    return hipGetLastError();
  }
  const int nchunks = a.u_stride / kChunk;
  const dim3 grid(nchunks, a.N);
  MISA_LAUNCH(K_TOPK_HIST1, topk_hist_kernel, grid, dim3(256), 0, st, a.u, a.u_stride, a.q_pos,
              a.fixed_len, a.hist, a.topk, 1);
  MISA_LAUNCH(K_TOPK_HIST2, topk_hist_kernel, grid, dim3(256), 0, st, a.u, a.u_stride, a.q_pos,
              a.fixed_len, a.hist, a.topk, 2);
  MISA_LAUNCH(K_TOPK_COUNT, topk_count_kernel, grid, dim3(256), 0, st, a.u, a.u_stride, a.q_pos,
              a.fixed_len, a.hist, a.cnt, nchunks, a.topk);
  MISA_LAUNCH(K_TOPK_WRITE, topk_write_kernel, grid, dim3(256), 0, st, a.u, a.u_stride, a.q_pos,
              a.fixed_len, a.hist, a.cnt, nchunks, a.topk, a.cand, a.cand_stride, a.idx,
              a.score);
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

}  // namespace misa
