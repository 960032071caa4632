// Pieces of the head router's selection step, shared by the router's own
// selection kernel and by the decode scoring kernel that routes in its
// prologue (MISA technical summary, gist.science, "Methodology" item 1):
//   r[n,j] = |w[n,j]| * sum_{b < M_n} ReLU(q[n,j,:] . kbar_n[b]),
// with the row's partial last block pooled from its visible keys only.  Both
// callers run these with 256 threads and in the same order, so they route
// bit-identically.
#pragma once

#include "common.hpp"
#include "partial_block.hpp"

namespace misa {

// Head row (D values) of q into registers as fp32.
template <int QT, int D>
__device__ __forceinline__ void load_q_row(const void* q, size_t row, float (&out)[D]) {
  if constexpr (QT == DT_F32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(q) + row * D);
#pragma unroll
    for (int i = 0; i < D / 4; ++i) {
      const float4 x = p[i];
      out[4 * i] = x.x;
      out[4 * i + 1] = x.y;
      out[4 * i + 2] = x.z;
      out[4 * i + 3] = x.w;
    }
  } else if constexpr (QT == DT_BF16) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(q) + row * D);
#pragma unroll
    for (int i = 0; i < D / 8; ++i) unpack16<DT_BF16>(p[i], &out[8 * i]);
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(q) + row * D);
#pragma unroll
    for (int i = 0; i < D / 16; ++i) unpack16<DT_E4M3>(p[i], &out[16 * i]);
  }
}

// Chunk partial sums of one row: thread (g, j) = (tid / 64, tid % 64) sums
// chunks g, g + 4, g + 8, ... of head j in that order into red[g][j].
// load_chunk_partials issues the first pass's NP loads (so a caller can put
// other loads behind them), finish_chunk_partials adds them and runs the
// remaining passes (16 loads in flight each, 4 when NP < 16); the caller synchronises before
// reading red.  The sum does not depend on NP: the masked slots add +0 to a
// sum of non-negative terms.
template <int NP = 16>
__device__ __forceinline__ void load_chunk_partials(const float* __restrict__ partial_row,
                                                    int nchunks, int H_I, float (&v)[NP]) {
  const int j = threadIdx.x & 63, g = threadIdx.x >> 6;
  // every load is issued (clamped to an element of the row; the sum masks
  // them), so the wait for them is an exact count that leaves later loads in
  // flight
  const int jc = j < H_I ? j : H_I - 1;
#pragma unroll
  for (int u = 0; u < NP; ++u) {
    const int c = g + 4 * u;
    v[u] = partial_row[static_cast<size_t>(c < nchunks ? c : nchunks - 1) * H_I + jc];
  }
}

template <int NP = 16>
__device__ __forceinline__ void finish_chunk_partials(const float* __restrict__ partial_row,
                                                      int nchunks, int H_I, const float (&v)[NP],
                                                      float (&red)[4][64]) {
  const int j = threadIdx.x & 63, g = threadIdx.x >> 6;
  float a = 0.f;
#pragma unroll
  for (int u = 0; u < NP; ++u) a += (j < H_I && g + 4 * u < nchunks) ? v[u] : 0.f;
  if (j < H_I) {
    constexpr int RP = NP < 16 ? 4 : 16;   // loads in flight per remaining pass
    const float* pp = partial_row + j;
    for (int c0 = g + 4 * NP; c0 < nchunks; c0 += 4 * RP) {
      float w[RP];
#pragma unroll
      for (int u = 0; u < RP; ++u) {
        const int c = c0 + 4 * u;
        w[u] = c < nchunks ? pp[static_cast<size_t>(c) * H_I] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < RP; ++u) a += w[u];
    }
  }
  red[g][j] = a;
}

__device__ __forceinline__ float combine_partials(const float (&red)[4][64], int j) {
  return (red[0][j] + red[1][j]) + (red[2][j] + red[3][j]);
}

// Mean of the row's visible keys t in [t0, t1) of the partial block (cp of
// them) into mean[0 .. D); every thread calls it (two barriers).
template <int KT, int D>
__device__ __forceinline__ void partial_block_mean(const void* k, const float* k_scale,
                                                   const KeyIndex& ki, int s, int t0, int t1,
                                                   float (&psum)[PieceMap<KT, D>::RG][D + 1],
                                                   float (&mean)[D]) {
  using PM = PieceMap<KT, D>;
  const int piece = threadIdx.x % PM::PIECES, rg = threadIdx.x / PM::PIECES;
  float acc[PM::EPP];
  piece_sum<KT, D>(k, k_scale, ki, s, t0, t1, threadIdx.x, acc);
#pragma unroll
  for (int e = 0; e < PM::EPP; ++e) psum[rg][piece * PM::EPP + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < D) {
    float m = 0.f;
    for (int r = 0; r < PM::RG; ++r) m += psum[r][threadIdx.x];
    mean[threadIdx.x] = m / static_cast<float>(t1 - t0);
  }
  __syncthreads();
}

// A quarter of a head row of q as raw 16-byte pieces: thread (w, j) =
// (tid / 64, tid % 64) holds elements [w * D / 4, (w + 1) * D / 4) of head j
// (clamped to head H_I - 1, so every load is issued and the caller can wait
// for it with an exact count behind later loads).
template <int QT, int D>
struct QQuarter {
  static constexpr int DW = D / 4;
  static constexpr int NV = DW * KeyBytes<QT>::value / 16;
  static_assert(NV * 16 == DW * KeyBytes<QT>::value, "a quarter of d must be whole 16-byte loads");
  uint4 x[NV];
};

template <int QT, int D>
__device__ __forceinline__ void load_q_quarter(const void* q, size_t row0, int H_I,
                                               QQuarter<QT, D>& qq) {
  using QQ = QQuarter<QT, D>;
  const int j = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int jc = j < H_I ? j : H_I - 1;
  const uint4* p = reinterpret_cast<const uint4*>(
      static_cast<const uint8_t*>(q) +
      ((row0 + jc) * D + static_cast<size_t>(w) * QQ::DW) * KeyBytes<QT>::value);
#pragma unroll
  for (int i = 0; i < QQ::NV; ++i) qq.x[i] = p[i];
}

// The partial block's terms ReLU(q[row0 + j] . mean) of heads j < H_I: the 4
// wavefronts each take their quarter of d for every head (ascending fmaf), the
// quarters are added in a fixed order by lane j after the barrier
// (partial_block_term_sum).  Every thread calls it.
template <int QT, int D>
__device__ __forceinline__ void partial_block_terms(const QQuarter<QT, D>& qq, int H_I,
                                                    const float (&mean)[D],
                                                    float (&part)[4][64]) {
  using QQ = QQuarter<QT, D>;
  constexpr int EPV = 16 / KeyBytes<QT>::value;
  const int j = threadIdx.x & 63, w = threadIdx.x >> 6;
  float acc = 0.f;
  if (j < H_I) {
#pragma unroll
    for (int i = 0; i < QQ::NV; ++i) {
      float qv[EPV];
      unpack16<QT>(qq.x[i], qv);
#pragma unroll
      for (int e = 0; e < EPV; ++e) acc = fmaf(qv[e], mean[w * QQ::DW + i * EPV + e], acc);
    }
  }
  part[w][j] = acc;
  __syncthreads();
}

__device__ __forceinline__ float partial_block_term_sum(const float (&part)[4][64], int j) {
  return fmaxf((part[0][j] + part[1][j]) + (part[2][j] + part[3][j]), 0.f);
}

// Wavefront 0 only (lane j = head j, r = its importance >= 0, any value for
// j >= H_I): routes the first h heads under (r desc, head index asc) and
// writes them in ascending order to out[0 .. h).  The h-th largest r is found
// bit by bit with wavefront ballots (r >= 0, so its bits order like the
// value; -0 counts as +0), then the heads equal to it are taken by lowest
// index: the same set as "fewer than h heads beat it".
__device__ __forceinline__ void rank_heads(float r, int H_I, int h, int32_t* out) {
  const int j = threadIdx.x;
  const bool valid = j < H_I;
  const uint32_t key = r == 0.f ? 0u : __float_as_uint(r);
  uint32_t prefix = 0, need = static_cast<uint32_t>(h);
#pragma unroll
  for (int b = 31; b >= 0; --b) {
    const uint32_t hi = b == 31 ? 0u : (0xFFFFFFFFu << (b + 1));
    const bool in = valid && (key & hi) == prefix;
    const uint32_t ones = static_cast<uint32_t>(__popcll(__ballot(in && ((key >> b) & 1u))));
    if (ones >= need)
      prefix |= 1u << b;
    else
      need -= ones;
  }
  // prefix = the h-th largest key; `need` of the keys equal to it are taken
  const uint64_t below = (1ull << j) - 1ull;
  const uint64_t eq = __ballot(valid && key == prefix);
  const bool chosen =
      valid && (key > prefix || (key == prefix && static_cast<uint32_t>(__popcll(eq & below)) < need));
  const uint64_t mask = __ballot(chosen);
  if (chosen) out[__popcll(mask & below)] = j;
}

}  // namespace misa
