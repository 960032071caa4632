// The mean of one block of index keys, shared by the pooling kernel and by
// the decode router, which pools the blocks a call completes itself so it
// needs no separate pooling launch before it (MISA technical summary,
// gist.science, "Methodology" item 1: blocks summarised by mean-pooled index
// keys).  Both use this one function, so the table entries they produce are
// the same bits.
#pragma once

#include "common.hpp"

namespace misa {

template <int KT, int D>
struct PoolMap {
  static constexpr int EB = KeyBytes<KT>::value;
  static constexpr int ROW_BYTES = D * EB;
  static constexpr int CPR = ROW_BYTES / 16;   // 16-byte pieces per row
  static constexpr int EPC = 16 / EB;          // elements per piece
  static constexpr int RG = 256 / CPR;         // row groups
};

// One batch of a thread's rows: rows t, t + RG, ..., t + (U - 1) RG of its
// piece (rows at or past t1 reread row t; the sum skips them).
template <int KT, int D>
struct PoolBatch {
  static constexpr int U = 8;
  uint4 x[U];
  float sc[U];
};

template <int KT, int D>
__device__ __forceinline__ void pool_batch_load(const uint8_t* __restrict__ k,
                                                const float* __restrict__ k_scale,
                                                const KeyIndex& ki, int s, int t, int t1,
                                                PoolBatch<KT, D>& pb) {
  using PM = PoolMap<KT, D>;
  constexpr int U = PoolBatch<KT, D>::U;
  const int c = threadIdx.x % PM::CPR;
  int tc[U];
#pragma unroll
  for (int r = 0; r < U; ++r) {
    const int tt = t + r * PM::RG;
    tc[r] = tt < t1 ? tt : t;                    // stay in bounds; masked below
  }
  size_t row[U];
  if (ki.table) {
    // paged keys: every row's page number in flight together, then the rows
    int pg[U];
#pragma unroll
    for (int r = 0; r < U; ++r) pg[r] = ki.page(s, tc[r]);
#pragma unroll
    for (int r = 0; r < U; ++r) row[r] = ki.row_in_page(pg[r], tc[r]);
  } else {
#pragma unroll
    for (int r = 0; r < U; ++r) row[r] = static_cast<size_t>(s) * ki.L + tc[r];
  }
#pragma unroll
  for (int r = 0; r < U; ++r) {
    pb.x[r] = *reinterpret_cast<const uint4*>(k + row[r] * PM::ROW_BYTES + c * 16);
    pb.sc[r] = 1.f;
    if constexpr (KT == DT_E4M3) pb.sc[r] = k_scale[row[r]];
  }
}

template <int KT, int D>
__device__ __forceinline__ void pool_batch_add(const PoolBatch<KT, D>& pb, int t, int t1,
                                               float (&acc)[PoolMap<KT, D>::EPC]) {
  using PM = PoolMap<KT, D>;
#pragma unroll
  for (int r = 0; r < PoolBatch<KT, D>::U; ++r) {
    if (t + r * PM::RG < t1) {
      float v[PM::EPC];
      unpack16<KT>(pb.x[r], v);
#pragma unroll
      for (int e = 0; e < PM::EPC; ++e) {
        // an explicit fma: the compiler may not contract a separate multiply
        // and add differently at different call sites
        if constexpr (KT == DT_E4M3)
          acc[e] = fmaf(v[e], pb.sc[r], acc[e]);
        else
          acc[e] += v[e];
      }
    }
  }
}

// The row groups' sums added in order through `part`; thread i < D returns
// the mean of element i (other threads 0).  Ends with the threads < D still
// reading `part`, so a caller reusing `part` synchronises first.
template <int KT, int D>
__device__ __forceinline__ float pool_reduce(const float (&acc)[PoolMap<KT, D>::EPC], int t0,
                                             int t1, float (&part)[PoolMap<KT, D>::RG][D + 1]) {
  using PM = PoolMap<KT, D>;
  const int c = threadIdx.x % PM::CPR, g = threadIdx.x / PM::CPR;
#pragma unroll
  for (int e = 0; e < PM::EPC; ++e) part[g][c * PM::EPC + e] = acc[e];
  __syncthreads();
  float sum = 0.f;
  if (threadIdx.x < D) {
#pragma unroll 8
    for (int r = 0; r < PM::RG; ++r) sum += part[r][threadIdx.x];
    sum /= static_cast<float>(t1 - t0);
  }
  return sum;
}

// Mean of key rows [t0, t1) of sequence s with 256 threads: thread
// (g, c) = (tid / CPR, tid % CPR) sums rows t0 + g, t0 + g + RG, ... of its
// 16-byte piece c (e4m3 codes times the row's scale) in batches of U rows,
// then pool_reduce.  Every thread calls it.
template <int KT, int D>
__device__ __forceinline__ float pool_block_mean(const uint8_t* __restrict__ k,
                                                 const float* __restrict__ k_scale,
                                                 const KeyIndex& ki, int s, int t0, int t1,
                                                 float (&part)[PoolMap<KT, D>::RG][D + 1]) {
  using PM = PoolMap<KT, D>;
  const int g = threadIdx.x / PM::CPR;
  float acc[PM::EPC];
#pragma unroll
  for (int e = 0; e < PM::EPC; ++e) acc[e] = 0.f;
  for (int t = t0 + g; t < t1; t += PoolBatch<KT, D>::U * PM::RG) {
    PoolBatch<KT, D> pb;
    pool_batch_load<KT, D>(k, k_scale, ki, s, t, t1, pb);
    pool_batch_add<KT, D>(pb, t, t1, acc);
  }
  return pool_reduce<KT, D>(acc, t0, t1, part);
}

}  // namespace misa
