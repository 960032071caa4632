// Partial-block key sums for the router and the block prefilter, gfx950.
//
// A query row whose visible prefix ends inside a block pools that block from
// its visible keys only (the mean of keys [t0, t1) of sequence s).  The 256
// threads of a workgroup split each key row into 16-byte pieces: thread
// (rg, piece) sums rows t0 + rg, t0 + rg + RG, ... of its piece, in that order.
// All loads of a batch are issued before any is used, so a 64-key block costs
// one memory round trip instead of one per pass.
#pragma once

#include "common.hpp"

namespace misa {

template <int KT, int D>
struct PieceMap {
  static constexpr int EB = KeyBytes<KT>::value;
  static constexpr int PIECES = D * EB / 16;   // 16-byte pieces per key row
  static constexpr int EPP = 16 / EB;          // elements per piece
  static constexpr int RG = 256 / PIECES;      // key rows per pass
};

// acc[e] = sum over this thread's rows t of element (piece * EPP + e) of key t
// (e4m3 keys times their per-token scale).
template <int KT, int D>
__device__ __forceinline__ void piece_sum(const void* k, const float* k_scale, const KeyIndex& ki,
                                          int s, int t0, int t1, int tid,
                                          float (&acc)[PieceMap<KT, D>::EPP]) {
  using PM = PieceMap<KT, D>;
  // enough loads in flight to cover a 64-key block in one round trip (more
  // would only hold registers; a longer range takes further passes)
  constexpr int BATCH = PM::RG >= 64 ? 1 : (64 / PM::RG > 8 ? 8 : 64 / PM::RG);
  const int piece = tid % PM::PIECES, rg = tid / PM::PIECES;
  const uint8_t* kb = static_cast<const uint8_t*>(k);
#pragma unroll
  for (int e = 0; e < PM::EPP; ++e) acc[e] = 0.f;
  for (int tb = t0 + rg; tb < t1; tb += PM::RG * BATCH) {
    // every load issued (rows past t1 read row t0 and add 0), page numbers
    // first for paged keys, so the batch is one round trip (two paged)
    uint4 x[BATCH];
    float sc[BATCH];
    size_t row[BATCH];
    if (ki.table) {
      int pg[BATCH];
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int t = tb + u * PM::RG;
        pg[u] = ki.page(s, t < t1 ? t : t0);
      }
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int t = tb + u * PM::RG;
        row[u] = ki.row_in_page(pg[u], t < t1 ? t : t0);
      }
    } else {
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int t = tb + u * PM::RG;
        row[u] = static_cast<size_t>(s) * ki.L + (t < t1 ? t : t0);
      }
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      x[u] = *reinterpret_cast<const uint4*>(kb + row[u] * (D * PM::EB) + piece * 16);
      sc[u] = (KT == DT_E4M3) ? k_scale[row[u]] : 1.f;
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      if (tb + u * PM::RG >= t1) {
        x[u] = make_uint4(0u, 0u, 0u, 0u);
        sc[u] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      float v[PM::EPP];
      unpack16<KT>(x[u], v);
#pragma unroll
      for (int e = 0; e < PM::EPP; ++e)   // explicit fma: the same at every call site
        acc[e] = (KT == DT_E4M3) ? fmaf(v[e], sc[u], acc[e]) : acc[e] + v[e];
    }
  }
}

}  // namespace misa
