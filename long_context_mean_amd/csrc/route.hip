// Block-pooled head router, gfx950.
//
// For query row n the router scores every indexer head j against the pooled
// block keys and keeps the top-h heads (MISA technical summary, gist.science,
// "Methodology" item 1; cost O(H_I M)).  The head importance is
//   r[n,j] = |w[n,j]| * sum_{b < M_n} ReLU(q[n,j,:] . kbar_n[b]),
// the indexer's own ReLU term at block granularity.  Blocks fully visible to
// the row are read from the pooled table; the row's partial last block (when
// L_n is not a multiple of B) is the mean of its visible keys only.
//
// Two kernels:
//  route_partial: grid (chunk of 32 full blocks, row).  The row's query heads
//    (fp32, padded rows) and the chunk's pooled keys sit in LDS; each lane
//    owns one head and walks four blocks at a time, so a q element read from
//    LDS feeds four FMAs.  Partial sums go to the workspace (no float
//    atomics: the final sum is taken in a fixed order and is deterministic).
//  route_select: one workgroup per row.  Sums the chunk partials, adds the
//    partial-block term, applies |w|, and picks the top-h heads with
//    wavefront reductions (ties -> lower head index); heads are written
//    ascending.
#include "common.hpp"
#include "kernels.hpp"

namespace misa {
namespace {

constexpr int kRouteBlocks = 32;     // pooled blocks per route_partial workgroup

template <int QT>
__device__ __forceinline__ float load_q(const void* q, size_t i) {
  if constexpr (QT == DT_F32)
    return static_cast<const float*>(q)[i];
  else
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(q)[i]) << 16);
}

template <int KT>
__device__ __forceinline__ float load_key(const void* k, const float* k_scale, size_t row, int D,
                                          int i) {
  if constexpr (KT == DT_F32) {
    return static_cast<const float*>(k)[row * D + i];
  } else if constexpr (KT == DT_BF16) {
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(k)[row * D + i])
                           << 16);
  } else {
    const uint32_t code = static_cast<const uint8_t*>(k)[row * D + i];
    uint32_t lo, hi;
    e4m3x4_to_bf16x4(code, lo, hi);
    return bf16_lo(lo) * k_scale[row];
  }
}

template <int QT, int D>
__global__ __launch_bounds__(256) void route_partial_kernel(
    const void* __restrict__ q, const float* __restrict__ kbar, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_pos, int L, int B, int H_I, int nchunks,
    float* __restrict__ partial) {
  __shared__ float q_lds[64][D + 1];
  __shared__ float kb_lds[kRouteBlocks][D + 4];
  __shared__ float red[4 * 64];

  const int n = blockIdx.y, chunk = blockIdx.x;
  const int Ln = q_pos[n] + 1;
  const int Mf = Ln / B;                       // blocks fully visible to row n
  const int M = (L + B - 1) / B;               // rows of the pooled table
  const int b0 = chunk * kRouteBlocks;
  const int b1 = (b0 + kRouteBlocks < Mf) ? b0 + kRouteBlocks : Mf;
  float* out = partial + (static_cast<size_t>(n) * nchunks + chunk) * H_I;
  if (b0 >= b1) {
    for (int j = threadIdx.x; j < H_I; j += 256) out[j] = 0.f;
    return;
  }
  const int s = q_seq[n];
  for (int e = threadIdx.x; e < H_I * D; e += 256)
    q_lds[e / D][e % D] = load_q<QT>(q, static_cast<size_t>(n) * H_I * D + e);
  const int nb = b1 - b0;
  for (int e = threadIdx.x; e < nb * D; e += 256)
    kb_lds[e / D][e % D] = kbar[(static_cast<size_t>(s) * M + b0) * D + e];
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = 64 / H_I;                      // lane groups per wave
  const int j = lane % H_I, sub = lane / H_I;
  const bool active = sub < G;
  const int slot = wave * G + sub;             // 0 .. 4G-1
  const int nslots = 4 * G;
  float acc = 0.f;
  if (active) {
    for (int bb = slot * 4; bb < nb; bb += nslots * 4) {
      float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f;
      const int r1 = bb + 1 < nb ? bb + 1 : bb, r2 = bb + 2 < nb ? bb + 2 : bb,
                r3 = bb + 3 < nb ? bb + 3 : bb;
#pragma unroll 8
      for (int i = 0; i < D; ++i) {
        const float qv = q_lds[j][i];
        d0 += qv * kb_lds[bb][i];
        d1 += qv * kb_lds[r1][i];
        d2 += qv * kb_lds[r2][i];
        d3 += qv * kb_lds[r3][i];
      }
      acc += fmaxf(d0, 0.f);
      if (bb + 1 < nb) acc += fmaxf(d1, 0.f);
      if (bb + 2 < nb) acc += fmaxf(d2, 0.f);
      if (bb + 3 < nb) acc += fmaxf(d3, 0.f);
    }
  }
  if (active) red[slot * H_I + j] = acc;          // nslots * H_I <= 256
  __syncthreads();
  for (int jj = threadIdx.x; jj < H_I; jj += 256) {
    float sum = 0.f;
    for (int sl = 0; sl < nslots; ++sl) sum += red[sl * H_I + jj];
    out[jj] = sum;
  }
}

template <int QT, int KT, int D>
__global__ __launch_bounds__(256) void route_select_kernel(
    const void* __restrict__ q, const float* __restrict__ w, const void* __restrict__ k,
    const float* __restrict__ k_scale, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_pos, int L, int B, int H_I, int h, int nchunks,
    const float* __restrict__ partial, int32_t* __restrict__ heads,
    float* __restrict__ head_score) {
  __shared__ float psum[256];
  __shared__ float mean[D];

  const int n = blockIdx.x;
  const int Ln = q_pos[n] + 1;
  const int Mf = Ln / B;
  const int cp = Ln - Mf * B;                 // visible keys of the partial block
  const int s = q_seq[n];

  // partial-block mean over the row's visible keys of that block
  if (cp > 0) {
    constexpr int SUBS = 256 / D;
    const int i = threadIdx.x % D, sub = threadIdx.x / D;
    float acc = 0.f;
    for (int t = Mf * B + sub; t < Ln; t += SUBS)
      acc += load_key<KT>(k, k_scale, static_cast<size_t>(s) * L + t, D, i);
    psum[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x < D) {
      float m = 0.f;
#pragma unroll
      for (int sb = 0; sb < SUBS; ++sb) m += psum[sb * D + threadIdx.x];
      mean[threadIdx.x] = m / static_cast<float>(cp);
    }
    __syncthreads();
  }

  if (threadIdx.x < 64) {
    const int j = threadIdx.x;
    float r = -1.f;
    if (j < H_I) {
      float a = 0.f;
      const float* pp = partial + static_cast<size_t>(n) * nchunks * H_I + j;
      for (int c = 0; c < nchunks; ++c) a += pp[static_cast<size_t>(c) * H_I];
      if (cp > 0) {
        float dt = 0.f;
        const size_t qb = (static_cast<size_t>(n) * H_I + j) * D;
        for (int i = 0; i < D; ++i) dt += load_q<QT>(q, qb + i) * mean[i];
        a += fmaxf(dt, 0.f);
      }
      r = fabsf(w[static_cast<size_t>(n) * H_I + j]) * a;
      if (head_score) head_score[static_cast<size_t>(n) * H_I + j] = r;
    }
    // top-h: h rounds of a wavefront arg-max (ties -> lower head index)
    float v = r;
    bool chosen = false;
    for (int it = 0; it < h; ++it) {
      float bv = v;
      int bj = j;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oj = __shfl_xor(bj, o, 64);
        if (ov > bv || (ov == bv && oj < bj)) {
          bv = ov;
          bj = oj;
        }
      }
      if (bj == j) {
        chosen = true;
        v = -2.f;
      }
    }
    const uint64_t mask = __ballot(chosen);
    if (chosen) {
      const int pos = __popcll(mask & ((1ull << j) - 1ull));
      heads[static_cast<size_t>(n) * h + pos] = j;
    }
  }
}

template <int QT, int KT, int D>
hipError_t launch_route_t(const RouteArgs& a, hipStream_t st) {
  MISA_LAUNCH(K_ROUTE_PARTIAL, (route_partial_kernel<QT, D>), dim3(a.nchunks, a.N), dim3(256),
              0, st, a.q, a.kbar, a.q_seq, a.q_pos, a.L, a.B, a.H_I, a.nchunks, a.partial);
  MISA_LAUNCH(K_ROUTE_SELECT, (route_select_kernel<QT, KT, D>), dim3(a.N), dim3(256), 0, st,
              a.q, a.w, a.k, a.k_scale, a.q_seq, a.q_pos, a.L, a.B, a.H_I, a.h, a.nchunks,
              a.partial, a.heads, a.head_score);
  return hipGetLastError();
}

template <int D>
hipError_t launch_route_d(const RouteArgs& a, hipStream_t st) {
  if (a.q_dt == DT_F32) return launch_route_t<DT_F32, DT_F32, D>(a, st);
  if (a.k_dt == DT_BF16) return launch_route_t<DT_BF16, DT_BF16, D>(a, st);
  return launch_route_t<DT_BF16, DT_E4M3, D>(a, st);
}

}  // namespace

int route_blocks_per_chunk() { return kRouteBlocks; }

hipError_t launch_route(const RouteArgs& a, hipStream_t st) {
  return a.d == 64 ? launch_route_d<64>(a, st) : launch_route_d<128>(a, st);
}

}  // namespace misa
