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
//  route_partial: grid (chunk of 16 full blocks, row).  Lane j of every
//    wavefront holds head j's query row in registers (fp32); the chunk's
//    pooled keys sit in LDS and are read as broadcasts, each wavefront taking
//    every fourth block.  Per-chunk sums go to the workspace (no float
//    atomics: the final sum runs in a fixed order and is deterministic).
//  route_select: one workgroup per row.  Sums the chunk partials, adds the
//    partial-block term, applies |w|, and routes every head that fewer than
//    h heads beat under (r desc, head index asc); heads are written in
//    ascending order.
#include "common.hpp"
#include "kernels.hpp"

namespace misa {
namespace {

constexpr int kRouteBlocks = 16;     // pooled blocks per route_partial workgroup

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
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(q) + row * D);
#pragma unroll
    for (int i = 0; i < D / 8; ++i) unpack16<DT_BF16>(p[i], &out[8 * i]);
  }
}

template <int QT, int D>
__global__ __launch_bounds__(256) void route_partial_kernel(
    const void* __restrict__ q, const float* __restrict__ kbar, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_pos, int L, int B, int H_I, int nchunks,
    float* __restrict__ partial) {
  __shared__ __align__(16) float kb_lds[kRouteBlocks][D];
  __shared__ float red[4][64];

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
  const int nb = b1 - b0;
  // all loads in flight at once: pooled keys of the chunk, then the head row
  constexpr int NF = kRouteBlocks * D / 4 / 256;      // float4 per thread
  const float4* src = reinterpret_cast<const float4*>(kbar + (static_cast<size_t>(s) * M + b0) * D);
  float4 tmp[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int e = threadIdx.x + f * 256;
    tmp[f] = e < nb * D / 4 ? src[e] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float qr[D];
  if (lane < H_I) load_q_row<QT, D>(q, static_cast<size_t>(n) * H_I + lane, qr);
#pragma unroll
  for (int f = 0; f < NF; ++f)
    reinterpret_cast<float4*>(&kb_lds[0][0])[threadIdx.x + f * 256] = tmp[f];
  __syncthreads();

  float acc = 0.f;
  if (lane < H_I) {
    for (int b = wave; b < nb; b += 8) {
      const int b2 = b + 4 < nb ? b + 4 : b;
      float d0 = 0.f, d1 = 0.f;
#pragma unroll
      for (int i = 0; i < D; i += 4) {
        const float4 x = *reinterpret_cast<const float4*>(&kb_lds[b][i]);
        const float4 y = *reinterpret_cast<const float4*>(&kb_lds[b2][i]);
        d0 += qr[i] * x.x + qr[i + 1] * x.y + qr[i + 2] * x.z + qr[i + 3] * x.w;
        d1 += qr[i] * y.x + qr[i + 1] * y.y + qr[i + 2] * y.z + qr[i + 3] * y.w;
      }
      acc += fmaxf(d0, 0.f);
      if (b + 4 < nb) acc += fmaxf(d1, 0.f);
    }
  }
  red[wave][lane] = acc;
  __syncthreads();
  if (threadIdx.x < H_I)
    out[threadIdx.x] = (red[0][threadIdx.x] + red[1][threadIdx.x]) +
                       (red[2][threadIdx.x] + red[3][threadIdx.x]);
}

template <int QT, int KT, int D>
__global__ __launch_bounds__(256) void route_select_kernel(
    const void* __restrict__ q, const float* __restrict__ w, const void* __restrict__ k,
    const float* __restrict__ k_scale, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_pos, int L, int B, int H_I, int h, int nchunks,
    const float* __restrict__ partial, int32_t* __restrict__ heads,
    float* __restrict__ head_score) {
  constexpr int EB = KeyBytes<KT>::value;
  constexpr int PIECES = D * EB / 16;          // 16-byte pieces per key row
  constexpr int EPP = 16 / EB;                 // elements per piece
  constexpr int RG = 256 / PIECES;             // key rows per pass
  __shared__ float psum[RG][D + 1];
  __shared__ float mean[D];
  __shared__ float red[4][64];
  __shared__ float rs[64];

  const int n = blockIdx.x;
  const int Ln = q_pos[n] + 1;
  const int Mf = Ln / B;
  const int cp = Ln - Mf * B;                 // visible keys of the partial block
  const int s = q_seq[n];

  // chunk partial sums: 4 groups of 64 threads, 8 loads in flight per pass,
  // fixed summation order
  {
    const int j = threadIdx.x & 63, g = threadIdx.x >> 6;
    float a = 0.f;
    if (j < H_I) {
      const float* pp = partial + static_cast<size_t>(n) * nchunks * H_I + j;
      for (int c0 = g; c0 < nchunks; c0 += 32) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int c = c0 + 4 * u;
          v[u] = c < nchunks ? pp[static_cast<size_t>(c) * H_I] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) a += v[u];
      }
    }
    red[g][j] = a;
  }
  // partial-block mean over the row's visible keys of that block
  if (cp > 0) {
    const int piece = threadIdx.x % PIECES, rg = threadIdx.x / PIECES;
    float acc[EPP];
#pragma unroll
    for (int e = 0; e < EPP; ++e) acc[e] = 0.f;
    const uint8_t* kb = static_cast<const uint8_t*>(k);
    for (int t = Mf * B + rg; t < Ln; t += RG) {
      const size_t row = static_cast<size_t>(s) * L + t;
      const uint4 x = *reinterpret_cast<const uint4*>(kb + row * (D * EB) + piece * 16);
      float v[EPP];
      unpack16<KT>(x, v);
      const float sc = (KT == DT_E4M3) ? k_scale[row] : 1.f;
#pragma unroll
      for (int e = 0; e < EPP; ++e) acc[e] += (KT == DT_E4M3) ? v[e] * sc : v[e];
    }
#pragma unroll
    for (int e = 0; e < EPP; ++e) psum[rg][piece * EPP + e] = acc[e];
  }
  __syncthreads();
  if (cp > 0 && threadIdx.x < D) {
    float m = 0.f;
    for (int r = 0; r < RG; ++r) m += psum[r][threadIdx.x];
    mean[threadIdx.x] = m / static_cast<float>(cp);
  }
  __syncthreads();

  if (threadIdx.x < 64) {
    const int j = threadIdx.x;
    float r = -1.f;
    if (j < H_I) {
      float a = (red[0][j] + red[1][j]) + (red[2][j] + red[3][j]);
      if (cp > 0) {
        float qr[D];
        load_q_row<QT, D>(q, static_cast<size_t>(n) * H_I + j, qr);
        float dt = 0.f;
#pragma unroll
        for (int i = 0; i < D; ++i) dt += qr[i] * mean[i];
        a += fmaxf(dt, 0.f);
      }
      r = fabsf(w[static_cast<size_t>(n) * H_I + j]) * a;
      if (head_score) head_score[static_cast<size_t>(n) * H_I + j] = r;
    }
    // top-h: a head is routed when fewer than h heads beat it under
    // (r desc, head index asc); the 64 scores sit in LDS for the ranking
    rs[j] = r;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    int rank = 0;
    if (j < H_I) {
      for (int o = 0; o < H_I; ++o) {
        const float ro = rs[o];
        rank += (ro > r || (ro == r && o < j)) ? 1 : 0;
      }
    }
    const bool chosen = j < H_I && rank < h;
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
