// Token scoring for the MISA indexer (routed or all-head), gfx950.
//
//   I_n(s) = sum over the row's heads j of w[n,j] * ReLU(q[n,j,:] . key_s)
// (DSA token-wise indexer score; MISA scores only the h routed heads, MISA
// technical summary, gist.science, "Methodology" item 2.)
//
// score_mfma_kernel (bf16 or fp8 keys): one query row against a stream of
// keys.  The row's heads form the A operand of v_mfma_f32_16x16x32_bf16
// (16 head rows per tile, zero-padded), 16 keys form the B operand, so one
// MFMA per 32 elements of d yields 16 heads x 16 keys of dot products in fp32
// from exact bf16 products.  Keys go straight from global memory into the B
// registers: each lane reads d/4 contiguous elements of one key row (a
// wavefront reads 16 whole rows per tile), four tiles in flight per wave.
// fp8 keys are widened to bf16 in registers (exact) and their per-token
// scale is applied to the fp32 dot before the ReLU.  The epilogue applies
// ReLU, multiplies by the head weight and sums the heads (4 rows per lane, 2
// cross-lane adds), then writes a 32-bit order key per token and counts it in
// an LDS histogram of the top 12 key bits (flushed with integer atomics, so
// results do not depend on scheduling).
//
// score_f32_kernel (fp32 keys): one thread per key, plain FMAs (fp32 inputs
// have no exact low-precision MFMA form).
#include "common.hpp"
#include "kernels.hpp"

namespace misa {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

struct ScoreParams {
  const uint16_t* q;
  const float* w;
  const uint8_t* k;
  const float* k_scale;
  const int32_t* q_seq;
  const int32_t* q_pos;
  const int32_t* heads;
  const int32_t* cand;
  int L, H_I, nrows, ncols;
  uint32_t* u;
  int u_stride;
  uint32_t* hist0;
  int tiles_per_wave;
};

template <int KT, int D>
struct KeyLayout {
  static constexpr int EB = KT == DT_E4M3 ? 1 : 2;     // bytes per element
  static constexpr int ROW = D * EB;                   // bytes per key row
  static constexpr int LANE_BYTES = ROW / 4;           // bytes per lane (d/4 elements)
  static constexpr int NLOAD = LANE_BYTES / 16;        // 16-byte loads per lane per tile
  static constexpr int KK = D / 32;                    // MFMAs per head tile
};

// B fragments for one tile: lane (g = lane/16, c = lane%16) holds elements
// [g*d/4, (g+1)*d/4) of key row c, split in KK pieces of 8.
template <int KT, int D>
__device__ __forceinline__ void to_fragments(const u32x4_t (&raw)[KeyLayout<KT, D>::NLOAD],
                                             bf16x8_t (&b)[KeyLayout<KT, D>::KK]) {
  constexpr int KK = KeyLayout<KT, D>::KK;
  if constexpr (KT == DT_BF16) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) b[kk] = __builtin_bit_cast(bf16x8_t, raw[kk]);
  } else {
    // 8 codes (2 words) per piece -> 4 packed bf16 words
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const u32x4_t& r = raw[kk / 2];
      const uint32_t w0 = (kk & 1) ? r.z : r.x;
      const uint32_t w1 = (kk & 1) ? r.w : r.y;
      u32x4_t o;
      uint32_t a0, a1, a2, a3;
      e4m3x4_to_bf16x4(w0, a0, a1);
      e4m3x4_to_bf16x4(w1, a2, a3);
      o.x = a0;
      o.y = a1;
      o.z = a2;
      o.w = a3;
      b[kk] = __builtin_bit_cast(bf16x8_t, o);
    }
  }
}

template <int KT, int NT, int D>
__global__ __launch_bounds__(256) void score_mfma_kernel(ScoreParams p) {
  using LY = KeyLayout<KT, D>;
  constexpr int KK = LY::KK;
  constexpr int NLOAD = LY::NLOAD;
  constexpr int U = 4;                                 // tiles in flight per wave
  __shared__ uint32_t lh[kBins0];

  const int n = blockIdx.y;
  const int len = p.cand ? p.ncols : p.q_pos[n] + 1;
  const int tiles_per_wg = 4 * p.tiles_per_wave;
  const int chunk0 = blockIdx.x * tiles_per_wg * 16;
  if (chunk0 >= len) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const bool do_hist = p.hist0 != nullptr;
  if (do_hist) {
    for (int b = threadIdx.x; b < kBins0; b += 256) lh[b] = 0u;
  }

  // A operand: head rows of this query row; W: weights of this lane's D rows.
  bf16x8_t a[NT][KK];
  float wv[NT][4];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = nt * 16 + c;
    int j = 0;
    const bool rv = r < p.nrows;
    if (rv) j = p.heads ? p.heads[static_cast<size_t>(n) * p.nrows + r] : r;
    const u32x4_t* qp = reinterpret_cast<const u32x4_t*>(
        p.q + (static_cast<size_t>(n) * p.H_I + j) * D + g * (D / 4));
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4_t x = qp[kk];
      if (!rv) x = u32x4_t{0u, 0u, 0u, 0u};
      a[nt][kk] = __builtin_bit_cast(bf16x8_t, x);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = nt * 16 + 4 * g + i;
      float wf = 0.f;
      if (rr < p.nrows) {
        const int jj = p.heads ? p.heads[static_cast<size_t>(n) * p.nrows + rr] : rr;
        wf = p.w[static_cast<size_t>(n) * p.H_I + jj];
      }
      wv[nt][i] = wf;
    }
  }
  const int s = p.q_seq[n];
  const uint8_t* kseq = p.k + static_cast<size_t>(s) * p.L * LY::ROW + g * LY::LANE_BYTES;
  const float* sseq = (KT == DT_E4M3) ? p.k_scale + static_cast<size_t>(s) * p.L : nullptr;
  const int32_t* crow = p.cand ? p.cand + static_cast<size_t>(n) * p.ncols : nullptr;
  uint32_t* urow = p.u + static_cast<size_t>(n) * p.u_stride;
  if (do_hist) __syncthreads();

  const int wave_e0 = chunk0 + wave * p.tiles_per_wave * 16;
  for (int tb = 0; tb < p.tiles_per_wave; tb += U) {
    if (wave_e0 + tb * 16 >= len) break;
    u32x4_t raw[U][NLOAD];
    float sc[U];
    int ev[U];
    bool valid[U];
#pragma unroll
    for (int t = 0; t < U; ++t) {
      const int e = wave_e0 + (tb + t) * 16 + c;
      int tok = -1;
      if (e < len) tok = crow ? crow[e] : e;
      ev[t] = e;
      valid[t] = tok >= 0;
      const int tt = tok >= 0 ? tok : 0;
      const u32x4_t* kp = reinterpret_cast<const u32x4_t*>(kseq + static_cast<size_t>(tt) * LY::ROW);
#pragma unroll
      for (int i = 0; i < NLOAD; ++i) raw[t][i] = kp[i];
      sc[t] = (KT == DT_E4M3) ? sseq[tt] : 1.f;
    }
#pragma unroll
    for (int t = 0; t < U; ++t) {
      bf16x8_t b[KK];
      to_fragments<KT, D>(raw[t], b);
      float part = 0.f;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[nt][kk], b[kk], acc, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = acc[i];
          if (KT == DT_E4M3) v *= sc[t];
          part += wv[nt][i] * fmaxf(v, 0.f);
        }
      }
      part += __shfl_xor(part, 16, 64);
      part += __shfl_xor(part, 32, 64);
      const int e = ev[t];
      if (g == 0 && e < len) {
        const uint32_t key = valid[t] ? order_key(part) : 0u;
        urow[e] = key;
        if (do_hist && valid[t]) atomicAdd(&lh[key >> kShift0], 1u);
      }
    }
  }
  if (do_hist) {
    __syncthreads();
    uint32_t* hg = p.hist0 + static_cast<size_t>(n) * kHistWords;
    for (int b = threadIdx.x; b < kBins0; b += 256) {
      const uint32_t cnt = lh[b];
      if (cnt) atomicAdd(&hg[b], cnt);
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void score_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ w, const float* __restrict__ k,
    const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ heads, const int32_t* __restrict__ cand, int L, int H_I,
    int nrows, int ncols, uint32_t* __restrict__ u, int u_stride, uint32_t* __restrict__ hist0) {
  __shared__ float q_lds[64][D];
  __shared__ float w_lds[64];
  __shared__ uint32_t lh[kBins0];
  const int n = blockIdx.y;
  const int len = cand ? ncols : q_pos[n] + 1;
  const int e0 = blockIdx.x * 256;
  if (e0 >= len) return;
  for (int x = threadIdx.x; x < nrows * D; x += 256) {
    const int r = x / D, i = x % D;
    const int j = heads ? heads[static_cast<size_t>(n) * nrows + r] : r;
    q_lds[r][i] = q[(static_cast<size_t>(n) * H_I + j) * D + i];
  }
  for (int r = threadIdx.x; r < nrows; r += 256) {
    const int j = heads ? heads[static_cast<size_t>(n) * nrows + r] : r;
    w_lds[r] = w[static_cast<size_t>(n) * H_I + j];
  }
  if (hist0)
    for (int b = threadIdx.x; b < kBins0; b += 256) lh[b] = 0u;
  __syncthreads();
  const int e = e0 + threadIdx.x;
  if (e < len) {
    const int tok = cand ? cand[static_cast<size_t>(n) * ncols + e] : e;
    uint32_t key = 0u;
    if (tok >= 0) {
      float kr[D];
      const float4* kp =
          reinterpret_cast<const float4*>(k + (static_cast<size_t>(q_seq[n]) * L + tok) * D);
#pragma unroll
      for (int i = 0; i < D / 4; ++i) {
        const float4 x = kp[i];
        kr[4 * i] = x.x;
        kr[4 * i + 1] = x.y;
        kr[4 * i + 2] = x.z;
        kr[4 * i + 3] = x.w;
      }
      float acc = 0.f;
      for (int r = 0; r < nrows; ++r) {
        float dt = 0.f;
#pragma unroll
        for (int i = 0; i < D; ++i) dt += q_lds[r][i] * kr[i];
        acc += w_lds[r] * fmaxf(dt, 0.f);
      }
      key = order_key(acc);
      if (hist0) atomicAdd(&lh[key >> kShift0], 1u);
    }
    u[static_cast<size_t>(n) * u_stride + e] = key;
  }
  if (hist0) {
    __syncthreads();
    uint32_t* hg = hist0 + static_cast<size_t>(n) * kHistWords;
    for (int b = threadIdx.x; b < kBins0; b += 256) {
      const uint32_t cnt = lh[b];
      if (cnt) atomicAdd(&hg[b], cnt);
    }
  }
}

template <int KT, int NT, int D>
hipError_t launch_mfma(const ScoreArgs& a, hipStream_t st, int tiles_per_wave) {
  ScoreParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.w = a.w;
  p.k = static_cast<const uint8_t*>(a.k);
  p.k_scale = a.k_scale;
  p.q_seq = a.q_seq;
  p.q_pos = a.q_pos;
  p.heads = a.heads;
  p.cand = a.cand;
  p.L = a.L;
  p.H_I = a.H_I;
  p.nrows = a.heads ? a.h : a.H_I;
  p.ncols = a.ncols;
  p.u = a.u;
  p.u_stride = a.u_stride;
  p.hist0 = a.hist0;
  p.tiles_per_wave = tiles_per_wave;
  const int maxlen = a.cand ? a.ncols : a.L;
  const int per_wg = 4 * tiles_per_wave * 16;
  const int nchunks = (maxlen + per_wg - 1) / per_wg;
  MISA_LAUNCH(K_SCORE_MFMA, (score_mfma_kernel<KT, NT, D>), dim3(nchunks, a.N), dim3(256), 0,
              st, p);
  return hipGetLastError();
}

template <int KT, int D>
hipError_t launch_mfma_rows(const ScoreArgs& a, hipStream_t st, int tpw) {
  const int nrows = a.heads ? a.h : a.H_I;
  if (nrows <= 16) return launch_mfma<KT, 1, D>(a, st, tpw);
  if (nrows <= 32) return launch_mfma<KT, 2, D>(a, st, tpw);
  if (nrows <= 48) return launch_mfma<KT, 3, D>(a, st, tpw);
  return launch_mfma<KT, 4, D>(a, st, tpw);
}

}  // namespace

hipError_t launch_score(const ScoreArgs& a, hipStream_t st) {
  if (a.k_dt == DT_F32) {
    const int maxlen = a.cand ? a.ncols : a.L;
    const dim3 grid((maxlen + 255) / 256, a.N);
    const int nrows = a.heads ? a.h : a.H_I;
    if (a.d == 64)
      MISA_LAUNCH(K_SCORE_F32, score_f32_kernel<64>, grid, dim3(256), 0, st,
                  static_cast<const float*>(a.q), a.w, static_cast<const float*>(a.k), a.q_seq,
                  a.q_pos, a.heads, a.cand, a.L, a.H_I, nrows, a.ncols, a.u, a.u_stride,
                  a.hist0);
    else
      MISA_LAUNCH(K_SCORE_F32, score_f32_kernel<128>, grid, dim3(256), 0, st,
                  static_cast<const float*>(a.q), a.w, static_cast<const float*>(a.k), a.q_seq,
                  a.q_pos, a.heads, a.cand, a.L, a.H_I, nrows, a.ncols, a.u, a.u_stride,
                  a.hist0);
    return hipGetLastError();
  }
  // short candidate lists: smaller chunks so more workgroups share the gather
  const int tpw = a.cand ? 4 : 16;
  if (a.k_dt == DT_BF16)
    return a.d == 64 ? launch_mfma_rows<DT_BF16, 64>(a, st, tpw)
                     : launch_mfma_rows<DT_BF16, 128>(a, st, tpw);
  return a.d == 64 ? launch_mfma_rows<DT_E4M3, 64>(a, st, tpw)
                   : launch_mfma_rows<DT_E4M3, 128>(a, st, tpw);
}

}  // namespace misa
