// Block prefilter for routed scoring, gfx950: head routing composed with a
// token-axis hierarchy (the MISA pages call head-axis routing complementary
// to token-axis hierarchies, technical summary "Key contributions"; HISA,
// gonzo_ML TL;DR: a coarse block filter, then token-level refinement that
// keeps the exact top-k output structure).
//
// block_score_kernel: one workgroup per (64 blocks, row).  A block's key is
// the mean of the row's visible keys of that block (the pooled table for
// complete blocks; a partial last block is averaged from the keys), and its
// score is the indexer score under the row's routed heads,
//   I_blk(b) = sum_{j routed} w_j ReLU(q_j . kbar_b).
// The routed query heads and the 64 block keys sit in LDS as fp32; thread t
// takes block t/4 and a quarter of d, the quarters meet with two cross-lane
// adds per head.  Output: order keys of the block scores [N, stride], and
// the row's last block index (the row length for the select).
// expand_blocks_kernel: the tokens of each row's kept blocks (ascending,
// -1 past the row's visible prefix or for unused block slots).
#include "common.hpp"
#include "kernels.hpp"
#include "partial_block.hpp"

namespace misa {
namespace {

constexpr int kBlocksPerWG = 64;

template <int QT, int KT, int D>
__global__ __launch_bounds__(256) void block_score_kernel(BlockScoreArgs a) {
  constexpr int EB = KeyBytes<KT>::value;
  constexpr int PIECES = D * EB / 16;          // 16-byte pieces per key row
  constexpr int EPP = 16 / EB;                 // elements per piece
  constexpr int RG = 256 / PIECES;             // key rows per pass
  constexpr int QD = D / 4;                    // dims per quarter
  __shared__ float kb[kBlocksPerWG][D + 1];
  __shared__ float qh[64][D];
  __shared__ float wh[64];
  __shared__ float psum[RG][D + 1];

  const int n = blockIdx.y, b0 = blockIdx.x * kBlocksPerWG, tid = threadIdx.x;
  const int Ln = a.q_pos[n] + 1;
  const int Mf = Ln / a.B, Mn = (Ln + a.B - 1) / a.B;
  if (blockIdx.x == 0 && tid == 0) a.last_block[n] = Mn - 1;
  if (b0 >= Mn) return;
  const int nb = min(kBlocksPerWG, Mn - b0);
  const int s = a.q_seq[n];
  const int M = (a.L + a.B - 1) / a.B;

  // routed query heads (fp32) and their weights, in batches of 8 elements
  // per thread whose reads are all issued (elements past h * D re-read head
  // h - 1 and are not stored), the head indices first
  constexpr int QB = 8;
  for (int f0 = tid; f0 < a.h * D; f0 += 256 * QB) {
    int head[QB];
#pragma unroll
    for (int k = 0; k < QB; ++k) {
      const int j = (f0 + 256 * k) / D;
      head[k] = a.heads[static_cast<size_t>(n) * a.h + (j < a.h ? j : a.h - 1)];
    }
    float qv[QB], wv[QB];
#pragma unroll
    for (int k = 0; k < QB; ++k) {
      const size_t e = (static_cast<size_t>(n) * a.H_I + head[k]) * D + (f0 + 256 * k) % D;
      qv[k] = QT == DT_F32 ? static_cast<const float*>(a.q)[e]
                           : bf16_lo(static_cast<const uint16_t*>(a.q)[e]);
      wv[k] = a.w[static_cast<size_t>(n) * a.H_I + head[k]];
    }
#pragma unroll
    for (int k = 0; k < QB; ++k) {
      const int f = f0 + 256 * k;
      if (f < a.h * D) {
        qh[f / D][f % D] = qv[k];
        if (f % D == 0) wh[f / D] = wv[k];
      }
    }
  }
  // complete blocks from the pooled table: 16-byte reads, all in flight
  // (blocks past the table's end re-read its last one; only the row's
  // complete blocks are stored)
  {
    constexpr int V4 = kBlocksPerWG * D / 4 / 256;      // float4 reads per thread
    float4 tv[V4];
#pragma unroll
    for (int k = 0; k < V4; ++k) {
      const int f = tid + 256 * k;
      const int i = f / (D / 4), c4 = f % (D / 4);
      const int bb = b0 + i < M ? b0 + i : M - 1;
      tv[k] = *reinterpret_cast<const float4*>(a.kbar + (static_cast<size_t>(s) * M + bb) * D +
                                               4 * c4);
    }
#pragma unroll
    for (int k = 0; k < V4; ++k) {
      const int f = tid + 256 * k;
      const int i = f / (D / 4), c4 = f % (D / 4);
      if (i < nb && b0 + i < Mf) {
        kb[i][4 * c4] = tv[k].x;
        kb[i][4 * c4 + 1] = tv[k].y;
        kb[i][4 * c4 + 2] = tv[k].z;
        kb[i][4 * c4 + 3] = tv[k].w;
      }
    }
  }
  // a partial last block: the mean of the row's visible keys of that block
  const int cp = Ln - Mf * a.B;
  if (cp > 0 && Mf >= b0 && Mf < b0 + nb) {
    const int piece = tid % PIECES, rg = tid / PIECES;
    float acc[EPP];
    piece_sum<KT, D>(a.k, a.k_scale, a.kidx, s, Mf * a.B, Ln, tid, acc);
#pragma unroll
    for (int e = 0; e < EPP; ++e) psum[rg][piece * EPP + e] = acc[e];
    __syncthreads();
    if (tid < D) {
      float m = 0.f;
      for (int r = 0; r < RG; ++r) m += psum[r][tid];
      kb[Mf - b0][tid] = m / static_cast<float>(cp);
    }
  }
  __syncthreads();

  // block t/4, dims [QD * (t%4), +QD): dot with every routed head
  const int bi = tid >> 2, qt = tid & 3;
  float score = 0.f;
  if (bi < nb) {
    for (int j = 0; j < a.h; ++j) {
      float dsum = 0.f;
#pragma unroll 8
      for (int x = 0; x < QD; ++x) dsum = fmaf(qh[j][qt * QD + x], kb[bi][qt * QD + x], dsum);
      dsum += __shfl_xor(dsum, 1, 64);
      dsum += __shfl_xor(dsum, 2, 64);
      score = fmaf(wh[j], relu(dsum), score);
    }
    if (qt == 0) a.ub[static_cast<size_t>(n) * a.ub_stride + b0 + bi] = order_key(score);
  }
}

__global__ __launch_bounds__(256) void expand_blocks_kernel(const int32_t* __restrict__ blocks,
                                                            const int32_t* __restrict__ q_pos,
                                                            int m, int B,
                                                            int32_t* __restrict__ cand) {
  const int n = blockIdx.y;
  const int Ln = q_pos[n] + 1;
  const int total = m * B;
  for (int e = blockIdx.x * 256 + threadIdx.x; e < total; e += gridDim.x * 256) {
    const int b = blocks[static_cast<size_t>(n) * m + e / B];
    const int t = b * B + e % B;
    cand[static_cast<size_t>(n) * total + e] = (b >= 0 && t < Ln) ? t : -1;
  }
}

template <int QT, int KT, int D>
hipError_t launch_t(const BlockScoreArgs& a, hipStream_t st) {
  const int mmax = (a.L + a.B - 1) / a.B;
  const dim3 grid((mmax + kBlocksPerWG - 1) / kBlocksPerWG, a.N);
  MISA_LAUNCH(K_BLOCK_SCORE, (block_score_kernel<QT, KT, D>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const BlockScoreArgs& a, hipStream_t st) {
  if (a.q_dt == DT_F32) return launch_t<DT_F32, DT_F32, D>(a, st);
  if (a.k_dt == DT_BF16) return launch_t<DT_BF16, DT_BF16, D>(a, st);
  return launch_t<DT_BF16, DT_E4M3, D>(a, st);
}

}  // namespace

hipError_t launch_block_scores(const BlockScoreArgs& a, hipStream_t st) {
  return a.d == 64 ? launch_d<64>(a, st) : launch_d<128>(a, st);
}

hipError_t launch_expand_blocks(const int32_t* blocks, const int32_t* q_pos, int N, int m, int B,
                                int32_t* cand, hipStream_t st) {
  const int total = m * B;
  const int gx = (total + 255) / 256 < 64 ? (total + 255) / 256 : 64;
  MISA_LAUNCH(K_EXPAND_BLOCKS, expand_blocks_kernel, dim3(gx, N), dim3(256), 0, st, blocks,
              q_pos, m, B, cand);
  return hipGetLastError();
}

}  // namespace misa
