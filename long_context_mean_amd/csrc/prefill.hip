// Prefill scoring for the MISA indexer: many query rows over one causal key
// sequence, gfx950.
//
//   I_t(s) = sum over row t's heads j of w[t,j] * ReLU(q[t,j,:] . k_s),  s <= pos_t
// (DSA token-wise indexer score; MISA scores only the h routed heads of each
// row, MISA technical summary, gist.science, "Methodology" item 2.)
//
// In prefill the rows share the keys, so the work is a GEMM: the gathered
// routed head rows of a block of query rows, [rows x HP, d] with HP = the
// head count rounded up to a power of two (padding rows have zero weight),
// times the key matrix [d, L].  One workgroup (4 wavefronts) owns 256 such
// head rows (256 / HP query rows) and one slice of the key range; each
// wavefront keeps its 4 row tiles of v_mfma_f32_16x16x32_bf16 A operands in
// registers for the whole slice.  Key tiles of 64 keys stream into a
// three-stage LDS ring by direct-to-LDS buffer loads (buffer_load ... lds,
// 16 bytes per lane, no VGPR round trip); each lane's source offset is
// XOR-swizzled so the B-fragment reads of a tile are free of bank conflicts,
// an explicit vmcnt wait and one barrier hand a stage to the MFMAs, and each
// B fragment read from LDS feeds 4 MFMAs.  The epilogue applies
// ReLU, multiplies by the head weight, sums the HP rows of each query row
// (in-lane, then across lane groups) and writes the order key of every
// causally visible (row, key) pair; tiles away from the causal diagonal store
// without masks.
//
// fp8 variant (e4m3 queries and keys, d = 128): each 128-byte key row is one
// K = 128 step of v_mfma_f32_16x16x128_f8f6f4, so a row tile needs a single
// MFMA per 16 keys.  Scales are positive, so w * ReLU(sq * sk * x) =
// sk * (w * sq) * ReLU(x): the query head scale sq is folded into the head
// weight when the weights are loaded, and the key scale sk multiplies each
// key's head sum.  The key scales of a tile travel with it: every wavefront
// DMAs the tile's 64 scales into its own LDS slot.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace misa {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr int kRowsPerWG = 256;       // gathered head rows per workgroup
constexpr int kKeyTile = 64;          // keys per LDS tile

struct PrefillParams {
  const uint8_t* q;          // [N, H_I, D] bf16 or e4m3
  const float* w;
  const float* q_scale;      // e4m3 only: [N, H_I]
  const uint8_t* k;          // one key sequence [L, D] bf16 or e4m3
  const float* k_scale;      // e4m3 only: [L]
  const int32_t* q_pos;
  const int32_t* heads;      // [N, h] or NULL (all heads)
  int N, L, H_I, h;
  int keys_per_split;        // multiple of kKeyTile
  uint32_t* u;
  int u_stride;
  int key_step, pos_shift;   // scored keys are key_step * s (sample pass: s <= pos >> pos_shift)
  const uint32_t* block_flag;
  const float* tau;          // candidate mode: threshold score per row
  uint32_t* cnt_out;
  uint2* cand_out;
  int cap, splits;
  uint32_t k_bytes;          // bytes of the key sequence (below 4 GiB)
};

template <int D, bool F8>
struct PLayout {
  static constexpr int ROW = F8 ? D : D * 2;           // bytes per key row
  static constexpr int CH = ROW / 16;                  // 16-byte chunks per row
  static constexpr int TILE = kKeyTile * ROW;          // bytes per LDS key tile
  static constexpr int KK = F8 ? D / 128 : D / 32;     // MFMAs per 16x16 output tile
  static constexpr int ROW_LOADS = kKeyTile * CH / 256;  // 16-byte key loads per thread per tile
  static constexpr int PER_THREAD = ROW_LOADS + (F8 ? 1 : 0);  // + the key-scale load
  // Chunk q of row r sits at chunk position q ^ swz(r): the 16 rows read by
  // one MFMA B fragment then hit 16 different 16-byte bank groups.  With
  // 128-byte rows, rows r and r + 1 already differ in the upper half of a
  // 256-byte bank window, so r & 7 spreads 8 consecutive rows and the
  // r >> 3 term separates rows r and r + 8.
  __device__ static int swz(int r) { return CH == 16 ? (r & 15) : ((r ^ (r >> 3)) & 7); }
  // A / B fragment: 8 bf16 (16 bytes) or 32 e4m3 codes (32 bytes) per lane
  using Frag = std::conditional_t<F8, i32x8_t, bf16x8_t>;
};

constexpr int kStages = 3;                             // LDS key tiles in flight

// Key rows key_step * s for s in [key0, key0 + 64) straight into an LDS tile
// (global_load_lds_dwordx4: each wavefront instruction fills 1 KB of the
// tile, lane l the l-th 16 bytes).  s >= L (in the same units) reads row 0
// instead (masked later).  Completion is tracked by vmcnt.
//
// A lane's source offsets from the tile's first key row are the same for
// every tile, so they are formed once (DmaLane); a tile whose 64 keys are all
// below L is read with buffer loads whose per-tile part is one scalar offset,
// so it costs no per-lane address work.  The key sequence is below 4 GiB (the
// launcher checks), so every offset fits the 32-bit buffer offsets.
template <int D, bool F8>
struct DmaLane {
  // With 16 chunks per row, load j's rows are 16 j rows past load 0's and the
  // swizzle (row & 15) is the same, so one lane offset serves every load and
  // load j adds a scalar 16 j rows; otherwise each load keeps its own.
  static constexpr bool ONE = PLayout<D, F8>::CH == 16;
  static constexpr int NOFF = ONE ? 1 : PLayout<D, F8>::ROW_LOADS;
  uint32_t off[NOFF];                        // byte offset of the lane's chunk
  uint32_t soff;                             // fp8: byte offset of the lane's key scale
  uint32_t k_bytes;                          // bytes of the key sequence
  __device__ void init(uint32_t key_bytes, int key_step, int wave, int lane) {
    using LY = PLayout<D, F8>;
#pragma unroll
    for (int j = 0; j < NOFF; ++j) {
      const int f = (j * 4 + wave) * 64 + lane;
      const int r = f / LY::CH;
      off[j] = static_cast<uint32_t>(r * key_step * LY::ROW + 16 * ((f % LY::CH) ^ LY::swz(r)));
    }
    soff = static_cast<uint32_t>(lane * key_step * 4);
    k_bytes = key_bytes;
  }
};

// buffer_load_dword{,x4} ... lds: `bytes` per lane from rsrc at voff + soff
// into LDS at lds + 4 or 16 * lane
typedef __attribute__((address_space(3))) void* lds_void_ptr;
__device__ __forceinline__ void buffer_to_lds16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff,
                                                uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_ptr)(lds), 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void buffer_to_lds4(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff,
                                               uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_ptr)(lds), 4, voff, soff, 0, 0);
}

template <int D, bool F8>
__device__ __forceinline__ void dma_key_tile(const uint8_t* k, const float* k_scale, int key0,
                                             int L, int key_step, uint8_t* tile, float* scales,
                                             const DmaLane<D, F8>& dl, int wave, int lane) {
  using LY = PLayout<D, F8>;
  // buffer resources over the keys and their scales (uniform; formed in
  // scalar registers)
  const __amdgpu_buffer_rsrc_t keys = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(k), 0,
                                                      static_cast<int>(dl.k_bytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t kscl = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(k_scale), 0, static_cast<int>(dl.k_bytes / LY::ROW * 4u), 0x00020000);
  if (key0 + kKeyTile <= L) {
    const uint32_t row0 = static_cast<uint32_t>(key0) * static_cast<uint32_t>(key_step);
    if constexpr (F8)
      buffer_to_lds4(kscl, scales, dl.soff, row0 * 4u);
#pragma unroll
    for (int j = 0; j < LY::ROW_LOADS; ++j) {
      using DL = DmaLane<D, F8>;
      const uint32_t so = (row0 + (DL::ONE ? 16u * j * key_step : 0u)) * LY::ROW;
      buffer_to_lds16(keys, tile + (j * 4 + wave) * 1024, dl.off[DL::ONE ? 0 : j], so);
    }
    return;
  }
  if constexpr (F8) {
    // this wavefront's copy of the tile's 64 key scales (lane l -> key key0 + l)
    const int key = key0 + lane < L ? key0 + lane : 0;
    buffer_to_lds4(kscl, scales, static_cast<uint32_t>(key * key_step) * 4u, 0u);
  }
#pragma unroll
  for (int j = 0; j < LY::ROW_LOADS; ++j) {
    const int blk = j * 4 + wave;                       // 1 KB block of the tile
    const int f = blk * 64 + lane;                      // 16-byte chunk slot in the tile
    const int r = f / LY::CH;
    int key = key0 + r;
    key = key < L ? key : 0;
    const uint32_t off = static_cast<uint32_t>(key * key_step) * LY::ROW +
                         16u * ((f % LY::CH) ^ LY::swz(r));
    buffer_to_lds16(keys, tile + blk * 1024, off, 0u);
  }
}

// Wait until at most N vector memory operations of this wavefront are
// outstanding (loads complete in order), then a workgroup barrier.  No
// memory fence: the key tiles in flight stay in flight.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 16, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);              // expcnt, lgkmcnt: no wait
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Row mapping of the gathered A operand.  Each wavefront holds 4 row tiles of
// 16 MFMA rows; output lane (g, c) of v_mfma_f32_16x16x32_bf16 holds rows
// 4g..4g+3 of column c.
//  HP <= 16: a query row owns rows 4g..4g+3 of TQ = HP/4 consecutive row
//    tiles, so a lane sums whole query rows in registers; lane group g holds
//    query rows p*4 + g (p < NG).
//  HP >= 32: a query row owns TQ = HP/16 whole row tiles; each lane sums its
//    part and the 4 lane groups are combined with two cross-lane adds.
template <int HP>
struct RowMap {
  static constexpr bool IN_LANE = HP <= 16;
  static constexpr int TQ = IN_LANE ? HP / 4 : HP / 16;  // row tiles per query-row group
  static constexpr int NG = 4 / TQ;                      // query-row groups per wavefront
  static constexpr int QW = IN_LANE ? 4 * NG : NG;       // query rows per wavefront
  // query row (in the workgroup) and head slot of MFMA row m of row tile rt
  __device__ static void row(int wave, int rt, int m, int& qr, int& hs) {
    if constexpr (IN_LANE) {
      qr = wave * QW + (rt / TQ) * 4 + (m >> 2);
      hs = (rt % TQ) * 4 + (m & 3);
    } else {
      qr = wave * QW + rt / TQ;
      hs = (rt % TQ) * 16 + m;
    }
  }
  // query row whose sums lane group g holds for group p
  __device__ static int out_row(int wave, int p, int g) {
    return IN_LANE ? wave * QW + p * 4 + g : wave * QW + p;
  }
};

// Per-lane output state of the epilogue, one entry per query-row group.
template <int HP, bool CAND>
struct OutState {
  static constexpr int NG = RowMap<HP>::NG;
  int pos[NG];             // key s is visible iff s <= pos (-1: no row)
  uint32_t* urow;          // plain mode: order-key row of group 0 (group q: + q * step)
  size_t step;             // plain mode: elements from one group's row to the next
  // candidate mode: the workgroup's (score, token) lists of this split as a
  // buffer resource; a store at an offset past its end is dropped by the
  // hardware, which is how lanes without a candidate skip theirs
  __amdgpu_buffer_rsrc_t lists;
  uint32_t lbase[NG];      // byte offset of group q's list in `lists`
  uint32_t lt;             // lanes of the lane group below this one
  float tau[NG];           // candidate mode: threshold score
  uint32_t cnt[NG];        // candidate mode: scores >= tau so far (uniform over the lane group)
};

constexpr uint32_t kDropOffset = 0x80000000u;   // past every candidate resource's end

// One LDS key tile (64 keys) against the wavefront's 4 row tiles.  MASK: some
// (row, key) of the tile may be outside the causal prefix or the row block.
// B fragment kk of key row r (lane group g): bf16 K-chunk 4kk+g, or e4m3
// bytes 32g .. 32g+31 (chunks 2g, 2g+1).  A fragments use the same K order.
template <int D, bool F8>
__device__ __forceinline__ typename PLayout<D, F8>::Frag load_b(const uint8_t* tile, int r, int kk,
                                                                int g) {
  using LY = PLayout<D, F8>;
  const uint8_t* row = tile + r * LY::ROW;
  if constexpr (F8) {
    const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(row + 16 * ((2 * g) ^ LY::swz(r)));
    const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(row + 16 * ((2 * g + 1) ^ LY::swz(r)));
    return i32x8_t{static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z),
                   static_cast<int>(lo.w), static_cast<int>(hi.x), static_cast<int>(hi.y),
                   static_cast<int>(hi.z), static_cast<int>(hi.w)};
  } else {
    return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(
                                            row + 16 * ((4 * kk + g) ^ LY::swz(r))));
  }
}

template <bool F8, typename Frag>
__device__ __forceinline__ f32x4_t mfma_step(const Frag& a, const Frag& b, f32x4_t acc) {
  if constexpr (F8)   // e4m3 x e4m3 (format codes 0, 0), no block scales
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 0, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

template <int HP, int D, bool F8, bool MASK, bool CAND>
__device__ __forceinline__ void score_tile(const uint8_t* tile, const float* scales, int key0,
                                           const typename PLayout<D, F8>::Frag (&a)[4][PLayout<D, F8>::KK],
                                           const float (&wv)[4][4], OutState<HP, CAND>& o,
                                           int cap, int g, int c) {
  using LY = PLayout<D, F8>;
  using RM = RowMap<HP>;
  constexpr int KK = LY::KK;
#pragma unroll
  for (int ct = 0; ct < kKeyTile / 16; ++ct) {
    typename LY::Frag b[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) b[kk] = load_b<D, F8>(tile, ct * 16 + c, kk, g);
    float v[RM::NG];
#pragma unroll
    for (int q = 0; q < RM::NG; ++q) v[q] = 0.f;
    // the 4 row tiles' chains interleaved (consecutive MFMAs independent),
    // issued at raised wave priority: a wavefront with MFMAs ready goes ahead
    // of the others' epilogues, which fill the vector pipe meanwhile
    f32x4_t acc[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) acc[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) acc[rt] = mfma_step<F8>(a[rt][kk], b[kk], acc[rt]);
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        v[rt / RM::TQ] = fmaf(wv[rt][i], relu(acc[rt][i]), v[rt / RM::TQ]);
    const int key = key0 + ct * 16 + c;
    float ks = 1.f;
    if constexpr (F8) ks = scales[ct * 16 + c];
#pragma unroll
    for (int q = 0; q < RM::NG; ++q) {
      float x = v[q];
      if constexpr (!RM::IN_LANE) {
        x += __shfl_xor(x, 16, 64);
        x += __shfl_xor(x, 32, 64);
      }
      if constexpr (F8) x *= ks;
      const bool owner = RM::IN_LANE || g == 0;
      const bool vis = owner && (!MASK || key <= o.pos[q]);
      if constexpr (!CAND) {
        if (vis) o.urow[q * o.step + key] = order_key(x);
      } else {
        // score compare (same order as the keys: -0 == +0, no NaN scores);
        // the list keeps the score bits, the select turns them into keys
        const bool pass = vis && x >= o.tau[q];
        const uint64_t m = __ballot(pass);
        // slots in key order within the lane group (16 keys of one query row)
        const uint32_t grp = static_cast<uint32_t>(m >> (16 * g)) & 0xFFFFu;
        const uint32_t slot = o.cnt[q] + __popc(grp & o.lt);
        const uint32_t off =
            pass && slot < static_cast<uint32_t>(cap) ? o.lbase[q] + slot * 8u : kDropOffset;
        const u32x2_t e = {__float_as_uint(x), static_cast<uint32_t>(key)};
        __builtin_amdgcn_raw_buffer_store_b64(e, o.lists, off, 0, 0);
        o.cnt[q] += __popc(grp);
      }
    }
  }
}

template <int HP, int D, bool F8, bool CAND>
__global__ __launch_bounds__(256, HP == 4 ? 2 : 3) void score_prefill_kernel(PrefillParams p) {
  using LY = PLayout<D, F8>;
  using RM = RowMap<HP>;
  constexpr int KK = LY::KK;
  constexpr int QB = kRowsPerWG / HP;                  // query rows per workgroup
  __shared__ __align__(16) uint8_t tiles[kStages][LY::TILE];
  __shared__ float kscales[kStages][F8 ? 4 : 1][F8 ? kKeyTile : 1];   // per wavefront copies
  __shared__ int pos_lds[QB];

  if (p.block_flag && p.block_flag[blockIdx.y] == 0u) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int qrow0 = blockIdx.y * QB;
  for (int i = tid; i < QB; i += 256) {
    const int t = qrow0 + i;
    pos_lds[i] = t < p.N ? (p.q_pos[t] >> p.pos_shift) : -1;
  }
  __syncthreads();
  int kmax = 0;                                         // keys [0, kmax) are visible to some row
  for (int i = 0; i < QB; ++i) kmax = max(kmax, pos_lds[i] + 1);
  const int ks0 = blockIdx.x * p.keys_per_split;
  const int ks1 = min(ks0 + p.keys_per_split, kmax);
  if (ks0 >= ks1) {
    if constexpr (CAND) {
      for (int i = tid; i < QB; i += 256)
        if (qrow0 + i < p.N)
          p.cnt_out[static_cast<size_t>(qrow0 + i) * p.splits + blockIdx.x] = 0u;
    }
    return;
  }

  // A operand (4 row tiles of this wavefront) and the weights of the lane's
  // rows.  Every read is issued unconditionally (rows past N or past h read
  // row N - 1 / head slot h - 1 and are zeroed), the head indices first, so
  // the setup is two round trips rather than one per guarded read.
  typename LY::Frag a[4][KK];
  float wv[4][4];
  int ja[4], jw[4][4];
  bool va[4], vw[4][4];
  size_t ta[4], tw[4][4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    int qr, hs;
    RM::row(wave, rt, c, qr, hs);                       // row c of the tile: this lane's A data
    const int t = qrow0 + qr;
    va[rt] = t < p.N && hs < p.h;
    ta[rt] = static_cast<size_t>(t < p.N ? t : p.N - 1);
    const int hc = hs < p.h ? hs : p.h - 1;
    ja[rt] = p.heads ? p.heads[ta[rt] * p.h + hc] : hc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int qo, ho;
      RM::row(wave, rt, 4 * g + i, qo, ho);             // output rows of this lane's results
      const int tt = qrow0 + qo;
      vw[rt][i] = tt < p.N && ho < p.h;
      tw[rt][i] = static_cast<size_t>(tt < p.N ? tt : p.N - 1);
      const int hoc = ho < p.h ? ho : p.h - 1;
      jw[rt][i] = p.heads ? p.heads[tw[rt][i] * p.h + hoc] : hoc;
    }
  }
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const uint8_t* qrp = p.q + (ta[rt] * p.H_I + ja[rt]) * LY::ROW;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      if constexpr (F8) {
        i32x8_t x = *reinterpret_cast<const i32x8_t*>(qrp + 32 * g);
        if (!va[rt]) x = i32x8_t{0, 0, 0, 0, 0, 0, 0, 0};
        a[rt][kk] = x;
      } else {
        u32x4_t x = *reinterpret_cast<const u32x4_t*>(qrp + 64 * kk + 16 * g);
        if (!va[rt]) x = u32x4_t{0u, 0u, 0u, 0u};
        a[rt][kk] = __builtin_bit_cast(bf16x8_t, x);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const size_t wi = tw[rt][i] * p.H_I + jw[rt][i];
      float wf = p.w[wi];
      if constexpr (F8) wf *= p.q_scale[wi];
      wv[rt][i] = vw[rt][i] ? wf : 0.f;
    }
  }
  OutState<HP, CAND> o;
  // group q's row is group 0's row + q * rstep (rows past N are never written)
  constexpr int rstep = RM::IN_LANE ? 4 : 1;
  if constexpr (CAND) {
    // lists of rows qrow0 .. qrow0 + nrow - 1 for this split: row r's list
    // starts r * splits * cap entries after row 0's
    const int nrow = min(QB, p.N - qrow0);
    const uint32_t row_bytes = static_cast<uint32_t>(p.splits) * p.cap * 8u;
    o.lists = __builtin_amdgcn_make_buffer_rsrc(
        p.cand_out + (static_cast<size_t>(qrow0) * p.splits + blockIdx.x) * p.cap, 0,
        static_cast<int>((nrow - 1) * row_bytes + static_cast<uint32_t>(p.cap) * 8u), 0x00020000);
#pragma unroll
    for (int q = 0; q < RM::NG; ++q)
      o.lbase[q] = static_cast<uint32_t>(RM::out_row(wave, q, g)) * row_bytes;
    o.lt = (1u << c) - 1u;
  } else {
    const size_t t0 = static_cast<size_t>(qrow0 + RM::out_row(wave, 0, g));
    o.urow = p.u + t0 * p.u_stride;
    o.step = static_cast<size_t>(rstep) * p.u_stride;
  }
#pragma unroll
  for (int q = 0; q < RM::NG; ++q) {
    const int qr = RM::out_row(wave, q, g);
    o.pos[q] = pos_lds[qr];
    const int t = qrow0 + qr;
    if constexpr (CAND) {
      o.tau[q] = t < p.N ? p.tau[t] : __builtin_inff();
      o.cnt[q] = 0u;
    }
  }
  int minpos = 0x7FFFFFFF;                              // keys <= minpos are visible to every row
  for (int i = 0; i < QB; ++i) minpos = min(minpos, pos_lds[i] < 0 ? 0x7FFFFFFF : pos_lds[i]);
  const bool full_block = qrow0 + QB <= p.N;

  // kStages-stage ring: tiles i+1 .. i+kStages-1 stream into LDS while tile i
  // is scored; before each barrier a wavefront waits only for the tile the
  // next iteration reads (its DMA loads complete in order)
  constexpr int S = kStages;
  constexpr int AHEAD = (S - 2) * LY::PER_THREAD;      // loads still in flight after a wait
  const int ntiles = (ks1 - ks0 + kKeyTile - 1) / kKeyTile;
  DmaLane<D, F8> dl;
  dl.init(p.k_bytes, p.key_step, wave, lane);
#pragma unroll
  for (int j = 0; j < S - 1; ++j)
    if (j < ntiles)
      dma_key_tile<D, F8>(p.k, p.k_scale, ks0 + j * kKeyTile, p.L, p.key_step, tiles[j],
                          kscales[j][F8 ? wave : 0], dl, wave, lane);
  if (ntiles >= S - 1)
    wait_vm_barrier<AHEAD>();
  else
    wait_vm_barrier<0>();
  int buf = 0;
  for (int i = 0; i < ntiles; ++i) {
    const int key0 = ks0 + i * kKeyTile;
    // every (row, key) of the tile is visible: no masks
    const bool unmasked = full_block && key0 + kKeyTile - 1 <= minpos;
    const float* sc = kscales[buf][F8 ? wave : 0];
    if (unmasked)
      score_tile<HP, D, F8, false, CAND>(tiles[buf], sc, key0, a, wv, o, p.cap, g, c);
    else
      score_tile<HP, D, F8, true, CAND>(tiles[buf], sc, key0, a, wv, o, p.cap, g, c);
    const int nb = buf == 0 ? S - 1 : buf - 1;          // the buffer tile i-1 was read from
    if (i + S - 1 < ntiles) {
      dma_key_tile<D, F8>(p.k, p.k_scale, key0 + (S - 1) * kKeyTile, p.L, p.key_step, tiles[nb],
                          kscales[nb][F8 ? wave : 0], dl, wave, lane);
      wait_vm_barrier<AHEAD>();                         // tile i+1 has landed
    } else {
      wait_vm_barrier<0>();
    }
    buf = buf == S - 1 ? 0 : buf + 1;
  }
  if constexpr (CAND) {
#pragma unroll
    for (int q = 0; q < RM::NG; ++q) {
      const int t = qrow0 + RM::out_row(wave, q, g);
      if (c == 0 && (RM::IN_LANE || g == 0) && t < p.N)
        p.cnt_out[static_cast<size_t>(t) * p.splits + blockIdx.x] = o.cnt[q];
    }
  }
}

int hp_of(int h) {
  return h <= 4 ? 4 : h <= 8 ? 8 : h <= 16 ? 16 : h <= 32 ? 32 : 64;
}

// Workgroups of one kernel instantiation resident on the whole chip at once.
template <int HP, int D, bool F8, bool CAND>
int chip_slots() {
  static const int slots = [] {
    int dev = 0, cus = 0, per = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, score_prefill_kernel<HP, D, F8, CAND>, 256,
                                                      0) != hipSuccess ||
        cus < 1 || per < 1)
      return 1024;
    return cus * per;
  }();
  return slots;
}

int gcd(int a, int b) {
  while (b) {
    const int t = a % b;
    a = b;
    b = t;
  }
  return a;
}

// Key-range splits: about 4 rounds of chip-resident workgroups (the last
// round partly idle costs at most a quarter), rounded to whole rounds when
// the row-block count allows; at least min_tiles key tiles per split, at most
// 256 splits.
int choose_splits(int qblocks, int L, int slots, int min_tiles) {
  const int max_s = max(1, min(256, L / (min_tiles * kKeyTile)));
  int s = (4 * slots + qblocks - 1) / qblocks;
  const int m = slots / gcd(slots, qblocks);            // splits per whole round
  if (m <= max_s) s = (s + m - 1) / m * m;
  return max(1, min(s, max_s));
}

// min_tiles: key tiles per split at least (the sampled pass, with few keys
// per row, keeps longer splits so each workgroup's operand loads pay off)
template <int HP, int D, bool F8, bool CAND>
int splits_t(int N, int L, int min_tiles = 4) {
  constexpr int QB = kRowsPerWG / HP;
  return choose_splits((N + QB - 1) / QB, L, chip_slots<HP, D, F8, CAND>(), min_tiles);
}

template <int HP, int D, bool F8>
hipError_t launch_t(const PrefillArgs& a, hipStream_t st) {
  PrefillParams p;
  p.q = static_cast<const uint8_t*>(a.q);
  p.w = a.w;
  p.q_scale = a.q_scale;
  p.k = static_cast<const uint8_t*>(a.k);
  p.k_scale = a.k_scale;
  p.q_pos = a.q_pos;
  p.heads = a.heads;
  p.N = a.N;
  p.H_I = a.H_I;
  p.h = a.heads ? a.h : a.H_I;
  p.u = a.u;
  p.u_stride = a.u_stride;
  p.key_step = a.key_step;
  p.pos_shift = a.pos_shift;
  p.L = (a.L + a.key_step - 1) / a.key_step;           // keys in scored units
  p.block_flag = a.block_flag;
  p.tau = a.tau;
  p.cnt_out = a.cnt_out;
  p.cand_out = a.cand_out;
  p.cap = a.cap;
  const size_t k_bytes = static_cast<size_t>(a.L) * PLayout<D, F8>::ROW;
  if (k_bytes >= (size_t{1} << 32)) return hipErrorInvalidValue;
  p.k_bytes = static_cast<uint32_t>(k_bytes);
  constexpr int QB = kRowsPerWG / HP;
  const int qblocks = (a.N + QB - 1) / QB;
  const int splits = a.cand_out ? splits_t<HP, D, F8, true>(a.N, p.L)
                                : splits_t<HP, D, F8, false>(a.N, p.L, a.key_step > 1 ? 16 : 4);
  p.splits = splits;
  p.keys_per_split = ((p.L + splits - 1) / splits + kKeyTile - 1) / kKeyTile * kKeyTile;
  if (a.cand_out)
    MISA_LAUNCH(a.kernel_id, (score_prefill_kernel<HP, D, F8, true>), dim3(splits, qblocks),
                dim3(256), 0, st, p);
  else
    MISA_LAUNCH(a.kernel_id, (score_prefill_kernel<HP, D, F8, false>), dim3(splits, qblocks),
                dim3(256), 0, st, p);
  return hipGetLastError();
}

template <int D, bool F8>
int cand_splits_d(int N, int L, int hp) {
  switch (hp) {
    case 4: return splits_t<4, D, F8, true>(N, L);
    case 8: return splits_t<8, D, F8, true>(N, L);
    case 16: return splits_t<16, D, F8, true>(N, L);
    case 32: return splits_t<32, D, F8, true>(N, L);
    default: return splits_t<64, D, F8, true>(N, L);
  }
}

template <int D, bool F8>
hipError_t launch_d(const PrefillArgs& a, hipStream_t st) {
  switch (hp_of(a.heads ? a.h : a.H_I)) {
    case 4: return launch_t<4, D, F8>(a, st);
    case 8: return launch_t<8, D, F8>(a, st);
    case 16: return launch_t<16, D, F8>(a, st);
    case 32: return launch_t<32, D, F8>(a, st);
    default: return launch_t<64, D, F8>(a, st);
  }
}

}  // namespace

int prefill_rows_per_block(int h_eff) { return kRowsPerWG / hp_of(h_eff); }

int prefill_cand_splits(int N, int L, int h_eff, int d, bool fp8) {
  const int hp = hp_of(h_eff);
  if (fp8) return cand_splits_d<128, true>(N, L, hp);
  return d == 64 ? cand_splits_d<64, false>(N, L, hp) : cand_splits_d<128, false>(N, L, hp);
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  if (a.fp8) return a.d == 128 ? launch_d<128, true>(a, st) : hipErrorInvalidValue;
  return a.d == 64 ? launch_d<64, false>(a, st) : launch_d<128, false>(a, st);
}

}  // namespace misa
