// Blockwise E4M3 quantisers for gfx950.
//
// Puro-2B paper, zh-TW translation (papers.lianghsun.dev), section 3.2:
// scales are computed online for every local group; activations and
// activation gradients use 1-D groups of 128 consecutive values along the
// GEMM reduction dimension, weights 128x128 2-D blocks.  Scale = amax/448 and
// the saturating round-to-nearest-even E4M3 cast are the readings stated in
// include/bfp8.h.  The same section says the scales ran as powers of two on
// the MXFP8 path; every kernel also takes that rule (RULE 1: the least power
// of two covering amax/448, stored as an E8M0 byte), and the row / token
// kernels the MXFP8 group length of 32 (Puro-2B tutorial, MXFP figure).
//
// All three kernels are HBM-bound (about 3 bytes moved per bf16 element and
// a handful of VALU operations), so the design goal is wide coalesced loads,
// enough bytes in flight per CU, and reductions that stay in registers
// (DPP within 16 lanes) or in a few LDS words.

#include <stdlib.h>

#include <algorithm>
#include <atomic>

#include "common.h"

namespace bfp8 {
namespace {

// Eight consecutive input elements as float32.  bf16 elements are widened
// exactly; `nvalid` (0..8) masks a ragged tail to +0.
template <typename T>
struct Load8;

template <>
struct Load8<uint16_t> {
  static __device__ __forceinline__ void run(const uint16_t* p, float (&v)[8], int nvalid) {
    if (nvalid >= 8) {
      uint4 u = *reinterpret_cast<const uint4*>(p);
      uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
        v[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = i < nvalid ? bf16_bits_to_f32(p[i]) : 0.0f;
    }
  }
};

template <>
struct Load8<float> {
  static __device__ __forceinline__ void run(const float* p, float (&v)[8], int nvalid) {
    if (nvalid >= 8) {
      float4 a = reinterpret_cast<const float4*>(p)[0];
      float4 b = reinterpret_cast<const float4*>(p)[1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = i < nvalid ? p[i] : 0.0f;
    }
  }
};

__device__ __forceinline__ float absmax8(const float (&v)[8]) {
  float m = fabsf(v[0]);
#pragma unroll
  for (int i = 1; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  return m;
}

__device__ __forceinline__ uint2 encode8(const float (&v)[8], float inv) {
  uint2 r;
  r.x = encode4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
  r.y = encode4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
  return r;
}

// Max over the lanes of one group: 16 lanes per 128-group, 4 per 32-group.
template <int GROUP>
__device__ __forceinline__ float group_lanes_max(float v) {
  return GROUP == 128 ? row16_max(v) : quad_max(v);
}

// ---------------------------------------------------------------------------
// K1: groups along rows.  16 lanes own one 128-element chunk (8 elements
// each, one 16-byte load for bf16) -- one group, or four 32-groups of four
// lanes each; a 256-thread block covers 16 chunks per unrolled step and
// issues all UNROLL steps' loads before any reduction.
// ---------------------------------------------------------------------------
constexpr int kActUnroll = 2;  // 4 and 8 measured 6 % slower at 8192 x 2048

template <typename T, int RULE, int GROUP, bool KM>
__global__ __launch_bounds__(256) void quantize_act_kernel(
    const T* __restrict__ x, int64_t ldx, uint8_t* __restrict__ q, int64_t ldq,
    typename ScaleRule<RULE>::type* __restrict__ s, uint32_t gpr, uint32_t n_groups,
    uint32_t rows) {
  // gpr / n_groups count 128-element chunks; s holds gpr * (128 / GROUP)
  // scales per row ([rows][gpr]), or, with KM (GROUP 128), one row of
  // `rows` scales per chunk ([gpr][rows]): then consecutive slots take
  // consecutive rows of one chunk, so a step's scales land side by side.
  const uint32_t lane16 = threadIdx.x & 15u;
  const uint32_t slot = threadIdx.x >> 4;  // 0..15: group within a step
  const uint32_t per_block = 16u * kActUnroll;
  for (uint32_t base = blockIdx.x * per_block; base < n_groups; base += gridDim.x * per_block) {
    float v[kActUnroll][8];
    uint32_t row[kActUnroll], gc[kActUnroll];
#pragma unroll
    for (int u = 0; u < kActUnroll; ++u) {
      const uint32_t g = base + u * 16u + slot;
      const bool ok = g < n_groups;
      if (KM) {
        gc[u] = ok ? g / rows : 0u;
        row[u] = ok ? g - gc[u] * rows : 0u;
      } else {
        row[u] = ok ? g / gpr : 0u;
        gc[u] = ok ? g - row[u] * gpr : 0u;
      }
      const T* p = x + static_cast<int64_t>(row[u]) * ldx + gc[u] * kGroup + lane16 * 8u;
      Load8<T>::run(p, v[u], ok ? 8 : 0);
    }
#pragma unroll
    for (int u = 0; u < kActUnroll; ++u) {
      const uint32_t g = base + u * 16u + slot;
      const float amax = group_lanes_max<GROUP>(absmax8(v[u]));
      float inv;
      const auto sc = ScaleRule<RULE>::make(amax, inv);
      if (g < n_groups) {
        uint2 codes = encode8(v[u], inv);
        *reinterpret_cast<uint2*>(q + static_cast<int64_t>(row[u]) * ldq + gc[u] * kGroup +
                                  lane16 * 8u) = codes;
        constexpr uint32_t kLanes = GROUP / 8;  // lanes per group
        constexpr uint32_t kSub = kGroup / GROUP;
        if (KM) {
          if (lane16 == 0) s[static_cast<int64_t>(gc[u]) * rows + row[u]] = sc;
        } else if (lane16 % kLanes == 0) {
          s[static_cast<int64_t>(row[u]) * gpr * kSub + gc[u] * kSub + lane16 / kLanes] = sc;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// K2: token-axis groups, transposed output.  A block owns 128 tokens x 64
// channels: coalesced row loads into an fp32 LDS tile, then thread
// (channel c, quarter p) walks 32 tokens of its channel; for 128-token
// groups the four quarters combine their amax through LDS (a 32-token group
// is one quarter), and each thread writes its 32 codes as two 16-byte
// stores into row c of qt.
// ---------------------------------------------------------------------------
constexpr int kTrTok = 128;
constexpr int kTrCh = 64;
constexpr int kTrLd = kTrCh + 4;  // padded fp32 row stride (16-byte aligned)

template <typename T, int RULE, int GROUP, bool KM>
__global__ __launch_bounds__(256) void quantize_act_t_kernel(
    const T* __restrict__ x, int64_t ldx, int64_t cols, uint8_t* __restrict__ qt, int64_t ldqt,
    typename ScaleRule<RULE>::type* __restrict__ st, int64_t n_tok_blocks) {
  // n_tok_blocks counts 128-token blocks; st rows hold n_tok_blocks *
  // (128 / GROUP) scales ([cols][n_tok_blocks]), or, with KM (GROUP 128),
  // one row of `cols` scales per token block ([n_tok_blocks][cols]).
  __shared__ __attribute__((aligned(16))) float tile[kTrTok * kTrLd];
  __shared__ float part[4][kTrCh];
  const int tid = threadIdx.x;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kTrCh;
  const int64_t tb = blockIdx.y;
  const int64_t m0 = tb * kTrTok;

  // load 128 x 64 elements: 1024 vectors of 8, four per thread
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int u = tid + 256 * j;
    const int r = u >> 3;
    const int cu = u & 7;
    const int64_t c = c0 + cu * 8;
    const int64_t left = cols - c;
    const int nvalid = left >= 8 ? 8 : (left > 0 ? static_cast<int>(left) : 0);
    float v[8];
    Load8<T>::run(x + (m0 + r) * ldx + (nvalid > 0 ? c : 0), v, nvalid);
    float4* dst = reinterpret_cast<float4*>(&tile[r * kTrLd + cu * 8]);
    dst[0] = make_float4(v[0], v[1], v[2], v[3]);
    dst[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
  __syncthreads();

  const int c = tid & 63;
  const int p = tid >> 6;
  float v[32];
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    v[i] = tile[(32 * p + i) * kTrLd + c];
    m = fmaxf(m, fabsf(v[i]));
  }
  float amax = m;
  if (GROUP == 128) {
    part[p][c] = m;
    __syncthreads();
    amax = fmaxf(fmaxf(part[0][c], part[1][c]), fmaxf(part[2][c], part[3][c]));
  }
  float inv;
  const auto sc = ScaleRule<RULE>::make(amax, inv);
  if (c0 + c < cols) {
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      w[i] = encode4(v[4 * i] * inv, v[4 * i + 1] * inv, v[4 * i + 2] * inv, v[4 * i + 3] * inv);
    uint4* dst = reinterpret_cast<uint4*>(qt + (c0 + c) * ldqt + m0 + 32 * p);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
    if (GROUP == 128) {
      if (p == 0) {
        if (KM) st[tb * cols + c0 + c] = sc;
        else st[(c0 + c) * n_tok_blocks + tb] = sc;
      }
    } else {
      st[(c0 + c) * n_tok_blocks * 4 + tb * 4 + p] = sc;
    }
  }
}

// ---------------------------------------------------------------------------
// K3: one 128x128 block per 256-thread workgroup.  Each thread keeps its 64
// elements in registers between the block-wide amax and the encode; partial
// edge blocks mask their missing elements to zero and store byte-wise.
// ---------------------------------------------------------------------------
// One 128x128 block (block row bm, block column bk) by the calling 256-thread
// workgroup; `red` is the workgroup's 4-float reduction buffer in LDS.
template <typename T, int RULE>
__device__ __forceinline__ void quantize_weight_block(
    const T* __restrict__ w, int64_t ldw, int64_t rows, int64_t cols, uint8_t* __restrict__ q,
    int64_t ldq, typename ScaleRule<RULE>::type* __restrict__ s, int64_t n_col_blocks,
    int64_t bm, int64_t bk, float* red) {
  const int tid = threadIdx.x;
  const int64_t r0 = bm * kGroup, k0 = bk * kGroup;
  float v[8][8];
  int nv[8];
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int u = tid + 256 * j;
    const int64_t r = r0 + (u >> 4);
    const int64_t c = k0 + (u & 15) * 8;
    const int64_t left = cols - c;
    int n = left >= 8 ? 8 : (left > 0 ? static_cast<int>(left) : 0);
    if (r >= rows) n = 0;
    nv[j] = n;
    Load8<T>::run(w + (n > 0 ? r * ldw + c : 0), v[j], n);
    m = fmaxf(m, absmax8(v[j]));
  }
  m = wave_max(m);
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float inv;
  const auto sc = ScaleRule<RULE>::make(amax, inv);
  if (tid == 0) s[bm * n_col_blocks + bk] = sc;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int u = tid + 256 * j;
    const int64_t r = r0 + (u >> 4);
    const int64_t c = k0 + (u & 15) * 8;
    if (nv[j] == 0) continue;
    uint2 codes = encode8(v[j], inv);
    uint8_t* dst = q + r * ldq + c;
    if (nv[j] == 8) {
      *reinterpret_cast<uint2*>(dst) = codes;
    } else {
      for (int e = 0; e < nv[j]; ++e)
        dst[e] = static_cast<uint8_t>((e < 4 ? codes.x >> (8 * e) : codes.y >> (8 * (e - 4))) & 0xFFu);
    }
  }
}

template <typename T, int RULE>
__global__ __launch_bounds__(256) void quantize_weight_kernel(
    const T* __restrict__ w, int64_t ldw, int64_t rows, int64_t cols, uint8_t* __restrict__ q,
    int64_t ldq, typename ScaleRule<RULE>::type* __restrict__ s, int64_t n_col_blocks) {
  __shared__ float red[4];
  quantize_weight_block<T, RULE>(w, ldw, rows, cols, q, ldq, s, n_col_blocks, blockIdx.y,
                                 blockIdx.x, red);
}

constexpr int kWeightWgsPerCu = 4;  // at most (two raw blocks per thread: ~130 VGPRs)

// Several weights in one launch: a flat block index walks the weights in
// order (first_block holds each weight's first index, kMaxWeightJobs + 1
// entries), so the blocks of every weight run side by side and a weight too
// small to fill the GPU on its own no longer leaves it idle.  The grid is a
// fixed number of workgroups (a few per CU) that stride over the blocks;
// each loads its next block into registers (raw input words) before it
// reduces, encodes and stores the current one, so every workgroup keeps two
// blocks of loads in flight and the whole batch runs as one round.  The
// per-block arithmetic is that of quantize_weight_block.
template <typename T>
struct RawBlock;  // this thread's 64 input elements of one 128x128 block, as loaded
template <>
struct RawBlock<uint16_t> {
  uint4 v[8];
};
template <>
struct RawBlock<float> {
  float4 v[16];
};

struct BlockRef {
  int j;        // weight index
  int64_t bm;   // block row
  int64_t bk;   // block column
};

__device__ __forceinline__ BlockRef block_ref(const WeightBatch& b, int64_t blk) {
  int j = 0;
  while (j + 1 < b.n && blk >= b.first_block[j + 1]) ++j;
  const int64_t local = blk - b.first_block[j];
  const int64_t cb = b.col_blocks[j];
  return BlockRef{j, local / cb, local % cb};
}

// Row r and first column c of this thread's vector u (0..7) of a block, and
// how many of its 8 elements are inside the weight.
__device__ __forceinline__ int vec_extent(const WeightBatch& b, const BlockRef& br, int u,
                                          int64_t& r, int64_t& c) {
  const int e = threadIdx.x + 256 * u;
  r = br.bm * kGroup + (e >> 4);
  c = br.bk * kGroup + (e & 15) * 8;
  const int64_t left = b.cols[br.j] - c;
  int n = left >= 8 ? 8 : (left > 0 ? static_cast<int>(left) : 0);
  if (r >= b.rows[br.j]) n = 0;
  return n;
}

template <typename T>
__device__ __forceinline__ void load_raw(const WeightBatch& b, const BlockRef& br,
                                         RawBlock<T>& raw) {
  const T* w = static_cast<const T*>(b.w[br.j]);
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    int64_t r, c;
    const int n = vec_extent(b, br, u, r, c);
    const T* p = w + r * b.ldw[br.j] + c;
    if constexpr (sizeof(T) == 2) {
      if (n == 8) {
        raw.v[u] = *reinterpret_cast<const uint4*>(p);
      } else {
        uint32_t h[8];
        for (int e = 0; e < 8; ++e) h[e] = e < n ? p[e] : 0u;
        raw.v[u] = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                              h[6] | (h[7] << 16));
      }
    } else {
      if (n == 8) {
        raw.v[2 * u] = reinterpret_cast<const float4*>(p)[0];
        raw.v[2 * u + 1] = reinterpret_cast<const float4*>(p)[1];
      } else {
        float f[8];
        for (int e = 0; e < 8; ++e) f[e] = e < n ? p[e] : 0.0f;
        raw.v[2 * u] = make_float4(f[0], f[1], f[2], f[3]);
        raw.v[2 * u + 1] = make_float4(f[4], f[5], f[6], f[7]);
      }
    }
  }
}

template <typename T>
__device__ __forceinline__ void unpack8(const RawBlock<T>& raw, int u, float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    const uint32_t w[4] = {raw.v[u].x, raw.v[u].y, raw.v[u].z, raw.v[u].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
      v[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
    }
  } else {
    const float4 a = raw.v[2 * u], c = raw.v[2 * u + 1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = c.x; v[5] = c.y; v[6] = c.z; v[7] = c.w;
  }
}

// Block amax (elements outside the weight were loaded as +0), scale, codes.
template <typename T, int RULE>
__device__ __forceinline__ void quantize_raw_block(const WeightBatch& b, const BlockRef& br,
                                                   const RawBlock<T>& raw, float* red) {
  float m = 0.0f;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    float v[8];
    unpack8<T>(raw, u, v);
    m = fmaxf(m, absmax8(v));
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float inv;
  const auto sc = ScaleRule<RULE>::make(amax, inv);
  if (threadIdx.x == 0)
    static_cast<typename ScaleRule<RULE>::type*>(b.s[br.j])[br.bm * b.col_blocks[br.j] + br.bk] = sc;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    int64_t r, c;
    const int n = vec_extent(b, br, u, r, c);
    if (n == 0) continue;
    float v[8];
    unpack8<T>(raw, u, v);
    const uint2 codes = encode8(v, inv);
    uint8_t* dst = b.q[br.j] + r * b.ldq[br.j] + c;
    if (n == 8) {
      *reinterpret_cast<uint2*>(dst) = codes;
    } else {
      for (int e = 0; e < n; ++e)
        dst[e] = static_cast<uint8_t>((e < 4 ? codes.x >> (8 * e) : codes.y >> (8 * (e - 4))) & 0xFFu);
    }
  }
}

template <typename T, int RULE>
__global__ __launch_bounds__(256) void quantize_weight_batch_kernel(WeightBatch b) {
  // two reduction buffers, used alternately: a block's buffer is rewritten
  // two blocks later, after the barrier of the block in between, which no
  // thread passes before every thread has read the first
  __shared__ float red[2][4];
  const int64_t nblk = b.first_block[b.n];
  int64_t blk = blockIdx.x;
  if (blk >= nblk) return;  // uniform per workgroup
  RawBlock<T> cur;
  BlockRef cref = block_ref(b, blk);
  load_raw<T>(b, cref, cur);
  for (int ph = 0; blk < nblk; blk += gridDim.x, ph ^= 1) {
    const int64_t nb = blk + gridDim.x;
    RawBlock<T> nxt;
    BlockRef nref = cref;
    if (nb < nblk) {
      nref = block_ref(b, nb);
      load_raw<T>(b, nref, nxt);
    }
    quantize_raw_block<T, RULE>(b, cref, cur, red[ph]);
    cur = nxt;
    cref = nref;
  }
}

// ---------------------------------------------------------------------------
// K1+K2 fused (float32 inputs, 1x32 groups, and bf16 inputs of 6144 channels
// or more with row-major scales; other bf16 128-group inputs take
// quantize_dual_ct_kernel below): one read of a 128-token x (128*CB)-channel
// tile emits both the row-grouped codes (groups along channels: the fprop /
// dgrad operand) and the token-grouped codes written transposed (groups along
// tokens: the wgrad operand).  Phase 1 works from registers (16 lanes per row group, as
// K1) and parks the raw tile in LDS; phase 2 walks columns of the LDS tile
// (two channels per thread, a quarter of the tokens each) as K2 does.  Both
// outputs are bit-identical to the two separate quantisers.  CB = 2 (512
// threads) writes each row's two float32 scales as one 8-byte store: the
// scattered 4-byte scale stores are the kernel's largest cost after the
// codes themselves.
// ---------------------------------------------------------------------------
template <typename T>
struct DualTile;
template <>
struct DualTile<uint16_t> {
  static constexpr int kLd = 128 + 8;  // bf16 elements per LDS row (16-byte aligned rows)
};
template <>
struct DualTile<float> {
  static constexpr int kLd = 128 + 4;
};

// Two adjacent scales in one store (the index of the first is even).
__device__ __forceinline__ void store_scale_pair(float* p, float a, float b) {
  *reinterpret_cast<float2*>(p) = make_float2(a, b);
}
__device__ __forceinline__ void store_scale_pair(uint8_t* p, uint8_t a, uint8_t b) {
  *reinterpret_cast<uint16_t*>(p) = static_cast<uint16_t>(a | (b << 8));
}

template <typename T, int RULE, int GROUP, int CB, bool KM>
__global__ __launch_bounds__(256 * CB) void quantize_dual_kernel(
    const T* __restrict__ x, int64_t ldx, uint8_t* __restrict__ q, int64_t ldq,
    typename ScaleRule<RULE>::type* __restrict__ s, uint8_t* __restrict__ qt, int64_t ldqt,
    typename ScaleRule<RULE>::type* __restrict__ st, int64_t n_ch_blocks, int64_t n_tok_blocks) {
  // KM (GROUP 128): both scale tensors K-block major -- row scales
  // [n_ch_blocks][rows], token scales [n_tok_blocks][cols] -- so a tile's
  // 128 row scales per channel block and its 128 * CB token scales each
  // leave as one contiguous run.
  typedef typename ScaleRule<RULE>::type S;
  constexpr int kSub = kGroup / GROUP;  // groups per 128 along either axis
  constexpr int kLd = DualTile<T>::kLd + 128 * (CB - 1);
  constexpr int kCh = 128 * CB;         // channels per tile
  __shared__ __attribute__((aligned(16))) T tile[128 * kLd];
  __shared__ float part[4][kCh];
  __shared__ __attribute__((aligned(16))) S rsc[KM ? CB : 1][128];  // KM: row scales of the tile
  const int tid = threadIdx.x;
  const int64_t cb = static_cast<int64_t>(blockIdx.x) * CB, tb = blockIdx.y;
  const int64_t m0 = tb * 128, c0 = cb * 128;

  // ---- phase 1: row groups (one per token row of the tile) -------------
  // 16 lanes per 128-channel group, CB groups side by side per row
  const int lane16 = tid & 15, gsub = (tid >> 4) % CB, rsub = tid / (16 * CB);
  const int cofs = gsub * 128 + lane16 * 8;  // channel offset within the tile
  float v[8][8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int r = rsub + 16 * u;
    Load8<T>::run(x + (m0 + r) * ldx + c0 + cofs, v[u], 8);
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int r = rsub + 16 * u;
    const float amax = group_lanes_max<GROUP>(absmax8(v[u]));
    float inv;
    const auto sc = ScaleRule<RULE>::make(amax, inv);
    *reinterpret_cast<uint2*>(q + (m0 + r) * ldq + c0 + cofs) = encode8(v[u], inv);
    if (KM) {
      if (lane16 == 0) rsc[KM ? gsub : 0][r] = sc;
    } else if (CB == 2 && GROUP == 128 && RULE == 0) {
      // the row's two scales are adjacent: one 8-byte store from group 0
      const float sc1 = __shfl_down(static_cast<float>(sc), 16, 32);
      if (tid % 32 == 0)
        *reinterpret_cast<float2*>(reinterpret_cast<float*>(s) + (m0 + r) * n_ch_blocks + cb) =
            make_float2(static_cast<float>(sc), sc1);
    } else if (lane16 % (GROUP / 8) == 0) {
      s[(m0 + r) * n_ch_blocks * kSub + (cb + gsub) * kSub + lane16 / (GROUP / 8)] = sc;
    }
    T* dst = tile + r * kLd + cofs;
    if (sizeof(T) == 2) {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = (__float_as_uint(v[u][2 * i]) >> 16) | (__float_as_uint(v[u][2 * i + 1]) & 0xFFFF0000u);
      *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      reinterpret_cast<float4*>(dst)[0] = make_float4(v[u][0], v[u][1], v[u][2], v[u][3]);
      reinterpret_cast<float4*>(dst)[1] = make_float4(v[u][4], v[u][5], v[u][6], v[u][7]);
    }
  }
  __syncthreads();

  // ---- phase 2: token groups (one per channel), written transposed -----
  const int cp = tid % (64 * CB), p = tid / (64 * CB);  // channels 2cp, 2cp+1; tokens 32p..
  float a[32], b[32];
  float ma = 0.0f, mb = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const T* src = tile + (32 * p + i) * kLd + 2 * cp;
    if (sizeof(T) == 2) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(src);
      a[i] = bf16_bits_to_f32(w & 0xFFFFu);
      b[i] = bf16_bits_to_f32(w >> 16);
    } else {
      const float2 w = *reinterpret_cast<const float2*>(src);
      a[i] = w.x;
      b[i] = w.y;
    }
    ma = fmaxf(ma, fabsf(a[i]));
    mb = fmaxf(mb, fabsf(b[i]));
  }
  float amax_a = ma, amax_b = mb;
  if (GROUP == 128) {
    part[p][2 * cp] = ma;
    part[p][2 * cp + 1] = mb;
    __syncthreads();
    amax_a = fmaxf(fmaxf(part[0][2 * cp], part[1][2 * cp]), fmaxf(part[2][2 * cp], part[3][2 * cp]));
    amax_b = fmaxf(fmaxf(part[0][2 * cp + 1], part[1][2 * cp + 1]),
                   fmaxf(part[2][2 * cp + 1], part[3][2 * cp + 1]));
  }
  float inva, invb;
  const auto sa = ScaleRule<RULE>::make(amax_a, inva);
  const auto sb = ScaleRule<RULE>::make(amax_b, invb);
  uint32_t wa[8], wb[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    wa[i] = encode4(a[4 * i] * inva, a[4 * i + 1] * inva, a[4 * i + 2] * inva, a[4 * i + 3] * inva);
    wb[i] = encode4(b[4 * i] * invb, b[4 * i + 1] * invb, b[4 * i + 2] * invb, b[4 * i + 3] * invb);
  }
  uint4* da = reinterpret_cast<uint4*>(qt + (c0 + 2 * cp) * ldqt + m0 + 32 * p);
  uint4* db = reinterpret_cast<uint4*>(qt + (c0 + 2 * cp + 1) * ldqt + m0 + 32 * p);
  da[0] = make_uint4(wa[0], wa[1], wa[2], wa[3]);
  da[1] = make_uint4(wa[4], wa[5], wa[6], wa[7]);
  db[0] = make_uint4(wb[0], wb[1], wb[2], wb[3]);
  db[1] = make_uint4(wb[4], wb[5], wb[6], wb[7]);
  if (KM) {
    const int64_t cols = n_ch_blocks * 128;
    if (p == 0) store_scale_pair(st + tb * cols + c0 + 2 * cp, sa, sb);
    if (p == 1) {
      // row scales of channel block cb + cp / 64, rows 2 (cp % 64) and one more
      const int gs = cp / 64, rr = 2 * (cp % 64);
      store_scale_pair(s + (cb + gs) * (n_tok_blocks * 128) + m0 + rr, rsc[gs][rr], rsc[gs][rr + 1]);
    }
  } else if (GROUP == 128) {
    if (p == 0) {
      st[(c0 + 2 * cp) * n_tok_blocks + tb] = sa;
      st[(c0 + 2 * cp + 1) * n_tok_blocks + tb] = sb;
    }
  } else {
    st[(c0 + 2 * cp) * n_tok_blocks * kSub + tb * kSub + p] = sa;
    st[(c0 + 2 * cp + 1) * n_tok_blocks * kSub + tb * kSub + p] = sb;
  }
}

// ---------------------------------------------------------------------------
// K1+K2 fused, bf16 input, 128-groups, one 128 x 128 tile per 256-thread
// workgroup: the same outputs as quantize_dual_kernel, with the tile
// transposed through LDS as E4M3 codes (16 KiB) instead of as bf16 values
// (34 KiB), so the LDS traffic per tile halves and one barrier fewer is
// needed (10 % faster on 2048 channels, 0.9-1.0 of a plain device copy of
// the input at every width).
// Thread (rsub, lane16) holds tokens 8 rsub .. 8 rsub + 7 of channels
// 8 lane16 .. 8 lane16 + 7 as raw bf16 words.  Row groups are quantised
// from them directly; the column maxima of the four waves meet in LDS; each
// thread then encodes its 8 x 8 values with the column scales, and its 8
// codes of one channel (consecutive tokens) go to that channel's LDS row as
// one 8-byte write.  The rows of the code tile are finally copied to qt as
// 128-byte runs.  The 16-byte chunks of a code row are XOR-swizzled by
// (channel / 8) & 7 to spread the writes over the banks.
// ---------------------------------------------------------------------------
constexpr int kCtCh = 128;

template <int RULE, int GROUP, bool KM, bool ROWS>
__global__ __launch_bounds__(256) void quantize_dual_ct_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, uint8_t* __restrict__ q, int64_t ldq,
    typename ScaleRule<RULE>::type* __restrict__ s, uint8_t* __restrict__ qt, int64_t ldqt,
    typename ScaleRule<RULE>::type* __restrict__ st, int64_t n_ch_blocks, int64_t n_tok_blocks) {
  typedef typename ScaleRule<RULE>::type S;
  constexpr int kSub = kGroup / GROUP;  // groups per 128 along either axis
  __shared__ __attribute__((aligned(16))) uint8_t ct[kCtCh * 128];  // [channel][token]
  __shared__ float colmax[4][kCtCh];
  __shared__ __attribute__((aligned(16))) S rsc[128];
  const int tid = threadIdx.x;
  const int lane16 = tid & 15, rsub = tid >> 4, wave = tid >> 6;
  const int64_t cb = blockIdx.x, tb = blockIdx.y;
  const int64_t m0 = tb * 128, c0 = cb * 128;

  typedef uint32_t raw4 __attribute__((ext_vector_type(4)));
  raw4 raw[8];
#pragma unroll
  for (int u = 0; u < 8; ++u)
    raw[u] = *reinterpret_cast<const raw4*>(x + (m0 + 8 * rsub + u) * ldx + c0 + lane16 * 8);
  auto elem = [&](int u, int k) -> float {
    const uint32_t w = k < 2 ? raw[u].x : (k < 4 ? raw[u].y : (k < 6 ? raw[u].z : raw[u].w));
    return bf16_bits_to_f32((k & 1) ? (w >> 16) : (w & 0xFFFFu));
  };

  // ---- row groups (ROWS == false: the token-axis quantiser alone) ---------
  float cm[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) cm[k] = 0.0f;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      v[k] = elem(u, k);
      cm[k] = fmaxf(cm[k], fabsf(v[k]));
    }
    if constexpr (!ROWS) continue;
    const float amax = group_lanes_max<GROUP>(absmax8(v));
    float inv;
    const S sc = ScaleRule<RULE>::make(amax, inv);
    const int64_t r = m0 + 8 * rsub + u;
    *reinterpret_cast<uint2*>(q + r * ldq + c0 + lane16 * 8) = encode8(v, inv);
    if (lane16 % (GROUP / 8) == 0) {
      if (KM) rsc[8 * rsub + u] = sc;
      else s[r * n_ch_blocks * kSub + cb * kSub + lane16 / (GROUP / 8)] = sc;
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // the column pass re-reads the raw words (keeps the unpacked values from
  // living across both passes, which would halve the resident workgroups)
#pragma unroll
  for (int u = 0; u < 8; ++u) asm volatile("" : "+v"(raw[u]));

  // ---- column maxima: the wave's four token octets (a 32-token group), then
  // for 128-token groups the four waves ------------------------------------
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    cm[k] = fmaxf(cm[k], __shfl_xor(cm[k], 16));
    cm[k] = fmaxf(cm[k], __shfl_xor(cm[k], 32));
  }
  if (GROUP == 128) {
    if ((tid & 48) == 0) {
#pragma unroll
      for (int k = 0; k < 8; ++k) colmax[wave][lane16 * 8 + k] = cm[k];
    }
    __syncthreads();
  }

  // ---- token groups: encode with the column scales, transpose via LDS ----
  // (one channel at a time, its scale stored at once, so that only the raw
  // words stay live across the loop)
  const int chunk_w = (rsub >> 1) ^ (lane16 & 7);  // tokens 8 rsub .. +7: chunk rsub / 2
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int c = lane16 * 8 + k;
    const float amax = GROUP == 128 ? fmaxf(fmaxf(colmax[0][c], colmax[1][c]),
                                            fmaxf(colmax[2][c], colmax[3][c]))
                                    : cm[k];
    float inv;
    const S sc = ScaleRule<RULE>::make(amax, inv);
    const uint32_t lo = encode4(elem(0, k) * inv, elem(1, k) * inv, elem(2, k) * inv, elem(3, k) * inv);
    const uint32_t hi = encode4(elem(4, k) * inv, elem(5, k) * inv, elem(6, k) * inv, elem(7, k) * inv);
    *reinterpret_cast<uint2*>(&ct[c * 128 + chunk_w * 16 + (rsub & 1) * 8]) = make_uint2(lo, hi);
    if (GROUP == 128 && rsub == 0) {
      if (KM) st[tb * (n_ch_blocks * 128) + c0 + c] = sc;
      else st[(c0 + c) * n_tok_blocks + tb] = sc;
    } else if (GROUP == 32 && (rsub & 3) == 0) {
      st[(c0 + c) * n_tok_blocks * kSub + tb * kSub + wave] = sc;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();

  // ---- code rows -> qt (8 lanes per channel, 16 bytes each) ----------------
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int c = pass * 32 + (tid >> 3), chunk = tid & 7;
    const int phys = chunk ^ ((c >> 3) & 7);
    const uint4 w = *reinterpret_cast<const uint4*>(&ct[c * 128 + phys * 16]);
    *reinterpret_cast<uint4*>(qt + (c0 + c) * ldqt + m0 + chunk * 16) = w;
  }
  if (ROWS && KM && tid < 32) {
    // the tile's 128 row scales of channel block cb, one contiguous run
    S* dst = s + cb * (n_tok_blocks * 128) + m0;
    if constexpr (sizeof(S) == 4) {
      reinterpret_cast<float4*>(dst)[tid] = reinterpret_cast<const float4*>(rsc)[tid];
    } else {
      reinterpret_cast<uint32_t*>(dst)[tid] = reinterpret_cast<const uint32_t*>(rsc)[tid];
    }
  }
}

// ---- opt-in input check (BFP8_DEBUG) ---------------------------------------
// One flag word per GPU: set to 1 by any thread that finds a non-finite
// input element.  Cleared by a kernel (not a memset) before each check.
__device__ __align__(16) uint32_t nonfinite_flag[4];

__global__ __launch_bounds__(64) void clear_flag_kernel(uint32_t* flag) {
  if (threadIdx.x == 0) flag[0] = 0u;
}

// Grid-stride over the rows x cols elements of x (row stride ldx); exponent
// field all ones marks Inf or NaN for both bf16 and float32.
template <typename T>
__global__ __launch_bounds__(256) void find_nonfinite_kernel(const T* __restrict__ x, int64_t ldx,
                                                             int64_t rows, int64_t cols,
                                                             uint32_t* flag) {
  const int64_t n = rows * cols;
  bool bad = false;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t r = i / cols, c = i - r * cols;
    if constexpr (sizeof(T) == 2) {
      const uint32_t b = x[r * ldx + c];
      bad |= (b & 0x7F80u) == 0x7F80u;
    } else {
      const uint32_t b = __float_as_uint(x[r * ldx + c]);
      bad |= (b & 0x7F800000u) == 0x7F800000u;
    }
  }
  if (bad) flag[0] = 1u;
}

}  // namespace

// Instantiate a kernel for the (input type, rule, group) triple chosen at
// run time.  Valid triples: rule 0 with group 128; rule 1 with 32 or 128.
#define BFP8_DISPATCH(KERNEL_CALL)                                           \
  do {                                                                       \
    if (dt == BFP8_IN_BF16) {                                                \
      typedef uint16_t T;                                                    \
      if (rule == 0) { constexpr int R = 0, G = 128; KERNEL_CALL; }          \
      else if (group == 128) { constexpr int R = 1, G = 128; KERNEL_CALL; }  \
      else { constexpr int R = 1, G = 32; KERNEL_CALL; }                     \
    } else {                                                                 \
      typedef float T;                                                       \
      if (rule == 0) { constexpr int R = 0, G = 128; KERNEL_CALL; }          \
      else if (group == 128) { constexpr int R = 1, G = 128; KERNEL_CALL; }  \
      else { constexpr int R = 1, G = 32; KERNEL_CALL; }                     \
    }                                                                        \
  } while (0)

// As BFP8_DISPATCH, and the scale-layout flag: KMV = km (group 128 only).
#define BFP8_DISPATCH_KM(KERNEL_CALL)                                      \
  BFP8_DISPATCH(if constexpr (G == 128) {                                  \
    if (km) { constexpr bool KMV = true; KERNEL_CALL; }                    \
    else { constexpr bool KMV = false; KERNEL_CALL; }                      \
  } else { constexpr bool KMV = false; KERNEL_CALL; })

bfp8_status launch_quantize_act(const void* x, bfp8_in_dtype dt, int64_t rows, int64_t cols,
                                int64_t ldx, int rule, int group, uint8_t* q, int64_t ldq,
                                void* s, bool km, hipStream_t stream) {
  const int64_t gpr = cols / kGroup;
  const int64_t n_groups = rows * gpr;
  if (n_groups == 0) return BFP8_OK;
  const int64_t per_block = 16 * kActUnroll;
  int64_t blocks = (n_groups + per_block - 1) / per_block;
  if (blocks > 16384) blocks = 16384;
  bfp8_status st = BFP8_OK;
  BFP8_DISPATCH_KM((st = launch(&quantize_act_kernel<T, R, G, KMV>,
                                dim3(static_cast<unsigned>(blocks)), dim3(256), stream,
                                static_cast<const T*>(x), ldx, q, ldq,
                                static_cast<typename ScaleRule<R>::type*>(s),
                                static_cast<uint32_t>(gpr), static_cast<uint32_t>(n_groups),
                                static_cast<uint32_t>(rows))));
  return st;
}

bfp8_status launch_quantize_act_transposed(const void* x, bfp8_in_dtype dt, int64_t rows,
                                           int64_t cols, int64_t ldx, int rule, int group,
                                           uint8_t* qt, int64_t ldqt, void* st, bool km,
                                           hipStream_t stream) {
  if (rows == 0 || cols == 0) return BFP8_OK;
  const int64_t tok_blocks = rows / kTrTok;
  // bf16, whole 128-channel blocks: the code-transposing kernel without its
  // row groups (24 % faster than the fp32-tile kernel below at 8192 x 6144,
  // and faster than a plain copy of its input)
  if (dt == BFP8_IN_BF16 && cols % kGroup == 0) {
    const dim3 g2(static_cast<unsigned>(cols / kGroup), static_cast<unsigned>(tok_blocks));
    bfp8_status status = BFP8_OK;
    BFP8_DISPATCH_KM((status = launch(&quantize_dual_ct_kernel<R, G, KMV, false>, g2, dim3(256),
                                      stream, static_cast<const uint16_t*>(x), ldx, nullptr,
                                      int64_t(0), nullptr, qt, ldqt,
                                      static_cast<typename ScaleRule<R>::type*>(st),
                                      cols / kGroup, tok_blocks)));
    return status;
  }
  dim3 grid(static_cast<unsigned>((cols + kTrCh - 1) / kTrCh), static_cast<unsigned>(tok_blocks));
  bfp8_status status = BFP8_OK;
  BFP8_DISPATCH_KM((status = launch(&quantize_act_t_kernel<T, R, G, KMV>, grid, dim3(256),
                                    stream, static_cast<const T*>(x), ldx, cols, qt, ldqt,
                                    static_cast<typename ScaleRule<R>::type*>(st), tok_blocks)));
  return status;
}

bfp8_status launch_quantize_act_dual(const void* x, bfp8_in_dtype dt, int64_t rows, int64_t cols,
                                     int64_t ldx, int rule, int group, uint8_t* q, int64_t ldq,
                                     void* s, uint8_t* qt, int64_t ldqt, void* st, bool km,
                                     hipStream_t stream) {
  if (rows == 0 || cols == 0) return BFP8_OK;
  const int64_t ch_blocks = cols / kGroup, tok_blocks = rows / kGroup;
  // bf16 inputs of 6144 channels or more with row-major scales: 128 x 256
  // tiles (512 threads), whose row scales go out as 8-byte pairs (measured
  // 5-7 % faster there, slower on narrower inputs); with K-block-major
  // scales every tile's scales leave as contiguous runs anyway and the
  // code-transposing kernel below is as fast or faster at every width
  if (dt == BFP8_IN_BF16 && ch_blocks % 2 == 0 && ch_blocks >= 48 && group == kGroup && !km) {
    dim3 grid2(static_cast<unsigned>(ch_blocks / 2), static_cast<unsigned>(tok_blocks));
    bfp8_status status = BFP8_OK;
    BFP8_DISPATCH_KM((status = launch(&quantize_dual_kernel<uint16_t, R, G, 2, KMV>, grid2, dim3(512),
                                   stream, static_cast<const uint16_t*>(x), ldx, q, ldq,
                                   static_cast<typename ScaleRule<R>::type*>(s), qt, ldqt,
                                   static_cast<typename ScaleRule<R>::type*>(st), ch_blocks,
                                   tok_blocks)));
    return status;
  }
  dim3 grid(static_cast<unsigned>(ch_blocks), static_cast<unsigned>(tok_blocks));
  bfp8_status status = BFP8_OK;
  // bf16 inputs (all widths with K-block-major scales or 32-groups, fewer
  // than 6144 channels otherwise): the code-transposing form
  if (dt == BFP8_IN_BF16) {
    BFP8_DISPATCH_KM((status = launch(&quantize_dual_ct_kernel<R, G, KMV, true>, grid, dim3(256),
                                      stream, static_cast<const uint16_t*>(x), ldx, q, ldq,
                                      static_cast<typename ScaleRule<R>::type*>(s), qt, ldqt,
                                      static_cast<typename ScaleRule<R>::type*>(st), ch_blocks,
                                      tok_blocks)));
    return status;
  }
  BFP8_DISPATCH_KM((status = launch(&quantize_dual_kernel<T, R, G, 1, KMV>, grid, dim3(256), stream,
                                 static_cast<const T*>(x), ldx, q, ldq,
                                 static_cast<typename ScaleRule<R>::type*>(s), qt, ldqt,
                                 static_cast<typename ScaleRule<R>::type*>(st), ch_blocks,
                                 tok_blocks)));
  return status;
}

// Workgroups of quantize_weight_batch_kernel<T, RULE> resident per CU (at
// most kWeightWgsPerCu), queried once: every GPU the library runs on is the
// same gfx950 part.
template <typename T, int RULE>
static bfp8_status weight_batch_residency(int& per_cu) {
  static std::atomic<int> cached{0};
  per_cu = cached.load(std::memory_order_relaxed);
  if (per_cu > 0) return BFP8_OK;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, quantize_weight_batch_kernel<T, RULE>,
                                                   256, 0) != hipSuccess)
    return BFP8_ERR_HIP;
  per_cu = std::max(1, std::min(per_cu, kWeightWgsPerCu));
  cached.store(per_cu, std::memory_order_relaxed);
  return BFP8_OK;
}

bfp8_status launch_quantize_weight_batch(const WeightBatch& b, bfp8_in_dtype dt, int rule,
                                         hipStream_t stream) {
  const int64_t blocks = b.first_block[b.n];
  if (blocks == 0) return BFP8_OK;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return BFP8_ERR_HIP;
  // As many workgroups as are resident at once (the kernel is persistent: a
  // workgroup that has to wait for a slot would run its whole share late),
  // at most kWeightWgsPerCu per CU and never more than there are blocks.
  // Residency is register-limited and differs between instantiations.
  int per_cu = 0;
  bfp8_status st = BFP8_OK;
  if (dt == BFP8_IN_BF16)
    st = rule == 0 ? weight_batch_residency<uint16_t, 0>(per_cu)
                   : weight_batch_residency<uint16_t, 1>(per_cu);
  else
    st = rule == 0 ? weight_batch_residency<float, 0>(per_cu)
                   : weight_batch_residency<float, 1>(per_cu);
  if (st != BFP8_OK) return st;
  const int64_t wgs = std::min<int64_t>(blocks, static_cast<int64_t>(cus) * per_cu);
  const dim3 grid(static_cast<unsigned>(wgs)), block(256);
  if (dt == BFP8_IN_BF16) {
    if (rule == 0) return launch(&quantize_weight_batch_kernel<uint16_t, 0>, grid, block, stream, b);
    return launch(&quantize_weight_batch_kernel<uint16_t, 1>, grid, block, stream, b);
  }
  if (rule == 0) return launch(&quantize_weight_batch_kernel<float, 0>, grid, block, stream, b);
  return launch(&quantize_weight_batch_kernel<float, 1>, grid, block, stream, b);
}

bfp8_status launch_quantize_weight(const void* w, bfp8_in_dtype dt, int64_t rows, int64_t cols,
                                   int64_t ldw, int rule, uint8_t* q, int64_t ldq, void* s,
                                   hipStream_t stream) {
  if (rows == 0 || cols == 0) return BFP8_OK;
  const int64_t rb = (rows + kGroup - 1) / kGroup;
  const int64_t cb = (cols + kGroup - 1) / kGroup;
  dim3 grid(static_cast<unsigned>(cb), static_cast<unsigned>(rb));
  const int group = 128;
  bfp8_status status = BFP8_OK;
  BFP8_DISPATCH((status = launch(&quantize_weight_kernel<T, R>, grid, dim3(256), stream,
                                 static_cast<const T*>(w), ldw, rows, cols, q, ldq,
                                 static_cast<typename ScaleRule<R>::type*>(s), cb)));
  (void)group;
  return status;
}

#undef BFP8_DISPATCH_KM
#undef BFP8_DISPATCH

bool debug_checks_enabled() {
  static const bool on = [] {
    const char* v = getenv("BFP8_DEBUG");
    return v != nullptr && v[0] != '\0' && !(v[0] == '0' && v[1] == '\0');
  }();
  return on;
}

bfp8_status check_finite(const void* x, bfp8_in_dtype dt, int64_t rows, int64_t cols, int64_t ldx,
                         hipStream_t stream) {
  if (rows == 0 || cols == 0) return BFP8_OK;
  void* flag = nullptr;
  if (hipGetSymbolAddress(&flag, HIP_SYMBOL(nonfinite_flag)) != hipSuccess) return BFP8_ERR_HIP;
  uint32_t* f = static_cast<uint32_t*>(flag);
  bfp8_status st = launch(&clear_flag_kernel, dim3(1), dim3(64), stream, f);
  if (st != BFP8_OK) return st;
  int64_t blocks = (rows * cols + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  const dim3 grid(static_cast<unsigned>(blocks));
  st = dt == BFP8_IN_BF16
           ? launch(&find_nonfinite_kernel<uint16_t>, grid, dim3(256), stream,
                    static_cast<const uint16_t*>(x), ldx, rows, cols, f)
           : launch(&find_nonfinite_kernel<float>, grid, dim3(256), stream,
                    static_cast<const float*>(x), ldx, rows, cols, f);
  if (st != BFP8_OK) return st;
  uint32_t host = 0;
  if (hipMemcpyAsync(&host, f, sizeof(host), hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return BFP8_ERR_HIP;
  return host != 0u ? BFP8_ERR_NONFINITE : BFP8_OK;
}

}  // namespace bfp8
