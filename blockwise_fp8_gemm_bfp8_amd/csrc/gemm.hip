// Blockwise FP8 GEMM for gfx950: C = sum_kb (A_kb . B_kb) * sA * sB -> bf16.
//
// Puro-2B paper, zh-TW translation (papers.lianghsun.dev), section 2 and
// section 3.2: the main Transformer linear-layer GEMMs run on E4M3 operands
// with fine-grained (DeepSeek-V3 style) scales -- 1x128 groups along K for
// activations and activation gradients, 128x128 blocks for weights.  Each
// 128-deep K block yields an fp32 partial from the matrix cores that is
// multiplied by a_scale * b_scale and added into an fp32 accumulator; the
// result is stored as bf16.
//
// Kernel shape (one 256x256 output tile per 512-thread workgroup, one
// workgroup per CU):
//   * global -> LDS with buffer_load ... lds (no VGPR staging), two stages
//     of 256x128 A bytes + 256x128 B bytes + 2x256 act-mode scales;
//   * K-contiguous operands sit in LDS as [row][128 B] with their 16-byte
//     chunks XOR-swizzled by row and are read with ds_read_b128;
//     K-major operands (A of TN, B of NN/TN) sit as [k][256 B] with chunks
//     swizzled by k and are read with ds_read_b64_tr_b8, which transposes
//     8 k-rows x 16 columns of bytes across a 16-lane group -- no separate
//     transpose pass and no workspace;
//   * 8 waves as 4 (M) x 2 (N), wave tile 64 x 128 = 4 x 8 subtiles;
//   * v_mfma_f32_16x16x128_f8f6f4 (E4M3 x E4M3 -> fp32), one instruction per
//     16x16 subtile per K block, issued with the B tile as the first operand
//     so each lane owns 4 consecutive output columns of one row;
//   * promotion acc += P * (sA * sB) on the VALU, three MFMA issues behind
//     the MFMA that produced P, so it overlaps matrix-core work; the last
//     three partials of a K block are promoted after the barrier, under the
//     LDS reads of the next block's fragments;
//   * XCD-aware tile order: consecutive tiles go to the same XCD (the
//     hardware deals workgroups to the 8 XCDs round robin) and tiles are
//     grouped along M so concurrent tiles on an XCD share A rows and B
//     columns in that XCD's L2;
//   * grids that under-fill the GPU: whole waves of tiles run unsplit and
//     only the tiles of a last, partial wave are split along K (fp32
//     partials summed in split order by a second kernel), or, for NT
//     problems with 1x128 scales on B, 256 x 192 tiles where they fill
//     whole waves that 256 x 256 tiles would leave partly idle.
//
// Operands whose scales are powers of two stored as E8M0 bytes (Puro-2B
// translation, section 3.2: the SM120 runs used power-of-two block scales on
// the MXFP8 path) go to gemm_mx4_kernel: the same tile and LDS stages, but
// the scales ride in the matrix-core instruction
// (v_mfma_scale_f32_16x16x128_f8f6f4), the accumulators are the MFMA's C
// operand in the AGPR file, and no VALU promotion is needed, which lets 4
// waves of 128 x 128 replace 8 waves of 64 x 128.  That kernel is also
// persistent: one workgroup per CU walks its tiles, and each tile's last K
// block copies the next tile's first.  The instruction takes one
// scale byte per row and 32-deep K chunk: the register of lane group j
// (lane 16j + r) scales row r's K values [32j, 32j + 32) -- which the
// fragment layout below spreads over lane groups 2j mod 4 and 2j + 1 mod 4
// (measured on gfx950) -- so the lane's byte is always its row's scale of
// chunk j = lane / 16.

#include <atomic>
#include <mutex>

#include "common.h"

namespace bfp8 {
namespace {

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int kWavesM = 4, kWavesN = 2;
constexpr int WM = BM / kWavesM;  // 64
constexpr int WN = BN / kWavesN;  // 128
constexpr int TM = WM / 16;       // 4 row subtiles
constexpr int TN = WN / 16;       // 8 column subtiles
constexpr int kThreads = 64 * kWavesM * kWavesN;  // 512
constexpr int kTileABytes = BM * BK;              // 32 KiB
constexpr int kTileBBytes = BN * BK;              // 32 KiB
constexpr int kScaleBytes = (BM + BN) * 4;        // 2 KiB
constexpr int kStageBytes = kTileABytes + kTileBBytes + kScaleBytes;
constexpr int kEpiRowBytes = WN * 2 + 8;            // bf16 row of a wave tile, padded
constexpr int kEpiSlotBytes = WM * kEpiRowBytes;    // one wave's output tile
static_assert(4 * kEpiSlotBytes <= kStageBytes, "four epilogue slots per stage");
constexpr int kGroupM = 4;  // tile-order grouping along M (4 measured 2 % faster than 8 or 16)
constexpr int kXcds = 8;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format

typedef __attribute__((address_space(3))) v2i lds_v2i;
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// Work units of one launch.  Logical tiles [0, full) run over all of K and
// store bf16; every remaining tile is split into `splits` contiguous ranges
// of K blocks whose fp32 sums go to part[split][row - row0][ldp] (row0 =
// 256 trow0, the first row of the split tiles; ldp = N rounded up to 4), summed in
// split order by splitk_reduce_kernel.  Unit ids: [0, full) the whole
// tiles, then one segment of (tiles - full) ids per split.  With full a
// whole number of waves of workgroups, the split units are only the tiles
// that would leave the last wave under-filled.  full is a multiple of the
// tile walk's row groups, so the split tiles are whole rows of tiles.
struct UnitPlan {
  int tiles_m, tiles_n;
  int full;     // whole tiles (logical order); the rest are split
  int splits;   // K ranges per split tile (1: nothing is split), at most 8
  int piece;    // K blocks per range (splits * piece = K / 128)
  int trow0;    // first row of split tiles: full / tiles_n
  float* part;  // fp32 partials of the split tiles
};

// Offset (elements) of output row m in split `sp`'s partials.
__device__ __forceinline__ int64_t partial_row(const UnitPlan& p, int sp, int64_t m, int64_t M,
                                               int64_t ldp) {
  const int64_t row0 = static_cast<int64_t>(p.trow0) * BM;
  return (sp * (M - row0) + (m - row0)) * ldp;
}

// Logical index of the j-th id of a segment of n consecutive block ids:
// the hardware deals consecutive ids to the 8 XCDs round robin, so ids j
// with the same j % 8 run on one XCD; this gives each of those classes a
// contiguous range of logical indices.
__device__ __forceinline__ int undeal(int j, int n) {
  const int q = n / kXcds, r = n % kXcds;
  const int rank = j % kXcds, local = j / kXcds;
  return rank < r ? rank * (q + 1) + local : r * (q + 1) + (rank - r) * q + local;
}

// Tile of a logical index: tiles are walked in column-major groups of
// kGroupM rows, so concurrent tiles of an XCD share A rows and B columns.
__device__ __forceinline__ void tile_walk(int logical, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int per_group = kGroupM * tiles_n;
  const int group = logical / per_group;
  const int first_m = group * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int in_group = logical - group * per_group;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

// Tile and K-block range of unit u; returns its split (-1: a whole tile).
__device__ __forceinline__ int plan_unit(const UnitPlan& p, int u, int KB, int& tm, int& tn,
                                         int& kb0, int& kb1) {
  int logical, sp;
  if (u < p.full) {
    logical = undeal(u, p.full);
    sp = -1;
    kb0 = 0;
    kb1 = KB;
  } else {
    // split s is the id segment [full + s * rest, full + (s + 1) * rest)
    const int rest = p.tiles_m * p.tiles_n - p.full;
    int w = u - p.full;
    sp = 0;
#pragma unroll
    for (int s = 1; s < 8; ++s)  // no integer division: at most 8 splits
      if (w >= rest) {
        w -= rest;
        ++sp;
      }
    logical = p.full + undeal(w, rest);
    kb0 = sp * p.piece;
    kb1 = kb0 + p.piece;
  }
  tile_walk(logical, p.tiles_m, p.tiles_n, tm, tn);
  return sp;
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor (wave-uniform): base address, stride 0, `bytes`
// records (accesses at or past the end read as zero instead of faulting).
__device__ __forceinline__ i32x4 make_rsrc(const void* base, int64_t bytes) {
  const int64_t cap = 0x7FFFFFFF;
  const int n = static_cast<int>(bytes < 0 ? 0 : (bytes > cap ? cap : bytes));
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r.x = __builtin_amdgcn_readfirstlane(static_cast<int>(a & 0xFFFFFFFFu));
  r.y = __builtin_amdgcn_readfirstlane(static_cast<int>((a >> 32) & 0xFFFFu));
  r.z = __builtin_amdgcn_readfirstlane(n);
  r.w = kRsrcWord3;
  return r;
}

// Descriptor of base + kb * stride with a precomputed (wave-uniform) extent.
__device__ __forceinline__ i32x4 advanced_rsrc(uint64_t base, int64_t kb, int64_t stride, int ext) {
  const uint64_t a = base + static_cast<uint64_t>(kb) * static_cast<uint64_t>(stride);
  i32x4 r;
  r.x = __builtin_amdgcn_readfirstlane(static_cast<int>(a & 0xFFFFFFFFu));
  r.y = __builtin_amdgcn_readfirstlane(static_cast<int>((a >> 32) & 0xFFFFu));
  r.z = ext;
  r.w = kRsrcWord3;
  return r;
}

// Asynchronous buffer -> LDS copies (16 or 4 bytes per lane, the 64 lanes
// landing contiguously at LDS byte address `lds` + OFF).  They are issued
// from inline asm so the compiler does not treat them as stores that may
// alias every later LDS read: it would otherwise wait for the copy into one
// stage before reading fragments of the other.  Completion is awaited
// explicitly (s_waitcnt vmcnt(0) before the barrier that publishes a stage).
// The asm has no result registers; its inputs are read when it issues.  The
// s_nop covers the wait state an LDS-DMA load needs after an SALU write of
// M0.  The instruction's immediate offset OFF moves both the LDS
// destination and the memory address (so the caller passes voff - OFF); it
// lets the four 1 KiB copies of a wave share one M0 value instead of an
// SALU add each.
template <int OFF>
__device__ __forceinline__ void copy16_to_lds(uint32_t lds, uint32_t voff, i32x4 rsrc) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen offset:%3 lds"
               :
               : "s"(lds), "v"(voff), "s"(rsrc), "i"(OFF)
               : "memory", "m0");
}
__device__ __forceinline__ void copy4_to_lds(uint32_t lds, uint32_t voff, i32x4 rsrc) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// 16 bytes from an LDS address that is only 8-byte aligned (an epilogue row
// of a padded staging slot), as two 8-byte reads: a 16-byte read from such
// an address stalls the LDS for extra cycles.
__device__ __forceinline__ v4u lds_read16_a8(const uint8_t* p) {
  const uint2 lo = *reinterpret_cast<const uint2*>(p);
  const uint2 hi = *reinterpret_cast<const uint2*>(p + 8);
  return v4u{lo.x, lo.y, hi.x, hi.y};
}

// 16-byte chunk swizzle of a K-major LDS tile row k (256 B per row): the
// low three bits spread the 8 rows one tr8 read touches over 8 chunks, the
// fourth bit moves lane groups g and g+1 (k differs by 16) to different
// halves of the row.
__device__ __forceinline__ int kmajor_swizzle(int k) { return (k & 7) | (((k >> 4) & 1) << 3); }

// Per-operand loader/reader.  KMAJOR == false: stored [rows][K] (K
// contiguous); KMAJOR == true: stored [K][rows].  `rows` is M for A, N for B.
template <bool KMAJOR, int NP = 4>
struct Operand {
  uint64_t base;        // address of the tile's first row (K-contig) / first column (K-major)
  int64_t kstride;      // bytes between the starts of consecutive K blocks
  int ext;              // descriptor extent, the same for every K block
  uint32_t voff[NP];    // per-lane byte offsets of the wave's NP 1 KiB copies

  __device__ __forceinline__ void init(const uint8_t* p, int64_t ld_, int64_t r0, int64_t rows,
                                       int64_t K_, int wave, int lane) {
    (void)K_;
    rebase(p, ld_, r0, rows);
    kstride = KMAJOR ? BK * ld_ : BK;
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      if (!KMAJOR) {
        // LDS [256 rows][128 B]; copy (wave*NP+j) fills rows 8(wave*NP+j)..+7
        const int row = (wave * NP + j) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ (row & 7);
        voff[j] = static_cast<uint32_t>(row * ld_ + c * 16);
      } else {
        // LDS [128 k][256 B]; copy (wave*NP+j) fills k rows 4(wave*NP+j)..+3
        const int k = (wave * NP + j) * 4 + (lane >> 4);
        const int c = (lane & 15) ^ kmajor_swizzle(k);
        voff[j] = static_cast<uint32_t>(k * ld_ + c * 16);
      }
    }
  }

  // The tile-dependent part: base and extent of the tile whose rows (or
  // columns) start at r0 (the per-lane offsets do not depend on the tile).
  // Extent from the start of a K block.  K-contiguous: up to the end of that
  // block's part of the last valid row, so every copy of a row past the
  // valid ones (offset >= valid rows * ld) reads zeros.  K-major: the
  // block's 128 k rows, a ragged last column chunk read up to the next
  // 16-byte boundary, which the padded leading dimension covers.
  __device__ __forceinline__ void rebase(const uint8_t* p, int64_t ld_, int64_t r0, int64_t rows) {
    const int64_t rows_left = rows - r0;  // valid rows (or columns) from the tile start
    base = reinterpret_cast<uint64_t>(KMAJOR ? p + r0 : p + r0 * ld_);
    int64_t e;
    if (!KMAJOR) {
      const int64_t rv = rows_left > 256 ? 256 : rows_left;
      e = (rv - 1) * ld_ + BK;
    } else {
      const int64_t cols = rows_left > 256 ? 256 : ((rows_left + 15) & ~int64_t(15));
      e = (BK - 1) * ld_ + cols;
    }
    ext = __builtin_amdgcn_readfirstlane(static_cast<int>(e > 0x7FFFFFFF ? 0x7FFFFFFF : e));
  }

  // Buffer descriptor of K block kb: its first byte and the constant
  // extent.  Computed once per K block (a 64-bit scalar add); the four
  // copies of a wave then only differ in their offsets.
  __device__ __forceinline__ i32x4 block_rsrc(int64_t kb) const {
    return advanced_rsrc(base, kb, kstride, ext);
  }

  // Copy 1 KiB piece j (0..NP-1) of this wave's share of the K block
  // described by `r` into the LDS tile at `dst`.  Copies 4q..4q+3 share the
  // M0 value lbase + 4 KiB * q (the immediate offset field holds at most
  // 4095).
  __device__ __forceinline__ void load_piece(const i32x4& r, uint8_t* dst, int wave, int j) const {
    const uint32_t lbase =
        __builtin_amdgcn_readfirstlane(lds_addr(dst) + wave * NP * 1024 + (j >> 2) * 4096);
    const int jj = j & 3;
    if (jj == 0) copy16_to_lds<0>(lbase, voff[j], r);
    else if (jj == 1) copy16_to_lds<1024>(lbase, voff[j] - 1024u, r);
    else if (jj == 2) copy16_to_lds<2048>(lbase, voff[j] - 2048u, r);
    else copy16_to_lds<3072>(lbase, voff[j] - 3072u, r);
  }

  // Fragment of 16 rows starting at tile row `r0` (multiple of 16): 32 bytes
  // per lane; lane group g = lane/16 holds K bytes [16g, 16g+16) followed by
  // [64+16g, 64+16g+16) for both operands.  This is also the K order the
  // scaled MFMA assumes when it applies one scale per 32-deep K chunk (see
  // the file comment).  With this split the four lane groups of one
  // ds_read_b128 touch four adjacent 16-byte chunks of their rows, which the
  // LDS serves without bank conflicts; reading chunks 2g and 2g+1 instead
  // halves the read rate.
  __device__ __forceinline__ v8i frag(const uint8_t* tile, int r0, int lane) const {
    const int g = lane >> 4, q = lane & 15;
    if (!KMAJOR) {
      const int row = r0 + q;
      const uint8_t* p = tile + row * BK;
      const uint4 lo = *reinterpret_cast<const uint4*>(p + ((g ^ (row & 7)) << 4));
      const uint4 hi = *reinterpret_cast<const uint4*>(p + (((g + 4) ^ (row & 7)) << 4));
      return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                 (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    } else {
      // ds_read_b64_tr_b8: within each 16-lane group, lane pair (2r, 2r+1)
      // supplies the two 8-byte halves of one 16-byte row segment (row r of
      // 8) and lane c receives byte c of all 8 rows.  Here the 8 rows are
      // consecutive k and the segment holds columns r0..r0+15, so lane q gets
      // 8 consecutive K bytes of column r0+q.  Rows read: k = 16g + 8t' + r
      // for the first 16 bytes and 64 + 16g + 8t' + r for the last 16.
      const int kr = 16 * g + (q >> 1);
      const int cx = (r0 >> 4);
      const uint8_t* p0 = tile + kr * 256 + ((q & 1) << 3);
      const uint8_t* p1 = p0 + 8 * 256;
      const uint8_t* p2 = p0 + 64 * 256;
      const uint8_t* p3 = p0 + 72 * 256;
      // all four row sets have k & 7 == q/2 and (k >> 4) & 1 == g & 1
      const int ph = (cx ^ kmajor_swizzle(kr)) << 4;
      const v2i t0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(p0 + ph));
      const v2i t1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(p1 + ph));
      const v2i t2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(p2 + ph));
      const v2i t3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(p3 + ph));
      return v8i{t0.x, t0.y, t1.x, t1.y, t2.x, t2.y, t3.x, t3.y};
    }
  }
};

// E8M0 scale staging: for each of 256 consecutive rows (A) or columns (B),
// the aligned 32-bit word holding its scale byte(s) for K block kb goes to
// one LDS word (the reader picks the byte: `mx_byte_index`).  MODE 0: 1x128
// groups, one byte per row; MODE 2: 1x32 groups ([rows][K/32], K-contiguous
// only), the word holds the 4 bytes of the block's 32-groups; MODE 1:
// 128x128 blocks, lanes 0 and 1 fetch the two blocks the tile spans.  The
// scale tensor is read up to its size rounded up to 4 bytes.
template <bool KMAJOR, int MODE>
__device__ __forceinline__ int64_t mx_scale_index(int64_t r, int64_t rows, int64_t nblk,
                                                  int64_t KB, int64_t kb) {
  if (MODE == 1) return KMAJOR ? kb * nblk + r : r * KB + kb;  // r: block index
  if (MODE == 2) return r * KB * 4 + kb * 4;
  return KMAJOR ? kb * rows + r : r * KB + kb;
}
template <bool KMAJOR, int MODE>
__device__ __forceinline__ void load_mx_scales(const uint8_t* s, int64_t r0, int64_t rows,
                                               int64_t nblk, int64_t KB, int64_t kb, uint8_t* dst,
                                               int sub, int lane) {
  int64_t r;
  if (MODE == 1) {
    r = r0 / 128 + (lane < 2 ? lane : 0);
    if (r > nblk - 1) r = nblk - 1;
  } else {
    r = r0 + sub * 64 + lane;
    if (r > rows - 1) r = rows - 1;
  }
  const int64_t idx = mx_scale_index<KMAJOR, MODE>(r, rows, nblk, KB, kb);
  const int64_t bytes = MODE == 1 ? nblk * KB : (MODE == 2 ? rows * KB * 4 : rows * KB);
  copy4_to_lds(__builtin_amdgcn_readfirstlane(lds_addr(dst) + sub * 256),
               static_cast<uint32_t>(idx & ~int64_t(3)), make_rsrc(s, (bytes + 3) & ~int64_t(3)));
}

// K-block-major 1x128 scale bytes of 256 consecutive rows starting at byte
// `first` of the `bytes`-byte tensor: wave `sub` copies words [64 sub,
// 64 sub + 64) counted from the aligned word holding byte `first`, so the
// tile's bytes sit at LDS offsets (first & 3) .. (first & 3) + 255 (words
// past the tensor's end read as zero).
__device__ __forceinline__ void load_mx_scale_bytes(const uint8_t* s, int64_t bytes, int64_t first,
                                                    uint8_t* dst, int sub, int lane) {
  const int64_t off = (first & ~int64_t(3)) + 4 * (64 * sub + lane);
  copy4_to_lds(__builtin_amdgcn_readfirstlane(lds_addr(dst) + sub * 256), static_cast<uint32_t>(off),
               make_rsrc(s, (bytes + 3) & ~int64_t(3)));
}

template <bool A_KM, bool B_KM, int MODE_A, int MODE_B, int BNT>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(2, 2))) void
gemm_kernel(const uint8_t* __restrict__ A, int64_t lda, const void* __restrict__ sA_,
            const uint8_t* __restrict__ B, int64_t ldb, const void* __restrict__ sB_,
            uint16_t* __restrict__ C, int64_t ldc, int64_t M, int64_t N, int64_t K,
            const UnitPlan plan) {
  // BNT: output columns per tile, 256, or 192 (wave tile 64 x 96) for
  // K-contiguous B with 1x128 scales, whose 192 rows of B fill the copy
  // pieces of 8 waves evenly and whose scales are per column (a wave's 96
  // columns may straddle two 128-column weight blocks)
  static_assert(BNT == 256 || (BNT == 192 && !B_KM && (MODE_B == 0 || MODE_B == 3)),
                "192-column tiles: K-contiguous B with 1x128 scales");
  constexpr int WNT = BNT / kWavesN;          // 128 or 96
  constexpr int TNT = WNT / 16;               // 8 or 6 column subtiles
  constexpr int kTileBBytesT = BNT * BK;      // 32 or 24 KiB
  constexpr int kStageBytesT = kTileABytes + kTileBBytesT + kScaleBytes;
  constexpr int kEpiRowBytesT = WNT * 2 + 8;  // bf16 row of a wave tile, padded
  constexpr int kEpiSlotBytesT = WM * kEpiRowBytesT;
  static_assert(4 * kEpiSlotBytesT <= kStageBytesT, "four epilogue slots per stage");
  constexpr int kPiecesB = BNT / 64;          // 1 KiB copies of B per wave and K block
  const float* __restrict__ sA = static_cast<const float*>(sA_);
  const float* __restrict__ sB = static_cast<const float*>(sB_);
  // MODE 3: 1x128 groups like MODE 0, with the scale tensor stored K-block
  // major ([K/128][rows]) whatever the code orientation
  constexpr int MA = MODE_A == 3 ? 0 : MODE_A, MB = MODE_B == 3 ? 0 : MODE_B;
  constexpr bool SKA = A_KM || MODE_A == 3, SKB = B_KM || MODE_B == 3;
  // Two pipeline stages; block kb lives in stage kb % 2.
  __shared__ __attribute__((aligned(1024))) uint8_t stage0[kStageBytesT];
  __shared__ __attribute__((aligned(1024))) uint8_t stage1[kStageBytesT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % kWavesM;
  const int wn = wave / kWavesM;
  const int g = lane >> 4, r16 = lane & 15;

  const int64_t KB = K / BK;
  const int64_t MBk = (M + 127) / 128, NBk = (N + 127) / 128;
  // this workgroup's unit: a tile and a range of its K blocks; a split
  // unit's fp32 sum goes to part[split] and a second kernel sums the splits
  // in order
  int tm, tn, kb_begin, kb_end;
  const int split = plan_unit(plan, blockIdx.x, static_cast<int>(KB), tm, tn, kb_begin, kb_end);
  const int64_t m0 = static_cast<int64_t>(tm) * BM;
  const int64_t n0 = static_cast<int64_t>(tn) * BNT;

  Operand<A_KM> opa;
  Operand<B_KM, kPiecesB> opb;
  opa.init(A, lda, m0, M, K, wave, lane);
  opb.init(B, ldb, n0, N, K, wave, lane);

  // The copy of one K block is split into 9 pieces per wave (4 x 1 KiB of
  // A, 4 x 1 KiB of B -- 3 for 192-column tiles -- and one dword per lane of
  // act-mode scales) so the pieces can be spread over the MFMA issue slots
  // of the block before.
  constexpr int kLoadPieces = 4 + kPiecesB + 1;
  i32x4 rsrc_a, rsrc_b;  // descriptors of the K block being copied

  // float32 scales: the one dword-per-lane copy this wave makes per K block
  // (waves 0-3 stage A's scales, waves 4-7 B's; for 128x128 block scales
  // only the first wave of each half copies the two blocks the tile spans),
  // as a descriptor advanced by a fixed stride per K block.  Rows past the
  // end are clamped to the last valid one (their products are never stored).
  bool sc_active = false;
  uint64_t sc_base = 0;
  int64_t sc_stride = 0;
  int sc_ext = 0;
  uint32_t sc_voff = 0, sc_lds = 0;
  {
    const bool b_side = wave >= 4;
    const int sub = wave & 3;
    const int mode = b_side ? MB : MA;
    const bool km = b_side ? SKB : SKA;
    const float* sp = b_side ? sB : sA;
    const int64_t r0 = b_side ? n0 : m0, rows = b_side ? N : M, nblk = b_side ? NBk : MBk;
    sc_lds = (b_side ? 1024u : 0u) + (mode == 0 ? static_cast<uint32_t>(sub) * 256u : 0u);
    sc_active = mode == 0 || sub == 0;
    const float* b;
    int64_t e;
    if (mode == 0) {
      int64_t r = sub * 64 + lane;
      if (r > rows - r0 - 1) r = rows - r0 - 1;
      if (!km) {  // scales [rows][KB]
        b = sp + r0 * KB;
        sc_voff = static_cast<uint32_t>(r * KB * 4);
        sc_stride = 4;
        e = ((rows - r0 - 1) * KB + 1) * 4;
      } else {    // scales [KB][rows]
        b = sp + r0;
        sc_voff = static_cast<uint32_t>(r * 4);
        sc_stride = rows * 4;
        e = (rows - r0) * 4;
      }
    } else {
      int64_t blk = r0 / 128 + (lane < 2 ? lane : 0);
      if (blk > nblk - 1) blk = nblk - 1;
      b = sp;
      if (!km) {  // scales [nblk][KB]
        sc_voff = static_cast<uint32_t>(blk * KB * 4);
        sc_stride = 4;
      } else {    // scales [KB][nblk]
        sc_voff = static_cast<uint32_t>(blk * 4);
        sc_stride = nblk * 4;
      }
      e = nblk * KB * 4;
    }
    sc_base = reinterpret_cast<uint64_t>(b);
    sc_ext = __builtin_amdgcn_readfirstlane(static_cast<int>(e > 0x7FFFFFFF ? 0x7FFFFFFF : e));
  }
  auto issue_piece = [&](int64_t kb, uint8_t* st, int piece) {
    if (piece < 4) {
      opa.load_piece(rsrc_a, st, wave, piece);
    } else if (piece < 4 + kPiecesB) {
      opb.load_piece(rsrc_b, st + kTileABytes, wave, piece - 4);
    } else {
      uint8_t* sdst = st + kTileABytes + kTileBBytesT;
      if (sc_active) {
        copy4_to_lds(__builtin_amdgcn_readfirstlane(lds_addr(sdst) + sc_lds), sc_voff,
                     advanced_rsrc(sc_base, kb, sc_stride, sc_ext));
      }
    }
  };
  auto issue_loads = [&](int64_t kb, uint8_t* st) {
    rsrc_a = opa.block_rsrc(kb);
    rsrc_b = opb.block_rsrc(kb);
#pragma unroll
    for (int p = 0; p < kLoadPieces; ++p) issue_piece(kb, st, p);
  };

  // per-row multipliers of one K block: sA (act) or sA_blk, times sB_blk
  // (a wave's 64 rows / 128 columns sit in one 128-block); every scale
  // comes from the K block's LDS stage, copied with its codes
  auto row_mults = [&](const uint8_t* st, float (&ra)[TM]) {
    const float* s_lds = reinterpret_cast<const float*>(st + kTileABytes + kTileBBytesT);
    const float sb = MB == 1 ? s_lds[BM + wn] : 1.0f;
    if (MA == 0) {
#pragma unroll
      for (int i = 0; i < TM; ++i) ra[i] = s_lds[wm * WM + 16 * i + r16] * sb;
    } else {
      const float sa = s_lds[(wm * WM) / 128] * sb;
#pragma unroll
      for (int i = 0; i < TM; ++i) ra[i] = sa;
    }
  };
  auto col_mults = [&](const uint8_t* st, int j, float (&cb)[4]) {
    if (MB == 0) {
      const float* s_lds = reinterpret_cast<const float*>(st + kTileABytes + kTileBBytesT);
      const float4 v = *reinterpret_cast<const float4*>(s_lds + BM + wn * WNT + 16 * j + 4 * g);
      cb[0] = v.x; cb[1] = v.y; cb[2] = v.z; cb[3] = v.w;
    }
  };

  v4f acc[TM][TNT];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TNT; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // Promotion of one 16x16 partial: acc += P * (row multiplier * column
  // multiplier).  The partial of subtile (i, j) is promoted right after the
  // MFMA of the next subtile is issued, so the VALU work of one subtile hides
  // under the matrix-core time of the next.
  // The empty asm pins each updated accumulator at this point of the
  // program: without it the optimizer sinks all promotions below the K
  // block's last MFMA, which keeps every partial live at once.
  auto promote = [&](v4f& a, const v4f& p, float rmul, const float (&cm)[4]) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float x = a[r];
      x = fmaf(p[r], MB == 0 ? rmul * cm[r] : rmul, x);
      asm volatile("" : "+v"(x));
      a[r] = x;
    }
  };

  // ---- prologue -----------------------------------------------------------
  issue_loads(kb_begin, stage0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();

  v8i af[TM];
  v8i bq;
  float ra[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) af[i] = opa.frag(stage0, wm * WM + 16 * i, lane);
  bq = opb.frag(stage0 + kTileABytes, wn * WNT, lane);
  row_mults(stage0, ra);

  // Partials are promoted kLag MFMAs behind their issue (subtile order
  // t = j*TM + i), so the VALU never waits on a result still in the matrix
  // pipe; the last kLag partials of a K block are promoted after the barrier.
  constexpr int kLag = 3;
  v4f pend[kLag];
#pragma unroll
  for (int q = 0; q < kLag; ++q) pend[q] = v4f{0.f, 0.f, 0.f, 0.f};
  float cm_cur[4] = {1.f, 1.f, 1.f, 1.f}, cm_prev[4] = {1.f, 1.f, 1.f, 1.f};
  float ra_last[TM];

  // One K block computed from `cur` while the copy of block kb+1 into `nxt`
  // (free since the previous barrier) is issued piecewise between the MFMAs
  // of the block's first half; then, once every wave's copies have landed,
  // the fragments of block kb+1 are read from `nxt`.
  auto kblock = [&](int64_t kb, const uint8_t* cur, uint8_t* nxt) {
    const bool more = kb + 1 < kb_end;
    // The copies are issued unconditionally (no branch per piece): after the
    // last block they read nothing (an empty descriptor makes every access
    // out of range, which lands zeros in the idle stage) and the scale copies
    // repeat this block's scales.
    const int64_t kn = more ? kb + 1 : kb;
    rsrc_a = opa.block_rsrc(kn);
    rsrc_b = opb.block_rsrc(kn);
    if (!more) {
      rsrc_a.z = 0;
      rsrc_b.z = 0;
    }
#pragma unroll
    for (int j = 0; j < TNT; ++j) {
      v8i bn = bq;
      if (j + 1 < TNT) bn = opb.frag(cur + kTileABytes, wn * WNT + 16 * (j + 1), lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) cm_prev[r] = cm_cur[r];
      col_mults(cur, j, cm_cur);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int t = j * TM + i;
        // zero scales (E8M0 bytes 0 are ignored): the unscaled instruction
        const v4f pc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            bq, af[i], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
        if (t >= kLag) {
          const int i2 = (t - kLag) % TM, j2 = (t - kLag) / TM;
          promote(acc[i2][j2], pend[t % kLag], ra[i2], j2 == j ? cm_cur : cm_prev);
        }
        pend[t % kLag] = pc;
        // one copy piece every second MFMA slot (t = 1, 3, ..., 17): denser
        // issue bunches the copies' LDS writes, sparser issue leaves too
        // little time before the end-of-block wait (both measured slower)
        if (t >= 1 && (t - 1) % 2 == 0 && (t - 1) / 2 < kLoadPieces) issue_piece(kn, nxt, (t - 1) / 2);
        // one MFMA and the promotion of the partial kLag issues back per
        // scheduling region: the machine scheduler would otherwise pull each
        // promotion up against the MFMA that produces it and stall on it
        __builtin_amdgcn_sched_barrier(0);
      }
      bq = bn;
    }
    // all MFMAs of this K block are issued; the last kLag subtiles (all in
    // column TNT-1) are pending with this block's multipliers
#pragma unroll
    for (int i = 0; i < TM; ++i) ra_last[i] = ra[i];
    if (more) {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // this wave's copies of block kb+1 landed
      __syncthreads();                     // everyone's did, and `cur` is free
      // B fragment and A row 0 first: the next block's first MFMA needs
      // only those two
      bq = opb.frag(nxt + kTileABytes, wn * WNT, lane);
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = opa.frag(nxt, wm * WM + 16 * i, lane);
      row_mults(nxt, ra);
    }
#pragma unroll
    for (int q = 0; q < kLag; ++q) {
      const int t = TM * TNT - kLag + q;
      promote(acc[t % TM][TNT - 1], pend[t % kLag], ra_last[t % TM], cm_cur);
    }
  };

  for (int kb = kb_begin; kb < kb_end; kb += 2) {
    kblock(kb, stage0, stage1);
    if (kb + 1 < kb_end) kblock(kb + 1, stage1, stage0);
  }

  // the copies issued during the last block must land before the stages
  // are reused for the output
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  if (split >= 0) {
    // split-K partial: 4 consecutive fp32 columns per lane, 16-byte stores
    const int64_t ldp = (N + 3) & ~int64_t(3);
    float* pbase = plan.part + partial_row(plan, split, m0, M, ldp);
    if (m0 + wm * WM + WM <= M && n0 + wn * WNT + WNT <= N) {
      float* dst = pbase + (wm * WM + r16) * ldp + n0 + wn * WNT + 4 * g;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TNT; ++j)
          *reinterpret_cast<v4f*>(dst + 16 * i * ldp + 16 * j) = acc[i][j];
      return;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int64_t m = m0 + wm * WM + 16 * i + r16;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < TNT; ++j) {
        const int64_t n = n0 + wn * WNT + 16 * j + 4 * g;
        if (n < N) {
          float* dst = pbase + (m - m0) * ldp + n;
#pragma unroll
          for (int r = 0; r < 4; ++r) dst[r] = acc[i][j][r];
        }
      }
    }
    return;
  }

  // ---- epilogue: bf16 RNE, staged through LDS so that global stores write
  // whole 128-byte lines: each wave parks its 64 x 128 bf16 tile in its own
  // LDS slot (rows padded to 264 B), then 16 lanes store one 256-byte row.
  // The stores are non-temporal: the output is not read again by this
  // kernel, and keeping it out of L2 leaves the operand tiles other
  // workgroups still stream there.
  __syncthreads();  // every wave is done reading both stages
  uint8_t* slot = (wave < 4 ? stage0 : stage1) + (wave & 3) * kEpiSlotBytesT;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TNT; ++j) {
      *reinterpret_cast<uint2*>(slot + (16 * i + r16) * kEpiRowBytesT + (16 * j + 4 * g) * 2) =
          make_uint2(pack_bf16x2(acc[i][j][0], acc[i][j][1]),
                     pack_bf16x2(acc[i][j][2], acc[i][j][3]));
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's slot is written
  __builtin_amdgcn_wave_barrier();
  const int64_t mw = m0 + wm * WM, nw = n0 + wn * WNT;
  const int chunk = lane & 15;  // 8 bf16 columns
  // a 96-column wave tile has 12 chunks per row: lanes 12..15 of each row idle
  const bool chunk_ok = WNT == 128 || chunk < WNT / 8;
  if (mw + WM <= M && nw + WNT <= N) {
    // whole wave tile inside C: all row reads first, then the stores, with
    // no per-row tests (a read-then-test loop waits out the LDS latency
    // once per row)
    v4u v[WM / 4];
#pragma unroll
    for (int u = 0; u < WM / 4; ++u)
      v[u] = lds_read16_a8(slot + (4 * u + (lane >> 4)) * kEpiRowBytesT + chunk * 16);
    uint16_t* dst = C + (mw + (lane >> 4)) * ldc + nw + chunk * 8;
    if (chunk_ok) {
#pragma unroll
      for (int u = 0; u < WM / 4; ++u)
        __builtin_nontemporal_store(v[u], reinterpret_cast<v4u*>(dst + 4 * u * ldc));
    }
    return;
  }
#pragma unroll
  for (int u = 0; u < WM / 4; ++u) {
    const int row = 4 * u + (lane >> 4);
    const v4u v = lds_read16_a8(slot + row * kEpiRowBytesT + chunk * 16);
    const int64_t m = mw + row, n = nw + chunk * 8;
    if (m >= M || !chunk_ok) continue;
    uint16_t* dst = C + m * ldc + n;
    if (n + 7 < N) {
      __builtin_nontemporal_store(v4u{v.x, v.y, v.z, v.w}, reinterpret_cast<v4u*>(dst));
    } else if (n < N) {
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      for (int e = 0; e < 8 && n + e < N; ++e)
        dst[e] = static_cast<uint16_t>((w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
    }
  }
}

// ---------------------------------------------------------------------------
// Power-of-two (E8M0) scales, four waves: the same 256x256x128 tile and LDS
// stages as gemm_kernel, but 4 waves (one per SIMD) with a 128x128 share
// each (8 x 8 subtiles).  Without the float32 promotion nothing has to run
// on the VALU per K block, so the 256 accumulators per lane live in the
// AGPR file as the scaled MFMA's C operand, and the larger wave tile reads
// 128 KiB of fragments from LDS per K block instead of 192 KiB.  With one
// wave per SIMD nothing else covers the barrier at the end of a K block:
// the last column's eight MFMAs are issued after it, from registers, while
// the next block's fragments are read into the registers they free.
// ---------------------------------------------------------------------------
constexpr int k4Threads = 256;
constexpr int W4M = 128, W4N = 128;  // wave tile, 2 x 2 waves
constexpr int T4M = W4M / 16, T4N = W4N / 16;
constexpr int k4EpiRowBytes = W4N * 2 + 8;  // padded bf16 row of a wave tile
static_assert(4 * (W4M / 2) * k4EpiRowBytes <= kStageBytes, "four half-tile epilogue slots per stage");

template <bool A_KM, bool B_KM, int MODE_A, int MODE_B>
__global__ __attribute__((amdgpu_flat_work_group_size(k4Threads, k4Threads),
                          amdgpu_waves_per_eu(1, 1))) void
gemm_mx4_kernel(const uint8_t* __restrict__ A, int64_t lda, const void* __restrict__ sA_,
                const uint8_t* __restrict__ B, int64_t ldb, const void* __restrict__ sB_,
                uint16_t* __restrict__ C, int64_t ldc, int64_t M, int64_t N, int64_t K, int tiles_m,
                int tiles_n, int splits, float* __restrict__ part, int64_t ldp, int64_t pstride) {
  const uint8_t* __restrict__ eA = static_cast<const uint8_t*>(sA_);
  const uint8_t* __restrict__ eB = static_cast<const uint8_t*>(sB_);
  // MODE 3: 1x128 groups, scale bytes stored K-block major ([K/128][rows])
  constexpr int MA = MODE_A == 3 ? 0 : MODE_A, MB = MODE_B == 3 ? 0 : MODE_B;
  constexpr bool SKA = A_KM || MODE_A == 3, SKB = B_KM || MODE_B == 3;
  __shared__ __attribute__((aligned(1024))) uint8_t stage0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t stage1[kStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int g = lane >> 4, r16 = lane & 15;

  const int64_t KB = K / BK;
  const int64_t MBk = (M + 127) / 128, NBk = (N + 127) / 128;
  // Persistent: this workgroup runs the work units blockIdx.x, blockIdx.x +
  // gridDim.x, ... (a unit: one 256x256 output tile and one split-K range of
  // its K blocks; units tiles .. 2 tiles - 1 are split 1, and so on: every
  // tile is split alike, so the unit decode stays a few scalar operations
  // in a kernel that uses its whole register file).  The
  // last K block of a unit copies the next unit's first block, and the
  // output of a unit is stored while those copies land, so neither the
  // copy latency of a tile's first block nor a new workgroup's start sits
  // between two tiles.  The grid is a multiple of the 8 XCDs, so every unit
  // of a workgroup maps to the XCD it runs on.
  const int tiles = tiles_m * tiles_n;
  const int units = tiles * splits;
  auto unit_tile = [&](int v, int64_t& um0, int64_t& un0, int& ukb0, int& ukb1) {
    const int sp = v / tiles;
    int tm, tn;
    tile_walk(undeal(v - sp * tiles, tiles), tiles_m, tiles_n, tm, tn);
    um0 = static_cast<int64_t>(tm) * BM;
    un0 = static_cast<int64_t>(tn) * BN;
    ukb0 = static_cast<int>((sp * static_cast<int>(KB)) / splits);
    ukb1 = static_cast<int>(((sp + 1) * static_cast<int>(KB)) / splits);
    return sp;
  };

  // ---- per-unit state ---------------------------------------------------------
  int v = blockIdx.x;
  int64_t m0, n0;
  int kb_begin, kb_end;
  int split = unit_tile(v, m0, n0, kb_begin, kb_end);
  Operand<A_KM, 8> opa;
  Operand<B_KM, 8> opb;
  opa.init(A, lda, m0, M, K, wave, lane);
  opb.init(B, ldb, n0, N, K, wave, lane);
  // the unit whose first K block the current unit's last block copies
  int64_t xm0 = 0, xn0 = 0;
  int xkb0 = 0, xkb1 = 0;
  bool has_next = false;
  uint64_t xbase_a = 0, xbase_b = 0;
  int xext_a = 0, xext_b = 0;
  auto peek_next = [&]() {
    const int vn = v + static_cast<int>(gridDim.x);
    has_next = vn < units;
    if (has_next) {
      unit_tile(vn, xm0, xn0, xkb0, xkb1);
      Operand<A_KM, 8> xa = opa;
      Operand<B_KM, 8> xb = opb;
      xa.rebase(A, lda, xm0, M);
      xb.rebase(B, ldb, xn0, N);
      xbase_a = xa.base;
      xext_a = xa.ext;
      xbase_b = xb.base;
      xext_b = xb.ext;
    }
  };
  peek_next();

  // The copy of one K block: 8 x 1 KiB of A, 8 x 1 KiB of B and the scale
  // words of 64 rows of A and 64 columns of B per wave.  K-block-major 1x128
  // scales (kBytes*) are copied as the bytes themselves: the tile's 256
  // consecutive bytes of block kb, from the aligned word at or before the
  // first, so a lane reads its row's byte with one ds_read_u8 and passes it
  // to the MFMA as is.  cm0 / cn0: the tile the block belongs to.
  constexpr int kPieces = 18;
  constexpr bool kBytesA = SKA && MA == 0, kBytesB = SKB && MB == 0;
  i32x4 rsrc_a, rsrc_b;
  auto issue_piece = [&](int64_t kb, uint8_t* st, int piece, int64_t cm0, int64_t cn0) {
    if (piece < 8) {
      opa.load_piece(rsrc_a, st, wave, piece);
    } else if (piece < 16) {
      opb.load_piece(rsrc_b, st + kTileABytes, wave, piece - 8);
    } else {
      uint8_t* sdst = st + kTileABytes + kTileBBytes;
      // every wave copies (for 128x128 blocks the copies of waves 1-3 land
      // beside wave 0's and are never read): no wave-dependent branch
      if (piece == 16) {
        if constexpr (kBytesA) load_mx_scale_bytes(eA, M * KB, kb * M + cm0, sdst, wave, lane);
        else load_mx_scales<SKA, MA>(eA, cm0, M, MBk, KB, kb, sdst, wave, lane);
      } else {
        if constexpr (kBytesB) load_mx_scale_bytes(eB, N * KB, kb * N + cn0, sdst + 1024, wave, lane);
        else load_mx_scales<SKB, MB>(eB, cn0, N, NBk, KB, kb, sdst + 1024, wave, lane);
      }
    }
  };

  // E8M0 bytes, as in gemm_kernel: per-lane byte offsets packed 2 bits per
  // subtile, plus a K-block term
  auto byte_base = [&](bool b_side, int rt) -> uint32_t {
    const int mode = b_side ? MB : MA;
    const bool km = b_side ? SKB : SKA;
    const int64_t r0 = b_side ? n0 : m0, rows = b_side ? N : M, nblk = b_side ? NBk : MBk;
    if (mode == 2) return 0;
    if (mode == 1) {
      int64_t blk = (r0 + rt) / 128;
      if (blk > nblk - 1) blk = nblk - 1;
      return static_cast<uint32_t>(km ? blk : blk * KB) & 3u;
    }
    int64_t r = r0 + rt;
    if (r > rows - 1) r = rows - 1;
    return static_cast<uint32_t>(km ? r : r * KB) & 3u;
  };
  uint32_t pack_a = 0, pack_b = 0;
  auto set_packs = [&]() {
    pack_a = 0;
    pack_b = 0;
#pragma unroll
    for (int i = 0; i < T4M; ++i) pack_a |= byte_base(false, wm * W4M + 16 * i + r16) << (2 * i);
#pragma unroll
    for (int j = 0; j < T4N; ++j) pack_b |= byte_base(true, wn * W4N + 16 * j + r16) << (2 * j);
  };
  set_packs();
  auto kterm = [&](int mode, bool km, int64_t rows, int64_t nblk, int64_t kb) -> uint32_t {
    if (mode == 2) return 0;
    return static_cast<uint32_t>(km ? kb * (mode == 1 ? nblk : rows) : kb) & 3u;
  };
  // E8M0 scale words are read from LDS one column (B) or one block (A)
  // before the bytes are extracted, so the LDS latency hides under MFMAs
  // (byte mode: the byte itself, read at the block's misalignment o, which
  // depends on the tile cm0 / cn0 of the block)
  auto word_a = [&](const uint8_t* st, int i, int64_t kbw, int64_t cm0) -> uint32_t {
    const uint8_t* sb = st + kTileABytes + kTileBBytes;
    if constexpr (kBytesA) {
      const uint32_t o = static_cast<uint32_t>(kbw * M + cm0) & 3u;
      return sb[o + wm * W4M + 16 * i + r16];
    }
    // 1x32 groups: the row's word holds its four 32-deep chunks; the lane
    // reads the byte of its own chunk g
    if constexpr (MA == 2) return sb[4 * (wm * W4M + 16 * i + r16) + g];
    const uint32_t* w = reinterpret_cast<const uint32_t*>(sb);
    return MA == 1 ? w[(wm * W4M) / 128] : w[wm * W4M + 16 * i + r16];
  };
  auto byte_a = [&](uint32_t word, int64_t kb, int i) -> int {
    if constexpr (kBytesA || MA == 2) return static_cast<int>(word);
    const uint32_t ka = kterm(MA, SKA, M, MBk, kb);
    const uint32_t sh = MA == 2 ? 8u * g : 8u * (((pack_a >> (2 * i)) + ka) & 3u);
    return static_cast<int>((word >> sh) & 0xFFu);
  };
  auto word_b = [&](const uint8_t* st, int j, int64_t kbw, int64_t cn0) -> uint32_t {
    const uint8_t* sb = st + kTileABytes + kTileBBytes + 4 * BM;
    if constexpr (kBytesB) {
      const uint32_t o = static_cast<uint32_t>(kbw * N + cn0) & 3u;
      return sb[o + wn * W4N + 16 * j + r16];
    }
    if constexpr (MB == 2) return sb[4 * (wn * W4N + 16 * j + r16) + g];
    const uint32_t* w = reinterpret_cast<const uint32_t*>(sb);
    return MB == 1 ? w[(wn * W4N) / 128] : w[wn * W4N + 16 * j + r16];
  };
  auto byte_b = [&](uint32_t word, int64_t kb, int j) -> int {
    if constexpr (kBytesB || MB == 2) return static_cast<int>(word);
    const uint32_t kbb = kterm(MB, SKB, N, NBk, kb);
    const uint32_t sh = MB == 2 ? 8u * g : 8u * (((pack_b >> (2 * j)) + kbb) & 3u);
    return static_cast<int>((word >> sh) & 0xFFu);
  };

  v4f acc[T4M][T4N];

  // ---- prologue of the first unit -------------------------------------------
  rsrc_a = opa.block_rsrc(kb_begin);
  rsrc_b = opb.block_rsrc(kb_begin);
#pragma unroll
  for (int p = 0; p < kPieces; ++p) issue_piece(kb_begin, stage0, p, m0, n0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  v8i af[T4M];
  v8i bq = opb.frag(stage0 + kTileABytes, wn * W4N, lane);
#pragma unroll
  for (int i = 0; i < T4M; ++i) af[i] = opa.frag(stage0, wm * W4M + 16 * i, lane);
  uint32_t wa[T4M];
#pragma unroll
  for (int i = 0; i < T4M; ++i) wa[i] = word_a(stage0, i, kb_begin, m0);
  uint32_t wb = word_b(stage0, 0, kb_begin, n0);

  // One K block from `cur`; the copy of the next block (this unit's, or the
  // next unit's first) into `nxt` is issued between the MFMAs of the
  // block's first half.  The barrier sits before the last column: its MFMAs
  // run from registers while the next block's B fragment and, one subtile at
  // a time, its A fragments are read from `nxt`.
  auto kblock = [&](int64_t kb, const uint8_t* cur, uint8_t* nxt) {
    const bool more = kb + 1 < kb_end;
    const bool to_next = !more && has_next;  // the same for the whole workgroup
    const int64_t kn = more ? kb + 1 : (to_next ? xkb0 : kb);
    const int64_t cm0 = to_next ? xm0 : m0, cn0 = to_next ? xn0 : n0;
    rsrc_a = advanced_rsrc(to_next ? xbase_a : opa.base, kn, opa.kstride, to_next ? xext_a : opa.ext);
    rsrc_b = advanced_rsrc(to_next ? xbase_b : opb.base, kn, opb.kstride, to_next ? xext_b : opb.ext);
    if (!more && !to_next) {  // after the last unit: the copies read nothing
      rsrc_a.z = 0;
      rsrc_b.z = 0;
    }
    int mxa[T4M];
#pragma unroll
    for (int i = 0; i < T4M; ++i) mxa[i] = byte_a(wa[i], kb, i);
    // 128x128 blocks: one B scale byte for the wave's whole 128 columns
    const int mxb_blk = MB == 1 ? byte_b(wb, kb, 0) : 0;
#pragma unroll
    for (int j = 0; j < T4N; ++j) {
      const int mxb = MB == 1 ? mxb_blk : byte_b(wb, kb, j);
      v8i bn = bq;
      if (j + 1 < T4N) {
        bn = opb.frag(cur + kTileABytes, wn * W4N + 16 * (j + 1), lane);
        if constexpr (MB != 1) wb = word_b(cur, j + 1, kb, n0);
      }
      // (after the last K block of the last unit this barrier and the reads
      // below are harmless: the copies read nothing and the fragments go
      // unused; keeping them unconditional keeps the block body one basic
      // block)
      if (j == T4N - 1) {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // this wave's copies of the next block landed
        __syncthreads();                     // everyone's did, and `cur` is free
        bn = opb.frag(nxt + kTileABytes, wn * W4N, lane);
        wb = word_b(nxt, 0, kn, cn0);
      }
#pragma unroll
      for (int i = 0; i < T4M; ++i) {
        const int t = j * T4M + i;
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            bq, af[i], acc[i][j], 0, 0, 0, mxb, 0, mxa[i]);
        // one copy piece every second MFMA slot (t = 1, 3, ..., 35)
        if (t >= 1 && (t - 1) % 2 == 0 && (t - 1) / 2 < kPieces)
          issue_piece(kn, nxt, (t - 1) / 2, cm0, cn0);
        if (j == T4N - 1) {
          af[i] = opa.frag(nxt, wm * W4M + 16 * i, lane);
          wa[i] = word_a(nxt, i, kn, cm0);
        }
        // one MFMA per scheduling region (left to the scheduler, the
        // instruction order it picks runs 10 % slower)
        __builtin_amdgcn_sched_barrier(0);
      }
      bq = bn;
    }
  };

  // ---- epilogue pieces ----------------------------------------------------------
  // split-K partial: 4 consecutive fp32 columns per lane, 16-byte stores
  auto store_partial = [&]() {
    float* pbase = part + static_cast<int64_t>(split) * pstride;  // splits pstride apart
    if (m0 + wm * W4M + W4M <= M && n0 + wn * W4N + W4N <= N) {
      float* dst = pbase + (m0 + wm * W4M + r16) * ldp + n0 + wn * W4N + 4 * g;
#pragma unroll
      for (int i = 0; i < T4M; ++i)
#pragma unroll
        for (int j = 0; j < T4N; ++j)
          *reinterpret_cast<v4f*>(dst + 16 * i * ldp + 16 * j) = acc[i][j];
      return;
    }
#pragma unroll
    for (int i = 0; i < T4M; ++i) {
      const int64_t m = m0 + wm * W4M + 16 * i + r16;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < T4N; ++j) {
        const int64_t n = n0 + wn * W4N + 16 * j + 4 * g;
        if (n < N) {
          float* dst = pbase + m * ldp + n;
#pragma unroll
          for (int r = 0; r < 4; ++r) dst[r] = acc[i][j][r];
        }
      }
    }
  };
  // bf16 through LDS: the stage of the unit's last K block (the other one
  // holds the next unit's first block) takes each wave's tile in two halves
  // of 64 padded rows; 16 lanes store each 256-byte output row, non-temporal
  auto store_out = [&](uint8_t* stg) {
    uint8_t* slot = stg + wave * (W4M / 2) * k4EpiRowBytes;
    const int64_t mw = m0 + wm * W4M, nw = n0 + wn * W4N;
    const bool whole = mw + W4M <= M && nw + W4N <= N;
    const int chunk = lane & 15;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (h == 1) __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): first half read back
#pragma unroll
      for (int i = 0; i < T4M / 2; ++i) {
#pragma unroll
        for (int j = 0; j < T4N; ++j) {
          const v4f& x = acc[(T4M / 2) * h + i][j];
          *reinterpret_cast<uint2*>(slot + (16 * i + r16) * k4EpiRowBytes + (16 * j + 4 * g) * 2) =
              make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's half is written
      __builtin_amdgcn_wave_barrier();
      if (whole) {
        v4u o[W4M / 8];
#pragma unroll
        for (int u = 0; u < W4M / 8; ++u)
          o[u] = lds_read16_a8(slot + (4 * u + (lane >> 4)) * k4EpiRowBytes + chunk * 16);
        uint16_t* dst = C + (mw + (W4M / 2) * h + (lane >> 4)) * ldc + nw + chunk * 8;
#pragma unroll
        for (int u = 0; u < W4M / 8; ++u)
          __builtin_nontemporal_store(o[u], reinterpret_cast<v4u*>(dst + 4 * u * ldc));
      } else {
#pragma unroll
        for (int u = 0; u < W4M / 8; ++u) {
          const int row = 4 * u + (lane >> 4);
          const v4u x = lds_read16_a8(slot + row * k4EpiRowBytes + chunk * 16);
          const int64_t m = mw + (W4M / 2) * h + row, n = nw + chunk * 8;
          if (m >= M) continue;
          uint16_t* dst = C + m * ldc + n;
          if (n + 7 < N) {
            __builtin_nontemporal_store(x, reinterpret_cast<v4u*>(dst));
          } else if (n < N) {
            const uint32_t w[4] = {x.x, x.y, x.z, x.w};
            for (int e = 0; e < 8 && n + e < N; ++e)
              dst[e] = static_cast<uint16_t>((w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
          }
        }
      }
    }
  };

  // ---- the units ------------------------------------------------------------------
  bool odd0 = false;  // this unit's first K block is in stage1
  while (true) {
#pragma unroll
    for (int i = 0; i < T4M; ++i)
#pragma unroll
      for (int j = 0; j < T4N; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int kb = kb_begin; kb < kb_end; ++kb) {
      const bool odd = (((kb - kb_begin) & 1) != 0) != odd0;
      kblock(kb, odd ? stage1 : stage0, odd ? stage0 : stage1);
    }
    // the copies issued during the last block (the next unit's first block)
    // have landed: the barrier before the last column waited for them
    const bool last_odd = (((kb_end - 1 - kb_begin) & 1) != 0) != odd0;
    if (part != nullptr) store_partial();
    else store_out(last_odd ? stage1 : stage0);
    if (!has_next) break;
    __syncthreads();  // every wave's staging reads are done before that stage is refilled
    // switch to the next unit; its first block's fragments and scale words
    // are already in registers
    v += static_cast<int>(gridDim.x);
    split = unit_tile(v, m0, n0, kb_begin, kb_end);
    opa.rebase(A, lda, m0, M);
    opb.rebase(B, ldb, n0, N);
    set_packs();
    odd0 = !last_odd;
    peek_next();
  }
}

__global__ __launch_bounds__(256) void fill_zero_bf16_kernel(uint16_t* __restrict__ C, int64_t M,
                                                             int64_t N, int64_t ldc) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= M * N) return;
  const int64_t r = i / N, c = i - r * N;
  C[r * ldc + c] = 0;
}

// Sum of the split-K partials in split order, rounded to bf16 (RNE): rows
// [0, rows) of C (the rows of the split tiles, C already pointing at the
// first) from partial rows [0, rows) of each split, splits pstride elements
// apart.
template <int S>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                            int64_t ldp, int64_t pstride,
                                                            uint16_t* __restrict__ C, int64_t ldc,
                                                            int64_t rows, int64_t N) {
  const int64_t quads = (N + 3) / 4;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= rows * quads) return;
  const int64_t m = i / quads, n = (i - m * quads) * 4;
  const float* p = part + m * ldp + n;
  // every split's load in flight at once (plain loads: the partials were
  // just written and are read from the caches; non-temporal loads and
  // non-temporal partial stores both measured slower)
  v4f v[S];
#pragma unroll
  for (int s = 0; s < S; ++s) v[s] = *reinterpret_cast<const v4f*>(p + s * pstride);
  v4f acc = v[0];
#pragma unroll
  for (int s = 1; s < S; ++s) {
    acc[0] += v[s][0]; acc[1] += v[s][1]; acc[2] += v[s][2]; acc[3] += v[s][3];
  }
  const uint32_t w0 = pack_bf16x2(acc[0], acc[1]), w1 = pack_bf16x2(acc[2], acc[3]);
  uint16_t* dst = C + m * ldc + n;
  if (n + 3 < N) {
    __builtin_nontemporal_store(v2u{w0, w1}, reinterpret_cast<v2u*>(dst));
  } else {
    const uint32_t h[4] = {w0 & 0xFFFFu, w0 >> 16, w1 & 0xFFFFu, w1 >> 16};
    for (int e = 0; e < 4 && n + e < N; ++e) dst[e] = static_cast<uint16_t>(h[e]);
  }
}

}  // namespace

template <bool A_KM, bool B_KM, bool MX>
static bfp8_status launch_layout(const GemmArgs& a, dim3 grid, dim3 pgrid, const UnitPlan& plan,
                                 int64_t pstride, hipStream_t stream) {
// float32 scales: the 8-wave kernel; E8M0 scales: the 4-wave kernel
#define BFP8_LAUNCH(MA, MB)                                                                   \
  do {                                                                                        \
    if constexpr (MX)                                                                         \
      return launch(&gemm_mx4_kernel<A_KM, B_KM, MA, MB>, pgrid, dim3(k4Threads), stream,    \
                    a.A, a.lda, a.sA, a.B, a.ldb, a.sB, a.C, a.ldc, a.M, a.N, a.K,            \
                    plan.tiles_m, plan.tiles_n, plan.splits, plan.part,                       \
                    (a.N + 3) & ~int64_t(3), pstride);                                        \
    else                                                                                      \
      return launch(&gemm_kernel<A_KM, B_KM, MA, MB, 256>, grid, dim3(kThreads), stream, a.A, \
                    a.lda, a.sA, a.B, a.ldb, a.sB, a.C, a.ldc, a.M, a.N, a.K, plan);          \
  } while (0)
  // mode 3 (K-block-major act scales) is mode 0 for a K-major operand
  const int ma = (A_KM && a.modeA == 3) ? 0 : a.modeA;
  const int mb = (B_KM && a.modeB == 3) ? 0 : a.modeB;
  if (ma == 0 && mb == 1) BFP8_LAUNCH(0, 1);
  else if (ma == 0 && mb == 0) BFP8_LAUNCH(0, 0);
  else if (ma == 1 && mb == 0) BFP8_LAUNCH(1, 0);
  else if (ma == 1 && mb == 1) BFP8_LAUNCH(1, 1);
  if constexpr (!A_KM) {
    if (ma == 3 && mb == 1) BFP8_LAUNCH(3, 1);
    else if (ma == 3 && mb == 0) BFP8_LAUNCH(3, 0);
    if constexpr (!B_KM) {
      if (ma == 3 && mb == 3) BFP8_LAUNCH(3, 3);
      else if (ma == 0 && mb == 3) BFP8_LAUNCH(0, 3);
      else if (ma == 1 && mb == 3) BFP8_LAUNCH(1, 3);
    }
  }
  if constexpr (MX) {
    // 1x32 groups (mode 2) exist only with E8M0 scales and K-contiguous storage
    if constexpr (!A_KM && !B_KM) {
      if (ma == 2 && mb == 2) BFP8_LAUNCH(2, 2);
      else if (ma == 2 && mb == 0) BFP8_LAUNCH(2, 0);
      else if (ma == 2 && mb == 1) BFP8_LAUNCH(2, 1);
      else if (ma == 0 && mb == 2) BFP8_LAUNCH(0, 2);
      else if (ma == 1 && mb == 2) BFP8_LAUNCH(1, 2);
    } else if constexpr (!A_KM) {
      if (ma == 2 && mb == 0) BFP8_LAUNCH(2, 0);
      else if (ma == 2 && mb == 1) BFP8_LAUNCH(2, 1);
    }
  }
#undef BFP8_LAUNCH
  return BFP8_ERR_SCALE_MODE;
}

// Split-K plan for shapes whose 256x256 tiles under-fill the chip.  The
// candidates: every tile split evenly into S ranges of K blocks, or whole
// waves of tiles run unsplit and only the tiles left over for a last,
// partial wave split into S ranges (so their units fill that wave).  Each is
// priced by a model of one workgroup per CU -- a unit costs a fixed
// prologue/epilogue plus a per-K-block time, units run in waves of 256 --
// plus the fp32 partials' round trip through HBM and the reduction's launch;
// the cheapest wins if it beats the unsplit plan by 5 %.  Splits keep >= 8
// K blocks.  The plan depends only on the shape, so the workspace query
// and every launch agree.
static int64_t split_ldp(int64_t N) { return (N + 3) & ~int64_t(3); }

GemmPlan gemm_plan(int64_t M, int64_t N, int64_t K, bool mx) {
  constexpr int64_t kCUs = 256;      // MI355X compute units: workgroups per wave
  constexpr double kBlockUs = 1.6;   // one 256x256x128 K block of one tile, measured order
  constexpr double kUnitUs = 5.0;    // a unit's prologue and epilogue
  constexpr double kBytesPerUs = 4.0e6;
  constexpr double kReduceUs = 4.0;  // the reduction kernel's launch
  const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int64_t tiles = tiles_m * tiles_n;
  const int64_t KB = K / BK;
  GemmPlan plan{tiles, 1, 0};
  if (tiles == 0 || KB == 0) return plan;
  auto waves = [&](int64_t units) { return static_cast<double>((units + kCUs - 1) / kCUs); };
  auto unit_us = [&](int64_t kblocks) { return kblocks * kBlockUs + kUnitUs; };
  auto partial_us = [&](int64_t S, int64_t rows) {
    return (static_cast<double>(S) * rows * split_ldp(N) * 8.0 + rows * N * 2.0) / kBytesPerUs +
           kReduceUs;
  };
  const double unsplit = waves(tiles) * unit_us(KB);
  double best_t = unsplit * 0.95;
  // whole waves first: a multiple of the CU count that is also a multiple of
  // the tile walk's row groups, so the split tiles are whole rows of tiles
  const int64_t full = (tiles / kCUs) * kCUs;
  // (the persistent power-of-two kernel runs such a plan as two launches of
  // whole rows of tiles, so for it the split rows must not end in a ragged
  // tile)
  const bool hybrid = full > 0 && full < tiles && full % (kGroupM * tiles_n) == 0 &&
                      (!mx || M % BM == 0);
  for (int64_t S : {2, 3, 4, 6, 8}) {
    if (KB / S < 8) break;
    if (KB % S != 0) continue;  // equal ranges of K blocks
    if (tiles * S >= (int64_t(1) << 30)) break;
    const int64_t piece = KB / S;
    const double even = waves(tiles * S) * unit_us(piece) + partial_us(S, M);
    if (even < best_t) {
      best_t = even;
      plan = GemmPlan{0, static_cast<int>(S), 0};
    }
    if (hybrid) {
      const int64_t row0 = (full / tiles_n) * BM;
      const double t = waves(full) * unit_us(KB) + waves((tiles - full) * S) * unit_us(piece) +
                       partial_us(S, M - row0);
      if (t < best_t) {
        best_t = t;
        plan = GemmPlan{full, static_cast<int>(S), row0};
      }
    }
  }
  return plan;
}

// Bytes of the fp32 partials of a plan, rounded up to 256.
static size_t partial_bytes(const GemmPlan& p, int64_t M, int64_t N) {
  const size_t b = static_cast<size_t>(p.splits) * (M - p.row0) * split_ldp(N) * sizeof(float);
  return (b + 255) & ~size_t(255);
}

size_t gemm_split_workspace(int64_t M, int64_t N, int64_t K, bool mx) {
  const GemmPlan p = gemm_plan(M, N, K, mx);
  if (p.splits == 1) return 0;
  // the power-of-two kernel's whole-wave plan also copies A's K-block-major
  // scale bytes of the split rows: K/128 x (M - row0) bytes at most, read as
  // aligned 32-bit words (so up to 3 bytes past the copy)
  const size_t extra =
      (mx && p.full > 0) ? (static_cast<size_t>(K / BK) * (M - p.row0) + 4 + 255) & ~size_t(255) : 0;
  return partial_bytes(p, M, N) + extra;
}

// Byte offset of the E8M0 scales of row r0 (a multiple of 128) of an A
// stored [M][K] with row-major scales in mode `mode` (0, 1 or 2).
static int64_t mx_scale_row_offset(int mode, int64_t r0, int64_t K) {
  const int64_t KB = K / BK;
  switch (mode) {
    case 1: return (r0 / 128) * KB;                 // [M/128][KB]
    case 2: return r0 * (K / 32);                   // [M][K/32]
    default: return r0 * KB;                        // 0: [M][KB]
  }
}

// 256 x 192 tiles for the float32 kernel (NT, 1x128 scales on B): taken
// when N is a multiple of 192, the 256-column plan runs unsplit, and the
// narrower tiles fill whole waves where the 256-column ones leave CUs idle
// (the 2048 x 6144 wgrad output: 256 tiles instead of 192).  A K block of
// such a tile is priced at 0.75 of a 256 x 256 block times 1.15 for its
// larger copy and fragment bytes per flop.
static bool use_192_columns(int64_t M, int64_t N, int64_t K) {
  constexpr int64_t kCUs = 256;
  constexpr double kBlockUs = 1.6, kUnitUs = 5.0;
  if (N % 192 != 0 || gemm_plan(M, N, K, false).splits > 1) return false;
  const int64_t KB = K / BK, tiles_m = (M + BM - 1) / BM;
  const int64_t t256 = tiles_m * ((N + BN - 1) / BN), t192 = tiles_m * (N / 192);
  if (t192 >= (int64_t(1) << 31)) return false;
  auto waves = [&](int64_t u) { return static_cast<double>((u + kCUs - 1) / kCUs); };
  const double c256 = waves(t256) * (KB * kBlockUs + kUnitUs);
  const double c192 = waves(t192) * (KB * kBlockUs * 0.75 * 1.15 + kUnitUs);
  return c192 < 0.95 * c256;
}

bfp8_status launch_gemm(const GemmArgs& a, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  if (!a.mx && !a.a_kmajor && !a.b_kmajor && (a.modeB == 0 || a.modeB == 3) &&
      (a.modeA == 0 || a.modeA == 3) && use_192_columns(a.M, a.N, a.K)) {
    UnitPlan p;
    p.tiles_m = static_cast<int>((a.M + BM - 1) / BM);
    p.tiles_n = static_cast<int>(a.N / 192);
    p.full = p.tiles_m * p.tiles_n;
    p.splits = 1;
    p.piece = static_cast<int>(a.K / BK);
    p.trow0 = 0;
    p.part = nullptr;
    const dim3 g(static_cast<unsigned>(p.full));
#define BFP8_LAUNCH192(MA, MB)                                                                 \
  return launch(&gemm_kernel<false, false, MA, MB, 192>, g, dim3(kThreads), stream, a.A,       \
                a.lda, a.sA, a.B, a.ldb, a.sB, a.C, a.ldc, a.M, a.N, a.K, p)
    if (a.modeA == 0 && a.modeB == 0) BFP8_LAUNCH192(0, 0);
    if (a.modeA == 0 && a.modeB == 3) BFP8_LAUNCH192(0, 3);
    if (a.modeA == 3 && a.modeB == 0) BFP8_LAUNCH192(3, 0);
    BFP8_LAUNCH192(3, 3);
#undef BFP8_LAUNCH192
  }
  const int64_t tiles_m = (a.M + BM - 1) / BM;
  const int64_t tiles_n = (a.N + BN - 1) / BN;
  const int64_t nblk = tiles_m * tiles_n;
  if (nblk == 0) return BFP8_OK;
  GemmPlan gp = gemm_plan(a.M, a.N, a.K, a.mx);
  if (gp.splits > 1 &&
      (workspace == nullptr || workspace_bytes < gemm_split_workspace(a.M, a.N, a.K, a.mx)))
    gp = GemmPlan{nblk, 1, 0};  // no room for partials: run unsplit
  UnitPlan plan;
  plan.tiles_m = static_cast<int>(tiles_m);
  plan.tiles_n = static_cast<int>(tiles_n);
  plan.full = static_cast<int>(gp.full);
  plan.splits = gp.splits;
  plan.piece = static_cast<int>(a.K / BK / gp.splits);
  plan.trow0 = static_cast<int>(gp.row0 / BM);
  plan.part = gp.splits > 1 ? static_cast<float*>(workspace) : nullptr;
  const int64_t ldp = split_ldp(a.N);
  const int64_t units = gp.full + (nblk - gp.full) * gp.splits;
  const dim3 grid(static_cast<unsigned>(units));
  // the power-of-two kernel is persistent: one workgroup per compute unit
  // (its LDS stages fill a CU), a multiple of the 8 XCDs, each running every
  // gridDim-th unit
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return BFP8_ERR_HIP;
  const int64_t wgs = cus >= kXcds ? (cus / kXcds) * kXcds : cus;
  const dim3 pgrid(static_cast<unsigned>(units < wgs ? units : wgs));
  // splits of the partials: (M - row0) rows apart, the rows of the split tiles
  const int64_t rows_all = a.M - gp.row0;
  auto launch_mx = [&](const GemmArgs& g, const UnitPlan& p, dim3 pg, int64_t pst) -> bfp8_status {
    if (!g.a_kmajor && !g.b_kmajor) return launch_layout<false, false, true>(g, grid, pg, p, pst, stream);
    if (!g.a_kmajor && g.b_kmajor) return launch_layout<false, true, true>(g, grid, pg, p, pst, stream);
    if (g.a_kmajor && g.b_kmajor) return launch_layout<true, true, true>(g, grid, pg, p, pst, stream);
    return BFP8_ERR_LAYOUT;
  };
  auto min_wgs = [&](int64_t u) { return dim3(static_cast<unsigned>(u < wgs ? u : wgs)); };
  bfp8_status st;
  if (a.mx && gp.splits > 1 && gp.full > 0) {
    // the persistent kernel splits every tile of a launch alike, so the plan
    // runs as two launches: the whole tiles (output rows [0, row0)), then the
    // rows [row0, M) as an (M - row0)-row GEMM of their own whose operand A,
    // its scales and C start row0 rows in, its partials (M - row0) rows per
    // split as in the float32 kernel.  Row-major scales ([rows][...]) are
    // used in place; K-block-major ones ([K/128][rows or row blocks], whose
    // row count is their stride) are first copied, rows [row0, M) of every
    // K block, to the end of the workspace.  M - row0 is a multiple of 256.
    UnitPlan p1 = plan, p2 = plan;
    p1.tiles_m = plan.trow0;
    p1.full = plan.trow0 * plan.tiles_n;
    p1.splits = 1;
    p1.part = nullptr;
    st = launch_mx(a, p1, min_wgs(p1.full), 0);
    if (st != BFP8_OK) return st;
    GemmArgs a2 = a;
    a2.M = a.M - gp.row0;
    a2.A = a.A + (a.a_kmajor ? gp.row0 : gp.row0 * a.lda);
    a2.C = a.C + gp.row0 * a.ldc;
    const uint8_t* sa8 = static_cast<const uint8_t*>(a.sA);
    if (!a.a_kmajor && a.modeA != 3) {
      a2.sA = sa8 + mx_scale_row_offset(a.modeA, gp.row0, a.K);
    } else {
      const bool blk = a.modeA == 1;
      const int64_t cols = blk ? a.M / 128 : a.M, sub = blk ? a2.M / 128 : a2.M;
      const int64_t off = blk ? gp.row0 / 128 : gp.row0;
      uint8_t* dst = static_cast<uint8_t*>(workspace) + partial_bytes(gp, a.M, a.N);
      if (hipMemcpy2DAsync(dst, static_cast<size_t>(sub), sa8 + off, static_cast<size_t>(cols),
                           static_cast<size_t>(sub), static_cast<size_t>(a.K / BK),
                           hipMemcpyDeviceToDevice, stream) != hipSuccess)
        return BFP8_ERR_HIP;
      a2.sA = dst;
    }
    p2.tiles_m = plan.tiles_m - plan.trow0;
    p2.full = 0;
    st = launch_mx(a2, p2, min_wgs(static_cast<int64_t>(p2.tiles_m) * p2.tiles_n * p2.splits),
                   rows_all * ldp);
  } else if (a.mx) {
    if (!a.a_kmajor && !a.b_kmajor) st = launch_layout<false, false, true>(a, grid, pgrid, plan, rows_all * ldp, stream);
    else if (!a.a_kmajor && a.b_kmajor) st = launch_layout<false, true, true>(a, grid, pgrid, plan, rows_all * ldp, stream);
    else if (a.a_kmajor && a.b_kmajor) st = launch_layout<true, true, true>(a, grid, pgrid, plan, rows_all * ldp, stream);
    else return BFP8_ERR_LAYOUT;
  } else {
    if (!a.a_kmajor && !a.b_kmajor) st = launch_layout<false, false, false>(a, grid, pgrid, plan, rows_all * ldp, stream);
    else if (!a.a_kmajor && a.b_kmajor) st = launch_layout<false, true, false>(a, grid, pgrid, plan, rows_all * ldp, stream);
    else if (a.a_kmajor && a.b_kmajor) st = launch_layout<true, true, false>(a, grid, pgrid, plan, rows_all * ldp, stream);
    else return BFP8_ERR_LAYOUT;
  }
  if (st != BFP8_OK || gp.splits == 1) return st;
  const int64_t rows = rows_all, pstride = rows_all * ldp;
  const int64_t n = rows * ((a.N + 3) / 4);
  const dim3 rgrid(static_cast<unsigned>((n + 255) / 256));
#define BFP8_REDUCE(S_)                                                                      \
  case S_:                                                                                   \
    return launch(&splitk_reduce_kernel<S_>, rgrid, dim3(256), stream, plan.part, ldp,      \
                  pstride, a.C + gp.row0 * a.ldc, a.ldc, rows, a.N)
  switch (gp.splits) {
    BFP8_REDUCE(2);
    BFP8_REDUCE(3);
    BFP8_REDUCE(4);
    BFP8_REDUCE(6);
    BFP8_REDUCE(8);
  }
#undef BFP8_REDUCE
  return BFP8_ERR_HIP;  // no plan has another split count
}

// ---- split-K partials in a static device array -------------------------
// For callers that cannot allocate (bfp8_gemm_static_scratch): the float32
// split-K partials live in this file-scope array instead of a caller
// workspace.  Each GPU the library runs on holds its own copy until the
// process ends.  In host code `scratch` names a host-side stand-in, not the
// device memory: its device address is looked up once per device with
// hipGetSymbolAddress and only that address is handed to kernels.
static __device__ __align__(256) uint8_t scratch[BFP8_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the calling thread's current device.
bfp8_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return BFP8_ERR_HIP;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
        return BFP8_ERR_HIP;
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return BFP8_OK;
}
}  // namespace

bfp8_status launch_gemm_static_scratch(const GemmArgs& a, hipStream_t stream) {
  const size_t need = gemm_split_workspace(a.M, a.N, a.K, a.mx);
  if (need > static_cast<size_t>(BFP8_STATIC_SCRATCH_BYTES)) return BFP8_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    const bfp8_status st = scratch_address(&ws);
    if (st != BFP8_OK) return st;
  }
  // every split writes all of its partials before the reduction reads them,
  // so nothing in the array needs clearing between calls
  return launch_gemm(a, ws, need, stream);
}

bfp8_status launch_fill_bf16_zero(uint16_t* C, int64_t M, int64_t N, int64_t ldc,
                                  hipStream_t stream) {
  const int64_t n = M * N;
  if (n == 0) return BFP8_OK;
  return launch(&fill_zero_bf16_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256),
                stream, C, M, N, ldc);
}

}  // namespace bfp8
