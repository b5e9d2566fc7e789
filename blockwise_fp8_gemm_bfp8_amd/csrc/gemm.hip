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
//     columns in that XCD's L2.
//
// Operands whose scales are powers of two stored as E8M0 bytes (Puro-2B
// translation, section 3.2: the SM120 runs used power-of-two block scales on
// the MXFP8 path) go to gemm_mx4_kernel: the same tile and LDS stages, but
// the scales ride in the matrix-core instruction
// (v_mfma_scale_f32_16x16x128_f8f6f4), the accumulators are the MFMA's C
// operand in the AGPR file, and no VALU promotion is needed, which lets 4
// waves of 128 x 128 replace 8 waves of 64 x 128.  The instruction takes one
// scale byte per row and 32-deep K chunk: the register of lane group j
// (lane 16j + r) scales row r's K values [32j, 32j + 32) -- which the
// fragment layout below spreads over lane groups 2j mod 4 and 2j + 1 mod 4
// (measured on gfx950) -- so the lane's byte is always its row's scale of
// chunk j = lane / 16.

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

// Map the hardware block id to a (tile_m, tile_n) pair: first undo the
// round-robin XCD dealing so each XCD owns a contiguous range of logical
// tiles, then walk tiles in column-major groups of kGroupM rows.
__device__ __forceinline__ void tile_coords(int bid, int nblk, int tiles_m, int tiles_n, int& tm,
                                            int& tn) {
  const int q = nblk / kXcds, r = nblk % kXcds;
  const int xcd = bid % kXcds, local = bid / kXcds;
  const int logical = xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
  const int per_group = kGroupM * tiles_n;
  const int group = logical / per_group;
  const int first_m = group * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int in_group = logical - group * per_group;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
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
    const int64_t rows_left = rows - r0;  // valid rows (or columns) from the tile start
    base = reinterpret_cast<uint64_t>(KMAJOR ? p + r0 : p + r0 * ld_);
    kstride = KMAJOR ? BK * ld_ : BK;
    // Extent from the start of a K block.  K-contiguous: up to the end of
    // that block's part of the last valid row, so every copy of a row past
    // the valid ones (offset >= valid rows * ld) reads zeros.  K-major: the
    // block's 128 k rows, a ragged last column chunk read up to the next
    // 16-byte boundary, which the padded leading dimension covers.
    int64_t e;
    if (!KMAJOR) {
      const int64_t rv = rows_left > 256 ? 256 : rows_left;
      e = (rv - 1) * ld_ + BK;
    } else {
      const int64_t cols = rows_left > 256 ? 256 : ((rows_left + 15) & ~int64_t(15));
      e = (BK - 1) * ld_ + cols;
    }
    ext = __builtin_amdgcn_readfirstlane(static_cast<int>(e > 0x7FFFFFFF ? 0x7FFFFFFF : e));
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

template <bool A_KM, bool B_KM, int MODE_A, int MODE_B>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(2, 2))) void
gemm_kernel(const uint8_t* __restrict__ A, int64_t lda, const void* __restrict__ sA_,
            const uint8_t* __restrict__ B, int64_t ldb, const void* __restrict__ sB_,
            uint16_t* __restrict__ C, int64_t ldc, int64_t M, int64_t N, int64_t K, int tiles_m,
            int tiles_n, float* __restrict__ part, int64_t ldp) {
  const float* __restrict__ sA = static_cast<const float*>(sA_);
  const float* __restrict__ sB = static_cast<const float*>(sB_);
  // Two pipeline stages; block kb lives in stage kb % 2.
  __shared__ __attribute__((aligned(1024))) uint8_t stage0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t stage1[kStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % kWavesM;
  const int wn = wave / kWavesM;
  const int g = lane >> 4, r16 = lane & 15;

  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = static_cast<int64_t>(tm) * BM;
  const int64_t n0 = static_cast<int64_t>(tn) * BN;
  const int64_t KB = K / BK;
  const int64_t MBk = (M + 127) / 128, NBk = (N + 127) / 128;
  // split-K: blockIdx.y selects a contiguous range of K blocks; with more
  // than one split the fp32 tile goes to part[split] and a second kernel
  // sums the splits in order.
  const int splits = gridDim.y, split = blockIdx.y;  // 32-bit: KB * splits < 2^31
  const int kb_begin = static_cast<int>((split * static_cast<int>(KB)) / splits);
  const int kb_end = static_cast<int>(((split + 1) * static_cast<int>(KB)) / splits);

  Operand<A_KM> opa;
  Operand<B_KM> opb;
  opa.init(A, lda, m0, M, K, wave, lane);
  opb.init(B, ldb, n0, N, K, wave, lane);

  // The copy of one K block is split into 9 pieces per wave (4 x 1 KiB of
  // A, 4 x 1 KiB of B, one dword per lane of act-mode scales) so the pieces
  // can be spread over the MFMA issue slots of the block before.
  constexpr int kLoadPieces = 9;
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
    const int mode = b_side ? MODE_B : MODE_A;
    const bool km = b_side ? B_KM : A_KM;
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
    } else if (piece < 8) {
      opb.load_piece(rsrc_b, st + kTileABytes, wave, piece - 4);
    } else {
      uint8_t* sdst = st + kTileABytes + kTileBBytes;
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
    const float* s_lds = reinterpret_cast<const float*>(st + kTileABytes + kTileBBytes);
    const float sb = MODE_B == 1 ? s_lds[BM + wn] : 1.0f;
    if (MODE_A == 0) {
#pragma unroll
      for (int i = 0; i < TM; ++i) ra[i] = s_lds[wm * WM + 16 * i + r16] * sb;
    } else {
      const float sa = s_lds[(wm * WM) / 128] * sb;
#pragma unroll
      for (int i = 0; i < TM; ++i) ra[i] = sa;
    }
  };
  auto col_mults = [&](const uint8_t* st, int j, float (&cb)[4]) {
    if (MODE_B == 0) {
      const float* s_lds = reinterpret_cast<const float*>(st + kTileABytes + kTileBBytes);
      const float4 v = *reinterpret_cast<const float4*>(s_lds + BM + wn * WN + 16 * j + 4 * g);
      cb[0] = v.x; cb[1] = v.y; cb[2] = v.z; cb[3] = v.w;
    }
  };

  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

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
      x = fmaf(p[r], MODE_B == 0 ? rmul * cm[r] : rmul, x);
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
  bq = opb.frag(stage0 + kTileABytes, wn * WN, lane);
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
  // (free since the previous barrier) is issued piecewise between the first
  // MFMAs; then, once every wave's copies have landed, the fragments of
  // block kb+1 are read from `nxt`.
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
    for (int j = 0; j < TN; ++j) {
      v8i bn = bq;
      if (j + 1 < TN) bn = opb.frag(cur + kTileABytes, wn * WN + 16 * (j + 1), lane);
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
        if (t >= 1 && t <= kLoadPieces) issue_piece(kn, nxt, t - 1);
        // one MFMA and the promotion of the partial kLag issues back per
        // scheduling region: the machine scheduler would otherwise pull each
        // promotion up against the MFMA that produces it and stall on it
        __builtin_amdgcn_sched_barrier(0);
      }
      bq = bn;
    }
    // all MFMAs of this K block are issued; the last kLag subtiles (all in
    // column TN-1) are pending with this block's multipliers
#pragma unroll
    for (int i = 0; i < TM; ++i) ra_last[i] = ra[i];
    if (more) {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // this wave's copies of block kb+1 landed
      __syncthreads();                     // everyone's did, and `cur` is free
      // B fragment and A row 0 first: the next block's first MFMA needs
      // only those two
      bq = opb.frag(nxt + kTileABytes, wn * WN, lane);
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = opa.frag(nxt, wm * WM + 16 * i, lane);
      row_mults(nxt, ra);
    }
#pragma unroll
    for (int q = 0; q < kLag; ++q) {
      const int t = TM * TN - kLag + q;
      promote(acc[t % TM][TN - 1], pend[t % kLag], ra_last[t % TM], cm_cur);
    }
  };

  for (int kb = kb_begin; kb < kb_end; kb += 2) {
    kblock(kb, stage0, stage1);
    if (kb + 1 < kb_end) kblock(kb + 1, stage1, stage0);
  }

  // the copies issued during the last block must land before the stages
  // are reused for the output
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  if (part != nullptr) {
    // split-K partial: 4 consecutive fp32 columns per lane, 16-byte stores
    float* pbase = part + static_cast<int64_t>(split) * M * ldp;
    if (m0 + wm * WM + WM <= M && n0 + wn * WN + WN <= N) {
      float* dst = pbase + (m0 + wm * WM + r16) * ldp + n0 + wn * WN + 4 * g;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          *reinterpret_cast<v4f*>(dst + 16 * i * ldp + 16 * j) = acc[i][j];
      return;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int64_t m = m0 + wm * WM + 16 * i + r16;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t n = n0 + wn * WN + 16 * j + 4 * g;
        if (n < N) {
          float* dst = pbase + m * ldp + n;
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
  uint8_t* slot = (wave < 4 ? stage0 : stage1) + (wave & 3) * kEpiSlotBytes;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      *reinterpret_cast<uint2*>(slot + (16 * i + r16) * kEpiRowBytes + (16 * j + 4 * g) * 2) =
          make_uint2(pack_bf16x2(acc[i][j][0], acc[i][j][1]),
                     pack_bf16x2(acc[i][j][2], acc[i][j][3]));
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's slot is written
  __builtin_amdgcn_wave_barrier();
  const int64_t mw = m0 + wm * WM, nw = n0 + wn * WN;
  const int chunk = lane & 15;  // 8 bf16 columns
  if (mw + WM <= M && nw + WN <= N) {
    // whole wave tile inside C: all row reads first, then the stores, with
    // no per-row tests (a read-then-test loop waits out the LDS latency
    // once per row)
    v4u v[WM / 4];
#pragma unroll
    for (int u = 0; u < WM / 4; ++u)
      v[u] = *reinterpret_cast<const v4u*>(slot + (4 * u + (lane >> 4)) * kEpiRowBytes + chunk * 16);
    uint16_t* dst = C + (mw + (lane >> 4)) * ldc + nw + chunk * 8;
#pragma unroll
    for (int u = 0; u < WM / 4; ++u)
      __builtin_nontemporal_store(v[u], reinterpret_cast<v4u*>(dst + 4 * u * ldc));
    return;
  }
#pragma unroll
  for (int u = 0; u < WM / 4; ++u) {
    const int row = 4 * u + (lane >> 4);
    const uint4 v = *reinterpret_cast<const uint4*>(slot + row * kEpiRowBytes + chunk * 16);
    const int64_t m = mw + row, n = nw + chunk * 8;
    if (m >= M) continue;
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
static_assert(2 * W4M * k4EpiRowBytes <= kStageBytes, "two epilogue slots per stage");

template <bool A_KM, bool B_KM, int MODE_A, int MODE_B>
__global__ __attribute__((amdgpu_flat_work_group_size(k4Threads, k4Threads),
                          amdgpu_waves_per_eu(1, 1))) void
gemm_mx4_kernel(const uint8_t* __restrict__ A, int64_t lda, const void* __restrict__ sA_,
                const uint8_t* __restrict__ B, int64_t ldb, const void* __restrict__ sB_,
                uint16_t* __restrict__ C, int64_t ldc, int64_t M, int64_t N, int64_t K, int tiles_m,
                int tiles_n, float* __restrict__ part, int64_t ldp) {
  const uint8_t* __restrict__ eA = static_cast<const uint8_t*>(sA_);
  const uint8_t* __restrict__ eB = static_cast<const uint8_t*>(sB_);
  __shared__ __attribute__((aligned(1024))) uint8_t stage0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t stage1[kStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int g = lane >> 4, r16 = lane & 15;

  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = static_cast<int64_t>(tm) * BM;
  const int64_t n0 = static_cast<int64_t>(tn) * BN;
  const int64_t KB = K / BK;
  const int64_t MBk = (M + 127) / 128, NBk = (N + 127) / 128;
  const int splits = gridDim.y, split = blockIdx.y;
  const int kb_begin = static_cast<int>((split * static_cast<int>(KB)) / splits);
  const int kb_end = static_cast<int>(((split + 1) * static_cast<int>(KB)) / splits);

  Operand<A_KM, 8> opa;
  Operand<B_KM, 8> opb;
  opa.init(A, lda, m0, M, K, wave, lane);
  opb.init(B, ldb, n0, N, K, wave, lane);

  // The copy of one K block: 8 x 1 KiB of A, 8 x 1 KiB of B and the scale
  // words of 64 rows of A and 64 columns of B per wave.
  constexpr int kPieces = 18;
  i32x4 rsrc_a, rsrc_b;
  auto issue_piece = [&](int64_t kb, uint8_t* st, int piece) {
    if (piece < 8) {
      opa.load_piece(rsrc_a, st, wave, piece);
    } else if (piece < 16) {
      opb.load_piece(rsrc_b, st + kTileABytes, wave, piece - 8);
    } else {
      uint8_t* sdst = st + kTileABytes + kTileBBytes;
      // every wave copies (for 128x128 blocks the copies of waves 1-3 land
      // beside wave 0's and are never read): no wave-dependent branch
      if (piece == 16)
        load_mx_scales<A_KM, MODE_A>(eA, m0, M, MBk, KB, kb, sdst, wave, lane);
      else
        load_mx_scales<B_KM, MODE_B>(eB, n0, N, NBk, KB, kb, sdst + 1024, wave, lane);
    }
  };

  // E8M0 bytes, as in gemm_kernel: per-lane byte offsets packed 2 bits per
  // subtile, plus a K-block term
  auto byte_base = [&](bool b_side, int rt) -> uint32_t {
    const int mode = b_side ? MODE_B : MODE_A;
    const bool km = b_side ? B_KM : A_KM;
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
#pragma unroll
  for (int i = 0; i < T4M; ++i) pack_a |= byte_base(false, wm * W4M + 16 * i + r16) << (2 * i);
#pragma unroll
  for (int j = 0; j < T4N; ++j) pack_b |= byte_base(true, wn * W4N + 16 * j + r16) << (2 * j);
  auto kterm = [&](int mode, bool km, int64_t rows, int64_t nblk, int64_t kb) -> uint32_t {
    if (mode == 2) return 0;
    return static_cast<uint32_t>(km ? kb * (mode == 1 ? nblk : rows) : kb) & 3u;
  };
  // E8M0 scale words are read from LDS one column (B) or one block (A)
  // before the bytes are extracted, so the LDS latency hides under MFMAs
  auto word_a = [&](const uint8_t* st, int i) -> uint32_t {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(st + kTileABytes + kTileBBytes);
    return MODE_A == 1 ? w[(wm * W4M) / 128] : w[wm * W4M + 16 * i + r16];
  };
  auto byte_a = [&](uint32_t word, int64_t kb, int i) -> int {
    const uint32_t ka = kterm(MODE_A, A_KM, M, MBk, kb);
    const uint32_t sh = MODE_A == 2 ? 8u * g : 8u * (((pack_a >> (2 * i)) + ka) & 3u);
    return static_cast<int>((word >> sh) & 0xFFu);
  };
  auto word_b = [&](const uint8_t* st, int j) -> uint32_t {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(st + kTileABytes + kTileBBytes) + BM;
    return MODE_B == 1 ? w[(wn * W4N) / 128] : w[wn * W4N + 16 * j + r16];
  };
  auto byte_b = [&](uint32_t word, int64_t kb, int j) -> int {
    const uint32_t kbb = kterm(MODE_B, B_KM, N, NBk, kb);
    const uint32_t sh = MODE_B == 2 ? 8u * g : 8u * (((pack_b >> (2 * j)) + kbb) & 3u);
    return static_cast<int>((word >> sh) & 0xFFu);
  };

  v4f acc[T4M][T4N];
#pragma unroll
  for (int i = 0; i < T4M; ++i)
#pragma unroll
    for (int j = 0; j < T4N; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // ---- prologue -----------------------------------------------------------
  rsrc_a = opa.block_rsrc(kb_begin);
  rsrc_b = opb.block_rsrc(kb_begin);
#pragma unroll
  for (int p = 0; p < kPieces; ++p) issue_piece(kb_begin, stage0, p);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  v8i af[T4M];
  v8i bq = opb.frag(stage0 + kTileABytes, wn * W4N, lane);
#pragma unroll
  for (int i = 0; i < T4M; ++i) af[i] = opa.frag(stage0, wm * W4M + 16 * i, lane);
  uint32_t wa[T4M];
#pragma unroll
  for (int i = 0; i < T4M; ++i) wa[i] = word_a(stage0, i);
  uint32_t wb = word_b(stage0, 0);

  // One K block from `cur`; the copy of block kb+1 into `nxt` is issued
  // between the first MFMAs.  The barrier sits before the last column: its
  // MFMAs run from registers while the next block's B fragment and, one
  // subtile at a time, its A fragments are read from `nxt`.
  auto kblock = [&](int64_t kb, const uint8_t* cur, uint8_t* nxt) {
    const bool more = kb + 1 < kb_end;
    const int64_t kn = more ? kb + 1 : kb;
    rsrc_a = opa.block_rsrc(kn);
    rsrc_b = opb.block_rsrc(kn);
    if (!more) {
      rsrc_a.z = 0;
      rsrc_b.z = 0;
    }
    int mxa[T4M];
#pragma unroll
    for (int i = 0; i < T4M; ++i) mxa[i] = byte_a(wa[i], kb, i);
#pragma unroll
    for (int j = 0; j < T4N; ++j) {
      const int mxb = byte_b(wb, kb, j);
      v8i bn = bq;
      if (j + 1 < T4N) {
        bn = opb.frag(cur + kTileABytes, wn * W4N + 16 * (j + 1), lane);
        wb = word_b(cur, j + 1);
      }
      // (after the last K block this barrier and the reads below are
      // harmless: the copies read nothing and the fragments go unused;
      // keeping them unconditional keeps the block body one basic block)
      if (j == T4N - 1) {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // this wave's copies of block kb+1 landed
        __syncthreads();                     // everyone's did, and `cur` is free
        bn = opb.frag(nxt + kTileABytes, wn * W4N, lane);
        wb = word_b(nxt, 0);
      }
#pragma unroll
      for (int i = 0; i < T4M; ++i) {
        const int t = j * T4M + i;
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            bq, af[i], acc[i][j], 0, 0, 0, mxb, 0, mxa[i]);
        // pin the accumulator of the MFMA three issues back (AGPR operand,
        // no copy): without an anchor the MFMAs drift away from the copies
        // and fragment reads they are meant to cover
        if (t >= 3) asm volatile("" : "+a"(acc[(t - 3) % T4M][(t - 3) / T4M]));
        if (t >= 1 && t <= kPieces) issue_piece(kn, nxt, t - 1);
        if (j == T4N - 1) {
          af[i] = opa.frag(nxt, wm * W4M + 16 * i, lane);
          wa[i] = word_a(nxt, i);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      bq = bn;
    }
#pragma unroll
    for (int q = 0; q < 3; ++q) asm volatile("" : "+a"(acc[(T4M * T4N - 3 + q) % T4M][T4N - 1]));
  };
  // one copy of the block body with the stages picked at run time
  for (int kb = kb_begin; kb < kb_end; ++kb) {
    const bool odd = ((kb - kb_begin) & 1) != 0;
    kblock(kb, odd ? stage1 : stage0, odd ? stage0 : stage1);
  }

  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the last copies landed
  if (part != nullptr) {
    float* pbase = part + static_cast<int64_t>(split) * M * ldp;
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
    return;
  }

  // ---- epilogue: bf16 through LDS (two padded 128 x 128 slots per stage),
  // then 16 lanes store each 256-byte output row, non-temporal
  __syncthreads();
  uint8_t* slot = (wave < 2 ? stage0 : stage1) + (wave & 1) * (W4M * k4EpiRowBytes);
#pragma unroll
  for (int i = 0; i < T4M; ++i) {
#pragma unroll
    for (int j = 0; j < T4N; ++j) {
      *reinterpret_cast<uint2*>(slot + (16 * i + r16) * k4EpiRowBytes + (16 * j + 4 * g) * 2) =
          make_uint2(pack_bf16x2(acc[i][j][0], acc[i][j][1]),
                     pack_bf16x2(acc[i][j][2], acc[i][j][3]));
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's slot is written
  __builtin_amdgcn_wave_barrier();
  const int64_t mw = m0 + wm * W4M, nw = n0 + wn * W4N;
  const int chunk = lane & 15;
  if (mw + W4M <= M && nw + W4N <= N) {
    uint16_t* dst = C + (mw + (lane >> 4)) * ldc + nw + chunk * 8;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      v4u v[W4M / 8];
#pragma unroll
      for (int u = 0; u < W4M / 8; ++u)
        v[u] = *reinterpret_cast<const v4u*>(slot + (64 * h + 4 * u + (lane >> 4)) * k4EpiRowBytes +
                                             chunk * 16);
#pragma unroll
      for (int u = 0; u < W4M / 8; ++u)
        __builtin_nontemporal_store(v[u], reinterpret_cast<v4u*>(dst + (64 * h + 4 * u) * ldc));
    }
    return;
  }
#pragma unroll
  for (int u = 0; u < W4M / 4; ++u) {
    const int row = 4 * u + (lane >> 4);
    const uint4 v = *reinterpret_cast<const uint4*>(slot + row * k4EpiRowBytes + chunk * 16);
    const int64_t m = mw + row, n = nw + chunk * 8;
    if (m >= M) continue;
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

__global__ __launch_bounds__(256) void fill_zero_bf16_kernel(uint16_t* __restrict__ C, int64_t M,
                                                             int64_t N, int64_t ldc) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= M * N) return;
  const int64_t r = i / N, c = i - r * N;
  C[r * ldc + c] = 0;
}

// Sum of the split-K partials in split order, rounded to bf16 (RNE).
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                            int64_t ldp, int64_t splits,
                                                            uint16_t* __restrict__ C, int64_t ldc,
                                                            int64_t M, int64_t N) {
  const int64_t quads = (N + 3) / 4;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= M * quads) return;
  const int64_t m = i / quads, n = (i - m * quads) * 4;
  const float* p = part + m * ldp + n;
  v4f acc = *reinterpret_cast<const v4f*>(p);
  for (int64_t s = 1; s < splits; ++s) {
    const v4f v = *reinterpret_cast<const v4f*>(p + s * M * ldp);
    acc[0] += v[0]; acc[1] += v[1]; acc[2] += v[2]; acc[3] += v[3];
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

inline bfp8_status last_launch_status() {
  return hipPeekAtLastError() == hipSuccess ? BFP8_OK : BFP8_ERR_HIP;
}

}  // namespace

template <bool A_KM, bool B_KM, bool MX>
static void launch_layout(const GemmArgs& a, dim3 grid, int tm, int tn, float* part,
                          int64_t ldp, hipStream_t stream) {
// float32 scales: the 8-wave kernel; E8M0 scales: the 4-wave kernel
#define BFP8_LAUNCH(MA, MB)                                                                  \
  do {                                                                                       \
    if constexpr (MX)                                                                        \
      gemm_mx4_kernel<A_KM, B_KM, MA, MB><<<grid, dim3(k4Threads), 0, stream>>>(             \
          a.A, a.lda, a.sA, a.B, a.ldb, a.sB, a.C, a.ldc, a.M, a.N, a.K, tm, tn, part, ldp); \
    else                                                                                     \
      gemm_kernel<A_KM, B_KM, MA, MB><<<grid, dim3(kThreads), 0, stream>>>(                  \
          a.A, a.lda, a.sA, a.B, a.ldb, a.sB, a.C, a.ldc, a.M, a.N, a.K, tm, tn, part, ldp); \
  } while (0)
  if (a.modeA == 0 && a.modeB == 1) BFP8_LAUNCH(0, 1);
  else if (a.modeA == 0 && a.modeB == 0) BFP8_LAUNCH(0, 0);
  else if (a.modeA == 1 && a.modeB == 0) BFP8_LAUNCH(1, 0);
  else if (a.modeA == 1 && a.modeB == 1) BFP8_LAUNCH(1, 1);
  else if constexpr (MX) {
    // 1x32 groups (mode 2) exist only with E8M0 scales and K-contiguous storage
    if constexpr (!A_KM && !B_KM) {
      if (a.modeA == 2 && a.modeB == 2) BFP8_LAUNCH(2, 2);
      else if (a.modeA == 2 && a.modeB == 0) BFP8_LAUNCH(2, 0);
      else if (a.modeA == 2 && a.modeB == 1) BFP8_LAUNCH(2, 1);
      else if (a.modeA == 0 && a.modeB == 2) BFP8_LAUNCH(0, 2);
      else if (a.modeA == 1 && a.modeB == 2) BFP8_LAUNCH(1, 2);
    } else if constexpr (!A_KM) {
      if (a.modeA == 2 && a.modeB == 0) BFP8_LAUNCH(2, 0);
      else if (a.modeA == 2 && a.modeB == 1) BFP8_LAUNCH(2, 1);
    }
  }
#undef BFP8_LAUNCH
}

// Split-K plan for shapes whose 256x256 tiles under-fill the chip: choose
// the split count that minimises (waves of tiles) x (K blocks per split)
// plus the cost of moving the fp32 partials.  Splits keep >= 8 K blocks.
static int64_t split_ldp(int64_t N) { return (N + 3) & ~int64_t(3); }

int gemm_splits(int64_t M, int64_t N, int64_t K) {
  constexpr double kCUs = 256.0;       // MI355X compute units
  constexpr double kBlockUs = 2.4;     // one 256x256x128 step of one tile, measured order
  constexpr double kBytesPerUs = 4.0e6;
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int64_t KB = K / BK;
  if (tiles == 0 || KB == 0) return 1;
  auto cost = [&](int64_t S) {
    const double waves = static_cast<double>((tiles * S + 255) / 256);
    double t = waves * (static_cast<double>(KB) / S) * kBlockUs;
    if (S > 1)
      t += (static_cast<double>(S) * M * split_ldp(N) * 8.0 + M * N * 2.0) / kBytesPerUs + 4.0;
    return t;
  };
  (void)kCUs;
  int best = 1;
  double best_t = cost(1);
  for (int S : {2, 3, 4, 6, 8}) {
    if (KB / S < 8) break;
    const double t = cost(S);
    if (t < best_t * 0.95) {
      best_t = t;
      best = S;
    }
  }
  return best;
}

size_t gemm_split_workspace(int64_t M, int64_t N, int64_t K) {
  const int S = gemm_splits(M, N, K);
  return S > 1 ? static_cast<size_t>(S) * M * split_ldp(N) * sizeof(float) : 0;
}

bfp8_status launch_gemm(const GemmArgs& a, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  const int64_t tiles_m = (a.M + BM - 1) / BM;
  const int64_t tiles_n = (a.N + BN - 1) / BN;
  const int64_t nblk = tiles_m * tiles_n;
  if (nblk == 0) return BFP8_OK;
  int S = gemm_splits(a.M, a.N, a.K);
  if (S > 1 && (workspace == nullptr || workspace_bytes < gemm_split_workspace(a.M, a.N, a.K)))
    S = 1;  // no room for partials: run unsplit
  float* part = S > 1 ? static_cast<float*>(workspace) : nullptr;
  const int64_t ldp = split_ldp(a.N);
  const dim3 grid(static_cast<unsigned>(nblk), static_cast<unsigned>(S));
  const int tm = static_cast<int>(tiles_m), tn = static_cast<int>(tiles_n);
  if (a.mx) {
    if (!a.a_kmajor && !a.b_kmajor) launch_layout<false, false, true>(a, grid, tm, tn, part, ldp, stream);
    else if (!a.a_kmajor && a.b_kmajor) launch_layout<false, true, true>(a, grid, tm, tn, part, ldp, stream);
    else if (a.a_kmajor && a.b_kmajor) launch_layout<true, true, true>(a, grid, tm, tn, part, ldp, stream);
    else return BFP8_ERR_LAYOUT;
  } else {
    if (!a.a_kmajor && !a.b_kmajor) launch_layout<false, false, false>(a, grid, tm, tn, part, ldp, stream);
    else if (!a.a_kmajor && a.b_kmajor) launch_layout<false, true, false>(a, grid, tm, tn, part, ldp, stream);
    else if (a.a_kmajor && a.b_kmajor) launch_layout<true, true, false>(a, grid, tm, tn, part, ldp, stream);
    else return BFP8_ERR_LAYOUT;
  }
  if (S > 1) {
    const int64_t n = a.M * ((a.N + 3) / 4);
    splitk_reduce_kernel<<<dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream>>>(
        part, ldp, S, a.C, a.ldc, a.M, a.N);
  }
  return last_launch_status();
}

bfp8_status launch_fill_bf16_zero(uint16_t* C, int64_t M, int64_t N, int64_t ldc,
                                  hipStream_t stream) {
  const int64_t n = M * N;
  if (n == 0) return BFP8_OK;
  fill_zero_bf16_kernel<<<dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream>>>(
      C, M, N, ldc);
  return last_launch_status();
}

}  // namespace bfp8
