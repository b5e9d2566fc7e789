/*
 * bfp8.h -- C ABI of libbfp8: blockwise FP8 (E4M3) linear-layer kernels for
 * AMD MI355X (gfx950).
 *
 * What is computed (the pages this follows):
 *   Puro-2B paper, zh-TW translation (papers.lianghsun.dev), section 3.2
 *   "FP8 mixed-precision training": every Transformer linear layer runs on
 *   E4M3 operands; scales are computed online per local group; activations
 *   and activation gradients use 1-D groups of 128 consecutive values along
 *   the reduction dimension of the GEMM they feed; weights use 128x128 2-D
 *   blocks (the DeepSeek-V3 fine-grained design).  Puro-2B tutorial
 *   (bloombook.cn), FP8/MuonH section, MXFP figure: an element decodes as
 *   code * shared scale.
 *
 * Readings where the pages are silent (fixed here, shared with the tests):
 *   - E4M3 is the OCP "E4M3FN" format (bias 7, max 448, no infinities,
 *     S.1111.111 = NaN), from FP8 Formats for Deep Learning (Micikevicius et
 *     al., 2022), which the translation cites.
 *   - scale s = fl32(amax / 448.0f) (IEEE float32 division); element code =
 *     E4M3(saturate(fl32(x * fl32(448.0f / amax)))), round to nearest even,
 *     saturating to +-448; signed zeros kept.  amax == 0 gives s = 1.0f.
 *   - Groups with 0 < amax < 448 * 2^-126 and non-finite inputs are outside
 *     the contract (output unspecified, no fault).
 *   - GEMM: C[m][n] = bf16_rne( sum_kb P_kb[m][n] * sA * sB ), where P_kb is
 *     the fp32 MFMA partial over one 128-deep K block and the sum is an fp32
 *     accumulator ("promotion" once per 128-K block).
 *
 * Layout letters (a reading; all matrices are row-major in memory):
 *   A 'N' stored [M][K] (lda >= K);   A 'T' stored [K][M] (lda >= M)
 *   B 'N' stored [K][N] (ldb >= N);   B 'T' stored [N][K] (ldb >= K)
 *   The three training GEMMs:
 *     fprop  Y  = X  W^T   : NT, A = quantize_act(X) [M][in],
 *                             B = quantize_weight(W) [out][in]
 *     dgrad  dX = dY W     : NN, A = quantize_act(dY) [M][out],
 *                             B = quantize_weight(W) as stored ([K=out][N=in])
 *     wgrad  dW = dY^T X   : NT, A = quantize_act_transposed(dY) [out][M],
 *                             B = quantize_act_transposed(X) [in][M]
 *   TN (A stored [K][M], B stored [K][N]) is provided for callers that keep
 *   token-grouped data in natural order.
 *
 * Scale tensors are dense row-major float32 arrays in the orientation of the
 * stored operand, with the grouped axis divided by 128:
 *   act mode (1x128 along K):  A 'N' [M][K/128]   A 'T' [K/128][M]
 *                              B 'T' [N][K/128]   B 'N' [K/128][N]
 *   block mode (128x128):      A 'N' [ceil(M/128)][K/128]   A 'T' [K/128][ceil(M/128)]
 *                              B 'T' [ceil(N/128)][K/128]   B 'N' [K/128][ceil(N/128)]
 *   act mode, K-block major (BFP8_SCALE_1x128_KMAJOR):  A [K/128][M]   B [K/128][N]
 *     for either orientation of the codes: the scales of one K block are
 *     contiguous, so each K block's scales are read as a few cache lines
 *     (for a K-major operand this is the act-mode layout itself).
 *
 * Ownership and threading: the caller allocates every buffer (inputs,
 * codes, scales, outputs, workspace) in device memory.  The library keeps
 * no state, allocates nothing, never synchronises, and enqueues all work on
 * the given stream; calls on different streams may run concurrently.
 *
 * Errors: every entry point validates its arguments on the host BEFORE any
 * HIP call and returns a bfp8_status; nothing aborts or throws.  A launch
 * failure returns BFP8_ERR_HIP.  The status is that of the call's own
 * launches (the return value of hipLaunchKernel), never an error an earlier,
 * unrelated HIP call left behind.  HIP also records a failed launch as the
 * calling thread's last error; the library never clears it, the caller reads
 * and clears it with hipGetLastError.
 *
 * Debug mode: with the environment variable BFP8_DEBUG set (to anything but
 * "" or "0"; read once per process), every quantiser first scans its input
 * for Inf / NaN, waits for the answer (a stream synchronisation) and returns
 * BFP8_ERR_NONFINITE, launching nothing, if it finds one.  Off by default:
 * the check costs a read of the input and a host round trip, and breaks the
 * never-synchronise contract, so it is for debugging only (not under graph
 * capture; concurrent debug-mode calls on one GPU share one flag word).
 * Without it, non-finite inputs are outside the contract (output
 * unspecified, no fault).
 *
 * Preconditions common to all calls: pointers of non-empty operands are
 * non-null and 16-byte aligned; leading dimensions are >= the row length
 * and keep every row 16-byte aligned (multiples of 16 bytes); sizes >= 0.
 * Empty problems (a zero extent) are valid and launch nothing, except a
 * GEMM with K == 0 and M, N > 0, which writes C = 0.
 */
#ifndef BFP8_H_
#define BFP8_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BFP8_ABI_VERSION 5

typedef enum {
  BFP8_OK = 0,
  BFP8_ERR_NULL = 1,        /* a required pointer is NULL                  */
  BFP8_ERR_SHAPE = 2,       /* negative size, or a grouped axis % 128 != 0 */
  BFP8_ERR_ALIGN = 3,       /* pointer or leading dimension misaligned     */
  BFP8_ERR_DTYPE = 4,       /* unknown input dtype                         */
  BFP8_ERR_LAYOUT = 5,      /* unknown GEMM layout                         */
  BFP8_ERR_SCALE_MODE = 6,  /* unknown scale mode                          */
  BFP8_ERR_WORKSPACE = 7,   /* workspace smaller than required             */
  BFP8_ERR_HIP = 8,         /* a HIP launch failed                         */
  BFP8_ERR_NONFINITE = 9    /* Inf / NaN input (only with BFP8_DEBUG set)  */
} bfp8_status;

typedef enum { BFP8_IN_BF16 = 0, BFP8_IN_F32 = 1 } bfp8_in_dtype;
typedef enum { BFP8_NN = 0, BFP8_NT = 1, BFP8_TN = 2 } bfp8_layout;
typedef enum {
  BFP8_SCALE_1x128 = 0,        /* 1 x 128 groups along K                          */
  BFP8_SCALE_128x128 = 1,      /* 128 x 128 blocks                                */
  BFP8_SCALE_1x32 = 2,         /* 1 x 32 groups along K (E8M0 scales only: MXFP8) */
  BFP8_SCALE_1x128_KMAJOR = 3  /* 1 x 128 groups along K, scale tensor stored
                                  [K/128][rows] whatever the code orientation */
} bfp8_scale_mode;

/*
 * Activation / activation-gradient quantiser: 1x128 groups along each row.
 * (Puro-2B translation, section 3.2: 1-D groups of 128 consecutive values
 * along the GEMM reduction dimension; here the reduction axis is the
 * contiguous axis.)
 *
 *   x   [rows][ldx] elements of dtype dt (bf16 or fp32); cols % 128 == 0
 *   q   [rows][ldq] uint8 E4M3 codes (ldq >= cols)
 *   s   [rows][cols/128] float32 scales, dense
 * rows may be any value >= 0 (no tail restriction on the token axis).
 */
bfp8_status bfp8_quantize_act(const void* x, bfp8_in_dtype dt, int64_t rows, int64_t cols,
                              int64_t ldx, uint8_t* q, int64_t ldq, float* s,
                              hipStream_t stream);

/*
 * Token-axis quantiser for wgrad operands, written transposed.
 * (Puro-2B translation, section 3.2: for the weight-gradient GEMM the
 * reduction dimension is the token axis, so the 1x128 groups run along
 * tokens.)  Bytes and scales equal bfp8_quantize_act applied to x^T.
 *
 *   x   [rows][ldx] (rows = tokens, rows % 128 == 0; cols = channels, any)
 *   qt  [cols][ldqt] uint8 (ldqt >= rows): qt[c][m] is the code of x[m][c]
 *   st  [cols][rows/128] float32: scale of tokens 128b..128b+127 of channel c
 */
bfp8_status bfp8_quantize_act_transposed(const void* x, bfp8_in_dtype dt, int64_t rows,
                                         int64_t cols, int64_t ldx, uint8_t* qt,
                                         int64_t ldqt, float* st, hipStream_t stream);

/*
 * Both activation layouts from one read: the row-grouped codes of
 * bfp8_quantize_act AND the token-grouped transposed codes of
 * bfp8_quantize_act_transposed, bit-identical to calling the two.
 * (Puro-2B translation, section 3.2: FP8 is the online compute and
 * activation-storage format -- the fprop quantisation of X keeps the codes
 * the wgrad GEMM needs, and one pass over dY serves both dgrad and wgrad.)
 *
 *   x   [rows][ldx] (rows = tokens, cols = channels; both % 128 == 0)
 *   q   [rows][ldq] uint8,  s  [rows][cols/128] float32   (as quantize_act)
 *   qt  [cols][ldqt] uint8, st [cols][rows/128] float32   (as quantize_act_transposed)
 */
bfp8_status bfp8_quantize_act_dual(const void* x, bfp8_in_dtype dt, int64_t rows, int64_t cols,
                                   int64_t ldx, uint8_t* q, int64_t ldq, float* s, uint8_t* qt,
                                   int64_t ldqt, float* st, hipStream_t stream);

/*
 * The same three quantisers with their scale tensors stored K-block major,
 * the layout of BFP8_SCALE_1x128_KMAJOR: the tensor's rows are the groups
 * along the grouped axis, its columns the other axis.  Codes are those of
 * the calls above, byte for byte; every scale is the same value, transposed:
 *   bfp8_quantize_act_kmajor             s  [cols/128][rows]
 *   bfp8_quantize_act_transposed_kmajor  st [rows/128][cols]
 *   bfp8_quantize_act_dual_kmajor        s  [cols/128][rows], st [rows/128][cols]
 * (Puro-2B translation, section 3.2: the same groups along the reduction
 * dimension.)  A quantiser then writes each tile's scales as one contiguous
 * run, and the GEMM reads each K block's scales as a few cache lines, where
 * [rows][groups] spreads them over one cache line per row.  Arguments and
 * errors as for the calls above.
 */
bfp8_status bfp8_quantize_act_kmajor(const void* x, bfp8_in_dtype dt, int64_t rows, int64_t cols,
                                     int64_t ldx, uint8_t* q, int64_t ldq, float* s,
                                     hipStream_t stream);
bfp8_status bfp8_quantize_act_transposed_kmajor(const void* x, bfp8_in_dtype dt, int64_t rows,
                                                int64_t cols, int64_t ldx, uint8_t* qt,
                                                int64_t ldqt, float* st, hipStream_t stream);
bfp8_status bfp8_quantize_act_dual_kmajor(const void* x, bfp8_in_dtype dt, int64_t rows,
                                          int64_t cols, int64_t ldx, uint8_t* q, int64_t ldq,
                                          float* s, uint8_t* qt, int64_t ldqt, float* st,
                                          hipStream_t stream);

/*
 * Weight quantiser: one scale per 128x128 block.
 * (Puro-2B translation, section 3.2; Puro-2B tutorial, FP8/MuonH section:
 * weights are cut into 128x128 2-D blocks that share one scale.)
 *
 *   w   [rows][ldw] (any rows, cols >= 0; edge blocks may be partial and
 *       take the amax of their valid elements only)
 *   q   [rows][ldq] uint8
 *   s   [ceil(rows/128)][ceil(cols/128)] float32, dense
 */
bfp8_status bfp8_quantize_weight(const void* w, bfp8_in_dtype dt, int64_t rows, int64_t cols,
                                 int64_t ldw, uint8_t* q, int64_t ldq, float* s,
                                 hipStream_t stream);

/*
 * Batched weight quantiser: several weights in one launch, each job's result
 * bit-identical to bfp8_quantize_weight on it.  The same 128x128 blocks
 * (Puro-2B translation, section 3.2).  The blocks of all jobs run side by
 * side, so weights too small to fill the GPU alone (for example 2048 x 2048:
 * 256 blocks) do not leave it idle.
 *
 *   jobs  host array of n job descriptions (read during the call only); each
 *         job's arguments mean what bfp8_quantize_weight's do, and all jobs
 *         share the input dtype dt
 *   n     0 .. BFP8_MAX_WEIGHT_JOBS
 * Every job is validated as bfp8_quantize_weight validates its arguments;
 * the first failing job's status is returned and nothing is launched.
 * Jobs must not overlap in their outputs.
 */
#define BFP8_MAX_WEIGHT_JOBS 16
typedef struct {
  const void* w;
  int64_t rows, cols, ldw;
  uint8_t* q;
  int64_t ldq;
  float* s;
} bfp8_weight_job;
bfp8_status bfp8_quantize_weight_batch(const bfp8_weight_job* jobs, int n, bfp8_in_dtype dt,
                                       hipStream_t stream);

/*
 * Blockwise FP8 GEMM with per-128-K-block scale promotion and bf16 output.
 * (Puro-2B translation, section 2 and section 3.2: the main Transformer
 * linear-layer GEMMs run in blockwise FP8; non-FP8 tensors stay in BF16.)
 *
 *   C[m][n] (bf16, [M][ldc], ldc >= N) = sum over 128-deep K blocks of the
 *   fp32 partial times sA * sB, accumulated in fp32, rounded to bf16 (RNE).
 *   K % 128 == 0; M and N may have ragged tails.  modeA / modeB select the
 *   scale layout of each operand (see the table at the top of this file).
 *   Every stored row of A and B must be backed by a full leading dimension
 *   of memory (lda / ldb bytes, including the last row): a K-major operand
 *   with a ragged extent is read in whole 16-byte chunks.  lda, ldb <= 2^22.
 *   workspace: device memory for fp32 split-K partials, used when the
 *   problem's 256x256 output tiles would under-fill the GPU (size from
 *   bfp8_gemm_workspace_bytes; 16-byte aligned).  It may be NULL or smaller
 *   than that size: the GEMM then runs unsplit (same contract, slower).
 *   With a split the partials are summed in a fixed order, so results are
 *   deterministic either way.
 */
bfp8_status bfp8_gemm(bfp8_layout layout, int64_t M, int64_t N, int64_t K, const uint8_t* A,
                      int64_t lda, const float* sA, bfp8_scale_mode modeA, const uint8_t* B,
                      int64_t ldb, const float* sB, bfp8_scale_mode modeB, void* C,
                      int64_t ldc, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/*
 * ---- Power-of-two (E8M0) scales: the MXFP8 form of the same recipe --------
 * (Puro-2B translation, section 3.2: on SM120 every logical block scale was
 * constrained to a power of two and ran on the native MXFP8 path; Puro-2B
 * tutorial, MXFP figure: MXFP8 shares one scale per 32 elements.)
 *
 * Scale rule (a reading): e = the least integer with 448 * 2^e >= amax of the
 * group, clamped to [-127, 127] (0 for an all-zero group); the scale is the
 * E8M0 byte e + 127 (value 2^(byte - 127)); codes are the round-to-nearest-
 * even E4M3 cast of x * 2^-e (no element saturates).  Groups whose amax is
 * below 2^-126 and non-finite inputs are outside the contract.
 * Scale tensors are dense row-major uint8 arrays with the same shapes as the
 * float32 scale tensors above, the grouped axis divided by the group length
 * (32 or 128).  Errors and ownership as above; `group` other than 32 or 128
 * returns BFP8_ERR_SCALE_MODE.
 */

/* Rows quantised in groups of `group` (32 or 128) consecutive values:
 * q [rows][ldq], s [rows][cols/group].  cols % 128 == 0. */
bfp8_status bfp8_quantize_mx_act(const void* x, bfp8_in_dtype dt, int64_t rows, int64_t cols,
                                 int64_t ldx, int group, uint8_t* q, int64_t ldq, uint8_t* s,
                                 hipStream_t stream);

/* Token-axis groups of `group` tokens, written transposed:
 * qt [cols][ldqt], st [cols][rows/group].  rows % 128 == 0. */
bfp8_status bfp8_quantize_mx_act_transposed(const void* x, bfp8_in_dtype dt, int64_t rows,
                                            int64_t cols, int64_t ldx, int group, uint8_t* qt,
                                            int64_t ldqt, uint8_t* st, hipStream_t stream);

/* Both of the above from one read (rows and cols % 128 == 0). */
bfp8_status bfp8_quantize_mx_act_dual(const void* x, bfp8_in_dtype dt, int64_t rows, int64_t cols,
                                      int64_t ldx, int group, uint8_t* q, int64_t ldq, uint8_t* s,
                                      uint8_t* qt, int64_t ldqt, uint8_t* st, hipStream_t stream);

/* bfp8_quantize_mx_act_dual with group 128 and both scale tensors stored
 * K-block major (s [cols/128][rows], st [rows/128][cols] E8M0 bytes), the
 * layout of BFP8_SCALE_1x128_KMAJOR. */
bfp8_status bfp8_quantize_mx_act_dual_kmajor(const void* x, bfp8_in_dtype dt, int64_t rows,
                                             int64_t cols, int64_t ldx, uint8_t* q, int64_t ldq,
                                             uint8_t* s, uint8_t* qt, int64_t ldqt, uint8_t* st,
                                             hipStream_t stream);

/* 128x128 weight blocks: q [rows][ldq], s [ceil(rows/128)][ceil(cols/128)]. */
bfp8_status bfp8_quantize_mx_weight(const void* w, bfp8_in_dtype dt, int64_t rows, int64_t cols,
                                    int64_t ldw, uint8_t* q, int64_t ldq, uint8_t* s,
                                    hipStream_t stream);

/* Batched form of bfp8_quantize_mx_weight, as bfp8_quantize_weight_batch is
 * of bfp8_quantize_weight: up to BFP8_MAX_WEIGHT_JOBS weights in one launch,
 * each job bit-identical to the single call, validated the same way. */
typedef struct {
  const void* w;
  int64_t rows, cols, ldw;
  uint8_t* q;
  int64_t ldq;
  uint8_t* s;
} bfp8_mx_weight_job;
bfp8_status bfp8_quantize_mx_weight_batch(const bfp8_mx_weight_job* jobs, int n,
                                          bfp8_in_dtype dt, hipStream_t stream);

/*
 * GEMM on E8M0-scaled operands: C[m][n] = sum over K of dec(A) * dec(B) with
 * each product scaled by its two groups' powers of two, accumulated in fp32,
 * rounded to bf16 (RNE).  On gfx950 the scales ride in the matrix-core
 * instruction itself (v_mfma_scale_f32_16x16x128_f8f6f4), so the exact
 * power-of-two scaling replaces the per-128-K promotion of bfp8_gemm.
 * Same layouts, shapes, leading-dimension and workspace rules as bfp8_gemm
 * (the workspace may also receive a copy of part of A's scales: under the
 * plan that splits only the tiles past whole waves, the split rows run as a
 * GEMM of their own, and K-block-major scales of those rows are copied for
 * it; bfp8_gemm_workspace_bytes counts this);
 * scale tensors are uint8 E8M0 in the layouts of the table at the top of
 * this file, with BFP8_SCALE_1x32 as [rows][K/32] (K-contiguous operands
 * only: A of NN/NT, B of NT; otherwise BFP8_ERR_SCALE_MODE).  Each scale
 * tensor must be readable up to the next multiple of 4 bytes past its end
 * (scales are fetched as aligned 32-bit words).
 */
bfp8_status bfp8_gemm_mx(bfp8_layout layout, int64_t M, int64_t N, int64_t K, const uint8_t* A,
                         int64_t lda, const uint8_t* sA, bfp8_scale_mode modeA, const uint8_t* B,
                         int64_t ldb, const uint8_t* sB, bfp8_scale_mode modeB, void* C,
                         int64_t ldc, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: bfp8_gemm
 * with no workspace argument and the same split-K plan, its float32 split-K
 * partials kept in a static device array of the library (one array of
 * BFP8_STATIC_SCRATCH_BYTES per GPU the library runs on, held until the
 * process ends).  Results are bit-identical to bfp8_gemm given the workspace
 * bfp8_gemm_workspace_bytes asks for.  Arguments, layouts and errors as for
 * bfp8_gemm; in addition BFP8_ERR_WORKSPACE, before any HIP call and with
 * nothing launched, when bfp8_gemm's split-K partials for the problem
 * (at most bfp8_gemm_workspace_bytes) exceed BFP8_STATIC_SCRATCH_BYTES -- such a
 * problem can run allocation-free through bfp8_gemm with a NULL workspace
 * (unsplit).  Allocates nothing and never synchronises.  The array's device
 * address is looked up on the calling thread's current device, which must be
 * the stream's device.  Every call on one GPU uses that GPU's one array:
 * calls that overlap in time on one GPU (concurrent streams, or threads)
 * race on it and must be serialised by the caller.
 */
#define BFP8_STATIC_SCRATCH_BYTES (64u << 20)
bfp8_status bfp8_gemm_static_scratch(bfp8_layout layout, int64_t M, int64_t N, int64_t K,
                                     const uint8_t* A, int64_t lda, const float* sA,
                                     bfp8_scale_mode modeA, const uint8_t* B, int64_t ldb,
                                     const float* sB, bfp8_scale_mode modeB, void* C, int64_t ldc,
                                     hipStream_t stream);

/* Workspace bytes that let bfp8_gemm and bfp8_gemm_mx use their split-K
 * plans for this problem (0 when both run unsplit; the larger of the two
 * when the plans differ: both may run whole waves of tiles unsplit and split
 * only the tiles of a last, partial wave, bfp8_gemm_mx only when M is a
 * multiple of 256).  Returns (size_t)-1 for an invalid layout, scale mode or
 * size. */
size_t bfp8_gemm_workspace_bytes(bfp8_layout layout, bfp8_scale_mode modeA,
                                 bfp8_scale_mode modeB, int64_t M, int64_t N, int64_t K);

/* Static description of a status code; never NULL. */
const char* bfp8_status_str(bfp8_status status);

/* BFP8_ABI_VERSION of the built library. */
int bfp8_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BFP8_H_ */
