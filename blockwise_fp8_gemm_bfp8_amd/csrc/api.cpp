// libbfp8 C ABI: argument validation and dispatch.
//
// Every entry point checks its arguments on the host before the first HIP
// call and reports problems as bfp8_status codes; the kernels themselves
// live in quantize.hip and gemm.hip.  See include/bfp8.h for the contract.

#include <stddef.h>
#include <stdint.h>

#include "common.h"

using namespace bfp8;

namespace {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int64_t elem_bytes(bfp8_in_dtype dt) { return dt == BFP8_IN_F32 ? 4 : 2; }

inline bool valid_dtype(bfp8_in_dtype dt) { return dt == BFP8_IN_BF16 || dt == BFP8_IN_F32; }

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int64_t kMaxGridY = 65535;

// Workspace: fp32 split-K partials for shapes whose output tiles under-fill
// the chip (zero for all other shapes), enough for whichever of bfp8_gemm
// and bfp8_gemm_mx takes these modes (1x32 groups: only bfp8_gemm_mx).  The
// GEMM runs unsplit when the caller passes less.
inline size_t gemm_workspace(bfp8_layout, bfp8_scale_mode modeA, bfp8_scale_mode modeB, int64_t M,
                             int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  const size_t mx = gemm_split_workspace(M, N, K, true);
  if (modeA == BFP8_SCALE_1x32 || modeB == BFP8_SCALE_1x32) return mx;
  const size_t f32 = gemm_split_workspace(M, N, K, false);
  return f32 > mx ? f32 : mx;
}

// Largest leading dimension (bytes) the GEMM addresses with 32-bit offsets.
constexpr int64_t kMaxGemmLd = int64_t(1) << 22;

inline bfp8_status check_quant_common(const void* x, bfp8_in_dtype dt, int64_t rows, int64_t cols,
                                      int64_t ldx, const void* q, int64_t ldq, const void* s) {
  if (!valid_dtype(dt)) return BFP8_ERR_DTYPE;
  if (rows < 0 || cols < 0) return BFP8_ERR_SHAPE;
  if (rows == 0 || cols == 0) return BFP8_OK;
  if (x == nullptr || q == nullptr || s == nullptr) return BFP8_ERR_NULL;
  if (!aligned16(x) || !aligned16(q) || !aligned16(s)) return BFP8_ERR_ALIGN;
  if (ldx < cols || ldq < 0) return BFP8_ERR_SHAPE;
  if ((ldx * elem_bytes(dt)) % 16 != 0 || ldq % 16 != 0) return BFP8_ERR_ALIGN;
  return BFP8_OK;
}

inline int mode_index(bfp8_scale_mode m) {
  switch (m) {
    case BFP8_SCALE_1x128: return 0;
    case BFP8_SCALE_128x128: return 1;
    case BFP8_SCALE_1x32: return 2;
    default: return 3;  // BFP8_SCALE_1x128_KMAJOR
  }
}

// Scale modes of the float32-scale GEMM.
inline bool fp32_mode(bfp8_scale_mode m) {
  return m == BFP8_SCALE_1x128 || m == BFP8_SCALE_128x128 || m == BFP8_SCALE_1x128_KMAJOR;
}

// Shape, pointer and alignment checks shared by the two GEMM entry points
// (layout and scale modes are checked by the callers), then the launch.
bfp8_status gemm_common(bfp8_layout layout, int64_t M, int64_t N, int64_t K, const uint8_t* A,
                        int64_t lda, const void* sA, bfp8_scale_mode modeA, const uint8_t* B,
                        int64_t ldb, const void* sB, bfp8_scale_mode modeB, void* C, int64_t ldc,
                        void* workspace, size_t workspace_bytes, bool mx, hipStream_t stream,
                        bool static_scratch = false) {
  if (M < 0 || N < 0 || K < 0 || K % 128 != 0) return BFP8_ERR_SHAPE;
  if (M == 0 || N == 0) return BFP8_OK;
  if (C == nullptr) return BFP8_ERR_NULL;
  if (!aligned16(C)) return BFP8_ERR_ALIGN;
  if (ldc < N) return BFP8_ERR_SHAPE;
  if (ldc % 8 != 0) return BFP8_ERR_ALIGN;
  if (cdiv(M, 256) * cdiv(N, 256) >= (int64_t(1) << 31)) return BFP8_ERR_SHAPE;
  if (K == 0) return launch_fill_bf16_zero(static_cast<uint16_t*>(C), M, N, ldc, stream);

  if (A == nullptr || B == nullptr || sA == nullptr || sB == nullptr) return BFP8_ERR_NULL;
  if (!aligned16(A) || !aligned16(B) || !aligned16(sA) || !aligned16(sB)) return BFP8_ERR_ALIGN;
  const bool a_kmajor = layout == BFP8_TN;   // A 'T' stored [K][M]
  const bool b_kmajor = layout != BFP8_NT;   // B 'N' stored [K][N]
  const int64_t a_row = a_kmajor ? M : K;    // stored row length
  const int64_t b_row = b_kmajor ? N : K;
  if (lda < a_row || ldb < b_row) return BFP8_ERR_SHAPE;
  if (lda % 16 != 0 || ldb % 16 != 0) return BFP8_ERR_ALIGN;
  if (lda > kMaxGemmLd || ldb > kMaxGemmLd) return BFP8_ERR_SHAPE;
  if (workspace != nullptr && !aligned16(workspace)) return BFP8_ERR_ALIGN;

  GemmArgs g;
  g.A = A;
  g.lda = lda;
  g.sA = sA;
  g.modeA = mode_index(modeA);
  g.a_kmajor = a_kmajor;
  g.B = B;
  g.ldb = ldb;
  g.sB = sB;
  g.modeB = mode_index(modeB);
  g.b_kmajor = b_kmajor;
  g.C = static_cast<uint16_t*>(C);
  g.ldc = ldc;
  g.M = M;
  g.N = N;
  g.K = K;
  g.mx = mx;
  if (static_scratch) return launch_gemm_static_scratch(g, stream);
  return launch_gemm(g, workspace, workspace_bytes, stream);
}

// Validate the jobs of a batched weight quantiser (each as the single call
// would) and launch them; JOB is bfp8_weight_job or bfp8_mx_weight_job.
template <typename JOB>
bfp8_status weight_batch(const JOB* jobs, int n, bfp8_in_dtype dt, int rule, hipStream_t stream) {
  if (n < 0 || n > BFP8_MAX_WEIGHT_JOBS) return BFP8_ERR_SHAPE;
  if (n == 0) return BFP8_OK;
  if (jobs == nullptr) return BFP8_ERR_NULL;
  if (!valid_dtype(dt)) return BFP8_ERR_DTYPE;
  WeightBatch b{};
  int m = 0;
  int64_t total = 0;
  for (int i = 0; i < n; ++i) {
    const JOB& j = jobs[i];
    bfp8_status st = check_quant_common(j.w, dt, j.rows, j.cols, j.ldw, j.q, j.ldq, j.s);
    if (st != BFP8_OK) return st;
    if (j.rows == 0 || j.cols == 0) continue;  // nothing to do for this job
    if (j.ldq < j.cols) return BFP8_ERR_SHAPE;
    const int64_t rb = cdiv(j.rows, 128), cb = cdiv(j.cols, 128);
    if (rb > kMaxGridY || cb >= (int64_t(1) << 31)) return BFP8_ERR_SHAPE;
    b.w[m] = j.w;
    b.q[m] = j.q;
    b.s[m] = j.s;
    b.ldw[m] = j.ldw;
    b.rows[m] = j.rows;
    b.cols[m] = j.cols;
    b.ldq[m] = j.ldq;
    b.col_blocks[m] = cb;
    b.first_block[m] = total;
    total += rb * cb;
    if (total >= (int64_t(1) << 31)) return BFP8_ERR_SHAPE;
    ++m;
  }
  b.n = m;
  b.first_block[m] = total;
  if (m == 0) return BFP8_OK;
  if (debug_checks_enabled()) {
    for (int i = 0; i < m; ++i) {
      const bfp8_status st = check_finite(b.w[i], dt, b.rows[i], b.cols[i], b.ldw[i], stream);
      if (st != BFP8_OK) return st;
    }
  }
  return launch_quantize_weight_batch(b, dt, rule, stream);
}

// Row-grouped quantiser (bfp8_quantize_act and its variants).
bfp8_status quant_act(const void* x, bfp8_in_dtype dt, int64_t rows, int64_t cols, int64_t ldx,
                      int rule, int group, uint8_t* q, int64_t ldq, void* s, bool km,
                      hipStream_t stream) {
  if (group != 32 && group != 128) return BFP8_ERR_SCALE_MODE;
  if (cols % 128 != 0 && cols > 0) return valid_dtype(dt) ? BFP8_ERR_SHAPE : BFP8_ERR_DTYPE;
  bfp8_status st = check_quant_common(x, dt, rows, cols, ldx, q, ldq, s);
  if (st != BFP8_OK || rows == 0 || cols == 0) return st;
  if (ldq < cols) return BFP8_ERR_SHAPE;
  if (rows * (cols / 128) >= (int64_t(1) << 31)) return BFP8_ERR_SHAPE;
  if (debug_checks_enabled() && (st = check_finite(x, dt, rows, cols, ldx, stream)) != BFP8_OK)
    return st;
  return launch_quantize_act(x, dt, rows, cols, ldx, rule, group, q, ldq, s, km, stream);
}

// Token-grouped quantiser written transposed (bfp8_quantize_act_transposed
// and its variants).
bfp8_status quant_act_t(const void* x, bfp8_in_dtype dt, int64_t rows, int64_t cols, int64_t ldx,
                        int rule, int group, uint8_t* qt, int64_t ldqt, void* st_, bool km,
                        hipStream_t stream) {
  if (group != 32 && group != 128) return BFP8_ERR_SCALE_MODE;
  if (rows % 128 != 0 && rows > 0) return valid_dtype(dt) ? BFP8_ERR_SHAPE : BFP8_ERR_DTYPE;
  bfp8_status st = check_quant_common(x, dt, rows, cols, ldx, qt, ldqt, st_);
  if (st != BFP8_OK || rows == 0 || cols == 0) return st;
  if (ldqt < rows) return BFP8_ERR_SHAPE;
  if (rows / 128 > kMaxGridY || cdiv(cols, 64) >= (int64_t(1) << 31)) return BFP8_ERR_SHAPE;
  if (debug_checks_enabled() && (st = check_finite(x, dt, rows, cols, ldx, stream)) != BFP8_OK)
    return st;
  return launch_quantize_act_transposed(x, dt, rows, cols, ldx, rule, group, qt, ldqt, st_, km,
                                        stream);
}

// Both layouts from one read (bfp8_quantize_act_dual and its variants).
bfp8_status quant_dual(const void* x, bfp8_in_dtype dt, int64_t rows, int64_t cols, int64_t ldx,
                       int rule, int group, uint8_t* q, int64_t ldq, void* s, uint8_t* qt,
                       int64_t ldqt, void* st_, bool km, hipStream_t stream) {
  if (group != 32 && group != 128) return BFP8_ERR_SCALE_MODE;
  if (((rows % 128 != 0 && rows > 0) || (cols % 128 != 0 && cols > 0)))
    return valid_dtype(dt) ? BFP8_ERR_SHAPE : BFP8_ERR_DTYPE;
  bfp8_status st = check_quant_common(x, dt, rows, cols, ldx, q, ldq, s);
  if (st != BFP8_OK || rows == 0 || cols == 0) return st;
  if (qt == nullptr || st_ == nullptr) return BFP8_ERR_NULL;
  if (!aligned16(qt) || !aligned16(st_)) return BFP8_ERR_ALIGN;
  if (ldq < cols || ldqt < rows) return BFP8_ERR_SHAPE;
  if (ldqt % 16 != 0) return BFP8_ERR_ALIGN;
  if (rows / 128 > kMaxGridY || cols / 128 >= (int64_t(1) << 31)) return BFP8_ERR_SHAPE;
  if (debug_checks_enabled() && (st = check_finite(x, dt, rows, cols, ldx, stream)) != BFP8_OK)
    return st;
  return launch_quantize_act_dual(x, dt, rows, cols, ldx, rule, group, q, ldq, s, qt, ldqt, st_,
                                  km, stream);
}
}  // namespace

extern "C" {

int bfp8_abi_version(void) { return BFP8_ABI_VERSION; }

const char* bfp8_status_str(bfp8_status status) {
  switch (status) {
    case BFP8_OK: return "ok";
    case BFP8_ERR_NULL: return "null pointer";
    case BFP8_ERR_SHAPE: return "invalid shape (negative size, grouped axis not a multiple of 128, "
                                "leading dimension too small, or size limit exceeded)";
    case BFP8_ERR_ALIGN: return "pointer or leading dimension not 16-byte aligned";
    case BFP8_ERR_DTYPE: return "unknown input dtype";
    case BFP8_ERR_LAYOUT: return "unknown GEMM layout";
    case BFP8_ERR_SCALE_MODE: return "unknown scale mode";
    case BFP8_ERR_WORKSPACE: return "workspace missing or too small (static-scratch GEMM: the "
                                    "split-K partials exceed BFP8_STATIC_SCRATCH_BYTES)";
    case BFP8_ERR_HIP: return "HIP launch failed";
    case BFP8_ERR_NONFINITE: return "input holds Inf or NaN (reported only with BFP8_DEBUG set)";
  }
  return "unknown status";
}

bfp8_status bfp8_quantize_act(const void* x, bfp8_in_dtype dt, int64_t rows, int64_t cols,
                              int64_t ldx, uint8_t* q, int64_t ldq, float* s,
                              hipStream_t stream) {
  return quant_act(x, dt, rows, cols, ldx, 0, 128, q, ldq, s, false, stream);
}

bfp8_status bfp8_quantize_act_kmajor(const void* x, bfp8_in_dtype dt, int64_t rows, int64_t cols,
                                     int64_t ldx, uint8_t* q, int64_t ldq, float* s,
                                     hipStream_t stream) {
  return quant_act(x, dt, rows, cols, ldx, 0, 128, q, ldq, s, true, stream);
}

bfp8_status bfp8_quantize_act_transposed(const void* x, bfp8_in_dtype dt, int64_t rows,
                                         int64_t cols, int64_t ldx, uint8_t* qt,
                                         int64_t ldqt, float* st_, hipStream_t stream) {
  return quant_act_t(x, dt, rows, cols, ldx, 0, 128, qt, ldqt, st_, false, stream);
}

bfp8_status bfp8_quantize_act_transposed_kmajor(const void* x, bfp8_in_dtype dt, int64_t rows,
                                                int64_t cols, int64_t ldx, uint8_t* qt,
                                                int64_t ldqt, float* st_, hipStream_t stream) {
  return quant_act_t(x, dt, rows, cols, ldx, 0, 128, qt, ldqt, st_, true, stream);
}

bfp8_status bfp8_quantize_act_dual(const void* x, bfp8_in_dtype dt, int64_t rows, int64_t cols,
                                   int64_t ldx, uint8_t* q, int64_t ldq, float* s, uint8_t* qt,
                                   int64_t ldqt, float* st_, hipStream_t stream) {
  return quant_dual(x, dt, rows, cols, ldx, 0, 128, q, ldq, s, qt, ldqt, st_, false, stream);
}

bfp8_status bfp8_quantize_act_dual_kmajor(const void* x, bfp8_in_dtype dt, int64_t rows,
                                          int64_t cols, int64_t ldx, uint8_t* q, int64_t ldq,
                                          float* s, uint8_t* qt, int64_t ldqt, float* st_,
                                          hipStream_t stream) {
  return quant_dual(x, dt, rows, cols, ldx, 0, 128, q, ldq, s, qt, ldqt, st_, true, stream);
}

bfp8_status bfp8_quantize_weight(const void* w, bfp8_in_dtype dt, int64_t rows, int64_t cols,
                                 int64_t ldw, uint8_t* q, int64_t ldq, float* s,
                                 hipStream_t stream) {
  bfp8_status st = check_quant_common(w, dt, rows, cols, ldw, q, ldq, s);
  if (st != BFP8_OK || rows == 0 || cols == 0) return st;
  if (ldq < cols) return BFP8_ERR_SHAPE;
  if (cdiv(rows, 128) > kMaxGridY || cdiv(cols, 128) >= (int64_t(1) << 31)) return BFP8_ERR_SHAPE;
  if (debug_checks_enabled() && (st = check_finite(w, dt, rows, cols, ldw, stream)) != BFP8_OK)
    return st;
  return launch_quantize_weight(w, dt, rows, cols, ldw, 0, q, ldq, s, stream);
}

bfp8_status bfp8_quantize_weight_batch(const bfp8_weight_job* jobs, int n, bfp8_in_dtype dt,
                                       hipStream_t stream) {
  return weight_batch(jobs, n, dt, 0, stream);
}

// ---- power-of-two (E8M0) scale rule ----------------------------------------

bfp8_status bfp8_quantize_mx_act(const void* x, bfp8_in_dtype dt, int64_t rows, int64_t cols,
                                 int64_t ldx, int group, uint8_t* q, int64_t ldq, uint8_t* s,
                                 hipStream_t stream) {
  return quant_act(x, dt, rows, cols, ldx, 1, group, q, ldq, s, false, stream);
}

bfp8_status bfp8_quantize_mx_act_transposed(const void* x, bfp8_in_dtype dt, int64_t rows,
                                            int64_t cols, int64_t ldx, int group, uint8_t* qt,
                                            int64_t ldqt, uint8_t* st_, hipStream_t stream) {
  return quant_act_t(x, dt, rows, cols, ldx, 1, group, qt, ldqt, st_, false, stream);
}

bfp8_status bfp8_quantize_mx_act_dual(const void* x, bfp8_in_dtype dt, int64_t rows, int64_t cols,
                                      int64_t ldx, int group, uint8_t* q, int64_t ldq, uint8_t* s,
                                      uint8_t* qt, int64_t ldqt, uint8_t* st_,
                                      hipStream_t stream) {
  return quant_dual(x, dt, rows, cols, ldx, 1, group, q, ldq, s, qt, ldqt, st_, false, stream);
}

bfp8_status bfp8_quantize_mx_act_dual_kmajor(const void* x, bfp8_in_dtype dt, int64_t rows,
                                             int64_t cols, int64_t ldx, uint8_t* q, int64_t ldq,
                                             uint8_t* s, uint8_t* qt, int64_t ldqt, uint8_t* st_,
                                             hipStream_t stream) {
  return quant_dual(x, dt, rows, cols, ldx, 1, 128, q, ldq, s, qt, ldqt, st_, true, stream);
}

bfp8_status bfp8_quantize_mx_weight(const void* w, bfp8_in_dtype dt, int64_t rows, int64_t cols,
                                    int64_t ldw, uint8_t* q, int64_t ldq, uint8_t* s,
                                    hipStream_t stream) {
  bfp8_status st = check_quant_common(w, dt, rows, cols, ldw, q, ldq, s);
  if (st != BFP8_OK || rows == 0 || cols == 0) return st;
  if (ldq < cols) return BFP8_ERR_SHAPE;
  if (cdiv(rows, 128) > kMaxGridY || cdiv(cols, 128) >= (int64_t(1) << 31)) return BFP8_ERR_SHAPE;
  if (debug_checks_enabled() && (st = check_finite(w, dt, rows, cols, ldw, stream)) != BFP8_OK)
    return st;
  return launch_quantize_weight(w, dt, rows, cols, ldw, 1, q, ldq, s, stream);
}

bfp8_status bfp8_quantize_mx_weight_batch(const bfp8_mx_weight_job* jobs, int n,
                                          bfp8_in_dtype dt, hipStream_t stream) {
  return weight_batch(jobs, n, dt, 1, stream);
}

size_t bfp8_gemm_workspace_bytes(bfp8_layout layout, bfp8_scale_mode modeA,
                                 bfp8_scale_mode modeB, int64_t M, int64_t N, int64_t K) {
  if (layout != BFP8_NN && layout != BFP8_NT && layout != BFP8_TN) return static_cast<size_t>(-1);
  if ((!fp32_mode(modeA) && modeA != BFP8_SCALE_1x32) ||
      (!fp32_mode(modeB) && modeB != BFP8_SCALE_1x32))
    return static_cast<size_t>(-1);
  if (M < 0 || N < 0 || K < 0 || K % 128 != 0) return static_cast<size_t>(-1);
  return gemm_workspace(layout, modeA, modeB, M, N, K);
}

bfp8_status bfp8_gemm(bfp8_layout layout, int64_t M, int64_t N, int64_t K, const uint8_t* A,
                      int64_t lda, const float* sA, bfp8_scale_mode modeA, const uint8_t* B,
                      int64_t ldb, const float* sB, bfp8_scale_mode modeB, void* C,
                      int64_t ldc, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  if (layout != BFP8_NN && layout != BFP8_NT && layout != BFP8_TN) return BFP8_ERR_LAYOUT;
  if (!fp32_mode(modeA) || !fp32_mode(modeB)) return BFP8_ERR_SCALE_MODE;
  return gemm_common(layout, M, N, K, A, lda, sA, modeA, B, ldb, sB, modeB, C, ldc, workspace,
                     workspace_bytes, false, stream);
}

bfp8_status bfp8_gemm_static_scratch(bfp8_layout layout, int64_t M, int64_t N, int64_t K,
                                     const uint8_t* A, int64_t lda, const float* sA,
                                     bfp8_scale_mode modeA, const uint8_t* B, int64_t ldb,
                                     const float* sB, bfp8_scale_mode modeB, void* C, int64_t ldc,
                                     hipStream_t stream) {
  if (layout != BFP8_NN && layout != BFP8_NT && layout != BFP8_TN) return BFP8_ERR_LAYOUT;
  if (!fp32_mode(modeA) || !fp32_mode(modeB)) return BFP8_ERR_SCALE_MODE;
  return gemm_common(layout, M, N, K, A, lda, sA, modeA, B, ldb, sB, modeB, C, ldc, nullptr, 0,
                     false, stream, true);
}

bfp8_status bfp8_gemm_mx(bfp8_layout layout, int64_t M, int64_t N, int64_t K, const uint8_t* A,
                         int64_t lda, const uint8_t* sA, bfp8_scale_mode modeA, const uint8_t* B,
                         int64_t ldb, const uint8_t* sB, bfp8_scale_mode modeB, void* C,
                         int64_t ldc, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  if (layout != BFP8_NN && layout != BFP8_NT && layout != BFP8_TN) return BFP8_ERR_LAYOUT;
  auto valid = [](bfp8_scale_mode m) { return fp32_mode(m) || m == BFP8_SCALE_1x32; };
  if (!valid(modeA) || !valid(modeB)) return BFP8_ERR_SCALE_MODE;
  // 1x32 scales only for K-contiguous operands (A of NN/NT, B of NT)
  if ((modeA == BFP8_SCALE_1x32 && layout == BFP8_TN) ||
      (modeB == BFP8_SCALE_1x32 && layout != BFP8_NT))
    return BFP8_ERR_SCALE_MODE;
  return gemm_common(layout, M, N, K, A, lda, sA, modeA, B, ldb, sB, modeB, C, ldc, workspace,
                     workspace_bytes, true, stream);
}

}  // extern "C"
