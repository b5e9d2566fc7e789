// Internal helpers shared by the libbfp8 HIP sources (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <utility>

#include "bfp8.h"

namespace bfp8 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kGroup = 128;        // elements per activation group / block edge
constexpr float kE4M3Max = 448.0f; // largest finite OCP E4M3 value

// Exact widening of a bfloat16 bit pattern to float32.
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// Two float32 -> packed bfloat16 pair (low half = a), round to nearest
// even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f2_ __attribute__((ext_vector_type(2)));
  typedef __bf16 bf2_ __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2_{a, b}), bf2_));
}

// Group scale and its reciprocal multiplier.  s = fl32(amax / 448) and
// inv = fl32(448 / amax), both IEEE-rounded divisions; an all-zero group
// gets s = inv = 1 so its (signed) zeros encode as zeros.
__device__ __forceinline__ void group_scale(float amax, float& s, float& inv) {
  if (amax == 0.0f) {
    s = 1.0f;
    inv = 1.0f;
  } else {
    s = amax / kE4M3Max;
    inv = kE4M3Max / amax;
  }
}

// Power-of-two group scale (E8M0): e = the least integer with
// 448 * 2^e >= amax, clamped to [-127, 127], found from amax's float32 bit
// fields (448 = 1.75 * 2^8: a mantissa above 1.75 needs one more binade);
// an all-zero group gets e = 0.  Returns the scale byte e + 127 and sets
// inv = 2^-e exactly.  (A float32-subnormal amax is outside the contract;
// it gets the clamped e = -127.)
__device__ __forceinline__ uint8_t group_scale_pow2(float amax, float& inv) {
  const uint32_t bits = __float_as_uint(amax);
  const int biased = static_cast<int>((bits >> 23) & 0xFFu);
  int e;
  if (amax == 0.0f) {
    e = 0;
  } else if (biased == 0) {
    e = -127;
  } else {
    e = biased - 127 - 8 + ((bits & 0x7FFFFFu) > 0x600000u ? 1 : 0);
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
  }
  inv = __uint_as_float(static_cast<uint32_t>(127 - e) << 23);
  return static_cast<uint8_t>(e + 127);
}

// The two scale rules behind one interface: RULE 0 = float32 amax / 448
// (scale type float), RULE 1 = power of two stored as an E8M0 byte.
template <int RULE>
struct ScaleRule;
template <>
struct ScaleRule<0> {
  typedef float type;
  static __device__ __forceinline__ float make(float amax, float& inv) {
    float s;
    group_scale(amax, s, inv);
    return s;
  }
};
template <>
struct ScaleRule<1> {
  typedef uint8_t type;
  static __device__ __forceinline__ uint8_t make(float amax, float& inv) {
    return group_scale_pow2(amax, inv);
  }
};

// Four float32 -> four E4M3 codes packed little-endian in one dword.
// Saturation is done by the clamp (the conversion instruction's own
// overflow result is NaN); the conversion rounds to nearest even and keeps
// the sign of zero.
__device__ __forceinline__ uint32_t encode4(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -kE4M3Max), kE4M3Max);
  b = fminf(fmaxf(b, -kE4M3Max), kE4M3Max);
  c = fminf(fmaxf(c, -kE4M3Max), kE4M3Max);
  d = fminf(fmaxf(d, -kE4M3Max), kE4M3Max);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return static_cast<uint32_t>(w);
}

// Max over the 16 lanes of a DPP row (the value is replicated to all 16).
__device__ __forceinline__ float row16_max(float v) {
  // quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));
  return v;
}

// Max over the 4 lanes of a quad.
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
  return v;
}

// Max over all 64 lanes of a wave (result valid in every lane).
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

// Kernel launch that reports this launch's own status: the return value of
// hipLaunchKernel, not HIP's thread-wide last error (which an unrelated
// earlier call may have left set).  The arguments are converted to the
// kernel's parameter types before their addresses are taken.  On failure
// HIP also records the error as the calling thread's last error; the caller
// reads and clears it with hipGetLastError.
template <typename... KArgs, size_t... I>
inline bfp8_status launch_packed(void (*kernel)(KArgs...), dim3 grid, dim3 block,
                                 hipStream_t stream, std::tuple<KArgs...>& vals,
                                 std::index_sequence<I...>) {
  void* argv[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1] = {static_cast<void*>(&std::get<I>(vals))...};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, 0, stream) ==
                 hipSuccess
             ? BFP8_OK
             : BFP8_ERR_HIP;
}
template <typename... KArgs, typename... Args>
inline bfp8_status launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t stream,
                          Args&&... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
  std::tuple<KArgs...> vals(static_cast<KArgs>(std::forward<Args>(args))...);
  return launch_packed(kernel, grid, block, stream, vals, std::index_sequence_for<KArgs...>{});
}

// Opt-in input check (environment variable BFP8_DEBUG set to anything but
// "" or "0", read once per process): true when enabled.
bool debug_checks_enabled();
// Scan x [rows][ldx] for Inf / NaN on `stream`, wait for the result, and
// return BFP8_ERR_NONFINITE if one is found (BFP8_ERR_HIP on a HIP failure).
bfp8_status check_finite(const void* x, bfp8_in_dtype dt, int64_t rows, int64_t cols, int64_t ldx,
                         hipStream_t stream);

// Host-side launch helpers (defined in the .hip files).  `rule` selects the
// scale rule (0: float32 amax/448, 1: power-of-two E8M0 byte) and `s` points
// to float or uint8_t scales accordingly; `group` is the group length along
// the grouped axis (128, or 32 for the power-of-two rule).  `km` (group 128
// only) stores the scale tensors K-block major: [groups][rows] instead of
// [rows][groups].
bfp8_status launch_quantize_act(const void* x, bfp8_in_dtype dt, int64_t rows, int64_t cols,
                                int64_t ldx, int rule, int group, uint8_t* q, int64_t ldq,
                                void* s, bool km, hipStream_t stream);
bfp8_status launch_quantize_act_transposed(const void* x, bfp8_in_dtype dt, int64_t rows,
                                           int64_t cols, int64_t ldx, int rule, int group,
                                           uint8_t* qt, int64_t ldqt, void* st, bool km,
                                           hipStream_t stream);
bfp8_status launch_quantize_act_dual(const void* x, bfp8_in_dtype dt, int64_t rows, int64_t cols,
                                     int64_t ldx, int rule, int group, uint8_t* q, int64_t ldq,
                                     void* s, uint8_t* qt, int64_t ldqt, void* st, bool km,
                                     hipStream_t stream);
bfp8_status launch_quantize_weight(const void* w, bfp8_in_dtype dt, int64_t rows, int64_t cols,
                                   int64_t ldw, int rule, uint8_t* q, int64_t ldq, void* s,
                                   hipStream_t stream);

// Kernel argument of the batched weight quantiser: the jobs' pointers and
// sizes (scales float32 or E8M0 bytes, by the launch's rule), and the flat
// index of each job's first 128x128 block (first_block[n] = total blocks).
constexpr int kMaxWeightJobs = BFP8_MAX_WEIGHT_JOBS;
struct WeightBatch {
  const void* w[kMaxWeightJobs];
  uint8_t* q[kMaxWeightJobs];
  void* s[kMaxWeightJobs];
  int64_t ldw[kMaxWeightJobs];
  int64_t rows[kMaxWeightJobs];
  int64_t cols[kMaxWeightJobs];
  int64_t ldq[kMaxWeightJobs];
  int64_t col_blocks[kMaxWeightJobs];
  int64_t first_block[kMaxWeightJobs + 1];
  int n;
};
bfp8_status launch_quantize_weight_batch(const WeightBatch& b, bfp8_in_dtype dt, int rule,
                                         hipStream_t stream);

struct GemmArgs {
  // Operands as stored.  a_kmajor: A stored [K][M] (else [M][K]);
  // b_kmajor: B stored [K][N] (else [N][K]).  Scale layouts follow the
  // stored orientation (see include/bfp8.h).
  const uint8_t* A;
  int64_t lda;
  const void* sA;  // float32 scales, or E8M0 bytes when mx
  int modeA;  // 0 = 1x128 act groups, 1 = 128x128 blocks, 2 = 1x32 groups (mx only)
  bool a_kmajor;
  const uint8_t* B;
  int64_t ldb;
  const void* sB;
  int modeB;
  bool b_kmajor;
  uint16_t* C;  // bf16 bits
  int64_t ldc;
  int64_t M, N, K;
  bool mx;  // power-of-two (E8M0) scales applied by the MFMA
};

bfp8_status launch_gemm(const GemmArgs& a, void* workspace, size_t workspace_bytes,
                        hipStream_t stream);
// bfp8_gemm with its split-K partials in the library's static device array:
// BFP8_ERR_WORKSPACE (before any HIP call) if they would not fit.
bfp8_status launch_gemm_static_scratch(const GemmArgs& a, hipStream_t stream);
// Split-K plan of an M x N x K GEMM: logical tiles [0, full) run unsplit,
// the others in `splits` ranges of K blocks (splits == 1: nothing is split,
// full == tiles); the split tiles cover output rows [row0, M).
struct GemmPlan {
  int64_t full;
  int splits;
  int64_t row0;
};
// mx: the plan of the power-of-two (E8M0) kernel, which splits all tiles alike.
GemmPlan gemm_plan(int64_t M, int64_t N, int64_t K, bool mx);
// fp32 partials of that plan: splits x (M - row0) rows x ceil4(N) floats
size_t gemm_split_workspace(int64_t M, int64_t N, int64_t K, bool mx);
bfp8_status launch_fill_bf16_zero(uint16_t* C, int64_t M, int64_t N, int64_t ldc,
                                  hipStream_t stream);

}  // namespace bfp8
