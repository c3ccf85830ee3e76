// Device-side building blocks of the linear_logp kernels (gfx950 only).
//
// Primitives and rounding points are fixed here once and used by every
// kernel (forward, range partial, merge, backward recompute), so that the
// same logit always produces the same bits on every path.  The pages make
// the primitives and rounding points part of the numerical contract
// ("vLLM RL-Kernel v0.1.0: Bitwise Train-Rollout Consistency on ROCm",
// "The Numerical Execution Contract", items 5 and 6) and name compiler
// fusion and math-function implementations as sources of last-bit drift
// ("Implementation on ROCm", "Math and Fusion").  Hence: the hardware
// exp2/log2 instructions with separately rounded scale factors, and the
// whole library is compiled with -ffp-contract=off.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rlk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kNSplit = 32;   // vocabulary splits (fixed by the contract)
constexpr int kChunk = 128;   // columns per chunk (fixed by the contract)

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

// exp(x) := exp2(x * log2 e): one rounded multiply, then v_exp_f32.
__device__ __forceinline__ float rlk_exp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

// log(x) := log2(x) * ln 2: v_log_f32, then one rounded multiply.
__device__ __forceinline__ float rlk_log(float x) { return __builtin_amdgcn_logf(x) * kLn2; }

// (max, sum of exp(z - max)) statistics of a set of logits.
struct MS {
  float m, s;
};

__device__ __forceinline__ MS ms_identity() { return {-INFINITY, 0.f}; }

// The one combination rule for statistics of two disjoint logit sets,
// a = lower vocabulary indices, b = higher ones:
//   m = max(ma, mb),  s = (sa * e(ma - m)) + (sb * e(mb - m)),
// two rounded products and one rounded add.  One exponent argument is
// exactly 0 (factor exactly 1).  Combining two empty sets gives the empty
// set without ever evaluating (-inf) - (-inf).
__device__ __forceinline__ MS ms_combine(MS a, MS b) {
  const float m = fmaxf(a.m, b.m);
  if (m == -INFINITY) return ms_identity();
  const float pa = a.s * rlk_exp(a.m - m);
  const float pb = b.s * rlk_exp(b.m - m);
  return {m, pa + pb};
}

// Pairwise tree over v[0..n), n a power of two <= 32: level by level,
// v[i] = v[i] (+) v[i + w] for i a multiple of 2w.  Left operand = lower
// vocabulary.  Result in v[0].
__device__ __forceinline__ MS ms_pairwise_tree(MS* v, int n) {
  for (int w = 1; w < n; w <<= 1)
    for (int i = 0; i + w < n; i += 2 * w) v[i] = ms_combine(v[i], v[i + w]);
  return v[0];
}

// Two fp32 values rounded to bf16 (round to nearest even, v_cvt_pk_bf16_f32),
// packed with `lo` in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

// Lane pair (l, l ^ 32): the value of lane l & 31 (lo) and of lane
// (l & 31) + 32 (hi), in both lanes (v_permlane32_swap).
__device__ __forceinline__ void lane_halves(float v, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}

}  // namespace rlk
