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

// Round fp32 to bf16, round-to-nearest-even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------------------
// NT tile engine: C[128 x 128] = A[128 x K] * B[128 x K]^T, bf16 in, fp32 out.
//
// Both operands are K-contiguous rows (the natural layout of h [T,H] and
// W [V,H]).  256 threads = 4 waves; wave w owns C rows 32w..32w+31 and all
// 128 columns as four 32x32 blocks, so a chunk row lives in one wave.
// Per 16-wide k step each wave issues one v_mfma_f32_32x32x16_bf16 per
// column block, always into the same accumulator: one fp32 chain per
// element, k ascending.  The tiling (rows per wave, waves per block, LDS
// staging) does not change any result bit.
//
// MFMA register layouts used (32x32x16 bf16):
//   A operand, lane l: row (l & 31), k = 8*(l >> 5) + 0..7 of the k step
//   B operand, lane l: col (l & 31), same k
//   D, lane l, element r (0..15): row 8*(r>>2) + 4*(l>>5) + (r&3), col l&31
// A and B use the same k assignment, so the product sums exactly the 16 k
// values of the step whatever the hardware's internal k order is.
//
// LDS: two stages of A and B tiles, 128 rows x 64 k each (16 KB), rows of
// eight 16-byte segments stored at segment (seg ^ (row & 7)) so that the
// 32 lanes reading one k segment of 32 consecutive rows spread over banks.
// ---------------------------------------------------------------------------
constexpr int kBM = 128, kBN = 128, kBK = 64, kThreads = 256;
constexpr int kLdsStage = 128 * 8;  // uint4 per operand per stage

__device__ __forceinline__ int lds_slot(int row, int seg) { return row * 8 + (seg ^ (row & 7)); }

// One k-block (64 wide) of MFMAs from LDS stage `st`.
__device__ __forceinline__ void mma_kblock(const uint4* __restrict__ sA, const uint4* __restrict__ sB, int arow,
                                           int lane, int khalf, f32x16 acc[4]) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int sg = 2 * kk + khalf;
    const bf16x8 a = __builtin_bit_cast(bf16x8, sA[lds_slot(arow, sg)]);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int bcol = 32 * b + (lane & 31);
      const bf16x8 bv = __builtin_bit_cast(bf16x8, sB[lds_slot(bcol, sg)]);
      acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bv, acc[b], 0, 0, 0);
    }
  }
}

// rowA / rowB: global row pointers (bf16, K-contiguous) of the four rows
// this thread copies, tile rows (tid >> 3) + 32 i.  nk = K / 64 k-blocks.
// Double-buffered: while k-block kt is multiplied from one LDS stage, block
// kt+1 is loaded into registers and then stored to the other stage.
struct TileRows {
  const uint16_t* a0;
  const uint16_t* a1;
  const uint16_t* a2;
  const uint16_t* a3;
  const uint16_t* b0;
  const uint16_t* b1;
  const uint16_t* b2;
  const uint16_t* b3;
};

__device__ __forceinline__ void load_kblock(const TileRows& R, int koff, uint4 (&ra)[4], uint4 (&rb)[4]) {
  ra[0] = *reinterpret_cast<const uint4*>(R.a0 + koff);
  ra[1] = *reinterpret_cast<const uint4*>(R.a1 + koff);
  ra[2] = *reinterpret_cast<const uint4*>(R.a2 + koff);
  ra[3] = *reinterpret_cast<const uint4*>(R.a3 + koff);
  rb[0] = *reinterpret_cast<const uint4*>(R.b0 + koff);
  rb[1] = *reinterpret_cast<const uint4*>(R.b1 + koff);
  rb[2] = *reinterpret_cast<const uint4*>(R.b2 + koff);
  rb[3] = *reinterpret_cast<const uint4*>(R.b3 + koff);
}

__device__ __forceinline__ void store_kblock(uint4* __restrict__ dst, int tid, const uint4 (&ra)[4],
                                             const uint4 (&rb)[4]) {
  const int seg = tid & 7;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 3) + 32 * i;
    dst[lds_slot(r, seg)] = ra[i];
    dst[kLdsStage + lds_slot(r, seg)] = rb[i];
  }
}

__device__ __forceinline__ void gemm_tile(const TileRows& R, int nk, f32x16 acc[4], uint4* lds) {
  if (nk <= 0) return;
  const int tid = threadIdx.x;
  const int seg = tid & 7;
  const int lane = tid & 63;
  const int arow = (tid >> 6) * 32 + (lane & 31);
  const int khalf = lane >> 5;
  uint4* st0 = lds;
  uint4* st1 = lds + 2 * kLdsStage;
  uint4 ra[4], rb[4];

  load_kblock(R, seg * 8, ra, rb);
  store_kblock(st0, tid, ra, rb);
  __syncthreads();
  int kt = 0;
  // two k-blocks per trip so that every LDS stage address is static
  for (; kt + 2 < nk; kt += 2) {
    load_kblock(R, (kt + 1) * kBK + seg * 8, ra, rb);
    mma_kblock(st0, st0 + kLdsStage, arow, lane, khalf, acc);
    store_kblock(st1, tid, ra, rb);
    __syncthreads();
    load_kblock(R, (kt + 2) * kBK + seg * 8, ra, rb);
    mma_kblock(st1, st1 + kLdsStage, arow, lane, khalf, acc);
    store_kblock(st0, tid, ra, rb);
    __syncthreads();
  }
  // one or two k-blocks left, the first in stage 0
  if (kt + 1 < nk) {
    load_kblock(R, (kt + 1) * kBK + seg * 8, ra, rb);
    mma_kblock(st0, st0 + kLdsStage, arow, lane, khalf, acc);
    store_kblock(st1, tid, ra, rb);
    __syncthreads();
    mma_kblock(st1, st1 + kLdsStage, arow, lane, khalf, acc);
  } else {
    mma_kblock(st0, st0 + kLdsStage, arow, lane, khalf, acc);
  }
  __syncthreads();
}

// Tile-local row of accumulator element r held by lane l (within wave's 32 rows).
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

__device__ __forceinline__ float acc_get(const f32x16 acc[4], int b, int r) {
  // b is wave-uniform or lane-varying; select without dynamic register indexing
  float v = acc[0][r];
  v = (b == 1) ? acc[1][r] : v;
  v = (b == 2) ? acc[2][r] : v;
  v = (b == 3) ? acc[3][r] : v;
  return v;
}

}  // namespace rlk
