// HIP kernels of the linear_logp path (gfx950).
//
// Forward / range partial:
//   compact_rows       order-preserving list of active rows (target != ignore)
//   fwd_chunks         MFMA logit tile + per-(row, chunk) statistics + target logit
//   merge_splits       chunk fold per split, pairwise tree over splits, epilogue
//   merge_parts        tree over per-range statistics (rlk_lse_merge)
// Backward (per vocabulary split c, ascending):
//   transpose_h        hT[k][i] = h[row_i][k] for the active rows, zero padded
//   transpose_w        WT[c][k][j] = W[c*S + j][k], zero padded
//   dz_tile            recomputed logits -> dz = g (onehot - softmax), bf16
//   grad_w_tile        grad_W rows of split c = dz_c^T h  (K = active rows)
//   grad_h_tile        fp32 accumulator += dz_c W_c; bf16 after the last split
//   zero_rows          zero grad_h rows of inactive rows
#pragma once

#include "rlk_device.h"

namespace rlk {

// ---------------------------------------------------------------------------
// Active-row compaction.  One block of 1024 threads scans y in order, so the
// list is the active rows in ascending order and independent of timing.
// Inactive rows get their final outputs here: logp = lse = 0 (forward) or
// the empty statistics {-inf, 0, 0, 0} (range partial).
// ---------------------------------------------------------------------------
struct PartialRec {
  float m, s, z_target;
  uint32_t owned;
};

__global__ __launch_bounds__(1024) void compact_rows(const int32_t* __restrict__ y, int T, int ignore_index,
                                                     int32_t* __restrict__ idx, int32_t* __restrict__ n_act,
                                                     float* __restrict__ logp, float* __restrict__ lse,
                                                     PartialRec* __restrict__ pout) {
  __shared__ int wave_tot[16];
  __shared__ int base_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) base_s = 0;
  __syncthreads();
  for (int t0 = 0; t0 < T; t0 += 1024) {
    const int t = t0 + tid;
    const bool act = (t < T) && (y[t] != ignore_index);
    if (t < T && !act) {
      if (logp) logp[t] = 0.f;
      if (lse) lse[t] = 0.f;
      if (pout) pout[t] = PartialRec{-INFINITY, 0.f, 0.f, 0u};
    }
    const uint64_t bal = __ballot(act);
    const int before = __popcll(bal & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
    if (lane == 0) wave_tot[wave] = __popcll(bal);
    __syncthreads();
    int off = base_s;
    for (int w = 0; w < wave; ++w) off += wave_tot[w];
    if (act) idx[off + before] = t;
    __syncthreads();
    if (tid == 0) {
      int tot = 0;
      for (int w = 0; w < 16; ++w) tot += wave_tot[w];
      base_s += tot;
    }
    __syncthreads();
  }
  if (tid == 0) *n_act = base_s;
}

// ---------------------------------------------------------------------------
// Forward chunk statistics.
// grid.x: 128-row tiles of the active rows; grid.y: chunk g of the processed
// split range (split = s0 + g / cps, chunk j = g % cps).  Writes
// rec[g * rec_stride + i] = (m, s) of chunk g for active row i, and zt[i] =
// logit of the target for the one chunk that holds it.
//
// Chunk statistics, for one row over the chunk's valid columns
// c = 32 b + q (b = 0..3 column block, q = 0..31 lane):
//   m = max_c z_c (exact);
//   e_c = exp(z_c - m), 0 for invalid columns;
//   a_q = ((e_q + e_{32+q}) + e_{64+q}) + e_{96+q};
//   s = pairwise tree over q = 0..31 of a_q (xor butterfly; every lane ends
//       with the same value because fp addition is commutative).
// ---------------------------------------------------------------------------
struct SplitGeom {
  int V;           // global vocabulary size
  int S;           // split width = ceil(V / 32)
  int cps;         // chunks per split = ceil(S / 128)
  int s0;          // first split of the processed range
  int vocab_start; // global index of row 0 of the W pointer given
};

__device__ __forceinline__ void chunk_cols(const SplitGeom& gm, int g, int& c0, int& c1) {
  const int split = gm.s0 + g / gm.cps;
  const int j = g - (g / gm.cps) * gm.cps;
  const int send = min(split * gm.S + gm.S, gm.V);
  c0 = split * gm.S + j * kChunk;
  c1 = min(c0 + kChunk, send);
}

__device__ __forceinline__ float xor_max(float v, int d) { return fmaxf(v, __shfl_xor(v, d, 64)); }
__device__ __forceinline__ float xor_add(float v, int d) { return v + __shfl_xor(v, d, 64); }

__global__ __launch_bounds__(kThreads) void fwd_chunks(const uint16_t* __restrict__ h, const uint16_t* __restrict__ W,
                                                       const int32_t* __restrict__ y, const int32_t* __restrict__ idx,
                                                       const int32_t* __restrict__ n_act_p, int H, SplitGeom gm,
                                                       size_t rec_stride, float2* __restrict__ rec,
                                                       float* __restrict__ zt) {
  __shared__ uint4 lds[4 * kLdsStage];
  const int n_act = *n_act_p;
  const int i0 = blockIdx.x * kBM;
  if (i0 >= n_act) return;
  const int g = blockIdx.y;
  int c0, c1;
  chunk_cols(gm, g, c0, c1);
  if (c0 >= c1) return;

  const int tid = threadIdx.x;
  const int r0 = tid >> 3;
  const int ia0 = idx[min(i0 + r0, n_act - 1)], ia1 = idx[min(i0 + r0 + 32, n_act - 1)];
  const int ia2 = idx[min(i0 + r0 + 64, n_act - 1)], ia3 = idx[min(i0 + r0 + 96, n_act - 1)];
  const int wb = c1 - 1 - gm.vocab_start, cb = c0 - gm.vocab_start;
  const TileRows R{h + (size_t)ia0 * H, h + (size_t)ia1 * H, h + (size_t)ia2 * H, h + (size_t)ia3 * H,
                   W + (size_t)min(cb + r0, wb) * H, W + (size_t)min(cb + r0 + 32, wb) * H,
                   W + (size_t)min(cb + r0 + 64, wb) * H, W + (size_t)min(cb + r0 + 96, wb) * H};
  f32x16 acc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) acc[b] = f32x16{};
  gemm_tile(R, H / kBK, acc, lds);

  // targets of the tile's rows, staged in LDS (the main loop ended with a barrier)
  int* ys = reinterpret_cast<int*>(lds);
  if (tid < kBM) {
    const int i = i0 + tid;
    ys[tid] = (i < n_act) ? y[idx[i]] : -1;
  }
  __syncthreads();

  const int lane = tid & 63, wave = tid >> 6, q = lane & 31;
  const int width = c1 - c0;
  bool valid[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) valid[b] = (32 * b + q) < width;

  float keep_m = 0.f, keep_s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float mx = -INFINITY;
#pragma unroll
    for (int b = 0; b < 4; ++b)
      if (valid[b]) mx = fmaxf(mx, acc[b][r]);
    mx = xor_max(mx, 1);
    mx = xor_max(mx, 2);
    mx = xor_max(mx, 4);
    mx = xor_max(mx, 8);
    mx = xor_max(mx, 16);
    float e[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) e[b] = valid[b] ? rlk_exp(acc[b][r] - mx) : 0.f;
    float a = ((e[0] + e[1]) + e[2]) + e[3];
    a = xor_add(a, 1);
    a = xor_add(a, 2);
    a = xor_add(a, 4);
    a = xor_add(a, 8);
    a = xor_add(a, 16);
    if (q == r) {
      keep_m = mx;
      keep_s = a;
    }
    // target logit: the lane holding column (y - c0) of this row
    const int row = wave * 32 + acc_row(r, lane);
    const int tc = ys[row] - c0;
    if (tc >= 0 && tc < width && (tc & 31) == q) zt[i0 + row] = acc_get(acc, tc >> 5, r);
  }
  if (q < 16) {
    const int row = wave * 32 + acc_row(q, lane);
    const int i = i0 + row;
    if (i < n_act) rec[(size_t)g * rec_stride + i] = make_float2(keep_m, keep_s);
  }
}

// ---------------------------------------------------------------------------
// Split fold + tree + epilogue.  grid.x: 64 active rows per block; 8 waves,
// wave w folds splits w, w+8, ... of the range (chunks left to right), the
// split statistics meet in LDS and one thread per row runs the pairwise
// tree over the nsplit splits.
// mode 0 (forward):  logp[t] = (z_t - m) - log s, lse[t] = m + log s
// mode 1 (partial):  pout[t] = {m, s, owned ? z_t : 0, owned}
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(512) void merge_splits(const float2* __restrict__ rec, size_t rec_stride,
                                                    const float* __restrict__ zt, const int32_t* __restrict__ idx,
                                                    const int32_t* __restrict__ n_act_p,
                                                    const int32_t* __restrict__ y, SplitGeom gm, int nsplit, int mode,
                                                    int own_lo, int own_hi, float* __restrict__ logp,
                                                    float* __restrict__ lse, PartialRec* __restrict__ pout) {
  __shared__ MS red[kNSplit][64];
  const int n_act = *n_act_p;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = blockIdx.x * 64 + lane;
  if (blockIdx.x * 64 >= n_act) return;
  for (int sl = wave; sl < nsplit; sl += 8) {
    MS r = ms_identity();
    if (i < n_act) {
      for (int j = 0; j < gm.cps; ++j) {
        const int g = sl * gm.cps + j;
        int c0, c1;
        chunk_cols(gm, g, c0, c1);
        if (c0 >= c1) break;
        const float2 v = rec[(size_t)g * rec_stride + i];
        r = ms_combine(r, MS{v.x, v.y});
      }
    }
    red[sl][lane] = r;
  }
  __syncthreads();
  if (wave != 0 || i >= n_act) return;
  MS v[kNSplit];
#pragma unroll
  for (int s = 0; s < kNSplit; ++s) v[s] = (s < nsplit) ? red[s][lane] : ms_identity();
  // pairwise tree over nsplit (a power of two <= 32)
#pragma unroll
  for (int w = 1; w < kNSplit; w <<= 1) {
    if (w < nsplit) {
#pragma unroll
      for (int s = 0; s + w < kNSplit; s += 2 * w) v[s] = ms_combine(v[s], v[s + w]);
    }
  }
  const MS tot = v[0];
  const int t = idx[i];
  const int yt = y[t];
  if (mode == 0) {
    const float L = rlk_log(tot.s);
    const bool ok = yt >= 0 && yt < gm.V;
    logp[t] = ok ? (zt[i] - tot.m) - L : __builtin_nanf("");
    if (lse) lse[t] = tot.m + L;
  } else {
    const bool owned = yt >= own_lo && yt < own_hi;
    pout[t] = PartialRec{tot.m, tot.s, owned ? zt[i] : 0.f, owned ? 1u : 0u};
  }
}

// ---------------------------------------------------------------------------
// rlk_lse_merge: per row, balanced tree over n_parts range statistics.
// The tree: left subtree = the largest power of two below the count.  The
// count is decomposed into power-of-two blocks from the front (its binary
// digits, most significant first); each block is a pairwise tree and the
// blocks are combined right to left: B1 (+) (B2 (+) (B3 ...)).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void merge_parts(const PartialRec* __restrict__ parts, int n_parts, int T,
                                                   const int32_t* __restrict__ y, int ignore_index,
                                                   float* __restrict__ logp, float* __restrict__ lse) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  if (y[t] == ignore_index) {
    logp[t] = 0.f;
    if (lse) lse[t] = 0.f;
    return;
  }
  MS v[kNSplit];
  int owners = 0;
  float z = 0.f;
  for (int p = 0; p < kNSplit; ++p) {
    if (p < n_parts) {
      const PartialRec r = parts[(size_t)p * T + t];
      v[p] = MS{r.m, r.s};
      if (r.owned) {
        ++owners;
        z = r.z_target;
      }
    } else {
      v[p] = ms_identity();
    }
  }
  MS acc = ms_identity();
  bool first = true;
  int end = n_parts;
  for (int bit = 0; bit < 6; ++bit) {
    if (!((n_parts >> bit) & 1)) continue;
    const int size = 1 << bit;
    const int lo = end - size;
    end = lo;
    // pairwise tree over v[lo .. lo+size)
    for (int w = 1; w < size; w <<= 1)
      for (int s = lo; s + w < lo + size; s += 2 * w) v[s] = ms_combine(v[s], v[s + w]);
    acc = first ? v[lo] : ms_combine(v[lo], acc);
    first = false;
  }
  const float L = rlk_log(acc.s);
  logp[t] = (owners == 1) ? (z - acc.m) - L : __builtin_nanf("");
  if (lse) lse[t] = acc.m + L;
}

// ---------------------------------------------------------------------------
// Backward helpers
// ---------------------------------------------------------------------------

// hT[k * ldt + i] = h[idx[i] * H + k] for i < n_act, 0 for n_act <= i < ldt.
// grid (ldt / 64, H / 64), block 256; 64x64 tile through LDS.
__global__ __launch_bounds__(256) void transpose_h(const uint16_t* __restrict__ h, const int32_t* __restrict__ idx,
                                                   const int32_t* __restrict__ n_act_p, int H, int ldt,
                                                   uint16_t* __restrict__ hT) {
  __shared__ uint16_t tile[64][65];
  const int n_act = *n_act_p;
  const int i0 = blockIdx.x * 64, k0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int r = ty; r < 64; r += 4) {
    const int i = i0 + r;
    tile[r][tx] = (i < n_act) ? h[(size_t)idx[i] * H + k0 + tx] : (uint16_t)0;
  }
  __syncthreads();
  for (int r = ty; r < 64; r += 4) hT[(size_t)(k0 + r) * ldt + i0 + tx] = tile[tx][r];
}

// WT[(c * H + k) * S_pad + j] = W[(c * S + j) * H + k] for j < valid(c), else 0.
// grid (S_pad / 64, H / 64, 32), block 256.
__global__ __launch_bounds__(256) void transpose_w(const uint16_t* __restrict__ W, int V, int H, int S, int S_pad,
                                                   uint16_t* __restrict__ WT) {
  __shared__ uint16_t tile[64][65];
  const int c = blockIdx.z;
  const int j0 = blockIdx.x * 64, k0 = blockIdx.y * 64;
  const int valid = max(0, min(S, V - c * S));
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int r = ty; r < 64; r += 4) {
    const int j = j0 + r;
    tile[r][tx] = (j < valid) ? W[(size_t)(c * S + j) * H + k0 + tx] : (uint16_t)0;
  }
  __syncthreads();
  uint16_t* dst = WT + (size_t)c * H * S_pad;
  for (int r = ty; r < 64; r += 4) dst[(size_t)(k0 + r) * S_pad + j0 + tx] = tile[tx][r];
}

// dz for split c: grid (row tiles, cps).  For active row i and column v of the
// split:  p = exp(z - lse_i),  dz = g_i * ([v == y_i] - p)  in fp32, then
// rounded to bf16 (RNE).  Written as dZ[i][v_local] (ld S_pad) and
// dZT[v_local][i] (ld T_pad); rows >= n_act and invalid columns get 0.
__global__ __launch_bounds__(kThreads) void dz_tile(const uint16_t* __restrict__ h, const uint16_t* __restrict__ W,
                                                    const int32_t* __restrict__ y, const int32_t* __restrict__ idx,
                                                    const int32_t* __restrict__ n_act_p, const float* __restrict__ lse,
                                                    const float* __restrict__ gup, int H, SplitGeom gm, int split,
                                                    int T_pad, int S_pad, uint16_t* __restrict__ dZ,
                                                    uint16_t* __restrict__ dZT) {
  __shared__ uint4 lds[4 * kLdsStage];
  const int n_act = *n_act_p;
  const int i0 = blockIdx.x * kBM;
  if (i0 >= n_act) return;
  const int j = blockIdx.y;
  const int sstart = split * gm.S;
  const int send = min(sstart + gm.S, gm.V);
  const int c0 = sstart + j * kChunk;
  const int c1 = min(c0 + kChunk, send);
  const int width = max(0, c1 - c0);
  const int tid = threadIdx.x;
  f32x16 acc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) acc[b] = f32x16{};
  if (width > 0) {
    const int r0 = tid >> 3;
    const int ia0 = idx[min(i0 + r0, n_act - 1)], ia1 = idx[min(i0 + r0 + 32, n_act - 1)];
    const int ia2 = idx[min(i0 + r0 + 64, n_act - 1)], ia3 = idx[min(i0 + r0 + 96, n_act - 1)];
    const int wb = c1 - 1;
    const TileRows R{h + (size_t)ia0 * H, h + (size_t)ia1 * H, h + (size_t)ia2 * H, h + (size_t)ia3 * H,
                     W + (size_t)min(c0 + r0, wb) * H, W + (size_t)min(c0 + r0 + 32, wb) * H,
                     W + (size_t)min(c0 + r0 + 64, wb) * H, W + (size_t)min(c0 + r0 + 96, wb) * H};
    gemm_tile(R, H / kBK, acc, lds);
  }
  float* rowv = reinterpret_cast<float*>(lds);  // [128] lse, [128] g, [128] y
  if (tid < kBM) {
    const int i = i0 + tid;
    if (i < n_act) {
      const int t = idx[i];
      rowv[tid] = lse[t];
      rowv[128 + tid] = gup[t];
      reinterpret_cast<int*>(rowv)[256 + tid] = y[t];
    } else {
      rowv[tid] = 0.f;
      rowv[128 + tid] = 0.f;
      reinterpret_cast<int*>(rowv)[256 + tid] = -1;
    }
  }
  __syncthreads();
  const int lane = tid & 63, wave = tid >> 6, q = lane & 31;
  const int vbase = j * kChunk;  // split-local column of the chunk start
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int cl = 32 * b + q;  // chunk-local column
    const bool cvalid = cl < width;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      uint16_t o[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int r = 4 * r4 + rr;
        const int row = wave * 32 + acc_row(r, lane);
        const int i = i0 + row;
        float d = 0.f;
        if (cvalid && i < n_act) {
          const float p = rlk_exp(acc[b][r] - rowv[row]);
          const float delta = (reinterpret_cast<const int*>(rowv)[256 + row] == c0 + cl) ? 1.f : 0.f;
          d = rowv[128 + row] * (delta - p);
        }
        o[rr] = f32_to_bf16_rne(d);
        dZ[(size_t)i * S_pad + vbase + cl] = o[rr];
      }
      // rows 8*r4 + 4*(lane>>5) + 0..3 are consecutive: one 8-byte store into dZT
      const int row0 = wave * 32 + acc_row(4 * r4, lane);
      uint2 pk;
      pk.x = (uint32_t)o[0] | ((uint32_t)o[1] << 16);
      pk.y = (uint32_t)o[2] | ((uint32_t)o[3] << 16);
      *reinterpret_cast<uint2*>(dZT + (size_t)(vbase + cl) * T_pad + i0 + row0) = pk;
    }
  }
}

// grad_W rows of split c: C[v][n] = sum_i dZT[v][i] hT[n][i], K = active rows
// rounded up to 64 (the padding rows of dZT and hT are zero).  grid
// (S_pad / 128, ceil(H / 128)).  Written once, fp32.
__global__ __launch_bounds__(kThreads) void grad_w_tile(const uint16_t* __restrict__ dZT,
                                                        const uint16_t* __restrict__ hT,
                                                        const int32_t* __restrict__ n_act_p, int H, int T_pad,
                                                        int valid_rows, size_t out_row0, float* __restrict__ grad_W) {
  __shared__ uint4 lds[4 * kLdsStage];
  const int n_act = *n_act_p;
  const int v0 = blockIdx.x * kBM, n0 = blockIdx.y * kBN;
  if (v0 >= valid_rows) return;
  const int tid = threadIdx.x;
  const int r0 = tid >> 3;
  const TileRows R{dZT + (size_t)(v0 + r0) * T_pad, dZT + (size_t)(v0 + r0 + 32) * T_pad,
                   dZT + (size_t)(v0 + r0 + 64) * T_pad, dZT + (size_t)(v0 + r0 + 96) * T_pad,
                   hT + (size_t)min(n0 + r0, H - 1) * T_pad, hT + (size_t)min(n0 + r0 + 32, H - 1) * T_pad,
                   hT + (size_t)min(n0 + r0 + 64, H - 1) * T_pad, hT + (size_t)min(n0 + r0 + 96, H - 1) * T_pad};
  f32x16 acc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) acc[b] = f32x16{};
  gemm_tile(R, (n_act + kBK - 1) / kBK, acc, lds);
  const int lane = tid & 63, wave = tid >> 6, q = lane & 31;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int n = n0 + 32 * b + q;
    if (n >= H) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int v = v0 + wave * 32 + acc_row(r, lane);
      if (v < valid_rows) grad_W[(out_row0 + v) * (size_t)H + n] = acc[b][r];
    }
  }
}

// grad_h: acc[i][n] (+)= sum_v dZ[i][v] WT_c[n][v] over split c, K = S_pad
// (zero padded).  The fp32 accumulator chain continues across splits through
// ghacc (exact fp32 store/load), so grad_h is one chain over the vocabulary
// in ascending order.  After the last split the result is rounded to bf16
// once and written to the row's place in grad_h.  grid (row tiles, ceil(H/128)).
__global__ __launch_bounds__(kThreads) void grad_h_tile(const uint16_t* __restrict__ dZ,
                                                        const uint16_t* __restrict__ WTc,
                                                        const int32_t* __restrict__ idx,
                                                        const int32_t* __restrict__ n_act_p, int H, int S_pad,
                                                        int first, int last, float* __restrict__ ghacc,
                                                        uint16_t* __restrict__ grad_h) {
  __shared__ uint4 lds[4 * kLdsStage];
  const int n_act = *n_act_p;
  const int i0 = blockIdx.x * kBM, n0 = blockIdx.y * kBN;
  if (i0 >= n_act) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, q = lane & 31;
  f32x16 acc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int n = n0 + 32 * b + q;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = i0 + wave * 32 + acc_row(r, lane);
      acc[b][r] = (!first && i < n_act && n < H) ? ghacc[(size_t)i * H + n] : 0.f;
    }
  }
  const int r0 = tid >> 3;
  const TileRows R{dZ + (size_t)(i0 + r0) * S_pad, dZ + (size_t)(i0 + r0 + 32) * S_pad,
                   dZ + (size_t)(i0 + r0 + 64) * S_pad, dZ + (size_t)(i0 + r0 + 96) * S_pad,
                   WTc + (size_t)min(n0 + r0, H - 1) * S_pad, WTc + (size_t)min(n0 + r0 + 32, H - 1) * S_pad,
                   WTc + (size_t)min(n0 + r0 + 64, H - 1) * S_pad, WTc + (size_t)min(n0 + r0 + 96, H - 1) * S_pad};
  gemm_tile(R, S_pad / kBK, acc, lds);
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int n = n0 + 32 * b + q;
    if (n >= H) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = i0 + wave * 32 + acc_row(r, lane);
      if (i >= n_act) continue;
      if (last)
        grad_h[(size_t)idx[i] * H + n] = f32_to_bf16_rne(acc[b][r]);
      else
        ghacc[(size_t)i * H + n] = acc[b][r];
    }
  }
}

// Zero the grad_h rows of inactive rows.  grid T, block 256.
__global__ __launch_bounds__(256) void zero_rows(const int32_t* __restrict__ y, int ignore_index, int H,
                                                 uint16_t* __restrict__ grad_h) {
  const int t = blockIdx.x;
  if (y[t] != ignore_index) return;
  for (int k = threadIdx.x; k < H; k += 256) grad_h[(size_t)t * H + k] = 0;
}

}  // namespace rlk
