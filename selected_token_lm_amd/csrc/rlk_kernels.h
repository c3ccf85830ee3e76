// HIP kernels of the linear_logp path (gfx950).
//
// Forward / range partial:
//   compact_rows       order-preserving list of active rows (target != ignore)
//   fwd_tiles          MFMA logit tiles + per-(row, chunk) statistics + target logit
//   merge_splits       chunk fold per split, pairwise tree over splits, epilogue
//   merge_parts        tree over per-range statistics (rlk_lse_merge)
// Backward (per group of vocabulary splits, ascending):
//   dz_tiles           recomputed logits -> dz = g (onehot - softmax), bf16
//   dz_saved           the same dz from logits the forward saved (no recompute)
//   grad_tiles         one launch of the group's tiles of
//                        grad_h: fp32 accumulator += dz W; bf16 after the last group
//                        grad_W: rows of the group = dz^T h  (K = active rows)
//   zero_rows          zero grad_h rows of inactive rows
// RL objective (O(T)):
//   rl_token_loss      clipped surrogate + k3 KL per token, and dL/dlogp
// Dense product (same engine):
//   gemm_tiles         C = A B^T, one MFMA chain per element
#pragma once

#include "rlk_args.h"
#include "rlk_gemm.h"

// Which unit builds which kernel: the eight-wave unit (RLK_ENGINE_W8) the
// plain forward's fwd_tiles instance, dz_tiles and grad_tiles; the
// four-wave unit the other fwd_tiles instances (save-logits, small
// batches), the dense product, the row kernels and the merges.
RLK_ENGINE_BEGIN

// ---------------------------------------------------------------------------
// Per-token RL objective on the selected logp (PPO / GRPO clipped surrogate
// and k3 KL to a reference), with its derivative g = dL/dlogp ready for the
// backward.  Every operation is a separately rounded fp32 operation in the
// order written; exp is the library's e(x).  One function for the
// standalone kernel and the forward's fused epilogue (the same bits).
// ---------------------------------------------------------------------------
// Loss and dL/dlogp of one active token t with selected log-probability lp.
__device__ __forceinline__ void rl_token(const RlLossArgs& a, int t, float lp, float& L, float& gt) {
  const float A = a.adv[t];
  const float r = rlk_exp(lp - a.logp_old[t]);
  // clip written with comparisons so that a NaN ratio (a row whose logp is
  // NaN: its target lies outside the vocabulary) stays NaN; for every other
  // value this is min(max(r, 1 - eps_low), 1 + eps_high)
  const float lo = 1.f - a.eps_low, hi = 1.f + a.eps_high;
  const float c = r < lo ? lo : (r > hi ? hi : r);
  const float ra = r * A, ca = c * A;
  L = -fminf(ra, ca);
  gt = (ra <= ca) ? -ra : ((ra > ca) ? 0.f : ra);  // unordered (NaN): NaN
  if (a.beta != 0.f) {
    const float d = a.logp_ref[t] - lp;
    const float ed = rlk_exp(d);
    L = L + a.beta * ((ed - d) - 1.f);
    gt = gt + a.beta * (1.f - ed);
  }
  L = a.scale * L;
  gt = a.scale * gt;
}

// ---------------------------------------------------------------------------
// Active-row compaction.  One block of 1024 threads scans y in order, so the
// list is the active rows in ascending order and independent of timing;
// yA (optional) receives their targets in the same order.
// Inactive rows get their final outputs here: logp = lse = 0 (forward) or
// the empty statistics {-inf, 0, 0, 0} (range partial), and loss = g = 0
// when the forward also evaluates the RL objective.
// ---------------------------------------------------------------------------
#ifndef RLK_ENGINE_W8
__global__ __launch_bounds__(1024) void compact_rows(const int32_t* __restrict__ y, int T, int ignore_index,
                                                     int32_t* __restrict__ idx, int32_t* __restrict__ yA,
                                                     int32_t* __restrict__ n_act,
                                                     float* __restrict__ logp, float* __restrict__ lse,
                                                     PartialRec* __restrict__ pout, float* __restrict__ rl_loss,
                                                     float* __restrict__ rl_g) {
  __shared__ int wave_tot[16];
  __shared__ int base_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) base_s = 0;
  __syncthreads();
  // a pass covers 1024 kPer rows, thread tid rows t0 + kPer tid .. + kPer - 1
  // (ascending), so the block-wide exclusive scan of the per-thread counts
  // gives every active row its place in row order
  constexpr int kPer = 4;
  for (int t0 = 0; t0 < T; t0 += 1024 * kPer) {
    int ys[kPer];
    int cnt = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int t = t0 + kPer * tid + e;
      ys[e] = (t < T) ? y[t] : ignore_index;
      cnt += ys[e] != ignore_index;
    }
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int t = t0 + kPer * tid + e;
      if (t < T && ys[e] == ignore_index) {
        if (logp) logp[t] = 0.f;
        if (lse) lse[t] = 0.f;
        if (pout) pout[t] = PartialRec{-INFINITY, 0.f, 0.f, 0u};
        if (rl_loss) rl_loss[t] = 0.f;
        if (rl_g) rl_g[t] = 0.f;
      }
    }
    // inclusive scan of the counts over the wave
    int incl = cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d);
      if (lane >= d) incl += v;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int pos = base_s + incl - cnt;
    for (int w = 0; w < wave; ++w) pos += wave_tot[w];
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      if (ys[e] != ignore_index) {
        idx[pos] = t0 + kPer * tid + e;
        if (yA) yA[pos] = ys[e];
        ++pos;
      }
    }
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
#endif

// ---------------------------------------------------------------------------
// Vocabulary geometry
// ---------------------------------------------------------------------------
__device__ __forceinline__ void chunk_cols(const SplitGeom& gm, int g, int& c0, int& c1) {
  const int split = gm.s0 + g / gm.cps;
  const int j = g - (g / gm.cps) * gm.cps;
  const int send = min(split * gm.S + gm.S, gm.V);
  c0 = split * gm.S + j * kChunk;
  c1 = min(c0 + kChunk, send);
}

// ---------------------------------------------------------------------------
// Forward chunk statistics on 256 x 256 tiles.
//
// Tile (rt, ct): active rows [256 rt, +256) x columns [c0, c0 + 256) of one
// split, c0 = split start + 256 j; wave (wm, wn) holds the 128-column chunk
// 2j + wn of that split.  Writes rec[g * rec_stride + i] = (m, s) of chunk g
// (g = local split * cps + chunk) for active row i, and zt[i] = the target's
// logit, written by the one chunk that holds it.
//
// A row's 128 chunk columns sit in kLPR lanes (the MFMA output layout):
// lane part r = row_lane(l) (0 .. kLPR-1) holds the kRowVals columns c with
// (c >> 2) % kLPR == r, in ascending order as its elements
// k = 4 kQL ni + 4 q + u, column chunk_col(k) + 4 r.  Chunk statistics of
// one row over the chunk's valid columns:
//   m   = max_c z_c (exact; invalid columns enter as -inf);
//   e_c = exp(z_c - m) (0 for invalid columns);
//   s   = combination over the parts of T(e of part r), T = balanced
//         pairwise tree over the part's columns in ascending order; two
//         parts (32 x 32 MFMAs): T0 + T1; four (16 x 16): (T0 + T1) + (T2 + T3).
// ---------------------------------------------------------------------------
constexpr int kRowVals = kNI * kQL * 4;  // a lane's values of one row of a chunk: 64 or 32
// Row blocks whose per-row inputs a tile kernel loads under the last k-block
// (the rest after the engine returns): all with four waves, one with eight.
constexpr int kTailRows = kWaves == 8 ? 1 : kMI;

// Chunk column of a lane's value k, relative to 4 row_lane(l).
__device__ __forceinline__ constexpr int chunk_col(int k) {
  return kBlk * (k / (4 * kQL)) + 4 * kLPR * (k / 4 % kQL) + (k & 3);
}

// The lane value index of chunk column c (in the lane with row_lane == (c >> 2) % kLPR).
__device__ __forceinline__ int chunk_val(int c) { return 4 * kQL * (c / kBlk) + 4 * (c % kBlk / (4 * kLPR)) + (c & 3); }

// Max and sum of one row over the kLPR lanes that hold it, the same value in
// each of them: with two parts the lane pair (l, l ^ 32); with four the
// lanes l ^ 16, then l ^ 32, so the sum is (s0 + s1) + (s2 + s3) for the
// parts' partials in part order (fp32 addition is commutative, so every
// lane forms the same sums).
__device__ __forceinline__ float row_max(float x) {
  if constexpr (kLPR == 2) {
    float lo, hi;
    lane_halves(x, lo, hi);
    return fmaxf(lo, hi);
  } else {
    x = fmaxf(x, __shfl_xor(x, 16));
    return fmaxf(x, __shfl_xor(x, 32));
  }
}
__device__ __forceinline__ float row_sum(float x) {
  if constexpr (kLPR == 2) {
    float lo, hi;
    lane_halves(x, lo, hi);
    return lo + hi;
  } else {
    x = x + __shfl_xor(x, 16);
    return x + __shfl_xor(x, 32);
  }
}

// sum over k in [k0, k0 + N) of e(v[k] - m) as a balanced pairwise tree
// (adjacent pairs, then pairs of pairs), evaluated subtree by subtree so
// that only one partial sum per level is live.
template <int N>
__device__ __forceinline__ float exp_tree(const float (&v)[kRowVals], int k0, float m) {
  if constexpr (N == 1) {
    return rlk_exp(v[k0] - m);
  } else {
    const float l = exp_tree<N / 2>(v, k0, m);
    const float r = exp_tree<N / 2>(v, k0 + N / 2, m);
    return l + r;
  }
}

// (m, s) of one row of a chunk from this lane's values v and those of the
// other lanes of the row; columns outside the chunk enter as -inf (they do
// not move the max, and their e is exp(-inf) = 0).
__device__ __forceinline__ float2 chunk_stats(const float (&v)[kRowVals]) {
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < kRowVals; ++k) mx = fmaxf(mx, v[k]);
  mx = row_max(mx);
  return make_float2(mx, row_sum(exp_tree<kRowVals>(v, 0, mx)));
}

// Engine call for a K-mode x K-mode tile.  kSkinny = 1..3 (four-wave
// layout only): the caller guarantees that every valid row of the tile lies
// below 32 kSkinny (a batch of at most 96 rows, one row tile), so the
// waves holding rows 128..255 compute nothing, the others only their first
// 32 kSkinny rows (kRB row blocks), and only the waves whose load rows
// (64 w .. 64 w + 63) meet those rows load the A tile.  Every element that
// is computed is the same MFMA chain as in the full tile.
template <int kSkinny, class LA, class LB, class Tail>
__device__ __forceinline__ void gemm_kk(const LA& la, const LB& lb, int nk, Acc& acc, u32x4* lds, const Tail& tail) {
  if constexpr (kSkinny == 0 || kWaves != 4) {
    gemm256<false, false>(la, lb, nk, acc, lds, tail);
  } else {
    constexpr int kRB = kSkinny * 32 / kBlk;  // row blocks below 32 kSkinny
    static_assert(kSkinny >= 1 && kRB < kMI, "row blocks of the first wave row");
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (w == 0) {
      gemm256<false, false, kRB, true>(la, lb, nk, acc, lds, tail);
    } else if (w == 2) {
      gemm256<false, false, kRB, false>(la, lb, nk, acc, lds, tail);
    } else if (w == 1 && kSkinny >= 3) {
      gemm256<false, false, 0, true>(la, lb, nk, acc, lds, tail);
    } else {
      gemm256<false, false, 0, false>(la, lb, nk, acc, lds, tail);
    }
  }
}

// kSave: also store every active row's fp32 logits (the values the chunk
// statistics are taken from) for a backward without recompute.  kSkinny:
// see gemm_kk (a batch of at most 32 kSkinny rows).
template <bool kSave, int kSkinny>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(RLK_WAVES / 4, RLK_WAVES / 4))) void fwd_tiles(FwdArgs a) {
  __shared__ u32x4 lds[kLdsU4];
  // tiles: the active-row tiles x every 256-column tile of the range (the
  // count goes through a scalar register: tile addresses derive from it)
  const int n_act = __builtin_amdgcn_readfirstlane(*a.n_act);
  const int rtiles = (n_act + kBM - 1) / kBM;
  const int C = a.nsplit * a.tg.tps;
  const int id = xcd_tile(rtiles * C, blockIdx.x);
  if (id < 0) return;
  int rt, ct;
  grouped_tile(id, rtiles, rt, ct, C, row_group(rtiles));
  const int i0 = rt * kBM;
  const int sl = ct / a.tg.tps, j = ct - sl * a.tg.tps;
  const int sbeg = (a.gm.s0 + sl) * a.gm.S;
  const int send = min(sbeg + a.gm.S, a.gm.V);
  const int c0 = sbeg + j * kBN;
  if (c0 >= send) return;
  const int c1 = min(c0 + kBN, send);

  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), wm = wave_m(w),
            wn = wave_n(w);
  // targets (and, kSave, original rows) of this lane's rows: those of the
  // first kTailRows row blocks are loaded while the last k-block's MFMAs run
  // (so that nothing of them is kept through the main loop), the others when
  // the epilogue starts, landing while the first blocks are processed (with
  // eight waves the last k-block leaves registers for one block's only)
  int tgt[kMI], trow[kMI];
  const auto load_row = [&](int mi, int ln) {
    const int r = min(i0 + acc_row(wm, mi, ln), n_act - 1);
    tgt[mi] = a.yA[r];
    if (kSave) trow[mi] = a.idx[r];
  };
  const auto load_rows = [&]() {
#pragma unroll
    for (int mi = 0; mi < kTailRows; ++mi) load_row(mi, lane);
  };

  const RowsK A = rows_k(a.hA + (size_t)i0 * a.H, kBM - 1, a.H);
  const RowsK B = rows_k(a.W + (size_t)(c0 - a.gm.vocab_start) * a.H, c1 - 1 - c0, a.H);
  Acc acc;
  acc_zero(acc);
  gemm_kk<kSkinny>(A, B, a.H / kBK, acc, lds, load_rows);

  const int cc0 = c0 + kChunk * wn;  // this wave's chunk
  const int width = min(cc0 + kChunk, c1) - cc0;
  if (width <= 0) return;
  const int g = sl * a.gm.cps + 2 * j + wn;
  // the lane's indices again, from an opaque copy of the lane id: computed
  // before the main loop they would be kept live through it
  int le = lane;
  asm volatile("" : "+v"(le));
  const int rl = row_lane(le);
  const int lim = width - 4 * rl;  // value k is valid iff chunk_col(k) < lim
#pragma unroll
  for (int mi = kTailRows; mi < kMI; ++mi) load_row(mi, le);

#pragma unroll
  for (int mi = 0; mi < kMI; ++mi) {
    const int i = i0 + acc_row(wm, mi, le);
    // the row's values of this lane, out of the accumulator once, one row
    // block at a time: its values leave the accumulators here and not
    // earlier (the scheduler would otherwise hoist every block's moves)
    __builtin_amdgcn_sched_barrier(0);
    float v[kRowVals];
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
      for (int r = 0; r < 4 * kQL; ++r) v[4 * kQL * ni + r] = acc.c[mi][ni][r];
    if (kSave && i < n_act) {
      // columns cc0 + 4 rl + chunk_col(k) (the chunk's first `width`);
      // cc0 - sbeg is a multiple of 128, so every float4 is 16-byte aligned
      float* zr = a.zsave + (size_t)trow[mi] * a.ldzs + (size_t)(a.gm.s0 + sl) * a.zs_spad + (cc0 - sbeg) + 4 * rl;
      if (width == kChunk) {
        // a whole chunk (wave-uniform): every float4 is inside it
#pragma unroll
        for (int k = 0; k < kRowVals; k += 4)
          *reinterpret_cast<float4*>(zr + chunk_col(k)) = make_float4(v[k], v[k + 1], v[k + 2], v[k + 3]);
      } else {
#pragma unroll
        for (int k = 0; k < kRowVals; k += 4) {
          const int c = chunk_col(k);  // column of element k, relative to cc0 + 4 rl
          if (c + 4 <= lim) {
            *reinterpret_cast<float4*>(zr + c) = make_float4(v[k], v[k + 1], v[k + 2], v[k + 3]);
          } else {
#pragma unroll
            for (int u = 0; u < 4; ++u)
              if (c + u < lim) zr[c + u] = v[k + u];
          }
        }
      }
    }
    // target logit: rare (a row's target lies in a given chunk about once in
    // a thousand).  When some lane of the wave needs one, the wave's values
    // go through LDS, which is free once the engine has returned: lane l
    // writes its element k at float4 slot 64 (k >> 2) + l of the wave's
    // 16 kRowVals float4 slots and reads back only its own.
    const int tc = tgt[mi] - cc0;
    const bool hit = i < n_act && tc >= 0 && tc < width && ((tc >> 2) & (kLPR - 1)) == rl;
    if (__builtin_amdgcn_ballot_w64(hit)) {
      float4* sl = reinterpret_cast<float4*>(lds) + 16 * kRowVals * w;
#pragma unroll
      for (int q = 0; q < kRowVals / 4; ++q)
        sl[64 * q + le] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
      if (hit) {
        const int k = chunk_val(tc);
        a.zt[i] = reinterpret_cast<const float*>(sl + 64 * (k >> 2) + le)[k & 3];
      }
    }
    // the short last chunk of a split (a wave-uniform branch): its missing
    // columns become -inf in place (v is this row block's own copy and is
    // not used after the statistics)
    if (width < kChunk) {
#pragma unroll
      for (int k = 0; k < kRowVals; ++k)
        if (chunk_col(k) >= lim) v[k] = -INFINITY;
    }
    const float2 st = chunk_stats(v);
    if (rl == 0 && i < n_act) a.rec[(size_t)g * a.rec_stride + i] = st;
  }
}

// ---------------------------------------------------------------------------
// Split fold + tree + epilogue.  grid.x: kMergeRows rows per block; thread
// (split s, row r) folds split s of the range for row r (chunks left to
// right), the split statistics meet in LDS and one thread per row runs the
// pairwise tree over the nsplit splits.
// mode 0 (forward):  logp[t] = (z_t - m) - log s, lse[t] = m + log s, and
//                    when rl.loss or rl.g is set the per-token RL objective
//                    of that logp (rl_token: the same bits as rl_token_loss)
// mode 1 (partial):  pout[t] = {m, s, owned ? z_t : 0, owned}
// ---------------------------------------------------------------------------
constexpr int kMergeRows = 16;  // rows per block of merge_splits (one thread per row and split)
#ifndef RLK_ENGINE_W8
__global__ __launch_bounds__(kMergeRows * kNSplit) void merge_splits(const float2* __restrict__ rec, size_t rec_stride,
                                                    const float* __restrict__ zt, const int32_t* __restrict__ idx,
                                                    const int32_t* __restrict__ n_act_p,
                                                    const int32_t* __restrict__ y, SplitGeom gm, int nsplit, int mode,
                                                    int own_lo, int own_hi, float* __restrict__ logp,
                                                    float* __restrict__ lse, PartialRec* __restrict__ pout,
                                                    RlLossArgs rl) {
  __shared__ MS red[kNSplit][kMergeRows];
  const int n_act = *n_act_p;
  const int lane = threadIdx.x % kMergeRows, sl = threadIdx.x / kMergeRows;
  const int i = blockIdx.x * kMergeRows + lane;
  if (blockIdx.x * kMergeRows >= n_act) return;
  {
    MS r = ms_identity();
    if (sl < nsplit && i < n_act) {
      // chunks of the split that hold vocabulary columns (the others carry
      // no record); their records are loaded kBatch at a time ahead of the
      // fold, which still takes them left to right
      int c0, c1;
      chunk_cols(gm, sl * gm.cps, c0, c1);
      const int send = min(c0 + gm.S, gm.V);
      const int nj = send > c0 ? (send - c0 + kChunk - 1) / kChunk : 0;
      const float2* rp = rec + (size_t)sl * gm.cps * rec_stride + i;
      constexpr int kBatch = 8;
      for (int j0 = 0; j0 < nj; j0 += kBatch) {
        float2 buf[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
          if (j0 + u < nj) buf[u] = rp[(size_t)(j0 + u) * rec_stride];
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
          if (j0 + u < nj) r = ms_combine(r, MS{buf[u].x, buf[u].y});
      }
    }
    red[sl][lane] = r;
  }
  __syncthreads();
  if (sl != 0 || i >= n_act) return;
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
    const float lp = ok ? (zt[i] - tot.m) - L : __builtin_nanf("");
    logp[t] = lp;
    if (lse) lse[t] = tot.m + L;
    if (rl.loss || rl.g) {
      // the RL objective on this token's log-probability, as rl_token_loss
      // computes it from the stored value
      float loss, gt;
      rl_token(rl, t, lp, loss, gt);
      if (rl.loss) rl.loss[t] = loss;
      if (rl.g) rl.g[t] = gt;
    }
  } else {
    const bool owned = yt >= own_lo && yt < own_hi;
    pout[t] = PartialRec{tot.m, tot.s, owned ? zt[i] : 0.f, owned ? 1u : 0u};
  }
}
#endif

// ---------------------------------------------------------------------------
// rlk_lse_merge: per row, balanced tree over n_parts range statistics.
// The tree: left subtree = the largest power of two below the count.  That
// is the pairwise tree over 32 slots (adjacent pairs, then pairs of pairs)
// with the slots past n_parts holding the empty statistics: combining with
// the empty statistics returns the other operand bit for bit, so the padded
// subtrees reduce to exactly the unpadded ones.  (Every index is a
// compile-time constant, so the 32 records stay in registers.)
// ---------------------------------------------------------------------------
#ifndef RLK_ENGINE_W8
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
#pragma unroll
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
#pragma unroll
  for (int w = 1; w < kNSplit; w <<= 1)
#pragma unroll
    for (int s = 0; s + w < kNSplit; s += 2 * w) v[s] = ms_combine(v[s], v[s + w]);
  const MS acc = v[0];
  const float L = rlk_log(acc.s);
  logp[t] = (owners == 1) ? (z - acc.m) - L : __builtin_nanf("");
  if (lse) lse[t] = acc.m + L;
}
#endif

// ---------------------------------------------------------------------------
// Backward.  The vocabulary splits are processed in groups of G consecutive
// splits [c_lo, c_lo + G); dz of a group lives in the workspace as
// dZ[t][sc * S_pad + v] (bf16, t = active-row index, sc = split within the
// group, v = column within the split, S_pad = S rounded up to 64, zero
// padded).  The grouping changes no result bit: grad_W's chain runs over
// rows and grad_h's chain runs over the vocabulary in ascending order with
// the same zero padding after every split, whatever G is.
// ---------------------------------------------------------------------------
// dz for the group's splits on 256 x 256 tiles (same tiles and logits as the
// forward): p = exp(z - lse_i), dz = g_i * ([v == y_i] - p) in fp32, rounded
// once to bf16.  Rows >= n_act of the tile and columns >= the split's width
// are written as zeros.  The tile is staged in LDS and stored row by row
// (16 bytes per lane, whole 512-byte rows per instruction pair of lanes).
#ifdef RLK_ENGINE_W8
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(RLK_WAVES / 4, RLK_WAVES / 4))) void dz_tiles(DzArgs a) {
  __shared__ u32x4 lds[kLdsU4];
  const int n_act = __builtin_amdgcn_readfirstlane(*a.n_act);
  const int rtiles = (n_act + kBM - 1) / kBM;
  const int C = a.bg.G * a.tg.tps;
  const int id = xcd_tile(rtiles * C, blockIdx.x);
  if (id < 0) return;
  int rt, ct;
  grouped_tile(id, rtiles, rt, ct, C, row_group(rtiles));
  const int i0 = rt * kBM;
  const int sc = ct / a.tg.tps, j = ct - sc * a.tg.tps;
  const int sbeg = (a.bg.c_lo + sc) * a.gm.S;
  const int valid_s = max(0, min(a.gm.S, a.gm.V - sbeg));  // columns of this split
  const int c0 = sbeg + j * kBN;
  const int c1 = sbeg + min(j * kBN + kBN, valid_s);
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), wm = wave_m(w),
            wn = wave_n(w);
  // this lane's rows' {lse, g, target}: those of the first kTailRows row
  // blocks loaded under the last k-block, the others when the epilogue
  // starts (as in fwd_tiles)
  float4 ri[kMI];
  const auto load_rows = [&]() {
#pragma unroll
    for (int mi = 0; mi < kTailRows; ++mi) ri[mi] = a.rowinfo[i0 + acc_row(wm, mi, lane)];
  };
  Acc acc;
  acc_zero(acc);
  {
    // a tile past the vocabulary (tiny vocabularies only: c0 >= c1) still
    // runs, on W's first row; its columns are all written as zeros below
    const RowsK A = rows_k(a.hA + (size_t)i0 * a.H, kBM - 1, a.H);
    const RowsK B = c0 < c1 ? rows_k(a.W + (size_t)c0 * a.H, c1 - 1 - c0, a.H) : rows_k(a.W, 0, a.H);
    gemm256<false, false>(A, B, a.H / kBK, acc, lds, load_rows);
  }
  // the lane's indices again, from an opaque copy of the lane id (see fwd_tiles)
  int le = lane;
  asm volatile("" : "+v"(le));
#pragma unroll
  for (int mi = kTailRows; mi < kMI; ++mi) ri[mi] = a.rowinfo[i0 + acc_row(wm, mi, le)];
  uint16_t* dzs = a.dZ + (size_t)sc * a.bg.S_pad;
  // The dz values go through LDS (free after the main loop) so that every
  // global store writes whole rows.  LDS tile: 256 rows x 512 bytes; the
  // 16-byte unit u of row r sits at r * 512 + 16 (u ^ (r & 31)), so the 32
  // rows that one store from the accumulators touches fall on different
  // banks and a row read back is still 512 contiguous bytes of one row.
  char* stage = reinterpret_cast<char*>(lds);
  auto put = [&](int r, int c, const float (&d)[4]) {
    const uint32_t off = 512u * r + 16u * ((c >> 3) ^ (r & 31)) + 8u * ((c >> 2) & 1);
    *reinterpret_cast<uint2*>(stage + off) = make_uint2(pack_bf16x2(d[0], d[1]), pack_bf16x2(d[2], d[3]));
  };
  // this wave's rows all active and 128 columns all inside the split
  // (wave-uniform; false only on the last row tile and last column tile)
  const int wc0 = j * kBN + 128 * wn;  // first column of the wave within the split
  const bool full = i0 + kWaveRows * wm + kWaveRows <= n_act && wc0 + 128 <= valid_s;
#pragma unroll
  for (int mi = 0; mi < kMI; ++mi) {
    const int r = acc_row(wm, mi, le);
    const bool rvalid = i0 + r < n_act;
    const float L = ri[mi].x, gi = ri[mi].y;
    const int yl = __float_as_int(ri[mi].z) - sbeg;  // target column within the split
    // does this lane hold its row's target column?  (rare)
    const int tl = yl - wc0;
    const bool hit = tl >= 0 && tl < 128 && ((tl >> 2) & (kLPR - 1)) == row_lane(le);
    if (full && !__builtin_amdgcn_ballot_w64(hit)) {
      // every element is off-target, active and inside the split: the same
      // formula with delta = 0, without the per-element tests
#pragma unroll
      for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
        for (int q = 0; q < kQL; ++q) {
          const int c = acc_col4(wn, ni, q, le);
          float d[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) d[e] = gi * (0.f - rlk_exp(acc.c[mi][ni][4 * q + e] - L));
          put(r, c, d);
        }
    } else {
#pragma unroll
      for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
        for (int q = 0; q < kQL; ++q) {
          // wave-uniform: the group's columns start at 128 wn + kBlk ni + 4 kLPR q
          if (j * kBN + 128 * wn + kBlk * ni + 4 * kLPR * q >= a.bg.S_pad) continue;  // never stored
          const int c = acc_col4(wn, ni, q, le);
          const int vl0 = j * kBN + c;
          float d[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int vl = vl0 + e;
            const float p = rlk_exp(acc.c[mi][ni][4 * q + e] - L);
            const float delta = (vl == yl) ? 1.f : 0.f;
            d[e] = (rvalid && vl < valid_s) ? gi * (delta - p) : 0.f;
          }
          put(r, c, d);
        }
    }
  }
  __syncthreads();
  // wave w stores tile rows kBM / kWaves * w ..: two rows per instruction,
  // lane l the 16-byte unit l & 31 of row 2 it + (l >> 5); units past the
  // split's padded width belong to the next split and are not written
  constexpr int kRowsW = kBM / kWaves;
  const int u = le & 31;
  const int col = j * kBN + 8 * u;  // column within the split
  if (col < a.bg.S_pad) {
#pragma unroll
    for (int it = 0; it < kRowsW / 2; ++it) {
      const int r = kRowsW * w + 2 * it + (le >> 5);
      const u32x4 v = *reinterpret_cast<const u32x4*>(stage + 512u * r + 16u * (u ^ (r & 31)));
      // streaming store: dz is read back only by the next launch, so it
      // should not displace the W and h lines the other tiles still use
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dzs + (size_t)(i0 + r) * a.bg.ldz + col));
    }
  }
}
#endif

// dz of the group from saved logits (the forward's kSave output, same split
// layout as dZ) instead of a recomputed tile: the same z bits, primitives
// and rounding as dz_tiles, so the same dz bits.  One thread per 8
// consecutive dZ columns of one compacted row; grid (G * S_pad / 8 / 256,
// min(T_pad, 65535)), rows blockIdx.y, + gridDim.y, ... (grid.y holds at
// most 65535); rows past the active row tiles are left alone (never read).
#ifndef RLK_ENGINE_W8
__global__ __launch_bounds__(256) void dz_saved(const float* __restrict__ zsave, int64_t ldzs,
                                                 const int32_t* __restrict__ idx, const float4* __restrict__ rowinfo,
                                                 const int32_t* __restrict__ n_act_p, SplitGeom gm, BwdGeom bg,
                                                 uint16_t* __restrict__ dZ) {
  const int col0 = 8 * (blockIdx.x * 256 + threadIdx.x);  // column within the group's dZ row
  if (col0 >= bg.ldz) return;
  const int n_act = *n_act_p;
  const int rows = ((n_act + kBM - 1) / kBM) * kBM;
  const int sc = col0 / bg.S_pad, vl0 = col0 - sc * bg.S_pad;
  const int sbeg = (bg.c_lo + sc) * gm.S;
  const int valid_s = max(0, min(gm.S, gm.V - sbeg));
  for (int i = blockIdx.y; i < rows; i += gridDim.y) {
    float d[8];
    if (i < n_act) {
      const float4 ri = rowinfo[i];
      const float L = ri.x, gi = ri.y;
      const int yl = __float_as_int(ri.z) - sbeg;
      // 16-byte aligned: ldzs, S_pad and col0 are multiples of 4
      const float4* zr = reinterpret_cast<const float4*>(zsave + (size_t)idx[i] * ldzs + (size_t)bg.c_lo * bg.S_pad + col0);
      const float4 z0 = zr[0], z1 = zr[1];
      const float z[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int vl = vl0 + e;
        if (vl < valid_s) {
          const float p = rlk_exp(z[e] - L);
          const float delta = (vl == yl) ? 1.f : 0.f;
          d[e] = gi * (delta - p);
        } else {
          d[e] = 0.f;
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) d[e] = 0.f;
    }
    *reinterpret_cast<u32x4*>(dZ + (size_t)i * bg.ldz + col0) =
        u32x4{pack_bf16x2(d[0], d[1]), pack_bf16x2(d[2], d[3]), pack_bf16x2(d[4], d[5]), pack_bf16x2(d[6], d[7])};
  }
}
#endif

// MN-mode loader over a row-major matrix: k-row t of k-block kt is matrix
// row kBK kt + t at this tile's columns (dz columns for grad_W's A operand,
// compacted hidden rows for its B operand).  base: matrix + first column of
// the tile; off[i]: (k-row * ld + column of piece i) in bytes.
struct ColsMN {
  const char* base;
  uint32_t off[kDma];
  size_t kstride;  // bytes per k-block
  __device__ __forceinline__ void one(int i, int kt, uint32_t m0w) const {
    dma16(base + kt * kstride, off[i], m0w + 1024u * i);
  }
  __device__ __forceinline__ void dma(int kt, uint32_t m0w) const {
#pragma unroll
    for (int i = 0; i < kDma; ++i) one(i, kt, m0w);
  }
};

// Columns [c0, c0 + 256) of a row-major matrix with leading dimension ld,
// piece columns clamped to ncol - 8.
__device__ __forceinline__ ColsMN cols_mn(const uint16_t* m, int c0, int ncol, int ld) {
  ColsMN L;
  L.base = reinterpret_cast<const char*>(m + c0);
  L.kstride = (size_t)2 * kBK * ld;
#pragma unroll
  for (int i = 0; i < kDma; ++i) {
    const int kr = dma_mn_krow(i);
    const int col = min(c0 + dma_mn_piece(kr) * 8, ncol - 8) - c0;
    L.off[i] = (uint32_t)(2 * ((size_t)kr * ld + col));
  }
  return L;
}

// MN-mode loader over the group's vocabulary rows of W: k-block kt of the
// group -> split sc = kt / kbps (kbps = S_pad / kBK k-blocks per split),
// rows (c_lo + sc) * S + kBK (kt - sc kbps) + 0 .. kBK-1, clamped to V - 1
// (those rows meet dz = 0).  A k-block never straddles two splits (S_pad is
// a multiple of kBK).  The split index is (kt * rcp) >> 32 with the
// reciprocal rcp = ceil(2^32 / kbps) (2^32 when kbps = 1), exact while
// kt kbps < 2^32 (kt < 32 kbps and kbps < 4096 here), so the main loop
// divides nothing; each load then costs one clamp and one multiply-add per
// lane.
struct WRowsMN {
  const char* base;     // W + first column of the tile
  uint32_t krow[kDma];  // k-row of piece i
  uint32_t col2[kDma];  // byte offset of piece i's column
  int H, S, kbps, c_lo, V;
  uint64_t rcp;
  __device__ __forceinline__ void one(int i, int kt, uint32_t m0w) const {
    const int sc = (int)(((uint64_t)(uint32_t)kt * rcp) >> 32);
    const int r0 = min((c_lo + sc) * S + kBK * (kt - sc * kbps), V - 1);
    const uint32_t last = (uint32_t)(V - 1 - r0);  // rows past it are clamped
    dma16(base + (size_t)r0 * (2 * H), min(krow[i], last) * (uint32_t)(2 * H) + col2[i], m0w + 1024u * i);
  }
  __device__ __forceinline__ void dma(int kt, uint32_t m0w) const {
#pragma unroll
    for (int i = 0; i < kDma; ++i) one(i, kt, m0w);
  }
};

// grad_W rows of the group's splits: C[v][n] = sum_t dz[t][v] h[t][n], the
// chain over active rows t ascending (K padded to 64 with zero dz rows).
// Both operands are MN mode.  Written once, fp32.  Tile id: (H tile, v tile),
// in groups of 4 H tiles: an XCD's ~32 running tiles are then 4 H tiles x 8
// v tiles, and the h columns it keeps re-reading (4 tiles of all active
// rows) stay small (measured against groups of 2, 8 and 16: the fastest).
constexpr int kGradWGroup = 4;
__device__ __forceinline__ void gradw_tile(GradWArgs a, int id, int n_act, u32x4* lds) {
  int nt, vt;
  grouped_tile(id, a.n_tiles, nt, vt, a.bg.G * a.tps, min(kGradWGroup, a.n_tiles));
  const int sc = vt / a.tps, j = vt - sc * a.tps;
  const int sbeg = (a.bg.c_lo + sc) * a.gm.S;
  const int valid_s = max(0, min(a.gm.S, a.gm.V - sbeg));
  const int v0 = j * kBM;  // within the split
  if (v0 >= valid_s) return;
  const int n0 = nt * kBN;
  const int tid = threadIdx.x;
  const ColsMN A = cols_mn(a.dZ + (size_t)sc * a.bg.S_pad, v0, a.bg.S_pad, a.bg.ldz);
  const ColsMN B = cols_mn(a.hA, n0, a.H, a.H);
  Acc acc;
  acc_zero(acc);
  // the accumulators enter the engine in accumulator registers (see gradh_tile)
#pragma unroll
  for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) asm volatile("" : "+a"(acc.c[mi][ni]));
  // no active rows: grad_W is zero
  if (n_act > 0) gemm256<true, true>(A, B, (n_act + kBK - 1) / kBK, acc, lds);
  const int lane = tid & 63, w = tid >> 6, wm = wave_m(w), wn = wave_n(w);
  float* out = a.grad_W + (size_t)sbeg * a.H;
#pragma unroll
  for (int mi = 0; mi < kMI; ++mi) {
    const int v = v0 + acc_row(wm, mi, lane);
    if (v >= valid_s) continue;
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
      for (int q = 0; q < kQL; ++q) {
        if (n0 + 128 * wn + kBlk * ni + 4 * kLPR * q >= a.H) continue;  // wave-uniform
        const AccBlk& c = acc.c[mi][ni];
        *reinterpret_cast<float4*>(out + (size_t)v * a.H + n0 + acc_col4(wn, ni, q, lane)) =
            make_float4(c[4 * q], c[4 * q + 1], c[4 * q + 2], c[4 * q + 3]);
      }
  }
}

// grad_h of the group: acc[i][n] (+)= sum_v dz[i][v] W[v][n] over the
// group's padded columns.  A (dz rows) is K mode, B (W rows) MN mode.  The
// fp32 chain continues across groups through ghacc (exact store/load); after
// the last group it is rounded to bf16 once and written to the row's place.
// kFirst / kLast: the group is the first / last one (compile-time, so that
// the accumulators never merge across a branch).  Tile id: (row tile, H tile).
//
// kPart: the tile's rows in two passes, id = 2 tile + p.  With R = kWaveRows
// / 2 rows per pass, pass p reads the dz tile from R p rows further down and
// every wave computes only its first kMI / 2 row blocks, i.e. tile rows
// R p + kWaveRows wm + 0 .. R - 1 (the two passes cover all of them); only the waves whose load
// rows meet those rows load the dz tile.  Twice the workgroups, each with
// half the MFMAs per k-block and three quarters of the loads: the k-block
// is then bound by its loads at ~70 % of a whole tile's time.  For
// batches whose few grad_h tiles would each run the vocabulary-long chain
// on a compute unit of their own while most units idle.  Every element is
// the same MFMA chain as in a whole tile.
template <bool kFirst, bool kLast, bool kPart>
__device__ __forceinline__ void gradh_tile(GradHArgs a, int id, int rtiles, int n_act, u32x4* lds) {
  constexpr int kPasses = kPart ? 2 : 1;
  constexpr int kBlocks = kMI / kPasses;  // row blocks per wave
  const int pass = id % kPasses;
  int rt, nt;
  grouped_tile(id / kPasses, rtiles, rt, nt, a.n_tiles, row_group(rtiles));
  const int i0 = rt * kBM + kBlk * kBlocks * pass, n0 = nt * kBN;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wm = wave_m(w), wn = wave_n(w);
  Acc acc;
  acc_zero(acc);
  if (!kFirst) {
    // continue the chain from the previous groups (rows/columns outside
    // the problem read a clamped, valid address; they are never stored)
#pragma unroll
    for (int mi = 0; mi < kBlocks; ++mi) {
      const float* src = a.ghacc + (size_t)min(i0 + acc_row(wm, mi, lane), n_act - 1) * a.H;
#pragma unroll
      for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
        for (int q = 0; q < kQL; ++q) {
          const float4 v = *reinterpret_cast<const float4*>(src + min(n0 + acc_col4(wn, ni, q, lane), a.H - 4));
          acc.c[mi][ni][4 * q] = v.x;
          acc.c[mi][ni][4 * q + 1] = v.y;
          acc.c[mi][ni][4 * q + 2] = v.z;
          acc.c[mi][ni][4 * q + 3] = v.w;
        }
      // bound the loads in flight (each block lands in its accumulator)
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // the accumulators enter the engine in accumulator registers: left to
  // itself, the register allocator splits reloaded chain values between the
  // register files and spills them, and with zeroed ones it rotates a block
  // through vector registers on every k-block (a wait on an MFMA result)
#pragma unroll
  for (int mi = 0; mi < kBlocks; ++mi)
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) asm volatile("" : "+a"(acc.c[mi][ni]));
  // (a pass's tile runs past the row tile; rows past dZ's last repeat it)
  const RowsK A = rows_k(a.dZ + (size_t)i0 * a.bg.ldz, min(kBM - 1, a.bg.T_pad - 1 - i0), a.bg.ldz);
  WRowsMN B;
  B.base = reinterpret_cast<const char*>(a.W + n0);
  B.H = a.H;
  B.S = a.gm.S;
  B.kbps = a.bg.S_pad / kBK;
  B.rcp = ((uint64_t(1) << 32) + (uint64_t)B.kbps - 1) / (uint64_t)B.kbps;
  B.c_lo = a.bg.c_lo;
  B.V = a.gm.V;
#pragma unroll
  for (int i = 0; i < kDma; ++i) {
    B.col2[i] = 2 * (min(n0 + dma_mn_piece(dma_mn_krow(i)) * 8, a.H - 8) - n0);
    B.krow[i] = (uint32_t)dma_mn_krow(i);
  }
  if constexpr (kPart) {
    static_assert(8 * kDma <= kBlk * kBlocks && kWaveRows % (8 * kDma) == 0, "a wave's load rows in one half of its wave row");
    const int wl = __builtin_amdgcn_readfirstlane(w);
    if ((8 * kDma * wl) % kWaveRows < kBlk * kBlocks)  // this wave's load rows hold computed rows
      gemm256<false, true, kBlocks, true>(A, B, a.bg.ldz / kBK, acc, lds);
    else
      gemm256<false, true, kBlocks, false>(A, B, a.bg.ldz / kBK, acc, lds);
  } else {
    gemm256<false, true>(A, B, a.bg.ldz / kBK, acc, lds);
  }
  // output rows of this lane's active rows: loaded after the vocabulary-long
  // chain (one load latency per tile; held through the loop they would take
  // registers the loop needs)
  int dst[kMI];
  if (kLast) {
#pragma unroll
    for (int mi = 0; mi < kBlocks; ++mi) dst[mi] = a.idx[min(i0 + acc_row(wm, mi, lane), n_act - 1)];
  }
#pragma unroll
  for (int mi = 0; mi < kBlocks; ++mi) {
    const int i = i0 + acc_row(wm, mi, lane);
    if (i >= n_act) continue;
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
      for (int q = 0; q < kQL; ++q) {
        if (n0 + 128 * wn + kBlk * ni + 4 * kLPR * q >= a.H) continue;  // wave-uniform
        const int n = n0 + acc_col4(wn, ni, q, lane);
        const AccBlk& c = acc.c[mi][ni];
        if (kLast)
          *reinterpret_cast<uint2*>(a.grad_h + (size_t)dst[mi] * a.H + n) =
              make_uint2(pack_bf16x2(c[4 * q], c[4 * q + 1]), pack_bf16x2(c[4 * q + 2], c[4 * q + 3]));
        else
          *reinterpret_cast<float4*>(a.ghacc + (size_t)i * a.H + n) =
              make_float4(c[4 * q], c[4 * q + 1], c[4 * q + 2], c[4 * q + 3]);
      }
  }
}

// The group's grad_h and grad_W tiles in one launch.  The grad_h tiles
// (K = the group's whole padded vocabulary, few of them) take the first
// blocks and start first; the grad_W tiles (K = active rows, many short
// ones) follow and fill the compute units that the grad_h tiles leave free,
// then all of them as the grad_h tiles finish.  Either part is skipped when
// its output pointer is NULL.
// kPart: grad_h tiles in two row passes (see gradh_tile).
template <bool kFirst, bool kLast, bool kPart>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(RLK_WAVES / 4, RLK_WAVES / 4))) void grad_tiles(GradHArgs ha,
                                                                                               GradWArgs wa) {
  __shared__ u32x4 lds[kLdsU4];
  const int n_act = __builtin_amdgcn_readfirstlane(*ha.n_act);
  const int rtiles = (n_act + kBM - 1) / kBM;
  const int nh = ha.grad_h ? rtiles * ha.n_tiles * (kPart ? 2 : 1) : 0;
  const int nh_blocks = 8 * ((nh + 7) >> 3);
  const int bid = blockIdx.x;
  if (bid < nh_blocks) {
    const int id = xcd_tile(nh, bid);
    if (id >= 0) gradh_tile<kFirst, kLast, kPart>(ha, id, rtiles, n_act, lds);
    return;
  }
  // nh_blocks is a multiple of 8: block bid - nh_blocks runs on the same XCD
  const int nw = wa.grad_W ? wa.n_tiles * wa.bg.G * wa.tps : 0;
  const int id = xcd_tile(nw, bid - nh_blocks);
  if (id >= 0) gradw_tile(wa, id, n_act, lds);
}


// Standalone per-token objective (rlk_rl_token_loss).  One thread per token.
#ifndef RLK_ENGINE_W8
__global__ __launch_bounds__(256) void rl_token_loss(RlLossArgs a) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= a.T) return;
  float L = 0.f, gt = 0.f;
  if (a.y[t] != a.ignore_index) rl_token(a, t, a.logp[t], L, gt);
  if (a.loss) a.loss[t] = L;
  if (a.g) a.g[t] = gt;
}
#endif

// ---------------------------------------------------------------------------
// Benchmark only: the MFMA ceiling of the part under realistic operands.
// Eight waves per workgroup (two per SIMD), each holding the eight-wave
// tile kernels' 64 x 128 fp32 wave tile in registers and issuing nothing but
// the engine's MFMA instruction (32 16 x 16 x 32 or 8 32 x 32 x 16 blocks
// per operand set), cycling through register sets of the caller's random
// bf16 data so the matrix cores see realistic bit toggling; no memory
// traffic in the loop.  Either shape does 2^20 FLOP per wave per
// iteration.  src: 24 * 512 16-byte pieces; out: one float per thread
// (keeps the result).
// ---------------------------------------------------------------------------
#ifndef RLK_ENGINE_W8
constexpr int kCeilThreads = 512;
__global__ __launch_bounds__(kCeilThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void mfma_ceiling(
    const u32x4* __restrict__ src, float* __restrict__ out, int iters) {
#if RLK_MFMA == 16
  constexpr int kS = 2, kA = 4, kB = 8;  // operand sets; A and B fragments per set (4 x 8 blocks)
#else
  constexpr int kS = 4, kA = 2, kB = 4;  // 2 x 4 blocks of 32 x 32
#endif
  bf16x8 fa[kS][kA], fb[kS][kB];
#pragma unroll
  for (int s = 0; s < kS; ++s) {
#pragma unroll
    for (int j = 0; j < kA; ++j)
      fa[s][j] = __builtin_bit_cast(bf16x8, src[(s * (kA + kB) + j) * kCeilThreads + threadIdx.x]);
#pragma unroll
    for (int j = 0; j < kB; ++j)
      fb[s][j] = __builtin_bit_cast(bf16x8, src[(s * (kA + kB) + kA + j) * kCeilThreads + threadIdx.x]);
  }
  AccBlk c[kA * kB];
#pragma unroll
  for (int j = 0; j < kA * kB; ++j) c[j] = AccBlk{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < kS; ++s)
#pragma unroll
      for (int j = 0; j < kA * kB; ++j)
#if RLK_MFMA == 16
        c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[s][j % kB], fa[s][j / kB], c[j], 0, 0, 0);
#else
        c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[s][j % kB], fa[s][j / kB], c[j], 0, 0, 0);
#endif
  }
  float t = 0.f;
#pragma unroll
  for (int j = 0; j < kA * kB; ++j)
#pragma unroll
    for (int i = 0; i < kBlk * kBlk / 64; ++i) t += c[j][i];
  out[blockIdx.x * kCeilThreads + threadIdx.x] = t;
}
#endif

// ---------------------------------------------------------------------------
// Deterministic dense product C = A B^T on the same tile engine: every
// element is one MFMA chain over k ascending, whatever the tile it falls in,
// so a row of C depends only on its row of A (and B).  Tile id: (row tile of
// A, row tile of B).  Rows past M / N are clamped loads that are never
// stored.  c_bf16: store bf16 (round to nearest even, once) instead of fp32.
// ---------------------------------------------------------------------------
#ifndef RLK_ENGINE_W8
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(RLK_WAVES / 4, RLK_WAVES / 4))) void gemm_tiles(GemmArgs a) {
  __shared__ u32x4 lds[kLdsU4];
  const int id = xcd_tile(a.rtiles * a.ctiles, blockIdx.x);
  if (id < 0) return;
  int rt, ct;
  grouped_tile(id, a.rtiles, rt, ct, a.ctiles, row_group(a.rtiles));
  const int m0 = rt * kBM, n0 = ct * kBN;
  const RowsK LA = rows_k(a.A + (size_t)m0 * a.K, min(kBM, a.M - m0) - 1, a.K);
  const RowsK LB = rows_k(a.B + (size_t)n0 * a.K, min(kBN, a.N - n0) - 1, a.K);
  Acc acc;
  acc_zero(acc);
  gemm256<false, false>(LA, LB, a.K / kBK, acc, lds);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wm = wave_m(w), wn = wave_n(w);
#pragma unroll
  for (int mi = 0; mi < kMI; ++mi) {
    const int i = m0 + acc_row(wm, mi, lane);
    if (i >= a.M) continue;
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
      for (int q = 0; q < kQL; ++q) {
        const int j = n0 + acc_col4(wn, ni, q, lane);
        const AccBlk& c = acc.c[mi][ni];
        const float v0 = c[4 * q], v1 = c[4 * q + 1], v2 = c[4 * q + 2], v3 = c[4 * q + 3];
        if (a.c_bf16) {
          uint16_t* row = static_cast<uint16_t*>(a.C) + (size_t)i * a.ldc;
          const uint32_t p01 = pack_bf16x2(v0, v1), p23 = pack_bf16x2(v2, v3);
          if (j + 3 < a.N) {
            *reinterpret_cast<uint2*>(row + j) = make_uint2(p01, p23);
          } else {
            if (j < a.N) row[j] = (uint16_t)(p01 & 0xFFFFu);
            if (j + 1 < a.N) row[j + 1] = (uint16_t)(p01 >> 16);
            if (j + 2 < a.N) row[j + 2] = (uint16_t)(p23 & 0xFFFFu);
          }
        } else {
          float* row = static_cast<float*>(a.C) + (size_t)i * a.ldc;
          if (j + 3 < a.N) {
            *reinterpret_cast<float4*>(row + j) = make_float4(v0, v1, v2, v3);
          } else {
            if (j < a.N) row[j] = v0;
            if (j + 1 < a.N) row[j + 1] = v1;
            if (j + 2 < a.N) row[j + 2] = v2;
          }
        }
      }
  }
}
#endif


// hA[i] = h[idx[i]] for active rows i < n_act, zero rows for n_act <= i <
// rows; rowinfo (optional) [i] = {lse, g, target, 0} of the row ({0, 0, -1,
// 0} past n_act).  An active row whose target lies outside [0, V) has no
// defined log-probability (the forward wrote NaN for it): its g becomes NaN,
// so that the backward's gradients show it (NaN in the row's grad_h and in
// every grad_W element it reaches) instead of silently dropping the target
// term.  Block 256, 16-byte pieces.
#ifndef RLK_ENGINE_W8
__global__ __launch_bounds__(256) void gather_rows(const uint16_t* __restrict__ h, const int32_t* __restrict__ idx,
                                                   const int32_t* __restrict__ n_act_p, int rows, int H, int V,
                                                   const int32_t* __restrict__ y, const float* __restrict__ lse,
                                                   const float* __restrict__ g, uint16_t* __restrict__ hA,
                                                   float4* __restrict__ rowinfo) {
  const int n_act = *n_act_p;
  // rows blockIdx.x, + gridDim.x, ... (a launch holds at most 2^31 - 1
  // threads along x, so the grid may be smaller than `rows`)
  for (int i = blockIdx.x; i < rows; i += gridDim.x) {
    u32x4* dst = reinterpret_cast<u32x4*>(hA + (size_t)i * H);
    if (i < n_act) {
      const int t = idx[i];
      const u32x4* src = reinterpret_cast<const u32x4*>(h + (size_t)t * H);
      for (int p = threadIdx.x; p < H / 8; p += 256) dst[p] = src[p];
      if (rowinfo && threadIdx.x == 0) {
        const int yt = y[t];
        const float gt = (yt >= 0 && yt < V) ? g[t] : __builtin_nanf("");
        rowinfo[i] = make_float4(lse[t], gt, __int_as_float(yt), 0.f);
      }
    } else {
      for (int p = threadIdx.x; p < H / 8; p += 256) dst[p] = u32x4{0u, 0u, 0u, 0u};
      if (rowinfo && threadIdx.x == 0) rowinfo[i] = make_float4(0.f, 0.f, __int_as_float(-1), 0.f);
    }
  }
}
#endif

// Zero the grad_h rows of inactive rows.  grid T, block 256.
#ifndef RLK_ENGINE_W8
__global__ __launch_bounds__(256) void zero_rows(const int32_t* __restrict__ y, int T, int ignore_index, int H,
                                                 uint16_t* __restrict__ grad_h) {
  for (int t = blockIdx.x; t < T; t += gridDim.x) {  // (as in gather_rows)
    if (y[t] != ignore_index) continue;
    for (int k = threadIdx.x; k < H; k += 256) grad_h[(size_t)t * H + k] = 0;
  }
}
#endif

RLK_ENGINE_END  // namespace rlk
