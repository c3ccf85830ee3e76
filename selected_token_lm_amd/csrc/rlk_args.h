// Argument records of the linear_logp kernels: plain data that the host
// fills and passes by value at launch.  They do not depend on the tile
// engine's wave count, so the four-wave and the eight-wave translation
// units (rlk_api.hip, rlk_tiles_w8.hip) share them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rlk {

// Per-token RL objective (rlk_rl_token_loss and the forward's fused mode).
struct RlLossArgs {
  const float* logp;
  const float* logp_old;
  const float* adv;
  const float* logp_ref;  // may be NULL when beta == 0
  const int32_t* y;
  int T;
  int ignore_index;
  float eps_low, eps_high, beta, scale;
  float* loss;  // may be NULL
  float* g;     // may be NULL
};

// Statistics of one row over a vocabulary range (rlk_lse_partial's output
// record, merged by rlk_lse_merge).
struct PartialRec {
  float m, s, z_target;
  uint32_t owned;
};

// Vocabulary geometry of a launch.
struct SplitGeom {
  int V;           // global vocabulary size
  int S;           // split width = ceil(V / 32)
  int cps;         // chunks per split = ceil(S / 128)
  int s0;          // first split of the processed range
  int vocab_start; // global index of row 0 of the W pointer given
};

struct TileGeom {
  int tps;  // 256-column tiles per split = ceil(S / 256)
};

// fwd_tiles: logit tiles of the active rows over a range of splits.
struct FwdArgs {
  const uint16_t* hA;  // active rows of h, compacted, zero padded to a multiple of 256
  const uint16_t* W;
  const int32_t* yA;  // targets of the active rows, compacted
  const int32_t* idx;
  const int32_t* n_act;
  int H;
  int nsplit;
  SplitGeom gm;
  TileGeom tg;
  size_t rec_stride;
  float2* rec;
  float* zt;
  float* zsave;  // kSave: fp32 logits of active rows: row t, split s, column c of
                 // the split at zsave + t * ldzs + s * zs_spad + c
  int64_t ldzs;
  int zs_spad;   // S rounded up to 64
};

// One backward group of vocabulary splits and its dz block.
struct BwdGeom {
  int c_lo;   // first split of the group
  int G;      // splits in the group
  int S_pad;  // S rounded up to 64
  int ldz;    // G * S_pad
  int T_pad;  // rows of dZ (multiple of 256)
};

// dz_tiles: recomputed logits -> dz of one group.
struct DzArgs {
  const uint16_t* hA;       // active rows of h, compacted, zero padded to T_pad
  const uint16_t* W;
  const float4* rowinfo;    // per active row {lse, g, target (bits), 0}; {0, 0, -1, 0} past n_act
  const int32_t* n_act;
  int H;
  SplitGeom gm;
  TileGeom tg;
  BwdGeom bg;
  uint16_t* dZ;
};

// grad_tiles, grad_W part: rows of the group's splits.
struct GradWArgs {
  const uint16_t* dZ;
  const uint16_t* hA;  // active rows of h, compacted, zero padded to T_pad
  const int32_t* n_act;
  int H;
  SplitGeom gm;
  BwdGeom bg;
  int tps;      // 256-row v tiles per split
  int n_tiles;  // 256-column tiles of H
  float* grad_W;  // NULL: not wanted
};

// grad_tiles, grad_h part: the fp32 chain over the group's columns.
struct GradHArgs {
  const uint16_t* dZ;
  const uint16_t* W;
  const int32_t* idx;
  const int32_t* n_act;
  int H;
  SplitGeom gm;
  BwdGeom bg;
  int n_tiles;  // 256-column tiles of H
  float* ghacc;
  uint16_t* grad_h;  // NULL: not wanted
};

// gemm_tiles: C = A B^T.
struct GemmArgs {
  const uint16_t* A;  // [M, K]
  const uint16_t* B;  // [N, K]
  int M, N, K;
  int rtiles, ctiles;
  int64_t ldc;
  int c_bf16;
  void* C;
};

}  // namespace rlk
