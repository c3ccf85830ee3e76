// 256 x 256 bf16 MFMA tile engine for gfx950.
//
// C[256 x 256] (fp32, in registers) = sum over k of A[m][k] * B[n][k], with
// k ascending in steps of 16: one v_mfma_f32_32x32x16_bf16 chain per output
// element, no split-K.  The tiling below (waves, LDS staging, swizzles,
// operand layouts) never changes a result bit: every element is the same
// chain of MFMA steps over the same k values.
//
// 256 threads = 4 waves, one per SIMD; wave w owns rows 128*(w & 1) .. +128
// and columns 128*(w >> 1) .. +128 of the tile, as 4 x 4 blocks of 32 x 32
// (256 accumulator registers).  A 128-column vocabulary chunk of a row
// therefore lives inside one wave.
//
// MFMA register layouts (32x32x16 bf16, D = X * Y^T):
//   X operand, lane l: row (l & 31), k = 8*(l >> 5) + 0..7 of the k step
//   Y operand, lane l: row (l & 31), same k
//   D, lane l, element r (0..15): X-row 8*(r>>2) + 4*(l>>5) + (r&3), Y-row l & 31
// X and Y use the same k assignment, so a step sums exactly its 16 k values.
// The tile's B fragments go in as X and its A fragments as Y, so that lane l
// of block (mi, ni) holds tile row 32 mi + (l & 31) and, in elements
// 4g .. 4g+3, the four consecutive tile columns 32 ni + 8 g + 4 (l >> 5) + 0..3:
// a row's values sit in one lane pair (l, l ^ 32) and stores write 4
// consecutive columns per lane.
//
// Operands come in one of two global layouts:
//   K mode : rows of the operand are contiguous in k (h [T,H], W [V,H], dz
//            [T, v] as the A operand of h-gradients).  LDS tile: 256 rows x
//            64 k (eight 16-byte pieces per row); fragments by ds_read_b128.
//   MN mode: rows are contiguous in m/n, consecutive k are separate rows
//            (W [V,H] and h [T,H] when the reduction runs over v or t).  LDS
//            tile: 64 k-rows x 256 columns; fragments by two
//            ds_read_b64_tr_b16, each giving a lane 4 consecutive k of one
//            column: within a group of 16 lanes, supplier lane 4j+q points at
//            row j, columns 4q..4q+3 and lane i receives column i of rows
//            0..3.
// Both LDS layouts are XOR-swizzled so that the 16 lanes served per LDS
// cycle hit distinct banks.
//
// Pipelined: k-blocks of 64 are loaded straight from global memory into two
// LDS stages, one k-block ahead of the MFMAs.  A K-mode row contributes 128
// contiguous bytes per k-block (one full cache line), which halves the
// number of memory requests per byte compared with 32-wide k-blocks: the
// direct loads are limited by the requests a CU can keep in flight.
#pragma once

#include "rlk_device.h"

namespace rlk {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
// native 16-byte vector (HIP's uint4 is a struct, which keeps staging
// registers in private memory)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 256, kBN = 256, kBK = 64, kThreads = 256;
constexpr int kMI = 4, kNI = 4;            // 32 x 32 blocks per wave
constexpr int kKK = kBK / 16;              // MFMA k steps per k-block
constexpr int kSegs = kBK / 8;             // 16-byte pieces per K-mode row
constexpr int kDma = kBK / 8;              // direct-load instructions per wave per operand per k-block
constexpr int kTileU4 = 256 * kSegs;       // u32x4 per operand tile (32 KB)
constexpr int kTileU4Check = 256 * kBK / 8;
static_assert(kTileU4 == kTileU4Check, "tile = 256 rows x kBK bf16");
constexpr int kStageU4 = 2 * kTileU4;      // A + B (64 KB)
constexpr int kNS = 2;                     // LDS stages
constexpr int kLdsU4 = kNS * kStageU4;     // 128 KB

// K-mode slot of (row, 16-byte piece seg), 128-byte rows: two consecutive
// rows fill a 256-byte bank row and the piece index is xor-ed with
// (row >> 1) & 7, so 16 consecutive rows of one k piece cover all banks.
__device__ __forceinline__ int slot_k(int row, int seg) { return row * kSegs + (seg ^ ((row >> 1) & 7)); }

// MN-mode slot of (k-row, 16-byte piece p of 32): 64-byte blocks of the row
// xor-ed with (k-row & 7).
__device__ __forceinline__ int slot_mn(int krow, int p) {
  return krow * 32 + ((((p >> 2) ^ (krow & 7)) << 2) | (p & 3));
}

// ---- operand fragments from LDS ----------------------------------------------
__device__ __forceinline__ bf16x8 frag_k(const u32x4* __restrict__ tile, int r0, int kk, int lane) {
  const int row = r0 + (lane & 31);
  const int seg = 2 * kk + (lane >> 5);
  return __builtin_bit_cast(bf16x8, tile[slot_k(row, seg)]);
}

__device__ __forceinline__ bf16x8 frag_mn(const u32x4* __restrict__ tile, int c0, int kk, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int col = c0 + 16 * (g & 1) + 4 * (s & 3);
  const int p = col >> 3, half = (col >> 2) & 1;
  const int krow = 16 * kk + 8 * (g >> 1) + (s >> 2);
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  const char* base = reinterpret_cast<const char*>(tile);
  const lds_bf16x4* p0 = (const lds_bf16x4*)(base + slot_mn(krow, p) * 16 + half * 8);
  const lds_bf16x4* p1 = (const lds_bf16x4*)(base + slot_mn(krow + 4, p) * 16 + half * 8);
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(const_cast<lds_bf16x4*>(p0));
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(const_cast<lds_bf16x4*>(p1));
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

template <bool A_MN>
__device__ __forceinline__ bf16x8 frag_a(const u32x4* t, int r0, int kk, int lane) {
  if constexpr (A_MN) return frag_mn(t, r0, kk, lane);
  else return frag_k(t, r0, kk, lane);
}

// ---- global -> LDS staging (direct loads) ----------------------------------------
// Tiles are filled with global_load_lds_dwordx4: one wave instruction loads
// 64 x 16 bytes and writes them to 1 KB of LDS at its (wave-uniform) base,
// lane l at byte 16 l.  Instruction i of wave w covers tile slots
// 64 (kDma w + i) .. +64, so lane l of it fills slot s = 64 (kDma w + i) + l and
// fetches the global piece that the swizzled layout puts there:
//   K mode : row 64 w + 8 i + (l >> 3), piece (l & 7) ^ ((row >> 1) & 7)
//   MN mode: k-row 16 w + 2 i + (l >> 5),
//            piece ((((l & 31) >> 2) ^ (k-row & 7)) << 2) | (l & 3)
// (i = 0 .. kDma-1).
// No registers hold the staged data.
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void dma16(const void* g, u32x4* tile, int slot0) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)(tile + slot0), 16, 0, 0);
}

// K-mode row and piece of instruction i for this thread
__device__ __forceinline__ int dma_k_row(int i) { return 64 * (threadIdx.x >> 6) + 8 * i + ((threadIdx.x & 63) >> 3); }
__device__ __forceinline__ int dma_k_seg(int row) { return (threadIdx.x & 7) ^ ((row >> 1) & 7); }
// MN-mode k-row and piece of instruction i for this thread
__device__ __forceinline__ int dma_mn_krow(int i) { return 16 * (threadIdx.x >> 6) + 2 * i + ((threadIdx.x & 63) >> 5); }
__device__ __forceinline__ int dma_mn_piece(int krow) {
  const int l = threadIdx.x & 31;
  return (((l >> 2) ^ (krow & 7)) << 2) | (l & 3);
}
__device__ __forceinline__ int dma_slot0(int i) { return 64 * (kDma * (threadIdx.x >> 6) + i); }

// K-mode loader over kDma rows whose pointers (with the piece offset) are
// resolved once: pointer i is for row dma_k_row(i).
struct RowsK8 {
  const uint16_t* p[kDma];
  __device__ __forceinline__ void dma(int kt, u32x4* tile) const {
    const int o = kt * kBK;
#pragma unroll
    for (int i = 0; i < kDma; ++i) dma16(p[i] + o, tile, dma_slot0(i));
  }
};

// K-mode rows r of a strided matrix (row pointer base + min(r, last) * ld)
__device__ __forceinline__ RowsK8 rows_k_strided(const uint16_t* base, int last, int ld) {
  RowsK8 R;
#pragma unroll
  for (int i = 0; i < kDma; ++i) {
    const int row = dma_k_row(i);
    R.p[i] = base + (size_t)min(row, last) * ld + dma_k_seg(row) * 8;
  }
  return R;
}

// K-mode rows gathered through idx: tile row r -> idx[min(first + r, n_last)]
__device__ __forceinline__ RowsK8 rows_k_gather(const uint16_t* base, const int32_t* idx, int first, int n_last,
                                               int ld) {
  RowsK8 R;
#pragma unroll
  for (int i = 0; i < kDma; ++i) {
    const int row = dma_k_row(i);
    R.p[i] = base + (size_t)idx[min(first + row, n_last)] * ld + dma_k_seg(row) * 8;
  }
  return R;
}

// ---- main loop -------------------------------------------------------------------
struct Acc {
  f32x16 c[kMI][kNI];
};

struct Frags {
  bf16x8 a0, a1, a2, a3, b0, b1, b2, b3;
};

template <bool A_MN, bool B_MN>
__device__ __forceinline__ void load_frags(const u32x4* __restrict__ sA, const u32x4* __restrict__ sB, int ra0,
                                           int rb0, int kk, int lane, Frags& f) {
  f.a0 = frag_a<A_MN>(sA, ra0, kk, lane);
  f.a1 = frag_a<A_MN>(sA, ra0 + 32, kk, lane);
  f.a2 = frag_a<A_MN>(sA, ra0 + 64, kk, lane);
  f.a3 = frag_a<A_MN>(sA, ra0 + 96, kk, lane);
  f.b0 = frag_a<B_MN>(sB, rb0, kk, lane);
  f.b1 = frag_a<B_MN>(sB, rb0 + 32, kk, lane);
  f.b2 = frag_a<B_MN>(sB, rb0 + 64, kk, lane);
  f.b3 = frag_a<B_MN>(sB, rb0 + 96, kk, lane);
}

__device__ __forceinline__ void mma16(const Frags& f, Acc& acc) {
#define RLK_MMA(mi, ni, A, B) acc.c[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.B, f.A, acc.c[mi][ni], 0, 0, 0);
  RLK_MMA(0, 0, a0, b0) RLK_MMA(0, 1, a0, b1) RLK_MMA(0, 2, a0, b2) RLK_MMA(0, 3, a0, b3)
  RLK_MMA(1, 0, a1, b0) RLK_MMA(1, 1, a1, b1) RLK_MMA(1, 2, a1, b2) RLK_MMA(1, 3, a1, b3)
  RLK_MMA(2, 0, a2, b0) RLK_MMA(2, 1, a2, b1) RLK_MMA(2, 2, a2, b2) RLK_MMA(2, 3, a2, b3)
  RLK_MMA(3, 0, a3, b0) RLK_MMA(3, 1, a3, b1) RLK_MMA(3, 2, a3, b2) RLK_MMA(3, 3, a3, b3)
#undef RLK_MMA
}

// Wait until at most n of this thread's vector memory operations are
// outstanding (they complete in issue order, so everything older has landed).
__device__ __forceinline__ void wait_vm(int n) {
  if (n >= 2 * kDma) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}
static_assert(2 * kDma == 16, "wait_vm counts assume 16 direct loads per k-block");

// nk k-blocks of kBK.  LA / LB: loaders with dma(kt, tile) that issue this
// thread's direct global->LDS loads of k-block kt.  Two LDS stages: block kt
// is read from stage kt & 1 while block kt+1 lands in the other one.  Per
// k-block (four MFMA k steps of 16 MFMAs each):
//   read step 1 | MFMAs step 0 | read step 2 | MFMAs step 1 | read step 3 |
//   MFMAs step 2 | wait for block kt+1 and for this wave's reads, barrier,
//   issue the loads of block kt+2 into stage kt & 1, read step 0 of block
//   kt+1 | MFMAs step 3
// so the one barrier per block sits between MFMA bursts, every LDS read
// overlaps an MFMA burst, and after the barrier no wave reads stage kt & 1
// any more.  Bare s_barrier: __syncthreads() would add a release fence that
// waits for all outstanding loads, including the next block in flight.
template <bool A_MN, bool B_MN, class LA, class LB>
__device__ __forceinline__ void gemm256(const LA& la, const LB& lb, int nk, Acc& acc, u32x4* lds) {
  if (nk <= 0) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int ra0 = 128 * (w & 1), rb0 = 128 * (w >> 1);
  static_assert(kNS == 2 && kKK == 4, "schedule written for two stages of four k steps");
  la.dma(0, lds);
  lb.dma(0, lds + kTileU4);
  if (nk > 1) {
    la.dma(1, lds + kStageU4);
    lb.dma(1, lds + kStageU4 + kTileU4);
  }
  wait_vm(nk > 1 ? 2 * kDma : 0);
  __builtin_amdgcn_s_barrier();
  Frags f;
  load_frags<A_MN, B_MN>(lds, lds + kTileU4, ra0, rb0, 0, lane, f);
  for (int kt = 0; kt < nk; ++kt) {
    const u32x4* sA = lds + (kt & 1) * kStageU4;
    const u32x4* sB = sA + kTileU4;
    Frags g;
#pragma unroll
    for (int kk = 1; kk < kKK; ++kk) {
      __builtin_amdgcn_sched_barrier(0);
      load_frags<A_MN, B_MN>(sA, sB, ra0, rb0, kk, lane, g);
      __builtin_amdgcn_sched_barrier(0);
      mma16(f, acc);
      __builtin_amdgcn_sched_barrier(0);
      f = g;
    }
    if (kt + 1 < nk) {
      wait_vm(0);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      if (kt + 2 < nk) {
        u32x4* st = lds + (kt & 1) * kStageU4;
        la.dma(kt + 2, st);
        lb.dma(kt + 2, st + kTileU4);
      }
      const u32x4* nA = lds + ((kt + 1) & 1) * kStageU4;
      load_frags<A_MN, B_MN>(nA, nA + kTileU4, ra0, rb0, 0, lane, g);
    }
    __builtin_amdgcn_sched_barrier(0);
    mma16(f, acc);
    __builtin_amdgcn_sched_barrier(0);
    f = g;
  }
  __syncthreads();
}

__device__ __forceinline__ void acc_zero(Acc& acc) {
#pragma unroll
  for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) acc.c[mi][ni] = f32x16{};
}

// Tile-local row held by lane l in block mi of wave (wm, *).
__device__ __forceinline__ int acc_row(int wm, int mi, int lane) { return 128 * wm + 32 * mi + (lane & 31); }

// Tile-local column of elements 4g .. 4g+3 (first of four) of block ni for
// lane l in wave (*, wn).
__device__ __forceinline__ int acc_col4(int wn, int ni, int g, int lane) {
  return 128 * wn + 32 * ni + 8 * g + 4 * (lane >> 5);
}

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2).  Give XCD x the contiguous range [x*per, (x+1)*per) of tile ids so
// that the tiles running together on one XCD share operand rows in its L2.
// The grid must hold 8*per blocks; ids >= the tile count exit.
__device__ __forceinline__ int xcd_tile(int per) {
  const int bid = blockIdx.x;
  return (bid & 7) * per + (bid >> 3);
}

// Tile id -> (fast index f < F, slow index c < C) in groups of GM fast
// indices: consecutive ids walk GM values of f, then the next c, so the
// ~32 tiles in flight on one XCD form a GM x (32 / GM) block of the output
// and share their operand rows in L2.
constexpr int kGroupM = 4;
__device__ __forceinline__ void grouped_tile(int id, int F, int& f, int& c, int C) {
  const int per_group = kGroupM * C;
  const int grp = id / per_group;
  const int gm = min(kGroupM, F - grp * kGroupM);
  const int within = id - grp * per_group;
  c = within / gm;
  f = grp * kGroupM + (within - c * gm);
}

}  // namespace rlk
