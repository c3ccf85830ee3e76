// 256 x 256 bf16 MFMA tile engine for gfx950.
//
// C[256 x 256] (fp32, in registers) = sum over k of A[m][k] * B[n][k], with
// k ascending in steps of 16: one v_mfma_f32_32x32x16_bf16 chain per output
// element, no split-K.  The tiling below (waves, LDS staging, swizzles,
// operand layouts) never changes a result bit: every element is the same
// chain of MFMA steps over the same k values.
//
// kWaves = 4 (one wave per SIMD) or 8 (two per SIMD, RLK_WAVES=8 at build
// time): wave w owns rows R*(w % (kWaves/2)) .. +R, R = 512 / kWaves, and
// columns 128*(w / (kWaves/2)) .. +128 of the tile, as (R/32) x 4 blocks of
// 32 x 32 (256 or 128 accumulator registers).  A 128-column vocabulary chunk
// of a row therefore lives inside one wave, and every output element is the
// same MFMA chain whatever the wave count.
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
// Pipelined: k-blocks of 64 are loaded straight from global memory into a
// ring of five 32 KB operand-tile slots in LDS (gemm256 below), 1 to 1.5
// k-blocks ahead of the MFMAs.  A K-mode row contributes 128 contiguous
// bytes per k-block (one full cache line), which halves the number of
// memory requests per byte compared with 32-wide k-blocks.
#pragma once

#include "rlk_device.h"

// The library is built from two translation units: rlk_api.hip compiles
// the engine with RLK_WAVES waves per tile (4 by default) in namespace rlk,
// and rlk_tiles_w8.hip compiles it with 8 waves (RLK_ENGINE_W8) in
// rlk::w8, so that the two flavours' device functions and kernels have
// distinct names in one library.
#ifdef RLK_ENGINE_W8
#define RLK_ENGINE_BEGIN \
  namespace rlk {        \
  inline namespace w8 {
#define RLK_ENGINE_END \
  }                    \
  }
#else
#define RLK_ENGINE_BEGIN namespace rlk {
#define RLK_ENGINE_END }
#endif

RLK_ENGINE_BEGIN

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
// native 16-byte vector (HIP's uint4 is a struct, which keeps staging
// registers in private memory)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#ifndef RLK_WAVES
#define RLK_WAVES 4
#endif
constexpr int kWaves = RLK_WAVES;
static_assert(kWaves == 4 || kWaves == 8, "four or eight waves per tile");
#ifdef RLK_ENGINE_W8
static_assert(kWaves == 8, "the eight-wave unit");
#endif
constexpr int kBM = 256, kBN = 256, kBK = 64, kThreads = 64 * kWaves;
constexpr int kWM = kWaves / 2;            // waves along the tile's rows (two along its columns)
constexpr int kWaveRows = kBM / kWM;       // tile rows per wave
constexpr int kMI = kWaveRows / 32, kNI = 4;  // 32 x 32 blocks per wave
constexpr int kMma = kMI * kNI;            // MFMAs per wave per k step
constexpr int kReads = kMI + kNI;          // fragment reads per wave per k step
constexpr int kKK = kBK / 16;              // MFMA k steps per k-block
constexpr int kSegs = kBK / 8;             // 16-byte pieces per K-mode row
constexpr int kTileU4 = 256 * kSegs;       // u32x4 per operand tile (32 KB)
constexpr int kDma = kTileU4 / 64 / kWaves;  // direct-load instructions per wave per operand per k-block
constexpr int kTileU4Check = 256 * kBK / 8;
static_assert(kTileU4 == kTileU4Check, "tile = 256 rows x kBK bf16");
constexpr int kSlots = 5;                  // LDS tile slots (a ring of operand tiles)
constexpr int kLdsU4 = kSlots * kTileU4;   // 160 KB, all of a CU's LDS

// K-mode slot of (row, 16-byte piece seg), 128-byte rows: two consecutive
// rows fill a 256-byte bank row and the piece index is xor-ed with
// (row >> 1) & 7, so 16 consecutive rows of one k piece cover all banks.
__device__ __forceinline__ int slot_k(int row, int seg) { return row * kSegs + (seg ^ ((row >> 1) & 7)); }

// MN-mode slot of (k-row, 16-byte piece p of 32): 64-byte blocks of the row
// xor-ed with (k-row & 7).
__device__ __forceinline__ int slot_mn(int krow, int p) {
  return krow * 32 + ((((p >> 2) ^ (krow & 7)) << 2) | (p & 3));
}

// Position of wave w in the tile's wave grid: row group wave_m (kWaveRows
// rows each), column group wave_n (128 columns each).
static_assert(kWM == 2 || kWM == 4, "power-of-two wave grid");
__device__ __forceinline__ int wave_m(int w) { return w & (kWM - 1); }
__device__ __forceinline__ int wave_n(int w) { return w >> (kWM == 2 ? 1 : 2); }

// ---- operand fragments from LDS ----------------------------------------------
// Per-lane LDS byte offsets of one operand's fragments within its tile,
// computed once per tile so that every read in the main loop is a base
// register plus an immediate:
//   K mode : fragment J (rows r0 + 32 J ..) of k step kk at o[kk] + 4096 J
//            (32 rows further keep the row's swizzle);
//   MN mode: fragment J (columns r0 + 32 J ..) of k step kk: reads at
//            o[J] + 8192 kk and o2[J] + 8192 kk (k-rows +16 keep the swizzle,
//            k-rows +4 do not, hence two offsets).
struct FragOffs {
  uint32_t o[4], o2[4];
};

template <bool MN>
__device__ __forceinline__ FragOffs frag_offs(int r0, int lane) {
  FragOffs f;
  if constexpr (!MN) {
    const int row = r0 + (lane & 31);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      f.o[kk] = 16u * (uint32_t)slot_k(row, 2 * kk + (lane >> 5));
      f.o2[kk] = 0u;
    }
  } else {
    const int g = lane >> 4, s = lane & 15;
    const int krow = 8 * (g >> 1) + (s >> 2);
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      const int col = r0 + 32 * J + 16 * (g & 1) + 4 * (s & 3);
      const int p = col >> 3, half = (col >> 2) & 1;
      f.o[J] = 16u * (uint32_t)slot_mn(krow, p) + 8u * half;
      f.o2[J] = 16u * (uint32_t)slot_mn(krow + 4, p) + 8u * half;
    }
  }
  return f;
}

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// Fragment J, k step kk of the tile at `tile` (a pointer into the kernel's
// LDS array, so that every read derives from that array).
template <bool MN, int J>
__device__ __forceinline__ bf16x8 frag_at(const u32x4* tile, const FragOffs& f, int kk) {
  const char* base = reinterpret_cast<const char*>(tile);
  if constexpr (!MN) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base + f.o[kk] + 4096u * J));
  } else {
    const lds_bf16x4* p0 = (const lds_bf16x4*)(base + f.o[J] + 8192u * kk);
    const lds_bf16x4* p1 = (const lds_bf16x4*)(base + f.o2[J] + 8192u * kk);
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(const_cast<lds_bf16x4*>(p0));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(const_cast<lds_bf16x4*>(p1));
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
}

// ---- global -> LDS staging (direct loads) ----------------------------------------
// Tiles are filled with global_load_lds_dwordx4: one wave instruction loads
// 64 x 16 bytes and writes them to 1 KB of LDS at its (wave-uniform) base,
// lane l at byte 16 l.  Instruction i of wave w covers tile slots
// 64 (kDma w + i) .. +64, so lane l of it fills slot s = 64 (kDma w + i) + l and
// fetches the global piece that the swizzled layout puts there:
//   K mode : row 8 (kDma w + i) + (l >> 3), piece (l & 7) ^ ((row >> 1) & 7)
//   MN mode: k-row 2 (kDma w + i) + (l >> 5),
//            piece ((((l & 31) >> 2) ^ (k-row & 7)) << 2) | (l & 3)
// (i = 0 .. kDma-1).
// No registers hold the staged data.
typedef __attribute__((address_space(3))) void lds_void;

// Written as inline assembly (uniform base in scalar registers, 32-bit lane
// offset): the compiler then does not know these loads write LDS, so it adds
// no waits of its own before later LDS reads (it cannot tell the slots
// apart for every read form).  gemm256 orders them explicitly: a slot is
// read only after wait_vm and a barrier, and refilled only after a barrier
// that follows the last reads of it.
// m0: LDS byte address of the instruction's 1 KB (wave-uniform), bound to
// the M0 register by the operand constraint, so the compiler sets M0 itself
// and knows the statement reads it; the s_nop is the one wait state that a
// write of M0 needs before an LDS-direct load.
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t m0) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(off), "s"(base), "{m0}"(m0) : "memory");
}

// K-mode row and piece of instruction i for this thread
__device__ __forceinline__ int dma_k_row(int i) { return 8 * kDma * (threadIdx.x >> 6) + 8 * i + ((threadIdx.x & 63) >> 3); }
__device__ __forceinline__ int dma_k_seg(int row) { return (threadIdx.x & 7) ^ ((row >> 1) & 7); }
// MN-mode k-row and piece of instruction i for this thread
__device__ __forceinline__ int dma_mn_krow(int i) { return 2 * kDma * (threadIdx.x >> 6) + 2 * i + ((threadIdx.x & 63) >> 5); }
__device__ __forceinline__ int dma_mn_piece(int krow) {
  const int l = threadIdx.x & 31;
  return (((l >> 2) ^ (krow & 7)) << 2) | (l & 3);
}
// LDS byte address of this wave's first direct-load slot in the tile at
// LDS byte address t (instruction i then writes 1 KB further per i).
__device__ __forceinline__ uint32_t dma_wave_base(uint32_t t) {
  return t + 1024u * kDma * (uint32_t)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}
// LDS byte address of a tile given as a pointer into the kernel's LDS array.
__device__ __forceinline__ uint32_t lds_addr(const u32x4* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void*)p);
}

// Loaders keep one uniform base pointer (scalar registers) and, per lane,
// 32-bit byte offsets of its kDma pieces (vector registers); the base moves
// by one k-block per call.  one(i, kt, m0w) issues instruction i of k-block
// kt into the tile whose wave slot base is m0w (dma_wave_base).
//
// K-mode loader: tile row r is matrix row min(r, last) at base + row * ld
// (bf16 elements).
struct RowsK {
  const char* base;
  uint32_t off[kDma];
  __device__ __forceinline__ void one(int i, int kt, uint32_t m0w) const {
    dma16(base + (size_t)kt * (2 * kBK), off[i], m0w + 1024u * i);
  }
  __device__ __forceinline__ void dma(int kt, uint32_t m0w) const {
#pragma unroll
    for (int i = 0; i < kDma; ++i) one(i, kt, m0w);
  }
};

__device__ __forceinline__ RowsK rows_k(const uint16_t* base, int last, int ld) {
  RowsK R;
  R.base = reinterpret_cast<const char*>(base);
#pragma unroll
  for (int i = 0; i < kDma; ++i) {
    const int row = dma_k_row(i);
    R.off[i] = (uint32_t)(2 * ((size_t)min(row, last) * ld + dma_k_seg(row) * 8));
  }
  return R;
}

// ---- main loop -------------------------------------------------------------------
struct Acc {
  f32x16 c[kMI][kNI];
};

struct Frags {
  bf16x8 a0, a1, a2, a3, b0, b1, b2, b3;  // a2, a3 unused with 8 waves
};

// Fragment J of a set (0..3: A blocks, 4..7: B blocks), by compile-time index.
template <int J>
__device__ __forceinline__ bf16x8& frag(Frags& f) {
  static_assert(J >= 0 && J < 8, "fragment index");
  if constexpr (J == 0) return f.a0;
  else if constexpr (J == 1) return f.a1;
  else if constexpr (J == 2) return f.a2;
  else if constexpr (J == 3) return f.a3;
  else if constexpr (J == 4) return f.b0;
  else if constexpr (J == 5) return f.b1;
  else if constexpr (J == 6) return f.b2;
  else return f.b3;
}
template <int J>
__device__ __forceinline__ const bf16x8& frag(const Frags& f) {
  return frag<J>(const_cast<Frags&>(f));
}

// Fragment J of k step kk (J < 4: A block J, else B block J - 4) of the
// k-block whose A and B tiles are at tA, tB in LDS.
template <bool A_MN, bool B_MN, int J>
__device__ __forceinline__ void load_frag(const u32x4* tA, const u32x4* tB, const FragOffs& fa, const FragOffs& fb,
                                          int kk, Frags& g) {
  if constexpr (J < 4) frag<J>(g) = frag_at<A_MN, J>(tA, fa, kk);
  else frag<J>(g) = frag_at<B_MN, J - 4>(tB, fb, kk);
}

// Fragment requested r-th (r < kReads) for a k step: A0, B0, B1, B2, B3, A1
// (, A2, A3).  MFMA j of a step uses A (j >> 2) and B (j & 3), so with reads
// completing in order the step's first MFMA waits for two reads only.
__device__ __forceinline__ constexpr int read_frag(int r) { return r == 0 ? 0 : (r <= 4 ? r + 3 : r - 4); }

// Row blocks: a wave may compute only its first kRB row blocks (kRB < kMI
// when the tile's remaining rows are known to be padding); the fragments
// and MFMAs of the others are skipped.  Fragment J (J < 4: A block J, else
// B block J - 4) is needed iff this holds.
template <int kRB>
__device__ __forceinline__ constexpr bool frag_used(int J) { return J < 4 ? J < kRB : kRB > 0; }

// Fragment J of k step kk if the wave uses it.
template <bool A_MN, bool B_MN, int kRB, int J>
__device__ __forceinline__ void load_frag_if(const u32x4* tA, const u32x4* tB, const FragOffs& fa, const FragOffs& fb,
                                             int kk, Frags& g) {
  if constexpr (frag_used<kRB>(J)) load_frag<A_MN, B_MN, J>(tA, tB, fa, fb, kk, g);
}

template <bool A_MN, bool B_MN, int kRB = kMI>
__device__ __forceinline__ void load_frags(const u32x4* tA, const u32x4* tB, const FragOffs& fa, const FragOffs& fb,
                                           int kk, Frags& g) {
  load_frag_if<A_MN, B_MN, kRB, read_frag(0)>(tA, tB, fa, fb, kk, g);
  load_frag_if<A_MN, B_MN, kRB, read_frag(1)>(tA, tB, fa, fb, kk, g);
  load_frag_if<A_MN, B_MN, kRB, read_frag(2)>(tA, tB, fa, fb, kk, g);
  load_frag_if<A_MN, B_MN, kRB, read_frag(3)>(tA, tB, fa, fb, kk, g);
  load_frag_if<A_MN, B_MN, kRB, read_frag(4)>(tA, tB, fa, fb, kk, g);
  load_frag_if<A_MN, B_MN, kRB, read_frag(5)>(tA, tB, fa, fb, kk, g);
  if constexpr (kReads == 8) {
    load_frag_if<A_MN, B_MN, kRB, read_frag(6)>(tA, tB, fa, fb, kk, g);
    load_frag_if<A_MN, B_MN, kRB, read_frag(7)>(tA, tB, fa, fb, kk, g);
  }
}

// MFMA J of a k step: block (mi, ni) = (J >> 2, J & 3); skipped for row
// blocks mi >= kRB.
template <int J, int kRB = kMI>
__device__ __forceinline__ void mma1(const Frags& f, Acc& acc) {
  constexpr int mi = J >> 2, ni = J & 3;
  if constexpr (mi < kRB)
    acc.c[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag<4 + ni>(f), frag<mi>(f), acc.c[mi][ni], 0, 0, 0);
}

// Wait until at most n (0 or kDma) of this thread's vector memory operations
// are outstanding (they complete in issue order, so everything older has
// landed).
__device__ __forceinline__ void wait_vm(int n) {
  if (n >= kDma) {
    if constexpr (kDma == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
}
// ... at most 2 kDma (the prologue's second k-block)
__device__ __forceinline__ void wait_vm_two_tiles() {
  if constexpr (kDma == 8) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
}
static_assert(kDma == 8 || kDma == 4, "wait_vm counts assume 8 or 4 direct loads per operand tile");

// Wait for all of this thread's LDS reads (s_waitcnt lgkmcnt(0) through the
// builtin, which the compiler's own wait insertion takes into account).
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// What a k step does besides its kMma MFMAs on f (16 with 4 waves, 8 with 8).
enum StepKind {
  kStepRead,   // request the next step's fragments (g: k step kk of tiles tA, tB): with 4 waves
               // one per two MFMAs, with 8 one per MFMA from the first; with kDmaB also direct
               // loads kDma/2 kB0 .. of a B tile (lb, k-block kb, wave slot base dB), one per
               // four MFMAs
  kStepSwap,   // last step of a k-block: kMma/2 MFMAs; wait until the next k-block has landed
               // and this wave's reads are done; barrier; then the next block's first-step
               // fragments (g from tA, tB: one per MFMA with 4 waves, two with 8) and one direct
               // load of an A tile per MFMA (la, k-block kb, wave slot base dA)
  kStepLast,   // MFMAs only
};

// One k step.  No LDS wait is written for the fragment reads: before each
// MFMA the compiler waits for exactly the reads it needs (LDS reads
// complete in order).  In a kStepSwap step the barrier sits halfway: by
// then every fragment of the block has long been read, so the wait before
// it is short, and after it no wave reads the block's tiles.
// Bare s_barrier: __syncthreads() would add a release fence that waits for
// all outstanding loads.  Direct loads are spread one per one to four MFMAs
// so that the address path never backs up into the wave's in-order issue.
template <bool A_MN, bool B_MN, StepKind kKind, bool kDmaB = false, int kB0 = 0, int kRB = kMI, bool kLoadA = true,
          class LA, class LB>
__device__ __forceinline__ void kstep(const Frags& f, Frags& g, Acc& acc, const u32x4* tA, const u32x4* tB,
                                      const FragOffs& fa, const FragOffs& fb, int kk, const LA& la, const LB& lb,
                                      int kb, uint32_t dA, uint32_t dB) {
#define RLK_STEP(J)                                                                              \
  if constexpr ((J) < kMma) {                                                                    \
    constexpr int kHalf = kMma / 2;                                                              \
    if constexpr (kKind == kStepRead && kReads == 8 && (J) % 2 == 0) {                           \
      load_frag_if<A_MN, B_MN, kRB, read_frag((J) / 2)>(tA, tB, fa, fb, kk, g);                  \
    } else if constexpr (kKind == kStepRead && kReads == 6 && (J) < 6) {                         \
      load_frag_if<A_MN, B_MN, kRB, read_frag(J)>(tA, tB, fa, fb, kk, g);                        \
    }                                                                                            \
    if constexpr (kKind == kStepRead && kDmaB && (J) % 4 == 1) {                                 \
      lb.one(kDma / 2 * kB0 + (J) / 4, kb, dB);                                                  \
    } else if constexpr (kKind == kStepSwap && (J) == kHalf) {                                   \
      wait_vm(kDma);                                                                             \
      wait_lds();                                                                                \
      __builtin_amdgcn_s_barrier();                                                              \
      __builtin_amdgcn_sched_barrier(0);                                                         \
    }                                                                                            \
    if constexpr (kKind == kStepSwap && (J) >= kHalf) {                                          \
      if constexpr (kReads == 8) {                                                               \
        load_frag_if<A_MN, B_MN, kRB, read_frag((J) - kHalf)>(tA, tB, fa, fb, 0, g);             \
      } else if constexpr (2 * ((J) - kHalf) < kReads) {                                         \
        load_frag_if<A_MN, B_MN, kRB, read_frag(2 * ((J) - kHalf))>(tA, tB, fa, fb, 0, g);       \
        load_frag_if<A_MN, B_MN, kRB, read_frag(2 * ((J) - kHalf) + 1)>(tA, tB, fa, fb, 0, g);   \
      }                                                                                          \
      if constexpr (kLoadA) la.one((J) - kHalf, kb, dA);                                         \
    }                                                                                            \
    mma1<J, kRB>(f, acc);                                                                        \
    __builtin_amdgcn_sched_barrier(0);                                                           \
  }
  static_assert(kDma == kMma / 2, "one direct load per MFMA in the second half of a swap step");
  static_assert(kDma == 2 * (kMma / 4), "the B tile's loads spread over two read steps");
  __builtin_amdgcn_sched_barrier(0);
  RLK_STEP(0) RLK_STEP(1) RLK_STEP(2) RLK_STEP(3) RLK_STEP(4) RLK_STEP(5) RLK_STEP(6) RLK_STEP(7)
  RLK_STEP(8) RLK_STEP(9) RLK_STEP(10) RLK_STEP(11) RLK_STEP(12) RLK_STEP(13) RLK_STEP(14) RLK_STEP(15)
#undef RLK_STEP
}

// nk k-blocks of kBK.  LA / LB: loaders with one(i, kt, m0w) / dma(kt, m0w)
// that issue this thread's direct global->LDS loads of k-block kt.  lds:
// kLdsU4 words = a ring of 5 operand-tile slots.  Tile q = 2 kt (B of block
// kt) or 2 kt + 1 (A of block kt) lives in slot q mod 5, so at any time the
// ring holds the two tiles being read, the next block's two and one more.
// Per k-block kt, four MFMA k steps of 16 MFMAs each, each requesting the
// next step's fragments:
//   step 0 | step 1     (with the loads of B of block kt+2, 1 per 4 MFMAs)
//   step 2 | step 3: 8 MFMAs, wait for block kt+1, barrier, 8 MFMAs with
//   the reads of block kt+1's step 0 and the loads of A of block kt+2
// so B tiles are issued about 1.5 blocks and A tiles 1 block before use.
// Loads past the last block repeat the last block's tile into the free slot
// (uniform load counts; nothing reads that copy); all have landed on return.
//
// kRB < kMI: this wave computes only its first kRB row blocks (the others
// are padding rows of the tile).  kLoadA = false: this wave issues none of
// its A-tile loads (the rows they cover are padding for every wave); B
// loads, barriers and waits are the same for every wave, so waves with
// different (kRB, kLoadA) run together in one tile.
//
// tail(): run once just before the last k-block's MFMAs, for loads whose
// values only the caller's epilogue needs (they land under that block's
// MFMAs and take no registers through the loop; all have landed on return).
struct NoTail {
  __device__ __forceinline__ void operator()() const {}
};

//
// nk >= 1 (callers with a possibly empty K skip the call: an early return
// here would join an all-zero accumulator path into the epilogue and make
// the register allocator shuffle, and spill, the accumulators).
template <bool A_MN, bool B_MN, int kRB = kMI, bool kLoadA = true, class LA, class LB, class Tail = NoTail>
__device__ __forceinline__ void gemm256(const LA& la, const LB& lb, int nk, Acc& acc, u32x4* lds,
                                        const Tail& tail = Tail{}) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int ra0 = kWaveRows * wave_m(w), rb0 = 128 * wave_n(w);
  static_assert(kKK == 4 && kSlots == 5, "schedule written for four k steps and five tile slots");
  // direct-load slot base of this wave in slot 0; slot s is kTileB * s further
  const uint32_t m0s = dma_wave_base(lds_addr(lds));
  constexpr uint32_t kTileB = 16u * kTileU4;
  // prologue: B0, A0 (slots 0, 1), then B1, A1 (slots 2, 3)
  lb.dma(0, m0s);
  if constexpr (kLoadA) la.dma(0, m0s + kTileB);
  const int k1 = min(1, nk - 1);
  lb.dma(k1, m0s + 2 * kTileB);
  if constexpr (kLoadA) la.dma(k1, m0s + 3 * kTileB);
  // B0 and A0 have landed (block 1's loads may still be in flight)
  if constexpr (kLoadA) wait_vm_two_tiles();
  else wait_vm(kDma);
  __builtin_amdgcn_s_barrier();
  const FragOffs fa = frag_offs<A_MN>(ra0, lane), fb = frag_offs<B_MN>(rb0, lane);
  Frags f, g;
  int sb = 0;  // slot of B of the current block (A is in slot sb + 1 mod 5)
  load_frags<A_MN, B_MN, kRB>(lds + kTileU4, lds, fa, fb, 0, f);
  for (int kt = 0; kt + 1 < nk; ++kt) {
    const int sa = sb == 4 ? 0 : sb + 1;
    const u32x4* tA = lds + sa * kTileU4;
    const u32x4* tB = lds + sb * kTileU4;
    // block kt+2: B into slot (sb + 4) mod 5 (freed by A of block kt-1), A into
    // slot sb (freed by B of block kt at this block's barrier)
    const int k2 = min(kt + 2, nk - 1);
    const int sb2 = sb == 0 ? 4 : sb - 1;
    kstep<A_MN, B_MN, kStepRead, true, 0, kRB, kLoadA>(f, g, acc, tA, tB, fa, fb, 1, la, lb, k2, 0u,
                                                         m0s + sb2 * kTileB);
    f = g;
    kstep<A_MN, B_MN, kStepRead, true, 1, kRB, kLoadA>(f, g, acc, tA, tB, fa, fb, 2, la, lb, k2, 0u,
                                                         m0s + sb2 * kTileB);
    f = g;
    kstep<A_MN, B_MN, kStepRead, false, 0, kRB, kLoadA>(f, g, acc, tA, tB, fa, fb, 3, la, lb, 0, 0u, 0u);
    f = g;
    const int sbn = sb >= 3 ? sb - 3 : sb + 2;  // slot of B of block kt+1
    const int san = sbn == 4 ? 0 : sbn + 1;
    kstep<A_MN, B_MN, kStepSwap, false, 0, kRB, kLoadA>(f, g, acc, lds + san * kTileU4, lds + sbn * kTileU4, fa, fb,
                                                        0, la, lb, k2, m0s + sb * kTileB, 0u);
    f = g;
    sb = sbn;
  }
  {
    tail();
    const int sa = sb == 4 ? 0 : sb + 1;
    const u32x4* tA = lds + sa * kTileU4;
    const u32x4* tB = lds + sb * kTileU4;
#pragma unroll
    for (int kk = 0; kk < kKK - 1; ++kk) {
      kstep<A_MN, B_MN, kStepRead, false, 0, kRB, kLoadA>(f, g, acc, tA, tB, fa, fb, kk + 1, la, lb, 0, 0u, 0u);
      f = g;
    }
    kstep<A_MN, B_MN, kStepLast, false, 0, kRB, kLoadA>(f, g, acc, tA, tB, fa, fb, 0, la, lb, 0, 0u, 0u);
  }
  // every load issued has landed and every wave is done with the ring
  wait_vm(0);
  __syncthreads();
}

__device__ __forceinline__ void acc_zero(Acc& acc) {
#pragma unroll
  for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) acc.c[mi][ni] = f32x16{};
}

// Tile-local row held by lane l in block mi of wave (wm, *).
__device__ __forceinline__ int acc_row(int wm, int mi, int lane) { return kWaveRows * wm + 32 * mi + (lane & 31); }

// Tile-local column of elements 4g .. 4g+3 (first of four) of block ni for
// lane l in wave (*, wn).
__device__ __forceinline__ int acc_col4(int wn, int ni, int g, int lane) {
  return 128 * wn + 32 * ni + 8 * g + 4 * (lane >> 5);
}

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2): block b runs on XCD b mod 8.  With `live` tiles to run (a count the
// device may only know at run time, such as the active-row tiles), XCD x
// takes the contiguous id range [x*per, (x+1)*per), per = ceil(live / 8):
// the tiles running together on one XCD share operand rows in its L2, and
// every XCD gets the same number of tiles.  Returns -1 for blocks beyond the
// live tiles (grids are sized for the largest possible count).
__device__ __forceinline__ int xcd_tile(int live, int bid) {
  const int per = (live + 7) >> 3;
  const int slot = bid >> 3;
  if (slot >= per) return -1;
  const int id = (bid & 7) * per + slot;
  return id < live ? id : -1;
}

// Tile id -> (fast index f < F, slow index c < C) in groups of GM fast
// indices: consecutive ids walk the GM values of f of a group, then the
// next c.  With GM near 8 the ~32 tiles an XCD runs together (its
// contiguous id range, see xcd_tile) form an 8 x 4 block whose 12 operand
// tiles per k-block are shared in its L2 (measured best among group sizes
// 4..16, on the LM-head and on square products).  row_group splits F into
// ceil(F / 8) groups of equal size (14 row tiles: two groups of 7, not 8 +
// 6), so that the XCD ranges do not straddle a short last group.
__device__ __forceinline__ int row_group(int F) {
  const int ng = (F + 7) >> 3;
  return (F + ng - 1) / ng;
}
__device__ __forceinline__ void grouped_tile(int id, int F, int& f, int& c, int C, int GM) {
  const int per_group = GM * C;
  const int grp = id / per_group;
  const int gm = min(GM, F - grp * GM);
  const int within = id - grp * per_group;
  c = within / gm;
  f = grp * GM + (within - c * gm);
}

RLK_ENGINE_END  // namespace rlk
