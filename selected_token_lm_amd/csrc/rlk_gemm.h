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

#include <utility>

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
// MFMA shape (RLK_MFMA at build time): 32 = v_mfma_f32_32x32x16_bf16
// (32 x 32 blocks, 16 k per step; the default), 16 =
// v_mfma_f32_16x16x32_bf16 (16 x 16 blocks, 32 k per step).  The shape is
// part of the numerical contract: it fixes how many products each MFMA step
// sums before the fp32 accumulation.
#ifndef RLK_MFMA
#define RLK_MFMA 16
#endif
constexpr int kBlk = RLK_MFMA;
static_assert(kBlk == 16 || kBlk == 32, "16 x 16 x 32 or 32 x 32 x 16 MFMAs");
constexpr int kKStep = 512 / kBlk;          // k summed per MFMA step: 32 or 16
constexpr int kLPR = 64 / kBlk;             // lanes holding one row of a block: 4 or 2
constexpr int kQL = kBlk * kBlk / 256;      // groups of 4 consecutive columns per lane per block: 1 or 4
constexpr int kMI = kWaveRows / kBlk, kNI = 128 / kBlk;  // blocks per wave
constexpr int kMma = kMI * kNI;            // MFMAs per wave per k step
constexpr int kReads = kMI + kNI;          // fragment reads per wave per k step
constexpr int kKK = kBK / kKStep;          // MFMA k steps per k-block
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

// MN-mode position of the 16-byte piece p (of 32) within its k-row's 512
// bytes; an involution in p, so the direct loads use it to pick the piece
// each lane fetches.  A transposing read (ds_read_b64_tr_b16) serves 32
// lanes per pass, each k-row contributing 32 contiguous bytes (16 columns):
//   16 x 16 x 32: the pass reads k-rows 8g + 0..3 and 8g + 8 .. 8g + 11 at
//     the same columns, so 32-byte units are xor-ed with
//     (k-row & 3) + 4 ((k-row >> 3) & 1): eight distinct bank ranges;
//   32 x 32 x 16: the pass reads k-rows 0..3 at two neighbouring 32-byte
//     column ranges, so 64-byte blocks are xor-ed with (k-row & 7).
// Both are unchanged by the k-step's row offset (32 or 16 rows).
__device__ __forceinline__ int mn_pos(int krow, int p) {
  if constexpr (kBlk == 16) {
    const int f = (krow & 3) | ((krow >> 1) & 4);
    return (((p >> 1) ^ f) << 1) | (p & 1);
  } else {
    return (((p >> 2) ^ (krow & 7)) << 2) | (p & 3);
  }
}

// MN-mode slot of (k-row, 16-byte piece p of 32).
__device__ __forceinline__ int slot_mn(int krow, int p) { return krow * 32 + mn_pos(krow, p); }

// Position of wave w in the tile's wave grid: row group wave_m (kWaveRows
// rows each), column group wave_n (128 columns each).
static_assert(kWM == 2 || kWM == 4, "power-of-two wave grid");
__device__ __forceinline__ int wave_m(int w) { return w & (kWM - 1); }
__device__ __forceinline__ int wave_n(int w) { return w >> (kWM == 2 ? 1 : 2); }

// ---- operand fragments from LDS ----------------------------------------------
// MFMA operand layout (both shapes, X and Y alike): lane l holds row
// (l % kBlk) of the block and k = 8 (l / kBlk) .. +7 of the k step, so a
// step sums exactly its kKStep k values.
//
// Per-lane LDS byte offsets of one operand's fragments within its tile,
// computed once per tile so that every read in the main loop is a base
// register plus an immediate:
//   K mode : fragment J (rows r0 + kBlk J ..) of k step kk at
//            o[kk] + 128 kBlk J (kBlk rows further keep the row's swizzle);
//   MN mode: fragment J (columns r0 + kBlk J ..) of k step kk: reads at
//            o[J] + 512 kKStep kk and o2[J] + 512 kKStep kk (k-rows +16 keep
//            the swizzle, k-rows +4 do not, hence two offsets).
constexpr int kMaxFrags = kMI > kNI ? kMI : kNI;
// With 16 x 16 blocks the second read's k-rows (+4) keep the swizzle
// (mn_pos), so it sits 4 rows = 2048 bytes after the first and needs no
// offset of its own.
constexpr bool kMnSecondByImm = kBlk == 16;
struct FragOffs {
  uint32_t o[kMaxFrags > kKK ? kMaxFrags : kKK], o2[kMnSecondByImm ? 1 : kMaxFrags];
};

template <bool MN>
__device__ __forceinline__ FragOffs frag_offs(int r0, int lane) {
  FragOffs f;
  if constexpr (!MN) {
    const int row = r0 + lane % kBlk;
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk) f.o[kk] = 16u * (uint32_t)slot_k(row, (kKStep / 8) * kk + lane / kBlk);
  } else {
    // ds_read_b64_tr_b16 serves 16 lanes at a time: supplier lane 4j+q of a
    // group points at k-row j, columns 4q..4q+3, and lane i of the group
    // receives column i of those 4 k-rows.  Group g of the wave covers
    // columns 16 (g % (kBlk/16)) .. +15 of the block and k-rows 8 (g / (kBlk/16)) + 0..3
    // (first read) and + 4..7 (second read).
    const int g = lane >> 4, s = lane & 15;
    constexpr int kG = kBlk / 16;  // 16-lane groups across a block's columns: 2 or 1
    const int krow = 8 * (g >> (kG - 1)) + (s >> 2);
#pragma unroll
    for (int J = 0; J < kMaxFrags; ++J) {
      const int col = r0 + kBlk * J + 16 * (g & (kG - 1)) + 4 * (s & 3);
      const int p = col >> 3, half = (col >> 2) & 1;
      f.o[J] = 16u * (uint32_t)slot_mn(krow, p) + 8u * half;
      if constexpr (!kMnSecondByImm) f.o2[J] = 16u * (uint32_t)slot_mn(krow + 4, p) + 8u * half;
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
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base + f.o[kk] + 128u * kBlk * J));
  } else {
    const lds_bf16x4* p0 = (const lds_bf16x4*)(base + f.o[J] + 512u * kKStep * kk);
    const uint32_t o1 = kMnSecondByImm ? f.o[J] + 2048u : f.o2[kMnSecondByImm ? 0 : J];
    const lds_bf16x4* p1 = (const lds_bf16x4*)(base + o1 + 512u * kKStep * kk);
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
//   MN mode: k-row 2 (kDma w + i) + (l >> 5), piece mn_pos(k-row, l & 31)
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
__device__ __forceinline__ int dma_mn_piece(int krow) { return mn_pos(krow, threadIdx.x & 31); }
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
// One accumulator block: kBlk x kBlk fp32, kBlk * kBlk / 64 values per lane.
typedef float AccBlk __attribute__((ext_vector_type(kBlk * kBlk / 64)));

struct Acc {
  AccBlk c[kMI][kNI];
};

// Operand fragments in registers.  A block mi is used by the kNI MFMAs
// (mi, 0 .. kNI-1) of a step, back to back, so the next step's A block mi is
// read into the same registers right after the last of them.  Every B block
// is used until the step's last row.  With four waves B fragments are
// double-buffered by step parity (b[s & 1] for step s; a k-block has an
// even number of steps) and the next step's are read over a step's first
// half; with eight waves (fewer registers per wave) there is one B buffer
// and block ni is re-read right after its last MFMA of the step (row
// kMI - 1), kNI MFMAs before its next use, a lead the SIMD's other wave
// stretches.
constexpr bool kDoubleB = kWaves == 4;
struct Frags {
  bf16x8 a[kMI], b[kDoubleB ? 2 : 1][kNI];
};
static_assert(!kDoubleB || kKK % 2 == 0, "B fragment buffers alternate by step parity");

// The B buffer that step parity p uses.
__device__ __forceinline__ constexpr int bbuf(int p) { return kDoubleB ? p : 0; }

// Fragment J (J < kMI: A block J, else B block J - kMI) of k step kk into
// B buffer p.
template <bool A_MN, bool B_MN, int J, int p>
__device__ __forceinline__ void load_frag(const u32x4* tA, const u32x4* tB, const FragOffs& fa, const FragOffs& fb,
                                          int kk, Frags& f) {
  if constexpr (J < kMI) f.a[J] = frag_at<A_MN, J>(tA, fa, kk);
  else f.b[bbuf(p)][J - kMI] = frag_at<B_MN, J - kMI>(tB, fb, kk);
}

// Row blocks: a wave may compute only its first kRB row blocks (kRB < kMI
// when the tile's remaining rows are known to be padding); the fragments
// and MFMAs of the others are skipped.  Fragment J is needed iff this holds.
template <int kRB>
__device__ __forceinline__ constexpr bool frag_used(int J) { return J < kMI ? J < kRB : kRB > 0; }

template <bool A_MN, bool B_MN, int kRB, int J, int p>
__device__ __forceinline__ void load_frag_if(const u32x4* tA, const u32x4* tB, const FragOffs& fa, const FragOffs& fb,
                                             int kk, Frags& f) {
  if constexpr (frag_used<kRB>(J)) load_frag<A_MN, B_MN, J, p>(tA, tB, fa, fb, kk, f);
}

// All fragments of k step kk (B into buffer p): A0 and B0 first, so that
// with reads completing in order the step's first MFMA waits for two only.
template <bool A_MN, bool B_MN, int kRB, int p, int r = 0>
__device__ __forceinline__ void load_frags(const u32x4* tA, const u32x4* tB, const FragOffs& fa, const FragOffs& fb,
                                           int kk, Frags& f) {
  if constexpr (r < kReads) {
    constexpr int J = r == 0 ? 0 : (r <= kNI ? kMI + r - 1 : r - kNI);
    load_frag_if<A_MN, B_MN, kRB, J, p>(tA, tB, fa, fb, kk, f);
    load_frags<A_MN, B_MN, kRB, p, r + 1>(tA, tB, fa, fb, kk, f);
  }
}

// B blocks r0 <= ni < r1 of k step kk into buffer p.
template <bool A_MN, bool B_MN, int kRB, int p, int r0, int r1>
__device__ __forceinline__ void load_bs(const u32x4* tA, const u32x4* tB, const FragOffs& fa, const FragOffs& fb,
                                        int kk, Frags& f) {
  if constexpr (r0 < r1) {
    load_frag_if<A_MN, B_MN, kRB, kMI + r0, p>(tA, tB, fa, fb, kk, f);
    load_bs<A_MN, B_MN, kRB, p, r0 + 1, r1>(tA, tB, fa, fb, kk, f);
  }
}

// A blocks r0 <= mi < r1 of k step kk.
template <bool A_MN, bool B_MN, int kRB, int r0, int r1>
__device__ __forceinline__ void load_as(const u32x4* tA, const u32x4* tB, const FragOffs& fa, const FragOffs& fb,
                                        int kk, Frags& f) {
  if constexpr (r0 < r1) {
    load_frag_if<A_MN, B_MN, kRB, r0, 0>(tA, tB, fa, fb, kk, f);
    load_as<A_MN, B_MN, kRB, r0 + 1, r1>(tA, tB, fa, fb, kk, f);
  }
}

// MFMA J of a k step (B buffer p): block (mi, ni) = (J / kNI, J % kNI);
// skipped for row blocks mi >= kRB.  The B fragment goes in as the X
// operand and the A fragment as Y, so that lane l of block (mi, ni) holds
// tile row kBlk mi + l % kBlk and, in elements 4q .. 4q+3, the four
// consecutive columns kBlk ni + 4 kLPR q + 4 (l / kBlk) + 0..3.
template <int J, int p, int kRB = kMI>
__device__ __forceinline__ void mma1(const Frags& f, Acc& acc) {
  constexpr int mi = J / kNI, ni = J % kNI;
  if constexpr (mi < kRB) {
#if RLK_MFMA == 32
    acc.c[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[bbuf(p)][ni], f.a[mi], acc.c[mi][ni], 0, 0, 0);
#else
    acc.c[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.b[bbuf(p)][ni], f.a[mi], acc.c[mi][ni], 0, 0, 0);
#endif
  }
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

// The schedule of a k-block.  Its kKK k steps of kMma MFMAs each (MFMA J
// on row block J / kNI, column block J % kNI) prepare the next step: the B
// fragments go into the other buffer, spread over the step's first half,
// and each A fragment is re-read right after its last MFMA of the step.
// The first kStepsB steps also issue the direct loads of the B tile of
// block kt+2 (kDmaB), spread over the step.  The last step (kStepSwap) runs
// half its MFMAs, waits until block kt+1 has landed and this wave's reads
// are done, passes the block's one barrier, and then reads block kt+1's
// first-step fragments (the A fragments whose MFMAs are done first, spread
// with the B fragments over the second half) and issues the direct loads of
// the A tile of block kt+2.
constexpr int kStepsB = kKK > 2 ? kKK - 2 : 1;  // steps that carry the B-tile loads
constexpr int kLoadsB = kDma / kStepsB;         // B-tile loads per such step
constexpr int kHalf = kMma / 2;
constexpr int kEarlyA = kHalf / kNI;            // A blocks done before the swap step's barrier
static_assert(kDma % kStepsB == 0 && kMma % kLoadsB == 0, "B-tile loads spread evenly");
static_assert(kHalf % kDma == 0 && kHalf % kNI == 0, "swap-step loads spread evenly");
static_assert(kDoubleB || (kMI - 1) * kNI >= kHalf, "one B buffer: the last row runs after the swap step's barrier");

enum StepKind {
  kStepRead,   // next step's fragments (k step kk of tiles tA, tB); with kDmaB the B-tile loads
               // kLoadsB kB0 .. of block kb into wave slot base dB
  kStepSwap,   // last step of a k-block: the next block's first step from tA, tB (see above);
               // A-tile loads of block kb into dA
  kStepLast,   // MFMAs only
};

// First of m items spread evenly over a span of n MFMAs that is due at
// MFMA j of the span.
__device__ __forceinline__ constexpr int spread(int j, int n, int m) { return (j * m + n - 1) / n; }

// MFMA J of a k step (B buffer p) with what comes before and after it.  No
// LDS wait is written for the fragment reads: before each MFMA the compiler
// waits for exactly the reads it needs (LDS reads complete in order).  The
// swap step's barrier is a bare s_barrier: __syncthreads() would add a
// release fence that waits for all outstanding loads.
template <bool A_MN, bool B_MN, StepKind kKind, bool kDmaB, int kB0, int kRB, bool kLoadA, int p, int J, class LA,
          class LB>
__device__ __forceinline__ void kslot(Frags& f, Acc& acc, const u32x4* tA, const u32x4* tB, const FragOffs& fa,
                                      const FragOffs& fb, int kk, const LA& la, const LB& lb, int kb, uint32_t dA,
                                      uint32_t dB) {
  constexpr int mi = J / kNI, ni = J % kNI;
  if constexpr (kKind == kStepRead) {
    if constexpr (kDoubleB && J < kHalf)
      load_bs<A_MN, B_MN, kRB, p ^ 1, spread(J, kHalf, kNI), spread(J + 1, kHalf, kNI)>(tA, tB, fa, fb, kk, f);
    if constexpr (kDmaB && J % (kMma / kLoadsB) == 1 % (kMma / kLoadsB))
      lb.one(kLoadsB * kB0 + J / (kMma / kLoadsB), kb, dB);
  } else if constexpr (kKind == kStepSwap && J >= kHalf) {
    if constexpr (J == kHalf) {
      wait_vm(kDma);
      wait_lds();
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
    constexpr int j = J - kHalf;
    load_as<A_MN, B_MN, kRB, spread(j, kHalf, kEarlyA), spread(j + 1, kHalf, kEarlyA)>(tA, tB, fa, fb, 0, f);
    if constexpr (kDoubleB)
      load_bs<A_MN, B_MN, kRB, p ^ 1, spread(j, kHalf, kNI), spread(j + 1, kHalf, kNI)>(tA, tB, fa, fb, 0, f);
    if constexpr (kLoadA && j % (kHalf / kDma) == 0) la.one(j / (kHalf / kDma), kb, dA);
  }
  mma1<J, p, kRB>(f, acc);
  if constexpr (!kDoubleB && mi == kMI - 1) {
    // B block ni is done for this step (one B buffer): the next step's
    // (in the swap step, the next block's first step, after the barrier)
    if constexpr (kKind == kStepRead) load_bs<A_MN, B_MN, kRB, 0, ni, ni + 1>(tA, tB, fa, fb, kk, f);
    else if constexpr (kKind == kStepSwap) load_bs<A_MN, B_MN, kRB, 0, ni, ni + 1>(tA, tB, fa, fb, 0, f);
  }
  if constexpr (ni == kNI - 1) {
    // A block mi is done for this step
    if constexpr (kKind == kStepRead) load_as<A_MN, B_MN, kRB, mi, mi + 1>(tA, tB, fa, fb, kk, f);
    else if constexpr (kKind == kStepSwap && mi >= kEarlyA) load_as<A_MN, B_MN, kRB, mi, mi + 1>(tA, tB, fa, fb, 0, f);
  }
  __builtin_amdgcn_sched_barrier(0);
}

template <bool A_MN, bool B_MN, StepKind kKind, bool kDmaB, int kB0, int kRB, bool kLoadA, int p, class LA, class LB,
          int... Js>
__device__ __forceinline__ void kslots(std::integer_sequence<int, Js...>, Frags& f, Acc& acc, const u32x4* tA,
                                       const u32x4* tB, const FragOffs& fa, const FragOffs& fb, int kk, const LA& la,
                                       const LB& lb, int kb, uint32_t dA, uint32_t dB) {
  (kslot<A_MN, B_MN, kKind, kDmaB, kB0, kRB, kLoadA, p, Js>(f, acc, tA, tB, fa, fb, kk, la, lb, kb, dA, dB), ...);
}

// One k step with B buffer p: kMma MFMAs, plus (by kKind) the next step's
// fragments (k step kk of tA, tB) and direct loads.
template <bool A_MN, bool B_MN, StepKind kKind, int p, bool kDmaB = false, int kB0 = 0, int kRB = kMI,
          bool kLoadA = true, class LA, class LB>
__device__ __forceinline__ void kstep(Frags& f, Acc& acc, const u32x4* tA, const u32x4* tB, const FragOffs& fa,
                                      const FragOffs& fb, int kk, const LA& la, const LB& lb, int kb, uint32_t dA,
                                      uint32_t dB) {
  __builtin_amdgcn_sched_barrier(0);
  kslots<A_MN, B_MN, kKind, kDmaB, kB0, kRB, kLoadA, p>(std::make_integer_sequence<int, kMma>{}, f, acc, tA, tB, fa,
                                                        fb, kk, la, lb, kb, dA, dB);
}

// The read steps kS .. kKK-2 of a k-block (step s reads step s + 1's
// fragments; steps below kStepsB issue the B-tile loads of block kb when
// `loads`).
template <bool A_MN, bool B_MN, int kRB, bool kLoadA, int kS, class LA, class LB>
__device__ __forceinline__ void read_steps(Frags& f, Acc& acc, const u32x4* tA, const u32x4* tB, const FragOffs& fa,
                                           const FragOffs& fb, const LA& la, const LB& lb, int kb, uint32_t dB,
                                           bool loads) {
  if constexpr (kS < kKK - 1) {
    if (loads)
      kstep<A_MN, B_MN, kStepRead, kS & 1, (kS < kStepsB), kS, kRB, kLoadA>(f, acc, tA, tB, fa, fb, kS + 1, la, lb,
                                                                           kb, 0u, dB);
    else
      kstep<A_MN, B_MN, kStepRead, kS & 1, false, kS, kRB, kLoadA>(f, acc, tA, tB, fa, fb, kS + 1, la, lb, 0, 0u, 0u);
    read_steps<A_MN, B_MN, kRB, kLoadA, kS + 1>(f, acc, tA, tB, fa, fb, la, lb, kb, dB, loads);
  }
}

// nk k-blocks of kBK.  LA / LB: loaders with one(i, kt, m0w) / dma(kt, m0w)
// that issue this thread's direct global->LDS loads of k-block kt.  lds:
// kLdsU4 words = a ring of 5 operand-tile slots.  Tile q = 2 kt (B of block
// kt) or 2 kt + 1 (A of block kt) lives in slot q mod 5, so at any time the
// ring holds the two tiles being read, the next block's two and one more.
// B tiles are issued about 1.5 blocks and A tiles 1 block before use.
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
  static_assert(kSlots == 5, "schedule written for five tile slots");
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
  Frags f;
  int sb = 0;  // slot of B of the current block (A is in slot sb + 1 mod 5)
  load_frags<A_MN, B_MN, kRB, 0>(lds + kTileU4, lds, fa, fb, 0, f);
  for (int kt = 0; kt + 1 < nk; ++kt) {
    const int sa = sb == 4 ? 0 : sb + 1;
    const u32x4* tA = lds + sa * kTileU4;
    const u32x4* tB = lds + sb * kTileU4;
    // block kt+2: B into slot (sb + 4) mod 5 (freed by A of block kt-1), A into
    // slot sb (freed by B of block kt at this block's barrier)
    const int k2 = min(kt + 2, nk - 1);
    const int sb2 = sb == 0 ? 4 : sb - 1;
    read_steps<A_MN, B_MN, kRB, kLoadA, 0>(f, acc, tA, tB, fa, fb, la, lb, k2, m0s + sb2 * kTileB, true);
    const int sbn = sb >= 3 ? sb - 3 : sb + 2;  // slot of B of block kt+1
    const int san = sbn == 4 ? 0 : sbn + 1;
    kstep<A_MN, B_MN, kStepSwap, (kKK - 1) & 1, false, 0, kRB, kLoadA>(f, acc, lds + san * kTileU4,
                                                                     lds + sbn * kTileU4, fa, fb, 0, la, lb, k2,
                                                                     m0s + sb * kTileB, 0u);
    sb = sbn;
  }
  {
    tail();
    const int sa = sb == 4 ? 0 : sb + 1;
    const u32x4* tA = lds + sa * kTileU4;
    const u32x4* tB = lds + sb * kTileU4;
    read_steps<A_MN, B_MN, kRB, kLoadA, 0>(f, acc, tA, tB, fa, fb, la, lb, 0, 0u, false);
    kstep<A_MN, B_MN, kStepLast, (kKK - 1) & 1, false, 0, kRB, kLoadA>(f, acc, tA, tB, fa, fb, 0, la, lb, 0, 0u, 0u);
  }
  // every load issued has landed and every wave is done with the ring
  wait_vm(0);
  __syncthreads();
}

__device__ __forceinline__ void acc_zero(Acc& acc) {
#pragma unroll
  for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) acc.c[mi][ni] = AccBlk{};
}

// Tile-local row held by lane l in block mi of wave (wm, *).
__device__ __forceinline__ int acc_row(int wm, int mi, int lane) {
  return kWaveRows * wm + kBlk * mi + lane % kBlk;
}

// Which of the kLPR lanes holding a row lane l is (0 .. kLPR-1).
__device__ __forceinline__ int row_lane(int lane) { return lane / kBlk; }

// Tile-local column of elements 4q .. 4q+3 (first of four consecutive
// columns; q < kQL) of block ni for lane l in wave (*, wn).
__device__ __forceinline__ int acc_col4(int wn, int ni, int q, int lane) {
  return 128 * wn + kBlk * ni + 4 * kLPR * q + 4 * row_lane(lane);
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
