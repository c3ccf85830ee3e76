/*
 * rlk_bench.h -- measurement helpers exported by librlk.so beside the
 * operator's C ABI (include/rlk.h).  They compute nothing of the operator;
 * benchmarks use them to price the kernels against the part's limits and to
 * time each kernel launch.  The operator's entry points never depend on them,
 * and with timing off (the default) a launch only reads one atomic flag.
 */
#ifndef RLK_BENCH_H_
#define RLK_BENCH_H_

#include <stddef.h>
#include <stdint.h>

#include "rlk.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Benchmark only (computes nothing of the operator): runs `blocks`
 * workgroups of 8 waves (two per SIMD, as the eight-wave tile kernels), each
 * wave issuing, per iteration, the tile engine's MFMA instruction on a
 * 64 x 128 accumulator tile (64 v_mfma_f32_16x16x32_bf16 over 2 register
 * sets of operands; a contract-1 build: 32 v_mfma_f32_32x32x16_bf16 over 4
 * sets), operands of random bf16 data, and no memory traffic in the loop:
 * the MFMA throughput the part sustains under its power limit with
 * realistic operand toggling (2^20 FLOP per wave, 2^23 per workgroup, per
 * iteration either way).
 *   src  bf16 device buffer of 24 * 512 * 8 values (random; 16-byte aligned)
 *   out  fp32 [blocks * 512] out (sums of the accumulators, so nothing is
 *        optimised away) */
rlk_status rlk_bench_mfma_ceiling(const void* src, float* out, int32_t blocks, int32_t iters,
                                  void* stream);

/* Per-kernel timing for benchmarks; computes nothing.  After
 * rlk_profile_begin(), every kernel the library launches (on any stream) is
 * bracketed by two HIP events recorded on that stream.  rlk_profile_end()
 * waits for those events, turns timing off and writes up to max_entries
 * per-kernel totals to `out` (launch count and summed event time in ms);
 * *n_entries receives the number of distinct kernels seen.  Not meant to be
 * used from several threads at once. */
typedef struct {
  char name[40];
  int64_t launches;
  double total_ms;
} rlk_kernel_time_t;

rlk_status rlk_profile_begin(void);
rlk_status rlk_profile_end(rlk_kernel_time_t* out, int32_t max_entries, int32_t* n_entries);

#ifdef __cplusplus
}
#endif

#endif /* RLK_BENCH_H_ */
