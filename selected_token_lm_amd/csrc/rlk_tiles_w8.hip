// The forward, dz and gradient tile kernels with eight waves per 256 x 256
// tile (two per SIMD, 64 x 128 each): the second wave per SIMD hides the
// stalls of the k-loop's instruction stream that one wave per SIMD leaves
// on the MFMA pipe.  rlk_api.hip's four-wave build keeps the save-logits
// and small-batch forwards (whose row-skipping layout is written for four
// waves) and the dense product.  Every output element is the same MFMA
// chain in both flavours, so the results are the same bits.
#ifdef RLK_WAVES
#undef RLK_WAVES
#endif
#define RLK_WAVES 8
#define RLK_ENGINE_W8
#include "rlk_kernels.h"
#include "rlk_tiles_w8.h"

namespace rlk {

static_assert(w8::kThreads == kThreadsW8, "block size of the eight-wave kernels");

void launch_fwd_tiles_w8(dim3 grid, hipStream_t st, const FwdArgs& a) {
  hipLaunchKernelGGL((w8::fwd_tiles<false, 0>), grid, dim3(w8::kThreads), 0, st, a);
}

void launch_dz_tiles_w8(dim3 grid, hipStream_t st, const DzArgs& a) {
  hipLaunchKernelGGL(w8::dz_tiles, grid, dim3(w8::kThreads), 0, st, a);
}

void launch_grad_tiles_w8(bool first, bool last, bool part, dim3 grid, hipStream_t st, const GradHArgs& ha,
                          const GradWArgs& wa) {
  void (*kfn)(GradHArgs, GradWArgs) =
      part ? (first ? (last ? w8::grad_tiles<true, true, true> : w8::grad_tiles<true, false, true>)
                    : (last ? w8::grad_tiles<false, true, true> : w8::grad_tiles<false, false, true>))
           : (first ? (last ? w8::grad_tiles<true, true, false> : w8::grad_tiles<true, false, false>)
                    : (last ? w8::grad_tiles<false, true, false> : w8::grad_tiles<false, false, false>));
  hipLaunchKernelGGL(kfn, grid, dim3(w8::kThreads), 0, st, ha, wa);
}

}  // namespace rlk
