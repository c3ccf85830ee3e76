// The forward and dz tile kernels with eight waves per 256 x 256 tile (two
// per SIMD, 64 x 128 each).  On these products (both operands K-contiguous)
// the second wave per SIMD hides more of the k-loop's stalls than its
// extra fragment reads cost; grad_tiles, whose operands are read through
// the transposing LDS loads, is faster with four and stays in rlk_api.hip's
// four-wave build.  Every output element is the same MFMA chain in both
// flavours, so the results are the same bits.
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

}  // namespace rlk
