// Launchers of the eight-wave tile kernels (rlk_tiles_w8.hip), called by the
// host side in rlk_api.hip; internal to the library (not exported).  They
// only enqueue the launch on `st`; the caller checks hipGetLastError.
#pragma once

#include <hip/hip_runtime.h>

#include "rlk_args.h"

namespace rlk {

constexpr int kThreadsW8 = 512;  // threads per block of the eight-wave kernels

// fwd_tiles<false, 0>: the forward's logit tiles (logits not saved, whole
// row tiles), eight waves per tile.
__attribute__((visibility("hidden"))) void launch_fwd_tiles_w8(dim3 grid, hipStream_t st, const FwdArgs& a);

// dz_tiles, eight waves per tile.
__attribute__((visibility("hidden"))) void launch_dz_tiles_w8(dim3 grid, hipStream_t st, const DzArgs& a);

// grad_tiles<first, last, part>: a backward group's grad_h and grad_W
// tiles, eight waves per tile.
__attribute__((visibility("hidden"))) void launch_grad_tiles_w8(bool first, bool last, bool part, dim3 grid,
                                                               hipStream_t st, const GradHArgs& ha,
                                                               const GradWArgs& wa);

}  // namespace rlk
