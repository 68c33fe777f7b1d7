// launch.hpp -- the GEMM kernels of each input type, launched for a plan on a
// stream.  Each is defined in a translation unit of its own (launch_bf16.hip,
// launch_f16.hip, launch_f32.hip) so the kernel instantiations compile in
// parallel; the C ABI (tile_gemm.hip) calls them after planning.
#pragma once

#include <hip/hip_runtime.h>

#include "gemm_kernel.hpp"
#include "tile_gemm.h"

namespace tg {

// tail: the fused-tail instantiation (the plan allows it at the default depth
// and swizzle only).  Returns TG_ERR_UNSUPPORTED for a combination not built.
tg_status launch_gemm_bf16(const GemmParams &gp, const tg_plan_info &p, hipStream_t s, bool tail);
tg_status launch_gemm_f16(const GemmParams &gp, const tg_plan_info &p, hipStream_t s, bool tail);
tg_status launch_gemm_f32(const GemmParams &gp, const tg_plan_info &p, hipStream_t s, bool tail);

}  // namespace tg
