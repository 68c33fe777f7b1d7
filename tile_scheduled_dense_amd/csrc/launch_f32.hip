// launch_f32.hip -- the fp32 GEMM kernels (launch.hpp): the ring tiles
// (TG_CFG_256x256, TG_CFG_128x128 with 16x16x4 MFMAs) and the register-staged
// 64 x 64 tile for small problems.
#include "launch_kernels.hpp"

namespace tg {

tg_status launch_gemm_f32(const GemmParams &gp, const tg_plan_info &p, hipStream_t s, bool tail) {
    if (p.config == TG_CFG_F32_64x64) return launch_variants<CfgF32>(gp, p, s, tail);
    if (p.persistent) return TG_ERR_INTERNAL;   // built for 16-bit inputs only (the plan never asks)
    if (p.config == TG_CFG_256x256) return launch_ring<RingF32_256, true>(gp, p, s, tail);
    if (p.config == TG_CFG_128x128) return launch_ring<RingF32_128, false>(gp, p, s, tail);
    return TG_ERR_UNSUPPORTED;
}

}  // namespace tg
