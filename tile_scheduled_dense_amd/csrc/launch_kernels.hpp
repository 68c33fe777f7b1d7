// launch_kernels.hpp -- the GEMM kernels' instantiations and launches for a plan.
// Included by one translation unit per input type (launch_bf16.hip,
// launch_f16.hip, launch_f32.hip), which the build compiles in parallel.
#pragma once

#include <hip/hip_runtime.h>

#include "gemm_ring.hpp"
#include "launch.hpp"

namespace tg {
namespace {

template <class C, int DEPTH, int SWZ, bool TAIL = false>
tg_status launch_one(const GemmParams &gp, int64_t grid, hipStream_t stream) {
    if (grid > 0x7fffffffLL) return TG_ERR_UNSUPPORTED;
    hipLaunchKernelGGL((gemm_kernel<C, DEPTH, SWZ, TAIL>), dim3((unsigned)grid), dim3(C::THREADS), 0, stream, gp);
    return hipGetLastError() == hipSuccess ? TG_OK : TG_ERR_LAUNCH;
}

// tail: the fused-tail instantiation (built for the default depth and swizzle only)
template <class C>
tg_status launch_variants(const GemmParams &gp, const tg_plan_info &p, hipStream_t s, bool tail) {
    if (tail) {
        if (p.pipeline_depth == 2 && p.swizzle == SWZ_XOR) return launch_one<C, 2, SWZ_XOR, true>(gp, p.grid, s);
        return TG_ERR_UNSUPPORTED;
    }
    if (p.pipeline_depth == 2 && p.swizzle == SWZ_XOR) return launch_one<C, 2, SWZ_XOR>(gp, p.grid, s);
    if (p.pipeline_depth == 1 && p.swizzle == SWZ_XOR) return launch_one<C, 1, SWZ_XOR>(gp, p.grid, s);
    if (p.pipeline_depth == 2 && p.swizzle == SWZ_NONE) return launch_one<C, 2, SWZ_NONE>(gp, p.grid, s);
    if (p.pipeline_depth == 1 && p.swizzle == SWZ_NONE) return launch_one<C, 1, SWZ_NONE>(gp, p.grid, s);
    return TG_ERR_UNSUPPORTED;
}

template <class C, int STAGES, int SWZ, int SCHED, bool TAIL = false>
tg_status launch_ring_one(const GemmParams &gp, int64_t grid, hipStream_t stream) {
    if (grid > 0x7fffffffLL) return TG_ERR_UNSUPPORTED;
    hipLaunchKernelGGL((gemm_ring_kernel<C, STAGES, SWZ, SCHED, TAIL>), dim3((unsigned)grid), dim3(C::THREADS), 0,
                       stream, gp);
    return hipGetLastError() == hipSuccess ? TG_OK : TG_ERR_LAUNCH;
}

// SWPIPE: the 256 x 256 tile (one wave per SIMD, a whole K tile of fragments
// in registers) whenever it has two or more LDS copies; RING otherwise.
template <class C, bool SWPIPE>
tg_status launch_ring(const GemmParams &gp, const tg_plan_info &p, hipStream_t s, bool tail) {
    constexpr int SCHED = SWPIPE ? SCHED_SWPIPE : SCHED_RING;
    if (tail) {     // built at the default depth and swizzle (make_plan refuses the others)
        if (p.pipeline_depth == 4 && p.swizzle == SWZ_XOR)
            return launch_ring_one<C, 4, SWZ_XOR, SCHED, true>(gp, p.grid, s);
        return TG_ERR_UNSUPPORTED;
    }
    if (p.swizzle == SWZ_XOR) {
        switch (p.pipeline_depth) {
            case 5:
                if constexpr (!SWPIPE) return launch_ring_one<C, 5, SWZ_XOR, SCHED>(gp, p.grid, s);
                return TG_ERR_UNSUPPORTED;
            case 4: return launch_ring_one<C, 4, SWZ_XOR, SCHED>(gp, p.grid, s);
            case 2: return launch_ring_one<C, 2, SWZ_XOR, SCHED>(gp, p.grid, s);
            case 1:
                if constexpr (SWPIPE && C::DT == DT_F32) return TG_ERR_UNSUPPORTED;   // not built (make_plan)
                else return launch_ring_one<C, 1, SWZ_XOR, SCHED_RING>(gp, p.grid, s);
        }
    } else if (p.pipeline_depth == 4 && p.swizzle == SWZ_NONE) {
        return launch_ring_one<C, 4, SWZ_NONE, SCHED>(gp, p.grid, s);
    } else if (p.pipeline_depth == 4 && p.swizzle == SWZ_PAD) {
        if constexpr (SWPIPE && C::DT != DT_F32) return launch_ring_one<C, 4, SWZ_PAD, SCHED>(gp, p.grid, s);
    }
    return TG_ERR_UNSUPPORTED;
}

template <int DT>
tg_status launch_dtype(const GemmParams &gp, const tg_plan_info &p, hipStream_t s, bool tail) {
    if (p.persistent && p.config == TG_CFG_288x160) {     // two batch entries per workgroup
        if (p.pipeline_depth != 4 || p.swizzle != SWZ_XOR) return TG_ERR_INTERNAL;
        using C = Ring288x160<DT>;
        if (tail)
            hipLaunchKernelGGL((gemm_ring_chain_kernel<C, 4, SWZ_XOR, true>), dim3((unsigned)p.grid), dim3(C::THREADS),
                               0, s, gp);
        else
            hipLaunchKernelGGL((gemm_ring_chain_kernel<C, 4, SWZ_XOR>), dim3((unsigned)p.grid), dim3(C::THREADS), 0, s,
                               gp);
        return hipGetLastError() == hipSuccess ? TG_OK : TG_ERR_LAUNCH;
    }
    if (p.persistent) {
        if (p.config != TG_CFG_256x256 || p.pipeline_depth != 4 || p.swizzle != SWZ_XOR) return TG_ERR_INTERNAL;
        using C = Ring256<DT>;
        if (tail) return TG_ERR_INTERNAL;   // the plan never pairs the persistent grid with a tail
        hipLaunchKernelGGL((gemm_ring_persistent_kernel<C, 4, SWZ_XOR>), dim3((unsigned)p.grid), dim3(C::THREADS), 0,
                           s, gp);
        return hipGetLastError() == hipSuccess ? TG_OK : TG_ERR_LAUNCH;
    }
    switch (p.config) {
        case TG_CFG_256x256: return launch_ring<Ring256<DT>, true>(gp, p, s, tail);
        case TG_CFG_128x128: return launch_ring<Ring128<DT>, false>(gp, p, s, tail);
        case TG_CFG_64x64: return launch_ring<Ring64<DT>, false>(gp, p, s, tail);
        case TG_CFG_288x160: {
            // the plain ring (all waves in step, fragments read per K tile) at depth 2
            // or 4; the placement ablation at depth 4.  This tile serves batches of
            // small problems, bound by memory, where the software pipeline's second
            // fragment set only costs registers (118 against 122 us on 512 problems
            // of 257 x 129 x 1000, the same MFMA order and result).
            using C = Ring288x160<DT>;
            if (tail) {
                if (p.pipeline_depth == 4 && p.swizzle == SWZ_XOR)
                    return launch_ring_one<C, 4, SWZ_XOR, SCHED_RING, true>(gp, p.grid, s);
                return TG_ERR_UNSUPPORTED;
            }
            if (p.swizzle == SWZ_XOR && p.pipeline_depth == 4) return launch_ring_one<C, 4, SWZ_XOR, SCHED_RING>(gp, p.grid, s);
            if (p.swizzle == SWZ_XOR && p.pipeline_depth == 2) return launch_ring_one<C, 2, SWZ_XOR, SCHED_RING>(gp, p.grid, s);
            if (p.swizzle == SWZ_NONE && p.pipeline_depth == 4)
                return launch_ring_one<C, 4, SWZ_NONE, SCHED_RING>(gp, p.grid, s);
            return TG_ERR_UNSUPPORTED;
        }
        default: return TG_ERR_UNSUPPORTED;
    }
}

}  // namespace
}  // namespace tg
