// launch_f16.hip -- the fp16 GEMM kernels (launch.hpp).
#include "launch_kernels.hpp"

namespace tg {

tg_status launch_gemm_f16(const GemmParams &gp, const tg_plan_info &p, hipStream_t s, bool tail) {
    return launch_dtype<DT_F16>(gp, p, s, tail);
}

}  // namespace tg
