// launch_bf16.hip -- the bf16 GEMM kernels (launch.hpp).
#include "launch_kernels.hpp"

namespace tg {

tg_status launch_gemm_bf16(const GemmParams &gp, const tg_plan_info &p, hipStream_t s, bool tail) {
    return launch_dtype<DT_BF16>(gp, p, s, tail);
}

}  // namespace tg
