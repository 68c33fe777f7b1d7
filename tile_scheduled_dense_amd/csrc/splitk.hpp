// splitk.hpp -- second pass of the split-K reduction.
//
// The deterministic two-pass split reduction of the OCANNL "Module Ir.Schedule"
// page (paragraph of that name): the first pass (the GEMM kernel with
// GemmParams::splits > 1) writes one fp32 partial per K slice, each written
// whole, so nothing needs zeroing; this pass folds the S partials of every
// output element in a fixed balanced-tree order and applies the epilogue.
// The tree is the same for every element and every run, so the result is
// bitwise reproducible for a given S.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_kernel.hpp"

namespace tg {

// Partial s of element idx (idx = b * M * N + i * N + j over all problems) is
// W[s * total + idx].  P is the power of two >= S the tree is laid out for:
// level w adds v[i + w] into v[i] for i = 0, 2w, 4w, ... whenever slice i + w
// exists, so slices beyond S are never touched.
template <int P>
__global__ __launch_bounds__(256) void splitk_combine_kernel(const float *__restrict__ W, float *__restrict__ C,
                                                             int64_t M, int64_t N, int64_t ldc, int64_t sC,
                                                             int64_t problems, int S, float alpha, float beta,
                                                             const float *__restrict__ bias, int64_t bias_stride,
                                                             int bias_mode, int act) {
    const int64_t plane = M * N, total = problems * plane;
    const int64_t step = (int64_t)gridDim.x * blockDim.x;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += step) {
        float v[P];
#pragma unroll
        for (int s = 0; s < P; ++s) v[s] = s < S ? W[s * total + idx] : 0.0f;
#pragma unroll
        for (int w = 1; w < P; w *= 2)
#pragma unroll
            for (int i = 0; i + w < P; i += 2 * w)
                if (i + w < S) v[i] += v[i + w];
        const int64_t b = idx / plane, r = idx - b * plane;
        const int64_t i = r / N, j = r - i * N;
        float *c = C + b * sC + i * ldc + j;
        if (bias_mode != 0 || act != 0) {
            const float bv = bias_mode == 1 ? bias[b * bias_stride + j] : (bias_mode == 2 ? bias[b * bias_stride + i] : 0.0f);
            *c = tail_value(v[0], alpha, bv, act, beta, beta != 0.0f ? *c : 0.0f);
        } else {
            *c = beta != 0.0f ? __builtin_fmaf(alpha, v[0], beta * *c) : alpha * v[0];
        }
    }
}

}  // namespace tg
