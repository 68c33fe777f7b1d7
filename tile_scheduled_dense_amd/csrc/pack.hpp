// pack.hpp -- repack of a 16-bit row-major operand into rows whose byte stride
// is a multiple of 16, zero-filled past the row's extent.
//
// A tile copy reads 64-byte row segments of A; when A's rows start at 2-byte
// offsets each segment straddles cache lines and costs the copy path half as
// much again.  For a plan that reads every A panel from many workgroups, one
// pass that writes A once with aligned rows is cheaper than that overhead.
// The packed rows hold the same values, so the GEMM that reads them computes
// the same MFMA sequence and a bitwise identical result.
#pragma once

#include "gemm_kernel.hpp"

namespace tg {

// One workgroup per row (of one batch entry): batch entry b = row / rows,
// source row src + (b * stride + r * ld) elements, destination row
// dst + (b * rows + r) * ld_out elements.  Each thread moves 16-byte chunks:
// an (unaligned) 16-byte load from the source, an aligned 16-byte store; the
// chunk holding the end of the row loads its valid elements one by one.
__global__ __launch_bounds__(256) void pack_rows_kernel(const char *__restrict__ src, int64_t ld, int64_t stride,
                                                        char *__restrict__ dst, int64_t ld_out, int64_t rows,
                                                        int64_t cols) {
    const int64_t row = blockIdx.x;
    const int64_t b = row / rows, r = row - b * rows;
    const char *s = src + (b * stride + r * ld) * 2;
    u32x4 *d = reinterpret_cast<u32x4 *>(dst + row * ld_out * 2);
    const rsrc_t rs = make_rsrc(s);
    const int64_t chunks = ld_out / 8;
    for (int64_t c = threadIdx.x; c < chunks; c += blockDim.x) {
        const int64_t left = cols - 8 * c;
        const int n = left <= 0 ? 0 : (left >= 8 ? 8 : (int)left);
        d[c] = bload16_n<2>(rs, (int)(16 * c), 0, n);
    }
}

}  // namespace tg
