// pack.hpp -- repack of a row-major operand into rows whose byte stride is a
// multiple of 16, zero-filled past the row's extent; and the transposing pack
// of B for operands kept as B's transpose.
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

// Rows of one batch entry are `rows` long: row index q (over all batch
// entries) is batch entry b = q / rows, source row src + (b * stride + r * ld)
// elements, destination row dst + q * ld_out elements, ESZ bytes per element.
// Each row is moved by a group of `group` threads, 64, 128 or 256: whole
// waves, so the row's buffer resource is uniform across a wave; 256 / group
// rows per workgroup, so short rows still fill it.  A thread moves 16-byte chunks: an (unaligned) 16-byte load from
// the source, an aligned 16-byte store; the chunk holding the end of the row
// loads its valid elements one by one, and chunks past it store zeros.
template <int ESZ>
__global__ __launch_bounds__(256) void pack_rows_kernel(const char *__restrict__ src, int64_t ld, int64_t stride,
                                                        char *__restrict__ dst, int64_t ld_out, int64_t rows,
                                                        int64_t cols, int64_t total_rows, int group) {
    constexpr int PER = 16 / ESZ;     // elements per chunk
    const int per_block = 256 / group;
    const int64_t q = (int64_t)blockIdx.x * per_block + threadIdx.x / group;
    if (q >= total_rows) return;
    const int64_t b = q / rows, r = q - b * rows;
    const char *s = src + (b * stride + r * ld) * ESZ;
    u32x4 *d = reinterpret_cast<u32x4 *>(dst + q * ld_out * ESZ);
    const rsrc_t rs = make_rsrc(s);        // one row per wave: a uniform base
    const int64_t chunks = ld_out / PER;
    for (int64_t c = threadIdx.x % group; c < chunks; c += group) {
        const int64_t left = cols - PER * c;
        const int n = left <= 0 ? 0 : (left >= PER ? PER : (int)left);
        d[c] = bload16_n<ESZ>(rs, (int)(16 * c), 0, n);
    }
}

// Transposing pack of B: the source holds B's transpose, N rows of K elements
// (element (k, n) at src[b * stride + n * ld + k]); the destination holds B,
// K rows of ld_out elements (element (k, n) at dst[(b * K + k) * ld_out + n]),
// zero past N.  A workgroup moves a 64 x 64 block through LDS so that both
// the reads (64 consecutive k of one source row per wave) and the writes (64
// consecutive n of one destination row) are contiguous; the LDS rows are 65
// elements long so the transposed accesses fall in different banks.
// grid = (ceil(K / 64), ceil(ld_out / 64), batch).
template <class T>
__global__ __launch_bounds__(256) void pack_transposed_kernel(const T *__restrict__ src, int64_t ld, int64_t stride,
                                                              T *__restrict__ dst, int64_t ld_out, int64_t K,
                                                              int64_t N) {
    __shared__ T tile[64][65];
    const int64_t k0 = (int64_t)blockIdx.x * 64, n0 = (int64_t)blockIdx.y * 64, b = blockIdx.z;
    const T *s = src + b * stride;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int idx = tid + 256 * i;
        const int rn = idx >> 6, ck = idx & 63;        // source row n0 + rn, column k0 + ck
        const int64_t n = n0 + rn, k = k0 + ck;
        tile[ck][rn] = (n < N && k < K) ? s[n * ld + k] : T(0);
    }
    __syncthreads();
    T *d = dst + b * K * ld_out;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int idx = tid + 256 * i;
        const int rk = idx >> 6, cn = idx & 63;        // destination row k0 + rk, column n0 + cn
        const int64_t k = k0 + rk, n = n0 + cn;
        if (k < K && n < ld_out) d[k * ld_out + n] = tile[rk][cn];
    }
}

}  // namespace tg
