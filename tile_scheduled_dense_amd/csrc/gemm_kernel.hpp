// gemm_kernel.hpp -- the gfx950 kernel family for C = alpha * A.B + beta * C.
//
// One workgroup computes one BM x BN tile of C (a Split of the M and N loops,
// OCANNL "Module Ir.Schedule", Split; the workgroups are LuisaCompute's
// independent `parallel` children, "Execution Nests and coordinates",
// structured-region calculus, so they write disjoint tiles with no atomics).
//
// Per workgroup:
//  1. block order: the hardware hands consecutive workgroup ids to the eight
//     XCDs in turn; the id is remapped so each XCD receives a contiguous run of
//     tiles, walked in groups of GROUP_M tile rows, so tiles that share A and B
//     panels are resident on one XCD's L2 at the same time: a remapping of the
//     parallel children's coordinates, which the ParallelMap of the LuisaCompute
//     "Execution Nests and coordinates" page permits (Ordering strength and
//     sibling scopes).
//  2. pad-to-tile + partition (OCANNL Pad and Partition paragraphs): the
//     extents are padded to the tile; a block whose tile lies inside M x N runs
//     the guard-free instantiation, a block crossing M or N runs the one whose
//     copies guard rows/columns.  The K loop is partitioned at the last whole
//     tile: every tile but a ragged last one uses unguarded loads; the tail tile
//     zero-fills k >= K in both operands (a NaN in A's lda padding times a zero
//     of B would otherwise poison C).  Row/column masks of the output sit only
//     on the accumulator store-back.
//  3. staging (OCANNL Stage paragraph, shared + cooperative): each element of
//     the A and B tiles is copied by exactly one thread with 16-byte global
//     loads; the A and B copies form one phase with no barrier between them.
//     B is transposed in registers on its way to LDS so both operands are held
//     k-contiguous.  Placement: the XOR swizzle in tile_config.hpp.
//  4. window-2 pipeline (OCANNL pipeline_depth = 2; LuisaCompute "Pipelines and
//     stage boundaries", window = 2): a prologue copies tile 0 into LDS copy 0;
//     iteration k issues the global loads of tile k+1, multiplies tile k from
//     copy k mod 2, then writes tile k+1 into copy (k+1) mod 2, and closes with
//     one barrier -- N + 1 barriers for N tiles.  The barrier is the release of
//     the copy read in iteration k before iteration k+1 overwrites it (issue,
//     completion and release are distinct events: a slot is reused only after
//     every reader is done).  Depth 1 (2 barriers per tile) is kept as an option
//     and reads the same values in the same order, so it is bitwise identical.
//  5. tensorized multiply-accumulate (OCANNL Tensorize; Privatize): MFMA
//     32x32x16 for bf16/fp16, 16x16x4 for fp32, over the wave's TM x TN
//     register tiles, accumulators privatised in registers from +0.
//  6. fused epilogue (OCANNL epilogue fusion): C = fma(alpha, acc, beta * C0)
//     (alpha * acc when beta == 0, C0 not read), one store per element.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "tile_config.hpp"

namespace tg {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct GemmParams {
    const char *A;
    const char *B;
    float *C;
    int64_t M, N, K;
    int64_t lda, ldb, ldc;
    int64_t sA, sB, sC;          // batch strides, elements
    int64_t tiles_m, tiles_n, batch;
    float alpha, beta;
    int block_order;             // 0: XCD-grouped, 1: plain
    int group_m;                 // tile rows per group in the grouped order
    // split-K: `batch` above counts (slice, problem) pairs, problem fastest;
    // slice s of problem b multiplies k in [s * k_slice, min(K, (s+1) * k_slice))
    // into the fp32 partial W + (s * problems + b) * M * N (row stride N).
    int splits;                  // 1: no split
    int64_t problems;            // batch of the call
    int64_t k_slice;
    float *W;
    // Thin fringe strips (16-bit 256 x 256 configuration): the first
    // tiles_m * tiles_n * batch workgroups run the main tiles, the rest, per
    // batch entry, strip_n blocks of 256 x 64 (tile rows 0.., columns from
    // n_main) and then strip_m blocks of 64 x 256 (rows from m_main, tile
    // columns 0..).  tiles_m / tiles_n then count the main tiles only.
    int64_t strip_n, strip_m;
    int64_t n_main, m_main;
    // Strip blocks split along K (strip_splits > 1): the grid holds
    // strip_splits copies of the strip blocks, slice s multiplying k in
    // [s * strip_k_slice, ...) into an unscaled fp32 partial in Ws: first the N
    // strips' region (strip_rows_n x (N - n_main) per slice and problem), then
    // the M strips' ((M - m_main) x N).
    int strip_splits;
    int64_t strip_k_slice, strip_rows_n;
    float *Ws;
    // Fused elementwise tail (bias_mode or act nonzero): out = act(alpha * acc
    // + bias) + beta * C0, the bias one value per column (bias_mode 1) or per
    // row (2) of each problem, problem b's vector at bias + b * bias_stride.
    const float *bias;
    int64_t bias_stride;
    int bias_mode, act;
};

// GELU in its exact form x * Phi(x), Phi the standard normal CDF, branch-free:
// with z = |x| / sqrt 2, h = erfc(z) / 2 = Phi(-|x|) and Phi(x) = x >= 0 ? 1 - h : h.
// erfc(z) for z >= 0 is t * exp(P(t) - z^2), t = 1 / (1 + z / 2), P the degree-9
// Chebyshev fit whose fractional error stays below 1.2e-7 (Press, Teukolsky,
// Vetterling and Flannery, Numerical Recipes, 2nd ed., section 6.2): one
// reciprocal, nine fma and one exp2, against a library erff that branches on
// |z| < 1 and runs both sides when the lanes of a wave differ.  The error is
// relative, so the negative tail keeps its accuracy, where x / 2 * (1 + erf)
// cancels; in fp32 the result is within 2.4e-7 |x| of x * Phi(x).
__device__ __forceinline__ float gelu(float x) {
    const float z = __builtin_fabsf(x) * 0.70710678118654752f;
    const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.5f, z, 1.0f));
    float q = 0.17087277f;
    q = __builtin_fmaf(q, t, -0.82215223f);
    q = __builtin_fmaf(q, t, 1.48851587f);
    q = __builtin_fmaf(q, t, -1.13520398f);
    q = __builtin_fmaf(q, t, 0.27886807f);
    q = __builtin_fmaf(q, t, -0.18628806f);
    q = __builtin_fmaf(q, t, 0.09678418f);
    q = __builtin_fmaf(q, t, 0.37409196f);
    q = __builtin_fmaf(q, t, 1.00002368f);
    q = __builtin_fmaf(q, t, -1.26551223f);
    const float h = 0.5f * t * __builtin_amdgcn_exp2f((q - z * z) * 1.4426950408889634f);
    return x * (x >= 0.0f ? 1.0f - h : h);
}

// The tail's activation: 1 = ReLU (x < 0 ? 0 : x, so a NaN stays NaN), 2 = GELU.
__device__ __forceinline__ float tail_activation(float x, int act) {
    if (act == 1) return x < 0.0f ? 0.0f : x;
    if (act == 2) return gelu(x);
    return x;
}

// One output of the fused tail: fma(alpha, acc, bias) rounded once, the
// activation, then beta * C0 added by one more fma (C0 not read when beta is 0).
__device__ __forceinline__ float tail_value(float acc, float alpha, float bias_v, int act, float beta, float c0) {
    const float y = tail_activation(__builtin_fmaf(alpha, acc, bias_v), act);
    return beta != 0.0f ? __builtin_fmaf(beta, c0, y) : y;
}

template <class C>
struct AccT {
    typedef typename std::conditional<C::MT == 32, f32x16, f32x4>::type type;
};

// ---- block order -----------------------------------------------------------
// Tile of workgroup id w (blockIdx.x, or a persistent workgroup's w-th
// virtual id).
__device__ __forceinline__ void block_coords_of(const GemmParams &p, uint32_t w, int64_t &b, int64_t &tm,
                                                int64_t &tn) {
    // The grid is below 2^31 workgroups (checked on the host): 32-bit math.
    const uint32_t tiles_m = (uint32_t)p.tiles_m, tiles_n = (uint32_t)p.tiles_n;
    const uint32_t per_batch = tiles_m * tiles_n;
    const uint32_t total = per_batch * (uint32_t)p.batch;
    uint32_t lid = w;
    if (p.block_order == 0) {
        // Undo the round-robin over 8 XCDs: XCD x = w % 8 gets the x-th
        // contiguous run of logical tiles.
        const uint32_t per = total / 8, rem = total % 8;
        const uint32_t x = w % 8, j = w / 8;
        lid = x * per + (x < rem ? x : rem) + j;
    }
    b = lid / per_batch;
    const uint32_t t = lid % per_batch;
    if (p.block_order == 0) {
        const uint32_t gm = (uint32_t)p.group_m;
        const uint32_t group = t / (gm * tiles_n);
        const uint32_t first_m = group * gm;
        const uint32_t rows = (tiles_m - first_m) < gm ? (tiles_m - first_m) : gm;
        const uint32_t in_g = t % (gm * tiles_n);
        tn = in_g / rows;
        // The row order turns by one for every 32 tiles of the group (an XCD's
        // round), so the blocks of a slower row (a fringe row past M) do not fall
        // to the same CUs round after round: 8191 x 8193 x 8190 926-928 us
        // against 910-914 turned, 8191 x 8192 x 8192 826-827 against 812-816.
        // The turn is the same for all the rows of one column: still a bijection.
        tm = first_m + (in_g % rows + tn * rows / 32) % rows;
    } else {
        tm = t / tiles_n;
        tn = t % tiles_n;
    }
}

__device__ __forceinline__ void block_coords(const GemmParams &p, int64_t &b, int64_t &tm, int64_t &tn) {
    block_coords_of(p, blockIdx.x, b, tm, tn);
}

// ---- 16-byte chunk loads -----------------------------------------------------
// Tile copies go through buffer loads: a 128-bit resource (base pointer, size
// limit) in scalar registers plus one 32-bit byte offset per lane, so a thread
// needs a single address register however many chunks it copies.  Rows need
// not be 16-byte aligned (odd lda, packed batches): gfx950 serves an unaligned
// 128-bit load as one instruction.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const char *base) {
    // The base is the same for the whole workgroup; say so, so the resource
    // lives in scalar registers.
    const uint64_t a = (uint64_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const char *u = (const char *)(((uint64_t)hi << 32) | lo);
    // stride 0 (raw buffer), offsets up to 2^31 - 1 bytes, gfx9 data format word
    return __builtin_amdgcn_make_buffer_rsrc((void *)u, (short)0, 0x7fffffff, 0x00020000);
}

// Resource over [base, base + nbytes): offsets past nbytes read as 0, and a
// store there is dropped.
__device__ __forceinline__ rsrc_t make_rsrc_n(const char *base, int64_t nbytes) {
    const uint64_t a = (uint64_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const char *u = (const char *)(((uint64_t)hi << 32) | lo);
    const int n = nbytes > 0x7fffffffLL ? 0x7fffffff : (int)nbytes;
    return __builtin_amdgcn_make_buffer_rsrc((void *)u, (short)0, __builtin_amdgcn_readfirstlane(n), 0x00020000);
}

constexpr int kOutOfRange = (int)0x80000000u;   // >= every resource size: reads as 0, stores dropped

__device__ __forceinline__ u32x4 bload16(rsrc_t r, int voff, int soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// A chunk of which only the first n elements exist (0 <= n <= CHUNK); the
// rest is +0 -- the zero fill of a staged tile's fringe.
template <int ELEM>
__device__ __forceinline__ u32x4 bload16_n(rsrc_t r, int voff, int soff, int n) {
    constexpr int CHUNK = 16 / ELEM;
    if (n >= CHUNK) return bload16(r, voff, soff);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (ELEM == 4) {
#pragma unroll
        for (int e = 0; e < 3; ++e)
            if (e < n) v[e] = __builtin_amdgcn_raw_buffer_load_b32(r, voff + 4 * e, soff, 0);
    } else {
#pragma unroll
        for (int e = 0; e < 7; ++e) {
            if (e < n) {
                const uint32_t h = __builtin_amdgcn_raw_buffer_load_b16(r, voff + 2 * e, soff, 0);
                v[e >> 1] |= (e & 1) ? (h << 16) : h;
            }
        }
    }
    return v;
}

// Transpose a CHUNK x CHUNK square held as CHUNK rows of 16 bytes: on return
// out[c] holds column c, i.e. the CHUNK k-values of one n.
template <int ELEM>
__device__ __forceinline__ void transpose_square(const u32x4 *in, u32x4 *out) {
    if (ELEM == 4) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
            out[c] = u32x4{in[0][c], in[1][c], in[2][c], in[3][c]};
    } else {
        // in[r][w] packs elements (r, 2w) (low half) and (r, 2w+1) (high half).
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            u32x4 ev, od;
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const uint32_t lo = in[2 * h][w], hi = in[2 * h + 1][w];
                ev[h] = (lo & 0xffffu) | (hi << 16);            // column 2w, k = 2h, 2h+1
                od[h] = (lo >> 16) | (hi & 0xffff0000u);        // column 2w+1
            }
            out[2 * w] = ev;
            out[2 * w + 1] = od;
        }
    }
}

// ---- MFMA ---------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ void mfma_chunk(const u32x4 &a, const u32x4 &b, f32x16 &acc) {
    if constexpr (DT == DT_BF16) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
    } else {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
    }
}

template <int DT>
__device__ __forceinline__ void mfma_chunk(const u32x4 &a, const u32x4 &b, f32x4 &acc) {
    if constexpr (DT == DT_BF16) {
        // one 16x16x32 MFMA: the chunks hold 8 consecutive k of one row / column
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
        return;
    } else if constexpr (DT == DT_F16) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
        return;
    }
    // fp32: four 16x16x4 MFMAs; element e of both chunks is the same k.
#pragma unroll
    for (int e = 0; e < 4; ++e)
    {
        // copy the element out first: a bit_cast of a vector-element lvalue
        // would read element 0
        const uint32_t ae = a[e], be = b[e];
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__builtin_bit_cast(float, ae), __builtin_bit_cast(float, be),
                                                   acc, 0, 0, 0);
    }
}

// ---- fused alpha/beta store-back -----------------------------------------------
// C = fma(alpha, acc, beta * C0), or alpha * acc when beta == 0 (C0 not read);
// masks (fringe blocks only) sit here, on the accumulator transfer.
// C0 and C are the same array, so the compiler may not move a C0 load above
// an earlier store; the MFMA tiles are therefore taken in chunks of 64 values
// per lane whose C0 loads are all issued before any of the chunk's stores:
// one memory round trip per chunk instead of one per MFMA tile.
// `acc(i, j, v)` is value v of MFMA tile (i, j) of this lane.
template <int I, int END, int STEP, class F>
__device__ __forceinline__ void static_for(const F &f) {
    if constexpr (I < END) {
        f(std::integral_constant<int, I>{});
        static_for<I + STEP, END, STEP>(f);
    }
}

// Store-back of a fringe block, through a buffer resource over the block's
// part of C (from its first element to one past its last valid one).  A
// value's byte offset is a row base (per MFMA row tile and value index: its
// row, and the lane's column in column tile 0) plus its column tile's step
// (MT columns a tile), so a chunk holds one base per row, not one offset per
// value.  A row outside C gets the base kFar, past every resource size, so its C0 load reads
// 0 and its store is dropped: no store sits under a lane mask for rows (a
// masked store is a branch of its own per value -- mask, exec save, store,
// exec restore -- which made the store-back of the batched 257 x 129 problems
// 3.9 times as long as unmasked stores of the whole tile).  A column outside C
// in a row inside C still addresses C (the next row's elements), so a block
// that cuts N masks its stores per column tile: one branch per MFMA column
// tile and chunk, not per value; its loads there read elements of C it does
// not use.  The host keeps every byte offset of a block's tile of C below
// 2^31 - 4097, so kFar plus a lane's column and the step stays below 2^32.
struct FringeC {
    static constexpr uint32_t kFar = 0x7ffff000u;
    rsrc_t r;
    __device__ __forceinline__ FringeC(float *Cblk, int64_t rows_left, int64_t cols_left, int64_t ldc)
        : r(make_rsrc_n((const char *)Cblk, ((rows_left - 1) * ldc + cols_left) * 4)) {}
    __device__ __forceinline__ static uint32_t base(int row, int col0, int ldc, int64_t rows_left) {
        return (row < rows_left ? (uint32_t)(row * ldc) * 4u : kFar) + (uint32_t)col0 * 4u;
    }
    __device__ __forceinline__ float load(uint32_t voff) const {
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, 0, 0));
    }
    __device__ __forceinline__ void put(uint32_t voff, float v) const {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, (int)voff, 0, 0);
    }
};

// The fused tail C = act(fma(alpha, acc, bias)) + beta * C0 (C0 not read when
// beta == 0), one instantiation per activation and per beta == 0 / != 0, so the
// per-value code is straight-line.  A lane's output column depends on its MFMA
// tile column j alone and its row on the tile row i and value index v alone
// (acc_coord), so the bias values it needs, TN of them per column or TM x V per
// row, are loaded once before any store.  No load is masked per lane: a masked
// load sits in a branch whose join waits for every memory operation in flight,
// stores included; bias indices are clamped into the vector instead, and a lane
// outside C reads C0 at the tile's origin (always inside C) and discards it.
// The chunk index is a template constant: with the activation inlined per value
// the epilogue is longer than the loop unroller accepts, and a rolled chunk
// loop would index the accumulators at run time, which moves them to scratch.
template <class C, bool FRINGE, class AccFn, int CHUNK_VALUES, int ACT, bool BETA>
__device__ __forceinline__ void store_tile_tail_as(const GemmParams &p, const AccFn &acc, int64_t b,
                                                   int64_t m0, int64_t n0, int wave, int lane) {
    float *Cblk = p.C + b * p.sC + m0 * p.ldc + n0;
    const int ldc = (int)p.ldc;
    const float alpha = p.alpha, beta = p.beta;
    const int64_t M = p.M, N = p.N;
    const float *bias = p.bias + b * p.bias_stride;
    const int bias_mode = p.bias_mode;
    const FringeC fc(Cblk, M - m0, N - n0, p.ldc);   // used by fringe blocks only
    constexpr int V = C::ACC_PER_MFMA;
    constexpr int TN = C::TN;
    constexpr int TILES = C::TM * C::TN;
    constexpr int CH = CHUNK_VALUES / V < TILES ? CHUNK_VALUES / V : TILES;   // MFMA tiles per chunk
    static_assert(TILES % CH == 0, "whole chunks");
    float bcol[TN], brow[C::TM][V];
#pragma unroll
    for (int j = 0; j < TN; ++j) bcol[j] = 0.0f;
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int v = 0; v < V; ++v) brow[i][v] = 0.0f;
    if (bias_mode == 1) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            int row, col;
            acc_coord<C>(wave, lane, j * V, row, col);
            const int64_t n = n0 + col;
            bcol[j] = bias[FRINGE && n >= N ? N - 1 : n];
        }
    } else if (bias_mode == 2) {
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
            for (int v = 0; v < V; ++v) {
                int row, col;
                acc_coord<C>(wave, lane, i * TN * V + v, row, col);
                const int64_t m = m0 + row;
                brow[i][v] = bias[FRINGE && m >= M ? M - 1 : m];
            }
    }
    // fringe blocks: this lane's column in column tile 0, and whether the block cuts N
    int col0 = 0;
    {
        int row;
        acc_coord<C>(wave, lane, 0, row, col0);
    }
    const bool cols_whole = n0 + C::BN <= N;
    static_for<0, TILES, CH>([&](auto chunk) {
        constexpr int c0t = decltype(chunk)::value;
        int off[CH][V];         // element offsets (interior) or byte offsets (fringe)
        uint32_t rb[CH][V];     // fringe: row bases
        float cv[CH][V];
#pragma unroll
        for (int t = 0; t < CH; ++t)
#pragma unroll
            for (int v = 0; v < V; ++v) {
                int row, col;
                acc_coord<C>(wave, lane, (c0t + t) * V + v, row, col);
                if constexpr (FRINGE) {
                    const int j = (c0t + t) % TN;
                    rb[t][v] = FringeC::base(row, col0, ldc, M - m0);
                    off[t][v] = (int)(rb[t][v] + (uint32_t)(j * C::MT * 4));
                    if constexpr (BETA) cv[t][v] = fc.load((uint32_t)off[t][v]);
                } else {
                    off[t][v] = row * ldc + col;
                    if constexpr (BETA) cv[t][v] = Cblk[off[t][v]];
                }
            }
        // the stores form their offsets anew from the row bases (as in
        // store_tile_epilogue: an opaque column step)
        uint32_t step = C::MT * 4;
        if constexpr (FRINGE && BETA) asm volatile("" : "+v"(step));
#pragma unroll
        for (int t = 0; t < CH; ++t) {
            const int i = (c0t + t) / TN, j = (c0t + t) % TN;
            const bool col_ok = !FRINGE || cols_whole || col0 + j * C::MT < N - n0;
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const float bv = bias_mode == 1 ? bcol[j] : brow[i][v];
                float y = tail_activation(__builtin_fmaf(alpha, acc(i, j, v), bv), ACT);
                if constexpr (BETA) y = __builtin_fmaf(beta, cv[t][v], y);
                if constexpr (FRINGE) {
                    if (col_ok) fc.put(rb[t][v] + j * step, y);
                } else {
                    Cblk[off[t][v]] = y;
                }
            }
        }
    });
}

template <class C, bool FRINGE, class AccFn, int CHUNK_VALUES>
__device__ __forceinline__ void store_tile_tail(const GemmParams &p, const AccFn &acc, int64_t b,
                                                int64_t m0, int64_t n0, int wave, int lane) {
#define TG_TAIL_AS(A, BT) store_tile_tail_as<C, FRINGE, AccFn, CHUNK_VALUES, A, BT>(p, acc, b, m0, n0, wave, lane)
    if (p.beta != 0.0f) {
        if (p.act == 2) TG_TAIL_AS(2, true);
        else if (p.act == 1) TG_TAIL_AS(1, true);
        else TG_TAIL_AS(0, true);
    } else {
        if (p.act == 2) TG_TAIL_AS(2, false);
        else if (p.act == 1) TG_TAIL_AS(1, false);
        else TG_TAIL_AS(0, false);
    }
#undef TG_TAIL_AS
}

template <class C, bool FRINGE, class AccFn, int CHUNK_VALUES = 64, bool TAIL = false>
__device__ __forceinline__ void store_tile_epilogue(const GemmParams &p, const AccFn &acc, int64_t b,
                                                    int64_t m0, int64_t n0, int wave, int lane) {
    if constexpr (TAIL) {
        store_tile_tail<C, FRINGE, AccFn, CHUNK_VALUES>(p, acc, b, m0, n0, wave, lane);
        return;
    }
    float *Cblk = p.C + b * p.sC + m0 * p.ldc + n0;
    const int ldc = (int)p.ldc;
    const float alpha = p.alpha, beta = p.beta;
    const int64_t M = p.M, N = p.N;
    const FringeC fc(Cblk, M - m0, N - n0, p.ldc);   // used by fringe blocks only
    constexpr int V = C::ACC_PER_MFMA;
    constexpr int TILES = C::TM * C::TN;
    constexpr int CH = CHUNK_VALUES / V < TILES ? CHUNK_VALUES / V : TILES;   // MFMA tiles per chunk
    static_assert(TILES % CH == 0, "whole chunks");
    // fringe blocks: this lane's column in column tile 0, and whether the block cuts N
    int col0 = 0;
    {
        int row;
        acc_coord<C>(wave, lane, 0, row, col0);
    }
    const bool cols_whole = n0 + C::BN <= N;
#pragma unroll
    for (int c0t = 0; c0t < TILES; c0t += CH) {
        int off[CH][V];         // element offsets (interior) or byte offsets (fringe)
        uint32_t rb[CH][V];     // fringe: row bases
#pragma unroll
        for (int t = 0; t < CH; ++t)
#pragma unroll
            for (int v = 0; v < V; ++v) {
                int row, col;
                acc_coord<C>(wave, lane, (c0t + t) * V + v, row, col);
                const int j = (c0t + t) % C::TN;
                rb[t][v] = FringeC::base(row, col0, ldc, M - m0);
                off[t][v] = FRINGE ? (int)(rb[t][v] + (uint32_t)(j * C::MT * 4)) : row * ldc + col;
            }
        if (beta != 0.0f) {
            float cv[CH][V];
#pragma unroll
            for (int t = 0; t < CH; ++t)
#pragma unroll
                for (int v = 0; v < V; ++v) cv[t][v] = FRINGE ? fc.load((uint32_t)off[t][v]) : Cblk[off[t][v]];
            // the stores form their offsets anew from the row bases: an opaque
            // column step keeps the compiler from holding the loads' offsets,
            // one register per value, across the loads
            uint32_t step = C::MT * 4;
            if constexpr (FRINGE) asm volatile("" : "+v"(step));
#pragma unroll
            for (int t = 0; t < CH; ++t) {
                const int i = (c0t + t) / C::TN, j = (c0t + t) % C::TN;
                const bool col_ok = !FRINGE || cols_whole || col0 + j * C::MT < N - n0;
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    const float y = __builtin_fmaf(alpha, acc(i, j, v), beta * cv[t][v]);
                    if constexpr (FRINGE) {
                        if (col_ok) fc.put(rb[t][v] + j * step, y);
                    } else {
                        Cblk[off[t][v]] = y;
                    }
                }
            }
        } else {
#pragma unroll
            for (int t = 0; t < CH; ++t) {
                const int i = (c0t + t) / C::TN, j = (c0t + t) % C::TN;
                const bool col_ok = !FRINGE || cols_whole || col0 + j * C::MT < N - n0;
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    if constexpr (FRINGE) {
                        if (col_ok) fc.put(rb[t][v] + (uint32_t)(j * C::MT * 4), alpha * acc(i, j, v));
                    } else {
                        Cblk[off[t][v]] = alpha * acc(i, j, v);
                    }
                }
            }
        }
    }
}

// ---- one workgroup tile ----------------------------------------------------------
template <class C, int DEPTH, int SWZ, bool FRINGE, bool TAIL>
__device__ __forceinline__ void gemm_tile(const GemmParams &p, char *smem, int64_t b, int64_t tm, int64_t tn) {
    using Acc = typename AccT<C>::type;
    constexpr int E = C::ELEM;
    constexpr int NST = C::A_PER_THREAD > C::B_PER_THREAD * C::CHUNK ? C::A_PER_THREAD
                                                                     : C::B_PER_THREAD * C::CHUNK;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const bool a_loader = tid < C::LOADERS;           // wave-uniform
    const int lt = a_loader ? tid : tid - C::LOADERS;  // loader-local thread id

    const int64_t M = p.M, N = p.N, K = p.K;
    const int64_t m0 = tm * C::BM, n0 = tn * C::BN;
    const int lda = (int)p.lda, ldb = (int)p.ldb;
    const char *Ablk = p.A + (b * p.sA + m0 * p.lda) * E;   // A[b][m0][0]
    const char *Bblk = p.B + (b * p.sB + n0) * E;           // B[b][0][n0]
    const int64_t nk = (K + C::BK - 1) / C::BK;
    const bool ragged_k = (K % C::BK) != 0;

    Acc acc[C::TM][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
            acc[i][j] = Acc{};

    u32x4 st[NST];

    // -- global -> registers for K tile kt (guard only where the tile needs it)
    auto gload = [&](int64_t kt) {
        const int64_t k0 = kt * C::BK;
        const bool guard = FRINGE || (ragged_k && kt == nk - 1);
        if (a_loader) {
            const rsrc_t ra = make_rsrc(Ablk + k0 * E);
#pragma unroll
            for (int q = 0; q < C::A_PER_THREAD; ++q) {
                int row, ch;
                copy_a_chunk<C>(lt, q, row, ch);
                const int off = (row * lda + ch * C::CHUNK) * E;
                if (!guard) {
                    st[q] = bload16(ra, off, 0);
                } else {
                    const int64_t left = K - (k0 + ch * C::CHUNK);
                    const bool row_ok = !FRINGE || (m0 + row < M);
                    const int n = !row_ok || left <= 0 ? 0 : (left >= C::CHUNK ? C::CHUNK : (int)left);
                    st[q] = bload16_n<E>(ra, off, 0, n);
                }
            }
        } else {
            const rsrc_t rb = make_rsrc(Bblk + k0 * p.ldb * E);
#pragma unroll
            for (int u = 0; u < C::B_PER_THREAD; ++u) {
                int kb, nb;
                copy_b_unit<C>(lt, u, kb, nb);
                const int64_t cols_left = N - (n0 + nb * C::CHUNK);
                const int ncol = !FRINGE ? C::CHUNK
                                 : (cols_left <= 0 ? 0 : (cols_left >= C::CHUNK ? C::CHUNK : (int)cols_left));
#pragma unroll
                for (int r = 0; r < C::CHUNK; ++r) {
                    const int krow = kb * C::CHUNK + r;
                    const int off = (krow * ldb + nb * C::CHUNK) * E;
                    if (!guard) {
                        st[u * C::CHUNK + r] = bload16(rb, off, 0);
                    } else {
                        const int n = k0 + krow < K ? ncol : 0;
                        st[u * C::CHUNK + r] = bload16_n<E>(rb, off, 0, n);
                    }
                }
            }
        }
    };

    // -- registers -> LDS copy `buf`
    auto lstore = [&](int buf) {
        char *sA = smem + buf * C::STAGE_BYTES;
        char *sB = sA + C::A_TILE_BYTES;
        if (a_loader) {
#pragma unroll
            for (int q = 0; q < C::A_PER_THREAD; ++q) {
                int row, ch;
                copy_a_chunk<C>(lt, q, row, ch);
                *(u32x4 *)(sA + lds_chunk_byte<C>(row, ch, SWZ)) = st[q];
            }
        } else {
#pragma unroll
            for (int u = 0; u < C::B_PER_THREAD; ++u) {
                int kb, nb;
                copy_b_unit<C>(lt, u, kb, nb);
                u32x4 col[C::CHUNK];
                transpose_square<E>(&st[u * C::CHUNK], col);
#pragma unroll
                for (int c = 0; c < C::CHUNK; ++c)
                    *(u32x4 *)(sB + lds_chunk_byte<C>(nb * C::CHUNK + c, kb, SWZ)) = col[c];
            }
        }
    };

    // -- MFMA over LDS copy `buf`
    const int wrow = (wave / C::WAVES_N) * C::WTM;
    const int wcol = (wave % C::WAVES_N) * C::WTN;
    auto compute = [&](int buf) {
        const char *sA = smem + buf * C::STAGE_BYTES;
        const char *sB = sA + C::A_TILE_BYTES;
#pragma unroll
        for (int s = 0; s < C::KSTEPS; ++s) {
            const int ch = frag_chunk<C>(s, lane);
            u32x4 af[C::TM], bfr[C::TN];
#pragma unroll
            for (int i = 0; i < C::TM; ++i)
                af[i] = *(const u32x4 *)(sA + lds_chunk_byte<C>(wrow + i * C::MT + lane % C::MT, ch, SWZ));
#pragma unroll
            for (int j = 0; j < C::TN; ++j)
                bfr[j] = *(const u32x4 *)(sB + lds_chunk_byte<C>(wcol + j * C::MT + lane % C::MT, ch, SWZ));
#pragma unroll
            for (int i = 0; i < C::TM; ++i)
#pragma unroll
                for (int j = 0; j < C::TN; ++j)
                    mfma_chunk<C::DT>(af[i], bfr[j], acc[i][j]);
        }
    };

    if (nk > 0) {
        // prologue: tile 0 -> copy 0
        gload(0);
        lstore(0);
        __syncthreads();
        if (DEPTH == 2) {
            for (int64_t kt = 0; kt < nk; ++kt) {
                const int cur = (int)(kt & 1);
                const bool more = kt + 1 < nk;
                if (more) gload(kt + 1);      // prefetch issued before the compute that hides it
                compute(cur);
                if (more) lstore(cur ^ 1);
                __syncthreads();             // publishes copy cur^1, releases copy cur
            }
        } else {
            for (int64_t kt = 0; kt < nk; ++kt) {
                compute(0);
                if (kt + 1 < nk) {
                    __syncthreads();         // every reader of copy 0 is done
                    gload(kt + 1);
                    lstore(0);
                    __syncthreads();         // copy 0 holds tile kt+1
                }
            }
        }
    }

    // -- epilogue: fused alpha/beta store-back, masks only here
    auto get = [&](int i, int j, int v) { return acc[i][j][v]; };
    store_tile_epilogue<C, FRINGE, decltype(get), 64, TAIL>(p, get, b, m0, n0, wave, lane);
}

template <class C, int DEPTH, int SWZ, bool TAIL = false>
__global__ __launch_bounds__(C::THREADS, 1) void gemm_kernel(GemmParams p) {
    __shared__ __attribute__((aligned(16))) char smem[(DEPTH == 2 ? 2 : 1) * C::STAGE_BYTES];
    int64_t b, tm, tn;
    block_coords(p, b, tm, tn);
    const bool interior = (tm + 1) * C::BM <= p.M && (tn + 1) * C::BN <= p.N;
    if (interior) gemm_tile<C, DEPTH, SWZ, false, TAIL>(p, smem, b, tm, tn);
    else gemm_tile<C, DEPTH, SWZ, true, TAIL>(p, smem, b, tm, tn);
}

}  // namespace tg
