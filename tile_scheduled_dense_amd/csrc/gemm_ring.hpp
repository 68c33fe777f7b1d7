// gemm_ring.hpp -- the gfx950 kernel for bf16/fp16 inputs: a K ring of LDS
// copies filled by direct global -> LDS copies.
//
// Same contraction, block order, partition and epilogue as gemm_kernel.hpp;
// what differs is the staging (OCANNL Stage paragraph: shared + cooperative,
// pipeline_depth; LuisaCompute "Pipelines and stage boundaries": window,
// prologue / steady state / epilogue, issue vs completion vs release):
//
//  * STAGES LDS copies of a 32-deep K tile (A [BM][32], B [32][BN]).  Each wave
//    issues, per tile, a few 1-KiB buffer-to-LDS copies (no registers hold the
//    data).  Tile kt + STAGES - 1 is issued while tile kt is multiplied, so a
//    copy has STAGES - 1 tiles of MFMA work to arrive: the window is STAGES - 1.
//  * Iteration kt: wait until this wave's copies of tile kt have landed
//    (vmcnt counts them in issue order), one barrier (every wave's copies of
//    tile kt are now visible, and every wave has finished reading tile kt - 1,
//    whose copy is released), issue tile kt + STAGES - 1 into that released
//    copy, multiply tile kt.  One barrier per tile; with STAGES == 1 the
//    unpipelined form with two barriers per tile.
//  * Pad-to-tile: rows of A beyond M and 8-column chunks of B beyond N are
//    fetched as zeros (their buffer offset is past the resource's size, which
//    the hardware answers with 0).  A chunk that crosses N carries the row's
//    own padding in its out-of-range columns; those columns only feed outputs
//    the masked store-back never writes.  The last K tile is always copied
//    through registers with element-exact guards (k >= K is +0 in both
//    operands, so NaN in a leading-dimension pad cannot meet a zero): it is
//    loaded in the prologue and written into its LDS copy when its turn comes.
//  * Fragments: A by ds_read_b128 (8 consecutive k of one row per lane), B by
//    two ds_read_b64_tr_b16 per MFMA (within each 16-lane group lane i receives
//    element e of source lane 4e + i/4, which turns 4 row-reads of 4 columns
//    into 4 k-values of one column per lane), so B needs no transpose in
//    registers.
#pragma once

#include "gemm_kernel.hpp"

namespace tg {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#define TG_LDS_PTR(p) ((__attribute__((address_space(3))) void *)(p))

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Resource over [base, base + nbytes): offsets past nbytes read as 0.
__device__ __forceinline__ rsrc_t make_rsrc_n(const char *base, int64_t nbytes) {
    const uint64_t a = (uint64_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const char *u = (const char *)(((uint64_t)hi << 32) | lo);
    const int n = nbytes > 0x7fffffffLL ? 0x7fffffff : (int)nbytes;
    return __builtin_amdgcn_make_buffer_rsrc((void *)u, (short)0, __builtin_amdgcn_readfirstlane(n), 0x00020000);
}

constexpr int kOutOfRange = (int)0x80000000u;   // >= every resource size: reads as 0

// One 1-KiB buffer -> LDS copy: lane l's 16 bytes at byte `voff` of the
// resource land at LDS byte lds_addr + 16 l.  Issued as inline assembly so the
// compiler does not treat it as an LDS write of unknown address and put a full
// vmcnt(0) wait in front of every later LDS read (which would empty the ring
// each iteration); the ring's own waits cover it.  The s_nop covers the
// SGPR-written-by-VALU and M0 hazards before the memory instruction; M0 is
// restored afterwards.
typedef int i32x4 __attribute__((ext_vector_type(4)));

// The same 128-bit resource as make_rsrc_n, as four scalar words: base (48
// bits), stride 0, size limit, gfx9 data-format word.
__device__ __forceinline__ i32x4 rsrc_words(const char *base, int64_t nbytes) {
    const uint64_t a = (uint64_t)base;
    const int lo = (int)__builtin_amdgcn_readfirstlane((uint32_t)a);
    const int hi = (int)(__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) & 0xffffu);
    const int n = __builtin_amdgcn_readfirstlane(nbytes > 0x7fffffffLL ? 0x7fffffff : (int)nbytes);
    return i32x4{lo, hi, n, 0x00020000};
}

__device__ __forceinline__ void copy_to_lds(i32x4 rs, uint32_t lds_addr, int voff) {
    int saved_m0;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 4\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved_m0)
        : "s"(lds_addr), "v"(voff), "s"(rs)
        : "memory");
}

__device__ __forceinline__ uint32_t lds_address(const char *p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)TG_LDS_PTR(p));
}

template <class C, int STAGES, int SWZ, bool FRINGE>
__device__ __forceinline__ void ring_tile(const GemmParams &p, char *smem, int64_t b, int64_t tm, int64_t tn) {
    using Acc = f32x16;
    constexpr int E = 2;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t M = p.M, N = p.N, K = p.K;
    const int64_t m0 = tm * C::BM, n0 = tn * C::BN;
    const int lda = (int)p.lda, ldb = (int)p.ldb;
    const char *Ablk = p.A + (b * p.sA + m0 * p.lda) * E;   // A[b][m0][0]
    const char *Bblk = p.B + (b * p.sB + n0) * E;           // B[b][0][n0]
    // bytes from the block bases to one past the last valid element
    const int64_t a_valid = ((M - m0 - 1) * p.lda + K) * E;
    const int64_t b_valid = ((K - 1) * p.ldb + (N - n0)) * E;
    const int64_t nk = (K + C::BK - 1) / C::BK;
    const int64_t ndma = nk > 0 ? nk - 1 : 0;             // tiles copied straight to LDS

    Acc acc[C::TM][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j) acc[i][j] = Acc{};

    // This lane's sources: A (row, k) and B (k, n) of each of its copies.
    int a_row[C::A_DMA], a_k[C::A_DMA], a_off[C::A_DMA];
    int b_k[C::B_DMA], b_n[C::B_DMA], b_off[C::B_DMA];
#pragma unroll
    for (int d = 0; d < C::A_DMA; ++d) {
        ring_a_source<C>(ring_block<C>(d, wave), lane, SWZ, a_row[d], a_k[d]);
        a_off[d] = (FRINGE && m0 + a_row[d] >= M) ? kOutOfRange : (a_row[d] * lda + a_k[d]) * E;
    }
#pragma unroll
    for (int d = 0; d < C::B_DMA; ++d) {
        ring_b_source<C>(ring_block<C>(d, wave), lane, SWZ, b_k[d], b_n[d]);
        b_off[d] = (FRINGE && n0 + b_n[d] >= N) ? kOutOfRange : (b_k[d] * ldb + b_n[d]) * E;
    }

    // -- direct copy of K tile kt into LDS copy `stage`
    auto dma = [&](int64_t kt, int stage) {
        const int64_t k0 = kt * C::BK;
        const i32x4 ra = rsrc_words(Ablk + k0 * E, a_valid - k0 * E);
        const i32x4 rb = rsrc_words(Bblk + k0 * p.ldb * E, b_valid - k0 * p.ldb * E);
        char *sA = smem + stage * C::STAGE_BYTES;
        char *sB = sA + C::A_TILE_BYTES;
#pragma unroll
        for (int d = 0; d < C::A_DMA; ++d) copy_to_lds(ra, lds_address(sA + ring_block<C>(d, wave) * 1024), a_off[d]);
#pragma unroll
        for (int d = 0; d < C::B_DMA; ++d) copy_to_lds(rb, lds_address(sB + ring_block<C>(d, wave) * 1024), b_off[d]);
    };

    // -- the last K tile through registers, element-exact zero fill
    u32x4 tail[C::COPIES];
    auto tail_load = [&]() {
        const int64_t k0 = (nk - 1) * C::BK;
        const rsrc_t ra = make_rsrc_n(Ablk + k0 * E, a_valid - k0 * E);
        const rsrc_t rb = make_rsrc_n(Bblk + k0 * p.ldb * E, b_valid - k0 * p.ldb * E);
#pragma unroll
        for (int d = 0; d < C::A_DMA; ++d) {
            const int64_t left = K - (k0 + a_k[d]);
            const bool row_ok = m0 + a_row[d] < M;
            const int n = !row_ok || left <= 0 ? 0 : (left >= C::CHUNK ? C::CHUNK : (int)left);
            tail[d] = bload16_n<E>(ra, (a_row[d] * lda + a_k[d]) * E, 0, n);
        }
#pragma unroll
        for (int d = 0; d < C::B_DMA; ++d) {
            const int64_t cols = N - (n0 + b_n[d]);
            const bool k_ok = k0 + b_k[d] < K;
            const int n = !k_ok || cols <= 0 ? 0 : (cols >= C::CHUNK ? C::CHUNK : (int)cols);
            tail[C::A_DMA + d] = bload16_n<E>(rb, (b_k[d] * ldb + b_n[d]) * E, 0, n);
        }
    };
    auto tail_store = [&](int stage) {
        char *sA = smem + stage * C::STAGE_BYTES;
        char *sB = sA + C::A_TILE_BYTES;
#pragma unroll
        for (int d = 0; d < C::A_DMA; ++d) *(u32x4 *)(sA + ring_block<C>(d, wave) * 1024 + 16 * lane) = tail[d];
#pragma unroll
        for (int d = 0; d < C::B_DMA; ++d)
            *(u32x4 *)(sB + ring_block<C>(d, wave) * 1024 + 16 * lane) = tail[C::A_DMA + d];
    };

    // -- MFMA over LDS copy `stage`
    const int wrow = (wave / C::WAVES_N) * C::WTM;
    const int wcol = (wave % C::WAVES_N) * C::WTN;
    const int grp = lane / 16, gi = lane % 16;
    auto compute = [&](int stage) {
        const char *sA = smem + stage * C::STAGE_BYTES;
        const char *sB = sA + C::A_TILE_BYTES;
#pragma unroll
        for (int s = 0; s < C::KSTEPS; ++s) {
            u32x4 af[C::TM], bfr[C::TN];
#pragma unroll
            for (int i = 0; i < C::TM; ++i)
                af[i] = *(const u32x4 *)(sA + ring_a_byte<C>(wrow + i * C::MT + lane % 32, 2 * s + lane / 32, SWZ));
#pragma unroll
            for (int j = 0; j < C::TN; ++j) {
                const int k = 16 * s + 8 * (grp / 2) + gi / 4;
                const int n = wcol + j * C::MT + 16 * (grp % 2) + 4 * (gi % 4);
                const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) v4i16 *)(sB + ring_b_byte<C>(k, n, SWZ)));
                const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) v4i16 *)(sB + ring_b_byte<C>(k + 4, n, SWZ)));
                const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                bfr[j] = u32x4{l2.x, l2.y, h2.x, h2.y};
            }
#pragma unroll
            for (int i = 0; i < C::TM; ++i)
#pragma unroll
                for (int j = 0; j < C::TN; ++j) mfma_chunk<C::DT>(af[i], bfr[j], acc[i][j]);
        }
    };

    if (nk > 0) {
        tail_load();
        if (STAGES == 1) {
            for (int64_t kt = 0; kt < nk; ++kt) {
                if (kt > 0) {
                    wait_lds();
                    block_barrier();        // every wave is done reading the single copy
                }
                if (kt < ndma) {
                    dma(kt, 0);
                    wait_vmcnt<0>();
                } else {
                    wait_vmcnt<0>();
                    tail_store(0);
                }
                wait_lds();
                block_barrier();            // tile kt is in LDS for every wave
                compute(0);
            }
        } else {
#pragma unroll
            for (int t = 0; t < STAGES - 1; ++t)
                if (t < ndma) dma(t, t);
            for (int64_t kt = 0; kt < nk; ++kt) {
                const int stage = (int)(kt % STAGES);
                if (kt < ndma) {
                    // copies issued after tile kt: tiles kt+1 .. min(kt+STAGES-2, ndma-1)
                    const int64_t later = ndma - 1 - kt;
                    if (STAGES >= 4 && later >= 2) wait_vmcnt<2 * C::COPIES>();
                    else if (STAGES >= 3 && later >= 1) wait_vmcnt<C::COPIES>();
                    else wait_vmcnt<0>();
                } else {
                    wait_vmcnt<0>();
                    tail_store(stage);
                }
                wait_lds();
                block_barrier();            // tile kt visible; copy of tile kt-1 released
                const int64_t t = kt + STAGES - 1;
                if (t < ndma) dma(t, (int)(t % STAGES));
                compute(stage);
            }
        }
    }

    // -- epilogue: fused alpha/beta store-back, masks only here
    store_tile_epilogue<C, FRINGE>(p, acc, b, m0, n0, wave, lane);
}

template <class C, int STAGES, int SWZ>
__global__ __launch_bounds__(C::THREADS, 1) void gemm_ring_kernel(GemmParams p) {
    static_assert(STAGES >= 1 && STAGES <= 4, "1 to 4 LDS copies");
    __shared__ __attribute__((aligned(1024))) char smem[STAGES * C::STAGE_BYTES];
    int64_t b, tm, tn;
    block_coords(p, b, tm, tn);
    const bool interior = (tm + 1) * C::BM <= p.M && (tn + 1) * C::BN <= p.N;
    if (interior) ring_tile<C, STAGES, SWZ, false>(p, smem, b, tm, tn);
    else ring_tile<C, STAGES, SWZ, true>(p, smem, b, tm, tn);
}

}  // namespace tg
