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

// The two K-loop schedules (template argument of gemm_ring_kernel).
enum { SCHED_RING = 0, SCHED_SWPIPE = 1 };

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#define TG_LDS_PTR(p) ((__attribute__((address_space(3))) void *)(p))

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }


// One 1-KiB buffer -> LDS copy: lane l's 16 bytes at byte `voff` of the
// resource land at LDS byte lds_addr + 16 l.  Issued as inline assembly so the
// compiler does not treat it as an LDS write of unknown address and put a full
// vmcnt(0) wait in front of every later LDS read (which would empty the ring
// each iteration); the ring's own waits cover it.  The s_nop covers the
// SGPR-written-by-VALU and M0 hazards before the memory instruction; M0 is
// declared clobbered, so the compiler sets it again wherever it needs it.
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

__device__ __forceinline__ uint64_t uniform_u64(uint64_t a) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// rsrc_words for a base already known to be uniform (no lane reads needed).
__device__ __forceinline__ i32x4 rsrc_words_u(uint64_t base, int64_t nbytes) {
    const int n = nbytes > 0x7fffffffLL ? 0x7fffffff : (int)nbytes;
    return i32x4{(int)(uint32_t)base, (int)((uint32_t)(base >> 32) & 0xffffu), n, 0x00020000};
}

// G (1, 2 or 4) adjacent 1-KiB buffer-to-LDS copies under one m0 value.
// Copy g lands at LDS address lds_addr + 1024 g (+ 16 per lane); the
// instruction's immediate offset 1024 g also moves the global address, so the
// caller passes voff[g] already reduced by 1024 g relative to the resource base
// (and the resource's base lowered to keep every voff non-negative).  Writing
// m0 while an earlier copy of the wave is still being issued holds the wave
// back, so one m0 write per group instead of one per copy roughly doubles the
// copy rate a wave can sustain.
// M0 is named in the clobber list, which clang flags as a reserved register
// (-Winline-asm); the kernels use M0 nowhere else (a test scans the built code
// object for any other M0 access), so the compiler has no value in it to lose.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int G>
__device__ __forceinline__ void copy_group_to_lds(i32x4 rs, uint32_t lds_addr, const int *voff) {
    static_assert(G == 1 || G == 2 || G == 4, "1, 2 or 4 copies per group");
    // both operands are uniform by construction; say so for the SGPR constraints
    lds_addr = __builtin_amdgcn_readfirstlane(lds_addr);
    rs = i32x4{__builtin_amdgcn_readfirstlane(rs.x), __builtin_amdgcn_readfirstlane(rs.y),
               __builtin_amdgcn_readfirstlane(rs.z), __builtin_amdgcn_readfirstlane(rs.w)};
    if constexpr (G == 1) {
        asm volatile(
            "s_mov_b32 m0, %0\n\t"
            "s_nop 0\n\t"
            "buffer_load_dwordx4 %1, %2, 0 offen lds"
            :
            : "s"(lds_addr), "v"(voff[0]), "s"(rs)
            : "memory", "m0");
    } else if constexpr (G == 2) {
        asm volatile(
            "s_mov_b32 m0, %0\n\t"
            "s_nop 0\n\t"
            "buffer_load_dwordx4 %1, %3, 0 offen lds\n\t"
            "buffer_load_dwordx4 %2, %3, 0 offen offset:1024 lds"
            :
            : "s"(lds_addr), "v"(voff[0]), "v"(voff[1]), "s"(rs)
            : "memory", "m0");
    } else {
        asm volatile(
            "s_mov_b32 m0, %0\n\t"
            "s_nop 0\n\t"
            "buffer_load_dwordx4 %1, %5, 0 offen lds\n\t"
            "buffer_load_dwordx4 %2, %5, 0 offen offset:1024 lds\n\t"
            "buffer_load_dwordx4 %3, %5, 0 offen offset:2048 lds\n\t"
            "buffer_load_dwordx4 %4, %5, 0 offen offset:3072 lds"
            :
            : "s"(lds_addr), "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "s"(rs)
            : "memory", "m0");
    }
}
#pragma clang diagnostic pop

__device__ __forceinline__ uint32_t lds_address(const char *p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)TG_LDS_PTR(p));
}

// The accumulators of one wave's TM x TN MFMA tiles: an f32x16 per 32x32
// tile, an f32x4 per 16x16 tile.
//
// 16x16x32 MFMAs are issued as inline assembly with the accumulator tied to
// AGPRs: through the builtin, the register allocator keeps a third of the 64
// four-register accumulators in VGPRs and copies them into AGPRs and back
// around their MFMAs every K tile.  The compiler does not see these as
// MFMAs, so the two hazards that involve them are handled here: the first
// K tile's MFMAs take a zero accumulator input (mma<true>, no VALU write of
// an accumulator ever precedes an MFMA), and settle() pads the last MFMA's
// results with wait states before anything else reads them.  Dependent MFMAs
// on one accumulator are a whole K tile apart.  INLINE = false keeps the
// compiler's builtin (and its hazard handling): the unpipelined depth-1
// schedule of the 256 x 256 tile spills accumulators, and the spill copies
// next to an MFMA the compiler cannot see would read its result too early.
template <class C, bool INLINE = true>
struct AccTiles {
    static constexpr bool ASM = INLINE && C::MT == 16;
    typename AccT<C>::type r[C::TM][C::TN];
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
            for (int j = 0; j < C::TN; ++j) r[i][j] = typename AccT<C>::type{};
    }
    // r[i][j] += a . b, or r[i][j] = a . b for the first K step (FIRST).  fp32:
    // one 16x16x4 MFMA on element e of both fragments (the same k).
    template <bool FIRST>
    __device__ __forceinline__ void mma(int i, int j, const u32x4 &a, const u32x4 &b, int e = 0) {
        if constexpr (C::DT == DT_F32) {
            if constexpr (ASM) {
                if (FIRST) asm volatile("v_mfma_f32_16x16x4_f32 %0, %1, %2, 0" : "=a"(r[i][j]) : "v"(a[e]), "v"(b[e]));
                else asm volatile("v_mfma_f32_16x16x4_f32 %0, %1, %2, %0" : "+a"(r[i][j]) : "v"(a[e]), "v"(b[e]));
            } else {
                // the element copied out first: a bit_cast of a vector-element
                // lvalue reads element 0
                const uint32_t ae = a[e], be = b[e];
                r[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(__builtin_bit_cast(float, ae),
                                                             __builtin_bit_cast(float, be), r[i][j], 0, 0, 0);
            }
        } else if constexpr (ASM) {
            if constexpr (C::DT == DT_BF16) {
                if (FIRST) asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(r[i][j]) : "v"(a), "v"(b));
                else asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(r[i][j]) : "v"(a), "v"(b));
            } else {
                if (FIRST) asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, 0" : "=a"(r[i][j]) : "v"(a), "v"(b));
                else asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(r[i][j]) : "v"(a), "v"(b));
            }
        } else {
            mfma_chunk<C::DT>(a, b, r[i][j]);
        }
    }
    // after the last MFMA: 32 wait states (an XDL result needs at most 19
    // before a VALU or memory instruction reads it), fenced so the scheduler
    // moves nothing across
    __device__ __forceinline__ void settle() {
        if constexpr (ASM) {
            __builtin_amdgcn_sched_barrier(0);
            asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // value v (0 <= v < ACC_PER_MFMA) of MFMA tile (i, j), after settle().  The
    // inline-assembly MFMAs' accumulators are read by an inline-assembly
    // v_accvgpr_read of the AGPR itself: left to the compiler, a value needed
    // later in a VGPR may be copied out right behind the MFMA that writes it,
    // before the result is there (the compiler does not know these are MFMAs).
    __device__ __forceinline__ float get(int i, int j, int v) const {
        if constexpr (ASM) {
            float x;
            asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(x) : "a"(r[i][j][v]));
            return x;
        } else {
            return r[i][j][v];
        }
    }
};

// One workgroup's tile of the 16-bit family: copy sources, the copies, the
// register-path last tile, fragment reads and the MFMAs, shared by the
// schedules below.
// FRINGE: rows past M and 8-column chunks past N are masked (read as 0, not
// stored).  LIMIT (fringe blocks only): every copy's resource also ends at the
// operand's last valid element, for a block whose N edge cuts a 16-byte chunk;
// without it the copies advance one resource per operand, as interior blocks
// do (the copied K tiles lie inside K, masked rows read nothing, and no chunk
// reaches past N).
template <class C, int STAGES, int SWZ, bool FRINGE, bool LIMIT = FRINGE>
struct RingBlock {
    static constexpr int E = C::ELEM;
    const GemmParams &p;
    char *smem;
    int lane, wave;
    int64_t b, m0, n0, nk, ndma;
    int lda, ldb;
    const char *Ablk, *Bblk;
    int64_t a_valid, b_valid;
    // the copy plan of each operand tile under this placement (tile_config.hpp)
    using CA = RingCopy<C, SWZ, 0>;
    using CB = RingCopy<C, SWZ, 1>;
    static constexpr int A_PER = CA::PER, B_PER = CB::PER;
    static constexpr int COPIES = A_PER + B_PER;             // copy instructions per wave per K tile
    static constexpr int A_PITCH = CA::PITCH, B_PITCH = CB::PITCH;
    static constexpr int A_STAGE = CA::REGION, B_STAGE = CB::REGION;   // LDS bytes per pipeline copy
    // A padded slot (fetched as zeros) keeps a k of kPadSlot: past every K (the
    // host keeps K below 2^30), so the register path of the last K tile loads
    // nothing for it either.
    static constexpr int kPadSlot = 1 << 30;
    int a_row[A_PER], a_k[A_PER], a_off[A_PER], a_voff[A_PER];
    int b_k[B_PER], b_n[B_PER], b_off[B_PER], b_voff[B_PER];
    // a group's resource base sits this far below the tile's first byte
    static constexpr int A_SHIFT = (CA::GMAX - 1) * 1024, B_SHIFT = (CB::GMAX - 1) * 1024;
    uint64_t a_base, b_base;    // Ablk, Bblk as workgroup-uniform integers
    uint32_t lds0;              // LDS address of smem
    int64_t b_step;             // bytes of B per K tile
    i32x4 rsa, rsb;             // interior blocks: resources of the next K tile to copy
    uint32_t a_rd[C::KSTEPS];           // LDS address of this lane's A fragment of row tile 0, copy 0
    uint32_t b_rd[C::KSTEPS][C::TN];    // ... of its B fragment (first read) of column tile j, copy 0
    u32x4 tail[COPIES];
    AccTiles<C, (STAGES > 1)> acc;

    // LDS: the STAGES copies of the B tile, then the STAGES copies of the A
    // tile, so a fragment read of a known copy is a fixed base register plus an
    // offset that fits the 16-bit immediate of a DS instruction.  B goes first:
    // its reads need one base register per MFMA column tile (the swizzle XOR
    // depends on it), A's a single one, which then absorbs the region offset.
    // (Under pad_stride the A offsets exceed the 16-bit immediate for the later
    // copies; the compiler then adds them in a register, which only costs time.)
    static constexpr int A_REGION = STAGES * B_STAGE;
    static constexpr int a_tile(int stage) { return A_REGION + stage * A_STAGE; }
    static constexpr int b_tile(int stage) { return stage * B_STAGE; }
    static_assert(SWZ == SWZ_PAD || ((STAGES - 1) * A_STAGE + (C::TM - 1) * C::MT * A_PITCH + 48 < 65536 &&
                                     (STAGES - 1) * B_STAGE + 4 * B_PITCH < 65536), "DS immediate offsets");

    __device__ __forceinline__ RingBlock(const GemmParams &p_, char *smem_, int64_t b_, int64_t tm, int64_t tn)
        : p(p_), smem(smem_), b(b_) {
        lane = threadIdx.x & 63;
        wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // the same in every lane of a wave
        m0 = tm * C::BM;
        n0 = tn * C::BN;
        lda = (int)p.lda;
        ldb = (int)p.ldb;
        Ablk = p.A + (b * p.sA + m0 * p.lda) * E;   // A[b][m0][0]
        Bblk = p.B + (b * p.sB + n0) * E;           // B[b][0][n0]
        // bytes from the block bases to one past the last valid element
        a_valid = ((p.M - m0 - 1) * p.lda + p.K) * E;
        b_valid = ((p.K - 1) * p.ldb + (p.N - n0)) * E;
        nk = (p.K + C::BK - 1) / C::BK;
        ndma = nk > 0 ? nk - 1 : 0;                 // tiles copied straight to LDS
        a_base = uniform_u64((uint64_t)Ablk);
        b_base = uniform_u64((uint64_t)Bblk);
        lds0 = lds_address(smem);
        b_step = (int64_t)C::BK * p.ldb * E;
        rsa = rsrc_words_u(a_base - A_SHIFT, 0x7fffffff);
        rsb = rsrc_words_u(b_base - B_SHIFT, 0x7fffffff);
        // Fragment read addresses: every read is one of these plus a constant
        // (the LDS copy, the row / column tile, the second half of a B read).
        // The empty asm keeps the compiler from splitting a base back into a
        // constant part, which would not fit the 16-bit DS offset.
        {
            const int wrow = (wave / C::WAVES_N) * C::WTM;
            const int wcol = (wave % C::WAVES_N) * C::WTN;
#pragma unroll
            for (int s = 0; s < C::KSTEPS; ++s) {
                a_rd[s] = lds0 + a_tile(0) + ring_a_byte<C>(a_frag_row(wrow, 0), a_frag_chunk(s), SWZ);
                asm("" : "+v"(a_rd[s]));
#pragma unroll
                for (int j = 0; j < C::TN; ++j) {
                    int k, n;
                    b_frag_src(wcol, j, s, 0, k, n);
                    b_rd[s][j] = lds0 + b_tile(0) + ring_b_byte<C>(k, n, SWZ);
                    asm("" : "+v"(b_rd[s][j]));
                }
            }
        }
        acc.zero();
#pragma unroll
        for (int d = 0; d < A_PER; ++d) {
            const bool ok = ring_a_source<C>(CA::block(d, wave), lane, SWZ, a_row[d], a_k[d]);
            a_off[d] = (!ok || (FRINGE && m0 + a_row[d] >= p.M)) ? kOutOfRange : (a_row[d] * lda + a_k[d]) * E;
            a_voff[d] = a_off[d] + A_SHIFT - 1024 * CA::pos(d);
            if (!ok) a_k[d] = kPadSlot;
        }
#pragma unroll
        for (int d = 0; d < B_PER; ++d) {
            const bool ok = ring_b_source<C>(CB::block(d, wave), lane, SWZ, b_k[d], b_n[d]);
            b_off[d] = (!ok || (FRINGE && n0 + b_n[d] >= p.N)) ? kOutOfRange : (b_k[d] * ldb + b_n[d]) * E;
            b_voff[d] = b_off[d] + B_SHIFT - 1024 * CB::pos(d);
            if (!ok) b_k[d] = kPadSlot;
        }
    }

    // Interior blocks of one problem (batch entry 0): point the copy resources
    // at K tile 0 of tile (tm, tn), leaving m0 / n0 (the epilogue's) alone.
    __device__ __forceinline__ void retarget(int64_t tm, int64_t tn) {
        a_base = uniform_u64((uint64_t)(p.A + tm * C::BM * p.lda * E));
        b_base = uniform_u64((uint64_t)(p.B + tn * C::BN * E));
        rsa = rsrc_words_u(a_base - A_SHIFT, 0x7fffffff);
        rsb = rsrc_words_u(b_base - B_SHIFT, 0x7fffffff);
    }

    // 64-bit add to the base address held in the first two resource words
    __device__ __forceinline__ static void advance(i32x4 &rs, uint64_t bytes) {
        const uint64_t a = (((uint64_t)(uint32_t)rs.y << 32) | (uint32_t)rs.x) + bytes;
        rs.x = (int)(uint32_t)a;
        rs.y = (int)(uint32_t)(a >> 32);
    }

    // The copies of one operand under resource rs into the LDS copy at `region`:
    // the wave's own run of Q adjacent blocks in groups of at most four under
    // one M0 value each, then the shared block, if any.
    template <class CP, int NPER>
    __device__ __forceinline__ void copy_operand(i32x4 rs, uint32_t region, const int (&voff)[NPER]) const {
        static_assert(NPER == CP::PER, "copy plan");
        constexpr int G0 = CP::Q < 4 ? CP::Q : 4;
        copy_group_to_lds<G0>(rs, region + CP::block(0, wave) * 1024, &voff[0]);
        if constexpr (CP::Q > 4) {
            constexpr int G1 = CP::Q - 4;
            static_assert(G1 == 1 || G1 == 2 || G1 == 4, "second group of the run");
            copy_group_to_lds<G1>(rs, region + CP::block(4, wave) * 1024, &voff[4]);
        }
        if constexpr (CP::SHARED) {
            copy_group_to_lds<1>(rs, region + CP::block(CP::Q, wave) * 1024, &voff[CP::Q]);
        }
    }

    // this wave's copies of one operand (0 = A, 1 = B) of K tile kt into LDS copy `stage`.
    // Every schedule copies the K tiles in increasing order, each once.
    __device__ __forceinline__ void dma_operand(int64_t kt, int stage, int operand) {
        // An interior block's copied tiles lie wholly inside A and B, so its
        // resources need no size limit beyond the 31-bit offsets and are
        // advanced by one K tile per copy; a LIMIT block's limit ends at the
        // last valid element (past it reads as 0).
        if (operand == 0) {
            const uint32_t region = lds0 + a_tile(stage);
            if (LIMIT) {
                const int64_t adv = kt * (C::BK * E);
                copy_operand<CA>(rsrc_words_u(a_base + adv - A_SHIFT, a_valid - adv + A_SHIFT), region, a_voff);
            } else {
                copy_operand<CA>(rsa, region, a_voff);
                advance(rsa, C::BK * E);
            }
        } else {
            const uint32_t region = lds0 + b_tile(stage);
            if (LIMIT) {
                const int64_t adv = kt * b_step;
                copy_operand<CB>(rsrc_words_u(b_base + adv - B_SHIFT, b_valid - adv + B_SHIFT), region, b_voff);
            } else {
                copy_operand<CB>(rsb, region, b_voff);
                advance(rsb, (uint64_t)b_step);
            }
        }
    }

    // direct copy of K tile kt into LDS copy `stage`
    __device__ __forceinline__ void dma(int64_t kt, int stage) {
        dma_operand(kt, stage, 0);
        dma_operand(kt, stage, 1);
    }

    // the last K tile through registers, element-exact zero fill
    __device__ __forceinline__ void tail_load() {
        const int64_t k0 = (nk - 1) * C::BK;
        const rsrc_t ra = make_rsrc_n(Ablk + k0 * E, a_valid - k0 * E);
        const rsrc_t rb = make_rsrc_n(Bblk + k0 * p.ldb * E, b_valid - k0 * p.ldb * E);
#pragma unroll
        for (int d = 0; d < A_PER; ++d) {
            const int64_t left = p.K - (k0 + a_k[d]);
            const bool row_ok = m0 + a_row[d] < p.M;
            const int n = !row_ok || left <= 0 ? 0 : (left >= C::CHUNK ? C::CHUNK : (int)left);
            tail[d] = bload16_n<E>(ra, n > 0 ? (a_row[d] * lda + a_k[d]) * E : 0, 0, n);
        }
#pragma unroll
        for (int d = 0; d < B_PER; ++d) {
            const int64_t cols = p.N - (n0 + b_n[d]);
            const bool k_ok = k0 + b_k[d] < p.K;
            const int n = !k_ok || cols <= 0 ? 0 : (cols >= C::CHUNK ? C::CHUNK : (int)cols);
            tail[A_PER + d] = bload16_n<E>(rb, n > 0 ? (b_k[d] * ldb + b_n[d]) * E : 0, 0, n);
        }
    }
    __device__ __forceinline__ void tail_store(int stage) {
        char *sA = smem + a_tile(stage);
        char *sB = smem + b_tile(stage);
#pragma unroll
        for (int d = 0; d < A_PER; ++d)
            *(u32x4 *)(sA + CA::block(d, wave) * 1024 + 16 * lane) = tail[d];
#pragma unroll
        for (int d = 0; d < B_PER; ++d)
            *(u32x4 *)(sB + CB::block(d, wave) * 1024 + 16 * lane) = tail[A_PER + d];
    }

    // Wait until this wave's share of tile t is in LDS (its copies, or for
    // the last tile its register stores), `ahead` = tiles issued after t at
    // most (the lookahead still in flight).
    template <int AHEAD>
    __device__ __forceinline__ void land_tile(int64_t t, int stage) {
        if (t < ndma) {
            const int64_t later = ndma - 1 - t;
            if (AHEAD >= 3 && later >= 3) wait_vmcnt<3 * COPIES>();
            else if (AHEAD >= 2 && later >= 2) wait_vmcnt<2 * COPIES>();
            else if (AHEAD >= 1 && later >= 1) wait_vmcnt<COPIES>();
            else wait_vmcnt<0>();
        } else {
            wait_vmcnt<0>();
            tail_store(stage);
        }
        wait_lds();
    }

    // A fragment of row tile i, K step s, from LDS copy `stage`: row tile i
    // lies i * MT rows on (the swizzle XOR is the same for it), so its address
    // is a_rd[s] plus a constant
    __device__ __forceinline__ u32x4 read_a(int stage, int s, int i) const {
        const uint32_t addr = a_rd[s] + stage * A_STAGE + i * C::MT * A_PITCH;
        return *(const __attribute__((address_space(3))) u32x4 *)(uintptr_t)addr;
    }
    // fp32: B element of MFMA step e (e rows on from the read step's first, the same XOR)
    __device__ __forceinline__ uint32_t read_b32(int stage, int s, int j, int e) const {
        const uint32_t addr = b_rd[s][j] + stage * B_STAGE + e * B_PITCH;
        return *(const __attribute__((address_space(3))) uint32_t *)(uintptr_t)addr;
    }
    // one of the two transposing B reads (half: 4 k rows on, the same XOR)
    __device__ __forceinline__ u32x2 read_b(int stage, int s, int j, int half) const {
        const uint32_t addr = b_rd[s][j] + stage * B_STAGE + half * 4 * B_PITCH;
        const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16 *)(uintptr_t)addr);
        return __builtin_bit_cast(u32x2, v);
    }

    // fragments of K step s of LDS copy `stage`
    __device__ __forceinline__ void read_frags(int stage, int s, u32x4 (&af)[C::TM], u32x4 (&bfr)[C::TN]) const {
#pragma unroll
        for (int i = 0; i < C::TM; ++i) af[i] = read_a(stage, s, i);
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
            if constexpr (C::DT == DT_F32) {
                bfr[j] = u32x4{read_b32(stage, s, j, 0), read_b32(stage, s, j, 1), read_b32(stage, s, j, 2),
                               read_b32(stage, s, j, 3)};
            } else {
                const u32x2 l2 = read_b(stage, s, j, 0), h2 = read_b(stage, s, j, 1);
                bfr[j] = u32x4{l2.x, l2.y, h2.x, h2.y};
            }
        }
    }

    // MFMA operand fragments.  A: lane l holds 8 consecutive k (one 16-byte
    // chunk) of row l % MT of MFMA row tile i; the LANE_GROUPS groups of MT
    // lanes take consecutive chunks.  B (transposing read): lane L = 16 g + i
    // of a 16-lane group supplies the address of 4 consecutive n of one k row
    // and receives 4 consecutive k of column i; (k, n) below is that row and
    // first column for the first of the two reads (the second is 4 rows on).
    __device__ __forceinline__ int a_frag_row(int wrow, int i) const { return wrow + i * C::MT + lane % C::MT; }
    __device__ __forceinline__ int a_frag_chunk(int s) const { return C::LANE_GROUPS * s + lane / C::MT; }
    __device__ __forceinline__ void b_frag_src(int wcol, int j, int s, int half, int &k, int &n) const {
        const int grp = lane / 16, gi = lane % 16;
        if (C::DT == DT_F32) {
            // fp32: lane L = 16 g + i reads B[4 g + e][column i] for MFMA step e
            // (`half` is e here); the rows of one read step are 4 g .. 4 g + 3
            k = C::MK * C::MFMA_PER_READ * s + 4 * grp + half;
            n = wcol + j * 16 + gi;
        } else if (C::MT == 32) {
            k = 16 * s + 8 * (grp / 2) + gi / 4 + 4 * half;
            n = wcol + j * 32 + 16 * (grp % 2) + 4 * (gi % 4);
        } else {
            k = 32 * s + 8 * grp + gi / 4 + 4 * half;
            n = wcol + j * 16 + 4 * (gi % 4);
        }
    }

    // Fragment piece r of K tile `stage` (r < READS): A pieces first
    // (s, i), then B reads (s, j, piece); a 16-bit B piece fills one half of a
    // u32x4, an fp32 one one element.
    static constexpr int READS = C::KSTEPS * (C::TM + C::B_PIECES * C::TN);
    __device__ __forceinline__ void read_piece(int stage, int r, u32x4 (&af)[C::KSTEPS][C::TM],
                                               u32x4 (&bfr)[C::KSTEPS][C::TN]) const {
        constexpr int NA = C::KSTEPS * C::TM;
        if (r < NA) {
            const int s = r / C::TM, i = r % C::TM;
            af[s][i] = read_a(stage, s, i);
        } else if constexpr (C::DT == DT_F32) {
            const int q = r - NA;
            const int s = q / (4 * C::TN), j = (q / 4) % C::TN, e = q % 4;
            bfr[s][j][e] = read_b32(stage, s, j, e);
        } else {
            const int q = r - NA;
            const int s = q / (2 * C::TN), j = (q / 2) % C::TN, half = q % 2;
            const u32x2 w2 = read_b(stage, s, j, half);
            if (half == 0) {
                bfr[s][j].x = w2.x;
                bfr[s][j].y = w2.y;
            } else {
                bfr[s][j].z = w2.x;
                bfr[s][j].w = w2.y;
            }
        }
    }

    // the MFMAs of one read step: MFMA step e outermost, so an accumulator's
    // consecutive MFMAs are TM x TN apart
    template <bool FIRST>
    __device__ __forceinline__ void mfmas(const u32x4 (&af)[C::TM], const u32x4 (&bfr)[C::TN]) {
        static_for<0, C::MFMA_PER_READ * C::TM * C::TN, 1>([&](auto qc) {
            constexpr int q = decltype(qc)::value;
            constexpr int e = q / (C::TM * C::TN), i = (q / C::TN) % C::TM, j = q % C::TN;
            if constexpr (FIRST && e == 0) acc.template mma<true>(i, j, af[i], bfr[j], e);
            else acc.template mma<false>(i, j, af[i], bfr[j], e);
        });
    }

    // the MFMAs of LDS copy `stage`; FIRST: the block's first K tile
    template <bool FIRST>
    __device__ __forceinline__ void compute(int stage) {
#pragma unroll
        for (int s = 0; s < C::KSTEPS; ++s) {
            u32x4 af[C::TM], bfr[C::TN];
            read_frags(stage, s, af, bfr);
            if (FIRST && s == 0) mfmas<true>(af, bfr);
            else mfmas<false>(af, bfr);
        }
    }
};

// Values per store-back chunk (the C0 loads of a chunk go out together): up
// to 64 for 16x16 tiles, whose accumulators sit in AGPRs; up to 32 for 32x32
// tiles, whose 64 accumulators per lane share the VGPRs with the chunk's
// offsets and C0 values (a chunk of 64 took the 128 x 128 kernel past 256
// registers, into scratch); up to 16 with the fused tail.  The chunk is a
// whole number of MFMA tiles that divides the wave's tiles (45 for the
// 288 x 160 tile: 15 per chunk, 5 with the tail).
template <class C, bool TAIL>
constexpr int chunk_values() {
    const int cap = (TAIL ? 16 : (C::MT == 32 ? 32 : 64)) / C::ACC_PER_MFMA;
    int ch = cap < C::TM * C::TN ? cap : C::TM * C::TN;
    while ((C::TM * C::TN) % ch) --ch;
    return ch * C::ACC_PER_MFMA;
}

// SCHED_RING (all waves in step): iteration kt waits for tile kt, one
// barrier (tile kt visible, copy of tile kt-1 released), issues tile
// kt + STAGES - 1, multiplies tile kt.  STAGES == 1 is the unpipelined form.
template <class C, int STAGES, int SWZ, bool FRINGE, bool TAIL = false, bool LIMIT = FRINGE>
__device__ __forceinline__ void ring_tile(const GemmParams &p, char *smem, int64_t b, int64_t tm, int64_t tn) {
    RingBlock<C, STAGES, SWZ, FRINGE, LIMIT> blk(p, smem, b, tm, tn);
    const int64_t nk = blk.nk, ndma = blk.ndma;
    if (nk > 0) {
        blk.tail_load();
        if (STAGES == 1) {
            for (int64_t kt = 0; kt < nk; ++kt) {
                if (kt > 0) {
                    wait_lds();
                    block_barrier();        // every wave is done reading the single copy
                }
                if (kt < ndma) blk.dma(kt, 0);
                blk.template land_tile<0>(kt, 0);
                block_barrier();            // tile kt is in LDS for every wave
                if (kt == 0) blk.template compute<true>(0);
                else blk.template compute<false>(0);
            }
        } else {
#pragma unroll
            for (int t = 0; t < STAGES - 1; ++t)
                if (t < ndma) blk.dma(t, t);
            int cur = 0, nxt = STAGES - 1;   // LDS copies of tile kt and of tile kt + STAGES - 1
            for (int64_t kt = 0; kt < nk; ++kt) {
                blk.template land_tile<STAGES - 2>(kt, cur);
                block_barrier();            // tile kt visible; copy of tile kt-1 released
                const int64_t t = kt + STAGES - 1;
                if (t < ndma) blk.dma(t, nxt);
                if (kt == 0) blk.template compute<true>(cur);
                else blk.template compute<false>(cur);
                cur = cur + 1 == STAGES ? 0 : cur + 1;
                nxt = nxt + 1 == STAGES ? 0 : nxt + 1;
            }
        }
        blk.acc.settle();
    }
    auto get = [&](int i, int j, int v) { return blk.acc.get(i, j, v); };
    store_tile_epilogue<C, FRINGE, decltype(get), chunk_values<C, TAIL>(), TAIL>(p, get, b, blk.m0, blk.n0, blk.wave,
                                                                                blk.lane);
}

// SCHED_SWPIPE (software pipeline, one wave per SIMD, large wave tiles): the
// fragments of a whole K tile live in registers, double-buffered.  Iteration
// t: land tile t + 1 (this wave's copies of it) and wait for tile t's
// fragments; one barrier (tile t + 1 is visible to every wave and nobody reads
// tile t's LDS copy any more); then the MFMAs of tile t, with the fragment
// reads of tile t + 1 and the copies of tile t + STAGES (into tile t's LDS
// copy) placed between them, so the matrix core is fed while LDS and the
// texture unit work.  Copies run STAGES - 1 tiles ahead of the tile being
// landed.
template <class C, int STAGES, int SWZ, bool FRINGE, bool LIMIT = FRINGE>
struct SwPipe {
    using Blk = RingBlock<C, STAGES, SWZ, FRINGE, LIMIT>;
    static constexpr int NMFMA = C::KSTEPS * C::MFMA_PER_READ * C::TM * C::TN;
    static constexpr int READS = Blk::READS;
    static_assert(READS <= NMFMA, "one fragment read per MFMA at most");

    // One iteration: multiply tile t from (fa, fb) while reading tile t + 1
    // into (na, nb).  STEADY: tile t + 1 exists and tile t + STAGES is copied
    // (no conditions inside the MFMA stream); otherwise both are checked.
    // READ = false (steady only): tile t + 1 is landed and published but its
    // fragments are left for the caller to read.
    template <bool STEADY, bool FIRST = false, bool READ = true>
    __device__ __forceinline__ static void iter(Blk &blk, int64_t t, int cur, int nxt_read,
                                                u32x4 (&fa)[C::KSTEPS][C::TM], u32x4 (&fb)[C::KSTEPS][C::TN],
                                                u32x4 (&na)[C::KSTEPS][C::TM], u32x4 (&nb)[C::KSTEPS][C::TN]) {
        const int64_t nk = blk.nk, ndma = blk.ndma;
        const bool more = STEADY || t + 1 < nk;
        if (STEADY) {
            // tile t + 1 is a copied tile with STAGES - 2 copied tiles issued after it
            wait_vmcnt<(STAGES - 2) * Blk::COPIES>();
            wait_lds();
        } else if (more) {
            blk.template land_tile<STAGES - 2>(t + 1, nxt_read);
        }
        wait_lds();
        __builtin_amdgcn_sched_barrier(0);
        block_barrier();
        __builtin_amdgcn_sched_barrier(0);
        const int64_t tc = t + STAGES;          // copy into tile t's LDS copy
        if (STEADY) {
            // a compile-time loop: every accumulator and fragment index is a
            // constant however long the stream (a loop the unroller declines
            // would index the accumulators at run time, i.e. in scratch)
            static_for<0, NMFMA, 1>([&](auto qc) {
                constexpr int q = decltype(qc)::value;
                constexpr int se = q / (C::TM * C::TN), i = (q / C::TN) % C::TM, j = q % C::TN;
                constexpr int s = se / C::MFMA_PER_READ, e = se % C::MFMA_PER_READ;
                if constexpr (FIRST && se == 0) blk.acc.template mma<true>(i, j, fa[s][i], fb[s][j], e);
                else blk.acc.template mma<false>(i, j, fa[s][i], fb[s][j], e);
                if constexpr (READ && q < READS) blk.read_piece(nxt_read, q, na, nb);
                if constexpr (q == NMFMA / 4 - 1 || q == 3 * NMFMA / 4 - 1)
                    blk.dma_operand(tc, cur, q < NMFMA / 2 ? 0 : 1);
                __builtin_amdgcn_sched_barrier(0);
            });
        } else {
            if (more) {
#pragma unroll
                for (int r = 0; r < READS; ++r) blk.read_piece(nxt_read, r, na, nb);
            }
            if (tc < ndma) blk.dma(tc, cur);
            static_for<0, NMFMA, 1>([&](auto qc) {
                constexpr int q = decltype(qc)::value;
                constexpr int se = q / (C::TM * C::TN), i = (q / C::TN) % C::TM, j = q % C::TN;
                constexpr int s = se / C::MFMA_PER_READ, e = se % C::MFMA_PER_READ;
                if constexpr (FIRST && se == 0) blk.acc.template mma<true>(i, j, fa[s][i], fb[s][j], e);
                else blk.acc.template mma<false>(i, j, fa[s][i], fb[s][j], e);
            });
        }
    }
};

template <class C, int STAGES, int SWZ, bool FRINGE, bool TAIL = false, bool LIMIT = FRINGE>
__device__ __forceinline__ void ring_tile_swpipe(const GemmParams &p, char *smem, int64_t b, int64_t tm, int64_t tn) {
    static_assert(STAGES >= 2, "software pipeline needs at least two LDS copies");
    using SP = SwPipe<C, STAGES, SWZ, FRINGE, LIMIT>;
    RingBlock<C, STAGES, SWZ, FRINGE, LIMIT> blk(p, smem, b, tm, tn);
    const int64_t nk = blk.nk, ndma = blk.ndma;
    if (nk > 0) {
        // With at most STAGES copied tiles the last tile is landed by the
        // prologue or the first iteration: load it first, before any copy.
        const bool early_tail = ndma <= STAGES;
        if (early_tail) blk.tail_load();
#pragma unroll
        for (int t = 0; t < STAGES; ++t)
            if (t < ndma) blk.dma(t, t);
        // tile 0: land, publish, read its fragments
        blk.template land_tile<STAGES - 1>(0, 0);
        __builtin_amdgcn_sched_barrier(0);
        block_barrier();
        __builtin_amdgcn_sched_barrier(0);
        u32x4 a0[C::KSTEPS][C::TM], b0[C::KSTEPS][C::TN], a1[C::KSTEPS][C::TM], b1[C::KSTEPS][C::TN];
#pragma unroll
        for (int r = 0; r < SP::READS; ++r) blk.read_piece(0, r, a0, b0);
        auto adv = [](int x) { return x + 1 == STAGES ? 0 : x + 1; };
        // tile 0, whose MFMAs start the accumulators; an iteration t is steady
        // when tile t + STAGES is copied (t + STAGES < ndma)
        if (STAGES < ndma) SP::template iter<true, true>(blk, 0, 0, 1, a0, b0, a1, b1);
        else SP::template iter<false, true>(blk, 0, 0, adv(0), a0, b0, a1, b1);
        int64_t t = 1;
        // steady state, four tiles per trip: tile t sits in LDS copy t % STAGES
        // (STAGES is 2 or 4) and the fragment buffers swap roles every tile, so
        // every copy index below is a constant
        static_assert(4 % STAGES == 0, "four tiles per trip cycle the LDS copies");
        for (; t + 3 + STAGES < ndma; t += 4) {
            SP::template iter<true>(blk, t, 1 % STAGES, 2 % STAGES, a1, b1, a0, b0);
            SP::template iter<true>(blk, t + 1, 2 % STAGES, 3 % STAGES, a0, b0, a1, b1);
            SP::template iter<true>(blk, t + 2, 3 % STAGES, 4 % STAGES, a1, b1, a0, b0);
            SP::template iter<true>(blk, t + 3, 4 % STAGES, 5 % STAGES, a0, b0, a1, b1);
        }
        int cur = (int)(t % STAGES);
        // drain.  With more than STAGES copied tiles the last K tile is landed
        // here (a steady iteration t lands tile t + 1 < ndma), so its register
        // loads are issued here rather than in the prologue and their
        // registers are not held through the steady state; they are younger
        // than some copies, which only makes the vmcnt waits of those copies
        // conservative (loads complete in issue order).
        if (!early_tail) blk.tail_load();
        for (; t + 1 < nk; t += 2) {
            const int c1 = adv(cur), c2 = adv(c1);
            SP::template iter<false>(blk, t, cur, c1, a1, b1, a0, b0);
            SP::template iter<false>(blk, t + 1, c1, c2, a0, b0, a1, b1);
            cur = c2;
        }
        if (t < nk) SP::template iter<false>(blk, t, cur, adv(cur), a1, b1, a0, b0);
        blk.acc.settle();
    }
    auto get = [&](int i, int j, int v) { return blk.acc.get(i, j, v); };
    store_tile_epilogue<C, FRINGE, decltype(get), chunk_values<C, TAIL>(), TAIL>(p, get, b, blk.m0, blk.n0, blk.wave,
                                                                                blk.lane);
}

// Persistent form of the software pipeline for a grid of interior tiles of
// one problem whose K is a multiple of 4 K tiles (at least 8): workgroup w
// takes tiles w, w + G, w + 2G, ... (G workgroups, a multiple of the 8 XCDs,
// so every id keeps its XCD and the XCDs' tile runs are those of the plain
// grid).  Every K tile is copied straight to LDS (K is whole tiles).  The
// pipeline does not stop between tiles: the last four iterations of a tile
// copy the next tile's K tiles 0..3 into LDS copies 0..3 (K tile t of any
// tile sits in copy t mod 4) and the last one lands and publishes K tile 0,
// so the next tile starts with its first copies in LDS.  Only its first
// fragments are read after the epilogue (holding them through it would take
// the epilogue's registers); no iteration but the last tile's drain leaves
// the steady form.
template <class C, int STAGES, int SWZ, bool TAIL = false>
__device__ __forceinline__ void ring_persistent(const GemmParams &p, char *smem) {
    static_assert(STAGES == 4, "four LDS copies: a tile's copies sit at t mod 4");
    using SP = SwPipe<C, STAGES, SWZ, false>;
    const uint32_t total = (uint32_t)(p.tiles_m * p.tiles_n);
    uint32_t v = blockIdx.x;
    int64_t b, tm, tn;
    block_coords_of(p, v, b, tm, tn);
    RingBlock<C, STAGES, SWZ, false> blk(p, smem, 0, tm, tn);
    blk.ndma = blk.nk;
    const int64_t nk = blk.nk;
#pragma unroll
    for (int t = 0; t < STAGES; ++t) blk.dma(t, t);
    blk.template land_tile<STAGES - 1>(0, 0);
    __builtin_amdgcn_sched_barrier(0);
    block_barrier();
    __builtin_amdgcn_sched_barrier(0);
    u32x4 a0[C::KSTEPS][C::TM], b0[C::KSTEPS][C::TN], a1[C::KSTEPS][C::TM], b1[C::KSTEPS][C::TN];
#pragma unroll
    for (int r = 0; r < SP::READS; ++r) blk.read_piece(0, r, a0, b0);
    while (true) {
        const uint32_t vn = v + gridDim.x;
        const bool next = vn < total;
        SP::template iter<true, true>(blk, 0, 0, 1, a0, b0, a1, b1);
        int64_t t = 1;
        for (; t + 3 + STAGES < nk; t += 4) {
            SP::template iter<true>(blk, t, 1, 2, a1, b1, a0, b0);
            SP::template iter<true>(blk, t + 1, 2, 3, a0, b0, a1, b1);
            SP::template iter<true>(blk, t + 2, 3, 0, a1, b1, a0, b0);
            SP::template iter<true>(blk, t + 3, 0, 1, a0, b0, a1, b1);
        }
        // t = nk - 7: seven K tiles left, in LDS copies 1, 2, 3, 0, 1, 2, 3.  The
        // last tile of a workgroup copies its own K tiles 0..3 again (unused), so
        // every tile ends the same way.
        int64_t bn, tmn = 0, tnn = 0;
        if (next) block_coords_of(p, vn, bn, tmn, tnn);
        else tmn = blk.m0 / C::BM, tnn = blk.n0 / C::BN;
        SP::template iter<true>(blk, t, 1, 2, a1, b1, a0, b0);           // copies K tile nk - 3
        SP::template iter<true>(blk, t + 1, 2, 3, a0, b0, a1, b1);       // nk - 2
        SP::template iter<true>(blk, t + 2, 3, 0, a1, b1, a0, b0);       // nk - 1
        blk.retarget(tmn, tnn);
        SP::template iter<true>(blk, t + 3, 0, 1, a0, b0, a1, b1);       // the next tile's 0
        SP::template iter<true>(blk, t + 4, 1, 2, a1, b1, a0, b0);       // its 1
        SP::template iter<true>(blk, t + 5, 2, 3, a0, b0, a1, b1);       // its 2
        SP::template iter<true, false, false>(blk, t + 6, 3, 0, a1, b1, a0, b0);   // its 3; lands its 0
        blk.acc.settle();
        auto get = [&](int i, int j, int v2) { return blk.acc.get(i, j, v2); };
        store_tile_epilogue<C, false, decltype(get), TAIL ? 16 : 64, TAIL>(p, get, 0, blk.m0, blk.n0, blk.wave, blk.lane);
        if (!next) break;
        blk.m0 = tmn * C::BM;
        blk.n0 = tnn * C::BN;
#pragma unroll
        for (int r = 0; r < SP::READS; ++r) blk.read_piece(0, r, a0, b0);
        // the epilogue's accumulator reads before the next tile's first MFMAs overwrite them
        blk.acc.settle();
        v = vn;
    }
    // the unused copies must land before the workgroup's LDS is released
    wait_vmcnt<0>();
}

// Two batch entries per workgroup on one ring, for batches of single-tile
// problems (each entry one fringe block) of more than one round and at most
// two: workgroup w takes entry w, then entry w + G when it exists (G =
// gridDim.x).  The first entry's last iterations copy the second entry's first
// K tiles into the LDS copies its own last tiles release, so the second starts
// with them landed or in flight while the first stores C, where a fresh
// workgroup of the plain grid starts cold.  Each entry's MFMA sequence is the
// plain ring's, so the result is bitwise the plain grid's.  The entries are
// straight-line code: a loop over entries kept neither the accumulators nor
// the copy state in registers.  The waits count copies only; loads and stores
// share one in-order completion count, so ignoring the C stores and register
// loads issued after some copies only makes a wait longer than it must be.
template <class C, int STAGES, int SWZ, bool TAIL, bool NEXT>
__device__ __forceinline__ void chain_entry(const GemmParams &p, RingBlock<C, STAGES, SWZ, true, true> &blk,
                                            int64_t v, int64_t vn, int &cur, int &nxt) {
    using Blk = RingBlock<C, STAGES, SWZ, true, true>;
    static_assert(STAGES == 4, "waits written for four LDS copies");
    const int64_t nk = blk.nk, ndma = blk.ndma;
    // copy tiles in issue order: this entry's 0 .. ndma - 1 (its last K tile goes
    // through registers), then the next entry's, numbered from nk
    auto copied = [&](int64_t g) { return g < ndma || (NEXT && g >= nk); };
    for (int64_t kt = 0; kt < nk; ++kt) {
        if (kt < ndma) {
            const int later = (copied(kt + 1) ? 1 : 0) + (copied(kt + 2) ? 1 : 0);
            if (later >= 2) wait_vmcnt<2 * Blk::COPIES>();
            else if (later == 1) wait_vmcnt<Blk::COPIES>();
            else wait_vmcnt<0>();
        } else {
            // the register tail is older than the next entry's two copies issued so far
            if (NEXT) wait_vmcnt<2 * Blk::COPIES>();
            else wait_vmcnt<0>();
            blk.tail_store(cur);
        }
        wait_lds();
        block_barrier();            // tile kt visible; the copy of tile kt - 1 released
        const int64_t g = kt + STAGES - 1;
        if (g < ndma) {
            blk.dma(g, nxt);
        } else if (NEXT && g >= nk) {
            if (g == nk) {          // this entry's copies are all issued: point the copies at the next
                blk.b = vn;
                blk.Ablk = p.A + vn * p.sA * C::ELEM;
                blk.Bblk = p.B + vn * p.sB * C::ELEM;
                blk.a_base = uniform_u64((uint64_t)blk.Ablk);
                blk.b_base = uniform_u64((uint64_t)blk.Bblk);
            }
            blk.dma(g - nk, nxt);
        }
        if (kt == 0) blk.template compute<true>(cur);
        else blk.template compute<false>(cur);
        cur = cur + 1 == STAGES ? 0 : cur + 1;
        nxt = nxt + 1 == STAGES ? 0 : nxt + 1;
    }
    blk.acc.settle();
    auto get = [&](int i, int j, int w) { return blk.acc.get(i, j, w); };
    store_tile_epilogue<C, true, decltype(get), chunk_values<C, TAIL>(), TAIL>(p, get, v, 0, 0, blk.wave, blk.lane);
}

// The host launches it for the 288 x 160 tile with G < batch <= 2 G and at
// least STAGES K tiles per entry.
template <class C, int STAGES, int SWZ, bool TAIL = false>
__global__ __launch_bounds__(C::THREADS, C::OCCUPANCY) void gemm_ring_chain_kernel(GemmParams p) {
    __shared__ __attribute__((aligned(1024))) char smem[STAGES * ring_stage_bytes<C, SWZ>()];
    const int64_t v = blockIdx.x, vn = v + gridDim.x;
    RingBlock<C, STAGES, SWZ, true, true> blk(p, smem, v, 0, 0);
    blk.tail_load();
#pragma unroll
    for (int t = 0; t < STAGES - 1; ++t) blk.dma(t, t);
    int cur = 0, nxt = STAGES - 1;
    if (vn < p.batch) {
        chain_entry<C, STAGES, SWZ, TAIL, true>(p, blk, v, vn, cur, nxt);
        blk.acc.settle();       // the store-back's accumulator reads before the next entry's first MFMAs
        blk.tail_load();
        chain_entry<C, STAGES, SWZ, TAIL, false>(p, blk, vn, vn, cur, nxt);
    } else {
        chain_entry<C, STAGES, SWZ, TAIL, false>(p, blk, v, v, cur, nxt);
    }
}

template <class C, int STAGES, int SWZ, bool TAIL = false>
__global__ __launch_bounds__(C::THREADS, C::OCCUPANCY) void gemm_ring_persistent_kernel(GemmParams p) {
    __shared__ __attribute__((aligned(1024))) char smem[STAGES * ring_stage_bytes<C, SWZ>()];
    ring_persistent<C, STAGES, SWZ, TAIL>(p, smem);
}

// The problem of grid batch entry b with its batch offsets folded into the
// pointers; for a split-K pass, its K slice, written unscaled to its fp32
// partial.  E: bytes per input element.
template <int E>
__device__ __forceinline__ GemmParams entry_params(const GemmParams &p, int64_t b) {
    GemmParams q = p;
    if (p.splits > 1) {
        const int64_t s = b / p.problems, pb = b - s * p.problems;
        const int64_t k0 = s * p.k_slice;
        q.A = p.A + (pb * p.sA + k0) * E;
        q.B = p.B + (pb * p.sB + k0 * p.ldb) * E;
        q.K = p.K - k0 < p.k_slice ? p.K - k0 : p.k_slice;
        q.C = p.W + b * p.M * p.N;
        q.ldc = p.N;
        q.alpha = 1.0f;
        q.beta = 0.0f;
        q.bias_mode = 0;        // the tail belongs to the combine pass
        q.act = 0;
    } else {
        q.A = p.A + b * p.sA * E;
        q.B = p.B + b * p.sB * E;
        q.C = p.C + b * p.sC;
        if (p.bias_mode != 0) q.bias = p.bias + b * p.bias_stride;   // the epilogue then sees entry 0
    }
    return q;
}

// A strip block's K slice (strip_splits > 1): its k range, and C pointed at the
// slice's partial of the strip region so that the strip's own (m0, n0)
// addressing lands there (row stride: the region's width).
template <int E>
__device__ __forceinline__ GemmParams strip_slice_params(const GemmParams &p, GemmParams q, int64_t b,
                                                         int64_t slice, bool n_strip) {
    const int64_t k0 = slice * p.strip_k_slice;
    q.A = q.A + k0 * E;
    q.B = q.B + k0 * q.ldb * E;
    q.K = p.K - k0 < p.strip_k_slice ? p.K - k0 : p.strip_k_slice;
    q.alpha = 1.0f;
    q.beta = 0.0f;
    q.bias_mode = 0;
    q.act = 0;
    const int64_t wn = p.N - p.n_main, rows_n = p.strip_rows_n, rows_m = p.M - p.m_main;
    if (n_strip) {
        q.C = p.Ws + (slice * p.batch + b) * rows_n * wn - p.n_main;
        q.ldc = wn;
    } else {
        const int64_t n_region = p.strip_n ? p.strip_splits * p.batch * rows_n * wn : 0;
        q.C = p.Ws + n_region + (slice * p.batch + b) * rows_m * p.N - p.m_main * p.N;
        q.ldc = p.N;
    }
    return q;
}

template <class C, int STAGES, int SWZ, int SCHED, bool FRINGE, bool TAIL, bool LIMIT = FRINGE>
__device__ __forceinline__ void run_tile(const GemmParams &q, char *smem, int64_t tm, int64_t tn) {
    if constexpr (SCHED == SCHED_SWPIPE) ring_tile_swpipe<C, STAGES, SWZ, FRINGE, TAIL, LIMIT>(q, smem, 0, tm, tn);
    else ring_tile<C, STAGES, SWZ, FRINGE, TAIL, LIMIT>(q, smem, 0, tm, tn);
}

template <class C, int STAGES, int SWZ, int SCHED, bool TAIL = false>
__global__ __launch_bounds__(C::THREADS, C::OCCUPANCY) void gemm_ring_kernel(GemmParams p) {
    static_assert(STAGES >= 1 && STAGES <= 5, "1 to 5 LDS copies");
    static_assert(SCHED == SCHED_RING || SCHED == SCHED_SWPIPE, "schedule");
    __shared__ __attribute__((aligned(1024))) char smem[STAGES * ring_stage_bytes<C, SWZ>()];
    if constexpr (std::is_same<C, Ring256<C::DT>>::value) {
        // thin fringe strips (Partition: a narrow block for a narrow remainder)
        using SN = Strip256xN<C::DT>;
        using SM = StripMx256<C::DT>;
        static_assert(SN::THREADS == C::THREADS && SM::THREADS == C::THREADS, "one workgroup size");
        static_assert(ring_stage_bytes<SN, SWZ>() <= ring_stage_bytes<C, SWZ>() &&
                      ring_stage_bytes<SM, SWZ>() <= ring_stage_bytes<C, SWZ>(), "LDS");
        const int64_t main_blocks = p.tiles_m * p.tiles_n * p.batch;
        if ((int64_t)blockIdx.x >= main_blocks) {
            const int64_t per = p.strip_n + p.strip_m;
            int64_t s = (int64_t)blockIdx.x - main_blocks;
            const int64_t slice = s / (per * p.batch);       // 0 unless the strips are split along K
            s -= slice * per * p.batch;
            const int64_t b = s / per, r = s - b * per;
            GemmParams q = entry_params<C::ELEM>(p, b);
            if (p.strip_splits > 1) q = strip_slice_params<C::ELEM>(p, q, b, slice, r < p.strip_n);
            if (r < p.strip_n) run_tile<SN, STAGES, SWZ, SCHED, true, TAIL>(q, smem, r, p.n_main / SN::BN);
            else run_tile<SM, STAGES, SWZ, SCHED, true, TAIL>(q, smem, p.m_main / SM::BM, r - p.strip_n);
            return;
        }
    }
    int64_t b, tm, tn;
    block_coords(p, b, tm, tn);
    const GemmParams q = entry_params<C::ELEM>(p, b);
    const bool full_m = (tm + 1) * C::BM <= p.M, full_n = (tn + 1) * C::BN <= p.N;
    // A block past M only, or past N where N ends on a 16-byte chunk, masks its
    // rows and chunks and copies like an interior block (the per-copy limits
    // cost 3% of a 256 x 256 tile's time); only an N edge inside a chunk needs
    // them.  Only in the 256 x 256 kernels, and not in those with the fused tail,
    // the unpipelined depth or the pad_stride placement: a third tile body took
    // those into scratch, and the smaller tiles past the register count of the
    // workgroups per CU they are planned for.
    constexpr bool UNLIMITED_FRINGE =
        std::is_same<C, Ring256<C::DT>>::value && !TAIL && STAGES > 1 && SWZ != SWZ_PAD;
    if (full_m && full_n) run_tile<C, STAGES, SWZ, SCHED, false, TAIL>(q, smem, tm, tn);
    else if (UNLIMITED_FRINGE && (full_n || p.N % C::CHUNK == 0))
        run_tile<C, STAGES, SWZ, SCHED, true, TAIL, !UNLIMITED_FRINGE>(q, smem, tm, tn);
    else run_tile<C, STAGES, SWZ, SCHED, true, TAIL, true>(q, smem, tm, tn);
}

}  // namespace tg
