// tile_config.hpp -- compile-time tile configurations and the index maps the
// kernels use, as __host__ __device__ functions so the host can evaluate
// exactly what the device computes.
//
// Vocabulary follows the OCANNL "Module Ir.Schedule" page: a block tile is a
// Split of the M and N loops, the K loop is Split by BK and Staged through a
// workgroup-shared tile with an XOR swizzle, the per-wave register tile is the
// materialised Unroll of the MFMA loop nest (register blocktiling), and the
// accumulator is Privatized into registers.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define TG_HD __host__ __device__ __forceinline__
#else
#define TG_HD inline
#endif

namespace tg {

enum DType : int { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };

// One configuration of the kernel family.
//  * BK is chosen so one tile row is 128 bytes -- exactly one LDS bank line of
//    32 x 4-byte banks, the row width for which the TIRx "Tensor Layout" page
//    (Worked example; Choosing the parameters) shows an 8-row, 16-byte column
//    read is conflict-free under Swizzle(M, 3, 3).
//  * Both operands are staged k-contiguous: A as [BM][BK], B transposed as
//    [BN][BK], so every MFMA operand fragment is one 16-byte LDS read.
template <int DT_, int BM_, int BN_, int WAVES_M_, int WAVES_N_>
struct TileCfg {
    static constexpr int DT = DT_;
    static constexpr int ELEM = DT_ == DT_F32 ? 4 : 2;       // bytes per input element
    static constexpr int BM = BM_, BN = BN_;
    static constexpr int BK = 128 / ELEM;                    // 64 (16-bit) or 32 (fp32)
    static constexpr int CHUNK = 16 / ELEM;                  // elements per 16-byte chunk
    static constexpr int CPR = BK / CHUNK;                   // chunks per tile row (8)
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int WAVES = WAVES_M_ * WAVES_N_;
    static constexpr int THREADS = 64 * WAVES;
    // MFMA shape: 32x32x16 for bf16/fp16, 16x16x4 for fp32.
    static constexpr int MT = DT_ == DT_F32 ? 16 : 32;       // MFMA tile edge (rows = cols)
    static constexpr int ACC_PER_MFMA = MT * MT / 64;        // accumulators per lane per MFMA tile
    static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;   // wave tile
    static constexpr int TM = WTM / MT, TN = WTN / MT;       // MFMA tiles per wave
    static constexpr int LANE_GROUPS = 64 / MT;              // lanes sharing a row: 2 or 4
    static constexpr int KSTEPS = CPR / LANE_GROUPS;         // fragment reads per K tile
    // Global -> LDS copy: the first half of the threads copy A, the second B.
    static constexpr int LOADERS = THREADS / 2;
    static constexpr int A_CHUNKS = BM * CPR;                // 16-byte chunks in an A tile
    static constexpr int A_PER_THREAD = A_CHUNKS / LOADERS;
    static constexpr int B_UNITS = (BK / CHUNK) * (BN / CHUNK);   // CHUNK x CHUNK squares
    static constexpr int B_PER_THREAD = B_UNITS / LOADERS;
    static constexpr int A_TILE_BYTES = BM * BK * ELEM;
    static constexpr int B_TILE_BYTES = BN * BK * ELEM;
    static constexpr int STAGE_BYTES = A_TILE_BYTES + B_TILE_BYTES;

    static_assert(BM % (WAVES_M * MT) == 0 && BN % (WAVES_N * MT) == 0, "wave tiling");
    static_assert(CPR == 8, "tile rows are one 128-byte bank line");
    static_assert(A_CHUNKS % LOADERS == 0 && A_PER_THREAD >= 1, "A copy split");
    static_assert(B_UNITS % LOADERS == 0 && B_PER_THREAD >= 1, "B copy split");
};

// The fp32 configuration (id TG_CFG_F32_64x64 in tile_gemm.h); the 16-bit
// configurations are the RingCfg family below.
using CfgF32 = TileCfg<DT_F32, 64, 64, 2, 2>;                  // 4 waves, wave tile 32 x 32 (16x16 MFMA)

// LDS placement of a staged tile (the swizzle codes of tg_options): 1 none (row-major),
// 2 pad_stride (row-major with a padded row pitch), 3 XOR swizzle.
enum Swz : int { SWZ_NONE = 1, SWZ_PAD = 2, SWZ_XOR = 3 };

// ---------------------------------------------------------------------------
// LDS placement of one operand tile (rows x BK, k contiguous).
//
// The tile layout S[(rows, BK):(BK@m, 1@m)] gives the row-major element
// address m = row*BK + k, which two swizzles of the TIRx page then permute,
//     addr(m) = f(m >> M) * 2^M + (m mod 2^M),  f(x) = x ^ ((x & ((2^B-1) << S)) >> S),
// first (B, S) = (3, 3), then (B, S) = (2, 6), with M = log2(elements per 16
// bytes) (3 for 16-bit, 2 for fp32).  With 8 chunks per 128-byte row this
// XORs  (row & 7) ^ ((row >> 3) & 3)  into the chunk index: a per-row bijection
// of 16-byte units (the Swizzle_b128 flavour of the OCANNL Stage paragraph),
// so every 16-byte fragment stays contiguous.
//
// Why two: the page's single Swizzle(M, 3, 3) makes any 8 consecutive rows hit
// 8 distinct 16-byte bank groups of a 128-byte line (32 banks x 4 bytes), which
// is what a 128-bit LDS write needs on gfx950 (8 lanes per cycle).  A 128-bit
// LDS read is served 16 lanes per cycle from 64 banks (a 256-byte line, two
// tile rows), so 16 consecutive rows at one chunk index must also be distinct
// among the rows of equal parity; the second term makes them so.  The mask uses
// row bits 0..4 only, so for every fragment read and copy it is a function of
// the lane alone (row offsets of 32 leave it unchanged).
// ---------------------------------------------------------------------------
TG_HD int64_t swizzle_apply(int64_t m, int M, int B, int S) {
    int64_t x = m >> M;
    int64_t f = x ^ ((x & (((int64_t(1) << B) - 1) << S)) >> S);
    return (f << M) + (m & ((int64_t(1) << M) - 1));
}

TG_HD int swizzle_row_mask(int row) { return (row & 7) ^ ((row >> 3) & 3); }

template <class C>
TG_HD int lds_elem(int row, int k, int swz) {
    int m = row * C::BK + k;
    if (swz != SWZ_XOR) return m;
    constexpr int M = C::ELEM == 2 ? 3 : 2;
    return (int)swizzle_apply(swizzle_apply(m, M, 3, 3), M, 2, 6);
}

// Byte offset of 16-byte chunk `chunk` of tile row `row` (the unit every
// LDS write and fragment read moves).
template <class C>
TG_HD int lds_chunk_byte(int row, int chunk, int swz) {
    int c = swz != SWZ_XOR ? chunk : (chunk ^ swizzle_row_mask(row));
    return (row * C::CPR + c) * 16;
}

// ---------------------------------------------------------------------------
// The 16-bit kernel family: a K ring of STAGES LDS copies filled by direct
// global -> LDS copies (no staging registers), BK = 32.
//
//  * A tile [BM][32] (64-byte rows, k contiguous) under Swizzle(3, 2, 4) (the
//    16-byte chunk index of row r XORed with (r >> 2) & 3) for 32x32x16 MFMAs,
//    Swizzle(3, 2, 3) ((r >> 1) & 3) for 16x16x32: the choice that measured
//    conflict-free for that MFMA's fragment reads (ring_a_mask).
//  * B tile [32][BN] (k rows, n contiguous) under Swizzle(5, B, S) on 64-byte
//    units (32 elements): the unit index w of row k is XORed with k & 3 when a
//    row has >= 4 units, with (k >> 1) & 1 when it has 2.  B is read with the
//    transposing ds_read_b64_tr_b16: 32 lanes per cycle read 4 consecutive k
//    rows x 64 bytes, which the XOR spreads over the four 64-byte quarters of
//    the bank line.
//  * Copies: each DMA instruction fills 1 KiB of LDS, lane l writing bytes
//    16l..16l+15; the swizzle is realised by choosing each lane's source.
//  * MFMA shape MT_: 32 (32x32x16, two K steps per tile) or 16 (16x16x32, one
//    K step per tile).  With 16x16x32 the four 16-lane groups of a B read take
//    k rows 8g.. of the same 16 columns, so groups 0 and 1 (read in one cycle)
//    touch rows k and k + 8; a second swizzle term XORs the 32-byte half of
//    each 64-byte unit with (k >> 3) & 1 to keep them on distinct banks.
//  * fp32 inputs (DT_F32, 16x16x4 MFMAs only): the same 64-byte A rows hold a
//    K tile of 16, so the A tile, its swizzle and its ds_read_b128 fragment
//    reads are those of the 16-bit 16x16x32 kernel byte for byte; lane l's
//    chunk holds k 4 (l / 16) .. + 3 and its element e feeds MFMA step e, which
//    thus sums k = 4 g + e over the lane groups g.  B rows are BN fp32 (64-byte
//    units of 16 n); the partner of that A element, B[4 g + e][n], is one
//    ds_read_b32 per step (no 32-bit transposing read exists), and the unit
//    XOR (k >> 2) & 3 puts the four lane groups' rows on four distinct
//    16-bank quarters of the bank line.
// ---------------------------------------------------------------------------
template <int DT_, int BM_, int BN_, int WAVES_M_, int WAVES_N_, int MT_ = 32>
struct RingCfg {
    static constexpr int DT = DT_;
    static constexpr int ELEM = DT_ == DT_F32 ? 4 : 2;       // bytes per input element
    static constexpr int BM = BM_, BN = BN_, BK = 64 / ELEM;  // K tile: 64-byte A rows (32 or 16 k)
    static constexpr int CHUNK = 16 / ELEM;                  // elements per 16 bytes
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int WAVES = WAVES_M_ * WAVES_N_;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int MT = MT_, ACC_PER_MFMA = MT_ * MT_ / 64;
    // k per MFMA: 16 (32x32x16), 32 (16x16x32) or 4 (fp32 16x16x4)
    static constexpr int MK = DT_ == DT_F32 ? 4 : 512 / MT_;
    static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    static constexpr int TM = WTM / MT, TN = WTN / MT;
    // MFMAs per (row tile, column tile) per fragment read (the fp32 chunk's 4 k)
    static constexpr int MFMA_PER_READ = DT_ == DT_F32 ? 4 : 1;
    // fragment read steps per K tile (one 16-byte A chunk per lane each)
    static constexpr int KSTEPS = BK / (MK * MFMA_PER_READ);
    // B reads per column tile and read step: two transposing 8-byte reads
    // (16-bit), four 4-byte reads (fp32, one per MFMA step)
    static constexpr int B_PIECES = DT_ == DT_F32 ? 4 : 2;
    static constexpr int A_ROW_BYTES = BK * ELEM;            // 64
    static constexpr int B_ROW_BYTES = BN * ELEM;
    static constexpr int B_UNITS = B_ROW_BYTES / 64;         // 64-byte units per B row
    static constexpr int A_TILE_BYTES = BM * A_ROW_BYTES;
    static constexpr int B_TILE_BYTES = BK * B_ROW_BYTES;
    static constexpr int STAGE_BYTES = A_TILE_BYTES + B_TILE_BYTES;
    // acc_coord() below is shared with TileCfg
    static constexpr int LANE_GROUPS = 64 / MT_;             // lanes sharing a row: 2 or 4
    static constexpr bool B_HALF_SWZ = MT_ == 16 && DT_ != DT_F32;   // (k >> 3) & 1 into the 32-byte half
    // Workgroups per CU the kernel is compiled for (its register budget): the
    // 256 x 256 tile takes a whole CU (512 registers per lane, 128 KiB of
    // LDS); the smaller tiles leave room for two, which memory-bound problems
    // need for the bytes in flight.  (A budget of four for the 64 x 64 tile
    // was never met: its software pipeline needs more than 128 registers, so
    // it ran two per CU anyway and spilled on the way; mid-size problems
    // measured the same either way.)
    // The rule: more than 128 accumulators per lane (256 for 256 x 256, 180 for
    // 288 x 160) take a whole CU; a tile sized by area alone compiled the
    // 288 x 160 kernel at depth 2 for two per CU and spilled accumulators.
    static constexpr int OCCUPANCY = WTM * WTN / 64 > 128 ? 1 : 2;

    static_assert(BM % (WAVES_M * MT) == 0 && BN % (WAVES_N * MT) == 0, "wave tiling");
    static_assert(B_ROW_BYTES % 64 == 0, "B rows of whole 64-byte units");
    static_assert(DT_ == DT_F32 ? (MT_ == 16 && (B_UNITS == 4 || B_UNITS == 8 || B_UNITS == 16))
                                : (B_UNITS == 2 || B_UNITS == 4 || B_UNITS == 8 || (B_UNITS == 5 && MT_ == 16)),
                  "16-bit B rows of 2, 4 or 8 units (XOR of the unit index) or of 5 (half XOR only); "
                  "fp32: 16x16x4 MFMAs, B rows of 4, 8 or 16 units");

};

template <int DT> using Ring256 = RingCfg<DT, 256, 256, 2, 2, 16>;      // 4 waves, wave tile 128 x 128, 16x16x32
template <int DT> using Ring256m32 = RingCfg<DT, 256, 256, 2, 2, 32>;   // the same with 32x32x16 MFMAs
// Thin fringe strips of the 256 x 256 configuration (4 waves, wave tile 64 x 64):
// a 256 x 64 block for a ragged N tail of at most 64 columns, a 64 x 256 block
// for a ragged M tail of at most 64 rows.
template <int DT> using Strip256xN = RingCfg<DT, 256, 64, 4, 1, 16>;
template <int DT> using StripMx256 = RingCfg<DT, 64, 256, 1, 4, 16>;
template <int DT> using Ring128 = RingCfg<DT, 128, 128, 2, 2>;   // 4 waves, wave tile 64 x 64
template <int DT> using Ring64 = RingCfg<DT, 64, 64, 1, 2>;      // 2 waves, wave tile 64 x 32
// One workgroup per small problem: a 288 x 160 tile (18 x 10 MFMA tiles of 16 x 16; 4 waves,
// wave tile 144 x 80) covers a whole problem of up to 288 x 160, e.g. 257 x 129 in one block
// with no strip and no second tile, so A and B are each read once.
template <int DT> using Ring288x160 = RingCfg<DT, 288, 160, 2, 2, 16>;
// fp32 inputs on the ring (16x16x4 MFMAs, K tile 16): the 256 x 256 tile (its
// strips as above) and the 128 x 128 tile, 4 waves each.
using RingF32_256 = RingCfg<DT_F32, 256, 256, 2, 2, 16>;
using RingF32_128 = RingCfg<DT_F32, 128, 128, 2, 2, 16>;

// A tile: the XOR applied to the 16-byte chunk index of row r.  Which row
// bits make the fragment reads conflict-free depends on the MFMA lane pattern
// and was measured on gfx950 (SQ_LDS_BANK_CONFLICT of ds_read_b128 over every
// candidate): (r >> 2) & 3 for the 32x32x16 pattern (lane l: row l % 32,
// chunk l / 32), (r >> 1) & 3 for the 16x16x32 pattern (row l % 16, chunk
// l / 16); the other choice costs one extra cycle in two.
template <class C>
TG_HD int ring_a_mask(int r, int swz) {
    if (swz != SWZ_XOR) return 0;
    return C::MT == 32 ? ((r >> 2) & 3) : ((r >> 1) & 3);
}

// pad_stride placement (OCANNL "Module Ir.Schedule", Stage paragraph, pad_stride):
// the tile's minor dimension is rounded up by one 16-byte unit -- A rows of 32 k
// to a pitch of 40 elements (80 bytes), B rows of BN n to BN + 8 -- which changes
// the row stride while the iterated extents stay as they are; the padded slots
// are never read.  A pitch that stays a multiple of 16 bytes keeps every
// 16-byte chunk of a row contiguous, as the copies and fragment reads need.
// With an 80-byte A pitch, 16 consecutive rows start on 16 distinct 4-bank
// groups of the 64 banks (row r at bank 20 r mod 64).  No row pitch makes the
// transposing B read conflict-free: it reads rows k and k + 8 in one cycle, and
// a linear pitch that separates rows k .. k + 3 maps k + 8 onto k's banks or
// half-overlaps them; +16 bytes leaves two-way conflicts (the XOR has none).
template <class C>
TG_HD constexpr int ring_a_pitch(int swz) { return C::A_ROW_BYTES + (swz == SWZ_PAD ? 16 : 0); }
template <class C>
TG_HD constexpr int ring_b_pitch(int swz) { return C::B_ROW_BYTES + (swz == SWZ_PAD ? 16 : 0); }

// A tile: byte offset of logical chunk c (0..3) of row r.
template <class C>
TG_HD int ring_a_byte(int r, int c, int swz) {
    return r * ring_a_pitch<C>(swz) + 16 * (c ^ ring_a_mask<C>(r, swz));
}

// B tile: the XOR applied to the 64-byte unit index of k row k.
//  * rows of 4 or 8 units: k & 3;
//  * rows of 2 units (128 bytes, two rows per 256-byte bank line): (k >> 1) & 1
//    for 32x32x16; (k >> 3) & 1 for 16x16x32, whose reads pair rows k and
//    k + 8 (the half swizzle below then takes (k >> 1) & 1).
template <class C>
TG_HD int ring_b_mask(int k, int swz) {
    if (swz != SWZ_XOR) return 0;
    // fp32: a B read takes rows 4 g + e of the four lane groups g (one MFMA step
    // e): XOR (k >> 2) & 3 = g moves group g's 16 columns to bank quarter g
    if (C::ELEM == 4) return (k >> 2) & 3;
    // 5 units (320-byte rows): rows k .. k + 3 already start 16 banks apart; the
    // half XOR below separates k from k + 8
    if (C::B_UNITS == 5) return 0;
    if (C::B_UNITS >= 4) return k & 3;
    return C::MT == 32 ? ((k >> 1) & 1) : ((k >> 3) & 1);
}

// B tile: the XOR applied to the 32-byte half of a 64-byte unit of k row k
// (16x16x32 only): with the unit XOR, the 16-column segments of the eight rows
// one B read pairs (k0..k0+3 and k0+8..k0+11) land on eight distinct 32-byte
// quarters of a bank line.
template <class C>
TG_HD int ring_b_half_mask(int k, int swz) {
    if (!C::B_HALF_SWZ || swz != SWZ_XOR) return 0;
    return C::B_UNITS >= 4 ? ((k >> 3) & 1) : ((k >> 1) & 1);
}

// B tile: byte offset of element (k, n).
template <class C>
TG_HD int ring_b_byte(int k, int n, int swz) {
    if (C::ELEM == 4) return k * ring_b_pitch<C>(swz) + 64 * ((n / 16) ^ ring_b_mask<C>(k, swz)) + 4 * (n % 16);
    const int w = n / 32, half = ((n % 32) / 16) ^ ring_b_half_mask<C>(k, swz), in_half = (n % 16) * 2;
    return k * ring_b_pitch<C>(swz) + 64 * (w ^ ring_b_mask<C>(k, swz)) + 32 * half + in_half;
}

// The copies of one operand tile (OP 0 = A, 1 = B) into one LDS pipeline copy:
// the tile's rows x pitch bytes in 1 KiB blocks, each filled by one copy
// instruction (lane l writes bytes 16 l .. 16 l + 15 of its block).  Wave w
// copies the Q adjacent blocks w * Q .. w * Q + Q - 1, so they share one LDS
// base and differ only by an immediate offset.  When the blocks do not divide
// evenly among the waves (a padded pitch, a tile of 18 or 10 KiB), the SHARED
// blocks left over are copied once more each by every wave w, block
// Q * WAVES + w % SHARED: a block copied by several waves gets the same source
// bytes at the same LDS bytes from each, so the concurrent writes agree.
template <class C, int SWZ, int OP>
struct RingCopy {
    static constexpr int PITCH = OP == 0 ? ring_a_pitch<C>(SWZ) : ring_b_pitch<C>(SWZ);
    static constexpr int ROWS = OP == 0 ? C::BM : C::BK;
    static constexpr int ROW_BYTES = OP == 0 ? C::A_ROW_BYTES : C::B_ROW_BYTES;   // valid bytes per row
    static constexpr int NB = (ROWS * PITCH + 1023) / 1024;     // 1 KiB blocks
    static constexpr int Q = NB / C::WAVES;                      // blocks of a wave's own run
    static constexpr int SHARED = NB - Q * C::WAVES;             // blocks left over (< WAVES)
    static constexpr int PER = Q + (SHARED ? 1 : 0);             // copies per wave per K tile
    static constexpr int REGION = NB * 1024;                     // LDS bytes per pipeline copy
    static constexpr int GMAX = Q < 4 ? Q : 4;                   // copies under one M0 value at most
    static_assert(Q >= 1 && Q <= 8, "copy split");
    // the block copy d of wave `wave` fills
    TG_HD static constexpr int block(int d, int wave) {
        return d < Q ? wave * Q + d : Q * C::WAVES + (SHARED ? wave % SHARED : 0);
    }
    // copy d's position within its group of adjacent copies (groups of at most four)
    TG_HD static constexpr int pos(int d) { return d < Q ? d % 4 : 0; }
};

// The A element (row, first k of the chunk) lane l of block J must fetch;
// false for a padded slot or a byte past the tile (fetched as zeros).
template <class C>
TG_HD bool ring_a_source(int J, int lane, int swz, int &row, int &k) {
    const int pitch = ring_a_pitch<C>(swz);
    const int byte = J * 1024 + 16 * lane;
    row = byte / pitch;
    const int p = (byte % pitch) / 16;
    if (row >= C::BM || 16 * p >= C::A_ROW_BYTES) {
        k = 0;
        return false;
    }
    k = C::CHUNK * (p ^ ring_a_mask<C>(row, swz));
    return true;
}

// The B element (k, first n of the chunk) lane l of block J must fetch; false
// for a padded slot or a byte past the tile.
template <class C>
TG_HD bool ring_b_source(int J, int lane, int swz, int &k, int &n) {
    const int pitch = ring_b_pitch<C>(swz);
    const int byte = J * 1024 + 16 * lane;
    k = byte / pitch;
    const int b = byte % pitch;
    if (k >= C::BK || b >= C::B_ROW_BYTES) {
        n = 0;
        return false;
    }
    const int w = (b / 64) ^ ring_b_mask<C>(k, swz);
    if (C::ELEM == 4) {
        n = 16 * w + (b % 64) / 4;
        return true;
    }
    const int half = ((b % 64) / 32) ^ ring_b_half_mask<C>(k, swz);
    n = 32 * w + 16 * half + (b % 32) / 2;
    return true;
}

// LDS bytes of one pipeline copy (A and B tiles) under a placement.
template <class C, int SWZ>
TG_HD constexpr int ring_stage_bytes() { return RingCopy<C, SWZ, 0>::REGION + RingCopy<C, SWZ, 1>::REGION; }

// ---------------------------------------------------------------------------
// MFMA register tiles.  Wave w owns the wave tile at
//   (w / WAVES_N) * WTM, (w % WAVES_N) * WTN
// split into TM x TN MFMA tiles; accumulator slot
//   s = (i * TN + j) * ACC_PER_MFMA + v
// of lane l holds element (row, col) of MFMA tile (i, j) with
//   32x32 (16-bit):  col = l % 32, row = 8 * (v / 4) + 4 * (l / 32) + v % 4
//   16x16 (fp32):    col = l % 16, row = 4 * (l / 16) + v
// ---------------------------------------------------------------------------
template <class C>
TG_HD void acc_coord(int wave, int lane, int slot, int &row, int &col) {
    int tile = slot / C::ACC_PER_MFMA, v = slot % C::ACC_PER_MFMA;
    int i = tile / C::TN, j = tile % C::TN;
    int r, c;
    if (C::MT == 32) {
        c = lane % 32;
        r = 8 * (v / 4) + 4 * (lane / 32) + v % 4;
    } else {
        c = lane % 16;
        r = 4 * (lane / 16) + v;
    }
    row = (wave / C::WAVES_N) * C::WTM + i * C::MT + r;
    col = (wave % C::WAVES_N) * C::WTN + j * C::MT + c;
}

// Fragment read: for K sub-step s, lane l reads 16-byte chunk
//   LANE_GROUPS * s + l / MT
// of tile row (wave row base + i*MT + l % MT).  For 16-bit inputs the chunk's
// 8 consecutive k are the lane's MFMA operand; for fp32 the chunk's 4 k feed 4
// consecutive 16x16x4 MFMAs (element e to MFMA e).  A and B lanes use the same
// k assignment, so every k of the tile meets its partner exactly once.
template <class C>
TG_HD int frag_chunk(int s, int lane) { return C::LANE_GROUPS * s + lane / C::MT; }

// Copy ownership of the A tile: loader thread t (0 <= t < LOADERS) copies
// chunks q = t + LOADERS * p, p < A_PER_THREAD, i.e. row q / 8, chunk q % 8:
// eight consecutive lanes cover one 128-byte row (a coalesced global read and
// eight distinct swizzled LDS slots).
template <class C>
TG_HD void copy_a_chunk(int t, int p, int &row, int &chunk) {
    int q = t + C::LOADERS * p;
    row = q / C::CPR;
    chunk = q % C::CPR;
}

// Copy ownership of the B tile: loader thread t copies the CHUNK x CHUNK
// square kb = u % 8, nb = u / 8 with u = t + LOADERS * p: CHUNK global rows of
// 16 bytes each, transposed in registers into CHUNK k-contiguous chunks (one
// per column n = nb*CHUNK + c), written to LDS row n, chunk kb.  Eight
// consecutive lanes take eight different kb, so their writes of one column
// index c land on eight distinct swizzled slots.
template <class C>
TG_HD void copy_b_unit(int t, int p, int &kb, int &nb) {
    int u = t + C::LOADERS * p;
    kb = u % C::CPR;
    nb = u / C::CPR;
}

}  // namespace tg
