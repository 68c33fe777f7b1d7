// layout.hip -- TileLayout / SwizzleLayout evaluation and the kernels' own
// placements described in that model (host code only).
//
// The model is the one of the Apache TVM TIRx "Tensor Layout" page: a layout
// maps a logical index to a SET of coordinates on named hardware axes,
// L(x) = { D(x) + r + O : r in R }, where D is the shard (a list of
// (extent, stride, axis) iters), R the replica iters and O a per-axis offset
// (TileLayout section), evaluated by flatten / split / accumulate + offset /
// broadcast (Forward mapping section).  A swizzle is a separate permutation of
// the memory-axis address composed after the tile layout (SwizzleLayout,
// ComposeLayout and The transform sections).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "tile_config.hpp"
#include "tile_gemm.h"

using namespace tg;

namespace {

bool layout_valid(const tg_layout *L) {
    if (!L || L->rank < 1 || L->rank > TG_LAYOUT_MAX_RANK) return false;
    if (L->n_shard < 1 || L->n_shard > TG_LAYOUT_MAX_ITERS) return false;
    if (L->n_replica < 0 || L->n_replica > TG_LAYOUT_MAX_ITERS) return false;
    int64_t size = 1, dsize = 1;
    for (int d = 0; d < L->rank; ++d) {
        if (L->shape[d] < 1) return false;
        size *= L->shape[d];
    }
    for (int k = 0; k < L->n_shard; ++k) {
        const tg_iter &it = L->shard[k];
        if (it.extent < 1 || it.axis < 0 || it.axis >= TG_AXIS_COUNT) return false;
        dsize *= it.extent;
    }
    for (int t = 0; t < L->n_replica; ++t) {
        const tg_iter &it = L->replica[t];
        if (it.extent < 1 || it.axis < 0 || it.axis >= TG_AXIS_COUNT) return false;
    }
    if (L->n_swizzle < 0 || L->n_swizzle > TG_LAYOUT_MAX_SWIZZLES) return false;
    for (int z = 0; z < L->n_swizzle; ++z) {
        const tg_swizzle &w = L->swizzle[z];
        if (w.m < 0 || w.b < 0 || w.s < w.b || w.m + w.s + w.b > 62) return false;
    }
    return size == dsize;   // a shape is admitted when its size equals the shard's
}

template <class C>
void describe_lds(tg_layout *L, int rows, int swz) {
    L->rank = 2;
    L->shape[0] = rows;
    L->shape[1] = C::BK;
    L->n_shard = 2;
    L->shard[0] = {rows, C::BK, TG_AXIS_M, 0};
    L->shard[1] = {C::BK, 1, TG_AXIS_M, 0};
    if (swz == SWZ_XOR) {
        const int32_t m = C::ELEM == 2 ? 3 : 2;
        L->n_swizzle = 2;
        L->swizzle[0] = {m, 3, 3};   // row bits 0..2 into the chunk index
        L->swizzle[1] = {m, 2, 6};   // row bits 3..4 into the chunk index
    }
}

template <class C>
void describe_acc(tg_layout *L) {
    L->rank = 2;
    L->shape[0] = C::BM;
    L->shape[1] = C::BN;
    int n = 0;
    auto push = [&](int64_t e, int64_t s, int ax) { L->shard[n++] = {e, s, ax, 0}; };
    if (C::MT == 32) {
        // row = ((wm*TM + i)*4 + r_hi)*8 + r_mid*4 + r_lo ; col = (wn*TN + j)*32 + c
        push(C::WAVES_M, C::WAVES_N, TG_AXIS_WAVE);
        push(C::TM, C::TN * C::ACC_PER_MFMA, TG_AXIS_M);
        push(4, 4, TG_AXIS_M);
        push(2, 32, TG_AXIS_LANE);
        push(4, 1, TG_AXIS_M);
        push(C::WAVES_N, 1, TG_AXIS_WAVE);
        push(C::TN, C::ACC_PER_MFMA, TG_AXIS_M);
        push(32, 1, TG_AXIS_LANE);
    } else {
        // row = ((wm*TM + i)*4 + g)*4 + v ; col = (wn*TN + j)*16 + c
        push(C::WAVES_M, C::WAVES_N, TG_AXIS_WAVE);
        push(C::TM, C::TN * C::ACC_PER_MFMA, TG_AXIS_M);
        push(4, 16, TG_AXIS_LANE);
        push(4, 1, TG_AXIS_M);
        push(C::WAVES_N, 1, TG_AXIS_WAVE);
        push(C::TN, C::ACC_PER_MFMA, TG_AXIS_M);
        push(16, 1, TG_AXIS_LANE);
    }
    L->n_shard = n;
}

template <class C>
void describe_copy_a(tg_layout *L) {
    // chunk q = row*8 + chunk = t + LOADERS*p, t = wave*64 + lane
    L->rank = 2;
    L->shape[0] = C::BM;
    L->shape[1] = C::CPR;
    L->n_shard = 3;
    L->shard[0] = {C::A_PER_THREAD, 1, TG_AXIS_M, 0};
    L->shard[1] = {C::LOADERS / 64, 1, TG_AXIS_WAVE, 0};
    L->shard[2] = {64, 1, TG_AXIS_LANE, 0};
}

template <class C>
tg_status describe(int swz, int kind, tg_layout *out) {
    switch (kind) {
        case TG_LAYOUT_LDS_A: describe_lds<C>(out, C::BM, swz); return TG_OK;
        case TG_LAYOUT_LDS_B: describe_lds<C>(out, C::BN, swz); return TG_OK;
        case TG_LAYOUT_ACC: describe_acc<C>(out); return TG_OK;
        case TG_LAYOUT_COPY_A: describe_copy_a<C>(out); return TG_OK;
    }
    return TG_ERR_INVALID_ARG;
}

constexpr int log2i(int x) { return x <= 1 ? 0 : 1 + log2i(x / 2); }

// The ring family: A [BM][BK] (64-byte rows) under Swizzle(3, 2, 4) or (M, 2, 3)
// with M = 3 for 16-bit, 2 for fp32 elements (the 16-byte chunk index); 16-bit
// B [32][BN] under Swizzle(5, B, S) on 64-byte units, fp32 B [16][BN] under
// Swizzle(4, 2, log2(units) + 2) (unit ^= (k >> 2) & 3); copies own physical
// 16-byte chunks.
template <class C>
void describe_ring_lds(tg_layout *L, int operand, int swz) {
    const int rows = operand == 0 ? C::BM : C::BK;
    const int cols = operand == 0 ? C::BK : C::BN;
    L->rank = 2;
    L->shape[0] = rows;
    L->shape[1] = cols;
    L->n_shard = 2;
    // pad_stride: the row stride is the padded pitch (in elements); no swizzle
    const int pitch = (operand == 0 ? ring_a_pitch<C>(swz) : ring_b_pitch<C>(swz)) / C::ELEM;
    L->shard[0] = {rows, pitch, TG_AXIS_M, 0};
    L->shard[1] = {cols, 1, TG_AXIS_M, 0};
    if (swz != SWZ_XOR) return;
    L->n_swizzle = 1;
    constexpr int CM = log2i(C::CHUNK);                     // element bits of a 16-byte chunk
    if (operand == 0) {
        if (C::MT == 32) L->swizzle[0] = {CM, 2, 4};        // chunk ^= (row >> 2) & 3
        else L->swizzle[0] = {CM, 2, 3};                    // chunk ^= (row >> 1) & 3
    } else if (C::ELEM == 4) {
        L->swizzle[0] = {4, 2, log2i(C::B_UNITS) + 2};      // 64-byte unit ^= (k >> 2) & 3
    } else if (C::B_UNITS >= 4) {
        L->swizzle[0] = {5, 2, C::B_UNITS == 8 ? 3 : 2};    // 64-byte unit ^= k & 3
        if (C::B_HALF_SWZ) {                                // 32-byte half ^= (k >> 3) & 1
            L->n_swizzle = 2;
            L->swizzle[1] = {4, 1, C::B_UNITS == 8 ? 7 : 6};
        }
    } else if (!C::B_HALF_SWZ) {
        L->swizzle[0] = {5, 1, 2};                          // 64-byte unit ^= (k >> 1) & 1
    } else {
        L->swizzle[0] = {5, 1, 4};                          // 64-byte unit ^= (k >> 3) & 1
        L->n_swizzle = 2;
        L->swizzle[1] = {4, 1, 3};                          // 32-byte half ^= (k >> 1) & 1
    }
}

template <class C>
void describe_ring_copy_a(tg_layout *L) {
    // physical chunk q = row*4 + p = (wave*A_DMA + d)*64 + lane
    L->rank = 2;
    L->shape[0] = C::BM;
    L->shape[1] = C::A_ROW_BYTES / 16;
    L->n_shard = 3;
    L->shard[0] = {C::WAVES, 1, TG_AXIS_WAVE, 0};
    L->shard[1] = {RingCopy<C, SWZ_XOR, 0>::Q, 1, TG_AXIS_M, 0};
    L->shard[2] = {64, 1, TG_AXIS_LANE, 0};
}

template <class C>
tg_status describe_ring(int swz, int kind, tg_layout *out) {
    // pad_stride is built for the 256 x 256 tile and its strips only; its copies
    // (padded slots, one block every wave copies) are not one shard layout
    if (swz == SWZ_PAD && (C::BM * C::BN < 256 * 64 || kind == TG_LAYOUT_COPY_A)) return TG_ERR_UNSUPPORTED;
    // 320-byte B rows (the 288 x 160 tile): the 32-byte half XOR of row k's bit 3
    // is not a swizzle of the linear address of a row pitch that is no power of
    // two, and the A copies end with blocks copied by several waves
    if (C::B_UNITS == 5 && ((kind == TG_LAYOUT_LDS_B && swz == SWZ_XOR) || kind == TG_LAYOUT_COPY_A))
        return TG_ERR_UNSUPPORTED;
    switch (kind) {
        case TG_LAYOUT_LDS_A: describe_ring_lds<C>(out, 0, swz); return TG_OK;
        case TG_LAYOUT_LDS_B: describe_ring_lds<C>(out, 1, swz); return TG_OK;
        case TG_LAYOUT_ACC: describe_acc<C>(out); return TG_OK;
        case TG_LAYOUT_COPY_A: describe_ring_copy_a<C>(out); return TG_OK;
    }
    return TG_ERR_INVALID_ARG;
}

// Element offset within one pipeline copy of element (i, j) of an operand
// tile as stored: fp32 family A (m, k), B (n, k); ring family A (m, k), B (k, n).
template <class C>
int64_t lds_offset(int swz, int operand, int64_t row, int64_t k) {
    const int rows = operand == 0 ? C::BM : C::BN;
    if (row < 0 || row >= rows || k < 0 || k >= C::BK) return -1;
    return lds_chunk_byte<C>((int)row, (int)(k / C::CHUNK), swz) / C::ELEM + k % C::CHUNK;
}

template <class C>
int64_t ring_lds_offset(int swz, int operand, int64_t i, int64_t j) {
    if (operand == 0) {
        if (i < 0 || i >= C::BM || j < 0 || j >= C::BK) return -1;
        return ring_a_byte<C>((int)i, (int)(j / C::CHUNK), swz) / C::ELEM + j % C::CHUNK;
    }
    if (i < 0 || i >= C::BK || j < 0 || j >= C::BN) return -1;
    return ring_b_byte<C>((int)i, (int)j, swz) / C::ELEM;
}

template <class C>
int acc_coord_checked(int wave, int lane, int slot, int64_t *row, int64_t *col) {
    if (wave < 0 || wave >= C::WAVES || lane < 0 || lane >= 64 || slot < 0 ||
        slot >= C::TM * C::TN * C::ACC_PER_MFMA || !row || !col)
        return -1;
    int r, c;
    acc_coord<C>(wave, lane, slot, r, c);
    *row = r;
    *col = c;
    return 0;
}

}  // namespace

extern "C" {

int64_t tg_layout_eval(const tg_layout *L, const int64_t *x, int64_t *out, int64_t max_out) {
    if (!layout_valid(L) || !x) return -1;
    // 1. flatten row-major
    int64_t flat = 0;
    for (int d = 0; d < L->rank; ++d) {
        if (x[d] < 0 || x[d] >= L->shape[d]) return -1;
        flat = flat * L->shape[d] + x[d];
    }
    // 2. split over the shard extents (component 0 most significant)
    // 3. accumulate each component on its axis, add the offset
    int64_t base[TG_AXIS_COUNT];
    for (int a = 0; a < TG_AXIS_COUNT; ++a) base[a] = L->offset[a];
    int64_t rest = flat;
    for (int k = L->n_shard - 1; k >= 0; --k) {
        const tg_iter &it = L->shard[k];
        const int64_t ck = rest % it.extent;
        rest /= it.extent;
        base[it.axis] += ck * it.stride;
    }
    // 4. broadcast the replica iters
    int64_t count = 1;
    for (int t = 0; t < L->n_replica; ++t) count *= L->replica[t].extent;
    for (int64_t r = 0; r < count && r < max_out; ++r) {
        int64_t coord[TG_AXIS_COUNT];
        std::memcpy(coord, base, sizeof coord);
        int64_t rr = r;
        for (int t = L->n_replica - 1; t >= 0; --t) {
            const tg_iter &it = L->replica[t];
            coord[it.axis] += (rr % it.extent) * it.stride;
            rr /= it.extent;
        }
        for (int z = 0; z < L->n_swizzle; ++z)
            coord[TG_AXIS_M] = swizzle_apply(coord[TG_AXIS_M], L->swizzle[z].m, L->swizzle[z].b, L->swizzle[z].s);
        if (out) std::memcpy(out + r * TG_AXIS_COUNT, coord, sizeof coord);
    }
    return count;
}

tg_status tile_gemm_describe_layout(int config, int swizzle, int kind, tg_layout *out) {
    if (!out) return TG_ERR_INVALID_ARG;
    if (swizzle == 0) swizzle = SWZ_XOR;
    if (swizzle != SWZ_NONE && swizzle != SWZ_PAD && swizzle != SWZ_XOR) return TG_ERR_INVALID_ARG;
    if (swizzle == SWZ_PAD && config != TG_CFG_256x256 && config != TG_LAYOUT_CFG_STRIP_N &&
        config != TG_LAYOUT_CFG_STRIP_M)
        return TG_ERR_UNSUPPORTED;
    std::memset(out, 0, sizeof *out);
    switch (config) {
        case TG_LAYOUT_CFG_F32_256: return describe_ring<RingF32_256>(swizzle, kind, out);
        case TG_LAYOUT_CFG_F32_128: return describe_ring<RingF32_128>(swizzle, kind, out);
        case TG_LAYOUT_CFG_F32_STRIP_N: return describe_ring<Strip256xN<DT_F32>>(swizzle, kind, out);
        case TG_LAYOUT_CFG_F32_STRIP_M: return describe_ring<StripMx256<DT_F32>>(swizzle, kind, out);
        case TG_CFG_256x256: return describe_ring<Ring256<DT_BF16>>(swizzle, kind, out);
        case TG_LAYOUT_CFG_STRIP_N: return describe_ring<Strip256xN<DT_BF16>>(swizzle, kind, out);
        case TG_LAYOUT_CFG_STRIP_M: return describe_ring<StripMx256<DT_BF16>>(swizzle, kind, out);
        case TG_CFG_128x128: return describe_ring<Ring128<DT_BF16>>(swizzle, kind, out);
        case TG_CFG_64x64: return describe_ring<Ring64<DT_BF16>>(swizzle, kind, out);
        case TG_CFG_288x160: return describe_ring<Ring288x160<DT_BF16>>(swizzle, kind, out);
        case TG_CFG_F32_64x64: return describe<CfgF32>(swizzle, kind, out);
    }
    return TG_ERR_INVALID_ARG;
}

int64_t tile_gemm_lds_offset(int config, int swizzle, int operand, int64_t row, int64_t k) {
    if (swizzle == 0) swizzle = SWZ_XOR;
    if ((swizzle != SWZ_NONE && swizzle != SWZ_PAD && swizzle != SWZ_XOR) || (operand != 0 && operand != 1)) return -1;
    if (swizzle == SWZ_PAD && config != TG_CFG_256x256 && config != TG_LAYOUT_CFG_STRIP_N &&
        config != TG_LAYOUT_CFG_STRIP_M)
        return -1;
    switch (config) {
        case TG_LAYOUT_CFG_F32_256: return ring_lds_offset<RingF32_256>(swizzle, operand, row, k);
        case TG_LAYOUT_CFG_F32_128: return ring_lds_offset<RingF32_128>(swizzle, operand, row, k);
        case TG_LAYOUT_CFG_F32_STRIP_N: return ring_lds_offset<Strip256xN<DT_F32>>(swizzle, operand, row, k);
        case TG_LAYOUT_CFG_F32_STRIP_M: return ring_lds_offset<StripMx256<DT_F32>>(swizzle, operand, row, k);
        case TG_CFG_256x256: return ring_lds_offset<Ring256<DT_BF16>>(swizzle, operand, row, k);
        case TG_LAYOUT_CFG_STRIP_N: return ring_lds_offset<Strip256xN<DT_BF16>>(swizzle, operand, row, k);
        case TG_LAYOUT_CFG_STRIP_M: return ring_lds_offset<StripMx256<DT_BF16>>(swizzle, operand, row, k);
        case TG_CFG_128x128: return ring_lds_offset<Ring128<DT_BF16>>(swizzle, operand, row, k);
        case TG_CFG_64x64: return ring_lds_offset<Ring64<DT_BF16>>(swizzle, operand, row, k);
        case TG_CFG_288x160: return ring_lds_offset<Ring288x160<DT_BF16>>(swizzle, operand, row, k);
        case TG_CFG_F32_64x64: return lds_offset<CfgF32>(swizzle, operand, row, k);
    }
    return -1;
}

int tile_gemm_acc_coord(int config, int wave, int lane, int slot, int64_t *row, int64_t *col) {
    switch (config) {
        case TG_LAYOUT_CFG_F32_256: return acc_coord_checked<RingF32_256>(wave, lane, slot, row, col);
        case TG_LAYOUT_CFG_F32_128: return acc_coord_checked<RingF32_128>(wave, lane, slot, row, col);
        case TG_LAYOUT_CFG_F32_STRIP_N: return acc_coord_checked<Strip256xN<DT_F32>>(wave, lane, slot, row, col);
        case TG_LAYOUT_CFG_F32_STRIP_M: return acc_coord_checked<StripMx256<DT_F32>>(wave, lane, slot, row, col);
        case TG_CFG_256x256: return acc_coord_checked<Ring256<DT_BF16>>(wave, lane, slot, row, col);
        case TG_LAYOUT_CFG_STRIP_N: return acc_coord_checked<Strip256xN<DT_BF16>>(wave, lane, slot, row, col);
        case TG_LAYOUT_CFG_STRIP_M: return acc_coord_checked<StripMx256<DT_BF16>>(wave, lane, slot, row, col);
        case TG_CFG_128x128: return acc_coord_checked<Ring128<DT_BF16>>(wave, lane, slot, row, col);
        case TG_CFG_64x64: return acc_coord_checked<Ring64<DT_BF16>>(wave, lane, slot, row, col);
        case TG_CFG_288x160: return acc_coord_checked<Ring288x160<DT_BF16>>(wave, lane, slot, row, col);
        case TG_CFG_F32_64x64: return acc_coord_checked<CfgF32>(wave, lane, slot, row, col);
    }
    return -1;
}

}  // extern "C"
