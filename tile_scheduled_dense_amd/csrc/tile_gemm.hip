// tile_gemm.hip -- the C ABI: argument validation, planning, kernel selection
// and launch on the caller's stream.  Declarations and contracts are in
// include/tile_gemm.h.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstddef>
#include <cstring>
#include <mutex>
#include <new>

#include "launch.hpp"
#include "pack.hpp"
#include "splitk.hpp"
#include "tile_gemm.h"

using namespace tg;

namespace {

constexpr int kMaxDevices = 64;

struct DeviceState {
    bool probed = false;
    bool gfx950 = false;
    void *scratch = nullptr;   // this device's address of `scratch` (tile_gemm_ex_noalloc)
};

std::mutex g_mutex;
DeviceState g_devices[kMaxDevices];

// gfx950 check for the current device, cached per device.
tg_status current_device_ok() {
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
        (void)hipGetLastError();
        return TG_ERR_UNSUPPORTED;
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return TG_ERR_UNSUPPORTED;
    }
    std::lock_guard<std::mutex> lock(g_mutex);
    DeviceState &d = g_devices[dev];
    if (!d.probed) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            return TG_ERR_UNSUPPORTED;
        }
        d.gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        d.probed = true;
    }
    return d.gfx950 ? TG_OK : TG_ERR_UNSUPPORTED;
}

// The scratch of tile_gemm_ex_noalloc (tile_gemm.h): split-K partials, the
// aligned copy of A and the remainder partials of calls that cannot allocate.
// Each device holds its own copy of the array at its own address; in host code
// the name stands for a host-side shadow, so the device address is looked up
// once per device (with that device current) and only that address is used.
static __device__ __align__(256) char scratch[TILE_GEMM_NOALLOC_SCRATCH_BYTES];

tg_status current_device_scratch(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return TG_ERR_UNSUPPORTED;
    }
    std::lock_guard<std::mutex> lock(g_mutex);
    DeviceState &d = g_devices[dev];
    if (!d.scratch) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
            (void)hipGetLastError();
            return TG_ERR_INTERNAL;
        }
        d.scratch = ptr;
    }
    *out = d.scratch;
    return TG_OK;
}

struct CfgDims {
    int bm, bn, bk, waves, stage_bytes, mfma_m, mfma_k;
};

template <class C>
CfgDims dims_of(int mfma_k) {
    return {C::BM, C::BN, C::BK, C::WAVES, C::STAGE_BYTES, C::MT, mfma_k};
}

// The tile of a configuration; the 256 x 256 and 128 x 128 ring tiles take
// fp32 inputs too (16x16x4 MFMAs, a K tile of 16).
CfgDims cfg_dims(int config, tg_dtype dtype) {
    const bool f32 = dtype == TG_F32;
    switch (config) {
        case TG_CFG_256x256:
            return f32 ? dims_of<RingF32_256>(RingF32_256::MK) : dims_of<Ring256<DT_BF16>>(Ring256<DT_BF16>::MK);
        case TG_CFG_128x128:
            return f32 ? dims_of<RingF32_128>(RingF32_128::MK) : dims_of<Ring128<DT_BF16>>(Ring128<DT_BF16>::MK);
        case TG_CFG_64x64: return dims_of<Ring64<DT_BF16>>(Ring64<DT_BF16>::MK);
        case TG_CFG_F32_64x64: return dims_of<CfgF32>(4);
        case TG_CFG_288x160: return dims_of<Ring288x160<DT_BF16>>(Ring288x160<DT_BF16>::MK);
        default: return {0, 0, 0, 0, 0, 0, 0};
    }
}

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The 256 x 256 partition of one M x N problem: main tile rows and columns,
// and the thin-remainder strips beside them (an N tail of at most 64 columns
// goes to 256 x 64 strip blocks, one per tile row; an M tail of at most 64
// rows to 64 x 256 strip blocks, one per tile column plus the corner) instead
// of a column or row of mostly empty tiles.  A strip needs a main tile beside
// it: N >= 256 for an N strip, M >= 256 for an M strip.
struct Partition256 {
    int64_t tiles_m, tiles_n, strip_n, strip_m;
    int64_t area() const { return (tiles_m * tiles_n * 256 + (strip_n + strip_m) * 64) * 256; }
};

Partition256 partition256(int64_t M, int64_t N) {
    const bool thin_n = N >= 256 && N % 256 != 0 && N % 256 <= 64;
    const bool thin_m = M >= 256 && M % 256 != 0 && M % 256 <= 64;
    Partition256 q;
    q.tiles_m = thin_m ? M / 256 : cdiv(M, 256);
    q.tiles_n = thin_n ? N / 256 : cdiv(N, 256);
    q.strip_n = thin_n ? q.tiles_m : 0;
    q.strip_m = thin_m ? q.tiles_n + (thin_n ? 1 : 0) : 0;
    return q;
}

// Default choice: the largest tile that still gives about one workgroup per
// CU (240 of the 256) and pads the output by at most a quarter more than the
// next smaller tile.  The 256-wide padding counts its strips: a 257 x 129
// problem covers 256 x 256 plus a 64 x 256 strip, 5/6 of the 384 x 256 it pads
// to in 128-wide tiles.  fp32 takes the same rule over its ring tiles (256 x 256,
// 128 x 128) with the register-staged 64 x 64 tile in place of the 16-bit
// 64 x 64 ring tile.
// part_fill: the 256 x 256 tiles that must be busy (of the 256 CUs) before one
// part-filled round of them is taken over a second round of 128 x 128 tiles.
static int choose_tile(int64_t batch, int64_t M, int64_t N, int64_t part_fill) {
    // Many small problems that each fit one 288 x 160 tile, at least half of it
    // output: one block per problem reads its A and B once (the 256 x 256 tile
    // plus a strip read B twice and multiplied 2.5 times the output of a
    // 257 x 129 problem).
    if (batch >= 128 && M <= 288 && N <= 160 && 2 * M * N >= 288 * 160) return TG_CFG_288x160;
    const Partition256 q = partition256(M, N);
    const int64_t big = (q.tiles_m * q.tiles_n + q.strip_n + q.strip_m) * batch;
    const int64_t mid = cdiv(M, 128) * cdiv(N, 128) * batch;
    const int64_t area_big = q.area() * batch, area_mid = mid * 128 * 128;
    if (big >= 240 && 4 * area_big <= 5 * area_mid) return TG_CFG_256x256;
    // A part-filled round of 256 x 256 tiles against a second round of 128 x 128
    // ones (two per CU).
    if (big >= part_fill && mid > 512 && 4 * area_big <= 5 * area_mid) return TG_CFG_256x256;
    if (mid >= 240) return TG_CFG_128x128;
    if (big >= 240) return TG_CFG_256x256;
    return TG_CFG_64x64;
}

int choose_config(int64_t batch, int64_t M, int64_t N, tg_dtype dtype) {
    if (dtype == TG_F32) {
        // Both fp32 ring tiles run 16x16x4 MFMAs, so a 256 x 256 tile does only
        // about 1.75 times the work of a 128 x 128 one per CU cycle: a part-filled
        // round of them wins from three quarters of the CUs (3072^3: 693 us against
        // 607 at 144 tiles; 3328^3: 748 / 658 at 169; 3584^3: 807 / 923 at 196).
        const int c = choose_tile(batch, M, N, 192);
        return c == TG_CFG_256x256 || c == TG_CFG_128x128 ? c : TG_CFG_F32_64x64;
    }
    // 16-bit: at least half the CUs busy with 256 x 256 tiles beats a second round
    // of 128 x 128 ones, whose 32x32x16 MFMAs do less than half the work per CU
    // cycle (3000^3 bf16: 76.5 us against 98.7).
    return choose_tile(batch, M, N, 128);
}

// Size of tg_options in ABI version 1 (five ints, before the split-K fields).
constexpr int kOptionsV1Size = 5 * (int)sizeof(int);
constexpr int64_t kMaxSplits = 64;

// Automatic split count: split only when the output tiles fill less than
// half the `slots` workgroups the GPU runs at once, doubling while the blocks
// still fit in one round and each slice keeps at least 1024 of K.
int64_t auto_splits(int64_t tiles, int64_t K, int64_t slots) {
    if (2 * tiles >= slots) return 1;
    int64_t s = 1;
    while (2 * s <= kMaxSplits && tiles * 2 * s <= slots && K / (2 * s) >= 1024) s *= 2;
    return s;
}

// fp32 ring tiles are bound by their MFMAs: a CU runs its share of the
// workgroups one after another, so a call takes about as long as its busiest
// CU's share, ceil(blocks / 256) slices of 1/s of a tile each.  Split in two or
// four when that share drops by a tenth or more, each slice keeping at least 512
// of K (3072^3 on 128 x 128 tiles: 607 us unsplit, 523 split 2, 491 split 4;
// 2048^3 gains nothing, and none is predicted).
int64_t f32_round_splits(int64_t tiles, int64_t K) {
    int64_t best = 1;
    double share = (double)cdiv(tiles, 256);
    for (int64_t s = 2; s <= 4; s *= 2) {
        if (K / s < 512) break;
        const double c = (double)cdiv(tiles * s, 256) / (double)s;
        if (c <= 0.9 * share) {
            best = s;
            share = c;
        }
    }
    return best;
}

// Workgroups of a configuration one CU holds at once, the lesser of what its
// registers and its LDS allow (a SIMD holds 512 registers per lane for its
// waves, a CU 160 KiB of LDS); the built kernels' register counts are checked
// against this table by a code-object test.
//   256 x 256: 510 registers a wave, 4 waves: one per CU.
//   128 x 128: under 256 registers, 4 waves: two waves per SIMD, two per CU
//              (LDS 64 / 80 KiB at depth 4 / 5 allows two as well).
//   64 x 64:   under 168 registers, 2 waves: three waves per SIMD, six per CU by
//              registers; LDS 8 KiB per depth: 5 at depth 4, 4 at depth 5.
int cfg_per_cu(int config, int depth, bool f32, int swz) {
    switch (config) {
        case TG_CFG_256x256: return 1;
        case TG_CFG_288x160: return 1;   // 320 registers a wave, 4 waves, 28 KiB per depth
        case TG_CFG_128x128: {
            // 16-bit: 164 registers a wave (three waves per SIMD); fp32: 193 (two);
            // 16 KiB of LDS per depth
            const int by_regs = f32 ? 2 : 3, by_lds = (160 * 1024) / (depth * 16 * 1024);
            return by_lds < by_regs ? by_lds : by_regs;
        }
        case TG_CFG_64x64: {
            // 128 registers a wave (148 with the fused tail, built at depth 4,
            // where the LDS holds five), 2 waves, 8 KiB of LDS per depth
            const int by_lds = (160 * 1024) / (depth * 8 * 1024);
            return by_lds < 8 ? by_lds : 8;
        }
        case TG_CFG_F32_64x64:
            // 4 waves; depth 1 at 100 registers (five waves per SIMD, five per CU;
            // 16 KiB of LDS), 84 without the swizzle (six), depth 2 at 108 (four;
            // 32 KiB allows five)
            return depth == 1 ? (swz == SWZ_NONE ? 6 : 5) : 4;
        default: return 1;
    }
}

// Workgroups the automatic split aims to fill: 256 for the 256 x 256 tile, 512
// for the smaller ones.  These are split targets that measured best, not the
// residency (cfg_per_cu): the 64 x 64 tile holds 5 workgroups per CU at depth
// 4, yet filling them all measured slower on every shape it changed (us):
// 8192 x 64 x 8192 35.8 against 29.6, 64 x 8192 x 8192 38.6 / 33.2,
// 256 x 256 x 65536 31.5 / 28.7, 512 x 2048 x 2048 23.4 / 21.2; more slices
// cost more partials while one wave per SIMD already feeds its matrix core.
// One wave per SIMD for the 128 x 128 tile as well (256) measured slower on
// 16384 x 96 x 4096 (55.2 against 39.7: the 64 x 64 tile unsplit won the
// comparison) and 384 x 4096 x 4096 (36.9 against 33.0), faster only on
// 8192 x 128 x 8192 (38.5 against 43.0).
int64_t cfg_slots(int config) { return config == TG_CFG_256x256 || config == TG_CFG_288x160 ? 256 : 512; }

// A thin remainder computed by a GEMM of its own (see tile_gemm.h): its
// extents, where it starts in C, and its K split and workspace region.
struct Tail {
    int64_t splits = 0;                // 0: none
    int64_t m0 = 0, n0 = 0, rows = 0, cols = 0;
    int64_t ws_offset = 0, ws_bytes = 0;
};

struct Plan {
    tg_plan_info info;
    int64_t strip_n = 0, strip_m = 0;  // strip blocks per problem (256 x 64, 64 x 256)
    Tail tail_n, tail_m;
    int64_t wanted_workspace = 0;      // bytes the split or the A copy it would like needs
    void *workspace = nullptr;         // set when the call splits or repacks A
    int64_t workspace_given = 0;
    int64_t lda_packed = 0;            // row stride of the A copy (elements)
    int64_t ldb_packed = 0;            // row stride of the B copy (elements)
    int64_t strip_k_slice = 0, strip_rows_n = 0, strip_ws_offset = 0;   // strips split along K
    int64_t b_offset = 0;              // workspace bytes before the B copy (the A copy)
};

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// lda, ldb: the call's (or, for the plan queries, the assumed) leading
// dimensions of A and B; a_aligned: A itself starts on a 16-byte boundary;
// b_two_byte: B's rows start on boundaries only 2-byte aligned (odd ldb or B).
tg_status make_plan(int64_t batch, int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                    const tg_options *opt, int64_t lda, bool a_aligned, int64_t ldb, bool b_two_byte, Plan &out) {
    if (batch < 0 || M < 0 || N < 0 || K < 0) return TG_ERR_INVALID_ARG;
    if (dtype != TG_F32 && dtype != TG_BF16 && dtype != TG_F16) return TG_ERR_INVALID_ARG;
    tg_options o{};
    if (opt) {
        // the caller's struct may predate the split-K fields: read what it has
        if (opt->struct_size < kOptionsV1Size) return TG_ERR_INVALID_ARG;
        std::memcpy(&o, opt, opt->struct_size < (int)sizeof o ? (size_t)opt->struct_size : sizeof o);
    }
    // Split-K (16-bit): a forced count applies to the chosen config; the
    // automatic choice splits only when the tiles cannot fill the GPU and K is
    // deep, and only if the caller's workspace holds the partials -- otherwise
    // the plain plan.
    if (o.split_k < 0) return TG_ERR_INVALID_ARG;
    const bool sixteen = dtype != TG_F32;
    const bool some = K > 0 && M > 0 && N > 0 && batch > 0;
    // the configurations this input type has: the ring tiles, and for fp32 the
    // register-staged 64 x 64 tile (no split) in place of the 16-bit 64 x 64
    const int small_cfg = sixteen ? TG_CFG_64x64 : TG_CFG_F32_64x64;
    auto cfg_ok = [&](int c) {
        return sixteen ? (c == TG_CFG_256x256 || c == TG_CFG_128x128 || c == TG_CFG_64x64 || c == TG_CFG_288x160)
                       : (c == TG_CFG_256x256 || c == TG_CFG_128x128 || c == TG_CFG_F32_64x64);
    };
    int64_t want = 1, wanted_bytes = 0;
    int config = o.force_cfg;
    // An always-repacked A (pack_a == 2) is built for the unsplit 256 x 256
    // tile: with the tile left to the library, that is the tile, unsplit.
    const bool pin256 = sixteen && (o.pack_a == 2 || o.pack_b == 2) && config == TG_CFG_AUTO;
    if (pin256) config = TG_CFG_256x256;
    if (some && o.split_k == 0 && !pin256) {
        // With a forced tile, that tile's own count.  Otherwise each tile with its
        // own count, and the one whose workgroups fill the most of its slots
        // (cfg_slots, the measured split targets; ties: the larger tile, fewer
        // re-reads of A and B); no split when that one needs none (the plain
        // choice below then picks the tile).
        // 1024 x 1024 x 4096 bf16: 128 x 128 split 4 (256 workgroups) takes
        // 25.6 us where 256 x 256 split 4 (64) took 35.6; 512 x 2048 x 2048: the
        // 64 x 64 tile unsplit (256) 19.4 us where 256 x 256 split 2 (32) took 33.7.
        // The fill is weighed by the share of the padded tiles that is output
        // (a 256 x 256 tile over 64 columns multiplies three quarters zeros):
        // 8192 x 64 x 8192 bf16 takes 64 x 64 split 4, 27.0 us, where 256 x 256
        // split 8 took 54.5.
        int cfg = o.force_cfg;
        if (!cfg) {
            double best = -1.0;
            for (int c : {(int)TG_CFG_256x256, (int)TG_CFG_128x128, small_cfg}) {
                const CfgDims dd = cfg_dims(c, dtype);
                const int64_t tm = cdiv(M, dd.bm), tn = cdiv(N, dd.bn), tiles = tm * tn * batch;
                const int64_t slots = cfg_slots(c);
                // the register-staged fp32 tile does not split
                const int64_t blocks = tiles * (c == TG_CFG_F32_64x64 ? 1 : auto_splits(tiles, K, slots));
                const double fill = (double)(blocks < slots ? blocks : slots) / (double)slots;
                const double useful = (double)M * (double)N / ((double)(tm * dd.bm) * (double)(tn * dd.bn));
                if (fill * useful > best * (1.0 + 1e-9)) {
                    best = fill * useful;
                    cfg = c;
                }
            }
        }
        if (cfg >= TG_CFG_256x256 && cfg <= TG_CFG_64x64 && cfg_ok(cfg)) {
            const CfgDims dd = cfg_dims(cfg, dtype);
            const int64_t tiles = cdiv(M, dd.bm) * cdiv(N, dd.bn) * batch;
            int64_t s_auto = auto_splits(tiles, K, cfg_slots(cfg));
            if (!sixteen && s_auto == 1 && (cfg == TG_CFG_256x256 || cfg == TG_CFG_128x128))
                s_auto = f32_round_splits(tiles, K);
            const int64_t slice = cdiv(cdiv(K, s_auto), dd.bk) * dd.bk;
            const int64_t s_eff = cdiv(K, slice);
            wanted_bytes = s_eff > 1 ? s_eff * batch * M * N * 4 : 0;
            if (s_eff > 1 && o.workspace && o.workspace_bytes >= wanted_bytes) {
                want = s_auto;
                config = cfg;
            }
        }
    } else if (some && o.split_k >= 2) {
        want = o.split_k < kMaxSplits ? o.split_k : kMaxSplits;
    }
    if (!config) config = choose_config(batch, M, N, dtype);
    const bool tail_req = o.bias_mode != 0 || o.activation != 0;   // the fused tail (tile_gemm.h)
    if (config < TG_CFG_256x256 || config > TG_CFG_288x160) return TG_ERR_INVALID_ARG;
    if (!cfg_ok(config)) return TG_ERR_UNSUPPORTED;
    // pipeline depth = LDS copies of the K tile (window = depth - 1); f32: the
    // register-staged fp32 tile (the fp32 ring tiles follow the 16-bit rules)
    const bool f32 = config == TG_CFG_F32_64x64;
    const int depth = o.pipeline_depth ? o.pipeline_depth : (f32 ? 2 : 4);
    // depth 5 (a window of 4 tiles) for the smaller 16-bit tiles, whose two
    // workgroups per CU still fit 160 KiB of LDS; the 256 x 256 tile's software
    // pipeline cycles its copies four at a time
    // (the unpipelined fp32 256 x 256 kernel is not built: its 256 MFMAs per K
    // tile through the compiler's builtin need scratch)
    const bool depth_ok = f32 ? (depth == 1 || depth == 2)
                          : config == TG_CFG_288x160 ? (depth == 2 || depth == 4)
                          : !sixteen && config == TG_CFG_256x256 ? (depth == 2 || depth == 4)
                          : (depth == 1 || depth == 2 || depth == 4 || (depth == 5 && config != TG_CFG_256x256));
    if (!depth_ok) return TG_ERR_UNSUPPORTED;
    const int swz = o.swizzle ? o.swizzle : SWZ_XOR;
    if (swz < 0 || swz > SWZ_XOR) return TG_ERR_INVALID_ARG;
    if (!f32 && swz == SWZ_NONE && depth != 4) return TG_ERR_UNSUPPORTED;   // ablation built at depth 4 only
    // pad_stride: the 16-bit 256 x 256 tile at depth 4 (the placement ablation of the default kernel)
    if (swz == SWZ_PAD && (config != TG_CFG_256x256 || depth != 4 || !sixteen)) return TG_ERR_UNSUPPORTED;
    const int order = o.block_order;
    if (order != 0 && order != 1) return TG_ERR_UNSUPPORTED;

    const CfgDims d = cfg_dims(config, dtype);
    tg_plan_info &p = out.info;
    std::memset(&p, 0, sizeof p);
    p.config = config;
    p.block_m = d.bm;
    p.block_n = d.bn;
    p.block_k = d.bk;
    p.waves = d.waves;
    p.threads = 64 * d.waves;
    p.pipeline_depth = depth;
    p.swizzle = swz;
    p.block_order = order;
    p.tiles_m = cdiv(M, d.bm);
    p.tiles_n = cdiv(N, d.bn);
    // Partition of a thin remainder into strips (partition256)
    int64_t strip_n = 0, strip_m = 0;
    if (config == TG_CFG_256x256) {
        const Partition256 q = partition256(M, N);
        p.tiles_m = q.tiles_m;
        p.tiles_n = q.tiles_n;
        strip_n = q.strip_n;
        strip_m = q.strip_m;
    }
    out.strip_n = strip_n;
    out.strip_m = strip_m;
    p.strip_blocks = strip_n + strip_m;
    p.grid = (p.tiles_m * p.tiles_n + p.strip_blocks) * batch;
    const int64_t full_m = M / d.bm < p.tiles_m ? M / d.bm : p.tiles_m;
    const int64_t full_n = N / d.bn < p.tiles_n ? N / d.bn : p.tiles_n;
    p.interior_blocks = full_m * full_n;
    p.fringe_blocks = p.tiles_m * p.tiles_n - p.interior_blocks;
    p.mfma_m = d.mfma_m;
    p.mfma_n = d.mfma_m;
    p.mfma_k = d.mfma_k;
    p.k_tiles = cdiv(K, d.bk);
    p.k_tail = K % d.bk;
    p.lds_bytes = depth * (swz == SWZ_PAD ? ring_stage_bytes<Ring256<DT_BF16>, SWZ_PAD>() : d.stage_bytes);
    p.per_cu = cfg_per_cu(config, depth, !sixteen, swz);

    // split-K
    if (f32 && o.split_k >= 2) return TG_ERR_UNSUPPORTED;
    const int64_t k_slice = K > 0 ? cdiv(cdiv(K, want), d.bk) * d.bk : 0;
    const int64_t splits = K > 0 ? cdiv(K, k_slice) : 1;
    const int64_t bytes = splits > 1 ? splits * batch * M * N * 4 : 0;
    out.wanted_workspace = o.split_k == 0 ? wanted_bytes : bytes;
    p.split_k = (int)splits;
    p.k_slice = splits > 1 ? k_slice : K;
    p.workspace_bytes = bytes;
    if (splits > 1) p.grid *= splits;
    out.workspace = splits > 1 ? o.workspace : nullptr;
    out.workspace_given = o.workspace_bytes;

    // the fused tail is built into the default depth and swizzle only (a split
    // call applies it in the combine pass)
    if ((o.bias_mode != 0 || o.activation != 0) && splits == 1 &&
        (depth != (f32 ? 2 : 4) || swz != SWZ_XOR))
        return TG_ERR_UNSUPPORTED;

    // Repack of A (see tile_gemm.h): rows not on 16-byte boundaries, a plan
    // whose A panels are each read by many workgroups, no split.
    if (o.pack_a < 0 || o.pack_a > 2) return TG_ERR_INVALID_ARG;
    if (o.pack_a == 2 && (!sixteen || config != TG_CFG_256x256 || splits > 1)) return TG_ERR_UNSUPPORTED;
    int64_t used = 0;         // workspace bytes taken so far by the A copy
    int64_t wanted_pack = 0;  // bytes of the A copy the plan would like
    if (sixteen && some && config == TG_CFG_256x256 && splits == 1 && o.pack_a != 1) {
        const int64_t ldp = round_up(K, 8);
        const int64_t bytes_a = round_up(batch * M * ldp * 2, 256);
        const bool misaligned = lda % 8 != 0 || !a_aligned;
        const bool worth = misaligned && p.tiles_n >= 8;
        if (o.pack_a == 2 || worth) {
            wanted_pack = bytes_a;
            out.wanted_workspace = out.wanted_workspace > bytes_a ? out.wanted_workspace : bytes_a;
            if (o.pack_a == 2 || (o.workspace && o.workspace_bytes >= bytes_a)) {
                p.pack_a = 1;
                p.workspace_bytes = bytes_a;
                out.lda_packed = ldp;
                out.workspace = o.workspace;
                used = bytes_a;
            }
        }
    }
    // Repack of B (see tile_gemm.h), after the A copy: rows only 2-byte aligned
    // (an odd ldb, or B itself on an odd 2-byte boundary), a plan whose B panels
    // are each read by many workgroups (at least 8 tile rows), no split.  Rows on
    // 4- or 8-byte boundaries cost their copies 17% more, less than the copy of
    // B: on 8191 x 8193 x 8190 (ldb = N + 5, rows 4-byte aligned) the repack made
    // the call 1052 us against 1000.
    if (o.pack_b < 0 || o.pack_b > 2) return TG_ERR_INVALID_ARG;
    if (o.pack_b == 2 && (!sixteen || config != TG_CFG_256x256 || splits > 1)) return TG_ERR_UNSUPPORTED;
    if (sixteen && some && config == TG_CFG_256x256 && splits == 1 && o.pack_b != 1) {
        const int64_t ldp = round_up(N, 8);
        const int64_t bytes_b = round_up(batch * K * ldp * 2, 256);
        const bool worth = b_two_byte && p.tiles_m >= 8;
        if (o.pack_b == 2 || worth) {
            wanted_pack += bytes_b;
            out.wanted_workspace = out.wanted_workspace > wanted_pack ? out.wanted_workspace : wanted_pack;
            if (o.pack_b == 2 || (o.workspace && o.workspace_bytes >= used + bytes_b)) {
                p.pack_b = 1;
                out.ldb_packed = ldp;
                out.b_offset = used;
                used += bytes_b;
                p.workspace_bytes = used;
                out.workspace = o.workspace;
            }
        }
    }

    // Thin remainders as GEMMs of their own (tile_gemm.h), when asked: each
    // tail is split along K until it has about 1024 workgroups of the 64 x 64
    // tile (four per CU), slices of at least 512, if the workspace past the A
    // copy holds the partials.  Not chosen automatically: on 8191 x 8193 x
    // 8190 the 32 strips that follow the 1024 main tiles cost the grid about
    // 8 us, the separate GEMM and its combine about 33 us.
    if (o.tail_gemm < 0 || o.tail_gemm > 3) return TG_ERR_INVALID_ARG;
    if (o.persistent < 0 || o.persistent > 2) return TG_ERR_INVALID_ARG;
    // the bias pointer itself is checked by the call (a plan query needs only the modes)
    if (o.bias_mode < 0 || o.bias_mode > 2 || o.activation < 0 || o.activation > 2 || o.bias_stride < 0 ||
        reinterpret_cast<uintptr_t>(o.bias) % 4)
        return TG_ERR_INVALID_ARG;
    if (some && strip_n + strip_m > 0 && splits == 1) {
        if (o.tail_gemm == 2 && !sixteen) return TG_ERR_UNSUPPORTED;   // remainder GEMMs: 16-bit 64 x 64 tile
        if (o.tail_gemm == 2) {
            const int64_t n_main = p.tiles_n * d.bn, m_main = p.tiles_m * d.bm;
            int64_t wanted_tail = wanted_pack;
            auto set_tail = [&](Tail &t, int64_t m0, int64_t n0, int64_t rows, int64_t cols) {
                t.m0 = m0;
                t.n0 = n0;
                t.rows = rows;
                t.cols = cols;
                const int64_t tiles = cdiv(rows, 64) * cdiv(cols, 64) * batch;
                int64_t sp = 1;
                while (2 * sp <= 16 && tiles * 2 * sp <= 1024 && K / (2 * sp) >= 512) sp *= 2;
                const int64_t bytes = sp > 1 ? round_up(sp * batch * rows * cols * 4, 256) : 0;
                wanted_tail += bytes;
                if (sp > 1 && o.workspace && o.workspace_bytes >= used + bytes) {
                    t.splits = sp;
                    t.ws_offset = used;
                    t.ws_bytes = bytes;
                    used += bytes;
                } else {
                    t.splits = 1;
                }
            };
            if (strip_n) set_tail(out.tail_n, 0, n_main, M, N - n_main);
            if (strip_m) set_tail(out.tail_m, m_main, 0, M - m_main, strip_n ? n_main : N);
            out.wanted_workspace = out.wanted_workspace > wanted_tail ? out.wanted_workspace : wanted_tail;
            p.tail_n_splits = (int)out.tail_n.splits;
            p.tail_m_splits = (int)out.tail_m.splits;
            out.strip_n = out.strip_m = 0;
            p.grid -= p.strip_blocks * batch;
            p.strip_blocks = 0;
            if (used > 0) {
                p.workspace_bytes = used;
                out.workspace = o.workspace;
            }
        }
    }

    // Thin strips split along K (tail_gemm == 3, or automatically, tile_gemm.h):
    // each strip block becomes S K slices (S doubled while the slices fill at
    // most the 256 slots and keep at least 512 of K), whose partials follow the
    // copies in the workspace; a combine pass over the strip region finishes
    // them.  Automatic when the whole strips would run as a part-filled round
    // of their own after the main tiles (these end a whole round, or leave too
    // few slots in their last one): 8191 x 8193 x 8190 (32 strips after 1024
    // main tiles) 953-964 us split 8 ways against 988-992 whole, 8193^2 x 8192
    // 862-866 against 898-900, 4096 x 4097 x 4096 133 against 160; where the
    // strips fit beside a part-filled last round they stay whole (6145^2 x 6144,
    // 49 strips beside 64 of 576 main tiles: 414 us whole, 428 split).
    p.strip_splits = 1;
    const int64_t main_blocks = p.tiles_m * p.tiles_n * batch, slots256 = cfg_slots(TG_CFG_256x256);
    const int64_t last_round = main_blocks % slots256;
    const bool auto_strip_split = o.tail_gemm == 0 && main_blocks > 0 &&
                                  (last_round == 0 || last_round + (out.strip_n + out.strip_m) * batch > slots256);
    if (some && out.strip_n + out.strip_m > 0 && splits == 1 && (o.tail_gemm == 3 || auto_strip_split)) {
        const int64_t strips = (out.strip_n + out.strip_m) * batch;
        const int64_t slots = cfg_slots(TG_CFG_256x256);
        int64_t sp = 1;
        while (2 * sp <= 16 && strips * 2 * sp <= slots && K / (2 * sp) >= 512) sp *= 2;
        if (sp > 1) {
            const int64_t k_slice_s = cdiv(cdiv(K, sp), d.bk) * d.bk;
            const int64_t s_eff = cdiv(K, k_slice_s);
            const int64_t n_main = p.tiles_n * d.bn, m_main = p.tiles_m * d.bm;
            const int64_t rows_n = out.strip_m ? m_main : M;
            const int64_t floats = s_eff * batch * ((out.strip_n ? rows_n * (N - n_main) : 0) +
                                                    (out.strip_m ? (M - m_main) * N : 0));
            const int64_t bytes = round_up(floats * 4, 256);
            const int64_t wanted = wanted_pack + bytes;
            out.wanted_workspace = out.wanted_workspace > wanted ? out.wanted_workspace : wanted;
            if (s_eff > 1 && o.workspace && o.workspace_bytes >= used + bytes) {
                p.strip_splits = (int)s_eff;
                out.strip_k_slice = k_slice_s;
                out.strip_rows_n = rows_n;
                out.strip_ws_offset = used;
                used += bytes;
                p.workspace_bytes = used;
                out.workspace = o.workspace;
                p.grid += (s_eff - 1) * strips;
            }
        }
    }

    // Persistent workgroups (tile_gemm.h), on request: a whole grid of
    // interior tiles of one problem, K in whole groups of four K tiles, at
    // least two tiles per workgroup.
    constexpr int64_t kPersistentBlocks = 256;
    if (sixteen && some && o.persistent == 2 && !tail_req && config == TG_CFG_256x256 && depth == 4 &&
        swz == SWZ_XOR && order == 0 && batch == 1 && splits == 1 && !p.pack_a && !p.pack_b && p.strip_blocks == 0 &&
        M % 256 == 0 &&
        N % 256 == 0 && K % (4 * d.bk) == 0 && K >= 8 * d.bk && p.tiles_m * p.tiles_n >= 2 * kPersistentBlocks) {
        p.persistent = 1;
        p.grid = kPersistentBlocks;
    }
    // Two batch entries per workgroup (tile_gemm.h): single-tile problems on the
    // 288 x 160 tile in more than one round and at most two, unless the caller
    // asks for the plain grid (512 x 257x129x1000 f16: 114.9 against 111.8 us
    // in a standalone copy of the kernel, the same result bit for bit).
    const int64_t chain_blocks = cfg_slots(TG_CFG_288x160);
    if (sixteen && some && o.persistent != 1 && config == TG_CFG_288x160 && depth == 4 && swz == SWZ_XOR &&
        splits == 1 && p.tiles_m == 1 && p.tiles_n == 1 && p.strip_blocks == 0 && !p.pack_a && !p.pack_b &&
        batch > chain_blocks && batch <= 2 * chain_blocks && cdiv(K, d.bk) >= depth) {
        p.persistent = 1;
        p.grid = chain_blocks;
    }
    return TG_OK;
}

// Byte extent [lo, hi) touched by a strided-batched row-major operand.
struct Range {
    uintptr_t lo, hi;
};

Range span(const void *p, int64_t batch, int64_t rows, int64_t cols, int64_t ld, int64_t stride, int esz) {
    if (batch == 0 || rows == 0 || cols == 0) return {0, 0};
    const uintptr_t base = reinterpret_cast<uintptr_t>(p);
    const int64_t last = (batch - 1) * stride + (rows - 1) * ld + cols;   // one past the last element
    return {base, base + static_cast<uintptr_t>(last) * esz};
}

bool overlaps(Range a, Range b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }

tg_status validate(int64_t batch, int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                   const void *A, int64_t lda, int64_t sA, const void *B, int64_t ldb, int64_t sB,
                   const float *C, int64_t ldc, int64_t sC) {
    if (batch < 0 || M < 0 || N < 0 || K < 0) return TG_ERR_INVALID_ARG;
    if (dtype != TG_F32 && dtype != TG_BF16 && dtype != TG_F16) return TG_ERR_INVALID_ARG;
    if (lda < (K > 1 ? K : 1) || ldb < (N > 1 ? N : 1) || ldc < (N > 1 ? N : 1)) return TG_ERR_INVALID_ARG;
    if (sA < 0 || sB < 0 || sC < 0) return TG_ERR_INVALID_ARG;
    const int esz = dtype == TG_F32 ? 4 : 2;
    const bool any_out = batch > 0 && M > 0 && N > 0;
    if (any_out && C == nullptr) return TG_ERR_INVALID_ARG;
    if (any_out && K > 0 && (A == nullptr || B == nullptr)) return TG_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(A) % esz || reinterpret_cast<uintptr_t>(B) % esz ||
        reinterpret_cast<uintptr_t>(C) % 4)
        return TG_ERR_INVALID_ARG;
    if (!any_out) return TG_OK;
    // distinct batch entries of C must not overlap each other
    if (batch > 1 && sC < (M - 1) * ldc + N) return TG_ERR_INVALID_ARG;
    if (K > 0) {
        const Range rc = span(C, batch, M, N, ldc, sC, 4);
        if (overlaps(rc, span(A, batch, M, K, lda, sA, esz)) || overlaps(rc, span(B, batch, K, N, ldb, sB, esz)))
            return TG_ERR_INVALID_ARG;
    }
    return TG_OK;
}

// Per-thread offsets inside a block are 32-bit: the byte offset of any element
// of an A or B tile from the tile's first row, and of any C element from the
// block's first row (a fringe block stores C through a buffer resource), must
// stay below 2^31, with 4 KiB to spare (the 16-bit kernel adds up to 3 KiB: a
// copy group's resource base sits below the tile).
bool offsets_fit(const tg_plan_info &p, int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int esz) {
    const int64_t lim = (int64_t(1) << 31) - 1 - 4096;
    return ((int64_t)p.block_m * lda + K) * esz < lim && ((int64_t)p.block_k * ldb + p.block_n) * esz < lim &&
           ((int64_t)p.block_m * ldc + p.block_n) * 4 < lim;
}

template <int P>
tg_status launch_combine_p(const float *W, float *C, int64_t M, int64_t N, int64_t ldc, int64_t sC,
                           int64_t problems, int S, float alpha, float beta, const float *bias,
                           int64_t bias_stride, int bias_mode, int act, hipStream_t stream) {
    const int64_t total = problems * M * N;
    const int64_t blocks = cdiv(total, 256) < 8192 ? cdiv(total, 256) : 8192;
    hipLaunchKernelGGL((splitk_combine_kernel<P>), dim3((unsigned)blocks), dim3(256), 0, stream, W, C, M, N, ldc,
                       sC, problems, S, alpha, beta, bias, bias_stride, bias_mode, act);
    return hipGetLastError() == hipSuccess ? TG_OK : TG_ERR_LAUNCH;
}

tg_status launch_combine(const float *W, float *C, int64_t M, int64_t N, int64_t ldc, int64_t sC,
                         int64_t problems, int S, float alpha, float beta, const float *bias, int64_t bias_stride,
                         int bias_mode, int act, hipStream_t stream) {
#define TG_COMBINE(P) launch_combine_p<P>(W, C, M, N, ldc, sC, problems, S, alpha, beta, bias, bias_stride, bias_mode, act, stream)
    if (S <= 2) return TG_COMBINE(2);
    if (S <= 4) return TG_COMBINE(4);
    if (S <= 8) return TG_COMBINE(8);
    if (S <= 16) return TG_COMBINE(16);
    if (S <= 32) return TG_COMBINE(32);
    if (S <= 64) return TG_COMBINE(64);
#undef TG_COMBINE
    return TG_ERR_INTERNAL;
}

tg_status launch_pack_rows(int esz, const void *src, int64_t ld, int64_t stride, void *dst, int64_t ld_out,
                           int64_t rows, int64_t cols, int64_t total_rows, hipStream_t s);

tg_status run(int64_t batch, int64_t M, int64_t N, int64_t K, tg_dtype dtype,
              const void *A, int64_t lda, int64_t sA, const void *B, int64_t ldb, int64_t sB,
              float *C, int64_t ldc, int64_t sC, float alpha, float beta, void *stream,
              const tg_options *opt) {
    tg_status st = validate(batch, M, N, K, dtype, A, lda, sA, B, ldb, sB, C, ldc, sC);
    if (st != TG_OK) return st;
    Plan plan;
    st = make_plan(batch, M, N, K, dtype, opt, lda, reinterpret_cast<uintptr_t>(A) % 16 == 0, ldb,
                   ldb % 2 != 0 || reinterpret_cast<uintptr_t>(B) % 4 != 0, plan);
    if (st != TG_OK) return st;
    // the fused tail (modes validated by make_plan): the caller's struct may predate it
    tg_options to{};
    if (opt) std::memcpy(&to, opt, opt->struct_size < (int)sizeof to ? (size_t)opt->struct_size : sizeof to);
    if ((to.bias_mode == 0) != (to.bias == nullptr)) return TG_ERR_INVALID_ARG;
    if (batch == 0 || M == 0 || N == 0) return TG_OK;
    if (!offsets_fit(plan.info, K, lda, ldb, ldc, dtype == TG_F32 ? 4 : 2)) return TG_ERR_UNSUPPORTED;
    const bool split = plan.info.split_k > 1;
    const bool pack = plan.info.pack_a != 0;
    const bool pack_b = plan.info.pack_b != 0;
    const bool tail_ws = plan.tail_n.ws_bytes > 0 || plan.tail_m.ws_bytes > 0 || plan.info.strip_splits > 1;
    if (split || pack || pack_b || tail_ws) {
        // a forced split or repack needs the workspace; an automatic one only happens with it
        if (!plan.workspace || plan.workspace_given < plan.info.workspace_bytes ||
            reinterpret_cast<uintptr_t>(plan.workspace) % 16)
            return TG_ERR_INVALID_ARG;
        const int esz = dtype == TG_F32 ? 4 : 2;
        const Range rw{reinterpret_cast<uintptr_t>(plan.workspace),
                       reinterpret_cast<uintptr_t>(plan.workspace) + (uintptr_t)plan.info.workspace_bytes};
        if (overlaps(rw, span(A, batch, M, K, lda, sA, esz)) || overlaps(rw, span(B, batch, K, N, ldb, sB, esz)) ||
            overlaps(rw, span(C, batch, M, N, ldc, sC, 4)))
            return TG_ERR_INVALID_ARG;
        if (split && !offsets_fit(plan.info, plan.info.k_slice, lda, ldb, N, esz)) return TG_ERR_UNSUPPORTED;
        const int64_t ldb_used = pack_b ? plan.ldb_packed : ldb;
        if (pack && (!offsets_fit(plan.info, K, plan.lda_packed, ldb_used, ldc, esz) || batch * M > 0x7fffffffLL))
            return TG_ERR_UNSUPPORTED;
        if (pack_b && (!offsets_fit(plan.info, K, pack ? plan.lda_packed : lda, ldb_used, ldc, esz) ||
                       batch * K > 0x7fffffffLL))
            return TG_ERR_UNSUPPORTED;
    }
    st = current_device_ok();
    if (st != TG_OK) return st;

    if (to.bias_mode != 0) {
        const int64_t len = to.bias_mode == 1 ? N : M;
        const Range rb{reinterpret_cast<uintptr_t>(to.bias),
                       reinterpret_cast<uintptr_t>(to.bias + (batch - 1) * to.bias_stride + len)};
        if (overlaps(rb, span(C, batch, M, N, ldc, sC, 4))) return TG_ERR_INVALID_ARG;
    }

    GemmParams gp;
    gp.A = static_cast<const char *>(A);
    gp.B = static_cast<const char *>(B);
    gp.C = C;
    gp.M = M;
    gp.N = N;
    gp.K = K;
    gp.lda = lda;
    gp.ldb = ldb;
    gp.ldc = ldc;
    gp.sA = sA;
    gp.sB = sB;
    gp.sC = sC;
    gp.tiles_m = plan.info.tiles_m;
    gp.tiles_n = plan.info.tiles_n;
    gp.batch = batch;
    gp.alpha = alpha;
    gp.beta = beta;
    gp.block_order = plan.info.block_order;
    // Tile rows per group of the XCD-grouped order: each XCD's 32 concurrent
    // tiles are group_m rows by 32 / group_m columns.  Four rows (4 A and 8 B
    // panels per K step, the A panels' 64-byte row segments being the costlier
    // copies) measured 2.6% faster than eight at 8192^3 and with a ragged K,
    // but slower with a fringe tile row (8191 x 8192 x 8192: 1%) and with thin
    // strips (8191 x 8193 x 8192: 3.5%; 8191 x 8193 x 8190: 2%): four only when
    // every 256 x 256 tile is whole.
    gp.group_m = plan.info.config == TG_CFG_256x256 && M % 256 == 0 && N % 256 == 0 ? 4 : 8;
    gp.splits = plan.info.split_k;
    gp.problems = batch;
    gp.k_slice = plan.info.k_slice;
    gp.W = static_cast<float *>(plan.workspace);
    gp.strip_n = plan.strip_n;
    gp.strip_m = plan.strip_m;
    gp.n_main = plan.info.tiles_n * plan.info.block_n;
    gp.m_main = plan.info.tiles_m * plan.info.block_m;
    gp.strip_splits = plan.info.strip_splits;
    gp.strip_k_slice = plan.strip_k_slice;
    gp.strip_rows_n = plan.strip_rows_n;
    gp.Ws = plan.info.strip_splits > 1
                ? reinterpret_cast<float *>(static_cast<char *>(plan.workspace) + plan.strip_ws_offset)
                : nullptr;
    gp.bias = to.bias;
    gp.bias_stride = to.bias_stride;
    gp.bias_mode = to.bias_mode;
    gp.act = to.activation;
    if (split) gp.batch = batch * plan.info.split_k;   // (slice, problem) pairs
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (pack) {
        // A -> aligned rows of lda_packed elements in the workspace, then the GEMM on that copy
        st = launch_pack_rows(2, A, lda, sA, plan.workspace, plan.lda_packed, M, K, batch * M, s);
        if (st != TG_OK) return st;
        gp.A = static_cast<const char *>(plan.workspace);
        gp.lda = plan.lda_packed;
        gp.sA = M * plan.lda_packed;
        gp.W = nullptr;
    }
    if (pack_b) {
        // B -> aligned rows of ldb_packed elements after the A copy
        char *dst = static_cast<char *>(plan.workspace) + plan.b_offset;
        st = launch_pack_rows(2, B, ldb, sB, dst, plan.ldb_packed, K, N, batch * K, s);
        if (st != TG_OK) return st;
        gp.B = dst;
        gp.ldb = plan.ldb_packed;
        gp.sB = K * plan.ldb_packed;
        gp.W = nullptr;
    }
    // the fused tail in the GEMM's own epilogue; a split call leaves it to the combine
    const bool tail = (to.bias_mode != 0 || to.activation != 0) && !split;
    switch (dtype) {
        case TG_BF16: st = launch_gemm_bf16(gp, plan.info, s, tail); break;
        case TG_F16: st = launch_gemm_f16(gp, plan.info, s, tail); break;
        case TG_F32: st = launch_gemm_f32(gp, plan.info, s, tail); break;
        default: return TG_ERR_INVALID_ARG;
    }
    if (st != TG_OK) return st;
    if (split)
        return launch_combine(gp.W, C, M, N, ldc, sC, batch, plan.info.split_k, alpha, beta, to.bias,
                              to.bias_stride, to.bias_mode, to.activation, s);
    if (plan.info.strip_splits > 1) {
        // the strip regions' partials: N strips (rows [0, strip_rows_n), columns
        // [n_main, N)), then M strips (rows [m_main, M), all columns)
        const int S = plan.info.strip_splits;
        const int64_t wn = N - gp.n_main, rows_m = M - gp.m_main;
        const float *bias_n = to.bias_mode == 1 ? to.bias + gp.n_main : to.bias;
        const float *bias_m = to.bias_mode == 2 ? to.bias + gp.m_main : to.bias;
        if (plan.strip_n) {
            st = launch_combine(gp.Ws, C + gp.n_main, gp.strip_rows_n, wn, ldc, sC, batch, S, alpha, beta, bias_n,
                                to.bias_stride, to.bias_mode, to.activation, s);
            if (st != TG_OK) return st;
        }
        if (plan.strip_m) {
            const float *w = gp.Ws + (plan.strip_n ? (int64_t)S * batch * gp.strip_rows_n * wn : 0);
            st = launch_combine(w, C + gp.m_main * ldc, rows_m, N, ldc, sC, batch, S, alpha, beta, bias_m,
                                to.bias_stride, to.bias_mode, to.activation, s);
            if (st != TG_OK) return st;
        }
    }
    // the thin remainders' own GEMMs (on the A copy when there is one)
    for (const Tail *t : {&plan.tail_n, &plan.tail_m}) {
        if (t->splits == 0) continue;
        tg_options sub{};
        sub.struct_size = (int)sizeof sub;
        sub.force_cfg = TG_CFG_64x64;
        sub.split_k = (int)t->splits;
        sub.workspace = t->ws_bytes ? static_cast<char *>(plan.workspace) + t->ws_offset : nullptr;
        sub.workspace_bytes = t->ws_bytes;
        sub.pack_a = 1;
        sub.tail_gemm = 1;
        // the remainder's own slice of a per-column / per-row bias
        sub.bias = to.bias_mode == 1 ? to.bias + t->n0 : (to.bias_mode == 2 ? to.bias + t->m0 : nullptr);
        sub.bias_stride = to.bias_stride;
        sub.bias_mode = to.bias_mode;
        sub.activation = to.activation;
        sub.pack_b = 1;
        st = run(batch, t->rows, t->cols, K, dtype, gp.A + t->m0 * gp.lda * 2, gp.lda, gp.sA, gp.B + t->n0 * 2,
                 gp.ldb, gp.sB, C + t->m0 * ldc + t->n0, ldc, sC, alpha, beta, stream, &sub);
        if (st != TG_OK) return st;
    }
    return TG_OK;
}

// Hoisted pack of B (tile_gemm.h): rows of a multiple of 16 bytes.

// Threads per row for pack_rows_kernel: whole waves, enough for the row's chunks.
int pack_group(int64_t chunks) { return chunks > 128 ? 256 : (chunks > 64 ? 128 : 64); }

tg_status launch_pack_rows(int esz, const void *src, int64_t ld, int64_t stride, void *dst, int64_t ld_out,
                           int64_t rows, int64_t cols, int64_t total_rows, hipStream_t s) {
    const int group = pack_group(ld_out * esz / 16);
    const int64_t blocks = cdiv(total_rows, 256 / group);
    if (blocks > 0x7fffffffLL || ld_out * esz > 0x7fffffffLL) return TG_ERR_UNSUPPORTED;
    if (esz == 4)
        hipLaunchKernelGGL(pack_rows_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, s,
                           static_cast<const char *>(src), ld, stride, static_cast<char *>(dst), ld_out, rows, cols,
                           total_rows, group);
    else
        hipLaunchKernelGGL(pack_rows_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, s,
                           static_cast<const char *>(src), ld, stride, static_cast<char *>(dst), ld_out, rows, cols,
                           total_rows, group);
    return hipGetLastError() == hipSuccess ? TG_OK : TG_ERR_LAUNCH;
}
int64_t packed_ld(int64_t N, tg_dtype dtype) {
    const int64_t per = dtype == TG_F32 ? 4 : 8;     // elements per 16 bytes
    const int64_t n = N > 1 ? N : 1;
    return (n + per - 1) / per * per;
}

tg_status packed_bytes_of(int64_t batch, int64_t K, int64_t N, tg_dtype dtype, int64_t &bytes) {
    if (batch < 0 || K < 0 || N < 0) return TG_ERR_INVALID_ARG;
    if (dtype != TG_F32 && dtype != TG_BF16 && dtype != TG_F16) return TG_ERR_INVALID_ARG;
    const int64_t esz = dtype == TG_F32 ? 4 : 2, ldp = packed_ld(N, dtype);
    if (N > (int64_t(1) << 40) || K > (int64_t(1) << 40) || batch > (int64_t(1) << 40) ||
        (K > 0 && batch > (int64_t(1) << 60) / K / ldp / esz))
        return TG_ERR_INVALID_ARG;
    bytes = batch * K * ldp * esz;
    return TG_OK;
}

tg_status pack_b(int64_t batch, int64_t K, int64_t N, tg_dtype dtype, const void *B, int64_t ldb, int64_t sB,
                 int transposed, void *packed, int64_t packed_size, void *stream) {
    int64_t bytes = 0;
    tg_status st = packed_bytes_of(batch, K, N, dtype, bytes);
    if (st != TG_OK) return st;
    if (transposed != 0 && transposed != 1) return TG_ERR_INVALID_ARG;
    if (batch == 0 || K == 0 || N == 0) return TG_OK;
    const int esz = dtype == TG_F32 ? 4 : 2;
    const int64_t rows = transposed ? N : K, cols = transposed ? K : N;   // the source as stored
    if (!B || !packed || ldb < cols || sB < 0) return TG_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(packed) % 256 || packed_size < bytes) return TG_ERR_INVALID_ARG;
    const Range rp{reinterpret_cast<uintptr_t>(packed), reinterpret_cast<uintptr_t>(packed) + (uintptr_t)bytes};
    if (overlaps(span(B, batch, rows, cols, ldb, sB, esz), rp)) return TG_ERR_INVALID_ARG;
    const int64_t ldp = packed_ld(N, dtype);
    if (ldp * esz > 0x7fffffffLL) return TG_ERR_UNSUPPORTED;
    st = current_device_ok();
    if (st != TG_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!transposed) return launch_pack_rows(esz, B, ldb, sB, packed, ldp, K, N, batch * K, s);
    {
        const int64_t gk = cdiv(K, 64), gn = cdiv(ldp, 64);
        if (gk > 0x7fffffffLL || gn > 65535 || batch > 65535) return TG_ERR_UNSUPPORTED;
        const dim3 grid((unsigned)gk, (unsigned)gn, (unsigned)batch);
        if (esz == 4)
            hipLaunchKernelGGL(pack_transposed_kernel<uint32_t>, grid, dim3(256), 0, s,
                               static_cast<const uint32_t *>(B), ldb, sB, static_cast<uint32_t *>(packed), ldp, K, N);
        else
            hipLaunchKernelGGL(pack_transposed_kernel<uint16_t>, grid, dim3(256), 0, s,
                               static_cast<const uint16_t *>(B), ldb, sB, static_cast<uint16_t *>(packed), ldp, K, N);
    }
    return hipGetLastError() == hipSuccess ? TG_OK : TG_ERR_LAUNCH;
}

// tile_gemm_ex_noalloc (tile_gemm.h): the plan tile_gemm_ex would make with a
// workspace of the scratch's size, checked against that size before any device
// work, then the same call with the scratch as its workspace.
tg_status run_noalloc(int64_t batch, int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                      const void *A, int64_t lda, int64_t sA, const void *B, int64_t ldb, int64_t sB,
                      float *C, int64_t ldc, int64_t sC, float alpha, float beta, void *stream,
                      const tg_options *opt) {
    tg_options o{};
    if (opt) {
        if (opt->struct_size < kOptionsV1Size) return TG_ERR_INVALID_ARG;
        std::memcpy(&o, opt, opt->struct_size < (int)sizeof o ? (size_t)opt->struct_size : sizeof o);
    }
    if (o.workspace != nullptr || o.workspace_bytes != 0) return TG_ERR_INVALID_ARG;
    o.struct_size = (int)sizeof o;
    tg_status st = validate(batch, M, N, K, dtype, A, lda, sA, B, ldb, sB, C, ldc, sC);
    if (st != TG_OK) return st;
    {
        // the plan only asks whether a workspace is there and how large it is
        tg_options q = o;
        q.workspace = reinterpret_cast<void *>(uintptr_t(256));
        q.workspace_bytes = TILE_GEMM_NOALLOC_SCRATCH_BYTES;
        Plan plan;
        st = make_plan(batch, M, N, K, dtype, &q, lda, reinterpret_cast<uintptr_t>(A) % 16 == 0, ldb,
                       ldb % 2 != 0 || reinterpret_cast<uintptr_t>(B) % 4 != 0, plan);
        if (st != TG_OK) return st;
        if (plan.info.workspace_bytes > TILE_GEMM_NOALLOC_SCRATCH_BYTES) return TG_ERR_SCRATCH_LIMIT;
    }
    if (batch == 0 || M == 0 || N == 0) return TG_OK;
    st = current_device_ok();
    if (st != TG_OK) return st;
    void *ws = nullptr;
    st = current_device_scratch(&ws);
    if (st != TG_OK) return st;
    o.workspace = ws;
    o.workspace_bytes = TILE_GEMM_NOALLOC_SCRATCH_BYTES;
    return run(batch, M, N, K, dtype, A, lda, sA, B, ldb, sB, C, ldc, sC, alpha, beta, stream, &o);
}

// The leading dimension the plan queries assume for A (or B): plan_lda
// (plan_ldb) when the caller's struct has it and it is positive, else 8 (a
// multiple of 8: aligned rows).
int64_t plan_ld(const tg_options *opt, bool a) {
    if (!opt) return 8;
    const size_t need = a ? offsetof(tg_options, plan_lda) + sizeof(int64_t) : offsetof(tg_options, plan_ldb) + sizeof(int64_t);
    if (opt->struct_size < (int)need) return 8;
    const int64_t ld = a ? opt->plan_lda : opt->plan_ldb;
    return ld > 0 ? ld : 8;
}

}  // namespace

extern "C" {

tg_status tile_gemm_ex(int64_t batch, int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                       const void *A, int64_t lda, int64_t strideA,
                       const void *B, int64_t ldb, int64_t strideB,
                       float *C, int64_t ldc, int64_t strideC,
                       float alpha, float beta, void *stream, const tg_options *opt) {
    try {
        return run(batch, M, N, K, dtype, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, alpha, beta,
                   stream, opt);
    } catch (...) {
        return TG_ERR_INTERNAL;
    }
}

tg_status tile_gemm_ex_noalloc(int64_t batch, int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                               const void *A, int64_t lda, int64_t strideA,
                               const void *B, int64_t ldb, int64_t strideB,
                               float *C, int64_t ldc, int64_t strideC,
                               float alpha, float beta, void *stream, const tg_options *opt) {
    try {
        return run_noalloc(batch, M, N, K, dtype, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, alpha, beta,
                           stream, opt);
    } catch (...) {
        return TG_ERR_INTERNAL;
    }
}

tg_status tile_gemm_strided_batched(int64_t batch, int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                                    const void *A, int64_t lda, int64_t strideA,
                                    const void *B, int64_t ldb, int64_t strideB,
                                    float *C, int64_t ldc, int64_t strideC,
                                    float alpha, float beta, void *stream) {
    return tile_gemm_ex(batch, M, N, K, dtype, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, alpha, beta,
                        stream, nullptr);
}

tg_status tile_gemm(int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                    const void *A, int64_t lda, const void *B, int64_t ldb,
                    float *C, int64_t ldc, float alpha, float beta, void *stream) {
    return tile_gemm_ex(1, M, N, K, dtype, A, lda, 0, B, ldb, 0, C, ldc, 0, alpha, beta, stream, nullptr);
}

tg_status tile_gemm_plan(int64_t batch, int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                         const tg_options *opt, tg_plan_info *out) {
    if (!out) return TG_ERR_INVALID_ARG;
    try {
        Plan p;
        const int64_t ldb = plan_ld(opt, false);
        tg_status st = make_plan(batch, M, N, K, dtype, opt, plan_ld(opt, true), true, ldb, ldb % 2 != 0, p);
        if (st == TG_OK) *out = p.info;
        return st;
    } catch (...) {
        return TG_ERR_INTERNAL;
    }
}

tg_status tile_gemm_workspace_size(int64_t batch, int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                                   const tg_options *opt, int64_t *bytes) {
    if (!bytes) return TG_ERR_INVALID_ARG;
    try {
        Plan p;
        const int64_t ldb = plan_ld(opt, false);
        tg_status st = make_plan(batch, M, N, K, dtype, opt, plan_ld(opt, true), true, ldb, ldb % 2 != 0, p);
        if (st == TG_OK) *bytes = p.wanted_workspace;
        return st;
    } catch (...) {
        return TG_ERR_INTERNAL;
    }
}

const char *tile_gemm_status_string(tg_status s) {
    switch (s) {
        case TG_OK: return "TG_OK";
        case TG_ERR_INVALID_ARG: return "TG_ERR_INVALID_ARG: extents, strides, pointers, dtype or overlap rejected";
        case TG_ERR_UNSUPPORTED: return "TG_ERR_UNSUPPORTED: no gfx950 device visible, or option not available";
        case TG_ERR_LAUNCH: return "TG_ERR_LAUNCH: the HIP runtime refused the kernel launch";
        case TG_ERR_INTERNAL: return "TG_ERR_INTERNAL: unexpected failure inside the library";
        case TG_ERR_SCRATCH_LIMIT:
            return "TG_ERR_SCRATCH_LIMIT: the call needs more scratch than tile_gemm_ex_noalloc holds "
                   "(TILE_GEMM_NOALLOC_SCRATCH_BYTES)";
    }
    return "unknown tg_status";
}

int tile_gemm_abi_version(void) { return TILE_GEMM_ABI_VERSION; }

int64_t tile_gemm_packed_b_ld(int64_t N, tg_dtype dtype) {
    if (N < 0 || (dtype != TG_F32 && dtype != TG_BF16 && dtype != TG_F16)) return -1;
    return packed_ld(N, dtype);
}

tg_status tile_gemm_packed_b_size(int64_t batch, int64_t K, int64_t N, tg_dtype dtype, int64_t *bytes) {
    if (!bytes) return TG_ERR_INVALID_ARG;
    int64_t b = 0;
    const tg_status st = packed_bytes_of(batch, K, N, dtype, b);
    if (st == TG_OK) *bytes = b;
    return st;
}

tg_status tile_gemm_pack_b(int64_t batch, int64_t K, int64_t N, tg_dtype dtype, const void *B, int64_t ldb,
                           int64_t strideB, int transposed, void *packed, int64_t packed_bytes, void *stream) {
    try {
        return pack_b(batch, K, N, dtype, B, ldb, strideB, transposed, packed, packed_bytes, stream);
    } catch (...) {
        return TG_ERR_INTERNAL;
    }
}

}  // extern "C"
