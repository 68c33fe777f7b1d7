/*
 * tile_gemm.h -- C ABI of the MI355X (gfx950) tiled dense contraction.
 *
 *     C[b] <- alpha * A[b] . B[b] + beta * C[b]          (row-major, any extents)
 *
 * The operation is the matmul micro-kernel d[i,j] += a[i,k] * b[k,j] that the
 * OCANNL "Module Ir.Schedule" page tensorizes (Tensorize paragraph: operands
 * row-major in their last two axes, not transposed), equivalently
 * acc = mma(a, b, acc) over a reduce region in LuisaCompute "Execution Nests and
 * coordinates" (structured-region calculus; logical anchor and frontier).  The
 * schedule it is built with -- pad-to-tile, partition into interior and fringe
 * blocks, staging through a swizzled on-chip tile, a window-2 software pipeline
 * over K, tensorized multiply-accumulate -- changes how the value is reached,
 * not the value, except that the k sum may be regrouped (the Interchange
 * paragraph of the OCANNL page; reduce's regrouping permission on the
 * LuisaCompute page).
 *
 * Conventions shared by every entry point
 *  - Element (i, k) of A is A[i*lda + k]; (k, j) of B is B[k*ldb + j]; (i, j) of
 *    C is C[i*ldc + j].  Leading dimensions and batch strides count ELEMENTS.
 *  - A and B have the same dtype (fp32, bf16 or fp16).  C is always fp32, and
 *    the products are accumulated in fp32.
 *  - beta == 0: C is write-only (it is not read, so NaN in C does not leak).
 *  - M == 0, N == 0 or batch == 0: nothing is launched, TG_OK.
 *    K == 0: C <- beta * C (zeros when beta == 0).
 *  - No alignment requirement: any lda/ldb/ldc, and A/B pointers need only be
 *    aligned to their element size, C to 4 bytes.
 *  - Device pointers.  The caller owns every buffer; the library never
 *    allocates, frees or keeps a pointer past the call.  Work is enqueued
 *    asynchronously on `stream` (a hipStream_t passed as void*, 0 = the null
 *    stream); buffers must stay alive until the stream reaches the work.
 *  - C must not overlap A or B (the source of a staged tile must not be
 *    written by the routine: OCANNL Stage paragraph).  Overlap is checked on
 *    the address ranges and rejected.
 *  - Errors are returned, never printed, and no C++ exception crosses the ABI.
 *    Argument errors are detected before any device work.  A device fault
 *    surfaces, as usual in HIP, at the caller's next synchronisation.
 *  - The library is stateless apart from a lazily filled, lock-protected cache
 *    of per-device properties; it is safe to call from several host threads.
 */
#ifndef TILE_GEMM_H
#define TILE_GEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TILE_GEMM_ABI_VERSION 11

typedef enum { TG_F32 = 0, TG_BF16 = 1, TG_F16 = 2 } tg_dtype;

/*
 * Every call reports its outcome as a tg_status and never prints or aborts.
 * A schedule operation that cannot apply fails loudly rather than computing
 * something else (OCANNL "Module Ir.Schedule", Interchange paragraph), and a
 * target refuses an execution scope it does not have rather than substituting
 * one (LuisaCompute "Execution Nests and coordinates", Ordering strength and
 * sibling scopes); a status of its own for each kind of refusal is that rule
 * across a C boundary.
 */
typedef enum {
    TG_OK = 0,
    TG_ERR_INVALID_ARG = 1,  /* extents, strides, pointers, dtype or overlap rejected */
    TG_ERR_UNSUPPORTED = 2,  /* no visible gfx950 device, an option not built, or a  */
                             /* block's tile of A, B or C spanning 2^31 bytes or more */
    TG_ERR_LAUNCH = 3,       /* the HIP runtime refused the launch */
    TG_ERR_INTERNAL = 4,     /* unexpected failure inside the library */
    TG_ERR_SCRATCH_LIMIT = 5 /* tile_gemm_ex_noalloc: the call needs more scratch than the library holds */
} tg_status;

/*
 * C = alpha * A . B + beta * C for one M x N x K problem.
 * A: M x K (lda >= max(1, K)); B: K x N (ldb >= max(1, N)); C: M x N fp32
 * (ldc >= max(1, N)).  Pointers may be NULL only where their extent is empty.
 */
tg_status tile_gemm(int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                    const void *A, int64_t lda, const void *B, int64_t ldb,
                    float *C, int64_t ldc, float alpha, float beta, void *stream);

/*
 * `batch` independent problems in one launch: problem b uses A + b*strideA,
 * B + b*strideB and C + b*strideC (element strides, >= 0).  The C ranges of
 * distinct b must not overlap each other (checked).  A stride of 0 shares an
 * operand across the batch.  The batch is one more independent parallel axis
 * of the same contraction: the problems are disjoint children of a `parallel`
 * region (LuisaCompute "Execution Nests and coordinates", structured-region
 * calculus), so they run in one launch with no ordering between them.
 */
tg_status tile_gemm_strided_batched(int64_t batch, int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                                    const void *A, int64_t lda, int64_t strideA,
                                    const void *B, int64_t ldb, int64_t strideB,
                                    float *C, int64_t ldc, int64_t strideC,
                                    float alpha, float beta, void *stream);

/* Schedule knobs, for tests and measurements; zero-initialise for defaults.
 * The tile configurations are block tiles of the M and N loops (OCANNL "Module
 * Ir.Schedule", Split paragraph) with their MFMA register tiles (Tensorize). */
typedef enum {
    TG_CFG_AUTO = 0,
    TG_CFG_256x256 = 1,     /* 256x256 block tile on the LDS ring, 4 waves: 16x16x32 MFMA for
                               16-bit inputs, 16x16x4 for fp32 (version 9 and later) */
    TG_CFG_128x128 = 2,     /* 128x128 block tile on the LDS ring, 4 waves: 32x32x16 MFMA for
                               16-bit inputs, 16x16x4 for fp32 (version 9 and later) */
    TG_CFG_64x64 = 3,       /* 16-bit inputs: 64x64 block tile, 2 waves          */
    TG_CFG_F32_64x64 = 4,   /* fp32 inputs: 64x64 block tile, 4 waves, staged through
                               registers (small problems; no split-K)           */
    TG_CFG_288x160 = 5      /* 16-bit inputs: 288x160 block tile, 4 waves, 16x16x32: one
                               block per problem of up to 288 x 160 (batched small GEMMs) */
} tg_config;

/*
 * Options.  struct_size is sizeof(tg_options) of the caller's header; it must
 * cover at least the first five fields (20 bytes, the version-1 layout), and
 * fields past it read as zero.
 *
 * pipeline_depth is the number of LDS copies of the K tile (the window is one
 * less; OCANNL "Module Ir.Schedule", Stage paragraph, pipeline_depth, and
 * LuisaCompute "Pipelines and stage boundaries", window): 16-bit inputs take 1,
 * 2 or 4 (default 4; 5 for TG_CFG_128x128 and TG_CFG_64x64; 2 or 4 for
 * TG_CFG_288x160), and so do fp32 inputs on TG_CFG_128x128 (on TG_CFG_256x256:
 * 2 or 4); fp32 inputs on TG_CFG_F32_64x64 take 1 or 2 (default 2).  Depth 1 is the
 * unpipelined form.
 *
 * swizzle is the placement of the staged tiles in LDS (OCANNL Stage paragraph,
 * swizzle and pad_stride; TVM TIRx "Tensor Layout", SwizzleLayout): 0 the
 * default (XOR); 1 none, the row-major tile; 2 pad_stride, the row-major tile
 * with its minor dimension rounded up by one 16-byte unit (A rows of 32 k at a
 * pitch of 40, B rows of BN n at BN + 8; built for TG_CFG_256x256 with 16-bit
 * inputs at depth 4, UNSUPPORTED elsewhere); 3 the XOR swizzle of 16-byte units (Swizzle_b128
 * flavour).  Placement changes which LDS bytes hold a value, never the value:
 * every placement gives a bitwise identical C.  (Version 7 and earlier: 2 was
 * the XOR swizzle.)
 *
 * Split-K (16-bit inputs, and fp32 inputs on the ring tiles): the
 * deterministic two-pass split reduction of the OCANNL "Module Ir.Schedule"
 * page (paragraph of that name).  The K range is
 * cut into S slices of a multiple of block_k elements (the last one shorter);
 * each slice's product goes, unscaled, to its own fp32 M x N partial in
 * `workspace` (slice s of problem b at float offset (s * batch + b) * M * N),
 * written whole by the first kernel (no zeroing pass); a second kernel then
 * adds the S partials of every element in a fixed balanced-tree order and
 * applies the epilogue, fma(alpha, sum, beta * C0) or alpha * sum.  The result
 * is bitwise reproducible for a given (config, S) but, as that paragraph
 * notes, not bitwise equal to the unsplit sum (the k sum is regrouped).
 *   split_k == 0: automatic -- split only when the plan has too few output
 *                 tiles to fill the GPU, K is deep, and `workspace` holds the
 *                 partials (tile_gemm_workspace_size says how many bytes);
 *                 without a forced config, each tile size is weighed with its
 *                 own split and the one whose workgroups best fill the GPU
 *                 (ties: the larger tile) is taken;
 *   split_k == 1: never split;
 *   split_k >= 2: at most split_k slices (fewer when K is short); the call
 *                 fails with TG_ERR_INVALID_ARG if the workspace is too small.
 * Repack of A (16-bit inputs, TG_CFG_256x256, no split): when A's rows do not
 * start on 16-byte boundaries (lda not a multiple of 8, or A itself not
 * 16-byte aligned), every 16-byte copy of an A tile straddles cache lines.  A
 * first kernel then copies A into `workspace` with rows of roundup(K, 8)
 * elements (batch entries packed, zero past K), and the GEMM reads that copy;
 * the values and the MFMA sequence are unchanged, so the result is bitwise the
 * unpacked one.
 *   pack_a == 0: automatic -- repack when the rows are misaligned, the plan
 *                has at least 8 tile columns (each A panel is read by that many
 *                workgroups), and `workspace` holds the copy;
 *   pack_a == 1: never;  pack_a == 2: always (TG_ERR_INVALID_ARG without the
 *                workspace; TG_ERR_UNSUPPORTED for another configuration).
 * plan_lda is the lda that tile_gemm_plan and tile_gemm_workspace_size assume
 * (0: a multiple of 8); tile_gemm_ex uses its own lda and A.
 * Repack of B: the same for B's rows when they are only 2-byte aligned (an odd
 * ldb, or B itself on an odd 2-byte boundary) and the plan has at least 8 tile
 * rows; B is copied into `workspace` after the A copy, with rows of
 * roundup(N, 8) elements (batch entries packed, zero past N).  pack_b 0 / 1 / 2
 * as pack_a (2 also for rows on 4- or 8-byte boundaries); plan_ldb is the ldb
 * the plan queries assume (0: a multiple of 8).
 * Thin remainders (TG_CFG_256x256): an N tail of at most 64 columns (N >= 256)
 * and an M tail of at most 64 rows (M >= 256) are fringe partitions of their
 * own (OCANNL "Module Ir.Schedule": index-set splitting of a block loop at
 * its last full tile, the Partition of a padded loop).  By default they run
 * as narrow strip blocks in the main grid.  On request the remainder is
 * computed instead by a second GEMM on TG_CFG_64x64: C[:, n0:N] from
 * A . B[:, n0:N] over all M rows for the N tail, C[m0:M, 0:n1] from
 * A[m0:M, :] . B[:, 0:n1] for the M tail (n1 = N, or n0 when the N tail has
 * its own GEMM), split along K as above when the workspace also holds its
 * partials (after the A copy, N tail first).  The value is the same
 * contraction; the tail's k sum may be regrouped by its split.
 *   tail_gemm == 0: strips in the grid, split along K as for tail_gemm == 3
 *                   when the whole strips would run after the main tiles as a
 *                   part-filled round of their own (the main tiles end a whole
 *                   round of 256 workgroups, or leave fewer free slots in their
 *                   last round than there are strips) and `workspace` holds the
 *                   partials; otherwise whole;
 *   tail_gemm == 1: strips in the grid, whole;
 *   tail_gemm == 2: the remainder GEMMs whenever there is a thin remainder;
 *   tail_gemm == 3: strips in the grid, each split along K into S slices (K
 *                   slices of a multiple of 32, S up to 16) that write unscaled
 *                   partials into `workspace` (after the copies of A and B),
 *                   and a combine pass over the strip region adds them in the
 *                   fixed tree order of the split reduction and applies the
 *                   epilogue and fused tail (the strips' k sum is regrouped);
 *                   unsplit when the workspace is too small.
 * Persistent workgroups (16-bit, TG_CFG_256x256, depth 4, XOR swizzle, the
 * grouped block order, one problem, no split, no repack, no strips, every
 * tile interior (M and N multiples of 256), K a multiple of 128 and at least
 * 256, at least 512 tiles): 256 workgroups each take every 256th tile, and
 * the software pipeline over K runs on from one tile into the next (the next
 * tile's first K tiles are copied during the current tile's last ones).  The
 * same MFMA sequence per tile: bitwise the plain grid's result.  Not the
 * default: a wave's loads and stores share one in-order completion count, so
 * the copies a workgroup issues after a tile's C stores can only be waited
 * for once those stores are done, which a fresh workgroup of the plain grid
 * never waits for (8192^3 bf16: 0.797 ms against 0.783 ms).
 * Two batch entries per workgroup (16-bit, TG_CFG_288x160, depth 4, XOR
 * swizzle, every entry one block of the tile, no split, no repack, more than
 * 256 and at most 512 entries, at least 4 K tiles): 256 workgroups, workgroup
 * w takes entry w and then entry w + 256; the first entry's last K iterations
 * copy the second's first K tiles, so the second does not start cold.  The
 * same MFMA sequence per entry: bitwise the plain grid's result.  This is the
 * automatic choice where it applies (512 x 257x129x1000 f16: 111.8 against
 * 114.9 us for the kernel).
 *   persistent == 0: the plain grid, or two entries per workgroup where that applies;
 *   persistent == 1: the plain grid;
 *   persistent == 2: as 0, and persistent workgroups where their conditions hold.
 * Fused elementwise tail (OCANNL "Module Ir.Schedule", epilogue fusion: the
 * bias add / activation / residual that follows a reduction, folded into its
 * store-back): with bias_mode or activation nonzero every output is
 *     C <- act(alpha * A.B + bias) + beta * C0
 * computed as y = act(fma(alpha, acc, bias)), then fma(beta, C0, y) (C0 not
 * read when beta == 0), in fp32.  bias_mode 1: bias[j], one value per column
 * (N floats per problem); 2: bias[i], one per row (M floats); problem b reads
 * its vector at bias + b * bias_stride (0 = one vector shared by the batch).
 * activation 1: ReLU, x < 0 ? 0 : x (NaN passes through); 2: GELU in its exact
 * form x * Phi(x) = x/2 * (1 + erf(x / sqrt(2))), Phi evaluated through a
 * Chebyshev fit of erfc with fractional error below 1.2e-7 (Numerical Recipes,
 * section 6.2): the fp32 result is within 2.4e-7 |x| of x * Phi(x).
 * Without them the epilogue is fma(alpha, acc, beta * C0) as before.  The
 * bias must be 4-byte aligned, non-NULL exactly when bias_mode != 0, and
 * must not overlap C (tile_gemm_plan and tile_gemm_workspace_size do not read
 * it: for them the modes alone shape the plan, and a NULL bias is accepted).
 * Every tile configuration carries the tail in its own store-back at the
 * default pipeline depth and swizzle (others: TG_ERR_UNSUPPORTED unless split);
 * a split call applies it once in the combine pass; the plan is otherwise the
 * one the call would take without the tail, except that persistent workgroups
 * are not used with it.
 *
 * The workspace is caller-owned device memory, 16-byte aligned, that must not
 * overlap A, B or C; its contents on entry do not matter and are undefined
 * afterwards.  Calls that share one workspace must be ordered (e.g. on one
 * stream).
 */
typedef struct {
    int struct_size;
    int force_cfg;       /* tg_config; TG_CFG_AUTO picks by dtype and shape           */
    int pipeline_depth;  /* 0 = default (see above)                                   */
    int swizzle;         /* 0 = default (XOR); 1 = none; 2 = pad_stride; 3 = XOR     */
    int block_order;     /* 0 = default (XCD-grouped); 1 = plain row-major          */
    int split_k;         /* 0 = automatic, 1 = off, S >= 2 = at most S K slices      */
    void *workspace;     /* device memory for split-K partials or the A copy, or NULL */
    int64_t workspace_bytes;
    int pack_a;          /* 0 = automatic, 1 = never, 2 = always (see above)        */
    int pad0_;
    int64_t plan_lda;    /* lda assumed by the plan queries (0: a multiple of 8)    */
    int tail_gemm;       /* 0 = strips, split when worth it; 1 = strips; 2 = GEMMs; 3 = split (above) */
    int persistent;      /* 0 automatic, 1 plain grid, 2 persistent where allowed (above) */
    const float *bias;   /* fused tail bias (see above), NULL when bias_mode == 0    */
    int64_t bias_stride; /* floats between the bias vectors of batch entries          */
    int bias_mode;       /* 0 = none, 1 = per column (bias[j]), 2 = per row (bias[i]) */
    int activation;      /* 0 = none, 1 = ReLU, 2 = GELU (erf form)                  */
    int pack_b;          /* 0 = automatic, 1 = never, 2 = always (see above)        */
    int pad1_;
    int64_t plan_ldb;    /* ldb assumed by the plan queries (0: a multiple of 8)    */
} tg_options;

/* tile_gemm_strided_batched with explicit schedule knobs (opt may be NULL).
 * Every combination computes the same value; options a build lacks return
 * TG_ERR_UNSUPPORTED. */
tg_status tile_gemm_ex(int64_t batch, int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                       const void *A, int64_t lda, int64_t strideA,
                       const void *B, int64_t ldb, int64_t strideB,
                       float *C, int64_t ldc, int64_t strideC,
                       float alpha, float beta, void *stream, const tg_options *opt);

/* ---- host-side introspection: no device needed, nothing launched ---------- */

/* The plan a call would launch (pure host arithmetic). */
typedef struct {
    int config;           /* tg_config actually chosen                             */
    int block_m, block_n, block_k;
    int waves, threads;
    int pipeline_depth, swizzle, block_order;
    int64_t tiles_m, tiles_n;     /* ceil(M / block_m), ceil(N / block_n)          */
    int64_t grid;                 /* tiles_m * tiles_n * batch workgroups          */
    int64_t interior_blocks;      /* blocks with no M/N fringe, per problem        */
    int64_t fringe_blocks;        /* blocks whose tile crosses M or N, per problem */
    int64_t k_tiles;              /* ceil(K / block_k)                             */
    int64_t k_tail;               /* K mod block_k (0: no peeled tail tile)        */
    int lds_bytes;                /* LDS per workgroup, all pipeline copies        */
    int split_k;                  /* K slices S (1: no split)                      */
    int64_t k_slice;              /* K elements per slice (the last may be shorter)*/
    int64_t workspace_bytes;      /* workspace the call uses: S * batch * M * N * 4, or the A copy
                                     plus the remainder GEMMs' partials                  */
    int mfma_m, mfma_n, mfma_k;   /* MFMA instruction shape: 32x32x16, 16x16x32 or 16x16x4 */
    int pack_a;                   /* 1: A is first copied to aligned rows in the workspace */
    int64_t strip_blocks;         /* thin fringe-strip blocks per problem (in grid) */
    int tail_n_splits;            /* 0: no N-remainder GEMM; S >= 1: one, with S K slices */
    int tail_m_splits;            /* the same for the M remainder                  */
    int persistent;               /* 1: persistent workgroups or two batch entries per
                                     workgroup (grid = their count) */
    int per_cu;                   /* workgroups of this configuration one CU holds at once
                                     (registers and LDS of the built kernel) */
    int pack_b;                   /* 1: B is first copied to aligned rows in the workspace */
    int strip_splits;             /* K slices of each strip block (1: not split)   */
} tg_plan_info;

tg_status tile_gemm_plan(int64_t batch, int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                         const tg_options *opt, tg_plan_info *out);

/* Workspace bytes a call with these arguments would use if the workspace were
 * large enough (0 when it would not split K).  With split_k == 0 this is the
 * size the automatic choice wants; pass that much to let it split. */
tg_status tile_gemm_workspace_size(int64_t batch, int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                                   const tg_options *opt, int64_t *bytes);

/*
 * Tile layouts in the TileLayout / SwizzleLayout model of the Apache TVM TIRx
 * "Tensor Layout" page (TileLayout, Forward mapping, SwizzleLayout and
 * ComposeLayout sections): a logical index is flattened row-major, split over
 * the shard iters, each component scaled by its stride onto its axis, the
 * offset added, and every replica combination added; swizzles, if present,
 * then permute the coordinate on the memory axis m, applied in order:
 *     addr(m) = f(m >> M) * 2^M + (m mod 2^M),  f(x) = x ^ ((x & ((2^B-1) << S)) >> S).
 */
#define TG_LAYOUT_MAX_ITERS 12
#define TG_LAYOUT_MAX_RANK 6
#define TG_LAYOUT_MAX_SWIZZLES 2

typedef enum { TG_AXIS_M = 0, TG_AXIS_LANE = 1, TG_AXIS_WAVE = 2, TG_AXIS_PID = 3,
               TG_AXIS_TLANE = 4, TG_AXIS_TCOL = 5, TG_AXIS_COUNT = 6 } tg_axis;

typedef struct { int64_t extent; int64_t stride; int32_t axis; int32_t pad_; } tg_iter;

typedef struct { int32_t m, b, s; } tg_swizzle;    /* SwizzleLayout(M, B, S), S >= B */

typedef struct {
    int32_t rank;                             /* logical rank                      */
    int32_t n_shard;                          /* D iters                           */
    int32_t n_replica;                        /* R iters                           */
    int32_t n_swizzle;                        /* swizzles composed after the tile  */
    int64_t shape[TG_LAYOUT_MAX_RANK];        /* logical shape                     */
    tg_iter shard[TG_LAYOUT_MAX_ITERS];
    tg_iter replica[TG_LAYOUT_MAX_ITERS];
    int64_t offset[TG_AXIS_COUNT];            /* O, one integer per axis           */
    tg_swizzle swizzle[TG_LAYOUT_MAX_SWIZZLES];
    int32_t pad_;
} tg_layout;

/*
 * Evaluate L(x) for the logical coordinate x[0..rank).  Writes up to max_out
 * coordinates (each TG_AXIS_COUNT int64s, row-major into out) and returns the
 * number of coordinates in L(x), or -1 if x or the layout is invalid (shape
 * not admitted: product of shape != product of shard extents).
 */
int64_t tg_layout_eval(const tg_layout *L, const int64_t *x, int64_t *out, int64_t max_out);

/* Layouts the kernels use, described as tg_layouts:
 *   TG_LAYOUT_LDS_A / _B : operand tile element (row, k) -> swizzled LDS element
 *                          offset within one pipeline copy (B is held as
 *                          [n][k], i.e. transposed, so both operands are
 *                          read as k-contiguous 16-byte fragments);
 *   TG_LAYOUT_ACC        : block accumulator element (row, col) -> (lane, wave,
 *                          register slot m) of the MFMA register tiles;
 *   TG_LAYOUT_COPY_A     : A tile 16-byte chunk (row, chunk) -> (lane, wave, m)
 *                          of the thread and the load slot m that copies it. */
typedef enum { TG_LAYOUT_LDS_A = 0, TG_LAYOUT_LDS_B = 1, TG_LAYOUT_ACC = 2,
               TG_LAYOUT_COPY_A = 3 } tg_layout_kind;

/* The introspection calls below take a tg_config, or one of these ids for the
 * thin fringe-strip blocks of TG_CFG_256x256 (256 x 64 for an N tail of at
 * most 64 columns, 64 x 256 for an M tail of at most 64 rows). */
enum { TG_LAYOUT_CFG_STRIP_N = 101, TG_LAYOUT_CFG_STRIP_M = 102,
       /* the same tiles for fp32 inputs (K tile 16, 16x16x4 MFMAs): TG_CFG_256x256,
        * TG_CFG_128x128 and the 256x256 tile's strips (version 9 and later) */
       TG_LAYOUT_CFG_F32_256 = 103, TG_LAYOUT_CFG_F32_128 = 104,
       TG_LAYOUT_CFG_F32_STRIP_N = 105, TG_LAYOUT_CFG_F32_STRIP_M = 106 };

tg_status tile_gemm_describe_layout(int config, int swizzle, int kind, tg_layout *out);

/* The LDS element offset the kernel itself computes for (row, k) of an operand
 * tile (operand 0 = A, 1 = B), from the same inline function the device code
 * calls; -1 for an invalid request.  For checking the kernel against its layout. */
int64_t tile_gemm_lds_offset(int config, int swizzle, int operand, int64_t row, int64_t k);

/* The accumulator (row, col) inside the block tile that (wave, lane, slot) of
 * the kernel's register tiles holds, as the epilogue computes it; returns 0,
 * or -1 for an invalid request. */
int tile_gemm_acc_coord(int config, int wave, int lane, int slot, int64_t *row, int64_t *col);

/* A fixed description of a status, for messages: never NULL, owned by the
 * library (the failure reports the status codes above stand for). */
const char *tile_gemm_status_string(tg_status s);

/* TILE_GEMM_ABI_VERSION of the built library, so a caller can refuse a library
 * built from another header instead of misreading its structs (the same
 * refuse-rather-than-guess rule as the status codes above). */
int tile_gemm_abi_version(void);

/*
 * Hoisted pre-pack of B (OCANNL "Module Ir.Schedule", the Stage paragraph's
 * hoisted option: a staged copy of an operand the loop nest does not change
 * is made once, outside it).  For callers that multiply by the same B many
 * times: tile_gemm_pack_b writes B once into rows of a multiple of 16 bytes
 * (16-byte aligned, zero-filled past N), the layout the tile copies read at
 * full rate, and every later call passes the packed copy as an ordinary B:
 *     B = packed, ldb = tile_gemm_packed_b_ld(N, dtype), strideB = K * ldb,
 * to tile_gemm / tile_gemm_strided_batched / tile_gemm_ex.  The values are
 * unchanged, so a call on the packed copy computes the same MFMA sequence and
 * a bitwise identical C.  The pack can also take B as stored transposed (an
 * N x K row-major matrix, as a layer's weight often is), which the GEMM itself
 * does not read.
 *
 * tile_gemm_packed_b_ld: the packed row length in elements, roundup(max(N, 1),
 *   16 / element size); -1 for a negative N or an unknown dtype.
 * tile_gemm_packed_b_size: *bytes = batch * K * tile_gemm_packed_b_ld(N) *
 *   element size (host only).
 * tile_gemm_pack_b: B is batch matrices of K x N (transposed == 0: element
 *   (k, n) at B[b * strideB + k * ldb + n], ldb >= N) or stored transposed
 *   (transposed == 1: element (k, n) at B[b * strideB + n * ldb + k], ldb >= K),
 *   fp32 / bf16 / fp16 storage, read only.  packed is caller-owned device
 *   memory, 256-byte aligned, packed_bytes >= tile_gemm_packed_b_size, not
 *   overlapping B; element (b, k, n) lands at packed[(b * K + k) * ld + n].
 *   Asynchronous on `stream`.  Errors: TG_ERR_INVALID_ARG for negative
 *   extents or stride, ldb too small, NULL or misaligned pointers, too small
 *   a buffer, an overlap or transposed not 0 / 1 (checked before any device
 *   work); TG_ERR_UNSUPPORTED without a gfx950 device or for more than 65535
 *   transposed batch entries.  An empty B (batch, K or N 0) does nothing.
 */
int64_t tile_gemm_packed_b_ld(int64_t N, tg_dtype dtype);
tg_status tile_gemm_packed_b_size(int64_t batch, int64_t K, int64_t N, tg_dtype dtype, int64_t *bytes);
tg_status tile_gemm_pack_b(int64_t batch, int64_t K, int64_t N, tg_dtype dtype, const void *B, int64_t ldb,
                           int64_t strideB, int transposed, void *packed, int64_t packed_bytes, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): tile_gemm_ex with the
 * library's own scratch instead of a caller workspace.
 *
 * The scratch is one file-scope device array of TILE_GEMM_NOALLOC_SCRATCH_BYTES
 * (64 MiB), held by every GPU the library runs on until the process ends; its
 * device address is looked up once per device on the first call there.  The
 * call takes the same arguments as tile_gemm_ex and computes the same plan as
 * tile_gemm_ex given a workspace of that size, so its C is bitwise the one
 * tile_gemm_ex writes with such a workspace: automatic split-K and the repack
 * of A happen only when they fit.  opt->workspace must be NULL and
 * opt->workspace_bytes 0 (TG_ERR_INVALID_ARG otherwise).  A call that would
 * need more scratch than the array holds (a forced split_k, pack_a == 2 or
 * tail_gemm == 2 whose partials or copy exceed it) returns TG_ERR_SCRATCH_LIMIT
 * before any device work.  It allocates nothing: no hipMalloc, no hipFree, no
 * allocating library routine, and no memset (nothing in the scratch has to
 * start at zero: split partials are written whole before they are read).
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents: calls that overlap in time on one GPU (different streams, or
 * several host threads without ordering) race on it and must not be issued.
 */
#define TILE_GEMM_NOALLOC_SCRATCH_BYTES (64LL << 20)

tg_status tile_gemm_ex_noalloc(int64_t batch, int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                               const void *A, int64_t lda, int64_t strideA,
                               const void *B, int64_t ldb, int64_t strideB,
                               float *C, int64_t ldc, int64_t strideC,
                               float alpha, float beta, void *stream, const tg_options *opt);

#ifdef __cplusplus
}
#endif

#endif /* TILE_GEMM_H */
