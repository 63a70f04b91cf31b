/*
 * lora.h - C ABI of the segmented multi-LoRA linear layer for MI355X (gfx950).
 *
 * The layer (Multi-LoRA Serving: adapter batching, charlestar.github.io,
 * sections "LoRA 在一层 Linear 上增加了什么" and "一个混合 Batch 的数学形式"):
 *
 *     Y = X W^T + s_a (X_a A_a^T) B_a^T,     s_a = alpha_a / r_a,
 *
 * where every token row i carries its own adapter slot a(i) (or none), the
 * base product X W^T is shared by all rows, and row i only ever uses its
 * own A_a, B_a, s_a.
 *
 * Conventions for every entry point
 * ---------------------------------
 * - Every pointer argument is a DEVICE pointer unless stated otherwise; the
 *   structs themselves live in host memory.  The caller owns every buffer;
 *   the library allocates nothing and keeps no state between calls, apart
 *   from the static device scratch of lora_linear_fused_static.
 * - Calls are asynchronous on the given HIP stream (`hipStream_t` passed as
 *   `void*`, NULL = the default stream).  Argument errors are detected on
 *   the host and returned before anything is launched; no output is touched
 *   then.  LORA_ERR_HIP reports a failed launch.
 * - Row-major storage.  Leading dimensions (`ld*`) are in elements, at least
 *   the row width, at most LORA_MAX_LD, and multiples of 8; every tensor base
 *   pointer is 16-byte aligned; d_in and d_out are positive multiples of 8.
 *   Otherwise LORA_ERR_ALIGN / LORA_ERR_SHAPE.
 * - X, W, Y, A and Bt share the pool's dtype (bf16 or fp32).  H is fp32.
 *   Accumulation is fp32.
 * - Data errors found on the device (a row's slot outside [-1, n_slots) or
 *   a slot rank outside [0, r_max]) never alias memory: the row is treated
 *   as base-only and counted in `*status` by lora_build_segments.
 * - Calls that share output buffers and overlap on one device race.
 */
#ifndef LORA_H_
#define LORA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LORA_ABI_VERSION 9
/* Largest pool: the segment builder keeps per-slot tables in LDS. */
#define LORA_MAX_SLOTS 4095
/* Limits of the allocation-free call lora_linear_fused_static: token rows,
 * and n_rows * r_max (the entries of its H). */
#define LORA_STATIC_MAX_ROWS 32768
#define LORA_STATIC_MAX_H (1 << 21)
/* Largest leading dimension of X, W, Y (elements): the GEMM addresses a tile's
 * rows with 32-bit byte offsets from its first row. */
#define LORA_MAX_LD (1 << 22)

/* lora_layer_fused: batches of up to this many rows (bf16 pools) run in one
 * launch; its sync buffer has this many bytes. */
#define LORA_LAYER_ONE_LAUNCH_ROWS 512
#define LORA_LAYER_SYNC_BYTES 4096

typedef enum {
  LORA_OK = 0,
  LORA_ERR_NULL = -1,      /* a required pointer is NULL */
  LORA_ERR_SHAPE = -2,     /* a size is out of range or inconsistent */
  LORA_ERR_RANK = -3,      /* r_max not one of 8, 16, 32, 64 */
  LORA_ERR_ALIGN = -4,     /* pointer not 16-byte aligned or ld not a multiple of 8 */
  LORA_ERR_DTYPE = -5,     /* unknown dtype */
  LORA_ERR_CAPACITY = -6,  /* segment arrays too small for the worst case */
  LORA_ERR_HIP = -7,       /* the HIP runtime reported an error at launch */
  LORA_ERR_POLICY = -8,    /* unknown rank policy */
  LORA_ERR_SCRATCH = -9    /* batch larger than the allocation-free call's scratch */
} lora_status;

typedef enum { LORA_F32 = 0, LORA_BF16 = 1 } lora_dtype;

/*
 * How a segment of true rank r is processed (adapter-batching page, section
 * "不同 LoRA Rank 会怎样影响 Kernel": padding every slot to r_max versus
 * kernels chosen per rank bucket).  Work and bytes read per segment scale
 * with the processed width; the result never depends on the policy, because
 * rank rows at or past r are masked to zero, never multiplied in.
 */
typedef enum {
  LORA_RANK_EXACT = 0,       /* r rounded up to the next of 8, 16, 32, 64 */
  LORA_RANK_TWO_BUCKETS = 1, /* r <= 16 -> 16, else 64 (the page's {8,16} / {32,64}) */
  LORA_RANK_PADDED = 2       /* every segment at r_max */
} lora_rank_policy;

/*
 * Fixed-slot adapter pool (LoRA/QLoRA 多租户 GPU 推理服务化实战, section 1.1
 * "Adapter的统一尺寸对齐": one preallocated buffer, uniform slot size, O(1)
 * lookup by slot offset).  Slot a holds, rank-major,
 *   A [n_slots][r_max][d_in]   row k = row k of A_a      (A_a in R^{r x d_in})
 *   Bt[n_slots][rs][d_out]     row k = column k of B_a   (B_a in R^{d_out x r})
 * with rs = r_max for a single projection (stacked pools below).
 * Rows k >= slot_rank[a] are padding and are never multiplied in.
 * slot_scale[a] is s_a = alpha_a / r_a (0 for a rank-0 slot), written by the
 * library (lora_pool_pack_slot, lora_pool_set_scales), never by the caller.
 * Optionally the pool also carries B in its own d_out-major layout,
 *   B [n_slots][d_out][rs]     row j = row j of B_a   (the layout of the
 *                              adapter's up-projection weight),
 * the same values as Bt (written by lora_pool_pack_slot, or from Bt by
 * lora_pool_write_b).  lora_linear_fused then reads whole 16-byte runs of
 * rank values per output column; with B NULL it gathers them from Bt.
 *
 * DoRA (ybb.press multi-LoRA serving article, section 9.2: the adapted
 * weight is a magnitude m times the direction W0 + BA over its norm, applied
 * at inference by one extra normalisation in an epilogue).  With the
 * optional fp32 array
 *   dora_scale[n_slots][d_out]   g_a[j] = m_a[j] / ||W0[j,:] + s_a (B_a A_a)[j,:]||_2
 * (0 where that norm is 0), every output element of a row on a slot of rank
 * r > 0 is multiplied by g_a[j] after the LoRA term is added and before the
 * rounding, in lora_expand and lora_linear_fused:
 *   Y[i][j] = g_a[j] (X[i] W^T + s_a H[i][0:r] B_a^T)[j].
 * The norm is taken over each output feature's weight row (the nn.Linear
 * row), which is what makes it a per-column epilogue factor.  A slot whose
 * g row is all ones is a plain LoRA adapter and gives plain LoRA's bits.
 * Base-only rows and rank-0 slots are never rescaled.  g rows are written by
 * lora_pool_dora_prepare (and set to ones by lora_pool_pack_slot).
 *
 * Stacked projections (adapter-batching page, section "Adapter 不是一块连续
 * Weight": every target module has its own A and B; a model with fused QKV
 * or stacked gate/up runs them as one weight).  With n_proj = P >= 2 the
 * pool serves P projections of the same input at once: output columns
 * [proj_cols[q], proj_cols[q + 1]) are projection q's, and with
 * rs = r_max / P, rank rows [q rs, q rs + r) of a slot are projection q's A
 * rows, while the slot's rs rank rows of Bt hold in each column that
 * column's own projection's B^T (every column belongs to one projection, so
 * Bt and B take no more room than one projection's would: [n_slots][rs]
 * [d_out] and [n_slots][d_out][rs]).  A slot's rank r (<= rs) and scale are
 * shared by its projections; H is [n][r_max] with projection q's ranks at
 * columns [q rs, q rs + r).  Every call then computes, for each projection,
 * exactly what it computes for a single one.  Requirements: proj_cols[0] =
 * 0, proj_cols[P] = d_out, strictly increasing multiples of 8
 * (LORA_ERR_SHAPE), rs in {8, 16, 32, 64} (LORA_ERR_RANK), proj_cols non-NULL
 * (LORA_ERR_NULL).  lora_pool_pack_slot writes this layout from each
 * projection's own A and B.
 */
typedef struct {
  int32_t n_slots;           /* 1 .. LORA_MAX_SLOTS */
  int32_t r_max;             /* rs = 8, 16, 32 or 64 (times n_proj for stacked pools) */
  int32_t d_in;
  int32_t d_out;
  int32_t dtype;             /* lora_dtype */
  int32_t rank_policy;       /* lora_rank_policy */
  const void *A;             /* device */
  const void *Bt;            /* device, [n_slots][rs][d_out] */
  const int32_t *slot_rank;  /* device, [n_slots] */
  const float *slot_scale;   /* device, [n_slots] */
  const void *B;             /* device, optional (NULL): [n_slots][d_out][rs] */
  const float *dora_scale;   /* device, optional (NULL): fp32 [n_slots][d_out] DoRA g */
  int32_t n_proj;            /* 0 or 1: one projection; 2..8: stacked projections */
  const int32_t *proj_cols;  /* HOST, [n_proj + 1] column offsets (stacked pools only) */
} lora_pool;

/*
 * Segment metadata (adapter-batching page, section "Segmented Kernel 需要哪些
 * Metadata": segment_offsets, adapter_slots, token_indices, ranks, scales).
 * Written by lora_build_segments, read by the other calls.  Host fields:
 * n_rows (token rows of the batch) and max_segments (capacity of the
 * per-segment arrays; must be >= min(n_rows, n_slots + 1)).  Device arrays:
 *   token_indices  [n_rows]          sorted position -> original row
 *   row_segment    [n_rows]          original row -> segment id
 *   segment_offsets[max_segments+1]  segment s = sorted positions [off[s], off[s+1])
 *   segment_slots  [max_segments]    slot, -1 for the base-only segment
 *   segment_ranks  [max_segments]    0 for base-only
 *   segment_scales [max_segments]    0 for base-only and rank-0 slots
 *   num_segments   [1]
 *   status         [1]               rows demoted to base-only (bad slot/rank)
 * Segments appear in first-appearance order of their slot; rows inside a
 * segment are ascending.  Entries past num_segments are left untouched.
 */
typedef struct {
  int32_t n_rows;
  int32_t max_segments;
  int32_t *token_indices;
  int32_t *row_segment;
  int32_t *segment_offsets;
  int32_t *segment_slots;
  int32_t *segment_ranks;
  float *segment_scales;
  int32_t *num_segments;
  int32_t *status;
} lora_segments;

/* ABI version of the loaded library (LORA_ABI_VERSION). */
int32_t lora_abi_version(void);

/* Static text for a status code; never NULL. */
const char *lora_status_str(int32_t status);

/*
 * Group the batch's token rows by slot (adapter-batching page, "Segmented
 * Kernel 需要哪些 Metadata"; one segment per distinct slot, as S-LoRA 深度解析
 * section 3.1 asks, requests of one adapter merged into one product).
 * row_slot: device int32 [seg->n_rows], -1 = base-only.  One launch, no
 * host synchronisation.  n_rows == 0 writes num_segments = 0,
 * segment_offsets[0] = 0 and status = 0.
 */
lora_status lora_build_segments(const int32_t *row_slot, const lora_pool *pool,
                                const lora_segments *seg, void *stream);

/*
 * Shrink, H_a = X_a A_a^T per segment (adapter-batching page, "Segmented
 * Kernel 需要哪些 Metadata").  X [n_rows][d_in] (ld ldx), pool dtype.
 * H: fp32 [n_rows][r_max] indexed by ORIGINAL row; for a row of a segment of
 * rank r > 0, H[i][0:r] is written; every other entry of H is untouched.
 */
lora_status lora_shrink(const void *X, int64_t ldx, const lora_segments *seg,
                        const lora_pool *pool, float *H, void *stream);

/*
 * Segment build and shrink in one call (the two sections above): the same
 * outputs as lora_build_segments(row_slot, pool, seg) followed by
 * lora_shrink(X, ldx, seg, pool, H), bit for bit, with the same arguments,
 * layouts and errors.  For decode-sized batches (up to 512 rows) both run in
 * one launch: one workgroup builds the metadata while the others compute H
 * slot by slot from the per-row slot ids, so the shrink does not wait for
 * the metadata.  Larger batches take the two launches.
 */
lora_status lora_build_shrink(const int32_t *row_slot, const void *X, int64_t ldx,
                              const lora_pool *pool, const lora_segments *seg, float *H,
                              void *stream);

/*
 * Expand and scatter-add, Y[i] += s_a H[i][0:r] B_a^T for every row i of a
 * segment of rank r > 0 (same section: Delta Y_a = s_a H_a B_a^T, added back
 * to the original rows).  Y [n_rows][d_out] (ld ldy), pool dtype; each Y
 * element is read, added in fp32 and rounded once.  With pool->dora_scale
 * the sum is multiplied by the slot's g before the rounding (see lora_pool):
 * Y[i][j] = g_a[j] (Y[i][j] + s_a H[i][0:r] B_a^T[j]).  Rows of base-only and
 * rank-0 segments are not touched.  Each row belongs to exactly one segment,
 * so no atomics are used and the result is deterministic.
 */
lora_status lora_expand(const float *H, const lora_segments *seg, const lora_pool *pool,
                        void *Y, int64_t ldy, void *stream);

/*
 * Base product only, Y = X W^T (adapter-batching page, "一个混合 Batch 的数学
 * 形式": one GEMM shared by all rows).  X [n_rows][d_in], W [d_out][d_in]
 * (nn.Linear layout), Y [n_rows][d_out], all of `dtype`.  bf16 runs on
 * MFMA with fp32 accumulation and one rounding.
 */
lora_status lora_base_gemm(const void *X, int64_t ldx, const void *W, int64_t ldw,
                           void *Y, int64_t ldy, int32_t n_rows, int32_t d_in,
                           int32_t d_out, int32_t dtype, void *stream);

/* Layout of the B sources of lora_pool_pack_slot. */
typedef enum {
  LORA_B_ROWS = 0,      /* B_q [d_out_q][ldb], ldb >= rank: the adapter weight's own layout */
  LORA_B_RANK_ROWS = 1  /* B_q^T [rank][ldb], ldb >= d_out_q: the pool's Bt layout */
} lora_b_layout;

/*
 * Pack one adapter into slot `slot` of the pool (LoRA/QLoRA 多租户GPU推理服务化实战,
 * section 1.1 "Adapter的统一尺寸对齐": one preallocated buffer, each adapter packed
 * into the slot its offset names, and section 1.2: the alpha / r scaling is the
 * kernel library's; adapter-batching page, "动态加载是一个安全边界": rank and sizes
 * bounded, a failed load leaves the old contents usable, the new slot published
 * only when its weights are complete; "Adapter 不是一块连续 Weight": each target
 * projection has its own A and B).  HOST arrays of P = max(1, pool->n_proj)
 * entries give projection q's sources, both device memory of the pool dtype:
 *   A_src[q]  [rank][lda[q]]   down-projection A_q   (lda % 8 == 0, 16-byte aligned)
 *   B_src[q]  up-projection B_q in b_layout: [d_out_q][ldb[q]] (LORA_B_ROWS)
 *             or its transpose [rank][ldb[q]] (LORA_B_RANK_ROWS),
 * with d_out_q the projection's column count (d_out for a single projection).
 * Writes, per projection q with rs = r_max / P: A rank rows [q rs, q rs + rank)
 * and zeros up to (q + 1) rs; Bt rank rows [0, rank) = B_q^T in the
 * projection's columns and zeros up to rs there (the other projections'
 * columns are left as they are); the pool's d_out-major B when it has one,
 * likewise; ones in the slot's dora_scale row
 * when the pool has that array (the new adapter starts as plain LoRA;
 * lora_pool_dora_prepare makes it DoRA).  Then, by a later kernel on the same
 * stream, slot_rank[slot] = rank and slot_scale[slot] = alpha / rank (the
 * double quotient rounded once to float; 0 for rank 0).  Work queued later
 * on `stream` sees the whole new adapter.  rank = 0 empties the slot (its
 * rows take the base-only path); the source arrays may then be NULL.  The
 * caller must not pack a slot that queued or running work on other streams
 * still reads (wait for it first).  The pool's slot_rank and slot_scale
 * arrays are written.  Errors (all before any write): NULL pool, or for
 * rank > 0 a NULL array or source (LORA_ERR_NULL); slot outside
 * [0, n_slots), rank outside [0, rs], lda[q] < d_in, ldb[q] below rank
 * (LORA_B_ROWS) or d_out_q (LORA_B_RANK_ROWS), or an unknown b_layout
 * (LORA_ERR_SHAPE); lda[q] not a multiple of 8 or A_src[q] not 16-byte
 * aligned (LORA_ERR_ALIGN).
 */
lora_status lora_pool_pack_slot(const lora_pool *pool, int32_t slot, int32_t rank, double alpha,
                                const void *const *A_src, const int64_t *lda,
                                const void *const *B_src, const int64_t *ldb, int32_t b_layout,
                                void *stream);

/*
 * The scale of every slot from its alpha (the scaling s = alpha / r of the
 * adapter-batching page, "LoRA 在一层 Linear 上增加了什么"; kept in the kernel
 * library as LoRA/QLoRA 多租户GPU推理服务化实战 section 1.2 asks):
 *   slot_scale[a] = alpha[a] / slot_rank[a]   (double quotient rounded once to
 *                                              float; 0 where slot_rank[a] <= 0)
 * slot_alpha: device double [n_slots], 8-byte aligned (LORA_ERR_ALIGN),
 * non-NULL (LORA_ERR_NULL).  For a pool whose A, Bt and slot_rank the
 * caller laid out directly; reads slot_rank as queued work on `stream`
 * leaves it.  Writes slot_scale only.
 */
lora_status lora_pool_set_scales(const lora_pool *pool, const double *slot_alpha, void *stream);

/*
 * The pool's d_out-major copy of B from its Bt, for every slot:
 * B[a][j][k] = Bt[a][k][j], k < rs (adapter-batching page, "Adapter 不是一块连续
 * Weight": B_a in R^{d_out x r} is the adapter weight's own layout).  pool->B
 * must be non-NULL (LORA_ERR_NULL).  Asynchronous on `stream`; writes B only.
 */
lora_status lora_pool_write_b(const lora_pool *pool, void *stream);

/*
 * DoRA column factors of one slot (ybb.press multi-LoRA serving article,
 * section 9.2): for every output feature j,
 *   dora_scale[slot][j] = magnitude[j] / ||W[j,:] + s (B_a A_a)[j,:]||_2
 * with A_a, B_a, the rank r and s = slot_scale[slot] as the pool holds them
 * when the call runs on `stream` (so it goes after lora_pool_pack_slot on
 * the same stream); 0 where the norm is 0.  Sums of squares in fp32 from the
 * stored weights.  W [d_out][d_in] (ld ldw) is the base weight, pool dtype;
 * magnitude is device fp32 [d_out], or NULL for all ones (the slot then acts
 * as a plain LoRA adapter).  For a rank-0 slot the factors are written but
 * never applied.  Work queued later on `stream` sees the new factors.  The
 * caller must not prepare a slot that work on other streams still reads.
 * Errors (before any write): NULL pool, pool->dora_scale or W
 * (LORA_ERR_NULL), slot outside [0, n_slots) or ldw < d_in (LORA_ERR_SHAPE),
 * dora_scale or W not 16-byte aligned, ldw not a multiple of 8 or magnitude
 * not 4-byte aligned (LORA_ERR_ALIGN).
 */
lora_status lora_pool_dora_prepare(const lora_pool *pool, int32_t slot, const void *W,
                                   int64_t ldw, const float *magnitude, void *stream);

/*
 * Base product with the LoRA expand fused into its epilogue:
 *   Y[i] = X[i] W^T + s_a H[i][0:r] B_a^T
 * (the second low-rank product added straight into the base output, as the
 * epilogue-fusion passage of the ybb.press multi-LoRA serving article,
 * section 5.3, describes).  H comes from lora_shrink on the same metadata.
 * The fp32 accumulator is rounded to the output dtype once.  Rows of
 * base-only and rank-0 segments equal lora_base_gemm's output bit for bit.
 * With pool->dora_scale, rows of rank > 0 are multiplied by their slot's g
 * before the rounding (see lora_pool).
 */
lora_status lora_linear_fused(const void *X, int64_t ldx, const void *W, int64_t ldw,
                              const float *H, const lora_segments *seg,
                              const lora_pool *pool, void *Y, int64_t ldy, void *stream);

/*
 * Quantized base weight (adapter-batching page, section "Quantized Base
 * Model 与 LoRA 的 Dtype 边界": the base weight may be INT4/INT8/FP8 while A
 * and B stay 16-bit; LoRA/QLoRA 多租户GPU推理服务化实战, section 1.2: the
 * base weight is dequantized inside the kernel, at register level, and the
 * alpha/r scaling stays inside the fused kernel).  Here the base weight is
 * FP8 E4M3 (the OCP 8-bit floating point format) with one float32 scale per
 * output row:
 *   W[j][c] = w_scale[j] * e4m3(Wq[j][c]),   Wq [d_out][d_in] bytes (ld ldw)
 * and the answers to the page's questions are:
 *   - the base GEMM reads Wq from HBM (one byte per weight), widens each
 *     code to bf16 in registers (exact: every E4M3 value is a bf16 value),
 *     multiplies by the bf16 activations on MFMA and accumulates in fp32;
 *     w_scale[j] multiplies the fp32 accumulator of column j;
 *   - the LoRA branch reuses the same, unquantized bf16 activations X
 *     (lora_shrink / lora_build_shrink are unchanged); A and B are bf16
 *     with scale s_a = alpha_a / r_a;
 *   - the two paths add in fp32 after the weight scale and before the one
 *     rounding to bf16 (and before a tensor-parallel reduction, which would
 *     sum the rounded partial outputs).
 * Requirements on top of the bf16 calls: X and Y bf16, d_in % 16 == 0,
 * ldw % 16 == 0, Wq and w_scale 16-byte aligned (LORA_ERR_ALIGN), Wq and
 * w_scale non-NULL (LORA_ERR_NULL), ldw >= d_in (LORA_ERR_SHAPE).  Codes
 * 0x7F / 0xFF (NaN) propagate NaN.
 */
lora_status lora_base_gemm_fp8w(const void *X, int64_t ldx, const void *Wq, int64_t ldw,
                                const float *w_scale, void *Y, int64_t ldy, int32_t n_rows,
                                int32_t d_in, int32_t d_out, void *stream);

/* lora_linear_fused with the FP8 base weight above; the pool must be bf16
 * (LORA_ERR_DTYPE otherwise).  Rows of base-only and rank-0 segments equal
 * lora_base_gemm_fp8w's output bit for bit. */
lora_status lora_linear_fused_fp8w(const void *X, int64_t ldx, const void *Wq, int64_t ldw,
                                   const float *w_scale, const float *H,
                                   const lora_segments *seg, const lora_pool *pool, void *Y,
                                   int64_t ldy, void *stream);

/*
 * The whole layer in one call: lora_build_segments, lora_shrink and
 * lora_linear_fused together (adapter-batching page, sections "一个混合
 * Batch 的数学形式" and "Segmented Kernel 需要哪些 Metadata"; its section
 * "Prefill 与 Decode 的 LoRA 形状不同" places decode's cost in launches,
 * gathers and metadata).  Arguments and layouts as in those three calls:
 * row_slot device int32 [seg->n_rows] (-1 = base-only), X [n][d_in],
 * W [d_out][d_in], Y [n][d_out] of the pool's dtype, H fp32 [n][r_max] and
 * the segment arrays are written.  Outputs: the segment metadata bit for bit
 * as lora_build_segments writes it, H[i][0:r] for the rows of a LoRA
 * segment (equal to lora_shrink's up to the order of the fp32 additions),
 * and Y = X W^T + s_a H[i][0:r] B_a^T with one rounding (rows of base-only
 * and rank-0 segments equal lora_base_gemm's output bit for bit).
 * For bf16 pools and 1 <= n <= LORA_LAYER_ONE_LAUNCH_ROWS this is one
 * kernel launch: every workgroup builds the metadata itself, computes H for
 * one row and hands it to the tiles that need it through `sync`; otherwise
 * it is lora_build_shrink followed by lora_linear_fused.
 * sync: NULL, or a device buffer of LORA_LAYER_SYNC_BYTES bytes, 16-byte
 * aligned, owned by the caller, zero-filled once before its first use and
 * then left to the library (it keeps a call counter there and leaves it
 * ready for the next call).  Calls that share a sync buffer must be ordered
 * on one stream (they race otherwise); with sync NULL every output tile
 * computes the H rows it needs itself (same results, more work).
 * Errors as the three calls; n_rows == 0 writes the empty metadata only.
 */
lora_status lora_layer_fused(const int32_t *row_slot, const void *X, int64_t ldx, const void *W,
                             int64_t ldw, const lora_pool *pool, const lora_segments *seg,
                             float *H, void *Y, int64_t ldy, void *sync, void *stream);

/*
 * lora_layer_fused with the base weight as FP8 E4M3 codes and one float32
 * scale per output row, as in lora_linear_fused_fp8w (quantized base with a
 * bf16 LoRA path, LoRA/QLoRA 多租户GPU推理服务化实战 section 1.2: the low-rank
 * term of the unquantized activations is added to the quantized base
 * product).  Wq uint8 [d_out][ldw] (ldw % 16 == 0, d_in % 16 == 0),
 * w_scale device float32 [d_out]; bf16 pools only (LORA_ERR_DTYPE
 * otherwise).  Metadata and H as lora_layer_fused writes them; Y as
 * lora_linear_fused_fp8w computes it, with one rounding (rows of base-only
 * and rank-0 segments equal lora_base_gemm_fp8w's output bit for bit).
 * One launch for 1 <= n <= LORA_LAYER_ONE_LAUNCH_ROWS, else
 * lora_build_shrink followed by lora_linear_fused_fp8w; sync and errors as
 * lora_layer_fused.
 */
lora_status lora_layer_fused_fp8w(const int32_t *row_slot, const void *X, int64_t ldx,
                                  const void *Wq, int64_t ldw, const float *w_scale,
                                  const lora_pool *pool, const lora_segments *seg, float *H,
                                  void *Y, int64_t ldy, void *sync, void *stream);

/*
 * The whole layer with no workspace arguments, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc):
 *   Y = X W^T + s_a H[i][0:r] B_a^T,   H = the shrink of X,
 * exactly what lora_build_shrink followed by lora_linear_fused computes (same
 * kernels, same bits), with the segment metadata and H kept in a static
 * device array of the library (about 8.4 MB per GPU, held until the process
 * ends) instead of caller buffers.  row_slot: device int32 [n_rows] (-1 =
 * base-only); X [n_rows][d_in] (ld ldx), W [d_out][d_in] (ld ldw), Y
 * [n_rows][d_out] (ld ldy), all of the pool's dtype, as for
 * lora_linear_fused.  Rows demoted for a bad slot or rank are base-only, as
 * there (their count is kept in the scratch, not returned).
 * Limits: n_rows <= LORA_STATIC_MAX_ROWS and n_rows * r_max <=
 * LORA_STATIC_MAX_H, else LORA_ERR_SCRATCH before anything is launched.
 * Nothing is allocated: no hipMalloc, no hipFree, no allocating library call.
 * Every call on one GPU uses that GPU's one scratch array, so calls that
 * overlap on a GPU (other streams, other threads) race; calls queued on one
 * stream are ordered.  The first call on a device looks the array's address
 * up (a HIP runtime call that does not allocate); later calls reuse it.
 * Other errors as lora_linear_fused.  n_rows == 0 is a no-op.
 */
lora_status lora_linear_fused_static(const int32_t *row_slot, const void *X, int64_t ldx,
                                     const void *W, int64_t ldw, const lora_pool *pool,
                                     int32_t n_rows, void *Y, int64_t ldy, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LORA_H_ */
