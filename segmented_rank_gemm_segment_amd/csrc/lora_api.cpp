// C ABI of the multi-LoRA layer: host-side argument validation and launch.
//
// Validation happens before any HIP call, so every argument error returns
// without touching device memory (and works on a machine with no GPU).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/lora.h"
#include "lora_kernels.h"

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_dtype(int32_t d) { return d == LORA_F32 || d == LORA_BF16; }

bool valid_rank_width(int32_t r) { return r == 8 || r == 16 || r == 32 || r == 64; }

// Per-projection rank stride of a pool (r_max for a single projection).
int32_t pool_rs(const lora_pool *pool) {
  return pool->n_proj >= 2 ? pool->r_max / pool->n_proj : pool->r_max;
}

lora_status check_proj(const lora_pool *pool) {
  if (pool->n_proj < 0 || pool->n_proj > lora::kMaxProj) return LORA_ERR_SHAPE;
  if (pool->n_proj <= 1) return valid_rank_width(pool->r_max) ? LORA_OK : LORA_ERR_RANK;
  if (pool->r_max % pool->n_proj || !valid_rank_width(pool->r_max / pool->n_proj))
    return LORA_ERR_RANK;
  if (!pool->proj_cols) return LORA_ERR_NULL;
  if (pool->proj_cols[0] != 0 || pool->proj_cols[pool->n_proj] != pool->d_out) return LORA_ERR_SHAPE;
  for (int q = 0; q < pool->n_proj; ++q)
    if (pool->proj_cols[q + 1] <= pool->proj_cols[q] || pool->proj_cols[q + 1] % 8)
      return LORA_ERR_SHAPE;
  return LORA_OK;
}

lora_status check_pool(const lora_pool *pool) {
  if (!pool) return LORA_ERR_NULL;
  if (!valid_dtype(pool->dtype)) return LORA_ERR_DTYPE;
  lora_status st = check_proj(pool);
  if (st != LORA_OK) return st;
  if (pool->rank_policy < LORA_RANK_EXACT || pool->rank_policy > LORA_RANK_PADDED)
    return LORA_ERR_POLICY;
  if (pool->n_slots < 1 || pool->n_slots > LORA_MAX_SLOTS) return LORA_ERR_SHAPE;
  if (pool->d_in <= 0 || pool->d_out <= 0) return LORA_ERR_SHAPE;
  if (pool->d_in % 8 || pool->d_out % 8) return LORA_ERR_ALIGN;
  if (!pool->A || !pool->Bt || !pool->slot_rank || !pool->slot_scale) return LORA_ERR_NULL;
  if (!aligned16(pool->A) || !aligned16(pool->Bt)) return LORA_ERR_ALIGN;
  if (pool->B && !aligned16(pool->B)) return LORA_ERR_ALIGN;
  if (pool->dora_scale && !aligned16(pool->dora_scale)) return LORA_ERR_ALIGN;
  return LORA_OK;
}

int32_t seg_worst_case(int32_t n_rows, int32_t n_slots) {
  return n_rows < n_slots + 1 ? n_rows : n_slots + 1;
}

lora_status check_segments(const lora_segments *seg, const lora_pool *pool) {
  if (!seg) return LORA_ERR_NULL;
  if (seg->n_rows < 0) return LORA_ERR_SHAPE;
  if (seg->max_segments < 0) return LORA_ERR_SHAPE;
  if (seg->max_segments < seg_worst_case(seg->n_rows, pool->n_slots)) return LORA_ERR_CAPACITY;
  if (!seg->segment_offsets || !seg->segment_slots || !seg->segment_ranks ||
      !seg->segment_scales || !seg->num_segments || !seg->status)
    return LORA_ERR_NULL;
  if (seg->n_rows > 0 && (!seg->token_indices || !seg->row_segment)) return LORA_ERR_NULL;
  return LORA_OK;
}

lora_status check_matrix(const void *p, int64_t ld, int32_t width, int32_t rows) {
  if (rows == 0) return LORA_OK;
  if (!p) return LORA_ERR_NULL;
  if (ld < width || ld > LORA_MAX_LD) return LORA_ERR_SHAPE;
  if (ld % 8 || !aligned16(p)) return LORA_ERR_ALIGN;
  return LORA_OK;
}

lora::SegView seg_view(const lora_segments *s) {
  return lora::SegView{s->n_rows,        s->max_segments,  s->token_indices,
                       s->row_segment,   s->segment_offsets, s->segment_slots,
                       s->segment_ranks, s->segment_scales,  s->num_segments};
}

lora::PoolView pool_view(const lora_pool *p) {
  lora::PoolView v{p->n_slots, p->r_max, p->d_in, p->d_out, p->dtype, p->rank_policy,
                   p->A,       p->Bt,      p->B,      p->dora_scale, {}};
  v.proj.n_proj = p->n_proj >= 2 ? p->n_proj : 1;
  v.proj.rs = pool_rs(p);
  for (int q = 0; q <= lora::kMaxProj; ++q)
    v.proj.col_off[q] = q <= v.proj.n_proj ? (v.proj.n_proj == 1 ? (q ? p->d_out : 0)
                                                                   : p->proj_cols[q])
                                           : p->d_out;
  return v;
}

// FP8 weight: E4M3 codes [d_out][ldw] (16-byte aligned rows, d_in % 16 == 0)
// and one float32 scale per output row.
lora_status check_fp8_weight(const void *Wq, int64_t ldw, const float *w_scale, int32_t d_in,
                             int32_t d_out) {
  if (d_in % 16) return LORA_ERR_ALIGN;
  if (!Wq || !w_scale) return LORA_ERR_NULL;
  if (ldw < d_in || ldw > LORA_MAX_LD) return LORA_ERR_SHAPE;
  if (ldw % 16 || !aligned16(Wq) || !aligned16(w_scale)) return LORA_ERR_ALIGN;
  (void)d_out;
  return LORA_OK;
}

lora_status hip_status(hipError_t e) { return e == hipSuccess ? LORA_OK : LORA_ERR_HIP; }

}  // namespace

extern "C" {

int32_t lora_abi_version(void) { return LORA_ABI_VERSION; }

const char *lora_status_str(int32_t status) {
  switch (status) {
    case LORA_OK: return "ok";
    case LORA_ERR_NULL: return "required pointer is NULL";
    case LORA_ERR_SHAPE: return "size out of range or inconsistent";
    case LORA_ERR_RANK: return "r_max must be 8, 16, 32 or 64";
    case LORA_ERR_ALIGN: return "pointer not 16-byte aligned, or ld / d not a multiple of 8";
    case LORA_ERR_DTYPE: return "unknown dtype";
    case LORA_ERR_CAPACITY: return "segment arrays smaller than min(n_rows, n_slots + 1)";
    case LORA_ERR_HIP: return "HIP runtime error at launch";
    case LORA_ERR_POLICY: return "unknown rank policy";
    case LORA_ERR_SCRATCH:
      return "batch exceeds the static scratch (LORA_STATIC_MAX_ROWS rows, LORA_STATIC_MAX_H H entries)";
    default: return "unknown status";
  }
}

lora_status lora_build_segments(const int32_t *row_slot, const lora_pool *pool,
                                const lora_segments *seg, void *stream) {
  lora_status st = check_pool(pool);
  if (st != LORA_OK) return st;
  st = check_segments(seg, pool);
  if (st != LORA_OK) return st;
  if (seg->n_rows > 0 && !row_slot) return LORA_ERR_NULL;
  return hip_status(lora::launch_build_segments(
      row_slot, seg->n_rows, pool->n_slots, pool_rs(pool), pool->slot_rank, pool->slot_scale,
      seg->token_indices, seg->row_segment, seg->segment_offsets, seg->segment_slots,
      seg->segment_ranks, seg->segment_scales, seg->num_segments, seg->status,
      static_cast<hipStream_t>(stream)));
}

lora_status lora_build_shrink(const int32_t *row_slot, const void *X, int64_t ldx,
                              const lora_pool *pool, const lora_segments *seg, float *H,
                              void *stream) {
  lora_status st = check_pool(pool);
  if (st != LORA_OK) return st;
  st = check_segments(seg, pool);
  if (st != LORA_OK) return st;
  if (seg->n_rows > 0 && !row_slot) return LORA_ERR_NULL;
  st = check_matrix(X, ldx, pool->d_in, seg->n_rows);
  if (st != LORA_OK) return st;
  if (seg->n_rows > 0) {
    if (!H) return LORA_ERR_NULL;
    if (!aligned16(H)) return LORA_ERR_ALIGN;
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const lora::BuildArgs a{row_slot,           seg->n_rows,         pool->n_slots,
                          pool_rs(pool),      pool->slot_rank,     pool->slot_scale,
                          seg->token_indices, seg->row_segment,    seg->segment_offsets,
                          seg->segment_slots, seg->segment_ranks,  seg->segment_scales,
                          seg->num_segments,  seg->status};
  const hipError_t e = lora::launch_build_shrink(a, X, ldx, pool_view(pool), H, s);
  if (e != hipErrorNotSupported) return hip_status(e);
  // outside the one-launch case: the two calls in sequence
  (void)hipGetLastError();
  st = lora_build_segments(row_slot, pool, seg, stream);
  if (st != LORA_OK || seg->n_rows == 0) return st;
  return hip_status(lora::launch_shrink(X, ldx, seg_view(seg), pool_view(pool), H, s));
}

lora_status lora_shrink(const void *X, int64_t ldx, const lora_segments *seg,
                        const lora_pool *pool, float *H, void *stream) {
  lora_status st = check_pool(pool);
  if (st != LORA_OK) return st;
  st = check_segments(seg, pool);
  if (st != LORA_OK) return st;
  st = check_matrix(X, ldx, pool->d_in, seg->n_rows);
  if (st != LORA_OK) return st;
  if (seg->n_rows == 0) return LORA_OK;
  if (!H) return LORA_ERR_NULL;
  if (!aligned16(H)) return LORA_ERR_ALIGN;
  return hip_status(lora::launch_shrink(X, ldx, seg_view(seg), pool_view(pool), H,
                                        static_cast<hipStream_t>(stream)));
}

lora_status lora_expand(const float *H, const lora_segments *seg, const lora_pool *pool,
                        void *Y, int64_t ldy, void *stream) {
  lora_status st = check_pool(pool);
  if (st != LORA_OK) return st;
  st = check_segments(seg, pool);
  if (st != LORA_OK) return st;
  st = check_matrix(Y, ldy, pool->d_out, seg->n_rows);
  if (st != LORA_OK) return st;
  if (seg->n_rows == 0) return LORA_OK;
  if (!H) return LORA_ERR_NULL;
  if (!aligned16(H)) return LORA_ERR_ALIGN;
  return hip_status(lora::launch_expand(H, seg_view(seg), pool_view(pool), Y, ldy,
                                        static_cast<hipStream_t>(stream)));
}

lora_status lora_pool_pack_slot(const lora_pool *pool, int32_t slot, int32_t rank, double alpha,
                                const void *const *A_src, const int64_t *lda,
                                const void *const *B_src, const int64_t *ldb, int32_t b_layout,
                                void *stream) {
  lora_status st = check_pool(pool);
  if (st != LORA_OK) return st;
  if (slot < 0 || slot >= pool->n_slots) return LORA_ERR_SHAPE;
  if (rank < 0 || rank > pool_rs(pool)) return LORA_ERR_SHAPE;
  if (b_layout != LORA_B_ROWS && b_layout != LORA_B_RANK_ROWS) return LORA_ERR_SHAPE;
  const int P = pool->n_proj >= 2 ? pool->n_proj : 1;
  if (rank > 0) {
    if (!A_src || !lda || !B_src || !ldb) return LORA_ERR_NULL;
    for (int q = 0; q < P; ++q) {
      const int64_t cols = P > 1 ? pool->proj_cols[q + 1] - pool->proj_cols[q] : pool->d_out;
      if (!A_src[q] || !B_src[q]) return LORA_ERR_NULL;
      if (lda[q] < pool->d_in) return LORA_ERR_SHAPE;
      if (lda[q] % 8 || !aligned16(A_src[q])) return LORA_ERR_ALIGN;
      if (ldb[q] < (b_layout == LORA_B_ROWS ? (int64_t)rank : cols)) return LORA_ERR_SHAPE;
    }
  }
  return hip_status(lora::launch_pack_slot(
      pool_view(pool), const_cast<int32_t *>(pool->slot_rank),
      const_cast<float *>(pool->slot_scale), slot, rank, alpha, A_src, lda, B_src, ldb,
      b_layout == LORA_B_RANK_ROWS, static_cast<hipStream_t>(stream)));
}

lora_status lora_pool_set_scales(const lora_pool *pool, const double *slot_alpha, void *stream) {
  lora_status st = check_pool(pool);
  if (st != LORA_OK) return st;
  if (!slot_alpha) return LORA_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(slot_alpha) & 7u) return LORA_ERR_ALIGN;
  return hip_status(lora::launch_set_scales(pool->slot_rank, slot_alpha,
                                            const_cast<float *>(pool->slot_scale), pool->n_slots,
                                            static_cast<hipStream_t>(stream)));
}

lora_status lora_pool_write_b(const lora_pool *pool, void *stream) {
  lora_status st = check_pool(pool);
  if (st != LORA_OK) return st;
  if (!pool->B) return LORA_ERR_NULL;
  return hip_status(lora::launch_write_b(pool_view(pool), static_cast<hipStream_t>(stream)));
}

lora_status lora_pool_dora_prepare(const lora_pool *pool, int32_t slot, const void *W,
                                   int64_t ldw, const float *magnitude, void *stream) {
  lora_status st = check_pool(pool);
  if (st != LORA_OK) return st;
  if (!pool->dora_scale) return LORA_ERR_NULL;
  if (slot < 0 || slot >= pool->n_slots) return LORA_ERR_SHAPE;
  st = check_matrix(W, ldw, pool->d_in, pool->d_out);
  if (st != LORA_OK) return st;
  if (magnitude && (reinterpret_cast<uintptr_t>(magnitude) & 3u)) return LORA_ERR_ALIGN;
  return hip_status(lora::launch_dora_prepare(pool_view(pool), pool->slot_rank, pool->slot_scale,
                                              slot, W, ldw, magnitude,
                                              static_cast<hipStream_t>(stream)));
}

lora_status lora_base_gemm(const void *X, int64_t ldx, const void *W, int64_t ldw, void *Y,
                           int64_t ldy, int32_t n_rows, int32_t d_in, int32_t d_out,
                           int32_t dtype, void *stream) {
  if (!valid_dtype(dtype)) return LORA_ERR_DTYPE;
  if (n_rows < 0 || d_in <= 0 || d_out <= 0) return LORA_ERR_SHAPE;
  if (d_in % 8 || d_out % 8) return LORA_ERR_ALIGN;
  lora_status st = check_matrix(X, ldx, d_in, n_rows);
  if (st != LORA_OK) return st;
  st = check_matrix(W, ldw, d_in, d_out);
  if (st != LORA_OK) return st;
  st = check_matrix(Y, ldy, d_out, n_rows);
  if (st != LORA_OK) return st;
  if (n_rows == 0) return LORA_OK;
  return hip_status(lora::launch_gemm(X, ldx, W, ldw, Y, ldy, n_rows, d_in, d_out, dtype,
                                      nullptr, nullptr, nullptr,
                                      static_cast<hipStream_t>(stream)));
}

lora_status lora_base_gemm_fp8w(const void *X, int64_t ldx, const void *Wq, int64_t ldw,
                                const float *w_scale, void *Y, int64_t ldy, int32_t n_rows,
                                int32_t d_in, int32_t d_out, void *stream) {
  if (n_rows < 0 || d_in <= 0 || d_out <= 0) return LORA_ERR_SHAPE;
  if (d_in % 8 || d_out % 8) return LORA_ERR_ALIGN;
  lora_status st = check_fp8_weight(Wq, ldw, w_scale, d_in, d_out);
  if (st != LORA_OK) return st;
  st = check_matrix(X, ldx, d_in, n_rows);
  if (st != LORA_OK) return st;
  st = check_matrix(Y, ldy, d_out, n_rows);
  if (st != LORA_OK) return st;
  if (n_rows == 0) return LORA_OK;
  return hip_status(lora::launch_gemm(X, ldx, Wq, ldw, Y, ldy, n_rows, d_in, d_out, LORA_BF16,
                                      nullptr, nullptr, nullptr,
                                      static_cast<hipStream_t>(stream), w_scale));
}

lora_status lora_linear_fused_fp8w(const void *X, int64_t ldx, const void *Wq, int64_t ldw,
                                   const float *w_scale, const float *H,
                                   const lora_segments *seg, const lora_pool *pool, void *Y,
                                   int64_t ldy, void *stream) {
  lora_status st = check_pool(pool);
  if (st != LORA_OK) return st;
  if (pool->dtype != LORA_BF16) return LORA_ERR_DTYPE;
  st = check_segments(seg, pool);
  if (st != LORA_OK) return st;
  st = check_fp8_weight(Wq, ldw, w_scale, pool->d_in, pool->d_out);
  if (st != LORA_OK) return st;
  const int32_t n = seg->n_rows;
  st = check_matrix(X, ldx, pool->d_in, n);
  if (st != LORA_OK) return st;
  st = check_matrix(Y, ldy, pool->d_out, n);
  if (st != LORA_OK) return st;
  if (n == 0) return LORA_OK;
  if (!H) return LORA_ERR_NULL;
  if (!aligned16(H)) return LORA_ERR_ALIGN;
  const lora::SegView sv = seg_view(seg);
  const lora::PoolView pv = pool_view(pool);
  return hip_status(lora::launch_gemm(X, ldx, Wq, ldw, Y, ldy, n, pool->d_in, pool->d_out,
                                      LORA_BF16, H, &sv, &pv,
                                      static_cast<hipStream_t>(stream), w_scale));
}

lora_status lora_linear_fused(const void *X, int64_t ldx, const void *W, int64_t ldw,
                              const float *H, const lora_segments *seg, const lora_pool *pool,
                              void *Y, int64_t ldy, void *stream) {
  lora_status st = check_pool(pool);
  if (st != LORA_OK) return st;
  st = check_segments(seg, pool);
  if (st != LORA_OK) return st;
  const int32_t n = seg->n_rows;
  st = check_matrix(X, ldx, pool->d_in, n);
  if (st != LORA_OK) return st;
  st = check_matrix(W, ldw, pool->d_in, pool->d_out);
  if (st != LORA_OK) return st;
  st = check_matrix(Y, ldy, pool->d_out, n);
  if (st != LORA_OK) return st;
  if (n == 0) return LORA_OK;
  if (!H) return LORA_ERR_NULL;
  if (!aligned16(H)) return LORA_ERR_ALIGN;
  const lora::SegView sv = seg_view(seg);
  const lora::PoolView pv = pool_view(pool);
  return hip_status(lora::launch_gemm(X, ldx, W, ldw, Y, ldy, n, pool->d_in, pool->d_out,
                                      pool->dtype, H, &sv, &pv,
                                      static_cast<hipStream_t>(stream)));
}

namespace {

// Both layer calls: W is bf16 (wscale NULL) or FP8 E4M3 codes with row scales.
lora_status layer_call(const int32_t *row_slot, const void *X, int64_t ldx, const void *W,
                       int64_t ldw, const float *wscale, const lora_pool *pool,
                       const lora_segments *seg, float *H, void *Y, int64_t ldy, void *sync,
                       void *stream) {
  lora_status st = check_pool(pool);
  if (st != LORA_OK) return st;
  if (wscale && pool->dtype != LORA_BF16) return LORA_ERR_DTYPE;
  st = check_segments(seg, pool);
  if (st != LORA_OK) return st;
  const int32_t n = seg->n_rows;
  if (n > 0 && !row_slot) return LORA_ERR_NULL;
  st = check_matrix(X, ldx, pool->d_in, n);
  if (st != LORA_OK) return st;
  st = wscale ? check_fp8_weight(W, ldw, wscale, pool->d_in, pool->d_out)
              : check_matrix(W, ldw, pool->d_in, pool->d_out);
  if (st != LORA_OK) return st;
  st = check_matrix(Y, ldy, pool->d_out, n);
  if (st != LORA_OK) return st;
  if (n > 0) {
    if (!H) return LORA_ERR_NULL;
    if (!aligned16(H)) return LORA_ERR_ALIGN;
  }
  if (sync && !aligned16(sync)) return LORA_ERR_ALIGN;
  if (n == 0) return lora_build_segments(row_slot, pool, seg, stream);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const lora::PoolView pv = pool_view(pool);
  const lora::LayerArgs lay{row_slot,
                            pool->A,
                            pool->slot_rank,
                            pool->slot_scale,
                            pool->n_slots,
                            pool_rs(pool),
                            pool->d_in,
                            pool->r_max,
                            pv.proj.rs,
                            pv.proj.n_proj,
                            H,
                            static_cast<uint32_t *>(sync),
                            seg->token_indices,
                            seg->row_segment,
                            seg->segment_offsets,
                            seg->segment_slots,
                            seg->segment_ranks,
                            seg->segment_scales,
                            seg->num_segments,
                            seg->status};
  const hipError_t e = lora::launch_layer(X, ldx, W, ldw, Y, ldy, n, pv, lay, s, wscale);
  if (e != hipErrorNotSupported) return hip_status(e);
  // outside the one-launch case: the two calls
  (void)hipGetLastError();
  st = lora_build_shrink(row_slot, X, ldx, pool, seg, H, stream);
  if (st != LORA_OK) return st;
  return wscale ? lora_linear_fused_fp8w(X, ldx, W, ldw, wscale, H, seg, pool, Y, ldy, stream)
                : lora_linear_fused(X, ldx, W, ldw, H, seg, pool, Y, ldy, stream);
}

}  // namespace

lora_status lora_layer_fused(const int32_t *row_slot, const void *X, int64_t ldx, const void *W,
                             int64_t ldw, const lora_pool *pool, const lora_segments *seg,
                             float *H, void *Y, int64_t ldy, void *sync, void *stream) {
  return layer_call(row_slot, X, ldx, W, ldw, nullptr, pool, seg, H, Y, ldy, sync, stream);
}

lora_status lora_layer_fused_fp8w(const int32_t *row_slot, const void *X, int64_t ldx,
                                  const void *Wq, int64_t ldw, const float *w_scale,
                                  const lora_pool *pool, const lora_segments *seg, float *H,
                                  void *Y, int64_t ldy, void *sync, void *stream) {
  if (!w_scale) return LORA_ERR_NULL;
  return layer_call(row_slot, X, ldx, Wq, ldw, w_scale, pool, seg, H, Y, ldy, sync, stream);
}

lora_status lora_linear_fused_static(const int32_t *row_slot, const void *X, int64_t ldx,
                                     const void *W, int64_t ldw, const lora_pool *pool,
                                     int32_t n_rows, void *Y, int64_t ldy, void *stream) {
  lora_status st = check_pool(pool);
  if (st != LORA_OK) return st;
  if (n_rows < 0) return LORA_ERR_SHAPE;
  if (n_rows > LORA_STATIC_MAX_ROWS || (int64_t)n_rows * pool->r_max > LORA_STATIC_MAX_H)
    return LORA_ERR_SCRATCH;
  if (n_rows > 0 && !row_slot) return LORA_ERR_NULL;
  st = check_matrix(X, ldx, pool->d_in, n_rows);
  if (st != LORA_OK) return st;
  st = check_matrix(W, ldw, pool->d_in, pool->d_out);
  if (st != LORA_OK) return st;
  st = check_matrix(Y, ldy, pool->d_out, n_rows);
  if (st != LORA_OK) return st;
  if (n_rows == 0) return LORA_OK;
  // the scratch's device address on the current device (never the array's
  // host-side name)
  void *base = nullptr;
  if (lora::static_scratch(&base) != hipSuccess) return LORA_ERR_HIP;
  unsigned char *b = static_cast<unsigned char *>(base);
  lora_segments seg;
  seg.n_rows = n_rows;
  seg.max_segments = seg_worst_case(n_rows, pool->n_slots);
  seg.token_indices = reinterpret_cast<int32_t *>(b + lora::kScrTok);
  seg.row_segment = reinterpret_cast<int32_t *>(b + lora::kScrRowSeg);
  seg.segment_offsets = reinterpret_cast<int32_t *>(b + lora::kScrSegOff);
  seg.segment_slots = reinterpret_cast<int32_t *>(b + lora::kScrSegSlot);
  seg.segment_ranks = reinterpret_cast<int32_t *>(b + lora::kScrSegRank);
  seg.segment_scales = reinterpret_cast<float *>(b + lora::kScrSegScale);
  seg.num_segments = reinterpret_cast<int32_t *>(b + lora::kScrNumSeg);
  seg.status = reinterpret_cast<int32_t *>(b + lora::kScrStatus);
  float *H = reinterpret_cast<float *>(b + lora::kScrH);
  // every entry the two calls read is written by them first: the metadata by
  // the build, H[i][0:r] by the shrink for the rows whose term is added
  st = lora_build_shrink(row_slot, X, ldx, pool, &seg, H, stream);
  if (st != LORA_OK) return st;
  return lora_linear_fused(X, ldx, W, ldw, H, &seg, pool, Y, ldy, stream);
}

}  // extern "C"
