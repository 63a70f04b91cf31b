// Host-side launchers of the HIP kernels (internal to liblora).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/lora.h"

namespace lora {

struct SegView {
  int n_rows;
  int max_segments;
  const int32_t *token_indices;
  const int32_t *row_segment;
  const int32_t *seg_off;
  const int32_t *seg_slot;
  const int32_t *seg_rank;
  const float *seg_scale;
  const int32_t *num_segments;
};

constexpr int kMaxProj = 8;

// Stacked projections: output columns [col_off[q], col_off[q + 1]) belong
// to projection q, whose rank rows are [q * rs, q * rs + rank) of a slot
// (rs = r_max / n_proj).  One projection: n_proj = 1, rs = r_max.
struct ProjView {
  int n_proj, rs;
  int col_off[kMaxProj + 1];
};

struct PoolView {
  int n_slots, r_max, d_in, d_out, dtype, policy;
  const void *A;
  const void *Bt;  // [n_slots][rs][d_out]: column j's rank rows are its own projection's
  const void *B;   // optional d_out-major copy of B ([n_slots][d_out][rs]) or null
  const float *dora;   // optional DoRA column factors ([n_slots][d_out]) or null
  ProjView proj;
};

// Projection of output column col (col < col_off[n_proj]).
__host__ __device__ inline int proj_of(const ProjView &pv, int col) {
  int q = 0;
#pragma unroll
  for (int i = 1; i < kMaxProj; ++i) q += (i < pv.n_proj && col >= pv.col_off[i]) ? 1 : 0;
  return q;
}

struct BuildArgs {
  const int32_t *row_slot;
  int n, n_slots, r_max;
  const int32_t *slot_rank;
  const float *slot_scale;
  int32_t *token_indices, *row_segment, *seg_off, *seg_slot, *seg_rank;
  float *seg_scale;
  int32_t *num_segments, *status;
};

hipError_t launch_build_segments(const int32_t *row_slot, int n, int n_slots, int r_max,
                                 const int32_t *slot_rank, const float *slot_scale,
                                 int32_t *token_indices, int32_t *row_segment, int32_t *seg_off,
                                 int32_t *seg_slot, int32_t *seg_rank, float *seg_scale,
                                 int32_t *num_segments, int32_t *status, hipStream_t stream);

hipError_t launch_shrink(const void *X, int64_t ldx, const SegView &seg, const PoolView &pool,
                         float *H, hipStream_t stream);

// Segment build and shrink as one launch when every segment is short: block
// 0 builds the metadata while the other blocks compute H slot by slot from
// the per-row slot ids.  Returns hipErrorNotSupported (nothing launched)
// when the batch is outside that case.
hipError_t launch_build_shrink(const BuildArgs &a, const void *X, int64_t ldx,
                               const PoolView &pool, float *H, hipStream_t stream);

hipError_t launch_expand(const float *H, const SegView &seg, const PoolView &pool, void *Y,
                         int64_t ldy, hipStream_t stream);

// Adapter weights into a slot (one source per projection), then the slot's
// rank and scale alpha / rank.  b_rank_rows: B sources are [rank][ldb]
// (B^T) instead of [d_out_q][ldb].
hipError_t launch_pack_slot(const PoolView &pool, int32_t *slot_rank, float *slot_scale, int slot,
                            int rank, double alpha, const void *const *A_src, const int64_t *lda,
                            const void *const *B_src, const int64_t *ldb, int b_rank_rows,
                            hipStream_t stream);

// slot_scale[a] = alpha[a] / slot_rank[a] (0 for rank <= 0), on the device.
hipError_t launch_set_scales(const int32_t *slot_rank, const double *alpha, float *slot_scale,
                             int n_slots, hipStream_t stream);

// The pool's d_out-major B from its Bt, every slot.
hipError_t launch_write_b(const PoolView &pool, hipStream_t stream);

// DoRA column factors of one slot from its current contents and W.
hipError_t launch_dora_prepare(const PoolView &pool, const int32_t *slot_rank,
                               const float *slot_scale, int slot, const void *W, int64_t ldw,
                               const float *magnitude, hipStream_t stream);

// Y = X W^T (+ fused LoRA when seg/pool/H are given).  With wscale, W holds
// FP8 E4M3 codes (bf16 X and Y) and row j of the weight is wscale[j] times
// its codes.
hipError_t launch_gemm(const void *X, int64_t ldx, const void *W, int64_t ldw, void *Y,
                       int64_t ldy, int M, int K, int N, int dtype, const float *H,
                       const SegView *seg, const PoolView *pool, hipStream_t stream,
                       const float *wscale = nullptr);

// Inputs and outputs of the one-launch layer beyond the product's own
// (layer.cuh): the per-row slot ids and the pool's shrink operands, H, the
// sync buffer (or null) and the segment metadata it writes.
struct LayerArgs {
  const int32_t *row_slot;
  const void *A;              // pool A, [n_slots][r_max][d_in] (bf16)
  const int32_t *slot_rank;
  const float *slot_scale;
  int n_slots, rank_bound;    // rank_bound: ranks above it demote a row to base-only
  int d_in, r_max, rs, n_proj;
  float *H;                   // [n][r_max], written and read back
  uint32_t *sync;             // LORA_LAYER_SYNC_BYTES bytes, or null (no hand-off)
  int32_t *token_indices, *row_segment, *seg_off, *seg_slot, *seg_rank;
  float *seg_scale;
  int32_t *num_segments, *status;
};

// The whole layer in one launch (segment metadata, H, Y) for bf16 pools and
// 1 <= M <= 512 rows; hipErrorNotSupported (nothing launched) otherwise.
// With wscale, W holds FP8 E4M3 codes and row j of the weight is wscale[j]
// times its codes.
hipError_t launch_layer(const void *X, int64_t ldx, const void *W, int64_t ldw, void *Y,
                        int64_t ldy, int M, const PoolView &pool, const LayerArgs &lay,
                        hipStream_t stream, const float *wscale = nullptr);

// Device scratch of the allocation-free call lora_linear_fused_static: byte
// offsets of its parts, each 256-byte aligned.  H is float [n][r_max]; the
// segment arrays hold up to LORA_MAX_SLOTS + 1 segments (min(n, n_slots + 1)).
constexpr size_t kScrAlign = 256;
constexpr size_t scr_up(size_t x) { return (x + kScrAlign - 1) / kScrAlign * kScrAlign; }
constexpr size_t kScrH = 0;
constexpr size_t kScrTok = scr_up(kScrH + 4ull * LORA_STATIC_MAX_H);
constexpr size_t kScrRowSeg = scr_up(kScrTok + 4ull * LORA_STATIC_MAX_ROWS);
constexpr size_t kScrSegOff = scr_up(kScrRowSeg + 4ull * LORA_STATIC_MAX_ROWS);
constexpr size_t kScrSegSlot = scr_up(kScrSegOff + 4ull * (LORA_MAX_SLOTS + 2));
constexpr size_t kScrSegRank = scr_up(kScrSegSlot + 4ull * (LORA_MAX_SLOTS + 1));
constexpr size_t kScrSegScale = scr_up(kScrSegRank + 4ull * (LORA_MAX_SLOTS + 1));
constexpr size_t kScrNumSeg = scr_up(kScrSegScale + 4ull * (LORA_MAX_SLOTS + 1));
constexpr size_t kScrStatus = kScrNumSeg + kScrAlign;
constexpr size_t kScratchBytes = kScrStatus + kScrAlign;

// Device address of this device's scratch (looked up once per device).
hipError_t static_scratch(void **out);

}  // namespace lora
