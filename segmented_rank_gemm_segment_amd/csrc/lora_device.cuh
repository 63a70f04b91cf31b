// Device-side helpers shared by the HIP kernels of the multi-LoRA layer.
// gfx950 (CDNA4): 64-lane wavefronts, 160 KB LDS per CU, bf16 MFMA.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lora {

constexpr int kWave = 64;

typedef uint16_t bf16_t;  // storage bits
typedef __bf16 mfma_bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// bf16 <-> fp32.  bf16 is the upper half of an IEEE-754 binary32; widening is
// a shift, narrowing rounds to nearest, ties to even.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

typedef __bf16 hw_bf16x2 __attribute__((ext_vector_type(2)));
typedef float hw_f32x2 __attribute__((ext_vector_type(2)));

// Round to nearest even with the gfx950 conversion instruction
// (v_cvt_pk_bf16_f32); NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two packed bf16 (low half = first element) -> two floats.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const hw_f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, hw_bf16x2));
}

// Element traits: 16-byte vectors hold 8 bf16 or 4 fp32.
template <typename T> struct Elem;
template <> struct Elem<bf16_t> {
  static constexpr int kVec = 8;
  __device__ static __forceinline__ void unpack(const uint4 &v, float *out) {
    out[0] = bf16_lo(v.x); out[1] = bf16_hi(v.x);
    out[2] = bf16_lo(v.y); out[3] = bf16_hi(v.y);
    out[4] = bf16_lo(v.z); out[5] = bf16_hi(v.z);
    out[6] = bf16_lo(v.w); out[7] = bf16_hi(v.w);
  }
  __device__ static __forceinline__ uint4 pack(const float *in) {
    uint4 v;
    v.x = pack_bf16x2(in[0], in[1]);
    v.y = pack_bf16x2(in[2], in[3]);
    v.z = pack_bf16x2(in[4], in[5]);
    v.w = pack_bf16x2(in[6], in[7]);
    return v;
  }
  __device__ static __forceinline__ float load1(const bf16_t *p) { return bf16_to_f32(*p); }
  __device__ static __forceinline__ void store1(bf16_t *p, float f) { *p = (bf16_t)f32_to_bf16_rne(f); }
};
template <> struct Elem<float> {
  static constexpr int kVec = 4;
  __device__ static __forceinline__ void unpack(const uint4 &v, float *out) {
    out[0] = __uint_as_float(v.x); out[1] = __uint_as_float(v.y);
    out[2] = __uint_as_float(v.z); out[3] = __uint_as_float(v.w);
  }
  __device__ static __forceinline__ uint4 pack(const float *in) {
    uint4 v;
    v.x = __float_as_uint(in[0]); v.y = __float_as_uint(in[1]);
    v.z = __float_as_uint(in[2]); v.w = __float_as_uint(in[3]);
    return v;
  }
  __device__ static __forceinline__ float load1(const float *p) { return *p; }
  __device__ static __forceinline__ void store1(float *p, float f) { *p = f; }
};

__device__ __forceinline__ uint4 ldg16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ void stg16(void *p, const uint4 &v) { *reinterpret_cast<uint4 *>(p) = v; }

// ---------------------------------------------------------------------------
// Rank handling: the width a segment of true rank r is processed at.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int rank_bucket(int r, int policy, int r_max) {
  if (r <= 0) return 0;
  int b;
  if (policy == 2) {
    b = r_max;                       // padded to the pool's maximum
  } else if (policy == 1) {
    b = r <= 16 ? 16 : 64;           // two buckets {8,16} and {32,64}
  } else {
    b = r <= 8 ? 8 : r <= 16 ? 16 : r <= 32 ? 32 : 64;
  }
  return b < r_max ? b : r_max;
}

// ---------------------------------------------------------------------------
// Wave utilities.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = __lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Mask of the active lanes whose `key` equals this lane's (lanes with
// valid == false take part in no group and get 0).  Loops once per distinct
// key in the wave.
__device__ __forceinline__ uint64_t match_key(int key, bool valid) {
  uint64_t remaining = __ballot(valid);
  uint64_t mine = 0;
  while (remaining) {
    const int leader = __ffsll((unsigned long long)remaining) - 1;  // wave-uniform
    const int lk = __builtin_amdgcn_readlane(key, leader);
    const uint64_t m = __ballot(valid && key == lk);
    if (valid && key == lk) mine = m;
    remaining &= ~m;
  }
  return mine;
}

// Per-segment metadata gathered with one vector load: lanes 0..5 read the
// batch's segment count and segment s's rank, two offsets, slot and scale
// (scale may be null), and every lane gets them by readlane.  One memory
// round trip instead of a chain of dependent scalar loads.  s must index
// the segment arrays in bounds (s < capacity); the caller compares s with S.
struct SegMeta {
  int S, r, o0, o1, slot;
  float sc;
};
__device__ __forceinline__ SegMeta load_seg_meta(int s, const int32_t *num_segments,
                                                 const int32_t *seg_rank, const int32_t *seg_off,
                                                 const int32_t *seg_slot, const float *seg_scale) {
  const int l = __lane_id();
  const int32_t *scale_bits =
      seg_scale != nullptr ? reinterpret_cast<const int32_t *>(seg_scale + s) : num_segments;
  const int32_t *p = l == 0   ? num_segments
                     : l == 1 ? seg_rank + s
                     : l == 2 ? seg_off + s
                     : l == 3 ? seg_off + s + 1
                     : l == 4 ? seg_slot + s
                              : scale_bits;
  const int v = l < 6 ? *p : 0;
  SegMeta m;
  m.S = __builtin_amdgcn_readlane(v, 0);
  m.r = __builtin_amdgcn_readlane(v, 1);
  m.o0 = __builtin_amdgcn_readlane(v, 2);
  m.o1 = __builtin_amdgcn_readlane(v, 3);
  m.slot = __builtin_amdgcn_readlane(v, 4);
  m.sc = __int_as_float(__builtin_amdgcn_readlane(v, 5));
  return m;
}

// Work items of the segmented kernels: the positions of the segment order
// (token_indices) in blocks of at most rb, cut at segment boundaries.  Item
// nb + s is segment s's head: the whole segment if it has at most rb rows,
// else from its start to the next multiple of rb.  Item y < nb is the block
// of positions [y rb, y rb + rb) inside the segment that holds position
// y rb, when that segment is longer than rb rows and does not start there.
// Every position lies in exactly one item, so a batch needs at most nb + S
// items whatever the segment lengths, and no item has more than rb rows.
// A short segment (a decode batch's usual case) is one head item: the
// position items, whose segment is found through two more dependent loads,
// then carry no rows and load nothing more.  ok is false for an item without
// rows (including s >= S).  Items y >= nb need y - nb < cap (the segment arrays'
// capacity); metadata from the build keeps every segment id below it.
struct SegItem {
  bool ok;
  int r, slot, o0, o1, p0, p1;
  float sc;
};
// Positions [p0, p1) of item y given its segment s = [o0, o1) among S.
__device__ __forceinline__ bool item_span(int y, int nb, int rb, int s, int S, int o0, int o1,
                                          int &p0, int &p1) {
  const bool whole = o1 - o0 <= rb;   // short segment: one head item
  if (y < nb) {
    p0 = y * rb;
    p1 = min(p0 + rb, o1);
    return s < S && !whole && o0 != p0 && p0 < p1;
  }
  p0 = o0;
  p1 = whole ? o1 : min(o1, (o0 / rb + 1) * rb);
  return s < S && p0 < p1;
}
// Segment of item y (clamped into the arrays for position items).
__device__ __forceinline__ int item_segment(int y, int nb, int rb, int cap,
                                            const int32_t *token_indices,
                                            const int32_t *row_segment) {
  if (y >= nb) return y - nb;
  const int s = row_segment[token_indices[y * rb]];
  return min(max(s, 0), cap - 1);
}
// One item per wave (y wave-uniform; the segment's fields are read by
// separate lanes).
__device__ __forceinline__ SegItem seg_item(int y, int nb, int rb, int cap,
                                            const int32_t *token_indices,
                                            const int32_t *row_segment,
                                            const int32_t *num_segments, const int32_t *seg_rank,
                                            const int32_t *seg_off, const int32_t *seg_slot,
                                            const float *seg_scale) {
  const int s = item_segment(y, nb, rb, cap, token_indices, row_segment);
  const SegMeta m = load_seg_meta(s, num_segments, seg_rank, seg_off, seg_slot, seg_scale);
  SegItem it;
  it.r = m.r;
  it.slot = m.slot;
  it.sc = m.sc;
  it.o0 = m.o0;
  it.o1 = m.o1;
  it.ok = item_span(y, nb, rb, s, m.S, m.o0, m.o1, it.p0, it.p1);
  return it;
}
// One item per lane (y per lane, S given).
__device__ __forceinline__ SegItem seg_item_lane(int y, int nb, int rb, int cap, int S,
                                                 const int32_t *token_indices,
                                                 const int32_t *row_segment,
                                                 const int32_t *seg_rank, const int32_t *seg_off,
                                                 const int32_t *seg_slot, const float *seg_scale) {
  const int s = item_segment(y, nb, rb, cap, token_indices, row_segment);
  SegItem it;
  it.r = seg_rank[s];
  it.slot = seg_slot[s];
  it.sc = seg_scale[s];
  it.o0 = seg_off[s];
  it.o1 = seg_off[s + 1];
  it.ok = item_span(y, nb, rb, s, S, it.o0, it.o1, it.p0, it.p1);
  return it;
}

// Segment-major items for when only short segments are wanted: item
// y = b cap + s is block b of segment s, [o0 + b rb, o0 + b rb + rb) inside
// the segment.  With y < bps cap, segments of up to bps rb rows are covered.
__device__ __forceinline__ SegItem seg_item_major(int y, int rb, int cap,
                                                  const int32_t *num_segments,
                                                  const int32_t *seg_rank, const int32_t *seg_off,
                                                  const int32_t *seg_slot, const float *seg_scale) {
  const int b = y / cap;
  const int s = y - b * cap;
  const SegMeta m = load_seg_meta(s, num_segments, seg_rank, seg_off, seg_slot, seg_scale);
  SegItem it;
  it.r = m.r;
  it.slot = m.slot;
  it.sc = m.sc;
  it.o0 = m.o0;
  it.o1 = m.o1;
  it.p0 = m.o0 + b * rb;
  it.p1 = min(m.o1, it.p0 + rb);
  it.ok = s < m.S && it.p0 < it.p1;
  return it;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

}  // namespace lora
