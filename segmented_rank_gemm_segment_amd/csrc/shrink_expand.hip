// Segmented shrink and expand of the multi-LoRA layer.
//
//   shrink:  H[i][k]  = sum_c X[i][c] A_a[k][c]          k < r_a
//   expand:  Y[i][j] += s_a sum_k H[i][k] B_a[j][k]      (Bt_a[k][j] in the pool)
//
// for every row i of a segment with slot a and rank r_a > 0 (adapter-batching
// page, Multi-LoRA Serving, section "Segmented Kernel 需要哪些 Metadata":
// H_a = X_a A_a^T and Delta Y_a = s_a H_a B_a^T scattered back to the
// original rows).  With DoRA column factors in the pool (ybb.press
// multi-LoRA serving article, section 9.2), the expand multiplies each sum
// by g_a[j] before the rounding: Y[i][j] = g_a[j] (Y[i][j] + s_a ...).
//
// Both are bandwidth-bound segmented GEMV / skinny products.  Work items are
// blocks of at most rb rows of one segment, cut from the segment order at
// multiples of rb and at segment starts (seg_item), so a batch has at most
// n / rb + S of them however long its segments are; a grid of one workgroup
// row per item (striding past a cap) walks them, so no host synchronisation
// sizes the launch.  Adapter
// rows are read once per work item with 16-byte coalesced loads along d, and
// every load of a work item is issued before its arithmetic, so a work item
// costs about one memory round trip.  Each token row lives in exactly one
// segment, so Y is updated without atomics and results are deterministic.
#include <algorithm>
#include <climits>

#include "lds_dma.cuh"
#include "lora_device.cuh"
#include "lora_kernels.h"
#include "shrink_rows.cuh"

namespace lora {
namespace {

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// ----------------------------------------------------------------------------
// shrink (segments below the MFMA threshold): a workgroup takes a block of RB
// rank rows of one segment and walks the segment's rows in groups of RQ.
// d_in is cut into chunks of one 16-byte vector per lane; chunk c belongs to
// wave c mod 4, which loads the RQ token rows and the RB adapter rows of the
// chunk (every load issued before any use) and keeps RQ x RB partial dot
// products per lane.  Each X element of a group is read once per rank block
// and each adapter element once per row group, instead of once per rank row.
// The partials are reduced over the lanes by a halving butterfly (after it,
// lane l holds pair l % 32), then over the waves through LDS in wave order.
// ----------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kShW * kWave, 3) void shrink_kernel(
    const T *__restrict__ X, int64_t ldx, const T *__restrict__ A, const int32_t *token_indices,
    const int32_t *row_segment, const int32_t *seg_off, const int32_t *seg_slot,
    const int32_t *seg_rank, const int32_t *num_segments, int r_max, int rs, int d_in, int policy,
    int rb, int nb, int seg_cap, int long_min, float *__restrict__ H) {
  __shared__ float s_part[kShW][kShNP];
  const int k0 = blockIdx.x * kShRB;       // rank row of the pool
  const int kl0 = k0 % rs;                 // ... and inside its projection's block
  // position blocks first, then the segments' first blocks (seg_item); when
  // the MFMA kernel takes the long segments, only the blocks of the short
  // ones, segment-major (seg_item_major)
  const bool major = long_min != INT_MAX;
  const int n_items = major ? nb * seg_cap : nb + seg_cap;
  // items are walked in ascending order; segment heads past the batch's
  // segment count are empty, and so are all later ones
  const int S = __builtin_amdgcn_readfirstlane(*num_segments);
  for (int item = blockIdx.y; item < n_items; item += gridDim.y) {
    if (!major && item >= nb && item - nb >= S) break;
    if (major && item % seg_cap >= S) continue;
    const SegItem it =
        major ? seg_item_major(item, rb, seg_cap, num_segments, seg_rank, seg_off, seg_slot,
                               nullptr)
              : seg_item(item, nb, rb, seg_cap, token_indices, row_segment, num_segments,
                         seg_rank, seg_off, seg_slot, nullptr);
    if (!it.ok) continue;
    const int R = rank_bucket(it.r, policy, rs);
    if (kl0 >= R) continue;
    if (it.o1 - it.o0 >= long_min) continue;   // long segment: tiled MFMA kernel
    shrink_rows<T>(X, ldx, A, it.slot, k0, kl0, min(kShRB, R - kl0), it.r, r_max, d_in,
                   token_indices, it.p0, it.p1, H, s_part);
  }
}

// ----------------------------------------------------------------------------
// shrink of long segments (prefill): a tiled MFMA product per segment,
//   H[rows of s][0:SN] = X[token_indices[rows]] A_slot[0:SN]^T,
// SM rows x SN rank columns per tile (one 32 x 32 MFMA block per wave),
// K = d_in streamed through a 6-stage LDS ring with direct global->LDS
// loads (the row gather is free: every lane supplies its own source
// address).  The workgroup has one wave per ring buffer: the four MFMA
// waves and two that only load.  Wave w owns ring buffer w and alone fills
// every stage that lands there, so a wave never has more than one stage in
// flight, and before a stage is read its owner waits for all of its loads
// (vmcnt(0)) and the workgroup passes a barrier: no wait depends on the
// order in which DMAs complete.  Every wave walks the same items and
// barriers (all control flow is workgroup-uniform).  Each X row is read once per segment tile instead of once per
// rank row.  Work items are the position blocks of the segment order
// (seg_item with rb = SM) of segments of at least kLongRows rows, times the
// rank tiles (blockIdx.x).  Rank rows past R are not fetched (their loads
// re-read row R-1); columns k >= r are not stored.
// ----------------------------------------------------------------------------
constexpr int kLongRows = 128;   // segments at least this long take the MFMA path
constexpr int kMfmaShrinkMinBatch = 2048;
constexpr int kMfmaShrinkFillTiles = 256;   // 64 x 64 work items that fill the CUs
constexpr int kShortRowBlk = 8;             // rows per GEMV item beside the MFMA kernel
constexpr int kSStages = 6;   // ring buffers = waves of the workgroup

template <int SM, int SN>
__global__ __launch_bounds__(kSStages * kWave) void shrink_mfma_kernel(
    const bf16_t *__restrict__ X, int64_t ldx, const bf16_t *__restrict__ A,
    const int32_t *token_indices, const int32_t *row_segment, const int32_t *seg_off,
    const int32_t *seg_slot, const int32_t *seg_rank, const int32_t *num_segments, int r_max,
    int rs, int d_in, int policy, int nb, int seg_cap, float *__restrict__ H) {
  constexpr int NWN = SN / 32;                      // waves along the rank columns
  constexpr int NWC = (SM / 32) * NWN;              // MFMA waves
  constexpr int AI = SM / 8, BI = SN / 8;            // 1 KB instructions of a stage (owner)
  static_assert(NWC <= kSStages, "one owner wave per ring buffer, MFMA waves among them");
  constexpr int STAGE = (SM + SN) * 128;
  constexpr int BK = 64;
  __shared__ __align__(16) unsigned char smem[kSStages * STAGE];
  const int tid = threadIdx.x;
  const int l = tid & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);
  const bool mfma_wave = wid < NWC;
  const int wm = (wid % NWC) / NWN, wn = wid % NWN;
  // 128-byte LDS rows, chunk c of row r at c ^ ((r >> 1) & 7): 16
  // consecutive rows at one chunk hit 16 distinct bank groups
  const int r8 = l >> 3;
  const uint32_t sbase = lds_offset(smem);
  const int a_row_off = (wm * 32 + (l & 31)) * 128;
  const int b_row_off = SM * 128 + (wn * 32 + (l & 31)) * 128;
  int chunk_off[BK / 16];
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) chunk_off[kk] = (((kk * 2 + (l >> 5)) ^ ((l >> 1) & 7)) * 16);
  // logical chunk of lane l in instruction i (rows i * 8 + l / 8 of the
  // stage's A or B part)
  int alc[AI], blc[BI];
#pragma unroll
  for (int i = 0; i < AI; ++i) alc[i] = (l & 7) ^ (((i * 8 + r8) >> 1) & 7);
#pragma unroll
  for (int i = 0; i < BI; ++i) blc[i] = (l & 7) ^ (((i * 8 + r8) >> 1) & 7);
  const int KT = (d_in + BK - 1) / BK;
  const bool ktail = (d_in % BK) != 0;
  const int S = __builtin_amdgcn_readfirstlane(*num_segments);
  const int rt = blockIdx.x;                        // rank tile of SN pool rank rows

  // position blocks first, then the segments' first blocks (seg_item), in
  // ascending order: heads past the batch's segment count end the walk
  for (int item = blockIdx.y; item < nb + seg_cap; item += gridDim.y) {
    if (item >= nb && item - nb >= S) break;
    const SegItem it = seg_item(item, nb, SM, seg_cap, token_indices, row_segment, num_segments,
                                seg_rank, seg_off, seg_slot, nullptr);
    if (!it.ok || it.o1 - it.o0 < kLongRows) continue;
    const int R = rank_bucket(it.r, policy, rs);
    if (R == 0) continue;
    const int p0 = it.p0, p1 = it.p1;
    const int slot = it.slot, r = it.r;

    const bf16_t *asrc[AI];
    const bf16_t *bsrc[BI];
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      const int p = min(p0 + i * 8 + r8, p1 - 1);
      asrc[i] = X + (int64_t)token_indices[p] * ldx + alc[i] * 8;
    }
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      // pool rank row kg, kl rows into its projection's block; rows past the
      // processed width R re-read the block's last processed row (in the
      // slot) and are not stored
      const int kg = rt * SN + i * 8 + r8;
      const int kl = kg % rs;
      const int k = min(kl < R ? kg : kg - kl + R - 1, r_max - 1);
      bsrc[i] = A + ((int64_t)slot * r_max + k) * d_in + blc[i] * 8;
    }
    // the whole stage at K position k0 into buffer `stage` (its owner only);
    // a chunk past d_in reads the row's first chunk instead (in bounds) and
    // is zeroed before use
    auto issue = [&](int stage, int k0) {
      const uint32_t dst = __builtin_amdgcn_readfirstlane(sbase + stage * STAGE);
      if (k0 + BK <= d_in) {
#pragma unroll
        for (int i = 0; i < AI; ++i) dma16(dst + i * 1024, asrc[i] + k0);
#pragma unroll
        for (int i = 0; i < BI; ++i) dma16(dst + SM * 128 + i * 1024, bsrc[i] + k0);
      } else {
#pragma unroll
        for (int i = 0; i < AI; ++i)
          dma16(dst + i * 1024, asrc[i] + ((k0 + alc[i] * 8 < d_in) ? k0 : -alc[i] * 8));
#pragma unroll
        for (int i = 0; i < BI; ++i)
          dma16(dst + SM * 128 + i * 1024, bsrc[i] + ((k0 + blc[i] * 8 < d_in) ? k0 : -blc[i] * 8));
      }
    };
    f32x16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.f;
    // prologue: stages 0 .. kSStages - 2, stage w by wave w
    if (wid < kSStages - 1 && wid < KT) issue(wid, wid * BK);
    for (int kt = 0; kt < KT; ++kt) {
      // stage kt lands: its owner waits for its one stage in flight
      if (wid == kt % kSStages) {
        vm_wait<0>();
        if (ktail && kt == KT - 1) {
          unsigned char *st = smem + wid * STAGE;
#pragma unroll
          for (int i = 0; i < AI; ++i)
            if (kt * BK + alc[i] * 8 >= d_in)
              *reinterpret_cast<u32x4 *>(st + i * 1024 + l * 16) = u32x4{0, 0, 0, 0};
#pragma unroll
          for (int i = 0; i < BI; ++i)
            if (kt * BK + blc[i] * 8 >= d_in)
              *reinterpret_cast<u32x4 *>(st + SM * 128 + i * 1024 + l * 16) = u32x4{0, 0, 0, 0};
        }
      }
      lgkm_barrier();
      // the buffer read in step kt - 1 is free: its owner loads stage
      // kt + kSStages - 1 into it
      const int nxt = kt + kSStages - 1;
      if (nxt < KT && wid == nxt % kSStages) issue(wid, nxt * BK);
      if (mfma_wave) {
        const unsigned char *st = smem + (kt % kSStages) * STAGE;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
          const mfma_bf16x8 af = as_bf16x8(*reinterpret_cast<const u32x4 *>(st + a_row_off + chunk_off[kk]));
          const mfma_bf16x8 bf = as_bf16x8(*reinterpret_cast<const u32x4 *>(st + b_row_off + chunk_off[kk]));
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf, acc, 0, 0, 0);
        }
      }
    }
    if (mfma_wave) {
      const int k = rt * SN + wn * 32 + (l & 31);
      const bool kok = k < r_max && k % rs < r;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int p = p0 + wm * 32 + acc_row(v, l);
        if (p < p1 && kok) H[(int64_t)token_indices[p] * r_max + k] = acc[v];
      }
    }
    lgkm_barrier();  // the next item's loads reuse the stages
  }
}

// ----------------------------------------------------------------------------
// expand: a wavefront covers 16 column vectors x 4 rank quarters.  Rank rows
// come in blocks of 4; lane (cv = l % 16, kq = l / 16) owns blocks kq,
// kq + 4, ... below R of its column vector (held in registers for the whole
// work item).  Where a rank row is summed never depends on R, so every rank
// policy gives the same bits.  Rows are processed four at a time: every lane
// loads the four rows' H values of its blocks (float4) and lane kq also
// loads Y of row kq; the four quarters are combined with two xor-shuffles.
// No LDS, no barriers.
// ----------------------------------------------------------------------------
constexpr int kExpWaves = 4;
constexpr int kExpSub = 4;    // rows per pass (one Y row per rank quarter)

template <typename T, int R, bool DORA>
__device__ __forceinline__ void expand_item(const float *__restrict__ H, const T *bt,
                                            const float *gp, int d_out, bool active, int r,
                                            float sc, int p0, int p1,
                                            const int32_t *token_indices, int r_max, int rs, T *Y,
                                            int64_t ldy, int col, int lane) {
  constexpr int V = Elem<T>::kVec;
  constexpr int NB = (R + 15) / 16;   // rank blocks of 4 per lane (at most)
  const int kq = lane >> 4;
  // the first group's row indices travel ahead of the adapter rows (one
  // vector load: lane q holds row q, lanes past the group repeat its last
  // row), so waiting for them does not wait for the adapter rows
  int tv = token_indices[p0 + min(lane, min(kExpSub, p1 - p0) - 1)];
  __builtin_amdgcn_sched_barrier(0);
  uint4 braw[NB][4];
  bool blk_ok[NB];
#pragma unroll
  for (int jb = 0; jb < NB; ++jb) {
    const int k0 = 4 * (kq + 4 * jb);
    blk_ok[jb] = k0 < R;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // rank rows in [r, R) are read, as a kernel compiled for width R
      // would; rows past the block are clamped into the slot.  Values are
      // masked where they are used (rank rows >= r) and inactive columns
      // are never stored.
      braw[jb][e] = ldg16(bt + (int64_t)min(k0 + e, rs - 1) * d_out);
    }
  }
  // DoRA column factors of the lane's V columns (same for every row)
  float gv[V];
  if constexpr (DORA) {
#pragma unroll
    for (int e4 = 0; e4 < V; e4 += 4) {
      const float4 t = *reinterpret_cast<const float4 *>(gp + e4);
      gv[e4] = t.x; gv[e4 + 1] = t.y; gv[e4 + 2] = t.z; gv[e4 + 3] = t.w;
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // one group of up to kExpSub rows whose indices are in tv
  auto group = [&](int q0, int tv) __attribute__((always_inline)) {
    const int nq = min(kExpSub, p1 - q0);
    int rows[kExpSub];
#pragma unroll
    for (int q = 0; q < kExpSub; ++q) rows[q] = __builtin_amdgcn_readlane(tv, q);
    const int myq = kq;  // Y row updated by this lane
    const int yrow = rows[0] * (myq == 0) + rows[1] * (myq == 1) + rows[2] * (myq == 2) +
                     rows[3] * (myq == 3);
    // inactive columns read column 0 of the row (in bounds) and never store.
    // An ordinary load, kept with the H loads (ahead of the arithmetic) by the
    // scheduling barrier below; the compiler waits for it before its use.
    const uint4 y4 = ldg16(Y + (int64_t)yrow * ldy + (active ? col : 0));
    float4 hv[kExpSub][NB];
#pragma unroll
    for (int q = 0; q < kExpSub; ++q)
#pragma unroll
      for (int jb = 0; jb < NB; ++jb) {
        // block start k0 < R <= r_max and r_max % 8 == 0: the float4 is in
        // the row; blocks past R read the row's last float4 and are zeroed
        // (masked where used, by the same rank test as the adapter rows)
        const int k0 = min(4 * (kq + 4 * jb), rs - 4);
        hv[q][jb] = *reinterpret_cast<const float4 *>(H + (int64_t)rows[q] * r_max + k0);
      }
    __builtin_amdgcn_sched_barrier(0);   // Y and H loads issued before any use
    // the adapter rows are first needed here, after this group's loads are
    // issued (the empty asm keeps their unpacking here: the compiler would
    // otherwise hoist it, and the wait for them, above those loads)
    uint4 bcur[NB][4];
#pragma unroll
    for (int jb = 0; jb < NB; ++jb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bcur[jb][e] = braw[jb][e];
        asm volatile("" : "+v"(bcur[jb][e].x), "+v"(bcur[jb][e].y), "+v"(bcur[jb][e].z),
                     "+v"(bcur[jb][e].w));
      }
    float acc[kExpSub][V];
#pragma unroll
    for (int q = 0; q < kExpSub; ++q)
#pragma unroll
      for (int e = 0; e < V; ++e) acc[q][e] = 0.f;
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) {
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int k = 4 * (kq + 4 * jb) + e4;
        const bool live = blk_ok[jb] && k < r;
        float bv[V];
        Elem<T>::unpack(bcur[jb][e4], bv);
#pragma unroll
        for (int e = 0; e < V; ++e) bv[e] = live ? bv[e] : 0.f;
#pragma unroll
        for (int q = 0; q < kExpSub; ++q) {
          const float4 h4 = hv[q][jb];
          const float hq = e4 == 0 ? h4.x : e4 == 1 ? h4.y : e4 == 2 ? h4.z : h4.w;
          const float h = live ? hq : 0.f;
#pragma unroll
          for (int e = 0; e < V; ++e) acc[q][e] = fmaf(h, bv[e], acc[q][e]);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kExpSub; ++q)
#pragma unroll
      for (int e = 0; e < V; ++e) {
        acc[q][e] += __shfl_xor(acc[q][e], 16);
        acc[q][e] += __shfl_xor(acc[q][e], 32);
      }
    // the sum is formed in every lane (so the Y load above is not sunk into
    // the guarded store) and stored by the lanes that own a row
    float yv[V];
    Elem<T>::unpack(y4, yv);
    float out[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
      // select this lane's row without dynamic register indexing
      float a = 0.f;
#pragma unroll
      for (int q = 0; q < kExpSub; ++q) a = (q == myq) ? acc[q][e] : a;
      out[e] = fmaf(sc, a, yv[e]);
      if constexpr (DORA) out[e] *= gv[e];
    }
    const uint4 packed = Elem<T>::pack(out);
    if (active && myq < nq) stg16(Y + (int64_t)yrow * ldy + col, packed);
  };
  // the first group straight after the adapter-row loads, the rest in a loop
  group(p0, tv);
  for (int q0 = p0 + kExpSub; q0 < p1; q0 += kExpSub)
    group(q0, token_indices[q0 + min(lane, min(kExpSub, p1 - q0) - 1)]);
}

// RMAX = the pool's r_max: only rank buckets up to it are compiled in, so a
// rank-16 pool does not pay the registers of the rank-64 case.
template <typename T, int RMAX, bool DORA>
__global__ __launch_bounds__(kExpWaves * kWave) void expand_kernel(
    const float *__restrict__ H, const T *__restrict__ Bt, const float *__restrict__ dora,
    const int32_t *token_indices, const int32_t *row_segment, const int32_t *seg_off,
    const int32_t *seg_slot, const int32_t *seg_rank, const float *seg_scale,
    const int32_t *num_segments, int r_max, int d_out, int policy, int rb, int nb, int seg_cap,
    T *__restrict__ Y, int64_t ldy, ProjView proj) {
  constexpr int V = Elem<T>::kVec;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int col = ((blockIdx.x * kExpWaves + wave) * 16 + (lane & 15)) * V;
  const bool active = col < d_out;
  // the lane's columns belong to one projection (its offsets are multiples
  // of 8): its rank entries start at q * rs in each H row; the slot's rs
  // rank rows of Bt hold every column's own projection
  const int qoff = proj_of(proj, active ? col : 0) * proj.rs;
  // position blocks first, then the segments' first blocks (seg_item), in
  // ascending order: heads past the batch's segment count are empty, and so
  // are all later ones
  const int S = __builtin_amdgcn_readfirstlane(*num_segments);
  for (int item = blockIdx.y; item < nb + seg_cap; item += gridDim.y) {
    if (item >= nb && item - nb >= S) break;
    const SegItem it = seg_item(item, nb, rb, seg_cap, token_indices, row_segment, num_segments,
                                seg_rank, seg_off, seg_slot, seg_scale);
    if (!it.ok) continue;
    const int r = it.r, slot = it.slot;
    const float sc = it.sc;
    const int R = rank_bucket(r, policy, proj.rs);
    if (R == 0) continue;
    const int p0 = it.p0, p1 = it.p1;
    const T *bt = Bt + (int64_t)slot * proj.rs * d_out + (active ? col : 0);
    const float *gp = DORA ? dora + (int64_t)slot * d_out + (active ? col : 0) : nullptr;
    const float *Hq = H + qoff;   // the projection's ranks in each H row
    const int rs = proj.rs;
    if (R == 8) {
      expand_item<T, 8, DORA>(Hq, bt, gp, d_out, active, r, sc, p0, p1, token_indices, r_max, rs,
                              Y, ldy, col, lane);
    } else if (RMAX >= 16 && R == 16) {
      expand_item<T, (RMAX >= 16 ? 16 : 8), DORA>(Hq, bt, gp, d_out, active, r, sc, p0, p1,
                                                  token_indices, r_max, rs, Y, ldy, col, lane);
    } else if (RMAX >= 32 && R == 32) {
      expand_item<T, (RMAX >= 32 ? 32 : 8), DORA>(Hq, bt, gp, d_out, active, r, sc, p0, p1,
                                                  token_indices, r_max, rs, Y, ldy, col, lane);
    } else if (RMAX >= 64) {
      expand_item<T, (RMAX >= 64 ? 64 : 8), DORA>(Hq, bt, gp, d_out, active, r, sc, p0, p1,
                                                  token_indices, r_max, rs, Y, ldy, col, lane);
    }
  }
}

inline int seg_bound(int n_rows, int n_slots, int max_segments) {
  int b = n_rows < n_slots + 1 ? n_rows : n_slots + 1;
  return b < max_segments ? b : max_segments;
}

// Workgroup rows for `items` work items when each row has `x` workgroups:
// one row per item, but at most kMaxItemWGs workgroups in all; the rows then
// walk the items with a stride.  Several rounds of workgroups at these
// kernels' occupancy (2 or fewer per CU at 256 VGPRs), so a large bound on
// the segment count (a 1000-slot pool) no longer launches thousands of
// empty workgroups.
constexpr int kMaxItemWGs = 2048;
inline int grid_items(int items, int x) {
  int cap = kMaxItemWGs / (x > 0 ? x : 1);
  cap = cap > 1 ? cap : 1;
  return items < cap ? (items > 0 ? items : 1) : cap;
}

// ----------------------------------------------------------------------------
// Expand of bf16 batches whose pool keeps B d_out-major (the batches are
// chosen by expand_on_mfma): per work item (at most kRowBlk rows of one
// segment: position blocks of kRowBlk rows and segment heads, as the GEMV
// expand cuts its items) and 256 output columns, the increment is a product
// over the rank, taken on the matrix cores in the orientation
// D^T = B_a (columns x ranks) (s_a H)^T (ranks x rows), with the item's Y as
// the accumulator's initial value: D = Y + s_a H B_a^T in fp32, times the
// DoRA factor, rounded once.  s_a H is fp32, so each value enters as a bf16
// high part plus the bf16 remainder (two products; about 16 significant
// bits, while B is bf16 and exact).  Rank entries past r are zeroed in both
// operands (a padded slot's values there are never used); the launcher
// gives each workgroup's columns a single projection.
//
// Y moves between HBM and the workgroup only in whole 512-byte row pieces
// (16 bytes per lane, 32 lanes per row), through an LDS tile: the
// accumulators read their start values from it and write the rounded
// results back in place, and the rows leave it the way they came.  The
// tile's 16-byte chunks are XOR-swizzled by row so that the accumulator
// layout (lanes along rows) spreads its reads and writes over the banks (at
// most two lanes of a half-wave on one bank).
// The item's s_a H rows are split into LDS once; each wave reads its
// operand fragments from there and its 64 columns of B from memory.
//
// A workgroup walks the items blockIdx.y + t gridDim.y.  It first reads the
// metadata of all of them at once (one item per thread) into an LDS table
// of the items that have rows; each item's row indices are requested during
// the previous item.
// ----------------------------------------------------------------------------
constexpr int kXmCols = 256;   // columns per workgroup: 4 waves x 64
constexpr int kXmPitch = 144;  // bytes per LDS row of 64 bf16 ranks (+16: spreads the banks)
constexpr int kXmItems = 64;   // items per workgroup at most (its metadata table)
constexpr int kXmRowBytes = kXmCols * 2;
static_assert(kRowBlk == 64, "an item's rows fill the two 32-row blocks of a lane");

__device__ __forceinline__ int xm_chunk(int row, int c) { return c ^ (row & 31); }

template <bool DORA>
__global__ __launch_bounds__(4 * kWave, 3) void expand_mfma_kernel(
    const float *__restrict__ H, const bf16_t *__restrict__ Bn, const float *__restrict__ dora,
    const int32_t *token_indices, const int32_t *row_segment, const int32_t *seg_off,
    const int32_t *seg_slot, const int32_t *seg_rank, const float *seg_scale,
    const int32_t *num_segments, int r_max, int d_out, int policy, int nb, int seg_cap,
    bf16_t *__restrict__ Y, int64_t ldy, ProjView proj) {
  __shared__ __align__(16) unsigned char s_y[kRowBlk * kXmRowBytes];  // the item's Y tile
  __shared__ __align__(16) unsigned char s_h[2][kRowBlk * kXmPitch];  // s_a H: high, low parts
  __shared__ int s_tab[5][kXmItems];     // slot, rank, scale bits, p0, p1 of the items with rows
  __shared__ int s_rows[2][kRowBlk];     // row indices of the current and the next item
  __shared__ int s_cnt[4];
  const int tid = threadIdx.x;
  const int l = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int l32 = l & 31, hf = l >> 5;
  const int c0 = blockIdx.x * kXmCols;               // the workgroup's first column
  const int nw = c0 + wave * 64;                     // the wave's first column
  const int rs = proj.rs;
  const int qoff = proj_of(proj, min(c0, d_out - 1)) * rs;
  {
    // item blockIdx.y + tid gridDim.y (the launcher keeps the walk within
    // kXmItems), kept if it has rows and a nonzero rank
    const int S = *num_segments;
    const int y = blockIdx.y + tid * gridDim.y;
    bool keep = false;
    SegItem it{};
    if (tid < kXmItems && y < nb + seg_cap && (y < nb || y - nb < S)) {
      it = seg_item_lane(y, nb, kRowBlk, seg_cap, S, token_indices, row_segment, seg_rank,
                         seg_off, seg_slot, seg_scale);
      keep = it.ok && rank_bucket(it.r, policy, rs) > 0;
    }
    // compact in item order: wave prefix by ballot, then the waves' counts
    const uint64_t bal = __ballot(keep);
    const int before = __popcll(bal & ((1ull << l) - 1ull));
    if (l == 0) s_cnt[wave] = __popcll(bal);
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += s_cnt[w];
    if (keep) {
      const int k = base + before;
      s_tab[0][k] = it.slot;
      s_tab[1][k] = it.r;
      s_tab[2][k] = __float_as_int(it.sc);
      s_tab[3][k] = it.p0;
      s_tab[4][k] = it.p1;
    }
    __syncthreads();
  }
  const int K = s_cnt[0] + s_cnt[1] + s_cnt[2] + s_cnt[3];
  if (K == 0) return;
  // row index of row t of item k (past the item's end: its last row, never stored)
  auto row_of = [&](int k, int t) {
    const int p0 = s_tab[3][k], nrow = s_tab[4][k] - p0;
    return token_indices[p0 + min(t, nrow - 1)];
  };
  if (tid < kRowBlk) s_rows[0][tid] = row_of(0, tid);
  __syncthreads();
  const int hm = tid >> 2, hc = (tid & 3) * 16;   // the H row and first rank this thread splits
  const int yr = tid >> 5, yc = tid & 31;         // Y pieces: rows yr + 8 i, chunk yc
  const int ycol = min(c0 + yc * 8, d_out - 8);   // (clamped into the row; never stored past it)
  const int hk = min(hc, rs - 16 > 0 ? rs - 16 : 0);
  // the row loads of item k: Y rows in 16-byte pieces, this thread's 16
  // ranks of H row hm (ranks past r, and past rs, zeroed where used), the
  // next item's row indices (the last item reads its own again)
  u32x4 ly[kRowBlk / 8];
  float4 lh[4];
  int lnxt;
  // (the loads are unconditional: rows past the item's end repeat its last
  // row; skipping them by branches measured heavy register spills)
  auto load_rows = [&](int k) __attribute__((always_inline)) {
    const int cq = k & 1;
#pragma unroll
    for (int i = 0; i < kRowBlk / 8; ++i)
      ly[i] = *reinterpret_cast<const u32x4 *>(Y + (int64_t)s_rows[cq][yr + 8 * i] * ldy + ycol);
    const int hrow = s_rows[cq][hm];
#pragma unroll
    for (int c = 0; c < 4; ++c)
      lh[c] = *reinterpret_cast<const float4 *>(H + (int64_t)hrow * r_max + qoff +
                                                min(hk + 4 * c, rs - 4));
    lnxt = row_of(min(k + 1, K - 1), tid & (kRowBlk - 1));
  };
  load_rows(0);
  for (int k = 0; k < K; ++k) {
    const int cur = k & 1;
    const int slot = __builtin_amdgcn_readfirstlane(s_tab[0][k]);
    const int r = __builtin_amdgcn_readfirstlane(s_tab[1][k]);
    const float sc = __int_as_float(__builtin_amdgcn_readfirstlane(s_tab[2][k]));
    const int nrow = __builtin_amdgcn_readfirstlane(s_tab[4][k] - s_tab[3][k]);
    const int R = rank_bucket(r, policy, rs);
    // B rows of the wave's columns, every rank step (ranks past r zeroed
    // below); the steps past the rank bucket R read a chunk inside [0, R)
    // instead (unused), so no load reaches sectors of ranks the item lacks
    const bf16_t *bs = Bn + (int64_t)slot * d_out * rs;
    u32x4 bv[4][2];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = min(nw + 32 * j + l32, d_out - 1);
        const int kc = min(ks * 16 + hf * 8, R - 8);
        bv[ks][j] = *reinterpret_cast<const u32x4 *>(bs + (int64_t)n * rs + kc);
      }
    // the 32-row blocks holding the item's rows: only those are computed,
    // and only the item's 8-row groups enter and leave the tile (tile rows
    // past its end keep stale values, which reach only accumulator rows that
    // are never stored: each output row depends on its own H and Y rows)
    const int nmb = nrow > 32 ? 2 : 1;
    {
      const float hv[16] = {lh[0].x, lh[0].y, lh[0].z, lh[0].w, lh[1].x, lh[1].y, lh[1].z, lh[1].w,
                            lh[2].x, lh[2].y, lh[2].z, lh[2].w, lh[3].x, lh[3].y, lh[3].z, lh[3].w};
      u32x4 phi[2], plo[2];
#pragma unroll
      for (int e2 = 0; e2 < 8; ++e2) {
        const int kk = hc + 2 * e2;
        const float v0 = kk < r ? sc * hv[2 * e2] : 0.f;
        const float v1 = kk + 1 < r ? sc * hv[2 * e2 + 1] : 0.f;
        const uint32_t hw = pack_bf16x2(v0, v1);
        phi[e2 >> 2][e2 & 3] = hw;
        plo[e2 >> 2][e2 & 3] = pack_bf16x2(v0 - bf16_lo(hw), v1 - bf16_hi(hw));
      }
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        *reinterpret_cast<u32x4 *>(s_h[0] + hm * kXmPitch + (hc + 8 * h2) * 2) = phi[h2];
        *reinterpret_cast<u32x4 *>(s_h[1] + hm * kXmPitch + (hc + 8 * h2) * 2) = plo[h2];
      }
    }
#pragma unroll
    for (int i = 0; i < kRowBlk / 8; ++i) {
      const int row = yr + 8 * i;
      if (8 * i < nrow)
        *reinterpret_cast<u32x4 *>(s_y + row * kXmRowBytes + xm_chunk(row, yc) * 16) = ly[i];
    }
    if (tid < kRowBlk) s_rows[cur ^ 1][tid] = lnxt;
    __syncthreads();
    // accumulators start at Y (accumulator v = 4 g + e of block (j, mb):
    // column nw + 32 j + 8 g + 4 hf + e, row m = l32 + 32 mb; its 8 bytes in
    // the tile at chunk wave * 8 + 4 j + g, offset 8 hf)
    f32x16 acc[2][2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int m = l32 + 32 * mb;
          const uint2 y = *reinterpret_cast<const uint2 *>(
              s_y + m * kXmRowBytes + xm_chunk(m, wave * 8 + 4 * j + g) * 16 + hf * 8);
          acc[j][mb][4 * g + 0] = bf16_lo(y.x);
          acc[j][mb][4 * g + 1] = bf16_hi(y.x);
          acc[j][mb][4 * g + 2] = bf16_lo(y.y);
          acc[j][mb][4 * g + 3] = bf16_hi(y.y);
        }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks * 16 >= R) break;
      const int k0 = ks * 16 + hf * 8;              // the lane's first rank of the step
      mfma_bf16x8 a[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        u32x4 v = bv[ks][j];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const int kk = k0 + 2 * e2;
          v[e2] &= (kk < r ? 0x0000ffffu : 0u) | (kk + 1 < r ? 0xffff0000u : 0u);
        }
        a[j] = as_bf16x8(v);
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        if (mb >= nmb) break;
        const int off = (l32 + 32 * mb) * kXmPitch + k0 * 2;
        const mfma_bf16x8 bh = as_bf16x8(*reinterpret_cast<const u32x4 *>(s_h[0] + off));
        const mfma_bf16x8 bl = as_bf16x8(*reinterpret_cast<const u32x4 *>(s_h[1] + off));
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[j][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], bh, acc[j][mb], 0, 0, 0);
          acc[j][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], bl, acc[j][mb], 0, 0, 0);
        }
      }
    }
    // rounded results back into the tile, each lane where it read
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float gv[4] = {1.f, 1.f, 1.f, 1.f};
        if constexpr (DORA) {
          const int n = nw + 32 * j + 8 * g + 4 * hf;
          const float4 t = *reinterpret_cast<const float4 *>(
              dora + (int64_t)slot * d_out + min(n, d_out - 4));
          gv[0] = t.x; gv[1] = t.y; gv[2] = t.z; gv[3] = t.w;
        }
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          if (mb >= nmb) break;
          const int m = l32 + 32 * mb;
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            o[e] = acc[j][mb][4 * g + e];
            if constexpr (DORA) o[e] *= gv[e];
          }
          *reinterpret_cast<uint2 *>(s_y + m * kXmRowBytes + xm_chunk(m, wave * 8 + 4 * j + g) * 16 +
                                     hf * 8) = uint2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
        }
      }
    __syncthreads();
    // the next item's loads go out before this item's stores, so waiting for
    // them later never waits for the stores (the last item loads itself again)
    load_rows(min(k + 1, K - 1));
    // the rows leave in 16-byte pieces
#pragma unroll
    for (int i = 0; i < kRowBlk / 8; ++i) {
      const int row = yr + 8 * i;
      if (8 * i >= nrow) break;
      const u32x4 v = *reinterpret_cast<const u32x4 *>(s_y + row * kXmRowBytes + xm_chunk(row, yc) * 16);
      if (row < nrow && c0 + yc * 8 < d_out)
        *reinterpret_cast<u32x4 *>(Y + (int64_t)s_rows[cur][row] * ldy + c0 + yc * 8) = v;
    }
    __syncthreads();   // the tile, the H split and s_rows[cur] are rewritten for the next item
  }
}

}  // namespace

template <int SM, int SN>
void launch_shrink_mfma(const void *X, int64_t ldx, const SegView &seg, const PoolView &pool,
                        float *H, hipStream_t stream) {
  const int n = seg.n_rows;
  const int nb = (n + SM - 1) / SM;
  const int S_bound = seg_bound(n, pool.n_slots, seg.max_segments);
  const int nrt = (pool.r_max + SN - 1) / SN;        // rank tiles of SN pool rank rows
  dim3 grid(nrt, grid_items(nb + S_bound, nrt));
  hipLaunchKernelGGL((shrink_mfma_kernel<SM, SN>), grid, dim3(kSStages * kWave), 0,
                     stream, (const bf16_t *)X, ldx, (const bf16_t *)pool.A, seg.token_indices,
                     seg.row_segment, seg.seg_off, seg.seg_slot, seg.seg_rank, seg.num_segments,
                     pool.r_max, pool.proj.rs, pool.d_in, pool.policy, nb, S_bound, H);
}

// Rows per work item: short blocks spread the rows of a long segment over
// many workgroups (a Zipf-skewed decode batch has segments of a hundred rows
// next to single rows); large batches take longer blocks, which read each
// adapter row fewer times.
inline int row_block(int n) { return n >= kLargeBatch ? kRowBlk : kRowBlkSmall; }

hipError_t launch_shrink(const void *X, int64_t ldx, const SegView &seg, const PoolView &pool,
                         float *H, hipStream_t stream) {
  const int n = seg.n_rows;
  const int rb = row_block(n);
  const int nb = (n + rb - 1) / rb;
  const int S_bound = seg_bound(n, pool.n_slots, seg.max_segments);
  // long segments (>= kLongRows rows) go to the tiled MFMA kernel in large
  // (prefill-sized) batches; decode-sized batches keep every segment on the
  // GEMV kernel and launch nothing more
  const bool use_mfma = pool.dtype == 1 && n >= kMfmaShrinkMinBatch;
  const int long_min = use_mfma ? kLongRows : INT_MAX;
  // one workgroup row per item up to the cap (an item without rows exits
  // after its metadata read).  With the MFMA kernel on the long segments, the
  // GEMV kernel walks the first blocks of every segment (nb of them below
  // kLongRows rows) instead of the position blocks.
  // The short segments of such a batch (decode rows beside prefill requests)
  // go in blocks of kShortRowBlk rows, so that the row groups of one segment
  // run in separate workgroups instead of one after another (each group
  // reads the adapter's rank rows over all of d_in, tens of KB per rank
  // block at d_in 8192 and more).
  const int rb_g = use_mfma ? kShortRowBlk : rb;
  const int nb_g = use_mfma ? (kLongRows + rb_g - 1) / rb_g : nb;
  const int items = use_mfma ? nb_g * S_bound : nb + S_bound;
  const int gx = (pool.r_max + kShRB - 1) / kShRB;
  dim3 grid(gx, grid_items(items, gx));
  dim3 block(kShW * kWave);
  if (pool.dtype == 1) {
    hipLaunchKernelGGL((shrink_kernel<bf16_t>), grid, block, 0, stream,
                       (const bf16_t *)X, ldx, (const bf16_t *)pool.A, seg.token_indices,
                       seg.row_segment, seg.seg_off, seg.seg_slot, seg.seg_rank, seg.num_segments,
                       pool.r_max, pool.proj.rs, pool.d_in, pool.policy, rb_g, nb_g, S_bound,
                       long_min, H);
  } else {
    hipLaunchKernelGGL((shrink_kernel<float>), grid, block, 0, stream,
                       (const float *)X, ldx, (const float *)pool.A, seg.token_indices,
                       seg.row_segment, seg.seg_off, seg.seg_slot, seg.seg_rank, seg.num_segments,
                       pool.r_max, pool.proj.rs, pool.d_in, pool.policy, rb_g, nb_g, S_bound,
                       long_min, H);
  }
  // 64 x 64 tiles when their work items fill the CUs; 32 x 32 tiles (one
  // MFMA wave each, four times the workgroups) when they would not, as for a
  // few long requests in a batch of a few thousand rows, where each of the
  // few 64 x 64 workgroups streams megabytes of X and A alone.  (On batches
  // that do fill the CUs the small tiles measured slower, 61 against about
  // 50 us at d_in 8192: too few bytes in flight per CU.)
  if (use_mfma) {
    const int tiles64 = ((n + 63) / 64) * ((pool.r_max + 63) / 64);
    if (tiles64 < kMfmaShrinkFillTiles)
      launch_shrink_mfma<32, 32>(X, ldx, seg, pool, H, stream);
    else
      launch_shrink_mfma<64, 64>(X, ldx, seg, pool, H, stream);
  }
  return hipGetLastError();
}

template <typename T, int RMAX>
void launch_expand_t(const float *H, const SegView &seg, const PoolView &pool, void *Y, int64_t ldy,
                     int rb, int nb, int S_bound, hipStream_t stream) {
  const int cols_per_block = kExpWaves * 16 * Elem<T>::kVec;
  const int gx = (pool.d_out + cols_per_block - 1) / cols_per_block;
  dim3 grid(gx, grid_items(nb + S_bound, gx));
  if (pool.dora)
    hipLaunchKernelGGL((expand_kernel<T, RMAX, true>), grid, dim3(kExpWaves * kWave), 0, stream,
                       H, (const T *)pool.Bt, pool.dora, seg.token_indices, seg.row_segment,
                       seg.seg_off, seg.seg_slot, seg.seg_rank, seg.seg_scale, seg.num_segments,
                       pool.r_max, pool.d_out, pool.policy, rb, nb, S_bound, (T *)Y, ldy,
                       pool.proj);
  else
    hipLaunchKernelGGL((expand_kernel<T, RMAX, false>), grid, dim3(kExpWaves * kWave), 0, stream,
                       H, (const T *)pool.Bt, nullptr, seg.token_indices, seg.row_segment,
                       seg.seg_off, seg.seg_slot, seg.seg_rank, seg.seg_scale, seg.num_segments,
                       pool.r_max, pool.d_out, pool.policy, rb, nb, S_bound, (T *)Y, ldy,
                       pool.proj);
}

template <typename T>
void launch_expand_r(const float *H, const SegView &seg, const PoolView &pool, void *Y, int64_t ldy,
                     int rb, int nb, int S_bound, hipStream_t stream) {
  switch (pool.proj.rs) {
    case 8: launch_expand_t<T, 8>(H, seg, pool, Y, ldy, rb, nb, S_bound, stream); break;
    case 16: launch_expand_t<T, 16>(H, seg, pool, Y, ldy, rb, nb, S_bound, stream); break;
    case 32: launch_expand_t<T, 32>(H, seg, pool, Y, ldy, rb, nb, S_bound, stream); break;
    default: launch_expand_t<T, 64>(H, seg, pool, Y, ldy, rb, nb, S_bound, stream); break;
  }
}

// The MFMA expand takes bf16 pools with the d_out-major B whose projections
// each start at a multiple of its 256-column blocks, for the batches where it
// beats the GEMV expand.  Its cost per work item hardly depends on the rank
// (a 64-row Y tile per item), while the GEMV expand's grows with the rank
// rows each item reads (d = 4096, uniform slots, us MFMA / GEMV: rank 16
// from 256 to 4096 rows 16 / 7 ... 46 / 40; rank 32 at 512 rows 19 / 15, at
// 1024 rows 20 / 24; rank 64 at 512 rows 25 / 35, at 2048 rows 42 / 90;
// rank 16 with segments of tens of rows at 2048 rows 12 / 35).  So: ranks of
// 32 and more once rank x rows reaches kXmMinRankRows, or segments of at
// least kXmMinSegRows rows on average (the segment bound taken as the count).
constexpr int kXmMinRankRows = 32768;
constexpr int kXmMinSegRows = 16;
inline bool expand_on_mfma(int n, int S_bound, const PoolView &pool) {
  if (pool.dtype != 1 || !pool.B || n == 0) return false;
  for (int q = 1; q < pool.proj.n_proj; ++q)
    if (pool.proj.col_off[q] % kXmCols) return false;
  const int rs = pool.proj.rs;
  if (rs >= 32 && (int64_t)rs * n >= kXmMinRankRows) return true;
  return n >= (int64_t)kXmMinSegRows * std::max(S_bound, 1);
}

hipError_t launch_expand(const float *H, const SegView &seg, const PoolView &pool, void *Y,
                         int64_t ldy, hipStream_t stream) {
  const int n = seg.n_rows;
  const int rb = row_block(n);
  const int nb = (n + rb - 1) / rb;
  const int S_bound = seg_bound(n, pool.n_slots, seg.max_segments);
  if (expand_on_mfma(n, S_bound, pool)) {
    // items of kRowBlk rows whatever the batch size
    // at most kXmItems items per workgroup (its metadata table)
    const int nbx = (n + kRowBlk - 1) / kRowBlk;
    const int gx = (pool.d_out + kXmCols - 1) / kXmCols;
    const int items = nbx + S_bound;
    const int gy = std::max(grid_items(items, gx), (items + kXmItems - 1) / kXmItems);
    const dim3 grid(gx, gy);
    if (pool.dora)
      hipLaunchKernelGGL(expand_mfma_kernel<true>, grid, dim3(4 * kWave), 0, stream, H,
                         (const bf16_t *)pool.B, pool.dora, seg.token_indices, seg.row_segment,
                         seg.seg_off, seg.seg_slot, seg.seg_rank, seg.seg_scale, seg.num_segments,
                         pool.r_max, pool.d_out, pool.policy, nbx, S_bound, (bf16_t *)Y, ldy,
                         pool.proj);
    else
      hipLaunchKernelGGL(expand_mfma_kernel<false>, grid, dim3(4 * kWave), 0, stream, H,
                         (const bf16_t *)pool.B, nullptr, seg.token_indices, seg.row_segment,
                         seg.seg_off, seg.seg_slot, seg.seg_rank, seg.seg_scale, seg.num_segments,
                         pool.r_max, pool.d_out, pool.policy, nbx, S_bound, (bf16_t *)Y, ldy,
                         pool.proj);
    return hipGetLastError();
  }
  if (pool.dtype == 1)
    launch_expand_r<bf16_t>(H, seg, pool, Y, ldy, rb, nb, S_bound, stream);
  else
    launch_expand_r<float>(H, seg, pool, Y, ldy, rb, nb, S_bound, stream);
  return hipGetLastError();
}

}  // namespace lora
