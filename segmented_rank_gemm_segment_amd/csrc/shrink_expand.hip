// Segmented shrink and expand of the multi-LoRA layer.
//
//   shrink:  H[i][k]  = sum_c X[i][c] A_a[k][c]          k < r_a
//   expand:  Y[i][j] += s_a sum_k H[i][k] B_a[j][k]      (Bt_a[k][j] in the pool)
//
// for every row i of a segment with slot a and rank r_a > 0 (adapter-batching
// page, Multi-LoRA Serving, section "Segmented Kernel 需要哪些 Metadata":
// H_a = X_a A_a^T and Delta Y_a = s_a H_a B_a^T scattered back to the
// original rows).
//
// Both kernels are bandwidth-bound segmented GEMV/skinny GEMMs.  Work items
// are (segment, block of up to kRowBlk rows of that segment); a fixed grid
// walks them with a stride so no host synchronisation is needed to size it.
// Every adapter row is read with 16-byte coalesced loads along d (A rows
// along d_in, Bt rows along d_out); the rank-r reduction of the shrink is a
// wavefront butterfly.  Each token row lives in exactly one segment, so Y is
// updated without atomics and the result is deterministic.
#include "lora_device.cuh"
#include "lora_kernels.h"

namespace lora {
namespace {

constexpr int kRowBlk = 64;   // rows of one segment per work item
constexpr int kSub = 8;       // rows processed together inside a work item

// Keep a loaded value alive (rank rows past r inside the processed width are
// read, as a padded kernel would, but contribute nothing).
__device__ __forceinline__ void keep(uint4 &v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}

// ----------------------------------------------------------------------------
// shrink: one wavefront per rank row k of a work item; lanes stride d_in with
// 16-byte vectors; blockIdx.x picks a group of waves-per-block rank rows.
// ----------------------------------------------------------------------------
template <typename T, int kWaves>
__global__ __launch_bounds__(kWaves * kWave) void shrink_kernel(
    const T *__restrict__ X, int64_t ldx, const T *__restrict__ A, const int32_t *token_indices,
    const int32_t *seg_off, const int32_t *seg_slot, const int32_t *seg_rank,
    const int32_t *num_segments, int r_max, int d_in, int policy, int blocks_per_seg,
    float *__restrict__ H) {
  constexpr int V = Elem<T>::kVec;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int k = blockIdx.x * kWaves + wave;
  const int S = *num_segments;
  const int items = S * blocks_per_seg;
  for (int item = blockIdx.y; item < items; item += gridDim.y) {
    const int s = item / blocks_per_seg;
    const int b = item - s * blocks_per_seg;
    const int r = seg_rank[s];
    const int R = rank_bucket(r, policy, r_max);
    if (k >= R) continue;
    const int p0 = seg_off[s] + b * kRowBlk;
    const int p1 = min(seg_off[s + 1], p0 + kRowBlk);
    if (p0 >= p1) continue;
    const int slot = seg_slot[s];
    const T *arow = A + ((int64_t)slot * r_max + k) * d_in;
    for (int q0 = p0; q0 < p1; q0 += kSub) {
      const int nq = min(kSub, p1 - q0);
      int rows[kSub];
#pragma unroll
      for (int q = 0; q < kSub; ++q) rows[q] = token_indices[q0 + min(q, nq - 1)];
      float acc[kSub];
#pragma unroll
      for (int q = 0; q < kSub; ++q) acc[q] = 0.f;
      for (int c = lane * V; c < d_in; c += kWave * V) {
        float av[V];
        Elem<T>::unpack(ldg16(arow + c), av);
#pragma unroll
        for (int q = 0; q < kSub; ++q) {
          if (q < nq) {
            float xv[V];
            Elem<T>::unpack(ldg16(X + (int64_t)rows[q] * ldx + c), xv);
#pragma unroll
            for (int e = 0; e < V; ++e) acc[q] = fmaf(av[e], xv[e], acc[q]);
          }
        }
      }
#pragma unroll
      for (int q = 0; q < kSub; ++q) {
        if (q < nq) {
          const float v = wave_sum(acc[q]);
          if (lane == 0 && k < r) H[(int64_t)rows[q] * r_max + k] = v;
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------
// expand: a thread owns V consecutive output columns; blockIdx.x picks the
// column chunk.  H rows of the current sub-block are staged in LDS.
// ----------------------------------------------------------------------------
template <typename T, int kThreads>
__global__ __launch_bounds__(kThreads) void expand_kernel(
    const float *__restrict__ H, const T *__restrict__ Bt, const int32_t *token_indices,
    const int32_t *seg_off, const int32_t *seg_slot, const int32_t *seg_rank,
    const float *seg_scale, const int32_t *num_segments, int r_max, int d_out, int policy,
    int blocks_per_seg, T *__restrict__ Y, int64_t ldy) {
  constexpr int V = Elem<T>::kVec;
  __shared__ float s_h[kSub][64];
  __shared__ int s_rows[kSub];
  const int col = (blockIdx.x * kThreads + threadIdx.x) * V;
  const bool active = col < d_out;
  const int S = *num_segments;
  const int items = S * blocks_per_seg;
  for (int item = blockIdx.y; item < items; item += gridDim.y) {
    const int s = item / blocks_per_seg;
    const int b = item - s * blocks_per_seg;
    const int r = seg_rank[s];
    const int R = rank_bucket(r, policy, r_max);
    if (R == 0) continue;
    const int p0 = seg_off[s] + b * kRowBlk;
    const int p1 = min(seg_off[s + 1], p0 + kRowBlk);
    if (p0 >= p1) continue;
    const float sc = seg_scale[s];
    const T *bt = Bt + (int64_t)seg_slot[s] * r_max * d_out + col;
    for (int q0 = p0; q0 < p1; q0 += kSub) {
      const int nq = min(kSub, p1 - q0);
      __syncthreads();
      if (threadIdx.x < kSub) s_rows[threadIdx.x] = token_indices[q0 + min((int)threadIdx.x, nq - 1)];
      __syncthreads();
      for (int t = threadIdx.x; t < kSub * R; t += kThreads) {
        const int q = t / R, kk = t - q * R;
        s_h[q][kk] = (q < nq && kk < r) ? H[(int64_t)s_rows[q] * r_max + kk] : 0.f;
      }
      __syncthreads();
      if (!active) continue;
      float acc[kSub][V];
#pragma unroll
      for (int q = 0; q < kSub; ++q)
#pragma unroll
        for (int e = 0; e < V; ++e) acc[q][e] = 0.f;
      for (int kk = 0; kk < R; ++kk) {
        uint4 raw = ldg16(bt + (int64_t)kk * d_out);
        keep(raw);
        float bv[V];
        Elem<T>::unpack(raw, bv);
        const bool live = kk < r;
#pragma unroll
        for (int e = 0; e < V; ++e) bv[e] = live ? bv[e] : 0.f;
#pragma unroll
        for (int q = 0; q < kSub; ++q) {
          const float h = s_h[q][kk];
#pragma unroll
          for (int e = 0; e < V; ++e) acc[q][e] = fmaf(h, bv[e], acc[q][e]);
        }
      }
#pragma unroll
      for (int q = 0; q < kSub; ++q) {
        if (q < nq) {
          T *y = Y + (int64_t)s_rows[q] * ldy + col;
          float yv[V];
          Elem<T>::unpack(ldg16(y), yv);
#pragma unroll
          for (int e = 0; e < V; ++e) yv[e] = fmaf(sc, acc[q][e], yv[e]);
          stg16(y, Elem<T>::pack(yv));
        }
      }
    }
  }
}

inline int seg_bound(int n_rows, int n_slots, int max_segments) {
  int b = n_rows < n_slots + 1 ? n_rows : n_slots + 1;
  return b < max_segments ? b : max_segments;
}

inline int grid_items(int bound_items) {
  const int cap = 4096;
  return bound_items < cap ? (bound_items > 0 ? bound_items : 1) : cap;
}

}  // namespace

hipError_t launch_shrink(const void *X, int64_t ldx, const SegView &seg, const PoolView &pool,
                         float *H, hipStream_t stream) {
  constexpr int kW = 4;
  const int n = seg.n_rows;
  const int bps = (n + kRowBlk - 1) / kRowBlk;
  const int S_bound = seg_bound(n, pool.n_slots, seg.max_segments);
  // Upper bound on real items: every segment has >= 1 row, so
  // sum_s ceil(n_s / kRowBlk) <= S + n / kRowBlk.
  const int real_bound = S_bound + n / kRowBlk;
  dim3 grid((pool.r_max + kW - 1) / kW, grid_items(real_bound));
  dim3 block(kW * kWave);
  if (pool.dtype == 1) {
    hipLaunchKernelGGL((shrink_kernel<bf16_t, kW>), grid, block, 0, stream,
                       (const bf16_t *)X, ldx, (const bf16_t *)pool.A, seg.token_indices,
                       seg.seg_off, seg.seg_slot, seg.seg_rank, seg.num_segments, pool.r_max,
                       pool.d_in, pool.policy, bps, H);
  } else {
    hipLaunchKernelGGL((shrink_kernel<float, kW>), grid, block, 0, stream, (const float *)X,
                       ldx, (const float *)pool.A, seg.token_indices, seg.seg_off, seg.seg_slot,
                       seg.seg_rank, seg.num_segments, pool.r_max, pool.d_in, pool.policy, bps,
                       H);
  }
  return hipGetLastError();
}

hipError_t launch_expand(const float *H, const SegView &seg, const PoolView &pool, void *Y,
                         int64_t ldy, hipStream_t stream) {
  constexpr int kT = 64;
  const int n = seg.n_rows;
  const int bps = (n + kRowBlk - 1) / kRowBlk;
  const int S_bound = seg_bound(n, pool.n_slots, seg.max_segments);
  const int real_bound = S_bound + n / kRowBlk;
  dim3 block(kT);
  if (pool.dtype == 1) {
    const int cols_per_block = kT * Elem<bf16_t>::kVec;
    dim3 grid((pool.d_out + cols_per_block - 1) / cols_per_block, grid_items(real_bound));
    hipLaunchKernelGGL((expand_kernel<bf16_t, kT>), grid, block, 0, stream, H,
                       (const bf16_t *)pool.Bt, seg.token_indices, seg.seg_off, seg.seg_slot,
                       seg.seg_rank, seg.seg_scale, seg.num_segments, pool.r_max, pool.d_out,
                       pool.policy, bps, (bf16_t *)Y, ldy);
  } else {
    const int cols_per_block = kT * Elem<float>::kVec;
    dim3 grid((pool.d_out + cols_per_block - 1) / cols_per_block, grid_items(real_bound));
    hipLaunchKernelGGL((expand_kernel<float, kT>), grid, block, 0, stream, H,
                       (const float *)pool.Bt, seg.token_indices, seg.seg_off, seg.seg_slot,
                       seg.seg_rank, seg.seg_scale, seg.num_segments, pool.r_max, pool.d_out,
                       pool.policy, bps, (float *)Y, ldy);
  }
  return hipGetLastError();
}

}  // namespace lora
