// Pool set-up: packing one adapter into a slot, the slots' scales, and the
// d_out-major copy of B.
//
// The multi-tenant serving article (LoRA/QLoRA 多租户GPU推理服务化实战,
// section 1.1 "Adapter的统一尺寸对齐") preallocates one buffer of uniform
// slots and packs each adapter's weights into the slot found by its offset;
// its section 1.2 keeps the alpha / r scaling inside the kernel library.  The
// adapter-batching page (section "动态加载是一个安全边界") asks for bounded
// ranks and sizes and for a failed load to leave the old contents in place;
// its replacement procedure publishes the new slot only once the new weights
// are complete.  Its section "Adapter 不是一块连续 Weight" gives every target
// projection its own A and B, laid out by the loader.
//
// Packing writes the weights first, one kernel per projection of the pool:
// projection q's A rows into rank rows [q rs, q rs + rank) (zeros up to
// (q + 1) rs), its B^T into rank rows [0, rank) of Bt over its own output
// columns only (zeros up to rs; the slot's rs rank rows of Bt hold every
// column's own projection, so the other projections' columns are left as
// they are), B likewise in the d_out-major copy when the pool has one, and
// ones in the slot's DoRA column
// factors when the pool has them (a fresh adapter is plain LoRA until its
// factors are prepared).  A one-thread kernel on the same stream then writes
// the slot's rank and scale alpha / rank, so work queued after the call sees
// either nothing of the new adapter (before) or all of it.  Every argument is
// checked on the host before any kernel is queued.
#include "lora_device.cuh"
#include "lora_kernels.h"

namespace lora {
namespace {

constexpr int kThreads = 256;

// One projection q of one slot.  Work items, in order: A rows of the block
// (16-byte vectors), Bt rows over the projection's columns (vectors of V
// columns), B's rank entries of those columns (one element each), the DoRA
// factors (float4).
template <typename T>
__global__ __launch_bounds__(kThreads) void pack_proj_kernel(
    T *__restrict__ A, T *__restrict__ Bt, T *__restrict__ Bn, float *__restrict__ D,
    int rs, int q, int c_lo, int c_hi, int d_in, int d_out, int rank, const T *__restrict__ A_src,
    int64_t lda, const T *__restrict__ B_src, int64_t ldb, int b_rank_rows, int64_t nA,
    int64_t nBt, int64_t nB, int64_t nD) {
  constexpr int V = Elem<T>::kVec;
  const int64_t v = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  // B value of output column j (in the projection) and rank k < rank
  auto bval = [&](int j, int k) -> T {
    const int64_t jj = j - c_lo;
    return b_rank_rows ? B_src[(int64_t)k * ldb + jj] : B_src[jj * ldb + k];
  };
  if (v < nA) {
    const int k = (int)(v / (d_in / V));                  // rank row inside the block
    const int c = (int)(v - (int64_t)k * (d_in / V)) * V;
    uint4 out = make_uint4(0u, 0u, 0u, 0u);
    if (k < rank) out = ldg16(A_src + (int64_t)k * lda + c);   // lda % 8 == 0: aligned
    stg16(A + ((int64_t)q * rs + k) * d_in + c, out);
    return;
  }
  if (v < nA + nBt) {
    // column offsets of projections are multiples of 8 >= V: the V columns
    // all lie inside the projection
    const int64_t w = v - nA;
    const int cv = (c_hi - c_lo) / V;                      // vectors per rank row
    const int k = (int)(w / cv);
    const int j = c_lo + (int)(w - (int64_t)k * cv) * V;
    T vals[V];
#pragma unroll
    for (int e = 0; e < V; ++e) vals[e] = k < rank ? bval(j + e, k) : T(0);
    uint4 out;
    __builtin_memcpy(&out, vals, sizeof(out));
    stg16(Bt + (int64_t)k * d_out + j, out);
    return;
  }
  if (v < nA + nBt + nB) {
    const int64_t w = v - nA - nBt;
    const int j = c_lo + (int)(w / rs);
    const int k = (int)(w - (int64_t)(j - c_lo) * rs);
    Bn[(int64_t)j * rs + k] = k < rank ? bval(j, k) : T(0);
    return;
  }
  if (v < nA + nBt + nB + nD) {
    const int64_t w = v - nA - nBt - nB;
    *reinterpret_cast<float4 *>(D + w * 4) = make_float4(1.f, 1.f, 1.f, 1.f);
  }
}

// Publication of the slot: its rank and scale alpha / rank (rounded once
// from the double quotient), after the weights.
__global__ void publish_slot_kernel(int32_t *slot_rank, float *slot_scale, int slot, int rank,
                                    double alpha) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    slot_rank[slot] = rank;
    slot_scale[slot] = rank > 0 ? (float)(alpha / (double)rank) : 0.0f;
  }
}

template <typename T>
hipError_t launch_pack_t(const PoolView &pool, int32_t *slot_rank, float *slot_scale, int slot,
                         int rank, double alpha, const void *const *A_src, const int64_t *lda,
                         const void *const *B_src, const int64_t *ldb, int b_rank_rows,
                         hipStream_t stream) {
  constexpr int V = Elem<T>::kVec;
  const int64_t r_max = pool.r_max, d_in = pool.d_in, d_out = pool.d_out;
  const int rs = pool.proj.rs;
  T *A = (T *)pool.A + (int64_t)slot * r_max * d_in;
  T *Bt = (T *)pool.Bt + (int64_t)slot * rs * d_out;
  T *Bn = pool.B ? (T *)pool.B + (int64_t)slot * d_out * rs : nullptr;
  float *D = pool.dora ? const_cast<float *>(pool.dora) + (int64_t)slot * d_out : nullptr;
  for (int q = 0; q < pool.proj.n_proj; ++q) {
    const int64_t cols = pool.proj.col_off[q + 1] - pool.proj.col_off[q];
    const int64_t nA = (int64_t)rs * d_in / V, nBt = (int64_t)rs * cols / V;
    const int64_t nB = Bn ? cols * rs : 0;
    const int64_t nD = (D && q == 0) ? d_out / 4 : 0;
    const int64_t total = nA + nBt + nB + nD;
    const int blocks = (int)((total + kThreads - 1) / kThreads);
    // rank 0 reads no source: the pool's own arrays stand in (never read)
    const T *as = rank > 0 ? (const T *)A_src[q] : A;
    const T *bs = rank > 0 ? (const T *)B_src[q] : Bt;
    hipLaunchKernelGGL((pack_proj_kernel<T>), dim3(blocks), dim3(kThreads), 0, stream, A, Bt,
                       Bn, D, rs, q, pool.proj.col_off[q], pool.proj.col_off[q + 1],
                       pool.d_in, pool.d_out, rank, as, rank > 0 ? lda[q] : d_in, bs,
                       rank > 0 ? ldb[q] : 1, b_rank_rows, nA, nBt, nB, nD);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(publish_slot_kernel, dim3(1), dim3(64), 0, stream, slot_rank, slot_scale,
                     slot, rank, alpha);
  return hipGetLastError();
}

// slot_scale[a] = alpha[a] / slot_rank[a] (double quotient rounded once to
// float), 0 for a slot of rank <= 0.
__global__ __launch_bounds__(kThreads) void set_scales_kernel(const int32_t *slot_rank,
                                                              const double *alpha,
                                                              float *slot_scale, int n_slots) {
  const int a = blockIdx.x * kThreads + threadIdx.x;
  if (a < n_slots) {
    const int r = slot_rank[a];
    slot_scale[a] = r > 0 ? (float)(alpha[a] / (double)r) : 0.0f;
  }
}

// B[a][j][k] = Bt[a][k][j] over the rs rank rows of every slot: one thread
// per 16-byte vector of B (V rank values of one output column), gathered
// from V rank rows of Bt.
template <typename T>
__global__ __launch_bounds__(kThreads) void write_b_kernel(const T *__restrict__ Bt,
                                                           T *__restrict__ Bn, int n_slots,
                                                           int rs, int d_out) {
  constexpr int V = Elem<T>::kVec;
  const int64_t v = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t per_slot = (int64_t)d_out * (rs / V);
  if (v >= per_slot * n_slots) return;
  const int a = (int)(v / per_slot);
  const int64_t w = v - (int64_t)a * per_slot;
  const int j = (int)(w / (rs / V));
  const int k0 = (int)(w - (int64_t)j * (rs / V)) * V;
  const T *src = Bt + ((int64_t)a * rs + k0) * d_out + j;
  T vals[V];
#pragma unroll
  for (int e = 0; e < V; ++e) vals[e] = src[(int64_t)e * d_out];
  uint4 out;
  __builtin_memcpy(&out, vals, sizeof(out));
  stg16(Bn + ((int64_t)a * d_out + j) * rs + k0, out);
}

}  // namespace

hipError_t launch_pack_slot(const PoolView &pool, int32_t *slot_rank, float *slot_scale, int slot,
                            int rank, double alpha, const void *const *A_src, const int64_t *lda,
                            const void *const *B_src, const int64_t *ldb, int b_rank_rows,
                            hipStream_t stream) {
  if (pool.dtype == 1)
    return launch_pack_t<bf16_t>(pool, slot_rank, slot_scale, slot, rank, alpha, A_src, lda,
                                 B_src, ldb, b_rank_rows, stream);
  return launch_pack_t<float>(pool, slot_rank, slot_scale, slot, rank, alpha, A_src, lda, B_src,
                              ldb, b_rank_rows, stream);
}

hipError_t launch_set_scales(const int32_t *slot_rank, const double *alpha, float *slot_scale,
                             int n_slots, hipStream_t stream) {
  hipLaunchKernelGGL(set_scales_kernel, dim3((n_slots + kThreads - 1) / kThreads),
                     dim3(kThreads), 0, stream, slot_rank, alpha, slot_scale, n_slots);
  return hipGetLastError();
}

hipError_t launch_write_b(const PoolView &pool, hipStream_t stream) {
  const int V = pool.dtype == 1 ? Elem<bf16_t>::kVec : Elem<float>::kVec;
  const int64_t total = (int64_t)pool.n_slots * pool.d_out * (pool.proj.rs / V);
  const int blocks = (int)((total + kThreads - 1) / kThreads);
  if (pool.dtype == 1)
    hipLaunchKernelGGL(write_b_kernel<bf16_t>, dim3(blocks), dim3(kThreads), 0, stream,
                       (const bf16_t *)pool.Bt, (bf16_t *)pool.B, pool.n_slots, pool.proj.rs,
                       pool.d_out);
  else
    hipLaunchKernelGGL(write_b_kernel<float>, dim3(blocks), dim3(kThreads), 0, stream,
                       (const float *)pool.Bt, (float *)pool.B, pool.n_slots, pool.proj.rs,
                       pool.d_out);
  return hipGetLastError();
}

}  // namespace lora
