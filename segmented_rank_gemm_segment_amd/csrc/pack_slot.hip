// Packing one adapter into a slot of the fixed-slot pool.
//
// The multi-tenant serving article (LoRA/QLoRA 多租户GPU推理服务化实战,
// section 1.1 "Adapter的统一尺寸对齐") preallocates one buffer of uniform
// slots and packs each adapter's weights into the slot found by its offset.
// The adapter-batching page (section "动态加载是一个安全边界") asks for bounded
// ranks and sizes and for a failed load to leave the old contents in place;
// its replacement procedure publishes the new slot only once the new
// weights are complete.
//
// Here the weights are written first, by one kernel: A rows [0, rank) and
// zeros up to r_max, Bt = B^T rows likewise, the d_out-major copy of B when
// the pool has one, and ones in the slot's DoRA column factors when the pool
// has them (a fresh adapter is plain LoRA until its factors are prepared).  A second, one-thread kernel on the same stream then
// writes the slot's rank and scale, so work queued after the call sees
// either nothing of the new adapter (before) or all of it.  Every argument is
// checked on the host before either kernel is queued.
#include "lora_device.cuh"
#include "lora_kernels.h"

namespace lora {
namespace {

constexpr int kThreads = 256;

// Output vectors of V elements: region A [r_max][d_in], then Bt
// [r_max][d_out], then B [d_out][r_max] (when present), then the DoRA
// factors [d_out] in float4 vectors (when present).
template <typename T>
__global__ __launch_bounds__(kThreads) void pack_weights_kernel(
    T *__restrict__ A, T *__restrict__ Bt, T *__restrict__ Bn, float *__restrict__ D, int r_max,
    int d_in, int d_out, int rank, const T *__restrict__ A_src, int64_t lda,
    const T *__restrict__ B_src, int64_t ldb, int64_t nA, int64_t nBt, int64_t nB, int64_t nD) {
  constexpr int V = Elem<T>::kVec;
  const int64_t v = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (v < nA) {
    const int k = (int)(v / (d_in / V));
    const int c = (int)(v - (int64_t)k * (d_in / V)) * V;
    uint4 out = make_uint4(0u, 0u, 0u, 0u);
    if (k < rank) out = ldg16(A_src + (int64_t)k * lda + c);   // lda % 8 == 0: aligned
    stg16(A + (int64_t)k * d_in + c, out);
    return;
  }
  if (v < nA + nBt) {
    const int64_t w = v - nA;
    const int k = (int)(w / (d_out / V));
    const int j = (int)(w - (int64_t)k * (d_out / V)) * V;
    T vals[V];
#pragma unroll
    for (int e = 0; e < V; ++e) vals[e] = k < rank ? B_src[(int64_t)(j + e) * ldb + k] : T(0);
    uint4 out;
    __builtin_memcpy(&out, vals, sizeof(out));
    stg16(Bt + (int64_t)k * d_out + j, out);
    return;
  }
  if (v < nA + nBt + nB) {
    const int64_t w = v - nA - nBt;
    const int j = (int)(w / (r_max / V));
    const int k0 = (int)(w - (int64_t)j * (r_max / V)) * V;
    T vals[V];
#pragma unroll
    for (int e = 0; e < V; ++e)
      vals[e] = k0 + e < rank ? B_src[(int64_t)j * ldb + k0 + e] : T(0);
    uint4 out;
    __builtin_memcpy(&out, vals, sizeof(out));
    stg16(Bn + (int64_t)j * r_max + k0, out);
    return;
  }
  if (v < nA + nBt + nB + nD) {
    const int64_t w = v - nA - nBt - nB;
    *reinterpret_cast<float4 *>(D + w * 4) = make_float4(1.f, 1.f, 1.f, 1.f);
  }
}

// Publication of the slot: its rank and scale, after the weights.
__global__ void publish_slot_kernel(int32_t *slot_rank, float *slot_scale, int slot, int rank,
                                    float scale) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    slot_rank[slot] = rank;
    slot_scale[slot] = rank > 0 ? scale : 0.0f;
  }
}

template <typename T>
hipError_t launch_pack_t(const PoolView &pool, int32_t *slot_rank, float *slot_scale, int slot,
                         int rank, float scale, const void *A_src, int64_t lda,
                         const void *B_src, int64_t ldb, hipStream_t stream) {
  constexpr int V = Elem<T>::kVec;
  const int64_t r_max = pool.r_max, d_in = pool.d_in, d_out = pool.d_out;
  T *A = (T *)pool.A + (int64_t)slot * r_max * d_in;
  T *Bt = (T *)pool.Bt + (int64_t)slot * r_max * d_out;
  T *Bn = pool.B ? (T *)pool.B + (int64_t)slot * d_out * r_max : nullptr;
  float *D = pool.dora ? const_cast<float *>(pool.dora) + (int64_t)slot * d_out : nullptr;
  const int64_t nA = r_max * d_in / V, nBt = r_max * d_out / V, nB = Bn ? d_out * r_max / V : 0;
  const int64_t nD = D ? d_out / 4 : 0;
  const int64_t total = nA + nBt + nB + nD;
  const int blocks = (int)((total + kThreads - 1) / kThreads);
  hipLaunchKernelGGL((pack_weights_kernel<T>), dim3(blocks), dim3(kThreads), 0, stream, A, Bt,
                     Bn, D, pool.r_max, pool.d_in, pool.d_out, rank, (const T *)A_src, lda,
                     (const T *)B_src, ldb, nA, nBt, nB, nD);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(publish_slot_kernel, dim3(1), dim3(64), 0, stream, slot_rank, slot_scale,
                     slot, rank, scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pack_slot(const PoolView &pool, int32_t *slot_rank, float *slot_scale, int slot,
                            int rank, float scale, const void *A_src, int64_t lda,
                            const void *B_src, int64_t ldb, hipStream_t stream) {
  if (pool.dtype == 1)
    return launch_pack_t<bf16_t>(pool, slot_rank, slot_scale, slot, rank, scale, A_src, lda,
                                 B_src, ldb, stream);
  return launch_pack_t<float>(pool, slot_rank, slot_scale, slot, rank, scale, A_src, lda, B_src,
                              ldb, stream);
}

}  // namespace lora
