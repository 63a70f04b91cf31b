// DoRA column factors of one pool slot.
//
// The ybb.press multi-LoRA serving article (section 9.2, DoRA) splits the
// adapted weight into a magnitude m and a direction W0 + BA divided by its
// norm; at inference that costs one extra normalisation, applied in the
// epilogue.  With the direction of slot a taken as the weight the layer
// applies, V_a = W0 + s_a B_a A_a, and the norm taken per output feature
// (one row of the nn.Linear weight), the layer's output for a row on slot a
// is g_a[j] times its plain LoRA output, with
//
//   g_a[j] = m_a[j] / ||V_a[j, :]||_2        (0 when the norm is 0).
//
// This kernel computes g_a once per adapter (when it is loaded), so the hot
// path only multiplies.  A workgroup owns kRows output features: it stages
// their rank values B_a[j][0:r] in LDS, then walks the input dimension in
// 16-byte vectors, forming V_a[j][c] = W0[j][c] + s_a sum_k B_a[j][k] A_a[k][c]
// in fp32 and summing squares in fp32, first per thread and then as a tree.
// Rank and scale are read on the device from the slot's published values,
// so the call follows a pack on the same stream without a host round trip.
#include "lora_device.cuh"
#include "lora_kernels.h"

namespace lora {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 8;        // output features per workgroup

template <typename T>
__global__ __launch_bounds__(kThreads) void dora_prepare_kernel(
    const T *__restrict__ W, int64_t ldw, const T *__restrict__ A, const T *__restrict__ Bt,
    const int32_t *__restrict__ slot_rank, const float *__restrict__ slot_scale, int slot,
    int r_max, int d_in, int d_out, const float *__restrict__ magnitude, float *__restrict__ g,
    ProjView proj) {
  constexpr int V = Elem<T>::kVec;
  __shared__ float s_b[kRows][64];
  __shared__ float s_red[kThreads / kWave][kRows];
  const int tid = threadIdx.x;
  const int j0 = blockIdx.x * kRows;
  int r = slot_rank[slot];
  r = (r < 0 || r > proj.rs) ? 0 : r;
  const float sc = r > 0 ? slot_scale[slot] : 0.f;
  // the workgroup's output features belong to one projection (offsets are
  // multiples of 8): its A rows start at qoff in the slot; the slot's rs
  // rank rows of Bt hold every column's own projection
  const int qoff = proj_of(proj, j0) * proj.rs;
  const T *a_slot = A + ((int64_t)slot * r_max + qoff) * d_in;
  const T *bt_slot = Bt + (int64_t)slot * proj.rs * d_out;
  // B_a[j0 + jj][k] for k < r (Bt row k is column k of B_a)
  for (int it = tid; it < kRows * 64; it += kThreads) {
    const int jj = it / 64, k = it - (it / 64) * 64;
    s_b[jj][k] = k < r ? Elem<T>::load1(bt_slot + (int64_t)k * d_out + j0 + jj) : 0.f;
  }
  __syncthreads();
  float sq[kRows];
#pragma unroll
  for (int jj = 0; jj < kRows; ++jj) sq[jj] = 0.f;
  for (int cv = tid; cv < d_in / V; cv += kThreads) {
    const int c = cv * V;
    float d[kRows][V];
#pragma unroll
    for (int jj = 0; jj < kRows; ++jj)
#pragma unroll
      for (int e = 0; e < V; ++e) d[jj][e] = 0.f;
    for (int k = 0; k < r; ++k) {
      float av[V];
      Elem<T>::unpack(ldg16(a_slot + (int64_t)k * d_in + c), av);
#pragma unroll
      for (int jj = 0; jj < kRows; ++jj) {
        const float b = s_b[jj][k];
#pragma unroll
        for (int e = 0; e < V; ++e) d[jj][e] = fmaf(b, av[e], d[jj][e]);
      }
    }
#pragma unroll
    for (int jj = 0; jj < kRows; ++jj) {
      float wv[V];
      Elem<T>::unpack(ldg16(W + (int64_t)(j0 + jj) * ldw + c), wv);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float v = fmaf(sc, d[jj][e], wv[e]);
        sq[jj] = fmaf(v, v, sq[jj]);
      }
    }
  }
  const int wave = tid / kWave, l = tid & (kWave - 1);
#pragma unroll
  for (int jj = 0; jj < kRows; ++jj) {
    const float t = wave_sum(sq[jj]);
    if (l == 0) s_red[wave][jj] = t;
  }
  __syncthreads();
  if (tid < kRows) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kThreads / kWave; ++w) t += s_red[w][tid];
    const int j = j0 + tid;
    const float m = magnitude ? magnitude[j] : 1.f;
    float out = 1.f;
    if (magnitude) out = t > 0.f ? m / sqrtf(t) : 0.f;
    g[(int64_t)slot * d_out + j] = out;
  }
}

}  // namespace

hipError_t launch_dora_prepare(const PoolView &pool, const int32_t *slot_rank,
                               const float *slot_scale, int slot, const void *W, int64_t ldw,
                               const float *magnitude, hipStream_t stream) {
  const dim3 grid(pool.d_out / kRows);    // d_out is a multiple of 8
  float *g = const_cast<float *>(pool.dora);
  if (pool.dtype == 1)
    hipLaunchKernelGGL(dora_prepare_kernel<bf16_t>, grid, dim3(kThreads), 0, stream,
                       (const bf16_t *)W, ldw, (const bf16_t *)pool.A, (const bf16_t *)pool.Bt,
                       slot_rank, slot_scale, slot, pool.r_max, pool.d_in, pool.d_out, magnitude,
                       g, pool.proj);
  else
    hipLaunchKernelGGL(dora_prepare_kernel<float>, grid, dim3(kThreads), 0, stream,
                       (const float *)W, ldw, (const float *)pool.A, (const float *)pool.Bt,
                       slot_rank, slot_scale, slot, pool.r_max, pool.d_in, pool.d_out, magnitude,
                       g, pool.proj);
  return hipGetLastError();
}

}  // namespace lora
