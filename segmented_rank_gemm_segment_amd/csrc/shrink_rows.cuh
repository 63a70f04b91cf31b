// Shrink of a short run of token rows against a block of rank rows of one
// adapter slot, H[row][k] = sum_c X[row][c] A_slot[k][c] (adapter-batching
// page, Multi-LoRA Serving, section "Segmented Kernel 需要哪些 Metadata":
// H_a = X_a A_a^T).  Shared by the metadata-driven shrink and the combined
// build + shrink launch, so both give the same bits.
//
// A workgroup of kShW waves takes kShRB rank rows and walks the rows in
// groups of kShRQ.  d_in is cut into chunks of one 16-byte vector per lane;
// chunk c belongs to wave c mod kShW, which loads the group's token rows and
// the block's adapter rows for the chunk (every load issued before any use)
// and keeps kShRQ x kShRB partial dot products per lane.  Each X element of
// a group is read once per rank block and each adapter element once per
// row group.  The partials are reduced over the lanes by a halving
// butterfly (after it lane l holds pair l mod 32), then over the waves
// through LDS in wave order.
#pragma once

#include "lora_device.cuh"

namespace lora {

constexpr int kRowBlk = 64;    // rows of one segment per work item (large batches)
constexpr int kRowBlkSmall = 16;  // ... in batches below kLargeBatch rows
constexpr int kLargeBatch = 2048;
constexpr int kShW = 4;        // waves per workgroup
constexpr int kShRQ = 4;       // token rows per group
constexpr int kShRB = 8;       // rank rows per workgroup
constexpr int kShCU = 2;       // chunks per wave in flight
constexpr int kShNP = kShRQ * kShRB;
static_assert(kShNP <= 32 && (kShNP & (kShNP - 1)) == 0, "pairs per lane");

// One halving step of the butterfly: the lanes with bit H set keep the
// upper half of the H * 2 live values, the others the lower half, and each
// adds its partner's copy of the half it keeps.
template <int H, int N>
__device__ __forceinline__ void butterfly_step(float (&v)[N], int lane) {
  const bool up = (lane & H) != 0;
#pragma unroll
  for (int i = 0; i < H; ++i) {
    const float keep = up ? v[i + H] : v[i];
    const float send = up ? v[i] : v[i + H];
    v[i] = keep + __shfl_xor(send, H);
  }
  if constexpr (H > 1) butterfly_step<H / 2>(v, lane);
}

// Sum of v[0..N) over the 64 lanes, one pair per lane: on return v[0] of
// lane l holds the total of pair l % N (N a power of two, 2 <= N <= 32).
template <int N>
__device__ __forceinline__ void butterfly_reduce(float (&v)[N], int lane) {
  butterfly_step<N / 2>(v, lane);
  // lanes l, l ^ N, l ^ 2N, ... hold partial totals of the same pair
#pragma unroll
  for (int h = N; h < kWave; h *= 2) v[0] += __shfl_xor(v[0], h);
}

// Rows rows[p0 .. p1) (original row indices; global or LDS memory) against
// rank rows k0 .. k0 + nk of `slot` (nk <= kShRB rows inside the processed
// width, so inside the slot); k0 is kl0 rows into its projection's rank
// block, and H entries of rank rows at or past the rank r in that block are
// not written.  Called by every thread of a kShW-wave workgroup (it passes
// barriers).
template <typename T>
__device__ __forceinline__ void shrink_rows(const T *__restrict__ X, int64_t ldx,
                                            const T *__restrict__ A, int slot, int k0, int kl0,
                                            int nk, int r, int r_max, int d_in,
                                            const int32_t *rows,
                                            int p0, int p1, float *__restrict__ H,
                                            float (*s_part)[kShNP]) {
  constexpr int V = Elem<T>::kVec;
  constexpr int CH = kWave * V;                 // elements per chunk
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const T *a0 = A + ((int64_t)slot * r_max + k0) * d_in;
  for (int q0 = p0; q0 < p1; q0 += kShRQ) {
    const int nq = min(kShRQ, p1 - q0);
    // row indices of the group in one vector load (lane q: row q; lanes past
    // the group repeat its last row), issued ahead of the adapter rows so
    // that waiting for them does not wait for those
    const int tv = rows[q0 + min(lane, nq - 1)];
    __builtin_amdgcn_sched_barrier(0);
    float acc[kShNP];
#pragma unroll
    for (int i = 0; i < kShNP; ++i) acc[i] = 0.f;
    for (int cb = wave * CH; cb < d_in; cb += kShW * CH * kShCU) {
      // Every load is unconditional: addresses past d_in are clamped into
      // the row (d_in % 8 == 0), rank rows past the block's width re-read
      // its last row and rows past the group re-read its last row; all of
      // those values are dropped where they are used.
      uint4 av[kShCU][kShRB], xv[kShCU][kShRQ];
#pragma unroll
      for (int u = 0; u < kShCU; ++u) {
        const int cc = min(cb + u * kShW * CH + lane * V, d_in - V);
#pragma unroll
        for (int kk = 0; kk < kShRB; ++kk)
          av[u][kk] = ldg16(a0 + (int64_t)min(kk, nk - 1) * d_in + cc);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < kShCU; ++u) {
        const int cc = min(cb + u * kShW * CH + lane * V, d_in - V);
#pragma unroll
        for (int q = 0; q < kShRQ; ++q)
          xv[u][q] = ldg16(X + (int64_t)__builtin_amdgcn_readlane(tv, q) * ldx + cc);
      }
      __builtin_amdgcn_sched_barrier(0);   // all loads issued before any use
      // each token row of the group unpacked once per chunk, each adapter
      // row once; every (row, rank row) sum still runs over the chunks and
      // their elements in order
#pragma unroll
      for (int u = 0; u < kShCU; ++u) {
        const bool ok = cb + u * kShW * CH + lane * V < d_in;
        float xf[kShRQ][V];
#pragma unroll
        for (int q = 0; q < kShRQ; ++q) {
          Elem<T>::unpack(xv[u][q], xf[q]);
#pragma unroll
          for (int e = 0; e < V; ++e) xf[q][e] = (ok && q < nq) ? xf[q][e] : 0.f;
        }
#pragma unroll
        for (int kk = 0; kk < kShRB; ++kk) {
          float af[V];
          Elem<T>::unpack(av[u][kk], af);
#pragma unroll
          for (int q = 0; q < kShRQ; ++q)
#pragma unroll
            for (int e = 0; e < V; ++e)
              acc[q * kShRB + kk] = fmaf(af[e], xf[q][e], acc[q * kShRB + kk]);
        }
      }
    }
    butterfly_reduce<kShNP>(acc, lane);
    if (lane < kShNP) s_part[wave][lane] = acc[0];
    __syncthreads();
    if (threadIdx.x < kShNP) {
      const int q = threadIdx.x / kShRB, kk = threadIdx.x % kShRB;
      float t = s_part[0][threadIdx.x];
#pragma unroll
      for (int w = 1; w < kShW; ++w) t += s_part[w][threadIdx.x];
      const int row = __shfl(tv, q);
      if (q < nq && kl0 + kk < r) H[(int64_t)row * r_max + k0 + kk] = t;
    }
    __syncthreads();   // s_part is rewritten by the next group
  }
}

}  // namespace lora
