// Base product Y = X W^T of the multi-LoRA layer, optionally with the LoRA
// expand fused into the epilogue:
//
//   Y[i] = X[i] W^T + s_a H[i][0:r_a] B_a^T          (fp32 accumulate, one rounding)
//
// The base GEMM is shared by all rows of the batch (adapter-batching page,
// Multi-LoRA Serving, section "一个混合 Batch 的数学形式"); adding the second
// low-rank product into the base output follows the epilogue-fusion
// structure of the ybb.press multi-LoRA serving article, section 5.3.
//
// bf16: MFMA v_mfma_f32_32x32x16_bf16 (gfx950), block tiles staged through
// LDS with double buffering, one barrier per K step.  Both operands are
// K-contiguous (X rows and nn.Linear W rows), so global loads are 16-byte
// vectors along K and LDS rows are padded by 16 bytes, which keeps the
// 16-byte fragment reads of 8 consecutive rows on distinct banks.
//
// Fused epilogue: the rows of an output tile may belong to several segments.
// For each distinct LoRA segment u in the tile, Bt_u[0:R][tile columns] is
// staged in LDS (K-contiguous per column), the scaled H rows of u form the
// A operand (split into a bf16 high part and a bf16 remainder, so H keeps
// about 16 significant bits), and the MFMA result is added only to rows of
// u.  Every row gets exactly its own segment's increment.
#include "lora_device.cuh"
#include "lora_kernels.h"

namespace lora {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct GemmArgs {
  const bf16_t *X;
  int64_t ldx;
  const bf16_t *W;
  int64_t ldw;
  bf16_t *Y;
  int64_t ldy;
  int M, K, N;
  // fused LoRA
  const float *H;
  const bf16_t *Bt;
  const int32_t *row_segment, *seg_slot, *seg_rank;
  const float *seg_scale;
  int r_max, policy;
};

constexpr int kBK = 64;
constexpr int kLdsStride = kBK + 8;  // elements; +16 bytes per row

template <int BM, int BN>
constexpr int lds_bytes_main() { return 2 * (BM + BN) * kLdsStride * 2; }
template <int BM, int BN>
constexpr int lds_bytes_lora() { return 2 * BM * 4 + 16 + BN * (64 + 8) * 2; }
template <int BM, int BN>
constexpr int lds_bytes() {
  return lds_bytes_main<BM, BN>() > lds_bytes_lora<BM, BN>() ? lds_bytes_main<BM, BN>()
                                                             : lds_bytes_lora<BM, BN>();
}

__device__ __forceinline__ mfma_bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(mfma_bf16x8, v); }

// Row of element v (0..15) of a 32x32 MFMA accumulator held by lane l
// (column is l % 32).
__device__ __forceinline__ int acc_row(int v, int l) { return (v >> 2) * 8 + (l >> 5) * 4 + (v & 3); }

template <int BM, int BN, int WM, int WN, bool LORA>
__global__ __launch_bounds__(WM *WN *kWave) void gemm_bf16_kernel(GemmArgs g) {
  constexpr int T = WM * WN * kWave;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int AV = BM * (kBK / 8) / T;  // 16-byte vectors per thread per stage
  constexpr int BV = BN * (kBK / 8) / T;
  static_assert(FM >= 1 && FN >= 1 && AV >= 1 && BV >= 1, "tile");
  static_assert(BM * (kBK / 8) % T == 0 && BN * (kBK / 8) % T == 0, "tile");

  __shared__ __align__(16) unsigned char smem[lds_bytes<BM, BN>()];
  bf16_t *sA = reinterpret_cast<bf16_t *>(smem);
  bf16_t *sB = sA + 2 * BM * kLdsStride;

  const int tid = threadIdx.x;
  const int l = tid & (kWave - 1);
  const int wid = tid / kWave;
  const int wm = wid / WN, wn = wid % WN;
  const int m0 = blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;
  const int M = g.M, N = g.N, K = g.K;

  u32x4 ra[AV], rb[BV];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      const int v = tid + i * T;
      const int row = v >> 3, ch = v & 7;
      const int gm = m0 + row, gk = k0 + ch * 8;
      ra[i] = (gm < M && gk < K) ? *reinterpret_cast<const u32x4 *>(g.X + (int64_t)gm * g.ldx + gk)
                                 : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < BV; ++i) {
      const int v = tid + i * T;
      const int row = v >> 3, ch = v & 7;
      const int gn = n0 + row, gk = k0 + ch * 8;
      rb[i] = (gn < N && gk < K) ? *reinterpret_cast<const u32x4 *>(g.W + (int64_t)gn * g.ldw + gk)
                                 : u32x4{0, 0, 0, 0};
    }
  };
  auto sstore = [&](int buf) {
    bf16_t *a = sA + buf * BM * kLdsStride;
    bf16_t *b = sB + buf * BN * kLdsStride;
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      const int v = tid + i * T;
      *reinterpret_cast<u32x4 *>(a + (v >> 3) * kLdsStride + (v & 7) * 8) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < BV; ++i) {
      const int v = tid + i * T;
      *reinterpret_cast<u32x4 *>(b + (v >> 3) * kLdsStride + (v & 7) * 8) = rb[i];
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int KT = (K + kBK - 1) / kBK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gload((kt + 1) * kBK);
    const bf16_t *a = sA + cur * BM * kLdsStride + (wm * TM + (l & 31)) * kLdsStride + (l >> 5) * 8;
    const bf16_t *b = sB + cur * BN * kLdsStride + (wn * TN + (l & 31)) * kLdsStride + (l >> 5) * 8;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      mfma_bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = as_bf16x8(*reinterpret_cast<const u32x4 *>(a + i * 32 * kLdsStride + kk * 16));
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = as_bf16x8(*reinterpret_cast<const u32x4 *>(b + j * 32 * kLdsStride + kk * 16));
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) sstore(cur ^ 1);
    __syncthreads();
  }

  if constexpr (LORA) {
    // LDS reuse: row -> LoRA segment of the tile, distinct segment list,
    // staged Bt tile [BN][RS] (K-contiguous per output column).
    int *s_rowseg = reinterpret_cast<int *>(smem);
    int *s_useg = s_rowseg + BM;
    int *s_nu = s_useg + BM;
    bf16_t *sBt = reinterpret_cast<bf16_t *>(smem + 2 * BM * 4 + 16);
    constexpr int RS = 64 + 8;
    for (int i = tid; i < BM; i += T) {
      const int row = m0 + i;
      int u = -1;
      if (row < M) {
        const int s = g.row_segment[row];
        if (g.seg_rank[s] > 0) u = s;
      }
      s_rowseg[i] = u;
    }
    if (tid == 0) *s_nu = 0;
    __syncthreads();
    for (int i = tid; i < BM; i += T) {
      const int u = s_rowseg[i];
      if (u >= 0) {
        bool first = true;
        for (int j = i - 1; j >= 0; --j)
          if (s_rowseg[j] == u) { first = false; break; }
        if (first) s_useg[atomicAdd(s_nu, 1)] = u;
      }
    }
    __syncthreads();
    const int nu = *s_nu;
    for (int ui = 0; ui < nu; ++ui) {
      const int u = s_useg[ui];
      const int slot = g.seg_slot[u];
      const int r = g.seg_rank[u];
      const float sc = g.seg_scale[u];
      const int R = rank_bucket(r, g.policy, g.r_max);
      const int Rp = (R + 15) & ~15;
      // stage Bt_slot[0:Rp][n0:n0+BN]; rows >= r (and columns >= N) are zero
      for (int v = tid; v < Rp * (BN / 8); v += T) {
        const int k = v / (BN / 8);
        const int c8 = (v - k * (BN / 8)) * 8;
        const int gcol = n0 + c8;
        u32x4 raw = {0, 0, 0, 0};
        if (k < R && gcol < N) {
          raw = *reinterpret_cast<const u32x4 *>(g.Bt + ((int64_t)slot * g.r_max + k) * N + gcol);
          asm volatile("" : "+v"(raw));
        }
        if (k >= r) raw = u32x4{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sBt[(c8 + 2 * e) * RS + k] = (bf16_t)(raw[e] & 0xffffu);
          sBt[(c8 + 2 * e + 1) * RS + k] = (bf16_t)(raw[e] >> 16);
        }
      }
      __syncthreads();
      const int KS = Rp / 16;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int lrow = wm * TM + i * 32 + (l & 31);
        const bool in_u = s_rowseg[lrow] == u;
        const float *hrow = g.H + (int64_t)(m0 + lrow) * g.r_max;
        mfma_bf16x8 ahi[4], alo[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          if (kk < KS) {
            u32x4 phi, plo;
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
              uint32_t hw = 0, lw = 0;
#pragma unroll
              for (int h2 = 0; h2 < 2; ++h2) {
                const int kidx = kk * 16 + (l >> 5) * 8 + e2 * 2 + h2;
                const float h = (in_u && kidx < r) ? sc * hrow[kidx] : 0.f;
                const uint32_t hb = f32_to_bf16_rne(h);
                const uint32_t lb = f32_to_bf16_rne(h - bf16_to_f32(hb));
                hw |= hb << (16 * h2);
                lw |= lb << (16 * h2);
              }
              phi[e2] = hw;
              plo[e2] = lw;
            }
            ahi[kk] = as_bf16x8(phi);
            alo[kk] = as_bf16x8(plo);
          }
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          f32x16 t;
#pragma unroll
          for (int v = 0; v < 16; ++v) t[v] = 0.f;
          const bf16_t *bcol = sBt + (wn * TN + j * 32 + (l & 31)) * RS + (l >> 5) * 8;
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            if (kk < KS) {
              const mfma_bf16x8 bv = as_bf16x8(*reinterpret_cast<const u32x4 *>(bcol + kk * 16));
              t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi[kk], bv, t, 0, 0, 0);
              t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo[kk], bv, t, 0, 0, 0);
            }
          }
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int lr = wm * TM + i * 32 + acc_row(v, l);
            if (s_rowseg[lr] == u) acc[i][j][v] += t[v];
          }
        }
      }
      __syncthreads();
    }
  }

  // store: bf16 round to nearest even, once
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = n0 + wn * TN + j * 32 + (l & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm * TM + i * 32 + acc_row(v, l);
        if (row < M && col < N) g.Y[(int64_t)row * g.ldy + col] = (bf16_t)f32_to_bf16_rne(acc[i][j][v]);
      }
    }
  }
}

// ----------------------------------------------------------------------------
// fp32: plain VALU tiles (64 x 64 per block, 4 x 4 per thread) through LDS;
// the fused increment is a direct sum over k < r per output element.
// ----------------------------------------------------------------------------
struct GemmF32Args {
  const float *X;
  int64_t ldx;
  const float *W;
  int64_t ldw;
  float *Y;
  int64_t ldy;
  int M, K, N;
  const float *H;
  const float *Bt;
  const int32_t *row_segment, *seg_slot, *seg_rank;
  const float *seg_scale;
  int r_max;
};

template <bool LORA>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmF32Args g) {
  constexpr int BMF = 64, BNF = 64, BKF = 16;
  __shared__ float sA[BKF][BMF + 4];
  __shared__ float sB[BKF][BNF + 4];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * BMF, n0 = blockIdx.x * BNF;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < g.K; k0 += BKF) {
    {
      const int row = tid >> 2, kq = (tid & 3) * 4;
      const int gm = m0 + row, gk = k0 + kq;
      float4 va = make_float4(0.f, 0.f, 0.f, 0.f), vb = va;
      if (gm < g.M && gk < g.K) va = *reinterpret_cast<const float4 *>(g.X + (int64_t)gm * g.ldx + gk);
      const int gn = n0 + row;
      if (gn < g.N && gk < g.K) vb = *reinterpret_cast<const float4 *>(g.W + (int64_t)gn * g.ldw + gk);
      sA[kq + 0][row] = va.x; sA[kq + 1][row] = va.y; sA[kq + 2][row] = va.z; sA[kq + 3][row] = va.w;
      sB[kq + 0][row] = vb.x; sB[kq + 1][row] = vb.y; sB[kq + 2][row] = vb.z; sB[kq + 3][row] = vb.w;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BKF; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sA[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sB[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + ty * 4 + i;
    if (row >= g.M) continue;
    if constexpr (LORA) {
      const int s = g.row_segment[row];
      const int r = g.seg_rank[s];
      if (r > 0) {
        const float sc = g.seg_scale[s];
        const float *hrow = g.H + (int64_t)row * g.r_max;
        const float *bt = g.Bt + (int64_t)g.seg_slot[s] * g.r_max * g.N;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = n0 + tx * 4 + j;
          if (col >= g.N) continue;
          float d = 0.f;
          for (int k = 0; k < r; ++k) d = fmaf(hrow[k], bt[(int64_t)k * g.N + col], d);
          acc[i][j] += sc * d;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      if (col < g.N) g.Y[(int64_t)row * g.ldy + col] = acc[i][j];
    }
  }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_bf16(const GemmArgs &g, bool lora, hipStream_t stream) {
  dim3 grid((g.N + BN - 1) / BN, (g.M + BM - 1) / BM);
  dim3 block(WM * WN * kWave);
  if (lora)
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, true>), grid, block, 0, stream, g);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, false>), grid, block, 0, stream, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const void *X, int64_t ldx, const void *W, int64_t ldw, void *Y,
                       int64_t ldy, int M, int K, int N, int dtype, const float *H,
                       const SegView *seg, const PoolView *pool, hipStream_t stream) {
  const bool lora = seg != nullptr;
  if (dtype == 1) {
    GemmArgs g{(const bf16_t *)X, ldx, (const bf16_t *)W, ldw, (bf16_t *)Y, ldy, M, K, N,
               H, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 0};
    if (lora) {
      g.Bt = (const bf16_t *)pool->Bt;
      g.row_segment = seg->row_segment;
      g.seg_slot = seg->seg_slot;
      g.seg_rank = seg->seg_rank;
      g.seg_scale = seg->seg_scale;
      g.r_max = pool->r_max;
      g.policy = pool->policy;
    }
    if (M <= 512) return launch_bf16<64, 64, 2, 2>(g, lora, stream);
    return launch_bf16<128, 128, 2, 2>(g, lora, stream);
  }
  GemmF32Args g{(const float *)X, ldx, (const float *)W, ldw, (float *)Y, ldy, M, K, N,
                H, nullptr, nullptr, nullptr, nullptr, nullptr, 0};
  if (lora) {
    g.Bt = (const float *)pool->Bt;
    g.row_segment = seg->row_segment;
    g.seg_slot = seg->seg_slot;
    g.seg_rank = seg->seg_rank;
    g.seg_scale = seg->seg_scale;
    g.r_max = pool->r_max;
  }
  dim3 grid((N + 63) / 64, (M + 63) / 64);
  if (lora)
    hipLaunchKernelGGL(gemm_f32_kernel<true>, grid, dim3(256), 0, stream, g);
  else
    hipLaunchKernelGGL(gemm_f32_kernel<false>, grid, dim3(256), 0, stream, g);
  return hipGetLastError();
}

}  // namespace lora
