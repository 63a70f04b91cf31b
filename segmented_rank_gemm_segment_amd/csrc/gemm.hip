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
// bf16: MFMA v_mfma_f32_32x32x16_bf16 (gfx950).  Both operands are
// K-contiguous (X rows and nn.Linear W rows).  Tiles stream into LDS with
// direct global->LDS loads through a multi-stage ring, so several K steps
// are in flight per workgroup; LDS rows are XOR-swizzled in 16-byte chunks
// so fragment reads are bank-conflict free.  Tiles are ordered per XCD.
//
// Fused LoRA: the rows of an output tile may belong to several segments.
// After the K loop, for each distinct LoRA segment u among the tile's rows,
// the scaled H rows of u (split into a bf16 high part and a bf16 remainder,
// so H keeps about 16 significant bits) and B_u are staged in LDS and
// multiplied by MFMA into the accumulators, zero rows standing in for rows
// of other segments.  Every row gets exactly its own segment's increment,
// added in fp32 and rounded once with the base product.
//
// The small tiles also run the whole layer in one launch (layer.cuh): the
// segment metadata and H are produced inside the same kernel, before each
// tile's K loop, and handed between workgroups through per-row flags.
#include <climits>

#include "layer.cuh"
#include "lds_dma.cuh"
#include "lora_device.cuh"
#include "lora_kernels.h"

namespace lora {
namespace {


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
  const bf16_t *Bn;   // optional d_out-major copy of B ([slot][d_out][rs]) or null
  const int32_t *row_segment, *seg_slot, *seg_rank;
  const float *seg_scale;
  int r_max, policy;
  const float *dora;   // optional DoRA column factors ([slot][N]) or null
  const float *wscale; // FP8 weight: one scale per output row (W then holds E4M3 codes)
  ProjView proj;       // projections of the output columns (one unless stacked)
  LayerArgs lay;       // the one-launch layer's inputs and outputs (layer.cuh)
};

// Tile configurations <BM, BN, waves along M, waves along N, K per group
// slice, LDS stages, K groups>: small-M (decode-like) batches and large
// batches.
#ifndef LORA_GEMM_SMALL
#define LORA_GEMM_SMALL 64, 64, 2, 2, 64, 4, 2
#endif
// The same tiles with two stages (64 KB of LDS, so two workgroups share a
// CU), for small batches whose grid has more tiles than there are CUs
// (measured: 512 x 4096 x 4096 in 29.5 us against 34.5, 256 x 4096 x 14336
// in 53 against 63; with at most one tile per CU the four stages are faster:
// 64 x 4096 x 14336 in 20 against 24 us).
#ifndef LORA_GEMM_SMALL_WIDE
#define LORA_GEMM_SMALL_WIDE 64, 64, 2, 2, 64, 2, 2
#endif
#ifndef LORA_GEMM_LARGE
#define LORA_GEMM_LARGE 256, 256, 2, 4, 64, 2, 1
#endif
// Mid-size tiles, for batches past LORA_GEMM_SMALL_M rows whose 256 x 256
// grid would not fill half of the 256 CUs (measured: 2304 x 1024 x 8192 in
// 88 us against 170 us, 1024 x 4096 x 4096 in 49 against 94 us).
#ifndef LORA_GEMM_MID
#define LORA_GEMM_MID 128, 128, 2, 2, 64, 4, 1
#endif
#ifndef LORA_GEMM_MID_TILES
#define LORA_GEMM_MID_TILES 128
#endif
#ifndef LORA_GEMM_SMALL_F8
#define LORA_GEMM_SMALL_F8 LORA_GEMM_SMALL
#endif
#ifndef LORA_GEMM_MID_F8
#define LORA_GEMM_MID_F8 LORA_GEMM_MID
#endif
#ifndef LORA_GEMM_LARGE_F8
#define LORA_GEMM_LARGE_F8 LORA_GEMM_LARGE
#endif
// 192-row large tiles (8 waves of 96 x 64), for batches whose 256 x 256 grid
// ends in a nearly empty round on the 256 CUs (2304 rows x 8192 columns:
// 288 tiles of 256 x 256 fill 1.125 rounds, 384 of 192 x 256 fill 1.5).
#ifndef LORA_GEMM_LARGE192
#define LORA_GEMM_LARGE192 192, 256, 2, 4, 64, 2, 1
#endif
#ifndef LORA_GEMM_LARGE192_F8
#define LORA_GEMM_LARGE192_F8 LORA_GEMM_LARGE192
#endif
// Relative cost per output element of a 192 x 256 tile against a 256 x 256
// one (more LDS fragment reads per flop), in percent.
#ifndef LORA_GEMM_192_COST
#define LORA_GEMM_192_COST 110
#endif
// Large and mid tiles with more LoRA runs than this (consecutive rows of one
// segment; decode rows make one each) finish row by row on the VALU instead
// of one staged MFMA increment per segment.
#ifndef LORA_GEMM_STAGED_RUNS
#define LORA_GEMM_STAGED_RUNS 4
#endif
#ifndef LORA_GEMM_SGB
#define LORA_GEMM_SGB 1
#endif
#ifndef LORA_GEMM_SMALL_M
#define LORA_GEMM_SMALL_M 512
#endif
// Tail split: a large batch whose 256 x 256 grid ends in a partial round of
// the CUs runs the rows of its whole rounds on the large tiles and the
// remaining rows (at most LORA_GEMM_SMALL_M) on the small tiles, as a
// second launch, when that remainder has at most this many small tiles
// (their per-CU bytes then stay under one round of large tiles).
#ifndef LORA_GEMM_TAIL_SPLIT
#define LORA_GEMM_TAIL_SPLIT 1
#endif
#ifndef LORA_GEMM_TAIL_TILES
#define LORA_GEMM_TAIL_TILES 1024
#endif

// KG wave groups split each K step: group g takes the g-th BK-wide slice of
// it with its own WM x WN waves and its own slice of the stage, and the
// groups' partial sums are added through LDS at the end (KG = 1: one group).
// EB: bytes per element of the B operand (W): 2 for bf16, 1 for FP8 codes.
template <int BM, int BN, int WM, int WN, int BK, int STAGES, int KG, int EB = 2>
struct TileCfg {
  static constexpr int kBM = BM, kBN = BN;
  static constexpr int NWG = WM * WN;               // waves per group
  static constexpr int NW = NWG * KG;
  static constexpr int T = NW * kWave;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 32, FN = TN / 32;
  static constexpr int CH = BK / 8;                 // 16-byte chunks per A row (bf16)
  static constexpr int RB = BK * 2;                 // bytes per A row in LDS
  static constexpr int RPI = 1024 / RB;             // A rows per 1 KB DMA instruction
  static constexpr int RBB = BK * EB;               // bytes per B row in LDS
  static constexpr int CHB = RBB / 16;              // 16-byte chunks per B row
  static constexpr int RPIB = 1024 / RBB;           // B rows per 1 KB DMA instruction
  static constexpr int EPCB = 16 / EB;              // B elements per 16-byte chunk
  static constexpr int AI = BM / RPI / NWG, BI = BN / RPIB / NWG;  // DMA instructions per wave
  static constexpr int IPW = AI + BI;
  static constexpr int GSTAGE = BM * RB + BN * RBB; // bytes of one group's slice
  static constexpr int STAGE = KG * GSTAGE;         // bytes of a stage
  static constexpr int KSTEP = KG * BK;             // K per stage
  static constexpr int LDS = STAGES * STAGE;
  static constexpr int RED = (KG - 1) * NWG * FM * FN * 16 * kWave * 4;  // partial sums
  static_assert(BK == 32 || BK == 64, "K per stage");
  static_assert(FM >= 1 && FN >= 1, "wave tile");
  static_assert(BM % (RPI * NWG) == 0 && BN % (RPIB * NWG) == 0, "DMA split");
  static_assert(EB == 2 || (EB == 1 && BK == 64), "FP8 B rows are 64 bytes");
  static_assert(STAGES >= 2 && STAGES - 2 <= 6 && (STAGES - 2) * IPW <= 63, "pipeline depth");
  static_assert(LDS <= 160 * 1024 && RED <= LDS, "LDS");
  // physical chunk of logical chunk c in row r.  The gfx950 LDS serves a
  // 16-byte read for 16 lanes at a time across 64 four-byte banks (256
  // bytes), i.e. two 128-byte rows or four 64-byte rows per bank row; the
  // XOR below gives 16 consecutive rows at one logical chunk 16 distinct
  // 16-byte bank groups (measured: c ^ (r & 7) left 2-way conflicts).
  __device__ static __forceinline__ int swz(int c, int r) {
    return CH == 8 ? (c ^ ((r >> 1) & 7)) : (c ^ ((r >> 2) & 3));
  }
  // the same for B rows (64-byte rows: four per bank row, so the chunk is
  // XORed with bits 2..3 of the row)
  __device__ static __forceinline__ int swzb(int c, int r) {
    return CHB == 8 ? (c ^ ((r >> 1) & 7)) : (c ^ ((r >> 2) & 3));
  }
};

// Eight E4M3 codes (bytes of lo, then hi; element e = byte e) to eight bf16
// for the MFMA, two per v_cvt_scalef32_pk_bf16_fp8 with scale 1: every E4M3
// value is exact in bf16, so this is exact.
__device__ __forceinline__ mfma_bf16x8 fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  return as_bf16x8(u32x4{
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true))});
}

// LoRA term of one output row over 8 consecutive columns, added to o in fp32:
// o[e] += sc sum_{k < r} H[grow][qoff + k] Bt_slot[k][gcol + e], k
// ascending, read in chunks of 8 rank rows; then, with DoRA, the slot's
// column factors.  r need not be a multiple of 8: a chunk's rank rows at or
// past r are read inside the slot's rs rank rows (rs a multiple of 8) and
// skipped.  qoff is the offset of the columns' projection in H's rank
// entries (offsets of projections are multiples of 8, so all 8 columns share
// it); Bt holds every column's own projection in rank rows [0, rs).  Shared by both row epilogues, so both give the same bits.
// (Loading two chunks per step measured no faster on 64x64 tiles.)
// COH: H was written by other workgroups of the same launch and is read
// with agent-scope loads (layer.cuh).
template <bool DORA, bool COH = false>
__device__ __forceinline__ void lora_row8(const GemmArgs &g, int grow, int gcol, int slot, int r,
                                          float sc, float (&o)[8]) {
  const int N = g.N;
  const int qoff = proj_of(g.proj, gcol) * g.proj.rs;
  const bf16_t *bt = g.Bt + (int64_t)slot * g.proj.rs * N + gcol;
  const float *hp = g.H + (int64_t)grow * g.r_max + qoff;
  float d[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int kc = 0; kc < r; kc += 8) {      // kc < r <= rs: the chunk is in the block
    float h[8];
    if constexpr (COH) {
#pragma unroll
      for (int q = 0; q < 8; ++q) h[q] = ld_agent(hp + kc + q);
    } else {
      const f32x4 h0 = *reinterpret_cast<const f32x4 *>(hp + kc);
      const f32x4 h1 = *reinterpret_cast<const f32x4 *>(hp + kc + 4);
      h[0] = h0[0]; h[1] = h0[1]; h[2] = h0[2]; h[3] = h0[3];
      h[4] = h1[0]; h[5] = h1[1]; h[6] = h1[2]; h[7] = h1[3];
    }
    u32x4 b[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) b[q] = *reinterpret_cast<const u32x4 *>(bt + (int64_t)(kc + q) * N);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const bool use = kc + q < r;
      float bv[8];
      Elem<bf16_t>::unpack(make_uint4(b[q][0], b[q][1], b[q][2], b[q][3]), bv);
#pragma unroll
      for (int e = 0; e < 8; ++e) d[e] = use ? fmaf(h[q], bv[e], d[e]) : d[e];
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = fmaf(sc, d[e], o[e]);
  if constexpr (DORA) {
    const float *gp = g.dora + (int64_t)slot * N + gcol;
    const f32x4 g0 = *reinterpret_cast<const f32x4 *>(gp);
    const f32x4 g1 = *reinterpret_cast<const f32x4 *>(gp + 4);
    o[0] *= g0[0]; o[1] *= g0[1]; o[2] *= g0[2]; o[3] *= g0[3];
    o[4] *= g1[0]; o[5] *= g1[1]; o[6] *= g1[2]; o[7] *= g1[3];
  }
}

// lora_row8 for two (row, 8 columns) items at once, so that the loads of
// both are in flight together: chunk kc of an item whose rank ends earlier
// re-reads its first chunk (in the block) and adds nothing.  Each item's sum
// is formed in the same order as lora_row8's, so the bits are the same.
template <bool DORA>
__device__ __forceinline__ void lora_row8_pair(const GemmArgs &g, const int (&grow)[2],
                                               const int (&gcol)[2], const int (&slot)[2],
                                               const int (&r)[2], const float (&sc)[2],
                                               float (&o)[2][8]) {
  const int N = g.N;
  const bf16_t *bt[2];
  const float *hp[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int qoff = proj_of(g.proj, gcol[u]) * g.proj.rs;
    bt[u] = g.Bt + (int64_t)slot[u] * g.proj.rs * N + gcol[u];
    hp[u] = g.H + (int64_t)grow[u] * g.r_max + qoff;
  }
  float d[2][8];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) d[u][e] = 0.f;
  const int rmax = max(r[0], r[1]);
  for (int kc = 0; kc < rmax; kc += 8) {
    f32x4 h0[2], h1[2];
    u32x4 b[2][8];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      // an item whose rank ends before kc re-reads its first chunk (in the
      // block) and adds nothing
      const int kk = kc < r[u] ? kc : 0;
      h0[u] = *reinterpret_cast<const f32x4 *>(hp[u] + kk);
      h1[u] = *reinterpret_cast<const f32x4 *>(hp[u] + kk + 4);
#pragma unroll
      for (int q = 0; q < 8; ++q)
        b[u][q] = *reinterpret_cast<const u32x4 *>(bt[u] + (int64_t)(kk + q) * N);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float h[8] = {h0[u][0], h0[u][1], h0[u][2], h0[u][3],
                          h1[u][0], h1[u][1], h1[u][2], h1[u][3]};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const bool use = kc + q < r[u];
        float bv[8];
        Elem<bf16_t>::unpack(make_uint4(b[u][q][0], b[u][q][1], b[u][q][2], b[u][q][3]), bv);
#pragma unroll
        for (int e = 0; e < 8; ++e) d[u][e] = use ? fmaf(h[q], bv[e], d[u][e]) : d[u][e];
      }
    }
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    if (r[u] <= 0) continue;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[u][e] = fmaf(sc[u], d[u][e], o[u][e]);
    if constexpr (DORA) {
      const float *gp = g.dora + (int64_t)slot[u] * N + gcol[u];
      const f32x4 g0 = *reinterpret_cast<const f32x4 *>(gp);
      const f32x4 g1 = *reinterpret_cast<const f32x4 *>(gp + 4);
      o[u][0] *= g0[0]; o[u][1] *= g0[1]; o[u][2] *= g0[2]; o[u][3] *= g0[3];
      o[u][4] *= g1[0]; o[u][5] *= g1[1]; o[u][6] *= g1[2]; o[u][7] *= g1[3];
    }
  }
}

// Tile order of the MFMA kernels.  Workgroup b runs on XCD b % 8 (the
// dispatcher deals consecutive ids round robin over the eight XCDs), and
// each XCD walks its tiles in groups of M-tiles sweeping N, so that
// neighbours share operand tiles in one L2.  Batches of at most
// kHeavyMaxTilesM M-tiles with at least 8 N-tiles: XCD x owns N-tiles
// [x tiles_n / 8, (x + 1) tiles_n / 8) of every M-tile, in groups of 16
// M-tiles (measured 2-4% faster than 8 at 9 M-tiles of 2304 rows), so any
// M-tile's work spreads over all eight XCDs, and an M-tile `heavy` (>= 0)
// comes before the groups, all of its tiles of the XCD first.  Larger batches: XCD x takes
// the x-th eighth of the order over all tiles in groups of 8 M-tiles (each
// XCD then holds a few M-tiles' X rows and streams W, half the L2 misses of
// the N split at 67 M-tiles).  Returns false for a workgroup past its XCD's tiles.
// tile_grid is the launch size that covers every tile.
constexpr int kTileGroup = 8;
constexpr int kTileGroupSplit = 16;   // M-tiles per group with the N split
constexpr int kHeavyMaxTilesM = 32;
constexpr int kCUs = 256;   // compute units of an MI355X
__host__ __device__ inline bool n_split(int tiles_m, int tiles_n) {
  return tiles_n >= 8 && tiles_m <= kHeavyMaxTilesM;
}
__host__ __device__ inline int tile_grid(int tiles_m, int tiles_n) {
  return n_split(tiles_m, tiles_n) ? 8 * ((tiles_n + 7) / 8) * tiles_m
                                   : (tiles_m * tiles_n + 7) / 8 * 8;
}
__device__ __forceinline__ bool tile_order(int b, int tiles_m, int tiles_n, int heavy, int &m_idx,
                                           int &n_idx) {
  const int x = b & 7, j = b >> 3;
  int n_lo, nx, t;
  if (n_split(tiles_m, tiles_n)) {
    n_lo = x * tiles_n / 8;
    nx = (x + 1) * tiles_n / 8 - n_lo;
    if (j >= nx * tiles_m) return false;
    t = j;
  } else {
    n_lo = 0;
    nx = tiles_n;
    t = x * ((tiles_m * tiles_n + 7) / 8) + j;
    if (t >= tiles_m * tiles_n) return false;
  }
  int tm = tiles_m;
  if (heavy >= 0) {
    if (t < nx) {
      m_idx = heavy;
      n_idx = n_lo + t;
      return true;
    }
    t -= nx;
    tm = tiles_m - 1;
  }
  const int G = n_split(tiles_m, tiles_n) ? kTileGroupSplit : kTileGroup;
  const int grp = t / (G * nx);
  const int first_m = grp * G;
  const int gcnt = min(G, tm - first_m);
  const int tin = t - grp * G * nx;
  m_idx = first_m + tin % gcnt;
  if (heavy >= 0 && m_idx >= heavy) ++m_idx;
  n_idx = n_lo + tin / gcnt;
  return true;
}

// Which end M-tile of the batch holds more runs of segment ids (a row
// whose segment differs from the previous row's starts one): tiles_m - 1 if
// the last, 0 if the first, -1 if neither.  The first wave counts them with
// ballots and shares the answer through one LDS word (s), which is free
// again on return.  Called by every thread, before the tile's first LDS
// write; tiles_m >= 2.
__device__ __forceinline__ int heavier_end_tile(const int32_t *row_segment, int M, int BM,
                                                int tiles_m, int *s) {
  if (threadIdx.x < kWave) {
    const int l = threadIdx.x;
    const int last0 = (tiles_m - 1) * BM;
    int c0 = 0, c1 = 0;
    for (int r = l; r < BM; r += kWave) {
      // the first M-tile is whole (tiles_m >= 2); a tile's first row starts no run
      const bool a = r > 0 && row_segment[r] != row_segment[r - 1];
      const bool b = last0 + r < M && r > 0 && row_segment[last0 + r] != row_segment[last0 + r - 1];
      c0 += __popcll(__ballot(a));
      c1 += __popcll(__ballot(b));
    }
    if (l == 0) s[0] = c1 > c0 ? tiles_m - 1 : (c0 > c1 ? 0 : -1);
  }
  __syncthreads();
  const int h = s[0];
  __syncthreads();   // every wave has read s before the ring is written
  return h;
}

// LDS layout of a stage: A rows [BM][BK] then B rows [BN][BK], 16-byte
// chunks XOR-swizzled per row (TileCfg::swz, swzb).  WF8: W holds E4M3 codes
// (one byte per element, 64-byte B rows in LDS), widened to bf16 as each
// fragment is read; the per-row weight scale multiplies the fp32 base
// accumulator before the LoRA term is added.
// LORA: 0 = plain product; 1 = fused LoRA with B gathered from Bt; 2 = fused
// LoRA with B read from its d_out-major copy.  DORA: rows of rank > 0 are
// multiplied by their slot's column factors before the rounding.  LAYER
// (small tiles): the whole layer in one launch (layer.cuh); the row
// metadata and H come from the launch itself instead of earlier calls.
template <int BM, int BN, int WM, int WN, int BK, int STAGES, int KG, int LORA, bool DORA,
          bool WF8, bool LAYER = false>
__global__ __launch_bounds__(WM *WN *KG *kWave) void gemm_bf16_kernel(GemmArgs g) {
  using C = TileCfg<BM, BN, WM, WN, BK, STAGES, KG, WF8 ? 1 : 2>;
  static_assert(!LAYER || (KG > 1 && LORA == 1 && WM * WN * KG * kWave == kLayerThreads),
                "the one-launch layer runs on the small tiles");
  static_assert(!LAYER || C::LDS >= (4 * 4095 + 2) * 4, "the build's tables fit in the ring");
  // LDS: the stage ring, or the fused LoRA epilogue of large tiles if larger:
  // the staged segment operands (EPI_STG bytes) or one 32-row fp32 slot per
  // wave (row stride TN + 4), then per-row rank, slot and scale and a word
  constexpr int EPI_STG = 3 * (BM > BN ? BM : BN) * 128 + 16 + 4 * BM;
  constexpr int EPI_ROW = C::NW * 32 * (BN / WN + 4) * 4;
  constexpr int EPI_META = ((EPI_ROW > EPI_STG ? EPI_ROW : EPI_STG) + 15) / 16 * 16;
  constexpr int LSTG = (LORA != 0 && KG == 1) ? EPI_META + 12 * BM + 16 : 0;
  constexpr int SMEM = C::LDS > LSTG ? C::LDS : LSTG;
  // the layer's LDS follows the ring (both live at once before the K loop)
  constexpr int LAYB = LAYER ? (int)sizeof(LayerLds) : 0;
  __shared__ __align__(16) unsigned char smem[SMEM + LAYB];
  LayerLds &Lay = *reinterpret_cast<LayerLds *>(smem + SMEM);

  const int tid = threadIdx.x;
  const int l = tid & (kWave - 1);
  // K group and wave within it (wave-uniform: scalar registers)
  const int kgrp = __builtin_amdgcn_readfirstlane(tid / (kWave * C::NWG));
  const int wid = __builtin_amdgcn_readfirstlane((tid / kWave) % C::NWG);
  const int wm = wid / WN, wn = wid % WN;
  const int kg0 = kgrp * BK;                        // the group's offset in a K step
  const int M = g.M, N = g.N, K = g.K;

  // XCD-aware tile order (tile_order): consecutive workgroup ids go to
  // different XCDs (round robin over 8), and each XCD walks its share of the
  // tiles in groups of M-tiles sweeping N, so operand tiles shared by
  // neighbours stay inside one L2.
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  // Tiles of many LoRA runs take the row epilogue, which costs more than
  // the staged one (decode rows beside a prefill request); so that they run
  // first rather than in a last, partly filled wave, the end M-tile of the
  // batch with more runs is taken first (longest first).  Only for grids of
  // more than one wave (these tiles run one workgroup per CU) and at most
  // kHeavyMaxTilesM M-tiles: the check costs a memory round trip per
  // workgroup.
  int heavy = -1;
  if constexpr (LORA != 0 && KG == 1) {
    if (tiles_m > 1 && tiles_m <= kHeavyMaxTilesM && tiles_m * tiles_n > kCUs)
      heavy = heavier_end_tile(g.row_segment, M, BM, tiles_m, reinterpret_cast<int *>(smem));
  }
  int m_idx = 0, n_idx = 0;
  const bool has_tile = tile_order(blockIdx.x, tiles_m, tiles_n, heavy, m_idx, n_idx);
  // (a layer workgroup without a tile still has its row of the layer to do)
  if (!LAYER && !has_tile) return;
  if (LAYER && !has_tile) m_idx = n_idx = 0;
  const int m0 = m_idx * BM;
  const int n0 = n_idx * BN;

  // Small tiles (two K groups) finish row by row: thread tid owns tile row
  // tid / (BN / 8) and 8 consecutive columns (see the end of the kernel);
  // in larger tiles thread tid < BM holds tile row tid's metadata for the
  // LoRA term.  The row's segment id (and, with an FP8 weight, the thread's
  // 8 column scales) are loaded before the first DMA, and the segment's
  // rank, slot and scale right after the prologue's wait, so all have
  // arrived by the epilogue.  They are ordinary loads, waited for by the
  // compiler: it does not see the DMAs, so its waits count only these loads,
  // and it can only wait for more than it needs (the column scales are
  // requested first, so the segment id is the newest load when it is used).
  constexpr bool ROWEPI = KG > 1;
  static_assert(!ROWEPI || C::T * 8 == BM * BN, "row epilogue: 8 outputs per thread");
  static_assert(ROWEPI || C::T >= BM, "one tile row per thread");
  const int e_row = ROWEPI ? tid / (BN / 8) : tid, e_c8 = (tid % (BN / 8)) * 8;
  const bool e_own = ROWEPI || tid < BM;            // the thread holds row e_row's metadata
  f32x4 e_ws0 = f32x4{0.f, 0.f, 0.f, 0.f}, e_ws1 = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (ROWEPI && WF8) {
    const float *ws = g.wscale + min(n0 + e_c8, N - 8);
    e_ws0 = *reinterpret_cast<const f32x4 *>(ws);
    e_ws1 = *reinterpret_cast<const f32x4 *>(ws + 4);
  }
  int e_seg = 0, e_r = 0, e_slot = 0, e_scb = 0;
  if constexpr (LORA != 0 && !LAYER)
    if (e_own) e_seg = g.row_segment[min(m0 + e_row, M - 1)];

  // DMA sources: lane l of an instruction fills tile row base + l / CH at
  // physical chunk l % CH, i.e. logical chunk swz(l % CH, row) (a function
  // of the row, so of the instruction too).  Rows past M / N are clamped to
  // the last valid row (their results are never stored).
  const int rr = l / C::CH, rrb = l / C::CHB;
  int alc[C::AI], blc[C::BI];
  const bf16_t *asrc[C::AI];
  const unsigned char *bsrc[C::BI];                 // B sources in bytes
#pragma unroll
  for (int i = 0; i < C::AI; ++i) {
    const int row = (wid * C::AI + i) * C::RPI + rr;
    alc[i] = C::swz(l % C::CH, row);
    asrc[i] = g.X + (int64_t)min(m0 + row, M - 1) * g.ldx + alc[i] * 8;
  }
#pragma unroll
  for (int i = 0; i < C::BI; ++i) {
    const int row = (wid * C::BI + i) * C::RPIB + rrb;
    blc[i] = C::swzb(l % C::CHB, row);
    bsrc[i] = reinterpret_cast<const unsigned char *>(g.W) +
              ((int64_t)min(n0 + row, N - 1) * g.ldw + blc[i] * C::EPCB) * (WF8 ? 1 : 2);
  }
  // byte offset of K position k0 in a B row's chunk, or back to the row's
  // first chunk when the chunk lies past K (in bounds; zeroed before use)
  auto boff = [&](int i, int k0) __attribute__((always_inline)) {
    return (k0 + blc[i] * C::EPCB < K) ? k0 * (WF8 ? 1 : 2) : -blc[i] * 16;
  };
  const uint32_t sbase = lds_offset(smem);
  const uint32_t a_dst =
      __builtin_amdgcn_readfirstlane(sbase + kgrp * C::GSTAGE + wid * C::AI * 1024);
  const uint32_t b_dst = __builtin_amdgcn_readfirstlane(sbase + kgrp * C::GSTAGE + BM * C::RB +
                                                        wid * C::BI * 1024);

  auto issue = [&](int stage, int k0) {
    // a chunk past K reads the row's first chunk instead (in bounds) and is
    // zeroed in LDS before use
#pragma unroll
    for (int i = 0; i < C::AI; ++i)
      dma16(a_dst + stage * C::STAGE + i * 1024,
            asrc[i] + ((k0 + alc[i] * 8 < K) ? k0 : -alc[i] * 8));
#pragma unroll
    for (int i = 0; i < C::BI; ++i) dma16(b_dst + stage * C::STAGE + i * 1024, bsrc[i] + boff(i, k0));
  };
  // instruction q of a stage's DMA (A rows first, then B rows)
  auto issue_one = [&](int q, int stage, int k0) __attribute__((always_inline)) {
    if (q < C::AI)
      dma16(a_dst + stage * C::STAGE + q * 1024,
            asrc[q] + ((k0 + alc[q] * 8 < K) ? k0 : -alc[q] * 8));
    else
      dma16(b_dst + stage * C::STAGE + (q - C::AI) * 1024, bsrc[q - C::AI] + boff(q - C::AI, k0));
  };
  // Stage ownership (rings of more than two stages): wave wid of each K
  // group owns ring buffer wid and alone fills its group's slice of every
  // stage that lands there -- the slice's A rows, then its B rows, NIG 1 KB
  // instructions, sources computed per instruction.  A wave therefore never
  // has more than one stage in flight, and before a stage is read its owners
  // wait for all of their loads (vmcnt(0)) and then the workgroup passes the
  // barrier: no wait depends on the order in which DMAs complete.  Two-stage
  // rings need no owners: at each wait only the stage about to be read is in
  // flight, so every wave waits vmcnt(0) for its share of it.
  constexpr bool OWNED = STAGES > 2;
  static_assert(!OWNED || C::NWG == STAGES, "one owner wave per ring buffer in each K group");
  constexpr int AIG = BM / C::RPI, NIG = AIG + BN / C::RPIB;   // instructions per slice
  constexpr int EBW = WF8 ? 1 : 2;                             // bytes per W element
  // Sources of the owner's instructions: the tile's first A and B rows as
  // scalar bases, and per lane the byte offset of its row (rows past M / N
  // clamped to the last) and chunk from them -- below 2^32 because leading
  // dimensions are below 2^22 elements and tiles have at most 256 rows.
  const unsigned char *const xa = reinterpret_cast<const unsigned char *>(g.X + (int64_t)m0 * g.ldx);
  const unsigned char *const wb = reinterpret_cast<const unsigned char *>(g.W) +
                                  (int64_t)n0 * g.ldw * EBW;
  uint32_t own_off[OWNED ? NIG : 1];
  if constexpr (OWNED) {
#pragma unroll
    for (int t = 0; t < NIG; ++t) {
      if (t < AIG) {
        const int row = t * C::RPI + rr;
        own_off[t] = (uint32_t)((min(m0 + row, M - 1) - m0) * g.ldx * 2) +
                     C::swz(l % C::CH, row) * 16;
      } else {
        const int row = (t - AIG) * C::RPIB + rrb;
        own_off[t] = (uint32_t)((min(n0 + row, N - 1) - n0) * g.ldw * EBW) +
                     C::swzb(l % C::CHB, row) * 16;
      }
    }
  }
  // instruction t of the group's slice of the stage at K position k0 into
  // buffer buf; `tail`: the stage reaches past K, where a chunk past K reads
  // its row's first chunk instead (in bounds; zeroed before use)
  auto issue_own_one = [&](int t, int buf, int k0, bool tail) __attribute__((always_inline)) {
    const uint32_t dst =
        __builtin_amdgcn_readfirstlane(sbase + buf * C::STAGE + kgrp * C::GSTAGE + t * 1024);
    if (t < AIG) {
      if (!tail) {
        dma16_s(dst, own_off[t], xa + (int64_t)k0 * 2);
      } else {
        // the base stays scalar: the K position goes into the lane offsets
        const int row = t * C::RPI + rr;
        const int c = C::swz(l % C::CH, row);
        dma16_s(dst, k0 + c * 8 < K ? own_off[t] + k0 * 2 : own_off[t] - c * 16, xa);
      }
    } else {
      if (!tail) {
        dma16_s(dst, own_off[t], wb + (int64_t)k0 * EBW);
      } else {
        const int row = (t - AIG) * C::RPIB + rrb;
        const int c = C::swzb(l % C::CHB, row);
        dma16_s(dst, k0 + c * C::EPCB < K ? own_off[t] + k0 * EBW : own_off[t] - c * 16, wb);
      }
    }
  };
  auto zero_tail_own = [&](int buf, int k0) {
    unsigned char *st = smem + buf * C::STAGE + kgrp * C::GSTAGE;
#pragma unroll
    for (int t = 0; t < NIG; ++t) {
      const bool past = t < AIG ? k0 + C::swz(l % C::CH, t * C::RPI + rr) * 8 >= K
                                : k0 + C::swzb(l % C::CHB, (t - AIG) * C::RPIB + rrb) * C::EPCB >= K;
      if (past) *reinterpret_cast<u32x4 *>(st + t * 1024 + l * 16) = u32x4{0, 0, 0, 0};
    }
  };
  auto zero_tail = [&](int stage, int k0) {
    unsigned char *st = smem + stage * C::STAGE + kgrp * C::GSTAGE;
#pragma unroll
    for (int i = 0; i < C::AI; ++i)
      if (k0 + alc[i] * 8 >= K)
        *reinterpret_cast<u32x4 *>(st + (wid * C::AI + i) * 1024 + l * 16) = u32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < C::BI; ++i)
      if (k0 + blc[i] * C::EPCB >= K)
        *reinterpret_cast<u32x4 *>(st + BM * C::RB + (wid * C::BI + i) * 1024 + l * 16) =
            u32x4{0, 0, 0, 0};
  };

  // With FP8 weights the K loop of small tiles is bound by its arithmetic
  // (fragment widening and MFMA), and a wave with a single 32x32 fragment
  // would chain every MFMA on one accumulator; it keeps two instead (even
  // and odd sub-steps) so that consecutive MFMAs are independent, and adds
  // them after the K loop.  (The bf16 K loop is bound by its loads.)
  constexpr bool DUAL = WF8 && C::FM * C::FN == 1;
  f32x16 acc[C::FM][C::FN], acc2[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = acc2[i][j][v] = 0.f;

  // per-lane fragment offsets inside a stage (fragment rows start at
  // multiples of 32, so the swizzle of row base + (l & 31) depends on l only)
  int a_row_off[C::FM], b_row_off[C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
    a_row_off[i] = kgrp * C::GSTAGE + (wm * C::TM + i * 32 + (l & 31)) * C::RB;
#pragma unroll
  for (int j = 0; j < C::FN; ++j)
    b_row_off[j] = kgrp * C::GSTAGE + BM * C::RB + (wn * C::TN + j * 32 + (l & 31)) * C::RBB;
  int chunk_off[BK / 16], chunkb_off[BK / 16];
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) {
    chunk_off[kk] = C::swz(kk * 2 + (l >> 5), l & 31) * 16;
    // bf16 B: as A; FP8 B: sub-step kk is chunk kk, half l / 32 (8 bytes)
    chunkb_off[kk] = WF8 ? C::swzb(kk, l & 31) * 16 + (l >> 5) * 8
                         : C::swzb(kk * 2 + (l >> 5), l & 31) * 16;
  }

  const int KT = (K + C::KSTEP - 1) / C::KSTEP;
  const bool ktail = (K % C::KSTEP) != 0;
  // every buffer of the ring is free at the start: fill all of them (with
  // owners, each wave fills its own buffer)
  auto prologue = [&]() __attribute__((always_inline)) {
    if constexpr (OWNED) {
      if (wid < KT) {
        const bool tail = ktail && wid == KT - 1;
#pragma unroll
        for (int t = 0; t < NIG; ++t) issue_own_one(t, wid, wid * C::KSTEP + kg0, tail);
      }
    } else {
#pragma unroll
      for (int s = 0; s < STAGES; ++s)
        if (s < KT) issue(s, s * C::KSTEP + kg0);
    }
  };
  if constexpr (!LAYER) prologue();

  // Software pipeline over K.  Fragments of sub-step kk + 1 are read from
  // LDS while the MFMAs of sub-step kk run.  Before the last sub-step of
  // stage kt the workgroup waits for stage kt + 1 and passes one barrier
  // (every wave has by then read all of stage kt into registers), refills
  // stage kt's buffer with stage kt + STAGES, reads the first fragments of
  // stage kt + 1, and only then issues the last MFMAs of stage kt, so the
  // barrier overlaps with the matrix pipe draining.
  constexpr int KK = BK / 16;
  mfma_bf16x8 af[2][C::FM], bfr[2][C::FN];
  auto load_frags = [&](int buf, const unsigned char *st, int kk) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
      af[buf][i] = as_bf16x8(*reinterpret_cast<const u32x4 *>(st + a_row_off[i] + chunk_off[kk]));
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      if constexpr (WF8) {
        const uint2 q = *reinterpret_cast<const uint2 *>(st + b_row_off[j] + chunkb_off[kk]);
        bfr[buf][j] = fp8x8_to_bf16x8(q.x, q.y);
      } else {
        bfr[buf][j] = as_bf16x8(*reinterpret_cast<const u32x4 *>(st + b_row_off[j] + chunkb_off[kk]));
      }
    }
  };
  auto mfmas = [&](int buf, bool odd) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        if (DUAL && odd)
          acc2[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[buf][i], bfr[buf][j], acc2[i][j], 0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[buf][i], bfr[buf][j], acc[i][j], 0, 0, 0);
      }
  };
  // interleave: one MFMA, then one LDS read, while reads remain
  auto interleave = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < C::FM * C::FN; ++q) {
      if (LORA_GEMM_SGB) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (LORA_GEMM_SGB && q < C::FM + C::FN) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };

  if constexpr (LAYER) {
    // The layer's metadata and this workgroup's row of H.  The build's
    // tables live beside the ring for pools of up to kLayerTabSlots slots,
    // and the ring fills meanwhile; for larger pools they use the ring's
    // LDS and the ring is filled afterwards.  The row's first shrink
    // operands are requested before the build.
    const bool early = g.lay.n_slots <= kLayerTabSlots;
    int *tab = early ? Lay.tab : reinterpret_cast<int *>(smem);
    if (early && has_tile) prologue();
    BuildRegs br;
    layer_build_load(g.lay, M, blockIdx.x, br);
    RowPrefetch pre;
    layer_prefetch(g.lay, g.X, g.ldx, min((int)blockIdx.x, M - 1), br.slot_mine, pre);
    pre.valid = pre.valid && (int)blockIdx.x < M;
    layer_stage(g.lay, br, tab);
    // this call's generation number (one thread; first needed to publish the row)
    uint32_t gen = 0;
    if (tid == 0 && g.lay.sync) gen = ld_agent(g.lay.sync + kSyncGen);
    layer_build(g.lay, M, blockIdx.x, br, Lay, tab);   // ends with a barrier
    if ((int)blockIdx.x < M) {
      const int row = blockIdx.x;
      const int r = Lay.rk[row];
      if (r > 0) {
        layer_row_shrink(g.lay, g.X, g.ldx, row, Lay.key[row] - 1, r, Lay, gen + 1u, pre,
                         pre.valid);
      } else if (tid == 0 && g.lay.sync) {
        st_agent(g.lay.sync + kSyncFlag0 + row, gen + 1u);
      }
    }
    if (tid == 0) Lay.misc[0] = (int)gen;          // for the wait and the exit
    layer_retire(pre);
    if (!has_tile) {
      layer_exit(g.lay, Lay);
      return;
    }
    if (!early) prologue();
    const int row = min(m0 + e_row, M - 1);
    e_r = Lay.rk[row];
    e_slot = Lay.key[row] - 1;
    e_scb = __float_as_int(Lay.sc[row]);
  }
  // Every wave waits for all of its prologue loads (its stage, or its share
  // of each stage, and the metadata above) before the first barrier.
  vm_wait<0>();
  if constexpr (LORA != 0 && !LAYER) {
    if (e_own) {
      e_r = g.seg_rank[e_seg];
      e_slot = g.seg_slot[e_seg];
      e_scb = __float_as_int(g.seg_scale[e_seg]);
    }
  }
  if (ktail && KT == 1) {
    if constexpr (OWNED) {
      if (wid == 0) zero_tail_own(0, kg0);
    } else {
      zero_tail(0, kg0);
    }
  }
  lgkm_barrier();
  load_frags(0, smem, 0);
  for (int kt = 0; kt < KT; ++kt) {
    const unsigned char *st = smem + (kt % STAGES) * C::STAGE;
#pragma unroll
    for (int kk = 0; kk < KK - 1; ++kk) {
      load_frags((kk + 1) & 1, st, kk + 1);
      mfmas(kk & 1, kk & 1);
      interleave();
    }
    if (kt + 1 < KT) {
      // stage kt + 1 lands: with owners, the owners of its buffer wait for
      // their one stage in flight; otherwise it is the only stage in flight
      // and every wave waits for its share
      if constexpr (OWNED) {
        if (wid == (kt + 1) % STAGES) {
          vm_wait<0>();
          if (ktail && kt + 1 == KT - 1) zero_tail_own(wid, (kt + 1) * C::KSTEP + kg0);
        }
      } else {
        static_assert(STAGES == 2, "without owners only one stage may be in flight");
        vm_wait<0>();
        if (ktail && kt + 1 == KT - 1) zero_tail((kt + 1) % STAGES, (kt + 1) * C::KSTEP + kg0);
      }
      lgkm_barrier();
    }
    // Last sub-step: its MFMAs with the refill of stage kt's buffer, one DMA
    // instruction between MFMAs (a burst of DMAs would hold up the MFMAs),
    // then the first fragments of stage kt + 1.  The MFMAs and fragment
    // reads are unconditional so the accumulators see one straight-line
    // update (after the last stage the reads hit a settled buffer and their
    // values go unused).
    // In tiles of one K group a wave past the barrier takes issue priority
    // over the SIMD's other waves for its refill DMA and MFMAs, so the
    // stage refill starts as early as possible (measured 3% on the prefill
    // and 70B-shaped products; the two-group decode tiles gain nothing).
    if constexpr (KG == 1) __builtin_amdgcn_s_setprio(1);
    // the freed buffer kt % STAGES takes stage kt + STAGES (with owners, only
    // its owners issue, their whole slices)
    const bool refill = kt + STAGES < KT && (!OWNED || wid == kt % STAGES);
    const int k0n = (kt + STAGES) * C::KSTEP + kg0;
    // the stage reaching past K (at most one) is issued whole, ahead of the
    // MFMAs, so the interleaved loop below needs no per-instruction test
    const bool tailn = ktail && kt + STAGES == KT - 1;
    if constexpr (OWNED) {
      if (refill && tailn) {
#pragma unroll
        for (int q = 0; q < NIG; ++q) issue_own_one(q, kt % STAGES, k0n, true);
      }
    }
    const bool refill_fast = refill && (!OWNED || !tailn);
    constexpr int NIS = OWNED ? NIG : C::IPW;         // instructions per issuing wave
#pragma unroll
    for (int q = 0; q < C::FM * C::FN || q < NIS; ++q) {
      if (q < NIS && refill_fast) {
        if constexpr (OWNED)
          issue_own_one(q, kt % STAGES, k0n, false);
        else
          issue_one(q, kt % STAGES, k0n);
      }
      if (q < C::FM * C::FN) {
        const int i = q / C::FN, j = q % C::FN;
        constexpr int b = (KK - 1) & 1;
        if (DUAL && b)
          acc2[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[b][i], bfr[b][j], acc2[i][j], 0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[b][i], bfr[b][j], acc[i][j], 0, 0, 0);
      }
    }
    load_frags(KK & 1, smem + ((kt + 1) % STAGES) * C::STAGE, 0);
    if constexpr (KG == 1) __builtin_amdgcn_s_setprio(0);
  }
  if constexpr (DUAL) {
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] += acc2[i][j][v];
  }

  if constexpr (ROWEPI) {
    // Row epilogue.  The K groups' partial tiles go to LDS row-major (every
    // read of the ring and every DMA into it has finished: the last stage
    // was waited for in full and the barrier drains the reads); each thread
    // adds its row's 8 columns over the groups in group order.  A LoRA row
    // of rank r > 0 then gets s_a sum_k H[row][k] Bt_a[k][cols] in fp32
    // (k ascending, read in chunks of 8 rank rows; rows at or past r are
    // read inside the slot and skipped), the DoRA factor when the pool has
    // one, and one rounding; the 8 results leave in one 16-byte store.
    if constexpr (LAYER) layer_wait_rows<BM>(g.lay, g.X, g.ldx, m0, M, Lay);
    lgkm_barrier();
    float *red = reinterpret_cast<float *>(smem);
    constexpr int RS = BN + 4;
    static_assert(KG * BM * RS * 4 <= C::LDS, "row epilogue staging");
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          red[(kgrp * BM + wm * C::TM + i * 32 + acc_row(v, l)) * RS + wn * C::TN + j * 32 + (l & 31)] =
              acc[i][j][v];
    lgkm_barrier();
    float o[8];
    {
      const f32x4 p0 = *reinterpret_cast<const f32x4 *>(red + e_row * RS + e_c8);
      const f32x4 p1 = *reinterpret_cast<const f32x4 *>(red + e_row * RS + e_c8 + 4);
      o[0] = p0[0]; o[1] = p0[1]; o[2] = p0[2]; o[3] = p0[3];
      o[4] = p1[0]; o[5] = p1[1]; o[6] = p1[2]; o[7] = p1[3];
    }
#pragma unroll
    for (int gi = 1; gi < KG; ++gi) {
      const f32x4 p0 = *reinterpret_cast<const f32x4 *>(red + (gi * BM + e_row) * RS + e_c8);
      const f32x4 p1 = *reinterpret_cast<const f32x4 *>(red + (gi * BM + e_row) * RS + e_c8 + 4);
      o[0] += p0[0]; o[1] += p0[1]; o[2] += p0[2]; o[3] += p0[3];
      o[4] += p1[0]; o[5] += p1[1]; o[6] += p1[2]; o[7] += p1[3];
    }
    const int grow = m0 + e_row, gcol = n0 + e_c8;
    const bool live = grow < M && gcol < N;       // N % 8 == 0: all 8 columns or none
    if constexpr (WF8) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[e] *= e_ws0[e];
        o[4 + e] *= e_ws1[e];
      }
    }
    if constexpr (LORA != 0) {
      if (live && e_r > 0)
        lora_row8<DORA, LAYER>(g, grow, gcol, e_slot, e_r, __int_as_float(e_scb), o);
    }
    if (live) stg16(g.Y + (int64_t)grow * g.ldy + gcol, Elem<bf16_t>::pack(o));
    if constexpr (LAYER) layer_exit(g.lay, Lay);
    return;
  }

  if constexpr (KG > 1) {
    // groups 1.. hand their partial sums to group 0 through LDS (every
    // read of the ring and every DMA into it has finished: the last stage
    // was waited for in full and the barrier drains the reads); group 0
    // adds them in group order
    lgkm_barrier();
    float *red = reinterpret_cast<float *>(smem);
    auto slot_of = [&](int gi, int i, int j, int v4) {
      return (((gi * C::NWG + wid) * C::FM * C::FN + i * C::FN + j) * 4 + v4) * (kWave * 4) + l * 4;
    };
    if (kgrp > 0) {
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4)
            *reinterpret_cast<f32x4 *>(red + slot_of(kgrp - 1, i, j, v4)) =
                f32x4{acc[i][j][4 * v4], acc[i][j][4 * v4 + 1], acc[i][j][4 * v4 + 2],
                      acc[i][j][4 * v4 + 3]};
    }
    lgkm_barrier();
    if (kgrp == 0)
#pragma unroll
    for (int gi = 0; gi < KG - 1; ++gi)
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) {
            const f32x4 p = *reinterpret_cast<const f32x4 *>(red + slot_of(gi, i, j, v4));
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][4 * v4 + e] += p[e];
          }
  }

  if constexpr (WF8 && !ROWEPI) {
    // FP8 weight: the per-row weight scale of each accumulator column
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const float sw = g.wscale[min(n0 + wn * C::TN + j * 32 + (l & 31), N - 1)];
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] *= sw;
    }
  }

  if constexpr (LORA != 0 && !ROWEPI) {
    // LoRA increment, after the K loop, one distinct LoRA segment u of the
    // tile's rows at a time (ascending id).  The whole workgroup stages the
    // operands of the small product s_u H_u B_u^T in LDS, in the layout of
    // a K stage (rows of 128 bytes, same swizzle):
    //   A_hi, A_lo [BM][64]: s_u H[row][k] split into a bf16 high part and
    //                        a bf16 remainder (about 16 significant bits);
    //                        rows outside u and k >= r are zero
    //   Bs        [BN][64]: B_u[col][k], zero for k >= r
    // and group 0's waves add A_hi Bs^T + A_lo Bs^T into their
    // accumulators, KS = ceil(R/16) MFMA sub-steps each.  Rows outside u
    // add exact zeros, so base-only rows stay bit-identical to the plain
    // product.
    constexpr int RBL = 128;                          // bytes per staged row
    static_assert(3 * (BM > BN ? BM : BN) * RBL + 16 + 4 * BM <= SMEM, "LoRA staging");
    static_assert(C::T >= BM, "one tile row per thread");
    unsigned char *s_ahi = smem;
    unsigned char *s_alo = smem + BM * RBL;
    unsigned char *s_b = smem + 2 * BM * RBL;
    int *s_next = reinterpret_cast<int *>(smem + 2 * BM * RBL + BN * RBL);
    // DoRA: slot of each tile row (-1 = not rescaled), read by the store
    int *s_rowslot = reinterpret_cast<int *>(smem + 2 * BM * RBL + BN * RBL + 16);
    auto sw = [](int c, int r) { return ((c ^ ((r >> 1) & 7)) * 16); };
    // this thread's tile row (threads past BM take no row): its segment if
    // that has a LoRA term
    const int my_seg = (tid < BM && m0 + tid < M && e_r > 0) ? e_seg : -1;
    int *s_rr = reinterpret_cast<int *>(smem + EPI_META);   // per row: segment, later rank
    int *s_rslot = s_rr + BM;                               //          slot
    float *s_rsc = reinterpret_cast<float *>(s_rslot + BM); //          scale
    int *s_runs = reinterpret_cast<int *>(s_rsc + BM);
    // previous readers of LDS (the K loop, the partial sums) are done
    lgkm_barrier();
    // Runs of LoRA rows: a row of a LoRA segment that differs from the
    // previous row's starts one.  A tile of few long runs (prefill requests)
    // takes the staged MFMA increment below, one segment at a time; a tile of
    // many short runs (decode rows, each of its own adapter) would repeat
    // that for each of them, and instead finishes row by row on the VALU.
    if (tid == 0) *s_runs = 0;
    if (tid < BM) s_rr[tid] = my_seg;
    lgkm_barrier();
    {
      const bool start = tid < BM && my_seg >= 0 && (tid == 0 || s_rr[tid - 1] != my_seg);
      const uint64_t bal = __ballot(start);
      if (l == 0 && bal != 0) atomicAdd(s_runs, (int)__popcll(bal));
    }
    lgkm_barrier();
    if (__builtin_amdgcn_readfirstlane(*s_runs) > LORA_GEMM_STAGED_RUNS) {
      // Row epilogue of a large tile, wave by wave: each wave puts one
      // 32-row fragment row of its accumulators (32 rows x TN columns) in its
      // own LDS slot, and its lanes take the (row, 8 columns) items of it,
      // TN / 8 lanes per row: lora_row8 (or lora_row8_pair, same bits) with
      // the row's own adapter, the rounding and one 16-byte store.  A
      // fragment's registers are free once it is in LDS; no workgroup
      // barrier is needed.
      if (tid < BM) {
        s_rr[tid] = my_seg >= 0 ? e_r : 0;
        s_rslot[tid] = my_seg >= 0 ? e_slot : 0;
        s_rsc[tid] = my_seg >= 0 ? __int_as_float(e_scb) : 0.f;
      }
      lgkm_barrier();                                 // the row metadata is visible
      constexpr int WRS = C::TN + 4;                  // row stride of a wave's slot
      constexpr int LPR = C::TN / 8;                  // lanes per row
      constexpr int WITEMS = 32 * LPR;                // items per fragment row
      static_assert(WITEMS % (2 * kWave) == 0, "whole steps of one or two items per lane");
      float *wbuf = reinterpret_cast<float *>(smem) + wid * 32 * WRS;
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        // the previous fragment's reads have landed before the slot is rewritten
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) wbuf[acc_row(v, l) * WRS + j * 32 + (l & 31)] = acc[i][j][v];
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // visible to the wave's lanes
        // two items at a time on tiles of at most four fragments per wave; on
        // 192x256 and 256x256 tiles the second item's registers would spill
        const bool PAIR = C::FM * C::FN <= 4;
        const int NU = PAIR ? 2 : 1;
        for (int it0 = l; it0 < WITEMS; it0 += NU * kWave) {
          int grow[2], gcol[2], slot[2], r[2];
          float sc[2], o[2][8];
          bool live[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            if (u >= NU) break;
            const int it = it0 + u * kWave;
            const int rf = it / LPR, c8 = (it % LPR) * 8;
            const int row = wm * C::TM + i * 32 + rf;
            live[u] = m0 + row < M && n0 + wn * C::TN + c8 < N;
            // dead items read a row and columns in bounds and add nothing
            grow[u] = min(m0 + row, M - 1);
            gcol[u] = min(n0 + wn * C::TN + c8, N - 8);
            const f32x4 p0 = *reinterpret_cast<const f32x4 *>(wbuf + rf * WRS + c8);
            const f32x4 p1 = *reinterpret_cast<const f32x4 *>(wbuf + rf * WRS + c8 + 4);
            o[u][0] = p0[0]; o[u][1] = p0[1]; o[u][2] = p0[2]; o[u][3] = p0[3];
            o[u][4] = p1[0]; o[u][5] = p1[1]; o[u][6] = p1[2]; o[u][7] = p1[3];
            r[u] = live[u] ? s_rr[row] : 0;
            slot[u] = s_rslot[row];
            sc[u] = s_rsc[row];
          }
          if (PAIR) {
            lora_row8_pair<DORA>(g, grow, gcol, slot, r, sc, o);
          } else {
            if (r[0] > 0) lora_row8<DORA>(g, grow[0], gcol[0], slot[0], r[0], sc[0], o[0]);
          }
#pragma unroll
          for (int u = 0; u < 2; ++u)
            if (u < NU && live[u]) stg16(g.Y + (int64_t)grow[u] * g.ldy + gcol[u], Elem<bf16_t>::pack(o[u]));
        }
      }
      return;
    }
    if constexpr (DORA) {
      if (tid < BM) s_rowslot[tid] = my_seg >= 0 ? e_slot : -1;
    }
    int prev = -1;
    while (true) {
      // next segment id above prev among the tile's rows: wave minimum,
      // then a workgroup minimum through one LDS word
      int cand = (my_seg > prev) ? my_seg : INT_MAX;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) cand = min(cand, __shfl_xor(cand, off));
      if (tid == 0) *s_next = INT_MAX;
      lgkm_barrier();
      if (l == 0 && cand != INT_MAX) atomicMin(s_next, cand);
      lgkm_barrier();
      const int u = __builtin_amdgcn_readfirstlane(*s_next);
      if (u == INT_MAX) break;
      prev = u;
      // u's slot, rank and scale from the rows of u (all write the same)
      if (my_seg == u) {
        s_next[1] = e_slot;
        s_next[2] = e_r;
        s_next[3] = e_scb;
      }
      lgkm_barrier();
      const int slot = __builtin_amdgcn_readfirstlane(s_next[1]);
      const int r = __builtin_amdgcn_readfirstlane(s_next[2]);
      const float sc = __int_as_float(__builtin_amdgcn_readfirstlane(s_next[3]));
      const int rs = g.proj.rs;
      const int R = rank_bucket(r, g.policy, rs);
      const int KS = (R + 15) / 16;
      const int NC = 2 * KS;                          // 16-byte chunks per staged row
      // one pass per projection among the tile's columns (one unless the
      // pool stacks projections and the tile straddles two): projection q's
      // rank rows start at qoff, and columns outside it stage zeros
      const int q_lo = proj_of(g.proj, n0), q_hi = proj_of(g.proj, min(n0 + BN, N) - 1);
      for (int q = q_lo; q <= q_hi; ++q) {
      const int qoff = q * rs;
      const int c_lo = g.proj.col_off[q], c_hi = g.proj.col_off[q + 1];
      // A: (row, chunk) items, at most JA per thread, then B likewise: each
      // operand's loads are all issued before its first LDS store (both at
      // once would spill on 256x256 tiles).  Loads are unconditional (rows
      // past M and chunks past rs read in bounds) and masked where used; a
      // row is in u by the tile's row -> segment table.
      constexpr int JA = (BM * 8 + C::T - 1) / C::T;
      float4 ha[JA], hb[JA];
#pragma unroll
      for (int j = 0; j < JA; ++j) {
        const int it = min(tid + j * C::T, BM * NC - 1);
        const int row = it / NC, c = it - (it / NC) * NC;
        const float *hp = g.H + (int64_t)min(m0 + row, M - 1) * g.r_max + qoff + min(c * 8, rs - 8);
        ha[j] = *reinterpret_cast<const float4 *>(hp);
        hb[j] = *reinterpret_cast<const float4 *>(hp + 4);
      }
#pragma unroll
      for (int j = 0; j < JA; ++j) {
        const int it = tid + j * C::T;
        if (it >= BM * NC) break;
        const int row = it / NC, c = it - (it / NC) * NC;
        // chunks past rs (k >= R >= r, only when rs = 8) stay zero
        const bool in_u = s_rr[row] == u && c * 8 < rs;
        const float h[8] = {ha[j].x, ha[j].y, ha[j].z, ha[j].w, hb[j].x, hb[j].y, hb[j].z, hb[j].w};
        u32x4 phi, plo;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const int k = c * 8 + e2 * 2;
          const float v0 = (in_u && k < r) ? sc * h[e2 * 2] : 0.f;
          const float v1 = (in_u && k + 1 < r) ? sc * h[e2 * 2 + 1] : 0.f;
          const uint32_t hw = pack_bf16x2(v0, v1);
          phi[e2] = hw;
          plo[e2] = pack_bf16x2(v0 - bf16_lo(hw), v1 - bf16_hi(hw));
        }
        *reinterpret_cast<u32x4 *>(s_ahi + row * RBL + sw(c, row)) = phi;
        *reinterpret_cast<u32x4 *>(s_alo + row * RBL + sw(c, row)) = plo;
      }
      // B: rank values of column col, k in chunk c, zero for k >= r
      constexpr int JB = (BN * 8 + C::T - 1) / C::T;
      u32x4 bv[JB];
      if constexpr (LORA == 2) {
        const bf16_t *bn = g.Bn + (int64_t)slot * N * rs;
#pragma unroll
        for (int j = 0; j < JB; ++j) {
          const int it = min(tid + j * C::T, BN * NC - 1);
          const int col = it / NC, c = it - (it / NC) * NC;
          const int colc = min(n0 + col, N - 1);     // columns past N: never stored
          // a chunk past rs (only when rs = 8) is read from the block's
          // first chunk and masked below
          bv[j] = *reinterpret_cast<const u32x4 *>(bn + (int64_t)colc * rs + min(c * 8, rs - 8));
        }
      }
      if constexpr (LORA == 2) {
#pragma unroll
        for (int j = 0; j < JB; ++j) {
          const int it = tid + j * C::T;
          if (it >= BN * NC) break;
          const int col = it / NC, c = it - (it / NC) * NC;
          const int colc = min(n0 + col, N - 1);
          const bool in_q = colc >= c_lo && colc < c_hi;
          u32x4 v = bv[j];
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            const int k = c * 8 + e2 * 2;
            v[e2] &= in_q ? ((k < r ? 0x0000ffffu : 0u) | (k + 1 < r ? 0xffff0000u : 0u)) : 0u;
          }
          *reinterpret_cast<u32x4 *>(s_b + col * RBL + sw(c, col)) = v;
        }
      } else {
        // from the rank-major Bt: 8 columns of one rank row per item,
        // transposed into the column rows with 2-byte stores
        const bf16_t *bt = g.Bt + (int64_t)slot * rs * N;
        constexpr int CC = BN / 8;
        for (int it = tid; it < 8 * NC * CC; it += C::T) {
          const int k = it / CC, cc = it - (it / CC) * CC;
          const int col0 = n0 + cc * 8;
          u32x4 v = u32x4{0, 0, 0, 0};
          if (k < r && col0 >= c_lo && col0 < c_hi)
            v = *reinterpret_cast<const u32x4 *>(bt + (int64_t)k * N + min(col0, N - 8));
          const int c = k >> 3, kin = k & 7;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int col = cc * 8 + e;
            const uint16_t hv = (uint16_t)(e & 1 ? (v[e >> 1] >> 16) : (v[e >> 1] & 0xffffu));
            *reinterpret_cast<uint16_t *>(s_b + col * RBL + sw(c, col) + kin * 2) = hv;
          }
        }
      }
      lgkm_barrier();
      if (kgrp == 0) {
        int ar[C::FM], br[C::FN];
#pragma unroll
        for (int i = 0; i < C::FM; ++i) ar[i] = (wm * C::TM + i * 32 + (l & 31)) * RBL;
#pragma unroll
        for (int j = 0; j < C::FN; ++j) br[j] = (wn * C::TN + j * 32 + (l & 31)) * RBL;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          if (kk < KS) {
            const int co = sw(kk * 2 + (l >> 5), l & 31);
            mfma_bf16x8 bv[C::FN];
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
              bv[j] = as_bf16x8(*reinterpret_cast<const u32x4 *>(s_b + br[j] + co));
#pragma unroll
            for (int i = 0; i < C::FM; ++i) {
              const mfma_bf16x8 ah = as_bf16x8(*reinterpret_cast<const u32x4 *>(s_ahi + ar[i] + co));
              const mfma_bf16x8 al = as_bf16x8(*reinterpret_cast<const u32x4 *>(s_alo + ar[i] + co));
#pragma unroll
              for (int j = 0; j < C::FN; ++j) {
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bv[j], acc[i][j], 0, 0, 0);
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bv[j], acc[i][j], 0, 0, 0);
              }
            }
          }
        }
      }
      // the staging area is rewritten for the next projection or segment
      lgkm_barrier();
      }
    }
  }

  if (KG > 1 && kgrp > 0) return;

  // DoRA: rows of rank > 0 are multiplied by g[slot][col]; the tile's
  // row -> slot table (-1 = not rescaled) was written before the segment
  // loop, whose barriers order it before these reads.  Rows without a
  // factor read slot 0's in bounds and multiply by 1.  One fragment row
  // block at a time, so the factors of only one block are live.
  if constexpr (DORA) {
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
      int rs[16];
      const int *s_rowslot = reinterpret_cast<const int *>(smem + 2 * BM * 128 + BN * 128 + 16);
#pragma unroll
      for (int v = 0; v < 16; ++v) rs[v] = s_rowslot[wm * C::TM + i * 32 + acc_row(v, l)];
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const int colc = min(n0 + wn * C::TN + j * 32 + (l & 31), N - 1);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float f = g.dora[(int64_t)max(rs[v], 0) * N + colc];
          acc[i][j][v] *= rs[v] >= 0 ? f : 1.f;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Store: bf16 round to nearest even, once.  A lane holds one column of
  // each 32x32 fragment, so the rounded tile goes through LDS row-major
  // (RCH rows per pass, rows padded by 8 elements) and leaves as 16-byte
  // row segments: an eighth of the store instructions of storing the
  // fragments' 2-byte elements directly (measured: those took about 5% of
  // the prefill product).
  constexpr int RSB = BN + 8;                         // bf16 elements per staged row
  constexpr int RCH = (BM * RSB * 2 <= SMEM) ? BM : BM / 2;
  static_assert(RCH * RSB * 2 <= SMEM && RCH % C::TM == 0, "store staging");
  constexpr int CPR = BN / 8;                         // 16-byte segments per row
  uint16_t *s16 = reinterpret_cast<uint16_t *>(smem);
  lgkm_barrier();                                     // every LDS read above is done
#pragma unroll
  for (int p0 = 0; p0 < BM; p0 += RCH) {
    if (wm * C::TM >= p0 && wm * C::TM < p0 + RCH) {
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            s16[(wm * C::TM - p0 + i * 32 + acc_row(v, l)) * RSB + wn * C::TN + j * 32 + (l & 31)] =
                f32_to_bf16_rne(acc[i][j][v]);
    }
    lgkm_barrier();
#pragma unroll
    for (int q = tid; q < RCH * CPR; q += C::T) {
      const int r = q / CPR, c8 = (q % CPR) * 8;
      const int row = m0 + p0 + r, col = n0 + c8;    // N % 8 == 0: all 8 columns or none
      if (row < M && col < N)
        stg16(g.Y + (int64_t)row * g.ldy + col, *reinterpret_cast<const uint4 *>(s16 + r * RSB + c8));
    }
    if (p0 + RCH < BM) lgkm_barrier();               // the next pass rewrites the rows
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
  const float *dora;
  ProjView proj;
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
        const float *bt = g.Bt + (int64_t)g.seg_slot[s] * g.proj.rs * g.N;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = n0 + tx * 4 + j;
          if (col >= g.N) continue;
          const int qoff = proj_of(g.proj, col) * g.proj.rs;
          float d = 0.f;
          for (int k = 0; k < r; ++k)
            d = fmaf(hrow[qoff + k], bt[(int64_t)k * g.N + col], d);
          acc[i][j] += sc * d;
          if (g.dora) acc[i][j] *= g.dora[(int64_t)g.seg_slot[s] * g.N + col];
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

template <int BM, int BN, int WM, int WN, int BK, int STAGES, int KG, bool WF8>
hipError_t launch_bf16_w(const GemmArgs &g, bool lora, hipStream_t stream) {
  dim3 grid(tile_grid((g.M + BM - 1) / BM, (g.N + BN - 1) / BN));
  dim3 block(WM * WN * KG * kWave);
  const bool dora = lora && g.dora;
  if (lora && g.Bn && dora)
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, BK, STAGES, KG, 2, true, WF8>), grid,
                       block, 0, stream, g);
  else if (lora && g.Bn)
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, BK, STAGES, KG, 2, false, WF8>), grid,
                       block, 0, stream, g);
  else if (lora && dora)
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, BK, STAGES, KG, 1, true, WF8>), grid,
                       block, 0, stream, g);
  else if (lora)
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, BK, STAGES, KG, 1, false, WF8>), grid,
                       block, 0, stream, g);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, BK, STAGES, KG, 0, false, WF8>), grid,
                       block, 0, stream, g);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int BK, int STAGES, int KG>
hipError_t launch_bf16(const GemmArgs &g, bool lora, hipStream_t stream) {
  return launch_bf16_w<BM, BN, WM, WN, BK, STAGES, KG, false>(g, lora, stream);
}
template <int BM, int BN, int WM, int WN, int BK, int STAGES, int KG>
hipError_t launch_fp8w(const GemmArgs &g, bool lora, hipStream_t stream) {
  return launch_bf16_w<BM, BN, WM, WN, BK, STAGES, KG, true>(g, lora, stream);
}

// The one-launch layer on small tiles: one workgroup per tile, and at least
// one per row (workgroups past the tiles only do their row).
template <bool WF8, int BM, int BN, int WM, int WN, int BK, int STAGES, int KG>
hipError_t launch_layer_t(const GemmArgs &g, hipStream_t stream) {
  const int tiles = tile_grid((g.M + BM - 1) / BM, (g.N + BN - 1) / BN);
  dim3 grid(tiles > g.M ? tiles : g.M);
  dim3 block(WM * WN * KG * kWave);
  if (g.dora)
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, BK, STAGES, KG, 1, true, WF8, true>),
                       grid, block, 0, stream, g);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, BK, STAGES, KG, 1, false, WF8, true>),
                       grid, block, 0, stream, g);
  return hipGetLastError();
}

// Rows that go to the large tiles when the batch is split (0: no split).
int tail_split_rows(int M, int N) {
  if (!LORA_GEMM_TAIL_SPLIT || M <= LORA_GEMM_SMALL_M) return 0;
  const int64_t tn = (N + 255) / 256, tm = (M + 255) / 256;
  const int64_t tiles = tm * tn;
  if (tm * tn <= LORA_GEMM_MID_TILES || tiles % kCUs == 0 || tiles < kCUs) return 0;
  const int64_t a = tiles / kCUs * kCUs / tn;   // 256-row M-tiles inside the whole rounds
  const int64_t M2 = M - a * 256;
  if (a < 1 || M2 <= 0 || M2 > LORA_GEMM_SMALL_M) return 0;
  const int64_t small_tiles = (M2 + 63) / 64 * ((N + 63) / 64);
  return small_tiles <= LORA_GEMM_TAIL_TILES ? (int)(a * 256) : 0;
}

// Tile configuration for a batch of g.M rows, and the launch.
hipError_t launch_bf16_rows(const GemmArgs &g, bool lora, hipStream_t stream) {
  const int M = g.M, N = g.N;
  const bool mid = ((int64_t)(M + 255) / 256) * ((N + 255) / 256) <= LORA_GEMM_MID_TILES;
  // Large tiles: 256 x 256, or 192 x 256 when its rounds of kCUs tiles cost
  // less (rounds times tile area, the narrower tile charged its extra LDS
  // traffic per flop).
  const int64_t tn256 = (N + 255) / 256;
  const int64_t r256 = ((int64_t)(M + 255) / 256 * tn256 + kCUs - 1) / kCUs;
  const int64_t r192 = ((int64_t)(M + 191) / 192 * tn256 + kCUs - 1) / kCUs;
  const bool use192 = r192 * 192 * LORA_GEMM_192_COST < r256 * 256 * 100;
  if (g.wscale) {
    if (M <= LORA_GEMM_SMALL_M) return launch_fp8w<LORA_GEMM_SMALL_F8>(g, lora, stream);
    if (mid) return launch_fp8w<LORA_GEMM_MID_F8>(g, lora, stream);
    if (use192) return launch_fp8w<LORA_GEMM_LARGE192_F8>(g, lora, stream);
    return launch_fp8w<LORA_GEMM_LARGE_F8>(g, lora, stream);
  }
  if (M <= LORA_GEMM_SMALL_M) {
    using S = TileCfg<LORA_GEMM_SMALL>;
    const int64_t tiles = (int64_t)((M + S::kBM - 1) / S::kBM) * ((N + S::kBN - 1) / S::kBN);
    if (tiles > kCUs) return launch_bf16<LORA_GEMM_SMALL_WIDE>(g, lora, stream);
    return launch_bf16<LORA_GEMM_SMALL>(g, lora, stream);
  }
  if (mid) return launch_bf16<LORA_GEMM_MID>(g, lora, stream);
  if (use192) return launch_bf16<LORA_GEMM_LARGE192>(g, lora, stream);
  return launch_bf16<LORA_GEMM_LARGE>(g, lora, stream);
}

}  // namespace

hipError_t launch_gemm(const void *X, int64_t ldx, const void *W, int64_t ldw, void *Y,
                       int64_t ldy, int M, int K, int N, int dtype, const float *H,
                       const SegView *seg, const PoolView *pool, hipStream_t stream,
                       const float *wscale) {
  const bool lora = seg != nullptr;
  if (dtype == 1) {
    GemmArgs g{(const bf16_t *)X, ldx, (const bf16_t *)W, ldw, (bf16_t *)Y, ldy, M, K, N,
               H, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 0, nullptr, wscale};
    g.proj.n_proj = 1;
    g.proj.rs = 64;
    for (int q = 0; q <= kMaxProj; ++q) g.proj.col_off[q] = q ? N : 0;
    if (lora) {
      g.proj = pool->proj;
      g.Bt = (const bf16_t *)pool->Bt;
      g.Bn = (const bf16_t *)pool->B;
      g.dora = pool->dora;
      g.row_segment = seg->row_segment;
      g.seg_slot = seg->seg_slot;
      g.seg_rank = seg->seg_rank;
      g.seg_scale = seg->seg_scale;
      g.r_max = pool->r_max;
      g.policy = pool->policy;
    }
    const int M1 = tail_split_rows(M, N);
    if (M1 > 0) {
      // rows [0, M1) on the large tiles, rows [M1, M) on the small ones
      GemmArgs g2 = g;
      g.M = M1;
      g2.M = M - M1;
      g2.X += (int64_t)M1 * ldx;
      g2.Y += (int64_t)M1 * ldy;
      if (lora) {
        g2.row_segment += M1;
        g2.H += (int64_t)M1 * g.r_max;
      }
      const hipError_t e = launch_bf16_rows(g, lora, stream);
      if (e != hipSuccess) return e;
      return launch_bf16_rows(g2, lora, stream);
    }
    return launch_bf16_rows(g, lora, stream);
  }
  GemmF32Args g{(const float *)X, ldx, (const float *)W, ldw, (float *)Y, ldy, M, K, N,
                H, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr};
  g.proj.n_proj = 1;
  g.proj.rs = 64;
  for (int q = 0; q <= kMaxProj; ++q) g.proj.col_off[q] = q ? N : 0;
  if (lora) {
    g.proj = pool->proj;
    g.Bt = (const float *)pool->Bt;
    g.dora = pool->dora;
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

hipError_t launch_layer(const void *X, int64_t ldx, const void *W, int64_t ldw, void *Y,
                        int64_t ldy, int M, const PoolView &pool, const LayerArgs &lay,
                        hipStream_t stream, const float *wscale) {
  if (pool.dtype != 1 || M < 1 || M > kLayerMaxRows) return hipErrorNotSupported;
  const int K = pool.d_in, N = pool.d_out;
  GemmArgs g{(const bf16_t *)X, ldx, (const bf16_t *)W, ldw, (bf16_t *)Y, ldy, M, K, N,
             lay.H, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 0, nullptr, nullptr};
  g.wscale = wscale;
  g.proj = pool.proj;
  g.Bt = (const bf16_t *)pool.Bt;
  g.Bn = (const bf16_t *)pool.B;
  g.dora = pool.dora;
  g.r_max = pool.r_max;
  g.policy = pool.policy;
  g.lay = lay;
  using S = TileCfg<LORA_GEMM_SMALL>;
  const int64_t tiles = (int64_t)((M + S::kBM - 1) / S::kBM) * ((N + S::kBN - 1) / S::kBN);
  // FP8 weights: the four-stage ring only (the two-stage ring of codes is
  // too small to hold a large pool's build tables)
  if (wscale) return launch_layer_t<true, LORA_GEMM_SMALL_F8>(g, stream);
  if (tiles > kCUs) return launch_layer_t<false, LORA_GEMM_SMALL_WIDE>(g, stream);
  return launch_layer_t<false, LORA_GEMM_SMALL>(g, stream);
}

}  // namespace lora
