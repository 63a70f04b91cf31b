// The whole layer in one launch for decode-sized batches: segment metadata,
// shrink, base product and LoRA epilogue (adapter-batching page, Multi-LoRA
// Serving, sections "一个混合 Batch 的数学形式" and "Segmented Kernel 需要哪些
// Metadata"; its section "Prefill 与 Decode 的 LoRA 形状不同" puts the cost of
// decode in launches, gathers and metadata rather than in arithmetic).
//
// Every workgroup of the launch is a tile of the small-batch GEMM (8 waves,
// 512 threads).  Before its K loop it
//   1. builds the batch's whole segment metadata in LDS from the per-row
//      slot ids (n <= 512 rows: one row per thread, per-slot first row and
//      count by LDS atomics in tables that live in the stage ring before
//      it is filled, two block scans), and writes the part of it that
//      belongs to row blockIdx.x -- every output word is written by exactly
//      one workgroup, with the values a single-workgroup build gives;
//   2. computes H for row blockIdx.x (X row against its slot's rank rows)
//      and publishes it: the H entries with agent-scope stores, then a
//      per-row flag holding this launch's generation number.
// After its K loop it needs H for the LoRA rows of its tile, which other
// workgroups produced: it reads their flags (agent-scope loads, so no L2 of
// another XCD can hold a stale copy), waits a bounded time for any that are
// not yet set, and computes the rows still missing itself (the same sums,
// so the same bits).  No workgroup ever waits for one that may not be
// running, so every schedule finishes.  H values are read back with
// agent-scope loads too.  Cross-XCD ordering uses only per-access scope
// and s_waitcnt, never a whole-L2 write-back or invalidate.
//
// The sync buffer (caller-owned, zero-filled once) holds the generation
// number, an exit counter and one flag per row.  The last workgroup to
// finish resets the counter and advances the generation, so flags from an
// earlier call never match; calls that share a buffer must therefore run
// in stream order.  Without a sync buffer every tile computes its own
// rows' H (no hand-off at all).
#pragma once

#include <climits>

#include "lora_device.cuh"
#include "lora_kernels.h"
#include "shrink_rows.cuh"

namespace lora {

constexpr int kLayerMaxRows = 512;    // rows of a one-launch batch (one per thread)
constexpr int kLayerThreads = 512;    // threads of the small tiles' workgroup
constexpr int kLayerWaves = kLayerThreads / kWave;
constexpr int kSyncGen = 0;           // sync word: generation of the last finished call
constexpr int kSyncExit = 1;          // sync word: workgroups of this call that finished
constexpr int kSyncFlag0 = 64;        // sync word of row 0's flag
constexpr int kLayerRankBlk = 16;     // rank rows per pass of the row shrink
constexpr int kLayerSpin = 256;       // flag polls before a tile computes a row itself
constexpr int kLayerTabSlots = 255;   // pools up to this size keep the build's tables here

static_assert(kLayerMaxRows == kLayerThreads, "one row per thread in the build");

// LDS of the build's tables: 4 n_slots + 2 ints.
__host__ __device__ constexpr int layer_tab_ints(int n_slots) { return 4 * n_slots + 2; }

// LDS of the layer's workgroup-wide work (beside the GEMM's stage ring).
struct LayerLds {
  int key[kLayerMaxRows];     // row -> validated slot + 1, 0 = base-only, -1 past n
  int rk[kLayerMaxRows];      // row -> rank of its slot (0: base-only or demoted)
  float sc[kLayerMaxRows];    // row -> scale of its slot
  int wsum[kLayerWaves][4];
  float red[kLayerWaves][kLayerRankBlk];
  int misc[8];                // [0] generation, [1..2] pending rows mask, [3..4] segment of mine
  int tab[layer_tab_ints(kLayerTabSlots)];   // the build's tables for pools of <= kLayerTabSlots
};

// Agent-scope relaxed accesses: on gfx950 these bypass the non-coherent
// caches, so a value stored on one XCD is seen by a load on another.
__device__ __forceinline__ uint32_t ld_agent(const uint32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint32_t *p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Inclusive scan of v over the 64 lanes.
__device__ __forceinline__ int wave_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int u = __shfl_up(v, d);
    if (lane >= d) v += u;
  }
  return v;
}

// Operands of the first pass of a row's shrink (projection 0, rank rows
// 0..15, d_in chunk tid), requested before the metadata build so that they
// arrive during it.
struct RowPrefetch {
  uint4 x;
  uint4 a[kLayerRankBlk];
  bool valid;
};

// Request the first-pass operands of row `row` (< n) of slot `slot`: the X
// chunk and 16 rank rows of the slot (rows past rs - 1 clamped into the
// slot; their sums are dropped).  A slot id out of range reads slot 0 and
// marks the operands unusable.  No branch around the loads, so that the
// compiler's waits for earlier loads never have to cover these.
__device__ __forceinline__ void layer_prefetch(const LayerArgs &a, const bf16_t *X, int64_t ldx,
                                               int row, int slot_in, RowPrefetch &p) {
  p.valid = slot_in >= 0 && slot_in < a.n_slots;
  const int slot = p.valid ? slot_in : 0;
  const int c = threadIdx.x * 8;
  const int cc = c < a.d_in ? c : a.d_in - 8;
  p.x = ldg16(X + (int64_t)row * ldx + cc);
  const bf16_t *ab = static_cast<const bf16_t *>(a.A) + (int64_t)slot * a.r_max * a.d_in + cc;
#pragma unroll
  for (int j = 0; j < kLayerRankBlk; ++j) p.a[j] = ldg16(ab + (int64_t)min(j, a.rs - 1) * a.d_in);
}

// The prefetched registers are read here on every path, so the compiler
// waits for their loads once, before the K loop, instead of inside it where
// the registers are reused (a row of rank 0 never consumes them).
__device__ __forceinline__ void layer_retire(const RowPrefetch &p) {
  asm volatile("" ::"v"(p.x.x), "v"(p.x.y), "v"(p.x.z), "v"(p.x.w));
#pragma unroll
  for (int j = 0; j < kLayerRankBlk; ++j)
    asm volatile("" ::"v"(p.a[j].x), "v"(p.a[j].y), "v"(p.a[j].z), "v"(p.a[j].w));
}

// Step 1a: the build's global loads, in one round trip and with no branch
// around them inside a wave (indices clamped in bounds, values selected
// afterwards): the row's slot id, a share of the slot rank and scale tables
// (slot k by thread k % 512) and workgroup row `mine`'s slot id.
constexpr int kLayerSlotsPerThread = 4096 / kLayerThreads;
struct BuildRegs {
  int slot, slot_mine;
  int rank[kLayerSlotsPerThread];
  float scale[kLayerSlotsPerThread];
};

__device__ __forceinline__ void layer_build_load(const LayerArgs &a, int n, int mine,
                                                 BuildRegs &b) {
  const int i = threadIdx.x;
  const int s = a.row_slot[min(i, n - 1)];
  b.slot = i < n ? s : -1;
  b.slot_mine = a.row_slot[min(mine, n - 1)];
#pragma unroll
  for (int u = 0; u < kLayerSlotsPerThread; ++u) {
    b.rank[u] = 0;
    b.scale[u] = 0.f;
    if (u * kLayerThreads < a.n_slots) {            // uniform: skips whole passes only
      const int kc = min(u * kLayerThreads + i, a.n_slots - 1);
      b.rank[u] = a.slot_rank[kc];
      b.scale[u] = a.slot_scale[kc];
    }
  }
}

// Step 1b: the slot tables to LDS (`tab`), the per-key tables cleared.
// Waits for the loads of step 1a, which were requested before the row's
// shrink operands.
__device__ __forceinline__ void layer_stage(const LayerArgs &a, const BuildRegs &b, int *tab) {
  const int i = threadIdx.x;
  const int K = a.n_slots + 1;
  int *T = tab, *C = tab + K, *R = tab + 2 * K;
  float *Sc = reinterpret_cast<float *>(R + a.n_slots);
#pragma unroll
  for (int u = 0; u < kLayerSlotsPerThread; ++u) {
    const int k = u * kLayerThreads + i;
    if (k < a.n_slots) {
      R[k] = b.rank[u];
      Sc[k] = b.scale[u];
    }
  }
  for (int k = i; k < K; k += kLayerThreads) {
    T[k] = INT_MAX;
    C[k] = 0;
  }
}

// Step 1c: the segment metadata of rows [0, n) and row `mine`'s part of the
// outputs (nothing for mine >= n).  Validation and every output value as
// the segment build defines them: key 0 (base-only segment) for slot -1 and
// for a bad slot or rank (counted in status); segments in order of their
// first row; rows ascending inside a segment.  The slot tables go to LDS;
// per key, the first row (atomic minimum) and the row count (atomic add)
// go to LDS tables too, and both commute, so the tables do not depend on
// the order in which the atomics land.  Segment ids and offsets are block
// scans over the rows; row mine's position inside its segment counts the
// earlier rows of its key.  `tab` holds 4 n_slots + 2 ints (the stage ring
// before it is filled), staged by step 1b.  Reads no global memory.  Puts
// the per-row key, rank and scale in L.  Ends with a barrier.
__device__ __forceinline__ void layer_build(const LayerArgs &a, int n, int mine,
                                            const BuildRegs &b, LayerLds &L, int *tab) {
  const int i = threadIdx.x, lane = i & (kWave - 1), wave = i / kWave;
  const int K = a.n_slots + 1;
  int *T = tab, *C = tab + K, *R = tab + 2 * K;
  float *Sc = reinterpret_cast<float *>(R + a.n_slots);
  __syncthreads();                                   // slot tables staged
  const int slot = b.slot;
  bool bad = false;
  int key = 0, r = 0;
  float sc = 0.f;
  if (i < n && slot != -1) {
    if (slot < -1 || slot >= a.n_slots) {
      bad = true;
    } else {
      r = R[slot];
      sc = Sc[slot];
      if (r < 0 || r > a.rank_bound) {
        bad = true;
        r = 0;
      } else {
        key = slot + 1;
      }
    }
  }
  L.key[i] = i < n ? key : -1;
  L.rk[i] = r;
  L.sc[i] = sc;
  if (i < n) {
    atomicMin(&T[key], i);
    atomicAdd(&C[key], 1);
  }
  __syncthreads();
  const int kmine = mine < n ? L.key[mine] : -2;
  const int first = i < n ? T[key] : -1;
  const bool head = first == i;
  // exclusive scans over rows of (head) and (head ? rows of its key : 0);
  // totals of bad rows and of rows before `mine` on its key
  const int h = head ? 1 : 0, c = head ? C[key] : 0;
  const int hi = wave_scan(h, lane), ci = wave_scan(c, lane);
  const uint64_t badm = __ballot(bad);
  const uint64_t befm = __ballot(i < n && i < mine && key == kmine);
  if (lane == kWave - 1) {
    L.wsum[wave][0] = hi;
    L.wsum[wave][1] = ci;
    L.wsum[wave][2] = __popcll(badm);
    L.wsum[wave][3] = __popcll(befm);
  }
  __syncthreads();
  int hb = 0, cb = 0, S = 0, nbad = 0, pos = 0;
#pragma unroll
  for (int w = 0; w < kLayerWaves; ++w) {
    hb += w < wave ? L.wsum[w][0] : 0;
    cb += w < wave ? L.wsum[w][1] : 0;
    S += L.wsum[w][0];
    nbad += L.wsum[w][2];
    pos += L.wsum[w][3];
  }
  // the head row of mine's key publishes its segment id and offset
  const int fmine = mine < n ? T[kmine] : -1;
  if (i == fmine) {
    L.misc[3] = hb + hi - h;
    L.misc[4] = cb + ci - c;
  }
  __syncthreads();
  if (i == mine && i < n) {
    const int seg = L.misc[3], off = L.misc[4];
    a.token_indices[off + pos] = i;
    a.row_segment[i] = seg;
    if (head) {
      a.seg_off[seg] = off;
      a.seg_slot[seg] = key - 1;
      a.seg_rank[seg] = key ? r : 0;
      a.seg_scale[seg] = r > 0 ? sc : 0.0f;
    }
  }
  if (mine == 0 && i == 0) {
    a.seg_off[S] = n;
    *a.num_segments = S;
    *a.status = nbad;
  }
  __syncthreads();                                   // the tables' LDS is free again
}

// H[row][q rs + k] = X[row] . A[slot][q rs + k] for k < r and every
// projection q, by the whole workgroup; then, with a sync buffer, the row's
// flag set to flag_val.  Thread t takes the 16-byte chunks t, t + 512, ...
// of d_in (d_in % 8 == 0); per pass of 16 rank rows each thread keeps 16
// partial sums (chunks ascending), then a halving butterfly over the lanes
// and the waves in order.  Rank rows past r re-read row r - 1 (inside the
// slot) and are dropped.  With use_pre, `pre` holds the first pass's
// operands.  Called by every thread; contains barriers.
__device__ __forceinline__ void layer_row_shrink(const LayerArgs &a, const bf16_t *X, int64_t ldx,
                                                 int row, int slot, int r, LayerLds &L,
                                                 uint32_t flag_val, const RowPrefetch &pre,
                                                 bool use_pre) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const bf16_t *xr = X + (int64_t)row * ldx;
  for (int q = 0; q < a.n_proj; ++q) {
    for (int kb = 0; kb < r; kb += kLayerRankBlk) {
      float acc[kLayerRankBlk];
#pragma unroll
      for (int j = 0; j < kLayerRankBlk; ++j) acc[j] = 0.f;
      const bf16_t *ab = static_cast<const bf16_t *>(a.A) + ((int64_t)slot * a.r_max + q * a.rs) * a.d_in;
      for (int c0 = 0; c0 < a.d_in; c0 += kLayerThreads * 8) {
        const int c = c0 + tid * 8;
        const bool ok = c < a.d_in;
        const int cc = ok ? c : a.d_in - 8;
        uint4 av[kLayerRankBlk], xv;
        if (use_pre && q == 0 && kb == 0 && c0 == 0) {
          xv = pre.x;
#pragma unroll
          for (int j = 0; j < kLayerRankBlk; ++j) av[j] = pre.a[j];
        } else {
          xv = ldg16(xr + cc);
#pragma unroll
          for (int j = 0; j < kLayerRankBlk; ++j)
            av[j] = ldg16(ab + (int64_t)min(kb + j, r - 1) * a.d_in + cc);
        }
        float xf[8];
        Elem<bf16_t>::unpack(xv, xf);
#pragma unroll
        for (int e = 0; e < 8; ++e) xf[e] = ok ? xf[e] : 0.f;
#pragma unroll
        for (int j = 0; j < kLayerRankBlk; ++j) {
          float af[8];
          Elem<bf16_t>::unpack(av[j], af);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[j] = fmaf(af[e], xf[e], acc[j]);
        }
      }
      butterfly_reduce<kLayerRankBlk>(acc, lane);   // lane l: total of pair l % 16
      if (lane < kLayerRankBlk) L.red[wave][lane] = acc[0];
      __syncthreads();
      if (tid < kLayerRankBlk && kb + tid < r) {
        float t = L.red[0][tid];
#pragma unroll
        for (int w = 1; w < kLayerWaves; ++w) t += L.red[w][tid];
        st_agent(a.H + (int64_t)row * a.r_max + q * a.rs + kb + tid, t);
      }
      __syncthreads();   // L.red is rewritten by the next pass
    }
  }
  // the H stores (lanes of wave 0) are complete at agent scope before the
  // flag is stored by the same wave, and before any wave passes the barrier
  if (wave == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (tid == 0 && a.sync) st_agent(a.sync + kSyncFlag0 + row, flag_val);
  }
  __syncthreads();
}

// After the K loop: H of every LoRA row of the tile [m0, m0 + BM) is
// published before the epilogue reads it.  Wave 0 polls the rows' flags (a
// bounded number of times); the rows still not set are computed here.
template <int BM>
__device__ __forceinline__ void layer_wait_rows(const LayerArgs &a, const bf16_t *X, int64_t ldx,
                                                int m0, int M, LayerLds &L) {
  static_assert(BM <= kWave, "one lane per tile row");
  const int tid = threadIdx.x;
  const uint32_t want = (uint32_t)L.misc[0] + 1u;
  if (tid < kWave) {
    const int row = m0 + tid;
    const bool need = tid < BM && row < M && L.rk[row] > 0;
    bool ready = !need;
    if (need && a.sync) ready = ld_agent(a.sync + kSyncFlag0 + row) == want;
    for (int it = 0; it < kLayerSpin && __ballot(!ready) != 0; ++it) {
      __builtin_amdgcn_s_sleep(8);
      if (!ready && a.sync) ready = ld_agent(a.sync + kSyncFlag0 + row) == want;
    }
    const uint64_t pend = __ballot(!ready);
    if (tid == 0) {
      L.misc[1] = (int)(uint32_t)pend;
      L.misc[2] = (int)(uint32_t)(pend >> 32);
    }
  }
  __syncthreads();
  uint64_t pend = (uint64_t)(uint32_t)L.misc[1] | ((uint64_t)(uint32_t)L.misc[2] << 32);
  while (pend) {                                 // workgroup-uniform
    const int t = __ffsll((unsigned long long)pend) - 1;
    pend &= pend - 1;
    const int row = m0 + t;
    RowPrefetch none;
    layer_row_shrink(a, X, ldx, row, L.key[row] - 1, L.rk[row], L, want, none, false);
  }
}

// End of a workgroup's part of the call: count it, and the last one resets
// the counter and advances the generation (every workgroup read the
// generation at its start, before any of them counted).
__device__ __forceinline__ void layer_exit(const LayerArgs &a, const LayerLds &L) {
  if (threadIdx.x == 0 && a.sync) {
    const uint32_t done = __hip_atomic_fetch_add(a.sync + kSyncExit, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    if (done == gridDim.x - 1) {
      st_agent(a.sync + kSyncExit, 0u);
      st_agent(a.sync + kSyncGen, (uint32_t)L.misc[0] + 1u);
    }
  }
}

}  // namespace lora
