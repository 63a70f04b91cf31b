// Segment metadata builder.
//
// Groups the token rows of a batch by adapter slot, as the adapter-batching
// page (Multi-LoRA Serving, charlestar.github.io, section "Segmented Kernel
// 需要哪些 Metadata") describes: one segment per distinct slot (base-only is
// its own segment with rank 0 and scale 0), segments in order of first
// appearance, rows ascending inside a segment, with segment_offsets,
// adapter slots, ranks, scales and the token permutation.
//
// One workgroup does the whole job with no host synchronisation: per-slot
// tables live in LDS (sized by the pool), rows are visited in chunks of one
// workgroup, and rows of one key inside a wavefront are grouped with a
// ballot loop (one iteration per distinct key in the wave).  Positions come
// from counts, never from the order in which atomics land, so the output is
// deterministic.  The same device routine runs as its own launch (up to
// 1024 threads) or as block 0 of the combined build + shrink launch.
#include <climits>

#include "lds_dma.cuh"
#include "lora_device.cuh"
#include "lora_kernels.h"
#include "shrink_rows.cuh"

namespace lora {
namespace {

constexpr int kThreads = 1024;
constexpr int kMaxKeys = 4096;  // n_slots + 1 (slot keys plus the base-only key)

// Keys of the first kRegChunks chunks of rows stay in registers between the
// passes; rows past that keep theirs in row_segment (read back by the same
// thread, two chunks ahead of their use).  Slot tables are staged in LDS
// once.  (More register chunks unroll the passes into more code than the
// instruction cache holds, which slows small batches down.)
constexpr int kRegChunks = 4;
// Batches up to kBitRows rows number their segments from a bitmap of the
// keys' first rows (one pass, no per-chunk barriers).
constexpr int kBitRows = 65536;
// Builds of at most kFastSegs segments place rows through a per-wave,
// per-segment count table (two barriers per chunk); more segments take the
// serial walk over the waves' group leaders.
constexpr int kFastSegs = 256;

struct Tables {
  int *first, *cnt, *off, *rank, *lead_key, *lead_cnt, *lead_base, *wave;
  float *scale;
};

// Key of row i: validated slot + 1; 0 = base-only (also for a bad slot or
// rank, counted in *bad).
__device__ __forceinline__ int row_key(int slot, const BuildArgs &a, const Tables &t, bool &bad) {
  if (slot == -1) return 0;
  if (slot < -1 || slot >= a.n_slots) {
    bad = true;
    return 0;
  }
  const int r = t.rank[slot];
  if (r < 0 || r > a.r_max) {
    bad = true;
    return 0;
  }
  return slot + 1;
}

// LDS words the routine needs for a pool of n_slots, n rows and a block of
// nthr threads; `table`: room for the per-wave segment counts.
int build_lds_words(int n_slots, int nthr, int n, bool table) {
  const int K = n_slots + 1;
  const int bits = n <= kBitRows ? 2 * ((n + 31) / 32) : 0;
  return 5 * K + 1 + 3 * nthr + nthr / kWave + 2 + bits +
         (table ? 2 * (nthr / kWave) * kFastSegs : 0);
}

}  // namespace

// The whole build by one workgroup (blockDim.x = 64..1024 threads, a
// multiple of 64) with `lds` pointing at build_lds_words(..., table) words.
__device__ __forceinline__ void build_segments_block(const BuildArgs &a, int *lds, bool table) {
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int nwaves = nthr / kWave;
  const int Kw = a.n_slots + 1;
  const int n = a.n;
  const int nbw = n <= kBitRows ? (n + 31) / 32 : 0;   // bitmap words (LDS layout)
  const bool bitmap = nbw > 0 && n > nthr;              // one chunk: numbered as it is walked
  int *s_first = lds;                   // first row of a key; later -(segment + 1)
  int *s_cnt = s_first + Kw;            // rows of a key; later the per-key cursor
  int *s_off = s_cnt + Kw;              // segment lengths, then exclusive offsets (Kw + 1)
  int *s_rank = s_off + Kw + 1;         // slot_rank staged
  float *s_scale = reinterpret_cast<float *>(s_rank + Kw);  // slot_scale staged
  int *s_lead_key = reinterpret_cast<int *>(s_scale + Kw);
  int *s_lead_cnt = s_lead_key + nthr;
  int *s_lead_base = s_lead_cnt + nthr;
  int *s_wave = s_lead_base + nthr;
  int &s_bad = s_wave[nwaves];
  int &s_total = s_wave[nwaves + 1];
  uint32_t *s_bits = reinterpret_cast<uint32_t *>(s_wave + nwaves + 2);  // [nbw]
  int *s_bpre = reinterpret_cast<int *>(s_bits + nbw);                    // [nbw]
  int *s_wcnt = s_bpre + nbw;            // [nwaves][kFastSegs] (table only)
  int *s_wbase = s_wcnt + nwaves * kFastSegs;

  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int K = a.n_slots + 1;
  const int nchunks = (n + nthr - 1) / nthr;
  const Tables t{s_first, s_cnt, s_off, s_rank, s_lead_key, s_lead_cnt, s_lead_base, s_wave,
                 s_scale};

  // Stage 0: one round of global loads: row slots of the register chunks and
  // the slot tables; LDS tables cleared.
  int keyreg[kRegChunks];
#pragma unroll
  for (int c = 0; c < kRegChunks; ++c) {
    const int i = c * nthr + tid;
    keyreg[c] = i < n ? a.row_slot[i] : -1;
  }
  for (int k = tid; k < a.n_slots; k += nthr) {
    s_rank[k] = a.slot_rank[k];
    s_scale[k] = a.slot_scale[k];
  }
  for (int k = tid; k < K; k += nthr) {
    s_first[k] = INT_MAX;
    s_cnt[k] = 0;
  }
  for (int w = tid; w < nbw; w += nthr) s_bits[w] = 0u;
  if (table)
    for (int e = tid; e < nwaves * kFastSegs; e += nthr) s_wcnt[e] = 0;
  if (tid == 0) {
    s_bad = 0;
    s_total = 0;
  }
  __syncthreads();

  // Pass 1: validate, remember keys, first row and row count per key.  One
  // LDS atomic per group of equal keys in a wave; min/add commute, so the
  // result does not depend on the order they land in.
  // Chunks past the registers, in groups of kGrp: the next group's values
  // are requested before this group is processed, so a chunk never waits a
  // memory round trip for its own.
  constexpr int kGrp = 4;
  auto walk = [&](auto load, auto body) {
    int cur[kGrp], nxt[kGrp];
#pragma unroll
    for (int u = 0; u < kGrp; ++u) cur[u] = load(kRegChunks + u);
    for (int g = kRegChunks; g < nchunks; g += kGrp) {
#pragma unroll
      for (int u = 0; u < kGrp; ++u) nxt[u] = load(g + kGrp + u);
#pragma unroll
      for (int u = 0; u < kGrp; ++u)
        if (g + u < nchunks) body(g + u, cur[u]);
#pragma unroll
      for (int u = 0; u < kGrp; ++u) cur[u] = nxt[u];
    }
  };
  uint64_t peersreg[kRegChunks];  // pass-1 groups of the register chunks, reused in pass 4
  auto pass1 = [&](int c, int slot, uint64_t &peers_out) -> int {
    const int i = c * nthr + tid;
    const bool valid = i < n;
    bool bad = false;
    const int key = valid ? row_key(slot, a, t, bad) : 0;
    const uint64_t badmask = __ballot(bad);
    if (lane == 0 && badmask) atomicAdd(&s_bad, __popcll(badmask));
    const uint64_t peers = match_key(key, valid);
    if (valid && (peers & lanemask_lt()) == 0) {  // lowest lane = lowest row of the group
      atomicMin(&s_first[key], i);
      atomicAdd(&s_cnt[key], __popcll(peers));
    }
    peers_out = peers;
    return key;
  };
#pragma unroll
  for (int c = 0; c < kRegChunks; ++c) {
    peersreg[c] = 0;
    if (c < nchunks) keyreg[c] = pass1(c, keyreg[c], peersreg[c]);
  }
  walk([&](int c) { const int i = c * nthr + tid; return i < n ? a.row_slot[i] : -1; },
       [&](int c, int slot) {
         const int i = c * nthr + tid;
         uint64_t unused;
         const int key = pass1(c, slot, unused);
         if (i < n) a.row_segment[i] = key;
       });
  __syncthreads();

  // From here on the barriers order LDS only (lgkm_barrier): the global
  // stores of pass 4 are read by no other thread, and pass 1's stores of the
  // keys were completed by the barrier above.
  // key of this thread's row in chunk c past the registers (row_segment holds
  // it from pass 1 until pass 4 overwrites it with the segment id; a chunk's
  // keys are read before its own pass 4 and before any later chunk's)
  auto key_at = [&](int c) { const int i = c * nthr + tid; return i < n ? a.row_segment[i] : 0; };

  // Pass 2: a row is the head of its segment iff it is its key's first row,
  // and segment ids count the heads in row order (first-appearance order).
  // Writes the segments' slot, rank, scale and length; s_first[key] becomes
  // -(segment + 1).
  auto head_out = [&](int key, int s) {
    const int slot = key - 1;
    const int r = key == 0 ? 0 : s_rank[slot];
    a.seg_slot[s] = slot;
    a.seg_rank[s] = r;
    a.seg_scale[s] = r > 0 ? s_scale[slot] : 0.0f;
    s_off[s] = s_cnt[key];
    s_first[key] = -(s + 1);
  };
  if (bitmap) {
    // heads as bits of a row bitmap; a head's id is the number of set bits
    // before it (a block scan of the words' popcounts)
    for (int k = tid; k < K; k += nthr) {
      const int f = s_first[k];
      if (f != INT_MAX) atomicOr(&s_bits[f >> 5], 1u << (f & 31));
    }
    lgkm_barrier();
    const int wpt = (nbw + nthr - 1) / nthr;     // words per thread, consecutive
    const int w0 = min(tid * wpt, nbw), w1 = min(w0 + wpt, nbw);
    int mine = 0;
    for (int w = w0; w < w1; ++w) mine += __popc(s_bits[w]);
    int incl = mine;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int u = __shfl_up(incl, d);
      if (lane >= d) incl += u;
    }
    if (lane == kWave - 1) s_wave[wave] = incl;
    lgkm_barrier();
    int before = incl - mine;
    for (int w = 0; w < wave; ++w) before += s_wave[w];
    for (int w = w0; w < w1; ++w) {
      s_bpre[w] = before;
      before += __popc(s_bits[w]);
    }
    if (tid == nthr - 1) s_total = before;       // the last thread's end: all heads
    lgkm_barrier();
    for (int k = tid; k < K; k += nthr) {
      const int f = s_first[k];
      if (f != INT_MAX)
        head_out(k, s_bpre[f >> 5] + __popc(s_bits[f >> 5] & ((1u << (f & 31)) - 1u)));
    }
    lgkm_barrier();
  } else {
    auto pass2 = [&](int c, int key) {
      const int i = c * nthr + tid;
      const bool valid = i < n;
      const bool head = valid && s_first[key] == i;
      const uint64_t hm = __ballot(head);
      if (lane == 0) s_wave[wave] = __popcll(hm);
      lgkm_barrier();
      int before = s_total;
      for (int w = 0; w < wave; ++w) before += s_wave[w];
      if (head) head_out(key, before + __popcll(hm & lanemask_lt()));
      lgkm_barrier();
      if (tid == 0) {
        int tot = 0;
        for (int w = 0; w < nwaves; ++w) tot += s_wave[w];
        s_total += tot;
      }
      lgkm_barrier();
    };
#pragma unroll
    for (int c = 0; c < kRegChunks; ++c)
      if (c < nchunks) pass2(c, keyreg[c]);
    walk(key_at, pass2);
  }
  const int S = s_total;

  // Pass 3: exclusive scan of the segment lengths; reset per-key cursors.
  for (int k = tid; k < K; k += nthr) s_cnt[k] = 0;
  int carry = 0;
  for (int c0 = 0; c0 < S; c0 += nthr) {
    const int s = c0 + tid;
    const int v = s < S ? s_off[s] : 0;
    int incl = v;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int u = __shfl_up(incl, d);
      if (lane >= d) incl += u;
    }
    if (lane == kWave - 1) s_wave[wave] = incl;
    lgkm_barrier();
    int before = carry;
    int chunk = 0;
    for (int w = 0; w < nwaves; ++w) {
      if (w < wave) before += s_wave[w];
      chunk += s_wave[w];
    }
    if (s < S) {
      const int excl = before + incl - v;
      s_off[s] = excl;
      a.seg_off[s] = excl;
    }
    carry += chunk;
    lgkm_barrier();
  }
  if (tid == 0) s_off[S] = n;
  lgkm_barrier();

  // Pass 4: position = segment offset + rows of the same key in earlier
  // chunks and waves + rows of the same key in lower lanes, so rows keep
  // their order inside a segment.
  if (table && S <= kFastSegs) {
    // Each wave's group leaders put their counts in the wave's row of a
    // [wave][segment] table; thread s turns column s into bases in wave
    // order, carrying the segment's running count (s_cnt[s]) across chunks.
    auto pass4t = [&](int c, int key, uint64_t peers) {
      const int i = c * nthr + tid;
      const bool valid = i < n;
      const int local = __popcll(peers & lanemask_lt());
      const int seg = -s_first[key] - 1;
      if (valid && local == 0) s_wcnt[wave * kFastSegs + seg] = __popcll(peers);
      lgkm_barrier();
      if (tid < S) {
        // the column's reads first, then its writes (no LDS round trip per wave)
        int v[kThreads / kWave];
#pragma unroll
        for (int w = 0; w < kThreads / kWave; ++w)
          v[w] = w < nwaves ? s_wcnt[w * kFastSegs + tid] : 0;
        int run = s_cnt[tid];
#pragma unroll
        for (int w = 0; w < kThreads / kWave; ++w) {
          if (w < nwaves) {
            s_wcnt[w * kFastSegs + tid] = 0;
            s_wbase[w * kFastSegs + tid] = run;
          }
          run += v[w];
        }
        s_cnt[tid] = run;
      }
      lgkm_barrier();
      if (valid) {
        a.token_indices[s_off[seg] + s_wbase[wave * kFastSegs + seg] + local] = i;
        a.row_segment[i] = seg;
      }
    };
#pragma unroll
    for (int c = 0; c < kRegChunks; ++c)
      if (c < nchunks) pass4t(c, keyreg[c], peersreg[c]);
    walk(key_at, [&](int c, int key) { pass4t(c, key, match_key(key, c * nthr + tid < n)); });
  } else {
    // Wave 0 walks the waves' group leaders in order, so the cross-wave
    // part follows row order exactly.
    auto pass4 = [&](int c, int key, uint64_t peers) {
      const int i = c * nthr + tid;
      const bool valid = i < n;
      const int local = __popcll(peers & lanemask_lt());
      s_lead_cnt[tid] = (valid && local == 0) ? __popcll(peers) : 0;
      s_lead_key[tid] = key;
      lgkm_barrier();
      if (wave == 0) {
        // waves past the last row of the chunk hold no leaders
        const int wend = min(nwaves, (n - c * nthr + kWave - 1) / kWave);
        for (int w = 0; w < wend; ++w) {
          const int u = w * kWave + lane;
          const int cnt = s_lead_cnt[u];
          if (cnt > 0) {
            const int k = s_lead_key[u];
            const int b = s_cnt[k];
            s_cnt[k] = b + cnt;
            s_lead_base[u] = b;
          }
        }
      }
      lgkm_barrier();
      if (valid) {
        const int seg = -s_first[key] - 1;
        const int lt = wave * kWave + (__ffsll((unsigned long long)peers) - 1);
        const int pos = s_off[seg] + s_lead_base[lt] + local;
        a.token_indices[pos] = i;
        a.row_segment[i] = seg;
      }
      lgkm_barrier();
    };
#pragma unroll
    for (int c = 0; c < kRegChunks; ++c)
      if (c < nchunks) pass4(c, keyreg[c], peersreg[c]);
    walk(key_at, [&](int c, int key) { pass4(c, key, match_key(key, c * nthr + tid < n)); });
  }

  if (tid == 0) {
    a.seg_off[S] = n;
    *a.num_segments = S;
    *a.status = s_bad;
  }
}

namespace {

__global__ __launch_bounds__(kThreads) void build_segments_kernel(BuildArgs a) {
  extern __shared__ int lds[];
  build_segments_block(a, lds, true);
}

// ----------------------------------------------------------------------------
// Build + shrink in one launch, for decode-sized batches (every segment
// short).  Block 0 builds the metadata; block 1 + ((rb * n_slots + slot) *
// nkb + kb) computes H for rank rows [8 kb, 8 kb + 8) of `slot` and the
// slot's rows [64 rb, 64 rb + 64) in row order.  Those blocks find their
// rows by scanning the per-row slot ids (wave ballots, counts in LDS), so
// they never wait for the metadata; each (row, rank row) sum is formed
// exactly as the metadata-driven shrink forms it, so H has the same bits.
// A row whose slot has a rank outside [0, r_max] is base-only (the build
// counts it), and so is its slot here: no block of that slot writes H.
// ----------------------------------------------------------------------------
constexpr int kBSMaxRows = 512;            // batches up to this many rows
constexpr int kBSThreads = kShW * kWave;
constexpr int kBSChunks = kBSMaxRows / kBSThreads;

template <typename T>
__global__ __launch_bounds__(kBSThreads) void build_shrink_kernel(BuildArgs a, const T *X,
                                                                  int64_t ldx, const T *A,
                                                                  int d_in, int policy, int r_max,
                                                                  int nkb, float *H) {
  extern __shared__ int lds[];
  if (blockIdx.x == 0) {
    build_segments_block(a, lds, false);
    return;
  }
  const int b = blockIdx.x - 1;
  const int kb = b % nkb;
  const int slot = (b / nkb) % a.n_slots;
  const int rb = b / (nkb * a.n_slots);
  const int k0 = kb * kShRB;              // rank row of the pool (a.r_max = rank bound)
  const int kl0 = k0 % a.r_max;           // ... and inside its projection's block
  float (*s_part)[kShNP] = reinterpret_cast<float (*)[kShNP]>(lds);
  int *s_wc = lds + kShW * kShNP;
  int *s_rows = s_wc + kShW;                // [n]
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  // every load of the block's set-up at once: the slot's rank and the
  // row slot ids (n <= kBSMaxRows)
  const int r = a.slot_rank[slot];
  int rs[kBSChunks];
#pragma unroll
  for (int c = 0; c < kBSChunks; ++c) {
    const int i = c * kBSThreads + tid;
    rs[c] = i < a.n ? a.row_slot[i] : -1;
  }
  if (r < 1 || r > a.r_max) return;         // rank-0 slot, or rows demoted by the build
  const int R = rank_bucket(r, policy, a.r_max);
  if (kl0 >= R) return;
  // rows of the slot in ascending order
  int cnt = 0;
#pragma unroll
  for (int c = 0; c < kBSChunks; ++c) {
    if (c * kBSThreads >= a.n) break;       // uniform
    const bool match = rs[c] == slot;
    const uint64_t m = __ballot(match);
    if (lane == 0) s_wc[wave] = __popcll(m);
    __syncthreads();
    int before = cnt, total = 0;
#pragma unroll
    for (int w = 0; w < kShW; ++w) {
      before += w < wave ? s_wc[w] : 0;
      total += s_wc[w];
    }
    if (match) s_rows[before + __popcll(m & lanemask_lt())] = c * kBSThreads + tid;
    cnt += total;
    __syncthreads();
  }
  const int p0 = rb * kRowBlk, p1 = min(cnt, p0 + kRowBlk);
  if (p0 >= p1) return;
  shrink_rows<T>(X, ldx, A, slot, k0, kl0, min(kShRB, R - kl0), r, r_max, d_in, s_rows, p0, p1,
                 H, s_part);
}

}  // namespace

hipError_t launch_build_shrink(const BuildArgs &a, const void *X, int64_t ldx,
                               const PoolView &pool, float *H, hipStream_t stream) {
  if (a.n < 1 || a.n > kBSMaxRows) return hipErrorNotSupported;
  const int nkb = (pool.r_max + kShRB - 1) / kShRB;
  const int nrb = (a.n + kRowBlk - 1) / kRowBlk;
  const long blocks = 1 + (long)pool.n_slots * nkb * nrb;
  if (blocks > 16384) return hipErrorNotSupported;
  const int words_build = build_lds_words(a.n_slots, kBSThreads, a.n, false);
  const int words_shrink = kShW * kShNP + kShW + a.n;
  const size_t lds = (size_t)(words_build > words_shrink ? words_build : words_shrink) * 4;
  if (pool.dtype == 1)
    hipLaunchKernelGGL(build_shrink_kernel<bf16_t>, dim3((unsigned)blocks), dim3(kBSThreads), lds,
                       stream, a, (const bf16_t *)X, ldx, (const bf16_t *)pool.A, pool.d_in,
                       pool.policy, pool.r_max, nkb, H);
  else
    hipLaunchKernelGGL(build_shrink_kernel<float>, dim3((unsigned)blocks), dim3(kBSThreads), lds,
                       stream, a, (const float *)X, ldx, (const float *)pool.A, pool.d_in,
                       pool.policy, pool.r_max, nkb, H);
  return hipGetLastError();
}

hipError_t launch_build_segments(const int32_t *row_slot, int n, int n_slots, int r_max,
                                 const int32_t *slot_rank, const float *slot_scale,
                                 int32_t *token_indices, int32_t *row_segment, int32_t *seg_off,
                                 int32_t *seg_slot, int32_t *seg_rank, float *seg_scale,
                                 int32_t *num_segments, int32_t *status, hipStream_t stream) {
  if (n_slots + 1 > kMaxKeys) return hipErrorInvalidValue;
  BuildArgs a{row_slot, n, n_slots, r_max, slot_rank, slot_scale, token_indices, row_segment,
              seg_off, seg_slot, seg_rank, seg_scale, num_segments, status};
  // one wave per 64 rows up to 16 waves
  int threads = ((n + kWave - 1) / kWave) * kWave;
  threads = threads < kWave ? kWave : (threads > kThreads ? kThreads : threads);
  const size_t lds = (size_t)build_lds_words(n_slots, threads, n, true) * 4;
  hipLaunchKernelGGL(build_segments_kernel, dim3(1), dim3(threads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace lora
