// Expert dispatch: per-expert histogram, exclusive prefix sum and a stable
// permutation of the (token, choice) pairs, grouped by expert and ordered by
// token inside a group, plus the tile list the grouped GEMMs walk.
//
// The pages only say that a token activates a small subset of the stored
// parameters (q4km.ai "Step-3.5-Flash", "Technical Overview"; nipponese.news
// article, architecture section); gathering each expert's tokens into
// contiguous rows is how the expert FFNs become dense GEMMs.
//
// One workgroup of 16 waves (up to 1024 tokens: a wave's slice is at most one
// token per lane, whose choices the lane loads once, all in flight together);
// deterministic without global atomics:
//   1. wave w counts the pairs of its token slice per expert (LDS atomics:
//      counts do not depend on their order);
//   2. per expert, the wave counts are scanned in wave order, the expert
//      totals are scanned in expert order;
//   3. a pair's rank inside its expert is the number of lower lanes of the
//      wave holding that expert (64-bit LDS masks + popcount) plus the counts
//      of earlier waves.
// The shared expert is group E: rows P .. P+T-1 hold tokens 0 .. T-1.
#include "moe_common.hpp"
#include "moe_kernels.hpp"
#include "moe_topk.hpp"

namespace moe {
namespace {

constexpr int kDispWaves = 16;
constexpr int kDispThreads = kDispWaves * kWave;

// Exclusive scan of buf[0..n) in place by wave 0 (n <= 64 * 16); every thread
// gets the total.  Lane l owns a run of ceil(n/64) consecutive entries.
__device__ int block_exclusive_scan(int* buf, int* total_slot, int n) {
  const int tid = threadIdx.x;
  __syncthreads();
  if (tid < kWave) {
    const int per = (n + kWave - 1) / kWave;
    const int beg = min(n, tid * per), end = min(n, beg + per);
    int sum = 0;
    for (int i = beg; i < end; ++i) sum += buf[i];
    int incl = sum;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int o = __shfl_up(incl, d);
      if (tid >= d) incl += o;
    }
    int run = incl - sum;
    for (int i = beg; i < end; ++i) {
      const int v = buf[i];
      buf[i] = run;
      run += v;
    }
    if (tid == kWave - 1) *total_slot = incl;
  }
  __syncthreads();
  return *total_slot;
}

// The whole dispatch for up to 64 * NW tokens, run by one workgroup of NW
// waves (the last one of the top-k + dispatch kernel).
template <int NW>
__device__ __forceinline__ void dispatch_body(
    const int32_t* __restrict__ idx, int T, int k, int E, int has_shared, TileLists lists,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
    int32_t* __restrict__ inv, int32_t* __restrict__ row_tok, const float* __restrict__ w,
    float* __restrict__ row_w, int32_t* __restrict__ dbg) {
  constexpr int NTH = NW * kWave;
  __shared__ int hist[NW][kMaxExperts];                 // 2 KiB per wave
  __shared__ unsigned long long mask[NW][kMaxExperts];  // 4 KiB per wave
  __shared__ int tot[kMaxExperts + 1];
  __shared__ int off[kMaxExperts + 1];
  __shared__ int ntile[kMaxExperts + 1];
  __shared__ int ntile2[kMaxExperts + 1];
  __shared__ int scan_total;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int P = T * k;
  const int tw = (T + NW - 1) / NW;  // tokens per wave, <= 64
  const int tbeg = min(T, wave * tw), tend = min(T, tbeg + tw);

  // this lane's token and its choices: unconditional loads (a lane without a
  // token re-reads token 0; choices past k re-read the last one), issued
  // before the LDS is cleared so that their latency overlaps it
  const int t = tbeg + lane;
  const bool ok = lane < tw && t < tend;
  const int tl = ok ? t : 0;
  int ej[kMaxTopK];
  float wj[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    ej[j] = idx[(size_t)tl * k + (j < k ? j : k - 1)];
    wj[j] = row_w ? w[(size_t)tl * k + (j < k ? j : k - 1)] : 0.f;
  }
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    dbg_check(dbg, !ok || (ej[j] >= 0 && ej[j] < E), kDbgExpert, ej[j]);
    ej[j] = ej[j] < 0 ? 0 : (ej[j] >= E ? E - 1 : ej[j]);
  }

  for (int i = tid; i < NW * E; i += NTH) {
    hist[i / E][i % E] = 0;
    mask[i / E][i % E] = 0ull;
  }
  __syncthreads();

  // 1. histogram per wave
  if (ok) {
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
      if (j < k)
        __hip_atomic_fetch_add(&hist[wave][ej[j]], 1, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  __syncthreads();

  // 2. per-expert scan over waves, then scan over experts
  for (int ex = tid; ex < E; ex += NTH) {
    int run = 0;
    for (int w = 0; w < NW; ++w) {
      const int c = hist[w][ex];
      hist[w][ex] = run;
      run += c;
    }
    tot[ex] = run;
    off[ex] = run;
  }
  __syncthreads();
  block_exclusive_scan(off, &scan_total, E);
  for (int ex = tid; ex < E; ex += NTH) {
    counts[ex] = tot[ex];
    offsets[ex] = off[ex];
    for (int w = 0; w < NW; ++w) hist[w][ex] += off[ex];
  }
  if (tid == 0) {
    counts[E] = has_shared ? T : 0;
    offsets[E] = P;
    offsets[E + 1] = P + (has_shared ? T : 0);
  }
  // tile counts per group and list
  for (int gr = tid; gr <= E; gr += NTH) {
    const int c = gr < E ? tot[gr] : (has_shared ? T : 0);
    const bool second = gr < E && lists.in_second(c);
    ntile[gr] = second ? 0 : (c + lists.bm - 1) / lists.bm;
    ntile2[gr] = second ? (c + lists.bm2 - 1) / lists.bm2 : 0;
  }
  __syncthreads();

  // tile lists: groups in order 0..E, m-tiles in order inside a group
  const int total_tiles = block_exclusive_scan(ntile, &scan_total, E + 1);
  const int total_tiles2 = lists.hot > 0 ? block_exclusive_scan(ntile2, &scan_total, E + 1) : 0;
  // ntile[] / ntile2[] now hold each group's first tile; the counts are recomputed
  for (int gr = tid; gr <= E; gr += NTH) {
    const int c = gr < E ? tot[gr] : (has_shared ? T : 0);
    if (gr < E && lists.in_second(c)) {
      const int nt = (c + lists.bm2 - 1) / lists.bm2;
      for (int m = 0; m < nt; ++m) lists.tiles2[ntile2[gr] + m] = (gr << 16) | m;
    } else {
      const int nt = (c + lists.bm - 1) / lists.bm;
      for (int m = 0; m < nt; ++m) lists.tiles[ntile[gr] + m] = (gr << 16) | m;
    }
  }
  if (tid == 0) {
    lists.ntiles[0] = total_tiles;
    if (lists.hot > 0) lists.ntiles2[0] = total_tiles2;
  }

  // 3. stable scatter: a pair's row = the wave's first row of its expert +
  // the lanes below holding that expert (a token holds an expert once)
  if (ok) {
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
      if (j < k)
        __hip_atomic_fetch_or(&mask[wave][ej[j]], 1ull << lane, __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  __syncthreads();
  if (ok) {
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j < k) {
        const int row = hist[wave][ej[j]] + __popcll(mask[wave][ej[j]] & below);
        const int p = t * k + j;
        perm[row] = p;
        inv[p] = row;
        row_tok[row] = t;
        if (row_w) row_w[row] = wj[j];
      }
    }
  }

  if (has_shared)
    for (int t = tid; t < T; t += NTH) row_tok[P + t] = t;
}

// Up to 64 tokens, the dispatch by one wave, lane = token: per expert, a
// 64-bit LDS mask of the tokens that chose it (a token holds an expert once),
// its popcount the expert's count; lane l scans the counts (and tile counts)
// of experts l*per .. l*per+per-1 with a wave-wide prefix sum; a pair's row
// is its expert's first row plus the tokens below it in that expert's mask.
// Same outputs as dispatch_body, which keeps the batches with a second tile
// list (never this small).
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(v, d);
    if (lane >= d) v += o;
  }
  return v;
}

__device__ __forceinline__ void dispatch_wave(const int32_t* __restrict__ idx, int T, int k, int E,
                                              int has_shared, const TileLists& lists,
                                              int32_t* __restrict__ counts,
                                              int32_t* __restrict__ offsets,
                                              int32_t* __restrict__ perm, int32_t* __restrict__ inv,
                                              int32_t* __restrict__ row_tok,
                                              const float* __restrict__ w,
                                              float* __restrict__ row_w,
                                              int32_t* __restrict__ dbg) {
  __shared__ unsigned long long mask[kMaxExperts];
  __shared__ int first[kMaxExperts];
  const int lane = threadIdx.x & 63;
  const int P = T * k;
  const bool ok = lane < T;
  // this lane's token's choices (a lane without a token re-reads token 0;
  // choices past k re-read the last one), in flight while the masks clear
  int ej[kMaxTopK];
  float wj[kMaxTopK];
  {
    const int tl = ok ? lane : 0;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      ej[j] = idx[(size_t)tl * k + (j < k ? j : k - 1)];
      wj[j] = row_w ? w[(size_t)tl * k + (j < k ? j : k - 1)] : 0.f;
    }
  }
  for (int e = lane; e < E; e += kWave) mask[e] = 0ull;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    dbg_check(dbg, !ok || (ej[j] >= 0 && ej[j] < E), kDbgExpert, ej[j]);
    ej[j] = ej[j] < 0 ? 0 : (ej[j] >= E ? E - 1 : ej[j]);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  if (ok) {
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
      if (j < k)
        __hip_atomic_fetch_or(&mask[ej[j]], 1ull << lane, __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_WAVEFRONT);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
  // counts, rows and tiles of experts e0 .. e0+per-1
  const int per = (E + kWave - 1) / kWave, e0 = lane * per;
  int c[kMaxExperts / kWave], sum = 0, nts = 0;
#pragma unroll
  for (int i = 0; i < kMaxExperts / kWave; ++i) {
    const int e = e0 + i;
    c[i] = (i < per && e < E) ? __popcll(mask[e]) : 0;
    sum += c[i];
    nts += (c[i] + lists.bm - 1) / lists.bm;
  }
  const int incl = wave_incl_scan(sum), incl_t = wave_incl_scan(nts);
  int row = incl - sum, tile = incl_t - nts;
#pragma unroll
  for (int i = 0; i < kMaxExperts / kWave; ++i) {
    const int e = e0 + i;
    if (i < per && e < E) {
      counts[e] = c[i];
      offsets[e] = row;
      first[e] = row;
      const int nt = (c[i] + lists.bm - 1) / lists.bm;
      for (int m = 0; m < nt; ++m) lists.tiles[tile + m] = (e << 16) | m;
      row += c[i];
      tile += nt;
    }
  }
  const int routed_tiles = __shfl(incl_t, kWave - 1);
  const int shared_tiles = has_shared ? (T + lists.bm - 1) / lists.bm : 0;
  for (int m = lane; m < shared_tiles; m += kWave) lists.tiles[routed_tiles + m] = (E << 16) | m;
  if (lane == 0) {
    counts[E] = has_shared ? T : 0;
    offsets[E] = P;
    offsets[E + 1] = P + (has_shared ? T : 0);
    lists.ntiles[0] = routed_tiles + shared_tiles;
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
  // stable scatter
  if (ok) {
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j < k) {
        const int r = first[ej[j]] + __popcll(mask[ej[j]] & below);
        const int p = lane * k + j;
        perm[r] = p;
        inv[p] = r;
        row_tok[r] = lane;
        if (row_w) row_w[r] = wj[j];
      }
    }
    if (has_shared) row_tok[P + lane] = lane;
  }
}

// Top-k for NW tokens per workgroup (one wave each), then the workgroup that
// finishes last runs the dispatch (one wave of it up to 64 tokens): one
// launch less on the path of small batches.  `done` counts finished
// workgroups; the router logits kernel
// clears it earlier on the same stream.  After the workgroup barrier (its
// waves' choices are in this XCD's L2), one thread releases them device-wide
// and counts the workgroup; the thread that counts last acquires every
// workgroup's choices for its own.
template <int NW, int NS>
__global__ __launch_bounds__(NW * 64) void topk_dispatch_kernel(
    const float* __restrict__ part, int ks, const float* __restrict__ bias, int bias_mode, int T,
    int E, int k, int score, int renorm, float scale, int32_t* __restrict__ idx,
    float* __restrict__ wout, float* __restrict__ gap, int32_t* __restrict__ done,
    int has_shared, TileLists lists, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv, int32_t* __restrict__ row_tok,
    float* __restrict__ row_w, int32_t* __restrict__ dbg) {
  __shared__ int last;
  const int t = blockIdx.x * NW + (threadIdx.x >> 6);
  if (t < T) topk_token<NS>(part, ks, bias, bias_mode, T, E, k, score, renorm, scale, t, idx, wout, gap);
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");  // this XCD's L2 -> memory
    const bool l = __hip_atomic_fetch_add(done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                   (int)gridDim.x - 1;
    if (l) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    last = l;
  }
  __syncthreads();
  if (!last) return;
  if constexpr (NW == 4) {  // the launch shape of up to 256 tokens
    if (T <= kWave && lists.hot == 0) {
      if (threadIdx.x < kWave)
        dispatch_wave(idx, T, k, E, has_shared, lists, counts, offsets, perm, inv, row_tok, wout,
                      row_w, dbg);
      return;
    }
  }
  dispatch_body<NW>(idx, T, k, E, has_shared, lists, counts, offsets, perm, inv, row_tok, wout,
                    row_w, dbg);
}

// ---------------------------------------------------------------- large batches
// Same result, spread over many workgroups: (1) each block of kBlkTokens
// tokens counts its pairs per expert and per wave; (2) one workgroup turns the
// block counts into each (block, expert)'s first row and builds the offsets
// and tile list; (3) each block scatters its pairs with the lane-mask ranks,
// starting from those rows.  Deterministic: no global atomics.
constexpr int kBlkWaves = 4;
constexpr int kBlkTokens = kBlkWaves * kWave;  // one 64-token step per wave

__global__ __launch_bounds__(kBlkWaves * kWave) void dispatch_hist_kernel(
    const int32_t* __restrict__ idx, int T, int k, int E, int32_t* __restrict__ blk_hist,
    int32_t* __restrict__ dbg) {
  __shared__ int hist[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int t = blockIdx.x * kBlkTokens + threadIdx.x;
  if (t < T)
    for (int j = 0; j < k; ++j) {
      int e = idx[(size_t)t * k + j];
      dbg_check(dbg, e >= 0 && e < E, kDbgExpert, e);
      e = e < 0 ? 0 : (e >= E ? E - 1 : e);
      atomicAdd(&hist[e], 1);
    }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) blk_hist[(size_t)blockIdx.x * E + e] = hist[e];
}

__global__ __launch_bounds__(kDispThreads) void dispatch_scan_kernel(
    int32_t* __restrict__ blk_hist, int nblk, int T, int k, int E, int has_shared, int bm,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ tiles,
    int32_t* __restrict__ ntiles_out) {
  __shared__ int tot[kMaxExperts + 1];
  __shared__ int off[kMaxExperts + 1];
  __shared__ int ntile[kMaxExperts + 1];
  __shared__ int scan_total;
  const int tid = threadIdx.x;
  const int P = T * k;
  constexpr int kChunk = 16;  // block counts loaded together (independent loads)
  // per expert: total over blocks
  if (tid < E) {
    int run = 0;
    for (int b0 = 0; b0 < nblk; b0 += kChunk) {
      int c[kChunk];
#pragma unroll
      for (int i = 0; i < kChunk; ++i)
        c[i] = b0 + i < nblk ? blk_hist[(size_t)(b0 + i) * E + tid] : 0;
#pragma unroll
      for (int i = 0; i < kChunk; ++i) run += c[i];
    }
    tot[tid] = run;
    off[tid] = run;
  }
  __syncthreads();
  block_exclusive_scan(off, &scan_total, E);
  // each (block, expert) count becomes that block's first row for the expert
  if (tid < E) {
    counts[tid] = tot[tid];
    offsets[tid] = off[tid];
    ntile[tid] = (tot[tid] + bm - 1) / bm;
    int run = off[tid];
    for (int b0 = 0; b0 < nblk; b0 += kChunk) {
      int c[kChunk];
#pragma unroll
      for (int i = 0; i < kChunk; ++i)
        c[i] = b0 + i < nblk ? blk_hist[(size_t)(b0 + i) * E + tid] : 0;
#pragma unroll
      for (int i = 0; i < kChunk; ++i)
        if (b0 + i < nblk) {
          blk_hist[(size_t)(b0 + i) * E + tid] = run;
          run += c[i];
        }
    }
  }
  if (tid == 0) {
    counts[E] = has_shared ? T : 0;
    offsets[E] = P;
    offsets[E + 1] = P + (has_shared ? T : 0);
    ntile[E] = has_shared ? (T + bm - 1) / bm : 0;
  }
  __syncthreads();
  const int total_tiles = block_exclusive_scan(ntile, &scan_total, E + 1);
  if (tid <= E) {
    const int c = tid < E ? tot[tid] : (has_shared ? T : 0);
    const int nt = (c + bm - 1) / bm;
    for (int m = 0; m < nt; ++m) tiles[ntile[tid] + m] = (tid << 16) | m;
  }
  if (tid == 0) ntiles_out[0] = total_tiles;
}

__global__ __launch_bounds__(kBlkWaves * kWave) void dispatch_scatter_kernel(
    const int32_t* __restrict__ idx, int T, int k, int E, int has_shared,
    const int32_t* __restrict__ blk_first, int32_t* __restrict__ perm, int32_t* __restrict__ inv,
    int32_t* __restrict__ row_tok, const float* __restrict__ w, float* __restrict__ row_w,
    int32_t* __restrict__ dbg) {
  __shared__ int base[kBlkWaves][kMaxExperts];
  __shared__ unsigned long long mask[kBlkWaves][kMaxExperts];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int P = T * k;
  for (int i = tid; i < kBlkWaves * E; i += blockDim.x) {
    base[i / E][i % E] = 0;
    mask[i / E][i % E] = 0ull;
  }
  __syncthreads();
  const int t = blockIdx.x * kBlkTokens + tid;  // wave w holds tokens 64w .. 64w+63 of the block
  const bool ok = t < T;
  int ej[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    ej[j] = 0;
    if (j < k && ok) {
      int e = idx[(size_t)t * k + j];
      dbg_check(dbg, e >= 0 && e < E, kDbgExpert, e);
      ej[j] = e < 0 ? 0 : (e >= E ? E - 1 : e);
      atomicOr(&mask[wave][ej[j]], 1ull << lane);
    }
  }
  __syncthreads();
  // first row of each (wave, expert): block start + pairs of earlier waves
  for (int e = tid; e < E; e += blockDim.x) {
    int run = blk_first[(size_t)blockIdx.x * E + e];
    for (int w = 0; w < kBlkWaves; ++w) {
      base[w][e] = run;
      run += __popcll(mask[w][e]);
    }
  }
  __syncthreads();
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j < k && ok) {
      const unsigned long long m = mask[wave][ej[j]];
      const int row = base[wave][ej[j]] + __popcll(m & below);
      const int p = t * k + j;
      perm[row] = p;
      inv[p] = row;
      row_tok[row] = t;
      if (row_w) row_w[row] = w[p];
    }
  }
  if (has_shared && ok) row_tok[P + t] = t;
}

}  // namespace

int dispatch_blocks(int T) { return (T + kBlkTokens - 1) / kBlkTokens; }

hipError_t launch_dispatch_large(const int32_t* idx, int T, int k, int E, int has_shared, int bm,
                                 int32_t* blk_hist, int32_t* counts, int32_t* offsets,
                                 int32_t* perm, int32_t* inv, int32_t* row_tok, int32_t* tiles,
                                 int32_t* ntiles, const float* w, float* row_w, int32_t* dbg,
                                 hipStream_t s) {
  const int nblk = dispatch_blocks(T);
  hipLaunchKernelGGL(dispatch_hist_kernel, dim3(nblk), dim3(kBlkTokens), 0, s, idx, T, k, E,
                     blk_hist, dbg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(kDispThreads), 0, s, blk_hist, nblk, T, k,
                     E, has_shared, bm, counts, offsets, tiles, ntiles);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dispatch_scatter_kernel, dim3(nblk), dim3(kBlkTokens), 0, s, idx, T, k, E,
                     has_shared, blk_hist, perm, inv, row_tok, w, row_w, dbg);
  return hipGetLastError();
}

hipError_t launch_topk_dispatch(const float* part, int ks, const float* bias, int bias_mode, int T,
                                int E, int k, int score, int renorm, float scale, int32_t* idx,
                                float* w, float* gap, int32_t* done, int has_shared,
                                const TileLists& tl, int32_t* counts, int32_t* offsets,
                                int32_t* perm, int32_t* inv, int32_t* row_tok, float* row_w,
                                int32_t* dbg, hipStream_t s) {
  if (T < 1 || T > kDispThreads || k < 1 || k > kMaxTopK) return hipErrorInvalidValue;
  if (tl.bm < 1 || (tl.hot > 0 && (tl.bm2 < 1 || !tl.tiles2 || !tl.ntiles2)))
    return hipErrorInvalidValue;
  // 4 tokens per workgroup up to 256 tokens (the top-k waves spread over more
  // CUs), 16 above
#define MOE_TD(NW, NS)                                                                          \
  hipLaunchKernelGGL((topk_dispatch_kernel<NW, NS>), dim3((T + NW - 1) / NW), dim3(NW * 64), 0, \
                     s, part, ks, bias, bias_mode, T, E, k, score, renorm, scale, idx, w, gap,    \
                     done, has_shared, tl, counts, offsets, perm, inv, row_tok, row_w, dbg)
#define MOE_TD_NS(NW)                    \
  switch (topk_slots(E)) {               \
    case 1: MOE_TD(NW, 1); break;        \
    case 2: MOE_TD(NW, 2); break;        \
    case 5: MOE_TD(NW, 5); break;        \
    default: MOE_TD(NW, kMaxPerLane);    \
  }
  if (T <= 4 * kWave) {
    MOE_TD_NS(4);
  } else {
    MOE_TD_NS(kDispWaves);
  }
#undef MOE_TD_NS
#undef MOE_TD
  return hipGetLastError();
}


}  // namespace moe
