// Per-token top-k selection over the router logits, shared by the top-k
// kernel and the fused top-k + dispatch kernel.
//
// Source: llm-atlas "Step-3.5-Flash", table "Champs bruts du config.json"
// (moe_top_k, norm_expert_weight, moe_router_activation,
// moe_router_scaling_factor, use_moe_router_bias).  Readings where the pages
// are silent: ties go to the lower expert index; the bias is added to the
// logits (bias_mode 0) or to the selection scores only (bias_mode 1).
#pragma once

#include "moe_common.hpp"

#include <math.h>

namespace moe {

// Orderable key of (score, expert): larger key = larger score, and on equal
// scores the lower expert index.  NaN ranks as -inf.
__device__ __forceinline__ unsigned long long rank_key(float s, int e) {
  if (s != s) s = -INFINITY;
  uint32_t u = __float_as_uint(s);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)u << 32) | (uint32_t)(0xffffffffu - (uint32_t)e);
}

__device__ __forceinline__ float key_score(unsigned long long key) {
  uint32_t u = (uint32_t)(key >> 32);
  u = (u & 0x80000000u) ? (u & 0x7fffffffu) : ~u;
  return __uint_as_float(u);
}

// Wave-wide reductions without LDS traffic: lane i ^ 1 and i ^ 2 through
// DPP quad permutations, i ^ 4 / i ^ 8 through the 8- and 16-lane mirrors
// (equivalent once every quad / octet holds one value), then the rows of 16
// and the halves of 32 through gfx950's permlane swaps.  Every lane ends with
// the same bits (each step combines two equal-structured partials with a
// commutative operation).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return __builtin_amdgcn_update_dpp(0u, v, CTRL, 0xF, 0xF, false);
}

template <class F>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, F op) {
  v = op(v, dpp<0xB1>(v));   // quad_perm [1,0,3,2]
  v = op(v, dpp<0x4E>(v));   // quad_perm [2,3,0,1]
  v = op(v, dpp<0x141>(v));  // row_half_mirror
  v = op(v, dpp<0x140>(v));  // row_mirror
  auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = op(r[0], r[1]);
  auto h = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return op(h[0], h[1]);
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  auto take = [&](uint32_t lo2, uint32_t hi2) {
    const unsigned long long o = ((unsigned long long)hi2 << 32) | lo2;
    const unsigned long long c = ((unsigned long long)hi << 32) | lo;
    const unsigned long long m = o > c ? o : c;
    lo = (uint32_t)m;
    hi = (uint32_t)(m >> 32);
  };
  take(dpp<0xB1>(lo), dpp<0xB1>(hi));
  take(dpp<0x4E>(lo), dpp<0x4E>(hi));
  take(dpp<0x141>(lo), dpp<0x141>(hi));
  take(dpp<0x140>(lo), dpp<0x140>(hi));
  {
    auto rl = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    auto rh = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    lo = rl[0];
    hi = rh[0];
    take(rl[1], rh[1]);
  }
  {
    auto rl = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    auto rh = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    lo = rl[0];
    hi = rh[0];
    take(rl[1], rh[1]);
  }
  return ((unsigned long long)hi << 32) | lo;
}

__device__ __forceinline__ float wave_max(float v) {
  return __uint_as_float(wave_reduce_u32(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  }));
}

__device__ __forceinline__ float wave_sum(float v) {
  return __uint_as_float(wave_reduce_u32(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  }));
}

constexpr int kMaxPerLane = kMaxExperts / kWave;  // 8

// Expert slots per lane a layer of E experts needs, rounded up to a compiled
// variant: 1, 2, 5 (up to 320 experts) or 8.
inline int topk_slots(int E) { return E <= 64 ? 1 : (E <= 128 ? 2 : (E <= 320 ? 5 : kMaxPerLane)); }

// One wave selects for token t.  Expert e lives in lane e % 64, slot e / 64
// (NS slots per lane, NS * 64 >= E).
// The logits are the sum of the ks K-slice partials part[s][t][e], added in
// slice order.  Each round takes the wave-wide largest remaining key; the
// owner lane retires it.  Writes idx[t][j], wout[t][j] (j in descending
// order) and gap[t].
template <int NS>
__device__ __forceinline__ void topk_token(const float* __restrict__ part, int ks,
                                           const float* __restrict__ bias, int bias_mode, int T,
                                           int E, int k, int score, int renorm, float scale, int t,
                                           int32_t* __restrict__ idx, float* __restrict__ wout,
                                           float* __restrict__ gap) {
  const int lane = threadIdx.x & 63;
  float lg[NS], v[NS];
  unsigned long long key[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) v[i] = 0.f;
  // K-slice partial sums, added in slice order; 8 slices of loads in flight
  for (int s0 = 0; s0 < ks; s0 += 8) {
    float ld[8][NS];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const int e = lane + i * kWave;
        ld[u][i] = (s0 + u < ks && e < E) ? part[((size_t)(s0 + u) * T + t) * E + e] : 0.f;
      }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int i = 0; i < NS; ++i) v[i] += ld[u][i];
  }
  // bias of each slot: all loads first (clamped index), then their uses
  float bv[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) bv[i] = 0.f;
  if (bias) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int e = lane + i * kWave;
      bv[i] = bias[e < E ? e : E - 1];
    }
  }
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int e = lane + i * kWave;
    lg[i] = -INFINITY;
    key[i] = 0ull;  // below every real key
    if (e < E) {
      const float b = bv[i];
      const float l = (bias && bias_mode == 0) ? v[i] + b : v[i];
      lg[i] = l;
      key[i] = rank_key((bias && bias_mode == 1) ? l + b : l, e);
    }
  }

  // softmax reference point: the largest logit (selection may use biased scores)
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < NS; ++i) m = fmaxf(m, lg[i]);
  m = wave_max(m);

  float denom = 0.f, kth = 0.f;
  int my_e = 0;
  float my_p = 0.f;
  for (int r = 0; r < k; ++r) {
    unsigned long long best = 0ull;
#pragma unroll
    for (int i = 0; i < NS; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
    // every lane holds the same best: make it scalar
    best = ((unsigned long long)__builtin_amdgcn_readfirstlane((uint32_t)(best >> 32)) << 32) |
           __builtin_amdgcn_readfirstlane((uint32_t)best);
    const int e = (int)(0xffffffffu - (uint32_t)best);
    const int owner = e & 63, slot = e >> 6;
    float l = 0.f;
#pragma unroll
    for (int i = 0; i < NS; ++i)
      if (i == slot) l = lg[i];
    l = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(l), owner));
    if (lane == owner) {
#pragma unroll
      for (int i = 0; i < NS; ++i)
        if (i == slot) key[i] = 0ull;
    }
    const float p = score == 0 ? expf(l - m) : 1.f / (1.f + expf(-l));
    denom += p;
    if (lane == r) {
      my_e = e;
      my_p = p;
    }
    if (r == k - 1) kth = key_score(best);
  }
  unsigned long long nxt = 0ull;
#pragma unroll
  for (int i = 0; i < NS; ++i) nxt = key[i] > nxt ? key[i] : nxt;
  nxt = wave_max_u64(nxt);

  if (!renorm) {
    if (score == 0) {
      float z = 0.f;
#pragma unroll
      for (int i = 0; i < NS; ++i)
        if (lane + i * kWave < E) z += expf(lg[i] - m);
      denom = wave_sum(z);
    } else {
      denom = 1.f;
    }
  }
  if (lane < k) {
    idx[(size_t)t * k + lane] = my_e;
    wout[(size_t)t * k + lane] = my_p * (scale / denom);
  }
  if (lane == 0) gap[t] = nxt ? kth - key_score(nxt) : INFINITY;
}

}  // namespace moe
