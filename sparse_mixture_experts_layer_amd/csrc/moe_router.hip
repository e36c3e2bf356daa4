// Router: logits l = x W_r^T (+ b) in fp32, then per token a wave-level
// softmax / sigmoid score, top-k selection and renormalisation.
//
// Source: llm-atlas "Step-3.5-Flash", table "Champs bruts du config.json"
// (moe_num_experts, moe_top_k, norm_expert_weight, need_fp32_gate,
// use_moe_router_bias, moe_router_activation, moe_router_scaling_factor).
// Readings where the pages are silent: softmax scoring by default, ties broken
// towards the lower expert index, bias added to the logits (or, in
// MOE_BIAS_SELECT mode, to the selection scores only).
//
// Logits: bf16 x bf16 products are exact in fp32 and MFMA accumulates in fp32
// (need_fp32_gate).  fp32 activations are split into bf16 hi + lo first.
#include "moe_common.hpp"
#include "moe_kernels.hpp"

#include <math.h>

namespace moe {
namespace {

// One workgroup: 64 tokens (16 per wave) x (16 * NE) experts x one K slice.
// Experts are on the MFMA A side, tokens on the B side, so each lane ends with
// 4 consecutive experts of one token.
template <bool XF32, int NE>
__global__ __launch_bounds__(256) void router_logits_kernel(const void* __restrict__ xv,
                                                            const uint16_t* __restrict__ wr,
                                                            float* __restrict__ part, int T, int H,
                                                            int E, int kchunk) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t0 = blockIdx.x * 64 + wave * 16;
  if (t0 >= T) return;
  const int e0 = blockIdx.y * (16 * NE);
  const int kbeg = blockIdx.z * kchunk;
  const int tok = t0 + (lane & 15);
  const bool tok_ok = tok < T;
  const int kl = (lane >> 4) * 8;

  f32x4 acc[NE];
#pragma unroll
  for (int n = 0; n < NE; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint16_t* wrow[NE];
  bool wok[NE];
#pragma unroll
  for (int n = 0; n < NE; ++n) {
    const int e = e0 + n * 16 + (lane & 15);
    wok[n] = e < E;
    wrow[n] = wr + (size_t)(wok[n] ? e : 0) * H + kl;
  }

  for (int k = kbeg; k < kbeg + kchunk; k += 32) {
    u32x4 bh = {0, 0, 0, 0}, bl = {0, 0, 0, 0};
    if (XF32) {
      const float* xp = reinterpret_cast<const float*>(xv) + (size_t)tok * H + k + kl;
      if (tok_ok) {
        float v[8];
        u32x4 a0 = load16(xp), a1 = load16(xp + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[i] = __uint_as_float(a0[i]);
          v[4 + i] = __uint_as_float(a1[i]);
        }
        split_f32x8(v, bh, bl);
      }
    } else {
      const uint16_t* xp = reinterpret_cast<const uint16_t*>(xv) + (size_t)tok * H + k + kl;
      if (tok_ok) bh = load16(xp);
    }
#pragma unroll
    for (int n = 0; n < NE; ++n) {
      u32x4 a = {0, 0, 0, 0};
      if (wok[n]) a = load16(wrow[n] + k);
      acc[n] = mfma16(as_bf16x8(a), as_bf16x8(bh), acc[n]);
      if (XF32) acc[n] = mfma16(as_bf16x8(a), as_bf16x8(bl), acc[n]);
    }
  }

  if (!tok_ok) return;
  float* dst = part + ((size_t)blockIdx.z * T + tok) * E;
#pragma unroll
  for (int n = 0; n < NE; ++n) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = e0 + n * 16 + (lane >> 4) * 4 + i;
      if (e < E) dst[e] = acc[n][i];
    }
  }
}

struct Cand {
  float s;   // selection score
  float l;   // logit used for the weight
  int e;     // expert index (E = none)
};

__device__ __forceinline__ bool better(const Cand& a, const Cand& b) {
  // a ranks before b: larger score, ties to the lower index; "none" never wins.
  if (a.e < 0x7fffffff && b.e == 0x7fffffff) return true;
  if (a.e == 0x7fffffff) return false;
  return a.s > b.s || (a.s == b.s && a.e < b.e);
}

__device__ __forceinline__ Cand shfl_xor(const Cand& c, int m) {
  Cand o;
  o.s = __shfl_xor(c.s, m);
  o.l = __shfl_xor(c.l, m);
  o.e = __shfl_xor(c.e, m);
  return o;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

constexpr int kMaxPerLane = kMaxExperts / kWave;  // 8

// One wave per token.  Expert e lives in lane e % 64, slot e / 64.
__global__ __launch_bounds__(256) void router_topk_kernel(
    const float* __restrict__ part, int ks, const float* __restrict__ bias, int bias_mode, int T,
    int E, int k, int score, int renorm, float scale, int32_t* __restrict__ idx,
    float* __restrict__ wout, float* __restrict__ gap) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  const int none = 0x7fffffff;

  float lg[kMaxPerLane], sc[kMaxPerLane];
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = lane + i * kWave;
    lg[i] = -INFINITY;
    sc[i] = -INFINITY;
    if (e < E) {
      float v = 0.f;
      for (int s = 0; s < ks; ++s) v += part[((size_t)s * T + t) * E + e];
      const float b = bias ? bias[e] : 0.f;
      float l = (bias && bias_mode == 0) ? v + b : v;
      float sel = (bias && bias_mode == 1) ? l + b : l;
      if (sel != sel) sel = -INFINITY;  // NaN never outranks a number
      lg[i] = l;
      sc[i] = sel;
    }
  }

  int win_e[kMaxTopK + 1];
  float win_l[kMaxTopK + 1];
  float kth = 0.f, next = -INFINITY;
  bool have_next = false;
#pragma unroll
  for (int r = 0; r <= kMaxTopK; ++r) {
    if (r > k) continue;
    Cand best{-INFINITY, 0.f, none};
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int e = lane + i * kWave;
      if (e < E && !((taken >> i) & 1u)) {
        Cand c{sc[i], lg[i], e};
        if (better(c, best)) best = c;
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      Cand o = shfl_xor(best, m);
      if (better(o, best)) best = o;
    }
    if (r < k) {
      // k <= E guarantees a candidate; guard anyway so indices stay in range.
      const int e = best.e == none ? 0 : best.e;
      win_e[r] = e;
      win_l[r] = best.l;
      if (r == k - 1) kth = best.s;
      if ((e & 63) == lane) taken |= 1u << (e >> 6);
    } else if (best.e != none) {
      next = best.s;
      have_next = true;
    }
  }

  // weights
  float wsel[kMaxTopK];
  float denom = 0.f;
  if (score == 0) {  // softmax
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) m = fmaxf(m, lg[i]);
    m = wave_max(m);
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      wsel[j] = 0.f;
      if (j < k) {
        wsel[j] = expf(win_l[j] - m);
        if (renorm) denom += wsel[j];
      }
    }
    if (!renorm) {
      float z = 0.f;
#pragma unroll
      for (int i = 0; i < kMaxPerLane; ++i)
        if (lane + i * kWave < E) z += expf(lg[i] - m);
      denom = wave_sum(z);
    }
  } else {  // sigmoid
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      wsel[j] = 0.f;
      if (j < k) {
        wsel[j] = 1.f / (1.f + expf(-win_l[j]));
        denom += wsel[j];
      }
    }
    if (!renorm) denom = 1.f;
  }
  const float inv = scale / denom;
  if (lane < k) {
    // select this lane's entry without dynamic register indexing
    int e = 0;
    float wv = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
      if (j < k && j == lane) {
        e = win_e[j];
        wv = wsel[j] * inv;
      }
    idx[(size_t)t * k + lane] = e;
    wout[(size_t)t * k + lane] = wv;
  }
  if (lane == 0) gap[t] = have_next ? kth - next : INFINITY;
}

}  // namespace

hipError_t launch_router_logits(bool x_f32, const void* x, const uint16_t* router_w, float* part,
                                int T, int H, int E, int ks, hipStream_t s) {
  const int kchunk = H / ks;
  const int ne = E <= 16 ? 1 : (E <= 32 ? 2 : 6);
  dim3 grid((T + 63) / 64, (E + 16 * ne - 1) / (16 * ne), ks);
  dim3 block(256);
#define MOE_ROUTER_CASE(XF, NE_)                                                             \
  hipLaunchKernelGGL((router_logits_kernel<XF, NE_>), grid, block, 0, s, x, router_w, part, T, \
                     H, E, kchunk)
  if (x_f32) {
    if (ne == 1) MOE_ROUTER_CASE(true, 1);
    else if (ne == 2) MOE_ROUTER_CASE(true, 2);
    else MOE_ROUTER_CASE(true, 6);
  } else {
    if (ne == 1) MOE_ROUTER_CASE(false, 1);
    else if (ne == 2) MOE_ROUTER_CASE(false, 2);
    else MOE_ROUTER_CASE(false, 6);
  }
#undef MOE_ROUTER_CASE
  return hipGetLastError();
}

hipError_t launch_router_topk(const float* part, int ks, const float* bias, int bias_mode, int T,
                              int E, int k, int score, int renorm, float scale, int32_t* idx,
                              float* w, float* gap, hipStream_t s) {
  dim3 grid((T + 3) / 4), block(256);
  hipLaunchKernelGGL(router_topk_kernel, grid, block, 0, s, part, ks, bias, bias_mode, T, E, k,
                     score, renorm, scale, idx, w, gap);
  return hipGetLastError();
}

}  // namespace moe
