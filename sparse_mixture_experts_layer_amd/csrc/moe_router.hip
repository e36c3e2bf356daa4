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
#include "moe_topk.hpp"

#include <math.h>

namespace moe {
namespace {

// Small batches: a workgroup computes 16*NT tokens x 16 experts over one K
// slice, which its 4 waves split in 4 and add up through LDS.  Tokens are the
// MFMA A operand and router rows the B operand, so a lane ends with one expert
// column of 4 token rows per token group.  At these sizes the kernel is a
// chain of memory latencies, so a wave issues the loads of up to kBatch
// k-steps before their MFMAs, every load unconditional (rows past T or E read
// row 0; their results are never stored).
template <bool XF32, int NT>
__global__ __launch_bounds__(256) void router_logits_kernel(const void* __restrict__ xv,
                                                            const uint16_t* __restrict__ wr,
                                                            float* __restrict__ part, int T, int H,
                                                            int E, int kchunk,
                                                            int32_t* __restrict__ done) {
  constexpr int kBatch = 4;
  __shared__ f32x4 red[3][NT][kWave];
  if (done && blockIdx.x + blockIdx.y + blockIdx.z + threadIdx.x == 0) *done = 0;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t0 = blockIdx.x * 16 * NT;
  const int e0 = blockIdx.y * 16;
  // this wave's k-steps: [s0, s1) of the slice's kchunk / 32
  const int nst = kchunk / 32, q = (nst + 3) / 4;
  const int s0 = min(nst, wave * q), s1 = min(nst, s0 + q);
  const int kl = (lane >> 4) * 8;
  const int kb = blockIdx.z * kchunk + kl;

  size_t xoff[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int tok = t0 + t * 16 + (lane & 15);
    xoff[t] = (size_t)(tok < T ? tok : 0) * H + kb;
  }
  const int e = e0 + (lane & 15);
  const uint16_t* wrow = wr + (size_t)(e < E ? e : 0) * H + kb;
  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int sb = s0; sb < s1; sb += kBatch) {
    u32x4 b[kBatch], a0[kBatch][NT], a1[kBatch][NT];
#pragma unroll
    for (int d = 0; d < kBatch; ++d) {
      const int k = 32 * min(sb + d, s1 - 1);  // past the end: reload the last step
      b[d] = load16(wrow + k);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (XF32) {
          const float* xp = reinterpret_cast<const float*>(xv) + xoff[t] + k;
          a0[d][t] = load16(xp);
          a1[d][t] = load16(xp + 4);
        } else {
          a0[d][t] = load16(reinterpret_cast<const uint16_t*>(xv) + xoff[t] + k);
        }
      }
    }
    // steps past the end contribute 0 x 0 (selected, not branched around:
    // a branch would let the compiler sink their loads behind the MFMAs)
#pragma unroll
    for (int d = 1; d < kBatch; ++d) {
      if (sb + d >= s1) {
        b[d] = u32x4{0, 0, 0, 0};
#pragma unroll
        for (int t = 0; t < NT; ++t) a0[d][t] = a1[d][t] = u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int d = 0; d < kBatch; ++d) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        u32x4 ah, al;
        if (XF32) {
          float v[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v[i] = __uint_as_float(a0[d][t][i]);
            v[4 + i] = __uint_as_float(a1[d][t][i]);
          }
          split_f32x8(v, ah, al);
          acc[t] = mfma16(as_bf16x8(ah), as_bf16x8(b[d]), acc[t]);
          acc[t] = mfma16(as_bf16x8(al), as_bf16x8(b[d]), acc[t]);
        } else {
          acc[t] = mfma16(as_bf16x8(a0[d][t]), as_bf16x8(b[d]), acc[t]);
        }
      }
    }
  }

  // waves 1-3 hand their sums to wave 0, which adds them in wave order
  if (wave > 0) {
#pragma unroll
    for (int t = 0; t < NT; ++t) red[wave - 1][t][lane] = acc[t];
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const f32x4 o = red[w][t][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[t][i] += o[i];
    }
  if (e >= E) return;
  float* dst = part + (size_t)blockIdx.z * T * E;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = t0 + t * 16 + (lane >> 4) * 4 + i;
      if (tok < T) dst[(size_t)tok * E + e] = acc[t][i];
    }
}

// Large batches, bf16 x: a workgroup of NW waves covers 16*NT tokens and
// NW*16*NE experts (all 288 with NT=4, NE=6, NW=3), so per k-step a wave loads
// NT + NE fragments for NT*NE MFMAs (the NT x fragments are shared by the
// workgroup's waves through L1).  The loads of step k+32 are issued before
// the MFMAs of step k.  Rows past T or E read row 0; their results are never
// stored.  kchunk / 32 must be even.
template <int NT, int NE, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2))) void router_logits_wide_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, float* __restrict__ part,
    int T, int H, int E, int kchunk, int32_t* __restrict__ done) {
  if (done && blockIdx.x + blockIdx.y + blockIdx.z + threadIdx.x == 0) *done = 0;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t0 = blockIdx.x * 16 * NT;
  const int e0 = (blockIdx.y * NW + wave) * 16 * NE;
  if (e0 >= E) return;
  const int kbeg = blockIdx.z * kchunk, kend = kbeg + kchunk;
  const int kl = (lane >> 4) * 8;
  const uint16_t* xrow[NT];
  const uint16_t* wrow[NE];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int tok = t0 + t * 16 + (lane & 15);
    xrow[t] = x + (size_t)(tok < T ? tok : 0) * H + kl;
  }
#pragma unroll
  for (int n = 0; n < NE; ++n) {
    const int e = e0 + n * 16 + (lane & 15);
    wrow[n] = wr + (size_t)(e < E ? e : 0) * H + kl;
  }
  f32x4 acc[NT][NE];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int n = 0; n < NE; ++n) acc[t][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 a0[NT], b0[NE], a1[NT], b1[NE];
  auto load = [&](u32x4(&a)[NT], u32x4(&b)[NE], int k) {
#pragma unroll
    for (int t = 0; t < NT; ++t) a[t] = load16(xrow[t] + k);
#pragma unroll
    for (int n = 0; n < NE; ++n) b[n] = load16(wrow[n] + k);
  };
  auto mma = [&](const u32x4(&a)[NT], const u32x4(&b)[NE]) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int n = 0; n < NE; ++n) acc[t][n] = mfma16(as_bf16x8(a[t]), as_bf16x8(b[n]), acc[t][n]);
  };
  load(a0, b0, kbeg);
  for (int k = kbeg; k < kend; k += 64) {
    load(a1, b1, k + 32);
    mma(a0, b0);
    if (k + 64 < kend) load(a0, b0, k + 64);
    mma(a1, b1);
  }
  float* dst = part + (size_t)blockIdx.z * T * E;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int n = 0; n < NE; ++n) {
      const int e = e0 + n * 16 + (lane & 15);
      if (e >= E) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = t0 + t * 16 + (lane >> 4) * 4 + i;
        if (tok < T) dst[(size_t)tok * E + e] = acc[t][n][i];
      }
    }
}

// One wave per token.
__global__ __launch_bounds__(256) void router_topk_kernel(
    const float* __restrict__ part, int ks, const float* __restrict__ bias, int bias_mode, int T,
    int E, int k, int score, int renorm, float scale, int32_t* __restrict__ idx,
    float* __restrict__ wout, float* __restrict__ gap) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  topk_token(part, ks, bias, bias_mode, T, E, k, score, renorm, scale, t, idx, wout, gap);
}

}  // namespace

// Launch shape of the logits kernel for a batch: 16*nt tokens x 16*ne*nw
// experts per workgroup.
namespace {
struct RouterShape {
  int nt, ne, nw;
  bool wide;
};
RouterShape router_shape(bool x_f32, int T, int ksteps) {
  if (!x_f32 && T > 256 && ksteps % 2 == 0) return {4, 6, 3, true};
  return {T <= 32 ? 2 : 4, 1, 1, false};
}
}  // namespace

int router_blocks(bool x_f32, int T, int E) {
  const RouterShape r = router_shape(x_f32, T, 2);
  return ((T + 16 * r.nt - 1) / (16 * r.nt)) * ((E + 16 * r.ne * r.nw - 1) / (16 * r.ne * r.nw));
}

hipError_t launch_router_logits(bool x_f32, const void* x, const uint16_t* router_w, float* part,
                                int T, int H, int E, int ks, int32_t* done, hipStream_t s) {
  const int kchunk = H / ks;
  // the wide kernel takes an even number of 32-wide k-steps per slice
  const RouterShape r = router_shape(x_f32, T, kchunk / 32);
  dim3 grid((T + 16 * r.nt - 1) / (16 * r.nt), (E + 16 * r.ne * r.nw - 1) / (16 * r.ne * r.nw), ks);
  if (r.wide) {
    hipLaunchKernelGGL((router_logits_wide_kernel<4, 6, 3>), grid, dim3(64 * 3), 0, s,
                       static_cast<const uint16_t*>(x), router_w, part, T, H, E, kchunk, done);
    return hipGetLastError();
  }
  dim3 block(256);
#define MOE_ROUTER_CASE(XF, NT_)                                                              \
  hipLaunchKernelGGL((router_logits_kernel<XF, NT_>), grid, block, 0, s, x, router_w, part, T, H, \
                     E, kchunk, done)
  if (x_f32) {
    if (r.nt == 2) MOE_ROUTER_CASE(true, 2);
    else MOE_ROUTER_CASE(true, 4);
  } else {
    if (r.nt == 2) MOE_ROUTER_CASE(false, 2);
    else MOE_ROUTER_CASE(false, 4);
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
