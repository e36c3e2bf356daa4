// Router: logits l = x W_r^T (+ b) in fp32, as K-slice partial sums; the
// per-token softmax / sigmoid score, top-k selection and renormalisation
// (moe_topk.hpp) run here for batches over 1024 tokens and inside the
// dispatch launch below that.
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
#include "moe_lds.hpp"
#include "moe_topk.hpp"

#include <math.h>

namespace moe {
namespace {

// Up to 640 tokens (or fp32 x): a workgroup computes 16*NT tokens x 16 experts over one K
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
                                                            int32_t* __restrict__ done,
                                                            int32_t* __restrict__ dbg) {
  constexpr int kBatch = 4;
  __shared__ f32x4 red[3][NT][kWave];
  if (blockIdx.x + blockIdx.y + blockIdx.z + threadIdx.x == 0) {
    if (done) *done = 0;
    if (dbg) dbg[0] = dbg[1] = 0;
  }
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

// Batches over 640 tokens, bf16 x: LDS-staged tiles of 256 tokens x 288 experts (all
// of Step-3.5-Flash's router) over one K slice, so each router row is fetched
// once per 256 tokens instead of once per 64.  8 waves, wave (wt, we) = (wave
// % 4, wave / 4) owns tokens 64*wt .. +63 and experts 144*we .. +143 (4 x 9
// fragments of 16x16, 144 fp32 accumulators per lane).  K advances 32 per
// step through a 3-slot LDS ring: 16 x fragments and 18 router fragments of
// 1 KiB, written by wave-wide global->LDS loads (every wave loads 2 x and 3
// router fragments; waves 6-7 fill 6 spare slots with row 0, so that every
// wave has the same wait counts); two steps stay in flight and the next
// step's fragments are read into registers during the current MFMAs.  Rows
// past T or E read a valid row; their results are never stored.
constexpr int kRlTokens = 256, kRlExperts = 288;
constexpr int kRlAFrags = kRlTokens / 16, kRlBFrags = kRlExperts / 16;  // 16, 18
constexpr int kRlBSlots = 24;                                            // 3 per wave
constexpr int kRlStage = (kRlAFrags + kRlBSlots) * kFragBytes;          // 40 KiB
constexpr int kRlStages = 3;

__global__ __launch_bounds__(512, 1) void router_logits_lds_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, float* __restrict__ part,
    int T, int H, int E, int kchunk, int32_t* __restrict__ done, int32_t* __restrict__ dbg) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kRlStages * kRlStage];
  if (blockIdx.x + blockIdx.y + blockIdx.z + threadIdx.x == 0) {
    if (done) *done = 0;
    if (dbg) dbg[0] = dbg[1] = 0;
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wt = wave & 3, we = wave >> 2;
  const int t0 = blockIdx.x * kRlTokens, e0 = blockIdx.y * kRlExperts;
  const int kbeg = blockIdx.z * kchunk, nk = kchunk / 32;
  const int kl = (lane >> 4) * 8;
  // this wave's loads per step: x fragments 2*wave, 2*wave+1; router
  // fragments (or spare slots) 3*wave .. 3*wave+2
  constexpr int per_step = 5;
  const uint16_t* a0p;
  const uint16_t* a1p;
  {
    int r0 = t0 + (2 * wave) * 16 + (lane & 15), r1 = r0 + 16;
    r0 = r0 < T ? r0 : 0;
    r1 = r1 < T ? r1 : 0;
    a0p = x + (size_t)r0 * H + kbeg + kl;
    a1p = x + (size_t)r1 * H + kbeg + kl;
  }
  const uint16_t* bp[3];
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    int e = e0 + (3 * wave + q) * 16 + (lane & 15);
    e = (3 * wave + q < kRlBFrags && e < E) ? e : 0;
    bp[q] = wr + (size_t)e * H + kbeg + kl;
  }
  auto issue = [&](int kk, int slot) {
    uint8_t* st = lds + slot * kRlStage;
    uint8_t* la = st + 2 * wave * kFragBytes;
    load_frag<0>(a0p + (size_t)kk * 32, la);
    load_frag<kFragBytes>(reinterpret_cast<const uint8_t*>(a1p + (size_t)kk * 32) - kFragBytes, la);
    uint8_t* lb = st + (kRlAFrags + 3 * wave) * kFragBytes;
    load_frag<0>(bp[0] + (size_t)kk * 32, lb);
    load_frag<kFragBytes>(reinterpret_cast<const uint8_t*>(bp[1] + (size_t)kk * 32) - kFragBytes, lb);
    load_frag<2 * kFragBytes>(
        reinterpret_cast<const uint8_t*>(bp[2] + (size_t)kk * 32) - 2 * kFragBytes, lb);
  };
  auto rd_a = [&](int kk, int m) {
    return as_bf16x8(*reinterpret_cast<const u32x4*>(lds + (kk % kRlStages) * kRlStage +
                                                     (4 * wt + m) * kFragBytes + lane * 16));
  };
  auto rd_b = [&](int kk, int j) {
    return as_bf16x8(*reinterpret_cast<const u32x4*>(
        lds + (kk % kRlStages) * kRlStage + (kRlAFrags + 9 * we + j) * kFragBytes + lane * 16));
  };

  f32x4 acc[4][9];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int j = 0; j < 9; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 a0[4], a1[4], b[9];
  // step kk: wait for step kk+1's loads (own: vmcnt, everyone's: barrier),
  // refill the slot of step kk (already in registers) with step kk+3, then
  // the MFMAs of step kk while step kk+1 is read into registers
  auto step = [&](int kk, bf16x8(&ca)[4], bf16x8(&na)[4], bool do_issue, bool do_read, int vm) {
    wait_vm_lgkm0(vm);
    barrier();
    if (do_issue) issue(kk + kRlStages, kk % kRlStages);
#pragma unroll
    for (int j = 0; j < 9; ++j) {
#pragma unroll
      for (int m = 0; m < 4; ++m) acc[m][j] = mfma16(ca[m], b[j], acc[m][j]);
      if (do_read) {
        b[j] = rd_b(kk + 1, j);
        if (j < 4) na[j] = rd_a(kk + 1, j);
      }
    }
  };
  const int pro = nk < kRlStages ? nk : kRlStages;
  for (int s = 0; s < pro; ++s) issue(s, s);
  wait_vm_lgkm0((pro - 1) * per_step);
  barrier();
#pragma unroll
  for (int m = 0; m < 4; ++m) a0[m] = rd_a(0, m);
#pragma unroll
  for (int j = 0; j < 9; ++j) b[j] = rd_b(0, j);
  // loads issued after step kk+1's that may still be in flight at step kk
  auto vm_at = [&](int kk) { return kk + 2 < nk ? per_step : 0; };
  int kk = 0;
  for (; kk + kRlStages + 1 < nk; kk += 2) {
    step(kk, a0, a1, true, true, per_step);
    step(kk + 1, a1, a0, true, true, per_step);
  }
  for (; kk < nk; kk += 2) {
    step(kk, a0, a1, kk + kRlStages < nk, kk + 1 < nk, vm_at(kk));
    if (kk + 1 < nk) step(kk + 1, a1, a0, kk + 1 + kRlStages < nk, kk + 2 < nk, vm_at(kk + 1));
  }

  float* dst = part + (size_t)blockIdx.z * T * E;
#pragma unroll
  for (int j = 0; j < 9; ++j) {
    const int e = e0 + (9 * we + j) * 16 + (lane & 15);
    if (e >= E) continue;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = t0 + 64 * wt + 16 * m + (lane >> 4) * 4 + i;
        if (tok < T) dst[(size_t)tok * E + e] = acc[m][j][i];
      }
  }
}

// One wave per token.
template <int NS>
__global__ __launch_bounds__(256) void router_topk_kernel(
    const float* __restrict__ part, int ks, const float* __restrict__ bias, int bias_mode, int T,
    int E, int k, int score, int renorm, float scale, int32_t* __restrict__ idx,
    float* __restrict__ wout, float* __restrict__ gap) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  topk_token<NS>(part, ks, bias, bias_mode, T, E, k, score, renorm, scale, t, idx, wout, gap);
}

}  // namespace

// Launch shape of the logits kernel for a batch: 16*nt tokens x 16*ne*nw
// experts per workgroup.
namespace {
struct RouterShape {
  int nt, ne, nw;
  bool lds;  // router_logits_lds_kernel
};
RouterShape router_shape(bool x_f32, int T) {
  // the LDS-staged tiles pay off once a few of them fill the GPU: measured
  // behind the small-batch kernel at 384-512 tokens, ahead from 1024
  if (!x_f32 && T > 640) return {kRlTokens / 16, kRlExperts / 16, 1, true};
  return {T <= 32 ? 2 : 4, 1, 1, false};
}
}  // namespace

int router_blocks(bool x_f32, int T, int E) {
  const RouterShape r = router_shape(x_f32, T);
  return ((T + 16 * r.nt - 1) / (16 * r.nt)) * ((E + 16 * r.ne * r.nw - 1) / (16 * r.ne * r.nw));
}

hipError_t launch_router_logits(bool x_f32, const void* x, const uint16_t* router_w, float* part,
                                int T, int H, int E, int ks, int32_t* done, int32_t* dbg,
                                hipStream_t s) {
  const int kchunk = H / ks;
  const RouterShape r = router_shape(x_f32, T);
  dim3 grid((T + 16 * r.nt - 1) / (16 * r.nt), (E + 16 * r.ne * r.nw - 1) / (16 * r.ne * r.nw), ks);
  if (r.lds) {
    hipLaunchKernelGGL(router_logits_lds_kernel, grid, dim3(512), 0, s,
                       static_cast<const uint16_t*>(x), router_w, part, T, H, E, kchunk, done, dbg);
    return hipGetLastError();
  }
  dim3 block(256);
#define MOE_ROUTER_CASE(XF, NT_)                                                              \
  hipLaunchKernelGGL((router_logits_kernel<XF, NT_>), grid, block, 0, s, x, router_w, part, T, H, \
                     E, kchunk, done, dbg)
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
#define MOE_RT(NS)                                                                               \
  hipLaunchKernelGGL((router_topk_kernel<NS>), grid, block, 0, s, part, ks, bias, bias_mode, T, E, \
                     k, score, renorm, scale, idx, w, gap)
  switch (topk_slots(E)) {
    case 1: MOE_RT(1); break;
    case 2: MOE_RT(2); break;
    case 5: MOE_RT(5); break;
    default: MOE_RT(kMaxPerLane);
  }
#undef MOE_RT
  return hipGetLastError();
}

}  // namespace moe
