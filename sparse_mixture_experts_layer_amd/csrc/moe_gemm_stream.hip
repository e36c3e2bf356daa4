// Grouped expert GEMMs that stream the packed weights once per tile:
//   gate/up:  h[r][f] = silu(sum_k x[tok(r)][k] Wg[f][k]) * (sum_k x[tok(r)][k] Wu[f][k])
//   down:     Y[r][n] = sum_f h[r][f] Wd[n][f]          (fp32 out)
// for every permuted row r of every expert group (the shared expert is the
// last group, over all tokens).  Expert FFN shape: llm-atlas "Step-3.5-Flash",
// "Champs bruts du config.json" (moe_intermediate_size, share_expert_dim);
// SiLU gating is the reading taken for the swiglu fields, whose limit is 0
// (no clamp) on every MoE layer.
//
// Work unit: one tile of up to 16*TG rows of one group x 64 output features
// (4 waves x 16).  Weights are the MFMA A operand (their rows land on C rows),
// the tile's rows the B operand, so the weight stream is one 1 KiB coalesced
// fragment per wave per 32-k step no matter how few tokens an expert has -- the
// decode regime, where nearly every byte moved is an expert weight.  Weight
// fragments are prefetched a group of U steps ahead (double buffer).
//
// INT4 (group 32): each lane's 16 bytes hold 4 k-groups x 8 nibbles of one
// row; they widen to exact bf16 values 136+q, one MFMA against -136 per
// k-group removes the offset, and each group's fp32 partial is multiplied by
// its fp16 scale before it joins the accumulator, so the only rounding beyond
// the fp32 sums is none: s*q is never formed in a narrower type.
#include "moe_common.hpp"
#include "moe_kernels.hpp"

namespace moe {
namespace {

// B operand source: bf16 rows (one 16-byte load per 32-k step) or fp32 rows
// (two loads, split into bf16 hi + lo and issued as two MFMAs).
template <bool F32>
struct BRow {
  static constexpr int kLoads = F32 ? 2 : 1;
  u32x4 v[kLoads];
  __device__ __forceinline__ void load(const void* base, size_t elem_off, bool ok) {
    if (F32) {
      const float* p = reinterpret_cast<const float*>(base) + elem_off;
      v[0] = ok ? load16(p) : u32x4{0, 0, 0, 0};
      v[kLoads - 1] = ok ? load16(p + 4) : u32x4{0, 0, 0, 0};
    } else {
      const uint16_t* p = reinterpret_cast<const uint16_t*>(base) + elem_off;
      v[0] = ok ? load16(p) : u32x4{0, 0, 0, 0};
    }
  }
  __device__ __forceinline__ void operands(bf16x8& hi, bf16x8& lo) const {
    if (F32) {
      float f[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[i] = __uint_as_float(v[0][i]);
        f[4 + i] = __uint_as_float(v[kLoads - 1][i]);
      }
      u32x4 h, l;
      split_f32x8(f, h, l);
      hi = as_bf16x8(h);
      lo = as_bf16x8(l);
    } else {
      hi = as_bf16x8(v[0]);
      lo = hi;
    }
  }
};

template <bool F32>
__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 bhi, bf16x8 blo, f32x4 c) {
  c = mfma16(a, bhi, c);
  if (F32) c = mfma16(a, blo, c);
  return c;
}

struct TileInfo {
  int group, row0, nrows, width;
};

__device__ __forceinline__ bool tile_info(const GemmGeom& g, int tile, TileInfo& ti) {
  if (tile >= *g.ntiles) return false;
  const int v = g.tiles[tile];
  ti.group = tile_group(v);
  const int bm = 16 * g.tg;
  const int m = tile_m(v);
  ti.row0 = g.offsets[ti.group] + m * bm;
  ti.nrows = min(bm, g.counts[ti.group] - m * bm);
  ti.width = ti.group == g.E ? g.Is : g.I;
  return ti.nrows > 0;
}

// ------------------------------------------------------------------ bf16 gate/up
template <bool F32, int TG, int U>
__global__ __launch_bounds__(256) void gateup_bf16_kernel(GemmGeom g, const void* __restrict__ x,
                                                          const int32_t* __restrict__ row_tok,
                                                          int T, float* __restrict__ hout,
                                                          int hstride, int nblk) {
  const int tile = blockIdx.x / nblk, nb = blockIdx.x % nblk;
  TileInfo ti;
  if (!tile_info(g, tile, ti)) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int f0 = nb * 64 + wave * 16;
  if (f0 >= ti.width) return;
  const int H = g.H, nk = H / 32;
  const uint8_t* wp = g.packed + (size_t)ti.group * g.expert_bytes +
                      (size_t)(f0 / 16) * nk * 2 * kFragBytes + lane * 16;

  size_t xoff[TG];
  bool ok[TG];
#pragma unroll
  for (int t = 0; t < TG; ++t) {
    const int r = t * 16 + (lane & 15);
    ok[t] = r < ti.nrows;
    int tok = ok[t] ? row_tok[ti.row0 + r] : 0;
    tok = tok < 0 ? 0 : (tok >= T ? T - 1 : tok);
    xoff[t] = (size_t)tok * H + (lane >> 4) * 8;
  }

  f32x4 accg[TG], accu[TG];
#pragma unroll
  for (int t = 0; t < TG; ++t) accg[t] = accu[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 wa[U][2], wn[U][2];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    wa[u][0] = load16_stream(wp + (size_t)u * 2 * kFragBytes);
    wa[u][1] = load16_stream(wp + (size_t)u * 2 * kFragBytes + kFragBytes);
  }
  for (int k0 = 0; k0 < nk; k0 += U) {
    BRow<F32> b[U][TG];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < TG; ++t) b[u][t].load(x, xoff[t] + (size_t)(k0 + u) * 32, ok[t]);
    const bool more = k0 + U < nk;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (more) {
        wn[u][0] = load16_stream(wp + (size_t)(k0 + U + u) * 2 * kFragBytes);
        wn[u][1] = load16_stream(wp + (size_t)(k0 + U + u) * 2 * kFragBytes + kFragBytes);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int t = 0; t < TG; ++t) {
        bf16x8 bh, bl;
        b[u][t].operands(bh, bl);
        accg[t] = mma<F32>(as_bf16x8(wa[u][0]), bh, bl, accg[t]);
        accu[t] = mma<F32>(as_bf16x8(wa[u][1]), bh, bl, accu[t]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      wa[u][0] = wn[u][0];
      wa[u][1] = wn[u][1];
    }
  }

  // epilogue: lane holds features f0 + 4*(lane/16) + i of row (lane % 16)
#pragma unroll
  for (int t = 0; t < TG; ++t) {
    if (!ok[t]) continue;
    const size_t row = (size_t)ti.row0 + t * 16 + (lane & 15);
    const int f = f0 + (lane >> 4) * 4;
    f32x4 hv;
#pragma unroll
    for (int i = 0; i < 4; ++i) hv[i] = silu(accg[t][i]) * accu[t][i];
    *reinterpret_cast<f32x4*>(hout + row * hstride + f) = hv;
  }
}

// ------------------------------------------------------------------ bf16 down
template <int TG, int U>
__global__ __launch_bounds__(256) void down_bf16_kernel(GemmGeom g, const float* __restrict__ h,
                                                        int hstride, float* __restrict__ y,
                                                        int nblk) {
  const int tile = blockIdx.x / nblk, nb = blockIdx.x % nblk;
  TileInfo ti;
  if (!tile_info(g, tile, ti)) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = nb * 64 + wave * 16;
  const int H = g.H;
  if (n0 >= H) return;
  const int K = ti.width, nk = K / 32;
  const uint8_t* wp = g.packed + (size_t)ti.group * g.expert_bytes +
                      (size_t)2 * ti.width * H * 2 + (size_t)(n0 / 16) * nk * kFragBytes +
                      lane * 16;

  size_t hoff[TG];
  bool ok[TG];
#pragma unroll
  for (int t = 0; t < TG; ++t) {
    const int r = t * 16 + (lane & 15);
    ok[t] = r < ti.nrows;
    hoff[t] = (size_t)(ti.row0 + (ok[t] ? r : 0)) * hstride + (lane >> 4) * 8;
  }
  f32x4 acc[TG];
#pragma unroll
  for (int t = 0; t < TG; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 wa[U], wn[U];
#pragma unroll
  for (int u = 0; u < U; ++u) wa[u] = load16_stream(wp + (size_t)u * kFragBytes);
  for (int k0 = 0; k0 < nk; k0 += U) {
    BRow<true> b[U][TG];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < TG; ++t) b[u][t].load(h, hoff[t] + (size_t)(k0 + u) * 32, ok[t]);
    const bool more = k0 + U < nk;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (more) wn[u] = load16_stream(wp + (size_t)(k0 + U + u) * kFragBytes);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < TG; ++t) {
        bf16x8 bh, bl;
        b[u][t].operands(bh, bl);
        acc[t] = mma<true>(as_bf16x8(wa[u]), bh, bl, acc[t]);
      }
#pragma unroll
    for (int u = 0; u < U; ++u) wa[u] = wn[u];
  }

#pragma unroll
  for (int t = 0; t < TG; ++t) {
    if (!ok[t]) continue;
    const size_t row = (size_t)ti.row0 + t * 16 + (lane & 15);
    float* yp = y + row * H + n0 + (lane >> 4) * 4;
    *reinterpret_cast<f32x4*>(yp) = acc[t];
  }
}

// ------------------------------------------------------------------ INT4 helpers
// Packed INT4 region of one group of width W (rows of gate/up = W, of down = H):
//   gate/up q      [W/16][H/128][2][64][16 B]          W*H bytes
//   gate/up scales [W/16][H/128][2][4 quads][4 kg][4]  W*H/8 bytes (fp16)
//   down q         [H/16][W/128][64][16 B]              H*W/2 bytes
//   down scales    [H/16][W/128][4][4][4]               H*W/16 bytes
__device__ __forceinline__ void load_scales(const uint8_t* p, float s[4][4]) {
  const u32x4 a = load16_stream(p), b = load16_stream(p + 16);
  const uint32_t w[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
  for (int kg = 0; kg < 4; ++kg)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t word = w[(kg * 4 + i) >> 1];
      const uint16_t bits = (uint16_t)(((kg * 4 + i) & 1) ? (word >> 16) : (word & 0xffff));
      s[kg][i] = (float)__builtin_bit_cast(_Float16, bits);
    }
}

constexpr uint32_t kMinus136x2 = 0xC308C308u;  // bf16 -136 in both halves

template <bool F32, int TG>
__device__ __forceinline__ void int4_group_step(const u32x4& qa, const float (&sc)[4][4],
                                                const BRow<F32> (&b)[4][TG], f32x4 (&acc)[TG],
                                                int kg) {
  const bf16x8 m136 = as_bf16x8(u32x4{kMinus136x2, kMinus136x2, kMinus136x2, kMinus136x2});
  const bf16x8 a = int4_to_bf16x8_biased(qa[kg]);
#pragma unroll
  for (int t = 0; t < TG; ++t) {
    bf16x8 bh, bl;
    b[kg][t].operands(bh, bl);
    f32x4 p = mma<F32>(m136, bh, bl, f32x4{0.f, 0.f, 0.f, 0.f});
    p = mma<F32>(a, bh, bl, p);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[t][i] += sc[kg][i] * p[i];
  }
}

// ------------------------------------------------------------------ INT4 gate/up
template <bool F32, int TG>
__global__ __launch_bounds__(256) void gateup_int4_kernel(GemmGeom g, const void* __restrict__ x,
                                                          const int32_t* __restrict__ row_tok,
                                                          int T, float* __restrict__ hout,
                                                          int hstride, int nblk) {
  const int tile = blockIdx.x / nblk, nb = blockIdx.x % nblk;
  TileInfo ti;
  if (!tile_info(g, tile, ti)) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int f0 = nb * 64 + wave * 16;
  if (f0 >= ti.width) return;
  const int H = g.H, nkb = H / 128;
  const uint8_t* base = g.packed + (size_t)ti.group * g.expert_bytes;
  const uint8_t* qp = base + (size_t)(f0 / 16) * nkb * 2 * kFragBytes + lane * 16;
  const uint8_t* sp = base + (size_t)ti.width * H + (size_t)(f0 / 16) * nkb * 2 * 128 +
                      (lane >> 4) * 32;

  size_t xoff[TG];
  bool ok[TG];
#pragma unroll
  for (int t = 0; t < TG; ++t) {
    const int r = t * 16 + (lane & 15);
    ok[t] = r < ti.nrows;
    int tok = ok[t] ? row_tok[ti.row0 + r] : 0;
    tok = tok < 0 ? 0 : (tok >= T ? T - 1 : tok);
    xoff[t] = (size_t)tok * H + (lane >> 4) * 8;
  }
  f32x4 accg[TG], accu[TG];
#pragma unroll
  for (int t = 0; t < TG; ++t) accg[t] = accu[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 qg = load16_stream(qp), qu = load16_stream(qp + kFragBytes);
  float sg[4][4], su[4][4];
  load_scales(sp, sg);
  load_scales(sp + 128, su);
  for (int kb = 0; kb < nkb; ++kb) {
    BRow<F32> b[4][TG];
#pragma unroll
    for (int kg = 0; kg < 4; ++kg)
#pragma unroll
      for (int t = 0; t < TG; ++t) b[kg][t].load(x, xoff[t] + (size_t)kb * 128 + kg * 32, ok[t]);
    u32x4 ng = qg, nu = qu;
    float nsg[4][4], nsu[4][4];
    const bool more = kb + 1 < nkb;
    if (more) {
      ng = load16_stream(qp + (size_t)(kb + 1) * 2 * kFragBytes);
      nu = load16_stream(qp + (size_t)(kb + 1) * 2 * kFragBytes + kFragBytes);
      load_scales(sp + (size_t)(kb + 1) * 256, nsg);
      load_scales(sp + (size_t)(kb + 1) * 256 + 128, nsu);
    }
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
      int4_group_step<F32, TG>(qg, sg, b, accg, kg);
      int4_group_step<F32, TG>(qu, su, b, accu, kg);
    }
    if (more) {
      qg = ng;
      qu = nu;
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sg[a][i] = nsg[a][i];
          su[a][i] = nsu[a][i];
        }
    }
  }

#pragma unroll
  for (int t = 0; t < TG; ++t) {
    if (!ok[t]) continue;
    const size_t row = (size_t)ti.row0 + t * 16 + (lane & 15);
    const int f = f0 + (lane >> 4) * 4;
    f32x4 hv;
#pragma unroll
    for (int i = 0; i < 4; ++i) hv[i] = silu(accg[t][i]) * accu[t][i];
    *reinterpret_cast<f32x4*>(hout + row * hstride + f) = hv;
  }
}

// ------------------------------------------------------------------ INT4 down
template <int TG>
__global__ __launch_bounds__(256) void down_int4_kernel(GemmGeom g, const float* __restrict__ h,
                                                        int hstride, float* __restrict__ y,
                                                        int nblk) {
  const int tile = blockIdx.x / nblk, nb = blockIdx.x % nblk;
  TileInfo ti;
  if (!tile_info(g, tile, ti)) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = nb * 64 + wave * 16;
  const int H = g.H;
  if (n0 >= H) return;
  const int W = ti.width, nkb = W / 128;
  const uint8_t* base = g.packed + (size_t)ti.group * g.expert_bytes + (size_t)W * H +
                        (size_t)W * H / 8;
  const uint8_t* qp = base + (size_t)(n0 / 16) * nkb * kFragBytes + lane * 16;
  const uint8_t* sp = base + (size_t)H * W / 2 + (size_t)(n0 / 16) * nkb * 128 + (lane >> 4) * 32;

  size_t hoff[TG];
  bool ok[TG];
#pragma unroll
  for (int t = 0; t < TG; ++t) {
    const int r = t * 16 + (lane & 15);
    ok[t] = r < ti.nrows;
    hoff[t] = (size_t)(ti.row0 + (ok[t] ? r : 0)) * hstride + (lane >> 4) * 8;
  }
  f32x4 acc[TG];
#pragma unroll
  for (int t = 0; t < TG; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 q = load16_stream(qp);
  float s[4][4];
  load_scales(sp, s);
  for (int kb = 0; kb < nkb; ++kb) {
    BRow<true> b[4][TG];
#pragma unroll
    for (int kg = 0; kg < 4; ++kg)
#pragma unroll
      for (int t = 0; t < TG; ++t) b[kg][t].load(h, hoff[t] + (size_t)kb * 128 + kg * 32, ok[t]);
    u32x4 nq = q;
    float ns[4][4];
    const bool more = kb + 1 < nkb;
    if (more) {
      nq = load16_stream(qp + (size_t)(kb + 1) * kFragBytes);
      load_scales(sp + (size_t)(kb + 1) * 128, ns);
    }
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) int4_group_step<true, TG>(q, s, b, acc, kg);
    if (more) {
      q = nq;
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[a][i] = ns[a][i];
    }
  }

#pragma unroll
  for (int t = 0; t < TG; ++t) {
    if (!ok[t]) continue;
    const size_t row = (size_t)ti.row0 + t * 16 + (lane & 15);
    float* yp = y + row * H + n0 + (lane >> 4) * 4;
    *reinterpret_cast<f32x4*>(yp) = acc[t];
  }
}

template <int TG>
hipError_t gateup_tg(const GemmGeom& g, bool int4, bool f32, const void* x,
                     const int32_t* row_tok, int T, float* h, int hstride, hipStream_t s) {
  const int wmax = g.I > g.Is ? g.I : g.Is;
  const int nblk = (wmax + 63) / 64;
  dim3 grid((unsigned)g.max_tiles * nblk), block(256);
  const int nk = g.H / 32;
  if (int4) {
    if (f32)
      hipLaunchKernelGGL((gateup_int4_kernel<true, TG>), grid, block, 0, s, g, x, row_tok, T, h,
                         hstride, nblk);
    else
      hipLaunchKernelGGL((gateup_int4_kernel<false, TG>), grid, block, 0, s, g, x, row_tok, T, h,
                         hstride, nblk);
  } else if (nk % 4 == 0) {
    if (f32)
      hipLaunchKernelGGL((gateup_bf16_kernel<true, TG, 4>), grid, block, 0, s, g, x, row_tok, T,
                         h, hstride, nblk);
    else
      hipLaunchKernelGGL((gateup_bf16_kernel<false, TG, 4>), grid, block, 0, s, g, x, row_tok, T,
                         h, hstride, nblk);
  } else {
    if (f32)
      hipLaunchKernelGGL((gateup_bf16_kernel<true, TG, 2>), grid, block, 0, s, g, x, row_tok, T,
                         h, hstride, nblk);
    else
      hipLaunchKernelGGL((gateup_bf16_kernel<false, TG, 2>), grid, block, 0, s, g, x, row_tok, T,
                         h, hstride, nblk);
  }
  return hipGetLastError();
}

template <int TG>
hipError_t down_tg(const GemmGeom& g, bool int4, const float* h, int hstride, float* y,
                   hipStream_t s) {
  const int nblk = g.H / 64;
  dim3 grid((unsigned)g.max_tiles * nblk), block(256);
  const int nk_i = g.I / 32, nk_s = g.Is > 0 ? g.Is / 32 : nk_i;
  const bool u4 = nk_i % 4 == 0 && nk_s % 4 == 0;
  if (int4)
    hipLaunchKernelGGL((down_int4_kernel<TG>), grid, block, 0, s, g, h, hstride, y, nblk);
  else if (u4)
    hipLaunchKernelGGL((down_bf16_kernel<TG, 4>), grid, block, 0, s, g, h, hstride, y, nblk);
  else
    hipLaunchKernelGGL((down_bf16_kernel<TG, 1>), grid, block, 0, s, g, h, hstride, y, nblk);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gateup(const GemmGeom& g, bool int4, bool act_f32, const void* x,
                         const int32_t* row_tok, float* h, int hstride, hipStream_t s) {
  const int T = g.T;
  switch (g.tg) {
    case 1: return gateup_tg<1>(g, int4, act_f32, x, row_tok, T, h, hstride, s);
    case 2: return gateup_tg<2>(g, int4, act_f32, x, row_tok, T, h, hstride, s);
    default: return gateup_tg<4>(g, int4, act_f32, x, row_tok, T, h, hstride, s);
  }
}

hipError_t launch_down(const GemmGeom& g, bool int4, const float* h, int hstride, float* y,
                       hipStream_t s) {
  switch (g.tg) {
    case 1: return down_tg<1>(g, int4, h, hstride, y, s);
    case 2: return down_tg<2>(g, int4, h, hstride, y, s);
    default: return down_tg<4>(g, int4, h, hstride, y, s);
  }
}

}  // namespace moe
