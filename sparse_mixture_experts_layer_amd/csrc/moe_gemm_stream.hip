// Grouped expert GEMMs that stream the packed weights once per tile:
//   gate/up:  h[r][f] = silu(sum_k x[tok(r)][k] Wg[f][k]) * (sum_k x[tok(r)][k] Wu[f][k])
//             (both sums first bounded by the group's SwiGLU limit, if any)
//   down:     Y[r][n] = sum_f h[r][f] Wd[n][f]          (fp32 out)
// for every permuted row r of every expert group (the shared expert is the
// last group, over all tokens).  Expert FFN shape: llm-atlas "Step-3.5-Flash",
// "Champs bruts du config.json" (moe_intermediate_size, share_expert_dim);
// SiLU gating is the reading taken for the swiglu fields, whose limit is 0
// (no clamp) on every MoE layer.
//
// Work unit: one tile of up to 16*TG rows of one group x the output features
// of 4 waves.  The tile's rows are the MFMA A operand and the weights the B
// operand, so a lane's four C values belong to one weight row (one INT4 scale
// per k-group) and four token rows.  Every wave streams one contiguous 4 KiB
// block of packed weights per 32-k step (bf16: gate f, gate f+16, up f, up f+16
// for gate/up; four 16-row blocks for down), no matter how few rows an expert
// has -- the decode regime, where nearly every byte moved is an expert weight.
// Weights and activations of the next group of k-steps are in flight while the
// current group is multiplied.
//
// INT4 (group 32): one 4 KiB block covers 128 k; each lane's 16 bytes hold
// 4 k-groups x 8 nibbles of one row and widen to exact bf16 values 136+q; an
// MFMA of the activations against -136 (shared by the four weight blocks of a
// k-group) removes the offset, and each group's fp32 partial is multiplied by
// its fp16 scale before it joins the accumulator.
#include "moe_common.hpp"
#include "moe_kernels.hpp"

namespace moe {
namespace {

constexpr int kBlockBytes = 4 * kFragBytes;  // one wave's weights per k-step

// A operand (16 rows x 32 k) from bf16 rows (one 16-byte load) or fp32 rows
// (two loads).  fp32 rows enter as bf16 hi + lo (SPLIT) or rounded to bf16.
template <bool F32>
struct ARow {
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

// c += A * B, A given as hi (+ lo when SPLIT).
template <bool SPLIT>
__device__ __forceinline__ f32x4 mma(bf16x8 ahi, bf16x8 alo, bf16x8 b, f32x4 c) {
  c = mfma16(ahi, b, c);
  if (SPLIT) c = mfma16(alo, b, c);
  return c;
}

struct TileInfo {
  int group, row0, nrows, width;
};

__device__ __forceinline__ bool tile_info(const GemmGeom& g, int tile, TileInfo& ti) {
  // The entry is read alongside the tile count (tile < max_tiles: in bounds;
  // an entry past the count is never used), then the group's offset alongside
  // its count: two dependent scalar round trips before the first weight loads
  // instead of four.
  const int nt = *g.ntiles;
  const int v = g.tiles[tile];
  const int grp = tile_group(v);
  if (tile >= nt || grp < 0 || grp > g.E) {  // never a bad group below the count
    if (MOE_DEBUG && tile < nt) dbg_check(g.dbg, false, kDbgTile, v);
    return false;
  }
  const int bm = 16 * g.tg;
  const int m = tile_m(v);
  const int off = g.offsets[grp], cnt = g.counts[grp];
  ti.group = grp;
  ti.row0 = off + m * bm;
  ti.nrows = min(bm, cnt - m * bm);
  ti.width = grp == g.E ? g.Is : g.I;
  return ti.nrows > 0;
}

// Rows of the A operand: lane (l % 16) of token group t reads row t*16 + l%16.
template <int TG>
struct TileRows {
  size_t off[TG];
  bool ok[TG];
  // gathered activation rows (token ids via row_tok), row stride H
  __device__ __forceinline__ void gather(const TileInfo& ti, const int32_t* row_tok, int T, int H,
                                         int lane, int32_t* dbg) {
#pragma unroll
    for (int t = 0; t < TG; ++t) {
      const int r = t * 16 + (lane & 15);
      ok[t] = r < ti.nrows;
      int tok = ok[t] ? row_tok[ti.row0 + r] : 0;
      dbg_check(dbg, tok >= 0 && tok < T, kDbgToken, tok);
      tok = tok < 0 ? 0 : (tok >= T ? T - 1 : tok);
      off[t] = (size_t)tok * H + (lane >> 4) * 8;
    }
  }
  // contiguous rows of a permuted buffer, row stride `stride`
  __device__ __forceinline__ void direct(const TileInfo& ti, int stride, int lane) {
#pragma unroll
    for (int t = 0; t < TG; ++t) {
      const int r = t * 16 + (lane & 15);
      ok[t] = r < ti.nrows;
      off[t] = (size_t)(ti.row0 + (ok[t] ? r : 0)) * stride + (lane >> 4) * 8;
    }
  }
};

// ---------------------------------------------------------- down GEMM output
// With g.y_bf16 a routed row goes to yb at its pair's row, as bf16 of its gate
// weight times the row, and a shared-expert row to ys at its token's row in
// fp32; both are staged through LDS (a private region per wave, rows padded
// against bank conflicts) so that each lane stores 16 contiguous bytes -- from
// the MFMA layout a lane would store 4 bytes at a time and a wave 64-byte
// pieces, a long tail at the end of every workgroup.  Ordinary stores: with
// the nontemporal hint the INT4 decode layer measured 1.6% slower.  Otherwise fp32 rows of
// Y at the permuted row, stored from the MFMA layout.
// The rows' gate weights (staging layout: row t*16 + 4*(lane/16) + i) and
// pairs (store layout: row 8q + lane/8), loaded before the first weight loads
// and copied to a per-wave LDS region once those are issued, so that no
// register stays live across the k loop (the INT4 kernel has none to spare):
// the copy waits for these loads only, which land with the first weight
// blocks the loop waits for anyway.  Rows past the tile read its first row.
template <int TG>
struct DownRows {
  static constexpr int kSlots = 6 * TG;  // 4*TG weights, then 2*TG pairs, 64 lanes each
  uint32_t v[kSlots];
  __device__ __forceinline__ void fetch(const GemmGeom& g, const TileInfo& ti, int lane) {
#pragma unroll
    for (int t = 0; t < TG; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = t * 16 + (lane >> 4) * 4 + i;
        v[t * 4 + i] = __float_as_uint(g.row_w[ti.row0 + (r < ti.nrows ? r : 0)]);
      }
#pragma unroll
    for (int q = 0; q < 2 * TG; ++q) {
      const int r = q * 8 + (lane >> 3);
      v[4 * TG + q] = (uint32_t)g.perm[ti.row0 + (r < ti.nrows ? r : 0)];
    }
  }
  __device__ __forceinline__ void stash(uint32_t* region, int lane) const {
#pragma unroll
    for (int j = 0; j < kSlots; ++j) region[j * kWave + lane] = v[j];
  }
};

// Per-wave LDS of the down epilogue: row weights and pairs, then the staging
// rows (pitch 68 floats for fp32, 72 halves for bf16, against bank conflicts).
template <int TG>
struct DownLds {
  static constexpr int kPF = 68, kPB = 72;
  uint32_t rows[4][DownRows<TG>::kSlots * kWave];
  float stg[4][16 * TG * kPF];
};

// The kernel's DownLds, allocated only in the kernels that can store bf16 Y
// (bf16 activations), null in the others.
template <int TG, bool USE>
__device__ __forceinline__ DownLds<TG>* down_lds() {
  if constexpr (USE) {
    __shared__ DownLds<TG> d;
    return &d;
  } else {
    return nullptr;
  }
}

template <int TG>
__device__ __forceinline__ void store_down(const GemmGeom& g, const TileInfo& ti,
                                           const f32x4 (&acc)[TG][4], DownLds<TG>* sh, int f0,
                                           float* __restrict__ out, int wave, int lane) {
  const int H = g.H;
  if (!g.y_bf16 || !sh) {
#pragma unroll
    for (int t = 0; t < TG; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = t * 16 + (lane >> 4) * 4 + i;
        if (r >= ti.nrows) continue;
        const size_t row = (size_t)ti.row0 + r;
#pragma unroll
        for (int f = 0; f < 4; ++f) out[row * H + f0 + f * 16 + (lane & 15)] = acc[t][f][i];
      }
    return;
  }
  constexpr int kPF = DownLds<TG>::kPF, kPB = DownLds<TG>::kPB;
  float* st = sh->stg[wave];
  if (ti.group == g.E) {
#pragma unroll
    for (int t = 0; t < TG; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int f = 0; f < 4; ++f)
          st[(t * 16 + (lane >> 4) * 4 + i) * kPF + f * 16 + (lane & 15)] = acc[t][f][i];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int tok0 = ti.row0 - g.offsets[g.E];
#pragma unroll
    for (int q = 0; q < 4 * TG; ++q) {
      const int r = q * 4 + (lane >> 4);
      if (r < ti.nrows) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(st + r * kPF + (lane & 15) * 4);
        *reinterpret_cast<f32x4*>(g.ys + (size_t)(tok0 + r) * H + f0 + (lane & 15) * 4) = v;
      }
    }
    return;
  }
  const uint32_t* rw = sh->rows[wave];
  uint16_t* sb = reinterpret_cast<uint16_t*>(st);
#pragma unroll
  for (int t = 0; t < TG; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float wr = __uint_as_float(rw[(t * 4 + i) * kWave + lane]);
#pragma unroll
      for (int f = 0; f < 4; ++f)
        sb[(t * 16 + (lane >> 4) * 4 + i) * kPB + f * 16 + (lane & 15)] =
            f32_to_bf16_bits(wr * acc[t][f][i]);
    }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int q = 0; q < 2 * TG; ++q) {
    const int r = q * 8 + (lane >> 3);
    if (r < ti.nrows) {
      const int p = (int)rw[(4 * TG + q) * kWave + lane];
      const u32x4 v = *reinterpret_cast<const u32x4*>(sb + r * kPB + (lane & 7) * 8);
      *reinterpret_cast<u32x4*>(g.yb + (size_t)p * H + f0 + (lane & 7) * 8) = v;
    }
  }
}

// ------------------------------------------------------------------ bf16 weights
// MODE 0: gate/up (A = gathered x, fp32 or bf16; out h with SiLU*up)
// MODE 1: down    (A = h; out Y fp32)
// HM (h format): 0 = fp32 h, entering the down MFMA as hi + lo (layers with fp32
// activations, whose fp32 output is held to a tight bound); 1 = bf16 h for the
// routed rows, 2 = bf16 h plus a bf16 remainder plane h_lo for the shared
// expert's rows (layers with bf16 activations: the routed terms are weighted
// by ~1/k, the unweighted shared expert keeps its h to ~16 bits).  In the down
// GEMM, HM 1 runs the routed tiles and HM 2 the shared tiles, the latter with
// one more MFMA per k-step over h_lo; HM 3 runs both in one launch (the
// shared tiles alone are too few to fill the GPU at decode batch sizes).
// Packed block of a wave: gate/up [W/32][H/32][g0 g1 u0 u1]; down [H/64][W/32][f0..f3].
template <int MODE, bool XF32, int TG, int U, int HM>
__global__ __launch_bounds__(256) void stream_bf16_kernel(GemmGeom g, const void* __restrict__ a_src,
                                                          const int32_t* __restrict__ row_tok,
                                                          float* __restrict__ out, int hstride,
                                                          uint16_t* __restrict__ h_lo, int nblk) {
  constexpr bool AF32 = MODE == 1 ? HM == 0 : XF32;
  constexpr bool SPLIT = AF32;            // fp32 A rows always enter as hi + lo
  constexpr bool LO = MODE == 1 && (HM == 2 || HM == 3);  // h_lo operand compiled in
  // down with HM 2 walks the shared group's tiles only (the last ones of the list)
  const int nsh = MODE == 1 && HM == 2 ? g.shared_tiles : 0;
  const int tile = nsh ? *g.ntiles - nsh + (int)(blockIdx.x / nblk) : (int)(blockIdx.x / nblk);
  const int nb = blockIdx.x % nblk;
  TileInfo ti;
  if (!tile_info(g, tile, ti)) return;
  if (MODE == 1 && HM == 1 && ti.group == g.E) return;  // shared tiles: the HM 2 launch
  if (MODE == 1 && HM == 2 && ti.group != g.E) return;
  const bool lo = LO && ti.group == g.E;  // workgroup-uniform
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int H = g.H;
  int f0, K;
  const uint8_t* wp = g.packed + (size_t)ti.group * g.expert_bytes + lane * 16;
  TileRows<TG> rows;
  if (MODE == 0) {
    f0 = nb * 128 + wave * 32;
    if (f0 >= ti.width) return;
    K = H;
    wp += (size_t)(f0 / 32) * (K / 32) * kBlockBytes;
    rows.gather(ti, row_tok, g.T, H, lane, g.dbg);
  } else {
    f0 = nb * 256 + wave * 64;
    if (f0 >= H) return;
    K = ti.width;
    wp += (size_t)2 * ti.width * H * 2 + (size_t)(f0 / 64) * (K / 32) * kBlockBytes;
    rows.direct(ti, hstride, lane);
  }
  const int nk = K / 32;

  f32x4 acc[TG][4];
#pragma unroll
  for (int t = 0; t < TG; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // remainder rows of the shared expert: h_lo row = permuted row - first shared row
  size_t lo_off[TG];
  if (lo) {
#pragma unroll
    for (int t = 0; t < TG; ++t) lo_off[t] = rows.off[t] - (size_t)g.offsets[g.E] * hstride;
  }
  constexpr int NL = LO ? 1 : 0;
  DownLds<TG>* dsh = down_lds<TG, MODE == 1 && HM != 0>();
  const bool yrows = dsh && g.y_bf16 && ti.group != g.E;  // workgroup-uniform
  DownRows<TG> dr;
  if (yrows) dr.fetch(g, ti, lane);
  u32x4 w[U][4], wn[U][4];
  ARow<AF32> a[U][TG], an[U][TG];
  ARow<false> l[U][TG * NL + 1 - NL], ln[U][TG * NL + 1 - NL];
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int j = 0; j < 4; ++j) w[u][j] = load16_stream(wp + (size_t)u * kBlockBytes + j * kFragBytes);
#pragma unroll
    for (int t = 0; t < TG; ++t) {
      a[u][t].load(a_src, rows.off[t] + u * 32, rows.ok[t]);
      if (lo) l[u][t].load(h_lo, lo_off[t] + u * 32, rows.ok[t]);
    }
  }
  if (yrows) dr.stash(dsh->rows[wave], lane);
  for (int k0 = 0; k0 < nk; k0 += U) {
    const bool more = k0 + U < nk;
    if (more) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          wn[u][j] = load16_stream(wp + (size_t)(k0 + U + u) * kBlockBytes + j * kFragBytes);
#pragma unroll
        for (int t = 0; t < TG; ++t) {
          an[u][t].load(a_src, rows.off[t] + (size_t)(k0 + U + u) * 32, rows.ok[t]);
          if (lo) ln[u][t].load(h_lo, lo_off[t] + (size_t)(k0 + U + u) * 32, rows.ok[t]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < TG; ++t) {
        bf16x8 ah, al;
        a[u][t].operands(ah, al);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[t][j] = mma<SPLIT>(ah, al, as_bf16x8(w[u][j]), acc[t][j]);
        if (lo) {
          bf16x8 lh, ll;
          l[u][t].operands(lh, ll);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[t][j] = mfma16(lh, as_bf16x8(w[u][j]), acc[t][j]);
        }
      }
    if (more) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int j = 0; j < 4; ++j) w[u][j] = wn[u][j];
#pragma unroll
        for (int t = 0; t < TG; ++t) {
          a[u][t] = an[u][t];
          if (lo) l[u][t] = ln[u][t];
        }
      }
    }
  }

  // epilogue: lane holds rows t*16 + 4*(lane/16) + i of weight column (lane % 16)
  if (MODE == 1) {
    store_down<TG>(g, ti, acc, dsh, f0, out, wave, lane);
    return;
  }
#pragma unroll
  for (int t = 0; t < TG; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = t * 16 + (lane >> 4) * 4 + i;
      if (r >= ti.nrows) continue;
      const size_t row = (size_t)ti.row0 + r;
      if (MODE == 0 && HM == 0) {
        const float lim = ti.group == g.E ? g.limit_shared : g.limit;
#pragma unroll
        for (int f = 0; f < 2; ++f)
          out[row * hstride + f0 + f * 16 + (lane & 15)] =
              swiglu(acc[t][f][i], acc[t][2 + f][i], lim);
      } else if (MODE == 0) {
        uint16_t* hb = reinterpret_cast<uint16_t*>(out);
        const bool shared = ti.group == g.E;
        const float lim = shared ? g.limit_shared : g.limit;
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const float hv = swiglu(acc[t][f][i], acc[t][2 + f][i], lim);
          const uint16_t hi = f32_to_bf16_bits(hv);
          hb[row * hstride + f0 + f * 16 + (lane & 15)] = hi;
          if (shared)
            h_lo[(row - g.offsets[g.E]) * hstride + f0 + f * 16 + (lane & 15)] =
                f32_to_bf16_bits(hv - bf16_bits_to_f32(hi));
        }
      }
    }
}

// ------------------------------------------------------------------ INT4 weights
// Per group of width W:
//   gate/up q      [W/32][H/128][g0 g1 u0 u1][64 lanes][16 B]      W*H bytes
//   gate/up scales [W/32][H/128][16 rows][4 blocks][4 kg] fp16     W*H/8 bytes
//   down q         [H/64][W/128][f0..f3][64][16 B]                 H*W/2 bytes
//   down scales    [H/64][W/128][16 rows][4 blocks][4 kg] fp16     H*W/16 bytes
// MODE 0: gate/up (A = gathered x), h stored as bf16; MODE 1: down (A = bf16 h).
constexpr uint32_t kMinus136x2 = 0xC308C308u;  // bf16 -136 in both halves

// Occupancy: three waves per SIMD for one token group of bf16 rows (what
// decode batches use), which fits the three register sets in 168 registers.
template <int MODE, bool XF32, int TG>
__global__ __launch_bounds__(256, XF32 ? 1 : (TG == 1 ? 3 : (TG == 2 ? 2 : 1)))
void stream_int4_kernel(GemmGeom g, const void* __restrict__ a_src,
                                                          const int32_t* __restrict__ row_tok,
                                                          float* __restrict__ out, int hstride,
                                                          int nblk) {
  constexpr bool AF32 = MODE == 1 ? false : XF32;  // h is stored as bf16
  constexpr bool SPLIT = MODE == 0 && XF32;
  const int tile = blockIdx.x / nblk, nb = blockIdx.x % nblk;
  TileInfo ti;
  if (!tile_info(g, tile, ti)) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int H = g.H, W = ti.width;
  const uint8_t* base = g.packed + (size_t)ti.group * g.expert_bytes;
  int f0, K;
  const uint8_t *qp, *sp;
  TileRows<TG> rows;
  if (MODE == 0) {
    f0 = nb * 128 + wave * 32;
    if (f0 >= W) return;
    K = H;
    qp = base + (size_t)(f0 / 32) * (K / 128) * kBlockBytes;
    sp = base + (size_t)W * H + (size_t)(f0 / 32) * (K / 128) * 512;
    rows.gather(ti, row_tok, g.T, H, lane, g.dbg);
  } else {
    f0 = nb * 256 + wave * 64;
    if (f0 >= H) return;
    K = W;
    const uint8_t* dbase = base + (size_t)W * H + (size_t)W * H / 8;
    qp = dbase + (size_t)(f0 / 64) * (K / 128) * kBlockBytes;
    sp = dbase + (size_t)H * W / 2 + (size_t)(f0 / 64) * (K / 128) * 512;
    rows.direct(ti, hstride, lane);
  }
  qp += lane * 16;
  sp += (lane & 15) * 32;
  const int nkb = K / 128;
  const bf16x8 m136 = as_bf16x8(u32x4{kMinus136x2, kMinus136x2, kMinus136x2, kMinus136x2});

  f32x4 acc[TG][4];
#pragma unroll
  for (int t = 0; t < TG; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Blocks of 128 k (4 weight fragments, their scales, the A rows) rotate
  // through three register sets, loaded two blocks ahead: the packed INT4
  // stream is a quarter of the bf16 bytes per MFMA, so more of it must be in
  // flight to cover HBM latency.  The loop is unrolled by three so the sets
  // are never copied (a copy would wait for the loads just issued), and every
  // load is unconditional (past the last block the last one is re-read; rows
  // past the tile read a valid row whose results are never stored), which
  // keeps the compiler's wait counts exact.
  struct Blk {
    u32x4 q[4], s[2];
    ARow<AF32> a[4][TG];
  } b0, b1, b2;
  auto load_blk = [&](Blk& b, int kb) {
    kb = kb < nkb ? kb : nkb - 1;
#pragma unroll
    for (int j = 0; j < 4; ++j) b.q[j] = load16_stream(qp + (size_t)kb * kBlockBytes + j * kFragBytes);
    b.s[0] = load16_stream(sp + (size_t)kb * 512);
    b.s[1] = load16_stream(sp + (size_t)kb * 512 + 16);
#pragma unroll
    for (int kg = 0; kg < 4; ++kg)
#pragma unroll
      for (int t = 0; t < TG; ++t) b.a[kg][t].load(a_src, rows.off[t] + (size_t)kb * 128 + kg * 32, true);
  };
  // 8 nibbles -> 8 bf16 (128 + u): the OR constant sits in a register so each
  // pair is one v_and_or_b32 (a VOP3 cannot take two literals)
  uint32_t c4300;
  asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(c4300));
  auto widen = [c4300](uint32_t w) {
    u32x4 r;
    r[0] = (w & 0x000f000fu) | c4300;
    r[1] = ((w >> 4) & 0x000f000fu) | c4300;
    r[2] = ((w >> 8) & 0x000f000fu) | c4300;
    r[3] = ((w >> 12) & 0x000f000fu) | c4300;
    return as_bf16x8(r);
  };
  auto compute = [&](const Blk& b) {
    // scales of this lane's weight row: [4 blocks][4 kg] fp16
    float sc[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int kg = 0; kg < 4; ++kg) {
        const int e = j * 4 + kg;
        const uint32_t word = b.s[e >> 3][(e >> 1) & 3];
        const uint16_t bits = (uint16_t)((e & 1) ? (word >> 16) : (word & 0xffffu));
        sc[j][kg] = (float)__builtin_bit_cast(_Float16, bits);
      }
#pragma unroll
    for (int kg = 0; kg < 4; ++kg)
#pragma unroll
      for (int t = 0; t < TG; ++t) {
        bf16x8 ah, al;
        b.a[kg][t].operands(ah, al);
        const f32x4 corr = mma<SPLIT>(ah, al, m136, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 p = mma<SPLIT>(ah, al, widen(b.q[j][kg]), corr);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[t][j][i] += sc[j][kg] * p[i];
        }
      }
  };
  DownLds<TG>* dsh = down_lds<TG, MODE == 1>();
  const bool yrows = dsh && g.y_bf16 && ti.group != g.E;  // workgroup-uniform
  DownRows<TG> dr;
  if (yrows) dr.fetch(g, ti, lane);
  load_blk(b0, 0);
  load_blk(b1, 1);
  if (yrows) dr.stash(dsh->rows[wave], lane);
  int kb = 0;
  for (; kb + 3 <= nkb; kb += 3) {
    load_blk(b2, kb + 2);
    __builtin_amdgcn_sched_barrier(0);
    compute(b0);
    load_blk(b0, kb + 3);
    __builtin_amdgcn_sched_barrier(0);
    compute(b1);
    load_blk(b1, kb + 4);
    __builtin_amdgcn_sched_barrier(0);
    compute(b2);
  }
  // 0-2 blocks left, already in b0 (and b1)
  if (kb < nkb) compute(b0);
  if (kb + 1 < nkb) compute(b1);
  if (MODE == 1) {
    store_down<TG>(g, ti, acc, dsh, f0, out, wave, lane);
    return;
  }

#pragma unroll
  for (int t = 0; t < TG; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = t * 16 + (lane >> 4) * 4 + i;
      if (r >= ti.nrows) continue;
      const size_t row = (size_t)ti.row0 + r;
      if (MODE == 0) {
        uint16_t* hb = reinterpret_cast<uint16_t*>(out);
        const float lim = ti.group == g.E ? g.limit_shared : g.limit;
#pragma unroll
        for (int f = 0; f < 2; ++f)
          hb[row * hstride + f0 + f * 16 + (lane & 15)] =
              f32_to_bf16_bits(swiglu(acc[t][f][i], acc[t][2 + f][i], lim));
      }
    }
}

template <int MODE, int TG>
hipError_t launch_mode(const GemmGeom& g, bool int4, bool act_f32, const void* a,
                       const int32_t* row_tok, float* out, uint16_t* h_lo, int hstride,
                       hipStream_t s) {
  const int wmax = g.I > g.Is ? g.I : g.Is;
  const int nblk = MODE == 0 ? (wmax + 127) / 128 : (g.H + 255) / 256;
  dim3 grid((unsigned)g.max_tiles * nblk), block(256);
  if (int4) {
    if (act_f32 && MODE == 0)
      hipLaunchKernelGGL((stream_int4_kernel<MODE, true, TG>), grid, block, 0, s, g, a, row_tok,
                         out, hstride, nblk);
    else
      hipLaunchKernelGGL((stream_int4_kernel<MODE, false, TG>), grid, block, 0, s, g, a, row_tok,
                         out, hstride, nblk);
    return hipGetLastError();
  }
#define MOE_L(GRID, ...)                                                                         \
  hipLaunchKernelGGL((stream_bf16_kernel<__VA_ARGS__>), GRID, block, 0, s, g, a, row_tok, out, \
                     hstride, h_lo, nblk)
  if constexpr (MODE == 0) {
    if (act_f32) MOE_L(grid, MODE, true, TG, 2, 0);
    else MOE_L(grid, MODE, false, TG, 2, 1);
    return hipGetLastError();
  } else {
    // down: k-steps per group U must divide every group's K/32 (the expert
    // widths are only multiples of 32): 4 when divisible by 4 (twice the bytes
    // in flight per wave: 0.5% on the decode-sized launch, 1.6% on the
    // 32-row-tile one of the verify batch), else 2 when even
    const bool even = (g.I / 32) % 2 == 0 && (g.Is / 32) % 2 == 0;
    const bool quad = (g.I / 32) % 4 == 0 && (g.Is / 32) % 4 == 0;
    const int nsh = g.shared_tiles;
    dim3 grid_sh((unsigned)nsh * nblk);
    if (act_f32) {
      if (even) MOE_L(grid, MODE, false, TG, 2, 0);
      else MOE_L(grid, MODE, false, TG, 1, 0);
      return hipGetLastError();
    }
    if constexpr (TG == 1) {  // decode-sized: one launch for routed and shared tiles
      if (quad) MOE_L(grid, MODE, false, TG, 4, 3);
      else if (even) MOE_L(grid, MODE, false, TG, 2, 3);
      else MOE_L(grid, MODE, false, TG, 1, 3);
      return hipGetLastError();
    } else {
      if (quad) MOE_L(grid, MODE, false, TG, 4, 1);
      else if (even) MOE_L(grid, MODE, false, TG, 2, 1);
      else MOE_L(grid, MODE, false, TG, 1, 1);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess || nsh == 0) return e;
      if (quad) MOE_L(grid_sh, MODE, false, TG, 4, 2);
      else if (even) MOE_L(grid_sh, MODE, false, TG, 2, 2);
      else MOE_L(grid_sh, MODE, false, TG, 1, 2);
      return hipGetLastError();
    }
  }
#undef MOE_L
}

template <int MODE>
hipError_t launch_tg(const GemmGeom& g, bool int4, bool act_f32, const void* a,
                     const int32_t* row_tok, float* out, uint16_t* h_lo, int hstride,
                     hipStream_t s) {
  switch (g.tg) {
    case 1: return launch_mode<MODE, 1>(g, int4, act_f32, a, row_tok, out, h_lo, hstride, s);
    case 2: return launch_mode<MODE, 2>(g, int4, act_f32, a, row_tok, out, h_lo, hstride, s);
    default: return launch_mode<MODE, 4>(g, int4, act_f32, a, row_tok, out, h_lo, hstride, s);
  }
}

}  // namespace

hipError_t launch_gateup(const GemmGeom& g, bool int4, bool act_f32, const void* x,
                         const int32_t* row_tok, void* h, uint16_t* h_lo, int hstride,
                         hipStream_t s) {
  return launch_tg<0>(g, int4, act_f32, x, row_tok, static_cast<float*>(h), h_lo, hstride, s);
}

hipError_t launch_down(const GemmGeom& g, bool int4, bool act_f32, const void* h,
                       const uint16_t* h_lo, int hstride, float* y, hipStream_t s) {
  return launch_tg<1>(g, int4, act_f32, h, nullptr, y, const_cast<uint16_t*>(h_lo), hstride, s);
}

}  // namespace moe
