// Host-side launchers of the gfx950 MoE kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

// Index checks of debug builds (see moe_common.hpp); 0 in release builds.
#ifndef MOE_DEBUG
#define MOE_DEBUG 0
#endif

namespace moe {

// ---- router: logits (fp32 partial sums over KS slices of H) + top-k ----------
// Workgroups of the router logits kernel for a batch (before the K split).
int router_blocks(bool x_f32, int T, int E);
// done, if not null, is set to 0 (the counter of launch_topk_dispatch); so
// are dbg[0] and dbg[1], if dbg is not null (the debug word pair).
hipError_t launch_router_logits(bool x_f32, const void* x, const uint16_t* router_w, float* part,
                                int T, int H, int E, int ks, int32_t* done, int32_t* dbg,
                                hipStream_t s);
hipError_t launch_router_topk(const float* part, int ks, const float* bias, int bias_mode, int T,
                              int E, int k, int score, int renorm, float scale, int32_t* idx,
                              float* w, float* gap, hipStream_t s);

// ---- dispatch: counts, offsets, stable permutation, GEMM tile list ----------
// counts/offsets have E+1 / E+2 entries (group E = shared expert, T rows).
// row_w, if not null, receives each routed row's gate weight (w of the pair
// stored at that row), read by the down GEMMs that weight Y themselves.
// GEMM tile lists written by the dispatch: a routed expert with fewer than
// `hot` rows goes to list 1 in tiles of bm rows, one with `hot` rows or more
// to list 2 in tiles of bm2 rows; the shared expert (group E) always to list
// 1, last; hot == 0 puts every group in list 1 (list 2 is then neither used
// nor written).
struct TileLists {
  int bm, hot, bm2;
  int32_t *tiles, *ntiles, *tiles2, *ntiles2;
  __host__ __device__ bool in_second(int rows) const { return hot > 0 && rows >= hot; }
};

// Top-k (as launch_router_topk) and the dispatch in one launch, T <= 1024:
// the last workgroup to finish its tokens' top-k runs the dispatch as one
// workgroup (one wave of it up to 64 tokens).  done is a device counter that must read 0 at launch
// (launch_router_logits clears it).
hipError_t launch_topk_dispatch(const float* part, int ks, const float* bias, int bias_mode, int T,
                                int E, int k, int score, int renorm, float scale, int32_t* idx,
                                float* w, float* gap, int32_t* done, int has_shared,
                                const TileLists& tl, int32_t* counts, int32_t* offsets,
                                int32_t* perm, int32_t* inv, int32_t* row_tok, float* row_w,
                                int32_t* dbg, hipStream_t s);

// Multi-workgroup variant for large batches (same outputs); blk_hist is
// scratch of dispatch_blocks(T) * E int32.
int dispatch_blocks(int T);
hipError_t launch_dispatch_large(const int32_t* idx, int T, int k, int E, int has_shared, int bm,
                                 int32_t* blk_hist, int32_t* counts, int32_t* offsets,
                                 int32_t* perm, int32_t* inv, int32_t* row_tok, int32_t* tiles,
                                 int32_t* ntiles, const float* w, float* row_w, int32_t* dbg,
                                 hipStream_t s);

// ---- grouped expert GEMMs ----------------------------------------------------
struct GemmGeom {
  int H, I, Is, E, T;         // shapes (T = tokens of this call)
  size_t expert_bytes;        // packed bytes of one routed expert
  const uint8_t* packed;      // packed weights (shared expert = group E, after the routed ones)
  const int32_t* tiles;       // tile list
  const int32_t* ntiles;      // device scalar: number of valid tiles
  const int32_t* offsets;     // [E+2] first permuted row of each group
  const int32_t* counts;      // [E+1] rows of each group
  int max_tiles;              // grid bound
  int tg;                     // token groups of 16 per tile (tile rows = 16 * tg)
  int shared_tiles;           // tiles of the shared group at the end of this list (0: none)
  float limit, limit_shared;  // SwiGLU limits of the routed / shared experts (0 = none)
  // LDS-tiled down GEMM only: K split into ksplit equal parts (ksplit divides
  // every group's width/32), part s writing its partial sums to Y plane s, y_plane
  // floats after plane s-1 (the combine adds the planes in order)
  int ksplit;
  size_t y_plane;
  // LDS-tiled gate/up only: K split into ksplit_gu parts (each an even number
  // of k-steps), part s writing fp32 partial sums of gate and up to
  // gu_part + s * gu_plane, row r's gate at [2r][f], its up at [2r+1][f] (rows
  // of 2 * hstride floats); launch_gateup_reduce then forms h
  int ksplit_gu;
  float* gu_part;
  size_t gu_plane;
  int32_t* dbg;  // debug word pair (debug builds report out-of-range indices there)
  // y_bf16 set (bf16 activations, no K split): the down GEMMs store a routed
  // row of Y as bf16 of its gate weight times the row at its pair's row of yb
  // ([P][H], row p = t*k + j for permuted row r with perm[r] = p), the shared
  // group's rows as fp32 by token (ys, [T][H]); row_w[r] is routed row r's
  // gate weight (written by the dispatch).
  int y_bf16;
  uint16_t* yb;
  float* ys;
  const float* row_w;
  const int32_t* perm;
};

// h[row][f] = silu(x W_gate^T) * (x W_up^T) for every permuted row; h is fp32
// when the activations are fp32 (bf16 weights), bf16 otherwise, with the shared
// expert's rows also leaving a bf16 remainder in h_lo ([T][hstride]; bf16
// weights only).
hipError_t launch_gateup(const GemmGeom& g, bool int4, bool act_f32, const void* x,
                         const int32_t* row_tok, void* h, uint16_t* h_lo, int hstride,
                         hipStream_t s);
// Y[row][:] = h[row] W_down^T (fp32) for every permuted row, h as left by
// launch_gateup (fp32 h enters the MFMA as bf16 hi + lo).
hipError_t launch_down(const GemmGeom& g, bool int4, bool act_f32, const void* h,
                       const uint16_t* h_lo, int hstride, float* y, hipStream_t s);

// Large-batch variants: LDS-staged tiles of 128 or 256 rows (g.tg 8 or 16,
// any other value is rejected), bf16 h in packed fragment order: 1 KiB
// fragments of 16 rows x 32 features, fragment (b, kb) at (b * hstride/32 +
// kb) KiB, group e's row r in packed row 16 * (ceil(offsets[e]/16) + e) + r;
// h needs tiled_h_rows(P + T, E) rows of hstride bf16.  The shared group's h
// also gets a bf16 remainder plane h_lo, packed the same way by its row
// (tiled_h_rows(T, 0) rows).
inline size_t tiled_h_rows(int rows, int groups) {
  return 16 * ((size_t)(rows + 15) / 16 + groups + 1) + 256;
}
hipError_t launch_gateup_tiled(const GemmGeom& g, const uint16_t* x, const int32_t* row_tok,
                               uint16_t* h, uint16_t* h_lo, int hstride, hipStream_t s);
hipError_t launch_down_tiled(const GemmGeom& g, const uint16_t* h, const uint16_t* h_lo,
                             int hstride, float* y, hipStream_t s);
// After a split-K gate/up: for each of the `rows` permuted rows, gate and up
// summed over the parts in order, then h = SwiGLU written as
// launch_gateup_tiled writes it (packed h, the shared group's remainder plane).
hipError_t launch_gateup_reduce(const GemmGeom& g, int rows, uint16_t* h, uint16_t* h_lo,
                                int hstride, hipStream_t s);

// ---- combine: out[t] = Y[shared row of t] + sum_j w[t,j] Y[inv[t,j]] -------
// Y may come in `planes` partial-sum planes, `plane` floats apart: each row is
// then the sum of its planes, added in plane order.  With yb (the down GEMMs'
// y_bf16 layout), the routed rows come from yb, already weighted, at the
// pairs' rows (out[t] = ys[t] + sum_j yb[t*k + j]), the shared ones from ys.
hipError_t launch_combine(bool out_f32, const float* y, int H, const int32_t* inv, const float* w,
                          int k, int P, int has_shared, void* out, int T, int planes,
                          size_t plane, const uint16_t* yb, const float* ys, int32_t* dbg,
                          hipStream_t s);

// ---- weight packing ----------------------------------------------------------
// bf16 [N][K] of S sources (1 or 2) -> blocks of F*S fragments per 32-k step.
hipError_t launch_pack_bf16(const uint16_t* src0, const uint16_t* src1, int S, int F, int N,
                            int K, int batch, size_t src_batch_stride, uint8_t* dst,
                            size_t dst_batch_stride, hipStream_t s);
// INT4 nibbles [N][K/2] + fp16 scales [N][K/32] -> blocks per 128-k step + scales.
hipError_t launch_pack_int4(const uint8_t* q0, const uint8_t* q1, const uint16_t* s0,
                            const uint16_t* s1, int S, int F, int N, int K, int batch,
                            size_t q_batch_stride, size_t s_batch_stride, uint8_t* dst_q,
                            uint8_t* dst_s, size_t dst_batch_stride, hipStream_t s);

}  // namespace moe
