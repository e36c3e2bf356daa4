// Combine / unpermute: y[t] = Y[shared row of t] + sum_j w[t,j] * Y[inv[t,j]],
// accumulated in fp32 in a fixed order (shared first, then j = 0..k-1) and
// rounded once to the output dtype.  Down GEMMs that weight their rows
// themselves (bf16 activations, no K split) leave bf16 rows of w[t,j] * Y at
// the pairs' rows t*k + j and the shared rows in fp32 by token: then
// y[t] = ys[t] + sum_j yb[t*k + j], in the same order.  The shared expert is always on and enters
// unweighted (llm-atlas "Step-3.5-Flash", "Champs bruts du config.json",
// share_expert_dim; that it is added outside the renormalised weights is the
// reading taken where the pages are silent).
#include "moe_common.hpp"
#include "moe_kernels.hpp"

namespace moe {
namespace {

// Four output columns at element offset off, rounded once to the output dtype.
template <bool OUT_F32>
__device__ __forceinline__ void store_out(void* out, size_t off, const f32x4& acc) {
  if (OUT_F32) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + off) = acc;
  } else {
    uint2 pk;
    pk.x = pack_bf16x2(acc[0], acc[1]);
    pk.y = pack_bf16x2(acc[2], acc[3]);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + off) = pk;
  }
}

// Small batches: one thread per 4 output columns of one token, a token's
// row spread over ceil(H / 1024) workgroups.  The token's routing entries are
// the same for every thread (scalar loads), and the thread issues the loads of
// all KMAX >= k rows before any arithmetic (a loop over the rows would wait
// for each row in turn): rows past k re-read row k-1 and are zeroed by a
// select.  Y is read once: nontemporal loads keep it from displacing cached
// data.
template <bool OUT_F32, int KMAX, bool YB>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y, int H,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ w, int k, int P,
                                                      int has_shared, void* __restrict__ out,
                                                      int T, int planes, size_t plane,
                                                      const uint16_t* __restrict__ yb,
                                                      const float* __restrict__ ys,
                                                      int32_t* __restrict__ dbg) {
  const int t = blockIdx.x;
  const int col = (blockIdx.y * blockDim.x + threadIdx.x) * 4;
  if (t >= T || col >= H) return;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  if (YB) {  // routed rows already weighted, in bf16, at the pairs' rows; the shared row in fp32
    u32x2 b[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      b[j] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x2*>(yb + ((size_t)t * k + (j < k ? j : k - 1)) * H + col));
    f32x4 acc = has_shared ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(ys + (size_t)t * H + col))
                           : zero;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j >= k) break;
      acc[0] += bf16_bits_to_f32((uint16_t)b[j][0]);
      acc[1] += bf16_bits_to_f32((uint16_t)(b[j][0] >> 16));
      acc[2] += bf16_bits_to_f32((uint16_t)b[j][1]);
      acc[3] += bf16_bits_to_f32((uint16_t)(b[j][1] >> 16));
    }
    store_out<OUT_F32>(out, (size_t)t * H + col, acc);
    return;
  }
  int rows[KMAX];
  float wj[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const int jj = j < k ? j : k - 1;
    const int r = inv[(size_t)t * k + jj];
    dbg_check(dbg, r >= 0 && r < P, kDbgRow, r);
    rows[j] = r < 0 ? 0 : (r >= P ? P - 1 : r);
    wj[j] = w[(size_t)t * k + jj];
  }
  // shared row (or, without a shared expert, any valid row, then zeroed)
  const size_t srow = has_shared ? (size_t)(P + t) : (size_t)rows[0];
  f32x4 sh = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(y + srow * H + col));
  f32x4 v[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j)
    v[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(y + (size_t)rows[j] * H + col));
  // rows split into partial-sum planes (a down GEMM with a split K): each row's
  // planes added in order
#pragma unroll 4
  for (int q = 1; q < planes; ++q) {  // four planes' loads in flight together
    const float* yq = y + q * plane;
    sh += __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(yq + srow * H + col));
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      v[j] += __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(yq + (size_t)rows[j] * H + col));
  }
  // fixed order: shared, then j = 0 .. k-1
  f32x4 acc = has_shared ? sh : zero;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const f32x4 vj = j < k ? v[j] : zero;
    const float cw = j < k ? wj[j] : 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += cw * vj[e];
  }
  store_out<OUT_F32>(out, (size_t)t * H + col, acc);
}

// Large batches: one workgroup per token, a thread owns 4 groups of 4
// columns; the rows are walked in order, the 4 groups' loads of a row in
// flight together, so each row is read as one contiguous run per workgroup.
template <bool OUT_F32, bool YB>
__global__ __launch_bounds__(256) void combine_rows_kernel(const float* __restrict__ y, int H,
                                                           const int32_t* __restrict__ inv,
                                                           const float* __restrict__ w, int k,
                                                           int P, int has_shared,
                                                           void* __restrict__ out, int T,
                                                           int planes, size_t plane,
                                                           const uint16_t* __restrict__ yb,
                                                           const float* __restrict__ ys,
                                                           int32_t* __restrict__ dbg) {
  const int t = blockIdx.x;
  if (t >= T) return;
  __shared__ int rows[kMaxTopK];
  __shared__ float ws[kMaxTopK];
  if (!YB && threadIdx.x < k) {  // (bf16 rows: the pairs' own rows, already weighted)
    int r = inv[(size_t)t * k + threadIdx.x];
    dbg_check(dbg, r >= 0 && r < P, kDbgRow, r);
    rows[threadIdx.x] = r < 0 ? 0 : (r >= P ? P - 1 : r);
    ws[threadIdx.x] = w[(size_t)t * k + threadIdx.x];
  }
  __syncthreads();
  // Each thread owns kChunks column groups of 4 per pass, so every row's
  // loads for all of them are in flight together (bandwidth-bound kernel).
  // Y is read once: nontemporal loads keep it from displacing cached data.
  constexpr int kChunks = 4;
  const int stride = blockDim.x * 4;
  if (YB) {  // routed rows already weighted, in bf16; the shared row in fp32
    for (int c0 = 0; c0 < H; c0 += stride * kChunks) {
      f32x4 acc[kChunks];
      int col[kChunks];
#pragma unroll
      for (int i = 0; i < kChunks; ++i) {
        col[i] = c0 + i * stride + threadIdx.x * 4;
        acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (has_shared && col[i] < H)
          acc[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(ys + (size_t)t * H + col[i]));
      }
      for (int j = 0; j < k; ++j) {
        const uint16_t* yr = yb + ((size_t)t * k + j) * H;
        u32x2 v[kChunks];
#pragma unroll
        for (int i = 0; i < kChunks; ++i)
          v[i] = col[i] < H ? __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(yr + col[i]))
                            : u32x2{0u, 0u};
#pragma unroll
        for (int i = 0; i < kChunks; ++i) {
          acc[i][0] += bf16_bits_to_f32((uint16_t)v[i][0]);
          acc[i][1] += bf16_bits_to_f32((uint16_t)(v[i][0] >> 16));
          acc[i][2] += bf16_bits_to_f32((uint16_t)v[i][1]);
          acc[i][3] += bf16_bits_to_f32((uint16_t)(v[i][1] >> 16));
        }
      }
#pragma unroll
      for (int i = 0; i < kChunks; ++i)
        if (col[i] < H) store_out<OUT_F32>(out, (size_t)t * H + col[i], acc[i]);
    }
    return;
  }
  for (int c0 = 0; c0 < H; c0 += stride * kChunks) {
    f32x4 acc[kChunks];
    int col[kChunks];
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      col[i] = c0 + i * stride + threadIdx.x * 4;
      acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (has_shared && col[i] < H)
        acc[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(y + (size_t)(P + t) * H + col[i]));
    }
    if (has_shared)  // partial-sum planes of a split-K down GEMM
      for (int q = 1; q < planes; ++q)
#pragma unroll
        for (int i = 0; i < kChunks; ++i)
          if (col[i] < H)
            acc[i] += __builtin_nontemporal_load(
                reinterpret_cast<const f32x4*>(y + q * plane + (size_t)(P + t) * H + col[i]));
    for (int j = 0; j < k; ++j) {
      const float* yr = y + (size_t)rows[j] * H;
      const float wj = ws[j];
      f32x4 v[kChunks];
#pragma unroll
      for (int i = 0; i < kChunks; ++i)
        v[i] = col[i] < H ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(yr + col[i])) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
      for (int q = 1; q < planes; ++q)  // partial-sum planes of a split-K down GEMM
#pragma unroll
        for (int i = 0; i < kChunks; ++i)
          if (col[i] < H)
            v[i] += __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(yr + q * plane + col[i]));
#pragma unroll
      for (int i = 0; i < kChunks; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][e] += wj * v[i][e];
    }
#pragma unroll
    for (int i = 0; i < kChunks; ++i)
      if (col[i] < H) store_out<OUT_F32>(out, (size_t)t * H + col[i], acc[i]);
  }
}

}  // namespace

hipError_t launch_combine(bool out_f32, const float* y, int H, const int32_t* inv, const float* w,
                          int k, int P, int has_shared, void* out, int T, int planes,
                          size_t plane, const uint16_t* yb, const float* ys, int32_t* dbg,
                          hipStream_t s) {
  if (k < 1 || k > kMaxTopK || planes < 1 || (yb && (planes != 1 || (has_shared && !ys))))
    return hipErrorInvalidValue;
  const bool ybm = yb != nullptr;
  if (T >= 512) {  // bandwidth-bound: whole rows per workgroup
    dim3 grid(T), block(256);
#define MOE_CR(F32, YB)                                                                          \
  hipLaunchKernelGGL((combine_rows_kernel<F32, YB>), grid, block, 0, s, y, H, inv, w, k, P,     \
                     has_shared, out, T, planes, plane, yb, ys, dbg)
    if (out_f32) {
      if (ybm) MOE_CR(true, true); else MOE_CR(true, false);
    } else {
      if (ybm) MOE_CR(false, true); else MOE_CR(false, false);
    }
#undef MOE_CR
    return hipGetLastError();
  }
  dim3 grid(T, (H / 4 + 255) / 256), block(256);
#define MOE_CB(F32, KM)                                                                          \
  do {                                                                                           \
    if (ybm)                                                                                     \
      hipLaunchKernelGGL((combine_kernel<F32, KM, true>), grid, block, 0, s, y, H, inv, w, k, P, \
                         has_shared, out, T, planes, plane, yb, ys, dbg);                        \
    else                                                                                         \
      hipLaunchKernelGGL((combine_kernel<F32, KM, false>), grid, block, 0, s, y, H, inv, w, k,   \
                         P, has_shared, out, T, planes, plane, yb, ys, dbg);                     \
  } while (0)
#define MOE_CB_K(F32)                   \
  if (k <= 2) MOE_CB(F32, 2);           \
  else if (k <= 4) MOE_CB(F32, 4);      \
  else if (k <= 8) MOE_CB(F32, 8);      \
  else MOE_CB(F32, 16)
  if (out_f32) {
    MOE_CB_K(true);
  } else {
    MOE_CB_K(false);
  }
#undef MOE_CB_K
#undef MOE_CB
  return hipGetLastError();
}

}  // namespace moe
