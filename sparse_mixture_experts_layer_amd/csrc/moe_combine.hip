// Combine / unpermute: y[t] = Y[shared row of t] + sum_j w[t,j] * Y[inv[t,j]],
// accumulated in fp32 in a fixed order (shared first, then j = 0..k-1) and
// rounded once to the output dtype.  The shared expert is always on and enters
// unweighted (llm-atlas "Step-3.5-Flash", "Champs bruts du config.json",
// share_expert_dim; that it is added outside the renormalised weights is the
// reading taken where the pages are silent).
#include "moe_common.hpp"
#include "moe_kernels.hpp"

namespace moe {
namespace {

template <bool OUT_F32>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y, int H,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ w, int k, int P,
                                                      int has_shared, void* __restrict__ out,
                                                      int T) {
  const int t = blockIdx.x;
  if (t >= T) return;
  __shared__ int rows[kMaxTopK];
  __shared__ float ws[kMaxTopK];
  if (threadIdx.x < k) {
    int r = inv[(size_t)t * k + threadIdx.x];
    rows[threadIdx.x] = r < 0 ? 0 : (r >= P ? P - 1 : r);
    ws[threadIdx.x] = w[(size_t)t * k + threadIdx.x];
  }
  __syncthreads();
  // Each thread owns kChunks column groups of 4 per pass, so every row's
  // loads for all of them are in flight together (bandwidth-bound kernel).
  // Y is read once: nontemporal loads keep it from displacing cached data.
  constexpr int kChunks = 4;
  const int stride = blockDim.x * 4;
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
    for (int j = 0; j < k; ++j) {
      const float* yr = y + (size_t)rows[j] * H;
      const float wj = ws[j];
      f32x4 v[kChunks];
#pragma unroll
      for (int i = 0; i < kChunks; ++i)
        v[i] = col[i] < H ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(yr + col[i])) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < kChunks; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][e] += wj * v[i][e];
    }
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      if (col[i] >= H) continue;
      if (OUT_F32) {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + (size_t)t * H + col[i]) = acc[i];
      } else {
        uint2 pk;
        pk.x = pack_bf16x2(acc[i][0], acc[i][1]);
        pk.y = pack_bf16x2(acc[i][2], acc[i][3]);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + (size_t)t * H + col[i]) = pk;
      }
    }
  }
}

}  // namespace

hipError_t launch_combine(bool out_f32, const float* y, int H, const int32_t* inv, const float* w,
                          int k, int P, int has_shared, void* out, int T, hipStream_t s) {
  dim3 grid(T), block(256);
  if (out_f32)
    hipLaunchKernelGGL((combine_kernel<true>), grid, block, 0, s, y, H, inv, w, k, P, has_shared,
                       out, T);
  else
    hipLaunchKernelGGL((combine_kernel<false>), grid, block, 0, s, y, H, inv, w, k, P, has_shared,
                       out, T);
  return hipGetLastError();
}

}  // namespace moe
