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
  for (int c = threadIdx.x * 4; c < H; c += blockDim.x * 4) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (has_shared) acc = *reinterpret_cast<const f32x4*>(y + (size_t)(P + t) * H + c);
    for (int j = 0; j < k; ++j) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(y + (size_t)rows[j] * H + c);
      const float wj = ws[j];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] += wj * v[i];
    }
    if (OUT_F32) {
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + (size_t)t * H + c) = acc;
    } else {
      uint2 pk;
      pk.x = pack_bf16x2(acc[0], acc[1]);
      pk.y = pack_bf16x2(acc[2], acc[3]);
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + (size_t)t * H + c) = pk;
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
