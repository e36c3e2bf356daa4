// Weight packing (run once per layer): canonical [N][K] matrices -> the layouts
// the streaming GEMMs read as one contiguous 4 KiB block per wave per k-step.
//
// A 16x32 bf16 fragment is stored as 64 lanes x 8 bf16 in MFMA operand order
// (lane l: row l % 16, k 8*(l/16) .. +7).  A block is F*S fragments of S
// sources: block (nb, kk) holds, for source g and sub-block f, rows
// (nb*F + f)*16 .. +15 and k 32*kk .. +31, at position j = g*F + f.
//   gate/up: S = 2 (gate, up), F = 2 -> [W/32][H/32][g0 g1 u0 u1]
//   down:    S = 1,           F = 4 -> [H/64][W/32][f0 f1 f2 f3]
// INT4 blocks cover 128 k: lane l holds row l % 16 as four dwords, dword kg
// covering k = 128*kb + 32*kg + 8*(l/16) + [0..7] with nibbles in the order
// k0,k2,k4,k6,k1,k3,k5,k7 (what the in-register widening expects).  The scales
// of block (nb, kb) follow as [16 rows][F*S][4 kg] fp16, so a lane reads the
// 16 scales of its row contiguously.
#include "moe_common.hpp"
#include "moe_kernels.hpp"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void pack_bf16_kernel(const uint16_t* __restrict__ src0,
                                                        const uint16_t* __restrict__ src1, int S,
                                                        int F, int N, int K, size_t src_stride,
                                                        uint8_t* __restrict__ dst,
                                                        size_t dst_stride) {
  const size_t nchunks = (size_t)N / 16 * S * (K / 32) * 64;
  const size_t b = blockIdx.y;
  const int FS = F * S;
  for (size_t c = (size_t)blockIdx.x * blockDim.x + threadIdx.x; c < nchunks;
       c += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(c & 63);
    size_t q = c >> 6;
    const int j = (int)(q % FS);
    q /= FS;
    const int kk = (int)(q % (K / 32));
    const int nb = (int)(q / (K / 32));
    const int g = j / F, f = j % F;
    const uint16_t* src = (g == 0 ? src0 : src1) + b * src_stride;
    const size_t so = (size_t)((nb * F + f) * 16 + (lane & 15)) * K + kk * 32 + (lane >> 4) * 8;
    *reinterpret_cast<u32x4*>(dst + b * dst_stride + c * 16) = load16(src + so);
  }
}

__device__ __forceinline__ uint32_t nibble(const uint8_t* row, int k) {
  const uint8_t byte = row[k >> 1];
  return (k & 1) ? (byte >> 4) : (byte & 0xf);
}

__global__ __launch_bounds__(256) void pack_int4_kernel(
    const uint8_t* __restrict__ q0, const uint8_t* __restrict__ q1, const uint16_t* __restrict__ s0,
    const uint16_t* __restrict__ s1, int S, int F, int N, int K, size_t q_stride, size_t s_stride,
    uint8_t* __restrict__ dq, uint8_t* __restrict__ ds, size_t dst_stride) {
  const int nkb = K / 128, FS = F * S;
  const size_t nchunks = (size_t)N / 16 * S * nkb * 64;
  const size_t b = blockIdx.y;
  for (size_t c = (size_t)blockIdx.x * blockDim.x + threadIdx.x; c < nchunks;
       c += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(c & 63);
    size_t qb = c >> 6;
    const int j = (int)(qb % FS);
    qb /= FS;
    const int kb = (int)(qb % nkb);
    const int nb = (int)(qb / nkb);
    const int g = j / F, f = j % F;
    const uint8_t* q = (g == 0 ? q0 : q1) + b * q_stride;
    const uint16_t* s = (g == 0 ? s0 : s1) + b * s_stride;
    const int r16 = lane & 15;
    const int row = (nb * F + f) * 16 + r16;
    const uint8_t* qrow = q + (size_t)row * (K / 2);
    u32x4 out;
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
      const int k0 = kb * 128 + kg * 32 + (lane >> 4) * 8;
      const int order[8] = {0, 2, 4, 6, 1, 3, 5, 7};
      uint32_t w = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) w |= nibble(qrow, k0 + order[i]) << (4 * i);
      out[kg] = w;
    }
    *reinterpret_cast<u32x4*>(dq + b * dst_stride + c * 16) = out;
    if (lane < 16) {  // the 4 scales of (row, block j) for the 4 k-groups
      uint16_t* sd = reinterpret_cast<uint16_t*>(ds + b * dst_stride) +
                     ((size_t)(nb * nkb + kb) * 16 + r16) * FS * 4 + j * 4;
#pragma unroll
      for (int kg = 0; kg < 4; ++kg) sd[kg] = s[(size_t)row * (K / 32) + kb * 4 + kg];
    }
  }
}

unsigned grid_x(size_t nchunks) {
  const size_t blocks = (nchunks + 255) / 256;
  return (unsigned)(blocks < 4096 ? blocks : 4096);
}

}  // namespace

hipError_t launch_pack_bf16(const uint16_t* src0, const uint16_t* src1, int S, int F, int N,
                            int K, int batch, size_t src_batch_stride, uint8_t* dst,
                            size_t dst_batch_stride, hipStream_t s) {
  const size_t nchunks = (size_t)N / 16 * S * (K / 32) * 64;
  hipLaunchKernelGGL(pack_bf16_kernel, dim3(grid_x(nchunks), batch), dim3(256), 0, s, src0, src1,
                     S, F, N, K, src_batch_stride, dst, dst_batch_stride);
  return hipGetLastError();
}

hipError_t launch_pack_int4(const uint8_t* q0, const uint8_t* q1, const uint16_t* s0,
                            const uint16_t* s1, int S, int F, int N, int K, int batch,
                            size_t q_batch_stride, size_t s_batch_stride, uint8_t* dst_q,
                            uint8_t* dst_s, size_t dst_batch_stride, hipStream_t s) {
  const size_t nchunks = (size_t)N / 16 * S * (K / 128) * 64;
  hipLaunchKernelGGL(pack_int4_kernel, dim3(grid_x(nchunks), batch), dim3(256), 0, s, q0, q1, s0,
                     s1, S, F, N, K, q_batch_stride, s_batch_stride, dst_q, dst_s,
                     dst_batch_stride);
  return hipGetLastError();
}

}  // namespace moe
