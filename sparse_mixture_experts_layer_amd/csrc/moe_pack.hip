// Weight packing (run once per layer): canonical [N][K] matrices -> the layouts
// the streaming GEMMs read with one coalesced 1 KiB access per wave.
//
// bf16:  fragment (nb, kk, g) = rows 16*nb .. +15, k 32*kk .. +31 of source g,
//        stored as 64 lanes x 8 bf16 in MFMA operand order (lane l: row l % 16,
//        k 8*(l/16) .. +7); order [N/16][K/32][G][64][8].  G = 2 interleaves
//        gate and up so one wave reads both halves of its 16 output features.
// INT4:  block (nb, kb, g) = rows 16*nb .. +15, k 128*kb .. +127: lane l holds
//        row l % 16 as four dwords, dword kg covering k = 128*kb + 32*kg +
//        8*(l/16) + [0..7] with nibbles in the order k0,k2,k4,k6,k1,k3,k5,k7
//        (what the in-register widening expects); 1 KiB per block.  Scales of
//        a block: [4 quads][4 kg][4 rows] fp16 = 128 bytes, quad q holding rows
//        4q .. 4q+3 (the C rows a lane of that quad owns).
#include "moe_common.hpp"
#include "moe_kernels.hpp"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void pack_bf16_kernel(const uint16_t* __restrict__ src0,
                                                        const uint16_t* __restrict__ src1, int G,
                                                        int N, int K, size_t src_stride,
                                                        uint8_t* __restrict__ dst,
                                                        size_t dst_stride) {
  const size_t nchunks = (size_t)(N / 16) * (K / 32) * G * 64;
  const size_t b = blockIdx.y;
  for (size_t c = (size_t)blockIdx.x * blockDim.x + threadIdx.x; c < nchunks;
       c += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(c & 63);
    size_t rest = c >> 6;
    const int g = (int)(rest % G);
    rest /= G;
    const int kk = (int)(rest % (K / 32));
    const int nb = (int)(rest / (K / 32));
    const uint16_t* src = (g == 0 ? src0 : src1) + b * src_stride;
    const size_t so = (size_t)(nb * 16 + (lane & 15)) * K + kk * 32 + (lane >> 4) * 8;
    const u32x4 v = load16(src + so);
    *reinterpret_cast<u32x4*>(dst + b * dst_stride + c * 16) = v;
  }
}

__device__ __forceinline__ uint32_t nibble(const uint8_t* row, int k) {
  const uint8_t byte = row[k >> 1];
  return (k & 1) ? (byte >> 4) : (byte & 0xf);
}

__global__ __launch_bounds__(256) void pack_int4_kernel(
    const uint8_t* __restrict__ q0, const uint8_t* __restrict__ q1, const uint16_t* __restrict__ s0,
    const uint16_t* __restrict__ s1, int G, int N, int K, size_t q_stride, size_t s_stride,
    uint8_t* __restrict__ dq, uint8_t* __restrict__ ds, size_t dst_stride) {
  const int nkb = K / 128;
  const size_t nchunks = (size_t)(N / 16) * nkb * G * 64;
  const size_t b = blockIdx.y;
  for (size_t c = (size_t)blockIdx.x * blockDim.x + threadIdx.x; c < nchunks;
       c += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(c & 63);
    size_t rest = c >> 6;
    const int g = (int)(rest % G);
    rest /= G;
    const int kb = (int)(rest % nkb);
    const int nb = (int)(rest / nkb);
    const uint8_t* q = (g == 0 ? q0 : q1) + b * q_stride;
    const uint16_t* s = (g == 0 ? s0 : s1) + b * s_stride;
    const uint8_t* row = q + (size_t)(nb * 16 + (lane & 15)) * (K / 2);
    u32x4 out;
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
      const int k0 = kb * 128 + kg * 32 + (lane >> 4) * 8;
      const int order[8] = {0, 2, 4, 6, 1, 3, 5, 7};
      uint32_t w = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) w |= nibble(row, k0 + order[i]) << (4 * i);
      out[kg] = w;
    }
    *reinterpret_cast<u32x4*>(dq + b * dst_stride + c * 16) = out;
    // scales: lanes 0..15 of each (nb, kb, g) write the 64 entries, 4 each
    if (lane < 16) {
      const int quad = lane >> 2, kg = lane & 3;
      uint16_t* sd = reinterpret_cast<uint16_t*>(ds + b * dst_stride) + (c >> 6) * 64 +
                     quad * 16 + kg * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sd[i] = s[(size_t)(nb * 16 + quad * 4 + i) * (K / 32) + kb * 4 + kg];
    }
  }
}

}  // namespace

hipError_t launch_pack_bf16(const uint16_t* src0, const uint16_t* src1, int G, int N, int K,
                            int batch, size_t src_batch_stride, uint8_t* dst,
                            size_t dst_batch_stride, hipStream_t s) {
  const size_t nchunks = (size_t)(N / 16) * (K / 32) * G * 64;
  const unsigned gx = (unsigned)((nchunks + 255) / 256 < 4096 ? (nchunks + 255) / 256 : 4096);
  hipLaunchKernelGGL(pack_bf16_kernel, dim3(gx, batch), dim3(256), 0, s, src0, src1, G, N, K,
                     src_batch_stride, dst, dst_batch_stride);
  return hipGetLastError();
}

hipError_t launch_pack_int4(const uint8_t* q0, const uint8_t* q1, const uint16_t* s0,
                            const uint16_t* s1, int G, int N, int K, int batch,
                            size_t q_batch_stride, size_t s_batch_stride, uint8_t* dst_q,
                            uint8_t* dst_s, size_t dst_batch_stride, hipStream_t s) {
  const size_t nchunks = (size_t)(N / 16) * (K / 128) * G * 64;
  const unsigned gx = (unsigned)((nchunks + 255) / 256 < 4096 ? (nchunks + 255) / 256 : 4096);
  hipLaunchKernelGGL(pack_int4_kernel, dim3(gx, batch), dim3(256), 0, s, q0, q1, s0, s1, G, N, K,
                     q_batch_stride, s_batch_stride, dst_q, dst_s, dst_batch_stride);
  return hipGetLastError();
}

}  // namespace moe
