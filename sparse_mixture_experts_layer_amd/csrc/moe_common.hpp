// Shared device helpers for the gfx950 MoE kernels: bf16 bit conversions,
// 16-byte vector loads, and the MFMA fragment conventions every kernel uses.
//
// MFMA v_mfma_f32_16x16x32_bf16 (wave64), as used throughout:
//   A operand (16 x 32): lane l holds row (l % 16), k = 8*(l / 16) + [0..7]
//   B operand (32 x 16): lane l holds col (l % 16), k = 8*(l / 16) + [0..7]
//   C/D (16 x 16 fp32):  lane l holds rows 4*(l / 16) + [0..3] of col (l % 16)
// A packed weight "fragment" is 16 rows x 32 k of a [N][K] matrix stored as
// 64 lanes x 8 bf16 (1 KiB) in exactly the A/B register order, so one
// 16-byte load per lane fetches a whole operand with a fully coalesced 1 KiB
// wave access.  Weights sit on the A side (their rows become C rows) and
// tokens on the B side; the sum over k is order-free, so A and B only have to
// agree on which k each (lane, element) holds.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kFragBytes = 1024;   // one 16x32 bf16 fragment
constexpr int kMaxTopK = 16;
constexpr int kMaxExperts = 512;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even (NaN to a quiet NaN): gfx950's
// v_cvt_pk_bf16_f32, two values per instruction (lo in the low half).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Streamed once: no reuse expected in the caches.
__device__ __forceinline__ u32x4 load16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Split 8 fp32 values into bf16 hi + lo with x ~= hi + lo (relative residual
// below 2^-16): two MFMAs over (hi, lo) give near-fp32 products against a bf16
// operand.  hi is x rounded to nearest even; lo is the rounded remainder.
__device__ __forceinline__ void split_f32x8(const float* x, u32x4& hi, u32x4& lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t h = pack_bf16x2(x[2 * i], x[2 * i + 1]);
    const float r0 = x[2 * i] - __uint_as_float(h << 16);
    const float r1 = x[2 * i + 1] - __uint_as_float(h & 0xffff0000u);
    hi[i] = h;
    lo[i] = pack_bf16x2(r0, r1);
  }
}

// SiLU with the hardware exponential and reciprocal (about 1 ulp each, far
// below the bf16 rounding of h; an IEEE division cost the gate/up epilogue a
// fifth of its time).
__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// h = silu(g) * u; a limit lim > 0 first bounds g to at most lim and u to
// [-lim, lim] (the SwiGLU limits of Step-3.5-Flash's last layers, 7 routed and
// 16 shared); lim == 0 leaves both untouched.
__device__ __forceinline__ float swiglu(float g, float u, float lim) {
  if (lim > 0.f) {
    g = fminf(g, lim);
    u = fminf(fmaxf(u, -lim), lim);
  }
  return silu(g) * u;
}

// Expanding an INT4 dword (8 nibbles stored in the order k0,k2,k4,k6,k1,k3,k5,k7)
// into 8 bf16 values 128 + u, u = q + 8 in [0, 15]: bf16 bits 0x4300 | u are
// exactly 128 + u, so two masks and an OR per pair produce exact operands; the
// constant 136 = 128 + 8 is removed by a second MFMA against -136.
__device__ __forceinline__ bf16x8 int4_to_bf16x8_biased(uint32_t w) {
  u32x4 r;
  r[0] = (w & 0x000f000fu) | 0x43004300u;
  r[1] = ((w >> 4) & 0x000f000fu) | 0x43004300u;
  r[2] = ((w >> 8) & 0x000f000fu) | 0x43004300u;
  r[3] = ((w >> 12) & 0x000f000fu) | 0x43004300u;
  return as_bf16x8(r);
}

// Index checks of debug builds (compiled with MOE_DEBUG=1).  Where a kernel
// reads an index from memory and keeps it in range (an expert id, a token id,
// a permuted row, a tile-list entry), a debug build also reports a value that
// was out of range: the first report of a call stores its code in flag[0]
// and the value in flag[1] (a workspace word pair the router kernel clears);
// the kernel then goes on as a release build does, with the index clamped or
// the tile skipped -- no trap.  Release builds compile the checks away.
#ifndef MOE_DEBUG
#define MOE_DEBUG 0
#endif
enum { kDbgExpert = 1, kDbgToken = 2, kDbgRow = 3, kDbgTile = 4 };

__device__ __forceinline__ void dbg_check(int32_t* flag, bool ok, int code, int value) {
#if MOE_DEBUG
  if (!ok && flag && atomicCAS(flag, 0, code) == 0) atomicExch(flag + 1, value);
#else
  (void)flag, (void)ok, (void)code, (void)value;
#endif
}

// Workspace tile-list entry: (group << 16) | m, group = expert (E = shared).
__device__ __forceinline__ int tile_group(int v) { return v >> 16; }
__device__ __forceinline__ int tile_m(int v) { return v & 0xffff; }

}  // namespace moe
