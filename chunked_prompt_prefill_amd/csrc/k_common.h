// Device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace cp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

__device__ __forceinline__ uint16_t float_to_half_bits(float v) {
  return __builtin_bit_cast(uint16_t, (_Float16)v);   // IEEE round-to-nearest-even
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
}

// 16 signed bytes times a scale, exactly (|q| <= 128, d from fp16: the product fits in
// float32), then rounded to bf16.  q is formed as ubyte(x ^ 0x80) - 128 so that each
// value costs one byte convert and one fused multiply-add: u*d - 128*d == q*d exactly.
__device__ __forceinline__ void dequant16_bf16(uint4 raw, float d, uint4& lo, uint4& hi) {
  const float nd = -128.0f * d;
  uint32_t w[4] = {raw.x ^ 0x80808080u, raw.y ^ 0x80808080u, raw.z ^ 0x80808080u,
                   raw.w ^ 0x80808080u};
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float f0 = fmaf((float)(w[i] & 0xFFu), d, nd);
    float f1 = fmaf((float)((w[i] >> 8) & 0xFFu), d, nd);
    float f2 = fmaf((float)((w[i] >> 16) & 0xFFu), d, nd);
    float f3 = fmaf((float)(w[i] >> 24), d, nd);
    o[2 * i] = pack_bf16x2(f0, f1);
    o[2 * i + 1] = pack_bf16x2(f2, f3);
  }
  lo = make_uint4(o[0], o[1], o[2], o[3]);
  hi = make_uint4(o[4], o[5], o[6], o[7]);
}

// 8 signed bytes (two dwords) times per-element float scales -> 8 f16 (one uint4).
__device__ __forceinline__ uint4 dequant8_f16(uint32_t w0, uint32_t w1, const float* d) {
  uint32_t w[2] = {w0, w1};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    float f0 = (float)(int8_t)(w[i] & 0xFFu) * d[4 * i + 0];
    float f1 = (float)(int8_t)((w[i] >> 8) & 0xFFu) * d[4 * i + 1];
    float f2 = (float)(int8_t)((w[i] >> 16) & 0xFFu) * d[4 * i + 2];
    float f3 = (float)(int8_t)(w[i] >> 24) * d[4 * i + 3];
    o[2 * i] = pack_f16x2(f0, f1);
    o[2 * i + 1] = pack_f16x2(f2, f3);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

__device__ __forceinline__ float warp_max32(float v) {   // max over aligned groups of 32 lanes
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

}  // namespace cp
