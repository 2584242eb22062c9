// Device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace cp {

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

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
}

// Two int8 weights as exact fp16 integers: byte b of x (x = raw ^ 0x80808080, so b is
// the weight + 128) becomes the fp16 bit pattern 0x64bb = 1024 + b, and subtracting 1152
// leaves the weight itself (every integer below 2048 is exact in fp16).  sel picks the two
// bytes (v_perm_b32: bytes 0-3 from x, byte 4 = 0x64 from the constant).
__device__ __forceinline__ f16x2 q8_pair_f16(uint32_t x, uint32_t sel) {
  const uint32_t bits = __builtin_amdgcn_perm(0x64646464u, x, sel);
  const f16x2 big = __builtin_bit_cast(f16x2, bits);
  const f16x2 off = {(_Float16)1152.0f, (_Float16)1152.0f};
  return big - off;
}

// 4 int8 weights (one dword) times the block's fp16 scale d -> two packed fp16 pairs, each
// the correctly rounded fp16 of d*q (one packed fp16 multiply of exact operands).
__device__ __forceinline__ void dequant4_f16(uint32_t raw, f16x2 d2, uint32_t& lo, uint32_t& hi) {
  const uint32_t x = raw ^ 0x80808080u;
  lo = __builtin_bit_cast(uint32_t, q8_pair_f16(x, 0x04010400u) * d2);
  hi = __builtin_bit_cast(uint32_t, q8_pair_f16(x, 0x04030402u) * d2);
}

// 16 signed bytes times a block scale (fp16 bits) -> 16 fp16 in two uint4, in byte order.
__device__ __forceinline__ void dequant16_f16(uint4 raw, uint32_t d_bits, uint4& lo, uint4& hi) {
  const _Float16 d = __builtin_bit_cast(_Float16, (uint16_t)d_bits);
  const f16x2 d2 = {d, d};
  uint32_t o[8];
  dequant4_f16(raw.x, d2, o[0], o[1]);
  dequant4_f16(raw.y, d2, o[2], o[3]);
  dequant4_f16(raw.z, d2, o[4], o[5]);
  dequant4_f16(raw.w, d2, o[6], o[7]);
  lo = make_uint4(o[0], o[1], o[2], o[3]);
  hi = make_uint4(o[4], o[5], o[6], o[7]);
}

// 16 signed bytes, each with its own fp16 scale (s0: scales of bytes 0-7, s1: of bytes
// 8-15, two per dword in byte order) -> 16 fp16, each the correctly rounded d*q.
__device__ __forceinline__ void dequant16_f16_scales(uint4 raw, uint4 s0, uint4 s1, uint4& lo, uint4& hi) {
  const uint32_t sc[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t x = w[i] ^ 0x80808080u;
    o[2 * i] = __builtin_bit_cast(uint32_t, q8_pair_f16(x, 0x04010400u) * __builtin_bit_cast(f16x2, sc[2 * i]));
    o[2 * i + 1] = __builtin_bit_cast(uint32_t, q8_pair_f16(x, 0x04030402u) * __builtin_bit_cast(f16x2, sc[2 * i + 1]));
  }
  lo = make_uint4(o[0], o[1], o[2], o[3]);
  hi = make_uint4(o[4], o[5], o[6], o[7]);
}

// float -> fp16 for stored activations that are not bounded by construction (the SwiGLU
// product): saturated to the finite fp16 range, then rounded to nearest even.
__device__ __forceinline__ _Float16 f16_sat(float v) {
  return (_Float16)__builtin_amdgcn_fmed3f(v, -65504.0f, 65504.0f);
}

__device__ __forceinline__ float warp_max32(float v) {   // max over aligned groups of 32 lanes
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// silu(g) = g / (1 + e^-g), with the hardware reciprocal (1 ulp) in place of an IEEE
// division: the product is rounded to fp16 afterwards.  e^-g overflows to +inf for
// g < about -88, and then the reciprocal gives 0 and silu gives -0.
__device__ __forceinline__ float silu(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// The split-K sum of `splits` planes at p, p + plane, ... in plane order, p0 + p1 + p2 + ...
// in float32 (the fixed order every reader of split partial sums uses).  The loads are
// issued four at a time, so that they are in flight together instead of one per add.
__device__ __forceinline__ float4 split_sum4(const float* p, int64_t plane, int splits) {
  float4 acc = *reinterpret_cast<const float4*>(p);
  int s = 1;
  for (; s + 3 < splits; s += 4) {
    float4 a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = *reinterpret_cast<const float4*>(p + (s + j) * plane);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc.x += a[j].x; acc.y += a[j].y; acc.z += a[j].z; acc.w += a[j].w;
    }
  }
  for (; s < splits; ++s) {
    const float4 a = *reinterpret_cast<const float4*>(p + s * plane);
    acc.x += a.x; acc.y += a.y; acc.z += a.z; acc.w += a.w;
  }
  return acc;
}
__device__ __forceinline__ float split_sum1(const float* p, int64_t plane, int splits) {
  float acc = p[0];
  int s = 1;
  for (; s + 3 < splits; s += 4) {
    float a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = p[(s + j) * plane];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc += a[j];
  }
  for (; s < splits; ++s) acc += p[s * plane];
  return acc;
}

}  // namespace cp
