// The roofline's two denominators, measured on the device the library runs on.
//
//   * mfma_peak_kernel: fp16 v_mfma_f32_32x32x16 on register operands only, four
//     independent accumulators per wave so consecutive products never wait on each other,
//     two waves per SIMD; no memory traffic except one float per wave at the end (so the
//     work cannot be discarded).  Its rate is the dense fp16 MFMA rate at the clock the
//     chip holds under a pure matrix load.
//   * stream_read_kernel: every byte of a buffer read once with 16-byte loads in a
//     grid-stride loop, folded into one value per thread; its rate is the HBM read
//     bandwidth an access pattern like the kernels' weight streams can reach.
#include "cp_internal.h"
#include "k_common.h"

#include <algorithm>

namespace cp {

__global__ __launch_bounds__(256) void mfma_peak_kernel(int32_t iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const _Float16 va = (_Float16)(1.0f + 0.001f * (float)lane);
  const _Float16 vb = (_Float16)(0.5f - 0.001f * (float)lane);
  const f16x8 a = {va, va, va, va, va, va, va, va};
  const f16x8 b = {vb, vb, vb, vb, vb, vb, vb, vb};
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c3, 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
  if (lane == 0) sink[(int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6)] = s;
}

typedef unsigned int u32x4_p __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_p* __restrict__ buf, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
    const u32x4_p v = __builtin_nontemporal_load(buf + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// Launch shapes: 2048 workgroups of 4 waves (8 per CU over the 256 CUs) for the MFMA loop;
// 4096 workgroups of 256 threads for the stream.  The sinks take one float per wave and
// one word per thread respectively.
constexpr int kPeakWgs = 2048;
constexpr int kStreamWgs = 4096;

size_t peak_sink_bytes() {
  return std::max<size_t>((size_t)kPeakWgs * 4 * sizeof(float), (size_t)kStreamWgs * 256 * sizeof(uint32_t));
}

hipError_t launch_mfma_peak(int32_t iters, float* sink, hipStream_t s, double* flops) {
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(kPeakWgs), dim3(256), 0, s, iters, sink);
  *flops = (double)kPeakWgs * 4 * iters * 4 * (2.0 * 32 * 32 * 16);
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* buf, int64_t n_bytes, uint32_t* sink, hipStream_t s) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(kStreamWgs), dim3(256), 0, s,
                     reinterpret_cast<const u32x4_p*>(buf), n_bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace cp
