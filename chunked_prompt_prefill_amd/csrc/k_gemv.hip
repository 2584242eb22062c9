// q8_0-weight GEMM for a handful of rows (chunks of 1-4 tokens), gfx950.
//
//   out[m][n] = sum_k A[m][k] * W[n][k],  M <= 4, A fp16, W q8_0 blocks of 32.
//
// With so few rows there is nothing for the matrix cores to amortise: the launch is a
// stream of the weights, and what matters is keeping enough bytes in flight and spending
// few VALU cycles per weight byte.  The arithmetic is the same as the MFMA kernels':
// every weight is the correctly rounded fp16 of d*q (byte permute, packed add, packed
// multiply by the block scale) and products of fp16 values accumulate in fp32
// (v_dot2_f32_f16, two products per instruction).
//
// Mapping.  The weights sit in the MFMA-ordered arena: per 32-row group and q8_0 block,
// 64 16-byte pieces, piece 32*h + r holding row r's block columns 16h..16h+15.  A wave
// owns a pair of 32-row groups (2j, 2j+1) — for the SwiGLU weights that pair is one gate
// group and its up group — lane 32*g + r holding row r of group 2j+g for all of K.  It
// reads piece 32*h + r of both groups (two contiguous 512-byte runs), so at each step all
// 64 lanes need the same 16 activations per row: those come through the scalar unit
// (s_load from a wave-uniform address) and feed v_dot2 as a scalar operand, with no LDS
// traffic.  Each lane's dot product runs over whole rows, so no lane-to-lane reduction is
// needed; per 128-wide K stage a lane loads 8 pieces and one 8-byte group of four block
// scales.
//
// Work split.  A workgroup of 4 waves owns one pair of groups (64 output columns) and a
// range of K stages, in rounds of 8 stages with two adjacent stages per wave; the waves'
// sums meet in LDS and are added in wave order.  S workgroups split K for each pair, one
// round each as planned (so a wave issues all of its loads before it waits: the memory
// parallelism comes from many resident waves, not from a software pipeline).  With S > 1
// they write partial sums [S][M][N] that the split-K reduction kernel adds in split order
// and passes through the epilogue (a kernel boundary is the cheap way to make partials of
// all eight XCDs visible; a device-wide fence per workgroup writes back and invalidates
// the XCD's L2 and costs far more).  The result is deterministic for a given M, N, K.
#include "cp_internal.h"
#include "k_common.h"

namespace cp {

namespace {

typedef const __attribute__((address_space(4))) uint32_t* cptr_t;   // scalar-loadable

constexpr int SW = 4;   // waves per workgroup

typedef unsigned int u32x4_g __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_g __attribute__((ext_vector_type(2)));

// loads through global (address space 1) pointers; the struct-argument pointers would
// otherwise become flat loads
__device__ __forceinline__ uint4 gload16(const int8_t* base, int64_t piece) {
  const u32x4_g v = *((const __attribute__((address_space(1))) u32x4_g*)base + piece);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 gload8(const uint32_t* base, int64_t idx) {
  const u32x2_g v = *((const __attribute__((address_space(1))) u32x2_g*)base + idx);
  return make_uint2(v.x, v.y);
}

struct Stage {
  uint4 q[4][2];   // [block][half]
  uint2 d;         // the lane's row: four block scales (fp16 bits)
};

template <int MR, int MODE>
__global__ __launch_bounds__(256) void gemm_q8_skinny_kernel(GemmArgs g) {
  __shared__ float sred[SW][MR][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int S = g.splits;
  const int j = blockIdx.x / S, s = blockIdx.x % S;
  const int grp = lane >> 5, r = lane & 31;
  const int KB = g.K / QK, KQ = g.K / 128;
  const int64_t n32 = 2 * j + grp;
  const int st0 = (int)((int64_t)s * KQ / S), st1 = (int)((int64_t)(s + 1) * KQ / S);
  const int M = g.M;

  float acc[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m] = 0.0f;

  auto load = [&](int kq, Stage& b) {
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        b.q[jb][h] = gload16(g.wq, (n32 * KB + 4 * kq + jb) * 64 + 32 * h + r);
    b.d = gload8(g.wd, (n32 * KQ + kq) * 32 + r);
  };
  auto compute = [&](int kq, const Stage& b) {
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      const uint32_t dbits = ((jb < 2 ? b.d.x : b.d.y) >> (16 * (jb & 1))) & 0xFFFFu;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint4 lo, hi;
        dequant16_f16(b.q[jb][h], dbits, lo, hi);
        const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        const int64_t col = (int64_t)(4 * kq + jb) * QK + 16 * h;
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          if (m >= M) break;
          const cptr_t a = (cptr_t)(g.A + (int64_t)m * g.lda + col);
#pragma unroll
          for (int i = 0; i < 8; ++i)
            acc[m] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a[i]), __builtin_bit_cast(f16x2, w[i]),
                                            acc[m], false);
        }
      }
    }
  };

  // Rounds of 8 stages: wave w takes stages 2w and 2w+1 of the round, both loaded before
  // either is multiplied (18 loads in flight per lane); a stage past the range re-reads the
  // range's last one (in bounds, never multiplied), so the loads are unconditional.  The
  // planned split gives each workgroup one round.
  for (int base = st0; base < st1; base += 2 * SW) {
    const int k0 = base + 2 * wave, k1 = k0 + 1, last = st1 - 1;
    Stage b0, b1;
    load(min(k0, last), b0);
    load(min(k1, last), b1);
    if (k0 < st1) compute(k0, b0);
    if (k1 < st1) compute(k1, b1);
  }

#pragma unroll
  for (int m = 0; m < MR; ++m) sred[wave][m][lane] = acc[m];
  __syncthreads();
  if (wave != 0) return;

  float v[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) v[m] = ((sred[0][m][lane] + sred[1][m][lane]) + sred[2][m][lane]) + sred[3][m][lane];
  const int64_t n = (int64_t)j * 64 + lane;

  if constexpr (MODE == GM_PARTIAL) {
#pragma unroll
    for (int m = 0; m < MR; ++m)
      if (m < M) g.partial[((int64_t)s * M + m) * g.N + n] = v[m];
    return;
  }

#pragma unroll
  for (int m = 0; m < MR; ++m) {
    if (m >= M) break;
    if constexpr (MODE == GM_SWIGLU) {
      const float up = __shfl(v[m], (lane & 31) + 32, 64);
      if (lane < 32)
        reinterpret_cast<_Float16*>(g.out)[(int64_t)m * g.ldo + (int64_t)j * 32 + lane] = f16_sat(silu(v[m]) * up);
    } else if constexpr (MODE == GM_F32_ADD) {
      float* p = reinterpret_cast<float*>(g.out) + (int64_t)m * g.ldo + n;
      *p = *p + v[m];
    } else {
      reinterpret_cast<float*>(g.out)[(int64_t)m * g.ldo + n] = v[m];
    }
  }
}

template <int MR>
hipError_t launch_mr(const GemmArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((a.N / 64) * a.splits)), block(64 * SW);
  const int mode = a.splits > 1 ? GM_PARTIAL : a.mode;
  switch (mode) {
    case GM_F32: hipLaunchKernelGGL((gemm_q8_skinny_kernel<MR, GM_F32>), grid, block, 0, s, a); break;
    case GM_F32_ADD: hipLaunchKernelGGL((gemm_q8_skinny_kernel<MR, GM_F32_ADD>), grid, block, 0, s, a); break;
    case GM_SWIGLU: hipLaunchKernelGGL((gemm_q8_skinny_kernel<MR, GM_SWIGLU>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((gemm_q8_skinny_kernel<MR, GM_PARTIAL>), grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_skinny(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (a.M > kSkinnyMaxRows || a.N % 64 || a.K % 128 || a.n0 != 0 || a.splits < 1 ||
      (a.splits > 1 && !a.partial) || a.mode == GM_PARTIAL)
    return hipErrorInvalidValue;
  if (a.M == 1) return launch_mr<1>(a, s);
  if (a.M == 2) return launch_mr<2>(a, s);
  return launch_mr<4>(a, s);
}

}  // namespace cp
