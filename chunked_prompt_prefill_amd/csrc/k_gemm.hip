// q8_0-weight GEMM on bf16 MFMA (gfx950), fp32 accumulate.
//
//   out[m][n] = sum_k A[m][k] * W[n][k],  A bf16 activations, W q8_0 blocks of 32.
//
// Tiling.  A workgroup of 4 waves owns an MT x 256 output tile (MT = 32*MI); each wave
// owns 64 columns (two 32-column MFMA blocks) across all MT rows, so every weight
// element is dequantised exactly once per workgroup.  Per 64-wide K stage:
//   * A: MT x 64 bf16 staged in LDS (double buffered, 16-byte chunks XOR-swizzled by
//     row), read as the MFMA A operand by all four waves;
//   * W: loaded straight into registers from the repacked layout (1 KiB contiguous per
//     wave per 32-row group and 32-column block, already in MFMA lane order), dequantised
//     in registers (d*q exact in fp32, rounded to bf16) as the MFMA B operand.
// The K index inside a q8_0 block is permuted consistently on both operands so that a
// lane's 16 weight bytes are contiguous: lane half h, MFMA step s, element c <-> block
// column 16h + 8s + c.
// Epilogues: fp32 store, fp32 residual add, SwiGLU (gate/up columns interleaved in
// 32-column groups) to bf16, or split-K partials reduced by a separate kernel in a
// fixed order (deterministic: no float atomics).
// Grouped mode (routed experts): the row tile comes from a device tile table
// {expert, m0, m1}; A rows may be gathered through an index array.
#include "cp_internal.h"
#include "k_common.h"

namespace cp {

constexpr int KT = 64;
constexpr int NT = 256;

template <int MI, int MODE, bool GROUPED>
__global__ __launch_bounds__(256, 1) void gemm_q8_kernel(GemmArgs g) {
  constexpr int MT = MI * 32;
  constexpr int CHUNKS = MT * 8;           // 16-byte chunks per stage (8 per row)
  constexpr int LOADS = CHUNKS / 256;      // per thread
  __shared__ uint4 sA[2][CHUNKS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int KS = g.K / KT;

  int m0, rows, ntile, split, expert = 0;
  if constexpr (GROUPED) {
    const int t = blockIdx.x;
    if (t >= *g.n_tiles) return;
    const int4 tile = reinterpret_cast<const int4*>(g.tiles)[t];
    expert = tile.x;
    m0 = tile.y;
    rows = tile.z - tile.y;
    ntile = blockIdx.y;
    split = 0;
  } else {
    // XCD-aware order: workgroup i runs on XCD i % 8; give each XCD a contiguous range
    // of logical tiles (row tiles fastest) so tiles sharing weight columns share an L2.
    const int mtiles = (int)ceil_div(g.M, MT);
    const int ntiles = (int)ceil_div(g.N, NT);
    const int total = mtiles * ntiles * g.splits;
    const int i = blockIdx.x;
    const int xcd = i & 7, idx = i >> 3;
    const int q = total >> 3, r = total & 7;
    const int logical = (xcd < r) ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
    const int mt = logical % mtiles;
    const int rest = logical / mtiles;
    ntile = rest % ntiles;
    split = rest / ntiles;
    m0 = mt * MT;
    rows = min(MT, g.M - m0);
  }

  const int ks0 = (int)((int64_t)split * KS / g.splits);
  const int ks1 = (int)((int64_t)(split + 1) * KS / g.splits);
  const int n_wave = ntile * NT + wave * 64;
  const bool col_ok0 = n_wave < g.N;
  const bool col_ok1 = n_wave + 32 < g.N;

  // Per-thread A rows: row i*32 + tid/8, chunk tid%8.
  const __bf16* arow[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int r = i * 32 + (tid >> 3);
    if (r < rows) {
      int64_t pr = m0 + r;
      if (g.a_rows) pr = g.a_rows[m0 + r] / g.a_row_div;
      arow[i] = g.A + pr * g.lda + (tid & 7) * 8;
    } else {
      arow[i] = nullptr;
    }
  }

  const int KB = g.K / QK, KP = g.K / KT;
  const uint4* bq[2];
  const uint32_t* bd[2];
#pragma unroll
  for (int ni = 0; ni < 2; ++ni) {
    const int64_t n32 = (n_wave >> 5) + ni;
    bq[ni] = reinterpret_cast<const uint4*>(g.wq + expert * g.wq_estride) + n32 * KB * 64 + lane;
    bd[ni] = g.wd + expert * g.wd_estride + n32 * KP * 32 + l32;
  }

  uint4 ra[LOADS];
  uint4 rb[2][2];
  uint32_t rs[2];
  auto load_stage = [&](int ks) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i)
      ra[i] = arow[i] ? *reinterpret_cast<const uint4*>(arow[i] + ks * KT) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const bool ok = ni ? col_ok1 : col_ok0;
      if (ok) {
        rb[ni][0] = bq[ni][(2 * ks) * 64];
        rb[ni][1] = bq[ni][(2 * ks + 1) * 64];
        rs[ni] = bd[ni][ks * 32];
      } else {
        rb[ni][0] = rb[ni][1] = make_uint4(0, 0, 0, 0);
        rs[ni] = 0;
      }
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int r = i * 32 + (tid >> 3);
      const int c = tid & 7;
      sA[buf][r * 8 + (c ^ (r & 7))] = ra[i];
    }
  };

  f32x16 acc[MI][2];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mi][ni][e] = 0.0f;

  if (ks0 < ks1) {
    load_stage(ks0);
    store_stage(0);
  }
  __syncthreads();

  for (int ks = ks0; ks < ks1; ++ks) {
    const int cur = (ks - ks0) & 1;
    uint4 cb[2][2] = {{rb[0][0], rb[0][1]}, {rb[1][0], rb[1][1]}};
    uint32_t cs[2] = {rs[0], rs[1]};
    const bool more = ks + 1 < ks1;
    if (more) load_stage(ks + 1);
#pragma unroll
    for (int kbl = 0; kbl < 2; ++kbl) {
      uint4 b[2][2];
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const float d = half_bits_to_float(kbl ? (cs[ni] >> 16) : (cs[ni] & 0xFFFFu));
        dequant16_bf16(cb[ni][kbl], d, b[ni][0], b[ni][1]);
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
          const int r = mi * 32 + l32;
          const int c = kbl * 4 + 2 * h + s;
          const uint4 a = sA[cur][r * 8 + (c ^ (r & 7))];
          const bf16x8 av = __builtin_bit_cast(bf16x8, a);
          if (col_ok0)
            acc[mi][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                av, __builtin_bit_cast(bf16x8, b[0][s]), acc[mi][0], 0, 0, 0);
          if (col_ok1)
            acc[mi][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                av, __builtin_bit_cast(bf16x8, b[1][s]), acc[mi][1], 0, 0, 0);
        }
      }
    }
    if (more) store_stage(cur ^ 1);
    __syncthreads();
  }

  // Epilogue.  acc[mi][ni][e]: row mi*32 + 8*(e/4) + 4*h + e%4, column n_wave + 32*ni + l32.
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = mi * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
      if (r >= rows) continue;
      const int64_t row = m0 + r;
      if constexpr (MODE == GM_SWIGLU) {
        if (!col_ok0) continue;
        const int f = (n_wave >> 1) + l32;
        const float gte = acc[mi][0][e], up = acc[mi][1][e];
        reinterpret_cast<__bf16*>(g.out)[row * g.ldo + f] = (__bf16)(silu(gte) * up);
      } else {
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          if (!(ni ? col_ok1 : col_ok0)) continue;
          const int64_t col = n_wave + 32 * ni + l32;
          const float v = acc[mi][ni][e];
          if constexpr (MODE == GM_F32) {
            reinterpret_cast<float*>(g.out)[row * g.ldo + col] = v;
          } else if constexpr (MODE == GM_F32_ADD) {
            float* p = reinterpret_cast<float*>(g.out) + row * g.ldo + col;
            *p = *p + v;
          } else {
            g.partial[((int64_t)split * g.M + row) * g.N + col] = v;
          }
        }
      }
    }
  }
}

// Sum split-K partials in split order and apply the epilogue.  One thread per 4 output
// columns (SwiGLU: 4 gate/up pairs).
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ partial,
                                                            int32_t splits, int32_t M, int32_t N,
                                                            int32_t mode, void* out, int32_t ldo) {
  const int64_t ncols = (mode == GM_SWIGLU) ? N / 2 : N;
  const int64_t quads = ncols / 4;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)M * quads) return;
  const int64_t row = i / quads;
  const int64_t c4 = (i % quads) * 4;
  const int64_t plane = (int64_t)M * N;
  if (mode == GM_SWIGLU) {
    const int64_t gc = (c4 / 32) * 64 + (c4 % 32);
    float4 gs = *reinterpret_cast<const float4*>(partial + row * N + gc);
    float4 us = *reinterpret_cast<const float4*>(partial + row * N + gc + 32);
    for (int s = 1; s < splits; ++s) {
      const float4 a = *reinterpret_cast<const float4*>(partial + s * plane + row * N + gc);
      const float4 b = *reinterpret_cast<const float4*>(partial + s * plane + row * N + gc + 32);
      gs.x += a.x; gs.y += a.y; gs.z += a.z; gs.w += a.w;
      us.x += b.x; us.y += b.y; us.z += b.z; us.w += b.w;
    }
    __bf16* o = reinterpret_cast<__bf16*>(out) + row * ldo + c4;
    o[0] = (__bf16)(silu(gs.x) * us.x);
    o[1] = (__bf16)(silu(gs.y) * us.y);
    o[2] = (__bf16)(silu(gs.z) * us.z);
    o[3] = (__bf16)(silu(gs.w) * us.w);
    return;
  }
  float4 acc = *reinterpret_cast<const float4*>(partial + row * N + c4);
  for (int s = 1; s < splits; ++s) {
    const float4 a = *reinterpret_cast<const float4*>(partial + s * plane + row * N + c4);
    acc.x += a.x; acc.y += a.y; acc.z += a.z; acc.w += a.w;
  }
  float4* o = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + row * ldo + c4);
  if (mode == GM_F32_ADD) {
    const float4 x = *o;
    acc.x = x.x + acc.x; acc.y = x.y + acc.y; acc.z = x.z + acc.z; acc.w = x.w + acc.w;
  }
  *o = acc;
}

template <int MI, bool GROUPED>
static hipError_t launch_mode(const GemmArgs& a, int grid_m_tiles, hipStream_t s) {
  const int ntiles = (int)ceil_div(a.N, NT);
  dim3 grid, block(256);
  if (GROUPED) {
    grid = dim3(grid_m_tiles, ntiles);
  } else {
    grid = dim3((unsigned)(ceil_div(a.M, MI * 32) * ntiles * a.splits));
  }
  const int mode = (a.splits > 1 && !GROUPED) ? GM_PARTIAL : a.mode;
  switch (mode) {
    case GM_F32: hipLaunchKernelGGL((gemm_q8_kernel<MI, GM_F32, GROUPED>), grid, block, 0, s, a); break;
    case GM_F32_ADD: hipLaunchKernelGGL((gemm_q8_kernel<MI, GM_F32_ADD, GROUPED>), grid, block, 0, s, a); break;
    case GM_SWIGLU: hipLaunchKernelGGL((gemm_q8_kernel<MI, GM_SWIGLU, GROUPED>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((gemm_q8_kernel<MI, GM_PARTIAL, GROUPED>), grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& a, int grid_m_tiles, int mt, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  const bool grouped = a.tiles != nullptr;
  hipError_t e;
  if (grouped) {
    if (mt == 128) e = launch_mode<4, true>(a, grid_m_tiles, s);
    else if (mt == 64) e = launch_mode<2, true>(a, grid_m_tiles, s);
    else e = launch_mode<8, true>(a, grid_m_tiles, s);
    return e;
  }
  if (mt == 64) e = launch_mode<2, false>(a, 0, s);
  else if (mt == 128) e = launch_mode<4, false>(a, 0, s);
  else e = launch_mode<8, false>(a, 0, s);
  if (e != hipSuccess || a.splits <= 1) return e;
  return launch_splitk_reduce(a.partial, a.splits, a.M, a.N, a.mode, a.out, a.ldo, s);
}

hipError_t launch_splitk_reduce(const float* partial, int32_t splits, int32_t M, int32_t N,
                                int32_t mode, void* out, int32_t ldo, hipStream_t s) {
  const int64_t ncols = (mode == GM_SWIGLU) ? N / 2 : N;
  const int64_t work = (int64_t)M * (ncols / 4);
  const unsigned blocks = (unsigned)ceil_div(work, 256);
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(blocks), dim3(256), 0, s, partial, splits, M, N,
                     mode, out, ldo);
  return hipGetLastError();
}

}  // namespace cp
