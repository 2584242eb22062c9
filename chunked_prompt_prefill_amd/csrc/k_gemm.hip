// q8_0-weight GEMM on fp16 MFMA (gfx950), fp32 accumulate.
//
//   out[m][n] = sum_k A[m][k] * W[n][k],  A fp16 activations, W q8_0 blocks of 32.
//
// This kernel takes row tiles of 64 and 128 (two workgroups per CU) and the grouped
// expert GEMMs; 256-row tiles run the deeper-pipelined kernel in k_gemm_big.hip.
//
// Tiling.  A workgroup of 4 waves owns an MT x 256 output tile (MT = 32*MI); each wave
// owns 64 columns (two 32-column MFMA blocks) across all MT rows, so every weight
// element is dequantised exactly once per workgroup.  Per 128-wide K stage (4 q8_0
// blocks):
//   * A: MT x 128 fp16 staged in LDS by asynchronous global->LDS loads (16 bytes per
//     lane, landing in lane order), double buffered; the 16-byte chunks of a row are
//     XOR-swizzled by the row so the 32 rows an MFMA operand spans hit distinct banks.
//     The swizzle is applied by choosing each lane's source address.
//   * W: loaded straight into registers one stage ahead from the repacked layout (1 KiB
//     contiguous per wave per 32-row group and block, already in MFMA lane order),
//     dequantised in registers as the B operand: each int8 becomes an exact fp16
//     integer by a byte permute and a packed add, and one packed fp16 multiply by the
//     block scale gives the correctly rounded fp16 of d*q.
// The K index inside a q8_0 block is permuted consistently on both operands so that a
// lane's 16 weight bytes are contiguous: lane half h, MFMA step s, element c <-> block
// column 16h + 8s + c.
// Rows beyond M and columns beyond N are computed from clamped (valid) addresses and
// simply not stored, so the main loop has no branches.
// Epilogues: fp32 store, fp32 residual add, SwiGLU (gate/up columns interleaved in
// 32-column groups) to fp16, or split-K partials summed by a separate kernel in split
// order (deterministic: no float atomics).  A launch may cover a column range [n0, N)
// so that the host can run the tiles that fill whole rounds of the chip without
// splitting and split only the tail.
// Grouped mode (routed experts): the row tile comes from a device tile table
// {expert, m0, m1}; A rows may be gathered through an index array.
#include "cp_internal.h"
#include "k_common.h"

namespace cp {

constexpr int KT = 128;
constexpr int NT = 256;
constexpr int CPR = KT * 2 / 16;   // 16-byte chunks per A row per stage

typedef __attribute__((address_space(1))) const void gvoid_t;
typedef __attribute__((address_space(3))) void lvoid_t;

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// Loads through global (address space 1) pointers: the pointers come from a struct
// argument, so without this the compiler would emit flat loads.
__device__ __forceinline__ uint4 gload(const uint4* p) {
  const u32x4_t v = *(const __attribute__((address_space(1))) u32x4_t*)(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 gload(const uint2* p) {
  const u32x2_t v = *(const __attribute__((address_space(1))) u32x2_t*)(p);
  return make_uint2(v.x, v.y);
}

__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)

template <int MI>
struct MinBlocks { static constexpr int v = MI >= 8 ? 1 : 2; };

template <int MI, int MODE, bool GROUPED>
__global__ __launch_bounds__(256, MinBlocks<MI>::v) void gemm_q8_kernel(GemmArgs g) {
  constexpr int MT = MI * 32;
  constexpr int NCH = MT * CPR;      // 16-byte chunks per stage
  constexpr int JPW = NCH / 256;     // async A loads per thread per stage
  __shared__ uint4 sA[2][NCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
    const int ntiles = (int)ceil_div(g.N - g.n0, NT);
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
  const int n_wave = g.n0 + ntile * NT + wave * 64;
  const bool col_ok0 = n_wave < g.N;
  const bool col_ok1 = n_wave + 32 < g.N;

  // A: async load j of wave w fills physical chunks [(4j + w)*64, +64) of a stage; lane L
  // lands on row r = 16j + 4w + L/16, physical chunk L%16, which holds logical chunk
  // (L%16) ^ (r%16) = (L%16) ^ (4w + L/16).
  const int rsub = 4 * wave + (lane >> 4);
  const int lchunk = (lane & 15) ^ rsub;
  int32_t aoff[JPW];
#pragma unroll
  for (int j = 0; j < JPW; ++j) {
    const int r = min(16 * j + rsub, rows - 1);
    int32_t pr = m0 + r;
    if (g.a_rows) pr = g.a_rows[m0 + r] / g.a_row_div;
    aoff[j] = pr * g.lda + lchunk * 8;
  }
  auto issue_a = [&](int ks, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < JPW; ++j)
      __builtin_amdgcn_global_load_lds((gvoid_t*)(g.A + aoff[j] + ks * KT),
                                       (lvoid_t*)&sA[buf][(4 * j + wave) * 64], 16, 0, 0);
  };

  const int KB = g.K / QK, KQ = g.K / KT;
  const int last32 = g.N / 32 - 1;
  const uint4* bq[2];
  const uint2* bd[2];
#pragma unroll
  for (int ni = 0; ni < 2; ++ni) {
    const int64_t n32 = min((n_wave >> 5) + ni, last32);
    bq[ni] = reinterpret_cast<const uint4*>(g.wq + expert * g.wq_estride) + n32 * KB * 64 + lane;
    bd[ni] = reinterpret_cast<const uint2*>(g.wd + expert * g.wd_estride) + n32 * KQ * 32 + l32;
  }
  auto load_b = [&](int ks, uint4 (&rb)[2][4], uint2 (&rs)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) rb[ni][kb] = gload(bq[ni] + (4 * ks + kb) * 64);
      rs[ni] = gload(bd[ni] + ks * 32);
    }
  };

  f32x16 acc[MI][2];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mi][ni][e] = 0.0f;

  auto compute = [&](int buf, const uint4 (&rb)[2][4], const uint2 (&rs)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      uint4 b[2][2];
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const uint32_t pair = (kb < 2) ? rs[ni].x : rs[ni].y;
        dequant16_f16(rb[ni][kb], (kb & 1) ? (pair >> 16) : (pair & 0xFFFFu), b[ni][0], b[ni][1]);
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
          const int c = kb * 4 + 2 * h + s;
          const uint4 a = sA[buf][(mi * 32 + l32) * CPR + (c ^ (l32 & 15))];
          const f16x8 av = __builtin_bit_cast(f16x8, a);
          acc[mi][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, __builtin_bit_cast(f16x8, b[0][s]),
                                                              acc[mi][0], 0, 0, 0);
          acc[mi][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, __builtin_bit_cast(f16x8, b[1][s]),
                                                              acc[mi][1], 0, 0, 0);
        }
      }
    }
  };

  if (ks0 < ks1) {
    uint4 rb0[2][4], rb1[2][4];
    uint2 rs0[2], rs1[2];
    issue_a(ks0, 0);
    load_b(ks0, rb0, rs0);
    int ks = ks0;
    for (; ks + 1 < ks1; ks += 2) {
      wait_vm0();
      __syncthreads();                 // stage ks in LDS (all waves); buffer 1 free
      issue_a(ks + 1, 1);
      load_b(ks + 1, rb1, rs1);
      compute(0, rb0, rs0);
      wait_vm0();
      __syncthreads();                 // stage ks+1 in LDS; buffer 0 free
      if (ks + 2 < ks1) {
        issue_a(ks + 2, 0);
        load_b(ks + 2, rb0, rs0);
      }
      compute(1, rb1, rs1);
    }
    if (ks < ks1) {                    // odd number of stages: the last one is in buffer 0
      wait_vm0();
      __syncthreads();
      compute(0, rb0, rs0);
    }
  }

  // Epilogue.  acc[mi][ni][e]: row mi*32 + 8*(e/4) + 4*h + e%4, column n_wave + 32*ni + l32.
  // A lane's rows are 4h plus constants, so each store address is a per-lane base plus a
  // constant times the (uniform) row stride; whole tiles skip the row check.
  const int pn = g.N - g.n0;
  const bool full = rows >= MT;
  auto each = [&](auto&& st) __attribute__((always_inline)) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int rc = mi * 32 + 8 * (e >> 2) + (e & 3);   // row minus 4h
        if (full || rc + 4 * h < rows) st(mi, e, rc);
      }
  };
  if constexpr (MODE == GM_SWIGLU) {
    if (col_ok0) {
      _Float16* ob = reinterpret_cast<_Float16*>(g.out) + ((int64_t)m0 + 4 * h) * g.ldo + (n_wave >> 1) + l32;
      each([&](int mi, int e, int rc) {
        ob[(int64_t)rc * g.ldo] = f16_sat(silu(acc[mi][0][e]) * acc[mi][1][e]);
      });
    }
  } else if constexpr (MODE == GM_PARTIAL) {
    float* pb = g.partial + ((int64_t)split * g.M + m0 + 4 * h) * pn + (n_wave - g.n0) + l32;
    each([&](int mi, int e, int rc) {
      if (col_ok0) pb[(int64_t)rc * pn] = acc[mi][0][e];
      if (col_ok1) pb[(int64_t)rc * pn + 32] = acc[mi][1][e];
    });
  } else {
    float* ob = reinterpret_cast<float*>(g.out) + ((int64_t)m0 + 4 * h) * g.ldo + n_wave + l32;
    each([&](int mi, int e, int rc) {
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        if (!(ni ? col_ok1 : col_ok0)) continue;
        float* p = ob + (int64_t)rc * g.ldo + 32 * ni;
        if constexpr (MODE == GM_F32) *p = acc[mi][ni][e];
        else *p = *p + acc[mi][ni][e];
      }
    });
  }
}

// Sum split-K partials of columns [n0, N) in split order and apply the epilogue.  One
// thread per 4 output columns (SwiGLU: 4 gate/up pairs).
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ partial,
                                                            int32_t splits, int32_t M, int32_t n0,
                                                            int32_t N, int32_t mode, void* out,
                                                            int32_t ldo) {
  const int64_t pn = N - n0;
  const int64_t ncols = (mode == GM_SWIGLU) ? pn / 2 : pn;
  const int64_t quads = ncols / 4;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)M * quads) return;
  const int64_t row = i / quads;
  const int64_t c4 = (i % quads) * 4;
  const int64_t plane = (int64_t)M * pn;
  if (mode == GM_SWIGLU) {
    const int64_t gc = (c4 / 32) * 64 + (c4 % 32);
    const float4 gs = split_sum4(partial + row * pn + gc, plane, splits);
    const float4 us = split_sum4(partial + row * pn + gc + 32, plane, splits);
    _Float16* o = reinterpret_cast<_Float16*>(out) + row * ldo + n0 / 2 + c4;
    o[0] = f16_sat(silu(gs.x) * us.x);
    o[1] = f16_sat(silu(gs.y) * us.y);
    o[2] = f16_sat(silu(gs.z) * us.z);
    o[3] = f16_sat(silu(gs.w) * us.w);
    return;
  }
  float4 acc = split_sum4(partial + row * pn + c4, plane, splits);
  float4* o = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + row * ldo + n0 + c4);
  if (mode == GM_F32_ADD) {
    const float4 x = *o;
    acc.x = x.x + acc.x; acc.y = x.y + acc.y; acc.z = x.z + acc.z; acc.w = x.w + acc.w;
  }
  *o = acc;
}

template <int MI, bool GROUPED>
static hipError_t launch_mode(const GemmArgs& a, int grid_m_tiles, hipStream_t s) {
  const int ntiles = (int)ceil_div(a.N - a.n0, NT);
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

hipError_t launch_gemm(const GemmArgs& a, int grid_m_tiles, int mt, hipStream_t s, bool reduce) {
  if (a.M <= 0 || a.N <= a.n0) return hipSuccess;
  const bool grouped = a.tiles != nullptr;
  hipError_t e;
  if (grouped) {
    if (mt == 256) return launch_gemm_big(a, grid_m_tiles, s);
    return mt == 64 ? launch_mode<2, true>(a, grid_m_tiles, s) : launch_mode<4, true>(a, grid_m_tiles, s);
  }
  if (mt == 1) e = launch_gemm_skinny(a, s);
  else if (mt == 64) e = launch_mode<2, false>(a, 0, s);
  else if (mt == 128) e = launch_mode<4, false>(a, 0, s);
  else e = launch_gemm_big(a, 0, s);
  if (e != hipSuccess || a.splits <= 1 || !reduce) return e;
  return launch_splitk_reduce(a.partial, a.splits, a.M, a.n0, a.N, a.mode, a.out, a.ldo, s);
}

hipError_t launch_splitk_reduce(const float* partial, int32_t splits, int32_t M, int32_t n0,
                                int32_t N, int32_t mode, void* out, int32_t ldo, hipStream_t s) {
  const int64_t pn = N - n0;
  const int64_t ncols = (mode == GM_SWIGLU) ? pn / 2 : pn;
  const int64_t work = (int64_t)M * (ncols / 4);
  const unsigned blocks = (unsigned)ceil_div(work, 256);
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(blocks), dim3(256), 0, s, partial, splits, M, n0, N,
                     mode, out, ldo);
  return hipGetLastError();
}

}  // namespace cp
