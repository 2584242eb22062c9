// Non-GEMM kernels of the prefill path (gfx950): weight repack, q8_0 encode, RMSNorm,
// RoPE + K/V cache append, state pack/unpack, and the routed-expert router / permute /
// unpermute.  Every kernel that decides stored bytes or integers (q8_0 codes, cache rows,
// expert indices) uses one float32 rounding per operation (explicit _rn intrinsics; the
// library is also built without floating-point contraction).
#include <mutex>

#include "cp_internal.h"
#include "k_common.h"

namespace cp {

// ======================================================================================
// Weight repack: interchange q8_0 rows -> QMat (lane-ordered quants, paired fp16 scales)
// ======================================================================================
__global__ void repack_kernel(const uint8_t* __restrict__ src0, const uint8_t* __restrict__ src1,
                              int64_t src_rows, int32_t nb_src, int64_t dst_row0, int64_t dst_rows,
                              int32_t mode, int8_t* __restrict__ dq, uint16_t* __restrict__ dd,
                              int32_t K) {
  const int KB = K / QK, KQ = K / 128;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= dst_rows * KB) return;
  const int64_t nl = i / KB;
  const int kb = (int)(i % KB);
  int64_t n, sr;
  const uint8_t* src;
  if (mode == 0) {
    n = dst_row0 + nl;
    sr = nl;
    src = src0;
  } else {
    n = nl;
    const int64_t grp = n / 64, w = (n % 64) / 32, ii = n % 32;
    sr = grp * 32 + ii;
    src = w ? src1 : src0;
  }
  uint32_t wds[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  uint16_t dbits = 0;
  if (sr < src_rows && kb < nb_src) {
    const uint8_t* p = src + (sr * nb_src + kb) * 34;
    dbits = (uint16_t)(p[0] | (p[1] << 8));
#pragma unroll
    for (int j = 0; j < 8; ++j)
      wds[j] = (uint32_t)p[2 + 4 * j] | ((uint32_t)p[3 + 4 * j] << 8) |
               ((uint32_t)p[4 + 4 * j] << 16) | ((uint32_t)p[5 + 4 * j] << 24);
  }
  const int64_t n32 = n / 32, r = n % 32;
  uint4* q = reinterpret_cast<uint4*>(dq);
  q[(n32 * KB + kb) * 64 + r] = make_uint4(wds[0], wds[1], wds[2], wds[3]);
  q[(n32 * KB + kb) * 64 + 32 + r] = make_uint4(wds[4], wds[5], wds[6], wds[7]);
  dd[((n32 * KQ + kb / 4) * 32 + r) * 4 + (kb & 3)] = dbits;
}

hipError_t launch_repack_q8_0(const void* src0, const void* src1, int64_t src_rows, int32_t k_src,
                              int64_t dst_row0, int64_t dst_rows, int32_t mode, QMat dst,
                              hipStream_t s) {
  const int32_t nb_src = (k_src + QK - 1) / QK;
  const int64_t work = dst_rows * (dst.K / QK);
  if (work == 0) return hipSuccess;
  hipLaunchKernelGGL(repack_kernel, dim3((unsigned)ceil_div(work, 256)), dim3(256), 0, s,
                     (const uint8_t*)src0, (const uint8_t*)src1, src_rows, nb_src, dst_row0,
                     dst_rows, mode, dst.q, reinterpret_cast<uint16_t*>(dst.d), dst.K);
  return hipGetLastError();
}

// ======================================================================================
// q8_0 encode of float32 rows (interchange layout).  32 lanes per block; the block amax
// is a wavefront reduction; d = amax/127 and 1/d correctly rounded; q rounds half away.
// ======================================================================================
__device__ __forceinline__ void q8_encode_lane(float x, float& d, int& q) {
  const float amax = warp_max32(fabsf(x));
  d = __fdiv_rn(amax, 127.0f);
  const float id = d != 0.0f ? __fdiv_rn(1.0f, d) : 0.0f;
  int v = (int)roundf(__fmul_rn(x, id));
  q = v > 127 ? 127 : (v < -127 ? -127 : v);
}

__global__ void quantize_kernel(const float* __restrict__ x, int64_t rows, int32_t k, int64_t ldx,
                                uint8_t* __restrict__ out) {
  const int nb = (k + QK - 1) / QK;
  const int64_t bi = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
  if (bi >= rows * nb) return;
  const int64_t row = bi / nb;
  const int blk = (int)(bi % nb);
  const int l = threadIdx.x & 31;
  const int col = blk * QK + l;
  const float v = col < k ? x[row * ldx + col] : 0.0f;
  float d;
  int q;
  q8_encode_lane(v, d, q);
  uint8_t* o = out + (row * nb + blk) * 34;
  if (l == 0) {
    const uint16_t b = float_to_half_bits(d);
    o[0] = (uint8_t)(b & 0xFF);
    o[1] = (uint8_t)(b >> 8);
  }
  o[2 + l] = (uint8_t)(int8_t)q;
}

hipError_t launch_quantize_q8_0(const float* x, int64_t rows, int32_t k, int64_t ldx, void* out,
                                hipStream_t s) {
  const int64_t nb = (k + QK - 1) / QK;
  const int64_t blocks = ceil_div(rows * nb, 8);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, rows, k, ldx,
                     (uint8_t*)out);
  return hipGetLastError();
}

// ======================================================================================
// RMSNorm: y = x / sqrt(mean(x^2) + eps) * gamma  -> fp16 (and optionally float32)
// ======================================================================================
// Four consecutive elements (col % 4 == 0; n0 % 4 == 0) of row `row` of a matrix [rows][ld]
// whose split-K sums may still be pending (PendingSum).
__device__ __forceinline__ float4 pend_load4(const float* base, int64_t ld, const PendingSum& ps,
                                             int64_t row, int col) {
  const float4 b = *reinterpret_cast<const float4*>(base + row * ld + col);
  if (!ps.partial || col < ps.n0) return b;
  const int64_t pn = ps.N - ps.n0, plane = (int64_t)ps.M * pn;
  float4 acc = split_sum4(ps.partial + row * pn + (col - ps.n0), plane, ps.splits);
  if (ps.add) { acc.x = b.x + acc.x; acc.y = b.y + acc.y; acc.z = b.z + acc.z; acc.w = b.w + acc.w; }
  return acc;
}
// One row per workgroup of nthr threads (a multiple of 64, at most 1024; about two float4
// columns per thread, so that a row's loads are spread over many waves).  Pass 1 takes the
// pending sums into x (written back) and forms the sum of squares; pass 2 re-reads the row
// (this thread's own writes) and scales it.
__global__ __launch_bounds__(1024) void rmsnorm_kernel(float* x, const float* __restrict__ gamma,
                                                       int32_t d, float eps, _Float16* __restrict__ y,
                                                       float* __restrict__ y32, PendingSum ps) {
  __shared__ float red[16];
  const int nthr = blockDim.x;
  const int64_t row = blockIdx.x;
  float* xr = x + row * d;
  const bool pend = ps.partial != nullptr;
  float ss = 0.0f;
  for (int i = threadIdx.x * 4; i < d; i += 4 * nthr) {
    const float4 v = pend ? pend_load4(x, d, ps, row, i) : *reinterpret_cast<const float4*>(xr + i);
    if (pend && i >= ps.n0) *reinterpret_cast<float4*>(xr + i) = v;
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  ss = red[0];
  for (int w = 1; w < nthr / 64; ++w) ss += red[w];
  const float scale = 1.0f / sqrtf(ss / (float)d + eps);
  for (int i = threadIdx.x * 4; i < d; i += 4 * nthr) {
    const float4 v = *reinterpret_cast<const float4*>(xr + i);
    const float4 gm = *reinterpret_cast<const float4*>(gamma + i);
    const float a = v.x * scale * gm.x, b = v.y * scale * gm.y;
    const float c = v.z * scale * gm.z, e = v.w * scale * gm.w;
    uint2 pk = make_uint2(pack_f16x2(a, b), pack_f16x2(c, e));
    *reinterpret_cast<uint2*>(y + row * d + i) = pk;
    if (y32) *reinterpret_cast<float4*>(y32 + row * d + i) = make_float4(a, b, c, e);
  }
}

hipError_t launch_rmsnorm(float* x, const float* gamma, int32_t n, int32_t d, float eps,
                          _Float16* y, float* y32, hipStream_t s, const PendingSum& ps) {
  if (n <= 0) return hipSuccess;
  if (d <= 0 || d % 4) return hipErrorInvalidValue;
  const int nthr = (int)std::min<int64_t>(1024, std::max<int64_t>(64, ceil_div(ceil_div(d, 8), 64) * 64));
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(n), dim3(nthr), 0, s, x, gamma, d, eps, y, y32, ps);
  return hipGetLastError();
}

// ======================================================================================
// KV cache layout of one layer (capacity n_ctx, a multiple of 64):
//   f16 : K [Hkv][n_ctx][hd] f16, V transposed [Hkv][hd][n_ctx] f16
//   q8_0: K int8 [Hkv][n_ctx][hd] + fp16 scales [Hkv][n_ctx][hd/32];
//         V int8 [Hkv][hd][n_ctx] + fp16 scales [Hkv][hd/32][n_ctx]
// ======================================================================================
size_t kv_layer_bytes(int32_t Hkv, int32_t hd, int32_t n_ctx, int32_t kv_type) {
  const size_t elems = (size_t)Hkv * hd * n_ctx;
  if (kv_type == CP_KV_F16) return 2 * align_up(elems * 2);
  return 2 * align_up(elems) + 2 * align_up(elems / QK * 2);
}

KvLayer kv_layer_at(void* base, int32_t Hkv, int32_t hd, int32_t n_ctx, int32_t kv_type) {
  KvLayer L;
  uint8_t* p = (uint8_t*)base;
  const size_t elems = (size_t)Hkv * hd * n_ctx;
  if (kv_type == CP_KV_F16) {
    L.k = p;
    L.v = p + align_up(elems * 2);
  } else {
    L.k = p;
    L.v = p + align_up(elems);
    L.kd = (uint16_t*)(p + 2 * align_up(elems));
    L.vd = (uint16_t*)(p + 2 * align_up(elems) + align_up(elems / QK * 2));
  }
  return L;
}

// Where RoPE and the K/V append read the QKV projection: its output rows, or, for a split
// GEMM of a few rows whose partial planes were left unsummed, those planes added in split
// order exactly as the split-K reduction adds them (p0 + p1 + ... in float32).
__device__ __forceinline__ float4 qkv_load4(const QkvSrc& src, int64_t off) {
  if (src.splits == 0) return *reinterpret_cast<const float4*>(src.qkv + off);
  return split_sum4(src.partial + off, src.plane, src.splits);
}
__device__ __forceinline__ float qkv_load1(const QkvSrc& src, int64_t off) {
  if (src.splits == 0) return src.qkv[off];
  return split_sum1(src.partial + off, src.plane, src.splits);
}

// RoPE on q and k (rotate-half pairs (i, i+hd/2)), then q -> f16 output and k -> cache.
// Each lane handles 4 consecutive values of one head (16-byte loads); a wave covers 256
// values of one token.  For a q8_0 cache the 32 values of a block sit in 8 lanes and
// their amax is a reduction over those lanes.  (block: this workgroup's index in the
// RoPE part of the grid.)
__device__ __forceinline__ void rope_qk_body(int64_t block, const QkvSrc& src,
                                             const float* __restrict__ cos_t,
                                             const float* __restrict__ sin_t, int32_t n,
                                             int32_t start, int32_t Hq, int32_t Hkv, int32_t hd,
                                             int32_t kv_type, int32_t n_ctx,
                                             _Float16* __restrict__ q_out, const KvLayer& kv) {
  const int lane = threadIdx.x & 63;
  const int E = (Hq + Hkv) * hd;                      // rotated values per token
  const int segs = (E + 255) / 256;
  const int64_t seg = block * 4 + (threadIdx.x >> 6);
  const int64_t t = seg / segs;
  if (t >= n) return;
  const int e0 = (int)(seg % segs) * 256 + lane * 4;
  if (e0 >= E) return;                                // whole 8-lane groups drop out together
  const int64_t p = start + t;
  const int half = hd / 2;
  const int64_t Nqkv = (int64_t)(Hq + 2 * Hkv) * hd;
  const int head = e0 / hd, i0 = e0 % hd;
  const bool lo = i0 < half;
  const int ic0 = lo ? i0 : i0 - half;
  const float4 x = qkv_load4(src, t * Nqkv + e0);
  const float4 y = qkv_load4(src, t * Nqkv + head * hd + (lo ? i0 + half : i0 - half));
  const float4 c = *reinterpret_cast<const float4*>(cos_t + p * half + ic0);
  const float4 s = *reinterpret_cast<const float4*>(sin_t + p * half + ic0);
  const float xs[4] = {x.x, x.y, x.z, x.w}, ys[4] = {y.x, y.y, y.z, y.w};
  const float cs[4] = {c.x, c.y, c.z, c.w}, ss[4] = {s.x, s.y, s.z, s.w};
  float out[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
    out[k] = lo ? __fsub_rn(__fmul_rn(xs[k], cs[k]), __fmul_rn(ys[k], ss[k]))
                : __fadd_rn(__fmul_rn(xs[k], cs[k]), __fmul_rn(ys[k], ss[k]));
  if (head < Hq) {
    *reinterpret_cast<uint2*>(q_out + (t * Hq + head) * hd + i0) =
        make_uint2(pack_f16x2(out[0], out[1]), pack_f16x2(out[2], out[3]));
    return;
  }
  const int64_t gi = (int64_t)(head - Hq) * n_ctx + p;
  if (kv_type == CP_KV_F16) {
    *reinterpret_cast<uint2*>(reinterpret_cast<_Float16*>(kv.k) + gi * hd + i0) =
        make_uint2(pack_f16x2(out[0], out[1]), pack_f16x2(out[2], out[3]));
    return;
  }
  float amax = fmaxf(fmaxf(fabsf(out[0]), fabsf(out[1])), fmaxf(fabsf(out[2]), fabsf(out[3])));
#pragma unroll
  for (int o = 4; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  const float d = __fdiv_rn(amax, 127.0f);
  const float id = d != 0.0f ? __fdiv_rn(1.0f, d) : 0.0f;
  uint32_t packed = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    int v = (int)roundf(__fmul_rn(out[k], id));
    v = v > 127 ? 127 : (v < -127 ? -127 : v);
    packed |= (uint32_t)(uint8_t)(int8_t)v << (8 * k);
  }
  *reinterpret_cast<uint32_t*>(reinterpret_cast<int8_t*>(kv.k) + gi * hd + i0) = packed;
  if ((i0 & 31) == 0) kv.kd[gi * (hd / QK) + i0 / QK] = float_to_half_bits(d);
}

__global__ __launch_bounds__(256) void rope_qk_kernel(QkvSrc src, const float* __restrict__ cos_t,
                                                      const float* __restrict__ sin_t, int32_t n,
                                                      int32_t start, int32_t Hq, int32_t Hkv,
                                                      int32_t hd, int32_t kv_type, int32_t n_ctx,
                                                      _Float16* __restrict__ q_out, KvLayer kv) {
  rope_qk_body(blockIdx.x, src, cos_t, sin_t, n, start, Hq, Hkv, hd, kv_type, n_ctx, q_out, kv);
}

int64_t rope_qk_blocks(int32_t n, int32_t n_head, int32_t n_kv_head, int32_t head_dim) {
  return ceil_div(ceil_div((int64_t)(n_head + n_kv_head) * head_dim, 256) * n, 4);
}

hipError_t launch_rope_qk(const float* qkv, const float* cos_t, const float* sin_t, int32_t n,
                          int32_t start, int32_t n_head, int32_t n_kv_head, int32_t head_dim,
                          int32_t kv_type, int32_t n_ctx, _Float16* q_out, KvLayer kv,
                          hipStream_t s) {
  if (n <= 0) return hipSuccess;
  QkvSrc src;
  src.qkv = qkv;
  hipLaunchKernelGGL(rope_qk_kernel, dim3((unsigned)rope_qk_blocks(n, n_head, n_kv_head, head_dim)),
                     dim3(256), 0, s, src, cos_t, sin_t, n, start, n_head, n_kv_head, head_dim,
                     kv_type, n_ctx, q_out, kv);
  return hipGetLastError();
}

// V rows -> transposed cache.  A workgroup takes 32 tokens x 64 dims of one kv head: each
// wave converts 64 consecutive dims of a token row (q8_0: per-32 amax by wavefront
// reduction), the codes are transposed through LDS, then written 32 positions per dim.
// (bx: token tile, by: kv head x 64-dim slice.)
constexpr int VT = 32;
__device__ __forceinline__ void v_append_body(int bx, int by, const QkvSrc& src, int32_t n,
                                              int32_t start, int32_t Hq, int32_t Hkv, int32_t hd,
                                              int32_t kv_type, int32_t n_ctx, const KvLayer& kv) {
  __shared__ uint16_t sv[64][VT + 2];
  __shared__ int8_t sq[64][VT + 4];
  __shared__ uint16_t sd[2][VT];
  const int t0 = bx * VT;
  const int g = by / (hd / 64);
  const int d0 = (by % (hd / 64)) * 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t Nqkv = (int64_t)(Hq + 2 * Hkv) * hd;
  const int64_t vcol = (int64_t)(Hq + Hkv + g) * hd + d0;
  for (int tl = wave; tl < VT; tl += 4) {
    const int t = t0 + tl;
    const float v = t < n ? qkv_load1(src, (int64_t)t * Nqkv + vcol + lane) : 0.0f;
    if (kv_type == CP_KV_F16) {
      sv[lane][tl] = float_to_half_bits(v);
    } else {
      float d;
      int q;
      q8_encode_lane(v, d, q);
      sq[lane][tl] = (int8_t)q;
      if ((lane & 31) == 0) sd[lane / QK][tl] = float_to_half_bits(d);
    }
  }
  __syncthreads();
  const int nt = min(VT, n - t0);
  for (int e = threadIdx.x; e < 64 * VT; e += 256) {
    const int i = e / VT, tl = e % VT;
    if (tl >= nt) continue;
    const int64_t dst = ((int64_t)g * hd + d0 + i) * n_ctx + start + t0 + tl;
    if (kv_type == CP_KV_F16) reinterpret_cast<uint16_t*>(kv.v)[dst] = sv[i][tl];
    else reinterpret_cast<int8_t*>(kv.v)[dst] = sq[i][tl];
  }
  if (kv_type != CP_KV_F16 && threadIdx.x < 2 * VT) {
    const int b = threadIdx.x / VT, tl = threadIdx.x % VT;
    if (tl < nt) kv.vd[((int64_t)g * (hd / QK) + d0 / QK + b) * n_ctx + start + t0 + tl] = sd[b][tl];
  }
}

__global__ __launch_bounds__(256) void v_append_kernel(QkvSrc src, int32_t n, int32_t start,
                                                       int32_t Hq, int32_t Hkv, int32_t hd,
                                                       int32_t kv_type, int32_t n_ctx, KvLayer kv) {
  v_append_body(blockIdx.x, blockIdx.y, src, n, start, Hq, Hkv, hd, kv_type, n_ctx, kv);
}

hipError_t launch_v_append(const float* qkv, int32_t n, int32_t start, int32_t n_head,
                           int32_t n_kv_head, int32_t head_dim, int32_t kv_type, int32_t n_ctx,
                           KvLayer kv, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  QkvSrc src;
  src.qkv = qkv;
  hipLaunchKernelGGL(v_append_kernel, dim3((unsigned)ceil_div(n, VT), n_kv_head * (head_dim / 64)),
                     dim3(256), 0, s, src, n, start, n_head, n_kv_head, head_dim, kv_type, n_ctx, kv);
  return hipGetLastError();
}

// Both in one launch, for chunks of a few tokens: the first workgroups run RoPE and the K
// append, the rest the V append, straight from the QKV output or its split planes (one
// launch instead of the split-K reduction, RoPE and the V append).
__global__ __launch_bounds__(256) void qkv_post_kernel(QkvSrc src, const float* __restrict__ cos_t,
                                                       const float* __restrict__ sin_t, int32_t n,
                                                       int32_t start, int32_t Hq, int32_t Hkv,
                                                       int32_t hd, int32_t kv_type, int32_t n_ctx,
                                                       _Float16* __restrict__ q_out, KvLayer kv,
                                                       int32_t rope_blocks) {
  const int b = blockIdx.x;
  if (b < rope_blocks) {
    rope_qk_body(b, src, cos_t, sin_t, n, start, Hq, Hkv, hd, kv_type, n_ctx, q_out, kv);
    return;
  }
  const int vb = b - rope_blocks, nby = Hkv * (hd / 64);
  v_append_body(vb / nby, vb % nby, src, n, start, Hq, Hkv, hd, kv_type, n_ctx, kv);
}

hipError_t launch_qkv_post(const float* qkv, const PendingSum& ps, const float* cos_t,
                           const float* sin_t, int32_t n, int32_t start, int32_t n_head,
                           int32_t n_kv_head, int32_t head_dim, int32_t kv_type, int32_t n_ctx,
                           _Float16* q_out, KvLayer kv, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t Nqkv = (int64_t)(n_head + 2 * n_kv_head) * head_dim;
  QkvSrc src;
  src.qkv = qkv;
  if (ps.partial) {
    // the planes must be the whole QKV output of these rows, unsummed
    if (ps.M != n || ps.n0 != 0 || ps.N != Nqkv || ps.add || ps.splits < 1) return hipErrorInvalidValue;
    src.partial = ps.partial;
    src.splits = ps.splits;
    src.plane = (int64_t)n * Nqkv;
  }
  const int64_t rb = rope_qk_blocks(n, n_head, n_kv_head, head_dim);
  const int64_t vb = ceil_div(n, VT) * n_kv_head * (head_dim / 64);
  hipLaunchKernelGGL(qkv_post_kernel, dim3((unsigned)(rb + vb)), dim3(256), 0, s, src, cos_t, sin_t,
                     n, start, n_head, n_kv_head, head_dim, kv_type, n_ctx, q_out, kv, (int32_t)rb);
  return hipGetLastError();
}

// ======================================================================================
// State pack / unpack: device cache <-> serialized rows (token-major (t, h); f16 rows of
// hd binary16, or q8_0 rows of hd/32 blocks {fp16 d, int8 q[32]}).  which: 0 = K, 1 = V.
// ======================================================================================
__device__ __forceinline__ int64_t kv_units(int32_t nt, int32_t Hkv, int32_t hd, int32_t kv_type) {
  return kv_type == CP_KV_F16 ? (int64_t)nt * Hkv * hd : (int64_t)nt * Hkv * (hd / QK) * 34;
}

template <bool PACK>
__global__ void kv_pack_kernel(KvLayer kv, int32_t t0, int32_t nt, int32_t Hkv, int32_t hd,
                               int32_t kv_type, int32_t n_ctx, int which, uint8_t* io) {
  const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= kv_units(nt, Hkv, hd, kv_type)) return;
  if (kv_type == CP_KV_F16) {
    const int64_t tl = u / ((int64_t)Hkv * hd);
    const int h = (int)((u / hd) % Hkv), i = (int)(u % hd);
    const int64_t t = t0 + tl;
    uint16_t* base = reinterpret_cast<uint16_t*>(which ? kv.v : kv.k);
    const int64_t off = which ? ((int64_t)h * hd + i) * n_ctx + t : ((int64_t)h * n_ctx + t) * hd + i;
    uint16_t* o = reinterpret_cast<uint16_t*>(io) + u;
    if (PACK) *o = base[off];
    else base[off] = *o;
    return;
  }
  const int nb = hd / QK;
  const int bb = (int)(u % 34);
  const int b = (int)((u / 34) % nb);
  const int h = (int)((u / (34 * nb)) % Hkv);
  const int64_t t = t0 + u / ((int64_t)34 * nb * Hkv);
  uint8_t* p;
  if (bb < 2) {
    const int64_t si = which ? ((int64_t)h * nb + b) * n_ctx + t : ((int64_t)h * n_ctx + t) * nb + b;
    p = reinterpret_cast<uint8_t*>(which ? kv.vd : kv.kd) + si * 2 + bb;
  } else {
    const int j = b * QK + bb - 2;
    const int64_t qi = which ? ((int64_t)h * hd + j) * n_ctx + t : ((int64_t)h * n_ctx + t) * hd + j;
    p = reinterpret_cast<uint8_t*>(which ? kv.v : kv.k) + qi;
  }
  if (PACK) io[u] = *p;
  else *p = io[u];
}

hipError_t launch_kv_pack(const KvLayer kv, int32_t t0, int32_t nt, int32_t Hkv, int32_t hd,
                          int32_t kv_type, int32_t n_ctx, int which, uint8_t* out, hipStream_t s) {
  const int64_t units = (kv_type == CP_KV_F16) ? (int64_t)nt * Hkv * hd : (int64_t)nt * Hkv * (hd / QK) * 34;
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL(kv_pack_kernel<true>, dim3((unsigned)ceil_div(units, 256)), dim3(256), 0, s,
                     kv, t0, nt, Hkv, hd, kv_type, n_ctx, which, out);
  return hipGetLastError();
}

hipError_t launch_kv_unpack(KvLayer kv, int32_t t0, int32_t nt, int32_t Hkv, int32_t hd,
                            int32_t kv_type, int32_t n_ctx, int which, const uint8_t* in,
                            hipStream_t s) {
  const int64_t units = (kv_type == CP_KV_F16) ? (int64_t)nt * Hkv * hd : (int64_t)nt * Hkv * (hd / QK) * 34;
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL(kv_pack_kernel<false>, dim3((unsigned)ceil_div(units, 256)), dim3(256), 0, s,
                     kv, t0, nt, Hkv, hd, kv_type, n_ctx, which, const_cast<uint8_t*>(in));
  return hipGetLastError();
}

// ======================================================================================
// Routed experts
// ======================================================================================
__global__ void unpack_router_kernel(const uint8_t* __restrict__ src, int32_t E, int32_t d,
                                     int8_t* __restrict__ q, uint16_t* __restrict__ dd) {
  const int nb = d / QK;
  const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= (int64_t)E * nb * 34) return;
  const int64_t blk = u / 34;
  const int bb = (int)(u % 34);
  const uint8_t* p = src + blk * 34;
  if (bb == 0) dd[blk] = (uint16_t)(p[0] | (p[1] << 8));
  else if (bb >= 2) q[blk * QK + bb - 2] = (int8_t)p[bb];
}

hipError_t launch_unpack_router(const void* src, int32_t E, int32_t d, int8_t* q, uint16_t* dd,
                                hipStream_t s) {
  const int64_t units = (int64_t)E * (d / QK) * 34;
  hipLaunchKernelGGL(unpack_router_kernel, dim3((unsigned)ceil_div(units, 256)), dim3(256), 0, s,
                     (const uint8_t*)src, E, d, q, dd);
  return hipGetLastError();
}

// Top-k of one token's E logits (descending logit, ties to the lower expert index) and
// the softmax over the k selected ones, by one wave: lane l holds experts l, l+64, l+128
// and l+192.  lg may point to LDS or to global memory.
__device__ void route_topk(const float* lg, int32_t E, int32_t k, int lane, int32_t* idx_row,
                           float* w_row) {
  float v[4];
  bool used[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    v[j] = e < E ? lg[e] : -INFINITY;
    used[j] = e >= E;
  }
  float selv[16];
  int sele[16];
  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      if (!used[j] && (v[j] > bv || (v[j] == bv && e < be))) { bv = v[j]; be = e; }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oe = __shfl_xor(be, o, 64);
      if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (lane + 64 * j == be) used[j] = true;
    selv[r] = bv;
    sele[r] = be;
  }
  if (lane == 0) {
    float z = 0.0f;
    float ex[16];
    for (int r = 0; r < k; ++r) { ex[r] = expf(selv[r] - selv[0]); z += ex[r]; }
    for (int r = 0; r < k; ++r) {
      idx_row[r] = sele[r];
      w_row[r] = ex[r] / z;
    }
  }
}

// One router block product in the fixed float32 order: P = sum_j q_j * y_j, products
// rounded, then added in ascending j.
__device__ __forceinline__ float router_block_dot(const float* qf, const float4* ys) {
  float4 yv = ys[0];
  float P = __fmul_rn(qf[0], yv.x);
  P = __fadd_rn(P, __fmul_rn(qf[1], yv.y));
  P = __fadd_rn(P, __fmul_rn(qf[2], yv.z));
  P = __fadd_rn(P, __fmul_rn(qf[3], yv.w));
#pragma unroll
  for (int j4 = 1; j4 < QK / 4; ++j4) {
    yv = ys[j4];
    P = __fadd_rn(P, __fmul_rn(qf[4 * j4 + 0], yv.x));
    P = __fadd_rn(P, __fmul_rn(qf[4 * j4 + 1], yv.y));
    P = __fadd_rn(P, __fmul_rn(qf[4 * j4 + 2], yv.z));
    P = __fadd_rn(P, __fmul_rn(qf[4 * j4 + 3], yv.w));
  }
  return P;
}

__device__ __forceinline__ void router_raw_weights(uint4 qa, uint4 qb, float* qf) {
  const uint32_t w[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
#pragma unroll
  for (int j = 0; j < QK; ++j) qf[j] = (float)(int8_t)((w[j >> 2] >> (8 * (j & 3))) & 0xFF);
}

__device__ __forceinline__ void router_block_weights(const int8_t* rq_blk, float* qf) {
  const uint4* qp = reinterpret_cast<const uint4*>(rq_blk);
  router_raw_weights(qp[0], qp[1], qf);
}

// Router logits in the fixed float32 order (per block: products and sums ascending,
// then acc += d_b * P_b over blocks ascending), then top-k and softmax (route_topk).
// Threads are (expert, token group): with E <= 128 two groups of 128 threads each take 4
// of the workgroup's 8 tokens, otherwise one group of 256 takes 4 (small workgroups: many
// of them in flight, since each thread's sums are serial chains).  Each thread converts a
// block's 32 weights to float once and applies them to its 4 tokens; y is staged 256
// columns at a time and read from LDS as a broadcast.  With few waves per SIMD nothing
// hides a load's latency but the kernel's own prefetch: a thread's next q8_0 block is
// loaded while the current one is applied, and the y columns of step s+1 are loaded into
// registers during step s - 1 and stored into the other LDS buffer at the end of step s.
constexpr int RT = 8;        // tokens per workgroup, at most
constexpr int RTT = 4;       // tokens per thread
__global__ __launch_bounds__(256) void router_kernel(const float* __restrict__ y,
                                                     const int8_t* __restrict__ rq,
                                                     const uint16_t* __restrict__ rd, int32_t n,
                                                     int32_t d, int32_t E, int32_t k,
                                                     float* __restrict__ logits,
                                                     int32_t* __restrict__ idx,
                                                     float* __restrict__ wout) {
  __shared__ float4 sy4[2][RT][64];
  __shared__ float slog[RT][256];
  const int tid = threadIdx.x;
  const int groups = E <= 128 ? 2 : 1;
  const int EP = 256 / groups;
  const int e = tid % EP, grp = tid / EP;
  const int RTW = RTT * groups;
  const int t0 = blockIdx.x * RTW;
  const int nb = d / QK;
  const int nsteps = (d + 255) / 256;
  const bool has_e = e < E;
  const uint4* wrow = reinterpret_cast<const uint4*>(rq + (int64_t)(has_e ? e : 0) * d);
  const uint16_t* drow = rd + (int64_t)(has_e ? e : 0) * nb;

  // y of one 256-column step: RTW x 64 float4, at most two per thread
  float4 yv[2];
  auto load_y = [&](int c0) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int u = tid + 256 * r;
      const int tt = u / 64, j4 = u % 64;
      const int t = t0 + tt, col = c0 + 4 * j4;
      yv[r] = (u < RTW * 64 && t < n && col < d)
                  ? *reinterpret_cast<const float4*>(y + (int64_t)t * d + col)
                  : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto store_y = [&](int buf) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int u = tid + 256 * r;
      if (u < RTW * 64) sy4[buf][u / 64][u % 64] = yv[r];
    }
  };
  load_y(0);
  store_y(0);
  if (nsteps > 1) load_y(256);
  uint4 qa = make_uint4(0, 0, 0, 0), qb = qa;
  uint16_t dbits = 0;
  if (has_e) { qa = wrow[0]; qb = wrow[1]; dbits = drow[0]; }
  __syncthreads();

  float acc[RTT];
#pragma unroll
  for (int tt = 0; tt < RTT; ++tt) acc[tt] = 0.0f;
  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    if (has_e) {
      const int blk0 = s * (256 / QK);
      const int nbs = min(256 / QK, nb - blk0);
      for (int b = 0; b < nbs; ++b) {
        const int blk = blk0 + b;
        float qf[QK];
        router_raw_weights(qa, qb, qf);
        const float ds = half_bits_to_float(dbits);
        if (blk + 1 < nb) {
          qa = wrow[2 * (blk + 1)];
          qb = wrow[2 * (blk + 1) + 1];
          dbits = drow[blk + 1];
        }
        // the RTT tokens' sums are independent chains: advance them together, one
        // product and one add per token and weight, in the same per-token order
        float P[RTT];
#pragma unroll
        for (int j4 = 0; j4 < QK / 4; ++j4) {
          float4 yq[RTT];
#pragma unroll
          for (int tt = 0; tt < RTT; ++tt) yq[tt] = sy4[buf][grp * RTT + tt][b * (QK / 4) + j4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
#pragma unroll
            for (int tt = 0; tt < RTT; ++tt) {
              const float yc = c == 0 ? yq[tt].x : c == 1 ? yq[tt].y : c == 2 ? yq[tt].z : yq[tt].w;
              const float prod = __fmul_rn(qf[4 * j4 + c], yc);
              P[tt] = (j4 == 0 && c == 0) ? prod : __fadd_rn(P[tt], prod);
            }
          }
        }
#pragma unroll
        for (int tt = 0; tt < RTT; ++tt) {
          const float term = __fmul_rn(ds, P[tt]);
          acc[tt] = (blk == 0) ? term : __fadd_rn(acc[tt], term);
        }
      }
    }
    if (s + 1 < nsteps) {
      // buffer buf ^ 1 was last read in step s - 1, which every thread finished before
      // the barrier that opened step s
      store_y(buf ^ 1);
      if (s + 2 < nsteps) load_y((s + 2) * 256);
      __syncthreads();
    }
  }
  __syncthreads();
  if (has_e) {
#pragma unroll
    for (int tt = 0; tt < RTT; ++tt) {
      const int tw = grp * RTT + tt;
      slog[tw][e] = acc[tt];
      if (t0 + tw < n) logits[(int64_t)(t0 + tw) * E + e] = acc[tt];
    }
  }
  __syncthreads();
  const int lane = tid & 63, wave = tid >> 6;
  for (int tt = wave; tt < RTW; tt += 4) {
    const int t = t0 + tt;
    if (t >= n) break;
    route_topk(slog[tt], E, k, lane, idx + (int64_t)t * k, wout + (int64_t)t * k);
  }
}

// Few tokens (decode-sized chunks): the per-token work of the kernel above is one serial
// chain per expert, too long for a handful of workgroups.  Here a wave owns one expert and
// RSN tokens; lane b computes the block products d_b * P_b of blocks b, b+64, ... (same
// float32 order), parks them in LDS, and lane t then adds them in ascending block order.
// Top-k follows in router_topk_kernel, over the logits written here.
constexpr int RSN = 4;          // tokens per wave
constexpr int kRouterSmallMaxBlocks = 256;   // d <= 8192
__global__ __launch_bounds__(64) void router_small_kernel(const float* __restrict__ y,
                                                          const int8_t* __restrict__ rq,
                                                          const uint16_t* __restrict__ rd,
                                                          int32_t n, int32_t d, int32_t E,
                                                          float* __restrict__ logits) {
  __shared__ float sterm[RSN][kRouterSmallMaxBlocks];
  const int lane = threadIdx.x;
  const int e = blockIdx.x;
  const int t0 = blockIdx.y * RSN;
  const int nt = min(RSN, n - t0);
  const int nb = d / QK;
  for (int blk = lane; blk < nb; blk += 64) {
    float qf[QK];
    router_block_weights(rq + (int64_t)e * d + blk * QK, qf);
    const float ds = half_bits_to_float(rd[(int64_t)e * nb + blk]);
    for (int tt = 0; tt < nt; ++tt) {
      const float4* ys = reinterpret_cast<const float4*>(y + (int64_t)(t0 + tt) * d + blk * QK);
      sterm[tt][blk] = __fmul_rn(ds, router_block_dot(qf, ys));
    }
  }
  __syncthreads();
  if (lane < nt) {
    float acc = sterm[lane][0];
    for (int blk = 1; blk < nb; ++blk) acc = __fadd_rn(acc, sterm[lane][blk]);
    logits[(int64_t)(t0 + lane) * E + e] = acc;
  }
}

__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ logits,
                                                          int32_t n, int32_t E, int32_t k,
                                                          int32_t* __restrict__ idx,
                                                          float* __restrict__ wout) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= n) return;
  route_topk(logits + (int64_t)t * E, E, k, threadIdx.x & 63, idx + (int64_t)t * k,
             wout + (int64_t)t * k);
}

// token count up to which the wave-per-expert router runs
constexpr int32_t kRouterSmallN = 16;

hipError_t launch_router(const float* y, const int8_t* rq, const uint16_t* rd, int32_t n, int32_t d,
                         int32_t E, int32_t k, float* logits, int32_t* idx, float* w,
                         hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (n <= kRouterSmallN && d / QK <= kRouterSmallMaxBlocks) {
    hipLaunchKernelGGL(router_small_kernel, dim3((unsigned)E, (unsigned)ceil_div(n, RSN)), dim3(64), 0, s,
                       y, rq, rd, n, d, E, logits);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(router_topk_kernel, dim3((unsigned)ceil_div(n, 4)), dim3(256), 0, s, logits, n, E,
                       k, idx, w);
    return hipGetLastError();
  }
  const int rtw = RTT * (E <= 128 ? 2 : 1);
  hipLaunchKernelGGL(router_kernel, dim3((unsigned)ceil_div(n, rtw)), dim3(256), 0, s, y, rq, rd, n,
                     d, E, k, logits, idx, w);
  return hipGetLastError();
}

// Permute: slots s = t*k + rank are grouped by expert, stable in slot order.
//  (1) per chunk of 256 slots: rank of each slot among earlier equal-expert slots in the
//      chunk, and the chunk's per-expert counts;
//  (2) one workgroup: per-expert exclusive sums over chunks, expert offsets, tile table;
//  (3) per chunk: position = base(chunk, expert) + rank.
__global__ __launch_bounds__(256) void moe_rank_kernel(const int32_t* __restrict__ idx, int32_t n_slots,
                                                       int32_t E, int32_t* __restrict__ rank,
                                                       int32_t* __restrict__ chunk_cnt) {
  __shared__ int32_t se[kMoeChunk];
  __shared__ int32_t scnt[256];
  const int tid = threadIdx.x;
  const int64_t s = (int64_t)blockIdx.x * kMoeChunk + tid;
  const bool valid = s < n_slots;
  se[tid] = valid ? idx[s] : -1;
  for (int e = tid; e < E; e += 256) scnt[e] = 0;
  __syncthreads();
  if (valid) {
    const int e = se[tid];
    int r = 0;
    for (int j = 0; j < tid; ++j) r += (se[j] == e);
    rank[s] = r;
    atomicAdd(&scnt[e], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) chunk_cnt[(int64_t)blockIdx.x * E + e] = scnt[e];
}

// per-chunk counts staged in LDS by the scan when they fit (16K counts = 64 KiB)
constexpr int64_t kMoeScanLds = 16384;

__global__ __launch_bounds__(256) void moe_scan_kernel(int32_t n_chunks, int32_t E, int32_t mt,
                                                       int32_t max_tiles,
                                                       int32_t* __restrict__ chunk_cnt,
                                                       int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ tiles,
                                                       int32_t* __restrict__ n_tiles) {
  __shared__ int32_t stot[256];
  __shared__ int32_t soff[257];
  extern __shared__ int32_t scnt[];     // [n_chunks][E] when it fits (see the launch)
  const int tid = threadIdx.x;
  const int64_t ncnt = (int64_t)n_chunks * E;
  const bool staged = ncnt <= kMoeScanLds;
  if (staged) {
    // coalesced loads into LDS, the per-expert running sums there, coalesced stores back
    for (int64_t u = tid; u < ncnt; u += 256) scnt[u] = chunk_cnt[u];
    __syncthreads();
    for (int e = tid; e < E; e += 256) {
      int total = 0;
      for (int c = 0; c < n_chunks; ++c) {
        const int v = scnt[c * E + e];
        scnt[c * E + e] = total;
        total += v;
      }
      stot[e] = total;
    }
  } else {
    for (int e = tid; e < E; e += 256) {
      int total = 0;
      for (int c = 0; c < n_chunks; ++c) {
        const int v = chunk_cnt[(int64_t)c * E + e];
        chunk_cnt[(int64_t)c * E + e] = total;
        total += v;
      }
      stot[e] = total;
    }
  }
  __syncthreads();
  // expert offsets and tile-table offsets: exclusive prefix sums over the experts (E <= 256,
  // one thread each; a log-step scan in LDS)
  __shared__ int32_t ssum[2][256];
  __shared__ int32_t tsum[2][256];
  {
    const int cnt = tid < E ? stot[tid] : 0;
    const int ntl = tid < E ? (cnt + mt - 1) / mt : 0;
    ssum[0][tid] = cnt;
    tsum[0][tid] = ntl;
    __syncthreads();
    int src = 0;
    for (int o = 1; o < 256; o <<= 1) {
      const int v = ssum[src][tid] + (tid >= o ? ssum[src][tid - o] : 0);
      const int u = tsum[src][tid] + (tid >= o ? tsum[src][tid - o] : 0);
      ssum[src ^ 1][tid] = v;
      tsum[src ^ 1][tid] = u;
      __syncthreads();
      src ^= 1;
    }
    const int off = ssum[src][tid] - cnt;            // exclusive sums
    const int t0 = tsum[src][tid] - ntl;
    if (tid < E) {
      soff[tid] = off;
      offsets[tid] = off;
      for (int i = 0; i < ntl; ++i) {
        const int m = i * mt;
        if (t0 + i < max_tiles)
          reinterpret_cast<int4*>(tiles)[t0 + i] = make_int4(tid, off + m, off + min(m + mt, cnt), 0);
      }
    }
    if (tid == 255) {
      offsets[E] = ssum[src][255];
      *n_tiles = min(tsum[src][255], max_tiles);
    }
  }
  __syncthreads();
  if (staged) {
    for (int64_t u = tid; u < ncnt; u += 256) chunk_cnt[u] = scnt[u] + soff[u % E];
  } else {
    for (int e = tid; e < E; e += 256)
      for (int c = 0; c < n_chunks; ++c) chunk_cnt[(int64_t)c * E + e] += soff[e];
  }
}

__global__ __launch_bounds__(256) void moe_scatter_kernel(const int32_t* __restrict__ idx, int32_t n_slots,
                                                          int32_t E, const int32_t* __restrict__ rank,
                                                          const int32_t* __restrict__ chunk_cnt,
                                                          int32_t* __restrict__ perm,
                                                          int32_t* __restrict__ inv) {
  const int64_t s = (int64_t)blockIdx.x * kMoeChunk + threadIdx.x;
  if (s >= n_slots) return;
  const int e = idx[s];
  const int pos = chunk_cnt[(int64_t)blockIdx.x * E + e] + rank[s];
  perm[pos] = (int32_t)s;
  inv[s] = pos;
}

hipError_t launch_moe_permute(const MoeBuffers& b, int32_t n, int32_t E, int32_t k, int32_t mt,
                              int32_t max_tiles, hipStream_t s) {
  const int32_t n_slots = n * k;
  const int32_t n_chunks = (int32_t)ceil_div(n_slots, kMoeChunk);
  hipLaunchKernelGGL(moe_rank_kernel, dim3(n_chunks), dim3(kMoeChunk), 0, s, b.idx, n_slots, E,
                     b.rank, b.chunk_cnt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t scan_lds = (int64_t)n_chunks * E <= kMoeScanLds ? (size_t)n_chunks * E * 4 : 0;
  hipLaunchKernelGGL(moe_scan_kernel, dim3(1), dim3(256), scan_lds, s, n_chunks, E, mt, max_tiles,
                     b.chunk_cnt, b.offsets, b.tiles, b.n_tiles);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(moe_scatter_kernel, dim3(n_chunks), dim3(kMoeChunk), 0, s, b.idx, n_slots, E,
                     b.rank, b.chunk_cnt, b.perm, b.inv);
  return hipGetLastError();
}

// Unpermute: x_out[t] = x_res[t] + sum_{rank} w[t][rank] * y_perm[pos(t, rank)], summed in
// rank order.  One thread per 4 columns of a token; the rows of eight ranks are loaded
// before any of them is added, so their loads are in flight together.
__global__ __launch_bounds__(256) void moe_unpermute_kernel(const float* __restrict__ y_perm,
                                                            const int32_t* __restrict__ inv,
                                                            const float* __restrict__ w, int32_t n,
                                                            int32_t d, int32_t k,
                                                            const float* x_res, float* x_out) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t quads = d / 4;
  if (q >= (int64_t)n * quads) return;
  const int64_t t = q / quads, c = (q % quads) * 4;
  float4 m = make_float4(0.f, 0.f, 0.f, 0.f);
  int r = 0;
  for (; r + 8 <= k; r += 8) {
    float wr[8];
    float4 yv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      wr[j] = w[t * k + r + j];
      yv[j] = *reinterpret_cast<const float4*>(y_perm + (int64_t)inv[t * k + r + j] * d + c);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      m.x += wr[j] * yv[j].x; m.y += wr[j] * yv[j].y; m.z += wr[j] * yv[j].z; m.w += wr[j] * yv[j].w;
    }
  }
  for (; r < k; ++r) {
    const float wr = w[t * k + r];
    const float4 yv = *reinterpret_cast<const float4*>(y_perm + (int64_t)inv[t * k + r] * d + c);
    m.x += wr * yv.x; m.y += wr * yv.y; m.z += wr * yv.z; m.w += wr * yv.w;
  }
  const float4 xr = *reinterpret_cast<const float4*>(x_res + t * d + c);
  *reinterpret_cast<float4*>(x_out + t * d + c) =
      make_float4(xr.x + m.x, xr.y + m.y, xr.z + m.z, xr.w + m.w);
}

hipError_t launch_moe_unpermute(const float* y_perm, const MoeBuffers& b, int32_t n, int32_t d,
                                int32_t k, const float* x_res, float* x_out, hipStream_t s) {
  const int64_t work = (int64_t)n * (d / 4);
  if (work == 0) return hipSuccess;
  hipLaunchKernelGGL(moe_unpermute_kernel, dim3((unsigned)ceil_div(work, 256)), dim3(256), 0, s,
                     y_perm, b.inv, b.w, n, d, k, x_res, x_out);
  return hipGetLastError();
}

}  // namespace cp

namespace cp {

// ======================================================================================
// Last-position logits: RMSNorm of one row, then logits[v] = sum_b d_vb * sum_j q_vbj * y_j
// over the q8_0 LM head in its interchange layout (rows of d/32 blocks of 34 bytes).
// HBM-bound: every head byte is read once.  The normed row is staged in LDS (float32,
// 33 floats per block: lanes on consecutive blocks then read distinct banks, where a
// stride of 32 floats would put every lane of the wave on one bank);
// a wave takes one vocabulary row at a time, its lanes consecutive blocks (so a load
// instruction covers 64 adjacent blocks), each lane reading its block as 17 halfwords;
// the per-lane partial dot products are summed across the wave.
// ======================================================================================
constexpr int LMW = 4;   // waves per workgroup

__global__ __launch_bounds__(LMW * 64) void last_logits_kernel(const float* __restrict__ x,
                                                               const float* __restrict__ gamma,
                                                               const uint8_t* __restrict__ head,
                                                               int32_t vocab, int32_t d, float eps,
                                                               float* __restrict__ logits) {
  extern __shared__ float sy[];
  __shared__ float red[LMW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // RMSNorm of the row (every workgroup recomputes it: d values, negligible next to the head)
  float ss = 0.0f;
  for (int i = tid; i < d; i += LMW * 64) ss += x[i] * x[i];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int w = 0; w < LMW; ++w) tot += red[w];
  const float scale = 1.0f / sqrtf(tot / (float)d + eps);
  for (int i = tid; i < d; i += LMW * 64) sy[i + i / QK] = x[i] * scale * gamma[i];
  __syncthreads();
  const int nb = d / QK;
  const int64_t row_bytes = (int64_t)nb * 34;
  for (int64_t v = (int64_t)blockIdx.x * LMW + wave; v < vocab; v += (int64_t)gridDim.x * LMW) {
    const uint16_t* row = reinterpret_cast<const uint16_t*>(head + v * row_bytes);
    float part = 0.0f;
    for (int b = lane; b < nb; b += 64) {
      const uint16_t* blk = row + b * 17;           // 34 bytes = 17 halfwords
      const float db = half_bits_to_float(blk[0]);
      const float* ys = sy + b * (QK + 1);
      float p = 0.0f;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint16_t two = blk[1 + j];
        p = fmaf((float)(int8_t)(two & 0xFF), ys[2 * j], p);
        p = fmaf((float)(int8_t)(two >> 8), ys[2 * j + 1], p);
      }
      part = fmaf(db, p, part);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) part += __shfl_xor(part, o, 64);
    if (lane == 0) logits[v] = part;
  }
}

// Streaming form for rows that are whole 16-byte chunks (d % 256 == 0, head 16-byte
// aligned): a wave reads its rows segment by segment (LL_SEGB blocks, 4352 bytes) with
// coalesced 16-byte loads, keeping the next segment's loads in flight while the current
// one is staged in the wave's LDS slot and decoded there (lane b takes blocks b, b + 64;
// a block is 17 halfwords).  The halfword-per-lane global reads of the form above make
// each load touch 34 cache lines, which caps that form far below the HBM rate.
constexpr int LL_SEGB = 128;                      // q8_0 blocks per segment
constexpr int LL_SEGBYTES = LL_SEGB * 34;         // 4352 bytes = 272 chunks of 16
constexpr int LL_CHL = (LL_SEGBYTES / 16 + 63) / 64;   // chunks per lane per segment

__global__ __launch_bounds__(LMW * 64) void last_logits_stream_kernel(const float* __restrict__ x,
                                                                      const float* __restrict__ gamma,
                                                                      const uint8_t* __restrict__ head,
                                                                      int32_t vocab, int32_t d, float eps,
                                                                      float* __restrict__ logits) {
  extern __shared__ float sy[];                   // y (swizzled, see below), then LMW segment slots
  __shared__ float red[LMW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float ss = 0.0f;
  for (int i = tid; i < d; i += LMW * 64) ss += x[i] * x[i];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int w = 0; w < LMW; ++w) tot += red[w];
  const float scale = 1.0f / sqrtf(tot / (float)d + eps);
  // float4 group g of block b sits at group (g + b) % 8 of the block's 32 floats: lanes on
  // consecutive blocks reading the same group then hit distinct banks, and every read is
  // an aligned 16-byte one
  for (int i = tid; i < d; i += LMW * 64) {
    const int b = i / QK, g = (i % QK) / 4;
    sy[b * QK + 4 * ((g + b) & 7) + (i & 3)] = x[i] * scale * gamma[i];
  }
  __syncthreads();

  uint8_t* slot = reinterpret_cast<uint8_t*>(sy + d) + wave * LL_SEGBYTES;
  const int nb = d / QK, nseg = (nb + LL_SEGB - 1) / LL_SEGB;
  const int64_t row_bytes = (int64_t)nb * 34;
  // Items are (row, segment) pairs, segments fastest, walked incrementally: row v0, then
  // every vstep-th row.  (Deriving the pair from a flat 64-bit item index took a 64-bit
  // division per item, more scalar work than the item's own.)
  const int v0 = blockIdx.x * LMW + wave, vstep = gridDim.x * LMW;
  auto seg_blocks = [&](int sg) { return min(LL_SEGB, nb - sg * LL_SEGB); };
  auto load = [&](int v, int sg, uint4 (&r)[LL_CHL]) {
    const int nc = seg_blocks(sg) * 34 / 16;
    const uint4* src = reinterpret_cast<const uint4*>(head + (int64_t)v * row_bytes + (int64_t)sg * LL_SEGBYTES);
#pragma unroll
    for (int c = 0; c < LL_CHL; ++c) {
      const int ch = lane + 64 * c;
      r[c] = ch < nc ? src[ch] : make_uint4(0, 0, 0, 0);
    }
  };
  uint4 cur[LL_CHL], nxt[LL_CHL];
  if (v0 < vocab) load(v0, 0, cur);
  float part = 0.0f;
  for (int v = v0, sg = 0; v < vocab;) {
    const int nsg = sg + 1 < nseg ? sg + 1 : 0;
    const int nv = sg + 1 < nseg ? v : (v < vocab - vstep ? v + vstep : vocab);   // no int overflow
    if (nv < vocab) load(nv, nsg, nxt);
    const int nbs = seg_blocks(sg), nc = nbs * 34 / 16;
    // The slot belongs to this wave alone, and a wave's LDS operations take effect in
    // program order: the reads below see these writes, and the next item's writes come
    // after these reads.
#pragma unroll
    for (int c = 0; c < LL_CHL; ++c) {
      const int ch = lane + 64 * c;
      if (ch < nc) reinterpret_cast<uint4*>(slot)[ch] = cur[c];
    }
    __builtin_amdgcn_wave_barrier();
    for (int b = lane; b < nbs; b += 64) {
      // the block's 34 bytes from nine aligned words of the slot: block b starts at byte
      // 34b, which is 0 or 2 past a word boundary; byte shifts realign them
      const int a = (34 * b) >> 2, r = (34 * b) & 3;
      const uint32_t* sw = reinterpret_cast<const uint32_t*>(slot) + a;
      uint32_t u[9];
#pragma unroll
      for (int i = 0; i < 9; ++i) u[i] = sw[i];
#pragma unroll
      for (int i = 0; i < 8; ++i) u[i] = __builtin_amdgcn_alignbyte(u[i + 1], u[i], r);
      u[8] = __builtin_amdgcn_alignbyte(0u, u[8], r);
      const float db = half_bits_to_float(u[0] & 0xFFFFu);
      const int blk = sg * LL_SEGB + b;
      const float4* ys = reinterpret_cast<const float4*>(sy + blk * QK);
      float p = 0.0f;
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const float4 yv = ys[(g + blk) & 7];
        const float yy[4] = {yv.x, yv.y, yv.z, yv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 4 * g + e, byte = j + 2;        // q_j is byte j + 2 of the block
          const int q = __builtin_amdgcn_sbfe((int)u[byte >> 2], 8 * (byte & 3), 8);
          p = fmaf((float)q, yy[e], p);
        }
      }
      part = fmaf(db, p, part);
    }
    __builtin_amdgcn_wave_barrier();
    if (sg == nseg - 1) {
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) part += __shfl_xor(part, o, 64);
      if (lane == 0) logits[v] = part;
      part = 0.0f;
    }
#pragma unroll
    for (int c = 0; c < LL_CHL; ++c) cur[c] = nxt[c];
    v = nv;
    sg = nsg;
  }
}

// Row-pair form for heads whose two rows fit a wave's LDS slot (d % 256 == 0, d <= 5120):
// an item is two consecutive rows (contiguous bytes, whole 16-byte chunks), so a wave's
// lanes run over 2*d/32 blocks with none idle at the row's end, and the per-item work
// (loads, staging, the cross-lane sums) is shared by two rows.  y is staged with a
// 36-float stride per block: 16 lanes on consecutive blocks reading 16 bytes each then
// hit 16 distinct 4-bank groups, and the eight reads of a block take immediate offsets.
constexpr int LLP_CH = 11;                                // 16-byte chunks per lane per item
constexpr int LLP_SLOT = LLP_CH * 64 * 16;                // 11,264 bytes: two rows at d = 5120
constexpr int LLP_YS = 36;                                // floats per staged y block

__global__ __launch_bounds__(LMW * 64) void last_logits_pair_kernel(const float* __restrict__ x,
                                                                    const float* __restrict__ gamma,
                                                                    const uint8_t* __restrict__ head,
                                                                    int32_t vocab, int32_t d, float eps,
                                                                    float* __restrict__ logits) {
  extern __shared__ float sy[];                   // y (nb blocks of LLP_YS floats), then LMW slots
  __shared__ float red[LMW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float ss = 0.0f;
  for (int i = tid; i < d; i += LMW * 64) ss += x[i] * x[i];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int w = 0; w < LMW; ++w) tot += red[w];
  const float scale = 1.0f / sqrtf(tot / (float)d + eps);
  for (int i = tid; i < d; i += LMW * 64) sy[(i / QK) * LLP_YS + i % QK] = x[i] * scale * gamma[i];
  __syncthreads();

  const int nb = d / QK;
  uint8_t* slot = reinterpret_cast<uint8_t*>(sy + nb * LLP_YS) + wave * LLP_SLOT;
  const int row_bytes = nb * 34;
  const int npair = (vocab + 1) / 2;
  const int p0 = blockIdx.x * LMW + wave, pstep = gridDim.x * LMW;
  auto load = [&](int p, uint4 (&r)[LLP_CH]) {
    const int nc = min(2, vocab - 2 * p) * row_bytes / 16;
    const uint4* src = reinterpret_cast<const uint4*>(head + (int64_t)(2 * p) * row_bytes);
#pragma unroll
    for (int c = 0; c < LLP_CH; ++c) {
      const int ch = lane + 64 * c;
      r[c] = ch < nc ? src[ch] : make_uint4(0, 0, 0, 0);
    }
  };
  uint4 cur[LLP_CH], nxt[LLP_CH];
  if (p0 < npair) load(p0, cur);
  for (int p = p0; p < npair;) {
    const int np = p < npair - pstep ? p + pstep : npair;   // no int overflow
    if (np < npair) load(np, nxt);
    const int rows = min(2, vocab - 2 * p);
    const int nc = rows * row_bytes / 16;
    // The slot belongs to this wave alone, and a wave's LDS operations take effect in
    // program order: the reads below see these writes, and the next item's writes come
    // after these reads.
#pragma unroll
    for (int c = 0; c < LLP_CH; ++c) {
      const int ch = lane + 64 * c;
      if (ch < nc) reinterpret_cast<uint4*>(slot)[ch] = cur[c];
    }
    __builtin_amdgcn_wave_barrier();
    float part0 = 0.0f, part1 = 0.0f;
    for (int b = lane; b < rows * nb; b += 64) {
      // block b of the item starts at byte 34b (0 or 2 past a word boundary); nine aligned
      // words and byte shifts give its 34 bytes
      const int a = (34 * b) >> 2, r = (34 * b) & 3;
      const uint32_t* sw = reinterpret_cast<const uint32_t*>(slot) + a;
      uint32_t u[9];
#pragma unroll
      for (int i = 0; i < 9; ++i) u[i] = sw[i];
#pragma unroll
      for (int i = 0; i < 8; ++i) u[i] = __builtin_amdgcn_alignbyte(u[i + 1], u[i], r);
      u[8] = __builtin_amdgcn_alignbyte(0u, u[8], r);
      const float db = half_bits_to_float(u[0] & 0xFFFFu);
      const bool second = b >= nb;
      const int blk = second ? b - nb : b;
      const float4* ys = reinterpret_cast<const float4*>(sy + blk * LLP_YS);
      float q = 0.0f;
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const float4 yv = ys[g];
        const float yy[4] = {yv.x, yv.y, yv.z, yv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 4 * g + e, byte = j + 2;        // q_j is byte j + 2 of the block
          const int qv = __builtin_amdgcn_sbfe((int)u[byte >> 2], 8 * (byte & 3), 8);
          q = fmaf((float)qv, yy[e], q);
        }
      }
      if (second) part1 = fmaf(db, q, part1);
      else part0 = fmaf(db, q, part0);
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      part0 += __shfl_xor(part0, o, 64);
      part1 += __shfl_xor(part1, o, 64);
    }
    if (lane == 0) {
      logits[2 * p] = part0;
      if (rows == 2) logits[2 * p + 1] = part1;
    }
#pragma unroll
    for (int c = 0; c < LLP_CH; ++c) cur[c] = nxt[c];
    p = np;
  }
}

// The largest dynamic LDS each last-logits kernel has been allowed on each device: the
// attribute is set only when a launch needs more (a call per launch costs host time of the
// order of the kernel's own).
hipError_t allow_dyn_lds(const void* fn, int which, size_t bytes) {
  static std::mutex mu;
  static size_t allowed[3][64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  std::lock_guard<std::mutex> lk(mu);
  if (allowed[which][dev] >= bytes) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) allowed[which][dev] = bytes;
  return e;
}

hipError_t launch_last_logits(const float* x, const float* gamma, const void* head, int32_t vocab,
                              int32_t d, float eps, float* logits, hipStream_t s) {
  if (d % 256 == 0 && (uintptr_t)head % 16 == 0 && 2 * (d / QK) * 34 <= LLP_SLOT) {
    // two workgroups per CU (the LDS allows two) that stay resident and walk every
    // 2048th row pair: fewer, longer-lived waves streamed faster than more of them
    const unsigned pgrid = (unsigned)std::min<int64_t>(ceil_div(ceil_div(vocab, 2), LMW), 512);
    const size_t lds = (size_t)(d / QK) * LLP_YS * sizeof(float) + (size_t)LMW * LLP_SLOT;
    hipError_t e = allow_dyn_lds((const void*)last_logits_pair_kernel, 0, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(last_logits_pair_kernel, dim3(pgrid), dim3(LMW * 64), lds, s, x, gamma,
                       (const uint8_t*)head, vocab, d, eps, logits);
    return hipGetLastError();
  }
  const unsigned grid = (unsigned)std::min<int64_t>(ceil_div(vocab, LMW), 2048);
  if (d % 256 == 0 && (uintptr_t)head % 16 == 0) {
    const size_t lds = (size_t)d * sizeof(float) + (size_t)LMW * LL_SEGBYTES;
    hipError_t e = allow_dyn_lds((const void*)last_logits_stream_kernel, 1, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(last_logits_stream_kernel, dim3(grid), dim3(LMW * 64), lds, s, x, gamma,
                       (const uint8_t*)head, vocab, d, eps, logits);
    return hipGetLastError();
  }
  const size_t lds = (size_t)(d + d / QK) * sizeof(float);
  hipError_t e = allow_dyn_lds((const void*)last_logits_kernel, 2, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(last_logits_kernel, dim3(grid), dim3(LMW * 64), lds, s,
                     x, gamma, (const uint8_t*)head, vocab, d, eps, logits);
  return hipGetLastError();
}

}  // namespace cp
