// Causal GQA flash attention of a chunk against the KV cache (gfx950, f16 MFMA, fp32
// online softmax).
//
// Query rows of one kv head are packed token-major: row r = t*G + hh (G = Hq/Hkv), so a
// K/V tile staged once in LDS serves all G query heads of that kv head.  Each wave owns
// 32 query rows and computes S^T = K Q^T (32x32x16 MFMA, A = K rows from LDS, B = Q
// fragments held in registers for the whole kernel).  In the S^T accumulator a lane
// holds one query's scores for 16 keys, which is exactly a B operand of the next
// product O^T += V^T P^T once the key index is permuted consistently on V^T's side, so
// the probabilities never leave registers.  Softmax statistics are per lane (one query
// per lane pair).  K/V tiles are 64 positions; the V tile is stored transposed ([dim]
// [position]) in the cache so it stages with contiguous loads.  q8_0 caches are
// dequantised to f16 while staging.  Long KV ranges with few query tiles are split
// across workgroups and merged by a log-sum-exp combine kernel.
#include "cp_internal.h"
#include "k_common.h"

namespace cp {

constexpr int KVT = 64;
constexpr int QROWS = 128;   // query rows per workgroup (4 waves x 32)

int attention_rows_total(int32_t n, int32_t n_head) { return n * n_head; }

template <int HD, bool Q8>
__global__ __launch_bounds__(256, 2) void attn_kernel(AttnArgs a) {
  constexpr int NCH = HD / 8;      // 16-byte chunks per K row
  constexpr int KSTEPS = HD / 16;
  constexpr int DB = HD / 32;
  __shared__ uint4 sK[KVT * NCH];
  __shared__ uint2 sV[HD * 16];    // [dim][8-byte chunk = 4 positions], XOR-swizzled

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int G = a.n_head / a.n_kv_head;
  const int R = a.n * G;
  const int n_qt = (R + QROWS - 1) / QROWS;
  const int qt = n_qt - 1 - (int)blockIdx.x;       // longest KV ranges first
  const int g = blockIdx.y;
  const int split = blockIdx.z;
  const int64_t n_ctx = a.n_ctx;

  const int rw0 = qt * QROWS + wave * 32;
  const int i = rw0 + l32;
  const bool row_ok = i < R;
  const int t_i = row_ok ? i / G : 0;
  const int hq = g * G + (row_ok ? i % G : 0);
  const int qpos = a.start + t_i;

  const int last_row = min(R - 1, qt * QROWS + QROWS - 1);
  const int kv_end = a.start + last_row / G + 1;
  const int n_kvt = (kv_end + KVT - 1) / KVT;
  const int jt0 = (int)((int64_t)split * n_kvt / a.splits);
  const int jt1 = (int)((int64_t)(split + 1) * n_kvt / a.splits);
  const int wave_qmin = a.start + min(rw0, R - 1) / G;

  uint4 qf[KSTEPS];
  {
    const _Float16* qrow = a.q + ((int64_t)t_i * a.n_head + hq) * HD;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk)
      qf[kk] = row_ok ? *reinterpret_cast<const uint4*>(qrow + kk * 16 + 8 * h) : make_uint4(0, 0, 0, 0);
  }

  const float scale = 1.4426950408889634f / sqrtf((float)HD);
  float m = -INFINITY, l = 0.0f;
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[db][e] = 0.0f;

  for (int jt = jt0; jt < jt1; ++jt) {
    const int j0 = jt * KVT;
    __syncthreads();
    // ---- stage K tile [64][HD] ----
    for (int c = tid; c < KVT * NCH; c += 256) {
      const int row = c / NCH, ch = c % NCH;
      const int pos = j0 + row;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (pos < kv_end) {
        const int64_t ri = (int64_t)g * n_ctx + pos;
        if constexpr (!Q8) {
          v = *reinterpret_cast<const uint4*>(reinterpret_cast<const _Float16*>(a.kv.k) + ri * HD + ch * 8);
        } else {
          const uint2 w = *reinterpret_cast<const uint2*>(reinterpret_cast<const int8_t*>(a.kv.k) + ri * HD + ch * 8);
          const float d = half_bits_to_float(a.kv.kd[ri * (HD / QK) + (ch * 8) / QK]);
          const float ds[8] = {d, d, d, d, d, d, d, d};
          v = dequant8_f16(w.x, w.y, ds);
        }
      }
      sK[row * NCH + (ch ^ (row % NCH))] = v;
    }
    // ---- stage V^T tile [HD][64] ----
    for (int c = tid; c < HD * 8; c += 256) {
      const int dd = c >> 3, pc = c & 7;
      const int pos0 = j0 + pc * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (pos0 < kv_end) {
        const int64_t ri = ((int64_t)g * HD + dd) * n_ctx + pos0;
        const bool full = pos0 + 8 <= kv_end;
        if constexpr (!Q8) {
          const _Float16* src = reinterpret_cast<const _Float16*>(a.kv.v) + ri;
          if (full) {
            v = *reinterpret_cast<const uint4*>(src);
          } else {
            uint16_t tmp[8];
            for (int e = 0; e < 8; ++e)
              tmp[e] = pos0 + e < kv_end ? __builtin_bit_cast(uint16_t, src[e]) : (uint16_t)0;
            v = make_uint4(tmp[0] | (tmp[1] << 16), tmp[2] | (tmp[3] << 16),
                           tmp[4] | (tmp[5] << 16), tmp[6] | (tmp[7] << 16));
          }
        } else {
          const int8_t* src = reinterpret_cast<const int8_t*>(a.kv.v) + ri;
          const uint16_t* sd = a.kv.vd + ((int64_t)g * (HD / QK) + dd / QK) * n_ctx + pos0;
          float ds[8];
          uint32_t w0 = 0, w1 = 0;
          if (full) {
            const uint2 w = *reinterpret_cast<const uint2*>(src);
            w0 = w.x;
            w1 = w.y;
            const uint4 sv = *reinterpret_cast<const uint4*>(sd);
            const uint32_t s4[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              ds[2 * e] = half_bits_to_float(s4[e] & 0xFFFFu);
              ds[2 * e + 1] = half_bits_to_float(s4[e] >> 16);
            }
          } else {
            for (int e = 0; e < 8; ++e) {
              const bool ok = pos0 + e < kv_end;
              const uint32_t b = ok ? (uint32_t)(uint8_t)src[e] : 0u;
              if (e < 4) w0 |= b << (8 * e);
              else w1 |= b << (8 * (e - 4));
              ds[e] = ok ? half_bits_to_float(sd[e]) : 0.0f;
            }
          }
          v = dequant8_f16(w0, w1, ds);
        }
      }
      const int q0 = 2 * pc, q1 = 2 * pc + 1, sw = dd & 15;
      sV[dd * 16 + (q0 ^ sw)] = make_uint2(v.x, v.y);
      sV[dd * 16 + (q1 ^ sw)] = make_uint2(v.z, v.w);
    }
    __syncthreads();

    // ---- S^T = K Q^T ----
    f32x16 s[2];
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[jb][e] = 0.0f;
      const int row = jb * 32 + l32;
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        const int ch = kk * 2 + h;
        const uint4 av = sK[row * NCH + (ch ^ (row % NCH))];
        s[jb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, av),
                                                       __builtin_bit_cast(f16x8, qf[kk]), s[jb], 0, 0, 0);
      }
    }
    // ---- causal mask (only tiles reaching past the wave's earliest query) ----
    if (j0 + KVT - 1 > wave_qmin || !row_ok) {
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int j = j0 + jb * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
          if (j > qpos || !row_ok) s[jb][e] = -INFINITY;
        }
    }
    // ---- online softmax (log2 domain) ----
    float mx = -INFINITY;
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[jb][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mnew = fmaxf(m, mx * scale);
    const float msafe = (mnew == -INFINITY) ? 0.0f : mnew;
    const float alpha = __builtin_amdgcn_exp2f(m - msafe);
    float ls = 0.0f;
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[jb][e], scale, -msafe));
        s[jb][e] = p;
        ls += p;
      }
    ls += __shfl_xor(ls, 32, 64);
    l = l * alpha + ls;
    m = mnew;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[db][e] *= alpha;

    // ---- O^T += V^T P^T ----
    uint4 pb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int jb = ks >> 1, kk = ks & 1;
      pb[ks] = make_uint4(pack_f16x2(s[jb][8 * kk + 0], s[jb][8 * kk + 1]),
                          pack_f16x2(s[jb][8 * kk + 2], s[jb][8 * kk + 3]),
                          pack_f16x2(s[jb][8 * kk + 4], s[jb][8 * kk + 5]),
                          pack_f16x2(s[jb][8 * kk + 6], s[jb][8 * kk + 7]));
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int dd = db * 32 + l32, sw = dd & 15;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const uint2 lo = sV[dd * 16 + ((ks * 4 + h) ^ sw)];
        const uint2 hi = sV[dd * 16 + ((ks * 4 + 2 + h) ^ sw)];
        const uint4 av = make_uint4(lo.x, lo.y, hi.x, hi.y);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, av),
                                                       __builtin_bit_cast(f16x8, pb[ks]), o[db], 0, 0, 0);
      }
    }
  }

  if (!row_ok) return;
  if (a.splits == 1) {
    const float inv_l = 1.0f / l;
    __bf16* orow = a.out + ((int64_t)t_i * a.n_head + hq) * HD;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = db * 32 + 8 * rq + 4 * h;
        const uint2 pk = make_uint2(pack_bf16x2(o[db][4 * rq] * inv_l, o[db][4 * rq + 1] * inv_l),
                                    pack_bf16x2(o[db][4 * rq + 2] * inv_l, o[db][4 * rq + 3] * inv_l));
        *reinterpret_cast<uint2*>(orow + d0) = pk;
      }
  } else {
    const int64_t rows_total = (int64_t)a.n_kv_head * R;
    const int64_t rg = (int64_t)g * R + i;
    float* po = a.part_o + ((int64_t)split * rows_total + rg) * HD;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = db * 32 + 8 * rq + 4 * h;
        *reinterpret_cast<float4*>(po + d0) =
            make_float4(o[db][4 * rq], o[db][4 * rq + 1], o[db][4 * rq + 2], o[db][4 * rq + 3]);
      }
    if (h == 0) {
      float* pm = a.part_ml + ((int64_t)split * rows_total + rg) * 2;
      pm[0] = m;
      pm[1] = l;
    }
  }
}

// Merge split-KV partials: o = sum_s 2^(m_s - m*) O_s / sum_s 2^(m_s - m*) l_s.
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  const int G = a.n_head / a.n_kv_head;
  const int64_t R = (int64_t)a.n * G;
  const int64_t rows_total = (int64_t)a.n_kv_head * R;
  const int hd = a.head_dim;
  const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= rows_total * (hd / 4)) return;
  const int64_t rg = u / (hd / 4);
  const int d0 = (int)(u % (hd / 4)) * 4;
  float mstar = -INFINITY;
  for (int s = 0; s < a.splits; ++s) mstar = fmaxf(mstar, a.part_ml[((int64_t)s * rows_total + rg) * 2]);
  float den = 0.0f;
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < a.splits; ++s) {
    const float ms = a.part_ml[((int64_t)s * rows_total + rg) * 2];
    if (ms == -INFINITY) continue;
    const float w = __builtin_amdgcn_exp2f(ms - mstar);
    den += w * a.part_ml[((int64_t)s * rows_total + rg) * 2 + 1];
    const float4 po = *reinterpret_cast<const float4*>(a.part_o + ((int64_t)s * rows_total + rg) * hd + d0);
    num.x += w * po.x; num.y += w * po.y; num.z += w * po.z; num.w += w * po.w;
  }
  const float inv = 1.0f / den;
  const int64_t g = rg / R, i = rg % R;
  const int64_t t = i / G, hq = g * G + i % G;
  __bf16* orow = a.out + (t * a.n_head + hq) * hd + d0;
  *reinterpret_cast<uint2*>(orow) = make_uint2(pack_bf16x2(num.x * inv, num.y * inv),
                                              pack_bf16x2(num.z * inv, num.w * inv));
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  const int G = a.n_head / a.n_kv_head;
  const int R = a.n * G;
  dim3 grid((R + QROWS - 1) / QROWS, a.n_kv_head, a.splits);
  const bool q8 = a.kv_type != CP_KV_F16;
  if (a.head_dim == 128) {
    if (q8) hipLaunchKernelGGL((attn_kernel<128, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((attn_kernel<128, false>), grid, dim3(256), 0, s, a);
  } else {
    if (q8) hipLaunchKernelGGL((attn_kernel<64, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((attn_kernel<64, false>), grid, dim3(256), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits <= 1) return e;
  const int64_t work = (int64_t)a.n_kv_head * R * (a.head_dim / 4);
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)ceil_div(work, 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace cp
