// Causal GQA flash attention of a chunk against the KV cache (gfx950, f16 MFMA, fp32
// online softmax).
//
// Query rows of one kv head are packed token-major: row r = t*G + hh (G = Hq/Hkv), so a
// K/V tile staged once in LDS serves all G query heads of that kv head.  A workgroup of
// 8 waves owns 256 query rows; each wave owns 32 and computes S^T = K Q^T (32x32x16
// MFMA, A = K rows from LDS, B = Q fragments held in registers for the whole kernel).
// In the S^T accumulator a lane holds one query's scores for 16 keys, which is exactly a
// B operand of the next product O^T += V^T P^T, so the probabilities never leave
// registers.  Lane l of the K operand loads key row l with bits 2 and 3 swapped; then
// the eight probabilities a lane feeds to each V^T P^T step are eight consecutive keys,
// and the matching V^T fragment is one 16-byte LDS read.  Softmax
// statistics are per lane (one query per lane pair); the running maximum is raised
// lazily: O and l are rescaled only when some lane's maximum grew by more than 2^8,
// which keeps every probability below 2^8 (safe in f16) and skips the rescale on most
// tiles.  K/V tiles are 64 positions, double buffered in LDS; the V tile is stored
// transposed ([dim][position]) in the cache.  f16 tiles arrive by asynchronous
// global->LDS loads (the swizzle is chosen through each lane's source address); q8_0
// tiles are loaded into registers two tiles ahead and dequantised into LDS.  Long KV
// ranges with few query tiles are split across workgroups and merged by a log-sum-exp
// combine kernel.
#include "cp_internal.h"
#include "k_common.h"

namespace cp {

constexpr int KVT = 64;
constexpr int AW = 8;              // waves per workgroup
constexpr int QROWS = AW * 32;     // query rows per workgroup

typedef __attribute__((address_space(1))) const void gvoid_a;
typedef __attribute__((address_space(3))) void lvoid_a;

int attention_rows_total(int32_t n, int32_t n_head) { return n * n_head; }

__device__ __forceinline__ void attn_wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt vmcnt(N) lgkmcnt(0) (gfx9 encoding, expcnt not waited).
template <int N>
__device__ __forceinline__ void attn_wait_vm_lgkm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070);
}
// Compiler-only fence: memory operations are not moved across it.
__device__ __forceinline__ void attn_cfence() { __atomic_signal_fence(__ATOMIC_SEQ_CST); }
// 16-byte buffer load into LDS.  Buffer loads (unlike the global form) are not counted
// as LDS events, so LDS reads of the current tile keep partial lgkmcnt waits while the
// next tiles are in flight; the scalar offset is made explicitly uniform (otherwise the
// compiler may wrap each load in a loop over its distinct values).
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs, lvoid_a* dst, int32_t voff, int32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, voff, __builtin_amdgcn_readfirstlane(soff), 0, 0);
}

// V^T tile swizzle: 16-byte chunk lc of row d sits at physical chunk lc ^ vswz(d).
__device__ __forceinline__ int vswz(int d) { return (d >> 1) & 7; }

template <int HD, bool Q8>
__global__ __launch_bounds__(AW * 64, 1) void attn_kernel(AttnArgs a) {
  constexpr int NCH = HD / 8;      // 16-byte chunks per K row
  constexpr int KSTEPS = HD / 16;
  constexpr int DB = HD / 32;
  constexpr int KCH = KVT * NCH;   // chunks per K tile
  constexpr int VCH = HD * 8;      // chunks per V tile (8 per dim row)
  constexpr int NKL = KCH / (AW * 64); // K loads per thread per tile (f16)
  constexpr int NVL = VCH / (AW * 64); // V loads per thread per tile (f16)
  constexpr int NLOAD = NKL + NVL;
  // three tile buffers, separate LDS objects so the compiler can tell reads of one tile
  // from asynchronous writes into another
  __shared__ uint4 sK0[KCH], sK1[KCH], sK2[Q8 ? 1 : KCH];
  __shared__ uint4 sV0[VCH], sV1[VCH], sV2[Q8 ? 1 : VCH];
  auto bufK = [&](auto J) __attribute__((always_inline)) -> uint4* {
    constexpr int j = decltype(J)::value;
    if constexpr (j == 0) return sK0; else if constexpr (j == 1) return sK1; else return sK2;
  };
  auto bufV = [&](auto J) __attribute__((always_inline)) -> uint4* {
    constexpr int j = decltype(J)::value;
    if constexpr (j == 0) return sV0; else if constexpr (j == 1) return sV1; else return sV2;
  };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int G = a.n_head / a.n_kv_head;
  const int R = a.n * G;
  const int n_qt = (R + QROWS - 1) / QROWS;
  // Workgroup order.  Workgroup i runs on XCD i % 8; each XCD gets a contiguous range of
  // logical indices, query tile fastest, so the query tiles that walk the same K/V range
  // (one kv head, one split) share an XCD's L2 instead of fetching it once per XCD.
  // Within a range the longest KV spans go first.
  const int total = n_qt * a.n_kv_head * a.splits;
  const int bi = blockIdx.x;
  const int xcd = bi & 7, idx = bi >> 3;
  const int q8 = total >> 3, r8 = total & 7;
  const int logical = (xcd < r8) ? xcd * (q8 + 1) + idx : r8 * (q8 + 1) + (xcd - r8) * q8 + idx;
  const int qt = n_qt - 1 - logical % n_qt;
  const int g = (logical / n_qt) % a.n_kv_head;
  const int split = logical / (n_qt * a.n_kv_head);
  const int64_t n_ctx = a.n_ctx;

  const int rw0 = qt * QROWS + wave * 32;
  // A wave whose 32 rows all lie past the last query row (a short chunk: one token has G
  // rows) still loads its share of every tile and joins every barrier, but skips the
  // arithmetic, leaving its SIMD to the wave it shares it with.
  const bool wave_rows = rw0 < R;
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
  const int krow = (l32 & ~12) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);   // bits 2, 3 swapped

  uint4 qf[KSTEPS];
  {
    const _Float16* qrow = a.q + ((int64_t)t_i * a.n_head + hq) * HD;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk)
      qf[kk] = row_ok ? *reinterpret_cast<const uint4*>(qrow + kk * 16 + 8 * h) : make_uint4(0, 0, 0, 0);
  }

  // ---- tile staging ----
  // f16: buffer loads into LDS.  Load j of wave w fills physical chunks [(j*AW + w)*64,
  // +64); the swizzle is chosen through each lane's source offset (constant per lane; the
  // tile's first position goes into the scalar offset).
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(reinterpret_cast<const _Float16*>(a.kv.k) + (int64_t)g * n_ctx * HD), (short)0,
      (int)min(n_ctx * HD * 2, (int64_t)0x7FFFFFFF), 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(reinterpret_cast<const _Float16*>(a.kv.v) + (int64_t)g * HD * n_ctx), (short)0,
      (int)min(n_ctx * HD * 2, (int64_t)0x7FFFFFFF), 0x00020000);
  int32_t koff[NKL], voff[NVL];
#pragma unroll
  for (int j = 0; j < NKL; ++j) {
    const int P = (j * AW + wave) * 64 + lane;
    const int row = P / NCH, lc = (P % NCH) ^ (row % NCH);
    koff[j] = (row * HD + lc * 8) * 2;
  }
#pragma unroll
  for (int j = 0; j < NVL; ++j) {
    const int P = (j * AW + wave) * 64 + lane;
    const int d = P >> 3, lc = (P & 7) ^ vswz(d);
    voff[j] = (int32_t)(((int64_t)d * n_ctx + lc * 8) * 2);
  }
  auto issue_f16 = [&](auto J, int jt) __attribute__((always_inline)) {
    const int j0 = jt * KVT;
#pragma unroll
    for (int j = 0; j < NKL; ++j) lds_dma16(krs, (lvoid_a*)&bufK(J)[(j * AW + wave) * 64], koff[j], j0 * HD * 2);
#pragma unroll
    for (int j = 0; j < NVL; ++j) lds_dma16(vrs, (lvoid_a*)&bufV(J)[(j * AW + wave) * 64], voff[j], j0 * 2);
  };
  // q8_0: one 16-int8 chunk of K and of V per thread (and its scales), held in registers.
  // A tile's positions are all below the cache capacity (a multiple of the tile), so every
  // thread loads its chunk unconditionally: the same loads for every tile, which keeps the
  // compiler's load-count waits exact while the next tiles are in flight.
  constexpr int KQ = KVT * (HD / 16), VQ = HD * (KVT / 16);   // int8 chunks per tile
  static_assert(!Q8 || (KQ <= AW * 64 && VQ <= AW * 64), "at most one K and one V chunk per thread");
  constexpr bool all_k = KQ == AW * 64, all_v = VQ == AW * 64;   // every thread has one
  const int8_t* Kq = reinterpret_cast<const int8_t*>(a.kv.k) + (int64_t)g * n_ctx * HD;
  const int8_t* Vq = reinterpret_cast<const int8_t*>(a.kv.v) + (int64_t)g * HD * n_ctx;
  const uint16_t* Kd = a.kv.kd + (int64_t)g * n_ctx * (HD / QK);
  const uint16_t* Vd = a.kv.vd + (int64_t)g * (HD / QK) * n_ctx;
  const int qk_row = tid / (HD / 16), qk_c16 = tid % (HD / 16);
  const int qv_d = tid / (KVT / 16), qv_c16 = tid % (KVT / 16);
  struct Q8Regs { uint4 k, v, vs0, vs1; uint16_t ks; };
  auto load_q8 = [&](int jt, Q8Regs& r) __attribute__((always_inline)) {
    const int j0 = jt * KVT;
    if (all_k || tid < KQ) {
      const int pos = j0 + qk_row;
      r.k = *reinterpret_cast<const uint4*>(Kq + (int64_t)pos * HD + qk_c16 * 16);
      r.ks = Kd[(int64_t)pos * (HD / QK) + qk_c16 / 2];
    }
    if (all_v || tid < VQ) {
      const int pos0 = j0 + qv_c16 * 16;
      r.v = *reinterpret_cast<const uint4*>(Vq + (int64_t)qv_d * n_ctx + pos0);
      const uint16_t* sd = Vd + (int64_t)(qv_d / QK) * n_ctx + pos0;
      r.vs0 = *reinterpret_cast<const uint4*>(sd);
      r.vs1 = *reinterpret_cast<const uint4*>(sd + 8);
    }
  };
  // Dequantisation into LDS: packed fp16, each value the correctly rounded fp16 of d*q.
  // V positions at or past kv_end are stored as zeros (their probabilities are zero; this
  // keeps whatever the cache holds there out of the product).  K rows there need no
  // care: their scores are masked to -inf.
  auto store_q8 = [&](const Q8Regs& r, int jt, uint4* kb, uint4* vb) __attribute__((always_inline)) {
    if (all_k || tid < KQ) {
      const int sw = qk_row % NCH;
      uint4 lo, hi;
      dequant16_f16(r.k, r.ks, lo, hi);
      kb[qk_row * NCH + ((2 * qk_c16) ^ sw)] = lo;
      kb[qk_row * NCH + ((2 * qk_c16 + 1) ^ sw)] = hi;
    }
    if (all_v || tid < VQ) {
      uint4 qv = r.v, s0 = r.vs0, s1 = r.vs1;
      const int nv = kv_end - (jt * KVT + qv_c16 * 16);   // valid positions of the chunk
      if (nv < 16) {
        auto keep = [&](int first, int per) -> uint32_t {   // mask of the valid lanes of a dword
          const int k = min(max(nv - first, 0), 32 / per);
          return k >= 32 / per ? 0xFFFFFFFFu : (1u << (per * k)) - 1u;
        };
        qv.x &= keep(0, 8); qv.y &= keep(4, 8); qv.z &= keep(8, 8); qv.w &= keep(12, 8);
        s0.x &= keep(0, 16); s0.y &= keep(2, 16); s0.z &= keep(4, 16); s0.w &= keep(6, 16);
        s1.x &= keep(8, 16); s1.y &= keep(10, 16); s1.z &= keep(12, 16); s1.w &= keep(14, 16);
      }
      const int sw = vswz(qv_d);
      uint4 lo, hi;
      dequant16_f16_scales(qv, s0, s1, lo, hi);
      vb[qv_d * 8 + ((2 * qv_c16) ^ sw)] = lo;
      vb[qv_d * 8 + ((2 * qv_c16 + 1) ^ sw)] = hi;
    }
  };

  const float scale = 1.4426950408889634f / sqrtf((float)HD);
  float m = -INFINITY, l = 0.0f;
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[db][e] = 0.0f;

  // ---- S^T = K Q^T of one tile (16 MFMAs).  The first product of each block takes a zero
  // accumulator operand (an inline constant), so no registers are cleared per tile.
  auto qk = [&](const uint4* kb, f32x16 (&s)[2]) __attribute__((always_inline)) {
    const f32x16 zero = {};
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
      const int row = jb * 32 + krow;
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        const int ch = kk * 2 + h;
        const uint4 av = kb[row * NCH + (ch ^ (row % NCH))];
        s[jb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, av),
                                                       __builtin_bit_cast(f16x8, qf[kk]),
                                                       kk == 0 ? zero : s[jb], 0, 0, 0);
      }
    }
  };
  // ---- causal mask (only tiles reaching past the wave's earliest query), the tile's row
  // maximum, and the lazy rescale of O and l; returns the offset the probabilities take.
  auto stats = [&](f32x16 (&s)[2], int j0) __attribute__((always_inline)) -> float {
    if (j0 + KVT - 1 > wave_qmin || !row_ok) {
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          // accumulator row 8*(e/4) + 4h + e%4 holds key (that row with bits 2, 3 swapped)
          const int j = j0 + jb * 32 + 16 * (e >> 3) + 8 * h + (e & 7);
          if (j > qpos || !row_ok) s[jb][e] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[jb][e]);
    {
      // The other lane half holds the same query row's other keys.  v_permlane32_swap
      // moves the lower half's values into the upper lanes of its first result and the
      // upper half's into the lower lanes of its second; each lane takes the one from the
      // other half (selecting, not max-ing, the two results: with equal inputs the
      // compiler treats them as equal values).
      const uint32_t b = __builtin_bit_cast(uint32_t, mx);
      const auto sw = __builtin_amdgcn_permlane32_swap(b, b, false, false);
      mx = fmaxf(mx, __builtin_bit_cast(float, h ? sw[0] : sw[1])) * scale;
    }
    if (__builtin_amdgcn_ballot_w64(mx > m + 8.0f)) {
      const float mnew = fmaxf(m, mx);
      const float alpha = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - mnew);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
      m = mnew;
    }
    return (m == -INFINITY) ? 0.0f : m;
  };
  // ---- probabilities p = 2^(s*scale - m) (every one below 2^8: safe in fp16), the fp16
  // B operands of O^T += V^T P^T (keys 16*ks + 8h .. +7 per lane), and the row sum of
  // those fp16 values (the weights the product applies), two per v_dot2 against (1, 1).
  auto probs = [&](f32x16 (&s)[2], float msafe, uint4 (&pb)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[jb][e] = __builtin_amdgcn_exp2f(fmaf(s[jb][e], scale, -msafe));
    const f16x2 one2 = {(_Float16)1.0f, (_Float16)1.0f};
    float ls = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int jb = ks >> 1, kk = ks & 1;
      pb[ks] = make_uint4(pack_f16x2(s[jb][8 * kk + 0], s[jb][8 * kk + 1]),
                          pack_f16x2(s[jb][8 * kk + 2], s[jb][8 * kk + 3]),
                          pack_f16x2(s[jb][8 * kk + 4], s[jb][8 * kk + 5]),
                          pack_f16x2(s[jb][8 * kk + 6], s[jb][8 * kk + 7]));
      const uint32_t w[4] = {pb[ks].x, pb[ks].y, pb[ks].z, pb[ks].w};
#pragma unroll
      for (int c = 0; c < 4; ++c) ls = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w[c]), one2, ls, false);
    }
    l += ls;                           // lane half; halves are combined at the end
  };
  // ---- O^T += V^T P^T (16 MFMAs)
  auto pv = [&](const uint4* vb, const uint4 (&pb)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int dd = db * 32 + l32, sw = vswz(dd);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        // keys 16*ks + 8h .. +7: one 16-byte chunk of the V^T row
        const uint4 av = vb[dd * 8 + ((2 * ks + h) ^ sw)];
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, av),
                                                       __builtin_bit_cast(f16x8, pb[ks]), o[db], 0, 0, 0);
      }
    }
  };
  // One whole tile, in order (the q8_0 path).
  auto compute = [&](const uint4* kb, const uint4* vb, int j0) __attribute__((always_inline)) {
    f32x16 s[2];
    uint4 pb[4];
    qk(kb, s);
    const float msafe = stats(s, j0);
    probs(s, msafe, pb);
    pv(vb, pb);
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  if (jt0 < jt1) {
    const int last = jt1 - 1;
    // Tile t lives in buffer (t - jt0) % NB.  The loops run in unrolled groups of steps;
    // loads past the range are clamped repeats of the last tile.  The f16 loop skips the
    // steps past the range whole; the q8_0 loop's last pair may run one step past it, which
    // waits, synchronises and issues like the others (every wave sees the same loads in
    // flight) but skips the arithmetic.
    if constexpr (!Q8) {
      // NB = 3, software-pipelined across tiles.  Step t waits for tile t+1 (the only loads
      // in flight), synchronises (every wave is done with tile t-1), and refills the buffer
      // of t-1 with tile t+2.  Then, after tile t's mask, maximum and rescale, the K Q^T
      // products of tile t+1 (issued unconditionally: past the range the clamped loads
      // keep the buffer valid, and the result is unused) interleave with tile t's
      // exponentials, so the MFMAs of one tile run under the softmax of the other; V^T P^T
      // of tile t follows.
      // Two score sets alternate between "this tile" and "the next" (P selects which holds
      // this tile), so no scores are copied: six steps cover both buffer and set cycles.
      f32x16 sa[2], sb[2];
      auto step = [&](auto J, auto P, int t) __attribute__((always_inline)) {
        constexpr int j = decltype(J)::value;
        f32x16 (&sc)[2] = decltype(P)::value ? sb : sa;
        f32x16 (&sn)[2] = decltype(P)::value ? sa : sb;
        attn_wait_vm_lgkm<0>();
        __builtin_amdgcn_s_barrier();
        attn_cfence();
        issue_f16(std::integral_constant<int, (j + 2) % 3>{}, min(t + 2, last));
        attn_cfence();
        if (t < jt1 && wave_rows) {
          uint4 pb[4];
          const float msafe = stats(sc, t * KVT);
          qk(bufK(std::integral_constant<int, (j + 1) % 3>{}), sn);
          probs(sc, msafe, pb);
          // three K fragment reads ahead, then {one MFMA of K Q^T, one VALU of the
          // softmax, the next fragment read} per MFMA (the rest of the softmax is scheduled
          // freely; five VALU per MFMA were 3-5% slower, none 1-2%)
          __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
            if (i < 13) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          pv(bufV(J), pb);
          // V^T P^T: three V fragment reads ahead, then {one MFMA, the next read}
          __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (i < 13) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
        }
      };
      using P0 = std::false_type;
      using P1 = std::true_type;
      issue_f16(I0{}, jt0);
      issue_f16(I1{}, min(jt0 + 1, last));
      attn_wait_vm_lgkm<NLOAD>();      // tile jt0 landed (own loads)
      __builtin_amdgcn_s_barrier();    // everyone's
      attn_cfence();
      if (wave_rows) qk(bufK(I0{}), sa);
      // (the steps past the range are skipped whole, by every wave alike: their waits and
      // barriers would only delay a short range, such as a decode-sized chunk's KV split)
      for (int t = jt0; t < jt1; t += 6) {
        step(I0{}, P0{}, t);
        if (t + 1 < jt1) step(I1{}, P1{}, t + 1);
        if (t + 2 < jt1) step(I2{}, P0{}, t + 2);
        if (t + 3 < jt1) step(I0{}, P1{}, t + 3);
        if (t + 4 < jt1) step(I1{}, P0{}, t + 4);
        if (t + 5 < jt1) step(I2{}, P1{}, t + 5);
      }
      attn_wait_vm0();
    } else {
      // NB = 2 LDS buffers and two register sets: tile t+2 is loaded to registers while tile
      // t is computed, and tile t+1 (loaded one step earlier) is dequantised into the other
      // buffer after it, so a tile's loads have two tiles' arithmetic to land.  Every step
      // issues the same loads and stores (past the range they repeat the last tile, and
      // only the arithmetic is skipped), so the compiler's load-count waits stay exact; the
      // barrier waits only for this wave's LDS writes, not for the loads in flight.
      auto barrier = [&]() __attribute__((always_inline)) {
        attn_cfence();
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        attn_cfence();
      };
      const int t0 = __builtin_amdgcn_readfirstlane(jt0);
      const int tl = __builtin_amdgcn_readfirstlane(last);
      const int npairs = __builtin_amdgcn_readfirstlane((jt1 - jt0 + 1) / 2);
      Q8Regs ra, rb;
      load_q8(t0, ra);
      load_q8(min(t0 + 1, tl), rb);
      store_q8(ra, t0, sK0, sV0);
      attn_wait_vm0();                 // (the Q fragments too: nothing older is in flight)
      for (int pr = 0; pr < npairs; ++pr) {
        const int t = t0 + 2 * pr;
        barrier();                     // tile t in buffer 0; buffer 1 is free
        load_q8(min(t + 2, tl), ra);
        if (wave_rows) compute(sK0, sV0, t * KVT);
        store_q8(rb, min(t + 1, tl), sK1, sV1);
        barrier();                     // tile t+1 in buffer 1; buffer 0 is free
        load_q8(min(t + 3, tl), rb);
        if (t + 1 <= tl && wave_rows) compute(sK1, sV1, (t + 1) * KVT);
        store_q8(ra, min(t + 2, tl), sK0, sV0);
      }
      attn_wait_vm0();
    }
  }
  l += __shfl_xor(l, 32, 64);          // per-lane partial sums -> row sum

  if (!row_ok) return;
  if (a.splits == 1) {
    const float inv_l = 1.0f / l;
    _Float16* orow = a.out + ((int64_t)t_i * a.n_head + hq) * HD;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = db * 32 + 8 * rq + 4 * h;
        const uint2 pk = make_uint2(pack_f16x2(o[db][4 * rq] * inv_l, o[db][4 * rq + 1] * inv_l),
                                    pack_f16x2(o[db][4 * rq + 2] * inv_l, o[db][4 * rq + 3] * inv_l));
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
// A row's hd/4 column quads times SL "split lanes" share the work: split lane j takes the
// splits j, j+SL, ..., so the partial loads of one row are in flight together; the lanes'
// maxima, weights and sums meet in LDS and are added in lane order (a fixed order).  SL
// grows (up to 8, and not past the split count) only while rows x quads alone would leave
// the chip short of threads, as with decode-sized chunks.
__host__ __device__ constexpr int combine_split_lanes(int splits, int64_t row_quads) {
  int sl = 1;
  while (sl < 8 && sl < splits && row_quads * sl < (int64_t(1) << 18)) sl *= 2;
  return sl;
}

__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  __shared__ float red[5][256];
  const int G = a.n_head / a.n_kv_head;
  const int64_t R = (int64_t)a.n * G;
  const int64_t rows_total = (int64_t)a.n_kv_head * R;
  const int hd = a.head_dim;
  const int Q = hd / 4;
  const int SL = combine_split_lanes(a.splits, rows_total * Q);
  const int per_row = Q * SL;
  const int tid = threadIdx.x;
  const int rl = tid / per_row, sl = (tid % per_row) / Q, q = tid % Q;
  const int64_t rg = (int64_t)blockIdx.x * (256 / per_row) + rl;
  const bool live = rl < 256 / per_row && rg < rows_total;
  const int d0 = q * 4;
  float m = -INFINITY;
  if (live) {
#pragma unroll 4
    for (int s = sl; s < a.splits; s += SL) m = fmaxf(m, a.part_ml[((int64_t)s * rows_total + rg) * 2]);
  }
  red[0][tid] = m;
  __syncthreads();
  float mstar = -INFINITY;
  const int base = rl * per_row + q;
  if (live)
    for (int j = 0; j < SL; ++j) mstar = fmaxf(mstar, red[0][base + j * Q]);
  float den = 0.0f;
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
  if (live) {
    // A split without keys for this row left m = -inf, l = 0 and O = 0: its weight is
    // exp2(-inf) = 0 and it adds exact zeros, so no branch holds back the loads.
#pragma unroll 4
    for (int s = sl; s < a.splits; s += SL) {
      const float2 ml = *reinterpret_cast<const float2*>(a.part_ml + ((int64_t)s * rows_total + rg) * 2);
      const float4 po = *reinterpret_cast<const float4*>(a.part_o + ((int64_t)s * rows_total + rg) * hd + d0);
      const float w = __builtin_amdgcn_exp2f(ml.x - mstar);
      den += w * ml.y;
      num.x += w * po.x; num.y += w * po.y; num.z += w * po.z; num.w += w * po.w;
    }
  }
  __syncthreads();
  red[0][tid] = den;
  red[1][tid] = num.x; red[2][tid] = num.y; red[3][tid] = num.z; red[4][tid] = num.w;
  __syncthreads();
  if (!live || sl != 0) return;
  for (int j = 1; j < SL; ++j) {
    const int o = base + j * Q;
    den += red[0][o];
    num.x += red[1][o]; num.y += red[2][o]; num.z += red[3][o]; num.w += red[4][o];
  }
  const float inv = 1.0f / den;
  const int64_t g = rg / R, i = rg % R;
  const int64_t t = i / G, hq = g * G + i % G;
  _Float16* orow = a.out + (t * a.n_head + hq) * hd + d0;
  *reinterpret_cast<uint2*>(orow) = make_uint2(pack_f16x2(num.x * inv, num.y * inv),
                                              pack_f16x2(num.z * inv, num.w * inv));
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  const int G = a.n_head / a.n_kv_head;
  const int R = a.n * G;
  dim3 grid((unsigned)(((R + QROWS - 1) / QROWS) * a.n_kv_head * a.splits));
  const bool q8 = a.kv_type != CP_KV_F16;
  if (a.head_dim == 128) {
    if (q8) hipLaunchKernelGGL((attn_kernel<128, true>), grid, dim3(AW * 64), 0, s, a);
    else hipLaunchKernelGGL((attn_kernel<128, false>), grid, dim3(AW * 64), 0, s, a);
  } else {
    if (q8) hipLaunchKernelGGL((attn_kernel<64, true>), grid, dim3(AW * 64), 0, s, a);
    else hipLaunchKernelGGL((attn_kernel<64, false>), grid, dim3(AW * 64), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits <= 1) return e;
  const int64_t rows_total = (int64_t)a.n_kv_head * R;
  const int rows_per_wg = 256 / (a.head_dim / 4 * combine_split_lanes(a.splits, rows_total * (a.head_dim / 4)));
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)ceil_div(rows_total, rows_per_wg)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace cp
