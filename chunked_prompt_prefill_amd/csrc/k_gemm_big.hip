// q8_0-weight GEMM on fp16 MFMA (gfx950) for 256-row tiles, fp32 accumulate.
//
//   out[m][n] = sum_k A[m][k] * W[n][k],  A fp16 activations, W q8_0 blocks of 32.
//
// One workgroup of 4 waves per CU owns a 256 x 256 output tile; each wave owns 64 columns
// (two 32-column MFMA blocks) over all 256 rows, i.e. 256 fp32 accumulators per lane in
// the AGPRs.  A weight is dequantised once per workgroup and feeds 256 rows, so the
// dequantisation (per two weights: a byte permute that makes them exact fp16 integers, a
// packed add and a packed multiply by the fp16 block scale, correctly rounded) hides
// under the MFMA issue time.
//
// Every operand travels global -> LDS by asynchronous loads (no register staging), in
// 64-wide K stages (two q8_0 blocks) through three LDS buffers:
//   * A: 256 x 64 fp16 (32 KiB), the eight 16-byte chunks of a row XOR-swizzled by the
//     row so that the 16 rows a 16-byte LDS read serves per pass hit distinct banks
//     (the swizzle is chosen through each lane's source address);
//   * W: each wave's 64 columns x 64 K int8 (4 KiB) in the repacked lane order, and their
//     fp16 scales (256 bytes).
// The loads of stage s+2 are issued while stage s computes.  A stage waits with an exact
// vmcnt for its own loads, then a bare barrier makes every wave's part of the A tile
// visible (the wait already covers the asynchronous LDS writes; every LDS read of the
// stage before has been consumed by its MFMA).  The three buffers are separate LDS
// objects so the compiler can tell reads of one stage from DMA writes into another.
//
// Within a stage the B operand of block 1 is dequantised while the MFMAs of block 0 run,
// and block 0 of the next stage while those of block 1 run (its weights and scales are
// loaded first in every stage, so a partial vmcnt wait suffices).
//
// The K index inside a q8_0 block is permuted consistently on both operands so that a
// lane's 16 weight bytes are contiguous: lane half h, MFMA step s, element c <-> block
// column 16h + 8s + c.  Rows beyond M and columns beyond N are computed from clamped
// (valid) addresses and not stored.  Epilogues as in the smaller-tile kernel: fp32 store,
// fp32 residual add, SwiGLU to fp16, or split-K partials.
#include <type_traits>
#include <utility>

#include "cp_internal.h"
#include "k_common.h"

namespace cp {
namespace {

constexpr int BK = 64;               // K per stage
constexpr int BCPR = BK * 2 / 16;    // 16-byte A chunks per row per stage
constexpr int BMT = 256, BNT = 256;
constexpr int BNCH = BMT * BCPR;     // A chunks per stage
constexpr int BJPW = BNCH / 256;     // A loads per thread per stage
constexpr int BNLOAD = 4 + 2 + BJPW; // loads per thread per stage: W (4), scales (2), A
constexpr int NBUFA = 4;             // pipeline depth: stages in flight

typedef __attribute__((address_space(3))) void lptr_t;
typedef unsigned int u32x4_v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4_v u32x4_g;

// s_waitcnt vmcnt(N), no wait on the other counters (gfx9 encoding).
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// s_waitcnt vmcnt(N) lgkmcnt(0): also every LDS read of this wave has returned.
template <int N>
__device__ __forceinline__ void vm_lgkm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070);
}

// 16 and 4 bytes through a buffer descriptor (per-lane offset, uniform offset).
__device__ __forceinline__ u32x4_v buf_load16(__amdgpu_buffer_rsrc_t r, int32_t voff, int32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, int32_t voff, int32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

// Compiler-only fence: memory operations are not moved across it, so the loads a stage
// issues are counted where the vmcnt waits assume them.
__device__ __forceinline__ void cfence() { __atomic_signal_fence(__ATOMIC_SEQ_CST); }

template <typename F, int... I>
__device__ __forceinline__ void sfor_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>()), ...);
}
// f(integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time.
template <int N, typename F>
__device__ __forceinline__ void sfor(F&& f) {
  sfor_impl(f, std::make_integer_sequence<int, N>());
}

template <int MODE, bool GROUPED>
__global__ __launch_bounds__(256, 1) void gemm_q8_big_kernel(GemmArgs g) {
  __shared__ uint4 sA0[BNCH], sA1[BNCH], sA2[BNCH], sA3[BNCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int KS = g.K / BK;

  int m0, rows, split, ntile, expert = 0;
  const int ntiles = (int)ceil_div(g.N - g.n0, BNT);
  if constexpr (GROUPED) {
    // Routed experts: row tiles come from the device tile table {expert, m0, m1}, whose
    // length is known only on the device; the grid covers the table's capacity.  The
    // valid (tile, column tile) pairs, column tile fastest, are dealt to the eight XCDs in
    // contiguous ranges (so a row tile's A rows stay in one L2), and the rest exit.
    const int valid = *g.n_tiles * ntiles;
    const int per_xcd = (valid + 7) >> 3;
    const int i = blockIdx.x;
    const int xcd = i & 7, idx = i >> 3;
    const int logical = xcd * per_xcd + idx;
    if (idx >= per_xcd || logical >= valid) return;
    const int4 tile = reinterpret_cast<const int4*>(g.tiles)[logical / ntiles];
    expert = tile.x;
    m0 = tile.y;
    rows = tile.z - tile.y;
    ntile = logical % ntiles;
    split = 0;
  } else {
    // Tile order.  Workgroup i runs on XCD i % 8 and each XCD gets a contiguous range of
    // logical tiles, so the ~32 workgroups an XCD runs at once are consecutive logical
    // tiles.  Those are laid out in groups of up to 8 row tiles: 32 consecutive tiles form
    // an 8 x 4 block (rows x columns) that shares 8 A row panels and 4 weight column
    // panels in the XCD's L2, instead of 32 A panels for one weight panel.
    const int mtiles = (int)ceil_div(g.M, BMT);
    const int per_split = mtiles * ntiles;
    const int total = per_split * g.splits;
    const int i = blockIdx.x;
    const int xcd = i & 7, idx = i >> 3;
    const int q8 = total >> 3, r8 = total & 7;
    const int logical = (xcd < r8) ? xcd * (q8 + 1) + idx : r8 * (q8 + 1) + (xcd - r8) * q8 + idx;
    split = logical / per_split;
    const int lt = logical % per_split;
    constexpr int GM = 8;
    const int group = lt / (GM * ntiles);
    const int first_m = group * GM;
    const int gm = min(GM, mtiles - first_m);
    const int within = lt - group * GM * ntiles;
    const int mt = first_m + within % gm;
    ntile = within / gm;
    m0 = mt * BMT;
    rows = min(BMT, g.M - m0);
  }

  const int ks0 = (int)((int64_t)split * KS / g.splits);
  const int ks1 = (int)((int64_t)(split + 1) * KS / g.splits);
  const int n_wave = g.n0 + ntile * BNT + wave * 64;
  const bool col_ok0 = n_wave < g.N;
  const bool col_ok1 = n_wave + 32 < g.N;

  // A: load j of wave w fills physical chunks [(4j + w)*64, +64) of a stage; lane L lands
  // on row r = 32j + 8w + L/8, physical chunk L%8, which holds logical chunk
  // (L%8) ^ swz(r), swz(r) = (r/2) % 8 = (4w + L/16) % 8.  A 16-byte LDS read is served
  // 16 lanes at a time (256 bytes over the 64 banks); rows r and r+1 sit in the two halves
  // of a 256-byte bank line, so swz must differ over every 8 consecutive even (or odd)
  // rows: the 16 rows of one pass then hit 16 distinct 16-byte bank groups.
  // The loads are buffer loads to LDS (a buffer descriptor over A, bounds-checked): unlike
  // the global form they are not counted as LDS events, so the LDS reads of the current
  // stage keep exact, partial lgkmcnt waits while the next stages' tiles are in flight.
  const int rsub = 8 * wave + (lane >> 3);
  const int lchunk = (lane & 7) ^ ((4 * wave + (lane >> 4)) & 7);
  const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)g.A, (short)0, (int)min((int64_t)g.M * g.lda * 2, (int64_t)0x7FFFFFFF), 0x00020000);
  int32_t aoff[BJPW];   // byte offset of each lane's 16-byte chunk at K stage 0
#pragma unroll
  for (int j = 0; j < BJPW; ++j) {
    int32_t pr = m0 + min(32 * j + rsub, rows - 1);
    if (GROUPED && g.a_rows) pr = g.a_rows[pr] / g.a_row_div;   // gathered A rows
    aoff[j] = (pr * g.lda + lchunk * 8) * 2;
  }

  const int KB = g.K / QK, KQ = g.K / 128;
  const int last32 = g.N / 32 - 1;
  // W and its scales through buffer descriptors (uniform base and size), with one
  // per-lane 32-bit offset each; the second column block and the stage are uniform
  // offsets.  Column blocks past N re-read the last one (not stored).
  const int n32_0 = min(n_wave >> 5, last32), n32_1 = min((n_wave >> 5) + 1, last32);
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.wq + expert * g.wq_estride), (short)0, (int)min((int64_t)g.N * g.K, (int64_t)0x7FFFFFFF), 0x00020000);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.wd + expert * g.wd_estride), (short)0, (int)min((int64_t)g.N * g.K / 16, (int64_t)0x7FFFFFFF),
      0x00020000);
  const int32_t woff = n32_0 * KB * 1024 + lane * 16;   // 1 KiB per (32 columns, q8_0 block)
  // scales: four fp16 per row per 128 columns; a stage takes one 32-bit pair
  const int32_t soff = (n32_0 * KQ * 32 + l32) * 8;
  const int32_t wdelta = (n32_1 - n32_0) * KB * 1024, sdelta = (n32_1 - n32_0) * KQ * 256;
  auto bufA = [&](auto J) __attribute__((always_inline)) -> uint4* {
    if constexpr (decltype(J)::value == 0) return sA0;
    else if constexpr (decltype(J)::value == 1) return sA1;
    else if constexpr (decltype(J)::value == 2) return sA2;
    else return sA3;
  };

  // Raw W bytes and scales of one stage, in registers.
  struct Raw { uint4 q[2][2]; uint32_t sc[2]; };
  // The loads of stage ks, as BNLOAD pieces issued one per MFMA slot (a burst of vector
  // memory instructions would stall the wave's in-order issue): this wave's W blocks and
  // scales (into registers, which the compiler tracks itself), then the A tile
  // (asynchronously into LDS buffer J).
  auto issue_piece = [&](auto J, auto P, int ks, Raw& w) __attribute__((always_inline)) {
    constexpr int p = decltype(P)::value;
    if constexpr (p < 4) {
      constexpr int ni = p / 2, kb = p % 2;
      const u32x4_v v = buf_load16(wrs, woff, (ni ? wdelta : 0) + (2 * ks + kb) * 1024);
      w.q[ni][kb] = make_uint4(v.x, v.y, v.z, v.w);
    } else if constexpr (p < 6) {
      constexpr int ni = p - 4;
      w.sc[ni] = buf_load4(srs, soff, (ni ? sdelta : 0) + ((ks >> 1) * 64 + (ks & 1)) * 4);
    } else {
      constexpr int j = p - 6;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(arsrc, (lptr_t*)&bufA(J)[(4 * j + wave) * 64], 16, aoff[j],
                                               ks * BK * 2, 0, 0);
    }
  };
  auto issue = [&](auto J, int ks, Raw& w) __attribute__((always_inline)) {
    sfor<BNLOAD>([&](auto P) __attribute__((always_inline)) { issue_piece(J, P, ks, w); });
  };

  f32x16 acc[8][2];
#pragma unroll
  for (int mi = 0; mi < 8; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mi][ni][e] = 0.0f;

  // Dequantised B of one block: dq[ni][s] = the 8 fp16 that MFMA step s of column block
  // ni takes.  Two sets alternate: one block's MFMAs read one set while the VALU fills the
  // other for the next block.
  typedef uint4 Deq[2][2];
  Deq dq0, dq1;

  // Half-piece p (0..15) of dequantising a block: column block ni = p/8, byte pair
  // (p%8) of the 16 bytes -> two fp16 (one dword of dq[ni][p%8/4]).  valid == false (a
  // padding stage) uses scale 0: the block's B is exactly zero.
  f16x2 dsc[2];
  uint32_t xq[2];
  auto deq_piece = [&](auto P, int kb, const Raw& w, bool valid, Deq& dq) __attribute__((always_inline)) {
    constexpr int p = decltype(P)::value;
    constexpr int ni = p / 8, pp = p % 8, dw = pp / 2, hf = pp % 2;
    if constexpr (pp == 0) {
      const uint32_t bits = valid ? (kb ? (w.sc[ni] >> 16) : (w.sc[ni] & 0xFFFFu)) : 0u;
      const _Float16 d = __builtin_bit_cast(_Float16, (uint16_t)bits);
      dsc[ni] = f16x2{d, d};
    }
    if constexpr (hf == 0) {
      const uint4 q = w.q[ni][kb];
      xq[ni] = (dw == 0 ? q.x : dw == 1 ? q.y : dw == 2 ? q.z : q.w) ^ 0x80808080u;
    }
    const uint32_t packed =
        __builtin_bit_cast(uint32_t, q8_pair_f16(xq[ni], hf ? 0x04030402u : 0x04010400u) * dsc[ni]);
    uint4& o = dq[ni][dw >> 1];
    const int comp = (dw & 1) * 2 + hf;
    if (comp == 0) o.x = packed;
    else if (comp == 1) o.y = packed;
    else if (comp == 2) o.z = packed;
    else o.w = packed;
  };

  // A fragment of slot t of block kb (step s = t/8, row block mi = t%8).
  auto frag = [&](auto J, int kb, int t) __attribute__((always_inline)) -> uint4 {
    const uint4* sA = bufA(J);
    const int c = kb * 4 + 2 * h + t / 8;
    return sA[((t % 8) * 32 + l32) * BCPR + (c ^ ((l32 >> 1) & 7))];
  };

  // One block of a stage in A buffer J: 16 slots, each {MFMA pair, the A fragment read
  // three slots ahead, a dequantisation half-piece of the next block}, in a fixed order
  // (sched_barrier).  af holds fragments t..t+2 on entry; with NEXTA the last slots
  // prefetch the first three fragments of block kb+1 of the same buffer.
  uint4 af[4];
  auto block = [&](auto J, auto KB, auto NEXTA, const Deq& dq, auto DEQ, const Raw& w, int wkb,
                   bool valid, Deq& dqn, auto ISS, auto JI, int iks, Raw& wi) __attribute__((always_inline)) {
    constexpr int kb = decltype(KB)::value;
    sfor<16>([&](auto T) __attribute__((always_inline)) {
      constexpr int t = decltype(T)::value;
      if constexpr (decltype(ISS)::value && t < BNLOAD) issue_piece(JI, T, iks, wi);
      constexpr int mi = t % 8, st = t / 8;
      const f16x8 av = __builtin_bit_cast(f16x8, af[t % 4]);
      const f16x8 b0 = __builtin_bit_cast(f16x8, dq[0][st]), b1 = __builtin_bit_cast(f16x8, dq[1][st]);
      if constexpr (MODE == GM_SWIGLU) {   // transposed tile (see the epilogue)
        acc[mi][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b0, av, acc[mi][0], 0, 0, 0);
        acc[mi][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b1, av, acc[mi][1], 0, 0, 0);
      } else {
        acc[mi][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, b0, acc[mi][0], 0, 0, 0);
        acc[mi][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, b1, acc[mi][1], 0, 0, 0);
      }
      if constexpr (t + 3 < 16) af[(t + 3) % 4] = frag(J, kb, t + 3);
      else if constexpr (decltype(NEXTA)::value) af[(t + 3) % 4] = frag(J, kb + 1, t + 3 - 16);
      else af[(t + 3) % 4] = frag(std::integral_constant<int, (decltype(J)::value + 1) % NBUFA>(), 0, t + 3 - 16);
      if constexpr (decltype(DEQ)::value) {
        // the raw bytes were read at the start of the block: pieces from slot 2 on
        if constexpr (t == 2) {
          deq_piece(std::integral_constant<int, 0>(), wkb, w, valid, dqn);
          deq_piece(std::integral_constant<int, 1>(), wkb, w, valid, dqn);
        } else if constexpr (t == 3) {
          deq_piece(std::integral_constant<int, 2>(), wkb, w, valid, dqn);
          deq_piece(std::integral_constant<int, 3>(), wkb, w, valid, dqn);
        } else if constexpr (t >= 4) {
          deq_piece(std::integral_constant<int, t>(), wkb, w, valid, dqn);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;

  if (ks0 < ks1) {
    const int S = ks1 - ks0;
    const int last = ks1 - 1;
    // Stages past the end re-load the last stage into a buffer nobody reads again, so that
    // every step issues the same number of loads and every wait count is exact.
    Raw w0, w1, w2, w3;
    issue(I0(), ks0, w0);
    issue(I1(), min(ks0 + 1, last), w1);
    issue(I2(), min(ks0 + 2, last), w2);
    cfence();
    vm_lgkm_wait<2 * BNLOAD>();
    __builtin_amdgcn_s_barrier();
    cfence();
    af[0] = frag(I0(), 0, 0);
    af[1] = frag(I0(), 0, 1);
    af[2] = frag(I0(), 0, 2);
    sfor<16>([&](auto P) __attribute__((always_inline)) { deq_piece(P, 0, w0, true, dq0); });
    // One stage r in buffer J (raw W in wc).  Its tile is already complete and its first
    // A fragments are in registers: the wait and barrier at the top make the NEXT stage's
    // tile complete and visible (so the last slots can prefetch its first fragments, and
    // no stage starts with an LDS round trip), and free the buffer of stage r-1, which the
    // block-0 slots refill with stage r+3 (A tile and raw registers wi).  Block 0 runs
    // while block 1 is dequantised, block 1 while block 0 of the next stage is (raw
    // registers wn; the compiler waits for exactly those loads).
    using T = std::true_type;
    using F = std::false_type;
    auto step = [&](auto J, int r, const Raw& wc, const Raw& wn, Raw& wi) __attribute__((always_inline)) {
      constexpr int j = decltype(J)::value;
      cfence();
      vm_lgkm_wait<BNLOAD>();
      __builtin_amdgcn_s_barrier();
      cfence();
      using JI = std::integral_constant<int, (j + 3) % NBUFA>;
      const int iks = min(ks0 + r + 3, last);
      block(J, I0(), T(), dq0, T(), wc, 1, r < S, dq1, T(), JI(), iks, wi);
      block(J, I1(), F(), dq1, T(), wn, 0, r + 1 < S, dq0, F(), JI(), iks, wi);
      cfence();
    };
    // The stage count is padded to a multiple of four with zero-weight stages (clamped
    // re-loads, B = 0), so the loop body is four identical steps with a single exit:
    // separate tail code or early exits make the register allocator shuffle the 256
    // accumulators.
    for (int r = 0; r < S; r += 4) {
      step(I0(), r, w0, w1, w3);
      step(I1(), r + 1, w1, w2, w0);
      step(I2(), r + 2, w2, w3, w1);
      step(I3(), r + 3, w3, w0, w2);
    }
    // Re-loads past the end may still be landing in LDS: drain them before the workgroup
    // can finish and release its LDS.
    vm_wait<0>();
  }

  // Epilogue.  acc[mi][ni][e]: row mi*32 + 8*(e/4) + 4*h + e%4, column n_wave + 32*ni + l32.
  // A lane's rows are 4h plus constants, so each store address is a per-lane base plus a
  // constant times the (uniform) row stride; whole tiles skip the row check.  The SwiGLU
  // tile is held transposed instead (weights as the MFMA's first operand): acc[mi][ni][e]
  // is row mi*32 + l32, column n_wave + 32*ni + 8*(e/4) + 4h + e%4, so a lane's four
  // consecutive outputs of group e/4 leave in one 8-byte store (a quarter of the store
  // instructions; the fp32 epilogues keep the row-contiguous form, whose stores fill
  // whole 128-byte lines).
  const int pn = g.N - g.n0;
  const bool full = rows >= BMT;
  auto each = [&](auto&& st) __attribute__((always_inline)) {
#pragma unroll
    for (int mi = 0; mi < 8; ++mi)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int rc = mi * 32 + 8 * (e >> 2) + (e & 3);   // row minus 4h
        if (full || rc + 4 * h < rows) st(mi, e, rc);
      }
  };
  if constexpr (MODE == GM_SWIGLU) {
    if (col_ok0) {
      _Float16* ob = reinterpret_cast<_Float16*>(g.out) + (m0 + l32) * (int64_t)g.ldo + (n_wave >> 1) + 4 * h;
#pragma unroll
      for (int mi = 0; mi < 8; ++mi)
        if (full || mi * 32 + l32 < rows) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            f16x4 v;
#pragma unroll
            for (int c = 0; c < 4; ++c) v[c] = f16_sat(silu(acc[mi][0][4 * q + c]) * acc[mi][1][4 * q + c]);
            *reinterpret_cast<f16x4*>(ob + (int64_t)(mi * 32) * g.ldo + 8 * q) = v;
          }
        }
    }
  } else if constexpr (MODE == GM_PARTIAL) {
    float* pb = g.partial + ((int64_t)split * g.M + m0 + 4 * h) * pn + (n_wave - g.n0) + l32;
    each([&](int mi, int e, int rc) {
      if (col_ok0) pb[(int64_t)rc * pn] = acc[mi][0][e];
      if (col_ok1) pb[(int64_t)rc * pn + 32] = acc[mi][1][e];
    });
  } else {
    float* ob = reinterpret_cast<float*>(g.out) + (m0 + 4 * h) * (int64_t)g.ldo + n_wave + l32;
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

}  // namespace

hipError_t launch_gemm_big(const GemmArgs& a, int grid_m_tiles, hipStream_t s) {
  if (a.M <= 0 || a.N <= a.n0) return hipSuccess;
  if (a.tiles) {
    // grouped: one workgroup per (tile table capacity x column tile), unsplit, rounded up
    // to a multiple of 8 so that every XCD's range of the valid pairs is covered
    const unsigned grid = (unsigned)(ceil_div((int64_t)grid_m_tiles * ceil_div(a.N - a.n0, BNT), 8) * 8);
    switch (a.mode) {
      case GM_F32: hipLaunchKernelGGL((gemm_q8_big_kernel<GM_F32, true>), dim3(grid), dim3(256), 0, s, a); break;
      case GM_F32_ADD: hipLaunchKernelGGL((gemm_q8_big_kernel<GM_F32_ADD, true>), dim3(grid), dim3(256), 0, s, a); break;
      default: hipLaunchKernelGGL((gemm_q8_big_kernel<GM_SWIGLU, true>), dim3(grid), dim3(256), 0, s, a); break;
    }
    return hipGetLastError();
  }
  const unsigned grid = (unsigned)(ceil_div(a.M, BMT) * ceil_div(a.N - a.n0, BNT) * a.splits);
  const int mode = a.splits > 1 ? GM_PARTIAL : a.mode;
  switch (mode) {
    case GM_F32: hipLaunchKernelGGL((gemm_q8_big_kernel<GM_F32, false>), dim3(grid), dim3(256), 0, s, a); break;
    case GM_F32_ADD: hipLaunchKernelGGL((gemm_q8_big_kernel<GM_F32_ADD, false>), dim3(grid), dim3(256), 0, s, a); break;
    case GM_SWIGLU: hipLaunchKernelGGL((gemm_q8_big_kernel<GM_SWIGLU, false>), dim3(grid), dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((gemm_q8_big_kernel<GM_PARTIAL, false>), dim3(grid), dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace cp
