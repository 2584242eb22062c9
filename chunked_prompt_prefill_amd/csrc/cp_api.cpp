// Host runtime and C ABI of the chunked prefill library.
//
// A context holds pointers into three caller-owned device arenas (repacked weights, KV
// cache, workspace), the caller's stream and n_past.  prefill_chunk() validates on the
// host, then enqueues, per layer: RMSNorm -> QKV GEMM -> RoPE + K append -> V append
// -> attention -> O GEMM (+residual) -> RMSNorm -> SwiGLU FFN (dense, or router ->
// permute -> grouped GEMMs -> unpermute) (+residual).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "cp_internal.h"

using namespace cp;

namespace {

// --------------------------------------------------------------------------------------
// Geometry
// --------------------------------------------------------------------------------------
struct Dims {
  int L, d, Hq, Hkv, hd, G, F, E, k, Fe;
  int Nqkv, Dq, Fp, Fep;
  int n_ctx, Cm;
  bool moe;
  int kv_type;
};

int64_t round_up(int64_t v, int64_t g) { return (v + g - 1) / g * g; }

// Most chunks prefill_chunks keeps in flight (one stream and one workspace each).
constexpr int kMaxLanes = 8;

// Size of the static scratch array that prefill_chunk_static takes a chunk's buffers from.
constexpr size_t kStaticScratchBytes = (size_t)256 << 20;

std::string validate(const cp_config* c) {
  if (!c) return "config is NULL";
  if (c->n_layer < 1) return "n_layer must be >= 1";
  if (c->d_model < 128 || c->d_model % 128) return "d_model must be a positive multiple of 128";
  if (c->head_dim != 64 && c->head_dim != 128) return "head_dim must be 64 or 128";
  if (c->n_kv_head < 1 || c->n_head < 1 || c->n_head % c->n_kv_head)
    return "n_head must be a positive multiple of n_kv_head";
  if ((c->n_head * c->head_dim) % 128) return "n_head * head_dim must be a multiple of 128";
  if (c->n_head / c->n_kv_head > 64) return "n_head / n_kv_head must be <= 64";
  const bool moe = c->n_expert > 0;
  if (!moe && c->ffn_dim < 1) return "dense FFN needs ffn_dim >= 1";
  if (moe) {
    if (c->ffn_dim != 0) return "routed experts need ffn_dim == 0";
    if (c->n_expert > 256) return "n_expert must be <= 256";
    if (c->n_expert_used < 1 || c->n_expert_used > c->n_expert || c->n_expert_used > 16)
      return "n_expert_used must be in [1, min(n_expert, 16)]";
    if (c->expert_ffn_dim < 1) return "expert_ffn_dim must be >= 1";
  } else if (c->n_expert_used || c->expert_ffn_dim) {
    return "dense FFN needs n_expert_used == expert_ffn_dim == 0";
  }
  if (!(c->rms_eps > 0.0f) || !std::isfinite(c->rms_eps)) return "rms_eps must be > 0";
  if (!(c->rope_theta > 0.0f) || !std::isfinite(c->rope_theta)) return "rope_theta must be > 0";
  if (c->kv_type != CP_KV_F16 && c->kv_type != CP_KV_Q8_0) return "kv_type must be 0 (f16) or 1 (q8_0)";
  if (c->n_ctx_max < 1 || c->n_ctx_max > (1 << 24)) return "n_ctx_max must be in [1, 2^24]";
  // attention addresses one kv head's cache (n_ctx x head_dim f16) with 32-bit byte offsets
  if ((int64_t)(c->n_ctx_max + 63) * c->head_dim * 2 >= (1LL << 31)) return "n_ctx_max * head_dim too large";
  if (c->n_chunk_max < 1 || c->n_chunk_max > c->n_ctx_max) return "n_chunk_max must be in [1, n_ctx_max]";
  if ((int64_t)c->n_chunk_max * c->n_head * c->head_dim > (1LL << 31)) return "n_chunk_max too large";
  // The GEMMs address their fp16 A operand (n_chunk_max rows of the normed input, the
  // attention output, the FFN intermediate, or the routed slots' intermediate) with 32-bit
  // byte offsets from the buffer's base, so the largest such operand stays below 2 GiB.
  {
    const int64_t Fp = round_up(c->ffn_dim, 128), Fep = round_up(c->expert_ffn_dim, 128);
    const int64_t widest = std::max<int64_t>({(int64_t)c->d_model, (int64_t)c->n_head * c->head_dim, Fp});
    const int64_t a_bytes = std::max<int64_t>((int64_t)c->n_chunk_max * widest * 2,
                                              moe ? (int64_t)c->n_chunk_max * c->n_expert_used * Fep * 2 : 0);
    if (a_bytes >= (1LL << 31))
      return "n_chunk_max rows of the widest fp16 GEMM operand must stay below 2 GiB";
    // The 256-row GEMM kernel addresses a weight matrix's int8 values (N x K bytes) with
    // 32-bit byte offsets from the matrix's base.
    const int64_t d = c->d_model, Dq = (int64_t)c->n_head * c->head_dim;
    const int64_t Nqkv = (int64_t)(c->n_head + 2 * c->n_kv_head) * c->head_dim;
    const int64_t w_bytes = std::max<int64_t>({Nqkv * d, d * Dq, 2 * Fp * d, moe ? 2 * Fep * d : 0});
    if (w_bytes >= (1LL << 31)) return "each weight matrix must stay below 2^31 int8 values";
  }
  return "";
}

// The checks prefill_chunk makes before enqueuing anything: pointers, their 16-byte
// alignment (the row kernels move x in float4 units), and the chunk's bounds.
int chunk_check(const cp_config* c, int64_t n_past, const float* x_in, const float* x_out, int32_t n,
                std::string& err) {
  if (!x_in || !x_out) { err = "x_in / x_out is NULL"; return CP_E_INVALID; }
  if ((uintptr_t)x_in % 16 || (uintptr_t)x_out % 16) { err = "x_in / x_out must be 16-byte aligned"; return CP_E_INVALID; }
  if (n < 1 || n > c->n_chunk_max) { err = "n_tokens outside [1, n_chunk_max]"; return CP_E_CAPACITY; }
  if (n_past + n > c->n_ctx_max) { err = "n_past + n_tokens > n_ctx_max"; return CP_E_CAPACITY; }
  return CP_OK;
}

Dims dims_of(const cp_config* c) {
  Dims D;
  D.L = c->n_layer; D.d = c->d_model; D.Hq = c->n_head; D.Hkv = c->n_kv_head; D.hd = c->head_dim;
  D.G = D.Hq / D.Hkv; D.F = c->ffn_dim; D.E = c->n_expert; D.k = c->n_expert_used;
  D.Fe = c->expert_ffn_dim; D.moe = D.E > 0; D.kv_type = c->kv_type;
  D.Nqkv = (D.Hq + 2 * D.Hkv) * D.hd; D.Dq = D.Hq * D.hd;
  D.Fp = (int)round_up(D.F, 128); D.Fep = (int)round_up(D.Fe, 128);
  D.n_ctx = (int)round_up(c->n_ctx_max, 64);
  D.Cm = c->n_chunk_max;
  return D;
}

// --------------------------------------------------------------------------------------
// Launch policies
// --------------------------------------------------------------------------------------
constexpr int g_cus = 256;   // compute units of an MI355X; plans and workspace sizes use it
// workgroups resident per CU for a row tile (the 256-row tile takes all of LDS)
inline int wg_per_cu(int mt) { return mt >= 256 ? 1 : 2; }
// Sustained fraction of the CU's MFMA rate per row tile (measured): the 256-row kernel
// dequantises each weight for 256 rows, the smaller tiles for 128 or 64.
inline double tile_eff(int mt) { return mt >= 256 ? 0.60 : (mt >= 128 ? 0.40 : 0.25); }

// A GEMM call runs as one or two launches over column ranges: the tiles that fill whole
// rounds of the chip run unsplit, and (optionally) a tail of whole 256-column tiles runs
// with split-K so that it fills the chip too.  For each row tile the plan minimises a
// simple time model (rounds of workgroups x K stages per workgroup, plus the partial-sum
// traffic and an extra launch for any split); the cheapest row tile wins.
struct GemmPart { int n0, n1, splits; };
struct GemmPlan {
  int mt = 256, nparts = 0;
  GemmPart part[2];
  size_t partial_bytes = 0;
  double cost = 0.0;
};

GemmPlan plan_gemm_mt(int M, int N, int K, int mt, int force_splits) {
  GemmPlan p;
  p.mt = mt;
  const int64_t Mt = ceil_div(M, p.mt), Nt = ceil_div(N, 256), KS = K / 128, T = Mt * Nt;
  const int slots = g_cus * wg_per_cu(p.mt);
  // one 128-wide K stage of a tile, with wg_per_cu tiles sharing a CU
  const double t_stage = 2.0 * p.mt * 256 * 128 * wg_per_cu(p.mt) / (9.77e12 * tile_eff(p.mt));
  const double launch = 4e-6;
  auto red = [&](int64_t S, int64_t cols) { return (double)(S + 1) * M * cols * 4 / 5e12 + launch; };
  // an unsplit range's own epilogue writes (and, adding to the residual, reads) its
  // fp32 outputs; counted once (measured: without it a 2048-row output projection ran
  // unsplit on 160 of the 256 CUs, 25% slower than three splits)
  auto epi = [&](int64_t cols) { return (double)M * cols * 4 / 5e12; };
  auto rounds = [&](int64_t wgs) { return (double)ceil_div(wgs, slots); };
  // 128-wide K stages a workgroup runs for S splits.  The 256-row kernel runs 64-wide
  // stages in groups of four: a split's count is padded to a multiple of four with
  // zero-weight stages, which take as long as real ones (80 stages in 6 splits run 16
  // each, as in 5 splits).
  auto kst = [&](int64_t S) {
    if (p.mt < 256) return (double)ceil_div(KS, S);
    return (double)(ceil_div(ceil_div(K / 64, S), 4) * 4) / 2.0;
  };
  if (force_splits > 0) {
    const int S = (int)std::min<int64_t>(force_splits, KS);
    p.nparts = 1;
    p.part[0] = {0, N, S};
    p.partial_bytes = S > 1 ? (size_t)S * M * N * 4 : 0;
    p.cost = rounds(T * S) * kst(S) * t_stage;
    return p;
  }
  double best = rounds(T) * kst(1) * t_stage + epi(N);
  p.nparts = 1;
  p.part[0] = {0, N, 1};
  for (int64_t S = 2; S <= std::min<int64_t>(16, KS); ++S) {
    const double c = rounds(T * S) * kst(S) * t_stage + red(S, N);
    if (c < best) {
      best = c;
      p.nparts = 1;
      p.part[0] = {0, N, (int)S};
    }
  }
  if (T > slots) {
    const int64_t Nf = (T / slots) * slots / Mt;
    if (Nf > 0 && Nf < Nt) {
      const int64_t R = Mt * (Nt - Nf);
      const int64_t cols = N - Nf * 256;
      for (int64_t S = 2; S <= std::min<int64_t>(16, KS); ++S) {
        const double c = rounds(Mt * Nf) * kst(1) * t_stage + epi(Nf * 256) +
                         rounds(R * S) * kst(S) * t_stage + red(S, cols);
        if (c < best) {
          best = c;
          p.nparts = 2;
          p.part[0] = {0, (int)(Nf * 256), 1};
          p.part[1] = {(int)(Nf * 256), N, (int)S};
        }
      }
    }
  }
  for (int i = 0; i < p.nparts; ++i)
    if (p.part[i].splits > 1)
      p.partial_bytes = std::max(p.partial_bytes, (size_t)p.part[i].splits * M * (p.part[i].n1 - p.part[i].n0) * 4);
  p.cost = best;
  return p;
}

// A few rows (decode-sized chunks): the weight-streaming kernel, "row tile" 1, one
// workgroup per 64 columns and K split S ways.  Measured on the 27B-class shapes, the
// stream runs near the HBM rate once about 600-900 workgroups are in flight, and each
// split costs a reduction launch (about 4 us plus the gap between launches), so S brings
// the workgroup count near 768 and no further (at most one 4-stage share per split).  A
// single row does less arithmetic per weight byte, and there about 1536 workgroups did
// best (the 16-layer share per one-token chunk: 1.94 ms against 1.99 at 768 and 1.97 at
// 1100; with three rows 1536 was 6% slower than 768).
GemmPlan plan_gemm_skinny(int M, int N, int K, int force_splits) {
  GemmPlan p;
  p.mt = 1;
  p.nparts = 1;
  const int KQ = K / 128, P = N / 64;
  int S;
  if (force_splits > 0) S = std::min(force_splits, KQ);
  else S = std::max(1, std::min(((M == 1 ? 1536 : 768) + P / 2) / P, std::max(1, KQ / 4)));
  p.part[0] = {0, N, S};
  p.partial_bytes = S > 1 ? (size_t)S * M * N * 4 : 0;
  return p;
}

bool skinny_fits(int M, int N) { return M <= kSkinnyMaxRows && N % 64 == 0; }

// force_mt > 0 pins the row tile (tests; 1 = the weight-streaming kernel, which needs
// M <= kSkinnyMaxRows and N % 64 == 0); force_splits > 0 forces one launch with that
// split-K factor.
//
// plan: kPlanSingle for a device of its own; with other chunks in flight
// (prefill_chunks with several lanes) kPlanShared, or kPlanSharedDeferred for a GEMM whose
// split-K sums the next kernel adds as it reads them (the output and down projections),
// so that splitting adds no pass of its own.  Beside other chunks the CUs a launch leaves
// idle (a partial round, a narrow launch) are filled by the other lanes' kernels, so rounds
// and tails no longer decide; what a split still buys is a shorter workgroup on a narrow
// launch, at the price of partial sums and padding stages.  Chunks of more than 128 rows
// then take one launch of 256-row tiles: unsplit when its tiles cover three quarters of
// the CUs or its sums would need a reduction pass, else in two K splits.  (Measured with
// three lanes against the single-lane plans and fixed split counts: +9% at 512-row
// chunks, +2% at 2048, +1% at 3328.)
constexpr int kPlanSingle = 0, kPlanShared = 1, kPlanSharedDeferred = 2;
constexpr int kSharedUnsplitTiles = 192;
GemmPlan plan_gemm(int M, int N, int K, int force_splits = 0, int force_mt = 0, int plan = kPlanSingle) {
  if (force_mt == 1 || (force_mt == 0 && skinny_fits(M, N))) return plan_gemm_skinny(M, N, K, force_splits);
  if (force_mt > 0) return plan_gemm_mt(M, N, K, force_mt, force_splits);
  if (plan != kPlanSingle && M > 128 && force_splits == 0) {
    const int64_t T = ceil_div(M, 256) * ceil_div(N, 256);
    return plan_gemm_mt(M, N, K, 256, (T >= kSharedUnsplitTiles || plan != kPlanSharedDeferred) ? 1 : 2);
  }
  if (M <= 64) return plan_gemm_mt(M, N, K, 64, force_splits);
  GemmPlan best = plan_gemm_mt(M, N, K, 128, force_splits);
  if (M <= 128) {
    // (measured at 128 rows: two 64-row tiles with more workgroups in flight beat one
    // 128-row tile on every weight stream but the widest)
    const GemmPlan small = plan_gemm_mt(M, N, K, 64, force_splits);
    if (small.cost < best.cost) best = small;
  }
  if (M > 128) {
    const GemmPlan big = plan_gemm_mt(M, N, K, 256, force_splits);
    if (big.cost < best.cost) best = big;
  }
  return best;
}

// Split-KV factor of a chunk's attention.  Its workgroups (256 query rows of one kv head;
// one per CU, their LDS tiles take 96 KiB) run in rounds of g_cus; s splits multiply the
// workgroups and divide the 64-key tiles each one walks, and add a combine pass that
// reads the s partial rows.  The factor minimises rounds x tiles per workgroup (the
// longest query tile's range) plus that pass.
//
// shared (prefill_chunks with several lanes): the other lanes' kernels fill the CUs an
// unsplit launch leaves idle, so once the unsplit grid has kSharedAttnUnsplit workgroups
// or more the combine pass and its partial rows are not worth it (measured with three
// lanes: +3.6% on the routed-expert share at 3328-token chunks, +2.5% on the q8_0 share at
// 2048, even at 512); decode-sized chunks, a handful of workgroups, still split.
constexpr int64_t kSharedAttnUnsplit = 64;
int attn_splits(const Dims& D, int n, int start, bool shared = false) {
  const int64_t base = ceil_div((int64_t)n * D.G, 256) * D.Hkv;
  if (shared && base >= kSharedAttnUnsplit) return 1;
  const int kvt = (int)ceil_div(start + n, 64);
  const double t_tile = 1.5e-6;                              // one tile, one workgroup
  const double part = (double)n * D.Hq * D.hd * 4;          // fp32 partial rows of a split
  double best = 1e30;
  int bs = 1;
  for (int s = 1; s <= 32 && s <= kvt; ++s) {
    double c = (double)ceil_div(base * s, g_cus) * ceil_div(kvt, s) * t_tile;
    if (s > 1) c += 4e-6 + 1.5 * s * part / 4e12;
    if (c < best) { best = c; bs = s; }
  }
  return bs;
}

// --------------------------------------------------------------------------------------
// Arena layouts
// --------------------------------------------------------------------------------------
struct Bump {
  size_t off = 0;
  size_t take(size_t bytes) { size_t o = off; off += align_up(bytes); return o; }
};

struct QOff { size_t q = 0, d = 0; int N = 0, K = 0; };

QOff qmat_off(Bump& b, int64_t N, int64_t K) {
  QOff o;
  o.N = (int)N; o.K = (int)K;
  o.q = b.take(QMat::q_bytes(N, K));
  o.d = b.take(QMat::d_bytes(N, K));
  return o;
}

struct WLayout {
  size_t attn_norm, ffn_norm, rq, rd;
  QOff qkv, o, gu, dn;
  std::vector<QOff> egu, edn;
  size_t per_layer;
};

WLayout weights_layout(const Dims& D) {
  WLayout W;
  Bump b;
  W.attn_norm = b.take((size_t)D.d * 4);
  W.ffn_norm = b.take((size_t)D.d * 4);
  W.qkv = qmat_off(b, D.Nqkv, D.d);
  W.o = qmat_off(b, D.d, D.Dq);
  if (!D.moe) {
    W.gu = qmat_off(b, 2LL * D.Fp, D.d);
    W.dn = qmat_off(b, D.d, D.Fp);
    W.rq = W.rd = 0;
  } else {
    W.rq = b.take((size_t)D.E * D.d);
    W.rd = b.take((size_t)D.E * (D.d / QK) * 2);
    for (int e = 0; e < D.E; ++e) W.egu.push_back(qmat_off(b, 2LL * D.Fep, D.d));
    for (int e = 0; e < D.E; ++e) W.edn.push_back(qmat_off(b, D.d, D.Fep));
  }
  W.per_layer = b.off;
  return W;
}

struct WsLayout {
  size_t cos, sin, stage;            // rope tables, then everything else (also state staging)
  size_t xn, xn32, qkv, q, attn, h, yperm;
  size_t logits, idx, w, rank, ccnt, offsets, perm, inv, tiles, ntiles;
  size_t partial, partial_bytes;
  size_t apo, apml, arows;   // split-KV partials: rows of capacity
  int max_tiles;
  size_t total;
};

size_t max_partial_bytes(const Dims& D) {
  size_t best = 0;
  const int Ns[4] = {D.Nqkv, D.d, D.moe ? 0 : 2 * D.Fp, D.d};
  const int Ks[4] = {D.d, D.Dq, D.d, D.moe ? 0 : D.Fp};
  for (int g = 0; g < 4; ++g) {
    if (!Ns[g] || !Ks[g]) continue;
    for (int M = 1; M <= D.Cm; ++M)
      for (const int plan : {kPlanSingle, kPlanShared, kPlanSharedDeferred})
        best = std::max(best, plan_gemm(M, Ns[g], Ks[g], 0, 0, plan).partial_bytes);
  }
  return best;
}

size_t max_attn_partial_rows(const Dims& D) {
  size_t best = 0;
  for (int n = 1; n <= D.Cm; ++n) {
    const int s = attn_splits(D, n, std::max(0, D.n_ctx - n));
    if (s > 1) best = std::max(best, (size_t)s * D.Hkv * n * D.G);
  }
  return best;
}

WsLayout workspace_layout(const Dims& D) {
  WsLayout S;
  Bump b;
  const size_t half = (size_t)D.hd / 2;
  S.cos = b.take((size_t)D.n_ctx * half * 4);
  S.sin = b.take((size_t)D.n_ctx * half * 4);
  S.stage = b.off;
  const size_t Cm = D.Cm;
  S.xn = b.take(Cm * D.d * 2);
  S.xn32 = D.moe ? b.take(Cm * D.d * 4) : 0;
  S.qkv = b.take(Cm * D.Nqkv * 4);
  S.q = b.take(Cm * D.Dq * 2);
  S.attn = b.take(Cm * D.Dq * 2);
  if (!D.moe) {
    S.h = b.take(Cm * D.Fp * 2);
    S.yperm = S.logits = S.idx = S.w = S.rank = S.ccnt = S.offsets = S.perm = S.inv = 0;
    S.tiles = S.ntiles = 0;
    S.max_tiles = 0;
  } else {
    const size_t slots = Cm * D.k;
    S.h = b.take(slots * D.Fep * 2);
    S.yperm = b.take(slots * D.d * 4);
    S.logits = b.take(Cm * D.E * 4);
    S.idx = b.take(slots * 4);
    S.w = b.take(slots * 4);
    S.rank = b.take(slots * 4);
    S.ccnt = b.take((size_t)ceil_div(slots, kMoeChunk) * D.E * 4);
    S.offsets = b.take((size_t)(D.E + 1) * 4);
    S.perm = b.take(slots * 4);
    S.inv = b.take(slots * 4);
    S.max_tiles = (int)(ceil_div(slots, 128) + D.E);
    S.tiles = b.take((size_t)S.max_tiles * 16);
    S.ntiles = b.take(16);
  }
  S.partial_bytes = max_partial_bytes(D);
  S.partial = S.partial_bytes ? b.take(S.partial_bytes) : 0;
  const size_t arows = max_attn_partial_rows(D);
  S.arows = arows;
  S.apo = arows ? b.take(arows * D.hd * 4) : 0;
  S.apml = arows ? b.take(arows * 2 * 4) : 0;
  S.total = b.off;
  return S;
}

size_t kv_per_layer(const Dims& D) { return align_up(kv_layer_bytes(D.Hkv, D.hd, D.n_ctx, D.kv_type)); }

size_t row_bytes(int hd, int kv_type) { return kv_type == CP_KV_F16 ? (size_t)hd * 2 : (size_t)(hd / QK) * 34; }

size_t state_size(const Dims& D, int64_t n_tokens) {
  return 32 + (size_t)D.L * 2 * n_tokens * D.Hkv * row_bytes(D.hd, D.kv_type);
}

struct StateHeader {
  char magic[4];
  uint32_t version, kv_type, n_layer, n_kv_head, head_dim, n_tokens;
  float rope_theta;
};
static_assert(sizeof(StateHeader) == 32, "state header is 32 bytes");

int check_state(const cp_config* c, const void* src, size_t n, std::string& err, uint32_t* n_tok) {
  if (!src) { err = "state source is NULL"; return CP_E_INVALID; }
  if (n < sizeof(StateHeader)) { err = "state shorter than its header"; return CP_E_STATE; }
  StateHeader h;
  std::memcpy(&h, src, sizeof h);
  if (std::memcmp(h.magic, "CPKV", 4)) { err = "state magic mismatch"; return CP_E_STATE; }
  if (h.version != 1) { err = "state version mismatch"; return CP_E_STATE; }
  if ((int)h.kv_type != c->kv_type) { err = "state kv_type mismatch"; return CP_E_STATE; }
  if ((int)h.n_layer != c->n_layer) { err = "state n_layer mismatch"; return CP_E_STATE; }
  if ((int)h.n_kv_head != c->n_kv_head) { err = "state n_kv_head mismatch"; return CP_E_STATE; }
  if ((int)h.head_dim != c->head_dim) { err = "state head_dim mismatch"; return CP_E_STATE; }
  if (std::memcmp(&h.rope_theta, &c->rope_theta, 4)) { err = "state rope_theta mismatch"; return CP_E_STATE; }
  if (h.n_tokens > (uint32_t)c->n_ctx_max) { err = "state longer than n_ctx_max"; return CP_E_STATE; }
  const Dims D = dims_of(c);
  if (n != state_size(D, h.n_tokens)) { err = "state length does not match its header"; return CP_E_STATE; }
  if (n_tok) *n_tok = h.n_tokens;
  return CP_OK;
}

struct LayerW {
  float* attn_norm;
  float* ffn_norm;
  QMat qkv, o, gu, dn;
  int8_t* rq;
  uint16_t* rd;
  int8_t* egu_q; uint32_t* egu_d; int64_t egu_qs, egu_ds;
  int8_t* edn_q; uint32_t* edn_d; int64_t edn_qs, edn_ds;
  KvLayer kv;
};

QMat qmat_at(uint8_t* base, const QOff& o) {
  QMat m;
  m.q = reinterpret_cast<int8_t*>(base + o.q);
  m.d = reinterpret_cast<uint32_t*>(base + o.d);
  m.N = o.N; m.K = o.K;
  return m;
}

}  // namespace

struct cp_ctx {
  cp_config cfg;
  Dims D;
  WLayout WL;
  WsLayout WS;
  hipStream_t stream = nullptr;
  PendingSum pend_x;            // split-K sums into the chunk's x not yet added
  bool plan_shared = false;      // GEMM launch plans for a device shared with other lanes
  uint8_t* warena = nullptr;
  uint8_t* kv = nullptr;
  uint8_t* ws = nullptr;
  uint8_t* stage = nullptr;     // the per-chunk buffers (offsets WS.stage on): ws + WS.stage,
                                // or this device's static array during prefill_chunk_static
  int device = 0;               // the device current at prefill_init
  std::vector<hipEvent_t> wave_ev; // prefill_chunks: [lane][layer] "layer done" events
  std::vector<LayerW> layers;
  int32_t n_past = 0;
  std::string err;
  // timing
  bool timing = false;
  std::string timing_classes;   // comma-separated class names, or "*" for all
  struct Rec { std::string cls; hipEvent_t a, b; };
  std::vector<Rec> pending;
  std::vector<hipEvent_t> pool;
  std::map<std::string, std::pair<double, int>> totals;

  template <typename T> T* wsp(size_t off) {
    return reinterpret_cast<T*>(off >= WS.stage ? stage + (off - WS.stage) : ws + off);
  }

  hipEvent_t ev() {
    if (!pool.empty()) { hipEvent_t e = pool.back(); pool.pop_back(); return e; }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};

namespace {

int fail(cp_ctx* c, int code, const std::string& msg) {
  if (c) c->err = msg;
  return code;
}

int hip_fail(cp_ctx* c, hipError_t e, const char* what) {
  return fail(c, CP_E_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
}

#define CP_HIP(ctx, call, what)                          \
  do {                                                   \
    hipError_t _e = (call);                              \
    if (_e != hipSuccess) return hip_fail(ctx, _e, what);\
  } while (0)

// Runs `launch` bracketed by timing events when timing is on for this context.
template <typename F>
hipError_t timed(cp_ctx* c, const char* cls, F&& launch) {
  if (!c->timing) return launch();
  if (c->timing_classes != "*") {
    const std::string key = std::string(",") + cls + ",";
    if (("," + c->timing_classes + ",").find(key) == std::string::npos) return launch();
  }
  hipEvent_t a = c->ev(), b = c->ev();
  if (!a || !b) return launch();
  hipEventRecord(a, c->stream);
  hipError_t e = launch();
  hipEventRecord(b, c->stream);
  c->pending.push_back({cls, a, b});
  return e;
}

// defer (optional): a split launch covering the last column range leaves its partial
// sums pending and describes them there (PendingSum) for the kernel that reads the
// result, instead of running the reduction pass; *defer is cleared otherwise.  This holds
// for chunks of any size: at a few rows the reading kernel (RMSNorm, one workgroup per
// row) has few workgroups for the partial reads, but it still costs less than the launch
// of the reduction pass it replaces.
// chunks of up to this many tokens run RoPE and the K/V append as one launch, reading the
// QKV GEMM's split planes directly
constexpr int kQkvPostMaxRows = kSkinnyMaxRows;
hipError_t gemm(cp_ctx* c, const char* cls, const _Float16* A, int lda, int M, const QMat& W,
                int mode, void* out, int ldo, PendingSum* defer = nullptr) {
  // (split sums are deferred only for a non-SwiGLU launch)
  const bool deferrable = defer && mode != GM_SWIGLU;
  const GemmPlan p = plan_gemm(M, W.N, W.K, 0, 0,
                               !c->plan_shared ? kPlanSingle : deferrable ? kPlanSharedDeferred : kPlanShared);
  if (defer) *defer = PendingSum();
  return timed(c, cls, [&] {
    for (int i = 0; i < p.nparts; ++i) {
      const bool leave = deferrable && p.part[i].splits > 1 && i == p.nparts - 1;
      GemmArgs g;
      g.A = A; g.lda = lda; g.M = M; g.N = p.part[i].n1; g.K = W.K; g.n0 = p.part[i].n0;
      g.wq = W.q; g.wd = W.d; g.mode = mode; g.out = out; g.ldo = ldo;
      g.splits = p.part[i].splits;
      g.partial = c->wsp<float>(c->WS.partial);
      // each launch is also timed on its own: "<class>/full" for an unsplit column range
      // (one kernel), "<class>/split" for a split-K range (partial GEMM + ordered reduce),
      // "<class>/skinny" for the weight-streaming kernel of a few rows
      const std::string sub = std::string(cls) + (p.mt == 1 ? "/skinny" : g.splits > 1 ? "/split" : "/full");
      const hipError_t e = timed(c, sub.c_str(), [&] { return launch_gemm(g, 0, p.mt, c->stream, !leave); });
      if (e != hipSuccess) return e;
      if (leave) {
        defer->partial = g.partial;
        defer->splits = g.splits; defer->M = M; defer->n0 = g.n0; defer->N = g.N;
        defer->add = mode == GM_F32_ADD;
      }
    }
    return hipSuccess;
  });
}

// One layer of one chunk.  The split-K sums of the output projection are taken by the FFN
// RMSNorm, and those of the down projection by the next layer's first RMSNorm
// (c->pend_x), or, with flush_end, by a reduction pass at the end of the layer.
int run_layer(cp_ctx* c, int li, const float* x_res_in, float* x, int n, int start, bool flush_end) {
  const Dims& D = c->D;
  const LayerW& L = c->layers[li];
  hipStream_t s = c->stream;
  _Float16* xn = c->wsp<_Float16>(c->WS.xn);
  float* qkv = c->wsp<float>(c->WS.qkv);
  _Float16* q = c->wsp<_Float16>(c->WS.q);
  _Float16* attn = c->wsp<_Float16>(c->WS.attn);
  const float* cos_t = c->wsp<float>(c->WS.cos);
  const float* sin_t = c->wsp<float>(c->WS.sin);

  // pending sums into x exist only from the previous layer, which wrote x itself
  const PendingSum px = c->pend_x;
  c->pend_x = PendingSum();
  if (px.partial && x_res_in != x) return fail(c, CP_E_DEVICE, "pending sums on the chunk input");
  // (x_res_in is written only when sums are pending, and then it is x)
  CP_HIP(c, timed(c, "rmsnorm", [&] { return launch_rmsnorm(const_cast<float*>(x_res_in), L.attn_norm, n, D.d, c->cfg.rms_eps, xn, nullptr, s, px); }), "rmsnorm");
  // (the QKV sums of a larger chunk are reduced in their own pass: RoPE reads each q/k
  // value twice, as a value and as its rotation partner, so it would read the partials
  // twice.  A chunk of a few tokens hands its unsummed planes to the one-launch RoPE +
  // append instead, which saves two launches per layer.)
  const bool few = n <= kQkvPostMaxRows;
  PendingSum pq;
  CP_HIP(c, gemm(c, "gemm_qkv", xn, D.d, n, L.qkv, GM_F32, qkv, D.Nqkv, few ? &pq : nullptr), "gemm_qkv");
  CP_HIP(c, timed(c, "rope_kv_append", [&] {
    if (few)
      return launch_qkv_post(qkv, pq, cos_t, sin_t, n, start, D.Hq, D.Hkv, D.hd, D.kv_type, D.n_ctx, q, L.kv, s);
    hipError_t e = launch_rope_qk(qkv, cos_t, sin_t, n, start, D.Hq, D.Hkv, D.hd, D.kv_type, D.n_ctx, q, L.kv, s);
    if (e != hipSuccess) return e;
    return launch_v_append(qkv, n, start, D.Hq, D.Hkv, D.hd, D.kv_type, D.n_ctx, L.kv, s);
  }), "rope_kv_append");
  AttnArgs aa;
  aa.q = q; aa.kv = L.kv; aa.n = n; aa.start = start; aa.n_head = D.Hq; aa.n_kv_head = D.Hkv;
  aa.head_dim = D.hd; aa.kv_type = D.kv_type; aa.n_ctx = D.n_ctx; aa.out = attn;
  // at most the splits whose partial rows the workspace holds (sized for the deepest
  // chunk of each length)
  const int64_t rows1 = (int64_t)D.Hkv * n * D.G;
  aa.splits = (int)std::max<int64_t>(1, std::min<int64_t>(attn_splits(D, n, start, c->plan_shared),
                                                          (int64_t)c->WS.arows / rows1));
  aa.part_o = c->wsp<float>(c->WS.apo);
  aa.part_ml = c->wsp<float>(c->WS.apml);
  CP_HIP(c, timed(c, "attention", [&] { return launch_attention(aa, s); }), "attention");
  if (x != x_res_in)
    CP_HIP(c, hipMemcpyAsync(x, x_res_in, (size_t)n * D.d * 4, hipMemcpyDeviceToDevice, s), "residual copy");
  PendingSum po;
  CP_HIP(c, gemm(c, "gemm_o", attn, D.Dq, n, L.o, GM_F32_ADD, x, D.d, &po), "gemm_o");

  if (!D.moe) {
    CP_HIP(c, timed(c, "rmsnorm", [&] { return launch_rmsnorm(x, L.ffn_norm, n, D.d, c->cfg.rms_eps, xn, nullptr, s, po); }), "rmsnorm");
    _Float16* hbuf = c->wsp<_Float16>(c->WS.h);
    CP_HIP(c, gemm(c, "gemm_gate_up", xn, D.d, n, L.gu, GM_SWIGLU, hbuf, D.Fp), "gemm_gate_up");
    CP_HIP(c, gemm(c, "gemm_down", hbuf, D.Fp, n, L.dn, GM_F32_ADD, x, D.d, &c->pend_x), "gemm_down");
    if (flush_end && c->pend_x.partial) {
      const PendingSum& pd = c->pend_x;
      CP_HIP(c, timed(c, "gemm_down", [&] {
        return launch_splitk_reduce(pd.partial, pd.splits, pd.M, pd.n0, pd.N, GM_F32_ADD, x, D.d, s);
      }), "gemm_down reduce");
      c->pend_x = PendingSum();
    }
    return CP_OK;
  }
  float* xn32 = c->wsp<float>(c->WS.xn32);
  CP_HIP(c, timed(c, "rmsnorm", [&] { return launch_rmsnorm(x, L.ffn_norm, n, D.d, c->cfg.rms_eps, xn, xn32, s, po); }), "rmsnorm");
  MoeBuffers mb;
  mb.logits = c->wsp<float>(c->WS.logits); mb.idx = c->wsp<int32_t>(c->WS.idx);
  mb.w = c->wsp<float>(c->WS.w); mb.rank = c->wsp<int32_t>(c->WS.rank);
  mb.chunk_cnt = c->wsp<int32_t>(c->WS.ccnt); mb.offsets = c->wsp<int32_t>(c->WS.offsets);
  mb.perm = c->wsp<int32_t>(c->WS.perm); mb.inv = c->wsp<int32_t>(c->WS.inv);
  mb.tiles = c->wsp<int32_t>(c->WS.tiles); mb.n_tiles = c->wsp<int32_t>(c->WS.ntiles);
  CP_HIP(c, timed(c, "moe_route", [&] { return launch_router(xn32, L.rq, L.rd, n, D.d, D.E, D.k, mb.logits, mb.idx, mb.w, s); }), "moe_route");
  // expert row tiles of 256 (the one-workgroup-per-CU kernel) once the experts average
  // 128 token-slots or more, else 128
  const int mt = (int64_t)n * D.k >= 128LL * D.E ? 256 : 128;
  const int max_tiles = (int)(ceil_div((int64_t)n * D.k, mt) + D.E);
  CP_HIP(c, timed(c, "moe_permute", [&] { return launch_moe_permute(mb, n, D.E, D.k, mt, max_tiles, s); }), "moe_permute");
  _Float16* hperm = c->wsp<_Float16>(c->WS.h);
  float* yperm = c->wsp<float>(c->WS.yperm);
  GemmArgs g;
  g.A = xn; g.lda = D.d; g.a_rows = mb.perm; g.a_row_div = D.k;
  g.wq = L.egu_q; g.wd = L.egu_d; g.wq_estride = L.egu_qs; g.wd_estride = L.egu_ds;
  g.M = n * D.k; g.N = 2 * D.Fep; g.K = D.d; g.tiles = mb.tiles; g.n_tiles = mb.n_tiles;
  g.mode = GM_SWIGLU; g.out = hperm; g.ldo = D.Fep; g.splits = 1;
  CP_HIP(c, timed(c, "moe_gemm_gate_up", [&] { return launch_gemm(g, max_tiles, mt, s); }), "moe_gemm_gate_up");
  GemmArgs g2 = g;
  g2.A = hperm; g2.lda = D.Fep; g2.a_rows = nullptr; g2.a_row_div = 1;
  g2.wq = L.edn_q; g2.wd = L.edn_d; g2.wq_estride = L.edn_qs; g2.wd_estride = L.edn_ds;
  g2.N = D.d; g2.K = D.Fep; g2.mode = GM_F32; g2.out = yperm; g2.ldo = D.d;
  CP_HIP(c, timed(c, "moe_gemm_down", [&] { return launch_gemm(g2, max_tiles, mt, s); }), "moe_gemm_down");
  CP_HIP(c, timed(c, "moe_unpermute", [&] { return launch_moe_unpermute(yperm, mb, n, D.d, D.k, x, x, s); }), "moe_unpermute");
  return CP_OK;
}

// All layers of one checked chunk at positions n_past .. n_past+n-1; advances n_past.
int run_chunk(cp_ctx* c, const float* x_in, float* x_out, int n) {
  const int start = c->n_past;
  c->pend_x = PendingSum();
  for (int l = 0; l < c->D.L; ++l) {
    const int r = run_layer(c, l, l == 0 ? x_in : x_out, x_out, n, start, l == c->D.L - 1);
    if (r != CP_OK) return r;
  }
  c->n_past = start + n;
  return CP_OK;
}

// The workspace layout of a chunk of exactly n tokens whose per-chunk part (offsets from
// WS.stage on) must fit kStaticScratchBytes.  The RoPE tables before it keep their offsets
// (they depend on n_ctx only).  If the split-KV partial rows do not fit, they are dropped:
// attention then runs unsplit (same result to rounding, no partials).  False when even
// that does not fit.
bool static_stage_layout(const Dims& D0, int n, WsLayout* out) {
  Dims D = D0;
  D.Cm = n;
  WsLayout L = workspace_layout(D);
  if (L.total - L.stage > kStaticScratchBytes && L.arows) {
    L.total = L.apo;
    L.arows = 0;
    L.apo = L.apml = 0;
  }
  if (L.total - L.stage > kStaticScratchBytes) return false;
  *out = L;
  return true;
}

bool aligned(const void* p) { return ((uintptr_t)p % kAlign) == 0; }

}  // namespace

// --------------------------------------------------------------------------------------
// The static scratch array of prefill_chunk_static: one copy per device, which that device
// holds from the library's load until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is a stand-in, not a device address): it looks
// the device address up once per device with hipGetSymbolAddress and uses that.
// --------------------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

// This device's address of `scratch`, looked up on the first call for the device with
// that device current (then restored), and kept.
hipError_t static_scratch(int device, uint8_t** out) {
  static std::mutex mu;
  static uint8_t* addr[kMaxDevices] = {};
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[device]) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != device) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!p || (uintptr_t)p % kAlign) return hipErrorInvalidSymbol;
    addr[device] = static_cast<uint8_t*>(p);
  }
  *out = addr[device];
  return hipSuccess;
}

}  // namespace

// ======================================================================================
// C ABI
// ======================================================================================
extern "C" {

int cp_validate_config(const cp_config* cfg) { return validate(cfg).empty() ? CP_OK : CP_E_INVALID; }

const char* cp_config_error(const cp_config* cfg) {
  static thread_local std::string msg;
  msg = validate(cfg);
  return msg.c_str();
}

size_t cp_weights_arena_bytes(const cp_config* cfg) {
  if (!validate(cfg).empty()) return 0;
  const Dims D = dims_of(cfg);
  return weights_layout(D).per_layer * D.L;
}

size_t cp_kv_bytes(const cp_config* cfg) {
  if (!validate(cfg).empty()) return 0;
  const Dims D = dims_of(cfg);
  return kv_per_layer(D) * D.L;
}

size_t cp_workspace_bytes(const cp_config* cfg) {
  if (!validate(cfg).empty()) return 0;
  return workspace_layout(dims_of(cfg)).total;
}

size_t cp_state_bytes(const cp_config* cfg, int32_t n_tokens) {
  if (!validate(cfg).empty() || n_tokens < 0) return 0;
  return state_size(dims_of(cfg), n_tokens);
}

int cp_state_check(const cp_config* cfg, const void* src, size_t n_bytes) {
  if (!validate(cfg).empty()) return CP_E_INVALID;
  std::string err;
  return check_state(cfg, src, n_bytes, err, nullptr);
}

int cp_chunk_check(const cp_config* cfg, int32_t n_past, const float* x_in, const float* x_out,
                   int32_t n_tokens) {
  if (!validate(cfg).empty() || n_past < 0) return CP_E_INVALID;
  std::string err;
  return chunk_check(cfg, n_past, x_in, x_out, n_tokens, err);
}

int prefill_init(const cp_config* cfg, const cp_layer_weights* layers, void* weights_arena,
                 void* kv_buf, void* workspace, void* hip_stream, cp_ctx** out) {
  if (!out) return CP_E_INVALID;
  *out = nullptr;
  if (!validate(cfg).empty()) return CP_E_INVALID;
  if (!layers || !weights_arena || !kv_buf || !workspace) return CP_E_INVALID;
  if (!aligned(weights_arena) || !aligned(kv_buf) || !aligned(workspace)) return CP_E_ARENA;
  cp_ctx* c = new cp_ctx();
  c->cfg = *cfg;
  c->D = dims_of(cfg);
  c->WL = weights_layout(c->D);
  c->WS = workspace_layout(c->D);
  c->stream = (hipStream_t)hip_stream;
  c->warena = (uint8_t*)weights_arena;
  c->kv = (uint8_t*)kv_buf;
  c->ws = (uint8_t*)workspace;
  c->stage = c->ws + c->WS.stage;
  const Dims& D = c->D;
  auto bail = [&](int code) { delete c; return code; };
  if (hipGetDevice(&c->device) != hipSuccess) return bail(CP_E_DEVICE);
  const WLayout& W = c->WL;
  hipStream_t s = c->stream;
  for (int l = 0; l < D.L; ++l) {
    const cp_layer_weights& src = layers[l];
    if (!src.wq || !src.wk || !src.wv || !src.wo || !src.attn_norm || !src.ffn_norm || !src.w_gate ||
        !src.w_up || !src.w_down || (D.moe && !src.w_router))
      return bail(CP_E_INVALID);
  }
  for (int l = 0; l < D.L; ++l) {
    const cp_layer_weights& src = layers[l];
    uint8_t* base = c->warena + W.per_layer * l;
    LayerW L{};
    L.attn_norm = reinterpret_cast<float*>(base + W.attn_norm);
    L.ffn_norm = reinterpret_cast<float*>(base + W.ffn_norm);
    hipError_t e = hipMemcpyAsync(L.attn_norm, src.attn_norm, (size_t)D.d * 4, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess) e = hipMemcpyAsync(L.ffn_norm, src.ffn_norm, (size_t)D.d * 4, hipMemcpyDeviceToDevice, s);
    L.qkv = qmat_at(base, W.qkv);
    L.o = qmat_at(base, W.o);
    const int64_t nq = (int64_t)D.Hq * D.hd, nk = (int64_t)D.Hkv * D.hd;
    if (e == hipSuccess) e = launch_repack_q8_0(src.wq, nullptr, nq, D.d, 0, nq, 0, L.qkv, s);
    if (e == hipSuccess) e = launch_repack_q8_0(src.wk, nullptr, nk, D.d, nq, nk, 0, L.qkv, s);
    if (e == hipSuccess) e = launch_repack_q8_0(src.wv, nullptr, nk, D.d, nq + nk, nk, 0, L.qkv, s);
    if (e == hipSuccess) e = launch_repack_q8_0(src.wo, nullptr, D.d, D.Dq, 0, D.d, 0, L.o, s);
    if (!D.moe) {
      L.gu = qmat_at(base, W.gu);
      L.dn = qmat_at(base, W.dn);
      if (e == hipSuccess)
        e = launch_repack_q8_0(src.w_gate, src.w_up, D.F, D.d, 0, 2LL * D.Fp, 1, L.gu, s);
      if (e == hipSuccess) e = launch_repack_q8_0(src.w_down, nullptr, D.d, D.F, 0, D.d, 0, L.dn, s);
    } else {
      L.rq = reinterpret_cast<int8_t*>(base + W.rq);
      L.rd = reinterpret_cast<uint16_t*>(base + W.rd);
      if (e == hipSuccess) e = launch_unpack_router(src.w_router, D.E, D.d, L.rq, L.rd, s);
      const QMat g0 = qmat_at(base, W.egu[0]), d0 = qmat_at(base, W.edn[0]);
      L.egu_q = g0.q; L.egu_d = g0.d; L.edn_q = d0.q; L.edn_d = d0.d;
      L.egu_qs = D.E > 1 ? (int64_t)(W.egu[1].q - W.egu[0].q) : 0;
      L.egu_ds = D.E > 1 ? (int64_t)(W.egu[1].d - W.egu[0].d) / 4 : 0;
      L.edn_qs = D.E > 1 ? (int64_t)(W.edn[1].q - W.edn[0].q) : 0;
      L.edn_ds = D.E > 1 ? (int64_t)(W.edn[1].d - W.edn[0].d) / 4 : 0;
      const size_t gate_bytes = (size_t)D.Fe * ((D.d + QK - 1) / QK) * 34;
      const size_t down_bytes = (size_t)D.d * ((D.Fe + QK - 1) / QK) * 34;
      for (int x = 0; x < D.E && e == hipSuccess; ++x) {
        const uint8_t* gsrc = (const uint8_t*)src.w_gate + gate_bytes * x;
        const uint8_t* usrc = (const uint8_t*)src.w_up + gate_bytes * x;
        e = launch_repack_q8_0(gsrc, usrc, D.Fe, D.d, 0, 2LL * D.Fep, 1, qmat_at(base, W.egu[x]), s);
        if (e == hipSuccess)
          e = launch_repack_q8_0((const uint8_t*)src.w_down + down_bytes * x, nullptr, D.d, D.Fe, 0, D.d, 0,
                                 qmat_at(base, W.edn[x]), s);
      }
    }
    L.kv = kv_layer_at(c->kv + kv_per_layer(D) * l, D.Hkv, D.hd, D.n_ctx, D.kv_type);
    if (e != hipSuccess) { int r = hip_fail(c, e, "weight repack"); delete c; return r; }
    c->layers.push_back(L);
  }
  // The cache starts zeroed: attention stages whole 64-position tiles, so cells past the
  // valid range are read (and weighted by zero); they must hold finite values.
  {
    const hipError_t ez = hipMemsetAsync(c->kv, 0, kv_per_layer(D) * D.L, s);
    if (ez != hipSuccess) { int r = hip_fail(c, ez, "cache clear"); delete c; return r; }
  }
  // RoPE table: omega_i = theta^(-2i/hd), angle = p * omega_i in float64, cos/sin rounded
  // to float32.
  const int half = D.hd / 2;
  std::vector<float> ct((size_t)D.n_ctx * half), st((size_t)D.n_ctx * half);
  const double theta = (double)cfg->rope_theta;
  for (int i = 0; i < half; ++i) {
    const double w = std::pow(theta, -2.0 * i / D.hd);
    for (int p = 0; p < D.n_ctx; ++p) {
      const double a = (double)p * w;
      ct[(size_t)p * half + i] = (float)std::cos(a);
      st[(size_t)p * half + i] = (float)std::sin(a);
    }
  }
  hipError_t e = hipMemcpyAsync(c->ws + c->WS.cos, ct.data(), ct.size() * 4, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(c->ws + c->WS.sin, st.data(), st.size() * 4, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) { int r = hip_fail(c, e, "init"); delete c; return r; }
  *out = c;
  return CP_OK;
}

int prefill_chunk(cp_ctx* c, const float* x_in, float* x_out, int32_t n) {
  if (!c) return CP_E_INVALID;
  if (const int r = chunk_check(&c->cfg, c->n_past, x_in, x_out, n, c->err); r != CP_OK) return r;
  return run_chunk(c, x_in, x_out, n);
}

int prefill_chunk_static(cp_ctx* c, const float* x_in, float* x_out, int32_t n) {
  if (!c) return CP_E_INVALID;
  if (const int r = chunk_check(&c->cfg, c->n_past, x_in, x_out, n, c->err); r != CP_OK) return r;
  WsLayout L;
  if (!static_stage_layout(c->D, n, &L))
    return fail(c, CP_E_CAPACITY, "the chunk's buffers exceed the static scratch array (" +
                                      std::to_string(kStaticScratchBytes >> 20) + " MiB)");
  uint8_t* base = nullptr;
  const hipError_t e = static_scratch(c->device, &base);
  if (e != hipSuccess) return hip_fail(c, e, "static scratch address");
  // the chunk's buffers are taken from the static array for this call only
  struct Swap {
    cp_ctx* c; WsLayout ws; uint8_t* stage;
    ~Swap() { c->WS = ws; c->stage = stage; }
  } restore{c, c->WS, c->stage};
  c->WS = L;
  c->stage = base;
  return run_chunk(c, x_in, x_out, n);
}

int prefill_chunks(cp_ctx* c, const float* x_in, float* x_out, int32_t n_tokens, int32_t chunk,
                   int32_t n_lanes, void* const* workspaces, void* const* hip_streams) {
  if (!c) return CP_E_INVALID;
  if (n_lanes < 1 || n_lanes > kMaxLanes) return fail(c, CP_E_INVALID, "n_lanes outside [1, 8]");
  if (n_lanes > 1 && (!workspaces || !hip_streams)) return fail(c, CP_E_INVALID, "workspaces / hip_streams is NULL");
  for (int j = 1; j < n_lanes; ++j) {
    if (!workspaces[j - 1] || !aligned(workspaces[j - 1]))
      return fail(c, CP_E_ARENA, "a lane's workspace is NULL or not 256-byte aligned");
    if ((hipStream_t)hip_streams[j - 1] == c->stream)
      return fail(c, CP_E_INVALID, "a lane's stream is the context's stream");
    for (int i = 1; i < j; ++i)
      if (hip_streams[i - 1] == hip_streams[j - 1]) return fail(c, CP_E_INVALID, "two lanes share a stream");
  }
  if (chunk < 1 || chunk > c->cfg.n_chunk_max) return fail(c, CP_E_CAPACITY, "chunk outside [1, n_chunk_max]");
  if (n_tokens < 1) return fail(c, CP_E_INVALID, "n_tokens < 1");
  // every chunk's checks before anything is enqueued (rows are d_model floats apart, so a
  // chunk's rows keep the 16-byte alignment of x_in / x_out)
  if (const int r = chunk_check(&c->cfg, c->n_past, x_in, x_out, std::min(chunk, n_tokens), c->err); r != CP_OK)
    return r;
  if ((int64_t)c->n_past + n_tokens > c->cfg.n_ctx_max) return fail(c, CP_E_CAPACITY, "n_past + n_tokens > n_ctx_max");
  const Dims& D = c->D;
  const int L = D.L;
  // events: [lane][layer] "layer done", one "lane done" per lane,
  // and one join event (the context's stream at entry)
  const size_t n_ev = (size_t)kMaxLanes * (L + 1) + 1;
  if (c->wave_ev.size() != n_ev) {
    for (auto& e : c->wave_ev) if (e) hipEventDestroy(e);
    c->wave_ev.assign(n_ev, nullptr);
    for (auto& e : c->wave_ev) {
      const hipError_t er = hipEventCreateWithFlags(&e, hipEventDisableTiming);
      if (er != hipSuccess) {
        for (auto& f : c->wave_ev) if (f) hipEventDestroy(f);
        c->wave_ev.clear();
        return hip_fail(c, er, "event create");
      }
    }
  }
  auto ev = [&](int lane, int layer) { return c->wave_ev[(size_t)lane * L + layer]; };
  auto lane_done = [&](int lane) { return c->wave_ev[(size_t)kMaxLanes * L + lane]; };
  struct Lane { hipStream_t stream; uint8_t* stage; };
  Lane lanes[kMaxLanes];
  lanes[0] = {c->stream, c->stage};
  for (int j = 1; j < n_lanes; ++j)
    lanes[j] = {(hipStream_t)hip_streams[j - 1], (uint8_t*)workspaces[j - 1] + c->WS.stage};
  const hipStream_t saved_stream = c->stream;
  uint8_t* const saved_stage = c->stage;
  const bool saved_shared = c->plan_shared;
  auto restore = [&] {
    c->stream = saved_stream; c->stage = saved_stage; c->pend_x = PendingSum(); c->plan_shared = saved_shared;
  };
  const int K = (n_tokens + chunk - 1) / chunk;
  const int used = std::min(n_lanes, K);
  // the other lanes start after the work already on the context's stream
  hipEvent_t join = c->wave_ev[n_ev - 1];
  CP_HIP(c, hipEventRecord(join, lanes[0].stream), "event record");
  for (int j = 1; j < used; ++j) CP_HIP(c, hipStreamWaitEvent(lanes[j].stream, join, 0), "stream wait");
  const int start0 = c->n_past;
  if (n_lanes > 1) c->plan_shared = true;     // restored with the rest
  // Chunk i runs on lane i mod n_lanes, its layers in order; its layer l starts once chunk
  // i-1 (the previous lane) has finished layer l, whose cache rows it attends to.  So while
  // chunk i runs layer l, chunk i+1 runs layer l-1, and so on.  A lane runs its chunks
  // whole, one after another, so its buffers (and the split-K sums one layer leaves to the
  // next) belong to one chunk at a time.  An event is re-recorded by chunk i+n_lanes only
  // after chunk i+1's wait on it has been enqueued.
  for (int i = 0; i < K; ++i) {
    const int li = i % n_lanes, lp = (i + n_lanes - 1) % n_lanes;
    const Lane& ln = lanes[li];
    const int s = i * chunk, n = std::min(chunk, n_tokens - s);
    const float* xi = x_in + (int64_t)s * D.d;
    float* xo = x_out + (int64_t)s * D.d;
    c->stream = ln.stream;
    c->stage = ln.stage;
    c->pend_x = PendingSum();
    for (int l = 0; l < L; ++l) {
      if (i > 0 && n_lanes > 1) {
        const hipError_t e = hipStreamWaitEvent(ln.stream, ev(lp, l), 0);
        if (e != hipSuccess) { restore(); return hip_fail(c, e, "stream wait"); }
      }
      const int r = run_layer(c, l, l == 0 ? xi : xo, xo, n, start0 + s, l == L - 1);
      if (r != CP_OK) { restore(); return r; }
      if (n_lanes > 1) {
        const hipError_t e = hipEventRecord(ev(li, l), ln.stream);
        if (e != hipSuccess) { restore(); return hip_fail(c, e, "event record"); }
      }
    }
  }
  restore();
  // the context's stream continues after every lane's last chunk
  for (int j = 1; j < used; ++j) {
    CP_HIP(c, hipEventRecord(lane_done(j), lanes[j].stream), "event record");
    CP_HIP(c, hipStreamWaitEvent(lanes[0].stream, lane_done(j), 0), "stream wait");
  }
  c->n_past = start0 + n_tokens;
  return CP_OK;
}

int prefill_chunk_trace(cp_ctx* c, const float* x_in, float* x_out, int32_t n, float* layer_out,
                        int64_t layer_stride, int32_t* route_idx, int64_t route_stride) {
  if (!c) return CP_E_INVALID;
  if (const int r = chunk_check(&c->cfg, c->n_past, x_in, x_out, n, c->err); r != CP_OK) return r;
  if (layer_out && layer_stride < (int64_t)n * c->D.d) return fail(c, CP_E_INVALID, "layer_stride too small");
  if (route_idx && (!c->D.moe || route_stride < (int64_t)n * c->D.k))
    return fail(c, CP_E_INVALID, "route_idx needs routed experts and route_stride >= n * n_expert_used");
  const int start = c->n_past;
  c->pend_x = PendingSum();
  for (int l = 0; l < c->D.L; ++l) {
    const int r = run_layer(c, l, l == 0 ? x_in : x_out, x_out, n, start, true);
    if (r != CP_OK) return r;
    if (layer_out)
      CP_HIP(c, hipMemcpyAsync(layer_out + layer_stride * l, x_out, (size_t)n * c->D.d * 4,
                               hipMemcpyDeviceToDevice, c->stream), "trace copy");
    if (route_idx)
      CP_HIP(c, hipMemcpyAsync(route_idx + route_stride * l, c->wsp<int32_t>(c->WS.idx),
                               (size_t)n * c->D.k * 4, hipMemcpyDeviceToDevice, c->stream), "trace copy");
  }
  c->n_past = start + n;
  return CP_OK;
}

int prefill_chunk_timed(cp_ctx* c, const float* x_in, float* x_out, int32_t n, float* layer_ms) {
  if (!c) return CP_E_INVALID;
  if (!layer_ms) return fail(c, CP_E_INVALID, "layer_ms is NULL");
  if (const int r = chunk_check(&c->cfg, c->n_past, x_in, x_out, n, c->err); r != CP_OK) return r;
  const int L = c->D.L;
  std::vector<hipEvent_t> ev(L + 1, nullptr);
  for (auto& e : ev) CP_HIP(c, hipEventCreate(&e), "event create");
  const int start = c->n_past;
  int rc = CP_OK;
  if (hipEventRecord(ev[0], c->stream) != hipSuccess) rc = fail(c, CP_E_DEVICE, "event record");
  c->pend_x = PendingSum();
  for (int l = 0; l < L && rc == CP_OK; ++l) {
    rc = run_layer(c, l, l == 0 ? x_in : x_out, x_out, n, start, l == L - 1);
    if (rc == CP_OK && hipEventRecord(ev[l + 1], c->stream) != hipSuccess) rc = fail(c, CP_E_DEVICE, "event record");
  }
  if (rc == CP_OK) {
    hipError_t e = hipEventSynchronize(ev[L]);
    if (e != hipSuccess) rc = hip_fail(c, e, "event sync");
    for (int l = 0; l < L && rc == CP_OK; ++l) hipEventElapsedTime(&layer_ms[l], ev[l], ev[l + 1]);
  }
  for (auto& e : ev) hipEventDestroy(e);
  if (rc == CP_OK) c->n_past = start + n;
  return rc;
}

int kv_cache_get_state(cp_ctx* c, void* dst, size_t cap, size_t* n_bytes) {
  if (!c || !n_bytes) return CP_E_INVALID;
  const Dims& D = c->D;
  const size_t need = state_size(D, c->n_past);
  *n_bytes = need;
  if (!dst) return CP_OK;
  if (cap < need) return fail(c, CP_E_ARENA, "destination smaller than the state");
  CP_HIP(c, hipStreamSynchronize(c->stream), "stream sync");
  StateHeader h;
  std::memcpy(h.magic, "CPKV", 4);
  h.version = 1; h.kv_type = (uint32_t)D.kv_type; h.n_layer = (uint32_t)D.L;
  h.n_kv_head = (uint32_t)D.Hkv; h.head_dim = (uint32_t)D.hd; h.n_tokens = (uint32_t)c->n_past;
  h.rope_theta = c->cfg.rope_theta;
  std::memcpy(dst, &h, sizeof h);
  uint8_t* o = (uint8_t*)dst + sizeof h;
  const size_t rb = row_bytes(D.hd, D.kv_type) * D.Hkv;
  uint8_t* stage = c->ws + c->WS.stage;
  const size_t stage_cap = c->WS.total - c->WS.stage;
  const int64_t slice = std::max<int64_t>(1, (int64_t)(stage_cap / rb));
  for (int l = 0; l < D.L; ++l)
    for (int which = 0; which < 2; ++which)
      for (int64_t t0 = 0; t0 < c->n_past; t0 += slice) {
        const int nt = (int)std::min<int64_t>(slice, c->n_past - t0);
        CP_HIP(c, launch_kv_pack(c->layers[l].kv, (int)t0, nt, D.Hkv, D.hd, D.kv_type, D.n_ctx, which, stage, c->stream), "state pack");
        CP_HIP(c, hipMemcpyAsync(o, stage, rb * nt, hipMemcpyDeviceToHost, c->stream), "state copy");
        CP_HIP(c, hipStreamSynchronize(c->stream), "stream sync");
        o += rb * nt;
      }
  return CP_OK;
}

int kv_cache_set_state(cp_ctx* c, const void* src, size_t n_bytes) {
  if (!c) return CP_E_INVALID;
  uint32_t nt_total = 0;
  const int r = check_state(&c->cfg, src, n_bytes, c->err, &nt_total);
  if (r != CP_OK) return r;
  const Dims& D = c->D;
  CP_HIP(c, hipStreamSynchronize(c->stream), "stream sync");
  const uint8_t* p = (const uint8_t*)src + sizeof(StateHeader);
  const size_t rb = row_bytes(D.hd, D.kv_type) * D.Hkv;
  uint8_t* stage = c->ws + c->WS.stage;
  const size_t stage_cap = c->WS.total - c->WS.stage;
  const int64_t slice = std::max<int64_t>(1, (int64_t)(stage_cap / rb));
  for (int l = 0; l < D.L; ++l)
    for (int which = 0; which < 2; ++which)
      for (int64_t t0 = 0; t0 < (int64_t)nt_total; t0 += slice) {
        const int nt = (int)std::min<int64_t>(slice, nt_total - t0);
        CP_HIP(c, hipMemcpyAsync(stage, p, rb * nt, hipMemcpyHostToDevice, c->stream), "state copy");
        CP_HIP(c, launch_kv_unpack(c->layers[l].kv, (int)t0, nt, D.Hkv, D.hd, D.kv_type, D.n_ctx, which, stage, c->stream), "state unpack");
        CP_HIP(c, hipStreamSynchronize(c->stream), "stream sync");
        p += rb * nt;
      }
  c->n_past = (int32_t)nt_total;
  return CP_OK;
}

int kv_cache_truncate(cp_ctx* c, int32_t n_keep) {
  if (!c) return CP_E_INVALID;
  if (n_keep < 0 || n_keep > c->n_past) return fail(c, CP_E_INVALID, "n_keep outside [0, n_past]");
  c->n_past = n_keep;
  return CP_OK;
}

int32_t prefill_n_past(const cp_ctx* c) { return c ? c->n_past : -1; }

const char* prefill_last_error(const cp_ctx* c) { return c ? c->err.c_str() : "context is NULL"; }

void prefill_free(cp_ctx* c) {
  if (!c) return;
  hipStreamSynchronize(c->stream);
  for (auto& r : c->pending) { hipEventDestroy(r.a); hipEventDestroy(r.b); }
  for (auto e : c->pool) hipEventDestroy(e);
  for (auto e : c->wave_ev) hipEventDestroy(e);
  delete c;
}

int cp_test_set_plan_shared(cp_ctx* c, int32_t shared) {
  if (!c || (shared != 0 && shared != 1)) return CP_E_INVALID;
  c->plan_shared = shared != 0;
  return CP_OK;
}

int cp_kernel_timing(cp_ctx* c, const char* classes) {
  if (!c) return CP_E_INVALID;
  CP_HIP(c, hipStreamSynchronize(c->stream), "stream sync");
  for (auto& r : c->pending) { c->pool.push_back(r.a); c->pool.push_back(r.b); }
  c->pending.clear();
  c->totals.clear();
  c->timing = classes != nullptr;
  c->timing_classes = classes ? classes : "";
  return CP_OK;
}

int cp_kernel_times(cp_ctx* c, const char* cls, float* total_ms, int32_t* launches) {
  if (!c || !cls || !total_ms || !launches) return CP_E_INVALID;
  CP_HIP(c, hipStreamSynchronize(c->stream), "stream sync");
  for (auto& r : c->pending) {
    float ms = 0.0f;
    hipEventElapsedTime(&ms, r.a, r.b);
    auto& t = c->totals[r.cls];
    t.first += ms;
    t.second += 1;
    c->pool.push_back(r.a);
    c->pool.push_back(r.b);
  }
  c->pending.clear();
  auto it = c->totals.find(cls);
  *total_ms = it == c->totals.end() ? 0.0f : (float)it->second.first;
  *launches = it == c->totals.end() ? 0 : it->second.second;
  return CP_OK;
}

int cp_quantize_q8_0(const float* x, int64_t rows, int32_t k, int64_t ldx, void* out, void* stream) {
  if (!x || !out || rows < 0 || k < 1 || ldx < k) return CP_E_INVALID;
  return launch_quantize_q8_0(x, rows, k, ldx, out, (hipStream_t)stream) == hipSuccess ? CP_OK : CP_E_DEVICE;
}

int cp_last_logits(const float* x_row, const float* norm_gain, const void* lm_head, int32_t vocab,
                   int32_t d_model, float eps, float* logits, void* hip_stream) {
  if (!x_row || !norm_gain || !lm_head || !logits || vocab < 1 || d_model < QK || d_model % QK ||
      d_model > 32768 || !(eps > 0.0f) || ((uintptr_t)lm_head % 2))
    return CP_E_INVALID;
  return launch_last_logits(x_row, norm_gain, lm_head, vocab, d_model, eps, logits,
                            (hipStream_t)hip_stream) == hipSuccess ? CP_OK : CP_E_DEVICE;
}

int32_t cp_plan_chunk(int32_t n_tokens, int32_t cap, int32_t stages, double b_over_a) {
  if (n_tokens < 0 || cap < 1 || stages < 1 || !(b_over_a > 0.0) || !std::isfinite(b_over_a))
    return CP_E_INVALID;
  if (n_tokens == 0) return 0;
  if (stages == 1) return std::min(n_tokens, cap);
  // (S - 1 + n/C) chunk-steps of (b + a*C): smallest at C = sqrt(n * (b/a) / (S - 1))
  auto up256 = [](int64_t v) { return (v + 255) / 256 * 256; };
  const double c = std::sqrt((double)n_tokens * b_over_a / (double)(stages - 1));
  int64_t c0 = up256((int64_t)std::ceil(c));
  c0 = std::max<int64_t>(512, std::min<int64_t>(cap, c0));
  const int64_t k = (n_tokens + c0 - 1) / c0;
  if (k <= 1) return std::min(n_tokens, cap);
  return (int32_t)std::min<int64_t>(cap, up256((n_tokens + k - 1) / k));
}

size_t cp_peak_sink_bytes(void) { return peak_sink_bytes(); }

int cp_measure_peaks(const void* read_buf, size_t read_bytes, void* sink, size_t sink_bytes,
                     void* stream, double* mfma_tflops, double* hbm_gbs) {
  if (!read_buf || !sink || !mfma_tflops || !hbm_gbs || read_bytes < ((size_t)1 << 24) ||
      read_bytes % 16 || ((uintptr_t)read_buf % 16) || sink_bytes < peak_sink_bytes())
    return CP_E_INVALID;
  hipStream_t s = (hipStream_t)stream;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    if (e0) hipEventDestroy(e0);
    return CP_E_DEVICE;
  }
  int rc = CP_OK;
  double fl = 0.0;
  float ms = 0.0f;
  // MFMA loop: one short warm-up launch, then a timed one of about a millisecond
  if (launch_mfma_peak(64, (float*)sink, s, &fl) != hipSuccess || hipEventRecord(e0, s) != hipSuccess ||
      launch_mfma_peak(2048, (float*)sink, s, &fl) != hipSuccess || hipEventRecord(e1, s) != hipSuccess ||
      hipEventSynchronize(e1) != hipSuccess || hipEventElapsedTime(&ms, e0, e1) != hipSuccess || ms <= 0.0f) {
    rc = CP_E_DEVICE;
  } else {
    *mfma_tflops = fl / (ms * 1e-3) / 1e12;
  }
  // streaming read: one warm-up pass, then three timed passes
  if (rc == CP_OK) {
    const int64_t nb = (int64_t)read_bytes;
    bool ok = launch_stream_read(read_buf, nb, (uint32_t*)sink, s) == hipSuccess && hipEventRecord(e0, s) == hipSuccess;
    for (int r = 0; ok && r < 3; ++r) ok = launch_stream_read(read_buf, nb, (uint32_t*)sink, s) == hipSuccess;
    ok = ok && hipEventRecord(e1, s) == hipSuccess && hipEventSynchronize(e1) == hipSuccess &&
         hipEventElapsedTime(&ms, e0, e1) == hipSuccess && ms > 0.0f;
    if (ok) *hbm_gbs = 3.0 * (double)read_bytes / (ms * 1e-3) / 1e9;
    else rc = CP_E_DEVICE;
  }
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  return rc;
}

// ---------------------------------------------------------------------------------- tests
size_t cp_test_kv_layer_bytes(int32_t n_kv_head, int32_t head_dim, int32_t n_ctx, int32_t kv_type) {
  return kv_layer_bytes(n_kv_head, head_dim, (int32_t)round_up(n_ctx, 64), kv_type);
}

int cp_test_rope_kv_append(const float* qkv, const float* cos_t, const float* sin_t, int32_t n,
                           int32_t start, int32_t n_head, int32_t n_kv_head, int32_t head_dim,
                           int32_t kv_type, int32_t n_ctx, void* q_out, void* kv, void* stream) {
  if (!qkv || !cos_t || !sin_t || !q_out || !kv || n < 1 || start < 0 || start + n > n_ctx) return CP_E_INVALID;
  if ((head_dim != 64 && head_dim != 128) || n_kv_head < 1 || n_head % n_kv_head) return CP_E_INVALID;
  const int nc = (int)round_up(n_ctx, 64);
  KvLayer L = kv_layer_at(kv, n_kv_head, head_dim, nc, kv_type);
  hipStream_t s = (hipStream_t)stream;
  if (launch_rope_qk(qkv, cos_t, sin_t, n, start, n_head, n_kv_head, head_dim, kv_type, nc, (_Float16*)q_out, L, s) != hipSuccess)
    return CP_E_DEVICE;
  return launch_v_append(qkv, n, start, n_head, n_kv_head, head_dim, kv_type, nc, L, s) == hipSuccess ? CP_OK : CP_E_DEVICE;
}

int cp_test_rope_kv_append_planes(const float* partial, int32_t splits, const float* cos_t,
                                  const float* sin_t, int32_t n, int32_t start, int32_t n_head,
                                  int32_t n_kv_head, int32_t head_dim, int32_t kv_type, int32_t n_ctx,
                                  void* q_out, void* kv, void* work, void* stream) {
  if (!partial || !cos_t || !sin_t || !q_out || !kv || !work || splits < 1 || n < 1 || start < 0 ||
      start + n > n_ctx)
    return CP_E_INVALID;
  if ((head_dim != 64 && head_dim != 128) || n_kv_head < 1 || n_head % n_kv_head) return CP_E_INVALID;
  const int nc = (int)round_up(n_ctx, 64);
  KvLayer L = kv_layer_at(kv, n_kv_head, head_dim, nc, kv_type);
  hipStream_t s = (hipStream_t)stream;
  const int32_t Nqkv = (n_head + 2 * n_kv_head) * head_dim;
  float* qkv = (float*)work;
  if (n <= kQkvPostMaxRows) {
    PendingSum ps;
    if (splits > 1) {
      ps.partial = partial; ps.splits = splits; ps.M = n; ps.n0 = 0; ps.N = Nqkv;
    } else {
      qkv = const_cast<float*>(partial);
    }
    return launch_qkv_post(qkv, ps, cos_t, sin_t, n, start, n_head, n_kv_head, head_dim, kv_type, nc,
                           (_Float16*)q_out, L, s) == hipSuccess ? CP_OK : CP_E_DEVICE;
  }
  if (launch_splitk_reduce(partial, splits, n, 0, Nqkv, GM_F32, qkv, Nqkv, s) != hipSuccess) return CP_E_DEVICE;
  if (launch_rope_qk(qkv, cos_t, sin_t, n, start, n_head, n_kv_head, head_dim, kv_type, nc, (_Float16*)q_out, L, s) != hipSuccess)
    return CP_E_DEVICE;
  return launch_v_append(qkv, n, start, n_head, n_kv_head, head_dim, kv_type, nc, L, s) == hipSuccess ? CP_OK : CP_E_DEVICE;
}

int cp_test_kv_rows(const void* kv, int32_t n_tokens, int32_t n_kv_head, int32_t head_dim,
                    int32_t kv_type, int32_t n_ctx, void* out, void* stream) {
  if (!kv || !out || n_tokens < 1 || n_tokens > n_ctx) return CP_E_INVALID;
  const int nc = (int)round_up(n_ctx, 64);
  KvLayer L = kv_layer_at(const_cast<void*>(kv), n_kv_head, head_dim, nc, kv_type);
  const size_t rb = row_bytes(head_dim, kv_type) * n_kv_head;
  hipStream_t s = (hipStream_t)stream;
  if (launch_kv_pack(L, 0, n_tokens, n_kv_head, head_dim, kv_type, nc, 0, (uint8_t*)out, s) != hipSuccess) return CP_E_DEVICE;
  return launch_kv_pack(L, 0, n_tokens, n_kv_head, head_dim, kv_type, nc, 1, (uint8_t*)out + rb * n_tokens, s) == hipSuccess
             ? CP_OK : CP_E_DEVICE;
}

size_t cp_test_router_scratch_bytes(int32_t n_expert, int32_t d) {
  return align_up((size_t)n_expert * d) + align_up((size_t)n_expert * (d / QK) * 2);
}

int cp_test_router(const float* y, const void* w_router, int32_t n, int32_t d, int32_t E, int32_t k,
                   float* logits, int32_t* idx, float* weight, void* work, void* stream) {
  if (!y || !w_router || !logits || !idx || !weight || !work || n < 1 || d < 32 || d % 32 ||
      E < 1 || E > 256 || k < 1 || k > E || k > 16)
    return CP_E_INVALID;
  int8_t* q = (int8_t*)work;
  uint16_t* dd = (uint16_t*)((uint8_t*)work + align_up((size_t)E * d));
  hipStream_t s = (hipStream_t)stream;
  if (launch_unpack_router(w_router, E, d, q, dd, s) != hipSuccess) return CP_E_DEVICE;
  return launch_router(y, q, dd, n, d, E, k, logits, idx, weight, s) == hipSuccess ? CP_OK : CP_E_DEVICE;
}

bool test_row_tile_ok(int32_t M, int32_t N, int32_t row_tile) {
  if (row_tile == 1) return skinny_fits(M, N);
  return row_tile == 0 || row_tile == 64 || row_tile == 128 || row_tile == 256;
}

size_t cp_test_gemm_scratch_bytes_ex(int32_t M, int32_t N, int32_t K, int32_t splits, int32_t row_tile) {
  if (M < 1 || N < 32 || N % 32 || K < 128 || K % 128 || splits < 0) return 0;
  if (!test_row_tile_ok(M, N, row_tile)) return 0;
  const GemmPlan p = plan_gemm(M, N, K, splits, row_tile);
  return align_up(QMat::q_bytes(N, K)) + align_up(QMat::d_bytes(N, K)) + align_up(p.partial_bytes + 4);
}

size_t cp_test_gemm_scratch_bytes(int32_t M, int32_t N, int32_t K, int32_t splits) {
  return cp_test_gemm_scratch_bytes_ex(M, N, K, splits, 0);
}

int cp_test_gemm_ex(const void* A, const void* W, int32_t M, int32_t N, int32_t K, int32_t mode,
                    int32_t splits, int32_t row_tile, void* out, void* work, void* stream) {
  if (!A || !W || !out || !work || M < 1 || N < 32 || N % 32 || K < 128 || K % 128 || mode < 0 ||
      mode > 2 || splits < 0)
    return CP_E_INVALID;
  if (!test_row_tile_ok(M, N, row_tile)) return CP_E_INVALID;
  if (mode == GM_SWIGLU && N % 64) return CP_E_INVALID;
  hipStream_t s = (hipStream_t)stream;
  QMat q;
  q.q = (int8_t*)work;
  q.d = (uint32_t*)((uint8_t*)work + align_up(QMat::q_bytes(N, K)));
  q.N = N; q.K = K;
  float* partial = (float*)((uint8_t*)q.d + align_up(QMat::d_bytes(N, K)));
  const GemmPlan p = plan_gemm(M, N, K, splits, row_tile);
  hipError_t e;
  if (mode == GM_SWIGLU) {
    const int F = N / 2;
    const uint8_t* up = (const uint8_t*)W + (size_t)F * (K / QK) * 34;
    e = launch_repack_q8_0(W, up, F, K, 0, N, 1, q, s);
  } else {
    e = launch_repack_q8_0(W, nullptr, N, K, 0, N, 0, q, s);
  }
  if (e != hipSuccess) return CP_E_DEVICE;
  for (int i = 0; i < p.nparts; ++i) {
    GemmArgs g;
    g.A = (const _Float16*)A; g.lda = K; g.M = M; g.N = p.part[i].n1; g.K = K; g.n0 = p.part[i].n0;
    g.wq = q.q; g.wd = q.d;
    g.mode = mode; g.out = out; g.ldo = mode == GM_SWIGLU ? N / 2 : N;
    g.splits = p.part[i].splits;
    g.partial = partial;
    if (launch_gemm(g, 0, p.mt, s) != hipSuccess) return CP_E_DEVICE;
  }
  return CP_OK;
}

int cp_test_gemm(const void* A, const void* W, int32_t M, int32_t N, int32_t K, int32_t mode,
                 int32_t splits, void* out, void* work, void* stream) {
  return cp_test_gemm_ex(A, W, M, N, K, mode, splits, 0, out, work, stream);
}

int cp_test_gemm_plan(int32_t M, int32_t N, int32_t K, int32_t plan, int32_t* out6) {
  if (!out6 || M < 1 || N < 32 || K < 128 || plan < kPlanSingle || plan > kPlanSharedDeferred) return CP_E_INVALID;
  const GemmPlan p = plan_gemm(M, N, K, 0, 0, plan);
  out6[0] = p.mt; out6[1] = p.nparts;
  for (int i = 0; i < 2; ++i) {
    out6[2 + 2 * i] = i < p.nparts ? p.part[i].n0 : 0;
    out6[3 + 2 * i] = i < p.nparts ? p.part[i].splits : 0;
  }
  return CP_OK;
}

size_t cp_test_attention_scratch_bytes(int32_t n, int32_t n_head, int32_t head_dim, int32_t kv_splits) {
  const int s = kv_splits > 0 ? kv_splits : 32;
  return align_up((size_t)s * n * n_head * head_dim * 4) + align_up((size_t)s * n * n_head * 2 * 4);
}

int cp_test_attention(const void* q, const void* kv, int32_t n, int32_t start, int32_t n_head,
                      int32_t n_kv_head, int32_t head_dim, int32_t kv_type, int32_t n_ctx,
                      int32_t kv_splits, void* out, void* work, void* stream) {
  if (!q || !kv || !out || !work || n < 1 || start < 0 || start + n > n_ctx) return CP_E_INVALID;
  if ((head_dim != 64 && head_dim != 128) || n_kv_head < 1 || n_head % n_kv_head || kv_splits < 0 || kv_splits > 32)
    return CP_E_INVALID;
  Dims D{};
  D.Hq = n_head; D.Hkv = n_kv_head; D.hd = head_dim; D.G = n_head / n_kv_head;
  const int nc = (int)round_up(n_ctx, 64);
  AttnArgs a;
  a.q = (const _Float16*)q;
  a.kv = kv_layer_at(const_cast<void*>(kv), n_kv_head, head_dim, nc, kv_type);
  a.n = n; a.start = start; a.n_head = n_head; a.n_kv_head = n_kv_head; a.head_dim = head_dim;
  a.kv_type = kv_type; a.n_ctx = nc; a.out = (_Float16*)out;
  a.splits = kv_splits > 0 ? kv_splits : attn_splits(D, n, start);
  a.part_o = (float*)work;
  a.part_ml = (float*)((uint8_t*)work + align_up((size_t)a.splits * n * n_head * head_dim * 4));
  return launch_attention(a, (hipStream_t)stream) == hipSuccess ? CP_OK : CP_E_DEVICE;
}

}  // extern "C"
