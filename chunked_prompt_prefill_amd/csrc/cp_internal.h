// Internal declarations shared by the host runtime and the kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "chunk_prefill.h"

namespace cp {

constexpr int QK = 32;              // q8_0 block length
constexpr int kAlign = 256;         // every arena sub-buffer starts on 256 bytes

__host__ __device__ inline size_t align_up(size_t v, size_t a = kAlign) { return (v + a - 1) / a * a; }
__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// --------------------------------------------------------------------------------------
// Repacked q8_0 matrix [N][K] (N % 32 == 0, K % 128 == 0).
//   q: int8, for every 32-row group n32 and 32-column block kb, 1 KiB laid out in MFMA
//      lane order: lane l (row n32*32 + l%32) holds bytes 16*(l/32) .. +15 of that
//      row's block -> offset ((n32*KB + kb)*64 + l)*16.
//   d: fp16 scales, four per 8 bytes: for 32-row group n32 and block quad kq (blocks
//      4kq .. 4kq+3) -> fp16 index ((n32*KQ + kq)*32 + row%32)*4 + kb%4.
// --------------------------------------------------------------------------------------
struct QMat {
  int8_t* q = nullptr;
  uint32_t* d = nullptr;
  int32_t N = 0, K = 0;
  static size_t q_bytes(int64_t N, int64_t K) { return (size_t)(N * K); }
  static size_t d_bytes(int64_t N, int64_t K) { return (size_t)(N * (K / QK) * 2); }
};

enum GemmMode : int32_t { GM_F32 = 0, GM_F32_ADD = 1, GM_SWIGLU = 2, GM_PARTIAL = 3 };

struct GemmArgs {
  const _Float16* A = nullptr;    // [rows][lda]
  int32_t lda = 0;
  const int32_t* a_rows = nullptr;   // grouped: physical A row = a_rows[m] / a_row_div
  int32_t a_row_div = 1;
  const int8_t* wq = nullptr;
  const uint32_t* wd = nullptr;
  int64_t wq_estride = 0, wd_estride = 0;   // grouped: per-expert strides (elements)
  int32_t M = 0, N = 0, K = 0;
  int32_t n0 = 0;                     // first output column of this launch (N = end)
  const int32_t* tiles = nullptr;     // grouped: [max_tiles][4] {expert, m0, m1, 0}
  const int32_t* n_tiles = nullptr;   // grouped: device count of valid tiles
  int32_t mode = GM_F32;
  void* out = nullptr;
  int32_t ldo = 0;
  float* partial = nullptr;           // split-K partial sums [splits][M][N - n0]
  int32_t splits = 1;
};

// Rows up to which the weight-streaming kernel (k_gemv.hip) takes a GEMM.
constexpr int kSkinnyMaxRows = 4;

// A split-K GEMM result whose partial sums have not been added yet.  Column c >= n0 of
// row m of the result is partial[0][m][c-n0] + ... + partial[splits-1][m][c-n0] (added in
// split order), then, when add is set, base[m][c] + that sum; columns below n0 are final
// in the base matrix.  A consumer kernel that reads the result through this description
// replaces the separate reduction pass (same arithmetic, same order).
struct PendingSum {
  const float* partial = nullptr;   // nullptr: nothing pending
  int32_t splits = 0, M = 0, n0 = 0, N = 0;
  bool add = false;
};

// Kernel launchers (return hipError_t of the launch).  With reduce = false a split launch
// leaves its partial sums for the caller (who describes them with a PendingSum).
hipError_t launch_gemm(const GemmArgs& a, int grid_m_tiles, int mt, hipStream_t s, bool reduce = true);
// 256-row tiles, one workgroup per CU; the partial-sum reduction of a split launch is left
// to the caller.  Grouped (a.tiles set): grid_m_tiles is the tile table's capacity.
hipError_t launch_gemm_big(const GemmArgs& a, int grid_m_tiles, hipStream_t s);
// M <= kSkinnyMaxRows, N % 64 == 0, whole column range; splits = K splits.  With one
// split it applies the epilogue itself; with more it writes partial [S][M][N] and the
// caller runs the split-K reduction (launch_gemm does).
hipError_t launch_gemm_skinny(const GemmArgs& a, hipStream_t s);
hipError_t launch_splitk_reduce(const float* partial, int32_t splits, int32_t M, int32_t n0,
                                int32_t N, int32_t mode, void* out, int32_t ldo, hipStream_t s);
// Repack interchange q8_0 rows into a QMat.  mode 0: destination rows dst_row0 ..
// dst_row0+dst_rows-1 take source rows 0 .. (rows >= src_rows are zero).  mode 1 (gate/up
// interleave for the SwiGLU epilogue): destination row n = 64*g + 32*w + i takes row
// 32*g + i of src0 (w = 0, gate) or src1 (w = 1, up); rows >= src_rows are zero.
// Source blocks beyond ceil(k_src/32) are zero.
hipError_t launch_repack_q8_0(const void* src0, const void* src1, int64_t src_rows, int32_t k_src,
                              int64_t dst_row0, int64_t dst_rows, int32_t mode, QMat dst,
                              hipStream_t s);
hipError_t launch_quantize_q8_0(const float* x, int64_t rows, int32_t k, int64_t ldx,
                                void* out, hipStream_t s);
// y = RMSNorm(x) * gamma (fp16; y32: the same in float32, or nullptr).  With ps pending,
// x first takes its pending sums (see PendingSum; x is the base matrix) and the result is
// written back to x.
hipError_t launch_rmsnorm(float* x, const float* gamma, int32_t n, int32_t d, float eps,
                          _Float16* y, float* y32, hipStream_t s, const PendingSum& ps = PendingSum());

struct KvLayer {          // one layer's cache (device pointers), capacity n_ctx
  void* k = nullptr;      // f16 [Hkv][n_ctx][hd]  | int8 [Hkv][n_ctx][hd]
  void* v = nullptr;      // f16 [Hkv][hd][n_ctx]  | int8 [Hkv][hd][n_ctx]
  uint16_t* kd = nullptr; // q8_0: fp16 [Hkv][n_ctx][hd/32]
  uint16_t* vd = nullptr; // q8_0: fp16 [Hkv][hd/32][n_ctx]
};
size_t kv_layer_bytes(int32_t n_kv_head, int32_t head_dim, int32_t n_ctx, int32_t kv_type);
KvLayer kv_layer_at(void* base, int32_t n_kv_head, int32_t head_dim, int32_t n_ctx,
                    int32_t kv_type);

hipError_t launch_rope_qk(const float* qkv, const float* cos_t, const float* sin_t, int32_t n,
                          int32_t start, int32_t n_head, int32_t n_kv_head, int32_t head_dim,
                          int32_t kv_type, int32_t n_ctx, _Float16* q_out, KvLayer kv,
                          hipStream_t s);
hipError_t launch_v_append(const float* qkv, int32_t n, int32_t start, int32_t n_head,
                           int32_t n_kv_head, int32_t head_dim, int32_t kv_type, int32_t n_ctx,
                           KvLayer kv, hipStream_t s);
// The QKV values RoPE and the append read: output rows qkv [n][Nqkv] (splits == 0), or the
// split planes partial [splits][n][Nqkv] of a split GEMM, added in split order.
struct QkvSrc {
  const float* qkv = nullptr;
  const float* partial = nullptr;
  int32_t splits = 0;
  int64_t plane = 0;
};
// RoPE + K append + V append in one launch (chunks of a few tokens), from qkv or, when ps
// holds them, the QKV GEMM's unsummed split planes (M == n, whole column range).
hipError_t launch_qkv_post(const float* qkv, const PendingSum& ps, const float* cos_t,
                           const float* sin_t, int32_t n, int32_t start, int32_t n_head,
                           int32_t n_kv_head, int32_t head_dim, int32_t kv_type, int32_t n_ctx,
                           _Float16* q_out, KvLayer kv, hipStream_t s);

struct AttnArgs {
  const _Float16* q = nullptr;   // [n][Hq][hd]
  KvLayer kv;
  int32_t n = 0, start = 0, n_head = 0, n_kv_head = 0, head_dim = 0, kv_type = 0, n_ctx = 0;
  _Float16* out = nullptr;         // [n][Hq*hd]
  int32_t splits = 1;
  float* part_o = nullptr;       // [splits][rows_total][hd]
  float* part_ml = nullptr;      // [splits][rows_total][2]
};
int attention_rows_total(int32_t n, int32_t n_head);
hipError_t launch_attention(const AttnArgs& a, hipStream_t s);

hipError_t launch_kv_pack(const KvLayer kv, int32_t t0, int32_t nt, int32_t n_kv_head,
                          int32_t head_dim, int32_t kv_type, int32_t n_ctx, int which,
                          uint8_t* out, hipStream_t s);
hipError_t launch_kv_unpack(KvLayer kv, int32_t t0, int32_t nt, int32_t n_kv_head,
                            int32_t head_dim, int32_t kv_type, int32_t n_ctx, int which,
                            const uint8_t* in, hipStream_t s);

// Routed experts.
struct MoeBuffers {
  float* logits = nullptr;     // [n][E]
  int32_t* idx = nullptr;      // [n][k]
  float* w = nullptr;          // [n][k]
  int32_t* rank = nullptr;     // [n*k]   rank of a slot among equal experts in its chunk
  int32_t* chunk_cnt = nullptr;// [n_chunks][E]
  int32_t* offsets = nullptr;  // [E+1]
  int32_t* perm = nullptr;     // [n*k]  permuted position -> slot (t*k + rank)
  int32_t* inv = nullptr;      // [n*k]  slot -> permuted position
  int32_t* tiles = nullptr;    // [max_tiles][4]
  int32_t* n_tiles = nullptr;  // [1]
};
hipError_t launch_router(const float* y, const int8_t* rq, const uint16_t* rd, int32_t n, int32_t d,
                         int32_t E, int32_t k, float* logits, int32_t* idx, float* w,
                         hipStream_t s);
hipError_t launch_moe_permute(const MoeBuffers& b, int32_t n, int32_t E, int32_t k, int32_t mt,
                              int32_t max_tiles, hipStream_t s);
hipError_t launch_moe_unpermute(const float* y_perm, const MoeBuffers& b, int32_t n, int32_t d,
                                int32_t k, const float* x_res, float* x_out, hipStream_t s);

// Router weights unpacked from the interchange layout: int8 [E][d] + fp16 [E][d/32].
hipError_t launch_unpack_router(const void* src, int32_t E, int32_t d, int8_t* q, uint16_t* dd,
                                hipStream_t s);

constexpr int kMoeChunk = 256;   // slots per permute chunk

// Peak measurement kernels (k_peak.hip).
size_t peak_sink_bytes();
hipError_t launch_mfma_peak(int32_t iters, float* sink, hipStream_t s, double* flops);
hipError_t launch_stream_read(const void* buf, int64_t n_bytes, uint32_t* sink, hipStream_t s);

// Last-position logits (k_elem.hip).
hipError_t launch_last_logits(const float* x, const float* gamma, const void* head, int32_t vocab,
                              int32_t d, float eps, float* logits, hipStream_t s);

}  // namespace cp
