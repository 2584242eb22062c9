/*
 * chunk_prefill.h - C ABI of the MI355X (gfx950) chunked prompt prefill library.
 *
 * What it computes.  Chunked prompt prefill of a decoder transformer, as measured
 * throughout the pages "completion : allow the prompt to be processed under its own
 * split mode", "llama : switch the split mode of a live context", the llama.cpp
 * "--split-overlap" pull request, "refactor: one prefill planner and one pad-trim hook
 * for CLI and server" and "Prompt chunks sized for a layer split's pipeline": a prompt
 * is read in chunks of C tokens; each chunk runs through every layer of this GPU's
 * share of the model, appends its K/V rows to a device-resident cache (f16 or q8_0),
 * and attends causally to the whole cache so far.  Per layer:
 *   RMSNorm -> q8_0 QKV projection -> RoPE -> K/V append -> causal GQA attention
 *   -> q8_0 output projection + residual -> RMSNorm -> SwiGLU FFN (dense, or top-k
 *   routed experts) + residual.
 * There is no final norm and no LM head: the chunk's output is the residual stream
 * after the last layer.
 *
 * Arithmetic.  The residual stream, norms, RoPE and softmax are float32.  Every matrix
 * product (the q8_0 projections and both attention products) runs on fp16 MFMA with
 * float32 accumulation: activations are rounded to fp16 and each q8_0 weight enters as
 * the correctly rounded fp16 of d*q.  fp16 runs at the bf16 rate on gfx950 and keeps 3
 * more mantissa bits, which is what holds a full-size layer within 1e-2 of a float64
 * evaluation (max|delta| / max|ref|).  The SwiGLU product is saturated to +-65504
 * before its fp16 rounding.
 *
 * Conventions shared by every call.
 *   - "dev" pointers are device (HBM) addresses, "host" pointers are host memory.
 *   - The caller owns every buffer: weights, arenas, cache, workspace, inputs and
 *     outputs.  The library never allocates device memory.  A context borrows the
 *     arenas and the stream until prefill_free().
 *   - Work is enqueued on the caller's hipStream_t (passed as void*); calls that return
 *     data to the host synchronise that stream.
 *   - Every call returns CP_OK (0) or a negative CP_E_* code and never aborts on bad
 *     input.  Validation happens on the host before anything is enqueued, so a rejected
 *     call leaves the context (its cache and n_past) exactly as it was; the pages ask
 *     that a failure leave a working context with its cache intact ("llama : switch the
 *     split mode of a live context", section "What this adds"; "completion : allow the
 *     prompt ...", section "Memory": an allocation failure is reported, not asserted).
 *   - A context is thread-compatible, not thread-safe.
 *
 * q8_0 interchange layout (how weights are handed in).  A matrix [N_out][K_in] is
 * row-major; each row is ceil(K_in/32) blocks of 34 bytes: a little-endian fp16 scale
 * d, then 32 int8 values q; value = float(d) * q.  Rows with K_in % 32 != 0 are
 * zero-padded to the next multiple of 32.  prefill_init() repacks these bytes into its
 * own arena layout; the interchange copies may be freed after it returns.
 */
#ifndef CHUNK_PREFILL_H
#define CHUNK_PREFILL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum cp_status {
  CP_OK = 0,
  CP_E_INVALID = -1,   /* bad argument: NULL pointer, unsupported shape, bad size     */
  CP_E_CAPACITY = -2,  /* n_tokens > n_chunk_max, or n_past + n_tokens > n_ctx_max     */
  CP_E_STATE = -3,     /* serialized state does not match this context / is truncated */
  CP_E_DEVICE = -4,    /* a HIP runtime call failed (message in prefill_last_error)    */
  CP_E_ARENA = -5      /* caller buffer too small or misaligned (256-byte alignment)   */
};

enum cp_kv_type { CP_KV_F16 = 0, CP_KV_Q8_0 = 1 };

/* Model geometry and capacities.  Supported shapes: head_dim in {64, 128};
 * n_head % n_kv_head == 0 and n_head / n_kv_head <= 64; d_model % 128 == 0;
 * (n_head * head_dim) % 128 == 0; dense ffn_dim > 0 with n_expert == 0, or routed
 * experts with ffn_dim == 0, n_expert in [1, 256], 1 <= n_expert_used <=
 * min(n_expert, 16), expert_ffn_dim > 0.  Capacities: 1 <= n_ctx_max <= 2^24 with
 * (n_ctx_max rounded up to 64) * head_dim * 2 < 2^31 (one kv head's cache is addressed
 * with 32-bit byte offsets); 1 <= n_chunk_max <= n_ctx_max, with n_chunk_max * n_head *
 * head_dim <= 2^31 and, because the GEMMs address their fp16 input with 32-bit byte
 * offsets, n_chunk_max * W * 2 < 2^31 for the widest GEMM input row W = max(d_model,
 * n_head*head_dim, ffn_dim rounded up to 128) (and n_expert_used * expert_ffn_dim
 * rounded up to 128 for routed experts).  Each weight matrix holds fewer than 2^31
 * values (N * K < 2^31 for QKV, the output projection, the gate/up pair 2 * ffn_dim
 * rounded up to 128 by d_model, and one expert's gate/up pair), as the weight tiles are
 * addressed with 32-bit byte offsets.  Anything else is rejected with CP_E_INVALID
 * (cp_validate_config, cp_config_error). */
typedef struct cp_config {
  int32_t n_layer, d_model, n_head, n_kv_head, head_dim;
  int32_t ffn_dim;                                 /* dense FFN width; 0 for experts  */
  int32_t n_expert, n_expert_used, expert_ffn_dim; /* 0, 0, 0 for a dense FFN          */
  float rms_eps, rope_theta;                       /* RMSNorm epsilon, RoPE base       */
  int32_t kv_type;                                 /* CP_KV_F16 or CP_KV_Q8_0          */
  int32_t n_ctx_max;                               /* cache capacity in tokens         */
  int32_t n_chunk_max;                             /* largest chunk prefill_chunk takes */
} cp_config;

/* One layer's weights, as device pointers in the q8_0 interchange layout (above).
 *   wq [n_head*head_dim][d_model], wk/wv [n_kv_head*head_dim][d_model],
 *   wo [d_model][n_head*head_dim]; attn_norm / ffn_norm: float32 [d_model] gains.
 *   Dense:   w_gate, w_up [ffn_dim][d_model], w_down [d_model][ffn_dim].
 *   Experts: w_router [n_expert][d_model]; w_gate, w_up [n_expert][expert_ffn_dim]
 *            [d_model] and w_down [n_expert][d_model][expert_ffn_dim], experts stored
 *            one after another, each in the interchange layout. */
typedef struct cp_layer_weights {
  const void *wq, *wk, *wv, *wo;
  const float *attn_norm, *ffn_norm;
  const void *w_gate, *w_up, *w_down;
  const void *w_router;   /* NULL for a dense FFN */
} cp_layer_weights;

typedef struct cp_ctx cp_ctx;

/* Sizes (bytes) of the three caller-owned device arenas for a configuration, or 0 when
 * the configuration is invalid.  Host-only; no GPU needed. */
size_t cp_weights_arena_bytes(const cp_config* cfg);  /* repacked weights of all layers */
size_t cp_kv_bytes(const cp_config* cfg);             /* KV cache at n_ctx_max tokens   */
size_t cp_workspace_bytes(const cp_config* cfg);      /* per-chunk scratch + RoPE table */

/* Host-only check of a configuration: CP_OK or CP_E_INVALID (message via
 * cp_config_error()). */
int cp_validate_config(const cp_config* cfg);
const char* cp_config_error(const cp_config* cfg);

/* Create a context.  layers: host array of n_layer descriptors (device pointers inside).
 * weights_arena / kv_buf / workspace: device buffers of at least the sizes above,
 * 256-byte aligned.  hip_stream: the hipStream_t all work is enqueued on (NULL = the
 * default stream).  Repacks the weights into the arena and builds the RoPE table
 * (angles in float64, cos/sin rounded to float32) on that stream, then synchronises.
 * On success *out holds the context and n_past = 0. */
int prefill_init(const cp_config* cfg, const cp_layer_weights* layers, void* weights_arena,
                 void* kv_buf, void* workspace, void* hip_stream, cp_ctx** out);

/* Process one chunk of n_tokens rows at positions n_past .. n_past+n_tokens-1.
 * x_in, x_out: dev float32 [n_tokens][d_model] row-major, 16-byte aligned (else
 * CP_E_INVALID, nothing enqueued); x_out may equal x_in.
 * Every layer appends the chunk's K/V (post-RoPE K) to its cache, then attends to cache
 * rows 0 .. n_past+n_tokens-1 ("append, then attend").  Requires 1 <= n_tokens <=
 * n_chunk_max and n_past + n_tokens <= n_ctx_max (else CP_E_CAPACITY, nothing
 * enqueued).  Returns once the work is enqueued; n_past advances by n_tokens. */
int prefill_chunk(cp_ctx* ctx, const float* x_in, float* x_out, int32_t n_tokens);

/* A prompt of n_tokens rows read in consecutive chunks of `chunk` tokens (the last one
 * shorter): the work of calling prefill_chunk for each chunk in turn, with up to n_lanes
 * chunks in flight on one device.  This is the
 * lane scheme of the llama.cpp "--split-overlap" pull request (section "How"):
 * consecutive chunks alternate between lanes, each with its own stream and its own
 * per-chunk buffers, sharing the weights and the KV cache, and a lane's step waits by
 * event only for the other lanes' work on the cache it reads.  There two lanes hide a
 * multi-device AllReduce; on one device the lanes let each chunk fill the compute units
 * the others leave idle (launch tails, small kernels, the gaps between launches).
 * Chunk i runs on lane i % n_lanes (lane 0 is the context's stream and workspace), its
 * layers in order; its layer l starts once chunk i-1 has finished layer l, whose cache
 * rows it attends to, so while one chunk runs layer l the next runs layer l-1.  With two
 * or more lanes the kernels take launch plans sized for a shared device (the GEMMs of
 * chunks above 128 tokens at most two K splits, attention of 64+ workgroups no KV splits;
 * see cp_test_set_plan_shared), so the result equals prefill_chunk per chunk up to the
 * order of split sums, and bitwise equals prefill_chunk per chunk under the shared plans.
 *   x_in, x_out: dev float32 [n_tokens][d_model], 16-byte aligned; x_out may equal x_in.
 *   n_lanes: 1 .. 8 (1: prefill_chunk for each chunk in turn, with the context's plans).
 *   workspaces[j], hip_streams[j] (j < n_lanes - 1): lane j+1's buffers (dev,
 *     cp_workspace_bytes(cfg) bytes each, 256-byte aligned; the context's own workspace
 *     keeps the RoPE tables) and stream (not the context's, all distinct, default
 *     priority); caller-owned, borrowed for the call's work.  May be NULL for one lane.
 * Requires 1 <= chunk <= n_chunk_max and n_past + n_tokens <= n_ctx_max (else
 * CP_E_CAPACITY), n_tokens >= 1, distinct streams and the alignments (else CP_E_INVALID /
 * CP_E_ARENA); every check is made before anything is enqueued.  Returns once the work is
 * enqueued; work enqueued later on the context's stream runs after all of it.  n_past
 * advances by n_tokens. */
int prefill_chunks(cp_ctx* ctx, const float* x_in, float* x_out, int32_t n_tokens, int32_t chunk,
                   int32_t n_lanes, void* const* workspaces, void* const* hip_streams);

/* prefill_chunk for callers that cannot allocate device memory at the call (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation): the
 * chunk's per-chunk buffers (normed rows, projections, attention output, FFN
 * intermediate, split-K and split-KV partial sums, routing tables) are taken from a
 * static device array of 256 MiB inside the library instead of the context's workspace,
 * whose RoPE tables are still read.  Same arguments, checks, kernels and result as
 * prefill_chunk (bitwise, whenever the chunk's split-KV partials fit beside the other
 * buffers; else attention runs unsplit, the same to rounding).  Allocates nothing: no
 * hipMalloc, hipFree or allocating library call.
 *   - The array holds the buffers of one chunk of exactly n_tokens rows; a chunk whose
 *     buffers exceed 256 MiB (e.g. more than about 600 rows at d_model 5120, FFN 17408)
 *     is rejected with CP_E_CAPACITY before anything is enqueued, and the context is
 *     unchanged (prefill_last_error says why).
 *   - One array per device, held from the library's load until the process ends.  Every
 *     call on a device shares it, and it keeps the last call's contents (nothing in it
 *     needs to start at zero): calls that overlap on one device (two streams, or two
 *     host threads) race and give wrong results.  Serialise them.
 *   - The device is the one current at prefill_init.
 * Returns as prefill_chunk, and CP_E_DEVICE if the array's address cannot be found. */
int prefill_chunk_static(cp_ctx* ctx, const float* x_in, float* x_out, int32_t n_tokens);

/* Same as prefill_chunk, then synchronises and writes the time of each layer (ms,
 * hipEvents recorded on the stream at every layer boundary) to host layer_ms[n_layer].
 * This is the per-layer t(C, D) the b + a*C cost model is fitted to ("Prompt chunks
 * sized for a layer split's pipeline", sections "Summary" and "What changed"). */
int prefill_chunk_timed(cp_ctx* ctx, const float* x_in, float* x_out, int32_t n_tokens,
                        float* layer_ms);

/* Same as prefill_chunk, and also copies, after every layer l, the residual stream of the
 * chunk to layer_out + l*layer_stride (dev float32 [n_tokens][d_model], NULL to skip) and,
 * for routed experts, the selected expert indices to route_idx + l*route_stride (dev int32
 * [n_tokens][n_expert_used], NULL to skip).  For checking each layer on its own. */
int prefill_chunk_trace(cp_ctx* ctx, const float* x_in, float* x_out, int32_t n_tokens,
                        float* layer_out, int64_t layer_stride, int32_t* route_idx,
                        int64_t route_stride);

/* Serialized, layout-independent KV state ("completion : allow the prompt to be
 * processed under its own split mode", section "What this does"; "llama : switch the
 * split mode of a live context", section "What this adds", step 1).  Little-endian:
 *   magic "CPKV", u32 version 1, u32 kv_type, u32 n_layer, u32 n_kv_head, u32 head_dim,
 *   u32 n_tokens, f32 rope_theta (32-byte header), then for every layer K then V, each
 *   n_tokens x n_kv_head rows in token-major order; an f16 row is head_dim binary16
 *   values, a q8_0 row is head_dim/32 blocks {fp16 d; int8 q[32]}.  K is post-RoPE.
 * The form depends on none of n_ctx_max, n_chunk_max or the device layout.
 *
 * kv_cache_get_state: dst = host buffer of cap bytes, or NULL to query the size.  Writes
 * the first n_past tokens; *n_bytes = blob size.  CP_E_ARENA if cap is too small.
 * Synchronises the stream; stages through the workspace. */
int kv_cache_get_state(cp_ctx* ctx, void* dst, size_t cap, size_t* n_bytes);

/* Restore a blob from host memory.  The whole header (magic, version, kv_type, n_layer,
 * n_kv_head, head_dim, rope_theta) and the exact length are validated against the
 * context first; on any mismatch, or n_tokens > n_ctx_max, returns CP_E_STATE and the
 * previous cache and n_past are untouched.  On success n_past = n_tokens.  The bytes a
 * following kv_cache_get_state returns are identical to src.  Synchronises the stream. */
int kv_cache_set_state(cp_ctx* ctx, const void* src, size_t n_bytes);

/* Host-only: the argument checks prefill_chunk (and its _timed / _trace forms) makes
 * before enqueuing anything, for a context of configuration cfg at n_past: CP_E_INVALID
 * for a NULL or not 16-byte aligned x_in / x_out (or an invalid cfg, n_past < 0),
 * CP_E_CAPACITY for n_tokens outside [1, n_chunk_max] or n_past + n_tokens > n_ctx_max,
 * else CP_OK.  The pointers are only inspected, never dereferenced. */
int cp_chunk_check(const cp_config* cfg, int32_t n_past, const float* x_in, const float* x_out,
                   int32_t n_tokens);

/* Host-only header check of a blob against a configuration (the same validation
 * kv_cache_set_state does before touching the cache). */
int cp_state_check(const cp_config* cfg, const void* src, size_t n_bytes);
size_t cp_state_bytes(const cp_config* cfg, int32_t n_tokens);

/* Forget cache rows n_keep .. n_past-1 (0 <= n_keep <= n_past): n_past = n_keep.  Rows
 * at or beyond n_past are scratch and are overwritten by the next chunk. */
int kv_cache_truncate(cp_ctx* ctx, int32_t n_keep);

int32_t prefill_n_past(const cp_ctx* ctx);
const char* prefill_last_error(const cp_ctx* ctx);
void prefill_free(cp_ctx* ctx);   /* releases host-side state only; buffers stay the caller's */

/* The launch plans (GEMM K splits, attention KV splits) of later prefill_chunk /
 * prefill_chunk_trace / prefill_chunk_timed calls on this context: shared = 1 takes the
 * plans prefill_chunks uses with several lanes (sized for a device shared with other
 * chunks in flight), 0 (the default) the single-lane plans.  Both give the same result up
 * to the order of the split sums; a
 * chunk's result under one plan is bitwise the same whether or not other chunks run
 * beside it.  CP_E_INVALID for a NULL context or shared outside {0, 1}. */
int cp_test_set_plan_shared(cp_ctx* ctx, int32_t shared);

/* Per-kernel timing.  classes: NULL turns timing off; "*" times every kernel class; else
 * a comma-separated list of class names.  While on, every launch of a selected class is
 * bracketed by hipEvents on the context's stream; cp_kernel_times() synchronises and
 * returns the summed duration (ms) and launch count since the last cp_kernel_timing()
 * call.  Classes: "gemm_qkv", "gemm_o", "gemm_gate_up", "gemm_down", "attention",
 * "rope_kv_append", "rmsnorm", "moe_route", "moe_permute", "moe_gemm_gate_up",
 * "moe_gemm_down", "moe_unpermute".  A dense GEMM class runs as one or two launches over
 * column ranges; each launch is also its own class, "<gemm class>/full" for an unsplit
 * range (one kernel launch), "<gemm class>/split" for a split-K range (the partial
 * GEMM and its ordered reduce), e.g. "gemm_gate_up/full", and "<gemm class>/skinny" for
 * the weight-streaming kernel that takes chunks of at most 4 tokens (with its reduce
 * when it splits K). */
int cp_kernel_timing(cp_ctx* ctx, const char* classes);
int cp_kernel_times(cp_ctx* ctx, const char* kernel_class, float* total_ms, int32_t* launches);

/* Logits of the last prompt position, the step after prefill: y = RMSNorm(x_row) * gain
 * (float32, eps inside the square root), logits[v] = sum_b d_vb * sum_j q_vbj * y_32b+j
 * over a q8_0 LM head (float32 accumulation).  The prefill planner page checks chunked
 * against unchunked prefill by the logits at the last prompt position ("refactor: one
 * prefill planner and one pad-trim hook for CLI and server", sections "Current Behavior"
 * and "Acceptance Criteria").
 *   x_row: dev float32 [d_model] (e.g. the last row of prefill_chunk's x_out);
 *   norm_gain: dev float32 [d_model];
 *   lm_head: dev q8_0 interchange [vocab][d_model/32 x 34 bytes], 2-byte aligned;
 *   logits: dev float32 [vocab].
 * d_model % 32 == 0 and <= 32768.  The head streams at close to the HBM rate when
 * d_model % 256 == 0 and lm_head is 16-byte aligned (rows are then whole 16-byte chunks);
 * other heads take a slower per-block path with the same result to float32 rounding.
 * Enqueued on hip_stream.  Returns CP_OK, CP_E_INVALID for bad arguments, CP_E_DEVICE if
 * the launch fails.  No allocation, no state. */
int cp_last_logits(const float* x_row, const float* norm_gain, const void* lm_head, int32_t vocab,
                   int32_t d_model, float eps, float* logits, void* hip_stream);

/* Chunk size for an n_tokens prompt read over `stages` layer-split pipeline stages, from a
 * layer's fitted cost per chunk b and per token a (as b/a, in tokens): "Prompt chunks sized
 * for a layer split's pipeline", sections "Summary" and "What changed".  A prompt in chunks
 * of C over S stages takes (S - 1 + n/C) chunk-steps of (b + a*C), least at
 * C0 = sqrt(n * (b/a) / (S - 1)); C0 is rounded up to a multiple of 256 and kept within
 * [512, cap], then evened over the k = ceil(n / C0) chunks it takes:
 * C = min(cap, roundup_256(ceil(n / k))).  A prompt that fits one chunk, and a single stage
 * (S = 1), take min(n, cap).  Host only.  Returns the chunk (0 for n = 0), or CP_E_INVALID
 * for n < 0, cap < 1, stages < 1 or a b/a that is not a positive finite number. */
int32_t cp_plan_chunk(int32_t n_tokens, int32_t cap, int32_t stages, double b_over_a);

/* The roofline's denominators, measured on this device (bench reports against both these
 * and the published 2.5 PFLOP/s dense fp16 / 8 TB/s HBM figures).  Runs, on hip_stream and
 * synchronising it:
 *   - an MFMA-only kernel: fp16 32x32x16 MFMAs on register operands, four independent
 *     accumulators per wave, 2048 workgroups of 4 waves, no memory traffic -> *mfma_tflops;
 *   - a streaming read of read_buf (dev, 16-byte aligned, read_bytes a multiple of 16 and at
 *     least 16 MiB; contents ignored) with 16-byte loads, three passes after a warm-up
 *     -> *hbm_gbs.
 * sink: dev scratch of at least cp_peak_sink_bytes() bytes (overwritten).  Returns CP_OK,
 * CP_E_INVALID for bad arguments, CP_E_DEVICE if a HIP call fails. */
size_t cp_peak_sink_bytes(void);
int cp_measure_peaks(const void* read_buf, size_t read_bytes, void* sink, size_t sink_bytes,
                     void* hip_stream, double* mfma_tflops, double* hbm_gbs);

/* q8_0 encode of float32 rows into the interchange layout, on the GPU (used to build
 * seeded weights in device memory).  x: dev float32 [rows][ldx], first k columns used;
 * out: dev bytes [rows][ceil(k/32)*34].  Per block of 32: d = amax/127 (float32,
 * correctly rounded), q = round-half-away-from-zero(x * (1/d)), stored d = fp16 (RNE);
 * values beyond k count as 0.  The amax is a wavefront reduction over the block. */
int cp_quantize_q8_0(const float* x, int64_t rows, int32_t k, int64_t ldx, void* out,
                     void* hip_stream);

/* ----------------------------------------------------------------------------------
 * Test exports: each runs one kernel of the path on caller buffers, so that a test can
 * feed it the oracle's inputs and compare the outputs bit for bit or to tolerance.
 * All pointers are device pointers unless stated; all are enqueued on hip_stream.
 * ---------------------------------------------------------------------------------- */

/* RoPE + K/V append for one chunk, exactly as prefill_chunk runs it.
 * qkv: float32 [n][(n_head + 2*n_kv_head)*head_dim] (q, then k, then v columns);
 * cos/sin: float32 [n_pos][head_dim/2] tables (rows = absolute positions);
 * q_out: f16 [n][n_head][head_dim] (RoPE applied); the rows are written at positions
 * start .. start+n-1 of a one-layer cache kv (layout as in cp_kv_bytes for n_layer = 1,
 * capacity n_ctx).  Read them back with cp_test_kv_rows. */
/* Bytes of a one-layer cache of capacity n_ctx (rounded up to 64 positions internally). */
size_t cp_test_kv_layer_bytes(int32_t n_kv_head, int32_t head_dim, int32_t n_ctx, int32_t kv_type);

int cp_test_rope_kv_append(const float* qkv, const float* cos_t, const float* sin_t,
                           int32_t n, int32_t start, int32_t n_head, int32_t n_kv_head,
                           int32_t head_dim, int32_t kv_type, int32_t n_ctx, void* q_out,
                           void* kv, void* hip_stream);

/* The same from the split planes of the QKV GEMM, as prefill_chunk runs it: the values
 * are partial[0] + partial[1] + ... + partial[splits-1] (float32, added in split order),
 * partial: float32 [splits][n][(n_head + 2*n_kv_head)*head_dim].  Chunks of up to four
 * tokens take the one-launch RoPE + append that reads the planes directly; larger ones
 * sum them first (into work: float32 [n][(n_head + 2*n_kv_head)*head_dim], dev, unused
 * otherwise but required).  CP_E_INVALID for splits < 1 and as cp_test_rope_kv_append. */
int cp_test_rope_kv_append_planes(const float* partial, int32_t splits, const float* cos_t,
                                  const float* sin_t, int32_t n, int32_t start, int32_t n_head,
                                  int32_t n_kv_head, int32_t head_dim, int32_t kv_type, int32_t n_ctx,
                                  void* q_out, void* kv, void* work, void* hip_stream);

/* Copy rows [0, n_tokens) of a one-layer cache into the serialized row form (K rows then
 * V rows, token-major, as in the state blob).  out: dev bytes. */
int cp_test_kv_rows(const void* kv, int32_t n_tokens, int32_t n_kv_head, int32_t head_dim,
                    int32_t kv_type, int32_t n_ctx, void* out, void* hip_stream);

/* Router logits (float32, fixed order: per 32-block ascending products and sums, then
 * scale-times-partial accumulated over blocks ascending, no fused multiply-add), top-k
 * (descending logit, ties to the lower expert index) and softmax weights over the k.
 * y: float32 [n][d]; w_router: q8_0 interchange [n_expert][d]; logits: float32
 * [n][n_expert]; idx: int32 [n][k]; weight: float32 [n][k]; scratch: dev buffer of
 * cp_test_router_scratch_bytes(n_expert, d) bytes (router weights unpacked). */
size_t cp_test_router_scratch_bytes(int32_t n_expert, int32_t d);
int cp_test_router(const float* y, const void* w_router, int32_t n, int32_t d, int32_t n_expert,
                   int32_t k, float* logits, int32_t* idx, float* weight, void* scratch,
                   void* hip_stream);

/* One q8_0 GEMM as the layer runs it: out = A * W^T with A fp16 [M][K] (lda = K,
 * K % 128 == 0), W in the interchange layout [N][K] (N % 32 == 0).  mode 0: out float32
 * [M][N] = result; mode 1: out float32 [M][N] += result; mode 2 (SwiGLU): W holds gate rows
 * then up rows ([2F][K], F % 32 == 0) and out is fp16 [M][F] = silu(gate) * up.  splits > 0
 * forces one launch with that split-K factor and a deterministic reduction (0 = the
 * layer's own launch plan, cp_test_gemm_plan).  scratch: dev
 * buffer of cp_test_gemm_scratch_bytes(M, N, K, splits) bytes (repacked weights and
 * partial sums). */
size_t cp_test_gemm_scratch_bytes(int32_t M, int32_t N, int32_t K, int32_t splits);
/* The launch plan the layer uses for an M x N x K GEMM (host only).  plan: 0 on a device of
 * its own; beside other chunks in flight (prefill_chunks with several lanes) 1, or 2 for a
 * GEMM whose split-K sums the next kernel adds as it reads them (the output and down
 * projections).  out6 = {row tile (1 = the weight-streaming kernel), number of launches,
 * first column of launch 0, its split-K factor, first column of launch 1, its split-K
 * factor}.  CP_E_INVALID for plan outside 0..2. */
int cp_test_gemm_plan(int32_t M, int32_t N, int32_t K, int32_t plan, int32_t* out6);
int cp_test_gemm(const void* A, const void* W, int32_t M, int32_t N, int32_t K, int32_t mode,
                 int32_t splits, void* out, void* scratch, void* hip_stream);
/* Same with the row tile pinned: row_tile 64 or 128 runs the kernel that keeps two
 * workgroups per CU, 256 the one-workgroup-per-CU kernel with the three-stage LDS
 * pipeline, 1 the weight-streaming kernel of 1-4 rows (M <= 4 and N % 64 == 0, else
 * CP_E_INVALID); 0 = the layer's own choice.  Scratch: cp_test_gemm_scratch_bytes_ex. */
size_t cp_test_gemm_scratch_bytes_ex(int32_t M, int32_t N, int32_t K, int32_t splits,
                                     int32_t row_tile);
int cp_test_gemm_ex(const void* A, const void* W, int32_t M, int32_t N, int32_t K, int32_t mode,
                    int32_t splits, int32_t row_tile, void* out, void* scratch, void* hip_stream);

/* Causal flash attention of a chunk against a one-layer cache (rows already appended):
 * q: f16 [n][n_head][head_dim]; kv: one-layer cache (capacity n_ctx) holding positions
 * 0 .. start+n-1; out: fp16 [n][n_head*head_dim].  kv_splits > 0 forces that many
 * KV-range splits (0 = the library's choice).  scratch: dev buffer of
 * cp_test_attention_scratch_bytes(...) bytes. */
size_t cp_test_attention_scratch_bytes(int32_t n, int32_t n_head, int32_t head_dim,
                                       int32_t kv_splits);
int cp_test_attention(const void* q, const void* kv, int32_t n, int32_t start, int32_t n_head,
                      int32_t n_kv_head, int32_t head_dim, int32_t kv_type, int32_t n_ctx,
                      int32_t kv_splits, void* out, void* scratch, void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* CHUNK_PREFILL_H */
