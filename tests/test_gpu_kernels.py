"""Kernel-boundary parity: each HIP kernel fed the oracle's inputs (GPU)."""
import math

import numpy as np
import pytest

import oracle
import synth
from gpu_util import cache_row_bytes, log, need_gpu, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    return need_gpu()


@pytest.fixture(scope="module")
def cpa(torch):
    import chunked_prompt_prefill_amd as m
    from chunked_prompt_prefill_amd import prefill as p
    return p


# --------------------------------------------------------------------------- q8_0 encode
def special_rows(k):
    rows = []
    tie = np.zeros(k, np.float32)
    tie[:8] = [127.0, 2.5, -2.5, 0.5, -0.5, 1.5, -1.5, 126.5]
    rows.append(tie)
    rows.append(np.zeros(k, np.float32))
    sub = np.full(k, 3e-5, np.float32)
    sub[3] = -1.3e-4
    rows.append(sub)
    rows.append(np.full(k, -7.0, np.float32))
    big = synth.normal(99, (k,), scale=2.0e4)
    rows.append(big)
    return np.stack(rows)


@pytest.mark.parametrize("k", [32, 50, 2048, 5120])
def test_q8_0_encode_bit_exact(torch, cpa, k):
    x = np.concatenate([special_rows(k), synth.normal(k, (123, k), scale=0.02),
                        synth.uniform(k + 1, (40, k), -3, 3)]).astype(np.float32)
    log(f"q8_0 encode rows={x.shape[0]} k={k}")
    got = cpa.cp_quantize_q8_0(torch.from_numpy(x).cuda()).cpu().numpy()
    ref = oracle.q8_0_encode_bytes(x)
    assert got.shape == ref.shape
    assert np.array_equal(got, ref), f"{np.count_nonzero(got != ref)} bytes differ"


def test_q8_0_encode_bit_exact_weight_scale(torch, cpa):
    """A 5120 x 5120 weight matrix (one projection of the dense 27B-class layer)."""
    x = synth.normal(synth.tensor_seed("q8-stress"), (5120, 5120))
    got = cpa.cp_quantize_q8_0(torch.from_numpy(x).cuda()).cpu().numpy()
    assert np.array_equal(got, oracle.q8_0_encode_bytes(x))


# --------------------------------------------------------------------------- RoPE + append
@pytest.mark.parametrize("kv", ["f16", "q8_0"])
@pytest.mark.parametrize("hd,Hq,Hkv,n,start", [(64, 4, 2, 37, 5), (128, 8, 2, 130, 64),
                                               (128, 40, 8, 64, 1000), (64, 2, 2, 1, 0)])
def test_rope_kv_append_bit_exact(torch, cpa, kv, hd, Hq, Hkv, n, start):
    kv_code = 0 if kv == "f16" else 1
    n_ctx = start + n + 3
    log(f"rope_kv_append kv={kv} hd={hd} Hq={Hq} Hkv={Hkv} n={n} start={start}")
    qkv = synth.normal(synth.tensor_seed("qkv", hd, Hq, n), (n, (Hq + 2 * Hkv) * hd), scale=1.0)
    cos, sin = oracle.rope_table(n_ctx, hd, 1e6)
    q_out = torch.empty((n, Hq, hd), dtype=torch.float16, device="cuda")
    kvbuf = torch.zeros(cpa.cp_test_kv_layer_bytes(Hkv, hd, n_ctx, kv_code), dtype=torch.uint8,
                        device="cuda")
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    cpa.cp_test_rope_kv_append(T(qkv), T(cos), T(sin), n, start, Hq, Hkv, hd, kv_code, n_ctx,
                               q_out, kvbuf)
    rb = (hd * 2) if kv == "f16" else (hd // 32) * 34
    rows = torch.empty(2 * (start + n) * Hkv * rb, dtype=torch.uint8, device="cuda")
    cpa.cp_test_kv_rows(kvbuf, start + n, Hkv, hd, kv_code, n_ctx, rows)
    torch.cuda.synchronize()
    rows = rows.cpu().numpy().reshape(2, start + n, Hkv, rb)[:, start:]
    # oracle
    q = qkv[:, :Hq * hd].reshape(n, Hq, hd)
    k = qkv[:, Hq * hd:(Hq + Hkv) * hd].reshape(n, Hkv, hd)
    v = qkv[:, (Hq + Hkv) * hd:].reshape(n, Hkv, hd)
    cs, sn = cos[start:start + n], sin[start:start + n]
    q32 = oracle.rope_apply_f32(q, cs, sn)
    k32 = oracle.rope_apply_f32(k, cs, sn)
    assert np.array_equal(q_out.cpu().numpy().view(np.uint16), q32.astype(np.float16).view(np.uint16))
    kref = cache_row_bytes(oracle.cache_encode_rows(k32, kv), kv)
    vref = cache_row_bytes(oracle.cache_encode_rows(v, kv), kv)
    assert np.array_equal(rows[0], kref), "K rows differ"
    assert np.array_equal(rows[1], vref), "V rows differ"


# The same from the QKV GEMM's split planes, as prefill_chunk runs it: chunks of up to four
# tokens through the one-launch RoPE + append reading the planes, a larger one through the
# split-K reduction first.  The planes' float32 sum in split order is formed on the host
# and the result must match the oracle on it bit for bit, as above.
@pytest.mark.parametrize("kv", ["f16", "q8_0"])
@pytest.mark.parametrize("hd,Hq,Hkv,n,start,splits", [(128, 40, 8, 1, 17000, 7), (128, 40, 8, 3, 100, 3),
                                                      (64, 4, 2, 4, 0, 1), (128, 8, 2, 2, 63, 16),
                                                      (128, 40, 8, 5, 700, 3)])
def test_rope_kv_append_from_split_planes_bit_exact(torch, cpa, kv, hd, Hq, Hkv, n, start, splits):
    kv_code = 0 if kv == "f16" else 1
    n_ctx = start + n + 3
    W = (Hq + 2 * Hkv) * hd
    log(f"rope_kv_append planes kv={kv} hd={hd} Hq={Hq} Hkv={Hkv} n={n} start={start} splits={splits}")
    planes = synth.normal(synth.tensor_seed("qkv-planes", hd, Hq, n, splits), (splits, n, W), scale=0.5)
    qkv = planes[0].copy()
    for k in range(1, splits):
        qkv = (qkv + planes[k]).astype(np.float32)
    cos, sin = oracle.rope_table(n_ctx, hd, 1e6)
    q_out = torch.empty((n, Hq, hd), dtype=torch.float16, device="cuda")
    kvbuf = torch.zeros(cpa.cp_test_kv_layer_bytes(Hkv, hd, n_ctx, kv_code), dtype=torch.uint8,
                        device="cuda")
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    cpa.cp_test_rope_kv_append_planes(T(planes), splits, T(cos), T(sin), n, start, Hq, Hkv, hd,
                                      kv_code, n_ctx, q_out, kvbuf)
    rb = (hd * 2) if kv == "f16" else (hd // 32) * 34
    rows = torch.empty(2 * (start + n) * Hkv * rb, dtype=torch.uint8, device="cuda")
    cpa.cp_test_kv_rows(kvbuf, start + n, Hkv, hd, kv_code, n_ctx, rows)
    torch.cuda.synchronize()
    rows = rows.cpu().numpy().reshape(2, start + n, Hkv, rb)[:, start:]
    q = qkv[:, :Hq * hd].reshape(n, Hq, hd)
    k = qkv[:, Hq * hd:(Hq + Hkv) * hd].reshape(n, Hkv, hd)
    v = qkv[:, (Hq + Hkv) * hd:].reshape(n, Hkv, hd)
    cs, sn = cos[start:start + n], sin[start:start + n]
    q32 = oracle.rope_apply_f32(q, cs, sn)
    k32 = oracle.rope_apply_f32(k, cs, sn)
    assert np.array_equal(q_out.cpu().numpy().view(np.uint16), q32.astype(np.float16).view(np.uint16))
    assert np.array_equal(rows[0], cache_row_bytes(oracle.cache_encode_rows(k32, kv), kv)), "K rows differ"
    assert np.array_equal(rows[1], cache_row_bytes(oracle.cache_encode_rows(v, kv), kv)), "V rows differ"


# --------------------------------------------------------------------------- GEMM
def f16_round(a: np.ndarray) -> np.ndarray:
    return a.astype(np.float16).astype(np.float32)


def gemm_bound(A, Wd, ref, K, mode):
    """Per-element error bound of the fp16-operand GEMM: each dequantised weight is the
    correctly rounded fp16 of d*q (relative 2^-11, or 2^-25 absolute when it lands in the
    subnormal range), fp16 x fp16 products are exact in float32, and float32 accumulation
    over K terms adds (K+2) * 2^-24 of sum_k |a_k w_k|; mode 1 adds one final rounding."""
    a = np.abs(A.astype(np.float64))
    mag = a @ np.abs(Wd).T
    sub = a.sum(axis=1, keepdims=True) * 2.0 ** -25
    return ((2.0 ** -11 * 1.001 + (K + 2) * 2.0 ** -24) * mag + sub +
            (np.abs(ref) * 2.0 ** -23 if mode == 1 else 0))


# The planned launches; the last two shapes plan 256-row tiles with an unsplit column range
# and a split-K tail (ragged rows; a one-tile tail).
@pytest.mark.parametrize("M,N,K,splits", [(1, 256, 256, 0), (57, 512, 256, 0), (128, 5120, 512, 0),
                                          (300, 768, 2048, 1), (300, 768, 2048, 3), (513, 1024, 768, 0),
                                          (64, 7168, 5120, 0), (1000, 256, 17408, 0),
                                          (512, 7168, 5120, 0), (2048, 5120, 5120, 0),
                                          (300, 34816, 1024, 0), (512, 33024, 1280, 0)])
@pytest.mark.parametrize("mode", [0, 1])
def test_gemm_q8_0_within_f16_bound(torch, cpa, M, N, K, splits, mode):
    log(f"gemm M={M} N={N} K={K} splits={splits} mode={mode} plan={cpa.cp_test_gemm_plan(M, N, K)}")
    A = f16_round(synth.normal(synth.tensor_seed("A", M, K), (M, K), scale=1.0))
    W = synth.normal(synth.tensor_seed("W", N, K), (N, K))
    Wb = oracle.q8_0_encode_bytes(W)
    Wd = oracle.q8_0_decode_bytes(Wb, K).astype(np.float64)
    X0 = synth.normal(synth.tensor_seed("X0", M, N), (M, N), scale=1.0)
    out = torch.from_numpy(X0.copy() if mode == 1 else np.zeros((M, N), np.float32)).cuda()
    At = torch.from_numpy(A).cuda().to(torch.float16)
    cpa.cp_test_gemm(At, torch.from_numpy(Wb).cuda(), M, N, K, mode, splits, out)
    got = out.cpu().numpy().astype(np.float64)
    ref = A.astype(np.float64) @ Wd.T + (X0.astype(np.float64) if mode == 1 else 0.0)
    bound = gemm_bound(A, Wd, ref, K, mode)
    err = np.abs(got - ref)
    log(f"  max rel err {rel_err(got, ref):.3e}, worst err/bound {np.max(err / (bound + 1e-30)):.3f}")
    assert np.all(err <= bound + 1e-30)


@pytest.mark.parametrize("row_tile", [128, 256])
@pytest.mark.parametrize("M,N,K,splits", [(1, 256, 256, 0), (200, 512, 384, 0), (300, 768, 2048, 3),
                                          (513, 1024, 768, 0), (777, 1280, 1152, 5),
                                          (2048, 5120, 5120, 0), (256, 7168, 5120, 7)])
@pytest.mark.parametrize("mode", [0, 1])
def test_gemm_q8_0_row_tiles(torch, cpa, M, N, K, splits, mode, row_tile):
    """Both GEMM kernels with the row tile pinned: ragged M and N, K stage counts that are
    and are not multiples of the 256-row kernel's three-stage pipeline, split-K."""
    log(f"gemm row_tile={row_tile} M={M} N={N} K={K} splits={splits} mode={mode}")
    A = f16_round(synth.normal(synth.tensor_seed("A", M, K), (M, K), scale=1.0))
    W = synth.normal(synth.tensor_seed("W", N, K), (N, K))
    Wb = oracle.q8_0_encode_bytes(W)
    Wd = oracle.q8_0_decode_bytes(Wb, K).astype(np.float64)
    X0 = synth.normal(synth.tensor_seed("X0", M, N), (M, N), scale=1.0)
    out = torch.from_numpy(X0.copy() if mode == 1 else np.zeros((M, N), np.float32)).cuda()
    At = torch.from_numpy(A).cuda().to(torch.float16)
    cpa.cp_test_gemm(At, torch.from_numpy(Wb).cuda(), M, N, K, mode, splits, out, row_tile=row_tile)
    got = out.cpu().numpy().astype(np.float64)
    ref = A.astype(np.float64) @ Wd.T + (X0.astype(np.float64) if mode == 1 else 0.0)
    bound = gemm_bound(A, Wd, ref, K, mode)
    err = np.abs(got - ref)
    log(f"  max rel err {rel_err(got, ref):.3e}, worst err/bound {np.max(err / (bound + 1e-30)):.3f}")
    assert np.all(err <= bound + 1e-30)


# The weight-streaming kernel (row tile 1) of chunks of 1-4 tokens: every row count it
# templates (1, 2, and 3-4), K with fewer stages than waves and with many (several rounds
# per workgroup, one with a partial last round), the planned split count, one split, an
# uneven split and one stage per workgroup (idle waves), in the three epilogues.  Two calls must agree bit for bit (fixed summation order).
@pytest.mark.parametrize("M,N,K,splits", [(1, 64, 128, 0), (2, 5120, 640, 0), (3, 6144, 5120, 0),
                                          (4, 5120, 17408, 0), (1, 34816, 5120, 0), (3, 1024, 5120, 1),
                                          (4, 512, 2048, 3), (2, 256, 1024, 8), (2, 768, 1664, 1),
                                          (1, 5120, 17408, 0)])
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_gemm_skinny(torch, cpa, M, N, K, splits, mode):
    log(f"gemm skinny M={M} N={N} K={K} splits={splits} mode={mode}")
    A = f16_round(synth.normal(synth.tensor_seed("As", M, K), (M, K), scale=1.0))
    W = synth.normal(synth.tensor_seed("Ws", N, K), (N, K))
    Wb = oracle.q8_0_encode_bytes(W)
    Wd = oracle.q8_0_decode_bytes(Wb, K).astype(np.float64)
    At = torch.from_numpy(A).cuda().to(torch.float16)
    Wt = torch.from_numpy(Wb).cuda()
    F = N // 2
    X0 = synth.normal(synth.tensor_seed("X0s", M, N), (M, N), scale=1.0)
    outs = []
    for _ in range(2):
        if mode == 2:
            out = torch.zeros((M, F), dtype=torch.float16, device="cuda")
        else:
            out = torch.from_numpy(X0.copy() if mode == 1 else np.zeros((M, N), np.float32)).cuda()
        cpa.cp_test_gemm(At, Wt, M, N, K, mode, splits, out, row_tile=1)
        outs.append(out.float().cpu().numpy())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    got = outs[0].astype(np.float64)
    if mode == 2:
        g = A.astype(np.float64) @ Wd[:F].T
        u = A.astype(np.float64) @ Wd[F:].T
        ref = g / (1 + np.exp(-g)) * u
        e = rel_err(got, ref)
        log(f"  max rel err {e:.3e}")
        assert e < 1e-2
        return
    ref = A.astype(np.float64) @ Wd.T + (X0.astype(np.float64) if mode == 1 else 0.0)
    bound = gemm_bound(A, Wd, ref, K, mode)
    err = np.abs(got - ref)
    log(f"  max rel err {rel_err(got, ref):.3e}, worst err/bound {np.max(err / (bound + 1e-30)):.3f}")
    assert np.all(err <= bound + 1e-30)


@pytest.mark.parametrize("M,F,K,splits,row_tile", [(130, 128, 256, 0, 0), (77, 704, 256, 0, 0),
                                                   (512, 1024, 2048, 2, 0), (512, 17408, 5120, 0, 0),
                                                   (159, 17408, 5120, 0, 0), (300, 17408, 1024, 0, 0),
                                                   (300, 1024, 2048, 0, 256),
                                                   (2048, 2048, 1280, 0, 256), (600, 1536, 768, 4, 256)])
def test_gemm_swiglu(torch, cpa, M, F, K, splits, row_tile):
    log(f"gemm swiglu M={M} F={F} K={K} row_tile={row_tile} plan={cpa.cp_test_gemm_plan(M, 2 * F, K)}")
    A = f16_round(synth.normal(synth.tensor_seed("A", M, K), (M, K), scale=1.0))
    W = synth.normal(synth.tensor_seed("Wgu", F, K), (2 * F, K))
    Wb = oracle.q8_0_encode_bytes(W)
    Wd = oracle.q8_0_decode_bytes(Wb, K).astype(np.float64)
    out = torch.zeros((M, F), dtype=torch.float16, device="cuda")
    cpa.cp_test_gemm(torch.from_numpy(A).cuda().to(torch.float16), torch.from_numpy(Wb).cuda(),
                     M, 2 * F, K, 2, splits, out, row_tile=row_tile)
    got = out.float().cpu().numpy()
    g = A.astype(np.float64) @ Wd[:F].T
    u = A.astype(np.float64) @ Wd[F:].T
    ref = g / (1 + np.exp(-g)) * u
    e = rel_err(got, ref)
    log(f"  max rel err {e:.3e}")
    assert e < 1e-2


@pytest.mark.parametrize("row_tile", [128, 256])
def test_gemm_deterministic_split_k(torch, cpa, row_tile):
    M, N, K = 200, 5120, 5120
    A = torch.from_numpy(synth.normal(5, (M, K), scale=1.0)).cuda().to(torch.float16)
    Wb = torch.from_numpy(oracle.q8_0_encode_bytes(synth.normal(6, (N, K)))).cuda()
    outs = []
    for _ in range(2):
        o = torch.zeros((M, N), dtype=torch.float32, device="cuda")
        cpa.cp_test_gemm(A, Wb, M, N, K, 0, 4, o, row_tile=row_tile)
        outs.append(o.cpu().numpy())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))


# --------------------------------------------------------------------------- attention
def build_cache(torch, cpa, Hq, Hkv, hd, kv, T, seed, k_gain=None):
    """Cache rows for positions 0..T-1 written by the append kernel from seeded qkv rows;
    the oracle side re-derives the same rows itself.  k_gain: optional per-position factor
    on the K part of the rows."""
    kv_code = 0 if kv == "f16" else 1
    qkv = synth.normal(seed, (T, (Hq + 2 * Hkv) * hd), scale=1.0)
    if k_gain is not None:
        qkv[:, Hq * hd:(Hq + Hkv) * hd] *= np.asarray(k_gain, np.float32)[:, None]
    cos, sin = oracle.rope_table(T, hd, 1e6)
    q_out = torch.empty((T, Hq, hd), dtype=torch.float16, device="cuda")
    kvbuf = torch.zeros(cpa.cp_test_kv_layer_bytes(Hkv, hd, T, kv_code), dtype=torch.uint8, device="cuda")
    Tn = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    cpa.cp_test_rope_kv_append(Tn(qkv), Tn(cos), Tn(sin), T, 0, Hq, Hkv, hd, kv_code, T, q_out, kvbuf)
    q = qkv[:, :Hq * hd].reshape(T, Hq, hd)
    k = qkv[:, Hq * hd:(Hq + Hkv) * hd].reshape(T, Hkv, hd)
    v = qkv[:, (Hq + Hkv) * hd:].reshape(T, Hkv, hd)
    q32 = oracle.rope_apply_f32(q, cos, sin)
    k32 = oracle.rope_apply_f32(k, cos, sin)
    Kv = oracle.cache_decode_rows(oracle.cache_encode_rows(k32, kv), kv)
    Vv = oracle.cache_decode_rows(oracle.cache_encode_rows(v, kv), kv)
    qf16 = q32.astype(np.float16).astype(np.float64)
    return q_out, kvbuf, qf16, Kv, Vv


@pytest.mark.parametrize("kv", ["f16", "q8_0"])
@pytest.mark.parametrize("hd,Hq,Hkv,n,start,splits", [
    (64, 4, 2, 40, 0, 0), (64, 4, 2, 33, 100, 0), (128, 40, 8, 70, 300, 0),
    (128, 40, 8, 128, 700, 5), (128, 32, 4, 200, 0, 0), (128, 8, 8, 1, 250, 0),
    (128, 40, 8, 300, 1234, 1), (128, 40, 8, 256, 1000, 3), (64, 8, 2, 3, 900, 6),
    # decode-sized chunks: one token deep in the cache, three tokens, two tokens of a G = 8
    # model, head_dim 64 with a ragged last tile, the most forced splits (32) over few tiles
    (128, 40, 8, 1, 17000, 0), (128, 40, 8, 3, 5000, 0), (128, 32, 4, 2, 100, 0),
    (64, 4, 2, 8, 333, 0), (128, 40, 8, 2, 1000, 32),
    # 64, 60 and 65 query rows per kv head
    (128, 8, 2, 16, 2000, 0), (128, 40, 8, 12, 3000, 0), (64, 5, 1, 13, 700, 0)])
def test_attention_matches_oracle(torch, cpa, kv, hd, Hq, Hkv, n, start, splits):
    log(f"attention kv={kv} hd={hd} Hq={Hq} Hkv={Hkv} n={n} start={start} splits={splits}")
    T = start + n
    q_all, kvbuf, qf, Kv, Vv = build_cache(torch, cpa, Hq, Hkv, hd, kv, T, synth.tensor_seed("att", hd, Hq, T))
    q = q_all[start:].contiguous()
    out = torch.zeros((n, Hq * hd), dtype=torch.float16, device="cuda")
    cpa.cp_test_attention(q, kvbuf, n, start, Hq, Hkv, hd, 0 if kv == "f16" else 1, T, splits, out)
    got = out.float().cpu().numpy().reshape(n, Hq, hd)
    ref = oracle.attention(qf[start:], Kv, Vv, np.arange(start, T))
    e = rel_err(got, ref)
    log(f"  max rel err {e:.3e}")
    assert e < 1e-2
    assert np.all(np.isfinite(got))


@pytest.mark.parametrize("kv", ["f16", "q8_0"])
@pytest.mark.parametrize("n,bit", [(96, 8), (1, 8), (3, 8)])
def test_attention_keys_of_one_lane_half_dominate(torch, cpa, kv, n, bit):
    """Keys whose position has the given bit set get 8x larger K rows, so the scores one
    half of the lanes holds exceed the other half's by far more than fp16 can carry: the
    running maximum must combine both lane halves of each query row, which split each
    16-key group by bit 3 of the position; chunks of 96, 1 and 3 tokens."""
    hd, Hq, Hkv, start = 128, 40, 8, 160
    T = start + n
    gain = np.where((np.arange(T) & bit) != 0, 8.0, 1.0)
    log(f"attention kv={kv} n={n} with dominant keys at positions with bit {bit} set")
    q_all, kvbuf, qf, Kv, Vv = build_cache(torch, cpa, Hq, Hkv, hd, kv, T,
                                           synth.tensor_seed("att-half", T), k_gain=gain)
    q = q_all[start:].contiguous()
    for splits in (1, 3):
        out = torch.zeros((n, Hq * hd), dtype=torch.float16, device="cuda")
        cpa.cp_test_attention(q, kvbuf, n, start, Hq, Hkv, hd, 0 if kv == "f16" else 1, T, splits, out)
        got = out.float().cpu().numpy().reshape(n, Hq, hd)
        assert np.all(np.isfinite(got))
        ref = oracle.attention(qf[start:], Kv, Vv, np.arange(start, T))
        e = rel_err(got, ref)
        log(f"  splits {splits}: max rel err {e:.3e}")
        assert e < 1e-2


# --------------------------------------------------------------------------- router
# n <= 16 takes the wave-per-expert kernel (decode-sized chunks), larger n the
# token-tiled one; d = 8224 (257 blocks) sends a small n to the tiled kernel too.
@pytest.mark.parametrize("n,d,E,k", [(37, 2048, 128, 8), (5, 256, 8, 2), (64, 512, 256, 16),
                                     (1, 2048, 128, 8), (3, 2048, 128, 8), (16, 4096, 64, 4),
                                     (17, 4096, 64, 4), (2, 8224, 16, 2)])
def test_router_bit_exact(torch, cpa, n, d, E, k):
    log(f"router n={n} d={d} E={E} k={k}")
    y = synth.normal(synth.tensor_seed("y", n, d), (n, d), scale=1.0)
    W = synth.normal(synth.tensor_seed("wr", E, d), (E, d))
    W[E // 2] = W[1]            # identical experts: exact ties, lower index must win
    Wb = oracle.q8_0_encode_bytes(W)
    logits = torch.empty((n, E), dtype=torch.float32, device="cuda")
    idx = torch.empty((n, k), dtype=torch.int32, device="cuda")
    wt = torch.empty((n, k), dtype=torch.float32, device="cuda")
    cpa.cp_test_router(torch.from_numpy(y).cuda(), torch.from_numpy(Wb).cuda(), n, d, E, k, logits, idx, wt)
    d16, q = oracle.q8_0_from_bytes(Wb, d // 32)
    r = oracle.router_logits_ordered(y, d16, q)
    ridx, rw = oracle.moe_route(r, k)
    assert np.array_equal(logits.cpu().numpy().view(np.uint32), r.view(np.uint32))
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.allclose(wt.cpu().numpy(), rw, rtol=1e-5, atol=1e-7)


# --------------------------------------------------------------------------- last logits
# d % 256 == 0 with an aligned head: up to d = 5120 the row-pair kernel (an odd vocabulary
# ends on a single row), above it the streaming kernel (one and a half, four and eight
# segments of 128 blocks); d = 2080 and a head at an odd halfword offset take the
# per-block kernel.
@pytest.mark.parametrize("vocab,d,offset", [(4096, 5120, 0), (1000, 256, 0), (33, 2048, 0), (4097, 5120, 0),
                                            (77, 2080, 0), (65, 6144, 0), (129, 16384, 0), (40, 32768, 0),
                                            (300, 5120, 2)])
def test_last_logits_matches_oracle(torch, cpa, vocab, d, offset):
    """RMSNorm + q8_0 LM head on one row: float32 accumulation against the float64
    definition, to 1e-4 of the largest logit."""
    log(f"last logits vocab={vocab} d={d} head offset={offset}")
    x = synth.normal(synth.tensor_seed("xrow", d), (d,), scale=1.0)
    gamma = (1.0 + synth.normal(synth.tensor_seed("g", d), (d,))).astype(np.float32)
    head = oracle.q8_0_encode_bytes(synth.normal(synth.tensor_seed("head", vocab, d), (vocab, d)))
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    hbuf = torch.zeros(head.size + offset, dtype=torch.uint8, device="cuda")
    hbuf[offset:] = T(head.reshape(-1))
    got = cpa.cp_last_logits(T(x), T(gamma), hbuf[offset:], vocab, 1e-6).cpu().numpy()
    ref = oracle.last_logits(x, gamma, head, d, 1e-6)
    e = rel_err(got, ref)
    log(f"  max rel err {e:.3e}")
    assert e < 1e-4
