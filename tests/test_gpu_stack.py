"""Layer-stack parity, state and error paths of the HIP path through the C ABI (GPU)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import log, need_gpu, rel_err, routing_agreement, run_prefill
from model_inputs import q8_layers

pytestmark = pytest.mark.gpu

# Small configurations the library accepts (head_dim 64, d_model a multiple of 64), with
# FFN widths that are not multiples of 64 so the padding paths run.
GPU_DENSE = synth.Workload("gpu_tiny_dense", 2, 128, 4, 2, 64, 200, kv_type="f16",
                           n_prompt=150, chunk=37)
GPU_MOE = synth.Workload("gpu_tiny_moe", 2, 128, 4, 2, 64, 0, n_expert=8, n_expert_used=2,
                         expert_ffn_dim=96, kv_type="f16", n_prompt=150, chunk=37)
TOL = 1e-2   # max|delta| / max|ref| on hidden states, fp16-operand MFMA against the oracle


@pytest.fixture(scope="module")
def torch():
    return need_gpu()


def route_gap(r: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Per token: max logit outside idx minus min logit inside idx (<= 0 for an exact top-k)."""
    mask = np.zeros(r.shape, bool)
    np.put_along_axis(mask, idx.astype(np.int64), True, axis=1)
    inside = np.where(mask, r, np.inf).min(axis=1)
    outside = np.where(mask, -np.inf, r).max(axis=1)
    return outside - inside


def check_layers(w, qlayers, x, lo, ro, tol=TOL):
    """The GPU's output of every layer against the oracle's own layer-major run from the
    same seeded input (nothing the GPU produced is fed to the oracle).

    Routed layers: a GPU expert set may differ from the oracle's only at a near tie of the
    oracle's logits (gap below 1e-3 * max|r|); the hidden states are compared where both
    sides chose the same set, which the seeded inputs here make every token.  Returns the
    oracle's final output."""
    m = oracle.OracleModel(w, qlayers)
    ref_lo, routing = [], []
    ref = m.prefill_layer_major(x, layer_outputs=ref_lo, routing_out=routing)
    for l in range(w.n_layer):
        if ro is not None:
            r, own, _ = routing[l]
            same = routing_agreement(r, own, ro[l])
            log(f"  layer {l}: routing agreement {float(np.mean(same)):.5f}, "
                f"worst top-k gap {route_gap(r, ro[l]).max():.3e}")
            assert np.all(same), "expert sets differ at a near tie: compare per token instead"
        e = rel_err(lo[l], ref_lo[l])
        log(f"  layer {l}: max rel err {e:.3e}")
        assert e < tol
    return ref


@pytest.mark.parametrize("base", [GPU_DENSE, GPU_MOE])
@pytest.mark.parametrize("kv", ["f16", "q8_0"])
def test_stack_end_to_end_and_per_layer(torch, base, kv):
    w = base.with_(kv_type=kv)
    log(f"stack {w.name} kv={kv} n={w.n_prompt} chunk={w.chunk}")
    ql = q8_layers(w)
    x = synth.prompt_inputs(w)
    out, ctx, lo, ro = run_prefill(torch, w, ql, x, w.chunk, trace=True)
    assert ctx.n_past == w.n_prompt
    assert np.all(np.isfinite(out))
    ref = check_layers(w, ql, x, lo, ro)
    e = rel_err(out, ref)
    log(f"  end-to-end max rel err {e:.3e}")
    assert e < TOL


# Few experts and long chunks: 4 experts, top-2, chunks of 700 tokens (1400 token-slots,
# about 350 per expert), so the expert GEMMs run in 256-row tiles, several per expert,
# with a ragged last tile.
GPU_MOE_WIDE = synth.Workload("gpu_moe_wide", 2, 128, 4, 2, 64, 0, n_expert=4, n_expert_used=2,
                              expert_ffn_dim=96, kv_type="f16", n_prompt=1000, chunk=700)


def test_stack_routed_experts_in_256_row_tiles(torch):
    w = GPU_MOE_WIDE
    log(f"stack {w.name} n={w.n_prompt} chunk={w.chunk}")
    ql = q8_layers(w)
    x = synth.prompt_inputs(w)
    out, ctx, lo, ro = run_prefill(torch, w, ql, x, w.chunk, trace=True)
    assert np.all(np.isfinite(out))
    ref = check_layers(w, ql, x, lo, ro)
    e = rel_err(out, ref)
    log(f"  end-to-end max rel err {e:.3e}")
    assert e < TOL


def test_tiny_dense_workload_chunk_sizes(torch):
    """The 2-layer d=256 workload: 512 token ids read in chunks of 1, 3, 7, 128 and 512
    (1 and 3: every GEMM on the weight-streaming kernel, its counters reused launch after
    launch)."""
    w = synth.WORKLOADS["tiny_dense"]
    ql = q8_layers(w, gains="ones")
    x = synth.prompt_inputs(w)
    ref = oracle.OracleModel(w, ql).prefill_layer_major(x)
    outs = {}
    for chunk in (128, 1, 3, 7, 512):
        log(f"tiny_dense chunk={chunk}")
        out, ctx = run_prefill(torch, w, ql, x, chunk)
        outs[chunk] = out
        e = rel_err(out, ref)
        log(f"  max rel err {e:.3e}")
        assert e < TOL
    for c in (1, 3, 7, 512):
        assert rel_err(outs[c], outs[128]) < TOL


# a wide FFN (K = 2048 in the down projection) so that chunks of 1-4 rows split it as well
WIDE_FFN = synth.Workload("gpu_wide_ffn", 2, 256, 4, 2, 64, 2048, kv_type="f16", n_prompt=90, chunk=3)


@pytest.mark.parametrize("wname,chunks", [("tiny_dense", (37, 128, 512)), ("wide_ffn", (1, 3, 37))])
def test_deferred_split_sums_bitwise_equal_reduction_pass(torch, wname, chunks):
    """Chunks of every size leave the split-K sums of the output and down projections to
    the RMSNorm that reads them (the down sums cross into the next layer).  The traced
    entry point adds each layer's down sums in the reduction pass instead; the arithmetic
    and its order are the same, so outputs and cache state must agree bit for bit."""
    import chunked_prompt_prefill_amd as cpa
    w = synth.WORKLOADS["tiny_dense"] if wname == "tiny_dense" else WIDE_FFN
    ql = q8_layers(w)
    x = torch.from_numpy(synth.prompt_inputs(w)).cuda()
    n = x.shape[0]
    dev = [cpa.to_device(l) for l in ql]
    for chunk in chunks:
        plan = cpa.cp_test_gemm_plan(chunk, w.d_model, -(-w.ffn_dim // 128) * 128)
        log(f"deferred sums {wname} chunk={chunk} plan(down)={plan}")
        assert max(s for _, s in plan[1]) > 1          # the down projection is split
        a = cpa.PrefillContext(cpa.make_config(w, n, chunk), dev)
        b = cpa.PrefillContext(cpa.make_config(w, n, chunk), dev)
        ya, yb = torch.empty_like(x), torch.empty_like(x)
        lo = torch.empty((w.n_layer, chunk, w.d_model), dtype=torch.float32, device="cuda")
        for s0 in range(0, n, chunk):
            e0 = min(n, s0 + chunk)
            a.prefill_chunk(x[s0:e0], ya[s0:e0])
            b.prefill_chunk_trace(x[s0:e0], yb[s0:e0], lo[:, :e0 - s0], chunk * w.d_model)
        torch.cuda.synchronize()
        assert torch.equal(ya, yb)
        assert torch.equal(lo[-1, :n - (n - 1) // chunk * chunk], yb[(n - 1) // chunk * chunk:])
        assert a.kv_cache_get_state() == b.kv_cache_get_state()


def test_state_round_trip_restore_and_continuation(torch):
    import chunked_prompt_prefill_amd as cpa
    for kv in ("f16", "q8_0"):
        w = GPU_DENSE.with_(kv_type=kv)
        log(f"state kv={kv}")
        ql = q8_layers(w)
        x = synth.prompt_inputs(w, 150)
        dev = [cpa.to_device(l) for l in ql]
        cfg = cpa.make_config(w, 200, 64)
        a = cpa.PrefillContext(cfg, dev)
        b = cpa.PrefillContext(cpa.make_config(w, 300, 16), dev)   # other capacities
        xt = torch.from_numpy(x).cuda()
        ya = torch.empty_like(xt)
        a.prefill_chunk(xt[:64], ya[:64])
        a.prefill_chunk(xt[64:100], ya[64:100])
        blob = a.kv_cache_get_state()
        assert len(blob) == oracle.state_size(w.n_layer, w.n_kv_head, w.head_dim, 100, kv)
        assert b.kv_cache_set_state(blob) == 0 and b.n_past == 100
        assert b.kv_cache_get_state() == blob
        # continuation from the restored state is bitwise equal to continuing the original
        yb = torch.empty_like(xt)
        a.prefill_chunk(xt[100:150], ya[100:150])
        c = cpa.PrefillContext(cfg, dev)
        assert c.kv_cache_set_state(blob) == 0
        c.prefill_chunk(xt[100:150], yb[100:150])
        torch.cuda.synchronize()
        assert torch.equal(ya[100:150], yb[100:150])
        # an oracle-built blob restores into the GPU cache byte-identically
        m = oracle.OracleModel(w, ql)
        oc = m.new_cache(200)
        m.prefill(x[:77], 77, cache=oc)
        oblob = oracle.state_bytes(oc, w.rope_theta)
        assert c.kv_cache_set_state(oblob) == 0 and c.n_past == 77
        assert c.kv_cache_get_state() == oblob
        # mutated headers are rejected and leave the cache and n_past untouched
        for off in (0, 4, 8, 12, 16, 20, 24, 28):
            bad = bytearray(oblob)
            bad[off] ^= 0x41
            assert c.kv_cache_set_state(bytes(bad)) == -3
        assert c.kv_cache_set_state(oblob[:-1]) == -3
        assert c.n_past == 77 and c.kv_cache_get_state() == oblob


def test_determinism_truncate_and_error_paths(torch):
    import chunked_prompt_prefill_amd as cpa
    w = GPU_MOE
    ql = q8_layers(w)
    x = torch.from_numpy(synth.prompt_inputs(w, 120)).cuda()
    ctx = cpa.PrefillContext(cpa.make_config(w, 130, 64), [cpa.to_device(l) for l in ql])
    y1 = torch.empty_like(x)
    ctx.prefill_chunk(x[:64], y1[:64])
    ctx.prefill_chunk(x[64:120], y1[64:120])
    s1 = ctx.kv_cache_get_state()
    # rejected calls: nothing enqueued, n_past unchanged
    assert ctx.prefill_chunk_raw(x.data_ptr(), y1.data_ptr(), 65) == -2
    assert ctx.prefill_chunk_raw(x.data_ptr(), y1.data_ptr(), 0) == -2
    assert ctx.prefill_chunk_raw(x.data_ptr(), y1.data_ptr(), 11) == -2   # 120 + 11 > 130
    assert ctx.kv_cache_truncate(121) == -1
    assert ctx.n_past == 120
    # same chunks again after truncation: bitwise identical outputs and state
    assert ctx.kv_cache_truncate(0) == 0
    y2 = torch.empty_like(x)
    ctx.prefill_chunk(x[:64], y2[:64])
    ctx.prefill_chunk(x[64:120], y2[64:120])
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert ctx.kv_cache_get_state() == s1


@pytest.mark.parametrize("kv", ["f16", "q8_0"])
def test_prefix_resume_equals_full_prefill(torch, kv):
    """A prompt-cache hit: the state of a 64-token prefix restored into a fresh context (or
    the cache truncated back to it), then only the suffix prefilled.  With the same chunk
    boundaries the suffix outputs and the final state are bitwise those of the full
    prefill; with other boundaries they agree to the tolerance, and with the oracle."""
    import chunked_prompt_prefill_amd as cpa
    w = GPU_DENSE.with_(kv_type=kv)
    ql = q8_layers(w)
    x = synth.prompt_inputs(w, 150)
    dev = [cpa.to_device(l) for l in ql]
    cfg = cpa.make_config(w, 160, 64)
    xt = torch.from_numpy(x).cuda()
    bounds = [(0, 64), (64, 128), (128, 150)]
    full = cpa.PrefillContext(cfg, dev)
    y_full = torch.empty_like(xt)
    for s, e in bounds:
        full.prefill_chunk(xt[s:e], y_full[s:e])
    state_full = full.kv_cache_get_state()
    pre = cpa.PrefillContext(cfg, dev)
    y_pre = torch.empty_like(xt)
    pre.prefill_chunk(xt[:64], y_pre[:64])
    blob = pre.kv_cache_get_state()
    # restored prefix, same boundaries: bitwise
    hit = cpa.PrefillContext(cfg, dev)
    assert hit.kv_cache_set_state(blob) == 0 and hit.n_past == 64
    y_hit = torch.empty_like(xt)
    for s, e in bounds[1:]:
        hit.prefill_chunk(xt[s:e], y_hit[s:e])
    torch.cuda.synchronize()
    assert torch.equal(y_hit[64:], y_full[64:])
    assert hit.kv_cache_get_state() == state_full
    # truncation back to the prefix, same boundaries: bitwise
    assert full.kv_cache_truncate(64) == 0
    y_tr = torch.empty_like(xt)
    for s, e in bounds[1:]:
        full.prefill_chunk(xt[s:e], y_tr[s:e])
    torch.cuda.synchronize()
    assert torch.equal(y_tr[64:], y_full[64:])
    assert full.kv_cache_get_state() == state_full
    # restored prefix, the suffix in other chunks (40, 40, 6): within tolerance
    other = cpa.PrefillContext(cpa.make_config(w, 160, 40), dev)
    y_other = torch.empty_like(xt)
    assert other.kv_cache_set_state(blob) == 0
    for s, e in ((64, 104), (104, 144), (144, 150)):
        other.prefill_chunk(xt[s:e], y_other[s:e])
    torch.cuda.synchronize()
    ref = oracle.OracleModel(w, ql).prefill_layer_major(x)
    got = y_other.cpu().numpy()[64:]
    e1 = rel_err(got, y_full.cpu().numpy()[64:])
    e2 = rel_err(got, ref[64:])
    log(f"  prefix resume kv={kv}: other chunking vs full {e1:.3e}, vs oracle {e2:.3e}")
    assert e1 < TOL and e2 < TOL


def test_last_position_logits_chunked_and_unchunked(torch):
    """The tiny dense decoder's 512-token prompt read in chunks of 1, 7, 128 and 512: the
    last-position logits (RMSNorm + a q8_0 head of 4096 rows) agree with each other and with
    the oracle's."""
    import chunked_prompt_prefill_amd as cpa
    w = synth.WORKLOADS["tiny_dense"]
    ql = q8_layers(w, gains="ones")
    x = synth.prompt_inputs(w)
    head = oracle.q8_0_encode_bytes(synth.normal(synth.tensor_seed("lm_head", w.vocab, w.d_model),
                                                 (w.vocab, w.d_model)))
    gamma = np.ones(w.d_model, np.float32)
    ref = oracle.last_logits(oracle.OracleModel(w, ql).prefill_layer_major(x)[-1], gamma, head,
                             w.d_model, w.rms_eps)
    hd, gd = torch.from_numpy(head).cuda(), torch.from_numpy(gamma).cuda()
    outs = {}
    for chunk in (1, 7, 128, 512):
        out, ctx = run_prefill(torch, w, ql, x, chunk)
        row = torch.from_numpy(np.ascontiguousarray(out[-1])).cuda()
        outs[chunk] = cpa.cp_last_logits(row, gd, hd, w.vocab, w.rms_eps).cpu().numpy()
        e = rel_err(outs[chunk], ref)
        log(f"  chunk {chunk}: last logits max rel err {e:.3e}, argmax {int(np.argmax(outs[chunk]))} "
            f"(oracle {int(np.argmax(ref))})")
        assert e < TOL
    for c in (1, 7, 512):
        assert rel_err(outs[c], outs[128]) < TOL


@pytest.mark.parametrize("base", [GPU_DENSE, GPU_MOE])
@pytest.mark.parametrize("chunk", [3, 37])
def test_stack_with_zero_queries_matches_the_closed_form(torch, base, chunk):
    """W_q = 0 and W_down = 0: every layer is the residual plus the causal prefix mean of
    the cached V rows through W_o (see test_oracle_closed_form), a form evaluated here in
    numpy, not by the oracle."""
    from test_oracle_closed_form import closed_form, zero_q_and_down
    w = base.with_(kv_type="f16")
    log(f"closed-form stack {w.name} chunk={chunk}")
    ql = zero_q_and_down(q8_layers(w))
    x = synth.prompt_inputs(w)
    out, ctx = run_prefill(torch, w, ql, x, chunk)[:2]
    assert ctx.n_past == w.n_prompt
    ref = closed_form(w, ql, x)
    e = float(np.max(np.abs(out - ref)) / np.max(np.abs(ref - x)))
    log(f"  max|d| / max|attention term| = {e:.3e}")
    assert e < TOL
