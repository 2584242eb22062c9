"""Full-size parity of the HIP path, in the launch configuration the benchmark times (GPU).

Each large workload runs at its real shapes, prompt length and chunk size through every
layer of its share.  The oracle cannot follow a whole 16-layer prefill of tens of
thousands of tokens in seconds, so the checks are:
  * layer 0 at sampled rows: the oracle evaluates the first layer at those rows from the
    same seeded prompt and the same interchange bytes (Oracle.layer_rows), and the GPU's
    layer-0 output there must agree to max|d|/max|ref| <= 1e-2;
  * layer 0's whole K/V cache (every position) against the oracle's, to the same bar;
  * properties that hold at any size: every layer's output is finite, a second run of
    the same chunks is bitwise identical, and the saved state restores byte-identically.
Layer 0's weights are encoded by the oracle; the deeper layers, which only the property
checks see, are generated and encoded on the GPU as the benchmark does.  The whole-prompt
runs take the GEMM launch plans of the benchmark's timed steps (a device shared by several
chunks in flight: cp_test_set_plan_shared), the chunk-size sweep those of its one-lane
sweep.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import log, need_gpu, rel_err, routing_agreement
from model_inputs import q8_layer_full

# the oracle's share of each case takes up to a minute on a 16-core host
pytestmark = [pytest.mark.gpu, pytest.mark.timeout(300)]

TOL = 1e-2          # max|delta| / max|ref|: fp16-operand MFMA, fp32 accumulate, against the oracle


@pytest.fixture(scope="module")
def torch():
    return need_gpu()


def gpu_layer(torch, cpa, w, l):
    """Layer l generated and q8_0-encoded on the GPU (norm gains all ones)."""
    lw = {}
    for name, shape in synth.weight_shapes(w):
        t = synth.layer_weight(w, l, name, shape, backend="torch", device="cuda")
        lw[name] = t if name.endswith("_norm") else cpa.cp_quantize_q8_0(t)
        del t
    return lw


def sample_rows(lo, hi, chunk, seed, n_random=24):
    """First rows, chunk boundaries, the last rows and seeded random rows in [lo, hi)."""
    rows = {lo, lo + 1, hi - 2, hi - 1}
    for s in range(lo + chunk, hi, chunk):
        rows |= {s - 1, s}
    g = np.random.Generator(np.random.PCG64(seed))
    rows |= set(int(r) for r in g.integers(lo, hi, size=n_random))
    return np.array(sorted(r for r in rows if lo <= r < hi), dtype=np.int64)


def layer0_kv_values(blob, n_tokens):
    """Layer 0's K and V values [n][Hkv][hd] float32 from a state blob (oracle parser)."""
    magic, ver, kvc, L, H, hd, n, theta = oracle.state.HEADER.unpack_from(blob, 0)
    assert n == n_tokens
    kv_type = "f16" if kvc == 0 else "q8_0"
    rb = oracle.row_bytes(hd, kv_type)
    body = blob[32:32 + 2 * n * H * rb]
    sub = oracle.state.HEADER.pack(magic, ver, kvc, 1, H, hd, n, theta) + body
    _, layers = oracle.parse_state(sub)
    k, v = layers[0]
    return oracle.cache_decode_rows(k, kv_type), oracle.cache_decode_rows(v, kv_type)


class FullRun:
    """The workload's whole share on the GPU; layer 0 from oracle-encoded bytes."""

    def __init__(self, torch, w, n_ctx, chunk_max, shared_plans=False):
        import chunked_prompt_prefill_amd as cpa
        self.torch, self.cpa, self.w = torch, cpa, w
        log(f"{w.name}: encoding layer 0 with the oracle")
        self.ql0 = q8_layer_full(w, 0)
        dev = [cpa.to_device(self.ql0)] + [gpu_layer(torch, cpa, w, l) for l in range(1, w.n_layer)]
        torch.cuda.synchronize()
        self.cfg = cpa.make_config(w, n_ctx, chunk_max)
        self.ctx = cpa.PrefillContext(self.cfg, dev)
        self.ctx.set_plan_shared(shared_plans)
        self.dev = dev

    def run(self, x_dev, out, chunks, lo=None, ro=None, n_total=0):
        w = self.w
        for s, e in chunks:
            if lo is None:
                self.ctx.prefill_chunk(x_dev[s:e], out[s:e])
            else:
                self.ctx.prefill_chunk_trace(
                    x_dev[s:e], out[s:e], lo[:, s:e], n_total * w.d_model,
                    None if ro is None else ro[:, s:e], n_total * w.n_expert_used if ro is not None else 0)
        self.torch.cuda.synchronize()


def check_layer0_rows(w, ql0, x, rows, got_rows, got_routes=None):
    """Oracle layer 0 at `rows` against the GPU's layer-0 output there; returns the oracle
    cache (rows 0 .. max(rows))."""
    m = oracle.OracleModel(w.with_(n_layer=1), [ql0])
    ref, cache = m.layer_rows(0, x, rows)
    ok = np.ones(len(rows), dtype=bool)
    if got_routes is not None:
        # every differing expert set must sit at a near tie of the oracle's logits; those
        # rows (if any) legitimately differ and are left out of the comparison
        r, own, _ = m.last_routing
        ok = routing_agreement(r, own, got_routes)
        log(f"  routing: {int(ok.sum())}/{len(rows)} sampled rows choose the oracle's set")
    e = rel_err(got_rows[ok], ref[ok])
    log(f"  layer 0 at {int(ok.sum())} sampled rows: max rel err {e:.3e}")
    assert e < TOL
    return cache


def check_layer0_cache(blob, cache, n_tokens):
    k, v = layer0_kv_values(blob, n_tokens)
    for name, got, ref in (("K", k, cache.kval[0][:n_tokens]), ("V", v, cache.vval[0][:n_tokens])):
        e = rel_err(got, ref)
        log(f"  layer 0 {name} cache over {n_tokens} positions: max rel err {e:.3e}")
        assert e < TOL


def whole_prompt(torch, w, kv_state_check=False):
    n, C = w.n_prompt, w.chunk
    log(f"{w.name}: {w.n_layer} layers, {n} tokens in chunks of {C}, {w.kv_type} cache")
    # the launch plans of the benchmark's timed steps (several chunks in flight)
    fr = FullRun(torch, w, n, C, shared_plans=True)
    x = synth.prompt_inputs(w)
    xd = torch.from_numpy(x).cuda()
    out = torch.empty_like(xd)
    lo = torch.empty((w.n_layer, n, w.d_model), dtype=torch.float32, device="cuda")
    ro = torch.empty((w.n_layer, n, w.n_expert_used), dtype=torch.int32, device="cuda") \
        if w.n_expert else None
    chunks = [(s, min(n, s + C)) for s in range(0, n, C)]
    fr.run(xd, out, chunks, lo, ro, n)
    assert fr.ctx.n_past == n
    assert bool(torch.isfinite(lo).all())
    assert torch.equal(lo[-1], out)
    rows = sample_rows(0, n, C, seed=n)
    got = lo[0][torch.from_numpy(rows).cuda()].cpu().numpy()
    routes = None if ro is None else ro[0][torch.from_numpy(rows).cuda()].cpu().numpy()
    del lo
    blob = fr.ctx.kv_cache_get_state()
    assert len(blob) == oracle.state_size(w.n_layer, w.n_kv_head, w.head_dim, n, w.kv_type)
    # the same chunks again: bitwise identical output and state
    out2 = torch.empty_like(xd)
    assert fr.ctx.kv_cache_truncate(0) == 0
    fr.run(xd, out2, chunks)
    assert torch.equal(out, out2)
    if kv_state_check:
        ctx2 = fr.cpa.PrefillContext(fr.cfg, fr.dev)
        ctx2.set_plan_shared(True)
        assert ctx2.kv_cache_set_state(blob) == 0 and ctx2.n_past == n
        assert ctx2.kv_cache_get_state() == blob
        log(f"  state of {len(blob)} bytes restores byte-identically")
        ctx2.close()
    assert fr.ctx.kv_cache_get_state() == blob
    fr.ctx.close()
    ql0 = fr.ql0
    del fr
    torch.cuda.empty_cache()
    return x, rows, got, routes, blob, ql0


def test_dense27b_f16_full_size(torch):
    w = synth.WORKLOADS["dense27b_f16"]
    x, rows, got, _, blob, ql0 = whole_prompt(torch, w)
    cache = check_layer0_rows(w, ql0, x, rows, got)
    check_layer0_cache(blob, cache, int(rows.max()) + 1)


def test_dense27b_q8_0_full_size_and_state(torch):
    w = synth.WORKLOADS["dense27b_q8"]
    x, rows, got, _, blob, ql0 = whole_prompt(torch, w, kv_state_check=True)
    cache = check_layer0_rows(w, ql0, x, rows, got)
    check_layer0_cache(blob, cache, int(rows.max()) + 1)


def test_moe_full_size(torch):
    w = synth.WORKLOADS["moe_a3b"]
    x, rows, got, routes, blob, ql0 = whole_prompt(torch, w)
    cache = check_layer0_rows(w, ql0, x, rows, got, routes)
    check_layer0_cache(blob, cache, int(rows.max()) + 1)


def test_sweep_shapes_every_chunk_size_at_depth(torch):
    """Four layers of the dense shapes: 16,384 positions prefilled in 8192-token chunks
    (the first of them the depth-0 8192-token chunk), then, after truncation back to
    16,384 each time, one chunk of every sweep size (128 ... 8192) at that depth, in the
    bench's launch plans, and decode-sized chunks of 1 and 3 tokens there (the
    weight-streaming GEMMs, the one-launch RoPE + append, split attention).  One oracle
    layer-0 evaluation at sampled rows serves all of them: the depth-0 chunk's rows, and
    for each size rows of [16,384, 16,384 + C)."""
    w = synth.WORKLOADS["dense27b_sweep"]
    D, sizes = w.depth_prefill, w.chunk_sweep
    Cmax = max(sizes)
    n = D + Cmax
    fr = FullRun(torch, w, n, Cmax)
    x = synth.prompt_inputs(w, n)
    xd = torch.from_numpy(x).cuda()
    out = torch.empty_like(xd)
    lo = torch.empty((w.n_layer, n, w.d_model), dtype=torch.float32, device="cuda")
    fr.run(xd, out, [(s, s + Cmax) for s in range(0, D, Cmax)], lo, None, n)
    rows0 = sample_rows(0, Cmax, Cmax, seed=Cmax)
    got = {0: lo[0][torch.from_numpy(rows0).cuda()].cpu().numpy()}
    rows = {0: rows0}
    decode = (1, 3)
    for C in decode + tuple(sizes):     # the largest last: the state below holds it
        assert fr.ctx.kv_cache_truncate(D) == 0
        lo[:, D:].zero_()
        fr.run(xd, out, [(D, D + C)], lo, None, n)
        assert bool(torch.isfinite(lo[:, D:D + C]).all())
        rows[C] = sample_rows(D, D + C, C, seed=C, n_random=8)
        got[C] = lo[0][torch.from_numpy(rows[C]).cuda()].cpu().numpy()
    blob = fr.ctx.kv_cache_get_state()      # the depth plus the last (largest) chunk
    fr.ctx.close()
    ql0 = fr.ql0
    del lo, fr
    torch.cuda.empty_cache()
    allrows = np.unique(np.concatenate(list(rows.values())))
    m = oracle.OracleModel(w.with_(n_layer=1), [ql0])
    ref, cache = m.layer_rows(0, x, allrows)
    for C in [0] + list(decode) + list(sizes):
        sel = np.searchsorted(allrows, rows[C])
        e = rel_err(got[C], ref[sel])
        log(f"  {'depth-0 chunk of ' + str(Cmax) if C == 0 else f'chunk {C} at depth {D}'}: "
            f"layer 0 at {len(sel)} sampled rows: max rel err {e:.3e}")
        assert e < TOL
    check_layer0_cache(blob, cache, int(allrows.max()) + 1)
