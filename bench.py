#!/usr/bin/env python3
"""Chunked prompt prefill benchmark on one MI355X.

A step is one full prefill of the workload's prompt from an empty cache: every chunk
through every layer of the GPU's share (RMSNorm, q8_0 QKV GEMM, RoPE + KV append,
causal GQA flash attention, output GEMM, SwiGLU FFN).  Weights and inputs are
synthetic N(0, 0.02) values of the workload's shapes, generated in device memory and
q8_0-encoded by the library.  Default workload: the dense 27B-class share of 16 layers
(d_model 5120, 40/8 heads, head_dim 128, SwiGLU 17408, f16 cache), a 17,055-token prompt
in 512-token chunks.

Also reported: the chunk-size sweep (4 layers, chunks 128..8192, depth 0 and 16,384)
with the per-layer cost fit t = b + a*C ("Prompt chunks sized for a layer split's
pipeline", sections "Summary" and "What changed"), the dominant kernel's roofline
fraction from HIP events around its launches, and the CPU oracle timed on a bounded
sample on this host.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-sweep] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_F16_TFLOPS = 2500.0    # MI355X dense fp16 / bf16 MFMA (same rate)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
DECODE_ROOM = 128           # cache positions past the prompt for the decode-sized chunks
LOGITS_VOCAB = 152064       # rows of the synthetic LM head of the last-logits measurement


def note(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def dense_params(w) -> int:
    d, hd = w.d_model, w.head_dim
    attn = (w.n_head + 2 * w.n_kv_head) * hd * d + d * w.n_head * hd
    if w.n_expert:
        return attn + w.n_expert * d + w.n_expert * 3 * w.expert_ffn_dim * d
    return attn + 3 * w.ffn_dim * d


def active_params(w) -> int:
    d, hd = w.d_model, w.head_dim
    attn = (w.n_head + 2 * w.n_kv_head) * hd * d + d * w.n_head * hd
    if w.n_expert:
        return attn + w.n_expert * d + w.n_expert_used * 3 * w.expert_ffn_dim * d
    return attn + 3 * w.ffn_dim * d


def chunk_flops(w, C: int, D: int) -> float:
    """Algorithmic flops of one chunk through one layer: 2*P_active*C plus the unmasked
    causal half of attention, 4*Hq*hd*(C*D + C(C+1)/2)."""
    return 2.0 * active_params(w) * C + 4.0 * w.n_head * w.head_dim * (C * D + C * (C + 1) / 2)


def chunk_bytes(w, C: int, D: int) -> float:
    """Algorithmic HBM bytes of one chunk-layer: q8_0 weights (all experts touched), K/V
    read over D + C positions, K/V write of C rows, x in and out."""
    e = 2.0 if w.kv_type == "f16" else 34.0 / 32.0
    kv = 2.0 * w.n_kv_head * w.head_dim * e
    return dense_params(w) * 34.0 / 32.0 + kv * (D + C) + kv * C + 2.0 * C * w.d_model * 4


def roofline_s(w, C, D):
    return max(chunk_flops(w, C, D) / (PEAK_F16_TFLOPS * 1e12),
               chunk_bytes(w, C, D) / (PEAK_HBM_GBS * 1e9))


def fit_linear(C, t):
    """Least-squares line t = b + a*C: returns (b, a, r2)."""
    import numpy as np
    C = np.asarray(C, dtype=np.float64)
    t = np.asarray(t, dtype=np.float64)
    a, b = np.polyfit(C, t, 1)
    res = t - (b + a * C)
    sst = float(np.sum((t - t.mean()) ** 2))
    return float(b), float(a), (1.0 - float(np.sum(res ** 2)) / sst) if sst > 0 else 1.0


def gpu_layers(w, torch, cpa, synth):
    layers = []
    for l in range(w.n_layer):
        lw = {}
        for name, shape in synth.weight_shapes(w):
            t = synth.layer_weight(w, l, name, shape, backend="torch", device="cuda")
            lw[name] = t if name.endswith("_norm") else cpa.cp_quantize_q8_0(t)
            del t
        layers.append(lw)
    torch.cuda.synchronize()
    return layers


def dominant_work(w, cpa, chunks):
    """Algorithmic work of the dominant kernel's launches in one pass over `chunks`.

    Dense: the SwiGLU gate/up GEMM of a chunk-layer as one operation: every column range
    of its launch plan, split or not, and the split-K reduction (the library's
    "gemm_gate_up" timing class brackets all of them with one pair of events).  Per chunk
    of M rows, N = 2 * FFN (padded to 128) columns of W_gate|W_up, K = d_model: flops
    2*M*N*K; bytes = q8_0 weights N*K*34/32 + A rows M*K*2 (fp16) + h written M*N/2*2.
    Routed experts: the grouped gate/up GEMM over the C*k token-slots, flops 2*C*k*2*Fe*d,
    bytes = every expert's gate/up weights + the gathered A rows + h.
    Returns (flops, bytes, per-launch figures of the full-size chunk)."""
    flops = bytes_ = 0.0
    launches = 0
    first = None
    for s, e in chunks:
        M = e - s
        if w.n_expert:
            Fe = w.expert_ffn_dim
            f = 2.0 * M * w.n_expert_used * 2 * Fe * w.d_model
            b = w.n_expert * 2 * Fe * w.d_model * 34 / 32 + M * w.n_expert_used * (w.d_model + Fe) * 2
        else:
            N = 2 * (-(-w.ffn_dim // 128) * 128)
            K = w.d_model
            f = 2.0 * M * N * K
            b = N * K * 34 / 32 + M * K * 2 + M * N // 2 * 2
        flops += f
        bytes_ += b
        launches += 1
        if first is None:
            first = {"flops": f, "bytes": b, "rows": M}
    first = dict(first or {"flops": 0.0, "bytes": 0.0, "rows": 0})
    first["launches"] = launches
    return flops, bytes_, first


def measured_traffic(kernel, per_launch):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3 PMC
    readings (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy's reading), or None when the
    readings are absent or were taken on another version of the kernel's source or under
    another launch plan."""
    import hashlib
    import chunked_prompt_prefill_amd as cpa
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    r = rec.get(kernel)
    if not r:
        return None
    h = hashlib.sha256()
    for src in r.get("sources", []):
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != r.get("sources_sha256") or r.get("rows") != per_launch.get("rows"):
        return None
    if r.get("plan") != plan_record(cpa):
        return None
    return r.get("hbm_bytes_per_launch")


# sources whose text defines the dominant kernel's code: a change to any of them, or to
# its launch plan at 512 rows (plan_record), makes the stored counter readings stale
# (measured_traffic then reports None)
PMC_SOURCES = ["chunked_prompt_prefill_amd/csrc/k_gemm_big.hip",
               "chunked_prompt_prefill_amd/csrc/k_gemm.hip",
               "chunked_prompt_prefill_amd/csrc/k_common.h",
               "chunked_prompt_prefill_amd/csrc/cp_internal.h"]


def plan_record(cpa):
    """The single-lane launch plan of the 512-row gate/up GEMM: [row tile, [[first column,
    split-K factor], ...]]."""
    mt, parts = cpa.cp_test_gemm_plan(512, 34816, 5120)
    return [mt, [list(p) for p in parts]]


def pmc_digest(fetch_csv, write_csv, copy_mib):
    """Fold two rocprofv3 --pmc counter files of the --pmc-probe run (FETCH_SIZE, then
    WRITE_SIZE; 512-token chunk) into profiles/pmc_traffic.json: the readings of the
    gate/up GEMM's dispatches (its unsplit launch, then, when the plan has a split-K
    column tail, the tail's launch and its reduction, in dispatch order), each scaled by
    what the same counter reads for the plain copy of copy_mib MiB that the probe runs
    first (the copy reads and writes exactly that many bytes)."""
    import csv
    import hashlib
    import chunked_prompt_prefill_amd as cpa
    _, parts = cpa.cp_test_gemm_plan(512, 34816, 5120)
    n_disp = len(parts) + (1 if any(sp > 1 for _, sp in parts) else 0)

    def readings(path):
        with open(path) as f:
            rows = sorted(csv.DictReader(f), key=lambda r: int(r["Dispatch_Id"]))
        copy = [float(r["Counter_Value"]) for r in rows if r["Kernel_Name"].startswith("__amd_rocclr_copyBuffer")]
        first = [i for i, r in enumerate(rows) if "gemm_q8_big_kernel<2, false>" in r["Kernel_Name"]]
        if not copy or len(first) != 1:
            raise SystemExit(f"{path}: expected the copy and one unsplit gate/up launch, got {len(copy)} / {len(first)}")
        op = rows[first[0]:first[0] + n_disp]
        def short(name):
            return name.rsplit("(", 1)[0].replace("void ", "").replace("cp::(anonymous namespace)::", "").replace("cp::", "")
        return copy[0], sum(float(r["Counter_Value"]) for r in op), [short(r["Kernel_Name"]) for r in op]

    cf, kf, names = readings(fetch_csv)
    cw, kw, _ = readings(write_csv)
    probe_kib = copy_mib * 1024
    ff, fw = probe_kib / cf, probe_kib / cw
    h = hashlib.sha256()
    for src in PMC_SOURCES:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    rec = {"gemm_gate_up": {
        "kernel": "the gate/up GEMM of a 512-token chunk-layer: " + " + ".join(names),
        "rows": 512, "fetch_size_kib": kf, "write_size_kib": kw,
        "copy_probe_bytes": probe_kib * 1024, "copy_fetch_size_kib": cf, "copy_write_size_kib": cw,
        "fetch_factor": ff, "write_factor": fw,
        "hbm_read_bytes_per_launch": kf * 1024 * ff, "hbm_write_bytes_per_launch": kw * 1024 * fw,
        "hbm_bytes_per_launch": kf * 1024 * ff + kw * 1024 * fw,
        "sources": PMC_SOURCES, "sources_sha256": h.hexdigest(), "plan": plan_record(cpa)}}
    with open(os.path.join(ROOT, "profiles", "pmc_traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def run_main(args, torch, cpa, synth):
    w = synth.WORKLOADS[args.workload]
    n, C = w.n_prompt, w.chunk
    note(f"workload {w.name}: {w.n_layer} layers, {n} tokens in {C}-token chunks, {w.kv_type} cache")
    t = time.time()
    layers = gpu_layers(w, torch, cpa, synth)
    # the context's own stream (not the default one, which would serialise with the
    # other lanes' streams); prefill_chunks adds a stream per further lane
    ctx = cpa.PrefillContext(cpa.make_config(w, n + DECODE_ROOM, C), layers, stream=torch.cuda.Stream())
    del layers
    torch.cuda.empty_cache()
    x = synth.prompt_inputs(w, backend="torch", device="cuda")
    out = torch.empty_like(x)
    torch.cuda.synchronize()          # inputs are read on the context's own streams
    note(f"weights generated, encoded and repacked in {time.time() - t:.1f}s")
    chunks = [(s, min(n, s + C)) for s in range(0, n, C)]

    def step():
        # the whole prompt in chunks of C, args.lanes chunks in flight on as many streams
        ctx.kv_cache_truncate(0)
        rc = ctx.prefill_chunks_raw(x.data_ptr(), out.data_ptr(), n, C, args.lanes)
        if rc != 0:
            raise RuntimeError(f"prefill_chunks failed: {rc} {ctx.last_error()}")

    def step_one_lane():
        # the same chunks one after another through prefill_chunk
        ctx.kv_cache_truncate(0)
        for s, e in chunks:
            rc = ctx.prefill_chunk_raw(x[s:e].data_ptr(), out[s:e].data_ptr(), e - s)
            if rc != 0:
                raise RuntimeError(f"prefill_chunk failed: {rc} {ctx.last_error()}")

    run_step = step if args.lanes > 1 else step_one_lane
    for i in range(args.warmup):
        run_step()
        torch.cuda.synchronize()
        note(f"warmup step {i + 1}/{args.warmup} done")
    # headline: K steps, args.lanes chunks in flight (prefill_chunks) unless --lanes 1
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run_step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    note(f"timed {args.steps} steps in {t1 - t0:.3f}s ({args.lanes} lane(s))")
    total = t1 - t0
    tps = n * args.steps / total
    # the dominant kernel's roofline, timed by HIP events around its launches over K more
    # steps on one lane, where each launch has the device to itself: the SwiGLU gate/up GEMM
    # of each chunk-layer as a whole (all of its launches and the reduction), or the
    # grouped expert gate/up GEMM of a routed FFN
    dom = "moe_gemm_gate_up" if w.n_expert else "gemm_gate_up"
    step_one_lane()
    ctx.cp_kernel_timing(dom)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for i in range(args.steps):
        step_one_lane()
    torch.cuda.synchronize()
    one_lane = n * args.steps / (time.perf_counter() - t2)
    dom_ms, dom_launches = ctx.cp_kernel_times(dom)
    ctx.cp_kernel_timing(None)
    note(f"one lane: {one_lane:.0f} tokens/s (with events around the {dom} launches)")
    # roofline of the dominant kernel: algorithmic flops of every timed launch
    dom_flops, dom_bytes, per_launch = dominant_work(w, cpa, chunks)
    dom_flops *= w.n_layer * args.steps
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12 if dom_ms > 0 else 0.0
    expect = per_launch["launches"] * w.n_layer * args.steps
    if dom_launches != expect:
        raise RuntimeError(f"timed {dom_launches} launches of {dom}, expected {expect}")
    # Decode-sized chunks at the end of the prompt (the pages' "pp3" / "tg32" regime, run on
    # the same kernels): 32 chunks of 1 token, then 32 of 3, each series from depth n.
    decode = {}
    for dc in (1, 3):
        ctx.kv_cache_truncate(n)
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        for i in range(32):
            rc = ctx.prefill_chunk_raw(x[i * dc:(i + 1) * dc].data_ptr(), out[i * dc:(i + 1) * dc].data_ptr(), dc)
            if rc != 0:
                raise RuntimeError(f"prefill_chunk failed: {rc} {ctx.last_error()}")
        torch.cuda.synchronize()
        dt2 = time.perf_counter() - t2
        # the same 32 chunks as one prompt through prefill_chunks, 2 and 3 tiny chunks in
        # flight (prompt tokens known in advance; generated tokens would depend on the
        # previous one)
        lanes_ms = {}
        for nl in (2, 3):
            ctx.kv_cache_truncate(n)
            torch.cuda.synchronize()
            t3 = time.perf_counter()
            rc = ctx.prefill_chunks_raw(x.data_ptr(), out.data_ptr(), 32 * dc, dc, nl)
            if rc != 0:
                raise RuntimeError(f"prefill_chunks failed: {rc} {ctx.last_error()}")
            torch.cuda.synchronize()
            lanes_ms[str(nl)] = (time.perf_counter() - t3) / 32 * 1e3
        decode[f"chunk_{dc}"] = {"tokens_per_s": 32 * dc / dt2, "ms_per_chunk": dt2 / 32 * 1e3,
                                 "lanes_ms_per_chunk": lanes_ms,
                                 "depth": n,
                                 "hbm_roofline_ms_per_chunk": roofline_s(w, dc, n) * w.n_layer * 1e3}
    # The step after the prompt: logits of the last position over a q8_0 LM head of
    # LOGITS_VOCAB rows (seeded synthetic bytes with a fixed scale), HBM-bound: every head
    # byte is read once.
    last_logits = None
    if not w.n_expert:
        nb = w.d_model // 32
        gen = torch.Generator(device="cuda").manual_seed(7)
        head = torch.randint(0, 256, (LOGITS_VOCAB, nb, 34), dtype=torch.uint8, device="cuda", generator=gen)
        head[:, :, 0] = 0x00
        head[:, :, 1] = 0x20
        head = head.reshape(-1)
        gain = torch.ones(w.d_model, device="cuda")
        lg = torch.empty(LOGITS_VOCAB, device="cuda")
        xr = out[n - 1]
        for _ in range(3):
            cpa.cp_last_logits(xr, gain, head, LOGITS_VOCAB, 1e-6, lg)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for _ in range(20):
            cpa.cp_last_logits(xr, gain, head, LOGITS_VOCAB, 1e-6, lg)
        ev1.record()
        torch.cuda.synchronize()
        us = ev0.elapsed_time(ev1) / 20 * 1e3
        last_logits = {"vocab": LOGITS_VOCAB, "d_model": w.d_model, "head_bytes": head.numel(),
                       "us": us, "tb_per_s": head.numel() / us / 1e6,
                       "frac_of_hbm": head.numel() / us / 1e6 / (PEAK_HBM_GBS / 1e3)}
        del head, lg
    # whole-prompt roofline: sum of per-chunk-layer bounds
    bound = sum(roofline_s(w, e - s, s) for s, e in chunks) * w.n_layer
    res = {
        "value": tps,
        "ms_per_step": total / args.steps * 1e3,
        "roofline": {"bound": "mfma", "kernel": dom, "timed_on": "one lane (each launch alone)",
                     "achieved": achieved,
                     "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_F16_TFLOPS,
                     "traffic": measured_traffic(dom, per_launch),
                     "launches": dom_launches, "avg_launch_us": dom_ms * 1e3 / max(1, dom_launches),
                     "flops_per_launch": per_launch["flops"],
                     "algorithmic_bytes_per_launch": per_launch["bytes"]},
        "prompt_roofline": {"bound_ms_per_step": bound * 1e3,
                            "frac": bound / (total / args.steps)},
        "one_lane_tokens_per_s": one_lane,
        "decode_regime": decode,
        "last_logits": last_logits,
    }
    ctx.close()
    del x, out
    torch.cuda.empty_cache()
    return w, res


def run_config(name, torch, cpa, synth, steps=1, warmup=1, attention_roofline=False, lanes=2):
    """Whole-prompt prefill rate of another workload (chunks of its own size from an empty
    cache), with its roofline fraction: the sum over chunk-layers of max(flops / MFMA peak,
    bytes / HBM peak) against the measured time.  Same seeded synthetic weights and inputs."""
    w = synth.WORKLOADS[name]
    n, C = w.n_prompt, w.chunk
    note(f"config {w.name}: {w.n_layer} layers, {n} tokens in {C}-token chunks, {w.kv_type} cache")
    layers = gpu_layers(w, torch, cpa, synth)
    ctx = cpa.PrefillContext(cpa.make_config(w, n, C), layers, stream=torch.cuda.Stream())
    del layers
    torch.cuda.empty_cache()
    if w.vocab:
        x = torch.from_numpy(synth.prompt_inputs(w)).cuda()
    else:
        x = synth.prompt_inputs(w, backend="torch", device="cuda")
    out = torch.empty_like(x)
    torch.cuda.synchronize()          # inputs are read on the context's own streams
    chunks = [(s, min(n, s + C)) for s in range(0, n, C)]

    def step_lanes():
        ctx.kv_cache_truncate(0)
        rc = ctx.prefill_chunks_raw(x.data_ptr(), out.data_ptr(), n, C, lanes)
        if rc != 0:
            raise RuntimeError(f"prefill_chunks failed: {rc} {ctx.last_error()}")

    def step_one_lane():
        ctx.kv_cache_truncate(0)
        for s, e in chunks:
            rc = ctx.prefill_chunk_raw(x[s:e].data_ptr(), out[s:e].data_ptr(), e - s)
            if rc != 0:
                raise RuntimeError(f"prefill_chunk failed: {rc} {ctx.last_error()}")

    step = step_lanes if lanes > 1 else step_one_lane
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    bound = sum(roofline_s(w, e - s, s) for s, e in chunks) * w.n_layer
    flops = sum(chunk_flops(w, e - s, s) for s, e in chunks) * w.n_layer
    res = {"workload": w.name, "n_layer": w.n_layer, "prompt_tokens": n, "chunk": C,
           "kv_type": w.kv_type, "lanes": lanes, "tokens_per_s": n / dt, "ms_per_prompt": dt * 1e3,
           "algorithmic_tflop_per_s": flops / dt / 1e12,
           "roofline_bound_ms": bound * 1e3, "roofline_frac": bound / dt}
    if attention_roofline:
        # one more step, on one lane (each launch alone on the device), with HIP events
        # around every attention launch (the kernel and, for split KV, its merge) on the
        # library's stream; algorithmic flops of the unmasked causal part,
        # 4*Hq*hd*(C*D + C(C+1)/2) per chunk-layer
        ctx.cp_kernel_timing("attention")
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        step_one_lane()
        torch.cuda.synchronize()
        dt1 = time.perf_counter() - t1
        ms, launches = ctx.cp_kernel_times("attention")
        ctx.cp_kernel_timing(None)
        af = sum(4.0 * w.n_head * w.head_dim * ((e - s) * s + (e - s) * (e - s + 1) / 2)
                 for s, e in chunks) * w.n_layer
        ach = af / (ms * 1e-3) / 1e12 if ms > 0 else 0.0
        res["roofline"] = {"bound": "mfma", "kernel": f"attention ({w.kv_type} cache)",
                           "achieved": ach, "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                           "frac": ach / PEAK_F16_TFLOPS, "traffic": None, "launches": launches,
                           "avg_launch_us": ms * 1e3 / max(1, launches),
                           "flops_per_launch": af / max(1, launches),
                           "share_of_one_lane_step": ms * 1e-3 / dt1}
    ctx.close()
    del x, out
    torch.cuda.empty_cache()
    return res


def run_pmc_probe(args, torch, cpa, synth):
    """One chunk of the workload's chunk size through one layer of its shapes, from an
    empty cache: every kernel of the layer is dispatched once in the launch configuration
    the benchmark times (the GEMM plans and tiles depend on the chunk size, not the
    depth), with few enough dispatches for per-dispatch counter collection."""
    w = synth.WORKLOADS[args.workload].with_(n_layer=1)
    if args.pmc_chunk:
        w = w.with_(chunk=args.pmc_chunk)
    C, D = w.chunk, args.pmc_depth
    layers = gpu_layers(w, torch, cpa, synth)
    ctx = cpa.PrefillContext(cpa.make_config(w, D + C, C), layers)
    x = synth.prompt_inputs(w, D + C, backend="torch", device="cuda")
    out = torch.empty_like(x)
    torch.cuda.synchronize()
    for s in range(0, D + C, C):
        ctx.prefill_chunk(x[s:min(D + C, s + C)], out[s:min(D + C, s + C)])
    torch.cuda.synchronize()
    note(f"pmc probe: {C}-token chunks through one {w.name} layer up to depth {D}; gemm plan "
         f"{cpa.cp_test_gemm_plan(C, 2 * (-(-w.ffn_dim // 128) * 128), w.d_model) if w.ffn_dim else None}")
    ctx.close()


def run_sweep(args, torch, cpa, synth, oracle_fit):
    w = synth.WORKLOADS["dense27b_sweep"]
    sizes, depths = w.chunk_sweep, w.depths
    Cmax = max(sizes)
    note(f"sweep {w.name}: {w.n_layer} layers, chunks {list(sizes)}, depths {list(depths)}")
    layers = gpu_layers(w, torch, cpa, synth)
    ctx = cpa.PrefillContext(cpa.make_config(w, w.depth_prefill + Cmax, Cmax), layers)
    del layers
    torch.cuda.empty_cache()
    x = synth.prompt_inputs(w, w.depth_prefill + Cmax, backend="torch", device="cuda")
    out = torch.empty_like(x)
    table = {}
    for D in depths:
        ctx.kv_cache_truncate(0)
        for s in range(0, D, Cmax):
            ctx.prefill_chunk(x[s:s + Cmax], out[s:s + Cmax])
        torch.cuda.synchronize()
        for C in sizes:
            reps = []
            for r in range(2 + args.sweep_reps):          # two warm-up chunks, then R timed
                ctx.kv_cache_truncate(D)
                _, ms = ctx.prefill_chunk_timed(x[D:D + C], out[D:D + C])
                if r >= 2:
                    reps.append(ms)
            import numpy as np
            med = np.median(np.array(reps), axis=0)       # per layer
            table[(C, D)] = med
        note(f"sweep depth {D} done")
    import numpy as np
    fit = {}
    for D in depths:
        per_layer = []
        for l in range(w.n_layer):
            b, a, r2 = oracle_fit(list(sizes), [table[(C, D)][l] for C in sizes])
            per_layer.append({"b_ms": b, "a_ms_per_token": a, "r2": r2})
        fit[str(D)] = {"per_layer": per_layer,
                       "mean_b_ms": float(np.mean([p["b_ms"] for p in per_layer])),
                       "mean_a_ms_per_token": float(np.mean([p["a_ms_per_token"] for p in per_layer])),
                       "b_over_a_tokens": float(np.mean([p["b_ms"] for p in per_layer]) /
                                                np.mean([p["a_ms_per_token"] for p in per_layer]))}
    points = []
    for D in depths:
        for C in sizes:
            t_layer = float(np.mean(table[(C, D)]))
            points.append({"chunk": C, "depth": D, "ms_per_layer": t_layer,
                           "tokens_per_s_per_layer": C / (t_layer * 1e-3),
                           "tokens_per_s_4_layers": C / (float(np.sum(table[(C, D)])) * 1e-3),
                           "roofline_frac": roofline_s(w, C, D) / (t_layer * 1e-3),
                           "mfma_frac": chunk_flops(w, C, D) / (PEAK_F16_TFLOPS * 1e12) / (t_layer * 1e-3)})
    ctx.close()
    # the pipeline chunk rule of "Prompt chunks sized for a layer split's pipeline" fed with
    # the fitted b/a: chunk sizes for these prompt lengths over S layer-split stages
    planner = {}
    for D in depths:
        ba = fit[str(D)]["b_over_a_tokens"]
        planner[str(D)] = {"b_over_a_tokens": ba, "chunks": {
            str(n): {str(S): cpa.cp_plan_chunk(n, Cmax, S, ba) for S in (1, 2, 4, 8)}
            for n in (2013, 3865, 10041, 17055, 28998, 58300)}}
    return {"workload": f"{w.name}: {w.n_layer} layers of the dense 27B-class shapes, f16 cache",
            "fit": fit, "points": points, "planner": planner}


def run_cpu_baseline(args, w):
    """The oracle as it stands, on a bounded sample: one of the share's layers over the whole
    prompt (layer-major from an empty cache, so every attention depth of the prompt is in
    the sample), weights dequantised inside the timed region.  The layers of a share have
    identical shapes and cost, so the share's rate is tokens / (n_layer * seconds per
    layer).  --cpu-tokens N limits the prompt to its first N tokens instead (attention at
    depth is then under-represented and the rate overstated)."""
    import numpy as np
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        blas = [(i.get("internal_api"), i.get("num_threads")) for i in threadpool_info()]
    except Exception:
        blas = []
    n = min(args.cpu_tokens, w.n_prompt) if args.cpu_tokens > 0 else w.n_prompt
    one = w.with_(n_layer=1)
    note(f"cpu baseline: generating one {w.d_model}-wide layer and {n} input rows")
    fp = {name: synth.layer_weight(one, 0, name, shape) for name, shape in synth.weight_shapes(one)}
    ql = [oracle.quantize_layer(fp)]
    del fp
    x = synth.prompt_inputs(w, n)
    m = oracle.OracleModel(one, ql)
    t0 = time.perf_counter()
    m.prefill_layer_major(x)
    dt = time.perf_counter() - t0
    threads = max([t for _, t in blas if t] or [os.cpu_count() or 1])
    note(f"cpu baseline: {dt:.1f}s for one layer x {n} tokens")
    what = "the whole prompt" if n == w.n_prompt else f"the first {n} prompt tokens"
    return {"value": n / (w.n_layer * dt), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"1 of the {w.n_layer} identical layers over {what} ({n} tokens, every "
                      f"attention depth), float64 NumPy, weights dequantised in the timed region "
                      f"({dt:.2f} s); rate = tokens / ({w.n_layer} x that time)",
            "host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "blas": blas}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="dense27b_f16")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the whole-prompt rates of the other workloads")
    ap.add_argument("--sweep-reps", type=int, default=5)
    ap.add_argument("--lanes", type=int, choices=range(1, 9), default=3,
                    help="chunks in flight in the timed steps: 2 .. 8 (prefill_chunks, one "
                         "stream per lane) or 1 (prefill_chunk for each chunk in turn)")
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="CPU baseline over the first N prompt tokens (0: the whole prompt)")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="for rocprofv3 --pmc: the copy probe, then one chunk of the workload's "
                         "chunk size through one of its layers (no timing events), and exit")
    ap.add_argument("--pmc-chunk", type=int, default=0,
                    help="with --pmc-probe: chunk size instead of the workload's own")
    ap.add_argument("--pmc-depth", type=int, default=0,
                    help="with --pmc-probe: first prefill this many positions (in chunks of the "
                         "workload's chunk size), so the probed chunk attends at that depth")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first run one plain device-to-device copy of this many MiB: the "
                         "reference reading that scales rocprofv3 FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--pmc-digest", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU work: fold the counter files of the two --pmc-probe runs "
                         "(taken with --copy-probe-mib 1024) into profiles/pmc_traffic.json")
    args = ap.parse_args()
    if args.pmc_digest:
        pmc_digest(*args.pmc_digest, copy_mib=1024)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported "
              "(the multi-GPU layer split is a design note, not part of this build)", flush=True)
        sys.exit(2)
    import torch
    import chunked_prompt_prefill_amd as cpa
    import synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", flush=True)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.copy_probe_mib > 0:
        src = torch.ones(args.copy_probe_mib << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        note(f"copy probe: {args.copy_probe_mib} MiB device-to-device")
        del src, dst
    if args.pmc_probe:
        run_pmc_probe(args, torch, cpa, synth)
        return
    mf_tflops, hbm_gbs = cpa.cp_measure_peaks()
    note(f"measured peaks: fp16 MFMA {mf_tflops:.0f} TFLOP/s, HBM read {hbm_gbs:.0f} GB/s")
    w, res = run_main(args, torch, cpa, synth)
    res["roofline"]["measured_peak"] = mf_tflops
    res["roofline"]["frac_of_measured_peak"] = res["roofline"]["achieved"] / mf_tflops
    configs = []
    if not args.no_configs:
        for name in ("tiny_dense", "dense27b_q8", "moe_a3b"):
            # the 58,300-token q8_0-cache share is the largest that fits one GPU; its
            # dominant kernel is attention over the q8_0 cache
            # the tiny decoder is launch-bound: one lane (more lanes only add event waits)
            configs.append(run_config(name, torch, cpa, synth, attention_roofline=name != "tiny_dense",
                                      lanes=1 if name == "tiny_dense" else args.lanes))
    sweep = None
    if not args.no_sweep:
        sweep = run_sweep(args, torch, cpa, synth, fit_linear)
    cpu = None if args.no_cpu else run_cpu_baseline(args, w)
    line = {
        "metric": "prefill tokens/s at chunk C and KV depth (1 GPU); fitted b, a per layer",
        "value": res["value"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": res["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic (seeded N(0,0.02) q8_0 weights and hidden states)",
        "config": {"workload": f"{w.name}: {w.n_layer}-layer share, d_model {w.d_model}, "
                               f"{w.n_head}/{w.n_kv_head} heads, head_dim {w.head_dim}, "
                               f"{'experts' if w.n_expert else 'SwiGLU ' + str(w.ffn_dim)}, "
                               f"{w.kv_type} cache, {w.n_prompt}-token prompt in {w.chunk}-token chunks",
                   "n_layer": w.n_layer, "prompt_tokens": w.n_prompt, "chunk": w.chunk,
                   "kv_type": w.kv_type},
        "roofline": res["roofline"],
        "prompt_roofline": res["prompt_roofline"],
        "lanes": args.lanes,
        "one_lane_tokens_per_s": res["one_lane_tokens_per_s"],
        "decode_regime": res["decode_regime"],
        "last_logits": res["last_logits"],
        "measured_peaks": {"mfma_f16_tflops": mf_tflops, "hbm_read_gbs": hbm_gbs,
                           "published": {"mfma_f16_tflops": PEAK_F16_TFLOPS, "hbm_gbs": PEAK_HBM_GBS}},
        "cpu_baseline": cpu,
        "sweep_mfma_frac_chunks_ge_1024": None if sweep is None else {
            str(D): [round(p["mfma_frac"], 3) for p in sweep["points"] if p["depth"] == D and p["chunk"] >= 1024]
            for D in sorted({p["depth"] for p in sweep["points"]})},
        "configs": configs,
        "sweep": sweep,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
