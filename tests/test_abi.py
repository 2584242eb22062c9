"""The C-ABI library loads without a GPU, exports every declared call, and its host-only
logic (configuration checks, arena sizing, state header validation) behaves (CPU only)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "chunk_prefill.h")


@pytest.fixture(scope="module")
def cpa():
    import chunked_prompt_prefill_amd as m
    m.lib()
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if not n.startswith("_")))


def test_every_declared_symbol_is_exported(cpa):
    names = declared_functions()
    assert "prefill_init" in names and "kv_cache_set_state" in names and len(names) >= 25
    lib = ctypes.CDLL(cpa.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    from chunked_prompt_prefill_amd._lib import SIGNATURES
    assert set(SIGNATURES) == set(names), set(names) ^ set(SIGNATURES)


def test_arena_sizes_for_every_workload(cpa):
    for name, w in synth.WORKLOADS.items():
        n_ctx = w.n_prompt + max(w.depths, default=0)
        chunk = max(w.chunk_sweep) if w.chunk_sweep else w.chunk
        cfg = cpa.make_config(w, n_ctx, chunk)
        assert cpa.validate_config(cfg) == "", name
        wb, kb, sb = cpa.arena_sizes(cfg)
        assert wb > 0 and kb > 0 and sb > 0
        # the cache holds K and V of every layer at capacity
        row = w.head_dim * 2 if w.kv_type == "f16" else w.head_dim // 32 * 34
        assert kb >= w.n_layer * 2 * n_ctx * w.n_kv_head * row


@pytest.mark.parametrize("field,value", [("head_dim", 96), ("n_kv_head", 3), ("d_model", 100),
                                         ("kv_type", 2), ("n_chunk_max", 0), ("rms_eps", 0.0),
                                         ("n_expert_used", 3), ("n_ctx_max", 0)])
def test_invalid_configs_are_rejected(cpa, field, value):
    cfg = cpa.make_config(synth.WORKLOADS["dense27b_f16"], 1024, 512)
    setattr(cfg, field, value)
    assert cpa.validate_config(cfg) != ""
    assert cpa.arena_sizes(cfg) == (0, 0, 0)


def test_state_header_check_matches_oracle_blobs(cpa):
    from model_inputs import TINY_DENSE, q8_layers
    w = synth.Workload("abi_state", 2, 128, 4, 2, 64, 64, kv_type="q8_0")
    m = oracle.OracleModel(w, q8_layers(w))
    cache = m.new_cache(32)
    m.prefill(synth.prompt_inputs(w, 9), 4, cache=cache)
    blob = oracle.state_bytes(cache, w.rope_theta)
    L = cpa.lib()
    cfg = cpa.make_config(w, 32, 8)
    assert L.cp_state_bytes(ctypes.byref(cfg), 9) == len(blob)
    assert L.cp_state_check(ctypes.byref(cfg), blob, len(blob)) == 0
    for off in (0, 4, 8, 12, 16, 20, 24, 28):
        bad = bytearray(blob)
        bad[off] ^= 0x11
        assert L.cp_state_check(ctypes.byref(cfg), bytes(bad), len(bad)) == -3
    assert L.cp_state_check(ctypes.byref(cfg), blob[:-2], len(blob) - 2) == -3
    small = cpa.make_config(w, 8, 8)      # capacity below the blob's 9 tokens
    assert L.cp_state_check(ctypes.byref(small), blob, len(blob)) == -3


def test_plan_chunk_matches_the_oracle_rule_and_the_page_table(cpa):
    """The library's pipeline chunk rule (host code) against the oracle's restatement over
    a grid of prompt lengths, capacities, stage counts and cost ratios, and against the
    chunks the page prints for four stages."""
    import os
    golden = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "pipeline_chunks.txt")
    rows = [l.split() for l in open(golden) if l.strip() and not l.startswith("#")]
    for n, stages, chunk in ((int(a), int(b), int(c)) for a, b, c in rows):
        assert cpa.cp_plan_chunk(n, 8192, stages, 1024.0) == chunk
    for n in (0, 1, 300, 511, 512, 513, 2013, 3865, 10041, 17055, 28998, 58300, 100000):
        for cap in (128, 512, 2048, 3328, 8192):
            for stages in (1, 2, 3, 4, 8):
                for ba in (50.0, 183.0, 1000.0, 1024.0, 1820.0, 5000.0):
                    assert cpa.cp_plan_chunk(n, cap, stages, ba) == oracle.pipeline_chunk(n, cap, stages, ba), \
                        (n, cap, stages, ba)
    for bad in ((-1, 8192, 4, 1024.0), (100, 0, 4, 1024.0), (100, 8192, 0, 1024.0),
                (100, 8192, 4, 0.0), (100, 8192, 4, float("nan")), (100, 8192, 4, float("inf"))):
        with pytest.raises(Exception):
            cpa.cp_plan_chunk(*bad)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 37, 64, 65, 128, 159, 300, 512, 956, 2048, 3328, 8192])
@pytest.mark.parametrize("N,K", [(34816, 5120), (5120, 17408), (7168, 5120), (5120, 5120), (5120, 2048),
                                 (2048, 4096), (1536, 2048), (256, 256), (96, 768)])
def test_gemm_launch_plans_cover_the_columns(cpa, M, N, K):
    """Every launch plan the layers use (host only): one or two launches covering [0, N) in
    order, the first starting at column 0 and the second at a whole 256-column tile; split
    factors within [1, 16] and the K stages; the weight-streaming kernel (row tile 1) only
    for 1-4 rows with N a multiple of 64; 256-row tiles only above 128 rows."""
    mt, parts = cpa.cp_test_gemm_plan(M, N, K)
    assert 1 <= len(parts) <= 2
    assert parts[0][0] == 0
    for i, (n0, splits) in enumerate(parts):
        assert 1 <= splits <= max(16, K // 128)
        assert splits <= K // 128
        if i:
            assert n0 % 256 == 0 and 0 < n0 < N
            assert parts[0][1] == 1          # the whole rounds run unsplit
    if mt == 1:
        assert M <= 4 and N % 64 == 0 and len(parts) == 1
    else:
        assert mt in (64, 128, 256)
        assert not (M <= 4 and N % 64 == 0)
        assert mt != 256 or M > 128
        assert mt != 128 or M > 64


@pytest.mark.parametrize("M", [1, 4, 64, 128, 129, 300, 512, 2048, 3328, 8192])
@pytest.mark.parametrize("N,K", [(34816, 5120), (5120, 17408), (7168, 5120), (5120, 5120), (5120, 2048),
                                 (2048, 4096), (256, 256)])
def test_gemm_launch_plans_beside_other_chunks(cpa, M, N, K):
    """The plans of a device shared with other chunks in flight (host only): chunks of up
    to 128 rows keep the single-lane plan; larger ones take one launch of 256-row tiles,
    unsplit when the tiles number 192 or more or the split sums would need a pass of their
    own (plan 1), else (plan 2, sums added by the next kernel) two K splits."""
    tiles = -(-M // 256) * -(-N // 256)
    for plan in (1, 2):
        shared = cpa.cp_test_gemm_plan(M, N, K, plan)
        if M <= 128:
            assert shared == cpa.cp_test_gemm_plan(M, N, K)
            continue
        assert shared == (256, [(0, 2 if plan == 2 and tiles < 192 else 1)])
    with pytest.raises(Exception):
        cpa.cp_test_gemm_plan(M, N, K, 3)


def test_chunk_limit_of_the_gemm_operand_offsets(cpa):
    """The GEMMs address their fp16 input with 32-bit byte offsets: a chunk whose widest
    operand (the dense FFN intermediate, 17,408 columns at the 27B-class shapes) reaches
    2 GiB is refused at configuration time instead of reading zeros past 2 GiB."""
    w = synth.WORKLOADS["dense27b_f16"]
    limit = (1 << 31) // (2 * 17408)          # 61,680 rows of the FFN intermediate
    ok = cpa.make_config(w, limit, limit)
    assert cpa.validate_config(ok) == ""
    bad = cpa.make_config(w, limit + 1, limit + 1)
    assert "2 GiB" in cpa.validate_config(bad)
    assert cpa.arena_sizes(bad) == (0, 0, 0)
    # routed experts: the slots' intermediate (n * n_expert_used rows) counts
    m = synth.WORKLOADS["moe_a3b"]
    lim_m = (1 << 31) // (2 * 8 * 768)
    assert cpa.validate_config(cpa.make_config(m, lim_m, lim_m)) == ""
    assert cpa.validate_config(cpa.make_config(m, lim_m + 1, lim_m + 1)) != ""


def test_weight_matrix_limit_of_the_weight_offsets(cpa):
    """The 256-row GEMM kernel addresses a weight matrix's int8 values with 32-bit byte
    offsets: the gate/up pair (2 * ffn_dim rounded up to 128, by d_model) must hold fewer
    than 2^31 values, and a wider FFN is refused at configuration time."""
    w = synth.WORKLOADS["dense27b_f16"]
    cfg = cpa.make_config(w, 4096, 512)
    cfg.ffn_dim = (1 << 31) // (2 * 5120) // 128 * 128        # 209,664: just below
    assert cpa.validate_config(cfg) == ""
    cfg.ffn_dim += 128
    assert "2^31" in cpa.validate_config(cfg)


@pytest.mark.parametrize("field,value", [("d_model", 5120 + 64), ("n_head", 41)])
def test_shape_multiples_of_128(cpa, field, value):
    """d_model and n_head*head_dim must be multiples of 128, as the header documents."""
    cfg = cpa.make_config(synth.WORKLOADS["dense27b_f16"], 1024, 512)
    setattr(cfg, field, value)
    if field == "n_head":
        cfg.n_kv_head, cfg.head_dim = 41, 64   # 41 x 64 = 2624: only the 128 rule fails
    assert "128" in cpa.validate_config(cfg)


def test_chunk_argument_checks(cpa):
    """prefill_chunk's host-side checks (run before anything is enqueued): NULL and
    misaligned x_in / x_out are CP_E_INVALID, a chunk outside [1, n_chunk_max] or past
    n_ctx_max is CP_E_CAPACITY.  The addresses are never dereferenced."""
    cfg = cpa.make_config(synth.WORKLOADS["dense27b_f16"], 1024, 512)
    base = 1 << 20
    assert cpa.chunk_check(cfg, 0, base, base + 4096, 512) == 0
    assert cpa.chunk_check(cfg, 0, base, base, 1) == 0                 # in place
    assert cpa.chunk_check(cfg, 0, None, base, 1) == -1
    assert cpa.chunk_check(cfg, 0, base, None, 1) == -1
    for off in (4, 8, 12):
        assert cpa.chunk_check(cfg, 0, base + off, base, 1) == -1
        assert cpa.chunk_check(cfg, 0, base, base + off, 1) == -1
    assert cpa.chunk_check(cfg, 0, base, base, 0) == -2
    assert cpa.chunk_check(cfg, 0, base, base, 513) == -2
    assert cpa.chunk_check(cfg, 600, base, base, 425) == -2            # 600 + 425 > 1024
    assert cpa.chunk_check(cfg, 600, base, base, 424) == 0
    assert cpa.chunk_check(cfg, -1, base, base, 1) == -1
