"""Host-side logic on the CPU: the seeded input generator, the workload shapes, the
algorithmic-work accounting used for the rooflines, and the planner's workspace sizing
as reported through the C ABI (host code only; no kernel is launched)."""

import os

import numpy as np
import pytest
import torch

from shared_rank_kv_amd import accounting, inputs, workloads


# ---------------------------------------------------------------------------------------
# seeded inputs
# ---------------------------------------------------------------------------------------

def test_gaussian_is_deterministic_and_row_ranges_regenerate_exactly():
    full = inputs.gaussian(7, (3, 1), (5000, 4, 8), std=0.5)
    again = inputs.gaussian(7, (3, 1), (5000, 4, 8), std=0.5)
    assert torch.equal(full, again)
    for r0, r1 in ((0, 1), (2047, 2049), (4095, 5000), (1234, 1234)):
        part = inputs.gaussian(7, (3, 1), (5000, 4, 8), std=0.5, rows=(r0, r1))
        assert torch.equal(part, full[r0:r1])
    other = inputs.gaussian(7, (3, 2), (5000, 4, 8), std=0.5)
    assert not torch.equal(full, other)


def test_gaussian_statistics_and_rounding():
    x = inputs.gaussian(11, (0,), (4096, 256), std=0.05)
    assert x.dtype == torch.bfloat16
    v = x.float().numpy()
    assert abs(v.mean()) < 2e-4
    assert abs(v.std() - 0.05) < 1e-3
    f = inputs.gaussian(11, (0,), (64, 8), std=1.0, dtype="f32")
    assert f.dtype == torch.float32


# ---------------------------------------------------------------------------------------
# workload shapes (the configurations the benchmark and the parity tests use)
# ---------------------------------------------------------------------------------------

def test_llama_prefill_shapes():
    p = workloads.llama_prefill(agents=(0,))
    assert (p.n_q_heads, p.n_kv_heads, p.head_dim) == (32, 8, 128)
    assert int(p.q_len[0]) == 1024 and int(p.k_len[0]) == 9216
    assert p.ranks == (16, 16, 16)
    assert p.q_rows == 1024 and p.kv_rows == 9216


def test_decode_batch_shapes():
    p = workloads.decode_batch()
    assert p.batch == 64
    assert (p.q_len == 1).all() and (p.k_len == 16384).all()
    # every request has its own base rows
    assert sorted(p.k_start.tolist()) == list(range(0, 64 * 16384, 16384))


def test_mixed_batch_draws_in_range():
    ctx, q, ag = workloads.mixed_batch_draws()
    assert len(ctx) == len(q) == len(ag) == 32
    assert ((2048 <= ctx) & (ctx <= 16384)).all()
    assert ((1 <= q) & (q <= 512)).all()
    assert ((0 <= ag) & (ag <= 3)).all()


# ---------------------------------------------------------------------------------------
# accounting: the counting rules, checked against closed forms
# ---------------------------------------------------------------------------------------

def _pairs(lq, lk):
    # bottom-right causal: query t (0-based) sees keys 0 .. lk - lq + t
    return sum(lk - lq + t + 1 for t in range(lq))


def test_attention_work_llama_prefill():
    p = workloads.llama_prefill(agents=(0,))
    flop, nbytes = accounting.attention_work(p)
    pairs = _pairs(1024, 9216)
    qk = 32 * pairs * 2 * 128
    pv = 32 * pairs * 2 * 128
    pl = 32 * pairs * 2 * 16
    epi = 32 * 1024 * 2 * 16 * 128
    assert flop == qk + pv + pl + epi
    assert round(qk / 1e9, 1) == 73.0 and round(pl / 1e9, 1) == 9.1
    assert round(flop / 1e9, 1) == 155.3
    kv = 9216 * 8 * 128 * 2 * 2
    lr = 9216 * 16 * 2
    b = 16 * 1024 * 2
    qo = 1024 * 32 * 128 * 2 * 2
    assert nbytes == kv + lr + b + qo
    assert round(nbytes / 1e6, 1) == 54.9


def test_attention_work_decode_and_long_context():
    d = workloads.decode_batch()
    _, nbytes = accounting.attention_work(d)
    assert round(nbytes / 1e9, 2) == 4.33
    lc = workloads.longctx_prefill(agents=(0,))
    flop, nbytes = accounting.attention_work(lc)
    assert round(flop / 1e9, 1) == 341.2
    assert round(nbytes / 1e6, 1) == 146.9


def test_decode_shared_batch_work():
    p = workloads.decode_shared_batch()
    assert p.batch == 64 and p.kv_rows == 16 * 16384
    # four requests per context, one per agent, all reading the context's rows
    for c in range(16):
        assert (p.k_start[4 * c:4 * c + 4] == c * 16384).all()
        assert sorted(p.agent_idx[4 * c:4 * c + 4].tolist()) == [0, 1, 2, 3]
    _, nbytes = accounting.attention_work(p)
    kv = 16 * 16384 * 8 * 128 * 2 * 2          # each context's K/V rows once
    lr = 64 * 16384 * 16 * 2                   # every request's own LR rows
    b = 4 * 16 * 1024 * 2
    qo = 64 * 32 * 128 * 2 * 2
    assert nbytes == kv + lr + b + qo == 1108475904


def test_cache_memory_closed_forms():
    # Llama-3-8B shapes (8 kv heads x 128, 32 layers, bf16), 4 agents of rank 16, 16384 tokens
    m = accounting.cache_memory(16384, (16, 16, 16, 16), 8, 128)
    full = 2 * 8 * 128 * 16384 * 32 * 2
    assert m["full_shared"] == full == 2 ** 31
    assert m["non_shared"] == 4 * full
    assert m["base_shared"] == m["pre_lr_shared"] == full + 4 * 16 * 16384 * 32 * 2
    assert m["base_lr_shared"] == full + 16 * 16384 * 32 * 2
    s = accounting.cache_memory_summary(16384, (16, 16, 16, 16), 8, 128)
    assert s["base_over_non_shared"] == (2048 + 64) / (4 * 2048)
    assert abs(s["lr_share_of_base_shared"] - 1 / 33) < 1e-15      # 64 / (2048 + 64)


def test_cache_memory_invariants():
    for ranks in ((8,), (16, 16, 16), (8, 16, 32, 64), (0, 0, 0, 0)):
        m = accounting.cache_memory(1000, ranks, 4, 64, n_layers=3)
        n = len(ranks)
        assert m["non_shared"] == n * m["full_shared"]
        assert m["full_shared"] <= m["base_lr_shared"] <= m["base_shared"]
        if n == 1:
            assert m["base_lr_shared"] == m["base_shared"]
    # without adapter state BaseShared is exactly 1/N of Non-Shared
    s = accounting.cache_memory_summary(1000, (0, 0, 0, 0), 8, 128)
    assert s["base_over_non_shared"] == 0.25 and s["lr_share_of_base_shared"] == 0.0


def test_cache_memory_matches_the_shared_decode_buffers():
    # one layer of the shared-context decode batch: the K/V and LR buffers the call reads
    # are the PreLRShared cache of its 16 contexts
    p = workloads.decode_shared_batch()
    m = accounting.cache_memory(16384, p.ranks, p.n_kv_heads, p.head_dim, n_layers=1)
    kv_alloc = p.kv_rows * p.n_kv_heads * p.head_dim * 2 * 2
    lr_alloc = sum(p.kv_rows * r * 2 for r in p.ranks)
    assert kv_alloc == 16 * m["full_shared"]
    assert kv_alloc + lr_alloc == 16 * m["pre_lr_shared"]


def test_shared_rows_count_once():
    # two requests reading the same base rows: K/V bytes counted once, LR rows per request
    p = workloads.custom("s", "bf16", 8, 2, 64, (16,), [4, 4], [100, 100], [0, 0], seed=1,
                         shared_k=True)
    _, nbytes = accounting.attention_work(p)
    kv = 100 * 2 * 64 * 2 * 2
    lr = 2 * 100 * 16 * 2
    b = 16 * 2 * 64 * 2
    qo = 8 * 8 * 64 * 2 * 2
    assert nbytes == kv + lr + b + qo


def test_per_request_work_sums_to_total_for_disjoint_requests():
    p = workloads.mixed_batch_layer(0)
    flop, nbytes = accounting.attention_work(p)
    per = accounting.attention_work_per_request(p)
    assert sum(f for f, _ in per) == flop
    # B is counted once per agent in the total but once per request alone
    used = {int(a) for a, q in zip(p.agent_idx, p.q_len) if q > 0}
    b_total = sum(p.ranks[a] * p.n_kv_heads * p.head_dim * 2 for a in used)
    b_per = sum(p.ranks[int(a)] * p.n_kv_heads * p.head_dim * 2
                for a, q in zip(p.agent_idx, p.q_len) if q > 0)
    assert sum(b for _, b in per) - b_per == nbytes - b_total


def test_precompute_work():
    pre = workloads.longctx_precompute()
    flop, nbytes = accounting.precompute_work(pre)
    assert flop == 2 * 32768 * 4096 * 192
    assert round(flop / 1e9, 1) == 51.5
    assert nbytes == (32768 * 4096 + 4096 * 192 + 32768 * 192) * 2
    assert round(nbytes / 1e6, 1) == 282.6


# ---------------------------------------------------------------------------------------
# planner, through the C ABI's workspace query (host code only)
# ---------------------------------------------------------------------------------------

@pytest.fixture(scope="module")
def lra():
    from shared_rank_kv_amd import lra as mod
    return mod


def _part_bytes(rows, D):
    return rows * (D + 2) * 4 + 256


def test_workspace_decode_splits_keys_in_1024_chunks(lra, monkeypatch):
    monkeypatch.delenv("LRA_DECODE_CHUNK", raising=False)
    n = lra.lra_attn_workspace_bytes(torch.bfloat16, True, None, [16384] * 64, 32, 8, 128, 16)
    # 16 splits x 64 requests x 32 q heads partial rows
    assert n == _part_bytes(16 * 64 * 32, 128)
    n1 = lra.lra_attn_workspace_bytes(torch.bfloat16, True, None, [1000], 32, 8, 128, 16)
    assert n1 == 0          # one split: O is written directly


def test_workspace_prefill_fills_the_cus(lra, monkeypatch):
    monkeypatch.delenv("LRA_PREFILL_TARGET_WG", raising=False)
    # Llama prefill: 8 kv heads x 16 row tiles of 256 rows = 128 workgroups -> 2 splits
    n = lra.lra_attn_workspace_bytes(torch.bfloat16, False, [1024], [9216], 32, 8, 128, 16)
    assert n == _part_bytes(2 * 1024 * 32, 128)
    # enough row tiles on their own: no split, no workspace
    n = lra.lra_attn_workspace_bytes(torch.bfloat16, False, [8192], [8192], 32, 8, 128, 16)
    assert n == 0
    # fp32 never splits
    assert lra.lra_attn_workspace_bytes(torch.float32, False, [64], [9216], 8, 2, 128, 16) == 0


def test_workspace_rejects_invalid_arguments(lra):
    with pytest.raises(lra.LraError):
        lra.lra_attn_workspace_bytes(torch.bfloat16, False, [10], [5], 32, 8, 128, 16)
    with pytest.raises(lra.LraError):
        lra.lra_attn_workspace_bytes(torch.bfloat16, False, [10], [50], 32, 8, 96, 16)
    with pytest.raises(lra.LraError):
        lra.lra_attn_workspace_bytes(torch.bfloat16, True, None, [0], 32, 8, 128, 16)


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus above 1 exits with status 2 and says why, before
    touching the GPU."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_bench_traffic_figures_follow_the_sources():
    """The HBM traffic figures are reported only for the library sources they were
    measured with (the digest covers the header and every source of liblra.so)."""
    import importlib.util
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(root, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    assert len(bench.TRAFFIC_SOURCES_SHA256) == 64
    if bench.sources_sha256() == bench.TRAFFIC_SOURCES_SHA256:
        assert bench.traffic_bytes("llama8b-prefill-1024q-9216k-r16") > 0
    r = bench.roof(500.0, 2500.0, "TFLOP/s", "mfma", None)
    assert r == {"bound": "mfma", "achieved": 500.0, "peak": 2500.0, "unit": "TFLOP/s",
                 "frac": 0.2, "traffic": None}
