"""GPU parity of the HIP path against the CPU fp64 oracle, element by element, at sizes the
oracle finishes in seconds (several tiles, ragged tails, edge cases).  Calls go through the
C ABI (ctypes binding); nothing here computes on the GPU other than liblra.so's kernels."""

import os

import numpy as np
import pytest
import torch

from shared_rank_kv_amd import workloads

import helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from shared_rank_kv_amd import lra   # fails loudly if liblra.so is missing
    assert torch.cuda.is_available()
    return lra


def _cmp_full(prob, cpu, O, bf16=True, what=None, rel_frob=H.REL_FROB):
    rows = H.covered_rows(prob)
    want = H.oracle_all(prob, cpu)[rows]
    got = O.float().cpu().numpy()[rows]
    what = what or prob.name
    if bf16:
        return H.assert_bf16_close(got, want, what, rel_frob)
    return H.assert_f32_close(got, want, what)


# ---------------------------------------------------------------------------------------
# fp32 path
# ---------------------------------------------------------------------------------------

def test_tiny_fp32_both_agents():
    prob = workloads.tiny_fp32()
    cpu, dev = H.device_inputs(prob)
    O = H.run_prefill(prob, dev)
    mx, _, _ = _cmp_full(prob, cpu, O, bf16=False)
    print(f"tiny fp32 max-abs {mx:.2e}")
    # the LR term is far above the fp32 tolerance here, so this also pins it
    lr_only = H.oracle_all(prob, cpu) - H.oracle_all(prob, {**cpu, "B": [torch.zeros_like(b) for b in cpu["B"]]})
    assert np.abs(lr_only).max() > 100 * H.F32_MAX_ABS


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 8, 2), (64, 4, 4)])
def test_fp32_ragged_batch(D, Hq, Hkv):
    prob = workloads.custom("f32-ragged", "f32", Hq, Hkv, D, (16, 0, 64), q_len=[1, 70, 33],
                            k_len=[9, 70, 190], agent_idx=[0, 1, 2], seed=501)
    cpu, dev = H.device_inputs(prob)
    _cmp_full(prob, cpu, H.run_prefill(prob, dev), bf16=False)


def test_fp32_decode():
    prob = workloads.custom("f32-decode", "f32", 8, 2, 128, (8, 32), q_len=[1, 1, 1],
                            k_len=[1, 100, 700], agent_idx=[1, 0, 1], seed=502)
    cpu, dev = H.device_inputs(prob)
    O = H.run_decode(prob, dev)
    _cmp_full(prob, cpu, O, bf16=False)


# ---------------------------------------------------------------------------------------
# bf16 path
# ---------------------------------------------------------------------------------------

BF16_SHAPES = [
    # D, Hq, Hkv, ranks, q_len, k_len, agents
    (128, 8, 2, (16, 64, 8, 0), [1, 37, 200, 64], [5, 300, 700, 64], [0, 1, 2, 3]),
    (128, 32, 8, (16, 32), [130, 3], [450, 1000], [1, 0]),
    (64, 4, 4, (24, 48), [100, 17], [333, 17], [0, 1]),
    (128, 8, 1, (40,), [20, 9], [150, 9], [0, 0]),
    (64, 16, 8, (8, 56), [64, 65], [128, 129], [1, 0]),
]


@pytest.mark.parametrize("shape", BF16_SHAPES, ids=[f"D{s[0]}-Hq{s[1]}-Hkv{s[2]}" for s in BF16_SHAPES])
def test_bf16_ragged_batch(shape):
    D, Hq, Hkv, ranks, q_len, k_len, agents = shape
    prob = workloads.custom("bf16-ragged", "bf16", Hq, Hkv, D, ranks, q_len, k_len, agents,
                            seed=600 + D + Hq)
    cpu, dev = H.device_inputs(prob)
    O = H.run_prefill(prob, dev)
    _cmp_full(prob, cpu, O)


def test_bf16_many_requests_longest_first():
    """150 prefill requests: three launches (64 requests each at most), each sorted longest
    first and dealt over the XCDs; every request's rows must match the oracle."""
    rng = np.random.default_rng(660)
    k_len = [int(x) for x in rng.integers(1, 600, 150)]
    q_len = [int(rng.integers(0, min(k, 40) + 1)) for k in k_len]
    agents = [int(a) for a in rng.integers(0, 3, 150)]
    prob = workloads.custom("bf16-many", "bf16", 16, 4, 128, (16, 0, 64), q_len, k_len, agents,
                            seed=661)
    cpu, dev = H.device_inputs(prob)
    _cmp_full(prob, cpu, H.run_prefill(prob, dev))


def test_bf16_lr_isolated_and_peaked():
    # V_base = 0 leaves only (P·L)·B, which the default tolerances would barely see.
    prob = workloads.custom("bf16-lr-only", "bf16", 8, 2, 128, (16, 64), [50, 120], [400, 900],
                            [0, 1], seed=610)
    cpu, dev = H.device_inputs(prob, zero_v=True)
    O = H.run_prefill(prob, dev)
    mx, mean, rel = _cmp_full(prob, cpu, O, what="lr-only")
    print(f"LR-isolated rel-frob {rel:.2e}")
    cpu, dev = H.device_inputs(prob, q_scale=8.0)
    _cmp_full(prob, cpu, H.run_prefill(prob, dev), what="peaked")


def test_bf16_shared_context_and_shared_lr_cache():
    # BaseShared: every request reads the same base rows; BaseLRShared: one LR cache for all.
    prob = workloads.custom("bf16-shared", "bf16", 8, 2, 128, (16, 16, 16), [40, 40, 40],
                            [500, 500, 500], [0, 1, 2], seed=620, shared_k=True)
    cpu, dev = H.device_inputs(prob)
    _cmp_full(prob, cpu, H.run_prefill(prob, dev))
    cpu["L"] = [cpu["L"][0]] * 3
    dev["L"] = [dev["L"][0]] * 3
    _cmp_full(prob, cpu, H.run_prefill(prob, dev), what="shared LR cache")


def test_bf16_split_invariance_and_determinism(monkeypatch):
    prob = workloads.custom("bf16-split", "bf16", 8, 2, 128, (32,), [90], [3000], [0], seed=630)
    cpu, dev = H.device_inputs(prob)
    outs = {}
    # 90 queries x 4 heads per kv head = 2 row tiles per kv head, 4 workgroups unsplit:
    # targets 8, 12 and 16 split the keys 2, 3 and 4 ways, 64 and 4096 split them 5 ways
    # (47 key tiles / 8)
    for target in ("1", "8", "12", "16", "64", "4096"):
        monkeypatch.setenv("LRA_PREFILL_TARGET_WG", target)
        outs[target] = H.run_prefill(prob, dev).float().cpu().numpy()
        again = H.run_prefill(prob, dev).float().cpu().numpy()
        assert np.array_equal(outs[target], again), "repeat call not bitwise identical"
    want = H.oracle_all(prob, cpu)
    for k, v in outs.items():
        H.assert_bf16_close(v, want, f"target {k}")
    for k in ("8", "12", "16", "64", "4096"):
        assert np.abs(outs[k] - outs["1"]).max() <= 4e-3


def test_bf16_empty_requests():
    prob = workloads.custom("bf16-empty", "bf16", 8, 2, 128, (16,), [0, 20, 0], [10, 80, 0],
                            [0, 0, 0], seed=640)
    cpu, dev = H.device_inputs(prob)
    O = torch.full_like(dev["Q"], 7.0)
    H.run_prefill(prob, dev, O=O)
    _cmp_full(prob, cpu, O)


def test_bf16_decode_small_batch():
    prob = workloads.custom("bf16-decode", "bf16", 32, 8, 128, (16, 64, 8), [1] * 6,
                            [1, 63, 64, 65, 1000, 5000], [0, 1, 2, 0, 1, 2], seed=650)
    cpu, dev = H.device_inputs(prob)
    _cmp_full(prob, cpu, H.run_decode(prob, dev))
    # prefill with one query per request is the same computation
    _cmp_full(prob, cpu, H.run_prefill(prob, dev), what="decode via prefill")


@pytest.mark.parametrize("chunk", ["64", "1024", "100000"])
def test_bf16_decode_split_counts(chunk, monkeypatch):
    monkeypatch.setenv("LRA_DECODE_CHUNK", chunk)
    prob = workloads.custom("bf16-decode-split", "bf16", 16, 2, 64, (32,), [1, 1], [2000, 129],
                            [0, 0], seed=660)
    cpu, dev = H.device_inputs(prob)
    _cmp_full(prob, cpu, H.run_decode(prob, dev))


# (D, Hq, Hkv, ranks, k_len, agents): group sizes 1, 2, 4 and 8, rank-0 agents next to
# rank-64 ones (the LR tile of a rank-0 agent stays zero and its B is never read), key
# counts around the 32-key wave tile and the 128-key workgroup round.
DECODE_SHAPES = [
    (128, 8, 1, (0, 64), [1, 31, 32, 33, 127, 128, 129, 3000], [0, 1, 0, 1, 0, 1, 0, 1]),
    (128, 4, 4, (24,), [7, 500, 2049], [0, 0, 0]),
    (64, 16, 2, (64, 0, 40), [96, 1, 700, 4100], [0, 1, 2, 2]),
    (64, 8, 2, (0,), [200, 65], [0, 0]),
]


@pytest.mark.parametrize("shape", DECODE_SHAPES, ids=lambda s: f"D{s[0]}-Hq{s[1]}-Hkv{s[2]}-r{max(s[3])}")
@pytest.mark.parametrize("chunk", ["64", "1024"])
def test_bf16_decode_shapes(shape, chunk, monkeypatch):
    monkeypatch.setenv("LRA_DECODE_CHUNK", chunk)
    D, Hq, Hkv, ranks, k_len, agents = shape
    prob = workloads.custom("bf16-decode-shape", "bf16", Hq, Hkv, D, ranks, [1] * len(k_len),
                            k_len, agents, seed=670 + D + Hq)
    cpu, dev = H.device_inputs(prob)
    _cmp_full(prob, cpu, H.run_decode(prob, dev))


# Shared contexts in decode (BaseShared): requests that read the same base rows are served
# by one work item.  (D, Hq, Hkv, ranks, contexts): units of 4 members (G = 4), of 2 (G = 8),
# of 4 with one column per member (G = 1); member counts that are not a multiple of the unit
# size; the same agent twice in a unit; rank-0, rank-8 and rank-64 agents in one unit; key
# counts around the 32-key tile.
SHARED_DECODE = [
    (128, 32, 8, (16, 16, 16, 16), [(2000, [0, 1, 2, 3]), (700, [3, 2, 1]), (33, [0, 0]),
                                    (5000, [1])]),
    (64, 16, 2, (64, 0, 8), [(1500, [0, 1, 2, 0, 1, 2, 0])]),
    (128, 8, 8, (32, 24), [(900, [0, 1, 0, 1, 0, 1]), (64, [1, 0])]),
    (128, 16, 8, (64, 64, 64), [(4100, [0, 1, 2]), (1, [2, 1])]),
]


@pytest.mark.parametrize("shape", SHARED_DECODE, ids=lambda s: f"D{s[0]}-Hq{s[1]}-Hkv{s[2]}-r{max(s[3])}")
@pytest.mark.parametrize("chunk", ["64", "1024"])
def test_bf16_decode_shared_contexts(shape, chunk, monkeypatch):
    monkeypatch.setenv("LRA_DECODE_CHUNK", chunk)
    D, Hq, Hkv, ranks, contexts = shape
    n = sum(len(a) for _, a in contexts)
    order = np.random.default_rng(n + D).permutation(n)     # members interleaved in the batch
    prob = workloads.shared_decode("bf16-decode-shared", Hq, Hkv, D, ranks, contexts,
                                   seed=680 + D + Hq, order=order)
    cpu, dev = H.device_inputs(prob)
    grouped = H.run_decode(prob, dev)
    _cmp_full(prob, cpu, grouped)
    again = H.run_decode(prob, dev)
    assert torch.equal(grouped, again), "repeat call not bitwise identical"
    monkeypatch.setenv("LRA_DECODE_GROUP", "0")
    single = H.run_decode(prob, dev)
    assert (grouped.float() - single.float()).abs().max().item() <= 4e-3


@pytest.mark.parametrize("chunk", ["1024", "100000"])
def test_bf16_decode_shared_context_unequal_lengths(chunk, monkeypatch):
    """Agents that have seen different lengths of one context: same first row, different
    k_len.  Requests with equal solo split counts form one unit that streams the longest
    member's rows once; every member's columns are masked past its own length."""
    monkeypatch.setenv("LRA_DECODE_CHUNK", chunk)
    k_len = [3000, 2500, 2049, 1025, 3000, 700, 1]
    agents = [0, 1, 2, 3, 1, 2, 0]
    n = len(k_len)
    prob = workloads.AttnProblem(
        name="bf16-decode-nested", dtype="bf16", n_q_heads=32, n_kv_heads=8, head_dim=128,
        ranks=(16, 64, 8, 0), q_start=np.arange(n, dtype=np.int32), q_len=np.ones(n, np.int32),
        k_start=np.full(n, 100, np.int32), k_len=np.asarray(k_len, np.int32),
        agent_idx=np.asarray(agents, np.int32), q_rows=n, kv_rows=3100, seed=697)
    cpu, dev = H.device_inputs(prob)
    grouped = H.run_decode(prob, dev)
    _cmp_full(prob, cpu, grouped, what="nested contexts")
    assert torch.equal(grouped, H.run_decode(prob, dev)), "repeat call not bitwise identical"
    monkeypatch.setenv("LRA_DECODE_GROUP", "0")
    single = H.run_decode(prob, dev)
    assert (grouped.float() - single.float()).abs().max().item() <= 4e-3


def test_bf16_decode_shared_lr_cache():
    # BaseLRShared: every agent's LR cache is one buffer; the B_a still differ
    prob = workloads.shared_decode("bf16-decode-lrshared", 32, 8, 128, (16, 16, 16),
                                   [(3000, [0, 1, 2]), (800, [2, 0])], seed=690)
    cpu, dev = H.device_inputs(prob)
    cpu["L"] = [cpu["L"][0]] * 3
    dev["L"] = [dev["L"][0]] * 3
    _cmp_full(prob, cpu, H.run_decode(prob, dev), what="shared LR cache")


def test_bf16_lr_cache_padding_never_read():
    """LR caches that are column views of wider buffers whose padding holds NaN: a unit of
    the shared-context decode mixes ranks 8 and 64 (one accumulator serves both members),
    and prefill and ungrouped decode read the same views.  No padding value may reach an
    output."""
    prob = workloads.shared_decode("bf16-padding", 32, 8, 128, (8, 64, 16),
                                   [(1500, [0, 1, 2, 0]), (300, [1, 0])], seed=695)
    cpu, dev = H.device_inputs(prob)
    views = []
    for a, L in enumerate(dev["L"]):
        buf = torch.full((prob.kv_rows, 64 + 8), float("nan"), dtype=torch.bfloat16, device="cuda")
        buf[:, :L.shape[1]] = L
        views.append(buf[:, :L.shape[1]])
    dev["L"] = views
    grouped = H.run_decode(prob, dev)
    assert torch.isfinite(grouped.float()).all()
    _cmp_full(prob, cpu, grouped, what="shared decode, NaN padding")
    os.environ["LRA_DECODE_GROUP"] = "0"
    try:
        single = H.run_decode(prob, dev)
    finally:
        del os.environ["LRA_DECODE_GROUP"]
    _cmp_full(prob, cpu, single, what="decode, NaN padding")
    pre = workloads.custom("bf16-padding-prefill", "bf16", 32, 8, 128, (8, 64, 16), [40, 7, 90],
                           [1500, 300, 1500], [0, 1, 2], seed=696)
    cpu, dev = H.device_inputs(pre)
    views = []
    for L in dev["L"]:
        buf = torch.full((pre.kv_rows, 72), float("nan"), dtype=torch.bfloat16, device="cuda")
        buf[:, :L.shape[1]] = L
        views.append(buf[:, :L.shape[1]])
    dev["L"] = views
    _cmp_full(pre, cpu, H.run_prefill(pre, dev), what="prefill, NaN padding")


# ---------------------------------------------------------------------------------------
# LR precompute
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,T,dm,ranks", [("bf16", 300, 256, (8, 16, 64)),
                                              ("bf16", 1000, 512, (64, 64, 64)),
                                              ("bf16", 129, 4096, (32,)),
                                              # d_model chunks not a multiple of the
                                              # prefetch depth; widest and narrowest R
                                              ("bf16", 517, 320, (64, 64, 64, 64)),
                                              ("bf16", 64, 1344, (8,)),
                                              ("bf16", 255, 192, (0, 40, 24)),
                                              ("f32", 77, 136, (8, 24))])
def test_precompute(dtype, T, dm, ranks):
    import oracle
    from shared_rank_kv_amd import inputs, lra
    p = workloads.PrecomputeProblem("pre-small", dtype, T, dm, ranks, seed=700 + T)
    X = p.X()
    A = [p.A(a) for a in range(len(ranks))]
    A_cat = torch.cat(A, dim=1).contiguous()
    outs = [torch.full((T, r), float("nan"), dtype=X.dtype, device="cuda") for r in ranks]
    lra.lra_precompute_lr(X.cuda(), A_cat.cuda(), ranks, outs)
    torch.cuda.synchronize()
    Xf = inputs.to_f64(X)
    want = oracle.lr_precompute(Xf, [inputs.to_f64(a) for a in A])
    for a in range(len(ranks)):
        got = outs[a].double().cpu().numpy()
        # fp32 accumulation bound plus (bf16) half an ulp of the rounded output
        bound = dm * 2.0 ** -23 * (np.abs(Xf) @ np.abs(inputs.to_f64(A[a])))
        if dtype == "bf16":
            bound = bound + 2.0 ** -8 * np.abs(want[a])
        assert np.all(np.abs(got - want[a]) <= bound + 1e-30), f"agent {a}"


def test_precompute_into_column_blocks_of_one_buffer():
    from shared_rank_kv_amd import lra
    p = workloads.PrecomputeProblem("pre-cols", "bf16", 200, 256, (16, 32), seed=710)
    X, A = p.X(), [p.A(0), p.A(1)]
    A_cat = torch.cat(A, 1).contiguous().cuda()
    buf = torch.zeros(200, 48, dtype=torch.bfloat16, device="cuda")
    lra.lra_precompute_lr(X.cuda(), A_cat, (16, 32), [buf[:, :16], buf[:, 16:]])
    sep = [torch.zeros(200, r, dtype=torch.bfloat16, device="cuda") for r in (16, 32)]
    lra.lra_precompute_lr(X.cuda(), A_cat, (16, 32), sep)
    torch.cuda.synchronize()
    assert torch.equal(buf[:, :16], sep[0]) and torch.equal(buf[:, 16:], sep[1])


def test_precompute_into_rows_of_odd_stride():
    # rows of 50 elements (a stride that is not a multiple of 4): the epilogue cannot use
    # 8-byte stores; the results must not change
    from shared_rank_kv_amd import lra
    p = workloads.PrecomputeProblem("pre-odd", "bf16", 333, 512, (16, 32), seed=711)
    X, A = p.X(), [p.A(0), p.A(1)]
    A_cat = torch.cat(A, 1).contiguous().cuda()
    buf = torch.zeros(333, 50, dtype=torch.bfloat16, device="cuda")
    lra.lra_precompute_lr(X.cuda(), A_cat, (16, 32), [buf[:, 2:18], buf[:, 18:50]])
    sep = [torch.zeros(333, r, dtype=torch.bfloat16, device="cuda") for r in (16, 32)]
    lra.lra_precompute_lr(X.cuda(), A_cat, (16, 32), sep)
    torch.cuda.synchronize()
    assert torch.equal(buf[:, 2:18], sep[0]) and torch.equal(buf[:, 18:50], sep[1])
    assert (buf[:, :2] == 0).all()


# ---------------------------------------------------------------------------------------
# Decode-step LR append
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,batch,dm,ranks,l_rows", [
    ("bf16", 64, 4096, (16, 16, 16, 16), 3000),   # a decode batch, four rank-16 agents
    ("bf16", 37, 512, (64, 64, 64), 300),          # ragged token block, R = 192
    ("bf16", 1, 128, (8,), 5),                     # one token, one column block
    ("bf16", 300, 256, (0, 40, 24, 64, 64, 64), 700),   # two launches, R = 256, rank 0
    ("bf16", 256, 4096, (64, 64, 64, 64), 600),    # 16 output blocks: one slice of 16 rounds
    ("bf16", 64, 16384, (16, 16, 16, 16), 100),    # 16 slices of 4 rounds each
    ("f32", 20, 136, (8, 24), 50),
])
def test_append_lr(dtype, batch, dm, ranks, l_rows):
    import oracle
    from shared_rank_kv_amd import inputs, lra
    p = workloads.PrecomputeProblem("append", dtype, batch, dm, ranks, seed=720 + batch)
    X = p.X()
    A = [p.A(a) for a in range(len(ranks))]
    A_cat = torch.cat(A, dim=1).contiguous()
    rows = np.random.default_rng(batch).choice(l_rows, size=batch, replace=False)
    outs = [torch.full((l_rows, r), float("nan"), dtype=X.dtype, device="cuda") for r in ranks]
    lra.lra_append_lr(X.cuda(), A_cat.cuda(), ranks, outs, rows)
    torch.cuda.synchronize()
    again = [o.clone() for o in outs]
    lra.lra_append_lr(X.cuda(), A_cat.cuda(), ranks, again, rows)
    torch.cuda.synchronize()
    Xf = inputs.to_f64(X)
    want = oracle.lr_precompute(Xf, [inputs.to_f64(a) for a in A])
    others = np.setdiff1d(np.arange(l_rows), rows)
    for a in range(len(ranks)):
        got = outs[a].double().cpu().numpy()
        bound = dm * 2.0 ** -23 * (np.abs(Xf) @ np.abs(inputs.to_f64(A[a])))
        if dtype == "bf16":
            bound = bound + 2.0 ** -8 * np.abs(want[a])
        assert np.all(np.abs(got[rows] - want[a]) <= bound + 1e-30), f"agent {a}"
        assert np.isnan(got[others]).all(), f"agent {a}: rows outside `rows` were written"
        assert torch.equal(outs[a][rows], again[a][rows]), "repeat call not bitwise identical"


def test_append_lr_reads_only_d_model_columns_and_reuses_workspace():
    """X is a column block of a wider NaN-filled buffer and d_model (320) ends inside a
    256-value round: the chunks past d_model must read zeros, not the padding.  A caller
    workspace, dirty from an earlier call, serves two calls of different sizes."""
    import oracle
    from shared_rank_kv_amd import inputs, lra
    dm, ranks = 320, (8, 16, 24)
    p = workloads.PrecomputeProblem("append-pad", "bf16", 70, dm, ranks, seed=733)
    X = p.X()
    A = [p.A(a) for a in range(len(ranks))]
    A_cat = torch.cat(A, dim=1).contiguous().cuda()
    wide = torch.full((70, dm + 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    wide[:, :dm] = X.cuda()
    need = max(lra.lra_append_workspace_bytes(torch.bfloat16, n, dm, ranks) for n in (70, 9))
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda")
    want = oracle.lr_precompute(inputs.to_f64(X), [inputs.to_f64(a) for a in A])
    for n in (70, 9):
        rows = np.arange(n) * 3 + 1
        outs = [torch.full((300, r), float("nan"), dtype=torch.bfloat16, device="cuda")
                for r in ranks]
        lra.lra_append_lr(wide[:n, :dm], A_cat, ranks, outs, rows, workspace=ws)
        torch.cuda.synchronize()
        for a in range(len(ranks)):
            got = outs[a].double().cpu().numpy()[rows]
            bound = dm * 2.0 ** -23 * (np.abs(inputs.to_f64(X[:n])) @ np.abs(inputs.to_f64(A[a])))
            bound = bound + 2.0 ** -8 * np.abs(want[a][:n])
            assert np.all(np.abs(got - want[a][:n]) <= bound + 1e-30), f"n {n} agent {a}"



# ---------------------------------------------------------------------------------------
# Maximum sizes: LRA_MAX_BATCH requests in one call (several launches of at most 64
# requests each) over LRA_MAX_AGENTS agents of every rank 0..64
# ---------------------------------------------------------------------------------------

MAX_RANKS = (0, 8, 16, 24, 32, 40, 48, 56, 64, 8, 16, 32, 64, 0, 48, 16)


def _max_problem(dtype, decode, D, Hq, Hkv, seed):
    from shared_rank_kv_amd import lra
    n = 1024
    assert len(MAX_RANKS) == 16
    rng = np.random.default_rng(seed)
    k_len = [int(k) for k in rng.integers(1, 160, n)]
    q_len = [1] * n if decode else [int(rng.integers(0, min(k, 5) + 1)) for k in k_len]
    agents = [int(a) for a in rng.integers(0, 16, n)]
    return workloads.custom(f"max-{dtype}-{'dec' if decode else 'pre'}", dtype, Hq, Hkv, D,
                            MAX_RANKS, q_len, k_len, agents, seed=seed)


@pytest.mark.parametrize("decode", [False, True], ids=["prefill", "decode"])
def test_bf16_max_batch_and_agents(decode):
    prob = _max_problem("bf16", decode, 128, 32, 8, seed=780 + decode)
    cpu, dev = H.device_inputs(prob)
    O = H.run_decode(prob, dev) if decode else H.run_prefill(prob, dev)
    _cmp_full(prob, cpu, O)


def test_fp32_max_batch_and_agents():
    prob = _max_problem("f32", False, 64, 8, 2, seed=790)
    cpu, dev = H.device_inputs(prob)
    _cmp_full(prob, cpu, H.run_prefill(prob, dev), bf16=False)
