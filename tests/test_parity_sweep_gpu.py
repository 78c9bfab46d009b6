"""A seeded sweep of small random problems through the C ABI, each compared with the oracle
element by element: random head_dim, GQA group, kv heads, agents and ranks (0 and every
multiple of 8 up to 64), request counts, lengths (empty requests, q = k, ragged tails),
dtype, prefill or decode, shared contexts for decode, and forced key splits.  The cases
are fixed by the seed, so a failure names a reproducible case."""

import os

import numpy as np
import pytest
import torch

from shared_rank_kv_amd import workloads

import helpers as H

pytestmark = pytest.mark.gpu

N_CASES = 96


def _case(i):
    rng = np.random.default_rng(4242 + i)
    D = int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2, 3]))
    n_agents = int(rng.integers(1, 5))
    ranks = tuple(int(r) for r in rng.choice([0, 8, 16, 24, 32, 40, 48, 56, 64], n_agents))
    dtype = "f32" if rng.random() < 0.25 else "bf16"
    decode = rng.random() < 0.4
    batch = int(rng.integers(1, 6))
    agents = [int(a) for a in rng.integers(0, n_agents, batch)]
    env = {}
    if decode:
        shared = dtype == "bf16" and batch > 1 and rng.random() < 0.5
        kl0 = int(rng.integers(1, 3000))
        k_len = [kl0] * batch if shared else [int(x) for x in rng.integers(1, 3000, batch)]
        q_len = [1] * batch
        env["LRA_DECODE_CHUNK"] = str(int(rng.choice([64, 256, 1024])))
    else:
        shared = False
        k_len = [int(x) for x in rng.integers(1, 700, batch)]
        q_len = [int(rng.integers(0, k + 1)) if rng.random() < 0.8 else k for k in k_len]
        q_len = [min(q, 300) for q in q_len]
        env["LRA_PREFILL_TARGET_WG"] = str(int(rng.choice([1, 64, 256, 4096])))
    prob = workloads.custom(f"sweep-{i}", dtype, G * Hkv, Hkv, D, ranks, q_len, k_len, agents,
                            seed=9000 + i, shared_k=shared)
    return prob, decode, env


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from shared_rank_kv_amd import lra   # fails loudly if liblra.so is missing
    assert torch.cuda.is_available()
    return lra


@pytest.mark.parametrize("i", range(N_CASES))
def test_sweep(i, monkeypatch):
    prob, decode, env = _case(i)
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    print(f"case {i}: {prob.dtype} D={prob.head_dim} Hq={prob.n_q_heads} Hkv={prob.n_kv_heads} "
          f"ranks={prob.ranks} q={prob.q_len.tolist()} k={prob.k_len.tolist()} "
          f"agents={prob.agent_idx.tolist()} decode={decode} env={env}", flush=True)
    cpu, dev = H.device_inputs(prob)
    O = H.run_decode(prob, dev) if decode else H.run_prefill(prob, dev)
    rows = H.covered_rows(prob)
    if len(rows) == 0:
        return
    want = H.oracle_all(prob, cpu)[rows]
    got = O.float().cpu().numpy()[rows]
    if prob.dtype == "bf16":
        H.assert_bf16_close(got, want, prob.name)
    else:
        H.assert_f32_close(got, want, prob.name)


# ---------------------------------------------------------------------------------------
# LR precompute and decode-step append: random token counts, d_model (multiples of 64 for
# bf16 and of 8 for fp32, the boundary's requirements), agent counts and ranks (sum <= 256),
# against the fp32-accumulation bound plus half a bf16 ulp of the rounded output.
# ---------------------------------------------------------------------------------------

N_LR_CASES = 32


def _lr_case(i):
    rng = np.random.default_rng(7070 + i)
    dtype = "f32" if rng.random() < 0.25 else "bf16"
    dm = int(rng.integers(1, 40)) * 64 if dtype == "bf16" else int(rng.integers(1, 75)) * 8
    ranks = []
    while not ranks or (rng.random() < 0.6 and len(ranks) < 8):
        r = int(rng.choice([0, 8, 16, 24, 32, 40, 48, 56, 64]))
        if sum(ranks) + r <= 256:
            ranks.append(r)
    append = rng.random() < 0.5
    T = int(rng.integers(1, 257)) if append else int(rng.integers(1, 1500))
    return dtype, T, dm, tuple(ranks), append


def _lr_check(dtype, dm, X, A, got_rows, what):
    import oracle
    from shared_rank_kv_amd import inputs
    Xf = inputs.to_f64(X)
    want = oracle.lr_precompute(Xf, [inputs.to_f64(a) for a in A])
    for a in range(len(A)):
        bound = dm * 2.0 ** -23 * (np.abs(Xf) @ np.abs(inputs.to_f64(A[a])))
        if dtype == "bf16":
            bound = bound + 2.0 ** -8 * np.abs(want[a])
        assert np.all(np.abs(got_rows[a] - want[a]) <= bound + 1e-30), f"{what}: agent {a}"


@pytest.mark.parametrize("i", range(N_LR_CASES))
def test_lr_sweep(i):
    from shared_rank_kv_amd import lra
    dtype, T, dm, ranks, append = _lr_case(i)
    print(f"lr case {i}: {dtype} T={T} d_model={dm} ranks={ranks} append={append}", flush=True)
    p = workloads.PrecomputeProblem(f"lr-sweep-{i}", dtype, T, dm, ranks, seed=7500 + i)
    X = p.X()
    A = [p.A(a) for a in range(len(ranks))]
    A_cat = torch.cat(A, dim=1).contiguous()
    if append:
        l_rows = T + int(np.random.default_rng(i).integers(0, 500))
        rows = np.random.default_rng(100 + i).choice(l_rows, size=T, replace=False)
        outs = [torch.full((l_rows, r), float("nan"), dtype=X.dtype, device="cuda")
                for r in ranks]
        lra.lra_append_lr(X.cuda(), A_cat.cuda(), ranks, outs, rows)
        torch.cuda.synchronize()
        got = [o.double().cpu().numpy()[rows] for o in outs]
        others = np.setdiff1d(np.arange(l_rows), rows)
        for a, o in enumerate(outs):
            assert np.isnan(o.double().cpu().numpy()[others]).all(), f"agent {a}: stray rows"
    else:
        outs = [torch.full((T, r), float("nan"), dtype=X.dtype, device="cuda") for r in ranks]
        lra.lra_precompute_lr(X.cuda(), A_cat.cuda(), ranks, outs)
        torch.cuda.synchronize()
        got = [o.double().cpu().numpy() for o in outs]
    _lr_check(dtype, dm, X, A, got, f"lr case {i}")
