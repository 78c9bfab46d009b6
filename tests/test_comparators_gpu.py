"""The comparators of the regrouping, through the C ABI, against the fp64 oracle:
  - the naive route: lra_expand_values writes the agent's full-width values
    V_full = V_base + L·B (checked against the oracle's full value cache within the bound of
    fp32 accumulation plus the bf16 rounding), then plain attention with no adapter;
  - the in-tile expansion route: lra_attn_prefill_expand / lra_attn_decode_expand.
Both round V_full to bf16 before P·V, so they are held to the same bf16 tolerances as the
regrouped kernels, plus the relative Frobenius gate, also LR-isolated (V_base = 0)."""

import os

import numpy as np
import pytest
import torch

import oracle
from shared_rank_kv_amd import inputs, workloads

import helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lra():
    from shared_rank_kv_amd import lra   # fails loudly if liblra.so is missing
    assert torch.cuda.is_available()
    return lra


def _cmp(prob, cpu, O, what):
    rows = H.covered_rows(prob)
    return H.assert_bf16_close(O.float().cpu().numpy()[rows], H.oracle_all(prob, cpu)[rows], what)


def _naive_prefill(lra, prob, dev):
    Vf = lra.lra_expand_values(dev["V"], dev["L"], dev["B"], prob.k_start, prob.k_len,
                               prob.agent_idx)
    O = lra.lra_attn_prefill(dev["Q"], dev["K"], Vf, [None], [None], prob.q_start, prob.q_len,
                             prob.k_start, prob.k_len, np.zeros(prob.batch, np.int32))
    torch.cuda.synchronize()
    return O


def _naive_decode(lra, prob, dev):
    Vf = lra.lra_expand_values(dev["V"], dev["L"], dev["B"], prob.k_start, prob.k_len,
                               prob.agent_idx)
    O = lra.lra_attn_decode(dev["Q"], dev["K"], Vf, [None], [None], prob.k_start, prob.k_len,
                            np.zeros(prob.batch, np.int32))
    torch.cuda.synchronize()
    return O


@pytest.mark.parametrize("D,Hkv,ranks", [(128, 8, (8, 16, 40, 64, 0)), (64, 2, (24, 64, 8, 32, 16))])
def test_expand_values_against_the_full_value_cache(lra, D, Hkv, ranks):
    prob = workloads.custom("expand-spans", "bf16", Hkv * 2, Hkv, D, ranks, [1] * 6,
                            [1, 37, 512, 513, 1500, 700], [0, 1, 2, 3, 4, 1], seed=910 + D)
    cpu, dev = H.device_inputs(prob)
    out = torch.full_like(dev["V"], 7.0)
    # every request's rows but the last request's, which must stay untouched
    lra.lra_expand_values(dev["V"], dev["L"], dev["B"], prob.k_start[:5], prob.k_len[:5],
                          prob.agent_idx[:5], V_full=out)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    V64 = inputs.to_f64(cpu["V"])
    for b in range(5):
        ks, kl, a = int(prob.k_start[b]), int(prob.k_len[b]), int(prob.agent_idx[b])
        r = prob.ranks[a]
        L64 = inputs.to_f64(cpu["L"][a][ks:ks + kl]) if r else np.zeros((kl, 0))
        B64 = inputs.to_f64(cpu["B"][a]) if r else np.zeros((0, Hkv * D))
        want = oracle.full_value_cache(V64[ks:ks + kl], L64, B64)
        bound = (max(r, 1) * 2.0 ** -23 * (np.abs(L64) @ np.abs(B64)).reshape(want.shape)
                 + 2.0 ** -8 * np.abs(want))
        assert np.all(np.abs(got[ks:ks + kl] - want) <= bound), f"span {b} (rank {r})"
    ks5 = int(prob.k_start[5])
    assert np.all(got[ks5:ks5 + int(prob.k_len[5])] == 7.0), "rows outside the spans changed"
    # in place gives the same bytes
    again = dev["V"].clone()
    lra.lra_expand_values(again, dev["L"], dev["B"], prob.k_start[:5], prob.k_len[:5],
                          prob.agent_idx[:5], V_full=again)
    torch.cuda.synchronize()
    rows = np.concatenate([np.arange(int(prob.k_start[b]), int(prob.k_start[b] + prob.k_len[b]))
                           for b in range(5)])
    assert torch.equal(again[rows], out[rows])


# (D, Hq, Hkv, ranks, q_len, k_len, agents): GQA 1-8, ranks 0-64, ragged tails, q = k
PREFILL = [
    (128, 8, 2, (16, 64, 8, 0), [1, 37, 200, 64], [5, 300, 700, 64], [0, 1, 2, 3]),
    (128, 32, 8, (16, 32), [130, 3], [450, 1000], [1, 0]),
    (64, 4, 4, (24, 48), [100, 17], [333, 17], [0, 1]),
    (128, 8, 1, (40,), [20, 9], [150, 9], [0, 0]),
    (64, 16, 8, (8, 56), [64, 65], [128, 129], [1, 0]),
]


@pytest.mark.parametrize("shape", PREFILL, ids=[f"D{s[0]}-Hq{s[1]}-Hkv{s[2]}" for s in PREFILL])
def test_prefill_comparators(lra, shape):
    D, Hq, Hkv, ranks, q_len, k_len, agents = shape
    prob = workloads.custom("cmp-prefill", "bf16", Hq, Hkv, D, ranks, q_len, k_len, agents,
                            seed=920 + D + Hq)
    cpu, dev = H.device_inputs(prob)
    _cmp(prob, cpu, _naive_prefill(lra, prob, dev), "naive expansion")
    O = lra.lra_attn_prefill_expand(dev["Q"], dev["K"], dev["V"], dev["L"], dev["B"],
                                    prob.q_start, prob.q_len, prob.k_start, prob.k_len,
                                    prob.agent_idx)
    torch.cuda.synchronize()
    _cmp(prob, cpu, O, "in-tile expansion")


def test_prefill_in_tile_lr_isolated_splits_and_shared_context(lra, monkeypatch):
    prob = workloads.custom("cmp-lr", "bf16", 8, 2, 128, (16, 64), [50, 120], [400, 900],
                            [0, 1], seed=930)
    cpu, dev = H.device_inputs(prob, zero_v=True)
    run = lambda: lra.lra_attn_prefill_expand(dev["Q"], dev["K"], dev["V"], dev["L"], dev["B"],  # noqa: E731
                                              prob.q_start, prob.q_len, prob.k_start,
                                              prob.k_len, prob.agent_idx)
    O = run()
    torch.cuda.synchronize()
    mx, mean, rel = _cmp(prob, cpu, O, "in-tile, LR-isolated")
    print(f"in-tile LR-isolated rel-frob {rel:.2e}")
    _cmp(prob, cpu, _naive_prefill(lra, prob, dev), "naive, LR-isolated")
    # key splits (the combine pass) and repeat determinism
    one = O.clone()
    for target in ("8", "64", "4096"):
        monkeypatch.setenv("LRA_PREFILL_TARGET_WG", target)
        a = run().clone()
        b = run()
        torch.cuda.synchronize()
        assert torch.equal(a, b)
        _cmp(prob, cpu, a, f"in-tile, target {target}")
        assert (a.float() - one.float()).abs().max().item() <= 4e-3
    monkeypatch.delenv("LRA_PREFILL_TARGET_WG")
    # several agents over one shared context (each request expands its own tiles)
    sh = workloads.custom("cmp-shared", "bf16", 8, 2, 128, (16, 32, 64), [40, 40, 40],
                          [500, 500, 500], [0, 1, 2], seed=931, shared_k=True)
    cpu, dev = H.device_inputs(sh)
    O = lra.lra_attn_prefill_expand(dev["Q"], dev["K"], dev["V"], dev["L"], dev["B"], sh.q_start,
                                    sh.q_len, sh.k_start, sh.k_len, sh.agent_idx)
    torch.cuda.synchronize()
    _cmp(sh, cpu, O, "in-tile, shared context")


DECODE = [
    (128, 8, 1, (0, 64), [1, 31, 32, 33, 127, 128, 129, 3000], [0, 1, 0, 1, 0, 1, 0, 1]),
    (128, 32, 8, (16, 64, 8), [1, 63, 64, 65, 1000, 5000], [0, 1, 2, 0, 1, 2]),
    (64, 16, 2, (64, 0, 40), [96, 1, 700, 4100], [0, 1, 2, 2]),
]


@pytest.mark.parametrize("shape", DECODE, ids=lambda s: f"D{s[0]}-Hq{s[1]}-Hkv{s[2]}")
@pytest.mark.parametrize("chunk", ["64", "1024"])
def test_decode_comparators(lra, shape, chunk, monkeypatch):
    monkeypatch.setenv("LRA_DECODE_CHUNK", chunk)
    D, Hq, Hkv, ranks, k_len, agents = shape
    prob = workloads.custom("cmp-decode", "bf16", Hq, Hkv, D, ranks, [1] * len(k_len), k_len,
                            agents, seed=940 + D + Hq)
    cpu, dev = H.device_inputs(prob)
    _cmp(prob, cpu, _naive_decode(lra, prob, dev), "naive expansion")
    O = lra.lra_attn_decode_expand(dev["Q"], dev["K"], dev["V"], dev["L"], dev["B"],
                                   prob.k_start, prob.k_len, prob.agent_idx)
    torch.cuda.synchronize()
    _cmp(prob, cpu, O, "in-tile expansion")
    again = lra.lra_attn_decode_expand(dev["Q"], dev["K"], dev["V"], dev["L"], dev["B"],
                                       prob.k_start, prob.k_len, prob.agent_idx)
    torch.cuda.synchronize()
    assert torch.equal(O, again)


def test_decode_in_tile_shared_contexts_and_lr_isolated(lra):
    prob = workloads.shared_decode("cmp-decode-shared", 32, 8, 128, (8, 64, 16),
                                   [(1500, [0, 1, 2, 0]), (300, [1, 0])], seed=950)
    cpu, dev = H.device_inputs(prob)
    O = lra.lra_attn_decode_expand(dev["Q"], dev["K"], dev["V"], dev["L"], dev["B"],
                                   prob.k_start, prob.k_len, prob.agent_idx)
    torch.cuda.synchronize()
    _cmp(prob, cpu, O, "in-tile, shared contexts")
    cpu, dev = H.device_inputs(prob, zero_v=True)
    O = lra.lra_attn_decode_expand(dev["Q"], dev["K"], dev["V"], dev["L"], dev["B"],
                                   prob.k_start, prob.k_len, prob.agent_idx)
    torch.cuda.synchronize()
    _cmp(prob, cpu, O, "in-tile, LR-isolated")
