"""Seeded random shapes through the C ABI, every output row against the CPU fp64 oracle.

Each case draws head_dim, the GQA group, the kv heads, 1-6 agents with ranks 0-64, 1-12
requests over 1-4 shared contexts (each request reads a prefix of its context, so agents
that share a context see different lengths of it), empty and ragged query counts, and LR
caches that are column views of wider buffers whose padding holds NaN.  Decode cases take
the shared-context grouping path wherever requests share a first base row.  Each case runs
the regrouped route and the in-tile expansion comparator (which expands V tiles in LDS and
does not group requests); the naive route needs non-overlapping spans per agent and is
covered by the comparator tests."""

import numpy as np
import pytest
import torch

from shared_rank_kv_amd import workloads

import helpers as H

pytestmark = pytest.mark.gpu

RANKS = (0, 8, 16, 24, 32, 40, 48, 56, 64)


def _random_problem(seed, decode):
    rng = np.random.default_rng(seed)
    D = int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2, 4] if G == 8 else [1, 2, 4, 8]))
    n_agents = int(rng.integers(1, 7))
    ranks = tuple(int(r) for r in rng.choice(RANKS, n_agents))
    n_ctx = int(rng.integers(1, 5))
    ctx_len = [int(rng.integers(1, 600)) for _ in range(n_ctx)]
    ctx_start = np.concatenate([[0], np.cumsum(ctx_len)[:-1]]).astype(int)
    batch = int(rng.integers(1, 13))
    k_start, k_len, q_len, agent = [], [], [], []
    for _ in range(batch):
        c = int(rng.integers(n_ctx))
        kl = int(rng.integers(1, ctx_len[c] + 1))
        k_start.append(int(ctx_start[c]))
        k_len.append(kl)
        q_len.append(1 if decode else int(rng.integers(0, min(kl, 150) + 1)))
        agent.append(int(rng.integers(n_agents)))
    q_len = np.array(q_len, np.int32)
    q_start = (np.arange(batch) if decode else
               np.concatenate([[0], np.cumsum(q_len)[:-1]])).astype(np.int32)
    prob = workloads.AttnProblem(
        name=f"random-{'decode' if decode else 'prefill'}-{seed}", dtype="bf16",
        n_q_heads=G * Hkv, n_kv_heads=Hkv, head_dim=D, ranks=ranks, q_start=q_start,
        q_len=q_len, k_start=np.array(k_start, np.int32), k_len=np.array(k_len, np.int32),
        agent_idx=np.array(agent, np.int32), q_rows=max(int(q_len.sum()), 1),
        kv_rows=int(sum(ctx_len)), seed=seed)
    wide = [bool(rng.integers(2)) for _ in ranks]
    pads = [8 * int(rng.integers(1, 4)) for _ in ranks]
    return prob, wide, pads


def _widen(dev, prob, wide, pads):
    """Replace the chosen LR caches by column views of NaN-filled wider buffers."""
    for a, r in enumerate(prob.ranks):
        if r and wide[a]:
            buf = torch.full((prob.kv_rows, r + pads[a]), float("nan"), dtype=torch.bfloat16,
                             device="cuda")
            buf[:, :r] = dev["L"][a]
            dev["L"][a] = buf[:, :r]


def _describe(prob, wide):
    return (f"{prob.name}: D={prob.head_dim} Hq={prob.n_q_heads} Hkv={prob.n_kv_heads} "
            f"ranks={prob.ranks} wide={wide} q_len={prob.q_len.tolist()} "
            f"k_start={prob.k_start.tolist()} k_len={prob.k_len.tolist()} "
            f"agents={prob.agent_idx.tolist()}")


@pytest.mark.parametrize("seed", range(40))
@pytest.mark.parametrize("decode", [False, True], ids=["prefill", "decode"])
@pytest.mark.parametrize("route", ["regrouped", "in_tile"])
def test_random_shapes(route, decode, seed):
    from shared_rank_kv_amd import lra
    prob, wide, pads = _random_problem(5000 + seed + (1000 if decode else 0), decode)
    print(f"{route} {_describe(prob, wide)}", flush=True)
    cpu, dev = H.device_inputs(prob)
    _widen(dev, prob, wide, pads)
    if route == "regrouped":
        O = H.run_decode(prob, dev) if decode else H.run_prefill(prob, dev)
    elif decode:
        O = lra.lra_attn_decode_expand(dev["Q"], dev["K"], dev["V"], dev["L"], dev["B"],
                                       prob.k_start, prob.k_len, prob.agent_idx)
    else:
        O = lra.lra_attn_prefill_expand(dev["Q"], dev["K"], dev["V"], dev["L"], dev["B"],
                                        prob.q_start, prob.q_len, prob.k_start, prob.k_len,
                                        prob.agent_idx)
    torch.cuda.synchronize()
    rows = H.covered_rows(prob)
    if len(rows) == 0:
        return
    H.assert_bf16_close(O.float().cpu().numpy()[rows], H.oracle_all(prob, cpu)[rows],
                        prob.name)
