"""Shared helpers of the GPU parity tests: run a workload through the C ABI, and evaluate the
oracle on the same stored inputs (whole, or sampled query rows of chosen requests)."""

from __future__ import annotations

import numpy as np
import torch

import oracle
from shared_rank_kv_amd import inputs

BF16_MAX_ABS = 2e-2       # max |GPU - oracle| for bf16 inputs with fp32 accumulation
BF16_MEAN_ABS = 2e-3      # mean |GPU - oracle|
REL_FROB = 1e-2           # ||GPU - oracle||_F / ||oracle||_F (supplementary gate)
F32_MAX_ABS = 1e-5        # fp32 path


def device_inputs(prob, zero_v=False, q_scale=1.0):
    """Generate the workload's tensors on the CPU and upload them (same stored bytes)."""
    cpu = {"Q": prob.Q(), "K": prob.K(), "V": prob.V()}
    if zero_v:
        cpu["V"] = torch.zeros_like(cpu["V"])
    if q_scale != 1.0:
        cpu["Q"] = (cpu["Q"].float() * q_scale).to(cpu["Q"].dtype)
    cpu["L"] = [prob.L(a) if prob.ranks[a] else None for a in range(prob.n_agents)]
    cpu["B"] = [prob.B(a) if prob.ranks[a] else None for a in range(prob.n_agents)]
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else [x.cuda() if x is not None else None
                                                              for x in v])
           for k, v in cpu.items()}
    return cpu, dev


def run_prefill(prob, dev, **kw):
    from shared_rank_kv_amd import lra
    O = lra.lra_attn_prefill(dev["Q"], dev["K"], dev["V"], dev["L"], dev["B"], prob.q_start,
                             prob.q_len, prob.k_start, prob.k_len, prob.agent_idx, **kw)
    torch.cuda.synchronize()
    return O


def run_decode(prob, dev, **kw):
    from shared_rank_kv_amd import lra
    O = lra.lra_attn_decode(dev["Q"], dev["K"], dev["V"], dev["L"], dev["B"], prob.k_start,
                            prob.k_len, prob.agent_idx, **kw)
    torch.cuda.synchronize()
    return O


def oracle_rows(prob, cpu, b, rows=None):
    """Oracle output of request b for query rows `rows` (indices into the request's
    queries; all when None), float64 [len(rows), Hq, D]."""
    qs, lq = int(prob.q_start[b]), int(prob.q_len[b])
    ks, lk = int(prob.k_start[b]), int(prob.k_len[b])
    a = int(prob.agent_idx[b])
    rows = np.arange(lq) if rows is None else np.asarray(rows)
    Q = inputs.to_f64(cpu["Q"][qs:qs + lq])[rows]
    K = inputs.to_f64(cpu["K"][ks:ks + lk])
    V = inputs.to_f64(cpu["V"][ks:ks + lk])
    if prob.ranks[a]:
        L = inputs.to_f64(cpu["L"][a][ks:ks + lk])
        B = inputs.to_f64(cpu["B"][a])
    else:
        L = np.zeros((lk, 0))
        B = np.zeros((0, prob.kv_dim))
    return oracle.attention_request(Q, K, V, L, B, positions=(lk - lq) + rows)


def oracle_all(prob, cpu):
    out = np.zeros((prob.q_rows, prob.n_q_heads, prob.head_dim))
    for b in range(prob.batch):
        lq = int(prob.q_len[b])
        if lq:
            qs = int(prob.q_start[b])
            out[qs:qs + lq] = oracle_rows(prob, cpu, b)
    return out


def covered_rows(prob):
    idx = [np.arange(int(prob.q_start[b]), int(prob.q_start[b]) + int(prob.q_len[b]))
           for b in range(prob.batch)]
    return np.concatenate(idx) if idx else np.zeros(0, dtype=np.int64)


def errors(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    d = np.abs(got - want)
    rel = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30)
    return float(d.max()), float(d.mean()), float(rel)


def assert_bf16_close(got, want, what="", rel_frob=REL_FROB):
    mx, mean, rel = errors(got, want)
    assert np.isfinite(np.asarray(got, dtype=np.float64)).all(), f"{what}: non-finite output"
    assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS and rel <= rel_frob, \
        f"{what}: max-abs {mx:.3e} mean-abs {mean:.3e} rel-frob {rel:.3e}"
    return mx, mean, rel


def assert_f32_close(got, want, what=""):
    mx, mean, rel = errors(got, want)
    assert mx <= F32_MAX_ABS, f"{what}: max-abs {mx:.3e} mean-abs {mean:.3e} rel {rel:.3e}"
    return mx, mean, rel


def sample_rows(lq, n, rng):
    """First, last and n-2 random query rows of a request (sorted, unique)."""
    pick = {0, lq - 1}
    if lq > 2:
        pick.update(rng.choice(np.arange(1, lq - 1), size=min(n - 2, lq - 2), replace=False).tolist())
    return np.array(sorted(pick))
