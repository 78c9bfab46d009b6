"""Algorithmic work of the hot path, for roofline reporting.

Counting rules (algorithmic work only):
* attention FLOP = sum over q heads and unmasked (query, key) pairs of 4*D + 2*r
  (Q·Kᵀ, P·V_base and P·L, 2 FLOP per multiply-add) plus 2*r*D per query row and q head
  for the up-projection (P·L)·B; softmax work, padding (rank to 32-wide MFMA blocks,
  unused rows of a tile) and the full-width expansion the method avoids are not counted;
* attention bytes = K_base and V_base rows once (rows shared by several requests count
  once), each request's selected LR-cache rows, B once per agent used, Q and O;
* precompute FLOP = 2*T*d_model*sum(r); bytes = X + A_cat + the L outputs.
The split-key workspace traffic is implementation overhead and is not counted.
"""

from __future__ import annotations

import numpy as np

PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
PEAK_FP32_TFLOPS = 157.3


def _elem(dtype):
    return 2 if dtype == "bf16" else 4


def attention_work(prob):
    """(flop, bytes) of one lra_attn_prefill / lra_attn_decode call on ``prob``."""
    e = _elem(prob.dtype)
    D, Hq, Hkv = prob.head_dim, prob.n_q_heads, prob.n_kv_heads
    flop = 0
    l_bytes = 0
    agents = set()
    spans = []
    for b in range(prob.batch):
        lq, lk = int(prob.q_len[b]), int(prob.k_len[b])
        if lq == 0:
            continue
        r = prob.ranks[int(prob.agent_idx[b])]
        pairs = lq * (lk - lq) + lq * (lq + 1) // 2
        flop += Hq * pairs * (4 * D + 2 * r) + Hq * lq * 2 * r * D
        l_bytes += lk * r * e
        if r:
            agents.add(int(prob.agent_idx[b]))
        spans.append((int(prob.k_start[b]), int(prob.k_start[b]) + lk))
    # unique key rows
    rows = 0
    end = -1
    for s, t in sorted(spans):
        if t > end:
            rows += t - max(s, end)
            end = t
    kv_bytes = rows * Hkv * D * e * 2
    b_bytes = sum(prob.ranks[a] * Hkv * D * e for a in agents)
    qo_bytes = int(np.sum(prob.q_len)) * Hq * D * e * 2
    return flop, kv_bytes + l_bytes + b_bytes + qo_bytes


def attention_work_per_request(prob):
    """[(flop, bytes)] of each request on its own: its K/V rows, its LR rows, its agent's
    B, its Q and O.  For requests with disjoint key rows the sums equal attention_work."""
    e = _elem(prob.dtype)
    D, Hq, Hkv = prob.head_dim, prob.n_q_heads, prob.n_kv_heads
    out = []
    for b in range(prob.batch):
        lq, lk = int(prob.q_len[b]), int(prob.k_len[b])
        if lq == 0:
            continue
        r = prob.ranks[int(prob.agent_idx[b])]
        pairs = lq * (lk - lq) + lq * (lq + 1) // 2
        flop = Hq * pairs * (4 * D + 2 * r) + Hq * lq * 2 * r * D
        nbytes = lk * Hkv * D * e * 2 + lk * r * e + r * Hkv * D * e + lq * Hq * D * e * 2
        out.append((flop, nbytes))
    return out


def lr_term_work(prob, route, rows_per_tile=256, keys_per_tile=64):
    """(flop, bytes) the LR term adds to plain attention on ``prob``, by route:
    * "regrouped" (Flash-LoRA-Attention): 2*r per unmasked pair and q head (P·L) plus 2*r*D
      per query row and q head ((P·L)·B); bytes: the LR rows and B;
    * "naive": the expansion V_full = V_base + L·B of every key row of every request,
      2*r*D*Hkv per row, before plain attention; bytes: V_base read, V_full written, the
      LR rows and B (the plain attention then reads V_full instead of V_base);
    * "in_tile": the same expansion repeated per work item inside the kernel: every key
      tile a row tile of rows_per_tile (query, head) rows visits is expanded once, 2*r*D
      per key per kv head; no bytes beyond the regrouped route's.
    Rank-0 requests add nothing."""
    e = _elem(prob.dtype)
    D, Hq, Hkv = prob.head_dim, prob.n_q_heads, prob.n_kv_heads
    G = Hq // Hkv
    flop = nbytes = 0
    agents = set()
    for b in range(prob.batch):
        lq, lk = int(prob.q_len[b]), int(prob.k_len[b])
        r = prob.ranks[int(prob.agent_idx[b])]
        if lq == 0 or r == 0:
            continue
        agents.add(int(prob.agent_idx[b]))
        if route == "regrouped":
            pairs = lq * (lk - lq) + lq * (lq + 1) // 2
            flop += Hq * pairs * 2 * r + Hq * lq * 2 * r * D
            nbytes += lk * r * e
        elif route == "naive":
            flop += lk * 2 * r * D * Hkv
            nbytes += lk * Hkv * D * e * 2 + lk * r * e
        elif route == "in_tile":
            keys = 0
            rows = lq * G
            for r0 in range(0, rows, rows_per_tile):
                last = min(r0 + rows_per_tile, rows) - 1
                kend = lk - lq + last // G + 1
                keys += -(-kend // keys_per_tile) * keys_per_tile if lq > 1 else lk
            flop += Hkv * keys * 2 * r * D
            nbytes += lk * r * e
        else:
            raise ValueError(route)
    nbytes += sum(prob.ranks[a] * Hkv * D * e for a in agents)
    return flop, nbytes


def precompute_work(p):
    e = _elem(p.dtype)
    R = sum(p.ranks)
    flop = 2 * p.T * p.d_model * R
    return flop, (p.T * p.d_model + p.d_model * R + p.T * R) * e


def append_work(p):
    """(flop, bytes) of one lra_append_lr call: the new tokens' rows of X, A_cat, and one
    output row per token and agent (the precompute's counting rule on T new tokens)."""
    return precompute_work(p)


# ---------------------------------------------------------------------------------------
# KV-cache memory of the sharing schemes (LRAgent summary, section 2; PReCache abstract)
# ---------------------------------------------------------------------------------------

SCHEMES = ("non_shared", "base_shared", "base_lr_shared", "pre_lr_shared", "full_shared")


def cache_memory(tokens, ranks, n_kv_heads, head_dim, n_layers=32, dtype="bf16",
                 shared_rank=None):
    """Bytes of KV cache that `len(ranks)` agents keep for one shared context of `tokens`
    tokens, per sharing scheme (all layers):

    * non_shared: every agent its own K and V caches (the adapter output folded in);
    * base_shared: one base K/V cache for all agents, plus each agent's LR cache
      [tokens, r_a] (the adapter's down-projection activations, x·A_a);
    * base_lr_shared: one base K/V cache and one LR cache [tokens, shared_rank] for all
      agents (a shared down-projection A makes the LR caches equal); shared_rank defaults
      to the largest rank;
    * pre_lr_shared: the memory of base_shared; every agent's LR cache is computed in one
      pass over the shared context instead of on each switch of agent;
    * full_shared: one K/V cache for all agents, no adapter state (the bound of sharing).
    Keys are not decomposed: only the value side carries the adapter term."""
    e = _elem(dtype)
    n = len(ranks)
    kv = 2 * n_kv_heads * head_dim * tokens * n_layers * e          # one K + V cache
    lr_each = sum(ranks) * tokens * n_layers * e
    r_shared = max(ranks) if shared_rank is None else shared_rank
    lr_one = r_shared * tokens * n_layers * e
    return {"non_shared": n * kv, "base_shared": kv + lr_each, "base_lr_shared": kv + lr_one,
            "pre_lr_shared": kv + lr_each, "full_shared": kv}


def cache_memory_summary(tokens, ranks, n_kv_heads, head_dim, n_layers=32, dtype="bf16"):
    """cache_memory plus the two ratios the pages state in words: BaseShared against
    Non-Shared (about 1/N) and the LR caches' share of BaseShared (small)."""
    m = cache_memory(tokens, ranks, n_kv_heads, head_dim, n_layers, dtype)
    n = len(ranks)
    return {"bytes": m, "agents": n,
            "base_over_non_shared": m["base_shared"] / m["non_shared"],
            "one_over_n": 1.0 / n,
            "lr_share_of_base_shared": (m["base_shared"] - m["full_shared"]) / m["base_shared"]}
