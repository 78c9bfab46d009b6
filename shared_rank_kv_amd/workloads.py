"""Synthetic workloads: Llama-3-8B-shaped caches for Flash-LoRA-Attention and the LR precompute.

Each workload fixes shapes, request layout and seeded value distributions; tensors are
drawn on demand through ``inputs`` (whole, or a row range for sampled checks).  Nothing
here computes any part of the method.

Tensor stream keys, appended to the workload's key prefix: Q (0,), K_base (1,),
V_base (2,), L_a (3, a), B_a (4, a), X (5,), A_a (6, a), request draws (7, i).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import inputs

SEED_BASE = 20260


@dataclass
class AttnProblem:
    """A batch of Flash-LoRA-Attention requests over packed buffers.

    Request b: query rows [q_start[b], +q_len[b]) of Q/O attend (bottom-right causal) to
    rows [k_start[b], +k_len[b]) of K_base/V_base and of agent agent_idx[b]'s LR cache.
    """

    name: str
    dtype: str
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ranks: tuple
    q_start: np.ndarray
    q_len: np.ndarray
    k_start: np.ndarray
    k_len: np.ndarray
    agent_idx: np.ndarray
    q_rows: int
    kv_rows: int
    seed: int
    key: tuple = ()
    std_b: float = 0.05
    q_period: int | None = None   # Q row i is drawn row i % q_period (same queries per agent)
    lr_from_precompute: "PrecomputeProblem | None" = None
    extra: dict = field(default_factory=dict)

    @property
    def batch(self):
        return len(self.q_len)

    @property
    def n_agents(self):
        return len(self.ranks)

    @property
    def kv_dim(self):
        return self.n_kv_heads * self.head_dim

    def _k(self, *k):
        return tuple(self.key) + tuple(k)

    def Q(self, rows=None):
        r0, r1 = (0, self.q_rows) if rows is None else rows
        shape = (self.q_rows, self.n_q_heads, self.head_dim)
        if self.q_period is None:
            return inputs.gaussian(self.seed, self._k(0), shape, 1.0, self.dtype, (r0, r1))
        import torch
        base = inputs.gaussian(self.seed, self._k(0),
                               (self.q_period, self.n_q_heads, self.head_dim), 1.0, self.dtype)
        idx = torch.arange(r0, r1) % self.q_period
        return base[idx].contiguous()

    def K(self, rows=None):
        return inputs.gaussian(self.seed, self._k(1),
                               (self.kv_rows, self.n_kv_heads, self.head_dim), 1.0,
                               self.dtype, rows)

    def V(self, rows=None):
        return inputs.gaussian(self.seed, self._k(2),
                               (self.kv_rows, self.n_kv_heads, self.head_dim), 1.0,
                               self.dtype, rows)

    def L(self, a, rows=None):
        """LR cache of agent a, [kv_rows, r_a] (drawn N(0,1) unless it comes from a precompute)."""
        if self.lr_from_precompute is not None:
            raise ValueError("this workload's LR caches are the precompute's outputs")
        return inputs.gaussian(self.seed, self._k(3, a), (self.kv_rows, self.ranks[a]), 1.0,
                               self.dtype, rows)

    def B(self, a):
        return inputs.gaussian(self.seed, self._k(4, a), (self.ranks[a], self.kv_dim),
                               self.std_b, self.dtype)

    def with_agents(self, agent_idx):
        """Same data, requests re-pointed to other agents."""
        p = AttnProblem(**{**self.__dict__})
        p.agent_idx = np.asarray(agent_idx, dtype=np.int32)
        return p


@dataclass
class PrecomputeProblem:
    """L_a = X·A_a for all agents in one pass: X [T, d_model], A_a [d_model, r_a]."""

    name: str
    dtype: str
    T: int
    d_model: int
    ranks: tuple
    seed: int
    key: tuple = ()
    std_a: float | None = None   # default 1/sqrt(d_model)

    def X(self, rows=None):
        return inputs.gaussian(self.seed, tuple(self.key) + (5,), (self.T, self.d_model), 1.0,
                               self.dtype, rows)

    def A(self, a):
        std = self.std_a if self.std_a is not None else 1.0 / np.sqrt(self.d_model)
        return inputs.gaussian(self.seed, tuple(self.key) + (6, a),
                               (self.d_model, self.ranks[a]), std, self.dtype)


def _i32(x):
    return np.asarray(x, dtype=np.int32)


def _packed(q_len, k_len):
    q_len, k_len = _i32(q_len), _i32(k_len)
    q_start = np.concatenate([[0], np.cumsum(q_len)[:-1]]).astype(np.int32)
    k_start = np.concatenate([[0], np.cumsum(k_len)[:-1]]).astype(np.int32)
    return q_start, q_len, k_start, k_len, int(q_len.sum()), int(k_len.sum())


# ---------------------------------------------------------------------------------------
# The five workloads
# ---------------------------------------------------------------------------------------

def tiny_fp32():
    """Single layer, fp32, 2 agents of rank 8: 16 queries at the end of a 256-token shared
    context, 4 q heads = 4 kv heads, head_dim 64.  Both agents read the same base rows."""
    return AttnProblem(
        name="tiny-fp32-16q-256k-h4-d64-r8", dtype="f32", n_q_heads=4, n_kv_heads=4,
        head_dim=64, ranks=(8, 8), q_start=_i32([0, 16]), q_len=_i32([16, 16]),
        k_start=_i32([0, 0]), k_len=_i32([256, 256]), agent_idx=_i32([0, 1]), q_rows=32,
        kv_rows=256, seed=SEED_BASE + 0, std_b=0.05, q_period=16)


def llama_prefill(agents=(0,)):
    """Llama-3-8B-shaped single-layer prefill, bf16: 1024 new causal queries after an
    8192-token shared context (9216 keys), 32 q / 8 kv heads, head_dim 128, 3 agents of
    rank 16.  One request per listed agent, all reading the same base rows and queries."""
    n = len(agents)
    return AttnProblem(
        name="llama8b-prefill-1024q-9216k-r16", dtype="bf16", n_q_heads=32, n_kv_heads=8,
        head_dim=128, ranks=(16, 16, 16), q_start=_i32([1024 * i for i in range(n)]),
        q_len=_i32([1024] * n), k_start=_i32([0] * n), k_len=_i32([9216] * n),
        agent_idx=_i32(list(agents)), q_rows=1024 * n, kv_rows=9216, seed=SEED_BASE + 1,
        std_b=0.05, q_period=1024)


def decode_batch():
    """Decode, bf16: 64 requests, each one query token over its own 16384-token context,
    32 q / 8 kv heads, head_dim 128, 4 agents of rank 16, agent per request uniform."""
    seed = SEED_BASE + 2
    batch, ctx = 64, 16384
    agent_idx = inputs.integers(seed, (7, 0), 0, 3, batch)
    return AttnProblem(
        name="decode-64x16384-r16", dtype="bf16", n_q_heads=32, n_kv_heads=8, head_dim=128,
        ranks=(16, 16, 16, 16), q_start=np.arange(batch, dtype=np.int32),
        q_len=np.ones(batch, np.int32), k_start=(np.arange(batch) * ctx).astype(np.int32),
        k_len=np.full(batch, ctx, np.int32), agent_idx=agent_idx, q_rows=batch,
        kv_rows=batch * ctx, seed=seed, std_b=0.05)


def decode_shared_batch():
    """Shared-context decode, bf16: 16 contexts of 16384 tokens, each read by all 4 agents
    (rank 16) with one query token apiece: 64 requests, 32 q / 8 kv heads, head_dim 128.
    Every agent keeps its own LR cache over all contexts (the PreLRShared layout)."""
    return shared_decode("decode-shared-16x4x16384-r16", 32, 8, 128, (16, 16, 16, 16),
                         [(16384, [0, 1, 2, 3])] * 16, seed=SEED_BASE + 5)


def decode_append():
    """Decode-step LR append for the decode batch: the 64 requests' new tokens (X [64, 4096]
    ~ N(0,1)) into the four rank-16 agents' LR caches (A_a [4096, 16] ~ N(0, 1/4096)); token
    b lands on row 16384 b + 16383 of every agent's cache [64 x 16384, 16]."""
    return PrecomputeProblem(name="lr-append-64x4096-4x16", dtype="bf16", T=64, d_model=4096,
                             ranks=(16, 16, 16, 16), seed=SEED_BASE + 6)


def longctx_precompute():
    """LR precompute for the 32768-token context: X [32768, 4096] ~ N(0,1), three agents'
    A_a [4096, 64] ~ N(0, 1/4096)."""
    return PrecomputeProblem(name="lr-precompute-32768x4096-3x64", dtype="bf16", T=32768,
                             d_model=4096, ranks=(64, 64, 64), seed=SEED_BASE + 3)


def longctx_prefill(agents=(0,)):
    """512 causal queries over a 32768-token shared context, 32 q / 8 kv heads, head_dim
    128, rank 64, B_a ~ N(0, 0.02^2); the LR caches are the precompute's outputs."""
    n = len(agents)
    return AttnProblem(
        name="longctx-prefill-512q-32768k-r64", dtype="bf16", n_q_heads=32, n_kv_heads=8,
        head_dim=128, ranks=(64, 64, 64), q_start=_i32([512 * i for i in range(n)]),
        q_len=_i32([512] * n), k_start=_i32([0] * n), k_len=_i32([32768] * n),
        agent_idx=_i32(list(agents)), q_rows=512 * n, kv_rows=32768, seed=SEED_BASE + 3,
        std_b=0.02, q_period=512, lr_from_precompute=longctx_precompute())


MIXED_RANKS = (8, 16, 32, 64)


def mixed_batch_draws():
    """Request draws of the 32-layer mixed batch: 32 requests, shared context uniform in
    [2048, 16384], new causal queries uniform in [1, 512], agent uniform in {0..3}."""
    seed = SEED_BASE + 4
    ctx = inputs.integers(seed, (7, 0), 2048, 16384, 32)
    q = inputs.integers(seed, (7, 1), 1, 512, 32)
    agent = inputs.integers(seed, (7, 2), 0, 3, 32)
    return ctx, q, agent


def mixed_batch_layer(layer):
    """One layer of the 32-layer Llama-3-8B-shaped mixed batch (bf16, ranks 8/16/32/64);
    each layer has its own seeded K/V, LR caches and B."""
    ctx, q, agent = mixed_batch_draws()
    q_start, q_len, k_start, k_len, q_rows, kv_rows = _packed(q, ctx + q)
    return AttnProblem(
        name=f"mixed32-layer{layer}", dtype="bf16", n_q_heads=32, n_kv_heads=8,
        head_dim=128, ranks=MIXED_RANKS, q_start=q_start, q_len=q_len, k_start=k_start,
        k_len=k_len, agent_idx=agent, q_rows=q_rows, kv_rows=kv_rows,
        seed=SEED_BASE + 4, key=(100 + layer,), std_b=0.05)


MIXED_LAYERS = 32


def shared_decode(name, n_q_heads, n_kv_heads, head_dim, ranks, contexts, seed, order=None,
                  std_b=0.05):
    """bf16 decode over shared contexts: contexts = [(k_len, [agent, ...]), ...]; each listed
    agent has one request (one query token) over that context's base rows, and reads its own
    LR cache over the same rows.  `order` permutes the requests (default: context by
    context)."""
    starts = np.concatenate([[0], np.cumsum([kl for kl, _ in contexts])[:-1]]).astype(np.int64)
    reqs = [(int(starts[c]), int(kl), int(a)) for c, (kl, ags) in enumerate(contexts) for a in ags]
    if order is not None:
        reqs = [reqs[i] for i in order]
    n = len(reqs)
    return AttnProblem(
        name=name, dtype="bf16", n_q_heads=n_q_heads, n_kv_heads=n_kv_heads, head_dim=head_dim,
        ranks=tuple(ranks), q_start=np.arange(n, dtype=np.int32), q_len=np.ones(n, np.int32),
        k_start=_i32([r[0] for r in reqs]), k_len=_i32([r[1] for r in reqs]),
        agent_idx=_i32([r[2] for r in reqs]), q_rows=n,
        kv_rows=int(sum(kl for kl, _ in contexts)), seed=seed, std_b=std_b)


def custom(name, dtype, n_q_heads, n_kv_heads, head_dim, ranks, q_len, k_len, agent_idx,
           seed, std_b=0.05, shared_k=False):
    """A small problem for parity tests.  shared_k=True makes every request read the same
    base rows (a shared context), which needs equal k_len."""
    q_len, k_len = _i32(q_len), _i32(k_len)
    q_start, q_len, k_start, k_len, q_rows, kv_rows = _packed(q_len, k_len)
    if shared_k:
        assert len(set(k_len.tolist())) == 1
        k_start = np.zeros_like(k_start)
        kv_rows = int(k_len[0])
    return AttnProblem(name=name, dtype=dtype, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads,
                       head_dim=head_dim, ranks=tuple(ranks), q_start=q_start, q_len=q_len,
                       k_start=k_start, k_len=k_len, agent_idx=_i32(agent_idx),
                       q_rows=max(q_rows, 1), kv_rows=max(kv_rows, 1), seed=seed, std_b=std_b)
