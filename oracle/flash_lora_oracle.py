"""Plain CPU fp64 oracle for Flash-LoRA-Attention and the low-rank (LR) cache precompute.

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously correct reference that
the GPU library is checked against.  Only the test suite, the smoke check of the
package entry point and the ``cpu_baseline`` leg of the benchmark may import it.  It
shares no code with the GPU path: no kernels, headers, helpers or constants, and it
imports nothing from the product package.

What it computes (sources are the pages on the method):

* LRAgent, "Resumen Técnico" (gist.science, Spanish summary), section
  "1. Descomposición de la Caché": the value cache of an agent is a base part produced
  by the frozen pretrained weights W0, shared by every agent, plus an adapter part
  produced by that agent's LoRA weights (A, B).
* Same page, section "2. Esquemas de Intercambio", BaseShared: the adapter part is kept
  as the LR cache, the activations after the LoRA down-projection, X·A_i, of width r;
  the full-width adapter contribution is rebuilt by multiplying it by the LoRA
  up-projection B_i.
* Same page, section "3. Flash-LoRA-Attention": the kernel evaluates
  P·(V_base + V_lr·B) as P·V_base + (P·V_lr)·B.  That is an exact regrouping, so the
  oracle evaluates the ungrouped left-hand side: it materialises the full value cache
  V_full = V_base + L·B and runs naive softmax attention over it.
* PReCache abstract (arxivdaily page, English abstract), PreLRShared: when the shared
  context is first processed, the LR caches of all agents are computed at once,
  L = X·[A_1 .. A_N].

Readings where the pages are silent (each is listed with its reason in the design notes):

* softmax scale 1/sqrt(head_dim); no LoRA alpha/r factor (the caller folds it into B);
* the LR term touches values only; keys come from the base cache;
* one LR row per token, shared by every head of the layer; B_i is [r, Hkv*d] and
  column g*d + j feeds kv head g, lane j;
* grouped-query attention: q head h reads kv head h // (Hq // Hkv);
* causal alignment is bottom-right: of Lq queries over Lk keys, query t sits at
  absolute position Lk - Lq + t and sees keys s <= that position.

Everything runs in float64 on the exact stored input values (bf16 and fp32 inputs
widen to float64 exactly).  numpy's matmul (BLAS) is the only library primitive used.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "lr_precompute",
    "full_value_cache",
    "softmax_scale",
    "kv_head_of",
    "query_positions",
    "visible",
    "attention_request",
    "attention_batch",
]


# ---------------------------------------------------------------------------------------
# LR precompute (PreLRShared)
# ---------------------------------------------------------------------------------------

def lr_precompute(X, A_list):
    """Every agent's LR cache from one pass over the shared context.

    PReCache abstract (English abstract on the arxivdaily page), PreLRShared: the LR
    caches of all agents are computed when the shared context is first processed.
    LRAgent summary, section 2 (BaseShared): the LR cache of agent i holds X·A_i, the
    activations after the LoRA down-projection, r values per token.

    X: [T, d_model]; A_list: list of [d_model, r_a].  Returns the list of L_a [T, r_a],
    computed as the column blocks of X·[A_1 .. A_N], in float64.
    """
    X = np.asarray(X, dtype=np.float64)
    ranks = [int(np.shape(A)[1]) for A in A_list]
    A_cat = np.concatenate([np.asarray(A, dtype=np.float64) for A in A_list], axis=1)
    L_cat = X @ A_cat
    out, off = [], 0
    for r in ranks:
        out.append(L_cat[:, off:off + r])
        off += r
    return out


# ---------------------------------------------------------------------------------------
# Flash-LoRA-Attention, evaluated through its plain definition
# ---------------------------------------------------------------------------------------

def full_value_cache(V_base, L, B):
    """V_full = V_base + L·B, the value cache with the adapter part expanded to full width.

    LRAgent summary, section 1 (the value cache is base part plus adapter part) and
    section 2, BaseShared (the adapter part is rebuilt as LR cache times B_i).
    V_base: [Lk, Hkv, d]; L: [Lk, r]; B: [r, Hkv*d]; column g*d + j of B feeds kv head g,
    lane j.  Returns [Lk, Hkv, d] float64.
    """
    V_base = np.asarray(V_base, dtype=np.float64)
    Lk, Hkv, d = V_base.shape
    L = np.asarray(L, dtype=np.float64).reshape(Lk, -1)
    B = np.asarray(B, dtype=np.float64).reshape(L.shape[1], Hkv * d)
    return V_base + (L @ B).reshape(Lk, Hkv, d)


def softmax_scale(head_dim):
    """Scores are q·k / sqrt(head_dim) (standard scaled dot-product attention)."""
    return 1.0 / math.sqrt(head_dim)


def kv_head_of(h, n_q_heads, n_kv_heads):
    """Grouped-query attention: consecutive groups of Hq/Hkv query heads share a kv head."""
    return h // (n_q_heads // n_kv_heads)


def query_positions(q_len, k_len):
    """Bottom-right causal alignment: the Lq queries are the last Lq of the Lk positions."""
    return (k_len - q_len) + np.arange(q_len)


def visible(positions, k_len):
    """[len(positions), Lk] bool: key s is visible to a query at position p iff s <= p."""
    return np.arange(k_len)[None, :] <= np.asarray(positions)[:, None]


def attention_request(Q, K_base, V_base, L, B, positions=None, return_diag=False):
    """Flash-LoRA-Attention output of one request, by the plain definition.

    LRAgent summary, section 3: O = P·(V_base + V_lr·B) with P the causal softmax of the
    scaled scores against the base keys.  The value cache is expanded explicitly
    (``full_value_cache``) and attention is computed naively per query head.

    Q: [Lq, Hq, d] query rows; K_base, V_base: [Lk, Hkv, d]; L: [Lk, r]; B: [r, Hkv*d].
    positions: absolute position of each query row; by default the bottom-right
    alignment (``query_positions``).  Passing a subset of rows with their positions
    evaluates only those rows (used for sampled checks of large problems).

    Returns O [Lq, Hq, d] float64, and with return_diag a dict holding, per query head h,
    the probability matrix P[h] ([Lq, Lk]) and the two terms O_base = P·V_base and
    O_lr = P·(L·B) of the output.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K_base = np.asarray(K_base, dtype=np.float64)
    Lq, Hq, d = Q.shape
    Lk, Hkv, d_k = K_base.shape
    assert d_k == d and Hq % Hkv == 0
    if positions is None:
        positions = query_positions(Lq, Lk)
    positions = np.asarray(positions)
    assert positions.shape == (Lq,)

    V_full = full_value_cache(V_base, L, B)
    allowed = visible(positions, Lk)
    scale = softmax_scale(d)

    O = np.zeros((Lq, Hq, d), dtype=np.float64)
    diag = {"P": [], "O_base": np.zeros_like(O), "O_lr": np.zeros_like(O)}
    if return_diag:
        V_lr = V_full - np.asarray(V_base, dtype=np.float64)
    for h in range(Hq):
        g = kv_head_of(h, Hq, Hkv)
        S = (Q[:, h, :] @ K_base[:, g, :].T) * scale
        S = np.where(allowed, S, -np.inf)
        S = S - S.max(axis=1, keepdims=True)
        E = np.exp(S)
        P = E / E.sum(axis=1, keepdims=True)
        O[:, h, :] = P @ V_full[:, g, :]
        if return_diag:
            diag["P"].append(P)
            diag["O_base"][:, h, :] = P @ np.asarray(V_base, dtype=np.float64)[:, g, :]
            diag["O_lr"][:, h, :] = P @ V_lr[:, g, :]
    if return_diag:
        return O, diag
    return O


def attention_batch(Q, K_base, V_base, L_list, B_list, q_start, q_len, k_start, k_len,
                    agent_idx, out=None):
    """A batch of requests over packed buffers, with the library's request semantics.

    Request b takes query rows [q_start[b], q_start[b] + q_len[b]) of Q and attends to
    rows [k_start[b], k_start[b] + k_len[b]) of K_base / V_base and of the LR cache of
    agent agent_idx[b]; requests may read the same base rows (a shared context, the
    BaseShared scheme of the LRAgent summary, section 2).  Rows of the output that no
    request covers are left as they are in ``out`` (zeros when out is None).
    """
    Q = np.asarray(Q, dtype=np.float64)
    O = np.zeros(Q.shape, dtype=np.float64) if out is None else out
    for b in range(len(q_len)):
        lq, lk = int(q_len[b]), int(k_len[b])
        if lq == 0:
            continue
        qs, ks, a = int(q_start[b]), int(k_start[b]), int(agent_idx[b])
        L = np.asarray(L_list[a])[ks:ks + lk]
        O[qs:qs + lq] = attention_request(
            Q[qs:qs + lq], np.asarray(K_base)[ks:ks + lk], np.asarray(V_base)[ks:ks + lk],
            L, B_list[a])
    return O
