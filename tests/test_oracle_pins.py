"""Pins of the CPU fp64 oracle to facts outside itself (CPU only).

The pages print no tensors, so the pins are: hand-derived worked examples
(tests/golden), closed forms, a library routine on the special case with no adapter
(torch's scaled_dot_product_attention), brute-force scalar loops on tiny inputs, and
invariants the method fixes (the regrouping identity of Flash-LoRA-Attention, GQA as
repeated-head MHA, agent relabelling, softmax rows).  The last test plants plausible
mistakes in the oracle and checks that these pins catch every one of them.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import flash_lora_oracle as fo

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(12345)


def _rand_problem(Lq, Lk, Hq, Hkv, d, r, rng=RNG, b_std=0.5):
    Q = rng.standard_normal((Lq, Hq, d))
    K = rng.standard_normal((Lk, Hkv, d))
    V = rng.standard_normal((Lk, Hkv, d))
    L = rng.standard_normal((Lk, r))
    B = rng.standard_normal((r, Hkv * d)) * b_std
    return Q, K, V, L, B


def _brute_force(Q, K, V, L, B):
    """Scalar loops with math.exp, straight from the definition of causal softmax attention
    over the expanded value cache; for tiny shapes only."""
    Lq, Hq, d = Q.shape
    Lk, Hkv, _ = K.shape
    r = L.shape[1]
    G = Hq // Hkv
    out = np.zeros((Lq, Hq, d))
    for t in range(Lq):
        pos = Lk - Lq + t
        for h in range(Hq):
            g = h // G
            scores = []
            for s in range(pos + 1):
                acc = 0.0
                for i in range(d):
                    acc += float(Q[t, h, i]) * float(K[s, g, i])
                scores.append(acc / math.sqrt(d))
            mx = max(scores)
            w = [math.exp(x - mx) for x in scores]
            z = sum(w)
            for j in range(d):
                acc = 0.0
                for s in range(pos + 1):
                    v = float(V[s, g, j])
                    for rho in range(r):
                        v += float(L[s, rho]) * float(B[rho, g * d + j])
                    acc += (w[s] / z) * v
                out[t, h, j] = acc
    return out


# ---------------------------------------------------------------------------------------
# Pin suite (also run against planted mistakes at the end)
# ---------------------------------------------------------------------------------------

def pin_worked_example():
    ex = json.load(open(os.path.join(GOLDEN, "worked_example_attention.json")))
    Q = np.array(ex["Q"], dtype=np.float64)
    K = np.zeros((3, 1, 4))
    for s in range(3):
        K[s, 0, 0] = 2.0 * math.log(s + 1)
    V = np.array(ex["V_base"], dtype=np.float64)
    L = np.array(ex["L"], dtype=np.float64)
    B = np.array(ex["B"], dtype=np.float64)
    want = np.array([[[float(Fraction(x)) for x in row] for row in t] for t in ex["expected_O"]])
    got = oracle.attention_request(Q, K, V, L, B)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)


def pin_brute_force():
    rng = np.random.default_rng(7)
    for (Lq, Lk, Hq, Hkv, d, r) in [(1, 1, 1, 1, 2, 1), (3, 5, 2, 1, 3, 2), (4, 8, 4, 2, 4, 2),
                                    (2, 6, 3, 3, 2, 0), (4, 4, 2, 2, 4, 1)]:
        Q, K, V, L, B = _rand_problem(Lq, Lk, Hq, Hkv, d, r, rng)
        np.testing.assert_allclose(oracle.attention_request(Q, K, V, L, B),
                                   _brute_force(Q, K, V, L, B), rtol=1e-12, atol=1e-12)


def pin_gqa_is_repeated_mha():
    rng = np.random.default_rng(8)
    Lq, Lk, Hq, Hkv, d, r = 5, 11, 6, 2, 8, 3
    G = Hq // Hkv
    Q, K, V, L, B = _rand_problem(Lq, Lk, Hq, Hkv, d, r, rng)
    K_rep = np.repeat(K, G, axis=1)      # MHA head h holds kv head h // G
    V_rep = np.repeat(V, G, axis=1)
    B_rep = np.concatenate([B[:, (h // G) * d:(h // G + 1) * d] for h in range(Hq)], axis=1)
    np.testing.assert_allclose(oracle.attention_request(Q, K, V, L, B),
                               oracle.attention_request(Q, K_rep, V_rep, L, B_rep),
                               rtol=1e-12, atol=1e-12)


def pin_single_key():
    rng = np.random.default_rng(9)
    Hq, Hkv, d, r = 4, 2, 5, 3
    Q, K, V, L, B = _rand_problem(1, 1, Hq, Hkv, d, r, rng)
    got = oracle.attention_request(Q, K, V, L, B)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        for j in range(d):
            want = V[0, g, j] + sum(L[0, p] * B[p, g * d + j] for p in range(r))
            assert abs(got[0, h, j] - want) < 1e-13


def pin_base_only_is_sdpa():
    rng = np.random.default_rng(10)
    for (Lq, Lk, Hq, Hkv, d) in [(7, 19, 4, 2, 16), (19, 19, 2, 2, 8), (1, 33, 8, 1, 32)]:
        Q, K, V, L, B = _rand_problem(Lq, Lk, Hq, Hkv, d, 4, rng)
        G = Hq // Hkv
        mask = torch.ones(Lq, Lk, dtype=torch.bool).tril(diagonal=Lk - Lq)   # bottom-right
        q = torch.from_numpy(Q).permute(1, 0, 2)
        k = torch.from_numpy(np.repeat(K, G, axis=1)).permute(1, 0, 2)
        v = torch.from_numpy(np.repeat(V, G, axis=1)).permute(1, 0, 2)
        want = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)
        want = want.permute(1, 0, 2).numpy()
        # B = 0 and rank 0 both reduce Flash-LoRA-Attention to plain attention.
        np.testing.assert_allclose(oracle.attention_request(Q, K, V, L, np.zeros_like(B)),
                                   want, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(
            oracle.attention_request(Q, K, V, L[:, :0], B[:0]), want, rtol=1e-11, atol=1e-12)


def pin_uniform_attention_prefix_mean():
    # K = 0: every visible key gets the same weight, so row t is the mean of the
    # expanded values over keys 0 .. Lk-Lq+t.
    rng = np.random.default_rng(11)
    Lq, Lk, Hq, Hkv, d, r = 6, 13, 4, 2, 8, 3
    Q, K, V, L, B = _rand_problem(Lq, Lk, Hq, Hkv, d, r, rng)
    K[:] = 0.0
    LB = (L @ B).reshape(Lk, Hkv, d)
    Vf = V + LB
    csum = np.cumsum(Vf, axis=0)
    got = oracle.attention_request(Q, K, V, L, B)
    for t in range(Lq):
        p = Lk - Lq + t
        for h in range(Hq):
            g = h // (Hq // Hkv)
            np.testing.assert_allclose(got[t, h], csum[p, g] / (p + 1), rtol=1e-12, atol=1e-12)


def pin_peaked_attention():
    # Orthogonal keys; query = big multiple of one visible key: softmax is one-hot to
    # far below fp64 resolution, so the output is that key's expanded value.
    rng = np.random.default_rng(12)
    Lk, Lq, Hkv, Hq, d, r = 6, 3, 1, 2, 8, 2
    _, _, V, L, B = _rand_problem(Lq, Lk, Hq, Hkv, d, r, rng)
    c = 12.0 * d ** 0.25
    K = np.zeros((Lk, Hkv, d))
    for s in range(Lk):
        K[s, 0, s] = c
    Q = np.zeros((Lq, Hq, d))
    pick = [[1, 3], [0, 2], [5, 3]]        # visible key per (row, head)
    for t in range(Lq):
        for h in range(Hq):
            Q[t, h, pick[t][h]] = c
    got = oracle.attention_request(Q, K, V, L, B)
    for t in range(Lq):
        for h in range(Hq):
            s = pick[t][h]
            want = V[s, 0] + L[s] @ B
            np.testing.assert_allclose(got[t, h], want, rtol=1e-12, atol=1e-12)


def pin_mask_boundary():
    # Row t must ignore keys after position Lk-Lq+t and must depend on the key at it.
    rng = np.random.default_rng(13)
    Lq, Lk, Hq, Hkv, d, r = 4, 9, 2, 1, 4, 2
    Q, K, V, L, B = _rand_problem(Lq, Lk, Hq, Hkv, d, r, rng)
    base = oracle.attention_request(Q, K, V, L, B)
    for t in range(Lq - 1):
        p = Lk - Lq + t
        K2, V2 = K.copy(), V.copy()
        K2[p + 1] += 3.0
        V2[p + 1] += 3.0
        o2 = oracle.attention_request(Q, K2, V2, L, B)
        np.testing.assert_array_equal(o2[:t + 1], base[:t + 1])
        assert np.abs(o2[t + 1:] - base[t + 1:]).max() > 1e-3
        V3 = V.copy()
        V3[p] += 3.0
        o3 = oracle.attention_request(Q, K, V3, L, B)
        assert np.abs(o3[t] - base[t]).max() > 1e-3


PINS = [pin_worked_example, pin_brute_force, pin_gqa_is_repeated_mha, pin_single_key,
        pin_base_only_is_sdpa, pin_uniform_attention_prefix_mean, pin_peaked_attention,
        pin_mask_boundary]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# ---------------------------------------------------------------------------------------
# Invariants the method fixes
# ---------------------------------------------------------------------------------------

def test_regrouping_identity_and_softmax_rows():
    # LRAgent section 3: P(V_base + V_lr B) = P V_base + (P V_lr) B.
    rng = np.random.default_rng(14)
    Lq, Lk, Hq, Hkv, d, r = 9, 23, 4, 2, 8, 5
    Q, K, V, L, B = _rand_problem(Lq, Lk, Hq, Hkv, d, r, rng)
    O, diag = oracle.attention_request(Q, K, V, L, B, return_diag=True)
    G = Hq // Hkv
    pos = Lk - Lq + np.arange(Lq)
    for h in range(Hq):
        g = h // G
        P = diag["P"][h]
        assert np.all(P >= 0)
        np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-14)
        masked = np.arange(Lk)[None, :] > pos[:, None]
        assert np.all(P[masked] == 0.0)
        regrouped = P @ V[:, g, :] + (P @ L) @ B[:, g * d:(g + 1) * d]
        np.testing.assert_allclose(O[:, h, :], regrouped, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(diag["O_base"][:, h] + diag["O_lr"][:, h], O[:, h],
                                   rtol=1e-12, atol=1e-13)


def test_linearity_in_values():
    rng = np.random.default_rng(15)
    Q, K, V, L, B = _rand_problem(5, 12, 4, 4, 8, 3, rng)
    o = oracle.attention_request(Q, K, V, L, B)
    o_base = oracle.attention_request(Q, K, V, L, np.zeros_like(B))
    o_lr = oracle.attention_request(Q, K, np.zeros_like(V), L, B)
    np.testing.assert_allclose(o, o_base + o_lr, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(oracle.attention_request(Q, K, 2.5 * V, L, 2.5 * B), 2.5 * o,
                               rtol=1e-12, atol=1e-13)


def test_batch_semantics_shared_context_and_relabelling():
    rng = np.random.default_rng(16)
    Hq, Hkv, d = 4, 2, 8
    ranks = [2, 3, 0]
    Lk = 17
    K = rng.standard_normal((Lk, Hkv, d))
    V = rng.standard_normal((Lk, Hkv, d))
    Ls = [rng.standard_normal((Lk, r)) for r in ranks]
    Bs = [rng.standard_normal((r, Hkv * d)) for r in ranks]
    Q = rng.standard_normal((12, Hq, d))
    q_start, q_len = [0, 5, 9], [5, 4, 3]
    k_start, k_len = [0, 0, 4], [17, 9, 13]          # requests 0 and 1 share base rows
    agent = [0, 1, 2]
    O = oracle.attention_batch(Q, K, V, Ls, Bs, q_start, q_len, k_start, k_len, agent)
    for b in range(3):
        qs, ks = q_start[b], k_start[b]
        want = oracle.attention_request(Q[qs:qs + q_len[b]], K[ks:ks + k_len[b]],
                                        V[ks:ks + k_len[b]], Ls[agent[b]][ks:ks + k_len[b]],
                                        Bs[agent[b]])
        np.testing.assert_array_equal(O[qs:qs + q_len[b]], want)
    perm = [2, 0, 1]                                   # new index of old agent a
    Ls2, Bs2 = [None] * 3, [None] * 3
    for a in range(3):
        Ls2[perm[a]], Bs2[perm[a]] = Ls[a], Bs[a]
    O2 = oracle.attention_batch(Q, K, V, Ls2, Bs2, q_start, q_len, k_start, k_len,
                                [perm[a] for a in agent])
    np.testing.assert_array_equal(O, O2)


def test_precompute_worked_example_and_brute_force():
    ex = json.load(open(os.path.join(GOLDEN, "worked_example_precompute.json")))
    X = np.array(ex["X"], dtype=np.float64)
    A = [np.array(a, dtype=np.float64) for a in ex["A"]]
    got = oracle.lr_precompute(X, A)
    for g, w in zip(got, ex["expected_L"]):
        np.testing.assert_array_equal(g, np.array(w, dtype=np.float64))
    rng = np.random.default_rng(17)
    X = rng.standard_normal((7, 5))
    A = [rng.standard_normal((5, r)) for r in (1, 3, 2)]
    got = oracle.lr_precompute(X, A)
    for a, Aa in enumerate(A):
        for t in range(7):
            for j in range(Aa.shape[1]):
                want = sum(X[t, i] * Aa[i, j] for i in range(5))
                assert abs(got[a][t, j] - want) < 1e-12


# ---------------------------------------------------------------------------------------
# Planted mistakes: each must make at least one pin fail
# ---------------------------------------------------------------------------------------

def _drop_lr(V_base, L, B):
    return np.asarray(V_base, dtype=np.float64)


def _lr_sign(V_base, L, B):
    Vb = np.asarray(V_base, dtype=np.float64)
    Lk, Hkv, d = Vb.shape
    return Vb - (np.asarray(L) @ np.asarray(B)).reshape(Lk, Hkv, d)


def _b_head_major_wrong(V_base, L, B):
    Vb = np.asarray(V_base, dtype=np.float64)
    Lk, Hkv, d = Vb.shape
    return Vb + (np.asarray(L) @ np.asarray(B)).reshape(Lk, d, Hkv).transpose(0, 2, 1)


MUTATIONS = {
    "lr term dropped": ("full_value_cache", _drop_lr),
    "lr term sign": ("full_value_cache", _lr_sign),
    "B columns read head-minor": ("full_value_cache", _b_head_major_wrong),
    "scale 1/d": ("softmax_scale", lambda d: 1.0 / d),
    "no scale": ("softmax_scale", lambda d: 1.0),
    "gqa h mod Hkv": ("kv_head_of", lambda h, hq, hkv: h % hkv),
    "mask off by one (strict)": ("visible", lambda pos, lk: np.arange(lk)[None, :] < np.asarray(pos)[:, None]),
    "mask off by one (lax)": ("visible", lambda pos, lk: np.arange(lk)[None, :] <= np.asarray(pos)[:, None] + 1),
    "top-left causal": ("query_positions", lambda lq, lk: np.arange(lq)),
    "no mask": ("visible", lambda pos, lk: np.ones((len(pos), lk), dtype=bool)),
}


# a planted strict mask leaves a query row with no visible key: its softmax is 0/0 (NaN),
# which the pins then reject, as they should
@pytest.mark.filterwarnings("ignore:invalid value encountered:RuntimeWarning")
@pytest.mark.parametrize("name", list(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(fo, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"planted mistake '{name}' passed every pin"
