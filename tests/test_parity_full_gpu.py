"""GPU parity at the benchmark workloads' full sizes, in the launch configurations the
benchmark times, against the fp64 oracle on the same stored inputs.

Every output row is compared for the tiny fp32 workload, the Llama prefill (all three
agents), the decode batch, the shared-context decode batch and the long-context prefill
(all three agents, on the GPU's own LR precompute).  The LR term (P·L)·B is small next to
P·V_base at these sizes, so each of those workloads is also run LR-isolated (V_base = 0,
O = (P·L)·B) under the relative Frobenius gate.  The 32-layer mixed batch checks every
request of every layer (first, last and two random query rows) and every row of layers
0, 17 and 31.  The comparators of the regrouping (the naive expansion route and the
in-tile expansion route) are checked on the same rows at the Llama prefill, decode and
long-context shapes."""

import numpy as np
import pytest
import torch

import oracle
from shared_rank_kv_amd import inputs, workloads

import helpers as H

pytestmark = pytest.mark.gpu
RNG = np.random.default_rng(2026)


def _check_rows(prob, cpu, O, requests, what, n_rows=None, rel_frob=H.REL_FROB, also=None):
    """Compare the rows of `requests` (all rows, or first/last/random n_rows of each); the
    outputs in `also` ({name: O}) are compared with the same oracle rows."""
    outs = {what: O, **{f"{what}, {k}": v for k, v in (also or {}).items()}}
    got_all = {k: v.float().cpu().numpy() for k, v in outs.items()}
    idx, wants = [], []
    for b in requests:
        lq, qs = int(prob.q_len[b]), int(prob.q_start[b])
        if lq == 0:
            continue
        rows = np.arange(lq) if n_rows is None else H.sample_rows(lq, n_rows, RNG)
        wants.append(H.oracle_rows(prob, cpu, b, rows))
        idx.append(qs + rows)
    idx, want = np.concatenate(idx), np.concatenate(wants)
    for name, got in got_all.items():
        mx, mean, rel = H.assert_bf16_close(got[idx], want, name, rel_frob)
        print(f"{name}: {len(idx)} rows, max-abs {mx:.2e} mean-abs {mean:.2e} rel-frob {rel:.2e}")


def _comparators(prob, dev, decode):
    """The naive route (V_full materialised, then plain attention) and the in-tile expansion
    route on the same device inputs, in the benchmark's launch configuration."""
    from shared_rank_kv_amd import lra
    Vf = lra.lra_expand_values(dev["V"], dev["L"], dev["B"], prob.k_start, prob.k_len,
                               prob.agent_idx)
    zero = np.zeros(prob.batch, np.int32)
    if decode:
        naive = lra.lra_attn_decode(dev["Q"], dev["K"], Vf, [None], [None], prob.k_start,
                                    prob.k_len, zero)
        tile = lra.lra_attn_decode_expand(dev["Q"], dev["K"], dev["V"], dev["L"], dev["B"],
                                          prob.k_start, prob.k_len, prob.agent_idx)
    else:
        naive = lra.lra_attn_prefill(dev["Q"], dev["K"], Vf, [None], [None], prob.q_start,
                                     prob.q_len, prob.k_start, prob.k_len, zero)
        tile = lra.lra_attn_prefill_expand(dev["Q"], dev["K"], dev["V"], dev["L"], dev["B"],
                                           prob.q_start, prob.q_len, prob.k_start, prob.k_len,
                                           prob.agent_idx)
    torch.cuda.synchronize()
    del Vf
    return {"naive expansion": naive, "in-tile expansion": tile}


def test_tiny_fp32_full():
    prob = workloads.tiny_fp32()
    cpu, dev = H.device_inputs(prob)
    O = H.run_prefill(prob, dev)
    mx, _, _ = H.assert_f32_close(O.cpu().numpy(), H.oracle_all(prob, cpu), prob.name)
    print(f"{prob.name}: max-abs {mx:.2e}")


def test_llama_prefill_9216k_every_row():
    base = workloads.llama_prefill(agents=(0,))
    cpu, dev = H.device_inputs(base)
    for agent in range(3):
        prob = base.with_agents([agent])
        O = H.run_prefill(prob, dev)
        also = _comparators(prob, dev, False) if agent == 0 else None
        _check_rows(prob, cpu, O, [0], f"llama prefill agent {agent}", also=also)
    # LR-isolated: V_base = 0 leaves O = (P·L)·B
    dev["V"].zero_()
    cpu["V"] = torch.zeros_like(cpu["V"])
    O = H.run_prefill(base, dev)
    _check_rows(base, cpu, O, [0], "llama prefill agent 0, LR-isolated")


def test_decode_64x16k_every_request():
    prob = workloads.decode_batch()
    cpu, dev = H.device_inputs(prob)
    O = H.run_decode(prob, dev)
    _check_rows(prob, cpu, O, range(prob.batch), "decode 64x16384",
                also=_comparators(prob, dev, True))
    dev["V"].zero_()
    cpu["V"] = torch.zeros_like(cpu["V"])
    O = H.run_decode(prob, dev)
    _check_rows(prob, cpu, O, range(prob.batch), "decode 64x16384, LR-isolated")


def test_decode_shared_16x4x16k_every_request():
    prob = workloads.decode_shared_batch()
    cpu, dev = H.device_inputs(prob)
    O = H.run_decode(prob, dev)
    _check_rows(prob, cpu, O, range(prob.batch), "shared-context decode 16x4x16384")
    dev["V"].zero_()
    cpu["V"] = torch.zeros_like(cpu["V"])
    O = H.run_decode(prob, dev)
    _check_rows(prob, cpu, O, range(prob.batch), "shared-context decode, LR-isolated")


def test_longctx_precompute_then_prefill_every_row():
    from shared_rank_kv_amd import lra
    pre = workloads.longctx_precompute()
    X = pre.X()
    A = [pre.A(a) for a in range(3)]
    Xd = X.cuda()
    A_cat = torch.cat(A, 1).contiguous().cuda()
    Ls = [torch.empty(pre.T, r, dtype=torch.bfloat16, device="cuda") for r in pre.ranks]
    lra.lra_precompute_lr(Xd, A_cat, pre.ranks, Ls)
    torch.cuda.synchronize()
    del Xd
    # the precompute against the oracle's: every row, within the error bound of fp32
    # accumulation plus the final rounding to bf16
    Xf = inputs.to_f64(X)
    del X
    Af = [inputs.to_f64(a) for a in A]
    L_oracle = oracle.lr_precompute(Xf, Af)
    absX = np.abs(Xf)
    for a in range(3):
        got = Ls[a].double().cpu().numpy()
        bound = pre.d_model * 2.0 ** -23 * (absX @ np.abs(Af[a])) + 2.0 ** -8 * np.abs(L_oracle[a])
        assert np.all(np.abs(got - L_oracle[a]) <= bound), f"precompute agent {a}"
    del Xf, absX
    # attention over the GPU's LR caches vs the oracle chained on its own fp64 LR caches
    base = workloads.longctx_prefill(agents=(0,))
    cpu = {"Q": base.Q(), "K": base.K(), "V": base.V(), "B": [base.B(a) for a in range(3)]}
    dev = {"Q": cpu["Q"].cuda(), "K": cpu["K"].cuda(), "V": cpu["V"].cuda(), "L": Ls,
           "B": [b.cuda() for b in cpu["B"]]}
    Q64, K64 = inputs.to_f64(cpu["Q"]), inputs.to_f64(cpu["K"])
    rows = np.arange(512)

    def check(agent, V64, what, comparators=False):
        prob = base.with_agents([agent])
        outs = {what: H.run_prefill(prob, dev)}
        if comparators:
            outs.update({f"{what}, {k}": v for k, v in _comparators(prob, dev, False).items()})
        want = oracle.attention_request(Q64, K64, V64, L_oracle[agent],
                                        inputs.to_f64(cpu["B"][agent]),
                                        positions=(32768 - 512) + rows)
        for name, O in outs.items():
            mx, mean, rel = H.assert_bf16_close(O.float().cpu().numpy(), want, name)
            print(f"{name}: 512 rows, max-abs {mx:.2e} mean-abs {mean:.2e} rel-frob {rel:.2e}")

    V64 = inputs.to_f64(cpu["V"])
    for agent in range(3):
        check(agent, V64, f"longctx agent {agent}", comparators=agent == 0)
    dev["V"].zero_()
    check(0, np.zeros_like(V64), "longctx agent 0, LR-isolated")


@pytest.mark.parametrize("layer", range(workloads.MIXED_LAYERS))
def test_mixed_batch_layer(layer):
    prob = workloads.mixed_batch_layer(layer)
    cpu, dev = H.device_inputs(prob)
    O = H.run_prefill(prob, dev)
    if layer in (0, 17, 31):
        _check_rows(prob, cpu, O, range(prob.batch), f"mixed layer {layer}, every row")
    else:
        _check_rows(prob, cpu, O, range(prob.batch), f"mixed layer {layer}", n_rows=4)
