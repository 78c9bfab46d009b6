"""GPU parity at the benchmark workloads' full sizes, in the launch configuration the benchmark
times, on outputs sampled so the fp64 oracle can evaluate them row by row."""

import numpy as np
import pytest
import torch

import oracle
from shared_rank_kv_amd import inputs, workloads

import helpers as H

pytestmark = pytest.mark.gpu
RNG = np.random.default_rng(2026)


def _check_sampled(prob, cpu, O, requests, n_rows, what):
    got_all = O.float().cpu().numpy()
    gots, wants = [], []
    for b in requests:
        lq, qs = int(prob.q_len[b]), int(prob.q_start[b])
        rows = H.sample_rows(lq, n_rows, RNG)
        wants.append(H.oracle_rows(prob, cpu, b, rows))
        gots.append(got_all[qs + rows])
    got, want = np.concatenate(gots), np.concatenate(wants)
    mx, mean, rel = H.assert_bf16_close(got, want, what)
    print(f"{what}: max-abs {mx:.2e} mean-abs {mean:.2e} rel-frob {rel:.2e}")


@pytest.mark.parametrize("agent", [0, 1, 2])
def test_llama_prefill_9216k(agent):
    prob = workloads.llama_prefill(agents=(agent,))
    cpu, dev = H.device_inputs(prob)
    O = H.run_prefill(prob, dev)
    _check_sampled(prob, cpu, O, [0], 40, f"llama prefill agent {agent}")


def test_decode_64x16k():
    prob = workloads.decode_batch()
    cpu, dev = H.device_inputs(prob)
    O = H.run_decode(prob, dev)
    reqs = sorted(RNG.choice(prob.batch, size=8, replace=False).tolist() + [0, prob.batch - 1])
    _check_sampled(prob, cpu, O, sorted(set(reqs)), 1, "decode 64x16384")


def test_decode_shared_16x4x16k():
    # every member of the first and last context, and a random request of every other one
    prob = workloads.decode_shared_batch()
    cpu, dev = H.device_inputs(prob)
    O = H.run_decode(prob, dev)
    reqs = [0, 1, 2, 3, 60, 61, 62, 63] + [4 * c + int(RNG.integers(4)) for c in range(1, 15)]
    _check_sampled(prob, cpu, O, sorted(set(reqs)), 1, "shared-context decode 16x4x16384")


def test_longctx_precompute_then_prefill():
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
    # precompute parity on sampled rows, against the error bound of fp32 accumulation + bf16
    rows = np.sort(RNG.choice(pre.T, size=64, replace=False))
    Xs = inputs.to_f64(X[torch.from_numpy(rows)])
    Af = [inputs.to_f64(a) for a in A]
    want = oracle.lr_precompute(Xs, Af)
    for a in range(3):
        got = Ls[a].double().cpu().numpy()[rows]
        bound = pre.d_model * 2.0 ** -23 * (np.abs(Xs) @ np.abs(Af[a])) + 2.0 ** -8 * np.abs(want[a])
        assert np.all(np.abs(got - want[a]) <= bound), f"precompute agent {a}"
    # attention over the GPU's LR caches vs the oracle chained on its own fp64 LR caches
    L_oracle = oracle.lr_precompute(inputs.to_f64(X), Af)
    del X
    for agent in range(3):
        prob = workloads.longctx_prefill(agents=(agent,))
        cpu = {"Q": prob.Q(), "K": prob.K(), "V": prob.V(),
               "B": [prob.B(a) for a in range(3)]}
        dev = {"Q": cpu["Q"].cuda(), "K": cpu["K"].cuda(), "V": cpu["V"].cuda(), "L": Ls,
               "B": [b.cuda() for b in cpu["B"]]}
        O = H.run_prefill(prob, dev)
        rows = H.sample_rows(512, 24, RNG)
        want = oracle.attention_request(inputs.to_f64(cpu["Q"])[rows], inputs.to_f64(cpu["K"]),
                                        inputs.to_f64(cpu["V"]), L_oracle[agent],
                                        inputs.to_f64(cpu["B"][agent]),
                                        positions=(32768 - 512) + rows)
        got = O.float().cpu().numpy()[rows]
        mx, mean, rel = H.assert_bf16_close(got, want, f"longctx agent {agent}")
        print(f"longctx agent {agent}: max-abs {mx:.2e} mean-abs {mean:.2e} rel-frob {rel:.2e}")


@pytest.mark.parametrize("layer", [0, 17, 31])
def test_mixed_batch_layer(layer):
    prob = workloads.mixed_batch_layer(layer)
    cpu, dev = H.device_inputs(prob)
    O = H.run_prefill(prob, dev)
    reqs = sorted(set(RNG.choice(prob.batch, size=6, replace=False).tolist()))
    _check_sampled(prob, cpu, O, reqs, 8, f"mixed layer {layer}")
