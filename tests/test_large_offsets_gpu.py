"""Maximum-size addressing: small seeded problems placed at the far end of large device
buffers, so that every row the kernels touch lies beyond 2^31 (and 2^32) bytes from the
buffer's start.  The results must be bitwise equal to the same problems at offset 0, which
the oracle also checks.  Only the rows the requests name are written into the large
buffers (the rest stay uninitialised: the kernels must not read them)."""

import numpy as np
import pytest
import torch

from shared_rank_kv_amd import workloads

import helpers as H

pytestmark = pytest.mark.gpu

KV_BIG = (1 << 21) + 4096      # K/V rows: 4.3 GB per tensor at 8 kv heads x 128, bf16
Q_BIG = 300_000                # Q/O rows: 2.5 GB at 32 q heads x 128, bf16


@pytest.fixture(scope="module")
def lra():
    from shared_rank_kv_amd import lra   # fails loudly if liblra.so is missing
    assert torch.cuda.is_available()
    return lra


def _far(dev, prob, q_big):
    """The problem's tensors copied to the end of large buffers; returns them and offsets."""
    offk = KV_BIG - prob.kv_rows
    big = {"K": torch.empty((KV_BIG,) + tuple(dev["K"].shape[1:]), dtype=dev["K"].dtype,
                            device="cuda")}
    big["V"] = torch.empty_like(big["K"])
    big["K"][offk:] = dev["K"]
    big["V"][offk:] = dev["V"]
    big["L"] = []
    for L in dev["L"]:
        if L is None:
            big["L"].append(None)
            continue
        Lb = torch.empty((KV_BIG, L.shape[1]), dtype=L.dtype, device="cuda")
        Lb[offk:] = L
        big["L"].append(Lb)
    big["B"] = dev["B"]
    offq = 0
    if q_big:
        offq = Q_BIG - prob.q_rows
        big["Q"] = torch.empty((Q_BIG,) + tuple(dev["Q"].shape[1:]), dtype=dev["Q"].dtype,
                               device="cuda")
        big["Q"][offq:] = dev["Q"]
    else:
        big["Q"] = dev["Q"]
    return big, offk, offq


def test_prefill_far_rows(lra):
    prob = workloads.custom("far-prefill", "bf16", 32, 8, 128, (16, 64), [100, 37],
                            [700, 2000], [0, 1], seed=800)
    cpu, dev = H.device_inputs(prob)
    near = H.run_prefill(prob, dev)
    big, offk, offq = _far(dev, prob, q_big=True)
    assert offk * 8 * 128 * 2 > (1 << 32) and offq * 32 * 128 * 2 > (1 << 31)
    O = torch.empty_like(big["Q"])
    lra.lra_attn_prefill(big["Q"], big["K"], big["V"], big["L"], big["B"],
                         prob.q_start + offq, prob.q_len, prob.k_start + offk, prob.k_len,
                         prob.agent_idx, O=O)
    torch.cuda.synchronize()
    far = O[offq:]
    assert torch.equal(far, near), "prefill at large offsets differs from offset 0"
    rows = H.covered_rows(prob)
    H.assert_bf16_close(far.float().cpu().numpy()[rows], H.oracle_all(prob, cpu)[rows],
                        prob.name)


@pytest.mark.parametrize("shared", [False, True], ids=["own-contexts", "shared-context"])
def test_decode_far_rows(lra, shared):
    if shared:
        prob = workloads.custom("far-decode-shared", "bf16", 32, 8, 128, (16, 64, 8), [1] * 4,
                                [6000] * 4, [0, 1, 2, 1], seed=802, shared_k=True)
    else:
        prob = workloads.custom("far-decode", "bf16", 32, 8, 128, (16, 64), [1] * 3,
                                [5000, 77, 16384], [0, 1, 1], seed=801)
    cpu, dev = H.device_inputs(prob)
    near = H.run_decode(prob, dev)
    big, offk, _ = _far(dev, prob, q_big=False)
    O = torch.empty_like(dev["Q"])
    lra.lra_attn_decode(big["Q"], big["K"], big["V"], big["L"], big["B"], prob.k_start + offk,
                        prob.k_len, prob.agent_idx, O=O)
    torch.cuda.synchronize()
    assert torch.equal(O, near), "decode at large offsets differs from offset 0"
    H.assert_bf16_close(O.float().cpu().numpy(), H.oracle_all(prob, cpu), prob.name)


def test_append_far_rows(lra):
    p = workloads.PrecomputeProblem("far-append", "bf16", 48, 1024, (16, 64), seed=803)
    X = p.X().cuda()
    A_cat = torch.cat([p.A(0), p.A(1)], 1).contiguous().cuda()
    rows_near = np.arange(48) * 3 + 1
    near = [torch.zeros((200, r), dtype=torch.bfloat16, device="cuda") for r in (16, 64)]
    lra.lra_append_lr(X, A_cat, (16, 64), near, rows_near)
    # the LR caches as column blocks of one [2^21 + 16, 1024] buffer (4.3 GB); rows at its end
    buf = torch.empty(((1 << 21) + 16, 1024), dtype=torch.bfloat16, device="cuda")
    far = [buf[:, 100:116], buf[:, 512:576]]
    rows_far = rows_near + (1 << 21) - 200
    lra.lra_append_lr(X, A_cat, (16, 64), far, rows_far)
    torch.cuda.synchronize()
    for a in range(2):
        assert torch.equal(far[a][rows_far], near[a][rows_near]), f"agent {a}"


def test_precompute_far_rows(lra):
    # X rows 1 MB apart (ldx = 2^19 elements): the last rows sit ~4 GB into the buffer
    p = workloads.PrecomputeProblem("far-pre", "bf16", 4096, 512, (64, 64, 64), seed=804)
    X = p.X().cuda()
    A_cat = torch.cat([p.A(a) for a in range(3)], 1).contiguous().cuda()
    near = [torch.empty((4096, 64), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    lra.lra_precompute_lr(X, A_cat, (64, 64, 64), near)
    wide = torch.empty((4096, 1 << 19), dtype=torch.bfloat16, device="cuda")
    wide[:, :512] = X
    far = [torch.empty((4096, 64), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    lra.lra_precompute_lr(wide[:, :512], A_cat, (64, 64, 64), far)
    torch.cuda.synchronize()
    for a in range(3):
        assert torch.equal(far[a], near[a]), f"agent {a}"
