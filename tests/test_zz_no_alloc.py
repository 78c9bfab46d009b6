"""lra_attn_decode_noalloc through the C ABI: the decode with the library's fixed scratch
array instead of a caller workspace.  Its outputs must equal lra_attn_decode's bitwise (the
same plan and kernels) and the oracle's within the bf16 tolerances, on two calls in a row
(the second smaller, with the first call's contents left in the scratch), and a call whose
plan needs more scratch than the array holds is refused before anything is queued."""

import ctypes

import numpy as np
import pytest
import torch

from shared_rank_kv_amd import workloads

import helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lra():
    from shared_rank_kv_amd import lra   # fails loudly if liblra.so is missing
    assert torch.cuda.is_available()
    return lra


def _check(lra, prob):
    cpu, dev = H.device_inputs(prob)
    need = lra.lra_attn_workspace_bytes(torch.bfloat16, True, None, prob.k_len, prob.n_q_heads,
                                        prob.n_kv_heads, prob.head_dim, max(prob.ranks))
    assert 0 < need <= lra.lib_noalloc_scratch_bytes()
    want = H.run_decode(prob, dev).clone()
    O = torch.full_like(dev["Q"], 5.0)
    lra.lra_attn_decode_noalloc(dev["Q"], dev["K"], dev["V"], dev["L"], dev["B"], prob.k_start,
                                prob.k_len, prob.agent_idx, O)
    torch.cuda.synchronize()
    assert torch.equal(O, want), f"{prob.name}: differs from lra_attn_decode"
    H.assert_bf16_close(O.float().cpu().numpy(), H.oracle_all(prob, cpu), prob.name)
    return need


def test_noalloc_decode_matches_the_workspace_decode(lra):
    big = workloads.decode_batch()                  # 64 x 16384 keys: 16 splits each
    small = workloads.custom("noalloc-small", "bf16", 32, 8, 128, (16, 64, 0), [1] * 7,
                             [1, 33, 1000, 3000, 5000, 64, 2049], [0, 1, 2, 1, 0, 1, 0],
                             seed=901)
    n_big = _check(lra, big)
    n_small = _check(lra, small)                    # the scratch still holds the big call's
    assert n_small < n_big


def test_noalloc_decode_refuses_a_plan_beyond_the_scratch(lra):
    # 1024 requests over one 65536-key context plan 64 splits each: far more scratch than
    # the fixed array; the call is refused on the host and the output stays untouched
    batch, Hq, Hkv, D = 1024, 32, 8, 128
    K = torch.zeros(65536, Hkv, D, dtype=torch.bfloat16, device="cuda")
    Q = torch.zeros(batch, Hq, D, dtype=torch.bfloat16, device="cuda")
    O = torch.full_like(Q, 3.0)
    need = lra.lra_attn_workspace_bytes(torch.bfloat16, True, None, [65536] * batch, Hq, Hkv, D, 0)
    assert need > lra.lib_noalloc_scratch_bytes()
    with pytest.raises(lra.LraError) as e:
        lra.lra_attn_decode_noalloc(Q, K, K, [None], [None], [0] * batch, [65536] * batch,
                                    [0] * batch, O)
    assert e.value.code == lra.LRA_ERR_WORKSPACE and "fixed scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((O == 3.0).all())
