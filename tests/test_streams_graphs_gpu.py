"""The C ABI's calls on a caller's stream: work goes to the stream passed in (here a side
stream), and a call queues kernels only (no allocation, copy or synchronisation), so a
sequence of calls can be captured into a HIP graph and replayed.  Outputs are compared
bitwise with the same calls made eagerly on the default stream, and once against the
oracle."""

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


def _problems():
    # prefill whose keys the planner splits 5 ways (combine pass) and a decode batch with
    # key splits (combine pass) and a request short enough for one split
    pre = workloads.custom("graph-prefill", "bf16", 8, 2, 128, (32,), [90], [3000], [0],
                           seed=700)
    dec = workloads.custom("graph-decode", "bf16", 32, 8, 128, (16, 64), [1] * 5,
                           [70, 1500, 4096, 9000, 33], [0, 1, 1, 0, 1], seed=701)
    return pre, dec


def _prepared(lra, pre, dev_p, dec, dev_d):
    """Both calls with their outputs and workspaces allocated up front."""
    O_p = torch.empty_like(dev_p["Q"])
    O_d = torch.empty_like(dev_d["Q"])
    ws_p = torch.empty(max(1, lra.lra_attn_workspace_bytes(
        torch.bfloat16, False, pre.q_len, pre.k_len, 8, 2, 128, 32)), dtype=torch.uint8,
        device="cuda")
    ws_d = torch.empty(max(1, lra.lra_attn_workspace_bytes(
        torch.bfloat16, True, None, dec.k_len, 32, 8, 128, 64)), dtype=torch.uint8,
        device="cuda")
    fp = lra.prepare_attn_prefill(dev_p["Q"], dev_p["K"], dev_p["V"], dev_p["L"], dev_p["B"],
                                  pre.q_start, pre.q_len, pre.k_start, pre.k_len,
                                  pre.agent_idx, O=O_p, workspace=ws_p)
    fd = lra.prepare_attn_decode(dev_d["Q"], dev_d["K"], dev_d["V"], dev_d["L"], dev_d["B"],
                                 dec.k_start, dec.k_len, dec.agent_idx, O=O_d, workspace=ws_d)
    return fp, fd, O_p, O_d


def test_calls_on_a_side_stream(lra, monkeypatch):
    monkeypatch.setenv("LRA_PREFILL_TARGET_WG", "64")
    pre, dec = _problems()
    cpu_p, dev_p = H.device_inputs(pre)
    cpu_d, dev_d = H.device_inputs(dec)
    fp, fd, O_p, O_d = _prepared(lra, pre, dev_p, dec, dev_d)
    fp()
    fd()
    torch.cuda.synchronize()
    want_p, want_d = O_p.clone(), O_d.clone()
    H.assert_bf16_close(want_p.float().cpu().numpy(), H.oracle_all(pre, cpu_p), "prefill")
    H.assert_bf16_close(want_d.float().cpu().numpy(), H.oracle_all(dec, cpu_d), "decode")
    O_p.zero_()
    O_d.zero_()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        fp()          # the binding passes the current (side) stream to the library
        fd()
    side.synchronize()
    assert torch.equal(O_p, want_p) and torch.equal(O_d, want_d)


def test_one_shot_call_on_a_side_stream_keeps_its_scratch(lra, monkeypatch):
    """A one-shot call with stream=side and no workspace: the binding allocates the
    workspace and the output itself, queues the split kernels and the combine pass on the
    side stream and returns.  Memory allocated and filled on the default stream right after
    must not land in that scratch while the side stream may still use it."""
    monkeypatch.setenv("LRA_PREFILL_TARGET_WG", "64")
    pre, dec = _problems()
    cpu_p, dev_p = H.device_inputs(pre)
    cpu_d, dev_d = H.device_inputs(dec)
    want_p = H.run_prefill(pre, dev_p).clone()
    want_d = H.run_decode(dec, dev_d).clone()
    ws_p = lra.lra_attn_workspace_bytes(torch.bfloat16, False, pre.q_len, pre.k_len, 8, 2, 128, 32)
    ws_d = lra.lra_attn_workspace_bytes(torch.bfloat16, True, None, dec.k_len, 32, 8, 128, 64)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        outs.append(lra.lra_attn_prefill(dev_p["Q"], dev_p["K"], dev_p["V"], dev_p["L"],
                                         dev_p["B"], pre.q_start, pre.q_len, pre.k_start,
                                         pre.k_len, pre.agent_idx, stream=side))
        outs.append(lra.lra_attn_decode(dev_d["Q"], dev_d["K"], dev_d["V"], dev_d["L"],
                                        dev_d["B"], dec.k_start, dec.k_len, dec.agent_idx,
                                        stream=side))
        # blocks of the scratch's own sizes, written on the default stream at once
        junk = [torch.full((n,), 0x7F, dtype=torch.uint8, device="cuda")
                for n in (ws_p, ws_d, ws_p, ws_d) if n]
        junk += [torch.full_like(dev_p["Q"], 9.0), torch.full_like(dev_d["Q"], 9.0)]
        del junk
    side.synchronize()
    torch.cuda.synchronize()
    for i, O in enumerate(outs):
        assert torch.equal(O, want_p if i % 2 == 0 else want_d), f"call {i}"
    H.assert_bf16_close(want_p.float().cpu().numpy(), H.oracle_all(pre, cpu_p), "prefill")
    H.assert_bf16_close(want_d.float().cpu().numpy(), H.oracle_all(dec, cpu_d), "decode")


def test_graph_capture_and_replay(lra, monkeypatch):
    monkeypatch.setenv("LRA_PREFILL_TARGET_WG", "64")
    pre, dec = _problems()
    _, dev_p = H.device_inputs(pre)
    _, dev_d = H.device_inputs(dec)
    fp, fd, O_p, O_d = _prepared(lra, pre, dev_p, dec, dev_d)
    fp()
    fd()
    torch.cuda.synchronize()
    want_p, want_d = O_p.clone(), O_d.clone()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fp()
        fd()
    for rep in range(4):
        # eager work between replays: clear the outputs (a fill kernel) and make an eager
        # call that reuses both workspaces
        O_p.zero_()
        O_d.zero_()
        fd()
        torch.cuda.synchronize()
        O_d.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(O_p, want_p), f"prefill differs on replay {rep}"
        assert torch.equal(O_d, want_d), f"decode differs on replay {rep}"
    del g


def test_append_graph_capture_and_replay(lra):
    """The two-pass bf16 append (slice partials in a caller workspace, then the ordered
    sums) captured into a graph: every replay writes the eager result, bitwise, with an
    eager call that reuses the workspace between replays."""
    p = workloads.PrecomputeProblem("graph-append", "bf16", 64, 4096, (16, 16, 16, 16), seed=702)
    X = p.X().cuda()
    A_cat = torch.cat([p.A(a) for a in range(4)], 1).contiguous().cuda()
    rows = np.arange(64) * 7 + 3
    outs = [torch.zeros(500, 16, dtype=torch.bfloat16, device="cuda") for _ in range(4)]
    ws = torch.empty(lra.lra_append_workspace_bytes(torch.bfloat16, 64, 4096, (16,) * 4),
                     dtype=torch.uint8, device="cuda")
    fa = lra.prepare_append_lr(X, A_cat, (16,) * 4, outs, rows, workspace=ws)
    fa()
    torch.cuda.synchronize()
    want = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa()
    for rep in range(4):
        for o in outs:
            o.zero_()
        fa()
        torch.cuda.synchronize()
        for o in outs:
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        for a in range(4):
            assert torch.equal(outs[a], want[a]), f"agent {a} differs on replay {rep}"
    del g
