"""The C-ABI boundary on the host (no GPU, no kernel launches).

Checks that liblra.so loads and exports every function include/lra.h declares, and that
each malformed or unsupported call is rejected with its status code and a message before
anything is queued (every call here fails validation, so no HIP work is attempted; the
device pointers are fake, aligned addresses that are never dereferenced).
"""

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

lra = pytest.importorskip("shared_rank_kv_amd.lra")


def test_exports_every_declared_symbol():
    header = open(os.path.join(ROOT, "include", "lra.h")).read()
    declared = set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(lra_\w+)\s*\(", header, re.M))
    assert declared == set(lra.SYMBOLS)
    for name in declared:
        assert hasattr(lra.lib, name), name


FAKE = 0x10000          # 16-byte aligned, never dereferenced: every call below is rejected


class Call:
    """Arguments of one lra_attn_prefill call, valid by default, editable per test."""

    def __init__(self):
        self.dtype = lra.LRA_DTYPE_BF16
        self.Hq, self.Hkv, self.D = 8, 2, 128
        self.q_start, self.q_len = [0, 10], [10, 5]
        self.k_start, self.k_len = [0, 0], [100, 50]
        self.agent = [0, 1]
        self.q_rows, self.kv_rows = 15, 100
        self.ranks = [16, 8]
        self.L = [FAKE, FAKE + 4096]
        self.ldl = [16, 8]
        self.B = [FAKE, FAKE + 8192]
        self.Q = self.K = self.V = self.O = FAKE
        self.ws, self.ws_bytes = FAKE, 1 << 30
        self.batch = None

    def run(self):
        I = lambda a: (ctypes.c_int32 * max(1, len(a)))(*a)  # noqa: E731
        P = lambda a: (ctypes.c_void_p * max(1, len(a)))(*a)  # noqa: E731
        L64 = lambda a: (ctypes.c_int64 * max(1, len(a)))(*a)  # noqa: E731
        batch = len(self.q_len) if self.batch is None else self.batch
        cast_i = lambda a: ctypes.cast(a, ctypes.POINTER(ctypes.c_int32)) if a is not None else None  # noqa
        arrs = [I(x) if x is not None else None for x in
                (self.q_start, self.q_len, self.k_start, self.k_len, self.agent)]
        rc = lra.lib.lra_attn_prefill(
            self.dtype, batch, self.Hq, self.Hkv, self.D, *[cast_i(a) for a in arrs],
            self.Q, self.q_rows, self.K, self.V, self.kv_rows, len(self.ranks),
            cast_i(I(self.ranks)), ctypes.cast(P(self.L), ctypes.POINTER(ctypes.c_void_p)),
            ctypes.cast(L64(self.ldl), ctypes.POINTER(ctypes.c_int64)),
            ctypes.cast(P(self.B), ctypes.POINTER(ctypes.c_void_p)), self.O, self.ws,
            self.ws_bytes, None)
        return rc, lra.lra_last_error()


def _expect(call, code, fragment):
    rc, msg = call.run()
    assert rc == code, (rc, msg)
    assert fragment in msg, msg


INVALID_CASES = {
    "bad dtype": (lambda c: setattr(c, "dtype", 7), lra.LRA_ERR_INVALID, "dtype"),
    "negative batch": (lambda c: setattr(c, "batch", -1), lra.LRA_ERR_INVALID, "batch"),
    "heads not divisible": (lambda c: setattr(c, "Hq", 6) or setattr(c, "Hkv", 4),
                            lra.LRA_ERR_INVALID, "multiple"),
    "zero heads": (lambda c: setattr(c, "Hkv", 0), lra.LRA_ERR_INVALID, "positive"),
    "q_len > k_len": (lambda c: c.q_len.__setitem__(1, 60), lra.LRA_ERR_INVALID, "q_len"),
    "negative length": (lambda c: c.k_len.__setitem__(0, -1), lra.LRA_ERR_INVALID, "negative"),
    "query rows out of range": (lambda c: setattr(c, "q_rows", 12), lra.LRA_ERR_INVALID, "query rows"),
    "key rows out of range": (lambda c: c.k_start.__setitem__(1, 60), lra.LRA_ERR_INVALID, "key rows"),
    "agent out of range": (lambda c: c.agent.__setitem__(1, 2), lra.LRA_ERR_INVALID, "agent_idx"),
    "negative agent": (lambda c: c.agent.__setitem__(0, -1), lra.LRA_ERR_INVALID, "agent_idx"),
    "overlapping outputs": (lambda c: c.q_start.__setitem__(1, 5), lra.LRA_ERR_INVALID, "overlap"),
    "null Q": (lambda c: setattr(c, "Q", None), lra.LRA_ERR_INVALID, "non-null"),
    "misaligned K": (lambda c: setattr(c, "K", FAKE + 8), lra.LRA_ERR_INVALID, "aligned"),
    "null L": (lambda c: c.L.__setitem__(0, None), lra.LRA_ERR_INVALID, "null"),
    "ldl < rank": (lambda c: c.ldl.__setitem__(0, 8), lra.LRA_ERR_INVALID, "ldl"),
    "ldl not multiple of 8": (lambda c: c.ldl.__setitem__(0, 20), lra.LRA_ERR_INVALID, "multiple"),
    "misaligned L": (lambda c: c.L.__setitem__(1, FAKE + 2), lra.LRA_ERR_INVALID, "aligned"),
    "negative rank": (lambda c: c.ranks.__setitem__(1, -8), lra.LRA_ERR_INVALID, "< 0"),
    "null request array": (lambda c: setattr(c, "agent", None), lra.LRA_ERR_INVALID, "non-null"),
    "no agents": (lambda c: setattr(c, "ranks", []), lra.LRA_ERR_INVALID, "n_agents"),
}

UNSUPPORTED_CASES = {
    "head_dim 96": (lambda c: setattr(c, "D", 96), "head_dim"),
    "group 16": (lambda c: setattr(c, "Hq", 32) or setattr(c, "Hkv", 2), "group"),
    "rank 12": (lambda c: c.ranks.__setitem__(0, 12), "multiples of 8"),
    "rank 128": (lambda c: c.ranks.__setitem__(0, 128) or c.ldl.__setitem__(0, 128), "multiples of 8"),
    "17 agents": (lambda c: setattr(c, "ranks", [8] * 17) or setattr(c, "L", [FAKE] * 17)
                  or setattr(c, "B", [FAKE] * 17) or setattr(c, "ldl", [8] * 17), "LRA_MAX_AGENTS"),
    "batch 2000": (lambda c: setattr(c, "batch", 2000), "LRA_MAX_BATCH"),
    # 64 bf16 rows of K/V (n_kv_heads * head_dim * 2 bytes each) or of an LR cache must stay
    # below 2 GiB: the kernels address a tile with 32-bit byte offsets
    "K/V rows of 32 MiB": (lambda c: setattr(c, "Hq", 1 << 17) or setattr(c, "Hkv", 1 << 17),
                           "2 GiB"),
    "LR rows of 32 MiB": (lambda c: c.ldl.__setitem__(0, 1 << 24), "2 GiB"),
}


@pytest.mark.parametrize("name", list(INVALID_CASES))
def test_invalid_arguments_rejected(name):
    c = Call()
    edit, code, frag = INVALID_CASES[name]
    edit(c)
    _expect(c, code, frag)


@pytest.mark.parametrize("name", list(UNSUPPORTED_CASES))
def test_unsupported_arguments_rejected(name):
    c = Call()
    edit, frag = UNSUPPORTED_CASES[name]
    edit(c)
    _expect(c, lra.LRA_ERR_UNSUPPORTED, frag)


def test_workspace_checks():
    # a small batch over long keys gets split key ranges, hence a workspace
    c = Call()
    c.k_len, c.kv_rows = [4096, 4096], 4096
    need = lra.lra_attn_workspace_bytes(lra.LRA_DTYPE_BF16, False, c.q_len, c.k_len, c.Hq, c.Hkv,
                                        c.D, 16)
    assert need > 0
    c.ws = None
    _expect(c, lra.LRA_ERR_WORKSPACE, "null")
    c.ws, c.ws_bytes = FAKE, need - 1
    _expect(c, lra.LRA_ERR_WORKSPACE, "needed")
    # the query rejects what the call would reject
    assert lra.lib.lra_attn_workspace_bytes(7, 0, 0, None, None, 8, 2, 128, 16) == ctypes.c_size_t(-1).value
    # fp32 never needs scratch
    assert lra.lra_attn_workspace_bytes(lra.LRA_DTYPE_F32, False, [10], [4096], 8, 2, 128, 16) == 0


def test_workspace_size_is_monotone_in_keys_and_decode_splits():
    sizes = [lra.lra_attn_workspace_bytes(lra.LRA_DTYPE_BF16, True, None, [k] * 64, 32, 8, 128, 16)
             for k in (64, 1024, 4096, 16384)]
    assert sizes[0] == 0 and sizes == sorted(sizes)


def test_empty_calls_are_noops():
    c = Call()
    c.q_len = [0, 0]
    c.Q = c.K = c.V = c.O = None
    rc, _ = c.run()
    assert rc == lra.LRA_OK
    c.batch = 0
    rc, _ = c.run()
    assert rc == lra.LRA_OK


def _precompute(dtype=lra.LRA_DTYPE_BF16, T=100, dm=64, X=FAKE, ldx=64, A=FAKE, lda=24,
                ranks=(8, 16), L=(FAKE, FAKE + 4096), ldl=(8, 16)):
    I = (ctypes.c_int32 * len(ranks))(*ranks)
    P = (ctypes.c_void_p * len(L))(*L)
    LD = (ctypes.c_int64 * len(ldl))(*ldl)
    rc = lra.lib.lra_precompute_lr(dtype, T, dm, X, ldx, A, lda, len(ranks),
                                   ctypes.cast(I, ctypes.POINTER(ctypes.c_int32)),
                                   ctypes.cast(P, ctypes.POINTER(ctypes.c_void_p)),
                                   ctypes.cast(LD, ctypes.POINTER(ctypes.c_int64)), None)
    return rc, lra.lra_last_error()


@pytest.mark.parametrize("kw,code,frag", [
    (dict(dtype=3), lra.LRA_ERR_INVALID, "dtype"),
    (dict(T=-1), lra.LRA_ERR_INVALID, "T"),
    (dict(dm=0), lra.LRA_ERR_INVALID, "d_model"),
    (dict(dm=60, ldx=64), lra.LRA_ERR_UNSUPPORTED, "d_model"),
    (dict(dm=72, ldx=72), lra.LRA_ERR_UNSUPPORTED, "% 64"),
    (dict(ldx=32), lra.LRA_ERR_INVALID, "ldx"),
    (dict(lda=16), lra.LRA_ERR_INVALID, "lda"),
    (dict(lda=28), lra.LRA_ERR_INVALID, "lda"),
    (dict(ranks=(8, 20)), lra.LRA_ERR_UNSUPPORTED, "multiples of 8"),
    (dict(ranks=(8, -8)), lra.LRA_ERR_INVALID, "< 0"),
    (dict(ldl=(8, 8)), lra.LRA_ERR_INVALID, "ldl"),
    (dict(L=(FAKE, None)), lra.LRA_ERR_INVALID, "null"),
    (dict(X=FAKE + 4), lra.LRA_ERR_INVALID, "aligned"),
    (dict(X=None), lra.LRA_ERR_INVALID, "non-null"),
    (dict(ranks=(64,) * 5, L=(FAKE,) * 5, ldl=(64,) * 5, lda=320), lra.LRA_ERR_UNSUPPORTED, "256"),
])
def test_precompute_rejections(kw, code, frag):
    rc, msg = _precompute(**kw)
    assert rc == code, (rc, msg)
    assert frag in msg, msg


def test_precompute_empty_is_noop():
    assert _precompute(T=0, X=None, A=None)[0] == lra.LRA_OK


def _append(rows=(5, 0, 9), l_rows=10, batch=None, **kw):
    d = dict(dtype=lra.LRA_DTYPE_BF16, dm=64, X=FAKE, ldx=64, A=FAKE, lda=24, ranks=(8, 16),
             L=(FAKE, FAKE + 4096), ldl=(8, 16), ws=FAKE, ws_bytes=1 << 20)
    d.update(kw)
    batch = len(rows) if batch is None else batch
    I = (ctypes.c_int32 * len(d["ranks"]))(*d["ranks"])
    P = (ctypes.c_void_p * len(d["L"]))(*d["L"])
    LD = (ctypes.c_int64 * len(d["ldl"]))(*d["ldl"])
    RW = (ctypes.c_int32 * max(1, len(rows)))(*rows) if rows is not None else None
    rc = lra.lib.lra_append_lr(d["dtype"], batch, d["dm"], d["X"], d["ldx"], d["A"], d["lda"],
                               len(d["ranks"]), ctypes.cast(I, ctypes.POINTER(ctypes.c_int32)),
                               ctypes.cast(P, ctypes.POINTER(ctypes.c_void_p)),
                               ctypes.cast(LD, ctypes.POINTER(ctypes.c_int64)),
                               ctypes.cast(RW, ctypes.POINTER(ctypes.c_int32)) if RW else None,
                               l_rows, d["ws"], d["ws_bytes"], None)
    return rc, lra.lra_last_error()


@pytest.mark.parametrize("kw,code,frag", [
    (dict(rows=(5, 5, 1)), lra.LRA_ERR_INVALID, "twice"),
    (dict(rows=(5, 10)), lra.LRA_ERR_INVALID, "outside"),
    (dict(rows=(-1,)), lra.LRA_ERR_INVALID, "outside"),
    (dict(rows=None, batch=2), lra.LRA_ERR_INVALID, "rows"),
    (dict(batch=-1, rows=()), lra.LRA_ERR_INVALID, "batch"),
    (dict(batch=2000, rows=()), lra.LRA_ERR_UNSUPPORTED, "LRA_MAX_BATCH"),
    (dict(dm=72, ldx=72), lra.LRA_ERR_UNSUPPORTED, "% 64"),
    (dict(ranks=(8, 20)), lra.LRA_ERR_UNSUPPORTED, "multiples of 8"),
    (dict(L=(FAKE, None)), lra.LRA_ERR_INVALID, "null"),
    (dict(X=None), lra.LRA_ERR_INVALID, "non-null"),
    (dict(ws=None, ws_bytes=0), lra.LRA_ERR_WORKSPACE, "workspace is null"),
    (dict(ws_bytes=16), lra.LRA_ERR_WORKSPACE, "workspace of 16 bytes"),
    (dict(ws=FAKE + 4), lra.LRA_ERR_INVALID, "16-byte aligned"),
])
def test_append_rejections(kw, code, frag):
    rc, msg = _append(**kw)
    assert rc == code, (rc, msg)
    assert frag in msg, msg


def test_append_empty_is_noop():
    assert _append(rows=(), X=None, A=None, ws=None, ws_bytes=0)[0] == lra.LRA_OK


def test_append_workspace_bytes():
    ws = lra.lra_append_workspace_bytes
    assert ws(lra.LRA_DTYPE_BF16, 64, 4096, (16, 16, 16, 16)) == 16 * 64 * 64 * 4
    assert ws(lra.LRA_DTYPE_F32, 64, 4096, (16, 16, 16, 16)) == 0
    assert ws(lra.LRA_DTYPE_BF16, 0, 4096, (16,)) == 0
    assert ws(lra.LRA_DTYPE_BF16, 64, 4096, (0, 0)) == 0
    assert ws(lra.LRA_DTYPE_BF16, 300, 256, (0, 40, 24, 64, 64, 64)) >= 256 * 256 * 4
    with pytest.raises(lra.LraError):
        ws(lra.LRA_DTYPE_BF16, -1, 4096, (16,))
    # arguments lra_append_lr refuses get no size either
    for batch, dm, ranks in [(8, 4096, (12,)), (8, 4096, (72,)), (8, 4096, (-8,)),
                             (8, 4096, (64, 64, 64, 64, 8)), (8, 4000, (16,)), (8, 4100, (16,))]:
        with pytest.raises(lra.LraError):
            ws(lra.LRA_DTYPE_BF16, batch, dm, ranks)
    assert ws(lra.LRA_DTYPE_F32, 8, 4000, (16,)) == 0       # fp32 only needs d_model % 8
    # one byte short of that size is refused before anything is queued
    n = ws(lra.LRA_DTYPE_BF16, 3, 64, (8, 16))
    assert _append(ws_bytes=n - 1)[0] == lra.LRA_ERR_WORKSPACE


def test_decode_rejections():
    I = lambda a: ctypes.cast((ctypes.c_int32 * len(a))(*a), ctypes.POINTER(ctypes.c_int32))  # noqa
    P = lambda a: ctypes.cast((ctypes.c_void_p * len(a))(*a), ctypes.POINTER(ctypes.c_void_p))  # noqa
    L64 = lambda a: ctypes.cast((ctypes.c_int64 * len(a))(*a), ctypes.POINTER(ctypes.c_int64))  # noqa

    def call(k_len, agent=(0, 0)):
        return lra.lib.lra_attn_decode(lra.LRA_DTYPE_BF16, 2, 8, 2, 128, I([0, 100]), I(k_len),
                                       I(agent), FAKE, FAKE, FAKE, 200, 1, I([16]), P([FAKE]),
                                       L64([16]), P([FAKE]), FAKE, FAKE, 1 << 30, None)
    assert call([100, 0]) == lra.LRA_ERR_INVALID          # a decode query needs >= 1 key
    assert "q_len" in lra.lra_last_error()
    assert call([100, 101]) == lra.LRA_ERR_INVALID        # past kv_rows
    assert call([100, 100], agent=(0, 1)) == lra.LRA_ERR_INVALID


# ---------------------------------------------------------------------------------------
# Checks the Python binding makes before it marshals a call: the C ABI receives raw
# pointers and strides, so a wrong dtype, device or a transposed view of an LR cache or
# an up-projection would be misread there without an error.
# ---------------------------------------------------------------------------------------

def test_binding_checks_adapter_tensors():
    import torch
    bf = torch.bfloat16
    Q = torch.zeros(4, 8, 128, dtype=bf)
    L = torch.zeros(100, 16, dtype=bf)
    B = torch.zeros(16, 2 * 128, dtype=bf)
    assert lra._adapter_ranks(Q, [L, None], [B, None], 100, 2, 128) == [16, 0]
    # a column view of a wider buffer (row stride 64) is a valid LR cache
    assert lra._adapter_ranks(Q, [torch.zeros(100, 64, dtype=bf)[:, :16]], [B], 100, 2, 128) == [16]
    bad = [
        ([L.float()], [B], "L[0] must be a torch.bfloat16"),
        ([L], [B.float()], "B[0] must be a torch.bfloat16"),
        ([torch.zeros(16, 100, dtype=bf).t()], [B], "unit column stride"),
        ([L[:50]], [B], "kv_rows >= 100"),
        ([L], [torch.zeros(256, 16, dtype=bf).t()], "contiguous [16, 256]"),
        ([L], [torch.zeros(16, 128, dtype=bf)], "contiguous [16, 256]"),
        ([L], [None], "B[0] is None"),
        ([L, L], [B], "2 LR caches but 1"),
    ]
    for Ls, Bs, frag in bad:
        with pytest.raises(ValueError) as e:
            lra._adapter_ranks(Q, Ls, Bs, 100, 2, 128)
        assert frag in str(e.value), (frag, str(e.value))


def test_binding_checks_precompute_operands():
    import torch
    bf = torch.bfloat16
    X = torch.zeros(10, 64, dtype=bf)
    A = torch.zeros(64, 24, dtype=bf)
    outs = [torch.zeros(10, 8, dtype=bf), torch.zeros(10, 16, dtype=bf)]
    bad = [
        (X, A.float(), outs, "A_cat must be a torch.bfloat16"),
        (X, A.t(), outs, "unit column stride"),
        (X, A[:32], outs, "does not match d_model"),
        (X, A[:, :16], outs, "does not match d_model"),
        (X, A, outs[:1], "1 outputs for 2 ranks"),
        (X, A, [outs[0].float(), outs[1]], "L_out[0] must be a torch.bfloat16"),
        (X, A, [outs[0], torch.zeros(16, 10, dtype=bf).t()], "L_out[1] must be [rows, 16]"),
        (X, A, outs, "X must be a GPU tensor"),     # every other check passes on the CPU
    ]
    for x, a, o, frag in bad:
        with pytest.raises(ValueError) as e:
            lra._lr_outputs(x, a, (8, 16), o)
        assert frag in str(e.value), (frag, str(e.value))


def test_binding_checks_lr_cache_rows():
    """The precompute writes X's rows to every LR cache; the append checks its rows against
    one row count, which every cache must then have (a shorter one would be written past
    its end)."""
    import torch
    bf = torch.bfloat16
    X = torch.zeros(10, 64, dtype=bf)
    A = torch.zeros(64, 24, dtype=bf)
    with pytest.raises(ValueError, match="at least X's 10 rows"):
        lra._lr_outputs(X, A, (8, 16), [torch.zeros(10, 8, dtype=bf), torch.zeros(9, 16, dtype=bf)])
    with pytest.raises(ValueError, match="share one row count"):
        lra._lr_outputs(X, A, (8, 16), [torch.zeros(40, 8, dtype=bf), torch.zeros(30, 16, dtype=bf)],
                        append=True)
    # caches longer than X are fine for the precompute, and a rank-0 agent may have none
    with pytest.raises(ValueError, match="X must be a GPU tensor"):
        lra._lr_outputs(X, A, (8, 0, 16), [torch.zeros(12, 8, dtype=bf), None,
                                           torch.zeros(10, 16, dtype=bf)])


def test_binding_checks_attention_tensors():
    import torch
    bf = torch.bfloat16
    Q = torch.zeros(4, 8, 128, dtype=bf)
    K = torch.zeros(100, 2, 128, dtype=bf)
    bad = [
        (Q[0], K, K, None, "Q must be 3-D"),
        (Q, K.float(), K, None, "K_base must be a torch.bfloat16"),
        (Q, K, K[:90], None, "must share one shape"),
        (Q, torch.zeros(100, 2, 64, dtype=bf), torch.zeros(100, 2, 64, dtype=bf), None,
         "must share one shape"),
        (Q, K, K, Q.float(), "O must be a torch.bfloat16"),
        (Q, K, K, Q[:2], "must have Q's shape"),
        (Q, K, K, Q, "Q must be a contiguous GPU tensor"),   # every other check passes
    ]
    for q, k, v, o, frag in bad:
        with pytest.raises(ValueError) as e:
            lra._attn_tensors(q, k, v, o)
        assert frag in str(e.value), (frag, str(e.value))


def test_binding_checks_caller_workspace():
    import torch
    with pytest.raises(ValueError, match="contiguous tensor on cuda:0"):
        lra._workspace(256, torch.device("cuda", 0), torch.empty(256, dtype=torch.uint8))
    with pytest.raises(ValueError, match="contiguous tensor on cpu"):
        lra._workspace(256, torch.device("cpu"), torch.empty(512, dtype=torch.uint8)[::2])
    ws = torch.empty(300, dtype=torch.uint8)
    assert lra._workspace(256, torch.device("cpu"), ws) == (ws, 300)
    assert lra._workspace(0, torch.device("cpu"), ws) == (None, 0)
