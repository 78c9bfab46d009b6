"""ctypes binding of liblra.so (C ABI in include/lra.h), with the same entry-point names.

Argument marshalling only: tensors are turned into device pointers and host metadata
arrays, the call goes to the library on the caller's current HIP stream, and a non-zero
status becomes ``LraError``.  Every computation runs in the library's kernels; there is
no fallback of any kind, and importing this module fails loudly when liblra.so is
missing (build it with ``python -m shared_rank_kv_amd.build``).
"""

from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblra.so")

LRA_OK, LRA_ERR_INVALID, LRA_ERR_UNSUPPORTED, LRA_ERR_WORKSPACE, LRA_ERR_HIP = range(5)
LRA_DTYPE_F32, LRA_DTYPE_BF16 = 0, 1
SYMBOLS = ("lra_precompute_lr", "lra_append_lr", "lra_attn_prefill", "lra_attn_decode",
           "lra_attn_workspace_bytes", "lra_last_error")

_c_i32p = ctypes.POINTER(ctypes.c_int32)
_c_i64p = ctypes.POINTER(ctypes.c_int64)
_c_vpp = ctypes.POINTER(ctypes.c_void_p)


class LraError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"liblra status {code}: {msg}")
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m shared_rank_kv_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    I, L, P, S = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    lib.lra_precompute_lr.argtypes = [ctypes.c_int, L, L, P, L, P, L, I, _c_i32p, _c_vpp, _c_i64p, P]
    lib.lra_precompute_lr.restype = ctypes.c_int
    lib.lra_append_lr.argtypes = [ctypes.c_int, I, L, P, L, P, L, I, _c_i32p, _c_vpp, _c_i64p,
                                  _c_i32p, L, P]
    lib.lra_append_lr.restype = ctypes.c_int
    lib.lra_attn_prefill.argtypes = [ctypes.c_int, I, I, I, I, _c_i32p, _c_i32p, _c_i32p, _c_i32p,
                                     _c_i32p, P, L, P, P, L, I, _c_i32p, _c_vpp, _c_i64p, _c_vpp,
                                     P, P, S, P]
    lib.lra_attn_prefill.restype = ctypes.c_int
    lib.lra_attn_decode.argtypes = [ctypes.c_int, I, I, I, I, _c_i32p, _c_i32p, _c_i32p, P, P, P, L,
                                    I, _c_i32p, _c_vpp, _c_i64p, _c_vpp, P, P, S, P]
    lib.lra_attn_decode.restype = ctypes.c_int
    lib.lra_attn_workspace_bytes.argtypes = [ctypes.c_int, ctypes.c_int, I, _c_i32p, _c_i32p, I, I,
                                             I, I]
    lib.lra_attn_workspace_bytes.restype = ctypes.c_size_t
    lib.lra_last_error.argtypes = []
    lib.lra_last_error.restype = ctypes.c_char_p
    return lib


lib = _load()


# ---------------------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------------------

def _i32(a):
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return arr, arr.ctypes.data_as(_c_i32p)


def _i64(a):
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.int64))
    return arr, arr.ctypes.data_as(_c_i64p)


def _ptrs(ts):
    arr = (ctypes.c_void_p * max(1, len(ts)))(*[(t.data_ptr() if t is not None else None) for t in ts])
    return arr, ctypes.cast(arr, _c_vpp)


def _dtype(t):
    if t.dtype == torch.bfloat16:
        return LRA_DTYPE_BF16
    if t.dtype == torch.float32:
        return LRA_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(rc):
    if rc != LRA_OK:
        raise LraError(rc, lra_last_error())


def _dev(t, name):
    if not (t.is_cuda and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous GPU tensor")
    return t


# ---------------------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------------------

def lra_last_error():
    return lib.lra_last_error().decode()


def lra_attn_workspace_bytes(dtype, is_decode, q_len, k_len, n_q_heads, n_kv_heads, head_dim,
                             max_rank):
    """Scratch bytes for a call (dtype: torch dtype or LRA_DTYPE_*)."""
    if isinstance(dtype, torch.dtype):
        dtype = LRA_DTYPE_BF16 if dtype == torch.bfloat16 else LRA_DTYPE_F32
    kl, klp = _i32(k_len)
    ql, qlp = _i32(q_len if q_len is not None else np.ones(len(kl)))
    n = lib.lra_attn_workspace_bytes(dtype, int(bool(is_decode)), len(kl), qlp, klp, n_q_heads,
                                     n_kv_heads, head_dim, max_rank)
    if n == ctypes.c_size_t(-1).value:
        raise LraError(LRA_ERR_INVALID, "invalid arguments to lra_attn_workspace_bytes")
    return int(n)


def _workspace(nbytes, device, workspace):
    if nbytes == 0:
        return None, 0
    if workspace is not None:
        return workspace, workspace.numel() * workspace.element_size()
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


class Prepared:
    """A marshalled call: the ctypes arguments (and the host arrays and tensors they point
    to) are built once; calling it only runs the C entry point on the current stream."""

    def __init__(self, cfn, args, keep, result, stream_index):
        self._cfn, self._args, self._keep, self.result = cfn, list(args), keep, result
        self._si = stream_index

    def __call__(self, stream=None):
        self._args[self._si] = _stream(stream)
        _check(self._cfn(*self._args))
        return self.result


def prepare_precompute_lr(X, A_cat, ranks, L_out):
    """Prepared lra_precompute_lr: L_out[a] <- X · A_cat[:, off_a:off_a + ranks[a]].

    X [T, d_model], A_cat [d_model, sum(ranks)] (row strides may exceed the widths),
    L_out: list of [T, r_a] GPU tensors (row stride = stride(0)).
    """
    _dtype(X)
    assert X.dim() == 2 and A_cat.dim() == 2 and X.stride(1) == 1 and A_cat.stride(1) == 1
    rk, rkp = _i32(ranks)
    pk, ptrs = _ptrs(L_out)
    ld, ldp = _i64([t.stride(0) for t in L_out])
    args = (_dtype(X), X.shape[0], X.shape[1], X.data_ptr(), X.stride(0), A_cat.data_ptr(),
            A_cat.stride(0), len(rk), rkp, ptrs, ldp, None)
    return Prepared(lib.lra_precompute_lr, args, (X, A_cat, L_out, rk, pk, ld), L_out, 11)


def lra_precompute_lr(X, A_cat, ranks, L_out, stream=None):
    """L_out[a] <- X · A_cat[:, off_a:off_a + ranks[a]] (PreLRShared precompute)."""
    return prepare_precompute_lr(X, A_cat, ranks, L_out)(stream)


def prepare_append_lr(X, A_cat, ranks, L_out, rows):
    """Prepared lra_append_lr: L_out[a][rows[b]] <- X[b] · A_cat[:, off_a:off_a + ranks[a]].

    X [batch, d_model] (the new tokens), A_cat [d_model, sum(ranks)], L_out: list of
    [l_rows, r_a] GPU tensors sharing l_rows (row stride = stride(0)), rows: batch
    distinct cache rows.
    """
    _dtype(X)
    assert X.dim() == 2 and A_cat.dim() == 2 and X.stride(1) == 1 and A_cat.stride(1) == 1
    rk, rkp = _i32(ranks)
    pk, ptrs = _ptrs(L_out)
    ld, ldp = _i64([t.stride(0) if t is not None else 0 for t in L_out])
    rw, rwp = _i32(rows)
    l_rows = max([t.shape[0] for t in L_out if t is not None] + [0])
    args = (_dtype(X), X.shape[0], X.shape[1], X.data_ptr(), X.stride(0), A_cat.data_ptr(),
            A_cat.stride(0), len(rk), rkp, ptrs, ldp, rwp, l_rows, None)
    return Prepared(lib.lra_append_lr, args, (X, A_cat, L_out, rk, pk, ld, rw), L_out, 13)


def lra_append_lr(X, A_cat, ranks, L_out, rows, stream=None):
    """L_out[a][rows[b]] <- X[b] · A_cat[:, off_a:off_a + ranks[a]] (decode-step LR append)."""
    return prepare_append_lr(X, A_cat, ranks, L_out, rows)(stream)


def prepare_attn_prefill(Q, K_base, V_base, L, B, q_start, q_len, k_start, k_len, agent_idx,
                         O=None, workspace=None):
    """Prepared lra_attn_prefill (see lra_attn_prefill)."""
    _dev(Q, "Q"), _dev(K_base, "K_base"), _dev(V_base, "V_base")
    dt = _dtype(Q)
    q_rows, Hq, D = Q.shape
    kv_rows, Hkv, _ = K_base.shape
    ranks = [0 if (l is None) else l.shape[1] for l in L]
    if O is None:
        O = torch.empty_like(Q)
    qs, qsp = _i32(q_start)
    ql, qlp = _i32(q_len)
    ks, ksp = _i32(k_start)
    kl, klp = _i32(k_len)
    ag, agp = _i32(agent_idx)
    rk, rkp = _i32(ranks)
    lk, lp = _ptrs(L)
    ld, ldp = _i64([(l.stride(0) if l is not None else 0) for l in L])
    bk, bp = _ptrs(B)
    need = lib.lra_attn_workspace_bytes(dt, 0, len(ql), qlp, klp, Hq, Hkv, D, max(ranks + [0]))
    if need == ctypes.c_size_t(-1).value:
        need = 0      # invalid arguments: the call reports why
    ws, ws_bytes = _workspace(need, Q.device, workspace)
    args = (dt, len(ql), Hq, Hkv, D, qsp, qlp, ksp, klp, agp, Q.data_ptr(), q_rows,
            K_base.data_ptr(), V_base.data_ptr(), kv_rows, len(rk), rkp, lp, ldp, bp,
            O.data_ptr(), ws.data_ptr() if ws is not None else None, ws_bytes, None)
    keep = (Q, K_base, V_base, L, B, O, ws, qs, ql, ks, kl, ag, rk, lk, ld, bk)
    return Prepared(lib.lra_attn_prefill, args, keep, O, 23)


def lra_attn_prefill(Q, K_base, V_base, L, B, q_start, q_len, k_start, k_len, agent_idx, O=None,
                     workspace=None, stream=None):
    """Flash-LoRA-Attention over a batch of requests; returns O [q_rows, Hq, D].

    Q [q_rows, Hq, D]; K_base, V_base [kv_rows, Hkv, D]; L: list of per-agent [kv_rows, r_a]
    LR caches (row stride may exceed r_a; None for rank 0); B: list of [r_a, Hkv*D].
    """
    return prepare_attn_prefill(Q, K_base, V_base, L, B, q_start, q_len, k_start, k_len,
                                agent_idx, O, workspace)(stream)


def prepare_attn_decode(Q, K_base, V_base, L, B, k_start, k_len, agent_idx, O=None,
                        workspace=None):
    """Prepared lra_attn_decode (see lra_attn_decode)."""
    _dev(Q, "Q"), _dev(K_base, "K_base"), _dev(V_base, "V_base")
    dt = _dtype(Q)
    batch, Hq, D = Q.shape
    kv_rows, Hkv, _ = K_base.shape
    ranks = [0 if (l is None) else l.shape[1] for l in L]
    if O is None:
        O = torch.empty_like(Q)
    ks, ksp = _i32(k_start)
    kl, klp = _i32(k_len)
    ag, agp = _i32(agent_idx)
    rk, rkp = _i32(ranks)
    lk, lp = _ptrs(L)
    ld, ldp = _i64([(l.stride(0) if l is not None else 0) for l in L])
    bk, bp = _ptrs(B)
    need = lib.lra_attn_workspace_bytes(dt, 1, batch, None, klp, Hq, Hkv, D, max(ranks + [0]))
    if need == ctypes.c_size_t(-1).value:
        need = 0
    ws, ws_bytes = _workspace(need, Q.device, workspace)
    args = (dt, batch, Hq, Hkv, D, ksp, klp, agp, Q.data_ptr(), K_base.data_ptr(),
            V_base.data_ptr(), kv_rows, len(rk), rkp, lp, ldp, bp, O.data_ptr(),
            ws.data_ptr() if ws is not None else None, ws_bytes, None)
    keep = (Q, K_base, V_base, L, B, O, ws, ks, kl, ag, rk, lk, ld, bk)
    return Prepared(lib.lra_attn_decode, args, keep, O, 20)


def lra_attn_decode(Q, K_base, V_base, L, B, k_start, k_len, agent_idx, O=None, workspace=None,
                    stream=None):
    """One query token per request: Q, O [batch, Hq, D]; request b attends to key rows
    [k_start[b], k_start[b] + k_len[b]) of its agent."""
    return prepare_attn_decode(Q, K_base, V_base, L, B, k_start, k_len, agent_idx, O,
                               workspace)(stream)
