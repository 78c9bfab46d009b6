"""ctypes binding of liblra.so (C ABI in include/lra.h), with the same entry-point names.

Argument marshalling only: tensors are turned into device pointers and host metadata
arrays, the call goes to the library on the caller's current HIP stream, and a non-zero
status becomes ``LraError``.  Every computation runs in the library's kernels; there is
no fallback of any kind, and importing this module fails loudly when liblra.so is
missing (build it with ``python -m shared_rank_kv_amd.build``).
"""

from __future__ import annotations

import contextlib
import ctypes
import os

import numpy as np
import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblra.so")

LRA_OK, LRA_ERR_INVALID, LRA_ERR_UNSUPPORTED, LRA_ERR_WORKSPACE, LRA_ERR_HIP = range(5)
LRA_DTYPE_F32, LRA_DTYPE_BF16 = 0, 1
NOALLOC_SCRATCH_BYTES = 32 << 20      # LRA_NOALLOC_SCRATCH_BYTES of include/lra.h
SYMBOLS = ("lra_precompute_lr", "lra_append_lr", "lra_attn_prefill", "lra_attn_decode",
           "lra_expand_values", "lra_attn_prefill_expand", "lra_attn_decode_expand",
           "lra_attn_decode_noalloc", "lra_attn_workspace_bytes", "lra_append_workspace_bytes",
           "lra_last_error")

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
                                  _c_i32p, L, P, S, P]
    lib.lra_append_lr.restype = ctypes.c_int
    lib.lra_attn_prefill.argtypes = [ctypes.c_int, I, I, I, I, _c_i32p, _c_i32p, _c_i32p, _c_i32p,
                                     _c_i32p, P, L, P, P, L, I, _c_i32p, _c_vpp, _c_i64p, _c_vpp,
                                     P, P, S, P]
    lib.lra_attn_prefill.restype = ctypes.c_int
    lib.lra_attn_decode.argtypes = [ctypes.c_int, I, I, I, I, _c_i32p, _c_i32p, _c_i32p, P, P, P, L,
                                    I, _c_i32p, _c_vpp, _c_i64p, _c_vpp, P, P, S, P]
    lib.lra_attn_decode.restype = ctypes.c_int
    lib.lra_attn_prefill_expand.argtypes = lib.lra_attn_prefill.argtypes
    lib.lra_attn_prefill_expand.restype = ctypes.c_int
    lib.lra_attn_decode_expand.argtypes = lib.lra_attn_decode.argtypes
    lib.lra_attn_decode_expand.restype = ctypes.c_int
    lib.lra_expand_values.argtypes = [ctypes.c_int, I, _c_i32p, _c_i32p, _c_i32p, P, L, I, I, I,
                                      _c_i32p, _c_vpp, _c_i64p, _c_vpp, P, P]
    lib.lra_expand_values.restype = ctypes.c_int
    lib.lra_attn_decode_noalloc.argtypes = [ctypes.c_int, I, I, I, I, _c_i32p, _c_i32p, _c_i32p,
                                            P, P, P, L, I, _c_i32p, _c_vpp, _c_i64p, _c_vpp, P,
                                            P]
    lib.lra_attn_decode_noalloc.restype = ctypes.c_int
    lib.lra_attn_workspace_bytes.argtypes = [ctypes.c_int, ctypes.c_int, I, _c_i32p, _c_i32p, I, I,
                                             I, I]
    lib.lra_attn_workspace_bytes.restype = ctypes.c_size_t
    lib.lra_append_workspace_bytes.argtypes = [ctypes.c_int, I, L, I, _c_i32p]
    lib.lra_append_workspace_bytes.restype = ctypes.c_size_t
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


def _nullctx():
    return contextlib.nullcontext()


def _check(rc):
    if rc != LRA_OK:
        raise LraError(rc, lra_last_error())


def _dev(t, name):
    if not (t.is_cuda and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous GPU tensor")
    return t


def _like(t, ref, name):
    if t.dtype != ref.dtype or t.device != ref.device:
        raise ValueError(f"{name} must be a {ref.dtype} tensor on {ref.device} "
                         f"(got {t.dtype} on {t.device})")


def _attn_tensors(Q, K_base, V_base, O=None):
    """Checks of the attention operands the C ABI cannot see: shapes, dtypes and devices of
    Q [rows, Hq, D], K_base and V_base [kv_rows, Hkv, D] and a caller's O (Q's shape); the
    GPU check comes last."""
    for t, name in ((Q, "Q"), (K_base, "K_base"), (V_base, "V_base")):
        if t.dim() != 3:
            raise ValueError(f"{name} must be 3-D [rows, heads, head_dim] (got {tuple(t.shape)})")
    _like(K_base, Q, "K_base"), _like(V_base, Q, "V_base")
    if V_base.shape != K_base.shape or K_base.shape[2] != Q.shape[2]:
        raise ValueError(f"K_base {tuple(K_base.shape)} and V_base {tuple(V_base.shape)} must "
                         f"share one shape with Q's head_dim {Q.shape[2]}")
    if O is not None:
        _like(O, Q, "O")
        if O.shape != Q.shape:
            raise ValueError(f"O {tuple(O.shape)} must have Q's shape {tuple(Q.shape)}")
    _dev(Q, "Q"), _dev(K_base, "K_base"), _dev(V_base, "V_base")
    if O is not None:
        _dev(O, "O")


def _adapter_ranks(Q, L, B, kv_rows, Hkv, D):
    """Checks every agent's LR cache and up-projection against the call (the C ABI cannot
    see dtypes, devices or a transposed view) and returns the ranks.  L[a] is None (rank 0)
    or a [kv_rows, r_a] tensor with unit column stride (its row stride may exceed r_a);
    B[a] is a contiguous [r_a, Hkv*D] tensor."""
    if len(L) != len(B):
        raise ValueError(f"{len(L)} LR caches but {len(B)} up-projections")
    ranks = []
    for a, (l, b) in enumerate(zip(L, B)):
        if l is None or l.shape[-1] == 0:
            ranks.append(0)
            continue
        _like(l, Q, f"L[{a}]")
        if l.dim() != 2 or l.stride(1) != 1 or l.shape[0] < kv_rows:
            raise ValueError(f"L[{a}] must be [kv_rows >= {kv_rows}, r] with unit column "
                             f"stride (got shape {tuple(l.shape)}, strides {l.stride()})")
        r = int(l.shape[1])
        if b is None:
            raise ValueError(f"B[{a}] is None for an agent of rank {r}")
        _like(b, Q, f"B[{a}]")
        if tuple(b.shape) != (r, Hkv * D) or not b.is_contiguous():
            raise ValueError(f"B[{a}] must be a contiguous [{r}, {Hkv * D}] tensor "
                             f"(got shape {tuple(b.shape)}, strides {b.stride()})")
        ranks.append(r)
    return ranks


def _lr_outputs(X, A_cat, ranks, L_out, append=False):
    """Checks of the precompute / append operands the C ABI cannot see; returns the LR
    caches' row count.  The precompute writes X's rows to every cache, so each needs at
    least that many; the append writes the listed rows, checked against one row count
    that every cache must share."""
    if X.dim() != 2 or A_cat.dim() != 2 or X.stride(1) != 1 or A_cat.stride(1) != 1:
        raise ValueError("X and A_cat must be 2-D with unit column stride")
    _like(A_cat, X, "A_cat")
    if A_cat.shape[0] != X.shape[1] or A_cat.shape[1] < sum(int(r) for r in ranks):
        raise ValueError(f"A_cat {tuple(A_cat.shape)} does not match d_model {X.shape[1]} "
                         f"and ranks {tuple(ranks)}")
    if len(L_out) != len(ranks):
        raise ValueError(f"{len(L_out)} outputs for {len(ranks)} ranks")
    for a, (t, r) in enumerate(zip(L_out, ranks)):
        if int(r) == 0 and t is None:
            continue
        _like(t, X, f"L_out[{a}]")
        if t.dim() != 2 or t.stride(1) != 1 or t.shape[1] != int(r):
            raise ValueError(f"L_out[{a}] must be [rows, {r}] with unit column stride "
                             f"(got shape {tuple(t.shape)}, strides {t.stride()})")
    counts = sorted({int(t.shape[0]) for t in L_out if t is not None})
    if append and len(counts) > 1:
        raise ValueError(f"L_out tensors must share one row count (got {counts})")
    if not append and counts and counts[0] < X.shape[0]:
        raise ValueError(f"L_out tensors need at least X's {X.shape[0]} rows (got {counts[0]})")
    if not X.is_cuda:
        raise ValueError("X must be a GPU tensor")
    return counts[0] if counts else 0


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
        if workspace.device != device or not workspace.is_contiguous():
            raise ValueError(f"workspace must be a contiguous tensor on {device}")
        return workspace, workspace.numel() * workspace.element_size()
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


class Prepared:
    """A marshalled call: the ctypes arguments (and the host arrays and tensors they point
    to) are built once; calling it only runs the C entry point on the given stream (default:
    the current one).

    Tensors the binding allocated itself (`owned`: a workspace, an output) are recorded on
    the stream each call runs on, so torch's caching allocator does not hand their memory
    to another stream's allocation while that call's kernels may still use it, even once
    this object is gone."""

    def __init__(self, cfn, args, keep, result, stream_index, owned=()):
        self._cfn, self._args, self._keep, self.result = cfn, list(args), keep, result
        self._si = stream_index
        self._owned = tuple(t for t in owned if t is not None)

    def __call__(self, stream=None):
        s = torch.cuda.current_stream() if stream is None else stream
        self._args[self._si] = ctypes.c_void_p(s.cuda_stream)
        _check(self._cfn(*self._args))
        for t in self._owned:
            t.record_stream(s)
        return self.result


def prepare_precompute_lr(X, A_cat, ranks, L_out):
    """Prepared lra_precompute_lr: L_out[a] <- X · A_cat[:, off_a:off_a + ranks[a]].

    X [T, d_model], A_cat [d_model, sum(ranks)] (row strides may exceed the widths),
    L_out: list of [T, r_a] GPU tensors (row stride = stride(0)).
    """
    _dtype(X)
    _lr_outputs(X, A_cat, ranks, L_out)
    rk, rkp = _i32(ranks)
    pk, ptrs = _ptrs(L_out)
    ld, ldp = _i64([t.stride(0) if t is not None else 0 for t in L_out])
    args = (_dtype(X), X.shape[0], X.shape[1], X.data_ptr(), X.stride(0), A_cat.data_ptr(),
            A_cat.stride(0), len(rk), rkp, ptrs, ldp, None)
    return Prepared(lib.lra_precompute_lr, args, (X, A_cat, L_out, rk, pk, ld), L_out, 11)


def lra_precompute_lr(X, A_cat, ranks, L_out, stream=None):
    """L_out[a] <- X · A_cat[:, off_a:off_a + ranks[a]] (PreLRShared precompute)."""
    return prepare_precompute_lr(X, A_cat, ranks, L_out)(stream)


def lra_append_workspace_bytes(dtype, batch, d_model, ranks):
    """Scratch bytes of an lra_append_lr call (dtype: torch dtype or LRA_DTYPE_*)."""
    if isinstance(dtype, torch.dtype):
        dtype = LRA_DTYPE_BF16 if dtype == torch.bfloat16 else LRA_DTYPE_F32
    rk, rkp = _i32(ranks)
    n = lib.lra_append_workspace_bytes(dtype, int(batch), int(d_model), len(rk), rkp)
    if n == ctypes.c_size_t(-1).value:
        raise LraError(LRA_ERR_INVALID, "invalid arguments to lra_append_workspace_bytes")
    return int(n)


def prepare_append_lr(X, A_cat, ranks, L_out, rows, workspace=None):
    """Prepared lra_append_lr: L_out[a][rows[b]] <- X[b] · A_cat[:, off_a:off_a + ranks[a]].

    X [batch, d_model] (the new tokens), A_cat [d_model, sum(ranks)], L_out: list of
    [l_rows, r_a] GPU tensors sharing l_rows (row stride = stride(0)), rows: batch
    distinct cache rows.  workspace: optional GPU tensor of at least
    lra_append_workspace_bytes bytes (allocated here when None).
    """
    _dtype(X)
    l_rows = _lr_outputs(X, A_cat, ranks, L_out, append=True)
    rk, rkp = _i32(ranks)
    pk, ptrs = _ptrs(L_out)
    ld, ldp = _i64([t.stride(0) if t is not None else 0 for t in L_out])
    rw, rwp = _i32(rows)
    need = lib.lra_append_workspace_bytes(_dtype(X), X.shape[0], X.shape[1], len(rk), rkp)
    if need == ctypes.c_size_t(-1).value:
        need = 0      # invalid arguments: the call reports why
    ws, ws_bytes = _workspace(need, X.device, workspace)
    args = (_dtype(X), X.shape[0], X.shape[1], X.data_ptr(), X.stride(0), A_cat.data_ptr(),
            A_cat.stride(0), len(rk), rkp, ptrs, ldp, rwp, l_rows,
            ws.data_ptr() if ws is not None else None, ws_bytes, None)
    return Prepared(lib.lra_append_lr, args, (X, A_cat, L_out, rk, pk, ld, rw, ws), L_out, 15,
                    owned=(ws if workspace is None else None,))


def lra_append_lr(X, A_cat, ranks, L_out, rows, workspace=None, stream=None):
    """L_out[a][rows[b]] <- X[b] · A_cat[:, off_a:off_a + ranks[a]] (decode-step LR append)."""
    with torch.cuda.stream(stream) if stream is not None else _nullctx():
        return prepare_append_lr(X, A_cat, ranks, L_out, rows, workspace)(stream)


def prepare_attn_prefill(Q, K_base, V_base, L, B, q_start, q_len, k_start, k_len, agent_idx,
                         O=None, workspace=None, expand=False):
    """Prepared lra_attn_prefill (see lra_attn_prefill); expand=True prepares the in-tile
    expansion comparator lra_attn_prefill_expand instead."""
    _attn_tensors(Q, K_base, V_base, O)
    dt = _dtype(Q)
    q_rows, Hq, D = Q.shape
    kv_rows, Hkv, _ = K_base.shape
    ranks = _adapter_ranks(Q, L, B, kv_rows, Hkv, D)
    owned_O = O is None
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
    owned = (O if owned_O else None, ws if workspace is None else None)
    cfn = lib.lra_attn_prefill_expand if expand else lib.lra_attn_prefill
    return Prepared(cfn, args, keep, O, 23, owned)


def lra_attn_prefill(Q, K_base, V_base, L, B, q_start, q_len, k_start, k_len, agent_idx, O=None,
                     workspace=None, stream=None):
    """Flash-LoRA-Attention over a batch of requests; returns O [q_rows, Hq, D].

    Q [q_rows, Hq, D]; K_base, V_base [kv_rows, Hkv, D]; L: list of per-agent [kv_rows, r_a]
    LR caches (row stride may exceed r_a; None for rank 0); B: list of [r_a, Hkv*D].
    """
    with torch.cuda.stream(stream) if stream is not None else _nullctx():
        return prepare_attn_prefill(Q, K_base, V_base, L, B, q_start, q_len, k_start, k_len,
                                    agent_idx, O, workspace)(stream)


def prepare_attn_decode(Q, K_base, V_base, L, B, k_start, k_len, agent_idx, O=None,
                        workspace=None, expand=False):
    """Prepared lra_attn_decode (see lra_attn_decode); expand=True prepares the in-tile
    expansion comparator lra_attn_decode_expand instead."""
    _attn_tensors(Q, K_base, V_base, O)
    dt = _dtype(Q)
    batch, Hq, D = Q.shape
    kv_rows, Hkv, _ = K_base.shape
    ranks = _adapter_ranks(Q, L, B, kv_rows, Hkv, D)
    owned_O = O is None
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
    owned = (O if owned_O else None, ws if workspace is None else None)
    cfn = lib.lra_attn_decode_expand if expand else lib.lra_attn_decode
    return Prepared(cfn, args, keep, O, 20, owned)


def lra_attn_decode(Q, K_base, V_base, L, B, k_start, k_len, agent_idx, O=None, workspace=None,
                    stream=None):
    """One query token per request: Q, O [batch, Hq, D]; request b attends to key rows
    [k_start[b], k_start[b] + k_len[b]) of its agent."""
    with torch.cuda.stream(stream) if stream is not None else _nullctx():
        return prepare_attn_decode(Q, K_base, V_base, L, B, k_start, k_len, agent_idx, O,
                                   workspace)(stream)


def prepare_attn_decode_noalloc(Q, K_base, V_base, L, B, k_start, k_len, agent_idx, O):
    """Prepared lra_attn_decode_noalloc: the decode with the library's fixed scratch; O is
    the caller's output [batch, Hq, D] (nothing is allocated)."""
    _attn_tensors(Q, K_base, V_base, O)
    dt = _dtype(Q)
    batch, Hq, D = Q.shape
    kv_rows, Hkv, _ = K_base.shape
    ranks = _adapter_ranks(Q, L, B, kv_rows, Hkv, D)
    ks, ksp = _i32(k_start)
    kl, klp = _i32(k_len)
    ag, agp = _i32(agent_idx)
    rk, rkp = _i32(ranks)
    lk, lp = _ptrs(L)
    ld, ldp = _i64([(l.stride(0) if l is not None else 0) for l in L])
    bk, bp = _ptrs(B)
    args = (dt, batch, Hq, Hkv, D, ksp, klp, agp, Q.data_ptr(), K_base.data_ptr(),
            V_base.data_ptr(), kv_rows, len(rk), rkp, lp, ldp, bp, O.data_ptr(), None)
    keep = (Q, K_base, V_base, L, B, O, ks, kl, ag, rk, lk, ld, bk)
    return Prepared(lib.lra_attn_decode_noalloc, args, keep, O, 18)


def lib_noalloc_scratch_bytes():
    """Size of the library's fixed decode scratch (LRA_NOALLOC_SCRATCH_BYTES)."""
    return NOALLOC_SCRATCH_BYTES


def lra_attn_decode_noalloc(Q, K_base, V_base, L, B, k_start, k_len, agent_idx, O, stream=None):
    """lra_attn_decode without a workspace: the split-key scratch is the library's fixed
    per-GPU array (calls that may overlap on one GPU race on it)."""
    return prepare_attn_decode_noalloc(Q, K_base, V_base, L, B, k_start, k_len, agent_idx,
                                       O)(stream)


# ---------------------------------------------------------------------------------------
# comparators of the regrouping (naive expansion, in-tile expansion)
# ---------------------------------------------------------------------------------------

def lra_attn_prefill_expand(Q, K_base, V_base, L, B, q_start, q_len, k_start, k_len,
                            agent_idx, O=None, workspace=None, stream=None):
    """The in-tile expansion route of lra_attn_prefill (same arguments and result)."""
    with torch.cuda.stream(stream) if stream is not None else _nullctx():
        return prepare_attn_prefill(Q, K_base, V_base, L, B, q_start, q_len, k_start, k_len,
                                    agent_idx, O, workspace, expand=True)(stream)


def lra_attn_decode_expand(Q, K_base, V_base, L, B, k_start, k_len, agent_idx, O=None,
                           workspace=None, stream=None):
    """The in-tile expansion route of lra_attn_decode (same arguments and result)."""
    with torch.cuda.stream(stream) if stream is not None else _nullctx():
        return prepare_attn_decode(Q, K_base, V_base, L, B, k_start, k_len, agent_idx, O,
                                   workspace, expand=True)(stream)


def prepare_expand_values(V_base, L, B, start, length, agent_idx, V_full):
    """Prepared lra_expand_values: V_full[s] <- V_base[s] + L_a[s]·B_a over the spans."""
    _dev(V_base, "V_base"), _dev(V_full, "V_full")
    _like(V_full, V_base, "V_full")
    if V_full.shape != V_base.shape:
        raise ValueError(f"V_full {tuple(V_full.shape)} must have V_base's shape "
                         f"{tuple(V_base.shape)}")
    kv_rows, Hkv, D = V_base.shape
    ranks = _adapter_ranks(V_base, L, B, kv_rows, Hkv, D)
    st, stp = _i32(start)
    ln, lnp = _i32(length)
    ag, agp = _i32(agent_idx)
    rk, rkp = _i32(ranks)
    lk, lp = _ptrs(L)
    ld, ldp = _i64([(l.stride(0) if l is not None else 0) for l in L])
    bk, bp = _ptrs(B)
    args = (_dtype(V_base), len(st), stp, lnp, agp, V_base.data_ptr(), kv_rows, Hkv, D,
            len(rk), rkp, lp, ldp, bp, V_full.data_ptr(), None)
    keep = (V_base, L, B, V_full, st, ln, ag, rk, lk, ld, bk)
    return Prepared(lib.lra_expand_values, args, keep, V_full, 15)


def lra_expand_values(V_base, L, B, start, length, agent_idx, V_full=None, stream=None):
    """The naive reconstruction: V_full[s] = V_base[s] + L_a[s]·B_a for the rows of every span
    (rows outside the spans are left as they are; a new V_full starts uninitialised)."""
    with torch.cuda.stream(stream) if stream is not None else _nullctx():
        owned = V_full is None
        if owned:
            V_full = torch.empty_like(V_base)
        p = prepare_expand_values(V_base, L, B, start, length, agent_idx, V_full)
        if owned:
            p._owned = (V_full,)
        return p(stream)
