"""Python binding of the DSA C ABI (``include/dsa.h``).

Argument marshalling only: torch tensors are checked for device, dtype,
shape and contiguity, their data pointers and the current HIP stream are
passed to ``libdsa.so``, and a non-OK status is raised as ``DSAError``.
Every step of the computation runs in the library's HIP kernels; there is no
fallback of any kind -- a missing library raises at the first call.
"""
from __future__ import annotations

import ctypes
import os

import torch

from .configs import Workload

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsa.so")

DSA_F32, DSA_BF16, DSA_FP8_E4M3 = 0, 1, 2
DSA_MHA, DSA_MLA = 0, 1
DSA_OP_TOPK, DSA_OP_ATTENTION, DSA_OP_FORWARD, DSA_OP_KL = 0, 1, 2, 3

DTYPE_CODES = {torch.float32: DSA_F32, torch.bfloat16: DSA_BF16,
               torch.float8_e4m3fn: DSA_FP8_E4M3}
NAME_CODES = {"f32": DSA_F32, "bf16": DSA_BF16, "fp8": DSA_FP8_E4M3}
FORM_CODES = {"mha": DSA_MHA, "mla": DSA_MLA}
EXPORTED = ("dsa_abi_version", "dsa_status_string", "dsa_indexer_scores",
            "dsa_indexer_scores_ex", "dsa_topk",
            "dsa_topk_ex", "dsa_sparse_attention", "dsa_sparse_attention_ex", "dsa_forward",
            "dsa_forward_ex", "dsa_forward_ex_noalloc",
            "dsa_indexer_kl", "dsa_indexer_kl_ex", "dsa_workspace_bytes")
DSA_SEL_INCLUDE_CURRENT = 1
DSA_ATTN_CAUSAL_PREFIX = 1
DSA_IDX_CAUSAL_ONLY = 1


class DSAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"DSA status {status}: {message}")
        self.status = status


class AttnDesc(ctypes.Structure):
    _fields_ = [("form", ctypes.c_int), ("num_heads", ctypes.c_int), ("d_qk", ctypes.c_int),
                ("d_v", ctypes.c_int), ("scale", ctypes.c_float), ("dtype", ctypes.c_int),
                ("out_dtype", ctypes.c_int)]


_p = ctypes.c_void_p
_i = ctypes.c_int
_lib = None


def lib_path() -> str:
    return _LIB_PATH


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libdsa.so and declare the exported signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with __graft_entry__.build() "
                           "(python -m learned_sparse_attention_lightning_amd.build)")
    lib = ctypes.CDLL(p)
    lib.dsa_abi_version.restype = _i
    lib.dsa_abi_version.argtypes = []
    lib.dsa_status_string.restype = ctypes.c_char_p
    lib.dsa_status_string.argtypes = [_i]
    lib.dsa_indexer_scores.restype = _i
    lib.dsa_indexer_scores.argtypes = [_p, _p, _i, _p, _p, _i, _i, _i, _i, _i, _p, _p]
    lib.dsa_indexer_scores_ex.restype = _i
    lib.dsa_indexer_scores_ex.argtypes = [_p, _p, _i, _p, _p, _i, _i, _i, _i, _i, _i, _p, _p]
    lib.dsa_topk.restype = _i
    lib.dsa_topk.argtypes = [_p, _p, _i, _i, _i, _i, _p, _p, ctypes.c_size_t, _p]
    lib.dsa_topk_ex.restype = _i
    lib.dsa_topk_ex.argtypes = [_p, _p, _i, _i, _i, _i, _i, _p, _p, ctypes.c_size_t, _p]
    lib.dsa_sparse_attention.restype = _i
    lib.dsa_sparse_attention.argtypes = [ctypes.POINTER(AttnDesc), _p, _p, _p, _p, _i, _i, _i,
                                         _i, _p, _p, _p, ctypes.c_size_t, _p]
    lib.dsa_sparse_attention_ex.restype = _i
    lib.dsa_sparse_attention_ex.argtypes = [ctypes.POINTER(AttnDesc), _p, _p, _p, _p, _p, _i, _i,
                                            _i, _i, _i, _p, _p, _p, ctypes.c_size_t, _p]
    lib.dsa_forward.restype = _i
    lib.dsa_forward.argtypes = [ctypes.POINTER(AttnDesc), _p, _p, _i, _p, _p, _p, _p, _p, _i,
                                _i, _i, _i, _i, _i, _p, _p, _p, ctypes.c_size_t, _p]
    lib.dsa_forward_ex.restype = _i
    lib.dsa_forward_ex.argtypes = [ctypes.POINTER(AttnDesc), _p, _p, _i, _p, _p, _p, _p, _p,
                                   _i, _i, _i, _i, _i, _i, _i, _p, _p, _p, ctypes.c_size_t, _p]
    lib.dsa_forward_ex_noalloc.restype = _i
    lib.dsa_forward_ex_noalloc.argtypes = [ctypes.POINTER(AttnDesc), _p, _p, _i, _p, _p, _p, _p,
                                           _p, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p]
    lib.dsa_indexer_kl.restype = _i
    lib.dsa_indexer_kl.argtypes = [ctypes.POINTER(AttnDesc), _p, _p, _p, _p, _p, _i, _i, _i, _i,
                                   _p, _p]
    lib.dsa_indexer_kl_ex.restype = _i
    lib.dsa_indexer_kl_ex.argtypes = [ctypes.POINTER(AttnDesc), _p, _p, _p, _p, _p, _i, _i, _i,
                                      _i, _p, _p, ctypes.c_size_t, _p]
    lib.dsa_workspace_bytes.restype = ctypes.c_size_t
    lib.dsa_workspace_bytes.argtypes = [_i, ctypes.POINTER(AttnDesc), _i, _i, _i, _i, _i, _i]
    if path is None:
        _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise DSAError(status, load().dsa_status_string(status).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _need(t, name, dtype=None, ndim=None, device=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")
    return t


def make_desc(form: str, num_heads: int, d_qk: int, d_v: int, scale: float, dtype,
              out_dtype) -> AttnDesc:
    code = lambda d: NAME_CODES[d] if isinstance(d, str) else DTYPE_CODES[d]  # noqa: E731
    return AttnDesc(FORM_CODES[form], num_heads, d_qk, d_v, float(scale), code(dtype),
                    code(out_dtype))


def desc_for(w: Workload) -> AttnDesc:
    return make_desc(w.form, w.num_heads, w.d_qk, w.d_v, w.scale, w.dtype, w.out_dtype)


def workspace_bytes(op: int, desc: AttnDesc | None, B: int, T: int, S: int, H_I: int, d_I: int,
                    k: int) -> int:
    n = load().dsa_workspace_bytes(op, ctypes.byref(desc) if desc is not None else None, B, T,
                                   S, H_I, d_I, k)
    if n == ctypes.c_size_t(-1).value:
        raise DSAError(2, "invalid sizes for workspace query")
    return n


def dsa_indexer_scores(q_idx, k_idx, w, q_pos=None, scores=None, stream=None,
                       causal_only=False):
    """scores [B,T,S] fp32 = sum_j w ReLU(q_idx . k_idx) for s <= t, -inf after.
    causal_only: entries s > t are left unwritten (dsa_indexer_scores_ex)."""
    _need(q_idx, "q_idx", ndim=4)
    _need(k_idx, "k_idx", dtype=q_idx.dtype, ndim=3)
    _need(w, "w", dtype=torch.float32, ndim=3)
    B, T, H, D = q_idx.shape
    S = k_idx.shape[1]
    if scores is None:
        scores = torch.empty((B, T, S), dtype=torch.float32, device=q_idx.device)
    _need(scores, "scores", dtype=torch.float32, ndim=3)
    if q_pos is not None:
        _need(q_pos, "q_pos", dtype=torch.int32, ndim=2)
    if causal_only:
        _check(load().dsa_indexer_scores_ex(_ptr(q_idx), _ptr(k_idx), DTYPE_CODES[q_idx.dtype],
                                            _ptr(w), _ptr(q_pos), B, T, S, H, D,
                                            DSA_IDX_CAUSAL_ONLY, _ptr(scores), _stream(stream)))
    else:
        _check(load().dsa_indexer_scores(_ptr(q_idx), _ptr(k_idx), DTYPE_CODES[q_idx.dtype],
                                         _ptr(w), _ptr(q_pos), B, T, S, H, D, _ptr(scores),
                                         _stream(stream)))
    return scores


def dsa_topk(scores, k: int, q_pos=None, idx=None, stream=None, include_current=False):
    """idx [B,T,k] int32: selected positions ascending, -1 padded.
    include_current: the query's own position is always kept (dsa_topk_ex)."""
    _need(scores, "scores", dtype=torch.float32, ndim=3)
    B, T, S = scores.shape
    if idx is None:
        idx = torch.empty((B, T, k), dtype=torch.int32, device=scores.device)
    _need(idx, "idx", dtype=torch.int32, ndim=3)
    if q_pos is not None:
        _need(q_pos, "q_pos", dtype=torch.int32, ndim=2)
    nws = workspace_bytes(DSA_OP_TOPK, None, B, T, S, 1, 1, k)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=scores.device)
    if include_current:
        _check(load().dsa_topk_ex(_ptr(scores), _ptr(q_pos), B, T, S, k,
                                  DSA_SEL_INCLUDE_CURRENT, _ptr(idx), _ptr(ws), nws,
                                  _stream(stream)))
    else:
        _check(load().dsa_topk(_ptr(scores), _ptr(q_pos), B, T, S, k, _ptr(idx), _ptr(ws), nws,
                               _stream(stream)))
    return idx


def dsa_sparse_attention(desc: AttnDesc, q, kv, v, idx, out=None, lse=None, stream=None,
                         causal_prefix=False, q_pos=None):
    """out [B,T,H,d_v] over the selected rows idx [B,T,k].  causal_prefix:
    idx rows are min(k, t+1) positions then -1, as dsa_topk writes them
    (dsa_sparse_attention_ex; q_pos gives t, else the default positions)."""
    _need(q, "q", ndim=4)
    _need(kv, "kv", dtype=q.dtype)
    if v is not None:
        _need(v, "v", dtype=q.dtype)
    _need(idx, "idx", dtype=torch.int32, ndim=3)
    B, T, H, _ = q.shape
    S = kv.shape[1]
    k = idx.shape[-1]
    odt = {DSA_F32: torch.float32, DSA_BF16: torch.bfloat16}[desc.out_dtype]
    if out is None:
        out = torch.empty((B, T, H, desc.d_v), dtype=odt, device=q.device)
    _need(out, "out", dtype=odt, ndim=4)
    if lse is not None:
        _need(lse, "lse", dtype=torch.float32, ndim=3)
    nws = workspace_bytes(DSA_OP_ATTENTION, desc, B, T, S, 1, 1, k)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=q.device)
    if causal_prefix:
        if q_pos is not None:
            _need(q_pos, "q_pos", dtype=torch.int32, ndim=2)
        _check(load().dsa_sparse_attention_ex(ctypes.byref(desc), _ptr(q), _ptr(kv), _ptr(v),
                                              _ptr(idx), _ptr(q_pos), DSA_ATTN_CAUSAL_PREFIX, B,
                                              T, S, k, _ptr(out), _ptr(lse), _ptr(ws), nws,
                                              _stream(stream)))
    else:
        _check(load().dsa_sparse_attention(ctypes.byref(desc), _ptr(q), _ptr(kv), _ptr(v),
                                           _ptr(idx), B, T, S, k, _ptr(out), _ptr(lse),
                                           _ptr(ws), nws, _stream(stream)))
    return out


def dsa_forward(desc: AttnDesc, q_idx, k_idx, w, q, kv, v, k: int, q_pos=None, out=None,
                idx_out=None, workspace=None, stream=None, include_current=False):
    """Indexer -> top-k -> sparse attention; returns out (and fills idx_out).
    include_current: the query's own position is always kept (dsa_forward_ex)."""
    _need(q_idx, "q_idx", ndim=4)
    _need(k_idx, "k_idx", dtype=q_idx.dtype, ndim=3)
    _need(w, "w", dtype=torch.float32, ndim=3)
    _need(q, "q", ndim=4)
    _need(kv, "kv", dtype=q.dtype)
    B, T, H_I, D_I = q_idx.shape
    S = k_idx.shape[1]
    odt = {DSA_F32: torch.float32, DSA_BF16: torch.bfloat16}[desc.out_dtype]
    if out is None:
        out = torch.empty((B, T, desc.num_heads, desc.d_v), dtype=odt, device=q.device)
    if idx_out is not None:
        _need(idx_out, "idx_out", dtype=torch.int32, ndim=3)
    if q_pos is not None:
        _need(q_pos, "q_pos", dtype=torch.int32, ndim=2)
    nws = workspace_bytes(DSA_OP_FORWARD, desc, B, T, S, H_I, D_I, k)
    if workspace is None or workspace.numel() < nws:
        workspace = torch.empty(nws, dtype=torch.uint8, device=q.device)
    if include_current:
        _check(load().dsa_forward_ex(ctypes.byref(desc), _ptr(q_idx), _ptr(k_idx),
                                     DTYPE_CODES[q_idx.dtype], _ptr(w), _ptr(q), _ptr(kv),
                                     _ptr(v), _ptr(q_pos), B, T, S, H_I, D_I, k,
                                     DSA_SEL_INCLUDE_CURRENT, _ptr(out), _ptr(idx_out),
                                     _ptr(workspace), workspace.numel(), _stream(stream)))
    else:
        _check(load().dsa_forward(ctypes.byref(desc), _ptr(q_idx), _ptr(k_idx),
                                  DTYPE_CODES[q_idx.dtype], _ptr(w), _ptr(q), _ptr(kv), _ptr(v),
                                  _ptr(q_pos), B, T, S, H_I, D_I, k, _ptr(out), _ptr(idx_out),
                                  _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def dsa_forward_noalloc(desc: AttnDesc, q_idx, k_idx, w, q, kv, v, k: int, q_pos=None,
                        out=None, idx_out=None, stream=None, include_current=False):
    """dsa_forward through dsa_forward_ex_noalloc: no workspace, the library's
    per-device scratch array instead (sizes up to its 128 MiB)."""
    _need(q_idx, "q_idx", ndim=4)
    _need(k_idx, "k_idx", dtype=q_idx.dtype, ndim=3)
    _need(w, "w", dtype=torch.float32, ndim=3)
    _need(q, "q", ndim=4)
    _need(kv, "kv", dtype=q.dtype)
    B, T, H_I, D_I = q_idx.shape
    S = k_idx.shape[1]
    odt = {DSA_F32: torch.float32, DSA_BF16: torch.bfloat16}[desc.out_dtype]
    if out is None:
        out = torch.empty((B, T, desc.num_heads, desc.d_v), dtype=odt, device=q.device)
    if idx_out is not None:
        _need(idx_out, "idx_out", dtype=torch.int32, ndim=3)
    if q_pos is not None:
        _need(q_pos, "q_pos", dtype=torch.int32, ndim=2)
    _check(load().dsa_forward_ex_noalloc(ctypes.byref(desc), _ptr(q_idx), _ptr(k_idx),
                                         DTYPE_CODES[q_idx.dtype], _ptr(w), _ptr(q), _ptr(kv),
                                         _ptr(v), _ptr(q_pos), B, T, S, H_I, D_I, k,
                                         DSA_SEL_INCLUDE_CURRENT if include_current else 0,
                                         _ptr(out), _ptr(idx_out), _stream(stream)))
    return out


def dsa_indexer_kl(desc: AttnDesc, q, kv, idx, lse, scores, loss=None, stream=None,
                   workspace=None):
    """Per-row KL(head-mean attention weights || softmax of the indexer
    scores) over each row's selected set -> loss [B,T] fp32 (MLA or MHA).
    Through dsa_indexer_kl_ex with the workspace it asks for (allocated here
    when not given), so the MHA masked-dense form runs where it applies."""
    mha = desc.form == DSA_MHA
    _need(q, "q", ndim=4)
    _need(kv, "kv", dtype=q.dtype, ndim=4 if mha else 3)
    _need(idx, "idx", dtype=torch.int32, ndim=3)
    _need(lse, "lse", dtype=torch.float32, ndim=3)
    _need(scores, "scores", dtype=torch.float32, ndim=3)
    B, T, H, D = q.shape
    S = kv.shape[1]
    k = idx.shape[-1]
    want_kv = (B, S, H, D) if mha else (B, S, D)
    if H != desc.num_heads or D != desc.d_qk or tuple(kv.shape) != want_kv:
        raise ValueError("q [B,T,H,d_qk] and kv (MLA [B,S,d_qk], MHA [B,S,H,d_qk]) must "
                         "match desc")
    if tuple(idx.shape[:2]) != (B, T) or tuple(lse.shape) != (B, T, H) or \
            tuple(scores.shape) != (B, T, S):
        raise ValueError("idx [B,T,k], lse [B,T,H] and scores [B,T,S] must match q and kv")
    if loss is None:
        loss = torch.empty((B, T), dtype=torch.float32, device=q.device)
    _need(loss, "loss", dtype=torch.float32, ndim=2)
    if tuple(loss.shape) != (B, T):
        raise ValueError("loss must be [B,T]")
    nws = workspace_bytes(DSA_OP_KL, desc, B, T, S, 1, 1, k)
    if nws and (workspace is None or workspace.numel() < nws):
        workspace = torch.empty(nws, dtype=torch.uint8, device=q.device)
    _check(load().dsa_indexer_kl_ex(ctypes.byref(desc), _ptr(q), _ptr(kv), _ptr(idx), _ptr(lse),
                                    _ptr(scores), B, T, S, k, _ptr(loss),
                                    _ptr(workspace) if nws else None, nws, _stream(stream)))
    return loss
