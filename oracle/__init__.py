"""CPU oracle for the DeepSeek Sparse Attention forward path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product library
never links, loads or calls it, and it shares no code with the HIP path.

The arithmetic lives in ``dsa_oracle.c`` (plain C, IEEE double, built with
``-O2 -fopenmp`` and without fast-math).  This module only converts arrays to
float64 exactly, allocates outputs and calls the C routines through ctypes.

Page references (titles as published):
  [P1] "DeepSeek Sparse Attention: Learned Token Selection from Scratch"
  [P4] "DeepSeek NSA and DSA: From Native Sparse Attention to Fine-Grained
       Token Selection"
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dsa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def build(force: bool = False, src: str = _SRC, out: str = _LIB) -> str:
    """Compile the C oracle into a shared library (gcc, -O2, OpenMP)."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
               "-Wall", "-Wextra", "-o", out, src, "-lm"]
        subprocess.run(cmd, check=True)
    return out


def load(path: str | None = None) -> ctypes.CDLL:
    lib = ctypes.CDLL(path or build())
    lib.oracle_indexer_scores.argtypes = [_p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64, _p]
    lib.oracle_indexer_scores.restype = None
    lib.oracle_indexer_scores_exact.argtypes = [_p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64, _p]
    lib.oracle_indexer_scores_exact.restype = None
    lib.oracle_topk.argtypes = [_p, _p, _i64, _i64, _i64, _i64, _i64, _p]
    lib.oracle_topk.restype = None
    lib.oracle_sparse_attention.argtypes = [ctypes.c_int, _p, _p, _p, _p, _i64, _i64, _i64,
                                            _i64, _i64, _i64, _i64, ctypes.c_double, _p, _p]
    lib.oracle_sparse_attention.restype = None
    lib.oracle_dense_causal_attention.argtypes = [ctypes.c_int, _p, _p, _p, _p, _i64, _i64,
                                                  _i64, _i64, _i64, _i64, ctypes.c_double, _p]
    lib.oracle_dense_causal_attention.restype = None
    lib.oracle_masked_dense_attention.argtypes = [ctypes.c_int, _p, _p, _p, _p, _i64, _i64,
                                                  _i64, _i64, _i64, _i64, _i64,
                                                  ctypes.c_double, _p]
    lib.oracle_masked_dense_attention.restype = None
    lib.oracle_warmup_target.argtypes = [_p, _p, _p, _i64, _i64, _i64, _i64, _i64,
                                         ctypes.c_double, _p]
    lib.oracle_warmup_target.restype = None
    lib.oracle_sparse_target.argtypes = [ctypes.c_int, _p, _p, _p, _i64, _i64, _i64, _i64,
                                         _i64, _i64, ctypes.c_double, _p]
    lib.oracle_sparse_target.restype = None
    lib.oracle_indexer_kl.argtypes = [_p, _p, _p, _i64, _i64]
    lib.oracle_indexer_kl.restype = ctypes.c_double
    return lib


_lib = None


def _get():
    global _lib
    if _lib is None:
        # DSA_ORACLE_LIB lets the mutation test load a deliberately broken build
        _lib = load(os.environ.get("DSA_ORACLE_LIB") or None)
    return _lib


def as_f64(x) -> np.ndarray:
    """Exact conversion to a C-contiguous float64 array (bf16/fp8/fp32 embed
    exactly in double).  Accepts numpy arrays and CPU or GPU torch tensors."""
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _pos(q_pos):
    if q_pos is None:
        return None, None
    a = np.ascontiguousarray(np.asarray(
        q_pos.detach().cpu().numpy() if hasattr(q_pos, "detach") else q_pos, dtype=np.int64))
    return a, a.ctypes.data


def _ptr(a):
    return None if a is None else a.ctypes.data


def indexer_scores(q_idx, k_idx, w, q_pos=None) -> np.ndarray:
    """I[b,i,s] per [P1] section 2.1; -inf for s > t.  q_idx [B,T,H,D],
    k_idx [B,S,D], w [B,T,H] -> [B,T,S] float64."""
    q = as_f64(q_idx)
    k = as_f64(k_idx)
    wt = as_f64(w)
    B, T, H, D = q.shape
    S = k.shape[1]
    assert k.shape == (B, S, D) and wt.shape == (B, T, H)
    pos, pos_p = _pos(q_pos)
    out = np.empty((B, T, S), dtype=np.float64)
    _get().oracle_indexer_scores(q.ctypes.data, k.ctypes.data, wt.ctypes.data, pos_p,
                                 B, T, S, H, D, out.ctypes.data)
    return out


def indexer_scores_exact(q_idx, k_idx, w, den: int, q_pos=None) -> np.ndarray:
    """den * I as exact int64 for integer q/k and w*den integer; s > t holds
    INT64_MIN.  Raises if an input is not integer-valued as required."""
    q = as_f64(q_idx)
    k = as_f64(k_idx)
    wn = as_f64(w) * den
    for name, a in (("q_idx", q), ("k_idx", k), ("w*den", wn)):
        if not np.array_equal(a, np.round(a)):
            raise ValueError(f"{name} is not integer-valued")
    q, k, wn = (np.ascontiguousarray(a.astype(np.int64)) for a in (q, k, wn))
    B, T, H, D = q.shape
    S = k.shape[1]
    pos, pos_p = _pos(q_pos)
    out = np.empty((B, T, S), dtype=np.int64)
    _get().oracle_indexer_scores_exact(q.ctypes.data, k.ctypes.data, wn.ctypes.data, pos_p,
                                       B, T, S, H, D, out.ctypes.data)
    return out


def topk(scores, k: int, q_pos=None, include_current: bool = False) -> np.ndarray:
    """Selected positions per row in rank order (score desc, position asc),
    min(k, t+1) valid entries then -1.  scores [B,T,S] -> int32 [B,T,k].
    include_current: position t itself first, then the best k-1 of s < t
    ([P1] section 3.4, the current-token variant)."""
    sc = as_f64(scores)
    B, T, S = sc.shape
    pos, pos_p = _pos(q_pos)
    out = np.empty((B, T, k), dtype=np.int32)
    _get().oracle_topk(sc.ctypes.data, pos_p, B, T, S, k, 1 if include_current else 0,
                       out.ctypes.data)
    return out


def _form(form) -> int:
    return {"mha": 0, "mla": 1, 0: 0, 1: 1}[form]


def sparse_attention(form, q, kv, v, idx, scale: float, d_v: int | None = None,
                     with_lse: bool = False):
    """Softmax attention over the selected set ([P1] sections 3.3, 10.1).
    MHA: q [B,T,H,d], kv=K [B,S,H,d], v=V [B,S,H,dv].
    MLA: q [B,T,H,dqk], kv=latent [B,S,dqk], v=None, values = latent[..., :d_v]."""
    f = _form(form)
    qq = as_f64(q)
    kk = as_f64(kv)
    B, T, H, dqk = qq.shape
    S = kk.shape[1]
    if f == 0:
        vv = as_f64(v)
        dv = vv.shape[-1]
        vp = vv.ctypes.data
    else:
        vv = None
        dv = int(d_v)
        vp = None
    ix = np.ascontiguousarray(np.asarray(
        idx.detach().cpu().numpy() if hasattr(idx, "detach") else idx, dtype=np.int32))
    k = ix.shape[-1]
    out = np.empty((B, T, H, dv), dtype=np.float64)
    lse = np.empty((B, T, H), dtype=np.float64)
    _get().oracle_sparse_attention(f, qq.ctypes.data, kk.ctypes.data, vp, ix.ctypes.data,
                                   B, T, S, H, dqk, dv, k, float(scale), out.ctypes.data,
                                   lse.ctypes.data)
    return (out, lse) if with_lse else out


def dense_causal_attention(form, q, kv, v, scale: float, d_v: int | None = None,
                           q_pos=None) -> np.ndarray:
    """Textbook causal softmax attention over every s <= t."""
    f = _form(form)
    qq = as_f64(q)
    kk = as_f64(kv)
    B, T, H, dqk = qq.shape
    S = kk.shape[1]
    vv = as_f64(v) if f == 0 else None
    dv = vv.shape[-1] if f == 0 else int(d_v)
    pos, pos_p = _pos(q_pos)
    out = np.empty((B, T, H, dv), dtype=np.float64)
    _get().oracle_dense_causal_attention(f, qq.ctypes.data, kk.ctypes.data, _ptr(vv), pos_p,
                                         B, T, S, H, dqk, dv, float(scale), out.ctypes.data)
    return out


def masked_dense_attention(form, q, kv, v, idx, scale: float,
                           d_v: int | None = None) -> np.ndarray:
    """Full-row softmax with -inf outside the selected set ([P1] section 9.3)."""
    f = _form(form)
    qq = as_f64(q)
    kk = as_f64(kv)
    B, T, H, dqk = qq.shape
    S = kk.shape[1]
    vv = as_f64(v) if f == 0 else None
    dv = vv.shape[-1] if f == 0 else int(d_v)
    ix = np.ascontiguousarray(np.asarray(
        idx.detach().cpu().numpy() if hasattr(idx, "detach") else idx, dtype=np.int32))
    out = np.empty((B, T, H, dv), dtype=np.float64)
    _get().oracle_masked_dense_attention(f, qq.ctypes.data, kk.ctypes.data, _ptr(vv),
                                         ix.ctypes.data, B, T, S, H, dqk, dv, ix.shape[-1],
                                         float(scale), out.ctypes.data)
    return out


def warmup_target(q, K, scale: float, q_pos=None) -> np.ndarray:
    """Head-mean dense attention distribution p[t,s] ([P1] section 5.2)."""
    qq = as_f64(q)
    kk = as_f64(K)
    B, T, H, d = qq.shape
    S = kk.shape[1]
    pos, pos_p = _pos(q_pos)
    out = np.empty((B, T, S), dtype=np.float64)
    _get().oracle_warmup_target(qq.ctypes.data, kk.ctypes.data, pos_p, B, T, S, H, d,
                                float(scale), out.ctypes.data)
    return out


def sparse_target(form, q, kv, idx, scale: float) -> np.ndarray:
    """Head-mean of the sparse attention weights over the selected set
    ([P1] sections 5.2, 6.2-6.3).  MHA: kv = K [B,S,H,d]; MLA: kv = latent
    [B,S,d].  -> p [B,T,S], zero outside the set."""
    f = _form(form)
    qq = as_f64(q)
    kk = as_f64(kv)
    B, T, H, dqk = qq.shape
    S = kk.shape[1]
    ix = np.ascontiguousarray(np.asarray(
        idx.detach().cpu().numpy() if hasattr(idx, "detach") else idx, dtype=np.int32))
    out = np.empty((B, T, S), dtype=np.float64)
    _get().oracle_sparse_target(f, qq.ctypes.data, kk.ctypes.data, ix.ctypes.data, B, T, S, H,
                                dqk, ix.shape[-1], float(scale), out.ctypes.data)
    return out


def selection_mask(idx, S: int) -> np.ndarray:
    """[B,T,k] selection -> [B,T,S] int8 membership mask."""
    ix = np.asarray(idx.detach().cpu().numpy() if hasattr(idx, "detach") else idx)
    B, T, _ = ix.shape
    m = np.zeros((B, T, S), dtype=np.int8)
    for b in range(B):
        for i in range(T):
            v = ix[b, i][ix[b, i] >= 0]
            m[b, i, v] = 1
    return m


def indexer_kl_rows(p, scores, mask) -> np.ndarray:
    """KL(p || softmax(I)) of every row separately -> [B,T] float64."""
    pp, sc = as_f64(p), as_f64(scores)
    mk = np.asarray(mask)
    B, T, _ = pp.shape
    return np.array([[indexer_kl(pp[b, i:i + 1], sc[b, i:i + 1], mk[b, i:i + 1])
                      for i in range(T)] for b in range(B)])


def indexer_kl(p, scores, mask) -> float:
    """Sum over rows of KL(p || softmax(I)) over the masked positions
    ([P1] sections 5.4, 6.2)."""
    pp = as_f64(p)
    sc = as_f64(scores)
    S = pp.shape[-1]
    rows = pp.size // S
    mk = np.ascontiguousarray(np.asarray(mask, dtype=np.int8))
    assert mk.shape == pp.shape == sc.shape
    return float(_get().oracle_indexer_kl(pp.ctypes.data, sc.ctypes.data, mk.ctypes.data,
                                          rows, S))
