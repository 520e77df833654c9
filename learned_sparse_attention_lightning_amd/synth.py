"""Seeded synthetic inputs for the DSA forward path.

This module draws random tensors of the workloads' shapes, dtypes and value
ranges and nothing else: it holds none of the method's arithmetic, so both the
CPU oracle and the HIP path can be fed from it.

Recipe (one stream per tensor, spawned from a ``numpy.random.SeedSequence``
of the workload seed, in the fixed order q_idx, k_idx, w, q, kv, v):
  * indexer q/k: integers uniform on [int_lo, int_hi] (numpy PCG64), stored
    in the indexer dtype, which represents them exactly (fp32, bf16, fp8 e4m3);
  * head weights w: j / w_den with j uniform on 0..w_den (fp32, exact);
  * attention q / K / V / latent: standard normal drawn in fp32 by a torch
    generator on the target device (seeded from the tensor's stream), then
    rounded to the attention dtype (round-to-nearest-even for bf16).
"""
from __future__ import annotations

import numpy as np
import torch

from .configs import Workload

TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}
STREAMS = ("q_idx", "k_idx", "w", "q", "kv", "v")


def default_seed(w: Workload) -> int:
    return 1000 + int(w.name[1:]) if w.name[:1] == "c" and w.name[1:].isdigit() else 1000


def _streams(seed: int):
    children = np.random.SeedSequence(seed).spawn(len(STREAMS))
    return dict(zip(STREAMS, children))


def _ints(ss, shape, lo, hi) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(ss))
    return rng.integers(lo, hi, size=shape, dtype=np.int8, endpoint=True)


def _to_dtype(a_int8: np.ndarray, dtype: str, device) -> torch.Tensor:
    t = torch.from_numpy(a_int8).to(device)
    return t.to(torch.float32).to(TORCH_DTYPES[dtype])


def _normal(ss, shape, dtype: str, device) -> torch.Tensor:
    seed = int(ss.generate_state(1, dtype=np.uint64)[0] & 0x7FFFFFFFFFFFFFFF)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, dtype=torch.float32, device=device)
    return x.to(TORCH_DTYPES[dtype])


def indexer_inputs(w: Workload, device="cpu", seed: int | None = None):
    """q_idx [B,T,H_I,d_I], k_idx [B,S,d_I] in the indexer dtype; w [B,T,H_I] fp32."""
    st = _streams(default_seed(w) if seed is None else seed)
    B, T, S, H, D = w.B, w.T, w.S, w.index_n_heads, w.index_head_dim
    q_idx = _to_dtype(_ints(st["q_idx"], (B, T, H, D), w.int_lo, w.int_hi), w.idx_dtype, device)
    k_idx = _to_dtype(_ints(st["k_idx"], (B, S, D), w.int_lo, w.int_hi), w.idx_dtype, device)
    rng = np.random.Generator(np.random.PCG64(st["w"]))
    num = rng.integers(0, w.w_den, size=(B, T, H), dtype=np.int32, endpoint=True)
    wt = torch.from_numpy(num.astype(np.float32) / np.float32(w.w_den)).to(device)
    return q_idx, k_idx, wt


def attention_inputs(w: Workload, device="cpu", seed: int | None = None):
    """q [B,T,H,d_qk]; MHA: K [B,S,H,d_qk], V [B,S,H,d_v]; MLA: latent
    [B,S,d_qk] and V=None."""
    st = _streams(default_seed(w) if seed is None else seed)
    B, T, S, H = w.B, w.T, w.S, w.num_heads
    q = _normal(st["q"], (B, T, H, w.d_qk), w.dtype, device)
    if w.form == "mha":
        kv = _normal(st["kv"], (B, S, H, w.d_qk), w.dtype, device)
        v = _normal(st["v"], (B, S, H, w.d_v), w.dtype, device)
    else:
        kv = _normal(st["kv"], (B, S, w.d_qk), w.dtype, device)
        v = None
    return q, kv, v


def make_inputs(w: Workload, device="cpu", seed: int | None = None) -> dict:
    q_idx, k_idx, wt = indexer_inputs(w, device, seed)
    q, kv, v = attention_inputs(w, device, seed)
    return {"q_idx": q_idx, "k_idx": k_idx, "w": wt, "q": q, "kv": kv, "v": v}


def random_scores(shape, device="cpu", seed: int = 0, levels: int | None = None) -> torch.Tensor:
    """fp32 score rows for exercising the top-k alone: standard normal, or, with
    ``levels``, integers on 0..levels-1 (many ties)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    if levels is None:
        a = rng.standard_normal(size=shape, dtype=np.float32)
    else:
        a = rng.integers(0, levels, size=shape).astype(np.float32)
    return torch.from_numpy(a).to(device)
