"""Workload shapes of the DSA forward path.

Pure data: sizes, dtypes and value ranges of the synthetic workloads.  The
indexer shape (64 heads x 128 dims, top-2048) is the public DeepSeek-V3.2
configuration named on "DeepSeek NSA and DSA" (section 3.2); the n=16, H_I=2,
d_I=2, k=3 case is the running example of "DeepSeek Sparse Attention: Learned
Token Selection from Scratch".  MLA rows are 576 wide (512 latent + 64 rope)
with the first 512 entries as the value.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    description: str
    B: int                 # sequences
    T: int                 # query rows per sequence (T == S prefill, 1 decode)
    S: int                 # cache length per sequence
    index_n_heads: int     # H_I
    index_head_dim: int    # d_I
    index_topk: int        # k
    idx_dtype: str         # "f32" | "bf16" | "fp8"
    int_lo: int            # indexer q/k are integers in [int_lo, int_hi]
    int_hi: int
    w_den: int             # indexer head weights are j / w_den, j = 0..w_den
    form: str              # "mha" | "mla"
    num_heads: int
    d_qk: int
    d_v: int
    dtype: str             # attention input dtype "f32" | "bf16"
    out_dtype: str         # attention output dtype
    scale: float

    @property
    def decode(self) -> bool:
        return self.T == 1 and self.S > 1

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "c0": Workload(
        name="c0", description="tiny causal prefill, running example shape: n=16, H_I=2, "
        "d_I=2, k=3, MHA 8x64 fp32",
        B=1, T=16, S=16, index_n_heads=2, index_head_dim=2, index_topk=3, idx_dtype="f32",
        int_lo=-3, int_hi=3, w_den=8, form="mha", num_heads=8, d_qk=64, d_v=64,
        dtype="f32", out_dtype="f32", scale=1.0 / 8.0),
    "c1": Workload(
        name="c1", description="MHA prefill: n=4096, H_I=64, d_I=128 bf16, k=2048, "
        "16 heads x 128 bf16",
        B=1, T=4096, S=4096, index_n_heads=64, index_head_dim=128, index_topk=2048,
        idx_dtype="bf16", int_lo=-4, int_hi=4, w_den=16, form="mha", num_heads=16, d_qk=128,
        d_v=128, dtype="bf16", out_dtype="bf16", scale=1.0 / math.sqrt(128.0)),
    "c2": Workload(
        name="c2", description="MLA prefill: n=32768, indexer 64x128 bf16, k=2048, "
        "128 heads, latent 576/512 bf16",
        B=1, T=32768, S=32768, index_n_heads=64, index_head_dim=128, index_topk=2048,
        idx_dtype="bf16", int_lo=-4, int_hi=4, w_den=16, form="mla", num_heads=128, d_qk=576,
        d_v=512, dtype="bf16", out_dtype="bf16", scale=1.0 / math.sqrt(192.0)),
    # the 32K prefill with the indexer's q_I and k_I in fp8 (the pages' indexer
    # precision; exact here, the inputs are small integers)
    "c2-fp8": Workload(
        name="c2-fp8", description="MLA prefill: n=32768, indexer 64x128 fp8, k=2048, "
        "128 heads, latent 576/512 bf16",
        B=1, T=32768, S=32768, index_n_heads=64, index_head_dim=128, index_topk=2048,
        idx_dtype="fp8", int_lo=-4, int_hi=4, w_den=16, form="mla", num_heads=128, d_qk=576,
        d_v=512, dtype="bf16", out_dtype="bf16", scale=1.0 / math.sqrt(192.0)),
    # a context no longer than the budget: every causal position is selected
    # (the dense limit), so the forward pass skips the indexer and the top-k
    "short2k": Workload(
        name="short2k", description="MLA prefill at the dense limit: n=2048 = k, "
        "128 heads, latent 576/512 bf16 (indexer and top-k skipped)",
        B=1, T=2048, S=2048, index_n_heads=64, index_head_dim=128, index_topk=2048,
        idx_dtype="bf16", int_lo=-4, int_hi=4, w_den=16, form="mla", num_heads=128, d_qk=576,
        d_v=512, dtype="bf16", out_dtype="bf16", scale=1.0 / math.sqrt(192.0)),
    "c3": Workload(
        name="c3", description="MLA batched decode: 64 sequences x 32768 cached tokens, "
        "bf16 indexer keys, k=2048",
        B=64, T=1, S=32768, index_n_heads=64, index_head_dim=128, index_topk=2048,
        idx_dtype="bf16", int_lo=-4, int_hi=4, w_den=16, form="mla", num_heads=128, d_qk=576,
        d_v=512, dtype="bf16", out_dtype="bf16", scale=1.0 / math.sqrt(192.0)),
    "c4": Workload(
        name="c4", description="MLA long-context decode: 8 sequences x 131072 cached tokens, "
        "fp8 e4m3 indexer keys, k=2048",
        B=8, T=1, S=131072, index_n_heads=64, index_head_dim=128, index_topk=2048,
        idx_dtype="fp8", int_lo=-4, int_hi=4, w_den=16, form="mla", num_heads=128, d_qk=576,
        d_v=512, dtype="bf16", out_dtype="bf16", scale=1.0 / math.sqrt(192.0)),
    # 128K-context prefill: the 32K prefill shape at n = 131072 (the score
    # matrix of the whole sequence, 64 GiB, is never held at once: the forward
    # pass runs query rows in chunks)
    "p128k": Workload(
        name="p128k", description="MLA prefill at 128K context: n=131072, indexer 64x128 "
        "bf16, k=2048, 128 heads, latent 576/512 bf16",
        B=1, T=131072, S=131072, index_n_heads=64, index_head_dim=128, index_topk=2048,
        idx_dtype="bf16", int_lo=-4, int_hi=4, w_den=16, form="mla", num_heads=128, d_qk=576,
        d_v=512, dtype="bf16", out_dtype="bf16", scale=1.0 / math.sqrt(192.0)),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def selected_entries(T: int, S: int, k: int) -> int:
    """Number of (query, selected position) pairs of a causal block of T query
    rows ending at position S-1: sum over t of min(t+1, k)."""
    return sum(min(t + 1, k) for t in range(S - T, S))


def causal_pairs(T: int, S: int) -> int:
    """Number of (query, candidate) pairs s <= t of the same block."""
    return sum(t + 1 for t in range(S - T, S))
