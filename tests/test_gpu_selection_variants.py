"""The selection variants of the HIP path against the CPU oracle: the
current-token flag (the query's own position always kept, the other k-1
slots ranked among earlier positions) and contexts no longer than the
budget (every causal position selected; the forward pass skips the indexer
and the top-k).  Bar as for the plain path: index sets bit-exact, attention
outputs within max-abs 2e-2 (bf16)."""
import numpy as np
import pytest
import torch

import oracle
from parity_util import TOL, assert_selection_equal, max_abs_err

from learned_sparse_attention_lightning_amd import configs, dsa, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsa.load()
    oracle.build()


def _say(msg):
    print(msg, flush=True)


def _current_kept(idx, pos):
    """Every row with a position t >= 0 holds t as its last valid entry."""
    g = idx.cpu().numpy()
    p = np.asarray(pos)
    nvalid = (g >= 0).sum(-1)
    for b, i in np.ndindex(p.shape):
        if p[b, i] >= 0:
            assert g[b, i, nvalid[b, i] - 1] == p[b, i], (b, i)


# ------------------------------------------------------------------- top-k --

@pytest.mark.parametrize("levels", [None, 3])
@pytest.mark.parametrize("k", [1, 2, 7, 64, 300, 400])
def test_topk_include_current_rows(levels, k):
    B, T, S = 2, 300, 300
    sc = synth.random_scores((B, T, S), seed=k * 3 + (levels or 0), levels=levels)
    idx = dsa.dsa_topk(sc.to(DEV), k, include_current=True)
    assert_selection_equal(idx, oracle.topk(sc, k, include_current=True),
                           f"current levels={levels} k={k}")
    _current_kept(idx, np.arange(T)[None, :].repeat(B, 0))


@pytest.mark.parametrize("S", [32768, 131072])
def test_topk_include_current_wide_rows(S):
    B, k = 4, 2048
    pos = torch.tensor([[S - 1], [S // 2], [2048], [0]], dtype=torch.int32)
    sc = synth.random_scores((B, 1, S), seed=S + 1, levels=None)
    sc[1, 0, : S // 4] = 0.5  # a block of ties
    sc[0, 0, S - 1] = -10.0   # the current token far below the threshold
    idx = dsa.dsa_topk(sc.to(DEV), k, q_pos=pos.to(DEV), include_current=True)
    assert_selection_equal(idx, oracle.topk(sc, k, q_pos=pos, include_current=True),
                           f"current wide S={S}")
    _current_kept(idx, pos.numpy())


def test_topk_include_current_many_long_rows():
    B, T, S, k = 1, 520, 40001, 2048
    pos = torch.tensor([[S - 1 - 37 * j for j in range(T)]], dtype=torch.int32)
    sc = synth.random_scores((B, T, S), seed=12, levels=None)
    idx = dsa.dsa_topk(sc.to(DEV), k, q_pos=pos.to(DEV), include_current=True)
    rows = [0, 1, 100, 519]
    ref = oracle.topk(sc[:, rows], k, q_pos=pos[:, rows], include_current=True)
    assert_selection_equal(idx[:, rows], ref, "current many long rows")
    _current_kept(idx, pos.numpy())


def test_topk_budget_above_context():
    B, T, S, k = 2, 50, 50, 80
    sc = synth.random_scores((B, T, S), seed=3, levels=4)
    idx = dsa.dsa_topk(sc.to(DEV), k)
    assert_selection_equal(idx, oracle.topk(sc, k), "k > S")


# ----------------------------------------------------------------- forward --

def _run_forward(w, seed, include_current):
    x = synth.make_inputs(w, device=DEV, seed=seed)
    idx = torch.empty((w.B, w.T, w.index_topk), dtype=torch.int32, device=DEV)
    out = dsa.dsa_forward(dsa.desc_for(w), x["q_idx"], x["k_idx"], x["w"], x["q"], x["kv"],
                          x["v"], w.index_topk, idx_out=idx, include_current=include_current)
    torch.cuda.synchronize()
    return x, idx, out


def _oracle_forward(w, x, include_current):
    sc = oracle.indexer_scores(x["q_idx"], x["k_idx"], x["w"])
    ref_idx = oracle.topk(sc, w.index_topk, include_current=include_current)
    ref = oracle.sparse_attention(w.form, x["q"], x["kv"], x["v"], ref_idx, w.scale, d_v=w.d_v)
    return ref_idx, ref


# 128 heads run the MLA matrix-core kernel; 16 heads the gather kernel
CURRENT_CASES = {
    "mla-prefill-h16": ("c2", dict(B=2, T=700, S=700, index_topk=64, num_heads=16)),
    "mla-prefill-h128": ("c2", dict(B=2, T=700, S=700, index_topk=64)),
    "mha-prefill": ("c1", dict(B=1, T=1500, S=1500, index_topk=256)),
    "mla-decode-fp8-h16": ("c4", dict(B=2, T=1, S=40000, num_heads=16)),
    "mla-decode-fp8-h128": ("c4", dict(B=2, T=1, S=40000)),
}


@pytest.mark.parametrize("case", list(CURRENT_CASES))
def test_forward_include_current(case):
    base, kw = CURRENT_CASES[case]
    w = configs.get(base).with_(name=f"current-{case}", **kw)
    x, idx, out = _run_forward(w, 17, True)
    ref_idx, ref = _oracle_forward(w, x, True)
    assert_selection_equal(idx, ref_idx, case)
    pos = np.arange(w.S - w.T, w.S)[None, :].repeat(w.B, 0)
    _current_kept(idx, pos)
    err = max_abs_err(out, ref)
    _say(f"{case} with the current token: max-abs err {err:.3e}")
    assert err <= TOL["bf16"]


DENSE_CASES = {
    "mla-n1000-k2048-h16": ("c2", dict(B=1, T=1000, S=1000, index_topk=2048, num_heads=16)),
    "mla-n1000-k2048-h128": ("c2", dict(B=1, T=1000, S=1000, index_topk=2048)),
    "mla-k-equals-n-h16": ("c2", dict(B=2, T=256, S=256, index_topk=256, num_heads=16)),
    "mla-k-equals-n-h128": ("c2", dict(B=2, T=256, S=256, index_topk=256)),
    "mha-n777-k1024": ("c1", dict(B=1, T=777, S=777, index_topk=1024)),
    "mla-decode-n1500-h16": ("c4", dict(B=3, T=1, S=1500, num_heads=16)),
    "mla-decode-n1500-h128": ("c4", dict(B=3, T=1, S=1500)),
}


@pytest.mark.parametrize("case", list(DENSE_CASES))
def test_forward_dense_when_context_within_budget(case):
    """S <= k: every causal position is selected (the dense limit); the result
    equals the oracle's top-k path, and the current-token flag changes
    nothing."""
    base, kw = DENSE_CASES[case]
    w = configs.get(base).with_(name=f"dense-{case}", **kw)
    x, idx, out = _run_forward(w, 23, False)
    ref_idx, ref = _oracle_forward(w, x, False)
    assert_selection_equal(idx, ref_idx, case)
    g = idx.cpu().numpy()
    for b in range(w.B):
        for i in range(w.T):
            t = w.S - w.T + i
            assert np.array_equal(g[b, i, : t + 1], np.arange(t + 1))
    err = max_abs_err(out, ref)
    _say(f"{case} dense: max-abs err {err:.3e}")
    assert err <= TOL["bf16"]
    idx2 = torch.empty_like(idx)
    out2 = dsa.dsa_forward(dsa.desc_for(w), x["q_idx"], x["k_idx"], x["w"], x["q"], x["kv"],
                           x["v"], w.index_topk, idx_out=idx2, include_current=True)
    torch.cuda.synchronize()
    assert torch.equal(idx2, idx) and torch.equal(out2, out)


def test_forward_dense_limit_2048_h128():
    """The dense-limit workload as benchmarked (n = k = 2048, 128 heads): the
    selection fill on every row and the matrix-core attention against the
    oracle's textbook dense causal attention on a stratified row sample."""
    w = configs.get("short2k")
    x, idx, out = _run_forward(w, 23, False)
    g = idx.cpu().numpy()
    for i in range(w.T):
        assert np.array_equal(g[0, i, : i + 1], np.arange(i + 1)) and np.all(g[0, i, i + 1:] == -1)
    rows = sorted({0, 1, 31, 32, 1000, 2046, 2047} | set(range(3, 2047, 41)))
    _say(f"dense limit 2048 x 128 heads: oracle dense attention on {len(rows)} rows")
    ref = oracle.dense_causal_attention("mla", x["q"][:, rows], x["kv"], None, w.scale,
                                        d_v=w.d_v, q_pos=np.array([rows]))
    err = max_abs_err(out[:, rows], ref)
    _say(f"dense limit 2048: max-abs err {err:.3e}")
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("case", ["prefill-h32", "decode-splits-h16", "prefill-h128",
                                  "decode-splits-h128"])
def test_attention_causal_prefix_matches_plain(case):
    """Stopping at each row's selected count (dsa_sparse_attention_ex with
    DSA_ATTN_CAUSAL_PREFIX) skips only empty tiles: outputs and lse are
    bitwise those of the plain call, and both match the oracle."""
    heads = int(case.rsplit("-h", 1)[1])
    if case.startswith("prefill"):
        w = configs.get("c2").with_(name="prefix", B=1, T=3000, S=3000, num_heads=heads)
        pos = None
    else:
        # t < k leaves whole entry splits empty (each runs one masked tile)
        w = configs.get("c4").with_(name="prefix-dec", B=4, T=1, S=3000, num_heads=heads)
        pos = torch.tensor([[2999], [100], [2047], [0]], dtype=torch.int32, device=DEV)
    x = synth.make_inputs(w, device=DEV, seed=29)
    sc = dsa.dsa_indexer_scores(x["q_idx"], x["k_idx"], x["w"], q_pos=pos)
    idx = dsa.dsa_topk(sc, w.index_topk, q_pos=pos)
    desc = dsa.desc_for(w)
    lse0 = torch.empty((w.B, w.T, w.num_heads), dtype=torch.float32, device=DEV)
    lse1 = torch.empty_like(lse0)
    out0 = dsa.dsa_sparse_attention(desc, x["q"], x["kv"], None, idx, lse=lse0)
    out1 = dsa.dsa_sparse_attention(desc, x["q"], x["kv"], None, idx, lse=lse1,
                                    causal_prefix=True, q_pos=pos)
    torch.cuda.synchronize()
    assert torch.equal(out0, out1) and torch.equal(lse0, lse1)
    rows = [0, 1, 100, 2046, 2047, 2048, w.T - 1] if w.T > 1 else [0]
    ref, ref_lse = oracle.sparse_attention("mla", x["q"][:, rows], x["kv"], None,
                                           idx[:, rows].cpu(), w.scale, d_v=w.d_v,
                                           with_lse=True)
    assert max_abs_err(out1[:, rows], ref) <= TOL["bf16"]
    assert np.abs(lse1[:, rows].cpu().numpy() - ref_lse).max() < 1e-3


def test_forward_include_current_c4_full():
    """The 128K decode workload at full size with the current token kept."""
    w = configs.get("c4")
    x, idx, out = _run_forward(w, None, True)
    sc = oracle.indexer_scores(x["q_idx"], x["k_idx"], x["w"])
    ref_idx = oracle.topk(sc, w.index_topk, include_current=True)
    assert_selection_equal(idx, ref_idx, "c4 current")
    _current_kept(idx, np.full((w.B, 1), w.S - 1))
    ref = oracle.sparse_attention("mla", x["q"], x["kv"], None, ref_idx, w.scale, d_v=w.d_v)
    err = max_abs_err(out, ref)
    _say(f"c4 with the current token: max-abs err {err:.3e}")
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("case", ["mla-decode-h128", "mla-prefill-h128", "mla-decode-h16",
                                  "mha-prefill-h16"])
def test_attention_entries_past_cache_count_as_unused(case):
    """Selection entries at or past the cache's end (s >= S) are outside the
    selection's contract; every attention kernel counts them as unused slots,
    like -1, and reads nothing past the sequence's rows: outputs equal the
    oracle's on the selection with those entries set to -1."""
    form, kind, h = case.split("-")
    heads = int(h[1:])
    if form == "mla":
        base = configs.get("c4" if kind == "decode" else "c2")
    else:
        base = configs.get("c1")
    T = 1 if kind == "decode" else 300
    w = base.with_(name=f"wild-{case}", B=4 if kind == "decode" else 1, T=T, S=3000,
                   num_heads=heads)
    x = synth.make_inputs(w, device=DEV, seed=31)
    sc = dsa.dsa_indexer_scores(x["q_idx"], x["k_idx"], x["w"])
    idx = dsa.dsa_topk(sc, w.index_topk).cpu()
    rng = np.random.default_rng(37)
    wild = torch.from_numpy(rng.random(idx.shape) < 0.2) & (idx >= 0)
    vals = torch.tensor([w.S, w.S + 1, w.S + 4097, 2**31 - 1], dtype=torch.int32)
    pick = torch.from_numpy(rng.integers(0, len(vals), idx.shape))
    idx_wild = torch.where(wild, vals[pick], idx)
    idx_ref = torch.where(wild, torch.full_like(idx, -1), idx)
    _say(f"{case}: {int(wild.sum())} entries past the cache of {idx.numel()}")
    desc = dsa.desc_for(w)
    out = dsa.dsa_sparse_attention(desc, x["q"], x["kv"], x.get("v"), idx_wild.to(DEV))
    torch.cuda.synchronize()
    rows = list(range(T)) if T <= 8 else [0, 1, 2, 150, T - 2, T - 1]
    ref = oracle.sparse_attention(form, x["q"][:, rows], x["kv"], x.get("v"),
                                  idx_ref[:, rows], w.scale, d_v=w.d_v)
    assert max_abs_err(out[:, rows], ref) <= TOL["bf16"]
