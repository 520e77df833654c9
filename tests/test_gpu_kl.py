"""The indexer's distillation loss (forward) on the GPU against the oracle.

The GPU pipeline (indexer scores, top-k, attention with its log-sum-exp, then
the loss kernel) runs on seeded inputs; the oracle computes its own scores,
selection, head-mean target over the set and per-row KL in fp64.  Scores and
selections are bit-exact (integer indexer inputs), so the rows compare term
by term.  Tolerance: the logits are fp32 sums of bf16 products recomputed
beside the attention's own, so p carries ~1e-6 relative error per entry and
the fp32 sums over <= 2048 entries add ~1e-5 relative: |gpu - ref| <=
1e-3 * max(1, |ref|)."""
import numpy as np
import pytest
import torch

import oracle

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


def _gpu_loss(w, x, k, include_current=False):
    desc = dsa.desc_for(w)
    sc = dsa.dsa_indexer_scores(x["q_idx"], x["k_idx"], x["w"])
    idx = dsa.dsa_topk(sc, k, include_current=include_current)
    lse = torch.empty((w.B, w.T, w.num_heads), dtype=torch.float32, device=DEV)
    dsa.dsa_sparse_attention(desc, x["q"], x["kv"], None, idx, lse=lse)
    loss = dsa.dsa_indexer_kl(desc, x["q"], x["kv"], idx, lse, sc)
    torch.cuda.synchronize()
    return sc, idx, loss


def _oracle_loss(w, x, rows, k, include_current=False):
    pos = np.array([[w.S - w.T + r for r in rows]] * w.B)
    sc = oracle.indexer_scores(x["q_idx"][:, rows], x["k_idx"], x["w"][:, rows], q_pos=pos)
    sel = oracle.topk(sc, k, q_pos=pos, include_current=include_current)
    p = oracle.sparse_target("mla", x["q"][:, rows], x["kv"], sel, w.scale)
    return sel, oracle.indexer_kl_rows(p, sc, oracle.selection_mask(sel, w.S))


def _check(loss, ref, where):
    g = loss.double().cpu().numpy()
    err = np.abs(g - ref) / np.maximum(1.0, np.abs(ref))
    _say(f"{where}: loss range {ref.min():.4g}..{ref.max():.4g}, max rel err {err.max():.3e}")
    assert np.all(np.isfinite(g)) and err.max() <= 1e-3, where


@pytest.mark.parametrize("heads", [32, 64, 128])
def test_indexer_kl_sparse_stage(heads):
    w = configs.get("c2").with_(name=f"kl-{heads}", B=2, T=300, S=300, index_topk=64,
                                num_heads=heads)
    x = synth.make_inputs(w, device=DEV, seed=31 + heads)
    sc, idx, loss = _gpu_loss(w, x, w.index_topk)
    rows = list(range(w.T))
    _, ref = _oracle_loss(w, x, rows, w.index_topk)
    _check(loss, ref, f"sparse stage H={heads}")
    # row 0 selects only itself: p = softmax = 1 there, KL = 0
    assert np.abs(loss[:, 0].cpu().numpy()).max() <= 1e-5


def test_indexer_kl_dense_warmup():
    """Every causal position selected (k >= S): the warm-up loss."""
    w = configs.get("c2").with_(name="kl-dense", B=1, T=200, S=200, index_topk=256,
                                num_heads=32)
    x = synth.make_inputs(w, device=DEV, seed=5)
    sc, idx, loss = _gpu_loss(w, x, w.index_topk)
    _, ref = _oracle_loss(w, x, list(range(w.T)), w.index_topk)
    _check(loss, ref, "dense warm-up")


def test_indexer_kl_long_rows_sampled():
    """k = 2048 over 6000 keys at 128 heads: several tile pairs per wave."""
    w = configs.get("c2").with_(name="kl-long", B=1, T=6000, S=6000)
    x = synth.make_inputs(w, device=DEV, seed=8)
    sc, idx, loss = _gpu_loss(w, x, w.index_topk, include_current=True)
    rows = [0, 1, 2047, 2048, 4000, 5999]
    sel, ref = _oracle_loss(w, x, rows, w.index_topk, include_current=True)
    _check(loss[:, rows], ref, "long rows")


def test_indexer_kl_unit_scale_scores():
    """Scores of unit scale (softmax far from one-hot): every term of the
    divergence matters; the selection is the top-k of those scores."""
    w = configs.get("c2").with_(name="kl-unit", B=2, T=400, S=400, index_topk=128,
                                num_heads=64)
    x = synth.make_inputs(w, device=DEV, seed=12)
    sc = synth.random_scores((w.B, w.T, w.S), seed=4)
    desc = dsa.desc_for(w)
    idx = dsa.dsa_topk(sc.to(DEV), w.index_topk)
    lse = torch.empty((w.B, w.T, w.num_heads), dtype=torch.float32, device=DEV)
    dsa.dsa_sparse_attention(desc, x["q"], x["kv"], None, idx, lse=lse)
    loss = dsa.dsa_indexer_kl(desc, x["q"], x["kv"], idx, lse, sc.to(DEV))
    torch.cuda.synchronize()
    sel = oracle.topk(sc, w.index_topk)
    p = oracle.sparse_target("mla", x["q"], x["kv"], sel, w.scale)
    ref = oracle.indexer_kl_rows(p, sc, oracle.selection_mask(sel, w.S))
    _check(loss, ref, "unit-scale scores")
    assert ref[:, 50:].min() > 0.05  # far from zero: p and softmax differ


def test_indexer_kl_unordered_selection_with_holes():
    """Any set of distinct positions in any slot order, unused slots anywhere
    (the loss is a function of the set): permuted rows with holes punched in."""
    w = configs.get("c2").with_(name="kl-holes", B=1, T=256, S=256, index_topk=96,
                                num_heads=32)
    x = synth.make_inputs(w, device=DEV, seed=41)
    sc = synth.random_scores((w.B, w.T, w.S), seed=6)
    sel = oracle.topk(sc, w.index_topk)           # rank order, -1 padded
    rng = np.random.default_rng(2)
    for i in range(w.T):
        sel[0, i] = sel[0, i, rng.permutation(w.index_topk)]
        holes = rng.choice(w.index_topk, size=10, replace=False)
        sel[0, i, holes] = -1
    sel[0, 7, :] = -1                             # an empty row: loss 0
    idx = torch.from_numpy(sel).to(DEV)
    desc = dsa.desc_for(w)
    lse = torch.empty((w.B, w.T, w.num_heads), dtype=torch.float32, device=DEV)
    dsa.dsa_sparse_attention(desc, x["q"], x["kv"], None, idx, lse=lse)
    loss = dsa.dsa_indexer_kl(desc, x["q"], x["kv"], idx, lse, sc.to(DEV))
    torch.cuda.synchronize()
    p = oracle.sparse_target("mla", x["q"], x["kv"], sel, w.scale)
    ref = oracle.indexer_kl_rows(p, sc, oracle.selection_mask(sel, w.S))
    _check(loss, ref, "unordered with holes")
    assert loss[0, 7].item() == 0.0


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_indexer_kl_mha_sparse_stage(dtype):
    """MHA form (a key row per head): the pipeline's loss against the oracle."""
    w = configs.get("c1").with_(name=f"kl-mha-{dtype}", B=2, T=300, S=300, index_topk=64,
                                dtype=dtype, out_dtype=dtype)
    x = synth.make_inputs(w, device=DEV, seed=51)
    desc = dsa.desc_for(w)
    sc = dsa.dsa_indexer_scores(x["q_idx"], x["k_idx"], x["w"])
    idx = dsa.dsa_topk(sc, w.index_topk)
    lse = torch.empty((w.B, w.T, w.num_heads), dtype=torch.float32, device=DEV)
    dsa.dsa_sparse_attention(desc, x["q"], x["kv"], x["v"], idx, lse=lse)
    loss = dsa.dsa_indexer_kl(desc, x["q"], x["kv"], idx, lse, sc)
    torch.cuda.synchronize()
    rsc = oracle.indexer_scores(x["q_idx"], x["k_idx"], x["w"])
    sel = oracle.topk(rsc, w.index_topk)
    p = oracle.sparse_target("mha", x["q"], x["kv"], sel, w.scale)
    ref = oracle.indexer_kl_rows(p, rsc, oracle.selection_mask(sel, w.S))
    _check(loss, ref, f"MHA {dtype}")


def test_indexer_kl_mha_dense_warmup_target():
    """Every causal position selected: the GPU loss against KL(p || softmax(I))
    with p the oracle's dense warm-up target ([P1] section 5.2)."""
    w = configs.get("c1").with_(name="kl-mha-warm", B=1, T=200, S=200, index_topk=256)
    x = synth.make_inputs(w, device=DEV, seed=52)
    desc = dsa.desc_for(w)
    sc = dsa.dsa_indexer_scores(x["q_idx"], x["k_idx"], x["w"])
    idx = dsa.dsa_topk(sc, w.index_topk)
    lse = torch.empty((w.B, w.T, w.num_heads), dtype=torch.float32, device=DEV)
    dsa.dsa_sparse_attention(desc, x["q"], x["kv"], x["v"], idx, lse=lse)
    loss = dsa.dsa_indexer_kl(desc, x["q"], x["kv"], idx, lse, sc)
    torch.cuda.synchronize()
    rsc = oracle.indexer_scores(x["q_idx"], x["k_idx"], x["w"])
    p = oracle.warmup_target(x["q"], x["kv"], w.scale)
    causal = np.tril(np.ones((w.T, w.S), dtype=np.int8))[None]
    ref = oracle.indexer_kl_rows(p, rsc, causal)
    _check(loss, ref, "MHA dense warm-up")


def _mha_dense_case(w, seed, holes=False, any_position=False):
    """Seeded inputs, integer-valued scores and the oracle's own selection
    (ranked, or shuffled with holes; any_position: every row ranks all S
    positions, so early rows also select later ones), the GPU attention's
    lse over it, then the GPU loss and the oracle's."""
    x = synth.make_inputs(w, device=DEV, seed=seed)
    desc = dsa.desc_for(w)
    g = torch.Generator().manual_seed(seed)
    sc = torch.randint(-64, 64, (w.B, w.T, w.S), generator=g).to(torch.float32) / 8
    pos = np.full((w.B, w.T), w.S - 1, dtype=np.int32) if any_position else None
    sel = oracle.topk(sc, w.index_topk, q_pos=pos)
    if holes:  # unordered rows, a few entries dropped (still distinct positions)
        rng = np.random.default_rng(seed)
        for b in range(w.B):
            for i in range(w.T):
                rng.shuffle(sel[b, i])
                sel[b, i, rng.random(w.index_topk) < 0.05] = -1
    idx = torch.from_numpy(sel).to(DEV)
    assert dsa.workspace_bytes(dsa.DSA_OP_KL, desc, w.B, w.T, w.S, 1, 1, w.index_topk) > 0
    lse = torch.empty((w.B, w.T, w.num_heads), dtype=torch.float32, device=DEV)
    dsa.dsa_sparse_attention(desc, x["q"], x["kv"], x["v"], idx, lse=lse)
    loss = dsa.dsa_indexer_kl(desc, x["q"], x["kv"], idx, lse, sc.to(DEV))
    torch.cuda.synchronize()
    p = oracle.sparse_target("mha", x["q"], x["kv"], sel, w.scale)
    ref = oracle.indexer_kl_rows(p, sc, oracle.selection_mask(sel, w.S))
    return loss, ref


@pytest.mark.parametrize("heads,dim", [(16, 128), (8, 128), (16, 64), (8, 64)])
def test_indexer_kl_mha_masked_dense(heads, dim):
    """The masked-dense MHA form (k >= S/4): 1500 rows and keys, so the query
    blocks of 32 rows, the 32-key tiles and the splits of 256 keys all end
    ragged; against the oracle's loss over the same selection."""
    w = configs.get("c1").with_(name=f"kl-mha-dense-{heads}x{dim}", B=2, T=1500, S=1500,
                                index_topk=512, num_heads=heads, d_qk=dim, d_v=dim,
                                index_n_heads=4, index_head_dim=32)
    loss, ref = _mha_dense_case(w, seed=61)
    _check(loss, ref, f"MHA masked-dense {heads}x{dim}")


def test_indexer_kl_mha_masked_dense_rows_at_the_end():
    """Rows at the end of a longer cache (row t at position S - T + t) and 20
    key splits (three per XCD, the last XCD slot partly past the last
    split): every launched (split, query block) pair and only those."""
    w = configs.get("c1").with_(name="kl-mha-dense-offset", B=2, T=300, S=5000,
                                index_topk=1300, num_heads=16, d_qk=64, d_v=64,
                                index_n_heads=4, index_head_dim=32)
    loss, ref = _mha_dense_case(w, seed=63)
    _check(loss, ref, "MHA masked-dense, rows at the end of a 5000-key cache")


def test_indexer_kl_mha_masked_dense_any_position():
    """Selections that include positions past a row's own (the entry point
    takes any distinct positions < S): the key ranges past the causal area
    are launched too, after it, and fold what is selected there."""
    w = configs.get("c1").with_(name="kl-mha-dense-any", B=1, T=700, S=700, index_topk=256,
                                num_heads=8, d_qk=64, d_v=64, index_n_heads=4, index_head_dim=32)
    loss, ref = _mha_dense_case(w, seed=64, any_position=True)
    _check(loss, ref, "MHA masked-dense, selections past the row's position")


def test_indexer_kl_mha_masked_dense_holes():
    """Unordered selection rows with holes through the masked-dense form."""
    w = configs.get("c1").with_(name="kl-mha-dense-holes", B=1, T=700, S=700, index_topk=256,
                                index_n_heads=4, index_head_dim=32)
    loss, ref = _mha_dense_case(w, seed=62, holes=True)
    _check(loss, ref, "MHA masked-dense, unordered with holes")


@pytest.mark.timeout(600)
def test_indexer_kl_c1_sampled_rows():
    """The 4K MHA prefill (n = 4096, 16 heads x 128, k = 2048): the GPU
    pipeline's scores, selection and lse, the masked-dense loss; the oracle's
    loss over the GPU's selection and scores on 96 rows spread over the
    causal range (sets and scores equal the oracle's bit for bit in the
    parity tests)."""
    w = configs.get("c1")
    x = synth.make_inputs(w, device=DEV, seed=synth.default_seed(w))
    desc = dsa.desc_for(w)
    sc = dsa.dsa_indexer_scores(x["q_idx"], x["k_idx"], x["w"])
    idx = dsa.dsa_topk(sc, w.index_topk)
    lse = torch.empty((w.B, w.T, w.num_heads), dtype=torch.float32, device=DEV)
    dsa.dsa_sparse_attention(desc, x["q"], x["kv"], x["v"], idx, lse=lse)
    loss = dsa.dsa_indexer_kl(desc, x["q"], x["kv"], idx, lse, sc)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, 8), np.linspace(8, w.T - 9, 80).astype(int),
                                     np.arange(w.T - 8, w.T)]))
    sel = idx[:, rows].cpu().numpy()
    p = oracle.sparse_target("mha", x["q"][:, rows], x["kv"], sel, w.scale)
    ref = oracle.indexer_kl_rows(p, sc[:, rows].cpu(), oracle.selection_mask(sel, w.S))
    _check(loss[:, rows], ref, f"c1 masked-dense loss, {len(rows)} rows")
