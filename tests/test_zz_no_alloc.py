"""The allocation-free forward entry point (dsa_forward_ex_noalloc) through the
C ABI against dsa_forward_ex with a caller workspace: identical selections and
outputs (same kernels, same launches) on two calls in a row, the second with a
smaller input, and sizes beyond the scratch rejected before any launch."""
import ctypes

import pytest
import torch

from learned_sparse_attention_lightning_amd import configs, dsa, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsa.load()


def _say(msg):
    print(msg, flush=True)


def _both(w, seed, include_current=False):
    x = synth.make_inputs(w, device=DEV, seed=seed)
    desc = dsa.desc_for(w)
    idx_a = torch.full((w.B, w.T, w.index_topk), -7, dtype=torch.int32, device=DEV)
    idx_b = torch.full_like(idx_a, -9)
    out_a = dsa.dsa_forward(desc, x["q_idx"], x["k_idx"], x["w"], x["q"], x["kv"], x["v"],
                            w.index_topk, idx_out=idx_a, include_current=include_current)
    out_b = dsa.dsa_forward_noalloc(desc, x["q_idx"], x["k_idx"], x["w"], x["q"], x["kv"],
                                    x["v"], w.index_topk, idx_out=idx_b,
                                    include_current=include_current)
    torch.cuda.synchronize()
    return idx_a, out_a, idx_b, out_b


def test_noalloc_matches_workspace_entry_two_calls():
    # first call: the 128K decode workload at full size
    w1 = configs.get("c4")
    _say("noalloc: 128K decode, 8 x 131072")
    idx_a, out_a, idx_b, out_b = _both(w1, seed=5)
    assert torch.equal(idx_a, idx_b), "selections differ (128K decode)"
    assert torch.equal(out_a, out_b), "outputs differ (128K decode)"
    # second call, smaller: 3 sequences x 20000 with the current token kept
    # (the scratch holds the previous call's contents)
    w2 = configs.get("c4").with_(name="small", B=3, S=20000)
    _say("noalloc: 3 x 20000 decode, current token kept")
    idx_a, out_a, idx_b, out_b = _both(w2, seed=6, include_current=True)
    assert torch.equal(idx_a, idx_b), "selections differ (small decode)"
    assert torch.equal(out_a, out_b), "outputs differ (small decode)"
    # and a small prefill (one chunk of rows, the per-row top-k, no splits)
    w3 = configs.get("c2").with_(name="small-prefill", T=600, S=600, index_topk=256)
    _say("noalloc: 600-token MLA prefill")
    idx_a, out_a, idx_b, out_b = _both(w3, seed=7)
    assert torch.equal(idx_a, idx_b) and torch.equal(out_a, out_b), "small prefill differs"


def test_noalloc_rejects_sizes_beyond_the_scratch():
    lib = dsa.load()
    w = configs.get("c2")
    desc = dsa.desc_for(w)
    need = dsa.workspace_bytes(dsa.DSA_OP_FORWARD, desc, w.B, w.T, w.S, w.index_n_heads,
                               w.index_head_dim, w.index_topk)
    assert need > (128 << 20)
    fake = ctypes.c_void_p(0x10000)  # aligned, never dereferenced: the size check fails first
    st = lib.dsa_forward_ex_noalloc(ctypes.byref(desc), fake, fake, dsa.DSA_BF16, fake, fake,
                                    fake, None, None, w.B, w.T, w.S, w.index_n_heads,
                                    w.index_head_dim, w.index_topk, 0, fake, None, None)
    assert st == 5  # DSA_ERR_WORKSPACE
