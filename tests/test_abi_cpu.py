"""The C-ABI library loads, exports every symbol its header declares, and
rejects bad arguments on the host before anything is enqueued (no GPU)."""
import ctypes
import os
import re

import pytest

from learned_sparse_attention_lightning_amd import dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")

OK, NULL, SHAPE, DTYPE, UNSUP, WS, ALIGN = 0, 1, 2, 3, 4, 5, 6
A = 0x10000  # a 16-byte aligned fake address: never dereferenced, checks fail first
M = 0x10004  # misaligned


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dsa.lib_path()):
        import __graft_entry__
        __graft_entry__.build()
    return dsa.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(dsa_\w+)\s*\(", text, re.M)))


def test_header_declares_the_binding_names():
    assert set(declared_functions()) == set(dsa.EXPORTED)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.dsa_abi_version() == 4
    for s in range(8):
        assert lib.dsa_status_string(s)
    assert lib.dsa_status_string(99) == b"unknown status"


def _desc(form=dsa.DSA_MLA, H=128, dqk=576, dv=512, dt=dsa.DSA_BF16, odt=dsa.DSA_BF16):
    return dsa.AttnDesc(form, H, dqk, dv, 0.07, dt, odt)


def test_workspace_sizes(lib):
    d = _desc()
    ws = lambda op, *a: lib.dsa_workspace_bytes(op, ctypes.byref(d), *a)  # noqa: E731
    bad = ctypes.c_size_t(-1).value
    assert ws(dsa.DSA_OP_TOPK, 1, 16, 16, 2, 2, 3) != bad
    assert ws(dsa.DSA_OP_FORWARD, 1, 4096, 4096, 64, 128, 2048) >= 4096 * 4096 * 4
    # the score block is bounded (1 GiB) for long prefill: 32K and 128K
    # contexts need the score block, the selection and a little more
    assert ws(dsa.DSA_OP_FORWARD, 1, 32768, 32768, 64, 128, 2048) < (1 << 30) + (512 << 20)
    assert ws(dsa.DSA_OP_FORWARD, 1, 131072, 131072, 64, 128, 2048) < (3 << 30)
    assert ws(dsa.DSA_OP_FORWARD, 1, 16, 16, 2, 2, 17) != bad  # k > S is allowed
    assert ws(dsa.DSA_OP_FORWARD, 1, 16, 16, 2, 2, (1 << 20) + 1) == bad
    assert ws(dsa.DSA_OP_FORWARD, 0, 16, 16, 2, 2, 3) == bad
    assert lib.dsa_workspace_bytes(dsa.DSA_OP_FORWARD, None, 1, 16, 16, 2, 2, 3) == bad
    assert ws(7, 1, 16, 16, 2, 2, 3) == bad


def test_indexer_argument_checks(lib):
    f = lib.dsa_indexer_scores
    assert f(None, A, 1, A, None, 1, 4, 4, 64, 128, A, None) == NULL
    assert f(A, A, 1, A, None, 1, 4, 4, 64, 128, None, None) == NULL
    assert f(A, A, 9, A, None, 1, 4, 4, 64, 128, A, None) == DTYPE
    assert f(A, A, 1, A, None, 0, 4, 4, 64, 128, A, None) == SHAPE
    assert f(A, A, 1, A, None, 1, 5, 4, 64, 128, A, None) == SHAPE  # T > S without q_pos
    assert f(A, A, 1, A, None, 1, 4, 4, 0, 128, A, None) == SHAPE
    assert f(A, A, 1, A, None, 1, 4, 4, 129, 128, A, None) == SHAPE
    assert f(A, A, 1, A, None, 1, 4, 4, 128, 256, A, None) == UNSUP
    assert f(M, A, 1, A, None, 1, 4, 4, 64, 128, A, None) == ALIGN
    assert f(A, A, 1, A, None, 1, 4, 4, 64, 128, M, None) == ALIGN


def test_indexer_ex_flags(lib):
    f = lib.dsa_indexer_scores_ex
    assert f(A, A, 1, A, None, 1, 4, 4, 64, 128, 2, A, None) == UNSUP   # unknown flag bit
    assert f(None, A, 1, A, None, 1, 4, 4, 64, 128, 1, A, None) == NULL
    assert f(A, A, 1, A, None, 1, 4, 4, 64, 128, 1, M, None) == ALIGN


def test_attention_scale_must_be_positive(lib):
    f = lib.dsa_sparse_attention
    for bad_scale in (0.0, -0.5, float("inf"), float("nan")):
        d = dsa.AttnDesc(dsa.DSA_MLA, 128, 576, 512, bad_scale, dsa.DSA_BF16, dsa.DSA_BF16)
        assert f(ctypes.byref(d), A, A, None, A, 1, 4, 4, 2, A, None, None, 0, None) == SHAPE


def test_noalloc_forward_rejects_sizes_beyond_its_scratch(lib):
    """dsa_forward_ex_noalloc: sizes whose forward workspace exceeds the
    128 MiB scratch are rejected on the host before anything is enqueued."""
    d = _desc()
    f = lib.dsa_forward_ex_noalloc
    need = lib.dsa_workspace_bytes(dsa.DSA_OP_FORWARD, ctypes.byref(d), 1, 32768, 32768, 64,
                                   128, 2048)
    assert need > (128 << 20)
    assert f(ctypes.byref(d), A, A, 1, A, A, A, None, None, 1, 32768, 32768, 64, 128, 2048, 0,
             A, None, None) == WS
    assert f(ctypes.byref(d), None, A, 1, A, A, A, None, None, 8, 1, 131072, 64, 128, 2048, 0,
             A, None, None) == NULL
    assert f(ctypes.byref(d), A, A, 1, A, A, A, None, None, 8, 1, 131072, 64, 128, 2048, 2,
             A, None, None) == UNSUP


def test_topk_argument_checks(lib):
    f = lib.dsa_topk
    assert f(None, None, 1, 4, 4, 2, A, None, 0, None) == NULL
    assert f(A, None, 1, 4, 4, 0, A, None, 0, None) == SHAPE
    assert f(A, None, 1, 4, 4, (1 << 20) + 1, A, None, 0, None) == SHAPE  # k may exceed S, to 2^20
    assert f(A, None, 1, 4, 4, 2, M, None, 0, None) == ALIGN
    assert f(A, None, 70000, 4, 4, 2, A, None, 0, None) == SHAPE


def test_topk_ex_argument_checks(lib):
    f = lib.dsa_topk_ex
    cur = dsa.DSA_SEL_INCLUDE_CURRENT
    assert f(None, None, 1, 4, 4, 2, cur, A, None, 0, None) == NULL
    assert f(A, None, 1, 4, 4, 0, cur, A, None, 0, None) == SHAPE
    assert f(A, None, 1, 4, 4, 2, 2, A, None, 0, None) == UNSUP  # unknown flag bit
    assert f(A, None, 1, 4, 4, 2, cur, M, None, 0, None) == ALIGN


def test_attention_argument_checks(lib):
    f = lib.dsa_sparse_attention
    d = _desc()
    assert f(None, A, A, None, A, 1, 1, 8, 2, A, None, None, 0, None) == NULL
    assert f(ctypes.byref(d), A, A, A, A, 1, 1, 8, 2, A, None, None, 0, None) == SHAPE  # v for MLA
    d2 = _desc(form=dsa.DSA_MHA, H=4, dqk=64, dv=64)
    assert f(ctypes.byref(d2), A, A, None, A, 1, 1, 8, 2, A, None, None, 0, None) == NULL
    d3 = _desc(dt=7)
    assert f(ctypes.byref(d3), A, A, None, A, 1, 1, 8, 2, A, None, None, 0, None) == DTYPE
    d4 = _desc(dt=dsa.DSA_FP8_E4M3)
    assert f(ctypes.byref(d4), A, A, None, A, 1, 1, 8, 2, A, None, None, 0, None) == UNSUP
    d5 = _desc(dqk=600)
    assert f(ctypes.byref(d5), A, A, None, A, 1, 1, 8, 2, A, None, None, 0, None) == SHAPE
    assert f(ctypes.byref(d), M, A, None, A, 1, 1, 8, 2, A, None, None, 0, None) == ALIGN
    assert f(ctypes.byref(d), A, A, None, A, 1, 1, 8, (1 << 20) + 1, A, None, None, 0,
             None) == SHAPE
    d6 = _desc(form=5)
    assert f(ctypes.byref(d6), A, A, None, A, 1, 1, 8, 2, A, None, None, 0, None) == SHAPE


def test_forward_argument_checks(lib):
    f = lib.dsa_forward
    d = _desc()
    args = [ctypes.byref(d), A, A, 1, A, A, A, None, None, 1, 1, 8, 64, 128, 2, A, None]
    assert f(*args, None, 0, None) == WS
    assert f(*args, A, 16, None) == WS
    bad = list(args)
    bad[1] = None
    assert f(*bad, A, 1 << 40, None) == NULL
    bad = list(args)
    bad[15] = M
    assert f(*bad, A, 1 << 40, None) == ALIGN


def test_forward_ex_argument_checks(lib):
    f = lib.dsa_forward_ex
    d = _desc()
    head = [ctypes.byref(d), A, A, 1, A, A, A, None, None, 1, 1, 8, 64, 128, 2]
    cur = dsa.DSA_SEL_INCLUDE_CURRENT
    assert f(*head, cur, A, None, None, 0, None) == WS
    assert f(*head, 4, A, None, A, 1 << 40, None) == UNSUP
    bad = list(head)
    bad[1] = None
    assert f(*bad, cur, A, None, A, 1 << 40, None) == NULL


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 4, 2, 2)
    with pytest.raises(ValueError):
        dsa.dsa_indexer_scores(x, torch.zeros(1, 4, 2), torch.zeros(1, 4, 2))


def test_indexer_kl_argument_checks(lib):
    f = lib.dsa_indexer_kl
    d = _desc()
    assert f(None, A, A, A, A, A, 1, 4, 8, 2, A, None) == NULL
    d2 = _desc(form=dsa.DSA_MHA, H=4, dqk=96, dv=96)
    assert f(ctypes.byref(d2), A, A, A, A, A, 1, 4, 8, 2, A, None) == UNSUP
    d3 = _desc(form=dsa.DSA_MHA, H=65, dqk=64, dv=64)
    assert f(ctypes.byref(d3), A, A, A, A, A, 1, 4, 8, 2, A, None) == UNSUP
    assert f(ctypes.byref(d), A, A, None, A, A, 1, 4, 8, 2, A, None) == NULL
    assert f(ctypes.byref(d), A, A, A, A, A, 1, 4, 8, 0, A, None) == SHAPE
    assert f(ctypes.byref(d), A, A, A, M, A, 1, 4, 8, 2, A, None) == ALIGN


def test_indexer_kl_ex_workspace(lib):
    """dsa_indexer_kl_ex: the masked-dense MHA form asks for a workspace (one
    bit per (row, key), the rows' last selected positions, the split states);
    other shapes ask for none; a workspace below the need is refused on the
    host."""
    ws = lib.dsa_workspace_bytes
    mha = _desc(form=dsa.DSA_MHA, H=16, dqk=128, dv=128)
    need = ws(dsa.DSA_OP_KL, ctypes.byref(mha), 1, 4096, 4096, 1, 1, 2048)
    rows, words, splits = 4096, 4096 // 32, 4096 // 256
    r256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
    assert need == r256(rows * words * 4) + r256(rows * 4) + r256(rows * splits * 20)
    # a sparse selection (k < S/4), the MLA form, fp32 and 32 heads: the
    # per-entry form, no workspace
    assert ws(dsa.DSA_OP_KL, ctypes.byref(mha), 1, 4096, 4096, 1, 1, 1000) == 0
    assert ws(dsa.DSA_OP_KL, ctypes.byref(_desc()), 1, 4096, 4096, 1, 1, 2048) == 0
    f32 = _desc(form=dsa.DSA_MHA, H=16, dqk=128, dv=128, dt=dsa.DSA_F32, odt=dsa.DSA_F32)
    assert ws(dsa.DSA_OP_KL, ctypes.byref(f32), 1, 4096, 4096, 1, 1, 2048) == 0
    h32 = _desc(form=dsa.DSA_MHA, H=32, dqk=128, dv=128)
    assert ws(dsa.DSA_OP_KL, ctypes.byref(h32), 1, 4096, 4096, 1, 1, 2048) == 0
    f = lib.dsa_indexer_kl_ex
    assert f(ctypes.byref(mha), A, A, A, A, A, 1, 4096, 4096, 2048, A, A, need - 1, None) == WS
    assert f(ctypes.byref(mha), A, A, A, A, A, 1, 4096, 4096, 2048, A, M, need, None) == WS
    assert f(None, A, A, A, A, A, 1, 4, 8, 2, A, None, 0, None) == NULL


def test_attention_ex_argument_checks(lib):
    f = lib.dsa_sparse_attention_ex
    d = _desc()
    pre = dsa.DSA_ATTN_CAUSAL_PREFIX
    assert f(None, A, A, None, A, None, pre, 1, 1, 8, 2, A, None, None, 0, None) == NULL
    assert f(ctypes.byref(d), A, A, None, A, None, 2, 1, 1, 8, 2, A, None, None, 0, None) == UNSUP
    # default positions need T <= S
    assert f(ctypes.byref(d), A, A, None, A, None, pre, 1, 9, 8, 2, A, None, None, 0, None) == SHAPE
    assert f(ctypes.byref(d), M, A, None, A, None, pre, 1, 1, 8, 2, A, None, None, 0, None) == ALIGN
