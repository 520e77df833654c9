"""Host replay of the MLA attention kernel's schedule and addressing (no GPU).

tests/replay/mla_replay.cpp walks every workgroup, wave and step of the
kernel's launches through the same functions the kernel takes its ring slots,
tile schedule, workgroup mapping, split plan and global addresses from
(csrc/mla_schedule.h), and checks every LDS ring access against the barrier
schedule and every global address against its buffer.  The launches include
the 128K-context decode (8 x 131072, 128 heads, k = 2048) with valid, extreme
(every entry S-1), holed, short (t < k), past-the-cache positions and
out-of-contract entries (>= S) selections, and a
model of the kernel as committed at 07:13 on the day a GPU fault was reported
at that shape.

The mutation test plants plausible mistakes in a copy of the schedule header
and requires the replay to reject each one, so a pass means something.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "replay", "mla_replay.cpp")
CSRC = os.path.join(ROOT, "learned_sparse_attention_lightning_amd", "csrc")
HEADER = os.path.join(CSRC, "mla_schedule.h")


def _build(out, include, sanitize=False, opt="-O2"):
    cmd = ["g++", "-std=c++17", opt, "-Wall", "-Wextra", f"-I{include}", SRC, "-o", out]
    if sanitize:
        cmd[3:3] = ["-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    return r


@pytest.fixture(scope="module")
def replay_bin(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    d = tmp_path_factory.mktemp("replay")
    exe = str(d / "mla_replay")
    r = _build(exe, CSRC)
    assert r.returncode == 0, r.stderr
    return exe


def test_replay_every_launch(replay_bin):
    r = subprocess.run([replay_bin], capture_output=True, text=True, timeout=600)
    print(r.stdout)
    assert r.returncode == 0, r.stdout[-4000:]
    assert "128K decode (forward: causal tail)" in r.stdout
    assert "[07:13 kernel]" in r.stdout
    assert r.stdout.strip().endswith("ok: 0 failed checks")


def test_replay_under_host_sanitizers(tmp_path):
    """The replay itself is clean under AddressSanitizer/UBSan (mini list)."""
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "mla_replay_asan")
    r = _build(exe, CSRC, sanitize=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe, "--mini"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]


# (description, text in mla_schedule.h, replacement)
MUTANTS = [
    ("latent ring reused one slot early",
     "constexpr int ring_slot(int tile) { return tile % kRing; }",
     "constexpr int ring_slot(int tile) { return tile % (kRing - 1); }"),
    ("selection ring of half the size",
     "constexpr int sel_slot(int tile) { return tile % kSelRing; }",
     "constexpr int sel_slot(int tile) { return tile % (kSelRing / 2); }"),
    ("masked entries gather row -1",
     "const int32_t r = s > 0 ? (s < last ? s : last) : 0;",
     "const int32_t r = s < last ? s : last;"),
    ("entries past the cache not clamped",
     "const int32_t r = s > 0 ? (s < last ? s : last) : 0;",
     "const int32_t r = s > 0 ? s : 0;"),
    ("rope pieces one piece too far",
     "return latent_row_offset(s, last) + (uint64_t)kVRowBytes + 16ull * (uint64_t)half +",
     "return latent_row_offset(s, last) + (uint64_t)kVRowBytes + 16ull + 16ull * (uint64_t)half +"),
    ("partials without the dim offset",
     "return (prow * splits * H + head) * kDv + d + (size_t)split * part_split_stride(H);",
     "return (prow * splits * H + head) * kDv + (size_t)split * part_split_stride(H);"),
    ("XCD mapping drops the row group",
     "w.qidx = 8 * qg + x;",
     "w.qidx = qg + x;"),
    ("last partial split dropped",
     "p.splits = (k + p.per_split - 1) / p.per_split;",
     "p.splits = k / p.per_split;"),
    ("query block of the wrong head tile",
     "return (rowq * H + head0 + ht * 32 + l32) * kDqk",
     "return (rowq * H + head0 + ht * 64 + l32) * kDqk"),
    ("merge reads one split too many",
     "return s0 + j < splits - 1 ? s0 + j : splits - 1;",
     "return s0 + j < splits ? s0 + j : splits;"),
    ("selection written one step late",
     "constexpr int kSelAhead = 5;",
     "constexpr int kSelAhead = 6;"),
]


def _mutant_rejected(tmp, name, old, new):
    text = open(HEADER).read()
    if text.count(old) != 1:
        return f"mutation site not found: {old}"
    d = os.path.join(tmp, str(abs(hash(name))))
    os.makedirs(d)
    with open(os.path.join(d, "mla_schedule.h"), "w") as f:
        f.write(text.replace(old, new))
    exe = os.path.join(d, "mla_replay_mut")
    r = _build(exe, d, opt="-O1")
    if r.returncode != 0:
        # caught at compile time, by a static_assert of the schedule
        ok = "static assertion failed" in r.stderr or "static_assert" in r.stderr
        return None if ok else f"{name}: does not compile:\n{r.stderr[-1500:]}"
    r = subprocess.run([exe, "--mini"], capture_output=True, text=True, timeout=600)
    return None if r.returncode != 0 else f"replay accepted the mutant '{name}'"


def test_replay_rejects_planted_mistakes(tmp_path):
    """Every planted mistake in the schedule header is rejected (by the
    replay or by a static_assert of the header)."""
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        errs = list(ex.map(lambda m: _mutant_rejected(str(tmp_path), *m), MUTANTS))
    errs = [e for e in errs if e]
    assert not errs, "\n".join(errs)
