"""Host replay of the workgroup order of the masked-dense distillation-loss
kernel (no GPU).

tests/replay/kl_replay.cpp calls the functions the kernel takes its
(batch, key split, query block) and launch size from (csrc/kl_schedule.h)
for every workgroup id of a list of launches, and checks that every pair is
taken exactly once, by a workgroup of the right XCD, the causal pairs first
in per-split runs, longest block first, with equal XCD shares of the causal
triangle, and that the split merge reads only written states.

The mutation test plants plausible mistakes in a copy of the schedule header
and requires the replay to reject each one, so a pass means something.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "replay", "kl_replay.cpp")
CSRC = os.path.join(ROOT, "learned_sparse_attention_lightning_amd", "csrc")
HEADER = os.path.join(CSRC, "kl_schedule.h")


def _build_and_run(include, out):
    r = subprocess.run(["g++", "-std=c++17", "-O2", "-Wall", "-Wextra", f"-I{include}", SRC,
                        "-o", out], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return subprocess.run([out], capture_output=True, text=True, timeout=300)


@pytest.fixture(autouse=True)
def _gxx():
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")


def test_replay_every_launch(tmp_path):
    r = _build_and_run(CSRC, str(tmp_path / "kl_replay"))
    print(r.stdout)
    assert r.returncode == 0, r.stdout[-3000:]
    assert "B=1 T=4096 S=4096: 2048 workgroups" in r.stdout  # the 4K MHA prefill
    assert r.stdout.strip().endswith("ok: 0 failed checks")


MUTANTS = {
    # a block index past the causal area shifted by one
    "noncausal_block": ("w.qb = pass == 0 ? nqb - 1 - rem : rem;",
                        "w.qb = pass == 0 ? nqb - 1 - rem : rem + 1;"),
    # the causal run walked shortest block first
    "causal_order": ("w.qb = pass == 0 ? nqb - 1 - rem : rem;",
                     "w.qb = pass == 0 ? first + rem : rem;"),
    # splits dealt to XCDs in plain order (unequal shares of the triangle)
    "no_snake": ("return kXcds * k + ((k & 1) ? kXcds - 1 - x : x);",
                 "return kXcds * k + x;"),
    # the first reaching block one too late
    "first_block": ("const int qb = q <= 0 ? 0 : (q + kQ - 1) / kQ;",
                    "const int qb = q <= 0 ? 0 : (q + kQ) / kQ;"),
    # a launch one XCD share short
    "per_xcd": ("most = n > most ? n : most;", "most = n > most ? n - 1 : most;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_replay_rejects_planted_mistakes(tmp_path, name):
    a, b = MUTANTS[name]
    src = open(HEADER).read()
    assert src.count(a) == 1, name
    (tmp_path / "kl_schedule.h").write_text(src.replace(a, b))
    r = _build_and_run(str(tmp_path), str(tmp_path / "kl_replay"))
    assert r.returncode != 0, f"mutant {name} passed the replay:\n{r.stdout[-2000:]}"
