"""Build libdsa.so: every HIP source under csrc/ compiled for gfx950 with
hipcc, then linked into one shared library placed next to this file; and
libdsa_probes.so from probes/ (device peak probes the benchmark uses for its
roofline fractions; not part of the forward path).

    python -m learned_sparse_attention_lightning_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdsa.so")
PROBES = os.path.join(PKG, "probes")
PROBE_LIB = os.path.join(PKG, "libdsa_probes.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# packed fp32 ops are switched off for every HIP translation unit
FLAGS = ["-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}", "-fvisibility=hidden",
         "-Wall", "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", f"-I{INCLUDE}", f"-I{CSRC}"]
# Per-file extras.  The indexer's MFMA results feed VALU arithmetic right away
# (ReLU, head weights), so they go to ordinary VGPRs rather than AGPRs, which
# would need a v_accvgpr_read per element.
EXTRA = {"indexer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def sources(d=CSRC):
    return sorted(os.path.join(d, f) for f in os.listdir(d) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    # the host pass does not know the packed-fp32 feature; drop that warning
    noise = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    r = subprocess.run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(jobs: int | None = None) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    probe_srcs = sources(PROBES)
    with cf.ThreadPoolExecutor(max_workers=jobs or min(8, len(srcs) + len(probe_srcs))) as ex:
        objs = list(ex.map(_compile, srcs + probe_srcs))
    _link(objs[: len(srcs)], LIB)
    _link(objs[len(srcs):], PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build())
