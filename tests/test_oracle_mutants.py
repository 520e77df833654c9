"""The oracle's pins must catch plausible mistakes.

Each case below plants one mistake in a copy of the oracle's C source (a
dropped term, a wrong sign, index or bound, a transposed operand), builds the
copy on the CPU and runs the pin suite against it in a child process.  The
suite must fail for every mutant; the unmodified source must pass.
"""
import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "dsa_oracle.c")

MUTANTS = {
    "relu_dropped": ("const double relu = dot > 0.0 ? dot : 0.0;", "const double relu = dot;"),
    "relu_sign": ("const double relu = dot > 0.0 ? dot : 0.0;", "const double relu = dot < 0.0 ? -dot : 0.0;"),
    "head_weight_dropped": ("total += w[(b * T + i) * H + j] * relu;", "total += relu;"),
    "head_weight_index": ("total += w[(b * T + i) * H + j] * relu;", "total += w[(b * T + i) * H + (H - 1 - j)] * relu;"),
    "query_head_shared": ("const double *qv = q_idx + ((b * T + i) * H + j) * D;", "const double *qv = q_idx + ((b * T + i) * H) * D;"),
    "causal_excludes_self": ("if (s > t) {\n                    row[s] = -INFINITY;", "if (s >= t) {\n                    row[s] = -INFINITY;"),
    "tie_higher_index": ("return (a->pos < b->pos) ? -1 : (a->pos > b->pos);", "return (a->pos > b->pos) ? -1 : (a->pos < b->pos);"),
    "ascending_scores": ("if (a->score > b->score) return -1;\n    if (a->score < b->score) return 1;", "if (a->score < b->score) return -1;\n    if (a->score > b->score) return 1;"),
    "candidates_exclude_self": ("const int64_t n_cand = t + 1 - forced;", "const int64_t n_cand = (t > 0 ? t : 1) - forced;"),
    "sparse_target_head_sum": ("if (sel[r] >= 0) prow[sel[r]] += alpha[r] / z / (double)H;", "if (sel[r] >= 0) prow[sel[r]] += alpha[r] / z;"),
    "sparse_target_unscaled": ("                    alpha[r] = scale * dot;", "                    alpha[r] = dot;"),
    "current_not_forced": ("const int64_t forced = (include_current && t >= 0) ? 1 : 0;", "const int64_t forced = 0;"),
    "current_budget_not_reduced": ("const int64_t n_cand = t + 1 - forced;", "const int64_t n_cand = t + 1;"),
    "scale_dropped": ("logit[r] = scale * dot;", "logit[r] = dot;"),
    "not_normalised": ("for (int64_t d = 0; d < dv; ++d) o[d] /= denom;", ""),
    "mla_value_tail": ("    return kv + (b * S + s) * dqk;\n}\n\n/*\n * Attention restricted", "    return kv + (b * S + s) * dqk + (dqk - dv);\n}\n\n/*\n * Attention restricted"),
    "mha_key_head_transposed": ("if (form == 0) return kv + ((b * S + s) * H + h) * dqk;", "if (form == 0) return kv + ((b * S + s) * H + (H - 1 - h)) * dqk;"),
    "warmup_target_head_sum": ("for (int64_t s = 0; s <= t; ++s) prow[s] /= total;", ""),
    "position_not_clamped": ("return t >= S ? S - 1 : t;", "return t;"),
    "dense_excludes_self": ("for (int64_t s = 0; s <= t; ++s) {\n                    const double *key = key_row", "for (int64_t s = 0; s < t; ++s) {\n                    const double *key = key_row"),
}


def _run_suite(lib_path):
    env = dict(os.environ, DSA_ORACLE_LIB=lib_path, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    return r.returncode


def _build_and_run(name, src_text, tmp):
    import oracle
    c = os.path.join(tmp, f"{name}.c")
    so = os.path.join(tmp, f"{name}.so")
    with open(c, "w") as f:
        f.write(src_text)
    oracle.build(force=True, src=c, out=so)
    return name, _run_suite(so)


def test_pins_kill_every_mutant():
    with open(SRC) as f:
        base = f.read()
    with tempfile.TemporaryDirectory() as tmp:
        jobs = {"unmodified": base}
        for name, (old, new) in MUTANTS.items():
            assert base.count(old) >= 1, f"mutation site of {name} not found"
            jobs[name] = base.replace(old, new, 1)
        with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            results = dict(ex.map(lambda kv: _build_and_run(kv[0], kv[1], tmp), jobs.items()))
    assert results.pop("unmodified") == 0, "pin suite fails on the unmodified oracle"
    survivors = [n for n, rc in results.items() if rc == 0]
    assert not survivors, f"mutants not caught by the pins: {survivors}"
