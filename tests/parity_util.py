"""Comparison helpers for the GPU parity tests."""
import numpy as np

# Tolerances on attention outputs (max-abs over every compared element):
# fp32 storage 1e-5, bf16 storage 2e-2 (bf16 rounding of |o| < 8 is <= 1.6e-2).
TOL = {"f32": 1e-5, "bf16": 2e-2}


def assert_selection_equal(gpu_idx, ref_idx, where=""):
    """Same selected set on every row; the GPU emits its set in ascending
    order followed by -1 padding."""
    g = gpu_idx.cpu().numpy() if hasattr(gpu_idx, "cpu") else np.asarray(gpu_idx)
    r = np.asarray(ref_idx)
    assert g.shape == r.shape, (g.shape, r.shape)
    g2 = g.reshape(-1, g.shape[-1])
    r2 = r.reshape(-1, r.shape[-1])
    nvalid = (g2 >= 0).sum(-1)
    assert np.array_equal(nvalid, (r2 >= 0).sum(-1)), f"{where}: selected counts differ"
    # valid entries first, strictly ascending, then -1
    k = g2.shape[1]
    pos = np.arange(k)[None, :]
    assert np.all((g2 >= 0) == (pos < nvalid[:, None])), f"{where}: padding not at the tail"
    diffs = np.diff(np.where(g2 >= 0, g2, np.iinfo(np.int32).max), axis=-1)
    inside = pos[:, 1:] < nvalid[:, None]
    assert np.all(diffs[inside] > 0), f"{where}: selection not strictly ascending"
    gs = np.sort(np.where(g2 >= 0, g2, -1), -1)
    rs = np.sort(np.where(r2 >= 0, r2, -1), -1)
    bad = np.nonzero(~np.all(gs == rs, -1))[0]
    assert bad.size == 0, f"{where}: {bad.size} rows differ, first row {bad[0]}"


def max_abs_err(gpu, ref) -> float:
    g = gpu.detach().double().cpu().numpy() if hasattr(gpu, "detach") else np.asarray(gpu)
    return float(np.abs(g - np.asarray(ref)).max())
