"""Shared helpers of the GPU parity tests: uploads, downloads and the parity
rules (row-wise relative error, top-k band rule)."""
import numpy as np
import torch

from long_context_sparse_11_amd import synth
from long_context_sparse_11_amd.device import to_device

# Parity bars (attention/compress: max over rows of ||gpu - ref||_inf / ||ref||_inf)
TOL_F32 = 1e-5
TOL_BF16 = 2e-2
BAND = 1e-4   # top-k: symmetric difference only within this of the K-th score


def dev(x, dtype=None):
    """Host array / synth.Tensor -> contiguous CUDA tensor (bf16 bits kept)."""
    t = to_device(x)
    return t if dtype is None else t.to(dtype)


def bf16_dev_from_f32(a: np.ndarray):
    return dev(synth.Tensor(np.asarray(a, dtype=np.float32), "bf16"))


def host(t) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def rowwise_rel_err(got, want, axis=-1):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    num = np.abs(got - want).max(axis=axis)
    den = np.abs(want).max(axis=axis)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max())


def check_band(gpu_idx, ref_idx, ref_scores32, n_vis, K, band=BAND):
    """Selection parity rule for one query: equal set sizes and sentinel counts; the
    symmetric difference holds only entries whose float32 oracle score lies
    within `band` of the oracle's K-th score.  Returns the excused count."""
    g = sorted(int(v) for v in gpu_idx if v >= 0)
    r = sorted(int(v) for v in ref_idx if v >= 0)
    assert len(g) == len(r) == min(n_vis, K), (len(g), len(r), n_vis)
    assert int((np.asarray(gpu_idx) < 0).sum()) == int((np.asarray(ref_idx) < 0).sum())
    assert len(set(g)) == len(g), "duplicate index in a selection"
    assert all(0 <= v < n_vis for v in g), "selected entry not visible"
    diff = set(g) ^ set(r)
    if diff:
        kth = np.sort(ref_scores32[:n_vis].astype(np.float64))[-K]
        bad = [e for e in diff if abs(float(ref_scores32[e]) - kth) > band]
        assert not bad, f"entries {bad[:8]} outside the band around the K-th score {kth}"
    return len(diff)
