"""Helpers shared by the tests (no arithmetic of the method here)."""
import numpy as np
import torch


def tol_check(y, y_ref, rel=1e-2, what=""):
    """|y - y_ref| <= rel · (|y_ref| + rms(y_ref)), rms over all compared outputs.
    Returns the worst ratio |y - y_ref| / bound."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    assert y.shape == y_ref.shape, (y.shape, y_ref.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite outputs"
    rms = float(np.sqrt(np.mean(y_ref ** 2))) if y_ref.size else 0.0
    bound = rel * (np.abs(y_ref) + rms)
    err = np.abs(y - y_ref)
    worst = float(np.max(err / np.maximum(bound, 1e-300))) if y.size else 0.0
    bad = np.count_nonzero(err > bound)
    assert bad == 0, f"{what}: {bad} of {y.size} outputs outside tolerance (worst ratio {worst:.3g})"
    return worst


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.numpy()


def cuda(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()
