"""Helpers shared by the tests (no arithmetic of the method here)."""
import concurrent.futures
import os

import numpy as np
import torch


def pmap(fn, items, workers=None):
    """[fn(x) for x in items] on a thread pool (numpy releases the GIL in its array
    loops and BLAS calls), at most 16 threads: the oracle's full-size checks run
    expert by expert or row block by row block side by side."""
    items = list(items)
    n = workers or min(16, len(os.sched_getaffinity(0)), max(len(items), 1))
    with concurrent.futures.ThreadPoolExecutor(n) as ex:
        return list(ex.map(fn, items))


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


def codes_close(q, q_ref, s, s_ref, rtol, min_equal=0.999, max_step=1, what=""):
    """The several-correct-answers bar for e4m3 codes computed from values that
    carry rounding differences: scales within rtol, at least min_equal of the
    codes identical, and every other code with the same sign (or one side zero)
    and at most max_step steps away in the code order (max_step None: not
    checked, for inputs that differ by more than rounding)."""
    q = np.asarray(q); q_ref = np.asarray(q_ref)
    assert q.shape == q_ref.shape, (q.shape, q_ref.shape)
    np.testing.assert_allclose(s, s_ref, rtol=rtol, atol=0, err_msg=what)
    same = q == q_ref
    assert same.mean() >= min_equal, f"{what}: only {same.mean():.5f} of the codes equal"
    mism = ~same
    if mism.any():
        a, b = q[mism].astype(int), q_ref[mism].astype(int)
        # across zero: a zero code on either side, or both codes within the e4m3 subnormal
        # range (|value| < 2^-6 of the scale's 448), where the matrix core's block sums
        # (accurate to ~1e-4 of the sum of |products|) can move a value across zero
        zero = ((a & 0x7F) == 0) | ((b & 0x7F) == 0) | (((a & 0x7F) < 8) & ((b & 0x7F) < 8))
        flip = ~(((a & 0x80) == (b & 0x80)) | zero)
        assert not flip.any(), (f"{what}: {int(flip.sum())} sign flips of {q.size} codes, e.g. "
                                f"{list(zip(a[flip][:8].tolist(), b[flip][:8].tolist()))}")
        if max_step is not None:
            assert np.all(np.abs((a & 0x7F) - (b & 0x7F)) <= max_step), f"{what}: codes more than {max_step} step apart"
