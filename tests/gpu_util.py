"""Helpers for the GPU parity tests: device copies and the tolerance check."""
import numpy as np


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.cpu().numpy()


def check_tol(got, ref, abs_terms, rel=1e-4, what=""):
    """|got - ref| <= rel * sum|terms| elementwise (the stated fp32 tolerance)."""
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref)
    bound = rel * np.asarray(abs_terms, np.float64)
    bad = err > bound
    assert np.isfinite(got).all(), f"{what}: non-finite outputs"
    if bad.any():
        i = np.unravel_index(np.argmax(err / np.maximum(bound, 1e-300)), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} outputs outside tolerance; worst at {i}: got {got[i]} "
                             f"ref {ref[i]} bound {bound[i]}")
    return float((err / np.maximum(bound, 1e-300)).max())
