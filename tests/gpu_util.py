"""Helpers shared by the GPU parity tests (not collected by pytest)."""
import numpy as np
import torch


def np_(t):
    """Device tensor -> numpy (bf16 is widened to float32 exactly)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.numpy()


def rel_fro(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.linalg.norm(want)
    return float(np.linalg.norm(got - want) / (den if den > 0 else 1.0))


def assert_finite(*arrs):
    for a in arrs:
        a = np.asarray(a, dtype=np.float64)
        assert np.isfinite(a).all(), "NaN/Inf in a GPU output"


def say(*a):
    print("[case]", *a, flush=True)
