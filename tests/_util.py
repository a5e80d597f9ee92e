"""Helpers shared by the GPU parity tests (comparison and conversion only)."""
import numpy as np
import pytest
import torch


def f64(t):
    """Exact widening of a (bf16 / fp32) torch tensor to a float64 numpy array."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_l2(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-300))


def worst_rel_l2(x, ref, axis):
    """Worst relative L2 error over the slices of `axis` (e.g. per head)."""
    x = np.moveaxis(np.asarray(x), axis, 0)
    ref = np.moveaxis(np.asarray(ref), axis, 0)
    return max(rel_l2(a, b) for a, b in zip(x, ref))


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def announce(msg):
    print("[case] " + msg, flush=True)
