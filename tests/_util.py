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


def _segment_rel(x, ref, starts):
    """Relative L2 error of each (token segment, head) of [T, H, ...] arrays; segments begin at
    `starts` (sorted, first 0) and run to the next start or T."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    T, H = x.shape[:2]
    e2 = ((x - ref) ** 2).reshape(T, H, -1).sum(-1)
    r2 = (ref ** 2).reshape(T, H, -1).sum(-1)
    starts = np.asarray(starts, dtype=np.int64)
    se, sr = np.add.reduceat(e2, starts, axis=0), np.add.reduceat(r2, starts, axis=0)
    return np.sqrt(se) / np.maximum(np.sqrt(sr), 1e-300)


def _nonempty_starts(cu, step=None):
    cu = [int(c) for c in cu]
    starts = []
    for a, b in zip(cu[:-1], cu[1:]):
        if b > a:
            starts.extend(range(a, b, step) if step else [a])
    return starts


def worst_seq_head(x, ref, cu):
    """Worst relative L2 error over the (sequence, head) slices of [T_total, H, ...] arrays
    (sequences given by cu_seqlens; empty ones skipped)."""
    starts = _nonempty_starts(cu)
    return float(_segment_rel(x, ref, starts).max()) if starts else 0.0


def worst_chunk_head(x, ref, cu, chunk=64):
    """Worst relative L2 error over the (64-token chunk, head) slices of [T_total, H, ...]
    arrays; chunks restart at every sequence start."""
    starts = _nonempty_starts(cu, chunk)
    return float(_segment_rel(x, ref, starts).max()) if starts else 0.0


def worst_state(x, ref):
    """Worst relative L2 error over the (sequence, head) states of [N, H, dk, dv] arrays."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if x.size == 0:
        return 0.0
    e = np.sqrt(((x - ref) ** 2).sum(axis=(-2, -1)))
    r = np.maximum(np.sqrt((ref ** 2).sum(axis=(-2, -1))), 1e-300)
    return float((e / r).max())


def worst_decode(x, ref):
    """Worst relative L2 error over the (sequence, head) slices of [N, T, H, dv] arrays."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if x.size == 0:
        return 0.0
    e = np.sqrt(((x - ref) ** 2).sum(axis=(1, 3)))
    r = np.maximum(np.sqrt((ref ** 2).sum(axis=(1, 3))), 1e-300)
    return float((e / r).max())


def check_prefill_parity(o, o_ref, h, h_ref, cu, tol, label=""):
    """Whole-tensor and worst per-(sequence, head) relative L2 of o and the final states."""
    e = dict(o=rel_l2(o, o_ref), o_worst=worst_seq_head(o, o_ref, cu), h=rel_l2(h, h_ref),
             h_worst=worst_state(h, h_ref))
    announce("%s rel-L2 o %.3g (worst seq/head %.3g), state %.3g (worst %.3g)"
             % (label, e["o"], e["o_worst"], e["h"], e["h_worst"]))
    for name, val in e.items():
        assert val <= tol, (name, val, tol)
    return e
