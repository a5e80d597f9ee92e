"""ctypes front end of the fp64 CPU oracle (oracle/kda_oracle.c).

TEST INFRASTRUCTURE ONLY: tests, the smoke check and the CPU-baseline leg of the
benchmark may import this module; the product package never does.  It shares no
code with the HIP library.  Every function takes numpy arrays (any float dtype;
they are widened to fp64, which is exact for bf16 and fp32 values) and returns
fp64 numpy arrays.

The arithmetic lives in kda_oracle.c; see its header for the formula and the
page sections it follows.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None
_DP = ctypes.POINTER(ctypes.c_double)
_I64P = ctypes.POINTER(ctypes.c_int64)

EPS = 1e-6  # L2-norm epsilon inside the square root (the pages give none)


def _lib():
    global _LIB
    if _LIB is None:
        # KDA_ORACLE_LIB selects another build of the same source (the sanitizer build)
        path = os.environ.get("KDA_ORACLE_LIB") or _build.LIB
        if not os.path.exists(path):
            _build.build(force=True)
        lib = ctypes.CDLL(path)
        lib.kda_oracle_recurrent.restype = ctypes.c_int
        lib.kda_oracle_recurrent.argtypes = [_DP] * 5 + [_I64P] + [ctypes.c_int] * 4 + [
            ctypes.c_double, ctypes.c_int, ctypes.c_double, _DP, _DP, _DP, _DP, ctypes.c_int]
        lib.kda_oracle_chunked.restype = ctypes.c_int
        lib.kda_oracle_chunked.argtypes = [_DP] * 5 + [_I64P] + [ctypes.c_int] * 4 + [
            ctypes.c_double, ctypes.c_int, ctypes.c_double, _DP, _DP, _DP, ctypes.c_int,
            ctypes.c_int]
        lib.kda_oracle_backward.restype = ctypes.c_int
        lib.kda_oracle_backward.argtypes = [_DP] * 5 + [_I64P] + [ctypes.c_int] * 4 + [
            ctypes.c_double, ctypes.c_int, ctypes.c_double] + [_DP] * 9 + [ctypes.c_int]
        lib.kda_oracle_replay.restype = ctypes.c_int
        lib.kda_oracle_replay.argtypes = [_DP, _DP, _I64P] + [ctypes.c_int] * 5
        _LIB = lib
    return _LIB


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(_DP)


def default_threads():
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _prep(q, k, v, g, beta, cu_seqlens, h0):
    q, k, v, g, beta = (_f64(a) for a in (q, k, v, g, beta))
    if q.ndim != 3 or k.shape != q.shape or g.shape != q.shape:
        raise ValueError("q, k, g must share shape [T_total, H, dk]")
    T, H, dk = q.shape
    if v.ndim != 3 or v.shape[:2] != (T, H):
        raise ValueError("v must be [T_total, H, dv]")
    if beta.shape != (T, H):
        raise ValueError("beta must be [T_total, H]")
    dv = v.shape[2]
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    if cu.ndim != 1 or cu.size < 1 or cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at T_total")
    ns = cu.size - 1
    if h0 is not None:
        h0 = _f64(h0)
        if h0.shape != (ns, H, dk, dv):
            raise ValueError("h0 must be [num_seqs, H, dk, dv]")
    return q, k, v, g, beta, cu, h0, T, H, dk, dv, ns


def recurrent(q, k, v, g, beta, cu_seqlens, h0=None, scale=None, use_qk_l2norm=True,
              eps=EPS, want_records=False, nthreads=None):
    """Token-by-token fp64 recurrence.  Returns (o, ht, records or None)."""
    q, k, v, g, beta, cu, h0, T, H, dk, dv, ns = _prep(q, k, v, g, beta, cu_seqlens, h0)
    if scale is None:
        scale = dk ** -0.5
    o = np.zeros((T, H, dv))
    ht = np.zeros((ns, H, dk, dv))
    rec = np.zeros((T, H, 2 * dk + dv)) if want_records else None
    st = _lib().kda_oracle_recurrent(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), cu.ctypes.data_as(_I64P), ns, H, dk,
        dv, float(scale), int(bool(use_qk_l2norm)), float(eps), _ptr(h0), _ptr(o), _ptr(ht),
        _ptr(rec), int(nthreads or default_threads()))
    if st != 0:
        raise RuntimeError("kda_oracle_recurrent failed with status %d" % st)
    return o, ht, rec


def chunked(q, k, v, g, beta, cu_seqlens, h0=None, scale=None, use_qk_l2norm=True, eps=EPS,
            chunk=64, nthreads=None):
    """fp64 chunk form (inclusive gate cumsum, UT forward substitution).  Returns (o, ht)."""
    q, k, v, g, beta, cu, h0, T, H, dk, dv, ns = _prep(q, k, v, g, beta, cu_seqlens, h0)
    if scale is None:
        scale = dk ** -0.5
    o = np.zeros((T, H, dv))
    ht = np.zeros((ns, H, dk, dv))
    st = _lib().kda_oracle_chunked(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), cu.ctypes.data_as(_I64P), ns, H, dk,
        dv, float(scale), int(bool(use_qk_l2norm)), float(eps), _ptr(h0), _ptr(o), _ptr(ht),
        int(chunk), int(nthreads or default_threads()))
    if st != 0:
        raise RuntimeError("kda_oracle_chunked failed with status %d" % st)
    return o, ht


def backward(q, k, v, g, beta, cu_seqlens, do, dht=None, h0=None, scale=None, use_qk_l2norm=True,
             eps=EPS, nthreads=None):
    """fp64 gradients of sum(do * o) + sum(dht * ht) of the token recurrence (kda_oracle.c,
    run_chain_backward).  Returns (dq, dk, dv, dg, dbeta, dh0)."""
    q, k, v, g, beta, cu, h0, T, H, dk, dv, ns = _prep(q, k, v, g, beta, cu_seqlens, h0)
    do = _f64(do)
    if do.shape != (T, H, dv):
        raise ValueError("do must be [T_total, H, dv]")
    if dht is not None:
        dht = _f64(dht)
        if dht.shape != (ns, H, dk, dv):
            raise ValueError("dht must be [num_seqs, H, dk, dv]")
    if scale is None:
        scale = dk ** -0.5
    dq, dk_, dg = np.zeros((T, H, dk)), np.zeros((T, H, dk)), np.zeros((T, H, dk))
    dvv, dbeta = np.zeros((T, H, dv)), np.zeros((T, H))
    dh0 = np.zeros((ns, H, dk, dv))
    st = _lib().kda_oracle_backward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), cu.ctypes.data_as(_I64P), ns, H, dk, dv,
        float(scale), int(bool(use_qk_l2norm)), float(eps), _ptr(h0), _ptr(do), _ptr(dht),
        _ptr(dq), _ptr(dk_), _ptr(dvv), _ptr(dg), _ptr(dbeta), _ptr(dh0),
        int(nthreads or default_threads()))
    if st != 0:
        raise RuntimeError("kda_oracle_backward failed with status %d" % st)
    return dq, dk_, dvv, dg, dbeta, dh0


def replay(state, records, accepted):
    """ReplaySSM commit: applies records[n, :accepted[n]] to state[n] ([N, H, dk, dv]).

    records is [N, T, H, 2*dk + dv] = {kh | alpha | u}.  Returns the new state.
    """
    S = _f64(state).copy()
    R = _f64(records)
    acc = np.ascontiguousarray(np.asarray(accepted, dtype=np.int64))
    N, H, dk, dv = S.shape
    if R.ndim != 4 or R.shape[0] != N or R.shape[2] != H or R.shape[3] != 2 * dk + dv:
        raise ValueError("records must be [N, T, H, 2*dk + dv]")
    T = R.shape[1]
    if acc.shape != (N,):
        raise ValueError("accepted must be [N]")
    st = _lib().kda_oracle_replay(_ptr(S), _ptr(R), acc.ctypes.data_as(_I64P), N, T, H, dk, dv)
    if st != 0:
        raise RuntimeError("kda_oracle_replay failed with status %d" % st)
    return S


def decode(q, k, v, g, beta, h0, scale=None, use_qk_l2norm=True, eps=EPS, want_records=False,
           nthreads=None):
    """Decode/MTP form: q, k, g [N, T, H, dk], v [N, T, H, dv], beta [N, T, H], h0 [N, H, dk, dv].

    Same memory as the varlen form with cu_seqlens = {0, T, 2T, ...}.
    Returns (o [N, T, H, dv], ht [N, H, dk, dv], records [N, T, H, 2dk+dv] or None).
    """
    q = _f64(q)
    N, T, H, dk = q.shape
    dv = np.asarray(v).shape[-1]
    cu = np.arange(N + 1, dtype=np.int64) * T
    o, ht, rec = recurrent(q.reshape(N * T, H, dk), _f64(k).reshape(N * T, H, dk),
                           _f64(v).reshape(N * T, H, dv), _f64(g).reshape(N * T, H, dk),
                           _f64(beta).reshape(N * T, H), cu, h0=h0, scale=scale,
                           use_qk_l2norm=use_qk_l2norm, eps=eps, want_records=want_records,
                           nthreads=nthreads)
    o = o.reshape(N, T, H, dv)
    if rec is not None:
        rec = rec.reshape(N, T, H, 2 * dk + dv)
    return o, ht, rec
