"""Pins of the fp64 backward oracle (oracle/kda_backward.py), CPU only.

1. Every gradient (q, k, v, g, beta, h0) against central finite differences of the C forward
   oracle (oracle/kda_oracle.c, a separate implementation) on a two-sequence varlen case with
   random initial states and a final-state cotangent, with and without the L2 norm.
2. Closed form: with beta = 0 and g = 0 the state never changes (S_t = h0), so o_t =
   scale h0^T q_t (no norm) is a linear readout: dq_t = scale h0 do_t, dh0 = dht + scale
   sum_t q_t do_t^T, and dv = dk = 0.
"""
import numpy as np
import pytest

from oracle import kda_oracle as O
from oracle.kda_backward import recurrent_backward

pytestmark = pytest.mark.filterwarnings("ignore")


def _case(seed, T_lens=(3, 4), H=2, dk=3, dv=2):
    r = np.random.default_rng(seed)
    T = sum(T_lens)
    cu = np.concatenate([[0], np.cumsum(T_lens)]).astype(np.int64)
    x = dict(q=r.normal(size=(T, H, dk)), k=r.normal(size=(T, H, dk)), v=r.normal(size=(T, H, dv)),
             g=-0.3 * np.log1p(np.exp(r.normal(size=(T, H, dk)))),
             beta=1.0 / (1.0 + np.exp(-r.normal(size=(T, H)))),
             h0=0.5 * r.normal(size=(len(T_lens), H, dk, dv)))
    do = r.normal(size=(T, H, dv))
    dht = r.normal(size=(len(T_lens), H, dk, dv))
    return x, cu, do, dht


def _loss(x, cu, do, dht, l2):
    o, ht, _ = O.recurrent(x["q"], x["k"], x["v"], x["g"], x["beta"], cu, h0=x["h0"],
                           use_qk_l2norm=l2, nthreads=1)
    return float((do * o).sum() + (dht * ht).sum())


@pytest.mark.parametrize("l2", [True, False])
def test_gradients_match_central_differences_of_the_forward_oracle(l2):
    x, cu, do, dht = _case(3)
    dq, dk, dv, dg, dbeta, dh0 = recurrent_backward(x["q"], x["k"], x["v"], x["g"], x["beta"], cu,
                                                    do, dht=dht, h0=x["h0"], use_qk_l2norm=l2)
    grads = dict(q=dq, k=dk, v=dv, g=dg, beta=dbeta, h0=dh0)
    eps = 1e-6
    for name, grad in grads.items():
        num = np.zeros_like(grad)
        base = x[name]
        for idx in np.ndindex(base.shape):
            keep = base[idx]
            base[idx] = keep + eps
            lp = _loss(x, cu, do, dht, l2)
            base[idx] = keep - eps
            lm = _loss(x, cu, do, dht, l2)
            base[idx] = keep
            num[idx] = (lp - lm) / (2 * eps)
        err = np.abs(num - grad).max()
        assert err <= 1e-6 * max(1.0, np.abs(num).max()), (name, err)


def test_constant_state_readout_closed_form():
    x, cu, do, dht = _case(5)
    x["beta"][:] = 0.0
    x["g"][:] = 0.0
    scale = x["q"].shape[-1] ** -0.5
    dq, dk, dv, dg, dbeta, dh0 = recurrent_backward(x["q"], x["k"], x["v"], x["g"], x["beta"], cu,
                                                    do, dht=dht, h0=x["h0"], use_qk_l2norm=False)
    for n in range(len(cu) - 1):
        b, e = cu[n], cu[n + 1]
        for h in range(x["q"].shape[1]):
            H0 = x["h0"][n, h]
            for t in range(b, e):
                assert np.allclose(dq[t, h], scale * H0 @ do[t, h], rtol=0, atol=1e-12)
            want = dht[n, h] + scale * sum(np.outer(x["q"][t, h], do[t, h]) for t in range(b, e))
            assert np.allclose(dh0[n, h], want, rtol=0, atol=1e-12)
    assert np.all(dv == 0) and np.allclose(dk, 0, atol=1e-15)


def test_c_backward_equals_the_numpy_backward():
    """The C backward (kda_oracle.c: forward kept every 64 tokens, spans recomputed) and the
    numpy backward are two implementations of the same reverse recurrence: equal to 1e-12
    over sequences that cross several 64-token spans, with and without the norm, h0 and dht."""
    r = np.random.default_rng(7)
    lens = (1, 64, 65, 130, 0, 7)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T, H, dk, dv = int(cu[-1]), 2, 5, 4
    for l2, with_state in ((True, True), (False, True), (True, False)):
        x = dict(q=r.normal(size=(T, H, dk)), k=r.normal(size=(T, H, dk)) * (1 if l2 else 0.4),
                 v=r.normal(size=(T, H, dv)), g=-0.2 * np.log1p(np.exp(r.normal(size=(T, H, dk)))),
                 beta=1.0 / (1.0 + np.exp(-r.normal(size=(T, H)))))
        h0 = 0.3 * r.normal(size=(len(lens), H, dk, dv)) if with_state else None
        dht = r.normal(size=(len(lens), H, dk, dv)) if with_state else None
        do = r.normal(size=(T, H, dv))
        a = O.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], cu, do, dht=dht, h0=h0,
                       use_qk_l2norm=l2, nthreads=3)
        b = recurrent_backward(x["q"], x["k"], x["v"], x["g"], x["beta"], cu, do, dht=dht, h0=h0,
                               use_qk_l2norm=l2)
        for name, ga, gb in zip(("dq", "dk", "dv", "dg", "dbeta", "dh0"), a, b):
            assert np.abs(ga - gb).max() <= 1e-12 * max(1.0, np.abs(gb).max()), (name, l2)


def test_c_backward_matches_central_differences_across_spans():
    """The C backward against central finite differences of the C forward oracle on a sequence
    of 70 tokens (two 64-token spans of the recomputation) plus a 3-token one."""
    x, cu, do, dht = _case(11, T_lens=(70, 3), H=1, dk=3, dv=2)
    dq, dk, dv, dg, dbeta, dh0 = O.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], cu, do,
                                            dht=dht, h0=x["h0"], nthreads=1)
    grads = dict(q=dq, k=dk, v=dv, g=dg, beta=dbeta, h0=dh0)
    eps = 1e-6
    for name, grad in grads.items():
        base = x[name]
        for idx in list(np.ndindex(base.shape))[::7]:
            keep = base[idx]
            base[idx] = keep + eps
            lp = _loss(x, cu, do, dht, True)
            base[idx] = keep - eps
            lm = _loss(x, cu, do, dht, True)
            base[idx] = keep
            num = (lp - lm) / (2 * eps)
            assert abs(num - grad[idx]) <= 1e-6 * max(1.0, abs(num)), (name, idx, num, grad[idx])
