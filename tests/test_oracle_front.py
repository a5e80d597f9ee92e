"""Pins of the front reference (oracle/kda_front.py): ShortConv, gate and beta processing,
checked against library routines (numpy's convolution, scipy's logistic function, torch's
softplus and sigmoid as the workloads use them), closed forms and invariants."""
import numpy as np
import pytest
import scipy.special
import torch

from oracle import kda_front as F


def test_logistic_and_softplus_against_libraries():
    x = np.concatenate([np.linspace(-40, 40, 801), [-745.0, -700.0, 0.0, 700.0, 745.0]])
    np.testing.assert_allclose(F.sigmoid(x), scipy.special.expit(x), rtol=1e-15, atol=1e-300)
    np.testing.assert_allclose(F.softplus(x), np.logaddexp(0.0, x), rtol=1e-15, atol=0)
    np.testing.assert_allclose(F.silu(x), x * scipy.special.expit(x), rtol=1e-15, atol=1e-300)
    assert F.sigmoid(0.0) == 0.5
    assert F.softplus(0.0) == np.log(2.0)
    # softplus(x) - softplus(-x) = x, sigmoid(x) + sigmoid(-x) = 1
    y = np.linspace(-30, 30, 61)
    np.testing.assert_allclose(F.softplus(y) - F.softplus(-y), y, rtol=0, atol=1e-13)
    np.testing.assert_allclose(F.sigmoid(y) + F.sigmoid(-y), 1.0, rtol=0, atol=1e-15)


def test_gate_and_beta_match_the_workload_recipe():
    """The workloads draw g = -0.1 softplus(N(0,1)) and beta = sigmoid(N(0,1)) with torch;
    the front with a_h = 0.1 on the same draws gives the same values."""
    gen = torch.Generator().manual_seed(3)
    z = torch.randn(40, 3, 16, generator=gen, dtype=torch.float64)
    b = torch.randn(40, 3, generator=gen, dtype=torch.float64)
    x = np.zeros((40, 3, 16))
    w = np.ones((3, 16, 1))
    _, _, _, g, beta, _ = F.front(x, x, x, z.numpy(), b.numpy(), [0, 40], np.full(3, 0.1), w, w, w)
    np.testing.assert_allclose(g, (-0.1 * torch.nn.functional.softplus(z)).numpy(), rtol=1e-14)
    np.testing.assert_allclose(beta, torch.sigmoid(b).numpy(), rtol=1e-14)


def test_hand_worked_conv():
    """One channel, W = 2, weights (10, 1), earlier input 5, inputs 1, 2, 3:
    y = 10*5 + 1, 10*1 + 2, 10*2 + 3 = 51, 12, 23; the state after is the last input, 3."""
    x = np.array([1.0, 2.0, 3.0]).reshape(3, 1, 1)
    w = np.array([10.0, 1.0]).reshape(1, 1, 2)
    y, st = F.short_conv(x, w, [0, 3], state=np.array([5.0]).reshape(1, 1, 1, 1))
    assert y.ravel().tolist() == [51.0, 12.0, 23.0]
    assert st.ravel().tolist() == [3.0]


def test_width_one_unit_weight_is_the_identity():
    gen = np.random.default_rng(0)
    x = gen.standard_normal((50, 2, 8))
    y, st = F.short_conv(x, np.ones((2, 8, 1)), [0, 20, 20, 50])
    assert np.array_equal(y, x)
    assert st.shape == (3, 2, 0, 8)


@pytest.mark.parametrize("W", [2, 3, 4])
def test_conv_matches_numpy_convolution(W):
    """Each sequence and channel against np.convolve over [earlier inputs; sequence]."""
    gen = np.random.default_rng(W)
    cu = [0, 1, 3, 30, 30, 47]
    T, H, C = 47, 2, 5
    x = gen.standard_normal((T, H, C))
    w = gen.standard_normal((H, C, W))
    st0 = gen.standard_normal((5, H, W - 1, C))
    y, st = F.short_conv(x, w, cu, st0)
    for s in range(5):
        bos, eos = cu[s], cu[s + 1]
        for h in range(H):
            for c in range(C):
                X = np.concatenate([st0[s, h, :, c], x[bos:eos, h, c]])
                if eos > bos:  # (np.convolve swaps its operands when the first is shorter)
                    ref = np.convolve(X, w[h, c, ::-1], mode="valid")
                    np.testing.assert_allclose(y[bos:eos, h, c], ref, rtol=1e-13, atol=1e-13)
                np.testing.assert_array_equal(st[s, h, :, c], X[len(X) - (W - 1):])


@pytest.mark.parametrize("j", [0, 1, 2, 3])
def test_single_tap_shifts_the_sequence(j):
    """A weight with one nonzero tap j (W = 4) delays the input by 3 - j tokens, the earlier
    inputs coming from the state."""
    gen = np.random.default_rng(10 + j)
    L, d = 9, 3 - j
    x = gen.standard_normal((L, 1, 3))
    st0 = gen.standard_normal((1, 1, 3, 3))
    w = np.zeros((1, 3, 4))
    w[:, :, j] = 1.0
    y, _ = F.short_conv(x, w, [0, L], st0)
    for t in range(L):
        want = x[t - d, 0] if t - d >= 0 else st0[0, 0, 3 + t - d]
        np.testing.assert_array_equal(y[t, 0], want)


@pytest.mark.parametrize("split", [0, 1, 2, 5, 11, 12])
def test_splitting_a_sequence_carries_the_state(split):
    """A sequence convolved in two calls, the state of the first passed to the second, equals
    one call (including a first part shorter than W - 1)."""
    gen = np.random.default_rng(split)
    L, H, C, W = 12, 2, 4, 4
    x = gen.standard_normal((L, H, C))
    w = gen.standard_normal((H, C, W))
    st0 = gen.standard_normal((1, H, W - 1, C))
    y, st = F.short_conv(x, w, [0, L], st0, use_silu=True)
    y1, st1 = F.short_conv(x[:split], w, [0, split], st0, use_silu=True)
    y2, st2 = F.short_conv(x[split:], w, [0, L - split], st1, use_silu=True)
    np.testing.assert_allclose(np.concatenate([y1, y2]), y, rtol=1e-14, atol=1e-14)
    np.testing.assert_array_equal(st2, st)


def test_front_state_layout_is_q_k_v():
    """The front's state holds q, k and v channels in that order (dk, dk, dv)."""
    gen = np.random.default_rng(5)
    T, H, dk, dv, W = 6, 1, 2, 3, 3
    q, k, v = (gen.standard_normal((T, H, n)) for n in (dk, dk, dv))
    wq, wk, wv = (gen.standard_normal((H, n, W)) for n in (dk, dk, dv))
    st0 = gen.standard_normal((1, H, W - 1, 2 * dk + dv))
    out = F.front(q, k, v, np.zeros((T, H, dk)), np.zeros((T, H)), [0, T], np.ones(H), wq, wk, wv, st0)
    for x, w, lo, hi, got in ((q, wq, 0, dk, out[0]), (k, wk, dk, 2 * dk, out[1]), (v, wv, 2 * dk, 2 * dk + dv, out[2])):
        y, s = F.short_conv(x, w, [0, T], st0[..., lo:hi])
        np.testing.assert_array_equal(got, y)
        np.testing.assert_array_equal(out[5][..., lo:hi], s)
