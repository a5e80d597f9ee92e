"""fp64 reference of the input front: ShortConv, gate and beta processing.

TEST INFRASTRUCTURE ONLY: tests, the smoke check and the CPU-baseline leg of the benchmark
may import this module; the product package never does.  It shares no code with the HIP
library.  Plain numpy in fp64 (inputs are widened, which is exact for bf16 and fp32).

What it computes.  The CANN Kimi K3 inference page (section 03, MegaKDA) names the steps
that sit in front of the recurrence -- the input projections, ShortConv, and the gate and
beta processing -- and says the fused operator takes them in, but gives no formula for any
of them.  The readings taken here (each the plainest one the pages and their workloads
support):
  * ShortConv: a causal depthwise convolution along the tokens of each sequence, channel by
    channel, over each of q, k and v with its own weights [H, channels, W], W in 1..4:
        y_t[c] = sum_{j=0}^{W-1} w[c, j] x_{t-(W-1)+j}[c],
    where the W-1 inputs before a sequence's first token come from its convolution state
    (zeros if it has none), optionally followed by SiLU, y * sigmoid(y).  The state after a
    sequence is its last W-1 inputs (earlier state rows where the sequence is shorter).
  * gate: the recurrence's log-decay is g = -a_h softplus(z) for a raw gate z and a scale
    a_h >= 0 per head.  The workloads draw g as -0.1 softplus(N(0, 1)), which is this with
    a_h = 0.1 and z ~ N(0, 1).
  * beta: beta = sigmoid(b) for a raw b; the workloads draw beta as sigmoid(N(0, 1)).
The input projections are not part of this reference (the pages give no weight shapes).

Layouts: the convolution state of a sequence is [H, W-1, 2 dk + dv], channels q | k | v,
row 0 the oldest input.
"""
import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def sigmoid(x):
    """1 / (1 + e^-x), evaluated without overflow on either side."""
    x = _f64(x)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def softplus(x):
    """log(1 + e^x) = max(x, 0) + log1p(e^-|x|)."""
    x = _f64(x)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def silu(x):
    x = _f64(x)
    return x * sigmoid(x)


def short_conv(x, w, cu_seqlens, state=None, use_silu=False):
    """Causal depthwise convolution of each sequence of x [T, H, C] with weights w [H, C, W].

    state: [num_seqs, H, W-1, C] inputs before each sequence's first token (None: zeros).
    Returns (y [T, H, C], the state after each sequence [num_seqs, H, W-1, C])."""
    x, w = _f64(x), _f64(w)
    T, H, C = x.shape
    W = w.shape[2]
    assert w.shape == (H, C, W) and 1 <= W
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    ns = cu.size - 1
    st = np.zeros((ns, H, W - 1, C)) if state is None else _f64(state)
    assert st.shape == (ns, H, W - 1, C)
    y = np.zeros((T, H, C))
    new_state = np.zeros((ns, H, W - 1, C))
    for s in range(ns):
        bos, eos = int(cu[s]), int(cu[s + 1])
        # the sequence's inputs with its W-1 earlier inputs in front, time first
        X = np.concatenate([st[s].transpose(1, 0, 2), x[bos:eos]], axis=0)  # [W-1+L, H, C]
        L = eos - bos
        for t in range(L):
            # X[t + j] is input t - (W-1) + j of the sequence
            acc = np.zeros((H, C))
            for j in range(W):
                acc += w[:, :, j] * X[t + j]
            y[bos + t] = acc
        new_state[s] = X[L:L + W - 1].transpose(1, 0, 2)
    if use_silu:
        y = silu(y)
    return y, new_state


def front(q_raw, k_raw, v_raw, z, b, cu_seqlens, gate_scale, conv_q, conv_k, conv_v,
          conv_state=None, use_silu=False):
    """The whole front: q, k, v convolved (and SiLU), g = -a_h softplus(z), beta = sigmoid(b).

    q_raw, k_raw [T, H, dk]; v_raw [T, H, dv]; z [T, H, dk]; b [T, H]; gate_scale [H];
    conv_q, conv_k [H, dk, W]; conv_v [H, dv, W]; conv_state [num_seqs, H, W-1, 2 dk + dv]
    or None.  Returns (q, k, v, g, beta, new_conv_state)."""
    q_raw, k_raw, v_raw = _f64(q_raw), _f64(k_raw), _f64(v_raw)
    dk, dv = q_raw.shape[2], v_raw.shape[2]
    parts = (None, None, None) if conv_state is None else (
        _f64(conv_state)[..., :dk], _f64(conv_state)[..., dk:2 * dk], _f64(conv_state)[..., 2 * dk:])
    q, sq = short_conv(q_raw, conv_q, cu_seqlens, parts[0], use_silu)
    k, sk = short_conv(k_raw, conv_k, cu_seqlens, parts[1], use_silu)
    v, sv = short_conv(v_raw, conv_v, cu_seqlens, parts[2], use_silu)
    g = -_f64(gate_scale)[None, :, None] * softplus(z)
    beta = sigmoid(b)
    return q, k, v, g, beta, np.concatenate([sq, sk, sv], axis=-1)
