"""fp64 backward of the KDA recurrence (plain numpy, token by token).

TEST INFRASTRUCTURE ONLY, like the rest of oracle/: tests may import it; the product package
never does, and it shares no code with the HIP library.

What it differentiates: the forward recurrence of the KDA section of the Kimi K3 day-0
adaptation page (per sequence and head, S is dk x dv; L2 norm of q and k, alpha = exp(g) per key
channel, decay, delta rule, rank-1 update, output read from the updated state), restated:

    qh = q / sqrt(|q|^2 + eps), kh likewise          (when use_qk_l2norm)
    S'_t = diag(alpha_t) S_{t-1},  p_t = S'_t^T kh_t
    u_t  = beta_t (v_t - p_t),     S_t = S'_t + kh_t u_t^T
    o_t  = scale S_t^T qh_t

The same page's training section (the item on the linear-attention kernels built with
Triton-Ascend) names forward and backward kernels for training but prints no backward formula.
The gradients below are the chain rule through those steps in reverse token order, with
D = dL/dS_t carried backwards:

    dqh_t = scale S_t do_t ;  D += scale qh_t do_t^T
    du_t = D^T kh_t ;  dkh_t = D u_t
    dbeta_t = du_t . (v_t - p_t) ;  dv_t = beta_t du_t ;  dp_t = -beta_t du_t
    D' = D + kh_t dp_t^T ;  dkh_t += S'_t dp_t
    dalpha_t = rowsum(D' * S_{t-1}) ;  dg_t = alpha_t * dalpha_t ;  D <- diag(alpha_t) D'
    dq_t = (dqh_t - qh_t (qh_t . dqh_t)) / sqrt(|q_t|^2 + eps)   (k likewise; identity without
                                                                  the norm)
    dh0 = D after the first token.

The forward states are recomputed here and kept, one per token (fine at test sizes).  Pinned by
central finite differences of the C forward oracle (oracle/kda_oracle.c, a separate
implementation) and by closed forms (tests/test_oracle_backward.py).
"""
import numpy as np

EPS = 1e-6


def recurrent_backward(q, k, v, g, beta, cu_seqlens, do, dht=None, h0=None, scale=None,
                       use_qk_l2norm=True, eps=EPS):
    """Gradients of L = sum(do * o) + sum(dht * ht) for the varlen recurrence.

    q, k, g [T, H, dk]; v, do [T, H, dv]; beta [T, H]; cu_seqlens [num_seqs + 1];
    h0, dht [num_seqs, H, dk, dv] or None (zero).  Returns (dq, dk, dv, dg, dbeta, dh0)."""
    f = lambda x: np.asarray(x, dtype=np.float64)
    q, k, v, g, beta, do = f(q), f(k), f(v), f(g), f(beta), f(do)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T, H, dk = q.shape
    dv_ = v.shape[-1]
    ns = cu.shape[0] - 1
    if scale is None:
        scale = dk ** -0.5
    dq, dk_, dvv, dg = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v), np.zeros_like(g)
    dbeta = np.zeros_like(beta)
    dh0 = np.zeros((ns, H, dk, dv_))
    for n in range(ns):
        bos, eos = int(cu[n]), int(cu[n + 1])
        for h in range(H):
            S = f(h0[n, h]).copy() if h0 is not None else np.zeros((dk, dv_))
            steps = []
            for t in range(bos, eos):
                nq = np.sqrt(q[t, h] @ q[t, h] + eps) if use_qk_l2norm else 1.0
                nk = np.sqrt(k[t, h] @ k[t, h] + eps) if use_qk_l2norm else 1.0
                qh, kh = q[t, h] / nq, k[t, h] / nk
                a = np.exp(g[t, h])
                Sp = a[:, None] * S
                p = Sp.T @ kh
                u = beta[t, h] * (v[t, h] - p)
                Sn = Sp + np.outer(kh, u)
                steps.append((t, S, Sp, Sn, qh, kh, nq, nk, a, p, u))
                S = Sn
            D = f(dht[n, h]).copy() if dht is not None else np.zeros((dk, dv_))
            for t, Sprev, Sp, Sn, qh, kh, nq, nk, a, p, u in reversed(steps):
                dqh = scale * (Sn @ do[t, h])
                D = D + scale * np.outer(qh, do[t, h])
                du = D.T @ kh
                dkh = D @ u
                dbeta[t, h] = du @ (v[t, h] - p)
                dvv[t, h] = beta[t, h] * du
                dp = -beta[t, h] * du
                Dp = D + np.outer(kh, dp)
                dkh = dkh + Sp @ dp
                dg[t, h] = a * (Dp * Sprev).sum(axis=1)
                D = a[:, None] * Dp
                if use_qk_l2norm:
                    dq[t, h] = (dqh - qh * (qh @ dqh)) / nq
                    dk_[t, h] = (dkh - kh * (kh @ dkh)) / nk
                else:
                    dq[t, h] = dqh
                    dk_[t, h] = dkh
            dh0[n, h] = D
    return dq, dk_, dvv, dg, dbeta, dh0
