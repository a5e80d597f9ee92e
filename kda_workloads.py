"""Seeded synthetic inputs for the KDA hot path (shared by tests, smoke and bench).

This module holds no arithmetic of the method itself: it only draws random
tensors with the shapes and value distributions of the five workloads below and
returns them as CPU torch tensors.  Both the HIP path and the fp64 oracle are
fed from it.

Random stream: one torch CPU generator per workload, seeded, drawing in the
fixed order q, k, v, g_raw, beta_raw, state, slots, accepted lengths.

Distributions (per workload description):
  q, k, v ~ N(0, 1)                       (tiny fp32 case: q and k L2-normalised per head)
  g       = -0.1 * softplus(N(0, 1))      per key channel, fp32, always <= 0
  beta    = sigmoid(N(0, 1))              per (token, head), fp32
  state   ~ N(0, 0.05^2)                  fp32 pool slots (0.05 read as the standard deviation)
"""
import torch
import torch.nn.functional as F

# The five workloads: tiny recurrent fp32, decode over a state pool, speculative
# verify + replay commit, chunked prefill, long-context varlen prefill (one GPU's
# head share).
TINY = dict(name="tiny_fp32_T64_H2_d64", T=64, H=2, dk=64, dv=64)
DECODE = dict(name="decode_pool512_N64_H32_d128", num_slots=512, N=64, T=1, H=32, dk=128, dv=128)
VERIFY = dict(name="verify_replay_N32_T8_H32_d128", num_slots=512, N=32, T=8, H=32, dk=128, dv=128)
PREFILL = dict(name="prefill_T8192_H32_d128", T=8192, H=32, dk=128, dv=128)
VARLEN = dict(name="varlen_prefill_4seq_128076tok_H16_d128", seqlens=(100000, 16384, 8192, 3500),
              num_slots=512, H=16, dk=128, dv=128)


def _gen(seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _normal(gen, shape, std=1.0):
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    return x * std if std != 1.0 else x


def _gate(gen, shape):
    return -0.1 * F.softplus(_normal(gen, shape))


def _beta(gen, shape):
    return torch.sigmoid(_normal(gen, shape))


def _distinct_slots(gen, num_slots, n):
    return torch.randperm(num_slots, generator=gen)[:n].to(torch.int32)


def tiny(seed=0, T=None, H=None, dk=None, dv=None):
    """Tiny fp32 case: one sequence, zero initial state.

    Returns dict(q, k, v [T, H, d] fp32, g [T, H, dk], beta [T, H]).  q and k are
    L2-normalised per head with torch.nn.functional.normalize.
    """
    T = T or TINY["T"]; H = H or TINY["H"]; dk = dk or TINY["dk"]; dv = dv or TINY["dv"]
    gen = _gen(seed)
    q = F.normalize(_normal(gen, (T, H, dk)), dim=-1)
    k = F.normalize(_normal(gen, (T, H, dk)), dim=-1)
    v = _normal(gen, (T, H, dv))
    g = _gate(gen, (T, H, dk))
    beta = _beta(gen, (T, H))
    return dict(q=q, k=k, v=v, g=g, beta=beta)


def decode(seed=0, N=None, T=None, H=None, dk=None, dv=None, num_slots=None,
           dtype=torch.bfloat16, with_accepted=False):
    """Decode / MTP / verify over a state pool.

    Returns dict(q, k [N, T, H, dk] dtype, v [N, T, H, dv] dtype, g [N, T, H, dk] fp32,
    beta [N, T, H] fp32, pool [num_slots, H, dk, dv] fp32, slot_idx [N] int32 (distinct),
    and, with with_accepted, accepted [N] int32 uniform in 1..T).
    """
    N = N or DECODE["N"]; T = T or DECODE["T"]; H = H or DECODE["H"]
    dk = dk or DECODE["dk"]; dv = dv or DECODE["dv"]; num_slots = num_slots or DECODE["num_slots"]
    if N > num_slots:
        raise ValueError("need N <= num_slots for distinct slots")
    gen = _gen(seed)
    q = _normal(gen, (N, T, H, dk)).to(dtype)
    k = _normal(gen, (N, T, H, dk)).to(dtype)
    v = _normal(gen, (N, T, H, dv)).to(dtype)
    g = _gate(gen, (N, T, H, dk))
    beta = _beta(gen, (N, T, H))
    pool = _normal(gen, (num_slots, H, dk, dv), std=0.05)
    slot_idx = _distinct_slots(gen, num_slots, N)
    out = dict(q=q, k=k, v=v, g=g, beta=beta, pool=pool, slot_idx=slot_idx)
    if with_accepted:
        out["accepted"] = torch.randint(1, T + 1, (N,), generator=gen, dtype=torch.int32)
    return out


def verify(seed=0, **kw):
    """Speculative verify + replay: decode() at N=32, T=8 with accepted lengths."""
    args = dict(N=VERIFY["N"], T=VERIFY["T"], H=VERIFY["H"], dk=VERIFY["dk"], dv=VERIFY["dv"],
                num_slots=VERIFY["num_slots"], with_accepted=True)
    args.update(kw)
    return decode(seed, **args)


def prefill(seed=0, seqlens=(8192,), H=None, dk=None, dv=None, num_slots=None, h0_std=None,
            dtype=torch.bfloat16):
    """Varlen chunked prefill inputs.

    Returns dict(q, k [T_total, H, dk] dtype, v [T_total, H, dv] dtype, g [T_total, H, dk] fp32,
    beta [T_total, H] fp32, cu_seqlens [num_seqs + 1] int32, pool [num_slots, H, dk, dv] fp32,
    slot_idx [num_seqs] int32 distinct).  With h0_std None the pool is zero (zero initial
    state); otherwise it is drawn ~ N(0, h0_std^2).
    """
    H = H or PREFILL["H"]; dk = dk or PREFILL["dk"]; dv = dv or PREFILL["dv"]
    seqlens = tuple(int(s) for s in seqlens)
    ns = len(seqlens)
    num_slots = num_slots or ns
    T = sum(seqlens)
    gen = _gen(seed)
    q = _normal(gen, (T, H, dk)).to(dtype)
    k = _normal(gen, (T, H, dk)).to(dtype)
    v = _normal(gen, (T, H, dv)).to(dtype)
    g = _gate(gen, (T, H, dk))
    beta = _beta(gen, (T, H))
    if h0_std is None:
        pool = torch.zeros(num_slots, H, dk, dv, dtype=torch.float32)
    else:
        pool = _normal(gen, (num_slots, H, dk, dv), std=h0_std)
    slot_idx = _distinct_slots(gen, num_slots, ns)
    cu = torch.zeros(ns + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(seqlens, dtype=torch.int64), 0).to(torch.int32)
    return dict(q=q, k=k, v=v, g=g, beta=beta, cu_seqlens=cu, pool=pool, slot_idx=slot_idx)


def front_params(seed, H, dk, dv, num_slots, width=4, dtype=torch.bfloat16):
    """Parameters and state of the input front (ShortConv, gate and beta processing).

    Returns dict(gate_scale [H] fp32 = 0.1 (the workloads' gate g = -0.1 softplus(N(0, 1))),
    conv_q, conv_k [H, dk, width] and conv_v [H, dv, width] fp32 ~ N(0, 1 / width) (so a
    convolution of unit-variance inputs keeps unit variance), conv_state
    [num_slots, H, width - 1, 2 dk + dv] in dtype ~ N(0, 1) (the raw inputs' distribution)).
    """
    gen = _gen(seed)
    std = width ** -0.5
    return dict(gate_scale=torch.full((H,), 0.1, dtype=torch.float32),
                conv_q=_normal(gen, (H, dk, width), std=std), conv_k=_normal(gen, (H, dk, width), std=std),
                conv_v=_normal(gen, (H, dv, width), std=std),
                conv_state=_normal(gen, (num_slots, H, width - 1, 2 * dk + dv)).to(dtype))


def decode_front(seed=0, N=None, T=None, H=None, dk=None, dv=None, num_slots=None, width=4,
                 dtype=torch.bfloat16):
    """Decode inputs for the front: raw q, k, v ~ N(0, 1) (the convolution's inputs), raw gates
    z ~ N(0, 1) in g's place and raw beta values b ~ N(0, 1) (the draws the workloads pass
    through -0.1 softplus and sigmoid), the pool and slots as decode(), plus front_params()."""
    x = decode(seed, N=N, T=T, H=H, dk=dk, dv=dv, num_slots=num_slots, dtype=dtype)
    gen = _gen(seed + 1)
    N, T, H, dk = x["q"].shape
    x["g"] = _normal(gen, (N, T, H, dk))
    x["beta"] = _normal(gen, (N, T, H))
    x.update(front_params(seed + 2, H, dk, x["v"].shape[-1], x["pool"].shape[0], width, dtype))
    return x


def prefill_front(seed=0, seqlens=(8192,), H=None, dk=None, dv=None, num_slots=None, h0_std=None,
                  width=4, dtype=torch.bfloat16):
    """Prefill inputs for the front: prefill() with raw gates z ~ N(0, 1) in g's place and raw
    beta values b ~ N(0, 1) (the draws the workloads pass through -0.1 softplus and sigmoid),
    plus front_params() for the pool's slots."""
    x = prefill(seed, seqlens=seqlens, H=H, dk=dk, dv=dv, num_slots=num_slots, h0_std=h0_std, dtype=dtype)
    gen = _gen(seed + 1)
    T, H, dk = x["q"].shape
    x["g"] = _normal(gen, (T, H, dk))
    x["beta"] = _normal(gen, (T, H))
    x.update(front_params(seed + 2, H, dk, x["v"].shape[-1], x["pool"].shape[0], width, dtype))
    return x


def prefill_long(seed=0, **kw):
    """Long-context varlen prefill: 4 sequences (100000, 16384, 8192, 3500), H=16,
    initial states from 4 distinct slots of a 512-slot pool ~ N(0, 0.05^2)."""
    args = dict(seqlens=VARLEN["seqlens"], H=VARLEN["H"], dk=VARLEN["dk"], dv=VARLEN["dv"],
                num_slots=VARLEN["num_slots"], h0_std=0.05)
    args.update(kw)
    return prefill(seed, **args)



def cancellation(seed=0, seqlens=(64,), H=4, dk=128, dv=128, gate="channel", dtype=torch.bfloat16,
                 num_slots=None):
    """Prefill inputs whose q.k products cancel (for use without the L2 norm).

    Keys k ~ 0.25 N(0, 1).  Each query starts as 0.25 N(0, 1) and has its least-squares
    projection on the keys of its own sequence up to and including its own token removed, so
    q_t . k_s = 0 for s <= t before q and k are rounded to dtype (after rounding the products
    are small but not zero).  Sequences need at most dk tokens.  gate: 'channel' (per key
    channel, -0.1 softplus(N(0, 1)) as in the other workloads), 'scalar' (one such value per
    token and head, the same on every channel) or 'zero'.  v ~ N(0, 1), beta = sigmoid(N(0, 1)),
    zero pool (initial state).  Returns the dict of prefill().
    """
    seqlens = tuple(int(s) for s in seqlens)
    if max(seqlens) > dk:
        raise ValueError("cancellation needs sequences of at most dk tokens")
    ns = len(seqlens)
    T = sum(seqlens)
    gen = _gen(seed)
    k = (_normal(gen, (T, H, dk)) * 0.25).to(dtype).double()
    r = _normal(gen, (T, H, dk)).double() * 0.25
    q = torch.empty(T, H, dk, dtype=torch.float64)
    t0 = 0
    for L in seqlens:
        for t in range(L):
            for h in range(H):
                K = k[t0:t0 + t + 1, h]                                   # [t + 1, dk]
                coef = torch.linalg.lstsq(K.T, r[t0 + t, h].unsqueeze(1)).solution
                q[t0 + t, h] = r[t0 + t, h] - (K.T @ coef).squeeze(1)
        t0 += L
    v = _normal(gen, (T, H, dv)).to(dtype)
    if gate == "channel":
        g = _gate(gen, (T, H, dk))
    elif gate == "scalar":
        g = _gate(gen, (T, H, 1)).expand(T, H, dk).contiguous()
    elif gate == "zero":
        g = torch.zeros(T, H, dk)
    else:
        raise ValueError("gate must be 'channel', 'scalar' or 'zero'")
    beta = _beta(gen, (T, H))
    num_slots = num_slots or ns
    cu = torch.zeros(ns + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(seqlens, dtype=torch.int64), 0).to(torch.int32)
    return dict(q=q.to(dtype), k=k.to(dtype), v=v, g=g, beta=beta, cu_seqlens=cu,
                pool=torch.zeros(num_slots, H, dk, dv), slot_idx=_distinct_slots(gen, num_slots, ns))


# ---------------------------------------------------------------------------
# Random cases for the parity sweep: one seed gives one decode / MTP / verify case (even seeds) or
# one varlen prefill case (odd seeds), with random head shape, dtype, lengths, slot map, accepted
# lengths, gate strength (15% of the cases x20) and L2-norm switch.
_SWEEP_DIMS = ((64, 64), (64, 128), (128, 64), (128, 128))


def sweep_case(seed):
    """Returns dict(kind='decode'|'prefill', desc, and the inputs of that kind):
    decode: q, k, v [N, T, H, d], g, beta, pool, slot_idx (distinct; -1 = skipped), accepted,
            verify (bool), use_l2, dtype;
    prefill: q, k, v [T_total, H, d], g, beta, cu_seqlens, pool, slot_idx, h0_from_pool, use_l2,
             dtype."""
    gen = _gen(seed)
    pick = lambda n: int(torch.randint(n, (1,), generator=gen))
    uni = lambda: float(torch.rand(1, generator=gen))
    use_l2 = uni() < 0.8
    strong = uni() < 0.15
    sc = 1.0 if use_l2 else 0.25  # without the norm, smaller keys keep the state bounded
    if seed % 2 == 0:
        dk, dv = _SWEEP_DIMS[pick(4)]
        dtype = torch.float32 if uni() < 0.4 else torch.bfloat16
        N = 1 + pick(40)
        T = (1, 1, 2, 3, 5, 7, 8, 9, 12, 16, 20)[pick(11)]
        H = 1 + pick(8)
        num_slots = N + pick(20)
        lead = (N, T)
    else:
        dtype = torch.float32 if uni() < 0.3 else torch.bfloat16
        dk, dv = _SWEEP_DIMS[pick(4)] if dtype == torch.bfloat16 else (64, (64, 128)[pick(2)])
        ns = 1 + pick(6)
        choices = (0, 1, 2, 31, 63, 64, 65, 127, 128, 129, 200, 500, 1000, 1025)
        seqlens = [choices[pick(len(choices))] if uni() < 0.9 else 1 + pick(2000) for _ in range(ns)]
        H = 1 + pick(4)
        num_slots = ns + pick(8)
        lead = (sum(seqlens),)
    q = (_normal(gen, lead + (H, dk)) * sc).to(dtype)
    k = (_normal(gen, lead + (H, dk)) * sc).to(dtype)
    v = _normal(gen, lead + (H, dv)).to(dtype)
    g = _gate(gen, lead + (H, dk)) * (20.0 if strong else 1.0)
    beta = _beta(gen, lead + (H,))
    pool = _normal(gen, (num_slots, H, dk, dv), std=0.05)
    if seed % 2 == 0:
        slot_idx = _distinct_slots(gen, num_slots, N)
        slot_idx[torch.rand(N, generator=gen) < 0.1] = -1
        accepted = torch.randint(0, T + 1, (N,), generator=gen, dtype=torch.int32)
        verify = uni() < 0.5
        desc = "decode N%d T%d H%d dk%d dv%d %s l2=%d strong=%d verify=%d" % (
            N, T, H, dk, dv, str(dtype).split(".")[-1], use_l2, strong, verify)
        return dict(kind="decode", desc=desc, q=q, k=k, v=v, g=g, beta=beta, pool=pool,
                    slot_idx=slot_idx, accepted=accepted, verify=verify, use_l2=use_l2, dtype=dtype)
    slot_idx = _distinct_slots(gen, num_slots, ns)
    h0_from_pool = uni() < 0.6
    cu = torch.zeros(ns + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(seqlens, dtype=torch.int64), 0).to(torch.int32)
    desc = "prefill lens %s H%d dk%d dv%d %s l2=%d strong=%d h0pool=%d" % (
        seqlens, H, dk, dv, str(dtype).split(".")[-1], use_l2, strong, h0_from_pool)
    return dict(kind="prefill", desc=desc, q=q, k=k, v=v, g=g, beta=beta, cu_seqlens=cu, pool=pool,
                slot_idx=slot_idx, h0_from_pool=h0_from_pool, use_l2=use_l2, dtype=dtype)
