"""GPU parity of the decode / MTP / verify kernel and the ReplaySSM commit kernel
against the fp64 oracle, through the C ABI (python binding -> libkda.so).

Tolerances (relative L2 over the whole tensor): 1e-4 for fp32 q/k/v, 1e-2 for bf16
q/k/v with an fp32 state.  Slot mapping, untouched slots and the bf16 output
rounding are checked bit for bit.
"""
import numpy as np
import pytest
import torch

import kda_gated_delta_rule_amd as kda
import kda_workloads as W
from oracle import kda_oracle as O
from tests._util import announce, f64, need_gpu, rel_l2, worst_decode, worst_rel_l2, worst_state

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "g", "beta")


def run_decode(x, dev, records=False, **kw):
    pool = x["pool"].to(dev)
    args = [x[n].to(dev) for n in NAMES]
    rec = None
    if records:
        N, T, H, dk = x["q"].shape
        dv = x["v"].shape[-1]
        rec = torch.full((N, T, H, 2 * dk + dv), float("nan"), device=dev)
    o = kda.decode_step(*args, pool, x["slot_idx"].to(dev), records=rec, **kw)
    torch.cuda.synchronize()
    return o, pool, rec


def oracle_decode(x, want_records=False, **kw):
    sl = x["slot_idx"].long()
    return O.decode(*(f64(x[n]) for n in NAMES), f64(x["pool"][sl]), want_records=want_records, **kw)



def check_decode_parity(o, o_ref, h, h_ref, tol, label):
    """Whole-tensor and worst (sequence, head) relative L2 of o [N, T, H, dv] and the states."""
    e = dict(o=rel_l2(f64(o), o_ref), o_worst=worst_decode(f64(o), o_ref), h=rel_l2(f64(h), h_ref),
             h_worst=worst_state(f64(h), h_ref))
    announce("%s rel-L2 o %.3g (worst seq/head %.3g), state %.3g (worst %.3g)"
             % (label, e["o"], e["o_worst"], e["h"], e["h_worst"]))
    for name, val in e.items():
        assert val <= tol, (name, val, tol)

def test_tiny_fp32_through_decode():
    """Tiny fp32 recurrent case (1 sequence, T = 64, H = 2, d = 64) run as one 64-token MTP call."""
    dev = need_gpu()
    announce("decode tiny fp32 T=64 H=2 d=64")
    t = W.tiny(seed=0)
    x = {n: t[n][None] for n in NAMES}
    x["pool"] = torch.zeros(1, 2, 64, 64)
    x["slot_idx"] = torch.zeros(1, dtype=torch.int32)
    o, pool, _ = run_decode(x, dev, scale=64 ** -0.5)
    o_ref, h_ref, _ = oracle_decode(x, scale=64 ** -0.5)
    check_decode_parity(o, o_ref, pool.cpu(), h_ref, 1e-4, "tiny fp32 through decode")


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_decode_pool_full_size(seed):
    """Decode step over a state pool: 512 slots [H=32, 128, 128], 64 sequences, bf16 q/k/v."""
    dev = need_gpu()
    announce("decode pool512 N64 H32 d128 bf16 seed=%d" % seed)
    x = W.decode(seed=seed)
    o, pool, _ = run_decode(x, dev)
    o_ref, h_ref, _ = oracle_decode(x)
    sl = x["slot_idx"].long()
    got = pool.cpu()
    check_decode_parity(o, o_ref, got[sl], h_ref, 1e-2, "decode pool512 N64 H32 seed=%d" % seed)
    untouched = torch.ones(x["pool"].shape[0], dtype=torch.bool)
    untouched[sl] = False
    assert torch.equal(got[untouched], x["pool"][untouched])


@pytest.mark.parametrize("T", [1, 3])
@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_decode_head_dims(dk, dv, dtype, T):
    """Both decode kernels (T = 1: four-wave tiles; T > 1: the multi-token kernel, one wave
    per 64-column tile) at every head shape."""
    dev = need_gpu()
    announce("decode dims dk=%d dv=%d %s T=%d" % (dk, dv, dtype, T))
    x = W.decode(seed=3, N=5, T=T, H=3, dk=dk, dv=dv, num_slots=9, dtype=dtype)
    o, pool, _ = run_decode(x, dev)
    o_ref, h_ref, _ = oracle_decode(x)
    tol = 1e-4 if dtype == torch.float32 else 1e-2
    check_decode_parity(o, o_ref, pool.cpu()[x["slot_idx"].long()], h_ref, tol,
                        "decode dims dk=%d dv=%d %s T=%d" % (dk, dv, dtype, T))


@pytest.mark.parametrize("T", [2, 8, 9, 20])
def test_mtp_multi_token(T):
    """T > 1 (MTP): tokens are applied in order with the state kept on chip; crosses the
    8-token LDS blocks."""
    dev = need_gpu()
    announce("decode MTP T=%d" % T)
    x = W.decode(seed=4, N=6, T=T, H=4, dk=128, dv=128, num_slots=16, dtype=torch.float32)
    o, pool, _ = run_decode(x, dev)
    o_ref, h_ref, _ = oracle_decode(x)
    check_decode_parity(o, o_ref, pool.cpu()[x["slot_idx"].long()], h_ref, 1e-4, "MTP fp32")


@pytest.mark.parametrize("T", [1, 3])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_slot_mapping_bit_exact(dtype, T):
    """beta = 0, g = 0, no norm, scale = 1, q = e_i for every token: o[n, t, h] = S[slot_n, h,
    i, :] exactly (rounded by the hardware bf16 conversion in bf16 mode, which must equal
    torch's cast), and every slot of the pool is byte-identical afterwards.  T = 1 runs the
    one-token kernel, T = 3 the multi-token one (its fp32 MFMA sums S0 entries times 1 and
    0, which is exact)."""
    dev = need_gpu()
    announce("decode slot mapping %s T=%d" % (dtype, T))
    N, H, d, num_slots = 24, 4, 128, 64
    gen = torch.Generator().manual_seed(7)
    pool = torch.randn(num_slots, H, d, d, generator=gen) * 3.0
    slots = torch.randperm(num_slots, generator=gen)[:N].to(torch.int32)
    rows = torch.randint(0, d, (N, H), generator=gen)
    q = torch.zeros(N, T, H, d)
    q[torch.arange(N)[:, None, None], torch.arange(T)[None, :, None], torch.arange(H)[None, None, :],
      rows[:, None, :]] = 1.0
    x = dict(q=q.to(dtype), k=torch.randn(N, T, H, d, generator=gen).to(dtype),
             v=torch.randn(N, T, H, d, generator=gen).to(dtype), g=torch.zeros(N, T, H, d),
             beta=torch.zeros(N, T, H), pool=pool, slot_idx=slots)
    o, pool_after, _ = run_decode(x, dev, scale=1.0, use_qk_l2norm=False)
    expect = pool[slots.long()[:, None], torch.arange(H)[None, :], rows]  # [N, H, d]
    for t in range(T):
        assert torch.equal(o.cpu()[:, t], expect.to(dtype)), t
    assert torch.equal(pool_after.cpu(), pool)


@pytest.mark.parametrize("T", [5, 11])
def test_mtp_without_l2norm(T):
    """use_qk_l2norm = 0 on the multi-token kernel (its norm factors are then 1): fp32
    parity of outputs and states, within and across 8-token blocks."""
    dev = need_gpu()
    announce("MTP without l2 norm T=%d" % T)
    x = W.decode(seed=10, N=4, T=T, H=2, dk=128, dv=128, num_slots=8, dtype=torch.float32)
    x["q"] = x["q"] * 0.1
    x["k"] = torch.nn.functional.normalize(x["k"], dim=-1)
    o, pool, _ = run_decode(x, dev, use_qk_l2norm=False)
    o_ref, h_ref, _ = oracle_decode(x, use_qk_l2norm=False)
    assert rel_l2(f64(o), o_ref) <= 1e-4
    assert rel_l2(f64(pool.cpu()[x["slot_idx"].long()]), h_ref) <= 1e-4


@pytest.mark.parametrize("T", [1, 2])
def test_skipped_slot(T):
    """A negative slot index skips the sequence: zero output, pool untouched."""
    dev = need_gpu()
    announce("decode skipped slot T=%d" % T)
    x = W.decode(seed=5, N=4, T=T, H=2, dk=128, dv=128, num_slots=8)
    x["slot_idx"][2] = -1
    o, pool, _ = run_decode(x, dev)
    assert torch.count_nonzero(o[2]).item() == 0
    keep = [0, 1, 3]
    y = {n: x[n][keep] for n in NAMES}
    y["pool"], y["slot_idx"] = x["pool"], x["slot_idx"][keep]
    o_ref, h_ref, _ = oracle_decode(y)
    assert rel_l2(f64(o[keep]), o_ref) <= 1e-2
    got = pool.cpu()
    assert rel_l2(f64(got[y["slot_idx"].long()]), h_ref) <= 1e-2
    others = torch.ones(8, dtype=torch.bool)
    others[y["slot_idx"].long()] = False
    assert torch.equal(got[others], x["pool"][others])


@pytest.mark.parametrize("seed", [0, 1])
def test_verify_and_replay_full_size(seed):
    """Speculative verify (32 sequences x 8 tokens, H = 32, d = 128) then ReplaySSM commit of
    accepted lengths drawn from 1..8, against direct recurrence over the accepted tokens."""
    dev = need_gpu()
    announce("verify+replay N32 T8 H32 d128 seed=%d" % seed)
    x = W.verify(seed=seed)
    o, pool, rec = run_decode(x, dev, records=True)
    got = pool.cpu()
    assert torch.equal(got, x["pool"]), "verify must not touch the pool"
    o_ref, _, rec_ref = oracle_decode(x, want_records=True)
    assert rel_l2(f64(o), o_ref) <= 1e-2
    assert rel_l2(f64(rec), rec_ref) <= 1e-2
    assert worst_decode(f64(o), o_ref) <= 1e-2
    acc = x["accepted"]
    kda.replay_commit(pool, x["slot_idx"].to(dev), rec, acc.to(dev))
    torch.cuda.synchronize()
    got = pool.cpu()
    sl = x["slot_idx"].long()
    worst = 0.0
    for n in range(x["q"].shape[0]):
        a = int(acc[n])
        _, h_n, _ = O.decode(*(f64(x[nm][n:n + 1, :a]) for nm in NAMES), f64(x["pool"][sl[n:n + 1]]))
        assert rel_l2(f64(got[sl[n]]), h_n[0]) <= 1e-2, n
        worst = max(worst, worst_state(f64(got[sl[n]])[None], h_n))
    announce("verify+replay seed=%d: rel-L2 o %.3g (worst seq/head %.3g), records %.3g, "
             "replayed state worst seq/head %.3g" % (seed, rel_l2(f64(o), o_ref),
                                                    worst_decode(f64(o), o_ref),
                                                    rel_l2(f64(rec), rec_ref), worst))
    assert worst <= 1e-2
    others = torch.ones(x["pool"].shape[0], dtype=torch.bool)
    others[sl] = False
    assert torch.equal(got[others], x["pool"][others])


@pytest.mark.parametrize("dk,dv,T", [(128, 128, 8), (64, 64, 8), (128, 64, 8), (128, 128, 12)])
def test_replay_bit_exact_with_commit(dk, dv, T):
    """Replaying a prefix of verify records reproduces, bit for bit, the state that committing
    the same tokens gives when the commit takes two or more tokens: one kernel forms u for
    both, and the commit applies it with the replay kernel's fp32 operations (T = 12 crosses
    the 8-token blocks on both sides).  A one-token commit runs the T = 1 kernel, whose
    reduction over dk is ordered differently: equal up to fp32 rounding."""
    dev = need_gpu()
    announce("replay vs commit bit-exact dk=%d dv=%d T=%d" % (dk, dv, T))
    x = W.verify(seed=3, N=12, T=T, H=4, dk=dk, dv=dv, num_slots=32)
    x["accepted"][0], x["accepted"][1], x["accepted"][2] = 1, T, 2
    if T > 8:
        x["accepted"][3] = 9
    _, pool_v, rec = run_decode(x, dev, records=True)
    acc = x["accepted"]
    kda.replay_commit(pool_v, x["slot_idx"].to(dev), rec, acc.to(dev))
    pool_c = x["pool"].to(dev)
    for a in sorted(set(int(v) for v in acc)):
        idx = (acc == a).nonzero().flatten()
        args = [x[n][idx, :a].contiguous().to(dev) for n in NAMES]
        kda.decode_step(*args, pool_c, x["slot_idx"][idx].contiguous().to(dev))
    torch.cuda.synchronize()
    pv, pc = pool_v.cpu(), pool_c.cpu()
    sl = x["slot_idx"].long()
    many, one = sl[acc > 1], sl[acc == 1]
    assert torch.equal(pv[many], pc[many])
    assert rel_l2(f64(pv[one]), f64(pc[one])) <= 1e-6
    others = torch.ones(pv.shape[0], dtype=torch.bool)
    others[sl] = False
    assert torch.equal(pv[others], pc[others])


@pytest.mark.parametrize("verify", [False, True])
def test_mtp_strong_decay(verify):
    """Gates far below the workloads' range (per-token g down to about -25, so the in-block
    factors exp(G_t - G_s) span many orders of magnitude and underflow): fp32 parity of
    outputs, states and records over 8- and 12-token calls."""
    dev = need_gpu()
    announce("MTP strong decay verify=%d" % verify)
    for T in (8, 12):
        x = W.decode(seed=9, N=4, T=T, H=2, dk=128, dv=128, num_slots=8, dtype=torch.float32)
        x["g"] = x["g"] * 50.0
        o, pool, rec = run_decode(x, dev, records=verify)
        o_ref, h_ref, rec_ref = oracle_decode(x, want_records=verify)
        assert rel_l2(f64(o), o_ref) <= 1e-4
        if verify:
            assert rel_l2(f64(rec), rec_ref) <= 1e-4
            assert torch.equal(pool.cpu(), x["pool"])
        else:
            assert rel_l2(f64(pool.cpu()[x["slot_idx"].long()]), h_ref) <= 1e-4


@pytest.mark.parametrize("T", [3, 5])
def test_verify_short_block(T):
    """Verify calls of fewer than 8 tokens (the one-block kernel, whose solve also runs over
    the absent tokens of the block): fp32 parity of outputs and records, the pool untouched,
    and replaying every prefix of two or more tokens equals committing it bit for bit."""
    dev = need_gpu()
    announce("verify short block T=%d" % T)
    x = W.decode(seed=11, N=6, T=T, H=3, dk=128, dv=128, num_slots=12, dtype=torch.float32,
                 with_accepted=True)
    x["accepted"] = torch.tensor([T, 2, T, 2, T, 2][:6], dtype=torch.int32)
    o, pool_v, rec = run_decode(x, dev, records=True)
    o_ref, _, rec_ref = oracle_decode(x, want_records=True)
    assert rel_l2(f64(o), o_ref) <= 1e-4
    assert rel_l2(f64(rec), rec_ref) <= 1e-4
    assert torch.equal(pool_v.cpu(), x["pool"])
    acc = x["accepted"]
    kda.replay_commit(pool_v, x["slot_idx"].to(dev), rec, acc.to(dev))
    pool_c = x["pool"].to(dev)
    for a in sorted(set(int(v) for v in acc)):
        idx = (acc == a).nonzero().flatten()
        args = [x[n][idx, :a].contiguous().to(dev) for n in NAMES]
        kda.decode_step(*args, pool_c, x["slot_idx"][idx].contiguous().to(dev))
    torch.cuda.synchronize()
    assert torch.equal(pool_v.cpu(), pool_c.cpu())


def test_replay_accept_zero_and_skip():
    dev = need_gpu()
    announce("replay accepted=0 and skipped slot")
    x = W.verify(seed=6, N=4, H=2, num_slots=8)
    _, pool, rec = run_decode(x, dev, records=True)
    acc = torch.tensor([0, 8, 3, 5], dtype=torch.int32)
    slots = x["slot_idx"].clone()
    slots[3] = -1
    kda.replay_commit(pool, slots.to(dev), rec, acc.to(dev))
    torch.cuda.synchronize()
    got = pool.cpu()
    sl = x["slot_idx"].long()
    assert torch.equal(got[sl[0]], x["pool"][sl[0]])
    assert torch.equal(got[sl[3]], x["pool"][sl[3]])
    for n in (1, 2):
        a = int(acc[n])
        _, h_n, _ = O.decode(*(f64(x[nm][n:n + 1, :a]) for nm in NAMES), f64(x["pool"][sl[n:n + 1]]))
        assert rel_l2(f64(got[sl[n]]), h_n[0]) <= 1e-2


def test_invariant_beta1_unit_key_on_gpu():
    """beta = 1 with a unit key (fp32): after the step S^T k = v up to fp32 rounding."""
    dev = need_gpu()
    announce("decode invariant beta=1 unit key")
    x = W.decode(seed=8, N=8, T=1, H=4, dk=128, dv=128, num_slots=8, dtype=torch.float32)
    x["beta"] = torch.ones_like(x["beta"])
    x["k"] = torch.nn.functional.normalize(x["k"], dim=-1)
    _, pool, _ = run_decode(x, dev, use_qk_l2norm=False)
    S = f64(pool.cpu()[x["slot_idx"].long()])
    k = f64(x["k"])[:, 0]
    got = np.einsum("nhcj,nhc->nhj", S, k)
    assert np.abs(got - f64(x["v"])[:, 0]).max() <= 1e-5 * max(1.0, np.abs(S).max())


def test_pool_offsets_beyond_32_bits():
    """Slots whose state lies beyond 2^31 elements (9 GB into a 9.2 GB pool of 140,100 slots of
    [1, 128, 128] fp32): the one-token and multi-token kernels, verify + replay, and the prefill
    (initial and final state in such slots) match the oracle, and the neighbouring slots keep
    their sentinel values."""
    dev = need_gpu()
    announce("pool offsets beyond 32 bits")
    S, d = 140_100, 128
    big = torch.empty(S, 1, d, d, device=dev)
    far = torch.tensor([140_050, 70_001, 139_998], dtype=torch.int32)
    sentinels = torch.cat([far.long() - 1, far.long() + 1])
    for T in (1, 3):
        x = W.decode(seed=12 + T, N=3, T=T, H=1, dk=d, dv=d, num_slots=3, dtype=torch.float32)
        sl = x["slot_idx"].long()
        big[far.long()] = x["pool"][sl].to(dev)
        big[sentinels] = 7.0
        args = [x[n].to(dev) for n in NAMES]
        o = kda.decode_step(*args, big, far.to(dev))
        torch.cuda.synchronize()
        o_ref, h_ref, _ = oracle_decode(x)
        assert rel_l2(f64(o), o_ref) <= 1e-4, T
        assert rel_l2(f64(big[far.long()].cpu()), h_ref) <= 1e-4, T
        assert bool((big[sentinels] == 7.0).all()), T
    # verify + replay through the same far slots
    x = W.decode(seed=20, N=3, T=4, H=1, dk=d, dv=d, num_slots=3, dtype=torch.float32, with_accepted=True)
    sl = x["slot_idx"].long()
    big[far.long()] = x["pool"][sl].to(dev)
    rec = torch.empty(3, 4, 1, 3 * d, device=dev)
    kda.decode_step(*(x[n].to(dev) for n in NAMES), big, far.to(dev), records=rec)
    assert torch.equal(big[far.long()].cpu(), x["pool"][sl])
    kda.replay_commit(big, far.to(dev), rec, x["accepted"].to(dev))
    torch.cuda.synchronize()
    for n in range(3):
        a = int(x["accepted"][n])
        _, h_n, _ = O.decode(*(f64(x[nm][n:n + 1, :a]) for nm in NAMES), f64(x["pool"][sl[n:n + 1]]))
        assert rel_l2(f64(big[far.long()[n]].cpu()), h_n[0]) <= 1e-4, n
    assert bool((big[sentinels] == 7.0).all())
    # prefill: initial states read from, final states written to far slots
    y = W.prefill(seed=21, seqlens=(100, 37), H=1, dk=d, dv=d, num_slots=2, h0_std=0.05)
    far2 = torch.tensor([140_020, 90_000], dtype=torch.int32)
    big[far2.long()] = y["pool"][y["slot_idx"].long()].to(dev)
    o = kda.chunk_prefill(*(y[n].to(dev) for n in ("q", "k", "v", "g", "beta", "cu_seqlens")), big,
                          far2.to(dev), h0_from_pool=True)
    torch.cuda.synchronize()
    o_ref, h_ref, _ = O.recurrent(f64(y["q"]), f64(y["k"]), f64(y["v"]), f64(y["g"]), f64(y["beta"]),
                                  y["cu_seqlens"].numpy(), h0=f64(y["pool"][y["slot_idx"].long()]))
    assert rel_l2(f64(o), o_ref) <= 1e-2
    assert rel_l2(f64(big[far2.long()].cpu()), h_ref) <= 1e-2
    del big
    torch.cuda.empty_cache()


def test_diag_state_stream_leaves_the_pool_unchanged():
    """The diagnostic memory pass (the decode kernel's state access pattern, no arithmetic) reads
    and rewrites the slots bit for bit, skips negative slots, and touches nothing else."""
    dev = need_gpu()
    announce("diag state stream")
    from kda_gated_delta_rule_amd import ops
    for dk, dv in ((128, 128), (64, 128), (128, 64), (64, 64)):
        x = W.decode(seed=70, N=6, H=3, dk=dk, dv=dv, num_slots=10)
        pool = x["pool"].to(dev)
        sl = x["slot_idx"].clone()
        sl[1] = -1
        ops.diag_state_stream(pool, sl.to(dev))
        torch.cuda.synchronize()
        assert torch.equal(pool.cpu(), x["pool"])
