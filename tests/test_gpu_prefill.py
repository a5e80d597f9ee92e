"""GPU parity of the chunked prefill against the fp64 token recurrence (oracle),
through the C ABI.  Every case is compared element-wise in full, the two full-size
workloads (T = 8192 x H = 32, and the 4-sequence 128,076-token H = 16 batch) included;
besides the whole-tensor relative L2, the worst (sequence, head) value is checked.
"""
import numpy as np
import pytest
import torch

import kda_gated_delta_rule_amd as kda
import kda_workloads as W
from oracle import kda_oracle as O
from tests._util import (announce, check_prefill_parity, f64, need_gpu, rel_l2, worst_chunk_head,
                         worst_rel_l2, worst_seq_head, worst_state)

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "g", "beta")


def run_prefill(y, dev, h0_from_pool=True, **kw):
    pool = y["pool"].to(dev)
    o = kda.chunk_prefill(*(y[n].to(dev) for n in NAMES), y["cu_seqlens"].to(dev), pool,
                          y["slot_idx"].to(dev), h0_from_pool=h0_from_pool, **kw)
    torch.cuda.synchronize()
    return o, pool


def oracle_prefill(y, h0_from_pool=True, heads=None, **kw):
    sl = y["slot_idx"].long()
    pick = (lambda t: t) if heads is None else (lambda t: t[:, heads])
    h0 = f64(y["pool"][sl]) if h0_from_pool else None
    if h0 is not None and heads is not None:
        h0 = h0[:, heads]
    return O.recurrent(*(f64(pick(y[n])) for n in NAMES), y["cu_seqlens"].numpy(), h0=h0, **kw)


def test_tiny_fp32_through_prefill():
    """Tiny fp32 case (T = 64, H = 2, d = 64): exactly one 64-token chunk; rel-L2 <= 1e-4."""
    dev = need_gpu()
    announce("prefill tiny fp32 one chunk")
    t = W.tiny(seed=0)
    y = dict(t)
    y["cu_seqlens"] = torch.tensor([0, 64], dtype=torch.int32)
    y["pool"] = torch.full((1, 2, 64, 64), 7.0)  # h0_from_pool = 0: contents must not matter
    y["slot_idx"] = torch.zeros(1, dtype=torch.int32)
    o, pool = run_prefill(y, dev, h0_from_pool=False, scale=64 ** -0.5)
    o_ref, h_ref, _ = oracle_prefill(y, h0_from_pool=False, scale=64 ** -0.5)
    check_prefill_parity(f64(o), o_ref, f64(pool.cpu()), h_ref, y["cu_seqlens"], 1e-4, "tiny fp32")


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_fp32_varlen_ragged(dk, dv):
    """fp32: ragged varlen batch with tails, an empty sequence and h0 from slots."""
    dev = need_gpu()
    announce("prefill fp32 varlen dk=%d dv=%d" % (dk, dv))
    y = W.prefill(seed=1, seqlens=(1, 63, 64, 65, 0, 200, 130), H=3, dk=dk, dv=dv, num_slots=10,
                  h0_std=0.05, dtype=torch.float32)
    o, pool = run_prefill(y, dev)
    o_ref, h_ref, _ = oracle_prefill(y)
    check_prefill_parity(f64(o), o_ref, f64(pool.cpu()[y["slot_idx"].long()]), h_ref, y["cu_seqlens"],
                         1e-4, "fp32")


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64), (64, 128)])
def test_bf16_varlen_ragged(dk, dv):
    dev = need_gpu()
    announce("prefill bf16 varlen dk=%d dv=%d" % (dk, dv))
    y = W.prefill(seed=2, seqlens=(1, 63, 64, 65, 0, 200, 777), H=4, dk=dk, dv=dv, num_slots=12,
                  h0_std=0.05)
    o, pool = run_prefill(y, dev)
    o_ref, h_ref, _ = oracle_prefill(y)
    got = pool.cpu()
    sl = y["slot_idx"].long()
    check_prefill_parity(f64(o), o_ref, f64(got[sl]), h_ref, y["cu_seqlens"], 1e-2, "bf16 ragged")
    others = torch.ones(12, dtype=torch.bool)
    others[sl] = False
    assert torch.equal(got[others], y["pool"][others])


# Sequences longer than one segment (16 chunks at these sizes) go through the segment
# scan: a local pass from [0 | I], the fp32 scan of segment start states, and the output
# pass.  Lengths cover 1-chunk tail segments, exact multiples of the segment and of the
# chunk.
MULTI_SEG = (4200, 2049, 64, 0, 4097, 2048)


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_fp32_multi_segment(dk, dv):
    """fp32 through several segments per sequence with h0 from slots; <= 1e-4.  At dk = dv =
    128 the local pass splits [S | Phi] over two workgroups by columns."""
    dev = need_gpu()
    announce("prefill fp32 multi-segment dk=%d dv=%d" % (dk, dv))
    y = W.prefill(seed=7, seqlens=MULTI_SEG, H=2, dk=dk, dv=dv, num_slots=8, h0_std=0.05,
                  dtype=torch.float32)
    o, pool = run_prefill(y, dev)
    o_ref, h_ref, _ = oracle_prefill(y)
    check_prefill_parity(f64(o), o_ref, f64(pool.cpu()[y["slot_idx"].long()]), h_ref, y["cu_seqlens"],
                         1e-4, "fp32")


@pytest.mark.parametrize("h0", [True, False])
def test_bf16_multi_segment(h0):
    """bf16 dk = dv = 128 through several segments per sequence; rel-L2 <= 1e-2."""
    dev = need_gpu()
    announce("prefill bf16 multi-segment h0_from_pool=%d" % h0)
    y = W.prefill(seed=8, seqlens=MULTI_SEG, H=3, dk=128, dv=128, num_slots=8, h0_std=0.05)
    o, pool = run_prefill(y, dev, h0_from_pool=h0)
    o_ref, h_ref, _ = oracle_prefill(y, h0_from_pool=h0)
    check_prefill_parity(f64(o), o_ref, f64(pool.cpu()[y["slot_idx"].long()]), h_ref, y["cu_seqlens"],
                         1e-2, "bf16 multi-segment")


def test_many_short_sequences_scan_grid_loops():
    """520 sequences x 64 heads = 33,280 (sequence, head) scan groups, more than the scan
    launch covers at once (4,096 groups of 8), so its blocks loop; lengths 0..70 (empty,
    single-token, one- and two-chunk sequences), h0 from slots, bf16 dk = dv = 64."""
    dev = need_gpu()
    announce("prefill 520 short sequences x 64 heads")
    gen = np.random.default_rng(11)
    lens = gen.choice([0, 1, 2, 3, 5, 17, 63, 64, 65, 70], size=520).tolist()
    y = W.prefill(seed=9, seqlens=tuple(lens), H=64, dk=64, dv=64, num_slots=520, h0_std=0.05)
    assert 520 * 64 > 4096 * 8
    o, pool = run_prefill(y, dev)
    o_ref, h_ref, _ = oracle_prefill(y)
    check_prefill_parity(f64(o), o_ref, f64(pool.cpu()[y["slot_idx"].long()]), h_ref, y["cu_seqlens"],
                         1e-2, "520 short sequences")


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float32, 64), (torch.float32, 128)])
def test_beta0_g0_keeps_the_state_exactly(dtype, d):
    """beta = 0 and g = 0: every chunk leaves the state unchanged (W = 0, Ut = 0, exp(G_L) = 1),
    the local pass keeps Phi = I and S_loc = 0, and the scan multiplies by I, all exactly, so
    the final state equals the initial one bit for bit across several segments; o = scale
    q_hat^T h0 (rel-L2 at the dtype's bar)."""
    dev = need_gpu()
    announce("prefill beta=0 g=0 %s d=%d" % (dtype, d))
    y = W.prefill(seed=10, seqlens=(3000, 1100, 7), H=2, dk=d, dv=d, num_slots=3, h0_std=0.5,
                  dtype=dtype)
    y["beta"] = torch.zeros_like(y["beta"])
    y["g"] = torch.zeros_like(y["g"])
    o, pool = run_prefill(y, dev)
    sl = y["slot_idx"].long()
    assert torch.equal(pool.cpu()[sl], y["pool"][sl])
    o_ref, h_ref, _ = oracle_prefill(y)
    assert np.array_equal(h_ref, f64(y["pool"][sl]))  # the oracle agrees: state unchanged
    assert rel_l2(f64(o), o_ref) <= (1e-4 if dtype == torch.float32 else 1e-2)


@pytest.mark.parametrize("h0", [True, False])
def test_all_sequences_empty(h0):
    """Every sequence empty (no chunks: only the scan's pass-through runs): the final state
    is the initial one (h0 from the slot) or zero; other slots are untouched."""
    dev = need_gpu()
    announce("prefill all sequences empty h0_from_pool=%d" % h0)
    y = W.prefill(seed=12, seqlens=(0, 0, 0), H=2, dk=128, dv=128, num_slots=5, h0_std=0.3)
    o, pool = run_prefill(y, dev, h0_from_pool=h0)
    assert o.shape[0] == 0
    got, sl = pool.cpu(), y["slot_idx"].long()
    if h0:
        assert torch.equal(got[sl], y["pool"][sl])
    else:
        assert torch.count_nonzero(got[sl]).item() == 0
    others = torch.ones(5, dtype=torch.bool)
    others[sl] = False
    assert torch.equal(got[others], y["pool"][others])


def test_workspace_reused_across_calls():
    """One workspace buffer (filled with garbage first) serves two calls of different shapes
    in a row; its contents on entry do not matter."""
    dev = need_gpu()
    announce("prefill workspace reuse")
    ya = W.prefill(seed=13, seqlens=(300, 1500), H=2, dk=128, dv=128, num_slots=2, h0_std=0.05)
    yb = W.prefill(seed=14, seqlens=(70, 5, 64), H=2, dk=128, dv=128, num_slots=3, h0_std=0.05)
    need = max(kda.chunk_prefill_workspace_size(2, 1800, 2, 128, 128),
               kda.chunk_prefill_workspace_size(3, 139, 2, 128, 128))
    ws = torch.full((need,), 0xAB, dtype=torch.uint8, device=dev)
    for y in (ya, yb):
        pool = y["pool"].to(dev)
        o = kda.chunk_prefill(*(y[n].to(dev) for n in NAMES), y["cu_seqlens"].to(dev), pool,
                              y["slot_idx"].to(dev), workspace=ws)
        torch.cuda.synchronize()
        o_ref, h_ref, _ = oracle_prefill(y)
        check_prefill_parity(f64(o), o_ref, f64(pool.cpu()[y["slot_idx"].long()]), h_ref,
                             y["cu_seqlens"], 1e-2, "workspace reuse")


def prefix_states(y, requests, h0_from_pool=True):
    """Oracle states after the first p tokens of sequence i, for each (i, p) in requests: one
    fp64 recurrence call over a batch whose sequences are those prefixes."""
    cu = y["cu_seqlens"].tolist()
    parts = {n: [] for n in NAMES}
    lens, h0 = [], []
    for i, p in requests:
        for n in NAMES:
            parts[n].append(y[n][cu[i]:cu[i] + p])
        lens.append(p)
        h0.append(f64(y["pool"][int(y["slot_idx"][i])]) if h0_from_pool
                  else np.zeros(y["pool"].shape[1:]))
    cat = {n: torch.cat(parts[n]) for n in NAMES}
    cu_p = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    _, ht, _ = O.recurrent(*(f64(cat[n]) for n in NAMES), cu_p, h0=np.stack(h0))
    return ht


@pytest.mark.parametrize("dtype,d,tol", [(torch.bfloat16, 128, 1e-2), (torch.float32, 64, 1e-4)])
def test_prefix_snapshots(dtype, d, tol):
    """kda_chunk_prefill_snapshots: the state after every 256 tokens of each sequence lands in
    its snapshot slot and equals the recurrence's state at that position (one at a segment
    start, one at a full length); skipped (-1) and out-of-range entries leave slots untouched;
    o and the final states are those of the plain call."""
    dev = need_gpu()
    announce("prefill prefix snapshots %s d=%d" % (dtype, d))
    seqlens, every, max_snaps = (1500, 512, 200, 0, 2049), 256, 9
    ns = len(seqlens)
    num_slots = ns + ns * max_snaps
    y = W.prefill(seed=15, seqlens=seqlens, H=2, dk=d, dv=d, num_slots=num_slots, h0_std=0.05,
                  dtype=dtype)
    taken = set(y["slot_idx"].tolist())
    free = [s for s in range(num_slots) if s not in taken]
    snap = torch.tensor(free[:ns * max_snaps], dtype=torch.int32).reshape(ns, max_snaps)
    snap[0, 1] = -1  # skipped
    pool = y["pool"].to(dev)
    o = kda.chunk_prefill(*(y[n].to(dev) for n in NAMES), y["cu_seqlens"].to(dev), pool,
                          y["slot_idx"].to(dev), snapshot_every=every,
                          snapshot_slots=snap.to(dev))
    torch.cuda.synchronize()
    got = pool.cpu()
    o_ref, h_ref, _ = oracle_prefill(y)
    check_prefill_parity(f64(o), o_ref, f64(got[y["slot_idx"].long()]), h_ref, y["cu_seqlens"], tol,
                         "snapshots")
    requests, slots = [], []
    untouched = set(range(num_slots)) - taken
    for i, L in enumerate(seqlens):
        for j in range(max_snaps):
            p = (j + 1) * every
            if p <= L and snap[i, j] >= 0:
                requests.append((i, p))
                slots.append(int(snap[i, j]))
                untouched.discard(int(snap[i, j]))
    assert (4, 2048) in requests and (1, 512) in requests  # a segment start, a full length
    ref = prefix_states(y, requests)
    for n, (req, sl) in enumerate(zip(requests, slots)):
        assert rel_l2(f64(got[sl]), ref[n]) <= tol, req
    for sl in sorted(untouched):
        assert torch.equal(got[sl], y["pool"][sl]), sl


def test_resume_from_snapshot_matches_the_longer_call():
    """Prefix-cache use: a 2,500-token prefill keeps a snapshot after 1,024 tokens; a second
    prefill of tokens 1,024.. that starts from the snapshot slot gives the outputs and final
    state of the longer call."""
    dev = need_gpu()
    announce("prefill resume from snapshot")
    y = W.prefill(seed=16, seqlens=(2500,), H=3, dk=128, dv=128, num_slots=3, h0_std=0.05)
    pool = y["pool"].to(dev)
    fin = int(y["slot_idx"][0])
    ss = [s for s in range(3) if s != fin][0]  # snapshot slot
    snap = torch.tensor([[ss, -1]], dtype=torch.int32, device=dev)  # after 1024 tokens
    full = kda.chunk_prefill(*(y[n].to(dev) for n in NAMES), y["cu_seqlens"].to(dev), pool,
                             y["slot_idx"].to(dev), snapshot_every=1024, snapshot_slots=snap)
    a = 1024
    tail = [y[n][a:].contiguous().to(dev) for n in NAMES]
    pool2 = pool.clone()
    rest = kda.chunk_prefill(*tail, torch.tensor([0, 2500 - a], dtype=torch.int32, device=dev),
                             pool2, torch.tensor([ss], dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    assert rel_l2(f64(rest), f64(full[a:])) <= 1e-2
    assert rel_l2(f64(pool2.cpu()[ss]), f64(pool.cpu()[fin])) <= 1e-2
    o_ref, _, _ = oracle_prefill(y)
    assert rel_l2(f64(rest), o_ref[a:]) <= 1e-2


def test_zero_initial_state_ignores_pool_contents():
    dev = need_gpu()
    announce("prefill h0 zero")
    y = W.prefill(seed=3, seqlens=(150, 20), H=2, dk=128, dv=128, num_slots=2, h0_std=1.0)
    o, pool = run_prefill(y, dev, h0_from_pool=False)
    o_ref, h_ref, _ = oracle_prefill(y, h0_from_pool=False)
    check_prefill_parity(f64(o), o_ref, f64(pool.cpu()[y["slot_idx"].long()]), h_ref, y["cu_seqlens"],
                         1e-2, "h0 zero")


def test_empty_sequence_passes_state_through():
    dev = need_gpu()
    announce("prefill empty sequence")
    y = W.prefill(seed=4, seqlens=(0, 70, 0), H=2, dk=128, dv=128, num_slots=3, h0_std=0.05)
    _, pool = run_prefill(y, dev)
    got = pool.cpu()
    sl = y["slot_idx"].long()
    assert torch.equal(got[sl[0]], y["pool"][sl[0]])
    assert torch.equal(got[sl[2]], y["pool"][sl[2]])


@pytest.mark.parametrize("dtype,d,tol", [(torch.float32, 64, 1e-4), (torch.bfloat16, 128, 1e-2)])
def test_prefill_then_decode_equals_longer_prefill(dtype, d, tol):
    """Checkpoint / resume through the pool: prefill(x[:a]) then decode(x[a:]) equals the
    recurrence over x (state handed over in the slot)."""
    dev = need_gpu()
    announce("prefill then decode handover %s d=%d" % (dtype, d))
    y = W.prefill(seed=5, seqlens=(131,), H=4, dk=d, dv=d, num_slots=1, h0_std=0.05, dtype=dtype)
    a = 128
    head = {n: y[n][:a] for n in NAMES}
    head.update(cu_seqlens=torch.tensor([0, a], dtype=torch.int32), pool=y["pool"],
                slot_idx=y["slot_idx"])
    _, pool = run_prefill(head, dev)
    tail = [y[n][a:][None].contiguous().to(dev) for n in NAMES]
    o_tail = kda.decode_step(*tail, pool, y["slot_idx"].to(dev))
    torch.cuda.synchronize()
    o_ref, h_ref, _ = oracle_prefill(y)
    assert rel_l2(f64(o_tail[0]), o_ref[a:]) <= tol
    assert rel_l2(f64(pool.cpu()[0]), h_ref[0]) <= tol


def test_prefill_full_size_T8192_H32():
    """Chunked prefill workload: T = 8192, H = 32, dk = dv = 128, bf16, zero initial state.
    Every head against the oracle (32 full 8192-token chains): whole tensor, worst head and
    worst (64-token chunk, head) for o, whole and worst head for the final state."""
    dev = need_gpu()
    announce("prefill T8192 H32 d128")
    y = W.prefill(seed=0, seqlens=(8192,), H=32, dk=128, dv=128, num_slots=1)
    o, pool = run_prefill(y, dev, h0_from_pool=False)
    o_ref, h_ref, _ = oracle_prefill(y, h0_from_pool=False)
    oc, hc = f64(o), f64(pool.cpu()[y["slot_idx"].long()])
    check_prefill_parity(oc, o_ref, hc, h_ref, y["cu_seqlens"], 1e-2, "T8192 H32")
    wc = worst_chunk_head(oc, o_ref, y["cu_seqlens"])
    announce("T8192 H32: worst (chunk, head) rel-L2 %.3g" % wc)
    assert wc <= 2e-2


def test_prefill_full_size_varlen_long_context():
    """Long-context varlen workload: 4 sequences (100000, 16384, 8192, 3500) packed with
    cu_seqlens, H = 16, initial states from 4 pool slots.  Every head of every sequence
    against the oracle (the 100,000-token chains included): whole tensor, worst (sequence,
    head), worst (64-token chunk, head) for o; whole and worst for the final states."""
    dev = need_gpu()
    announce("prefill varlen 128076 tokens H16")
    y = W.prefill_long(seed=0)
    o, pool = run_prefill(y, dev)
    o_ref, h_ref, _ = oracle_prefill(y)
    oc, hc = f64(o), f64(pool.cpu()[y["slot_idx"].long()])
    check_prefill_parity(oc, o_ref, hc, h_ref, y["cu_seqlens"], 1e-2, "varlen 128076 H16")
    wc = worst_chunk_head(oc, o_ref, y["cu_seqlens"])
    announce("varlen 128076 H16: worst (chunk, head) rel-L2 %.3g" % wc)
    assert wc <= 2e-2
