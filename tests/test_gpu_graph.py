"""The entry points inside a captured HIP graph (as the benchmark and serving loops run them):
every replay equals the same calls made eagerly, bit for bit; and on concurrent streams, where
they equal the same calls made one after another.

Each case keeps two copies of the pool, one driven eagerly and one by the graph, replays the graph
three times with eager work and a synchronisation between replays, and compares outputs, records
and pool contents after every replay.  The library launches kernels only (no memsets, copies or
allocations), so nothing but kernel nodes is captured."""
import pytest
import torch

import kda_gated_delta_rule_amd as kda
import kda_workloads as W
from _util import announce, need_gpu

pytestmark = pytest.mark.gpu


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("T", [1, 4])
def test_decode_commit_in_a_graph(T):
    dev = need_gpu()
    announce("graph: decode commit T=%d" % T)
    x = W.decode(seed=11, N=16, T=T, H=8)
    q, k, v, g, beta = (x[n].to(dev) for n in ("q", "k", "v", "g", "beta"))
    sl = x["slot_idx"].to(dev)
    pool0 = x["pool"].to(dev)
    pool_g = pool0.clone()
    o_g = torch.empty_like(q)
    graph = _capture(lambda: kda.decode_step(q, k, v, g, beta, pool_g, sl, o=o_g))
    # the warm-up and the capture itself ran once (capture does not execute): realign both pools
    pool_g.copy_(pool0)
    pool_e = pool0.clone()
    torch.cuda.synchronize()
    for rep in range(3):
        o_e = kda.decode_step(q, k, v, g, beta, pool_e, sl)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), rep
        assert torch.equal(pool_g, pool_e), rep
        (pool_e.sum() + 1.0).item()  # unrelated eager work between replays


def test_verify_and_replay_in_a_graph():
    dev = need_gpu()
    announce("graph: verify + replay commit")
    x = W.verify(seed=12, N=16, H=8)
    q, k, v, g, beta = (x[n].to(dev) for n in ("q", "k", "v", "g", "beta"))
    sl, acc = x["slot_idx"].to(dev), x["accepted"].to(dev)
    N, T, H, dk = q.shape
    dv = v.shape[-1]
    pool0 = x["pool"].to(dev)
    pool_g = pool0.clone()
    o_g = torch.empty_like(q)
    rec_g = torch.empty(N, T, H, 2 * dk + dv, device=dev)

    def step():
        kda.decode_step(q, k, v, g, beta, pool_g, sl, o=o_g, records=rec_g)
        kda.replay_commit(pool_g, sl, rec_g, acc)

    graph = _capture(step)
    pool_g.copy_(pool0)
    pool_e = pool0.clone()
    rec_e = torch.empty_like(rec_g)
    torch.cuda.synchronize()
    for rep in range(3):
        o_e = kda.decode_step(q, k, v, g, beta, pool_e, sl, records=rec_e)
        kda.replay_commit(pool_e, sl, rec_e, acc)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), rep
        assert torch.equal(rec_g, rec_e), rep
        assert torch.equal(pool_g, pool_e), rep
        (pool_e.sum() + 1.0).item()


def test_prefill_in_a_graph():
    dev = need_gpu()
    announce("graph: varlen prefill with h0 from the pool")
    y = W.prefill(seed=13, seqlens=(700, 64, 1, 300), H=4, num_slots=8, h0_std=0.05)
    q, k, v, g, beta, cu = (y[n].to(dev) for n in ("q", "k", "v", "g", "beta", "cu_seqlens"))
    sl = y["slot_idx"].to(dev)
    Tt, H, dk = q.shape
    dv = v.shape[-1]
    ns = cu.shape[0] - 1
    ws_g = torch.empty(kda.chunk_prefill_workspace_size(ns, Tt, H, dk, dv), dtype=torch.uint8, device=dev)
    pool0 = y["pool"].to(dev)
    pool_g = pool0.clone()
    o_g = torch.empty_like(v)
    graph = _capture(lambda: kda.chunk_prefill(q, k, v, g, beta, cu, pool_g, sl, h0_from_pool=True,
                                               o=o_g, workspace=ws_g))
    pool_g.copy_(pool0)
    pool_e = pool0.clone()
    torch.cuda.synchronize()
    for rep in range(3):
        # each call reads the initial states from the slots and writes the final ones back, so
        # consecutive calls continue from the previous final state
        o_e = kda.chunk_prefill(q, k, v, g, beta, cu, pool_e, sl, h0_from_pool=True)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), rep
        assert torch.equal(pool_g, pool_e), rep
        (pool_e.sum() + 1.0).item()


def test_concurrent_streams_match_sequential_calls():
    """Decode, verify + replay and prefill on three streams at once (disjoint slots of one pool)
    equal the same calls made one after another: each entry point runs on the stream it is
    given and touches only its own slots."""
    dev = need_gpu()
    announce("streams: decode | verify + replay | prefill concurrently on one pool")
    H = 8
    xd = W.decode(seed=21, N=12, T=1, H=H, num_slots=64)
    xv = W.verify(seed=22, N=12, H=H, num_slots=64)
    y = W.prefill(seed=23, seqlens=(500, 130), H=H, num_slots=64, h0_std=0.05)
    pool0 = xd["pool"].to(dev)
    # disjoint slot sets: 0-11 decode, 12-23 verify, 24-25 prefill
    sd = torch.arange(0, 12, dtype=torch.int32, device=dev)
    sv = torch.arange(12, 24, dtype=torch.int32, device=dev)
    sp = torch.arange(24, 26, dtype=torch.int32, device=dev)
    d_in = [xd[n].to(dev) for n in ("q", "k", "v", "g", "beta")]
    v_in = [xv[n].to(dev) for n in ("q", "k", "v", "g", "beta")]
    acc = xv["accepted"].to(dev)
    p_in = [y[n].to(dev) for n in ("q", "k", "v", "g", "beta", "cu_seqlens")]
    N, T, _, dk = v_in[0].shape
    dv = v_in[2].shape[-1]
    Tt = p_in[0].shape[0]

    def run(pool, streams):
        od, ov, op = torch.empty_like(d_in[0]), torch.empty_like(v_in[0]), torch.empty_like(p_in[2])
        rec = torch.empty(N, T, H, 2 * dk + dv, device=dev)
        ws = torch.empty(kda.chunk_prefill_workspace_size(2, Tt, H, dk, dv), dtype=torch.uint8,
                         device=dev)
        torch.cuda.synchronize()
        with torch.cuda.stream(streams[0]):
            kda.decode_step(*d_in, pool, sd, o=od)
        with torch.cuda.stream(streams[1]):
            kda.decode_step(*v_in, pool, sv, o=ov, records=rec)
            kda.replay_commit(pool, sv, rec, acc)
        with torch.cuda.stream(streams[2]):
            kda.chunk_prefill(*p_in, pool, sp, h0_from_pool=True, o=op, workspace=ws)
        torch.cuda.synchronize()
        return od, ov, rec, op

    cur = torch.cuda.current_stream()
    pool_seq, pool_par = pool0.clone(), pool0.clone()
    seq = run(pool_seq, [cur, cur, cur])
    par = run(pool_par, [torch.cuda.Stream() for _ in range(3)])
    for a, b in zip(seq, par):
        assert torch.equal(a, b)
    assert torch.equal(pool_seq, pool_par)
    assert torch.equal(pool_par[26:], pool0[26:])  # slots outside the calls untouched


def test_prefill_snapshots_in_a_graph():
    dev = need_gpu()
    announce("graph: prefill with prefix-cache snapshots every 128 tokens")
    y = W.prefill(seed=14, seqlens=(600, 200), H=4, num_slots=16, h0_std=0.05)
    q, k, v, g, beta, cu = (y[n].to(dev) for n in ("q", "k", "v", "g", "beta", "cu_seqlens"))
    Tt, H, dk = q.shape
    dv = v.shape[-1]
    sl = torch.tensor([0, 1], dtype=torch.int32, device=dev)
    # snapshot slots 2.. (sequence 0: 4 snapshots at 128..512; sequence 1: 1 at 128, rest skipped)
    snap = torch.tensor([[2, 3, 4, 5], [6, -1, -1, -1]], dtype=torch.int32, device=dev)
    ws_g = torch.empty(kda.chunk_prefill_workspace_size(2, Tt, H, dk, dv), dtype=torch.uint8, device=dev)
    pool0 = y["pool"].to(dev)
    pool_g = pool0.clone()
    o_g = torch.empty_like(v)
    graph = _capture(lambda: kda.chunk_prefill(q, k, v, g, beta, cu, pool_g, sl, h0_from_pool=False,
                                               o=o_g, workspace=ws_g, snapshot_every=128,
                                               snapshot_slots=snap))
    pool_g.copy_(pool0)
    pool_e = pool0.clone()
    torch.cuda.synchronize()
    for rep in range(3):
        o_e = kda.chunk_prefill(q, k, v, g, beta, cu, pool_e, sl, h0_from_pool=False,
                                snapshot_every=128, snapshot_slots=snap)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), rep
        assert torch.equal(pool_g, pool_e), rep
        assert torch.equal(pool_g[7:], pool0[7:]), rep  # slots outside the call untouched
        (pool_e.sum() + 1.0).item()
