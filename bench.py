#!/usr/bin/env python3
"""Benchmark of the KDA hot path on one MI355X.

Timed step (the headline metric): one fused decode step over the state pool of
the decode workload -- 512 fp32 slots of [H=32, 128, 128], 64 active sequences,
1 token each, bf16 q/k/v, state updated in place.  Successive steps cycle through
8 disjoint sets of 64 slots (the whole 1 GiB pool), so state reads come from HBM
rather than the 256 MB Infinity Cache.

value = state updates per second = (sequences x heads) x steps / elapsed.

Also measured in the same run (reported under "extra", not part of the timed
step): chunked prefill (T = 8192, H = 32) and the long-context varlen prefill
(4 sequences, 128,076 tokens, H = 16) as tokens/s with their MFMA and HBM
fractions; speculative verify + ReplaySSM commit (32 x 8 tokens, H = 32); the
chunked backward on the T = 8192, H = 32 shape; a device copy of 1 GiB as a
bandwidth reference; and the fp64 CPU oracle on a
bounded sample of the decode workload (cpu_baseline).

Prints ONE JSON line.
"""
import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, vendor figure
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 (matrix and vector), vendor figure
METRIC = ("KDA decode state-updates/s (HBM GB/s % peak); "
          "chunked-prefill tokens/s (MFMA %)")


def decode_bytes_per_update(dk, dv, io_bytes):
    """Algorithmic HBM bytes of one (token, head) decode update: the fp32 state read and
    written once, q, k, v and o in the io dtype, g (fp32 per key channel) and beta."""
    return 2 * dk * dv * 4 + (2 * dk + dv) * io_bytes + dk * 4 + 4 + dv * io_bytes


def mtp_bytes_per_head(dk, dv, T, io_bytes):
    """Algorithmic HBM bytes of one (sequence, head) multi-token commit of T tokens: the fp32
    state read and written once, and each token's q, k, v, o (io dtype), g (fp32) and beta."""
    return 2 * dk * dv * 4 + T * prefill_bytes_per_token_head(dk, dv, io_bytes)


def prefill_bytes_per_token_head(dk, dv, io_bytes):
    """q, k, v read + o written (io dtype), g (fp32) and beta read, once each."""
    return (2 * dk + dv) * io_bytes + dk * 4 + 4 + dv * io_bytes


def front_decode_bytes_per_update(dk, dv, width, io_bytes, sequences):
    """A decode update with the input front: decode_bytes_per_update (the raw q, k, v, gate and
    beta in place of the processed ones, same sizes), the slot's convolution state read and
    written ((width - 1) rows of 2 dk + dv channels, io dtype), and the head's fp32 convolution
    weights (width taps per channel) read once per launch, shared by its `sequences` updates."""
    return (decode_bytes_per_update(dk, dv, io_bytes) + 2 * (width - 1) * (2 * dk + dv) * io_bytes
            + (2 * dk + dv) * width * 4 / sequences)


def prefill_flops_per_token_head(dk, dv, C=64):
    """Algorithmic flops per (token, head) of the 64-token chunk form as the kernels compute it,
    counting every intra-chunk product as a dense C x C tile: A and P (2 C^2 dk each), W = T KG
    (2 C^2 dk), Ut = T V (2 C^2 dv) and P U (2 C^2 dv) -- together 2 C^2 (3 dk + 2 dv) -- plus
    the three state products W S, QG S and Kt^T U (2 C dk dv each); divided by the C tokens of
    a chunk."""
    per_chunk = 2 * C * C * (3 * dk + 2 * dv) + 3 * 2 * C * dk * dv
    return per_chunk / C


def backward_flops_per_token_head(dk, dv, C=64):
    """Algorithmic flops per (token, head) of the chunked backward as the kernels compute it
    (dense C x C tiles), divided by the C tokens of a chunk: the forward pass it runs again
    (prefill_flops_per_token_head), the recomputed A, P, W, Ut (2 C^2 (3 dk + dv)), the reverse
    recurrence's Mt = W^T Kt, P W and b = Q'^T dO (2 C dk^2 + 2 C^2 dk + 2 C dk dv) and its
    step Mt dS (2 dk^2 dv), the products with the state and its gradient (W S, Kt dH, dO S^T,
    dU S^T, U dH^T: 5 x 2 C dk dv; P^T dO and dO U^T: 2 x 2 C^2 dv), the UT backward (dT, dBK,
    dBV: 2 C^2 (2 dk + 2 dv); T^T dT and its product with T^T: 2 x 2 C^3) and the four decayed
    token products (4 x 2 C^2 dk)."""
    per_chunk = (2 * C * C * (3 * dk + dv)
                 + 2 * C * dk * dk + 2 * C * C * dk + 2 * C * dk * dv + 2 * dk * dk * dv
                 + 5 * 2 * C * dk * dv + 2 * 2 * C * C * dv
                 + 2 * C * C * (2 * dk + 2 * dv) + 2 * 2 * C ** 3
                 + 4 * 2 * C * C * dk)
    return per_chunk / C + prefill_flops_per_token_head(dk, dv, C)


def backward_bytes_per_token_head(dk, dv, io_bytes):
    """q, k, v and the output gradient read (io dtype), g and beta read; dq, dk, dv written (io
    dtype), dg and dbeta written (fp32), once each."""
    return (4 * dk + 3 * dv) * io_bytes + 8 * dk + 8


def counted_traffic(path):
    """HBM bytes per launch measured by the rocprofv3 FETCH_SIZE / WRITE_SIZE runs recorded in
    `path` (scaled by a copy kernel of known size), or None when the kernel sources have changed
    since those counters were taken."""
    import hashlib

    try:
        rec = json.load(open(path))
        src = b"".join(open(os.path.join(ROOT, f), "rb").read() for f in rec["sources"])
    except (OSError, ValueError, KeyError):
        return None
    if hashlib.sha256(src).hexdigest() != rec.get("source_sha256"):
        return None
    return rec["traffic_bytes_per_launch"]


def counted_mfma(path, workload, us_per_call):
    """MFMA evidence of one prefill call from the rocprofv3 counter record in `path` (per kernel:
    MFMA busy %, executed MFMA flops; see profiles/): the executed MFMA flops per call, their rate
    over the measured call time as a fraction of the bf16 peak, and the MFMA busy % weighted by
    each kernel's traced duration.  None when the kernel sources have changed since."""
    import hashlib

    try:
        rec = json.load(open(path))
        src = b"".join(open(os.path.join(ROOT, f), "rb").read() for f in rec["sources"])
        ks = rec["workloads"][workload]
    except (OSError, ValueError, KeyError):
        return None
    if hashlib.sha256(src).hexdigest() != rec.get("source_sha256"):
        return None
    flops = sum(k["mfma_flops_bf16"] + k["mfma_flops_f32"] for k in ks.values())
    t = sum(k["us"] for k in ks.values())
    return {"executed_mfma_flops": flops,
            "executed_mfma_frac": flops / (us_per_call * 1e-6) / (BF16_PEAK_TFLOPS * 1e12),
            "mfma_busy_frac": sum(k["us"] * k["mfma_busy_pct"] for k in ks.values()) / t / 100.0,
            "per_kernel_mfma_busy_pct": {n: k["mfma_busy_pct"] for n, k in ks.items()}}


def counted_prefill_traffic(path, workload, us_per_call, algorithmic_bytes):
    """HBM bytes of one prefill call from the rocprofv3 FETCH_SIZE / WRITE_SIZE record in `path`
    (per kernel, scaled by a copy kernel of known size): bytes per call, their ratio to the
    algorithmic bytes and their rate over the measured call time.  None when the kernel sources
    have changed since the counters were taken."""
    import hashlib

    try:
        rec = json.load(open(path))
        src = b"".join(open(os.path.join(ROOT, f), "rb").read() for f in rec["sources"])
        wl = rec["workloads"][workload]
    except (OSError, ValueError, KeyError):
        return None
    if hashlib.sha256(src).hexdigest() != rec.get("source_sha256"):
        return None
    b = wl["bytes_per_call"]
    return {"bytes_per_call": b, "ratio_to_algorithmic": b / algorithmic_bytes,
            "GBs_at_call_time": b / (us_per_call * 1e-6) / 1e9,
            "per_kernel_bytes": {n: k["fetch_bytes"] + k["write_bytes"]
                                 for n, k in wl["per_kernel"].items()}}


def time_loop(fn, steps, sync):
    """Runs fn(i) for i in range(steps) with HIP events around every call on the current
    stream; returns (total elapsed seconds, mean per-call seconds)."""
    import torch

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    sync()
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record()
        fn(i)
        ends[i].record()
    sync()
    total = time.perf_counter() - t0
    per = sum(s.elapsed_time(e) for s, e in zip(starts, ends)) / steps / 1e3
    return total, per


def bench_decode(args, dev, log):
    import torch

    import kda_gated_delta_rule_amd as kda
    import kda_workloads as W
    from kda_gated_delta_rule_amd import ops

    cfg = W.DECODE
    x = W.decode(seed=0)
    N, H, dk, dv, ns = cfg["N"], cfg["H"], cfg["dk"], cfg["dv"], cfg["num_slots"]
    pool = x["pool"].to(dev)
    q, k, v, g, beta = (x[n].to(dev) for n in ("q", "k", "v", "g", "beta"))
    o = torch.empty_like(q)
    # 8 disjoint 64-slot sets covering the pool; set 0 is the workload's own slot set
    rest = [s for s in torch.randperm(ns, generator=torch.Generator().manual_seed(1)).tolist()
            if s not in set(x["slot_idx"].tolist())]
    sets = [x["slot_idx"]] + [torch.tensor(rest[i * N:(i + 1) * N], dtype=torch.int32)
                              for i in range(ns // N - 1)]
    sets = [s.to(dev) for s in sets]

    def step(i):
        kda.decode_step(q, k, v, g, beta, pool, sets[i % len(sets)], o=o)

    # Decode runs as a captured HIP graph (as serving engines run it): the warmup graph
    # holds exactly `warmup` steps, the timed graph exactly `steps` steps.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for n in (args.warmup, args.steps):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for i in range(n):
                step(i)
        graphs.append(gr)
    if args.warmup:
        graphs[0].replay()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    graphs[1].replay()
    ev1.record()
    torch.cuda.synchronize()
    total = time.perf_counter() - t0
    per = ev0.elapsed_time(ev1) / 1e3 / args.steps  # HIP-event time per launch
    updates = N * H
    bpu = decode_bytes_per_update(dk, dv, 2)
    achieved = updates * bpu / per / 1e9
    log("decode (graph): %.2f us/step wall, %.2f us/launch (events), %.3f GB/s algorithmic"
        % (total / args.steps * 1e6, per * 1e6, achieved))
    # the floor of the same state traffic: kda_diag_state_stream over the same slot sets, the
    # decode kernel's access pattern with no token inputs or arithmetic, timed the same way
    gd = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gd):
        for i in range(args.steps):
            ops.diag_state_stream(pool, sets[i % len(sets)])
    gd.replay()
    torch.cuda.synchronize()
    ev0.record()
    gd.replay()
    ev1.record()
    torch.cuda.synchronize()
    per_pat = ev0.elapsed_time(ev1) / 1e3 / args.steps
    state_bytes = updates * 2 * dk * dv * 4
    log("state traffic floor (same pattern, no compute): %.2f us/launch, %.0f GB/s; decode at %.1f%% of it"
        % (per_pat * 1e6, state_bytes / per_pat / 1e9, 100 * per_pat / per))
    pattern = {"kernel": "kda_diag_state_stream (the decode kernel's state loads and stores, no inputs or arithmetic)",
               "us_per_launch": per_pat * 1e6, "state_bytes": state_bytes,
               "GBs": state_bytes / per_pat / 1e9, "decode_speed_vs_floor": per_pat / per}
    return dict(total=total, per=per, updates=updates, bytes_per_update=bpu, achieved=achieved,
                inputs=x, pattern=pattern)


def bench_mtp(args, dev, log, T):
    """Multi-token commit (MTP decode: T tokens per sequence, state updated in place) on the
    decode workload's pool and sequences, the 8 disjoint slot sets in turn, replayed from a
    captured HIP graph."""
    import torch

    import kda_gated_delta_rule_amd as kda
    import kda_workloads as W

    cfg = W.DECODE
    x = W.decode(seed=0, T=T)
    N, H, dk, dv, ns = cfg["N"], cfg["H"], cfg["dk"], cfg["dv"], cfg["num_slots"]
    pool = x["pool"].to(dev)
    q, k, v, g, beta = (x[n].to(dev) for n in ("q", "k", "v", "g", "beta"))
    o = torch.empty_like(q)
    rest = [s for s in torch.randperm(ns, generator=torch.Generator().manual_seed(1)).tolist()
            if s not in set(x["slot_idx"].tolist())]
    sets = [x["slot_idx"]] + [torch.tensor(rest[i * N:(i + 1) * N], dtype=torch.int32)
                              for i in range(ns // N - 1)]
    sets = [st.to(dev) for st in sets]

    def step(i):
        kda.decode_step(q, k, v, g, beta, pool, sets[i % len(sets)], o=o)

    iters = max(len(sets), args.steps // 4)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        for i in range(iters):
            step(i)
    gr.replay()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    gr.replay()
    ev1.record()
    torch.cuda.synchronize()
    per = ev0.elapsed_time(ev1) / 1e3 / iters
    byts = N * H * mtp_bytes_per_head(dk, dv, T, 2)
    gbs = byts / per / 1e9
    log("MTP commit T = %d: %.2f us/call (graph), %.3g sequence-tokens/s, %.1f GB/s (%.1f%% HBM)"
        % (T, per * 1e6, N * T / per, gbs, 100 * gbs / HBM_PEAK_GBS))
    return {"workload": "mtp_commit_N%d_T%d_H%d_d%d" % (N, T, H, dk), "us_per_call": per * 1e6,
            "timing": "graph replay of %d calls, %d disjoint slot sets in turn" % (iters, len(sets)),
            "sequence_tokens_per_s": N * T / per, "algorithmic_bytes": byts, "achieved_GBs": gbs,
            "hbm_frac": gbs / HBM_PEAK_GBS}


def bench_verify_replay(args, dev, log):
    import torch

    import kda_gated_delta_rule_amd as kda
    import kda_workloads as W

    x = W.verify(seed=0)
    N, T, H, dk, dv = x["q"].shape[0], x["q"].shape[1], x["q"].shape[2], 128, 128
    ns = x["pool"].shape[0]
    pool = x["pool"].to(dev)
    q, k, v, g, beta = (x[n].to(dev) for n in ("q", "k", "v", "g", "beta"))
    acc = x["accepted"].to(dev)
    # disjoint N-slot sets covering the pool (1 GiB, more than the 256 MB Infinity Cache), one
    # per step in turn, so the state is read from HBM; set 0 is the workload's own slot set
    rest = [s for s in torch.randperm(ns, generator=torch.Generator().manual_seed(2)).tolist()
            if s not in set(x["slot_idx"].tolist())]
    sets = [x["slot_idx"]] + [torch.tensor(rest[i * N:(i + 1) * N], dtype=torch.int32)
                              for i in range(ns // N - 1)]
    sets = [st.to(dev) for st in sets]
    rec = torch.empty(N, T, H, 2 * dk + dv, device=dev)
    o = torch.empty_like(q)
    pool_bytes = dk * dv * 4

    def step(i):
        sl = sets[i % len(sets)]
        kda.decode_step(q, k, v, g, beta, pool, sl, o=o, records=rec)
        kda.replay_commit(pool, sl, rec, acc)

    iters = max(len(sets), args.steps // 4)
    for i in range(3):
        step(i)
    _, per_eager = time_loop(step, iters, torch.cuda.synchronize)
    # replayed from one captured HIP graph, as the decode step
    gr = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(gr):
        for i in range(iters):
            step(i)
    gr.replay()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    gr.replay()
    ev1.record()
    torch.cuda.synchronize()
    per = ev0.elapsed_time(ev1) / 1e3 / iters
    acc_sum = int(x["accepted"].sum())
    verify_bytes = N * H * (pool_bytes + T * ((2 * dk + dv) * 2 + dk * 4 + 4 + dv * 2 +
                                               (2 * dk + dv) * 4))
    commit_bytes = N * H * 2 * pool_bytes + acc_sum * H * (2 * dk + dv) * 4
    gbs = (verify_bytes + commit_bytes) / per / 1e9
    log("verify+replay: %.2f us/step (graph; %.2f us eager), %.1f GB/s" % (per * 1e6, per_eager * 1e6, gbs))
    return {"workload": W.VERIFY["name"], "us_per_step": per * 1e6,
            "timing": "graph replay of %d steps, %d disjoint slot sets in turn" % (iters, len(sets)),
            "us_per_step_eager": per_eager * 1e6,
            "sequence_tokens_per_s": N * T / per, "accepted_tokens": acc_sum,
            "algorithmic_bytes": verify_bytes + commit_bytes, "achieved_GBs": gbs,
            "hbm_frac": gbs / HBM_PEAK_GBS}


def bench_front(args, dev, log, prefill_us):
    """The input front fused into the kernels (kda_decode_step_front, kda_chunk_prefill_front:
    width-4 convolution with SiLU, gate and beta processing, the convolution state kept in the
    slots).  Decode on the decode workload's pool and sequences (8 disjoint slot sets in turn,
    graph replay), beside the same front run as separate torch operators followed by
    kda_decode_step (the unfused pipeline); prefill on the T = 8192 x H = 32 workload beside the
    plain prefill's graph time."""
    import torch
    import torch.nn.functional as Fn

    import kda_gated_delta_rule_amd as kda
    import kda_workloads as W

    cfg = W.DECODE
    x = W.decode_front(seed=0)
    N, H, dk, dv, ns = cfg["N"], cfg["H"], cfg["dk"], cfg["dv"], cfg["num_slots"]
    width = x["conv_q"].shape[-1]
    pool = x["pool"].to(dev)
    cs = x["conv_state"].to(dev)
    q, k, v, z, b = (x[n].to(dev) for n in ("q", "k", "v", "g", "beta"))
    fr = {n: x[n].to(dev) for n in ("gate_scale", "conv_q", "conv_k", "conv_v")}
    o = torch.empty_like(q)
    rest = [s for s in torch.randperm(ns, generator=torch.Generator().manual_seed(1)).tolist()
            if s not in set(x["slot_idx"].tolist())]
    sets = [x["slot_idx"]] + [torch.tensor(rest[i * N:(i + 1) * N], dtype=torch.int32)
                              for i in range(ns // N - 1)]
    sets = [st.to(dev) for st in sets]
    wcat = torch.cat([fr["conv_q"], fr["conv_k"], fr["conv_v"]], dim=1).permute(0, 2, 1).contiguous()

    def fused(i):
        kda.decode_step_front(q, k, v, z, b, pool, sets[i % len(sets)], conv_state=cs, conv_silu=True,
                              o=o, **fr)

    def unfused(i):
        sl = sets[i % len(sets)]
        sll = sl.long()
        X = torch.cat([cs[sll], torch.cat([q, k, v], dim=-1).permute(0, 2, 1, 3)], dim=2)  # [N, H, W, C]
        y = Fn.silu((X.float() * wcat[None]).sum(2)).to(q.dtype)  # [N, H, C]
        cs[sll] = X[:, :, 1:]
        y = y[:, None]
        g = -fr["gate_scale"][None, None, :, None] * Fn.softplus(z)
        kda.decode_step(y[..., :dk].contiguous(), y[..., dk:2 * dk].contiguous(), y[..., 2 * dk:].contiguous(),
                        g, torch.sigmoid(b), pool, sl, o=o)

    iters = max(len(sets), args.steps // 4)

    def graph_time(step):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(0)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for i in range(iters):
                step(i)
        gr.replay()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record()
        gr.replay()
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / 1e3 / iters

    per = graph_time(fused)
    per_unfused = graph_time(unfused)
    bpu = front_decode_bytes_per_update(dk, dv, width, 2, N)
    gbs = N * H * bpu / per / 1e9
    log("front decode: %.2f us/call fused, %.2f us unfused (torch front + decode_step), %.1f GB/s (%.1f%% HBM)"
        % (per * 1e6, per_unfused * 1e6, gbs, 100 * gbs / HBM_PEAK_GBS))
    dec = {"workload": cfg["name"] + "_front_w%d_silu" % width, "us_per_call": per * 1e6,
           "timing": "graph replay of %d calls, %d disjoint slot sets in turn" % (iters, len(sets)),
           "unfused_us_per_call": per_unfused * 1e6,
           "unfused": "the front as torch operators (gather, convolution, SiLU, softplus, sigmoid, "
                      "state scatter) then kda_decode_step",
           "updates_per_s": N * H / per, "bytes_per_update": bpu, "achieved_GBs": gbs,
           "hbm_frac": gbs / HBM_PEAK_GBS}
    del pool, cs

    y = W.prefill_front(seed=0)
    Tt, H, dk = y["q"].shape
    dv = y["v"].shape[-1]
    ins = two_input_copies(y, dev)
    cu = y["cu_seqlens"].to(dev)
    pool, slots = y["pool"].to(dev), y["slot_idx"].to(dev)
    cs = y["conv_state"].to(dev)
    fr = {n: y[n].to(dev) for n in ("gate_scale", "conv_q", "conv_k", "conv_v")}
    o = torch.empty_like(ins[0][2])
    ws = torch.empty(kda.chunk_prefill_workspace_size(1, Tt, H, dk, dv), dtype=torch.uint8, device=dev)

    def pstep(i):
        qq, kk, vv, zz, bb = ins[i % 2]
        kda.chunk_prefill_front(qq, kk, vv, zz, bb, cu, pool, slots, conv_state=cs, conv_silu=True,
                                h0_from_pool=False, o=o, workspace=ws, **fr)

    iters = max(5, args.steps // 10)
    pper = graph_time(pstep)
    th = Tt * H
    byts = th * prefill_bytes_per_token_head(dk, dv, 2)
    log("front prefill %s: %.1f us/call (graph), plain prefill %.1f us" % (W.PREFILL["name"], pper * 1e6, prefill_us))
    pre = {"workload": W.PREFILL["name"] + "_front_w%d_silu" % width, "us_per_call": pper * 1e6,
           "timing": "graph replay of %d calls, two input copies in turn" % iters,
           "plain_us_per_call": prefill_us, "overhead": pper * 1e6 / prefill_us - 1.0,
           "tokens_per_s": Tt / pper, "hbm_frac": byts / pper / 1e9 / HBM_PEAK_GBS}
    return {"decode": dec, "prefill": pre}


def two_input_copies(y, dev):
    """The prefill inputs (q, k, v, g, beta) twice on the device: consecutive calls alternate
    between the copies, so no call finds its inputs in the Infinity Cache from the call before."""
    first = tuple(y[n].to(dev) for n in ("q", "k", "v", "g", "beta"))
    return [first, tuple(t.clone() for t in first)]


def bench_prefill(args, dev, log, which):
    import torch

    import kda_gated_delta_rule_amd as kda
    import kda_workloads as W

    if which == "prefill":
        y, name, h0 = W.prefill(seed=0), W.PREFILL["name"], False
    else:
        y, name, h0 = W.prefill_long(seed=0), W.VARLEN["name"], True
    Tt, H, dk = y["q"].shape
    dv = y["v"].shape[-1]
    ns = y["cu_seqlens"].shape[0] - 1
    ins = two_input_copies(y, dev)
    cu = y["cu_seqlens"].to(dev)
    pool, slots = y["pool"].to(dev), y["slot_idx"].to(dev)
    o = torch.empty_like(ins[0][2])
    ws = torch.empty(kda.chunk_prefill_workspace_size(ns, Tt, H, dk, dv), dtype=torch.uint8,
                     device=dev)

    def step(i):
        q, k, v, g, beta = ins[i % 2]
        kda.chunk_prefill(q, k, v, g, beta, cu, pool, slots, h0_from_pool=h0, o=o, workspace=ws)

    iters = max(5, args.steps // 10)
    for i in range(2):
        step(i)
    _, per_eager = time_loop(step, iters, torch.cuda.synchronize)
    # As decode: the calls replayed from one captured HIP graph (as serving engines run the
    # prefill), HIP-event time per call.
    gr = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(gr):
        for i in range(iters):
            step(i)
    gr.replay()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    gr.replay()
    ev1.record()
    torch.cuda.synchronize()
    per = ev0.elapsed_time(ev1) / 1e3 / iters
    th = Tt * H
    flops = th * prefill_flops_per_token_head(dk, dv)
    byts = th * prefill_bytes_per_token_head(dk, dv, 2)
    tflops = flops / per / 1e12
    gbs = byts / per / 1e9
    log("%s: %.1f us/call (graph; %.1f us eager), %.3g tokens/s, %.1f TFLOP/s (%.1f%% MFMA), "
        "%.0f GB/s (%.1f%% HBM)" % (name, per * 1e6, per_eager * 1e6, Tt / per, tflops,
                                    100 * tflops / BF16_PEAK_TFLOPS, gbs, 100 * gbs / HBM_PEAK_GBS))
    return {"workload": name, "us_per_call": per * 1e6,
            "timing": "graph replay of %d calls, two input copies in turn" % iters,
            "us_per_call_eager": per_eager * 1e6, "tokens_per_s": Tt / per,
            "token_heads_per_s": th / per, "algorithmic_flops": flops, "algorithmic_bytes": byts,
            "achieved_TFLOPs": tflops, "mfma_frac": tflops / BF16_PEAK_TFLOPS,
            "achieved_GBs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
            "binding_roofline_frac": max(tflops / BF16_PEAK_TFLOPS, gbs / HBM_PEAK_GBS),
            "mfma_counters": counted_mfma(os.path.join(ROOT, "profiles", "prefill_mfma_counters.json"),
                                          name, per * 1e6),
            "traffic": counted_prefill_traffic(os.path.join(ROOT, "profiles", "prefill_traffic.json"),
                                               name, per * 1e6, byts)}


def bench_backward(args, dev, log):
    """The chunked backward (kda_chunk_backward) on the prefill workload's shape (T = 8192,
    H = 32, dk = dv = 128, bf16, zero initial state, random output and final-state gradients):
    eager time per call over alternating input copies; every product runs on fp32 MFMA, so the
    compute roofline is the fp32 matrix peak."""
    import torch

    import kda_gated_delta_rule_amd as kda
    import kda_workloads as W

    y = W.prefill(seed=0)
    Tt, H, dk = y["q"].shape
    dv = y["v"].shape[-1]
    gen = torch.Generator().manual_seed(1)
    do = torch.randn(Tt, H, dv, generator=gen).to(torch.bfloat16).to(dev)
    dht = torch.randn(1, H, dk, dv, generator=gen).to(dev)
    ins = two_input_copies(y, dev)
    cu = y["cu_seqlens"].to(dev)
    ws = torch.empty(kda.chunk_backward_workspace_size(1, Tt, H, dk, dv), dtype=torch.uint8, device=dev)

    def step(i):
        q, k, v, g, beta = ins[i % 2]
        kda.chunk_backward(q, k, v, g, beta, cu, do, dht=dht, workspace=ws)

    iters = max(4, args.steps // 20)
    for i in range(2):
        step(i)
    _, per = time_loop(step, iters, torch.cuda.synchronize)
    th = Tt * H
    flops = th * backward_flops_per_token_head(dk, dv)
    byts = th * backward_bytes_per_token_head(dk, dv, 2)
    tflops = flops / per / 1e12
    gbs = byts / per / 1e9
    log("%s backward: %.1f us/call (eager), %.3g tokens/s, %.1f TFLOP/s (%.1f%% of fp32 MFMA), "
        "%.0f GB/s (%.1f%% HBM)" % (W.PREFILL["name"], per * 1e6, Tt / per, tflops,
                                    100 * tflops / FP32_PEAK_TFLOPS, gbs, 100 * gbs / HBM_PEAK_GBS))
    return {"workload": W.PREFILL["name"], "us_per_call": per * 1e6,
            "timing": "eager, %d calls, two input copies in turn" % iters,
            "tokens_per_s": Tt / per, "token_heads_per_s": th / per,
            "algorithmic_flops": flops, "algorithmic_bytes": byts, "achieved_TFLOPs": tflops,
            "fp32_mfma_frac": tflops / FP32_PEAK_TFLOPS, "achieved_GBs": gbs,
            "hbm_frac": gbs / HBM_PEAK_GBS,
            "binding_roofline_frac": max(tflops / FP32_PEAK_TFLOPS, gbs / HBM_PEAK_GBS)}


def bench_prefill_snapshots(args, dev, log, plain_us):
    """The T = 8192 x H = 32 prefill with prefix-cache snapshots every 1,024 tokens (8 states
    per head written to extra pool slots); reports the eager time per call and the cost over
    the plain call timed the same way."""
    import torch

    import kda_gated_delta_rule_amd as kda
    import kda_workloads as W

    y = W.prefill(seed=0)
    Tt, H, dk = y["q"].shape
    dv = y["v"].shape[-1]
    every = 1024
    nsnap = Tt // every
    ins = two_input_copies(y, dev)
    cu = y["cu_seqlens"].to(dev)
    pool = torch.zeros(1 + nsnap, H, dk, dv, device=dev)
    slots = torch.zeros(1, dtype=torch.int32, device=dev)
    snap = torch.arange(1, 1 + nsnap, dtype=torch.int32, device=dev).reshape(1, nsnap)
    o = torch.empty_like(ins[0][2])
    ws = torch.empty(kda.chunk_prefill_workspace_size(1, Tt, H, dk, dv), dtype=torch.uint8,
                     device=dev)

    def step(i):
        q, k, v, g, beta = ins[i % 2]
        kda.chunk_prefill(q, k, v, g, beta, cu, pool, slots, h0_from_pool=False, o=o, workspace=ws,
                          snapshot_every=every, snapshot_slots=snap)

    iters = max(5, args.steps // 10)
    for i in range(2):
        step(i)
    total, per = time_loop(step, iters, torch.cuda.synchronize)
    log("%s with %d snapshots per head: %.1f us/call eager (plain %.1f us eager)"
        % (W.PREFILL["name"], nsnap, per * 1e6, plain_us))
    return {"workload": W.PREFILL["name"] + "_snapshots_every1024", "snapshot_every": every,
            "snapshots_per_head": nsnap, "snapshot_bytes": nsnap * H * dk * dv * 4,
            "us_per_call": per * 1e6, "plain_us_per_call": plain_us,
            "overhead": per * 1e6 / plain_us - 1.0}


def bench_copy(dev, log):
    """Reference device copy of 1 GiB (fp32), also the known-size kernel that scales the
    FETCH_SIZE / WRITE_SIZE counters."""
    import torch

    n = 1 << 28
    src = torch.ones(n, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    total, per = time_loop(lambda i: dst.copy_(src), 10, torch.cuda.synchronize)
    gbs = 2 * n * 4 / per / 1e9
    log("copy 1 GiB: %.1f us, %.0f GB/s (read + write)" % (per * 1e6, gbs))
    del src, dst
    return {"bytes_read": n * 4, "bytes_written": n * 4, "us": per * 1e6, "GBs": gbs}


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo, or None where it is not readable."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(x, log, budget_s=10.0, prefill_budget_s=5.0):
    """fp64 oracle on the decode workload's step (all 64 x 32 (sequence, head) updates),
    repeated until about budget_s seconds of wall time."""
    import numpy as np

    from oracle import kda_oracle as O

    f = lambda t: t.float().numpy().astype(np.float64)
    sl = x["slot_idx"].long()
    ins = [f(x[n]) for n in ("q", "k", "v", "g", "beta")]
    h0 = f(x["pool"][sl])
    threads = O.default_threads()
    reps, t0 = 0, time.perf_counter()
    while True:
        O.decode(*ins, h0, nthreads=threads)
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    n_upd = x["q"].shape[0] * x["q"].shape[2] * reps
    log("cpu oracle: %d decode steps in %.1f s on %d threads" % (reps, el, threads))
    return {"value": n_upd / el, "unit": "state-updates/s", "cores": threads, "kind": "oracle",
            "sample": "%d full decode steps of the workload (64 sequences x 32 heads, 1 token, "
                      "dk = dv = 128), fp64, %.1f s" % (reps, el),
            "cpu": cpu_model() or platform.processor() or platform.machine(),
            "prefill": cpu_prefill_baseline(log, threads, prefill_budget_s)}


def cpu_prefill_baseline(log, threads, budget_s):
    """fp64 oracle (the token recurrence, its plain definition) on whole calls of the
    T = 8192 x H = 32 prefill workload, repeated until about budget_s seconds."""
    import numpy as np

    import kda_workloads as W
    from oracle import kda_oracle as O

    y = W.prefill(seed=0)
    f = lambda t: t.float().numpy().astype(np.float64)
    ins = [f(y[n]) for n in ("q", "k", "v", "g", "beta")]
    cu = y["cu_seqlens"].numpy().astype(np.int64)
    reps, t0 = 0, time.perf_counter()
    while True:
        O.recurrent(*ins, cu, nthreads=threads)
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    tokens = int(cu[-1]) * reps
    log("cpu oracle: %d prefill calls (%s) in %.1f s on %d threads" % (reps, W.PREFILL["name"], el,
                                                                       threads))
    return {"value": tokens / el, "unit": "tokens/s", "workload": W.PREFILL["name"],
            "sample": "%d full calls of the workload through the token recurrence, fp64, %.1f s"
                      % (reps, el)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--decode-only", action="store_true",
                    help="measure only the decode step and the copy reference (for counter runs)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="measure only the copy reference and the two prefill workloads (for counter "
                         "runs); prints their figures without the headline metric")
    ap.add_argument("--verify-only", action="store_true",
                    help="measure only the copy reference and verify + replay (for counter runs); "
                         "prints their figures without the headline metric")
    ap.add_argument("--backward-only", action="store_true",
                    help="measure only the chunked backward (for counter and trace runs)")
    ap.add_argument("--front-only", action="store_true",
                    help="measure only the fused input front (decode and prefill)")
    ap.add_argument("--quiet", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build measures one GPU only (--gpus 1); the KDA kernels shard "
              "by head and sequence with no exchange, and no multi-GPU run is provided.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import kda_gated_delta_rule_amd as kda

    log = (lambda m: None) if args.quiet else (lambda m: print("[bench] " + m, file=sys.stderr,
                                                               flush=True))
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(2)
    kda.load()
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(0)
    device = {"name": props.name, "arch": getattr(props, "gcnArchName", None),
              "compute_units": props.multi_processor_count,
              "memory_bytes": props.total_memory}
    log("device: %s (%s, %d CUs)" % (props.name, device["arch"], props.multi_processor_count))

    if args.prefill_only:
        extra = {"copy_reference": bench_copy(dev, log),
                 "prefill": bench_prefill(args, dev, log, "prefill"),
                 "prefill_varlen": bench_prefill(args, dev, log, "varlen")}
        print(json.dumps({"mode": "prefill-only", "extra": extra}))
        return

    if args.front_only:
        pre = bench_prefill(args, dev, log, "prefill")
        print(json.dumps({"mode": "front-only", "extra": {"prefill": pre,
                                                          "front": bench_front(args, dev, log, pre["us_per_call"])}}))
        return

    if args.backward_only:
        print(json.dumps({"mode": "backward-only", "extra": {"backward": bench_backward(args, dev, log)}}))
        return

    if args.verify_only:
        extra = {"copy_reference": bench_copy(dev, log),
                 "verify_replay": bench_verify_replay(args, dev, log)}
        print(json.dumps({"mode": "verify-only", "extra": extra}))
        return

    dec = bench_decode(args, dev, log)
    value = dec["updates"] * args.steps / dec["total"]
    extra = {"copy_reference": bench_copy(dev, log), "decode_state_traffic_floor": dec["pattern"]}
    if not args.decode_only:
        extra["verify_replay"] = bench_verify_replay(args, dev, log)
        extra["mtp_commit_T2"] = bench_mtp(args, dev, log, 2)
        extra["mtp_commit_T4"] = bench_mtp(args, dev, log, 4)
        extra["prefill"] = bench_prefill(args, dev, log, "prefill")
        extra["prefill_varlen"] = bench_prefill(args, dev, log, "varlen")
        extra["prefill_snapshots"] = bench_prefill_snapshots(args, dev, log,
                                                             extra["prefill"]["us_per_call_eager"])
        extra["backward"] = bench_backward(args, dev, log)
        extra["front"] = bench_front(args, dev, log, extra["prefill"]["us_per_call"])
    cpu = None if args.decode_only else cpu_baseline(dec["inputs"], log)

    import kda_workloads as W

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "state-updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dec["total"] / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "device": device,
        "config": {"workload": W.DECODE["name"], "num_slots": 512, "sequences": 64, "tokens": 1,
                   "heads": 32, "dk": 128, "dv": 128, "io_dtype": "bf16", "state_dtype": "fp32",
                   "slot_rotation": "8 disjoint sets of 64 slots (1 GiB pool)",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": dec["achieved"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": dec["achieved"] / HBM_PEAK_GBS,
                     "traffic": counted_traffic(os.path.join(
                         ROOT, "profiles", "decode_pool512_N64_H32_d128_traffic.json")),
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                                     "scaled by a 1 GiB copy)",
                     "kernel": "decode_kernel<dk=128,dv=128,BV=128,T=1,bf16,commit,512 threads>",
                     "bytes_per_update": dec["bytes_per_update"],
                     "updates_per_launch": dec["updates"],
                     "avg_launch_us": dec["per"] * 1e6},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
