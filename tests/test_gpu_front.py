"""GPU parity of the input front (ShortConv, gate and beta processing) fused into the decode
kernel, against the fp64 front reference (oracle/kda_front.py) followed by the fp64 token
recurrence (oracle/kda_oracle.c), through the C ABI.  The convolution state after the call is
a copy of raw inputs and is compared bit for bit; o and the recurrent state by relative L2
(whole tensor and worst (sequence, head)) at 1e-4 for fp32 inputs and 1e-2 for bf16."""
import numpy as np
import pytest
import torch

import kda_gated_delta_rule_amd as kda
import kda_workloads as W
from oracle import kda_front as F
from oracle import kda_oracle as O
from tests._util import announce, f64, need_gpu, rel_l2, worst_decode, worst_state

pytestmark = pytest.mark.gpu

FRONT = ("gate_scale", "conv_q", "conv_k", "conv_v")


def run_decode_front(x, dev, silu=True):
    pool = x["pool"].to(dev)
    cs = x["conv_state"].to(dev) if x["conv_q"].shape[-1] > 1 else None
    o = kda.decode_step_front(*(x[n].to(dev) for n in ("q", "k", "v", "g", "beta")), pool,
                              x["slot_idx"].to(dev), conv_state=cs, conv_silu=silu,
                              **{n: x[n].to(dev) for n in FRONT})
    torch.cuda.synchronize()
    return o, pool, cs


def oracle_decode_front(x, silu=True):
    """The front over each sequence's T tokens (state from its slot), then the recurrence."""
    N, T, H, dk = x["q"].shape
    dv = x["v"].shape[-1]
    sl = x["slot_idx"].long()
    live = sl >= 0
    W_ = x["conv_q"].shape[-1]
    flat = lambda t: f64(t).reshape((N * T,) + tuple(t.shape[2:]))
    cu = np.arange(N + 1) * T
    st0 = f64(x["conv_state"])[sl.clamp(min=0).numpy()] if W_ > 1 else None
    q, k, v, g, beta, st = F.front(flat(x["q"]), flat(x["k"]), flat(x["v"]), flat(x["g"]),
                                   flat(x["beta"]), cu, f64(x["gate_scale"]), f64(x["conv_q"]),
                                   f64(x["conv_k"]), f64(x["conv_v"]), st0, use_silu=silu)
    unflat = lambda a: a.reshape((N, T) + a.shape[1:])
    o, h, _ = O.decode(unflat(q), unflat(k), unflat(v), unflat(g), unflat(beta), f64(x["pool"][sl]))
    return o, h, st, live.numpy()


def check(x, dev, tol, label, silu=True):
    announce(label)
    o, pool, cs = run_decode_front(x, dev, silu)
    o_ref, h_ref, st_ref, live = oracle_decode_front(x, silu)
    sl = x["slot_idx"].long().numpy()
    o = f64(o)
    h = f64(pool.cpu())[sl[live]]
    e = dict(o=rel_l2(o[live], o_ref[live]), o_worst=worst_decode(o[live], o_ref[live]),
             h=rel_l2(h, h_ref[live]), h_worst=worst_state(h, h_ref[live]))
    announce("%s rel-L2 o %.3g (worst seq/head %.3g), state %.3g (worst %.3g)"
             % (label, e["o"], e["o_worst"], e["h"], e["h_worst"]))
    for name, val in e.items():
        assert val <= tol, (name, val, tol)
    assert np.all(o[~live] == 0)
    if cs is not None:
        got = cs.cpu()
        want = x["conv_state"].clone()
        want[torch.as_tensor(sl[live])] = torch.as_tensor(st_ref[live]).to(want.dtype)
        assert torch.equal(got, want), "convolution state"  # live slots updated, others kept
    # pool slots no sequence uses are untouched
    others = torch.ones(x["pool"].shape[0], dtype=torch.bool)
    others[torch.as_tensor(sl[live])] = False
    assert torch.equal(pool.cpu()[others], x["pool"][others])


def test_decode_workload_shape_bf16():
    """The decode workload's shape (512 slots, 64 sequences x 32 heads, d = 128, bf16), T = 1,
    width 4 with SiLU."""
    dev = need_gpu()
    x = W.decode_front(seed=1)
    check(x, dev, 1e-2, "front decode bf16 N64 H32 d128 T1")


@pytest.mark.parametrize("T", [2, 3, 5, 8])
def test_multi_token_commit(T):
    """T tokens in one call (fewer than, equal to and more than the width's 3 earlier inputs,
    up to the front's limit of 8)."""
    dev = need_gpu()
    x = W.decode_front(seed=2 + T, N=8, T=T, H=4, num_slots=16)
    check(x, dev, 1e-2, "front decode bf16 T=%d" % T)


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("width,silu", [(1, False), (2, True), (4, False)])
def test_fp32_shapes_and_widths(dk, dv, width, silu):
    dev = need_gpu()
    x = W.decode_front(seed=20 + width, N=6, T=3, H=3, dk=dk, dv=dv, num_slots=9, width=width,
                       dtype=torch.float32)
    check(x, dev, 1e-4, "front decode fp32 dk=%d dv=%d W=%d silu=%d" % (dk, dv, width, silu), silu)


def test_skipped_sequence_keeps_its_states():
    """A negative slot: zero output; its slot's recurrent and convolution states stay as they
    were (every slot not used by a live sequence is compared bit for bit)."""
    dev = need_gpu()
    x = W.decode_front(seed=30, N=6, T=2, H=2, num_slots=8)
    x["slot_idx"][2] = -1
    x["slot_idx"][5] = -1
    check(x, dev, 1e-2, "front decode with skipped sequences")


def test_two_calls_equal_one():
    """Two T = 2 calls, the convolution and recurrent states carried in the slots, give the
    outputs and states of one T = 4 call."""
    dev = need_gpu()
    x = W.decode_front(seed=40, N=5, T=4, H=2, num_slots=7, dtype=torch.float32)
    o_all, pool_all, cs_all = run_decode_front(x, dev)
    pool = x["pool"].to(dev)
    cs = x["conv_state"].to(dev)
    outs = []
    for part in (slice(0, 2), slice(2, 4)):
        outs.append(kda.decode_step_front(*(x[n][:, part].contiguous().to(dev) for n in ("q", "k", "v", "g", "beta")),
                                          pool, x["slot_idx"].to(dev), conv_state=cs, conv_silu=True,
                                          **{n: x[n].to(dev) for n in FRONT}))
    torch.cuda.synchronize()
    o2 = torch.cat(outs, dim=1)
    assert rel_l2(f64(o2), f64(o_all)) <= 1e-6
    assert rel_l2(f64(pool), f64(pool_all)) <= 1e-6
    assert torch.equal(cs.cpu(), cs_all.cpu())


# ---- prefill -------------------------------------------------------------------------------

def run_prefill_front(y, dev, h0_from_pool=True, silu=True):
    pool = y["pool"].to(dev)
    cs = y["conv_state"].to(dev) if y["conv_q"].shape[-1] > 1 else None
    o = kda.chunk_prefill_front(*(y[n].to(dev) for n in ("q", "k", "v", "g", "beta")),
                                y["cu_seqlens"].to(dev), pool, y["slot_idx"].to(dev), conv_state=cs,
                                conv_silu=silu, h0_from_pool=h0_from_pool,
                                **{n: y[n].to(dev) for n in FRONT})
    torch.cuda.synchronize()
    return o, pool, cs


def oracle_prefill_front(y, h0_from_pool=True, silu=True):
    sl = y["slot_idx"].long()
    W_ = y["conv_q"].shape[-1]
    st0 = f64(y["conv_state"][sl]) if (W_ > 1 and h0_from_pool) else None
    q, k, v, g, beta, st = F.front(*(f64(y[n]) for n in ("q", "k", "v", "g", "beta")),
                                   y["cu_seqlens"].numpy(), f64(y["gate_scale"]), f64(y["conv_q"]),
                                   f64(y["conv_k"]), f64(y["conv_v"]), st0, use_silu=silu)
    h0 = f64(y["pool"][sl]) if h0_from_pool else None
    o, h, _ = O.recurrent(q, k, v, g, beta, y["cu_seqlens"].numpy(), h0=h0)
    return o, h, st


def check_prefill(y, dev, tol, label, h0_from_pool=True, silu=True):
    announce(label)
    o, pool, cs = run_prefill_front(y, dev, h0_from_pool, silu)
    o_ref, h_ref, st_ref = oracle_prefill_front(y, h0_from_pool, silu)
    sl = y["slot_idx"].long()
    cu = y["cu_seqlens"]
    from tests._util import worst_seq_head
    h = f64(pool.cpu()[sl])
    e = dict(o=rel_l2(f64(o), o_ref), o_worst=worst_seq_head(f64(o), o_ref, cu), h=rel_l2(h, h_ref),
             h_worst=worst_state(h, h_ref))
    announce("%s rel-L2 o %.3g (worst seq/head %.3g), state %.3g (worst %.3g)"
             % (label, e["o"], e["o_worst"], e["h"], e["h_worst"]))
    for name, val in e.items():
        assert val <= tol, (name, val, tol)
    if cs is not None:
        got = cs.cpu()
        want = y["conv_state"].clone()
        want[sl] = torch.as_tensor(st_ref).to(want.dtype)
        assert torch.equal(got, want), "convolution state"


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64), (64, 128)])
def test_prefill_bf16_varlen(dk, dv):
    """Ragged varlen batch: sequences of 1, 2, 3 and 4 tokens (shorter than and equal to the
    width), chunk tails, an empty sequence, h0 and convolution states from the slots."""
    dev = need_gpu()
    y = W.prefill_front(seed=50, seqlens=(1, 2, 3, 4, 63, 64, 65, 0, 200, 777), H=3, dk=dk, dv=dv,
                        num_slots=12, h0_std=0.05)
    check_prefill(y, dev, 1e-2, "front prefill bf16 varlen dk=%d dv=%d" % (dk, dv))


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128)])
@pytest.mark.parametrize("width,silu,h0", [(4, True, True), (2, False, True), (1, True, True), (3, True, False)])
def test_prefill_fp32(dk, dv, width, silu, h0):
    """fp32 through several segments (sequences longer than 1,024 tokens), every width, with and
    without the slots' initial states; <= 1e-4."""
    dev = need_gpu()
    y = W.prefill_front(seed=51 + width, seqlens=(2100, 3, 0, 130), H=2, dk=dk, dv=dv, num_slots=5,
                        h0_std=0.05, width=width, dtype=torch.float32)
    check_prefill(y, dev, 1e-4, "front prefill fp32 dk=%d dv=%d W=%d silu=%d h0=%d" % (dk, dv, width, silu, h0),
                  h0_from_pool=h0, silu=silu)


def test_prefill_workload_shape():
    """The chunked prefill workload's shape (T = 8192, H = 32, d = 128, bf16, zero initial
    states), width 4 with SiLU, every head against the oracle."""
    dev = need_gpu()
    y = W.prefill_front(seed=52, seqlens=(8192,), H=32, dk=128, dv=128)
    check_prefill(y, dev, 1e-2, "front prefill bf16 T8192 H32", h0_from_pool=False)


def test_prefill_then_decode_continues_the_sequence():
    """A prefill of 70 tokens then a 3-token decode step on the same slots equals one prefill
    of 73 tokens (outputs of the last 3 tokens, recurrent and convolution states), fp32."""
    dev = need_gpu()
    y = W.prefill_front(seed=53, seqlens=(73, 73), H=2, dk=64, dv=64, num_slots=3, h0_std=0.05,
                        dtype=torch.float32)
    o_all, pool_all, cs_all = run_prefill_front(y, dev)
    # first 70 tokens of each sequence through the prefill, the last 3 through the decode
    idx = torch.cat([torch.arange(0, 70), torch.arange(73, 143)])
    tail = torch.cat([torch.arange(70, 73), torch.arange(143, 146)])
    y1 = dict(y)
    for n in ("q", "k", "v", "g", "beta"):
        y1[n] = y[n][idx].contiguous()
    y1["cu_seqlens"] = torch.tensor([0, 70, 140], dtype=torch.int32)
    _, pool, cs = run_prefill_front(y1, dev)
    shp = lambda t: t[tail].reshape((2, 3) + tuple(t.shape[1:])).contiguous().to(dev)
    o_dec = kda.decode_step_front(*(shp(y[n]) for n in ("q", "k", "v", "g", "beta")), pool,
                                  y["slot_idx"].to(dev), conv_state=cs, conv_silu=True,
                                  **{n: y[n].to(dev) for n in FRONT})
    torch.cuda.synchronize()
    o_ref = o_all[tail.to(dev)].reshape(2, 3, *o_all.shape[1:])
    assert rel_l2(f64(o_dec), f64(o_ref)) <= 1e-5
    assert rel_l2(f64(pool), f64(pool_all)) <= 1e-5
    assert torch.equal(cs.cpu(), cs_all.cpu())
