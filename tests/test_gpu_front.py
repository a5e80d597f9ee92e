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


@pytest.mark.parametrize("T", [2, 3, 5, 9])
def test_multi_token_commit(T):
    """T tokens in one call (fewer than, equal to and more than the width's 3 earlier inputs;
    more than one 4-token LDS block)."""
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
