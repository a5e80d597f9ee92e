"""GPU parity of the chunked prefill on inputs at the edges of its arithmetic, against the fp64
token recurrence (oracle), through the C ABI:

- cancellation: q.k products that cancel (queries orthogonal to the keys of their sequence up to
  the bf16 rounding), without the L2 norm, with per-channel, per-token (channel-constant) and
  zero gates, in 1-, 2- and 64-token sequences; and seed 631 of the random sweep (a one-token
  sequence whose q.k cancels).  The outputs are small against |q||k|, so these check that every
  A/P entry is accurate to its own size;
- strong gates: g scaled by 20 and 50 (per-token log-decays of several units, a 64-token chunk
  summing to about -100 and -250), fp32 and bf16, through several chunks and segments;
- weak gates over a long sequence: g around -1e-3, so the state keeps contributions over
  thousands of tokens and the bf16 state operands of the carry accumulate.
Bars: rel-L2 <= 1e-4 (fp32 inputs) and <= 1e-2 (bf16), whole tensor and worst (sequence, head).
"""
import numpy as np
import pytest
import torch

import kda_gated_delta_rule_amd as kda
import kda_workloads as W
from oracle import kda_oracle as O
from tests._util import announce, check_prefill_parity, f64, need_gpu, worst_chunk_head

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "g", "beta")


def run(y, dev, h0_from_pool, use_l2):
    pool = y["pool"].to(dev)
    o = kda.chunk_prefill(*(y[n].to(dev) for n in NAMES), y["cu_seqlens"].to(dev), pool,
                          y["slot_idx"].to(dev), h0_from_pool=h0_from_pool, use_qk_l2norm=use_l2)
    torch.cuda.synchronize()
    sl = y["slot_idx"].long()
    h0 = f64(y["pool"][sl]) if h0_from_pool else None
    o_ref, h_ref, _ = O.recurrent(*(f64(y[n]) for n in NAMES), y["cu_seqlens"].numpy(), h0=h0,
                                  use_qk_l2norm=use_l2)
    return f64(o), o_ref, f64(pool.cpu()[sl]), h_ref


@pytest.mark.parametrize("gate", ["channel", "scalar", "zero"])
@pytest.mark.parametrize("use_l2", [False, True])
def test_cancelling_qk(gate, use_l2):
    """Sequences of 1, 2, 17 and 64 tokens whose queries are orthogonal to all keys so far
    (bf16, dk = dv = 128, H = 4, zero initial state)."""
    dev = need_gpu()
    y = W.cancellation(seed=21, seqlens=(1, 2, 17, 64, 1, 64), H=4, gate=gate)
    o, o_ref, h, h_ref = run(y, dev, h0_from_pool=False, use_l2=use_l2)
    check_prefill_parity(o, o_ref, h, h_ref, y["cu_seqlens"], 1e-2,
                         "cancellation gate=%s l2=%d" % (gate, use_l2))


def test_sweep_seed_631():
    """The random sweep's seed 631: a one-token bf16 sequence without the L2 norm whose q.k is
    -0.053 against |q||k| = 4.36 in one head."""
    dev = need_gpu()
    c = W.sweep_case(631)
    announce("sweep seed 631: %s" % c["desc"])
    o, o_ref, h, h_ref = run(c, dev, h0_from_pool=c["h0_from_pool"], use_l2=c["use_l2"])
    e = check_prefill_parity(o, o_ref, h, h_ref, c["cu_seqlens"], 1e-2, "seed 631")
    assert e["o"] <= 5e-3


@pytest.mark.parametrize("dtype,d,tol", [(torch.bfloat16, 128, 1e-2), (torch.bfloat16, 64, 1e-2),
                                         (torch.float32, 64, 1e-4)])
@pytest.mark.parametrize("strength", [20.0, 50.0])
def test_strong_gates(dtype, d, tol, strength):
    """g x20 and x50 (a 64-token chunk's gate sum about -100 and -250 per channel; per token up
    to about -30): ragged varlen batch through several chunks and segments, h0 from slots."""
    dev = need_gpu()
    y = W.prefill(seed=22, seqlens=(1, 63, 64, 65, 200, 2100), H=3, dk=d, dv=d, num_slots=8,
                  h0_std=0.05, dtype=dtype)
    y["g"] = y["g"] * strength
    o, o_ref, h, h_ref = run(y, dev, h0_from_pool=True, use_l2=True)
    assert np.isfinite(o).all() and np.isfinite(h).all()
    check_prefill_parity(o, o_ref, h, h_ref, y["cu_seqlens"], tol,
                         "strong gates x%g %s d=%d" % (strength, dtype, d))


def test_weak_gates_long_sequence():
    """g around -1e-3 (decay ~0.999 per token) over one 20,000-token bf16 sequence and a
    short one: the carried state sums contributions over thousands of tokens."""
    dev = need_gpu()
    y = W.prefill(seed=23, seqlens=(20000, 300), H=2, dk=128, dv=128, num_slots=2, h0_std=0.05)
    y["g"] = y["g"] * 0.01
    o, o_ref, h, h_ref = run(y, dev, h0_from_pool=True, use_l2=True)
    check_prefill_parity(o, o_ref, h, h_ref, y["cu_seqlens"], 1e-2, "weak gates 20000 tokens")
    wc = worst_chunk_head(o, o_ref, y["cu_seqlens"])
    announce("weak gates: worst (chunk, head) rel-L2 %.3g" % wc)
    assert wc <= 2e-2
