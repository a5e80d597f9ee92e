"""GPU parity of the chunked backward (kda_chunk_backward) against the fp64 backward oracle
(oracle/kda_oracle.c kda_oracle_backward, itself pinned by finite differences of the forward
oracle), through the C ABI.  For each gradient (q, k, v, g, beta, h0): whole-tensor relative L2
and the worst (sequence, head) value; bars 1e-4 for fp32 inputs, 1e-2 for bf16."""
import numpy as np
import pytest
import torch

import kda_gated_delta_rule_amd as kda
import kda_workloads as W
from oracle import kda_oracle as O
from tests._util import announce, f64, need_gpu, rel_l2, worst_seq_head, worst_state

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "g", "beta")
GRADS = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


def grads_case(y, seed, with_h0=True, with_dht=True):
    gen = torch.Generator().manual_seed(seed)
    T, H, dv = y["v"].shape
    ns = y["cu_seqlens"].shape[0] - 1
    dk = y["q"].shape[-1]
    do = torch.randn(T, H, dv, generator=gen).to(y["q"].dtype)
    dht = torch.randn(ns, H, dk, dv, generator=gen) if with_dht else None
    h0 = y["pool"][y["slot_idx"].long()].contiguous() if with_h0 else None
    return do, dht, h0


def run_and_compare(y, do, dht, h0, tol, label, use_l2=True, heads_check=True):
    dev = need_gpu()
    cu = y["cu_seqlens"]
    got = kda.chunk_backward(*(y[n].to(dev) for n in NAMES), cu.to(dev), do.to(dev),
                             h0=None if h0 is None else h0.to(dev),
                             dht=None if dht is None else dht.to(dev), use_qk_l2norm=use_l2)
    torch.cuda.synchronize()
    ref = O.backward(*(f64(y[n]) for n in NAMES), cu.numpy(), f64(do),
                     dht=None if dht is None else f64(dht), h0=None if h0 is None else f64(h0),
                     use_qk_l2norm=use_l2)
    msg = []
    for name, a, b in zip(GRADS, got, ref):
        a = f64(a)
        e = rel_l2(a, b)
        if name == "dh0":
            w = worst_state(a, b)
        elif name == "dbeta":
            w = worst_seq_head(a[..., None], b[..., None], cu)
        else:
            w = worst_seq_head(a, b, cu)
        msg.append("%s %.3g/%.3g" % (name, e, w))
        assert np.isfinite(a).all(), name
        assert e <= tol, (label, name, e)
        if heads_check:
            assert w <= tol, (label, name, "worst", w)
    announce("%s: rel-L2 whole/worst %s" % (label, ", ".join(msg)))


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_fp32_varlen(dk, dv):
    """fp32: ragged varlen batch (1, 63, 64, 65, 0, 200, 130 tokens), h0 and dht."""
    y = W.prefill(seed=41, seqlens=(1, 63, 64, 65, 0, 200, 130), H=2, dk=dk, dv=dv, num_slots=7,
                  h0_std=0.05, dtype=torch.float32)
    do, dht, h0 = grads_case(y, 1)
    run_and_compare(y, do, dht, h0, 1e-4, "backward fp32 dk=%d dv=%d" % (dk, dv))


def test_fp32_multi_segment_dk128():
    """fp32, dk = dv = 128, sequences of several segments: the forward's local pass splits
    [S | Phi] over two workgroups by columns."""
    y = W.prefill(seed=45, seqlens=(2100, 1030), H=1, dk=128, dv=128, num_slots=2, h0_std=0.05,
                  dtype=torch.float32)
    do, dht, h0 = grads_case(y, 6)
    run_and_compare(y, do, dht, h0, 1e-4, "backward fp32 multi-segment dk=128")


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64), (64, 128)])
def test_bf16_varlen(dk, dv):
    y = W.prefill(seed=42, seqlens=(1, 63, 64, 65, 0, 200, 333), H=3, dk=dk, dv=dv, num_slots=7,
                  h0_std=0.05)
    do, dht, h0 = grads_case(y, 2)
    run_and_compare(y, do, dht, h0, 1e-2, "backward bf16 dk=%d dv=%d" % (dk, dv))


@pytest.mark.parametrize("dtype,d,tol", [(torch.float32, 64, 1e-4), (torch.bfloat16, 128, 1e-2)])
def test_without_norm_and_states(dtype, d, tol):
    """No L2 norm (keys scaled by 0.25), zero h0 and dht (None), one long and one short sequence."""
    y = W.prefill(seed=43, seqlens=(700, 17), H=2, dk=d, dv=d, num_slots=2, dtype=dtype)
    y["k"] = (y["k"].float() * 0.25).to(dtype)
    y["q"] = (y["q"].float() * 0.25).to(dtype)
    do, _, _ = grads_case(y, 3, with_h0=False, with_dht=False)
    run_and_compare(y, do, None, None, tol, "backward no norm %s" % dtype, use_l2=False)


@pytest.mark.parametrize("dtype,d,tol", [(torch.float32, 64, 1e-4), (torch.bfloat16, 128, 1e-2)])
@pytest.mark.parametrize("strength", [20.0, 50.0])
def test_strong_gates(dtype, d, tol, strength):
    y = W.prefill(seed=44, seqlens=(1, 64, 129, 300), H=2, dk=d, dv=d, num_slots=4, h0_std=0.05,
                  dtype=dtype)
    y["g"] = y["g"] * strength
    do, dht, h0 = grads_case(y, 4)
    run_and_compare(y, do, dht, h0, tol, "backward strong gates x%g %s" % (strength, dtype))


def test_full_size_T8192_H32():
    """The chunked prefill workload's shape (T = 8192, H = 32, dk = dv = 128, bf16, zero initial
    state), every head against the oracle."""
    y = W.prefill(seed=0, seqlens=(8192,), H=32, dk=128, dv=128, num_slots=1)
    do, dht, _ = grads_case(y, 5)
    run_and_compare(y, do, dht, None, 1e-2, "backward T8192 H32")
