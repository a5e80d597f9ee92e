"""kda_chunk_prefill_noalloc (the prefill on the library's static workspace, for callers that
cannot allocate) against kda_chunk_prefill with a caller workspace: the same kernels on the same
inputs, so outputs and final states must be equal bit for bit, and both within the oracle's bar.
Two calls in a row share the static array; the second is smaller than the first, so it runs on
what the first left behind."""
import pytest
import torch

import kda_gated_delta_rule_amd as kda
import kda_workloads as W
from oracle import kda_oracle as O
from tests._util import announce, check_prefill_parity, f64, need_gpu

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "g", "beta")


def both(y, dev):
    ins = [y[n].to(dev) for n in NAMES] + [y["cu_seqlens"].to(dev)]
    sl = y["slot_idx"].to(dev)
    pa, pb = y["pool"].to(dev), y["pool"].to(dev)
    oa = kda.chunk_prefill(*ins, pa, sl)
    ob = kda.chunk_prefill_noalloc(*ins, pb, sl)
    torch.cuda.synchronize()
    return oa, ob, pa, pb


@pytest.mark.parametrize("dtype,d,tol", [(torch.bfloat16, 128, 1e-2), (torch.float32, 64, 1e-4)])
def test_noalloc_equals_workspace_call_twice(dtype, d, tol):
    dev = need_gpu()
    cases = [W.prefill(seed=31, seqlens=(1500, 700, 33, 0), H=8, dk=d, dv=d, num_slots=6,
                       h0_std=0.05, dtype=dtype),
             W.prefill(seed=32, seqlens=(100, 5), H=2, dk=d, dv=d, num_slots=3, h0_std=0.05,
                       dtype=dtype)]
    for n, y in enumerate(cases):
        announce("noalloc prefill call %d %s d=%d, %d tokens" % (n, dtype, d, y["q"].shape[0]))
        oa, ob, pa, pb = both(y, dev)
        assert torch.equal(oa, ob)
        assert torch.equal(pa, pb)
        sl = y["slot_idx"].long()
        o_ref, h_ref, _ = O.recurrent(*(f64(y[m]) for m in NAMES), y["cu_seqlens"].numpy(),
                                      h0=f64(y["pool"][sl]))
        check_prefill_parity(f64(ob), o_ref, f64(pb.cpu()[sl]), h_ref, y["cu_seqlens"], tol,
                             "noalloc call %d" % n)


def test_noalloc_rejects_a_workspace_beyond_the_static_array():
    dev = need_gpu()
    y = W.prefill(seed=33, seqlens=(8192,), H=32, dk=128, dv=128, num_slots=1)
    ins = [y[n].to(dev) for n in NAMES] + [y["cu_seqlens"].to(dev)]
    with pytest.raises(kda.KdaError) as e:
        kda.chunk_prefill_noalloc(*ins, y["pool"].to(dev), y["slot_idx"].to(dev))
    assert e.value.status == -3
