"""Randomised parity sweep: decode / MTP (commit), verify + replay and varlen prefill through the
C ABI against the fp64 oracle, over random head shapes, dtypes, token counts, ragged sequence
lengths (empty, 1, 63-65, 127-129, >1000), slot maps with skipped sequences, accepted lengths,
strong gates and the L2-norm switch (kda_workloads.sweep_case).  Bars: rel-L2 <= 1e-4 for fp32
inputs, <= 1e-2 for bf16; skipped sequences, untouched slots and the pool under verify are
checked exactly.  Cases whose q.k products cancel are in test_gpu_prefill_range.py (among
them seed 631 of this generator, a one-token bf16 sequence without the L2 norm)."""
import numpy as np
import pytest
import torch

import kda_gated_delta_rule_amd as kda
import kda_workloads as W
from oracle import kda_oracle as O
from _util import announce, f64, need_gpu, rel_l2, worst_decode, worst_seq_head, worst_state

pytestmark = pytest.mark.gpu


def _tol(dtype):
    return 1e-4 if dtype == torch.float32 else 1e-2


def _check_decode(c, dev):
    q, k, v, g, beta, pool = c["q"], c["k"], c["v"], c["g"], c["beta"], c["pool"]
    N, T, H, dk = q.shape
    dv = v.shape[-1]
    slots = c["slot_idx"].numpy()
    live = slots >= 0
    h0 = np.zeros((N, H, dk, dv))
    h0[live] = f64(pool)[slots[live]]
    o_ref, h_ref, r_ref = O.decode(f64(q), f64(k), f64(v), f64(g), f64(beta), h0,
                                   use_qk_l2norm=c["use_l2"], want_records=True)
    dpool, sl = pool.to(dev), c["slot_idx"].to(dev)
    rec = torch.empty(N, T, H, 2 * dk + dv, device=dev) if c["verify"] else None
    o = kda.decode_step(q.to(dev), k.to(dev), v.to(dev), g.to(dev), beta.to(dev), dpool, sl,
                        records=rec, use_qk_l2norm=c["use_l2"])
    torch.cuda.synchronize()
    tol = _tol(c["dtype"])
    oc = f64(o.cpu())
    if live.any():
        assert rel_l2(oc[live], o_ref[live]) <= tol
        assert worst_decode(oc[live], o_ref[live]) <= tol
    assert np.all(oc[~live] == 0), "a skipped sequence's output is not zero"
    untouched = np.setdiff1d(np.arange(pool.shape[0]), slots[live])
    if c["verify"]:
        assert torch.equal(dpool.cpu(), pool), "verify wrote the pool"
        if live.any():
            assert rel_l2(f64(rec.cpu())[live], r_ref[live]) <= tol
        acc = c["accepted"]
        kda.replay_commit(dpool, sl, rec, acc.to(dev))
        torch.cuda.synchronize()
        pc = f64(dpool.cpu())
        if live.any():
            s_ref = O.replay(h0[live], r_ref[live], acc.numpy()[live])
            assert rel_l2(pc[slots[live]], s_ref) <= tol
            assert worst_state(pc[slots[live]], s_ref) <= tol
    else:
        pc = f64(dpool.cpu())
        if live.any():
            assert rel_l2(pc[slots[live]], h_ref[live]) <= tol
            assert worst_state(pc[slots[live]], h_ref[live]) <= tol
    assert np.array_equal(pc[untouched], f64(pool)[untouched]), "a slot outside the call changed"


def _check_prefill(c, dev):
    q, k, v, g, beta, pool, cu = c["q"], c["k"], c["v"], c["g"], c["beta"], c["pool"], c["cu_seqlens"]
    slots = c["slot_idx"].numpy()
    ns = slots.shape[0]
    H, dk, dv = pool.shape[1:]
    h0 = f64(pool)[slots] if c["h0_from_pool"] else np.zeros((ns, H, dk, dv))
    o_ref, h_ref, _ = O.recurrent(f64(q), f64(k), f64(v), f64(g), f64(beta),
                                  cu.numpy().astype(np.int64), h0=h0, use_qk_l2norm=c["use_l2"])
    dpool = pool.to(dev)
    o = kda.chunk_prefill(q.to(dev), k.to(dev), v.to(dev), g.to(dev), beta.to(dev), cu.to(dev), dpool,
                          c["slot_idx"].to(dev), h0_from_pool=c["h0_from_pool"],
                          use_qk_l2norm=c["use_l2"])
    torch.cuda.synchronize()
    tol = _tol(c["dtype"])
    if q.shape[0] > 0:
        assert rel_l2(f64(o.cpu()), o_ref) <= tol
        assert worst_seq_head(f64(o.cpu()), o_ref, cu.numpy()) <= tol
    pc = f64(dpool.cpu())
    assert rel_l2(pc[slots], h_ref) <= tol
    assert worst_state(pc[slots], h_ref) <= tol
    untouched = np.setdiff1d(np.arange(pool.shape[0]), slots)
    assert np.array_equal(pc[untouched], f64(pool)[untouched]), "a slot outside the call changed"


@pytest.mark.parametrize("seed", range(80))
def test_random_case_matches_the_oracle(seed):
    dev = need_gpu()
    c = W.sweep_case(seed)
    announce("sweep seed %d: %s" % (seed, c["desc"]))
    (_check_decode if c["kind"] == "decode" else _check_prefill)(c, dev)
