"""Thin wrappers: torch tensors -> C ABI calls of libkda.so (marshalling only).

The C ABI does not read the device-resident index arrays on the host (out-of-range or duplicate
slots, accepted lengths outside 0..T and inconsistent cu_seqlens are undefined behaviour there).
With the environment variable KDA_DEBUG_VALIDATE=1, every wrapper here first copies those arrays
to the host and checks them, raising ValueError before any launch (a synchronising debug aid)."""
import ctypes
import os

import torch

from . import _lib

_DTYPES = {torch.float32: _lib.KDA_F32, torch.bfloat16: _lib.KDA_BF16}


def _stream(t):
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _contig(*ts):
    for t in ts:
        if t is not None:
            _need(t.is_contiguous(), "tensors must be contiguous")


def debug_validate_enabled():
    """True when KDA_DEBUG_VALIDATE is set to a non-empty value other than 0."""
    return os.environ.get("KDA_DEBUG_VALIDATE", "0") not in ("", "0")


def _host(t):
    return [int(x) for x in t.detach().to("cpu").reshape(-1).tolist()]


def validate_slots(slot_idx, num_slots, allow_skip):
    """Slots in range and distinct; negative entries (skipped) only where allowed."""
    s = _host(slot_idx)
    live = [x for x in s if x >= 0]
    _need(allow_skip or len(live) == len(s), "KDA_DEBUG_VALIDATE: negative slot index")
    _need(all(x < num_slots for x in live), "KDA_DEBUG_VALIDATE: slot index >= num_slots")
    _need(len(set(live)) == len(live), "KDA_DEBUG_VALIDATE: duplicate slot index")
    return live


def validate_accepted(accepted_len, T):
    a = _host(accepted_len)
    _need(all(0 <= x <= T for x in a), "KDA_DEBUG_VALIDATE: accepted_len outside 0..T")


def validate_cu_seqlens(cu_seqlens, total_tokens):
    cu = _host(cu_seqlens)
    _need(len(cu) >= 1 and cu[0] == 0, "KDA_DEBUG_VALIDATE: cu_seqlens[0] != 0")
    _need(all(b >= a for a, b in zip(cu[:-1], cu[1:])), "KDA_DEBUG_VALIDATE: cu_seqlens decreases")
    _need(cu[-1] == total_tokens, "KDA_DEBUG_VALIDATE: cu_seqlens[-1] != total_tokens")


def validate_snapshots(snapshot_slots, slot_idx, num_slots):
    snaps = [x for x in _host(snapshot_slots) if x >= 0]
    fin = set(_host(slot_idx))
    _need(all(x < num_slots for x in snaps), "KDA_DEBUG_VALIDATE: snapshot slot >= num_slots")
    _need(len(set(snaps)) == len(snaps), "KDA_DEBUG_VALIDATE: duplicate snapshot slot")
    _need(not (set(snaps) & fin), "KDA_DEBUG_VALIDATE: snapshot slot equals a final-state slot")


def decode_step(q, k, v, g, beta, state_pool, slot_idx, *, o=None, records=None, scale=None,
                use_qk_l2norm=True):
    """Decode / MTP step (kda_decode_step).

    q, k [N, T, H, dk], v [N, T, H, dv] (bf16 or fp32); g [N, T, H, dk] fp32; beta [N, T, H]
    fp32; state_pool [num_slots, H, dk, dv] fp32 (updated in place unless records is given);
    slot_idx [N] int32.  records: None (commit) or an fp32 [N, T, H, 2dk + dv] tensor to fill
    (verify: the pool is left untouched).  Returns o [N, T, H, dv] in the dtype of q.
    """
    N, T, H, dk = q.shape
    dv = v.shape[-1]
    _need(q.dtype in _DTYPES and k.dtype == q.dtype and v.dtype == q.dtype, "q/k/v dtype")
    _need(g.dtype == torch.float32 and beta.dtype == torch.float32, "g and beta must be fp32")
    _need(state_pool.dtype == torch.float32 and slot_idx.dtype == torch.int32, "pool/slot dtype")
    _need(k.shape == q.shape and g.shape == q.shape and v.shape == (N, T, H, dv), "q/k/v/g shape")
    _need(beta.shape == (N, T, H) and slot_idx.shape == (N,), "beta/slot_idx shape")
    _need(state_pool.dim() == 4 and state_pool.shape[1:] == (H, dk, dv), "state_pool shape")
    if o is None:
        o = torch.empty(N, T, H, dv, dtype=q.dtype, device=q.device)
    _need(o.shape == (N, T, H, dv) and o.dtype == q.dtype, "o shape/dtype")
    if records is not None:
        _need(records.shape == (N, T, H, 2 * dk + dv) and records.dtype == torch.float32,
              "records shape/dtype")
    _contig(q, k, v, g, beta, state_pool, slot_idx, o, records)
    if debug_validate_enabled():
        validate_slots(slot_idx, state_pool.shape[0], allow_skip=True)
    if scale is None:
        scale = dk ** -0.5
    st = _lib.load().kda_decode_step(
        _ptr(q), _ptr(k), _ptr(v), _DTYPES[q.dtype], _ptr(g), _ptr(beta), _ptr(state_pool),
        state_pool.shape[0], _ptr(slot_idx), N, T, H, dk, dv, float(scale), int(bool(use_qk_l2norm)),
        _ptr(o), _ptr(records), _stream(q))
    _lib.check("kda_decode_step", st)
    return o


def _front(gate_scale, conv_q, conv_k, conv_v, conv_state, conv_silu, H, dk, dv, num_slots, dtype):
    """Checks the front's tensors and returns the kda_front struct (a reference to it)."""
    W = conv_q.shape[-1]
    _need(1 <= W <= 4, "conv width must be 1..4")
    _need(gate_scale.dtype == torch.float32 and gate_scale.shape == (H,), "gate_scale [H] fp32")
    for w, d in ((conv_q, dk), (conv_k, dk), (conv_v, dv)):
        _need(w.dtype == torch.float32 and w.shape == (H, d, W), "conv weights [H, d, W] fp32")
    if W > 1:
        _need(conv_state is not None and conv_state.dtype == dtype and
              conv_state.shape == (num_slots, H, W - 1, 2 * dk + dv),
              "conv_state [num_slots, H, W - 1, 2 dk + dv] in the dtype of q")
    _contig(gate_scale, conv_q, conv_k, conv_v, conv_state if W > 1 else None)
    return _lib.KdaFront(_ptr(gate_scale), _ptr(conv_q), _ptr(conv_k), _ptr(conv_v),
                         _ptr(conv_state) if W > 1 else None, W, int(bool(conv_silu)))


def decode_step_front(q, k, v, gate, beta, state_pool, slot_idx, *, gate_scale, conv_q, conv_k,
                      conv_v, conv_state=None, conv_silu=False, o=None, scale=None,
                      use_qk_l2norm=True):
    """Decode / MTP commit step with the input front fused in (kda_decode_step_front).

    q, k [N, T, H, dk], v [N, T, H, dv]: raw convolution inputs (bf16 or fp32); gate
    [N, T, H, dk] fp32 raw gates z (g = -gate_scale softplus(z)); beta [N, T, H] fp32 raw
    values (sigmoid applied); gate_scale [H] fp32; conv_q/conv_k [H, dk, W], conv_v [H, dv, W]
    fp32; conv_state [num_slots, H, W - 1, 2 dk + dv] in the dtype of q (updated in place;
    may be None for W = 1); state_pool and slot_idx as decode_step.  Returns o.
    """
    N, T, H, dk = q.shape
    dv = v.shape[-1]
    _need(q.dtype in _DTYPES and k.dtype == q.dtype and v.dtype == q.dtype, "q/k/v dtype")
    _need(gate.dtype == torch.float32 and beta.dtype == torch.float32, "gate and beta must be fp32")
    _need(state_pool.dtype == torch.float32 and slot_idx.dtype == torch.int32, "pool/slot dtype")
    _need(k.shape == q.shape and gate.shape == q.shape and v.shape == (N, T, H, dv), "q/k/v/gate shape")
    _need(beta.shape == (N, T, H) and slot_idx.shape == (N,), "beta/slot_idx shape")
    _need(state_pool.dim() == 4 and state_pool.shape[1:] == (H, dk, dv), "state_pool shape")
    front = _front(gate_scale, conv_q, conv_k, conv_v, conv_state, conv_silu, H, dk, dv,
                   state_pool.shape[0], q.dtype)
    if o is None:
        o = torch.empty(N, T, H, dv, dtype=q.dtype, device=q.device)
    _need(o.shape == (N, T, H, dv) and o.dtype == q.dtype, "o shape/dtype")
    _contig(q, k, v, gate, beta, state_pool, slot_idx, o)
    if debug_validate_enabled():
        validate_slots(slot_idx, state_pool.shape[0], allow_skip=True)
    if scale is None:
        scale = dk ** -0.5
    st = _lib.load().kda_decode_step_front(
        _ptr(q), _ptr(k), _ptr(v), _DTYPES[q.dtype], _ptr(gate), _ptr(beta), ctypes.byref(front),
        _ptr(state_pool), state_pool.shape[0], _ptr(slot_idx), N, T, H, dk, dv, float(scale),
        int(bool(use_qk_l2norm)), _ptr(o), _stream(q))
    _lib.check("kda_decode_step_front", st)
    return o


def diag_state_stream(state_pool, slot_idx):
    """Diagnostic (kda_diag_state_stream): reads and rewrites, unchanged, the state of each
    slot in slot_idx with the T = 1 decode kernel's access pattern; its time is the floor the
    decode step's state traffic sets."""
    _need(state_pool.dtype == torch.float32 and state_pool.dim() == 4, "state_pool")
    _need(slot_idx.dtype == torch.int32 and slot_idx.dim() == 1, "slot_idx")
    _contig(state_pool, slot_idx)
    ns, H, dk, dv = state_pool.shape
    st = _lib.load().kda_diag_state_stream(_ptr(state_pool), ns, _ptr(slot_idx), slot_idx.shape[0], H, dk,
                                           dv, _stream(state_pool))
    _lib.check("kda_diag_state_stream", st)


def replay_commit(state_pool, slot_idx, records, accepted_len):
    """ReplaySSM commit (kda_replay_commit): applies records[n, :accepted_len[n]] to the slots."""
    N, T, H, R = records.shape
    dk = state_pool.shape[2]
    dv = state_pool.shape[3]
    _need(R == 2 * dk + dv and state_pool.shape[1] == H, "records/state_pool shape")
    _need(slot_idx.shape == (N,) and accepted_len.shape == (N,), "slot_idx/accepted_len shape")
    _need(accepted_len.dtype == torch.int32 and slot_idx.dtype == torch.int32, "index dtype")
    _contig(state_pool, slot_idx, records, accepted_len)
    if debug_validate_enabled():
        validate_slots(slot_idx, state_pool.shape[0], allow_skip=True)
        validate_accepted(accepted_len, T)
    st = _lib.load().kda_replay_commit(_ptr(state_pool), state_pool.shape[0], _ptr(slot_idx),
                                       _ptr(records), _ptr(accepted_len), N, T, H, dk, dv,
                                       _stream(state_pool))
    _lib.check("kda_replay_commit", st)


def chunk_prefill_workspace_size(num_seqs, total_tokens, H, dk, dv, dtype=torch.bfloat16):
    return int(_lib.load().kda_chunk_prefill_workspace_size(num_seqs, total_tokens, H, dk, dv,
                                                            _DTYPES[dtype]))


def chunk_prefill(q, k, v, g, beta, cu_seqlens, state_pool, slot_idx, *, h0_from_pool=True,
                  o=None, workspace=None, scale=None, use_qk_l2norm=True, snapshot_every=None,
                  snapshot_slots=None):
    """Varlen chunked prefill (kda_chunk_prefill, or kda_chunk_prefill_snapshots when
    snapshot_every is given).

    q, k [T_total, H, dk], v [T_total, H, dv] (bf16 or fp32); g [T_total, H, dk] fp32;
    beta [T_total, H] fp32; cu_seqlens [num_seqs + 1] int32; state_pool [num_slots, H, dk, dv]
    fp32 (final states written to slot_idx [num_seqs] int32).  workspace: a uint8 tensor of at
    least chunk_prefill_workspace_size(...) bytes, or None to allocate one.  snapshot_every (a
    multiple of 64) with snapshot_slots [num_seqs, max_snaps] int32: the state of sequence i
    after (j + 1) * snapshot_every tokens is also written to slot snapshot_slots[i, j] (negative
    entries skipped).  Returns o.
    """
    Tt, H, dk = q.shape
    dv = v.shape[-1]
    ns = cu_seqlens.shape[0] - 1
    _need(q.dtype in _DTYPES and k.dtype == q.dtype and v.dtype == q.dtype, "q/k/v dtype")
    _need(g.dtype == torch.float32 and beta.dtype == torch.float32, "g and beta must be fp32")
    _need(k.shape == q.shape and g.shape == q.shape and v.shape == (Tt, H, dv), "q/k/v/g shape")
    _need(beta.shape == (Tt, H), "beta shape")
    _need(cu_seqlens.dtype == torch.int32 and slot_idx.dtype == torch.int32, "index dtype")
    _need(slot_idx.shape == (ns,), "slot_idx shape")
    _need(state_pool.dim() == 4 and state_pool.shape[1:] == (H, dk, dv), "state_pool shape")
    if o is None:
        o = torch.empty(Tt, H, dv, dtype=q.dtype, device=q.device)
    if debug_validate_enabled():
        validate_cu_seqlens(cu_seqlens, Tt)
        validate_slots(slot_idx, state_pool.shape[0], allow_skip=False)
        if snapshot_slots is not None:
            validate_snapshots(snapshot_slots, slot_idx, state_pool.shape[0])
    need = chunk_prefill_workspace_size(ns, Tt, H, dk, dv, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _contig(q, k, v, g, beta, cu_seqlens, state_pool, slot_idx, o, workspace)
    if scale is None:
        scale = dk ** -0.5
    args = (_ptr(q), _ptr(k), _ptr(v), _DTYPES[q.dtype], _ptr(g), _ptr(beta), _ptr(cu_seqlens),
            ns, Tt, _ptr(state_pool), state_pool.shape[0], _ptr(slot_idx), int(bool(h0_from_pool)),
            H, dk, dv, float(scale), int(bool(use_qk_l2norm)), _ptr(o), _ptr(workspace),
            workspace.numel() * workspace.element_size())
    if snapshot_every is None:
        _need(snapshot_slots is None, "snapshot_slots needs snapshot_every")
        st = _lib.load().kda_chunk_prefill(*args, _stream(q))
        _lib.check("kda_chunk_prefill", st)
    else:
        _need(snapshot_slots is not None and snapshot_slots.dtype == torch.int32
              and snapshot_slots.dim() == 2 and snapshot_slots.shape[0] == ns, "snapshot_slots")
        _contig(snapshot_slots)
        st = _lib.load().kda_chunk_prefill_snapshots(*args, int(snapshot_every), _ptr(snapshot_slots),
                                                     snapshot_slots.shape[1], _stream(q))
        _lib.check("kda_chunk_prefill_snapshots", st)
    return o


def chunk_prefill_front(q, k, v, gate, beta, cu_seqlens, state_pool, slot_idx, *, gate_scale, conv_q,
                        conv_k, conv_v, conv_state=None, conv_silu=False, h0_from_pool=True, o=None,
                        workspace=None, scale=None, use_qk_l2norm=True):
    """Varlen chunked prefill with the input front fused in (kda_chunk_prefill_front).

    q, k [T_total, H, dk], v [T_total, H, dv]: raw convolution inputs; gate [T_total, H, dk]
    fp32 raw gates z; beta [T_total, H] fp32 raw values; the front's tensors as
    decode_step_front (conv_state [num_slots, H, W - 1, 2 dk + dv] read when h0_from_pool and
    written back per sequence); the rest as chunk_prefill.  Returns o.
    """
    Tt, H, dk = q.shape
    dv = v.shape[-1]
    ns = cu_seqlens.shape[0] - 1
    _need(q.dtype in _DTYPES and k.dtype == q.dtype and v.dtype == q.dtype, "q/k/v dtype")
    _need(gate.dtype == torch.float32 and beta.dtype == torch.float32, "gate and beta must be fp32")
    _need(k.shape == q.shape and gate.shape == q.shape and v.shape == (Tt, H, dv), "q/k/v/gate shape")
    _need(beta.shape == (Tt, H), "beta shape")
    _need(cu_seqlens.dtype == torch.int32 and slot_idx.dtype == torch.int32, "index dtype")
    _need(slot_idx.shape == (ns,), "slot_idx shape")
    _need(state_pool.dim() == 4 and state_pool.shape[1:] == (H, dk, dv), "state_pool shape")
    front = _front(gate_scale, conv_q, conv_k, conv_v, conv_state, conv_silu, H, dk, dv,
                   state_pool.shape[0], q.dtype)
    if o is None:
        o = torch.empty(Tt, H, dv, dtype=q.dtype, device=q.device)
    if debug_validate_enabled():
        validate_cu_seqlens(cu_seqlens, Tt)
        validate_slots(slot_idx, state_pool.shape[0], allow_skip=False)
    need = chunk_prefill_workspace_size(ns, Tt, H, dk, dv, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _contig(q, k, v, gate, beta, cu_seqlens, state_pool, slot_idx, o, workspace)
    if scale is None:
        scale = dk ** -0.5
    st = _lib.load().kda_chunk_prefill_front(
        _ptr(q), _ptr(k), _ptr(v), _DTYPES[q.dtype], _ptr(gate), _ptr(beta), ctypes.byref(front),
        _ptr(cu_seqlens), ns, Tt, _ptr(state_pool), state_pool.shape[0], _ptr(slot_idx),
        int(bool(h0_from_pool)), H, dk, dv, float(scale), int(bool(use_qk_l2norm)), _ptr(o),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(q))
    _lib.check("kda_chunk_prefill_front", st)
    return o


def chunk_prefill_noalloc(q, k, v, g, beta, cu_seqlens, state_pool, slot_idx, *, h0_from_pool=True,
                          o=None, scale=None, use_qk_l2norm=True):
    """Varlen chunked prefill on the library's static workspace (kda_chunk_prefill_noalloc):
    no device allocation inside the call (pass o to avoid the output allocation here too).
    Arguments and result as chunk_prefill; sizes whose workspace exceeds
    KDA_NOALLOC_SCRATCH_BYTES raise KdaError(KDA_ERR_WORKSPACE).  Calls that overlap in time on
    one GPU share the workspace and race."""
    Tt, H, dk = q.shape
    dv = v.shape[-1]
    ns = cu_seqlens.shape[0] - 1
    _need(q.dtype in _DTYPES and k.dtype == q.dtype and v.dtype == q.dtype, "q/k/v dtype")
    _need(g.dtype == torch.float32 and beta.dtype == torch.float32, "g and beta must be fp32")
    _need(k.shape == q.shape and g.shape == q.shape and v.shape == (Tt, H, dv), "q/k/v/g shape")
    _need(beta.shape == (Tt, H), "beta shape")
    _need(cu_seqlens.dtype == torch.int32 and slot_idx.dtype == torch.int32, "index dtype")
    _need(slot_idx.shape == (ns,), "slot_idx shape")
    _need(state_pool.dim() == 4 and state_pool.shape[1:] == (H, dk, dv), "state_pool shape")
    if o is None:
        o = torch.empty(Tt, H, dv, dtype=q.dtype, device=q.device)
    _need(o.shape == (Tt, H, dv) and o.dtype == q.dtype, "o shape/dtype")
    _contig(q, k, v, g, beta, cu_seqlens, state_pool, slot_idx, o)
    if debug_validate_enabled():
        validate_cu_seqlens(cu_seqlens, Tt)
        validate_slots(slot_idx, state_pool.shape[0], allow_skip=False)
    if scale is None:
        scale = dk ** -0.5
    st = _lib.load().kda_chunk_prefill_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _DTYPES[q.dtype], _ptr(g), _ptr(beta), _ptr(cu_seqlens), ns, Tt,
        _ptr(state_pool), state_pool.shape[0], _ptr(slot_idx), int(bool(h0_from_pool)), H, dk, dv,
        float(scale), int(bool(use_qk_l2norm)), _ptr(o), _stream(q))
    _lib.check("kda_chunk_prefill_noalloc", st)
    return o


def chunk_backward_workspace_size(num_seqs, total_tokens, H, dk, dv, dtype=torch.bfloat16):
    return int(_lib.load().kda_chunk_backward_workspace_size(num_seqs, total_tokens, H, dk, dv,
                                                             _DTYPES[dtype]))


def chunk_backward(q, k, v, g, beta, cu_seqlens, do, *, h0=None, dht=None, workspace=None,
                   scale=None, use_qk_l2norm=True, want_dh0=True):
    """Gradients of sum(do * o) + sum(dht * ht) of chunk_prefill (kda_chunk_backward).

    q, k [T, H, dk], v [T, H, dv] (bf16 or fp32); g [T, H, dk] fp32; beta [T, H] fp32;
    cu_seqlens [num_seqs + 1] int32; do [T, H, dv] (dtype of q); h0, dht [num_seqs, H, dk, dv]
    fp32 or None (zero).  Returns (dq, dk, dv, dg, dbeta, dh0): dq, dk, dv in the dtype of q,
    dg, dbeta and dh0 fp32 (dh0 None when want_dh0 is False)."""
    Tt, H, dk = q.shape
    dv = v.shape[-1]
    ns = cu_seqlens.shape[0] - 1
    _need(q.dtype in _DTYPES and k.dtype == q.dtype and v.dtype == q.dtype and do.dtype == q.dtype,
          "q/k/v/do dtype")
    _need(g.dtype == torch.float32 and beta.dtype == torch.float32, "g and beta must be fp32")
    _need(k.shape == q.shape and g.shape == q.shape and v.shape == (Tt, H, dv) and do.shape == v.shape,
          "q/k/v/g/do shape")
    _need(beta.shape == (Tt, H) and cu_seqlens.dtype == torch.int32, "beta shape / cu_seqlens dtype")
    for st in (h0, dht):
        if st is not None:
            _need(st.dtype == torch.float32 and st.shape == (ns, H, dk, dv), "h0/dht [num_seqs, H, dk, dv] fp32")
    if debug_validate_enabled():
        validate_cu_seqlens(cu_seqlens, Tt)
    dq, dk_, dv_ = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dg = torch.empty_like(g)
    dbeta = torch.empty_like(beta)
    dh0 = torch.empty(ns, H, dk, dv, dtype=torch.float32, device=q.device) if want_dh0 else None
    need = chunk_backward_workspace_size(ns, Tt, H, dk, dv, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _contig(q, k, v, g, beta, cu_seqlens, do, h0, dht, workspace)
    if scale is None:
        scale = dk ** -0.5
    st = _lib.load().kda_chunk_backward(
        _ptr(q), _ptr(k), _ptr(v), _DTYPES[q.dtype], _ptr(g), _ptr(beta), _ptr(cu_seqlens), ns, Tt,
        _ptr(h0), _ptr(do), _ptr(dht), H, dk, dv, float(scale), int(bool(use_qk_l2norm)), _ptr(dq),
        _ptr(dk_), _ptr(dv_), _ptr(dg), _ptr(dbeta), _ptr(dh0), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(q))
    _lib.check("kda_chunk_backward", st)
    return dq, dk_, dv_, dg, dbeta, dh0
