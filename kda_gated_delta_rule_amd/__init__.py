"""Kimi Delta Attention (KDA) gated delta-rule hot path for AMD MI355X (gfx950).

Python front end of the C ABI in include/kda.h.  Tensors are torch tensors on
the GPU; they provide device memory and the stream, nothing else:

  decode_step    fused decode / MTP step over state-pool slots (commit or verify)
  decode_step_front  the commit step with the input front (ShortConv, gate and beta) fused in
  replay_commit  ReplaySSM commit of accepted update records
  chunk_prefill  varlen 64-token chunked prefill with initial / final states
  chunk_prefill_front  the prefill with the input front fused in
  chunk_prefill_noalloc  the same on the library's static workspace (no allocation)
  chunk_backward gradients of the chunked prefill (training)

All arithmetic runs in the HIP kernels of libkda.so.
"""
from ._lib import KdaError, load, status_string  # noqa: F401
from .ops import (chunk_backward, chunk_backward_workspace_size, chunk_prefill,  # noqa: F401
                  chunk_prefill_front,
                  chunk_prefill_noalloc, chunk_prefill_workspace_size, decode_step,
                  decode_step_front, replay_commit)

__all__ = ["decode_step", "decode_step_front", "replay_commit", "chunk_prefill", "chunk_prefill_front", "chunk_prefill_noalloc",
           "chunk_prefill_workspace_size", "chunk_backward", "chunk_backward_workspace_size",
           "KdaError", "load", "status_string"]
