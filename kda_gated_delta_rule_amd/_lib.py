"""ctypes binding of libkda.so (the C ABI in include/kda.h).

Argument marshalling only: torch tensors supply device pointers, shapes and the
current HIP stream; every step of the computation runs in the HIP kernels behind
the C ABI.  If the library has not been built, loading fails loudly: there is no
fallback path.
"""
import ctypes
import os

from . import _build

KDA_OK = 0
KDA_ERR_INVALID_ARG = -1
KDA_ERR_UNSUPPORTED = -2
KDA_ERR_WORKSPACE = -3
KDA_ERR_HIP = -4
KDA_F32 = 0
KDA_BF16 = 1
KDA_NOALLOC_SCRATCH_BYTES = 256 << 20  # include/kda.h

_c_p = ctypes.c_void_p
_c_i = ctypes.c_int
_c_i64 = ctypes.c_int64
_c_f = ctypes.c_float
_c_sz = ctypes.c_size_t


class KdaFront(ctypes.Structure):
    """struct kda_front (include/kda.h)."""
    _fields_ = [("gate_scale", _c_p), ("conv_q", _c_p), ("conv_k", _c_p), ("conv_v", _c_p),
                ("conv_state", _c_p), ("conv_width", _c_i), ("conv_silu", _c_i)]


_FRONT_P = ctypes.POINTER(KdaFront)

# name -> (restype, argtypes); mirrors include/kda.h
SIGNATURES = {
    "kda_decode_step": (_c_i, [_c_p, _c_p, _c_p, _c_i, _c_p, _c_p, _c_p, _c_i64, _c_p, _c_i, _c_i,
                               _c_i, _c_i, _c_i, _c_f, _c_i, _c_p, _c_p, _c_p]),
    "kda_replay_commit": (_c_i, [_c_p, _c_i64, _c_p, _c_p, _c_p, _c_i, _c_i, _c_i, _c_i, _c_i,
                                 _c_p]),
    "kda_chunk_prefill_workspace_size": (_c_sz, [_c_i, _c_i64, _c_i, _c_i, _c_i, _c_i]),
    "kda_chunk_prefill": (_c_i, [_c_p, _c_p, _c_p, _c_i, _c_p, _c_p, _c_p, _c_i, _c_i64, _c_p,
                                 _c_i64, _c_p, _c_i, _c_i, _c_i, _c_i, _c_f, _c_i, _c_p, _c_p, _c_sz,
                                 _c_p]),
    "kda_chunk_prefill_snapshots": (_c_i, [_c_p, _c_p, _c_p, _c_i, _c_p, _c_p, _c_p, _c_i, _c_i64,
                                           _c_p, _c_i64, _c_p, _c_i, _c_i, _c_i, _c_i, _c_f, _c_i,
                                           _c_p, _c_p, _c_sz, _c_i, _c_p, _c_i, _c_p]),
    "kda_chunk_prefill_noalloc": (_c_i, [_c_p, _c_p, _c_p, _c_i, _c_p, _c_p, _c_p, _c_i, _c_i64,
                                         _c_p, _c_i64, _c_p, _c_i, _c_i, _c_i, _c_i, _c_f, _c_i,
                                         _c_p, _c_p]),
    "kda_chunk_backward_workspace_size": (_c_sz, [_c_i, _c_i64, _c_i, _c_i, _c_i, _c_i]),
    "kda_chunk_backward": (_c_i, [_c_p, _c_p, _c_p, _c_i, _c_p, _c_p, _c_p, _c_i, _c_i64, _c_p, _c_p,
                                  _c_p, _c_i, _c_i, _c_i, _c_f, _c_i, _c_p, _c_p, _c_p, _c_p, _c_p,
                                  _c_p, _c_p, _c_sz, _c_p]),
    "kda_decode_step_front": (_c_i, [_c_p, _c_p, _c_p, _c_i, _c_p, _c_p, _FRONT_P, _c_p, _c_i64, _c_p,
                                     _c_i, _c_i, _c_i, _c_i, _c_i, _c_f, _c_i, _c_p, _c_p]),
    "kda_chunk_prefill_front": (_c_i, [_c_p, _c_p, _c_p, _c_i, _c_p, _c_p, _FRONT_P, _c_p, _c_i, _c_i64,
                                       _c_p, _c_i64, _c_p, _c_i, _c_i, _c_i, _c_i, _c_f, _c_i, _c_p,
                                       _c_p, _c_sz, _c_p]),
    "kda_diag_state_stream": (_c_i, [_c_p, _c_i64, _c_p, _c_i, _c_i, _c_i, _c_i, _c_p]),
    "kda_status_string": (ctypes.c_char_p, [_c_i]),
}

_LIB = None


class KdaError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__("%s failed: %s" % (fn, status_string(status)))


def lib_path():
    return _build.LIB


def load():
    """Loads libkda.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        path = lib_path()
        if not os.path.exists(path):
            raise ImportError("libkda.so is not built (%s); run __graft_entry__.build() or "
                              "python -m kda_gated_delta_rule_amd._build" % path)
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def status_string(status):
    return load().kda_status_string(int(status)).decode()


def check(fn, status):
    if status != KDA_OK:
        raise KdaError(fn, status)
