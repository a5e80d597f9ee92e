"""CPU checks of the C ABI: the library loads, exports every function include/kda.h
declares, and rejects invalid arguments on the host before any HIP call (so these
run without a GPU).  Pointers here are fake, never dereferenced: every call below
fails validation or returns early before a launch.
"""
import ctypes
import os
import re

import pytest

from kda_gated_delta_rule_amd import _build, _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_build.LIB):
        _build.build(force=True)
    return _lib.load()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "kda.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(kda_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(_lib.SIGNATURES), names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4):
        s = _lib.status_string(code)
        assert s.startswith("KDA_")
    assert "unknown" in _lib.status_string(7)


A = 0x10000  # a 16-byte aligned fake address


def decode_args(**over):
    args = dict(q=A, k=A, v=A, dtype=1, g=A, beta=A, pool=A, num_slots=8, slot=A, N=4, T=1, H=2,
                dk=128, dv=128, scale=0.1, l2=1, o=A, rec=None, stream=None)
    args.update(over)
    return list(args.values())


@pytest.mark.parametrize("over,code", [
    (dict(q=None), _lib.KDA_ERR_INVALID_ARG),
    (dict(o=None), _lib.KDA_ERR_INVALID_ARG),
    (dict(slot=None), _lib.KDA_ERR_INVALID_ARG),
    (dict(q=A + 4), _lib.KDA_ERR_INVALID_ARG),
    (dict(rec=A + 8), _lib.KDA_ERR_INVALID_ARG),
    (dict(dtype=2), _lib.KDA_ERR_INVALID_ARG),
    (dict(T=0), _lib.KDA_ERR_INVALID_ARG),
    (dict(H=0), _lib.KDA_ERR_INVALID_ARG),
    (dict(N=-1), _lib.KDA_ERR_INVALID_ARG),
    (dict(N=(1 << 21) + 1), _lib.KDA_ERR_INVALID_ARG),  # N * H above 2^22 (H = 2)
    (dict(num_slots=0), _lib.KDA_ERR_INVALID_ARG),
    (dict(l2=2), _lib.KDA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), _lib.KDA_ERR_INVALID_ARG),
    (dict(dk=96), _lib.KDA_ERR_UNSUPPORTED),
    (dict(dv=256), _lib.KDA_ERR_UNSUPPORTED),
    (dict(N=0), _lib.KDA_OK),  # nothing to do: returns before any launch
])
def test_decode_validation(lib, over, code):
    assert lib.kda_decode_step(*decode_args(**over)) == code


@pytest.mark.parametrize("over,code", [
    (dict(pool=None), _lib.KDA_ERR_INVALID_ARG),
    (dict(rec=None), _lib.KDA_ERR_INVALID_ARG),
    (dict(acc=None), _lib.KDA_ERR_INVALID_ARG),
    (dict(acc=A + 4), _lib.KDA_ERR_INVALID_ARG),
    (dict(T=0), _lib.KDA_ERR_INVALID_ARG),
    (dict(dk=32), _lib.KDA_ERR_UNSUPPORTED),
    (dict(N=(1 << 21) + 1), _lib.KDA_ERR_INVALID_ARG),  # N * H above 2^22 (H = 2)
    (dict(N=0), _lib.KDA_OK),
])
def test_replay_validation(lib, over, code):
    args = dict(pool=A, num_slots=8, slot=A, rec=A, acc=A, N=2, T=8, H=2, dk=128, dv=128,
                stream=None)
    args.update(over)
    assert lib.kda_replay_commit(*args.values()) == code


def prefill_args(**over):
    args = dict(q=A, k=A, v=A, dtype=1, g=A, beta=A, cu=A, ns=2, T=200, pool=A, num_slots=4,
                slot=A, h0=1, H=2, dk=128, dv=128, scale=0.1, l2=1, o=A, ws=A, ws_bytes=0,
                stream=None)
    args.update(over)
    return args


def test_prefill_workspace_size(lib):
    f = lib.kda_chunk_prefill_workspace_size
    small = f(1, 64, 1, 128, 128, 1)
    assert small > 0
    assert f(1, 128, 1, 128, 128, 1) > small
    assert f(1, 64, 2, 128, 128, 1) > small
    assert f(1, 64, 1, 128, 128, 0) > small  # fp32 operands are wider
    assert f(1, 64, 1, 96, 128, 1) == 0      # unsupported dim
    assert f(-1, 64, 1, 128, 128, 1) == 0


@pytest.mark.parametrize("over,code", [
    (dict(q=None), _lib.KDA_ERR_INVALID_ARG),
    (dict(cu=None), _lib.KDA_ERR_INVALID_ARG),
    (dict(g=A + 4), _lib.KDA_ERR_INVALID_ARG),
    (dict(h0=3), _lib.KDA_ERR_INVALID_ARG),
    (dict(ns=0), _lib.KDA_ERR_INVALID_ARG),  # tokens without sequences
    (dict(ns=0, T=0), _lib.KDA_OK),
    (dict(T=-5), _lib.KDA_ERR_INVALID_ARG),
    (dict(dk=100), _lib.KDA_ERR_UNSUPPORTED),
    (dict(dtype=0, dk=128), _lib.KDA_ERR_WORKSPACE),  # fp32 at dk = 128 is supported
    (dict(ws=None), _lib.KDA_ERR_WORKSPACE),
    (dict(ws_bytes=1024), _lib.KDA_ERR_WORKSPACE),
])
def test_prefill_validation(lib, over, code):
    # ws_bytes stays too small, so a case that passes every other check stops at the
    # workspace check, before any launch
    assert lib.kda_chunk_prefill(*prefill_args(**over).values()) == code


@pytest.mark.parametrize("every,slots,max_snaps,code", [
    (0, A, 4, _lib.KDA_ERR_INVALID_ARG),
    (32, A, 4, _lib.KDA_ERR_INVALID_ARG),     # not chunk aligned
    (100, A, 4, _lib.KDA_ERR_INVALID_ARG),
    (256, A, 0, _lib.KDA_ERR_INVALID_ARG),    # no snapshot row
    (256, None, 4, _lib.KDA_ERR_INVALID_ARG),
    (256, A + 4, 4, _lib.KDA_ERR_INVALID_ARG),
    (256, A, 4, _lib.KDA_ERR_WORKSPACE),      # valid: stops at the workspace check
])
def test_prefill_snapshot_validation(lib, every, slots, max_snaps, code):
    args = list(prefill_args().values())
    args = args[:-1] + [every, slots, max_snaps, None]
    assert lib.kda_chunk_prefill_snapshots(*args) == code


def test_prefill_valid_arguments_reach_workspace_check(lib):
    # all arguments valid except the workspace size: the call must stop at that check
    assert lib.kda_chunk_prefill(*prefill_args().values()) == _lib.KDA_ERR_WORKSPACE


def noalloc_args(**over):
    args = prefill_args(**over)
    del args["ws"], args["ws_bytes"]
    return list(args.values())


def test_noalloc_rejects_sizes_beyond_the_static_workspace(lib):
    # T = 8192 x H = 32 needs about 350 MB of workspace, more than the 256 MiB array: the
    # call stops at the size check, before any HIP call
    f = lib.kda_chunk_prefill_workspace_size
    assert f(1, 8192, 32, 128, 128, 1) > _lib.KDA_NOALLOC_SCRATCH_BYTES
    assert f(1, 4096, 32, 128, 128, 1) <= _lib.KDA_NOALLOC_SCRATCH_BYTES
    assert lib.kda_chunk_prefill_noalloc(*noalloc_args(ns=1, T=8192, H=32)) == _lib.KDA_ERR_WORKSPACE


@pytest.mark.parametrize("over,code", [
    (dict(q=None), _lib.KDA_ERR_INVALID_ARG),
    (dict(h0=3), _lib.KDA_ERR_INVALID_ARG),
    (dict(ns=0, T=0), _lib.KDA_OK),
    (dict(dk=100), _lib.KDA_ERR_UNSUPPORTED),
])
def test_noalloc_validation(lib, over, code):
    assert lib.kda_chunk_prefill_noalloc(*noalloc_args(**over)) == code


def test_noalloc_limit_matches_the_header():
    text = open(os.path.join(ROOT, "include", "kda.h")).read()
    m = re.search(r"#define KDA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.KDA_NOALLOC_SCRATCH_BYTES


def backward_args(**over):
    args = dict(q=A, k=A, v=A, dtype=1, g=A, beta=A, cu=A, ns=2, T=200, h0=None, do=A, dht=None,
                H=2, dk=128, dv=128, scale=0.1, l2=1, dq=A, dk_=A, dv_=A, dg=A, dbeta=A, dh0=None,
                ws=A, ws_bytes=0, stream=None)
    args.update(over)
    return list(args.values())


def test_backward_workspace_size(lib):
    f = lib.kda_chunk_backward_workspace_size
    small = f(1, 64, 1, 128, 128, 1)
    assert small > lib.kda_chunk_prefill_workspace_size(1, 64, 1, 128, 128, 1)
    assert f(1, 128, 1, 128, 128, 1) > small
    assert f(1, 64, 1, 96, 128, 1) == 0


@pytest.mark.parametrize("over,code", [
    (dict(q=None), _lib.KDA_ERR_INVALID_ARG),
    (dict(do=None), _lib.KDA_ERR_INVALID_ARG),
    (dict(dg=A + 4), _lib.KDA_ERR_INVALID_ARG),
    (dict(h0=A + 8), _lib.KDA_ERR_INVALID_ARG),
    (dict(l2=2), _lib.KDA_ERR_INVALID_ARG),
    (dict(ns=0, T=0), _lib.KDA_OK),
    (dict(dv=32), _lib.KDA_ERR_UNSUPPORTED),
    (dict(dtype=0, dk=128), _lib.KDA_ERR_WORKSPACE),  # fp32 at dk = 128 is supported
    (dict(), _lib.KDA_ERR_WORKSPACE),  # valid: stops at the workspace check
    (dict(ws=None, ws_bytes=1 << 40), _lib.KDA_ERR_WORKSPACE),
])
def test_backward_validation(lib, over, code):
    assert lib.kda_chunk_backward(*backward_args(**over)) == code


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_LIB", None)
    monkeypatch.setattr(_lib, "lib_path", lambda: str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        _lib.load()


def test_isa_has_no_mfma_result_read_through_short_branch_path():
    """Compiles the kernels to gfx950 assembly and checks that no MFMA accumulator is
    read through a forward branch with fewer than 10 wait states (a stale-result hazard
    the compiler left uncovered once, behind a data-dependent loop)."""
    from kda_gated_delta_rule_amd import isa_lint

    findings = isa_lint.lint()
    assert not findings, findings[:3]


def front(**over):
    f = dict(gate_scale=A, conv_q=A, conv_k=A, conv_v=A, conv_state=A, conv_width=4, conv_silu=1)
    f.update(over)
    return _lib.KdaFront(*f.values())


def decode_front_args(fr, **over):
    args = dict(q=A, k=A, v=A, dtype=1, g=A, beta=A, front=ctypes.byref(fr), pool=A, num_slots=8,
                slot=A, N=0, T=1, H=2, dk=128, dv=128, scale=0.1, l2=1, o=A, stream=None)
    args.update(over)
    return list(args.values())


@pytest.mark.parametrize("fover,over,code", [
    (dict(), dict(), _lib.KDA_OK),  # valid, N = 0: returns before any launch
    (dict(conv_width=1, conv_state=None), dict(), _lib.KDA_OK),  # width 1 needs no state
    (dict(conv_width=0), dict(), _lib.KDA_ERR_INVALID_ARG),
    (dict(conv_width=5), dict(), _lib.KDA_ERR_INVALID_ARG),
    (dict(conv_silu=2), dict(), _lib.KDA_ERR_INVALID_ARG),
    (dict(conv_state=None), dict(), _lib.KDA_ERR_INVALID_ARG),
    (dict(conv_state=A + 4), dict(), _lib.KDA_ERR_INVALID_ARG),
    (dict(gate_scale=None), dict(), _lib.KDA_ERR_INVALID_ARG),
    (dict(conv_v=A + 8), dict(), _lib.KDA_ERR_INVALID_ARG),
    (dict(), dict(T=9), _lib.KDA_ERR_INVALID_ARG),  # at most 8 tokens with the front
    (dict(), dict(front=None), _lib.KDA_ERR_INVALID_ARG),
    (dict(), dict(dk=96), _lib.KDA_ERR_UNSUPPORTED),
])
def test_decode_front_validation(lib, fover, over, code):
    fr = front(**fover)
    assert lib.kda_decode_step_front(*decode_front_args(fr, **over)) == code


@pytest.mark.parametrize("fover,code", [
    (dict(), _lib.KDA_ERR_WORKSPACE),  # valid: stops at the workspace check
    (dict(conv_width=7), _lib.KDA_ERR_INVALID_ARG),
    (dict(conv_q=None), _lib.KDA_ERR_INVALID_ARG),
])
def test_prefill_front_validation(lib, fover, code):
    fr = front(**fover)
    p = prefill_args()
    args = list(p.values())
    # kda_chunk_prefill_front takes the front after beta (position 6)
    args = args[:6] + [ctypes.byref(fr)] + args[6:]
    assert lib.kda_chunk_prefill_front(*args) == code
