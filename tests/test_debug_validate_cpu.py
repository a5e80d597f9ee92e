"""KDA_DEBUG_VALIDATE (CPU): with the variable set, the Python wrappers copy the device-resident
index arrays to the host and reject out-of-range or duplicate slots, accepted lengths outside
0..T and inconsistent cu_seqlens with ValueError before any call into the library.  CPU tensors
stand in for device tensors: every call here fails validation before a launch."""
import pytest
import torch

from kda_gated_delta_rule_amd import ops


@pytest.fixture
def on(monkeypatch):
    monkeypatch.setenv("KDA_DEBUG_VALIDATE", "1")


def decode_inputs(N=3, T=1, H=2, d=64, num_slots=5):
    z = lambda *s: torch.zeros(*s)
    return dict(q=z(N, T, H, d), k=z(N, T, H, d), v=z(N, T, H, d), g=z(N, T, H, d),
                beta=z(N, T, H), state_pool=z(num_slots, H, d, d))


def prefill_inputs(T=10, H=2, d=64, num_slots=4):
    z = lambda *s: torch.zeros(*s)
    return dict(q=z(T, H, d), k=z(T, H, d), v=z(T, H, d), g=z(T, H, d), beta=z(T, H),
                state_pool=z(num_slots, H, d, d))


def i32(*x):
    return torch.tensor(x, dtype=torch.int32)


def test_switch(monkeypatch):
    monkeypatch.delenv("KDA_DEBUG_VALIDATE", raising=False)
    assert not ops.debug_validate_enabled()
    monkeypatch.setenv("KDA_DEBUG_VALIDATE", "0")
    assert not ops.debug_validate_enabled()
    monkeypatch.setenv("KDA_DEBUG_VALIDATE", "1")
    assert ops.debug_validate_enabled()


@pytest.mark.parametrize("slots,msg", [((0, 1, 1), "duplicate"), ((0, 5, 1), ">= num_slots")])
def test_decode_slots(on, slots, msg):
    x = decode_inputs()
    with pytest.raises(ValueError, match=msg):
        ops.decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], x["state_pool"], i32(*slots))


def test_skipped_decode_slots_are_allowed():
    assert ops.validate_slots(i32(-1, 3, -1, 0), 4, allow_skip=True) == [3, 0]
    with pytest.raises(ValueError, match="negative"):
        ops.validate_slots(i32(-1, 3), 4, allow_skip=False)


@pytest.mark.parametrize("acc", [(0, 9), (-1, 2)])
def test_replay_accepted_lengths(on, acc):
    pool = torch.zeros(4, 2, 64, 64)
    rec = torch.zeros(2, 8, 2, 192)
    with pytest.raises(ValueError, match="accepted_len"):
        ops.replay_commit(pool, i32(0, 1), rec, i32(*acc))


def test_replay_duplicate_slots(on):
    with pytest.raises(ValueError, match="duplicate"):
        ops.replay_commit(torch.zeros(4, 2, 64, 64), i32(2, 2), torch.zeros(2, 8, 2, 192),
                          i32(1, 1))


@pytest.mark.parametrize("cu,msg", [((1, 4, 10), r"\[0\]"), ((0, 6, 4, 10), "decreases"),
                                    ((0, 4, 9), r"\[-1\]")])
def test_prefill_cu_seqlens(on, cu, msg):
    x = prefill_inputs()
    slots = i32(*range(len(cu) - 1))
    with pytest.raises(ValueError, match=msg):
        ops.chunk_prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], i32(*cu), x["state_pool"],
                          slots)


@pytest.mark.parametrize("slots,msg", [((0, -1), "negative"), ((3, 3), "duplicate"),
                                       ((0, 4), ">= num_slots")])
def test_prefill_slots(on, slots, msg):
    x = prefill_inputs()
    for fn in (ops.chunk_prefill, ops.chunk_prefill_noalloc):
        with pytest.raises(ValueError, match=msg):
            fn(x["q"], x["k"], x["v"], x["g"], x["beta"], i32(0, 4, 10), x["state_pool"], i32(*slots))


def test_prefill_snapshot_slots(on):
    x = prefill_inputs(num_slots=8)
    args = (x["q"], x["k"], x["v"], x["g"], x["beta"], i32(0, 4, 10), x["state_pool"], i32(0, 1))
    for snaps, msg in (([[2, 1], [3, -1]], "final-state"), ([[2, 3], [3, -1]], "duplicate"),
                       ([[2, 8], [3, -1]], ">= num_slots")):
        with pytest.raises(ValueError, match=msg):
            ops.chunk_prefill(*args, snapshot_every=64, snapshot_slots=torch.tensor(snaps, dtype=torch.int32))


def front_tensors(H=2, d=64, num_slots=5, W=4):
    z = lambda *s: torch.zeros(*s)
    return dict(gate_scale=z(H), conv_q=z(H, d, W), conv_k=z(H, d, W), conv_v=z(H, d, W),
                conv_state=z(num_slots, H, W - 1, 3 * d))


@pytest.mark.parametrize("slots,msg", [((0, 7, 1), "num_slots"), ((2, 2, 1), "duplicate")])
def test_decode_front_slots(on, slots, msg):
    x = decode_inputs()
    with pytest.raises(ValueError, match=msg):
        ops.decode_step_front(x["q"], x["k"], x["v"], x["g"], x["beta"], x["state_pool"], i32(*slots),
                              **front_tensors())


@pytest.mark.parametrize("cu,msg", [((0, 4, 11), "total_tokens"), ((1, 4, 10), r"\[0\]")])
def test_prefill_front_cu_seqlens(on, cu, msg):
    x = prefill_inputs()
    with pytest.raises(ValueError, match=msg):
        ops.chunk_prefill_front(x["q"], x["k"], x["v"], x["g"], x["beta"], i32(*cu), x["state_pool"], i32(0, 1),
                                **front_tensors(num_slots=4))
