"""Session snapshot and restore on the device ([LM] MoshiState::snapshot: the ring, the offset and
the KV cache together restore a primed session).  A restored conversation must continue exactly
as the original did (bitwise, same executor), and as the oracle's snapshot does; restoring into
another session or conversation (another batch or kv_capacity) must match the oracle too."""
import time

import numpy as np
import pytest

import rq_transformer_frame_amd as rq
import synth
from oracle import OracleLM
from tests.gpu_util import rel_err

pytestmark = pytest.mark.gpu

CFG = synth.TINY
TOL = 1e-4


@pytest.fixture(scope="module")
def weights():
    return synth.gen_weights(CFG)


@pytest.fixture(scope="module")
def oracle(weights):
    return OracleLM(CFG, weights)


def check(tr, ref, what):
    assert tr["input_tokens"].tolist() == ref["input_tokens"].tolist(), what
    assert rel_err(tr["text_logits"], ref["text_logits"]) <= TOL, what
    assert tr["tokens"].tolist() == [ref["text_token"]] + ref["audio_tokens"], what


@pytest.mark.parametrize("exec_mode", ["persistent", "graph"])
def test_restore_replays_the_same_frames(weights, oracle, exec_mode):
    T = 30
    text, agent, user = synth.prefill_tokens(CFG, T, conv=4)
    text %= CFG.text_card
    users = synth.user_tokens(CFG, 9, conv=4, start_frame=T)
    ost = oracle.new_state()
    oracle.prefill_forced(ost, text, agent, user)
    with rq.Session(CFG, exec=exec_mode) as s:
        s.load_weights(weights)
        s.prefill_forced(0, text, agent, user)
        for f in range(3):
            s.step(users[f])
            oracle.step(ost, users[f])
        snap = s.snapshot(0)
        osnap = ost.snapshot()
        assert snap.info()[:2] == (T + 3, T + 3)
        first = []
        for f in range(3, 9):
            _, out, has = s.step(users[f])
            first.append((s.read_trace(0), out.copy()))
        s.restore(0, snap)
        assert s.offset(0) == T + 3
        for f in range(3, 9):
            _, out, has = s.step(users[f])
            tr = s.read_trace(0)
            a, a_out = first[f - 3]
            assert tr["tokens"].tolist() == a["tokens"].tolist(), f
            assert tr["text_logits"].tobytes() == a["text_logits"].tobytes(), f
            assert tr["audio_logits"].tobytes() == a["audio_logits"].tobytes(), f
            assert out.tolist() == a_out.tolist(), f
            check(tr, oracle.step(osnap, users[f]), f)
        snap.free()


def test_restore_into_another_session_and_conversation_past_the_window(weights, oracle):
    """A snapshot taken past the context window (70 positions, context 64: the KV ring has
    wrapped) restored into conversation 1 of a three-conversation session (batched frame path)
    and into a fresh single-conversation persistent session."""
    users = synth.user_tokens(CFG, 76, conv=5)
    ost = oracle.new_state()
    with rq.Session(CFG, exec="graph") as s:
        s.load_weights(weights)
        for f in range(70):
            s.step(users[f])
            oracle.step(ost, users[f])
        snap = s.snapshot(0)
    osnap = ost.snapshot()
    assert snap.info()[:2] == (70, 64)
    with rq.Session(CFG, exec="graph", batch=3) as b3, rq.Session(CFG, exec="persistent") as p1:
        b3.load_weights(weights)
        p1.load_weights(weights)
        b3.restore(1, snap)
        p1.restore(0, snap)
        assert b3.offset(1) == 70 and b3.offset(0) == 0 and p1.offset(0) == 70
        for f in range(70, 76):
            ref = oracle.step(osnap, users[f])
            b3.step(np.stack([users[f]] * 3))
            check(b3.read_trace(1), ref, ("batch", f))
            p1.step(users[f])
            check(p1.read_trace(0), ref, ("persistent", f))
    snap.free()


def test_restore_rejects_other_models_and_small_capacity(weights):
    with rq.Session(CFG, exec="graph") as s:
        s.load_weights(weights)
        for f in range(5):
            s.step(synth.user_tokens(CFG, 5)[f])
        snap = s.snapshot(0)
    with rq.Session(CFG, exec="graph", band="bf16") as other:
        with pytest.raises(rq.MoshiError) as ei:
            other.restore(0, snap)
        assert ei.value.status == rq.MOSHI_EINVAL
    with rq.Session(CFG, exec="graph", kv_capacity=4) as small:
        with pytest.raises(rq.MoshiError) as ei:
            small.restore(0, snap)
        assert ei.value.status == rq.MOSHI_ERANGE
    with rq.Session(CFG, exec="graph", kv_capacity=8) as roomy:
        roomy.load_weights(weights)
        roomy.restore(0, snap)
        assert roomy.offset(0) == 5
    snap.free()


@pytest.mark.timeout(600)
def test_long_context_restore_is_instant_and_exact():
    """Moshi-7B shape after the 2900-frame prefill: restoring the primed session (2 x 32 layers x
    2900 positions of float32 KV, 3 GB) takes milliseconds on the device, and the frame after the
    restore equals the frame after the prefill bit for bit."""
    cfg = synth.MOSHI7B_LONG
    T = cfg.prefill
    w = synth.gen_weights(cfg)
    text, agent, user = synth.prefill_tokens(cfg, T)
    u = synth.user_tokens(cfg, 1, start_frame=T)[0]
    with rq.Session(cfg, exec="persistent") as s:
        s.load_weights(w)
        t0 = time.perf_counter()
        s.prefill_forced(0, text, agent, user)
        t_pre = time.perf_counter() - t0
        snap = s.snapshot(0)
        s.step(u)
        a = s.read_trace(0)
        t0 = time.perf_counter()
        s.restore(0, snap)
        t_res = time.perf_counter() - t0
        s.step(u)
        b = s.read_trace(0)
        off, n, nbytes = snap.info()
        print(f"prefill of {T} frames {t_pre:.3f}s; restore of {n} positions ({nbytes / 1e9:.2f} GB) "
              f"{1e3 * t_res:.2f} ms", flush=True)
        assert (off, n) == (T, T)
        assert a["tokens"].tolist() == b["tokens"].tolist()
        assert a["text_logits"].tobytes() == b["text_logits"].tobytes()
        assert t_res < t_pre
        snap.free()
