"""Sampled decoding on the GPU against the oracle ([LM] Sampling, MoshiLm::pick, topk_sample,
gumbel_full_pick, xorshift_u01).  Both sides draw from their own xorshift stream started at the
same seed: the oracle sequentially, the GPU with jump-ahead tables (a thread starts at its own
index).  The tokens, the logits and the stream state after every frame must match; the GPU's
picks must also equal the oracle's pick functions applied to the GPU's own logits (the sampling
arithmetic alone)."""
import numpy as np
import pytest

import rq_transformer_frame_amd as rq
import synth
from oracle import OracleLM, moshi_oracle as O
from tests.gpu_util import TraceStats, rel_err

pytestmark = pytest.mark.gpu

CFG = synth.TINY
TOL = 1e-4
SEED = 0x5EED1234


@pytest.fixture(scope="module")
def weights():
    return synth.gen_weights(CFG)


@pytest.fixture(scope="module")
def oracle(weights):
    return OracleLM(CFG, weights)


def picks_from_own_logits(tr, mode, state):
    """The oracle's pick functions on the GPU's logits, from the stream state before the frame."""
    smp = O.Sampling(seed=state, gumbel_full=(mode == "gumbel"))
    toks = [O.pick(tr["text_logits"], True, smp)]
    toks += [O.pick(tr["audio_logits"][cb], False, smp) for cb in range(CFG.dep_q)]
    return toks, smp.state


@pytest.mark.parametrize("exec_mode,mode", [("graph", "topk"), ("graph", "gumbel"), ("stream", "topk"),
                                            ("persistent", "gumbel")])
def test_sampled_frames_match_oracle(weights, oracle, exec_mode, mode):
    frames = 12
    users = synth.user_tokens(CFG, frames, conv=7)
    smp = O.Sampling(seed=SEED, gumbel_full=(mode == "gumbel"))
    ost = oracle.new_state()
    with rq.Session(CFG, exec=exec_mode) as s:
        s.load_weights(weights)
        s.set_sampling(0, mode, seed=SEED)
        assert s.sampler_state(0) == SEED
        for f in range(frames):
            before = s.sampler_state(0)
            ref = oracle.step(ost, users[f], smp)
            st, out, has = s.step(users[f])
            tr = s.read_trace(0)
            assert rel_err(tr["text_logits"], ref["text_logits"]) <= TOL, f
            own, after = picks_from_own_logits(tr, mode, before)
            assert tr["tokens"].tolist() == own, f  # the sampling arithmetic alone
            assert tr["tokens"].tolist() == [ref["text_token"]] + ref["audio_tokens"], f
            assert s.sampler_state(0) == smp.state == after, f
            if ref["out"] is not None:
                assert out[0].tolist() == ref["out"], f


def test_batched_conversations_sample_their_own_streams(weights, oracle):
    """Three conversations stepped together on the batched path: greedy, top-k and Gumbel-max,
    each with its own seed, each equal to its own oracle run."""
    frames = 8
    modes = ["greedy", "topk", "gumbel"]
    users = [synth.user_tokens(CFG, frames, conv=10 + b) for b in range(3)]
    smps = [None if m == "greedy" else O.Sampling(seed=SEED + 17 * b, gumbel_full=(m == "gumbel"))
            for b, m in enumerate(modes)]
    osts = [oracle.new_state() for _ in range(3)]
    with rq.Session(CFG, exec="graph", batch=3) as s:
        s.load_weights(weights)
        for b, m in enumerate(modes):
            s.set_sampling(b, m, seed=SEED + 17 * b)
        for f in range(frames):
            s.step(np.stack([users[b][f] for b in range(3)]))
            for b in range(3):
                ref = oracle.step(osts[b], users[b][f], smps[b])
                tr = s.read_trace(b)
                assert rel_err(tr["text_logits"], ref["text_logits"]) <= TOL, (b, f)
                assert tr["tokens"].tolist() == [ref["text_token"]] + ref["audio_tokens"], (b, f)
                if smps[b] is not None:
                    assert s.sampler_state(b) == smps[b].state, (b, f)


def test_switching_modes_recaptures_and_keeps_parity(weights, oracle):
    """greedy -> top-k (non-default k and temperatures) -> greedy on one graph session."""
    users = synth.user_tokens(CFG, 9, conv=12)
    ost = oracle.new_state()
    with rq.Session(CFG, exec="graph") as s:
        s.load_weights(weights)
        smp = None
        for f in range(9):
            if f == 3:
                s.set_sampling(0, "topk", seed=99, temp=1.3, temp_text=0.5, top_k=40, top_k_text=7)
                smp = O.Sampling(seed=99, temp=1.3, temp_text=0.5, top_k=40, top_k_text=7)
            if f == 6:
                s.set_sampling(0, "greedy")
                smp = None
            ref = oracle.step(ost, users[f], smp)
            s.step(users[f])
            tr = s.read_trace(0)
            assert tr["tokens"].tolist() == [ref["text_token"]] + ref["audio_tokens"], f


def test_sampling_arguments_are_checked(weights):
    with rq.Session(CFG, exec="persistent") as p:
        with pytest.raises(rq.MoshiError) as ei:
            p.set_sampling(0, "topk")
        assert ei.value.status == rq.MOSHI_EINVAL
        p.set_sampling(0, "gumbel", seed=3)
    with rq.Session(CFG, exec="graph") as g:
        for kw in (dict(temp=0.0), dict(top_k=0), dict(top_k_text=2000), dict(temp_text=float("nan"))):
            with pytest.raises(rq.MoshiError) as ei:
                g.set_sampling(0, "topk", **kw)
            assert ei.value.status == rq.MOSHI_EINVAL


@pytest.mark.timeout(900)
@pytest.mark.parametrize("exec_mode,mode", [("persistent", "gumbel"), ("graph", "topk")])
def test_moshi7b_sampled_frames_match_oracle(exec_mode, mode):
    """Moshi-7B shape, bf16 weights: 30 sampled frames, the GPU teacher-forced onto the oracle's
    sampled tokens (both streams advance by the same draws whatever is picked: Gumbel-max one per
    logit, top-k one per pick); logits cosine >= 0.999, tokens >= 99% equal, every differing pick
    explained by the GPU's own logits, and the stream states equal after every frame."""
    cfg = synth.MOSHI7B
    frames = 30
    w = synth.gen_weights(cfg)
    lm = OracleLM(cfg, w)
    users = synth.user_tokens(cfg, frames, conv=3)
    smp = O.Sampling(seed=SEED, gumbel_full=(mode == "gumbel"))
    ost = lm.new_state()
    stats = TraceStats()
    own_ok = 0
    with rq.Session(cfg, exec=exec_mode) as s:
        s.load_weights(w)
        s.set_sampling(0, mode, seed=SEED)
        for f in range(frames):
            before = s.sampler_state(0)
            ref = lm.step(ost, users[f], smp)
            s.step(users[f])
            tr = s.read_trace(0)
            stats.add(tr, ref)
            own, after = picks_from_own_logits(tr, mode, before)
            own_ok += int(tr["tokens"].tolist() == own)
            assert s.sampler_state(0) == smp.state == after, f
            s.force_generated(0, ref["text_token"], ref["audio_tokens"])
    print(f"7B {mode} ({exec_mode}): {stats}; frames whose picks equal the oracle's on the GPU logits "
          f"{own_ok}/{frames}", flush=True)
    assert own_ok == frames
    assert stats.cos_min >= 0.999
    assert stats.rate >= 0.99
