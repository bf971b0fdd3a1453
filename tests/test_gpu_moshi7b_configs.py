"""Moshi-7B-shaped parity of the other workloads, each teacher-forced onto a reference run
([LM] force_generated) and judged per frame: every logits row whose conditioning tokens agree at
cosine >= 0.999, and >= 99% of the greedy tokens equal.

- long context: a 2900-frame teacher-forced prefill (row batches on the matrix cores) then greedy
  frames at positions 2900.. on the graph and the persistent executor, against the oracle's
  batched causal prefill;
- int8 weights (per-row scales): against the int8-dequantised oracle (storage loss only); the
  float32 oracle's agreement is printed to separate quantisation loss from kernel error;
- 64 conversations stepped together after per-conversation prefixes: every conversation against
  the same conversation run alone on the single-conversation path (batch invariance), and a
  subset of 8 (b = 0, 63, the smallest and largest prefix, four more) against the oracle.
"""
import time

import numpy as np
import pytest

import rq_transformer_frame_amd as rq
import synth
from oracle import OracleLM
from tests.gpu_util import frame_agreement

pytestmark = pytest.mark.gpu


def tick(msg, t0):
    print(f"{msg} ({time.time() - t0:.1f}s)", flush=True)
    return time.time()


@pytest.mark.timeout(1200)
def test_long_context_prefill_then_greedy_matches_oracle():
    cfg = synth.MOSHI7B_LONG
    T, frames = cfg.prefill, 2
    t0 = time.time()
    w = synth.gen_weights(cfg)
    text, agent, user = synth.prefill_tokens(cfg, T)
    users = synth.user_tokens(cfg, frames, start_frame=T)
    t0 = tick("weights", t0)
    lm = OracleLM(cfg, w)
    st = lm.new_state()
    lm.prefill_forced(st, text, agent, user)
    t0 = tick("oracle prefill", t0)
    refs = []
    for f in range(frames):
        ref = lm.step(st, users[f])
        refs.append(ref)
        lm.force_generated(st, ref["text_token"], ref["audio_tokens"])
    t0 = tick("oracle frames", t0)
    del lm
    # the graph executor, and the persistent one the bench times
    for mode in ("graph", "persistent"):
        with rq.Session(cfg, exec=mode) as s:
            s.load_weights(w)
            s.prefill_forced(0, text, agent, user)
            assert s.offset(0) == T
            t0 = tick(f"{mode}: GPU prefill", t0)
            cos_min, agree, total = 1.0, 0, 0
            for f, ref in enumerate(refs):
                s.step(users[f])
                tr = s.read_trace(0)
                assert tr["input_tokens"].tolist() == ref["input_tokens"].tolist(), (mode, f)
                c, a = frame_agreement(tr, ref)
                cos_min, agree, total = min(cos_min, c), agree + a, total + 9
                s.force_generated(0, ref["text_token"], ref["audio_tokens"])
                t0 = tick(f"{mode}: frame at position {T + f}: min cos {c:.6f}, tokens {a}/9", t0)
        print(f"long context ({mode}): min cosine {cos_min:.6f}, agreement {agree}/{total}")
        assert cos_min >= 0.999
        assert agree / total >= 0.99


@pytest.mark.timeout(1200)
def test_int8_weights_match_dequantised_oracle():
    cfg = synth.MOSHI7B_I8
    frames = 3
    t0 = time.time()
    w = synth.gen_weights(cfg)
    users = synth.user_tokens(cfg, frames)
    t0 = tick("weights", t0)
    lm = OracleLM(cfg, w, band="i8sim")
    t0 = tick("int8-dequantised oracle", t0)
    results = {}
    with rq.Session(cfg) as s:
        s.load_weights(w)
        st = lm.new_state()
        cos_min, agree, total = 1.0, 0, 0
        traces = []
        for f in range(frames):
            ref = lm.step(st, users[f])
            s.step(users[f])
            tr = s.read_trace(0)
            traces.append((tr, ref))
            c, a = frame_agreement(tr, ref)
            cos_min, agree, total = min(cos_min, c), agree + a, total + 9
            lm.force_generated(st, ref["text_token"], ref["audio_tokens"])
            s.force_generated(0, ref["text_token"], ref["audio_tokens"])
            t0 = tick(f"frame {f}: min cos {c:.6f}, tokens {a}/9", t0)
        results["i8sim"] = (cos_min, agree, total)
    del lm
    # quantisation loss, reported: the float32 oracle on the same teacher-forced inputs
    lm32 = OracleLM(cfg, w)
    st = lm32.new_state()
    agree32 = 0
    for f, (tr, ref) in enumerate(traces):
        r32 = lm32.step(st, users[f])
        agree32 += frame_agreement(tr, r32)[1]
        lm32.force_generated(st, ref["text_token"], ref["audio_tokens"])
    print(f"int8: vs dequantised oracle min cosine {results['i8sim'][0]:.6f}, agreement "
          f"{results['i8sim'][1]}/{results['i8sim'][2]}; vs float32 oracle agreement {agree32}/{3 * 9}")
    assert results["i8sim"][0] >= 0.999
    assert results["i8sim"][1] / results["i8sim"][2] >= 0.99


@pytest.mark.timeout(1500)
def test_batch64_matches_single_conversations_and_oracle_subset():
    cfg = synth.MOSHI7B_B64
    B, frames = cfg.batch, 2
    t0 = time.time()
    w = synth.gen_weights(cfg)
    starts = synth.start_offsets(cfg).astype(int)
    pre = [synth.prefill_tokens(cfg, int(starts[b]), conv=b) for b in range(B)]
    users = np.stack([synth.user_tokens(cfg, frames, conv=b, start_frame=int(starts[b])) for b in range(B)], axis=1)
    cap = int(starts.max()) + frames + 1
    t0 = tick("weights and tokens", t0)

    # every conversation alone, on the single-conversation path
    single = []
    with rq.Session(cfg, batch=1, kv_capacity=cap) as s1:
        s1.load_weights(w)
        for b in range(B):
            s1.reset()
            if starts[b]:
                s1.prefill_forced(0, *pre[b])
            run = []
            for f in range(frames):
                s1.step(users[f, b])
                tr = s1.read_trace(0)
                run.append(tr)
                s1.force_generated(0, tr["text_token"], tr["audio_tokens"])
            single.append(run)
    t0 = tick("64 single-conversation runs", t0)

    batched = [[None] * frames for _ in range(B)]
    with rq.Session(cfg, kv_capacity=cap) as s:
        s.load_weights(w)
        for b in range(B):
            if starts[b]:
                s.prefill_forced(b, *pre[b])
        t0 = tick("64 prefixes", t0)
        for f in range(frames):
            s.step(users[f])
            for b in range(B):
                batched[b][f] = s.read_trace(b)
                ref = single[b][f]
                s.force_generated(b, ref["text_token"], ref["audio_tokens"])
    t0 = tick("batched frames", t0)
    cos_min, agree, total = 1.0, 0, 0
    for b in range(B):
        for f in range(frames):
            c, a = frame_agreement(batched[b][f], single[b][f])
            cos_min, agree, total = min(cos_min, c), agree + a, total + 9
    print(f"B=64 vs B=1: min cosine {cos_min:.6f}, agreement {agree}/{total}")
    assert cos_min >= 0.999
    assert agree / total >= 0.99

    # oracle subset: b = 0, 63, the smallest and largest prefix, and four more
    order = np.argsort(starts, kind="stable")
    subset = sorted({0, B - 1, int(order[0]), int(order[-1]), 16, 31, 40, 52})
    lm = OracleLM(cfg, w)
    cos_min, agree, total = 1.0, 0, 0
    for b in subset:
        st = lm.new_state()
        if starts[b]:
            lm.prefill_forced(st, *pre[b])
        for f in range(frames):
            ref = lm.step(st, users[f, b])
            c, a = frame_agreement(batched[b][f], ref)
            cos_min, agree, total = min(cos_min, c), agree + a, total + 9
            tr = single[b][f]
            lm.force_generated(st, tr["text_token"], tr["audio_tokens"])
        t0 = tick(f"oracle conversation {b} (prefix {starts[b]})", t0)
    print(f"B=64 vs oracle on {subset}: min cosine {cos_min:.6f}, agreement {agree}/{total}")
    assert cos_min >= 0.999
    assert agree / total >= 0.99
