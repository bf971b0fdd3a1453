"""Moshi-7B-shaped bfloat16 parity (B=1, seed-1 weights): the GPU frame step, teacher-forced onto
the CPU oracle's greedy trajectory ([LM] force_generated), must keep every logits row at cosine
>= 0.999 and agree on >= 99% of the greedy tokens.  The oracle runs the same bf16 weights widened
to float32.  Runs in the persistent configuration the bench times, and in the graph one."""
import time

import numpy as np
import pytest

import rq_transformer_frame_amd as rq
import synth
from oracle import OracleLM
from tests.gpu_util import cosine, top2_margin

pytestmark = pytest.mark.gpu

CFG = synth.MOSHI7B
FRAMES = 4


@pytest.fixture(scope="module")
def weights():
    t = time.time()
    w = synth.gen_weights(CFG)
    print(f"generated 7B weights in {time.time() - t:.1f}s", flush=True)
    return w


@pytest.fixture(scope="module")
def oracle(weights):
    return OracleLM(CFG, weights)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("exec_mode", ["persistent", "graph"])
def test_moshi7b_bf16_teacher_forced_matches_oracle(weights, oracle, exec_mode):
    users = synth.user_tokens(CFG, FRAMES)
    with rq.Session(CFG, exec=exec_mode) as s:
        t = time.time()
        s.load_weights(weights)
        print(f"loaded in {time.time() - t:.1f}s", flush=True)
        lm = oracle
        ost = lm.new_state()
        agree = total = 0
        cos_min = 1.0
        for f in range(FRAMES):
            t = time.time()
            ref = lm.step(ost, users[f])
            s.step(users[f])
            tr = s.read_trace(0)
            assert tr["input_tokens"].tolist() == ref["input_tokens"].tolist()
            rows = [(tr["text_logits"], ref["text_logits"])] + [
                (tr["audio_logits"][c], ref["audio_logits"][c]) for c in range(CFG.dep_q)]
            cs = [cosine(g, o) for g, o in rows]
            cos_min = min(cos_min, *cs)
            got = [tr["text_token"]] + tr["audio_tokens"]
            want = [ref["text_token"]] + ref["audio_tokens"]
            agree += sum(int(a == b) for a, b in zip(got, want))
            total += len(got)
            print(f"frame {f}: min cos {min(cs):.6f} tokens {sum(int(a == b) for a, b in zip(got, want))}/9 "
                  f"text margin {top2_margin(ref['text_logits']):.2e} ({time.time() - t:.1f}s)", flush=True)
            lm.force_generated(ost, ref["text_token"], ref["audio_tokens"])
            s.force_generated(0, ref["text_token"], ref["audio_tokens"])
        print(f"7B bf16: min cosine {cos_min:.6f}, agreement {agree}/{total}", flush=True)
        assert cos_min >= 0.999
        assert agree / total >= 0.99
