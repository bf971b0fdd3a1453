"""The float32 oracle against an independent float64 implementation (tests/ref_f64.py) of the
whole frame on the tiny configuration: 16 frames, the f64 side fed the oracle's generated tokens.
Logits agree to 1e-5 of their largest magnitude (float32 rounding over 2 + 2 layers), the
gathered inputs exactly, and every greedy token whose float64 top-2 margin is clear of that
error."""
import numpy as np

import synth
from oracle import OracleLM
from tests.ref_f64 import RefF64


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / np.max(np.abs(b)))


def test_oracle_matches_an_independent_float64_frame():
    cfg = synth.TINY
    w = synth.gen_weights(cfg)
    lm = OracleLM(cfg, w)
    st = lm.new_state()
    ref = RefF64(cfg, w)
    users = synth.user_tokens(cfg, cfg.frames)
    worst, checked = 0.0, 0
    for t in range(cfg.frames):
        tr = lm.step(st, users[t])
        toks, emb, hid, tlog = ref.frame(t, users[t])
        assert [int(v) for v in tr["input_tokens"]] == toks, t
        np.testing.assert_allclose(tr["emb_sum"], emb, rtol=1e-6, atol=1e-7)
        worst = max(worst, _rel(tr["transformer_out"], hid), _rel(tr["text_logits"], tlog))
        prevs = [tr["text_token"]] + tr["audio_tokens"][:-1]
        alog = ref.depformer(tr["transformer_out"].astype(np.float64), prevs)
        for cb in range(cfg.dep_q):
            worst = max(worst, _rel(tr["audio_logits"][cb], alog[cb]))
        for lg, tok in [(tlog, tr["text_token"])] + [(alog[cb], tr["audio_tokens"][cb]) for cb in range(cfg.dep_q)]:
            s = np.sort(lg)
            if s[-1] - s[-2] > 1e-3 * np.max(np.abs(lg)):
                assert int(np.argmax(lg)) == tok, t
                checked += 1
        ref.gen[t] = [tr["text_token"]] + tr["audio_tokens"]
    assert worst <= 1e-5, worst
    assert checked >= 0.9 * cfg.frames * (1 + cfg.dep_q)
