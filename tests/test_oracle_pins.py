"""Pins of the CPU oracle to facts the pages and mathematics fix (no GPU).

Each test targets a plausible mistake: a dropped term, a wrong sign or index, a swapped operand,
eps outside the mean, rotate-half instead of interleaved pairs, a norm in the wrong place, a wrong
ring slot.  Page references are to the docs.rs source page inferencelayer 0.2.4 src/moshi_lm.rs
("[LM]") unless stated.
"""
import math

import numpy as np
import pytest

import synth
from oracle import moshi_oracle as O

F32 = np.float32


# ------------------------------------------------------------------ RMSNorm ([LM] rms_norm)

def test_rms_norm_constant_vector_closed_form():
    alpha = np.arange(1, 9, dtype=F32)
    y = O.rms_norm(np.full(8, 3.0, F32), alpha, 1e-8)
    np.testing.assert_allclose(y, alpha * 3.0 / math.sqrt(1e-8 + 9.0), rtol=1e-6)


def test_rms_norm_eps_inside_the_mean():
    # mean(x^2) == eps, so eps inside the mean gives x / sqrt(2 x^2) = 1/sqrt(2); eps outside the
    # square root or no eps would give ~1.
    y = O.rms_norm(np.full(16, 1e-4, F32), np.ones(16, F32), 1e-8)
    np.testing.assert_allclose(y, 1 / math.sqrt(2), rtol=2e-6)


def test_rms_norm_zero_and_scale_invariance():
    assert np.all(O.rms_norm(np.zeros(5, F32), np.ones(5, F32), 1e-8) == 0)
    x = synth.normal(7, "pin/rms", (64,), 1.0)
    a = O.rms_norm(x, np.ones(64, F32), 1e-8)
    b = O.rms_norm(x * F32(1000), np.ones(64, F32), 1e-8)
    np.testing.assert_allclose(a, b, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(np.mean(a.astype(np.float64) ** 2), 1.0, rtol=1e-5)


def test_rms_norm_matches_float64_definition():
    x = synth.normal(7, "pin/rms2", (300,), 2.0)
    al = synth.normal(7, "pin/rms2a", (300,), 1.0)
    x64, a64 = x.astype(np.float64), al.astype(np.float64)
    ref = x64 * a64 / np.sqrt(1e-8 + np.mean(x64 * x64))
    np.testing.assert_allclose(O.rms_norm(x, al, 1e-8), ref, rtol=2e-6, atol=1e-7)


# ------------------------------------------------------------------ rope ([LM] rope_row)

def test_rope_position_zero_is_identity():
    x = synth.normal(1, "pin/rope0", (256,), 1.0)
    assert np.array_equal(O.rope_interleaved(x, 0, 64), x)


def test_rope_head_dim_two_rotates_by_pos_radians_counterclockwise():
    for p in (1, 2, 7, 100):
        y = O.rope_interleaved(np.array([1.0, 0.0], F32), p, 2)
        np.testing.assert_allclose(y, [math.cos(p), math.sin(p)], atol=2e-6)


def test_rope_frequency_exponent_uses_2i_over_head_dim():
    # head_dim 4: pair 1 has f = theta^(-2/4) = 0.01, so at pos 3 it turns by 0.03 rad.
    y = O.rope_interleaved(np.array([0, 0, 1, 0], F32), 3, 4)
    np.testing.assert_allclose(y, [0, 0, math.cos(0.03), math.sin(0.03)], atol=1e-6)
    np.testing.assert_allclose(O.rope_freqs(128)[:3], [1.0, 10000 ** (-2 / 128), 10000 ** (-4 / 128)], rtol=1e-6)


def test_rope_pairs_are_interleaved_not_rotate_half():
    # element 1 is the imaginary part of pair (0, 1), which turns at f_0 = 1; rotate-half would pair
    # it with element 3 at f_1 = 0.01.
    p = 5
    y = O.rope_interleaved(np.array([0, 1, 0, 0], F32), p, 4)
    np.testing.assert_allclose(y, [-math.sin(p), math.cos(p), 0, 0], atol=2e-6)


def test_rope_preserves_pair_norms_and_relative_position():
    q = synth.normal(2, "pin/rq", (128,), 1.0)
    k = synth.normal(2, "pin/rk", (128,), 1.0)
    for m, n in ((9, 4), (40, 40), (300, 17)):
        rq = O.rope_interleaved(q, m, 128)
        np.testing.assert_allclose(np.hypot(rq[0::2], rq[1::2]), np.hypot(q[0::2], q[1::2]), rtol=1e-5)
        lhs = float(np.dot(rq.astype(np.float64), O.rope_interleaved(k, n, 128)))
        rhs = float(np.dot(O.rope_interleaved(q, m - n, 128).astype(np.float64), k))
        assert abs(lhs - rhs) < 2e-4 * (1 + abs(rhs))


# ------------------------------------------------------------------ attention ([LM] attend)

def test_attend_single_key_returns_value_exactly():
    q = synth.normal(3, "pin/aq", (8,), 1.0)
    K = synth.normal(3, "pin/ak", (1, 8), 1.0)
    V = synth.normal(3, "pin/av", (1, 8), 1.0)
    assert np.array_equal(O.attend(q, K, V, 2, 4), V[0])


def test_attend_equal_keys_average_values():
    q = synth.normal(3, "pin/aq2", (8,), 1.0)
    K = np.tile(synth.normal(3, "pin/ak2", (1, 8), 1.0), (5, 1))
    V = synth.normal(3, "pin/av2", (5, 8), 1.0)
    np.testing.assert_allclose(O.attend(q, K, V, 2, 4), V.mean(0), rtol=1e-5, atol=1e-6)


def test_attend_scale_is_one_over_sqrt_head_dim():
    # head_dim 4: scores a/2 and 0 -> weight on key 1 is sigmoid(a/2).
    a = 3.0
    q = np.array([a, 0, 0, 0], F32)
    K = np.array([[1, 0, 0, 0], [0, 0, 0, 0]], F32)
    V = np.array([[1, 0, 0, 0], [0, 0, 0, 0]], F32)
    w = 1 / (1 + math.exp(-a / 2))
    np.testing.assert_allclose(O.attend(q, K, V, 1, 4)[0], w, rtol=1e-6)


def test_attend_brute_force_float64():
    H, hd, n = 3, 4, 6
    q = synth.normal(4, "pin/bq", (H * hd,), 1.0)
    K = synth.normal(4, "pin/bk", (n, H * hd), 1.0)
    V = synth.normal(4, "pin/bv", (n, H * hd), 1.0)
    ref = np.zeros(H * hd)
    for h in range(H):
        s = [sum(float(q[h * hd + d]) * float(K[j, h * hd + d]) for d in range(hd)) / math.sqrt(hd) for j in range(n)]
        m = max(s)
        e = [math.exp(v - m) for v in s]
        for d in range(hd):
            ref[h * hd + d] = sum(e[j] * float(V[j, h * hd + d]) for j in range(n)) / sum(e)
    np.testing.assert_allclose(O.attend(q, K, V, H, hd), ref, rtol=1e-5, atol=1e-6)


def test_attend_heads_are_independent():
    q = synth.normal(5, "pin/hq", (8,), 1.0)
    K = synth.normal(5, "pin/hk", (3, 8), 1.0)
    V = synth.normal(5, "pin/hv", (3, 8), 1.0)
    a = O.attend(q, K, V, 2, 4)
    K2 = K.copy()
    K2[0, 4:] += 5
    b = O.attend(q, K2, V, 2, 4)
    assert np.array_equal(a[:4], b[:4]) and not np.allclose(a[4:], b[4:])


# ------------------------------------------------------------------ silu, argmax, embed

def test_silu_closed_forms():
    y = O.silu(np.array([0, 1, -1, 20, -20], F32))
    np.testing.assert_allclose(y[:3], [0, 1 / (1 + math.exp(-1)), -1 / (1 + math.exp(1))], rtol=1e-6)
    np.testing.assert_allclose(y[3], 20, rtol=1e-6)
    assert abs(y[4]) < 1e-6


@pytest.mark.parametrize("vals,idx", [
    ([1, 3, 3, 2], 1),
    ([float("nan"), 0], 1),
    ([-math.inf, -math.inf], 0),
    ([float("nan"), float("nan")], 0),
    ([-math.inf, 5, 5], 1),
    ([math.inf, 1, math.inf], 0),
    ([-1, -2, -1], 0),
    ([2, float("nan"), 3], 2),
    ([], 0),
])
def test_argmax_first_wins(vals, idx):
    assert O.argmax_first(np.array(vals, F32)) == idx


def test_embed_minus_one_adds_exact_zero_and_clamps_below():
    table = synth.normal(6, "pin/emb", (5, 4), 1.0)
    acc = synth.normal(6, "pin/acc", (4,), 1.0)
    before = acc.copy()
    O.embed_add(acc, table, -1)
    assert acc.tobytes() == before.tobytes()
    O.embed_add(acc, table, -2)
    np.testing.assert_array_equal(acc, before + table[0])
    z = np.zeros(4, F32)
    O.embed_add(z, table, 4)
    np.testing.assert_array_equal(z, table[4])  # the INITIAL token is the last row


# ------------------------------------------------------------------ int8 quantiser

def test_int8_quantiser_hand_values():
    W = np.array([[127.0, 2.5, -2.5, 0.5, -0.5, 1.49, -126.6],
                  [0.0] * 7,
                  [0.254, 0.127, -0.0635, 0.0, 0.01, -0.01, 0.0]], F32)
    q, s = O.quantize_rows_int8(W)
    assert s[0] == 1.0 and s[1] == 0.0
    assert q[0].tolist() == [127, 3, -3, 1, -1, 1, -127]
    assert q[1].tolist() == [0] * 7
    np.testing.assert_allclose(s[2], 0.254 / 127, rtol=1e-6)
    assert q[2].tolist()[:4] == [127, 64, -32, 0]
    err = np.abs(O.dequantize_rows_int8(q, s) - W)
    assert np.all(err <= s[:, None] / 2 + 1e-7)


# ------------------------------------------------------------------ contract constants

def test_stream_delays_and_initial_tokens_as_printed():
    # [LM] DELAYS constant and the module doc's INITIAL tokens (text 32000 / audio 2048)
    assert O.stream_delays(8) == [0, 0, 1, 1, 1, 1, 1, 1, 1, 0, 1, 1, 1, 1, 1, 1, 1]
    assert O.initial_token(0, 32000, 2048) == 32000 and O.initial_token(5, 32000, 2048) == 2048
    assert O.UNGENERATED == -2 and O.RING == 3


# ------------------------------------------------------------------ small model helpers

MINI = synth.Config(
    name="mini", n_layers=2, d_model=16, n_heads=2, ffn_hidden=24, context=4, text_card=40,
    audio_card=32, dep_layers=2, dep_d_model=8, dep_heads=2, dep_ffn_hidden=12, dtype="f32",
    band="f32", seed=11, weight_std=0.5,
)


def mini_weights(cfg=MINI, seed=11):
    return synth.gen_weights(cfg, seed=seed, dtype="f32")


# ------------------------------------------------------------------ ring schedule

def test_ring_schedule_closed_form_with_stub_network():
    """Module doc of [LM]: user tokens are written at (offset + delay) % 3, inputs read at
    offset % 3 with INITIAL while offset <= delay, and from the second step on the output is read
    at (offset - max_delay + delay) % 3.  Worked out by hand this gives, at step t:
      inputs  text, cb0 = INIT if t == 0 else generated(t-1); cb1..7 = INIT if t <= 1 else
              generated(t-1); user cb0 = INIT if t == 0 else user(t); user cb1..7 = INIT if
              t <= 1 else user(t-1)
      output  none at t == 0, else [text(t-1), audio0(t-1), audio1..7(t)]."""
    lm = O.OracleLM(MINI, mini_weights())
    st = lm.new_state()
    Vt, Va = MINI.text_card, MINI.audio_card
    text = lambda t: (100 + t) % Vt  # noqa: E731
    audio = lambda t, cb: (3 * cb + t) % Va  # noqa: E731
    user = lambda t: [(5 * t + k) % Va for k in range(8)]  # noqa: E731
    for t in range(7):
        inp, tt, aa, out = lm.step_with_network(st, user(t), lambda x, pos, t=t: (text(t), [audio(t, c) for c in range(8)]))
        exp_in = [Vt if t == 0 else text(t - 1)]
        exp_in += [Va if t == 0 else audio(t - 1, 0)]
        exp_in += [Va if t <= 1 else audio(t - 1, cb) for cb in range(1, 8)]
        exp_in += [Va if t == 0 else user(t)[0]]
        exp_in += [Va if t <= 1 else user(t - 1)[k] for k in range(1, 8)]
        assert inp.tolist() == exp_in, t
        if t == 0:
            assert out is None
        else:
            assert out == [text(t - 1), audio(t - 1, 0)] + [audio(t, cb) for cb in range(1, 8)], t
        assert st.offset == t + 1


def test_force_generated_replaces_what_the_next_step_reads():
    lm = O.OracleLM(MINI, mini_weights())
    st = lm.new_state()
    net = lambda x, pos: (7, [1, 2, 3, 4, 5, 6, 7, 8])  # noqa: E731
    lm.step_with_network(st, [0] * 8, net)
    lm.step_with_network(st, [0] * 8, net)
    lm.force_generated(st, 33, [9, 10, 11, 12, 13, 14, 15, 16])
    inp, _, _, out = lm.step_with_network(st, [0] * 8, net)
    assert inp[:9].tolist() == [33, 9, 10, 11, 12, 13, 14, 15, 16]
    assert out == [33, 9, 2, 3, 4, 5, 6, 7, 8]


# ------------------------------------------------------------------ model wiring

def _zero_temporal(w, cfg):
    for l in range(cfg.n_layers):
        p = f"transformer.layers.{l}"
        for n in ("self_attn.in_projs.0", "self_attn.out_projs.0", "gating.linear_in", "gating.linear_out"):
            w[f"{p}.{n}.weight"][:] = 0


def _zero_depformer_layers(w, cfg):
    for l in range(cfg.dep_layers):
        p = f"depformer.layers.{l}"
        for s in range(cfg.dep_q):
            for n in (f"self_attn.in_projs.{s}", f"self_attn.out_projs.{s}", f"gating.{s}.linear_in", f"gating.{s}.linear_out"):
                w[f"{p}.{n}.weight"][:] = 0


def test_embedding_sum_residual_path_and_out_norm_before_head():
    """With every temporal linear zero the stack is the identity on the residual stream, so the
    hidden is out_norm(embedding sum) and the text logits are text_linear . hidden."""
    w = mini_weights()
    _zero_temporal(w, MINI)
    w["out_norm.alpha"][:] = synth.normal(1, "pin/outnorm", (MINI.d_model,), 1.0)
    lm = O.OracleLM(MINI, w)
    st = lm.new_state()
    tr = lm.step(st, list(range(8)))
    Vt, Va = MINI.text_card, MINI.audio_card
    x0 = sum(w[f"emb.{k}.weight"][Va].astype(np.float64) for k in range(16)) + w["text_emb.weight"][Vt]
    np.testing.assert_allclose(tr["emb_sum"], x0, rtol=1e-5, atol=1e-6)
    x064 = x0.astype(np.float64)
    hid = x064 * w["out_norm.alpha"] / np.sqrt(1e-8 + np.mean(x064 ** 2))
    np.testing.assert_allclose(tr["transformer_out"], hid, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(tr["text_logits"], w["text_linear.weight"].astype(np.float64) @ hid, rtol=1e-4, atol=1e-5)
    assert tr["text_token"] == int(np.argmax(tr["text_logits"]))


def test_depformer_input_tables_prev_chain_and_head_without_norm():
    """With the depformer layers zero, step cb's logits are linears[cb] . (depformer_in[cb] .
    hidden + table_cb[prev]), table_0 = the depformer text table with prev = text token and
    table_cb = depformer_emb[cb-1] with prev = audio[cb-1]; no norm before the head."""
    w = mini_weights()
    _zero_depformer_layers(w, MINI)
    lm = O.OracleLM(MINI, w)
    st = lm.new_state()
    for t in range(3):
        tr = lm.step(st, [(t + k) % MINI.audio_card for k in range(8)])
        hid = tr["transformer_out"].astype(np.float64)
        prev = tr["text_token"]
        for cb in range(8):
            table = w["depformer_text_emb.weight"] if cb == 0 else w[f"depformer_emb.{cb - 1}.weight"]
            y = w[f"depformer_in.{cb}.weight"].astype(np.float64) @ hid + table[prev]
            np.testing.assert_allclose(tr["audio_logits"][cb], w[f"linears.{cb}.weight"] @ y, rtol=1e-4, atol=1e-5)
            prev = tr["audio_tokens"][cb]


def test_gated_ffn_uses_silu_of_first_half_times_second_half():
    """One temporal layer with the attention branch zero: x1 = x0 + W_out_ffn (silu(g[:F]) * g[F:])
    with g = linear_in . rms_norm(x0; norm2)."""
    cfg = MINI.with_(n_layers=1)
    w = mini_weights(cfg)
    p = "transformer.layers.0"
    w[f"{p}.self_attn.out_projs.0.weight"][:] = 0
    w[f"{p}.norm2.alpha"][:] = synth.normal(2, "pin/n2", (cfg.d_model,), 1.0)
    w["out_norm.alpha"][:] = 1
    lm = O.OracleLM(cfg, w)
    tr = lm.step(lm.new_state(), [1] * 8)
    x0 = tr["emb_sum"].astype(np.float64)
    h = x0 * w[f"{p}.norm2.alpha"] / np.sqrt(1e-8 + np.mean(x0 ** 2))
    g = w[f"{p}.gating.linear_in.weight"] @ h
    F = cfg.ffn_hidden
    x1 = x0 + w[f"{p}.gating.linear_out.weight"] @ (g[:F] / (1 + np.exp(-g[:F])) * g[F:])
    np.testing.assert_allclose(tr["transformer_out"], x1 / np.sqrt(1e-8 + np.mean(x1 ** 2)), rtol=1e-4, atol=1e-5)


def test_temporal_window_and_kv_push_order():
    """q rows zero make every score 0, so attention is the plain mean of the values in the window;
    with v rows = identity and out_proj = identity (FFN zero) the layer adds the mean of
    rms_norm(x_j) over the last `context` positions j <= pos ([LM] temporal_step window)."""
    cfg = MINI.with_(n_layers=1, context=3)
    D = cfg.d_model
    w = mini_weights(cfg)
    p = "transformer.layers.0"
    Win = np.zeros((3 * D, D), F32)
    Win[D:2 * D] = synth.normal(3, "pin/wk", (D, D), 1.0)
    Win[2 * D:] = np.eye(D, dtype=F32)
    w[f"{p}.self_attn.in_projs.0.weight"][:] = Win
    w[f"{p}.self_attn.out_projs.0.weight"][:] = np.eye(D, dtype=F32)
    w[f"{p}.gating.linear_out.weight"][:] = 0
    lm = O.OracleLM(cfg, w)
    st = lm.new_state()
    hs = []
    for t in range(7):
        tr = lm.step(st, [(3 * t + k) % cfg.audio_card for k in range(8)])
        x0 = tr["emb_sum"].astype(np.float64)
        hs.append(x0 / np.sqrt(1e-8 + np.mean(x0 ** 2)))
        x1 = x0 + np.mean(hs[-3:], axis=0)
        np.testing.assert_allclose(tr["transformer_out"], x1 / np.sqrt(1e-8 + np.mean(x1 ** 2)), rtol=1e-4, atol=1e-5)


def test_depformer_step_cb_attends_exactly_cb_plus_one_entries():
    """In the first dep layer, q and k rows zero give uniform attention; v rows = identity and
    out_proj = identity add the mean of rms_norm(y_j) over j <= cb (the per-frame KV); a second
    layer and the FFNs are zero and linears[cb] = [I; 0] exposes y in the logits."""
    cfg = MINI.with_(dep_layers=1)
    Dd = cfg.dep_d_model
    w = mini_weights(cfg)
    p = "depformer.layers.0"
    for s in range(8):
        Win = np.zeros((3 * Dd, Dd), F32)
        Win[2 * Dd:] = np.eye(Dd, dtype=F32)
        w[f"{p}.self_attn.in_projs.{s}.weight"][:] = Win
        w[f"{p}.self_attn.out_projs.{s}.weight"][:] = np.eye(Dd, dtype=F32)
        w[f"{p}.gating.{s}.linear_out.weight"][:] = 0
        lin = np.zeros((cfg.audio_card, Dd), F32)
        lin[:Dd] = np.eye(Dd, dtype=F32)
        w[f"linears.{s}.weight"][:] = lin
    lm = O.OracleLM(cfg, w)
    st = lm.new_state()
    for t in range(2):
        tr = lm.step(st, [t] * 8)
        hid = tr["transformer_out"].astype(np.float64)
        prev = tr["text_token"]
        ys = []
        for cb in range(8):
            table = w["depformer_text_emb.weight"] if cb == 0 else w[f"depformer_emb.{cb - 1}.weight"]
            y0 = w[f"depformer_in.{cb}.weight"] @ hid + table[prev]
            ys.append(y0 / np.sqrt(1e-8 + np.mean(y0 ** 2)))
            y1 = y0 + np.mean(ys, axis=0)
            np.testing.assert_allclose(tr["audio_logits"][cb][:Dd], y1, rtol=1e-4, atol=1e-5)
            prev = tr["audio_tokens"][cb]


def test_step_forced_sequence_equals_batched_prefill():
    """Decode position by position (step_forced) and the one-shot causal sequence form give the
    same KV cache, ring and following step, also across the context window."""
    cfg = MINI.with_(context=4)
    w = mini_weights(cfg)
    lm = O.OracleLM(cfg, w)
    T = 7
    text = synth.uniform_int(5, "pin/pt", (T,), cfg.text_card)
    agent = synth.uniform_int(5, "pin/pa", (T, 8), cfg.audio_card)
    user = synth.uniform_int(5, "pin/pu", (T, 8), cfg.audio_card)
    a, b = lm.new_state(), lm.new_state()
    for t in range(T):
        lm.step_forced(a, int(text[t]), agent[t], user[t])
    lm.prefill_forced(b, text[:3], agent[:3], user[:3])
    lm.prefill_forced(b, text[3:], agent[3:], user[3:])
    assert a.offset == b.offset == T
    assert np.array_equal(a.ring, b.ring)
    for l in range(cfg.n_layers):
        np.testing.assert_allclose(a.K[l], b.K[l], rtol=1e-4, atol=1e-5)
        np.testing.assert_allclose(a.V[l], b.V[l], rtol=1e-4, atol=1e-5)
    ta, tb = lm.step(a, [1] * 8), lm.step(b, [1] * 8)
    np.testing.assert_allclose(ta["text_logits"], tb["text_logits"], rtol=1e-4, atol=1e-5)


def test_reset_state_repeats_the_first_frame():
    w = mini_weights()
    lm = O.OracleLM(MINI, w)
    st = lm.new_state()
    first = lm.step(st, [3] * 8)
    lm.step(st, [4] * 8)
    again = lm.step(lm.new_state(), [3] * 8)
    assert first["text_token"] == again["text_token"] and first["audio_tokens"] == again["audio_tokens"]
    np.testing.assert_array_equal(first["text_logits"], again["text_logits"])


# ------------------------------------------------------------------ bf16 widening

def test_bf16_widening_hand_values():
    """bfloat16 bits are the top half of the float32: 0x3F80 is 1.0, 0xC020 is -2.5 and the
    smallest subnormal 0x0001 is 2^-133."""
    got = O.bf16_to_f32(np.array([0x3F80, 0xC020, 0x0001, 0x0000, 0x8000, 0x7F80], np.uint16))
    assert got[0] == 1.0 and got[1] == -2.5 and got[2] == 2.0 ** -133
    assert got[3] == 0.0 and np.signbit(got[4]) and got[5] == np.inf


# ------------------------------------------------------------------ per-step depformer weights

def test_depformer_steps_use_their_own_weights_and_cache_entries():
    """Every step cb has its own projections ([LM] depformer_cycle reads in_projs[cb] etc.), and a
    cached entry keeps the value its own step computed.  With q and k rows zero (uniform
    attention), v rows = d[j][s] * I, out_proj = c[j][s] * I and the FFN zero, layer j gives
    y_cb += c[j][cb] * mean_{p <= cb} d[j][p] * rms_norm(y_p; norm1_j), and linears[cb] = [I; 0]
    exposes y in the logits.  Using step 0's (or layer j's) weights for every step, or recomputing
    the cached values with the current step's weights, changes the logits."""
    cfg = MINI.with_(dep_layers=2)
    Dd, Q = cfg.dep_d_model, cfg.dep_q
    w = mini_weights(cfg)
    c = lambda j, s: 0.3 + 0.1 * s + 0.05 * j  # noqa: E731
    dv = lambda j, s: 1.0 + 0.2 * s - 0.1 * j  # noqa: E731
    alpha = [np.abs(synth.normal(8, f"pin/dn{j}", (Dd,), 1.0)) + F32(0.5) for j in range(2)]
    for j in range(2):
        p = f"depformer.layers.{j}"
        w[f"{p}.norm1.alpha"][:] = alpha[j]
        for s in range(Q):
            Win = np.zeros((3 * Dd, Dd), F32)
            Win[2 * Dd:] = F32(dv(j, s)) * np.eye(Dd, dtype=F32)
            w[f"{p}.self_attn.in_projs.{s}.weight"][:] = Win
            w[f"{p}.self_attn.out_projs.{s}.weight"][:] = F32(c(j, s)) * np.eye(Dd, dtype=F32)
            w[f"{p}.gating.{s}.linear_out.weight"][:] = 0
    for s in range(Q):
        lin = np.zeros((cfg.audio_card, Dd), F32)
        lin[:Dd] = np.eye(Dd, dtype=F32)
        w[f"linears.{s}.weight"][:] = lin
    lm = O.OracleLM(cfg, w)
    st = lm.new_state()
    rms = lambda y, a: y * a / np.sqrt(1e-8 + np.mean(y * y))  # noqa: E731
    for t in range(2):
        tr = lm.step(st, [t + 3] * 8)
        hid = tr["transformer_out"].astype(np.float64)
        prev = tr["text_token"]
        cache = [[], []]
        for cb in range(Q):
            table = w["depformer_text_emb.weight"] if cb == 0 else w[f"depformer_emb.{cb - 1}.weight"]
            y = w[f"depformer_in.{cb}.weight"].astype(np.float64) @ hid + table[prev]
            for j in range(2):
                cache[j].append(dv(j, cb) * rms(y, alpha[j].astype(np.float64)))
                y = y + c(j, cb) * np.mean(cache[j], axis=0)
            np.testing.assert_allclose(tr["audio_logits"][cb][:Dd], y, rtol=1e-4, atol=1e-5)
            prev = tr["audio_tokens"][cb]


# ------------------------------------------------------------------ rope inside the temporal step

def test_temporal_step_ropes_q_and_k_at_the_absolute_position():
    """One temporal layer whose q and k read only dims 0..3 of a residual that keeps those dims
    (and its norm) fixed: the user's codebook-0 table writes a one-hot of the token into dims
    4..11, every other table adds the same vector a on dims 0..3, the text table a too.  Then the
    pre-rope q and k are the same at every position, and with interleaved rope the score of query
    t against key j is (sum_i cos(f_i (t - j)) (q_2i k_2i + q_2i+1 k_2i+1) + sin(f_i (t - j))
    (q_2i k_2i+1 - q_2i+1 k_2i)) / sqrt(hd), f_i = theta^(-2i/hd); v reads the one-hot dims, so
    the attention output is a closed-form mix of the earlier tokens' one-hots.  out_proj = I, the
    FFN is zero and text_linear = [I; 0] exposes out_norm(x + o).  Also the cached key of position
    j is the pre-rope k turned by f_i * j.  Skipping rope, roping v, or turning q and k by
    different positions changes these values.  (Turning both by pos + 1 leaves every score, and so
    every output, unchanged; the cached-key check catches it.)"""
    cfg = MINI.with_(n_layers=1, context=8, text_card=40, audio_card=32)
    D, H = cfg.d_model, cfg.n_heads
    hd = D // H
    w = mini_weights(cfg)
    for k in range(16):
        w[f"emb.{k}.weight"][:] = 0
    a = np.zeros(D, F32)
    a[:4] = [0.8, -0.5, 0.3, 0.6]
    w["text_emb.weight"][:] = a
    cu = F32(0.9)
    t8 = np.zeros((cfg.audio_card + 1, D), F32)
    for r in range(cfg.audio_card + 1):
        t8[r, 4 + r % 8] = cu
    w["emb.8.weight"][:] = t8  # stream 9: the user's codebook 0 (delay 0)
    p = "transformer.layers.0"
    Win = np.zeros((3 * D, D), F32)
    Win[:D, :4] = synth.normal(9, "pin/ropeq", (D, 4), 1.0)
    Win[D:2 * D, :4] = synth.normal(9, "pin/ropek", (D, 4), 1.0)
    for h in range(H):
        Win[2 * D + h * hd: 2 * D + (h + 1) * hd, 4:12] = np.eye(hd, dtype=F32)
    w[f"{p}.self_attn.in_projs.0.weight"][:] = Win
    w[f"{p}.self_attn.out_projs.0.weight"][:] = np.eye(D, dtype=F32)
    w[f"{p}.gating.linear_out.weight"][:] = 0
    tl = np.zeros((cfg.text_card, D), F32)
    tl[:D] = np.eye(D, dtype=F32)
    w["text_linear.weight"][:] = tl
    lm = O.OracleLM(cfg, w)
    st = lm.new_state()
    users = [[(5 * t + 3) % cfg.audio_card] + [1] * 7 for t in range(7)]
    f = 10000.0 ** (-2.0 * np.arange(hd // 2) / hd)

    def rot(v, ang):  # turn each interleaved pair of one head by ang[i]
        z = v[0::2] + 1j * v[1::2]
        z = z * np.exp(1j * ang)
        out = np.empty(hd)
        out[0::2], out[1::2] = z.real, z.imag
        return out

    onehots = []
    for t in range(7):
        tr = lm.step(st, users[t])
        x = tr["emb_sum"].astype(np.float64)
        inv = 1 / np.sqrt(1e-8 + np.mean(x * x))
        q0 = Win[:D].astype(np.float64) @ (x * inv)
        k0 = Win[D:2 * D].astype(np.float64) @ (x * inv)
        onehots.append(x[4:12] * inv)
        o = np.zeros(D)
        for h in range(H):
            sl = slice(h * hd, (h + 1) * hd)
            qh, kh = q0[sl], k0[sl]
            s = np.array([(rot(qh, f * (t - j)) @ kh) / np.sqrt(hd) for j in range(t + 1)])
            e = np.exp(s - s.max())
            o[sl] = (e / e.sum()) @ np.array(onehots)
            # cached key of every position j <= t: k0 turned by f_i * j
            for j in range(t + 1):
                np.testing.assert_allclose(st.K[0][j][sl], rot(kh, f * j), rtol=1e-4, atol=1e-5)
        x1 = x + o
        hid = x1 / np.sqrt(1e-8 + np.mean(x1 * x1))
        np.testing.assert_allclose(tr["text_logits"][:D], hid, rtol=1e-4, atol=1e-5)


# ------------------------------------------------------------------ bf16 KV storage option

def test_round_bf16_hand_values():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties to the even mantissa (1.0);
    # 1 + 3 * 2^-8 ties upward to 1 + 2^-6; just above a tie rounds up; signs are kept
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -(1 + 2 ** -8 + 2 ** -20), 3.0, 0.0], F32)
    np.testing.assert_array_equal(O.round_bf16(x), np.array([1.0, 1 + 2 ** -6, 1 + 2 ** -7, -(1 + 2 ** -7), 3.0, 0.0], F32))


def test_bf16_kv_option_stores_rounded_keys_and_values():
    """With kv='bf16' every cached key and value is the bfloat16 rounding of the float32 one (low
    16 bits zero), in the decode step and in the batched prefill; the default keeps float32."""
    cfg = MINI.with_(context=6)
    w = mini_weights(cfg)
    lm, lm16 = O.OracleLM(cfg, w), O.OracleLM(cfg, w, kv="bf16")
    a, b = lm.new_state(), lm16.new_state()
    text = synth.uniform_int(5, "pin/kvt", (4,), cfg.text_card)
    agent = synth.uniform_int(5, "pin/kva", (4, 8), cfg.audio_card)
    user = synth.uniform_int(5, "pin/kvu", (4, 8), cfg.audio_card)
    lm16.prefill_forced(b, text, agent, user)
    lm16.step(b, [2] * 8)
    lm.step(a, [2] * 8)
    for l in range(cfg.n_layers):
        for arr in (b.K[l], b.V[l]):
            assert not np.any(arr.view(np.uint32) & 0xFFFF)
    assert np.any(a.K[0].view(np.uint32) & 0xFFFF)
    # the first decode key of layer 0 is the rounded float32 key
    c = lm16.new_state()
    lm16.step(c, [2] * 8)
    np.testing.assert_array_equal(c.K[0][0], O.round_bf16(a.K[0][0]))
