"""Pins of the oracle's sampled modes, block quantisers and session snapshot (no GPU).

Page references are to the docs.rs source page inferencelayer 0.2.4 src/moshi_lm.rs ("[LM]"):
xorshift_u01, topk_sample, gumbel_full_pick, Sampling, MoshiLm::pick, qn_roundtrip,
q4_roundtrip, MoshiLm::load_q4sim and MoshiState::snapshot.
"""
import math

import numpy as np
import pytest

import synth
from oracle import moshi_oracle as O

F32 = np.float32


# ------------------------------------------------------------------ xorshift

def test_xorshift_first_outputs_by_hand():
    # x = 1: x ^= x << 13 -> 8193; x ^= x >> 7 -> 8257; x ^= x << 17 -> 8257 + 8257 * 2^17
    assert O.xorshift64(1) == 8257 + 8257 * (1 << 17) == 1082269761
    u, st = O.u01(1)
    assert st == 1082269761 and u == (1082269761 >> 11) / 2.0 ** 53
    # bits shifted out of the top are dropped (64-bit arithmetic)
    x = (1 << 63) | 1
    y = x ^ ((x << 13) & ((1 << 64) - 1))
    y ^= y >> 7
    y ^= (y << 17) & ((1 << 64) - 1)
    assert O.xorshift64(x) == y and y < (1 << 64)


def test_xorshift_is_the_linear_map_over_gf2():
    """The step is x -> (I + L^17)(I + R^7)(I + L^13) x over GF(2)^64: check it bit by bit as a
    matrix (columns = images of the unit vectors) applied to random states."""
    cols = [O.xorshift64(1 << j) for j in range(64)]
    rng = np.random.default_rng(3)
    for _ in range(20):
        x = int(rng.integers(1, 2 ** 63)) * 2 + 1
        y = 0
        for j in range(64):
            if (x >> j) & 1:
                y ^= cols[j]
        assert y == O.xorshift64(x)


def test_sampling_defaults_and_seed():
    s = O.Sampling(seed=0)
    assert (float(s.temp), float(s.temp_text), s.top_k, s.top_k_text, s.gumbel_full) == (
        pytest.approx(0.8), pytest.approx(0.7), 250, 25, False)
    assert s.state == 1  # [LM] set_sampling: seed.max(1)
    assert O.Sampling(seed=7).state == 7


# ------------------------------------------------------------------ top-k

def fixed_draws(*us):
    it = iter(us)
    return lambda: next(it)


def test_topk_hand_worked_three_logits():
    # logits [1, 2, 0], T = 1, k = 3: order 1, 0, 2 with p proportional to 1, e^-1, e^-2
    lg = np.array([1.0, 2.0, 0.0], F32)
    e = [1.0, math.exp(-1), math.exp(-2)]
    p = [v / sum(e) for v in e]  # 0.665, 0.245, 0.090
    assert O.topk_sample(lg, 1.0, 3, fixed_draws(0.5)) == 1
    assert O.topk_sample(lg, 1.0, 3, fixed_draws(p[0] + 0.01)) == 0
    assert O.topk_sample(lg, 1.0, 3, fixed_draws(p[0] + p[1] + 0.01)) == 2
    assert O.topk_sample(lg, 1.0, 3, fixed_draws(p[0] - 1e-9)) == 1
    # k = 2 drops index 2 and renormalises over {1, 0}
    q0 = 1.0 / (1.0 + math.exp(-1))
    assert O.topk_sample(lg, 1.0, 2, fixed_draws(q0 + 1e-6)) == 0
    assert O.topk_sample(lg, 1.0, 2, fixed_draws(0.999999)) == 0
    # temperature divides the logit gaps: T = 0.5 doubles them
    r0 = 1.0 / (1.0 + math.exp(-2))
    assert O.topk_sample(lg, 0.5, 2, fixed_draws(r0 - 1e-6)) == 1
    assert O.topk_sample(lg, 0.5, 2, fixed_draws(r0 + 1e-6)) == 0


def test_topk_reduces_to_argmax():
    lg = synth.normal(4, "pin/topk", (300,), 1.0)
    best = int(np.argmax(lg))
    for u in (0.0, 0.3, 0.999999):
        assert O.topk_sample(lg, 0.8, 1, fixed_draws(u)) == best  # k = 1
    assert O.topk_sample(lg, 1e-6, 250, fixed_draws(0.999)) == best  # T -> 0


def test_topk_ties_order_by_index():
    lg = np.array([0.0, 5.0, 5.0, 1.0, 5.0], F32)
    # k = 2 keeps indexes 1 and 2 (equal logits by increasing index), each p = 1/2
    assert O.topk_sample(lg, 1.0, 2, fixed_draws(0.49)) == 1
    assert O.topk_sample(lg, 1.0, 2, fixed_draws(0.51)) == 2


def test_topk_frequencies_follow_the_truncated_softmax():
    lg = np.array([0.3, 1.2, -0.5, 0.9, 2.0, -1.0], F32)
    s = O.Sampling(seed=12345)
    n = 20000
    cnt = np.bincount([O.topk_sample(lg, 0.8, 4, s.draw) for _ in range(n)], minlength=6)
    top = np.argsort(-lg.astype(np.float64), kind="stable")[:4]
    p = np.zeros(6)
    p[top] = np.exp((lg[top] - lg.max()) / 0.8)
    p /= p.sum()
    assert cnt[[i for i in range(6) if i not in top]].sum() == 0
    assert np.all(np.abs(cnt / n - p) < 4 * np.sqrt(p * (1 - p) / n) + 1e-9)


# ------------------------------------------------------------------ Gumbel-max

def test_gumbel_transform_by_hand():
    # g = -ln(-ln u): u = exp(-exp(-g)) gives g back, so scores l/T + g are known
    u_of = lambda g: math.exp(-math.exp(-g))  # noqa: E731
    lg = np.array([0.0, 0.0, 0.0], F32)
    assert O.gumbel_full_pick(lg, 1.0, fixed_draws(u_of(0.0), u_of(1.0), u_of(-1.0))) == 1
    assert O.gumbel_full_pick(lg, 1.0, fixed_draws(u_of(2.0), u_of(1.0), u_of(-1.0))) == 0
    # the noise adds to l / T: l = [0, 3] at T = 0.5 is [0, 6]; noise +5 / -0.5 leaves index 1
    lg2 = np.array([0.0, 3.0], F32)
    assert O.gumbel_full_pick(lg2, 0.5, fixed_draws(u_of(5.0), u_of(-0.5))) == 1
    assert O.gumbel_full_pick(lg2, 1.0, fixed_draws(u_of(5.0), u_of(-0.5))) == 0
    # u = 0 is clamped to 1e-300 (finite noise); ties keep the first index
    assert O.gumbel_full_pick(np.array([1.0, 1.0], F32), 1.0, fixed_draws(u_of(0.5), u_of(0.5))) == 0


def test_gumbel_draws_one_uniform_per_logit_in_index_order():
    s1, s2 = O.Sampling(seed=99), O.Sampling(seed=99)
    O.gumbel_full_pick(np.zeros(37, F32), 0.7, s1.draw)
    for _ in range(37):
        s2.draw()
    assert s1.state == s2.state


def test_gumbel_frequencies_follow_the_softmax():
    lg = np.array([0.3, 1.2, -0.5, 0.9], F32)
    s = O.Sampling(seed=777)
    n = 20000
    cnt = np.bincount([O.gumbel_full_pick(lg, 0.8, s.draw) for _ in range(n)], minlength=4)
    p = np.exp(lg.astype(np.float64) / 0.8)
    p /= p.sum()
    assert np.all(np.abs(cnt / n - p) < 4 * np.sqrt(p * (1 - p) / n))


def test_pick_routes_text_and_audio_settings():
    lg = synth.normal(5, "pin/pick", (64,), 1.0)
    assert O.pick(lg, True, None) == O.argmax_first(lg)
    a, b = O.Sampling(seed=5, top_k_text=1), O.Sampling(seed=5, top_k=1)
    assert O.pick(lg, True, a) == O.argmax_first(lg)  # text uses top_k_text
    assert O.pick(lg, False, b) == O.argmax_first(lg)  # audio uses top_k
    g1, g2 = O.Sampling(seed=5, gumbel_full=True, temp_text=0.3), O.Sampling(seed=5)
    assert O.pick(lg, True, g1) == O.gumbel_full_pick(lg, F32(0.3), g2.draw)


def test_sampled_frames_are_reproducible_and_advance_the_stream():
    cfg = synth.TINY.with_(n_layers=1, dep_layers=1, d_model=64, n_heads=1, ffn_hidden=64, dep_d_model=64,
                           dep_heads=1, dep_ffn_hidden=64, text_card=50, audio_card=40)
    w = synth.gen_weights(cfg, dtype="f32")
    lm = O.OracleLM(cfg, w)
    runs = []
    for _ in range(2):
        st, smp = lm.new_state(), O.Sampling(seed=42, top_k=10, top_k_text=5)
        runs.append([lm.step(st, [1] * 8, smp)["audio_tokens"] for _ in range(3)] + [smp.state])
    assert runs[0] == runs[1]
    # top-k draws one uniform per pick: 9 per frame
    s = O.Sampling(seed=42)
    for _ in range(27):
        s.draw()
    assert runs[0][-1] == s.state


# ------------------------------------------------------------------ block quantisers

def test_q4_block_hand_values():
    # one 32-column block: the largest magnitude is -3.2 (first on ties with +3.2 later), so
    # d = -3.2 / -8 = 0.4; codes round x / 0.4 half away from zero, clamped to [-8, 7]
    row = np.zeros(32, F32)
    row[:8] = [-3.2, 0.2, -0.2, 0.6, 1.0, 2.79, 3.2, 0.0]
    q, d = O.quantize_blocks(row[None], 4)
    assert d.shape == (1, 1) and d[0, 0] == F32(-3.2) / F32(-8)
    assert q[0, :8].tolist() == [-8, 1, -1, 2, 3, 7, 7, 0]  # 0.5 -> 1, 1.5 -> 2, 2.5 -> 3, 6.97 -> 7, +8 clamps
    deq = O.dequantize_blocks(q, d)
    assert deq[0, 0] == F32(-3.2) and abs(deq[0, 6] - 2.8) < 1e-6
    # a zero block keeps d = 0 and codes 0
    q0, d0 = O.quantize_blocks(np.zeros((2, 64), F32), 4)
    assert np.all(q0 == 0) and np.all(d0 == 0)


def test_q8_block_hand_values_and_error_bound():
    row = np.linspace(-1.0, 2.0, 32).astype(F32)
    q, d = O.quantize_blocks(row[None], 8)
    assert d[0, 0] == F32(F32(2.0) / F32(-128))
    assert q[0, -1] == -128 and q[0, 0] == 64
    W = synth.normal(6, "pin/q8", (16, 128), 0.02)
    for bits in (4, 8):
        q, d = O.quantize_blocks(W, bits)
        err = np.abs(O.dequantize_blocks(q, d) - W).reshape(16, 4, 32)
        lim = np.abs(d)[..., None]
        assert np.all(err <= lim + 1e-9)
        assert q.min() >= -(1 << (bits - 1)) and q.max() <= (1 << (bits - 1)) - 1


def test_q4_nibble_layout():
    # byte i of a block: element i in the low nibble, element i + 16 in the high, both + 8
    q = np.zeros((1, 64), np.int8)
    q[0, 0], q[0, 16], q[0, 15], q[0, 31], q[0, 32] = -8, 7, 3, -1, 5
    nib = O.pack_q4_0(q)
    assert nib.shape == (1, 32)
    assert nib[0, 0] == (0 | (15 << 4)) and nib[0, 15] == (11 | (7 << 4)) and nib[0, 16] == (13 | (8 << 4))
    assert nib[0, 1] == (8 | (8 << 4))
    full = np.random.default_rng(1).integers(-8, 8, (3, 96)).astype(np.int8)
    assert np.array_equal(O.unpack_q4_0(O.pack_q4_0(full), 96), full)


def test_block_bands_in_the_model():
    """The q4sim / q8sim oracles replace each linear by its block roundtrip, embeddings untouched."""
    cfg = synth.TINY
    w = synth.gen_weights(cfg)
    for band, bits in (("q4sim", 4), ("q8sim", 8)):
        lm = O.OracleLM(cfg, w, band=band)
        W = w["transformer.layers.1.gating.linear_out.weight"]
        assert np.array_equal(lm.layers[1]["w_gout"], O.dequantize_blocks(*O.quantize_blocks(W, bits)))
        assert np.array_equal(lm.emb[3], w["emb.3.weight"])
        assert np.array_equal(lm.dep_tables[0], w["depformer_text_emb.weight"])


# ------------------------------------------------------------------ snapshot

def test_snapshot_restores_a_primed_session():
    cfg = synth.TINY
    w = synth.gen_weights(cfg)
    lm = O.OracleLM(cfg, w)
    st = lm.new_state()
    text, agent, user = synth.prefill_tokens(cfg, 6)
    lm.prefill_forced(st, text, agent, user)
    users = synth.user_tokens(cfg, 5, start_frame=6)
    lm.step(st, users[0])
    snap = st.snapshot()
    a = [lm.step(st, users[f]) for f in range(1, 5)]
    assert snap.offset == 7 and st.offset == 11
    b = [lm.step(snap, users[f]) for f in range(1, 5)]
    for x, y in zip(a, b):
        assert x["text_token"] == y["text_token"] and x["audio_tokens"] == y["audio_tokens"] and x["out"] == y["out"]
        assert x["text_logits"].tobytes() == y["text_logits"].tobytes()
    assert np.array_equal(st.ring, snap.ring)
