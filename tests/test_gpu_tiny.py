"""GPU parity on the tiny float32 RQ-Transformer (2+2 layers, d256/d128, 17 streams, 16 frames):
tokens, ring and outputs bit-exact against the CPU oracle, logits within 1e-4 relative error,
plus the edge cases of the boundary (reset, -1 tokens, invalid tokens, capacity, eviction,
teacher forcing, prefill, batches)."""
import numpy as np
import pytest

import rq_transformer_frame_amd as rq
import synth
from oracle import OracleLM
from tests.gpu_util import cosine, frame_agreement, rel_err

pytestmark = pytest.mark.gpu

CFG = synth.TINY
TOL = 1e-4


@pytest.fixture(scope="module")
def weights():
    return synth.gen_weights(CFG)


@pytest.fixture(scope="module")
def oracle(weights):
    return OracleLM(CFG, weights)


def compare_step(tr, ref, st, out, has, frame):
    assert tr["input_tokens"].tolist() == ref["input_tokens"].tolist(), frame
    np.testing.assert_allclose(tr["emb_sum"], ref["emb_sum"], rtol=1e-6, atol=1e-7)
    assert rel_err(tr["transformer_out"], ref["transformer_out"]) <= TOL, frame
    assert rel_err(tr["text_logits"], ref["text_logits"]) <= TOL, frame
    for cb in range(CFG.dep_q):
        assert rel_err(tr["audio_logits"][cb], ref["audio_logits"][cb]) <= TOL, (frame, cb)
    assert tr["text_token"] == ref["text_token"], frame
    assert tr["audio_tokens"] == ref["audio_tokens"], frame
    assert bool(has[0]) == (ref["out"] is not None), frame
    assert st == (rq.MOSHI_NONE if ref["out"] is None else rq.MOSHI_OK)
    if ref["out"] is not None:
        assert out[0].tolist() == ref["out"], frame


@pytest.mark.parametrize("exec_mode", ["graph", "stream", "persistent"])
def test_tiny_free_running_matches_oracle(weights, oracle, exec_mode):
    users = synth.user_tokens(CFG, CFG.frames)
    ost = oracle.new_state()
    with rq.Session(CFG, exec=exec_mode) as s:
        s.load_weights(weights)
        for f in range(CFG.frames):
            ref = oracle.step(ost, users[f])
            st, out, has = s.step(users[f])
            compare_step(s.read_trace(0), ref, st, out, has, f)
            assert s.offset(0) == f + 1


@pytest.mark.parametrize("exec_mode", ["graph", "persistent"])
def test_tiny_sliding_window_past_context(weights, oracle, exec_mode):
    """74 frames with context 64: the KV ring wraps and attention keeps the last 64 positions."""
    users = synth.user_tokens(CFG, 74)
    ost = oracle.new_state()
    with rq.Session(CFG, exec=exec_mode) as s:
        s.load_weights(weights)
        for f in range(74):
            ref = oracle.step(ost, users[f])
            st, out, has = s.step(users[f])
            compare_step(s.read_trace(0), ref, st, out, has, f)


@pytest.mark.parametrize("exec_mode", ["graph", "persistent"])
def test_tiny_runs_are_bitwise_deterministic(weights, exec_mode):
    users = synth.user_tokens(CFG, 6)
    logs = []
    for _ in range(2):
        with rq.Session(CFG, exec=exec_mode) as s:
            s.load_weights(weights)
            for f in range(6):
                s.step(users[f])
            logs.append(s.read_trace(0))
    for k in ("text_logits", "audio_logits", "transformer_out"):
        assert logs[0][k].tobytes() == logs[1][k].tobytes(), k


def test_reset_mid_stream_repeats_frame_zero(weights, oracle):
    users = synth.user_tokens(CFG, 5)
    with rq.Session(CFG) as s:
        s.load_weights(weights)
        s.step(users[0])
        first = s.read_trace(0)
        for f in range(1, 5):
            s.step(users[f])
        s.reset(0)
        assert s.offset(0) == 0
        st, _, has = s.step(users[0])
        again = s.read_trace(0)
        assert st == rq.MOSHI_NONE and not has[0]
        assert again["text_logits"].tobytes() == first["text_logits"].tobytes()
        assert again["tokens"].tolist() == first["tokens"].tolist()


def test_minus_one_user_tokens_embed_to_zero(weights, oracle):
    users = synth.user_tokens(CFG, 4)
    users[1, 3] = -1
    users[2, :] = -1
    ost = oracle.new_state()
    with rq.Session(CFG) as s:
        s.load_weights(weights)
        for f in range(4):
            ref = oracle.step(ost, users[f])
            st, out, has = s.step(users[f])
            compare_step(s.read_trace(0), ref, st, out, has, f)


def test_invalid_user_token_leaves_state_unchanged(weights, oracle):
    users = synth.user_tokens(CFG, 3)
    ost = oracle.new_state()
    with rq.Session(CFG) as s:
        s.load_weights(weights)
        ref = oracle.step(ost, users[0])
        st, out, has = s.step(users[0])
        compare_step(s.read_trace(0), ref, st, out, has, 0)
        for bad in (2048, -2, 99999):
            u = users[1].copy()
            u[5] = bad
            with pytest.raises(rq.MoshiError) as ei:
                s.step(u)
            assert ei.value.status == rq.MOSHI_EINVAL
            assert s.offset(0) == 1
        ref = oracle.step(ost, users[1])
        st, out, has = s.step(users[1])
        compare_step(s.read_trace(0), ref, st, out, has, 1)


def test_step_before_weights_is_a_state_error(weights):
    with rq.Session(CFG) as s:
        with pytest.raises(rq.MoshiError) as ei:
            s.step(np.zeros(8, np.int32))
        assert ei.value.status == rq.MOSHI_ESTATE
        part = {k: v for k, v in list(weights.items())[:10]}
        s.load_weights(part)
        with pytest.raises(rq.MoshiError) as ei:
            s.step(np.zeros(8, np.int32))
        assert ei.value.status == rq.MOSHI_ESTATE


def test_load_rejects_unknown_names_and_bad_shapes(weights):
    with rq.Session(CFG) as s:
        with pytest.raises(rq.MoshiError) as ei:
            s.load_weights({"no.such.weight": np.zeros((2, 2), np.float32)})
        assert ei.value.status == rq.MOSHI_ESHAPE
        with pytest.raises(rq.MoshiError) as ei:
            s.load_weights({"text_linear.weight": np.zeros((999, 256), np.float32)})
        assert ei.value.status == rq.MOSHI_ESHAPE


def test_kv_capacity_below_context_refuses_to_overflow(weights, oracle):
    users = synth.user_tokens(CFG, 5)
    ost = oracle.new_state()
    with rq.Session(CFG, kv_capacity=4) as s:
        s.load_weights(weights)
        for f in range(4):
            ref = oracle.step(ost, users[f])
            st, out, has = s.step(users[f])
            compare_step(s.read_trace(0), ref, st, out, has, f)
        with pytest.raises(rq.MoshiError) as ei:
            s.step(users[4])
        assert ei.value.status == rq.MOSHI_ERANGE
        assert s.offset(0) == 4


def test_teacher_forcing_follows_the_reference_trajectory(weights, oracle):
    """[LM] force_generated: after each step the generated slot is overwritten with reference
    tokens, so each step is judged on the reference trajectory."""
    users = synth.user_tokens(CFG, 8)
    forced = synth.uniform_int(9, "t/force", (8, 9), CFG.audio_card)
    forced[:, 0] %= CFG.text_card
    ost = oracle.new_state()
    with rq.Session(CFG) as s:
        s.load_weights(weights)
        for f in range(8):
            ref = oracle.step(ost, users[f])
            st, out, has = s.step(users[f])
            compare_step(s.read_trace(0), ref, st, out, has, f)
            oracle.force_generated(ost, int(forced[f, 0]), forced[f, 1:])
            s.force_generated(0, int(forced[f, 0]), forced[f, 1:])


def test_persistent_executor_needs_batch_one(weights):
    with pytest.raises(rq.MoshiError) as ei:
        rq.Session(CFG, batch=2, exec="persistent")
    assert ei.value.status == rq.MOSHI_EINVAL


def test_persistent_and_graph_executors_agree(weights):
    """Both executors run the same per-row arithmetic: the logits agree to float32 rounding and
    the tokens exactly over a free-running trace."""
    users = synth.user_tokens(CFG, 10)
    traces = {}
    for mode in ("graph", "persistent"):
        with rq.Session(CFG, exec=mode) as s:
            s.load_weights(weights)
            traces[mode] = []
            for f in range(10):
                s.step(users[f])
                traces[mode].append(s.read_trace(0))
    for f in range(10):
        g, p = traces["graph"][f], traces["persistent"][f]
        assert g["tokens"].tolist() == p["tokens"].tolist(), f
        assert rel_err(p["text_logits"], g["text_logits"]) <= 1e-5, f


@pytest.mark.parametrize("T", [1, 5, 70])
@pytest.mark.parametrize("exec_mode", ["graph", "persistent"])
def test_prefill_forced_then_greedy(weights, oracle, T, exec_mode):
    text, agent, user = synth.prefill_tokens(CFG, T)
    text %= CFG.text_card
    ost = oracle.new_state()
    oracle.prefill_forced(ost, text, agent, user)
    users = synth.user_tokens(CFG, 3, start_frame=T)
    with rq.Session(CFG, exec=exec_mode) as s:
        s.load_weights(weights)
        s.prefill_forced(0, text, agent, user)
        assert s.offset(0) == T
        for f in range(3):
            ref = oracle.step(ost, users[f])
            st, out, has = s.step(users[f])
            compare_step(s.read_trace(0), ref, st, out, has, T + f)


def test_batch_of_three_conversations_matches_single_runs(weights, oracle):
    B = 3
    users = np.stack([synth.user_tokens(CFG, 6, conv=b) for b in range(B)], axis=1)  # [f][b][8]
    refs = []
    for b in range(B):
        ost = oracle.new_state()
        refs.append([oracle.step(ost, users[f, b]) for f in range(6)])
    with rq.Session(CFG, batch=B) as s:
        s.load_weights(weights)
        for f in range(6):
            st, out, has = s.step(users[f])
            for b in range(B):
                tr = s.read_trace(b)
                ref = refs[b][f]
                assert tr["tokens"].tolist() == [ref["text_token"]] + ref["audio_tokens"], (f, b)
                assert rel_err(tr["text_logits"], ref["text_logits"]) <= TOL
                assert bool(has[b]) == (ref["out"] is not None)
                if ref["out"] is not None:
                    assert out[b].tolist() == ref["out"]
        s.reset(1)
        assert [s.offset(b) for b in range(B)] == [6, 0, 6]


def test_batch_of_256_after_prefixes_matches_oracle(weights, oracle):
    """256 conversations with prefixes of 0..61 positions, then 6 greedy frames (some caches pass
    the 64-position window).  With 4 heads and 256 rows the attention takes one block per (head,
    conversation) on a 256-CU part: the single-pass online-softmax kernel.  Tokens equal the
    oracle's; logits within TOL."""
    B, F = 256, 6
    starts = synth.uniform_int(11, "b256/start", (B,), 62).astype(int)
    pre = [synth.prefill_tokens(CFG, int(starts[b]), conv=b) for b in range(B)]
    users = np.stack([synth.user_tokens(CFG, F, conv=b, start_frame=int(starts[b])) for b in range(B)], axis=1)
    refs = []
    for b in range(B):
        ost = oracle.new_state()
        if starts[b]:
            oracle.prefill_forced(ost, *pre[b])
        refs.append([oracle.step(ost, users[f, b]) for f in range(F)])
    with rq.Session(CFG, batch=B) as s:
        s.load_weights(weights)
        for b in range(B):
            if starts[b]:
                s.prefill_forced(b, *pre[b])
        for f in range(F):
            st, out, has = s.step(users[f])
            for b in range(B):
                tr = s.read_trace(b)
                ref = refs[b][f]
                assert tr["tokens"].tolist() == [ref["text_token"]] + ref["audio_tokens"], (f, b, int(starts[b]))
                assert rel_err(tr["text_logits"], ref["text_logits"]) <= TOL, (f, b)


SIM = {"bf16": "f32", "i8": "i8sim", "q4": "q4sim", "q8": "q8sim"}


@pytest.mark.parametrize("exec_mode", ["graph", "persistent"])
@pytest.mark.parametrize("band", ["bf16", "i8", "q4", "q8"])
def test_low_precision_bands_on_the_tiny_model(weights, band, exec_mode):
    """bf16 band vs the oracle on the same bf16-rounded weights; int8, Q4_0 and q8_0 bands vs the
    oracle on the same quantise-dequantise round trip (storage loss only, [LM] load_q4sim).
    Teacher-forced onto the oracle's tokens."""
    w16 = {k: (synth.f32_to_bf16_bits(v) if v.ndim == 2 else v) for k, v in weights.items()}
    ref_lm = OracleLM(CFG, w16, band=SIM[band])
    users = synth.user_tokens(CFG, 8)
    ost = ref_lm.new_state()
    agree, total, cos_min = 0, 0, 1.0
    with rq.Session(CFG, band=band, exec=exec_mode) as s:
        s.load_weights(w16)
        for f in range(8):
            ref = ref_lm.step(ost, users[f])
            s.step(users[f])
            c, a = frame_agreement(s.read_trace(0), ref)
            cos_min, agree, total = min(cos_min, c), agree + a, total + 9
            ref_lm.force_generated(ost, ref["text_token"], ref["audio_tokens"])
            s.force_generated(0, ref["text_token"], ref["audio_tokens"])
    print(f"{band}: min cosine {cos_min:.6f}, agreement {agree}/{total}")
    assert cos_min >= 0.999
    assert agree / total >= 0.99


@pytest.mark.parametrize("band", ["bf16", "i8"])
def test_batched_low_precision_bands_match_oracle(weights, band):
    """Three conversations on the matrix-core path in the bf16 and int8 bands, each teacher-forced
    onto its own oracle run (bf16-rounded weights; the int8 band against the int8-dequantised
    oracle).  The batched path also rounds its projection inputs to bf16."""
    B = 3
    w16 = {k: (synth.f32_to_bf16_bits(v) if v.ndim == 2 else v) for k, v in weights.items()}
    ref_lm = OracleLM(CFG, w16, band="i8sim" if band == "i8" else "f32")
    users = np.stack([synth.user_tokens(CFG, 8, conv=b) for b in range(B)], axis=1)
    osts = [ref_lm.new_state() for _ in range(B)]
    agree, total, cos_min = 0, 0, 1.0
    with rq.Session(CFG, band=band, batch=B) as s:
        s.load_weights(w16)
        for f in range(8):
            s.step(users[f])
            for b in range(B):
                ref = ref_lm.step(osts[b], users[f, b])
                c, a = frame_agreement(s.read_trace(b), ref)
                cos_min, agree, total = min(cos_min, c), agree + a, total + 9
                ref_lm.force_generated(osts[b], ref["text_token"], ref["audio_tokens"])
                s.force_generated(b, ref["text_token"], ref["audio_tokens"])
    print(f"batched {band}: min cosine {cos_min:.6f}, agreement {agree}/{total}")
    assert cos_min >= 0.999
    assert agree / total >= 0.99


def test_prefill_row_batches_then_single_frames(weights, oracle):
    """A prefill long enough to run row batches up to the context limit and then single frames
    past it (window slide), against the oracle."""
    T = 67
    text, agent, user = synth.prefill_tokens(CFG, T, conv=1)
    text %= CFG.text_card
    ost = oracle.new_state()
    oracle.prefill_forced(ost, text, agent, user)
    users = synth.user_tokens(CFG, 4, conv=1, start_frame=T)
    with rq.Session(CFG) as s:
        s.load_weights(weights)
        s.prefill_forced(0, text[:30], agent[:30], user[:30])
        s.prefill_forced(0, text[30:], agent[30:], user[30:])
        assert s.offset(0) == T
        for f in range(4):
            ref = oracle.step(ost, users[f])
            st, out, has = s.step(users[f])
            compare_step(s.read_trace(0), ref, st, out, has, T + f)


@pytest.mark.parametrize("batch", [1, 3, 256])
def test_bf16_kv_cache_on_the_tiny_model(weights, batch):
    """The opt-in bfloat16 KV cache (bf16 band), single-conversation and batched paths, against the
    oracle on the same bf16-rounded weights (the KV storage loss stays within the bar at this
    context length).  With 256 conversations the attention takes one block per (head,
    conversation): the single-pass kernel on the bfloat16 cache."""
    w16 = {k: (synth.f32_to_bf16_bits(v) if v.ndim == 2 else v) for k, v in weights.items()}
    ref_lm = OracleLM(CFG, w16)
    users = np.stack([synth.user_tokens(CFG, 8, conv=b) for b in range(batch)], axis=1)
    osts = [ref_lm.new_state() for _ in range(batch)]
    agree, total, cos_min = 0, 0, 1.0
    with rq.Session(CFG, band="bf16", batch=batch, kv="bf16") as s:
        s.load_weights(w16)
        for f in range(8):
            s.step(users[f])
            for b in range(batch):
                ref = ref_lm.step(osts[b], users[f, b])
                c, a = frame_agreement(s.read_trace(b), ref)
                cos_min, agree, total = min(cos_min, c), agree + a, total + 9
                ref_lm.force_generated(osts[b], ref["text_token"], ref["audio_tokens"])
                s.force_generated(b, ref["text_token"], ref["audio_tokens"])
    print(f"bf16 KV batch {batch}: min cosine {cos_min:.6f}, agreement {agree}/{total}")
    assert cos_min >= 0.999
    assert agree / total >= 0.99



@pytest.mark.parametrize("exec_mode", ["graph", "persistent"])
def test_long_prefill_many_attention_splits_matches_oracle(exec_mode):
    """16 heads and 1400 cached positions: the temporal attention runs in many position splits
    per head, more than the persistent grid has blocks per head (256 blocks / 16 heads, so the
    split count is capped at 16), and the splits are merged by their running max and sum.
    Float32, against the oracle."""
    cfg = CFG.with_(name="tiny_f32_h16_long", d_model=1024, n_heads=16, context=1536)
    T = 1400
    w = synth.gen_weights(cfg)
    lm = OracleLM(cfg, w)
    text, agent, user = synth.prefill_tokens(cfg, T, conv=2)
    text %= cfg.text_card
    ost = lm.new_state()
    lm.prefill_forced(ost, text, agent, user)
    users = synth.user_tokens(cfg, 3, conv=2, start_frame=T)
    with rq.Session(cfg, exec=exec_mode) as s:
        s.load_weights(w)
        s.prefill_forced(0, text, agent, user)
        for f in range(3):
            ref = lm.step(ost, users[f])
            st, out, has = s.step(users[f])
            tr = s.read_trace(0)
            assert tr["input_tokens"].tolist() == ref["input_tokens"].tolist(), f
            assert rel_err(tr["transformer_out"], ref["transformer_out"]) <= TOL, f
            assert rel_err(tr["text_logits"], ref["text_logits"]) <= TOL, f
            for cb in range(cfg.dep_q):
                assert rel_err(tr["audio_logits"][cb], ref["audio_logits"][cb]) <= TOL, (f, cb)
            assert tr["tokens"].tolist() == [ref["text_token"]] + ref["audio_tokens"], f


def test_long_prefill_bf16_head_dim_128_matches_oracle():
    """The bf16 band with 128-dim heads (the 7B head shape): the prefill's causal attention on the
    matrix cores and its projections on the 128 x 256 tiles over a full 1024-position chunk and a
    ragged one of 76, then 3 frames (graph executor: the prefill is the same row-batched path on
    every executor, and no persistent instance serves this shape).  Against the oracle holding the
    same bf16 weights."""
    exec_mode = "graph"
    cfg = CFG.with_(name="tiny_bf16_h8_long", d_model=1024, n_heads=8, context=1536, band="bf16", dtype="bf16")
    T = 1100
    w = synth.gen_weights(cfg)
    lm = OracleLM(cfg, w)
    text, agent, user = synth.prefill_tokens(cfg, T, conv=4)
    text %= cfg.text_card
    ost = lm.new_state()
    lm.prefill_forced(ost, text, agent, user)
    users = synth.user_tokens(cfg, 3, conv=4, start_frame=T)
    with rq.Session(cfg, exec=exec_mode) as s:
        s.load_weights(w)
        s.prefill_forced(0, text, agent, user)
        for f in range(3):
            ref = lm.step(ost, users[f])
            s.step(users[f])
            tr = s.read_trace(0)
            assert tr["input_tokens"].tolist() == ref["input_tokens"].tolist(), f
            assert rel_err(tr["transformer_out"], ref["transformer_out"]) <= TOL, f
            assert rel_err(tr["text_logits"], ref["text_logits"]) <= TOL, f
            for cb in range(cfg.dep_q):
                assert rel_err(tr["audio_logits"][cb], ref["audio_logits"][cb]) <= TOL, (f, cb)
            assert tr["tokens"].tolist() == [ref["text_token"]] + ref["audio_tokens"], f


def test_long_prefill_int8_band_matches_dequantised_oracle():
    """The int8 band's prefill on the 128 x 256 tiles (int8 weights widened in registers), with the
    gated unit's silu(gate) * mult formed in the first product's epilogue: a full 1024-position
    chunk and a ragged one of 76, then 3 frames, against the oracle on the same int8
    quantise-dequantise round trip of the bf16-rounded weights ([LM] load_q4sim's storage-loss
    reading, int8 per-row scales)."""
    cfg = CFG.with_(name="tiny_i8_h8_long", d_model=1024, n_heads=8, context=1536)
    T = 1100
    w = synth.gen_weights(cfg)
    w16 = {k: (synth.f32_to_bf16_bits(v) if v.ndim == 2 else v) for k, v in w.items()}
    lm = OracleLM(cfg, w16, band="i8sim")
    text, agent, user = synth.prefill_tokens(cfg, T, conv=5)
    text %= cfg.text_card
    ost = lm.new_state()
    lm.prefill_forced(ost, text, agent, user)
    users = synth.user_tokens(cfg, 3, conv=5, start_frame=T)
    with rq.Session(cfg, band="i8", exec="graph") as s:
        s.load_weights(w16)
        s.prefill_forced(0, text, agent, user)
        for f in range(3):
            ref = lm.step(ost, users[f])
            s.step(users[f])
            tr = s.read_trace(0)
            assert tr["input_tokens"].tolist() == ref["input_tokens"].tolist(), f
            assert rel_err(tr["transformer_out"], ref["transformer_out"]) <= TOL, f
            assert rel_err(tr["text_logits"], ref["text_logits"]) <= TOL, f
            for cb in range(cfg.dep_q):
                assert rel_err(tr["audio_logits"][cb], ref["audio_logits"][cb]) <= TOL, (f, cb)
            assert tr["tokens"].tolist() == [ref["text_token"]] + ref["audio_tokens"], f


def test_persistent_wait_timeout_exits_and_reset_recovers(weights, oracle):
    """A wait of the persistent frame kernel that gives up (forced from the host: zero polls
    allowed) raises the error flag, every block leaves the kernel, and the step returns
    MOSHI_EDEVICE.  After a reset the frames match the oracle from offset 0 again: nothing the
    aborted frame left in the phase flags or the depformer's tagged exchange values is taken for
    a later frame's."""
    users = synth.user_tokens(CFG, 6)
    with rq.Session(CFG, exec="persistent") as s:
        s.load_weights(weights)
        s.step(users[0])  # a completed frame first: the exchange buffers hold its tagged values
        s.set_spin_limit(0)
        with pytest.raises(rq.MoshiError) as ei:
            s.step(users[1])
        assert ei.value.status == rq.MOSHI_EDEVICE
        s.set_spin_limit(1 << 20)
        s.reset()
        ost = oracle.new_state()
        for f in range(6):
            ref = oracle.step(ost, users[f])
            st, out, has = s.step(users[f])
            compare_step(s.read_trace(0), ref, st, out, has, f)
    with rq.Session(CFG, exec="graph") as g:
        with pytest.raises(rq.MoshiError) as ei:
            g.set_spin_limit(10)
        assert ei.value.status == rq.MOSHI_ESTATE


def test_persistent_timeout_with_attention_splits_then_reset_recovers():
    """The timed-out frame of the test above, at a position where the temporal attention runs in
    several position splits per head (16 heads, 200 cached positions): blocks that got past the
    q|k|v wait raise their head's split counter before the next wait gives up.  After a reset and
    a fresh prefill the frames must match the oracle, so the abandoned frame's counters must not
    survive the reset."""
    cfg = CFG.with_(name="tiny_f32_h16_long", d_model=1024, n_heads=16, context=1536)
    T = 200
    w = synth.gen_weights(cfg)
    lm = OracleLM(cfg, w)
    text, agent, user = synth.prefill_tokens(cfg, T, conv=3)
    text %= cfg.text_card
    users = synth.user_tokens(cfg, 4, conv=3, start_frame=T)
    with rq.Session(cfg, exec="persistent") as s:
        s.load_weights(w)
        s.prefill_forced(0, text, agent, user)
        s.step(users[0])
        s.set_spin_limit(0)
        with pytest.raises(rq.MoshiError) as ei:
            s.step(users[1])
        assert ei.value.status == rq.MOSHI_EDEVICE
        s.set_spin_limit(1 << 20)
        s.reset()
        s.prefill_forced(0, text, agent, user)
        ost = lm.new_state()
        lm.prefill_forced(ost, text, agent, user)
        for f in range(3):
            ref = lm.step(ost, users[f])
            s.step(users[f])
            tr = s.read_trace(0)
            assert rel_err(tr["transformer_out"], ref["transformer_out"]) <= TOL, f
            assert rel_err(tr["text_logits"], ref["text_logits"]) <= TOL, f
            assert tr["tokens"].tolist() == [ref["text_token"]] + ref["audio_tokens"], f


def _contract_weights(weights, oracle):
    """Text head: row 0 NaN, rows 17 and 990 both 4 x the oracle's frame-0 hidden (a tie far above
    every other logit at frame 0), the rest as generated.  Codebook heads: row 0 NaN, rows 700 and
    1900 one shared random vector, every other row zero, so the logits are NaN, 0 ... 0 and a tie
    of two equal values: the token is 700 when that value is positive, else 1 (the first zero)."""
    w = {k: v.copy() for k, v in weights.items()}
    hid0 = oracle.step(oracle.new_state(), synth.user_tokens(CFG, 1)[0])["transformer_out"]
    tl = w["text_linear.weight"]
    tl[0] = np.nan
    tl[17] = tl[990] = 4.0 * hid0
    v = synth.normal(5, "contract/v", (CFG.dep_d_model,), 1.0)
    for cb in range(CFG.dep_q):
        lin = np.zeros((CFG.audio_card, CFG.dep_d_model), np.float32)
        lin[0] = np.nan
        lin[700] = lin[1900] = v
        w[f"linears.{cb}.weight"] = lin
    return w


@pytest.mark.parametrize("exec_mode,batch", [("graph", 1), ("stream", 1), ("persistent", 1), ("graph", 3)])
def test_greedy_contract_ties_first_wins_and_nan_never_chosen(weights, oracle, exec_mode, batch):
    """[LM] argmax (a strict '>' scan from -inf): among equal maxima the first index wins and NaN
    is never chosen.  Checked on the single-conversation heads (graph, stream, persistent) and on
    the batched frame's row argmax, against the oracle and the closed-form expectation."""
    w = _contract_weights(weights, oracle)
    lm = OracleLM(CFG, w)
    frames = 5
    users = [synth.user_tokens(CFG, frames, conv=b) for b in range(batch)]
    refs = []
    for b in range(batch):
        st = lm.new_state()
        refs.append([lm.step(st, users[b][f]) for f in range(frames)])
    assert refs[0][0]["text_token"] == 17
    for r in (x for run in refs for x in run):
        assert all(t in (700, 1) for t in r["audio_tokens"])
    seen = {t for run in refs for x in run for t in x["audio_tokens"]}
    print(f"audio tokens seen: {sorted(seen)}")
    with rq.Session(CFG, exec=exec_mode, batch=batch) as s:
        s.load_weights(w)
        for f in range(frames):
            s.step(np.stack([users[b][f] for b in range(batch)]))
            for b in range(batch):
                tr = s.read_trace(b)
                ref = refs[b][f]
                assert tr["tokens"].tolist() == [ref["text_token"]] + ref["audio_tokens"], (b, f)
                ok = np.isfinite(ref["text_logits"])
                assert rel_err(tr["text_logits"][ok], ref["text_logits"][ok]) <= TOL
                assert np.isnan(tr["text_logits"][0]) and np.isnan(tr["audio_logits"][:, 0]).all()


@pytest.mark.parametrize("exec_mode,batch", [("graph", 1), ("persistent", 1), ("graph", 3)])
def test_greedy_contract_all_equal_logits_pick_index_zero(weights, oracle, exec_mode, batch):
    """Every head zero: all logits are exactly 0 and every token is 0 (the first index)."""
    w = {k: v.copy() for k, v in weights.items()}
    w["text_linear.weight"][:] = 0
    for cb in range(CFG.dep_q):
        w[f"linears.{cb}.weight"][:] = 0
    users = synth.user_tokens(CFG, 3)
    with rq.Session(CFG, exec=exec_mode, batch=batch) as s:
        s.load_weights(w)
        for f in range(3):
            s.step(np.stack([users[f]] * batch))
            for b in range(batch):
                tr = s.read_trace(b)
                assert tr["tokens"].tolist() == [0] * (1 + CFG.dep_q), (b, f)
                assert not tr["text_logits"].any() and not tr["audio_logits"].any()


@pytest.mark.parametrize("band", ["q4", "q8"])
def test_block_bands_free_running_and_prefill(weights, band):
    """Q4_0 and q8_0 on the stream executor, free-running against the round-trip oracle with a
    prefill first (the block bands prefill one frame at a time): logits within 1e-4, tokens and
    outputs exact.  The weights are given as bf16, since these bands keep the embedding tables in
    bf16."""
    weights = {k: (synth.f32_to_bf16_bits(v) if v.ndim == 2 else v) for k, v in weights.items()}
    lm = OracleLM(CFG, weights, band=SIM[band])
    T = 5
    text, agent, user = synth.prefill_tokens(CFG, T, conv=6)
    text %= CFG.text_card
    users = synth.user_tokens(CFG, 6, conv=6, start_frame=T)
    ost = lm.new_state()
    lm.prefill_forced(ost, text, agent, user)
    with rq.Session(CFG, band=band, exec="stream") as s:
        s.load_weights(weights)
        s.prefill_forced(0, text, agent, user)
        for f in range(6):
            ref = lm.step(ost, users[f])
            st, out, has = s.step(users[f])
            tr = s.read_trace(0)
            assert rel_err(tr["text_logits"], ref["text_logits"]) <= TOL, f
            for cb in range(CFG.dep_q):
                assert rel_err(tr["audio_logits"][cb], ref["audio_logits"][cb]) <= TOL, (f, cb)
            assert tr["tokens"].tolist() == [ref["text_token"]] + ref["audio_tokens"], f
            assert out[0].tolist() == ref["out"], f


def test_block_bands_refuse_batches(weights):
    for band in ("q4", "q8"):
        with pytest.raises(rq.MoshiError) as ei:
            rq.Session(CFG, band=band, batch=2)
        assert ei.value.status == rq.MOSHI_EINVAL
