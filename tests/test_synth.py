"""The seeded input generator: reproducible, chunk-invariant, distributed as stated."""
import numpy as np

import synth


def test_stream_is_reproducible_and_chunk_invariant():
    a = synth.normal(3, "t/x", (1001,), 0.02)
    b = synth.normal(3, "t/x", (1001,), 0.02)
    assert a.tobytes() == b.tobytes()
    c = synth.normal(3, "t/x", (100,), 0.02, start=401)
    assert np.array_equal(a[401:501], c)
    assert not np.array_equal(a, synth.normal(4, "t/x", (1001,), 0.02))
    assert not np.array_equal(a, synth.normal(3, "t/y", (1001,), 0.02))


def test_normal_moments_and_bf16_rounding():
    a = synth.normal(5, "t/m", (400000,), 0.02)
    assert abs(a.mean()) < 2e-4 and abs(a.std() - 0.02) < 2e-4
    b = synth.normal(5, "t/m", (400000,), 0.02, dtype="bf16")
    assert np.array_equal(b, synth.f32_to_bf16_bits(a))
    back = synth.bf16_bits_to_f32(b)
    assert np.all(np.abs(back - a) <= np.abs(a) * 2.0 ** -8)


def test_bf16_round_to_nearest_even_hand_values():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 65504.0], np.float32)
    bits = synth.f32_to_bf16_bits(x)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins; 1 + 3*2^-8 rounds up.
    assert bits.tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x4780]


def test_uniform_tokens_cover_the_range():
    t = synth.uniform_int(0, "t/u", (200000,), 2048)
    assert t.min() == 0 and t.max() == 2047
    h = np.bincount(t, minlength=2048)
    assert h.min() > 40 and h.max() < 160


def test_weight_specs_match_the_checkpoint_byte_count():
    specs = synth.weight_specs(synth.MOSHI7B)
    lin = sum(int(np.prod(s)) for _, s, k in specs if k == "linear")
    assert lin * 2 == 14_749_270_016
    names = [n for n, _, _ in specs]
    assert len(names) == len(set(names))
