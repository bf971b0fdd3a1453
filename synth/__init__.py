"""Seeded synthetic inputs for the Moshi RQ-Transformer frame step.

This module is shared by the oracle tests, the GPU tests, ``smoke()`` and ``bench.py``.  It holds
none of the frame step's arithmetic: it knows the workload shapes, the checkpoint tensor names and
shapes, and how to draw reproducible numbers (see ``rqgen.c`` for the generator's definition).

Tensor names and shapes follow the checkpoint layout that the inferencelayer 0.2.4
``src/moshi_lm.rs`` page loads in ``MoshiLm::load_band`` (embedding tables with one extra row for
the INITIAL token, fused ``in_projs`` q|k|v, ``gating.linear_in`` packing [gate | mult]).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "_rqgen.so")
_SRC_PATH = os.path.join(_HERE, "rqgen.c")


def build_generator(force: bool = False) -> str:
    """Compile rqgen.c into _rqgen.so with gcc (OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC_PATH, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _gen():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build_generator())
        u64, i64, dbl = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double
        vp = ctypes.c_void_p
        lib.rqgen_key.restype = u64
        lib.rqgen_key.argtypes = [u64, ctypes.c_char_p]
        lib.rqgen_normal_f32.argtypes = [u64, u64, i64, dbl, vp]
        lib.rqgen_normal_bf16.argtypes = [u64, u64, i64, dbl, vp]
        lib.rqgen_uniform_int.argtypes = [u64, u64, i64, i64, vp]
        lib.rqgen_uniform_f64.argtypes = [u64, u64, i64, vp]
        lib.rqgen_f32_to_bf16.argtypes = [vp, i64, vp]
        _lib = lib
    return _lib


def stream_key(seed: int, name: str) -> int:
    return int(_gen().rqgen_key(seed & 0xFFFFFFFFFFFFFFFF, name.encode()))


def normal(seed: int, name: str, shape, std: float = 1.0, dtype: str = "f32", start: int = 0) -> np.ndarray:
    """N(0, std^2) values of stream `name`; dtype 'f32' (float32) or 'bf16' (uint16 raw bits, RNE)."""
    n = int(np.prod(shape))
    key = stream_key(seed, name)
    if dtype == "f32":
        out = np.empty(shape, np.float32)
        _gen().rqgen_normal_f32(key, start, n, std, out.ctypes.data)
    elif dtype == "bf16":
        out = np.empty(shape, np.uint16)
        _gen().rqgen_normal_bf16(key, start, n, std, out.ctypes.data)
    else:
        raise ValueError(dtype)
    return out


def uniform_int(seed: int, name: str, shape, card: int, start: int = 0) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(shape, np.int32)
    _gen().rqgen_uniform_int(stream_key(seed, name), start, n, card, out.ctypes.data)
    return out


def uniform_f64(seed: int, name: str, n: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, np.float64)
    _gen().rqgen_uniform_f64(stream_key(seed, name), start, n, out.ctypes.data)
    return out


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """bfloat16 round-to-nearest-even of float32 data, returned as uint16 raw bits."""
    a = np.ascontiguousarray(a, np.float32)
    out = np.empty(a.shape, np.uint16)
    _gen().rqgen_f32_to_bf16(a.ctypes.data, a.size, out.ctypes.data)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 raw bits to float32."""
    return (np.ascontiguousarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------------------------
# Workloads
# --------------------------------------------------------------------------------------------


@dataclass(frozen=True)
class Config:
    """Model shape + workload.  Field names mirror the C ABI's moshi_config."""

    name: str
    n_layers: int
    d_model: int
    n_heads: int
    ffn_hidden: int
    context: int
    text_card: int
    audio_card: int
    dep_layers: int
    dep_d_model: int
    dep_heads: int
    dep_ffn_hidden: int
    dep_q: int = 8
    rope_theta: float = 10000.0
    rms_eps: float = 1e-8
    dtype: str = "bf16"  # storage of the generated weights: 'f32' or 'bf16'
    band: str = "bf16"  # weight band on the device: 'f32', 'bf16', 'i8', 'q4' or 'q8'
    batch: int = 1
    seed: int = 0
    frames: int = 16
    prefill: int = 0  # teacher-forced frames before the measured/greedy frames
    max_start_offset: int = 0  # >0: per-conversation start offsets U{0..max-1} (teacher-forced)
    weight_std: float = 0.02
    extra: dict = field(default_factory=dict, compare=False)

    @property
    def n_streams(self) -> int:
        return 2 * self.dep_q + 1

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


TINY = Config(
    name="tiny_f32", n_layers=2, d_model=256, n_heads=4, ffn_hidden=704, context=64,
    text_card=1000, audio_card=2048, dep_layers=2, dep_d_model=128, dep_heads=2,
    dep_ffn_hidden=352, dtype="f32", band="f32", seed=0, frames=16,
)

MOSHI7B = Config(
    name="moshi7b_bf16_b1", n_layers=32, d_model=4096, n_heads=32, ffn_hidden=11264, context=3000,
    text_card=32000, audio_card=2048, dep_layers=6, dep_d_model=1024, dep_heads=16,
    dep_ffn_hidden=2816, dtype="bf16", band="bf16", seed=1, frames=250,
)

MOSHI7B_LONG = MOSHI7B.with_(name="moshi7b_bf16_long", seed=2, prefill=2900, frames=100)
MOSHI7B_B64 = MOSHI7B.with_(name="moshi7b_bf16_b64", seed=3, batch=64, frames=200, max_start_offset=1000)
MOSHI7B_I8 = MOSHI7B.with_(name="moshi7b_i8_b1", seed=4, band="i8", frames=250)

# the 4-bit and 8-bit block bands ([LM] load_q4sim's Q4_0, qn_roundtrip's q8_0 at group 32)
MOSHI7B_Q4 = MOSHI7B.with_(name="moshi7b_q4_b1", seed=5, band="q4", frames=250)
MOSHI7B_Q8 = MOSHI7B.with_(name="moshi7b_q8_b1", seed=6, band="q8", frames=250)

# teacher-forced priming as a workload of its own: prefill 2900 frames from offset 0, timed
MOSHI7B_PREFILL = MOSHI7B.with_(name="moshi7b_bf16_prefill", seed=2, prefill=2900, frames=5)

CONFIGS = {c.name: c for c in (TINY, MOSHI7B, MOSHI7B_LONG, MOSHI7B_B64, MOSHI7B_I8, MOSHI7B_Q4, MOSHI7B_Q8,
                               MOSHI7B_PREFILL)}


def weight_specs(cfg: Config):
    """(name, shape, kind) for every tensor, in the checkpoint load order; kind is
    'embedding', 'linear' or 'norm'."""
    D, F, L = cfg.d_model, cfg.ffn_hidden, cfg.n_layers
    Dd, Fd, Q = cfg.dep_d_model, cfg.dep_ffn_hidden, cfg.dep_q
    Vt, Va = cfg.text_card, cfg.audio_card
    specs = []
    for k in range(2 * Q):
        specs.append((f"emb.{k}.weight", (Va + 1, D), "embedding"))
    for l in range(L):
        p = f"transformer.layers.{l}"
        specs += [
            (f"{p}.norm1.alpha", (D,), "norm"),
            (f"{p}.self_attn.in_projs.0.weight", (3 * D, D), "linear"),
            (f"{p}.self_attn.out_projs.0.weight", (D, D), "linear"),
            (f"{p}.norm2.alpha", (D,), "norm"),
            (f"{p}.gating.linear_in.weight", (2 * F, D), "linear"),
            (f"{p}.gating.linear_out.weight", (D, F), "linear"),
        ]
    for l in range(cfg.dep_layers):
        p = f"depformer.layers.{l}"
        specs += [(f"{p}.norm1.alpha", (Dd,), "norm"), (f"{p}.norm2.alpha", (Dd,), "norm")]
        for s in range(Q):
            specs += [
                (f"{p}.self_attn.in_projs.{s}.weight", (3 * Dd, Dd), "linear"),
                (f"{p}.self_attn.out_projs.{s}.weight", (Dd, Dd), "linear"),
                (f"{p}.gating.{s}.linear_in.weight", (2 * Fd, Dd), "linear"),
                (f"{p}.gating.{s}.linear_out.weight", (Dd, Fd), "linear"),
            ]
    for s in range(Q):
        specs.append((f"depformer_in.{s}.weight", (Dd, D), "linear"))
        specs.append((f"linears.{s}.weight", (Va, Dd), "linear"))
    for k in range(Q - 1):
        specs.append((f"depformer_emb.{k}.weight", (Va + 1, Dd), "embedding"))
    specs += [
        ("text_emb.weight", (Vt + 1, D), "embedding"),
        ("out_norm.alpha", (D,), "norm"),
        ("text_linear.weight", (Vt, D), "linear"),
        ("depformer_text_emb.weight", (Vt + 1, Dd), "embedding"),
    ]
    return specs


def gen_weights(cfg: Config, seed: int | None = None, dtype: str | None = None) -> dict:
    """All tensors of `cfg`: linears and embeddings N(0, weight_std^2) in `dtype` ('f32' float32 or
    'bf16' uint16 bits); norm gains are all ones (float32)."""
    seed = cfg.seed if seed is None else seed
    dtype = dtype or cfg.dtype
    out = {}
    for name, shape, kind in weight_specs(cfg):
        if kind == "norm":
            out[name] = np.ones(shape, np.float32)
        else:
            out[name] = normal(seed, "w/" + name, shape, cfg.weight_std, dtype)
    return out


def user_tokens(cfg: Config, frames: int, conv: int = 0, start_frame: int = 0) -> np.ndarray:
    """User audio tokens [frames][dep_q], uniform on {0 .. audio_card-1}, stream user/<conv>."""
    return uniform_int(cfg.seed, f"user/{conv}", (frames, cfg.dep_q), cfg.audio_card,
                       start=start_frame * cfg.dep_q)


def prefill_tokens(cfg: Config, T: int, conv: int = 0):
    """Teacher-forced prefill streams: text [T] on {0..text_card-1}; agent and user audio [T][dep_q]
    on {0..audio_card-1}."""
    text = uniform_int(cfg.seed, f"prefill_text/{conv}", (T,), cfg.text_card)
    agent = uniform_int(cfg.seed, f"prefill_agent/{conv}", (T, cfg.dep_q), cfg.audio_card)
    user = uniform_int(cfg.seed, f"prefill_user/{conv}", (T, cfg.dep_q), cfg.audio_card)
    return text, agent, user


def start_offsets(cfg: Config) -> np.ndarray:
    """Per-conversation start offsets U{0..max_start_offset-1} (batched workload)."""
    if cfg.max_start_offset <= 0:
        return np.zeros(cfg.batch, np.int32)
    return uniform_int(cfg.seed, "start_offset", (cfg.batch,), cfg.max_start_offset)
