"""Plain CPU oracle of the Moshi RQ-Transformer frame step, in float32.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg use it.

What it follows (docs.rs source pages, cited by page title and item):
  [LM]   inferencelayer 0.2.4, src/moshi_lm.rs -- the module doc (the contract: streams, delays,
         ring, summed embeddings, RMSNorm with eps inside, interleaved rope, gated FFN, out_norm
         before both consumers, depformer reset and per-step weights, first-wins greedy) and the
         items rms_norm, silu, argmax, rope_row, attend, MoshiLm::embed, temporal_step,
         depformer_cycle, step_ext, step_forced, step_full_ext, force_generated, state,
         MoshiState::snapshot; for the sampled modes xorshift_u01, topk_sample,
         gumbel_full_pick, Sampling and MoshiLm::pick; for the 4-bit and 8-bit block bands
         q4_roundtrip, qn_roundtrip and MoshiLm::load_q4sim.
  [RLX]  rlx-moshi 0.2.11, src/rlx_lm.rs -- build_temporal_graph: the same temporal stack run
         over a whole causal sequence, used here for the teacher-forced prefill form.

Precision: float32, as the [LM] page computes.  Matrix-vector and matrix-matrix products are
numpy float32 matmuls (a library primitive); every other step is written out.  Transcendentals
whose argument the page builds in float32 (ln/exp of the rope frequency, sin/cos of the rope
angle) are evaluated in float64 and rounded once to float32, i.e. the correctly rounded float32
value of the page's float32 argument.  The samplers work in float64 where the page does
(softmax weights, the uniform, the Gumbel transform) and in float32 where it does (logit / T).

Readings where the pages leave a step open:
  * rope pairs are interleaved (2i, 2i+1) -- [LM] module doc and rope_row (rlx_lm.rs says
    rotate-half; [LM] wins);
  * the depformer is conditioned on the post-out_norm hidden ([LM]; rlx_lm.rs feeds pre-norm);
  * depformer norms are shared across the 8 steps ([LM] DepLayer);
  * the text head has text_card rows (32000), the embedding tables text_card + 1;
  * int8 band: per output row s = max|w| / 127 (float32), q = round-half-away(w / s) clamped to
    [-127, 127], q = 0 where s = 0; y = s * (q . x).
  * window: keep the last `context` positions, current one included ([LM] temporal_step).
  * top-k sampling: the page keeps the k largest logits in the unspecified order a partial
    selection leaves them and walks the inverse CDF in that order; here the candidates are
    ordered by decreasing logit, equal logits by increasing index, and equal logits at the k-th
    place are taken by increasing index.
  * Q4_0 quantiser (quantize_q4_0 itself is not printed): per row and 32-column block, the
    symmetric rule qn_roundtrip prints at 4 bits -- d = (the block's value of largest magnitude,
    the first one on ties) / -8, q = clamp(round-half-away(x * (1 / d)), -8, 7), q = 0 where
    d = 0 -- stored as the nibble q + 8, byte i of a block holding element i (low nibble) and
    element i + 16 (high nibble); float32 scales.  q8_0: the same rule at 8 bits (d = value /
    -128, q in [-128, 127]), int8 codes and one float32 scale per 32 columns.
  * the sampler's xorshift state belongs to the sampler (one per conversation here, one per model
    on the page, the same thing for a single conversation); a session snapshot does not hold it.

Pins: tests/test_oracle_pins.py checks every function against closed forms, brute force on tiny
inputs, invariants, the ring schedule that the [LM] module doc fixes, and (tests/ref_f64.py) an
independent float64 implementation of the whole frame.
"""
from __future__ import annotations

import copy
import math

import numpy as np

F32 = np.float32
UNGENERATED = -2  # [LM] constant: the ring's initial token
MAX_DELAY = 1  # [LM] constants: max delay and ring length max_delay + 2
RING = MAX_DELAY + 2


def stream_delays(dep_q: int = 8) -> list[int]:
    """[LM] DELAYS: text 0 | generated cb0 0, cb1.. 1 | user cb0 0, cb1.. 1."""
    gen = [0] + [1] * (dep_q - 1)
    return [0] + gen + gen


def initial_token(stream: int, text_card: int, audio_card: int) -> int:
    """[LM] INITIAL token: text_card for the text stream, audio_card for audio streams."""
    return text_card if stream == 0 else audio_card


# ------------------------------------------------------------------------------------------
# Primitives
# ------------------------------------------------------------------------------------------


def rms_norm(x, alpha, eps: float):
    """[LM] rms_norm: y = x * alpha * 1/sqrt(eps + mean(x^2)); eps inside the mean, no centering."""
    x = np.asarray(x, F32)
    var = F32(eps) + F32(np.sum(x * x, dtype=F32)) / F32(x.shape[-1])
    inv = F32(1.0) / np.sqrt(var)
    return (x * np.asarray(alpha, F32)) * inv


def rms_norm_rows(X, alpha, eps: float):
    """rms_norm applied to each row of X independently."""
    return np.stack([rms_norm(r, alpha, eps) for r in np.asarray(X, F32)]) if len(X) else np.zeros_like(X, F32)


def rope_freqs(head_dim: int, theta: float = 10000.0):
    """[LM] rope_row frequencies: f_i = exp(-ln(theta) * 2 * i / head_dim), built in float32."""
    ln_theta = F32(np.log(np.float64(F32(theta))))
    i = np.arange(head_dim // 2, dtype=F32)
    arg = ((-ln_theta) * F32(2.0)) * i / F32(head_dim)
    return np.exp(arg.astype(np.float64)).astype(F32)


def rope_interleaved(row, pos: int, head_dim: int, theta: float = 10000.0):
    """[LM] rope_row: rotate each interleaved pair (2i, 2i+1) of every head by f_i * pos radians
    (angle formed in float32)."""
    row = np.asarray(row, F32).copy()
    freqs = rope_freqs(head_dim, theta)
    ang = freqs * F32(pos)
    sin = np.sin(ang.astype(np.float64)).astype(F32)
    cos = np.cos(ang.astype(np.float64)).astype(F32)
    heads = row.reshape(-1, head_dim)
    re = heads[:, 0::2].copy()
    im = heads[:, 1::2].copy()
    heads[:, 0::2] = re * cos - im * sin
    heads[:, 1::2] = re * sin + im * cos
    return heads.reshape(-1)


def attend(q, K, V, heads: int, head_dim: int):
    """[LM] attend: one query against cached keys/values [n, heads*head_dim]; per head the scores
    (q.k) are scaled by 1/sqrt(head_dim) after the dot, softmaxed with the max subtracted, and
    the output is sum_j (e_j / den) v_j."""
    q = np.asarray(q, F32)
    K = np.asarray(K, F32)
    V = np.asarray(V, F32)
    scale = F32(1.0) / np.sqrt(F32(head_dim))
    out = np.zeros(heads * head_dim, F32)
    for h in range(heads):
        sl = slice(h * head_dim, (h + 1) * head_dim)
        scores = (K[:, sl] @ q[sl]) * scale
        e = np.exp(scores - scores.max())
        den = np.sum(e, dtype=F32)
        out[sl] = (e / den) @ V[:, sl]
    return out


def silu(x):
    """[LM] silu: x / (1 + exp(-x))."""
    x = np.asarray(x, F32)
    return x / (F32(1.0) + np.exp(-x))


def argmax_first(v) -> int:
    """[LM] argmax: strict '>' scan from (-inf, 0), i.e. the first index holding the maximum of
    the values above -inf; NaN is never chosen; nothing above -inf gives 0."""
    v = np.asarray(v, F32)
    ok = v > -np.inf
    if not ok.any():
        return 0
    return int(np.flatnonzero(v == v[ok].max())[0])


def embed_add(acc, table, tok: int):
    """[LM] MoshiLm::embed: token -1 adds nothing; otherwise add row max(tok, 0)."""
    if tok == -1:
        return acc
    acc += table[max(int(tok), 0)]
    return acc


def quantize_rows_int8(W):
    """int8 band quantiser (per output row, symmetric): returns (q int8 [N,K], s float32 [N])."""
    W = np.asarray(W, F32)
    amax = np.max(np.abs(W), axis=1)
    s = (amax / F32(127.0)).astype(F32)
    safe = np.where(s > 0, s, F32(1.0)).astype(F32)
    v = (W / safe[:, None]).astype(F32)
    r = np.floor(np.abs(v.astype(np.float64)) + 0.5) * np.sign(v)
    q = np.clip(r, -127, 127).astype(np.int8)
    q[s == 0] = 0
    return q, s


def dequantize_rows_int8(q, s):
    return q.astype(F32) * np.asarray(s, F32)[:, None]


def round_bf16(x):
    """float32 -> the nearest bfloat16 value (ties to even), returned as float32: keep the top 16
    bits after adding 0x7FFF plus the lowest kept bit (finite inputs)."""
    u = np.asarray(x, F32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(F32)


def bf16_to_f32(b):
    """Exact widening of bfloat16 raw bits (uint16) to float32: the bits become the top half."""
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(F32)


_bf16_to_f32 = bf16_to_f32


# ------------------------------------------------------------------------------------------
# Block quantisers ([LM] qn_roundtrip, q4_roundtrip; the Q4_0 and q8_0 bands)
# ------------------------------------------------------------------------------------------

GROUP = 32  # columns per quantisation block


def _round_half_away(v):
    """Rust f32::round on float32 values: ties away from zero (exact in float64)."""
    v64 = np.asarray(v, np.float64)
    return np.sign(v64) * np.floor(np.abs(v64) + 0.5)


def quantize_blocks(W, bits: int):
    """[LM] qn_roundtrip's symmetric rule, per row and 32-column block: the block's value of
    largest magnitude (the first one on ties) divided by -2^(bits-1) is the scale d; the code is
    round-half-away(x * (1/d)) clamped to [-2^(bits-1), 2^(bits-1) - 1], 0 where d = 0.
    Returns (codes int8 [N, K], d float32 [N, K/32])."""
    W = np.asarray(W, F32)
    N, K = W.shape
    assert K % GROUP == 0, K
    qmin, qmax = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    blk = W.reshape(N, K // GROUP, GROUP)
    first = np.argmax(np.abs(blk), axis=2)  # first index of the largest magnitude
    mx = np.take_along_axis(blk, first[..., None], axis=2)[..., 0]
    d = (mx / F32(qmin)).astype(F32)
    inv = np.zeros_like(d)
    nz = d != 0
    inv[nz] = F32(1.0) / d[nz]
    v = (blk * inv[..., None]).astype(F32)
    q = np.clip(_round_half_away(v), qmin, qmax).astype(np.int8)
    return q.reshape(N, K), d


def dequantize_blocks(q, d):
    N, K = q.shape
    return (q.reshape(N, K // GROUP, GROUP).astype(F32) * np.asarray(d, F32)[..., None]).reshape(N, K)


def pack_q4_0(q):
    """Q4_0 storage of 4-bit codes [N, K]: per 32-column block 16 bytes, byte i = (q[i] + 8) |
    (q[i + 16] + 8) << 4 ([LM] q4_roundtrip's layout)."""
    N, K = q.shape
    u = (q.astype(np.int16) + 8).astype(np.uint8).reshape(N, K // GROUP, GROUP)
    return (u[..., :16] | (u[..., 16:] << 4)).reshape(N, K // 2)


def unpack_q4_0(nib, K: int):
    """Codes [N, K] of Q4_0 storage (byte i of a block: low nibble element i, high element i+16)."""
    N = nib.shape[0]
    b = np.asarray(nib, np.uint8).reshape(N, K // GROUP, 16)
    lo = (b & 0x0F).astype(np.int16) - 8
    hi = (b >> 4).astype(np.int16) - 8
    return np.concatenate([lo, hi], axis=2).reshape(N, K).astype(np.int8)


# ------------------------------------------------------------------------------------------
# Samplers ([LM] xorshift_u01, topk_sample, gumbel_full_pick, Sampling, MoshiLm::pick)
# ------------------------------------------------------------------------------------------

_M64 = (1 << 64) - 1


def xorshift64(state: int) -> int:
    """One step of the 64-bit xorshift (shifts 13, 7, 17) the [LM] sampler draws from."""
    x = state & _M64
    x ^= (x << 13) & _M64
    x ^= x >> 7
    x ^= (x << 17) & _M64
    return x


def u01(state: int):
    """[LM] xorshift_u01: advance, then the top 53 bits as a uniform in [0, 1).  Returns
    (u, new_state)."""
    x = xorshift64(state)
    return (x >> 11) / float(1 << 53), x


class Sampling:
    """[LM] Sampling (LMGen defaults: audio T 0.8, text T 0.7, top-k 250 / 25) and its xorshift
    state, seeded with max(seed, 1) as [LM] set_sampling does."""

    def __init__(self, seed: int, temp=0.8, temp_text=0.7, top_k=250, top_k_text=25, gumbel_full=False):
        self.temp, self.temp_text = F32(temp), F32(temp_text)
        self.top_k, self.top_k_text = int(top_k), int(top_k_text)
        self.gumbel_full = bool(gumbel_full)
        self.state = max(int(seed) & _M64, 1)

    def draw(self) -> float:
        u, self.state = u01(self.state)
        return u


def topk_sample(logits, temp, k: int, draw) -> int:
    """[LM] topk_sample: the k largest logits (order: decreasing logit, then increasing index),
    weights exp(float64((l - max) / T)) normalised by their float64 sum, one uniform, and the
    first candidate at which the running u - p_1 - ... - p_i reaches <= 0 (else the last)."""
    lg = np.asarray(logits, F32)
    k = min(int(k), len(lg))
    order = sorted(range(len(lg)), key=lambda i: (-float(lg[i]), i))[:k]
    vals = [lg[i] for i in order]
    mx = F32(max(vals))
    t = F32(temp)
    probs = [math.exp(float(F32(F32(v - mx) / t))) for v in vals]
    total = 0.0
    for p in probs:
        total += p
    probs = [p / total for p in probs]
    u = draw()
    for p, i in zip(probs, order):
        u -= p
        if u <= 0.0:
            return int(i)
    return int(order[-1])


def gumbel_full_pick(logits, temp, draw) -> int:
    """[LM] gumbel_full_pick: one uniform per logit in index order, g = float32(-ln(-ln(max(u,
    1e-300)))), score float32(l / T) + g, the first index of the largest score (strict '>' from
    -inf)."""
    lg = np.asarray(logits, F32)
    t = F32(temp)
    best_v, best_i = -math.inf, 0
    for i in range(len(lg)):
        u = max(draw(), 1e-300)
        g = F32(-math.log(-math.log(u)))
        sc = F32(F32(lg[i] / t) + g)
        if sc > best_v:
            best_v, best_i = sc, i
    return best_i


def pick(logits, text: bool, sampler) -> int:
    """[LM] MoshiLm::pick: greedy argmax without a sampler; else the text or audio temperature and
    k, full-vocabulary Gumbel-max or top-k."""
    if sampler is None:
        return argmax_first(logits)
    temp, k = (sampler.temp_text, sampler.top_k_text) if text else (sampler.temp, sampler.top_k)
    if sampler.gumbel_full:
        return gumbel_full_pick(logits, temp, sampler.draw)
    return topk_sample(logits, temp, k, sampler.draw)


# ------------------------------------------------------------------------------------------
# Model
# ------------------------------------------------------------------------------------------


class OracleState:
    """[LM] MoshiState: the 17x3 token ring, the offset and the temporal KV cache (position
    order, at most `context` entries)."""

    def __init__(self, n_streams: int, n_layers: int, d_model: int, context: int):
        self.ring = np.full((n_streams, RING), UNGENERATED, np.int64)
        self.offset = 0
        self.context = context
        self.K = [np.zeros((0, d_model), F32) for _ in range(n_layers)]
        self.V = [np.zeros((0, d_model), F32) for _ in range(n_layers)]

    def push_kv(self, layer: int, k, v):
        """Append one position; drop the oldest beyond `context` ([LM] temporal_step)."""
        K = np.concatenate([self.K[layer], np.asarray(k, F32)[None]])
        V = np.concatenate([self.V[layer], np.asarray(v, F32)[None]])
        if len(K) > self.context:
            K, V = K[1:], V[1:]
        self.K[layer], self.V[layer] = K, V
        return K, V

    def snapshot(self) -> "OracleState":
        """[LM] MoshiState::snapshot: an independent copy of the ring, the offset and the KV."""
        c = OracleState.__new__(OracleState)
        c.ring = self.ring.copy()
        c.offset = self.offset
        c.context = self.context
        c.K = [k.copy() for k in self.K]
        c.V = [v.copy() for v in self.V]
        return c


def block(x, norm1, norm2, W_in, W_out, W_gin, W_gout, eps, heads, hd, qk, kv):
    """One pre-norm layer of either transformer ([LM] temporal_step / depformer_cycle):
    h = rms_norm(x; norm1); [q | k | v] = W_in . h; q, k go through `qk` (rope, or nothing);
    kv(k, v) stores the new entry and returns the keys and values attended to;
    x += W_out . attend(q, K, V); h = rms_norm(x; norm2); g = W_gin . h; x += W_gout .
    (silu(g[:F]) * g[F:])."""
    D = x.shape[0]
    F = W_gout.shape[1]
    qkv = W_in @ rms_norm(x, norm1, eps)
    K, V = kv(qk(qkv[D:2 * D]), qkv[2 * D:])
    x = x + W_out @ attend(qk(qkv[:D]), K, V, heads, hd)
    g = W_gin @ rms_norm(x, norm2, eps)
    return x + W_gout @ (silu(g[:F]) * g[F:])


class OracleLM:
    """The frame step of [LM] MoshiLm for one conversation.

    `weights` maps the checkpoint names to arrays: float32, or uint16 bfloat16 bits (widened
    exactly to float32).  `band` picks the storage loss applied to every linear: 'f32' none,
    'i8sim' the per-row int8 band, 'q4sim' Q4_0 ([LM] load_q4sim), 'q8sim' q8_0 (float32 compute
    throughout).  `kv='bf16'` stores the temporal keys and values rounded to bfloat16 (the
    storage loss of a bfloat16 cache; attention reads every position from the cache)."""

    def __init__(self, cfg, weights: dict, band: str = "f32", kv: str = "f32"):
        self.cfg = c = cfg
        self.band = band
        if kv not in ("f32", "bf16"):
            raise ValueError(kv)
        self.kv_store = (lambda a: a) if kv == "f32" else round_bf16
        self.Q = c.dep_q
        self.NS = 2 * c.dep_q + 1
        self.delays = stream_delays(c.dep_q)
        self._delay = np.asarray(self.delays, np.int64)
        self._init = np.array([initial_token(s, c.text_card, c.audio_card) for s in range(self.NS)], np.int64)

        def emb(name):
            a = weights[name]
            return bf16_to_f32(a) if a.dtype == np.uint16 else np.asarray(a, F32)

        def lin(name):
            W = emb(name)
            if band == "i8sim":
                W = dequantize_rows_int8(*quantize_rows_int8(W))
            elif band == "q4sim":
                W = dequantize_blocks(*quantize_blocks(W, 4))
            elif band == "q8sim":
                W = dequantize_blocks(*quantize_blocks(W, 8))
            elif band != "f32":
                raise ValueError(band)
            return np.ascontiguousarray(W, F32)

        def layer(p, proj, gating):
            return dict(norm1=emb(f"{p}.norm1.alpha"), norm2=emb(f"{p}.norm2.alpha"),
                        w_in=lin(f"{p}.self_attn.in_projs.{proj}.weight"),
                        w_out=lin(f"{p}.self_attn.out_projs.{proj}.weight"),
                        w_gin=lin(f"{p}.{gating}.linear_in.weight"), w_gout=lin(f"{p}.{gating}.linear_out.weight"))

        self.emb = [emb(f"emb.{k}.weight") for k in range(2 * c.dep_q)]
        self.text_emb = emb("text_emb.weight")
        self.layers = [layer(f"transformer.layers.{l}", 0, "gating") for l in range(c.n_layers)]
        self.out_norm = emb("out_norm.alpha")
        self.text_linear = lin("text_linear.weight")
        self.dep_in = [lin(f"depformer_in.{s}.weight") for s in range(c.dep_q)]
        self.linears = [lin(f"linears.{s}.weight") for s in range(c.dep_q)]
        # the table the entry of step cb adds: the depformer text table for cb 0, else the
        # previous codebook's depformer_emb
        self.dep_tables = [emb("depformer_text_emb.weight")] + [emb(f"depformer_emb.{k}.weight") for k in range(c.dep_q - 1)]
        # dep_layers[j][cb]: layer j's weights as step cb uses them (norms shared by the steps)
        self.dep_layers = [[layer(f"depformer.layers.{j}", s, f"gating.{s}") for s in range(c.dep_q)]
                           for j in range(c.dep_layers)]

    def with_kv(self, kv: str) -> "OracleLM":
        """The same model (weights shared, not copied) with another KV storage ('f32' or 'bf16')."""
        other = copy.copy(self)
        if kv not in ("f32", "bf16"):
            raise ValueError(kv)
        other.kv_store = (lambda a: a) if kv == "f32" else round_bf16
        return other

    # -- session: the ring of the [LM] module doc ----------------------------------------------
    # Stream s holds RING slots; a token for step `offset` sits at slot (offset + delay[s]) % 3 and
    # is read at slot offset % 3, so a delayed stream is read one step after it was written.

    def new_state(self) -> OracleState:
        """[LM] state(): ring all UNGENERATED, offset 0, empty KV."""
        c = self.cfg
        return OracleState(self.NS, c.n_layers, c.d_model, c.context)

    def write_user(self, st: OracleState, user):
        """The user's codebooks go to streams Q+1 .. 2Q, each `delay` slots ahead."""
        s = np.arange(self.Q + 1, self.NS)
        st.ring[s, (st.offset + self._delay[s]) % RING] = np.asarray(user, np.int64)

    def gather(self, st: OracleState):
        """Model inputs: every stream's slot offset % 3, the INITIAL token while offset <= delay."""
        cur = st.ring[np.arange(self.NS), st.offset % RING]
        return np.where(st.offset <= self._delay, self._init, cur)

    def embed_sum(self, inp):
        """[LM] embed over the streams: the 2Q audio tables in order, then the text table."""
        x = np.zeros(self.cfg.d_model, F32)
        for k, table in enumerate(self.emb):
            embed_add(x, table, inp[1 + k])
        embed_add(x, self.text_emb, inp[0])
        return x

    def _record(self, st: OracleState, gen):
        """The step's generated tokens (text, audio...) go to slot offset % 3 of streams 0..Q."""
        st.ring[:self.Q + 1, st.offset % RING] = np.asarray(gen, np.int64)

    def advance(self, st: OracleState, text: int, audio):
        """Clock + 1, record the generated tokens, and once offset > max_delay return the
        delay-realigned output: stream s at slot (offset - max_delay + delay[s]) % 3."""
        st.offset += 1
        self._record(st, [text] + list(audio))
        if st.offset <= MAX_DELAY:
            return None
        s = np.arange(self.Q + 1)
        return st.ring[s, (st.offset - MAX_DELAY + self._delay[s]) % RING].tolist()

    def force_generated(self, st: OracleState, text: int, audio):
        """[LM] force_generated: overwrite what the last step recorded."""
        self._record(st, [text] + list(audio))

    # -- networks ----------------------------------------------------------------------------

    def temporal_step(self, x, st: OracleState):
        """[LM] temporal_step at pos = offset: every layer is `block` with interleaved rope at the
        absolute position on q and k and the sliding KV window of `context` entries; returns
        out_norm(x)."""
        c = self.cfg
        hd = c.d_model // c.n_heads
        pos = st.offset
        rope = lambda r: rope_interleaved(r, pos, hd, c.rope_theta)  # noqa: E731
        x = np.asarray(x, F32).copy()
        kvs = self.kv_store
        for l, ly in enumerate(self.layers):
            x = block(x, ly["norm1"], ly["norm2"], ly["w_in"], ly["w_out"], ly["w_gin"], ly["w_gout"], c.rms_eps,
                      c.n_heads, hd, rope, lambda k, v, l=l: st.push_kv(l, kvs(k), kvs(v)))
        return rms_norm(x, self.out_norm, c.rms_eps)

    def depformer_cycle(self, hidden, text_token: int, sampler=None):
        """[LM] depformer_cycle: Q sequential steps sharing a KV that lives only within the frame
        (one list of entries per layer).  Step cb's input is depformer_in[cb] . hidden plus the
        entry table's row of the previous token (the text token for cb 0); its layers use step
        cb's projections, the shared norms and no rope; its logits are linears[cb] . y with no
        norm, and its token (greedy, or the sampler's pick) feeds step cb + 1."""
        c = self.cfg
        hdd = c.dep_d_model // c.dep_heads
        keys = [[] for _ in self.dep_layers]
        vals = [[] for _ in self.dep_layers]

        def store(j):
            def kv(k, v):
                keys[j].append(k)
                vals[j].append(v)
                return np.stack(keys[j]), np.stack(vals[j])
            return kv

        same = lambda r: r  # noqa: E731
        hidden = np.asarray(hidden, F32)
        logits_all, tokens = [], []
        prev = int(text_token)
        for cb in range(self.Q):
            y = embed_add(self.dep_in[cb] @ hidden, self.dep_tables[cb], prev)
            for j, steps in enumerate(self.dep_layers):
                ly = steps[cb]
                y = block(y, ly["norm1"], ly["norm2"], ly["w_in"], ly["w_out"], ly["w_gin"], ly["w_gout"], c.rms_eps,
                          c.dep_heads, hdd, same, store(j))
            logits = self.linears[cb] @ y
            prev = pick(logits, False, sampler)
            logits_all.append(logits)
            tokens.append(prev)
        return np.stack(logits_all), tokens

    # -- steps -------------------------------------------------------------------------------

    def step(self, st: OracleState, user, sampler=None) -> dict:
        """[LM] step / step_ext: one 80 ms frame (greedy, or sampled with `sampler`).  Returns the
        StepTrace fields."""
        self.write_user(st, user)
        inp = self.gather(st)
        x = self.embed_sum(inp)
        hidden = self.temporal_step(x, st)
        text_logits = self.text_linear @ hidden
        text = pick(text_logits, True, sampler)
        audio_logits, audio = self.depformer_cycle(hidden, text, sampler)
        out = self.advance(st, text, audio)
        return dict(input_tokens=inp, emb_sum=x, transformer_out=hidden, text_logits=text_logits,
                    audio_logits=audio_logits, text_token=text, audio_tokens=audio, out=out)

    def step_with_network(self, st: OracleState, user, network):
        """[LM] step_full_ext: the ring bookkeeping around a caller-supplied network
        network(emb_sum, pos) -> (text, audio[Q])."""
        self.write_user(st, user)
        inp = self.gather(st)
        x = self.embed_sum(inp)
        text, audio = network(x, st.offset)
        out = self.advance(st, text, audio)
        return inp, text, list(audio), out

    def step_forced(self, st: OracleState, text: int, agent, user):
        """[LM] step_forced: teacher-forced step; the temporal advances on the gathered inputs,
        outputs are discarded and the ring records the forced text/agent tokens."""
        self.write_user(st, user)
        self.temporal_step(self.embed_sum(self.gather(st)), st)
        st.offset += 1
        self._record(st, [text] + list(agent))

    def prefill_forced(self, st: OracleState, text, agent, user):
        """T teacher-forced steps at once.  The forced tokens fix every input up front, so the T
        positions run as one causal sequence through the temporal stack ([RLX]
        build_temporal_graph), each position attending to the last `context` positions up to
        itself.  Leaves the state exactly as T calls of step_forced would (up to float32
        rounding order)."""
        c = self.cfg
        D, hd, F, C = c.d_model, c.d_model // c.n_heads, c.ffn_hidden, c.context
        T = len(text)
        if T == 0:
            return
        p0 = st.offset
        X = np.zeros((T, D), F32)
        for t in range(T):
            self.write_user(st, user[t])
            X[t] = self.embed_sum(self.gather(st))
            st.offset += 1
            self._record(st, [int(text[t])] + [int(a) for a in agent[t]])
        pos = np.arange(p0, p0 + T)
        scale = F32(1.0) / np.sqrt(F32(hd))
        for l, ly in enumerate(self.layers):
            H = rms_norm_rows(X, ly["norm1"], c.rms_eps)
            QKV = H @ ly["w_in"].T
            Qm = np.stack([rope_interleaved(QKV[t, :D], pos[t], hd, c.rope_theta) for t in range(T)])
            Km = self.kv_store(np.stack([rope_interleaved(QKV[t, D:2 * D], pos[t], hd, c.rope_theta) for t in range(T)]))
            Vm = self.kv_store(QKV[:, 2 * D:])
            n0 = len(st.K[l])
            Kall = np.concatenate([st.K[l], Km])
            Vall = np.concatenate([st.V[l], Vm])
            pall = np.arange(p0 - n0, p0 + T)
            mask = (pall[None, :] <= pos[:, None]) & (pall[None, :] > pos[:, None] - C)
            O = np.zeros((T, D), F32)
            for h in range(c.n_heads):
                sl = slice(h * hd, (h + 1) * hd)
                S = (Qm[:, sl] @ Kall[:, sl].T) * scale
                S = np.where(mask, S, F32(-np.inf))
                E = np.exp(S - S.max(axis=1, keepdims=True))
                den = np.sum(E, axis=1, dtype=F32, keepdims=True)
                O[:, sl] = (E / den) @ Vall[:, sl]
            X = X + O @ ly["w_out"].T
            H = rms_norm_rows(X, ly["norm2"], c.rms_eps)
            G = H @ ly["w_gin"].T
            X = X + (silu(G[:, :F]) * G[:, F:]) @ ly["w_gout"].T
            st.K[l], st.V[l] = Kall[-C:], Vall[-C:]
