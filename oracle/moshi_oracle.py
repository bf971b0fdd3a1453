"""Plain CPU oracle of the Moshi RQ-Transformer frame step, in float32.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg use it.

What it follows (docs.rs source pages, cited by page title and item):
  [LM]   inferencelayer 0.2.4, src/moshi_lm.rs -- the module doc (the contract: streams, delays,
         ring, summed embeddings, RMSNorm with eps inside, interleaved rope, gated FFN, out_norm
         before both consumers, depformer reset and per-step weights, first-wins greedy) and the
         items rms_norm, silu, argmax, rope_row, attend, MoshiLm::embed, temporal_step,
         depformer_cycle, step_ext, step_forced, step_full_ext, force_generated, state.
  [RLX]  rlx-moshi 0.2.11, src/rlx_lm.rs -- build_temporal_graph: the same temporal stack run
         over a whole causal sequence, used here for the teacher-forced prefill form.

Precision: float32, as the [LM] page computes.  Matrix-vector and matrix-matrix products are
numpy float32 matmuls (a library primitive); every other step is written out.  Transcendentals
whose argument the page builds in float32 (ln/exp of the rope frequency, sin/cos of the rope
angle) are evaluated in float64 and rounded once to float32, i.e. the correctly rounded float32
value of the page's float32 argument.

Readings where the pages leave a step open:
  * rope pairs are interleaved (2i, 2i+1) -- [LM] module doc and rope_row (rlx_lm.rs says
    rotate-half; [LM] wins);
  * the depformer is conditioned on the post-out_norm hidden ([LM]; rlx_lm.rs feeds pre-norm);
  * depformer norms are shared across the 8 steps ([LM] DepLayer);
  * the text head has text_card rows (32000), the embedding tables text_card + 1;
  * int8 band: per output row s = max|w| / 127 (float32), q = round-half-away(w / s) clamped to
    [-127, 127], q = 0 where s = 0; y = s * (q . x).
  * window: keep the last `context` positions, current one included ([LM] temporal_step).

Pins: tests/test_oracle_pins.py checks every function against closed forms, brute force on tiny
inputs, invariants and the ring schedule that the [LM] module doc fixes.
"""
from __future__ import annotations

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


def _bf16_to_f32(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(F32)


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


class OracleLM:
    """The frame step of [LM] MoshiLm for one conversation.

    `weights` maps the checkpoint names to arrays: float32, or uint16 bfloat16 bits (widened
    exactly to float32).  `band='i8sim'` replaces every linear by its int8-dequantised copy
    (storage loss only, float32 compute)."""

    def __init__(self, cfg, weights: dict, band: str = "f32"):
        self.cfg = cfg
        self.band = band
        c = cfg
        self.Q = c.dep_q
        self.NS = 2 * c.dep_q + 1
        self.delays = stream_delays(c.dep_q)

        def emb(name):
            a = weights[name]
            return _bf16_to_f32(a) if a.dtype == np.uint16 else np.asarray(a, F32)

        def lin(name):
            W = emb(name)
            if band == "i8sim":
                W = dequantize_rows_int8(*quantize_rows_int8(W))
            return np.ascontiguousarray(W, F32)

        self.emb = [emb(f"emb.{k}.weight") for k in range(2 * c.dep_q)]
        self.text_emb = emb("text_emb.weight")
        self.layers = []
        for l in range(c.n_layers):
            p = f"transformer.layers.{l}"
            self.layers.append(dict(
                norm1=emb(f"{p}.norm1.alpha"), norm2=emb(f"{p}.norm2.alpha"),
                w_in=lin(f"{p}.self_attn.in_projs.0.weight"), w_out=lin(f"{p}.self_attn.out_projs.0.weight"),
                w_gin=lin(f"{p}.gating.linear_in.weight"), w_gout=lin(f"{p}.gating.linear_out.weight"),
            ))
        self.out_norm = emb("out_norm.alpha")
        self.text_linear = lin("text_linear.weight")
        self.dep_in = [lin(f"depformer_in.{s}.weight") for s in range(c.dep_q)]
        self.linears = [lin(f"linears.{s}.weight") for s in range(c.dep_q)]
        self.dep_text_emb = emb("depformer_text_emb.weight")
        self.dep_emb = [emb(f"depformer_emb.{k}.weight") for k in range(c.dep_q - 1)]
        self.dep_layers = []
        for l in range(c.dep_layers):
            p = f"depformer.layers.{l}"
            self.dep_layers.append(dict(
                norm1=emb(f"{p}.norm1.alpha"), norm2=emb(f"{p}.norm2.alpha"),
                w_in=[lin(f"{p}.self_attn.in_projs.{s}.weight") for s in range(c.dep_q)],
                w_out=[lin(f"{p}.self_attn.out_projs.{s}.weight") for s in range(c.dep_q)],
                w_gin=[lin(f"{p}.gating.{s}.linear_in.weight") for s in range(c.dep_q)],
                w_gout=[lin(f"{p}.gating.{s}.linear_out.weight") for s in range(c.dep_q)],
            ))

    # -- session -----------------------------------------------------------------------------

    def new_state(self) -> OracleState:
        """[LM] state(): ring all UNGENERATED, offset 0, empty KV."""
        c = self.cfg
        return OracleState(self.NS, c.n_layers, c.d_model, c.context)

    def write_user(self, st: OracleState, user):
        """[LM] step_ext step 1: user token k goes to stream Q+1+k at slot (offset + delay) % 3."""
        for k, tok in enumerate(user):
            s = self.Q + 1 + k
            st.ring[s][(st.offset + self.delays[s]) % RING] = int(tok)

    def gather(self, st: OracleState):
        """[LM] step_ext step 2: read slot offset % 3; INITIAL while offset <= delay."""
        c = self.cfg
        inp = np.zeros(self.NS, np.int64)
        for s in range(self.NS):
            if st.offset <= self.delays[s]:
                inp[s] = initial_token(s, c.text_card, c.audio_card)
            else:
                inp[s] = st.ring[s][st.offset % RING]
        return inp

    def embed_sum(self, inp):
        """[LM] step_ext step 3: the 2Q audio tables in order, then the text table."""
        x = np.zeros(self.cfg.d_model, F32)
        for k in range(2 * self.Q):
            embed_add(x, self.emb[k], inp[1 + k])
        embed_add(x, self.text_emb, inp[0])
        return x

    def advance(self, st: OracleState, text: int, audio):
        """[LM] step_ext steps 7-8: offset += 1, write text/audio at offset % 3, then the
        delay-realigned output once offset > max_delay."""
        st.offset += 1
        p = st.offset % RING
        st.ring[0][p] = int(text)
        for cb, tok in enumerate(audio):
            st.ring[1 + cb][p] = int(tok)
        if st.offset > MAX_DELAY:
            return [int(st.ring[s][(st.offset - MAX_DELAY + self.delays[s]) % RING]) for s in range(self.Q + 1)]
        return None

    def force_generated(self, st: OracleState, text: int, audio):
        """[LM] force_generated: overwrite the just-generated slot offset % 3."""
        p = st.offset % RING
        st.ring[0][p] = int(text)
        for cb, tok in enumerate(audio):
            st.ring[1 + cb][p] = int(tok)

    # -- networks ----------------------------------------------------------------------------

    def temporal_step(self, x, st: OracleState):
        """[LM] temporal_step at pos = offset: per layer norm1 -> fused qkv -> rope q,k -> push KV
        -> attend -> out_proj + residual -> norm2 -> gate_in -> silu(gate) * mult -> gate_out +
        residual; returns out_norm(x)."""
        c = self.cfg
        D, hd, F = c.d_model, c.d_model // c.n_heads, c.ffn_hidden
        pos = st.offset
        x = np.asarray(x, F32).copy()
        for l, ly in enumerate(self.layers):
            h = rms_norm(x, ly["norm1"], c.rms_eps)
            qkv = ly["w_in"] @ h
            q = rope_interleaved(qkv[:D], pos, hd, c.rope_theta)
            k = rope_interleaved(qkv[D:2 * D], pos, hd, c.rope_theta)
            v = qkv[2 * D:]
            st.push_kv(l, k, v)
            o = attend(q, st.K[l], st.V[l], c.n_heads, hd)
            x = x + ly["w_out"] @ o
            h = rms_norm(x, ly["norm2"], c.rms_eps)
            g = ly["w_gin"] @ h
            x = x + ly["w_gout"] @ (silu(g[:F]) * g[F:])
        return rms_norm(x, self.out_norm, c.rms_eps)

    def depformer_cycle(self, hidden, text_token: int):
        """[LM] depformer_cycle: 8 sequential steps with a KV that lives only within the frame.
        Step cb: x = depformer_in[cb] . hidden + emb(prev) (prev = text for cb 0 with the depformer
        text table, else the previous codebook's token with depformer_emb[cb-1]); the dep layers
        use per-step projections, shared norms and no rope; logits = linears[cb] . x (no norm)."""
        c = self.cfg
        Dd, hdd, Fd = c.dep_d_model, c.dep_d_model // c.dep_heads, c.dep_ffn_hidden
        Kc = [np.zeros((0, Dd), F32) for _ in self.dep_layers]
        Vc = [np.zeros((0, Dd), F32) for _ in self.dep_layers]
        logits_all, tokens = [], []
        prev = int(text_token)
        for cb in range(self.Q):
            x = self.dep_in[cb] @ np.asarray(hidden, F32)
            table = self.dep_text_emb if cb == 0 else self.dep_emb[cb - 1]
            embed_add(x, table, prev)
            for l, ly in enumerate(self.dep_layers):
                h = rms_norm(x, ly["norm1"], c.rms_eps)
                qkv = ly["w_in"][cb] @ h
                Kc[l] = np.concatenate([Kc[l], qkv[None, Dd:2 * Dd]])
                Vc[l] = np.concatenate([Vc[l], qkv[None, 2 * Dd:]])
                o = attend(qkv[:Dd], Kc[l], Vc[l], c.dep_heads, hdd)
                x = x + ly["w_out"][cb] @ o
                h = rms_norm(x, ly["norm2"], c.rms_eps)
                g = ly["w_gin"][cb] @ h
                x = x + ly["w_gout"][cb] @ (silu(g[:Fd]) * g[Fd:])
            logits = self.linears[cb] @ x
            tok = argmax_first(logits)
            logits_all.append(logits)
            tokens.append(tok)
            prev = tok
        return np.stack(logits_all), tokens

    # -- steps -------------------------------------------------------------------------------

    def step(self, st: OracleState, user) -> dict:
        """[LM] step / step_ext: one 80 ms frame, greedy.  Returns the StepTrace fields."""
        self.write_user(st, user)
        inp = self.gather(st)
        x = self.embed_sum(inp)
        hidden = self.temporal_step(x, st)
        text_logits = self.text_linear @ hidden
        text = argmax_first(text_logits)
        audio_logits, audio = self.depformer_cycle(hidden, text)
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
        inp = self.gather(st)
        x = self.embed_sum(inp)
        self.temporal_step(x, st)
        st.offset += 1
        p = st.offset % RING
        st.ring[0][p] = int(text)
        for cb, tok in enumerate(agent):
            st.ring[1 + cb][p] = int(tok)

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
            p = st.offset % RING
            st.ring[0][p] = int(text[t])
            for cb, tok in enumerate(agent[t]):
                st.ring[1 + cb][p] = int(agent[t][cb])
        pos = np.arange(p0, p0 + T)
        scale = F32(1.0) / np.sqrt(F32(hd))
        for l, ly in enumerate(self.layers):
            H = rms_norm_rows(X, ly["norm1"], c.rms_eps)
            QKV = H @ ly["w_in"].T
            Qm = np.stack([rope_interleaved(QKV[t, :D], pos[t], hd, c.rope_theta) for t in range(T)])
            Km = np.stack([rope_interleaved(QKV[t, D:2 * D], pos[t], hd, c.rope_theta) for t in range(T)])
            Vm = QKV[:, 2 * D:]
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
