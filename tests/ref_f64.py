"""An independent float64 implementation of the Moshi RQ-Transformer frame step, used only to pin
the float32 oracle (tests).  It shares no code with oracle/ and is written in another style:

* the token ring is replaced by its closed form (the input of a stream at step t is the token its
  producer made for step t - 1 - delay (generated) or t - delay (user), INITIAL before that), as
  the docs.rs page "inferencelayer 0.2.4 src/moshi_lm.rs" ([LM]) fixes it in its module doc;
* rope multiplies each interleaved pair, taken as a complex number, by exp(i f pos) with
  f = theta^(-2i/hd) in float64 ([LM] rope_row);
* attention is a masked softmax over all cached rows at once, per head ([LM] attend);
* RMSNorm, silu and the gated FFN are written from the module doc's formulas.
"""
import numpy as np

F64 = np.float64


def widen(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(F64)
    return a.astype(F64)


def rmsn(x, g, eps):
    return g * x / np.sqrt(eps + np.mean(x * x))


def rope_c(v, pos, hd, theta):
    heads = v.reshape(-1, hd)
    z = heads[:, 0::2] + 1j * heads[:, 1::2]
    z = z * np.exp(1j * pos * theta ** (-np.arange(0, hd, 2) / hd))
    out = np.empty_like(heads)
    out[:, 0::2], out[:, 1::2] = z.real, z.imag
    return out.reshape(-1)


def attention(q, K, V, heads):
    hd = q.shape[0] // heads
    qh = q.reshape(heads, hd)
    Kh = K.reshape(len(K), heads, hd)
    Vh = V.reshape(len(V), heads, hd)
    s = np.einsum("hd,nhd->hn", qh, Kh) / np.sqrt(hd)
    s = np.exp(s - s.max(axis=1, keepdims=True))
    s /= s.sum(axis=1, keepdims=True)
    return np.einsum("hn,nhd->hd", s, Vh).reshape(-1)


def gated(x, Win, Wout, g, eps):
    h = Win @ rmsn(x, g, eps)
    F = h.shape[0] // 2
    a, m = h[:F], h[F:]
    return x + Wout @ (a / (1 + np.exp(-a)) * m)


class RefF64:
    """Whole-frame float64 reference for one conversation, driven step by step.  `generated(t)`
    gives the text and audio tokens recorded for step t (the test feeds the oracle's own, so both
    sides see the same inputs)."""

    def __init__(self, cfg, w):
        self.c = cfg
        self.w = {k: widen(v) for k, v in w.items()}
        Q = cfg.dep_q
        self.delay = np.array([0] + [0] + [1] * (Q - 1) + [0] + [1] * (Q - 1))
        self.K = [[] for _ in range(cfg.n_layers)]
        self.V = [[] for _ in range(cfg.n_layers)]
        self.gen = {}   # step -> [text, audio...]
        self.user = {}  # step -> user tokens

    def inputs(self, t):
        c, Q = self.c, self.c.dep_q
        out = []
        for s in range(2 * Q + 1):
            d = int(self.delay[s])
            if t <= d:
                out.append(c.text_card if s == 0 else c.audio_card)
            elif s <= Q:
                out.append(self.gen[t - 1 - d][s] if d == 0 else self.gen[t - 1][s])
            else:
                out.append(self.user[t - d][s - Q - 1])
        return out

    def temporal(self, t, toks):
        c, w = self.c, self.w
        Q = c.dep_q
        x = np.zeros(c.d_model)
        for k in range(2 * Q):
            if toks[1 + k] != -1:
                x += w[f"emb.{k}.weight"][max(toks[1 + k], 0)]
        if toks[0] != -1:
            x += w["text_emb.weight"][max(toks[0], 0)]
        emb = x.copy()
        D, hd = c.d_model, c.d_model // c.n_heads
        for l in range(c.n_layers):
            p = f"transformer.layers.{l}"
            qkv = w[f"{p}.self_attn.in_projs.0.weight"] @ rmsn(x, w[f"{p}.norm1.alpha"], c.rms_eps)
            self.K[l].append(rope_c(qkv[D:2 * D], t, hd, c.rope_theta))
            self.V[l].append(qkv[2 * D:])
            self.K[l], self.V[l] = self.K[l][-c.context:], self.V[l][-c.context:]
            o = attention(rope_c(qkv[:D], t, hd, c.rope_theta), np.array(self.K[l]), np.array(self.V[l]), c.n_heads)
            x = x + w[f"{p}.self_attn.out_projs.0.weight"] @ o
            x = gated(x, w[f"{p}.gating.linear_in.weight"], w[f"{p}.gating.linear_out.weight"], w[f"{p}.norm2.alpha"],
                      c.rms_eps)
        return emb, rmsn(x, w["out_norm.alpha"], c.rms_eps)

    def depformer(self, hid, prevs):
        """Logits of every codebook step; prevs[cb] is the token step cb conditions on."""
        c, w = self.c, self.w
        Dd = c.dep_d_model
        Ks = [[] for _ in range(c.dep_layers)]
        Vs = [[] for _ in range(c.dep_layers)]
        out = []
        for cb in range(c.dep_q):
            table = w["depformer_text_emb.weight"] if cb == 0 else w[f"depformer_emb.{cb - 1}.weight"]
            y = w[f"depformer_in.{cb}.weight"] @ hid + table[prevs[cb]]
            for j in range(c.dep_layers):
                p = f"depformer.layers.{j}"
                qkv = w[f"{p}.self_attn.in_projs.{cb}.weight"] @ rmsn(y, w[f"{p}.norm1.alpha"], c.rms_eps)
                Ks[j].append(qkv[Dd:2 * Dd])
                Vs[j].append(qkv[2 * Dd:])
                y = y + w[f"{p}.self_attn.out_projs.{cb}.weight"] @ attention(qkv[:Dd], np.array(Ks[j]), np.array(Vs[j]),
                                                                              c.dep_heads)
                y = gated(y, w[f"{p}.gating.{cb}.linear_in.weight"], w[f"{p}.gating.{cb}.linear_out.weight"],
                          w[f"{p}.norm2.alpha"], c.rms_eps)
            out.append(w[f"linears.{cb}.weight"] @ y)
        return np.array(out)

    def frame(self, t, user):
        """Step t (offset t before the step): returns inputs, emb_sum, hidden, text logits."""
        self.user[t] = list(user)
        toks = self.inputs(t)
        emb, hid = self.temporal(t, toks)
        return toks, emb, hid, self.w["text_linear.weight"] @ hid
