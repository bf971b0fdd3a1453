"""Helpers shared by the GPU parity tests (comparison metrics, oracle runs)."""
import numpy as np


def rel_err(g, o):
    """max_i |g_i - o_i| / max_i |o_i| over one row."""
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    return float(np.max(np.abs(g - o)) / max(np.max(np.abs(o)), 1e-30))


def cosine(g, o):
    g = np.asarray(g, np.float64).ravel()
    o = np.asarray(o, np.float64).ravel()
    return float(g @ o / max(np.linalg.norm(g) * np.linalg.norm(o), 1e-300))


def top2_margin(v):
    s = np.sort(np.asarray(v, np.float64))
    return float(s[-1] - s[-2])


def frame_agreement(tr, ref):
    """Per-frame comparison for the low-precision bands: the cosine of every logits vector whose
    conditioning agrees (the text head always; the head of codebook c only while the text token and
    codebooks < c picked the oracle's tokens, since within a frame each depformer step feeds on the
    previous step's own token), and the token matches."""
    got = [tr["text_token"]] + tr["audio_tokens"]
    want = [ref["text_token"]] + ref["audio_tokens"]
    cos = [cosine(tr["text_logits"], ref["text_logits"])]
    for c in range(len(want) - 1):
        if got[: c + 1] != want[: c + 1]:
            break
        cos.append(cosine(tr["audio_logits"][c], ref["audio_logits"][c]))
    return min(cos), sum(int(a == b) for a, b in zip(got, want))


class TraceStats:
    """Running comparison of a GPU trace against a reference, frame by frame, under the judging
    rule of frame_agreement: the text logits always, a codebook's logits while the tokens before it
    agree.  Keeps the minimum cosine, the largest relative error (max |g - o| / max |o| per row)
    and the token agreement."""

    def __init__(self, tie_tol: float = 0.0):
        self.cos_min, self.rel_max, self.agree, self.total, self.frames = 1.0, 0.0, 0, 0, 0
        self.tie_tol = tie_tol
        self.unexplained = 0  # differing tokens that are not near-ties of the reference's logits

    def add(self, tr, ref):
        got = [tr["text_token"]] + tr["audio_tokens"]
        want = [ref["text_token"]] + ref["audio_tokens"]
        rows = [(tr["text_logits"], ref["text_logits"])]
        for c in range(len(want) - 1):
            if got[: c + 1] != want[: c + 1]:
                break
            rows.append((tr["audio_logits"][c], ref["audio_logits"][c]))
        for i, (g, o) in enumerate(rows):
            self.cos_min = min(self.cos_min, cosine(g, o))
            self.rel_max = max(self.rel_max, rel_err(g, o))
            # a differing pick on an agreeing conditioning: is it a near-tie of the reference?
            if got[i] != want[i]:
                o64 = np.asarray(o, np.float64)
                margin = (o64[want[i]] - o64[got[i]]) / max(np.max(np.abs(o64)), 1e-30)
                self.unexplained += int(not (margin <= self.tie_tol))
        a = sum(int(x == y) for x, y in zip(got, want))
        self.agree += a
        self.total += len(got)
        self.frames += 1
        return a

    @property
    def rate(self):
        return self.agree / max(self.total, 1)

    def __str__(self):
        return (f"{self.frames} frames: min cosine {self.cos_min:.6f}, max rel logit err {self.rel_max:.2e}, "
                f"tokens {self.agree}/{self.total}, differing picks that are not near-ties {self.unexplained}")
