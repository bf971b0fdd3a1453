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
