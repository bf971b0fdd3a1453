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
