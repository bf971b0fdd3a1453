"""Python binding of the MI355X Moshi RQ-Transformer frame-step library (libmoshi_mi355x.so).

Argument marshalling only: every step of the frame runs in the library's HIP kernels.  The names
mirror the C ABI in include/moshi_mi355x.h.  There is no CPU fallback: if the library is not
built, importing the session class raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoshi_mi355x.so")

MOSHI_OK, MOSHI_NONE = 0, 1
MOSHI_EINVAL, MOSHI_ESTATE, MOSHI_ESHAPE, MOSHI_ENOMEM, MOSHI_EDEVICE, MOSHI_ERANGE = -1, -2, -3, -4, -5, -6
BANDS = {"f32": 0, "bf16": 1, "i8": 2, "q4": 3, "q8": 4}
EXEC = {"graph": 0, "stream": 1, "persistent": 2}
KV = {"f32": 0, "bf16": 1}
DTYPE_F32, DTYPE_BF16 = 0, 1

# every function the header declares, with (restype, argtypes)
_vp, _i32, _i64, _f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
_SIGS = {
    "moshi_create": (_i32, [_vp, _vp, _vp]),
    "moshi_load_weights": (_i32, [_vp, _vp, _i32]),
    "moshi_frame_step": (_i32, [_vp, _vp, _vp, _vp]),
    "moshi_reset": (_i32, [_vp, _i32]),
    "moshi_destroy": (None, [_vp]),
    "moshi_last_error": (ctypes.c_char_p, [_vp]),
    "moshi_status_string": (ctypes.c_char_p, [_i32]),
    "moshi_get_offset": (_i32, [_vp, _i32, _vp]),
    "moshi_force_generated": (_i32, [_vp, _i32, _i32, _vp]),
    "moshi_read_trace": (_i32, [_vp, _i32, _vp]),
    "moshi_prefill_forced": (_i32, [_vp, _i32, _i32, _vp, _vp, _vp]),
    "moshi_weight_bytes": (_i32, [_vp, _vp, _vp]),
    "moshi_stream": (_vp, [_vp]),
    "moshi_debug_gemv": (_i32, [_i32, _i32, _i32, _vp, _vp, _vp, _i32, _vp]),
    "moshi_debug_gemm": (_i32, [_i32, _i32, _i32, _i32, _vp, _vp, _vp, _i32, _vp]),
    "moshi_block_times": (_i32, [_vp, _vp, _i32, _vp]),
    "moshi_profile_frames": (_i32, [_vp, _i32, _vp, _vp, _vp]),
    "moshi_gpu_time": (_i32, [_vp, _i32, _vp, _vp]),
    "moshi_phase_times": (_i32, [_vp, _i32, _vp, _i32, _vp]),
    "moshi_set_spin_limit": (_i32, [_vp, _i32]),
    "moshi_debug_read_bw": (_i32, [_i64, _i32, _vp]),
    "moshi_snapshot_take": (_i32, [_vp, _i32, _vp]),
    "moshi_snapshot_restore": (_i32, [_vp, _i32, _vp]),
    "moshi_snapshot_info": (_i32, [_vp, _vp, _vp, _vp]),
    "moshi_snapshot_free": (None, [_vp]),
    "moshi_set_sampling": (_i32, [_vp, _i32, _vp]),
    "moshi_sampler_state": (_i32, [_vp, _i32, _vp]),
    "moshi_gemm_noalloc": (_i32, [_i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp]),
}

STAGES = ["embed", "qkv", "attn", "out_proj", "gate_in", "gate_out", "text_head", "dep_in", "dep_qkv", "dep_out",
          "dep_gate_in", "dep_gate_out", "dep_head", "frame_end"]


class MoshiError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with __graft_entry__.build() "
                              "(rq_transformer_frame_amd/build.py); there is no CPU fallback")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class _Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("n_layers", "d_model", "n_heads", "ffn_hidden", "context",
                                               "text_card", "audio_card", "dep_layers", "dep_d_model",
                                               "dep_heads", "dep_ffn_hidden", "dep_q")] + [
        ("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float)] + [
        (n, ctypes.c_int32) for n in ("band", "batch", "kv_capacity", "exec", "kv_dtype")]


class _Tensor(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 2), ("data", ctypes.c_void_p)]


class _Sampling(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("temp", ctypes.c_float), ("temp_text", ctypes.c_float),
                ("top_k", ctypes.c_int32), ("top_k_text", ctypes.c_int32), ("seed", ctypes.c_uint64)]


PICK = {"greedy": 0, "topk": 1, "gumbel": 2}


class _Trace(ctypes.Structure):
    _fields_ = [("input_tokens", ctypes.c_void_p), ("emb_sum", ctypes.c_void_p),
                ("transformer_out", ctypes.c_void_p), ("text_logits", ctypes.c_void_p),
                ("audio_logits", ctypes.c_void_p), ("tokens", ctypes.c_void_p)]


_SHAPE_FIELDS = ("n_layers", "d_model", "n_heads", "ffn_hidden", "context", "text_card", "audio_card",
                 "dep_layers", "dep_d_model", "dep_heads", "dep_ffn_hidden", "dep_q", "rope_theta", "rms_eps")


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


class Snapshot:
    """A moshi_snapshot (freed with free() or when collected)."""

    def __init__(self, lib, h):
        self.lib, self.h = lib, h

    def info(self):
        """(offset, cached positions, device bytes)."""
        o, n, b = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        self.lib.moshi_snapshot_info(self.h, ctypes.byref(o), ctypes.byref(n), ctypes.byref(b))
        return o.value, n.value, b.value

    def free(self):
        if getattr(self, "h", None):
            self.lib.moshi_snapshot_free(self.h)
            self.h = None

    def __del__(self):
        self.free()


class Session:
    """A moshi_state.  `shape` is any object with the moshi_config field names as attributes
    (n_layers, d_model, ...); band is 'f32', 'bf16' or 'i8'; kv is the KV cache storage, 'f32'
    (default) or 'bf16' (bf16 and i8 bands); exec is 'graph', 'stream' or 'persistent'; `stream`
    is an optional hipStream_t handle (int) to run on."""

    def __init__(self, shape, band: str | None = None, batch: int | None = None, kv_capacity: int = 0,
                 exec: str = "graph", stream: int | None = None, kv: str | None = None):
        self.lib = load_library()
        c = _Config()
        for f in _SHAPE_FIELDS:
            setattr(c, f, getattr(shape, f))
        c.band = BANDS[band or getattr(shape, "band")]
        c.batch = batch if batch is not None else getattr(shape, "batch", 1)
        c.kv_capacity = kv_capacity
        c.exec = EXEC[exec]
        c.kv_dtype = KV[kv or getattr(shape, "kv", "f32")]
        self.cfg = c
        self.B, self.Q = c.batch, c.dep_q
        self.NS = 2 * c.dep_q + 1
        h = ctypes.c_void_p()
        st = self.lib.moshi_create(ctypes.byref(c), stream, ctypes.byref(h))
        if st != MOSHI_OK:
            raise MoshiError(st, f"moshi_create failed: {self.lib.moshi_status_string(st).decode()}")
        self.h = h

    # -- helpers -----------------------------------------------------------------------------
    def _check(self, st: int, what: str) -> int:
        if st < 0:
            raise MoshiError(st, f"{what}: {self.lib.moshi_status_string(st).decode()}: "
                                 f"{self.lib.moshi_last_error(self.h).decode()}")
        return st

    def close(self):
        if getattr(self, "h", None):
            self.lib.moshi_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *a):
        self.close()

    # -- API ---------------------------------------------------------------------------------
    def load_weights(self, weights: dict, chunk: int = 64):
        """weights: name -> float32 array or uint16 array of bfloat16 bits."""
        items = list(weights.items())
        for i in range(0, len(items), chunk):
            part = items[i:i + chunk]
            arr = (_Tensor * len(part))()
            keep = []
            for j, (name, a) in enumerate(part):
                a = np.ascontiguousarray(a)
                if a.dtype == np.float32:
                    dt = DTYPE_F32
                elif a.dtype == np.uint16:
                    dt = DTYPE_BF16
                else:
                    raise TypeError(f"{name}: dtype {a.dtype} (want float32 or uint16 bf16 bits)")
                nb = name.encode()
                keep += [a, nb]
                arr[j].name = nb
                arr[j].dtype = dt
                arr[j].ndim = a.ndim
                arr[j].shape[0] = a.shape[0]
                arr[j].shape[1] = a.shape[1] if a.ndim > 1 else 0
                arr[j].data = _ptr(a)
            self._check(self.lib.moshi_load_weights(self.h, arr, len(part)), "moshi_load_weights")

    def step(self, user):
        """One frame.  user: [batch][dep_q] (or [dep_q] at batch 1).  Returns (status, out
        [batch][1+dep_q] int32, has_out [batch] bool)."""
        u = np.ascontiguousarray(np.asarray(user, np.int32).reshape(self.B, self.Q))
        out = np.full((self.B, self.Q + 1), -3, np.int32)
        has = np.zeros(self.B, np.uint8)
        st = self._check(self.lib.moshi_frame_step(self.h, _ptr(u), _ptr(out), _ptr(has)), "moshi_frame_step")
        return st, out, has.astype(bool)

    def reset(self, conv: int = -1):
        self._check(self.lib.moshi_reset(self.h, conv), "moshi_reset")

    def set_sampling(self, conv: int = -1, mode: str = "topk", seed: int = 0, temp: float = 0.8,
                     temp_text: float = 0.7, top_k: int = 250, top_k_text: int = 25):
        """moshi_set_sampling: 'greedy', 'topk' or 'gumbel' picks for conversation `conv` (-1: all)."""
        c = _Sampling(PICK[mode], temp, temp_text, top_k, top_k_text, seed)
        self._check(self.lib.moshi_set_sampling(self.h, conv, ctypes.byref(c)), "moshi_set_sampling")

    def sampler_state(self, conv: int = 0) -> int:
        v = ctypes.c_uint64()
        self._check(self.lib.moshi_sampler_state(self.h, conv, ctypes.byref(v)), "moshi_sampler_state")
        return v.value

    def snapshot(self, conv: int = 0) -> "Snapshot":
        """moshi_snapshot_take: a device copy of conversation `conv`'s ring, offset and KV."""
        h = ctypes.c_void_p()
        self._check(self.lib.moshi_snapshot_take(self.h, conv, ctypes.byref(h)), "moshi_snapshot_take")
        return Snapshot(self.lib, h)

    def restore(self, conv: int, snap: "Snapshot"):
        """moshi_snapshot_restore: conversation `conv` continues from `snap`."""
        self._check(self.lib.moshi_snapshot_restore(self.h, conv, snap.h), "moshi_snapshot_restore")

    def offset(self, conv: int = 0) -> int:
        v = ctypes.c_int64()
        self._check(self.lib.moshi_get_offset(self.h, conv, ctypes.byref(v)), "moshi_get_offset")
        return v.value

    def force_generated(self, conv: int, text: int, audio):
        a = np.ascontiguousarray(np.asarray(audio, np.int32))
        self._check(self.lib.moshi_force_generated(self.h, conv, int(text), _ptr(a)), "moshi_force_generated")

    def read_trace(self, conv: int = 0) -> dict:
        c = self.cfg
        t = dict(input_tokens=np.zeros(self.NS, np.int32), emb_sum=np.zeros(c.d_model, np.float32),
                 transformer_out=np.zeros(c.d_model, np.float32), text_logits=np.zeros(c.text_card, np.float32),
                 audio_logits=np.zeros((c.dep_q, c.audio_card), np.float32), tokens=np.zeros(1 + c.dep_q, np.int32))
        tr = _Trace(*[_ptr(t[k]) for k in ("input_tokens", "emb_sum", "transformer_out", "text_logits",
                                           "audio_logits", "tokens")])
        self._check(self.lib.moshi_read_trace(self.h, conv, ctypes.byref(tr)), "moshi_read_trace")
        t["text_token"] = int(t["tokens"][0])
        t["audio_tokens"] = [int(v) for v in t["tokens"][1:]]
        return t

    def prefill_forced(self, conv: int, text, agent, user):
        text = np.ascontiguousarray(np.asarray(text, np.int32))
        agent = np.ascontiguousarray(np.asarray(agent, np.int32))
        user = np.ascontiguousarray(np.asarray(user, np.int32))
        T = len(text)
        self._check(self.lib.moshi_prefill_forced(self.h, conv, T, _ptr(text), _ptr(agent), _ptr(user)),
                    "moshi_prefill_forced")

    def weight_bytes(self):
        a, b = ctypes.c_int64(), ctypes.c_int64()
        self._check(self.lib.moshi_weight_bytes(self.h, ctypes.byref(a), ctypes.byref(b)), "moshi_weight_bytes")
        return a.value, b.value

    def profile_frames(self, users):
        """Run len(users) real frames with every kernel launch timed by HIP events.  users:
        [frames][batch][dep_q].  Returns {stage: (launches, total_us)}."""
        u = np.ascontiguousarray(np.asarray(users, np.int32).reshape(-1, self.B, self.Q))
        us = np.zeros(len(STAGES), np.float64)
        n = np.zeros(len(STAGES), np.int64)
        self._check(self.lib.moshi_profile_frames(self.h, len(u), _ptr(u), _ptr(us), _ptr(n)), "moshi_profile_frames")
        return {name: (int(n[i]), float(us[i])) for i, name in enumerate(STAGES)}

    def gpu_time(self, enable: int = -1):
        """Totals of the per-frame HIP-event GPU time (us, frames) since the last clear; enable 1/0
        switches the timing on/off and clears, -1 only reads."""
        us, n = ctypes.c_double(), ctypes.c_int64()
        self._check(self.lib.moshi_gpu_time(self.h, enable, ctypes.byref(us), ctypes.byref(n)), "moshi_gpu_time")
        return us.value, n.value

    def phase_times(self, enable: int = -1):
        """Persistent executor: per-phase [block-0 arrival, completion] times (us) of the last
        frame; enable 1/0 switches the recording on/off, 2 also records every block's arrival
        (block_times)."""
        n = ctypes.c_int32()
        self._check(self.lib.moshi_phase_times(self.h, -1, None, 0, ctypes.byref(n)), "moshi_phase_times")
        ts = np.zeros((n.value, 2), np.float64)
        self._check(self.lib.moshi_phase_times(self.h, enable, _ptr(ts), n.value, ctypes.byref(n)),
                    "moshi_phase_times")
        return ts

    def set_spin_limit(self, spins: int):
        """Persistent executor: polls before a wait of the frame kernel gives up (test hook)."""
        self._check(self.lib.moshi_set_spin_limit(self.h, int(spins)), "moshi_set_spin_limit")

    def block_times(self):
        """Persistent executor, after phase_times(2): every block's arrival time (us) at every
        phase of the last frame, [phases][blocks]."""
        n = ctypes.c_int32()
        self._check(self.lib.moshi_phase_times(self.h, -1, None, 0, ctypes.byref(n)), "moshi_phase_times")
        nb = ctypes.c_int32()
        self._check(self.lib.moshi_block_times(self.h, None, 0, ctypes.byref(nb)), "moshi_block_times")
        ts = np.zeros((n.value, nb.value), np.float64)
        self._check(self.lib.moshi_block_times(self.h, _ptr(ts), ts.size, ctypes.byref(nb)), "moshi_block_times")
        return ts

    @property
    def stream(self) -> int:
        return self.lib.moshi_stream(self.h)


def debug_gemv(band: str, W: np.ndarray, x: np.ndarray, iters: int = 0):
    """y = W . x with the library's GEMV kernel (W float32 [N, K], converted per band).  Returns
    (y, mean kernel microseconds or None)."""
    lib = load_library()
    W = np.ascontiguousarray(W, np.float32)
    x = np.ascontiguousarray(x, np.float32)
    N, K = W.shape
    y = np.zeros(N, np.float32)
    us = ctypes.c_float(0)
    st = lib.moshi_debug_gemv(BANDS[band], N, K, _ptr(W), _ptr(x), _ptr(y), iters, ctypes.byref(us))
    if st != MOSHI_OK:
        raise MoshiError(st, f"moshi_debug_gemv: {lib.moshi_status_string(st).decode()}")
    return y, (us.value if iters > 0 else None)


def debug_gemm(band: str, W: np.ndarray, X: np.ndarray, iters: int = 0):
    """Y = X . W^T with the library's matrix-core projection (W float32 [N, K] stored per band, X
    float32 [M, K], rounded to bf16 for the bf16 and int8 bands).  Returns (Y, mean kernel
    microseconds or None)."""
    lib = load_library()
    W = np.ascontiguousarray(W, np.float32)
    X = np.ascontiguousarray(X, np.float32)
    N, K = W.shape
    M, K2 = X.shape
    if K2 != K:
        raise ValueError("X and W disagree on K")
    Y = np.zeros((M, N), np.float32)
    us = ctypes.c_float(0)
    st = lib.moshi_debug_gemm(BANDS[band], M, N, K, _ptr(W), _ptr(X), _ptr(Y), iters, ctypes.byref(us))
    if st != MOSHI_OK:
        raise MoshiError(st, f"moshi_debug_gemm: {lib.moshi_status_string(st).decode()}")
    return Y, (us.value if iters > 0 else None)


def debug_read_bw(nbytes: int = 1 << 30, iters: int = 20) -> float:
    """Streaming-read rate of the device in GB/s (moshi_debug_read_bw)."""
    lib = load_library()
    g = ctypes.c_double(0)
    st = lib.moshi_debug_read_bw(int(nbytes), int(iters), ctypes.byref(g))
    if st != MOSHI_OK:
        raise MoshiError(st, f"moshi_debug_read_bw: {lib.moshi_status_string(st).decode()}")
    return g.value


def gemm_noalloc(band: str, M: int, N: int, K: int, W_ptr: int, scale_ptr, X_ptr: int, Y_ptr: int, stream=None) -> int:
    """moshi_gemm_noalloc on device pointers (ints); enqueues only.  Returns the status."""
    lib = load_library()
    return lib.moshi_gemm_noalloc(BANDS[band], M, N, K, W_ptr, scale_ptr, X_ptr, Y_ptr, stream)
