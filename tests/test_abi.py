"""The C-ABI library loads and exports every symbol its header declares; host-side argument
checks that run before any device work (no GPU needed)."""
import ctypes
import os
import re

import pytest

import rq_transformer_frame_amd as rq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h")]


def declared_functions():
    names = []
    for h in HEADERS:
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*(moshi_[a-z_0-9]+)\s*\(", src, re.M)
    return sorted(set(names))


def test_header_declares_the_boundary_calls():
    names = declared_functions()
    for must in ("moshi_create", "moshi_load_weights", "moshi_frame_step", "moshi_reset"):
        assert must in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(rq.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_covers_every_declared_symbol():
    assert set(declared_functions()) <= set(rq._SIGS)


def test_status_strings():
    lib = rq.load_library()
    assert lib.moshi_status_string(0) == b"MOSHI_OK"
    assert lib.moshi_status_string(-6) == b"MOSHI_ERANGE"


def _cfg(**kw):
    c = rq._Config()
    base = dict(n_layers=2, d_model=256, n_heads=4, ffn_hidden=704, context=64, text_card=1000, audio_card=2048,
                dep_layers=2, dep_d_model=128, dep_heads=2, dep_ffn_hidden=352, dep_q=8, rope_theta=1e4,
                rms_eps=1e-8, band=0, batch=1, kv_capacity=0, exec=0)
    base.update(kw)
    for k, v in base.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("bad", [
    dict(n_heads=3), dict(d_model=512, n_heads=2), dict(ffn_hidden=700), dict(dep_q=17), dict(batch=0),
    dict(kv_capacity=65), dict(band=5), dict(exec=3), dict(context=0), dict(dep_heads=3),
    dict(kv_dtype=2), dict(band=0, kv_dtype=1),
    dict(band=3, batch=2), dict(band=4, ffn_hidden=720),  # block bands: batch 1, widths multiples of 32
])
def test_create_rejects_bad_configs_before_touching_the_device(bad):
    lib = rq.load_library()
    h = ctypes.c_void_p(123)
    st = lib.moshi_create(ctypes.byref(_cfg(**bad)), None, ctypes.byref(h))
    assert st == rq.MOSHI_EINVAL and not h.value


def test_null_arguments_are_rejected():
    lib = rq.load_library()
    assert lib.moshi_create(None, None, None) == rq.MOSHI_EINVAL
    assert lib.moshi_frame_step(None, None, None, None) == rq.MOSHI_EINVAL
    assert lib.moshi_reset(None, -1) == rq.MOSHI_EINVAL
    lib.moshi_destroy(None)


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="a GPU driver is present")
def test_create_without_a_gpu_reports_a_device_error():
    lib = rq.load_library()
    h = ctypes.c_void_p()
    assert lib.moshi_create(ctypes.byref(_cfg()), None, ctypes.byref(h)) == rq.MOSHI_EDEVICE
    assert not h.value
