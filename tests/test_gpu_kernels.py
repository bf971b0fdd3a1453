"""Kernel-level parity of the weight-streaming GEMV (float32, bfloat16 and int8 bands) against
float64 products of the same stored weights, at ragged small shapes and at the Moshi-7B
projection shapes (sampled rows)."""
import numpy as np
import pytest

import rq_transformer_frame_amd as rq
import synth
from oracle import quantize_rows_int8
from oracle.moshi_oracle import dequantize_blocks, quantize_blocks

pytestmark = pytest.mark.gpu


def stored(band, W):
    """The weights as the band stores them, widened to float64 (and the int8 scales)."""
    if band == "f32":
        return W.astype(np.float64), None
    if band == "bf16":
        return synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(W)).astype(np.float64), None
    if band in ("q4", "q8"):
        return dequantize_blocks(*quantize_blocks(W, 4 if band == "q4" else 8)).astype(np.float64), None
    q, s = quantize_rows_int8(W)
    return q.astype(np.float64), s.astype(np.float64)


BYTES_PER_WEIGHT = {"bf16": 2.0, "i8": 1.0, "q4": 0.5 + 4 / 32, "q8": 1.0 + 4 / 32}


@pytest.mark.parametrize("band", ["f32", "bf16", "i8", "q4", "q8"])
@pytest.mark.parametrize("N,K", [(1, 32), (37, 64), (130, 288), (1000, 256), (2048, 1024), (333, 2816)])
def test_gemv_small_and_ragged(band, N, K):
    W = synth.normal(1, f"k/W{N}x{K}", (N, K), 0.02)
    x = synth.normal(1, f"k/x{K}", (K,), 1.0)
    y, _ = rq.debug_gemv(band, W, x)
    Ws, s = stored(band, W)
    ref = Ws @ x.astype(np.float64)
    if s is not None:
        ref *= s
    err = np.max(np.abs(y - ref)) / np.max(np.abs(ref))
    assert err < 2e-6, err


@pytest.mark.parametrize("band", ["bf16", "i8", "q4", "q8"])
@pytest.mark.parametrize("N,K", [(12288, 4096), (22528, 4096), (4096, 11264), (32000, 4096), (8192, 4096)])
def test_gemv_moshi7b_shapes_sampled_rows(band, N, K):
    W = synth.normal(2, f"k7/W{N}x{K}", (N, K), 0.02)
    x = synth.normal(2, f"k7/x{K}", (K,), 1.0)
    y, us = rq.debug_gemv(band, W, x, iters=10)
    rows = np.unique(synth.uniform_int(2, f"k7/rows{N}", (256,), N))
    rows = np.concatenate([[0, N - 1], rows])
    Ws, s = stored(band, W[rows])
    ref = Ws @ x.astype(np.float64)
    if s is not None:
        ref *= s
    err = np.max(np.abs(y[rows] - ref)) / np.max(np.abs(ref))
    bytes_ = N * K * BYTES_PER_WEIGHT[band] + (N * 4 if band == "i8" else 0)
    print(f"gemv {band} {N}x{K}: {us:.1f} us, {bytes_ / us / 1e3:.0f} GB/s")
    assert err < 2e-6, err


def rounded_x(band, X):
    """The activations as the matrix-core path feeds them: float32 values, split for the bf16 and
    int8 bands into bf16 hi and lo parts whose sum keeps about 16 significant bits."""
    X = X.astype(np.float64)
    if band == "f32":
        return X
    hi = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(X.astype(np.float32))).astype(np.float64)
    lo = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits((X - hi).astype(np.float32))).astype(np.float64)
    return hi + lo


@pytest.mark.parametrize("band", ["f32", "bf16", "i8"])
@pytest.mark.parametrize("M,N,K", [(1, 1, 16), (2, 37, 48), (5, 64, 352), (64, 96, 256), (70, 1000, 704),
                                   (3, 130, 1040), (64, 2048, 1024), (200, 300, 48), (257, 520, 1040),
                                   (129, 257, 4112), (513, 300, 64), (700, 520, 1040)])
def test_gemm_small_and_ragged(band, M, N, K):
    W = synth.normal(3, f"g/W{N}x{K}", (N, K), 0.02)
    X = synth.normal(3, f"g/X{M}x{K}", (M, K), 1.0)
    Y, _ = rq.debug_gemm(band, W, X)
    Ws, s = stored(band, W)
    ref = rounded_x(band, X) @ Ws.T
    if s is not None:
        ref *= s[None, :]
    err = np.max(np.abs(Y - ref)) / np.max(np.abs(ref))
    assert err < 1e-5, err


@pytest.mark.parametrize("band", ["bf16", "i8"])
@pytest.mark.parametrize("N,K", [(12288, 4096), (4096, 4096), (22528, 4096), (4096, 11264)])
def test_gemm_moshi7b_shapes_prefill_chunk(band, N, K):
    """The prefill's 1024-row chunks (256 x 256 tiles, K split where the tiles alone do not cover
    the CUs), checked on sampled output columns and every row."""
    M = 1024
    W = synth.normal(5, f"g8/W{N}x{K}", (N, K), 0.02)
    X = synth.normal(5, f"g8/X{K}", (M, K), 1.0)
    Y, us = rq.debug_gemm(band, W, X, iters=5)
    rows = np.unique(synth.uniform_int(5, f"g8/rows{N}", (96,), N))
    rows = np.concatenate([[0, N - 1], rows])
    Ws, s = stored(band, W[rows])
    ref = rounded_x(band, X) @ Ws.T
    if s is not None:
        ref *= s[None, :]
    err = np.max(np.abs(Y[:, rows] - ref)) / np.max(np.abs(ref))
    print(f"gemm M=1024 {band} {N}x{K}: {us:.1f} us, {2 * M * N * K / us / 1e6:.1f} TFLOP/s "
          f"({4 * M * N * K / us / 1e6:.1f} issued)")
    assert err < 1e-5, err


@pytest.mark.parametrize("band", ["bf16", "i8"])
@pytest.mark.parametrize("N,K", [(12288, 4096), (4096, 4096), (22528, 4096), (4096, 11264), (32000, 4096)])
def test_gemm_moshi7b_shapes_batch64(band, N, K):
    M = 64
    W = synth.normal(4, f"g7/W{N}x{K}", (N, K), 0.02)
    X = synth.normal(4, f"g7/X{K}", (M, K), 1.0)
    Y, us = rq.debug_gemm(band, W, X, iters=10)
    rows = np.unique(synth.uniform_int(4, f"g7/rows{N}", (128,), N))
    rows = np.concatenate([[0, N - 1], rows])
    Ws, s = stored(band, W[rows])
    ref = rounded_x(band, X) @ Ws.T
    if s is not None:
        ref *= s[None, :]
    err = np.max(np.abs(Y[:, rows] - ref)) / np.max(np.abs(ref))
    bytes_ = N * K * (2 if band == "bf16" else 1) + (N * 4 if band == "i8" else 0)
    print(f"gemm M=64 {band} {N}x{K}: {us:.1f} us, {bytes_ / us / 1e3:.0f} GB/s weights, "
          f"{2 * M * N * K / us / 1e6:.1f} TFLOP/s")
    assert err < 1e-5, err
