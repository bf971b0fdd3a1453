"""moshi_gemm_noalloc (the projection that allocates nothing, for callers that cannot allocate)
against the entry point it varies, moshi_debug_gemm, through the C ABI: calls in a row, the second
with a smaller input and the third with more than one 64-row activation tile, for every band.  Device buffers come from torch (plumbing only)."""
import ctypes

import numpy as np
import pytest

import rq_transformer_frame_amd as rq
import synth
from oracle import moshi_oracle as O

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def device_weights(band, W):
    """The band's storage of W on the device: float32, bf16 (round to nearest even) or int8 with
    per-row scales (the quantiser of moshi_load_weights)."""
    if band == "f32":
        return torch.from_numpy(W).cuda(), None
    if band == "bf16":
        return torch.from_numpy(W).cuda().to(torch.bfloat16), None
    q, s = O.quantize_rows_int8(W)
    return torch.from_numpy(q).cuda(), torch.from_numpy(s).cuda()


@pytest.mark.parametrize("band", ["bf16", "i8", "f32"])
def test_noalloc_gemm_matches_debug_gemm_on_two_calls(band):
    lib = rq.load_library()
    stream = torch.cuda.current_stream().cuda_stream
    for call, (M, N, K) in enumerate([(64, 4096, 4096), (5, 1000, 352), (200, 1000, 1040)]):
        W = synth.normal(21 + call, "noalloc/w", (N, K), 0.02)
        X = synth.normal(21 + call, "noalloc/x", (M, K), 1.0)
        ref, _ = rq.debug_gemm(band, W, X)
        dW, dS = device_weights(band, W)
        dX = torch.from_numpy(X).cuda()
        dY = torch.full((M, N), float("nan"), device="cuda")
        torch.cuda.synchronize()
        st = lib.moshi_gemm_noalloc(rq.BANDS[band], M, N, K, dW.data_ptr(), None if dS is None else dS.data_ptr(),
                                    dX.data_ptr(), dY.data_ptr(), ctypes.c_void_p(stream))
        assert st == rq.MOSHI_OK
        torch.cuda.synchronize()
        Y = dY.cpu().numpy()
        assert np.isfinite(Y).all(), call
        err = float(np.max(np.abs(Y - ref)) / np.max(np.abs(ref)))
        print(f"{band} call {call} M={M} N={N} K={K}: max rel diff vs moshi_debug_gemm {err:.2e}")
        assert err <= 1e-5, (call, err)


def test_noalloc_gemm_rejects_sizes_beyond_its_scratch():
    lib = rq.load_library()
    dW = torch.zeros((16, 16384), dtype=torch.bfloat16, device="cuda")
    dX = torch.zeros((256, 16384), device="cuda")
    dY = torch.zeros((256, 16), device="cuda")
    assert lib.moshi_gemm_noalloc(rq.BANDS["bf16"], 257, 16, 16384, dW.data_ptr(), None, dX.data_ptr(),
                                  dY.data_ptr(), None) == rq.MOSHI_EINVAL
    assert lib.moshi_gemm_noalloc(rq.BANDS["bf16"], 256, 16, 16384, dW.data_ptr(), None, dX.data_ptr(),
                                  dY.data_ptr(), None) == rq.MOSHI_OK  # 4 M K = 16 MiB: the limit
    torch.cuda.synchronize()
    assert lib.moshi_gemm_noalloc(rq.BANDS["i8"], 4, 16, 64, dW.data_ptr(), None, dX.data_ptr(),
                                  dY.data_ptr(), None) == rq.MOSHI_EINVAL  # int8 needs its scales
