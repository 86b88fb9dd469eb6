"""GPU: the allocation-free W8A16 entry point (nomas_w8a16_linear_noalloc)
against the workspace entry point (nomas_w8a16_linear), through the C ABI.

Both run the same kernels, so their outputs must agree bit for bit.  Two calls
in a row share the library's static scratch; the second, with a smaller
input, must not see anything of the first.  Runs alone in a fresh process and
after the other tests."""
import ctypes

import numpy as np
import pytest
import torch

import segment_causal_attention_amd as nomas
from gpu_util import dev, dev16, say

pytestmark = pytest.mark.gpu


def _inputs(M, K, N, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((M, K), dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    codes = rng.integers(-127, 128, size=(N, K), dtype=np.int8)
    scale = (rng.random(N, dtype=np.float32) * 0.02 + 1e-3).astype(np.float32)
    return dev16(x), dev(codes), dev(scale)


def _noalloc(x, codes, scale, M, K, N):
    L = nomas.lib()
    y = torch.full((M, N), 0x7FC0, dtype=torch.int16, device="cuda:0")      # NaN bits, must be overwritten
    P = ctypes.c_void_p
    rc = L.nomas_w8a16_linear_noalloc(P(x.data_ptr()), M, K, P(codes.data_ptr()), P(scale.data_ptr()), N,
                                      P(y.data_ptr()), P(torch.cuda.current_stream().cuda_stream))
    assert rc == nomas.OK, nomas.strerror(rc)
    return y


def _with_workspace(x, codes, scale, M, K, N):
    L = nomas.lib()
    y = torch.empty((M, N), dtype=torch.int16, device="cuda:0")
    ws = torch.empty(L.nomas_w8a16_linear_workspace(K, N), dtype=torch.uint8, device="cuda:0")
    P = ctypes.c_void_p
    rc = L.nomas_w8a16_linear(P(x.data_ptr()), M, K, P(codes.data_ptr()), P(scale.data_ptr()), N, P(y.data_ptr()),
                              P(ws.data_ptr()), ws.numel(), P(torch.cuda.current_stream().cuda_stream))
    assert rc == nomas.OK, nomas.strerror(rc)
    return y


def test_w8a16_noalloc_matches_workspace_entry_point():
    # first call at the scratch's limit (2048 -> 8192: 32 MiB of bf16 weights), then a smaller one
    for M, K, N, seed in ((1000, 2048, 8192, 1), (300, 1024, 2048, 2)):
        say("w8a16 noalloc M %d K %d N %d" % (M, K, N))
        x, codes, scale = _inputs(M, K, N, seed)
        got = _noalloc(x, codes, scale, M, K, N)
        torch.cuda.synchronize()
        ref = _with_workspace(x, codes, scale, M, K, N)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), "noalloc output differs from the workspace entry point"
        assert not torch.isnan(got.view(torch.bfloat16)).any()
    # the scratch keeps the last call's contents; a call with M = 0 only dequantises
    x, codes, scale = _inputs(1, 64, 256, 3)
    y = torch.empty((0, 256), dtype=torch.int16, device="cuda:0")
    L = nomas.lib()
    P = ctypes.c_void_p
    assert L.nomas_w8a16_linear_noalloc(None, 0, 64, P(codes.data_ptr()), P(scale.data_ptr()), 256, None,
                                        P(torch.cuda.current_stream().cuda_stream)) == nomas.OK
    torch.cuda.synchronize()
