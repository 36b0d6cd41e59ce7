"""lowbit_gemm_noalloc (the entry point for callers that cannot allocate)
against lowbit_gemm through the C ABI: the same result bits, on two calls in
a row, the second with a smaller input, on shapes whose plan needs the split-K
scratch (automatic and forced) and on one that needs none. The scratch is one
array per GPU that every call shares, so the second call also checks that the
first left its counters at zero."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import banner, dev_bits, dev_weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lb():
    import bit_weight_gemm_int2_amd as b
    b.lib()
    return b


def _operands(lb, fmt, M, N, K, seed):
    lin = wl.make_linear(f"na{seed}", fmt, M, N, K, seed=seed, p0=0.35, with_bias=True)
    x = dev_bits(lin.x, "bf16")
    p, s = dev_weights(fmt, lin.codes, lin.scales)
    b = torch.from_numpy(lin.bias.view(np.int16)).cuda().view(torch.float16)
    return x, p, s, b


def _noalloc(lb, fmt, x, p, s, b, y):
    M, K = x.shape
    N = p.shape[0]
    return lb.lib().lowbit_gemm_noalloc(
        lb._FMT[fmt], x.data_ptr(), lb.BF16, M, K, x.stride(0), p.data_ptr(), s.data_ptr(), 128, N,
        b.data_ptr(), lb.F16, y.data_ptr(), lb.BF16, y.stride(0), lb.ACT_GELU, torch.cuda.current_stream().cuda_stream)


def _gemm(lb, fmt, x, p, s, b, y):
    M, K = x.shape
    N = p.shape[0]
    need = lb.workspace_bytes(fmt, M, N, K)
    ws = lb.new_workspace(need) if need else None
    return lb.lib().lowbit_gemm(
        lb._FMT[fmt], x.data_ptr(), lb.BF16, M, K, x.stride(0), p.data_ptr(), s.data_ptr(), 128, N,
        b.data_ptr(), lb.F16, y.data_ptr(), lb.BF16, y.stride(0), lb.ACT_GELU,
        None if ws is None else ws.data_ptr(), 0 if ws is None else ws.numel(),
        torch.cuda.current_stream().cuda_stream), ws


# (variant, fmt, (M, N, K) of the first call, (M, N, K) of the second, smaller call)
CASES = [
    ("small-split", "ternary", (16, 3072, 9216), (5, 1024, 4096)),
    ("small-split", "binary", (16, 4096, 12288), (1, 640, 2048)),
    (None, "ternary", (16, 6144, 12288), (3, 2048, 9216)),
    (None, "ternary", (64, 1024, 1024), (16, 512, 512)),
]


@pytest.mark.parametrize("variant,fmt,first,second", CASES)
def test_noalloc_matches_lowbit_gemm(lb, variant, fmt, first, second):
    banner(f"noalloc {variant or 'auto'} {fmt} {first} then {second}")
    lb.force_variant(variant)
    try:
        for i, (M, N, K) in enumerate((first, second)):
            x, p, s, b = _operands(lb, fmt, M, N, K, seed=8800 + 10 * i + M)
            need = lb.workspace_bytes(fmt, M, N, K)
            assert need <= lb.lib().lowbit_gemm_workspace_bytes(lb._FMT[fmt], M, N, K) + 1
            y0 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
            y1 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
            st, ws = _gemm(lb, fmt, x, p, s, b, y0)
            assert st == lb.OK, lb.status_string(st)
            assert _noalloc(lb, fmt, x, p, s, b, y1) == lb.OK
            torch.cuda.synchronize()
            assert torch.equal(y0.view(torch.int16), y1.view(torch.int16)), f"call {i} ({M}x{N}x{K}) differs"
            if variant == "small-split" and i == 0:
                assert need > 0, "the forced split must use the scratch"
    finally:
        lb.force_variant(None)


def test_noalloc_refuses_what_lowbit_gemm_refuses(lb):
    banner("noalloc argument errors")
    x, p, s, b = _operands(lb, "ternary", 4, 256, 256, seed=8900)
    y = torch.empty((4, 256), dtype=torch.bfloat16, device="cuda")
    L = lb.lib()
    st = torch.cuda.current_stream().cuda_stream
    assert L.lowbit_gemm_noalloc(lb.TERNARY, x.data_ptr(), lb.BF16, 4, 256, 256, p.data_ptr(), s.data_ptr(), 64,
                                 256, None, lb.NONE, y.data_ptr(), lb.BF16, 256, 0, st) == lb.ERR_GROUP
    assert L.lowbit_gemm_noalloc(lb.TERNARY, x.data_ptr(), lb.BF16, 4, 256, 256, p.data_ptr(), s.data_ptr(), 128,
                                 256, None, lb.NONE, x.data_ptr(), lb.BF16, 256, 0, st) == lb.ERR_OVERLAP
