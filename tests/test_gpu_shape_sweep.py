"""Seeded sweep of random GEMM problems against the oracle: shapes drawn across
both the small-M (M <= 16) and the large-M paths, ragged N, K from one to a
hundred 128-groups, both formats, both activation types, all output types,
with and without bias and the fused GELU. The draw is fixed by its seed, so
every run checks the same cases."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import TORCH_DT, banner, dev_bits, dev_weights, oracle_linear, to_host64

pytestmark = pytest.mark.gpu


def _cases(seed=2024, count=40, max_work=2e9):
    g = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        small = len(out) % 2 == 0
        M = int(g.integers(1, 17)) if small else int(g.integers(17, 701))
        N = int(np.exp(g.uniform(0, np.log(20000))))
        K = 128 * int(g.integers(1, 101))
        if M * N * K > max_work:
            continue
        fmt = ("ternary", "binary")[len(out) % 4 // 2]
        xd = ("bf16", "f16")[int(g.integers(0, 2))]
        gelu = g.uniform() < 0.25
        yd = "f32" if gelu else ("bf16", "f16", "f32")[int(g.integers(0, 3))]
        bias = bool(g.uniform() < 0.5)
        out.append((len(out), M, N, K, fmt, xd, yd, bias, gelu))
    return out


@pytest.fixture(scope="module")
def lb():
    import bit_weight_gemm_int2_amd as b
    b.lib()
    return b


@pytest.mark.parametrize("i,M,N,K,fmt,xd,yd,bias,gelu", _cases())
def test_seeded_random_problem(lb, i, M, N, K, fmt, xd, yd, bias, gelu):
    banner(f"sweep case {i}: M={M} N={N} K={K} {fmt} {xd}->{yd} bias={bias} gelu={gelu}")
    lin = wl.make_linear(f"sweep{i}", fmt, M, N, K, x_dtype=xd, y_dtype=yd, seed=9000 + i,
                         p0=0.35, with_bias=bias)
    x = dev_bits(lin.x, xd)
    packed, s = dev_weights(fmt, lin.codes, lin.scales)
    b = torch.from_numpy(lin.bias.view(np.int16)).cuda().view(torch.float16) if bias else None
    y = lb.gemm(x, packed, s, fmt, bias=b, out_dtype=TORCH_DT[yd], activation="gelu" if gelu else None)
    torch.cuda.synchronize()
    Y = to_host64(y)
    A, Mg = oracle_linear(lin)
    if gelu:
        # GELU of the exact sum; its slope is below 1.13, so the sum's bound
        # carries through scaled by that, plus FP32 rounding of the GELU itself
        G = oracle.gelu(A)
        lim = 1.13 * (oracle.REL_TOL * Mg + oracle.ABS_TOL) + 4 * oracle.ulp(G, "f32")
        bad = np.abs(Y - G) > lim
        assert not bad.any(), f"case {i}: {bad.sum()} elements outside the GELU bound"
    else:
        ok, worst, nfail = oracle.check(Y, A, Mg, yd)
        assert ok, f"case {i}: {nfail} elements outside the bound, worst ratio {worst:.3g}"
