"""Parity of the 100-linear transformer pass at its own size: the five
distinct linear shapes of the pass (hidden 3072, MLP x3; double-stream Q/K/V/
out 3072x3072, MLP-in 9216x3072, MLP-out 3072x9216; single-stream fused
QKV+MLP-in 18432x3072 and fused out+MLP-out 3072x12288) at M = 4608 tokens,
bf16 activations, ternary codes with P(0) = 0.35 (every matmul linear of the
model is ternary: "Como Bonsai Ternary 4B revoluciona la difusion
texto-imagen", sections "Representacion y almacenamiento de los pesos
ternarios" and "Arquitectura de despliegue y eficiencia en tiempo de
ejecucion"), plus the binary format on the longest-K shape. Each launch runs
the kernel configuration the automatic plan picks, the one the pass is timed
with; the two single-stream shapes also run the other large-M tile
configuration. The oracle checks a seeded sample of 256 rows (plus the first
and last) element by element."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import banner, dev_bits, dev_weights, to_host64

pytestmark = pytest.mark.gpu

M = 4608
SHAPES = [(3072, 3072), (9216, 3072), (3072, 9216), (18432, 3072), (3072, 12288)]


@pytest.fixture(scope="module")
def lb():
    import bit_weight_gemm_int2_amd as b
    b.lib()
    return b


@pytest.fixture(scope="module")
def acts():
    return wl.config5_activations(M)            # one bf16 X per distinct K, seed 10004


def _rows():
    r = np.sort(wl.generator(4608).choice(M, size=256, replace=False))
    return np.unique(np.concatenate([[0], r, [M - 1]]))


CASES = [("ternary", N, K, None) for N, K in SHAPES] + [
    ("binary", 3072, 12288, None),
    ("ternary", 18432, 3072, "large-wide"),      # the automatic plan takes pair tiles here
    ("ternary", 3072, 12288, "large-pair"),      # and wide tiles here
]


@pytest.mark.parametrize("fmt,N,K,variant", CASES)
def test_pass_shape_at_4608_tokens(lb, acts, fmt, N, K, variant):
    banner(f"M=4608 pass shape {fmt} {N}x{K} variant={variant or 'auto'}")
    seed = 4600 + SHAPES.index((N, K)) + (10 if fmt == "binary" else 0)
    g = wl.generator(seed)
    codes = wl.ternary_codes(g, N, K, 0.35) if fmt == "ternary" else wl.binary_codes(g, N, K)
    scales = wl.group_scales(g, N, K)
    xb = acts[K]
    x = dev_bits(xb, "bf16")
    packed, s = dev_weights(fmt, codes, scales)
    lb.force_variant(variant)
    try:
        y = lb.gemm(x, packed, s, fmt)
        torch.cuda.synchronize()
    finally:
        lb.force_variant(None)
    rows = _rows()
    Y = to_host64(y)[rows]
    A = oracle.linear(xb[rows], "bf16", codes, scales)
    Mg = oracle.magnitude(xb[rows], "bf16", codes, scales)
    ok, worst, nfail = oracle.check(Y, A, Mg, "bf16")
    assert ok, f"{fmt} {N}x{K}: {nfail} of {Y.size} sampled outputs outside the bound (worst ratio {worst:.3g})"
    assert np.isfinite(to_host64(y)).all()
