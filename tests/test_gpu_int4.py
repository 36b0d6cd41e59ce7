"""GPU parity of the 4-bit group-quantised path (lowbit_gemm_int4, pack_int4)
against the CPU oracle: packing bit-exact; the GEMM element by element within
the header's contract, |d| <= 1e-3 * sum|x w| + 1e-5 + 2^-19 (128 + max|z|)
sum|x s| (+ half an output ulp for 16-bit outputs).

The layout (zero points, group of 128) is this library's reading of "4-bit
HQQ": the pages name the format without defining it, so that part is parity
unpinned; the arithmetic w = s (q - z) is pinned by the oracle's tests."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import TORCH_DT, banner, dev_bits, to_host64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lb():
    import bit_weight_gemm_int2_amd as b
    b.lib()
    return b


def _f16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float16).view(np.int16)).cuda().view(torch.float16)


def _dev(lb, lin):
    q = torch.from_numpy(np.ascontiguousarray(lin.q)).cuda()
    return lb.pack_int4(q), _f16(lin.scales), _f16(lin.zeros)


def _extra(lin, x_bits=None) -> np.ndarray:
    """2^-19 (128 + max_g |z[n, g]|) sum_k |x[m, k] s[n, k/128]|: the rounding
    of the two FP32 sums the zero-point form subtracts."""
    xb = lin.x if x_bits is None else x_bits
    ax = np.abs(oracle.decode(xb, lin.x_dtype))
    s = np.repeat(np.abs(lin.scales.astype(np.float64)), oracle.GROUP, axis=1)
    zmax = np.abs(lin.zeros.astype(np.float64)).max(axis=1)
    return 2.0 ** -19 * (128.0 + zmax)[None, :] * (ax @ s.T)


def _assert_parity(Y, lin, what, rows=None, bias=True, act=None):
    xb = lin.x if rows is None else lin.x[rows]
    b = lin.bias if bias else None
    A = oracle.linear_int4(xb, lin.x_dtype, lin.q, lin.scales, lin.zeros, b)
    Mg = oracle.magnitude_int4(xb, lin.x_dtype, lin.q, lin.scales, lin.zeros, b)
    extra = _extra(lin, xb)
    if act == "gelu":
        # |GELU(a') - GELU(a)| <= 1.13 |a' - a|; the epilogue rounds once more
        A = oracle.gelu(A)
        Mg, extra = 1.13 * Mg, 1.13 * extra
    bnd = oracle.bound(A, Mg, lin.y_dtype, Y) + extra
    d = np.abs(Y - A)
    bad = ~(d <= bnd)
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside the bound, "
                           f"worst ratio {float(np.max(d / bnd)):.3g}")


def _run(lb, lin, bias=True, act=None, out=None):
    x = dev_bits(lin.x, lin.x_dtype)
    p, s, z = _dev(lb, lin)
    b = _f16(lin.bias) if bias and lin.bias is not None else None
    y = lb.gemm_int4(x, p, s, z, bias=b, out_dtype=TORCH_DT[lin.y_dtype], activation=act, out=out)
    torch.cuda.synchronize()
    return to_host64(y)


# ------------------------------------------------------------------ packing ---

def test_pack_int4_bit_exact(lb):
    banner("int4 pack 300x1024 + round trip")
    g = wl.generator(40)
    q = wl.int4_codes(g, 300, 1024)
    p = lb.pack_int4(torch.from_numpy(q).cuda())
    got = p.cpu().numpy()
    assert np.array_equal(got, oracle.pack_int4(q))
    codes, bad = lb.unpack("int4", p, 1024)
    assert bad == 0
    assert codes.dtype == torch.uint8 and np.array_equal(codes.cpu().numpy(), q)


def test_pack_int4_counts_out_of_range_codes(lb):
    banner("int4 pack with codes above 15")
    g = wl.generator(41)
    q = wl.int4_codes(g, 17, 64)
    q[3, 5], q[16, 63], q[0, 0] = 16, 255, 200
    p = lb.pack_int4(torch.from_numpy(q).cuda(), check=False)
    torch.cuda.synchronize()
    fixed = np.where(q > 15, 0, q).astype(np.uint8)
    assert np.array_equal(p.cpu().numpy(), oracle.pack_int4(fixed))
    with pytest.raises(ValueError):
        lb.pack_int4(torch.from_numpy(q).cuda(), check=True)


# --------------------------------------------------------------------- GEMM ---

# (M, N, K): several tiles and ragged tails on every side
SHAPES = [(1, 64, 256), (2, 200, 384), (7, 33, 128), (16, 520, 1024), (17, 130, 640), (64, 256, 256),
          (100, 96, 1152), (127, 300, 512), (128, 128, 2560), (129, 520, 256), (300, 264, 768),
          (600, 1000, 384)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_int4_shapes_bf16(lb, M, N, K):
    banner(f"int4 gemm bf16 {M}x{N}x{K}")
    lin = wl.make_int4_linear(f"i4_{M}x{N}x{K}", M, N, K, "bf16", seed=M * 7 + N + K, with_bias=(M % 2 == 1))
    _assert_parity(_run(lb, lin), lin, lin.name)


@pytest.mark.parametrize("variant", ["large-wide", "large-pair"])
@pytest.mark.parametrize("M,N,K", [(1, 64, 256), (17, 130, 640), (127, 300, 512), (129, 520, 256),
                                   (300, 2600, 768), (600, 1000, 384)])
def test_int4_each_tile_configuration(lb, variant, M, N, K):
    """Both tile configurations of the 4-bit kernel on every shape (forced):
    128-row tiles ("large-wide") and 64-row tiles, two workgroups per CU
    ("large-pair"); ragged rows and columns on both."""
    banner(f"int4 gemm {variant} {M}x{N}x{K}")
    lin = wl.make_int4_linear(f"i4v_{M}x{N}x{K}", M, N, K, "bf16", seed=M + 3 * N + K, with_bias=True)
    lb.force_variant(variant)
    try:
        Y = _run(lb, lin, act="gelu" if M % 2 else None)
    finally:
        lb.force_variant(None)
    _assert_parity(Y, lin, f"{lin.name} {variant}", act="gelu" if M % 2 else None)


@pytest.mark.parametrize("M,N,K,act", [(33, 300, 2048, None), (200, 520, 1280, "gelu"), (77, 1030, 4096, None),
                                       (1, 256, 1024, "gelu")])
def test_int4_k_split(lb, M, N, K, act):
    """The K split of the 64-row configuration (forced with "small-split": the
    largest split the groups allow, up to four): FP32 partial planes added in
    split order by the finishing kernel, then bias, activation and the cast."""
    banner(f"int4 gemm K split {M}x{N}x{K}")
    lin = wl.make_int4_linear(f"i4s_{M}x{N}x{K}", M, N, K, "bf16", seed=5 * M + N + K, with_bias=True)
    lb.force_variant("small-split")
    try:
        Y = _run(lb, lin, act=act)
        Y2 = _run(lb, lin, act=act)
    finally:
        lb.force_variant(None)
    assert np.array_equal(Y, Y2, equal_nan=True), "K-split result differs between two calls"
    _assert_parity(Y, lin, f"{lin.name} split", act=act)


@pytest.mark.parametrize("M,N,K,yd", [(5, 136, 512, "f16"), (96, 264, 1280, "f32"), (257, 72, 256, "f16"),
                                      (33, 4096, 2560, "bf16")])
def test_int4_f16_activations_and_outputs(lb, M, N, K, yd):
    banner(f"int4 gemm f16 in, {yd} out {M}x{N}x{K}")
    lin = wl.make_int4_linear(f"i4f_{M}x{N}x{K}", M, N, K, "f16", yd, seed=K + M, with_bias=True)
    _assert_parity(_run(lb, lin), lin, lin.name)


@pytest.mark.parametrize("xd", ["bf16", "f16"])
def test_int4_gelu_epilogue(lb, xd):
    banner(f"int4 gemm + GELU {xd}")
    lin = wl.make_int4_linear("i4_gelu", 70, 392, 640, xd, seed=9, with_bias=True, scale_std=0.03)
    _assert_parity(_run(lb, lin, act="gelu"), lin, "gelu", act="gelu")


def test_int4_degenerate_groups(lb):
    """Zero and subnormal scales, zero points at 0, 15, far outside the code
    range and fractional; all-zero and all-15 code groups."""
    banner("int4 gemm degenerate groups")
    lin = wl.make_int4_linear("i4_degen", 48, 160, 1024, "bf16", seed=11)
    lin.scales[0, :] = 0
    lin.scales[1, 3] = np.float16(6e-8)
    lin.scales[2, :] = np.float16(2.0 ** -20)
    lin.zeros[3, :] = 0
    lin.zeros[4, :] = 15
    lin.zeros[5, :] = np.float16(-37.25)
    lin.zeros[6, :] = np.float16(300.5)
    lin.zeros[7, :] = np.float16(0.001)
    lin.q[8, :] = 0
    lin.q[9, :] = 15
    lin.q[10, 128:256] = 7
    lin.zeros[10, 1] = 7          # a group whose weights are all exactly zero
    _assert_parity(_run(lb, lin), lin, "degenerate")


def test_int4_exact_case_is_bit_exact(lb):
    """Small integers everywhere: every product and partial sum is an integer
    below 2^24, so the FP32 result is exact and the output must match exactly."""
    banner("int4 gemm exact integers")
    g = wl.generator(12)
    M, N, K = 40, 96, 512
    x = wl.to_bits(g.integers(-3, 4, size=(M, K)).astype(np.float32), "bf16")
    lin = wl.Int4Linear("i4_exact", M, N, K, "bf16", "f32", x, wl.int4_codes(g, N, K),
                        np.ones((N, K // 128), np.float16), g.integers(0, 16, size=(N, K // 128)).astype(np.float16))
    Y = _run(lb, lin)
    A = oracle.linear_int4(lin.x, "bf16", lin.q, lin.scales, lin.zeros)
    assert np.array_equal(Y, A)


def test_int4_strided_x_and_output(lb):
    banner("int4 gemm strided X / Y")
    lin = wl.make_int4_linear("i4_strided", 37, 200, 512, "bf16", seed=13, with_bias=True)
    xfull = torch.zeros((37, 512 + 64), dtype=torch.bfloat16, device="cuda")
    xfull[:, :512] = dev_bits(lin.x, "bf16")
    yfull = torch.full((37, 200 + 24), 7.0, dtype=torch.bfloat16, device="cuda")
    p, s, z = _dev(lb, lin)
    lb.gemm_int4(xfull[:, :512], p, s, z, bias=_f16(lin.bias), out=yfull[:, :200])
    torch.cuda.synchronize()
    _assert_parity(to_host64(yfull[:, :200]), lin, "strided")
    assert bool((yfull[:, 200:] == 7.0).all())


def test_int4_workspace_reuse(lb):
    """One workspace for two calls of different M in a row; its prior contents
    never leak into a result."""
    banner("int4 gemm workspace reuse")
    big = wl.make_int4_linear("i4_ws_big", 260, 128, 768, "bf16", seed=14)
    small = wl.make_int4_linear("i4_ws_small", 9, 128, 768, "bf16", seed=15)
    ws = torch.full((lb.lib().lowbit_gemm_int4_workspace_bytes(260, 128, 768),), 0x7F, dtype=torch.uint8,
                    device="cuda")
    for lin in (big, small):
        p, s, z = _dev(lb, lin)
        y = lb.gemm_int4(dev_bits(lin.x, "bf16"), p, s, z, workspace=ws)
        torch.cuda.synchronize()
        _assert_parity(to_host64(y), lin, lin.name)


# ------------------------------------------------- text-encoder layer shapes ---

@pytest.mark.parametrize("name,N,K", wl.text_encoder_shapes() + [("qkv_fused", 6144, 2560), ("gate_up_fused", 19456, 2560)])
def test_int4_text_encoder_layer(lb, name, N, K):
    """The seven linears of one text-encoder layer at 512 prompt tokens, and
    the two same-input fusions (q|k|v, gate|up rows concatenated); the oracle
    checks 96 sampled rows (first and last included) of each."""
    banner(f"int4 text encoder {name} 512x{N}x{K}")
    lin = wl.make_int4_linear(f"te_{name}", wl.TE_TOKENS, N, K, "bf16", seed=N + K)
    Y = _run(lb, lin)
    rows = np.unique(np.concatenate([wl.generator(N).choice(lin.M, 94, replace=False), [0, lin.M - 1]]))
    sub = wl.Int4Linear(lin.name, len(rows), N, K, "bf16", "bf16", lin.x[rows], lin.q, lin.scales, lin.zeros)
    _assert_parity(Y[rows], sub, lin.name)
