"""GPU GEMM parity against the CPU oracle, element by element, within the stated
tolerance |d| <= 1e-3 * sum_k |x_k w_k| + 1e-5 (+ half an output ulp for
16-bit outputs); bit-exact where every partial sum is exact in FP32."""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import TORCH_DT, banner, dev_bits, dev_weights, oracle_linear, run_linear, to_host64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lb():
    import bit_weight_gemm_int2_amd as b
    b.lib()
    return b


def _assert_parity(Y, A, Mg, y_dtype, what):
    ok, worst, nfail = oracle.check(Y, A, Mg, y_dtype)
    assert ok, f"{what}: {nfail} elements outside the bound, worst ratio {worst:.3g}"
    return worst


@pytest.fixture
def force_variant(lb):
    yield lb.force_variant
    lb.force_variant(None)


# ------------------------------------------------------------- workloads ---

def test_config1_ternary_f16(lb):
    banner("gemm config1 64x256x256 f16")
    lin = wl.config1()
    Y, _ = run_linear(lin)
    A, Mg = oracle_linear(lin)
    _assert_parity(Y, A, Mg, "f16", "config1")


def test_config2_ternary_bf16_bias(lb):
    banner("gemm config2 1536x3072x3072 bf16 + bias")
    lin = wl.config2()
    Y, _ = run_linear(lin)
    A, Mg = oracle_linear(lin)
    _assert_parity(Y, A, Mg, "bf16", "config2")


@pytest.mark.parametrize("M", [1536, 16, 1])
def test_config4_binary(lb, M):
    banner(f"gemm config4 binary M={M}")
    for lin in wl.config4(M):
        Y, _ = run_linear(lin)
        A, Mg = oracle_linear(lin)
        _assert_parity(Y, A, Mg, "bf16", lin.name)


def test_config3_mlp_pair(lb):
    """Up-proj with fused GELU, the standalone GELU kernel, and the down-proj fed
    with the oracle's own bf16 GELU output; rows sampled for the oracle."""
    banner("gemm config3 MLP pair 4608x9216x3072 / 4608x3072x9216")
    up, down = wl.config3()
    rows = np.sort(wl.generator(77).choice(up.M, 384, replace=False))
    rows = np.concatenate([rows, [0, up.M - 1]])
    x = dev_bits(up.x, "bf16")
    pu, su = dev_weights("ternary", up.codes, up.scales)
    pre = lb.gemm(x, pu, su, "ternary")                       # bf16, no activation
    h_fused = lb.gemm(x, pu, su, "ternary", activation="gelu")
    h_split = lb.gelu(pre)
    torch.cuda.synchronize()
    A, Mg = oracle.linear(up.x[rows], "bf16", up.codes, up.scales), None
    Mg = oracle.magnitude(up.x[rows], "bf16", up.codes, up.scales)
    _assert_parity(to_host64(pre)[rows], A, Mg, "bf16", "up")
    # GELU: |GELU(a') - GELU(a)| <= max|GELU'| * |a' - a|, max|GELU'| < 1.13
    G = oracle.gelu(A)
    for name, h in (("fused", h_fused), ("split", h_split)):
        H = to_host64(h)[rows]
        lim = 1.13 * (oracle.REL_TOL * Mg + oracle.ABS_TOL) + 0.5 * oracle.ulp(np.maximum(abs(G), abs(H)), "bf16") \
            + 4 * oracle.ulp(G, "f32")
        if name == "split":   # GELU of the bf16-rounded pre-activation: one more bf16 half ulp inside
            lim = lim + 1.13 * 0.5 * oracle.ulp(A, "bf16")
        bad = np.abs(H - G) > lim
        assert not bad.any(), f"GELU {name}: {bad.sum()} elements out of bound"
    # down-proj on the oracle's bf16 GELU output (all rows of H from the oracle)
    Hb = oracle.encode(oracle.gelu(oracle.linear(up.x, "bf16", up.codes, up.scales)), "bf16")
    Yd = lb.gemm(dev_bits(Hb, "bf16"), *dev_weights("ternary", down.codes, down.scales), "ternary")
    torch.cuda.synchronize()
    A2 = oracle.linear(Hb[rows], "bf16", down.codes, down.scales)
    Mg2 = oracle.magnitude(Hb[rows], "bf16", down.codes, down.scales)
    _assert_parity(to_host64(Yd)[rows], A2, Mg2, "bf16", "down")


# --------------------------------------------------------- random shapes ---

_SHAPES = [(1, 1, 128), (5, 15, 256), (16, 64, 384), (17, 130, 128), (100, 300, 1024),
           (130, 129, 256), (257, 64, 512), (64, 513, 640), (33, 1000, 2048)]


@pytest.mark.parametrize("i,shape", list(enumerate(_SHAPES)))
@pytest.mark.parametrize("fmt", ["ternary", "binary"])
def test_random_shapes(lb, i, shape, fmt):
    M, N, K = shape
    xd = ("bf16", "f16")[i % 2]
    yd = ("bf16", "f16", "f32")[i % 3]
    with_bias = i % 2 == 1
    lin = wl.make_linear(f"rand{i}", fmt, M, N, K, x_dtype=xd, y_dtype=yd, seed=100 + i,
                         p0=0.35, with_bias=with_bias)
    Y, _ = run_linear(lin)
    A, Mg = oracle_linear(lin)
    _assert_parity(Y, A, Mg, yd, f"{fmt} {shape} {xd}->{yd}")


# ------------------------------------------------------------ exact cases ---

@pytest.mark.parametrize("fmt", ["ternary", "binary"])
@pytest.mark.parametrize("M", [3, 16, 200])
def test_exact_arithmetic_is_bit_exact(lb, fmt, M):
    """Small integer activations and power-of-two scales: every partial sum is an
    exactly representable FP32 value, so any summation order gives the oracle's
    value bit for bit."""
    g = wl.generator(300 + M)
    N, K = 96, 256
    x = g.integers(-8, 9, size=(M, K)).astype(np.float32)
    t = wl.ternary_codes(g, N, K, 0.35) if fmt == "ternary" else wl.binary_codes(g, N, K)
    s = (2.0 ** g.integers(-6, 3, size=(N, K // 128))).astype(np.float16)
    for xd in ("bf16", "f16"):
        lin = wl.Linear("exact", fmt, M, N, K, xd, "f32", wl.to_bits(x, xd), t, s)
        Y, _ = run_linear(lin)
        A, _ = oracle_linear(lin)
        assert np.array_equal(Y, A)


def test_special_scales_and_codes(lb):
    g = wl.generator(400)
    M, N, K = 20, 70, 384
    xb = wl.activations(g, M, K, "bf16")
    t = wl.ternary_codes(g, N, K, 0.35)
    s = wl.group_scales(g, N, K)
    s[0, :] = 0                                        # all-zero row of scales
    s[1, 1] = 0
    s[2, :] = np.float16(2.0 ** -24)                   # smallest subnormal
    s[3, 0] = np.float16(3.0 * 2.0 ** -20)             # another subnormal
    s[4, :] = -s[4, :]                                 # negative scales
    s[5, 2] = np.float16(60000.0)                      # large
    b = wl.bias_f16(g, N)
    lin = wl.Linear("special", "ternary", M, N, K, "bf16", "f32", xb, t, s, b)
    Y, _ = run_linear(lin)
    A, Mg = oracle_linear(lin)
    _assert_parity(Y, A, Mg, "f32", "special scales")
    assert np.all(Y[:, 0] == np.float32(b[0]))          # zero scales -> bias exactly
    # all-zero codes -> output equals the bias exactly
    lin0 = wl.Linear("zero", "ternary", M, N, K, "bf16", "bf16", xb, np.zeros_like(t), s, b)
    Y0, _ = run_linear(lin0)
    assert np.array_equal(Y0, np.broadcast_to(oracle.decode(oracle.encode(b.astype(np.float64), "bf16"), "bf16"), (M, N)))


# ---------------------------------------------------- variants / safety ---

# shapes that reach every compiled variant of the two small-M kernels: the
# one with the K split inside the workgroup (N / 16 below the CU count; one
# chunk of 2 or 4 groups per wave, or 3 .. 8 double-buffered chunks of 2 for
# long K) and the one with column tiles of 48 .. 128 columns (3, 4, 5, 6, 8
# column waves), slices of 4 .. 32 groups split into K parts, one or many K
# splits; odd group counts, ragged N, M < 16
_SMALL_SHAPES = [(5, 64, 512), (16, 3072, 3072), (7, 520, 6144), (1, 200, 12288),
                 (16, 8192, 1024), (3, 8200, 2048), (16, 18432, 3072), (2, 8192, 8192),
                 (16, 100, 16384), (16, 100, 4096), (9, 3000, 2560), (16, 1000, 4608),
                 (4, 4000, 128), (13, 2048, 1152), (16, 3072, 9216), (6, 2000, 12288),
                 (16, 300, 4736), (16, 500, 7168), (2, 1500, 13312), (16, 22000, 3072),
                 (5, 30000, 3072), (4, 3072, 9216), (8, 9216, 3072), (12, 520, 6144), (4, 3072, 3072)]


@pytest.mark.parametrize("fmt", ["ternary", "binary"])
@pytest.mark.parametrize("M,N,K", _SMALL_SHAPES)
def test_small_and_large_kernels_agree_with_oracle(lb, force_variant, fmt, M, N, K):
    lin = wl.make_linear("both", fmt, M, N, K, seed=500 + M, p0=0.35)
    A, Mg = oracle_linear(lin)
    for v in ("small", "small-split", "large"):
        force_variant(v)
        Y, _ = run_linear(lin)
        _assert_parity(Y, A, Mg, "bf16", f"{v} kernel")


# shapes for both large-M tile configurations (128 x 512 / 128 x 256 wide
# tiles, 96 x 256 pair tiles): ragged M and N, one or several tiles, odd
# group counts, and one to three groups (fewer groups than the three-stage
# pipeline is deep: no group is staged past the last)
_LARGE_SHAPES = [(100, 300, 1024), (257, 2100, 384), (96, 256, 128), (191, 4097, 640), (500, 1030, 1152),
                 (130, 2200, 256)]


@pytest.mark.parametrize("fmt", ["ternary", "binary"])
@pytest.mark.parametrize("M,N,K", _LARGE_SHAPES)
def test_large_m_tile_configurations(lb, force_variant, fmt, M, N, K):
    lin = wl.make_linear("tiles", fmt, M, N, K, seed=520 + M, p0=0.35, with_bias=True)
    A, Mg = oracle_linear(lin)
    for v in ("large-wide", "large-pair"):
        force_variant(v)
        Y, _ = run_linear(lin)
        _assert_parity(Y, A, Mg, "bf16", f"{v} tiles")
    # fused GELU through the pair tiles (the epilogue runs per workgroup)
    force_variant("large-pair")
    Yg, _ = run_linear(lin, activation="gelu", out_dtype=torch.float32)
    G = oracle.gelu(A)
    lim = 1.13 * (oracle.REL_TOL * Mg + oracle.ABS_TOL) + 4 * oracle.ulp(G, "f32")
    assert not (np.abs(Yg - G) > lim).any()


@pytest.mark.parametrize("fmt", ["ternary", "binary"])
@pytest.mark.parametrize("variant,M,N,K", [(None, 5, 520, 2048),           # K split inside the workgroup
                                           (None, 16, 8192, 1024),         # column tiles
                                           ("small-split", 7, 3072, 9216),  # K split across workgroups
                                           (None, 3, 100, 40960)])         # runtime chunk count
def test_small_m_bias_gelu_epilogue(lb, force_variant, fmt, variant, M, N, K):
    """fp16 activations, fp16 bias and the fused exact-erf GELU to FP32
    outputs through each small-M path (bias and GELU are applied once, to the
    full FP32 sum, also after the cross-workgroup combine)."""
    force_variant(variant)
    lin = wl.make_linear("epi", fmt, M, N, K, x_dtype="f16", seed=660 + M, p0=0.35, with_bias=True)
    A, Mg = oracle_linear(lin)
    Yg, _ = run_linear(lin, activation="gelu", out_dtype=torch.float32)
    G = oracle.gelu(A)
    lim = 1.13 * (oracle.REL_TOL * Mg + oracle.ABS_TOL) + 4 * oracle.ulp(G, "f32")
    bad = np.abs(Yg - G) > lim
    assert not bad.any(), f"{int(bad.sum())} outputs outside the bound"


@pytest.mark.parametrize("fmt", ["ternary", "binary"])
@pytest.mark.parametrize("M,N,K", [(16, 100, 98304), (1, 40, 40960), (3, 4100, 65664)])
def test_small_m_beyond_the_column_tile_plan(lb, fmt, M, N, K):
    """M <= 16 with more than 8 chunks of K per wave (runtime chunk count) and,
    for wide N, more K groups than the column-tile kernel covers (513 > 512):
    the kernel with the K split inside the workgroup takes both. Checked on
    sampled columns against the oracle restricted to them."""
    banner(f"beyond the column-tile plan {fmt} {M}x{N}x{K}")
    lin = wl.make_linear("beyond", fmt, M, N, K, seed=640 + M, p0=0.35, with_bias=False)
    Y, _ = run_linear(lin, bias=False)
    rng = np.random.default_rng(N)
    cols = np.unique(np.concatenate([np.arange(16), np.arange(N - 16, N), rng.integers(0, N, 32)]))
    A = oracle.linear(lin.x, lin.x_dtype, lin.codes[cols], lin.scales[cols], None)
    Mg = oracle.magnitude(lin.x, lin.x_dtype, lin.codes[cols], lin.scales[cols], None)
    _assert_parity(Y[:, cols], A, Mg, lin.y_dtype, f"{fmt} {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K,ldx", [(4200, 512, 256, 1 << 19),         # large-M kernel, 2 chunks
                                         (16, 8192, 256, 150_000_000),     # column tiles, 2 chunks of 8
                                         (5, 640, 256, 600_000_000)])      # thin kernel, chunks of 3 and 2
def test_activations_spanning_4gib_run_in_row_chunks(lb, M, N, K, ldx):
    """X whose row stride makes it span 4 GiB or more: the kernels address X
    by 32-bit byte offsets, so the library runs it in row chunks that span
    less. Every row must meet the bound (4.4 to 5 GB of device memory)."""
    banner(f"strided X {M}x{N}x{K} ldx={ldx}")
    lin = wl.make_linear("stride", "ternary", M, N, K, seed=610 + M, p0=0.35, with_bias=False)
    A, Mg = oracle_linear(lin)
    xs = torch.empty((M, ldx), dtype=torch.bfloat16, device="cuda")
    xs[:, :K] = dev_bits(lin.x, "bf16")
    packed, s = dev_weights("ternary", lin.codes, lin.scales)
    y = lb.gemm(xs[:, :K], packed, s, "ternary")
    torch.cuda.synchronize()
    del xs
    torch.cuda.empty_cache()
    _assert_parity(to_host64(y), A, Mg, "bf16", f"strided X ldx={ldx}")


@pytest.mark.parametrize("fmt", ["ternary", "binary"])
@pytest.mark.parametrize("M,N,K", [(16, 3072, 9216), (3, 3072, 12288), (1, 200, 12288)])
def test_split_k_small_m_is_deterministic_and_reusable(lb, force_variant, fmt, M, N, K):
    """Split-K at small M (the column-tile kernel, forced: these narrow shapes
    otherwise take the kernel with the K split inside the workgroup): the
    workgroups of a column tile combine their FP32 partials in split order
    through the workspace, and the last one resets its counter. Forty calls in
    a row on one workspace (each into a NaN-filled output) must all write every
    element and give identical bits; a workspace smaller than required is
    refused. Afterwards the whole workspace is zero again: tickets, the
    counter of bounded waits that gave up, and every partial slot."""
    force_variant("small-split")
    need = lb.workspace_bytes(fmt, M, N, K)
    assert need > 0                                   # these shapes split K
    lin = wl.make_linear("split", fmt, M, N, K, seed=560 + M, p0=0.35)
    x = dev_bits(lin.x, "bf16")
    packed, s = dev_weights(fmt, lin.codes, lin.scales)
    ws = lb.new_workspace(need)
    outs = []
    for _ in range(40):
        y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        lb.gemm(x, packed, s, fmt, out=y, workspace=ws)
        outs.append(y)
    torch.cuda.synchronize()
    assert not torch.isnan(outs[0]).any()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int32), outs[0].view(torch.int32))
    # every ticket, the give-up counter and every partial slot are zero again
    # (each reducer stores zeros over the partials it consumed)
    assert int(ws.count_nonzero()) == 0
    A, Mg = oracle_linear(lin)
    _assert_parity(to_host64(outs[0]), A, Mg, "f32", "split-K small M")
    with pytest.raises(ValueError):
        lb.gemm(x, packed, s, fmt, workspace=ws[: need // 2])


@pytest.mark.parametrize("M", [16, 1536])
def test_same_input_linears_fused_by_concatenated_rows(lb, M):
    """Linears that share an input (Q, K, V) run as one launch over their
    packed rows and scales concatenated along N (the packed layout is row-major
    in N, so concatenating packed rows equals packing the concatenated codes);
    each column slice of the fused output meets the bound against its own
    linear, and the packed bytes match the separate packs exactly."""
    g = wl.generator(950 + M)
    K = 3072
    x = wl.activations(g, M, K, "bf16")
    lins = [wl.make_linear(f"qkv{i}", "ternary", M, 3072, K, g=g, x=x, p0=0.35) for i in range(3)]
    parts = [dev_weights("ternary", l.codes, l.scales) for l in lins]
    packed = torch.cat([p for p, _ in parts], dim=0)
    scales = torch.cat([sc for _, sc in parts], dim=0)
    whole, _ = dev_weights("ternary", np.concatenate([l.codes for l in lins], axis=0),
                           np.concatenate([l.scales for l in lins], axis=0))
    assert torch.equal(packed, whole)
    y = lb.gemm(dev_bits(x, "bf16"), packed, scales, "ternary", out_dtype=torch.float32)
    torch.cuda.synchronize()
    Y = to_host64(y)
    for i, l in enumerate(lins):
        A, Mg = oracle_linear(l)
        _assert_parity(Y[:, 3072 * i: 3072 * (i + 1)], A, Mg, "f32", f"fused slice {i}")


def test_very_long_k_small_m(lb):
    """A long K with an odd group count (129 groups: many splits, a short last one)."""
    lin = wl.make_linear("longk", "ternary", 2, 64, 129 * 128, seed=550, p0=0.35)
    Y, _ = run_linear(lin)
    A, Mg = oracle_linear(lin)
    _assert_parity(Y, A, Mg, "bf16", "long K")


@pytest.mark.parametrize("M", [4, 300])
def test_deterministic_and_every_output_written(lb, M):
    lin = wl.make_linear("det", "ternary", M, 777, 1280, seed=600 + M, p0=0.35)
    x = dev_bits(lin.x, "bf16")
    packed, s = dev_weights("ternary", lin.codes, lin.scales)
    out1 = torch.full((M, 777), float("nan"), dtype=torch.float32, device="cuda")
    out2 = torch.full((M, 777), float("nan"), dtype=torch.float32, device="cuda")
    lb.gemm(x, packed, s, "ternary", out=out1)
    lb.gemm(x, packed, s, "ternary", out=out2)
    torch.cuda.synchronize()
    assert not torch.isnan(out1).any()
    assert torch.equal(out1.view(torch.int32), out2.view(torch.int32))


def test_strided_activation_and_output(lb):
    """ldx > K and ldy > N: only the addressed region is read and written."""
    g = wl.generator(700)
    M, N, K = 40, 96, 256
    lin = wl.make_linear("stride", "ternary", M, N, K, seed=701)
    big = np.zeros((M, K + 64), dtype=np.uint16)
    big[:, :K] = lin.x
    x = dev_bits(big, "bf16")[:, :K]
    packed, s = dev_weights("ternary", lin.codes, lin.scales)
    yfull = torch.full((M, N + 8), 7.0, dtype=torch.bfloat16, device="cuda")
    lb.gemm(x, packed, s, "ternary", out=yfull[:, :N])
    torch.cuda.synchronize()
    A, Mg = oracle_linear(lin)
    _assert_parity(to_host64(yfull[:, :N].contiguous()), A, Mg, "bf16", "strided")
    assert torch.all(yfull[:, N:] == 7.0)


def test_gelu_kernel(lb):
    g = wl.generator(800)
    v = (g.standard_normal(100_000) * 3).astype(np.float32)
    v[:5] = [0.0, -0.0, 10.0, -10.0, 1e-30]
    for dt in ("bf16", "f16", "f32"):
        if dt == "f32":
            x = torch.from_numpy(v).cuda()
            xin = v.astype(np.float64)
        else:
            bits = wl.to_bits(v, dt)
            x = dev_bits(bits, dt)
            xin = oracle.decode(bits, dt)
        y = to_host64(lb.gelu(x))
        ref = oracle.gelu(xin)
        # FP32 erfc: relative error of a few 1e-7 where GELU is not tiny; in the far
        # negative tail (x < -8, |GELU| < 1e-14) the device erfcf loses relative
        # accuracy, so an absolute floor of 1e-6 applies (ten times below the 1e-5
        # floor of the layer tolerance the activation feeds); then one cast
        lim = 1e-6 * np.abs(ref) + 1e-6
        if dt != "f32":
            lim = lim + 0.5 * oracle.ulp(np.maximum(abs(ref), abs(y)), dt)
        bad = np.flatnonzero(np.abs(y - ref) > lim)
        assert bad.size == 0, (dt, [(float(xin[i]), float(y[i]), float(ref[i]), float(lim[i])) for i in bad[:5]])


def test_workspace_errors(lb, force_variant):
    """A call whose plan needs a workspace: none, one byte too small, or not
    256-byte aligned is refused before any launch (single and grouped)."""
    force_variant("small-split")
    M, N, K = 16, 3072, 9216
    L = lb.lib()
    need = L.lowbit_gemm_workspace_bytes(lb.TERNARY, M, N, K)
    assert need > 0
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    p = torch.zeros((N, K // 4), dtype=torch.uint8, device="cuda")
    s = torch.zeros((N, K // 128), dtype=torch.float16, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(need + 512, dtype=torch.uint8, device="cuda")

    def call(wptr, wbytes):
        return L.lowbit_gemm(lb.TERNARY, x.data_ptr(), lb.BF16, M, K, K, p.data_ptr(), s.data_ptr(), 128, N,
                             None, lb.NONE, y.data_ptr(), lb.BF16, N, 0, wptr, wbytes, None)
    assert call(None, 0) == lb.ERR_WORKSPACE
    assert call(ws.data_ptr(), need - 1) == lb.ERR_WORKSPACE
    assert call(ws.data_ptr() + 16, need) == lb.ERR_ALIGN
    assert call(ws.data_ptr(), need) == lb.OK
    arr = lambda *ptrs: (ctypes.c_void_p * len(ptrs))(*ptrs)
    gneed = L.lowbit_gemm_grouped_workspace_bytes(2, lb.TERNARY, M, N, K)
    assert gneed > need

    def gcall(wptr, wbytes):
        return L.lowbit_gemm_grouped(2, lb.TERNARY, arr(x.data_ptr(), x.data_ptr()), lb.BF16, M, K, K,
                                     arr(p.data_ptr(), p.data_ptr()), arr(s.data_ptr(), s.data_ptr()), 128, N,
                                     None, lb.NONE, arr(y.data_ptr(), y2.data_ptr()), lb.BF16, N, 0,
                                     wptr, wbytes, None)
    gws = torch.zeros(gneed, dtype=torch.uint8, device="cuda")
    assert gcall(ws.data_ptr(), need) == lb.ERR_WORKSPACE
    assert gcall(None, 0) == lb.ERR_WORKSPACE
    torch.cuda.synchronize()
    del gws


def test_device_side_errors(lb):
    x = torch.zeros((4, 128), dtype=torch.bfloat16, device="cuda")
    p = torch.zeros((4, 32), dtype=torch.uint8, device="cuda")
    s = torch.zeros((4, 1), dtype=torch.float16, device="cuda")
    y = torch.empty((4, 8), dtype=torch.bfloat16, device="cuda")     # ldy = 8 >= N
    L = lb.lib()
    need = L.lowbit_gemm_workspace_bytes(lb.TERNARY, 4, 4, 128)
    st = L.lowbit_gemm(lb.TERNARY, x.data_ptr(), lb.BF16, 4, 128, 128, p.data_ptr(), s.data_ptr(), 128, 4,
                       None, lb.NONE, y.data_ptr(), lb.BF16, 8, 0, None, 0, None)
    assert st == lb.OK if need == 0 else st == lb.ERR_WORKSPACE
    assert L.lowbit_init() == lb.OK


def test_binding_refuses_mismatched_tensors(lb):
    """The C ABI takes raw pointers and cannot see buffer sizes; the binding
    checks every tensor against the problem's shape before the call."""
    M, N, K = 8, 64, 256
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    p = torch.zeros((N, K // 4), dtype=torch.uint8, device="cuda")
    s = torch.zeros((N, K // 128), dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError, match="packed"):
        lb.gemm(x, p[:, :32], s, "ternary")                       # codes for K = 128
    with pytest.raises(ValueError, match="packed"):
        lb.gemm(x, p, s, "binary")                                # ternary bytes as binary
    with pytest.raises(ValueError, match="scales"):
        lb.gemm(x, p, s[:, :1], "ternary")
    with pytest.raises(ValueError, match="bias"):
        lb.gemm(x, p, s, "ternary", bias=torch.zeros(N - 1, dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError, match="out"):
        lb.gemm(x, p, s, "ternary", out=torch.empty((M, N - 1), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError, match="x must"):
        lb.gemm(x.float(), p, s, "ternary")
    with pytest.raises(ValueError, match="packed"):
        lb.unpack("ternary", p, K + 16)
    with pytest.raises(ValueError, match="scales"):
        lb.gemm_grouped([x, x], [p, p], [s, s[:, :1]], "ternary")
    with pytest.raises(ValueError, match="outs"):
        lb.gemm_grouped([x, x], [p, p], [s, s], "ternary",
                        outs=[torch.empty((M, N), dtype=torch.bfloat16, device="cuda")] * 1)
    torch.cuda.synchronize()


@pytest.mark.parametrize("bias_dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("variant,M,N,K", [(None, 5, 520, 2048), ("small-split", 16, 3072, 9216),
                                           ("large-pair", 200, 1030, 1152), ("large-wide", 130, 2100, 384)])
def test_bias_dtypes_on_every_path(lb, force_variant, bias_dtype, variant, M, N, K):
    """Bias in f16, bf16 or f32 is added once, in FP32, before the single
    rounding: against the oracle's sum plus the bias's exact value."""
    force_variant(variant)
    lin = wl.make_linear("biasdt", "ternary", M, N, K, seed=880 + M, p0=0.35, with_bias=True)
    b16 = lin.bias.astype(np.float32)
    if bias_dtype == "f16":
        bdev = torch.from_numpy(lin.bias.view(np.int16)).cuda().view(torch.float16)
        bval = b16.astype(np.float64)
    elif bias_dtype == "bf16":
        bits = oracle.encode(b16.astype(np.float64) * 3.0, "bf16")     # values f16 cannot hold exactly
        bdev = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
        bval = oracle.decode(bits, "bf16")
    else:
        v = (b16 * np.float32(1.0 / 3.0)).astype(np.float32)          # full FP32 significands
        bdev = torch.from_numpy(v).cuda()
        bval = v.astype(np.float64)
    x = dev_bits(lin.x, "bf16")
    packed, s = dev_weights("ternary", lin.codes, lin.scales)
    y = lb.gemm(x, packed, s, "ternary", bias=bdev, out_dtype=torch.float32)
    torch.cuda.synchronize()
    A0 = oracle.linear(lin.x, "bf16", lin.codes, lin.scales)
    Mg0 = oracle.magnitude(lin.x, "bf16", lin.codes, lin.scales)
    A = A0 + bval[None, :]
    Mg = Mg0 + np.abs(bval)[None, :]
    _assert_parity(to_host64(y), A, Mg, "f32", f"bias {bias_dtype} {variant}")


@pytest.mark.parametrize("variant,M", [(None, 4), ("small-split", 16), (None, 1), ("large-pair", 40),
                                       ("large-wide", 40)])
def test_special_scales_on_every_path(lb, force_variant, variant, M):
    """Zero, subnormal, negative and large FP16 scales, through the small-M
    kernels as well as the large-M ones."""
    force_variant(variant)
    g = wl.generator(410 + M)
    N, K = 300, 2304
    xb = wl.activations(g, M, K, "bf16")
    t = wl.ternary_codes(g, N, K, 0.35)
    s = wl.group_scales(g, N, K)
    s[0, :] = 0
    s[1, 1] = 0
    s[2, :] = np.float16(2.0 ** -24)
    s[3, 0] = np.float16(3.0 * 2.0 ** -20)
    s[4, :] = -s[4, :]
    s[5, 2] = np.float16(60000.0)
    s[6, ::2] = 0
    lin = wl.Linear("special2", "ternary", M, N, K, "bf16", "f32", xb, t, s, None)
    Y, _ = run_linear(lin)
    A, Mg = oracle_linear(lin)
    _assert_parity(Y, A, Mg, "f32", f"special scales {variant}")
    assert np.all(Y[:, 0] == 0.0)


@pytest.mark.parametrize("variant,M", [(None, 4), ("small-split", 16), ("large-pair", 40), ("large-wide", 40)])
def test_fp16_output_overflows_to_infinity(lb, force_variant, variant, M):
    """Sums beyond the FP16 range round to infinity of their sign (one RNE
    cast); sums well inside it meet the bound; the band where the tolerance
    can move a value across 65520 may give either."""
    force_variant(variant)
    g = wl.generator(420 + M)
    N, K = 200, 1024
    xv = np.abs(g.standard_normal((M, K))) * 4.0 + 1.0
    xb = oracle.encode(xv, "f16")
    t = wl.ternary_codes(g, N, K, 0.1)
    t[: N // 4] = 1                                                    # sums of +2.7e5 or so
    t[N // 4: N // 2] = -1                                             # and of -2.7e5
    s = np.full((N, K // 128), np.float16(64.0), dtype=np.float16)   # sums of several 10^5
    s[N // 2:] = np.float16(0.25)                                      # these stay finite
    lin = wl.Linear("ovf", "ternary", M, N, K, "f16", "f16", xb, t, s, None)
    Y, _ = run_linear(lin)
    A, Mg = oracle_linear(lin)
    lim = 65520.0
    big = np.abs(A) > lim * 1.01
    small = np.abs(A) < 65504.0 * 0.99
    assert big.any() and small.any()
    assert np.all(np.isinf(Y[big])) and np.all(np.sign(Y[big]) == np.sign(A[big]))
    ok, worst, nfail = oracle.check(Y[small], A[small], Mg[small], "f16")
    assert ok, f"{nfail} finite outputs outside the bound"


@pytest.mark.parametrize("variant,M", [(None, 4), ("small-split", 16), (None, 1), ("large-pair", 40),
                                       ("large-wide", 40)])
def test_non_finite_activations_propagate(lb, force_variant, variant, M):
    """NaN and infinities in X give the oracle's non-finite outputs in place
    (IEEE: infinity times a zero weight is NaN, opposite infinities add to
    NaN); every other output meets the bound."""
    force_variant(variant)
    g = wl.generator(430 + M)
    N, K = 160, 1024
    xv = g.standard_normal((M, K))
    xv[0, 5] = np.nan
    if M > 1:
        xv[1, 7] = np.inf
    if M > 2:
        xv[2, 9] = -np.inf
        xv[2, 700] = np.inf
    xb = oracle.encode(xv, "bf16")
    t = wl.ternary_codes(g, N, K, 0.35)
    s = wl.group_scales(g, N, K)
    lin = wl.Linear("nonfinite", "ternary", M, N, K, "bf16", "f32", xb, t, s, None)
    Y, _ = run_linear(lin)
    with np.errstate(invalid="ignore"):               # the oracle's own inf - inf and inf * 0
        A, Mg = oracle_linear(lin)
        ok, worst, nfail = oracle.check(Y, A, Mg, "f32")
    assert not np.isfinite(A[0]).any()
    assert ok, f"{nfail} outputs differ (non-finite in place, finite within the bound)"


@pytest.mark.parametrize("variant,M", [(None, 4), ("small-split", 16), (None, 1), ("large-pair", 40),
                                       ("large-wide", 40)])
def test_invalid_ternary_code_acts_as_zero(lb, force_variant, variant, M):
    """The INT2 pattern 10 (never written by the packer; what the base-3
    transcoder writes for an invalid byte) is read by every GEMM path as t = 0."""
    force_variant(variant)
    g = wl.generator(440 + M)
    N, K = 96, 1024
    lin = wl.make_linear("code10", "ternary", M, N, K, seed=441 + M, p0=0.35)
    packed = oracle.pack_ternary(lin.codes)
    rows = g.choice(N, size=20, replace=False)
    cols = g.choice(K // 4, size=20)
    for r, c in zip(rows, cols):
        packed[r, c] = 0xAA                                  # four fields of 10
    t_eff, bad = oracle.unpack_ternary(packed, K)           # 10 -> 0, counted
    assert bad == 80
    x = dev_bits(lin.x, "bf16")
    s = torch.from_numpy(lin.scales.view(np.int16)).cuda().view(torch.float16)
    y = lb.gemm(x, torch.from_numpy(packed).cuda(), s, "ternary", out_dtype=torch.float32)
    torch.cuda.synchronize()
    A = oracle.linear(lin.x, "bf16", t_eff, lin.scales)
    Mg = oracle.magnitude(lin.x, "bf16", t_eff, lin.scales)
    _assert_parity(to_host64(y), A, Mg, "f32", f"code 10 {variant}")
