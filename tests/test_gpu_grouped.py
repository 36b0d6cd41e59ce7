"""lowbit_gemm_grouped: several independent linears of one shape in one launch.
Every problem against the oracle, through each small-M path (K split inside
the workgroup, column tiles, column tiles with the K split across workgroups,
the any-N fallback) and the one-problem-after-another path for M > 16;
deterministic, equal to lowbit_gemm for one problem, and replayable from a
HIP graph."""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import TORCH_DT, banner, dev_bits, dev_weights, oracle_linear, to_host64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lb():
    import bit_weight_gemm_int2_amd as b
    b.lib()
    return b


def _problems(count, fmt, M, N, K, seed, xd="bf16", bias=False):
    return [wl.make_linear(f"g{z}", fmt, M, N, K, x_dtype=xd, seed=seed + 17 * z, p0=0.35, with_bias=bias)
            for z in range(count)]


def _run(lb, lins, yd=None, gelu=False, workspace=None):
    xd = lins[0].x_dtype
    xs = [dev_bits(l.x, xd) for l in lins]
    ws = [dev_weights(l.fmt, l.codes, l.scales) for l in lins]
    bs = None
    if lins[0].bias is not None:
        bs = [torch.from_numpy(l.bias.view(np.int16)).cuda().view(torch.float16) for l in lins]
    ys = lb.gemm_grouped(xs, [w[0] for w in ws], [w[1] for w in ws], lins[0].fmt, biases=bs,
                         out_dtype=TORCH_DT[yd or lins[0].y_dtype], activation="gelu" if gelu else None,
                         workspace=workspace)
    torch.cuda.synchronize()
    return [to_host64(y) for y in ys], (xs, ws, bs)


def _check(lins, Ys, yd, gelu=False):
    for z, (l, Y) in enumerate(zip(lins, Ys)):
        A, Mg = oracle_linear(l)
        if gelu:
            G = oracle.gelu(A)
            lim = 1.13 * (oracle.REL_TOL * Mg + oracle.ABS_TOL) + 4 * oracle.ulp(G, "f32")
            assert not (np.abs(Y - G) > lim).any(), f"problem {z}: GELU bound"
        else:
            ok, worst, nfail = oracle.check(Y, A, Mg, yd)
            assert ok, f"problem {z}: {nfail} outside the bound (worst {worst:.3g})"


@pytest.mark.parametrize("fmt", ["ternary", "binary"])
@pytest.mark.parametrize("count,M,N,K", [
    (2, 16, 3072, 3072),      # two 3072 x 3072 linears: 384 column blocks -> thin, two workgroups a CU
    (2, 16, 3072, 9216),      # long K: the same thin pair, nine chunks a wave (runtime count)
    (2, 1, 3072, 9216),       # the thin pair copying one row quad (M <= 4)
    (2, 7, 3000, 2048),       # the thin pair with ragged N, two row quads and two chunks a wave
    (3, 16, 1500, 4096),      # three problems, 282 blocks
    (2, 16, 9216, 3072),      # the double-stream fused QKV pair
    (6, 1, 3072, 3072),       # Q, K, V of both streams at M = 1
    (3, 5, 520, 6144),        # ragged N, K split inside the workgroup
    (8, 8, 64, 512),          # eight tiny problems (thin plan over 32 blocks)
    (2, 3, 100, 98304),       # beyond the column-tile plan: the any-N fallback
    (3, 100, 300, 1024),      # M > 16: one launch per problem
])
def test_grouped_problems_match_the_oracle(lb, fmt, count, M, N, K):
    banner(f"grouped {fmt} count={count} {M}x{N}x{K}")
    lins = _problems(count, fmt, M, N, K, seed=7000 + M + count)
    Ys, _ = _run(lb, lins)
    _check(lins, Ys, "bf16")


def test_grouped_bias_gelu_f16_to_f32(lb):
    banner("grouped bias + GELU, f16 -> f32")
    lins = _problems(4, "ternary", 12, 1000, 2560, seed=7100, xd="f16", bias=True)
    Ys, _ = _run(lb, lins, yd="f32", gelu=True)
    _check(lins, Ys, "f32", gelu=True)


def test_grouped_split_k_workspace_and_determinism(lb):
    """Forced cross-workgroup K split: the tickets of all problems sit side
    by side in one workspace, come back to zero, and a second call gives the
    same bits."""
    banner("grouped split-K workspace")
    lb.force_variant("small-split")
    try:
        lins = _problems(3, "ternary", 16, 2048, 12288, seed=7200)
        need = lb.lib().lowbit_gemm_grouped_workspace_bytes(3, lb.TERNARY, 16, 2048, 12288)
        assert need > 0
        ws = lb.new_workspace(need)
        Ys, _ = _run(lb, lins, workspace=ws)
        _check(lins, Ys, "bf16")
        assert int(ws.count_nonzero()) == 0     # tickets and partial slots
        Ys2, _ = _run(lb, lins, workspace=ws)
        for a, b in zip(Ys, Ys2):
            assert np.array_equal(a, b)
    finally:
        lb.force_variant(None)


def test_one_problem_group_equals_lowbit_gemm(lb):
    banner("grouped count=1 vs lowbit_gemm")
    lins = _problems(1, "binary", 16, 9216, 3072, seed=7300)
    Ys, (xs, ws, _) = _run(lb, lins)
    y = lb.gemm(xs[0], ws[0][0], ws[0][1], "binary")
    torch.cuda.synchronize()
    assert np.array_equal(Ys[0], to_host64(y))


def test_grouped_graph_replay(lb):
    banner("grouped graph replay")
    count, M, N, K = 2, 16, 3072, 9216
    lins = _problems(count, "ternary", M, N, K, seed=7400)
    ws = [dev_weights("ternary", l.codes, l.scales) for l in lins]
    g = wl.generator(7401)
    inputs = [[dev_bits(wl.activations(g, M, K, "bf16"), "bf16") for _ in range(count)] for _ in range(3)]
    xs = [x.clone() for x in inputs[0]]
    ys = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for _ in range(count)]
    need = lb.lib().lowbit_gemm_grouped_workspace_bytes(count, lb.TERNARY, M, N, K)
    wsp = lb.new_workspace(need)
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        lb.gemm_grouped(xs, [w[0] for w in ws], [w[1] for w in ws], "ternary", outs=ys, workspace=wsp)
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=st):
        lb.gemm_grouped(xs, [w[0] for w in ws], [w[1] for w in ws], "ternary", outs=ys, workspace=wsp)
    torch.cuda.synchronize()
    for r, xin in enumerate(inputs):
        for x, xn in zip(xs, xin):
            x.copy_(xn)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        refs = lb.gemm_grouped(xin, [w[0] for w in ws], [w[1] for w in ws], "ternary",
                               workspace=lb.new_workspace(need))
        torch.cuda.synchronize()
        for z in range(count):
            assert torch.equal(ys[z].view(torch.int16), refs[z].view(torch.int16)), f"replay {r} problem {z}"


@pytest.mark.parametrize("variant", ["large", "large-pair", "small", "small-split"])
def test_grouped_under_forced_variants(lb, variant):
    """Every kernel family a group can land on: forced large-M kernels run the
    problems one launch each even at M <= 16; forced small-M kernels group them."""
    banner(f"grouped forced {variant}")
    lb.force_variant(variant)
    try:
        lins = _problems(3, "binary", 16, 1000, 4608, seed=7500)
        Ys, _ = _run(lb, lins)
        _check(lins, Ys, "bf16")
    finally:
        lb.force_variant(None)
