"""lowbit_gemm captured in a HIP graph and replayed: every replay, with new
activations copied into the captured input between replays (eager work and a
synchronisation in between), must give the bits of an eager call on the same
inputs. Covers each launch path: the small-M kernel with the K split inside
the workgroup, the column-tile small-M kernel with a cross-workgroup K split
(tickets and partials in the workspace, which must come back to zero after
every replay), and the large-M kernel with wide and with pair tiles."""
import os

import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import banner, dev_bits, dev_weights

pytestmark = pytest.mark.gpu

CASES = [  # (variant forced or None, fmt, M, N, K)
    (None, "ternary", 16, 3072, 3072),          # thin, one chunk per wave
    (None, "binary", 3, 3072, 9216),            # thin, chunked
    ("small-split", "ternary", 16, 3072, 9216),  # column tiles, split K
    ("large-wide", "ternary", 300, 2048, 1024),
    ("large-pair", "binary", 300, 2048, 1024),
]


@pytest.fixture(scope="module")
def lb():
    import bit_weight_gemm_int2_amd as b
    b.lib()
    return b


@pytest.mark.parametrize("variant,fmt,M,N,K", CASES)
def test_graph_replay_matches_eager(lb, variant, fmt, M, N, K):
    banner(f"graph replay {variant} {fmt} {M}x{N}x{K}")
    if variant:
        lb.force_variant(variant)
    try:
        lin = wl.make_linear("graph", fmt, M, N, K, seed=900 + M, p0=0.35, with_bias=True)
        packed, s = dev_weights(fmt, lin.codes, lin.scales)
        b = torch.from_numpy(lin.bias.view(np.int16)).cuda().view(torch.float16)
        g = wl.generator(901)
        xs = [dev_bits(wl.activations(g, M, K, "bf16"), "bf16") for _ in range(4)]
        x = xs[0].clone()
        need = lb.workspace_bytes(fmt, M, N, K)
        if variant == "small-split":
            assert need > 0
        ws = lb.new_workspace(need)
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            lb.gemm(x, packed, s, fmt, bias=b, out=y, workspace=ws)          # warm-up on the capture stream
        torch.cuda.current_stream().wait_stream(st)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=st):
            lb.gemm(x, packed, s, fmt, bias=b, out=y, workspace=ws)
        torch.cuda.synchronize()
        for r, xn in enumerate(xs):
            x.copy_(xn)                                                      # eager work between replays
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            ref = lb.gemm(xn, packed, s, fmt, bias=b, workspace=lb.new_workspace(need))
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), f"replay {r}"
        if need:
            assert int(ws.count_nonzero()) == 0        # tickets and partial slots back to zero
    finally:
        lb.force_variant(None)


def test_graph_replay_base3_transcode(lb):
    """base3_to_int2 with its invalid-value counter, captured once and replayed
    on new base-3 inputs copied in between (some with invalid bytes): every
    replay must match the oracle, counter included (the counter is cleared by
    a kernel inside the graph, not by a memset node)."""
    import oracle
    banner("graph replay base3_to_int2")
    N, K = 300, 1008
    g = wl.generator(902)
    inputs = []
    for r in range(4):
        p = oracle.pack_base3(wl.ternary_codes(g, N, K, 0.35))
        if r % 2:
            p[r, 3] = 243 + r
            p[N - 1, -1] = 255
        inputs.append(p)
    p_dev = torch.from_numpy(inputs[0]).cuda()
    out = torch.empty((N, K // 4), dtype=torch.uint8, device="cuda")
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    L = lb.lib()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())

    def call():
        return L.base3_to_int2(p_dev.data_ptr(), N, K, out.data_ptr(), cnt.data_ptr(), st.cuda_stream)
    with torch.cuda.stream(st):
        assert call() == 0
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=st):
        assert call() == 0
    torch.cuda.synchronize()
    for r, p in enumerate(inputs):
        p_dev.copy_(torch.from_numpy(p))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref, bad = oracle.base3_to_ternary(p, K)
        assert np.array_equal(out.cpu().numpy(), ref), f"replay {r}"
        assert int(cnt.item()) == bad, f"replay {r}"
