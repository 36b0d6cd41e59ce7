"""GPU group quantiser (lowbit_quantize): packed codes and FP16 scale bits
identical to the oracle's rule on the same FP16 weights."""
import ctypes
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lb():
    import bit_weight_gemm_int2_amd as b
    b.lib()
    return b


def _dev16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.float16)


def _expect(w_bits: np.ndarray, fmt: str):
    t, s, bad = oracle.quantize(w_bits, fmt)
    return (oracle.pack_ternary(t) if fmt == "ternary" else oracle.pack_binary(t)), s, bad


def _check(lb, w_bits: np.ndarray, fmt: str, w_dev=None):
    p_ref, s_ref, _ = _expect(w_bits, fmt)
    packed, scales = lb.quantize(_dev16(w_bits) if w_dev is None else w_dev, fmt)
    assert np.array_equal(packed.cpu().numpy(), p_ref)
    assert np.array_equal(scales.view(torch.int16).cpu().numpy().view(np.uint16), s_ref)


@pytest.mark.parametrize("fmt", ["ternary", "binary"])
@pytest.mark.parametrize("N,K,seed", [(1, 128, 0), (3, 256, 1), (7, 384, 2), (33, 1152, 3), (130, 3072, 4)])
def test_quantize_bit_exact_small(lb, fmt, N, K, seed):
    print(f"[gpu] quantize {fmt} {N}x{K}", flush=True)
    g = wl.generator(40 + seed)
    _check(lb, wl.fp16_weights(g, N, K, outliers=0.01), fmt)


@pytest.mark.parametrize("fmt", ["ternary", "binary"])
def test_quantize_strided_rows(lb, fmt):
    """Row stride above K: only the first K columns of each row are read."""
    g = wl.generator(50)
    full = wl.fp16_weights(g, 45, 640)
    w = _dev16(full)[:, :512]
    assert w.stride(0) == 640
    _check(lb, np.ascontiguousarray(full[:, :512]), fmt, w_dev=w)


def test_quantize_hand_groups(lb, golden_dir):
    """The hand-derived groups (threshold ties, rounding midpoints, subnormal
    and zero means, signed zeros, non-finite weights) as rows of one matrix."""
    with open(os.path.join(golden_dir, "quantize_groups.json")) as f:
        cases = json.load(f)["cases"]
    for fmt in ("ternary", "binary"):
        rows = [[int(h, 16) for n, h in c["w"] for _ in range(n)] for c in cases]
        w = np.array(rows, dtype=np.uint16)
        p_ref, s_ref, bad_ref = _expect(w, fmt)
        with pytest.raises(ValueError):
            lb.quantize(_dev16(w), fmt)                  # the NaN / inf row is reported
        packed, scales = lb.quantize(_dev16(w), fmt, check=False)
        assert np.array_equal(packed.cpu().numpy(), p_ref)
        assert np.array_equal(scales.view(torch.int16).cpu().numpy().view(np.uint16), s_ref)
        for c, srow in zip(cases, s_ref[:, 0]):
            if c["fmt"] == fmt:
                assert int(srow) == int(c["s_hex"], 16), c["name"]


def test_quantize_counts_nonfinite(lb):
    g = wl.generator(51)
    w = wl.fp16_weights(g, 20, 512)
    where = [(0, 0), (3, 200), (19, 511), (7, 7), (7, 8)]
    vals = [0x7E00, 0x7C00, 0xFC00, 0xFE01, 0x7C01]
    for (n, k), v in zip(where, vals):
        w[n, k] = v
    cnt = torch.empty(1, dtype=torch.int32, device="cuda")
    packed = torch.empty((20, 128), dtype=torch.uint8, device="cuda")
    scales = torch.empty((20, 4), dtype=torch.float16, device="cuda")
    wd = _dev16(w)
    st = lb.lib().lowbit_quantize(lb.TERNARY, wd.data_ptr(), 20, 512, 512, packed.data_ptr(), scales.data_ptr(),
                                  cnt.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == lb.OK
    assert int(cnt.item()) == len(where)
    p_ref, s_ref, bad = _expect(w, "ternary")
    assert bad == len(where)
    assert np.array_equal(packed.cpu().numpy(), p_ref)
    assert np.array_equal(scales.view(torch.int16).cpu().numpy().view(np.uint16), s_ref)


@pytest.mark.parametrize("fmt", ["ternary", "binary"])
def test_quantize_guard_bands(lb, fmt):
    """Nothing is written past the packed rows or the scales."""
    N, K = 37, 768
    g = wl.generator(52)
    w = wl.fp16_weights(g, N, K)
    row = K // 4 if fmt == "ternary" else K // 8
    pbuf = torch.full((N * row + 4096,), 0xA5, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((N * K // 128 + 2048,), -7, dtype=torch.int16, device="cuda")
    wd = _dev16(w)
    st = lb.lib().lowbit_quantize(lb.TERNARY if fmt == "ternary" else lb.BINARY, wd.data_ptr(), N, K, K,
                                  pbuf.data_ptr() + 2048, sbuf.data_ptr() + 2048, None,
                                  torch.cuda.current_stream().cuda_stream)
    assert st == lb.OK
    p_ref, s_ref, _ = _expect(w, fmt)
    ph, sh = pbuf.cpu().numpy(), sbuf.cpu().numpy()
    assert (ph[:2048] == 0xA5).all() and (ph[2048 + N * row:] == 0xA5).all()
    assert np.array_equal(ph[2048:2048 + N * row].reshape(N, row), p_ref)
    assert (sh[:1024] == -7).all() and (sh[1024 + N * K // 128:] == -7).all()
    assert np.array_equal(sh[1024:1024 + N * K // 128].view(np.uint16).reshape(N, K // 128), s_ref)


@pytest.mark.parametrize("fmt", ["ternary", "binary"])
@pytest.mark.parametrize("N,K", [(3072, 3072), (9216, 3072)])
def test_quantize_full_size_bit_exact(lb, fmt, N, K):
    """The transformer's linear shapes, every group compared."""
    print(f"[gpu] quantize {fmt} {N}x{K} full", flush=True)
    g = wl.generator(60 + N // 1024)
    _check(lb, wl.fp16_weights(g, N, K, outliers=0.001), fmt)


def test_quantize_many_passes_sampled_rows(lb):
    """More groups than one pass of the grid covers (2^21 groups), checked on
    sampled rows; the rule is row-local, so a row's oracle result does not
    depend on the others."""
    N, K = 21001, 12928                                  # 101 groups a row; N * 101 % 4 == 1
    print(f"[gpu] quantize ternary {N}x{K}, sampled rows", flush=True)
    g = wl.generator(70)
    w = wl.fp16_weights(g, N, K)
    packed, scales = lb.quantize(_dev16(w), "ternary")
    rows = np.unique(np.concatenate([[0, 1, N // 2, N - 2, N - 1], wl.generator(71).integers(0, N, 40)]))
    p_ref, s_ref, _ = _expect(w[rows], "ternary")
    assert np.array_equal(packed[torch.from_numpy(rows).cuda()].cpu().numpy(), p_ref)
    assert np.array_equal(scales[torch.from_numpy(rows).cuda()].view(torch.int16).cpu().numpy().view(np.uint16),
                          s_ref)


@pytest.fixture
def quant_variant(lb, request):
    lb.force_variant(request.param)
    yield request.param
    lb.force_variant(None)


@pytest.mark.parametrize("quant_variant", ["quant-eighth", "quant-lane"], indirect=True)
def test_each_ternary_team_size(lb, quant_variant):
    """The ternary team sizes the automatic choice does not take (eight lanes
    per group, one lane per group; it takes two) on small, ragged, strided and
    hand-built inputs, with the non-finite count and guard bands."""
    print(f"[gpu] quantize ternary, {quant_variant}", flush=True)
    for (N, K), seed in zip([(1, 128), (3, 256), (7, 384), (33, 1152), (130, 3072), (257, 640)], range(6)):
        g = wl.generator(80 + seed)
        _check(lb, wl.fp16_weights(g, N, K, outliers=0.01), "ternary")
    full = wl.fp16_weights(wl.generator(86), 45, 640)
    w = _dev16(full)[:, :512]
    _check(lb, np.ascontiguousarray(full[:, :512]), "ternary", w_dev=w)
    with open(os.path.join(os.path.dirname(__file__), "golden", "quantize_groups.json")) as f:
        cases = json.load(f)["cases"]
    w = np.array([[int(h, 16) for n, h in c["w"] for _ in range(n)] for c in cases], dtype=np.uint16)
    p_ref, s_ref, bad_ref = _expect(w, "ternary")
    N, K = w.shape
    cnt = torch.empty(1, dtype=torch.int32, device="cuda")
    pbuf = torch.full((N * K // 4 + 4096,), 0xA5, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((N * K // 128 + 2048,), -7, dtype=torch.int16, device="cuda")
    wd = _dev16(w)
    st = lb.lib().lowbit_quantize(lb.TERNARY, wd.data_ptr(), N, K, K, pbuf.data_ptr() + 2048,
                                  sbuf.data_ptr() + 2048, cnt.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == lb.OK
    assert int(cnt.item()) == bad_ref
    ph, sh = pbuf.cpu().numpy(), sbuf.cpu().numpy()
    assert (ph[:2048] == 0xA5).all() and (ph[2048 + N * K // 4:] == 0xA5).all()
    assert np.array_equal(ph[2048:2048 + N * K // 4].reshape(N, K // 4), p_ref)
    assert (sh[:1024] == -7).all() and (sh[1024 + N * K // 128:] == -7).all()
    assert np.array_equal(sh[1024:1024 + N * K // 128].view(np.uint16).reshape(N, K // 128), s_ref)


def test_quantized_weights_feed_the_gemm(lb):
    """Quantise, then run the layer on the result: the output meets the
    tolerance against the oracle's product with the oracle's own (t, s)."""
    g = wl.generator(72)
    N, K, M = 512, 1024, 40
    w = wl.fp16_weights(g, N, K)
    x = wl.activations(g, M, K, "bf16")
    packed, scales = lb.quantize(_dev16(w), "ternary")
    xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    y = lb.gemm(xd, packed, scales, "ternary", out_dtype=torch.float32)
    t, s, _ = oracle.quantize(w, "ternary")
    s16 = s.view(np.float16)
    A = oracle.linear(x, "bf16", t, s16)
    Mg = oracle.magnitude(x, "bf16", t, s16)
    ok, worst, nfail = oracle.check(y.cpu().numpy().astype(np.float64), A, Mg, "f32")
    assert ok, (worst, nfail)
