"""GPU base-3 storage (five ternary values per byte): the packer, the unpacker
and the transcoder to INT2, bit-exact against the oracle; the GEMM on
transcoded weights against the oracle's linear."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import banner, dev_bits, oracle_linear, to_host64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lb():
    import bit_weight_gemm_int2_amd as b
    b.lib()
    return b


def _dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


# K = 1 .. 7 and other K mod 5 != 0 give a partial last byte; rows of
# ceil(K/5) bytes put most rows at an odd byte offset
@pytest.mark.parametrize("N,K,seed", [
    (1, 1, 0), (3, 2, 1), (2, 3, 2), (5, 4, 3), (4, 5, 4), (9, 7, 5), (2, 13, 6),
    (64, 128, 7), (77, 1001, 8), (300, 3072, 9), (3, 65541, 10),
])
def test_pack_base3_bit_exact(lb, N, K, seed):
    banner(f"base3 pack N={N} K={K}")
    t = wl.ternary_codes(wl.generator(seed), N, K, 0.35)
    p = lb.pack_base3(_dev(t))
    torch.cuda.synchronize()
    assert tuple(p.shape) == (N, (K + 4) // 5)
    assert np.array_equal(p.cpu().numpy(), oracle.pack_base3(t))


@pytest.mark.parametrize("N,K,seed", [(1, 1, 20), (7, 6, 21), (33, 130, 22), (128, 3072, 23), (5, 9217, 24)])
def test_unpack_base3_round_trip(lb, N, K, seed):
    banner(f"base3 unpack N={N} K={K}")
    t = wl.ternary_codes(wl.generator(seed), N, K, None)
    back, bad = lb.unpack("base3", _dev(oracle.pack_base3(t)), K)
    assert bad == 0 and np.array_equal(back.cpu().numpy(), t)


def test_unpack_base3_invalid_bytes(lb):
    banner("base3 unpack invalid bytes")
    N, K = 6, 33                                  # 7 bytes a row, last one holds 3 values
    t = wl.ternary_codes(wl.generator(25), N, K, 0.35)
    p = oracle.pack_base3(t)
    p[0, 0] = 243
    p[2, 3] = 255
    p[5, 6] = 250                                 # the partial last byte: 3 values
    ref_t, ref_bad = oracle.unpack_base3(p, K)
    back, bad = lb.unpack("base3", _dev(p), K)
    assert ref_bad == 13 and bad == ref_bad
    assert np.array_equal(back.cpu().numpy(), ref_t)


def test_pack_base3_reports_invalid_codes(lb):
    banner("base3 pack invalid codes")
    t = np.zeros((4, 23), dtype=np.int8)
    t[0, 0] = 2
    t[3, 22] = -7
    with pytest.raises(ValueError, match="2 code"):
        lb.pack_base3(_dev(t))
    # unchecked, an invalid value is stored as t = 0
    p = lb.pack_base3(_dev(t), check=False)
    torch.cuda.synchronize()
    assert np.array_equal(p.cpu().numpy(), oracle.pack_base3(np.zeros((4, 23), dtype=np.int8)))


@pytest.mark.parametrize("N,K,seed", [(1, 16, 30), (3, 80, 31), (5, 128, 32), (41, 1008, 33),
                                      (257, 3072, 34), (6, 9216, 35)])
def test_base3_to_int2_bit_exact(lb, N, K, seed):
    banner(f"base3 -> int2 N={N} K={K}")
    t = wl.ternary_codes(wl.generator(seed), N, K, 0.35)
    p = oracle.pack_base3(t)
    ref, ref_bad = oracle.base3_to_ternary(p, K)
    out = lb.base3_to_int2(_dev(p), K)
    torch.cuda.synchronize()
    assert ref_bad == 0
    assert np.array_equal(out.cpu().numpy(), ref)


def test_base3_to_int2_invalid_bytes(lb):
    banner("base3 -> int2 invalid bytes")
    N, K = 4, 48                                  # 10 bytes a row, last one holds 3 values
    t = wl.ternary_codes(wl.generator(36), N, K, 0.35)
    p = oracle.pack_base3(t)
    p[0, 0] = 249
    p[1, 3] = 243                                 # k = 15 .. 19: straddles two INT2 words
    p[3, 9] = 255
    ref, ref_bad = oracle.base3_to_ternary(p, K)
    assert ref_bad == 13
    with pytest.raises(ValueError, match="13 invalid"):
        lb.base3_to_int2(_dev(p), K)
    out = lb.base3_to_int2(_dev(p), K, check=False)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), ref)
    # the INT2 unpacker counts the same values again
    _, bad2 = lb.unpack("ternary", out, K)
    assert bad2 == 13


def test_sweep_shapes_sampled_rows(lb):
    """The three weight shapes of the 100-linear sweep at full size: every row
    transcoded on the device; sampled rows against the oracle."""
    g = wl.generator(37)
    for N, K in [(3072, 3072), (18432, 3072), (3072, 12288)]:
        banner(f"base3 full-size N={N} K={K}")
        t = wl.ternary_codes(g, N, K, 0.35)
        pb = lb.pack_base3(_dev(t))
        out = lb.base3_to_int2(pb, K)
        torch.cuda.synchronize()
        rows = np.sort(g.choice(N, size=48, replace=False))
        rows[0], rows[-1] = 0, N - 1
        p_ref = oracle.pack_base3(t[rows])
        assert np.array_equal(pb.cpu().numpy()[rows], p_ref)
        ref, _ = oracle.base3_to_ternary(p_ref, K)
        assert np.array_equal(out.cpu().numpy()[rows], ref)


@pytest.mark.parametrize("M,N,K", [(16, 520, 3072), (300, 640, 1024)])
def test_gemm_on_transcoded_weights(lb, M, N, K):
    banner(f"gemm on base3-transcoded weights M={M} N={N} K={K}")
    lin = wl.make_linear("base3", "ternary", M, N, K, seed=38)
    packed = lb.base3_to_int2(_dev(oracle.pack_base3(lin.codes)), K)
    s = _dev(lin.scales.view(np.int16)).view(torch.float16)
    y = lb.gemm(dev_bits(lin.x, "bf16"), packed, s, "ternary", out_dtype=torch.float32)
    torch.cuda.synchronize()
    A, Mg = oracle_linear(lin)
    ok, worst, nfail = oracle.check(to_host64(y), A, Mg, "f32")
    assert ok, (worst, nfail)


def test_gemm_rejects_base3_format(lb):
    x = torch.zeros((16, 128), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((16, 26), dtype=torch.uint8, device="cuda")
    s = torch.ones((16, 1), dtype=torch.float16, device="cuda")
    with pytest.raises(lb.LowbitError, match="format"):
        lb.gemm(x, w, s, "base3")
