"""GPU packer / unpacker: bit-exact against the oracle's packing."""
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


def _pack_dev(lb, fmt, t):
    c = torch.from_numpy(np.ascontiguousarray(t)).cuda()
    p = lb.pack_ternary(c) if fmt == "ternary" else lb.pack_binary(c)
    return p.cpu().numpy()


@pytest.mark.parametrize("fmt,N,K,seed", [
    ("ternary", 1, 16, 0), ("ternary", 3, 48, 1), ("ternary", 256, 256, 2), ("ternary", 77, 1152, 3),
    ("binary", 1, 32, 4), ("binary", 5, 96, 5), ("binary", 300, 640, 6),
])
def test_pack_bit_exact_small(lb, fmt, N, K, seed):
    g = wl.generator(seed)
    t = wl.ternary_codes(g, N, K, 0.35) if fmt == "ternary" else wl.binary_codes(g, N, K)
    ref = oracle.pack_ternary(t) if fmt == "ternary" else oracle.pack_binary(t)
    assert np.array_equal(_pack_dev(lb, fmt, t), ref)


def test_pack_bit_exact_workload_weights(lb):
    print("[gpu] pack: config weights", flush=True)
    c1 = wl.config1()
    assert np.array_equal(_pack_dev(lb, "ternary", c1.codes), oracle.pack_ternary(c1.codes))
    c2 = wl.config2()
    assert np.array_equal(_pack_dev(lb, "ternary", c2.codes), oracle.pack_ternary(c2.codes))
    for lin in wl.config4(16):
        assert np.array_equal(_pack_dev(lb, "binary", lin.codes), oracle.pack_binary(lin.codes))
    up, down = wl.config3()
    for lin in (up, down):
        assert np.array_equal(_pack_dev(lb, "ternary", lin.codes), oracle.pack_ternary(lin.codes))


def test_unpack_round_trip_and_invalid_codes(lb):
    g = wl.generator(12)
    t = wl.ternary_codes(g, 64, 512, None)
    p = torch.from_numpy(oracle.pack_ternary(t)).cuda()
    back, bad = lb.unpack("ternary", p, 512)
    assert bad == 0 and np.array_equal(back.cpu().numpy(), t)
    # plant invalid 2-bit fields (pattern 10) in the packed bytes
    pb = oracle.pack_ternary(t)
    pb[0, 0] = (pb[0, 0] & 0xFC) | 0b10
    pb[5, 17] = (pb[5, 17] & 0x3F) | 0b10000000
    pb[63, 127] = 0xAA
    ref_t, ref_bad = oracle.unpack_ternary(pb, 512)
    back, bad = lb.unpack("ternary", torch.from_numpy(pb).cuda(), 512)
    assert bad == ref_bad and np.array_equal(back.cpu().numpy(), ref_t)
    tb = wl.binary_codes(g, 33, 256)
    back, bad = lb.unpack("binary", torch.from_numpy(oracle.pack_binary(tb)).cuda(), 256)
    assert bad == 0 and np.array_equal(back.cpu().numpy(), tb)


def test_pack_reports_invalid_codes(lb):
    t = np.zeros((8, 64), dtype=np.int8)
    t[0, 3] = 2
    t[7, 63] = -5
    t[4, 10] = 127
    c = torch.from_numpy(t).cuda()
    with pytest.raises(ValueError, match="3 code"):
        lb.pack_ternary(c)
    tb = np.ones((4, 64), dtype=np.int8)
    tb[1, 1] = 0
    with pytest.raises(ValueError, match="1 code"):
        lb.pack_binary(torch.from_numpy(tb).cuda())
    # invalid entries are stored as t = 0 (ternary); the rest is unaffected
    p = lb.pack_ternary(c, check=False).cpu().numpy()
    t_fixed = t.copy()
    t_fixed[(t_fixed < -1) | (t_fixed > 1)] = 0
    assert np.array_equal(p, oracle.pack_ternary(t_fixed))


def test_pack_is_deterministic(lb):
    g = wl.generator(13)
    t = torch.from_numpy(wl.ternary_codes(g, 1000, 3072, 0.35)).cuda()
    a = lb.pack_ternary(t)
    b = lb.pack_ternary(t)
    assert torch.equal(a, b)
