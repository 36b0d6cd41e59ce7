"""Pins for the CPU oracle: values, closed forms and invariants that come from the
pages and from mathematics, not from the oracle itself. CPU only."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as wl


def _golden(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- packing ---

def test_ternary_pack_hand_literal(golden_dir):
    g = _golden(golden_dir, "ternary_pack_word.json")
    t = np.array([g["t"]], dtype=np.int8)
    p = oracle.pack_ternary(t)
    assert p.tobytes().hex() == g["packed_hex"]


def test_binary_pack_hand_literal(golden_dir):
    g = _golden(golden_dir, "binary_pack_word.json")
    t = -np.ones((1, g["K"]), dtype=np.int8)
    t[0, g["plus_positions"]] = 1
    assert oracle.pack_binary(t).tobytes().hex() == g["packed_hex"]


# which k (inside one 16-code word) each 2-bit field of each byte carries
_TERNARY_BYTE_K = {0: [0, 2, 4, 6], 1: [8, 10, 12, 14], 2: [1, 3, 5, 7], 3: [9, 11, 13, 15]}


@pytest.mark.parametrize("byte", [0, 1, 2, 3])
def test_ternary_every_valid_byte(byte):
    """All 3^4 = 81 valid contents of each byte position, against base-4 digits
    of the 2-bit two's-complement codes (0 -> 0, +1 -> 1, -1 -> 3)."""
    ks = _TERNARY_BYTE_K[byte]
    code = {0: 0, 1: 1, -1: 3}
    for v in range(81):
        tvals = [(v // 3 ** j) % 3 - 1 for j in range(4)]   # t in {-1, 0, 1}
        t = np.zeros((1, 16), dtype=np.int8)                 # code 0 elsewhere
        for k, tv in zip(ks, tvals):
            t[0, k] = tv
        p = oracle.pack_ternary(t)[0]
        expect = sum(code[tv] << (2 * j) for j, tv in enumerate(tvals))
        assert p[byte] == expect
        assert all(p[b] == 0 for b in range(4) if b != byte)
        # no field ever holds the invalid pattern 10
        assert all(((p[byte] >> (2 * j)) & 3) != 2 for j in range(4))


_BINARY_BYTE_K = {0: list(range(0, 16, 2)), 1: list(range(16, 32, 2)),
                  2: list(range(1, 16, 2)), 3: list(range(17, 32, 2))}


@pytest.mark.parametrize("byte", [0, 1, 2, 3])
def test_binary_every_byte(byte):
    ks = _BINARY_BYTE_K[byte]
    for v in range(256):
        t = -np.ones((1, 32), dtype=np.int8)
        for j, k in enumerate(ks):
            if (v >> j) & 1:
                t[0, k] = 1
        p = oracle.pack_binary(t)[0]
        assert p[byte] == v
        assert all(p[b] == 0 for b in range(4) if b != byte)


def test_pack_unpack_round_trip():
    g = wl.generator(11)
    for N, K in [(1, 16), (3, 128), (17, 384), (64, 1024)]:
        t = wl.ternary_codes(g, N, K, 0.35)
        p = oracle.pack_ternary(t)
        assert p.shape == (N, K // 4) and p.dtype == np.uint8
        back, bad = oracle.unpack_ternary(p, K)
        assert bad == 0 and np.array_equal(back, t)
    for N, K in [(1, 32), (5, 128), (33, 2048)]:
        t = wl.binary_codes(g, N, K)
        p = oracle.pack_binary(t)
        assert p.shape == (N, K // 8)
        assert np.array_equal(oracle.unpack_binary(p, K), t)


def test_unpack_counts_invalid_code():
    p = np.full((2, 8), 0xFF, dtype=np.uint8)     # all fields 11 -> t = -1
    p[0, 0] = 0b11111110                           # k=0 field = 10 (invalid)
    p[1, 7] = 0b10111110                           # two invalid fields
    t, bad = oracle.unpack_ternary(p, 32)
    assert bad == 3
    assert t[0, 0] == 0 and t[0, 1] == -1
    assert set(np.unique(t)) <= {-1, 0}
    p2 = np.array([[0b01000100, 0, 0, 0]], dtype=np.uint8)   # fields (k=0,2,4,6) = 00,01,00,01
    t2, bad2 = oracle.unpack_ternary(p2, 16)
    assert bad2 == 0 and list(t2[0, 0:8:2]) == [0, 1, 0, 1]


def test_pack_rejects_out_of_set_codes():
    with pytest.raises(ValueError):
        oracle.pack_ternary(np.full((1, 16), 2, dtype=np.int8))
    with pytest.raises(ValueError):
        oracle.pack_binary(np.zeros((1, 32), dtype=np.int8))


# ------------------------------------------------------ base-3 storage ---

def test_base3_pack_hand_literal(golden_dir):
    g = _golden(golden_dir, "base3_pack.json")
    t = np.array([g["t"]], dtype=np.int8)
    assert oracle.pack_base3(t).tobytes().hex() == g["packed_hex"]
    back, bad = oracle.unpack_base3(oracle.pack_base3(t), t.shape[1])
    assert bad == 0 and np.array_equal(back, t)


def test_base3_every_byte_against_python_base3_parser():
    """All 3^5 = 243 valid bytes: the packer must agree with Python's own base-3
    integer parser (int(text, 3)) with the digit of the lowest k written last, and
    the unpacker with numpy's base_repr."""
    import itertools
    seen = set()
    for ts in itertools.product((-1, 0, 1), repeat=5):
        t = np.array([ts], dtype=np.int8)
        b = int(oracle.pack_base3(t)[0, 0])
        text = "".join(str(v + 1) for v in reversed(ts))     # most significant first
        assert b == int(text, 3)
        seen.add(b)
    assert seen == set(range(243))
    for b in range(243):
        text = np.base_repr(b, 3).rjust(5, "0")
        expect = [int(ch) - 1 for ch in reversed(text)]
        t, bad = oracle.unpack_base3(np.array([[b]], dtype=np.uint8), 5)
        assert bad == 0 and list(t[0]) == expect


def test_base3_ragged_rows_and_padding():
    g = wl.generator(13)
    for N, K in [(1, 1), (2, 2), (3, 3), (1, 4), (4, 5), (3, 7), (5, 128), (2, 3072), (7, 1001)]:
        t = wl.ternary_codes(g, N, K, 0.35)
        p = oracle.pack_base3(t)
        assert p.shape == (N, -(-K // 5)) and p.dtype == np.uint8
        assert oracle.packed_bytes("base3", N, K) == p.size
        back, bad = oracle.unpack_base3(p, K)
        assert bad == 0 and np.array_equal(back, t)
        r = K % 5
        if r:   # the last byte holds r digits, so it stays below 3^r
            assert (p[:, -1].astype(int) < 3 ** r).all()
    # an all-zero row: every full byte is 11111 in base 3 = 121
    z = oracle.pack_base3(np.zeros((1, 13), dtype=np.int8))
    assert list(z[0]) == [121, 121, 1 + 3 + 9]


def test_base3_invalid_bytes_decode_to_zero_and_count():
    p = np.array([[121, 243, 255, 0]], dtype=np.uint8)        # K = 18: last byte holds 3
    t, bad = oracle.unpack_base3(p, 18)
    assert bad == 10
    assert list(t[0, 5:15]) == [0] * 10
    assert list(t[0, :5]) == [0] * 5 and list(t[0, 15:]) == [-1, -1, -1]
    p2 = np.array([[0, 0, 250]], dtype=np.uint8)             # K = 12: invalid last byte, 2 weights
    assert oracle.unpack_base3(p2, 12)[1] == 2
    with pytest.raises(ValueError):
        oracle.pack_base3(np.full((1, 5), 2, dtype=np.int8))


def test_base3_to_ternary_matches_int2_packing():
    g = wl.generator(14)
    for N, K in [(1, 16), (3, 80), (4, 128), (9, 3072), (2, 1008)]:
        t = wl.ternary_codes(g, N, K, 0.35)
        int2, bad = oracle.base3_to_ternary(oracle.pack_base3(t), K)
        assert bad == 0 and np.array_equal(int2, oracle.pack_ternary(t))
    # an invalid base-3 byte becomes the invalid INT2 pattern 10 at its five weights
    t = np.zeros((1, 16), dtype=np.int8)
    p = oracle.pack_base3(t)
    p[0, 1] = 250                                             # k = 5 .. 9
    int2, bad = oracle.base3_to_ternary(p, 16)
    assert bad == 5
    back, bad2 = oracle.unpack_ternary(int2, 16)
    assert bad2 == 5 and not back.any()
    word = int.from_bytes(int2[0].tobytes(), "little")
    for k in range(16):
        field = (word >> (16 * (k & 1) + 2 * (k >> 1))) & 3
        assert field == (2 if 5 <= k <= 9 else 0)
    with pytest.raises(ValueError):
        oracle.base3_to_ternary(oracle.pack_base3(np.zeros((1, 20), dtype=np.int8)), 20)


def test_base3_storage_rate():
    # 1.6 bits per ternary value for long rows, plus the 16/128 bits of scale:
    # within 0.02 of the 1.71 bits per weight the pages print as the ternary rate,
    # against 2.125 for the INT2 storage.
    N, K = 3072, 3072
    bits = (oracle.packed_bytes("base3", N, K) + oracle.scale_bytes(N, K)) * 8 / (N * K)
    assert abs(bits - 1.71) < 0.02 and bits < 2.125
    assert oracle.packed_bytes("base3", N, K) == N * 615


# -------------------------------------------------------- storage / bits ---

def test_storage_sizes_exact():
    for N, K in [(3072, 3072), (9216, 3072), (3072, 9216), (18432, 3072), (3072, 12288)]:
        assert oracle.packed_bytes("ternary", N, K) * 8 == 2 * N * K
        assert oracle.packed_bytes("binary", N, K) * 8 == N * K
        assert oracle.scale_bytes(N, K) == 2 * N * K // 128
        t = np.zeros((2, K), dtype=np.int8)
        assert oracle.pack_ternary(t).nbytes == 2 * K // 4
        assert oracle.pack_binary(t + 1 - 2 * (t == 0)).nbytes == 2 * K // 8


def test_effective_bits_match_printed_values():
    # Binary: 1 bit + 16/128 bits of scale = 1.125 (printed on "Bonsai Image 4B 1-bit
    # untuk pembuatan gambar di perangkat lokal", section on the two variants, and in
    # "量化数学" of "Introducing 1-bit and Ternary Bonsai Image 4B"). Storage of this
    # library is the same.
    N, K = 3072, 3072
    bits_bin = (oracle.packed_bytes("binary", N, K) + oracle.scale_bytes(N, K)) * 8 / (N * K)
    assert bits_bin == 1.125
    # Ternary information rate log2(3) + 16/128 ~= 1.71 (printed), and INT2 storage
    # is 2 + 16/128 = 2.125 bits (2 bits per ternary: "Cómo Bonsai Ternary 4B revoluciona
    # la difusión texto-imagen", section "Representación y almacenamiento de los pesos
    # ternarios").
    assert round(math.log2(3) + 16 / 128, 2) == 1.71
    bits_tern = (oracle.packed_bytes("ternary", N, K) + oracle.scale_bytes(N, K)) * 8 / (N * K)
    assert bits_tern == 2.125
    # Layer-level reductions printed in "量化数学" of "Introducing 1-bit and Ternary Bonsai
    # Image 4B": 16/1.125 ~ 14x, 16/1.71 ~ 9.4x
    assert round(16 / 1.125) == 14
    assert round(16 / 1.71, 1) == 9.4


def test_generated_code_entropy():
    g = wl.generator(5)
    t = wl.ternary_codes(g, 512, 4096, None)
    p = np.array([(t == v).mean() for v in (-1, 0, 1)])
    H = -(p * np.log2(p)).sum()
    assert abs(H - math.log2(3)) < 1e-3
    t = wl.ternary_codes(g, 512, 4096, 0.35)
    assert abs((t == 0).mean() - 0.35) < 3e-3
    assert set(np.unique(t)) == {-1, 0, 1}


# ------------------------------------------------------- dequant / GEMM ---

def test_dequantize_closed_form():
    t = np.array([[1, 0, -1] * 128], dtype=np.int8)[:, :256]
    s = np.array([[0.5, -3.0]], dtype=np.float16)
    W = oracle.dequantize(t, s)
    assert W[0, 0] == 0.5 and W[0, 1] == 0 and W[0, 2] == -0.5
    assert np.all(W[0, 128:][t[0, 128:] == 1] == -3.0)
    assert np.all(W[0, 128:][t[0, 128:] == -1] == 3.0)
    # subnormal fp16 scale survives exactly
    s2 = np.array([[np.float16(2.0 ** -24), 0.0]], dtype=np.float16)
    W2 = oracle.dequantize(t, s2)
    assert W2[0, 0] == 2.0 ** -24 and np.all(W2[0, 128:] == 0)


def test_worked_example(golden_dir):
    g = _golden(golden_dir, "worked_linear.json")
    K = 128
    x = np.zeros((2, K), dtype=np.float32)
    x[0] = 1.0
    x[1, 0::2] = 0.5
    x[1, 1::2] = -0.25
    t = np.zeros((3, K), dtype=np.int8)
    t[0, :64] = 1
    t[0, 64:] = -1
    t[1, 5], t[1, 6] = 1, -1
    t[2, 0::2] = 1
    s = np.array([[0.25], [2.0], [0.125]], dtype=np.float16)
    b = np.array([1.0, -1.0, 0.5], dtype=np.float16)
    for xd in ("f16", "bf16"):
        xb = wl.to_bits(x, xd)
        A = oracle.linear(xb, xd, t, s, b)
        assert np.array_equal(A, np.array(g["Y"]))
        assert np.array_equal(oracle.magnitude(xb, xd, t, s, b), np.array(g["Mag"]))
        for yd in ("f16", "bf16", "f32"):
            assert np.array_equal(oracle.decode(oracle.encode(A, yd), yd), A)


def _exact(xb, xd, t, s, b):
    """Exact rational value of one output element via fractions (brute force)."""
    X = oracle.decode(xb, xd)
    S = s.astype(np.float64)
    M, K = X.shape
    N = t.shape[0]
    out = np.empty((M, N), dtype=object)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += Fraction(float(X[m, k])) * Fraction(float(S[n, k // 128])) * int(t[n, k])
            if b is not None:
                acc += Fraction(float(b[n]))
            out[m, n] = acc
    return out


@pytest.mark.parametrize("xd", ["f16", "bf16"])
@pytest.mark.parametrize("K", [128, 256])
def test_linear_against_exact_rationals(xd, K):
    g = wl.generator(21 + K)
    M, N = 3, 4
    xb = wl.activations(g, M, K, xd, std=3.0)
    t = wl.ternary_codes(g, N, K, 0.35)
    s = wl.group_scales(g, N, K)
    b = wl.bias_f16(g, N)
    A = oracle.linear(xb, xd, t, s, b)
    E = _exact(xb, xd, t, s, b)
    Mg = oracle.magnitude(xb, xd, t, s, b)
    for m in range(M):
        for n in range(N):
            err = abs(Fraction(float(A[m, n])) - E[m, n])
            assert err <= Fraction(K * 2.0 ** -52) * Fraction(float(Mg[m, n]))
    # sum|x w| against brute force too
    X = oracle.decode(xb, xd)
    W = s.astype(np.float64).repeat(128, axis=1) * t
    for m in range(M):
        for n in range(N):
            ref = math.fsum(abs(X[m, k] * W[n, k]) for k in range(K)) + abs(float(b[n]))
            assert abs(Mg[m, n] - ref) <= 1e-12 * ref


def test_special_cases():
    g = wl.generator(7)
    M, N, K = 5, 6, 256
    xb = wl.activations(g, M, K, "bf16")
    X = oracle.decode(xb, "bf16")
    b = wl.bias_f16(g, N)
    s = wl.group_scales(g, N, K)
    # t == 0 -> Y = bias exactly
    A = oracle.linear(xb, "bf16", np.zeros((N, K), np.int8), s, b)
    assert np.array_equal(A, np.broadcast_to(b.astype(np.float64), (M, N)))
    # identity codes, unit scales -> selection of the first N columns of X
    t = np.zeros((N, K), np.int8)
    t[np.arange(N), np.arange(N)] = 1
    A = oracle.linear(xb, "bf16", t, np.ones((N, K // 128), np.float16))
    assert np.array_equal(A, X[:, :N])
    # all +1 -> s * row sum per group; binary all -1 -> minus that
    ones = np.ones((N, K), np.int8)
    A = oracle.linear(xb, "bf16", ones, s)
    G = X.reshape(M, K // 128, 128).sum(axis=2)        # per-group row sums
    R = G @ s.astype(np.float64).T
    assert np.allclose(A, R, rtol=1e-13, atol=1e-13)
    A2 = oracle.linear(xb, "bf16", -ones, s)
    assert np.allclose(A2, -R, rtol=1e-13, atol=1e-13)
    # doubling every scale doubles the output exactly
    t = wl.ternary_codes(g, N, K, 0.35)
    A1 = oracle.linear(xb, "bf16", t, s)
    A2 = oracle.linear(xb, "bf16", t, (s.astype(np.float32) * 2).astype(np.float16))
    assert np.array_equal(A2, 2 * A1)
    # a group whose scale is zero contributes nothing
    s0 = s.copy()
    s0[:, 1] = 0
    A0 = oracle.linear(xb, "bf16", t, s0)
    A_first = oracle.linear(xb[:, :128].copy(), "bf16", t[:, :128], s[:, :1])
    assert np.allclose(A0, A_first, rtol=1e-13, atol=1e-13)


def test_f32_gemm_meets_the_bound():
    """An FP32-accumulated GEMM of the dequantised weights (what the method
    specifies) lands inside the tolerance around the near-exact oracle value."""
    g = wl.generator(9)
    M, N, K = 64, 96, 3072
    xb = wl.activations(g, M, K, "bf16")
    t = wl.ternary_codes(g, N, K, 0.35)
    s = wl.group_scales(g, N, K)
    A = oracle.linear(xb, "bf16", t, s)
    Mg = oracle.magnitude(xb, "bf16", t, s)
    X32 = oracle.decode(xb, "bf16").astype(np.float32)
    W32 = oracle.dequantize(t, s).astype(np.float32)
    Y32 = (X32 @ W32.T).astype(np.float64)
    ok, worst, _ = oracle.check(Y32, A, Mg, "f32")
    assert ok and worst < 0.1


# --------------------------------------------------- rounding / tolerance ---

def test_bf16_rounding_literals(golden_dir):
    for val, hexbits, _why in _golden(golden_dir, "bf16_rounding.json")["cases"]:
        got = oracle.encode(np.array([float(val)]), "bf16")[0]
        assert got == int(hexbits, 16), (val, hex(got), hexbits)


def test_f16_rounding_matches_numpy():
    g = wl.generator(3)
    v = np.concatenate([
        g.standard_normal(20000) * 10.0 ** g.integers(-9, 5, 20000),
        (np.arange(-2000, 2000) + 0.5) * 2.0 ** -24,          # ties in the subnormal range
        np.array([65504.0, 65519.99, 65520.0, -65520.0, 0.0, -0.0]),
    ])
    mine = oracle.encode(v, "f16")
    ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(mine, ref)


def test_bf16_rounding_matches_f32_route_on_f32_values():
    # For values already in float32 the direct rounding equals the usual
    # add-0x7FFF-plus-lsb bit trick on the float32 pattern.
    g = wl.generator(4)
    v = (g.standard_normal(50000) * 10.0 ** g.integers(-30, 30, 50000)).astype(np.float32)
    u = v.view(np.uint32).astype(np.uint64)
    trick = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    assert np.array_equal(oracle.encode(v.astype(np.float64), "bf16"), trick)


def test_ulp_values():
    assert oracle.ulp(np.array([1.0]), "bf16")[0] == 2.0 ** -7
    assert oracle.ulp(np.array([1.0]), "f16")[0] == 2.0 ** -10
    assert oracle.ulp(np.array([0.0]), "f16")[0] == 2.0 ** -24
    assert oracle.ulp(np.array([3.0]), "bf16")[0] == 2.0 ** -6


def test_gelu_table_values(golden_dir):
    for x, y in _golden(golden_dir, "gelu_values.json")["cases"]:
        assert abs(oracle.gelu(np.array([x]))[0] - y) <= 1e-15 * max(1.0, abs(y))
    x = np.linspace(-6, 6, 101)
    assert np.allclose(oracle.gelu(-x), oracle.gelu(x) - x, atol=1e-14)


def test_check_detects_planted_errors():
    g = wl.generator(8)
    M, N, K = 8, 16, 256
    xb = wl.activations(g, M, K, "bf16")
    t = wl.ternary_codes(g, N, K, 0.35)
    s = wl.group_scales(g, N, K)
    A = oracle.linear(xb, "bf16", t, s)
    Mg = oracle.magnitude(xb, "bf16", t, s)
    Y = oracle.decode(oracle.encode(A, "bf16"), "bf16")
    assert oracle.check(Y, A, Mg, "bf16")[0]
    # a dropped term, a flipped sign or a transposed operand must all fail
    t_drop = t.copy()
    t_drop[:, 0] = 0
    t_drop[t[:, 0] == 0, 0] = 1
    for wrong in (oracle.linear(xb, "bf16", t_drop, s), -A, A + 0.01 * Mg):
        assert not oracle.check(wrong, A, Mg, "f32")[0]
    Ynan = Y.copy()
    Ynan[0, 0] = np.nan
    assert not oracle.check(Ynan, A, Mg, "bf16")[0]


# ------------------------------------------------------- 4-bit with zero point ---

def test_int4_pack_hand_literal(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "int4_pack_word.json")))
    q = np.array([g["q"]], dtype=np.uint8)
    assert oracle.pack_int4(q).tobytes().hex() == g["packed_hex"]


def test_int4_every_code_at_every_position_by_byte_and_nibble():
    """Byte B of a word holds the codes of two k in its two nibbles: with bit
    position p = 16h + 4i for k = 2i + h, byte B = p // 8 and nibble (p % 8) // 4,
    so the low nibble of byte B is k = 4 (B % 2) + B // 2 and the high nibble
    k = 4 (B % 2) + 2 + B // 2. Every code value at every position."""
    for v in range(16):
        for j in range(8):
            q = np.zeros((1, 8), dtype=np.uint8)
            q[0, j] = v
            b = oracle.pack_int4(q)[0]
            for B in range(4):
                lo_k, hi_k = 4 * (B % 2) + B // 2, 4 * (B % 2) + 2 + B // 2
                assert b[B] & 15 == q[0, lo_k] and b[B] >> 4 == q[0, hi_k], (v, j, B)


def test_int4_round_trip_and_rejects_out_of_range():
    g = np.random.default_rng(7)
    q = g.integers(0, 16, size=(5, 256), dtype=np.uint8)
    p = oracle.pack_int4(q)
    assert p.shape == (5, 128)
    assert np.array_equal(oracle.unpack_int4(p, 256), q)
    with pytest.raises(ValueError):
        oracle.pack_int4(np.full((1, 8), 16, dtype=np.uint8))
    with pytest.raises(ValueError):
        oracle.pack_int4(np.zeros((1, 12), dtype=np.uint8))


def test_int4_dequantize_closed_forms():
    q = np.tile(np.arange(16, dtype=np.uint8), (3, 8))          # [3, 128]
    # z = q's own integer value -> w = 0 where q == z; s = 1, z = 0 -> w = q
    s1 = np.ones((3, 1), dtype=np.float16)
    z0 = np.zeros((3, 1), dtype=np.float16)
    assert np.array_equal(oracle.dequantize_int4(q, s1, z0), q.astype(np.float64))
    z7 = np.full((3, 1), 7.0, dtype=np.float16)
    W = oracle.dequantize_int4(q, s1, z7)
    assert (W[q == 7] == 0).all() and W.min() == -7.0 and W.max() == 8.0
    # a subnormal scale and a non-integer zero point stay exact
    s_sub = np.full((3, 1), 2.0 ** -24, dtype=np.float16)
    zf = np.full((3, 1), 7.5, dtype=np.float16)
    W = oracle.dequantize_int4(q, s_sub, zf)
    assert np.array_equal(W, (q.astype(np.float64) - 7.5) * 2.0 ** -24)


def test_int4_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "int4_worked_linear.json")))
    k = np.arange(128)
    q = np.stack([np.full(128, 5), k % 16]).astype(np.uint8)
    x = np.stack([np.ones(128), np.where(k < 16, 2.0, 0.0)]).astype(np.float32)
    xb = wl.to_bits(x, "bf16")
    A = oracle.linear_int4(xb, "bf16", q, np.array(g["scales"], np.float16), np.array(g["zeros"], np.float16))
    assert np.array_equal(A, np.array(g["Y"]))


@pytest.mark.parametrize("K", [128, 256])
def test_int4_linear_against_exact_rationals(K):
    g = np.random.default_rng(K)
    M, N = 3, 4
    xb = wl.activations(np.random.Generator(np.random.PCG64(K)), M, K, "bf16")
    q = g.integers(0, 16, size=(N, K), dtype=np.uint8)
    s = (np.abs(g.standard_normal((N, K // 128))) * 0.01 + 1e-3).astype(np.float16)
    z = (7.5 + g.standard_normal((N, K // 128))).astype(np.float16)
    A = oracle.linear_int4(xb, "bf16", q, s, z)
    X = oracle.decode(xb, "bf16")
    for m in range(M):
        for n in range(N):
            exact = sum(Fraction(float(X[m, kk])) * Fraction(float(s[n, kk // 128])) *
                        (Fraction(int(q[n, kk])) - Fraction(float(z[n, kk // 128]))) for kk in range(K))
            assert abs(Fraction(A[m, n]) - exact) <= abs(exact) * Fraction(2) ** -45 + Fraction(2) ** -60


# -------------------------------------------------------------- quantiser ---

def _runs(runs):
    return [v for n, v in runs for _ in range(n)]


def test_quantize_hand_cases(golden_dir):
    """Hand-derived groups: the threshold (strict, with an exact tie), the kept
    mean and its rounding (both kinds of midpoint), zero and subnormal means,
    signed zeros, non-finite weights."""
    g = _golden(golden_dir, "quantize_groups.json")
    for case in g["cases"]:
        w = np.array([[int(h, 16) for h in _runs(case["w"])]], dtype=np.uint16)
        t, s, bad = oracle.quantize(w, case["fmt"])
        assert t[0].tolist() == _runs(case["t"]), case["name"]
        assert int(s[0, 0]) == int(case["s_hex"], 16), case["name"]
        assert bad == case["nonfinite"], case["name"]


def _f16_nearest_exact(q: Fraction) -> int:
    """FP16 bits of the value nearest the non-negative rational q (ties to an
    even bit pattern), by bisection over the ordered finite FP16 values."""
    lo, hi = 0, 0x7BFF
    val = lambda b: Fraction(float(np.array(b, dtype=np.uint16).view(np.float16)))
    if q >= val(hi):
        return hi
    while hi - lo > 1:                      # val(lo) <= q < val(hi)
        mid = (lo + hi) // 2
        if val(mid) <= q:
            lo = mid
        else:
            hi = mid
    dl, dh = q - val(lo), val(hi) - q
    if dl != dh:
        return lo if dl < dh else hi
    return lo if lo % 2 == 0 else hi


@pytest.mark.parametrize("fmt", ["ternary", "binary"])
def test_quantize_against_exact_rationals(fmt):
    """Random groups (normal, with outliers, many exact zeros, subnormal) against
    the rule carried out in exact rational arithmetic with a brute-force FP16
    rounding."""
    g = wl.generator(31)
    rows = [wl.fp16_weights(g, 3, 256), wl.fp16_weights(g, 3, 256, outliers=0.05),
            wl.fp16_weights(g, 2, 256, std=1e-6)]
    z = wl.fp16_weights(g, 2, 256)
    z[:, ::3] = 0
    rows.append(z)
    w = np.concatenate(rows)
    t, s, bad = oracle.quantize(w, fmt)
    assert bad == 0
    vals = w.view(np.float16).astype(np.float64)
    for n in range(w.shape[0]):
        for gi in range(2):
            grp = [Fraction(float(v)) for v in vals[n, 128 * gi:128 * gi + 128]]
            total = sum(abs(v) for v in grp)
            if fmt == "ternary":
                keep = [abs(v) > Fraction(7, 10) * total / 128 for v in grp]
                kept = [abs(v) for v, k in zip(grp, keep) if k]
                mean = sum(kept) / len(kept) if kept else Fraction(0)
                expect_t = [(1 if v > 0 else -1) if k else 0 for v, k in zip(grp, keep)]
            else:
                mean = total / 128
                expect_t = [1 if v >= 0 else -1 for v in grp]
            assert int(s[n, gi]) == _f16_nearest_exact(mean)
            assert t[n, 128 * gi:128 * gi + 128].tolist() == expect_t


@pytest.mark.parametrize("fmt", ["ternary", "binary"])
def test_quantize_recovers_quantised_weights(fmt):
    """Weights that already are s * t (FP16 s per group) come back unchanged:
    ternary keeps exactly the non-zero ones (|w| = s > 0.7 * p s for a non-zero
    fraction p <= 1), binary's mean|w| is s."""
    g = wl.generator(32)
    N, K = 6, 512
    t0 = wl.ternary_codes(g, N, K, 0.35) if fmt == "ternary" else wl.binary_codes(g, N, K)
    s0 = wl.group_scales(g, N, K, offset=1e-3)
    w = (np.repeat(s0.astype(np.float64), 128, axis=1) * t0).astype(np.float16).view(np.uint16)
    t, s, bad = oracle.quantize(w, fmt)
    assert bad == 0 and np.array_equal(t, t0) and np.array_equal(s, s0.view(np.uint16))


def test_quantize_invariants():
    """Scaling by a power of two scales s and keeps t; negation flips t and keeps
    s (ternary; binary away from zero)."""
    g = wl.generator(33)
    w = wl.fp16_weights(g, 4, 384, std=0.5)
    wf = w.view(np.float16)
    for fmt in ("ternary", "binary"):
        t, s, _ = oracle.quantize(w, fmt)
        t2, s2, _ = oracle.quantize((wf * np.float16(4)).view(np.uint16), fmt)
        assert np.array_equal(t2, t)
        assert np.array_equal(s2.view(np.float16), s.view(np.float16) * np.float16(4))
        tn, sn, _ = oracle.quantize((-wf).view(np.uint16), fmt)
        assert np.array_equal(sn, s)
        nz = wf != 0
        assert np.array_equal(tn[nz], -t[nz])


def test_quantize_planted_rule_changes_are_caught(golden_dir):
    """The hand cases fail a threshold taken with >= and a mean over the whole
    group instead of the kept weights (mistakes planted in a copy of the rule)."""
    g = _golden(golden_dir, "quantize_groups.json")
    tie = next(c for c in g["cases"] if c["name"] == "ternary: tie at the threshold")
    w = np.array([[int(h, 16) for h in _runs(tie["w"])]], dtype=np.float16)
    a = np.abs(w.view(np.uint16).view(np.float16).astype(np.float64))
    total = a.sum()
    keep_ge = 1280.0 * a >= 7.0 * total                      # planted: >= instead of >
    assert keep_ge.sum() != sum(n for n, v in tie["t"] if v != 0)
    first = g["cases"][0]
    w1 = np.array([int(h, 16) for h in _runs(first["w"])], dtype=np.uint16).view(np.float16).astype(np.float64)
    whole_mean = oracle.encode(np.array([np.abs(w1).mean()]), "f16")[0]   # planted: mean of all
    assert int(whole_mean) != int(first["s_hex"], 16)


def test_linear_f32_form():
    """The FP32-BLAS form of the layer: bit-equal to the float64 one where every
    partial sum is exact in FP32 (small integers, power-of-two scales), and
    inside the tolerance elsewhere."""
    g = wl.generator(34)
    M, N, K = 6, 10, 256
    xi = g.integers(-8, 9, size=(M, K)).astype(np.float32)
    xb = wl.to_bits(xi, "bf16")
    t = wl.ternary_codes(g, N, K, 0.35)
    s = np.ldexp(1.0, g.integers(-3, 3, size=(N, K // 128))).astype(np.float16)
    b = np.ldexp(1.0, g.integers(-2, 2, size=N)).astype(np.float16)
    assert np.array_equal(oracle.linear_f32(xb, "bf16", t, s, b).astype(np.float64),
                          oracle.linear(xb, "bf16", t, s, b))
    lin = wl.make_linear("f32form", "ternary", 32, 64, 1024, seed=35)
    A = oracle.linear(lin.x, lin.x_dtype, lin.codes, lin.scales)
    Mg = oracle.magnitude(lin.x, lin.x_dtype, lin.codes, lin.scales)
    A32 = oracle.linear_f32(lin.x, lin.x_dtype, lin.codes, lin.scales).astype(np.float64)
    assert oracle.check(A32, A, Mg, "f32")[0]
