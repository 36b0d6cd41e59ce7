"""Plain CPU oracle for the low-bit-weight linear layer.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import or call this
module: only the tests, the package smoke check and the benchmark's CPU-baseline
leg use it. It shares no code with the GPU library.

What it computes, and where the pages say so
---------------------------------------------
* Weight definition (page "Cómo Bonsai Ternary 4B revoluciona la difusión
  texto-imagen", section "Representación y almacenamiento de los pesos
  ternarios"): each weight is ``w = scale_g * t`` with ``t`` in {-1, 0, +1} and one
  FP16 scale shared by every group of 128 weights; the CUDA deployment stores
  ``t`` with 2 bits per ternary value (INT2).
* Binary variant (page "Bonsai Image 4B 1-bit untuk pembuatan gambar di
  perangkat lokal", section on the two variants; page "Introducing 1-bit and
  Ternary Bonsai Image 4B", section "量化数学"): ``t`` in {-1, +1}, same FP16 group
  scale, 1 bit per weight plus 16/128 bits of scale = 1.125 bits per weight.
* The layer computes ``Y = X W^T (+ bias)``. The oracle dequantises W exactly and
  forms the matrix product in float64, which for these operands is the exact real
  result up to a relative error of about K * 2^-53 (every product
  ``x * s * t`` is exact in float64: 8 or 11 significand bits times 11 bits).

Readings where the pages are silent (each is listed in the design notes):
* INT2 code of a ternary value: the 2-bit two's complement of t, ``c = t & 3``:
  0 -> 00, +1 -> 01, -1 -> 11; the pattern 10 is invalid.
* Bit order: a packed row is a sequence of little-endian 32-bit words. Ternary:
  word ``u`` holds k = 16u .. 16u+15; the code of k = 16u + 2i + h (i in 0..7,
  h in {0, 1}) sits at bits [16h + 2i, 16h + 2i + 1]. Even k fill the low half
  word, odd k the high half word. Binary: word ``u`` holds k = 32u .. 32u+31; the
  bit of k = 32u + 2i + h (i in 0..15) sits at bit 16h + i; bit 1 means +1.
* Base-3 storage (five ternary values per byte, the form that approaches the
  information rate the pages quote): digit ``d = t + 1``, byte ``j`` holds
  k = 5j .. 5j+4 with ``d[5j]`` least significant, rows of ceil(K/5) bytes; bytes
  243 .. 255 are invalid. The pages print no such layout; see the section
  "Base-3 storage" below.
* Quantiser (FP16 weights -> t and s): the pages name BinaryConnect and Ternary
  Weight Networks (page "cuantificación de modelos de difusión para inferencia
  local en dispositivos edge", section "Fundamentos Teóricos") but do not say
  how the released weights were quantised. ``quantize`` applies those two rules
  per 128-group; it is pinned to the rules' own definition (hand-derived groups,
  exact rationals, round trips), and its agreement with the pages' actual
  quantiser is parity unpinned.
* Groups run along K inside one output row; K must be a multiple of 128.
* The bias, when present, is added once in the output row sum.
* Output cast: round to nearest, ties to even.

Parity: the GPU result must satisfy, per element,
``|Y - A| <= 1e-3 * sum_k |x_k w_k| + 1e-5`` (the stated tolerance; the bias
magnitude joins the sum as one more term), plus half an output ulp when the
output type is fp16 or bf16, and non-finite values must match in place.
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np

GROUP = 128

# ---------------------------------------------------------------------------
# 16-bit float formats: decode exactly, encode with round-to-nearest-even
# ---------------------------------------------------------------------------

# (significand bits incl. the implicit one, minimum normal exponent, maximum finite)
_FORMATS = {
    "f16": (11, -14, 65504.0),
    "bf16": (8, -126, float(np.float32(3.3895313892515355e38))),
}


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """16-bit pattern -> float64 (exact). ``dtype`` 'f16', 'bf16' or 'f32' (32-bit bits)."""
    bits = np.asarray(bits)
    if dtype == "f16":
        return bits.astype(np.uint16).view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return bits.astype(np.uint32).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to the nearest value of ``dtype`` (ties to even).

    Returns float64 values that are exactly representable in ``dtype``; overflow
    past the largest finite value (by half an ulp or more) gives +-inf.
    """
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    p, emin, fmax = _FORMATS[dtype]
    out = np.array(x, dtype=np.float64, copy=True)
    fin = np.isfinite(x) & (x != 0)
    v = x[fin]
    _, e = np.frexp(v)                       # v = m * 2^e, 0.5 <= |m| < 1
    # exponent of the leading bit is e-1; quantum = 2^(e-1-(p-1)) but never below
    # the subnormal spacing 2^(emin-(p-1))
    q_exp = np.maximum(e - p, emin - (p - 1))
    q = np.ldexp(1.0, q_exp)
    r = np.rint(v / q) * q                   # np.rint: ties to even; v/q exact (power of 2)
    # overflow: anything that rounded above the largest finite value. A value at
    # fmax + ulp/2 is a tie whose even neighbour is the next power of two, so it
    # also lands here and becomes inf, as round-to-nearest-even requires.
    big = np.abs(r) > fmax
    r[big] = np.copysign(np.inf, r[big])
    out[fin] = r
    return out


def encode(x: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> bit pattern of ``dtype`` after round-to-nearest-even."""
    r = round_to(x, dtype)
    if dtype == "f16":
        return r.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        f = r.astype(np.float32)             # exact: r is a bf16 value
        u = f.view(np.uint32)
        out = (u >> 16).astype(np.uint16)
        nan = np.isnan(r)
        out[nan] = 0x7FC0
        return out
    if dtype == "f32":
        return r.astype(np.float32).view(np.uint32)
    raise ValueError(dtype)


def ulp(v: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of ``dtype`` values at magnitude |v| (subnormal spacing near 0)."""
    v = np.abs(np.asarray(v, dtype=np.float64))
    if dtype == "f32":
        p, emin = 24, -126
    else:
        p, emin, _ = _FORMATS[dtype]
    with np.errstate(divide="ignore"):
        _, e = np.frexp(np.where(v > 0, v, 1.0))
    e = np.where(v > 0, e, emin + 1)
    return np.ldexp(1.0, np.maximum(e - p, emin - (p - 1)))


# ---------------------------------------------------------------------------
# Packing (the INT2 / 1-bit storage the pages describe, in this library's layout)
# ---------------------------------------------------------------------------

def pack_ternary(t: np.ndarray) -> np.ndarray:
    """int8 codes [N, K] in {-1,0,+1} -> uint8 [N, K/4] (2 bits per weight)."""
    t = np.asarray(t)
    N, K = t.shape
    if K % 16:
        raise ValueError("ternary packing needs K % 16 == 0")
    if not np.isin(t, (-1, 0, 1)).all():
        raise ValueError("ternary codes must lie in {-1, 0, +1}")
    c = (t.astype(np.int64) & 3).astype(np.uint32)          # 2-bit two's complement
    words = np.zeros((N, K // 16), dtype=np.uint32)
    for j in range(16):                                      # position inside the word
        i, h = divmod(j, 2)
        words |= c[:, j::16] << np.uint32(16 * h + 2 * i)
    return words.astype("<u4").view(np.uint8).reshape(N, K // 4)


def pack_binary(t: np.ndarray) -> np.ndarray:
    """int8 codes [N, K] in {-1,+1} -> uint8 [N, K/8] (1 bit per weight, 1 = +1)."""
    t = np.asarray(t)
    N, K = t.shape
    if K % 32:
        raise ValueError("binary packing needs K % 32 == 0")
    if not np.isin(t, (-1, 1)).all():
        raise ValueError("binary codes must lie in {-1, +1}")
    b = (t == 1).astype(np.uint32)
    words = np.zeros((N, K // 32), dtype=np.uint32)
    for j in range(32):
        i, h = divmod(j, 2)
        words |= b[:, j::32] << np.uint32(16 * h + i)
    return words.astype("<u4").view(np.uint8).reshape(N, K // 8)


def unpack_ternary(packed: np.ndarray, K: int) -> Tuple[np.ndarray, int]:
    """uint8 [N, K/4] -> (int8 codes [N, K], number of invalid 2-bit fields).

    A 2-bit field is read as a two's-complement number; the pattern 10 (-2) is
    invalid, decodes to 0 and is counted."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    N = packed.shape[0]
    words = packed.reshape(N, K // 4).view("<u4").astype(np.uint32)
    t = np.zeros((N, K), dtype=np.int8)
    invalid = 0
    for j in range(16):
        i, h = divmod(j, 2)
        c = ((words >> np.uint32(16 * h + 2 * i)) & np.uint32(3)).astype(np.int64)
        v = np.where(c >= 2, c - 4, c)                       # two's complement
        invalid += int((v == -2).sum())
        t[:, j::16] = np.where(v == -2, 0, v).astype(np.int8)
    return t, invalid


def unpack_binary(packed: np.ndarray, K: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    N = packed.shape[0]
    words = packed.reshape(N, K // 8).view("<u4").astype(np.uint32)
    t = np.zeros((N, K), dtype=np.int8)
    for j in range(32):
        i, h = divmod(j, 2)
        b = (words >> np.uint32(16 * h + i)) & np.uint32(1)
        t[:, j::32] = (2 * b.astype(np.int64) - 1).astype(np.int8)
    return t


# ---------------------------------------------------------------------------
# Base-3 storage: five ternary values per byte (the information-rate form)
# ---------------------------------------------------------------------------
#
# The pages price a ternary value at its information content, log2(3) ~ 1.585
# bits, and quote about 1.71 bits per weight with the group scale (page "Cómo
# Bonsai Ternary 4B revoluciona la difusión texto-imagen", section
# "Representación y almacenamiento de los pesos ternarios"; page "Introducing
# 1-bit and Ternary Bonsai Image 4B", section "量化数学"), while the deployment
# they describe stores 2 bits per value. Five values fit one byte (3^5 = 243 <=
# 256), 1.6 bits per weight. The pages do not print a layout; this library's
# reading:
# * digit d = t + 1 in {0, 1, 2};
# * byte j of row n holds k = 5j .. 5j+4 as the base-3 number with d[5j] as its
#   least significant digit: byte = sum_i d[5j+i] * 3^i;
# * a row is ceil(K/5) bytes, rows back to back; the last byte of a row holds the
#   K mod 5 leftover values (when K mod 5 != 0) and no further digits;
# * a byte of value 243 .. 255 is invalid: its weights decode to 0 and count.

def _base3_digits_per_row(K: int) -> int:
    return (K + 4) // 5


def pack_base3(t: np.ndarray) -> np.ndarray:
    """int8 codes [N, K] in {-1,0,+1} -> uint8 [N, ceil(K/5)] (five per byte)."""
    t = np.asarray(t)
    N, K = t.shape
    if K < 1:
        raise ValueError("K must be >= 1")
    if not np.isin(t, (-1, 0, 1)).all():
        raise ValueError("ternary codes must lie in {-1, 0, +1}")
    nb = _base3_digits_per_row(K)
    d = np.zeros((N, 5 * nb), dtype=np.int64)
    d[:, :K] = t.astype(np.int64) + 1
    out = np.zeros((N, nb), dtype=np.int64)
    for i in range(5):                     # digit i of every byte: k = 5j + i
        out += d[:, i::5] * 3 ** i
    return out.astype(np.uint8)


def unpack_base3(packed: np.ndarray, K: int) -> Tuple[np.ndarray, int]:
    """uint8 [N, ceil(K/5)] -> (int8 codes [N, K], number of weights in invalid bytes)."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    N = packed.shape[0]
    nb = _base3_digits_per_row(K)
    if packed.shape != (N, nb):
        raise ValueError("base-3 rows must be ceil(K/5) bytes")
    v = packed.astype(np.int64)
    bad = v >= 243
    t = np.zeros((N, 5 * nb), dtype=np.int8)
    for i in range(5):
        digit = (v // 3 ** i) % 3
        t[:, i::5] = np.where(bad, 0, digit - 1)
    badk = np.repeat(bad, 5, axis=1)[:, :K]
    return t[:, :K].copy(), int(badk.sum())


def _int2_words(c: np.ndarray) -> np.ndarray:
    """2-bit codes [N, K] (K % 16 == 0) -> uint8 [N, K/4] in the INT2 word layout."""
    N, K = c.shape
    c = c.astype(np.uint32)
    words = np.zeros((N, K // 16), dtype=np.uint32)
    for j in range(16):
        i, h = divmod(j, 2)
        words |= c[:, j::16] << np.uint32(16 * h + 2 * i)
    return words.astype("<u4").view(np.uint8).reshape(N, K // 4)


def base3_to_ternary(packed: np.ndarray, K: int) -> Tuple[np.ndarray, int]:
    """Base-3 rows -> the INT2 packed form of the same codes (K % 16 == 0).

    Weights of an invalid base-3 byte get the INT2 pattern 10, which is itself
    invalid, so the INT2 unpacker counts them again; the count is returned too."""
    if K % 16:
        raise ValueError("the INT2 form needs K % 16 == 0")
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    t, invalid = unpack_base3(packed, K)
    bad = np.repeat(packed.astype(np.int64) >= 243, 5, axis=1)[:, :K]
    c = np.where(bad, 2, t.astype(np.int64) & 3)
    return _int2_words(c), invalid


def packed_bytes(fmt: str, N: int, K: int) -> int:
    if fmt == "base3":
        return N * _base3_digits_per_row(K)
    return N * K // (4 if fmt == "ternary" else 8)


def scale_bytes(N: int, K: int, group: int = GROUP) -> int:
    return 2 * N * (K // group)


# ---------------------------------------------------------------------------
# Dequantisation and the layer
# ---------------------------------------------------------------------------

def dequantize(t: np.ndarray, scales: np.ndarray, group: int = GROUP) -> np.ndarray:
    """W[n, k] = float(scale[n, k // group]) * t[n, k], exactly, in float64."""
    t = np.asarray(t)
    N, K = t.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    s = np.asarray(scales, dtype=np.float16).astype(np.float64)
    if s.shape != (N, K // group):
        raise ValueError("scales must have shape [N, K/group]")
    return np.repeat(s, group, axis=1) * t.astype(np.float64)


def linear(x_bits: np.ndarray, x_dtype: str, t: np.ndarray, scales: np.ndarray,
           bias: Optional[np.ndarray] = None) -> np.ndarray:
    """A[m, n] = sum_k x[m, k] * w[n, k] (+ bias[n]) in float64 (near exact)."""
    X = decode(x_bits, x_dtype)
    W = dequantize(t, scales)
    A = X @ W.T
    if bias is not None:
        A = A + np.asarray(bias, dtype=np.float16).astype(np.float64)[None, :]
    return A


def linear_f32(x_bits: np.ndarray, x_dtype: str, t: np.ndarray, scales: np.ndarray,
               bias: Optional[np.ndarray] = None) -> np.ndarray:
    """The same layer in FP32 arithmetic: exact FP32 dequantisation (s * t),
    one FP32 BLAS matrix product (sgemm), the bias added in FP32. The CPU
    baseline's second form; parity uses the float64 ``linear``. Returns
    float32 values."""
    X = decode(x_bits, x_dtype).astype(np.float32)           # exact: 16-bit inputs
    s = np.asarray(scales, dtype=np.float16).astype(np.float32)
    W = np.repeat(s, GROUP, axis=1) * np.asarray(t).astype(np.float32)   # exact
    A = X @ W.T
    if bias is not None:
        A = A + np.asarray(bias, dtype=np.float16).astype(np.float32)[None, :]
    return A


def magnitude(x_bits: np.ndarray, x_dtype: str, t: np.ndarray, scales: np.ndarray,
              bias: Optional[np.ndarray] = None) -> np.ndarray:
    """sum_k |x[m, k] * w[n, k]| (+ |bias[n]|): the scale of the tolerance."""
    X = np.abs(decode(x_bits, x_dtype))
    W = np.abs(dequantize(t, scales))
    Mg = X @ W.T
    if bias is not None:
        Mg = Mg + np.abs(np.asarray(bias, dtype=np.float16).astype(np.float64))[None, :]
    return Mg


def gelu(a: np.ndarray) -> np.ndarray:
    """Exact-erf GELU, x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2)), in float64."""
    from scipy.special import erf
    a = np.asarray(a, dtype=np.float64)
    return 0.5 * a * (1.0 + erf(a / math.sqrt(2.0)))


# ---------------------------------------------------------------------------
# 4-bit group-quantised weights with a zero point (the text encoder's format)
#
# Page "Cómo Bonsai Ternary 4B revoluciona la difusión texto-imagen", section
# "Arquitectura de despliegue y eficiencia en tiempo de ejecución": the
# pipeline's text encoder runs compressed to 4-bit HQQ. The pages give no
# layout. Reading taken here (parity of the HQQ layout itself is unpinned):
# a weight is an unsigned 4-bit code q in 0..15 with an FP16 scale s and an
# FP16 zero point z per group of 128 weights along K,
#     w = s * (q - z),
# and the packed row is a sequence of little-endian 32-bit words, word u
# holding k = 8u .. 8u+7, the code of k = 8u + 2i + h (i in 0..3, h in {0, 1})
# in bits [16h + 4i, 16h + 4i + 3] (even k in the low half word, odd k in the
# high one, as the ternary layout).
# ---------------------------------------------------------------------------

def pack_int4(q: np.ndarray) -> np.ndarray:
    """uint8 codes [N, K] in 0..15 -> uint8 [N, K/2] (4 bits per weight)."""
    q = np.asarray(q)
    N, K = q.shape
    if K % 8:
        raise ValueError("4-bit packing needs K % 8 == 0")
    if (q < 0).any() or (q > 15).any():
        raise ValueError("4-bit codes must lie in 0..15")
    c = q.astype(np.uint32)
    words = np.zeros((N, K // 8), dtype=np.uint32)
    for j in range(8):                                       # position inside the word
        i, h = divmod(j, 2)
        words |= c[:, j::8] << np.uint32(16 * h + 4 * i)
    return words.astype("<u4").view(np.uint8).reshape(N, K // 2)


def unpack_int4(packed: np.ndarray, K: int) -> np.ndarray:
    """uint8 [N, K/2] -> uint8 codes [N, K] (every 4-bit pattern is valid)."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    N = packed.shape[0]
    words = packed.reshape(N, K // 2).view("<u4").astype(np.uint32)
    q = np.zeros((N, K), dtype=np.uint8)
    for j in range(8):
        i, h = divmod(j, 2)
        q[:, j::8] = ((words >> np.uint32(16 * h + 4 * i)) & np.uint32(15)).astype(np.uint8)
    return q


def dequantize_int4(q: np.ndarray, scales: np.ndarray, zeros: np.ndarray, group: int = GROUP) -> np.ndarray:
    """W[n, k] = s[n, g] * (q[n, k] - z[n, g]), g = k // group, exactly in float64
    (q - z is exact: z has an 11-bit significand and q < 16; the product of two
    numbers of at most 11 and 16 significant bits is exact)."""
    q = np.asarray(q)
    N, K = q.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    s = np.asarray(scales, dtype=np.float16).astype(np.float64)
    z = np.asarray(zeros, dtype=np.float16).astype(np.float64)
    if s.shape != (N, K // group) or z.shape != (N, K // group):
        raise ValueError("scales and zeros must have shape [N, K/group]")
    return np.repeat(s, group, axis=1) * (q.astype(np.float64) - np.repeat(z, group, axis=1))


def linear_int4(x_bits: np.ndarray, x_dtype: str, q: np.ndarray, scales: np.ndarray, zeros: np.ndarray,
                bias: Optional[np.ndarray] = None) -> np.ndarray:
    """A[m, n] = sum_k x[m, k] * s (q[n, k] - z) (+ bias[n]) in float64."""
    A = decode(x_bits, x_dtype) @ dequantize_int4(q, scales, zeros).T
    if bias is not None:
        A = A + np.asarray(bias, dtype=np.float16).astype(np.float64)[None, :]
    return A


def magnitude_int4(x_bits: np.ndarray, x_dtype: str, q: np.ndarray, scales: np.ndarray, zeros: np.ndarray,
                   bias: Optional[np.ndarray] = None) -> np.ndarray:
    """sum_k |x[m, k] * w[n, k]| (+ |bias[n]|)."""
    Mg = np.abs(decode(x_bits, x_dtype)) @ np.abs(dequantize_int4(q, scales, zeros)).T
    if bias is not None:
        Mg = Mg + np.abs(np.asarray(bias, dtype=np.float16).astype(np.float64))[None, :]
    return Mg


# ---------------------------------------------------------------------------
# Quantiser: FP16 weights -> (t, s) per 128-group
#
# The pages do not say how t and s are obtained from trained weights. Page
# "cuantificación de modelos de difusión para inferencia local en dispositivos
# edge", section "Fundamentos Teóricos", names the two lines of work the
# variants descend from, BinaryConnect (binary weights, Courbariaux et al.
# 2015) and Ternary Weight Networks (Li et al. 2016), and says the FP16 group
# scale restores each group's range. Reading taken here (parity of the method
# itself against the pages is unpinned; the rule below is pinned to its own
# definition), applied to each group of 128 weights of a row:
# * ternary (TWN): a weight is kept when |w| > 0.7 * mean|w| over the group;
#   t = sign(w) for kept weights and 0 otherwise; s = the mean of |w| over the
#   kept weights (0 when none is kept);
# * binary (BinaryConnect's deterministic sign with a group scale): t = +1 when
#   w >= 0 (so -0.0 gives +1) and -1 otherwise; s = mean|w| over the group
#   (the scale that minimises sum (w - s t)^2 for those signs);
# * s is the FP16 value nearest the exact mean (ties to even);
# * a non-finite weight (NaN or infinity) is counted and acts as +0.0.
#
# Exactness: every |w| is an FP16 value, a multiple of 2^-24 below 2^16, so
# sums of up to 128 of them are multiples of 2^-24 below 2^23 and are exact in
# float64 (at most 47 significant bits), whatever the order. The threshold test
# |w| > 0.7 mean|w| is 1280 |w| > 7 sum|w| (both sides exact in float64). The
# mean of the kept weights is sum/c with c <= 128: float64 division rounds it
# once, and rounding that to FP16 cannot differ from rounding the exact
# quotient, because a quotient with odd denominator part <= 127 that is not
# itself a 12-bit number lies at least 2^-19 (relative) from every FP16
# rounding midpoint, far beyond the 2^-53 of the float64 rounding.
# ---------------------------------------------------------------------------

def quantize(w_bits: np.ndarray, fmt: str, group: int = GROUP) -> Tuple[np.ndarray, np.ndarray, int]:
    """FP16 weights [N, K] (uint16 bit patterns) -> (int8 t [N, K], uint16 FP16
    scale bits [N, K/group], number of non-finite weights)."""
    w = decode(np.asarray(w_bits, dtype=np.uint16), "f16")
    N, K = w.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    bad = ~np.isfinite(w)
    w = np.where(bad, 0.0, w)
    a = np.abs(w).reshape(N, K // group, group)
    total = a.sum(axis=2)                                   # exact (see above)
    if fmt == "ternary":
        keep = 1280.0 * a > 7.0 * total[:, :, None]          # |w| > 0.7 * mean|w|
        count = keep.sum(axis=2)
        kept = np.where(keep, a, 0.0).sum(axis=2)
        mean = np.where(count > 0, kept / np.maximum(count, 1), 0.0)
        t = np.where(keep.reshape(N, K), np.sign(w), 0.0)
    elif fmt == "binary":
        mean = total / group
        t = np.where(w >= 0.0, 1.0, -1.0)
    else:
        raise ValueError(fmt)
    return t.astype(np.int8), encode(mean, "f16"), int(bad.sum())


# ---------------------------------------------------------------------------
# Tolerance
# ---------------------------------------------------------------------------

REL_TOL = 1e-3
ABS_TOL = 1e-5


def bound(A: np.ndarray, Mg: np.ndarray, y_dtype: str, Y: Optional[np.ndarray] = None) -> np.ndarray:
    """Largest admissible |Y - A| per element.

    1e-3 * Mg + 1e-5, plus half an output ulp (taken at the larger of |A| and |Y|)
    when the output is fp16 or bf16, because the final cast may move the value by
    that much on its own."""
    b = REL_TOL * Mg + ABS_TOL
    if y_dtype in ("f16", "bf16"):
        ref = np.abs(A) if Y is None else np.maximum(np.abs(A), np.abs(Y))
        b = b + 0.5 * ulp(ref, y_dtype)
    return b


def check(Y: np.ndarray, A: np.ndarray, Mg: np.ndarray, y_dtype: str):
    """Return (ok, worst ratio |Y-A|/bound, number of failing elements).

    ``Y`` is float64 (decoded output). Non-finite entries must match in place
    (NaN where A is NaN, equal infinities)."""
    Y = np.asarray(Y, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    fin = np.isfinite(A)
    bad_nf = int((~fin & ~((np.isnan(A) & np.isnan(Y)) | (A == Y))).sum())
    d = np.abs(Y[fin] - A[fin])
    b = bound(A[fin], Mg[fin], y_dtype, Y[fin])
    with np.errstate(invalid="ignore"):
        ratio = np.where(b > 0, d / b, np.where(d > 0, np.inf, 0.0))
    ratio = np.where(np.isnan(ratio), np.inf, ratio)
    nfail = int((ratio > 1.0).sum()) + bad_nf
    worst = float(ratio.max()) if ratio.size else 0.0
    return nfail == 0, worst, nfail
