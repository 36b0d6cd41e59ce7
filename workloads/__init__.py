"""Seeded synthetic inputs for the low-bit-weight linear layer.

This module only draws numbers. It holds none of the layer's arithmetic: no
packing, no dequantisation, no products or sums. The CPU oracle and the GPU
path both take their inputs from here, so the two sides always see identical
host arrays.

Workload shapes follow the pages' description of Bonsai Image 4B: a FLUX.2
Klein 4B MMDiT backbone with hidden size 3072, MLP ratio 3, 5 double-stream and
20 single-stream blocks ("Cómo Bonsai Ternary 4B revoluciona la difusión
texto-imagen", section "Arquitectura de despliegue y eficiencia en tiempo de
ejecución"), ternary weights with P(0)=0.35 or uniform codes, one FP16 scale per
128 weights ("Representación y almacenamiento de los pesos ternarios").
Token counts stand in for the 512x512 and 1024x1024 images the pages time:
1024 image + 512 text tokens, and 4096 image + 512 text tokens.

Conventions
-----------
* Random numbers come from ``numpy.random.Generator(PCG64(seed))``.
* Activations are returned as 16-bit patterns (``uint16``) plus a dtype tag,
  ``"f16"`` or ``"bf16"``, because numpy has no bfloat16. A normal draw is made in
  float32 and rounded to the 16-bit type with round-to-nearest-even.
* Codes are ``int8`` in {-1, 0, +1} (ternary) or {-1, +1} (binary), shape [N, K].
* Scales are ``float16`` of shape [N, K/128]: abs of a normal with standard
  deviation 0.02 (plus an optional offset), drawn in float32, rounded to fp16.
* Draw order inside one linear: X, codes, scales, bias.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

GROUP = 128


def generator(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the bits.

    Input generation only: the rounded values ARE the activations both sides
    receive, so how they were rounded cannot influence parity.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def to_bits(a32: np.ndarray, dtype: str) -> np.ndarray:
    """float32 -> 16-bit pattern of ``dtype`` ('f16' or 'bf16')."""
    if dtype == "f16":
        return np.ascontiguousarray(a32.astype(np.float16)).view(np.uint16)
    if dtype == "bf16":
        return _f32_to_bf16_bits(a32)
    raise ValueError(f"unknown 16-bit dtype {dtype!r}")


def activations(g: np.random.Generator, M: int, K: int, dtype: str, std: float = 1.0) -> np.ndarray:
    x = g.standard_normal((M, K), dtype=np.float32) * np.float32(std)
    return to_bits(x, dtype)


def ternary_codes(g: np.random.Generator, N: int, K: int, p0: Optional[float] = None) -> np.ndarray:
    """Codes in {-1,0,+1}. ``p0=None`` draws the three values uniformly; otherwise
    u ~ U[0,1): 0 if u < p0, +1 if u < p0 + (1-p0)/2, else -1."""
    if p0 is None:
        return (g.integers(0, 3, size=(N, K), dtype=np.int8) - 1).astype(np.int8)
    u = g.random((N, K), dtype=np.float32)
    t = np.full((N, K), -1, dtype=np.int8)
    t[u < np.float32(p0 + (1.0 - p0) / 2.0)] = 1
    t[u < np.float32(p0)] = 0
    return t


def binary_codes(g: np.random.Generator, N: int, K: int) -> np.ndarray:
    return (g.integers(0, 2, size=(N, K), dtype=np.int8) * 2 - 1).astype(np.int8)


def group_scales(g: np.random.Generator, N: int, K: int, offset: float = 0.0, std: float = 0.02) -> np.ndarray:
    assert K % GROUP == 0
    s = np.abs(g.standard_normal((N, K // GROUP), dtype=np.float32)) * np.float32(std)
    if offset:
        s = s + np.float32(offset)
    return s.astype(np.float16)


def bias_f16(g: np.random.Generator, N: int, std: float = 0.01) -> np.ndarray:
    return (g.standard_normal(N, dtype=np.float32) * np.float32(std)).astype(np.float16)


@dataclass
class Linear:
    """One synthetic low-bit linear: X[M,K] (16-bit bits), codes[N,K], scales[N,K/128]."""
    name: str
    fmt: str                # "ternary" | "binary"
    M: int
    N: int
    K: int
    x_dtype: str            # "f16" | "bf16"
    y_dtype: str            # "f16" | "bf16" | "f32"
    x: np.ndarray           # uint16 [M, K]
    codes: np.ndarray       # int8 [N, K]
    scales: np.ndarray      # float16 [N, K/128]
    bias: Optional[np.ndarray] = None   # float16 [N] or None
    meta: dict = field(default_factory=dict)

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


def make_linear(name, fmt, M, N, K, x_dtype="bf16", y_dtype=None, seed=0, p0=0.35,
                scale_offset=0.0, with_bias=False, g=None, x=None) -> Linear:
    g = generator(seed) if g is None else g
    if x is None:
        x = activations(g, M, K, x_dtype)
    if fmt == "ternary":
        codes = ternary_codes(g, N, K, p0)
    elif fmt == "binary":
        codes = binary_codes(g, N, K)
    else:
        raise ValueError(fmt)
    scales = group_scales(g, N, K, offset=scale_offset)
    b = bias_f16(g, N) if with_bias else None
    return Linear(name, fmt, M, N, K, x_dtype, y_dtype or x_dtype, x, codes, scales, b)


# ---------------------------------------------------------------------------
# The five workloads
# ---------------------------------------------------------------------------

def config1() -> Linear:
    """Small ternary linear: X f16 [64x256] ~N(0,1); codes uniform over {-1,0,1}
    [256x256]; scales |N(0,0.02)| + 1e-3; Y f16; seed 0."""
    return make_linear("c1_ternary_f16_64x256x256", "ternary", 64, 256, 256,
                       x_dtype="f16", y_dtype="f16", seed=0, p0=None, scale_offset=1e-3)


def config2() -> Linear:
    """Ternary linear shaped like a 512x512 step: 1536 tokens (1024 image + 512
    text), hidden 3072, bf16 X, P(0)=0.35, fp16 bias ~N(0,0.01); seed 1."""
    return make_linear("c2_ternary_bf16_1536x3072x3072_bias", "ternary", 1536, 3072, 3072,
                       x_dtype="bf16", y_dtype="bf16", seed=1, p0=0.35, with_bias=True)


def config3():
    """Ternary MLP pair shaped like a 1024x1024 step: 4608 tokens (4096 image + 512
    text); up [9216x3072] -> GELU -> down [3072x9216]; bf16; seed 2.

    Returns (up, down). ``down.x`` is None: its input is GELU(up output)."""
    g = generator(2)
    up = make_linear("c3_up_ternary_bf16_4608x9216x3072", "ternary", 4608, 9216, 3072,
                     x_dtype="bf16", y_dtype="bf16", g=g, p0=0.35)
    codes = ternary_codes(g, 3072, 9216, 0.35)
    scales = group_scales(g, 3072, 9216)
    down = Linear("c3_down_ternary_bf16_4608x3072x9216", "ternary", 4608, 3072, 9216,
                  "bf16", "bf16", None, codes, scales, None)
    return up, down


def config4(M: int = 1536) -> List[Linear]:
    """Binary 1-bit linears: [3072x3072] and fused QKV [9216x3072], uniform {-1,+1},
    bf16 X at row count M (1536, 16 or 1); seed 3. The weights do not depend on M."""
    g = generator(3)
    codes_a = binary_codes(g, 3072, 3072)
    scales_a = group_scales(g, 3072, 3072)
    codes_b = binary_codes(g, 9216, 3072)
    scales_b = group_scales(g, 9216, 3072)
    gx = generator(1000 + M)
    x = activations(gx, M, 3072, "bf16")
    return [
        Linear(f"c4_binary_bf16_{M}x3072x3072", "binary", M, 3072, 3072, "bf16", "bf16", x, codes_a, scales_a),
        Linear(f"c4_binary_bf16_{M}x9216x3072", "binary", M, 9216, 3072, "bf16", "bf16", x, codes_b, scales_b),
    ]


# Synthetic 25-block MMDiT linear inventory (hidden 3072, MLP x3).
# Double-stream block: per stream (image, text) Q, K, V, out [3072x3072],
# MLP-in [9216x3072], MLP-out [3072x9216]  -> 12 linears.
# Single-stream block: fused QKV+MLP-in [18432x3072], fused out+MLP-out
# [3072x12288] -> 2 linears. 5*12 + 20*2 = 100 ternary linears.
HIDDEN = 3072
MLP = 3 * HIDDEN


def mmdit_linear_shapes(fuse_qkv: bool = False):
    """List of (name, N, K) for the 100 ternary linears of one transformer pass;
    with fuse_qkv, the Q, K and V linears of each double-stream stream (same
    input) are one [9216x3072] linear with their packed rows concatenated,
    80 linears in all."""
    shapes = []
    for b in range(5):
        for s in ("img", "txt"):
            if fuse_qkv:
                shapes.append((f"double{b}.{s}.qkv", 3 * HIDDEN, HIDDEN))
                shapes.append((f"double{b}.{s}.out", HIDDEN, HIDDEN))
            else:
                for p in ("q", "k", "v", "out"):
                    shapes.append((f"double{b}.{s}.{p}", HIDDEN, HIDDEN))
            shapes.append((f"double{b}.{s}.mlp_in", MLP, HIDDEN))
            shapes.append((f"double{b}.{s}.mlp_out", HIDDEN, MLP))
    for b in range(20):
        shapes.append((f"single{b}.qkv_mlp_in", 3 * HIDDEN + MLP, HIDDEN))
        shapes.append((f"single{b}.out_mlp_out", HIDDEN, HIDDEN + MLP))
    assert len(shapes) == (80 if fuse_qkv else 100)
    return shapes


def config5_weights(seed: int = 4, fmt: str = "ternary", limit: Optional[int] = None):
    """Codes and scales of the 100-linear sweep (one generator, in inventory order)."""
    g = generator(seed)
    out = []
    for i, (name, N, K) in enumerate(mmdit_linear_shapes()):
        if limit is not None and i >= limit:
            break
        codes = ternary_codes(g, N, K, 0.35) if fmt == "ternary" else binary_codes(g, N, K)
        out.append((name, codes, group_scales(g, N, K)))
    return out


def config5_activations(M: int = 4608, seed: int = 4):
    """One bf16 X per distinct K (3072, 9216, 12288), shared by every linear with that K."""
    g = generator(10_000 + seed)
    return {K: activations(g, M, K, "bf16") for K in (HIDDEN, MLP, HIDDEN + MLP)}


# ---------------------------------------------------------------------------
# 4-bit text-encoder weights
# ---------------------------------------------------------------------------
# The pages compress the Qwen3-4B text encoder to 4-bit HQQ ("Cómo Bonsai
# Ternary 4B revoluciona la difusión texto-imagen", section "Arquitectura de
# despliegue y eficiencia en tiempo de ejecución"). They give neither its
# shapes nor the HQQ layout; the shapes below are those of the public
# Qwen3-4B architecture (hidden 2560, 32 query and 8 key/value heads of 128,
# MLP 9728), the layout is 4-bit codes with an FP16 scale and zero point per
# 128 weights along K, and 512 prompt tokens stand in for a prompt.
TE_HIDDEN, TE_Q, TE_KV, TE_MLP, TE_TOKENS = 2560, 4096, 1024, 9728, 512


def int4_codes(g: np.random.Generator, N: int, K: int) -> np.ndarray:
    """Unsigned 4-bit codes, uniform over 0..15, uint8 [N, K]."""
    return g.integers(0, 16, size=(N, K), dtype=np.uint8)


def int4_zeros(g: np.random.Generator, N: int, K: int, center: float = 7.5, std: float = 0.5) -> np.ndarray:
    """FP16 zero points [N, K/128]: center + N(0, std), drawn in float32."""
    assert K % GROUP == 0
    z = np.float32(center) + g.standard_normal((N, K // GROUP), dtype=np.float32) * np.float32(std)
    return z.astype(np.float16)


@dataclass
class Int4Linear:
    """One synthetic 4-bit linear: X[M,K] (16-bit bits), q[N,K] in 0..15,
    scales and zero points [N,K/128] FP16."""
    name: str
    M: int
    N: int
    K: int
    x_dtype: str
    y_dtype: str
    x: np.ndarray
    q: np.ndarray
    scales: np.ndarray
    zeros: np.ndarray
    bias: Optional[np.ndarray] = None

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


def make_int4_linear(name, M, N, K, x_dtype="bf16", y_dtype=None, seed=0, with_bias=False, g=None, x=None,
                     zero_center=7.5, zero_std=0.5, scale_std=0.003) -> Int4Linear:
    """Draw order: X, codes, scales (|N(0, scale_std)| + 1e-4), zero points, bias."""
    g = generator(seed) if g is None else g
    if x is None:
        x = activations(g, M, K, x_dtype)
    q = int4_codes(g, N, K)
    scales = group_scales(g, N, K, offset=1e-4, std=scale_std)
    zeros = int4_zeros(g, N, K, zero_center, zero_std)
    b = bias_f16(g, N) if with_bias else None
    return Int4Linear(name, M, N, K, x_dtype, y_dtype or x_dtype, x, q, scales, zeros, b)


def text_encoder_shapes():
    """(name, N, K) of the seven linears of one text-encoder layer."""
    return [("q", TE_Q, TE_HIDDEN), ("k", TE_KV, TE_HIDDEN), ("v", TE_KV, TE_HIDDEN), ("o", TE_HIDDEN, TE_Q),
            ("gate", TE_MLP, TE_HIDDEN), ("up", TE_MLP, TE_HIDDEN), ("down", TE_HIDDEN, TE_MLP)]


def fp16_weights(g: np.random.Generator, N: int, K: int, std: float = 0.02, outliers: float = 0.0) -> np.ndarray:
    """Dense FP16 weights [N, K] as uint16 bit patterns, the input of the
    quantiser: a normal with standard deviation ``std`` drawn in float32 and
    rounded to FP16 (the spread of a trained transformer's linear weights is of
    that order), and, when ``outliers`` > 0, that fraction of the weights
    multiplied by 8 (the few large weights trained layers carry)."""
    w = g.standard_normal((N, K), dtype=np.float32) * np.float32(std)
    if outliers:
        w = np.where(g.random((N, K), dtype=np.float32) < np.float32(outliers), w * np.float32(8.0), w)
    return np.ascontiguousarray(w.astype(np.float16)).view(np.uint16)
