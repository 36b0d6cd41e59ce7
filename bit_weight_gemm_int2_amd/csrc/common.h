// Shared device helpers of the gfx950 low-bit-weight GEMM library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lowbit {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

enum { DT_F16 = 0, DT_BF16 = 1, DT_F32 = 2, DT_NONE = 3 };
enum { FMT_BINARY = 1, FMT_TERNARY = 2, FMT_BASE3 = 3, FMT_INT4 = 4 };
enum { ACT_NONE = 0, ACT_GELU = 1 };

struct GemmArgs {
  const uint16_t* X;   // [M][ldx] 16-bit activations
  int64_t ldx;
  const uint8_t* W;    // packed codes, row stride K/4 (ternary) or K/8 (binary) bytes
  const uint16_t* S;   // fp16 scales [N][K/128]
  const void* bias;
  int bias_dtype;
  void* Y;
  int64_t ldy;
  int y_dtype;
  int act;
  int M, N, K;
  float* ws;           // caller workspace: split-K partials (small M) or the 4-bit row sums
  const uint16_t* Z;   // fp16 zero points [N][K/128] (4-bit format only)
  int64_t ldr;         // row stride of the 4-bit row sums [K/128][ldr]
  float* part;         // large-M kernel with a K split (gridDim.y > 1): FP32 partial planes [split][M][N]
};

// The operands of the problems of one grouped launch: same shapes, types and
// activation, different buffers; problem z runs as blockIdx.z. Only the
// small-M kernels take groups.
constexpr int kMaxGroup = 8;
struct GemmGroup {
  const uint16_t* X[kMaxGroup];
  const uint8_t* W[kMaxGroup];
  const uint16_t* S[kMaxGroup];
  const void* bias[kMaxGroup];
  void* Y[kMaxGroup];
};

// Point `a` at the operands of problem z (wave-uniform) of a grouped launch.
__device__ __forceinline__ void select_problem(GemmArgs& a, const GemmGroup& g, int z) {
#pragma unroll
  for (int i = 1; i < kMaxGroup; ++i) {
    if (z == i) {
      a.X = g.X[i];
      a.W = g.W[i];
      a.S = g.S[i];
      a.bias = g.bias[i];
      a.Y = g.Y[i];
    }
  }
}

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ float bf16_bits_to_float(uint16_t h) {
  return __builtin_bit_cast(float, (uint32_t)h << 16);
}

// float -> bf16 bits, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ uint16_t float_to_half_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);   // RNE conversion
}

__device__ __forceinline__ float load_bias(const void* bias, int dtype, int n) {
  if (dtype == DT_F16) return half_bits_to_float(((const uint16_t*)bias)[n]);
  if (dtype == DT_BF16) return bf16_bits_to_float(((const uint16_t*)bias)[n]);
  if (dtype == DT_F32) return ((const float*)bias)[n];
  return 0.0f;
}

// GELU with the error function, x * Phi(x), Phi(x) = (1 + erf(x / sqrt 2)) / 2.
// erf is evaluated with the rational-exponential approximation of
// Abramowitz & Stegun, Handbook of Mathematical Functions, eq. 7.1.26:
//   erfc(z) ~ (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-z^2),
//   t = 1 / (1 + p z), z >= 0, |error in erf| <= 1.5e-7.
// For x < 0 Phi is taken directly as erfc(|x|/sqrt2)/2, so there is no
// cancellation; the absolute error of GELU is below 1e-7 * |x| + a few FP32 ulps.
__device__ __forceinline__ float gelu_erf(float x) {
  const float z = fabsf(x) * 0.70710678118654752440f;
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.3275911f, z, 1.0f));
  float poly = __builtin_fmaf(1.061405429f, t, -1.453152027f);
  poly = __builtin_fmaf(poly, t, 1.421413741f);
  poly = __builtin_fmaf(poly, t, -0.284496736f);
  poly = __builtin_fmaf(poly, t, 0.254829592f);
  poly *= t;
  const float e = poly * __builtin_amdgcn_exp2f(-z * z * 1.44269504088896340736f);   // ~erfc(z)
  const float phi = x >= 0.0f ? __builtin_fmaf(-0.5f, e, 1.0f) : 0.5f * e;
  return x * phi;
}

__device__ __forceinline__ float finish(float acc, float b, int act) {
  float v = acc + b;
  return act == ACT_GELU ? gelu_erf(v) : v;
}

__device__ __forceinline__ void store_out(void* Y, int64_t ldy, int dtype, int m, int n, float v) {
  int64_t off = (int64_t)m * ldy + n;
  if (dtype == DT_BF16) ((uint16_t*)Y)[off] = float_to_bf16_bits(v);
  else if (dtype == DT_F16) ((uint16_t*)Y)[off] = float_to_half_bits(v);
  else ((float*)Y)[off] = v;
}

// s_waitcnt immediate for vmcnt(n), expcnt(7), lgkmcnt(0)
constexpr int waitcnt_vm(int n) { return (n & 15) | (7 << 4) | ((n >> 4) << 14); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Direct global -> LDS loads (global_load_lds_*) issued from inline assembly:
// the address is a wave-uniform 64-bit base (SGPRs) plus a 32-bit per-lane
// byte offset, and lane l's data lands at LDS byte lds + 16 l (16-byte form)
// or in the 4-byte slot lds + 4 l, zero-extended (2-byte form). The compiler
// does not see these as memory operations: the caller waits for them with
// an explicit s_waitcnt (they count in vmcnt) before reading the LDS.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_ptr_t)p;
}
__device__ __forceinline__ void dma_lds16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(sbase)
               : "memory", "m0");
}
__device__ __forceinline__ void dma_lds2(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_ushort %1, %2" ::"s"(lds), "v"(voff), "s"(sbase)
               : "memory", "m0");
}

// ---------------------------------------------------------------------------
// Code unpacking into MFMA operand registers.
//
// An MFMA operand register holds two 16-bit values. The kernels feed the MFMA
// with 2t (ternary) or -2t (binary) instead of t. In both FP16 and BF16 the
// value 2.0 is the single exponent bit 14, so +-2.0 is (bit 15 = sign,
// bit 14 = 1) and 0 is all zeros; the factor 1/2 (or -1/2) is folded into the
// group scale, where it is exact. Every value is then built by one rotate and
// one mask (ternary) or one rotate and one AND-OR (binary), with no lookup.
//
// Ternary: the 2-bit two's complement code (bit 0: t != 0, bit 1: t < 0) is
// bits 14..15 of 2t as they stand. Pair i of a packed word (its k = 2i and
// 2i + 1) sits at bits 2i and 16 + 2i; rotating right by 18 + 2i (mod 32)
// moves the pair to bits 14 and 30, and the mask 0xC000C000 leaves the two
// values. The invalid code 10 becomes -0.0, i.e. t = 0.
// Binary: pair i of a packed word (its k = 2i and 2i + 1) sits at bits i and
// 16 + i; rotating right by 17 + i (mod 32) puts it on the two sign bits, and
// OR-ing 2.0 into both halves gives -2t (bit 1 means t = +1).
// ---------------------------------------------------------------------------
constexpr uint32_t TERN_MASK = 0xC000C000u;
constexpr uint32_t BIN_SIGN = 0x80008000u, BIN_TWO = 0x40004000u;

__device__ __forceinline__ uint32_t rotr(uint32_t w, int n) {
  n &= 31;
  return n ? __builtin_amdgcn_alignbit(w, w, (uint32_t)n) : w;
}

// Eight consecutive k of a ternary word: pairs 4c .. 4c+3 (c = 0, 1);
// register v holds pair 4c + v. A zero mask gives an all-zero operand.
__device__ __forceinline__ u32x4 tern_chunk(uint32_t w, int c, uint32_t mask) {
  u32x4 r;
#pragma unroll
  for (int v = 0; v < 4; ++v) r[v] = rotr(w, 18 + 2 * (4 * c + v)) & mask;
  return r;
}

// Eight consecutive k of a binary word: pairs 4c .. 4c+3 (c = 0..3).
// Zero sign mask and base give an all-zero operand.
__device__ __forceinline__ u32x4 bin_chunk(uint32_t w, int c, uint32_t sign, uint32_t two) {
  u32x4 r;
#pragma unroll
  for (int v = 0; v < 4; ++v) r[v] = (rotr(w, 17 + 4 * c + v) & sign) | two;
  return r;
}

// Eight consecutive k of a 4-bit word (k = 2v and 2v + 1 at bits 4v and
// 16 + 4v) as the MFMA values 128 + q, exact in both 16-bit types: in BF16
// the values 128 .. 143 are 0x4300 | q (exponent of 128, q in the seven
// mantissa bits), in FP16 they are 0x5800 | q << 3 (mantissa spacing 1/8 of
// the ten bits, so q sits three bits up). One shift and one AND-OR per
// register; zero mask and base give an all-zero operand.
template <bool BF16>
__device__ __forceinline__ u32x4 int4_chunk(uint32_t w, uint32_t mask, uint32_t base) {
  u32x4 r;
  if constexpr (BF16) {
#pragma unroll
    for (int v = 0; v < 4; ++v) r[v] = ((w >> (4 * v)) & mask) | base;
  } else {
    r[0] = ((w << 3) & mask) | base;
#pragma unroll
    for (int v = 1; v < 4; ++v) r[v] = ((w >> (4 * v - 3)) & mask) | base;
  }
  return r;
}
template <bool BF16> __device__ __forceinline__ constexpr uint32_t int4_mask() { return BF16 ? 0x000F000Fu : 0x00780078u; }
template <bool BF16> __device__ __forceinline__ constexpr uint32_t int4_base() { return BF16 ? 0x43004300u : 0x58005800u; }

// Factor that turns an MFMA sum of the fed values back into sum x * t.
template <bool TERN>
__device__ __forceinline__ constexpr float code_factor() {
  return TERN ? 0.5f : -0.5f;
}

template <bool BF16>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <bool BF16>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}


}  // namespace lowbit
