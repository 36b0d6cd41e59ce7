// Shared device helpers of the gfx950 low-bit-weight GEMM library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lowbit {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

enum { DT_F16 = 0, DT_BF16 = 1, DT_F32 = 2, DT_NONE = 3 };
enum { FMT_BINARY = 1, FMT_TERNARY = 2 };
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
  float* ws;           // split-K partials [splits][M][N] (small-M path only)
  int splits;          // number of K slices
  int gps;             // 128-groups per K slice
};

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

// ---------------------------------------------------------------------------
// Code unpacking into MFMA operand registers.
//
// An MFMA operand register holds two 16-bit values. The kernels feed the MFMA
// with t/2 (ternary) or -t/2 (binary) instead of t: both are exact in FP16 and
// BF16 and their low byte is zero, so one byte lookup (ternary) or one
// sign-bit insert (binary) builds a value. The factor 2 (or -2) is folded into
// the group scale, where it is exact.
//
// Ternary codes are the 2-bit two's complement of t (00 = 0, 01 = +1,
// 11 = -1). After a right rotation the two codes of a register sit at bits
// [9:8] and [25:24]; masking leaves a v_perm selector whose bytes 1 and 3 are
// the codes and whose bytes 0 and 2 are zero. Byte 0 of the table is 0x00, so
// the low bytes and t = 0 both read zero; bytes 1 and 3 hold the high bytes
// of +0.5 and -0.5 (the invalid code 10 reads byte 2 = 0x00).
// ---------------------------------------------------------------------------
template <bool BF16>
__device__ __forceinline__ constexpr uint32_t tern_table() {
  return BF16 ? 0xBF003F00u : 0xB8003800u;
}

template <bool BF16>
__device__ __forceinline__ uint32_t tern_pair(uint32_t w, uint32_t rot) {
  uint32_t x = rot ? __builtin_amdgcn_alignbit(w, w, rot) : w;
  return __builtin_amdgcn_perm(0u, tern_table<BF16>(), x & 0x03000300u);
}

// Variants with the table (ternary) or the sign mask and base (binary) passed
// in registers, so a group whose scale is zero can use an all-zero table.
__device__ __forceinline__ uint32_t tern_pair_t(uint32_t w, uint32_t rot, uint32_t table) {
  uint32_t x = rot ? __builtin_amdgcn_alignbit(w, w, rot) : w;
  return __builtin_amdgcn_perm(0u, table, x & 0x03000300u);
}

__device__ __forceinline__ u32x4 tern_chunk_t(uint32_t w, int c, uint32_t table) {
  u32x4 r;
#pragma unroll
  for (int v = 0; v < 4; ++v) r[v] = tern_pair_t(w, (uint32_t)((8 * (c & 1) + 2 * v + 24) & 31), table);
  return r;
}

__device__ __forceinline__ u32x4 bin_chunk_t(uint32_t w, int c, uint32_t mask, uint32_t base) {
  u32x4 r;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const uint32_t rot = (uint32_t)((4 * c + v + 17) & 31);
    const uint32_t x = rot ? __builtin_amdgcn_alignbit(w, w, rot) : w;
    r[v] = (x & mask) | base;
  }
  return r;
}

// Binary: after a right rotation the two bits of a register sit at bits 15
// and 31, i.e. on the sign bits of the two halves of +0.5; bit 1 (t = +1)
// gives -0.5 = -t/2.
template <bool BF16>
__device__ __forceinline__ uint32_t bin_pair(uint32_t w, uint32_t rot) {
  uint32_t x = rot ? __builtin_amdgcn_alignbit(w, w, rot) : w;
  return (x & 0x80008000u) | (BF16 ? 0x3F003F00u : 0x38003800u);
}

// Operand registers for chunk c (c = 0..3) of one 128-group, for the lane
// group that owns k-local [32q, 32q+32) of the group. Slot s of the chunk is
// k-local 32q + 8c + s; register v holds slots 2v (low half) and 2v+1.
//
// Ternary: the lane group's 32 codes are words w0 (k-local 32q..32q+15) and
// w1 (32q+16..32q+31). k-local 32q + 8c + 2v + h lives in word c/2 at bit
// 16h + 2(4(c%2) + v); rotating right by 8(c%2) + 2v - 8 (mod 32) puts the
// pair at bits 8 and 24.
template <bool BF16>
__device__ __forceinline__ u32x4 tern_chunk(uint32_t w0, uint32_t w1, int c) {
  uint32_t w = (c < 2) ? w0 : w1;
  u32x4 r;
#pragma unroll
  for (int v = 0; v < 4; ++v) r[v] = tern_pair<BF16>(w, (uint32_t)((8 * (c & 1) + 2 * v + 24) & 31));
  return r;
}

// Binary: the lane group's 32 bits are one word w; k-local 32q + 8c + 2v + h
// is bit 16h + 4c + v; rotating right by 4c + v + 17 (mod 32) puts the pair
// at bits 15 and 31.
template <bool BF16>
__device__ __forceinline__ u32x4 bin_chunk(uint32_t w, int c) {
  u32x4 r;
#pragma unroll
  for (int v = 0; v < 4; ++v) r[v] = bin_pair<BF16>(w, (uint32_t)((4 * c + v + 17) & 31));
  return r;
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

template <bool BF16>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

}  // namespace lowbit
