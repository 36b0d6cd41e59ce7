// Group quantiser: dense FP16 weights -> packed codes t and FP16 group scales
// s, written straight into the INT2 or 1-bit layout that lowbit_gemm reads.
//
// The pages name the two lines of work the variants come from, BinaryConnect
// and Ternary Weight Networks ("cuantificacion de modelos de difusion para
// inferencia local en dispositivos edge", section "Fundamentos Teoricos"),
// and an FP16 scale per group of 128 weights ("Como Bonsai Ternary 4B
// revoluciona la difusion texto-imagen", section "Representacion y
// almacenamiento de los pesos ternarios"); how the released weights were
// quantised is not stated. The rule applied per group (see lowbit.h):
//  * ternary: keep |w| > 0.7 mean|w|; t = sign(w) when kept, else 0;
//    s = mean of the kept |w| (0 when none is kept);
//  * binary: t = +1 for w >= 0 (-0.0 included), else -1; s = mean|w|;
//  * s = the FP16 value nearest the exact mean, ties to even;
//  * NaN and infinities are counted and act as +0.0.
//
// Every decision is exact, so the result is a pure function of the input:
//  * |w| of an FP16 value is a multiple of 2^-24 below 2^16, so sums of up to
//    128 of them are exact in FP64 in any order (at most 47 significant
//    bits), and the wave reductions below give every lane the same sum;
//  * |w| > 0.7 mean|w| is evaluated as 1280 |w| > 7 sum|w| (the left side
//    exact in FP32, the right one in FP64; the comparison is described
//    under "Work layout");
//  * the kept mean sum / count is one correctly rounded FP64 division; a
//    quotient with denominator <= 128 either is a 12-bit number (then the
//    division is exact) or lies at least 2^-19 (relative) from every FP16
//    rounding midpoint, so rounding the FP64 quotient to FP16 gives the
//    FP16 rounding of the exact mean;
//  * that last rounding is done on the FP64 bit pattern (f64_to_f16_rne).
//
// Work layout: HBM-bound (2 bytes read, 0.25 or 0.125 written per weight).
// An 8-lane eighth of a wave owns kQGroups consecutive groups of the
// flattened [N][K/128] group array per pass; lane `sub` holds weights
// 16 sub .. 16 sub + 15 of each group (two 16-byte loads per group, all
// issued before any is used), which is exactly one INT2 word. The FP64 work
// per weight is one conversion and the exact sums; the threshold test runs
// in FP32 as 1280 |w| > RD(7 sum|w|) (RD: the FP32 value at or below), which
// is exact because 1280 |w| is an FP32 value and x > t <=> x > RD(t) for any
// FP32 x. Group sums are exchanged within the eighth (xor shuffles 1, 2, 4);
// binary lanes pair their bits into a word with one more shuffle.
#include "common.h"

namespace lowbit {

constexpr int kQGroups = 2;   // groups per 8-lane eighth and pass

// Non-negative finite double -> FP16 bits, round to nearest, ties to even.
__device__ __forceinline__ uint32_t f64_to_f16_rne(double d) {
  const uint64_t b = (uint64_t)__double_as_longlong(d);
  if (b == 0) return 0;
  const int e = (int)(b >> 52) - 1023;                        // d = 1.f * 2^e
  if (e > 15) return 0x7C00;
  const uint64_t m = (b & ((1ull << 52) - 1)) | (1ull << 52);  // 53-bit significand
  // keep 11 significant bits (normal range) or the multiples of 2^-24 (below)
  const int shift = 42 + (e < -14 ? -14 - e : 0);
  if (shift > 60) return 0;                                   // below 2^-43: rounds to 0
  uint64_t r = m >> shift;
  const uint64_t rem = m & ((1ull << shift) - 1), half = 1ull << (shift - 1);
  r += (rem > half || (rem == half && (r & 1))) ? 1 : 0;
  // normal: exponent field e + 15 over a mantissa of r - 1024 (a carry to
  // r = 2048 moves into the exponent by itself); subnormal: r itself, where
  // r = 1024 is the smallest normal value
  return e >= -14 ? (uint32_t)(((e + 15) << 10) + (int)r - 1024) : (uint32_t)r;
}

// Non-negative double -> the largest FP32 value at or below it.
__device__ __forceinline__ float f64_to_f32_down(double d) {
  const float f = (float)d;                                   // nearest
  return (double)f > d ? __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, f) - 1u) : f;
}

__device__ __forceinline__ double qsum8(double v) {
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ int isum8(int v) {
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

template <bool TERN>
__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t* __restrict__ W, int64_t ldw, int64_t N,
                                                       int G, uint32_t* __restrict__ packed,
                                                       uint16_t* __restrict__ scales, int32_t* counter) {
  const int sub = threadIdx.x & 7;
  const int64_t total = N * G;
  const int64_t eighth = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 3;
  const int64_t eighths = ((int64_t)gridDim.x * blockDim.x) >> 3;
  const int64_t wpg = TERN ? 8 : 4;                 // packed words per group
  int bad = 0;
  // every lane of an eighth takes the same trip count and the same groups,
  // so the eighth is either wholly active or wholly idle at each shuffle
  for (int64_t first = eighth * kQGroups; first < total; first += eighths * kQGroups) {
    u32x4 v[kQGroups][2];
    int64_t row[kQGroups];
    int col[kQGroups];
#pragma unroll
    for (int q = 0; q < kQGroups; ++q) {
      const int64_t grp = first + q < total ? first + q : total - 1;   // past the end: reread the last
      row[q] = grp / G;
      col[q] = (int)(grp - row[q] * G);
      const uint16_t* src = W + row[q] * ldw + 128 * col[q] + 16 * sub;
      v[q][0] = *(const u32x4*)src;
      v[q][1] = *(const u32x4*)(src + 8);
    }
#pragma unroll
    for (int q = 0; q < kQGroups; ++q) {
      const bool live = first + q < total;
      float a[16];                                  // |w|, exact in FP32
      uint32_t neg = 0;                             // bit j: weight j has its sign bit set
      double part = 0.0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint32_t h = (v[q][j >> 3][(j >> 1) & 3] >> (16 * (j & 1))) & 0xFFFFu;
        const uint32_t mag = h & 0x7FFFu;
        const bool fin = mag < 0x7C00u;
        bad += (fin || !live) ? 0 : 1;
        a[j] = half_bits_to_float((uint16_t)(fin ? mag : 0u));
        neg |= (h >> 15) << j;
        part += (double)a[j];
      }
      const double sum = qsum8(part);               // exact, the same in every lane
      uint32_t word = 0, sbits;
      if constexpr (TERN) {
        const float thr = f64_to_f32_down(7.0 * sum);
        double kept = 0.0;
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const bool keep = 1280.0f * a[j] > thr;    // |w| > 0.7 mean|w|
          kept += keep ? (double)a[j] : 0.0;
          cnt += keep ? 1 : 0;
          const uint32_t code = keep ? (((neg >> j) & 1u) ? 3u : 1u) : 0u;
          word |= code << (16 * (j & 1) + 2 * (j >> 1));
        }
        kept = qsum8(kept);
        cnt = isum8(cnt);
        sbits = cnt ? f64_to_f16_rne(kept / (double)cnt) : 0u;
        if (live) packed[row[q] * (G * wpg) + col[q] * wpg + sub] = word;
      } else {
        const int base = 8 * (sub & 1);               // bit index of this lane's first weight in its half
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          // t = -1 only for a negative nonzero weight (-0.0 and non-finite give +1)
          const uint32_t bit = (((neg >> j) & 1u) && a[j] != 0.0f) ? 0u : 1u;
          word |= bit << (16 * (j & 1) + base + (j >> 1));
        }
        sbits = f64_to_f16_rne(sum * 0.0078125);      // sum / 128, exact
        word |= __shfl_xor(word, 1);
        if (live && (sub & 1) == 0) packed[row[q] * (G * wpg) + col[q] * wpg + (sub >> 1)] = word;
      }
      if (live && sub == 0) scales[row[q] * G + col[q]] = (uint16_t)sbits;
    }
  }
  if (counter) {
    const unsigned long long m = __ballot(bad != 0);
    if (m) {
      int t = bad;
      for (int off = 32; off > 0; off >>= 1) t += __shfl_xor(t, off);
      if ((threadIdx.x & 63) == __builtin_ctzll(m)) atomicAdd(counter, t);
    }
  }
}

__global__ void quant_zero_kernel(int32_t* p) { *p = 0; }

hipError_t launch_quantize(int fmt, const uint16_t* W, int64_t ldw, int64_t N, int64_t K, uint8_t* packed,
                           uint16_t* scales, int32_t* counter, hipStream_t st) {
  if (counter) hipLaunchKernelGGL(quant_zero_kernel, dim3(1), dim3(1), 0, st, counter);
  const int G = (int)(K / 128);
  const int64_t eighths = (N * G + kQGroups - 1) / kQGroups;
  int64_t blocks = (eighths + 31) / 32;
  blocks = blocks < 1 ? 1 : (blocks > 32768 ? 32768 : blocks);
  if (fmt == FMT_TERNARY)
    hipLaunchKernelGGL(quantize_kernel<true>, dim3((int)blocks), dim3(256), 0, st, W, ldw, N, G,
                       (uint32_t*)packed, scales, counter);
  else
    hipLaunchKernelGGL(quantize_kernel<false>, dim3((int)blocks), dim3(256), 0, st, W, ldw, N, G,
                       (uint32_t*)packed, scales, counter);
  return hipGetLastError();
}

}  // namespace lowbit
