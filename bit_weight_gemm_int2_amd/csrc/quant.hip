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
//    bits), and the wave reductions below give every lane the same sum S;
//  * |w| > 0.7 mean|w| means 1280 |w| > 7 S. For an FP16 value x and a real
//    t >= 0, x > t holds exactly when x > RD(t), RD(t) being the largest FP16
//    value at or below t; for non-negative FP16 values the order of the bit
//    patterns is the order of the values. So the test is an integer compare
//    of the 15-bit magnitude against RD(7 S / 1280), found once per group
//    (f16_floor_ratio) and applied to two weights at once;
//  * every kept weight exceeds 0.7 S / 128 >= 0.7 max|w| / 128 > 2^(E-8),
//    with 2^E <= max|w| < 2^(E+1), so it is a multiple of 2^(E-18); the 16
//    kept weights of a lane then sum to a multiple of 2^(E-18) below 2^(E+5),
//    23 significant bits, which FP32 holds exactly in any order. Lane sums
//    are added in FP64;
//  * the kept mean sum / count is one correctly rounded FP64 division; a
//    quotient with denominator <= 128 either is a 12-bit number (then the
//    division is exact) or lies at least 2^-19 (relative) from every FP16
//    rounding midpoint, so rounding the FP64 quotient to FP16 gives the
//    FP16 rounding of the exact mean;
//  * that last rounding is done on the FP64 bit pattern (f64_to_f16_rne).
//
// Work layout: HBM-bound (2 bytes read, 0.25 or 0.125 written per weight).
// Two kernels:
//  * quantize_kernel (both formats): an 8-lane eighth of a wave owns
//    kQGroups consecutive groups of the flattened [N][K/128] group array per
//    pass; lane `sub` holds weights 16 sub .. 16 sub + 15 of each group (two
//    16-byte loads per group, all issued before any is used), which is
//    exactly one INT2 word. Group sums are exchanged within the eighth (DPP
//    moves); binary lanes pair their bits into a word with one more move.
//  * quantize_lane_kernel (ternary, many groups): one lane owns a whole group
//    (sixteen 16-byte loads), so the per-group work (threshold, division,
//    rounding) is done once instead of in all eight lanes of an eighth, with
//    no exchange at all. Its loads touch 64 cache lines per instruction and
//    it needs many groups to fill the GPU: it gains only on launches of
//    about half a gigabyte and more (from 2^21 groups); binary (already at
//    the copy rate with eighths) and smaller ternary launches keep
//    quantize_kernel.
// In both, weights stay in their 32-bit pairs: magnitudes, keep flags (one
// packed 16-bit subtract per pair), signs and codes are formed two at a time
// with bit operations, and non-finite weights are looked for with one packed
// maximum per pair (only a wave or lane that holds one takes the branch that
// counts and clears them). In the lane kernel the kept weights are summed in
// FP32 over each 16-weight word (exact, as above) and the word sums in FP64.
#include "common.h"

namespace lowbit {

constexpr int kQGroups = 2;   // groups per 8-lane eighth and pass

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// Non-negative finite double -> FP16 bits, round to nearest, ties to even.
// (Branch-free: every lane of a wave runs the same instructions.)
__device__ __forceinline__ uint32_t f64_to_f16_rne(double d) {
  const uint64_t b = (uint64_t)__double_as_longlong(d);
  const int e = (int)(b >> 52) - 1023;                        // d = 1.f * 2^e (b > 0)
  const uint64_t m = (b & ((1ull << 52) - 1)) | (1ull << 52);  // 53-bit significand
  // keep 11 significant bits (normal range) or the multiples of 2^-24 (below);
  // below 2^-43 (and for d = 0) everything rounds to 0
  const int sh = 42 + (e < -14 ? -14 - e : 0);
  const int shift = sh > 60 ? 60 : sh;
  uint64_t r = m >> shift;
  const uint64_t rem = m & ((1ull << shift) - 1), half = 1ull << (shift - 1);
  r += (rem > half || (rem == half && (r & 1))) ? 1 : 0;
  r = sh > 60 ? 0 : r;
  // normal: exponent field e + 15 over a mantissa of r - 1024 (a carry to
  // r = 2048 moves into the exponent by itself); subnormal: r itself, where
  // r = 1024 is the smallest normal value
  const uint32_t h = e >= -14 ? (uint32_t)(((e + 15) << 10) + (int)r - 1024) : (uint32_t)r;
  return e > 15 ? 0x7C00u : h;
}

// Non-negative double below 65520 -> bits of the largest FP16 value at or
// below it (truncation of the same fields).
__device__ __forceinline__ uint32_t f64_to_f16_down(double d) {
  const uint64_t b = (uint64_t)__double_as_longlong(d);
  const int e = (int)(b >> 52) - 1023;
  const uint64_t m = (b & ((1ull << 52) - 1)) | (1ull << 52);
  const int sh = 42 + (e < -14 ? -14 - e : 0);
  const uint64_t r = sh > 60 ? 0 : m >> (sh > 60 ? 60 : sh);
  return e >= -14 ? (uint32_t)(((e + 15) << 10) + (int)r - 1024) : (uint32_t)r;
}

// The largest FP16 value h with 1280 h <= q (q = 7 S, exact): the FP64
// quotient truncated to FP16, then moved by at most one FP16 step, checked
// with exact products (an FP16 value times 1280 has at most 14 bits).
__device__ __forceinline__ uint32_t f16_floor_ratio(double q) {
  uint32_t h = f64_to_f16_down(q * (1.0 / 1280.0));
  h = h > 0x7BFFu ? 0x7BFFu : h;
  const bool over = h > 0 && 1280.0 * (double)half_bits_to_float((uint16_t)h) > q;
  const bool under = h < 0x7BFFu && 1280.0 * (double)half_bits_to_float((uint16_t)(h + 1)) <= q;
  return over ? h - 1 : (under ? h + 1 : h);
}

// Sums over the eight lanes of an eighth, every lane getting the total, by
// DPP moves inside the eighth: swap neighbours, swap pairs, then mirror the
// eight lanes (after the first two steps every lane of a quad holds the quad's
// sum, so the mirror pairs each quad with the other). DPP controls: quad_perm
// [1,0,3,2] = 0xB1, quad_perm [2,3,0,1] = 0x4E, row_half_mirror = 0x141.
template <int CTRL>
__device__ __forceinline__ int dpp32(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ double dpp64(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)dpp32<CTRL>((int)(uint32_t)b), hi = (uint32_t)dpp32<CTRL>((int)(uint32_t)(b >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ double qsum8(double v) {
  v += dpp64<0xB1>(v);
  v += dpp64<0x4E>(v);
  return v + dpp64<0x141>(v);
}
__device__ __forceinline__ int isum8(int v) {
  v += dpp32<0xB1>(v);
  v += dpp32<0x4E>(v);
  return v + dpp32<0x141>(v);
}

// Both 16-bit halves: a - b modulo 2^16 (bit 15 / 31: b > a for 15-bit values).
__device__ __forceinline__ uint32_t sub16x2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, a) - __builtin_bit_cast(u16x2, b));
}
__device__ __forceinline__ uint32_t max16x2(uint32_t a, uint32_t b) {
  const u16x2 x = __builtin_bit_cast(u16x2, a), y = __builtin_bit_cast(u16x2, b);
  return __builtin_bit_cast(uint32_t, u16x2{x[0] > y[0] ? x[0] : y[0], x[1] > y[1] ? x[1] : y[1]});
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
  // the group `first` as (row r0, column c0), advanced by the grid stride
  // without a division per pass
  const int64_t stride = eighths * kQGroups, srow = stride / G;
  const int scol = (int)(stride - srow * G);
  int64_t r0 = (eighth * kQGroups) / G;
  int c0 = (int)(eighth * kQGroups - r0 * G);
  // every lane of an eighth takes the same trip count and the same groups,
  // so the eighth is either wholly active or wholly idle at each exchange
  for (int64_t first = eighth * kQGroups; first < total; first += stride) {
    u32x4 v[kQGroups][2];
    int64_t row[kQGroups];
    int col[kQGroups];
#pragma unroll
    for (int q = 0; q < kQGroups; ++q) {
      row[q] = q == 0 ? r0 : (col[q - 1] + 1 == G ? row[q - 1] + 1 : row[q - 1]);
      col[q] = q == 0 ? c0 : (col[q - 1] + 1 == G ? 0 : col[q - 1] + 1);
      // past the end: reread the last group (nothing of it is written)
      const bool in = first + q < total;
      const uint16_t* src = W + (in ? row[q] : N - 1) * ldw + 128 * (in ? col[q] : G - 1) + 16 * sub;
      v[q][0] = *(const u32x4*)src;
      v[q][1] = *(const u32x4*)(src + 8);
    }
    c0 += scol;
    r0 += srow + (c0 >= G ? 1 : 0);
    c0 -= c0 >= G ? G : 0;
#pragma unroll
    for (int q = 0; q < kQGroups; ++q) {
      const bool live = first + q < total;
      // pair j holds weights 2j (low half) and 2j + 1 (high half)
      uint32_t h[8], P[8], mx = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        h[j] = v[q][j >> 2][j & 3];
        P[j] = h[j] & 0x7FFF7FFFu;                   // magnitude bits
        mx = max16x2(mx, P[j]);
      }
      const bool nonfinite = (mx & 0xFFFFu) >= 0x7C00u || (mx >> 16) >= 0x7C00u;
      if (__ballot(nonfinite)) {
        // count the non-finite weights and let them act as +0.0
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t nf = (P[j] + 0x04000400u) & 0x80008000u;   // magnitude >= 0x7C00
          bad += live ? __builtin_popcount(nf) : 0;
          P[j] &= ~(nf - (nf >> 15));
        }
      }
      float a[16];                                  // |w|, exact in FP32
      double part = 0.0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        a[2 * j] = half_bits_to_float((uint16_t)(P[j] & 0xFFFFu));
        a[2 * j + 1] = half_bits_to_float((uint16_t)(P[j] >> 16));
        part += (double)a[2 * j];
        part += (double)a[2 * j + 1];
      }
      const double sum = qsum8(part);               // exact, the same in every lane
      uint32_t word = 0, sbits;
      if constexpr (TERN) {
        const uint32_t thr = f16_floor_ratio(7.0 * sum);
        const uint32_t thr2 = thr | (thr << 16);
        float kept = 0.0f;
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t keep = sub16x2(thr2, P[j]) & 0x80008000u;  // |w| > threshold
          cnt += __builtin_popcount(keep);
          // code 01 for +1, 11 for -1 at bits 2j (weight 2j) and 16 + 2j (weight 2j + 1)
          word |= (keep >> (15 - 2 * j)) | ((h[j] & keep) >> (14 - 2 * j));
          const uint32_t lo = (uint32_t)((int32_t)(keep << 16) >> 31), hi = (uint32_t)((int32_t)keep >> 31);
          kept += __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, a[2 * j]) & lo);
          kept += __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, a[2 * j + 1]) & hi);
        }
        const double ksum = qsum8((double)kept);
        cnt = isum8(cnt);
        sbits = cnt ? f64_to_f16_rne(ksum / (double)cnt) : 0u;
        if (live) packed[row[q] * (G * wpg) + col[q] * wpg + sub] = word;
      } else {
        const int base = 8 * (sub & 1);               // bit index of this lane's first weight in its half
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          // t = -1 only for a negative nonzero weight (-0.0 and non-finite give +1)
          const uint32_t nz = (P[j] + 0x7FFF7FFFu) & 0x80008000u;
          const uint32_t one = ~(h[j] & nz) & 0x80008000u;
          word |= one >> (15 - base - j);
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

// One 128-weight group per lane (ternary only; see the work layout above).
constexpr int64_t kQuantLaneGroups = (int64_t)1 << 21;   // from this many groups on

__global__ __launch_bounds__(256) void quantize_lane_kernel(const uint16_t* __restrict__ W, int64_t ldw, int64_t N,
                                                            int G, uint32_t* __restrict__ packed,
                                                            uint16_t* __restrict__ scales, int32_t* counter) {
  const int64_t total = N * G;
  const int64_t lanes = (int64_t)gridDim.x * blockDim.x;
  int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  // (row, col) of group gid, advanced by the grid stride without a division per pass
  const int64_t srow = lanes / G;
  const int scol = (int)(lanes - srow * G);
  int64_t row = gid / G;
  int col = (int)(gid - row * G);
  int bad = 0;
  for (; gid < total; gid += lanes) {
    const uint16_t* src = W + row * ldw + 128 * col;
    uint32_t h[64];                                  // pair p: weights 2p (low half), 2p + 1
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const u32x4 v = *(const u32x4*)(src + 8 * i);
      h[4 * i] = v[0];
      h[4 * i + 1] = v[1];
      h[4 * i + 2] = v[2];
      h[4 * i + 3] = v[3];
    }
    uint32_t mx = 0;
#pragma unroll
    for (int p = 0; p < 64; ++p) mx = max16x2(mx, h[p] & 0x7FFF7FFFu);
    if ((mx & 0xFFFFu) >= 0x7C00u || (mx >> 16) >= 0x7C00u) {
      // count the non-finite weights and let them act as +0.0 (magnitude cleared)
#pragma unroll
      for (int p = 0; p < 64; ++p) {
        const uint32_t nf = ((h[p] & 0x7FFF7FFFu) + 0x04000400u) & 0x80008000u;
        bad += __builtin_popcount(nf);
        h[p] &= ~(nf - (nf >> 15));
      }
    }
    // exact FP64 sum of the magnitudes (four chains)
    double part[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int p = 0; p < 64; ++p) {
      part[p & 3] += (double)half_bits_to_float((uint16_t)(h[p] & 0x7FFFu));
      part[p & 3] += (double)half_bits_to_float((uint16_t)((h[p] >> 16) & 0x7FFFu));
    }
    const double sum = (part[0] + part[1]) + (part[2] + part[3]);
    const uint32_t thr = f16_floor_ratio(7.0 * sum);
    const uint32_t thr2 = thr | (thr << 16);
    double ksum = 0.0;
    int cnt = 0;
    u32x4 out[2];
#pragma unroll
    for (int u = 0; u < 8; ++u) {                    // INT2 word u: weights 16u .. 16u + 15
      uint32_t word = 0;
      float kept = 0.0f;                            // exact: 16 kept weights
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t hp = h[8 * u + j];
        const uint32_t keep = sub16x2(thr2, hp & 0x7FFF7FFFu) & 0x80008000u;   // |w| > threshold
        cnt += __builtin_popcount(keep);
        // code 01 for +1, 11 for -1 at bits 2j (weight 2j) and 16 + 2j (weight 2j + 1)
        word |= (keep >> (15 - 2 * j)) | ((hp & keep) >> (14 - 2 * j));
        const uint32_t hk = hp & (keep - (keep >> 15));   // kept magnitudes, the others 0
        kept += half_bits_to_float((uint16_t)(hk & 0xFFFFu));
        kept += half_bits_to_float((uint16_t)(hk >> 16));
      }
      out[u >> 2][u & 3] = word;
      ksum += (double)kept;
    }
    uint32_t* dst = packed + row * ((int64_t)G * 8) + 8 * col;
    *(u32x4*)dst = out[0];
    *(u32x4*)(dst + 4) = out[1];
    scales[row * G + col] = (uint16_t)(cnt ? f64_to_f16_rne(ksum / (double)cnt) : 0u);
    col += scol;
    row += srow + (col >= G ? 1 : 0);
    col -= col >= G ? G : 0;
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

// variant: 8 forces quantize_kernel, 9 the lane kernel (ternary); otherwise
// ternary launches of at least kQuantLaneGroups groups take the lane kernel.
hipError_t launch_quantize(int fmt, const uint16_t* W, int64_t ldw, int64_t N, int64_t K, uint8_t* packed,
                           uint16_t* scales, int32_t* counter, int variant, hipStream_t st) {
  if (counter) hipLaunchKernelGGL(quant_zero_kernel, dim3(1), dim3(1), 0, st, counter);
  const int G = (int)(K / 128);
  if (fmt == FMT_TERNARY && (variant == 9 || (variant != 8 && N * G >= kQuantLaneGroups))) {
    // at most 8192 workgroups (2^21 lanes, the same groups per pass as the
    // eighths' grid below); the lanes walk the rest
    int64_t blocks = (N * G + 255) / 256;
    blocks = blocks < 1 ? 1 : (blocks > 8192 ? 8192 : blocks);
    hipLaunchKernelGGL(quantize_lane_kernel, dim3((int)blocks), dim3(256), 0, st, W, ldw, N, G,
                       (uint32_t*)packed, scales, counter);
    return hipGetLastError();
  }
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
