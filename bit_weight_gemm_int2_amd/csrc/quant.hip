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
//    bits), and the lane reductions below give every lane of a team the
//    same sum S;
//  * |w| > 0.7 mean|w| means 1280 |w| > 7 S. For an FP16 value x and a real
//    t >= 0, x > t holds exactly when x > RD(t), RD(t) being the largest FP16
//    value at or below t; for non-negative FP16 values the order of the bit
//    patterns is the order of the values. So the test is an integer compare
//    of the 15-bit magnitude against RD(7 S / 1280), found once per group
//    (f16_floor_ratio) and applied to two weights at once;
//  * every kept weight exceeds 0.7 S / 128 >= 0.7 max|w| / 128 > 2^(E-8),
//    with 2^E <= max|w| < 2^(E+1), so it is a multiple of 2^(E-18); the kept
//    weights of one 16-weight INT2 word then sum to a multiple of 2^(E-18)
//    below 2^(E+5), 23 significant bits, which FP32 holds exactly in any
//    order. Word sums are added in FP64;
//  * the kept mean sum / count is one correctly rounded FP64 division; a
//    quotient with denominator <= 128 either is a 12-bit number (then the
//    division is exact) or lies at least 2^-19 (relative) from every FP16
//    rounding midpoint, so rounding the FP64 quotient to FP16 gives the
//    FP16 rounding of the exact mean;
//  * that last rounding is done on the FP64 bit pattern (f64_to_f16_rne).
//
// Work layout: HBM-bound (2 bytes read, 0.25 or 0.125 written per weight).
// A team of LPG lanes (a power of two up to 8) owns one 128-weight group at a
// time, GPT consecutive groups of the flattened [N][K/128] group array per
// pass, so that every lane has at least four 16-byte loads in flight; lane
// `sub` of the team holds the weights 128/LPG sub .. 128/LPG (sub + 1) - 1 of
// each group and writes their packed words (binary teams of eight pair
// their half words with one lane move). Group sums are added across the
// team with DPP moves (neighbour swap, pair swap, half-row mirror). Weights
// stay in their 32-bit pairs: magnitudes, keep flags (one packed 16-bit
// subtract per pair), signs and codes are formed two at a time with bit
// operations, and non-finite weights are looked for with one packed maximum
// per pair (only a wave that holds one takes the branch that counts and
// clears them). The per-group work (threshold, division, rounding) is done
// by every lane of the team. Team size: ternary 2 (fewer lanes repeat the
// per-group work; eight lanes issue 45 % more instructions, one lane per
// group holds 64 pairs in registers and leaves too few waves), binary 8
// (its per-group work is small, and eight lanes per group reach the copy
// rate).
#include "common.h"

namespace lowbit {

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
template <int CTRL>
__device__ __forceinline__ int dppT(int v) { return dpp32<CTRL>(v); }
template <int CTRL>
__device__ __forceinline__ uint32_t dppT(uint32_t v) { return (uint32_t)dpp32<CTRL>((int)v); }
template <int CTRL>
__device__ __forceinline__ double dppT(double v) { return dpp64<CTRL>(v); }

// Sum over the LPG lanes of a team (aligned groups of 2, 4 or 8 lanes); every
// lane gets the total.
template <int LPG, class T>
__device__ __forceinline__ T team_sum(T v) {
  if constexpr (LPG >= 2) v += dppT<0xB1>(v);
  if constexpr (LPG >= 4) v += dppT<0x4E>(v);
  if constexpr (LPG >= 8) v += dppT<0x141>(v);
  return v;
}

// Both 16-bit halves: a - b modulo 2^16 (bit 15 / 31: b > a for 15-bit values).
__device__ __forceinline__ uint32_t sub16x2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, a) - __builtin_bit_cast(u16x2, b));
}
__device__ __forceinline__ uint32_t max16x2(uint32_t a, uint32_t b) {
  const u16x2 x = __builtin_bit_cast(u16x2, a), y = __builtin_bit_cast(u16x2, b);
  return __builtin_bit_cast(uint32_t, u16x2{x[0] > y[0] ? x[0] : y[0], x[1] > y[1] ? x[1] : y[1]});
}

// LPG lanes per group (ternary: 1, 2 or 8; binary: 8).
template <bool TERN, int LPG>
__global__ __launch_bounds__(256) void quantize_team_kernel(const uint16_t* __restrict__ W, int64_t ldw, int64_t N,
                                                            int G, uint32_t* __restrict__ packed,
                                                            uint16_t* __restrict__ scales, int32_t* counter) {
  static_assert(TERN || LPG == 8, "binary groups are taken by eight lanes");
  // weights, 32-bit pairs and 16-byte loads per lane and group; groups per
  // team and pass
  constexpr int WPL = 128 / LPG, PPL = WPL / 2, NLD = WPL / 8;
  constexpr int GPT = NLD >= 4 ? 1 : 4 / NLD;
  const int sub = threadIdx.x & (LPG - 1);
  const int64_t total = N * G;
  const int64_t team = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / LPG;
  const int64_t teams = ((int64_t)gridDim.x * blockDim.x) / LPG;
  int bad = 0;
  // the group `first` as (row r0, column c0), advanced by the grid stride
  // without a division per pass
  const int64_t stride = teams * GPT, srow = stride / G;
  const int scol = (int)(stride - srow * G);
  int64_t r0 = (team * GPT) / G;
  int c0 = (int)(team * GPT - r0 * G);
  // every lane of a team takes the same trip count and the same groups, so
  // the team is either wholly active or wholly idle at each exchange
  for (int64_t first = team * GPT; first < total; first += stride) {
    uint32_t h[GPT][PPL];                           // pair p: weights 2p (low half), 2p + 1
    int64_t row[GPT];
    int col[GPT];
#pragma unroll
    for (int q = 0; q < GPT; ++q) {
      row[q] = q == 0 ? r0 : (col[q - 1] + 1 == G ? row[q - 1] + 1 : row[q - 1]);
      col[q] = q == 0 ? c0 : (col[q - 1] + 1 == G ? 0 : col[q - 1] + 1);
      // past the end: reread the last group (nothing of it is written)
      const bool in = first + q < total;
      const uint16_t* src = W + (in ? row[q] : N - 1) * ldw + 128 * (in ? col[q] : G - 1) + WPL * sub;
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const u32x4 v = *(const u32x4*)(src + 8 * i);
        h[q][4 * i] = v[0];
        h[q][4 * i + 1] = v[1];
        h[q][4 * i + 2] = v[2];
        h[q][4 * i + 3] = v[3];
      }
    }
    c0 += scol;
    r0 += srow + (c0 >= G ? 1 : 0);
    c0 -= c0 >= G ? G : 0;
#pragma unroll
    for (int q = 0; q < GPT; ++q) {
      const bool live = first + q < total;
      uint32_t mx = 0;
#pragma unroll
      for (int p = 0; p < PPL; ++p) mx = max16x2(mx, h[q][p] & 0x7FFF7FFFu);
      if (__ballot((mx & 0xFFFFu) >= 0x7C00u || (mx >> 16) >= 0x7C00u)) {
        // count the non-finite weights and let them act as +0.0 (magnitude cleared)
#pragma unroll
        for (int p = 0; p < PPL; ++p) {
          const uint32_t nf = ((h[q][p] & 0x7FFF7FFFu) + 0x04000400u) & 0x80008000u;
          bad += live ? __builtin_popcount(nf) : 0;
          h[q][p] &= ~(nf - (nf >> 15));
        }
      }
      double part[2] = {0.0, 0.0};                  // exact FP64 sums of the magnitudes
#pragma unroll
      for (int p = 0; p < PPL; ++p) {
        part[p & 1] += (double)half_bits_to_float((uint16_t)(h[q][p] & 0x7FFFu));
        part[p & 1] += (double)half_bits_to_float((uint16_t)((h[q][p] >> 16) & 0x7FFFu));
      }
      const double sum = team_sum<LPG>(part[0] + part[1]);
      uint32_t sbits;
      if constexpr (TERN) {
        constexpr int WD = WPL / 16;                  // INT2 words per lane
        const uint32_t thr = f16_floor_ratio(7.0 * sum);
        const uint32_t thr2 = thr | (thr << 16);
        double ksum = 0.0;
        int cnt = 0;
        uint32_t words[WD];
#pragma unroll
        for (int u = 0; u < WD; ++u) {
          uint32_t word = 0;
          float kept = 0.0f;                          // exact: one word's kept weights
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const uint32_t hp = h[q][8 * u + j];
            const uint32_t keep = sub16x2(thr2, hp & 0x7FFF7FFFu) & 0x80008000u;   // |w| > threshold
            cnt += __builtin_popcount(keep);
            // code 01 for +1, 11 for -1 at bits 2j (weight 2j) and 16 + 2j (weight 2j + 1)
            word |= (keep >> (15 - 2 * j)) | ((hp & keep) >> (14 - 2 * j));
            const uint32_t hk = hp & (keep - (keep >> 15));   // kept magnitudes, the others 0
            kept += half_bits_to_float((uint16_t)(hk & 0xFFFFu));
            kept += half_bits_to_float((uint16_t)(hk >> 16));
          }
          words[u] = word;
          ksum += (double)kept;
        }
        ksum = team_sum<LPG>(ksum);
        cnt = team_sum<LPG>(cnt);
        sbits = cnt ? f64_to_f16_rne(ksum / (double)cnt) : 0u;
        if (live) {
          uint32_t* dst = packed + row[q] * ((int64_t)G * 8) + 8 * col[q] + WD * sub;
          if constexpr (WD == 1) *dst = words[0];
          else if constexpr (WD == 2) *(u32x2*)dst = u32x2{words[0], words[1]};
          else {
#pragma unroll
            for (int v4 = 0; v4 < WD / 4; ++v4)
              *(u32x4*)(dst + 4 * v4) = u32x4{words[4 * v4], words[4 * v4 + 1], words[4 * v4 + 2], words[4 * v4 + 3]};
          }
        }
      } else {
        // bit 1 for t = +1: every weight but a negative nonzero one (-0.0 and
        // non-finite give +1); this lane's 8 pairs are half of binary word
        // sub / 2, at bits 8 (sub & 1) + p and 16 + 8 (sub & 1) + p
        uint32_t word = 0;
#pragma unroll
        for (int p = 0; p < PPL; ++p) {
          const uint32_t hp = h[q][p];
          const uint32_t nz = ((hp & 0x7FFF7FFFu) + 0x7FFF7FFFu) & 0x80008000u;
          word |= (~(hp & nz) & 0x80008000u) >> (15 - 8 * (sub & 1) - p);
        }
        sbits = f64_to_f16_rne(sum * 0.0078125);      // sum / 128, exact
        word |= dppT<0xB1>(word);
        if (live && (sub & 1) == 0) packed[row[q] * ((int64_t)G * 4) + 4 * col[q] + (sub >> 1)] = word;
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

// One launch of the team kernel, LPG lanes per group.
template <bool TERN, int LPG>
static void launch_team(const uint16_t* W, int64_t ldw, int64_t N, int G, uint8_t* packed, uint16_t* scales,
                        int32_t* counter, hipStream_t st) {
  constexpr int NLD = 128 / LPG / 8, GPT = NLD >= 4 ? 1 : 4 / NLD;
  // at most 2^21 groups a pass (the teams walk the rest)
  constexpr int64_t kMaxBlocks = ((int64_t)1 << 21) / GPT * LPG / 256;
  int64_t blocks = ((N * G + GPT - 1) / GPT * LPG + 255) / 256;
  blocks = blocks < 1 ? 1 : (blocks > kMaxBlocks ? kMaxBlocks : blocks);
  hipLaunchKernelGGL((quantize_team_kernel<TERN, LPG>), dim3((int)blocks), dim3(256), 0, st, W, ldw, N, G,
                     (uint32_t*)packed, scales, counter);
}

// variant (test hook): 8 forces eight lanes per ternary group, 9 one lane.
hipError_t launch_quantize(int fmt, const uint16_t* W, int64_t ldw, int64_t N, int64_t K, uint8_t* packed,
                           uint16_t* scales, int32_t* counter, int variant, hipStream_t st) {
  if (counter) hipLaunchKernelGGL(quant_zero_kernel, dim3(1), dim3(1), 0, st, counter);
  const int G = (int)(K / 128);
  if (fmt != FMT_TERNARY) launch_team<false, 8>(W, ldw, N, G, packed, scales, counter, st);
  else if (variant == 8) launch_team<true, 8>(W, ldw, N, G, packed, scales, counter, st);
  else if (variant == 9) launch_team<true, 1>(W, ldw, N, G, packed, scales, counter, st);
  else launch_team<true, 2>(W, ldw, N, G, packed, scales, counter, st);
  return hipGetLastError();
}

}  // namespace lowbit
