// gfx950 low-bit-weight GEMM, large M: Y = act(X W^T + bias), W = scale_g * t.
//
// The weight definition is the one of "Como Bonsai Ternary 4B revoluciona la
// difusion texto-imagen", section "Representacion y almacenamiento de los
// pesos ternarios": w = scale_g * t, one FP16 scale per 128 weights along K,
// t stored with 2 bits (ternary) or 1 bit (binary).
//
// For every output element and every 128-group g the kernel computes
//   P_g = sum_{k in g} x_k * (2 t_k)        (MFMA, FP32 accumulation, exact
//                                             products: 2t is 0 or +-2)
//   acc += (s_g / 2) * P_g                  (FP32, in Horner form, below)
// which is the definition up to FP32 rounding order. Zero, subnormal and
// negative scales need no special case. The same kernel runs the 4-bit
// format with zero points (128 + q on the MFMA, the zero point's share taken
// off with the activations' group sums). The small-M kernels and the
// dispatcher are in gemm.hip.
//
// MFMA: v_mfma_f32_32x32x16_{bf16,f16}. Lane l supplies
// operand row / output column l % 32 and K slots 8*(l/32) .. +7 of each MFMA.
// The K order inside a 128-group is free as long as both operands use the same
// one, so lane group q = l/32 owns k-local [64q, 64q+64) of every group and
// MFMA step s (0..7) uses its slots 64q + 8s .. +7: a lane reads its
// activations as 16 contiguous bytes per step and its codes for the whole
// group as one 16-byte (ternary) or 8-byte (binary) load.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "common.h"

namespace lowbit {

// ===========================================================================
// Large-M kernel (v_mfma_f32_32x32x16): a workgroup computes a BMT x 64 WN
// tile of Y with WN waves side by side along N, each wave BMT x 64 (BMT/32
// x 2 blocks of 32 x 32). One pipeline stage is one 128-group along K.
// Configurations (chosen per shape by the launcher):
//  * BMT = 128, WN = 8 (two waves per SIMD), three LDS stages: one
//    workgroup per CU (WN = 4 for narrow N);
//  * BMT = 96, WN = 4, two stages: two workgroups per CU.
//
//  * Everything a group needs reaches LDS through direct LDS DMA loads
//    (global_load_lds, issued from inline assembly with a scalar base and a
//    loop-invariant lane offset), so no global load writes or reads a
//    register the loop rewrites, and the only wait on loads in the loop is
//    the explicit one at each group start (compiler-placed waits on register
//    loads that cross the loop back-edge drain every load in flight):
//    - activations: BMT rows x 256 bytes; each row's sixteen 16-byte chunks
//      are XOR-swizzled by row % 16, which makes the fragment reads (32 rows,
//      same chunk) bank-conflict free;
//    - the packed codes of each wave's 64 columns, [column][32 bytes]
//      (ternary; the two 16-byte halves swapped when bit 3 of the column is
//      set, which keeps the fragment reads bank-conflict free) or
//      [column][16 bytes] (binary);
//    - each wave's 64 fp16 scales, one 4-byte LDS slot each.
//  * Three stages: at the start of group g a wave waits until only its
//    loads of stage g+1 are in flight (stage g was issued two groups
//    earlier), passes the barrier, and issues stage g+2 into the buffer of
//    group g-1. Two stages: it waits for all its loads (stage g, issued one
//    group earlier), passes the barrier and issues stage g+1 into the buffer
//    of group g-1. The DMAs of that stage are spread over the group's first
//    MFMA steps (all eight with three stages, four with two) rather than
//    issued in one burst after the barrier.
//  * Per MFMA step the wave reads the A fragments of the next step while
//    the MFMAs of the current step run; the B operands of the step are
//    unpacked from the group's codes (one 16- or 8-byte LDS read per column
//    block and group).
//  * Group scales, Horner form: the MFMAs accumulate in units of the current
//    group's scale c_g = +-s_g / 2, and at each group boundary the accumulator
//    is rescaled by c_{g-1} / c_g (one FP32 multiply per element; the ratio
//    itself from the hardware reciprocal); after the last group it is
//    multiplied by c_G. In exact arithmetic this is sum_g c_g P_g; in FP32
//    each rescale adds a few roundings (about 4G ulps of relative error over
//    the whole sum, far inside the 1e-3 tolerance). A
//    group whose scale is zero is fed as zero codes and keeps the previous
//    reference scale, so zero and subnormal scales are exact. Requires finite
//    scales and |partial sums| < 2^100 (the quotient of two FP16 scales is at
//    most 2^40, so a partial sum can grow by that much in accumulator units).
//
// K order inside a group: lane group q = lane / 32 owns k-local [64q, 64q+64);
// MFMA step s (0..7) uses its slots 64q + 8s .. +7.
// ===========================================================================
namespace large {
// WN waves side by side along N: a tile is BMT x 64 WN (BMT = 128 by default)
constexpr int BM = 128;
constexpr int ROW_BYTES = 256;                 // 128 k x 2 bytes
template <int BMT> constexpr int x_bytes() { return BMT * ROW_BYTES; }   // activations per stage
template <int WN> constexpr int bn() { return 64 * WN; }
// LDS bytes of packed codes per column and group (binary uses 16 of its 32)
template <int FMT> constexpr int code_bytes() { return FMT == FMT_INT4 ? 64 : 32; }
template <int FMT, int WN> constexpr int w_bytes() { return bn<WN>() * code_bytes<FMT>(); }
template <int WN> constexpr int s_bytes() { return bn<WN>() * 4; }    // scales, 4-byte slots
// a stage: activations, codes, scales, and for the 4-bit format the zero
// points (4-byte slots) and the tile rows' activation sums of the group
template <int FMT, int WN, int BMT> constexpr int stage_bytes() {
  return x_bytes<BMT>() + w_bytes<FMT, WN>() + s_bytes<WN>() + (FMT == FMT_INT4 ? s_bytes<WN>() + BMT * 4 : 0);
}
// DMA loads per wave and stage: activations (BMT rows, 4 per load, split
// over the waves) + codes (2 ternary, 1 binary, 4 for 4-bit) + scales (1)
// (+ zero points and row sums for 4-bit)
template <int FMT, int WN, int BMT>
constexpr int stage_loads() {
  return BMT / (4 * WN) + (FMT == FMT_TERNARY ? 2 : FMT == FMT_INT4 ? 4 : 1) + 1 + (FMT == FMT_INT4 ? 2 : 0);
}
}  // namespace large

template <bool BF16, int FMT, int WN, int BMT = 128, int NST = 3>
__global__ __launch_bounds__(64 * WN) void gemm_large_kernel(GemmArgs a, int tiles_m, int tiles_n, int xcd_rows) {
  using namespace large;
  constexpr bool TERN = FMT == FMT_TERNARY, I4 = FMT == FMT_INT4;
  constexpr int BN = bn<WN>(), XR = BMT / (4 * WN);     // activation loads per wave and stage
  constexpr int IB = BMT / 32;                          // 32-row blocks per wave
  constexpr int CB = code_bytes<FMT>();
  constexpr int X_BYTES = x_bytes<BMT>(), W_BYTES = w_bytes<FMT, WN>(), STAGE_BYTES = stage_bytes<FMT, WN, BMT>();
  constexpr int RW = BMT / WN;                          // 4-bit: row sums each wave copies per stage
  static_assert(!I4 || (NST == 2 && RW % 4 == 0), "4-bit: two stages, row sums in 16-byte loads");
  static_assert(NST == 2 || NST == 3, "two or three stages");
  static_assert(BMT % (4 * WN) == 0 && BMT % 32 == 0, "tile height");
  static_assert(WN * BMT * 128 <= NST * STAGE_BYTES, "epilogue staging fits in the stages");
  __shared__ __align__(16) uint8_t smem[NST][STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63, q = lane >> 5, r32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // XCD-aware tile order: workgroup i runs on XCD i % 8 (round-robin
  // dispatch), and each XCD gets one eighth of the tiles to share its L2
  // (plan: xcd_order). xcd_rows = 0: a contiguous range of tiles, N fastest;
  // xcd_rows = a > 0: the tile grid cut into a x (8 / a) equal blocks, block
  // x for XCD x, row by row inside it (so the packed codes of a block's
  // columns stay in the XCD's L2 while its rows stream through).
  int tm_i, tn_i;
  {
    const int T = tiles_m * tiles_n;
    const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
    if (xcd_rows > 0) {
      const int b = 8 / xcd_rows, cols = tiles_n / b;
      tm_i = (x / b) * (tiles_m / xcd_rows) + j / cols;
      tn_i = (x % b) * cols + j % cols;
    } else {
      const int t = (T & 7) == 0 ? x * (T >> 3) + j : (int)blockIdx.x;
      tm_i = t / tiles_n;
      tn_i = t % tiles_n;
    }
  }
  const int m0 = tm_i * BMT, n0 = tn_i * BN;
  const int G = a.K >> 7;
  // K split (gridDim.y > 1, 4-bit launches only): this workgroup takes the
  // groups [gb, ge) and leaves an FP32 partial tile; one split: all of K
  const int gb = (int)(((int64_t)G * blockIdx.y) / gridDim.y), ge = (int)(((int64_t)G * (blockIdx.y + 1)) / gridDim.y);
  const int64_t wrow = I4 ? (a.K >> 1) : TERN ? (a.K >> 2) : (a.K >> 3);
  const float factor = I4 ? 1.0f : code_factor<TERN>();
  const int wcol0 = n0 + 64 * wave;                     // first column of this wave

  // ---- stage g -> LDS buffer `buf` (DMA only) ----
  // Per-lane byte offsets are computed once; per group only the wave-uniform
  // base pointers move (the loads then address as scalar base + 32-bit lane
  // offset, and no vector register a DMA in flight reads is rewritten).
  uint32_t xoff[XR];
#pragma unroll
  for (int it = 0; it < XR; ++it) {
    const int r = 4 * XR * wave + 4 * it + (lane >> 4);
    const int c = (lane & 15) ^ (r & 15);               // chunk stored in slot lane&15
    const int m = min(m0 + r, a.M - 1);                 // rows past M: any valid row
    xoff[it] = (uint32_t)(((int64_t)m * a.ldx + 8 * c) * 2);
  }
  uint32_t woff[I4 ? 4 : 2], soff;
  if (I4) {
    // 64 bytes per column: LDS slot h of local column c holds 16-byte chunk
    // h ^ ((c >> 2) & 3), which keeps the fragment reads bank-conflict free
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int c = 16 * it + (lane >> 2);
      woff[it] = (uint32_t)(min(wcol0 + c, a.N - 1) * wrow + 16 * ((lane & 3) ^ ((c >> 2) & 3)));
    }
  } else if (TERN) {
    // LDS slot h of local column c holds 16-byte half h ^ bit 3 of c, so the
    // fragment reads (16 consecutive columns, same half) hit distinct banks
#pragma unroll
    for (int it = 0; it < 2; ++it) {                    // columns past N: any valid column
      const int c = 32 * it + (lane >> 1);
      woff[it] = (uint32_t)(min(wcol0 + c, a.N - 1) * wrow + 16 * ((lane & 1) ^ ((c >> 3) & 1)));
    }
  } else {
    woff[0] = woff[1] = (uint32_t)(min(wcol0 + lane, a.N - 1) * wrow);
  }
  soff = (uint32_t)(min(wcol0 + lane, a.N - 1) * (int64_t)G * 2);
  // DMA number d of stage g into LDS buffer `buf`, in this order: the
  // activation rows (XR), the codes (one to four), the scales, and for the
  // 4-bit format the zero points and the row sums
  constexpr int NCODE = I4 ? 4 : TERN ? 2 : 1;
  constexpr int ND = XR + NCODE + 1 + (I4 ? 2 : 0);
  static_assert(ND == stage_loads<FMT, WN, BMT>(), "DMA count");
  auto dma = [&](int g, int buf, int d) __attribute__((always_inline)) {
    uint8_t* base = smem[buf];
    if (d < XR) {
      const uint8_t* xg = (const uint8_t*)a.X + ((int64_t)g << 8);
      dma_lds16(xg, xoff[d], lds_addr(base + (4 * XR * wave + 4 * d) * ROW_BYTES));
    } else if (d < XR + NCODE) {
      const uint8_t* wg = a.W + g * (I4 ? 64 : TERN ? 32 : 16);
      dma_lds16(wg, woff[d - XR], lds_addr(base + X_BYTES + wave * (64 * CB) + 1024 * (d - XR)));
    } else if (d == XR + NCODE) {
      // scales: lane l -> 4-byte slot l (2-byte load, zero-extended)
      dma_lds2((const uint8_t*)a.S + 2 * g, soff, lds_addr(base + X_BYTES + W_BYTES + wave * 256));
    } else if (d == XR + NCODE + 1) {
      // zero points likewise
      dma_lds2((const uint8_t*)a.Z + 2 * g, soff, lds_addr(base + X_BYTES + W_BYTES + BN * 4 + wave * 256));
    } else {
      // this wave's RW rows of the group's row sums (row-sum array padded
      // past M, so every row read exists)
      const float* rg = a.ws + g * a.ldr + m0 + RW * wave;
      if (lane < RW / 4)
        dma_lds16(rg, 16 * lane, lds_addr(base + X_BYTES + W_BYTES + 2 * BN * 4 + 4 * RW * wave));
    }
  };
  auto stage = [&](int g, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int d = 0; d < ND; ++d) dma(g, buf, d);
  };
  // Inside the loop a stage's DMAs are spread over the first NP MFMA steps
  // of the group (about one per step with three stages; over half the group
  // with two, whose next wait comes one group later). Issued all at once
  // right after the barrier, they would queue on the CU's memory pipeline
  // and hold every wave's rescale and first MFMAs behind them.
  constexpr int NP = NST == 3 ? 8 : 4;

  auto afrag = [&](const uint8_t* xb, int i, int s) -> u32x4 {
    const int r = 32 * i + r32;
    const int p = (8 * q + s) ^ (r & 15);
    return *(const u32x4*)(xb + r * ROW_BYTES + p * 16);
  };

  f32x16 acc[IB][2];
#pragma unroll
  for (int i = 0; i < IB; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  float cref[2] = {1.0f, 1.0f};                 // reference scale of the accumulator

  stage(gb, 0);
  if (NST == 3 && gb + 1 < ge) stage(gb + 1, 1);
  int buf = 0;
  // One group; MORE: the group NST - 1 ahead is staged during this one (the
  // last NST - 1 groups run the same body without it, so no DMA is in flight
  // after the last group that the epilogue would have to wait for).
  auto run_group = [&](int g, auto more_tag) __attribute__((always_inline)) {
    constexpr bool MORE = decltype(more_tag)::value;
    // stage g complete (three stages: only this wave's stage g+1 loads, if
    // there is a group g+1, may be in flight), and every wave's part of it
    // visible
    if (NST == 3 && g + 1 < ge) __builtin_amdgcn_s_waitcnt(waitcnt_vm(stage_loads<FMT, WN, BMT>()));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
    // the stage issued during this group (group g+2 with three stages, g+1
    // with two) goes into the buffer of group g-1, which every wave has
    // finished reading once past the barrier (4-bit: past the end, a copy
    // of the last group into a buffer nobody reads)
    const int sg = min(NST == 3 ? g + 2 : g + 1, ge - 1);
    const int sb = NST == 3 ? (buf == 0 ? 2 : buf - 1) : buf ^ 1;
    const uint8_t* xb = smem[buf];
    const uint8_t* wb = smem[buf] + X_BYTES + wave * (64 * CB);
    const uint8_t* sbuf = smem[buf] + X_BYTES + W_BYTES + wave * 256;

    // codes, scale and Horner rescale of each column block
    u32x4 bw[2], bw2[2];
    uint32_t tm[2], mk[2], bs[2];
    float zc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = 32 * j + r32;
      if (I4) {
        const int sw = (col >> 2) & 3;
        bw[j] = *(const u32x4*)(wb + col * 64 + 16 * ((2 * q) ^ sw));
        bw2[j] = *(const u32x4*)(wb + col * 64 + 16 * ((2 * q + 1) ^ sw));
      } else if (TERN) {
        bw[j] = *(const u32x4*)(wb + col * 32 + 16 * (q ^ ((col >> 3) & 1)));
      } else {
        const u32x2 v = *(const u32x2*)(wb + col * 16 + 8 * q);
        bw[j] = u32x4{v[0], v[1], 0u, 0u};
      }
      const float sc = factor * half_bits_to_float((uint16_t)*(const uint32_t*)(sbuf + col * 4));
      const bool zero = sc == 0.0f;
      // ratio of the old to the new reference scale, by the hardware
      // reciprocal (1 ulp): deterministic, and its error is one more
      // rounding-size term per group, far inside the accuracy bound
      const float r = zero ? 1.0f : cref[j] * __builtin_amdgcn_rcpf(sc);
      cref[j] = zero ? cref[j] : sc;
      tm[j] = zero ? 0u : I4 ? int4_mask<BF16>() : TERN_MASK;
      mk[j] = zero ? 0u : BIN_SIGN;
      bs[j] = zero ? 0u : I4 ? int4_base<BF16>() : BIN_TWO;
      if (I4) {
        // the MFMAs add sum x (128 + q); (128 + z) times the row sum comes off
        zc[j] = zero ? 0.0f : 128.0f + half_bits_to_float((uint16_t)*(const uint32_t*)(sbuf + BN * 4 + col * 4));
      }
#pragma unroll
      for (int i = 0; i < IB; ++i) acc[i][j] *= r;
    }

    // eight MFMA steps; the A fragments of step st+1 are read during step st
    u32x4 A[2][IB];
#pragma unroll
    for (int i = 0; i < IB; ++i) A[0][i] = afrag(xb, i, 0);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      if (st < 7) {
#pragma unroll
        for (int i = 0; i < IB; ++i) A[(st + 1) & 1][i] = afrag(xb, i, st + 1);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        u32x4 bf;
        if constexpr (I4) bf = int4_chunk<BF16>(st < 4 ? bw[j][st] : bw2[j][st - 4], tm[j], bs[j]);
        else if constexpr (TERN) bf = tern_chunk(bw[j][st >> 1], st & 1, tm[j]);
        else bf = bin_chunk(bw[j][st >> 2], st & 3, mk[j], bs[j]);
#pragma unroll
        for (int i = 0; i < IB; ++i) acc[i][j] = mfma32<BF16>(A[st & 1][i], bf, acc[i][j]);
      }
      // this step's share of the next stage's DMAs
      if constexpr (MORE) {
#pragma unroll
        for (int d = 0; d < ND; ++d)
          if (d * NP / ND == st) dma(sg, sb, d);
      }
    }
    if constexpr (I4) {
      // acc -= (128 + z) * (sum of the group's activations) per row, in the
      // group's scale units; lane rows 32 i + 8 e4 + 4 q + (0..3)
      const float* rs = (const float*)(smem[buf] + X_BYTES + W_BYTES + 2 * BN * 4);
#pragma unroll
      for (int i = 0; i < IB; ++i)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const f32x4 rv = *(const f32x4*)(rs + 32 * i + 8 * e4 + 4 * q);
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc[i][j][4 * e4 + e] = __builtin_fmaf(-zc[j], rv[e], acc[i][j][4 * e4 + e]);
        }
    }
    buf = NST == 3 ? (buf == 2 ? 0 : buf + 1) : buf ^ 1;
  };
  int g = gb;
  if constexpr (I4) {
    // one loop body: a second copy makes the eight-wave 4-bit instance spill
    for (; g < ge; ++g) run_group(g, std::true_type{});
  } else {
    for (; g + NST - 1 < ge; ++g) run_group(g, std::true_type{});
    for (; g < ge; ++g) run_group(g, std::false_type{});
  }
  __builtin_amdgcn_s_waitcnt(0);                       // no DMA may still write LDS

  // ---- epilogue: final scale, bias, activation, one RNE cast, store ----
  // (with a K split: the FP32 partial tile into plane blockIdx.y, nothing
  // else; the reduce kernel adds the planes in split order and finishes)
  if (gridDim.y > 1) {
    float* P = a.part + (int64_t)blockIdx.y * a.M * a.N;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + 64 * wave + 32 * j + r32;
      if (n >= a.N) continue;
      const float c = cref[j];
#pragma unroll
      for (int i = 0; i < IB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + 32 * i + 8 * (r >> 2) + 4 * q + (r & 3);
          if (m < a.M) P[(int64_t)m * a.N + n] = acc[i][j][r] * c;
        }
    }
    return;
  }
  const bool y16 = a.y_dtype != DT_F32;
  const bool vec = y16 && (a.ldy & 7) == 0 && ((uintptr_t)a.Y & 15) == 0;
  if (vec) {
    // 16-bit outputs go through LDS (each wave: its 128 x 64 tile, 16 KiB,
    // 16-byte chunks XOR-swizzled by row % 8) and leave as 16-byte stores
    // covering whole 128-byte row segments.
    __syncthreads();                                  // LDS stages are free now
    uint8_t* sY = &smem[0][0] + wave * (BMT * 128);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + 64 * wave + 32 * j + r32;
      const float b = (a.bias && n < a.N) ? load_bias(a.bias, a.bias_dtype, n) : 0.0f;
      const float c = cref[j];
      const int col = 32 * j + r32;
#pragma unroll
      for (int i = 0; i < IB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 32 * i + 8 * (r >> 2) + 4 * q + (r & 3);
          const float v = finish(acc[i][j][r] * c, b, a.act);
          const uint16_t h = a.y_dtype == DT_BF16 ? float_to_bf16_bits(v) : float_to_half_bits(v);
          const int chunk = (col >> 3) ^ (row & 7);
          *(uint16_t*)(sY + row * 128 + chunk * 16 + (col & 7) * 2) = h;
        }
    }
    __syncthreads();                                  // staged tile complete
#pragma unroll
    for (int it = 0; it < BMT / 8; ++it) {
      const int idx = it * 64 + lane;
      const int row = idx >> 3, ch = idx & 7;
      const int m = m0 + row, n = n0 + 64 * wave + 8 * ch;
      const u32x4 v = *(const u32x4*)(sY + row * 128 + ((ch ^ (row & 7)) * 16));
      if (m < a.M) {
        uint16_t* dst = (uint16_t*)a.Y + (int64_t)m * a.ldy + n;
        if (n + 8 <= a.N) {
          // non-temporal: the output is not read again by this launch, and
          // keeping it out of L2 leaves room for the activation and code
          // slices that the other workgroups of the XCD still read
          __builtin_nontemporal_store(v, (u32x4*)dst);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (n + e < a.N) dst[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + 64 * wave + 32 * j + r32;
      if (n >= a.N) continue;
      const float b = a.bias ? load_bias(a.bias, a.bias_dtype, n) : 0.0f;
      const float c = cref[j];
#pragma unroll
      for (int i = 0; i < IB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + 32 * i + 8 * (r >> 2) + 4 * q + (r & 3);
          if (m < a.M) store_out(a.Y, a.ldy, a.y_dtype, m, n, finish(acc[i][j][r] * c, b, a.act));
        }
    }
  }
}

// Row sums of the activations per 128-group for the 4-bit format:
// R[g][m] = sum_{k in group g} x[m][k] in FP32, rows m >= M up to the padded
// row count written as zeros. One thread per (group, row); sixteen sums of
// eight consecutive values, then a pairwise tree over the sixteen (at most
// 11 roundings on the way to any one result).
__global__ void rowsum_kernel(const uint16_t* X, int64_t ldx, int M, int G, int64_t ldr, float* R, int bf16) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < (int64_t)G * ldr;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int g = (int)(i / ldr);
    const int64_t m = i - (int64_t)g * ldr;
    float c16[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) c16[c] = 0.0f;
    if (m < M) {
      const uint16_t* x = X + m * ldx + ((int64_t)g << 7);
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const u32x4 v = *(const u32x4*)(x + 8 * c);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint16_t h = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
          c16[c] += bf16 ? bf16_bits_to_float(h) : half_bits_to_float(h);
        }
      }
    }
#pragma unroll
    for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
      for (int c = 0; c < w; ++c) c16[c] += c16[c + w];
    R[(int64_t)g * ldr + m] = c16[0];
  }
}

// The K-split 4-bit launch's second step: Y = act(sum over the splits, in
// split order, of the FP32 partial planes + bias), one RNE cast. One thread
// per output element (consecutive threads along N).
__global__ void splitk_finish_kernel(const float* __restrict__ part, int S, int M, int N, const void* bias,
                                     int bias_dtype, void* Y, int64_t ldy, int y_dtype, int act) {
  const int64_t plane = (int64_t)M * N;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < plane;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int m = (int)(i / N), n = (int)(i - (int64_t)m * N);
    float v = part[i];
    for (int s = 1; s < S; ++s) v += part[s * plane + i];
    const float b = bias ? load_bias(bias, bias_dtype, n) : 0.0f;
    store_out(Y, ldy, y_dtype, m, n, finish(v, b, act));
  }
}

// Large-M tile configurations:
//  * wide: 128 x 512 tiles, 8 waves (two per SIMD), three stages; one
//    workgroup fills a CU's LDS (128 x 256 and 4 waves when N < 2048);
//  * pair: 96 x 256 tiles, 4 waves, two stages (66 KiB of LDS), so two
//    independent workgroups share a CU: while one runs its epilogue (bias,
//    GELU, stores) or its group-boundary rescale the other keeps the MFMA
//    pipes busy; and with fewer tiles than CUs, the smaller tiles spread the
//    work over more CUs.
// The choice compares estimated times in units of tile area per CU:
//   wide: rounds of tiles over the CUs x tile area (4-wave wide tiles, one
//         wave per SIMD, at 0.69 of a full CU's rate);
//   pair: at most one tile per CU: tile area / 0.69; else rounds of two
//         tiles per CU x 2 x tile area x 0.93 (the overlap gain).
// The rates were measured on MI355X (1536 x 3072 x 3072: 36 against 67 us;
// 4608 x 9216 x 3072: 0.232 against 0.250 ms). Pair tiles are taken when
// they are estimated more than 3 % faster.
// variant: 5 forces wide tiles, 6 forces pair tiles.
static bool large_pair(int M, int N, int num_cu, int variant) {
  if (variant == 5) return false;
  if (variant == 6) return true;
  constexpr double ALONE = 0.69, OVERLAP = 0.93;
  const double P = num_cu;
  const bool w8 = N >= 2048;
  const double tw = (double)((M + 127) / 128) * ((N + (w8 ? 511 : 255)) / (w8 ? 512 : 256));
  const double tp = (double)((M + 95) / 96) * ((N + 255) / 256);
  const double wide = std::ceil(tw / P) * (w8 ? 128.0 * 512.0 : 128.0 * 256.0 / ALONE);
  const double pair = tp <= P ? 96.0 * 256.0 / ALONE : std::ceil(tp / (2 * P)) * 2.0 * 96.0 * 256.0 * OVERLAP;
  return pair < 0.97 * wide;
}

// Which eighth of the tile grid each XCD takes (the kernel's xcd_rows): a
// contiguous range (0) or a x (8 / a) equal blocks (a = 1, 2, 4, 8), the
// one with the fewest bytes an XCD must fetch into its 4 MB L2, estimated
// as its activation rows once plus its packed-code columns once if they fit
// in about 2.5 MB, else once per tile row that a round of its concurrently
// resident tiles starts (slots: workgroups resident on one XCD).
static int xcd_order(int M, int N, int K, int fmt, int tm, int tn, int bmt, int bn, int slots) {
  if ((tm * tn) % 8) return 0;
  const double xrow = 2.0 * K * bmt;                                 // bytes of one tile row of X
  const double wcol = (fmt == FMT_INT4 ? K / 2.0 : fmt == FMT_TERNARY ? K / 4.0 : K / 8.0) * bn +
                      (fmt == FMT_INT4 ? 4.0 : 2.0) * bn * (K / 128);
  auto cost = [&](double rows, double cols, double conc_rows) {
    const double w = cols * wcol;
    const double refetch = w <= 2.5e6 ? 1.0 : std::max(1.0, rows / std::max(1.0, conc_rows));
    return rows * xrow + w * refetch;
  };
  // contiguous ranges: T / 8 tiles, N fastest
  const double per = (double)tm * tn / 8;
  int best = 0;
  double bc = cost(per / tn, std::min<double>(tn, per), (double)slots / tn);
  for (int a = 1; a <= 8; a *= 2) {
    const int b = 8 / a;
    if (tm % a || tn % b) continue;
    const double c = cost((double)tm / a, (double)tn / b, (double)slots / (tn / b));
    if (c < 0.97 * bc) {
      bc = c;
      best = a;
    }
  }
  (void)M;
  (void)N;
  return best;
}

template <bool BF16, int FMT>
static void launch_large_t(const GemmArgs& a, int num_cu, int variant, hipStream_t st) {
  const int xcd_cu = std::max(1, num_cu / 8);
  if (large_pair(a.M, a.N, num_cu, variant)) {
    const int tm = (a.M + 95) / 96, tn = (a.N + 255) / 256;
    const int xr = xcd_order(a.M, a.N, a.K, FMT, tm, tn, 96, 256, 2 * xcd_cu);
    hipLaunchKernelGGL((gemm_large_kernel<BF16, FMT, 4, 96, 2>), dim3(tm * tn), dim3(256), 0, st, a, tm, tn, xr);
    return;
  }
  const int tm = (a.M + large::BM - 1) / large::BM;
  if (a.N >= 2048) {
    const int tn = (a.N + large::bn<8>() - 1) / large::bn<8>();
    const int xr = xcd_order(a.M, a.N, a.K, FMT, tm, tn, 128, 512, xcd_cu);
    hipLaunchKernelGGL((gemm_large_kernel<BF16, FMT, 8>), dim3(tm * tn), dim3(512), 0, st, a, tm, tn, xr);
  } else {
    const int tn = (a.N + large::bn<4>() - 1) / large::bn<4>();
    const int xr = xcd_order(a.M, a.N, a.K, FMT, tm, tn, 128, 256, xcd_cu);
    hipLaunchKernelGGL((gemm_large_kernel<BF16, FMT, 4>), dim3(tm * tn), dim3(256), 0, st, a, tm, tn, xr);
  }
}

// One large-M launch (ternary or binary codes), tile configuration chosen
// as above; called by the dispatcher (launch_gemm) for M > 16.
void launch_large(int fmt, bool x_bf16, const GemmArgs& a, int num_cu, int variant, hipStream_t st) {
  if (fmt == FMT_TERNARY) {
    if (x_bf16) launch_large_t<true, FMT_TERNARY>(a, num_cu, variant, st);
    else launch_large_t<false, FMT_TERNARY>(a, num_cu, variant, st);
  } else {
    if (x_bf16) launch_large_t<true, FMT_BINARY>(a, num_cu, variant, st);
    else launch_large_t<false, FMT_BINARY>(a, num_cu, variant, st);
  }
}

// Padded row count of the 4-bit row sums: every tile row the kernel reads.
int64_t int4_rows(int64_t M) { return (M + 127) / 128 * 128 + 128; }

struct Int4Plan {
  bool small;   // 64 x 256 tiles
  int splits;   // K split (1: none)
};

// Tile choice and K split of a 4-bit launch. 128-row tiles (128 x 512, or
// 128 x 256 for N < 2048) unless they number fewer than the CUs; then 64 x
// 256 tiles, two workgroups per CU, and while those still number no more
// than the CUs allow, K is split (at most 4 ways, at least 4 groups
// a split) so that splits x tiles stays within the CUs. variant 5 forces the
// 128-row tiles, 6 the 64-row tiles without a split, 7 the 64-row tiles with
// the largest split the groups allow (at most 4).
Int4Plan int4_plan(int M, int N, int K, int num_cu, int variant) {
  Int4Plan p{};
  const int G = K >> 7;
  const int64_t wide_tiles = (int64_t)((M + 127) / 128) * ((N + (N >= 2048 ? 511 : 255)) / (N >= 2048 ? 512 : 256));
  p.small = variant == 6 || variant == 7 || (variant != 5 && wide_tiles < num_cu);
  p.splits = 1;
  if (p.small) {
    const int64_t t = (int64_t)((M + 63) / 64) * ((N + 255) / 256);
    if (variant == 7) {
      p.splits = std::max(1, std::min(4, G / 4));
    } else if (variant != 6) {
      while (p.splits < 4 && t * (p.splits + 1) <= num_cu && G / (p.splits + 1) >= 4) ++p.splits;
    }
  }
  return p;
}

// Workspace of a 4-bit launch: the row sums, then (K split) the partial
// planes from the next 256-byte boundary.
size_t int4_workspace(int M, int N, int K, int num_cu, int variant) {
  const size_t sums = (size_t)(K / 128) * (size_t)int4_rows(M) * sizeof(float);
  const Int4Plan p = int4_plan(M, N, K, num_cu, variant);
  if (p.splits == 1) return sums;
  return (sums + 255) / 256 * 256 + (size_t)p.splits * M * N * sizeof(float);
}

// 4-bit GEMM (any M): the row sums, then the large-M kernel with two stages
// (a.ws: the row sums, a.ldr: int4_rows(M)). Tiles: 128 x 512 (eight waves,
// one workgroup per CU) or 128 x 256 for narrow N; when those would leave
// CUs idle (the prompt-sized M of a text encoder: 512 rows make 4 tile
// rows), 64 x 256 tiles of four waves, 68.5 KiB of LDS, two workgroups per
// CU. variant: 5 forces the 128-row tiles, 6 the 64-row tiles.
hipError_t launch_gemm_int4(bool x_bf16, GemmArgs a, int num_cu, int variant, hipStream_t st) {
  const int G = a.K >> 7;
  const int64_t work = (int64_t)G * a.ldr;
  const int64_t blocks = std::min<int64_t>((work + 255) / 256, 65535);
  hipLaunchKernelGGL(rowsum_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a.X, a.ldx, a.M, G, a.ldr, a.ws,
                     x_bf16 ? 1 : 0);
  const int tm = (a.M + large::BM - 1) / large::BM;
  const int xcd_cu = std::max(1, num_cu / 8);
  const Int4Plan plan = int4_plan(a.M, a.N, a.K, num_cu, variant);
  if (plan.small) {
    const int tm4 = (a.M + 63) / 64, tn = (a.N + 255) / 256;
    const int xr = xcd_order(a.M, a.N, a.K, FMT_INT4, tm4, tn, 64, 256, 2 * xcd_cu);
    const dim3 grid(tm4 * tn, plan.splits);
    if (plan.splits > 1) {
      const size_t sums = (size_t)(a.K / 128) * (size_t)a.ldr * sizeof(float);
      a.part = (float*)((uint8_t*)a.ws + (sums + 255) / 256 * 256);
    }
    if (x_bf16) hipLaunchKernelGGL((gemm_large_kernel<true, FMT_INT4, 4, 64, 2>), grid, dim3(256), 0, st, a, tm4, tn, xr);
    else hipLaunchKernelGGL((gemm_large_kernel<false, FMT_INT4, 4, 64, 2>), grid, dim3(256), 0, st, a, tm4, tn, xr);
    if (plan.splits > 1) {
      const int64_t n = (int64_t)a.M * a.N;
      const int64_t fb = std::min<int64_t>((n + 255) / 256, 16384);
      hipLaunchKernelGGL(splitk_finish_kernel, dim3((unsigned)fb), dim3(256), 0, st, (const float*)a.part,
                         plan.splits, a.M, a.N, a.bias, a.bias_dtype, a.Y, a.ldy, a.y_dtype, a.act);
    }
  } else if (a.N >= 2048) {
    const int tn = (a.N + large::bn<8>() - 1) / large::bn<8>();
    const int xr = xcd_order(a.M, a.N, a.K, FMT_INT4, tm, tn, 128, 512, xcd_cu);
    if (x_bf16) hipLaunchKernelGGL((gemm_large_kernel<true, FMT_INT4, 8, 128, 2>), dim3(tm * tn), dim3(512), 0, st, a, tm, tn, xr);
    else hipLaunchKernelGGL((gemm_large_kernel<false, FMT_INT4, 8, 128, 2>), dim3(tm * tn), dim3(512), 0, st, a, tm, tn, xr);
  } else {
    const int tn = (a.N + large::bn<4>() - 1) / large::bn<4>();
    const int xr = xcd_order(a.M, a.N, a.K, FMT_INT4, tm, tn, 128, 256, xcd_cu);
    if (x_bf16) hipLaunchKernelGGL((gemm_large_kernel<true, FMT_INT4, 4, 128, 2>), dim3(tm * tn), dim3(256), 0, st, a, tm, tn, xr);
    else hipLaunchKernelGGL((gemm_large_kernel<false, FMT_INT4, 4, 128, 2>), dim3(tm * tn), dim3(256), 0, st, a, tm, tn, xr);
  }
  return hipGetLastError();
}

}  // namespace lowbit
