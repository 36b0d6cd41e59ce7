// gfx950 low-bit-weight GEMM: Y = act(X W^T + bias), W = scale_g * t.
//
// The weight definition is the one of "Como Bonsai Ternary 4B revoluciona la
// difusion texto-imagen", section "Representacion y almacenamiento de los
// pesos ternarios": w = scale_g * t, one FP16 scale per 128 weights along K,
// t stored with 2 bits (ternary) or 1 bit (binary).
//
// Both kernels compute, for every output element and every 128-group g,
//   P_g = sum_{k in g} x_k * (2 t_k)        (MFMA, FP32 accumulation, exact
//                                             products: 2t is 0 or +-2)
//   acc += (s_g / 2) * P_g                  (FP32; the large-M kernel does
//                                             this in Horner form, below)
// which is the definition up to FP32 rounding order. Zero, subnormal and
// negative scales need no special case.
//
// MFMA: v_mfma_f32_32x32x16_{bf16,f16} in both kernels. Lane l supplies
// operand row / output column l % 32 and K slots 8*(l/32) .. +7 of each MFMA.
// The K order inside a 128-group is free as long as both operands use the same
// one, so lane group q = l/32 owns k-local [64q, 64q+64) of every group and
// MFMA step s (0..7) uses its slots 64q + 8s .. +7: a lane reads its
// activations as 16 contiguous bytes per step and its codes for the whole
// group as one 16-byte (ternary) or 8-byte (binary) load.
#include <cmath>

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
//    of group g-1.
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
// s_waitcnt immediate for vmcnt(n), expcnt(7), lgkmcnt(0)
constexpr int waitcnt_vm(int n) { return (n & 15) | (7 << 4) | ((n >> 4) << 14); }
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
  auto stage = [&](int g, int buf) {
    uint8_t* base = smem[buf];
    const uint8_t* xg = (const uint8_t*)a.X + ((int64_t)g << 8);
#pragma unroll
    for (int it = 0; it < XR; ++it)
      dma_lds16(xg, xoff[it], lds_addr(base + (4 * XR * wave + 4 * it) * ROW_BYTES));
    uint8_t* wb = base + X_BYTES + wave * (64 * CB);
    const uint8_t* wg = a.W + g * (I4 ? 64 : TERN ? 32 : 16);
    dma_lds16(wg, woff[0], lds_addr(wb));
    if (TERN || I4) dma_lds16(wg, woff[1], lds_addr(wb + 1024));
    if (I4) {
      dma_lds16(wg, woff[2], lds_addr(wb + 2048));
      dma_lds16(wg, woff[3], lds_addr(wb + 3072));
    }
    // scales: lane l -> 4-byte slot l (2-byte load, zero-extended)
    dma_lds2((const uint8_t*)a.S + 2 * g, soff, lds_addr(base + X_BYTES + W_BYTES + wave * 256));
    if (I4) {
      // zero points likewise, then this wave's RW rows of the group's row
      // sums (row-sum array padded past M, so every row read exists)
      dma_lds2((const uint8_t*)a.Z + 2 * g, soff, lds_addr(base + X_BYTES + W_BYTES + BN * 4 + wave * 256));
      const float* rg = a.ws + g * a.ldr + m0 + RW * wave;
      if (lane < RW / 4)
        dma_lds16(rg, 16 * lane, lds_addr(base + X_BYTES + W_BYTES + 2 * BN * 4 + 4 * RW * wave));
    }
  };

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
  if (NST == 3) stage(min(gb + 1, ge - 1), 1);
  int buf = 0;
  for (int g = gb; g < ge; ++g) {
    // stage g complete (three stages: only this wave's stage g+1 loads may
    // be in flight), and every wave's part of it visible
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(NST == 3 ? stage_loads<FMT, WN, BMT>() : 0));
    __syncthreads();
    // past the end this copies the last group into a buffer nobody reads
    if (NST == 3) stage(min(g + 2, ge - 1), buf == 0 ? 2 : buf - 1);
    else stage(min(g + 1, ge - 1), buf ^ 1);
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
          *(u32x4*)dst = v;
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

// ===========================================================================
// Small-M kernel (M <= 16): weight streaming with v_mfma_f32_16x16x32.
// The grid is (column tiles) x (K splits). A workgroup owns a tile of 16 WC
// output columns and one slice of at most GS 128-groups of K; its WC x KH
// waves are WC column waves (16 columns each) times KH parts of the slice
// along K, whose FP32 results meet in LDS and are added in part order:
//  * The activations of the slice go global -> LDS once per workgroup with
//    direct LDS DMA loads, each instruction reading four whole 256-byte group
//    rows; 16-byte chunks are XOR-swizzled by row, which makes the MFMA
//    fragment reads conflict-free. Only the ceil(M / 4) row quads that hold
//    rows < M are copied (rounded to 1, 2 or 4; rows past M inside a quad
//    repeat row M - 1), and the fragment reads of the rows past them use row
//    r & (4 quads - 1): MFMA rows are independent and outputs of rows >= M
//    are never stored.
//  * Codes: every lane issues 16-byte loads that cover two groups of its
//    column (ternary: the four lane groups read 64 contiguous bytes of the
//    column) or one group (binary: 16 bytes = 128 codes), so a wave-wide
//    instruction reads 64 contiguous bytes per column. v_permlane32_swap
//    (and v_permlane16_swap for binary) then hands every lane its own share
//    of each group.
//  * Load order: all activation DMAs first (from inline assembly, so the
//    compiler neither counts them nor makes LDS reads wait for them), then
//    the codes and scales block by block (a block is four groups of a K
//    part). One explicit wait and a barrier cover the activations; each
//    block's MFMAs then wait only for that block's codes, so the later
//    blocks' code loads are still in flight while the earlier blocks are
//    computed.
//  * MFMA rows are output rows, MFMA columns are output columns; each group
//    is four chained MFMAs, then acc += (scale * factor) * tmp in FP32. Four
//    groups are interleaved (four independent chains); slots past the slice
//    up to the next multiple of four hold zeros and a zero scale.
//  * K order inside a group (both operands): binary lane group q takes
//    k-local [32q, 32q+32) in steps of 8; ternary lane group q takes
//    b + {0..15} and b + {32..47} with b = {0, 64, 16, 80}[q], which is what
//    the lane exchange leaves in its registers.
//  * With one split the result is stored directly. Otherwise every workgroup
//    writes its FP32 partial tile as 64-bit atomic words whose zero bits mean
//    "not written" and takes a ticket for its column tile (agent-scope atomic
//    add); the workgroup that takes the last ticket reads the other splits'
//    words (polling any not yet written), sums the splits in split order
//    (deterministic), stores zeros back, applies bias and activation, stores
//    Y and resets the ticket to zero (details at the combine below).
// ===========================================================================
namespace stream {
constexpr int MAXGS = 32;                      // groups per workgroup slice
constexpr int MAXSPLIT = 16;                   // K splits
__host__ __device__ constexpr size_t lds_bytes(int gs) { return (size_t)gs * 16 * 256; }
// workspace: one 32-bit ticket per column tile in a fixed region at the
// start (so calls of any shape reuse the same, zero, counters; its last word
// counts bounded waits that gave up, which never happens in a correct run),
// then the FP32 partials [splits][tiles][waves][lanes][4]
constexpr int MAXTILES = 16384;
constexpr int ERR_SLOT = MAXTILES - 1;
constexpr size_t TICKET_BYTES = (size_t)MAXTILES * 4;
// polls of a partial word before a wait gives up (about a quarter second)
constexpr uint32_t POLL_LIMIT = 1u << 22;
// a 64-bit partial word holds two written values (zero bits mean unwritten)
__device__ __forceinline__ bool written(uint64_t w) { return (uint32_t)w != 0u && (uint32_t)(w >> 32) != 0u; }
// K parts per workgroup: the largest KH <= 4 with WC * KH <= 16 waves and
// whole blocks of four groups per part (GS % 4 KH == 0)
__host__ __device__ constexpr int kparts(int wc, int gs) {
  return (wc * 4 <= 16 && gs % 16 == 0) ? 4 : (wc * 3 <= 16 && gs % 12 == 0) ? 3
       : (wc * 2 <= 16 && gs % 8 == 0) ? 2 : 1;
}
}  // namespace stream

template <bool TERN>
__device__ __forceinline__ int stream_chunk(int q, int s) {
  // 8-k chunk of the group row used by lane group q at MFMA step s
  return TERN ? ((q & 1) * 8 + (q >> 1) * 2 + (s & 1) + (s >> 1) * 4) : (4 * q + s);
}

// GRP: a grouped launch (problem blockIdx.z of two or more); compiled
// separately so that single-problem launches carry no selection code.
template <bool BF16, int FMT, int WC, int GS, bool GRP>
__global__ __launch_bounds__(64 * WC * stream::kparts(WC, GS)) void gemm_stream_kernel(GemmArgs a, int splits, int gps, GemmGroup grp) {
  if constexpr (GRP) select_problem(a, grp, blockIdx.z);
  constexpr bool TERN = FMT == FMT_TERNARY;
  constexpr int KH = stream::kparts(WC, GS), GH = GS / KH;   // K parts, slots per part
  constexpr int NW = TERN ? GH / 2 : (GH + 3) / 4;    // 16-byte code loads per lane
  constexpr int NT = WC * KH;                          // waves
  extern __shared__ __align__(16) uint8_t smem[];      // [GS][16 rows][256 B] activations
  __shared__ f32x4 red[KH][WC][64];                    // partials of the K parts
  __shared__ int last_flag;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cwv = wave % WC, kh = wave / WC;           // column wave, K part
  const int gk0 = kh * GH;                             // first slot of this K part
  const int q = lane >> 4, c16 = lane & 15;
  const int G = a.K >> 7;
  const int tile = blockIdx.x, split = blockIdx.y;
  const int g0 = split * gps;
  const int ng = min(gps, G - g0);                      // 1 .. GS (host plan)
  const int n = (tile * WC + cwv) * 16 + c16;
  const int64_t nc = min(n, a.N - 1);                   // clamped: loads stay in bounds
  const int64_t wrow = TERN ? (a.K >> 2) : (a.K >> 3);
  const float factor = code_factor<TERN>();

  // the bias of this lane's column, loaded first so that its latency hides
  // behind the whole kernel (the oldest load: every wait below covers it)
  const float bias_v = (a.bias && n < a.N) ? load_bias(a.bias, a.bias_dtype, n) : 0.0f;

  // (1) activations of the slice -> LDS: instruction t of this wave covers
  // rows 4j .. 4j+3 of group i (slot i of the tile). Issued from inline
  // assembly (scalar base + lane offset), so the compiler neither counts them
  // in its own waits nor makes LDS reads wait for them: one explicit wait
  // below covers them all.
  constexpr int NB = GH / 4;                           // blocks of four groups per K part
  constexpr int CB = TERN ? 2 : 1;                     // code loads per block
  // only the row quads that hold rows < M are copied (rq of 1, 2 or 4);
  // fragment reads of rows past them read row r & (4 rq - 1) instead:
  // MFMA rows are independent and outputs of rows >= M are never stored
  const int lrq = a.M <= 4 ? 0 : a.M <= 8 ? 1 : 2, rq = 1 << lrq;
  const int rr = c16 & (4 * rq - 1);                   // LDS row of this lane's fragment reads
#pragma unroll
  for (int t = 0; t < (4 * GS + NT - 1) / NT; ++t) {     // (group slot, row quad) pairs over the waves
    const int idx = t * NT + wave;
    const int i = idx >> lrq, j = idx & (rq - 1);
    if (i < ng) {                                       // wave-uniform
      const int r = 4 * j + q;                          // tile row of this lane
      const uint32_t voff = (uint32_t)(((int64_t)min(r, a.M - 1) * a.ldx + 8 * ((c16 ^ r) & 15)) * 2);
      dma_lds16((const uint8_t*)a.X + ((int64_t)(g0 + i) << 8), voff, lds_addr(smem + i * 4096 + j * 1024));
    }
  }
  // slots past the slice up to the next multiple of 4 are computed with zero
  // activations (and a zero scale), so they add exactly zero
  {
    const int zend = min(GS, (ng + 3) & ~3);
    for (int z = ng * 256 + tid; z < zend * 256; z += 64 * NT)
      *(u32x4*)(smem + (size_t)z * 16) = u32x4{0u, 0u, 0u, 0u};
  }
  // (2) codes and raw scales of this wave's K part, block by block (a block
  // is four groups), so each block's MFMAs wait only for its own codes and
  // the later blocks' loads stay in flight meanwhile. Ternary load p covers
  // slots gk0 + 2p (lane groups 0, 1) and gk0 + 2p + 1 (lane groups 2, 3);
  // binary load p: lane group q reads slot gk0 + 4p + q; scale word b: lane
  // group q holds slot gk0 + 4b + q of its column
  const uint8_t* wp = a.W + nc * wrow;
  u32x4 cw[NW];
  uint32_t sr[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
#pragma unroll
    for (int c = 0; c < CB; ++c) {
      const int p = CB * b + c;
      if (TERN) {
        const int g = g0 + min(gk0 + 2 * p + (q >> 1), ng - 1);
        cw[p] = *(const u32x4*)(wp + g * 32 + 16 * (q & 1));
      } else {
        const int g = g0 + min(gk0 + 4 * p + q, ng - 1);
        cw[p] = *(const u32x4*)(wp + g * 16);
      }
    }
    sr[b] = a.S[nc * G + g0 + min(gk0 + 4 * b + q, ng - 1)];
  }
  // every activation DMA of this wave done (only the NB (CB + 1) register
  // loads above, issued after them, may be in flight), then everyone's
  __builtin_amdgcn_s_waitcnt(large::waitcnt_vm(NB * (CB + 1)));
  __syncthreads();

  // (3) per block: lane exchange (afterwards ternary group 2p is in
  // (cw[p][0], cw[p][2]) and group 2p+1 in (cw[p][1], cw[p][3]); binary
  // group 4p+j is cw[p][j]), then the MFMAs, four groups at a time: four
  // independent chains, no branch inside a block (groups past the slice
  // read zero activations)
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int bk = 0; bk < NB; ++bk) {
    if (gk0 + 4 * bk < ng) {                            // wave-uniform
#pragma unroll
      for (int c = 0; c < CB; ++c) {
        const int p = CB * bk + c;
        if (TERN) {
          auto x = __builtin_amdgcn_permlane32_swap(cw[p][0], cw[p][1], false, false);
          auto y = __builtin_amdgcn_permlane32_swap(cw[p][2], cw[p][3], false, false);
          cw[p] = u32x4{x[0], x[1], y[0], y[1]};
        } else {
          auto x = __builtin_amdgcn_permlane32_swap(cw[p][0], cw[p][2], false, false);
          auto y = __builtin_amdgcn_permlane32_swap(cw[p][1], cw[p][3], false, false);
          auto u = __builtin_amdgcn_permlane16_swap(x[0], y[0], false, false);
          auto v = __builtin_amdgcn_permlane16_swap(x[1], y[1], false, false);
          cw[p] = u32x4{u[0], u[1], v[0], v[1]};
        }
      }
      float sc[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int sbits = __shfl((int)sr[bk], 16 * u + c16);
        sc[u] = gk0 + 4 * bk + u < ng ? factor * half_bits_to_float((uint16_t)sbits) : 0.0f;
      }
      f32x4 tmp[4];
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = 4 * bk + u;                     // slot within the K part
          const u32x4 af = *(const u32x4*)(smem + (gk0 + i) * 4096 + rr * 256 + ((stream_chunk<TERN>(q, s) ^ rr) << 4));
          u32x4 bf;
          if (TERN) bf = tern_chunk(cw[i >> 1][(i & 1) + 2 * (s >> 1)], s & 1, TERN_MASK);
          else bf = bin_chunk(cw[i >> 2][i & 3], s, BIN_SIGN, BIN_TWO);
          tmp[u] = mfma16<BF16>(af, bf, s == 0 ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : tmp[u]);
        }
#pragma unroll
      for (int u = 0; u < 4; ++u) acc += sc[u] * tmp[u];
    }
  }

  // (6) the K parts meet in LDS and are added in part order (K part 0's
  // waves go on with the sum)
  if (KH > 1) {
    red[kh][cwv][lane] = acc;
    __syncthreads();
    if (kh == 0) {
#pragma unroll
      for (int k2 = 1; k2 < KH; ++k2) acc += red[k2][cwv][lane];
    }
  }
  const bool lead = kh == 0;

  // (7) output: lane holds rows 4q + e (e = 0..3) of column n
  const bool col_ok = n < a.N && lead;
  if (splits == 1) {
    if (col_ok) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * q + e < a.M) store_out(a.Y, a.ldy, a.y_dtype, 4 * q + e, n, finish(acc[e], bias_v, a.act));
    }
    return;
  }
  // Partial tiles, lane-major: [split][tile][wave][lane] x 4 FP32 values (the
  // tiles of the problems of a grouped launch side by side), written and read
  // as two 64-bit agent-scope atomic words per lane. Every slot holds bits 0
  // except while it carries a partial that its reducer has not yet consumed:
  // a writer stores +0.0 as -0.0 (bits 0x80000000; a sum is unchanged by
  // it), so a word whose halves are both nonzero is always the value its own
  // split wrote in this launch. Each workgroup stores its partial, waits for
  // the stores, then takes a ticket for its column tile; the one that takes
  // the last ticket reads the other splits' words, polls any that do not yet
  // read as written (a bounded wait), adds the splits in split order (its
  // own from registers) and stores zeros over every split's words
  // (consumed). Every value crosses between workgroups inside one 64-bit
  // atomic object, so the result does not depend on ordering between
  // different locations and needs no cache-wide fence: a reader cannot see
  // an older value of a word than the zero its last consumer stored, since
  // that store happened before this launch began. (The wait before the
  // ticket only makes the first read succeed in practice.)
  const int wtile = GRP ? blockIdx.z * gridDim.x + tile : tile;
  int* ticket = (int*)a.ws + wtile;
  uint64_t* part = (uint64_t*)((uint8_t*)a.ws + stream::TICKET_BYTES);
  const int64_t tile_lanes = (int64_t)gridDim.x * (GRP ? gridDim.z : 1) * WC * 64;
  const int64_t my = (int64_t)(wtile * WC + cwv) * 64 + lane;
  if (lead) {
    uint64_t* dst = part + 2 * ((int64_t)split * tile_lanes + my);
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // (through a scalar: __builtin_bit_cast of a vector element
      // subscript reads element 0 with this compiler)
      const float v = acc[e];
      w[e] = __builtin_bit_cast(uint32_t, v);
      w[e] = w[e] ? w[e] : 0x80000000u;
    }
    __hip_atomic_store(dst, (uint64_t)w[0] | ((uint64_t)w[1] << 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(dst + 1, (uint64_t)w[2] | ((uint64_t)w[3] << 32), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0);                        // this wave's stores have completed
  __syncthreads();
  if (tid == 0)
    last_flag = __hip_atomic_fetch_add(ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == splits - 1;
  __syncthreads();
  if (!last_flag || !lead) return;
  // the reducer: every other split's loads in flight at once, then the
  // bounded poll of any word not yet read as written
  uint64_t pv[stream::MAXSPLIT][2];
#pragma unroll
  for (int t = 0; t < stream::MAXSPLIT; ++t) {
    if (t < splits && t != split) {
      const uint64_t* src = part + 2 * ((int64_t)t * tile_lanes + my);
      pv[t][0] = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      pv[t][1] = __hip_atomic_load(src + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  bool stuck = false;
#pragma unroll
  for (int t = 0; t < stream::MAXSPLIT; ++t) {
    if (t < splits && t != split) {
      const uint64_t* src = part + 2 * ((int64_t)t * tile_lanes + my);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        for (uint32_t n = 0; !stream::written(pv[t][h]); ++n) {
          if (n == stream::POLL_LIMIT) {
            stuck = true;
            break;
          }
          __builtin_amdgcn_s_sleep(2);
          pv[t][h] = __hip_atomic_load(src + h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  }
  f32x4 sum = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int t = 0; t < stream::MAXSPLIT; ++t) {
    if (t < splits) {
      if (t == split) {
        sum += acc;
      } else {
        sum += f32x4{__builtin_bit_cast(float, (uint32_t)pv[t][0]), __builtin_bit_cast(float, (uint32_t)(pv[t][0] >> 32)),
                     __builtin_bit_cast(float, (uint32_t)pv[t][1]), __builtin_bit_cast(float, (uint32_t)(pv[t][1] >> 32))};
      }
    }
  }
  // consumed: plain 16-byte stores suffice, since nothing in this launch
  // reads these words again and the next launch that uses the workspace
  // starts after this one has ended
#pragma unroll
  for (int t = 0; t < stream::MAXSPLIT; ++t) {
    if (t < splits) *(u32x4*)(part + 2 * ((int64_t)t * tile_lanes + my)) = u32x4{0u, 0u, 0u, 0u};
  }
  if (stuck) __hip_atomic_fetch_add((int*)a.ws + stream::ERR_SLOT, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (col_ok) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (4 * q + e < a.M) store_out(a.Y, a.ldy, a.y_dtype, 4 * q + e, n, finish(sum[e], bias_v, a.act));
  }
  if (tid == 0) __hip_atomic_store(ticket, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ===========================================================================
// Small-M kernel, K split inside the workgroup (M <= 16): weight streaming
// with v_mfma_f32_16x16x32 and no cross-workgroup traffic. A workgroup owns
// 16 output columns and all of K; its waves split K, wave w taking the
// GW * NCH groups from w GW NCH on (the last wave fewer), in NCH chunks of
// GW groups. Per wave and chunk:
//  * the activations of the chunk's groups go to the wave's own LDS region
//    by direct LDS DMA (whole 256-byte group rows, chunks XOR-swizzled by
//    row as in the kernel above; only the row quads that hold rows < M, as
//    in the kernel above), so only the wave's own wait is needed before it
//    reads them; the codes come as 16-byte loads covering two groups
//    (ternary) or one group (binary) per lane, exchanged with
//    v_permlane32_swap / v_permlane16_swap exactly as in the kernel above;
//    then the raw scales. Groups past the wave's share load the share's last
//    group again and get a zero scale, so every chunk issues the same loads;
//  * the groups run as chained MFMAs (four per group), then
//    acc += (scale * factor) * tmp.
// With one chunk every load is issued up front. With more, chunks c and c+1
// are in flight in two LDS buffers and two register sets: the wave waits
// for chunk c only (the loads of chunk c+1 may still be outstanding),
// computes it, and then issues chunk c+2 into the buffers chunk c used.
// The FP32 partial tiles of the waves meet in LDS and are added in wave
// order (deterministic); bias, activation, one RNE cast and the stores
// follow. With no split across workgroups there is no workspace and no
// global atomic, and with a K split inside each workgroup there are enough
// waves in flight even when N / 16 is below the CU count.
// ===========================================================================
namespace thin {
constexpr int MAXWAVES = 16;                   // one chunk: 1024 threads, at most 128 VGPRs
constexpr int MAXWAVES_CHUNKED = 8;            // several chunks: 512 threads
}

template <bool BF16, int FMT, int GW, int NCH, bool GRP>
__global__ __launch_bounds__(64 * (NCH == 1 ? thin::MAXWAVES : thin::MAXWAVES_CHUNKED)) void gemm_thin_kernel(GemmArgs a, int nch_rt, GemmGroup grp) {
  if constexpr (GRP) select_problem(a, grp, blockIdx.z);
  static_assert(GW == 2 || GW == 4, "two or four groups per chunk");
  constexpr bool TERN = FMT == FMT_TERNARY;
  constexpr int NW = TERN ? GW / 2 : 1;                     // 16-byte code loads per lane and chunk
  constexpr int NBUF = NCH == 1 ? 1 : 2;                    // chunk buffers in flight
  // activation DMA instructions per chunk. Waiting until at most this many
  // loads are outstanding guarantees chunk c's DMAs have landed once chunk
  // c+1's DMAs (issued after them, in order) are the only ones that may
  // still be in flight, wherever the compiler places the register loads.
  constexpr int XDMA = 4 * GW;
  extern __shared__ __align__(16) uint8_t smem[];          // [waves][NBUF][GW][16 rows][256 B] activations
  __shared__ f32x4 red[NCH == 1 ? thin::MAXWAVES : thin::MAXWAVES_CHUNKED][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nwav = blockDim.x >> 6;
  const int q = lane >> 4, c16 = lane & 15;
  const int G = a.K >> 7;
  const int nch = NCH > 0 ? NCH : nch_rt;                   // chunks per wave (NCH = 0: a runtime count)
  const int g0 = wave * GW * nch;
  const int ng = min(GW * nch, G - g0);                     // 1 .. GW nch (host plan)
  const int64_t wrow = TERN ? (a.K >> 2) : (a.K >> 3);
  const float factor = code_factor<TERN>();
  const int n = blockIdx.x * 16 + c16;
  const int64_t nc = min(n, a.N - 1);                       // columns past N: any valid column
  const uint8_t* wp = a.W + nc * wrow;
  uint8_t* xw = smem + (size_t)wave * NBUF * GW * 4096;
  // the bias of this lane's column, loaded first (the oldest load, so every
  // chunk wait below also covers it) and used only by wave 0 at the end
  const float bias_v = (wave == 0 && a.bias && n < a.N) ? load_bias(a.bias, a.bias_dtype, n) : 0.0f;
  // only the row quads that hold rows < M are copied (rq of 1, 2 or 4);
  // fragment reads of rows past them read row r & (4 rq - 1) instead:
  // MFMA rows are independent and outputs of rows >= M are never stored
  const int rq = a.M <= 4 ? 1 : a.M <= 8 ? 2 : 4;
  const int rr = c16 & (4 * rq - 1);                        // LDS row of this lane's fragment reads

  u32x4 cw[NBUF][NW];
  uint32_t sr[NBUF];
  // issue the loads of chunk c into buffer / register set bsel (always a
  // constant at the call site, so the register arrays stay in registers)
  auto issue = [&](int c, int bsel) __attribute__((always_inline)) {
    uint8_t* xs = xw + bsel * GW * 4096;
#pragma unroll
    for (int i = 0; i < GW; ++i) {
      const int gi = g0 + min(c * GW + i, ng - 1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (j >= rq) continue;                              // wave-uniform: rows >= 4 rq not needed
        const int r = 4 * j + q;                            // row of this lane
        const uint16_t* src = a.X + (int64_t)min(r, a.M - 1) * a.ldx + (gi << 7) + 8 * ((c16 ^ r) & 15);
        __builtin_amdgcn_global_load_lds((const void*)src, (lds_ptr_t)(xs + i * 4096 + j * 1024), 16, 0, 0);
      }
    }
#pragma unroll
    for (int p = 0; p < NW; ++p) {
      if (TERN) {
        const int g = g0 + min(c * GW + 2 * p + (q >> 1), ng - 1);
        cw[bsel][p] = *(const u32x4*)(wp + g * 32 + 16 * (q & 1));
      } else {
        const int g = g0 + min(c * GW + q, ng - 1);
        cw[bsel][p] = *(const u32x4*)(wp + g * 16);
      }
    }
    sr[bsel] = a.S[nc * G + g0 + min(c * GW + q, ng - 1)];  // lane group q: group c GW + q
    asm volatile("" ::: "memory");                          // keep the chunks' loads in order
  };

  // wait until the chunk about to be computed has landed: with a later
  // chunk's loads issued after it (more), only those may stay in flight
  auto wait_chunk = [&](bool more) __attribute__((always_inline)) {
    if (more) {
      if (rq == 1) __builtin_amdgcn_s_waitcnt(large::waitcnt_vm(XDMA / 4));
      else if (rq == 2) __builtin_amdgcn_s_waitcnt(large::waitcnt_vm(XDMA / 2));
      else __builtin_amdgcn_s_waitcnt(large::waitcnt_vm(XDMA));
    } else {
      __builtin_amdgcn_s_waitcnt(0);
    }
  };
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  auto compute = [&](int c, int bsel) __attribute__((always_inline)) {
    if (c * GW < ng) {                                      // wave-uniform
      // lane exchange (as in the kernel above)
      u32x4 w[NW];
#pragma unroll
      for (int p = 0; p < NW; ++p) {
        if (TERN) {
          auto x = __builtin_amdgcn_permlane32_swap(cw[bsel][p][0], cw[bsel][p][1], false, false);
          auto y = __builtin_amdgcn_permlane32_swap(cw[bsel][p][2], cw[bsel][p][3], false, false);
          w[p] = u32x4{x[0], x[1], y[0], y[1]};
        } else {
          auto x = __builtin_amdgcn_permlane32_swap(cw[bsel][p][0], cw[bsel][p][2], false, false);
          auto y = __builtin_amdgcn_permlane32_swap(cw[bsel][p][1], cw[bsel][p][3], false, false);
          auto u = __builtin_amdgcn_permlane16_swap(x[0], y[0], false, false);
          auto v = __builtin_amdgcn_permlane16_swap(x[1], y[1], false, false);
          w[p] = u32x4{u[0], u[1], v[0], v[1]};
        }
      }
      const uint8_t* xs = xw + bsel * GW * 4096;
      float sc[GW];
#pragma unroll
      for (int u = 0; u < GW; ++u) {
        const int sbits = __shfl((int)sr[bsel], 16 * u + c16);
        sc[u] = c * GW + u < ng ? factor * half_bits_to_float((uint16_t)sbits) : 0.0f;
      }
      f32x4 tmp[GW];
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int u = 0; u < GW; ++u) {
          u32x4 bf;
          if (TERN) bf = tern_chunk(w[u >> 1][(u & 1) + 2 * (s >> 1)], s & 1, TERN_MASK);
          else bf = bin_chunk(w[0][u], s, BIN_SIGN, BIN_TWO);
          const u32x4 af = *(const u32x4*)(xs + u * 4096 + rr * 256 + ((stream_chunk<TERN>(q, s) ^ rr) << 4));
          tmp[u] = mfma16<BF16>(af, bf, s == 0 ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : tmp[u]);
        }
#pragma unroll
      for (int u = 0; u < GW; ++u) acc += sc[u] * tmp[u];
    }
  };

  // chunk c+2 goes into the buffers of chunk c once chunk c is computed
  // (this wave's reads of them are done: their data fed the MFMAs)
  issue(0, 0);
  if (NCH != 1) issue(1, 1);
  if (NCH > 0) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      wait_chunk(c + 1 < NCH);
      compute(c, c % NBUF);
      if (c + 2 < NCH) issue(c + 2, c % NBUF);
    }
  } else {
    // any number of chunks: a loop over pairs, buffer 0 then buffer 1
    for (int c = 0; c < nch; c += 2) {
      wait_chunk(c + 1 < nch);
      compute(c, 0);
      if (c + 2 < nch) issue(c + 2, 0);
      if (c + 1 < nch) {
        wait_chunk(c + 2 < nch);
        compute(c + 1, 1);
        if (c + 3 < nch) issue(c + 3, 1);
      }
    }
  }
  red[wave][lane] = acc;
  __syncthreads();

  // sum of the waves' partials in wave order, epilogue; lane holds rows
  // 4q + e (e = 0..3) of column n
  if (wave == 0) {
    f32x4 sum;
    if constexpr (NCH != 1) {
      // several chunks (at most 8 waves): every partial read issued before
      // the first add (one LDS round trip instead of one per wave), then
      // added in wave order
      f32x4 pw[thin::MAXWAVES_CHUNKED];
#pragma unroll
      for (int w2 = 0; w2 < thin::MAXWAVES_CHUNKED; ++w2)
        pw[w2] = w2 < nwav ? red[w2][lane] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      sum = pw[0];
#pragma unroll
      for (int w2 = 1; w2 < thin::MAXWAVES_CHUNKED; ++w2)
        if (w2 < nwav) sum += pw[w2];
    } else {
      // one chunk (up to 16 waves): in wave order, one read at a time
      sum = red[0][lane];
      for (int w2 = 1; w2 < nwav; ++w2) sum += red[w2][lane];
    }
    if (n < a.N) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * q + e < a.M) store_out(a.Y, a.ldy, a.y_dtype, 4 * q + e, n, finish(sum[e], bias_v, a.act));
    }
  }
}

// Standalone exact-erf GELU.
__global__ void gelu_kernel(const void* in, void* out, int dtype, int64_t count) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * blockDim.x) {
    float x;
    if (dtype == DT_BF16) x = bf16_bits_to_float(((const uint16_t*)in)[i]);
    else if (dtype == DT_F16) x = half_bits_to_float(((const uint16_t*)in)[i]);
    else x = ((const float*)in)[i];
    float y = gelu_erf(x);
    if (dtype == DT_BF16) ((uint16_t*)out)[i] = float_to_bf16_bits(y);
    else if (dtype == DT_F16) ((uint16_t*)out)[i] = float_to_half_bits(y);
    else ((float*)out)[i] = y;
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

// ===========================================================================
// Host-side launch helpers
// ===========================================================================

// Plan of the small-M kernel with the K split inside the workgroup: used
// only while N / 16 is below the CU count (every workgroup reads all of X
// from L2; for wider N the kernel above, with X shared through LDS by 48 to
// 128 columns, is faster). One chunk per wave (all of the wave's
// activations in LDS at once) while K allows: GW = 2 with up to 16 waves,
// else GW = 4 within the LDS (K <= 4608). Longer K: 8 waves, chunks of
// GW = 2 groups, NCH >= 3 chunks per wave (compiled for 3 .. 8, a runtime
// count beyond), two chunks in flight. With any_n the plan is also made for
// wide N: the fallback when the column-tile plan cannot cover the shape
// (more than MAXGS * MAXSPLIT groups of K, or too many column tiles).
// A grouped launch of `count` problems counts the blocks of all of them; when
// those fill one to two workgroups per CU and K has 16 groups or more, four
// waves of two-group chunks (64 KiB of LDS) let two workgroups share a CU.
struct ThinPlan { int gw, nch, waves, blocks; };

static bool thin_plan(int M, int N, int K, int num_cu, ThinPlan* out, bool any_n = false, int count = 1) {
  if (M > 16) return false;
  const int G = K / 128;
  const int blocks = (N + 15) / 16;
  // grouped launches whose column blocks fill one to two workgroups per CU
  // (the image and text streams' 3072-column linears: 384 blocks): four
  // waves of two-group chunks, 64 KiB of LDS, so two workgroups share a CU
  // and every block runs in one round, with no K split across workgroups
  const int64_t wgs = (int64_t)count * blocks;
  if (!any_n && count > 1 && wgs >= num_cu && wgs <= 2 * (int64_t)num_cu && G >= 16) {
    const int nch = (G + 7) / 8;                            // two-group chunks per wave, four waves
    *out = ThinPlan{2, nch, (G + 2 * nch - 1) / (2 * nch), blocks};
    return true;
  }
  if (!any_n && wgs >= num_cu) return false;
  constexpr size_t LDS = 160 * 1024, RED = 16 * 1024;      // LDS per workgroup, partials
  if ((G + 1) / 2 <= thin::MAXWAVES) {
    *out = ThinPlan{2, 1, (G + 1) / 2, blocks};
    return true;
  }
  if ((G + 3) / 4 <= thin::MAXWAVES && (size_t)((G + 3) / 4) * 4 * 4096 + RED <= LDS) {
    *out = ThinPlan{4, 1, (G + 3) / 4, blocks};
    return true;
  }
  const int nch = (G + 2 * thin::MAXWAVES_CHUNKED - 1) / (2 * thin::MAXWAVES_CHUNKED);
  *out = ThinPlan{2, nch, (G + 2 * nch - 1) / (2 * nch), blocks};
  return true;
}

// Small-M plan: the tile width (16 WC columns, WC in 3, 4, 5, 6, 8) and the
// K split S (1 .. MAXSPLIT, at most MAXGS groups per slice) that minimise a
// rough time estimate:
//   rounds * (slice bytes through one CU at ~64 B/clk + slice MFMA work
//   shared by the slice's K parts)
//   + a fixed cost for the cross-workgroup combine when S > 1
// (the combine waits for written partials, a ticket and the read-back, each
// a memory round trip). The compiled slice size GS is gps rounded up to a
// multiple of 4 (8 from 16 on).
struct StreamPlan { int wc, gs, gps, splits, tiles; };

static int round_gs(int g) { return g <= 4 ? 4 : g <= 8 ? 8 : g <= 12 ? 12 : g <= 16 ? 16 : g <= 24 ? 24 : 32; }

// `tiles` is per problem; a grouped launch of `count` problems runs
// count * tiles column tiles side by side.
static bool stream_plan(int M, int N, int K, int num_cu, StreamPlan* out, int count = 1) {
  if (M > 16) return false;
  const int G = K / 128;
  if (G > stream::MAXGS * stream::MAXSPLIT) return false;
  double best = 1e30;
  StreamPlan bp{};
  for (int wc : {3, 4, 5, 6, 8}) {
  const int tiles = (N + 16 * wc - 1) / (16 * wc);
  if ((int64_t)tiles * count > stream::ERR_SLOT) continue;            // tickets below the error word
  for (int sp = 1; sp <= min(stream::MAXSPLIT, G); ++sp) {
    const int gps = (G + sp - 1) / sp;
    if (gps > stream::MAXGS) continue;
    const int S = (G + gps - 1) / gps;
    const int gs = round_gs(gps);
    const int kh = stream::kparts(wc, gs);
    const size_t lds = stream::lds_bytes(gs) + (size_t)kh * wc * 1024;
    const int per_cu = max(1, min((int)(160 * 1024 / lds), 32 / (wc * kh)));
    const int rounds = (tiles * count * S + num_cu * per_cu - 1) / (num_cu * per_cu);
    const double clk = gps * (4096.0 + wc * 16 * 32) / 64.0 + gps * 4 * 40.0 / kh;
    const double us = rounds * clk / 2100.0 + (S > 1 ? 3.0 : 0.0);
    if (us < best) {
      best = us;
      bp = StreamPlan{wc, gs, gps, S, tiles};
    }
  }
  }
  *out = bp;
  return best < 1e29;
}

// The small-M kernel covers every M <= 16 with N <= 16384 * 128 (unless the
// large-M kernel is forced).
bool small_path(int M, int N, int K, int variant, int count) {
  if (variant == 1 || variant == 5 || variant == 6) return false;
  StreamPlan p;
  ThinPlan tp;
  return (variant != 7 && thin_plan(M, N, K, 256, &tp, false, count)) ||
         stream_plan(M, N, K, 256, &p, count) || thin_plan(M, N, K, 256, &tp, true, count);
}

// Workspace of the small-M kernel when K is split: partials and tickets.
size_t small_workspace_bytes(int M, int N, int K, int num_cu, int variant, int count) {
  ThinPlan tp;
  if (variant != 7 && thin_plan(M, N, K, num_cu, &tp, false, count)) return 0;
  StreamPlan p;
  if (!stream_plan(M, N, K, num_cu, &p, count) || p.splits == 1) return 0;
  return stream::TICKET_BYTES + (size_t)p.splits * count * p.tiles * p.wc * 64 * 4 * sizeof(float);
}

template <bool BF16, int FMT>
static void launch_thin_t(const GemmArgs& a, const GemmGroup& g, int count, const ThinPlan& p, hipStream_t st) {
  const dim3 grid(p.blocks, 1, count), block(64 * p.waves);
  const size_t lds = (size_t)p.waves * (p.nch == 1 ? 1 : 2) * p.gw * 4096;
#define LOWBIT_THIN(GW, NCH)                                                                              \
  do {                                                                                                    \
    if (count > 1)                                                                                        \
      hipLaunchKernelGGL((gemm_thin_kernel<BF16, FMT, GW, NCH, true>), grid, block, lds, st, a, p.nch, g);  \
    else                                                                                                  \
      hipLaunchKernelGGL((gemm_thin_kernel<BF16, FMT, GW, NCH, false>), grid, block, lds, st, a, p.nch, g); \
  } while (0)
  if (p.nch == 1) {
    if (p.gw == 2) LOWBIT_THIN(2, 1);
    else LOWBIT_THIN(4, 1);
  } else {
    switch (p.nch) {
      case 3: LOWBIT_THIN(2, 3); break;
      case 4: LOWBIT_THIN(2, 4); break;
      case 5: LOWBIT_THIN(2, 5); break;
      case 6: LOWBIT_THIN(2, 6); break;
      case 7: LOWBIT_THIN(2, 7); break;
      case 8: LOWBIT_THIN(2, 8); break;
      default: LOWBIT_THIN(2, 0); break;              // runtime chunk count
    }
  }
#undef LOWBIT_THIN
}

template <bool BF16, int FMT>
static void launch_stream_t(const GemmArgs& a, const GemmGroup& g, int count, const StreamPlan& p,
                            hipStream_t st) {
  const dim3 grid(p.tiles, p.splits, count), block(64 * p.wc * stream::kparts(p.wc, p.gs));
  const size_t lds = stream::lds_bytes(p.gs);
#define LOWBIT_STREAM(WC, GS)                                                                      \
  do {                                                                                             \
    if (count > 1)                                                                                 \
      hipLaunchKernelGGL((gemm_stream_kernel<BF16, FMT, WC, GS, true>), grid, block, lds, st, a,    \
                         p.splits, p.gps, g);                                                      \
    else                                                                                           \
      hipLaunchKernelGGL((gemm_stream_kernel<BF16, FMT, WC, GS, false>), grid, block, lds, st, a,   \
                         p.splits, p.gps, g);                                                      \
  } while (0)
#define LOWBIT_STREAM_GS(WC)             \
  if (p.gs == 4) LOWBIT_STREAM(WC, 4);   \
  else if (p.gs == 8) LOWBIT_STREAM(WC, 8);   \
  else if (p.gs == 12) LOWBIT_STREAM(WC, 12); \
  else if (p.gs == 16) LOWBIT_STREAM(WC, 16); \
  else if (p.gs == 24) LOWBIT_STREAM(WC, 24); \
  else LOWBIT_STREAM(WC, 32);
  switch (p.wc) {
    case 3: LOWBIT_STREAM_GS(3) break;
    case 4: LOWBIT_STREAM_GS(4) break;
    case 5: LOWBIT_STREAM_GS(5) break;
    case 6: LOWBIT_STREAM_GS(6) break;
    default: LOWBIT_STREAM_GS(8) break;
  }
#undef LOWBIT_STREAM_GS
#undef LOWBIT_STREAM
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

hipError_t launch_gemm(int fmt, bool x_bf16, GemmArgs a, int num_cu, int variant, hipStream_t st,
                       const GemmGroup* group, int count) {
  // variant: 0 = automatic, 1 = force the large-M kernel, 2 = small-M
  // kernels only (M <= 16), 5 / 6 = large-M kernel with wide / pair tiles,
  // 7 = the small-M kernel with the K split across workgroups.
  // group / count: `count` problems of the same shape in one launch of a
  // small-M kernel (problem 0 is `a`, problem z > 0 takes its buffers from
  // `group`); the large-M kernel runs them one launch each.
  GemmGroup g{};
  if (group) g = *group;
  if (count < 1) count = 1;
  StreamPlan p;
  ThinPlan tp;
  const bool small_ok = variant != 1 && variant != 5 && variant != 6;
  bool thin = small_ok && variant != 7 && thin_plan(a.M, a.N, a.K, num_cu, &tp, false, count);
  const bool stream = !thin && small_ok && stream_plan(a.M, a.N, a.K, num_cu, &p, count);
  // beyond the column-tile plan's reach (very long K, very many columns) the
  // K-split-inside-the-workgroup kernel takes any N
  if (!thin && !stream && small_ok) thin = thin_plan(a.M, a.N, a.K, num_cu, &tp, true, count);
  if (thin) {
    if (fmt == FMT_TERNARY) {
      if (x_bf16) launch_thin_t<true, FMT_TERNARY>(a, g, count, tp, st);
      else launch_thin_t<false, FMT_TERNARY>(a, g, count, tp, st);
    } else {
      if (x_bf16) launch_thin_t<true, FMT_BINARY>(a, g, count, tp, st);
      else launch_thin_t<false, FMT_BINARY>(a, g, count, tp, st);
    }
  } else if (stream) {
    if (fmt == FMT_TERNARY) {
      if (x_bf16) launch_stream_t<true, FMT_TERNARY>(a, g, count, p, st);
      else launch_stream_t<false, FMT_TERNARY>(a, g, count, p, st);
    } else {
      if (x_bf16) launch_stream_t<true, FMT_BINARY>(a, g, count, p, st);
      else launch_stream_t<false, FMT_BINARY>(a, g, count, p, st);
    }
  } else {
    for (int z = 0; z < count; ++z) {
      if (z > 0) {
        a.X = g.X[z];
        a.W = g.W[z];
        a.S = g.S[z];
        a.bias = g.bias[z];
        a.Y = g.Y[z];
      }
      if (fmt == FMT_TERNARY) {
        if (x_bf16) launch_large_t<true, FMT_TERNARY>(a, num_cu, variant, st);
        else launch_large_t<false, FMT_TERNARY>(a, num_cu, variant, st);
      } else {
        if (x_bf16) launch_large_t<true, FMT_BINARY>(a, num_cu, variant, st);
        else launch_large_t<false, FMT_BINARY>(a, num_cu, variant, st);
      }
    }
  }
  return hipGetLastError();
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

hipError_t launch_gelu(const void* in, void* out, int dtype, int64_t count, hipStream_t st) {
  int64_t g = (count + 255) / 256;
  if (g > 8192) g = 8192;
  hipLaunchKernelGGL(gelu_kernel, dim3((int)(g < 1 ? 1 : g)), dim3(256), 0, st, in, out, dtype, count);
  return hipGetLastError();
}

}  // namespace lowbit
