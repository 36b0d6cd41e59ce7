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
#include "common.h"

namespace lowbit {

// ===========================================================================
// Large-M kernel (v_mfma_f32_32x32x16): a workgroup computes a 128 x 256 tile
// of Y with 4 waves side by side along N, each wave 128 x 64 (4 x 2 blocks of
// 32 x 32). One pipeline stage is one 128-group along K.
//
//  * Activations: global -> LDS with direct 16-byte LDS DMA loads
//    (global_load_lds_dwordx4), three stages in flight. LDS holds each row's
//    sixteen 16-byte chunks XOR-swizzled by (row % 16), which makes the
//    fragment reads (32 rows, same chunk) bank-conflict free. Every wave reads
//    the fragments of a whole group into registers (AGPRs, which MFMA reads
//    directly); those of group g+1 replace those of group g while the second
//    column block of group g is computed.
//  * Packed codes and scales: straight from global memory into VGPRs (each
//    wave owns distinct columns, so nothing is shared through LDS), one group
//    ahead of use. A lane loads 16 bytes (ternary) or 8 bytes (binary): the
//    64 codes its lane group contributes to the group.
//  * Group scales, Horner form: the MFMAs accumulate in units of the current
//    group's scale c_g = +-s_g / 2, and at each group boundary the accumulator
//    is rescaled by c_{g-1} / c_g (one FP32 multiply per element); after the
//    last group it is multiplied by c_G. In exact arithmetic this is
//    sum_g c_g P_g; in FP32 each rescale adds one rounding (about 2G ulps of
//    relative error over the whole sum, far inside the 1e-3 tolerance). A
//    group whose scale is zero is fed as zero codes and keeps the previous
//    reference scale, so zero and subnormal scales are exact. Requires finite
//    scales and |partial sums| < 2^100 (the quotient of two FP16 scales is at
//    most 2^40, so a partial sum can grow by that much in accumulator units).
//
// K order inside a group: lane group q = lane / 32 owns k-local [64q, 64q+64);
// MFMA step s (0..7) uses its slots 64q + 8s .. +7.
// ===========================================================================
namespace large {
constexpr int BM = 128, BN = 256, THREADS = 256, STAGES = 3;
constexpr int ROW_BYTES = 256;                 // 128 k x 2 bytes
constexpr int STAGE_BYTES = BM * ROW_BYTES;    // 32 KiB
}  // namespace large

typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <bool BF16, int FMT>
__global__ __launch_bounds__(256, 1) void gemm_large_kernel(GemmArgs a, int tiles_m, int tiles_n) {
  using namespace large;
  constexpr bool TERN = FMT == FMT_TERNARY;
  __shared__ __align__(16) uint8_t sA[STAGES][STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63, q = lane >> 5, r32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // XCD-aware tile order: consecutive workgroups land on different XCDs, so
  // give each XCD a contiguous range of tiles (N fastest) to share L2.
  int t = blockIdx.x;
  const int T = tiles_m * tiles_n;
  if ((T & 7) == 0) t = (t & 7) * (T >> 3) + (t >> 3);
  const int m0 = (t / tiles_n) * BM, n0 = (t % tiles_n) * BN;
  const int G = a.K >> 7;
  const int64_t wrow = TERN ? (a.K >> 2) : (a.K >> 3);
  const float factor = code_factor<TERN>();

  // ---- activation stage g -> LDS buffer `buf` (wave w: rows 32w .. 32w+31) ----
  auto dma = [&](int g, int buf) {
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int rb = 32 * wave + 4 * it;                    // wave-uniform first row
      const int r = rb + (lane >> 4);
      const int c = (lane & 15) ^ (r & 15);                 // chunk stored in slot lane&15
      const int m = min(m0 + r, a.M - 1);                   // rows past M: any valid row
      const uint16_t* src = a.X + (int64_t)m * a.ldx + (g << 7) + 8 * c;
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_ptr_t)(sA[buf] + rb * ROW_BYTES), 16, 0, 0);
    }
  };
  auto afrag = [&](int buf, int i, int s) -> u32x4 {
    const int r = 32 * i + r32;
    const int p = (8 * q + s) ^ (r & 15);
    return *(const u32x4*)(sA[buf] + r * ROW_BYTES + p * 16);
  };

  // ---- packed codes + scales of this lane's two columns ----
  int ncol[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) ncol[j] = min(n0 + 64 * wave + 32 * j + r32, a.N - 1);
  // raw scale bits are kept until the group starts: converting them at load
  // time would make the wave wait for the load (and everything issued before)
  auto bload = [&](int g, u32x4 (&bw)[2], uint16_t (&sb)[2]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint8_t* p = a.W + (int64_t)ncol[j] * wrow;
      if (TERN) {
        bw[j] = *(const u32x4*)(p + g * 32 + 16 * q);
      } else {
        u32x2 v = *(const u32x2*)(p + g * 16 + 8 * q);
        bw[j] = u32x4{v[0], v[1], 0u, 0u};
      }
      sb[j] = a.S[(int64_t)ncol[j] * G + g];
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  float cref[2] = {1.0f, 1.0f};                 // reference scale of the accumulator

  u32x4 A[4][8];

  // one column block of one group: rescale to the group's scale, then 32 MFMAs
  auto block = [&](int j, const u32x4 (&bw)[2], const uint16_t (&sb)[2], bool refill, int nbuf) {
    const float s = factor * half_bits_to_float(sb[j]);
    const bool zero = s == 0.0f;
    const float r = zero ? 1.0f : cref[j] / s;
    cref[j] = zero ? cref[j] : s;
    const uint32_t tm = zero ? 0u : TERN_MASK;
    const uint32_t mk = zero ? 0u : BIN_SIGN, bs = zero ? 0u : BIN_TWO;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i][j] *= r;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const u32x4 bf = TERN ? tern_chunk(bw[j][st >> 1], st & 1, tm)
                            : bin_chunk(bw[j][st >> 2], st & 3, mk, bs);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i][j] = mfma32<BF16>(A[i][st], bf, acc[i][j]);
      if (refill) {
#pragma unroll
        for (int i = 0; i < 4; ++i) A[i][st] = afrag(nbuf, i, st);
      }
    }
  };

  // One group. At its start a single wait + barrier covers everything issued
  // at the start of the previous group (codes and scales of this group, the
  // activation stage of the next one); then the codes and scales of group
  // g+1 (into the other register set: the loop is unrolled by two) and the
  // activation stage of group g+2 are issued, so every global load has a whole
  // group of compute to arrive. Column block 1 replaces the fragments of
  // group g by those of group g+1 as it goes.
  auto group = [&](int g, const u32x4 (&bw)[2], const uint16_t (&sb)[2], u32x4 (&bwn)[2],
                   uint16_t (&sbn)[2]) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const bool more = g + 1 < G;
    if (more) {
      bload(g + 1, bwn, sbn);
      // past the end this reloads the last group into the buffer of group
      // g-1, which nobody reads any more
      dma(min(g + 2, G - 1), (g + 2) % STAGES);
    }
    block(0, bw, sb, false, 0);
    if (more) block(1, bw, sb, true, (g + 1) % STAGES);
    else block(1, bw, sb, false, 0);
  };

  u32x4 bw0[2], bw1[2];
  uint16_t sb0[2], sb1[2];

  // prologue: stages 0 and 1 in flight, group-0 codes, then group-0 fragments
  dma(0, 0);
  if (G > 1) dma(1, 1);
  bload(0, bw0, sb0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int st = 0; st < 8; ++st) A[i][st] = afrag(0, i, st);

  for (int g = 0; g < G; g += 2) {
    group(g, bw0, sb0, bw1, sb1);
    if (g + 1 < G) group(g + 1, bw1, sb1, bw0, sb0);
  }

  // ---- epilogue: final scale, bias, activation, one RNE cast, store ----
  const bool y16 = a.y_dtype != DT_F32;
  const bool vec = y16 && (a.ldy & 7) == 0 && ((uintptr_t)a.Y & 15) == 0;
  if (vec) {
    // 16-bit outputs go through LDS (each wave: its 128 x 64 tile, 16 KiB,
    // 16-byte chunks XOR-swizzled by row % 8) and leave as 16-byte stores
    // covering whole 128-byte row segments.
    __syncthreads();                                  // LDS stages are free now
    uint8_t* sY = sA[0] + wave * (128 * 128);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + 64 * wave + 32 * j + r32;
      const float b = (a.bias && n < a.N) ? load_bias(a.bias, a.bias_dtype, n) : 0.0f;
      const float c = cref[j];
      const int col = 32 * j + r32;
#pragma unroll
      for (int i = 0; i < 4; ++i)
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
    for (int it = 0; it < 16; ++it) {
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
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + 32 * i + 8 * (r >> 2) + 4 * q + (r & 3);
          if (m < a.M) store_out(a.Y, a.ldy, a.y_dtype, m, n, finish(acc[i][j][r] * c, b, a.act));
        }
    }
  }
}

// ===========================================================================
// Small-M kernel (M <= 16): weight streaming with v_mfma_f32_32x32x16 (rows
// 16..31 of every MFMA are padding). A workgroup owns 4 column blocks of 32
// (one per wave) and a range of at most GMAX 128-groups.
//  1. The activations of that K range (M rows, zero rows up to 16) are staged
//     once in LDS, laid out so that an MFMA fragment read (16 lanes, 16 bytes
//     each) is one contiguous, conflict-free 256-byte block.
//  2. Each wave issues the code loads of its whole range (16 bytes per lane
//     per group, the lane-group K order of the large-M kernel) and the raw
//     scales before its first MFMA: one memory latency covers the kernel.
//  3. Per group: tmp = 8 MFMAs, part += (+-s / 2) * tmp on the accumulator
//     registers that hold real rows (8 of 16).
// With a.splits > 1 the group range is split across workgroups and FP32
// partials go to the workspace, summed afterwards in split order
// (deterministic).
// ===========================================================================
constexpr int MAX_SPLITS = 16;           // K splits of the small-M kernel

namespace small {
constexpr int GMAX = 16;                 // groups per workgroup (register budget)
constexpr int XROWS = 16;
}  // namespace small

template <bool BF16, int FMT>
__global__ __launch_bounds__(256) void gemm_small_kernel(GemmArgs a) {
  using namespace small;
  constexpr bool TERN = FMT == FMT_TERNARY;
  // [group][lane group q][step][row] of 16-byte activation chunks
  __shared__ u32x4 sX[GMAX * 2 * 8 * XROWS];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, q = lane >> 5, r32 = lane & 31;
  const int G = a.K >> 7;
  const int64_t wrow = TERN ? (a.K >> 2) : (a.K >> 3);
  const float factor = code_factor<TERN>();
  const int g0 = blockIdx.y * a.gps;
  const int ng = min(G - g0, a.gps);                    // 1 .. GMAX
  const int n = blockIdx.x * 128 + wave * 32 + r32;
  const int nc = min(n, a.N - 1);                       // clamped: loads stay in bounds

  // (1) activations of the range: every load is issued before any LDS write
  // (a loop that waited on each load would pay one memory latency per group).
  // Thread t covers row t/16, 16-byte chunk t%16 of each group (coalesced);
  // rows >= M and the padding groups up to the next multiple of four are
  // zero, so every fragment read below is unconditional.
  const int ng4 = (ng + 3) & ~3;
  u32x4 xs[GMAX];
  {
    const int row = tid >> 4, ch = tid & 15;
#pragma unroll
    for (int i = 0; i < GMAX; ++i) {
      xs[i] = u32x4{0u, 0u, 0u, 0u};
      if (i < ng && row < a.M) xs[i] = *(const u32x4*)(a.X + (int64_t)row * a.ldx + ((g0 + i) << 7) + 8 * ch);
    }
  }
  // (2) codes and scales of the whole range, in flight during the staging
  u32x4 wd[GMAX];
  uint16_t sb[GMAX];
  const uint8_t* wp = a.W + (int64_t)nc * wrow;
#pragma unroll
  for (int i = 0; i < GMAX; ++i) {
    const int g = g0 + min(i, ng - 1);
    if (TERN) {
      wd[i] = *(const u32x4*)(wp + g * 32 + 16 * q);
    } else {
      const u32x2 v = *(const u32x2*)(wp + g * 16 + 8 * q);
      wd[i] = u32x4{v[0], v[1], 0u, 0u};
    }
    sb[i] = a.S[(int64_t)nc * G + g];
  }

  {
    const int row = tid >> 4, ch = tid & 15;          // chunk ch = 8 * qq + st
#pragma unroll
    for (int i = 0; i < GMAX; ++i)
      if (i < ng4) sX[(i * 16 + ch) * XROWS + row] = xs[i];
  }
  __syncthreads();

  // (3) MFMAs: four groups at a time, so four independent accumulation
  // chains are interleaved (one chain alone would wait out the MFMA latency)
  float part[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) part[r] = 0.0f;
  // lanes 16..31 read row r32 - 16 again: MFMA rows 16..31 are never used
  const int xr = r32 & (XROWS - 1);
#pragma unroll
  for (int i0 = 0; i0 < GMAX; i0 += 4) {
    if (i0 < ng) {
      f32x16 tmp[4];
#pragma unroll
      for (int st = 0; st < 8; ++st) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = i0 + u;
          const u32x4 af = sX[((i * 2 + q) * 8 + st) * XROWS + xr];
          const u32x4 bf = TERN ? tern_chunk(wd[i][st >> 1], st & 1, TERN_MASK)
                                : bin_chunk(wd[i][st >> 2], st & 3, BIN_SIGN, BIN_TWO);
          tmp[u] = mfma32<BF16>(af, bf, st == 0 ? f32x16{} : tmp[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        // padding groups multiply zero activations; their scale is not used
        const float sc = (i0 + u < ng) ? factor * half_bits_to_float(sb[i0 + u]) : 0.0f;
#pragma unroll
        for (int r = 0; r < 8; ++r) part[r] += sc * tmp[u][r];
      }
    }
  }

  // registers r < 8 hold rows 8*(r/4) + 4q + (r%4) < 16 of column n
  if (a.splits == 1) {
    if (n < a.N) {
      const float b = a.bias ? load_bias(a.bias, a.bias_dtype, n) : 0.0f;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int m = 8 * (r >> 2) + 4 * q + (r & 3);
        if (m < a.M) store_out(a.Y, a.ldy, a.y_dtype, m, n, finish(part[r], b, a.act));
      }
    }
    return;
  }
  // split K: FP32 partials, summed by splitk_reduce_kernel in split order
  if (n < a.N) {
    const int64_t MN = (int64_t)a.M * a.N;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int m = 8 * (r >> 2) + 4 * q + (r & 3);
      if (m < a.M) a.ws[blockIdx.y * MN + (int64_t)m * a.N + n] = part[r];
    }
  }
}

// Sum of split-K partials in split order, then bias, activation and cast.
// The split loop is unrolled to a fixed bound so all partial loads of an
// element are in flight together (a rolled loop would wait once per split).
// A separate launch: completing the sum inside the GEMM would need a
// device-scope fence per workgroup, which on this multi-XCD part (one L2 per
// XCD) costs far more than the extra launch.
__global__ void splitk_reduce_kernel(GemmArgs a) {
  const int64_t total = (int64_t)a.M * a.N;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    float p[MAX_SPLITS];
#pragma unroll
    for (int s = 0; s < MAX_SPLITS; ++s) p[s] = s < a.splits ? a.ws[(int64_t)s * total + i] : 0.0f;
    float v = p[0];
#pragma unroll
    for (int s = 1; s < MAX_SPLITS; ++s)
      if (s < a.splits) v += p[s];
    const int m = (int)(i / a.N), n = (int)(i % a.N);
    const float b = a.bias ? load_bias(a.bias, a.bias_dtype, n) : 0.0f;
    store_out(a.Y, a.ldy, a.y_dtype, m, n, finish(v, b, a.act));
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

// ===========================================================================
// Host-side launch helpers
// ===========================================================================

// Small-M plan: column tiles of 128 (4 waves x 32) and a K split into ranges
// of at most small::GMAX groups; split further (down to 2 groups per range)
// while there are fewer than one workgroup per CU.
struct SmallPlan { int splits, gps; };

static SmallPlan small_plan(int M, int N, int K, int num_cu) {
  (void)M;
  const int G = K / 128;
  const int tiles = (N + 127) / 128;
  // candidates: every split count from the minimum (ranges of <= GMAX groups)
  // up to MAX_SPLITS with at least 2 groups per range; score = rounds of
  // workgroups over the CUs (2 resident per CU) weighted by the work of one
  // workgroup, plus the cost of writing and re-reading the partials
  const int smin = (G + small::GMAX - 1) / small::GMAX;
  SmallPlan best{1, G};
  double best_cost = 1e30;
  for (int sp = smin; sp <= MAX_SPLITS; ++sp) {
    const int gps = (G + sp - 1) / sp;
    if (gps > small::GMAX || (sp > smin && gps < 2)) continue;
    const int splits = (G + gps - 1) / gps;
    const int wgs = tiles * splits;
    const int rounds = (wgs + 2 * num_cu - 1) / (2 * num_cu);
    // one round costs about a memory latency plus its group count
    double cost = rounds * (8.0 + gps);
    if (splits > 1) cost += 6.0 + 0.05 * splits;   // reduce launch + partial traffic
    if (wgs < num_cu) cost += 4.0 * (num_cu - wgs) / num_cu;   // idle CUs
    if (cost < best_cost) {
      best_cost = cost;
      best.splits = splits;
      best.gps = gps;
    }
  }
  return best;
}

// The small-M kernel covers K up to GMAX * MAX_SPLITS groups; beyond that
// (K > 32768) the large-M kernel runs instead.
bool small_path(int M, int N, int K, int variant) {
  (void)N;
  if (M > 16 || K / 128 > small::GMAX * MAX_SPLITS) return false;
  return variant == 2 || (variant == 0 && M <= 16);
}

// Workspace: FP32 partials [splits][M][N].
size_t small_workspace_bytes(int M, int N, int K, int num_cu) {
  SmallPlan p = small_plan(M, N, K, num_cu);
  return p.splits > 1 ? (size_t)p.splits * M * N * sizeof(float) : 0;
}

template <bool BF16, int FMT>
static void launch_small_t(GemmArgs& a, const SmallPlan& p, hipStream_t st) {
  dim3 grid((a.N + 127) / 128, p.splits);
  hipLaunchKernelGGL((gemm_small_kernel<BF16, FMT>), grid, dim3(256), 0, st, a);
}

template <bool BF16, int FMT>
static void launch_large_t(GemmArgs& a, hipStream_t st) {
  const int tm = (a.M + large::BM - 1) / large::BM, tn = (a.N + large::BN - 1) / large::BN;
  hipLaunchKernelGGL((gemm_large_kernel<BF16, FMT>), dim3(tm * tn), dim3(large::THREADS), 0, st, a, tm, tn);
}

hipError_t launch_gemm(int fmt, bool x_bf16, GemmArgs a, int num_cu, int variant, hipStream_t st) {
  // variant: 0 = automatic, 1 = force large-M kernel, 2 = force small-M kernel (M <= 16)
  const bool small = small_path(a.M, a.N, a.K, variant);
  if (small) {
    SmallPlan p = small_plan(a.M, a.N, a.K, num_cu);
    a.splits = p.splits;
    a.gps = p.gps;
    if (fmt == FMT_TERNARY) {
      if (x_bf16) launch_small_t<true, FMT_TERNARY>(a, p, st);
      else launch_small_t<false, FMT_TERNARY>(a, p, st);
    } else {
      if (x_bf16) launch_small_t<true, FMT_BINARY>(a, p, st);
      else launch_small_t<false, FMT_BINARY>(a, p, st);
    }
    if (a.splits > 1) {
      const int64_t total = (int64_t)a.M * a.N;
      int grid = (int)((total + 255) / 256);
      if (grid > 4096) grid = 4096;
      hipLaunchKernelGGL(splitk_reduce_kernel, dim3(grid), dim3(256), 0, st, a);
    }
  } else {
    a.splits = 1;
    a.gps = a.K / 128;
    if (fmt == FMT_TERNARY) {
      if (x_bf16) launch_large_t<true, FMT_TERNARY>(a, st);
      else launch_large_t<false, FMT_TERNARY>(a, st);
    } else {
      if (x_bf16) launch_large_t<true, FMT_BINARY>(a, st);
      else launch_large_t<false, FMT_BINARY>(a, st);
    }
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
