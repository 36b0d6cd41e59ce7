// gfx950 low-bit-weight GEMM: Y = act(X W^T + bias), W = scale_g * t.
//
// The weight definition is the one of "Como Bonsai Ternary 4B revoluciona la
// difusion texto-imagen", section "Representacion y almacenamiento de los
// pesos ternarios": w = scale_g * t, one FP16 scale per 128 weights along K,
// t stored with 2 bits (ternary) or 1 bit (binary).
//
// Both kernels compute, for every output element and every 128-group g,
//   P_g = sum_{k in g} x_k * t_k            (MFMA, FP32 accumulation, exact
//                                             products: t/2 is a power of two)
//   acc += (2 s_g) * P_g                    (one FP32 FMA per group)
// which is the definition up to FP32 rounding order. Zero, subnormal and
// negative scales need no special case.
//
// MFMA: v_mfma_f32_16x16x32_{bf16,f16}. A lane l holds operand rows / output
// columns l % 16 and K slots 8*(l/16) .. +7; the K order inside a 128-group is
// free as long as both operands use the same one, so each lane group q = l/16
// owns k-local [32q, 32q+32) of every group and chunk c (one MFMA) uses its
// slots 32q + 8c .. +7. This lets a lane read its activations as 16 contiguous
// bytes and its codes as one or two packed words.
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
//    group's scale c_g = +-2 s_g, and at each group boundary the accumulator
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
  const float factor = TERN ? 2.0f : -2.0f;
  const uint32_t table = tern_table<BF16>();
  const uint32_t bmask = 0x80008000u, bbase = BF16 ? 0x3F003F00u : 0x38003800u;

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
  auto bload = [&](int g, u32x4 (&bw)[2], float (&sc)[2]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint8_t* p = a.W + (int64_t)ncol[j] * wrow;
      if (TERN) {
        bw[j] = *(const u32x4*)(p + g * 32 + 16 * q);
      } else {
        u32x2 v = *(const u32x2*)(p + g * 16 + 8 * q);
        bw[j] = u32x4{v[0], v[1], 0u, 0u};
      }
      sc[j] = factor * half_bits_to_float(a.S[(int64_t)ncol[j] * G + g]);
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  float cref[2] = {1.0f, 1.0f};                 // reference scale of the accumulator

  u32x4 A[4][8];
  u32x4 bw[2];
  float sc[2];

  // one column block of one group: rescale to the group's scale, then 32 MFMAs
  auto block = [&](int j, bool refill, int nbuf) {
    const float s = sc[j];
    const bool zero = s == 0.0f;
    const float r = zero ? 1.0f : cref[j] / s;
    cref[j] = zero ? cref[j] : s;
    const uint32_t tb = zero ? 0u : table;
    const uint32_t mk = zero ? 0u : bmask, bs = zero ? 0u : bbase;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i][j] *= r;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const u32x4 bf = TERN ? tern_chunk_t(bw[j][st >> 1], st & 1, tb)
                            : bin_chunk_t(bw[j][st >> 2], st & 3, mk, bs);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i][j] = mfma32<BF16>(A[i][st], bf, acc[i][j]);
      if (refill) {
#pragma unroll
        for (int i = 0; i < 4; ++i) A[i][st] = afrag(nbuf, i, st);
      }
    }
  };

  // prologue: stages 0 and 1 in flight, group-0 codes, then group-0 fragments
  dma(0, 0);
  if (G > 1) dma(1, 1);
  bload(0, bw, sc);
  __builtin_amdgcn_s_waitcnt(0);        // own DMA + loads done
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int st = 0; st < 8; ++st) A[i][st] = afrag(0, i, st);

  for (int g = 0; g < G; ++g) {
    const bool more = g + 1 < G;
    u32x4 bwn[2];
    float scn[2];
    block(0, false, 0);
    // pipeline point: stage g+1 landed everywhere; refill stage g+2
    if (more) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      bload(g + 1, bwn, scn);
      if (g + 2 < G) dma(g + 2, (g + 2) % STAGES);
      block(1, true, (g + 1) % STAGES);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        bw[j] = bwn[j];
        sc[j] = scn[j];
      }
    } else {
      block(1, false, 0);
    }
  }

  // ---- epilogue: final scale, bias, activation, one RNE cast, store ----
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

// ===========================================================================
// Small-M kernel (M <= 16): weight streaming. A workgroup owns NB column
// blocks of 16 and a K range; its 4 waves split the K range into slices of
// up to KS groups. Per round every wave keeps its activation fragments in
// registers and issues all its packed-word loads at once, so each wave has
// NB*KS*512 (ternary) bytes of weights in flight; the 4 wave partials are
// summed through LDS. With a.splits > 1 the K range is also split across
// workgroups and FP32 partials go to the workspace, summed afterwards in a
// fixed order (deterministic).
// ===========================================================================
template <bool BF16, int FMT, int NB, int KS>
__global__ __launch_bounds__(256) void gemm_small_kernel(GemmArgs a) {
  constexpr bool TERN = FMT == FMT_TERNARY;
  __shared__ f32x4 red[4][NB][64];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, q = lane >> 4, r16 = lane & 15;
  const int G = a.K >> 7;
  const int64_t wrow = TERN ? (a.K >> 2) : (a.K >> 3);
  const float factor = TERN ? 2.0f : -2.0f;
  const int gb0 = blockIdx.y * a.gps;
  const int gb1 = min(G, gb0 + a.gps);
  const bool mval = r16 < a.M;
  const uint16_t* xrow = a.X + (int64_t)(mval ? r16 : 0) * a.ldx;

  int ncol[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    int n = (blockIdx.x * NB + nb) * 16 + r16;
    ncol[nb] = n < a.N ? n : a.N - 1;                    // clamped: loads stay in bounds
  }

  f32x4 part[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) part[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int r0 = gb0; r0 < gb1; r0 += 4 * KS) {
    const int gw = r0 + wave * KS;
    const int ng = max(0, min(KS, gb1 - gw));
    u32x2 wd[NB][KS];
    float sc[NB][KS];
    u32x4 af[KS][4];
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      if (i < ng) {
        const int g = gw + i;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const uint8_t* p = a.W + (int64_t)ncol[nb] * wrow;
          if (TERN)
            wd[nb][i] = *(const u32x2*)(p + g * 32 + q * 8);
          else
            wd[nb][i] = u32x2{*(const uint32_t*)(p + g * 16 + q * 4), 0u};
          sc[nb][i] = factor * half_bits_to_float(a.S[(int64_t)ncol[nb] * G + g]);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c)
          af[i][c] = mval ? *(const u32x4*)(xrow + (g << 7) + 32 * q + 8 * c) : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      if (i < ng) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          f32x4 tmp = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            u32x4 bf = TERN ? tern_chunk<BF16>(wd[nb][i][0], wd[nb][i][1], c)
                            : bin_chunk<BF16>(wd[nb][i][0], c);
            tmp = mfma16<BF16>(af[i][c], bf, tmp);
          }
          part[nb] += sc[nb][i] * tmp;
        }
      }
    }
  }

#pragma unroll
  for (int nb = 0; nb < NB; ++nb) red[wave][nb][lane] = part[nb];
  __syncthreads();
  if (tid < NB * 64) {
    const int nb = tid >> 6, ln = tid & 63;
    f32x4 v = red[0][nb][ln];
#pragma unroll
    for (int w = 1; w < 4; ++w) v += red[w][nb][ln];
    const int n = (blockIdx.x * NB + nb) * 16 + (ln & 15);
    if (n < a.N) {
      const int mbase = 4 * (ln >> 4);
      if (a.splits == 1) {
        float b = a.bias ? load_bias(a.bias, a.bias_dtype, n) : 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (mbase + r < a.M) store_out(a.Y, a.ldy, a.y_dtype, mbase + r, n, finish(v[r], b, a.act));
      } else {
        float* ws = a.ws + (int64_t)blockIdx.y * a.M * a.N;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (mbase + r < a.M) ws[(int64_t)(mbase + r) * a.N + n] = v[r];
      }
    }
  }
}

// Sum of split-K partials in split order, then bias, activation and cast.
__global__ void splitk_reduce_kernel(GemmArgs a) {
  const int64_t total = (int64_t)a.M * a.N;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    float v = a.ws[i];
    for (int s = 1; s < a.splits; ++s) v += a.ws[(int64_t)s * total + i];
    const int m = (int)(i / a.N), n = (int)(i % a.N);
    float b = a.bias ? load_bias(a.bias, a.bias_dtype, n) : 0.0f;
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

// Small-M plan: NB column blocks per workgroup, KS groups per wave slice,
// splits across workgroups. Returns the number of splits (1 = no workspace).
struct SmallPlan { int nb, ks, splits, gps; };

static SmallPlan small_plan(int M, int N, int K, int num_cu) {
  (void)M;
  const int G = K / 128;
  SmallPlan p;
  p.ks = 4;
  // column blocks per workgroup: more when there are many columns
  const int nblk16 = (N + 15) / 16;
  p.nb = nblk16 >= 4 * num_cu ? 4 : (nblk16 >= 2 * num_cu ? 2 : 1);
  const int nwg = (nblk16 + p.nb - 1) / p.nb;
  // split K across workgroups until there are about 2 workgroups per CU,
  // but keep at least one full round (4 waves x ks groups) per split
  int splits = 1;
  while (nwg * splits < 2 * num_cu && (G + splits) / (splits + 1) >= 4 * p.ks) ++splits;
  p.gps = (G + splits - 1) / splits;
  p.splits = (G + p.gps - 1) / p.gps;
  return p;
}

size_t small_workspace_bytes(int M, int N, int K, int num_cu) {
  SmallPlan p = small_plan(M, N, K, num_cu);
  return p.splits > 1 ? (size_t)p.splits * M * N * sizeof(float) : 0;
}

template <bool BF16, int FMT>
static void launch_small_t(GemmArgs& a, const SmallPlan& p, hipStream_t st) {
  dim3 block(256);
  dim3 grid((a.N + 16 * p.nb - 1) / (16 * p.nb), p.splits);
  if (p.nb == 4)
    hipLaunchKernelGGL((gemm_small_kernel<BF16, FMT, 4, 4>), grid, block, 0, st, a);
  else if (p.nb == 2)
    hipLaunchKernelGGL((gemm_small_kernel<BF16, FMT, 2, 4>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((gemm_small_kernel<BF16, FMT, 1, 4>), grid, block, 0, st, a);
}

template <bool BF16, int FMT>
static void launch_large_t(GemmArgs& a, hipStream_t st) {
  const int tm = (a.M + large::BM - 1) / large::BM, tn = (a.N + large::BN - 1) / large::BN;
  hipLaunchKernelGGL((gemm_large_kernel<BF16, FMT>), dim3(tm * tn), dim3(large::THREADS), 0, st, a, tm, tn);
}

int small_m_limit() { return 16; }

hipError_t launch_gemm(int fmt, bool x_bf16, GemmArgs a, int num_cu, int variant, hipStream_t st) {
  // variant: 0 = automatic, 1 = force large-M kernel, 2 = force small-M kernel (M <= 16)
  bool small = variant == 2 || (variant == 0 && a.M <= small_m_limit());
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
      int64_t total = (int64_t)a.M * a.N;
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
