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
// Large-M kernel: 128x128 output tile per workgroup, 4 waves of 64x64, one
// 128-group (BK = 128) per pipeline stage, LDS double buffered.
//   LDS A : activations, 128 rows x 128 k, row stride 136 (bank-spread)
//   LDS B : packed codes kept packed: ternary [4 pair][128 n] x 8 bytes,
//           binary [4][128 n] x 4 bytes
//   LDS S : the FP32 factor +-2*scale per column
// ===========================================================================
namespace large {
constexpr int BM = 128, BN = 128, AST = 136, THREADS = 256;
}

template <bool BF16, int FMT>
__global__ __launch_bounds__(256) void gemm_large_kernel(GemmArgs a) {
  using namespace large;
  constexpr bool TERN = FMT == FMT_TERNARY;
  constexpr int BWORDS = TERN ? 8 : 4;               // packed words per row per group
  __shared__ __align__(16) uint16_t sA[2][BM * AST];
  __shared__ __align__(16) uint32_t sB[2][BWORDS * BN];
  __shared__ float sS[2][BN];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, q = lane >> 4, r16 = lane & 15;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int G = a.K >> 7;
  const int64_t wrow = TERN ? (a.K >> 2) : (a.K >> 3);   // packed bytes per weight row
  const float factor = TERN ? 2.0f : -2.0f;

  // ---- global -> register staging of one group ----
  u32x4 ra[8];
  u32x4 rb;
  float rs = 0.0f;
  auto gload = [&](int g) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int idx = tid + THREADS * i;
      int row = idx >> 4, c16 = idx & 15;
      int m = m0 + row;
      if (m < a.M)
        ra[i] = *(const u32x4*)(a.X + (int64_t)m * a.ldx + (g << 7) + c16 * 8);
      else
        ra[i] = u32x4{0u, 0u, 0u, 0u};
    }
    if (TERN) {
      int row = tid >> 1, half = tid & 1, n = n0 + row;
      if (n < a.N)
        rb = *(const u32x4*)(a.W + (int64_t)n * wrow + g * 32 + half * 16);
      else
        rb = u32x4{0x55555555u, 0x55555555u, 0x55555555u, 0x55555555u};   // t = 0
    } else if (tid < BN) {
      int n = n0 + tid;
      if (n < a.N)
        rb = *(const u32x4*)(a.W + (int64_t)n * wrow + g * 16);
      else
        rb = u32x4{0u, 0u, 0u, 0u};
    }
    if (tid < BN) {
      int n = n0 + tid;
      rs = n < a.N ? factor * half_bits_to_float(a.S[(int64_t)n * G + g]) : 0.0f;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int idx = tid + THREADS * i;
      int row = idx >> 4, c16 = idx & 15;
      *(u32x4*)&sA[buf][row * AST + c16 * 8] = ra[i];
    }
    if (TERN) {
      int row = tid >> 1, half = tid & 1;
      u32x2* b2 = (u32x2*)sB[buf];
      b2[(2 * half) * BN + row] = u32x2{rb[0], rb[1]};
      b2[(2 * half + 1) * BN + row] = u32x2{rb[2], rb[3]};
    } else if (tid < BN) {
#pragma unroll
      for (int j = 0; j < 4; ++j) sB[buf][j * BN + tid] = rb[j];
    }
    if (tid < BN) sS[buf][tid] = rs;
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  gload(0);
  sstore(0);
  __syncthreads();

  for (int g = 0; g < G; ++g) {
    const int cur = g & 1;
    if (g + 1 < G) gload(g + 1);

    // packed words of this lane group for the wave's 4 column blocks
    uint32_t w0[4], w1[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int nl = wn * 64 + j * 16 + r16;
      if (TERN) {
        u32x2 v = ((const u32x2*)sB[cur])[q * BN + nl];
        w0[j] = v[0];
        w1[j] = v[1];
      } else {
        w0[j] = sB[cur][q * BN + nl];
        w1[j] = 0u;
      }
    }
    f32x4 tmp[4][4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      u32x4 af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *(const u32x4*)&sA[cur][(wm * 64 + i * 16 + r16) * AST + 32 * q + 8 * c];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bf[j] = TERN ? tern_chunk<BF16>(w0[j], w1[j], c) : bin_chunk<BF16>(w0[j], c);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          tmp[i][j] = mfma16<BF16>(af[i], bf[j], c == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : tmp[i][j]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float s = sS[cur][wn * 64 + j * 16 + r16];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i][j] += s * tmp[i][j];
    }
    if (g + 1 < G) sstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: bias, activation, one RNE cast, store ----
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int n = n0 + wn * 64 + j * 16 + r16;
    if (n >= a.N) continue;
    float b = a.bias ? load_bias(a.bias, a.bias_dtype, n) : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int m = m0 + wm * 64 + i * 16 + 4 * q + r;
        if (m < a.M) store_out(a.Y, a.ldy, a.y_dtype, m, n, finish(acc[i][j][r], b, a.act));
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
  dim3 grid((a.N + large::BN - 1) / large::BN, (a.M + large::BM - 1) / large::BM);
  hipLaunchKernelGGL((gemm_large_kernel<BF16, FMT>), grid, dim3(large::THREADS), 0, st, a);
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
