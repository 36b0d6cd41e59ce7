// gfx950 low-bit-weight GEMM, small M (M <= 16): Y = act(X W^T + bias),
// W = scale_g * t, by weight streaming on v_mfma_f32_16x16x32, and the
// dispatcher that sends M > 16 to the large-M kernel (gemm_large.hip).
//
// The weight definition is the one of "Como Bonsai Ternary 4B revoluciona la
// difusion texto-imagen", section "Representacion y almacenamiento de los
// pesos ternarios": w = scale_g * t, one FP16 scale per 128 weights along K,
// t stored with 2 bits (ternary) or 1 bit (binary). Per output element and
// 128-group the kernels form P_g = sum_{k in g} x_k * (2 t_k) on the MFMA
// (FP32 accumulation, exact products) and add (s_g / 2) * P_g in FP32.
#include <algorithm>
#include <cmath>

#include "common.h"

namespace lowbit {

void launch_large(int fmt, bool x_bf16, const GemmArgs& a, int num_cu, int variant, hipStream_t st);

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
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(NB * (CB + 1)));
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
      if (rq == 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(XDMA / 4));
      else if (rq == 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(XDMA / 2));
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm(XDMA));
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
      launch_large(fmt, x_bf16, a, num_cu, variant, st);
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
