// INT2 / 1-bit / base-3 weight packers, the unpacker and the base-3 -> INT2
// transcoder (load-time kernels).
//
// The storage is the 2-bit-per-ternary ("INT2") and 1-bit-per-binary form the
// pages describe ("Como Bonsai Ternary 4B revoluciona la difusion
// texto-imagen", section "Representacion y almacenamiento de los pesos
// ternarios"). The bit layout is this library's own (see lowbit.h): even k
// in the low half of each 32-bit word, odd k in the high half.
//
// One thread builds one 32-bit output word from 16 (ternary) or 32 (binary)
// int8 codes read with 128-bit loads; consecutive threads own consecutive
// words, so reads and writes are fully coalesced. This is HBM-bound work
// (8 bits in, 2 or 1 bit out per weight).
#include "common.h"

namespace lowbit {

__device__ __forceinline__ void count_invalid(int32_t* counter, int bad) {
  // wave-level sum first: one atomic per wave that saw an invalid code
  unsigned long long m = __ballot(bad != 0);
  if (m == 0) return;
  int total = bad;
  for (int off = 32; off > 0; off >>= 1) total += __shfl_xor(total, off);
  if ((threadIdx.x & 63) == __builtin_ctzll(m)) atomicAdd(counter, total);
}

// ternary value -> 2-bit two's complement, invalid values -> code 0 (t = 0)
__device__ __forceinline__ uint32_t tern_code(int8_t t, int& bad) {
  bool ok = (t >= -1) && (t <= 1);
  bad += ok ? 0 : 1;
  return ok ? ((uint32_t)t & 3u) : 0u;
}

__global__ void pack_ternary_kernel(const int8_t* __restrict__ codes, uint32_t* __restrict__ out,
                                    int64_t nwords, int32_t* counter) {
  int bad = 0;
  for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < nwords;
       w += (int64_t)gridDim.x * blockDim.x) {
    // words are laid out row after row along K, and K % 16 == 0, so word w
    // covers codes 16w .. 16w+15 of the flattened [N][K] array
    u32x4 v = *(const u32x4*)(codes + 16 * w);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      int8_t t = (int8_t)((v[j >> 2] >> (8 * (j & 3))) & 0xFF);
      uint32_t c = tern_code(t, bad);
      if (j & 1) hi |= c << (2 * (j >> 1));
      else lo |= c << (2 * (j >> 1));
    }
    out[w] = lo | (hi << 16);
  }
  if (counter) count_invalid(counter, bad);
}

__global__ void pack_binary_kernel(const int8_t* __restrict__ codes, uint32_t* __restrict__ out,
                                   int64_t nwords, int32_t* counter) {
  int bad = 0;
  for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < nwords;
       w += (int64_t)gridDim.x * blockDim.x) {
    u32x4 v0 = *(const u32x4*)(codes + 32 * w);
    u32x4 v1 = *(const u32x4*)(codes + 32 * w + 16);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      uint32_t word = j < 16 ? v0[j >> 2] : v1[(j - 16) >> 2];
      int8_t t = (int8_t)((word >> (8 * (j & 3))) & 0xFF);
      bad += (t == 1 || t == -1) ? 0 : 1;
      uint32_t b = (t == 1) ? 1u : 0u;
      if (j & 1) hi |= b << (j >> 1);
      else lo |= b << (j >> 1);
    }
    out[w] = lo | (hi << 16);
  }
  if (counter) count_invalid(counter, bad);
}

__global__ void unpack_ternary_kernel(const uint32_t* __restrict__ in, int8_t* __restrict__ codes,
                                      int64_t nwords, int32_t* counter) {
  int bad = 0;
  for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < nwords;
       w += (int64_t)gridDim.x * blockDim.x) {
    uint32_t x = in[w];
    u32x4 o = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      uint32_t c = (x >> (16 * (j & 1) + 2 * (j >> 1))) & 3u;
      bad += (c == 2u) ? 1 : 0;                     // 10 is not a ternary code
      int t = (c == 2u) ? 0 : ((int)(c << 30) >> 30);   // sign-extend the 2-bit field
      o[j >> 2] |= ((uint32_t)(uint8_t)(int8_t)t) << (8 * (j & 3));
    }
    *(u32x4*)(codes + 16 * w) = o;
  }
  if (counter) count_invalid(counter, bad);
}

__global__ void unpack_binary_kernel(const uint32_t* __restrict__ in, int8_t* __restrict__ codes,
                                     int64_t nwords) {
  for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < nwords;
       w += (int64_t)gridDim.x * blockDim.x) {
    uint32_t x = in[w];
    u32x4 o0 = {0u, 0u, 0u, 0u}, o1 = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      uint32_t b = (x >> (16 * (j & 1) + (j >> 1))) & 1u;
      uint32_t byte = b ? 0x01u : 0xFFu;
      if (j < 16) o0[j >> 2] |= byte << (8 * (j & 3));
      else o1[(j - 16) >> 2] |= byte << (8 * (j & 3));
    }
    *(u32x4*)(codes + 32 * w) = o0;
    *(u32x4*)(codes + 32 * w + 16) = o1;
  }
}

// 4-bit codes (the text encoder's group-quantised weights, lowbit.h): uint8
// codes 0 .. 15, eight per word, the code of k = 2i + h at bits 16h + 4i.
// Codes above 15 are counted and stored as 0.
__global__ void pack_int4_kernel(const uint8_t* __restrict__ codes, uint32_t* __restrict__ out, int64_t nwords,
                                 int32_t* counter) {
  int bad = 0;
  for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < nwords;
       w += (int64_t)gridDim.x * blockDim.x) {
    const u32x2 v = *(const u32x2*)(codes + 8 * w);
    uint32_t r = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t q = (v[j >> 2] >> (8 * (j & 3))) & 0xFFu;
      bad += q > 15u ? 1 : 0;
      r |= (q > 15u ? 0u : q) << (16 * (j & 1) + 4 * (j >> 1));
    }
    out[w] = r;
  }
  if (counter) count_invalid(counter, bad);
}

__global__ void unpack_int4_kernel(const uint32_t* __restrict__ in, uint8_t* __restrict__ codes, int64_t nwords) {
  for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < nwords;
       w += (int64_t)gridDim.x * blockDim.x) {
    const uint32_t x = in[w];
    u32x2 o = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j >> 2] |= ((x >> (16 * (j & 1) + 4 * (j >> 1))) & 15u) << (8 * (j & 3));
    *(u32x2*)(codes + 8 * w) = o;
  }
}

// ---------------------------------------------------------------------------
// Base-3 storage: five ternary values per byte (3^5 = 243 <= 256), the form
// that approaches the log2(3) bits the pages price a ternary value at
// ("Representacion y almacenamiento de los pesos ternarios"; "Introducing
// 1-bit and Ternary Bonsai Image 4B", section on the quantisation
// arithmetic). Layout (lowbit.h): digit d = t + 1; byte j of a row holds
// k = 5j .. 5j+4 as sum_i d[5j+i] * 3^i; a row is ceil(K/5) bytes; bytes of
// value 243 and above are invalid. The GEMM reads the INT2 form, which
// base3_to_int2_kernel produces on the device at load time.
//
// These kernels walk (row, 64-item segment) pairs, one segment per wave:
// the 64-bit division that finds the row is wave-uniform and done once per
// segment, and each wave reads and writes contiguous runs of one row.

constexpr int kSeg = 64;

// f(n, i) for every item i < per_row of every row n < N, one item per lane.
template <class F>
__device__ __forceinline__ void for_row_items(int64_t N, int64_t per_row, F f) {
  const int64_t segs = (per_row + kSeg - 1) / kSeg;
  const int wpb = blockDim.x / 64;
  const int64_t stride = (int64_t)gridDim.x * wpb;
  const int lane = threadIdx.x & 63;
  for (int64_t s = (int64_t)blockIdx.x * wpb + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
       s < N * segs; s += stride) {
    const int64_t n = s / segs;
    const int64_t i = (s - n * segs) * kSeg + lane;
    if (i < per_row) f(n, i);
  }
}

__global__ void pack_base3_kernel(const int8_t* __restrict__ codes, uint8_t* __restrict__ out,
                                  int64_t N, int64_t K, int32_t* counter) {
  const int64_t nb = (K + 4) / 5;
  int bad = 0;
  for_row_items(N, nb, [&](int64_t n, int64_t j) {
    const int8_t* row = codes + n * K;
    uint32_t v = 0, p3 = 1;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const int64_t k = 5 * j + i;
      if (k < K) {
        const int t = row[k];
        const bool ok = t >= -1 && t <= 1;
        bad += ok ? 0 : 1;
        v += (uint32_t)(ok ? t + 1 : 1) * p3;      // an invalid value is stored as t = 0
      }
      p3 *= 3u;
    }
    out[n * nb + j] = (uint8_t)v;
  });
  if (counter) count_invalid(counter, bad);
}

__global__ void unpack_base3_kernel(const uint8_t* __restrict__ in, int8_t* __restrict__ codes,
                                    int64_t N, int64_t K, int32_t* counter) {
  const int64_t nb = (K + 4) / 5;
  int bad = 0;
  for_row_items(N, nb, [&](int64_t n, int64_t j) {
    uint32_t v = in[n * nb + j];
    const bool ok = v < 243u;
    int8_t* row = codes + n * K;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const int64_t k = 5 * j + i;
      if (k < K) {
        row[k] = ok ? (int8_t)((int)(v % 3u) - 1) : (int8_t)0;
        bad += ok ? 0 : 1;
      }
      v /= 3u;
    }
  });
  if (counter) count_invalid(counter, bad);
}

// Table entry of one base-3 byte v, split by the parity of k inside the
// 80-value units below: bits 0-5 hold the INT2 codes of digits 0, 2, 4,
// bits 8-11 those of digits 1, 3 (digit d = 0, 1, 2 -> t = -1, 0, +1 ->
// 11, 00, 01), bit 16 is set when v is invalid, whose five values all get
// the invalid INT2 pattern 10. The table is built by the compiler.
struct Base3Table {
  uint32_t e[256];
};

constexpr Base3Table make_base3_table() {
  Base3Table t{};
  for (uint32_t v = 0; v < 256; ++v) {
    if (v >= 243u) {
      t.e[v] = 0x2Au | (0xAu << 8) | (1u << 16);
      continue;
    }
    uint32_t c[5] = {0, 0, 0, 0, 0}, r = v;
    for (int i = 0; i < 5; ++i) {
      c[i] = ((r % 3u) + 3u) & 3u;
      r /= 3u;
    }
    t.e[v] = (c[0] | (c[2] << 2) | (c[4] << 4)) | ((c[1] | (c[3] << 2)) << 8);
  }
  return t;
}

__constant__ Base3Table kBase3Table = make_base3_table();

// OR `val` into the bit stream s[0..2] at constant bit position `pos`.
template <int POS>
__device__ __forceinline__ void put_bits(uint32_t (&s)[3], uint32_t val) {
  s[POS / 32] |= val << (POS % 32);
  if constexpr (POS % 32 > 26) s[POS / 32 + 1] |= val >> (32 - POS % 32);
}

// Byte b of a unit covers unit-local k = 5b .. 5b+4. For even b, digits
// 0, 2, 4 are the even k and enter the even-k stream after 5b/2 earlier
// codes (bit 5b), digits 1, 3 the odd-k stream at bit 5b; for odd b, digits
// 1, 3 are the even k (bit 5b+1) and digits 0, 2, 4 the odd k (bit 5b-1).
template <int B>
__device__ __forceinline__ void put_byte(uint32_t (&ev)[3], uint32_t (&od)[3], uint32_t e) {
  const uint32_t d024 = e & 0x3Fu, d13 = (e >> 8) & 0xFu;
  if constexpr (B % 2 == 0) {
    put_bits<5 * B>(ev, d024);
    put_bits<5 * B>(od, d13);
  } else {
    put_bits<5 * B + 1>(ev, d13);
    put_bits<5 * B - 1>(od, d024);
  }
}

template <int B>
__device__ __forceinline__ void put_bytes(uint32_t (&ev)[3], uint32_t (&od)[3], uint32_t& flags,
                                          const uint32_t (&u)[4], const uint32_t* lut) {
  if constexpr (B < 16) {
    const uint32_t e = lut[(u[B / 4] >> (8 * (B % 4))) & 0xFFu];
    flags |= ((e >> 16) & 1u) << B;
    put_byte<B>(ev, od, e);
    put_bytes<B + 1>(ev, od, flags, u, lut);
  }
}

// Decode one unit of 80 values (16 base-3 bytes u[0..3], little-endian)
// into its INT2 words; returns the invalid-byte flags, bit b for byte b.
__device__ __forceinline__ uint32_t base3_unit_decode(const uint32_t (&u)[4], const uint32_t* lut,
                                                      uint32_t (&words)[5]) {
  uint32_t ev[3] = {0u, 0u, 0u}, od[3] = {0u, 0u, 0u}, flags = 0;
  put_bytes<0>(ev, od, flags, u, lut);
#pragma unroll
  for (int j = 0; j < 5; ++j)
    words[j] = (j % 2 == 0) ? ((ev[j / 2] & 0xFFFFu) | (od[j / 2] << 16))
                            : ((ev[j / 2] >> 16) | (od[j / 2] & 0xFFFF0000u));
  return flags;
}

// Units of 80 values: 16 base-3 bytes in, five INT2 words out (80 = 16 * 5,
// so a unit starts on a byte and on a word). A row has ceil(K/80) units and
// its last one may hold fewer words (K % 16 == 0). Because a row's last unit
// uses exactly the row's remaining bytes and words, the units of the whole
// matrix, taken in row order, read one contiguous byte run and write one
// contiguous word run. Each wave takes 64 consecutive units: it copies their
// byte run into LDS with 16-byte loads (every 16-byte chunk read holds at
// least one byte of the run), each lane decodes its unit from LDS (a unit
// sits at any byte alignment: aligned dwords shifted with alignbyte) and
// stages its words in LDS, and the wave writes the word run with contiguous
// dword stores. LDS regions are per wave, so the waves of a workgroup never
// wait for one another inside the walk.
constexpr int kB3Waves = 4;
constexpr int kB3InDwords = 264;    // 65 chunks of 16 bytes, plus the 5-dword reach of the last lane
constexpr int kB3OutWords = 320;    // 64 units x 5 words

__global__ void __launch_bounds__(256) base3_to_int2_kernel(
    const uint8_t* __restrict__ in, uint32_t* __restrict__ out, int64_t N, int64_t K,
    int32_t* counter) {
  __shared__ uint32_t lut[256];
  __shared__ uint32_t stage_in[kB3Waves][kB3InDwords];
  __shared__ uint32_t stage_out[kB3Waves][kB3OutWords];
  lut[threadIdx.x] = kBase3Table.e[threadIdx.x];
  __syncthreads();
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  uint32_t* sin = stage_in[wv];
  uint32_t* sout = stage_out[wv];
  const int64_t nb = (K + 4) / 5, nw = K / 16, units = (nw + 4) / 5;
  const int64_t total = N * units;
  const bool small = total <= 0xFFFFFFFFll;
  const int64_t nchunks = (total + 63) / 64;
  // first byte and first word of unit x (x == total gives the ends of the runs)
  auto starts = [&](int64_t x, int64_t& b, int64_t& w, int64_t& u) {
    const int64_t n = small ? (int64_t)((uint32_t)x / (uint32_t)units) : x / units;
    u = x - n * units;
    b = n * nb + 16 * u;
    w = n * nw + 5 * u;
  };
  int bad = 0;
  for (int64_t c = (int64_t)blockIdx.x * kB3Waves + wv; c < nchunks; c += (int64_t)gridDim.x * kB3Waves) {
    const int64_t e0 = 64 * c, e = e0 + lane;
    const int64_t eend = min(e0 + 64, total);
    int64_t b0, w0, u0, bend, wend, uend;
    starts(e0, b0, w0, u0);
    starts(eend, bend, wend, uend);
    const int64_t A = b0 & ~(int64_t)15;
    const int nck = (int)((bend - A + 15) / 16);        // <= 65
    for (int k = lane; k < nck; k += 64) {
      const u32x4 v = *(const u32x4*)(in + A + 16 * k);
      sin[4 * k + 0] = v[0];
      sin[4 * k + 1] = v[1];
      sin[4 * k + 2] = v[2];
      sin[4 * k + 3] = v[3];
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if (e < eend) {
      int64_t b, w, u;
      starts(e, b, w, u);
      const int nwords = (int)min((int64_t)5, nw - 5 * u);
      const int o = (int)(b - A);
      const int oa = o >> 2;
      const uint32_t off = (uint32_t)o & 3u;
      uint32_t uu[4], words[5];
#pragma unroll
      for (int i = 0; i < 4; ++i) uu[i] = __builtin_amdgcn_alignbyte(sin[oa + i + 1], sin[oa + i], off);
      const uint32_t flags = base3_unit_decode(uu, lut, words);
      if (flags) {
        const int nvals = 16 * nwords;
#pragma unroll
        for (int bb = 0; bb < 16; ++bb)
          if ((flags >> bb) & 1u) bad += max(0, min(5, nvals - 5 * bb));
      }
      const int wo = (int)(w - w0);
#pragma unroll
      for (int j = 0; j < 5; ++j)
        if (j < nwords) sout[wo + j] = words[j];
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const int T = (int)(wend - w0);                      // <= 320
    for (int k = lane; k < T; k += 64) out[w0 + k] = sout[k];
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }
  if (counter) count_invalid(counter, bad);
}

__global__ void zero_int_kernel(int32_t* p) { *p = 0; }

static int grid_for(int64_t work, int block) {
  int64_t g = (work + block - 1) / block;
  if (g > 65536) g = 65536;
  return (int)(g < 1 ? 1 : g);
}

// blocks of four waves for a walk over N rows of per_row items
static int grid_for_rows(int64_t N, int64_t per_row) {
  const int64_t waves = N * ((per_row + kSeg - 1) / kSeg);
  int64_t g = (waves + 3) / 4;
  if (g > 65536) g = 65536;
  return (int)(g < 1 ? 1 : g);
}

hipError_t launch_pack(int fmt, const int8_t* codes, int64_t N, int64_t K, uint8_t* packed,
                       int32_t* counter, hipStream_t st) {
  if (counter) hipLaunchKernelGGL(zero_int_kernel, dim3(1), dim3(1), 0, st, counter);
  if (fmt == FMT_BASE3) {
    hipLaunchKernelGGL(pack_base3_kernel, dim3(grid_for_rows(N, (K + 4) / 5)), dim3(256), 0, st,
                       codes, packed, N, K, counter);
    return hipGetLastError();
  }
  if (fmt == FMT_INT4) {
    const int64_t nwords = N * K / 8;
    hipLaunchKernelGGL(pack_int4_kernel, dim3(grid_for(nwords, 256)), dim3(256), 0, st, (const uint8_t*)codes,
                       (uint32_t*)packed, nwords, counter);
    return hipGetLastError();
  }
  int64_t nwords = N * K / (fmt == FMT_TERNARY ? 16 : 32);
  const int block = 256;
  if (fmt == FMT_TERNARY)
    hipLaunchKernelGGL(pack_ternary_kernel, dim3(grid_for(nwords, block)), dim3(block), 0, st,
                       codes, (uint32_t*)packed, nwords, counter);
  else
    hipLaunchKernelGGL(pack_binary_kernel, dim3(grid_for(nwords, block)), dim3(block), 0, st,
                       codes, (uint32_t*)packed, nwords, counter);
  return hipGetLastError();
}

hipError_t launch_unpack(int fmt, const uint8_t* packed, int64_t N, int64_t K, int8_t* codes,
                         int32_t* counter, hipStream_t st) {
  if (counter) hipLaunchKernelGGL(zero_int_kernel, dim3(1), dim3(1), 0, st, counter);
  if (fmt == FMT_BASE3) {
    hipLaunchKernelGGL(unpack_base3_kernel, dim3(grid_for_rows(N, (K + 4) / 5)), dim3(256), 0, st,
                       packed, codes, N, K, counter);
    return hipGetLastError();
  }
  if (fmt == FMT_INT4) {
    const int64_t nwords = N * K / 8;
    hipLaunchKernelGGL(unpack_int4_kernel, dim3(grid_for(nwords, 256)), dim3(256), 0, st, (const uint32_t*)packed,
                       (uint8_t*)codes, nwords);
    return hipGetLastError();
  }
  int64_t nwords = N * K / (fmt == FMT_TERNARY ? 16 : 32);
  const int block = 256;
  if (fmt == FMT_TERNARY)
    hipLaunchKernelGGL(unpack_ternary_kernel, dim3(grid_for(nwords, block)), dim3(block), 0, st,
                       (const uint32_t*)packed, codes, nwords, counter);
  else
    hipLaunchKernelGGL(unpack_binary_kernel, dim3(grid_for(nwords, block)), dim3(block), 0, st,
                       (const uint32_t*)packed, codes, nwords);
  return hipGetLastError();
}

hipError_t launch_base3_to_int2(const uint8_t* base3, int64_t N, int64_t K, uint8_t* int2,
                                int32_t* counter, hipStream_t st) {
  if (counter) hipLaunchKernelGGL(zero_int_kernel, dim3(1), dim3(1), 0, st, counter);
  // 256 threads: one per table entry, four waves of 64 units per pass
  const int64_t units = N * ((K / 16 + 4) / 5);
  int64_t g = (units + 255) / 256;
  g = g < 1 ? 1 : (g > 65536 ? 65536 : g);
  hipLaunchKernelGGL(base3_to_int2_kernel, dim3((int)g), dim3(256), 0, st,
                     base3, (uint32_t*)int2, N, K, counter);
  return hipGetLastError();
}

}  // namespace lowbit
