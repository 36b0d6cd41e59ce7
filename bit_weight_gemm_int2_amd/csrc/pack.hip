// INT2 / 1-bit weight packers and the unpacker (load-time kernels).
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

__global__ void zero_int_kernel(int32_t* p) { *p = 0; }

static int grid_for(int64_t work, int block) {
  int64_t g = (work + block - 1) / block;
  if (g > 65536) g = 65536;
  return (int)(g < 1 ? 1 : g);
}

hipError_t launch_pack(int fmt, const int8_t* codes, int64_t N, int64_t K, uint8_t* packed,
                       int32_t* counter, hipStream_t st) {
  if (counter) hipLaunchKernelGGL(zero_int_kernel, dim3(1), dim3(1), 0, st, counter);
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

}  // namespace lowbit
