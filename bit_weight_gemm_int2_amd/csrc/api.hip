// C ABI of the low-bit-weight GEMM library: argument validation, device
// checks, plan selection and launches on the caller's stream. See
// include/lowbit.h for the contract of every entry point.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdlib>
#include <algorithm>
#include <cstring>
#include <mutex>

#include "../../include/lowbit.h"
#include "common.h"

namespace lowbit {
hipError_t launch_pack(int fmt, const int8_t* codes, int64_t N, int64_t K, uint8_t* packed,
                       int32_t* counter, hipStream_t st);
hipError_t launch_unpack(int fmt, const uint8_t* packed, int64_t N, int64_t K, int8_t* codes,
                         int32_t* counter, hipStream_t st);
hipError_t launch_base3_to_int2(const uint8_t* base3, int64_t N, int64_t K, uint8_t* int2,
                                int32_t* counter, hipStream_t st);
hipError_t launch_gemm(int fmt, bool x_bf16, GemmArgs a, int num_cu, int variant, hipStream_t st,
                       const GemmGroup* group = nullptr, int count = 1);
hipError_t launch_gelu(const void* in, void* out, int dtype, int64_t count, hipStream_t st);
hipError_t launch_gemm_int4(bool x_bf16, GemmArgs a, int num_cu, int variant, hipStream_t st);
hipError_t launch_quantize(int fmt, const uint16_t* W, int64_t ldw, int64_t N, int64_t K, uint8_t* packed,
                           uint16_t* scales, int32_t* counter, int variant, hipStream_t st);
int64_t int4_rows(int64_t M);
size_t int4_workspace(int M, int N, int K, int num_cu, int variant);
size_t small_workspace_bytes(int M, int N, int K, int num_cu, int variant, int count = 1);
bool small_path(int M, int N, int K, int variant, int count = 1);
}  // namespace lowbit

namespace {

constexpr int kMaxDevices = 64;

struct DeviceInfo {
  std::atomic<int> state{0};   // 0 unknown, 1 ok, 2 not gfx950
  int num_cu = 0;
};
DeviceInfo g_dev[kMaxDevices];
std::mutex g_mu;

// Returns LOWBIT_OK and the CU count of the current device, or an error.
int32_t current_device(int* num_cu) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LOWBIT_ERR_DEVICE;
  DeviceInfo& d = g_dev[dev];
  int s = d.state.load(std::memory_order_acquire);
  if (s == 0) {
    std::lock_guard<std::mutex> lk(g_mu);
    s = d.state.load(std::memory_order_relaxed);
    if (s == 0) {
      hipDeviceProp_t prop;
      if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return LOWBIT_ERR_DEVICE;
      bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
      d.num_cu = prop.multiProcessorCount;
      s = ok ? 1 : 2;
      d.state.store(s, std::memory_order_release);
    }
  }
  if (s != 1) return LOWBIT_ERR_DEVICE;
  if (num_cu) *num_cu = d.num_cu;
  return LOWBIT_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// [p, p + bytes) and [q, q + qbytes) share a byte (empty ranges never do)
bool overlaps(const void* p, int64_t bytes, const void* q, int64_t qbytes) {
  if (!p || !q || bytes <= 0 || qbytes <= 0) return false;
  const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
  return a < b + (uintptr_t)qbytes && b < a + (uintptr_t)bytes;
}

// Kernel-family test hook: -1 for a name that is not one.
int parse_variant(const char* v) {
  if (!v || !*v || !std::strcmp(v, "auto")) return 0;
  if (!std::strcmp(v, "large")) return 1;
  if (!std::strcmp(v, "small")) return 2;
  if (!std::strcmp(v, "large-wide")) return 5;
  if (!std::strcmp(v, "large-pair")) return 6;
  if (!std::strcmp(v, "small-split")) return 7;
  if (!std::strcmp(v, "quant-eighth")) return 8;
  if (!std::strcmp(v, "quant-lane")) return 9;
  return -1;
}

// The forced kernel family: LOWBIT_FORCE_VARIANT, read once per process (an
// unknown name counts as unset), unless lowbit_debug_force_variant set it.
std::atomic<int> g_variant{0};
std::once_flag g_variant_once;

void read_variant_env() {
  std::call_once(g_variant_once, [] {
    const int v = parse_variant(std::getenv("LOWBIT_FORCE_VARIANT"));
    g_variant.store(v < 0 ? 0 : v, std::memory_order_relaxed);
  });
}

int force_variant() {
  read_variant_env();
  return g_variant.load(std::memory_order_relaxed);
}

// Scratch of the allocation-free entry point: one array per GPU, for the
// life of the process (split-K counters, then partial sums). Host code never
// uses the array's name as an address: each device's copy is looked up once
// with hipGetSymbolAddress, with that device current, and kept below.
static __device__ __align__(256) uint8_t scratch[LOWBIT_NOALLOC_SCRATCH_BYTES];

std::atomic<void*> g_scratch[kMaxDevices];

// The current device's scratch address (looked up on first use per device).
int32_t scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LOWBIT_ERR_DEVICE;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lk(g_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LOWBIT_ERR_HIP;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return LOWBIT_OK;
}

constexpr int64_t kMaxDim = (int64_t)1 << 31;
// largest operand byte span the kernels' 32-bit offsets cover (with room
// for the last 16-byte load)
constexpr int64_t kOffsetSpan = ((int64_t)1 << 32) - 64;

}  // namespace

extern "C" {

int32_t lowbit_abi_version(void) { return LOWBIT_ABI_VERSION; }

const char* lowbit_status_string(int32_t s) {
  switch (s) {
    case LOWBIT_OK: return "ok";
    case LOWBIT_ERR_NULL: return "a required pointer is NULL";
    case LOWBIT_ERR_SHAPE: return "bad shape (sizes must be >= 1 and < 2^31; K must follow the format rule)";
    case LOWBIT_ERR_ALIGN: return "misaligned pointer or leading dimension";
    case LOWBIT_ERR_DTYPE: return "unsupported dtype, format or activation";
    case LOWBIT_ERR_GROUP: return "unsupported group size (only 128)";
    case LOWBIT_ERR_WORKSPACE: return "workspace missing or too small";
    case LOWBIT_ERR_DEVICE: return "current device is not a gfx950 GPU";
    case LOWBIT_ERR_HIP: return "HIP runtime error";
    case LOWBIT_ERR_OVERLAP: return "an output overlaps an input or another output";
    default: return "unknown status";
  }
}

int32_t lowbit_init(void) {
  int32_t st = current_device(nullptr);
  if (st) return st;
  void* p = nullptr;
  return scratch_address(&p);
}

int32_t lowbit_debug_force_variant(const char* name) {
  const int v = parse_variant(name);
  if (v < 0) return LOWBIT_ERR_DTYPE;
  read_variant_env();
  g_variant.store(v, std::memory_order_relaxed);
  return LOWBIT_OK;
}

int64_t lowbit_packed_bytes(int32_t format, int64_t N, int64_t K) {
  if (N < 1 || K < 1 || N >= kMaxDim || K >= kMaxDim) return -1;
  if (format == LOWBIT_TERNARY_INT2) return K % 16 ? -1 : N * (K / 4);
  if (format == LOWBIT_BINARY_1BIT) return K % 32 ? -1 : N * (K / 8);
  if (format == LOWBIT_TERNARY_BASE3) return N * ((K + 4) / 5);
  if (format == LOWBIT_INT4_ZP) return K % 8 ? -1 : N * (K / 2);
  return -1;
}

int64_t lowbit_scale_count(int64_t N, int64_t K, int32_t group) {
  if (group != LOWBIT_GROUP || N < 1 || K < 1 || K % group) return -1;
  return N * (K / group);
}

static int kernel_format(int32_t format) {
  return format == LOWBIT_TERNARY_INT2 ? lowbit::FMT_TERNARY
       : format == LOWBIT_BINARY_1BIT  ? lowbit::FMT_BINARY
       : format == LOWBIT_INT4_ZP      ? lowbit::FMT_INT4
                                       : lowbit::FMT_BASE3;
}

static int32_t pack_common(int fmt, const int8_t* codes, int64_t N, int64_t K, uint8_t* packed,
                           int32_t* invalid_count, void* stream) {
  if (!codes || !packed) return LOWBIT_ERR_NULL;
  if (lowbit_packed_bytes(fmt, N, K) < 0) return LOWBIT_ERR_SHAPE;
  if (!aligned(codes, 16) || !aligned(packed, 16) || (invalid_count && !aligned(invalid_count, 4)))
    return LOWBIT_ERR_ALIGN;
  const int64_t pbytes = lowbit_packed_bytes(fmt, N, K);
  if (overlaps(packed, pbytes, codes, N * K) || overlaps(invalid_count, 4, codes, N * K) ||
      overlaps(invalid_count, 4, packed, pbytes))
    return LOWBIT_ERR_OVERLAP;
  int32_t st = current_device(nullptr);
  if (st) return st;
  hipError_t e = lowbit::launch_pack(kernel_format(fmt), codes, N, K, packed, invalid_count,
                                     (hipStream_t)stream);
  return e == hipSuccess ? LOWBIT_OK : LOWBIT_ERR_HIP;
}

int32_t pack_ternary(const int8_t* codes, int64_t N, int64_t K, uint8_t* packed,
                     int32_t* invalid_count, void* stream) {
  return pack_common(LOWBIT_TERNARY_INT2, codes, N, K, packed, invalid_count, stream);
}

int32_t pack_binary(const int8_t* codes, int64_t N, int64_t K, uint8_t* packed,
                    int32_t* invalid_count, void* stream) {
  return pack_common(LOWBIT_BINARY_1BIT, codes, N, K, packed, invalid_count, stream);
}

int32_t pack_base3(const int8_t* codes, int64_t N, int64_t K, uint8_t* packed,
                   int32_t* invalid_count, void* stream) {
  return pack_common(LOWBIT_TERNARY_BASE3, codes, N, K, packed, invalid_count, stream);
}

int32_t pack_int4(const uint8_t* codes, int64_t N, int64_t K, uint8_t* packed, int32_t* invalid_count,
                  void* stream) {
  return pack_common(LOWBIT_INT4_ZP, (const int8_t*)codes, N, K, packed, invalid_count, stream);
}

int32_t unpack_lowbit(int32_t format, const uint8_t* packed, int64_t N, int64_t K, int8_t* codes,
                      int32_t* invalid_count, void* stream) {
  if (format != LOWBIT_TERNARY_INT2 && format != LOWBIT_BINARY_1BIT && format != LOWBIT_TERNARY_BASE3 &&
      format != LOWBIT_INT4_ZP)
    return LOWBIT_ERR_DTYPE;
  if (!codes || !packed) return LOWBIT_ERR_NULL;
  if (lowbit_packed_bytes(format, N, K) < 0) return LOWBIT_ERR_SHAPE;
  if (!aligned(codes, 16) || !aligned(packed, 16) || (invalid_count && !aligned(invalid_count, 4)))
    return LOWBIT_ERR_ALIGN;
  const int64_t pbytes = lowbit_packed_bytes(format, N, K);
  if (overlaps(codes, N * K, packed, pbytes) || overlaps(invalid_count, 4, codes, N * K) ||
      overlaps(invalid_count, 4, packed, pbytes))
    return LOWBIT_ERR_OVERLAP;
  int32_t st = current_device(nullptr);
  if (st) return st;
  hipError_t e = lowbit::launch_unpack(kernel_format(format), packed, N, K, codes, invalid_count,
                                       (hipStream_t)stream);
  return e == hipSuccess ? LOWBIT_OK : LOWBIT_ERR_HIP;
}

int32_t lowbit_quantize(int32_t format, const void* W, int64_t N, int64_t K, int64_t ldw, uint8_t* packed,
                        void* scales, int32_t* nonfinite_count, void* stream) {
  if (format != LOWBIT_TERNARY_INT2 && format != LOWBIT_BINARY_1BIT) return LOWBIT_ERR_DTYPE;
  if (!W || !packed || !scales) return LOWBIT_ERR_NULL;
  if (N < 1 || K < LOWBIT_GROUP || N >= kMaxDim || K >= kMaxDim || K % LOWBIT_GROUP || ldw < K || ldw >= kMaxDim)
    return LOWBIT_ERR_SHAPE;
  if (!aligned(W, 16) || ldw % 8 || !aligned(packed, 16) || !aligned(scales, 2) ||
      (nonfinite_count && !aligned(nonfinite_count, 4)))
    return LOWBIT_ERR_ALIGN;
  const int64_t wbytes = ((N - 1) * ldw + K) * 2, pbytes = lowbit_packed_bytes(format, N, K),
                sbytes = N * (K / LOWBIT_GROUP) * 2;
  if (overlaps(packed, pbytes, W, wbytes) || overlaps(scales, sbytes, W, wbytes) ||
      overlaps(scales, sbytes, packed, pbytes) || overlaps(nonfinite_count, 4, W, wbytes) ||
      overlaps(nonfinite_count, 4, packed, pbytes) || overlaps(nonfinite_count, 4, scales, sbytes))
    return LOWBIT_ERR_OVERLAP;
  int32_t st = current_device(nullptr);
  if (st) return st;
  hipError_t e = lowbit::launch_quantize(kernel_format(format), (const uint16_t*)W, ldw, N, K, packed,
                                         (uint16_t*)scales, nonfinite_count, force_variant(), (hipStream_t)stream);
  return e == hipSuccess ? LOWBIT_OK : LOWBIT_ERR_HIP;
}

int32_t base3_to_int2(const uint8_t* base3, int64_t N, int64_t K, uint8_t* int2,
                      int32_t* invalid_count, void* stream) {
  if (!base3 || !int2) return LOWBIT_ERR_NULL;
  if (lowbit_packed_bytes(LOWBIT_TERNARY_INT2, N, K) < 0) return LOWBIT_ERR_SHAPE;
  if (!aligned(base3, 16) || !aligned(int2, 16) || (invalid_count && !aligned(invalid_count, 4)))
    return LOWBIT_ERR_ALIGN;
  const int64_t b3 = lowbit_packed_bytes(LOWBIT_TERNARY_BASE3, N, K), i2 = N * (K / 4);
  if (overlaps(int2, i2, base3, b3) || overlaps(invalid_count, 4, base3, b3) || overlaps(invalid_count, 4, int2, i2))
    return LOWBIT_ERR_OVERLAP;
  int32_t st = current_device(nullptr);
  if (st) return st;
  hipError_t e = lowbit::launch_base3_to_int2(base3, N, K, int2, invalid_count, (hipStream_t)stream);
  return e == hipSuccess ? LOWBIT_OK : LOWBIT_ERR_HIP;
}

size_t lowbit_gemm_workspace_bytes(int32_t format, int64_t M, int64_t N, int64_t K) {
  if (format != LOWBIT_TERNARY_INT2 && format != LOWBIT_BINARY_1BIT) return 0;
  if (M < 1 || N < 1 || K < 128 || K % 128 || M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return 0;
  int num_cu = 0;
  if (current_device(&num_cu)) return 0;
  if (!lowbit::small_path((int)M, (int)N, (int)K, force_variant())) return 0;
  return lowbit::small_workspace_bytes((int)M, (int)N, (int)K, num_cu, force_variant());
}

}  // extern "C"

namespace {

// Every host-side check of one problem of lowbit_gemm (all but the
// workspace and the device). On success *rows_max is the number of X rows
// whose offsets fit the kernels' 32-bit addressing.
int32_t check_problem(int32_t format, const void* X, int32_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                      const uint8_t* W_packed, const void* scales, int32_t group, int64_t N,
                      const void* bias, int32_t bias_dtype, void* Y, int32_t y_dtype, int64_t ldy,
                      int32_t activation, int64_t* rows_max) {
  if (format != LOWBIT_TERNARY_INT2 && format != LOWBIT_BINARY_1BIT) return LOWBIT_ERR_DTYPE;
  if (x_dtype != LOWBIT_F16 && x_dtype != LOWBIT_BF16) return LOWBIT_ERR_DTYPE;
  if (y_dtype != LOWBIT_F16 && y_dtype != LOWBIT_BF16 && y_dtype != LOWBIT_F32) return LOWBIT_ERR_DTYPE;
  if (bias_dtype != LOWBIT_NONE && bias_dtype != LOWBIT_F16 && bias_dtype != LOWBIT_BF16 &&
      bias_dtype != LOWBIT_F32)
    return LOWBIT_ERR_DTYPE;
  if (activation != LOWBIT_ACT_NONE && activation != LOWBIT_ACT_GELU_ERF) return LOWBIT_ERR_DTYPE;
  if (group != LOWBIT_GROUP) return LOWBIT_ERR_GROUP;
  if (!X || !W_packed || !scales || !Y) return LOWBIT_ERR_NULL;
  if ((bias == nullptr) != (bias_dtype == LOWBIT_NONE)) return bias ? LOWBIT_ERR_DTYPE : LOWBIT_ERR_NULL;
  if (M < 1 || N < 1 || K < 128 || K % 128 || M >= kMaxDim || N >= kMaxDim || K >= kMaxDim)
    return LOWBIT_ERR_SHAPE;
  if (ldx < K || ldy < N || ldx >= kMaxDim || ldy >= kMaxDim) return LOWBIT_ERR_SHAPE;
  // The kernels address the packed codes (and scales) of a column, and the
  // activations of a row, by 32-bit byte offsets from the operand's base:
  // the packed weights must span less than 4 GiB; X is taken in row chunks
  // whose offsets fit (below).
  const int64_t wrow = format == LOWBIT_TERNARY_INT2 ? K / 4 : K / 8;
  if (N * wrow > kOffsetSpan) return LOWBIT_ERR_SHAPE;
  *rows_max = (kOffsetSpan - 2 * K) / (2 * ldx) + 1;   // rows whose X offsets fit
  // a problem with M > 16 keeps every chunk above 16 rows (same kernels and
  // workspace as the whole problem)
  if (M > 16 && M > *rows_max && *rows_max < 34) return LOWBIT_ERR_SHAPE;
  const size_t ysz = y_dtype == LOWBIT_F32 ? 4 : 2;
  if (!aligned(X, 16) || !aligned(W_packed, 16) || !aligned(scales, 2) || !aligned(Y, ysz) || ldx % 8)
    return LOWBIT_ERR_ALIGN;
  if (bias && !aligned(bias, bias_dtype == LOWBIT_F32 ? 4 : 2)) return LOWBIT_ERR_ALIGN;
  const int64_t yb = ((M - 1) * ldy + N) * (int64_t)ysz;
  if (overlaps(Y, yb, X, ((M - 1) * ldx + K) * 2) || overlaps(Y, yb, W_packed, N * wrow) ||
      overlaps(Y, yb, scales, N * (K / 128) * 2) ||
      overlaps(Y, yb, bias, N * (bias_dtype == LOWBIT_F32 ? 4 : 2)))
    return LOWBIT_ERR_OVERLAP;
  return LOWBIT_OK;
}

// bytes of Y one problem addresses
int64_t y_span(int64_t M, int64_t N, int64_t ldy, int32_t y_dtype) {
  return ((M - 1) * ldy + N) * (y_dtype == LOWBIT_F32 ? 4 : 2);
}

// Does a workspace of `need` bytes share a byte with any operand of one
// problem? (The kernels write partial sums and counters into it.)
bool workspace_overlaps(const void* ws, size_t need, int32_t format, const void* X, int64_t M, int64_t K,
                        int64_t ldx, const uint8_t* W, const void* scales, int64_t N, const void* bias,
                        int32_t bias_dtype, const void* Y, int32_t y_dtype, int64_t ldy) {
  const int64_t n = (int64_t)need;
  const int64_t wrow = format == LOWBIT_TERNARY_INT2 ? K / 4 : K / 8;
  return overlaps(ws, n, Y, y_span(M, N, ldy, y_dtype)) || overlaps(ws, n, X, ((M - 1) * ldx + K) * 2) ||
         overlaps(ws, n, W, N * wrow) || overlaps(ws, n, scales, N * (K / 128) * 2) ||
         overlaps(ws, n, bias, N * (bias_dtype == LOWBIT_F32 ? 4 : 2));
}

lowbit::GemmArgs make_args(int32_t format, int64_t K, int64_t ldx, const uint8_t* W_packed, const void* scales,
                           int64_t N, const void* bias, int32_t bias_dtype, int32_t y_dtype, int64_t ldy,
                           int32_t activation, void* workspace) {
  lowbit::GemmArgs a{};
  a.ldx = ldx;
  a.W = W_packed;
  a.S = (const uint16_t*)scales;
  a.bias = bias;
  a.bias_dtype = bias_dtype;
  a.ldy = ldy;
  a.y_dtype = y_dtype;
  a.act = activation;
  a.N = (int)N;
  a.K = (int)K;
  a.ws = (float*)workspace;
  (void)format;
  return a;
}

// One problem, in one launch unless X spans 4 GiB or more; then equal row
// chunks, in order on the stream (they may share the workspace).
int32_t run_problem(int32_t format, const void* X, int32_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                    lowbit::GemmArgs a, void* Y, int32_t y_dtype, int64_t ldy, int64_t rows_max, int num_cu,
                    int variant, void* stream) {
  const size_t ysz = y_dtype == LOWBIT_F32 ? 4 : 2;
  const int64_t nchunks = M <= rows_max ? 1 : (M + rows_max - 1) / rows_max;
  const int64_t chunk = (M + nchunks - 1) / nchunks;
  for (int64_t m0 = 0; m0 < M; m0 += chunk) {
    a.X = (const uint16_t*)X + m0 * ldx;
    a.Y = (uint8_t*)Y + m0 * ldy * (int64_t)ysz;
    a.M = (int)std::min(chunk, M - m0);
    hipError_t e = lowbit::launch_gemm(format == LOWBIT_TERNARY_INT2 ? lowbit::FMT_TERNARY : lowbit::FMT_BINARY,
                                       x_dtype == LOWBIT_BF16, a, num_cu, variant, (hipStream_t)stream);
    if (e != hipSuccess) return LOWBIT_ERR_HIP;
  }
  return LOWBIT_OK;
}

}  // namespace

extern "C" {

int32_t lowbit_gemm(int32_t format, const void* X, int32_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                    const uint8_t* W_packed, const void* scales, int32_t group, int64_t N,
                    const void* bias, int32_t bias_dtype, void* Y, int32_t y_dtype, int64_t ldy,
                    int32_t activation, void* workspace, size_t workspace_bytes, void* stream) {
  int64_t rows_max = 0;
  int32_t st = check_problem(format, X, x_dtype, M, K, ldx, W_packed, scales, group, N, bias, bias_dtype, Y,
                             y_dtype, ldy, activation, &rows_max);
  if (st) return st;
  // the whole workspace the caller hands over is scratch: none of its bytes
  // may belong to an operand (checked before the device, whatever is needed)
  if (workspace && workspace_overlaps(workspace, workspace_bytes, format, X, M, K, ldx, W_packed, scales, N, bias,
                                      bias_dtype, Y, y_dtype, ldy))
    return LOWBIT_ERR_OVERLAP;
  int num_cu = 0;
  st = current_device(&num_cu);
  if (st) return st;
  size_t need = lowbit_gemm_workspace_bytes(format, M, N, K);
  if (need && (!workspace || workspace_bytes < need)) return LOWBIT_ERR_WORKSPACE;
  if (need && !aligned(workspace, 256)) return LOWBIT_ERR_ALIGN;
  const lowbit::GemmArgs a = make_args(format, K, ldx, W_packed, scales, N, bias, bias_dtype, y_dtype, ldy,
                                       activation, workspace);
  return run_problem(format, X, x_dtype, M, K, ldx, a, Y, y_dtype, ldy, rows_max, num_cu, force_variant(), stream);
}

int32_t lowbit_gemm_noalloc(int32_t format, const void* X, int32_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                            const uint8_t* W_packed, const void* scales, int32_t group, int64_t N,
                            const void* bias, int32_t bias_dtype, void* Y, int32_t y_dtype, int64_t ldy,
                            int32_t activation, void* stream) {
  int64_t rows_max = 0;
  int32_t st = check_problem(format, X, x_dtype, M, K, ldx, W_packed, scales, group, N, bias, bias_dtype, Y,
                             y_dtype, ldy, activation, &rows_max);
  if (st) return st;
  int num_cu = 0;
  st = current_device(&num_cu);
  if (st) return st;
  const size_t need = lowbit_gemm_workspace_bytes(format, M, N, K);
  if (need > LOWBIT_NOALLOC_SCRATCH_BYTES) return LOWBIT_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need) {
    st = scratch_address(&ws);
    if (st) return st;
  }
  const lowbit::GemmArgs a = make_args(format, K, ldx, W_packed, scales, N, bias, bias_dtype, y_dtype, ldy,
                                       activation, ws);
  return run_problem(format, X, x_dtype, M, K, ldx, a, Y, y_dtype, ldy, rows_max, num_cu, force_variant(), stream);
}

size_t lowbit_gemm_grouped_workspace_bytes(int32_t count, int32_t format, int64_t M, int64_t N, int64_t K) {
  if (count < 1 || count > LOWBIT_MAX_GROUP) return 0;
  const size_t one = lowbit_gemm_workspace_bytes(format, M, N, K);
  if (count == 1 || M > 16 || (format != LOWBIT_TERNARY_INT2 && format != LOWBIT_BINARY_1BIT)) return one;
  if (M < 1 || N < 1 || K < 128 || K % 128 || N >= kMaxDim || K >= kMaxDim) return 0;
  int num_cu = 0;
  if (current_device(&num_cu)) return 0;
  const int v = force_variant();
  const size_t grouped = lowbit::small_path((int)M, (int)N, (int)K, v, count)
                             ? lowbit::small_workspace_bytes((int)M, (int)N, (int)K, num_cu, v, count)
                             : 0;
  // the problems may also run one by one (activations of 4 GiB or more)
  return std::max(one, grouped);
}

int32_t lowbit_gemm_grouped(int32_t count, int32_t format, const void* const* X, int32_t x_dtype, int64_t M,
                            int64_t K, int64_t ldx, const uint8_t* const* W_packed, const void* const* scales,
                            int32_t group, int64_t N, const void* const* bias, int32_t bias_dtype,
                            void* const* Y, int32_t y_dtype, int64_t ldy, int32_t activation,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (count < 1 || count > LOWBIT_MAX_GROUP) return LOWBIT_ERR_SHAPE;
  if (!X || !W_packed || !scales || !Y) return LOWBIT_ERR_NULL;
  if (!bias && bias_dtype != LOWBIT_NONE) return LOWBIT_ERR_NULL;
  int64_t rows_max = 0;
  for (int z = 0; z < count; ++z) {
    int32_t st = check_problem(format, X[z], x_dtype, M, K, ldx, W_packed[z], scales[z], group, N,
                               bias ? bias[z] : nullptr, bias_dtype, Y[z], y_dtype, ldy, activation, &rows_max);
    if (st) return st;
  }
  // each output against every other problem's inputs and output
  const int64_t yb = y_span(M, N, ldy, y_dtype);
  const int64_t wrow = format == LOWBIT_TERNARY_INT2 ? K / 4 : K / 8;
  for (int z = 0; z < count; ++z)
    for (int u = 0; u < count; ++u) {
      if (u == z) continue;
      if (overlaps(Y[z], yb, Y[u], yb) || overlaps(Y[z], yb, X[u], ((M - 1) * ldx + K) * 2) ||
          overlaps(Y[z], yb, W_packed[u], N * wrow) || overlaps(Y[z], yb, scales[u], N * (K / 128) * 2) ||
          (bias && overlaps(Y[z], yb, bias[u], N * (bias_dtype == LOWBIT_F32 ? 4 : 2))))
        return LOWBIT_ERR_OVERLAP;
    }
  // the whole workspace is scratch: no byte of it may belong to any problem
  for (int z = 0; workspace && z < count; ++z)
    if (workspace_overlaps(workspace, workspace_bytes, format, X[z], M, K, ldx, W_packed[z], scales[z], N,
                           bias ? bias[z] : nullptr, bias_dtype, Y[z], y_dtype, ldy))
      return LOWBIT_ERR_OVERLAP;
  int num_cu = 0;
  int32_t st = current_device(&num_cu);
  if (st) return st;
  size_t need = lowbit_gemm_grouped_workspace_bytes(count, format, M, N, K);
  if (need && (!workspace || workspace_bytes < need)) return LOWBIT_ERR_WORKSPACE;
  if (need && !aligned(workspace, 256)) return LOWBIT_ERR_ALIGN;
  const int variant = force_variant();
  lowbit::GemmArgs a = make_args(format, K, ldx, W_packed[0], scales[0], N, bias ? bias[0] : nullptr, bias_dtype,
                                 y_dtype, ldy, activation, workspace);
  if (count == 1 || M > 16 || M > rows_max) {
    // one problem, large M (launches big enough on their own), or activations
    // that need row chunks: one problem after the other on the stream
    for (int z = 0; z < count; ++z) {
      a.W = W_packed[z];
      a.S = (const uint16_t*)scales[z];
      a.bias = bias ? bias[z] : nullptr;
      st = run_problem(format, X[z], x_dtype, M, K, ldx, a, Y[z], y_dtype, ldy, rows_max, num_cu, variant, stream);
      if (st) return st;
    }
    return LOWBIT_OK;
  }
  lowbit::GemmGroup g{};
  for (int z = 0; z < count; ++z) {
    g.X[z] = (const uint16_t*)X[z];
    g.W[z] = W_packed[z];
    g.S[z] = (const uint16_t*)scales[z];
    g.bias[z] = bias ? bias[z] : nullptr;
    g.Y[z] = Y[z];
  }
  a.X = g.X[0];
  a.Y = g.Y[0];
  a.M = (int)M;
  hipError_t e = lowbit::launch_gemm(format == LOWBIT_TERNARY_INT2 ? lowbit::FMT_TERNARY : lowbit::FMT_BINARY,
                                     x_dtype == LOWBIT_BF16, a, num_cu, variant, (hipStream_t)stream, &g, count);
  return e == hipSuccess ? LOWBIT_OK : LOWBIT_ERR_HIP;
}

size_t lowbit_gemm_int4_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < 128 || K % 128 || M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return 0;
  int num_cu = 0;
  if (current_device(&num_cu) != LOWBIT_OK) num_cu = 256;   // no gfx950 device: the MI355X's count
  return lowbit::int4_workspace((int)M, (int)N, (int)K, num_cu, force_variant());
}

int32_t lowbit_gemm_int4(const void* X, int32_t x_dtype, int64_t M, int64_t K, int64_t ldx, const uint8_t* W_packed,
                         const void* scales, const void* zeros, int32_t group, int64_t N, const void* bias,
                         int32_t bias_dtype, void* Y, int32_t y_dtype, int64_t ldy, int32_t activation,
                         void* workspace, size_t workspace_bytes, void* stream) {
  // every check of lowbit_gemm (its packed-size rules read for K/2 bytes a row)
  if (!zeros) return LOWBIT_ERR_NULL;
  int64_t rows_max = 0;
  int32_t st = check_problem(LOWBIT_TERNARY_INT2, X, x_dtype, M, K, ldx, W_packed, scales, group, N, bias,
                             bias_dtype, Y, y_dtype, ldy, activation, &rows_max);
  if (st) return st;
  if (N * (K / 2) > kOffsetSpan || M > rows_max) return LOWBIT_ERR_SHAPE;
  if (!aligned(zeros, 2)) return LOWBIT_ERR_ALIGN;
  const int64_t yb = y_span(M, N, ldy, y_dtype), sb = N * (K / 128) * 2;
  if (overlaps(Y, yb, W_packed, N * (K / 2)) || overlaps(Y, yb, zeros, sb)) return LOWBIT_ERR_OVERLAP;
  const size_t need = lowbit_gemm_int4_workspace_bytes(M, N, K);
  if (!workspace || workspace_bytes < need) return LOWBIT_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return LOWBIT_ERR_ALIGN;
  const int64_t wn = (int64_t)workspace_bytes;
  if (overlaps(workspace, wn, Y, yb) || overlaps(workspace, wn, X, ((M - 1) * ldx + K) * 2) ||
      overlaps(workspace, wn, W_packed, N * (K / 2)) || overlaps(workspace, wn, scales, sb) ||
      overlaps(workspace, wn, zeros, sb) || overlaps(workspace, wn, bias, N * (bias_dtype == LOWBIT_F32 ? 4 : 2)))
    return LOWBIT_ERR_OVERLAP;
  int num_cu = 0;
  st = current_device(&num_cu);
  if (st) return st;
  lowbit::GemmArgs a = make_args(LOWBIT_INT4_ZP, K, ldx, W_packed, scales, N, bias, bias_dtype, y_dtype, ldy,
                                 activation, workspace);
  a.X = (const uint16_t*)X;
  a.Y = Y;
  a.M = (int)M;
  a.Z = (const uint16_t*)zeros;
  a.ldr = lowbit::int4_rows(M);
  hipError_t e = lowbit::launch_gemm_int4(x_dtype == LOWBIT_BF16, a, num_cu, force_variant(), (hipStream_t)stream);
  return e == hipSuccess ? LOWBIT_OK : LOWBIT_ERR_HIP;
}

int32_t lowbit_gelu(const void* in, void* out, int32_t dtype, int64_t count, void* stream) {
  if (!in || !out) return LOWBIT_ERR_NULL;
  if (dtype != LOWBIT_F16 && dtype != LOWBIT_BF16 && dtype != LOWBIT_F32) return LOWBIT_ERR_DTYPE;
  if (count < 1) return LOWBIT_ERR_SHAPE;
  if (!aligned(in, 16) || !aligned(out, 16)) return LOWBIT_ERR_ALIGN;
  const int64_t bytes = count * (dtype == LOWBIT_F32 ? 4 : 2);
  if (in != out && overlaps(in, bytes, out, bytes)) return LOWBIT_ERR_OVERLAP;
  int32_t st = current_device(nullptr);
  if (st) return st;
  hipError_t e = lowbit::launch_gelu(in, out, dtype, count, (hipStream_t)stream);
  return e == hipSuccess ? LOWBIT_OK : LOWBIT_ERR_HIP;
}

}  // extern "C"
