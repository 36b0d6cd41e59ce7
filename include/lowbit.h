/*
 * lowbit.h - C ABI of the MI355X (gfx950) low-bit-weight linear layer.
 *
 * The layer is the one the Bonsai Image 4B pages describe for the diffusion
 * transformer: every weight is w = scale_g * t, with t in {-1, 0, +1}
 * (ternary, stored with 2 bits per value, "INT2") or t in {-1, +1} (binary,
 * 1 bit per value), and one FP16 scale shared by each group of 128 weights
 * ("Como Bonsai Ternary 4B revoluciona la difusion texto-imagen", section
 * "Representacion y almacenamiento de los pesos ternarios"; "Bonsai Image 4B
 * 1-bit untuk pembuatan gambar di perangkat lokal", section on the two
 * variants). Activations are FP16 or BF16.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every data pointer is a DEVICE pointer owned by the caller. The library
 *    never allocates, frees or synchronises; work is enqueued on `stream`
 *    (a hipStream_t; NULL means the null stream) and runs asynchronously.
 *  - The return value reports argument errors (checked on the host before any
 *    launch) and launch errors (hipGetLastError after the launch). Errors
 *    that happen later on the device surface at the caller's next
 *    synchronisation, as for any HIP kernel.
 *  - Outputs may not overlap inputs (or, for lowbit_gemm_grouped, each other):
 *    the byte ranges each call addresses are compared on the host and an
 *    overlap returns LOWBIT_ERR_OVERLAP (lowbit_gelu alone may run in place,
 *    with in == out exactly).
 *  - Matrices are row-major. Sizes are element counts unless stated.
 *  - The library runs on gfx950 only; other devices get LOWBIT_ERR_DEVICE.
 *  - Every call is stateless apart from a per-device cache of device
 *    properties, and is safe to call from several host threads.
 *  - Test hook: lowbit_debug_force_variant (below) forces one kernel family
 *    so that tests reach every launch path; the environment variable
 *    LOWBIT_FORCE_VARIANT, read once per process, sets its initial value.
 *
 * Packed weight layout (this library's own; the pages fix only "2 bits per
 * ternary" and "1 bit per binary weight")
 * ---------------------------------------------------------------------------
 *  A packed matrix has N rows; row n is a run of little-endian 32-bit words
 *  along K, rows stored back to back (row stride K/4 bytes ternary, K/8
 *  bytes binary).
 *  Ternary: the code of t is its 2-bit two's complement (0 -> 00, +1 -> 01,
 *    -1 -> 11; 10 is invalid). Word u of a row holds
 *    k = 16u .. 16u+15; the code of k = 16u + 2i + h (i = 0..7, h = 0/1) sits
 *    at bits [16h + 2i, 16h + 2i + 1]: even k fill the low half word, odd k
 *    the high half word.
 *  Binary: bit b = 1 means t = +1, 0 means t = -1. Word u holds
 *    k = 32u .. 32u+31; the bit of k = 32u + 2i + h (i = 0..15) sits at
 *    bit 16h + i.
 *  Base-3 (storage and transport only; lowbit_gemm reads INT2): five ternary
 *    values per byte. Digit d = t + 1; byte j of a row holds k = 5j .. 5j+4 as
 *    sum_i d[5j+i] * 3^i (the lowest k is the least significant digit). A row
 *    is ceil(K/5) bytes with no padding to a word, rows back to back; the last
 *    byte of a row holds the K mod 5 leftover values when K mod 5 != 0. Bytes
 *    243 .. 255 are invalid. 1.6 bits per value, the nearest byte-aligned rate
 *    to the log2(3) ~ 1.585 bits the pages price a ternary value at.
 *  4-bit with a zero point (the text encoder's format; lowbit_gemm_int4):
 *    an unsigned code q in 0..15 per weight, w = s * (q - z) with an FP16
 *    scale s and an FP16 zero point z per group of 128 along K. Word u of a
 *    row holds k = 8u .. 8u+7; the code of k = 8u + 2i + h (i = 0..3,
 *    h = 0/1) sits at bits [16h + 4i, 16h + 4i + 3]. Row stride K/2 bytes.
 *  Scales: FP16, shape [N, K/128], row-major; scale[n, g] covers
 *    k = 128g .. 128g+127 of output row n. Any finite value is allowed
 *    (zero and subnormal included); non-finite scales give unspecified results.
 */
#ifndef LOWBIT_H
#define LOWBIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LOWBIT_ABI_VERSION 1
#define LOWBIT_GROUP 128
#define LOWBIT_MAX_GROUP 8   /* problems per lowbit_gemm_grouped call */
/* Scratch that lowbit_gemm_noalloc keeps on each GPU: 16 MiB + 64 KiB. */
#define LOWBIT_NOALLOC_SCRATCH_BYTES ((16u << 20) + (64u << 10))

typedef enum {
  LOWBIT_OK = 0,
  LOWBIT_ERR_NULL = 1,       /* a required pointer is NULL                      */
  LOWBIT_ERR_SHAPE = 2,      /* a size is < 1, too large, or K breaks its rule  */
  LOWBIT_ERR_ALIGN = 3,      /* a pointer or leading dimension breaks alignment */
  LOWBIT_ERR_DTYPE = 4,      /* unsupported dtype / format / activation code    */
  LOWBIT_ERR_GROUP = 5,      /* group size other than 128                       */
  LOWBIT_ERR_WORKSPACE = 6,  /* workspace missing or smaller than required      */
  LOWBIT_ERR_DEVICE = 7,     /* current device is not gfx950, or no device      */
  LOWBIT_ERR_HIP = 8,        /* the HIP runtime reported an error               */
  LOWBIT_ERR_OVERLAP = 9     /* an output's bytes overlap an input's or another output's */
} lowbit_status;

typedef enum { LOWBIT_F16 = 0, LOWBIT_BF16 = 1, LOWBIT_F32 = 2, LOWBIT_NONE = 3 } lowbit_dtype;
typedef enum { LOWBIT_BINARY_1BIT = 1, LOWBIT_TERNARY_INT2 = 2, LOWBIT_TERNARY_BASE3 = 3,
               LOWBIT_INT4_ZP = 4 } lowbit_format;
typedef enum { LOWBIT_ACT_NONE = 0, LOWBIT_ACT_GELU_ERF = 1 } lowbit_activation;

/* ABI version of the loaded library (LOWBIT_ABI_VERSION). */
int32_t lowbit_abi_version(void);

/* Human-readable text for a status code; never NULL, static storage. */
const char* lowbit_status_string(int32_t status);

/* Check that the current device is gfx950 and cache its properties.
 * Optional: every entry point does the same on first use. */
int32_t lowbit_init(void);

/* Test hook, for tests only: force one kernel family for every later call of
 * the process (all threads), so that tests reach every launch path on the
 * same shapes. name: "auto" or NULL (the automatic choice), "large" (the
 * large-M kernel at any M), "small" (the small-M kernels only), "large-wide"
 * / "large-pair" (one large-M tile configuration; for lowbit_gemm_int4 its
 * 128-row or its 64-row tiles; "small-split" its 64-row tiles with the
 * largest K split the groups allow), "small-split" (the
 * small-M column-tile kernel with its K split across workgroups),
 * "quant-eighth" / "quant-lane" (lowbit_quantize, ternary: eight lanes per
 * 128-weight group, or one lane per group, instead of the automatic two). Results keep the same accuracy contract (bit-identical
 * for lowbit_quantize) under every variant, and the workspace queries
 * follow it. The initial value comes from the environment variable
 * LOWBIT_FORCE_VARIANT, read once. Returns LOWBIT_ERR_DTYPE for an unknown
 * name (the setting is then unchanged). Not for concurrent use with calls on
 * other threads that depend on the automatic choice. */
int32_t lowbit_debug_force_variant(const char* name);

/* Bytes of packed codes for an N x K matrix: N*K/4 (ternary), N*K/8 (binary),
 * N*ceil(K/5) (base-3), N*K/2 (4-bit); -1 for a bad format or a K that
 * breaks the packing rule (ternary K % 16, binary K % 32, 4-bit K % 8) or
 * N, K < 1 or >= 2^31. */
int64_t lowbit_packed_bytes(int32_t format, int64_t N, int64_t K);

/* Number of FP16 scales, N * K / group; -1 if group != 128 or K % group != 0. */
int64_t lowbit_scale_count(int64_t N, int64_t K, int32_t group);

/* Pack int8 ternary codes t[N][K] in {-1,0,+1} into the INT2 layout above
 * (the 2-bit storage of "Representacion y almacenamiento de los pesos
 * ternarios"). codes: N*K bytes, 16-byte aligned. packed: N*K/4 bytes,
 * 16-byte aligned, must not overlap codes. K % 16 == 0.
 * invalid_count (nullable, device int32, 4-byte aligned): set to the number
 * of input bytes outside {-1,0,+1}; such values are packed as code 00 (t = 0).
 * Output bytes are a pure function of the input: bit-identical on every run. */
int32_t pack_ternary(const int8_t* codes, int64_t N, int64_t K, uint8_t* packed,
                     int32_t* invalid_count, void* stream);

/* Pack int8 binary codes t[N][K] in {-1,+1} into the 1-bit layout above
 * (1 bit per binary weight: "Bonsai Image 4B 1-bit untuk pembuatan gambar di
 * perangkat lokal", section on the two variants; the 1.125-bit arithmetic of
 * "Introducing 1-bit and Ternary Bonsai Image 4B", section on the quantisation
 * arithmetic). packed: N*K/8 bytes. K % 32 == 0.
 * Values other than -1/+1 are counted in invalid_count and packed as bit 0
 * (t = -1). Alignment and ownership as pack_ternary. */
int32_t pack_binary(const int8_t* codes, int64_t N, int64_t K, uint8_t* packed,
                    int32_t* invalid_count, void* stream);

/* Pack int8 ternary codes t[N][K] in {-1,0,+1} into the base-3 layout above
 * (five values per byte: the storage that comes nearest the log2(3)-bit
 * information rate of "Representacion y almacenamiento de los pesos
 * ternarios" and of the quantisation arithmetic on the "Introducing 1-bit and
 * Ternary Bonsai Image 4B" page). packed: N*ceil(K/5) bytes, must not overlap
 * codes. Any K >= 1. Values outside {-1,0,+1} are counted in invalid_count
 * and stored as t = 0. Alignment and ownership as pack_ternary. */
int32_t pack_base3(const int8_t* codes, int64_t N, int64_t K, uint8_t* packed,
                   int32_t* invalid_count, void* stream);

/* Pack 4-bit codes q[N][K] (uint8 values 0..15) into the 4-bit layout above
 * (the 4-bit group-quantised weights of the pipeline's text encoder, "Como
 * Bonsai Ternary 4B revoluciona la difusion texto-imagen", section
 * "Arquitectura de despliegue y eficiencia en tiempo de ejecucion"; the
 * layout is this library's own). packed: N*K/2 bytes. K % 8 == 0. Values
 * above 15 are counted in invalid_count and stored as 0. Alignment and
 * ownership as pack_ternary. */
int32_t pack_int4(const uint8_t* codes, int64_t N, int64_t K, uint8_t* packed,
                  int32_t* invalid_count, void* stream);

/* Quantise dense FP16 weights into packed codes and FP16 group scales, the
 * load-time step that makes (t, s) from trained weights. The pages name the
 * two lines of work the variants come from, BinaryConnect and Ternary Weight
 * Networks ("cuantificacion de modelos de difusion para inferencia local en
 * dispositivos edge", section "Fundamentos Teoricos"), with one FP16 scale per
 * group of 128 ("Representacion y almacenamiento de los pesos ternarios"), but
 * not the procedure; this library applies those two rules to each group of
 * 128 weights along K of each row:
 *   LOWBIT_TERNARY_INT2: a weight is kept when |w| > 0.7 * mean|w| of its
 *     group; t = sign(w) when kept, else 0; s = mean of the kept |w| (0 when
 *     none is kept);
 *   LOWBIT_BINARY_1BIT: t = +1 when w >= 0 (-0.0 included), else -1;
 *     s = mean|w| of the group;
 * with s the FP16 value nearest the exact mean (ties to even). Every decision
 * is exact, so the output is a pure function of the input: bit-identical on
 * every run and device.
 *   W        FP16 [N][ldw], the first K columns of each row are the weights;
 *            16-byte aligned, K <= ldw < 2^31, ldw % 8 == 0
 *   packed   [N][K/4] (ternary) or [N][K/8] (binary) bytes in the packed
 *            layout above, 16-byte aligned
 *   scales   FP16 [N][K/128], 2-byte aligned
 *   nonfinite_count  nullable device int32 (4-byte aligned): set to the
 *            number of NaN or infinite weights, which act as +0.0
 *   N, K     N >= 1; K >= 128, K % 128 == 0; both < 2^31
 * No output may overlap W or another output (LOWBIT_ERR_OVERLAP); other
 * formats give LOWBIT_ERR_DTYPE. */
int32_t lowbit_quantize(int32_t format, const void* W, int64_t N, int64_t K, int64_t ldw,
                        uint8_t* packed, void* scales, int32_t* nonfinite_count, void* stream);

/* Inverse of the packers: packed (format layout above) -> int8 codes[N][K]
 * (for LOWBIT_INT4_ZP the codes are the unsigned values 0..15).
 * Ternary code 10 and base-3 bytes 243 .. 255 are invalid: their values
 * decode to 0 and are counted, one per value, in invalid_count (nullable).
 * Binary has no invalid pattern (count set to 0). codes and packed are
 * 16-byte aligned and do not overlap. */
int32_t unpack_lowbit(int32_t format, const uint8_t* packed, int64_t N, int64_t K,
                      int8_t* codes, int32_t* invalid_count, void* stream);

/* Load-time transcoding of base-3 codes [N rows of ceil(K/5) bytes] into the
 * INT2 layout [N*K/4 bytes] that lowbit_gemm reads, on the device, so that
 * weights can be stored and moved at 1.6 bits per value and computed on at
 * 2. K % 16 == 0 (the INT2 rule). base3 and int2 are 16-byte aligned and do
 * not overlap. The values of an invalid base-3 byte become the invalid INT2
 * pattern 10 (which lowbit_gemm reads as t = 0 and unpack_lowbit counts) and
 * are counted in invalid_count (nullable, one per value). The output is a
 * pure function of the input. */
int32_t base3_to_int2(const uint8_t* base3, int64_t N, int64_t K, uint8_t* int2,
                      int32_t* invalid_count, void* stream);

/* Workspace bytes lowbit_gemm needs for this problem (0 when none). Depends
 * only on (format, M, N, K) and the current device. Non-zero only for
 * M <= 16 when K is split across workgroups: a fixed 64 KiB region of
 * 32-bit counters, one per column tile, followed by the FP32 partial sums. */
size_t lowbit_gemm_workspace_bytes(int32_t format, int64_t M, int64_t N, int64_t K);

/* The low-bit linear layer (w = scale_g * t from "Representacion y
 * almacenamiento de los pesos ternarios", applied as Y = X W^T):
 *
 *   Y[m, n] = act( sum_k X[m, k] * float(scales[n, k/128]) * t[n, k] + bias[n] )
 *
 * with FP32 accumulation, then one round-to-nearest-even cast to y_dtype.
 * Accuracy contract per element: |Y - exact| <= 1e-3 * (sum_k |x_k w_k| +
 * |bias|) + 1e-5, plus half an output ulp for FP16/BF16 outputs (before the
 * activation; GELU is then applied to the FP32 value). Range limit: the
 * kernels accumulate each 128-group's sum of x * (2t) in FP32 and rescale
 * between groups by ratios of the group scales, so the contract holds while
 * 2 * sum_k |x_k| * max_g |s_g| / min_g |s_g| (over a row's nonzero scales)
 * stays below about 2^100; FP16 activations always do, BF16 activations of
 * magnitude near 2^120 with scales spread by 2^30 could overflow to inf
 * where the exact result is finite.
 *
 *   format      LOWBIT_TERNARY_INT2 or LOWBIT_BINARY_1BIT (base-3 weights
 *               are transcoded first with base3_to_int2; LOWBIT_TERNARY_BASE3
 *               here gives LOWBIT_ERR_DTYPE)
 *   X           [M][ldx] of x_dtype (LOWBIT_F16 or LOWBIT_BF16); 16-byte
 *               aligned, K <= ldx < 2^31, ldx % 8 == 0. When X spans 4 GiB
 *               or more ((M-1)*ldx*2 + 2K bytes) it is processed in equal row
 *               chunks that span less, one launch each, in order on the
 *               stream; for M > 16 the chunks must stay above 16 rows
 *               (ldx below about 2^27), else LOWBIT_ERR_SHAPE
 *   W_packed    [N][K/4] or [N][K/8] bytes in the packed layout, 16-byte
 *               aligned, spanning less than 4 GiB (N*K/4 or N*K/8 bytes),
 *               else LOWBIT_ERR_SHAPE
 *   scales      FP16 [N][K/group], 2-byte aligned; group must be 128
 *   bias        nullable; [N] of bias_dtype (F16, BF16, F32), or
 *               bias_dtype = LOWBIT_NONE with bias = NULL
 *   Y           [M][ldy] of y_dtype (F16, BF16, F32); aligned to its element
 *               size, N <= ldy < 2^31; must not overlap X, W, scales, bias
 *   activation  LOWBIT_ACT_NONE or LOWBIT_ACT_GELU_ERF (x * Phi(x), exact erf)
 *   workspace   device scratch of at least lowbit_gemm_workspace_bytes(),
 *               256-byte aligned; may be NULL when that is 0. Its bytes must
 *               be zero before the first call that uses it (allocate it
 *               zeroed); every call leaves the counters it used at zero
 *               again, so it can be reused without clearing. Calls that can
 *               run concurrently (other streams) must not share it. None of
 *               its workspace_bytes bytes may belong to X, W, scales, bias or
 *               Y (LOWBIT_ERR_OVERLAP, checked for any non-NULL workspace)
 *   M, N, K     M, N >= 1; K >= 128 and K % 128 == 0; M, N, K < 2^31
 *
 * Ternary codes 10 are not checked here (hot path); they act as t = 0.
 * The result is deterministic: the same inputs give the same bits on every
 * call on the same device (partial sums are combined in a fixed order). */
int32_t lowbit_gemm(int32_t format,
                    const void* X, int32_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                    const uint8_t* W_packed, const void* scales, int32_t group, int64_t N,
                    const void* bias, int32_t bias_dtype,
                    void* Y, int32_t y_dtype, int64_t ldy,
                    int32_t activation,
                    void* workspace, size_t workspace_bytes,
                    void* stream);

/* lowbit_gemm with no workspace argument, for callers that cannot allocate
 * device memory around a call: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. Same arguments (less workspace and
 * workspace_bytes), same result bits and the same accuracy contract as
 * lowbit_gemm. Where lowbit_gemm needs a workspace (M <= 16 with K split
 * across workgroups), this entry point uses a scratch array of the library
 * instead: LOWBIT_NOALLOC_SCRATCH_BYTES of device memory per GPU, held from
 * the first call (or lowbit_init) on that GPU until the process ends. A
 * problem that needs more than that returns LOWBIT_ERR_WORKSPACE. It calls
 * no allocating routine. Every call on one GPU shares that GPU's scratch:
 * calls that can overlap on one GPU (other streams, other host threads'
 * streams) race on it and give wrong results; serialise them on one stream.
 * Its counters start at zero and every call leaves them at zero. */
int32_t lowbit_gemm_noalloc(int32_t format,
                            const void* X, int32_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                            const uint8_t* W_packed, const void* scales, int32_t group, int64_t N,
                            const void* bias, int32_t bias_dtype,
                            void* Y, int32_t y_dtype, int64_t ldy,
                            int32_t activation, void* stream);

/* Workspace bytes lowbit_gemm_int4 needs (0 for a bad shape): the per-group
 * row sums of X, K/128 x (M rounded up to 128, plus 128) FP32 values, and,
 * when the launch splits K across workgroups (small grids: few tiles, long
 * K), from the next 256-byte boundary, splits x M x N FP32 partial sums.
 * Depends on (M, N, K) and the current device's CU count (256 is assumed
 * when no gfx950 device is current). */
size_t lowbit_gemm_int4_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* The 4-bit group-quantised linear (any M), with a zero point per group:
 *
 *   Y[m, n] = act( sum_k X[m, k] * s[n, k/128] * (q[n, k] - z[n, k/128]) + bias[n] )
 *
 * with FP32 accumulation and one RNE cast, for the text encoder's 4-bit
 * weights ("Como Bonsai Ternary 4B revoluciona la difusion texto-imagen",
 * section "Arquitectura de despliegue y eficiencia en tiempo de ejecucion").
 * Arguments as lowbit_gemm, with W_packed in the 4-bit layout ([N][K/2]
 * bytes), `zeros` FP16 [N][K/128] (2-byte aligned, finite) beside `scales`,
 * and a workspace of lowbit_gemm_int4_workspace_bytes (256-byte aligned;
 * its contents need no initialisation and are overwritten; calls that can
 * run concurrently must not share it). X must span less than 4 GiB.
 * Accuracy contract per element: |Y - exact| <= 1e-3 * sum_k |x_k w_k| + 1e-5
 * + 2^-19 * (128 + max|z|) * sum_k |x_k s_k| (plus half an output ulp for
 * FP16/BF16 outputs): the kernel accumulates sum x (128 + q) and takes
 * (128 + z) times the group's activation sum off it, so the FP32 roundings
 * of those two sums add the last term, which matters only when |q - z| is
 * small against 128. Deterministic. */
int32_t lowbit_gemm_int4(const void* X, int32_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                         const uint8_t* W_packed, const void* scales, const void* zeros, int32_t group,
                         int64_t N, const void* bias, int32_t bias_dtype,
                         void* Y, int32_t y_dtype, int64_t ldy, int32_t activation,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Several independent linears of one shape in one launch: problem z computes
 *
 *   Y[z] = act( X[z] W[z]^T + bias[z] )
 *
 * exactly as lowbit_gemm would (same accuracy contract and determinism), for
 * z = 0 .. count-1, 1 <= count <= LOWBIT_MAX_GROUP. Every problem shares
 * format, dtypes, activation, M, N, K, group, ldx and ldy; X, W_packed,
 * scales and Y are HOST arrays of count device pointers (each meeting the
 * rules of lowbit_gemm), and bias is NULL (no bias, bias_dtype
 * LOWBIT_NONE) or a host array of count device pointers. No Y may overlap
 * another Y or any input.
 *
 * The reason is launch count at small M: the double-stream blocks of the
 * transformer ("Arquitectura de despliegue y eficiencia en tiempo de
 * ejecucion": 5 double-stream and 20 single-stream blocks) run the same
 * linears on an image and a text stream, independent of each other, and at
 * M <= 16 each launch is bound by its own latency rather than by bytes. For
 * M <= 16 the problems run as one launch of the small-M kernels, planned over
 * the column tiles of all of them. For M > 16 (launches big enough on their
 * own), or activations that lowbit_gemm would split into row chunks, they
 * run one after the other on the stream.
 * workspace: lowbit_gemm_grouped_workspace_bytes(count, format, M, N, K)
 * bytes, with the rules of lowbit_gemm's workspace. */
int32_t lowbit_gemm_grouped(int32_t count, int32_t format,
                            const void* const* X, int32_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                            const uint8_t* const* W_packed, const void* const* scales, int32_t group,
                            int64_t N, const void* const* bias, int32_t bias_dtype,
                            void* const* Y, int32_t y_dtype, int64_t ldy,
                            int32_t activation,
                            void* workspace, size_t workspace_bytes,
                            void* stream);

/* Workspace bytes lowbit_gemm_grouped needs (0 when none); 0 as well for a
 * count outside 1 .. LOWBIT_MAX_GROUP. */
size_t lowbit_gemm_grouped_workspace_bytes(int32_t count, int32_t format, int64_t M, int64_t N, int64_t K);

/* Exact-erf GELU, y = x * Phi(x), computed in FP32, elementwise over `count`
 * values of `dtype` (F16, BF16 or F32); in and out may be the same buffer and
 * must be 16-byte aligned. The activation the 1024x1024 MLP pair applies
 * between its two linears when it is not fused into the first one. */
int32_t lowbit_gelu(const void* in, void* out, int32_t dtype, int64_t count, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* LOWBIT_H */
