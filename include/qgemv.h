/*
 * qgemv.h — C ABI of the MI355X (gfx950) fused dequantise + GEMV library.
 *
 * Every GEMV call computes, for ONE activation row,
 *     v[r] = sum_{i<K} x[i] * dequant(W)[r][i]        r = 0 .. M-1
 * i.e. v = x . dequant(W)^T ("Writing a high performant GEMV + dequant for
 * Metal", section "What is a GEMV").  The plain calls store y = v in fp32
 * (alpha = 1, beta = 0); the _ex calls apply the general output stage
 * y = alpha v + beta c in fp32, fp16 or bf16.  The row calls materialise rows
 * of dequant(W) as fp32, fp16 or bf16.
 *
 * Conventions shared by every entry point
 *   M       number of rows of W = number of outputs (the batch is always 1).
 *   K       reduction length (elements per row of W and of x).
 *   Layout  W is row-major with K contiguous, in the format's packed blocks;
 *           x is K contiguous 16-bit values; y is M contiguous values;
 *           materialised rows are contiguous and row-major.
 *   Memory  every pointer is DEVICE memory owned by the caller (e.g. torch
 *           tensors).  The library allocates nothing, keeps no per-call state
 *           and never synchronises.  y must not overlap x or W.
 *   Stream  work is enqueued on `stream` (NULL = the null stream) and returns
 *           immediately; results are visible once the stream has run it.
 *   Errors  arguments are validated in host code before any HIP call; a bad
 *           argument returns a negative QGEMV_E_* code and enqueues nothing.
 *           A failed launch returns QGEMV_E_HIP.  The library never prints or
 *           aborts.  M == 0 is a successful no-op.
 *   Alignment  W, x and materialised rows must be 16-byte aligned; y and c
 *              to their element size.
 *   Limits     M <= 2^31 - 1 and K <= 2^24 (the dense GEMV: K <= 65536; the
 *              prefill calls: K <= 2^20); larger sizes return QGEMV_E_SHAPE.
 *   Threads    calls are thread-safe (no global mutable state).
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t; /* hipStream_t is `struct ihipStream_t *` */

enum {
  QGEMV_OK = 0,
  QGEMV_E_NULL = -1,  /* a required pointer is NULL (with M > 0) */
  QGEMV_E_SHAPE = -2, /* M < 0, K <= 0, K not a multiple of the block, or sizes overflow */
  QGEMV_E_ALIGN = -3, /* a pointer is not aligned as required */
  QGEMV_E_HIP = -4,   /* the HIP runtime rejected the launch */
  QGEMV_E_ALIAS = -5, /* the output overlaps an input */
  QGEMV_E_DTYPE = -6, /* an element-type code is not one of QGEMV_F32 / QGEMV_F16 / QGEMV_BF16 */
  QGEMV_E_WORKSPACE = -7 /* a workspace smaller than qgemm_workspace_bytes asks for */
};

/* Element types of epilogue vectors and materialised rows: fp32, IEEE binary16
 * and bfloat16.  Conversions to the 16-bit types round to nearest even. */
enum { QGEMV_F32 = 0, QGEMV_F16 = 1, QGEMV_BF16 = 2 };

/* Q4_K ("Writing a high performant GEMV + dequant for Metal", sections "What is
 * a weight block?", "Compute", "Kernel code"): K % 256 == 0; each row holds K/256
 * super-blocks of 144 bytes: fp16 d @0, fp16 dmin @2, 12 bytes of packed 6-bit
 * group scales/mins @4, 128 bytes of 4-bit quants @16 (little-endian).  Weight i
 * of a block is d*s_g*q_i - dmin*m_g with g = i/32.  x is fp16.
 * W occupies M*(K/256)*144 bytes. */
int qgemv_q4k(const void* w, const void* x_f16, float* y, int64_t M, int64_t K,
              struct ihipStream_t* stream);

/* NVFP4 W4A16 (Mojo module "fp4_gemv", function enqueue_apple_fp4_gemv: out =
 * a @ dequant(packed, scales)^T at M = 1): K % 32 == 0.  W is ONE buffer of
 * M*K/2 bytes of E2M1 nibbles ([M][K/2], the even element in the low nibble)
 * followed, at byte offset M*K/2, by M*K/16 OCP FP8 E4M3 scale bytes ([M][K/16],
 * one per 16 consecutive weights of a row).  Weight = e2m1 * |scale|.  x is bf16.
 * W occupies M*K/2 + M*K/16 bytes. */
int qgemv_nvfp4(const void* w, const void* x_bf16, float* y, int64_t M, int64_t K,
                struct ihipStream_t* stream);

/* TQ1_0 ("metal: TQ1_0 kernel performance", sections 1 and 2): K % 256 == 0;
 * each row holds K/256 blocks of 54 bytes: qs[48] @0 (five base-3 digits per
 * byte), qh[4] @48 (four digits per byte), fp16 d @52.  Digit k of byte b is
 * floor(3*((3^k*b) mod 256)/256); digit k of qs[j] feeds element 32k+j (j<32)
 * or 160+16(k)+(j-32) (32<=j<48); digit k<4 of qh[m] feeds element 240+4k+m.
 * Weight = d*(digit-1).  x is fp16.  W occupies M*(K/256)*54 bytes. */
int qgemv_tq1(const void* w, const void* x_f16, float* y, int64_t M, int64_t K,
              struct ihipStream_t* stream);

/* General output stage ("Writing a high performant GEMV + dequant for Metal",
 * section "What is a GEMV": y = alpha * x . W^T + beta * c; that page's kernel
 * writes fp16 y, the Mojo fp4_gemv page ends in a final cast):
 *     y[r] = alpha * v_r + beta * c[r]      v_r = x . dequant(W)[r] in fp32
 * evaluated in fp32 (one fma for the beta term) and stored as y_dtype.
 *   alpha, beta  scalars (host values copied at the call).
 *   c            M elements of c_dtype in device memory, read only when
 *                beta != 0 (it may then be NULL).  c may be y itself when
 *                c_dtype == y_dtype (in place: y = alpha v + beta y); any other
 *                overlap of c with y returns QGEMV_E_ALIAS.
 *   y            M elements of y_dtype (aligned to its size).
 * A NULL epilogue pointer means alpha = 1, beta = 0, fp32 y. */
typedef struct qgemv_epilogue {
  float alpha;
  float beta;
  const void* c;
  int32_t c_dtype;
  int32_t y_dtype;
} qgemv_epilogue;

/* The three GEMVs above with the general output stage; W, x, M, K, stream and
 * the errors as for the plain calls, plus QGEMV_E_DTYPE for a bad type code. */
int qgemv_q4k_ex(const void* w, const void* x_f16, void* y, int64_t M, int64_t K, const qgemv_epilogue* ep,
                 struct ihipStream_t* stream);
int qgemv_nvfp4_ex(const void* w, const void* x_bf16, void* y, int64_t M, int64_t K, const qgemv_epilogue* ep,
                   struct ihipStream_t* stream);
int qgemv_tq1_ex(const void* w, const void* x_f16, void* y, int64_t M, int64_t K, const qgemv_epilogue* ep,
                 struct ihipStream_t* stream);

/* Dense GEMV, the uncompressed comparison point of the Mojo fp4_gemv page (its
 * NVFP4 GEMV against a bf16 GEMV of the same shape): W is [M][K] row-major in
 * the activations' type, fp16 for qgemv_f16 and bf16 for qgemv_bf16.
 * 0 < K <= 65536 and K % 8 == 0 (rows start 16-byte aligned); W occupies
 * 2*M*K bytes.  Other conventions as above; the _ex forms take the general
 * output stage. */
int qgemv_f16(const void* w, const void* x_f16, float* y, int64_t M, int64_t K, struct ihipStream_t* stream);
int qgemv_bf16(const void* w, const void* x_bf16, float* y, int64_t M, int64_t K, struct ihipStream_t* stream);
int qgemv_f16_ex(const void* w, const void* x_f16, void* y, int64_t M, int64_t K, const qgemv_epilogue* ep,
                 struct ihipStream_t* stream);
int qgemv_bf16_ex(const void* w, const void* x_bf16, void* y, int64_t M, int64_t K, const qgemv_epilogue* ep,
                  struct ihipStream_t* stream);

/* Row materialisation (GET_ROWS; the dequantize template of "metal: TQ1_0
 * kernel performance", section "Prefill", and the Mojo fp4_gemv page's
 * dequant): out[j][0..K) = row rows[j] of dequant(W) for j < nrows, each
 * weight rounded to fp32 and then to out_dtype.
 *   w, M, K   the packed matrix, as for the GEMVs of the same format.
 *   rows      nrows int32 row indices in device memory, or NULL for rows
 *             0..nrows-1 (then nrows <= M).  An index outside [0, M) gives a
 *             row of quiet NaNs (sign bit clear): indices are device data and
 *             are not checked on the host.
 *   out       nrows*K elements of out_dtype, 16-byte aligned, not overlapping
 *             W or rows.
 * nrows == 0 is a successful no-op. */
int qget_rows_q4k(const void* w, int64_t M, int64_t K, const int32_t* rows, int64_t nrows, void* out,
                  int32_t out_dtype, struct ihipStream_t* stream);
int qget_rows_nvfp4(const void* w, int64_t M, int64_t K, const int32_t* rows, int64_t nrows, void* out,
                    int32_t out_dtype, struct ihipStream_t* stream);
int qget_rows_tq1(const void* w, int64_t M, int64_t K, const int32_t* rows, int64_t nrows, void* out,
                  int32_t out_dtype, struct ihipStream_t* stream);

/* Prefill: T activation rows at once (the Mojo fp4_gemv page's M > 1 matmul
 * path; the TQ1_0 page's prefill):
 *     y[t][r] = sum_{i<K} x[t][i] * dequant(W)[r][i]     t < T, r < M
 * x is [T][K] row-major in the format's activation type (fp16 for Q4_K), y is
 * [T][M] row-major fp32.  W, M and K as for the GEMV of the same format, plus
 * K <= 2^20 and T <= 65535 * 128.  The weights are dequantised to the
 * activation type (one rounding per weight) and multiplied on the matrix
 * cores with fp32 accumulation.  Every element of y is overwritten.  When the
 * output has fewer tiles (256 or 512 tokens x 128 rows) than the device has
 * compute units, or 512-token tiles leave a last round of workgroups at most
 * a quarter full, the K range of those tiles is split across workgroups whose
 * partial sums are added into y with fp32 atomics (after their rows of y are
 * cleared on the same stream), so the last bits can differ from run to run;
 * the error bound is unchanged.  T == 0 or M == 0 is a successful no-op; y must not overlap W
 * or x. */
int qgemm_q4k(const void* w, const void* x_f16, float* y, int64_t T, int64_t M, int64_t K,
              struct ihipStream_t* stream);
/* NVFP4 prefill: x is [T][K] bf16; K % 64 == 0.  The weights e2m1 * |scale|
 * are exact in bf16, so the matrix cores see them unrounded. */
int qgemm_nvfp4(const void* w, const void* x_bf16, float* y, int64_t T, int64_t M, int64_t K,
                struct ihipStream_t* stream);
/* TQ1_0 prefill: x is [T][K] fp16.  The weights d * (t - 1) are exact in
 * fp16 ("metal: TQ1_0 kernel performance", section "Prefill": blocks are
 * unpacked into a tile that the matrix unit reads). */
int qgemm_tq1(const void* w, const void* x_f16, float* y, int64_t T, int64_t M, int64_t K,
              struct ihipStream_t* stream);

/* Prefill whose result does not vary from run to run: the same as qgemm_* but
 * the partial sums of tiles split over K go to `workspace` (device memory
 * owned by the caller) and a second kernel on the same stream adds them in a
 * fixed order into y, so no atomics and no clearing of y are involved.
 * qgemm_workspace_bytes(T, M, K) gives the bytes needed (0 when no tile is
 * split: the workspace may then be NULL; QGEMV_E_SHAPE for sizes no qgemm_*
 * call accepts).  The workspace must be 256-byte aligned, at least that large
 * and overlap none of W, x and y; its contents need no initialisation and
 * are overwritten, so calls that overlap in time must not share it.  Errors:
 * as qgemm_*, plus QGEMV_E_WORKSPACE when workspace_bytes is too small. */
int64_t qgemm_workspace_bytes(int64_t T, int64_t M, int64_t K);
int qgemm_q4k_ws(const void* w, const void* x_f16, float* y, int64_t T, int64_t M, int64_t K, void* workspace,
                 int64_t workspace_bytes, struct ihipStream_t* stream);
int qgemm_nvfp4_ws(const void* w, const void* x_bf16, float* y, int64_t T, int64_t M, int64_t K, void* workspace,
                   int64_t workspace_bytes, struct ihipStream_t* stream);
int qgemm_tq1_ws(const void* w, const void* x_f16, float* y, int64_t T, int64_t M, int64_t K, void* workspace,
                 int64_t workspace_bytes, struct ihipStream_t* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): Q4_K
 * prefill with the same result as qgemm_q4k_ws, whose workspace is instead a
 * fixed device array inside the library, QGEMV_NOALLOC_MAX_BYTES (32 MiB)
 * per device, reserved on each device the library is used on until the
 * process ends.  The call allocates nothing: no hipMalloc, no hipFree, no
 * allocating library routine.  Its first call on a device looks the array's
 * address up once (thread-safe).  The caller passes W, x and y as for
 * qgemm_q4k.  Errors: as qgemm_q4k, plus QGEMV_E_WORKSPACE when
 * qgemm_workspace_bytes(T, M, K) exceeds QGEMV_NOALLOC_MAX_BYTES.  Nothing in
 * the array needs to start at zero; every call on one device shares that
 * device's array and leaves its own partial sums there, so calls on one device
 * that overlap in time (on different streams, or from different threads)
 * race and must be serialised by the caller. */
#define QGEMV_NOALLOC_MAX_BYTES (32ll << 20)
int qgemm_q4k_noalloc(const void* w, const void* x_f16, float* y, int64_t T, int64_t M, int64_t K,
                      struct ihipStream_t* stream);

/* fp32 materialisation out[M][K] of the same formats (same W conventions as
 * above; the same as qget_rows_* with rows = NULL, nrows = M, QGEMV_F32).  Each value is the correctly rounded fp32 of the exact weight, which
 * for these formats is the exact weight itself whenever it is representable
 * (the bit-exact reference for the GEMVs; Mojo module "fp4_gemv", TQ1_0 PR
 * section "Correctness"). */
int qdequant_q4k(const void* w, float* out, int64_t M, int64_t K, struct ihipStream_t* stream);
int qdequant_nvfp4(const void* w, float* out, int64_t M, int64_t K, struct ihipStream_t* stream);
int qdequant_tq1(const void* w, float* out, int64_t M, int64_t K, struct ihipStream_t* stream);

/* Bandwidth ceiling probe: streams `bytes` bytes of device memory at `buf`
 * (16-byte aligned, bytes % 16 == 0) with the same dwordx4 loads the GEMVs use
 * and writes one fp32 per workgroup into `sink` (at least qgemv_read_sink_len(bytes)
 * floats) so the loads cannot be elided.  The practical roofline of the part
 * ("Writing a high performant GEMV + dequant for Metal", section "Roofline
 * Analysis": a memory-bound kernel is limited by the DRAM bandwidth). */
int qgemv_read_ceiling(const void* buf, int64_t bytes, float* sink, struct ihipStream_t* stream);
int64_t qgemv_read_sink_len(int64_t bytes);

/* Human-readable text of a QGEMV_* code (static storage). */
const char* qgemv_strerror(int code);

/* HIP error code of the last launch failure on the calling thread (0 if none). */
int qgemv_last_hip_error(void);

/* Provenance: hash of the sources this library was built from ("metal: TQ1_0
 * kernel performance", section "Measuring this yourself": confirm which build
 * is being measured immediately before measuring). */
const char* qgemv_build_id(void);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_H */
