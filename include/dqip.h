/*
 * dqip.h -- C ABI of libdqip.so: the dynamic quantized inner product and the
 * QuantizeLinear / DequantizeLinear element-wise operators on one AMD
 * Instinct MI355X (gfx950).
 *
 * Conventions for every entry point
 *  - Tensor pointers (A, B, C, buf, weight, scale, bias, x, y, scales, zero
 *    points, inspection outputs) are DEVICE pointers on the current HIP
 *    device, owned by the caller. `params` and `shape` are HOST pointers.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Work is enqueued on it asynchronously, except where an entry point
 *    says it synchronizes; the caller keeps its buffers alive until the
 *    stream has completed.
 *  - Every call returns a status (DQ_OK = 0, else a negative DQ_ERR_*).
 *    All arguments are checked before anything is launched: on an error
 *    nothing is enqueued and no output is touched. dqip_last_error() then
 *    returns a message (per thread). A launch failure returns DQ_ERR_HIP.
 *    A device fault surfaces at the caller's synchronization.
 *  - Matrices are dense and row-major: A [M,K], B [K,N] (element B[k,j] at
 *    k*N + j), C [M,N]. Per-column vectors (scales, bias, column sums) are [N].
 */
#ifndef DQIP_H
#define DQIP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
/* The enumerations are int-sized in C. Compiled as C++ they get int as
 * their fixed underlying type, so that any int a C caller passes (an
 * invalid code included, which the calls reject with an error) is a valid
 * value of the parameter's type. */
#define DQ_ENUM_INT : int
#else
#define DQ_ENUM_INT
#endif

/* Element types: fp32, bf16 (raw 16-bit patterns), int8, uint8, fp16 (IEEE
 * binary16 bit patterns). */
typedef enum DQ_ENUM_INT { DQ_F32 = 0, DQ_BF16 = 1, DQ_I8 = 2, DQ_U8 = 3, DQ_F16 = 4 } dq_dtype;

/* Activations applied after dequantization and bias. Leaky ReLU takes its
 * slope from params[0] of dqip_set_params (default 0.01). */
typedef enum DQ_ENUM_INT { DQ_ACT_IDENTITY = 0, DQ_ACT_RELU = 1, DQ_ACT_LEAKY_RELU = 2 } dq_act;

enum {
    DQ_OK = 0,
    DQ_ERR_ARG = -1,   /* NULL where required, size out of range, misaligned buf */
    DQ_ERR_TYPE = -2,  /* type combination the method does not define        */
    DQ_ERR_STATE = -3, /* no context, or forward before a required set_params */
    DQ_ERR_RANGE = -4, /* K beyond DQ_K_MAX, axis out of range                */
    DQ_ERR_ALLOC = -5, /* device allocation failed                            */
    DQ_ERR_HIP = -6    /* a HIP runtime call or a kernel launch failed        */
};

/* axis value selecting per-tensor quantization in qlinear_* */
#define DQ_PER_TENSOR INT32_MIN

/* Largest K: the exact int32 sum needs 255 * 128 * K < 2^31. */
#define DQ_K_MAX 65536

typedef struct dqip_ctx dqip_ctx;

/* ------------------------------------------------------------------------
 * Dynamic quantized inner product.
 * Defined by Simd "SynetDynamicQuantizedInnerProduct16b Class Reference",
 * Detailed Description: A[i,k] -> uA[i,k] (uint8), scaleA[i], zeroA[i];
 * B[k,j] -> iB[k,j] (int8), scaleB[j]; sum_k (uA - zeroA) * iB in integers;
 * val = sum * scaleA[i] * scaleB[j]; C = Convert(Activate(val + bias[j])).
 * This library quantizes A per row with min/max over the row and 0 in range:
 *   scaleA = (hi - lo) / 255, zeroA = sat[0,255](rne(-lo / scaleA)),
 *   uA = sat[0,255](rne(A / scaleA) + zeroA)
 * and B per column, symmetric: scaleB = max|B| / qmax,
 *   iB = sat[qmin,qmax](rne(B / scaleB)), (qmin,qmax) = (-128,127), or
 *   (-64,63) with avoidOverflow; an all-zero row/column has scale 1 and
 *   zero point 0. Divisions are IEEE fp32, rounding is half to even.
 * The epilogue is fp32: ((float)sum * scaleA) * scaleB, + bias, activation,
 * then fp32 or bf16 (round to nearest even).
 * ---------------------------------------------------------------------- */

/* Init(): create or re-create a context (same page, Init()).
 * *ctx NULL creates one. A non-NULL *ctx whose M, N, K, types, constB,
 * bias, activation and avoidOverflow all equal the arguments is kept as is
 * (parameters set earlier stay); otherwise a new context is created and,
 * only once that has succeeded, the old one is released and *ctx replaced
 * (dqip_set_params is needed again when constB is set). On any error *ctx
 * is left unchanged: the old context stays valid and owned by the caller.
 * typeA, typeC in {DQ_F32, DQ_BF16}. typeB in {DQ_F32, DQ_I8} when constB
 * (DQ_I8 = B already quantized, avoidOverflow then ignored), in
 * {DQ_F32, DQ_BF16} when not. 1 <= M, N <= 2^31-1, 1 <= K <= DQ_K_MAX.
 * Allocates the context's device buffers on the current device.
 * Errors: DQ_ERR_ARG, DQ_ERR_TYPE, DQ_ERR_RANGE, DQ_ERR_ALLOC, DQ_ERR_HIP. */
int dqip_init(dqip_ctx** ctx, size_t M, size_t N, size_t K, dq_dtype typeA,
              dq_dtype typeB, dq_dtype typeC, int constB, int bias,
              dq_act activation, int avoidOverflow);

/* Enable(): 1 if ctx is a created context, else 0. */
int dqip_enabled(const dqip_ctx* ctx);

/* InternalBufferSize(): device bytes held by the context now: packed
 * quantized B, its column sums and scales, bias, activation parameters and,
 * once a forward ran with buf == NULL, the fallback work buffer. 0 for NULL. */
size_t dqip_internal_buffer_size(const dqip_ctx* ctx);

/* ExternalBufferSize(): bytes the caller may pass as `buf` to dqip_forward:
 * the quantized copy of A with its per-row scales and zero points, plus,
 * when B is not constant, the quantized B with its scales and column sums.
 * 0 for NULL. */
size_t dqip_external_buffer_size(const dqip_ctx* ctx);

/* Info(): "<arch> <kernels>" description of the selected implementation,
 * owned by the context, valid until it is released. NULL for NULL. */
const char* dqip_info(const dqip_ctx* ctx);

/* SetParams() (same page, SetParams()).
 * weight: B with K*N elements of typeB (device); required when constB, else
 *   ignored (may be NULL). An fp32 B is quantized here, once.
 * scale: per-column fp32 scales [N] (device); required iff typeB == DQ_I8.
 * bias: [N] fp32 (device) or NULL (zeros); used when the context has bias.
 * params: activation parameters (HOST); params[0] is the leaky-ReLU slope;
 *   NULL keeps the default 0.01.
 * Enqueues on `stream`, then synchronizes it, so the caller may free its
 * inputs on return. Errors: DQ_ERR_STATE, DQ_ERR_ARG, DQ_ERR_HIP. */
int dqip_set_params(dqip_ctx* ctx, const void* weight, const float* scale,
                    const float* bias, const float* params, void* stream);

/* Forward() (same page, Forward()): C = the inner product of A and B.
 * A: [M,K] of typeA. B: [K,N] of typeB when B is not constant (quantized on
 * every call), ignored and may be NULL when constant. C: [M,N] of typeC.
 * buf: NULL (the context's own work buffer, allocated on first use) or at
 * least dqip_external_buffer_size() bytes, 256-byte aligned; it receives
 * the quantized A (and B) and must not be shared by calls in flight.
 * Asynchronous on `stream`. Errors: DQ_ERR_STATE (not created, or constant
 * B without dqip_set_params), DQ_ERR_ARG, DQ_ERR_ALLOC, DQ_ERR_HIP. */
int dqip_forward(dqip_ctx* ctx, const void* A, const void* B, void* buf,
                 void* C, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, hosts that forbid hipMalloc): the forward
 * above with its work buffer in the library's own static device scratch of
 * DQIP_NOALLOC_SCRATCH_BYTES (32 MiB; one copy per GPU the library runs on,
 * held until the process ends). It calls no hipMalloc / hipFree and no
 * allocating library routine. The context must need at most that much work
 * buffer (dqip_external_buffer_size(ctx) <= DQIP_NOALLOC_SCRATCH_BYTES, e.g.
 * a 4096 x 4096 x 4096 product with a constant B needs 16 MiB + 32 KiB),
 * else DQ_ERR_RANGE and nothing is launched. Every call on one GPU shares
 * that GPU's scratch: calls that overlap on one GPU (other streams, other
 * threads) race and must be serialized by the caller. A, B, C as for
 * dqip_forward. Errors: DQ_ERR_STATE, DQ_ERR_RANGE, DQ_ERR_ARG, DQ_ERR_TYPE,
 * DQ_ERR_HIP. */
#define DQIP_NOALLOC_SCRATCH_BYTES (32u << 20)
int dqip_forward_noalloc(dqip_ctx* ctx, const void* A, const void* B, void* C, void* stream);

/* Clear(): release the context and its device buffers (NULL is a no-op).
 * The caller makes sure no enqueued work still uses them. */
void dqip_release(dqip_ctx* ctx);

/* Message of the last failed call on this thread ("" if none). */
const char* dqip_last_error(void);

/* ---- inspection of the quantized operands (for parity checks) -------- */

/* Unpacks the quantized A left in `buf` (NULL = the internal buffer) by the
 * last dqip_forward: uA [M,K] uint8, scaleA [M] fp32, zeroA [M] int32. Any
 * output may be NULL. Asynchronous on `stream`. */
int dqip_read_quantized_a(const dqip_ctx* ctx, const void* buf, uint8_t* uA,
                          float* scaleA, int32_t* zeroA, void* stream);

/* Unpacks the quantized B -- the context's constant B, or the one the last
 * dqip_forward left in `buf` when B is not constant -- as iB [K,N] int8,
 * scaleB [N] fp32 and colsumB [N] int32 (sum over k of iB). Any output may
 * be NULL. Asynchronous on `stream`. */
int dqip_read_quantized_b(const dqip_ctx* ctx, const void* buf, int8_t* iB,
                          float* scaleB, int32_t* colsumB, void* stream);

/* dqip_forward with the integer sums as output: acc [M,N] int32 holds
 * sum_k (uA[i,k] - zeroA[i]) * iB[k,j] instead of C (no epilogue). */
int dqip_forward_accumulators(dqip_ctx* ctx, const void* A, const void* B,
                              void* buf, int32_t* acc, void* stream);

/* ---- per-kernel timing (for benchmarks) ------------------------------ */

/* Phases of one dqip_forward, in launch order. */
enum { DQ_PHASE_QUANT_A = 0, DQ_PHASE_QUANT_B = 1, DQ_PHASE_GEMM = 2, DQ_PHASES = 3 };

/* After dqip_profile_begin(ctx, capacity) each of the next `capacity`
 * dqip_forward / dqip_forward_accumulators calls has the first kernel of each
 * phase record a start event and the last kernel a stop event, taken from the
 * kernel dispatches themselves (hipExtLaunchKernel), so a phase's time is its
 * kernels' execution time without launch gaps (nothing else changes; no
 * sync).
 * dqip_profile_end waits for the recorded events and writes, per phase, the
 * summed milliseconds to ms[DQ_PHASES] (DQ_PHASE_QUANT_B stays 0 for a
 * constant B) and the number of recorded calls to *calls; it then stops
 * recording. Errors: DQ_ERR_STATE, DQ_ERR_ARG (capacity < 1), DQ_ERR_HIP. */
int dqip_profile_begin(dqip_ctx* ctx, int capacity);
int dqip_profile_end(dqip_ctx* ctx, float* ms, int* calls);

/* ---- measurement probes (not operations of the pages) -----------------
 * What the hardware reaches on its own, reported next to the published
 * peaks as context for the kernels' roofline fractions. Both launch one
 * kernel on `stream` (asynchronous; the caller times it, e.g. with events).
 *
 * dq_probe_mfma_loop: `workgroups` workgroups of 4 waves; each wave keeps
 * the int32 accumulators of a 128x128 tile (the GEMM's wave tile) and runs
 * `iters` iterations on register operands only, alternating two operand
 * sets taken from `operands` (device, at least 65536 bytes: random codes,
 * or zeros). shape 32: 16 blocks of 32x32, 32 v_mfma_i32_32x32x32_i8 an
 * iteration; shape 16: 64 blocks of 16x16, 64 v_mfma_i32_16x16x64_i8 an
 * iteration (the GEMM's instruction). Either way an iteration is
 * 32 * 65536 int8 ops: total workgroups * 4 * iters * 32 * 65536. sink
 * (device, at least workgroups * 256 int32) receives one checksum per
 * lane.
 * dq_probe_copy: copies `bytes` (multiple of 16) from src to dst (device,
 * 16-byte aligned, not overlapping): 16 KiB per workgroup of 256 threads,
 * each thread's four 16-byte non-temporal loads issued before its stores.
 * Errors: DQ_ERR_ARG, DQ_ERR_HIP. */
int dq_probe_mfma_loop(const void* operands, int shape, int iters, int workgroups, int32_t* sink,
                       void* stream);
int dq_probe_copy(const void* src, void* dst, size_t bytes, void* stream);

/* ------------------------------------------------------------------------
 * QuantizeLinear / DequantizeLinear.
 * Defined by onnxruntime quantization_defs.cc, QuantizeLinear and
 * DequantizeLinear docs: y = saturate(x / y_scale + y_zero_point) with
 * x / y_scale rounded to nearest, ties to even (IEEE fp32 division),
 * saturating to [0,255] (uint8) or [-128,127] (int8); and
 * y = (x - x_zero_point) * x_scale. Scale and zero point are one value
 * (axis = DQ_PER_TENSOR) or one per index of dimension `axis` (negative
 * axis counts from the end).
 * x, y: dense row-major tensors of the given shape (HOST array of ndim
 * sizes, 1 <= ndim <= 8, each >= 0; zero elements is a no-op). Scales are
 * fp32, zero points have the 8-bit type (NULL = 0).
 * Asynchronous on `stream`. Errors: DQ_ERR_ARG, DQ_ERR_TYPE (x must be
 * DQ_F32 to quantize, int8/uint8 to dequantize), DQ_ERR_RANGE (axis),
 * DQ_ERR_HIP.
 * ---------------------------------------------------------------------- */
int qlinear_quantize(const float* x, int ndim, const int64_t* shape, int axis,
                     const float* y_scale, const void* y_zero_point,
                     dq_dtype y_type, void* y, void* stream);

int qlinear_dequantize(const void* x, dq_dtype x_type, int ndim,
                       const int64_t* shape, int axis, const float* x_scale,
                       const void* x_zero_point, float* y, void* stream);

/* The same operators on fp16 tensors. The schemas constrain QuantizeLinear's
 * x and y_scale to one float type T1 and DequantizeLinear's x_scale and y to
 * one float type T2, each fp16 or fp32, while DequantizeLinear's shape
 * inference always makes y fp32. This library reads fp16 values exactly as
 * fp32 and applies the rules above: qlinear_quantize_f16 takes fp16 x and
 * y_scale; qlinear_dequantize_f16 takes fp16 x_scale and writes y as fp16
 * (y_type DQ_F16: the exact product (x - zp) * s, at most 19 significant
 * bits, rounded once to nearest even) or as fp32 (DQ_F32). Pointers,
 * shapes, axis and errors as above (DQ_ERR_TYPE for another y_type). */
int qlinear_quantize_f16(const void* x, int ndim, const int64_t* shape, int axis,
                         const void* y_scale, const void* y_zero_point, dq_dtype y_type,
                         void* y, void* stream);
int qlinear_dequantize_f16(const void* x, dq_dtype x_type, int ndim, const int64_t* shape,
                           int axis, const void* x_scale, const void* x_zero_point,
                           dq_dtype y_type, void* y, void* stream);

/* ------------------------------------------------------------------------
 * Requantizing 1x1 QLinearConv (stride 1, no padding, one group).
 * Defined by the ONNX "QLinearConv" operator (opset 10), description and
 * inputs: x, w and y are 8-bit tensors; x and y have one scale and zero
 * point each, w one per tensor or one per output channel; the optional bias
 * is int32, already quantized with scale x_scale * w_scale and zero point 0.
 * For each image n, output channel m and pixel p:
 *   acc  = sum_c (w[m,c] - w_zp[m]) * (x[n,c,p] - x_zp) + bias[m]
 *   real = ((float)acc * x_scale) * w_scale[m]
 *   y[n,m,p] = saturate(rne(real / y_scale) + y_zp)
 * with an IEEE fp32 quotient rounded to nearest, ties to even, and
 * saturation to [0,255] (uint8 y) or [-128,127] (int8 y).
 * x: [N, C, HW] (NCHW with H*W = HW), y: [N, M, HW], w: [M, C], all dense
 * row-major DEVICE tensors. x_scale, y_scale: one fp32 on the device.
 * x_zero_point / y_zero_point: one value of x's / y's type on the device
 * (NULL = 0). w_scale: w_len fp32, w_zero_point: w_len values of w's type
 * (NULL = 0), w_len = 1 or M. bias: M int32 (NULL = none).
 * The sum is exact while acc fits in int32 (C <= 32768 bounds the product
 * part; the caller keeps bias within range).
 * Asynchronous on `stream`. Zero N, HW or M is a no-op. Errors:
 * DQ_ERR_TYPE (a type other than DQ_I8 / DQ_U8), DQ_ERR_ARG (C < 1,
 * negative sizes, w_len, NULL tensors or scales), DQ_ERR_RANGE (C > 32768,
 * a grid beyond one launch), DQ_ERR_HIP.
 * ---------------------------------------------------------------------- */
int qlinear_conv1x1(const void* x, dq_dtype x_type, int64_t N, int64_t C,
                    int64_t HW, const float* x_scale, const void* x_zero_point,
                    const void* w, dq_dtype w_type, int64_t M,
                    const float* w_scale, const void* w_zero_point,
                    int64_t w_len, const float* y_scale,
                    const void* y_zero_point, dq_dtype y_type,
                    const int32_t* bias, void* y, void* stream);

/* ------------------------------------------------------------------------
 * Quantized matrix products: QGemm, MatMulIntegerToFloat and
 * DynamicQuantizeMatMul.
 * onnxruntime quantization_defs.cc, schemas QGemm, MatMulIntegerToFloat and
 * DynamicQuantizeMatMul, give the inputs (8-bit A and B with scales and zero
 * points, B's per tensor or per column; QGemm's int32 C "quantized with zero
 * point 0 and scale alpha / beta * a_scale * b_scale"; optional y_scale /
 * y_zero_point making Y 8-bit), the attributes (transA, transB, alpha) and
 * the types, but no formula. This library computes, for m < M, n < N:
 *   sum[m,n] = sum_k (A[m,k] - a_zp) * (B[k,n] - b_zp[n])      (exact int32)
 *   real     = ((float)(sum + C[m,n]) * fl(alpha * a_scale)) * b_scale[n]
 *              + bias[n]                       (fp32, in this order)
 *   Y[m,n]   = real (fp32 Y), or saturate(rne(real / y_scale) + y_zp)
 * (beta is read as 1; the IEEE fp32 quotient is rounded to nearest, ties to
 * even, as QuantizeLinear states). MatMulIntegerToFloat is an 8-bit A with
 * an fp32 Y and optional bias; DynamicQuantizeMatMul is an fp32 A, which
 * each forward quantizes per tensor to uint8 with lo = min(0, min A),
 * hi = max(0, max A), a_scale = (hi - lo) / 255 (1 if hi == lo),
 * a_zp = saturate(rne(-lo / a_scale)); QGemm adds C, alpha, transA and an
 * 8-bit Y. Life cycle as dqip: init, set the constant B once, forward.
 *
 * dq_qgemm_init: shapes (1 <= M, N < 2^31 - 256, 1 <= K <= DQ_QGEMM_K_MAX,
 * so every sum fits in int32), a_type DQ_F32 / DQ_U8 / DQ_I8 (DQ_F32 =
 * dynamic quantization, not with transA), transA (A given as [K,M]),
 * b_type DQ_U8 / DQ_I8, transB (B given as [N,K]), y_type DQ_F32 / DQ_U8 /
 * DQ_I8, alpha. Allocates every device buffer of the context (none later).
 * Errors: DQ_ERR_ARG, DQ_ERR_RANGE, DQ_ERR_TYPE, DQ_ERR_ALLOC, DQ_ERR_HIP.
 *
 * dq_qgemm_set_b: B ([K,N], or [N,K] with transB, dense row-major DEVICE
 * tensor of b_type), b_scale (b_scale_len = 1 or N fp32 on the device),
 * b_zero_point (b_zero_point_len = 1 or N values of b_type on the device,
 * NULL = 0). Packs B into the context; the caller may free its tensors when
 * the call returns (it synchronizes `stream`). Errors: DQ_ERR_STATE,
 * DQ_ERR_ARG, DQ_ERR_HIP.
 *
 * dq_qgemm_forward: A ([M,K], or [K,M] with transA, dense row-major DEVICE
 * tensor of a_type); a_scale (one fp32 on the device; NULL for an fp32 A);
 * a_zero_point (one value of a_type on the device, NULL = 0; NULL for an
 * fp32 A); C (int32 DEVICE tensor of shape [c_rows, c_cols], c_rows = 1 or
 * M and c_cols = 1 or N, broadcast to [M,N]; NULL = none); bias (N fp32 on
 * the device, fp32 Y only; NULL = none); y_scale / y_zero_point (8-bit Y:
 * one fp32 and one value of y_type on the device, zero point NULL = 0;
 * NULL for an fp32 Y); Y ([M,N] dense row-major DEVICE tensor of y_type).
 * Asynchronous on `stream`. Errors: DQ_ERR_STATE (no B yet, other device),
 * DQ_ERR_ARG, DQ_ERR_HIP.
 * dq_qgemm_forward_accumulators: the same with the int32 sum + C written to
 * acc [M,N] (inspection).
 * ---------------------------------------------------------------------- */
#define DQ_QGEMM_K_MAX 32768

typedef struct dq_qgemm_ctx dq_qgemm_ctx;

int dq_qgemm_init(dq_qgemm_ctx** ctx, int64_t M, int64_t N, int64_t K, dq_dtype a_type,
                  int transA, dq_dtype b_type, int transB, dq_dtype y_type, float alpha);
int dq_qgemm_set_b(dq_qgemm_ctx* ctx, const void* B, const float* b_scale, int64_t b_scale_len,
                   const void* b_zero_point, int64_t b_zero_point_len, void* stream);
int dq_qgemm_forward(dq_qgemm_ctx* ctx, const void* A, const float* a_scale,
                     const void* a_zero_point, const int32_t* C, int64_t c_rows, int64_t c_cols,
                     const float* bias, const float* y_scale, const void* y_zero_point, void* Y,
                     void* stream);
int dq_qgemm_forward_accumulators(dq_qgemm_ctx* ctx, const void* A, const float* a_scale,
                                  const void* a_zero_point, const int32_t* C, int64_t c_rows,
                                  int64_t c_cols, int32_t* acc, void* stream);
/* ------------------------------------------------------------------------
 * N-dimensional MatMulIntegerToFloat / DynamicQuantizeMatMul.
 * onnxruntime quantization_defs.cc, schemas MatMulIntegerToFloat and
 * DynamicQuantizeMatMul: A and B are "N-dimensional" matrices and Y's
 * shape is inferred as ONNX MatMul's, i.e. numpy.matmul's rules: the last
 * two dimensions are the matrices ([M,K] and [K,N]), the leading ones are
 * batch dimensions aligned from the right, and a batch dimension of 1 is
 * broadcast against the other side's (a 1-D operand is the caller's M = 1
 * or N = 1 with that dimension left out of Y). b_scale, b_zero_point (1 or
 * N values) and bias serve every batch; DynamicQuantizeMatMul quantizes
 * its fp32 A per tensor over all batches at once.
 *
 * dq_qgemm_init_batched: batch_rank (0 <= rank <= DQ_QGEMM_BATCH_RANK_MAX)
 * batch dimensions of A and of B (HOST arrays of batch_rank values >= 1,
 * shorter ranks left-padded with 1 by the caller; NULL when the rank is 0),
 * each pair equal or one of them 1; M, N, K as dq_qgemm_init; a_type
 * DQ_F32 / DQ_U8 / DQ_I8, b_type DQ_U8 / DQ_I8; Y is fp32, alpha 1, no
 * transposes. The broadcast batch count must not exceed DQ_QGEMM_BATCH_MAX.
 * The context then takes, in dq_qgemm_set_b, B as [B batches][K][N]
 * (dense row-major, batches in row-major order of b's batch dimensions), and
 * in dq_qgemm_forward A as [A batches][M][K] and Y as [Y batches][M][N]
 * (the broadcast batch shape, row-major); C must be NULL (these operators
 * have none). When B has a single batch the batches of A are its rows (one
 * [batches * M, K] product); otherwise each Y batch is one product.
 * Errors: DQ_ERR_ARG (ranks, dimensions, broadcasting), DQ_ERR_RANGE,
 * DQ_ERR_TYPE, DQ_ERR_ALLOC, DQ_ERR_HIP.
 * ---------------------------------------------------------------------- */
#define DQ_QGEMM_BATCH_RANK_MAX 8
#define DQ_QGEMM_BATCH_MAX 65536

int dq_qgemm_init_batched(dq_qgemm_ctx** ctx, int batch_rank, const int64_t* a_batch,
                          const int64_t* b_batch, int64_t M, int64_t N, int64_t K,
                          dq_dtype a_type, dq_dtype b_type);
/* A short description of the kernels the context runs (owned by it). */
const char* dq_qgemm_info(const dq_qgemm_ctx* ctx);
/* Frees the context and its device memory; NULL is a no-op. */
void dq_qgemm_release(dq_qgemm_ctx* ctx);

/* ------------------------------------------------------------------------
 * General 2-D QLinearConv as an implicit GEMM.
 * Defined by the ONNX "QLinearConv" operator (opset 10), description and
 * inputs, with ONNX Conv's attributes (the page names kernel size, stride,
 * pad lengths and group): x [N, C, H, W], w [M, C / group, kH, kW] and y
 * [N, M, oH, oW] are dense row-major 8-bit DEVICE tensors,
 *   oH = floor((H + pad_top + pad_bottom - dil_h (kH - 1) - 1) / stride_h) + 1
 * (likewise oW); output channel m of group g = m / (M / group) reads input
 * channels g C / group .. (g + 1) C / group - 1:
 *   acc  = sum_{c, kh, kw} (w[m,c,kh,kw] - w_zp[m]) (x[n, gC/group + c, ih, iw] - x_zp) + bias[m]
 *   real = ((float)acc * x_scale) * w_scale[m]
 *   y    = saturate(rne(real / y_scale) + y_zp)
 * with ih = oh stride_h - pad_top + kh dil_h, iw likewise; a tap outside the
 * image reads x_zp (a padded input is a real 0).
 *
 * dq_qconv_init: C, H, W, M, kH, kW >= 1; strides[2] (h, w; NULL = 1, 1),
 * pads[4] (top, left, bottom, right; NULL = 0), dilations[2] (NULL = 1, 1)
 * are HOST arrays; group >= 1 divides C and M; x_type, w_type, y_type are
 * DQ_I8 / DQ_U8. Limits: C / group * kH * kW <= 32768 (int32 sums), the
 * input patch of a workgroup (rows x padded width x 32 bytes) <= 112 KiB.
 * Allocates the context's device buffers (packed weights). Errors:
 * DQ_ERR_ARG, DQ_ERR_TYPE, DQ_ERR_RANGE, DQ_ERR_ALLOC, DQ_ERR_HIP.
 * dq_qconv_output_shape: oH, oW (host).
 * dq_qconv_set_w: w (DEVICE, the shape above, w_type), w_scale (w_len fp32
 * on the device, w_len = 1 or M), w_zero_point (w_len values of w_type on
 * the device, NULL = 0), bias (M int32 on the device, NULL = none). Packs
 * them into the context and synchronizes `stream`; the caller may free its
 * tensors afterwards. Errors: DQ_ERR_STATE, DQ_ERR_ARG, DQ_ERR_HIP.
 * dq_qconv_forward: x (N images), x_scale / y_scale (one fp32 each on the
 * device), x_zero_point / y_zero_point (one value of x's / y's type on the
 * device, NULL = 0), y (N x M x oH x oW). Asynchronous on `stream`; N = 0
 * is a no-op. When the tiles of the N images would leave the chip
 * under-filled (deep layers), the reduction is split over workgroups with
 * int32 partial sums in a context buffer of N x splits x (M + group) x
 * oH x oW int32; a call that needs a larger buffer than the context holds
 * synchronizes `stream`, frees the old one and allocates it (calls on one
 * context must not overlap). Errors: DQ_ERR_STATE (no weights, other
 * device), DQ_ERR_ARG, DQ_ERR_RANGE (N > 65535), DQ_ERR_ALLOC, DQ_ERR_HIP.
 * ---------------------------------------------------------------------- */
typedef struct dq_qconv_ctx dq_qconv_ctx;

int dq_qconv_init(dq_qconv_ctx** ctx, int64_t C, int64_t H, int64_t W, int64_t M, int64_t kH,
                  int64_t kW, const int64_t* strides, const int64_t* pads,
                  const int64_t* dilations, int64_t group, dq_dtype x_type, dq_dtype w_type,
                  dq_dtype y_type);
int dq_qconv_output_shape(const dq_qconv_ctx* ctx, int64_t* oH, int64_t* oW);
int dq_qconv_set_w(dq_qconv_ctx* ctx, const void* w, const float* w_scale,
                   const void* w_zero_point, int64_t w_len, const int32_t* bias, void* stream);
int dq_qconv_forward(dq_qconv_ctx* ctx, const void* x, int64_t N, const float* x_scale,
                     const void* x_zero_point, const float* y_scale, const void* y_zero_point,
                     void* y, void* stream);
/* The kernel shape the context runs (owned by it); NULL for NULL. */
const char* dq_qconv_info(const dq_qconv_ctx* ctx);
/* Frees the context and its device memory; NULL is a no-op. */
void dq_qconv_release(dq_qconv_ctx* ctx);

/* ------------------------------------------------------------------------
 * Element-wise quantized operators.
 * onnxruntime quantization_defs.cc, the contrib schemas QLinearAdd,
 * QLinearMul, MulInteger, QLinearLeakyRelu, QLinearSigmoid,
 * ReduceSumInteger, QLinearReduceMean and QLinearConcat, whose docs print:
 *   QLinearAdd  C = (A_scale (A - A_zp) + B_scale (B - B_zp)) / C_scale + C_zp
 *   QLinearMul  C = ((A - A_zp) (B - B_zp)) (A_scale B_scale) / C_scale + C_zp
 *   MulInteger  C (int32) = (A - A_zp) (B - B_zp)
 *   QLinearLeakyRelu  quantize(alpha x) where x = dequantize(X) < 0, else
 *                     quantize(x)
 *   QLinearSigmoid    quantize(1 / (1 + exp(-dequantize(X))))
 *   ReduceSumInteger  sum over axes; int32 for int8 X, uint32 for uint8 X
 *   QLinearReduceMean quantize(mean over axes of dequantize(X))
 *   QLinearConcat     the inputs joined along axis, each one dequantized
 *                     with its own scale / zero point and quantized with Y's
 * dequantize(x) = (x - zp) * scale and quantize(v) = saturate(rne(v / scale)
 * + zp) as in QuantizeLinear (IEEE fp32 quotient, ties to even, [0,255] or
 * [-128,127]). This library takes the fp32 steps one at a time in the
 * printed order (A_scale * B_scale is one fp32 product); the sigmoid is
 * evaluated in fp64 and rounded to fp32 once; the mean is
 * fp32(fp64(S * x_scale) / count) with S the exact integer sum of x - x_zp.
 *
 * Common conventions: every tensor is a dense row-major DEVICE tensor of
 * `type` (DQ_U8 or DQ_I8; all 8-bit tensors of one call share it), shapes
 * are HOST arrays of ndim sizes (0 <= ndim <= 8 for the binary operators,
 * 1 <= ndim <= 8 otherwise, sizes >= 0). Scales: one fp32 on the device;
 * zero points: one value of `type` on the device (NULL = 0); every scale is
 * finite and > 0 (results for others are unspecified). Zero output elements
 * is a no-op. Asynchronous on `stream`. Errors: DQ_ERR_TYPE (type),
 * DQ_ERR_ARG (NULL tensor or scale, negative size, shapes that do not
 * broadcast or concatenate), DQ_ERR_RANGE (limits below, axis out of
 * range), DQ_ERR_HIP.
 *
 * qlinear_add / qlinear_mul: A [a_shape], B [b_shape] broadcast numpy-style
 * (multidirectional) to C's shape, which the caller allocates; C has fewer
 * than 2^32 elements.
 * dq_mul_integer: the same broadcast with an int32 C; A, B of `type`.
 * qlinear_leaky_relu / qlinear_sigmoid: x and y hold n elements.
 * dq_reduce_sum_integer / qlinear_reduce_mean: X [shape] reduced over the
 * n_axes dims listed in axes (HOST int32, negative counts from the end,
 * repeats allowed; n_axes = 0 reduces over every dim). y holds the kept
 * dims in order (keepdims only changes its shape, which is the caller's):
 * 32-bit words for the sum (int32 / uint32 bit patterns, wrapping modulo
 * 2^32 like the int32 accumulation), `type` for the mean. Limits: fewer
 * than 2^31 outputs, fewer than 2^32 elements per output, and at most 2^23
 * elements per mean (the integer sum stays exact in int32); a mean over an
 * empty dim is DQ_ERR_ARG, a sum over one is 0. ReduceSumInteger may zero
 * y before adding into it with atomics: y must not alias x.
 * qlinear_concat: n_inputs tensors xs[j] (HOST array of DEVICE pointers) of
 * rank ndim, shapes in the HOST array shapes[j * ndim + d], equal in every
 * dim but `axis`; x_scales[j] (HOST array of DEVICE pointers to one fp32)
 * and x_zero_points[j] (HOST array of DEVICE pointers, NULL array or NULL
 * entry = 0); y of the joined shape. An input with zero length along axis
 * contributes nothing. One launch per eight inputs.
 * ---------------------------------------------------------------------- */
int qlinear_add(const void* A, int a_ndim, const int64_t* a_shape, const float* a_scale,
                const void* a_zero_point, const void* B, int b_ndim, const int64_t* b_shape,
                const float* b_scale, const void* b_zero_point, const float* c_scale,
                const void* c_zero_point, dq_dtype type, void* C, void* stream);
int qlinear_mul(const void* A, int a_ndim, const int64_t* a_shape, const float* a_scale,
                const void* a_zero_point, const void* B, int b_ndim, const int64_t* b_shape,
                const float* b_scale, const void* b_zero_point, const float* c_scale,
                const void* c_zero_point, dq_dtype type, void* C, void* stream);
int dq_mul_integer(const void* A, int a_ndim, const int64_t* a_shape, const void* a_zero_point,
                   const void* B, int b_ndim, const int64_t* b_shape, const void* b_zero_point,
                   dq_dtype type, int32_t* C, void* stream);
int qlinear_leaky_relu(const void* x, int64_t n, const float* x_scale, const void* x_zero_point,
                       const float* y_scale, const void* y_zero_point, float alpha,
                       dq_dtype type, void* y, void* stream);
int qlinear_sigmoid(const void* x, int64_t n, const float* x_scale, const void* x_zero_point,
                    const float* y_scale, const void* y_zero_point, dq_dtype type, void* y,
                    void* stream);
int dq_reduce_sum_integer(const void* x, dq_dtype type, int ndim, const int64_t* shape,
                          const int32_t* axes, int n_axes, void* y, void* stream);
int qlinear_reduce_mean(const void* x, dq_dtype type, int ndim, const int64_t* shape,
                        const int32_t* axes, int n_axes, const float* x_scale,
                        const void* x_zero_point, const float* y_scale,
                        const void* y_zero_point, void* y, void* stream);
int qlinear_concat(int n_inputs, const void* const* xs, const int64_t* shapes, int ndim,
                   int axis, const float* const* x_scales, const void* const* x_zero_points,
                   const float* y_scale, const void* y_zero_point, dq_dtype type, void* y,
                   void* stream);

/* ------------------------------------------------------------------------
 * DynamicQuantizeLSTM.
 * onnxruntime quantization_defs.cc, schema DynamicQuantizeLSTM (restated on
 * the graiphic.io DynamicQuantizeLSTM page), gives the tensors and
 * attributes; the cell equations are the ONNX LSTM's, which the schema
 * follows. Tensors (dense row-major, fp32 unless said otherwise; dirs = 2
 * for DQ_LSTM_BIDIRECTIONAL, else 1; h = hidden_size; gate blocks of the 4h
 * axis in the order i, o, f, c):
 *   X [seq, batch, input]; W [dirs, input, 4h] and R [dirs, h, 4h] (8-bit);
 *   W_scale / R_scale [dirs] (per tensor) or [dirs, 4h] (per column), zero
 *   points of W's / R's type with the same length (NULL = 0); B [dirs, 8h]
 *   = (Wb, Rb) (NULL = 0); P [dirs, 3h] peepholes i, o, f (NULL = 0);
 *   sequence_lens [batch] int32 (NULL = all seq); initial_h / initial_c
 *   [dirs, batch, h] (NULL = 0); outputs Y [seq, dirs, batch, h], Y_h and
 *   Y_c [dirs, batch, h] (each may be NULL).
 * The library computes (the schema leaves these open; this is the reading):
 *   xw = DynamicQuantizeMatMul(X as [seq * batch, input], W) + Wb, X
 *   quantized per tensor to uint8 once (lo = min(0, min X), hi = max(0,
 *   max X), scale = (hi - lo) / 255, zp = sat(rne(-lo / scale))); at every
 *   step hr = DynamicQuantizeMatMul(H_{s-1} [batch, h], R) + Rb with H
 *   quantized the same way as a whole; each product is
 *   ((float)sum * a_scale) * w_scale[n] + bias[n]. Then, in fp32 with one
 *   rounding per operation:
 *     pre = xw[t] + hr; pre_i += P_i * C_{s-1}; pre_f += P_f * C_{s-1};
 *     i = f(clip(pre_i)); ft = input_forget ? 1 - i : f(clip(pre_f));
 *     g = g(clip(pre_c)); C_s = ft * C_{s-1} + i * g;
 *     pre_o += P_o * C_s; o = f(clip(pre_o)); H_s = o * h(C_s)
 *   with every activation evaluated in fp64 and rounded to fp32 once, and
 *   clip(v) = min(max(v, -clip), clip) for clip > 0 (clip <= 0: none; only
 *   the four gate inputs are clipped). Entry b with length L takes steps
 *   s < L at time t = s (forward) or t = L - 1 - s (reverse) and writes
 *   Y[t]; at steps s >= L its H and C are held (and still enter H's
 *   quantization) and Y[s] = 0. Lengths outside [0, seq] are clamped.
 *   Y_h / Y_c are the state after the last step; a bidirectional LSTM runs
 *   direction 0 forward and direction 1 in reverse, independently. Inputs
 *   are finite fp32 values (a NaN or infinity is not given a meaning).
 *
 * dq_lstm_init: sizes (seq, batch >= 0; 1 <= input <= DQ_QGEMM_K_MAX;
 * 1 <= hidden <= DQ_LSTM_HIDDEN_MAX), direction (DQ_LSTM_*), W / R types
 * (DQ_I8 / DQ_U8), activations (3 * dirs dq_rnn_act values f, g, h per
 * direction; NULL = Sigmoid, Tanh, Tanh), activation_alpha / _beta (3 * dirs
 * values, one per activation slot, used by the activations that take the
 * parameter; NULL = the ONNX defaults: LeakyRelu 0.01, HardSigmoid 0.2 /
 * 0.5, Affine 1 / 0, ThresholdedRelu 1, ScaledTanh 1 / 1, Elu 1. The ONNX
 * attribute lists, consumed in order by the activations that take them,
 * map onto these slots), clip, input_forget. Allocates every device buffer
 * of the context. Errors: DQ_ERR_ARG, DQ_ERR_TYPE, DQ_ERR_RANGE,
 * DQ_ERR_ALLOC, DQ_ERR_HIP.
 * dq_lstm_set_weights: W, R, scales, zero points, B, P as above (DEVICE);
 * packs them into the context and synchronizes `stream`, so the caller may
 * free them on return. Errors: DQ_ERR_STATE, DQ_ERR_ARG, DQ_ERR_ALLOC,
 * DQ_ERR_HIP.
 * dq_lstm_forward: X, sequence_lens, initial_h, initial_c, Y, Y_h, Y_c as
 * above (DEVICE); one call runs the whole sequence, asynchronously on
 * `stream` (calls on one context must not overlap: its state buffers are
 * shared). Errors: DQ_ERR_STATE (no weights, other device), DQ_ERR_ARG,
 * DQ_ERR_HIP.
 * ---------------------------------------------------------------------- */
#define DQ_LSTM_HIDDEN_MAX 4096

typedef enum DQ_ENUM_INT { DQ_LSTM_FORWARD = 0, DQ_LSTM_REVERSE = 1, DQ_LSTM_BIDIRECTIONAL = 2 } dq_lstm_direction;

/* The ONNX RNN activation functions. */
typedef enum DQ_ENUM_INT {
    DQ_RNN_SIGMOID = 0,
    DQ_RNN_TANH = 1,
    DQ_RNN_RELU = 2,
    DQ_RNN_AFFINE = 3,           /* alpha * x + beta */
    DQ_RNN_LEAKY_RELU = 4,       /* x < 0 ? alpha * x : x */
    DQ_RNN_THRESHOLDED_RELU = 5, /* x > alpha ? x : 0 */
    DQ_RNN_SCALED_TANH = 6,      /* alpha * tanh(beta * x) */
    DQ_RNN_HARD_SIGMOID = 7,     /* min(max(alpha * x + beta, 0), 1) */
    DQ_RNN_ELU = 8,              /* x >= 0 ? x : alpha * (e^x - 1) */
    DQ_RNN_SOFTSIGN = 9,         /* x / (1 + |x|) */
    DQ_RNN_SOFTPLUS = 10         /* log(1 + e^x) */
} dq_rnn_act;

typedef struct dq_lstm_ctx dq_lstm_ctx;

int dq_lstm_init(dq_lstm_ctx** ctx, int64_t seq_length, int64_t batch_size, int64_t input_size,
                 int64_t hidden_size, int direction, dq_dtype w_type, dq_dtype r_type,
                 const int* activations, const float* activation_alpha,
                 const float* activation_beta, float clip, int input_forget);
int dq_lstm_set_weights(dq_lstm_ctx* ctx, const void* W, const float* W_scale, int64_t W_scale_len,
                        const void* W_zero_point, const void* R, const float* R_scale,
                        int64_t R_scale_len, const void* R_zero_point, const float* B,
                        const float* P, void* stream);
int dq_lstm_forward(dq_lstm_ctx* ctx, const float* X, const int32_t* sequence_lens,
                    const float* initial_h, const float* initial_c, float* Y, float* Y_h,
                    float* Y_c, void* stream);
/* A short description of the kernels the context runs (owned by it). */
const char* dq_lstm_info(const dq_lstm_ctx* ctx);
/* Frees the context and its device memory; NULL is a no-op. */
void dq_lstm_release(dq_lstm_ctx* ctx);

#ifdef __cplusplus
}
#endif

#endif /* DQIP_H */
