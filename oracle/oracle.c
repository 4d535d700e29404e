/*
 * oracle.c -- plain, slow CPU reference for the dynamic quantized inner
 * product, QuantizeLinear / DequantizeLinear and requantizing QLinearConv.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library. The product
 * library never calls it, includes it or shares a helper, header, table or
 * constant with it.
 *
 * What each function follows (page title, section):
 *  - Simd "SynetDynamicQuantizedInnerProduct16b Class Reference", Detailed
 *    Description: A[i,k] -> uA[i,k], scaleA[i], zeroA[i]; B[k,j] -> iB[k,j],
 *    scaleB[j]; sum over k of (uA - zeroA) * iB; val = sum * scaleA * scaleB;
 *    C = ConvertToTypeC(Activate(val + bias)). Same page, Init(): the
 *    avoidOverflow flag narrows B's range to [-64, 63]; SetParams(): B has
 *    K*N elements, per-output-channel scales for an already quantized B,
 *    bias NULL means zeros.
 *  - onnxruntime quantization_defs.cc, QuantizeLinear doc:
 *    y = saturate(x / y_scale + y_zero_point), x / y_scale rounded to
 *    nearest with ties to even, saturating to [0,255] or [-128,127];
 *    scale / zero point per tensor or per 'axis'.
 *  - same page, DequantizeLinear doc: y = (x - x_zero_point) * x_scale.
 *  - ONNX "QLinearConv" (opset 10), operator description and inputs: bias is
 *    int32, quantized with scale x_scale * w_scale and zero point 0; w scale
 *    and zero point per tensor or per output channel.
 *
 * Where the pages leave a step open, this oracle takes these readings:
 *  R1  uA: asymmetric min/max per row with 0 inside the range:
 *      lo = min(0, min_k A), hi = max(0, max_k A).
 *  R2  scaleA = (hi - lo) / 255 (fp32 subtract, then IEEE fp32 divide).
 *  R3  zeroA = saturate_[0,255](rne(-lo / scaleA)).
 *  R4  an all-zero row (hi == lo) or all-zero column has scale 1.0f and
 *      zero point 0, so every code is the zero point.
 *  R5  B is symmetric: scaleB = max_k |B| / qmax, qmax = 127 (63 with
 *      avoidOverflow), iB = saturate_[qmin,qmax](rne(B / scaleB)),
 *      qmin = -128 (-64).
 *  R6  every dynamic quantizer rounds the IEEE fp32 quotient half-to-even,
 *      as QuantizeLinear does.
 *  R7  the epilogue runs in fp32 in the printed order:
 *      val = ((float)sum * scaleA) * scaleB; val = val + bias; activation;
 *      then fp32 or bf16 (round to nearest even).
 *  R8  activations: identity, relu (val > 0 ? val : 0), leaky relu
 *      (val < 0 ? val * alpha : val).
 *  R11 requantization (QLinearConv): real = ((float)acc * x_scale) * w_scale,
 *      then QuantizeLinear with y_scale / y_zero_point.
 *  - onnxruntime quantization_defs.cc, schemas QGemm, MatMulIntegerToFloat
 *    and DynamicQuantizeMatMul (inputs, types and attributes only; no
 *    formula is printed):
 *  R15 sum[m,n] = sum_k (A[m,k] - a_zp) * (B[k,n] - b_zp[n]); a_scale and a_zp
 *      per tensor; b_scale, b_zp per tensor or per column n (b_zp default 0);
 *      transA / transB select A as (K,M) and B as (N,K).
 *  R16 QGemm's C is int32 with zero point 0 in the scale alpha * a_scale *
 *      b_scale (beta read as 1), so it is added to the integer sum, broadcast
 *      to (M,N) (strides 0 on broadcast axes).
 *  R17 real = ((float)(sum + C) * (alpha * a_scale)) * b_scale[n], alpha *
 *      a_scale rounded to fp32 once; + bias[n] for MatMulIntegerToFloat and
 *      DynamicQuantizeMatMul.
 *  R18 an 8-bit QGemm output: y = saturate(rne(real / y_scale) + y_zp).
 *  R19 DynamicQuantizeMatMul quantizes A per tensor to uint8 with R1-R4 over
 *      the whole tensor, then computes R15 + R17.
 *  - same page, the element-wise quantized operators (QLinearAdd, QLinearMul,
 *    MulInteger, QLinearLeakyRelu, QLinearSigmoid, ReduceSumInteger,
 *    QLinearReduceMean, QLinearConcat), whose docs print the formulas:
 *  R20 fp32 steps in the printed order, each rounded once; "quantize" is
 *      QuantizeLinear's rule (rne of the IEEE quotient, + zero point,
 *      saturate); inputs and output of QLinearAdd / Mul share one 8-bit type.
 *      QLinearAdd: (A_scale*(A-A_zp) + B_scale*(B-B_zp)) / C_scale, + C_zp.
 *      QLinearMul: the integer (A-A_zp)*(B-B_zp) times fl(A_scale*B_scale),
 *      then / C_scale, + C_zp. Numpy (multidirectional) broadcasting.
 *  R21 QLinearSigmoid: dequantize in fp32, 1 / (1 + exp(-x)) evaluated in
 *      fp64 and rounded to fp32 once (so it does not depend on an fp32 exp's
 *      last bit), then quantize.
 *  R22 QLinearReduceMean: the mean of the dequantized elements is taken as
 *      fl32(((double)S * x_scale) / count), S the exact integer sum of
 *      (x - x_zp) (a float sum would depend on its order, which the doc does
 *      not fix), then quantize. ReduceSumInteger: the exact sum, int32 for
 *      int8 input and uint32 for uint8.
 *  R23 QLinearConcat: each input is dequantized with its own scale / zero
 *      point (fp32) and quantized with Y's.
 *  R25 QLinearConv's attributes (the page names kernel size, stride, pad
 *      lengths and group): 2-D, strides, begin / end pads per axis,
 *      dilations (default 1) and groups as in ONNX Conv; a tap outside the
 *      image reads x_zero_point, i.e. a real 0.
 *  R24 fp16 QuantizeLinear / DequantizeLinear (the schemas allow fp16 x,
 *      scales and y): fp16 values are read exactly as fp32 and the fp32
 *      rules apply; an fp16 y is the fp32 result rounded once to nearest
 *      even (the product (x - zp) * s has at most 19 significant bits, so it
 *      is exact in fp32).
 *
 * Arithmetic: fp32 where the pages fix fp32 tensors, IEEE division,
 * nearbyintf in the default round-to-nearest mode for ties-to-even, int64
 * for every integer sum. Built with -O2 -ffp-contract=off and no fast-math,
 * so no product is fused into an add.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>

#define ORC_OK 0
#define ORC_ERR_ARG (-1)
#define ORC_ERR_OVERFLOW (-7)

/* element type tags, as passed by the Python wrapper */
#define ORC_F32 0
#define ORC_BF16 1
#define ORC_I8 2
#define ORC_U8 3

#define ORC_ACT_IDENTITY 0
#define ORC_ACT_RELU 1
#define ORC_ACT_LEAKY 2

/* ---------------------------------------------------------------- helpers */

/* bf16 -> fp32: a bf16 value is the top half of an fp32 bit pattern. */
float oracle_bf16_to_f32(uint16_t b)
{
    union { uint32_t u; float f; } v;
    v.u = (uint32_t)b << 16;
    return v.f;
}

/* fp32 -> bf16, round to nearest, ties to even, on the dropped 16 bits. */
uint16_t oracle_f32_to_bf16(float f)
{
    union { uint32_t u; float f; } v;
    v.f = f;
    if (isnan(f)) return (uint16_t)((v.u >> 16) | 0x40u);
    uint32_t upper = v.u >> 16;
    uint32_t lower = v.u & 0xFFFFu;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;
    return (uint16_t)upper;
}

/* IEEE binary16 -> fp32 (exact): sign, 5-bit exponent (bias 15), 10-bit
 * fraction; exponent 0 is zero / subnormal (fraction * 2^-24), 31 is
 * inf / NaN. */
float oracle_f16_to_f32(uint16_t h)
{
    int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    float v;
    if (e == 0) v = ldexpf((float)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexpf((float)(1024 + m), e - 25);
    return sign ? -v : v;
}

/* fp32 -> binary16, round to nearest, ties to even; beyond the largest
 * finite value (65504) by half an ulp or more -> inf; NaN -> quiet NaN. The
 * scaled magnitudes below are exact in double. */
uint16_t oracle_f32_to_f16(float f)
{
    uint16_t sign = signbit(f) ? 0x8000u : 0;
    if (isnan(f)) return (uint16_t)(sign | 0x7e00u);
    if (isinf(f)) return (uint16_t)(sign | 0x7c00u);
    double a = fabs((double)f);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);  /* a = frac * 2^e, frac in [0.5, 1) */
    e -= 1;        /* a in [2^e, 2^(e+1)) */
    if (e < -14) { /* subnormal range: units of 2^-24 */
        double q = nearbyint(ldexp(a, 24));
        return (uint16_t)(sign | (uint16_t)q); /* q == 1024 is the smallest normal */
    }
    double q = nearbyint(ldexp(a, 10 - e)); /* in [1024, 2048] */
    if (q == 2048.0) { q = 1024.0; e += 1; }
    if (e + 15 >= 31) return (uint16_t)(sign | 0x7c00u);
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(q - 1024.0));
}

void oracle_f16_to_f32_array(const uint16_t* h, int64_t n, float* f)
{
    for (int64_t i = 0; i < n; ++i) f[i] = oracle_f16_to_f32(h[i]);
}

void oracle_f32_to_f16_array(const float* f, int64_t n, uint16_t* h)
{
    for (int64_t i = 0; i < n; ++i) h[i] = oracle_f32_to_f16(f[i]);
}

/* round half to even (nearbyintf uses the current mode, which is the C
 * default round-to-nearest-even; nothing here changes it) */
static float rne(float v) { return nearbyintf(v); }

/* saturate an integral float plus an integer offset into [lo, hi]; done in
 * double, where rne(x)+zp is exact, so +-inf and huge values saturate too */
static int sat_add(float r, int zp, int lo, int hi)
{
    double v = (double)r + (double)zp;
    if (v < (double)lo) return lo;
    if (v > (double)hi) return hi;
    return (int)v;
}

static float load_real(const void* p, int type, int64_t idx)
{
    if (type == ORC_BF16) return oracle_bf16_to_f32(((const uint16_t*)p)[idx]);
    return ((const float*)p)[idx];
}

static int load_int8(const void* p, int type, int64_t idx)
{
    if (type == ORC_U8) return ((const uint8_t*)p)[idx];
    return ((const int8_t*)p)[idx];
}

static void store_int8(void* p, int type, int64_t idx, int v)
{
    if (type == ORC_U8) ((uint8_t*)p)[idx] = (uint8_t)v;
    else ((int8_t*)p)[idx] = (int8_t)v;
}

static int64_t inner_size(int ndim, const int64_t* shape, int axis)
{
    int64_t inner = 1;
    for (int d = axis + 1; d < ndim; ++d) inner *= shape[d];
    return inner;
}

static int64_t total_size(int ndim, const int64_t* shape)
{
    int64_t n = 1;
    for (int d = 0; d < ndim; ++d) n *= shape[d];
    return n;
}

/* ------------------------------------------------------- QuantizeLinear */

/* y = saturate(rne(x / scale[c]) + zp[c]); c = 0 per tensor (axis < 0),
 * else the index along 'axis'. y_type is ORC_I8 or ORC_U8. */
int oracle_quantize_linear(const float* x, int ndim, const int64_t* shape,
                           int axis, const float* scale, const int32_t* zp,
                           int y_type, void* y)
{
    if (axis >= ndim) return ORC_ERR_ARG;
    int lo = (y_type == ORC_U8) ? 0 : -128;
    int hi = (y_type == ORC_U8) ? 255 : 127;
    int64_t n = total_size(ndim, shape);
    int64_t inner = axis < 0 ? n : inner_size(ndim, shape, axis);
    int64_t cdim = axis < 0 ? 1 : shape[axis];
    for (int64_t idx = 0; idx < n; ++idx) {
        int64_t c = axis < 0 ? 0 : (idx / inner) % cdim;
        float q = x[idx] / scale[c];
        store_int8(y, y_type, idx, sat_add(rne(q), zp[c], lo, hi));
    }
    return ORC_OK;
}

/* ----------------------------------------------------- DequantizeLinear */

/* y = (float)(x - zp[c]) * scale[c]; x_type is ORC_I8 or ORC_U8. */
int oracle_dequantize_linear(const void* x, int x_type, int ndim,
                             const int64_t* shape, int axis,
                             const float* scale, const int32_t* zp, float* y)
{
    if (axis >= ndim) return ORC_ERR_ARG;
    int64_t n = total_size(ndim, shape);
    int64_t inner = axis < 0 ? n : inner_size(ndim, shape, axis);
    int64_t cdim = axis < 0 ? 1 : shape[axis];
    for (int64_t idx = 0; idx < n; ++idx) {
        int64_t c = axis < 0 ? 0 : (idx / inner) % cdim;
        int d = load_int8(x, x_type, idx) - zp[c];
        y[idx] = (float)d * scale[c];
    }
    return ORC_OK;
}

/* ------------------------------------------- dynamic quantization of A */

/* One row of A -> uA row, scaleA, zeroA (readings R1-R4, R6). */
static void quantize_row(const void* A, int typeA, int64_t K, int64_t i,
                         uint8_t* u, float* scale_out, int32_t* zero_out)
{
    float lo = 0.0f, hi = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
        float a = load_real(A, typeA, i * K + k);
        if (a < lo) lo = a;
        if (a > hi) hi = a;
    }
    float scale;
    int zero;
    if (hi == lo) {
        scale = 1.0f;
        zero = 0;
    } else {
        scale = (hi - lo) / 255.0f;
        zero = sat_add(rne(-lo / scale), 0, 0, 255);
    }
    for (int64_t k = 0; k < K; ++k) {
        float a = load_real(A, typeA, i * K + k);
        u[k] = (uint8_t)sat_add(rne(a / scale), zero, 0, 255);
    }
    *scale_out = scale;
    *zero_out = zero;
}

/* rows: indices of the rows to quantize (NULL = all M rows, nrows = M).
 * uA is [nrows, K]; scaleA, zeroA are [nrows]. */
int oracle_quantize_rows(const void* A, int typeA, int64_t M, int64_t K,
                         const int64_t* rows, int64_t nrows, uint8_t* uA,
                         float* scaleA, int32_t* zeroA)
{
    if (typeA != ORC_F32 && typeA != ORC_BF16) return ORC_ERR_ARG;
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t i = rows ? rows[r] : r;
        if (i < 0 || i >= M) return ORC_ERR_ARG;
        quantize_row(A, typeA, K, i, uA + r * K, &scaleA[r], &zeroA[r]);
    }
    return ORC_OK;
}

/* ------------------------------------------- dynamic quantization of B */

/* B [K,N] row-major -> iB [K,N], scaleB [N] (readings R4-R6). */
int oracle_quantize_cols(const void* B, int typeB, int64_t K, int64_t N,
                         int avoidOverflow, int8_t* iB, float* scaleB)
{
    if (typeB != ORC_F32 && typeB != ORC_BF16) return ORC_ERR_ARG;
    int qmax = avoidOverflow ? 63 : 127;
    int qmin = avoidOverflow ? -64 : -128;
    for (int64_t j = 0; j < N; ++j) {
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float b = fabsf(load_real(B, typeB, k * N + j));
            if (b > amax) amax = b;
        }
        float scale = amax > 0.0f ? amax / (float)qmax : 1.0f;
        for (int64_t k = 0; k < K; ++k) {
            float b = load_real(B, typeB, k * N + j);
            iB[k * N + j] = (int8_t)sat_add(rne(b / scale), 0, qmin, qmax);
        }
        scaleB[j] = scale;
    }
    return ORC_OK;
}

/* ReduceSumInteger of iB over axis 0: colsum[j] = sum_k iB[k,j]. */
int oracle_colsum(const int8_t* iB, int64_t K, int64_t N, int32_t* colsum)
{
    for (int64_t j = 0; j < N; ++j) {
        int64_t s = 0;
        for (int64_t k = 0; k < K; ++k) s += iB[k * N + j];
        colsum[j] = (int32_t)s;
    }
    return ORC_OK;
}

/* -------------------------------------------------- integer inner product */

/* acc[r,j] = sum_k (uA[r,k] - zeroA[r]) * iB[k,j], in int64; fails if a
 * result does not fit int32. */
int oracle_int_gemm(const uint8_t* uA, const int32_t* zeroA, const int8_t* iB,
                    int64_t M, int64_t N, int64_t K, int32_t* acc)
{
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            int64_t sum = 0;
            for (int64_t k = 0; k < K; ++k)
                sum += ((int64_t)uA[i * K + k] - zeroA[i]) * iB[k * N + j];
            if (sum > INT32_MAX || sum < INT32_MIN) return ORC_ERR_OVERFLOW;
            acc[i * N + j] = (int32_t)sum;
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------ epilogue */

static float activate(float v, int act, float alpha)
{
    if (act == ORC_ACT_RELU) return v > 0.0f ? v : 0.0f;
    if (act == ORC_ACT_LEAKY) return v < 0.0f ? v * alpha : v;
    return v;
}

/* C[r,j] = Convert(Activate(((float)acc * scaleA[r]) * scaleB[j] (+ bias[j])))
 * has_bias = 0 skips the add; has_bias = 1 with bias NULL adds zeros. */
int oracle_epilogue(const int32_t* acc, const float* scaleA,
                    const float* scaleB, int has_bias, const float* bias,
                    int act, float alpha, int64_t M, int64_t N, int typeC,
                    void* C)
{
    if (typeC != ORC_F32 && typeC != ORC_BF16) return ORC_ERR_ARG;
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            float val = (float)acc[i * N + j] * scaleA[i];
            val = val * scaleB[j];
            if (has_bias) val = val + (bias ? bias[j] : 0.0f);
            val = activate(val, act, alpha);
            if (typeC == ORC_BF16)
                ((uint16_t*)C)[i * N + j] = oracle_f32_to_bf16(val);
            else
                ((float*)C)[i * N + j] = val;
        }
    }
    return ORC_OK;
}

/* --------------------------------------------- the whole forward pass */

/*
 * Forward over the selected rows of A (rows NULL = all M rows).
 * typeB: ORC_F32 / ORC_BF16 (quantized here, per column) or ORC_I8 (already
 * quantized; scaleB_in gives its per-column scales).
 * Optional outputs (NULL to skip): uA [nrows,K], scaleA/zeroA [nrows],
 * iB [K,N], scaleB [N], acc [nrows,N]. C is [nrows,N] of typeC.
 * The caller provides work_uA [nrows*K], work_iB [K*N] (when typeB is not
 * I8), work_acc [nrows*N], work_scaleB [N] and work_sz [2*nrows] when it
 * does not ask for the matching optional output.
 */
int oracle_dqip_forward(const void* A, int typeA, const void* B, int typeB,
                        const float* scaleB_in, int64_t M, int64_t N, int64_t K,
                        const int64_t* rows, int64_t nrows, int avoidOverflow,
                        int has_bias, const float* bias, int act, float alpha,
                        int typeC, void* C, uint8_t* uA, float* scaleA,
                        int32_t* zeroA, int8_t* iB, float* scaleB, int32_t* acc)
{
    if (!A || !B || !C || !uA || !scaleA || !zeroA || !iB || !scaleB || !acc)
        return ORC_ERR_ARG;
    int rc = oracle_quantize_rows(A, typeA, M, K, rows, nrows, uA, scaleA, zeroA);
    if (rc) return rc;
    if (typeB == ORC_I8) {
        const int8_t* b = (const int8_t*)B;
        for (int64_t t = 0; t < K * N; ++t) iB[t] = b[t];
        for (int64_t j = 0; j < N; ++j) scaleB[j] = scaleB_in[j];
    } else {
        rc = oracle_quantize_cols(B, typeB, K, N, avoidOverflow, iB, scaleB);
        if (rc) return rc;
    }
    rc = oracle_int_gemm(uA, zeroA, iB, nrows, N, K, acc);
    if (rc) return rc;
    return oracle_epilogue(acc, scaleA, scaleB, has_bias, bias, act, alpha,
                           nrows, N, typeC, C);
}

/* -------------------------------------------------------- QLinearConv */

/*
 * 2-D QLinearConv, stride 1, no padding, no dilation, group 1.
 * x [Nb, C, H, W] (x_type I8/U8), w [M, C, kH, kW] (w_type I8/U8),
 * w_scale / w_zp of length w_len (1 = per tensor, M = per output channel),
 * bias [M] int32 or NULL, y [Nb, M, H-kH+1, W-kW+1] (y_type I8/U8).
 * acc = sum (w - w_zp) * (x - x_zp) + bias;
 * real = ((float)acc * x_scale) * w_scale[m];  y = QuantizeLinear(real).
 */
int oracle_qlinear_conv(const void* x, int x_type, int64_t Nb, int64_t C,
                        int64_t H, int64_t W, float x_scale, int32_t x_zp,
                        const void* w, int w_type, int64_t M, int64_t kH,
                        int64_t kW, const float* w_scale, const int32_t* w_zp,
                        int64_t w_len, const int32_t* bias, float y_scale,
                        int32_t y_zp, int y_type, void* y)
{
    if (kH > H || kW > W || (w_len != 1 && w_len != M)) return ORC_ERR_ARG;
    int64_t oH = H - kH + 1, oW = W - kW + 1;
    int lo = (y_type == ORC_U8) ? 0 : -128;
    int hi = (y_type == ORC_U8) ? 255 : 127;
    for (int64_t n = 0; n < Nb; ++n)
        for (int64_t m = 0; m < M; ++m) {
            int64_t wi = (w_len == 1) ? 0 : m;
            for (int64_t oh = 0; oh < oH; ++oh)
                for (int64_t ow = 0; ow < oW; ++ow) {
                    int64_t acc = 0;
                    for (int64_t c = 0; c < C; ++c)
                        for (int64_t r = 0; r < kH; ++r)
                            for (int64_t s = 0; s < kW; ++s) {
                                int64_t xi = ((n * C + c) * H + oh + r) * W + ow + s;
                                int64_t wk = ((m * C + c) * kH + r) * kW + s;
                                acc += (int64_t)(load_int8(w, w_type, wk) - w_zp[wi]) *
                                       (load_int8(x, x_type, xi) - x_zp);
                            }
                    if (bias) acc += bias[m];
                    if (acc > INT32_MAX || acc < INT32_MIN) return ORC_ERR_OVERFLOW;
                    float real = (float)(int32_t)acc * x_scale;
                    real = real * w_scale[wi];
                    float q = real / y_scale;
                    int64_t yi = ((n * M + m) * oH + oh) * oW + ow;
                    store_int8(y, y_type, yi, sat_add(rne(q), y_zp, lo, hi));
                }
        }
    return ORC_OK;
}

/* General 2-D QLinearConv (ONNX QLinearConv, opset 10): x [Nb, C, H, W],
 * w [M, C / group, kH, kW], y [Nb, M, oH, oW] with
 *   oH = (H + pad_t + pad_b - dil_h (kH - 1) - 1) / stride_h + 1 (floor),
 * likewise oW. Output channel m belongs to group g = m / (M / group) and
 * reads input channels g (C / group) .. +C / group. A tap outside the image
 * reads x_zp (R25: a padded input is a real 0, so it adds nothing), then R11
 * requantizes. acc_out (optional) receives the int32 sums with the bias. */
int oracle_qlinear_conv2d(const void* x, int x_type, int64_t Nb, int64_t C, int64_t H, int64_t W,
                          float x_scale, int32_t x_zp, const void* w, int w_type, int64_t M,
                          int64_t kH, int64_t kW, int64_t stride_h, int64_t stride_w,
                          int64_t pad_t, int64_t pad_l, int64_t pad_b, int64_t pad_r,
                          int64_t dil_h, int64_t dil_w, int64_t group, const float* w_scale,
                          const int32_t* w_zp, int64_t w_len, const int32_t* bias, float y_scale,
                          int32_t y_zp, int y_type, void* y, int32_t* acc_out)
{
    if (group < 1 || C % group || M % group || stride_h < 1 || stride_w < 1 || dil_h < 1 ||
        dil_w < 1 || (w_len != 1 && w_len != M))
        return ORC_ERR_ARG;
    int64_t oH = (H + pad_t + pad_b - dil_h * (kH - 1) - 1) / stride_h + 1;
    int64_t oW = (W + pad_l + pad_r - dil_w * (kW - 1) - 1) / stride_w + 1;
    if (oH < 1 || oW < 1) return ORC_ERR_ARG;
    int64_t Cg = C / group, Mg = M / group;
    int lo = (y_type == ORC_U8) ? 0 : -128;
    int hi = (y_type == ORC_U8) ? 255 : 127;
    for (int64_t n = 0; n < Nb; ++n)
        for (int64_t m = 0; m < M; ++m) {
            int64_t g = m / Mg;
            int64_t wi = (w_len == 1) ? 0 : m;
            for (int64_t oh = 0; oh < oH; ++oh)
                for (int64_t ow = 0; ow < oW; ++ow) {
                    int64_t acc = 0;
                    for (int64_t c = 0; c < Cg; ++c)
                        for (int64_t r = 0; r < kH; ++r)
                            for (int64_t s = 0; s < kW; ++s) {
                                int64_t ih = oh * stride_h - pad_t + r * dil_h;
                                int64_t iw = ow * stride_w - pad_l + s * dil_w;
                                int xv = x_zp;
                                if (ih >= 0 && ih < H && iw >= 0 && iw < W)
                                    xv = load_int8(x, x_type, ((n * C + g * Cg + c) * H + ih) * W + iw);
                                int64_t wk = ((m * Cg + c) * kH + r) * kW + s;
                                acc += (int64_t)(load_int8(w, w_type, wk) - w_zp[wi]) * (xv - x_zp);
                            }
                    if (bias) acc += bias[m];
                    if (acc > INT32_MAX || acc < INT32_MIN) return ORC_ERR_OVERFLOW;
                    int64_t yi = ((n * M + m) * oH + oh) * oW + ow;
                    if (acc_out) acc_out[yi] = (int32_t)acc;
                    float real = (float)(int32_t)acc * x_scale;
                    real = real * w_scale[wi];
                    float q = real / y_scale;
                    store_int8(y, y_type, yi, sat_add(rne(q), y_zp, lo, hi));
                }
        }
    return ORC_OK;
}

/* --------------------------------------------------- QGemm family (R15-R19) */

/* The whole tensor A (n values) to uint8 with one scale and zero point: R1-R4
 * applied to all of A at once (R19). */
int oracle_quantize_tensor_u8(const float* A, int64_t n, float* scale, int32_t* zp, uint8_t* q)
{
    float lo = 0.0f, hi = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        if (A[i] < lo) lo = A[i];
        if (A[i] > hi) hi = A[i];
    }
    float s = 1.0f;
    int z = 0;
    if (hi != lo) {
        float range = hi - lo;
        s = range / 255.0f;
        z = sat_add(rne(-lo / s), 0, 0, 255);
    }
    for (int64_t i = 0; i < n; ++i) q[i] = (uint8_t)sat_add(rne(A[i] / s), z, 0, 255);
    *scale = s;
    *zp = z;
    return ORC_OK;
}

/* R15-R18. A is (M,K) row-major, or (K,M) with transA; B is (K,N), or (N,K)
 * with transB. b_scale / b_zp have 1 or N entries (b_zp NULL: 0). C (NULL:
 * none) is read at m * c_rs + n * c_cs. y_type ORC_F32 gives float Y;
 * ORC_U8 / ORC_I8 requantize with y_scale / y_zp. acc_out (optional)
 * receives sum + C as int32. Returns ORC_ERR_OVERFLOW when sum + C leaves
 * int32. */
int oracle_qgemm(const void* A, int a_type, int transA, int64_t M, int64_t K, float a_scale,
                 int32_t a_zp, const void* B, int b_type, int transB, int64_t N,
                 const float* b_scale, int64_t b_scale_len, const int32_t* b_zp,
                 int64_t b_zp_len, const int32_t* Cm, int64_t c_rs, int64_t c_cs, float alpha,
                 const float* bias, int y_type, float y_scale, int32_t y_zp, void* Y,
                 int32_t* acc_out)
{
    if ((b_scale_len != 1 && b_scale_len != N) || (b_zp && b_zp_len != 1 && b_zp_len != N))
        return ORC_ERR_ARG;
    float sa = alpha * a_scale;
    int lo = (y_type == ORC_U8) ? 0 : -128;
    int hi = (y_type == ORC_U8) ? 255 : 127;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            int32_t zb = b_zp ? b_zp[b_zp_len == 1 ? 0 : n] : 0;
            int64_t sum = 0;
            for (int64_t k = 0; k < K; ++k) {
                int64_t ai = transA ? k * M + m : m * K + k;
                int64_t bi = transB ? n * K + k : k * N + n;
                sum += (int64_t)(load_int8(A, a_type, ai) - a_zp) * (load_int8(B, b_type, bi) - zb);
            }
            if (Cm) sum += Cm[m * c_rs + n * c_cs];
            if (sum > INT32_MAX || sum < INT32_MIN) return ORC_ERR_OVERFLOW;
            if (acc_out) acc_out[m * N + n] = (int32_t)sum;
            float real = (float)(int32_t)sum * sa;
            real = real * b_scale[b_scale_len == 1 ? 0 : n];
            if (bias) real = real + bias[n];
            if (y_type == ORC_F32)
                ((float*)Y)[m * N + n] = real;
            else
                store_int8(Y, y_type, m * N + n, sat_add(rne(real / y_scale), y_zp, lo, hi));
        }
    return ORC_OK;
}

/* ------------------------------------------ element-wise family (R20-R23) */

#define ORC_MAXD 8

/* numpy broadcasting of two shapes; returns ORC_ERR_ARG when they do not
 * broadcast. */
int oracle_broadcast_shape(int na, const int64_t* sa, int nb, const int64_t* sb, int* ny, int64_t* sy)
{
    int n = na > nb ? na : nb;
    if (n > ORC_MAXD) return ORC_ERR_ARG;
    for (int d = 0; d < n; ++d) {
        int64_t a = d - (n - na) >= 0 ? sa[d - (n - na)] : 1;
        int64_t b = d - (n - nb) >= 0 ? sb[d - (n - nb)] : 1;
        if (a != b && a != 1 && b != 1) return ORC_ERR_ARG;
        sy[d] = a == 1 ? b : a;
    }
    *ny = n;
    return ORC_OK;
}

/* offset in a tensor of shape s (ns dims, right-aligned against the output
 * of ny dims) of the output coordinate c (size-1 dims broadcast) */
static int64_t bcast_offset(const int64_t* c, int ny, int ns, const int64_t* s)
{
    int64_t off = 0;
    for (int d = 0; d < ns; ++d) {
        int64_t cd = c[d + (ny - ns)];
        off = off * s[d] + (s[d] == 1 ? 0 : cd);
    }
    return off;
}

static int quantize_f(float v, float y_scale, int y_zp, int y_type)
{
    int lo = (y_type == ORC_U8) ? 0 : -128;
    int hi = (y_type == ORC_U8) ? 255 : 127;
    return sat_add(rne(v / y_scale), y_zp, lo, hi);
}

/* op 0: QLinearAdd, 1: QLinearMul (Y of the inputs' 8-bit type t),
 *    2: MulInteger (int32 Y; scales unused). */
int oracle_qlinear_binary(int op, int t, const void* A, int na, const int64_t* sa, float a_scale, int32_t a_zp,
                          const void* B, int nb, const int64_t* sb, float b_scale, int32_t b_zp,
                          float c_scale, int32_t c_zp, void* Y)
{
    int ny;
    int64_t sy[ORC_MAXD], c[ORC_MAXD];
    if (oracle_broadcast_shape(na, sa, nb, sb, &ny, sy)) return ORC_ERR_ARG;
    int64_t n = total_size(ny, sy);
    float ab = a_scale * b_scale;
    for (int64_t i = 0; i < n; ++i) {
        int64_t r = i;
        for (int d = ny - 1; d >= 0; --d) {
            c[d] = r % sy[d];
            r /= sy[d];
        }
        int32_t a = load_int8(A, t, bcast_offset(c, ny, na, sa)) - a_zp;
        int32_t b = load_int8(B, t, bcast_offset(c, ny, nb, sb)) - b_zp;
        if (op == 2) {
            ((int32_t*)Y)[i] = a * b;
        } else if (op == 0) {
            float fa = (float)a * a_scale;
            float fb = (float)b * b_scale;
            float v = fa + fb;
            store_int8(Y, t, i, quantize_f(v, c_scale, c_zp, t));
        } else {
            float v = (float)(a * b) * ab;
            store_int8(Y, t, i, quantize_f(v, c_scale, c_zp, t));
        }
    }
    return ORC_OK;
}

/* op 0: QLinearLeakyRelu (alpha), 1: QLinearSigmoid; X and Y of type t. */
int oracle_qlinear_unary(int op, int t, const void* X, int64_t n, float x_scale, int32_t x_zp,
                         float y_scale, int32_t y_zp, float alpha, void* Y)
{
    for (int64_t i = 0; i < n; ++i) {
        float x = (float)(load_int8(X, t, i) - x_zp) * x_scale;
        float v;
        if (op == 0)
            v = x < 0.0f ? alpha * x : x;
        else
            v = (float)(1.0 / (1.0 + exp(-(double)x)));
        store_int8(Y, t, i, quantize_f(v, y_scale, y_zp, t));
    }
    return ORC_OK;
}

/* Reduction of X (ndim dims of shape s) over the dims whose bit is set in
 * axes_mask; the output holds the kept dims in order (keepdims only changes
 * the shape). op 0: ReduceSumInteger (Y int32 for int8 input, uint32 for
 * uint8: written as 32-bit words), 1: QLinearReduceMean (Y of type t). */
int oracle_reduce(int op, int t, const void* X, int ndim, const int64_t* s, int axes_mask,
                  float x_scale, int32_t x_zp, float y_scale, int32_t y_zp, void* Y)
{
    if (ndim < 1 || ndim > ORC_MAXD) return ORC_ERR_ARG;
    int64_t nout = 1, count = 1;
    for (int d = 0; d < ndim; ++d) {
        if (axes_mask & (1 << d)) count *= s[d];
        else nout *= s[d];
    }
    int64_t n = total_size(ndim, s);
    int64_t c[ORC_MAXD];
    int64_t* acc = (int64_t*)calloc((size_t)(nout > 0 ? nout : 1), sizeof(int64_t));
    if (!acc) return ORC_ERR_ARG;
    for (int64_t i = 0; i < n; ++i) {
        int64_t r = i;
        for (int d = ndim - 1; d >= 0; --d) {
            c[d] = r % s[d];
            r /= s[d];
        }
        int64_t o = 0;
        for (int d = 0; d < ndim; ++d)
            if (!(axes_mask & (1 << d))) o = o * s[d] + c[d];
        acc[o] += load_int8(X, t, i) - (op == 1 ? x_zp : 0);
    }
    for (int64_t o = 0; o < nout; ++o) {
        if (op == 0) {
            if (t == ORC_U8) ((uint32_t*)Y)[o] = (uint32_t)acc[o];
            else ((int32_t*)Y)[o] = (int32_t)acc[o];
        } else {
            float mean = (float)(((double)acc[o] * (double)x_scale) / (double)count);
            store_int8(Y, t, o, quantize_f(mean, y_scale, y_zp, t));
        }
    }
    free(acc);
    return ORC_OK;
}

/* QLinearConcat of n_in tensors of type t along axis: input j has the
 * shape of Y except dim `axis`, which is lens[j]; outer / inner are the
 * products of Y's dims before / after axis. */
int oracle_qlinear_concat(int t, int n_in, const void* const* xs, const int64_t* lens,
                          const float* scales, const int32_t* zps, int64_t outer, int64_t inner,
                          float y_scale, int32_t y_zp, void* Y)
{
    int64_t total = 0;
    for (int j = 0; j < n_in; ++j) total += lens[j];
    for (int64_t o = 0; o < outer; ++o) {
        int64_t base = 0;
        for (int j = 0; j < n_in; ++j) {
            for (int64_t k = 0; k < lens[j] * inner; ++k) {
                float x = (float)(load_int8(xs[j], t, o * lens[j] * inner + k) - zps[j]) * scales[j];
                store_int8(Y, t, (o * total + base) * inner + k, quantize_f(x, y_scale, y_zp, t));
            }
            base += lens[j];
        }
    }
    return ORC_OK;
}
