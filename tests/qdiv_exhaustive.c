/* qdiv_exhaustive.c -- exhaustive CPU check of the quantizers' division.
 *
 * Test infrastructure, not part of the library: it restates, in plain C on
 * the host, the fp32 operation sequences the gfx950 kernels use to turn
 * x / s into a quantized code, and compares each with the definition the
 * ONNX Runtime QuantizeLinear schema gives (the IEEE quotient rounded to
 * nearest, ties to even, plus the zero point, saturated to the type's range),
 * over every fp32 bit pattern x (NaNs excluded), for each scale s given on
 * the command line as a hexadecimal bit pattern.
 *
 * The sequences (y = RN(1/s) computed once per scale; all products and sums
 * rounded to nearest; fma fused; M = 1.5 * 2^23; med3 = median of three):
 *   residual   q0 = RN(x*y); r = fma(-q0, s, x); q = fma(r, y, q0)
 *              (Markstein's correction step)
 *   F1 bounded q = residual(x); t = med3(q + M, M + lo - zp, M + hi - zp)
 *              (used where |x/s| is bounded by construction: rows of A,
 *              columns of B, an 8-bit operand packed with a tensor scale)
 *   F2 clamped q0 = med3(RN(x*y), -2^22, 2^22); r = fma(-q0, s, x);
 *              t = med3(fma(r, y, q0) + M, M + lo - zp, M + hi - zp)
 *              (QuantizeLinear, every requantizing epilogue)
 *   F3 generic q = residual(x) unless |q0| > 2^24 (then q = q0);
 *              code = clamp(rne(q), lo - zp, hi - zp) + zp
 * The code of F1 / F2 is the low byte of t's bits (t = M + k holds k in
 * its low mantissa bits) added bytewise to the zero point. The kernels take
 * these forms only when make_qdiv's test passes (|s| >= 2^-100 and 1/s a
 * normal number); any other scale takes the IEEE division, which is the
 * definition itself. That gating is restated here too.
 *
 * Output, one line per scale:
 *   s=<bits> fast=<0|1> n=<x tested> qmis=<quotient != IEEE quotient with
 *   |x/s| >= 1/4> f1=<code mismatches> f2=<...> f3=<...>
 * Build: gcc -O2 -ffp-contract=off -mfma -msse4.1 -fopenmp (no fast-math:
 * `/` must stay the correctly rounded IEEE division; SSE4.1 makes rintf one
 * round-to-nearest-even instruction).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static inline float f_of(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
/* median of a and the bounds lo <= hi (no NaN reaches it) */
static inline float med3(float a, float lo, float hi) { return a < lo ? lo : (a > hi ? hi : a); }

/* the definition: clamp(rne(x / s) + zp) in the float domain (an overflowed
 * quotient is +-inf and saturates); rq = rne(x / s) */
static inline int code_ref(float rq, int lo, int hi, int zp) {
    return (int)med3(rq + (float)zp, (float)lo, (float)hi);
}

/* M + k -> (k + zp) wrapped to a byte, read back as the signed / unsigned type */
static inline int code_from_magic(float t, int lo, int zp) {
    int32_t bits;
    memcpy(&bits, &t, 4);
    const uint32_t byte = ((uint32_t)bits + (uint32_t)zp) & 0xffu;
    return lo < 0 ? (int)(int8_t)byte : (int)byte;
}

/* one row of 2^16 consecutive bit patterns; branch-free so that it
 * vectorizes (a NaN x is computed through and masked out of the counts) */
static inline void sweep16(uint32_t hi16, float s, float y, int fast, long long cnt[5]) {
    const float M = 12582912.0f, BIG = 4194304.0f;
    long long n = 0, qmis = 0, f1 = 0, f2 = 0, f3 = 0;
    for (uint32_t lo16 = 0; lo16 < 65536; ++lo16) {
        const float x = f_of((hi16 << 16) | lo16);
        const int valid = x == x;
        const float ref = x / s;
        const float q0 = x * y;
        const float res = fmaf(fmaf(-q0, s, x), y, q0);
        const int in24 = fabsf(q0) <= 16777216.0f;
        const float q0c = med3(q0, -BIG, BIG);
        const float t2 = fmaf(fmaf(-q0c, s, x), y, q0c) + M;
        const float q3 = in24 ? res : q0;
        const float rref = rintf(ref), r3 = rintf(q3);
        /* F1 only where |x/s| is bounded (the kernels that use it guarantee
         * |x/s| <= 255) */
        const int bounded = fabsf(q0) <= 2097152.0f;
        n += valid;
        qmis += valid & fast & in24 & (fabsf(ref) >= 0.25f) & (res != ref);
#define DQ_CFG(LO, HI, ZP)                                                                       \
        {                                                                                        \
            const int want = code_ref(rref, LO, HI, ZP);                                         \
            const float lof = M + (float)(LO - ZP), hif = M + (float)(HI - ZP);                  \
            int g1, g2, g3;                                                                      \
            if (fast) {                                                                          \
                g1 = code_from_magic(med3(res + M, lof, hif), LO, ZP);                           \
                g2 = code_from_magic(med3(t2, lof, hif), LO, ZP);                                \
                g3 = (int)med3(r3, (float)(LO - ZP), (float)(HI - ZP)) + ZP;                     \
            } else { /* the IEEE division, as the kernels take it */                             \
                g1 = code_from_magic(M + med3(rref, (float)(LO - ZP), (float)(HI - ZP)), LO, ZP); \
                g2 = code_from_magic(med3(med3(ref, -BIG, BIG) + M, lof, hif), LO, ZP);          \
                g3 = (int)med3(rref, (float)(LO - ZP), (float)(HI - ZP)) + ZP;                   \
            }                                                                                    \
            f1 += valid & bounded & (g1 != want);                                                \
            f2 += valid & (g2 != want);                                                          \
            f3 += valid & (g3 != want);                                                          \
        }
        /* int8 and uint8, zero points at, off and far from the middle */
        DQ_CFG(-128, 127, 0)
        DQ_CFG(-128, 127, -10)
        DQ_CFG(0, 255, 128)
        DQ_CFG(0, 255, 3)
#undef DQ_CFG
    }
    cnt[0] += n; cnt[1] += qmis; cnt[2] += f1; cnt[3] += f2; cnt[4] += f3;
}

int main(int argc, char** argv) {
    for (int a = 1; a < argc; ++a) {
        const uint32_t sb = (uint32_t)strtoul(argv[a], NULL, 16);
        const float s = f_of(sb);
        const float y = 1.0f / s;
        const int fast = fabsf(s) >= 0x1p-100f && fabsf(y) >= 1.17549435e-38f && fabsf(y) <= 3.40282347e+38f;
        long long n = 0, qmis = 0, f1 = 0, f2 = 0, f3 = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : n, qmis, f1, f2, f3)
        for (int hi16 = 0; hi16 < 65536; ++hi16) {
            long long c[5] = {0, 0, 0, 0, 0};
            if (fast) sweep16((uint32_t)hi16, s, y, 1, c);
            else sweep16((uint32_t)hi16, s, y, 0, c);
            n += c[0]; qmis += c[1]; f1 += c[2]; f2 += c[3]; f3 += c[4];
        }
        printf("s=%08x fast=%d n=%lld qmis=%lld f1=%lld f2=%lld f3=%lld\n", sb, fast, n, qmis, f1, f2, f3);
        fflush(stdout);
    }
    return 0;
}
