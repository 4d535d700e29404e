// quant_row_dev.h -- device code that quantizes one row of A in registers
// (internal; shared by the row-quantization kernels and the fused GEMM).
//
// Simd "SynetDynamicQuantizedInnerProduct16b Class Reference", Detailed
// Description: A[i,k] -> uA[i,k] (uint8), scaleA[i], zeroA[i], with this
// library's asymmetric min/max reading (0 kept inside the range):
//   lo = min(0, min_k A), hi = max(0, max_k A),
//   scaleA = (hi - lo) / 255, zeroA = sat[0,255](rne(-lo / scaleA)),
//   uA = sat[0,255](rne(A / scaleA) + zeroA),
// scale 1 and zero point 0 for an all-zero row; stored as sA = uA - 128 in
// MFMA fragment order.
#pragma once

#include "dq_device.h"

namespace dqrow {

__device__ __forceinline__ void row_params(float lo, float hi, float& scale, int& zero) {
    if (hi == lo) {
        scale = 1.0f;
        zero = 0;
    } else {
        scale = (hi - lo) / 255.0f;
        zero = dq::sat_add(dq::rne(-lo / scale), 0, 0, 255);
    }
}

// 16 codes uA - 128 of one group, stored as one 16-byte vector. FAST: the
// row's scale has a normal reciprocal, and |A / scale| <= 256 holds by the
// scale's construction, so the bounded residual division applies.
// sA = sat[0,255](rne(q) + zero) - 128 = (int)clamp(rne(q), -zero, 255 - zero)
// + (zero - 128), taken as a byte.
template <bool FAST>
__device__ __forceinline__ void store_group(int8_t* __restrict__ sA, size_t row, int g, int KF,
                                            const float (&x)[16], const dq::QDiv& d, int zero) {
    const float lo = (float)(-zero), hi = (float)(255 - zero);
    const int shift = zero - 128;
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint32_t packed = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float qt = FAST ? dq::qdiv_fast(x[4 * q + b], d) : x[4 * q + b] / d.s;
            const float r = __builtin_fminf(__builtin_fmaxf(dq::rne(qt), lo), hi);
            packed |= ((uint32_t)((int)r + shift) & 0xffu) << (8 * b);
        }
        w[q] = packed;
    }
    const dq::u4 o = {w[0], w[1], w[2], w[3]};
    *reinterpret_cast<dq::u4*>(sA + dq::frag_offset(row, (size_t)g * 16, KF)) = o;
}

// Row statistics come out of the reductions as wave-uniform values, which
// makes scale, zero point and the division path scalar, so the row takes one
// branch instead of one per element.
__device__ __forceinline__ void uniform_minmax(float& lo, float& hi) {
    lo = dq::wave_min_uniform(lo);
    hi = dq::wave_max_uniform(hi);
}

template <bool BF16, int NV>
struct RawRow {
    static constexpr int U = BF16 ? 2 : 4;  // 16-byte vectors per group
    dq::u4 v[NV][U];
};

template <bool BF16, int NV>
__device__ __forceinline__ void load_row(const void* __restrict__ A, int row, int K, int lane,
                                         RawRow<BF16, NV>& r) {
    constexpr int U = RawRow<BF16, NV>::U;
    const int ngroups = K >> 4;
    const dq::u4* base = reinterpret_cast<const dq::u4*>(
        reinterpret_cast<const char*>(A) + (size_t)row * K * (BF16 ? 2 : 4));
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int g = lane + 64 * v;
#pragma unroll
        for (int u = 0; u < U; ++u) r.v[v][u] = g < ngroups ? base[(size_t)g * U + u] : dq::u4{0, 0, 0, 0};
    }
}

// Element e (0..15) of group v as fp32 (a bf16 value is the top half of its
// fp32 bit pattern).
template <bool BF16, int NV>
__device__ __forceinline__ float elem(const RawRow<BF16, NV>& r, int v, int e) {
    if (BF16) {
        const uint32_t w = r.v[v][e >> 3][(e >> 1) & 3];
        return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
    }
    return __uint_as_float(r.v[v][e >> 2][e & 3]);
}

// Quantizes one row held in registers. Fast path (the scale has a normal
// reciprocal; |A / scale| <= 256 by construction): q = corrected quotient;
// adding 1.5 * 2^23 rounds q half to even into the low mantissa bits
// (the float add rounds to nearest even, and 1.5 * 2^23 is even), so the
// bit pattern is 0x4B400000 + rne(q); a median against the integers
// 1.5 * 2^23 - zero and 1.5 * 2^23 + 255 - zero clamps it to
// rne(q) + zero in [0, 255]; the low bytes of four codes are packed and
// zero - 128 is added to every byte at once (a carry-free bytewise add),
// giving uA - 128.
template <bool BF16, int NV>
__device__ __forceinline__ void quantize_row(const RawRow<BF16, NV>& r, int row, int K, int KF,
                                             int lane, int8_t* __restrict__ sA,
                                             float* __restrict__ scaleA,
                                             int32_t* __restrict__ zeroA) {
    const int ngroups = K >> 4;
    float lo = 0.0f, hi = 0.0f;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        if (lane + 64 * v < ngroups) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float x = elem(r, v, e);
                lo = __builtin_fminf(lo, x);
                hi = __builtin_fmaxf(hi, x);
            }
        }
    }
    uniform_minmax(lo, hi);
    float scale;
    int zero;
    row_params(lo, hi, scale, zero);
    const dq::QDiv d = dq::make_qdiv(scale);
    if (d.fast) {
        constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
        // 1.5 * 2^23 + n is exact for |n| < 2^22, so the clamp bounds are too
        const float lof = kMagic - (float)zero, hif = kMagic + (float)(255 - zero);
        const uint32_t C = (uint32_t)((zero - 128) & 0xff) * 0x01010101u;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int g = lane + 64 * v;
            if (g >= ngroups) continue;
            uint32_t w[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint32_t b[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float t = dq::qdiv_fast(elem(r, v, 4 * q + e), d) + kMagic;
                    b[e] = (uint32_t)__float_as_int(__builtin_amdgcn_fmed3f(t, lof, hif));
                }
                const uint32_t packed = (b[0] & 0xffu) | ((b[1] & 0xffu) << 8) | ((b[2] & 0xffu) << 16) | (b[3] << 24);
                w[q] = ((packed & 0x7f7f7f7fu) + (C & 0x7f7f7f7fu)) ^ ((packed ^ C) & 0x80808080u);
            }
            const dq::u4 o = {w[0], w[1], w[2], w[3]};
            *reinterpret_cast<dq::u4*>(sA + dq::frag_offset(row, (size_t)g * 16, KF)) = o;
        }
    } else {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int g = lane + 64 * v;
            if (g >= ngroups) continue;
            float x[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) x[e] = elem(r, v, e);
            store_group<false>(sA, row, g, KF, x, d, zero);
        }
    }
    if (lane == 0) {
        scaleA[row] = scale;
        zeroA[row] = zero;
    }
}

}  // namespace dqrow
