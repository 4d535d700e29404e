// quant_rows.hip -- per-row dynamic quantization of A for gfx950.
//
// Simd "SynetDynamicQuantizedInnerProduct16b Class Reference", Detailed
// Description: A[i,k] -> uA[i,k] (uint8), scaleA[i], zeroA[i]. The page does
// not spell the formula out; this library uses the asymmetric min/max form
// with 0 kept inside the range (so zeroA is a uint8 value and 0.0 is exact):
//   lo = min(0, min_k A), hi = max(0, max_k A),
//   scaleA = (hi - lo) / 255, zeroA = sat[0,255](rne(-lo / scaleA)),
//   uA = sat[0,255](rne(A / scaleA) + zeroA),
// with scale 1 and zero point 0 for an all-zero row. The quotient rounds as
// the IEEE fp32 one, and rne is half to even, as QuantizeLinear (onnxruntime
// quantization_defs.cc) states for its own quotient.
//
// Output: sA = uA - 128 as int8 (the int8 MFMA is signed x signed), packed in
// MFMA fragment order; the GEMM adds (128 - zeroA) * colsum(iB) back, which
// is exact in int32.
//
// Design: one 64-lane wave per row, eight consecutive rows per 512-thread
// workgroup, so every 128-byte line of the packed output (eight rows x 16
// codes) is written whole by one workgroup. Lane l owns
// groups of 16 consecutive k (group g = l + 64 v); a row of up to 8 Ki values
// is read once with 16-byte loads and kept in VGPRs between the min/max
// reduction (xor shuffles, no LDS, no barrier) and the quantization, so A
// crosses HBM once and sA is written once, 16 bytes per lane. Longer rows
// take the streaming variant, whose second pass re-reads the row from L2.
#include "dq_device.h"
#include "dq_kernels.h"

#include <hip/hip_ext.h>

namespace {

constexpr int kRowsPerWave = 1;
constexpr int kWavesPerBlock = 8;
constexpr int kRowsPerBlock = kWavesPerBlock * kRowsPerWave;
constexpr int kThreads = 64 * kWavesPerBlock;

// 16 consecutive values of a row as fp32 (bf16 widened), from k0.
template <bool BF16, bool VEC>
__device__ __forceinline__ void load16(const void* __restrict__ A, size_t row_base, int k0, int K,
                                       float (&x)[16]) {
    if (VEC) {
        if (BF16) {
            const dq::u4* p = reinterpret_cast<const dq::u4*>(
                reinterpret_cast<const uint16_t*>(A) + row_base + k0);
            const dq::u4 a = p[0];
            const dq::u4 b = p[1];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                x[2 * w] = dq::bf16_bits_to_f32(a[w] & 0xffffu);
                x[2 * w + 1] = dq::bf16_bits_to_f32(a[w] >> 16);
                x[8 + 2 * w] = dq::bf16_bits_to_f32(b[w] & 0xffffu);
                x[8 + 2 * w + 1] = dq::bf16_bits_to_f32(b[w] >> 16);
            }
        } else {
            const dq::f4* p = reinterpret_cast<const dq::f4*>(
                reinterpret_cast<const float*>(A) + row_base + k0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const dq::f4 v = p[q];
                x[4 * q] = v[0];
                x[4 * q + 1] = v[1];
                x[4 * q + 2] = v[2];
                x[4 * q + 3] = v[3];
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int k = k0 + e;
            float v = 0.0f;  // past the row end: 0 is inside [lo, hi] already
            if (k < K) {
                if (BF16)
                    v = dq::bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(A)[row_base + k]);
                else
                    v = reinterpret_cast<const float*>(A)[row_base + k];
            }
            x[e] = v;
        }
    }
}

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

// Row cached in VGPRs: NV groups of 16 per lane (K <= 1024 * NV).
// VEC: K % 16 == 0 and a 16-byte aligned A (every group is a full vector).
template <bool BF16, bool VEC, int NV>
__global__ void __launch_bounds__(kThreads)
k_quant_rows(const void* __restrict__ A, int M, int K, int KF, int8_t* __restrict__ sA,
             float* __restrict__ scaleA, int32_t* __restrict__ zeroA) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int ngroups = (K + 15) >> 4;
    for (int rr = 0; rr < kRowsPerWave; ++rr) {
        const int row = blockIdx.x * kRowsPerBlock + wave * kRowsPerWave + rr;
        if (row >= M) return;
        const size_t base = (size_t)row * (size_t)K;
        float x[NV][16];
        float lo = 0.0f, hi = 0.0f;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int g = lane + 64 * v;
            if (g < ngroups) {
                load16<BF16, VEC>(A, base, g * 16, K, x[v]);
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    lo = __builtin_fminf(lo, x[v][e]);
                    hi = __builtin_fmaxf(hi, x[v][e]);
                }
            }
        }
        uniform_minmax(lo, hi);
        float scale;
        int zero;
        row_params(lo, hi, scale, zero);
        const dq::QDiv d = dq::make_qdiv(scale);
        if (d.fast) {
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const int g = lane + 64 * v;
                if (g < ngroups) store_group<true>(sA, row, g, KF, x[v], d, zero);
            }
        } else {
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const int g = lane + 64 * v;
                if (g < ngroups) store_group<false>(sA, row, g, KF, x[v], d, zero);
            }
        }
        if (lane == 0) {
            scaleA[row] = scale;
            zeroA[row] = zero;
        }
    }
}

// ---- persistent variant with the next row prefetched (vector loads only)
//
// Each wave quantizes rows w, w + W, w + 2W, ... (W waves in the grid) and
// issues the loads of its next row before it works on the current one, so
// the row's arithmetic overlaps the next row's memory traffic. Rows stay in
// VGPRs as loaded (NV groups of 16 values: 2 x 16 bytes of bf16 or 4 x 16
// bytes of fp32 per group).
constexpr int kPfWaves = 4096;  // four waves per SIMD on 256 CUs

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

template <bool BF16, int NV>
__global__ void __launch_bounds__(256)
k_quant_rows_pf(const void* __restrict__ A, int M, int K, int KF, int8_t* __restrict__ sA,
                float* __restrict__ scaleA, int32_t* __restrict__ zeroA) {
    const int lane = threadIdx.x & 63;
    const int W = gridDim.x * 4;
    int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= M) return;
    RawRow<BF16, NV> ra, rb;
    load_row(A, row, K, lane, ra);
    // ping-pong between two register buffers (no copies between them)
    for (;;) {
        int next = row + W;
        if (next < M) load_row(A, next, K, lane, rb);
        quantize_row(ra, row, K, KF, lane, sA, scaleA, zeroA);
        if (next >= M) return;
        row = next;
        next = row + W;
        if (next < M) load_row(A, next, K, lane, ra);
        quantize_row(rb, row, K, KF, lane, sA, scaleA, zeroA);
        if (next >= M) return;
        row = next;
    }
}

// Any K: min/max pass, then a second pass that re-reads each group.
template <bool BF16, bool VEC>
__global__ void __launch_bounds__(kThreads)
k_quant_rows_stream(const void* __restrict__ A, int M, int K, int KF, int8_t* __restrict__ sA,
                    float* __restrict__ scaleA, int32_t* __restrict__ zeroA) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int ngroups = (K + 15) >> 4;
    for (int rr = 0; rr < kRowsPerWave; ++rr) {
        const int row = blockIdx.x * kRowsPerBlock + wave * kRowsPerWave + rr;
        if (row >= M) return;
        const size_t base = (size_t)row * (size_t)K;
        float lo = 0.0f, hi = 0.0f;
        for (int g = lane; g < ngroups; g += 64) {
            float x[16];
            load16<BF16, VEC>(A, base, g * 16, K, x);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                lo = __builtin_fminf(lo, x[e]);
                hi = __builtin_fmaxf(hi, x[e]);
            }
        }
        uniform_minmax(lo, hi);
        float scale;
        int zero;
        row_params(lo, hi, scale, zero);
        const dq::QDiv d = dq::make_qdiv(scale);
        for (int g = lane; g < ngroups; g += 64) {
            float x[16];
            load16<BF16, VEC>(A, base, g * 16, K, x);
            if (d.fast) store_group<true>(sA, row, g, KF, x, d, zero);
            else store_group<false>(sA, row, g, KF, x, d, zero);
        }
        if (lane == 0) {
            scaleA[row] = scale;
            zeroA[row] = zero;
        }
    }
}

template <bool BF16, int NV>
void launch_pf(hipStream_t s, DqTiming t, const void* A, int M, int K, int KF, int8_t* sA,
               float* scaleA, int32_t* zeroA) {
    const int waves = M < kPfWaves ? M : kPfWaves;
    hipExtLaunchKernelGGL((k_quant_rows_pf<BF16, NV>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s,
                          t.start, t.stop, 0, A, M, K, KF, sA, scaleA, zeroA);
}

template <bool BF16, bool VEC>
void launch_rows(dim3 grid, hipStream_t s, DqTiming t, const void* A, int M, int K, int KF,
                 int8_t* sA, float* scaleA, int32_t* zeroA) {
    const int ngroups = (K + 15) / 16;
    const int nv = (ngroups + 63) / 64;
    // prefetching variant where two rows fit in registers (<= 64 VGPRs each)
    if (VEC && nv <= (BF16 ? 8 : 4)) {
        if (nv <= 1) launch_pf<BF16, 1>(s, t, A, M, K, KF, sA, scaleA, zeroA);
        else if (nv <= 2) launch_pf<BF16, 2>(s, t, A, M, K, KF, sA, scaleA, zeroA);
        else if (nv <= 4) launch_pf<BF16, 4>(s, t, A, M, K, KF, sA, scaleA, zeroA);
        else launch_pf<BF16, (BF16 ? 8 : 4)>(s, t, A, M, K, KF, sA, scaleA, zeroA);
        return;
    }
    if (nv <= 1)
        hipExtLaunchKernelGGL((k_quant_rows<BF16, VEC, 1>), grid, dim3(kThreads), 0, s, t.start, t.stop, 0, A, M, K, KF, sA, scaleA, zeroA);
    else if (nv <= 2)
        hipExtLaunchKernelGGL((k_quant_rows<BF16, VEC, 2>), grid, dim3(kThreads), 0, s, t.start, t.stop, 0, A, M, K, KF, sA, scaleA, zeroA);
    else if (nv <= 4)
        hipExtLaunchKernelGGL((k_quant_rows<BF16, VEC, 4>), grid, dim3(kThreads), 0, s, t.start, t.stop, 0, A, M, K, KF, sA, scaleA, zeroA);
    else if (nv <= 8)
        hipExtLaunchKernelGGL((k_quant_rows<BF16, VEC, 8>), grid, dim3(kThreads), 0, s, t.start, t.stop, 0, A, M, K, KF, sA, scaleA, zeroA);
    else
        hipExtLaunchKernelGGL((k_quant_rows_stream<BF16, VEC>), grid, dim3(kThreads), 0, s, t.start, t.stop, 0, A, M, K, KF, sA, scaleA, zeroA);
}

}  // namespace

int dq_launch_quant_rows(const void* A, bool bf16, int M, int K, int Kp, int8_t* sA,
                         float* scaleA, int32_t* zeroA, hipStream_t s, DqTiming t) {
    const bool vec = K % 16 == 0 && (uintptr_t)A % 16 == 0;
    const dim3 grid((unsigned)((M + kRowsPerBlock - 1) / kRowsPerBlock));
    const int KF = Kp / 32;
    if (bf16) {
        if (vec) launch_rows<true, true>(grid, s, t, A, M, K, KF, sA, scaleA, zeroA);
        else launch_rows<true, false>(grid, s, t, A, M, K, KF, sA, scaleA, zeroA);
    } else {
        if (vec) launch_rows<false, true>(grid, s, t, A, M, K, KF, sA, scaleA, zeroA);
        else launch_rows<false, false>(grid, s, t, A, M, K, KF, sA, scaleA, zeroA);
    }
    DQ_LAUNCH_CHECK("quant_rows");
    return DQ_OK;
}

// ------------------------------------------------------------ inspection

namespace {
__global__ void __launch_bounds__(256)
k_unpack_a(const int8_t* __restrict__ sA, int M, int K, int KF, uint8_t* __restrict__ uA) {
    const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= (size_t)M * K) return;
    const size_t i = t / K, k = t % K;
    uA[t] = (uint8_t)sA[dq::frag_offset(i, k, KF)] ^ 0x80u;
}
}  // namespace

int dq_launch_unpack_a(const int8_t* sA, int M, int K, int Kp, uint8_t* uA, hipStream_t s) {
    const size_t n = (size_t)M * K;
    if ((n + 255) / 256 > 0x7fffffffu) DQ_FAIL(DQ_ERR_ARG, "tensor too large to unpack");
    hipLaunchKernelGGL(k_unpack_a, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, sA, M, K,
                       Kp / 32, uA);
    DQ_LAUNCH_CHECK("unpack_a");
    return DQ_OK;
}
