// quant_rows.hip -- per-row dynamic quantization of A for gfx950.
//
// Simd "SynetDynamicQuantizedInnerProduct16b Class Reference", Detailed
// Description: A[i,k] -> uA[i,k] (uint8), scaleA[i], zeroA[i]. The page does
// not spell the formula out; this library uses the asymmetric min/max form
// with 0 kept inside the range (so zeroA is a uint8 value and 0.0 is exact):
//   lo = min(0, min_k A), hi = max(0, max_k A),
//   scaleA = (hi - lo) / 255, zeroA = sat[0,255](rne(-lo / scaleA)),
//   uA = sat[0,255](rne(A / scaleA) + zeroA),
// with scale 1 and zero point 0 for an all-zero row. The quotient is the
// IEEE fp32 one and rne is half to even, as QuantizeLinear (onnxruntime
// quantization_defs.cc) states for its own quotient.
//
// Output: sA = uA - 128 as int8 (the int8 MFMA is signed x signed); the
// GEMM adds (128 - zeroA) * colsum(iB) back, which is exact in int32.
//
// Design: one 64-lane wave per row, four rows per 256-thread workgroup. A
// row of up to 8 Ki fp32 / 16 Ki bf16 values is read once with coalesced
// 16-byte loads and kept in VGPRs between the min/max reduction (xor
// shuffles, no LDS, no barrier) and the quantization, so A crosses HBM once.
// Longer or misaligned rows take a two-pass lane-strided kernel whose second
// pass hits L2.
#include "dq_device.h"
#include "dq_kernels.h"

namespace {

template <bool BF16>
__device__ __forceinline__ void minmax_vec(const dq::u4& v, float& lo, float& hi) {
    if (BF16) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float a0 = dq::bf16_bits_to_f32(v[w] & 0xffffu);
            const float a1 = dq::bf16_bits_to_f32(v[w] >> 16);
            lo = __builtin_fminf(lo, __builtin_fminf(a0, a1));
            hi = __builtin_fmaxf(hi, __builtin_fmaxf(a0, a1));
        }
    } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float a = __uint_as_float(v[w]);
            lo = __builtin_fminf(lo, a);
            hi = __builtin_fmaxf(hi, a);
        }
    }
}

__device__ __forceinline__ uint32_t code(float a, float scale, int zero) {
    // uA - 128 as a byte: sat(rne(a/s) + zero) in [0,255], top bit flipped
    return (uint32_t)dq::sat_add(dq::rne(a / scale), zero, 0, 255) ^ 0x80u;
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

// NV 16-byte vectors per lane; requires K % (16 / sizeof(elem)) == 0, a
// 16-byte aligned A and K <= 64 * NV * elems_per_vector.
template <bool BF16, int NV>
__global__ void __launch_bounds__(256)
k_quant_rows(const void* __restrict__ A, int M, int K, int Kp, int8_t* __restrict__ sA,
             float* __restrict__ scaleA, int32_t* __restrict__ zeroA) {
    constexpr int EPV = BF16 ? 8 : 4;
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= M) return;
    const int nvec = K / EPV;
    const dq::u4* src = reinterpret_cast<const dq::u4*>(
        reinterpret_cast<const char*>(A) + (size_t)row * (size_t)K * (BF16 ? 2 : 4));
    dq::u4 v[NV];
    float lo = 0.0f, hi = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int vi = i * 64 + lane;
        if (vi < nvec) {
            v[i] = __builtin_nontemporal_load(src + vi);
            minmax_vec<BF16>(v[i], lo, hi);
        }
    }
    lo = dq::wave_min(lo);
    hi = dq::wave_max(hi);
    float scale;
    int zero;
    row_params(lo, hi, scale, zero);
    int8_t* dst = sA + (size_t)row * Kp;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int vi = i * 64 + lane;
        if (vi < nvec) {
            if (BF16) {
                uint32_t w[2] = {0, 0};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t bits = (v[i][e >> 1] >> (16 * (e & 1))) & 0xffffu;
                    w[e >> 2] |= code(dq::bf16_bits_to_f32(bits), scale, zero) << (8 * (e & 3));
                }
                const dq::u2 o = {w[0], w[1]};
                *reinterpret_cast<dq::u2*>(dst + (size_t)vi * 8) = o;
            } else {
                uint32_t w = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) w |= code(__uint_as_float(v[i][e]), scale, zero) << (8 * e);
                *reinterpret_cast<uint32_t*>(dst + (size_t)vi * 4) = w;
            }
        }
    }
    if (lane == 0) {
        scaleA[row] = scale;
        zeroA[row] = zero;
    }
}

// Any K, any alignment: two lane-strided passes over the row.
template <bool BF16>
__global__ void __launch_bounds__(256)
k_quant_rows_generic(const void* __restrict__ A, int M, int K, int Kp, int8_t* __restrict__ sA,
                     float* __restrict__ scaleA, int32_t* __restrict__ zeroA) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= M) return;
    const size_t base = (size_t)row * (size_t)K;
    auto load = [&](int k) -> float {
        if (BF16) return dq::bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(A)[base + k]);
        return reinterpret_cast<const float*>(A)[base + k];
    };
    float lo = 0.0f, hi = 0.0f;
    for (int k = lane; k < K; k += 64) {
        const float a = load(k);
        lo = __builtin_fminf(lo, a);
        hi = __builtin_fmaxf(hi, a);
    }
    lo = dq::wave_min(lo);
    hi = dq::wave_max(hi);
    float scale;
    int zero;
    row_params(lo, hi, scale, zero);
    int8_t* dst = sA + (size_t)row * Kp;
    for (int k = lane; k < K; k += 64) dst[k] = (int8_t)code(load(k), scale, zero);
    if (lane == 0) {
        scaleA[row] = scale;
        zeroA[row] = zero;
    }
}

}  // namespace

int dq_launch_quant_rows(const void* A, bool bf16, int M, int K, int Kp, int8_t* sA,
                         float* scaleA, int32_t* zeroA, hipStream_t s) {
    const int epv = bf16 ? 8 : 4;
    const bool vec_ok = K % epv == 0 && (uintptr_t)A % 16 == 0;
    const int nvec = K / epv;
    const int nv = (nvec + 63) / 64;  // vectors per lane
    const dim3 grid((unsigned)((M + 3) / 4)), block(256);
#define DQ_QR(B, NV)                                                                        \
    hipLaunchKernelGGL((k_quant_rows<B, NV>), grid, block, 0, s, A, M, K, Kp, sA, scaleA, \
                       zeroA)
#define DQ_QR_SWITCH(B)                   \
    if (nv <= 1) DQ_QR(B, 1);             \
    else if (nv <= 2) DQ_QR(B, 2);        \
    else if (nv <= 4) DQ_QR(B, 4);        \
    else if (nv <= 8) DQ_QR(B, 8);        \
    else if (nv <= 16) DQ_QR(B, 16);      \
    else DQ_QR(B, 32);
    if (vec_ok && nv <= 32) {
        if (bf16) {
            DQ_QR_SWITCH(true)
        } else {
            DQ_QR_SWITCH(false)
        }
    } else if (bf16) {
        hipLaunchKernelGGL((k_quant_rows_generic<true>), grid, block, 0, s, A, M, K, Kp, sA,
                           scaleA, zeroA);
    } else {
        hipLaunchKernelGGL((k_quant_rows_generic<false>), grid, block, 0, s, A, M, K, Kp, sA,
                           scaleA, zeroA);
    }
#undef DQ_QR_SWITCH
#undef DQ_QR
    DQ_LAUNCH_CHECK("quant_rows");
    return DQ_OK;
}

// ------------------------------------------------------------ inspection

namespace {
__global__ void __launch_bounds__(256)
k_unpack_a(const int8_t* __restrict__ sA, int M, int K, int Kp, uint8_t* __restrict__ uA) {
    const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= (size_t)M * K) return;
    const size_t i = t / K, k = t % K;
    uA[t] = (uint8_t)sA[i * Kp + k] ^ 0x80u;
}
}  // namespace

int dq_launch_unpack_a(const int8_t* sA, int M, int K, int Kp, uint8_t* uA, hipStream_t s) {
    const size_t n = (size_t)M * K;
    hipLaunchKernelGGL(k_unpack_a, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, sA, M, K,
                       Kp, uA);
    DQ_LAUNCH_CHECK("unpack_a");
    return DQ_OK;
}
