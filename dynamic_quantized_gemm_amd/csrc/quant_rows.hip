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
#include "quant_row_dev.h"

#include <hip/hip_ext.h>

namespace {

using namespace dqrow;

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
