// quant_cols.hip -- per-column quantization and packing of B for gfx950.
//
// Simd "SynetDynamicQuantizedInnerProduct16b Class Reference": B[k,j] ->
// iB[k,j] (int8), scaleB[j] (Detailed Description); with avoidOverflow the
// range narrows to [-64, 63] (Init()); an already quantized int8 B comes with
// its per-output-channel scales (SetParams()); the context keeps "weight
// column sums" (InternalBufferSize()). B has no zero point in the method's
// sum, so its quantization is symmetric:
//   scaleB = max_k |B[k,j]| / qmax, iB = sat[qmin,qmax](rne(B / scaleB)),
// (qmin, qmax) = (-128, 127), or (-64, 63) with avoidOverflow, scale 1 for an
// all-zero column.
//
// Output layout: iBp, B transposed (column j of B becomes packed row j) in
// MFMA fragment order, K zero-padded to Kp, and colsum[j] = sum_k iB[k,j]
// (ReduceSumInteger over axis 0).
//
// Kernels:
//  - k_zero:        clears the column maxima and sums (fill kernel; no memset
//                   node, so the sequence is safe under stream capture).
//  - k_col_absmax:  coalesced row sweeps (each thread owns four adjacent
//                   columns, a wave reads 1 KiB of a row), per-thread maxima
//                   merged with an integer atomicMax on the fp32 bit pattern
//                   (monotone for values >= 0).
//  - k_pack_cols:   64x64 tiles: coalesced loads, quantize, transpose through
//                   LDS, 16-byte stores of four whole packed fragments, and
//                   the column sums from the transposed tile (integer
//                   atomics: exact in any order).
#include "dq_device.h"
#include "dq_kernels.h"

#include <hip/hip_ext.h>

namespace {

constexpr int kT = 64;       // tile edge (k and n)
constexpr int kTS = kT + 4;  // LDS row stride of the transposed tile, bytes

__global__ void __launch_bounds__(256) k_zero(uint32_t* __restrict__ a, int n,
                                               int32_t* __restrict__ b) {
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t < n) {
        a[t] = 0u;
        b[t] = 0;
    }
}

template <bool BF16>
__device__ __forceinline__ float load_b(const void* B, size_t idx) {
    if (BF16) return dq::bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(B)[idx]);
    return reinterpret_cast<const float*>(B)[idx];
}

// VEC4: four adjacent columns per thread with one 16-byte (fp32) or 8-byte
// (bf16) load; needs N % 4 == 0 and an aligned B.
template <bool BF16, bool VEC4>
__global__ void __launch_bounds__(256)
k_col_absmax(const void* __restrict__ B, int K, int N, int kchunk, uint32_t* __restrict__ amax) {
    const int cols_per_thread = VEC4 ? 4 : 1;
    const int j0 = (blockIdx.x * 256 + threadIdx.x) * cols_per_thread;
    if (j0 >= N) return;
    const int k0 = blockIdx.y * kchunk;
    const int k1 = min(K, k0 + kchunk);
    float m[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int k = k0; k < k1; ++k) {
        const size_t idx = (size_t)k * N + j0;
        if (VEC4) {
            if (BF16) {
                const dq::u2 v = *reinterpret_cast<const dq::u2*>(
                    reinterpret_cast<const uint16_t*>(B) + idx);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    m[e] = __builtin_fmaxf(
                        m[e], __builtin_fabsf(dq::bf16_bits_to_f32((v[e >> 1] >> (16 * (e & 1))) & 0xffffu)));
            } else {
                const dq::f4 v = *reinterpret_cast<const dq::f4*>(reinterpret_cast<const float*>(B) + idx);
#pragma unroll
                for (int e = 0; e < 4; ++e) m[e] = __builtin_fmaxf(m[e], __builtin_fabsf(v[e]));
            }
        } else {
            m[0] = __builtin_fmaxf(m[0], __builtin_fabsf(load_b<BF16>(B, idx)));
        }
    }
#pragma unroll
    for (int e = 0; e < cols_per_thread; ++e) atomicMax(&amax[j0 + e], __float_as_uint(m[e]));
}

// One 64(k) x 64(n) tile per workgroup. IN: 0 fp32, 1 bf16, 2 int8.
template <int IN>
__global__ void __launch_bounds__(256)
k_pack_cols(const void* __restrict__ B, int K, int N, int Kp, int qmin, int qmax,
            const uint32_t* __restrict__ amax, int8_t* __restrict__ iBp,
            float* __restrict__ scaleB, int32_t* __restrict__ colsum) {
    __shared__ float s_scale[kT];
    __shared__ __attribute__((aligned(16))) uint8_t tile[kT * kTS];  // [n][k]
    const int tid = threadIdx.x;
    const int n0 = blockIdx.x * kT;
    const int k0 = blockIdx.y * kT;
    if (IN != 2 && tid < kT) {
        const int n = n0 + tid;
        float sc = 1.0f;
        if (n < N) {
            const float a = __uint_as_float(amax[n]);
            sc = a > 0.0f ? a / (float)qmax : 1.0f;
            if (k0 == 0) scaleB[n] = sc;
        }
        s_scale[tid] = sc;
    }
    __syncthreads();
    // loads: lane = column of the tile (a wave reads one contiguous row
    // segment per instruction), wave w takes rows w, w+4, ...; each code is
    // stored transposed, tile[n][k] (stride 68: the 64 lanes of a store hit
    // 64 distinct banks)
    {
        const int ln = tid & 63;
        const int n = n0 + ln;
        const float sc = IN != 2 ? s_scale[ln] : 1.0f;
#pragma unroll 4
        for (int i = 0; i < kT / 4; ++i) {
            const int kk = (tid >> 6) + 4 * i;
            const int k = k0 + kk;
            int q = 0;
            if (k < K && n < N) {
                const size_t idx = (size_t)k * N + n;
                if (IN == 2) {
                    q = reinterpret_cast<const int8_t*>(B)[idx];
                } else {
                    const float b = load_b<IN == 1>(B, idx);
                    q = dq::sat_add(dq::rne(b / sc), 0, qmin, qmax);
                }
            }
            tile[ln * kTS + kk] = (uint8_t)q;
        }
    }
    __syncthreads();
    // write the tile's four packed fragments (4 KiB, every 128-byte line
    // whole): thread -> column nn = tid / 4 of the tile, 16 codes of k-group
    // part = tid % 4, i.e. fragment (n / 32, (k0 + 16 part) / 32), lane slot
    // (n % 32) + 32 * (part % 2)
    const int nn = tid / 4;
    const int part = tid % 4;
    const uint8_t* src = tile + nn * kTS + part * 16;
    const uint32_t w0 = *reinterpret_cast<const uint32_t*>(src);
    const uint32_t w1 = *reinterpret_cast<const uint32_t*>(src + 4);
    const uint32_t w2 = *reinterpret_cast<const uint32_t*>(src + 8);
    const uint32_t w3 = *reinterpret_cast<const uint32_t*>(src + 12);
    int sum = 0;
    const uint32_t ws[4] = {w0, w1, w2, w3};
#pragma unroll
    for (int e = 0; e < 16; ++e) sum += (int)(int8_t)((ws[e >> 2] >> (8 * (e & 3))) & 0xffu);
    sum += __shfl_xor(sum, 1, 64);
    sum += __shfl_xor(sum, 2, 64);
    const int n = n0 + nn;
    if (n < N) {
        const dq::u4 o = {w0, w1, w2, w3};
        *reinterpret_cast<dq::u4*>(iBp + dq::frag_offset((size_t)n, (size_t)(k0 + part * 16), (size_t)(Kp / 32))) = o;
        if (part == 0 && sum != 0) atomicAdd(&colsum[n], sum);
    }
}

__global__ void __launch_bounds__(256)
k_unpack_b(const int8_t* __restrict__ iBp, int K, int N, int Kp, int8_t* __restrict__ iB) {
    const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= (size_t)K * N) return;
    const size_t k = t / N, j = t % N;
    iB[t] = iBp[dq::frag_offset(j, k, (size_t)(Kp / 32))];
}

}  // namespace

int dq_launch_quant_cols(const void* B, dq_dtype typeB, int K, int N, int Kp, int avoid,
                         int8_t* iBp, float* scaleB, int32_t* colsum, uint32_t* amax,
                         hipStream_t s, DqTiming t) {
    const int qmax = avoid ? 63 : 127;
    const int qmin = avoid ? -64 : -128;
    const dim3 pgrid((unsigned)((N + kT - 1) / kT), (unsigned)(Kp / kT));
    hipExtLaunchKernelGGL(k_zero, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, s, t.start,
                          nullptr, 0, amax, N, colsum);
    DQ_LAUNCH_CHECK("zero");
    if (typeB == DQ_I8) {
        hipExtLaunchKernelGGL((k_pack_cols<2>), pgrid, dim3(256), 0, s, nullptr, t.stop, 0, B, K, N,
                              Kp, qmin, qmax, amax, iBp, scaleB, colsum);
        DQ_LAUNCH_CHECK("pack_cols");
        return DQ_OK;
    }
    const bool bf16 = typeB == DQ_BF16;
    const bool vec4 = N % 4 == 0 && (uintptr_t)B % 16 == 0;
    const int kchunk = 64;
    const dim3 agrid((unsigned)((N + (vec4 ? 1024 : 256) - 1) / (vec4 ? 1024 : 256)),
                     (unsigned)((K + kchunk - 1) / kchunk));
    if (bf16) {
        if (vec4)
            hipLaunchKernelGGL((k_col_absmax<true, true>), agrid, dim3(256), 0, s, B, K, N, kchunk, amax);
        else
            hipLaunchKernelGGL((k_col_absmax<true, false>), agrid, dim3(256), 0, s, B, K, N, kchunk, amax);
    } else {
        if (vec4)
            hipLaunchKernelGGL((k_col_absmax<false, true>), agrid, dim3(256), 0, s, B, K, N, kchunk, amax);
        else
            hipLaunchKernelGGL((k_col_absmax<false, false>), agrid, dim3(256), 0, s, B, K, N, kchunk, amax);
    }
    DQ_LAUNCH_CHECK("col_absmax");
    if (bf16)
        hipExtLaunchKernelGGL((k_pack_cols<1>), pgrid, dim3(256), 0, s, nullptr, t.stop, 0, B, K, N,
                              Kp, qmin, qmax, amax, iBp, scaleB, colsum);
    else
        hipExtLaunchKernelGGL((k_pack_cols<0>), pgrid, dim3(256), 0, s, nullptr, t.stop, 0, B, K, N,
                              Kp, qmin, qmax, amax, iBp, scaleB, colsum);
    DQ_LAUNCH_CHECK("pack_cols");
    return DQ_OK;
}

int dq_launch_unpack_b(const int8_t* iBp, int K, int N, int Kp, int8_t* iB, hipStream_t s) {
    const size_t n = (size_t)K * N;
    if ((n + 255) / 256 > 0x7fffffffu) DQ_FAIL(DQ_ERR_ARG, "tensor too large to unpack");
    hipLaunchKernelGGL(k_unpack_b, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, iBp, K, N,
                       Kp, iB);
    DQ_LAUNCH_CHECK("unpack_b");
    return DQ_OK;
}
