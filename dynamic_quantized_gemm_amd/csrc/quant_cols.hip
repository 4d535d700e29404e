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
//  - k_col_absmax_v4: whole row segments per wave (lane = four adjacent
//                   columns), maxima merged across the workgroup in LDS and
//                   then with an integer atomicMax on the fp32 bit pattern
//                   (monotone for values >= 0); k_col_absmax is the
//                   one-column-per-thread form for other shapes.
//  - k_pack_cols(_v4): 64x64 tiles: coalesced loads, quantize, transpose through
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

// One column per thread (any N, any alignment): a serial sweep over a
// chunk of kchunk rows, merged with an integer atomicMax on the fp32 bit
// pattern (monotone for values >= 0).
template <bool BF16>
__global__ void __launch_bounds__(256)
k_col_absmax(const void* __restrict__ B, int K, int N, int kchunk, uint32_t* __restrict__ amax) {
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= N) return;
    const int k0 = blockIdx.y * kchunk;
    const int k1 = min(K, k0 + kchunk);
    float m = 0.0f;
#pragma unroll 8
    for (int k = k0; k < k1; ++k) m = __builtin_fmaxf(m, __builtin_fabsf(load_b<BF16>(B, (size_t)k * N + j)));
    atomicMax(&amax[j], __float_as_uint(m));
}

// N % 4 == 0 and an aligned B: a workgroup covers 256 columns x kAmaxRows
// rows. Each wave reads 8 whole row segments (lane = four adjacent columns,
// one 16-byte fp32 / 8-byte bf16 load per row, all issued before any is
// used), the four waves' maxima merge in LDS, and one atomicMax per column
// and workgroup goes to memory. Row blocks run bottom-up and the pack pass
// that follows walks top-down, so it starts on the rows read most recently
// (at these sizes that gains little: data read again right after a read of
// 64-512 MiB comes back only 5-15% faster than from a cold start, so the
// second pass costs about a full read of B). Out-of-range rows and columns load a
// clamped in-range address (harmless for a maximum; the columns past N are
// never stored).
constexpr int kAmaxRowsPerWave = 8;
constexpr int kAmaxRows = 4 * kAmaxRowsPerWave;

template <bool BF16>
__global__ void __launch_bounds__(256)
k_col_absmax_v4(const void* __restrict__ B, int K, int N, uint32_t* __restrict__ amax) {
    __shared__ float red[4][256];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int by = gridDim.y - 1 - blockIdx.y;
    const int jl = lane * 4;
    const int j0 = min((int)blockIdx.x * 256 + jl, N - 4);
    const int k0 = by * kAmaxRows + w * kAmaxRowsPerWave;
    float v[kAmaxRowsPerWave][4];
#pragma unroll
    for (int i = 0; i < kAmaxRowsPerWave; ++i) {
        const size_t idx = (size_t)min(k0 + i, K - 1) * N + j0;
        if (BF16) {
            const dq::u2 x = *reinterpret_cast<const dq::u2*>(reinterpret_cast<const uint16_t*>(B) + idx);
            v[i][0] = __uint_as_float(x[0] << 16);
            v[i][1] = __uint_as_float(x[0] & 0xffff0000u);
            v[i][2] = __uint_as_float(x[1] << 16);
            v[i][3] = __uint_as_float(x[1] & 0xffff0000u);
        } else {
            const dq::f4 x = *reinterpret_cast<const dq::f4*>(reinterpret_cast<const float*>(B) + idx);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[i][e] = x[e];
        }
    }
    float m[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < kAmaxRowsPerWave; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) m[e] = __builtin_fmaxf(m[e], __builtin_fabsf(v[i][e]));
#pragma unroll
    for (int e = 0; e < 4; ++e) red[w][jl + e] = m[e];
    __syncthreads();
    const int t = threadIdx.x;
    const int j = blockIdx.x * 256 + t;
    const float mm = __builtin_fmaxf(__builtin_fmaxf(red[0][t], red[1][t]), __builtin_fmaxf(red[2][t], red[3][t]));
    if (j < N) atomicMax(&amax[j], __float_as_uint(mm));
}

// One 64(k) x 64(n) tile per workgroup. IN: 0 fp32, 1 bf16, 2 int8, 3 uint8
// (packed as code - 128, the int8 the MFMA takes).
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
    if (IN < 2 && tid < kT) {
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
        const float sc = IN < 2 ? s_scale[ln] : 1.0f;
#pragma unroll 4
        for (int i = 0; i < kT / 4; ++i) {
            const int kk = (tid >> 6) + 4 * i;
            const int k = k0 + kk;
            int q = 0;
            if (k < K && n < N) {
                const size_t idx = (size_t)k * N + n;
                if (IN == 2) {
                    q = reinterpret_cast<const int8_t*>(B)[idx];
                } else if (IN == 3) {
                    q = (int)reinterpret_cast<const uint8_t*>(B)[idx] - 128;
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

// V4 (fp32 / bf16 B, N % 4 == 0, aligned): the same 64 x 64 tile, but lane
// (c4 = tid % 16, r = tid / 16) loads the four adjacent columns 4 c4 .. +3
// of the four consecutive rows 4 r .. 4 r + 3 with 16-byte (8-byte for
// bf16) loads, so a wave instruction reads four row segments of the tile
// whole. Codes: q0 = b * (1/s) and the residual step give the IEEE
// quotient's rounding (|b / s| <= qmax by the scale's construction); adding
// 1.5 * 2^23 rounds half to even into the low mantissa bits and a median
// clamps to [qmin, qmax]; the four codes of one column pack into a word
// written to the transposed tile with one 4-byte store (bank = 4 c4 + r
// (mod 64): conflict free).
template <bool BF16>
__global__ void __launch_bounds__(256)
k_pack_cols_v4(const void* __restrict__ B, int K, int N, int Kp, int qmin, int qmax,
               const uint32_t* __restrict__ amax, int8_t* __restrict__ iBp,
               float* __restrict__ scaleB, int32_t* __restrict__ colsum) {
    __shared__ __attribute__((aligned(16))) uint8_t tile[kT * kTS];  // [n][k]
    constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
    const int tid = threadIdx.x;
    const int n0 = blockIdx.x * kT;
    const int k0 = blockIdx.y * kT;
    const int c4 = tid & 15, r = tid >> 4;
    // the four columns' scales and reciprocals (each lane its own columns)
    float sc[4];
    dq::QDiv d[4];
    bool fast = true;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int n = n0 + 4 * c4 + e;
        float s = 1.0f;
        if (n < N) {
            const float a = __uint_as_float(amax[n]);
            s = a > 0.0f ? a / (float)qmax : 1.0f;
            if (k0 == 0 && r == 0) scaleB[n] = s;
        }
        sc[e] = s;
        d[e] = dq::make_qdiv(s);
        fast = fast && d[e].fast;
    }
    // loads: rows 4 r .. 4 r + 3 of the tile (zero past K or N)
    float v[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int k = k0 + 4 * r + i;
        const int n = n0 + 4 * c4;
        if (k < K && n < N) {
            const size_t idx = (size_t)k * N + n;
            if (BF16) {
                const dq::u2 w = *reinterpret_cast<const dq::u2*>(reinterpret_cast<const uint16_t*>(B) + idx);
                v[i][0] = __uint_as_float(w[0] << 16);
                v[i][1] = __uint_as_float(w[0] & 0xffff0000u);
                v[i][2] = __uint_as_float(w[1] << 16);
                v[i][3] = __uint_as_float(w[1] & 0xffff0000u);
            } else {
                const dq::f4 w = *reinterpret_cast<const dq::f4*>(reinterpret_cast<const float*>(B) + idx);
#pragma unroll
                for (int e = 0; e < 4; ++e) v[i][e] = w[e];
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[i][e] = 0.0f;
        }
    }
    const float lof = kMagic + (float)qmin, hif = kMagic + (float)qmax;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t b;
            if (fast) {
                const float t = dq::qdiv_fast(v[i][e], d[e]) + kMagic;
                b = (uint32_t)__float_as_int(__builtin_amdgcn_fmed3f(t, lof, hif));
            } else {
                b = (uint32_t)dq::sat_add(dq::rne(v[i][e] / sc[e]), 0, qmin, qmax);
            }
            word |= (b & 0xffu) << (8 * i);
        }
        *reinterpret_cast<uint32_t*>(&tile[(4 * c4 + e) * kTS + 4 * r]) = word;
    }
    __syncthreads();
    // the tile's four packed fragments and the column sums, as in k_pack_cols
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
    if (vec4) {
        const dim3 agrid((unsigned)((N + 255) / 256), (unsigned)((K + kAmaxRows - 1) / kAmaxRows));
        if (bf16)
            hipLaunchKernelGGL((k_col_absmax_v4<true>), agrid, dim3(256), 0, s, B, K, N, amax);
        else
            hipLaunchKernelGGL((k_col_absmax_v4<false>), agrid, dim3(256), 0, s, B, K, N, amax);
    } else {
        const int kchunk = 64;
        const dim3 agrid((unsigned)((N + 255) / 256), (unsigned)((K + kchunk - 1) / kchunk));
        if (bf16)
            hipLaunchKernelGGL((k_col_absmax<true>), agrid, dim3(256), 0, s, B, K, N, kchunk, amax);
        else
            hipLaunchKernelGGL((k_col_absmax<false>), agrid, dim3(256), 0, s, B, K, N, kchunk, amax);
    }
    DQ_LAUNCH_CHECK("col_absmax");
    if (vec4 && bf16)
        hipExtLaunchKernelGGL((k_pack_cols_v4<true>), pgrid, dim3(256), 0, s, nullptr, t.stop, 0, B, K, N,
                              Kp, qmin, qmax, amax, iBp, scaleB, colsum);
    else if (vec4)
        hipExtLaunchKernelGGL((k_pack_cols_v4<false>), pgrid, dim3(256), 0, s, nullptr, t.stop, 0, B, K, N,
                              Kp, qmin, qmax, amax, iBp, scaleB, colsum);
    else if (bf16)
        hipExtLaunchKernelGGL((k_pack_cols<1>), pgrid, dim3(256), 0, s, nullptr, t.stop, 0, B, K, N,
                              Kp, qmin, qmax, amax, iBp, scaleB, colsum);
    else
        hipExtLaunchKernelGGL((k_pack_cols<0>), pgrid, dim3(256), 0, s, nullptr, t.stop, 0, B, K, N,
                              Kp, qmin, qmax, amax, iBp, scaleB, colsum);
    DQ_LAUNCH_CHECK("pack_cols");
    return DQ_OK;
}

int dq_launch_pack_cols8(const void* src, bool u8, int K, int R, int Kp, int8_t* dst,
                         int32_t* sums, hipStream_t s) {
    const dim3 pgrid((unsigned)((R + kT - 1) / kT), (unsigned)(Kp / kT));
    // the sums are accumulated with atomics: clear them first (a fill
    // kernel, so the sequence stays valid under stream capture)
    hipLaunchKernelGGL(k_zero, dim3((unsigned)((R + 255) / 256)), dim3(256), 0, s,
                       reinterpret_cast<uint32_t*>(sums), R, sums);
    DQ_LAUNCH_CHECK("zero");
    if (u8)
        hipLaunchKernelGGL((k_pack_cols<3>), pgrid, dim3(256), 0, s, src, K, R, Kp, 0, 0, nullptr, dst,
                           nullptr, sums);
    else
        hipLaunchKernelGGL((k_pack_cols<2>), pgrid, dim3(256), 0, s, src, K, R, Kp, 0, 0, nullptr, dst,
                           nullptr, sums);
    DQ_LAUNCH_CHECK("pack_cols8");
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
