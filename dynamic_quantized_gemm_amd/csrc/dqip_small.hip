// dqip_small.hip -- the dynamic quantized inner product for small problems
// in one launch (gfx950).
//
// Simd "SynetDynamicQuantizedInnerProduct16b Class Reference", Detailed
// Description (the same method as quant_rows.hip + gemm_i8.hip): A's rows
// quantized to uint8 with their own scale and zero point (lo = min(0, min
// A), hi = max(0, max A), scale = (hi - lo) / 255, zero = sat(rne(-lo /
// scale)), uA = sat(rne(A / scale) + zero)), sum_k (uA - zeroA) iB in
// integers, then ((float)sum * scaleA) * scaleB (+ bias), activation and the
// conversion to fp32 or bf16.
//
// When the product is small (the 32 x 32 GEMM tile is the one chosen: a
// few rows, or few rows and columns) the two launches of the general path
// (row quantization, then the GEMM) cost more than their work, so here one
// workgroup per 32 x 32 tile of C does both. Its four waves split K: wave w
// takes k fragments 4 j + w, and lane l's share of the second MFMA operand
// is 16 values of row l % 32 of the tile at k = 32 kf + 16 (l / 32), which
// the lane loads and quantizes itself (so the codes never leave its
// registers). The rows' minima and maxima are combined across the lanes and
// waves holding each row (one exchange through LDS); the four partial
// tiles are summed through LDS, each thread taking four outputs, and the
// epilogue is the GEMM's. The workgroups of the first column tile also
// leave sA, scaleA and zeroA in the work buffer, as the two-launch path
// does, so they can be read back for inspection.
#include "dq_device.h"
#include "dq_kernels.h"

#include <hip/hip_ext.h>

namespace {

constexpr int kThreads = 256;
constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23: adding it rounds to an integer, half to even

struct SmallArgs {
    const void* A;
    const int8_t* iBp;   // packed B (rows = columns of B), Kp / 32 fragments a row block
    int M, N, K, KFp;    // KFp = Kp / 32
    DqEpilogue ep;
    int8_t* sA;          // inspection copies (written by column tile 0)
    float* scaleA;
    int32_t* zeroA;
};

// the GEMM epilogue's activation (act is uniform over the launch)
__device__ __forceinline__ float act_of(float v, int act, float alpha) {
    if (act == DQ_ACT_RELU) return v > 0.0f ? v : 0.0f;
    if (act == DQ_ACT_LEAKY_RELU) return v < 0.0f ? v * alpha : v;
    return v;
}

// 16 values to 16 codes uA - 128 in four words (byte e of word m is value
// 4 m + e): uA = sat[0,255](rne(x / s) + zero) = rne(clamp(x / s, -zero,
// 255 - zero)) + zero; the quotient is the IEEE one (the residual step of
// dq::qdiv when FAST, which holds since |x / s| <= 255, else the division).
template <bool FAST>
__device__ __forceinline__ dq::v4i codes16(const float (&x)[16], float s, float y, float lof, float hif,
                                           uint32_t z4) {
    dq::v4i out;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        uint32_t b[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float v = x[4 * m + e];
            float t;
            if (FAST) {
                const float q0 = v * y;
                t = __builtin_fmaf(__builtin_fmaf(-q0, s, v), y, q0);
            } else {
                t = v / s;
            }
            b[e] = (uint32_t)__float_as_int(__builtin_amdgcn_fmed3f(t + kMagic, lof, hif));
        }
        const uint32_t p = (b[0] & 0xffu) | ((b[1] & 0xffu) << 8) | ((b[2] & 0xffu) << 16) | (b[3] << 24);
        out[m] = (int)(((p & 0x7f7f7f7fu) + (z4 & 0x7f7f7f7fu)) ^ ((p ^ z4) & 0x80808080u));
    }
    return out;
}

template <bool BF16, int OUT, int NJ>
__global__ void __launch_bounds__(kThreads) k_dqip_small(SmallArgs a) {
    __shared__ int32_t red[4][16][64];
    __shared__ float rmm[4][32][2];
    __shared__ float rscale[32];
    __shared__ int32_t rzero[32];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int nt = blockIdx.x, mt = blockIdx.y;
    const int m0 = mt * 32, n0 = nt * 32;
    const int r = lane & 31, half = lane >> 5;
    const int row = m0 + r;
    const bool row_ok = row < a.M;

    // this wave's B fragments and A values (zeros past K and past M)
    const dq::v4i* bbase = reinterpret_cast<const dq::v4i*>(a.iBp + (size_t)nt * a.KFp * 1024) + lane;
    dq::v4i bf[NJ];
    float x[NJ][16];
    bool gok[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int kf = 4 * j + w;
        // fragments past packed B's width only meet codes forced to 0 below
        bf[j] = bbase[(size_t)(kf < a.KFp ? kf : 0) * 64];
        const int k0 = kf * 32 + 16 * half;
        const bool ok = row_ok && k0 < a.K;  // K % 16 == 0: a group is whole or absent
        gok[j] = ok;
        if (BF16) {
            const uint16_t* src = reinterpret_cast<const uint16_t*>(a.A) + (size_t)(ok ? row : 0) * a.K + (ok ? k0 : 0);
            const dq::u4 v0 = reinterpret_cast<const dq::u4*>(src)[0];
            const dq::u4 v1 = reinterpret_cast<const dq::u4*>(src)[1];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[j][2 * e] = ok ? dq::bf16_bits_to_f32(v0[e] & 0xffffu) : 0.0f;
                x[j][2 * e + 1] = ok ? dq::bf16_bits_to_f32(v0[e] >> 16) : 0.0f;
                x[j][8 + 2 * e] = ok ? dq::bf16_bits_to_f32(v1[e] & 0xffffu) : 0.0f;
                x[j][8 + 2 * e + 1] = ok ? dq::bf16_bits_to_f32(v1[e] >> 16) : 0.0f;
            }
        } else {
            const float* src = reinterpret_cast<const float*>(a.A) + (size_t)(ok ? row : 0) * a.K + (ok ? k0 : 0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const dq::f4 v = reinterpret_cast<const dq::f4*>(src)[q];
#pragma unroll
                for (int e = 0; e < 4; ++e) x[j][4 * q + e] = ok ? v[e] : 0.0f;
            }
        }
    }

    // the row's minimum and maximum, 0 included (padding values are 0)
    float lo = 0.0f, hi = 0.0f;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            lo = __builtin_fminf(lo, x[j][e]);
            hi = __builtin_fmaxf(hi, x[j][e]);
        }
    lo = __builtin_fminf(lo, __shfl_xor(lo, 32));
    hi = __builtin_fmaxf(hi, __shfl_xor(hi, 32));
    if (lane < 32) {
        rmm[w][lane][0] = lo;
        rmm[w][lane][1] = hi;
    }
    __syncthreads();
    if (tid < 32) {
        float l = rmm[0][tid][0], h = rmm[0][tid][1];
#pragma unroll
        for (int v = 1; v < 4; ++v) {
            l = __builtin_fminf(l, rmm[v][tid][0]);
            h = __builtin_fmaxf(h, rmm[v][tid][1]);
        }
        float scale = 1.0f;
        int zero = 0;
        if (h != l) {
            scale = (h - l) / 255.0f;
            zero = dq::sat_add(dq::rne(-l / scale), 0, 0, 255);
        }
        rscale[tid] = scale;
        rzero[tid] = zero;
        if (nt == 0 && m0 + tid < a.M) {
            a.scaleA[m0 + tid] = scale;
            a.zeroA[m0 + tid] = zero;
        }
    }
    __syncthreads();

    // codes and the product over this wave's fragments
    const float sc = rscale[r];
    const int zr = rzero[r];
    const dq::QDiv qd = dq::make_qdiv(sc);
    const float lof = kMagic + (float)(0 - zr), hif = kMagic + (float)(255 - zr);
    const uint32_t z4 = (uint32_t)((zr - 128) & 0xff) * 0x01010101u;
    dq::v16i acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        dq::v4i af = qd.fast ? codes16<true>(x[j], sc, qd.y, lof, hif, z4)
                             : codes16<false>(x[j], sc, qd.y, lof, hif, z4);
        // an absent group (k >= K or a row past M) contributes nothing
        if (!gok[j]) af = dq::v4i{0, 0, 0, 0};
        acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(bf[j], af, acc, 0, 0, 0);
        const int k0 = (4 * j + w) * 32 + 16 * half;
        if (nt == 0 && gok[j])
            *reinterpret_cast<dq::v4i*>(a.sA + dq::frag_offset(row, k0, a.KFp)) = af;
    }
    // the last MFMA's results need the ISA's wait states before they are read
    dq::mfma_result_drain();
#pragma unroll
    for (int e = 0; e < 16; ++e) red[w][e][lane] = acc[e];
    __syncthreads();

    // thread (w, lane): output row m0 + r, columns n0 + 8 w + 4 half + 0..3
    if (!row_ok) return;
    const int nb = n0 + 8 * w + 4 * half;
    if (nb >= a.N) return;
    const int32_t za = 128 - zr;
    const float sA_ = sc;
    int32_t sum[4];
    float val[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int rw = 4 * w + e;
        uint32_t s = (uint32_t)red[0][rw][lane] + (uint32_t)red[1][rw][lane] + (uint32_t)red[2][rw][lane] +
                     (uint32_t)red[3][rw][lane];
        const int n = nb + e < a.N ? nb + e : a.N - 1;
        s += (uint32_t)__mul24(za, a.ep.colsumB[n]);
        sum[e] = (int32_t)s;
        float v = (float)sum[e] * sA_;
        v = v * a.ep.scaleB[n];
        if (a.ep.bias) v = v + a.ep.bias[n];
        val[e] = act_of(v, a.ep.act, a.ep.alpha);
    }
    const size_t base = (size_t)row * a.N + nb;
    const bool whole = nb + 4 <= a.N;
    if (OUT == DQ_OUT_ACC) {
        int32_t* C = reinterpret_cast<int32_t*>(a.ep.C) + base;
        if (whole && a.N % 4 == 0) {
            *reinterpret_cast<dq::v4i*>(C) = dq::v4i{sum[0], sum[1], sum[2], sum[3]};
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (nb + e < a.N) C[e] = sum[e];
        }
    } else if (OUT == DQ_OUT_BF16) {
        uint16_t* C = reinterpret_cast<uint16_t*>(a.ep.C) + base;
        const dq::u2 p = dq::f32x4_to_bf16x4(dq::f4{val[0], val[1], val[2], val[3]});
        if (whole && a.N % 4 == 0) {
            *reinterpret_cast<dq::u2*>(C) = p;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (nb + e < a.N) C[e] = (uint16_t)(p[e >> 1] >> (16 * (e & 1)));
        }
    } else {
        float* C = reinterpret_cast<float*>(a.ep.C) + base;
        if (whole && a.N % 4 == 0) {
            *reinterpret_cast<dq::f4*>(C) = dq::f4{val[0], val[1], val[2], val[3]};
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (nb + e < a.N) C[e] = val[e];
        }
    }
}

template <bool BF16, int OUT>
void launch_nj(int nj, dim3 grid, hipStream_t s, DqTiming t, const SmallArgs& a) {
    switch (nj) {
        case 1: hipExtLaunchKernelGGL((k_dqip_small<BF16, OUT, 1>), grid, dim3(kThreads), 0, s, t.start, t.stop, 0, a); break;
        case 2: hipExtLaunchKernelGGL((k_dqip_small<BF16, OUT, 2>), grid, dim3(kThreads), 0, s, t.start, t.stop, 0, a); break;
        case 4: hipExtLaunchKernelGGL((k_dqip_small<BF16, OUT, 4>), grid, dim3(kThreads), 0, s, t.start, t.stop, 0, a); break;
        default: hipExtLaunchKernelGGL((k_dqip_small<BF16, OUT, 8>), grid, dim3(kThreads), 0, s, t.start, t.stop, 0, a); break;
    }
}

}  // namespace

bool dq_dqip_small_fits(int M, int N, int K, const void* A) {
    return dq_gemm_config(M, N) == 0 && K % 16 == 0 && K <= kDqipSmallKMax && (uintptr_t)A % 16 == 0;
}

int dq_launch_dqip_small(const void* A, bool bf16, int M, int N, int K, int Kp, const int8_t* iBp,
                         const DqEpilogue& ep, int8_t* sA, float* scaleA, int32_t* zeroA, hipStream_t s,
                         DqTiming t) {
    SmallArgs a;
    a.A = A;
    a.iBp = iBp;
    a.M = M;
    a.N = N;
    a.K = K;
    a.KFp = Kp / 32;
    a.ep = ep;
    a.sA = sA;
    a.scaleA = scaleA;
    a.zeroA = zeroA;
    const int KF = (K + 31) / 32, KFW = (KF + 3) / 4;
    const int nj = KFW <= 1 ? 1 : KFW <= 2 ? 2 : KFW <= 4 ? 4 : 8;
    const dim3 grid((unsigned)((N + 31) / 32), (unsigned)((M + 31) / 32));
    if (bf16) {
        if (ep.out == DQ_OUT_ACC) launch_nj<true, DQ_OUT_ACC>(nj, grid, s, t, a);
        else if (ep.out == DQ_OUT_BF16) launch_nj<true, DQ_OUT_BF16>(nj, grid, s, t, a);
        else launch_nj<true, DQ_OUT_F32>(nj, grid, s, t, a);
    } else {
        if (ep.out == DQ_OUT_ACC) launch_nj<false, DQ_OUT_ACC>(nj, grid, s, t, a);
        else if (ep.out == DQ_OUT_BF16) launch_nj<false, DQ_OUT_BF16>(nj, grid, s, t, a);
        else launch_nj<false, DQ_OUT_F32>(nj, grid, s, t, a);
    }
    DQ_LAUNCH_CHECK("dqip small");
    return DQ_OK;
}
