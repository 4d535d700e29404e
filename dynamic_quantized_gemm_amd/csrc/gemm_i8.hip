// gemm_i8.hip -- the integer inner product and its dequantizing epilogue on
// gfx950 matrix cores.
//
// Simd "SynetDynamicQuantizedInnerProduct16b Class Reference", Detailed
// Description: sum = sum_k (uA[i,k] - zeroA[i]) * iB[k,j];
// val = sum * scaleA[i] * scaleB[j]; C = Convert(Activate(val + bias[j])).
//
// The int8 MFMA multiplies signed by signed, while uA is unsigned. With
// sA = uA - 128 (int8) the sum splits exactly:
//   sum = sum_k sA[i,k] iB[k,j] + (128 - zeroA[i]) * colsum(iB)[j]
// The first term is the MFMA contraction (|term| <= 128*128*K < 2^31 for
// K <= 65536); the correction is added in wrapping 32-bit arithmetic, which
// yields the exact sum because the true sum fits in int32.
//
// Epilogue (fp32, no fused multiply-add, the page's order):
//   val = ((float)sum * scaleA[i]) * scaleB[j]; val = val + bias[j];
//   activation; store fp32, bf16 (round to nearest even) or, for
//   inspection, the int32 sum itself.
//
// Operands: sA [M][Kp] and iBt [N][Kp] (B transposed), both with the K codes
// of a row contiguous and K zero-padded to a multiple of 128, so a tile's
// global loads are unmasked 16-byte vectors along K.
//
// Kernel: 128x128 output tile per 256-thread workgroup, K-step 64. Four waves
// in a 2x2 grid each own 64x64 = 2x2 blocks of v_mfma_i32_32x32x32_i8
// (16 int32 accumulators per lane per block). Tiles are staged in LDS with a
// 16-byte row pad (stride 80 B: the 16-byte operand reads of 16 consecutive
// rows land in distinct banks); the next K-step is prefetched into registers
// while the current one is multiplied.
//
// MFMA operand layout (32x32x32 i8): lane l supplies 16 codes of row
// (l % 32) of the A block and 16 codes of column (l % 32) of the B block, at
// the same 16 K positions for A and B (so any fixed assignment of K
// positions to byte slots gives the same sum); the result block holds
// row 8*(r/4) + 4*(l/32) + (r%4), column l % 32 in accumulator r of lane l.
#include "dq_device.h"
#include "dq_kernels.h"

namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDSS = BK + 16;  // LDS row stride in bytes

__device__ __forceinline__ float activate(float v, int act, float alpha) {
    if (act == DQ_ACT_RELU) return v > 0.0f ? v : 0.0f;
    if (act == DQ_ACT_LEAKY_RELU) return v < 0.0f ? v * alpha : v;
    return v;
}

template <int OUT>
__global__ void __launch_bounds__(256)
k_gemm_i8(const int8_t* __restrict__ sA, const int8_t* __restrict__ iBt, int M, int N, int Kp,
          int tiles_n, DqEpilogue ep) {
    __shared__ __attribute__((aligned(16))) int8_t As[BM * LDSS];
    __shared__ __attribute__((aligned(16))) int8_t Bs[BN * LDSS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int tile_m = blockIdx.x / tiles_n;
    const int tile_n = blockIdx.x - tile_m * tiles_n;
    const int m0 = tile_m * BM, n0 = tile_n * BN;

    // global -> register load mapping: 16-byte chunk c in [0, 512) of a
    // 128x64 tile is row c / 4, byte (c % 4) * 16; thread t loads c = t and
    // c = t + 256 (row + 64). Rows past the edge re-read the last row.
    const int lr = tid >> 2, lc = (tid & 3) * 16;
    const int8_t* gA0 = sA + (size_t)min(m0 + lr, M - 1) * Kp + lc;
    const int8_t* gA1 = sA + (size_t)min(m0 + lr + 64, M - 1) * Kp + lc;
    const int8_t* gB0 = iBt + (size_t)min(n0 + lr, N - 1) * Kp + lc;
    const int8_t* gB1 = iBt + (size_t)min(n0 + lr + 64, N - 1) * Kp + lc;

    dq::v4i ra0 = *reinterpret_cast<const dq::v4i*>(gA0);
    dq::v4i ra1 = *reinterpret_cast<const dq::v4i*>(gA1);
    dq::v4i rb0 = *reinterpret_cast<const dq::v4i*>(gB0);
    dq::v4i rb1 = *reinterpret_cast<const dq::v4i*>(gB1);

    dq::v16i acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    const int arow = wm * 64 + (lane & 31);
    const int brow = wn * 64 + (lane & 31);
    const int kofs = (lane >> 5) * 16;

    for (int k0 = 0; k0 < Kp; k0 += BK) {
        *reinterpret_cast<dq::v4i*>(&As[lr * LDSS + lc]) = ra0;
        *reinterpret_cast<dq::v4i*>(&As[(lr + 64) * LDSS + lc]) = ra1;
        *reinterpret_cast<dq::v4i*>(&Bs[lr * LDSS + lc]) = rb0;
        *reinterpret_cast<dq::v4i*>(&Bs[(lr + 64) * LDSS + lc]) = rb1;
        __syncthreads();
        if (k0 + BK < Kp) {
            ra0 = *reinterpret_cast<const dq::v4i*>(gA0 + k0 + BK);
            ra1 = *reinterpret_cast<const dq::v4i*>(gA1 + k0 + BK);
            rb0 = *reinterpret_cast<const dq::v4i*>(gB0 + k0 + BK);
            rb1 = *reinterpret_cast<const dq::v4i*>(gB1 + k0 + BK);
        }
#pragma unroll
        for (int kk = 0; kk < BK; kk += 32) {
            dq::v4i a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                a[i] = *reinterpret_cast<const dq::v4i*>(&As[(arow + 32 * i) * LDSS + kk + kofs]);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                b[j] = *reinterpret_cast<const dq::v4i*>(&Bs[(brow + 32 * j) * LDSS + kk + kofs]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }

    // epilogue
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int col = n0 + wn * 64 + 32 * j + (lane & 31);
        if (col >= N) continue;
        const float sB = ep.scaleB[col];
        const uint32_t cs = (uint32_t)ep.colsumB[col];
        const float bj = ep.bias ? ep.bias[col] : 0.0f;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * 64 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (row >= M) continue;
                const uint32_t corr = (uint32_t)(128 - ep.zeroA[row]) * cs;
                const int32_t sum = (int32_t)((uint32_t)acc[i][j][r] + corr);
                const size_t o = (size_t)row * N + col;
                if (OUT == DQ_OUT_ACC) {
                    reinterpret_cast<int32_t*>(ep.C)[o] = sum;
                } else {
                    float v = (float)sum * ep.scaleA[row];
                    v = v * sB;
                    if (ep.bias) v = v + bj;
                    v = activate(v, ep.act, ep.alpha);
                    if (OUT == DQ_OUT_BF16)
                        reinterpret_cast<uint16_t*>(ep.C)[o] = (uint16_t)dq::f32_to_bf16_bits(v);
                    else
                        reinterpret_cast<float*>(ep.C)[o] = v;
                }
            }
        }
    }
}

}  // namespace

int dq_launch_gemm(const int8_t* sA, const int8_t* iBt, int M, int N, int Kp,
                   const DqEpilogue& ep, hipStream_t s) {
    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const size_t tiles = (size_t)tiles_m * tiles_n;
    if (tiles > 0x7fffffffu) DQ_FAIL(DQ_ERR_ARG, "problem too large for one launch");
    const dim3 grid((unsigned)tiles), block(256);
    switch (ep.out) {
        case DQ_OUT_ACC:
            hipLaunchKernelGGL((k_gemm_i8<DQ_OUT_ACC>), grid, block, 0, s, sA, iBt, M, N, Kp, tiles_n, ep);
            break;
        case DQ_OUT_BF16:
            hipLaunchKernelGGL((k_gemm_i8<DQ_OUT_BF16>), grid, block, 0, s, sA, iBt, M, N, Kp, tiles_n, ep);
            break;
        default:
            hipLaunchKernelGGL((k_gemm_i8<DQ_OUT_F32>), grid, block, 0, s, sA, iBt, M, N, Kp, tiles_n, ep);
            break;
    }
    DQ_LAUNCH_CHECK("gemm_i8");
    return DQ_OK;
}

const char* dq_gemm_info(int, int, int) {
    return "gemm_i8 v_mfma_i32_32x32x32_i8 128x128x64 LDS-staged, fused dequant epilogue";
}
