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
// Operands arrive packed in MFMA fragment order (1 KiB = 32 rows x 32 k,
// laid out exactly as v_mfma_i32_32x32x32_i8 takes them: lane l holds 16
// codes of row l % 32), so
//  - every global load is one 16-byte load per lane over a contiguous 1 KiB,
//  - every LDS write and read is lane-contiguous (no bank conflicts, no
//    swizzle arithmetic),
//  - no bounds checks are needed: M, N are padded to 256 and K to 128.
//
// Kernel k_gemm<WM, WN, FM, FN, KS>: a workgroup of WM x WN waves computes a
// (WM*FM*32) x (WN*FN*32) tile of C; each wave owns FM x FN 32x32 blocks
// (16 int32 accumulators per lane per block). K advances 32*KS per step: the
// step's fragments are staged global -> VGPR -> LDS into a double buffer
// while the previous step is multiplied, one barrier per step. Within a
// step the next step's global loads and the next sub-step's LDS reads are
// interleaved one by one with the MFMAs (scheduling groups), so the vector
// memory path, the LDS and the matrix cores work at the same time. The
// largest configuration, 256x256x128 with four 128x128 waves (256
// accumulator AGPRs per lane, 128 KiB of LDS), multiplies for 2048 MFMA
// cycles per step.
//
// The MFMA's first operand is the B fragment and its second the A fragment,
// so the accumulator block is C^T: lane l holds row (l % 32) of the block and,
// in accumulators 4g..4g+3, the four adjacent columns 8g + 4(l/32) + 0..3.
// Epilogue: the tile's row and column parameters are staged in LDS when the
// kernel starts; each wave finishes one 32-row strip at a time in
// registers (activation and bias are template parameters: no per-element
// branches), writes it to a wave-private, XOR-swizzled LDS strip and stores
// it back as whole row segments, 16 bytes per lane, so the stores of one
// strip overlap the arithmetic of the next.
//
// Tile order: consecutive workgroups land on different XCDs (round robin),
// so the workgroup index is first regrouped per XCD, then rastered in
// groups of four tile rows: the 32 tiles an XCD runs at once span 4 tile
// rows x 8 tile columns and share their A and B panels in that XCD's L2.
#include "dq_device.h"
#include "dq_kernels.h"

#include <type_traits>

namespace {

constexpr int kGM = 4;    // tile rows per raster group
constexpr int kXCD = 8;   // XCDs of an MI355X

template <int ACT>
__device__ __forceinline__ float activate(float v, float alpha) {
    if (ACT == DQ_ACT_RELU) return v > 0.0f ? v : 0.0f;
    if (ACT == DQ_ACT_LEAKY_RELU) return v < 0.0f ? v * alpha : v;
    return v;
}

template <int WM, int WN, int FM, int FN, int KS, int OUT, int ACT, bool BIAS>
__global__ void __launch_bounds__(WM * WN * 64)
k_gemm(const int8_t* __restrict__ Ap, const int8_t* __restrict__ Bp, int M, int N, int KF,
       int tiles_m, int tiles_n, int vec_store, DqEpilogue ep) {
    constexpr int NW = WM * WN;
    constexpr int NT = NW * 64;
    constexpr int BMF = WM * FM;        // A (row) fragments per tile
    constexpr int BNF = WN * FN;        // B (column) fragments per tile
    constexpr int BM = BMF * 32, BN = BNF * 32;
    constexpr int AF = BMF * KS;        // A fragments per step
    constexpr int TF = AF + BNF * KS;   // all fragments per step
    constexpr int FPW = (TF + NW - 1) / NW;
    constexpr int FPK = (FPW + KS - 1) / KS;  // global loads per sub-step
    __shared__ __attribute__((aligned(16))) int8_t lds[2][TF * 1024];
    __shared__ __attribute__((aligned(16))) int32_t s_cs[BN];
    __shared__ __attribute__((aligned(16))) float s_sb[BN];
    __shared__ __attribute__((aligned(16))) float s_bias[BN];
    __shared__ float s_sa[BM];
    __shared__ int32_t s_za[BM];

    const int lane = threadIdx.x & 63;
    // wave-uniform values live in SGPRs: every fragment address is a scalar
    // base plus the one per-lane offset lane * 16
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WN, wn = wave % WN;

    // XCD-aware tile order
    const int nb = tiles_m * tiles_n;
    int b = blockIdx.x;
    if (nb % kXCD == 0) b = (b % kXCD) * (nb / kXCD) + b / kXCD;
    const int group = b / (kGM * tiles_n);
    const int first_m = group * kGM;
    const int gm = min(tiles_m - first_m, kGM);
    const int in_group = b - group * kGM * tiles_n;
    const int tm = first_m + in_group % gm;
    const int tn = in_group / gm;
    const int m0 = tm * BM, n0 = tn * BN;

    const int8_t* a_tile = Ap + (size_t)(tm * BMF) * KF * 1024;
    const int8_t* b_tile = Bp + (size_t)(tn * BNF) * KF * 1024;
    const int lofs = lane * 16;
    // fragment f of a step (f < AF: A, else B) at step t
    auto frag_src = [&](int f, int t) -> const int8_t* {
        const int8_t* base = f < AF ? a_tile : b_tile;
        const int g = f < AF ? f : f - AF;
        return base + ((size_t)(g / KS) * KF + (size_t)t * KS + g % KS) * 1024;
    };
    constexpr bool kAllActive = TF % NW == 0;
    auto active = [&](int i) { return i < FPW && (kAllActive || wave + i * NW < TF); };

    // row / column parameters of the tile (column vectors hold Np entries)
    for (int c = threadIdx.x; c < BN; c += NT) {
        s_cs[c] = ep.colsumB[n0 + c];
        if (OUT != DQ_OUT_ACC) {
            s_sb[c] = ep.scaleB[n0 + c];
            s_bias[c] = BIAS ? ep.bias[n0 + c] : 0.0f;
        }
    }
    for (int r = threadIdx.x; r < BM; r += NT) {
        const int row = min(m0 + r, M - 1);
        s_za[r] = ep.zeroA[row];
        if (OUT != DQ_OUT_ACC) s_sa[r] = ep.scaleA[row];
    }

    dq::v4i stage[FPW];
#pragma unroll
    for (int i = 0; i < FPW; ++i)
        if (active(i)) stage[i] = *reinterpret_cast<const dq::v4i*>(frag_src(wave + i * NW, 0) + lofs);
#pragma unroll
    for (int i = 0; i < FPW; ++i)
        if (active(i)) *reinterpret_cast<dq::v4i*>(&lds[0][(wave + i * NW) * 1024 + lofs]) = stage[i];
    __syncthreads();

    dq::v16i acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    // One step: the MFMAs of buffer L; when FETCH, the global loads of step
    // `next` (FPK per sub-step) and, always, the LDS reads of sub-step kk+1
    // are interleaved with the MFMAs of sub-step kk.
    auto step = [&](const int8_t* L, auto fetch, int next) {
        constexpr bool FETCH = decltype(fetch)::value;
        dq::v4i fa[2][FM], fb[2][FN];
        auto read = [&](int kk, int set) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
                fa[set][i] = *reinterpret_cast<const dq::v4i*>(L + ((wm * FM + i) * KS + kk) * 1024 + lofs);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                fb[set][j] = *reinterpret_cast<const dq::v4i*>(L + (AF + (wn * FN + j) * KS + kk) * 1024 + lofs);
        };
        read(0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            const int set = kk & 1;
            if (FETCH) {
#pragma unroll
                for (int q = 0; q < FPK; ++q) {
                    const int i = kk * FPK + q;
                    if (active(i)) stage[i] = *reinterpret_cast<const dq::v4i*>(frag_src(wave + i * NW, next) + lofs);
                }
            }
            if (kk + 1 < KS) read(kk + 1, set ^ 1);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fb[set][j], fa[set][i], acc[i][j], 0, 0, 0);
            // order: one MFMA, then one global load and one LDS read, ...
#pragma unroll
            for (int m = 0; m < FM * FN; ++m) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (FETCH && m < FPK) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                if (kk + 1 < KS && m < FM + FN) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // main loop; the last step is peeled so the loop body has no
    // conditional code (a rolled condition here makes the compiler keep the
    // accumulators in scratch)
    const int nsteps = KF / KS;
    for (int t = 0; t + 1 < nsteps; ++t) {
        const int cur = t & 1;
        step(lds[cur], std::true_type{}, t + 1);
#pragma unroll
        for (int i = 0; i < FPW; ++i)
            if (active(i)) *reinterpret_cast<dq::v4i*>(&lds[cur ^ 1][(wave + i * NW) * 1024 + lofs]) = stage[i];
        __syncthreads();
    }
    step(lds[(nsteps - 1) & 1], std::false_type{}, 0);

    // ---- epilogue (see the header): wave-private strips of 32 rows
    constexpr int OB = OUT == DQ_OUT_BF16 ? 2 : 4;  // bytes per output
    constexpr int RB = FN * 32 * OB;                // bytes per strip row
    constexpr int CPR = RB / 16;                    // 16-byte chunks per strip row
    constexpr int EPC = 16 / OB;                    // elements per chunk
    constexpr int SB = 32 * RB;                     // bytes per strip
    static_assert(NW * SB <= 2 * TF * 1024, "epilogue strips do not fit in LDS");
    int8_t* strip = &lds[0][0] + wave * SB;
    __syncthreads();  // every wave is done reading the stage buffers
#pragma clang loop unroll(full)
    for (int i = 0; i < FM; ++i) {
        const int rt = (wm * FM + i) * 32 + (lane & 31);  // tile row
        const int rs = lane & 31;                        // strip row
        const uint32_t za = (uint32_t)(128 - s_za[rt]);
        const float sA = OUT == DQ_OUT_ACC ? 0.0f : s_sa[rt];
#pragma clang loop unroll(full)
        for (int j = 0; j < FN; ++j) {
#pragma clang loop unroll(full)
            for (int g = 0; g < 4; ++g) {
                const int cs_ = j * 32 + 8 * g + 4 * (lane >> 5);  // strip column
                const int ct = wn * FN * 32 + cs_;                  // tile column
                const dq::v4i cs = *reinterpret_cast<const dq::v4i*>(&s_cs[ct]);
                int32_t sum[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sum[e] = (int32_t)((uint32_t)acc[i][j][4 * g + e] + za * (uint32_t)cs[e]);
                const int byte = cs_ * OB;
                int8_t* dst = strip + rs * RB + (((byte >> 4) ^ (rs & (CPR - 1))) << 4) + (byte & 15);
                if (OUT == DQ_OUT_ACC) {
                    const dq::v4i v = {sum[0], sum[1], sum[2], sum[3]};
                    *reinterpret_cast<dq::v4i*>(dst) = v;
                } else {
                    const dq::f4 sB = *reinterpret_cast<const dq::f4*>(&s_sb[ct]);
                    dq::f4 bv = {0.0f, 0.0f, 0.0f, 0.0f};
                    if (BIAS) bv = *reinterpret_cast<const dq::f4*>(&s_bias[ct]);
                    dq::f4 val;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float v = (float)sum[e] * sA;
                        v = v * sB[e];
                        if (BIAS) v = v + bv[e];
                        val[e] = activate<ACT>(v, ep.alpha);
                    }
                    if (OUT == DQ_OUT_BF16)
                        *reinterpret_cast<dq::u2*>(dst) = dq::f32x4_to_bf16x4(val);
                    else
                        *reinterpret_cast<dq::f4*>(dst) = val;
                }
            }
        }
        // the strip back as row segments: chunk q -> strip row q / CPR;
        // LDS operations of one wave complete in order, so no barrier
        const int row0 = m0 + (wm * FM + i) * 32;
        const int col0 = n0 + wn * FN * 32;
#pragma unroll
        for (int q = lane; q < 32 * CPR; q += 64) {
            const int r = q / CPR, c = q % CPR;
            const int row = row0 + r, col = col0 + c * EPC;
            const dq::v4i v = *reinterpret_cast<const dq::v4i*>(strip + r * RB + ((c ^ (r & (CPR - 1))) << 4));
            if (row < M && col < N) {
                int8_t* C = reinterpret_cast<int8_t*>(ep.C) + ((size_t)row * N + col) * OB;
                if (vec_store && col + EPC <= N) {
                    *reinterpret_cast<dq::v4i*>(C) = v;
                } else {
#pragma unroll
                    for (int e = 0; e < EPC; ++e) {
                        if (col + e < N) {
                            const uint32_t w = (uint32_t)v[(e * OB) >> 2];
                            if (OB == 2)
                                reinterpret_cast<uint16_t*>(C)[e] = (uint16_t)(w >> (16 * (e & 1)));
                            else
                                reinterpret_cast<uint32_t*>(C)[e] = w;
                        }
                    }
                }
            }
        }
    }
}

template <int WM, int WN, int FM, int FN, int KS, int OUT, int ACT, bool BIAS>
void launch_one(dim3 grid, hipStream_t s, const int8_t* Ap, const int8_t* Bp, int M, int N, int KF,
                int tiles_m, int tiles_n, int vec_store, const DqEpilogue& ep) {
    hipLaunchKernelGGL((k_gemm<WM, WN, FM, FN, KS, OUT, ACT, BIAS>), grid, dim3(WM * WN * 64), 0, s,
                       Ap, Bp, M, N, KF, tiles_m, tiles_n, vec_store, ep);
}

template <int WM, int WN, int FM, int FN, int KS, int OUT>
void launch_act(dim3 grid, hipStream_t s, const int8_t* Ap, const int8_t* Bp, int M, int N, int KF,
                int tiles_m, int tiles_n, int vec_store, const DqEpilogue& ep) {
#define DQ_G(ACT, BIAS) launch_one<WM, WN, FM, FN, KS, OUT, ACT, BIAS>(grid, s, Ap, Bp, M, N, KF, tiles_m, tiles_n, vec_store, ep)
    const bool bias = ep.bias != nullptr;
    switch (ep.act) {
        case DQ_ACT_RELU: if (bias) DQ_G(DQ_ACT_RELU, true); else DQ_G(DQ_ACT_RELU, false); break;
        case DQ_ACT_LEAKY_RELU: if (bias) DQ_G(DQ_ACT_LEAKY_RELU, true); else DQ_G(DQ_ACT_LEAKY_RELU, false); break;
        default: if (bias) DQ_G(DQ_ACT_IDENTITY, true); else DQ_G(DQ_ACT_IDENTITY, false); break;
    }
#undef DQ_G
}

template <int WM, int WN, int FM, int FN, int KS>
int launch(const int8_t* Ap, const int8_t* Bp, int M, int N, int Kp, const DqEpilogue& ep,
           hipStream_t s) {
    constexpr int BM = WM * FM * 32, BN = WN * FN * 32;
    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const size_t tiles = (size_t)tiles_m * tiles_n;
    if (tiles > 0x7fffffffu) DQ_FAIL(DQ_ERR_ARG, "problem too large for one launch");
    // whole 16-byte chunks of C rows: 8 bf16 or 4 fp32 / int32 per chunk
    const int ob = ep.out == DQ_OUT_BF16 ? 2 : 4;
    const int vec_store = (uintptr_t)ep.C % 16 == 0 && ((size_t)N * ob) % 16 == 0;
    const dim3 grid((unsigned)tiles);
    const int KF = Kp / 32;
    switch (ep.out) {
        case DQ_OUT_ACC:
            launch_one<WM, WN, FM, FN, KS, DQ_OUT_ACC, DQ_ACT_IDENTITY, false>(grid, s, Ap, Bp, M, N, KF, tiles_m, tiles_n, vec_store, ep);
            break;
        case DQ_OUT_BF16:
            launch_act<WM, WN, FM, FN, KS, DQ_OUT_BF16>(grid, s, Ap, Bp, M, N, KF, tiles_m, tiles_n, vec_store, ep);
            break;
        default:
            launch_act<WM, WN, FM, FN, KS, DQ_OUT_F32>(grid, s, Ap, Bp, M, N, KF, tiles_m, tiles_n, vec_store, ep);
            break;
    }
    DQ_LAUNCH_CHECK("gemm_i8");
    return DQ_OK;
}

// Picks the tile: 256x256 when it yields enough workgroups to fill the
// chip's 256 CUs, else 128x128, else 32x32 for small / skinny problems.
int pick(int M, int N) {
    const long big = (long)((M + 255) / 256) * ((N + 255) / 256);
    const long mid = (long)((M + 127) / 128) * ((N + 127) / 128);
    if (big >= 192) return 2;
    if (mid >= 96) return 1;
    return 0;
}

}  // namespace

int dq_launch_gemm(const int8_t* Ap, const int8_t* Bp, int M, int N, int Kp, const DqEpilogue& ep,
                   hipStream_t s) {
    switch (pick(M, N)) {
        case 2: return launch<2, 2, 4, 4, 4>(Ap, Bp, M, N, Kp, ep, s);
        case 1: return launch<2, 2, 2, 2, 4>(Ap, Bp, M, N, Kp, ep, s);
        default: return launch<1, 1, 1, 1, 4>(Ap, Bp, M, N, Kp, ep, s);
    }
}

const char* dq_gemm_info(int M, int N, int) {
    switch (pick(M, N)) {
        case 2: return "gemm_i8 v_mfma_i32_32x32x32_i8 tile 256x256x128 (4 waves x 128x128), fragment-packed operands, LDS double buffer, fused dequant epilogue";
        case 1: return "gemm_i8 v_mfma_i32_32x32x32_i8 tile 128x128x128 (4 waves x 64x64), fragment-packed operands, LDS double buffer, fused dequant epilogue";
        default: return "gemm_i8 v_mfma_i32_32x32x32_i8 tile 32x32x128 (1 wave), fragment-packed operands, fused dequant epilogue";
    }
}
