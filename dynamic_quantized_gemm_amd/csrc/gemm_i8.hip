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
// Operands arrive packed in fragment order (1 KiB = 32 rows x 32 k, lane l
// of a wave holding 16 codes of row l % 32, k half l / 32), so
//  - every global -> LDS copy moves one contiguous 1 KiB per wave, 16 bytes
//    per lane, and lands in LDS in the same order,
//  - every LDS read is one 16-byte piece per lane, 256 contiguous bytes per
//    16 lanes (ds_read_b128, no bank conflicts, no swizzle arithmetic),
//  - no bounds checks are needed: M, N are padded to 256 and K to 256.
//
// Kernel k_gemm<WM, WN, FM, FN, KS>: a workgroup of WM x WN waves computes a
// (WM*FM*32) x (WN*FN*32) tile of C; each wave owns 2FM x 2FN blocks of
// 16x16, multiplied with v_mfma_i32_16x16x64_i8 (4 int32 accumulators per
// lane per block). K advances 32*KS = 64 per step. The fragments of a step go global -> LDS directly (gfx950
// global_load_lds_dwordx4, no trip through VGPRs) into a ring of four stage
// buffers: while step t is multiplied out of its stage, the copies for steps
// t+1 .. t+3 are in flight, so a copy has three steps of matrix work to
// arrive. The compiler does not see these copies as LDS writes, so the
// kernel waits for them itself (s_waitcnt vmcnt with the count of copies
// still allowed in flight) and crosses one bare s_barrier per step. Within a
// step the copies and the next sub-step's LDS reads are interleaved one by
// one with the MFMAs (in program order), so the vector memory path, the LDS
// and the matrix cores work at the same time. The largest configuration,
// 256x256 with four 128x128 waves, keeps 256 accumulator registers per lane
// in AGPRs and issues 64 MFMAs per wave per step. Of gfx950's two int8 MFMA
// shapes (32x32x32 and 16x16x64, the same operations per cycle) the 16x16x64
// one moves fewer accumulator bits per operation; on this power-limited part
// it runs at a higher clock (measured: an MFMA-only loop reaches 3.46 POP/s
// against 2.9-3.2 for 32x32x32, random operands).
//
// The MFMA's first operand is the B block and its second the A block, so
// the accumulator block is C^T: lane l holds row (l % 16) of the block and,
// in its four accumulators, the adjacent columns 4(l/16) + 0..3.
// Epilogue: the tile's row and column parameters are staged in LDS when the
// kernel starts; after the main loop each wave owns one quarter of the stage
// memory. Its rows are finished in passes of as many 32-row strips as fit
// there: for each column group (loaded once per pass) the accumulators are
// read one by one out of the AGPRs, corrected, scaled, biased and activated
// in registers (activation and bias are template parameters: no per-element
// branches) and written to an XOR-swizzled LDS image of the pass, which then
// goes back to C as whole row segments, 16 bytes per lane.
//
// Tile order: consecutive workgroups land on different XCDs (round robin),
// so the workgroup index is first regrouped per XCD, then rastered in
// groups of four tile rows: the 32 tiles an XCD runs at once span 4 tile
// rows x 8 tile columns and share their A and B panels in that XCD's L2.
#include "dq_device.h"
#include "dq_kernels.h"

#include <hip/hip_ext.h>

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

template <int WM, int WN, int FM, int FN, int KS, int OUT, int ACT, bool BIAS, bool EXT>
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
    static_assert(TF % NW == 0, "every wave copies the same number of fragments");
    constexpr int FPW = TF / NW;              // fragment copies per wave per step
    constexpr int FPK = (FPW + KS - 1) / KS;  // fragment copies per sub-step
    constexpr int NSTAGE = 4;                 // LDS ring: steps t .. t + 3
    constexpr int SBYTES = TF * 1024;         // bytes per stage
    // four separate arrays (not one indexed array): each gets its own alias
    // scope, so the compiler can see that a step's LDS reads never touch
    // the stage its in-flight copies write, and adds no waits for them
    __shared__ __attribute__((aligned(16))) int8_t st0[SBYTES];
    __shared__ __attribute__((aligned(16))) int8_t st1[SBYTES];
    __shared__ __attribute__((aligned(16))) int8_t st2[SBYTES];
    __shared__ __attribute__((aligned(16))) int8_t st3[SBYTES];
    __shared__ __attribute__((aligned(16))) int32_t s_cs[BN];
    __shared__ __attribute__((aligned(16))) float s_sb[BN];
    __shared__ __attribute__((aligned(16))) float s_bias[BN];
    __shared__ float s_sa[BM];
    __shared__ int32_t s_za[BM];
    // EXT (the quantized matrix products): B zero points against A's row sums
    __shared__ int32_t s_rb[EXT ? BM : 1];
    __shared__ __attribute__((aligned(16))) int32_t s_zb[EXT ? BN : 4];
    // EXT: a C broadcast along rows (one value per column) or along columns
    __shared__ int32_t s_crow[EXT ? BM : 1];
    __shared__ __attribute__((aligned(16))) int32_t s_ccol[EXT ? BN : 4];

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
    const int nsteps = KF / KS;

    // row / column parameters of the tile (column vectors hold Np entries;
    // bias may be a caller's tensor of N values, so its index is clamped)
    for (int c = threadIdx.x; c < BN; c += NT) {
        s_cs[c] = ep.colsumB[n0 + c];
        if (EXT) {
            s_zb[c] = ep.zeroB ? ep.zeroB[n0 + c] : 0;
            s_ccol[c] = ep.c_mode == 1 ? ep.addC[(long long)min(n0 + c, N - 1) * ep.c_cs] : 0;
        }
        if (OUT != DQ_OUT_ACC) {
            s_sb[c] = ep.scaleB[n0 + c];
            s_bias[c] = BIAS ? ep.bias[min(n0 + c, N - 1)] : 0.0f;
        }
    }
    for (int r = threadIdx.x; r < BM; r += NT) {
        const int row = min(m0 + r, M - 1);
        s_za[r] = ep.zeroA[row];
        if (EXT) {
            s_rb[r] = ep.rowsumA ? ep.rowsumA[row] : 0;
            s_crow[r] = ep.c_mode == 2 ? ep.addC[(long long)row * ep.c_rs] : 0;
        }
        if (OUT != DQ_OUT_ACC) s_sa[r] = ep.scaleA[row];
    }

    // Fragment copies go straight from global memory to LDS
    // (global_load_lds_dwordx4: a wave's 64 lanes x 16 bytes land as one
    // contiguous 1 KiB block, exactly a packed fragment), without VGPRs.
    // Step t lives in LDS stage t % 4; the copies of step t + 3 are issued
    // while step t is multiplied. The compiler does not track these writes,
    // so the waits are explicit (vector memory operations complete in
    // order; see the step below). Steps past the end re-load the last step
    // (in bounds, never used), which keeps the loop body free of
    // conditional code.
    auto stage = [&](auto S) -> int8_t* {
        constexpr int k = decltype(S)::value % NSTAGE;
        if constexpr (k == 0) return st0;
        else if constexpr (k == 1) return st1;
        else if constexpr (k == 2) return st2;
        else return st3;
    };
    // A copy's source is a per-step scalar base (the tile panel moved to
    // step t) plus a fixed 32-bit offset per copy slot (fragment row block
    // and k half inside the panel, and the lane's 16 bytes): the step moves
    // one base, not every address (fewer instructions between the MFMAs).
    uint32_t voff[FPW];
#pragma unroll
    for (int i = 0; i < FPW; ++i) {
        const int f = wave + i * NW;
        const int g = f < AF ? f : f - AF;
        voff[i] = (uint32_t)(((g / KS) * KF + g % KS) * 1024) + (uint32_t)lofs;
    }
    auto copy = [&](int i, int t, int8_t* dst) {
        const int f = wave + i * NW;
        const int tc = min(t, nsteps - 1);
        const int8_t* base = (f < AF ? a_tile : b_tile) + (size_t)tc * (KS * 1024);
        dq::copy16_to_lds(base + voff[i], dst + f * 1024);
    };
#pragma unroll
    for (int i = 0; i < FPW; ++i) copy(i, 0, st0);
#pragma unroll
    for (int i = 0; i < FPW; ++i) copy(i, 1, st1);
#pragma unroll
    for (int i = 0; i < FPW; ++i) copy(i, 2, st2);

    // Each wave multiplies 2FM x 2FN blocks of 16x16 with
    // v_mfma_i32_16x16x64_i8, 4 accumulators per lane per block, held in
    // AGPRs and read one by one in the epilogue (dq::acc_read).
    constexpr int HM = 2 * FM, HN = 2 * FN;  // 16-row / 16-column blocks per wave
    dq::v4i acc[HM][HN];
#pragma unroll
    for (int i = 0; i < HM; ++i)
#pragma unroll
        for (int j = 0; j < HN; ++j) acc[i][j] = dq::v4i{0, 0, 0, 0};

    // Operand blocks. The 16x16x64 MFMA takes, in lane l, 16 codes of row
    // (or column) l % 16 from k group l / 16 of a 64-deep step. Those 16
    // codes sit, in the packed 32x32 fragments, in the 16-byte piece of
    // packed lane (l % 16) + 16 h + 32 (g % 2) of the step's 32-deep
    // fragment g / 2 (h: which half of the 32 rows). A and B are packed
    // alike and read through the same map, so every k group meets the same
    // k values in both operands: the integer sum is the same sum in another
    // order (exact). Each lane still reads one 16-byte piece per block, and
    // each group of 16 lanes a contiguous 256 bytes.
    static_assert(KS == 2, "a step is two 32-deep packed fragments");
    const int hofs = ((lane >> 5) & 1) * 1024 + ((lane >> 4) & 1) * 512 + (lane & 15) * 16;
    auto rdA = [&](const int8_t* L, int hb) {
        return *reinterpret_cast<const dq::v4i*>(L + (wm * FM + (hb >> 1)) * KS * 1024 + (hb & 1) * 256 + hofs);
    };
    auto rdB = [&](const int8_t* L, int hb) {
        return *reinterpret_cast<const dq::v4i*>(L + (AF + (wn * FN + (hb >> 1)) * KS) * 1024 + (hb & 1) * 256 + hofs);
    };
    // The MFMA accumulates in place (dst = srcC). It is written as inline
    // assembly: with 4-register accumulators the compiler's builtin form
    // lets the register allocator move whole accumulator sets between
    // AGPRs and VGPRs inside the loop (hundreds of moves a step). Hazards
    // the compiler therefore does not see:
    //  (1) the zeroing writes (VALU) before the first MFMA reads them as
    //      srcC: an empty volatile statement per block pins the zeros in
    //      their AGPRs, then a drain of more wait states than the ISA asks
    //      for a VALU write followed by an MFMA srcC read;
    //  (2) the epilogue's reads of the results: mfma_result_drain after the
    //      loop.
    // The operand VGPRs come from LDS reads, whose completion the
    // compiler's waitcnt pass tracks for inline-assembly operands as for
    // any other use; nothing but these MFMAs writes the accumulators, and
    // consecutive updates of one block are a whole sub-step apart.
    auto mfma = [](dq::v4i& c, const dq::v4i& b, const dq::v4i& a) {
        asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(c) : "v"(b), "v"(a));
    };
#pragma unroll
    for (int i = 0; i < HM; ++i)
#pragma unroll
        for (int j = 0; j < HN; ++j) asm volatile("" : "+a"(acc[i][j]));
    dq::mfma_result_drain();

    // A step is two sub-steps: the first multiplies the wave's upper FM row
    // blocks (faL) by all its column blocks, the second the lower FM
    // (faH). B blocks live for a whole step, in two register sets that
    // alternate between steps. The first sub-step reads faH of the same
    // step; the second, after the step's barrier, reads faL and the other B
    // set of the next step. Within a sub-step the copies and reads are
    // interleaved one by one with the MFMAs, in program order (the inline
    // MFMAs are volatile, so the compiler keeps the order): one MFMA, then
    // one copy and one read, ...
    dq::v4i faL[FM], faH[FM], fb[2][HN];
    // slots of a sub-step: its MFMAs, or more where a small tile has more
    // copies or reads than MFMAs
    constexpr int kSlots = FM * HN > FPK ? (FM * HN > FM + HN ? FM * HN : FM + HN)
                                         : (FPK > FM + HN ? FPK : FM + HN);

    // Step t multiplies stage L = t % 4; its faL and B blocks were read
    // during step t - 1. The one barrier of the step sits between its two
    // sub-steps: before it, this wave's reads of L have completed (lgkmcnt
    // 0) and its copies of step t + 1 have landed (at most the copies of step
    // t + 2 and the first half of step t + 3's are still in flight); after
    // it, every wave's copies of step t + 1 are visible, so the second
    // sub-step can read step t + 1's blocks, and no wave reads L any more,
    // so the copies of step t + 4, issued from step t + 1 on, may overwrite
    // it. No LDS read waits behind a barrier.
    // Not __syncthreads(): its fence would wait for every outstanding copy.
    auto one = [&](auto S, int t) {
        constexpr int c = decltype(S)::value & 1;  // B register set of step t
        using SN = std::integral_constant<int, decltype(S)::value + 1>;
        using SA = std::integral_constant<int, decltype(S)::value + NSTAGE - 1>;
        const int8_t* L = stage(S);
        const int8_t* Ln = stage(SN{});
        int8_t* dst = stage(SA{});
#pragma unroll
        for (int m = 0; m < kSlots; ++m) {
            if (m < FM * HN) mfma(acc[m / HN][m % HN], fb[c][m % HN], faL[m / HN]);
            if (m < FPK && m < FPW) copy(m, t + NSTAGE - 1, dst);
            if (m < FM) faH[m] = rdA(L, FM + m);
        }
        dq::wait_vmcnt_lgkm0<FPW + FPK>();
        dq::lds_barrier();
#pragma unroll
        for (int m = 0; m < kSlots; ++m) {
            if (m < FM * HN) mfma(acc[FM + m / HN][m % HN], fb[c][m % HN], faH[m / HN]);
            if (m < FPK && FPK + m < FPW) copy(FPK + m, t + NSTAGE - 1, dst);
            if (m < FM) faL[m] = rdA(Ln, m);
            else if (m < FM + HN) fb[c ^ 1][m - FM] = rdB(Ln, m - FM);
        }
    };
    // step 0's copies, then its first blocks
    dq::wait_vmcnt_lgkm0<2 * FPW>();
    dq::lds_barrier();
#pragma unroll
    for (int i = 0; i < FM; ++i) faL[i] = rdA(st0, i);
#pragma unroll
    for (int j = 0; j < HN; ++j) fb[0][j] = rdB(st0, j);
    // unrolled by the ring size so every stage reference and register set is
    // static (the step count is a multiple of 4: Kp is a multiple of 256);
    // the last step's look-ahead reads a re-loaded stage and is never used
    for (int t = 0; t < nsteps; t += NSTAGE) {
        one(std::integral_constant<int, 0>{}, t);
        one(std::integral_constant<int, 1>{}, t + 1);
        one(std::integral_constant<int, 2>{}, t + 2);
        one(std::integral_constant<int, 3>{}, t + 3);
    }
    dq::wait_vmcnt<0>();  // the trailing copies land before LDS is reused
    // the epilogue reads the accumulators through inline assembly
    // (dq::acc_read), which the compiler does not check against the last
    // MFMA: give the results the ISA's wait states first
    dq::mfma_result_drain();

    // ---- epilogue (see the header). The wave's output rows are cut into
    // strips of 32 (one per A fragment row); as many strips as fit in the
    // wave's private 1/4 of the stage memory are finished per pass. Column
    // groups are the outer loop, so each group's column parameters are read
    // from LDS once for all strips of the pass, and the strips give
    // independent work to hide the reads' latency.
    constexpr bool Q8 = OUT == DQ_OUT_U8 || OUT == DQ_OUT_I8;  // requantized 8-bit output
    constexpr int OB = Q8 ? 1 : OUT == DQ_OUT_BF16 ? 2 : 4;    // bytes per output
    constexpr int RB = FN * 32 * OB;                // bytes per strip row
    constexpr int CPR = RB / 16;                    // 16-byte chunks per strip row
    constexpr int EPC = 16 / OB;                    // elements per chunk
    constexpr int SB = 32 * RB;                     // bytes per strip
    constexpr int SPP = (SBYTES / SB) < FM ? (SBYTES / SB) : FM;  // strips per pass
    static_assert(SPP >= 1 && FM % SPP == 0 && NW <= NSTAGE, "epilogue strips do not fit in LDS");
    int8_t* region = wave == 0 ? st0 : wave == 1 ? st1 : wave == 2 ? st2 : st3;
    __syncthreads();  // every wave is done reading the stage buffers
    // in a 16x16 accumulator block lane l holds row l % 16 and, in its four
    // accumulators, the adjacent columns 4 (l / 16) + 0..3
    const int rq = lane & 15;
    const int col0 = n0 + wn * FN * 32;
    // requantization of an 8-bit output: y = sat(rne(val / y_scale) + y_zp),
    // with the corrected quotient where the scale allows it (as the
    // quantizers round), the 1.5 * 2^23 rounding add, a median clamp against
    // the saturation bounds minus the zero point, and the zero point added to
    // four packed codes at once (carry-free bytewise add)
    constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
    dq::QDiv yd = {1.0f, 1.0f, true};
    int yz = 0;
    float ylo = 0.0f, yhi = 0.0f;
    if (Q8) {
        yd = dq::make_qdiv(ep.y_scale[0]);
        if (ep.y_zp) yz = OUT == DQ_OUT_U8 ? (int)*reinterpret_cast<const uint8_t*>(ep.y_zp)
                                           : (int)*reinterpret_cast<const int8_t*>(ep.y_zp);
        ylo = (float)((OUT == DQ_OUT_U8 ? 0 : -128) - yz);
        yhi = (float)((OUT == DQ_OUT_U8 ? 255 : 127) - yz);
    }
    const uint32_t yZ = (uint32_t)(yz & 0xff) * 0x01010101u;
#pragma clang loop unroll(full)
    for (int p0 = 0; p0 < FM; p0 += SPP) {
        // the correction (128 - zeroA) * colsum on the 24-bit multiplier (full
        // rate; a 32-bit product would take the quarter-rate 64-bit multiply-
        // add): |128 - zeroA| <= 128 and -2^23 <= colsum < 2^23 for K <= 65536,
        // so the product is exact and the wrapping add gives the exact sum
        // the lane's two rows of each strip: 16 h + rq, h = 0, 1
        int za[SPP][2], rb[SPP][2], cr[SPP][2];
        float sA[SPP][2];
#pragma unroll
        for (int u = 0; u < SPP; ++u)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int rt = (wm * FM + p0 + u) * 32 + 16 * h + rq;  // tile row
                za[u][h] = 128 - s_za[rt];
                rb[u][h] = EXT ? s_rb[rt] : 0;
                cr[u][h] = EXT ? s_crow[rt] : 0;
                sA[u][h] = OUT == DQ_OUT_ACC ? 0.0f : s_sa[rt];
            }
        // groups jg = 2 jb + h: column block jb, row half h; each column
        // block's parameters are read from LDS one block ahead, so their
        // latency hides behind the previous block's arithmetic
        dq::v4i csv[2], zbv[2], ccv[2];
        dq::f4 sBv[2], bvv[2];
        auto params = [&](int jb, int set) {
            const int ct = wn * FN * 32 + jb * 16 + 4 * (lane >> 4);  // tile column
            csv[set] = *reinterpret_cast<const dq::v4i*>(&s_cs[ct]);
            if (EXT) {
                zbv[set] = *reinterpret_cast<const dq::v4i*>(&s_zb[ct]);
                ccv[set] = *reinterpret_cast<const dq::v4i*>(&s_ccol[ct]);
            }
            if (OUT != DQ_OUT_ACC) sBv[set] = *reinterpret_cast<const dq::f4*>(&s_sb[ct]);
            if (OUT != DQ_OUT_ACC && BIAS) bvv[set] = *reinterpret_cast<const dq::f4*>(&s_bias[ct]);
        };
        params(0, 0);
#pragma clang loop unroll(full)
        for (int jg = 0; jg < HN * 2; ++jg) {
            const int jb = jg >> 1, h = jg & 1, set = jb & 1;
            if (h == 0 && jb + 1 < HN) params(jb + 1, set ^ 1);
            {
                const int rs = 16 * h + rq;                  // strip row
                const int cs_ = jb * 16 + 4 * (lane >> 4);  // strip column
                const dq::v4i cs = csv[set];
                dq::f4 sB = {0.0f, 0.0f, 0.0f, 0.0f}, bv = {0.0f, 0.0f, 0.0f, 0.0f};
                if (OUT != DQ_OUT_ACC) sB = sBv[set];
                if (OUT != DQ_OUT_ACC && BIAS) bv = bvv[set];
                const int byte = cs_ * OB;
#pragma unroll
                for (int u = 0; u < SPP; ++u) {
                    int32_t sum[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        sum[e] = (int32_t)((uint32_t)dq::acc_read(acc[2 * (p0 + u) + h][jb][e]) +
                                           (uint32_t)__mul24(za[u][h], cs[e]));
                    if (EXT) {
                        // B zero points: + rowsumA[i] * zb[j], where rowsumA holds
                        // sum_k A^[i,k] + K * (shift - a_zp), |.| <= 255 K < 2^23
                        // for K <= 32768, and |zb| <= 255: exact on the 24-bit
                        // multiplier; then the int32 C (a broadcast C from LDS,
                        // a full [M,N] C from memory; wrapping adds)
                        const dq::v4i zb = zbv[set], cc = ccv[set];
                        const int row = min(m0 + (wm * FM + p0 + u) * 32 + rs, M - 1);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            sum[e] = (int32_t)((uint32_t)sum[e] + (uint32_t)__mul24(rb[u][h], zb[e]) +
                                               (uint32_t)cr[u][h] + (uint32_t)cc[e]);
                            if (ep.c_mode == 3) {
                                const int col = min(col0 + cs_ + e, N - 1);
                                sum[e] = (int32_t)((uint32_t)sum[e] +
                                                   (uint32_t)ep.addC[(long long)row * ep.c_rs + (long long)col * ep.c_cs]);
                            }
                        }
                    }
                    int8_t* dst = region + u * SB + rs * RB + (((byte >> 4) ^ (rs & (CPR - 1))) << 4) + (byte & 15);
                    if (OUT == DQ_OUT_ACC) {
                        const dq::v4i v = {sum[0], sum[1], sum[2], sum[3]};
                        *reinterpret_cast<dq::v4i*>(dst) = v;
                    } else {
                        // a ReLU with bf16 output is applied after the
                        // rounding, on the packed pairs (dq::relu_bf16x4)
                        constexpr bool kReluPacked = OUT == DQ_OUT_BF16 && ACT == DQ_ACT_RELU;
                        dq::f4 val;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            float v = (float)sum[e] * sA[u][h];
                            v = v * sB[e];
                            if (BIAS) v = v + bv[e];
                            val[e] = kReluPacked ? v : activate<ACT>(v, ep.alpha);
                        }
                        if (Q8) {
                            uint32_t b[4];
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                float t;
                                if (yd.fast) {
                                    const float q0 = __builtin_amdgcn_fmed3f(val[e] * yd.y, -4194304.0f, 4194304.0f);
                                    const float r = __builtin_fmaf(-q0, yd.s, val[e]);
                                    t = __builtin_amdgcn_fmed3f(__builtin_fmaf(r, yd.y, q0) + kMagic,
                                                                kMagic + ylo, kMagic + yhi);
                                } else {
                                    t = kMagic + __builtin_fminf(__builtin_fmaxf(dq::rne(val[e] / yd.s), ylo), yhi);
                                }
                                b[e] = (uint32_t)__float_as_int(t);
                            }
                            const uint32_t packed = (b[0] & 0xffu) | ((b[1] & 0xffu) << 8) |
                                                    ((b[2] & 0xffu) << 16) | (b[3] << 24);
                            *reinterpret_cast<uint32_t*>(dst) =
                                ((packed & 0x7f7f7f7fu) + (yZ & 0x7f7f7f7fu)) ^ ((packed ^ yZ) & 0x80808080u);
                        } else if (OUT == DQ_OUT_BF16) {
                            const dq::u2 pk = dq::f32x4_to_bf16x4(val);
                            *reinterpret_cast<dq::u2*>(dst) = kReluPacked ? dq::relu_bf16x4(pk) : pk;
                        } else {
                            *reinterpret_cast<dq::f4*>(dst) = val;
                        }
                    }
                }
                // one column group at a time: keeps the accumulator reads of
                // later groups from being hoisted here (which would spill)
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // the pass back as row segments: chunk q -> row q / CPR of the pass;
        // LDS operations of one wave complete in order, so no barrier
        const int row0 = m0 + (wm * FM + p0) * 32;
#pragma unroll 8
        for (int q = lane; q < SPP * 32 * CPR; q += 64) {
            const int r = q / CPR, c = q % CPR;  // r: row of the pass
            const int row = row0 + r, col = col0 + c * EPC;
            const dq::v4i v = *reinterpret_cast<const dq::v4i*>(region + (r >> 5) * SB + (r & 31) * RB +
                                                                 ((c ^ (r & (CPR - 1))) << 4));
            if (row < M && col < N) {
                int8_t* C = reinterpret_cast<int8_t*>(ep.C) + ((size_t)row * N + col) * OB;
                if (vec_store && col + EPC <= N) {
                    // streaming store: C is written once and not read back
                    // here, and a launch's C (tens of MiB) is far larger than
                    // an XCD's L2; kept out of L2, it does not have to be
                    // written back when the kernel ends (measured: 4096 x
                    // 2048 x 512 fp32 C 13.7 -> 13.0 us, 4096^3 bf16 C
                    // 55.8 -> 54.9 us)
                    __builtin_nontemporal_store(v, reinterpret_cast<dq::v4i*>(C));
                } else {
#pragma unroll
                    for (int e = 0; e < EPC; ++e) {
                        if (col + e < N) {
                            const uint32_t w = (uint32_t)v[(e * OB) >> 2];
                            if (OB == 1)
                                reinterpret_cast<uint8_t*>(C)[e] = (uint8_t)(w >> (8 * (e & 3)));
                            else if (OB == 2)
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

template <int WM, int WN, int FM, int FN, int KS, int OUT, int ACT, bool BIAS, bool EXT = false>
void launch_one(dim3 grid, hipStream_t s, DqTiming t, const int8_t* Ap, const int8_t* Bp, int M,
                int N, int KF, int tiles_m, int tiles_n, int vec_store, const DqEpilogue& ep) {
    hipExtLaunchKernelGGL((k_gemm<WM, WN, FM, FN, KS, OUT, ACT, BIAS, EXT>), grid, dim3(WM * WN * 64), 0,
                          s, t.start, t.stop, 0, Ap, Bp, M, N, KF, tiles_m, tiles_n, vec_store, ep);
}

template <int WM, int WN, int FM, int FN, int KS, int OUT>
void launch_act(dim3 grid, hipStream_t s, DqTiming t, const int8_t* Ap, const int8_t* Bp, int M, int N, int KF,
                int tiles_m, int tiles_n, int vec_store, const DqEpilogue& ep) {
#define DQ_G(ACT, BIAS) launch_one<WM, WN, FM, FN, KS, OUT, ACT, BIAS>(grid, s, t, Ap, Bp, M, N, KF, tiles_m, tiles_n, vec_store, ep)
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
           hipStream_t s, DqTiming t) {
    static_assert(KS == 2 && kKpAlign % 256 == 0,
                  "the main loop needs a step count that is a multiple of 4: 64 per step, Kp % 256 == 0");
    constexpr int BM = WM * FM * 32, BN = WN * FN * 32;
    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const size_t tiles = (size_t)tiles_m * tiles_n;
    if (tiles > 0x7fffffffu) DQ_FAIL(DQ_ERR_ARG, "problem too large for one launch");
    // whole 16-byte chunks of C rows: 8 bf16 or 4 fp32 / int32 per chunk
    const int ob = (ep.out == DQ_OUT_U8 || ep.out == DQ_OUT_I8) ? 1 : ep.out == DQ_OUT_BF16 ? 2 : 4;
    const int vec_store = (uintptr_t)ep.C % 16 == 0 && ((size_t)N * ob) % 16 == 0;
    const dim3 grid((unsigned)tiles);
    const int KF = Kp / 32;
    // the quantized matrix products: B zero points, int32 C and 8-bit output
    // (identity activation); the inner product takes the plain epilogue
    if (ep.rowsumA || ep.zeroB || ep.addC || ep.out == DQ_OUT_U8 || ep.out == DQ_OUT_I8) {
        const bool bias = ep.bias != nullptr;
        switch (ep.out) {
            case DQ_OUT_U8:
                launch_one<WM, WN, FM, FN, KS, DQ_OUT_U8, DQ_ACT_IDENTITY, false, true>(grid, s, t, Ap, Bp, M, N, KF, tiles_m, tiles_n, vec_store, ep);
                break;
            case DQ_OUT_I8:
                launch_one<WM, WN, FM, FN, KS, DQ_OUT_I8, DQ_ACT_IDENTITY, false, true>(grid, s, t, Ap, Bp, M, N, KF, tiles_m, tiles_n, vec_store, ep);
                break;
            case DQ_OUT_ACC:
                launch_one<WM, WN, FM, FN, KS, DQ_OUT_ACC, DQ_ACT_IDENTITY, false, true>(grid, s, t, Ap, Bp, M, N, KF, tiles_m, tiles_n, vec_store, ep);
                break;
            default:
                if (bias)
                    launch_one<WM, WN, FM, FN, KS, DQ_OUT_F32, DQ_ACT_IDENTITY, true, true>(grid, s, t, Ap, Bp, M, N, KF, tiles_m, tiles_n, vec_store, ep);
                else
                    launch_one<WM, WN, FM, FN, KS, DQ_OUT_F32, DQ_ACT_IDENTITY, false, true>(grid, s, t, Ap, Bp, M, N, KF, tiles_m, tiles_n, vec_store, ep);
                break;
        }
        DQ_LAUNCH_CHECK("gemm_i8");
        return DQ_OK;
    }
    switch (ep.out) {
        case DQ_OUT_ACC:
            launch_one<WM, WN, FM, FN, KS, DQ_OUT_ACC, DQ_ACT_IDENTITY, false>(grid, s, t, Ap, Bp, M, N, KF, tiles_m, tiles_n, vec_store, ep);
            break;
        case DQ_OUT_BF16:
            launch_act<WM, WN, FM, FN, KS, DQ_OUT_BF16>(grid, s, t, Ap, Bp, M, N, KF, tiles_m, tiles_n, vec_store, ep);
            break;
        default:
            launch_act<WM, WN, FM, FN, KS, DQ_OUT_F32>(grid, s, t, Ap, Bp, M, N, KF, tiles_m, tiles_n, vec_store, ep);
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

int dq_gemm_config(int M, int N) { return pick(M, N); }

int dq_launch_gemm(const int8_t* Ap, const int8_t* Bp, int M, int N, int Kp, const DqEpilogue& ep,
                   hipStream_t s, DqTiming t) {
    switch (pick(M, N)) {
        case 2: return launch<2, 2, 4, 4, 2>(Ap, Bp, M, N, Kp, ep, s, t);
        case 1: return launch<2, 2, 2, 2, 2>(Ap, Bp, M, N, Kp, ep, s, t);
        default: return launch<1, 1, 1, 1, 2>(Ap, Bp, M, N, Kp, ep, s, t);
    }
}

const char* dq_gemm_info(int M, int N, int) {
    switch (pick(M, N)) {
        case 2: return "gemm_i8 v_mfma_i32_16x16x64_i8 tile 256x256, k-step 64 (4 waves x 128x128, accumulators in AGPRs), 4-stage global->LDS DMA ring, fused dequant epilogue";
        case 1: return "gemm_i8 v_mfma_i32_16x16x64_i8 tile 128x128, k-step 64 (4 waves x 64x64), 4-stage global->LDS DMA ring, fused dequant epilogue";
        default: return "gemm_i8 v_mfma_i32_16x16x64_i8 tile 32x32, k-step 64 (1 wave), 4-stage global->LDS DMA ring, fused dequant epilogue";
    }
}
