// qlstm.hip -- DynamicQuantizeLSTM on gfx950.
//
// onnxruntime quantization_defs.cc, schema DynamicQuantizeLSTM (restated on
// the graiphic.io DynamicQuantizeLSTM page), gives the tensors and the
// attributes; the cell is the ONNX LSTM's. This file computes (the readings
// are stated where the entry points are declared, include/dqip.h):
//   xw  = X W + Wb, X [seq * batch, input] quantized per tensor to uint8 once
//   per step s and direction d, for each batch entry b with s < L_b
//   (t = s, or L_b - 1 - s when d runs in reverse):
//     hr  = H_{s-1} R + Rb, H_{s-1} [batch, h] quantized per tensor to uint8
//     pre = xw[t] + hr; peepholes, clip, activations (fp64, rounded once),
//     C_s, H_s; Y[t] = H_s
//   and for the other entries H, C held and Y[s] = 0.
//
// Layout and kernels:
//  - The input projection of all times and both directions is one
//    DynamicQuantizeMatMul on the QGemm path (qgemm.hip) with W's columns
//    regrouped as [direction][unit][gate i, o, f, c] (k_lstm_pack_w), so the
//    four gate inputs of one cell are one 16-byte load of xw.
//  - R is packed once (k_lstm_pack_r) into v_mfma_i32_32x32x32_i8 fragments
//    of 32 gate columns (8 units x 4 gates, unit-major) by 32 k; a uint8 R
//    enters as code - 128. k_lstm_params writes the per-column vectors.
//  - Each step is one launch of k_lstm_step. Workgroup (nt, bt, d) owns
//    units 8 nt .. 8 nt + 7 of direction d for batch entries 32 bt ..
//    32 bt + 31. Its eight waves split K: wave w multiplies k fragments
//    8 j + w, R as the first MFMA operand (so a lane's 16 accumulators are
//    4 units x 4 gates of one batch entry) and H_{s-1}'s codes as the
//    second. Lane l's share of that operand is 16 values of one row of
//    H_{s-1}, which the lane loads and quantizes itself, with the
//    per-tensor scale from the extremes the previous step left in 64 slots
//    (atomics on order-preserving integers): the codes never touch LDS.
//    The eight partial tiles are summed through LDS, leaving each thread of
//    waves 0..3 the four gates of one cell; the cell update writes C in place, H_s into the
//    other state buffer (stored in the order the next step's lanes load it,
//    see hpos), Y, and H_s's extremes for the next step, and the
//    slot two steps ahead is cleared for the step after. Every load of a
//    step is issued at its start, at clamped addresses, so the kernel waits
//    on memory once (then once more for its xw, issued when the cell's time
//    is known and in flight during the product).
//  - The integer sum is exact with A^ = q - 128, R^ = r - rho (rho = 128 for
//    a uint8 R, else 0), alpha = 128 - zp_H, beta[n] = rho - rz[n]:
//      sum = sum_k A^ R^ + beta * rowsum(A^) + alpha * colsum(R^)[n]
//            + h * alpha * beta      (wrapping int32, exact for h <= 4096)
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>

#include "dq_device.h"

namespace {

#ifndef DQ_LSTM_WAVES
#define DQ_LSTM_WAVES 8
#endif
constexpr int kWaves = DQ_LSTM_WAVES;  // waves of a step workgroup: they split K, waves 0..3 update the cells
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxCN = kWaves >= 8 ? 2 : 4;  // fragments a wave holds at once (two waves a SIMD: 256 registers)
constexpr int kSlots = 64;      // extremes slots per step (workgroup b adds to slot b % 64)
constexpr uint32_t kPlusZero = 0x80000000u;  // dq::f2ord(+0.0f)

struct StepArgs {
    const float* xw;      // [seq * batch][N], column d * 4h + 4u + g
    const int8_t* rp;     // [dirs][NT][KFP][1024] packed R^
    const int32_t* rcs;   // [dirs][NT * 32] column sums of R^
    const int32_t* rbeta; // [dirs][NT * 32] rho - rz
    const float* rsc;     // [dirs][NT * 32] R scale
    const float* rbias;   // [dirs][NT * 32] Rb
    const float* pp;      // [dirs][NT * 8][4] peepholes i, o, f, 0
    const int32_t* lens;  // [batch] or NULL
    const float* hin;     // H_{s-1} in the state layout (hpos)
    float* hout;          // H_s in the state layout
    float* c;             // [dirs][batch][h], updated in place
    float* y;             // [seq][dirs][batch][h] or NULL
    float* yh;            // [dirs][batch][h], written by the last step (or NULL)
    float* yc;
    uint32_t* mm;         // [dirs][3][2][kSlots]
    int s, seq, batch, h, N, NT, KFP, BT, dirs;
    int rd_slot, wr_slot, clr_slot;
    int rev_mask;         // bit d set: direction d runs in reverse
    int act[6];           // f, g, h of direction 0, then of direction 1
    float alpha[6], beta[6];
    float clip;           // <= 0: no clip
    int input_forget;
};

// tanh in fp64 for a result that is rounded to fp32: for |x| >= 1/8,
// 1 - 2 / (e^{2|x|} + 1) (the subtraction loses at most 3 of fp64's 53
// bits); below, the Taylor series x + x^3 sum_k c_k x^{2k} through x^15
// (c_k = 2^{2n} (2^{2n} - 1) B_{2n} / (2n)!: -1/3, 2/15, -17/315, 62/2835,
// -1382/155925, 21844/6081075, -929569/638512875; the first omitted term is
// below 2^-55 of the result for |x| < 1/8). Both are far inside the half
// fp32 ulp that decides the rounding; the library's tanh carries extra-
// precision arithmetic (about 150 fp64 instructions) that this does not need.
__device__ __forceinline__ double tanh_d(double x) {
    const double ax = fabs(x);
    const double big = 1.0 - 2.0 / (exp(2.0 * ax) + 1.0);
    const double x2 = ax * ax;
    double p = -0.0014558343870513183;
    p = fma(p, x2, 0.003592128036572481);
    p = fma(p, x2, -0.008863235529902197);
    p = fma(p, x2, 0.021869488536155203);
    p = fma(p, x2, -0.05396825396825397);
    p = fma(p, x2, 0.13333333333333333);
    p = fma(p, x2, -0.3333333333333333);
    const double small = fma(ax * x2, p, ax);
    return copysign(ax < 0.125 ? small : big, x);
}

// One ONNX RNN activation, evaluated in fp64 from the fp32 argument and
// rounded to fp32 once.
__device__ float rnn_act(int kind, float xf, float af, float bf) {
    const double x = (double)xf, a = (double)af, b = (double)bf;
    double r;
    switch (kind) {
        case DQ_RNN_SIGMOID: r = 1.0 / (1.0 + exp(-x)); break;
        case DQ_RNN_TANH: r = tanh_d(x); break;
        case DQ_RNN_RELU: r = x > 0.0 ? x : 0.0; break;
        case DQ_RNN_AFFINE: r = a * x + b; break;
        case DQ_RNN_LEAKY_RELU: r = x < 0.0 ? a * x : x; break;
        case DQ_RNN_THRESHOLDED_RELU: r = x > a ? x : 0.0; break;
        case DQ_RNN_SCALED_TANH: r = a * tanh_d(b * x); break;
        case DQ_RNN_HARD_SIGMOID: r = fmin(fmax(a * x + b, 0.0), 1.0); break;
        case DQ_RNN_ELU: r = x >= 0.0 ? x : a * expm1(x); break;
        case DQ_RNN_SOFTSIGN: r = x / (1.0 + fabs(x)); break;
        default:  // softplus = log(1 + e^x), split so that e^x cannot overflow
            r = x == 0.0 ? 0.69314718055994530942 : x < 0.0 ? log1p(exp(x)) : x + log1p(exp(-x));
    }
    return (float)r;
}

// Index of H[d][b][u] in the state buffers: per direction and 32-entry batch
// tile, [fragment kf][quarter j][lane][4] with kf = u / 32, j = (u % 16) / 4
// and lane = b % 32 + 32 ((u % 32) / 16). Lane l's 16 values of fragment kf
// (its share of the MFMA operand) are four 16-byte pieces 1 KiB apart, so a
// wave's load instruction reads 1 KiB of consecutive bytes.
__host__ __device__ __forceinline__ size_t hpos(int d, int b, int u, int BT, int KFP) {
    const int lane = (b & 31) + ((u >> 4) & 1) * 32;
    return ((((size_t)d * BT + (b >> 5)) * KFP + (u >> 5)) * 4 + ((u >> 2) & 3)) * 256 + lane * 4 + (u & 3);
}

__device__ __forceinline__ float clipv(float v, float c) {
    return c > 0.0f ? __builtin_fminf(__builtin_fmaxf(v, -c), c) : v;
}

// The default activations (f = Sigmoid, g = h = Tanh) as inline code, so
// that the independent gates of a cell overlap; the same evaluation as
// rnn_act's.
__device__ __forceinline__ float sigmoid_r(float x) { return (float)(1.0 / (1.0 + exp(-(double)x))); }
__device__ __forceinline__ float tanh_r(float x) { return (float)tanh_d((double)x); }

constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23: adding it rounds to an integer, half to even

// H codes of one MFMA operand: 16 values of one row to 16 codes q - 128 in
// four words (byte e of word m is value 4 m + e), with
//   q = saturate(rne(x / scale) + zp) = rne(clamp(x / scale, -zp, 255 - zp)) + zp.
// The quotient is the IEEE one: the residual step of dq::qdiv when FAST
// (|x / scale| <= 255 here, since lo <= x <= hi and hi - lo = 255 scale), else
// the division. The magic add rounds half to even into the low mantissa bits,
// the median clamps, and zp - 128 is added to four bytes at once (each true
// sum lies in [-128, 127], so the carry-free bytewise add is exact).
struct HQuant {
    float s, y, lof, hif;
    uint32_t z4;  // (zp - 128) in each byte
};

template <bool FAST>
__device__ __forceinline__ dq::v4i quant16(const float (&x)[16], const HQuant& q, uint32_t valid16) {
    dq::v4i out;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        uint32_t b[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float v = x[4 * m + e];
            float t;
            if (FAST) {
                const float q0 = v * q.y;
                t = __builtin_fmaf(__builtin_fmaf(-q0, q.s, v), q.y, q0);
            } else {
                t = v / q.s;
            }
            b[e] = (uint32_t)__float_as_int(__builtin_amdgcn_fmed3f(t + kMagic, q.lof, q.hif));
        }
        const uint32_t p = (b[0] & 0xffu) | ((b[1] & 0xffu) << 8) | ((b[2] & 0xffu) << 16) | (b[3] << 24);
        const uint32_t c = ((p & 0x7f7f7f7fu) + (q.z4 & 0x7f7f7f7fu)) ^ ((p ^ q.z4) & 0x80808080u);
        // invalid values (k >= h, rows >= batch) give code 0
        const uint32_t nv = (valid16 >> (4 * m)) & 0xfu;
        const uint32_t mask = (nv & 1u ? 0xffu : 0u) | (nv & 2u ? 0xff00u : 0u) | (nv & 4u ? 0xff0000u : 0u) |
                              (nv & 8u ? 0xff000000u : 0u);
        out[m] = (int)(c & mask);
    }
    return out;
}

template <int CN, bool DEF>
__global__ void __launch_bounds__(kThreads) k_lstm_step(StepArgs a) {
    __shared__ int32_t red[kWaves][16][64];
    __shared__ int32_t rsw[kWaves][32];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int nt = blockIdx.x, bt = blockIdx.y, d = blockIdx.z;
    const int h = a.h, batch = a.batch, KFW = a.KFP / kWaves, nchunks = KFW / CN;
    const float* htile = a.hin + ((size_t)d * a.BT + bt) * a.KFP * 1024 + lane * 4;

    // Wave w multiplies k fragments kWaves j + w (j < KFW), CN at a time. Lane l
    // holds, as the second MFMA operand, 16 codes of row l % 32 of the tile
    // at k = 32 kf + 16 (l / 32): it quantizes exactly those 16 values of
    // H_{s-1}, so the codes never leave its registers.
    const dq::v4i* rbase =
        reinterpret_cast<const dq::v4i*>(a.rp + (size_t)(d * a.NT + nt) * a.KFP * 1024) + lane;
    const bool row_ok = bt * 32 + (lane & 31) < batch;
    const int hr_k = (lane >> 5) * 16;
    auto load_chunk = [&](int c, dq::v4i (&rr)[CN], float (&hx)[CN][16], uint32_t (&vm)[CN]) {
#pragma unroll
        for (int i = 0; i < CN; ++i) {
            const int kf = kWaves * (c * CN + i) + w;
            rr[i] = rbase[(size_t)kf * 64];
            const int k0 = kf * 32 + hr_k;
            const int n = row_ok ? (h - k0 < 0 ? 0 : h - k0 > 16 ? 16 : h - k0) : 0;  // values inside H
            vm[i] = n == 16 ? 0xffffu : (1u << n) - 1u;
            const float* src = htile + (size_t)kf * 1024;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const dq::f4 v = *reinterpret_cast<const dq::f4*>(src + j * 256);
                hx[i][4 * j] = v[0]; hx[i][4 * j + 1] = v[1]; hx[i][4 * j + 2] = v[2]; hx[i][4 * j + 3] = v[3];
            }
        }
    };

    // Every load of the step is issued here, at addresses clamped into the
    // tensors where an index runs past them, so none waits for another: the
    // first chunk of R fragments and H values, the extremes of H_{s-1}, and
    // the inputs of the thread's cell (unit u, batch entry b; accumulator
    // rows 8 w + 4 half + e are gate e of unit 2 w + half of the tile).
    dq::v4i rf[CN];
    float hx[CN][16];
    uint32_t vm[CN];
    load_chunk(0, rf, hx, vm);
    const uint32_t* mmr = a.mm + ((size_t)d * 3 + a.rd_slot) * 2 * kSlots;
    const uint32_t mlo = mmr[lane], mhi = mmr[kSlots + lane];
    // (waves 4 and up take the mapping of wave w % 4 for their clamped
    // loads but own no cell)
    const int half = lane >> 5, bl = lane & 31, wc = w & 3;
    const int b = bt * 32 + bl, ul = 2 * wc + half, u = nt * 8 + ul;
    const bool cell = w < 4 && b < batch && u < h;
    const int bc = b < batch ? b : batch - 1, uc = u < h ? u : h - 1;
    const size_t su = ((size_t)d * batch + bc) * h + uc;
    const int lraw = a.lens ? a.lens[bc] : a.seq;
    const size_t sh = hpos(d, bc, uc, a.BT, a.KFP);
    const float c0 = a.c[su], hold = a.hin[sh];
    const size_t pc = (size_t)d * a.NT * 32 + nt * 32 + 4 * ul;
    const dq::v4i cs4 = *reinterpret_cast<const dq::v4i*>(a.rcs + pc);
    const dq::v4i be4 = *reinterpret_cast<const dq::v4i*>(a.rbeta + pc);
    const dq::f4 rs4 = *reinterpret_cast<const dq::f4*>(a.rsc + pc);
    const dq::f4 rb4 = *reinterpret_cast<const dq::f4*>(a.rbias + pc);
    const dq::f4 p4 = *reinterpret_cast<const dq::f4*>(a.pp + ((size_t)d * a.NT * 8 + u) * 4);
    dq::issue_fence();

    // per-tensor quantization of H_{s-1}: lo = min(0, min H), hi = max(0, max H)
    const float lo = dq::wave_min_uniform(dq::ord2f(mlo));
    const float hi = dq::wave_max_uniform(dq::ord2f(mhi));
    float sc = 1.0f;
    int zp = 0;
    if (hi != lo) {
        sc = (hi - lo) / 255.0f;
        zp = dq::sat_add(dq::rne(-lo / sc), 0, 0, 255);
    }
    // the cell's time and its input projection, in flight during the product
    const int L = lraw < 0 ? 0 : lraw > a.seq ? a.seq : lraw;
    const bool live = cell && a.s < L;
    const int t = live ? (((a.rev_mask >> d) & 1) ? L - 1 - a.s : a.s) : 0;
    const dq::f4 x4 =
        *reinterpret_cast<const dq::f4*>(a.xw + ((size_t)t * batch + bc) * a.N + (size_t)d * 4 * h + 4 * uc);
    if (nt == 0 && bt == 0 && tid < 2 * kSlots)
        a.mm[((size_t)d * 3 + a.clr_slot) * 2 * kSlots + tid] = kPlusZero;

    // sum_k A^ R^ over this wave's fragments, the next chunk's loads in
    // flight while one is quantized and multiplied; rs sums the codes
    const dq::QDiv qd = dq::make_qdiv(sc);
    HQuant hq;
    hq.s = sc;
    hq.y = qd.y;
    hq.lof = kMagic + (float)(0 - zp);
    hq.hif = kMagic + (float)(255 - zp);
    hq.z4 = (uint32_t)((zp - 128) & 0xff) * 0x01010101u;
    dq::v16i acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0;
    int rs = 0;
    for (int c = 0; c < nchunks; ++c) {
        const bool more = c + 1 < nchunks;
        dq::v4i rn[CN];
        float hn[CN][16];
        uint32_t vn[CN];
        if (more) load_chunk(c + 1, rn, hn, vn);
#pragma unroll
        for (int i = 0; i < CN; ++i) {
            const dq::v4i hf = qd.fast ? quant16<true>(hx[i], hq, vm[i]) : quant16<false>(hx[i], hq, vm[i]);
            acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(rf[i], hf, acc, 0, 0, 0);
#pragma unroll
            for (int m = 0; m < 4; ++m) rs = __builtin_amdgcn_sdot4(hf[m], 0x01010101, rs, false);
        }
        if (more) {
#pragma unroll
            for (int i = 0; i < CN; ++i) {
                rf[i] = rn[i];
                vm[i] = vn[i];
#pragma unroll
                for (int j = 0; j < 16; ++j) hx[i][j] = hn[i][j];
            }
        }
    }
    // the last MFMA's results need the ISA's wait states before they are read
    dq::mfma_result_drain();
#pragma unroll
    for (int e = 0; e < 16; ++e) red[w][e][lane] = acc[e];
    rs += __shfl_xor(rs, 32);  // lanes l and l + 32 hold the two k halves of row l % 32
    if (lane < 32) rsw[w][lane] = rs;
    __syncthreads();

    float lo_n = 0.0f, hi_n = 0.0f;
    if (cell) {
        float hv, cv = c0;
        if (live) {
            const uint32_t al = (uint32_t)(128 - zp);
            uint32_t rsum = 0;
#pragma unroll
            for (int v = 0; v < kWaves; ++v) rsum += (uint32_t)rsw[v][bl];
            float pre[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 4 * wc + e;
                uint32_t sum = 0;
#pragma unroll
                for (int v = 0; v < kWaves; ++v) sum += (uint32_t)red[v][row][lane];
                const uint32_t be = (uint32_t)be4[e];
                sum += be * rsum + al * (uint32_t)cs4[e] + (uint32_t)h * al * be;
                const float hr = ((float)(int32_t)sum * sc) * rs4[e] + rb4[e];
                pre[e] = x4[e] + hr;
            }
            const int f0 = 3 * d;
            const float pi = clipv(pre[0] + p4[0] * c0, a.clip);
            const float pf = clipv(pre[2] + p4[2] * c0, a.clip);
            const float pg = clipv(pre[3], a.clip);
            float ig, fg, gg;
            if (DEF) {
                ig = sigmoid_r(pi);
                fg = a.input_forget ? 1.0f - ig : sigmoid_r(pf);
                gg = tanh_r(pg);
            } else {
                ig = rnn_act(a.act[f0], pi, a.alpha[f0], a.beta[f0]);
                fg = a.input_forget ? 1.0f - ig : rnn_act(a.act[f0], pf, a.alpha[f0], a.beta[f0]);
                gg = rnn_act(a.act[f0 + 1], pg, a.alpha[f0 + 1], a.beta[f0 + 1]);
            }
            cv = fg * c0 + ig * gg;
            const float po = clipv(pre[1] + p4[1] * cv, a.clip);
            if (DEF) {
                hv = sigmoid_r(po) * tanh_r(cv);
            } else {
                const float og = rnn_act(a.act[f0], po, a.alpha[f0], a.beta[f0]);
                hv = og * rnn_act(a.act[f0 + 2], cv, a.alpha[f0 + 2], a.beta[f0 + 2]);
            }
            a.c[su] = cv;
            if (a.y) a.y[(((size_t)t * a.dirs + d) * batch + b) * h + u] = hv;
        } else {
            hv = hold;
            if (a.y) a.y[(((size_t)a.s * a.dirs + d) * batch + b) * h + u] = 0.0f;
        }
        a.hout[sh] = hv;
        if (a.yh) a.yh[su] = hv;
        if (a.yc) a.yc[su] = cv;
        lo_n = __builtin_fminf(lo_n, hv);
        hi_n = __builtin_fmaxf(hi_n, hv);
    }
    if (w >= 4) return;
    lo_n = dq::wave_min_uniform(lo_n);
    hi_n = dq::wave_max_uniform(hi_n);
    if (lane == 0) {
        uint32_t* mmw = a.mm + ((size_t)d * 3 + a.wr_slot) * 2 * kSlots;
        const int slot = (blockIdx.x + blockIdx.y * gridDim.x) % kSlots;
        atomicMin(&mmw[slot], dq::f2ord(lo_n));
        atomicMax(&mmw[kSlots + slot], dq::f2ord(hi_n));
    }
}

// Every extremes slot of every direction to the encoding of +0.
__global__ void k_lstm_mm_reset(uint32_t* mm, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) mm[i] = kPlusZero;
}

// The initial state (zeros where not given) into the state buffers, its
// extremes into slot 0 of its direction; yh / yc (a sequence of length 0)
// receive it as the final state.
__global__ void __launch_bounds__(256) k_lstm_begin(const float* h0, const float* c0, int batch, int h, int BT,
                                                    int KFP, float* hs, float* cs, uint32_t* mm, float* yh,
                                                    float* yc) {
    const int d = blockIdx.y;
    const int per_dir = batch * h;
    const int i = blockIdx.x * 256 + threadIdx.x;
    float hv = 0.0f;
    if (i < per_dir) {
        const size_t k = (size_t)d * per_dir + i;
        hv = h0 ? h0[k] : 0.0f;
        const float cv = c0 ? c0[k] : 0.0f;
        hs[hpos(d, i / h, i % h, BT, KFP)] = hv;
        cs[k] = cv;
        if (yh) yh[k] = hv;
        if (yc) yc[k] = cv;
    }
    const float lo = dq::wave_min_uniform(__builtin_fminf(hv, 0.0f));
    const float hi = dq::wave_max_uniform(__builtin_fmaxf(hv, 0.0f));
    if ((threadIdx.x & 63) == 0) {
        uint32_t* m = mm + (size_t)d * 3 * 2 * kSlots;
        const int slot = (blockIdx.x * 4 + (threadIdx.x >> 6)) % kSlots;
        atomicMin(&m[slot], dq::f2ord(lo));
        atomicMax(&m[kSlots + slot], dq::f2ord(hi));
    }
}

// W [dirs][input][4h] -> Wcat [input][dirs * 4h], column d * 4h + 4u + g
// taking W's column g * h + u.
__global__ void k_lstm_pack_w(const uint8_t* W, int input, int h, int dirs, uint8_t* wcat) {
    const size_t n = (size_t)input * dirs * 4 * h;
    const size_t N = (size_t)dirs * 4 * h;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
        const size_t k = i / N, col = i - k * N;
        const int d = (int)(col / (4 * h)), p = (int)(col - (size_t)d * 4 * h);
        const int u = p >> 2, g = p & 3;
        wcat[i] = W[((size_t)d * input + k) * 4 * h + (size_t)g * h + u];
    }
}

// R [dirs][h][4h] -> fragments [dirs][NT][KFP][1024] of R^ = r - rho: one
// 16-byte lane slot per thread (gate column r, 16 k from 16 * khalf).
__global__ void k_lstm_pack_r(const uint8_t* R, int h, int NT, int KFP, int dirs, int rho, int8_t* rp) {
    const size_t nslots = (size_t)dirs * NT * KFP * 64;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nslots; i += (size_t)gridDim.x * blockDim.x) {
        const int slot = (int)(i & 63);
        const size_t frag = i >> 6;
        const int kf = (int)(frag % KFP);
        const size_t tile = frag / KFP;
        const int nt = (int)(tile % NT), d = (int)(tile / NT);
        const int r = slot & 31, kh = slot >> 5;
        const int u = nt * 8 + (r >> 2), g = r & 3;
        uint32_t pk[4] = {0u, 0u, 0u, 0u};
        if (u < h) {
            const uint8_t* col = R + (size_t)d * h * 4 * h + (size_t)g * h + u;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int k = kf * 32 + kh * 16 + j;
                const int v = k < h ? (int)col[(size_t)k * 4 * h] - rho : 0;
                pk[j >> 2] |= (uint32_t)(v & 0xff) << (8 * (j & 3));
            }
        }
        *reinterpret_cast<dq::u4*>(rp + i * 16) = dq::u4{pk[0], pk[1], pk[2], pk[3]};
    }
}

__device__ __forceinline__ int zp_at(const void* zp, bool u8, int64_t idx) {
    if (!zp) return 0;
    return u8 ? (int)reinterpret_cast<const uint8_t*>(zp)[idx] : (int)reinterpret_cast<const int8_t*>(zp)[idx];
}

struct ParamArgs {
    const uint8_t* R;
    const float *w_scale, *r_scale, *B, *P;
    const void *w_zp, *r_zp;
    int w_len, r_len;     // dirs or dirs * 4h
    int w_u8, r_u8, rho;
    int h, NT, dirs;
    // projection vectors [dirs * 4h]
    float* wsc;
    uint8_t* wzp;
    float* wb;
    // step vectors [dirs][NT * 32] and peepholes [dirs][NT * 8][4]
    int32_t* rcs;
    int32_t* rbeta;
    float* rsc;
    float* rbias;
    float* pp;
};

// One thread per packed gate column p of direction d (unit p / 4, gate p % 4).
__global__ void k_lstm_params(ParamArgs a) {
    const int d = blockIdx.y;
    const int p = blockIdx.x * blockDim.x + threadIdx.x;
    const int h = a.h;
    if (p >= a.NT * 32) return;
    const int u = p >> 2, g = p & 3;
    const size_t q = (size_t)d * a.NT * 32 + p;
    int32_t cs = 0, be = 0;
    float rs = 0.0f, rb = 0.0f;
    if (u < h) {
        const int64_t col = (int64_t)g * h + u;  // column of W / R / B in the gate-blocked order
        const int64_t wi = a.w_len == a.dirs ? d : (int64_t)d * 4 * h + col;
        const int64_t ri = a.r_len == a.dirs ? d : (int64_t)d * 4 * h + col;
        const size_t o = (size_t)d * 4 * h + p;
        a.wsc[o] = a.w_scale[wi];
        a.wzp[o] = (uint8_t)zp_at(a.w_zp, a.w_u8, wi);
        a.wb[o] = a.B ? a.B[(size_t)d * 8 * h + col] : 0.0f;
        // column sum of R^ = r - rho over the h rows
        const size_t c0 = (size_t)d * h * 4 * h + col;
        if (a.r_u8)
            for (int k = 0; k < h; ++k) cs += (int)a.R[c0 + (size_t)k * 4 * h] - 128;
        else
            for (int k = 0; k < h; ++k) cs += (int)(int8_t)a.R[c0 + (size_t)k * 4 * h];
        be = a.rho - zp_at(a.r_zp, a.r_u8, ri);
        rs = a.r_scale[ri];
        rb = a.B ? a.B[(size_t)d * 8 * h + 4 * h + col] : 0.0f;
    }
    a.rcs[q] = cs;
    a.rbeta[q] = be;
    a.rsc[q] = rs;
    a.rbias[q] = rb;
    if (g == 0) {
        float* pq = a.pp + ((size_t)d * a.NT * 8 + u) * 4;
        const bool on = a.P && u < h;
        pq[0] = on ? a.P[(size_t)d * 3 * h + u] : 0.0f;
        pq[1] = on ? a.P[(size_t)d * 3 * h + h + u] : 0.0f;
        pq[2] = on ? a.P[(size_t)d * 3 * h + 2 * h + u] : 0.0f;
        pq[3] = 0.0f;
    }
}

bool valid_act(int k) { return k >= DQ_RNN_SIGMOID && k <= DQ_RNN_SOFTPLUS; }

// ONNX defaults of the activations that take alpha / beta
float default_alpha(int k) {
    switch (k) {
        case DQ_RNN_LEAKY_RELU: return 0.01f;
        case DQ_RNN_HARD_SIGMOID: return 0.2f;
        case DQ_RNN_AFFINE:
        case DQ_RNN_THRESHOLDED_RELU:
        case DQ_RNN_SCALED_TANH:
        case DQ_RNN_ELU: return 1.0f;
        default: return 0.0f;
    }
}
float default_beta(int k) {
    switch (k) {
        case DQ_RNN_HARD_SIGMOID: return 0.5f;
        case DQ_RNN_SCALED_TANH: return 1.0f;
        default: return 0.0f;
    }
}

}  // namespace

struct dq_lstm_ctx {
    int64_t seq = 0, batch = 0, input = 0, h = 0;
    int dirs = 1, direction = 0;
    dq_dtype w_type = DQ_I8, r_type = DQ_I8;
    int NT = 0, KFP = 0, CN = 1;
    bool has_w = false;
    int BT = 0;
    bool def_act = true;  // Sigmoid, Tanh, Tanh in every direction
    int act[6] = {0, 1, 1, 0, 1, 1};
    float alpha[6] = {}, beta[6] = {};
    float clip = 0.0f;
    int input_forget = 0;
    int device = 0;
    dq_qgemm_ctx* qg = nullptr;
    float* xw = nullptr;       // [seq * batch][dirs * 4h]
    float* wsc = nullptr;      // [dirs * 4h]
    uint8_t* wzp = nullptr;
    float* wb = nullptr;
    int8_t* rp = nullptr;
    int32_t* rcs = nullptr;
    int32_t* rbeta = nullptr;
    float* rsc = nullptr;
    float* rbias = nullptr;
    float* pp = nullptr;
    float* hs = nullptr;       // two state buffers of dirs * BT * KFP * 1024 (hpos)
    float* cs = nullptr;       // [dirs][batch][h]
    uint32_t* mm = nullptr;    // [dirs][3][2][kSlots]
    std::string info;
};

namespace {

void free_ctx(dq_lstm_ctx* c) {
    if (!c) return;
    dq_qgemm_release(c->qg);
    void* bufs[] = {c->xw, c->wsc, c->wzp, c->wb, c->rp, c->rcs, c->rbeta, c->rsc, c->rbias, c->pp, c->hs, c->cs, c->mm};
    for (void* p : bufs) (void)hipFree(p);
    delete c;
}

int check_device(const dq_lstm_ctx* c) {
    int dev = 0;
    (void)hipGetDevice(&dev);
    if (dev != c->device) DQ_FAIL(DQ_ERR_STATE, "the context belongs to another device");
    return DQ_OK;
}

}  // namespace

extern "C" int dq_lstm_init(dq_lstm_ctx** ctx, int64_t seq_length, int64_t batch_size, int64_t input_size,
                            int64_t hidden_size, int direction, dq_dtype w_type, dq_dtype r_type,
                            const int* activations, const float* activation_alpha, const float* activation_beta,
                            float clip, int input_forget) {
    if (!ctx) DQ_FAIL(DQ_ERR_ARG, "ctx is NULL");
    *ctx = nullptr;
    if (seq_length < 0 || batch_size < 0 || input_size < 1 || hidden_size < 1)
        DQ_FAIL(DQ_ERR_ARG, "sizes must be seq, batch >= 0 and input, hidden >= 1");
    if (direction < DQ_LSTM_FORWARD || direction > DQ_LSTM_BIDIRECTIONAL)
        DQ_FAIL(DQ_ERR_ARG, "direction must be DQ_LSTM_FORWARD, _REVERSE or _BIDIRECTIONAL");
    if ((w_type != DQ_I8 && w_type != DQ_U8) || (r_type != DQ_I8 && r_type != DQ_U8))
        DQ_FAIL(DQ_ERR_TYPE, "W and R must be DQ_I8 or DQ_U8");
    if (hidden_size > DQ_LSTM_HIDDEN_MAX)
        DQ_FAIL(DQ_ERR_RANGE, "hidden_size exceeds %d", DQ_LSTM_HIDDEN_MAX);
    if (input_size > DQ_QGEMM_K_MAX) DQ_FAIL(DQ_ERR_RANGE, "input_size exceeds %d", DQ_QGEMM_K_MAX);
    const int dirs = direction == DQ_LSTM_BIDIRECTIONAL ? 2 : 1;
    if ((batch_size + 31) / 32 > 65535) DQ_FAIL(DQ_ERR_RANGE, "batch_size exceeds %d", 65535 * 32);
    const int64_t M = seq_length * batch_size;
    if (M > (int64_t)INT32_MAX - 256) DQ_FAIL(DQ_ERR_RANGE, "seq_length * batch_size too large");
    if (M * dirs * 4 * hidden_size > ((int64_t)1 << 36)) DQ_FAIL(DQ_ERR_RANGE, "input projection too large");
    if (activations)
        for (int i = 0; i < 3 * dirs; ++i)
            if (!valid_act(activations[i])) DQ_FAIL(DQ_ERR_ARG, "activation %d is not a dq_rnn_act", activations[i]);

    dq_lstm_ctx* c = new dq_lstm_ctx();
    c->seq = seq_length;
    c->batch = batch_size;
    c->input = input_size;
    c->h = hidden_size;
    c->dirs = dirs;
    c->direction = direction;
    c->w_type = w_type;
    c->r_type = r_type;
    for (int i = 0; i < 3 * dirs; ++i) {
        const int k = activations ? activations[i] : (i % 3 == 0 ? DQ_RNN_SIGMOID : DQ_RNN_TANH);
        c->act[i] = k;
        c->alpha[i] = activation_alpha ? activation_alpha[i] : default_alpha(k);
        c->beta[i] = activation_beta ? activation_beta[i] : default_beta(k);
    }
    for (int i = 0; i < 3 * dirs; ++i)
        c->def_act = c->def_act && c->act[i] == (i % 3 == 0 ? DQ_RNN_SIGMOID : DQ_RNN_TANH);
    c->clip = clip > 0.0f ? clip : 0.0f;
    c->input_forget = input_forget ? 1 : 0;
    const int h = (int)hidden_size;
    c->NT = (h + 7) / 8;
    const int KF = (h + 31) / 32, KFW = (KF + kWaves - 1) / kWaves;
    c->CN = KFW <= 1 ? 1 : KFW <= 2 ? 2 : kMaxCN;
    const int KFWp = (KFW + c->CN - 1) / c->CN * c->CN;
    c->KFP = kWaves * KFWp;
    c->BT = (int)((batch_size + 31) / 32);
    int rc = DQ_OK;
    (void)hipGetDevice(&c->device);
    const size_t N = (size_t)dirs * 4 * h, cols = (size_t)dirs * c->NT * 32;
    const size_t state = (size_t)dirs * batch_size * h;
    const size_t hstate = (size_t)dirs * c->BT * c->KFP * 1024;
    bool ok = hipMalloc(&c->wsc, N * 4) == hipSuccess && hipMalloc(&c->wzp, N) == hipSuccess &&
              hipMalloc(&c->wb, N * 4) == hipSuccess &&
              hipMalloc(&c->rp, (size_t)dirs * c->NT * c->KFP * 1024) == hipSuccess &&
              hipMalloc(&c->rcs, cols * 4) == hipSuccess && hipMalloc(&c->rbeta, cols * 4) == hipSuccess &&
              hipMalloc(&c->rsc, cols * 4) == hipSuccess && hipMalloc(&c->rbias, cols * 4) == hipSuccess &&
              hipMalloc(&c->pp, (size_t)dirs * c->NT * 8 * 16) == hipSuccess &&
              hipMalloc(&c->hs, std::max<size_t>(2 * hstate, 1) * 4) == hipSuccess &&
              hipMalloc(&c->cs, std::max<size_t>(state, 1) * 4) == hipSuccess &&
              hipMalloc(&c->mm, (size_t)dirs * 3 * 2 * kSlots * 4) == hipSuccess;
    if (ok && M > 0) ok = hipMalloc(&c->xw, (size_t)M * N * 4) == hipSuccess;
    if (!ok) {
        free_ctx(c);
        DQ_FAIL(DQ_ERR_ALLOC, "device allocation for the LSTM context failed");
    }
    if (M > 0) {
        rc = dq_qgemm_init(&c->qg, M, (int64_t)N, input_size, DQ_F32, 0, w_type, 0, DQ_F32, 1.0f);
        if (rc) {
            free_ctx(c);
            return rc;
        }
    }
    char buf[320];
    snprintf(buf, sizeof buf,
             "gfx950 DynamicQuantizeLSTM: input projection = %s; step = one k_lstm_step<%d,%d> launch, "
             "%d x %lld x %d workgroups of 8 units x 32 batch entries, mfma_i32_32x32x32_i8, H quantized in registers",
             c->qg ? dq_qgemm_info(c->qg) : "none", c->CN, (int)c->def_act, c->NT, (long long)((batch_size + 31) / 32),
             dirs);
    c->info = buf;
    *ctx = c;
    return DQ_OK;
}

extern "C" int dq_lstm_set_weights(dq_lstm_ctx* ctx, const void* W, const float* W_scale, int64_t W_scale_len,
                                   const void* W_zero_point, const void* R, const float* R_scale,
                                   int64_t R_scale_len, const void* R_zero_point, const float* B, const float* P,
                                   void* stream) {
    if (!ctx) DQ_FAIL(DQ_ERR_STATE, "no context");
    if (!W || !W_scale || !R || !R_scale) DQ_FAIL(DQ_ERR_ARG, "W, R and their scales must not be NULL");
    const int dirs = ctx->dirs;
    const int64_t h = ctx->h;
    if ((W_scale_len != dirs && W_scale_len != dirs * 4 * h) || (R_scale_len != dirs && R_scale_len != dirs * 4 * h))
        DQ_FAIL(DQ_ERR_ARG, "scale lengths must be num_directions or num_directions * 4 * hidden_size");
    if (int rc = check_device(ctx)) return rc;
    const hipStream_t st = (hipStream_t)stream;
    const size_t N = (size_t)dirs * 4 * h;
    uint8_t* wcat = nullptr;
    if (hipMalloc(&wcat, (size_t)ctx->input * N) != hipSuccess) DQ_FAIL(DQ_ERR_ALLOC, "device allocation failed");
    const size_t nw = (size_t)ctx->input * N;
    hipLaunchKernelGGL(k_lstm_pack_w, dim3((unsigned)std::min<size_t>((nw + 255) / 256, 65536)), dim3(256), 0, st,
                       (const uint8_t*)W, (int)ctx->input, (int)h, dirs, wcat);
    hipError_t e = hipGetLastError();
    const int rho = ctx->r_type == DQ_U8 ? 128 : 0;
    const size_t nslots = (size_t)dirs * ctx->NT * ctx->KFP * 64;
    if (e == hipSuccess) {
        hipLaunchKernelGGL(k_lstm_pack_r, dim3((unsigned)std::min<size_t>((nslots + 255) / 256, 65536)), dim3(256),
                           0, st, (const uint8_t*)R, (int)h, ctx->NT, ctx->KFP, dirs, rho, ctx->rp);
        e = hipGetLastError();
    }
    if (e == hipSuccess) {
        ParamArgs p{};
        p.R = (const uint8_t*)R;
        p.w_scale = W_scale;
        p.r_scale = R_scale;
        p.B = B;
        p.P = P;
        p.w_zp = W_zero_point;
        p.r_zp = R_zero_point;
        p.w_len = (int)W_scale_len;
        p.r_len = (int)R_scale_len;
        p.w_u8 = ctx->w_type == DQ_U8;
        p.r_u8 = ctx->r_type == DQ_U8;
        p.rho = rho;
        p.h = (int)h;
        p.NT = ctx->NT;
        p.dirs = dirs;
        p.wsc = ctx->wsc;
        p.wzp = ctx->wzp;
        p.wb = ctx->wb;
        p.rcs = ctx->rcs;
        p.rbeta = ctx->rbeta;
        p.rsc = ctx->rsc;
        p.rbias = ctx->rbias;
        p.pp = ctx->pp;
        hipLaunchKernelGGL(k_lstm_params, dim3((unsigned)((ctx->NT * 32 + 255) / 256), (unsigned)dirs), dim3(256), 0,
                           st, p);
        e = hipGetLastError();
    }
    int rc = DQ_OK;
    if (e != hipSuccess) {
        dq_set_error("launch of the LSTM weight packing failed: %s", hipGetErrorString(e));
        rc = DQ_ERR_HIP;
    } else if (ctx->qg) {
        rc = dq_qgemm_set_b(ctx->qg, wcat, ctx->wsc, (int64_t)N, ctx->wzp, (int64_t)N, stream);
    }
    if (rc == DQ_OK && hipStreamSynchronize(st) != hipSuccess) {
        dq_set_error("hipStreamSynchronize failed after the LSTM weight packing");
        rc = DQ_ERR_HIP;
    }
    (void)hipFree(wcat);
    if (rc == DQ_OK) ctx->has_w = true;
    return rc;
}

extern "C" int dq_lstm_forward(dq_lstm_ctx* ctx, const float* X, const int32_t* sequence_lens, const float* initial_h,
                               const float* initial_c, float* Y, float* Y_h, float* Y_c, void* stream) {
    if (!ctx) DQ_FAIL(DQ_ERR_STATE, "no context");
    if (!ctx->has_w) DQ_FAIL(DQ_ERR_STATE, "dq_lstm_set_weights has not been called");
    if (int rc = check_device(ctx)) return rc;
    const int64_t seq = ctx->seq, batch = ctx->batch, h = ctx->h;
    const int dirs = ctx->dirs;
    if (batch == 0) return DQ_OK;
    if (seq > 0 && !X) DQ_FAIL(DQ_ERR_ARG, "X must not be NULL");
    const hipStream_t st = (hipStream_t)stream;
    if (seq > 0) {
        if (int rc = dq_qgemm_forward(ctx->qg, X, nullptr, nullptr, nullptr, 0, 0, ctx->wb, nullptr, nullptr, ctx->xw,
                                      stream))
            return rc;
    }
    const int nmm = dirs * 3 * 2 * kSlots;
    hipLaunchKernelGGL(k_lstm_mm_reset, dim3((nmm + 255) / 256), dim3(256), 0, st, ctx->mm, nmm);
    DQ_LAUNCH_CHECK("LSTM extremes reset");
    const size_t hstate = (size_t)dirs * ctx->BT * ctx->KFP * 1024;
    const int per_dir = (int)(batch * h);
    hipLaunchKernelGGL(k_lstm_begin, dim3((unsigned)((per_dir + 255) / 256), (unsigned)dirs), dim3(256), 0, st,
                       initial_h, initial_c, (int)batch, (int)h, ctx->BT, ctx->KFP, ctx->hs, ctx->cs, ctx->mm,
                       seq == 0 ? Y_h : nullptr, seq == 0 ? Y_c : nullptr);
    DQ_LAUNCH_CHECK("LSTM initial state");
    StepArgs a{};
    a.xw = ctx->xw;
    a.rp = ctx->rp;
    a.rcs = ctx->rcs;
    a.rbeta = ctx->rbeta;
    a.rsc = ctx->rsc;
    a.rbias = ctx->rbias;
    a.pp = ctx->pp;
    a.lens = sequence_lens;
    a.c = ctx->cs;
    a.y = Y;
    a.mm = ctx->mm;
    a.seq = (int)seq;
    a.batch = (int)batch;
    a.h = (int)h;
    a.N = (int)(dirs * 4 * h);
    a.NT = ctx->NT;
    a.KFP = ctx->KFP;
    a.BT = ctx->BT;
    a.dirs = dirs;
    a.rev_mask = ctx->direction == DQ_LSTM_REVERSE ? 1 : ctx->direction == DQ_LSTM_BIDIRECTIONAL ? 2 : 0;
    for (int i = 0; i < 6; ++i) {
        a.act[i] = ctx->act[i];
        a.alpha[i] = ctx->alpha[i];
        a.beta[i] = ctx->beta[i];
    }
    a.clip = ctx->clip;
    a.input_forget = ctx->input_forget;
    const dim3 grid((unsigned)ctx->NT, (unsigned)((batch + 31) / 32), (unsigned)dirs);
    for (int64_t s = 0; s < seq; ++s) {
        a.s = (int)s;
        a.rd_slot = (int)(s % 3);
        a.wr_slot = (int)((s + 1) % 3);
        a.clr_slot = (int)((s + 2) % 3);
        a.hin = ctx->hs + (size_t)(s & 1) * hstate;
        a.hout = ctx->hs + (size_t)((s + 1) & 1) * hstate;
        a.yh = s == seq - 1 ? Y_h : nullptr;
        a.yc = s == seq - 1 ? Y_c : nullptr;
#define DQ_STEP(CN_)                                                                                      \
    do {                                                                                                  \
        if (ctx->def_act) hipLaunchKernelGGL((k_lstm_step<CN_, true>), grid, dim3(kThreads), 0, st, a);  \
        else hipLaunchKernelGGL((k_lstm_step<CN_, false>), grid, dim3(kThreads), 0, st, a);              \
    } while (0)
        switch (ctx->CN) {
            case 1: DQ_STEP(1); break;
            case 2: DQ_STEP(2); break;
            default: DQ_STEP(kMaxCN); break;
        }
#undef DQ_STEP
        DQ_LAUNCH_CHECK("LSTM step");
    }
    return DQ_OK;
}

extern "C" const char* dq_lstm_info(const dq_lstm_ctx* ctx) { return ctx ? ctx->info.c_str() : nullptr; }

extern "C" void dq_lstm_release(dq_lstm_ctx* ctx) { free_ctx(ctx); }
