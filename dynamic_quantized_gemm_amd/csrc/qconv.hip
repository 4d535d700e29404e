// qconv.hip -- general 2-D QLinearConv on gfx950 matrix cores (implicit GEMM).
//
// ONNX "QLinearConv" (opset 10), description and inputs: x [N, C, H, W] and
// w [M, C / group, kH, kW] are 8-bit with zero points (w's per tensor or per
// output channel), the optional bias is int32 with scale x_scale * w_scale
// and zero point 0, y is requantized with y_scale / y_zero_point; the output
// size follows the kernel, strides and pads (ONNX Conv's attributes:
// strides, begin / end pads, dilations, group). For output channel m of
// group g and output pixel (oh, ow):
//   acc  = sum_{c, kh, kw} (w[m,c,kh,kw] - w_zp[m]) * (x[n, g Cg + c, ih, iw] - x_zp)
//          + bias[m],   ih = oh sh - pt + kh dh,  iw = ow sw - pl + kw dw
//   real = ((float)acc * x_scale) * w_scale[m]
//   y    = saturate(rne(real / y_scale) + y_zp)
// where a tap outside the image reads x_zp (a padded input is a real 0).
//
// As in the 1x1 kernel the int8 MFMA takes w^ = w - a and x^ = x - b (a, b =
// 128 for uint8, 0 for int8) and
//   acc = sum w^ x^ + (b - x_zp) R[m] + (a - w_zp[m]) S[p] + K (a - w_zp[m]) (b - x_zp) + bias[m]
// with R[m] = sum w^ over the K = Cg kH kW real taps (computed when the
// weights are set) and S[p] = sum x^ over the same taps (one more MFMA
// against 1s, only when some a - w_zp[m] can be non-zero). Padded channels
// (past Cg in the last chunk) hold w^ = x^ = 0 and drop out of every term;
// spatial pads hold x^ = x_zp - b and cancel exactly.
//
// The reduction runs over (input channel chunk of 32, kernel tap). A first
// kernel (k_conv_prep_x) writes the prepared input: per image, group and
// chunk, rows x padded columns x 32 channels (channels contiguous, shifted
// to int8, spatial pads holding x_zp - b), so that the input patch a
// workgroup's pixels need for one chunk is one contiguous run. A workgroup
// of four waves owns 64 WM output channels x 64 (4 / WM) output pixels of
// one image and group and copies each chunk's patch straight into LDS
// (global_load_lds_dwordx4; two buffers, the next chunk's copy in flight
// during this chunk's MFMAs); for any tap a lane's MFMA operand (16 channels
// of one input pixel) is then one ds_read_b128 at the lane's pixel offset
// plus a tap offset that is the same for every lane. The weights are packed once per set_w into rows of
// [tap][channel] (32-channel runs contiguous), read as 16-byte fragments.
// The epilogue requantizes as the other quantizers do and stores whole
// 16-byte row segments of y (NCHW).
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <vector>

#include "dq_device.h"

namespace {

constexpr int kKC = 32;         // input channels per chunk
constexpr int kThreads = 256;
constexpr int kYPitch = 80;     // LDS bytes per staged output row (64 + 16)
constexpr int kPatchMax = 112 * 1024;  // with the 20 KiB output stage, within 160 KiB of LDS
constexpr int kKMax = 32768;    // real taps per output: int32 sums stay exact
constexpr int kTapGroup = 9;    // taps whose weight fragments a lane holds at once
constexpr int kTapMax = 1024;   // padded taps per kernel (a per-workgroup table of their offsets)
constexpr int kSplitBelow = 256;  // split the reduction when fewer workgroups than this would run

typedef dq::v4i v4i;

struct ConvShape {
    int C, H, W, M, KH, KW, sh, sw, pt, pl, dh, dw, G, Cg, Mg, OH, OW, P;
    int T;     // KH * KW
    int Tp;    // T rounded up to a tap group (padded taps hold zero weights)
    int Kc;    // Cg rounded up to a chunk
    int Mgp;   // Mg rounded up to the channel tile
    int K;     // Cg * KH * KW real taps
    int cpad;  // patch columns left of iw = 0 (a multiple of 4, >= pl)
    int ncol;  // patch columns (a multiple of 4)
    int mtiles;
    dq::FastDiv ow_div;
    // depthwise planes (k_qconv_dw): padded plane rows x columns, output
    // strips of four pixels per row
    int hp, wp, spr;
    dq::FastDiv spr_div, w_div, wq_div;  // wq_div: W / 4 (k_conv_prep_t)
    // virtual channels (vc = 1, few channels a group, kernel rows of at most
    // 8 taps): the implicit GEMM runs on a KH x 1 convolution whose 32
    // channels are (kernel column kw, input channel c < 4) pairs, channel
    // 4 kw + c of virtual column ow holding x[c, ih, ow sw - pl + kw dw]
    // (made by k_conv_prep_x). The fields above then describe that virtual
    // convolution (W = OW, KW = 1, stride, pad and dilation along columns
    // 1 / 0 / 1, Cg = Kc = 32; K stays the real tap count), and these the
    // real input.
    int vc, rW, rsw, rpl, rdw, rCg, rKW;
};

// Byte offset of w^[row][tap t][channel c] in the packed weights: 1 KiB
// MFMA fragments of 32 rows x 32 channels, fragment ((row / 32) Tp + t)
// (Kc / 32) + c / 32, and inside it lane slot (row % 32) + 32 ((c % 32) / 16)
// holds channels 16 ((c % 32) / 16) .. + 15 of the row: a wave's operand
// load of one fragment reads 1 KiB of consecutive bytes.
__host__ __device__ __forceinline__ size_t wpos(int row, int t, int c, int Tp, int Kc) {
    const size_t frag = ((size_t)(row >> 5) * Tp + t) * (Kc >> 5) + (c >> 5);
    return (frag << 10) + ((size_t)((row & 31) + ((c & 16) << 1)) << 4) + (c & 15);
}

struct ConvArgs {
    const uint8_t* x;
    const int8_t* wp;     // packed w^ (wpos), [G * Mgp] rows of [Tp][Kc]
    const int32_t* R;     // [G * Mgp]
    const float* ws;      // [M]
    const int32_t* wz;    // [M]
    const int32_t* bias;  // [M]
    const float* x_scale;
    const void* x_zp;
    const float* y_scale;
    const void* y_zp;
    uint8_t* y;
    uint32_t xflip;       // 0x80808080 for a uint8 x
    int kA, kB, x_u8, y_u8, vecy;
    int vecy4;            // y 4-byte aligned and OW % 4 == 0 (k_qconv_dw's word stores)
    // the prepared input of the implicit GEMM (k_conv_prep_x): bytes per
    // prepared row (ncol x 32) and per 32-channel chunk (rows x row bytes);
    // bytes of one LDS patch buffer (a multiple of 1 KiB)
    const uint8_t* xb;
    size_t xb_rs, xb_cs;
    int pbuf;
    int vecx_plane;       // x 4-byte aligned and H W % 4 == 0 (k_qconv_dw's word loads)
    int y_lo, y_hi;       // y's saturation range
    // split reduction: blockIdx.z = image * nsplit + split, each split walks
    // cps chunks and leaves int32 partial sums for k_qconv_reduce
    int nsplit, cps;
    int32_t* part;        // [N * nsplit][M][P]: sum w^ x^ over the split's chunks
    int32_t* spart;       // [N * nsplit][G][P]: sum x^ over them (XSUM)
};

// The requantization shared by the epilogue and the split reduction:
// y = saturate(rne(((float)acc * x_scale) * w_scale / y_scale) + y_zp), with
// the corrected quotient where the scale allows it (as the quantizers
// round), the 1.5 * 2^23 rounding add, a median clamp against the saturation
// bounds minus the zero point, and the zero point added to four packed
// codes at once (carry-free bytewise add).
constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
constexpr float kBig = 4194304.0f;     // 2^22

struct YQuant {
    float x_scale, lof, hif;
    dq::QDiv yd;
    int y_zp, y_lo, y_hi;
    uint32_t Yz;
};

__device__ __forceinline__ int zp8(const void* zp, bool u8) {
    if (!zp) return 0;
    return u8 ? (int)*(const uint8_t*)zp : (int)*(const int8_t*)zp;
}

__device__ __forceinline__ YQuant make_yquant(const ConvArgs& a) {
    YQuant q;
    q.x_scale = *a.x_scale;
    q.yd = dq::make_qdiv(*a.y_scale);
    q.y_zp = zp8(a.y_zp, a.y_u8);
    q.y_lo = a.y_lo;
    q.y_hi = a.y_hi;
    q.lof = kMagic + (float)(a.y_lo - q.y_zp);
    q.hif = kMagic + (float)(a.y_hi - q.y_zp);
    q.Yz = (uint32_t)(q.y_zp & 0xff) * 0x01010101u;
    return q;
}

// four exact sums of one output channel (scale wsc) to four packed codes
__device__ __forceinline__ uint32_t requant4(const uint32_t (&v)[4], float wsc, const YQuant& q) {
    if (q.yd.fast) {
        uint32_t b[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float real = (float)(int32_t)v[e] * q.x_scale;
            real = real * wsc;
            const float q0 = __builtin_amdgcn_fmed3f(real * q.yd.y, -kBig, kBig);
            const float rr = __builtin_fmaf(-q0, q.yd.s, real);
            const float tt = __builtin_fmaf(rr, q.yd.y, q0) + kMagic;
            b[e] = (uint32_t)__float_as_int(__builtin_amdgcn_fmed3f(tt, q.lof, q.hif));
        }
        const uint32_t packed = (b[0] & 0xffu) | ((b[1] & 0xffu) << 8) | ((b[2] & 0xffu) << 16) | (b[3] << 24);
        return ((packed & 0x7f7f7f7fu) + (q.Yz & 0x7f7f7f7fu)) ^ ((packed ^ q.Yz) & 0x80808080u);
    }
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float real = (float)(int32_t)v[e] * q.x_scale;
        real = real * wsc;
        const int code = dq::sat_add(dq::rne(real / q.yd.s), q.y_zp, q.y_lo, q.y_hi);
        word |= ((uint32_t)code & 0xffu) << (8 * e);
    }
    return word;
}


template <bool XSUM, int WM, int IB, bool SPLIT>
__global__ __launch_bounds__(kThreads) void k_qconv(ConvShape sh, ConvArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t patch[];
    __shared__ __attribute__((aligned(16))) uint8_t ys[4 * 64 * kYPitch];
    __shared__ int tapoff[kTapMax];  // patch byte offset of each tap (0 for padded taps)
    constexpr int WP = 4 / WM, PT = 32 * IB * WP, MT = 64 * WM;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % WM, wp = wave / WM;
    const int n = SPLIT ? (int)blockIdx.z / a.nsplit : (int)blockIdx.z;
    const int c_beg = SPLIT ? ((int)blockIdx.z - n * a.nsplit) * a.cps * kKC : 0;
    const int c_end = SPLIT ? std::min(c_beg + a.cps * kKC, sh.Kc) : sh.Kc;
    const int g = blockIdx.y / sh.mtiles, mt = blockIdx.y - g * sh.mtiles;
    const int m0 = mt * MT + 64 * wm;  // this wave's first channel within the group
    const int p0 = blockIdx.x * PT, pw0 = p0 + 32 * IB * wp;

    // the block's patch: output rows oh_a .. oh_b need prepared rows r0 ..
    // r0 + nr - 1 (prepared row r holds input row r - pt), every prepared
    // column, 32 channels: one contiguous run of the prepared input
    const int oh_a = (int)dq::fdiv((uint32_t)p0, sh.ow_div);
    const int oh_b = (int)dq::fdiv((uint32_t)(std::min(p0 + PT, sh.P) - 1), sh.ow_div);
    const int r0 = oh_a * sh.sh;
    const int nr = (oh_b - oh_a) * sh.sh + (sh.KH - 1) * sh.dh + 1;
    const int pbytes = nr * sh.ncol * kKC;

    // the lane's IB MFMA pixel rows: patch byte offsets for tap (0, 0)
    // (prepared column = input column + pl = ow sw + kw dw)
    int pix[IB];
#pragma unroll
    for (int pb = 0; pb < IB; ++pb) {
        const int p = std::min(pw0 + 32 * pb + (lane & 31), sh.P - 1);
        const int oh = (int)dq::fdiv((uint32_t)p, sh.ow_div), ow = p - oh * sh.OW;
        const int r = (oh - oh_a) * sh.sh, c = ow * sh.sw;
        pix[pb] = (r * sh.ncol + c) * kKC + 16 * (lane >> 5);
    }

    const int x_zp = zp8(a.x_zp, a.x_u8);

    // chunk cc's patch straight from the prepared input into LDS
    // (global_load_lds_dwordx4: 1 KiB a wave instruction, no VGPRs); the
    // last KiB may run past the patch, within the prepared buffer's slack
    // and the LDS buffer's rounding
    const uint8_t* xsrc = a.xb + ((size_t)(n * sh.G + g) * (sh.Kc / kKC)) * a.xb_cs + (size_t)r0 * a.xb_rs +
                          16 * lane;
    auto patch_copy = [&](int cc, uint8_t* dst) {
        const uint8_t* src = xsrc + (size_t)cc * a.xb_cs;
        for (int blk = wave; blk * 1024 < pbytes; blk += 4) dq::copy16_to_lds(src + blk * 1024, dst + blk * 1024);
    };

    dq::v16i acc[IB][2], sacc[IB];
#pragma unroll
    for (int i = 0; i < IB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            acc[i][0][r] = 0;
            acc[i][1][r] = 0;
            sacc[i][r] = 0;
        }
    const v4i ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
    // weights: this wave's fragments for tap t and chunk c0 start at
    // wbase + (t (Kc / 32) + c0 / 32) KiB (+ Tp (Kc / 32) KiB for the second
    // 32-channel block); each lane reads its 16 bytes at 16 lane
    const int kc32 = sh.Kc >> 5;
    const int8_t* wbase = a.wp + wpos(g * sh.Mgp + m0, 0, 0, sh.Tp, sh.Kc) + 16 * lane;
    const size_t wjb = (size_t)sh.Tp * kc32 << 10;
    // the tap offsets, once per workgroup (made visible by the first
    // chunk's barrier)
    for (int t = tid; t < sh.Tp; t += kThreads) {
        const int kh = t / sh.KW, kw = t - kh * sh.KW;
        tapoff[t] = t < sh.T ? (kh * sh.dh * sh.ncol + kw * sh.dw) * kKC : 0;
    }

    // The taps of a staged chunk: a tap group's weight fragments are all
    // requested before its first MFMA; every MFMA runs (a padded tap has zero
    // weights, reads the patch at tap (0, 0) and adds zeros to the pixel sums).
    const v4i zeros = {0, 0, 0, 0};
    auto load_w = [&](v4i (&wf)[kTapGroup][2], int tg, int c0) {
        const int8_t* wg = wbase + (((size_t)tg * kc32 + (c0 >> 5)) << 10);
#pragma unroll
        for (int i = 0; i < kTapGroup; ++i) {
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
                wf[i][jb] = *reinterpret_cast<const v4i*>(wg + (((size_t)i * kc32) << 10) + jb * wjb);
        }
    };
    auto mfma_group = [&](const v4i (&wf)[kTapGroup][2], const uint8_t* buf, int tg) {
#pragma unroll
        for (int i = 0; i < kTapGroup; ++i) {
            const int t = tg + i;
            const int off = tapoff[t];
            const v4i ones_t = t < sh.T ? ones : zeros;
            v4i xf[IB];
#pragma unroll
            for (int ib = 0; ib < IB; ++ib) xf[ib] = *reinterpret_cast<const v4i*>(&buf[pix[ib] + off]);
#pragma unroll
            for (int ib = 0; ib < IB; ++ib) {
#pragma unroll
                for (int jb = 0; jb < 2; ++jb)
                    acc[ib][jb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xf[ib], wf[i][jb], acc[ib][jb], 0, 0, 0);
                if (XSUM) sacc[ib] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xf[ib], ones_t, sacc[ib], 0, 0, 0);
            }
        }
    };

    // Two patch buffers: chunk c's MFMAs run while chunk c + 1's copy is in
    // flight. Per chunk: its first tap group's weights are requested, then
    // the next patch's copies (so that waiting for the weights does not wait
    // for the copies: vector memory operations complete in order), then the
    // MFMAs; at the end every wave waits for its copies and its LDS reads,
    // and one barrier makes the next patch visible and frees this one.
    patch_copy(c_beg / kKC, patch);
    dq::wait_vmcnt_lgkm0<0>();  // this wave's copies and tap offsets
    dq::lds_barrier();
    int bsel = 0;
    for (int c0 = c_beg; c0 < c_end; c0 += kKC) {
        const uint8_t* cur = patch + bsel * a.pbuf;
        v4i wf[kTapGroup][2];
        load_w(wf, 0, c0);
        if (c0 + kKC < c_end) patch_copy(c0 / kKC + 1, patch + (bsel ^ 1) * a.pbuf);
        mfma_group(wf, cur, 0);
        for (int tg = kTapGroup; tg < sh.Tp; tg += kTapGroup) {
            load_w(wf, tg, c0);
            mfma_group(wf, cur, tg);
        }
        dq::wait_vmcnt_lgkm0<0>();
        dq::lds_barrier();
        bsel ^= 1;
    }

    // the accumulators are read right below: the last MFMA's results first
    // need the ISA's wait states (dq::mfma_result_drain)
    dq::mfma_result_drain();

    // lane holds channel (lane % 32) of block jb and, in accumulators
    // 4q .. 4q+3, pixels 8q + 4 (lane / 32) + 0..3 of pixel block ib
    if (SPLIT) {
        // the split's raw sums (four consecutive pixels a lane and group),
        // and its pixel sums from one wave per pixel range
        const bool vec4 = sh.P % 4 == 0;
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            const int ml = m0 + 32 * jb + (lane & 31);
            if (ml >= sh.Mg) continue;
            int32_t* dst = a.part + ((size_t)blockIdx.z * sh.M + (size_t)g * sh.Mg + ml) * sh.P;
#pragma unroll
            for (int ib = 0; ib < IB; ++ib)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int p = pw0 + 32 * ib + 8 * q + 4 * (lane >> 5);
                    const v4i v = {acc[ib][jb][4 * q], acc[ib][jb][4 * q + 1], acc[ib][jb][4 * q + 2],
                                   acc[ib][jb][4 * q + 3]};
                    if (vec4 && p + 4 <= sh.P) {
                        *reinterpret_cast<v4i*>(dst + p) = v;
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (p + e < sh.P) dst[p + e] = v[e];
                    }
                }
        }
        if (XSUM && wm == 0 && (lane & 31) == 0) {
            int32_t* dst = a.spart + ((size_t)blockIdx.z * sh.G + g) * sh.P;
#pragma unroll
            for (int ib = 0; ib < IB; ++ib)
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int p = pw0 + 32 * ib + 8 * q + 4 * (lane >> 5) + e;
                        if (p < sh.P) dst[p] = sacc[ib][4 * q + e];
                    }
        }
        return;
    }

    // ---- requantizing epilogue
    const YQuant yq = make_yquant(a);
    uint8_t* ysw = ys + 64 * wave * kYPitch;
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
        const int ml = m0 + 32 * jb + (lane & 31);
        const bool mok = ml < sh.Mg;
        const int mg = g * sh.Mg + (mok ? ml : 0);
        const int32_t R = a.R[g * sh.Mgp + ml];
        const int coef = a.kA - (mok ? a.wz[mg] : 0);
        const float wsc = mok ? a.ws[mg] : 0.0f;
        const uint32_t xb = (uint32_t)(a.kB - x_zp);
        const uint32_t rowc = xb * (uint32_t)R + (uint32_t)sh.K * ((uint32_t)coef * xb) +
                              (uint32_t)(mok ? a.bias[mg] : 0);
#pragma unroll
        for (int ib = 0; ib < IB; ++ib) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint32_t v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[e] = (uint32_t)acc[ib][jb][4 * q + e] + rowc;
                    if (XSUM) v[e] += (uint32_t)coef * (uint32_t)sacc[ib][4 * q + e];
                }
                const uint32_t word = requant4(v, wsc, yq);
                const int pp = 32 * ib + 8 * q + 4 * (lane >> 5);
                *reinterpret_cast<uint32_t*>(&ysw[(32 * jb + (lane & 31)) * kYPitch + pp]) = word;
            }
        }
    }
    // the wave's 64 staged rows (32 IB pixels each) back as 16-byte
    // segments (one wave's LDS operations complete in order: no barrier)
    dq::wave_lds_fence();
#pragma unroll
    for (int it = 0; it < 2 * IB; ++it) {
        const int u = lane + 64 * it;
        const int rr = u / (2 * IB), qq = u % (2 * IB);
        const int ml = m0 + rr, p = pw0 + 16 * qq;
        if (ml < sh.Mg && p < sh.P) {
            const v4i v = *reinterpret_cast<const v4i*>(&ysw[rr * kYPitch + 16 * qq]);
            uint8_t* dst = a.y + ((size_t)n * sh.M + (size_t)g * sh.Mg + ml) * sh.P + p;
            if (a.vecy && p + 16 <= sh.P) {
                *reinterpret_cast<v4i*>(dst) = v;
            } else {
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    if (p + e < sh.P) dst[e] = (uint8_t)((uint32_t)v[e >> 2] >> (8 * (e & 3)));
            }
        }
    }
}

// The prepared input of the implicit GEMM: xb[n][g][chunk][r][col][32]
// holds x^ = x - b (int8; b = 128 for uint8 x) of channel 32 chunk + j of
// group g at input row r - pt, column col - pl; outside the image x_zp - b
// (a padded input is a real 0, which the correction terms cancel), past the
// group's channels 0. With virtual channels (sh.vc) channel j = 4 kw + c of
// prepared column col holds input column col sw - pl + kw dw of channel c
// (c < Cg, kw < KW; else 0). A thread makes the 32 bytes of one (row,
// column): lanes run along columns, so each of its byte loads reads
// consecutive bytes of one channel row across the wave, and its two 16-byte
// stores are contiguous across the wave.
__global__ __launch_bounds__(256) void k_conv_prep_x(ConvShape sh, ConvArgs a, int hx, uint8_t* __restrict__ xb) {
    const int col = blockIdx.x * 64 + (threadIdx.x & 63);
    const int r = blockIdx.y * 4 + (threadIdx.x >> 6);
    const int nch = sh.Kc / kKC;
    const int z = blockIdx.z;  // (image G + group) chunks + chunk
    const int ng = z / nch, cc = z - ng * nch;
    const int n = ng / sh.G, g = ng - n * sh.G;
    if (col >= sh.ncol || r >= hx) return;
    const uint32_t flip = a.xflip & 0xffu;
    const uint32_t zb = ((uint32_t)zp8(a.x_zp, a.x_u8) & 0xffu) ^ flip;  // x_zp - b as a byte
    const int ih = r - sh.pt;
    const bool hin = ih >= 0 && ih < sh.H;
    // all 32 byte loads first, from clamped in-range addresses (so that
    // they are in flight together), then the bytes of pads and padded
    // channels replaced
    uint32_t v[32];
    bool use[32], in[32];
    if (sh.vc) {
        const uint8_t* xg = a.x + ((size_t)n * sh.C + (size_t)g * sh.rCg) * sh.H * sh.rW;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            const int kw = j >> 2, c = j & 3;
            const int iw = col * sh.rsw - sh.rpl + kw * sh.rdw;
            use[j] = c < sh.rCg && kw < sh.rKW;
            in[j] = hin && iw >= 0 && iw < sh.rW;
            const size_t off = ((size_t)(use[j] ? c : 0) * sh.H + (hin ? ih : 0)) * sh.rW +
                               (size_t)min(max(iw, 0), sh.rW - 1);
            v[j] = xg[off];
        }
    } else {
        const uint8_t* xg = a.x + ((size_t)n * sh.C + (size_t)g * sh.Cg) * sh.H * sh.W;
        const int iw = col - sh.pl;
        const bool inside = hin && iw >= 0 && iw < sh.W;
        const size_t pix = (size_t)(hin ? ih : 0) * sh.W + (size_t)min(max(iw, 0), sh.W - 1);
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            const int c = cc * kKC + j;
            use[j] = c < sh.Cg;
            in[j] = inside;
            v[j] = xg[(size_t)(use[j] ? c : 0) * sh.H * sh.W + pix];
        }
    }
    uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        const uint32_t b = use[j] ? (in[j] ? (v[j] ^ flip) : zb) : 0u;
        w[j >> 2] |= b << (8 * (j & 3));
    }
    uint8_t* dst = xb + ((size_t)z * hx + r) * a.xb_rs + (size_t)col * kKC;
    const dq::u4 lo = {w[0], w[1], w[2], w[3]}, hi = {w[4], w[5], w[6], w[7]};
    *reinterpret_cast<dq::u4*>(dst) = lo;
    *reinterpret_cast<dq::u4*>(dst + 16) = hi;
}

// The same preparation for real channels with W % 4 == 0, a 4-byte aligned
// x and W <= 512: a workgroup turns four prepared rows of one chunk around
// through LDS. Its 32 channel rows x 4 input rows are read with coalesced
// 4-byte loads into LDS ([channel][row][column]); then each thread gathers
// 16 channels of one prepared column (byte reads from LDS; pads, rows
// outside the image and channels past the group filled in) and stores them
// as one 16-byte piece, consecutive threads writing consecutive pieces.
constexpr int kPrepRows = 4;
constexpr int kPrepMaxW = 512;

__global__ __launch_bounds__(256) void k_conv_prep_t(ConvShape sh, ConvArgs a, int hx, uint8_t* __restrict__ xb) {
    extern __shared__ __attribute__((aligned(16))) uint8_t t[];  // kKC * kPrepRows * W bytes
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nch = sh.Kc / kKC;
    const int z = blockIdx.y;  // (image G + group) chunks + chunk
    const int ng = z / nch, cc = z - ng * nch;
    const int n = ng / sh.G, g = ng - n * sh.G;
    const int W = sh.W;
    const int nrb = (hx + kPrepRows - 1) / kPrepRows;
    // row blocks blockIdx.x, + gridDim.x, ... (fewer, longer workgroups)
    for (int rb = blockIdx.x; rb < nrb; rb += gridDim.x) {
    const int r0 = rb * kPrepRows;
    const int ih0 = r0 - sh.pt;
    // loads: the four input rows of one channel are one run of W words; a
    // wave takes eight channels (one run each, lane = word), all eight loads
    // in flight; words of rows outside the image or past hx and channels
    // past the group are not stored (filled in below)
    const uint8_t* xg = a.x + ((size_t)n * sh.C + (size_t)g * sh.Cg) * sh.H * W;
    for (int k0 = 0; k0 < W; k0 += 64) {
        const int k = k0 + lane;
        const int i = (int)dq::fdiv((uint32_t)k, sh.wq_div);  // row of the run
        const int ih = ih0 + i;
        const bool rok = k < W && ih >= 0 && ih < sh.H && r0 + i < hx;
        uint32_t v[8];
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const int c = cc * kKC + 8 * wave + b;
            const bool ok = rok && c < sh.Cg;
            v[b] = *reinterpret_cast<const uint32_t*>(xg + (ok ? ((size_t)c * sh.H + ih0) * W + 4 * (size_t)k : 0));
        }
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const int c = cc * kKC + 8 * wave + b;
            if (rok && c < sh.Cg) *reinterpret_cast<uint32_t*>(&t[(8 * wave + b) * kPrepRows * W + 4 * k]) = v[b];
        }
    }
    __syncthreads();
    const uint32_t flip = a.xflip & 0xffu;
    const uint32_t zb = ((uint32_t)zp8(a.x_zp, a.x_u8) & 0xffu) ^ flip;  // x_zp - b as a byte
    // stores: thread (column, half h): 16 channels of one prepared column,
    // row by row; consecutive threads write consecutive 16-byte pieces
    const int h = tid & 1;
    const int jn = min(16, sh.Cg - cc * kKC - 16 * h);  // real channels of the half
    for (int i = 0; i < kPrepRows && r0 + i < hx; ++i) {
        const int ih = ih0 + i;
        const bool hin = ih >= 0 && ih < sh.H;
        uint8_t* drow = xb + ((size_t)z * hx + r0 + i) * a.xb_rs + 16 * h;
        const uint8_t* trow = t + (16 * h * kPrepRows + i) * W;
        for (int col = tid >> 1; col < sh.ncol; col += 128) {
            const int iw = col - sh.pl;
            const bool in = hin && iw >= 0 && iw < W;
            const int iwc = in ? iw : 0;
            // all sixteen LDS reads first (unconditional, in-range rows),
            // then the pads and padded channels replaced
            uint32_t raw[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) raw[e] = trow[min(e, max(jn - 1, 0)) * kPrepRows * W + iwc];
            uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const uint32_t b = e < jn ? (in ? raw[e] ^ flip : zb) : 0u;
                w[e >> 2] |= b << (8 * (e & 3));
            }
            const dq::u4 o = {w[0], w[1], w[2], w[3]};
            *reinterpret_cast<dq::u4*>(drow + (size_t)col * kKC) = o;
        }
    }
    __syncthreads();  // the next row block overwrites the tile
    }
}

// Groups of few channels (depthwise and the like: Cg <= 4 and Mg <= 4),
// where the implicit GEMM would pad almost all of K and of the channel tile:
// one thread per output pixel, a workgroup per (image, output channel,
// 256-pixel run), so the channel's weights are the same for every lane;
// acc = sum (w^ + a - w_zp) (x - x_zp) in 24-bit multiply-adds (taps outside
// the image add nothing), then the same requantization.
__global__ __launch_bounds__(256) void k_qconv_direct(ConvShape sh, ConvArgs a) {
    const int p = blockIdx.x * 256 + threadIdx.x;
    const int m = blockIdx.y, n = blockIdx.z;
    const int g = m / sh.Mg, ml = m - g * sh.Mg;
    const int pc = p < sh.P ? p : sh.P - 1;
    const int oh = (int)dq::fdiv((uint32_t)pc, sh.ow_div), ow = pc - oh * sh.OW;
    const int x_zp = zp8(a.x_zp, a.x_u8);
    const int coef = a.kA - a.wz[m];
    // channels c < 4 of a row lie in one lane slot: tap t is kc32 KiB further
    const int8_t* wr = a.wp + wpos(g * sh.Mgp + ml, 0, 0, sh.Tp, sh.Kc);
    const size_t tstride = (size_t)(sh.Kc >> 5) << 10;
    const uint8_t* xg = a.x + ((size_t)n * sh.C + (size_t)g * sh.Cg) * sh.H * sh.W;
    int32_t acc = 0;
    for (int c = 0; c < sh.Cg; ++c) {
        const uint8_t* xc = xg + (size_t)c * sh.H * sh.W;
        for (int kh = 0; kh < sh.KH; ++kh) {
            const int ih = oh * sh.sh - sh.pt + kh * sh.dh;
            if (ih < 0 || ih >= sh.H) continue;
            const uint8_t* xr = xc + (size_t)ih * sh.W;
            for (int kw = 0; kw < sh.KW; ++kw) {
                const int iw = ow * sh.sw - sh.pl + kw * sh.dw;
                const int wv = (int)wr[(size_t)(kh * sh.KW + kw) * tstride + c] + coef;
                const int xv = (iw >= 0 && iw < sh.W)
                                   ? (a.x_u8 ? (int)xr[iw] : (int)(int8_t)xr[iw]) - x_zp
                                   : 0;
                acc = __mul24(wv, xv) + acc;
            }
        }
    }
    if (p >= sh.P) return;
    acc += a.bias[m];
    float real = (float)acc * *a.x_scale;
    real = real * a.ws[m];
    const int code = dq::sat_add(dq::rne(real / *a.y_scale), zp8(a.y_zp, a.y_u8), a.y_lo, a.y_hi);
    a.y[((size_t)n * sh.M + m) * sh.P + p] = (uint8_t)code;
}

// Depthwise (one input and one output channel a group): a workgroup per
// (image, channel) plane. The plane's x - x_zp (int16, exact) is staged in
// LDS inside a border of zeros (a padded input is a real 0, so pads add
// nothing), the channel's tap weights w - w_zp[m] sit in LDS too; each
// thread then makes four adjacent outputs of a row at a time,
// acc = sum (w - w_zp)(x - x_zp) + bias in 24-bit multiply-adds (|terms| <
// 2^16, at most 1024 taps), and requantizes them as the other kernels do.
// KS3 specializes the 3x3 kernel at stride and dilation 1, where the six
// input columns of a strip's row are read once.
typedef short s2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ s2 as_s2(uint32_t v) { return __builtin_bit_cast(s2, v); }

constexpr int kDwLdsMax = 60 * 1024;  // dynamic LDS of the staged plane (with the 4 KiB of weights: 64 KiB)

template <bool KS3>
__global__ __launch_bounds__(256) void k_qconv_dw(ConvShape sh, ConvArgs a) {
    extern __shared__ __attribute__((aligned(16))) int16_t xs[];
    __shared__ int32_t wsh[kTapMax];
    const int tid = threadIdx.x;
    const int m = blockIdx.x, n = blockIdx.y;
    const int Wp = sh.wp;
    // the staged plane and its slack (the last strip of a row may read up
    // to 3 sw columns past the row, into the next one or the slack)
    const int nel = sh.hp * Wp + 3 * sh.sw + 1;
    for (int i = tid; i < (nel + 1) >> 1; i += 256) reinterpret_cast<int32_t*>(xs)[i] = 0;
    const int8_t* wr = a.wp + wpos(m * sh.Mgp, 0, 0, sh.Tp, sh.Kc);
    const size_t tstride = (size_t)(sh.Kc >> 5) << 10;
    const int coef = a.kA - a.wz[m];
    for (int t = tid; t < sh.T; t += 256) wsh[t] = (int)wr[(size_t)t * tstride] + coef;
    __syncthreads();
    const int x_zp = zp8(a.x_zp, a.x_u8);
    const uint8_t* xp = a.x + ((size_t)n * sh.C + m) * sh.H * sh.W;
    // the plane as 4-byte words (whole words when the plane's size and x
    // allow it, else byte by byte), four words a thread in flight, each
    // byte then placed at its padded position
    const int hw = sh.H * sh.W;
    const int nwords = (hw + 3) >> 2;
    if (a.vecx_plane && (sh.W & 3) == 0) {
        // a word never straddles two rows: one division a word
        for (int i0 = tid; i0 < nwords; i0 += 4 * 256) {
            uint32_t word[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                word[k] = *reinterpret_cast<const uint32_t*>(xp + 4 * min(i0 + 256 * k, nwords - 1));
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int i = i0 + 256 * k;
                if (i >= nwords) break;
                const int ih = (int)dq::fdiv((uint32_t)(4 * i), sh.w_div), iw = 4 * i - ih * sh.W;
                const int r = ih + sh.pt, c = iw + sh.pl;
                if (r >= sh.hp) continue;
                int16_t* d = xs + r * Wp + c;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t b = (word[k] >> (8 * e)) & 0xffu;
                    const int xv = a.x_u8 ? (int)b : (int)(int8_t)b;
                    if (c + e < Wp) d[e] = (int16_t)(xv - x_zp);
                }
            }
        }
    } else
    for (int i0 = tid; i0 < nwords; i0 += 4 * 256) {
        uint32_t word[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int i = min(i0 + 256 * k, nwords - 1);
            if (a.vecx_plane) {
                word[k] = *reinterpret_cast<const uint32_t*>(xp + 4 * i);
            } else {
                word[k] = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (4 * i + e < hw) word[k] |= (uint32_t)xp[4 * i + e] << (8 * e);
            }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int i = i0 + 256 * k;
            if (i >= nwords) break;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int f = 4 * i + e;
                if (f >= hw) break;
                const int ih = (int)dq::fdiv((uint32_t)f, sh.w_div), iw = f - ih * sh.W;
                const int r = ih + sh.pt, c = iw + sh.pl;
                const uint32_t b = (word[k] >> (8 * e)) & 0xffu;
                const int xv = a.x_u8 ? (int)b : (int)(int8_t)b;
                if (r < sh.hp && c < Wp) xs[r * Wp + c] = (int16_t)(xv - x_zp);
            }
        }
    }
    __syncthreads();
    const YQuant yq = make_yquant(a);
    const float wsc = a.ws[m];
    const uint32_t bias = (uint32_t)a.bias[m];
    uint8_t* yp = a.y + ((size_t)n * sh.M + m) * sh.P;
    // 3x3: each kernel row's weights as int16 pairs (w0 w1), (w2 0), (0 w2)
    s2 wA[3], wB[3], wC[3];
    if (KS3) {
#pragma unroll
        for (int kh = 0; kh < 3; ++kh) {
            const int w0 = wsh[3 * kh], w1 = wsh[3 * kh + 1], w2 = wsh[3 * kh + 2];
            wA[kh] = s2{(short)w0, (short)w1};
            wB[kh] = s2{(short)w2, 0};
            wC[kh] = s2{0, (short)w2};
        }
    }
    const int total = sh.OH * sh.spr;
    for (int s = tid; s < total; s += 256) {
        const int oh = (int)dq::fdiv((uint32_t)s, sh.spr_div), ow0 = 4 * (s - oh * sh.spr);
        int acc[4] = {0, 0, 0, 0};
        if (KS3) {
            // the row's six inputs as int16 pairs (x0 x1)(x2 x3)(x4 x5) from
            // three aligned words (Wp and ow0 are even), the odd pairs by a
            // byte shift, then two v_dot2_i32_i16 per output and row
#pragma unroll
            for (int kh = 0; kh < 3; ++kh) {
                const uint32_t* row = reinterpret_cast<const uint32_t*>(xs + (oh + kh) * Wp + ow0);
                const uint32_t p0 = row[0], p2 = row[1], p4 = row[2];
                const uint32_t p1 = __builtin_amdgcn_alignbyte(p2, p0, 2);
                const uint32_t p3 = __builtin_amdgcn_alignbyte(p4, p2, 2);
                acc[0] = __builtin_amdgcn_sdot2(as_s2(p0), wA[kh], acc[0], false);
                acc[0] = __builtin_amdgcn_sdot2(as_s2(p2), wB[kh], acc[0], false);
                acc[1] = __builtin_amdgcn_sdot2(as_s2(p1), wA[kh], acc[1], false);
                acc[1] = __builtin_amdgcn_sdot2(as_s2(p3), wB[kh], acc[1], false);
                acc[2] = __builtin_amdgcn_sdot2(as_s2(p2), wA[kh], acc[2], false);
                acc[2] = __builtin_amdgcn_sdot2(as_s2(p4), wB[kh], acc[2], false);
                acc[3] = __builtin_amdgcn_sdot2(as_s2(p3), wA[kh], acc[3], false);
                acc[3] = __builtin_amdgcn_sdot2(as_s2(p4), wC[kh], acc[3], false);
            }
        } else {
            for (int kh = 0; kh < sh.KH; ++kh) {
                const int16_t* row = xs + (oh * sh.sh + kh * sh.dh) * Wp + ow0 * sh.sw;
                for (int kw = 0; kw < sh.KW; ++kw) {
                    const int wv = wsh[kh * sh.KW + kw];
                    const int16_t* rk = row + kw * sh.dw;
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[e] = __mul24(wv, (int)rk[e * sh.sw]) + acc[e];
                }
            }
        }
        uint32_t v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (uint32_t)acc[e] + bias;
        const uint32_t word = requant4(v, wsc, yq);
        uint8_t* dst = yp + (size_t)oh * sh.OW + ow0;
        if (a.vecy4 && ow0 + 4 <= sh.OW) {
            *reinterpret_cast<uint32_t*>(dst) = word;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (ow0 + e < sh.OW) dst[e] = (uint8_t)(word >> (8 * e));
        }
    }
}

// The split reduction: the partial sums of every split, the zero-point and
// bias terms of the epilogue, then the same requantization. One thread per
// four consecutive pixels of (image n, output channel m).
template <bool XSUM>
__global__ __launch_bounds__(256) void k_qconv_reduce(ConvShape sh, ConvArgs a) {
    const int p = (blockIdx.x * 256 + threadIdx.x) * 4;
    const int m = blockIdx.y, n = blockIdx.z;
    if (p >= sh.P) return;
    const int g = m / sh.Mg, ml = m - g * sh.Mg;
    const int x_zp = zp8(a.x_zp, a.x_u8);
    const int coef = a.kA - a.wz[m];
    const uint32_t xb = (uint32_t)(a.kB - x_zp);
    const uint32_t rowc = xb * (uint32_t)a.R[g * sh.Mgp + ml] + (uint32_t)sh.K * ((uint32_t)coef * xb) +
                          (uint32_t)a.bias[m];
    const bool whole = sh.P % 4 == 0;  // then p + 3 < P and the rows are 16-byte aligned
    uint32_t v[4] = {rowc, rowc, rowc, rowc};
    for (int s = 0; s < a.nsplit; ++s) {
        const size_t z = (size_t)n * a.nsplit + s;
        const int32_t* src = a.part + (z * sh.M + m) * sh.P + p;
        const int32_t* ssrc = a.spart + (z * sh.G + g) * sh.P + p;
        if (whole) {
            const v4i t = *reinterpret_cast<const v4i*>(src);
            v4i st = {0, 0, 0, 0};
            if (XSUM) st = *reinterpret_cast<const v4i*>(ssrc);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] += (uint32_t)t[e] + (XSUM ? (uint32_t)coef * (uint32_t)st[e] : 0u);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (p + e < sh.P)
                    v[e] += (uint32_t)src[e] + (XSUM ? (uint32_t)coef * (uint32_t)ssrc[e] : 0u);
        }
    }
    const uint32_t word = requant4(v, a.ws[m], make_yquant(a));
    uint8_t* dst = a.y + ((size_t)n * sh.M + m) * sh.P + p;
    if (whole) {
        *reinterpret_cast<uint32_t*>(dst) = word;
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (p + e < sh.P) dst[e] = (uint8_t)(word >> (8 * e));
    }
}

// Packs w [M, Cg, kH, kW] into w^ rows [G * Mgp][Tp][Kc] (zeros past Cg,
// T and Mg) and R[row] = sum of the row's w^. One workgroup per row.
__global__ __launch_bounds__(256) void k_conv_pack_w(const uint8_t* __restrict__ w, ConvShape sh, int w_u8,
                                                     int8_t* __restrict__ wp, int32_t* __restrict__ R) {
    __shared__ int32_t part[256];
    const int row = blockIdx.x;
    const int g = row / sh.Mgp, ml = row - g * sh.Mgp;
    const bool mok = ml < sh.Mg;
    const int m = g * sh.Mg + ml;
    const int len = sh.Tp * sh.Kc;
    int32_t s = 0;
    for (int i = threadIdx.x; i < len; i += 256) {
        const int t = i / sh.Kc, c = i - t * sh.Kc;
        int v = 0;
        if (sh.vc) {
            // virtual tap t = kernel row kh, virtual channel c = 4 kw + input channel
            const int kw = c >> 2, ci = c & 3;
            if (mok && ci < sh.rCg && kw < sh.rKW && t < sh.T) {
                const uint32_t b = w[(((size_t)m * sh.rCg + ci) * sh.KH + t) * sh.rKW + kw];
                v = w_u8 ? (int)b - 128 : (int)(int8_t)b;
            }
        } else if (mok && c < sh.Cg && t < sh.T) {
            const uint32_t b = w[((size_t)m * sh.Cg + c) * sh.T + t];
            v = w_u8 ? (int)b - 128 : (int)(int8_t)b;
        }
        wp[wpos(row, t, c, sh.Tp, sh.Kc)] = (int8_t)v;
        s += v;
    }
    part[threadIdx.x] = s;
    __syncthreads();
    for (int k = 128; k > 0; k >>= 1) {
        if (threadIdx.x < k) part[threadIdx.x] += part[threadIdx.x + k];
        __syncthreads();
    }
    if (threadIdx.x == 0) R[row] = part[0];
}

// Per output channel: scale, zero point (as int) and bias, from one or M
// values.
__global__ __launch_bounds__(256) void k_conv_params(const float* __restrict__ w_scale,
                                                     const void* __restrict__ w_zp, int w_u8, int w_len,
                                                     const int32_t* __restrict__ bias, int M,
                                                     float* __restrict__ ws, int32_t* __restrict__ wz,
                                                     int32_t* __restrict__ bo) {
    const int m = blockIdx.x * 256 + threadIdx.x;
    if (m >= M) return;
    const int i = w_len == 1 ? 0 : m;
    ws[m] = w_scale[i];
    wz[m] = w_zp ? (w_u8 ? (int)((const uint8_t*)w_zp)[i] : (int)((const int8_t*)w_zp)[i]) : 0;
    bo[m] = bias ? bias[m] : 0;
}

bool is_8bit(dq_dtype t) { return t == DQ_I8 || t == DQ_U8; }

int round_up(int v, int m) { return (v + m - 1) / m * m; }

}  // namespace

struct dq_qconv_ctx {
    ConvShape sh{};
    dq_dtype x_type, w_type, y_type;
    int wm = 1;            // waves over output channels
    bool direct = false;   // few channels per group: k_qconv_direct
    bool dw = false;       // depthwise with a plane that fits LDS: k_qconv_dw
    int dw_lds = 0;        // its dynamic LDS bytes
    int ib = 2;            // 32-pixel MFMA rows per wave
    int patch_bytes = 0;
    bool has_w = false, xsum = false;
    int device = 0;
    int8_t* wp = nullptr;
    int32_t* R = nullptr;
    float* ws = nullptr;
    int32_t* wz = nullptr;
    int32_t* bias = nullptr;
    int32_t* part = nullptr;  // split partial sums, grown on demand by forward
    size_t part_bytes = 0;
    uint8_t* xb = nullptr;    // the prepared input, grown on demand by forward
    size_t xb_bytes = 0;
    int hx = 0;               // prepared rows an image and chunk
    std::string info;
};

namespace {

void free_ctx(dq_qconv_ctx* c) {
    if (!c) return;
    (void)hipFree(c->wp);
    (void)hipFree(c->R);
    (void)hipFree(c->ws);
    (void)hipFree(c->wz);
    (void)hipFree(c->bias);
    (void)hipFree(c->part);
    (void)hipFree(c->xb);
    delete c;
}

template <bool XSUM, int WM, int IB, bool SPLIT>
int set_lds(int bytes) {
    if (hipFuncSetAttribute((const void*)k_qconv<XSUM, WM, IB, SPLIT>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            bytes) != hipSuccess)
        DQ_FAIL(DQ_ERR_HIP, "hipFuncSetAttribute failed for the conv kernel");
    return DQ_OK;
}

// the LDS budget of the four kernels a context may launch
template <int WM>
int set_lds2(int bytes) {
    int rc = set_lds<true, WM, 2, false>(bytes);
    if (!rc) rc = set_lds<false, WM, 2, false>(bytes);
    if (!rc) rc = set_lds<true, WM, 2, true>(bytes);
    return rc ? rc : set_lds<false, WM, 2, true>(bytes);
}

}  // namespace

extern "C" int dq_qconv_init(dq_qconv_ctx** ctx, int64_t C, int64_t H, int64_t W, int64_t M, int64_t kH,
                             int64_t kW, const int64_t* strides, const int64_t* pads,
                             const int64_t* dilations, int64_t group, dq_dtype x_type, dq_dtype w_type,
                             dq_dtype y_type) {
    if (!ctx) DQ_FAIL(DQ_ERR_ARG, "ctx is NULL");
    *ctx = nullptr;
    if (!is_8bit(x_type) || !is_8bit(w_type) || !is_8bit(y_type))
        DQ_FAIL(DQ_ERR_TYPE, "x, w and y must be DQ_I8 or DQ_U8");
    const int64_t sh_ = strides ? strides[0] : 1, sw_ = strides ? strides[1] : 1;
    const int64_t pt = pads ? pads[0] : 0, pl = pads ? pads[1] : 0, pb = pads ? pads[2] : 0, pr = pads ? pads[3] : 0;
    const int64_t dh = dilations ? dilations[0] : 1, dw = dilations ? dilations[1] : 1;
    if (C < 1 || H < 1 || W < 1 || M < 1 || kH < 1 || kW < 1 || sh_ < 1 || sw_ < 1 || dh < 1 || dw < 1 ||
        pt < 0 || pl < 0 || pb < 0 || pr < 0 || group < 1)
        DQ_FAIL(DQ_ERR_ARG, "sizes, strides, dilations and group must be >= 1 and pads >= 0");
    if (C % group || M % group) DQ_FAIL(DQ_ERR_ARG, "group must divide C and M");
    const int64_t lim = 1 << 20;
    if (C > lim || H > lim || W > lim || M > lim || kH > 1024 || kW > 1024 || sh_ > 1024 || sw_ > 1024 ||
        dh > 1024 || dw > 1024 || pt > 1024 || pl > 1024 || pb > 1024 || pr > 1024)
        DQ_FAIL(DQ_ERR_RANGE, "a size or attribute beyond the kernel's range");
    const int64_t oH = (H + pt + pb - dh * (kH - 1) - 1) / sh_ + 1;
    const int64_t oW = (W + pl + pr - dw * (kW - 1) - 1) / sw_ + 1;
    if (H + pt + pb - dh * (kH - 1) - 1 < 0 || W + pl + pr - dw * (kW - 1) - 1 < 0 || oH < 1 || oW < 1)
        DQ_FAIL(DQ_ERR_ARG, "the kernel does not fit the padded input");
    const int64_t Cg = C / group, Mg = M / group;
    if (Cg * kH * kW > kKMax) DQ_FAIL(DQ_ERR_RANGE, "C / group * kH * kW exceeds %d (int32 sums)", kKMax);
    if (kH * kW > kTapMax - kTapGroup) DQ_FAIL(DQ_ERR_RANGE, "kH * kW exceeds %d", kTapMax - kTapGroup);
    if (oH * oW > (1LL << 30)) DQ_FAIL(DQ_ERR_RANGE, "output image too large");
    dq_qconv_ctx* c = new dq_qconv_ctx();
    ConvShape& s = c->sh;
    s.C = (int)C; s.H = (int)H; s.W = (int)W; s.M = (int)M; s.KH = (int)kH; s.KW = (int)kW;
    s.sh = (int)sh_; s.sw = (int)sw_; s.pt = (int)pt; s.pl = (int)pl; s.dh = (int)dh; s.dw = (int)dw;
    s.G = (int)group; s.Cg = (int)Cg; s.Mg = (int)Mg; s.OH = (int)oH; s.OW = (int)oW; s.P = (int)(oH * oW);
    s.T = s.KH * s.KW;
    s.Tp = round_up(s.T, kTapGroup);
    s.Kc = round_up(s.Cg, kKC);
    s.K = (int)(Cg * kH * kW);
    // prepared columns: input columns -pl .. the last one a tap reads
    s.cpad = s.pl;
    s.ncol = (s.OW - 1) * s.sw + (s.KW - 1) * s.dw + 1;
    s.ow_div = dq::make_fastdiv((uint32_t)s.OW);
    // waves over channels: 1 (64 channels x 256 pixels) while a group has
    // at most 64 channels, else 2 (128 x 128); the patch of the largest
    // pixel run must fit the LDS budget
    c->direct = Cg <= 4 && Mg <= 4;
    s.hp = (s.OH - 1) * s.sh + (s.KH - 1) * s.dh + 1;
    s.wp = round_up((s.OW - 1) * s.sw + (s.KW - 1) * s.dw + 1, 2);  // even: 4-byte aligned rows of int16
    s.spr = (s.OW + 3) / 4;
    s.spr_div = dq::make_fastdiv((uint32_t)s.spr);
    s.w_div = dq::make_fastdiv((uint32_t)s.W);
    s.wq_div = dq::make_fastdiv((uint32_t)std::max(s.W / 4, 1));
    if (Cg == 1 && Mg == 1) {
        const long long nel = (long long)s.hp * s.wp + 3LL * s.sw + 1;
        const long long bytes = (nel + 1) / 2 * 4;
        if (bytes <= kDwLdsMax) {
            c->dw = true;
            c->dw_lds = (int)bytes;
        }
    }
    s.vc = 0;
    if (!c->direct && !c->dw && Cg <= 4 && kW <= 8 && kW > 1) {
        // the virtual convolution (see ConvShape): kW times fewer MFMAs than
        // 32-channel chunks over every tap, and a patch of output columns
        s.vc = 1;
        s.rW = s.W; s.rsw = s.sw; s.rpl = s.pl; s.rdw = s.dw; s.rCg = s.Cg; s.rKW = s.KW;
        s.W = s.OW; s.KW = 1; s.sw = 1; s.pl = 0; s.dw = 1; s.Cg = kKC;
        s.T = s.KH;
        s.Tp = round_up(s.T, kTapGroup);
        s.Kc = kKC;
        s.cpad = 0;
        s.ncol = s.OW;
    }
    c->wm = Mg <= 64 ? 1 : 2;
    // two 32-pixel MFMA rows a wave (one row gave more workgroups but was
    // slower on every layer measured but the smallest)
    c->ib = 2;
    c->hx = (s.OH - 1) * s.sh + (s.KH - 1) * s.dh + 1;
    for (;;) {
        // two patch buffers of the largest patch a workgroup copies
        const int PT = 32 * c->ib * (4 / c->wm);
        const int rows = std::min(s.OH, (PT - 1) / s.OW + 2);
        const int nr = (rows - 1) * s.sh + (s.KH - 1) * s.dh + 1;
        const long long bytes = 2 * (((long long)nr * s.ncol * kKC + 1023) / 1024 * 1024);
        if (bytes <= kPatchMax || c->direct || c->dw) {
            c->patch_bytes = (int)std::min<long long>(bytes, kPatchMax);
            break;
        }
        if (c->wm == 2) {
            free_ctx(c);
            DQ_FAIL(DQ_ERR_RANGE, "input patch of %lld bytes exceeds the LDS budget", bytes);
        }
        c->wm = 2;
    }
    s.Mgp = round_up(s.Mg, 64 * c->wm);
    s.mtiles = s.Mgp / (64 * c->wm);
    if ((long long)s.G * s.mtiles > 65535 || (c->direct && s.M > 65535)) {
        free_ctx(c);
        DQ_FAIL(DQ_ERR_RANGE, "too many channel tiles for one launch");
    }
    c->x_type = x_type;
    c->w_type = w_type;
    c->y_type = y_type;
    // the kernels' dynamic-LDS limit is one setting per kernel and device,
    // shared by every context: raise it to the most any context may use
    // (not this one's patch), so a later context with smaller patches
    // cannot lower it under an earlier one's launches
    const int rc = c->wm == 1 ? set_lds2<1>(kPatchMax) : set_lds2<2>(kPatchMax);
    if (rc) {
        free_ctx(c);
        return rc;
    }
    (void)hipGetDevice(&c->device);
    const size_t rows = (size_t)s.G * s.Mgp;
    if (hipMalloc(&c->wp, rows * s.Tp * s.Kc) != hipSuccess || hipMalloc(&c->R, rows * 4) != hipSuccess ||
        hipMalloc(&c->ws, (size_t)s.M * 4) != hipSuccess || hipMalloc(&c->wz, (size_t)s.M * 4) != hipSuccess ||
        hipMalloc(&c->bias, (size_t)s.M * 4) != hipSuccess) {
        free_ctx(c);
        DQ_FAIL(DQ_ERR_ALLOC, "device allocation for the packed weights failed");
    }
    char buf[256];
    if (c->dw)
        snprintf(buf, sizeof buf, "gfx950 qconv depthwise: a plane (%d x %d, padded) a workgroup in LDS, four outputs a lane, %d taps",
                 s.hp, s.wp, s.T);
    else if (c->direct)
        snprintf(buf, sizeof buf, "gfx950 qconv direct: one output pixel a lane, %d taps x %d channels", s.T, s.Cg);
    else
        snprintf(buf, sizeof buf,
                 "gfx950 qconv implicit GEMM mfma_i32_32x32x32_i8: %d ch x %d px per workgroup, patch %d B "
                 "(%d x %d x 32)%s, K = %d",
                 64 * c->wm, 32 * c->ib * (4 / c->wm), c->patch_bytes, c->patch_bytes / (s.ncol * kKC), s.ncol,
                 s.vc ? ", virtual channels (kernel column, input channel)" : "", s.K);
    c->info = buf;
    *ctx = c;
    return DQ_OK;
}

extern "C" int dq_qconv_output_shape(const dq_qconv_ctx* ctx, int64_t* oH, int64_t* oW) {
    if (!ctx) DQ_FAIL(DQ_ERR_STATE, "no context");
    if (oH) *oH = ctx->sh.OH;
    if (oW) *oW = ctx->sh.OW;
    return DQ_OK;
}

extern "C" int dq_qconv_set_w(dq_qconv_ctx* ctx, const void* w, const float* w_scale, const void* w_zero_point,
                              int64_t w_len, const int32_t* bias, void* stream) {
    if (!ctx) DQ_FAIL(DQ_ERR_STATE, "no context");
    const ConvShape& s = ctx->sh;
    if (!w || !w_scale) DQ_FAIL(DQ_ERR_ARG, "w and w_scale must not be NULL");
    if (w_len != 1 && w_len != s.M) DQ_FAIL(DQ_ERR_ARG, "w_len must be 1 or M");
    int dev = 0;
    (void)hipGetDevice(&dev);
    if (dev != ctx->device) DQ_FAIL(DQ_ERR_STATE, "the context belongs to another device");
    const hipStream_t st = (hipStream_t)stream;
    const int wu8 = ctx->w_type == DQ_U8;
    hipLaunchKernelGGL(k_conv_pack_w, dim3((unsigned)(s.G * s.Mgp)), dim3(256), 0, st, (const uint8_t*)w, s, wu8,
                       ctx->wp, ctx->R);
    DQ_LAUNCH_CHECK("conv weight packing");
    hipLaunchKernelGGL(k_conv_params, dim3((unsigned)((s.M + 255) / 256)), dim3(256), 0, st, w_scale,
                       w_zero_point, wu8, (int)w_len, bias, s.M, ctx->ws, ctx->wz, ctx->bias);
    DQ_LAUNCH_CHECK("conv parameters");
    // S[p] is needed when some w zero point differs from w's shift
    std::vector<int32_t> wz(s.M);
    DQ_HIP_CHECK(hipMemcpyAsync(wz.data(), ctx->wz, (size_t)s.M * 4, hipMemcpyDeviceToHost, st));
    DQ_HIP_CHECK(hipStreamSynchronize(st));
    const int kA = wu8 ? 128 : 0;
    ctx->xsum = false;
    for (int v : wz) ctx->xsum = ctx->xsum || v != kA;
    ctx->has_w = true;
    return DQ_OK;
}

extern "C" int dq_qconv_forward(dq_qconv_ctx* ctx, const void* x, int64_t N, const float* x_scale,
                                const void* x_zero_point, const float* y_scale, const void* y_zero_point,
                                void* y, void* stream) {
    if (!ctx) DQ_FAIL(DQ_ERR_STATE, "no context");
    if (!ctx->has_w) DQ_FAIL(DQ_ERR_STATE, "dq_qconv_set_w has not been called");
    const ConvShape& s = ctx->sh;
    if (N < 0) DQ_FAIL(DQ_ERR_ARG, "N must be >= 0");
    if (N == 0) return DQ_OK;
    if (N > 65535) DQ_FAIL(DQ_ERR_RANGE, "N exceeds 65535");
    if (!x || !x_scale || !y_scale || !y) DQ_FAIL(DQ_ERR_ARG, "x, y and the scales must not be NULL");
    int dev = 0;
    (void)hipGetDevice(&dev);
    if (dev != ctx->device) DQ_FAIL(DQ_ERR_STATE, "the context belongs to another device");
    ConvArgs a{};
    a.x = (const uint8_t*)x;
    a.wp = ctx->wp;
    a.R = ctx->R;
    a.ws = ctx->ws;
    a.wz = ctx->wz;
    a.bias = ctx->bias;
    a.x_scale = x_scale;
    a.x_zp = x_zero_point;
    a.y_scale = y_scale;
    a.y_zp = y_zero_point;
    a.y = (uint8_t*)y;
    a.x_u8 = ctx->x_type == DQ_U8;
    a.y_u8 = ctx->y_type == DQ_U8;
    a.xflip = a.x_u8 ? 0x80808080u : 0u;
    a.y_lo = a.y_u8 ? 0 : -128;
    a.y_hi = a.y_u8 ? 255 : 127;
    a.kA = ctx->w_type == DQ_U8 ? 128 : 0;
    a.kB = a.x_u8 ? 128 : 0;
    a.vecy = s.P % 16 == 0 && (uintptr_t)y % 16 == 0;
    a.vecy4 = s.OW % 4 == 0 && (uintptr_t)y % 4 == 0;
    a.vecx_plane = ((long long)s.H * s.W) % 4 == 0 && (uintptr_t)x % 4 == 0;
    const hipStream_t st = (hipStream_t)stream;
    if (ctx->dw) {
        const dim3 grid((unsigned)s.M, (unsigned)N);
        const bool ks3 = s.KH == 3 && s.KW == 3 && s.sh == 1 && s.sw == 1 && s.dh == 1 && s.dw == 1;
        if (ks3) hipLaunchKernelGGL(k_qconv_dw<true>, grid, dim3(256), (size_t)ctx->dw_lds, st, s, a);
        else hipLaunchKernelGGL(k_qconv_dw<false>, grid, dim3(256), (size_t)ctx->dw_lds, st, s, a);
        DQ_LAUNCH_CHECK("qconv depthwise");
        return DQ_OK;
    }
    if (ctx->direct) {
        const dim3 grid((unsigned)((s.P + 255) / 256), (unsigned)s.M, (unsigned)N);
        hipLaunchKernelGGL(k_qconv_direct, grid, dim3(256), 0, st, s, a);
        DQ_LAUNCH_CHECK("qconv direct");
        return DQ_OK;
    }
    const int PT = 32 * ctx->ib * (4 / ctx->wm);
    const long long ptiles = (s.P + PT - 1) / PT, gy = (long long)s.G * s.mtiles;
    const size_t lds = (size_t)ctx->patch_bytes;
    // the prepared input (k_conv_prep_x), 1 KiB of slack for the last copy
    const int nch = s.Kc / kKC;
    if ((long long)N * s.G * nch > 65535) DQ_FAIL(DQ_ERR_RANGE, "N * group * channel chunks exceeds 65535");
    a.xb_rs = (size_t)s.ncol * kKC;
    a.xb_cs = (size_t)ctx->hx * a.xb_rs;
    a.pbuf = ctx->patch_bytes / 2;
    const size_t xb_need = (size_t)N * s.G * nch * a.xb_cs + 1024;
    if (xb_need > ctx->xb_bytes) {
        // the old buffer may still be in use by this stream's earlier work
        DQ_HIP_CHECK(hipStreamSynchronize(st));
        (void)hipFree(ctx->xb);
        ctx->xb = nullptr;
        ctx->xb_bytes = 0;
        if (hipMalloc(&ctx->xb, xb_need) != hipSuccess) DQ_FAIL(DQ_ERR_ALLOC, "device allocation of the prepared input failed");
        ctx->xb_bytes = xb_need;
    }
    a.xb = ctx->xb;
    if (!s.vc && s.W % 4 == 0 && s.W <= kPrepMaxW && (uintptr_t)x % 4 == 0) {
        const dim3 pgrid((unsigned)((ctx->hx + kPrepRows - 1) / kPrepRows), (unsigned)(N * s.G * nch));
        hipLaunchKernelGGL(k_conv_prep_t, pgrid, dim3(256), (size_t)kKC * kPrepRows * s.W, st, s, a, ctx->hx,
                           ctx->xb);
        DQ_LAUNCH_CHECK("qconv input preparation");
    } else {
        const dim3 pgrid((unsigned)((s.ncol + 63) / 64), (unsigned)((ctx->hx + 3) / 4), (unsigned)(N * s.G * nch));
        hipLaunchKernelGGL(k_conv_prep_x, pgrid, dim3(256), 0, st, s, a, ctx->hx, ctx->xb);
        DQ_LAUNCH_CHECK("qconv input preparation");
    }
    // Too few workgroups for the chip (deep layers: few pixels, many
    // channels): split the chunks of the reduction over workgroups, leave
    // int32 partial sums and requantize them in k_qconv_reduce.
    const int chunks = s.Kc / kKC;
    const long long wgs = ptiles * gy * N;
    int nsplit = 1;
    if (wgs < kSplitBelow && chunks >= 2) {
        nsplit = (int)std::min<long long>(chunks, (kSplitBelow + wgs - 1) / wgs);
        nsplit = (int)std::min<long long>(nsplit, 65535 / N);
    }
    if (nsplit > 1) {
        a.cps = (chunks + nsplit - 1) / nsplit;
        a.nsplit = (chunks + a.cps - 1) / a.cps;
        const size_t need = (size_t)N * a.nsplit * ((size_t)s.M + (ctx->xsum ? s.G : 0)) * s.P * 4;
        if (need > ctx->part_bytes) {
            // the old buffer may still be in use by this stream's earlier work
            DQ_HIP_CHECK(hipStreamSynchronize(st));
            (void)hipFree(ctx->part);
            ctx->part = nullptr;
            ctx->part_bytes = 0;
            if (hipMalloc(&ctx->part, need) != hipSuccess) DQ_FAIL(DQ_ERR_ALLOC, "device allocation of the split sums failed");
            ctx->part_bytes = need;
        }
        a.part = ctx->part;
        a.spart = ctx->part + (size_t)N * a.nsplit * s.M * s.P;
        const dim3 grid((unsigned)ptiles, (unsigned)gy, (unsigned)(N * a.nsplit));
#define DQ_CONV(XS, W_) hipLaunchKernelGGL((k_qconv<XS, W_, 2, true>), grid, dim3(kThreads), lds, st, s, a)
        if (ctx->wm == 1) {
            if (ctx->xsum) DQ_CONV(true, 1);
            else DQ_CONV(false, 1);
        } else {
            if (ctx->xsum) DQ_CONV(true, 2);
            else DQ_CONV(false, 2);
        }
#undef DQ_CONV
        DQ_LAUNCH_CHECK("qconv split");
        const dim3 rgrid((unsigned)((s.P + 1023) / 1024), (unsigned)s.M, (unsigned)N);
        if (ctx->xsum) hipLaunchKernelGGL(k_qconv_reduce<true>, rgrid, dim3(256), 0, st, s, a);
        else hipLaunchKernelGGL(k_qconv_reduce<false>, rgrid, dim3(256), 0, st, s, a);
        DQ_LAUNCH_CHECK("qconv split reduction");
        return DQ_OK;
    }
    const dim3 grid((unsigned)ptiles, (unsigned)gy, (unsigned)N);
#define DQ_CONV(XS, W_) hipLaunchKernelGGL((k_qconv<XS, W_, 2, false>), grid, dim3(kThreads), lds, st, s, a)
    if (ctx->wm == 1) {
        if (ctx->xsum) DQ_CONV(true, 1);
        else DQ_CONV(false, 1);
    } else {
        if (ctx->xsum) DQ_CONV(true, 2);
        else DQ_CONV(false, 2);
    }
#undef DQ_CONV
    DQ_LAUNCH_CHECK("qconv");
    return DQ_OK;
}

extern "C" const char* dq_qconv_info(const dq_qconv_ctx* ctx) { return ctx ? ctx->info.c_str() : nullptr; }

extern "C" void dq_qconv_release(dq_qconv_ctx* ctx) { free_ctx(ctx); }
