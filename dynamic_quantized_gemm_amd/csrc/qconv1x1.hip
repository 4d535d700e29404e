// qconv1x1.hip -- requantizing 1x1 QLinearConv on gfx950 matrix cores.
//
// ONNX "QLinearConv" (opset 10), description and inputs: x and w are 8-bit
// tensors with scales and zero points (w per tensor or per output channel),
// the optional bias is int32 with scale x_scale * w_scale and zero point 0,
// and y is requantized with y_scale / y_zero_point. For a 1x1 kernel with
// stride 1, no padding and one group, image n is a matrix product:
//   acc[m,p] = sum_c (w[m,c] - w_zp[m]) * (x[n,c,p] - x_zp) + bias[m]
//   real     = ((float)acc * x_scale) * w_scale[m]
//   y[n,m,p] = saturate(rne(real / y_scale) + y_zp)
// (requantization read as dequantize, then QuantizeLinear: IEEE quotient,
// ties to even, saturation to the 8-bit range of y).
//
// The int8 MFMA multiplies signed by signed. With shifts a = 128 for a uint8
// w (0 for int8) and b = 128 for a uint8 x (0 for int8), the operands
// w^ = w - a and x^ = x - b are int8 and the sum splits exactly:
//   acc = sum_c w^ x^ + (b - x_zp) * R[m] + (a - w_zp[m]) * S[p]
//         + C * (a - w_zp[m]) * (b - x_zp) + bias[m]
// with R[m] = sum_c w^[m,c] (from the weight fragments each lane holds) and
// S[p] = sum_c x^[c,p] (one extra MFMA against an all-ones operand, only when
// some a - w_zp[m] can be non-zero). The MFMA part is bounded by
// C * 128 * 128 < 2^31 for C <= 32768, and the corrections are added in
// wrapping 32-bit arithmetic, which yields acc exactly whenever acc fits in
// int32.
//
// Kernel k_qconv1x1: a workgroup of 4 waves computes 256 output channels x 64
// pixels of one image, each wave 64 channels x 64 pixels (2 x 2 blocks of
// 32x32). Per chunk of 256 input channels, every lane keeps its weight
// fragments in registers: w is [M, C] row-major, so a 32-channel run of one
// output channel is already the k-contiguous MFMA operand and is loaded as
// is. The image tile x[c, p] (pixels contiguous) is loaded with 4-byte loads
// along pixels, transposed 4x4 bytes in registers and written to LDS in
// fragment order (pixel rows, 16 channels per lane slot), from where each
// wave reads its operands with ds_read_b128. Each lane's accumulators hold
// one output channel (lane % 32) and, in accumulators 4g..4g+3, four
// consecutive pixels, so the requantized codes pack into 32-bit words; they
// are staged in LDS per wave and stored as 16-byte row segments.
#include "dq_device.h"
#include "dq_kernels.h"

namespace {

constexpr int kP = 64;        // pixels per tile
constexpr int kMT = 256;      // output channels per tile (4 waves x 64)
constexpr int kKC = 256;      // input channels per chunk
constexpr int kYPitch = 80;   // LDS bytes per staged output row (64 + 16)
constexpr int kThreads = 256;

__device__ __forceinline__ int load_zp(const uint8_t* zp, size_t i, bool u8) {
    if (!zp) return 0;
    return u8 ? (int)zp[i] : (int)(int8_t)zp[i];
}

// Byte i of each of d0..d3, as one word (d0 in the low byte).
__device__ __forceinline__ uint32_t gather_byte(uint32_t d0, uint32_t d1, uint32_t d2, uint32_t d3,
                                                int i) {
    const int s = 8 * i;
    return ((d0 >> s) & 0xffu) | (((d1 >> s) & 0xffu) << 8) | (((d2 >> s) & 0xffu) << 16) |
           (((d3 >> s) & 0xffu) << 24);
}

// Four consecutive bytes x[row, p .. p+3] as a word; bytes at p >= HW read as
// `pad`. VEC: HW % 4 == 0 and x 4-byte aligned, so the word is whole or out.
template <bool VEC>
__device__ __forceinline__ uint32_t load_x4(const uint8_t* row, int p, int HW, uint32_t pad) {
    if (VEC) return p < HW ? *reinterpret_cast<const uint32_t*>(row + p) : pad;
    uint32_t v = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t b = p + e < HW ? (uint32_t)row[p + e] : ((pad >> (8 * e)) & 0xffu);
        v |= b << (8 * e);
    }
    return v;
}

template <bool XU8, bool WU8, bool YU8, bool XSUM, bool VEC>
__global__ __launch_bounds__(kThreads) void k_qconv1x1(
    const uint8_t* __restrict__ x, const uint8_t* __restrict__ w, int C, int HW, int M,
    const float* __restrict__ x_scale_p, const uint8_t* __restrict__ x_zp_p,
    const float* __restrict__ w_scale, const uint8_t* __restrict__ w_zp, int w_per_channel,
    const float* __restrict__ y_scale_p, const uint8_t* __restrict__ y_zp_p,
    const int32_t* __restrict__ bias, int wvec, uint8_t* __restrict__ y) {
    __shared__ __attribute__((aligned(16))) int8_t xs[(kP / 32) * (kKC / 32) * 1024];
    __shared__ __attribute__((aligned(16))) uint8_t ys[kMT * kYPitch];

    constexpr uint32_t kXor = 0x80808080u;
    constexpr int kA = WU8 ? 128 : 0;  // shift of w
    constexpr int kB = XU8 ? 128 : 0;  // shift of x
    // raw byte that becomes x^ = 0 after the shift (padding channels / pixels)
    constexpr uint32_t kXPad = XU8 ? kXor : 0u;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int p0 = blockIdx.x * kP;
    const int mw0 = blockIdx.y * kMT + 64 * wave;  // first output channel of this wave
    const size_t n = blockIdx.z;
    const uint8_t* xn = x + n * (size_t)C * HW;

    typedef dq::v4i v4i;
    dq::v16i acc[2][2];  // [pixel block][channel block]
    dq::v16i sacc[2];    // column sums of x^ per pixel block (XSUM)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            acc[i][0][r] = 0;
            acc[i][1][r] = 0;
            sacc[i][r] = 0;
        }
    }
    int32_t rsum[2] = {0, 0};  // this lane's share of R for its two channels
    const v4i ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};

    for (int ch0 = 0; ch0 < C; ch0 += kKC) {
        // weight fragments: channel m = mw0 + 32 jb + lane % 32, input
        // channels ch0 + 32 kk + 16 (lane / 32) .. + 15
        v4i wf[2][kKC / 32];
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            const int m = mw0 + 32 * jb + (lane & 31);
            const uint8_t* wrow = w + (size_t)(m < M ? m : 0) * C;
#pragma unroll
            for (int kk = 0; kk < kKC / 32; ++kk) {
                const int c = ch0 + 32 * kk + 16 * (lane >> 5);
                v4i v = {0, 0, 0, 0};
                if (m < M && c < C) {
                    if (wvec) {
                        v = *reinterpret_cast<const v4i*>(wrow + c);
                        if (WU8) {
#pragma unroll
                            for (int e = 0; e < 4; ++e) v[e] ^= (int)kXor;
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            const uint32_t b = c + e < C ? (uint32_t)wrow[c + e] ^ (WU8 ? 0x80u : 0u) : 0u;
                            v[e >> 2] |= (int)(b << (8 * (e & 3)));
                        }
                    }
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) rsum[jb] = __builtin_amdgcn_sdot4(v[e], 0x01010101, rsum[jb], false);
                wf[jb][kk] = v;
            }
        }

        // the image tile: lane handles 4 pixels (p0 + 4 (tid % 16) ..) of
        // 16 input channels (ch0 + 16 (tid / 16) ..)
        __syncthreads();  // the previous chunk's operand reads are done
        {
            const int pq = tid & 15, cg = tid >> 4;
            const int p = p0 + 4 * pq;
            uint32_t d[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int c = ch0 + 16 * cg + j;
                d[j] = c < C ? load_x4<VEC>(xn + (size_t)c * HW, p, HW, kXPad) : kXPad;
                if (XU8) d[j] ^= kXor;
            }
            const int kb = (16 * cg) >> 5, h = cg & 1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * pq + i;  // pixel row of the tile
                v4i slot;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    slot[q] = (int)gather_byte(d[4 * q], d[4 * q + 1], d[4 * q + 2], d[4 * q + 3], i);
                *reinterpret_cast<v4i*>(&xs[((r >> 5) * (kKC / 32) + kb) * 1024 + ((r & 31) + 32 * h) * 16]) = slot;
            }
        }
        __syncthreads();

#pragma unroll
        for (int kk = 0; kk < kKC / 32; ++kk) {
            const v4i xf0 = *reinterpret_cast<const v4i*>(&xs[(0 * (kKC / 32) + kk) * 1024 + lane * 16]);
            const v4i xf1 = *reinterpret_cast<const v4i*>(&xs[(1 * (kKC / 32) + kk) * 1024 + lane * 16]);
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
                acc[0][jb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xf0, wf[jb][kk], acc[0][jb], 0, 0, 0);
                acc[1][jb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xf1, wf[jb][kk], acc[1][jb], 0, 0, 0);
            }
            if (XSUM) {
                sacc[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xf0, ones, sacc[0], 0, 0, 0);
                sacc[1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xf1, ones, sacc[1], 0, 0, 0);
            }
        }
    }

    // ---- requantizing epilogue
    const float x_scale = x_scale_p[0];
    const int x_zp = load_zp(x_zp_p, 0, XU8);
    const dq::QDiv yd = dq::make_qdiv(y_scale_p[0]);
    const int y_zp = load_zp(y_zp_p, 0, YU8);
    constexpr int lo = YU8 ? 0 : -128, hi = YU8 ? 255 : 127;
    uint8_t* ysw = ys + 64 * wave * kYPitch;
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
        const int m = mw0 + 32 * jb + (lane & 31);
        const bool mok = m < M;
        const int wi = w_per_channel ? m : 0;
        const int32_t R = rsum[jb] + __shfl_xor(rsum[jb], 32);
        const int coef = kA - (mok ? load_zp(w_zp, wi, WU8) : 0);
        const float ws = mok ? w_scale[wi] : 0.0f;
        const uint32_t rowc = (uint32_t)(kB - x_zp) * (uint32_t)R +
                              (uint32_t)C * ((uint32_t)coef * (uint32_t)(kB - x_zp)) +
                              (uint32_t)(mok && bias ? bias[m] : 0);
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                uint32_t word = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * g + e;
                    uint32_t v = (uint32_t)acc[ib][jb][r] + rowc;
                    if (XSUM) v += (uint32_t)coef * (uint32_t)sacc[ib][r];
                    float real = (float)(int32_t)v * x_scale;
                    real = real * ws;
                    const int code = dq::sat_add(dq::rne(dq::qdiv(real, yd)), y_zp, lo, hi);
                    word |= ((uint32_t)code & 0xffu) << (8 * e);
                }
                const int pp = 32 * ib + 8 * g + 4 * (lane >> 5);  // pixel of the tile
                *reinterpret_cast<uint32_t*>(&ysw[(32 * jb + (lane & 31)) * kYPitch + pp]) = word;
            }
        }
    }
    // the wave's 64 staged rows back as 16-byte segments (LDS operations of
    // one wave complete in order: no barrier)
    dq::wave_lds_fence();
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int u = lane + 64 * it;
        const int rr = u >> 2, q = u & 3;
        const int m = mw0 + rr, p = p0 + 16 * q;
        if (m < M && p < HW) {
            const v4i v = *reinterpret_cast<const v4i*>(&ysw[rr * kYPitch + 16 * q]);
            uint8_t* dst = y + (n * M + m) * (size_t)HW + p;
            if (VEC) {
                *reinterpret_cast<v4i*>(dst) = v;
            } else {
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    if (p + e < HW) dst[e] = (uint8_t)((uint32_t)v[e >> 2] >> (8 * (e & 3)));
            }
        }
    }
}

// ---- persistent variant: M <= 256 and C <= 256 (the weights of a wave fit in
// its registers for the whole launch).
//
// Work items are (image, 32-pixel tile). A workgroup loads its weight
// fragments once, then walks items g, g + G, ...: the raw image bytes of
// the next item are requested before the current item's MFMAs and
// requantization run, the tile is transposed into one of two LDS buffers
// (one barrier per item: the buffer written for item i + 2 was last read
// before every wave passed item i + 1's barrier), and each wave finishes 64
// output channels x 32 pixels. The requantization rounds as the other
// quantizers do: a corrected quotient clamped to +-2^22, 1.5 * 2^23 added for
// round-half-even, a median clamp and a bytewise zero-point add.
constexpr int kPP = 32;          // pixels per item
constexpr int kPersistentGroups = 512;
constexpr int kYPitchP = 48;     // LDS bytes per staged output row (32 + 16)
constexpr int kWPitch = 272;     // LDS bytes per staged weight row (256 + 16)

// The raw bytes of an item: lane handles pixels p .. p+3 (p = p0 + 4 (tid % 8))
// of channels 8 (tid / 8) .. + 7 (pad: bytes that become x^ = 0).
// FULL (every pixel in range, 4-byte loads): every lane loads from a clamped
// channel and the caller replaces channels past C by the pad when it uses
// the words, so the loads are unconditional and nothing waits for them
// before their use.
template <bool VEC, bool FULL>
__device__ __forceinline__ void load_item(const uint8_t* __restrict__ xn, int C, int HW, int p, int cg,
                                          uint32_t pad, uint32_t (&d)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int c = 8 * cg + j;
        if (FULL) {
            // raw word; channels past C are replaced by the pad at use
            d[j] = *reinterpret_cast<const uint32_t*>(xn + (size_t)(c < C ? c : C - 1) * HW + p);
        } else {
            d[j] = c < C ? load_x4<VEC>(xn + (size_t)c * HW, p, HW, pad) : pad;
        }
    }
}

// The wave's staged 64 rows x 32 pixels of one item back to y as 16-byte
// segments (lane handles two).
template <bool VEC, bool FULL>
__device__ __forceinline__ void store_staged(const uint8_t* ysw, uint8_t* __restrict__ y, int n, int p0,
                                             int mw0, int M, int HW, int lane) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int u = lane + 64 * k;
        const int rr = u >> 1, q = u & 1;
        const int m = mw0 + rr, p = p0 + 16 * q;
        if (FULL || (m < M && p < HW)) {
            const dq::v4i v = *reinterpret_cast<const dq::v4i*>(&ysw[rr * kYPitchP + 16 * q]);
            uint8_t* dst = y + ((size_t)n * M + m) * (size_t)HW + p;
            if (VEC || FULL) {
                *reinterpret_cast<dq::v4i*>(dst) = v;
            } else {
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    if (p + e < HW) dst[e] = (uint8_t)((uint32_t)v[e >> 2] >> (8 * (e & 3)));
            }
        }
    }
}

template <bool XU8, bool WU8, bool YU8, bool XSUM, bool VEC, bool FULL, bool WCOAL>
__global__ __launch_bounds__(kThreads) void k_qconv1x1_p(
    const uint8_t* __restrict__ x, const uint8_t* __restrict__ w, int C, int HW, int M,
    const float* __restrict__ x_scale_p, const uint8_t* __restrict__ x_zp_p,
    const float* __restrict__ w_scale, const uint8_t* __restrict__ w_zp, int w_per_channel,
    const float* __restrict__ y_scale_p, const uint8_t* __restrict__ y_zp_p,
    const int32_t* __restrict__ bias, int wvec, int nitems, int tiles, int per_xcd,
    uint8_t* __restrict__ y) {
    __shared__ __attribute__((aligned(16))) int8_t xs0[(kKC / 32) * 1024];
    __shared__ __attribute__((aligned(16))) int8_t xs1[(kKC / 32) * 1024];
    __shared__ __attribute__((aligned(16))) uint8_t ys[kMT * kYPitchP];
    // weight staging (WCOAL): each wave's 32-row half of its 64 rows at a
    // time, rows kWPitch bytes apart (256 + 16: the fragment reads of 16
    // rows at one column then fall on 16 distinct 4-bank groups)
    __shared__ __attribute__((aligned(16))) int8_t wst[WCOAL ? 4 * 32 * kWPitch : 16];

    constexpr uint32_t kXor = 0x80808080u;
    constexpr int kA = WU8 ? 128 : 0;
    constexpr int kB = XU8 ? 128 : 0;
    constexpr uint32_t kXPad = XU8 ? kXor : 0u;
    constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
    constexpr float kBig = 4194304.0f;     // 2^22
    typedef dq::v4i v4i;

    // XCD-aware item order: workgroups go round robin over the 8 XCDs, so
    // XCD (blockIdx % 8) owns the item range [xcd * per_xcd, ...), and its
    // workgroups walk that range with a stride of their count. Consecutive
    // workgroups of an XCD then hold the four 32-pixel tiles of one 128-byte
    // line of x at the same time and share its fetch in the XCD's L2.
    const int xcd = blockIdx.x % 8, local = blockIdx.x / 8, stride = gridDim.x / 8;
    const int first = xcd * per_xcd;
    const int end = min(first + per_xcd, nitems);
    int item = first + local;
    if (item >= end) return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int mw0 = 64 * wave;

    // every load that does not depend on another is issued first: the first
    // item's image bytes, the per-tensor and per-channel parameters, then the
    // weights, so their latencies overlap
    const int pq = tid & 7, cg = tid >> 3;
    uint32_t d[8];
    int prev_n = 0, prev_p0 = 0;
    {
        const int n = item / tiles, p0 = (item - n * tiles) * kPP;
        load_item<VEC, FULL>(x + (size_t)n * C * HW, C, HW, p0 + 4 * pq, cg, kXPad, d);
    }
    const float x_scale = x_scale_p[0];
    const float y_scale = y_scale_p[0];
    const int x_zp = load_zp(x_zp_p, 0, XU8);
    const int y_zp = load_zp(y_zp_p, 0, YU8);
    int wzp[2], bia[2];
    float wsc[2];
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
        const int m = mw0 + 32 * jb + (lane & 31);
        const bool mok = m < M;
        const int wi = w_per_channel ? m : 0;
        wzp[jb] = mok ? load_zp(w_zp, wi, WU8) : 0;
        wsc[jb] = mok ? w_scale[wi] : 0.0f;
        bia[jb] = mok && bias ? bias[m] : 0;
    }

    // weight fragments of the wave (channels mw0 + 32 jb + lane % 32), once
    v4i wf[2][kKC / 32];
    int32_t rsum[2] = {0, 0};
    if (WCOAL) {
        // all 256 input channels of all 64 rows exist (C == kKC, M == kMT):
        // the wave's rows are 16 KiB of consecutive bytes, read as whole
        // 1 KiB pieces per instruction (lane l: row 4 i + l / 16, bytes
        // 16 (l % 16) ..), staged in LDS per 32-row half and read back in
        // fragment order (row l % 32, bytes 32 kk + 16 (l / 32) ..)
        int8_t* stw = wst + wave * 32 * kWPitch;
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            v4i raw[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                raw[i] = *reinterpret_cast<const v4i*>(w + (size_t)(mw0 + 32 * jb) * kKC + 1024 * i + 16 * lane);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                *reinterpret_cast<v4i*>(stw + (4 * i + (lane >> 4)) * kWPitch + 16 * (lane & 15)) = raw[i];
            dq::wave_lds_fence();
#pragma unroll
            for (int kk = 0; kk < kKC / 32; ++kk) {
                v4i v = *reinterpret_cast<const v4i*>(stw + (lane & 31) * kWPitch + 32 * kk + 16 * (lane >> 5));
                if (WU8) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] ^= (int)kXor;
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) rsum[jb] = __builtin_amdgcn_sdot4(v[e], 0x01010101, rsum[jb], false);
                wf[jb][kk] = v;
            }
            // the next half overwrites the staging rows: every read of
            // this half has completed first
            dq::wave_lds_fence();
        }
    } else {
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
        const int m = mw0 + 32 * jb + (lane & 31);
        const uint8_t* wrow = w + (size_t)(m < M ? m : 0) * C;
#pragma unroll
        for (int kk = 0; kk < kKC / 32; ++kk) {
            const int c = 32 * kk + 16 * (lane >> 5);
            v4i v = {0, 0, 0, 0};
            if (m < M && c < C) {
                if (wvec) {
                    v = *reinterpret_cast<const v4i*>(wrow + c);
                    if (WU8) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] ^= (int)kXor;
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const uint32_t b = c + e < C ? (uint32_t)wrow[c + e] ^ (WU8 ? 0x80u : 0u) : 0u;
                        v[e >> 2] |= (int)(b << (8 * (e & 3)));
                    }
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) rsum[jb] = __builtin_amdgcn_sdot4(v[e], 0x01010101, rsum[jb], false);
            wf[jb][kk] = v;
        }
    }
    }

    // per-channel and per-tensor constants of the requantization
    const dq::QDiv yd = dq::make_qdiv(y_scale);
    constexpr int lo = YU8 ? 0 : -128, hi = YU8 ? 255 : 127;
    const float lof = kMagic + (float)(lo - y_zp), hif = kMagic + (float)(hi - y_zp);
    const uint32_t Yz = (uint32_t)(y_zp & 0xff) * 0x01010101u;
    uint32_t rowc[2];
    int coef[2];
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
        const int32_t R = rsum[jb] + __shfl_xor(rsum[jb], 32);
        coef[jb] = kA - wzp[jb];
        rowc[jb] = (uint32_t)(kB - x_zp) * (uint32_t)R +
                   (uint32_t)C * ((uint32_t)coef[jb] * (uint32_t)(kB - x_zp)) + (uint32_t)bia[jb];
    }
    const v4i ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
    uint8_t* ysw = ys + 64 * wave * kYPitchP;

    for (int it = 0;; ++it) {
        const int n = item / tiles, p0 = (item - n * tiles) * kPP;
        int8_t* xs = (it & 1) ? xs1 : xs0;
        // transpose: for pixel i, channels 8 cg .. 8 cg + 7 as 8 bytes of a slot
        {
            if (FULL) {
#pragma unroll
                for (int j = 0; j < 8; ++j) d[j] = 8 * cg + j < C ? d[j] : kXPad;
            }
            const int kb = cg >> 2, h = (cg >> 1) & 1, off = 8 * (cg & 1);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t lo4 = gather_byte(d[0] ^ (XU8 ? kXor : 0u), d[1] ^ (XU8 ? kXor : 0u),
                                                 d[2] ^ (XU8 ? kXor : 0u), d[3] ^ (XU8 ? kXor : 0u), i);
                const uint32_t hi4 = gather_byte(d[4] ^ (XU8 ? kXor : 0u), d[5] ^ (XU8 ? kXor : 0u),
                                                 d[6] ^ (XU8 ? kXor : 0u), d[7] ^ (XU8 ? kXor : 0u), i);
                const dq::u2 pr = {lo4, hi4};
                *reinterpret_cast<dq::u2*>(&xs[kb * 1024 + ((4 * pq + i) + 32 * h) * 16 + off]) = pr;
            }
        }
        // this wave's tile writes are done; the bare barrier then publishes
        // the tile (not __syncthreads(): its fence would also wait for the
        // previous item's output stores)
        dq::wait_lgkm0();
        dq::lds_barrier();
        // the previous item's codes leave before the next item's loads are
        // issued: no store sits between those loads and their use, so
        // waiting for them never waits for a store
        if (it > 0) store_staged<VEC, FULL>(ysw, y, prev_n, prev_p0, mw0, M, HW, lane);
        const int next = item + stride;
        if (next < end) {
            const int nn = next / tiles, np0 = (next - nn * tiles) * kPP;
            load_item<VEC, FULL>(x + (size_t)nn * C * HW, C, HW, np0 + 4 * pq, cg, kXPad, d);
        }
        dq::v16i acc[2], sacc;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            acc[0][r] = 0;
            acc[1][r] = 0;
            sacc[r] = 0;
        }
        // all of the item's operand fragments first, then the MFMAs
        v4i xfr[kKC / 32];
#pragma unroll
        for (int kk = 0; kk < kKC / 32; ++kk) xfr[kk] = *reinterpret_cast<const v4i*>(&xs[kk * 1024 + lane * 16]);
#pragma unroll
        for (int kk = 0; kk < kKC / 32; ++kk) {
            const v4i xf = xfr[kk];
            acc[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xf, wf[0][kk], acc[0], 0, 0, 0);
            acc[1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xf, wf[1][kk], acc[1], 0, 0, 0);
            if (XSUM) sacc = __builtin_amdgcn_mfma_i32_32x32x32_i8(xf, ones, sacc, 0, 0, 0);
        }
        // requantize: lane holds channel (lane % 32) of block jb and, in
        // accumulators 4g .. 4g+3, pixels 8g + 4 (lane / 32) + 0..3
        if (yd.fast) {
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    uint32_t b[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        uint32_t v = (uint32_t)acc[jb][4 * g + e] + rowc[jb];
                        if (XSUM) v += (uint32_t)coef[jb] * (uint32_t)sacc[4 * g + e];
                        float real = (float)(int32_t)v * x_scale;
                        real = real * wsc[jb];
                        const float q0 = __builtin_amdgcn_fmed3f(real * yd.y, -kBig, kBig);
                        const float r = __builtin_fmaf(-q0, yd.s, real);
                        const float t = __builtin_fmaf(r, yd.y, q0) + kMagic;
                        b[e] = (uint32_t)__float_as_int(__builtin_amdgcn_fmed3f(t, lof, hif));
                    }
                    const uint32_t packed = (b[0] & 0xffu) | ((b[1] & 0xffu) << 8) | ((b[2] & 0xffu) << 16) | (b[3] << 24);
                    const uint32_t word = ((packed & 0x7f7f7f7fu) + (Yz & 0x7f7f7f7fu)) ^ ((packed ^ Yz) & 0x80808080u);
                    const int pp = 8 * g + 4 * (lane >> 5);
                    *reinterpret_cast<uint32_t*>(&ysw[(32 * jb + (lane & 31)) * kYPitchP + pp]) = word;
                }
            }
        } else {
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    uint32_t word = 0;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        uint32_t v = (uint32_t)acc[jb][4 * g + e] + rowc[jb];
                        if (XSUM) v += (uint32_t)coef[jb] * (uint32_t)sacc[4 * g + e];
                        float real = (float)(int32_t)v * x_scale;
                        real = real * wsc[jb];
                        const int code = dq::sat_add(dq::rne(real / yd.s), y_zp, lo, hi);
                        word |= ((uint32_t)code & 0xffu) << (8 * e);
                    }
                    const int pp = 8 * g + 4 * (lane >> 5);
                    *reinterpret_cast<uint32_t*>(&ysw[(32 * jb + (lane & 31)) * kYPitchP + pp]) = word;
                }
            }
        }
        prev_n = n;
        prev_p0 = p0;
        if (next >= end) break;
        item = next;
    }
    dq::wave_lds_fence();  // the last item's codes, staged by this wave
    store_staged<VEC, FULL>(ysw, y, prev_n, prev_p0, mw0, M, HW, lane);
}

template <bool XU8, bool WU8, bool YU8, bool XSUM>
void launch_v(bool vec, dim3 grid, hipStream_t s, const uint8_t* x, const uint8_t* w, int C, int HW,
              int M, const float* xs, const uint8_t* xz, const float* ws, const uint8_t* wz, int wpc,
              const float* ys, const uint8_t* yz, const int32_t* bias, int wvec, uint8_t* y) {
    if (vec)
        hipLaunchKernelGGL((k_qconv1x1<XU8, WU8, YU8, XSUM, true>), grid, dim3(kThreads), 0, s, x, w, C,
                           HW, M, xs, xz, ws, wz, wpc, ys, yz, bias, wvec, y);
    else
        hipLaunchKernelGGL((k_qconv1x1<XU8, WU8, YU8, XSUM, false>), grid, dim3(kThreads), 0, s, x, w, C,
                           HW, M, xs, xz, ws, wz, wpc, ys, yz, bias, wvec, y);
}

template <bool XU8, bool WU8, bool YU8>
void launch_s(bool xsum, bool vec, dim3 grid, hipStream_t s, const uint8_t* x, const uint8_t* w, int C,
              int HW, int M, const float* xs, const uint8_t* xz, const float* ws, const uint8_t* wz,
              int wpc, const float* ys, const uint8_t* yz, const int32_t* bias, int wvec, uint8_t* y) {
    if (xsum)
        launch_v<XU8, WU8, YU8, true>(vec, grid, s, x, w, C, HW, M, xs, xz, ws, wz, wpc, ys, yz, bias, wvec, y);
    else
        launch_v<XU8, WU8, YU8, false>(vec, grid, s, x, w, C, HW, M, xs, xz, ws, wz, wpc, ys, yz, bias, wvec, y);
}

bool is_8bit(dq_dtype t) { return t == DQ_I8 || t == DQ_U8; }

}  // namespace

extern "C" int qlinear_conv1x1(const void* x, dq_dtype x_type, int64_t N, int64_t C, int64_t HW,
                               const float* x_scale, const void* x_zero_point, const void* w,
                               dq_dtype w_type, int64_t M, const float* w_scale,
                               const void* w_zero_point, int64_t w_len, const float* y_scale,
                               const void* y_zero_point, dq_dtype y_type, const int32_t* bias,
                               void* y, void* stream) {
    if (!is_8bit(x_type) || !is_8bit(w_type) || !is_8bit(y_type))
        DQ_FAIL(DQ_ERR_TYPE, "x, w and y must be DQ_I8 or DQ_U8");
    if (N < 0 || C < 1 || HW < 0 || M < 0) DQ_FAIL(DQ_ERR_ARG, "need N, HW, M >= 0 and C >= 1");
    if (C > 32768) DQ_FAIL(DQ_ERR_RANGE, "C = %lld exceeds 32768 (int32 sums)", (long long)C);
    if (w_len != 1 && w_len != M) DQ_FAIL(DQ_ERR_ARG, "w_len must be 1 or M");
    if (N == 0 || HW == 0 || M == 0) return DQ_OK;
    if (!x || !w || !x_scale || !w_scale || !y_scale || !y)
        DQ_FAIL(DQ_ERR_ARG, "x, w, y and the scales must not be NULL");
    if (HW > 0x7fffffffLL - kP || N > 65535 || (M + kMT - 1) / kMT > 65535)
        DQ_FAIL(DQ_ERR_RANGE, "shape too large for one launch");
    const bool vec = HW % 16 == 0 && (uintptr_t)x % 16 == 0 && (uintptr_t)y % 16 == 0;
    const int wvec = C % 16 == 0 && (uintptr_t)w % 16 == 0;
    // S[p] is needed unless every w zero point equals the shift of w (0 for
    // int8); a non-NULL zero point of a uint8 w or any zero point tensor of
    // an int8 w is taken as possibly needing it.
    const bool xsum = w_type == DQ_U8 || w_zero_point != nullptr;
    const hipStream_t s = (hipStream_t)stream;
    const uint8_t* xb = (const uint8_t*)x;
    const uint8_t* wb = (const uint8_t*)w;
    const uint8_t* xz = (const uint8_t*)x_zero_point;
    const uint8_t* wz = (const uint8_t*)w_zero_point;
    const uint8_t* yz = (const uint8_t*)y_zero_point;
    uint8_t* yb = (uint8_t*)y;
    const int wpc = w_len == M && M > 1;
    const int Ci = (int)C, HWi = (int)HW, Mi = (int)M;
    if (M <= kMT && C <= kKC) {
        // persistent variant: items of (image, 32-pixel tile) spread evenly
        // over at most kPersistentGroups workgroups
        const long long tiles = (HW + kPP - 1) / kPP, items = N * tiles;
        if (items > 0x7fffffffLL) DQ_FAIL(DQ_ERR_RANGE, "shape too large for one launch");
        // per XCD: a range of items (a multiple of 4 tiles, one 128-pixel
        // line) and a multiple of 4 workgroups, about two items each, at
        // most kPersistentGroups / 8
        const long long per_xcd = ((items + 7) / 8 + 3) / 4 * 4;
        long long g8 = ((per_xcd + 1) / 2 + 3) / 4 * 4;
        if (g8 > kPersistentGroups / 8) g8 = kPersistentGroups / 8;
        const unsigned groups = (unsigned)(8 * g8);
        const int ni = (int)items, nt = (int)tiles, px = (int)per_xcd;
        // FULL: all 256 channels and every pixel of every tile exist, so no
        // load or store is conditional
        const bool full = vec && M == kMT && HW % kPP == 0;
        // whole weight rows read as 1 KiB pieces: every row has kKC bytes
        const bool wcoal = wvec && C == kKC && M == kMT && (uintptr_t)w % 16 == 0;
#define DQ_P(XU, WU, YU, XS, V, F, WC)                                                                         \
    hipLaunchKernelGGL((k_qconv1x1_p<XU, WU, YU, XS, V, F, WC>), dim3(groups), dim3(kThreads), 0, s, xb, wb, Ci, \
                       HWi, Mi, x_scale, xz, w_scale, wz, wpc, y_scale, yz, bias, wvec, ni, nt, px, yb)
#define DQ_PX(XU, WU, YU, XS) \
    if (full && wcoal) DQ_P(XU, WU, YU, XS, true, true, true); \
    else if (full) DQ_P(XU, WU, YU, XS, true, true, false); else if (vec) DQ_P(XU, WU, YU, XS, true, false, false); \
    else DQ_P(XU, WU, YU, XS, false, false, false);
#define DQ_PV(XU, WU, YU) \
    if (xsum) { DQ_PX(XU, WU, YU, true) } else { DQ_PX(XU, WU, YU, false) }
        const bool xu = x_type == DQ_U8, wu = w_type == DQ_U8, yu = y_type == DQ_U8;
        if (xu) {
            if (wu) { if (yu) { DQ_PV(true, true, true) } else { DQ_PV(true, true, false) } }
            else { if (yu) { DQ_PV(true, false, true) } else { DQ_PV(true, false, false) } }
        } else {
            if (wu) { if (yu) { DQ_PV(false, true, true) } else { DQ_PV(false, true, false) } }
            else { if (yu) { DQ_PV(false, false, true) } else { DQ_PV(false, false, false) } }
        }
#undef DQ_PV
#undef DQ_PX
#undef DQ_P
        DQ_LAUNCH_CHECK("qlinear_conv1x1");
        return DQ_OK;
    }
    const dim3 grid((unsigned)((HW + kP - 1) / kP), (unsigned)((M + kMT - 1) / kMT), (unsigned)N);
#define DQ_C(XU, WU, YU)                                                                          \
    launch_s<XU, WU, YU>(xsum, vec, grid, s, xb, wb, Ci, HWi, Mi, x_scale, xz, w_scale, wz, wpc, \
                         y_scale, yz, bias, wvec, yb)
    const bool xu = x_type == DQ_U8, wu = w_type == DQ_U8, yu = y_type == DQ_U8;
    if (xu) {
        if (wu) { if (yu) DQ_C(true, true, true); else DQ_C(true, true, false); }
        else { if (yu) DQ_C(true, false, true); else DQ_C(true, false, false); }
    } else {
        if (wu) { if (yu) DQ_C(false, true, true); else DQ_C(false, true, false); }
        else { if (yu) DQ_C(false, false, true); else DQ_C(false, false, false); }
    }
#undef DQ_C
    DQ_LAUNCH_CHECK("qlinear_conv1x1");
    return DQ_OK;
}
