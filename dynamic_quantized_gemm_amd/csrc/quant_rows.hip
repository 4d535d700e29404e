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
// Design. A 128-byte line of sA holds the 16 codes of one k group for eight
// consecutive rows, so a kernel that writes each row's codes straight from
// the lanes that computed them scatters 16-byte pieces over 64 lines per
// store instruction; measured on 8192 x 8192 bf16, such stores alone cost
// as much as the loads and all the arithmetic together. The main kernel
// (k_quant_rows_lds, K % 16 == 0, aligned A, K <= 16384) therefore
// works in blocks of eight rows: a persistent workgroup of eight waves
// holds each row in VGPRs, spread over WPR waves (lane owns groups
// lane + 64 (wr + WPR v)), reduces min/max with DPP inside a wave and
// through LDS across the WPR waves, writes the codes to an LDS copy of the
// block, and then stores whole lines (eight lanes per line). The loads of
// the next rows are issued before the current ones are processed, so the
// arithmetic and the stores overlap them. Other shapes take a wave-per-row
// kernel (any K up to 8192 values, any alignment; also short aligned rows
// of a small A, where the LDS block's barrier costs more than the scattered
// stores) or a two-pass streaming kernel (longer rows, re-read from L2).
#include "dq_device.h"
#include "dq_kernels.h"

#include <hip/hip_ext.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <set>
#include <utility>

namespace {

constexpr int kRowsPerWave = 1;
constexpr int kWavesPerBlock = 8;
constexpr int kRowsPerBlock = kWavesPerBlock * kRowsPerWave;
constexpr int kThreads = 64 * kWavesPerBlock;
// dynamic LDS of the LDS-staged kernel: eight rows of at most 16384 codes
constexpr size_t kLdsMax = (size_t)8 * 16384;

__device__ __forceinline__ void row_params(float lo, float hi, float& scale, int& zero) {
    if (hi == lo) {
        scale = 1.0f;
        zero = 0;
    } else {
        scale = (hi - lo) / 255.0f;
        zero = dq::sat_add(dq::rne(-lo / scale), 0, 0, 255);
    }
}

// 16 codes uA - 128 of one group, stored as one 16-byte vector. FAST: the
// row's scale has a normal reciprocal, and |A / scale| <= 256 holds by the
// scale's construction, so the bounded residual division applies.
// sA = sat[0,255](rne(q) + zero) - 128 = (int)clamp(rne(q), -zero, 255 - zero)
// + (zero - 128), taken as a byte.
template <bool FAST>
__device__ __forceinline__ void store_group(int8_t* __restrict__ sA, size_t row, int g, int KF,
                                            const float (&x)[16], const dq::QDiv& d, int zero) {
    const float lo = (float)(-zero), hi = (float)(255 - zero);
    const int shift = zero - 128;
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint32_t packed = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float qt = FAST ? dq::qdiv_fast(x[4 * q + b], d) : x[4 * q + b] / d.s;
            const float r = __builtin_fminf(__builtin_fmaxf(dq::rne(qt), lo), hi);
            packed |= ((uint32_t)((int)r + shift) & 0xffu) << (8 * b);
        }
        w[q] = packed;
    }
    const dq::u4 o = {w[0], w[1], w[2], w[3]};
    *reinterpret_cast<dq::u4*>(sA + dq::frag_offset(row, (size_t)g * 16, KF)) = o;
}

// Row statistics come out of the reductions as wave-uniform values, which
// makes scale, zero point and the division path scalar, so the row takes one
// branch instead of one per element.
__device__ __forceinline__ void uniform_minmax(float& lo, float& hi) {
    lo = dq::wave_min_uniform(lo);
    hi = dq::wave_max_uniform(hi);
}

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

// ---- LDS-staged kernel: blocks of eight rows, whole-line stores
//
// Rows stay in VGPRs as loaded: NV groups of 16 values per lane (2 x 16
// bytes of bf16 or 4 x 16 bytes of fp32 per group).
template <bool BF16, int NV>
struct RawRow {
    static constexpr int U = BF16 ? 2 : 4;  // 16-byte vectors per group
    dq::u4 v[NV][U];
};

// Loads the groups this lane owns, g = lane + 64 (wr + WPR v). A group past
// the row end loads the row's last group instead: the loads stay
// unconditional (a load under a branch makes the compiler wait for every
// outstanding memory operation where the paths join, which would drain the
// prefetched rows), and the min/max and the stores skip those groups.
template <bool BF16, int NV, int WPR>
__device__ __forceinline__ void load_part(const void* __restrict__ A, int row, int K, int lane,
                                          int wr, RawRow<BF16, NV>& r) {
    constexpr int U = RawRow<BF16, NV>::U;
    const int ngroups = K >> 4;
    const dq::u4* base = reinterpret_cast<const dq::u4*>(
        reinterpret_cast<const char*>(A) + (size_t)row * K * (BF16 ? 2 : 4));
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int g = min(lane + 64 * (wr + WPR * v), ngroups - 1);
#pragma unroll
        for (int u = 0; u < U; ++u) r.v[v][u] = base[(size_t)g * U + u];
    }
}

// Element e (0..15) of group v as fp32 (a bf16 value is the top half of its
// fp32 bit pattern).
template <bool BF16, int NV>
__device__ __forceinline__ float elem(const RawRow<BF16, NV>& r, int v, int e) {
    if (BF16) {
        const uint32_t w = r.v[v][e >> 3][(e >> 1) & 3];
        return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
    }
    return __uint_as_float(r.v[v][e >> 2][e & 3]);
}

// Minimum and maximum (with 0) over the groups this lane holds, reduced over
// the wave to wave-uniform values. A group past the row end counts as zeros
// (a select, not a branch).
template <bool BF16, int NV, int WPR>
__device__ __forceinline__ void part_minmax(const RawRow<BF16, NV>& r, int K, int lane, int wr,
                                            float& lo, float& hi) {
    const int ngroups = K >> 4;
    lo = 0.0f;
    hi = 0.0f;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const bool in = lane + 64 * (wr + WPR * v) < ngroups;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const float x = in ? elem(r, v, e) : 0.0f;
            lo = __builtin_fminf(lo, x);
            hi = __builtin_fmaxf(hi, x);
        }
    }
    uniform_minmax(lo, hi);
}

// The 16 codes uA - 128 of group v. Fast path (the scale passes make_qdiv's
// test; |A / scale| <= 256 by construction): q = corrected quotient; adding
// 1.5 * 2^23 rounds q half to even into the low mantissa bits (the float add
// rounds to nearest even, and 1.5 * 2^23 is even), so the bit pattern is
// 0x4B400000 + rne(q); a median against the integers 1.5 * 2^23 - zero and
// 1.5 * 2^23 + 255 - zero clamps it to rne(q) + zero in [0, 255]; the low
// bytes of four codes are packed and zero - 128 is added to every byte at
// once (a carry-free bytewise add). Otherwise the IEEE quotient, rounded and
// clamped the same way.
struct RowCodes {
    dq::QDiv d;
    float lof, hif;  // 1.5 * 2^23 - zero, 1.5 * 2^23 + 255 - zero
    float lo, hi;    // -zero, 255 - zero
    uint32_t C;      // (zero - 128) in every byte
};

__device__ __forceinline__ RowCodes row_codes(float scale, int zero) {
    constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
    RowCodes c;
    c.d = dq::make_qdiv(scale);
    // 1.5 * 2^23 + n is exact for |n| < 2^22, so the clamp bounds are too
    c.lof = kMagic - (float)zero;
    c.hif = kMagic + (float)(255 - zero);
    c.lo = (float)(-zero);
    c.hi = (float)(255 - zero);
    c.C = (uint32_t)((zero - 128) & 0xff) * 0x01010101u;
    return c;
}

template <bool BF16, int NV>
__device__ __forceinline__ dq::u4 group_codes(const RawRow<BF16, NV>& r, int v, const RowCodes& c) {
    constexpr float kMagic = 12582912.0f;
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint32_t b[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float x = elem(r, v, 4 * q + e);
            float t;
            if (c.d.fast)
                t = __builtin_amdgcn_fmed3f(dq::qdiv_fast(x, c.d) + kMagic, c.lof, c.hif);
            else
                t = kMagic + __builtin_fminf(__builtin_fmaxf(dq::rne(x / c.d.s), c.lo), c.hi);
            b[e] = (uint32_t)__float_as_int(t);
        }
        const uint32_t packed = (b[0] & 0xffu) | ((b[1] & 0xffu) << 8) | ((b[2] & 0xffu) << 16) | (b[3] << 24);
        w[q] = ((packed & 0x7f7f7f7fu) + (c.C & 0x7f7f7f7fu)) ^ ((packed ^ c.C) & 0x80808080u);
    }
    return dq::u4{w[0], w[1], w[2], w[3]};
}

// LDS copy of a block: row r (0..7) at r * lds_row bytes (lds_row = K
// rounded up to 256), group g of it at 16 * (g ^ (2 r mod 16)). The xor
// permutes groups inside aligned runs of 16, so a wave writing consecutive
// groups of one row still writes a contiguous 1 KiB; and when sixteen
// lanes read the same two groups of the eight rows (the line-order read
// below) they hit sixteen distinct 16-byte bank groups.
__device__ __forceinline__ int lds_slot(int r, int g, int lds_row) {
    return r * lds_row + 16 * (g ^ ((2 * r) & 15));
}

template <bool BF16, int NV, int WPR>
__device__ __forceinline__ void quantize_part(const RawRow<BF16, NV>& r, int b, int t, int M, int K,
                                              int lane, int w, float (*red)[2], uint8_t* lds,
                                              int lds_row, float* __restrict__ scaleA,
                                              int32_t* __restrict__ zeroA) {
    constexpr int RPS = 8 / WPR;  // rows per step
    const int wr = w % WPR;
    float lo, hi;
    part_minmax<BF16, NV, WPR>(r, K, lane, wr, lo, hi);
    if (WPR > 1) {
        if (lane == 0) {
            red[w][0] = lo;
            red[w][1] = hi;
        }
        dq::wait_lgkm0();
        dq::lds_barrier();
        const int w0 = w - wr;
        lo = red[w0][0];
        hi = red[w0][1];
#pragma unroll
        for (int p = 1; p < WPR; ++p) {
            lo = __builtin_fminf(lo, red[w0 + p][0]);
            hi = __builtin_fmaxf(hi, red[w0 + p][1]);
        }
    }
    float scale;
    int zero;
    row_params(lo, hi, scale, zero);
    const RowCodes c = row_codes(scale, zero);
    const int rl = RPS * t + w / WPR;  // row within the block
    const int ngroups = K >> 4;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        // a group past the row end holds a copy of the last group: writing
        // it to that group's place stores the same codes again
        const int g = min(lane + 64 * (wr + WPR * v), ngroups - 1);
        *reinterpret_cast<dq::u4*>(lds + lds_slot(rl, g, lds_row)) = group_codes(r, v, c);
    }
    // every lane of the row's waves stores the same values (no branch); a
    // row past M holds row M - 1 and stores that row's own values again
    const int row = min(8 * b + rl, M - 1);
    scaleA[row] = scale;
    zeroA[row] = zero;
}

// Stores the block's codes from LDS: slot u = (line L = u / 8, row r = u % 8),
// so eight consecutive lanes write one whole 128-byte line of sA. The
// stores are unconditional, so that the compiler's wait counts for the
// prefetched rows stay exact: a slot past the row end stores the last group
// again, and a row past M (whose LDS copy holds row M - 1) stores row M - 1.
template <int SLOTS>  // slots per thread: 8 ngroups <= 512 SLOTS
__device__ __forceinline__ void store_block(const uint8_t* lds, int lds_row, int b, int M, int K,
                                            int KF, int8_t* __restrict__ sA) {
    const int ngroups = K >> 4;
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) {
        const int u = threadIdx.x + 512 * j;
        const int L = min(u >> 3, ngroups - 1), r = u & 7;
        const dq::u4 o = *reinterpret_cast<const dq::u4*>(lds + lds_slot(r, L, lds_row));
        const int row = min(8 * b + r, M - 1);
        // streaming store: the packed rows go to memory as they are made
        // rather than sitting dirty in this XCD's L2 until the kernel ends
        // (4096^2 bf16: 12.1 -> 11.5 us)
        __builtin_nontemporal_store(o, reinterpret_cast<dq::u4*>(sA + dq::frag_offset((size_t)row, (size_t)L * 16, KF)));
    }
}

// One block: WPR steps of 8 / WPR rows (the register buffer of step t is
// ra or rb by the parity of t + P, fixed at compile time), each step first
// prefetching the rows of the next one (past the workgroup's last block: the
// current rows again), then the block's store. Returns whether the
// workgroup has a next block.
template <bool BF16, int NV, int WPR, int P>
__device__ __forceinline__ bool lds_block(RawRow<BF16, NV>& ra, RawRow<BF16, NV>& rb, int& b,
                                          const void* __restrict__ A, int M, int K, int KF, int lane,
                                          int w, float (*red)[8][2], uint8_t* lds, int lds_row,
                                          int8_t* __restrict__ sA, float* __restrict__ scaleA,
                                          int32_t* __restrict__ zeroA) {
    constexpr int RPS = 8 / WPR;
    const int b2 = b + gridDim.x;
    const bool more = b2 < ((M + 7) >> 3);
    const int slot = w / WPR;
#pragma unroll
    for (int t = 0; t < WPR; ++t) {
        const int next = t + 1 < WPR ? 8 * b + RPS * (t + 1) + slot
                                     : (more ? 8 * b2 + slot : 8 * b + RPS * t + slot);
        RawRow<BF16, NV>& cur = ((t + P) & 1) ? rb : ra;
        RawRow<BF16, NV>& nxt = ((t + P) & 1) ? ra : rb;
        load_part<BF16, NV, WPR>(A, min(next, M - 1), K, lane, w % WPR, nxt);
        // keep the loads here: the memory clobber stops the optimizer from
        // sinking them below the work on the current rows, and the
        // scheduling barrier stops the scheduler from hoisting that work
        // above them (either way the wave would wait for the current rows
        // before the prefetch goes out)
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        quantize_part<BF16, NV, WPR>(cur, b, t, M, K, lane, w, red[(t + P) & 1], lds, lds_row, scaleA,
                                     zeroA);
    }
    dq::wait_lgkm0();
    dq::lds_barrier();
    store_block<WPR * NV>(lds, lds_row, b, M, K, KF, sA);
    // the next block's codes overwrite the LDS copy
    dq::wait_lgkm0();
    dq::lds_barrier();
    b = b2;
    return more;
}

// Persistent: workgroup i takes blocks i, i + G, .... Rows past M load row
// M - 1 (loads stay unconditional). All waves of a workgroup run the same
// steps, so every barrier is reached by all of them.
template <bool BF16, int NV, int WPR>
__global__ void __launch_bounds__(512)
k_quant_rows_lds(const void* __restrict__ A, int M, int K, int KF, int lds_row,
                 int8_t* __restrict__ sA, float* __restrict__ scaleA, int32_t* __restrict__ zeroA) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    // min/max exchange, two slots used alternately: a slot is rewritten two
    // steps after it was read, and the barrier of the step between orders
    // the two
    __shared__ float red[2][8][2];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    int b = blockIdx.x;
    if (b >= ((M + 7) >> 3)) return;  // uniform over the workgroup
    RawRow<BF16, NV> ra, rb;
    load_part<BF16, NV, WPR>(A, min(8 * b + w / WPR, M - 1), K, lane, w % WPR, ra);
    // ping-pong between the two register buffers (no copies): with WPR odd
    // consecutive blocks start in different buffers
    for (;;) {
        if (!lds_block<BF16, NV, WPR, 0>(ra, rb, b, A, M, K, KF, lane, w, red, lds, lds_row, sA, scaleA,
                                         zeroA))
            return;
        if constexpr (WPR & 1) {
            if (!lds_block<BF16, NV, WPR, 1>(ra, rb, b, A, M, K, KF, lane, w, red, lds, lds_row, sA,
                                             scaleA, zeroA))
                return;
        }
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

// Workgroups of k_quant_rows_lds<BF16, NV, WPR> resident at once with `lds`
// bytes of dynamic LDS (what the registers and LDS allow, times the CUs),
// cached per device and LDS size; thread-safe. The variant's dynamic-LDS
// limit is raised once per device to the most any launch of it asks for
// (eight rows of 16384 codes).
template <bool BF16, int NV, int WPR>
int resident_groups(size_t lds) {
    static std::mutex mu;
    static std::map<std::pair<int, size_t>, int> cache;
    static std::set<int> raised;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    std::lock_guard<std::mutex> lock(mu);
    const auto key = std::make_pair(dev, lds);
    const auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    if (!raised.count(dev)) {
        if (hipFuncSetAttribute((const void*)k_quant_rows_lds<BF16, NV, WPR>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsMax) != hipSuccess) {
            (void)hipGetLastError();
            return 256;  // not cached: the next call tries again
        }
        raised.insert(dev);
    }
    int cus = 0, per_cu = 0;
    int resident = 256;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_quant_rows_lds<BF16, NV, WPR>, 512, lds) ==
            hipSuccess &&
        cus * per_cu > 0)
        resident = cus * per_cu;
    else
        (void)hipGetLastError();
    cache.emplace(key, resident);
    return resident;
}

template <bool BF16, int NV, int WPR>
void launch_lds(hipStream_t s, DqTiming t, const void* A, int M, int K, int KF, int8_t* sA,
                float* scaleA, int32_t* zeroA) {
    const int lds_row = (K + 255) & ~255;
    const size_t lds = (size_t)8 * lds_row;
    const int groups = std::min(resident_groups<BF16, NV, WPR>(lds), (M + 7) / 8);
    hipExtLaunchKernelGGL((k_quant_rows_lds<BF16, NV, WPR>), dim3((unsigned)groups), dim3(512), lds, s,
                          t.start, t.stop, 0, A, M, K, KF, lds_row, sA, scaleA, zeroA);
}

// The LDS-staged kernel holds 16 VGPRs of row data per lane and buffer (one
// fp32 group, two bf16 groups), the row spread over as many of the eight
// waves as it needs; rows past 8192 fp32 / 16384 bf16 values take two fp32
// groups per lane. Measured on 8192 x 8192: fewer groups per lane over
// more waves beat more groups per lane (more workgroups fit a CU).
template <bool BF16>
bool launch_lds_for(int nv, hipStream_t s, DqTiming t, const void* A, int M, int K, int KF,
                    int8_t* sA, float* scaleA, int32_t* zeroA) {
    if (BF16) {
        if (nv <= 1) launch_lds<true, 1, 1>(s, t, A, M, K, KF, sA, scaleA, zeroA);
        else if (nv <= 2) launch_lds<true, 2, 1>(s, t, A, M, K, KF, sA, scaleA, zeroA);
        else if (nv <= 4) launch_lds<true, 2, 2>(s, t, A, M, K, KF, sA, scaleA, zeroA);
        else if (nv <= 8) launch_lds<true, 2, 4>(s, t, A, M, K, KF, sA, scaleA, zeroA);
        else if (nv <= 16) launch_lds<true, 2, 8>(s, t, A, M, K, KF, sA, scaleA, zeroA);
        else return false;
    } else {
        if (nv <= 1) launch_lds<false, 1, 1>(s, t, A, M, K, KF, sA, scaleA, zeroA);
        else if (nv <= 2) launch_lds<false, 1, 2>(s, t, A, M, K, KF, sA, scaleA, zeroA);
        else if (nv <= 4) launch_lds<false, 1, 4>(s, t, A, M, K, KF, sA, scaleA, zeroA);
        else if (nv <= 8) launch_lds<false, 1, 8>(s, t, A, M, K, KF, sA, scaleA, zeroA);
        else if (nv <= 16) launch_lds<false, 2, 8>(s, t, A, M, K, KF, sA, scaleA, zeroA);
        else return false;
    }
    return true;
}

template <bool BF16, bool VEC>
void launch_rows(dim3 grid, hipStream_t s, DqTiming t, const void* A, int M, int K, int KF,
                 int8_t* sA, float* scaleA, int32_t* zeroA) {
    const int ngroups = (K + 15) / 16;
    const int nv = (ngroups + 63) / 64;
    if (VEC) {
        // short rows of a small A: the wave-per-row kernel, stores straight
        // from registers (no LDS block, no barrier). Measured back to back /
        // cold: 4096 x 512 fp32 17.8 / 21.2 -> 16.6 / 20.6 us for the whole
        // forward, 4096 x 1024 and 8192 x 512 likewise faster; from about
        // 8 Mi values on, its scattered stores make the cold call slower
        // (16384 x 1024: 31.5 -> 34.5 us)
        if (nv <= 1 && (size_t)M * (size_t)K <= ((size_t)1 << 22)) {
            hipExtLaunchKernelGGL((k_quant_rows<BF16, true, 1>), grid, dim3(kThreads), 0, s, t.start, t.stop, 0, A,
                                  M, K, KF, sA, scaleA, zeroA);
            return;
        }
        if (!launch_lds_for<BF16>(nv, s, t, A, M, K, KF, sA, scaleA, zeroA))
            hipExtLaunchKernelGGL((k_quant_rows_stream<BF16, true>), grid, dim3(kThreads), 0, s, t.start, t.stop, 0, A, M, K, KF, sA, scaleA, zeroA);
        return;
    }
    if (nv <= 1)
        hipExtLaunchKernelGGL((k_quant_rows<BF16, false, 1>), grid, dim3(kThreads), 0, s, t.start, t.stop, 0, A, M, K, KF, sA, scaleA, zeroA);
    else if (nv <= 2)
        hipExtLaunchKernelGGL((k_quant_rows<BF16, false, 2>), grid, dim3(kThreads), 0, s, t.start, t.stop, 0, A, M, K, KF, sA, scaleA, zeroA);
    else if (nv <= 4)
        hipExtLaunchKernelGGL((k_quant_rows<BF16, false, 4>), grid, dim3(kThreads), 0, s, t.start, t.stop, 0, A, M, K, KF, sA, scaleA, zeroA);
    else if (nv <= 8)
        hipExtLaunchKernelGGL((k_quant_rows<BF16, false, 8>), grid, dim3(kThreads), 0, s, t.start, t.stop, 0, A, M, K, KF, sA, scaleA, zeroA);
    else
        hipExtLaunchKernelGGL((k_quant_rows_stream<BF16, false>), grid, dim3(kThreads), 0, s, t.start, t.stop, 0, A, M, K, KF, sA, scaleA, zeroA);
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
