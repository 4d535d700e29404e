// qelementwise.hip -- the element-wise quantized operators for gfx950.
//
// Operators (onnxruntime quantization_defs.cc, the contrib schemas and the
// formulas their docs print):
//  QLinearAdd   C = (A_scale (A - A_zp) + B_scale (B - B_zp)) / C_scale + C_zp
//  QLinearMul   C = ((A - A_zp) (B - B_zp)) (A_scale B_scale) / C_scale + C_zp
//  MulInteger   C (int32) = (A - A_zp) (B - B_zp)
//               (the three with numpy-style multidirectional broadcasting)
//  QLinearLeakyRelu  quantize(alpha x) where x = dequantize(X) < 0, else
//                    quantize(x); alpha defaults to 0.01
//  QLinearSigmoid    quantize(1 / (1 + exp(-dequantize(X))))
//  ReduceSumInteger  the sum over axes: int32 for int8 input, uint32 for uint8
//  QLinearReduceMean Dequantize -> ReduceMean in fp32 -> Quantize
//  QLinearConcat     inputs joined along an axis, each requantized from its
//                    own scale / zero point into Y's
// "quantize" is QuantizeLinear's rule: the IEEE quotient v / scale rounded
// half to even, plus the zero point, saturated to the 8-bit range. fp32 steps
// are single IEEE operations in the printed order (the library builds with
// -ffp-contract=off); the sigmoid is evaluated in fp64 and rounded to fp32
// once, and the mean is fp32(fp64(S * x_scale) / count) of the exact integer
// sum S of (x - x_zp).
//
// Every operator here moves bytes and does a little arithmetic per byte:
// all are bound by HBM bandwidth (none is a contraction, so none uses MFMA).
// The designs:
//  - Functions of one 8-bit code (LeakyRelu, Sigmoid, Concat's
//    requantization) take only 256 inputs: each workgroup evaluates the
//    function once per code into a 256-byte LDS table, exactly as the
//    formula states, and the stream loop is load 16 bytes, 16 table reads,
//    store 16 bytes.
//  - The binary operators see the broadcast as a canonical output shape of
//    at most eight dims, size-1 dims dropped and adjacent dims merged where
//    both operands continue contiguously; a lane handles E consecutive
//    output elements (E = 16 for 8-bit outputs, 4 for int32) of the
//    innermost dim, where each operand is either an E-byte vector or one
//    broadcast byte. The quotient by C_scale uses dq::qdiv's residual step
//    (the IEEE quotient's rounding) with a 1.5 * 2^23 add and a median
//    clamp, and the zero point goes into four bytes at once.
//  - Reductions see the input as [O, R, I] around one reduced group of dims:
//    I = 1 sums rows with v_dot4 against 1s (four bytes per instruction),
//    G lanes per row; I > 1 sums columns with 16-bit SWAR partial sums (two
//    per register, flushed every 256 rows). Integer sums are exact and
//    associative, so ReduceSumInteger may split R over workgroups and add
//    with atomics (into an output first zeroed by a fill kernel); the mean
//    finishes each output inside one workgroup, so no scratch memory is
//    needed. Any other set of axes takes a one-wave-per-output kernel.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <initializer_list>
#include <map>
#include <mutex>
#include <tuple>

#include "dq_device.h"

namespace {

constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
constexpr float kBig = 4194304.0f;     // 2^22
constexpr int kMaxDims = 8;

template <bool U8>
__device__ __forceinline__ int zp8(const void* zp) {
    if (!zp) return 0;
    return U8 ? (int)*(const uint8_t*)zp : (int)*(const int8_t*)zp;
}

template <bool U8>
__device__ __forceinline__ int code8(uint32_t byte) {
    return U8 ? (int)(byte & 0xffu) : (int)(int8_t)(byte & 0xffu);
}

__device__ __forceinline__ int quant_exact(float v, float s, int zp, bool u8) {
    return dq::sat_add(dq::rne(v / s), zp, u8 ? 0 : -128, u8 ? 255 : 127);
}

// Output quantizer of one per-tensor scale and zero point.
struct Quant {
    float s, y, lof, hif;  // scale, 1/scale, clamp bounds 1.5*2^23 + (lo|hi) - zp
    uint32_t z4;           // the zero point's byte in all four bytes
    bool fast;             // dq::qdiv's residual step is exact for this scale
};

template <bool U8>
__device__ __forceinline__ Quant make_quant(const float* scale, const void* zp) {
    Quant q;
    const dq::QDiv d = dq::make_qdiv(*scale);
    const int z = zp8<U8>(zp);
    q.s = d.s;
    q.y = d.y;
    q.fast = d.fast;
    q.z4 = (uint32_t)(z & 0xff) * 0x01010101u;
    q.lof = kMagic + (float)((U8 ? 0 : -128) - z);
    q.hif = kMagic + (float)((U8 ? 255 : 127) - z);
    return q;
}

// rne(v / s) clamped to [lo - zp, hi - zp], in the low byte of the result
// (the zero point is added later, four bytes at a time). The quotient is the
// IEEE one: the residual step of dq::qdiv when FAST, else the division.
// Adding 1.5 * 2^23 rounds it half to even into the low mantissa bits and
// the median clamps it; clamping the quotient to +-2^22 first keeps the
// residual finite and saturates the same way.
template <bool FAST>
__device__ __forceinline__ uint32_t pre_code(float v, const Quant& q) {
    float t;
    if (FAST) {
        const float q0 = __builtin_amdgcn_fmed3f(v * q.y, -kBig, kBig);
        const float r = __builtin_fmaf(-q0, q.s, v);
        t = __builtin_fmaf(r, q.y, q0);
    } else {
        t = __builtin_amdgcn_fmed3f(v / q.s, -kBig, kBig);
    }
    return (uint32_t)__float_as_int(__builtin_amdgcn_fmed3f(t + kMagic, q.lof, q.hif));
}

// four pre-codes to four bytes plus the zero point; each true sum lies in
// the 8-bit range, so the carry-free bytewise add is exact
__device__ __forceinline__ uint32_t pack4(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3,
                                          uint32_t z4) {
    const uint32_t p = (b0 & 0xffu) | ((b1 & 0xffu) << 8) | ((b2 & 0xffu) << 16) | (b3 << 24);
    return ((p & 0x7f7f7f7fu) + (z4 & 0x7f7f7f7fu)) ^ ((p ^ z4) & 0x80808080u);
}

// E bytes held in (E + 3) / 4 registers
template <int E>
struct Bytes {
    uint32_t w[(E + 3) / 4];
};

template <int E>
__device__ __forceinline__ Bytes<E> load_bytes(const uint8_t* p) {
    Bytes<E> b;
    if constexpr (E == 16) {
        const dq::u4 v = *reinterpret_cast<const dq::u4*>(p);
        b.w[0] = v[0];
        b.w[1] = v[1];
        b.w[2] = v[2];
        b.w[3] = v[3];
    } else if constexpr (E == 4) {
        b.w[0] = *reinterpret_cast<const uint32_t*>(p);
    } else {
        b.w[0] = *p;
    }
    return b;
}

template <int E>
__device__ __forceinline__ void store_bytes(uint8_t* p, const Bytes<E>& b) {
    if constexpr (E == 16) {
        const dq::u4 v = {b.w[0], b.w[1], b.w[2], b.w[3]};
        *reinterpret_cast<dq::u4*>(p) = v;
    } else if constexpr (E == 4) {
        *reinterpret_cast<uint32_t*>(p) = b.w[0];
    } else {
        *p = (uint8_t)b.w[0];
    }
}

__device__ __forceinline__ uint32_t byte_of(const uint32_t* w, int j) {
    return (w[j >> 2] >> (8 * (j & 3))) & 0xffu;
}

// Workgroups of `kernel` resident at once on the current device (the
// occupancy query times the CUs), cached per kernel, device and block size
// (the queries cost more than a launch); thread-safe.
template <typename K>
unsigned resident_blocks(K kernel, int threads) {
    static std::mutex mu;
    static std::map<std::tuple<const void*, int, int>, unsigned> cache;
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 2048;
    const auto key = std::make_tuple((const void*)kernel, dev, threads);
    std::lock_guard<std::mutex> lock(mu);
    const auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) == hipSuccess &&
        cus * per_cu > 0) {
        cache.emplace(key, (unsigned)(cus * per_cu));
        return (unsigned)(cus * per_cu);
    }
    (void)hipGetLastError();
    return 2048;  // not cached: the next call asks again
}

// ====================================================== one-code functions

enum { FN_LEAKY = 0, FN_SIGMOID = 1, FN_REQUANT = 2 };

struct TableArgs {
    const float* x_scale;
    const void* x_zp;
    const float* y_scale;
    const void* y_zp;
    float alpha;
};

// tab[b] = f(code b) for the 256 raw bytes b (blockDim.x == 256)
template <bool U8, int F>
__device__ __forceinline__ void build_table(uint8_t* tab, const TableArgs& a) {
    const int t = threadIdx.x;
    const float x = (float)(code8<U8>((uint32_t)t) - zp8<U8>(a.x_zp)) * *a.x_scale;
    float v;
    if (F == FN_LEAKY)
        v = x < 0.0f ? a.alpha * x : x;
    else if (F == FN_SIGMOID)
        v = (float)(1.0 / (1.0 + exp(-(double)x)));
    else
        v = x;
    tab[t] = (uint8_t)quant_exact(v, *a.y_scale, zp8<U8>(a.y_zp), U8);
}

template <int E>
__device__ __forceinline__ Bytes<E> lookup(const uint8_t* tab, const Bytes<E>& in) {
    Bytes<E> o;
#pragma unroll
    for (int k = 0; k < (E + 3) / 4; ++k) {
        const uint32_t w = in.w[k];
        if (E == 1)
            o.w[k] = tab[w & 0xffu];
        else
            o.w[k] = (uint32_t)tab[w & 0xffu] | ((uint32_t)tab[(w >> 8) & 0xffu] << 8) |
                     ((uint32_t)tab[(w >> 16) & 0xffu] << 16) | ((uint32_t)tab[w >> 24] << 24);
    }
    return o;
}

// Y = tab[X] over a flat tensor of n bytes in E-byte vectors (x, y
// E-aligned). A block-iteration covers 1024 whole vectors, four per lane,
// all loads issued before the first lookup; the vectors past the last whole
// block-iteration and the last n % E bytes go to the grid's last block.
template <bool U8, int F, int E>
__global__ void __launch_bounds__(256)
k_table_map(const uint8_t* __restrict__ x, uint64_t n, TableArgs a, uint8_t* __restrict__ y) {
    __shared__ uint8_t tab[256];
    build_table<U8, F>(tab, a);
    __syncthreads();
    const uint64_t nv = n / E;
    const uint64_t nfull = nv / 1024;
    for (uint64_t it = blockIdx.x; it < nfull; it += gridDim.x) {
        const uint64_t base = it * 1024 + threadIdx.x;
        Bytes<E> v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = load_bytes<E>(x + (base + q * 256) * E);
        dq::issue_fence();
#pragma unroll
        for (int q = 0; q < 4; ++q) store_bytes<E>(y + (base + q * 256) * E, lookup<E>(tab, v[q]));
    }
    if (blockIdx.x == gridDim.x - 1) {
        for (uint64_t i = nfull * 1024 + threadIdx.x; i < nv; i += 256)
            store_bytes<E>(y + i * E, lookup<E>(tab, load_bytes<E>(x + i * E)));
        if (E > 1 && threadIdx.x < n % E) {
            const uint64_t e = nv * E + threadIdx.x;
            y[e] = tab[x[e]];
        }
    }
}

// QLinearConcat of up to kCatMax inputs in one launch. Input j owns blocks
// [block0_j, block0_j + ceil(nchunks_j / 1024)): its rows (rows of len_j
// bytes, contiguous in x_j) go through the input's requantization table to
// y + o * ystride + yoff_j. len_j, ystride, yoff_j and every pointer are
// multiples of E; nchunks_j = rows * len_j / E < 2^32. A block covers 1024
// chunks, four per lane, loads issued before the table lookups.
constexpr int kCatMax = 8;

struct CatPart {
    const uint8_t* x;
    const float* scale;
    const void* zp;
    uint64_t yoff;
    dq::FastDiv row_chunks;
    uint32_t nchunks;
    uint32_t block0;
};

struct CatArgs {
    CatPart part[kCatMax];
    int n;
    uint64_t ystride;
    const float* y_scale;
    const void* y_zp;
    uint8_t* y;
};

template <bool U8, int E>
__global__ void __launch_bounds__(256) k_concat(CatArgs a) {
    __shared__ uint8_t tab[256];
    int j = 0;
    for (int k = 1; k < a.n; ++k)
        if (blockIdx.x >= a.part[k].block0) j = k;
    const CatPart& p = a.part[j];
    build_table<U8, FN_REQUANT>(tab, TableArgs{p.scale, p.zp, a.y_scale, a.y_zp, 0.0f});
    __syncthreads();
    auto put = [&](uint32_t c, const Bytes<E>& v) {
        const uint32_t o = dq::fdiv(c, p.row_chunks);
        const uint32_t k = c - o * p.row_chunks.d;
        store_bytes<E>(a.y + (uint64_t)o * a.ystride + p.yoff + (uint64_t)k * E, lookup<E>(tab, v));
    };
    const uint32_t base = (blockIdx.x - p.block0) * 1024 + threadIdx.x;
    if (base - threadIdx.x + 1024 <= p.nchunks) {
        Bytes<E> v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = load_bytes<E>(p.x + (uint64_t)(base + q * 256) * E);
        dq::issue_fence();
#pragma unroll
        for (int q = 0; q < 4; ++q) put(base + q * 256, v[q]);
    } else {
        for (uint32_t c = base; c < p.nchunks; c += 256) put(c, load_bytes<E>(p.x + (uint64_t)c * E));
    }
}

// ================================================================= binary

enum { OP_ADD = 0, OP_MUL = 1, OP_MULINT = 2 };

// Canonical broadcast: output dims 0 .. nd-1 (row-major, contiguous
// output); sa / sb are each operand's element strides per dim (0 where it
// broadcasts). The innermost dim has stride 1 or 0 for each operand.
struct BinArgs {
    const uint8_t* a;
    const uint8_t* b;
    void* c;
    const float* a_scale;
    const float* b_scale;
    const float* c_scale;
    const void* a_zp;
    const void* b_zp;
    const void* c_zp;
    uint32_t nd;
    dq::FastDiv dim[kMaxDims];  // sizes of dims 0 .. nd-2
    uint32_t sa[kMaxDims], sb[kMaxDims];
    dq::FastDiv inner_chunks;   // innermost size / E
    uint32_t nchunks;           // output elements / E
};

// element offsets of chunk c in A and B
template <int E>
__device__ __forceinline__ void chunk_offsets(const BinArgs& p, uint32_t c, uint32_t& oa, uint32_t& ob) {
    uint32_t o = dq::fdiv(c, p.inner_chunks);
    const uint32_t i0 = (c - o * p.inner_chunks.d) * E;
    oa = i0 * p.sa[p.nd - 1];
    ob = i0 * p.sb[p.nd - 1];
#pragma unroll
    for (int d = kMaxDims - 2; d >= 0; --d) {
        if (d <= (int)p.nd - 2) {
            const uint32_t q = dq::fdiv(o, p.dim[d]);
            const uint32_t cd = o - q * p.dim[d].d;
            oa += cd * p.sa[d];
            ob += cd * p.sb[d];
            o = q;
        }
    }
}

// E outputs of QLinearAdd / QLinearMul from E bytes of A and B (a broadcast
// operand holds its byte in w[0]); bytes are unsigned here (int8 codes were
// flipped by 0x80 and their zero points moved by 128).
template <int OP, bool FAST, int E, bool AV, bool BV>
__device__ __forceinline__ Bytes<E> quant_chunk(const Bytes<E>& A, const Bytes<E>& B, float za, float zb,
                                                float sa, float sb, float ab, const Quant& q) {
    uint32_t pre[E];
    const float a0 = (float)(A.w[0] & 0xffu) - za;
    const float b0 = (float)(B.w[0] & 0xffu) - zb;
    const float fa0 = a0 * sa, fb0 = b0 * sb;
#pragma unroll
    for (int j = 0; j < E; ++j) {
        const float a = AV ? (float)byte_of(A.w, j) - za : a0;
        const float b = BV ? (float)byte_of(B.w, j) - zb : b0;
        float v;
        if (OP == OP_ADD) {
            const float fa = AV ? a * sa : fa0;
            const float fb = BV ? b * sb : fb0;
            v = fa + fb;
        } else {
            v = (a * b) * ab;
        }
        pre[j] = pre_code<FAST>(v, q);
    }
    Bytes<E> o;
    if constexpr (E == 1) {
        o.w[0] = pack4(pre[0], 0, 0, 0, q.z4) & 0xffu;
    } else {
#pragma unroll
        for (int k = 0; k < E / 4; ++k)
            o.w[k] = pack4(pre[4 * k], pre[4 * k + 1], pre[4 * k + 2], pre[4 * k + 3], q.z4);
    }
    return o;
}

template <int OP, bool U8, int E, bool AV, bool BV>
__global__ void __launch_bounds__(256) k_binary(BinArgs p) {
    constexpr uint32_t kFlip = U8 ? 0u : 0x80808080u;
    const float za = (float)(zp8<U8>(p.a_zp) + (U8 ? 0 : 128));
    const float zb = (float)(zp8<U8>(p.b_zp) + (U8 ? 0 : 128));
    float sa = 0.0f, sb = 0.0f, ab = 0.0f;
    Quant q{};
    if (OP != OP_MULINT) {
        q = make_quant<U8>(p.c_scale, p.c_zp);
        if (OP == OP_ADD) {
            sa = *p.a_scale;
            sb = *p.b_scale;
        } else {
            ab = *p.a_scale * *p.b_scale;
        }
    }
    auto fetch = [&](uint32_t c, Bytes<E>& A, Bytes<E>& B) {
        uint32_t oa, ob;
        chunk_offsets<E>(p, c, oa, ob);
        A = Bytes<E>{};
        B = Bytes<E>{};
        if (AV) A = load_bytes<E>(p.a + oa);
        else A.w[0] = p.a[oa];
        if (BV) B = load_bytes<E>(p.b + ob);
        else B.w[0] = p.b[ob];
    };
    auto put = [&](uint32_t c, Bytes<E> A, Bytes<E> B) {
#pragma unroll
        for (int k = 0; k < (E + 3) / 4; ++k) {
            A.w[k] ^= kFlip;
            B.w[k] ^= kFlip;
        }
        if (OP == OP_MULINT) {
            const int iza = (int)za, izb = (int)zb;
            int32_t r[E];
#pragma unroll
            for (int j = 0; j < E; ++j) {
                const int a = (int)(AV ? byte_of(A.w, j) : (A.w[0] & 0xffu)) - iza;
                const int b = (int)(BV ? byte_of(B.w, j) : (B.w[0] & 0xffu)) - izb;
                r[j] = __mul24(a, b);
            }
            int32_t* out = (int32_t*)p.c + (uint64_t)c * E;
            if constexpr (E == 4) {
                const dq::v4i v = {r[0], r[1], r[2], r[3]};
                *reinterpret_cast<dq::v4i*>(out) = v;
            } else {
#pragma unroll
                for (int j = 0; j < E; ++j) out[j] = r[j];
            }
        } else {
            Bytes<E> o;
            if (q.fast)
                o = quant_chunk<OP, true, E, AV, BV>(A, B, za, zb, sa, sb, ab, q);
            else
                o = quant_chunk<OP, false, E, AV, BV>(A, B, za, zb, sa, sb, ab, q);
            store_bytes<E>((uint8_t*)p.c + (uint64_t)c * E, o);
        }
    };
    // whole block-iterations of 1024 chunks: the eight loads of a lane are
    // issued before any arithmetic; the rest goes to the grid's last block
    const uint32_t nfull = p.nchunks / 1024;
    for (uint32_t it = blockIdx.x; it < nfull; it += gridDim.x) {
        const uint32_t base = it * 1024 + threadIdx.x;
        Bytes<E> A[4], B[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) fetch(base + u * 256, A[u], B[u]);
        dq::issue_fence();
#pragma unroll
        for (int u = 0; u < 4; ++u) put(base + u * 256, A[u], B[u]);
    }
    if (blockIdx.x == gridDim.x - 1) {
        for (uint32_t c = nfull * 1024 + threadIdx.x; c < p.nchunks; c += 256) {
            Bytes<E> A, B;
            fetch(c, A, B);
            put(c, A, B);
        }
    }
}

// ============================================================== reductions

struct RedArgs {
    const uint8_t* x;
    void* y;               // int32 / uint32 sums, or 8-bit means
    const float* x_scale;  // the mean's parameters
    const void* x_zp;
    const float* y_scale;
    const void* y_zp;
    uint64_t count;        // elements per output
};

// output `idx` from the raw-code sum `s` (int32, wrapping) of `count` codes
template <bool U8, int MODE>
__device__ __forceinline__ void finish(const RedArgs& a, uint64_t idx, int32_t s) {
    if (MODE == 0) {
        ((int32_t*)a.y)[idx] = s;
    } else {
        const int64_t S = (int64_t)s - (int64_t)zp8<U8>(a.x_zp) * (int64_t)a.count;
        const float mean = (float)(((double)S * (double)*a.x_scale) / (double)a.count);
        ((uint8_t*)a.y)[idx] = (uint8_t)quant_exact(mean, *a.y_scale, zp8<U8>(a.y_zp), U8);
    }
}

template <bool U8, int E>
__device__ __forceinline__ int32_t sum_bytes(const Bytes<E>& b, int32_t acc) {
    if constexpr (E == 1) {
        return acc + code8<U8>(b.w[0]);
    } else {
#pragma unroll
        for (int k = 0; k < E / 4; ++k) {
            if (U8)
                acc = (int32_t)__builtin_amdgcn_udot4(b.w[k], 0x01010101u, (uint32_t)acc, false);
            else
                acc = __builtin_amdgcn_sdot4((int)b.w[k], 0x01010101, acc, false);
        }
        return acc;
    }
}

// Rows: X is [O, R] (R = a.count), G lanes per row, E-byte chunks (R % E
// == 0, x E-aligned); a 256-thread block covers 256 / G rows.
template <bool U8, int MODE, int G, int E>
__global__ void __launch_bounds__(256) k_reduce_rows(RedArgs a, uint32_t O) {
    const uint32_t row = blockIdx.x * (256 / G) + threadIdx.x / G;
    const uint32_t li = threadIdx.x % G;
    const uint32_t rr = row < O ? row : O - 1;
    const uint64_t nch = a.count / E;
    const uint8_t* xr = a.x + (uint64_t)rr * a.count;
    int32_t acc = 0;
    for (uint64_t k0 = li; k0 < nch; k0 += 4 * G) {
        Bytes<E> v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint64_t k = std::min(k0 + (uint64_t)u * G, nch - 1);
            v[u] = load_bytes<E>(xr + k * E);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int32_t s = sum_bytes<U8, E>(v[u], 0);
            acc += k0 + (uint64_t)u * G < nch ? s : 0;
        }
    }
#pragma unroll
    for (int m = G / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
    if (li == 0 && row < O) finish<U8, MODE>(a, row, acc);
}

// Short rows that are not a multiple of 16 bytes (e.g. 7 x 7 pooling): a
// block's rows [row0, row0 + nrows) are one contiguous span of the tensor,
// read in aligned 16-byte windows (bytewise only for a window that crosses
// the tensor's end) into LDS; a thread then sums a row from LDS as 4-byte
// words, masking the bytes of its neighbours in the first and last word.
// x is 16-aligned; rows_per_block * count + 32 <= kStageBytes.
constexpr uint32_t kStageBytes = 8192 + 32;

template <bool U8, int MODE>
__global__ void __launch_bounds__(256) k_reduce_rows_staged(RedArgs a, uint32_t O, uint32_t rows_per_block) {
    __shared__ uint32_t span[kStageBytes / 4];
    const uint64_t R = a.count;
    const uint64_t n = (uint64_t)O * R;
    const uint32_t row0 = blockIdx.x * rows_per_block;
    const uint32_t nrows = std::min(rows_per_block, O - row0);
    const uint64_t start = (uint64_t)row0 * R, end = start + (uint64_t)nrows * R;
    const uint64_t ws = start & ~(uint64_t)15;
    const uint32_t nw = (uint32_t)((((end + 15) & ~(uint64_t)15) - ws) / 16);
    for (uint32_t w = threadIdx.x; w < nw; w += 256) {
        const uint64_t off = ws + 16 * (uint64_t)w;
        Bytes<16> v;
        if (off + 16 <= n) {
            v = load_bytes<16>(a.x + off);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                uint32_t word = 0;
                for (int b = 0; b < 4; ++b) {
                    const uint64_t e = off + 4 * k + b;
                    if (e < n) word |= (uint32_t)a.x[e] << (8 * b);
                }
                v.w[k] = word;
            }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) span[4 * w + k] = v.w[k];
    }
    __syncthreads();
    for (uint32_t r = threadIdx.x; r < nrows; r += 256) {
        const uint32_t b0 = (uint32_t)((uint64_t)(row0 + r) * R - ws), b1 = b0 + (uint32_t)R;
        int32_t acc = 0;
        for (uint32_t d = b0 / 4; d < (b1 + 3) / 4; ++d) {
            const int lo = (int)std::max<int64_t>((int64_t)b0 - 4 * (int64_t)d, 0);
            const int hi = (int)std::min<int64_t>((int64_t)b1 - 4 * (int64_t)d, 4);
            const uint32_t mask = (hi == 4 ? 0xffffffffu : ((1u << (8 * hi)) - 1u)) & ~((1u << (8 * lo)) - 1u);
            Bytes<4> b;
            b.w[0] = span[d] & mask;
            acc = sum_bytes<U8, 4>(b, acc);
        }
        finish<U8, MODE>(a, row0 + r, acc);
    }
}

// Columns: X is [O, R, I] (R = a.count), I % E == 0, x E-aligned. Block
// (blockIdx.x = o * gx + column block, part = blockIdx.z): CW lanes over E-column
// chunks times 256 / CW lanes over rows, U rows a lane in flight; rows
// [r0, r1) of part z. The partial sums meet in LDS; ATOMIC adds each
// column's block sum into y.
template <int E>
struct ColAcc {
    uint32_t lo[(E + 3) / 4], hi[(E + 3) / 4];  // 16-bit pairs: bytes 0,2 and 1,3
    int32_t tot[E];
};

template <bool U8, int MODE, int E, bool ATOMIC, int U>
__global__ void __launch_bounds__(256)
k_reduce_cols(RedArgs a, uint32_t I, uint32_t CW, uint32_t gx, uint32_t rows_per_part) {
    __shared__ int32_t part[256 * E];
    constexpr uint32_t kFlip = U8 ? 0u : 0x80808080u;
    const uint32_t cl = threadIdx.x % CW, rs = threadIdx.x / CW, RS = 256 / CW;
    const uint32_t nchunks = I / E;
    const uint32_t o = blockIdx.x / gx;
    const uint32_t j = (blockIdx.x - o * gx) * CW + cl;
    const uint32_t jc = j < nchunks ? j : nchunks - 1;
    const uint64_t R = a.count;
    const uint64_t r0 = (uint64_t)blockIdx.z * rows_per_part;
    const uint64_t r1 = std::min(R, r0 + rows_per_part);
    const uint8_t* xo = a.x + (uint64_t)o * R * I + (uint64_t)jc * E;
    ColAcc<E> c;
#pragma unroll
    for (int k = 0; k < (E + 3) / 4; ++k) c.lo[k] = c.hi[k] = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) c.tot[e] = 0;
    uint32_t pending = 0;  // rows in the 16-bit partial sums (at most 255)
    for (uint64_t rb = r0 + rs; rb < r1; rb += U * RS) {
        Bytes<E> v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint64_t r = std::min(rb + (uint64_t)u * RS, r1 - 1);
            v[u] = load_bytes<E>(xo + r * I);
        }
        dq::issue_fence();
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool ok = rb + (uint64_t)u * RS < r1;
            if constexpr (E == 1) {
                c.tot[0] += ok ? code8<U8>(v[u].w[0]) : 0;
            } else {
#pragma unroll
                for (int k = 0; k < E / 4; ++k) {
                    const uint32_t w = ok ? (v[u].w[k] ^ kFlip) : 0u;
                    c.lo[k] += w & 0x00ff00ffu;
                    c.hi[k] += (w >> 8) & 0x00ff00ffu;
                }
            }
        }
        if (E > 1 && (pending += U) > 255 - U) {
#pragma unroll
            for (int k = 0; k < E / 4; ++k) {
                c.tot[4 * k] += (int32_t)(c.lo[k] & 0xffffu);
                c.tot[4 * k + 2] += (int32_t)(c.lo[k] >> 16);
                c.tot[4 * k + 1] += (int32_t)(c.hi[k] & 0xffffu);
                c.tot[4 * k + 3] += (int32_t)(c.hi[k] >> 16);
                c.lo[k] = c.hi[k] = 0;
            }
            pending = 0;
        }
    }
    if constexpr (E > 1) {
#pragma unroll
        for (int k = 0; k < E / 4; ++k) {
            c.tot[4 * k] += (int32_t)(c.lo[k] & 0xffffu);
            c.tot[4 * k + 2] += (int32_t)(c.lo[k] >> 16);
            c.tot[4 * k + 1] += (int32_t)(c.hi[k] & 0xffffu);
            c.tot[4 * k + 3] += (int32_t)(c.hi[k] >> 16);
        }
        if (!U8) {
            // the flipped bytes counted code + 128 for each of this lane's rows
            const uint64_t mine = r1 > r0 + rs ? (r1 - r0 - rs + RS - 1) / RS : 0;
#pragma unroll
            for (int e = 0; e < E; ++e) c.tot[e] -= (int32_t)(128u * (uint32_t)mine);
        }
    }
    // part[rs][col], col = cl * E + e over the block's CW * E columns: every
    // thread then sums the RS partials of its columns
#pragma unroll
    for (int e = 0; e < E; ++e) part[threadIdx.x * E + e] = c.tot[e];
    __syncthreads();
    const uint32_t ncol = CW * E;
    for (uint32_t col = threadIdx.x; col < ncol; col += 256) {
        int32_t s = 0;
        for (uint32_t t = 0; t < RS; ++t) s += part[t * ncol + col];
        const uint32_t jj = (blockIdx.x - o * gx) * CW + col / E;
        if (jj < nchunks) {
            const uint64_t idx = (uint64_t)o * I + (uint64_t)jj * E + col % E;
            if (ATOMIC)
                atomicAdd((int32_t*)a.y + idx, s);
            else
                finish<U8, MODE>(a, idx, s);
        }
    }
}

// Any set of axes: one wave per output. Canonical dims (size-1 dims
// dropped, neighbours of one kind merged): kept dims kd[0..nk) and reduced
// dims rd[0..nr), each with its input stride; output index -> kept
// coordinates, lane t -> reduced coordinates, by multiply-high division.
struct GenShape {
    uint32_t nk, nr;
    dq::FastDiv kd[kMaxDims], rd[kMaxDims];
    uint64_t ks[kMaxDims], rsd[kMaxDims];
};

template <bool U8, int MODE>
__global__ void __launch_bounds__(256) k_reduce_general(RedArgs a, GenShape g, uint32_t nout) {
    const uint32_t out = blockIdx.x * 4 + threadIdx.x / 64;
    const uint32_t lane = threadIdx.x % 64;
    const uint32_t oc = out < nout ? out : nout - 1;
    uint64_t base = 0;
    uint32_t o = oc;
    for (int d = (int)g.nk - 1; d >= 0; --d) {
        const uint32_t q = dq::fdiv(o, g.kd[d]);
        base += (uint64_t)(o - q * g.kd[d].d) * g.ks[d];
        o = q;
    }
    int32_t acc = 0;
    for (uint64_t t = lane; t < a.count; t += 64) {
        uint32_t r = (uint32_t)t;
        uint64_t off = base;
        for (int d = (int)g.nr - 1; d >= 0; --d) {
            const uint32_t q = dq::fdiv(r, g.rd[d]);
            off += (uint64_t)(r - q * g.rd[d].d) * g.rsd[d];
            r = q;
        }
        acc += code8<U8>(a.x[off]);
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
    if (lane == 0 && out < nout) finish<U8, MODE>(a, out, acc);
}

__global__ void __launch_bounds__(256) k_fill_zero32(int32_t* y, uint64_t n) {
    const uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) y[i] = 0;
}

// ------------------------------------------------------------------- host

int check_type8(dq_dtype t, const char* what) {
    if (t != DQ_U8 && t != DQ_I8) DQ_FAIL(DQ_ERR_TYPE, "%s: type must be int8 or uint8", what);
    return DQ_OK;
}

int tensor_size(int ndim, const int64_t* shape, uint64_t* n, const char* what) {
    if (ndim < 0 || ndim > kMaxDims) DQ_FAIL(DQ_ERR_ARG, "%s: ndim must be in [0, 8], got %d", what, ndim);
    if (ndim > 0 && !shape) DQ_FAIL(DQ_ERR_ARG, "%s: shape is NULL", what);
    uint64_t v = 1;
    for (int d = 0; d < ndim; ++d) {
        if (shape[d] < 0) DQ_FAIL(DQ_ERR_ARG, "%s: shape[%d] is negative", what, d);
        if (shape[d] != 0 && v > (UINT64_C(1) << 40) / (uint64_t)shape[d])
            DQ_FAIL(DQ_ERR_RANGE, "%s: tensor larger than 2^40 elements", what);
        v *= (uint64_t)shape[d];
    }
    *n = v;
    return DQ_OK;
}

int vec_width(uint64_t len, std::initializer_list<uintptr_t> ptrs, int max_e) {
    for (int e : {16, 4}) {
        if (e > max_e || len % e) continue;
        bool ok = true;
        for (uintptr_t p : ptrs) ok = ok && p % e == 0;
        if (ok) return e;
    }
    return 1;
}

// ---- one-code functions

template <int F>
int launch_table(const void* x, uint64_t n, const TableArgs& ta, dq_dtype type, void* y, hipStream_t s,
                 const char* name) {
    const int E = ((uintptr_t)x % 16 == 0 && (uintptr_t)y % 16 == 0) ? 16 : 1;
    const uint64_t want = (n / E + 1023) / 1024;
    const bool u8 = type == DQ_U8;
#define DQ_TM(U, EE)                                                                              \
    do {                                                                                          \
        const unsigned g = (unsigned)std::max<uint64_t>(                                          \
            1, std::min<uint64_t>(want, resident_blocks(k_table_map<U, F, EE>, 256)));            \
        hipLaunchKernelGGL((k_table_map<U, F, EE>), dim3(g), dim3(256), 0, s, (const uint8_t*)x, \
                           n, ta, (uint8_t*)y);                                                   \
    } while (0)
    if (u8) {
        if (E == 16) DQ_TM(true, 16);
        else DQ_TM(true, 1);
    } else {
        if (E == 16) DQ_TM(false, 16);
        else DQ_TM(false, 1);
    }
#undef DQ_TM
    DQ_LAUNCH_CHECK(name);
    return DQ_OK;
}

int unary_common(const void* x, int64_t n, const float* x_scale, const float* y_scale, dq_dtype type,
                 void* y, const char* name) {
    int rc = check_type8(type, name);
    if (rc) return rc;
    if (n < 0) DQ_FAIL(DQ_ERR_ARG, "%s: n is negative", name);
    if (n > 0 && (!x || !y || !x_scale || !y_scale))
        DQ_FAIL(DQ_ERR_ARG, "%s: x, y, x_scale and y_scale must not be NULL", name);
    return DQ_OK;
}

// ---- binary

struct Canon {
    int nd;
    uint64_t size[kMaxDims];
    uint64_t sa[kMaxDims], sb[kMaxDims];
    uint64_t n;
};

int canon_broadcast(int na, const int64_t* sha, int nb, const int64_t* shb, Canon* c, int64_t* yshape,
                    int* yndim) {
    const int ny = std::max(na, nb);
    int64_t ys[kMaxDims];
    uint64_t sa[kMaxDims], sb[kMaxDims];
    uint64_t ta = 1, tb = 1;
    for (int d = ny - 1; d >= 0; --d) {
        const int64_t a = d - (ny - na) >= 0 ? sha[d - (ny - na)] : 1;
        const int64_t b = d - (ny - nb) >= 0 ? shb[d - (ny - nb)] : 1;
        if (a != b && a != 1 && b != 1)
            DQ_FAIL(DQ_ERR_ARG, "shapes do not broadcast (dim %d: %lld vs %lld)", d, (long long)a,
                    (long long)b);
        ys[d] = a == 1 ? b : a;
        sa[d] = a == 1 ? 0 : ta;
        sb[d] = b == 1 ? 0 : tb;
        ta *= (uint64_t)a;
        tb *= (uint64_t)b;
    }
    for (int d = 0; d < ny; ++d) yshape[d] = ys[d];
    *yndim = ny;
    // drop size-1 dims, merge neighbours that continue contiguously in both
    c->nd = 0;
    c->n = 1;
    for (int d = 0; d < ny; ++d) {
        c->n *= (uint64_t)ys[d];
        if (ys[d] == 1) continue;
        const int k = c->nd;
        if (k > 0 && c->sa[k - 1] == sa[d] * (uint64_t)ys[d] && c->sb[k - 1] == sb[d] * (uint64_t)ys[d]) {
            c->size[k - 1] *= (uint64_t)ys[d];
            c->sa[k - 1] = sa[d];
            c->sb[k - 1] = sb[d];
        } else {
            c->size[k] = (uint64_t)ys[d];
            c->sa[k] = sa[d];
            c->sb[k] = sb[d];
            c->nd = k + 1;
        }
    }
    if (c->nd == 0) {  // one element
        c->nd = 1;
        c->size[0] = 1;
        c->sa[0] = c->sb[0] = 1;
    }
    return DQ_OK;
}

int run_binary(int op, const void* A, int a_ndim, const int64_t* a_shape, const float* a_scale,
               const void* a_zp, const void* B, int b_ndim, const int64_t* b_shape, const float* b_scale,
               const void* b_zp, const float* c_scale, const void* c_zp, dq_dtype type, void* C,
               void* stream, const char* name) {
    int rc = check_type8(type, name);
    if (rc) return rc;
    uint64_t na, nb;
    if ((rc = tensor_size(a_ndim, a_shape, &na, name))) return rc;
    if ((rc = tensor_size(b_ndim, b_shape, &nb, name))) return rc;
    Canon cn;
    int64_t ys[kMaxDims];
    int yn;
    if ((rc = canon_broadcast(a_ndim, a_shape, b_ndim, b_shape, &cn, ys, &yn))) return rc;
    if (cn.n == 0) return DQ_OK;
    if (cn.n >= (UINT64_C(1) << 32)) DQ_FAIL(DQ_ERR_RANGE, "%s: output of 2^32 or more elements", name);
    if (!A || !B || !C) DQ_FAIL(DQ_ERR_ARG, "%s: A, B and C must not be NULL", name);
    if (op != OP_MULINT && (!c_scale || !a_scale || !b_scale))
        DQ_FAIL(DQ_ERR_ARG, "%s: the scales must not be NULL", name);
    BinArgs p{};
    p.a = (const uint8_t*)A;
    p.b = (const uint8_t*)B;
    p.c = C;
    p.a_scale = a_scale;
    p.b_scale = b_scale;
    p.c_scale = c_scale;
    p.a_zp = a_zp;
    p.b_zp = b_zp;
    p.c_zp = c_zp;
    p.nd = (uint32_t)cn.nd;
    const int in = cn.nd - 1;
    const bool av = cn.sa[in] == 1, bv = cn.sb[in] == 1;
    // vector width: the innermost size and every vector operand's pointer
    const uint64_t inner = cn.size[in];
    const int max_e = op == OP_MULINT ? 4 : 16;
    int E = 1;
    for (int e : {16, 4}) {
        if (e > max_e || inner % e) continue;
        const uintptr_t cbytes = op == OP_MULINT ? 4 * (uintptr_t)e : (uintptr_t)e;
        if ((av && (uintptr_t)A % e) || (bv && (uintptr_t)B % e) || (uintptr_t)C % cbytes) continue;
        E = e;
        break;
    }
    for (int d = 0; d < cn.nd; ++d) {
        p.dim[d] = dq::make_fastdiv((uint32_t)cn.size[d]);
        p.sa[d] = (uint32_t)cn.sa[d];
        p.sb[d] = (uint32_t)cn.sb[d];
    }
    p.inner_chunks = dq::make_fastdiv((uint32_t)(inner / E));
    p.nchunks = (uint32_t)(cn.n / E);
    hipStream_t s = (hipStream_t)stream;
    const uint64_t want = ((uint64_t)p.nchunks + 1023) / 1024;
    const bool u8 = type == DQ_U8;
#define DQ_BIN(OPV, U, EE, AVV, BVV)                                                               \
    do {                                                                                           \
        const unsigned g = (unsigned)std::max<uint64_t>(                                           \
            1, std::min<uint64_t>(want, resident_blocks(k_binary<OPV, U, EE, AVV, BVV>, 256)));    \
        hipLaunchKernelGGL((k_binary<OPV, U, EE, AVV, BVV>), dim3(g), dim3(256), 0, s, p);         \
    } while (0)
#define DQ_BIN_AB(OPV, U, EE)                       \
    do {                                            \
        if (av && bv) DQ_BIN(OPV, U, EE, true, true);  \
        else if (av) DQ_BIN(OPV, U, EE, true, false);  \
        else DQ_BIN(OPV, U, EE, false, true);          \
    } while (0)
#define DQ_BIN_E(OPV, U)                            \
    do {                                            \
        if (E == 16) DQ_BIN_AB(OPV, U, 16);         \
        else if (E == 4) DQ_BIN_AB(OPV, U, 4);      \
        else DQ_BIN_AB(OPV, U, 1);                  \
    } while (0)
    if (op == OP_ADD) {
        if (u8) DQ_BIN_E(OP_ADD, true);
        else DQ_BIN_E(OP_ADD, false);
    } else if (op == OP_MUL) {
        if (u8) DQ_BIN_E(OP_MUL, true);
        else DQ_BIN_E(OP_MUL, false);
    } else {
        if (u8) {
            if (E == 4) DQ_BIN_AB(OP_MULINT, true, 4);
            else DQ_BIN_AB(OP_MULINT, true, 1);
        } else {
            if (E == 4) DQ_BIN_AB(OP_MULINT, false, 4);
            else DQ_BIN_AB(OP_MULINT, false, 1);
        }
    }
#undef DQ_BIN_E
#undef DQ_BIN_AB
#undef DQ_BIN
    DQ_LAUNCH_CHECK(name);
    return DQ_OK;
}

// ---- reductions

int run_reduce(int mode, const void* x, dq_dtype type, int ndim, const int64_t* shape, const int32_t* axes,
               int n_axes, const float* x_scale, const void* x_zp, const float* y_scale, const void* y_zp,
               void* y, void* stream, const char* name) {
    int rc = check_type8(type, name);
    if (rc) return rc;
    if (ndim < 1) DQ_FAIL(DQ_ERR_ARG, "%s: ndim must be in [1, 8], got %d", name, ndim);
    uint64_t n;
    if ((rc = tensor_size(ndim, shape, &n, name))) return rc;
    if (n_axes < 0 || (n_axes > 0 && !axes)) DQ_FAIL(DQ_ERR_ARG, "%s: bad axes list", name);
    unsigned mask = 0;
    if (n_axes == 0) mask = (1u << ndim) - 1;
    for (int i = 0; i < n_axes; ++i) {
        const int ax = axes[i];
        if (ax < -ndim || ax >= ndim) DQ_FAIL(DQ_ERR_RANGE, "%s: axis %d out of range", name, ax);
        mask |= 1u << (ax < 0 ? ax + ndim : ax);
    }
    uint64_t nout = 1, count = 1;
    for (int d = 0; d < ndim; ++d) (mask >> d & 1 ? count : nout) *= (uint64_t)shape[d];
    if (nout == 0) return DQ_OK;
    if (!y) DQ_FAIL(DQ_ERR_ARG, "%s: y must not be NULL", name);
    if (mode == 1) {
        if (count == 0) DQ_FAIL(DQ_ERR_ARG, "%s: the mean over an empty axis is undefined", name);
        if (count > (UINT64_C(1) << 23)) DQ_FAIL(DQ_ERR_RANGE, "%s: more than 2^23 elements per mean", name);
        if (!x_scale || !y_scale) DQ_FAIL(DQ_ERR_ARG, "%s: x_scale and y_scale must not be NULL", name);
    }
    if (nout >= (UINT64_C(1) << 31)) DQ_FAIL(DQ_ERR_RANGE, "%s: 2^31 or more outputs", name);
    if (count >= (UINT64_C(1) << 32)) DQ_FAIL(DQ_ERR_RANGE, "%s: 2^32 or more elements per output", name);
    hipStream_t s = (hipStream_t)stream;
    if (count == 0) {  // sums of nothing
        hipLaunchKernelGGL(k_fill_zero32, dim3((unsigned)((nout + 255) / 256)), dim3(256), 0, s, (int32_t*)y,
                           nout);
        DQ_LAUNCH_CHECK(name);
        return DQ_OK;
    }
    if (!x) DQ_FAIL(DQ_ERR_ARG, "%s: x must not be NULL", name);
    // canonical groups
    uint64_t gs[kMaxDims];
    int gk[kMaxDims], ng = 0;
    for (int d = 0; d < ndim; ++d) {
        if (shape[d] == 1) continue;
        const int kind = mask >> d & 1;
        if (ng > 0 && gk[ng - 1] == kind) {
            gs[ng - 1] *= (uint64_t)shape[d];
        } else {
            gs[ng] = (uint64_t)shape[d];
            gk[ng++] = kind;
        }
    }
    int nred = 0, rg = -1;
    for (int i = 0; i < ng; ++i)
        if (gk[i]) ++nred, rg = i;
    RedArgs a{(const uint8_t*)x, y, x_scale, x_zp, y_scale, y_zp, count};
    const bool u8 = type == DQ_U8;
    if (nred <= 1) {
        uint64_t O = 1, I = 1;
        for (int i = 0; i < ng; ++i) {
            if (i < rg) O *= gs[i];
            if (i > rg && rg >= 0) I *= gs[i];
        }
        if (rg < 0) O = n;  // nothing reduced: every output is one element
        if (I == 1 && count % 16 != 0 && count <= 4096 && (uintptr_t)x % 16 == 0) {
            const uint32_t rpb = (uint32_t)std::min<uint64_t>(O, (kStageBytes - 32) / count);
            const unsigned blocks = (unsigned)((O + rpb - 1) / rpb);
#define DQ_STAGED(U, M) \
    hipLaunchKernelGGL((k_reduce_rows_staged<U, M>), dim3(blocks), dim3(256), 0, s, a, (uint32_t)O, rpb)
            if (mode == 0) {
                if (u8) DQ_STAGED(true, 0);
                else DQ_STAGED(false, 0);
            } else {
                if (u8) DQ_STAGED(true, 1);
                else DQ_STAGED(false, 1);
            }
#undef DQ_STAGED
            DQ_LAUNCH_CHECK(name);
            return DQ_OK;
        }
        if (I == 1) {
            const int E = vec_width(count, {(uintptr_t)x}, 16);
            const uint64_t nch = count / E;
            int G = 1;
            while (G < 64 && (uint64_t)G * 8 < nch) G *= 2;
            const unsigned blocks = (unsigned)((O + 256 / G - 1) / (256 / G));
#define DQ_ROWS(U, M, GG, EE) \
    hipLaunchKernelGGL((k_reduce_rows<U, M, GG, EE>), dim3(blocks), dim3(256), 0, s, a, (uint32_t)O)
#define DQ_ROWS_G(U, M, EE)                 \
    do {                                    \
        switch (G) {                        \
            case 1: DQ_ROWS(U, M, 1, EE); break;  \
            case 2: DQ_ROWS(U, M, 2, EE); break;  \
            case 4: DQ_ROWS(U, M, 4, EE); break;  \
            case 8: DQ_ROWS(U, M, 8, EE); break;  \
            case 16: DQ_ROWS(U, M, 16, EE); break; \
            case 32: DQ_ROWS(U, M, 32, EE); break; \
            default: DQ_ROWS(U, M, 64, EE); break; \
        }                                   \
    } while (0)
#define DQ_ROWS_E(U, M)                        \
    do {                                       \
        if (E == 16) DQ_ROWS_G(U, M, 16);      \
        else if (E == 4) DQ_ROWS_G(U, M, 4);   \
        else DQ_ROWS_G(U, M, 1);               \
    } while (0)
            if (mode == 0) {
                if (u8) DQ_ROWS_E(true, 0);
                else DQ_ROWS_E(false, 0);
            } else {
                if (u8) DQ_ROWS_E(true, 1);
                else DQ_ROWS_E(false, 1);
            }
#undef DQ_ROWS_E
#undef DQ_ROWS_G
#undef DQ_ROWS
            DQ_LAUNCH_CHECK(name);
            return DQ_OK;
        }
        // columns
        const int E = vec_width(I, {(uintptr_t)x}, 16);
        const uint64_t nch = I / E;
        // CW lanes side by side over a row (64: a wave reads 1 KiB of a row
        // at 16 bytes a lane); the other 256 / CW lanes of the block take
        // rows in turn. The sum fills the chip by splitting rows over
        // workgroups; the mean narrows CW instead, down to 8 lanes (128
        // bytes a row), while the grid would not fill it
        uint32_t CW = 1;
        while (CW < 64 && CW < nch) CW *= 2;
        if (mode == 1)  // the mean cannot split rows over workgroups
            while (CW > 8 && O * ((nch + CW - 1) / CW) < 2048) CW /= 2;
        const uint64_t gx = (nch + CW - 1) / CW;
        if (gx * O >= (UINT64_C(1) << 31) || I >= (UINT64_C(1) << 32))
            DQ_FAIL(DQ_ERR_RANGE, "%s: shape beyond the column kernel's grid", name);
        // ReduceSumInteger splits long columns over workgroups when the
        // grid would not fill the chip
        // ... with at least one step of sixteen rows a lane per part (a
        // lane keeps sixteen 16-byte loads in flight), which bounds the
        // atomics to one per column per 16 * 256 / CW rows; finer parts
        // measured slower (the atomics), coarser ones left the loads of a
        // CU too few to cover the memory latency
        uint64_t parts = 1;
        if (mode == 0) {
            const uint64_t blocks = gx * O;
            const uint64_t rows_min = 16 * (256 / CW);
            while (blocks * parts < 2048 && count / (parts * 2) >= rows_min && parts < 65535) parts *= 2;
        }
        const uint64_t rpp = (count + parts - 1) / parts;
        if (parts > 1) {
            hipLaunchKernelGGL(k_fill_zero32, dim3((unsigned)((nout + 255) / 256)), dim3(256), 0, s,
                               (int32_t*)y, nout);
            DQ_LAUNCH_CHECK(name);
        }
        const dim3 grid((unsigned)(gx * O), 1, (unsigned)parts);
#define DQ_COLS(U, M, EE, AT) \
    hipLaunchKernelGGL((k_reduce_cols<U, M, EE, AT, (AT ? 16 : 4)>), grid, dim3(256), 0, s, a, (uint32_t)I, \
                       CW, (uint32_t)gx, (uint32_t)rpp)
#define DQ_COLS_E(U, M, AT)                     \
    do {                                        \
        if (E == 16) DQ_COLS(U, M, 16, AT);     \
        else if (E == 4) DQ_COLS(U, M, 4, AT);  \
        else DQ_COLS(U, M, 1, AT);              \
    } while (0)
        if (mode == 0) {
            if (parts > 1) {
                if (u8) DQ_COLS_E(true, 0, true);
                else DQ_COLS_E(false, 0, true);
            } else {
                if (u8) DQ_COLS_E(true, 0, false);
                else DQ_COLS_E(false, 0, false);
            }
        } else {
            if (u8) DQ_COLS_E(true, 1, false);
            else DQ_COLS_E(false, 1, false);
        }
#undef DQ_COLS_E
#undef DQ_COLS
        DQ_LAUNCH_CHECK(name);
        return DQ_OK;
    }
    // general: kept and reduced dims with their strides
    GenShape g{};
    uint64_t stride = 1;
    int dims_k = 0, dims_r = 0;
    uint64_t ks[kMaxDims], rs[kMaxDims], ksz[kMaxDims], rsz[kMaxDims];
    for (int d = ndim - 1; d >= 0; --d) {
        if (shape[d] != 1) {
            if (mask >> d & 1) {
                rsz[dims_r] = (uint64_t)shape[d];
                rs[dims_r++] = stride;
            } else {
                ksz[dims_k] = (uint64_t)shape[d];
                ks[dims_k++] = stride;
            }
        }
        stride *= (uint64_t)shape[d];
    }
    // innermost-first above; the kernel wants outermost-first
    g.nk = (uint32_t)dims_k;
    g.nr = (uint32_t)dims_r;
    for (int i = 0; i < dims_k; ++i) {
        g.kd[i] = dq::make_fastdiv((uint32_t)ksz[dims_k - 1 - i]);
        g.ks[i] = ks[dims_k - 1 - i];
    }
    for (int i = 0; i < dims_r; ++i) {
        g.rd[i] = dq::make_fastdiv((uint32_t)rsz[dims_r - 1 - i]);
        g.rsd[i] = rs[dims_r - 1 - i];
    }
    const unsigned blocks = (unsigned)((nout + 3) / 4);
#define DQ_GEN(U, M) hipLaunchKernelGGL((k_reduce_general<U, M>), dim3(blocks), dim3(256), 0, s, a, g, (uint32_t)nout)
    if (mode == 0) {
        if (u8) DQ_GEN(true, 0);
        else DQ_GEN(false, 0);
    } else {
        if (u8) DQ_GEN(true, 1);
        else DQ_GEN(false, 1);
    }
#undef DQ_GEN
    DQ_LAUNCH_CHECK(name);
    return DQ_OK;
}

}  // namespace

// =============================================================== C ABI

extern "C" int qlinear_add(const void* A, int a_ndim, const int64_t* a_shape, const float* a_scale,
                           const void* a_zero_point, const void* B, int b_ndim, const int64_t* b_shape,
                           const float* b_scale, const void* b_zero_point, const float* c_scale,
                           const void* c_zero_point, dq_dtype type, void* C, void* stream) {
    return run_binary(OP_ADD, A, a_ndim, a_shape, a_scale, a_zero_point, B, b_ndim, b_shape, b_scale,
                      b_zero_point, c_scale, c_zero_point, type, C, stream, "qlinear_add");
}

extern "C" int qlinear_mul(const void* A, int a_ndim, const int64_t* a_shape, const float* a_scale,
                           const void* a_zero_point, const void* B, int b_ndim, const int64_t* b_shape,
                           const float* b_scale, const void* b_zero_point, const float* c_scale,
                           const void* c_zero_point, dq_dtype type, void* C, void* stream) {
    return run_binary(OP_MUL, A, a_ndim, a_shape, a_scale, a_zero_point, B, b_ndim, b_shape, b_scale,
                      b_zero_point, c_scale, c_zero_point, type, C, stream, "qlinear_mul");
}

extern "C" int dq_mul_integer(const void* A, int a_ndim, const int64_t* a_shape, const void* a_zero_point,
                              const void* B, int b_ndim, const int64_t* b_shape, const void* b_zero_point,
                              dq_dtype type, int32_t* C, void* stream) {
    return run_binary(OP_MULINT, A, a_ndim, a_shape, nullptr, a_zero_point, B, b_ndim, b_shape, nullptr,
                      b_zero_point, nullptr, nullptr, type, C, stream, "mul_integer");
}

extern "C" int qlinear_leaky_relu(const void* x, int64_t n, const float* x_scale, const void* x_zero_point,
                                  const float* y_scale, const void* y_zero_point, float alpha,
                                  dq_dtype type, void* y, void* stream) {
    int rc = unary_common(x, n, x_scale, y_scale, type, y, "qlinear_leaky_relu");
    if (rc || n == 0) return rc;
    const TableArgs ta{x_scale, x_zero_point, y_scale, y_zero_point, alpha};
    return launch_table<FN_LEAKY>(x, (uint64_t)n, ta, type, y, (hipStream_t)stream, "qlinear_leaky_relu");
}

extern "C" int qlinear_sigmoid(const void* x, int64_t n, const float* x_scale, const void* x_zero_point,
                               const float* y_scale, const void* y_zero_point, dq_dtype type, void* y,
                               void* stream) {
    int rc = unary_common(x, n, x_scale, y_scale, type, y, "qlinear_sigmoid");
    if (rc || n == 0) return rc;
    const TableArgs ta{x_scale, x_zero_point, y_scale, y_zero_point, 0.0f};
    return launch_table<FN_SIGMOID>(x, (uint64_t)n, ta, type, y, (hipStream_t)stream, "qlinear_sigmoid");
}

extern "C" int dq_reduce_sum_integer(const void* x, dq_dtype type, int ndim, const int64_t* shape,
                                     const int32_t* axes, int n_axes, void* y, void* stream) {
    return run_reduce(0, x, type, ndim, shape, axes, n_axes, nullptr, nullptr, nullptr, nullptr, y, stream,
                      "reduce_sum_integer");
}

extern "C" int qlinear_reduce_mean(const void* x, dq_dtype type, int ndim, const int64_t* shape,
                                   const int32_t* axes, int n_axes, const float* x_scale,
                                   const void* x_zero_point, const float* y_scale, const void* y_zero_point,
                                   void* y, void* stream) {
    return run_reduce(1, x, type, ndim, shape, axes, n_axes, x_scale, x_zero_point, y_scale, y_zero_point, y,
                      stream, "qlinear_reduce_mean");
}

extern "C" int qlinear_concat(int n_inputs, const void* const* xs, const int64_t* shapes, int ndim, int axis,
                              const float* const* x_scales, const void* const* x_zero_points,
                              const float* y_scale, const void* y_zero_point, dq_dtype type, void* y,
                              void* stream) {
    const char* name = "qlinear_concat";
    int rc = check_type8(type, name);
    if (rc) return rc;
    if (n_inputs < 1) DQ_FAIL(DQ_ERR_ARG, "%s: at least one input", name);
    if (!xs || !shapes || !x_scales) DQ_FAIL(DQ_ERR_ARG, "%s: xs, shapes and x_scales must not be NULL", name);
    if (ndim < 1 || ndim > kMaxDims) DQ_FAIL(DQ_ERR_ARG, "%s: ndim must be in [1, 8]", name);
    if (axis < -ndim || axis >= ndim) DQ_FAIL(DQ_ERR_RANGE, "%s: axis %d out of range", name, axis);
    if (axis < 0) axis += ndim;
    uint64_t total = 0, outer = 1, inner = 1;
    for (int j = 0; j < n_inputs; ++j) {
        uint64_t nj;
        if ((rc = tensor_size(ndim, shapes + (size_t)j * ndim, &nj, name))) return rc;
        for (int d = 0; d < ndim; ++d)
            if (d != axis && shapes[(size_t)j * ndim + d] != shapes[d])
                DQ_FAIL(DQ_ERR_ARG, "%s: input %d differs from input 0 in dim %d", name, j, d);
        total += (uint64_t)shapes[(size_t)j * ndim + axis];
    }
    for (int d = 0; d < axis; ++d) outer *= (uint64_t)shapes[d];
    for (int d = axis + 1; d < ndim; ++d) inner *= (uint64_t)shapes[d];
    const unsigned __int128 ny = (unsigned __int128)outer * total * inner;
    if (ny == 0) return DQ_OK;
    if (ny > ((unsigned __int128)1 << 40)) DQ_FAIL(DQ_ERR_RANGE, "%s: output too large", name);
    if (!y || !y_scale) DQ_FAIL(DQ_ERR_ARG, "%s: y and y_scale must not be NULL", name);
    for (int j = 0; j < n_inputs; ++j)
        if (shapes[(size_t)j * ndim + axis] > 0 && (!xs[j] || !x_scales[j]))
            DQ_FAIL(DQ_ERR_ARG, "%s: input %d or its scale is NULL", name, j);
    hipStream_t s = (hipStream_t)stream;
    const bool u8 = type == DQ_U8;
    const uint64_t ystride = total * inner;
    // one vector width for the launch: every input's rows and offsets
    int E = 16;
    {
        uint64_t base = 0;
        for (int j = 0; j < n_inputs; ++j) {
            const uint64_t len = (uint64_t)shapes[(size_t)j * ndim + axis] * inner;
            const uint64_t yoff = base * inner;
            base += (uint64_t)shapes[(size_t)j * ndim + axis];
            if (len == 0) continue;
            while (E > 1 && (len % E || yoff % E || (uintptr_t)xs[j] % E)) E /= 4;
        }
        while (E > 1 && (ystride % E || (uintptr_t)y % E)) E /= 4;
    }
    CatArgs ca{};
    ca.ystride = ystride;
    ca.y_scale = y_scale;
    ca.y_zp = y_zero_point;
    ca.y = (uint8_t*)y;
    uint64_t blocks = 0, base = 0;
    auto flush = [&]() -> int {
        if (ca.n == 0) return DQ_OK;
#define DQ_CAT(U, EE) hipLaunchKernelGGL((k_concat<U, EE>), dim3((unsigned)blocks), dim3(256), 0, s, ca)
        if (u8) {
            if (E == 16) DQ_CAT(true, 16);
            else if (E == 4) DQ_CAT(true, 4);
            else DQ_CAT(true, 1);
        } else {
            if (E == 16) DQ_CAT(false, 16);
            else if (E == 4) DQ_CAT(false, 4);
            else DQ_CAT(false, 1);
        }
#undef DQ_CAT
        DQ_LAUNCH_CHECK(name);
        ca.n = 0;
        blocks = 0;
        return DQ_OK;
    };
    for (int j = 0; j < n_inputs; ++j) {
        const uint64_t len = (uint64_t)shapes[(size_t)j * ndim + axis] * inner;
        const uint64_t yoff = base * inner;
        base += (uint64_t)shapes[(size_t)j * ndim + axis];
        if (len == 0) continue;
        const uint64_t nch = outer * len / E;
        if (nch >= (UINT64_C(1) << 32) || len / E >= (UINT64_C(1) << 32))
            DQ_FAIL(DQ_ERR_RANGE, "%s: input %d too large", name, j);
        const uint64_t nb = (nch + 1023) / 1024;
        if (ca.n == kCatMax || blocks + nb >= (UINT64_C(1) << 31))
            if ((rc = flush())) return rc;
        CatPart& p = ca.part[ca.n++];
        p.x = (const uint8_t*)xs[j];
        p.scale = x_scales[j];
        p.zp = x_zero_points ? x_zero_points[j] : nullptr;
        p.yoff = yoff;
        p.row_chunks = dq::make_fastdiv((uint32_t)(len / E));
        p.nchunks = (uint32_t)nch;
        p.block0 = (uint32_t)blocks;
        blocks += nb;
    }
    if ((rc = flush())) return rc;
    return DQ_OK;
}
