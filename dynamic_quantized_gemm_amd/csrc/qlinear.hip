// qlinear.hip -- QuantizeLinear / DequantizeLinear for gfx950.
//
// Operators: onnxruntime quantization_defs.cc, QuantizeLinear doc
// (y = saturate(x / y_scale + y_zero_point), the quotient rounded to nearest
// with ties to even, saturating to [0,255] or [-128,127]) and
// DequantizeLinear doc (y = (x - x_zero_point) * x_scale); scale and zero
// point per tensor or per 'axis'.
//
// Both kernels are element-wise and bound by HBM bandwidth: each wave
// instruction moves one contiguous 1 KiB of fp32 (16 bytes per lane) or the
// matching 256 bytes of 8-bit codes (4 per lane), and a lane requests all
// four of its vectors before it computes. The tensor is viewed as
// [outer, C, inner]; the channel of element e is (e / inner) % C, found with
// multiply-high division by constants precomputed on the host. When inner
// is a multiple of 4 a 4-element vector never straddles two channels and the
// channel (and the reciprocal of its scale) is found once per vector. The
// quotient x / y_scale is rounded through dq::qdiv, which gives the IEEE
// quotient's rounding to an integer.
#include <stdarg.h>
#include <stdio.h>

#include "dq_device.h"

namespace {

struct AxisMap {
    dq::FastDiv inner, cdim;
    int per_axis;
};

__device__ __forceinline__ uint32_t channel_of(uint32_t e, const AxisMap& a) {
    if (!a.per_axis) return 0;
    uint32_t q = dq::fdiv(e, a.inner);
    return q - dq::fdiv(q, a.cdim) * a.cdim.d;
}

__device__ __forceinline__ uint32_t channel_of64(uint64_t e, uint64_t inner, uint64_t cdim) {
    return (uint32_t)((e / inner) % cdim);
}

// fp16 tensors: values convert to fp32 exactly; an fp16 output is the fp32
// value rounded once to nearest even (v_cvt_f16_f32 in the default mode).
typedef _Float16 h4 __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ float ld(const T* p, uint64_t i) {
    return (float)p[i];
}

// four consecutive elements (16 bytes of fp32, 8 of fp16) as fp32
template <typename T>
__device__ __forceinline__ dq::f4 ld4(const T* p) {
    if constexpr (sizeof(T) == 4) {
        return __builtin_nontemporal_load(reinterpret_cast<const dq::f4*>(p));
    } else {
        const h4 h = *reinterpret_cast<const h4*>(p);
        return dq::f4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
    }
}

template <typename T>
__device__ __forceinline__ void st4(T* p, dq::f4 v) {
    if constexpr (sizeof(T) == 4) {
        __builtin_nontemporal_store(v, reinterpret_cast<dq::f4*>(p));
    } else {
        const h4 h = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
        *reinterpret_cast<h4*>(p) = h;
    }
}

template <bool U8>
__device__ __forceinline__ int load_zp(const void* zp, uint32_t c) {
    if (!zp) return 0;
    return U8 ? (int)((const uint8_t*)zp)[c] : (int)((const int8_t*)zp)[c];
}

template <bool U8>
__device__ __forceinline__ int quant1(float x, float s, int zp) {
    return dq::sat_add(dq::rne(x / s), zp, U8 ? 0 : -128, U8 ? 255 : 127);
}

// ---------------------------------------------------------------- quantize

// VEC: a 256-thread block covers 4096 consecutive elements as four
// 1024-element slices; in slice q thread t handles elements 4t .. 4t+3, so
// every load instruction of a wave reads 1 KiB of fp32 (512 bytes of fp16)
// contiguously and every store writes 256 contiguous bytes (x 16-byte
// aligned, y 4-byte aligned, n < 2^32). CH4: inner % 4 == 0, so four
// adjacent elements share one channel. XT: fp32 or fp16 x and scale.
template <bool U8, bool VEC, bool CH4, typename XT>
__global__ void __launch_bounds__(256)
k_quantize_linear(const XT* __restrict__ x, uint64_t n, AxisMap am, uint64_t inner64,
                  uint64_t cdim64, const XT* __restrict__ scale,
                  const void* __restrict__ zp, uint8_t* __restrict__ y) {
    if (VEC) {
        const uint32_t base = blockIdx.x * 4096u + threadIdx.x * 4u;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t e0 = base + q * 1024u;
            if ((uint64_t)e0 + 4 <= n) {
                const dq::f4 v = ld4(x + e0);
                uint32_t packed = 0;
                if (CH4) {
                    const uint32_t c = channel_of(e0, am);
                    const dq::QDiv d = dq::make_qdiv(ld(scale, c));
                    const int z = load_zp<U8>(zp, c);
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        packed |= ((uint32_t)dq::sat_add(dq::rne(dq::qdiv(v[b], d)), z, U8 ? 0 : -128,
                                                         U8 ? 255 : 127) & 0xffu) << (8 * b);
                } else {
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const uint32_t c = channel_of(e0 + b, am);
                        packed |= ((uint32_t)quant1<U8>(v[b], ld(scale, c), load_zp<U8>(zp, c)) & 0xffu) << (8 * b);
                    }
                }
                *reinterpret_cast<uint32_t*>(y + e0) = packed;
            } else {
                for (uint64_t e = e0; e < n && e < (uint64_t)e0 + 4; ++e) {
                    const uint32_t c = channel_of((uint32_t)e, am);
                    y[e] = (uint8_t)quant1<U8>(ld(x, e), ld(scale, c), load_zp<U8>(zp, c));
                }
            }
        }
    } else {
        // one element per thread, any alignment, any size
        const uint64_t t = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
        if (t < n) {
            const uint32_t c = am.per_axis ? channel_of64(t, inner64, cdim64) : 0;
            y[t] = (uint8_t)quant1<U8>(ld(x, t), ld(scale, c), load_zp<U8>(zp, c));
        }
    }
}

// TAB: the 4096 elements of a block cover at most kTabMax channels (per
// tensor, or per axis with inner >= 64 and inner % 4 == 0, so the four
// elements of a vector share a channel). The block first builds a table of
// those channels' scale, correctly rounded reciprocal and zero point in LDS
// (one division per channel instead of one per vector), then each lane
// quantizes four 4-element vectors whose loads are 1 KiB contiguous per
// wave instruction. Fast path (normal reciprocal): q0 = x * (1/s) clamped
// to +-2^22 (an input so large that x / s overflows saturates either way,
// and the clamp keeps the residual finite), q = q0 + (x - q0 s) (1/s) (the
// IEEE quotient's rounding to an integer, see dq::qdiv); q + 1.5 * 2^23
// rounds it half to even into the low mantissa bits, a median clamps it to
// the saturation bounds minus the zero point, and the zero point is added
// to the four packed low bytes at once (carry-free bytewise add).
constexpr int kTabMax = 66;  // 4096 / 64 + 2

template <bool U8, typename XT>
__global__ void __launch_bounds__(256)
k_quantize_tab(const XT* __restrict__ x, uint64_t n, AxisMap am, const XT* __restrict__ scale,
               const void* __restrict__ zp, uint8_t* __restrict__ y) {
    __shared__ float t_s[kTabMax], t_y[kTabMax], t_lo[kTabMax], t_hi[kTabMax];
    __shared__ uint32_t t_z[kTabMax];
    __shared__ int t_fast[kTabMax];
    constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
    constexpr float kBig = 4194304.0f;     // 2^22
    const uint32_t eb = blockIdx.x * 4096u;
    const uint32_t last = (uint64_t)eb + 4095 < n ? eb + 4095u : (uint32_t)(n - 1);
    // the block's x first: the channel table below is built while these
    // loads are in flight
    const uint32_t base = eb + threadIdx.x * 4u;
    dq::f4 v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t e0 = base + q * 1024u;
        v[q] = (uint64_t)e0 + 4 <= n ? ld4(x + e0) : dq::f4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    // "rows" of inner elements: channel of row r is r % C
    const uint32_t r0 = am.per_axis ? dq::fdiv(eb, am.inner) : 0;
    const uint32_t nrows = am.per_axis ? dq::fdiv(last, am.inner) - r0 + 1 : 1;
    for (uint32_t k = threadIdx.x; k < nrows; k += 256) {
        const uint32_t row = r0 + k;
        const uint32_t c = am.per_axis ? row - dq::fdiv(row, am.cdim) * am.cdim.d : 0;
        const float sc = ld(scale, c);
        const int z = load_zp<U8>(zp, c);
        const dq::QDiv d = dq::make_qdiv(sc);
        t_s[k] = sc;
        t_y[k] = d.y;
        t_fast[k] = d.fast;
        t_z[k] = (uint32_t)(z & 0xff) * 0x01010101u;
        t_lo[k] = kMagic + (float)((U8 ? 0 : -128) - z);
        t_hi[k] = kMagic + (float)((U8 ? 255 : 127) - z);
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t e0 = base + q * 1024u;
        if ((uint64_t)e0 >= n) break;
        const uint32_t k = am.per_axis ? dq::fdiv(e0, am.inner) - r0 : 0;
        if ((uint64_t)e0 + 4 > n) {  // the tensor's last partial vector
            for (uint64_t e = e0; e < n; ++e) {
                const uint32_t c = channel_of((uint32_t)e, am);
                y[e] = (uint8_t)quant1<U8>(ld(x, e), ld(scale, c), load_zp<U8>(zp, c));
            }
            break;
        }
        uint32_t w;
        if (t_fast[k]) {
            const float sc = t_s[k], ry = t_y[k], lof = t_lo[k], hif = t_hi[k];
            uint32_t b[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float xe = v[q][e];
                const float q0 = __builtin_amdgcn_fmed3f(xe * ry, -kBig, kBig);
                const float r = __builtin_fmaf(-q0, sc, xe);
                const float t = __builtin_fmaf(r, ry, q0) + kMagic;
                b[e] = (uint32_t)__float_as_int(__builtin_amdgcn_fmed3f(t, lof, hif));
            }
            const uint32_t packed = (b[0] & 0xffu) | ((b[1] & 0xffu) << 8) | ((b[2] & 0xffu) << 16) | (b[3] << 24);
            const uint32_t Z = t_z[k];
            w = ((packed & 0x7f7f7f7fu) + (Z & 0x7f7f7f7fu)) ^ ((packed ^ Z) & 0x80808080u);
        } else {
            const float sc = t_s[k];
            const int z = (int)(U8 ? (t_z[k] & 0xffu) : (uint32_t)(int8_t)(t_z[k] & 0xffu));
            w = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) w |= ((uint32_t)quant1<U8>(v[q][e], sc, z) & 0xffu) << (8 * e);
        }
        __builtin_nontemporal_store(w, reinterpret_cast<uint32_t*>(y + e0));
    }
}

// -------------------------------------------------------------- dequantize

template <bool U8>
__device__ __forceinline__ float dequant1(uint32_t byte, float s, int zp) {
    const int q = U8 ? (int)(byte & 0xffu) : (int)(int8_t)(byte & 0xffu);
    return (float)(q - zp) * s;
}

// VEC: the same 4096-element block split as quantize: in slice q thread t
// reads the 4 codes 4t .. 4t+3 (256 contiguous bytes per wave) and writes
// their 4 values (1 KiB of fp32 or 512 bytes of fp16 contiguous per wave).
// ST / YT: fp32 or fp16 scale and y. (x - zp) * s has at most 19
// significant bits for an fp16 scale, so the fp32 product is exact and an
// fp16 y is rounded once.
template <bool U8, bool VEC, bool CH4, typename ST, typename YT>
__global__ void __launch_bounds__(256)
k_dequantize_linear(const uint8_t* __restrict__ x, uint64_t n, AxisMap am, uint64_t inner64,
                    uint64_t cdim64, const ST* __restrict__ scale,
                    const void* __restrict__ zp, YT* __restrict__ y) {
    if (VEC) {
        const uint32_t base = blockIdx.x * 4096u + threadIdx.x * 4u;
        // every slice's codes are requested before the first store
        uint32_t wq[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t e0 = base + q * 1024u;
            wq[q] = (uint64_t)e0 + 4 <= n ? *reinterpret_cast<const uint32_t*>(x + e0) : 0u;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t e0 = base + q * 1024u;
            if ((uint64_t)e0 + 4 <= n) {
                const uint32_t w = wq[q];
                dq::f4 out;
                if (CH4) {
                    const uint32_t c = channel_of(e0, am);
                    const float s = ld(scale, c);
                    const int z = load_zp<U8>(zp, c);
#pragma unroll
                    for (int b = 0; b < 4; ++b) out[b] = dequant1<U8>(w >> (8 * b), s, z);
                } else {
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const uint32_t c = channel_of(e0 + b, am);
                        out[b] = dequant1<U8>(w >> (8 * b), ld(scale, c), load_zp<U8>(zp, c));
                    }
                }
                st4(y + e0, out);
            } else {
                for (uint64_t e = e0; e < n && e < (uint64_t)e0 + 4; ++e) {
                    const uint32_t c = channel_of((uint32_t)e, am);
                    y[e] = (YT)dequant1<U8>(x[e], ld(scale, c), load_zp<U8>(zp, c));
                }
            }
        }
    } else {
        const uint64_t t = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
        if (t < n) {
            const uint32_t c = am.per_axis ? channel_of64(t, inner64, cdim64) : 0;
            y[t] = (YT)dequant1<U8>(x[t], ld(scale, c), load_zp<U8>(zp, c));
        }
    }
}

// ------------------------------------------------------------------- host

struct Plan {
    uint64_t n = 0, inner = 1, cdim = 1;
    int per_axis = 0;
};

int make_plan(int ndim, const int64_t* shape, int axis, Plan* p) {
    if (ndim < 1 || ndim > 8) DQ_FAIL(DQ_ERR_ARG, "ndim must be in [1, 8], got %d", ndim);
    if (!shape) DQ_FAIL(DQ_ERR_ARG, "shape is NULL");
    uint64_t n = 1;
    for (int d = 0; d < ndim; ++d) {
        if (shape[d] < 0) DQ_FAIL(DQ_ERR_ARG, "shape[%d] = %lld is negative", d, (long long)shape[d]);
        if (shape[d] != 0 && n > (UINT64_C(1) << 62) / (uint64_t)shape[d])
            DQ_FAIL(DQ_ERR_ARG, "tensor too large");
        n *= (uint64_t)shape[d];
    }
    p->n = n;
    if (axis == DQ_PER_TENSOR) {
        p->per_axis = 0;
        return DQ_OK;
    }
    if (axis < -ndim || axis >= ndim)
        DQ_FAIL(DQ_ERR_RANGE, "axis %d out of range for a rank-%d tensor", axis, ndim);
    if (axis < 0) axis += ndim;
    uint64_t inner = 1;
    for (int d = axis + 1; d < ndim; ++d) inner *= (uint64_t)shape[d];
    p->inner = inner ? inner : 1;
    p->cdim = (uint64_t)shape[axis];
    p->per_axis = p->cdim > 1 ? 1 : 0;  // a length-1 axis is per tensor
    return DQ_OK;
}

AxisMap make_axis_map(const Plan& p, bool small) {
    AxisMap am{};
    am.per_axis = p.per_axis;
    if (p.per_axis && small) {
        am.inner = dq::make_fastdiv((uint32_t)p.inner);
        am.cdim = dq::make_fastdiv((uint32_t)p.cdim);
    }
    return am;
}

// f32 side 16-byte aligned and 8-bit side 4-byte aligned for the vector
// kernels; anything else takes the one-element-per-thread kernels.
template <typename Launch>
int dispatch(const Plan& p, const void* f32_side, const void* i8_side, Launch&& launch) {
    const bool small = p.n < (UINT64_C(1) << 32) - 4096 && p.inner < (UINT64_C(1) << 32) &&
                       p.cdim < (UINT64_C(1) << 32);
    const bool aligned = ((uintptr_t)f32_side % 16 == 0) && ((uintptr_t)i8_side % 4 == 0);
    const bool vec = small && aligned;
    const bool ch16 = !p.per_axis || p.inner % 4 == 0;
    const AxisMap am = make_axis_map(p, small);
    const uint64_t blocks = vec ? (p.n + 4095) / 4096 : (p.n + 255) / 256;
    if (blocks > 0x7fffffffull) DQ_FAIL(DQ_ERR_ARG, "tensor too large");
    launch(vec, ch16, am, (unsigned)blocks);
    return DQ_OK;
}

template <typename XT>
int quantize_impl(const XT* x, int ndim, const int64_t* shape, int axis, const XT* y_scale,
                  const void* y_zero_point, dq_dtype y_type, void* y, void* stream, const char* name) {
    Plan p;
    int rc = make_plan(ndim, shape, axis, &p);
    if (rc) return rc;
    if (y_type != DQ_I8 && y_type != DQ_U8)
        DQ_FAIL(DQ_ERR_TYPE, "QuantizeLinear output must be int8 or uint8");
    if (p.n == 0) return DQ_OK;
    if (!x || !y || !y_scale) DQ_FAIL(DQ_ERR_ARG, "x, y and y_scale must not be NULL");
    hipStream_t s = (hipStream_t)stream;
    const bool u8 = y_type == DQ_U8;
    const bool small = p.n < (UINT64_C(1) << 32) - 4096 && p.inner < (UINT64_C(1) << 32) &&
                       p.cdim < (UINT64_C(1) << 32);
    if (small && (!p.per_axis || (p.inner >= 64 && p.inner % 4 == 0)) && (uintptr_t)x % 16 == 0 &&
        (uintptr_t)y % 4 == 0) {
        const AxisMap am = make_axis_map(p, true);
        const unsigned blocks = (unsigned)((p.n + 4095) / 4096);
        if (u8)
            hipLaunchKernelGGL((k_quantize_tab<true, XT>), dim3(blocks), dim3(256), 0, s, x, p.n, am, y_scale,
                               y_zero_point, (uint8_t*)y);
        else
            hipLaunchKernelGGL((k_quantize_tab<false, XT>), dim3(blocks), dim3(256), 0, s, x, p.n, am, y_scale,
                               y_zero_point, (uint8_t*)y);
        DQ_LAUNCH_CHECK(name);
        return DQ_OK;
    }
    rc = dispatch(p, x, y, [&](bool vec, bool ch16, AxisMap am, unsigned blocks) {
#define DQ_QL(U, V, C)                                                                         \
    hipLaunchKernelGGL((k_quantize_linear<U, V, C, XT>), dim3(blocks), dim3(256), 0, s, x, p.n, \
                       am, p.inner, p.cdim, y_scale, y_zero_point, (uint8_t*)y)
        if (u8) {
            if (!vec) DQ_QL(true, false, true);
            else if (ch16) DQ_QL(true, true, true);
            else DQ_QL(true, true, false);
        } else {
            if (!vec) DQ_QL(false, false, true);
            else if (ch16) DQ_QL(false, true, true);
            else DQ_QL(false, true, false);
        }
#undef DQ_QL
    });
    if (rc) return rc;
    DQ_LAUNCH_CHECK(name);
    return DQ_OK;
}

template <typename ST, typename YT>
int dequantize_impl(const void* x, dq_dtype x_type, int ndim, const int64_t* shape, int axis,
                    const ST* x_scale, const void* x_zero_point, YT* y, void* stream, const char* name) {
    Plan p;
    int rc = make_plan(ndim, shape, axis, &p);
    if (rc) return rc;
    if (x_type != DQ_I8 && x_type != DQ_U8)
        DQ_FAIL(DQ_ERR_TYPE, "DequantizeLinear input must be int8 or uint8");
    if (p.n == 0) return DQ_OK;
    if (!x || !y || !x_scale) DQ_FAIL(DQ_ERR_ARG, "x, y and x_scale must not be NULL");
    hipStream_t s = (hipStream_t)stream;
    const bool u8 = x_type == DQ_U8;
    rc = dispatch(p, y, x, [&](bool vec, bool ch16, AxisMap am, unsigned blocks) {
#define DQ_DQL(U, V, C)                                                                           \
    hipLaunchKernelGGL((k_dequantize_linear<U, V, C, ST, YT>), dim3(blocks), dim3(256), 0, s,      \
                       (const uint8_t*)x, p.n, am, p.inner, p.cdim, x_scale, x_zero_point, y)
        if (u8) {
            if (!vec) DQ_DQL(true, false, true);
            else if (ch16) DQ_DQL(true, true, true);
            else DQ_DQL(true, true, false);
        } else {
            if (!vec) DQ_DQL(false, false, true);
            else if (ch16) DQ_DQL(false, true, true);
            else DQ_DQL(false, true, false);
        }
#undef DQ_DQL
    });
    if (rc) return rc;
    DQ_LAUNCH_CHECK(name);
    return DQ_OK;
}

}  // namespace

extern "C" int qlinear_quantize(const float* x, int ndim, const int64_t* shape, int axis,
                                const float* y_scale, const void* y_zero_point,
                                dq_dtype y_type, void* y, void* stream) {
    return quantize_impl<float>(x, ndim, shape, axis, y_scale, y_zero_point, y_type, y, stream,
                                "quantize_linear");
}

extern "C" int qlinear_quantize_f16(const void* x, int ndim, const int64_t* shape, int axis,
                                    const void* y_scale, const void* y_zero_point, dq_dtype y_type,
                                    void* y, void* stream) {
    return quantize_impl<_Float16>((const _Float16*)x, ndim, shape, axis, (const _Float16*)y_scale,
                                   y_zero_point, y_type, y, stream, "quantize_linear_f16");
}

extern "C" int qlinear_dequantize(const void* x, dq_dtype x_type, int ndim, const int64_t* shape,
                                  int axis, const float* x_scale, const void* x_zero_point,
                                  float* y, void* stream) {
    return dequantize_impl<float, float>(x, x_type, ndim, shape, axis, x_scale, x_zero_point, y, stream,
                                         "dequantize_linear");
}

extern "C" int qlinear_dequantize_f16(const void* x, dq_dtype x_type, int ndim, const int64_t* shape,
                                      int axis, const void* x_scale, const void* x_zero_point,
                                      dq_dtype y_type, void* y, void* stream) {
    if (y_type == DQ_F16)
        return dequantize_impl<_Float16, _Float16>(x, x_type, ndim, shape, axis, (const _Float16*)x_scale,
                                                   x_zero_point, (_Float16*)y, stream, "dequantize_linear_f16");
    if (y_type == DQ_F32)
        return dequantize_impl<_Float16, float>(x, x_type, ndim, shape, axis, (const _Float16*)x_scale,
                                                x_zero_point, (float*)y, stream, "dequantize_linear_f16");
    DQ_FAIL(DQ_ERR_TYPE, "DequantizeLinear with fp16 scales writes fp16 or fp32");
}
