// qgemm.hip -- the quantized matrix products of the onnxruntime schemas
// QGemm, MatMulIntegerToFloat and DynamicQuantizeMatMul on gfx950.
//
// onnxruntime quantization_defs.cc gives these operators' inputs, types and
// attributes but prints no formula; this library computes (the readings are
// stated where the operators are declared, include/dqip.h):
//   sum[m,n] = sum_k (A[m,k] - a_zp) * (B[k,n] - b_zp[n])   (exact, int32)
//   real     = ((float)(sum + C[m,n]) * (alpha * a_scale)) * b_scale[n] (+ bias[n])
//   Y        = real, or saturate(rne(real / y_scale) + y_zp) for an 8-bit Y,
// with b_scale / b_zp per tensor or per column, A given as (K,M) under transA
// and B as (N,K) under transB, and for DynamicQuantizeMatMul A (fp32)
// quantized per tensor to uint8 first, with the row quantizer's rule over
// the whole tensor: lo = min(0, min A), hi = max(0, max A),
// scale = (hi - lo) / 255, zp = saturate(rne(-lo / scale)).
//
// The products run on the int8 GEMM of gemm_i8.hip. A uint8 operand enters
// as code - 128 (shift s = 128, 0 for int8), so with A^ = A - sa and
// B^ = B - sb:
//   sum = sum_k A^ B^ + (sa - a_zp) * colsum(B^)[n]
//         + (sb - b_zp[n]) * (rowsum(A^)[m] + K * (sa - a_zp)),
// all in wrapping int32 (exact whenever the true sum fits, which K <= 32768
// guarantees). The GEMM takes the first correction from its zeroA / colsum
// vectors (zeroA = a_zp + 128 - sa) and the second from rowsumA / zeroB.
//
// Kernels here:
//  - k_pack_rows<SRC>: an [R, K] source (int8, uint8, or fp32 quantized per
//    tensor) to packed MFMA fragments, with the row sums of the packed codes
//    and, for A, the per-row epilogue vectors. Lane (r = lane % 8, j =
//    lane / 8) of a wave takes 16-code group 8 * (8 it + w) + j of row r of
//    the block's eight rows, so one store instruction writes eight whole
//    128-byte lines of the packed operand (each line holds one group of
//    eight consecutive rows) and one 8-bit load instruction reads eight
//    whole 128-byte row segments.
//  - k_tensor_minmax: the per-tensor min / max of an fp32 A (atomics on an
//    order-preserving integer encoding of the fp32 bits), 0 included.
//  - k_a_params / k_b_params: per-row and per-column vectors for the GEMM.
// Transposed 8-bit sources (A under transA, B without transB) go through the
// column packer of quant_cols.hip.
//
// N-dimensional MatMulIntegerToFloat / DynamicQuantizeMatMul (the schemas'
// A and B are N-dimensional, with numpy.matmul's batch broadcasting): with
// a single B batch the A batches are just more rows of one product; else A
// and B are packed batch by batch (each padded like a 2-D operand) and each
// Y batch is one GEMM launch on its A and B batch.
#include <stdio.h>
#include <string.h>

#include <string>
#include <vector>

#include "dq_device.h"
#include "dq_kernels.h"

namespace {

constexpr size_t kAlign = 256;

enum { SRC_I8 = 0, SRC_U8 = 1, SRC_F32 = 2 };

// The tensor's min / max land in kMmSlots slot pairs (workgroup b adds to
// slot b % kMmSlots), so no single address takes every workgroup's atomics;
// mm[0 .. kMmSlots) hold minima, mm[kMmSlots .. 2 kMmSlots) maxima.
constexpr int kMmSlots = 64;

// Per-tensor quantization parameters from the slots (the row quantizer's
// rule over the whole tensor); a whole wave calls it and gets uniform values.
__device__ __forceinline__ void tensor_params(const uint32_t* mm, float& scale, int& zero) {
    const int lane = threadIdx.x & 63;
    const float lo = dq::wave_min_uniform(dq::ord2f(mm[lane]));
    const float hi = dq::wave_max_uniform(dq::ord2f(mm[kMmSlots + lane]));
    if (hi == lo) {
        scale = 1.0f;
        zero = 0;
    } else {
        scale = (hi - lo) / 255.0f;
        zero = dq::sat_add(dq::rne(-lo / scale), 0, 0, 255);
    }
}

__device__ __forceinline__ int load_zp8(const void* zp, bool u8) {
    if (!zp) return 0;
    return u8 ? (int)*reinterpret_cast<const uint8_t*>(zp) : (int)*reinterpret_cast<const int8_t*>(zp);
}

__global__ void k_minmax_init(uint32_t* mm) {
    if (threadIdx.x < 2 * kMmSlots) mm[threadIdx.x] = 0x80000000u;  // the encoding of +0.0
}

// Min / max of n fp32 values (0 included through the initial words).
template <bool VEC>
__global__ void __launch_bounds__(256) k_tensor_minmax(const float* __restrict__ A, size_t n,
                                                        uint32_t* __restrict__ mm) {
    float lo = 0.0f, hi = 0.0f;
    const size_t stride = (size_t)gridDim.x * 256;
    if (VEC) {
        // four 16-byte loads a thread in flight per pass, then the rest
        const dq::f4* a4 = reinterpret_cast<const dq::f4*>(A);
        const size_t n4 = n / 4;
        size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
        for (; i + 3 * stride < n4; i += 4 * stride) {
            dq::f4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = a4[i + u * stride];
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    lo = __builtin_fminf(lo, v[u][e]);
                    hi = __builtin_fmaxf(hi, v[u][e]);
                }
        }
        for (; i < n4; i += stride) {
            const dq::f4 v = a4[i];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                lo = __builtin_fminf(lo, v[e]);
                hi = __builtin_fmaxf(hi, v[e]);
            }
        }
    } else {
        for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
            lo = __builtin_fminf(lo, A[i]);
            hi = __builtin_fmaxf(hi, A[i]);
        }
    }
    __shared__ float s_lo[4], s_hi[4];
    lo = dq::wave_min_uniform(lo);
    hi = dq::wave_max_uniform(hi);
    if ((threadIdx.x & 63) == 0) {
        s_lo[threadIdx.x >> 6] = lo;
        s_hi[threadIdx.x >> 6] = hi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        lo = __builtin_fminf(__builtin_fminf(s_lo[0], s_lo[1]), __builtin_fminf(s_lo[2], s_lo[3]));
        hi = __builtin_fmaxf(__builtin_fmaxf(s_hi[0], s_hi[1]), __builtin_fmaxf(s_hi[2], s_hi[3]));
        const int slot = blockIdx.x % kMmSlots;
        atomicMin(&mm[slot], dq::f2ord(lo));
        atomicMax(&mm[kMmSlots + slot], dq::f2ord(hi));
    }
}

// What k_pack_rows writes besides the packed codes when it packs A (zeroA
// NULL: a B operand, sums only).
struct RowOut {
    int32_t* sums;      // [R]: row sum of the packed codes (+ K * (sa - a_zp) for A)
    int32_t* zeroA;     // [R]: a_zp + 128 - sa
    float* scaleA;      // [R]: alpha * a_scale
    const float* a_scale;
    const void* a_zp;   // device scalar of A's type (NULL: 0)
    const uint32_t* mm; // SRC_F32: the tensor's min / max words
    float alpha;
};

// 16 fp32 values from k0, quantized with the tensor's scale / zero point to
// uint8 and packed as code - 128 (corrected quotient, rounding add, median
// clamp, as the row quantizer); bytes past K stay zero (ALL: none is).
template <bool ALL>
__device__ __forceinline__ dq::u4 f32_codes(const float (&x)[16], int k0, int K, const dq::QDiv& d, int zero) {
    constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
    const float lof = kMagic - (float)zero, hif = kMagic + (float)(255 - zero);
    dq::u4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int k = k0 + 4 * q + e;
            uint32_t code;  // uA in [0, 255]
            if (d.fast) {
                const float t = dq::qdiv_fast(x[4 * q + e], d) + kMagic;
                code = (uint32_t)__float_as_int(__builtin_amdgcn_fmed3f(t, lof, hif)) + (uint32_t)zero;
            } else {
                code = (uint32_t)dq::sat_add(dq::rne(x[4 * q + e] / d.s), zero, 0, 255);
            }
            if (ALL || k < K) w |= ((code & 0xffu) ^ 0x80u) << (8 * e);
        }
        o[q] = w;
    }
    return o;
}

// 16 codes of group g of row `row` (zero past K or past R), as packed int8.
template <int SRC, bool VEC>
__device__ __forceinline__ dq::u4 load_group(const void* __restrict__ src, int R, int K, int row, int g,
                                             const dq::QDiv& d, int zero) {
    const int k0 = 16 * g;
    dq::u4 o = {0u, 0u, 0u, 0u};
    if (row >= R || k0 >= K) return o;
    if (SRC != SRC_F32) {
        const uint8_t* p = reinterpret_cast<const uint8_t*>(src) + (size_t)row * K + k0;
        if (VEC) {
            o = *reinterpret_cast<const dq::u4*>(p);
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (k0 + e < K) o[e >> 2] |= (uint32_t)p[e] << (8 * (e & 3));
        }
        if (SRC == SRC_U8) {
            // code - 128 as int8 is the code with its top bit flipped; bytes
            // past K stay zero
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint32_t m = 0x80808080u;
                if (!VEC) {
                    const int kq = k0 + 4 * q;
                    m = 0;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (kq + e < K) m |= 0x80u << (8 * e);
                }
                o[q] ^= m;
            }
        }
        return o;
    }
    const float* p = reinterpret_cast<const float*>(src) + (size_t)row * K + k0;
    float x[16];
    if (VEC) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const dq::f4 v = reinterpret_cast<const dq::f4*>(p)[q];
#pragma unroll
            for (int e = 0; e < 4; ++e) x[4 * q + e] = v[e];
        }
    } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) x[e] = k0 + e < K ? p[e] : 0.0f;
    }
    return f32_codes<VEC>(x, k0, K, d, zero);
}

// A block packs rows 8 b .. 8 b + 7 over all of Kp (padding groups are
// zero). Rows past R are packed as zeros (the buffer holds Rp rows).
template <int SRC, bool VEC>
__global__ void __launch_bounds__(256)
k_pack_rows(const void* __restrict__ src, int R, int K, int Kp, int8_t* __restrict__ dst, RowOut out) {
    __shared__ int32_t s_sum[4][8];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = lane & 7, j = lane >> 3;
    const int row = 8 * blockIdx.x + r;
    const int KF = Kp / 32, ngp = Kp / 16;
    dq::QDiv d = {1.0f, 1.0f, true};
    int zero = 0;
    float tscale = 1.0f;
    int sum = 0;
    auto put = [&](int g, const dq::u4& o) {
#pragma unroll
        for (int q = 0; q < 4; ++q) sum = __builtin_amdgcn_sdot4((int)o[q], 0x01010101, sum, false);
        *reinterpret_cast<dq::u4*>(dst + dq::frag_offset((size_t)row, (size_t)g * 16, (size_t)KF)) = o;
    };
    if constexpr (VEC && SRC != SRC_F32) {
        // 8-bit source in whole 16-byte groups: a lane takes its groups GP at
        // a time and issues the loads of the next GP before it codes and
        // stores the current ones, so its reads stay in flight meanwhile
        // (the plain loop below waits for each group: its loads sit under
        // the group's bounds branch). Loads are unconditional at clamped
        // addresses (a row past R reads row R - 1, a group past K the last
        // group); those groups code as 0.
        constexpr int GP = 8;      // groups per pass
        const int ngk = K / 16;    // groups that hold data
        const bool rin = row < R;
        const dq::u4* rp = reinterpret_cast<const dq::u4*>(reinterpret_cast<const uint8_t*>(src) +
                                                           (size_t)min(row, R - 1) * K);
        const int npass = (ngp + 32 * GP - 1) / (32 * GP);
        dq::u4 cur[GP], nxt[GP];
        auto load = [&](int p, dq::u4 (&v)[GP]) {
#pragma unroll
            for (int u = 0; u < GP; ++u) v[u] = rp[min(8 * w + j + 32 * (GP * p + u), ngk - 1)];
        };
        load(0, cur);
        for (int p = 0; p < npass; ++p) {
            if (p + 1 < npass) load(p + 1, nxt);
#pragma unroll
            for (int u = 0; u < GP; ++u) {
                const int g = 8 * w + j + 32 * (GP * p + u);
                dq::u4 o = {0u, 0u, 0u, 0u};
                if (rin && g < ngk) {
                    o = cur[u];
                    // code - 128 as int8 is the code with its top bit flipped
                    if (SRC == SRC_U8)
#pragma unroll
                        for (int q = 0; q < 4; ++q) o[q] ^= 0x80808080u;
                }
                if (g < ngp) put(g, o);
            }
#pragma unroll
            for (int u = 0; u < GP; ++u) cur[u] = nxt[u];
        }
    } else {
        if (SRC == SRC_F32) {
            tensor_params(out.mm, tscale, zero);  // the whole wave, before any branch
            d = dq::make_qdiv(tscale);
        }
#pragma unroll 4
        for (int g = 8 * w + j; g < ngp; g += 32) put(g, load_group<SRC, VEC>(src, R, K, row, g, d, zero));
    }
    // the row's sum: lanes r, r + 8, ..., r + 56 of each wave, then the waves
    sum += __shfl_xor(sum, 8, 64);
    sum += __shfl_xor(sum, 16, 64);
    sum += __shfl_xor(sum, 32, 64);
    if (j == 0) s_sum[w][r] = sum;
    __syncthreads();
    if (threadIdx.x < 8 && row < R) {
        int total = s_sum[0][r] + s_sum[1][r] + s_sum[2][r] + s_sum[3][r];
        if (out.zeroA) {
            // A: the per-row vectors of the GEMM's epilogue
            int azp, sa;
            float ascale;
            if (SRC == SRC_F32) {
                azp = zero;  // the tensor's scale and zero point, as used above
                ascale = tscale;
                sa = 128;
            } else {
                azp = load_zp8(out.a_zp, SRC == SRC_U8);
                sa = SRC == SRC_U8 ? 128 : 0;
                ascale = out.a_scale[0];
            }
            total = (int)((uint32_t)total + (uint32_t)K * (uint32_t)(sa - azp));
            out.zeroA[row] = azp + 128 - sa;
            out.scaleA[row] = out.alpha * ascale;
        }
        out.sums[row] = total;
    }
}

// A packed by the column packer (transA): sums hold the row sums of the
// packed codes; add K * (sa - a_zp) and write the per-row vectors.
__global__ void __launch_bounds__(256)
k_a_params(int M, int K, bool u8, const float* __restrict__ a_scale, const void* __restrict__ a_zp,
           float alpha, int32_t* __restrict__ sums, int32_t* __restrict__ zeroA, float* __restrict__ scaleA) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= M) return;
    const int azp = load_zp8(a_zp, u8), sa = u8 ? 128 : 0;
    sums[i] = (int)((uint32_t)sums[i] + (uint32_t)K * (uint32_t)(sa - azp));
    zeroA[i] = azp + 128 - sa;
    scaleA[i] = alpha * a_scale[0];
}

// Per-column vectors of B for j < Np: scaleB, zb = sb - b_zp (zero past N).
__global__ void __launch_bounds__(256)
k_b_params(int N, int Np, bool u8, const float* __restrict__ b_scale, int bs_len,
           const void* __restrict__ b_zp, int bz_len, float* __restrict__ scaleB, int32_t* __restrict__ zb) {
    const int jj = blockIdx.x * 256 + threadIdx.x;
    if (jj >= Np) return;
    if (jj >= N) {
        scaleB[jj] = 0.0f;
        zb[jj] = 0;
        return;
    }
    scaleB[jj] = b_scale[bs_len == 1 ? 0 : jj];
    int z = 0;
    if (b_zp) {
        const int k = bz_len == 1 ? 0 : jj;
        z = u8 ? (int)reinterpret_cast<const uint8_t*>(b_zp)[k] : (int)reinterpret_cast<const int8_t*>(b_zp)[k];
    }
    zb[jj] = (u8 ? 128 : 0) - z;
}

template <int SRC>
int launch_pack_rows(const void* src, int R, int K, int Kp, int8_t* dst, const RowOut& out, hipStream_t s) {
    const size_t esz = SRC == SRC_F32 ? 4 : 1;
    const bool vec = K % 16 == 0 && (uintptr_t)src % 16 == 0 && (esz * (size_t)K) % 16 == 0;
    const dim3 grid((unsigned)((R + 7) / 8));
    if (vec)
        hipLaunchKernelGGL((k_pack_rows<SRC, true>), grid, dim3(256), 0, s, src, R, K, Kp, dst, out);
    else
        hipLaunchKernelGGL((k_pack_rows<SRC, false>), grid, dim3(256), 0, s, src, R, K, Kp, dst, out);
    DQ_LAUNCH_CHECK("pack_rows");
    return DQ_OK;
}

const char* tname(dq_dtype t) {
    switch (t) {
        case DQ_F32: return "f32";
        case DQ_BF16: return "bf16";
        case DQ_I8: return "i8";
        case DQ_U8: return "u8";
    }
    return "?";
}

}  // namespace

struct dq_qgemm_ctx {
    int device;
    int M, N, K, Kp;
    dq_dtype a_type, b_type, y_type;
    int transA, transB;
    float alpha;
    int b_set;
    int zb_any;          // some column has sb - b_zp != 0
    std::vector<void*> owned;
    // B (set once)
    int8_t* Bp;          // [Np x Kp]
    int32_t* colsum;     // [Np]
    float* scaleB;       // [Np]
    int32_t* zb;         // [Np]
    // per forward
    int8_t* Ap;          // [Mp x Kp]
    int32_t* rowsum;     // [Mp]
    int32_t* zeroA;      // [Mp]
    float* scaleA;       // [Mp]
    uint32_t* mm;        // 2 x kMmSlots words: per-tensor min / max slots (fp32 A)
    // batches (dq_qgemm_init_batched): A and B hold nA and nB packed
    // operands Mp x Kp and Np x Kp apart (their row and column vectors Mp
    // and Np apart); Y batch z multiplies A batch ia[z] by B batch ib[z]
    // (ia, ib empty: one product)
    int batched;
    int64_t nA, nB;
    std::vector<int32_t> ia, ib;
    std::string info;
};

namespace {

int ctx_alloc(dq_qgemm_ctx* c, void** p, size_t bytes) {
    hipError_t e = hipMalloc(p, bytes ? bytes : 1);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        *p = nullptr;
        DQ_FAIL(DQ_ERR_ALLOC, "hipMalloc(%zu) failed: %s", bytes, hipGetErrorString(e));
    }
    c->owned.push_back(*p);
    return DQ_OK;
}

void ctx_free(dq_qgemm_ctx* c) {
    for (void* p : c->owned) (void)hipFree(p);
    c->owned.clear();
}

int check_device(const dq_qgemm_ctx* c) {
    int dev = -1;
    DQ_HIP_CHECK(hipGetDevice(&dev));
    if (dev != c->device)
        DQ_FAIL(DQ_ERR_STATE, "context was created on device %d, current device is %d", c->device, dev);
    return DQ_OK;
}

int run(dq_qgemm_ctx* c, const void* A, const float* a_scale, const void* a_zp, const int32_t* Cm,
        int64_t c_rows, int64_t c_cols, const float* bias, const float* y_scale, const void* y_zp,
        void* Y, int mode, hipStream_t s) {
    if (!c) DQ_FAIL(DQ_ERR_STATE, "context is NULL");
    if (!c->b_set) DQ_FAIL(DQ_ERR_STATE, "dq_qgemm_set_b has not been called");
    if (!A || !Y) DQ_FAIL(DQ_ERR_ARG, "A and Y must not be NULL");
    if (c->a_type == DQ_F32) {
        if (a_scale || a_zp) DQ_FAIL(DQ_ERR_ARG, "an fp32 A is quantized by the call: a_scale and a_zero_point must be NULL");
    } else if (!a_scale) {
        DQ_FAIL(DQ_ERR_ARG, "a_scale is NULL");
    }
    if (Cm && c->batched) DQ_FAIL(DQ_ERR_ARG, "C is not an input of the N-dimensional products");
    if (Cm && !((c_rows == 1 || c_rows == c->M) && (c_cols == 1 || c_cols == c->N)))
        DQ_FAIL(DQ_ERR_ARG, "C of shape (%lld, %lld) does not broadcast to (%d, %d)", (long long)c_rows,
                (long long)c_cols, c->M, c->N);
    if (bias && (mode != DQ_OUT_F32 && mode != DQ_OUT_ACC))
        DQ_FAIL(DQ_ERR_ARG, "bias is only defined for an fp32 Y");
    const bool q8 = mode == DQ_OUT_U8 || mode == DQ_OUT_I8;
    if (q8 && !y_scale) DQ_FAIL(DQ_ERR_ARG, "an 8-bit Y needs y_scale");
    if (!q8 && (y_scale || y_zp)) DQ_FAIL(DQ_ERR_ARG, "y_scale / y_zero_point are only defined for an 8-bit Y");
    int rc = check_device(c);
    if (rc) return rc;
    const int M = c->M, N = c->N, K = c->K, Kp = c->Kp;
    const size_t Mp = dq_mnp((size_t)M), Np = dq_mnp((size_t)N);
    const size_t esz = c->a_type == DQ_F32 ? 4 : 1;
    // A -> packed, row sums and per-row vectors, one A batch at a time (an
    // fp32 A quantized with the min / max of all its batches)
    if (c->a_type == DQ_F32) {
        const size_t n = (size_t)c->nA * M * K;
        hipLaunchKernelGGL(k_minmax_init, dim3(1), dim3(2 * kMmSlots), 0, s, c->mm);
        const bool vec = (uintptr_t)A % 16 == 0 && n % 4 == 0;
        const size_t need = (vec ? n / 4 : n + 255) / 256 + 1;
        // at most one workgroup a CU, each reading many vectors: 2048
        // workgroups measured 4-5 us slower on 64 MiB (dispatch and the
        // slots' atomics)
        const unsigned blocks = (unsigned)(need < 256 ? need : 256);
        if (vec)
            hipLaunchKernelGGL((k_tensor_minmax<true>), dim3(blocks), dim3(256), 0, s, (const float*)A, n, c->mm);
        else
            hipLaunchKernelGGL((k_tensor_minmax<false>), dim3(blocks), dim3(256), 0, s, (const float*)A, n, c->mm);
        DQ_LAUNCH_CHECK("tensor_minmax");
    }
    for (int64_t a = 0; a < c->nA && !rc; ++a) {
        const void* Aa = static_cast<const char*>(A) + (size_t)a * M * K * esz;
        int8_t* Apa = c->Ap + (size_t)a * Mp * Kp;
        const size_t ro = (size_t)a * Mp;
        if (c->a_type == DQ_F32) {
            RowOut o{c->rowsum + ro, c->zeroA + ro, c->scaleA + ro, nullptr, nullptr, c->mm, c->alpha};
            rc = launch_pack_rows<SRC_F32>(Aa, M, K, Kp, Apa, o, s);
        } else if (!c->transA) {
            RowOut o{c->rowsum + ro, c->zeroA + ro, c->scaleA + ro, a_scale, a_zp, nullptr, c->alpha};
            rc = c->a_type == DQ_U8 ? launch_pack_rows<SRC_U8>(Aa, M, K, Kp, Apa, o, s)
                                    : launch_pack_rows<SRC_I8>(Aa, M, K, Kp, Apa, o, s);
        } else {
            rc = dq_launch_pack_cols8(Aa, c->a_type == DQ_U8, K, M, Kp, Apa, c->rowsum + ro, s);
            if (!rc) {
                hipLaunchKernelGGL(k_a_params, dim3((unsigned)((M + 255) / 256)), dim3(256), 0, s, M, K,
                                   c->a_type == DQ_U8, a_scale, a_zp, c->alpha, c->rowsum + ro, c->zeroA + ro,
                                   c->scaleA + ro);
                DQ_LAUNCH_CHECK("a_params");
            }
        }
    }
    if (rc) return rc;
    DqEpilogue ep;
    ep.scaleB = c->scaleB;
    ep.bias = bias;  // N values: the GEMM clamps its column index
    ep.act = DQ_ACT_IDENTITY;
    ep.alpha = 0.0f;
    ep.out = mode;
    if (c->zb_any) ep.zeroB = c->zb;
    if (Cm) {
        ep.addC = Cm;
        ep.c_rs = c_rows == 1 ? 0 : c_cols;
        ep.c_cs = c_cols == 1 ? 0 : 1;
        ep.c_mode = c_rows == 1 ? 1 : c_cols == 1 ? 2 : 3;
    }
    ep.y_scale = y_scale;
    ep.y_zp = y_zp;
    const size_t osz = q8 ? 1 : 4;  // fp32 Y and int32 sums: 4 bytes
    const size_t nY = c->ia.empty() ? 1 : c->ia.size();
    for (size_t z = 0; z < nY && !rc; ++z) {
        const size_t a = c->ia.empty() ? 0 : (size_t)c->ia[z], b = c->ib.empty() ? 0 : (size_t)c->ib[z];
        ep.scaleA = c->scaleA + a * Mp;
        ep.zeroA = c->zeroA + a * Mp;
        ep.colsumB = c->colsum + b * Np;
        if (c->zb_any) ep.rowsumA = c->rowsum + a * Mp;
        ep.C = static_cast<char*>(Y) + z * M * N * osz;
        rc = dq_launch_gemm(c->Ap + a * Mp * Kp, c->Bp + b * Np * Kp, M, N, Kp, ep, s);
    }
    return rc;
}

}  // namespace

namespace {

// Validates the types and shapes shared by both initializers and makes the
// context with every device buffer: nA packed A batches and nB packed B
// batches (B's per-column scale, zero-point and bias vectors are one set).
int make_ctx(dq_qgemm_ctx** ctx, int64_t M, int64_t N, int64_t K, int64_t nA, int64_t nB, dq_dtype a_type,
             int transA, dq_dtype b_type, int transB, dq_dtype y_type, float alpha) {
    if (M > 0x7fffffff - 256 || N > 0x7fffffff - 256) DQ_FAIL(DQ_ERR_RANGE, "M and N must fit in int32");
    if (K > DQ_QGEMM_K_MAX) DQ_FAIL(DQ_ERR_RANGE, "K = %lld exceeds %d (int32 sums)", (long long)K, DQ_QGEMM_K_MAX);
    if (a_type != DQ_F32 && a_type != DQ_U8 && a_type != DQ_I8) DQ_FAIL(DQ_ERR_TYPE, "a_type must be f32, u8 or i8");
    if (a_type == DQ_F32 && transA) DQ_FAIL(DQ_ERR_ARG, "transA is defined for an 8-bit A only");
    if (b_type != DQ_U8 && b_type != DQ_I8) DQ_FAIL(DQ_ERR_TYPE, "b_type must be u8 or i8");
    if (y_type != DQ_F32 && y_type != DQ_U8 && y_type != DQ_I8) DQ_FAIL(DQ_ERR_TYPE, "y_type must be f32, u8 or i8");
    dq_qgemm_ctx* c = new dq_qgemm_ctx();
    int rc = DQ_OK;
    if (hipGetDevice(&c->device) != hipSuccess) {
        delete c;
        DQ_FAIL(DQ_ERR_HIP, "hipGetDevice failed");
    }
    c->M = (int)M;
    c->N = (int)N;
    c->K = (int)K;
    c->Kp = (int)dq_kp((size_t)K);
    c->a_type = a_type;
    c->b_type = b_type;
    c->y_type = y_type;
    c->transA = transA ? 1 : 0;
    c->transB = transB ? 1 : 0;
    c->alpha = alpha;
    c->nA = nA;
    c->nB = nB;
    const size_t Mp = dq_mnp((size_t)M), Np = dq_mnp((size_t)N), Kp = (size_t)c->Kp;
    const size_t a_n = (size_t)nA, b_n = (size_t)nB;
    if (!rc) rc = ctx_alloc(c, (void**)&c->Bp, b_n * Np * Kp);
    if (!rc) rc = ctx_alloc(c, (void**)&c->colsum, 4 * b_n * Np);
    if (!rc) rc = ctx_alloc(c, (void**)&c->scaleB, 4 * Np);
    if (!rc) rc = ctx_alloc(c, (void**)&c->zb, 4 * Np);
    if (!rc) rc = ctx_alloc(c, (void**)&c->Ap, a_n * Mp * Kp);
    if (!rc) rc = ctx_alloc(c, (void**)&c->rowsum, 4 * a_n * Mp);
    if (!rc) rc = ctx_alloc(c, (void**)&c->zeroA, 4 * a_n * Mp);
    if (!rc) rc = ctx_alloc(c, (void**)&c->scaleA, 4 * a_n * Mp);
    if (!rc) rc = ctx_alloc(c, (void**)&c->mm, 2 * kMmSlots * sizeof(uint32_t));
    if (rc) {
        ctx_free(c);
        delete c;
        return rc;
    }
    char buf[320];
    snprintf(buf, sizeof buf, "gfx950 qgemm A:%s%s%s B:%s%s Y:%s | %s", tname(a_type),
             a_type == DQ_F32 ? " (quantized per tensor to u8)" : "", transA ? " transposed" : "",
             tname(b_type), transB ? " transposed" : "", tname(y_type),
             dq_gemm_info((int)M, (int)N, c->Kp));
    c->info = buf;
    *ctx = c;
    return DQ_OK;
}

}  // namespace

extern "C" int dq_qgemm_init(dq_qgemm_ctx** ctx, int64_t M, int64_t N, int64_t K, dq_dtype a_type,
                             int transA, dq_dtype b_type, int transB, dq_dtype y_type, float alpha) {
    if (!ctx) DQ_FAIL(DQ_ERR_ARG, "ctx is NULL");
    *ctx = nullptr;
    if (M < 1 || N < 1 || K < 1) DQ_FAIL(DQ_ERR_ARG, "M, N, K must be >= 1");
    return make_ctx(ctx, M, N, K, 1, 1, a_type, transA, b_type, transB, y_type, alpha);
}

extern "C" int dq_qgemm_init_batched(dq_qgemm_ctx** ctx, int batch_rank, const int64_t* a_batch,
                                     const int64_t* b_batch, int64_t M, int64_t N, int64_t K,
                                     dq_dtype a_type, dq_dtype b_type) {
    if (!ctx) DQ_FAIL(DQ_ERR_ARG, "ctx is NULL");
    *ctx = nullptr;
    if (M < 1 || N < 1 || K < 1) DQ_FAIL(DQ_ERR_ARG, "M, N, K must be >= 1");
    if (batch_rank < 0 || batch_rank > DQ_QGEMM_BATCH_RANK_MAX)
        DQ_FAIL(DQ_ERR_ARG, "batch_rank must be in [0, %d]", DQ_QGEMM_BATCH_RANK_MAX);
    if (batch_rank > 0 && (!a_batch || !b_batch)) DQ_FAIL(DQ_ERR_ARG, "a_batch and b_batch must not be NULL");
    // the broadcast batch shape (numpy.matmul's rule) and the batch counts
    int64_t yb[DQ_QGEMM_BATCH_RANK_MAX];
    int64_t nA = 1, nB = 1, nY = 1;
    for (int d = 0; d < batch_rank; ++d) {
        const int64_t da = a_batch[d], db = b_batch[d];
        if (da < 1 || db < 1) DQ_FAIL(DQ_ERR_ARG, "batch dimension %d must be >= 1 (A %lld, B %lld)", d,
                                      (long long)da, (long long)db);
        if (da != db && da != 1 && db != 1)
            DQ_FAIL(DQ_ERR_ARG, "batch dimension %d does not broadcast (A %lld, B %lld)", d, (long long)da,
                    (long long)db);
        if (da > DQ_QGEMM_BATCH_MAX || db > DQ_QGEMM_BATCH_MAX)
            DQ_FAIL(DQ_ERR_RANGE, "more than %d batches", DQ_QGEMM_BATCH_MAX);
        yb[d] = da == 1 ? db : da;
        nA *= da;
        nB *= db;
        nY *= yb[d];
        if (nA > DQ_QGEMM_BATCH_MAX || nB > DQ_QGEMM_BATCH_MAX || nY > DQ_QGEMM_BATCH_MAX)
            DQ_FAIL(DQ_ERR_RANGE, "more than %d batches", DQ_QGEMM_BATCH_MAX);
    }
    if (nB == 1) {
        // one B: A's batches are rows of a single product ([nA * M, K])
        if (nA * M > 0x7fffffff - 256) DQ_FAIL(DQ_ERR_RANGE, "batches * M must fit in int32");
        const int rc = make_ctx(ctx, nA * M, N, K, 1, 1, a_type, 0, b_type, 0, DQ_F32, 1.0f);
        if (!rc) (*ctx)->batched = 1;
        return rc;
    }
    const int rc = make_ctx(ctx, M, N, K, nA, nB, a_type, 0, b_type, 0, DQ_F32, 1.0f);
    if (rc) return rc;
    dq_qgemm_ctx* c = *ctx;
    c->batched = 1;
    c->ia.resize((size_t)nY);
    c->ib.resize((size_t)nY);
    // Y batch z in row-major order of yb; A's (B's) batch number counts its
    // own dimensions, a broadcast dimension (1) contributing index 0
    for (int64_t z = 0; z < nY; ++z) {
        int64_t rem = z, ia = 0, ib = 0, sa = 1, sb = 1;
        for (int d = batch_rank - 1; d >= 0; --d) {
            const int64_t i = rem % yb[d];
            rem /= yb[d];
            if (a_batch[d] > 1) ia += i * sa;
            if (b_batch[d] > 1) ib += i * sb;
            sa *= a_batch[d];
            sb *= b_batch[d];
        }
        c->ia[(size_t)z] = (int32_t)ia;
        c->ib[(size_t)z] = (int32_t)ib;
    }
    char buf[96];
    snprintf(buf, sizeof buf, " | %lld products (%lld A, %lld B batches)", (long long)nY, (long long)nA,
             (long long)nB);
    c->info += buf;
    return DQ_OK;
}

extern "C" int dq_qgemm_set_b(dq_qgemm_ctx* c, const void* B, const float* b_scale, int64_t b_scale_len,
                              const void* b_zero_point, int64_t b_zero_point_len, void* stream) {
    if (!c) DQ_FAIL(DQ_ERR_STATE, "context is NULL");
    if (!B || !b_scale) DQ_FAIL(DQ_ERR_ARG, "B and b_scale must not be NULL");
    if (b_scale_len != 1 && b_scale_len != c->N) DQ_FAIL(DQ_ERR_ARG, "b_scale must have 1 or N entries");
    if (b_zero_point && b_zero_point_len != 1 && b_zero_point_len != c->N)
        DQ_FAIL(DQ_ERR_ARG, "b_zero_point must have 1 or N entries");
    int rc = check_device(c);
    if (rc) return rc;
    hipStream_t s = (hipStream_t)stream;
    const int N = c->N, K = c->K, Kp = c->Kp;
    const bool u8 = c->b_type == DQ_U8;
    const int Np = (int)dq_mnp((size_t)N);
    for (int64_t b = 0; b < c->nB && !rc; ++b) {
        const void* Bb = static_cast<const char*>(B) + (size_t)b * K * N;
        int8_t* Bpb = c->Bp + (size_t)b * Np * Kp;
        int32_t* cs = c->colsum + (size_t)b * Np;
        if (c->transB) {
            RowOut o{cs, nullptr, nullptr, nullptr, nullptr, nullptr, 1.0f};
            rc = u8 ? launch_pack_rows<SRC_U8>(Bb, N, K, Kp, Bpb, o, s)
                    : launch_pack_rows<SRC_I8>(Bb, N, K, Kp, Bpb, o, s);
        } else {
            rc = dq_launch_pack_cols8(Bb, u8, K, N, Kp, Bpb, cs, s);
        }
    }
    if (rc) return rc;
    hipLaunchKernelGGL(k_b_params, dim3((unsigned)((Np + 255) / 256)), dim3(256), 0, s, N, Np, u8, b_scale,
                       (int)b_scale_len, b_zero_point, (int)b_zero_point_len, c->scaleB, c->zb);
    DQ_LAUNCH_CHECK("b_params");
    // whether any column's sb - b_zp is non-zero (decides the row-sum term)
    std::vector<int32_t> hz((size_t)N);
    DQ_HIP_CHECK(hipMemcpyAsync(hz.data(), c->zb, 4 * (size_t)N, hipMemcpyDeviceToHost, s));
    DQ_HIP_CHECK(hipStreamSynchronize(s));
    c->zb_any = 0;
    for (int32_t z : hz) c->zb_any |= z != 0;
    c->b_set = 1;
    return DQ_OK;
}

extern "C" int dq_qgemm_forward(dq_qgemm_ctx* c, const void* A, const float* a_scale, const void* a_zero_point,
                                const int32_t* C, int64_t c_rows, int64_t c_cols, const float* bias,
                                const float* y_scale, const void* y_zero_point, void* Y, void* stream) {
    if (!c) DQ_FAIL(DQ_ERR_STATE, "context is NULL");
    const int mode = c->y_type == DQ_U8 ? DQ_OUT_U8 : c->y_type == DQ_I8 ? DQ_OUT_I8 : DQ_OUT_F32;
    return run(c, A, a_scale, a_zero_point, C, c_rows, c_cols, bias, y_scale, y_zero_point, Y, mode,
               (hipStream_t)stream);
}

extern "C" int dq_qgemm_forward_accumulators(dq_qgemm_ctx* c, const void* A, const float* a_scale,
                                             const void* a_zero_point, const int32_t* C, int64_t c_rows,
                                             int64_t c_cols, int32_t* acc, void* stream) {
    return run(c, A, a_scale, a_zero_point, C, c_rows, c_cols, nullptr, nullptr, nullptr, acc, DQ_OUT_ACC,
               (hipStream_t)stream);
}

extern "C" const char* dq_qgemm_info(const dq_qgemm_ctx* c) { return c ? c->info.c_str() : nullptr; }

extern "C" void dq_qgemm_release(dq_qgemm_ctx* c) {
    if (!c) return;
    ctx_free(c);
    delete c;
}
