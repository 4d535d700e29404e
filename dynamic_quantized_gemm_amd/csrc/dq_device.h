// dq_device.h -- device helpers shared by the gfx950 kernels of libdqip.
//
// All fp32 arithmetic here is IEEE: the library is built with
// -ffp-contract=off (no silent fusing of a multiply into an add) and without
// fast-math, so `/` is the correctly rounded division and every operation
// rounds once, in the order written.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dqip.h"

namespace dq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned u4 __attribute__((ext_vector_type(4)));
typedef unsigned u2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Round half to even (v_rndne_f32).
__device__ __forceinline__ float rne(float x) { return __builtin_rintf(x); }

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
    return __uint_as_float(b16 << 16);
}

// fp32 -> bf16 bits, round to nearest even on the 16 dropped bits; a NaN
// stays a (quiet) NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// saturate(r + zp) into [lo, hi] for an integral float r (possibly +-inf):
// clamping r to [lo - zp, hi - zp] first is exact, since both bounds are
// small integers, and keeps the int conversion in range.
__device__ __forceinline__ int sat_add(float r, int zp, int lo, int hi) {
    float c = __builtin_fminf(__builtin_fmaxf(r, (float)(lo - zp)), (float)(hi - zp));
    return (int)c + zp;
}

// Wave-wide min / max over 64 lanes (butterfly over xor shuffles).
__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = __builtin_fminf(v, __shfl_xor(v, o, kWave));
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

}  // namespace dq

// --- host-side helpers shared by the library's translation units ---------

// Thread-local error message for dqip_last_error().
void dq_set_error(const char* fmt, ...);

#define DQ_FAIL(code, ...)               \
    do {                                 \
        dq_set_error(__VA_ARGS__);       \
        return (code);                   \
    } while (0)

#define DQ_HIP_CHECK(expr)                                                         \
    do {                                                                           \
        hipError_t e_ = (expr);                                                    \
        if (e_ != hipSuccess)                                                      \
            DQ_FAIL(DQ_ERR_HIP, "%s failed: %s", #expr, hipGetErrorString(e_));    \
    } while (0)

// checks for a launch error right after a kernel launch
#define DQ_LAUNCH_CHECK(name)                                                     \
    do {                                                                          \
        hipError_t e_ = hipGetLastError();                                        \
        if (e_ != hipSuccess)                                                     \
            DQ_FAIL(DQ_ERR_HIP, "launch of %s failed: %s", name, hipGetErrorString(e_)); \
    } while (0)
