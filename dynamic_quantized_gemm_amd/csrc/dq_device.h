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

// Four fp32 values to packed bf16 with the gfx950 conversion instruction
// (v_cvt_pk_bf16_f32: round to nearest even, NaN stays NaN).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u2 f32x4_to_bf16x4(f4 v) {
    const f2 lo = {v[0], v[1]}, hi = {v[2], v[3]};
    const bf16x2 a = __builtin_convertvector(lo, bf16x2);
    const bf16x2 b = __builtin_convertvector(hi, bf16x2);
    const u2 r = {__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b)};
    return r;
}

// ReLU on four packed bf16 values, after the rounding: max(x, 0) per 16-bit
// signed integer (v_pk_max_i16). A bf16 with its sign bit set (a negative
// value or -0) is a negative int16 and becomes +0, any other is kept; and
// rounding to nearest even is monotone and maps negatives to negatives or
// -0, so bf16(relu(v)) == relu(bf16(v)) bit for bit. Two packed operations
// replace four fp32 max operations.
__device__ __forceinline__ uint32_t relu_bf16x2(uint32_t w) {
    uint32_t r;
    asm("v_pk_max_i16 %0, %1, 0" : "=v"(r) : "v"(w));
    return r;
}
__device__ __forceinline__ u2 relu_bf16x4(u2 p) {
    const u2 r = {relu_bf16x2(p[0]), relu_bf16x2(p[1])};
    return r;
}

// saturate(r + zp) into [lo, hi] for an integral float r (possibly +-inf):
// clamping r to [lo - zp, hi - zp] first is exact, since both bounds are
// small integers, and keeps the int conversion in range.
__device__ __forceinline__ int sat_add(float r, int zp, int lo, int hi) {
    float c = __builtin_fminf(__builtin_fmaxf(r, (float)(lo - zp)), (float)(hi - zp));
    return (int)c + zp;
}

// Quotient x / s where only its rounding to an integer matters (the
// quantizers). y = 1/s is the correctly rounded reciprocal, computed once
// per scale. One residual step, q = q0 + (x - q0*s) * y with both products
// fused, returns the IEEE quotient for every |x/s| >= 1/4 (checked over all
// 2^32 fp32 x for a set of scales), so rne(q) matches rne(x / s) at every tie
// and boundary; below 1/4 both round to 0. Beyond 2^24 the product q0 is
// used as is: it saturates exactly like the quotient. The residual is exact
// only while x - q0*s stays clear of the subnormal range: with |s| below
// about 2^-120 the rounded code differs from the IEEE one for a few x (an
// exhaustive check found 2 to 32 of 2^32 for scales 1.2e-38 .. 3e-39, none
// from 2^-100 up). So the step is used for 2^-100 <= |s| and a normal
// reciprocal; any other scale takes the IEEE division.
struct QDiv {
    float s, y;
    bool fast;
};

__device__ __forceinline__ QDiv make_qdiv(float s) {
    QDiv d;
    d.s = s;
    d.y = 1.0f / s;
    const float ay = __builtin_fabsf(d.y);
    d.fast = __builtin_fabsf(s) >= 0x1p-100f && ay >= 1.17549435e-38f && ay <= 3.40282347e+38f;
    return d;
}

__device__ __forceinline__ float qdiv(float x, const QDiv& d) {
    if (!d.fast) return x / d.s;
    const float q0 = x * d.y;
    if (!(__builtin_fabsf(q0) <= 16777216.0f)) return q0;
    const float r = __builtin_fmaf(-q0, d.s, x);
    return __builtin_fmaf(r, d.y, q0);
}

// The residual step alone, for callers that have checked d.fast and whose
// quotients are bounded (|x / s| <= 2^24) by construction.
__device__ __forceinline__ float qdiv_fast(float x, const QDiv& d) {
    const float q0 = x * d.y;
    const float r = __builtin_fmaf(-q0, d.s, x);
    return __builtin_fmaf(r, d.y, q0);
}

// Division of a 32-bit unsigned n by a runtime constant d >= 1 with one
// multiply-high: q = (umulhi(n, m) + n) >> s, s = ceil(log2 d),
// m = floor(2^32 (2^s - d) / d) + 1 (Granlund & Montgomery, "Division by
// invariant integers using multiplication", PLDI 1994, round-up variant).
struct FastDiv {
    uint32_t d, m, s;
};

inline FastDiv make_fastdiv(uint32_t d) {
    FastDiv f;
    f.d = d;
    f.s = 0;
    while ((1ull << f.s) < d) ++f.s;
    f.m = (uint32_t)(((1ull << 32) * ((1ull << f.s) - d)) / d + 1);
    return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) {
    uint32_t hi = __umulhi(n, f.m);
    return (uint32_t)(((uint64_t)hi + n) >> f.s);
}

// Byte offset of element (r, k) of an operand packed in MFMA fragment order:
// 1 KiB fragments of 32 rows x 32 k, fragment (r/32, k/32) at index
// (r/32) * KF + k/32 (KF = Kp/32); inside it, lane slot (r%32) + 32*((k%32)/16)
// holds the 16 codes k%32 in [0,16) or [16,32) of row r. One ds_read_b128 /
// global_load_dwordx4 per lane at slot*16 yields the v_mfma_i32_32x32x32_i8
// operand for rows (or columns) r%32.
__host__ __device__ __forceinline__ size_t frag_offset(size_t r, size_t k, size_t KF) {
    return (((r >> 5) * KF + (k >> 5)) << 10) + (((r & 31) + ((k & 16) << 1)) << 4) + (k & 15);
}

// s_waitcnt on the vector-memory counter alone: wait until at most N vector
// memory operations of this wave are outstanding (encoding of the gfx9
// family: vmcnt[3:0] in bits 3:0 and vmcnt[5:4] in bits 15:14; expcnt in
// bits 6:4 and lgkmcnt in bits 11:8 left at their maxima, i.e. not waited on).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// The same, and also wait until every LDS operation of this wave has
// completed (lgkmcnt 0).
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
    static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}

// Wait until every LDS operation of this wave has completed (lgkmcnt 0),
// leaving vector memory operations in flight.
__device__ __forceinline__ void wait_lgkm0() {
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

// 16 bytes per lane from global memory straight into LDS (gfx950
// global_load_lds_dwordx4): the wave's 64 lanes land as one contiguous
// 1 KiB block at lds_block (wave-uniform), lane l at offset 16 l. A plain
// __device__ function (not a lambda, which would also be compiled for the
// host and invalidate the kernel there).
__device__ __forceinline__ void copy16_to_lds(const void* gsrc, void* lds_block) {
    __builtin_amdgcn_global_load_lds(gsrc, lds_block, 16, 0, 0);
}

// Workgroup barrier without a memory fence: no wait on outstanding vector
// memory operations (the caller has waited for what it needs). The empty
// asm statements with a memory clobber keep the compiler from moving memory
// accesses across it; the scheduling barrier does the same for the
// machine scheduler.
// Keeps a lane's loads issued ahead of the work that uses them: the memory
// clobber stops the loads from sinking below it and the scheduling barrier
// stops later arithmetic from being hoisted above it, so all of them are in
// flight before the first wait.
__device__ __forceinline__ void issue_fence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// A wave reading back what its own lanes just wrote to LDS: the LDS
// operations of one wave complete in order, so only the compiler has to be
// kept from moving the reads above the writes (it may take two differently
// typed views of one array for unrelated memory); the memory clobbers do
// that, and the wait drains the writes.
__device__ __forceinline__ void wave_lds_fence() {
    asm volatile("" ::: "memory");
    wait_lgkm0();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
}

// MFMA results and the instructions that read them. The matrix core does
// not interlock its results against later VALU instructions: the ISA's table
// of required independent instructions (CDNA3 / CDNA4 instruction set
// references, dependency resolution for XDL / MFMA operations) asks for
// NumPasses + 3 wait states between an XDL instruction that writes
// accumulator registers and a VALU instruction or v_accvgpr_read that reads
// them (RAW), with one more on gfx950 for ops of more than two passes; the
// largest MFMA here has 16 passes, so at most 20. The compiler inserts these
// wait states for reads it can see, but not for a read inside inline
// assembly (acc_read below), whose operand it does not inspect for this
// hazard. Every kernel therefore crosses one drain of kMfmaDrainWaitStates
// (s_nop n gives n + 1 wait states) between its last MFMA and its first
// read of the accumulators; the scheduling barriers keep the compiler from
// moving an MFMA or a read across it. Cost: 24 cycles once per wave.
constexpr int kMfmaReadWaitStates = 20;
constexpr int kMfmaDrainWaitStates = 24;
static_assert(kMfmaDrainWaitStates >= kMfmaReadWaitStates, "drain shorter than the ISA's requirement");
__device__ __forceinline__ void mfma_result_drain() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Reads one accumulator register that an MFMA left in the accumulation
// register file (AGPRs). Handing the value to an explicit read at its point
// of use keeps the register allocator from copying every accumulator into
// ordinary VGPRs at once when a large tile's main loop ends (which spills).
__device__ __forceinline__ int32_t acc_read(int32_t a) {
    int32_t v;
    asm("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
    return v;
}

// fp32 <-> an unsigned integer with the same order, for atomicMin /
// atomicMax on fp32 values; f2ord(+0.0f) = 0x80000000, and -0 maps to +0.
__device__ __forceinline__ uint32_t f2ord(float f) {
    const uint32_t u = __float_as_uint(f + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ord2f(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// Wave-wide min / max over 64 lanes, returned as a wave-uniform value.
// Within each row of 16 lanes, four DPP moves combine every lane with its
// partners (quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror, row_mirror:
// after them every lane of the row holds the row's result); the four rows
// are then combined from lanes 0, 16, 32 and 48 with v_readlane. DPP moves
// stay inside the VALU (no LDS round trip as a shuffle would take), so the
// chain is short.
enum : int { kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppRowHalfMirror = 0x141, kDppRowMirror = 0x140 };

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_f(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ float wave_min_uniform(float v) {
    v = __builtin_fminf(v, dpp_f<kDppXor1>(v));
    v = __builtin_fminf(v, dpp_f<kDppXor2>(v));
    v = __builtin_fminf(v, dpp_f<kDppRowHalfMirror>(v));
    v = __builtin_fminf(v, dpp_f<kDppRowMirror>(v));
    return __builtin_fminf(__builtin_fminf(lane_f(v, 0), lane_f(v, 16)),
                           __builtin_fminf(lane_f(v, 32), lane_f(v, 48)));
}
__device__ __forceinline__ float wave_max_uniform(float v) {
    v = __builtin_fmaxf(v, dpp_f<kDppXor1>(v));
    v = __builtin_fmaxf(v, dpp_f<kDppXor2>(v));
    v = __builtin_fmaxf(v, dpp_f<kDppRowHalfMirror>(v));
    v = __builtin_fmaxf(v, dpp_f<kDppRowMirror>(v));
    return __builtin_fmaxf(__builtin_fmaxf(lane_f(v, 0), lane_f(v, 16)),
                           __builtin_fmaxf(lane_f(v, 32), lane_f(v, 48)));
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
