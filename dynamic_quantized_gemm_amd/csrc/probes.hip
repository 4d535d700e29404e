// probes.hip -- measurement probes: what the hardware reaches on its own,
// next to the published peaks, as context for the kernels' roofline
// fractions. Not operations of the method.
//
// k_probe_mfma<SHAPE>: every wave runs the int8 matrix-core work of the
// GEMM's 128x128 wave tile with nothing else, operands from registers only
// (no global or LDS traffic, no barriers): SHAPE 32 as 16 accumulator blocks
// of 32x32 with v_mfma_i32_32x32x32_i8, SHAPE 16 as 64 blocks of 16x16 with
// v_mfma_i32_16x16x64_i8 (the GEMM's instruction, in its order: one A block
// against every B block in turn). Two operand sets alternate from one
// iteration to the next, so the inputs toggle as they do when a GEMM walks
// along K; the operand bytes are the caller's (random codes, or zeros to
// see how much the data itself costs). An iteration is 32 x 32x32x32
// multiply-adds either way: 32 MFMAs of 32x32x32 or 64 of 16x16x64.
//
// k_probe_copy: a plain copy, 16 bytes a lane and four loads a lane in
// flight, non-temporal: the simplest kernel that moves HBM bytes both ways.
#include "dq_device.h"

#include <hip/hip_ext.h>

namespace {

template <int SHAPE>
__global__ void __launch_bounds__(256) k_probe_mfma(const int8_t* __restrict__ ops, int iters,
                                                    int32_t* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    uint32_t t = 0;
    if constexpr (SHAPE == 32) {
        // 16 operand fragments per set (4 "A" + 4 "B"), two sets; each lane
        // reads its 16 bytes of a 1 KiB fragment; the waves of a workgroup
        // and the workgroups read different bytes of the 64 KiB buffer
        const int8_t* base = ops + (size_t)((blockIdx.x * 4 + wave) % 4) * 16384 + lane * 16;
        dq::v4i fa[2][4], fb[2][4];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                fa[s][i] = *reinterpret_cast<const dq::v4i*>(base + (s * 8 + i) * 1024);
                fb[s][i] = *reinterpret_cast<const dq::v4i*>(base + (s * 8 + 4 + i) * 1024);
            }
        dq::v16i acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fb[s][j], fa[s][i], acc[i][j], 0, 0, 0);
        }
        dq::mfma_result_drain();
        // keep every accumulator live: one wrapping sum per lane
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) t += (uint32_t)dq::acc_read(acc[i][j][r]);
    } else {
        // 16 blocks per set (8 A + 8 B), two sets: 32 KiB of the buffer per
        // wave, two different halves per workgroup
        const int8_t* base = ops + (size_t)(wave & 1) * 32768 + lane * 16;
        dq::v4i fa[2][8], fb[2][8];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                fa[s][i] = *reinterpret_cast<const dq::v4i*>(base + (s * 16 + i) * 1024);
                fb[s][i] = *reinterpret_cast<const dq::v4i*>(base + (s * 16 + 8 + i) * 1024);
            }
        dq::v4i acc[8][8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[i][j] = dq::v4i{0, 0, 0, 0};
        // in-place inline MFMAs as in the GEMM; the zeros are pinned in
        // their AGPRs and drained before the first MFMA reads them as srcC
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) asm volatile("" : "+a"(acc[i][j]));
        dq::mfma_result_drain();
        // an iteration is one operand set's 64 MFMAs; the sets alternate
        auto pass = [&](int s) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0"
                                 : "+a"(acc[i][j]) : "v"(fb[s][j]), "v"(fa[s][i]));
        };
        for (int it = 0; it + 1 < iters; it += 2) {
            pass(0);
            pass(1);
        }
        if (iters & 1) pass(0);
        dq::mfma_result_drain();
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) t += (uint32_t)dq::acc_read(acc[i][j][r]);
    }
    sink[(size_t)blockIdx.x * 256 + threadIdx.x] = (int32_t)t;
}

// one block moves 16 KiB: each thread requests its four 16-byte pieces
// (1 KiB contiguous per wave instruction) before it stores any of them
__global__ void __launch_bounds__(256) k_probe_copy(const dq::v4i* __restrict__ src, dq::v4i* __restrict__ dst,
                                                    size_t n16) {
    const size_t b = (size_t)blockIdx.x * 1024 + threadIdx.x;
    dq::v4i v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
        if (b + q * 256 < n16) v[q] = __builtin_nontemporal_load(src + b + q * 256);
#pragma unroll
    for (int q = 0; q < 4; ++q)
        if (b + q * 256 < n16) __builtin_nontemporal_store(v[q], dst + b + q * 256);
}

}  // namespace

extern "C" int dq_probe_mfma_loop(const void* operands, int shape, int iters, int workgroups, int32_t* sink,
                                  void* stream) {
    if (!operands || !sink) DQ_FAIL(DQ_ERR_ARG, "operands and sink must be device pointers");
    if (shape != 16 && shape != 32) DQ_FAIL(DQ_ERR_ARG, "shape must be 16 (16x16x64) or 32 (32x32x32)");
    if (iters < 1 || workgroups < 1) DQ_FAIL(DQ_ERR_ARG, "iters and workgroups must be >= 1");
    if (shape == 32)
        hipLaunchKernelGGL(k_probe_mfma<32>, dim3((unsigned)workgroups), dim3(256), 0, (hipStream_t)stream,
                           (const int8_t*)operands, iters, sink);
    else
        hipLaunchKernelGGL(k_probe_mfma<16>, dim3((unsigned)workgroups), dim3(256), 0, (hipStream_t)stream,
                           (const int8_t*)operands, iters, sink);
    DQ_LAUNCH_CHECK("probe mfma");
    return DQ_OK;
}

extern "C" int dq_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
    if (!src || !dst) DQ_FAIL(DQ_ERR_ARG, "src and dst must be device pointers");
    if (bytes % 16 || (uintptr_t)src % 16 || (uintptr_t)dst % 16)
        DQ_FAIL(DQ_ERR_ARG, "bytes and both pointers must be multiples of 16");
    if (bytes == 0) return DQ_OK;
    const size_t blocks = (bytes / 16 + 1023) / 1024;
    if (blocks > 0x7fffffffu) DQ_FAIL(DQ_ERR_ARG, "copy too large for one launch");
    hipLaunchKernelGGL(k_probe_copy, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       (const dq::v4i*)src, (dq::v4i*)dst, bytes / 16);
    DQ_LAUNCH_CHECK("probe copy");
    return DQ_OK;
}
