// dq_kernels.h -- host launchers of libdqip's gfx950 kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dqip.h"

// Packed operands (MFMA fragment order, see frag_offset in dq_device.h):
// sA [Mp x Kp] holds uA - 128, iBp [Np x Kp] holds iB transposed (column j
// of B is packed row j). K is padded to Kp (multiple of 256) with zero codes
// in iBp, so the padding adds nothing to a sum; M and N are padded to
// multiples of 256 (the largest tile) and the padding rows / columns are
// never stored to C. Per-column vectors (scaleB, colsum) hold Np entries so
// the epilogue can read them in 16-byte vectors; a bias needs only N (the
// kernels clamp its column index).
constexpr int kKpAlign = 256;
constexpr int kMNAlign = 256;

inline size_t dq_kp(size_t K) { return (K + kKpAlign - 1) / kKpAlign * kKpAlign; }
inline size_t dq_mnp(size_t X) { return (X + kMNAlign - 1) / kMNAlign * kMNAlign; }

// Optional timing of one launcher call: the first kernel it launches records
// `start` when it begins and the last records `stop` when it ends (taken from
// the dispatches themselves, hipExtLaunchKernel), so the elapsed time is the
// kernels' own. NULL events: no timing.
struct DqTiming {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};

// Per-row dynamic quantization of A [M,K] (fp32 or bf16):
// sA (packed, uA - 128), scaleA [M], zeroA [M].
int dq_launch_quant_rows(const void* A, bool bf16, int M, int K, int Kp, int8_t* sA,
                         float* scaleA, int32_t* zeroA, hipStream_t s, DqTiming t = {});

// B [K,N] -> iBp (packed, zero K padding), colsum [N], and for an fp32/bf16 B
// also scaleB [N] (per-column symmetric quantization). For an int8 B the
// codes are packed as given and scaleB is left alone.
// amax: N words of scratch (fp32 / bf16 B only).
int dq_launch_quant_cols(const void* B, dq_dtype typeB, int K, int N, int Kp, int avoid,
                         int8_t* iBp, float* scaleB, int32_t* colsum, uint32_t* amax,
                         hipStream_t s, DqTiming t = {});

// 8-bit src [K, R] (row-major, R columns) -> packed [Rp x Kp]: column r of
// src becomes packed row r, as int8 (uint8 codes minus 128), K padded with
// zeros; sums[r] = sum over k of the packed codes.
int dq_launch_pack_cols8(const void* src, bool u8, int K, int R, int Kp, int8_t* dst,
                         int32_t* sums, hipStream_t s);

// The quantized matrix products (qgemm.hip): packs of an 8-bit [R, K] source
// by rows, and of an fp32 [M, K] tensor quantized per tensor to uint8.

// Inspection: packed sA -> uA [M,K]; packed iBp -> iB [K,N].
int dq_launch_unpack_a(const int8_t* sA, int M, int K, int Kp, uint8_t* uA, hipStream_t s);
int dq_launch_unpack_b(const int8_t* iBp, int K, int N, int Kp, int8_t* iB, hipStream_t s);

enum { DQ_OUT_F32 = 0, DQ_OUT_BF16 = 1, DQ_OUT_ACC = 2, DQ_OUT_U8 = 3, DQ_OUT_I8 = 4 };

struct DqEpilogue {
    const float* scaleA;
    const int32_t* zeroA;
    const float* scaleB;
    const int32_t* colsumB;
    const float* bias;  // N values; NULL: no bias add
    int act;            // dq_act
    float alpha;        // leaky-ReLU slope
    int out;            // DQ_OUT_*
    void* C;            // [M,N]
    // optional terms of the quantized matrix products (all NULL for dqip):
    const int32_t* rowsumA = nullptr;  // with zeroB: sum += rowsumA[i] * zeroB[j]
    const int32_t* zeroB = nullptr;
    const int32_t* addC = nullptr;     // int32 added to the sum, at i * c_rs + j * c_cs
    long long c_rs = 0, c_cs = 0;
    int c_mode = 0;                    // 0 none, 1 per column (or one value), 2 per row, 3 [M,N]
    const float* y_scale = nullptr;    // DQ_OUT_U8 / DQ_OUT_I8: device scalar
    const void* y_zp = nullptr;        // device scalar of the output's type (NULL: 0)
};

// acc = sA * iB + (128 - zeroA[i]) * colsumB[j] (+ rowsumA[i] * zeroB[j])
// (+ addC[i, j]), then the epilogue.
int dq_launch_gemm(const int8_t* sA, const int8_t* iBp, int M, int N, int Kp,
                   const DqEpilogue& ep, hipStream_t s, DqTiming t = {});

// A short description of the kernels dq_launch_gemm picks for a shape.
const char* dq_gemm_info(int M, int N, int Kp);

// The tile configuration dq_launch_gemm picks: 2 = 256x256, 1 = 128x128,
// 0 = 32x32 (small or skinny products).
int dq_gemm_config(int M, int N);

// The inner product of a small problem in one launch (dqip_small.hip): the
// rows of A quantized inside the GEMM's workgroups. Applies when the GEMM
// would take 32x32 tiles, K % 16 == 0, K <= kDqipSmallKMax and A is 16-byte
// aligned; B is packed (constant). Writes C per ep (F32, BF16 or ACC) and,
// for inspection, sA / scaleA / zeroA as the row quantizer does.
constexpr int kDqipSmallKMax = 1024;
bool dq_dqip_small_fits(int M, int N, int K, const void* A);
int dq_launch_dqip_small(const void* A, bool bf16, int M, int N, int K, int Kp, const int8_t* iBp,
                         const DqEpilogue& ep, int8_t* sA, float* scaleA, int32_t* zeroA, hipStream_t s,
                         DqTiming t = {});
