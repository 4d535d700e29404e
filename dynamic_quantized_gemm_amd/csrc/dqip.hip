// dqip.hip -- the C ABI of libdqip: context, argument checks, buffers.
//
// The API follows Simd "SynetDynamicQuantizedInnerProduct16b Class
// Reference": Init() (re-creates the context only when a parameter changed),
// Enable(), InternalBufferSize(), ExternalBufferSize(), Info(), SetParams(),
// Forward(), Clear(). Device memory is allocated only by dqip_init,
// dqip_set_params (never), and the first dqip_forward with buf == NULL.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "dq_device.h"
#include "dq_kernels.h"

static thread_local char g_err[512];

void dq_set_error(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
}

extern "C" const char* dqip_last_error(void) { return g_err; }

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Offsets of the per-call work buffer (external `buf` or the internal one).
struct WorkLayout {
    size_t sA, scaleA, zeroA;        // quantized A
    size_t iBt, scaleB, colsum, amax;  // quantized B (non-constant B only)
    size_t total;
};

}  // namespace

struct dqip_ctx {
    int device;
    size_t M, N, K, Kp;
    dq_dtype typeA, typeB, typeC;
    int constB, bias, avoid;
    dq_act act;
    float alpha;
    int params_set;
    // context-owned device memory
    int8_t* iBt;       // [Np x Kp] packed (constant B)
    float* scaleB;     // [Np]    (constant B)
    int32_t* colsum;   // [Np]    (constant B)
    uint32_t* amax;    // [N]     column-maxima scratch for set_params
    float* biasv;      // [Np]    (bias flag; zero past N)
    void* work;        // fallback work buffer (first forward with buf NULL)
    size_t owned_bytes;
    WorkLayout lay;
    std::string info;
    // per-phase timing: a start and a stop event per phase of each recorded
    // call, and which phases of the call launched kernels
    std::vector<hipEvent_t> prof_events;
    std::vector<uint8_t> prof_ran;
    int prof_capacity = 0;
    int prof_calls = 0;
};

namespace {

// Work buffer: packed sA [Mp x Kp], scaleA, zeroA [M]; for a non-constant B
// also packed iB [Np x Kp], scaleB, colsum [Np] and the column maxima [N].
WorkLayout make_layout(size_t M, size_t N, size_t Kp, int constB) {
    WorkLayout l{};
    const size_t Mp = dq_mnp(M), Np = dq_mnp(N);
    size_t o = 0;
    l.sA = o;
    o = align_up(o + Mp * Kp);
    l.scaleA = o;
    o = align_up(o + 4 * M);
    l.zeroA = o;
    o = align_up(o + 4 * M);
    if (!constB) {
        l.iBt = o;
        o = align_up(o + Np * Kp);
        l.scaleB = o;
        o = align_up(o + 4 * Np);
        l.colsum = o;
        o = align_up(o + 4 * Np);
        l.amax = o;
        o = align_up(o + 4 * N);
    }
    l.total = o;
    return l;
}

void free_profile_events(dqip_ctx* c) {
    for (hipEvent_t e : c->prof_events) (void)hipEventDestroy(e);
    c->prof_events.clear();
    c->prof_ran.clear();
    c->prof_capacity = 0;
    c->prof_calls = 0;
}

constexpr int kEventsPerCall = 2 * DQ_PHASES;

// Timing events for phase `p` of the current call (none when not profiling
// or when the capacity is used up); marks the phase as run.
DqTiming prof_phase(dqip_ctx* c, int p) {
    DqTiming t;
    if (c->prof_calls >= c->prof_capacity) return t;
    t.start = c->prof_events[(size_t)kEventsPerCall * c->prof_calls + 2 * p];
    t.stop = c->prof_events[(size_t)kEventsPerCall * c->prof_calls + 2 * p + 1];
    c->prof_ran[c->prof_calls] |= (uint8_t)(1u << p);
    return t;
}

void prof_call_done(dqip_ctx* c) {
    if (c->prof_calls < c->prof_capacity) ++c->prof_calls;
}

void free_ctx_memory(dqip_ctx* c) {
    void* ptrs[] = {c->iBt, c->scaleB, c->colsum, c->amax, c->biasv, c->work};
    for (void* p : ptrs)
        if (p) (void)hipFree(p);
    c->iBt = nullptr;
    c->scaleB = nullptr;
    c->colsum = nullptr;
    c->amax = nullptr;
    c->biasv = nullptr;
    c->work = nullptr;
    c->owned_bytes = 0;
}

int dev_alloc(dqip_ctx* c, void** p, size_t bytes) {
    if (const char* f = getenv("DQIP_FAIL_ALLOC")) {
        if (f[0] == '1') DQ_FAIL(DQ_ERR_ALLOC, "device allocation of %zu bytes refused (DQIP_FAIL_ALLOC)", bytes);
    }
    hipError_t e = hipMalloc(p, bytes ? bytes : 1);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        *p = nullptr;
        DQ_FAIL(DQ_ERR_ALLOC, "hipMalloc(%zu) failed: %s", bytes, hipGetErrorString(e));
    }
    c->owned_bytes += bytes;
    return DQ_OK;
}

const char* dtype_name(dq_dtype t) {
    switch (t) {
        case DQ_F32: return "f32";
        case DQ_BF16: return "bf16";
        case DQ_I8: return "i8";
        case DQ_U8: return "u8";
    }
    return "?";
}

int check_current_device(const dqip_ctx* c) {
    int dev = -1;
    DQ_HIP_CHECK(hipGetDevice(&dev));
    if (dev != c->device)
        DQ_FAIL(DQ_ERR_STATE, "context was created on device %d, current device is %d", c->device, dev);
    return DQ_OK;
}

// Resolves the work buffer of a call: the caller's `buf`, or the context's
// own (allocated on first use).
int resolve_work(dqip_ctx* c, void* buf, uint8_t** out) {
    if (buf) {
        if ((uintptr_t)buf % kAlign) DQ_FAIL(DQ_ERR_ARG, "buf must be %zu-byte aligned", kAlign);
        *out = (uint8_t*)buf;
        return DQ_OK;
    }
    if (!c->work) {
        int rc = dev_alloc(c, &c->work, c->lay.total);
        if (rc) return rc;
    }
    *out = (uint8_t*)c->work;
    return DQ_OK;
}

int run_forward(dqip_ctx* c, const void* A, const void* B, void* buf, void* out, int mode,
                hipStream_t s) {
    if (!c) DQ_FAIL(DQ_ERR_STATE, "context is NULL");
    if (!A) DQ_FAIL(DQ_ERR_ARG, "A is NULL");
    if (!out) DQ_FAIL(DQ_ERR_ARG, "output is NULL");
    if (c->constB && !c->params_set)
        DQ_FAIL(DQ_ERR_STATE, "B is constant: call dqip_set_params before dqip_forward");
    if (!c->constB && !B) DQ_FAIL(DQ_ERR_ARG, "B is not constant and is NULL");
    int rc = check_current_device(c);
    if (rc) return rc;
    uint8_t* w = nullptr;
    rc = resolve_work(c, buf, &w);
    if (rc) return rc;
    if (c->prof_calls < c->prof_capacity) c->prof_ran[c->prof_calls] = 0;
    const int M = (int)c->M, N = (int)c->N, K = (int)c->K, Kp = (int)c->Kp;
    int8_t* sA = (int8_t*)(w + c->lay.sA);
    float* scaleA = (float*)(w + c->lay.scaleA);
    int32_t* zeroA = (int32_t*)(w + c->lay.zeroA);
    if (c->constB && dq_dqip_small_fits(M, N, K, A)) {
        // small product: quantization and GEMM in one launch (timed as the GEMM phase)
        DqEpilogue ep;
        ep.scaleA = scaleA;
        ep.zeroA = zeroA;
        ep.scaleB = c->scaleB;
        ep.colsumB = c->colsum;
        ep.bias = c->bias ? c->biasv : nullptr;
        ep.act = c->act;
        ep.alpha = c->alpha;
        ep.out = mode;
        ep.C = out;
        rc = dq_launch_dqip_small(A, c->typeA == DQ_BF16, M, N, K, Kp, c->iBt, ep, sA, scaleA, zeroA, s,
                                  prof_phase(c, DQ_PHASE_GEMM));
        if (rc) return rc;
        prof_call_done(c);
        return DQ_OK;
    }
    rc = dq_launch_quant_rows(A, c->typeA == DQ_BF16, M, K, Kp, sA, scaleA, zeroA, s,
                              prof_phase(c, DQ_PHASE_QUANT_A));
    if (rc) return rc;
    const int8_t* iBt = c->iBt;
    const float* scaleB = c->scaleB;
    const int32_t* colsum = c->colsum;
    if (!c->constB) {
        int8_t* qB = (int8_t*)(w + c->lay.iBt);
        float* sB = (float*)(w + c->lay.scaleB);
        int32_t* cs = (int32_t*)(w + c->lay.colsum);
        uint32_t* am = (uint32_t*)(w + c->lay.amax);
        rc = dq_launch_quant_cols(B, c->typeB, K, N, Kp, c->avoid, qB, sB, cs, am, s,
                                  prof_phase(c, DQ_PHASE_QUANT_B));
        if (rc) return rc;
        iBt = qB;
        scaleB = sB;
        colsum = cs;
    }
    DqEpilogue ep;
    ep.scaleA = scaleA;
    ep.zeroA = zeroA;
    ep.scaleB = scaleB;
    ep.colsumB = colsum;
    ep.bias = c->bias ? c->biasv : nullptr;
    ep.act = c->act;
    ep.alpha = c->alpha;
    ep.out = mode;
    ep.C = out;
    rc = dq_launch_gemm(sA, iBt, M, N, Kp, ep, s, prof_phase(c, DQ_PHASE_GEMM));
    if (rc) return rc;
    prof_call_done(c);
    return DQ_OK;
}

}  // namespace

extern "C" int dqip_init(dqip_ctx** ctx, size_t M, size_t N, size_t K, dq_dtype typeA,
                         dq_dtype typeB, dq_dtype typeC, int constB, int bias,
                         dq_act activation, int avoidOverflow) {
    if (!ctx) DQ_FAIL(DQ_ERR_ARG, "ctx is NULL");
    if (M < 1 || N < 1 || K < 1) DQ_FAIL(DQ_ERR_ARG, "M, N, K must be >= 1");
    if (M > 0x7fffffffu || N > 0x7fffffffu) DQ_FAIL(DQ_ERR_ARG, "M and N must be < 2^31");
    if (K > DQ_K_MAX) DQ_FAIL(DQ_ERR_RANGE, "K = %zu exceeds %d (exact int32 sums)", K, DQ_K_MAX);
    constB = constB ? 1 : 0;
    bias = bias ? 1 : 0;
    avoidOverflow = avoidOverflow ? 1 : 0;
    if (typeA != DQ_F32 && typeA != DQ_BF16) DQ_FAIL(DQ_ERR_TYPE, "typeA must be f32 or bf16");
    if (typeC != DQ_F32 && typeC != DQ_BF16) DQ_FAIL(DQ_ERR_TYPE, "typeC must be f32 or bf16");
    if (constB ? (typeB != DQ_F32 && typeB != DQ_I8) : (typeB != DQ_F32 && typeB != DQ_BF16))
        DQ_FAIL(DQ_ERR_TYPE, "typeB %s is not allowed for a %s B", dtype_name(typeB),
                constB ? "constant" : "non-constant");
    if (activation != DQ_ACT_IDENTITY && activation != DQ_ACT_RELU && activation != DQ_ACT_LEAKY_RELU)
        DQ_FAIL(DQ_ERR_ARG, "unknown activation %d", (int)activation);
    if (typeB == DQ_I8) avoidOverflow = 0;  // ignored for an already quantized B

    // re-init: identical parameters keep the context; any change builds a
    // new one, and the old one is released only once the new one exists, so
    // a failed re-init leaves the caller's handle valid (and unchanged)
    dqip_ctx* old = *ctx;
    if (old && old->M == M && old->N == N && old->K == K && old->typeA == typeA &&
        old->typeB == typeB && old->typeC == typeC && old->constB == constB &&
        old->bias == bias && old->act == activation && old->avoid == avoidOverflow)
        return DQ_OK;
    int dev = 0;
    DQ_HIP_CHECK(hipGetDevice(&dev));
    dqip_ctx* c = new dqip_ctx();
    c->device = dev;
    c->M = M;
    c->N = N;
    c->K = K;
    c->Kp = dq_kp(K);
    c->typeA = typeA;
    c->typeB = typeB;
    c->typeC = typeC;
    c->constB = constB;
    c->bias = bias;
    c->avoid = avoidOverflow;
    c->act = activation;
    c->alpha = 0.01f;
    c->params_set = 0;
    c->lay = make_layout(M, N, c->Kp, constB);
    int rc = DQ_OK;
    const size_t Np = dq_mnp(N);
    if (constB) {
        if (!rc) rc = dev_alloc(c, (void**)&c->iBt, Np * c->Kp);
        if (!rc) rc = dev_alloc(c, (void**)&c->scaleB, 4 * Np);
        if (!rc) rc = dev_alloc(c, (void**)&c->colsum, 4 * Np);
        if (!rc) rc = dev_alloc(c, (void**)&c->amax, 4 * N);
    }
    if (!rc && bias) {
        rc = dev_alloc(c, (void**)&c->biasv, 4 * Np);
        if (!rc) {
            hipError_t e = hipMemset(c->biasv, 0, 4 * Np);
            if (e != hipSuccess) {
                dq_set_error("hipMemset failed: %s", hipGetErrorString(e));
                rc = DQ_ERR_HIP;
            }
        }
    }
    if (rc) {
        free_ctx_memory(c);
        delete c;
        return rc;
    }
    char buf[640];
    // small products with a constant B run both steps in one launch when A
    // is 16-byte aligned (dqip_small.hip); the alignment is the caller's
    const bool small = constB && dq_gemm_config((int)M, (int)N) == 0 && K % 16 == 0 && K <= kDqipSmallKMax;
    snprintf(buf, sizeof buf,
             "gfx950 A:%s B:%s%s C:%s | %squant_rows 8-row blocks staged in LDS, whole-line fragment stores | %s%s | %s",
             dtype_name(typeA), dtype_name(typeB), constB ? "(const)" : "(dynamic)", dtype_name(typeC),
             small ? "one launch (dqip_small: rows quantized inside the 32x32 GEMM tiles) for a 16-byte-aligned A, "
                     "else " : "",
             constB ? "" : "quant_cols absmax+pack | ",
             avoidOverflow ? "B range [-64,63]" : "B range [-128,127]",
             dq_gemm_info((int)M, (int)N, (int)c->Kp));
    c->info = buf;
    if (old) dqip_release(old);
    *ctx = c;
    return DQ_OK;
}

extern "C" int dqip_enabled(const dqip_ctx* ctx) { return ctx ? 1 : 0; }

extern "C" size_t dqip_internal_buffer_size(const dqip_ctx* ctx) {
    return ctx ? ctx->owned_bytes : 0;
}

extern "C" size_t dqip_external_buffer_size(const dqip_ctx* ctx) {
    return ctx ? ctx->lay.total : 0;
}

extern "C" const char* dqip_info(const dqip_ctx* ctx) { return ctx ? ctx->info.c_str() : nullptr; }

extern "C" int dqip_set_params(dqip_ctx* c, const void* weight, const float* scale,
                               const float* bias, const float* params, void* stream) {
    if (!c) DQ_FAIL(DQ_ERR_STATE, "context is NULL");
    if (c->constB && !weight) DQ_FAIL(DQ_ERR_ARG, "weight is NULL for a constant B");
    if (c->constB && c->typeB == DQ_I8 && !scale)
        DQ_FAIL(DQ_ERR_ARG, "an int8 B needs its per-column scales");
    int rc = check_current_device(c);
    if (rc) return rc;
    hipStream_t s = (hipStream_t)stream;
    const int N = (int)c->N, K = (int)c->K, Kp = (int)c->Kp;
    if (c->constB) {
        // packs [0, Kp) of every column, zero padding included
        rc = dq_launch_quant_cols(weight, c->typeB, K, N, Kp, c->avoid, c->iBt, c->scaleB,
                                  c->colsum, c->amax, s);
        if (rc) return rc;
        if (c->typeB == DQ_I8)
            DQ_HIP_CHECK(hipMemcpyAsync(c->scaleB, scale, 4 * (size_t)N, hipMemcpyDeviceToDevice, s));
    }
    if (c->bias) {
        if (bias)
            DQ_HIP_CHECK(hipMemcpyAsync(c->biasv, bias, 4 * (size_t)N, hipMemcpyDeviceToDevice, s));
        else
            DQ_HIP_CHECK(hipMemsetAsync(c->biasv, 0, 4 * (size_t)N, s));
    }
    if (params) c->alpha = params[0];
    DQ_HIP_CHECK(hipStreamSynchronize(s));
    c->params_set = 1;
    return DQ_OK;
}

extern "C" int dqip_forward(dqip_ctx* ctx, const void* A, const void* B, void* buf, void* C,
                            void* stream) {
    if (ctx && ctx->typeC != DQ_F32 && ctx->typeC != DQ_BF16) DQ_FAIL(DQ_ERR_TYPE, "bad typeC");
    return run_forward(ctx, A, B, buf, C, ctx && ctx->typeC == DQ_BF16 ? DQ_OUT_BF16 : DQ_OUT_F32,
                       (hipStream_t)stream);
}

// ---- the forward that allocates nothing ---------------------------------
// Its work buffer (quantized A with its row scales and zero points, and for
// a non-constant B the quantized B, its scales, column sums and column
// maxima) is this file-scope device array: one copy per GPU, resident from
// the library's load on that GPU until the process ends. Host code never
// passes the array's name (a host-side stand-in, not a device address) to a
// kernel or a memory call: the device address is taken once per device with
// hipGetSymbolAddress, with that device current, and used from then on.
// Nothing in the buffer needs to start at zero: every kernel of the forward
// writes what it later reads (the column maxima are cleared by a kernel).
static __device__ __align__(256) uint8_t scratch[DQIP_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_for_current_device(void** out) {
    int dev = -1;
    DQ_HIP_CHECK(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) DQ_FAIL(DQ_ERR_STATE, "device %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            DQ_FAIL(DQ_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                    hipGetErrorString(e));
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return DQ_OK;
}
}  // namespace

extern "C" int dqip_forward_noalloc(dqip_ctx* ctx, const void* A, const void* B, void* C,
                                    void* stream) {
    if (!ctx) DQ_FAIL(DQ_ERR_STATE, "context is NULL");
    if (ctx->typeC != DQ_F32 && ctx->typeC != DQ_BF16) DQ_FAIL(DQ_ERR_TYPE, "bad typeC");
    if (ctx->lay.total > (size_t)DQIP_NOALLOC_SCRATCH_BYTES)
        DQ_FAIL(DQ_ERR_RANGE,
                "dqip_forward_noalloc: the work buffer of this context needs %zu bytes, more than the "
                "%zu-byte static scratch; use dqip_forward with a caller buffer",
                ctx->lay.total, (size_t)DQIP_NOALLOC_SCRATCH_BYTES);
    int rc = check_current_device(ctx);
    if (rc) return rc;
    void* w = nullptr;
    rc = scratch_for_current_device(&w);
    if (rc) return rc;
    return run_forward(ctx, A, B, w, C, ctx->typeC == DQ_BF16 ? DQ_OUT_BF16 : DQ_OUT_F32,
                       (hipStream_t)stream);
}

extern "C" int dqip_forward_accumulators(dqip_ctx* ctx, const void* A, const void* B, void* buf,
                                         int32_t* acc, void* stream) {
    return run_forward(ctx, A, B, buf, acc, DQ_OUT_ACC, (hipStream_t)stream);
}

extern "C" int dqip_profile_begin(dqip_ctx* c, int capacity) {
    if (!c) DQ_FAIL(DQ_ERR_STATE, "context is NULL");
    if (capacity < 1) DQ_FAIL(DQ_ERR_ARG, "capacity must be >= 1");
    free_profile_events(c);
    c->prof_events.assign((size_t)kEventsPerCall * capacity, nullptr);
    c->prof_ran.assign((size_t)capacity, 0);
    for (size_t i = 0; i < c->prof_events.size(); ++i) {
        hipError_t e = hipEventCreate(&c->prof_events[i]);
        if (e != hipSuccess) {
            c->prof_events.resize(i);
            free_profile_events(c);
            DQ_FAIL(DQ_ERR_HIP, "hipEventCreate failed: %s", hipGetErrorString(e));
        }
    }
    c->prof_capacity = capacity;
    c->prof_calls = 0;
    return DQ_OK;
}

extern "C" int dqip_profile_end(dqip_ctx* c, float* ms, int* calls) {
    if (!c) DQ_FAIL(DQ_ERR_STATE, "context is NULL");
    if (!ms || !calls) DQ_FAIL(DQ_ERR_ARG, "ms and calls must not be NULL");
    for (int p = 0; p < DQ_PHASES; ++p) ms[p] = 0.0f;
    const int n = c->prof_calls;
    for (int i = 0; i < n; ++i) {
        const hipEvent_t* ev = &c->prof_events[(size_t)kEventsPerCall * i];
        hipError_t e = hipSuccess;
        for (int p = 0; p < DQ_PHASES && e == hipSuccess; ++p) {
            if (!(c->prof_ran[i] & (1u << p))) continue;  // no kernels in this phase
            float t = 0.0f;
            e = hipEventSynchronize(ev[2 * p + 1]);
            if (e == hipSuccess) e = hipEventElapsedTime(&t, ev[2 * p], ev[2 * p + 1]);
            ms[p] += t;
        }
        if (e != hipSuccess) {
            free_profile_events(c);
            DQ_FAIL(DQ_ERR_HIP, "event timing failed: %s", hipGetErrorString(e));
        }
    }
    *calls = n;
    free_profile_events(c);
    return DQ_OK;
}

extern "C" void dqip_release(dqip_ctx* ctx) {
    if (!ctx) return;
    free_profile_events(ctx);
    free_ctx_memory(ctx);
    delete ctx;
}

extern "C" int dqip_read_quantized_a(const dqip_ctx* c, const void* buf, uint8_t* uA,
                                     float* scaleA, int32_t* zeroA, void* stream) {
    if (!c) DQ_FAIL(DQ_ERR_STATE, "context is NULL");
    const uint8_t* w = buf ? (const uint8_t*)buf : (const uint8_t*)c->work;
    if (!w) DQ_FAIL(DQ_ERR_STATE, "no forward has used the internal buffer yet");
    hipStream_t s = (hipStream_t)stream;
    const size_t M = c->M;
    if (uA) {
        int rc = dq_launch_unpack_a((const int8_t*)(w + c->lay.sA), (int)M, (int)c->K, (int)c->Kp, uA, s);
        if (rc) return rc;
    }
    if (scaleA) DQ_HIP_CHECK(hipMemcpyAsync(scaleA, w + c->lay.scaleA, 4 * M, hipMemcpyDeviceToDevice, s));
    if (zeroA) DQ_HIP_CHECK(hipMemcpyAsync(zeroA, w + c->lay.zeroA, 4 * M, hipMemcpyDeviceToDevice, s));
    return DQ_OK;
}

extern "C" int dqip_read_quantized_b(const dqip_ctx* c, const void* buf, int8_t* iB, float* scaleB,
                                     int32_t* colsumB, void* stream) {
    if (!c) DQ_FAIL(DQ_ERR_STATE, "context is NULL");
    const int8_t* qB;
    const float* sB;
    const int32_t* cs;
    if (c->constB) {
        if (!c->params_set) DQ_FAIL(DQ_ERR_STATE, "dqip_set_params has not been called");
        qB = c->iBt;
        sB = c->scaleB;
        cs = c->colsum;
    } else {
        const uint8_t* w = buf ? (const uint8_t*)buf : (const uint8_t*)c->work;
        if (!w) DQ_FAIL(DQ_ERR_STATE, "no forward has used the internal buffer yet");
        qB = (const int8_t*)(w + c->lay.iBt);
        sB = (const float*)(w + c->lay.scaleB);
        cs = (const int32_t*)(w + c->lay.colsum);
    }
    hipStream_t s = (hipStream_t)stream;
    const size_t N = c->N;
    if (iB) {
        int rc = dq_launch_unpack_b(qB, (int)c->K, (int)N, (int)c->Kp, iB, s);
        if (rc) return rc;
    }
    if (scaleB) DQ_HIP_CHECK(hipMemcpyAsync(scaleB, sB, 4 * N, hipMemcpyDeviceToDevice, s));
    if (colsumB) DQ_HIP_CHECK(hipMemcpyAsync(colsumB, cs, 4 * N, hipMemcpyDeviceToDevice, s));
    return DQ_OK;
}
