// Machine peaks measured on the GPU itself, as the denominators the benchmark
// reports beside the vendor figures: a streaming HBM read, a dense bf16 MFMA
// loop and a v_exp_f32 loop.  Each entry point allocates what it needs, times
// its kernel with HIP events on a stream of its own and frees everything
// before it returns.  Not part of the attention library.
#include "pic_peaks.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Read n16 16-byte words, U in flight per thread and step (NT: non-temporal
// loads); each thread folds what it read into one word so that no load can
// be dropped.
template <int U, bool NT>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4 *__restrict__ p, size_t n16,
                                                          uint32_t *__restrict__ out) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = NT ? __builtin_nontemporal_load(p + i + u * stride) : p[i + u * stride];
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u];
    }
    for (; i < n16; i += stride) acc ^= p[i];
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// Four independent accumulator chains of v_mfma_f32_16x16x32_bf16 per wave.
__global__ __launch_bounds__(256) void mfma16_loop_kernel(float *out, int iters, uint32_t seed) {
    const uint32_t t = threadIdx.x + seed;
    const u32x4 a = {t * 0x00010001u, t ^ 0x3f803f80u, 0x3f003f00u, t};
    const u32x4 b = {0x3f803f80u, t, t * 3u, 0x3e803e80u};
    const bf16x8 A = __builtin_bit_cast(bf16x8, a), B = __builtin_bit_cast(bf16x8, b);
    f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0;
    for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, c3, 0, 0, 0);
    }
    const f32x4 s = c0 + c1 + c2 + c3;
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s[0] + s[1] + s[2] + s[3];
}

// Two independent accumulator chains of v_mfma_f32_32x32x16_bf16 per wave.
__global__ __launch_bounds__(256) void mfma32_loop_kernel(float *out, int iters, uint32_t seed) {
    const uint32_t t = threadIdx.x + seed;
    const u32x4 a = {t * 0x00010001u, t ^ 0x3f803f80u, 0x3f003f00u, t};
    const u32x4 b = {0x3f803f80u, t, t * 3u, 0x3e803e80u};
    const bf16x8 A = __builtin_bit_cast(bf16x8, a), B = __builtin_bit_cast(bf16x8, b);
    f32x16 c0 = {}, c1 = {};
    for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, c1, 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) s += c0[e] + c1[e];
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Eight independent chains x <- 2^(-x) per thread (the negation is a source
// modifier of v_exp_f32, so the loop issues exp instructions only); the map
// keeps x in [0.5, 1].
__global__ __launch_bounds__(256) void exp2_loop_kernel(float *out, int iters) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = 0.5f + 0.01f * (float)((threadIdx.x + e) & 31);
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = __builtin_amdgcn_exp2f(-x[e]);
    }
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) s += x[e];
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

constexpr int kGrid = 256 * 8;   // 8 workgroups of 4 waves per CU: 8 waves per SIMD

struct Timer {
    hipStream_t s = nullptr;
    hipEvent_t a = nullptr, b = nullptr;
    hipError_t init() {
        hipError_t e = hipStreamCreate(&s);
        if (e == hipSuccess) e = hipEventCreate(&a);
        if (e == hipSuccess) e = hipEventCreate(&b);
        return e;
    }
    ~Timer() {
        if (a) (void)hipEventDestroy(a);
        if (b) (void)hipEventDestroy(b);
        if (s) (void)hipStreamDestroy(s);
    }
};

int status(hipError_t e) { return e == hipSuccess ? 0 : (int)e; }

}  // namespace

extern "C" {

int pic_peak_hbm_read(size_t bytes, int reps, double *gbytes_per_s) {
    if (!gbytes_per_s || reps <= 0 || bytes < (1u << 20)) return -1;
    *gbytes_per_s = 0.0;
    Timer t;
    hipError_t e = t.init();
    void *buf = nullptr;
    uint32_t *out = nullptr;
    const size_t n16 = bytes / 16;
    constexpr int kMaxGrid = 256 * 16;
    if (e == hipSuccess) e = hipMalloc(&buf, n16 * 16);
    if (e == hipSuccess) e = hipMalloc(&out, (size_t)kMaxGrid * 256 * sizeof(uint32_t));
    if (e == hipSuccess) e = hipMemsetAsync(buf, 0x5a, n16 * 16, t.s);
    // the best of a few shapes: loads in flight per thread, non-temporal or
    // not, 8 or 16 workgroups per CU
    for (int variant = 0; e == hipSuccess && variant < 6; ++variant) {
        const int grid = variant & 1 ? 256 * 16 : 256 * 8;
        auto launch = [&]() {
            const u32x4 *src = (const u32x4 *)buf;
            switch (variant >> 1) {
            case 0: hipLaunchKernelGGL((stream_read_kernel<4, false>), dim3(grid), dim3(256), 0, t.s, src, n16, out); break;
            case 1: hipLaunchKernelGGL((stream_read_kernel<8, false>), dim3(grid), dim3(256), 0, t.s, src, n16, out); break;
            default: hipLaunchKernelGGL((stream_read_kernel<8, true>), dim3(grid), dim3(256), 0, t.s, src, n16, out); break;
            }
        };
        launch();   // untimed
        e = hipEventRecord(t.a, t.s);
        for (int r = 0; e == hipSuccess && r < reps; ++r) {
            launch();
            e = hipGetLastError();
        }
        if (e == hipSuccess) e = hipEventRecord(t.b, t.s);
        if (e == hipSuccess) e = hipEventSynchronize(t.b);
        float ms = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, t.a, t.b);
        if (e == hipSuccess && ms > 0.f) {
            const double gbs = (double)n16 * 16.0 * reps / (ms * 1e-3) / 1e9;
            if (gbs > *gbytes_per_s) *gbytes_per_s = gbs;
        }
    }
    if (buf) (void)hipFree(buf);
    if (out) (void)hipFree(out);
    return status(e);
}

int pic_peak_mfma_bf16(int shape, int iters, double *tflops) {
    if (!tflops || iters <= 0 || (shape != 16 && shape != 32)) return -1;
    *tflops = 0.0;
    Timer t;
    hipError_t e = t.init();
    float *out = nullptr;
    if (e == hipSuccess) e = hipMalloc(&out, (size_t)kGrid * 256 * sizeof(float));
    // flops of one wave: chains x iters x (2 m n k)
    const double per_wave = shape == 16 ? 4.0 * iters * 2.0 * 16 * 16 * 32 : 2.0 * iters * 2.0 * 32 * 32 * 16;
    for (int pass = 0; e == hipSuccess && pass < 2; ++pass) {   // pass 0 warms up
        if (pass == 1) e = hipEventRecord(t.a, t.s);
        if (shape == 16)
            hipLaunchKernelGGL(mfma16_loop_kernel, dim3(kGrid), dim3(256), 0, t.s, out, iters, (uint32_t)pass);
        else
            hipLaunchKernelGGL(mfma32_loop_kernel, dim3(kGrid), dim3(256), 0, t.s, out, iters, (uint32_t)pass);
        if (e == hipSuccess) e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipEventRecord(t.b, t.s);
    if (e == hipSuccess) e = hipEventSynchronize(t.b);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, t.a, t.b);
    if (e == hipSuccess && ms > 0.f) *tflops = per_wave * kGrid * 4 / (ms * 1e-3) / 1e12;
    if (out) (void)hipFree(out);
    return status(e);
}

int pic_peak_exp2(int iters, double *gexp_per_s) {
    if (!gexp_per_s || iters <= 0) return -1;
    *gexp_per_s = 0.0;
    Timer t;
    hipError_t e = t.init();
    float *out = nullptr;
    if (e == hipSuccess) e = hipMalloc(&out, (size_t)kGrid * 256 * sizeof(float));
    for (int pass = 0; e == hipSuccess && pass < 2; ++pass) {
        if (pass == 1) e = hipEventRecord(t.a, t.s);
        hipLaunchKernelGGL(exp2_loop_kernel, dim3(kGrid), dim3(256), 0, t.s, out, iters);
        if (e == hipSuccess) e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipEventRecord(t.b, t.s);
    if (e == hipSuccess) e = hipEventSynchronize(t.b);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, t.a, t.b);
    if (e == hipSuccess && ms > 0.f) *gexp_per_s = 8.0 * iters * kGrid * 256.0 / (ms * 1e-3) / 1e9;
    if (out) (void)hipFree(out);
    return status(e);
}

}  // extern "C"
