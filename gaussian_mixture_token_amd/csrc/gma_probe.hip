// Measurement support: the rate of the hardware base-2 exponential (v_exp_f32), and the rate at which
// the device reads HBM.
//
// The softmax over K of both posteriors takes 2 K exponentials per token-head (page "Attention par
// Mélange Gaussien (GMA)", section "Méthodologie", sub-section "Mécanisme Central", item 1), so the
// exponential rate bounds the vector side of the passes the way HBM and the matrix cores bound the
// rest.  The estimate from unit counts is 256 compute units x 4 SIMDs x 16 lanes at a quarter of the
// full rate x 2.4 GHz, about 9.8e12 per second; this kernel measures it.  Every lane runs eight
// independent chains x <- 2^x (the values reach +inf after a few steps and stay there; the
// instruction's rate does not depend on its input), and a store that no real input triggers keeps
// the chains live.
#include <hip/hip_runtime.h>

#include "gma.h"

namespace gma {

// externally visible, so that the store below (and with it the chains) cannot be removed
__device__ float g_exp2_sink;

namespace {

constexpr int kChains = 8;
constexpr int kIters = 2048;
constexpr int kThreads = 256;

__global__ void __launch_bounds__(kThreads) exp2_rate_kernel(float seed) {
    float x[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j) x[j] = seed - (float)(threadIdx.x * kChains + j) * 1e-3f;
    for (int i = 0; i < kIters; ++i) {
#pragma unroll
        for (int j = 0; j < kChains; ++j) x[j] = __builtin_amdgcn_exp2f(x[j]);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kChains; ++j) s += x[j];
    if (s == 12345.f) g_exp2_sink = s;
}

// Read rate: every thread loads 16-byte pieces at a grid stride (one load per iteration; the
// loads of consecutive iterations overlap across the wavefronts of a compute unit) and folds them
// into a sum that a store no real input triggers keeps live.
__global__ void __launch_bounds__(kThreads) read_rate_kernel(const float4* __restrict__ p, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) {
        const float4 v = p[i];
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
    }
    const float s = acc.x + acc.y + acc.z + acc.w;
    if (s == 12345.f) g_exp2_sink = s;
}

// One untimed launch of `launch`, then `reps` timed back to back on s; elapsed milliseconds or a
// negative value if a HIP call failed.
template <class L>
float time_launches(L&& launch, int reps, hipStream_t s) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (hipEventCreate(&e0) != hipSuccess) return -1.f;
    if (hipEventCreate(&e1) != hipSuccess) {
        (void)hipEventDestroy(e0);
        return -1.f;
    }
    bool ok = true;
    launch();
    ok = ok && hipGetLastError() == hipSuccess && hipEventRecord(e0, s) == hipSuccess;
    for (int r = 0; r < reps && ok; ++r) {
        launch();
        ok = hipGetLastError() == hipSuccess;
    }
    float ms = 0.f;
    ok = ok && hipEventRecord(e1, s) == hipSuccess && hipEventSynchronize(e1) == hipSuccess &&
         hipEventElapsedTime(&ms, e0, e1) == hipSuccess && ms > 0.f;
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    return ok ? ms : -1.f;
}

}  // namespace
}  // namespace gma

extern "C" gma_status_t gma_probe_read_rate(const void* buf, size_t bytes, double* bytes_per_second, void* stream) {
    if (!bytes_per_second) return GMA_ERROR_INVALID_VALUE;
    *bytes_per_second = 0.0;
    if (!buf || bytes < 16 || reinterpret_cast<uintptr_t>(buf) % 16 != 0) return GMA_ERROR_INVALID_VALUE;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        return GMA_ERROR_LAUNCH;
    const int64_t n = (int64_t)(bytes / 16);
    const int blocks = cus * 16;
    constexpr int kReps = 10;
    const float ms = gma::time_launches(
        [&] {
            hipLaunchKernelGGL(gma::read_rate_kernel, dim3((unsigned)blocks), dim3(gma::kThreads), 0, s,
                               reinterpret_cast<const float4*>(buf), n);
        },
        kReps, s);
    if (ms <= 0.f) return GMA_ERROR_LAUNCH;
    *bytes_per_second = (double)kReps * (double)n * 16.0 / (ms * 1e-3);
    return GMA_SUCCESS;
}

extern "C" gma_status_t gma_probe_exp2_rate(double* per_second, void* stream) {
    if (!per_second) return GMA_ERROR_INVALID_VALUE;
    *per_second = 0.0;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        return GMA_ERROR_LAUNCH;
    const int blocks = cus * 16;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (hipEventCreate(&e0) != hipSuccess) return GMA_ERROR_LAUNCH;
    if (hipEventCreate(&e1) != hipSuccess) {
        (void)hipEventDestroy(e0);
        return GMA_ERROR_LAUNCH;
    }
    gma_status_t st = GMA_SUCCESS;
    // one untimed launch (clocks, code object), then the timed one
    for (int rep = 0; rep < 2 && st == GMA_SUCCESS; ++rep) {
        if (rep == 1 && hipEventRecord(e0, s) != hipSuccess) st = GMA_ERROR_LAUNCH;
        hipLaunchKernelGGL(gma::exp2_rate_kernel, dim3((unsigned)blocks), dim3(gma::kThreads), 0, s, -1.f);
        if (hipGetLastError() != hipSuccess) st = GMA_ERROR_LAUNCH;
    }
    float ms = 0.f;
    if (st == GMA_SUCCESS && (hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
                              hipEventElapsedTime(&ms, e0, e1) != hipSuccess || ms <= 0.f))
        st = GMA_ERROR_LAUNCH;
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (st == GMA_SUCCESS)
        *per_second = (double)blocks * gma::kThreads * gma::kChains * gma::kIters / (ms * 1e-3);
    return st;
}
