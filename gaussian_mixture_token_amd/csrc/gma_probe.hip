// Measurement support: the rate of the hardware base-2 exponential (v_exp_f32).
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

}  // namespace
}  // namespace gma

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
