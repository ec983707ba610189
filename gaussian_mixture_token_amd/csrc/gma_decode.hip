// One-token causal decode step, one workgroup per (batch, head).
//
// Method: page "Attention par Mélange Gaussien (GMA)", section "Méthodologie", sub-section
// "Mécanisme Central": item 1 (posterior responsibilities of the new query and key under the
// head's diagonal GMM, softplus variances, softmax priors), item 2 (write Vt += gamma_K (x) v,
// Z += gamma_K; read O = gamma_Q Vt / (gamma_Q . Z + eps)) and item 3 (causal: the read includes the
// new token, and everything earlier enters through the carried [Vt | Z]).
//
// A step touches K (d_r + d_v + 1) numbers per head: plain vector code, no matrix cores, 16 waves per
// (batch, head).  Per-dimension terms (softplus, log, reciprocal) in fp32; the log-density sums
// over d_r and the prior log-sum-exp in fp64; the state in fp32.  With a prepared mixture
// (decode_prepare_kernel, once per parameter update) the step reads 1 / sigma^2 and the
// per-component constants instead of deriving them from the raw parameters every token.
#include "gma_decode.hpp"
#include "gma_device.hpp"

namespace gma {

namespace {

constexpr int kMax = 256;   // d_r, K, d_v <= 256
constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

template <bool F32>
__device__ __forceinline__ float load_elem(const void* base, int64_t i) {
    if constexpr (F32) return reinterpret_cast<const float*>(base)[i];
    else return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(base)[i] << 16);
}

template <bool F32>
__device__ __forceinline__ void store_elem(void* base, int64_t i, float x) {
    if constexpr (F32) reinterpret_cast<float*>(base)[i] = x;
    else reinterpret_cast<uint16_t*>(base)[i] = bf16_bits(x);
}

__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}
__device__ __forceinline__ double wave_max(double x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmax(x, __shfl_xor(x, o, 64));
    return x;
}

}  // namespace

// Per-component quantities of the decode step that depend on the mixture only, by one workgroup per
// head: 1 / sigma^2 (softplus in fp32, as in the step) and c_k = log pi_k - 1/2 sum_d log sigma^2_kd
// (the fp32 logs summed in fp64 by lanes over dims and fixed-order butterflies, the prior
// log-sum-exp in fp64).  With them a step's log-density is c_k - 1/2 sum_d (x_d - mu_kd)^2 / sigma^2_kd.
__global__ void __launch_bounds__(kThreads) decode_prepare_kernel(const DecodePrepArgs a) {
    const int h = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int K = a.K, dr = a.d_r;
    __shared__ double s_lse;
    if (w == 0) {
        double m = -INFINITY;
        for (int k = lane; k < K; k += 64) m = fmax(m, (double)a.prior[(int64_t)h * K + k]);
        m = wave_max(m);
        double e = 0.0;
        for (int k = lane; k < K; k += 64) e += exp((double)a.prior[(int64_t)h * K + k] - m);
        e = wave_sum(e);
        if (lane == 0) s_lse = m + log(e);
    }
    __syncthreads();
    const double lse = s_lse;
    for (int k = w; k < K; k += kWaves) {
        double sl = 0.0;
        for (int d = lane; d < dr; d += 64) {
            const int64_t i = ((int64_t)h * K + k) * dr + d;
            const float r = a.raw_var[i];
            const float var = fmaxf(r, 0.f) + log1pf(expf(-fabsf(r)));   // softplus
            a.inv_var[i] = 1.f / var;
            sl += (double)logf(var);
        }
        sl = wave_sum(sl);
        if (lane == 0) a.cconst[(int64_t)h * K + k] = ((double)a.prior[(int64_t)h * K + k] - lse) - 0.5 * sl;
    }
}

// PREP: the mixture comes as mu plus the prepared 1 / sigma^2 and c_k (decode_prepare_kernel).
template <bool F32, bool PREP>
__global__ void __launch_bounds__(kThreads) decode_kernel(const DecodeArgs a) {
    const int64_t bh = blockIdx.x;
    const int h = (int)(bh % a.H);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int K = a.K, dr = a.d_r, dv = a.d_v;
    __shared__ float s_xq[kMax], s_xk[kMax], s_v[kMax];
    __shared__ double s_lq[kMax], s_lk[kMax];
    __shared__ float s_gq[kMax], s_gk[kMax];
    __shared__ double s_red[2 * kWaves];
    __shared__ float s_redf[2 * kWaves];
    __shared__ float s_num[kThreads];

    for (int d = tid; d < dr; d += kThreads) {
        s_xq[d] = load_elem<F32>(a.qx, bh * dr + d);
        s_xk[d] = load_elem<F32>(a.kx, bh * dr + d);
    }
    for (int j = tid; j < dv; j += kThreads) s_v[j] = load_elem<F32>(a.v, bh * dv + j);

    // log pi = prior - log-sum-exp(prior), by wave 0 (fixed-order butterflies)
    if (!PREP && w == 0) {
        double m = -INFINITY;
        for (int k = lane; k < K; k += 64) m = fmax(m, (double)a.prior[(int64_t)h * K + k]);
        m = wave_max(m);
        double e = 0.0;
        for (int k = lane; k < K; k += 64) e += exp((double)a.prior[(int64_t)h * K + k] - m);
        e = wave_sum(e);
        if (lane == 0) s_red[0] = m + log(e);
    }
    __syncthreads();
    const double lse = PREP ? 0.0 : s_red[0];

    // log-densities of the query and the key: l_k(x) = log pi_k - 1/2 sum_d [log var + (x - mu)^2 / var]
    // (the d_r/2 log 2 pi term is common to all components and cancels).  Wave w takes components
    // w, w + kWaves, ... in groups of G (their loads in flight together), lanes take dimensions.
    constexpr int G = 4;
    for (int k0 = w; k0 < K; k0 += kWaves * G) {
        double sq[G], sk[G];
#pragma unroll
        for (int u = 0; u < G; ++u) {
            sq[u] = 0.0;
            sk[u] = 0.0;
        }
        for (int d = lane; d < dr; d += 64) {
            const double xq = s_xq[d], xk = s_xk[d];
            float r[G], m[G];
#pragma unroll
            for (int u = 0; u < G; ++u) {
                const int k = k0 + kWaves * u;
                const int64_t i = ((int64_t)h * K + (k < K ? k : 0)) * dr + d;
                r[u] = PREP ? a.inv_var[i] : a.raw_var[i];
                m[u] = a.mu[i];
            }
#pragma unroll
            for (int u = 0; u < G; ++u) {
                const float dq = (float)xq - m[u], dk = (float)xk - m[u];
                if constexpr (PREP) {
                    sq[u] += (double)(dq * dq * r[u]);
                    sk[u] += (double)(dk * dk * r[u]);
                } else {
                    const float var = fmaxf(r[u], 0.f) + log1pf(expf(-fabsf(r[u])));   // softplus
                    const float inv = 1.f / var;
                    const float lv = logf(var);
                    sq[u] += (double)(lv + dq * dq * inv);
                    sk[u] += (double)(lv + dk * dk * inv);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < G; ++u) {
            const int k = k0 + kWaves * u;
            const double tq = wave_sum(sq[u]), tk = wave_sum(sk[u]);
            if (lane == 0 && k < K) {
                const double lp = PREP ? a.cconst[(int64_t)h * K + k] : (double)a.prior[(int64_t)h * K + k] - lse;
                s_lq[k] = lp - 0.5 * tq;
                s_lk[k] = lp - 0.5 * tk;
            }
        }
    }
    __syncthreads();

    // softmax over the components (thread k), block reductions in a fixed order
    double mq = -INFINITY, mk = -INFINITY;
    for (int k = tid; k < K; k += kThreads) {
        mq = fmax(mq, s_lq[k]);
        mk = fmax(mk, s_lk[k]);
    }
    mq = wave_max(mq);
    mk = wave_max(mk);
    if (lane == 0) {
        s_red[w] = mq;
        s_red[kWaves + w] = mk;
    }
    __syncthreads();
    mq = s_red[0];
    mk = s_red[kWaves];
    for (int q = 1; q < kWaves; ++q) {
        mq = fmax(mq, s_red[q]);
        mk = fmax(mk, s_red[kWaves + q]);
    }
    __syncthreads();
    float eq = 0.f, ek = 0.f;
    for (int k = tid; k < K; k += kThreads) {
        const float xq = expf((float)(s_lq[k] - mq)), xk = expf((float)(s_lk[k] - mk));
        s_gq[k] = xq;
        s_gk[k] = xk;
        eq += xq;
        ek += xk;
    }
    eq = wave_sum(eq);
    ek = wave_sum(ek);
    if (lane == 0) {
        s_redf[w] = eq;
        s_redf[kWaves + w] = ek;
    }
    __syncthreads();
    float tq = 0.f, tk = 0.f;
    for (int q = 0; q < kWaves; ++q) {
        tq += s_redf[q];
        tk += s_redf[kWaves + q];
    }
    const float rq = 1.f / tq, rk = 1.f / tk;
    __syncthreads();
    for (int k = tid; k < K; k += kThreads) {
        s_gq[k] *= rq;
        s_gk[k] *= rk;
    }
    __syncthreads();

    // memory update and read (the read sees the new token).  Z[k] by thread k; column j of Vt by the
    // NP thread groups of NCOL threads, group g taking components g, g + NP, ...; every element is
    // read and written by one thread, so in-place is safe.  Partial numerators meet in LDS.
    const int64_t sb = bh * K * (dv + 1);
    float den = 0.f;
    for (int k = tid; k < K; k += kThreads) {
        const float z = (a.state_in ? a.state_in[sb + (int64_t)k * (dv + 1) + dv] : 0.f) + s_gk[k];
        if (a.state_out) a.state_out[sb + (int64_t)k * (dv + 1) + dv] = z;
        den += s_gq[k] * z;
    }
    den = wave_sum(den);
    if (lane == 0) s_redf[w] = den;
    const int ncol = (dv <= 64) ? 64 : (dv <= 128 ? 128 : 256);   // threads per column group
    const int np = kThreads / ncol;                                // column groups
    const int g = tid / ncol, j = tid % ncol;
    float num = 0.f;
    if (j < dv) {
        const float vj = s_v[j];
#pragma unroll 8
        for (int k = g; k < K; k += np) {
            const int64_t e = sb + (int64_t)k * (dv + 1) + j;
            const float sv = (a.state_in ? a.state_in[e] : 0.f) + s_gk[k] * vj;
            if (a.state_out) a.state_out[e] = sv;
            num += s_gq[k] * sv;
        }
    }
    s_num[tid] = num;
    __syncthreads();
    den = a.eps;
    {
        float t = 0.f;
        for (int q = 0; q < kWaves; ++q) t += s_redf[q];
        den += t;
    }
    if (tid < dv) {
        float n = 0.f;
        for (int q = 0; q < np; ++q) n += s_num[q * ncol + tid];
        store_elem<F32>(a.o, bh * dv + tid, n / den);
    }
}

void launch_decode(const DecodeArgs& a, int64_t bh, bool f32, hipStream_t s) {
    const dim3 g((unsigned)bh), b(kThreads);
    if (a.inv_var) {
        if (f32) hipLaunchKernelGGL((decode_kernel<true, true>), g, b, 0, s, a);
        else hipLaunchKernelGGL((decode_kernel<false, true>), g, b, 0, s, a);
    } else {
        if (f32) hipLaunchKernelGGL((decode_kernel<true, false>), g, b, 0, s, a);
        else hipLaunchKernelGGL((decode_kernel<false, false>), g, b, 0, s, a);
    }
}

void launch_decode_prepare(const DecodePrepArgs& a, int heads, hipStream_t s) {
    hipLaunchKernelGGL(decode_prepare_kernel, dim3((unsigned)heads), dim3(kThreads), 0, s, a);
}

}  // namespace gma
