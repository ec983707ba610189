// One-token causal decode step, one workgroup per (batch, head).
//
// Method: page "Attention par Mélange Gaussien (GMA)", section "Méthodologie", sub-section
// "Mécanisme Central": item 1 (posterior responsibilities of the new query and key under the
// head's diagonal GMM, softplus variances, softmax priors), item 2 (write Vt += gamma_K (x) v,
// Z += gamma_K; read O = gamma_Q Vt / (gamma_Q . Z + eps)) and item 3 (causal: the read includes the
// new token, and everything earlier enters through the carried [Vt | Z]).
//
// A step touches K (d_r + d_v + 1) numbers per head, so it is bound by launch latency and the state
// traffic, not by arithmetic: plain vector code, no matrix cores.  Softplus, log and exp in fp32;
// the log-density sums over d_r and the prior log-sum-exp in fp64; the state in fp32.
#include "gma_decode.hpp"
#include "gma_device.hpp"

namespace gma {

namespace {

constexpr int kMax = 256;   // d_r, K, d_v <= 256

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

template <bool F32>
__global__ void __launch_bounds__(256) decode_kernel(const DecodeArgs a) {
    const int64_t bh = blockIdx.x;
    const int h = (int)(bh % a.H);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int K = a.K, dr = a.d_r, dv = a.d_v;
    __shared__ float s_xq[kMax], s_xk[kMax], s_v[kMax];
    __shared__ double s_lq[kMax], s_lk[kMax];
    __shared__ float s_gq[kMax], s_gk[kMax];
    __shared__ double s_red[8];
    __shared__ float s_redf[8];

    for (int d = tid; d < dr; d += 256) {
        s_xq[d] = load_elem<F32>(a.qx, bh * dr + d);
        s_xk[d] = load_elem<F32>(a.kx, bh * dr + d);
    }
    for (int j = tid; j < dv; j += 256) s_v[j] = load_elem<F32>(a.v, bh * dv + j);

    // log pi = prior - log-sum-exp(prior), by wave 0 (fixed-order butterflies)
    if (w == 0) {
        double m = -INFINITY;
        for (int k = lane; k < K; k += 64) m = fmax(m, (double)a.prior[(int64_t)h * K + k]);
        m = wave_max(m);
        double e = 0.0;
        for (int k = lane; k < K; k += 64) e += exp((double)a.prior[(int64_t)h * K + k] - m);
        e = wave_sum(e);
        if (lane == 0) s_red[0] = m + log(e);
    }
    __syncthreads();
    const double lse = s_red[0];

    // log-densities of the query and the key: l_k(x) = log pi_k - 1/2 sum_d [log var + (x - mu)^2 / var]
    // (the d_r/2 log 2 pi term is common to all components and cancels); components round-robin over
    // the waves, dimensions over the lanes
    for (int k = w; k < K; k += 4) {
        double sq = 0.0, sk = 0.0;
        for (int d = lane; d < dr; d += 64) {
            const int64_t i = ((int64_t)h * K + k) * dr + d;
            const float r = a.raw_var[i];
            const float var = fmaxf(r, 0.f) + log1pf(expf(-fabsf(r)));   // softplus
            const double inv = 1.0 / (double)var;
            const double lv = (double)logf(var);
            const double mu = a.mu[i];
            const double dq = (double)s_xq[d] - mu, dk = (double)s_xk[d] - mu;
            sq += lv + dq * dq * inv;
            sk += lv + dk * dk * inv;
        }
        sq = wave_sum(sq);
        sk = wave_sum(sk);
        if (lane == 0) {
            const double lp = (double)a.prior[(int64_t)h * K + k] - lse;
            s_lq[k] = lp - 0.5 * sq;
            s_lk[k] = lp - 0.5 * sk;
        }
    }
    __syncthreads();

    // softmax over the components (thread k), block reductions in a fixed order
    double mq = -INFINITY, mk = -INFINITY;
    for (int k = tid; k < K; k += 256) {
        mq = fmax(mq, s_lq[k]);
        mk = fmax(mk, s_lk[k]);
    }
    mq = wave_max(mq);
    mk = wave_max(mk);
    if (lane == 0) {
        s_red[w] = mq;
        s_red[4 + w] = mk;
    }
    __syncthreads();
    mq = fmax(fmax(s_red[0], s_red[1]), fmax(s_red[2], s_red[3]));
    mk = fmax(fmax(s_red[4], s_red[5]), fmax(s_red[6], s_red[7]));
    __syncthreads();
    float eq = 0.f, ek = 0.f;
    for (int k = tid; k < K; k += 256) {
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
        s_redf[4 + w] = ek;
    }
    __syncthreads();
    const float rq = 1.f / ((s_redf[0] + s_redf[1]) + (s_redf[2] + s_redf[3]));
    const float rk = 1.f / ((s_redf[4] + s_redf[5]) + (s_redf[6] + s_redf[7]));
    __syncthreads();
    for (int k = tid; k < K; k += 256) {
        s_gq[k] *= rq;
        s_gk[k] *= rk;
    }
    __syncthreads();

    // memory update and read (the read sees the new token): column j of Vt by thread j, Z[k] by
    // thread k; every element is read and written by the same thread, so in-place is safe
    const int64_t sb = bh * K * (dv + 1);
    float den = 0.f;
    for (int k = tid; k < K; k += 256) {
        const float z = (a.state_in ? a.state_in[sb + (int64_t)k * (dv + 1) + dv] : 0.f) + s_gk[k];
        if (a.state_out) a.state_out[sb + (int64_t)k * (dv + 1) + dv] = z;
        den += s_gq[k] * z;
    }
    den = wave_sum(den);
    if (lane == 0) s_redf[w] = den;
    __syncthreads();
    den = ((s_redf[0] + s_redf[1]) + (s_redf[2] + s_redf[3])) + a.eps;
    for (int j = tid; j < dv; j += 256) {
        const float vj = s_v[j];
        float num = 0.f;
        for (int k = 0; k < K; ++k) {
            const int64_t e = sb + (int64_t)k * (dv + 1) + j;
            const float sv = (a.state_in ? a.state_in[e] : 0.f) + s_gk[k] * vj;
            if (a.state_out) a.state_out[e] = sv;
            num += s_gq[k] * sv;
        }
        store_elem<F32>(a.o, bh * dv + j, num / den);
    }
}

void launch_decode(const DecodeArgs& a, int64_t bh, bool f32, hipStream_t s) {
    if (f32) hipLaunchKernelGGL((decode_kernel<true>), dim3((unsigned)bh), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((decode_kernel<false>), dim3((unsigned)bh), dim3(256), 0, s, a);
}

}  // namespace gma
