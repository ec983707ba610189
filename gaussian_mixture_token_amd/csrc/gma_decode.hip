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

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }

// An empty use of a register: a value loaded before it is complete here (the compiler waits for the
// load at this point), so the load is issued before it and cannot be moved past a later barrier.
__device__ __forceinline__ void complete_here(float& x) { asm volatile("" : "+v"(x)); }

// Sums each of the V values of every lane over the wave's 64 lanes (V a power of two <= 64) by
// recursive halving: at the exchange with lane ^ O (O = 32, 16, ...) a lane keeps the half of its
// values that its bit O selects and adds the partner's copy of that half, so the V sums take V - 1
// exchanges before the last log2(64 / V) butterfly steps, instead of 6 V.  On return lane L holds the
// total of value (L >> (6 - log2 V)) % V (as do the 64 / V lanes that share those bits).  The order of
// the additions is fixed, so results are reproducible.  One template level per exchange, so that every
// index is a constant and the values stay in registers.
template <int V, int O>
__device__ __forceinline__ double sum_scatter_step(const double (&v)[V], int lane) {
    if constexpr (V == 1) {
        double x = v[0];
#pragma unroll
        for (int o = O; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
        return x;
    } else {
        constexpr int half = V / 2;
        const bool up = (lane & O) != 0;
        double kept[half];
#pragma unroll
        for (int i = 0; i < half; ++i) {
            const double send = up ? v[i] : v[i + half];
            const double keep = up ? v[i + half] : v[i];
            kept[i] = keep + __shfl_xor(send, O, 64);
        }
        return sum_scatter_step<half, O / 2>(kept, lane);
    }
}

template <int V>
__device__ __forceinline__ double wave_sum_scatter(const double (&v)[V], int lane) {
    static_assert(V >= 1 && V <= 64 && (V & (V - 1)) == 0, "V: a power of two <= 64");
    return sum_scatter_step<V, 32>(v, lane);
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
// DPL: dimensions of d_r per lane (1, 2 or 4: d_r <= 64, 128, 256).
//
// A step is a chain of dependent phases on one workgroup per (batch, head), and every launch meets
// cold caches, so one memory round trip costs microseconds.  The kernel therefore issues all of its
// loads at the start (the token's rows, the per-component constants, the mixture parameters of the
// wave's components, the state elements of the thread) and waits once where they fit the registers:
// mixture parameters for K <= 256 / DPL with the prepared mixture and d_r <= 128, else K <= 128 / DPL;
// state elements for K <= 128 with d_v <= 128, or K <= 256 with d_v <= 64.  Larger shapes take a
// round trip per further group of loads.
template <bool F32, bool PREP, int DPL>
__global__ void __launch_bounds__(kThreads) decode_kernel(const DecodeArgs a) {
    const int64_t bh = blockIdx.x;
    const int h = (int)(bh % a.H);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int K = a.K, dr = a.d_r, dv = a.d_v;
    __shared__ float s_xq[kMax], s_xk[kMax], s_v[kMax];
    __shared__ double s_lq[kMax], s_lk[kMax];
    __shared__ double s_cc[kMax];   // c_k (prepared) or the prior logit (raw)
    __shared__ float s_gq[kMax], s_gk[kMax];
    __shared__ double s_red[1];
    __shared__ float s_redf[kWaves];
    __shared__ float s_num[kThreads];

    // Wave w takes components w, w + kWaves, ... in groups of G (every component of the wave when
    // K <= kWaves G), lanes take dimensions lane, lane + 64, ...: G x DPL x 2 parameters per lane.
    constexpr int G = ((PREP && DPL < 4) ? 16 : 8) / DPL;
    float gr[G][DPL], gm[G][DPL];   // raw or prepared variance terms, means
    auto load_group = [&](int k0) {
#pragma unroll
        for (int u = 0; u < G; ++u)
#pragma unroll
            for (int t = 0; t < DPL; ++t) {
                const int k = k0 + kWaves * u, d = lane + 64 * t;
                const int64_t i = ((int64_t)h * K + (k < K ? k : 0)) * dr + (d < dr ? d : 0);
                gr[u][t] = PREP ? a.inv_var[i] : a.raw_var[i];
                gm[u][t] = a.mu[i];
            }
    };
    load_group(w);

    // The state elements this thread updates: Z[k] by thread k; column j of Vt by the NP thread groups
    // of NCOL threads, group g taking components g, g + NP, ...  They are loaded in batches of NB, a
    // batch before any of its elements is stored (each element is read and written by this one thread,
    // so the in-place update stays correct); the first batch here.
    const int64_t sb = bh * K * (dv + 1);
    const int ncol = (dv <= 64) ? 64 : (dv <= 128 ? 128 : 256);   // threads per column group
    const int np = kThreads / ncol;                                // column groups
    const int g = tid / ncol, j = tid % ncol;
    constexpr int NB = 16;
    float sv[NB];
    auto load_batch = [&](int e0) {
#pragma unroll
        for (int e = 0; e < NB; ++e) {
            const int k = g + (e0 + e) * np;
            sv[e] = (a.state_in && j < dv && k < K) ? a.state_in[sb + (int64_t)k * (dv + 1) + j] : 0.f;
        }
    };
    load_batch(0);
    const float zin = (a.state_in && tid < K) ? a.state_in[sb + (int64_t)tid * (dv + 1) + dv] : 0.f;

    for (int d = tid; d < dr; d += kThreads) {
        s_xq[d] = load_elem<F32>(a.qx, bh * dr + d);
        s_xk[d] = load_elem<F32>(a.kx, bh * dr + d);
    }
    for (int jj = tid; jj < dv; jj += kThreads) s_v[jj] = load_elem<F32>(a.v, bh * dv + jj);
    if (tid < K) s_cc[tid] = PREP ? a.cconst[(int64_t)h * K + tid] : (double)a.prior[(int64_t)h * K + tid];
    // every load above completes before the first barrier, where the token's rows are waited for anyway
#pragma unroll
    for (int u = 0; u < G; ++u)
#pragma unroll
        for (int t = 0; t < DPL; ++t) {
            complete_here(gr[u][t]);
            complete_here(gm[u][t]);
        }

    // log pi = prior - log-sum-exp(prior), by wave 0 from its own loads (fixed-order butterflies)
    if (!PREP && w == 0) {
        constexpr int KL = kMax / 64;
        double pr[KL];
        double pm = -INFINITY;
#pragma unroll
        for (int i = 0; i < KL; ++i) {
            const int k = lane + 64 * i;
            pr[i] = (k < K) ? (double)a.prior[(int64_t)h * K + k] : -INFINITY;
            pm = fmax(pm, pr[i]);
        }
        pm = wave_max(pm);
        double e = 0.0;
#pragma unroll
        for (int i = 0; i < KL; ++i)
            if (lane + 64 * i < K) e += exp(pr[i] - pm);
        e = wave_sum(e);
        if (lane == 0) s_red[0] = pm + log(e);
    }
    __syncthreads();
    const double lse = PREP ? 0.0 : s_red[0];

    // log-densities of the query and the key: l_k(x) = log pi_k - 1/2 sum_d [log var + (x - mu)^2 / var]
    // (the d_r/2 log 2 pi term is common to all components and cancels).  Each lane sums its
    // dimensions in increasing order; the lanes' sums of SG components at a time are then reduced
    // together across the wave.
    auto logits_group = [&](int k0) {
        constexpr int SG = (G < 4) ? G : 4;
#pragma unroll
        for (int u0 = 0; u0 < G; u0 += SG) {
            if (k0 + kWaves * u0 < K) {   // uniform in the wave
                // value 2u: the query's sum of component k0 + kWaves (u0 + u), value 2u + 1: the key's
                double vals[2 * SG];
#pragma unroll
                for (int u = 0; u < 2 * SG; ++u) vals[u] = 0.0;
#pragma unroll
                for (int t = 0; t < DPL; ++t) {
                    const int d = lane + 64 * t;
                    if (d < dr) {
                        const float xq = s_xq[d], xk = s_xk[d];
#pragma unroll
                        for (int u = 0; u < SG; ++u) {
                            const float r = gr[u0 + u][t], m = gm[u0 + u][t];
                            const float dq = xq - m, dk = xk - m;
                            if constexpr (PREP) {
                                vals[2 * u] += (double)(dq * dq * r);
                                vals[2 * u + 1] += (double)(dk * dk * r);
                            } else {
                                const float var = fmaxf(r, 0.f) + log1pf(expf(-fabsf(r)));   // softplus
                                const float inv = 1.f / var;
                                const float lv = logf(var);
                                vals[2 * u] += (double)(lv + dq * dq * inv);
                                vals[2 * u + 1] += (double)(lv + dk * dk * inv);
                            }
                        }
                    }
                }
                constexpr int LV = ilog2(2 * SG);
                const double tt = wave_sum_scatter<2 * SG>(vals, lane);
                const int idx = (lane >> (6 - LV)) & (2 * SG - 1);
                const int k = k0 + kWaves * (u0 + (idx >> 1));
                if ((lane & ((64 >> LV) - 1)) == 0 && k < K) {
                    const double lp = PREP ? s_cc[k] : s_cc[k] - lse;
                    ((idx & 1) ? s_lk : s_lq)[k] = lp - 0.5 * tt;
                }
            }
        }
    };
    // The first group straight-line; a further group (K > kWaves G) loads and uses its parameters in
    // one iteration, so that no load is outstanding past the loop (the compiler's waits after a loop
    // whose back edge issues loads cover stores too: the state update would then store serially).
    logits_group(w);
    for (int k0 = w + kWaves * G; k0 < K; k0 += kWaves * G) {
        load_group(k0);
        logits_group(k0);
    }
    __syncthreads();

    // softmax over the components: wave 0 the query's, wave 1 the key's, lane l taking components
    // l, l + 64, ... (K <= 256), wave reductions in a fixed order
    if (w < 2) {
        const double* l = (w == 0) ? s_lq : s_lk;
        float* gout = (w == 0) ? s_gq : s_gk;
        constexpr int KL = kMax / 64;
        double mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < KL; ++i) {
            const int k = lane + 64 * i;
            if (k < K) mx = fmax(mx, l[k]);
        }
        mx = wave_max(mx);
        float e[KL];
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < KL; ++i) {
            const int k = lane + 64 * i;
            e[i] = (k < K) ? expf((float)(l[k] - mx)) : 0.f;
            sum += e[i];
        }
        sum = wave_sum(sum);
        const float rs = 1.f / sum;
#pragma unroll
        for (int i = 0; i < KL; ++i) {
            const int k = lane + 64 * i;
            if (k < K) gout[k] = e[i] * rs;
        }
    }
    __syncthreads();

    // memory update and read (the read sees the new token); partial numerators meet in LDS.  A batch's
    // new values are all formed before any of them is stored: the stores are conditional, and after a
    // conditional store the compiler waits for every outstanding memory operation before a register
    // loaded from memory is used, which would make each store wait for the previous one.
    float zn = 0.f, den = 0.f;
    if (tid < K) {
        zn = zin + s_gk[tid];
        den = s_gq[tid] * zn;
    }
    den = wave_sum(den);
    if (lane == 0) s_redf[w] = den;
    float num = 0.f;
    const float vj = (j < dv) ? s_v[j] : 0.f;
    auto update_batch = [&](int e0) {
#pragma unroll
        for (int e = 0; e < NB; ++e) {
            const int k = g + (e0 + e) * np;
            if (j < dv && k < K) {
                sv[e] += s_gk[k] * vj;
                num += s_gq[k] * sv[e];
            }
        }
    };
    auto store_batch = [&](int e0) {
#pragma unroll
        for (int e = 0; e < NB; ++e) {
            const int k = g + (e0 + e) * np;
            if (j < dv && k < K) a.state_out[sb + (int64_t)k * (dv + 1) + j] = sv[e];
        }
    };
    // the first batch (loaded before the first barrier), then any further one (d_v > 128, K > 128)
    update_batch(0);
    if (a.state_out) {
        if (tid < K) a.state_out[sb + (int64_t)tid * (dv + 1) + dv] = zn;
        store_batch(0);
    }
    for (int e0 = NB; g + e0 * np < K; e0 += NB) {
        load_batch(e0);
        update_batch(e0);
        if (a.state_out) store_batch(e0);
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

template <int DPL>
void launch_decode_dpl(const DecodeArgs& a, const dim3& g, const dim3& b, bool f32, hipStream_t s) {
    if (a.inv_var) {
        if (f32) hipLaunchKernelGGL((decode_kernel<true, true, DPL>), g, b, 0, s, a);
        else hipLaunchKernelGGL((decode_kernel<false, true, DPL>), g, b, 0, s, a);
    } else {
        if (f32) hipLaunchKernelGGL((decode_kernel<true, false, DPL>), g, b, 0, s, a);
        else hipLaunchKernelGGL((decode_kernel<false, false, DPL>), g, b, 0, s, a);
    }
}

void launch_decode(const DecodeArgs& a, int64_t bh, bool f32, hipStream_t s) {
    const dim3 g((unsigned)bh), b(kThreads);
    if (a.d_r <= 64) launch_decode_dpl<1>(a, g, b, f32, s);
    else if (a.d_r <= 128) launch_decode_dpl<2>(a, g, b, f32, s);
    else launch_decode_dpl<4>(a, g, b, f32, s);
}

void launch_decode_prepare(const DecodePrepArgs& a, int heads, hipStream_t s) {
    hipLaunchKernelGGL(decode_prepare_kernel, dim3((unsigned)heads), dim3(kThreads), 0, s, a);
}

}  // namespace gma
