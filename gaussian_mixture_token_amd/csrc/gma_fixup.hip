// Out-of-range rows of the bf16 path, recomputed exactly.
//
// Method: page "Attention par Mélange Gaussien (GMA)", section "Méthodologie", sub-section
// "Mécanisme Central": item 1 (posterior responsibilities under the head's diagonal GMM, softplus
// variances, softmax priors), item 2 (write Vt = Gamma_K^T V, Z = Gamma_K^T 1; read
// O = Gamma_Q Vt / (Gamma_Q Z + eps)) and item 3 (causal: prefix sums, the current token included).
//
// The bf16 kernels form their logits on fp16 matrix-core operands, so a routing input with |x| >= 256
// (x^2 past the fp16 range), or a mixture whose coefficients leave that range, gives a row whose logits
// are not finite.  Those kernels flag the (batch, head) of such a row; the kernels here run after them
// and recompute every flagged (batch, head) from the inputs with the log-density in its direct form,
// log pi_k - 1/2 sum_d [log sigma^2_kd + (x_d - mu_kd)^2 / sigma^2_kd], summed in fp64 (so any finite
// bf16 input is in range), the posterior in fp64, and the state in fp32.  Slices that are not flagged
// are skipped.  A few workgroups of 1024 threads, each walking (batch, head) slices:
//   set-up   mu and 1 / sigma^2 of the head, transposed to [d][k] in the workspace (lanes read
//            consecutive components), and c_k = log pi_k - 1/2 sum_d log sigma^2_kd in LDS (fp64);
//   rows     one wave per row: lanes over components, a sequential loop over dims, the softmax by
//            fixed-order butterflies;
//   forward  chunks of T tokens: the chunk's Gamma_K and Gamma_Q rows in LDS, then token by token the
//            state update [Vt | Z] += gamma_K (x) [v | 1] and the read of the output row (causal: the
//            update first, so the read includes the token; bidirectional: every update, then every read).
#include "gma_fixup.hpp"
#include "gma_device.hpp"

namespace gma {

namespace {

constexpr int kFixThreads = 1024;
constexpr int kFixWaves = kFixThreads / 64;

__device__ __forceinline__ double fix_wave_max(double x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmax(x, __shfl_xor(x, o, 64));
    return x;
}
__device__ __forceinline__ double fix_wave_sum(double x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

__device__ __forceinline__ float load_bf16(const void* base, int64_t i) {
    return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(base)[i] << 16);
}

// mu and 1 / sigma^2 of head h transposed into mt, it [d_r][K] (fp32), and the per-component constants
// c_k = log pi_k - 1/2 sum_d log sigma^2_kd into s_c (fp64: the logs in fp32, summed in dim order).
template <int KC>
__device__ void fix_setup(const FixArgs& a, int h, float* mt, float* it, double (&s_c)[KC], double* s_red) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int K = a.K, dr = a.d_r;
    for (int e = tid; e < K * dr; e += kFixThreads) {
        const int k = e / dr, d = e % dr;
        const int64_t i = ((int64_t)h * K + k) * dr + d;
        const float r = a.raw_var[i];
        const float var = fmaxf(r, 0.f) + log1pf(expf(-fabsf(r)));   // softplus
        mt[(int64_t)d * K + k] = a.mu[i];
        it[(int64_t)d * K + k] = 1.f / var;
    }
    if (w == 0) {
        double m = -INFINITY;
        for (int k = lane; k < K; k += 64) m = fmax(m, (double)a.prior[(int64_t)h * K + k]);
        m = fix_wave_max(m);
        double e = 0.0;
        for (int k = lane; k < K; k += 64) e += exp((double)a.prior[(int64_t)h * K + k] - m);
        e = fix_wave_sum(e);
        if (lane == 0) s_red[0] = m + log(e);
    }
    __syncthreads();
    const double lse = s_red[0];
    for (int k = tid; k < K; k += kFixThreads) {
        double sl = 0.0;
        for (int d = 0; d < dr; ++d) {
            const float r = a.raw_var[((int64_t)h * K + k) * dr + d];
            sl += (double)logf(fmaxf(r, 0.f) + log1pf(expf(-fabsf(r))));
        }
        s_c[k] = ((double)a.prior[(int64_t)h * K + k] - lse) - 0.5 * sl;
    }
    __syncthreads();
}

// Responsibilities of one row x (bf16, d_r elements) by one wave: lane l gets components l, l + 64, ...
// in g[] (0 past K).
template <int KC>
__device__ void fix_row_vals(const FixArgs& a, const void* x, int64_t row, const float* mt, const float* it,
                             const double (&s_c)[KC], double (&g)[(KC + 63) / 64]) {
    constexpr int NK = (KC + 63) / 64;
    const int lane = threadIdx.x & 63;
    const int K = a.K, dr = a.d_r;
    double l[NK];
#pragma unroll
    for (int u = 0; u < NK; ++u) l[u] = 0.0;
    for (int d = 0; d < dr; ++d) {
        const double xd = (double)load_bf16(x, row * dr + d);
#pragma unroll
        for (int u = 0; u < NK; ++u) {
            const int k = lane + 64 * u;
            if (k < K) {
                const double t = xd - (double)mt[(int64_t)d * K + k];
                l[u] += t * t * (double)it[(int64_t)d * K + k];
            }
        }
    }
    double m = -INFINITY;
#pragma unroll
    for (int u = 0; u < NK; ++u) {
        const int k = lane + 64 * u;
        l[u] = (k < K) ? s_c[k] - 0.5 * l[u] : -INFINITY;
        m = fmax(m, l[u]);
    }
    m = fix_wave_max(m);
    double s = 0.0;
#pragma unroll
    for (int u = 0; u < NK; ++u) {
        l[u] = (lane + 64 * u < K) ? exp(l[u] - m) : 0.0;
        s += l[u];
    }
    s = fix_wave_sum(s);
#pragma unroll
    for (int u = 0; u < NK; ++u) g[u] = l[u] / s;
}

// The same, stored to out[k] (fp32, LDS or global).
template <int KC>
__device__ void fix_row(const FixArgs& a, const void* x, int64_t row, const float* mt, const float* it,
                        const double (&s_c)[KC], float* out) {
    constexpr int NK = (KC + 63) / 64;
    const int lane = threadIdx.x & 63;
    double g[NK];
    fix_row_vals<KC>(a, x, row, mt, it, s_c, g);
#pragma unroll
    for (int u = 0; u < NK; ++u) {
        const int k = lane + 64 * u;
        if (k < a.K) out[k] = (float)g[u];
    }
}

// Responsibilities of every row of a flagged (batch, head) into gamma [BH, N, K].
template <int KC>
__global__ void __launch_bounds__(kFixThreads) fixup_resp_kernel(const FixArgs a) {
    __shared__ double s_c[KC];
    __shared__ double s_red[4];
    for (int64_t bh = blockIdx.x; bh < a.BH; bh += gridDim.x) {
        if (!a.flags[bh]) continue;
        const int h = (int)(bh % a.H);
        float* mt = a.scratch + (int64_t)h * 2 * a.K * a.d_r;
        float* it = mt + (int64_t)a.K * a.d_r;
        fix_setup<KC>(a, h, mt, it, s_c, s_red);
        const int w = threadIdx.x >> 6;
        for (int64_t r = w; r < a.N; r += kFixWaves)
            fix_row<KC>(a, a.qx, bh * a.N + r, mt, it, s_c, a.gamma + (bh * a.N + r) * a.K);
        __syncthreads();
    }
}

// Diagnostics of a flagged (batch, head): usage and hard counts over all its rows, into segment 0 of the
// partials (the other segments zeroed, so the fixed-order combine gives the totals).  Usage per lane in
// fp64, the waves' sums added in wave order; counts in LDS (integer, order-free).
template <int KC>
__global__ void __launch_bounds__(kFixThreads) fixup_stats_kernel(const FixArgs a) {
    constexpr int NK = (KC + 63) / 64;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int K = a.K;
    __shared__ double s_c[KC];
    __shared__ double s_red[4];
    __shared__ double s_use[kFixWaves][KC];
    __shared__ uint32_t s_cnt[KC];
    for (int64_t bh = blockIdx.x; bh < a.BH; bh += gridDim.x) {
    if (!a.flags[bh]) continue;
    const int h = (int)(bh % a.H);
    float* mt = a.scratch + (int64_t)h * 2 * K * a.d_r;
    float* it = mt + (int64_t)K * a.d_r;
    for (int k = tid; k < KC; k += kFixThreads) s_cnt[k] = 0u;
    fix_setup<KC>(a, h, mt, it, s_c, s_red);
    double use[NK];
#pragma unroll
    for (int u = 0; u < NK; ++u) use[u] = 0.0;
    for (int64_t r = w; r < a.N; r += kFixWaves) {
        double g[NK];
        fix_row_vals<KC>(a, a.qx, bh * a.N + r, mt, it, s_c, g);
        double best = -1.0;
        int bi = 0x7fffffff;
#pragma unroll
        for (int u = 0; u < NK; ++u) {
            use[u] += g[u];
            if (lane + 64 * u < K && g[u] > best) {
                best = g[u];
                bi = lane + 64 * u;
            }
        }
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const double ob = __shfl_xor(best, o, 64);
            const int oi = __shfl_xor(bi, o, 64);
            if (ob > best || (ob == best && oi < bi)) {
                best = ob;
                bi = oi;
            }
        }
        if (lane == 0 && bi < K) atomicAdd(&s_cnt[bi], 1u);
    }
#pragma unroll
    for (int u = 0; u < NK; ++u)
        if (lane + 64 * u < KC) s_use[w][lane + 64 * u] = use[u];
    __syncthreads();
    for (int k = tid; k < K; k += kFixThreads) {
        double u = 0.0;
        for (int v = 0; v < kFixWaves; ++v) u += s_use[v][k];
        for (int q = 0; q < a.stat_segs; ++q) {
            const int64_t i = (bh * a.stat_segs + q) * K + k;
            a.stat_usage[i] = q == 0 ? (float)u : 0.f;
            a.stat_count[i] = q == 0 ? s_cnt[k] : 0u;
        }
    }
    __syncthreads();
    }
}

// Forward of a flagged (batch, head): T tokens per chunk (the LDS holds the state [KC][VC] fp32 and the
// chunk's Gamma rows of both sides).
template <int KC, int VC, int T, bool CAUSAL>
__global__ void __launch_bounds__(kFixThreads) fixup_forward_kernel(const FixArgs a) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int K = a.K, dv = a.d_v;
    constexpr int PARTS = kFixThreads / VC;   // partial sums per output column
    __shared__ float s_st[KC * VC];
    __shared__ float s_z[KC];
    __shared__ double s_c[KC];
    __shared__ float s_gk[T][KC], s_gq[T][KC];
    __shared__ float s_part[PARTS][VC];
    __shared__ double s_red[4];
    for (int64_t bh = blockIdx.x; bh < a.BH; bh += gridDim.x) {
    if (!a.flags[bh]) continue;
    const int h = (int)(bh % a.H);
    float* mt = a.scratch + (int64_t)h * 2 * K * a.d_r;
    float* it = mt + (int64_t)K * a.d_r;
    fix_setup<KC>(a, h, mt, it, s_c, s_red);
    // the state before the first token: the carried state, or zero.  The record holds element (k, j) of
    // Vt at ((k / 16 * VC / 16 + j / 16) * 64 + (k % 16) / 4 * 16 + j % 16) * 4 + k % 4 and Z[k] at KC VC + k.
    const float* rin = a.rec_in ? a.rec_in + bh * ((int64_t)KC * VC + KC) : nullptr;
    for (int e = tid; e < KC * VC; e += kFixThreads) {
        const int k = e / VC, j = e % VC;
        const int r = (((k / 16) * (VC / 16) + j / 16) * 64 + (k % 16) / 4 * 16 + j % 16) * 4 + k % 4;
        s_st[e] = rin ? rin[r] : 0.f;
    }
    for (int k = tid; k < KC; k += kFixThreads) s_z[k] = rin ? rin[KC * VC + k] : 0.f;
    const int64_t rows_q = bh * a.N, rows_kv = bh * a.N_kv;
    // state update with the key / value row n (chunk slot t)
    auto update = [&](int t, int64_t n) {
        for (int e = tid; e < K * dv; e += kFixThreads) {
            const int k = e / dv, j = e % dv;
            s_st[k * VC + j] += s_gk[t][k] * load_bf16(a.v, (rows_kv + n) * dv + j);
        }
        for (int k = tid; k < K; k += kFixThreads) s_z[k] += s_gk[t][k];
    };
    // output row n (chunk slot t) from the current state: thread (part p, column j) sums the components
    // k = p, p + PARTS, ...; the partials and the denominator are added in a fixed order
    auto read = [&](int t, int64_t n) {
        const int j = tid % VC, p = tid / VC;
        float acc = 0.f;
        if (j < dv)
            for (int k = p; k < K; k += PARTS) acc += s_gq[t][k] * s_st[k * VC + j];
        s_part[p][j] = acc;
        if (w == 0) {
            double den = 0.0;
            for (int k = lane; k < K; k += 64) den += (double)s_gq[t][k] * (double)s_z[k];
            den = fix_wave_sum(den);
            if (lane == 0) s_red[1] = den;
        }
        __syncthreads();
        if (tid < dv) {
            float num = 0.f;
            for (int q = 0; q < PARTS; ++q) num += s_part[q][tid];
            const float o = num / ((float)s_red[1] + a.eps);
            reinterpret_cast<uint16_t*>(a.o)[(rows_q + n) * dv + tid] = bf16_bits(o);
        }
        __syncthreads();
    };
    // Gamma rows of the chunk [c0, c0 + nt): one wave per (row, side)
    auto gammas = [&](int64_t c0, int nt, bool kside, bool qside) {
        for (int r = w; r < 2 * nt; r += kFixWaves) {
            const int t = r >> 1;
            const bool q = r & 1;
            if (q ? qside : kside)
                fix_row<KC>(a, q ? a.qx : a.kx, (q ? rows_q : rows_kv) + c0 + t, mt, it, s_c, q ? s_gq[t] : s_gk[t]);
        }
        __syncthreads();
    };
    __syncthreads();
    // causal: one pass, each token's update before its read; bidirectional: every key / value row
    // (pass 0), then every query row (pass 1)
    for (int pass = 0; pass < (CAUSAL ? 1 : 2); ++pass) {
        const int64_t N = (CAUSAL || pass == 1) ? a.N : a.N_kv;
        for (int64_t c0 = 0; c0 < N; c0 += T) {
            const int nt = (int)((N - c0 < T) ? N - c0 : T);
            gammas(c0, nt, CAUSAL || pass == 0, CAUSAL || pass == 1);
            for (int t = 0; t < nt; ++t) {
                if (CAUSAL || pass == 0) {
                    update(t, c0 + t);
                    __syncthreads();
                }
                if (CAUSAL || pass == 1) read(t, c0 + t);
            }
        }
    }
    if (CAUSAL && a.state_out) {
        for (int e = tid; e < K * (dv + 1); e += kFixThreads) {
            const int k = e / (dv + 1), j = e % (dv + 1);
            a.state_out[bh * K * (dv + 1) + e] = (j < dv) ? s_st[k * VC + j] : s_z[k];
        }
    }
    __syncthreads();
    }
}

// Workgroups of the launch (each walks the slices bh = blockIdx.x, + gridDim.x, ...): few enough that a
// call with no flagged slice pays little for the launch.
constexpr int64_t kFixGrid = 32;
unsigned fix_grid(int64_t BH) { return (unsigned)(BH < kFixGrid ? BH : kFixGrid); }

template <int KC, int VC, int T>
void launch_fixup_forward_t(const FixArgs& a, int64_t BH, bool causal, hipStream_t s) {
    if (causal) hipLaunchKernelGGL((fixup_forward_kernel<KC, VC, T, true>), dim3(fix_grid(BH)), dim3(kFixThreads), 0, s, a);
    else hipLaunchKernelGGL((fixup_forward_kernel<KC, VC, T, false>), dim3(fix_grid(BH)), dim3(kFixThreads), 0, s, a);
}

}  // namespace

size_t fixup_scratch_bytes(int H, int K, int d_r) { return (size_t)H * 2 * K * d_r * sizeof(float); }

bool launch_fixup_forward(const FixArgs& a, int kc, int vc, int64_t BH, bool causal, hipStream_t s) {
    if (kc == 32 && vc == 64) launch_fixup_forward_t<32, 64, 64>(a, BH, causal, s);
    else if (kc == 128 && vc == 128) launch_fixup_forward_t<128, 128, 48>(a, BH, causal, s);
    else if (kc == 256 && vc == 64) launch_fixup_forward_t<256, 64, 32>(a, BH, causal, s);
    else if (kc == 256 && vc == 128) launch_fixup_forward_t<256, 128, 8>(a, BH, causal, s);
    else return false;
    return true;
}

bool launch_fixup_stats(const FixArgs& a, int kc, int64_t BH, hipStream_t s) {
    if (kc == 32) hipLaunchKernelGGL((fixup_stats_kernel<32>), dim3(fix_grid(BH)), dim3(kFixThreads), 0, s, a);
    else if (kc == 128) hipLaunchKernelGGL((fixup_stats_kernel<128>), dim3(fix_grid(BH)), dim3(kFixThreads), 0, s, a);
    else if (kc == 256) hipLaunchKernelGGL((fixup_stats_kernel<256>), dim3(fix_grid(BH)), dim3(kFixThreads), 0, s, a);
    else return false;
    return true;
}

bool launch_fixup_resp(const FixArgs& a, int kc, int64_t BH, hipStream_t s) {
    if (kc == 32) hipLaunchKernelGGL((fixup_resp_kernel<32>), dim3(fix_grid(BH)), dim3(kFixThreads), 0, s, a);
    else if (kc == 128) hipLaunchKernelGGL((fixup_resp_kernel<128>), dim3(fix_grid(BH)), dim3(kFixThreads), 0, s, a);
    else if (kc == 256) hipLaunchKernelGGL((fixup_resp_kernel<256>), dim3(fix_grid(BH)), dim3(kFixThreads), 0, s, a);
    else return false;
    return true;
}

}  // namespace gma
