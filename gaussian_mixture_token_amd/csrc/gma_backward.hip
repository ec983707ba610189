// Backward of the mixer on gfx950: the gradients of a loss with respect to Q_X, K_X, V and the raw
// mixture parameters, given dL/dO.
//
// Method: page "Attention par Mélange Gaussien (GMA)", section "Méthodologie", sub-section
// "Mécanisme Central".  The layer is trained end to end (item 3, softplus variances and softmax
// priors), so the gradient is the chain rule through items 1-3:
//   read   O_i = num_i / den_i with num_i = Gamma_Q[i] Vt_i, den_i = Gamma_Q[i] . Z_i + eps:
//            g_i = dO_i / den_i, h_i = -(dO_i . O_i) / den_i,
//            dGamma_Q[i] = Vt_i g_i + Z_i h_i
//   write  dGamma_K[j] = R_j v_j + r_j, dv_j = R_j^T gamma_K[j], where R_j, r_j sum
//            Gamma_Q[i] (x) g_i and Gamma_Q[i] h_i over the queries i that see key j
//   posterior (item 1)  dl = gamma (dgamma - gamma . dgamma)
//   log-density         dx_d = sum_k dl_k (mu_kd - x_d) / s_kd and, summed over rows,
//                       dl^T [x | x^2 | 1] give dmu, ds and dlog pi
// The causal variant runs the two sums in chunks of tokens: the state before a chunk (an
// exclusive prefix over chunks) plus the masked intra-chunk products, and the suffix sums R, r the
// same way backwards.
//
// Every contraction runs on the fp32 matrix cores through one batched product kernel; rows are
// handled by small vector kernels.  All arithmetic is fp32 (inputs upcast exactly from bf16); the
// results are rounded to the storage dtype once, at the end.
#include "gma_backward.hpp"
#include "gma_device.hpp"

#include <algorithm>
#include <cmath>

namespace gma {

namespace {

template <bool F32>
__device__ __forceinline__ float ld_elem(const void* base, int64_t i) {
    if constexpr (F32) return reinterpret_cast<const float*>(base)[i];
    else return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(base)[i] << 16);
}

template <bool F32>
__device__ __forceinline__ void st_elem(void* base, int64_t i, float x) {
    if constexpr (F32) reinterpret_cast<float*>(base)[i] = x;
    else reinterpret_cast<uint16_t*>(base)[i] = bf16_bits(x);
}

__device__ __forceinline__ float wave_sum_f(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

int64_t grid_for(int64_t n, int64_t per_block) {
    return std::max<int64_t>(1, std::min<int64_t>((n + per_block - 1) / per_block, int64_t(1) << 20));
}

// ---------------------------------------------------------------------------------- products
constexpr int GM = 64, GN = 64, GK = 16, GLD = 80;   // tile, inner step, LDS row pitch (floats)

// Workgroup of four wavefronts; wave w computes the 32 x 32 quarter (w / 2, w % 2) of the 64 x 64
// tile as 2 x 2 accumulator tiles.  The operand tiles are staged in LDS inner-index-major
// (s_a[k][m], s_b[k][n]) with a pitch of 80 floats, so that the 16-lane groups of a fragment read
// (4 inner rows x 16 consecutive columns) fall in disjoint banks.
template <bool TA, bool TB, bool OUT_BF16>
__global__ void __launch_bounds__(256) bwd_gemm_kernel(const BwdGemm g) {
    __shared__ float s_a[GK][GLD];
    __shared__ float s_b[GK][GLD];
    const int tiles_m = (g.M + GM - 1) / GM, tiles_n = (g.N + GN - 1) / GN;
    int64_t bid = blockIdx.x;
    const int tn = (int)(bid % tiles_n);
    bid /= tiles_n;
    const int tm = (int)(bid % tiles_m);
    bid /= tiles_m;
    const int inner = (int)(bid % g.n_inner);
    const int64_t outer = bid / g.n_inner;
    const int64_t left = g.ntok - (int64_t)inner * g.tok_step;
    const int M = (g.tok_flags & 1) ? (int)std::min<int64_t>(g.M, left) : g.M;
    const int N = (g.tok_flags & 2) ? (int)std::min<int64_t>(g.N, left) : g.N;
    const int Kd = (g.tok_flags & 4) ? (int)std::max<int64_t>(0, std::min<int64_t>(g.Kd, left)) : g.Kd;
    const int m0 = tm * GM, n0 = tn * GN;
    if (m0 >= M || n0 >= N) return;   // whole workgroup: the tile lies past a ragged end

    const float* A = g.A + outer * g.sA0 + (int64_t)inner * g.sA1;
    const float* B = g.B + (g.modB > 0 ? outer % g.modB : outer) * g.sB0 + (int64_t)inner * g.sB1;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = (w >> 1) * 32, wn = (w & 1) * 32;
    const int r = lane & 15, q = lane >> 4;
    f32x4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int k0 = 0; k0 < Kd; k0 += GK) {
        if constexpr (!TA) {   // A[m][k]: four consecutive k per thread
            const int m = tid >> 2, kk = (tid & 3) * 4;
            const bool mv = m0 + m < M;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int k = k0 + kk + j;
                s_a[kk + j][m] = (mv && k < Kd) ? A[(int64_t)(m0 + m) * g.lda + k] : 0.f;
            }
        } else {               // A[k][m]: four consecutive m per thread
            const int kk = tid >> 4, m = (tid & 15) * 4;
            const bool kv = k0 + kk < Kd;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                s_a[kk][m + j] = (kv && m0 + m + j < M) ? A[(int64_t)(k0 + kk) * g.lda + m0 + m + j] : 0.f;
        }
        if constexpr (!TB) {   // B[k][n]
            const int kk = tid >> 4, n = (tid & 15) * 4;
            const bool kv = k0 + kk < Kd;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                s_b[kk][n + j] = (kv && n0 + n + j < N) ? B[(int64_t)(k0 + kk) * g.ldb + n0 + n + j] : 0.f;
        } else {               // B[n][k]
            const int n = tid >> 2, kk = (tid & 3) * 4;
            const bool nv = n0 + n < N;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int k = k0 + kk + j;
                s_b[kk + j][n] = (nv && k < Kd) ? B[(int64_t)(n0 + n) * g.ldb + k] : 0.f;
            }
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < GK; ks += 4) {
            const float a0 = s_a[ks + q][wm + r], a1 = s_a[ks + q][wm + 16 + r];
            const float b0 = s_b[ks + q][wn + r], b1 = s_b[ks + q][wn + 16 + r];
            acc[0][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, b0, acc[0][0], 0, 0, 0);
            acc[0][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, b1, acc[0][1], 0, 0, 0);
            acc[1][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, b0, acc[1][0], 0, 0, 0);
            acc[1][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, b1, acc[1][1], 0, 0, 0);
        }
        __syncthreads();
    }

    const int64_t coff = outer * g.sC0 + (int64_t)inner * g.sC1;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = m0 + wm + mt * 16 + 4 * q + i, n = n0 + wn + nt * 16 + r;
                if (m >= M || n >= N) continue;
                float val = g.alpha * acc[mt][nt][i];
                if (g.tril && n > m) val = 0.f;
                const int64_t o = coff + (int64_t)m * g.ldc + n;
                if (g.Cin) val += g.beta * g.Cin[o];
                if constexpr (OUT_BF16) reinterpret_cast<uint16_t*>(g.C)[o] = bf16_bits(val);
                else reinterpret_cast<float*>(g.C)[o] = val;
            }
}

// ---------------------------------------------------------------------------------- mixture
// One workgroup per head; thread e handles elements e, e + 256, ... of [K, d_r].
__global__ void __launch_bounds__(256) bwd_prep_kernel(const float* mu, const float* raw_var, const float* prior,
                                                       float* mw, float* cp, int K, int d_r) {
    const int h = blockIdx.x, tid = threadIdx.x;
    const float* m_h = mu + (int64_t)h * K * d_r;
    const float* r_h = raw_var + (int64_t)h * K * d_r;
    float* mw_h = mw + (int64_t)h * K * 2 * d_r;
    for (int e = tid; e < K * d_r; e += 256) {
        const int k = e / d_r, d = e % d_r;
        const float rv = r_h[e];
        const float s = fmaxf(rv, 0.f) + log1pf(expf(-fabsf(rv)));   // softplus
        const float wv = 1.f / s;
        mw_h[(int64_t)k * 2 * d_r + d] = m_h[e] * wv;
        mw_h[(int64_t)k * 2 * d_r + d_r + d] = wv;
    }
    // log pi_k (log-softmax of the prior logits) and the log-determinant terms, fp64 sums
    __shared__ double s_lse;
    if (tid < 64) {
        double mx = -INFINITY;
        for (int k = tid; k < K; k += 64) mx = fmax(mx, (double)prior[(int64_t)h * K + k]);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o, 64));
        double sm = 0.0;
        for (int k = tid; k < K; k += 64) sm += exp((double)prior[(int64_t)h * K + k] - mx);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) sm += __shfl_xor(sm, o, 64);
        if (tid == 0) s_lse = mx + log(sm);
    }
    __syncthreads();
    for (int k = tid; k < K; k += 256) {
        double ld = 0.0;
        for (int d = 0; d < d_r; ++d) {
            const double rv = r_h[(int64_t)k * d_r + d];
            ld += log(fmax(rv, 0.0) + log1p(exp(-fabs(rv))));
        }
        cp[(int64_t)h * K + k] = (float)((double)prior[(int64_t)h * K + k] - s_lse - 0.5 * ld);
    }
}

// Responsibilities in the direct form l_k = cp_k - 1/2 sum_d (x_d - mu_kd)^2 / s_kd.  Workgroup:
// 64 rows of one (batch, head); thread (tr, tk) = (tid / 16, tid % 16) accumulates rows 4 tr + i and
// components tk + 16 j (j < KJ); the softmax over components reduces over the 16 lanes of a row
// group.  x, mu and 1/s are staged through LDS 16 dimensions at a time.  Each term is formed in fp32
// and the sum over d_r runs in fp64: the logits reach a few hundred at d_r = 256, and an fp32 running
// sum would put an error of about 1e-4 into gamma (fp64 adds cost no more than fp32 ones here).
template <int KJ, bool F32>
__global__ void __launch_bounds__(256) bwd_gamma_kernel(const void* x, const float* mu, const float* mw,
                                                        const float* cp, float* gamma, int64_t N, int H, int K,
                                                        int d_r) {
    constexpr int KC = 16 * KJ;
    __shared__ float s_x[64][17];
    __shared__ float s_m[KC][17];
    __shared__ float s_w[KC][17];
    const int64_t tiles = (N + 63) / 64;
    const int64_t bh = (int64_t)blockIdx.x / tiles;
    const int h = (int)(bh % H);
    const int64_t row0 = ((int64_t)blockIdx.x % tiles) * 64;
    const int tid = threadIdx.x, tk = tid & 15, tr = tid >> 4;
    double acc[4][KJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < KJ; ++j) acc[i][j] = 0.0;
    const float* m_h = mu + (int64_t)h * K * d_r;
    const float* w_h = mw + (int64_t)h * K * 2 * d_r + d_r;
    for (int d0 = 0; d0 < d_r; d0 += 16) {
        for (int e = tid; e < 64 * 16; e += 256) {
            const int rr = e >> 4, dd = e & 15;
            const int64_t row = row0 + rr;
            s_x[rr][dd] = (row < N && d0 + dd < d_r) ? ld_elem<F32>(x, (bh * N + row) * d_r + d0 + dd) : 0.f;
        }
        for (int e = tid; e < KC * 16; e += 256) {
            const int k = e >> 4, dd = e & 15;
            const bool in = k < K && d0 + dd < d_r;
            s_m[k][dd] = in ? m_h[(int64_t)k * d_r + d0 + dd] : 0.f;
            s_w[k][dd] = in ? w_h[(int64_t)k * 2 * d_r + d0 + dd] : 0.f;
        }
        __syncthreads();
#pragma unroll 4
        for (int dd = 0; dd < 16; ++dd) {
            float xv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) xv[i] = s_x[4 * tr + i][dd];
#pragma unroll
            for (int j = 0; j < KJ; ++j) {
                const float mv = s_m[tk + 16 * j][dd], wv = s_w[tk + 16 * j][dd];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float df = xv[i] - mv;
                    acc[i][j] += (double)(wv * df * df);
                }
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        double ld[KJ];
        double mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < KJ; ++j) {
            const int k = tk + 16 * j;
            ld[j] = (k < K) ? (double)cp[(int64_t)h * K + k] - 0.5 * acc[i][j] : -INFINITY;
            mx = fmax(mx, ld[j]);
        }
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o, 64));
        float l[KJ];
        float sm = 0.f;
#pragma unroll
        for (int j = 0; j < KJ; ++j) {
            l[j] = expf((float)(ld[j] - mx));
            sm += l[j];
        }
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) sm += __shfl_xor(sm, o, 64);
        const float inv = 1.f / sm;
        const int64_t row = row0 + 4 * tr + i;
        if (row < N) {
#pragma unroll
            for (int j = 0; j < KJ; ++j) {
                const int k = tk + 16 * j;
                if (k < K) gamma[(bh * N + row) * K + k] = l[j] * inv;
            }
        }
    }
}

// ---------------------------------------------------------------------------------- rows
template <bool F32>
__global__ void __launch_bounds__(256) bwd_vaug_kernel(const void* v, float* vaug, int64_t rows, int d_v, int dva) {
    const int64_t total = rows * dva;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
        const int64_t rr = e / dva;
        const int c = (int)(e % dva);
        vaug[e] = (c < d_v) ? ld_elem<F32>(v, rr * d_v + c) : (c == d_v ? 1.f : 0.f);
    }
}

template <bool F32>
__global__ void __launch_bounds__(256) bwd_xaug_kernel(const void* x, float* xaug, int64_t rows, int d_r, int dxa) {
    const int64_t total = rows * dxa;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
        const int64_t rr = e / dxa;
        const int c = (int)(e % dxa);
        float val;
        if (c < d_r) val = ld_elem<F32>(x, rr * d_r + c);
        else if (c < 2 * d_r) {
            const float t = ld_elem<F32>(x, rr * d_r + c - d_r);
            val = t * t;
        } else val = (c == 2 * d_r) ? 1.f : 0.f;
        xaug[e] = val;
    }
}

// one wavefront per row; lane l holds columns l, l + 64, ...
template <bool F32>
__global__ void __launch_bounds__(256) bwd_gh_kernel(const float* p, const void* dout, float* gh, int64_t rows, int d_v,
                                                     int dva, float eps) {
    const int lane = threadIdx.x & 63;
    const int64_t rr = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (rr >= rows) return;
    const float* pr = p + rr * dva;
    const float den = pr[d_v] + eps;
    const float inv = 1.f / den;
    float dot = 0.f;
    for (int c = lane; c < d_v; c += 64) dot += ld_elem<F32>(dout, rr * d_v + c) * (pr[c] * inv);
    dot = wave_sum_f(dot);
    for (int c = lane; c < dva; c += 64) {
        float val = 0.f;
        if (c < d_v) val = ld_elem<F32>(dout, rr * d_v + c) * inv;
        else if (c == d_v) val = -dot * inv;
        gh[rr * dva + c] = val;
    }
}

__global__ void __launch_bounds__(256) bwd_dl_kernel(const float* gamma, float* dg, int64_t rows, int K) {
    const int lane = threadIdx.x & 63;
    const int64_t rr = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (rr >= rows) return;
    const float* gr = gamma + rr * K;
    float* dr = dg + rr * K;
    float dot = 0.f;
    for (int k = lane; k < K; k += 64) dot += gr[k] * dr[k];
    dot = wave_sum_f(dot);
    for (int k = lane; k < K; k += 64) dr[k] = gr[k] * (dr[k] - dot);
}

template <bool F32>
__global__ void __launch_bounds__(256) bwd_dx_kernel(const void* x, const float* p12, void* dx, int64_t rows, int d_r) {
    const int64_t total = rows * d_r;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
        const int64_t rr = e / d_r;
        const int d = (int)(e % d_r);
        const float* pr = p12 + rr * 2 * d_r;
        st_elem<F32>(dx, e, pr[d] - ld_elem<F32>(x, e) * pr[d_r + d]);
    }
}

// ---------------------------------------------------------------------------------- scans
// thread = one state element of one (batch, head); sequential over the n chunk entries
__global__ void __launch_bounds__(256) bwd_scan_kernel(float* st, int64_t n, int64_t rec, int mode) {
    const int64_t per = (rec + 255) / 256;   // workgroups per (batch, head)
    const int64_t e = ((int64_t)blockIdx.x % per) * 256 + threadIdx.x;
    if (e >= rec) return;
    float* base = st + ((int64_t)blockIdx.x / per) * n * rec + e;
    float run = 0.f;
    if (mode == 0) {
        for (int64_t c = 0; c < n; ++c) {
            const float x = base[c * rec];
            base[c * rec] = run;
            run += x;
        }
    } else if (mode == 1) {
        for (int64_t c = n - 1; c >= 0; --c) {
            const float x = base[c * rec];
            base[c * rec] = run;
            run += x;
        }
    } else {
        for (int64_t c = 0; c < n; ++c) run += base[c * rec];
        base[0] = run;
    }
}

// ---------------------------------------------------------------------------------- parameters
// gp [2][B * H][n_seg][K][dxa]; element (k, d) of head blockIdx.y sums its partials in a fixed order:
//   G1 = sum dl x_d, G2 = sum dl x_d^2, G0 = sum dl
//   dmu = (G1 - mu G0) / s, ds = ((G2 - 2 mu G1 + mu^2 G0) / s^2 - G0 / s) / 2, draw_var = ds sigmoid(rho)
__global__ void __launch_bounds__(256) bwd_param_kernel(const float* gp, const float* mu, const float* raw_var,
                                                        float* dmu, float* draw_var, int64_t B, int H, int K, int d_r,
                                                        int dxa, int64_t n_seg) {
    const int per = (K * d_r + 255) / 256;   // workgroups per head
    const int h = blockIdx.x / per;
    const int e = (blockIdx.x % per) * 256 + threadIdx.x;
    if (e >= K * d_r) return;
    const int k = e / d_r, d = e % d_r;
    const int64_t part = (int64_t)K * dxa;
    float g0 = 0.f, g1 = 0.f, g2 = 0.f;
    for (int side = 0; side < 2; ++side)
        for (int64_t b = 0; b < B; ++b) {
            const float* p = gp + ((side * B + b) * H + h) * n_seg * part + (int64_t)k * dxa;
            for (int64_t sg = 0; sg < n_seg; ++sg) {
                g1 += p[sg * part + d];
                g2 += p[sg * part + d_r + d];
                g0 += p[sg * part + 2 * d_r];
            }
        }
    const int64_t pe = (int64_t)h * K * d_r + e;
    const float m = mu[pe], rv = raw_var[pe];
    const float s = fmaxf(rv, 0.f) + log1pf(expf(-fabsf(rv)));
    const float wv = 1.f / s;
    dmu[pe] = (g1 - m * g0) * wv;
    const float ds = 0.5f * ((g2 - 2.f * m * g1 + m * m * g0) * wv * wv - g0 * wv);
    draw_var[pe] = ds / (1.f + expf(-rv));
}

// dlog pi_k = G0_k summed like above; dprior_logits_k = G0_k - pi_k sum_j G0_j
__global__ void __launch_bounds__(256) bwd_prior_kernel(const float* gp, const float* prior, float* dprior, int64_t B,
                                                        int H, int K, int d_r, int dxa, int64_t n_seg) {
    const int h = blockIdx.x, tid = threadIdx.x;
    __shared__ float s_g[256];
    __shared__ float s_p[256];
    const int64_t part = (int64_t)K * dxa;
    if (tid < K) {
        float g0 = 0.f;
        for (int side = 0; side < 2; ++side)
            for (int64_t b = 0; b < B; ++b) {
                const float* p = gp + ((side * B + b) * H + h) * n_seg * part + (int64_t)tid * dxa + 2 * d_r;
                for (int64_t sg = 0; sg < n_seg; ++sg) g0 += p[sg * part];
            }
        s_g[tid] = g0;
        s_p[tid] = prior[(int64_t)h * K + tid];
    }
    __syncthreads();
    if (tid < K) {
        float mx = -INFINITY, tot = 0.f, z = 0.f;
        for (int k = 0; k < K; ++k) mx = fmaxf(mx, s_p[k]);
        for (int k = 0; k < K; ++k) {
            tot += s_g[k];
            z += expf(s_p[k] - mx);
        }
        dprior[(int64_t)h * K + tid] = s_g[tid] - expf(s_p[tid] - mx) / z * tot;
    }
}

template <bool TA, bool TB>
void gemm_dispatch(const BwdGemm& g, bool out_bf16, int64_t grid, hipStream_t s) {
    if (out_bf16) bwd_gemm_kernel<TA, TB, true><<<dim3((unsigned)grid), dim3(256), 0, s>>>(g);
    else bwd_gemm_kernel<TA, TB, false><<<dim3((unsigned)grid), dim3(256), 0, s>>>(g);
}

template <int KJ>
void gamma_dispatch(const void* x, bool f32, const float* mu, const float* mw, const float* cp, float* gamma,
                    int64_t BH, int64_t N, int H, int K, int d_r, hipStream_t s) {
    const dim3 grid((unsigned)((N + 63) / 64 * BH));
    if (f32) bwd_gamma_kernel<KJ, true><<<grid, dim3(256), 0, s>>>(x, mu, mw, cp, gamma, N, H, K, d_r);
    else bwd_gamma_kernel<KJ, false><<<grid, dim3(256), 0, s>>>(x, mu, mw, cp, gamma, N, H, K, d_r);
}

}  // namespace

void launch_bwd_gemm(const BwdGemm& g, bool ta, bool tb, bool out_bf16, hipStream_t s) {
    const int64_t tiles = (int64_t)((g.M + GM - 1) / GM) * ((g.N + GN - 1) / GN);
    const int64_t grid = tiles * g.n_inner * g.n_outer;
    if (grid <= 0) return;
    if (!ta && !tb) gemm_dispatch<false, false>(g, out_bf16, grid, s);
    else if (!ta && tb) gemm_dispatch<false, true>(g, out_bf16, grid, s);
    else if (ta && !tb) gemm_dispatch<true, false>(g, out_bf16, grid, s);
    else gemm_dispatch<true, true>(g, out_bf16, grid, s);
}

void launch_bwd_prep(const float* mu, const float* raw_var, const float* prior, float* mw, float* cp, int H, int K,
                     int d_r, hipStream_t s) {
    bwd_prep_kernel<<<dim3(H), dim3(256), 0, s>>>(mu, raw_var, prior, mw, cp, K, d_r);
}

void launch_bwd_gamma(const void* x, bool f32, const float* mu, const float* mw, const float* cp, float* gamma,
                      int64_t BH, int64_t N, int H, int K, int d_r, hipStream_t s) {
    const int kj = (K + 15) / 16;
    if (kj <= 1) gamma_dispatch<1>(x, f32, mu, mw, cp, gamma, BH, N, H, K, d_r, s);
    else if (kj <= 2) gamma_dispatch<2>(x, f32, mu, mw, cp, gamma, BH, N, H, K, d_r, s);
    else if (kj <= 4) gamma_dispatch<4>(x, f32, mu, mw, cp, gamma, BH, N, H, K, d_r, s);
    else if (kj <= 8) gamma_dispatch<8>(x, f32, mu, mw, cp, gamma, BH, N, H, K, d_r, s);
    else gamma_dispatch<16>(x, f32, mu, mw, cp, gamma, BH, N, H, K, d_r, s);
}

void launch_bwd_vaug(const void* v, bool f32, float* vaug, int64_t rows, int d_v, int dva, hipStream_t s) {
    const dim3 grid((unsigned)grid_for(rows * dva, 256));
    if (f32) bwd_vaug_kernel<true><<<grid, dim3(256), 0, s>>>(v, vaug, rows, d_v, dva);
    else bwd_vaug_kernel<false><<<grid, dim3(256), 0, s>>>(v, vaug, rows, d_v, dva);
}

void launch_bwd_xaug(const void* x, bool f32, float* xaug, int64_t rows, int d_r, int dxa, hipStream_t s) {
    const dim3 grid((unsigned)grid_for(rows * dxa, 256));
    if (f32) bwd_xaug_kernel<true><<<grid, dim3(256), 0, s>>>(x, xaug, rows, d_r, dxa);
    else bwd_xaug_kernel<false><<<grid, dim3(256), 0, s>>>(x, xaug, rows, d_r, dxa);
}

void launch_bwd_gh(const float* p, const void* dout, bool f32, float* gh, int64_t rows, int d_v, int dva, float eps,
                   hipStream_t s) {
    const dim3 grid((unsigned)((rows + 3) / 4));
    if (f32) bwd_gh_kernel<true><<<grid, dim3(256), 0, s>>>(p, dout, gh, rows, d_v, dva, eps);
    else bwd_gh_kernel<false><<<grid, dim3(256), 0, s>>>(p, dout, gh, rows, d_v, dva, eps);
}

void launch_bwd_dl(const float* gamma, float* dg, int64_t rows, int K, hipStream_t s) {
    bwd_dl_kernel<<<dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s>>>(gamma, dg, rows, K);
}

void launch_bwd_dx(const void* x, const float* p12, void* dx, bool f32, int64_t rows, int d_r, hipStream_t s) {
    const dim3 grid((unsigned)grid_for(rows * d_r, 256));
    if (f32) bwd_dx_kernel<true><<<grid, dim3(256), 0, s>>>(x, p12, dx, rows, d_r);
    else bwd_dx_kernel<false><<<grid, dim3(256), 0, s>>>(x, p12, dx, rows, d_r);
}

void launch_bwd_scan(float* st, int64_t n_outer, int64_t n, int64_t rec, int mode, hipStream_t s) {
    bwd_scan_kernel<<<dim3((unsigned)((rec + 255) / 256 * n_outer)), dim3(256), 0, s>>>(st, n, rec, mode);
}

void launch_bwd_param(const float* gp, const float* mu, const float* raw_var, const float* prior, float* dmu,
                      float* draw_var, float* dprior, int64_t B, int H, int K, int d_r, int dxa, int64_t n_seg,
                      hipStream_t s) {
    bwd_param_kernel<<<dim3((unsigned)((K * d_r + 255) / 256 * H)), dim3(256), 0, s>>>(
        gp, mu, raw_var, dmu, draw_var, B, H, K, d_r, dxa, n_seg);
    bwd_prior_kernel<<<dim3((unsigned)H), dim3(256), 0, s>>>(gp, prior, dprior, B, H, K, d_r, dxa, n_seg);
}

}  // namespace gma
