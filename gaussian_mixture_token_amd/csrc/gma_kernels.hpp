// HIP kernels of the GMA forward mixer for gfx950.
//
// Method (page "Attention par Mélange Gaussien (GMA)", section "Méthodologie",
// sub-section "Mécanisme Central"):
//   item 1: gamma_k(x) = pi_k N(x; mu_k, diag sigma2_k) / sum_j pi_j N(x; mu_j, diag sigma2_j)
//   item 2: write Vt = Gamma_K^T V, Z = Gamma_K^T 1; read O = Gamma_Q Vt / (Gamma_Q Z + eps)
//   item 3: causal variant by prefix sums (O_i sees j <= i); softplus variances, softmax priors.
//
// GPU formulation.  The log-density is expanded so that one MFMA GEMM produces the logits
// (in log2 units):
//   l2_k(x) = c_k + sum_d a_kd x_d^2 + b_kd x_d,
//   a_kd = -log2(e) / (2 sigma2_kd),  b_kd = log2(e) mu_kd / sigma2_kd,
//   c_k  = log2(e) (log pi_k - 1/2 sum_d (log sigma2_kd + mu_kd^2 / sigma2_kd)),
// i.e. logits^T = [a | b] (K x 2d_r) . [x^2 ; x] (2d_r x rows) + c.  The d_r/2 log(2 pi) term is
// common to all components and cancels in the posterior.  A softmax over K in base 2 gives Gamma.
//
// Kernels:
//   prep_kernel      raw parameters -> [a | b] operand fragments (fp16 or fp32) and c.
//   main_kernel<..., MODE>
//     MODE_RESP        Gamma of every row, written out in fp32.
//     MODE_AGG         per sequence segment: [Vt | Z] = sum over the segment of gamma_K (x) [v | 1].
//     MODE_OUT_BIDIR   O = Gamma_Q Vt / (Gamma_Q Z + eps) with the whole-sequence [Vt | Z].
//     MODE_OUT_CAUSAL  chunked causal scan: per chunk of C tokens, the masked intra-chunk
//                      tril(Gamma_Q Gamma_K^T)[V | 1] plus Gamma_Q . carried state, then the state
//                      is advanced by Gamma_K^T [V | 1].  The carry-in of each segment is the
//                      exclusive prefix of the MODE_AGG aggregates.
//   scan_kernel      (gma_host.cpp) exclusive prefix (causal) or total (bidirectional) of the
//                    segment aggregates.
//
// Work split inside a workgroup of W wavefronts: the logits/softmax phase splits the K
// components across waves (each wave keeps its [a | b] fragments in registers); the
// contraction phase splits d_v across waves (each wave owns state columns for all K
// components).  Gamma moves between the two splits through LDS as ready-made operand
// fragments.
#pragma once
#include "gma_device.hpp"

namespace gma {

enum { MODE_RESP = 0, MODE_AGG = 1, MODE_OUT_BIDIR = 2, MODE_OUT_CAUSAL = 3 };

template <bool F32> struct Tr;
template <> struct Tr<true> {
    using elem_t = float;      // storage of Q_X, K_X, V, O
    using xfrag_t = f32x4;     // logits operands
    using gfrag_t = f32x4;     // contraction operands
    static constexpr int KS = 16;   // contraction extent of one fragment step
    static constexpr int ES = 4;    // bytes per stored element
    static constexpr int XES = 4;   // bytes per staged X element (fp32)
    static constexpr int GES = 4;   // bytes per staged Gamma / V element (fp32)
};
template <> struct Tr<false> {
    using elem_t = uint16_t;   // bf16 bits
    using xfrag_t = f16x8;     // logits operands in fp16 (3 more mantissa bits than bf16)
    using gfrag_t = bf16x8;    // contraction operands in bf16 (fp32 exponent range)
    static constexpr int KS = 32;
    static constexpr int ES = 2;
    static constexpr int XES = 2;   // staged X in fp16
    static constexpr int GES = 2;   // staged Gamma / V in bf16
};

struct MainArgs {
    const void* qx;        // [BH, N, d_r]
    const void* kx;        // [BH, N, d_r]
    const void* v;         // [BH, N, d_v]
    void* o;               // [BH, N, d_v]
    float* gamma;          // [BH, N, K] (MODE_RESP)
    const void* ab;        // [H, KC/16, NKS, 64] x 16 bytes
    const float* cvec;     // [H, KC]
    float* seg;            // [BH, P, KC*VC + KC]
    int64_t N;
    int H, P;
    int d_r, d_v, K;
    int seg_chunks;        // chunks of C tokens per segment
    int vec_x, vec_v, vec_o;  // 16-byte (x, v) / 4-element (o) vector access allowed
    int has_carry;         // causal: load the carried state (P > 1)
    float eps;
};

struct PrepArgs {
    const float* mu;        // [H, K, d_r]
    const float* raw_var;   // [H, K, d_r]
    const float* prior;     // [H, K]
    void* ab;               // out
    float* cvec;            // out [H, KC]
    int H, K, d_r;
};

// ---------------------------------------------------------------------------------------------
// prep: softplus variances, log-softmax priors, expanded-quadratic coefficients.
// One workgroup per head.  [a | b] is written in the exact per-lane fragment order the main
// kernel loads: ab[h][ct][ks][lane][j] = A[comp = 16 ct + lane % 16][k = ks*KS + (lane/16)*(KS/4) + j]
// with A = [a | b] (k < DRC: a_{comp,k}; k >= DRC: b_{comp,k-DRC}).  Pad components get
// a = b = 0 and c = -inf (their posterior is exactly 0); pad dimensions get a = b = 0.
template <bool F32, int KC, int DRC>
__global__ void __launch_bounds__(256) prep_kernel(const PrepArgs p) {
    using T = Tr<F32>;
    constexpr int KS = T::KS;
    constexpr int NKS = 2 * DRC / KS;
    constexpr int EPL = KS / 4;  // elements per lane per fragment
    const int h = blockIdx.x;
    const int tid = threadIdx.x;
    const double LOG2E = 1.4426950408889634073599246810019;
    __shared__ double s_red[256];
    __shared__ double s_lse;

    // log-sum-exp of the prior logits of this head
    double m = -INFINITY;
    for (int k = tid; k < p.K; k += 256) m = fmax(m, (double)p.prior[(int64_t)h * p.K + k]);
    s_red[tid] = m;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (tid < s) s_red[tid] = fmax(s_red[tid], s_red[tid + s]);
        __syncthreads();
    }
    const double mx = s_red[0];
    __syncthreads();
    double acc = 0.0;
    for (int k = tid; k < p.K; k += 256) acc += exp((double)p.prior[(int64_t)h * p.K + k] - mx);
    s_red[tid] = acc;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (tid < s) s_red[tid] += s_red[tid + s];
        __syncthreads();
    }
    if (tid == 0) s_lse = mx + log(s_red[0]);
    __syncthreads();
    const double lse = s_lse;

    // c_k
    for (int k = tid; k < KC; k += 256) {
        float c = -INFINITY;
        if (k < p.K) {
            double sum = 0.0;
            for (int d = 0; d < p.d_r; ++d) {
                const int64_t i = ((int64_t)h * p.K + k) * p.d_r + d;
                const double r = p.raw_var[i];
                const double var = fmax(r, 0.0) + log1p(exp(-fabs(r)));
                const double mu = p.mu[i];
                sum += log(var) + mu * mu / var;
            }
            const double logpi = (double)p.prior[(int64_t)h * p.K + k] - lse;
            c = (float)(LOG2E * (logpi - 0.5 * sum));
        }
        p.cvec[(int64_t)h * KC + k] = c;
    }

    // [a | b] fragments
    constexpr int TOTAL = (KC / 16) * NKS * 64 * EPL;
    for (int idx = tid; idx < TOTAL; idx += 256) {
        const int j = idx % EPL;
        const int lane = (idx / EPL) % 64;
        const int ks = (idx / (EPL * 64)) % NKS;
        const int ct = idx / (EPL * 64 * NKS);
        const int comp = ct * 16 + (lane & 15);
        const int kk = ks * KS + (lane >> 4) * EPL + j;
        const bool is_b = kk >= DRC;
        const int d = is_b ? kk - DRC : kk;
        double val = 0.0;
        if (comp < p.K && d < p.d_r) {
            const int64_t i = ((int64_t)h * p.K + comp) * p.d_r + d;
            const double r = p.raw_var[i];
            const double var = fmax(r, 0.0) + log1p(exp(-fabs(r)));
            val = is_b ? LOG2E * (double)p.mu[i] / var : -0.5 * LOG2E / var;
        }
        const int64_t out = (int64_t)h * TOTAL + idx;
        if constexpr (F32) {
            reinterpret_cast<float*>(p.ab)[out] = (float)val;
        } else {
            reinterpret_cast<_Float16*>(p.ab)[out] = (_Float16)(float)val;
        }
    }
}

// ---------------------------------------------------------------------------------------------
// Staging helpers (global -> LDS).

// X rows [C][DRC] -> LDS (fp16 for bf16 inputs, fp32 otherwise), zero-padded in d and in rows.
template <bool F32, int C, int DRC, int NTHR>
__device__ __forceinline__ void stage_x(char* lds, const typename Tr<F32>::elem_t* __restrict__ g,
                                        int rows_valid, int d_r, bool vec, int tid) {
    using T = Tr<F32>;
    constexpr int VEC = 16 / T::ES;              // elements per 16-byte global vector
    constexpr int XS = DRC * T::XES + 16;        // LDS row stride (bytes)
    constexpr int NV = DRC / VEC;                // vectors per row
    for (int i = tid; i < C * NV; i += NTHR) {
        const int r = i / NV;
        const int c0 = (i % NV) * VEC;
        char* dst = lds + r * XS + c0 * T::XES;
        if constexpr (F32) {
            f32x4 val = {0.f, 0.f, 0.f, 0.f};
            if (r < rows_valid && c0 < d_r) {
                const float* src = g + (int64_t)r * d_r + c0;
                if (vec) {
                    val = *reinterpret_cast<const f32x4*>(src);
                } else {
                    for (int e = 0; e < 4; ++e) val[e] = (c0 + e < d_r) ? src[e] : 0.f;
                }
            }
            *reinterpret_cast<f32x4*>(dst) = val;
        } else {
            u32x4 raw = {0u, 0u, 0u, 0u};
            if (r < rows_valid && c0 < d_r) {
                const uint16_t* src = g + (int64_t)r * d_r + c0;
                if (vec) {
                    raw = *reinterpret_cast<const u32x4*>(src);
                } else {
                    uint16_t tmp[8];
                    for (int e = 0; e < 8; ++e) tmp[e] = (c0 + e < d_r) ? src[e] : (uint16_t)0;
                    for (int e = 0; e < 4; ++e) raw[e] = (uint32_t)tmp[2 * e] | ((uint32_t)tmp[2 * e + 1] << 16);
                }
            }
            f16x8 h;
            for (int e = 0; e < 4; ++e) {
                h[2 * e] = (_Float16)bf16_bits_to_f32(raw[e] & 0xffffu);
                h[2 * e + 1] = (_Float16)bf16_bits_to_f32(raw[e] >> 16);
            }
            *reinterpret_cast<f16x8*>(dst) = h;
        }
    }
}

// V rows [C][VC] -> LDS transposed, VT[d][token], zero-padded.  Each thread moves a block of
// 4 tokens x VEC columns so that the transposed writes are 8 (bf16) or 16 (fp32) bytes wide.
template <bool F32, int C, int VC, int NTHR>
__device__ __forceinline__ void stage_vt(char* lds, const typename Tr<F32>::elem_t* __restrict__ g,
                                         int rows_valid, int d_v, bool vec, int tid) {
    using T = Tr<F32>;
    constexpr int VEC = 16 / T::ES;
    constexpr int VTS = C * T::GES + 16;         // LDS row stride (bytes) of VT
    constexpr int NV = VC / VEC;
    for (int i = tid; i < (C / 4) * NV; i += NTHR) {
        const int c0 = (i % NV) * VEC;
        const int t0 = (i / NV) * 4;
        if constexpr (F32) {
            f32x4 val[4];
            for (int t = 0; t < 4; ++t) {
                val[t] = f32x4{0.f, 0.f, 0.f, 0.f};
                const int r = t0 + t;
                if (r < rows_valid && c0 < d_v) {
                    const float* src = g + (int64_t)r * d_v + c0;
                    if (vec) {
                        val[t] = *reinterpret_cast<const f32x4*>(src);
                    } else {
                        for (int e = 0; e < 4; ++e) val[t][e] = (c0 + e < d_v) ? src[e] : 0.f;
                    }
                }
            }
            for (int e = 0; e < 4; ++e) {
                f32x4 col = {val[0][e], val[1][e], val[2][e], val[3][e]};
                *reinterpret_cast<f32x4*>(lds + (c0 + e) * VTS + t0 * 4) = col;
            }
        } else {
            uint16_t val[4][8];
            for (int t = 0; t < 4; ++t) {
                const int r = t0 + t;
                if (r < rows_valid && c0 < d_v) {
                    const uint16_t* src = g + (int64_t)r * d_v + c0;
                    if (vec) {
                        u32x4 raw = *reinterpret_cast<const u32x4*>(src);
                        for (int e = 0; e < 4; ++e) {
                            val[t][2 * e] = (uint16_t)(raw[e] & 0xffffu);
                            val[t][2 * e + 1] = (uint16_t)(raw[e] >> 16);
                        }
                    } else {
                        for (int e = 0; e < 8; ++e) val[t][e] = (c0 + e < d_v) ? src[e] : (uint16_t)0;
                    }
                } else {
                    for (int e = 0; e < 8; ++e) val[t][e] = 0;
                }
            }
            for (int e = 0; e < 8; ++e) {
                u32x2 col = {(uint32_t)val[0][e] | ((uint32_t)val[1][e] << 16),
                             (uint32_t)val[2][e] | ((uint32_t)val[3][e] << 16)};
                *reinterpret_cast<u32x2*>(lds + (c0 + e) * VTS + t0 * 2) = col;
            }
        }
    }
}

// ---------------------------------------------------------------------------------------------
// Main kernel.  Grid: BH * P workgroups (segment-major inside a head); block: W wavefronts.
template <bool F32, int KC, int VC, int DRC, int W, int C, int MODE>
__global__ void __launch_bounds__(W * 64) main_kernel(const MainArgs a) {
    using T = Tr<F32>;
    using elem_t = typename T::elem_t;
    using xfrag_t = typename T::xfrag_t;
    using gfrag_t = typename T::gfrag_t;
    constexpr int NTHR = W * 64;
    constexpr int KS = T::KS;
    constexpr int NT = C / 16;               // token tiles per chunk
    constexpr int NCT = KC / 16;             // component tiles
    constexpr int KT_W = NCT / W;            // component tiles per wave (logits phase)
    constexpr int NVT = VC / 16;             // d_v tiles
    constexpr int VT_W = (MODE == MODE_RESP) ? 1 : NVT / W;   // d_v tiles per wave (contraction phase)
    constexpr int NKS = 2 * DRC / KS;        // logits fragment steps ([x^2 | x])
    constexpr int NKS2 = NKS / 2;
    constexpr int NKQ = KC / KS;             // fragment steps over components
    constexpr int NTK = C / KS;              // fragment steps over tokens
    constexpr int XS = DRC * T::XES + 16;    // staged X row stride (bytes)
    constexpr int VTS = C * T::GES + 16;     // staged V^T row stride (bytes)
    constexpr bool NEED_Q = (MODE == MODE_RESP) || (MODE == MODE_OUT_BIDIR) || (MODE == MODE_OUT_CAUSAL);
    constexpr bool NEED_K = (MODE == MODE_AGG) || (MODE == MODE_OUT_CAUSAL);
    constexpr bool NEED_V = NEED_K;
    constexpr bool HAS_STATE = (MODE != MODE_RESP);
    static_assert(NCT % W == 0, "components must split evenly across waves");
    static_assert(MODE == MODE_RESP || NVT % W == 0, "d_v must split evenly across waves");
    static_assert(KC % KS == 0 && C % KS == 0 && (2 * DRC) % KS == 0, "tile shapes");
    static_assert(F32 || KT_W % 2 == 0 || W >= 1, "");

    __shared__ __attribute__((aligned(16))) char s_xq[NEED_Q ? C * XS : 16];
    __shared__ __attribute__((aligned(16))) char s_xk[NEED_K ? C * XS : 16];
    __shared__ __attribute__((aligned(16))) char s_vt[NEED_V ? VC * VTS : 16];
    __shared__ __attribute__((aligned(16))) char s_gq[(MODE == MODE_OUT_BIDIR || MODE == MODE_OUT_CAUSAL) ? NT * NKQ * 1024 : 16];
    __shared__ __attribute__((aligned(16))) char s_gk[(MODE == MODE_OUT_CAUSAL) ? NT * NKQ * 1024 : 16];
    __shared__ __attribute__((aligned(16))) char s_gkc[NEED_K ? NCT * NTK * 1024 : 16];
    __shared__ float s_ms[2][W][C][2];
    __shared__ float s_den[W][C];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int lr = lane & 15;
    const int lg = lane >> 4;
    const int bh = blockIdx.x / a.P;
    const int sidx = blockIdx.x % a.P;
    const int h = bh % a.H;
    const int64_t N = a.N;
    const int64_t n_chunks = (N + C - 1) / C;
    const int64_t ch0 = (int64_t)sidx * a.seg_chunks;
    const int64_t ch1 = (ch0 + a.seg_chunks < n_chunks) ? ch0 + a.seg_chunks : n_chunks;

    const elem_t* qx = reinterpret_cast<const elem_t*>(a.qx) + (int64_t)bh * N * a.d_r;
    const elem_t* kx = reinterpret_cast<const elem_t*>(a.kx) + (int64_t)bh * N * a.d_r;
    const elem_t* vv = reinterpret_cast<const elem_t*>(a.v) + (int64_t)bh * N * a.d_v;

    // ---- per-wave constants: [a | b] fragments and c for the wave's own components
    xfrag_t abf[KT_W][NKS];
    f32x4 cinit[KT_W];
    {
        const xfrag_t* abg = reinterpret_cast<const xfrag_t*>(a.ab) + (int64_t)h * NCT * NKS * 64;
#pragma unroll
        for (int kt = 0; kt < KT_W; ++kt) {
            const int ct = w * KT_W + kt;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) abf[kt][ks] = abg[((int64_t)ct * NKS + ks) * 64 + lane];
            const float* cv = a.cvec + (int64_t)h * KC + ct * 16 + lg * 4;
            cinit[kt] = f32x4{cv[0], cv[1], cv[2], cv[3]};
        }
    }

    // ---- running state: [Vt | Z] columns owned by this wave (all components), Z of own components
    constexpr int ST_T = HAS_STATE ? NCT : 1;
    constexpr int ST_V = HAS_STATE ? VT_W : 1;
    f32x4 st[ST_T][ST_V];
    f32x4 zown[KT_W];
    const int64_t rec = (int64_t)KC * VC + KC;
    float* segrec = a.seg + ((int64_t)bh * a.P + sidx) * rec;
    if constexpr (HAS_STATE) {
        const bool load = (MODE == MODE_OUT_BIDIR) || (MODE == MODE_OUT_CAUSAL && a.has_carry);
        const float* src = (MODE == MODE_OUT_BIDIR) ? a.seg + (int64_t)bh * a.P * rec : segrec;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int vt = 0; vt < VT_W; ++vt) {
                const int gvt = w * VT_W + vt;
                st[ct][vt] = load ? *reinterpret_cast<const f32x4*>(src + ((int64_t)(ct * NVT + gvt) * 64 + lane) * 4)
                                  : f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
        for (int kt = 0; kt < KT_W; ++kt) {
            const int ct = w * KT_W + kt;
            zown[kt] = load ? *reinterpret_cast<const f32x4*>(src + (int64_t)KC * VC + ct * 16 + lg * 4)
                            : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }

    for (int64_t ch = ch0; ch < ch1; ++ch) {
        const int64_t n0 = ch * C;
        const int rows_valid = (int)((N - n0 < C) ? N - n0 : C);

        // ---- stage inputs of this chunk
        if constexpr (NEED_Q) stage_x<F32, C, DRC, NTHR>(s_xq, qx + n0 * a.d_r, rows_valid, a.d_r, a.vec_x, tid);
        if constexpr (NEED_K) stage_x<F32, C, DRC, NTHR>(s_xk, kx + n0 * a.d_r, rows_valid, a.d_r, a.vec_x, tid);
        if constexpr (NEED_V) stage_vt<F32, C, VC, NTHR>(s_vt, vv + n0 * a.d_v, rows_valid, a.d_v, a.vec_v, tid);
        __syncthreads();

        // ---- logits^T tiles for own components: lq[kt][tt] (rows: comps 4g+i of tile ct, col: token 16tt+r)
        f32x4 lq[NEED_Q ? KT_W : 1][NT];
        f32x4 lk[NEED_K ? KT_W : 1][NT];
        auto logits = [&](const char* sx, f32x4 (&acc)[KT_W][NT]) {
#pragma unroll
            for (int kt = 0; kt < KT_W; ++kt)
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) acc[kt][tt] = cinit[kt];
#pragma unroll
            for (int ks = 0; ks < NKS2; ++ks) {
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) {
                    const xfrag_t xf = *reinterpret_cast<const xfrag_t*>(
                        sx + (tt * 16 + lr) * XS + (ks * KS + lg * (KS / 4)) * T::XES);
                    const xfrag_t x2 = xf * xf;
#pragma unroll
                    for (int kt = 0; kt < KT_W; ++kt) {
                        mma(acc[kt][tt], abf[kt][ks], x2);
                        mma(acc[kt][tt], abf[kt][ks + NKS2], xf);
                    }
                }
            }
        };
        if constexpr (NEED_Q) logits(s_xq, lq);
        if constexpr (NEED_K) logits(s_xk, lk);

        // ---- softmax over K, part 1: per-wave max and sum of exp2 over own components
        float mq[NT], mk[NT];
        auto local_softmax = [&](f32x4 (&acc)[KT_W][NT], float (&mloc)[NT], int which) {
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                float m = -INFINITY;
#pragma unroll
                for (int kt = 0; kt < KT_W; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) m = fmaxf(m, acc[kt][tt][i]);
                m = group4_max(m);
                const float msafe = (m == -INFINITY) ? 0.f : m;
                float s = 0.f;
#pragma unroll
                for (int kt = 0; kt < KT_W; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float p = fast_exp2(acc[kt][tt][i] - msafe);
                        acc[kt][tt][i] = p;
                        s += p;
                    }
                s = group4_sum(s);
                mloc[tt] = m;
                if (lg == 0) {
                    s_ms[which][w][tt * 16 + lr][0] = m;
                    s_ms[which][w][tt * 16 + lr][1] = s;
                }
            }
        };
        if constexpr (NEED_Q) local_softmax(lq, mq, 0);
        if constexpr (NEED_K) local_softmax(lk, mk, 1);
        __syncthreads();

        // ---- softmax part 2: combine the W partial (max, sum) pairs; scale to posteriors
        auto finish_softmax = [&](f32x4 (&acc)[KT_W][NT], const float (&mloc)[NT], int which) {
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                const int tok = tt * 16 + lr;
                float M = -INFINITY;
#pragma unroll
                for (int ww = 0; ww < W; ++ww) M = fmaxf(M, s_ms[which][ww][tok][0]);
                float S = 0.f;
#pragma unroll
                for (int ww = 0; ww < W; ++ww) S += s_ms[which][ww][tok][1] * fast_exp2(s_ms[which][ww][tok][0] - M);
                float f = (mloc[tt] == -INFINITY || tok >= rows_valid) ? 0.f : fast_exp2(mloc[tt] - M) / S;
#pragma unroll
                for (int kt = 0; kt < KT_W; ++kt) acc[kt][tt] *= f;
            }
        };
        if constexpr (NEED_Q) finish_softmax(lq, mq, 0);
        if constexpr (NEED_K) finish_softmax(lk, mk, 1);

        if constexpr (MODE == MODE_RESP) {
            // Gamma rows out: lane holds comps 16ct + 4g .. +3 of token 16tt + r
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                const int tok = tt * 16 + lr;
                if (tok >= rows_valid) continue;
                float* grow = a.gamma + ((int64_t)bh * N + n0 + tok) * a.K;
#pragma unroll
                for (int kt = 0; kt < KT_W; ++kt) {
                    const int c0 = (w * KT_W + kt) * 16 + lg * 4;
                    if ((a.K & 3) == 0 && c0 + 4 <= a.K) {
                        *reinterpret_cast<f32x4*>(grow + c0) = lq[kt][tt];
                    } else {
                        for (int i = 0; i < 4; ++i)
                            if (c0 + i < a.K) grow[c0 + i] = lq[kt][tt][i];
                    }
                }
            }
            __syncthreads();  // s_xq / s_ms reuse by the next chunk
            continue;
        }

        // ---- Gamma to LDS as operand fragments; denominators from the carried Z
        if constexpr (MODE == MODE_OUT_BIDIR || MODE == MODE_OUT_CAUSAL) {
            // token-row fragments of Gamma_Q: frag[tt][kq][lane] holds comps of step kq for token 16tt + r
#pragma unroll
            for (int kt = 0; kt < KT_W; ++kt) {
                const int ct = w * KT_W + kt;
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) {
                    if constexpr (F32) {
                        *reinterpret_cast<f32x4*>(s_gq + ((tt * NKQ + ct) * 64 + lane) * 16) = lq[kt][tt];
                    } else {
                        *reinterpret_cast<bf16x4*>(s_gq + ((tt * NKQ + (ct >> 1)) * 64 + lane) * 16 + (ct & 1) * 8) =
                            pack4(lq[kt][tt]);
                    }
                }
            }
            // partial denominators over own components: sum_k gamma_Q[n,k] Z[k]
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                float d = 0.f;
#pragma unroll
                for (int kt = 0; kt < KT_W; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) d += lq[kt][tt][i] * zown[kt][i];
                d = group4_sum(d);
                if (lg == 0) s_den[w][tt * 16 + lr] = d;
            }
        }
        if constexpr (NEED_K) {
            if constexpr (MODE == MODE_OUT_CAUSAL) {
#pragma unroll
                for (int kt = 0; kt < KT_W; ++kt) {
                    const int ct = w * KT_W + kt;
#pragma unroll
                    for (int tt = 0; tt < NT; ++tt) {
                        if constexpr (F32) {
                            *reinterpret_cast<f32x4*>(s_gk + ((tt * NKQ + ct) * 64 + lane) * 16) = lk[kt][tt];
                        } else {
                            *reinterpret_cast<bf16x4*>(s_gk + ((tt * NKQ + (ct >> 1)) * 64 + lane) * 16 + (ct & 1) * 8) =
                                pack4(lk[kt][tt]);
                        }
                    }
                }
            }
            // comp-row fragments of Gamma_K^T: frag[ct][tk][lane'] holds, for component 16ct + (lane' % 16),
            // the tokens of step tk in slots matching the V^T fragments (4 consecutive tokens per group).
#pragma unroll
            for (int kt = 0; kt < KT_W; ++kt) {
                const int ct = w * KT_W + kt;
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int lane2 = (lg * 4 + i) + 16 * (lr >> 2);
                        if constexpr (F32) {
                            const int slot = lr & 3;
                            reinterpret_cast<float*>(s_gkc + ((ct * NTK + tt) * 64 + lane2) * 16)[slot] = lk[kt][tt][i];
                        } else {
                            const int slot = (lr & 3) + 4 * (tt & 1);
                            reinterpret_cast<__bf16*>(s_gkc + ((ct * NTK + (tt >> 1)) * 64 + lane2) * 16)[slot] =
                                to_bf16(lk[kt][tt][i]);
                        }
                    }
                }
            }
        }
        __syncthreads();

        // ---- contraction phase: this wave owns d_v tiles [w*VT_W, (w+1)*VT_W)
        gfrag_t vf[NEED_V ? VT_W : 1][NTK];
        if constexpr (NEED_V) {
#pragma unroll
            for (int vt = 0; vt < VT_W; ++vt) {
                const int row = (w * VT_W + vt) * 16 + lr;
#pragma unroll
                for (int tk = 0; tk < NTK; ++tk) {
                    if constexpr (F32) {
                        vf[vt][tk] = *reinterpret_cast<const f32x4*>(s_vt + row * VTS + (tk * 16 + lg * 4) * 4);
                    } else {
                        const u32x2 lo = *reinterpret_cast<const u32x2*>(s_vt + row * VTS + ((2 * tk) * 16 + lg * 4) * 2);
                        const u32x2 hi = *reinterpret_cast<const u32x2*>(s_vt + row * VTS + ((2 * tk + 1) * 16 + lg * 4) * 2);
                        u32x4 both = {lo[0], lo[1], hi[0], hi[1]};
                        vf[vt][tk] = __builtin_bit_cast(bf16x8, both);
                    }
                }
            }
        }

        if constexpr (MODE == MODE_OUT_BIDIR || MODE == MODE_OUT_CAUSAL) {
            f32x4 oacc[VT_W][NT];
#pragma unroll
            for (int vt = 0; vt < VT_W; ++vt)
#pragma unroll
                for (int I = 0; I < NT; ++I) oacc[vt][I] = f32x4{0.f, 0.f, 0.f, 0.f};
            float den[NT];

            // state operand fragments (A: rows d_v, contraction over components)
            gfrag_t sf[VT_W][NKQ];
#pragma unroll
            for (int vt = 0; vt < VT_W; ++vt)
#pragma unroll
                for (int kq = 0; kq < NKQ; ++kq) {
                    if constexpr (F32) sf[vt][kq] = st[kq][vt];
                    else sf[vt][kq] = pack_pair(st[2 * kq][vt], st[2 * kq + 1][vt]);
                }

#pragma unroll
            for (int I = 0; I < NT; ++I) {
                gfrag_t gqf[NKQ];
#pragma unroll
                for (int kq = 0; kq < NKQ; ++kq)
                    gqf[kq] = *reinterpret_cast<const gfrag_t*>(s_gq + ((I * NKQ + kq) * 64 + lane) * 16);
                // inter: O^T(vt, I) += state^T . Gamma_Q^T
#pragma unroll
                for (int vt = 0; vt < VT_W; ++vt)
#pragma unroll
                    for (int kq = 0; kq < NKQ; ++kq) mma(oacc[vt][I], sf[vt][kq], gqf[kq]);
                float d = 0.f;
#pragma unroll
                for (int ww = 0; ww < W; ++ww) d += s_den[ww][I * 16 + lr];

                if constexpr (MODE == MODE_OUT_CAUSAL) {
                    // intra: S^T(J, I) = Gamma_K[J] Gamma_Q[I]^T for J <= I, masked j <= i
                    f32x4 sacc[NT];
                    float dsum = 0.f;
#pragma unroll
                    for (int J = 0; J < NT; ++J) {
                        sacc[J] = f32x4{0.f, 0.f, 0.f, 0.f};
                        if (J > I) continue;
#pragma unroll
                        for (int kq = 0; kq < NKQ; ++kq) {
                            const gfrag_t gkf = *reinterpret_cast<const gfrag_t*>(s_gk + ((J * NKQ + kq) * 64 + lane) * 16);
                            mma(sacc[J], gkf, gqf[kq]);
                        }
                        if (J == I) {
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                if (lg * 4 + i > lr) sacc[J][i] = 0.f;
                        }
                        if constexpr (!F32) {
                            // round to the operand precision so numerator and denominator agree
#pragma unroll
                            for (int i = 0; i < 4; ++i) sacc[J][i] = (float)to_bf16(sacc[J][i]);
                        }
#pragma unroll
                        for (int i = 0; i < 4; ++i) dsum += sacc[J][i];
                    }
                    d += group4_sum(dsum);
                    // O^T(vt, I) += V^T(vt, tokens) . S^T(tokens, I)
#pragma unroll
                    for (int tk = 0; tk < NTK; ++tk) {
                        if constexpr (F32) {
                            if (tk > I) continue;
#pragma unroll
                            for (int vt = 0; vt < VT_W; ++vt) mma(oacc[vt][I], vf[vt][tk], sacc[tk]);
                        } else {
                            if (2 * tk > I) continue;
                            const bf16x8 sfr = pack_pair(sacc[2 * tk], sacc[2 * tk + 1]);
#pragma unroll
                            for (int vt = 0; vt < VT_W; ++vt) mma(oacc[vt][I], vf[vt][tk], sfr);
                        }
                    }
                }
                den[I] = d + a.eps;
            }

            // ---- write O: lane holds d_v 16vt' + 4g .. +3 of token 16I + r
#pragma unroll
            for (int I = 0; I < NT; ++I) {
                const int tok = I * 16 + lr;
                if (tok >= rows_valid) continue;
                const float inv = 1.0f / den[I];
                elem_t* orow = reinterpret_cast<elem_t*>(a.o) + ((int64_t)bh * N + n0 + tok) * a.d_v;
#pragma unroll
                for (int vt = 0; vt < VT_W; ++vt) {
                    const int c0 = (w * VT_W + vt) * 16 + lg * 4;
                    f32x4 ov = oacc[vt][I] * inv;
                    if (a.vec_o && c0 + 4 <= a.d_v) {
                        if constexpr (F32) {
                            *reinterpret_cast<f32x4*>(orow + c0) = ov;
                        } else {
                            *reinterpret_cast<bf16x4*>(orow + c0) = pack4(ov);
                        }
                    } else {
                        for (int i = 0; i < 4; ++i) {
                            if (c0 + i < a.d_v) {
                                if constexpr (F32) orow[c0 + i] = ov[i];
                                else orow[c0 + i] = bf16_bits(ov[i]);
                            }
                        }
                    }
                }
            }
        }

        // ---- advance the state: [Vt | Z] += Gamma_K^T [V | 1]
        if constexpr (NEED_K) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int tk = 0; tk < NTK; ++tk) {
                    const gfrag_t gkc = *reinterpret_cast<const gfrag_t*>(s_gkc + ((ct * NTK + tk) * 64 + lane) * 16);
#pragma unroll
                    for (int vt = 0; vt < VT_W; ++vt) mma(st[ct][vt], gkc, vf[vt][tk]);
                }
#pragma unroll
            for (int kt = 0; kt < KT_W; ++kt) {
                f32x4 zs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) zs += lk[kt][tt];
#pragma unroll
                for (int i = 0; i < 4; ++i) zown[kt][i] += row16_sum(zs[i]);
            }
        }
        __syncthreads();  // LDS buffers are restaged by the next chunk
    }

    if constexpr (MODE == MODE_AGG) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int vt = 0; vt < VT_W; ++vt) {
                const int gvt = w * VT_W + vt;
                *reinterpret_cast<f32x4*>(segrec + ((int64_t)(ct * NVT + gvt) * 64 + lane) * 4) = st[ct][vt];
            }
        if (lr == 0) {
#pragma unroll
            for (int kt = 0; kt < KT_W; ++kt) {
                const int ct = w * KT_W + kt;
                *reinterpret_cast<f32x4*>(segrec + (int64_t)KC * VC + ct * 16 + lg * 4) = zown[kt];
            }
        }
    }
}

}  // namespace gma
