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
#include <type_traits>
#include <cmath>
#include <cstdlib>

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

// ---------------------------------------------------------------------------------- products
constexpr int GM = 64, GN = 64, GK = 32, GLD = 80;   // tile, inner step, LDS row pitch (floats)

// Eight fp32 values as bf16 hi (nearest even) and lo = the rounded remainder: hi + lo carries about 16
// significant bits of each value.
__device__ __forceinline__ void split_bf16x8(const float (&v)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const __bf16 h = (__bf16)v[j];
        hi[j] = h;
        lo[j] = (__bf16)(v[j] - (float)h);
    }
}

// Workgroup of four wavefronts; wave w computes the 32 x 32 quarter (w / 2, w % 2) of the 64 x 64
// tile as 2 x 2 accumulator tiles (v_mfma_f32_16x16x4_f32).  Operand tiles are staged in LDS
// inner-index-major (s_a[k][m], s_b[k][n]) with a pitch of 80 floats: the 16-lane groups of a
// fragment read (4 inner rows x 16 consecutive columns) fall in disjoint banks.  The next inner
// step's operands are fetched into registers while the current one is multiplied.
//
// Global fetch of an operand whose inner index is contiguous (A not transposed, B transposed):
// thread t takes row t % 64 and inner elements 8 (t / 64) .. + 7 of the step, so that each wave's
// LDS writes cover 64 consecutive columns of one inner row.  Of an operand whose outer index is
// contiguous: thread t takes inner row t / 8 and columns 8 (t % 8) .. + 7.  Eight consecutive
// elements inside the matrix are fetched as two 16-byte loads where the view allows it (vec*).
// GA / GB: operand A / B is generated (BwdGemm::ga / gb, GEN_*) instead of read.  DX: the routing-input
// gradient epilogue (BwdGemm::dx_x).
template <bool TA, bool TB, bool OUT_BF16, int GA = GEN_NONE, int GB = GEN_NONE, bool DX = false>
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

    const float* A = GA ? nullptr : g.A + outer * g.sA0 + (int64_t)inner * g.sA1;
    const float* B = GB ? nullptr : g.B + (g.modB > 0 ? outer % g.modB : outer) * g.sB0 + (int64_t)inner * g.sB1;
    // first row of a generated operand's view
    const int64_t ga0 = GA ? outer * g.sA0 + (int64_t)inner * g.sA1 : 0;
    const int64_t gb0 = GB ? outer * g.sB0 + (int64_t)inner * g.sB1 : 0;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = (w >> 1) * 32, wn = (w & 1) * 32;
    const int r = lane & 15, q = lane >> 4;

    // fetch of 8 elements: contiguous in the inner index (row `row` of the view, inner k .. k+7) or
    // in the outer one (inner row k, columns c .. c+7)
    auto fetch_inner = [](const float* X, int ld, bool vec, int row, bool row_ok, int k, int kd, float (&v)[8]) {
        const float* p = X + (int64_t)row * ld + k;
        if (vec && row_ok && k + 8 <= kd) {
            const f32x4 lo = *reinterpret_cast<const f32x4*>(p), hi = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
            for (int j = 0; j < 4; ++j) { v[j] = lo[j]; v[4 + j] = hi[j]; }
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = (row_ok && k + j < kd) ? p[j] : 0.f;
        }
    };
    auto fetch_outer = [](const float* X, int ld, bool vec, int k, bool k_ok, int c, int cn, float (&v)[8]) {
        const float* p = X + (int64_t)k * ld + c;
        if (vec && k_ok && c + 8 <= cn) {
            const f32x4 lo = *reinterpret_cast<const f32x4*>(p), hi = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
            for (int j = 0; j < 4; ++j) { v[j] = lo[j]; v[4 + j] = hi[j]; }
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = (k_ok && c + j < cn) ? p[j] : 0.f;
        }
    };
    float ra[8], rb[8];
    const int ri = tid & 63, ki = (tid >> 6) * 8;     // contiguous-inner mapping
    const int ko = tid >> 3, co = (tid & 7) * 8;      // contiguous-outer mapping
    // columns c .. c+7 (columns >= cn read as zero) of row `row` of a generated operand: one 16-byte
    // load of eight storage elements where the columns lie inside one part of the row and the layout
    // allows it, element by element otherwise
    auto gen = [&](auto kind_tag, const BwdGen& s, int64_t row, bool ok, int c, int cn, bool vec, float (&v)[8]) {
        constexpr int kind = decltype(kind_tag)::value;
        const int d = s.d;
        const int64_t e0 = row * d;
        auto ld1 = [&](int col) -> float {
            if (s.f32) return reinterpret_cast<const float*>(s.src)[e0 + col];
            return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(s.src)[e0 + col] << 16);
        };
        float scale = 1.f, tail = 1.f;   // GEN_GH: 1 / den and h of the row
        if constexpr (kind == GEN_GH) {
            if (ok) {
                scale = s.rs[2 * row];
                tail = s.rs[2 * row + 1];
            }
        }
        const bool sq = kind == GEN_XAUG && c >= d;   // the x^2 part
        const int d0 = sq ? c - d : c;
        if (ok && vec && c + 8 <= cn && d0 + 8 <= d && (!sq || c + 8 <= 2 * d)) {
            float x[8];
            if (s.f32) {
                const f32x4 lo = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(s.src) + e0 + d0);
                const f32x4 hi = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(s.src) + e0 + d0 + 4);
#pragma unroll
                for (int j = 0; j < 4; ++j) { x[j] = lo[j]; x[4 + j] = hi[j]; }
            } else {
                const u32x4 h = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(s.src) + e0 + d0);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    x[2 * j] = __uint_as_float(h[j] << 16);
                    x[2 * j + 1] = __uint_as_float(h[j] & 0xffff0000u);
                }
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = sq ? x[j] * x[j] : x[j] * scale;
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int col = c + j;
                float val = 0.f;
                if (ok && col < cn) {
                    if (col < d) {
                        val = ld1(col) * scale;
                    } else if (kind == GEN_XAUG) {
                        if (col < 2 * d) {
                            const float t = ld1(col - d);
                            val = t * t;
                        } else if (col == 2 * d) {
                            val = 1.f;
                        }
                    } else if (col == d) {
                        val = tail;
                    }
                }
                v[j] = val;
            }
        }
    };
    auto fetch = [&](int k0) {
        if constexpr (GA != GEN_NONE) {
            static_assert(!TA, "a generated A is read row by row");
            gen(std::integral_constant<int, GA>{}, g.ga, ga0 + m0 + ri, m0 + ri < M, k0 + ki, Kd, g.vecA, ra);
        } else if constexpr (!TA) fetch_inner(A, g.lda, g.vecA, m0 + ri, m0 + ri < M, k0 + ki, Kd, ra);
        else fetch_outer(A, g.lda, g.vecA, k0 + ko, k0 + ko < Kd, m0 + co, M, ra);
        if constexpr (GB != GEN_NONE) {
            if constexpr (TB) gen(std::integral_constant<int, GB>{}, g.gb, gb0 + n0 + ri, n0 + ri < N, k0 + ki, Kd, g.vecB, rb);
            else gen(std::integral_constant<int, GB>{}, g.gb, gb0 + k0 + ko, k0 + ko < Kd, n0 + co, N, g.vecB, rb);
        } else if constexpr (TB) fetch_inner(B, g.ldb, g.vecB, n0 + ri, n0 + ri < N, k0 + ki, Kd, rb);
        else fetch_outer(B, g.ldb, g.vecB, k0 + ko, k0 + ko < Kd, n0 + co, N, rb);
    };
    auto stage = [&]() {
        if constexpr (!TA) {
#pragma unroll
            for (int j = 0; j < 8; ++j) s_a[ki + j][ri] = ra[j];
        } else {
            *reinterpret_cast<f32x4*>(&s_a[ko][co]) = f32x4{ra[0], ra[1], ra[2], ra[3]};
            *reinterpret_cast<f32x4*>(&s_a[ko][co + 4]) = f32x4{ra[4], ra[5], ra[6], ra[7]};
        }
        if constexpr (TB) {
#pragma unroll
            for (int j = 0; j < 8; ++j) s_b[ki + j][ri] = rb[j];
        } else {
            *reinterpret_cast<f32x4*>(&s_b[ko][co]) = f32x4{rb[0], rb[1], rb[2], rb[3]};
            *reinterpret_cast<f32x4*>(&s_b[ko][co + 4]) = f32x4{rb[4], rb[5], rb[6], rb[7]};
        }
    };

    f32x4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // accumulator tiles wholly past a ragged edge are skipped (wave-uniform)
    const bool mok1 = m0 + wm + 16 < M, nok1 = n0 + wn + 16 < N;
    const bool wave_ok = m0 + wm < M && n0 + wn < N;

    if (Kd > 0) {
        fetch(0);
        stage();
        __syncthreads();
    }
    for (int k0 = 0; k0 < Kd; k0 += GK) {
        const bool more = k0 + GK < Kd;
        if (more) fetch(k0 + GK);
        if (wave_ok && g.split) {
            // one 32-deep step on the bf16 matrix cores: lane group q takes inner indices q, q + 4, ..,
            // q + 28 of both operands (the matrix core pairs element j of A's and B's fragments, so any
            // common order sums the same products; this one reads four disjoint bank groups at pitch 80)
            bf16x8 ah[2], al[2], bh[2], bl[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                float va[8], vb[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    va[j] = s_a[q + 4 * j][wm + 16 * t + r];
                    vb[j] = s_b[q + 4 * j][wn + 16 * t + r];
                }
                split_bf16x8(va, ah[t], al[t]);
                split_bf16x8(vb, bh[t], bl[t]);
            }
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    if ((mt && !mok1) || (nt && !nok1)) continue;
                    mma(acc[mt][nt], al[mt], bh[nt]);
                    mma(acc[mt][nt], ah[mt], bl[nt]);
                    mma(acc[mt][nt], ah[mt], bh[nt]);
                }
        } else if (wave_ok) {
#pragma unroll
            for (int ks = 0; ks < GK; ks += 4) {
                const float a0 = s_a[ks + q][wm + r], a1 = s_a[ks + q][wm + 16 + r];
                const float b0 = s_b[ks + q][wn + r], b1 = s_b[ks + q][wn + 16 + r];
                acc[0][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, b0, acc[0][0], 0, 0, 0);
                if (nok1) acc[0][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, b1, acc[0][1], 0, 0, 0);
                if (mok1) acc[1][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, b0, acc[1][0], 0, 0, 0);
                if (mok1 && nok1) acc[1][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, b1, acc[1][1], 0, 0, 0);
            }
        }
        __syncthreads();
        if (more) {
            stage();
            __syncthreads();
        }
    }

    const int64_t coff = outer * g.sC0 + (int64_t)inner * g.sC1;
    if constexpr (DX) {
        // lanes r and r ^ 1 hold columns 2d and 2d + 1 of the same row: the even lane forms dx of dim d
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float val = acc[mt][nt][i];
                    const float oth = __shfl_xor(val, 1, 64);
                    const int m = m0 + wm + mt * 16 + 4 * q + i, n = n0 + wn + nt * 16 + r;
                    if (m >= M || n >= N || (r & 1)) continue;
                    const int64_t o = coff + (int64_t)m * g.ldc + (n >> 1);
                    float xv;
                    if constexpr (OUT_BF16) xv = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(g.dx_x)[o] << 16);
                    else xv = reinterpret_cast<const float*>(g.dx_x)[o];
                    const float dxv = val - xv * oth;
                    if constexpr (OUT_BF16) reinterpret_cast<uint16_t*>(g.C)[o] = bf16_bits(dxv);
                    else reinterpret_cast<float*>(g.C)[o] = dxv;
                }
        return;
    }
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
// The operands of the matrix-core log-densities (expanded form
//   l_k = cq_k + sum_d (-s_kd^-1 / 2) x_d^2 + sum_d (mu_kd / s_kd) x_d,
//   cq_k = log pi_k - 1/2 sum_d (log s_kd + mu_kd^2 / s_kd), fp64):
// bf [H][d_r / 16 steps][2 parts (x^2, x)][KT][64 lanes][4]: lane (r, q) of component tile kt holds the
// coefficients of component 16 kt + r for dims 16 step + 4 q .. + 3 (zero past K or d_r), the order
// of the A fragments of the rows; cq [H][16 KT] with -inf past K.
// One workgroup per (head, component tile): workgroup h * KT + kt writes the coefficients of tile kt
// and the constants cq of its 16 components.  The terms log s_kd + mu_kd^2 / s_kd of cq are computed in
// parallel, 128 dims at a time, into LDS; one thread per component adds them in dim order.
// split (d_r a multiple of 32): the operands for bwd_gamma_split_kernel instead, in the same bytes:
// bf16 [H][d_r / 32 steps][KT][4 parts: a hi, a lo, b hi, b lo][64 lanes][8], lane (r, g) of tile kt
// holding component 16 kt + r, dims 32 step + 8 g .. + 7 (a = -1 / (2 s), b = mu / s, hi the nearest
// bf16, lo the bf16 of the remainder).
__global__ void __launch_bounds__(256) bwd_frag_kernel(const float* mu, const float* raw_var, const float* prior,
                                                       float* bf, double* cq, int K, int d_r, int KT, int split) {
    const int h = blockIdx.x / KT, kt = blockIdx.x % KT, tid = threadIdx.x;
    const int steps = (d_r + 15) / 16, KP = 16 * KT;
    const int64_t per_head = (int64_t)steps * 2 * KT * 256;
    if (split) {
        uint16_t* fb = reinterpret_cast<uint16_t*>(bf + (int64_t)h * per_head);
        const int S = d_r / 32;
        for (int i = tid; i < S * 512; i += 256) {
            const int st = i >> 9, lane = (i >> 3) & 63, e = i & 7;
            const int k = 16 * kt + (lane & 15), d = 32 * st + 8 * (lane >> 4) + e;
            float a = 0.f, b = 0.f;
            if (k < K) {
                const int64_t pe = ((int64_t)h * K + k) * d_r + d;
                const float rv = raw_var[pe];
                const float sv = fmaxf(rv, 0.f) + log1pf(expf(-fabsf(rv)));
                a = -0.5f / sv;
                b = mu[pe] / sv;
            }
            const float parts[2] = {a, b};
#pragma unroll
            for (int pb = 0; pb < 2; ++pb) {
                const uint16_t hb = bf16_bits(parts[pb]);
                const uint16_t lb = bf16_bits(parts[pb] - __uint_as_float((uint32_t)hb << 16));
                const int64_t base = ((int64_t)(st * KT + kt) * 4 + 2 * pb) * 512 + lane * 8 + e;
                fb[base] = hb;
                fb[base + 512] = lb;
            }
        }
    }
    // element e of the head's operands: e >> 8 = (2 st + part) KT + kt, e & 255 = 4 lane + j
    for (int i = tid; i < (split ? 0 : 2 * steps * 256); i += 256) {
        const int sp = i >> 8;
        const int64_t e = ((int64_t)sp * KT + kt) * 256 + (i & 255);
        const int j = i & 3, lane = (i >> 2) & 63;
        const int part = sp & 1, st = sp >> 1;
        const int k = 16 * kt + (lane & 15), d = 16 * st + 4 * (lane >> 4) + j;
        float val = 0.f;
        if (k < K && d < d_r) {
            const int64_t pe = ((int64_t)h * K + k) * d_r + d;
            const float rv = raw_var[pe];
            const float sv = fmaxf(rv, 0.f) + log1pf(expf(-fabsf(rv)));
            val = part == 0 ? -0.5f / sv : mu[pe] / sv;
        }
        bf[(int64_t)h * per_head + e] = val;
    }
    __shared__ double s_lse;
    __shared__ double s_term[16 * 128];
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
    double acc = 0.0;
    for (int d0 = 0; d0 < d_r; d0 += 128) {
        const int nd = d_r - d0 < 128 ? d_r - d0 : 128;
        for (int i = tid; i < 16 * 128; i += 256) {
            const int r = i >> 7, dd = i & 127, k = 16 * kt + r;
            double term = 0.0;
            if (k < K && dd < nd) {
                const int64_t pe = ((int64_t)h * K + k) * d_r + d0 + dd;
                const double rv = raw_var[pe], m = mu[pe];
                const double sv = fmax(rv, 0.0) + log1p(exp(-fabs(rv)));
                term = log(sv) + m * m / sv;
            }
            s_term[i] = term;
        }
        __syncthreads();
        if (tid < 16)
            for (int dd = 0; dd < nd; ++dd) acc += s_term[tid * 128 + dd];
        __syncthreads();
    }
    if (tid < 16) {
        const int k = 16 * kt + tid;
        double c = -INFINITY;
        if (k < K) c = (double)prior[(int64_t)h * K + k] - s_lse - 0.5 * acc;
        cq[(int64_t)h * KP + k] = c;
    }
}

// Element e = k d_r + d of [K, d_r] of head h: workgroup blockIdx.x = h * per + e / 256 with per
// workgroups per head, one thread per element.
__global__ void __launch_bounds__(256) bwd_prep_kernel(const float* mu, const float* raw_var, float* mw, int K,
                                                       int d_r) {
    const int per = (K * d_r + 255) / 256;
    const int h = blockIdx.x / per;
    const int e = (blockIdx.x % per) * 256 + threadIdx.x;
    if (e >= K * d_r) return;
    const float* m_h = mu + (int64_t)h * K * d_r;
    const float* r_h = raw_var + (int64_t)h * K * d_r;
    float* mw_h = mw + (int64_t)h * K * 2 * d_r;
    const int k = e / d_r, d = e % d_r;
    const float rv = r_h[e];
    const float s = fmaxf(rv, 0.f) + log1pf(expf(-fabsf(rv)));   // softplus
    const float wv = 1.f / s;
    mw_h[(int64_t)k * 2 * d_r + 2 * d] = m_h[e] * wv;
    mw_h[(int64_t)k * 2 * d_r + 2 * d + 1] = wv;
}

// Responsibilities on the fp32 matrix cores, expanded form (see bwd_frag_kernel).  Workgroup: 64 G
// rows of one (batch, head); wave w takes the 16-row groups w, w + 4, ... (G of them) against all 16 KT
// components.  Per step of 16 dims the step's coefficient fragments (2 KT KiB) are staged once in LDS
// for the workgroup (double-buffered, the next step's fetched into registers meanwhile); lane (r, q)
// holds x and x^2 of row r of a group, dims 4 q .. 4 q + 3 (the permuted contraction order of the
// fragments), and each component tile takes four v_mfma_f32_16x16x4_f32 per part.  The fp32
// accumulators of a step are added into fp64 ones after the step, so that no fp32 sum runs over more
// than 32 products (the logits reach a few hundred); constants in fp64.  Softmax over the components
// of each row: in registers over the tiles, butterflies over the 16 lanes of a column.
template <int KT, int G, bool F32>
__global__ void __launch_bounds__(256) bwd_gamma_mfma_kernel(const void* x, const float* bf, const double* cq,
                                                             float* gamma, int64_t N, int H, int K, int d_r,
                                                             int vecx) {
    constexpr int NF = 2 * KT * 64;                  // f32x4 fragments per step
    constexpr int NE = (NF + 255) / 256;             // ... staged per thread
    __shared__ f32x4 s_bf[2][NF];
    const int64_t tiles = (N + 64 * G - 1) / (64 * G);
    const int64_t bh = (int64_t)blockIdx.x / tiles;
    const int h = (int)(bh % H);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r = lane & 15, q = lane >> 4;
    const int64_t base = ((int64_t)blockIdx.x % tiles) * 64 * G;
    const int steps = (d_r + 15) / 16;
    const f32x4* bfh = reinterpret_cast<const f32x4*>(bf) + (int64_t)h * steps * NF;
    double acc[G][KT][4];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[g][kt][i] = 0.0;
    f32x4 pre[NE];
    auto fetch_b = [&](int st) {
#pragma unroll
        for (int e = 0; e < NE; ++e)
            if (tid + 256 * e < NF) pre[e] = bfh[(int64_t)st * NF + tid + 256 * e];
    };
    auto stage_b = [&](int buf) {
#pragma unroll
        for (int e = 0; e < NE; ++e)
            if (tid + 256 * e < NF) s_bf[buf][tid + 256 * e] = pre[e];
    };
    fetch_b(0);
    stage_b(0);
    __syncthreads();
    for (int st = 0; st < steps; ++st) {
        const int buf = st & 1;
        if (st + 1 < steps) fetch_b(st + 1);
        const int d0 = 16 * st + 4 * q;
        f32x4 xa[G], x2[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int64_t row = base + 16 * (w + 4 * g) + r;
            xa[g] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (row < N) {
                const int64_t off = (bh * N + row) * d_r + d0;
                if (vecx && d0 + 4 <= d_r) {
                    if constexpr (F32) {
                        xa[g] = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(x) + off);
                    } else {
                        const u32x2 u = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(x) + off);
                        xa[g] = f32x4{__uint_as_float(u[0] << 16), __uint_as_float(u[0] & 0xffff0000u),
                                      __uint_as_float(u[1] << 16), __uint_as_float(u[1] & 0xffff0000u)};
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (d0 + j < d_r) xa[g][j] = ld_elem<F32>(x, off + j);
                }
            }
            x2[g] = xa[g] * xa[g];
        }
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            const f32x4 bsq = s_bf[buf][kt * 64 + lane], blin = s_bf[buf][(KT + kt) * 64 + lane];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                f32x4 c = {0.f, 0.f, 0.f, 0.f};
                mma(c, x2[g], bsq);
                mma(c, xa[g], blin);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[g][kt][i] += (double)c[i];
            }
        }
        if (st + 1 < steps) stage_b(buf ^ 1);
        __syncthreads();
    }
    const double* cqh = cq + (int64_t)h * 16 * KT;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int64_t row0 = base + 16 * (w + 4 * g) + 4 * q;   // accumulator rows 4 q + i of the group
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            double mx = -INFINITY;
            double l[KT];
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
                l[kt] = cqh[16 * kt + r] + acc[g][kt][i];
                mx = fmax(mx, l[kt]);
            }
#pragma unroll
            for (int o = 8; o > 0; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o, 64));
            float e[KT];
            float sm = 0.f;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
                e[kt] = expf((float)(l[kt] - mx));
                sm += e[kt];
            }
#pragma unroll
            for (int o = 8; o > 0; o >>= 1) sm += __shfl_xor(sm, o, 64);
            const float inv = 1.f / sm;
            const int64_t rr = row0 + i;
            if (rr < N) {
#pragma unroll
                for (int kt = 0; kt < KT; ++kt) {
                    const int k = 16 * kt + r;
                    if (k < K) gamma[(bh * N + rr) * K + k] = e[kt] * inv;
                }
            }
        }
    }
}

// Responsibilities for bf16 storage on the bf16 matrix cores (d_r a multiple of 32): the expanded form
// with x exact in bf16 and x^2, a, b split into bf16 hi + lo (the lo lo products dropped), fp32
// accumulation: x b_lo + x b_hi + x^2_lo a_hi + x^2_hi a_lo + x^2_hi a_hi per 32 dims and component
// tile, five v_mfma_f32_16x16x32_bf16.  The head's operand fragments (bwd_frag_kernel, split) stay in
// LDS for the workgroup, which walks `rows` consecutive rows of one (batch, head) (a multiple of 64 G) in
// blocks of 64 G, wave w the G 16-row groups w, w + 4, .. of a block (lane (r, g): row r of a group, dims
// 8 g .. 8 g + 7 of a step), so that every fragment read from LDS serves G groups; the next block's x
// is loaded during the current block.  The product is formed transposed (coefficient fragments
// as A, the rows as B), so that each lane ends with four consecutive components of one row: the softmax
// runs in fp32 in the lane and across the four lane groups, and rows are stored 16 bytes per lane.
template <int KT, int SMAX, int G>
__global__ void __launch_bounds__(256) bwd_gamma_split_kernel(const uint16_t* x, const bf16x8* fr, const double* cq,
                                                              float* gamma, int64_t N, int H, int K, int d_r,
                                                              int rows) {
    __shared__ bf16x8 s_f[SMAX * KT * 4 * 64];
    const int S = d_r / 32;
    const int64_t blocks = (N + rows - 1) / rows;
    const int64_t bh = (int64_t)blockIdx.x / blocks;
    const int h = (int)(bh % H);
    const int64_t r0 = ((int64_t)blockIdx.x % blocks) * rows;
    const int64_t r1 = r0 + rows < N ? r0 + rows : N;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const bf16x8* fh = fr + (int64_t)h * S * KT * 4 * 64;
    {
        // the head's fragments into LDS, every load of a thread issued before the first store (one load
        // in flight at a time cost about 15 us per workgroup); S * KT of the SMAX * KT slots are used
        constexpr int NMAX = SMAX * KT;
        const int n = S * KT;
        bf16x8 tmp[NMAX];
#pragma unroll
        for (int j = 0; j < NMAX; ++j)
            if (j < n) tmp[j] = fh[tid + 256 * j];
#pragma unroll
        for (int j = 0; j < NMAX; ++j)
            if (j < n) s_f[tid + 256 * j] = tmp[j];
    }
    // constants of the components this lane's accumulator rows hold: 16 kt + 4 g + i
    float cr[KT][4];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) cr[kt][i] = (float)cq[(int64_t)h * 16 * KT + 16 * kt + 4 * g + i];
    __syncthreads();
    const uint16_t* xh = x + bh * N * d_r;
    float* gh = gamma + bh * N * K;
    // wave w takes the G 16-row groups w, w + 4, .. of each block of 64 G rows (lane (r, g): row r of a
    // group, dims 8 g .. 8 g + 7 of a step): every fragment read from LDS serves G groups
    auto load = [&](int64_t rb, u32x4 (&xr)[G][SMAX]) {
#pragma unroll
        for (int gg = 0; gg < G; ++gg) {
            const int64_t row = rb + 64 * gg + r;
#pragma unroll
            for (int st = 0; st < SMAX; ++st)
                xr[gg][st] = (st < S && row < r1) ? *reinterpret_cast<const u32x4*>(xh + row * d_r + 32 * st + 8 * g)
                                                  : u32x4{0u, 0u, 0u, 0u};
        }
    };
    u32x4 xn[G][SMAX];
    load(r0 + 16 * w, xn);
    for (int64_t rb = r0 + 16 * w; rb < r1; rb += 64 * G) {
        u32x4 xr[G][SMAX];
#pragma unroll
        for (int gg = 0; gg < G; ++gg)
#pragma unroll
            for (int st = 0; st < SMAX; ++st) xr[gg][st] = xn[gg][st];
        if (rb + 64 * G < r1) load(rb + 64 * G, xn);
        f32x4 acc[G][KT];
#pragma unroll
        for (int gg = 0; gg < G; ++gg)
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) acc[gg][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < SMAX; ++st) {
            if (st >= S) break;
            bf16x8 xa[G], qh[G], ql[G];
#pragma unroll
            for (int gg = 0; gg < G; ++gg) {
                xa[gg] = __builtin_bit_cast(bf16x8, xr[gg][st]);
                float sq[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float v = (float)xa[gg][e];
                    sq[e] = v * v;
                }
                split_bf16x8(sq, qh[gg], ql[gg]);
            }
            // transposed product (coefficients as A, the rows as B): acc[gg][kt] rows = components
            // 16 kt + 4 g + i, column = row rb + 64 gg + r
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
                const bf16x8* fb = s_f + (st * KT + kt) * 4 * 64 + lane;
                const bf16x8 ahi = fb[0], alo = fb[64], bhi = fb[128], blo = fb[192];
#pragma unroll
                for (int gg = 0; gg < G; ++gg) {
                    mma(acc[gg][kt], blo, xa[gg]);
                    mma(acc[gg][kt], bhi, xa[gg]);
                    mma(acc[gg][kt], ahi, ql[gg]);
                    mma(acc[gg][kt], alo, qh[gg]);
                    mma(acc[gg][kt], ahi, qh[gg]);
                }
            }
        }
        // row rb + 64 gg + r: softmax over its components (in the lane's registers, then across the four lane
        // groups), stored as 16-byte runs of four components
        constexpr float kLog2e = 1.4426950408889634f;
#pragma unroll
        for (int gg = 0; gg < G; ++gg) {
            float mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[gg][kt][i] += cr[kt][i];
                    mx = fmaxf(mx, acc[gg][kt][i]);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            // e^(l - max) as 2^((l - max) log2 e) on the hardware exp2 (about one ulp)
            float sm = 0.f;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[gg][kt][i] = __builtin_amdgcn_exp2f((acc[gg][kt][i] - mx) * kLog2e);
                    sm += acc[gg][kt][i];
                }
            sm += __shfl_xor(sm, 16, 64);
            sm += __shfl_xor(sm, 32, 64);
            const float inv = 1.f / sm;
            const int64_t row = rb + 64 * gg + r;
            if (row < r1) {
                float* grow = gh + row * K;
#pragma unroll
                for (int kt = 0; kt < KT; ++kt) {
                    const int k0 = 16 * kt + 4 * g;
                    if (k0 + 4 <= K && K % 4 == 0) {
                        *reinterpret_cast<f32x4*>(grow + k0) = acc[gg][kt] * inv;
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (k0 + i < K) grow[k0 + i] = acc[gg][kt][i] * inv;
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------------- rows
// One wavefront per group of consecutive rows (a million single-row waves of the short [g | h] rows
// per launch are bound by wave launch, not by memory): each row's loads are issued for the whole group
// first, then its sums; within a row lane l holds columns l, l + 64, ... and the per-row order of
// every sum is that of a one-row-per-wave kernel.
constexpr int kRowsPerWave = 4;

template <bool F32>
__global__ void __launch_bounds__(256) bwd_gh_kernel(const float* p, const void* dout, float* rs, int64_t rows, int d_v,
                                                     int dva, float eps) {
    const int lane = threadIdx.x & 63;
    const int64_t r0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * kRowsPerWave;
    if (r0 >= rows) return;
    if (d_v <= 128) {
        float den[kRowsPerWave], pv[kRowsPerWave][2], dv[kRowsPerWave][2];
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i) {
            const int64_t rr = r0 + i < rows ? r0 + i : rows - 1;   // clamped: results of rows past the end are dropped
            const float* pr = p + rr * dva;
            den[i] = pr[d_v];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int c = lane + 64 * j;
                pv[i][j] = c < d_v ? pr[c] : 0.f;
                dv[i][j] = c < d_v ? ld_elem<F32>(dout, rr * d_v + c) : 0.f;
            }
        }
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i) {
            const float inv = 1.f / (den[i] + eps);
            float dot = 0.f;
#pragma unroll
            for (int j = 0; j < 2; ++j)
                if (lane + 64 * j < d_v) dot += dv[i][j] * (pv[i][j] * inv);
            dot = wave_sum_f(dot);
            if (lane == 0 && r0 + i < rows) {
                rs[2 * (r0 + i)] = inv;
                rs[2 * (r0 + i) + 1] = -dot * inv;
            }
        }
        return;
    }
    for (int i = 0; i < kRowsPerWave && r0 + i < rows; ++i) {
        const int64_t rr = r0 + i;
        const float* pr = p + rr * dva;
        const float inv = 1.f / (pr[d_v] + eps);
        float dot = 0.f;
        for (int c = lane; c < d_v; c += 64) dot += ld_elem<F32>(dout, rr * d_v + c) * (pr[c] * inv);
        dot = wave_sum_f(dot);
        if (lane == 0) {
            rs[2 * rr] = inv;
            rs[2 * rr + 1] = -dot * inv;
        }
    }
}

// dl = gamma * (dg - <gamma, dg>) per row.  Rows of up to 256 entries stay in registers between the
// dot product and the update (element k on lane k % 64, slot k / 64); longer rows are read twice.
// Rows per wave R: 4 for short rows (K <= 64); rows of K > 64 already stream near the HBM rate at one
// row per wave and measured slower with four (271 -> 293 us at B1 H16 N65536 K128).
template <int R>
__global__ void __launch_bounds__(256) bwd_dl_kernel(const float* gamma, float* dg, int64_t rows, int K) {
    const int lane = threadIdx.x & 63;
    const int64_t r0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * R;
    if (r0 >= rows) return;
    if (K <= 256) {
        float g[R][4], d[R][4];
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int64_t rr = r0 + i < rows ? r0 + i : rows - 1;   // clamped: rows past the end are not written
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int k = lane + 64 * j;
                g[i][j] = k < K ? gamma[rr * K + k] : 0.f;
                d[i][j] = k < K ? dg[rr * K + k] : 0.f;
            }
        }
#pragma unroll
        for (int i = 0; i < R; ++i) {
            float dot = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (lane + 64 * j < K) dot += g[i][j] * d[i][j];
            dot = wave_sum_f(dot);
            if (r0 + i < rows) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int k = lane + 64 * j;
                    if (k < K) dg[(r0 + i) * K + k] = g[i][j] * (d[i][j] - dot);
                }
            }
        }
        return;
    }
    for (int i = 0; i < R && r0 + i < rows; ++i) {
        const float* gr = gamma + (r0 + i) * K;
        float* dr = dg + (r0 + i) * K;
        float dot = 0.f;
        for (int k = lane; k < K; k += 64) dot += gr[k] * dr[k];
        dot = wave_sum_f(dot);
        for (int k = lane; k < K; k += 64) dr[k] = gr[k] * (dr[k] - dot);
    }
}

// ---------------------------------------------------------------------------------- fused rows
// One side's posterior gradient, routing-input gradient and parameter partials in one pass (bf16
// storage, K = d_r = 128), instead of the dl row kernel and the two products that read dl:
//   dl = gamma (dgamma - gamma . dgamma)      per row, fp32
//   dx = dl [mu / s] - x (dl [1 / s])         v_mfma_f32_16x16x32_bf16
//   P += dl^T [x | x^2 | 1]                   the same matrix cores, summed over the segment
// Workgroup: four wavefronts over one (batch, head) and a segment of `seg` tokens (a multiple of 64),
// in chunks of 64 tokens.  gamma and dgamma rows arrive by LDS DMA; wave w forms dl of rows 16 w ..
// 16 w + 15 and leaves it in LDS as two bf16 images, hi and lo = the rounded remainder (about 16
// significant bits); x arrives by LDS DMA as an image as well.  Wave w then owns dims 32 w .. 32 w + 31
// of both products: the dx columns mu / s and 1 / s of those dims (their B fragments, split into hi
// and lo once, stay in registers), and the P columns x and x^2 of those dims for every component
// (accumulated in registers over the segment; the ones column for components 32 w .. 32 w + 31).
// Where both operands are fp32 values the product is hi hi + hi lo + lo hi; against the exact bf16 x
// and the ones column it is hi + lo.  dl never reaches HBM.
namespace {

// Byte offset of 16-byte chunk c of row `row` in a 64 x 256-byte LDS image: chunks are XOR-swizzled by
// the row's low four bits (written r2 r1 r0 r3), so that both read patterns are conflict-free: 16 rows
// of one chunk (row fragments) and 8 consecutive rows of one chunk pair (transposed fragments).
__device__ __forceinline__ int img_chunk(int row, int c) {
    const int f = ((row & 7) << 1) | ((row >> 3) & 1);
    return row * 256 + ((c ^ f) << 4);
}

// Operand fragments from the images, for v_mfma_f32_16x16x32_bf16.  Row fragment: lane (r, g) takes row
// row0 + r, columns 32 ks + 8 g .. + 7 (one 16-byte read).  Permuted row fragment: the same row,
// columns 32 ks + 4 g .. + 3 and 32 ks + 16 + 4 g .. + 3 (two 8-byte reads).  Transposed fragment
// (ds_read_b64_tr_b16): lane (r, g) takes column 16 ct + r, rows 32 tk + 4 g .. + 3 and 32 tk + 16 + 4 g
// .. + 3.  A product pairs row fragments with row fragments or register fragments of the same column
// order, and permuted or transposed fragments with each other.
__device__ __forceinline__ bf16x8 img_row(const lds_char* img, int row, int ks, int g) {
    return lds_ld<bf16x8>(img + img_chunk(row, 4 * ks + g));
}
__device__ __forceinline__ int img_slot(int row, int slot) { return img_chunk(row, slot >> 1) + ((slot & 1) << 3); }
__device__ __forceinline__ bf16x8 img_row_perm(const lds_char* img, int row, int ks, int g) {
    const u32x2 lo = lds_ld<u32x2>(img + img_slot(row, 8 * ks + g));
    const u32x2 hi = lds_ld<u32x2>(img + img_slot(row, 8 * ks + 4 + g));
    return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}
__device__ __forceinline__ bf16x8 img_tr(const lds_char* img, int ct, int tk, int lane) {
    const int q = lane & 3, i4 = (lane >> 2) & 3, g = lane >> 4;
    u32x2 part[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) part[hf] = ds_read_tr16_at(img + img_slot((2 * tk + hf) * 16 + g * 4 + i4, 4 * ct + q));
    return __builtin_bit_cast(bf16x8, u32x4{part[0][0], part[0][1], part[1][0], part[1][1]});
}
// One element (2 bytes) of an image.
__device__ __forceinline__ int img_elem(int row, int col) { return img_chunk(row, col >> 3) + (col & 7) * 2; }

__device__ __forceinline__ void split4(const f32x4& v, bf16x4& hi, bf16x4& lo) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        hi[e] = (__bf16)v[e];
        lo[e] = (__bf16)(v[e] - (float)hi[e]);
    }
}

}  // namespace

constexpr int kFusedChunk = 64;

// DL_IN: `dgamma` already holds dl (the fused chunk kernels formed it) and `gamma` is not read.
template <int KC, int DRC, bool DL_IN>
__global__ void __launch_bounds__(256) bwd_fused_rows_kernel(const float* gamma, const float* dgamma, const void* x,
                                                             const float* mw, void* dx, float* gp, int64_t N, int H,
                                                             int seg, int64_t n_seg, int dxa) {
    static_assert(KC == 128 && DRC == 128, "one 256-byte image row per token");
    constexpr int C = kFusedChunk;
    constexpr int ROWB = KC * 4;           // bytes per fp32 row of gamma
    constexpr int STG = C * ROWB;          // one staged array of the chunk
    constexpr int IMG = C * 256;           // one bf16 image of the chunk
    constexpr int NCT = KC / 16;           // component tiles
    constexpr int NST = 4 * 2;             // dx stores per wave and chunk
    __shared__ __attribute__((aligned(16))) char s_stage[(DL_IN ? 1 : 2) * STG];   // gamma, dgamma (or dl) rows
    __shared__ __attribute__((aligned(16))) char s_dl[2 * IMG];      // dl hi, dl lo
    __shared__ __attribute__((aligned(16))) char s_x[2 * IMG];       // x rows, two chunks
    lds_char* const LS = (lds_char*)s_stage;
    lds_char* const LDH = (lds_char*)s_dl;
    lds_char* const LDL = LDH + IMG;
    lds_char* const LX = (lds_char*)s_x;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int64_t bh = blockIdx.x / n_seg;
    const int64_t sg = blockIdx.x % n_seg;
    const int h = (int)(bh % H);
    const int64_t t0 = sg * seg;
    const int64_t t1 = t0 + seg < N ? t0 + seg : N;
    const int nch = (int)((t1 - t0 + C - 1) / C);

    // buffer descriptors over this (batch, head): rows past N read as zero, their stores are dropped
    // the first staged array: gamma, or dl with DL_IN; the second: dgamma
    const i32x4 rs_g = uniform_rsrc(make_rsrc_words((DL_IN ? dgamma : gamma) + bh * N * KC, (uint32_t)(N * ROWB)));
    const i32x4 rs_d = uniform_rsrc(make_rsrc_words(dgamma + bh * N * KC, (uint32_t)(N * ROWB)));
    const i32x4 rs_x =
        uniform_rsrc(make_rsrc_words(reinterpret_cast<const uint16_t*>(x) + bh * N * DRC, (uint32_t)(N * DRC * 2)));
    const __amdgpu_buffer_rsrc_t rs_o =
        make_rsrc(reinterpret_cast<uint16_t*>(dx) + bh * N * DRC, (uint32_t)(N * DRC * 2));
    const uint32_t ls_base = lds_addr(LS), lx_base = lds_addr(LX);

    // DMA of the chunk at token n0: wave w's 16 rows of gamma and of dgamma (blocks of two rows: lane l
    // takes row l / 32, floats 4 (l % 32) .. + 3) and 16 rows of x (blocks of four rows: lane l takes
    // row l / 16 and the global chunk that the image keeps at chunk l % 16)
    auto issue = [&](int64_t n0, int xbuf) {
        const uint32_t v0 = (uint32_t)(((n0 + 16 * w + (lane >> 5)) * KC + 4 * (lane & 31)) * 4);
        const uint32_t m0 = ls_base + (uint32_t)(16 * w * ROWB);
#pragma unroll
        for (int b = 0; b < 8; b += 4) {
            dma16x4(rs_g, m0 + b * 1024, m0 + (b + 1) * 1024, m0 + (b + 2) * 1024, m0 + (b + 3) * 1024, v0 + b * 1024,
                    v0 + (b + 1) * 1024, v0 + (b + 2) * 1024, v0 + (b + 3) * 1024);
            if constexpr (!DL_IN)
                dma16x4(rs_d, m0 + STG + b * 1024, m0 + STG + (b + 1) * 1024, m0 + STG + (b + 2) * 1024,
                        m0 + STG + (b + 3) * 1024, v0 + b * 1024, v0 + (b + 1) * 1024, v0 + (b + 2) * 1024,
                        v0 + (b + 3) * 1024);
        }
        uint32_t xv[4];
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            const int row = 16 * w + 4 * bb + (lane >> 4);
            const int gc = (lane & 15) ^ (((row & 7) << 1) | ((row >> 3) & 1));
            xv[bb] = (uint32_t)((n0 + row) * DRC * 2 + gc * 16);
        }
        const uint32_t mx = lx_base + (uint32_t)(xbuf * IMG + 16 * w * 256);
        dma16x4(rs_x, mx, mx + 1024, mx + 2048, mx + 3072, xv[0], xv[1], xv[2], xv[3]);
    };

    // transposed fragment: lane (r, g) gets column 16 ct + r of the image for tokens 32 tk + 4 g + i and
    // 32 tk + 16 + 4 g + i (i = 0..3), the contraction order of both operands of P
    auto tr_frag = [&](const lds_char* img, int ct, int tk) -> bf16x8 {
        const int q = lane & 3, i4 = (lane >> 2) & 3;
        u32x2 part[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int row = (2 * tk + hf) * 16 + g * 4 + i4;
            const int slot = 4 * ct + q;
            part[hf] = ds_read_tr16_at(img + img_chunk(row, slot >> 1) + ((slot & 1) << 3));
        }
        return __builtin_bit_cast(bf16x8, u32x4{part[0][0], part[0][1], part[1][0], part[1][1]});
    };

    // B fragments of dx: column tile j (0, 1: mu / s of dims 32 w + 16 j + r; 2, 3: 1 / s of dims
    // 32 w + 16 (j - 2) + r), inner step ks: components 32 ks + 8 g .. + 7 (mw interleaves mu / s and 1 / s)
    bf16x8 wh[4][4], wl[4][4];
    {
        const float* mwh = mw + (int64_t)h * KC * 2 * DRC;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int d = 32 * w + 16 * (j & 1) + r;
                float v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = mwh[(int64_t)(32 * ks + 8 * g + e) * 2 * DRC + 2 * d + (j >> 1)];
                split_bf16x8(v, wh[j][ks], wl[j][ks]);
            }
    }
    // P of the segment: px / p2 [ct][jj] = components 16 ct + 4 g + i, columns x / x^2 of dim
    // 16 (2 w + jj) + r; po[hh] = components 16 (2 w + hh) + 4 g + i, the ones column (column r = 0)
    f32x4 px[NCT][2], p2[NCT][2], po[2];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            px[ct][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
            p2[ct][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    po[0] = po[1] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 ones0;
    {
        const __bf16 o = (__bf16)(r == 0 ? 1.f : 0.f);
        ones0 = bf16x8{o, o, o, o, o, o, o, o};
    }

    if (nch > 0) issue(t0, 0);
    for (int c = 0; c < nch; ++c) {
        const int64_t n0 = t0 + (int64_t)c * C;
        const int xbuf = c & 1;
        // B0: this chunk's rows landed (after them only the previous chunk's dx stores were issued);
        // every wave is done with the previous chunk's images
        if (c == 0) wait_vmcnt<0>();
        else wait_vmcnt<NST>();
        block_barrier();
        {
            // dl of rows 16 w + 2 j + l / 32: lane l holds components 4 (l % 32) .. + 3
            const lds_char* gs = LS + 16 * w * ROWB;
            const int rl = lane >> 5, cl = lane & 31;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int rr = 2 * j + rl;
                const f32x4 gv = lds_ld<f32x4>(gs + rr * ROWB + cl * 16);
                f32x4 dl;
                if constexpr (DL_IN) {
                    dl = gv;
                } else {
                    const f32x4 dv = lds_ld<f32x4>(gs + STG + rr * ROWB + cl * 16);
                    float dot = gv[0] * dv[0] + gv[1] * dv[1] + gv[2] * dv[2] + gv[3] * dv[3];
#pragma unroll
                    for (int o = 1; o < 32; o <<= 1) dot += __shfl_xor(dot, o, 64);
                    dl = gv * (dv - dot);
                }
                bf16x4 hi, lo;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    hi[e] = (__bf16)dl[e];
                    lo[e] = (__bf16)(dl[e] - (float)hi[e]);
                }
                const int off = img_chunk(16 * w + rr, cl >> 1) + ((cl & 1) << 3);
                lds_st<bf16x4>(LDH + off, hi);
                lds_st<bf16x4>(LDL + off, lo);
            }
        }
        lds_barrier();   // B1: the dl images are complete and the staged rows consumed
        if (c + 1 < nch) issue(n0 + C, xbuf ^ 1);
        const lds_char* xi = LX + xbuf * IMG;
        {
            // P += dl^T [x | x^2 | 1]
            bf16x8 xf[2][2], xh[2][2], xl[2][2];
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                for (int tk = 0; tk < 2; ++tk) {
                    xf[jj][tk] = tr_frag(xi, 2 * w + jj, tk);
                    float sq[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) sq[e] = (float)xf[jj][tk][e] * (float)xf[jj][tk][e];
                    split_bf16x8(sq, xh[jj][tk], xl[jj][tk]);
                }
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int tk = 0; tk < 2; ++tk) {
                    const bf16x8 ah = tr_frag(LDH, ct, tk), al = tr_frag(LDL, ct, tk);
#pragma unroll
                    for (int jj = 0; jj < 2; ++jj) {
                        mma(px[ct][jj], al, xf[jj][tk]);
                        mma(px[ct][jj], ah, xf[jj][tk]);
                        mma(p2[ct][jj], al, xh[jj][tk]);
                        mma(p2[ct][jj], ah, xl[jj][tk]);
                        mma(p2[ct][jj], ah, xh[jj][tk]);
                    }
                    if ((ct >> 1) == w) {
                        mma(po[ct & 1], al, ones0);
                        mma(po[ct & 1], ah, ones0);
                    }
                }
        }
        {
            // dx of dims 32 w .. + 31, formed transposed (the B fragments of mu / s, 1 / s as A, dl as B):
            // acc[tt][j] rows = the dims of tile j (32 w + 16 (j % 2) + 4 g + i), column = token 16 tt + r
            f32x4 acc[4][4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[tt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                bf16x8 ah[4], al[4];
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    const int off = img_chunk(16 * tt + r, 4 * ks + g);
                    ah[tt] = lds_ld<bf16x8>(LDH + off);
                    al[tt] = lds_ld<bf16x8>(LDL + off);
                }
#pragma unroll
                for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        mma(acc[tt][j], wh[j][ks], al[tt]);
                        mma(acc[tt][j], wl[j][ks], ah[tt]);
                        mma(acc[tt][j], wh[j][ks], ah[tt]);
                    }
            }
            // lane (r, g): token 16 tt + r, dims d0 .. d0 + 3, 8 bytes per store
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    const int t = 16 * tt + r, d0 = 32 * w + 16 * jj + 4 * g;
                    const bf16x4 xv = __builtin_bit_cast(bf16x4, lds_ld<u32x2>(xi + img_slot(t, d0 >> 2)));
                    f32x4 val;
#pragma unroll
                    for (int i = 0; i < 4; ++i) val[i] = acc[tt][jj][i] - (float)xv[i] * acc[tt][jj + 2][i];
                    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, pack4(val)), rs_o,
                                                          (uint32_t)(((n0 + t) * DRC + d0) * 2), 0, 0);
                }
        }
    }

    // the segment's partial: gp [bh][sg][K][dxa], columns x | x^2 | 1 (dxa >= 2 d_r + 1)
    float* gpo = gp + (bh * n_seg + sg) * (int64_t)KC * dxa;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int k = 16 * ct + 4 * g + i, d = 16 * (2 * w + jj) + r;
                gpo[k * dxa + d] = px[ct][jj][i];
                gpo[k * dxa + DRC + d] = p2[ct][jj][i];
            }
    if (r == 0) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int i = 0; i < 4; ++i) gpo[(16 * (2 * w + hh) + 4 * g + i) * dxa + 2 * DRC] = po[hh][i];
    }
}

// ---------------------------------------------------------------------------------- fused rows, small classes
// The same three results for bf16 storage at K <= 64 and d_r <= 128 (K and d_r multiples of 4; padded to
// KC in {32, 64} and DRC in {64, 128}): dl, then dx = dl [mu / s] - x (dl [1 / s]) and P += dl^T [x | x^2],
// the sums of dl over tokens (the ones column) in fp32 on the vector units.  Workgroup: four wavefronts
// over one (batch, head) and a segment of `seg` tokens, in chunks of 64; wave w loads rows 16 w .. 16 w +
// 15 of each chunk into registers (lane (r, g): row r, components 32 ks + 8 g .. + 7 of gamma and dgamma,
// dims 16 j + 4 g .. + 3 of x), the next chunk's as soon as the current one's dl is formed.  dl stays in
// registers as the B fragments of dx (split bf16 hi + lo, formed transposed: lane (r, g) then holds dx of
// row r, dims 16 j + 4 g .. + 3); for P the chunk's dl and x go to LDS component- and dim-major (rows of
// 64 tokens padded to 144 bytes, so a fragment's 16 rows fall in disjoint banks) and each wave takes a
// quarter of the (component tile, dim tile) pairs over all 64 tokens.  The head's mu / s and 1 / s sit in
// LDS as split bf16 images for the whole segment.  Loads and stores go through buffer descriptors
// (rows past N, components past K and dims past d_r read as zero and are not written); their waits are
// placed by the compiler.  DL_IN: `dgamma` already holds dl and `gamma` is not read.
template <int KC, int DRC, bool DL_IN>
__global__ void __launch_bounds__(256) bwd_rows_small_kernel(const float* gamma, const float* dgamma, const void* x,
                                                             const float* mw, void* dx, float* gp, int64_t N, int H,
                                                             int K, int d_r, int seg, int64_t n_seg, int dxa) {
    static_assert(KC == 32 || KC == 64, "component padding");
    static_assert(DRC == 64 || DRC == 128, "dim padding");
    constexpr int C = kFusedChunk;
    constexpr int NKS = KC / 32;            // 32-component steps of dx's contraction
    constexpr int NDT = DRC / 16;           // dim tiles
    constexpr int NCT = KC / 16;            // component tiles
    constexpr int UPW = NCT * NDT / 4;      // (component tile, dim tile) pairs per wave
    constexpr int IS = 2 * C + 16;          // image row: 64 tokens of bf16 plus padding
    constexpr int WS = 2 * KC + 16;         // mu / s and 1 / s image row: KC components of bf16 plus padding
    __shared__ __attribute__((aligned(16))) char s_dl[2 * KC * IS];     // dl hi, dl lo: [component][token]
    __shared__ __attribute__((aligned(16))) char s_x[DRC * IS];         // x: [dim][token]
    __shared__ __attribute__((aligned(16))) char s_w[2 * 2 * DRC * WS]; // hi, lo: [part * DRC + dim][component]
    __shared__ float s_one[4][KC];
    lds_char* const LDH = (lds_char*)s_dl;
    lds_char* const LDL = LDH + KC * IS;
    lds_char* const LX = (lds_char*)s_x;
    lds_char* const LWH = (lds_char*)s_w;
    lds_char* const LWL = LWH + 2 * DRC * WS;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int64_t bh = blockIdx.x / n_seg;
    const int64_t sg = blockIdx.x % n_seg;
    const int h = (int)(bh % H);
    const int64_t t0 = sg * seg;
    const int64_t t1 = t0 + seg < N ? t0 + seg : N;
    const int nch = (int)((t1 - t0 + C - 1) / C);

    // mu / s (part 0) and 1 / s (part 1) of the head, zero past K and d_r
    {
        const float* mwh = mw + (int64_t)h * K * 2 * d_r;
        for (int e = tid; e < 2 * DRC * KC; e += 256) {
            const int k = e % KC, row = e / KC, p = row / DRC, d = row % DRC;
            const float v = (k < K && d < d_r) ? mwh[(int64_t)k * 2 * d_r + 2 * d + p] : 0.f;
            const __bf16 hi = (__bf16)v;
            lds_st<__bf16>(LWH + row * WS + 2 * k, hi);
            lds_st<__bf16>(LWL + row * WS + 2 * k, (__bf16)(v - (float)hi));
        }
    }

    // descriptors over this (batch, head): rows past N load as zero and their stores are dropped, and so
    // are components past K and dims past d_r (offsets with bit 31 set)
    const __amdgpu_buffer_rsrc_t rs_g = make_rsrc(gamma + bh * N * K, (uint32_t)(N * K * 4));
    const __amdgpu_buffer_rsrc_t rs_d = make_rsrc(dgamma + bh * N * K, (uint32_t)(N * K * 4));
    const __amdgpu_buffer_rsrc_t rs_x =
        make_rsrc(reinterpret_cast<const uint16_t*>(x) + bh * N * d_r, (uint32_t)(N * d_r * 2));
    const __amdgpu_buffer_rsrc_t rs_o = make_rsrc(reinterpret_cast<uint16_t*>(dx) + bh * N * d_r, (uint32_t)(N * d_r * 2));
    constexpr uint32_t kOut = 0x80000000u;

    // this lane's row of the chunk at n0: gamma and dgamma components 32 ks + 8 g .. + 7, x dims 16 j + 4 g .. + 3
    f32x4 ga[NKS][2], da[NKS][2];
    u32x2 xa[NDT];
    auto load = [&](int64_t n0) {
        const uint32_t t = (uint32_t)(n0 + 16 * w + r);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int k = 32 * ks + 8 * g + 4 * hf;
                const uint32_t off = k < K ? (t * K + k) * 4 : kOut;
                if constexpr (!DL_IN)
                    ga[ks][hf] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs_g, off, 0, 0));
                da[ks][hf] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs_d, off, 0, 0));
            }
#pragma unroll
        for (int j = 0; j < NDT; ++j) {
            const int d = 16 * j + 4 * g;
            xa[j] = __builtin_amdgcn_raw_buffer_load_b64(rs_x, d < d_r ? (t * d_r + d) * 2 : kOut, 0, 0);
        }
    };

    f32x4 px[UPW], p2[UPW];
#pragma unroll
    for (int q = 0; q < UPW; ++q) px[q] = p2[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    float s1[NKS][8];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) s1[ks][e] = 0.f;

    if (nch > 0) load(t0);
    for (int c = 0; c < nch; ++c) {
        const int64_t n0 = t0 + (int64_t)c * C;
        // dl of this lane's row; hi + lo split as dx's B fragments
        bf16x8 bh8[NKS], bl8[NKS];
        {
            float dot = 0.f;
            if constexpr (!DL_IN) {
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                        for (int e = 0; e < 4; ++e) dot += ga[ks][hf][e] * da[ks][hf][e];
                dot += __shfl_xor(dot, 16, 64);
                dot += __shfl_xor(dot, 32, 64);
            }
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                float v[8];
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        v[4 * hf + e] = DL_IN ? da[ks][hf][e] : ga[ks][hf][e] * (da[ks][hf][e] - dot);
#pragma unroll
                for (int e = 0; e < 8; ++e) s1[ks][e] += v[e];
                split_bf16x8(v, bh8[ks], bl8[ks]);
            }
        }
        u32x2 xcur[NDT];
#pragma unroll
        for (int j = 0; j < NDT; ++j) xcur[j] = xa[j];
        if (c + 1 < nch) load(n0 + C);
        // every wave is done with the previous chunk's images
        lds_barrier();
        {
            const int t = 16 * w + r;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int k = 32 * ks + 8 * g + e;
                    lds_st<__bf16>(LDH + k * IS + 2 * t, bh8[ks][e]);
                    lds_st<__bf16>(LDL + k * IS + 2 * t, bl8[ks][e]);
                }
#pragma unroll
            for (int j = 0; j < NDT; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int d = 16 * j + 4 * g + i;
                    const uint16_t xv = (uint16_t)(xcur[j][i >> 1] >> (16 * (i & 1)));
                    lds_st<uint16_t>(LX + d * IS + 2 * t, xv);
                }
        }
        lds_barrier();   // the chunk's images are complete
        // P += dl^T [x | x^2] for this wave's pairs over the chunk's 64 tokens
#pragma unroll
        for (int q = 0; q < UPW; ++q) {
            const int u = w + 4 * q, ct = u % NCT, dt = u / NCT;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                const int off = (32 * kt + 8 * g) * 2;
                const bf16x8 ah = lds_ld<bf16x8>(LDH + (16 * ct + r) * IS + off);
                const bf16x8 al = lds_ld<bf16x8>(LDL + (16 * ct + r) * IS + off);
                const bf16x8 xf = lds_ld<bf16x8>(LX + (16 * dt + r) * IS + off);
                float sq[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) sq[e] = (float)xf[e] * (float)xf[e];
                bf16x8 sh, sl;
                split_bf16x8(sq, sh, sl);
                mma(px[q], al, xf);
                mma(px[q], ah, xf);
                mma(p2[q], al, sh);
                mma(p2[q], ah, sl);
                mma(p2[q], ah, sh);
            }
        }
        // dx of this lane's row, dims 16 j + 4 g .. + 3
        {
            const uint32_t t = (uint32_t)(n0 + 16 * w + r);
#pragma unroll
            for (int j = 0; j < NDT; ++j) {
                f32x4 aa = f32x4{0.f, 0.f, 0.f, 0.f}, ab = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const int off = (32 * ks + 8 * g) * 2;
                    const bf16x8 wah = lds_ld<bf16x8>(LWH + (16 * j + r) * WS + off);
                    const bf16x8 wal = lds_ld<bf16x8>(LWL + (16 * j + r) * WS + off);
                    const bf16x8 wbh = lds_ld<bf16x8>(LWH + (DRC + 16 * j + r) * WS + off);
                    const bf16x8 wbl = lds_ld<bf16x8>(LWL + (DRC + 16 * j + r) * WS + off);
                    mma(aa, wah, bl8[ks]);
                    mma(aa, wal, bh8[ks]);
                    mma(aa, wah, bh8[ks]);
                    mma(ab, wbh, bl8[ks]);
                    mma(ab, wbl, bh8[ks]);
                    mma(ab, wbh, bh8[ks]);
                }
                const int d = 16 * j + 4 * g;
                f32x4 val;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float xv = __uint_as_float((xcur[j][i >> 1] >> (16 * (i & 1))) << 16);
                    val[i] = aa[i] - xv * ab[i];
                }
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, pack4(val)), rs_o,
                                                      d < d_r ? (t * d_r + d) * 2 : kOut, 0, 0);
            }
        }
    }

    // the segment's partial: gp [bh][sg][K][dxa], columns x | x^2 | 1
    float* gpo = gp + (bh * n_seg + sg) * (int64_t)K * dxa;
#pragma unroll
    for (int q = 0; q < UPW; ++q) {
        const int u = w + 4 * q, ct = u % NCT, dt = u / NCT;
        const int d = 16 * dt + r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = 16 * ct + 4 * g + i;
            if (k < K && d < d_r) {
                gpo[(int64_t)k * dxa + d] = px[q][i];
                gpo[(int64_t)k * dxa + d_r + d] = p2[q][i];
            }
        }
    }
    // ones column: sum over the 16 rows of each lane group, then over the waves in order
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float v = s1[ks][e];
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o, 64);
            if (r == 0) s_one[w][32 * ks + 8 * g + e] = v;
        }
    __syncthreads();
    if (tid < K) gpo[(int64_t)tid * dxa + 2 * d_r] = s_one[0][tid] + s_one[1][tid] + s_one[2][tid] + s_one[3][tid];
}

// ---------------------------------------------------------------------------------- bidirectional, small classes
// The bidirectional backward's products for bf16 storage at K <= 64 and d_v <= 128 (multiples of 4; padded
// to KC in {32, 64} and VC in {64, 128}), with the notation of the general path: the state
// S = Gamma_K^T [V | 1] (its last column Z), per row num = Gamma_Q S_v, den = Gamma_Q Z, inv = 1 / (den +
// eps), g = dO inv, h = -(dO . num) inv^2, then dGamma_Q = g S_v^T + h Z^T, R = Gamma_Q^T [g | h] summed
// over all rows, dGamma_K = V R_v^T + R_1^T and dV = Gamma_K R_v.  Three kernels over segments of `seg`
// tokens (a multiple of 64) of one (batch, head), four wavefronts in chunks of 64 tokens; wave w loads rows
// 16 w .. 16 w + 15 of each chunk (lane (r, g): row r, components 32 ks + 8 g .. + 7 of the Gamma rows,
// dims 16 j + 4 g .. + 3 of the bf16 rows), the next chunk's while the current one is in the products.
// Row-wise products are formed with that lane's registers as the B operand (Gamma split into bf16 hi + lo;
// dims in the permuted order 32 vs + 4 g .. + 3, 32 vs + 16 + 4 g .. + 3, the same order in both operands);
// sums over tokens go through LDS images, component- or dim-major with rows of 64 tokens.  S and R (one
// record per segment) are summed over the segments by the scan kernel (mode 2), in segment order; their
// last column is summed on the vector units in fp32.  Where both operands are fp32 values a product is
// hi hi + hi lo + lo hi, against exact bf16 values hi + lo.
namespace {

constexpr int kImgRow = 2 * 64 + 16;   // a 64-token bf16 image row plus padding (bytes)

// Element e of a lane's permuted 8-element group in step ks: 32 ks + 4 g + e for e < 4, then
// 32 ks + 16 + 4 g + e - 4 (the order of an accumulator tile pair's rows 16 ct + 4 g + i, ct = 2 ks, 2 ks + 1).
__device__ __forceinline__ int perm_comp(int ks, int g, int e) { return 32 * ks + 16 * (e >> 2) + 4 * g + (e & 3); }

// Permuted 8-element fragment of an LDS row of bf16 values: elements 32 vs + 4 g .. + 3 and
// 32 vs + 16 + 4 g .. + 3.
__device__ __forceinline__ bf16x8 row_perm(const lds_char* row, int vs, int g) {
    const u32x2 a = lds_ld<u32x2>(row + (32 * vs + 4 * g) * 2);
    const u32x2 b = lds_ld<u32x2>(row + (32 * vs + 16 + 4 * g) * 2);
    return __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], b[0], b[1]});
}

// A record [K][dva] (fp32) of this (batch, head) into split bf16 images, component-major [comp][dim]
// (rows of 2 VC + 16 bytes) and dim-major [dim][comp] (rows of 2 KC + 16 bytes), zero past K and d_v;
// its column d_v into last[comp].
template <int KC, int VC>
__device__ __forceinline__ void stage_record(const float* rec, int K, int d_v, int dva, lds_char* ch, lds_char* cl,
                                             lds_char* dh, lds_char* dl, float* last) {
    constexpr int WC = 2 * VC + 16, WD = 2 * KC + 16;
    for (int e = threadIdx.x; e < KC * VC; e += 256) {
        const int k = e / VC, d = e % VC;
        const float v = (k < K && d < d_v) ? rec[(int64_t)k * dva + d] : 0.f;
        const __bf16 hi = (__bf16)v, lo = (__bf16)(v - (float)hi);
        lds_st<__bf16>(ch + k * WC + 2 * d, hi);
        lds_st<__bf16>(cl + k * WC + 2 * d, lo);
        lds_st<__bf16>(dh + d * WD + 2 * k, hi);
        lds_st<__bf16>(dl + d * WD + 2 * k, lo);
    }
    for (int k = threadIdx.x; k < KC; k += 256) last[k] = k < K ? rec[(int64_t)k * dva + d_v] : 0.f;
}

// The record of a segment: the (component tile, dim tile) pairs of the wave (lane: components
// 16 ct + 4 g + i, dim 16 dt + r), the last column from each lane's per-row sums `z` (components
// 32 ks + 8 g + e) reduced over the rows and the waves in order, zeros after it.
template <int KC, int VC, int UPW, int NKS, bool PERM = false>
__device__ __forceinline__ void write_record(float* out, const f32x4 (&acc)[UPW], const float (&z)[NKS][8],
                                             float (*s_z)[KC], int K, int d_v, int dva) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int q = 0; q < UPW; ++q) {
        const int u = w + 4 * q, ct = u % (KC / 16), dt = u / (KC / 16);
        const int d = 16 * dt + r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = 16 * ct + 4 * g + i;
            if (k < K && d < d_v) out[(int64_t)k * dva + d] = acc[q][i];
        }
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float v = z[ks][e];
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o, 64);
            if (r == 0) s_z[w][PERM ? perm_comp(ks, g, e) : 32 * ks + 8 * g + e] = v;
        }
    __syncthreads();
    const int pad = dva - d_v;
    for (int e = threadIdx.x; e < K * pad; e += 256) {
        const int k = e / pad, c = e % pad;
        out[(int64_t)k * dva + d_v + c] = c == 0 ? s_z[0][k] + s_z[1][k] + s_z[2][k] + s_z[3][k] : 0.f;
    }
}

}  // namespace

// S per segment: st [BH][n_seg][K][dva].
template <int KC, int VC>
__global__ void __launch_bounds__(256) bwd_bidir_state_kernel(const float* gk, const void* v, float* st, int64_t N,
                                                              int K, int d_v, int dva, int seg, int64_t n_seg) {
    constexpr int C = kFusedChunk, NKS = KC / 32, NVT = VC / 16, NCT = KC / 16, UPW = NCT * NVT / 4;
    constexpr int IS = kImgRow;
    __shared__ __attribute__((aligned(16))) char s_g[2 * KC * IS];   // Gamma_K hi, lo: [comp][token]
    __shared__ __attribute__((aligned(16))) char s_v[VC * IS];       // V: [dim][token]
    __shared__ float s_z[4][KC];
    lds_char* const LGH = (lds_char*)s_g;
    lds_char* const LGL = LGH + KC * IS;
    lds_char* const LV = (lds_char*)s_v;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int64_t bh = blockIdx.x / n_seg, sg = blockIdx.x % n_seg;
    const int64_t t0 = sg * seg;
    const int64_t t1 = t0 + seg < N ? t0 + seg : N;
    const int nch = (int)((t1 - t0 + C - 1) / C);
    const __amdgpu_buffer_rsrc_t rs_g = make_rsrc(gk + bh * N * K, (uint32_t)(N * K * 4));
    const __amdgpu_buffer_rsrc_t rs_v =
        make_rsrc(reinterpret_cast<const uint16_t*>(v) + bh * N * d_v, (uint32_t)(N * d_v * 2));
    constexpr uint32_t kOut = 0x80000000u;

    f32x4 ga[NKS][2];
    u32x2 va[NVT];
    auto load = [&](int64_t n0) {
        const uint32_t t = (uint32_t)(n0 + 16 * w + r);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int k = 32 * ks + 8 * g + 4 * hf;
                ga[ks][hf] = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs_g, k < K ? (t * K + k) * 4 : kOut, 0, 0));
            }
#pragma unroll
        for (int j = 0; j < NVT; ++j) {
            const int d = 16 * j + 4 * g;
            va[j] = __builtin_amdgcn_raw_buffer_load_b64(rs_v, d < d_v ? (t * d_v + d) * 2 : kOut, 0, 0);
        }
    };

    f32x4 acc[UPW];
#pragma unroll
    for (int q = 0; q < UPW; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    float z[NKS][8];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) z[ks][e] = 0.f;

    if (nch > 0) load(t0);
    for (int c = 0; c < nch; ++c) {
        const int64_t n0 = t0 + (int64_t)c * C;
        bf16x8 gh8[NKS], gl8[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            float gv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                gv[e] = ga[ks][e >> 2][e & 3];
                z[ks][e] += gv[e];
            }
            split_bf16x8(gv, gh8[ks], gl8[ks]);
        }
        u32x2 vcur[NVT];
#pragma unroll
        for (int j = 0; j < NVT; ++j) vcur[j] = va[j];
        if (c + 1 < nch) load(n0 + C);
        lds_barrier();   // every wave is done with the previous chunk's images
        {
            const int t = 16 * w + r;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int k = 32 * ks + 8 * g + e;
                    lds_st<__bf16>(LGH + k * IS + 2 * t, gh8[ks][e]);
                    lds_st<__bf16>(LGL + k * IS + 2 * t, gl8[ks][e]);
                }
#pragma unroll
            for (int j = 0; j < NVT; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    lds_st<uint16_t>(LV + (16 * j + 4 * g + i) * IS + 2 * t,
                                     (uint16_t)(vcur[j][i >> 1] >> (16 * (i & 1))));
        }
        lds_barrier();   // the chunk's images are complete
#pragma unroll
        for (int q = 0; q < UPW; ++q) {
            const int u = w + 4 * q, ct = u % NCT, dt = u / NCT;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                const int off = (32 * kt + 8 * g) * 2;
                const bf16x8 ah = lds_ld<bf16x8>(LGH + (16 * ct + r) * IS + off);
                const bf16x8 al = lds_ld<bf16x8>(LGL + (16 * ct + r) * IS + off);
                const bf16x8 vf = lds_ld<bf16x8>(LV + (16 * dt + r) * IS + off);
                mma(acc[q], al, vf);
                mma(acc[q], ah, vf);
            }
        }
    }
    write_record<KC, VC, UPW, NKS>(st + (bh * n_seg + sg) * (int64_t)K * dva, acc, z, s_z, K, d_v, dva);
}

// Query side: dGamma_Q [BH][N][K] (EMIT_DL: dl = Gamma_Q (dGamma_Q - Gamma_Q . dGamma_Q) in its place) and
// the segments' R records r_seg [BH][n_seg][K][dva], from the summed state (entry 0 of st [BH][n_seg][K][dva]).
// Gamma_Q is loaded in the permuted component order (perm_comp), which is the order of dGamma_Q's
// accumulator rows, so that dl is formed in registers.
template <int KC, int VC, bool EMIT_DL>
__global__ void __launch_bounds__(256) bwd_bidir_q_kernel(const float* gq, const void* dout, const float* st,
                                                          float* dgq, float* r_seg, int64_t N, int K, int d_v,
                                                          int dva, int seg, int64_t n_seg, float eps) {
    constexpr int C = kFusedChunk, NKS = KC / 32, NVT = VC / 16, NVS = VC / 32, NCT = KC / 16;
    constexpr int UPW = NCT * NVT / 4, IS = kImgRow, WC = 2 * VC + 16, WD = 2 * KC + 16;
    __shared__ __attribute__((aligned(16))) char s_sc[2 * KC * WC];   // S_v hi, lo: [comp][dim]
    __shared__ __attribute__((aligned(16))) char s_sd[2 * VC * WD];   // S_v^T hi, lo: [dim][comp]
    __shared__ __attribute__((aligned(16))) char s_g[2 * KC * IS];    // Gamma_Q hi, lo: [comp][token]
    __shared__ __attribute__((aligned(16))) char s_x[2 * VC * IS];    // g hi, lo: [dim][token]
    __shared__ float s_zt[KC];
    __shared__ float s_z[4][KC];
    lds_char* const SCH = (lds_char*)s_sc;
    lds_char* const SCL = SCH + KC * WC;
    lds_char* const SDH = (lds_char*)s_sd;
    lds_char* const SDL = SDH + VC * WD;
    lds_char* const LGH = (lds_char*)s_g;
    lds_char* const LGL = LGH + KC * IS;
    lds_char* const LXH = (lds_char*)s_x;
    lds_char* const LXL = LXH + VC * IS;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int64_t bh = blockIdx.x / n_seg, sg = blockIdx.x % n_seg;
    const int64_t t0 = sg * seg;
    const int64_t t1 = t0 + seg < N ? t0 + seg : N;
    const int nch = (int)((t1 - t0 + C - 1) / C);
    const __amdgpu_buffer_rsrc_t rs_g = make_rsrc(gq + bh * N * K, (uint32_t)(N * K * 4));
    const __amdgpu_buffer_rsrc_t rs_o = make_rsrc(dgq + bh * N * K, (uint32_t)(N * K * 4));
    const __amdgpu_buffer_rsrc_t rs_d =
        make_rsrc(reinterpret_cast<const uint16_t*>(dout) + bh * N * d_v, (uint32_t)(N * d_v * 2));
    constexpr uint32_t kOut = 0x80000000u;

    stage_record<KC, VC>(st + bh * n_seg * (int64_t)K * dva, K, d_v, dva, SCH, SCL, SDH, SDL, s_zt);

    f32x4 ga[NKS][2];
    u32x2 da[NVT];
    auto load = [&](int64_t n0) {
        const uint32_t t = (uint32_t)(n0 + 16 * w + r);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int k = 32 * ks + 16 * hf + 4 * g;
                ga[ks][hf] = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs_g, k < K ? (t * K + k) * 4 : kOut, 0, 0));
            }
#pragma unroll
        for (int j = 0; j < NVT; ++j) {
            const int d = 16 * j + 4 * g;
            da[j] = __builtin_amdgcn_raw_buffer_load_b64(rs_d, d < d_v ? (t * d_v + d) * 2 : kOut, 0, 0);
        }
    };

    f32x4 acc[UPW];
#pragma unroll
    for (int q = 0; q < UPW; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    float z[NKS][8];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) z[ks][e] = 0.f;

    if (nch > 0) load(t0);
    __syncthreads();   // the staged state
    for (int c = 0; c < nch; ++c) {
        const int64_t n0 = t0 + (int64_t)c * C;
        const uint32_t t = (uint32_t)(n0 + 16 * w + r);
        float gv[NKS][8];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) gv[ks][e] = ga[ks][e >> 2][e & 3];
        float dov[NVT][4];
#pragma unroll
        for (int j = 0; j < NVT; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) dov[j][i] = __uint_as_float((da[j][i >> 1] >> (16 * (i & 1))) << 16);
        if (c + 1 < nch) load(n0 + C);

        // den and num of this lane's row (num: dims 16 j + 4 g .. + 3)
        bf16x8 gh8[NKS], gl8[NKS];
        float den = 0.f;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
            for (int e = 0; e < 8; ++e) den += gv[ks][e] * s_zt[perm_comp(ks, g, e)];
            split_bf16x8(gv[ks], gh8[ks], gl8[ks]);
        }
        den += __shfl_xor(den, 16, 64);
        den += __shfl_xor(den, 32, 64);
        const float inv = t < (uint32_t)t1 ? 1.f / (den + eps) : 0.f;
        float dot = 0.f;
#pragma unroll
        for (int j = 0; j < NVT; ++j) {
            f32x4 nm = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const bf16x8 ah = row_perm(SDH + (16 * j + r) * WD, ks, g);
                const bf16x8 al = row_perm(SDL + (16 * j + r) * WD, ks, g);
                mma(nm, ah, gl8[ks]);
                mma(nm, al, gh8[ks]);
                mma(nm, ah, gh8[ks]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) dot += dov[j][i] * (nm[i] * inv);
        }
        dot += __shfl_xor(dot, 16, 64);
        dot += __shfl_xor(dot, 32, 64);
        const float hv = -dot * inv;
        // g in the permuted dim order, split
        bf16x8 xh8[NVS], xl8[NVS];
#pragma unroll
        for (int vs = 0; vs < NVS; ++vs) {
            float gg[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                gg[e] = dov[2 * vs][e] * inv;
                gg[4 + e] = dov[2 * vs + 1][e] * inv;
            }
            split_bf16x8(gg, xh8[vs], xl8[vs]);
        }
        // dGamma_Q of this lane's row, components 16 ct + 4 g .. + 3 (ct = 2 ks + e / 4: the lane's own order)
        f32x4 dgo[NCT];
        float dot2 = 0.f;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            f32x4 dg = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int vs = 0; vs < NVS; ++vs) {
                const bf16x8 ah = row_perm(SCH + (16 * ct + r) * WC, vs, g);
                const bf16x8 al = row_perm(SCL + (16 * ct + r) * WC, vs, g);
                mma(dg, ah, xl8[vs]);
                mma(dg, al, xh8[vs]);
                mma(dg, ah, xh8[vs]);
            }
            const int k = 16 * ct + 4 * g;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                dgo[ct][i] = dg[i] + hv * s_zt[k + i];
                dot2 += gv[ct >> 1][4 * (ct & 1) + i] * dgo[ct][i];
            }
        }
        if constexpr (EMIT_DL) {
            dot2 += __shfl_xor(dot2, 16, 64);
            dot2 += __shfl_xor(dot2, 32, 64);
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const int k = 16 * ct + 4 * g;
            f32x4 o = dgo[ct];
            if constexpr (EMIT_DL) {
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] = gv[ct >> 1][4 * (ct & 1) + i] * (dgo[ct][i] - dot2);
            }
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), rs_o, k < K ? (t * K + k) * 4 : kOut,
                                                   0, 0);
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) z[ks][e] += gv[ks][e] * hv;

        // R += Gamma_Q^T g over the chunk
        lds_barrier();   // every wave is done with the previous chunk's images
        {
            const int tt = 16 * w + r;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int k = perm_comp(ks, g, e);
                    lds_st<__bf16>(LGH + k * IS + 2 * tt, gh8[ks][e]);
                    lds_st<__bf16>(LGL + k * IS + 2 * tt, gl8[ks][e]);
                }
#pragma unroll
            for (int vs = 0; vs < NVS; ++vs)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int d = 32 * vs + (e < 4 ? 4 * g + e : 16 + 4 * g + e - 4);
                    lds_st<__bf16>(LXH + d * IS + 2 * tt, xh8[vs][e]);
                    lds_st<__bf16>(LXL + d * IS + 2 * tt, xl8[vs][e]);
                }
        }
        lds_barrier();   // the chunk's images are complete
#pragma unroll
        for (int q = 0; q < UPW; ++q) {
            const int u = w + 4 * q, ct = u % NCT, dt = u / NCT;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                const int off = (32 * kt + 8 * g) * 2;
                const bf16x8 ah = lds_ld<bf16x8>(LGH + (16 * ct + r) * IS + off);
                const bf16x8 al = lds_ld<bf16x8>(LGL + (16 * ct + r) * IS + off);
                const bf16x8 bh = lds_ld<bf16x8>(LXH + (16 * dt + r) * IS + off);
                const bf16x8 bl = lds_ld<bf16x8>(LXL + (16 * dt + r) * IS + off);
                mma(acc[q], ah, bl);
                mma(acc[q], al, bh);
                mma(acc[q], ah, bh);
            }
        }
    }
    write_record<KC, VC, UPW, NKS, true>(r_seg + (bh * n_seg + sg) * (int64_t)K * dva, acc, z, s_z, K, d_v, dva);
}

// Key side: dGamma_K [BH][N][K] fp32 (EMIT_DL: dl in its place, as on the query side) and dV [BH][N][d_v]
// bf16 from the summed R (entry 0 of r_seg [BH][n_seg][K][dva]); Gamma_K in the permuted component order.
template <int KC, int VC, bool EMIT_DL>
__global__ void __launch_bounds__(256) bwd_bidir_k_kernel(const float* gk, const void* v, const float* r_seg,
                                                          float* dgk, void* dv, int64_t N, int K, int d_v, int dva,
                                                          int seg, int64_t n_seg) {
    constexpr int C = kFusedChunk, NKS = KC / 32, NVT = VC / 16, NVS = VC / 32, NCT = KC / 16;
    constexpr int WC = 2 * VC + 16, WD = 2 * KC + 16;
    __shared__ __attribute__((aligned(16))) char s_rc[2 * KC * WC];   // R_v hi, lo: [comp][dim]
    __shared__ __attribute__((aligned(16))) char s_rd[2 * VC * WD];   // R_v^T hi, lo: [dim][comp]
    __shared__ float s_r1[KC];
    lds_char* const RCH = (lds_char*)s_rc;
    lds_char* const RCL = RCH + KC * WC;
    lds_char* const RDH = (lds_char*)s_rd;
    lds_char* const RDL = RDH + VC * WD;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int64_t bh = blockIdx.x / n_seg, sg = blockIdx.x % n_seg;
    const int64_t t0 = sg * seg;
    const int64_t t1 = t0 + seg < N ? t0 + seg : N;
    const int nch = (int)((t1 - t0 + C - 1) / C);
    const __amdgpu_buffer_rsrc_t rs_g = make_rsrc(gk + bh * N * K, (uint32_t)(N * K * 4));
    const __amdgpu_buffer_rsrc_t rs_o = make_rsrc(dgk + bh * N * K, (uint32_t)(N * K * 4));
    const __amdgpu_buffer_rsrc_t rs_v =
        make_rsrc(reinterpret_cast<const uint16_t*>(v) + bh * N * d_v, (uint32_t)(N * d_v * 2));
    const __amdgpu_buffer_rsrc_t rs_w = make_rsrc(reinterpret_cast<uint16_t*>(dv) + bh * N * d_v, (uint32_t)(N * d_v * 2));
    constexpr uint32_t kOut = 0x80000000u;

    stage_record<KC, VC>(r_seg + bh * n_seg * (int64_t)K * dva, K, d_v, dva, RCH, RCL, RDH, RDL, s_r1);

    f32x4 ga[NKS][2];
    u32x2 va[NVT];
    auto load = [&](int64_t n0) {
        const uint32_t t = (uint32_t)(n0 + 16 * w + r);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int k = 32 * ks + 16 * hf + 4 * g;
                ga[ks][hf] = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs_g, k < K ? (t * K + k) * 4 : kOut, 0, 0));
            }
#pragma unroll
        for (int j = 0; j < NVT; ++j) {
            const int d = 16 * j + 4 * g;
            va[j] = __builtin_amdgcn_raw_buffer_load_b64(rs_v, d < d_v ? (t * d_v + d) * 2 : kOut, 0, 0);
        }
    };

    if (nch > 0) load(t0);
    __syncthreads();   // the staged R
    for (int c = 0; c < nch; ++c) {
        const int64_t n0 = t0 + (int64_t)c * C;
        const uint32_t t = (uint32_t)(n0 + 16 * w + r);
        bf16x8 gh8[NKS], gl8[NKS];
        float gv[NKS][8];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
            for (int e = 0; e < 8; ++e) gv[ks][e] = ga[ks][e >> 2][e & 3];
            split_bf16x8(gv[ks], gh8[ks], gl8[ks]);
        }
        bf16x8 vf[NVS];
#pragma unroll
        for (int vs = 0; vs < NVS; ++vs)
            vf[vs] = __builtin_bit_cast(bf16x8, u32x4{va[2 * vs][0], va[2 * vs][1], va[2 * vs + 1][0], va[2 * vs + 1][1]});
        if (c + 1 < nch) load(n0 + C);
        // dGamma_K of this lane's row, components 16 ct + 4 g .. + 3 (the lane's own order)
        f32x4 dgo[NCT];
        float dot2 = 0.f;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            f32x4 dg = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int vs = 0; vs < NVS; ++vs) {
                mma(dg, row_perm(RCL + (16 * ct + r) * WC, vs, g), vf[vs]);
                mma(dg, row_perm(RCH + (16 * ct + r) * WC, vs, g), vf[vs]);
            }
            const int k = 16 * ct + 4 * g;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                dgo[ct][i] = dg[i] + s_r1[k + i];
                dot2 += gv[ct >> 1][4 * (ct & 1) + i] * dgo[ct][i];
            }
        }
        if constexpr (EMIT_DL) {
            dot2 += __shfl_xor(dot2, 16, 64);
            dot2 += __shfl_xor(dot2, 32, 64);
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const int k = 16 * ct + 4 * g;
            f32x4 o = dgo[ct];
            if constexpr (EMIT_DL) {
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] = gv[ct >> 1][4 * (ct & 1) + i] * (dgo[ct][i] - dot2);
            }
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), rs_o, k < K ? (t * K + k) * 4 : kOut,
                                                   0, 0);
        }
        // dV of this lane's row, dims 16 j + 4 g .. + 3
#pragma unroll
        for (int j = 0; j < NVT; ++j) {
            f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const bf16x8 ah = row_perm(RDH + (16 * j + r) * WD, ks, g);
                const bf16x8 al = row_perm(RDL + (16 * j + r) * WD, ks, g);
                mma(o, ah, gl8[ks]);
                mma(o, al, gh8[ks]);
                mma(o, ah, gh8[ks]);
            }
            const int d = 16 * j + 4 * g;
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, pack4(o)), rs_w,
                                                  d < d_v ? (t * d_v + d) * 2 : kOut, 0, 0);
        }
    }
}

// ---------------------------------------------------------------------------------- chunk states
// The causal prefix states from the chunk terms Gamma_K^T [V | 1] (64 tokens per chunk, bf16 storage,
// K = d_v = 128), as [K][dva] records (columns d_v .. dva - 1: Z, then zeros), in two passes over segments
// of `per` consecutive chunks of one (batch, head): the first (totals) writes each segment's total into
// seg [BH][ceil(n_st / per)]; an exclusive scan over seg gives the segments' prefixes; the second starts
// a running sum at its segment's prefix and writes, for each chunk, the sum of the terms of all earlier
// chunks into stt.  The running sum stays in registers; the next chunk's rows are loaded ahead.  Gamma_K
// goes to LDS as a bf16 hi + lo image, V as an exact one.  The product is formed transposed, V^T Gamma_K
// (A = V^T, B = Gamma_K, both transposed fragments), so each lane stores four consecutive d_v columns of
// one component; the Z row comes from a ones fragment.  Wave w takes d_v tiles 2 w, 2 w + 1 for all
// components, and the Z row of component tiles 2 w, 2 w + 1.
template <int KC, int VC>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
bwd_chunk_state_kernel(const float* gk, const void* v, float* stt, float* seg, int64_t N, int64_t n_st, int per,
                       int dva, int totals) {
    static_assert(KC == 128 && VC == 128, "one 256-byte image row per token");
    constexpr int C = 64;
    constexpr int IMG = C * 256;
    __shared__ __attribute__((aligned(16))) char s_k[2 * IMG];   // Gamma_K hi, lo
    __shared__ __attribute__((aligned(16))) char s_v[IMG];       // V
    lds_char* const LKH = (lds_char*)s_k;
    lds_char* const LKL = LKH + IMG;
    lds_char* const LV = (lds_char*)s_v;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int64_t groups = (n_st + per - 1) / per;
    const int64_t bh = blockIdx.x / groups;
    const int64_t c0 = (blockIdx.x % groups) * per;
    const int64_t c1 = c0 + per < n_st ? c0 + per : n_st;
    const int64_t rec = (int64_t)KC * dva;

    f32x4 pk[8];
    u32x4 pv[4];
    auto fetch = [&](int64_t c) {
        const int64_t n0 = c * C;
        const int nv = (int)(N - n0 < C ? N - n0 : C);
        const float* gkh = gk + (bh * N + n0) * KC;
        const uint16_t* vh = reinterpret_cast<const uint16_t*>(v) + (bh * N + n0) * VC;
        const int rl = lane >> 5, cl = lane & 31;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int row = 16 * w + 2 * j + rl;
            pk[j] = row < nv ? *reinterpret_cast<const f32x4*>(gkh + (int64_t)row * KC + 4 * cl) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            const int row = 16 * w + 4 * bb + (lane >> 4);
            pv[bb] = row < nv ? *reinterpret_cast<const u32x4*>(vh + (int64_t)row * VC + 8 * (lane & 15)) : u32x4{0u, 0u, 0u, 0u};
        }
    };
    bf16x8 ones0;   // A fragment of the Z row: row 0 ones, the other rows zero
    {
        const __bf16 o = (__bf16)(r == 0 ? 1.f : 0.f);
        ones0 = bf16x8{o, o, o, o, o, o, o, o};
    }

    // running sums: run[t][ct] in the accumulator layout below, zrun[hh] of the Z rows; the second pass
    // starts at the segment's prefix
    float* seg_rec = seg + (bh * ((n_st + per - 1) / per) + c0 / per) * rec;
    f32x4 run[2][8], zrun[2];
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) run[0][ct] = run[1][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    zrun[0] = zrun[1] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (!totals) {
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            const float* row = seg_rec + (int64_t)(16 * ct + r) * dva;
#pragma unroll
            for (int t = 0; t < 2; ++t) run[t][ct] = *reinterpret_cast<const f32x4*>(row + 32 * w + 16 * t + 4 * g);
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
            if (g == 0) zrun[hh] = *reinterpret_cast<const f32x4*>(seg_rec + (int64_t)(16 * (2 * w + hh) + r) * dva + VC);
    }
    auto store_rec = [&](float* rec_c) {
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            float* row = rec_c + (int64_t)(16 * ct + r) * dva;
#pragma unroll
            for (int t = 0; t < 2; ++t) *reinterpret_cast<f32x4*>(row + 32 * w + 16 * t + 4 * g) = run[t][ct];
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
            if (g == 0) *reinterpret_cast<f32x4*>(rec_c + (int64_t)(16 * (2 * w + hh) + r) * dva + VC) = zrun[hh];
    };

    fetch(c0);
    for (int64_t c = c0; c < c1; ++c) {
        if (c > c0) lds_barrier();
        // this chunk's record: the terms of all earlier chunks
        if (!totals) store_rec(stt + (bh * n_st + c) * rec);
        {
            const int rl = lane >> 5, cl = lane & 31;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int off = img_slot(16 * w + 2 * j + rl, cl);
                bf16x4 hi, lo;
                split4(pk[j], hi, lo);
                lds_st<bf16x4>(LKH + off, hi);
                lds_st<bf16x4>(LKL + off, lo);
            }
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) lds_st<u32x4>(LV + img_chunk(16 * w + 4 * bb + (lane >> 4), lane & 15), pv[bb]);
        }
        if (c + 1 < c1) fetch(c + 1);
        lds_barrier();
        // the chunk's term, added to the running sums: run[t][ct] rows = d_v 32 w + 16 t + 4 g + i, column =
        // component 16 ct + r
#pragma unroll
        for (int tk = 0; tk < 2; ++tk) {
            bf16x8 av[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) av[t] = img_tr(LV, 2 * w + t, tk, lane);
#pragma unroll
            for (int ct = 0; ct < 8; ++ct) {
                const bf16x8 bh_ = img_tr(LKH, ct, tk, lane), bl = img_tr(LKL, ct, tk, lane);
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    mma(run[t][ct], av[t], bl);
                    mma(run[t][ct], av[t], bh_);
                }
            }
        }
        // Z (row 0 of the ones fragment's product; rows 1 .. 3 stay zero, the padding): component tiles 2 w,
        // 2 w + 1
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int ct = 2 * w + hh;
#pragma unroll
            for (int tk = 0; tk < 2; ++tk) {
                mma(zrun[hh], ones0, img_tr(LKL, ct, tk, lane));
                mma(zrun[hh], ones0, img_tr(LKH, ct, tk, lane));
            }
        }
    }
    // the segment's total (first pass)
    if (totals) store_rec(seg_rec);
}

// ---------------------------------------------------------------------------------- suffix states
// The causal suffix states R_c = sum over the chunks after c of Gamma_Q^T [g | h] (64 tokens per chunk,
// bf16 storage, K = d_v = 128), as [K][dva] records (columns d_v .. dva - 1: the h sums r, then zeros),
// from the recomputed Gamma_Q, dO and the per-row pairs rs = (1 / den, h): g = dO / den.  One pass over
// segments of `per` consecutive chunks of one (batch, head): seg holds each segment's suffix (the query-side
// chunk kernel writes the segment totals, an exclusive suffix scan turns them into suffixes), and each
// workgroup walks its segment backwards from there and writes each chunk's R.  Gamma_Q and g go to LDS as
// bf16 hi + lo images; the product is formed transposed, g^T Gamma_Q, so each lane stores four
// consecutive d_v columns of one component; the r row comes from an h fragment (row 0 = h).  Wave w takes
// d_v tiles 2 w, 2 w + 1 for all components and the r row of component tiles 2 w, 2 w + 1.
template <int KC, int VC>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
bwd_suffix_state_kernel(const float* gq, const void* dout, const float* rs, float* rt, const float* seg,
                        int64_t N, int64_t n_st, int per, int dva) {
    static_assert(KC == 128 && VC == 128, "one 256-byte image row per token");
    constexpr int C = 64;
    constexpr int IMG = C * 256;
    __shared__ __attribute__((aligned(16))) char s_q[2 * IMG];   // Gamma_Q hi, lo
    __shared__ __attribute__((aligned(16))) char s_g[2 * IMG];   // g hi, lo
    __shared__ float s_h[C];
    lds_char* const LQH = (lds_char*)s_q;
    lds_char* const LQL = LQH + IMG;
    lds_char* const LGH = (lds_char*)s_g;
    lds_char* const LGL = LGH + IMG;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int64_t groups = (n_st + per - 1) / per;
    const int64_t bh = blockIdx.x / groups;
    const int64_t c0 = (blockIdx.x % groups) * per;
    const int64_t c1 = c0 + per < n_st ? c0 + per : n_st;
    const int64_t rec = (int64_t)KC * dva;

    f32x4 pq[8];
    u32x4 pd[4];
    float pr0[4], pr1[4];
    auto fetch = [&](int64_t c) {
        const int64_t n0 = c * C;
        const int nv = (int)(N - n0 < C ? N - n0 : C);
        const float* gqh = gq + (bh * N + n0) * KC;
        const uint16_t* dh = reinterpret_cast<const uint16_t*>(dout) + (bh * N + n0) * VC;
        const int rl = lane >> 5, cl = lane & 31;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int row = 16 * w + 2 * j + rl;
            pq[j] = row < nv ? *reinterpret_cast<const f32x4*>(gqh + (int64_t)row * KC + 4 * cl) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            const int row = 16 * w + 4 * bb + (lane >> 4);
            const bool ok = row < nv;
            pd[bb] = ok ? *reinterpret_cast<const u32x4*>(dh + (int64_t)row * VC + 8 * (lane & 15)) : u32x4{0u, 0u, 0u, 0u};
            pr0[bb] = ok ? rs[(bh * N + n0 + row) * 2] : 0.f;
            pr1[bb] = ok ? rs[(bh * N + n0 + row) * 2 + 1] : 0.f;
        }
    };

    // running sums: run[t][ct] rows = d_v 32 w + 16 t + 4 g + i, column = component 16 ct + r; hrun[hh] row 0
    // = the r sums of component tile 2 w + hh.  They start at the segment's suffix.
    const float* seg_rec = seg + (bh * groups + c0 / per) * rec;
    f32x4 run[2][8], hrun[2];
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
        const float* row = seg_rec + (int64_t)(16 * ct + r) * dva;
#pragma unroll
        for (int t = 0; t < 2; ++t) run[t][ct] = *reinterpret_cast<const f32x4*>(row + 32 * w + 16 * t + 4 * g);
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
        hrun[hh] = (g == 0) ? *reinterpret_cast<const f32x4*>(seg_rec + (int64_t)(16 * (2 * w + hh) + r) * dva + VC)
                            : f32x4{0.f, 0.f, 0.f, 0.f};
    auto store_rec = [&](float* rec_c) {
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            float* row = rec_c + (int64_t)(16 * ct + r) * dva;
#pragma unroll
            for (int t = 0; t < 2; ++t) *reinterpret_cast<f32x4*>(row + 32 * w + 16 * t + 4 * g) = run[t][ct];
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
            if (g == 0) *reinterpret_cast<f32x4*>(rec_c + (int64_t)(16 * (2 * w + hh) + r) * dva + VC) = hrun[hh];
    };

    // the segment backwards (a suffix)
    fetch(c1 - 1);
    for (int64_t c = c1 - 1; c >= c0; --c) {
        if (c < c1 - 1) lds_barrier();
        store_rec(rt + (bh * n_st + c) * rec);   // the terms of all later chunks
        {
            const int rl = lane >> 5, cl = lane & 31;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int off = img_slot(16 * w + 2 * j + rl, cl);
                bf16x4 hi, lo;
                split4(pq[j], hi, lo);
                lds_st<bf16x4>(LQH + off, hi);
                lds_st<bf16x4>(LQL + off, lo);
            }
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                const int row = 16 * w + 4 * bb + (lane >> 4), ch = lane & 15;
                const bf16x8 dv8 = __builtin_bit_cast(bf16x8, pd[bb]);
                float gv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) gv[e] = (float)dv8[e] * pr0[bb];
                bf16x8 hi, lo;
                split_bf16x8(gv, hi, lo);
                lds_st<bf16x8>(LGH + img_chunk(row, ch), hi);
                lds_st<bf16x8>(LGL + img_chunk(row, ch), lo);
                if (ch == 0) s_h[row] = pr1[bb];
            }
        }
        if (c > c0) fetch(c - 1);
        lds_barrier();
#pragma unroll
        for (int tk = 0; tk < 2; ++tk) {
            bf16x8 agh[2], agl[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                agh[t] = img_tr(LGH, 2 * w + t, tk, lane);
                agl[t] = img_tr(LGL, 2 * w + t, tk, lane);
            }
#pragma unroll
            for (int ct = 0; ct < 8; ++ct) {
                const bf16x8 bh_ = img_tr(LQH, ct, tk, lane), bl = img_tr(LQL, ct, tk, lane);
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    mma(run[t][ct], agl[t], bh_);
                    mma(run[t][ct], agh[t], bl);
                    mma(run[t][ct], agh[t], bh_);
                }
            }
        }
        // the r row: A fragment row 0 = h of the tokens (split), rows 1 .. 15 zero
#pragma unroll
        for (int tk = 0; tk < 2; ++tk) {
            float hv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) hv[e] = r == 0 ? s_h[32 * tk + 16 * (e >> 2) + 4 * g + (e & 3)] : 0.f;
            bf16x8 hh_, hl;
            split_bf16x8(hv, hh_, hl);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int ct = 2 * w + hh;
                const bf16x8 bh_ = img_tr(LQH, ct, tk, lane), bl = img_tr(LQL, ct, tk, lane);
                mma(hrun[hh], hl, bh_);
                mma(hrun[hh], hh_, bl);
                mma(hrun[hh], hh_, bh_);
            }
        }
    }
}

// ---------------------------------------------------------------------------------- fused chunk, query side
// Ownership in the fused chunk kernels, for W = 4 or 8 wavefronts: TW = 8 / W of the eight 16-wide
// tiles of d_v or of the components per wave (tiles TW w .. TW w + TW - 1); for the 64 x 64 blocks,
// QW = W / 4 waves per q tile: wave w takes q tile w / QW and the key tiles kt = w % QW (mod QW);
// staging rows 64 / W per wave.
template <int W>
struct ChunkSplit {
    static_assert(W == 4 || W == 8, "four or eight wavefronts");
    static constexpr int TW = 8 / W;
    static constexpr int QW = W / 4;
    static constexpr int RPW = 64 / W;
};

// Epilogue of dGamma in the chunk kernels: acc[t][rt] rows = components 16 (TW w + t) + 4 g + i, column =
// row 16 rt + r of the chunk (a query or a key).  Stores dGamma, or with emit_dl the posterior gradient
// dl = gamma (dGamma - gamma . dGamma) of the row, gamma read back from the chunk's image (hi + lo, about
// 16 significant bits); the row dot goes through part [W][64] in LDS (one barrier).  Rows past nv are
// not stored.
template <int TW, int W>
__device__ __forceinline__ void finish_dgamma(f32x4 (&acc)[TW][4], const lds_char* gam_hi, const lds_char* gam_lo,
                                              float (*part)[64], float* out, int nv, int w, int lane, int emit_dl) {
    const int r = lane & 15, g = lane >> 4;
    if (emit_dl) {
        f32x4 gam[TW][4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            float d = 0.f;
#pragma unroll
            for (int t = 0; t < TW; ++t) {
                const int off = img_slot(16 * rt + r, 4 * (TW * w + t) + g);
                const bf16x4 hi = lds_ld<bf16x4>(gam_hi + off), lo = lds_ld<bf16x4>(gam_lo + off);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    gam[t][rt][i] = (float)hi[i] + (float)lo[i];
                    d += gam[t][rt][i] * acc[t][rt][i];
                }
            }
            d += __shfl_xor(d, 16, 64);
            d += __shfl_xor(d, 32, 64);
            if (g == 0) part[w][16 * rt + r] = d;
        }
        lds_barrier();
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            float dot = 0.f;
#pragma unroll
            for (int p = 0; p < W; ++p) dot += part[p][16 * rt + r];
#pragma unroll
            for (int t = 0; t < TW; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[t][rt][i] = gam[t][rt][i] * (acc[t][rt][i] - dot);
        }
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        const int row = 16 * rt + r;
        if (row >= nv) continue;
#pragma unroll
        for (int t = 0; t < TW; ++t)
            *reinterpret_cast<f32x4*>(out + (int64_t)row * 128 + 16 * (TW * w + t) + 4 * g) = acc[t][rt];
    }
}

// The query-side chunk work of the causal backward in one kernel (bf16 storage, K = d_v = 128).  From the
// recomputed posteriors, V, dO and the state before the chunk S = [Vt | Z] (the exclusive prefix over
// chunks of Gamma_K^T [V | 1]), per chunk of 64 tokens:
//   ac  = tril(Gamma_Q Gamma_K^T)
//   num = Gamma_Q Vt + ac V,   den = Gamma_Q . Z + ac 1 + eps
//   g   = dO / den,  h = -(dO . num / den) / den                -> rs = (1 / den, h)
//   rt  = Gamma_Q^T [g | h]                                      (the chunk's term of the suffix sums)
//   mt  = tril([g | h] [V | 1]^T)
//   dGamma_Q = [g | h] S^T + mt Gamma_K
// ac and mt go to HBM only where asked for.  A workgroup of W wavefronts walks `per` consecutive chunks
// of one (batch, head); the next chunk's token operands are loaded into registers while the current one
// is processed.  Gamma_Q, Gamma_K, g and the 64 x 64 blocks live in LDS as bf16 hi + lo images, V (and
// dO, for one step) as exact bf16 images; the state goes from HBM straight into split fragments (the
// wave's d_v tiles for num, its component tiles for dGamma_Q).  ac, mt, rt and dGamma_Q are formed
// transposed (their accumulator rows run along the stored rows), so that each lane stores 16
// contiguous bytes.  Products: hi hi + hi lo + lo hi between two fp32 operands, hi + lo against V,
// fp32 accumulation.
template <int KC, int VC, int W>
__global__ void __launch_bounds__(W * 64) bwd_chunk_q_kernel(const float* gq, const float* gk, const void* v,
                                                             const void* dout, const float* stt, float* rs, float* rt,
                                                             float* ac_out, float* mt_out, float* dgq, int64_t N,
                                                             int64_t n_st, int per, int dva, float eps, int emit_dl) {
    static_assert(KC == 128 && VC == 128, "one 256-byte image row per token");
    using CS = ChunkSplit<W>;
    constexpr int TW = CS::TW, QW = CS::QW, RPW = CS::RPW;
    constexpr int C = 64;
    constexpr int IMG = C * 256;
    __shared__ __attribute__((aligned(16))) char s_q[2 * IMG];   // Gamma_Q hi, lo
    __shared__ __attribute__((aligned(16))) char s_k[2 * IMG];   // Gamma_K hi, lo
    __shared__ __attribute__((aligned(16))) char s_v[IMG];       // V
    __shared__ __attribute__((aligned(16))) char s_g[2 * IMG];   // g hi, lo
    __shared__ __attribute__((aligned(16))) char s_m[2 * IMG];   // ac hi, lo; then dO; then mt hi, lo
    __shared__ float s_z[KC], s_den[C], s_inv[C], s_h[C], s_part[W][C], s_dpart[QW][C];
    lds_char* const LQH = (lds_char*)s_q;
    lds_char* const LQL = LQH + IMG;
    lds_char* const LKH = (lds_char*)s_k;
    lds_char* const LKL = LKH + IMG;
    lds_char* const LV = (lds_char*)s_v;
    lds_char* const LGH = (lds_char*)s_g;
    lds_char* const LGL = LGH + IMG;
    lds_char* const LMH = (lds_char*)s_m;
    lds_char* const LML = LMH + IMG;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int qw = w / QW, kp = w % QW;   // the wave's q tile and key-tile phase in the 64 x 64 blocks
    const int64_t groups = (n_st + per - 1) / per;
    const int64_t bh = blockIdx.x / groups;
    const int64_t c0 = (blockIdx.x % groups) * per;
    const int64_t c1 = c0 + per < n_st ? c0 + per : n_st;
    const int64_t rec = (int64_t)KC * dva;

    // ---- the token operands of one chunk, loaded a chunk ahead: Gamma_Q, Gamma_K rows RPW w + 2 j + l / 32
    // (components 4 (l % 32) .. + 3); V, dO rows RPW w + 4 bb + l / 16 (chunk l % 16)
    f32x4 pq[RPW / 2], pk[RPW / 2];
    u32x4 pv[RPW / 4], pd[RPW / 4];
    auto fetch = [&](int64_t c) {
        const int64_t n0 = c * C;
        const int nv = (int)(N - n0 < C ? N - n0 : C);
        const float* gqh = gq + (bh * N + n0) * KC;
        const float* gkh = gk + (bh * N + n0) * KC;
        const uint16_t* vh = reinterpret_cast<const uint16_t*>(v) + (bh * N + n0) * VC;
        const uint16_t* dh = reinterpret_cast<const uint16_t*>(dout) + (bh * N + n0) * VC;
        const int rl = lane >> 5, cl = lane & 31;
#pragma unroll
        for (int j = 0; j < RPW / 2; ++j) {
            const int row = RPW * w + 2 * j + rl;
            pq[j] = row < nv ? *reinterpret_cast<const f32x4*>(gqh + (int64_t)row * KC + 4 * cl) : f32x4{0.f, 0.f, 0.f, 0.f};
            pk[j] = row < nv ? *reinterpret_cast<const f32x4*>(gkh + (int64_t)row * KC + 4 * cl) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int bb = 0; bb < RPW / 4; ++bb) {
            const int row = RPW * w + 4 * bb + (lane >> 4), ch = lane & 15;
            pv[bb] = row < nv ? *reinterpret_cast<const u32x4*>(vh + (int64_t)row * VC + 8 * ch) : u32x4{0u, 0u, 0u, 0u};
            pd[bb] = row < nv ? *reinterpret_cast<const u32x4*>(dh + (int64_t)row * VC + 8 * ch) : u32x4{0u, 0u, 0u, 0u};
        }
    };

    // segment total of the suffix-state terms Gamma_Q^T [g | h] over this walk (rt non-null: the walk is one
    // state segment): racc[vt][t] rows = d_v 16 vt + 4 g + i (vt 8: the h row and zero padding), column =
    // component 16 (TW w + t) + r, summed over the walk's chunks in order
    f32x4 racc[9][TW];
#pragma unroll
    for (int vt = 0; vt < 9; ++vt)
#pragma unroll
        for (int t = 0; t < TW; ++t) racc[vt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    fetch(c0);
    for (int64_t c = c0; c < c1; ++c) {
        const int64_t n0 = c * C;
        const int nv = (int)(N - n0 < C ? N - n0 : C);   // rows of the chunk inside the sequence
        float* blk_ac = ac_out ? ac_out + (bh * n_st + c) * C * C : nullptr;   // null: the blocks are not stored
        float* blk_mt = mt_out ? mt_out + (bh * n_st + c) * C * C : nullptr;
        if (c > c0) lds_barrier();   // every wave is done with the previous chunk's images

        // ---- stage this chunk's operands
        {
            const int rl = lane >> 5, cl = lane & 31;
#pragma unroll
            for (int j = 0; j < RPW / 2; ++j) {
                const int off = img_slot(RPW * w + 2 * j + rl, cl);
                bf16x4 hi, lo;
                split4(pq[j], hi, lo);
                lds_st<bf16x4>(LQH + off, hi);
                lds_st<bf16x4>(LQL + off, lo);
                split4(pk[j], hi, lo);
                lds_st<bf16x4>(LKH + off, hi);
                lds_st<bf16x4>(LKL + off, lo);
            }
        }
        u32x4 dor[RPW / 4];
#pragma unroll
        for (int bb = 0; bb < RPW / 4; ++bb) {
            lds_st<u32x4>(LV + img_chunk(RPW * w + 4 * bb + (lane >> 4), lane & 15), pv[bb]);
            dor[bb] = pd[bb];
        }
        // the state before this chunk, split where it is used: for num (rows 32 ks + 8 g + e, the wave's d_v
        // columns 16 (TW w + t) + r) loaded now, for dGamma_Q (the wave's component rows 16 (TW w + t) + r,
        // columns 32 ks + 8 g .. + 7) loaded after rt; Z
        const float* S = stt + (bh * n_st + c) * rec;
        float psn[TW][4][8];
#pragma unroll
        for (int t = 0; t < TW; ++t)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) psn[t][ks][e] = S[(int64_t)(32 * ks + 8 * g + e) * dva + 16 * (TW * w + t) + r];
        const float pz = tid < KC ? S[(int64_t)tid * dva + VC] : 0.f;
        if (c + 1 < c1) fetch(c + 1);
        lds_barrier();

        // ---- ac^T = Gamma_K Gamma_Q^T, q tile qw, key tiles kp (mod QW): acc[kt] rows = keys 16 kt + 4 g + i,
        // column = q 16 qw + r; image (rows q), row-sum parts
        {
            const int q = 16 * qw + r;
            f32x4 acc[4];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) acc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8 bh_ = img_row(LQH, q, ks, g), bl = img_row(LQL, q, ks, g);
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) {
                    if (kt % QW != kp || kt > qw) continue;
                    const bf16x8 ah = img_row(LKH, 16 * kt + r, ks, g), al = img_row(LKL, 16 * kt + r, ks, g);
                    mma(acc[kt], al, bh_);
                    mma(acc[kt], ah, bl);
                    mma(acc[kt], ah, bh_);
                }
            }
            float rsum = 0.f;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                if (kt % QW != kp) continue;
                f32x4 val;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = 16 * kt + 4 * g + i;
                    val[i] = (kt <= qw && key <= q) ? acc[kt][i] : 0.f;
                    rsum += val[i];
                }
                bf16x4 hi, lo;
                split4(val, hi, lo);
                lds_st<bf16x4>(LMH + img_slot(q, 4 * kt + g), hi);
                lds_st<bf16x4>(LML + img_slot(q, 4 * kt + g), lo);
                if (blk_ac) *reinterpret_cast<f32x4*>(blk_ac + q * C + 16 * kt + 4 * g) = val;
            }
            rsum += __shfl_xor(rsum, 16, 64);
            rsum += __shfl_xor(rsum, 32, 64);
            if (g == 0) s_dpart[kp][q] = rsum;
        }
        if (tid < KC) s_z[tid] = pz;
        lds_barrier();
        bf16x8 snh[TW][4], snl[TW][4];
#pragma unroll
        for (int t = 0; t < TW; ++t)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) split_bf16x8(psn[t][ks], snh[t][ks], snl[t][ks]);

        // ---- num (the wave's d_v tiles: rows q 16 qt + 4 g + i), den of q tile qw (phase-0 waves)
        f32x4 num[4][TW];
#pragma unroll
        for (int qt = 0; qt < 4; ++qt)
#pragma unroll
            for (int t = 0; t < TW; ++t) num[qt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int qt = 0; qt < 4; ++qt) {
                const bf16x8 ah = img_row(LQH, 16 * qt + r, ks, g), al = img_row(LQL, 16 * qt + r, ks, g);
#pragma unroll
                for (int t = 0; t < TW; ++t) {
                    mma(num[qt][t], al, snh[t][ks]);
                    mma(num[qt][t], ah, snl[t][ks]);
                    mma(num[qt][t], ah, snh[t][ks]);
                }
            }
#pragma unroll
        for (int ks2 = 0; ks2 < 2; ++ks2) {
            bf16x8 vb[TW];
#pragma unroll
            for (int t = 0; t < TW; ++t) vb[t] = img_tr(LV, TW * w + t, ks2, lane);
#pragma unroll
            for (int qt = 0; qt < 4; ++qt) {
                if (ks2 == 1 && qt < 2) continue;   // keys 32 .. 63 lie above those rows: ac = 0
                const bf16x8 ah = img_row_perm(LMH, 16 * qt + r, ks2, g), al = img_row_perm(LML, 16 * qt + r, ks2, g);
#pragma unroll
                for (int t = 0; t < TW; ++t) {
                    mma(num[qt][t], al, vb[t]);
                    mma(num[qt][t], ah, vb[t]);
                }
            }
        }
        if (kp == 0) {
            f32x4 dacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8 ah = img_row(LQH, 16 * qw + r, ks, g), al = img_row(LQL, 16 * qw + r, ks, g);
                float zv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) zv[e] = r == 0 ? s_z[32 * ks + 8 * g + e] : 0.f;
                bf16x8 zh, zl;
                split_bf16x8(zv, zh, zl);
                mma(dacc, al, zh);
                mma(dacc, ah, zl);
                mma(dacc, ah, zh);
            }
            if (r == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int q = 16 * qw + 4 * g + i;
                    float d = 0.f;
#pragma unroll
                    for (int p = 0; p < QW; ++p) d += s_dpart[p][q];
                    s_den[q] = d + dacc[i] + eps;
                }
            }
        }
        lds_barrier();   // den complete; ac no longer read

        // ---- g, h: dO into the spare image, 1 / den, the wave's part of dO . num per row
#pragma unroll
        for (int bb = 0; bb < RPW / 4; ++bb)
            lds_st<u32x4>(LMH + img_chunk(RPW * w + 4 * bb + (lane >> 4), lane & 15), dor[bb]);
        if (tid < C) s_inv[tid] = tid < nv ? 1.f / s_den[tid] : 0.f;   // rows past N: g = h = 0 (even with eps = 0)
        lds_barrier();
#pragma unroll
        for (int qt = 0; qt < 4; ++qt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int q = 16 * qt + 4 * g + i;
                const float inv = s_inv[q];
                float d = 0.f;
#pragma unroll
                for (int t = 0; t < TW; ++t) {
                    const float dov = (float)lds_ld<__bf16>(LMH + img_elem(q, 16 * (TW * w + t) + r));
                    d += num[qt][t][i] * inv * dov;
                }
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) d += __shfl_xor(d, o, 64);
                if (r == 0) s_part[w][q] = d;
            }
        lds_barrier();
        if (tid < C) {
            const float inv = s_inv[tid];
            float d = 0.f;
#pragma unroll
            for (int p = 0; p < W; ++p) d += s_part[p][tid];
            const float hv = -d * inv;
            s_h[tid] = hv;
            if (tid < nv) {
                rs[(bh * N + n0 + tid) * 2] = inv;
                rs[(bh * N + n0 + tid) * 2 + 1] = hv;
            }
        }
#pragma unroll
        for (int bb = 0; bb < RPW / 4; ++bb) {
            const int row = RPW * w + 4 * bb + (lane >> 4), ch = lane & 15;
            const float inv = s_inv[row];
            const bf16x8 dv8 = __builtin_bit_cast(bf16x8, dor[bb]);
            float gv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) gv[e] = (float)dv8[e] * inv;
            bf16x8 hi, lo;
            split_bf16x8(gv, hi, lo);
            lds_st<bf16x8>(LGH + img_chunk(row, ch), hi);
            lds_st<bf16x8>(LGL + img_chunk(row, ch), lo);
        }
        lds_barrier();   // g, h visible; dO no longer read

        // ---- the chunk's term [g | h]^T Gamma_Q of the suffix states, added to the walk's total (where rt is
        // given: the segment totals that the suffix-state kernel starts from)
        if (rt) {
#pragma unroll
            for (int tk = 0; tk < 2; ++tk) {
                bf16x8 bqh[TW], bql[TW];
#pragma unroll
                for (int t = 0; t < TW; ++t) {
                    bqh[t] = img_tr(LQH, TW * w + t, tk, lane);
                    bql[t] = img_tr(LQL, TW * w + t, tk, lane);
                }
#pragma unroll
                for (int vt = 0; vt < 8; ++vt) {
                    const bf16x8 ah = img_tr(LGH, vt, tk, lane), al = img_tr(LGL, vt, tk, lane);
#pragma unroll
                    for (int t = 0; t < TW; ++t) {
                        mma(racc[vt][t], al, bqh[t]);
                        mma(racc[vt][t], ah, bql[t]);
                        mma(racc[vt][t], ah, bqh[t]);
                    }
                }
                float hv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) hv[e] = r == 0 ? s_h[32 * tk + 16 * (e >> 2) + 4 * g + (e & 3)] : 0.f;
                bf16x8 hh, hl;
                split_bf16x8(hv, hh, hl);
#pragma unroll
                for (int t = 0; t < TW; ++t) {
                    mma(racc[8][t], hl, bqh[t]);
                    mma(racc[8][t], hh, bql[t]);
                    mma(racc[8][t], hh, bqh[t]);
                }
            }
        }

        f32x4 psd[TW][4][2];
#pragma unroll
        for (int t = 0; t < TW; ++t)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const float* p = S + (int64_t)(16 * (TW * w + t) + r) * dva + 32 * ks + 8 * g;
                psd[t][ks][0] = *reinterpret_cast<const f32x4*>(p);
                psd[t][ks][1] = *reinterpret_cast<const f32x4*>(p + 4);
            }

        // ---- mt^T = [V | 1] [g | h]^T, q tile qw, key tiles kp (mod QW): macc[kt] rows = keys 16 kt + 4 g + i,
        // column = q 16 qw + r
        {
            const int q = 16 * qw + r;
            const float hq = s_h[q];
            f32x4 macc[4];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) macc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8 bh_ = img_row(LGH, q, ks, g), bl = img_row(LGL, q, ks, g);
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) {
                    if (kt % QW != kp || kt > qw) continue;
                    const bf16x8 av = img_row(LV, 16 * kt + r, ks, g);
                    mma(macc[kt], av, bl);
                    mma(macc[kt], av, bh_);
                }
            }
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                if (kt % QW != kp) continue;
                f32x4 val;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = 16 * kt + 4 * g + i;
                    val[i] = (kt <= qw && key <= q && key < nv) ? macc[kt][i] + hq : 0.f;
                }
                bf16x4 hi, lo;
                split4(val, hi, lo);
                lds_st<bf16x4>(LMH + img_slot(q, 4 * kt + g), hi);
                lds_st<bf16x4>(LML + img_slot(q, 4 * kt + g), lo);
                if (blk_mt) *reinterpret_cast<f32x4*>(blk_mt + q * C + 16 * kt + 4 * g) = val;
            }
        }
        lds_barrier();

        // ---- dGamma_Q^T = S [g | h]^T + Gamma_K^T mt^T: dacc[t][qt] rows = components 16 (TW w + t) + 4 g + i,
        // column = q 16 qt + r
        {
            bf16x8 sdh[TW][4], sdl[TW][4];
#pragma unroll
            for (int t = 0; t < TW; ++t)
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    float b[8];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        b[e] = psd[t][ks][0][e];
                        b[4 + e] = psd[t][ks][1][e];
                    }
                    split_bf16x8(b, sdh[t][ks], sdl[t][ks]);
                }
            f32x4 dacc[TW][4];
#pragma unroll
            for (int t = 0; t < TW; ++t)
#pragma unroll
                for (int qt = 0; qt < 4; ++qt) dacc[t][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int qt = 0; qt < 4; ++qt) {
                    const bf16x8 bh_ = img_row(LGH, 16 * qt + r, ks, g), bl = img_row(LGL, 16 * qt + r, ks, g);
#pragma unroll
                    for (int t = 0; t < TW; ++t) {
                        mma(dacc[t][qt], sdl[t][ks], bh_);
                        mma(dacc[t][qt], sdh[t][ks], bl);
                        mma(dacc[t][qt], sdh[t][ks], bh_);
                    }
                }
#pragma unroll
            for (int ks2 = 0; ks2 < 2; ++ks2) {
                bf16x8 akh[TW], akl[TW];
#pragma unroll
                for (int t = 0; t < TW; ++t) {
                    akh[t] = img_tr(LKH, TW * w + t, ks2, lane);
                    akl[t] = img_tr(LKL, TW * w + t, ks2, lane);
                }
#pragma unroll
                for (int qt = 0; qt < 4; ++qt) {
                    if (ks2 == 1 && qt < 2) continue;   // mt = 0 above the diagonal
                    const bf16x8 bh_ = img_row_perm(LMH, 16 * qt + r, ks2, g), bl = img_row_perm(LML, 16 * qt + r, ks2, g);
#pragma unroll
                    for (int t = 0; t < TW; ++t) {
                        mma(dacc[t][qt], akl[t], bh_);
                        mma(dacc[t][qt], akh[t], bl);
                        mma(dacc[t][qt], akh[t], bh_);
                    }
                }
            }
#pragma unroll
            for (int qt = 0; qt < 4; ++qt) {
                const float hq = s_h[16 * qt + r];
#pragma unroll
                for (int t = 0; t < TW; ++t) {
                    const int comp0 = 16 * (TW * w + t) + 4 * g;
#pragma unroll
                    for (int i = 0; i < 4; ++i) dacc[t][qt][i] += hq * s_z[comp0 + i];
                }
            }
            finish_dgamma<TW, W>(dacc, LQH, LQL, s_part, dgq + (bh * N + n0) * KC, nv, w, lane, emit_dl);
        }
    }
    if (rt) {
        float* seg_rec = rt + (bh * groups + c0 / per) * rec;
#pragma unroll
        for (int t = 0; t < TW; ++t) {
            float* row = seg_rec + (int64_t)(16 * (TW * w + t) + r) * dva;
#pragma unroll
            for (int vt = 0; vt < 8; ++vt) *reinterpret_cast<f32x4*>(row + 16 * vt + 4 * g) = racc[vt][t];
            if (g == 0) *reinterpret_cast<f32x4*>(row + VC) = racc[8][t];
        }
    }
}

// ---------------------------------------------------------------------------------- fused chunk, key side
// The key-side chunk work of the causal backward in one kernel (bf16 storage, K = d_v = 128).  From the
// recomputed posteriors, V, dO, the per-row pairs rs = (1 / den, h) and the state after the chunk
// R = [Rv | r] (the exclusive suffix over chunks of Gamma_Q^T [g | h]), per chunk of 64 tokens:
//   ac = tril(Gamma_Q Gamma_K^T),  mt = tril([g | h] [V | 1]^T)      (recomputed, never stored)
//   dV       = Gamma_K Rv + ac^T g
//   dGamma_K = [V | 1] R^T + mt^T Gamma_Q
// Layout, ownership and work split follow the query-side kernel: the wave's d_v tiles for dV, its
// component tiles for dGamma_K; both outputs formed transposed so that each lane stores contiguous bytes.
template <int KC, int VC, int W>
__global__ void __launch_bounds__(W * 64) bwd_chunk_k_kernel(const float* gq, const float* gk, const void* v,
                                                             const void* dout, const float* rs, const float* rt,
                                                             float* dgk, void* dv, int64_t N, int64_t n_st, int per,
                                                             int dva, int emit_dl) {
    static_assert(KC == 128 && VC == 128, "one 256-byte image row per token");
    using CS = ChunkSplit<W>;
    constexpr int TW = CS::TW, QW = CS::QW, RPW = CS::RPW;
    constexpr int C = 64;
    constexpr int IMG = C * 256;
    __shared__ __attribute__((aligned(16))) char s_q[2 * IMG];   // Gamma_Q hi, lo
    __shared__ __attribute__((aligned(16))) char s_k[2 * IMG];   // Gamma_K hi, lo
    __shared__ __attribute__((aligned(16))) char s_v[IMG];       // V
    __shared__ __attribute__((aligned(16))) char s_g[2 * IMG];   // g hi, lo
    __shared__ __attribute__((aligned(16))) char s_m[2 * IMG];   // ac hi, lo; then mt hi, lo
    __shared__ float s_h[C], s_part[W][C];
    lds_char* const LQH = (lds_char*)s_q;
    lds_char* const LQL = LQH + IMG;
    lds_char* const LKH = (lds_char*)s_k;
    lds_char* const LKL = LKH + IMG;
    lds_char* const LV = (lds_char*)s_v;
    lds_char* const LGH = (lds_char*)s_g;
    lds_char* const LGL = LGH + IMG;
    lds_char* const LMH = (lds_char*)s_m;
    lds_char* const LML = LMH + IMG;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int qw = w / QW, kp = w % QW;
    const int64_t groups = (n_st + per - 1) / per;
    const int64_t bh = blockIdx.x / groups;
    const int64_t c0 = (blockIdx.x % groups) * per;
    const int64_t c1 = c0 + per < n_st ? c0 + per : n_st;
    const int64_t rec = (int64_t)KC * dva;

    // token operands of one chunk, loaded a chunk ahead (rows as in the query-side kernel); rs of the
    // V / dO rows
    f32x4 pq[RPW / 2], pk[RPW / 2];
    u32x4 pv[RPW / 4], pd[RPW / 4];
    float pr0[RPW / 4], pr1[RPW / 4];
    auto fetch = [&](int64_t c) {
        const int64_t n0 = c * C;
        const int nv = (int)(N - n0 < C ? N - n0 : C);
        const float* gqh = gq + (bh * N + n0) * KC;
        const float* gkh = gk + (bh * N + n0) * KC;
        const uint16_t* vh = reinterpret_cast<const uint16_t*>(v) + (bh * N + n0) * VC;
        const uint16_t* dh = reinterpret_cast<const uint16_t*>(dout) + (bh * N + n0) * VC;
        const int rl = lane >> 5, cl = lane & 31;
#pragma unroll
        for (int j = 0; j < RPW / 2; ++j) {
            const int row = RPW * w + 2 * j + rl;
            pq[j] = row < nv ? *reinterpret_cast<const f32x4*>(gqh + (int64_t)row * KC + 4 * cl) : f32x4{0.f, 0.f, 0.f, 0.f};
            pk[j] = row < nv ? *reinterpret_cast<const f32x4*>(gkh + (int64_t)row * KC + 4 * cl) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int bb = 0; bb < RPW / 4; ++bb) {
            const int row = RPW * w + 4 * bb + (lane >> 4), ch = lane & 15;
            const bool ok = row < nv;
            pv[bb] = ok ? *reinterpret_cast<const u32x4*>(vh + (int64_t)row * VC + 8 * ch) : u32x4{0u, 0u, 0u, 0u};
            pd[bb] = ok ? *reinterpret_cast<const u32x4*>(dh + (int64_t)row * VC + 8 * ch) : u32x4{0u, 0u, 0u, 0u};
            pr0[bb] = ok ? rs[(bh * N + n0 + row) * 2] : 0.f;
            pr1[bb] = ok ? rs[(bh * N + n0 + row) * 2 + 1] : 0.f;
        }
    };

    fetch(c0);
    for (int64_t c = c0; c < c1; ++c) {
        const int64_t n0 = c * C;
        const int nv = (int)(N - n0 < C ? N - n0 : C);
        if (c > c0) lds_barrier();   // every wave is done with the previous chunk's images

        // ---- stage: Gamma_Q, Gamma_K, V, g = dO / den, h
        {
            const int rl = lane >> 5, cl = lane & 31;
#pragma unroll
            for (int j = 0; j < RPW / 2; ++j) {
                const int off = img_slot(RPW * w + 2 * j + rl, cl);
                bf16x4 hi, lo;
                split4(pq[j], hi, lo);
                lds_st<bf16x4>(LQH + off, hi);
                lds_st<bf16x4>(LQL + off, lo);
                split4(pk[j], hi, lo);
                lds_st<bf16x4>(LKH + off, hi);
                lds_st<bf16x4>(LKL + off, lo);
            }
        }
#pragma unroll
        for (int bb = 0; bb < RPW / 4; ++bb) {
            const int row = RPW * w + 4 * bb + (lane >> 4), ch = lane & 15;
            lds_st<u32x4>(LV + img_chunk(row, ch), pv[bb]);
            const bf16x8 dv8 = __builtin_bit_cast(bf16x8, pd[bb]);
            float gv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) gv[e] = (float)dv8[e] * pr0[bb];
            bf16x8 hi, lo;
            split_bf16x8(gv, hi, lo);
            lds_st<bf16x8>(LGH + img_chunk(row, ch), hi);
            lds_st<bf16x8>(LGL + img_chunk(row, ch), lo);
            if (ch == 0) s_h[row] = pr1[bb];
        }
        // the state after this chunk, loaded now and split where it is used: for dV (rows 32 ks + 8 g + e,
        // the wave's d_v columns 16 (TW w + t) + r), for dGamma_K (the wave's component rows 16 (TW w + t) +
        // r, columns 32 ks + 8 g .. + 7, and the r column of rows 16 (TW w + t) + 4 g + i)
        const float* R = rt + (bh * n_st + c) * rec;
        float prn[TW][4][8];
        f32x4 prd[TW][4][2];
        float prr[TW][4];
#pragma unroll
        for (int t = 0; t < TW; ++t) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
                for (int e = 0; e < 8; ++e) prn[t][ks][e] = R[(int64_t)(32 * ks + 8 * g + e) * dva + 16 * (TW * w + t) + r];
                const float* p = R + (int64_t)(16 * (TW * w + t) + r) * dva + 32 * ks + 8 * g;
                prd[t][ks][0] = *reinterpret_cast<const f32x4*>(p);
                prd[t][ks][1] = *reinterpret_cast<const f32x4*>(p + 4);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) prr[t][i] = R[(int64_t)(16 * (TW * w + t) + 4 * g + i) * dva + VC];
        }
        if (c + 1 < c1) fetch(c + 1);
        lds_barrier();

        // ---- ac^T = Gamma_K Gamma_Q^T, q tile qw, key tiles kp (mod QW), into the block image (rows q)
        {
            const int q = 16 * qw + r;
            f32x4 acc[4];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) acc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8 bh_ = img_row(LQH, q, ks, g), bl = img_row(LQL, q, ks, g);
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) {
                    if (kt % QW != kp || kt > qw) continue;
                    const bf16x8 ah = img_row(LKH, 16 * kt + r, ks, g), al = img_row(LKL, 16 * kt + r, ks, g);
                    mma(acc[kt], al, bh_);
                    mma(acc[kt], ah, bl);
                    mma(acc[kt], ah, bh_);
                }
            }
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                if (kt % QW != kp) continue;
                f32x4 val;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = 16 * kt + 4 * g + i;
                    val[i] = (kt <= qw && key <= q) ? acc[kt][i] : 0.f;
                }
                bf16x4 hi, lo;
                split4(val, hi, lo);
                lds_st<bf16x4>(LMH + img_slot(q, 4 * kt + g), hi);
                lds_st<bf16x4>(LML + img_slot(q, 4 * kt + g), lo);
            }
        }
        lds_barrier();

        // ---- dV^T = Rv^T Gamma_K^T + g^T ac: vacc[t][kt] rows = d_v 16 (TW w + t) + 4 g + i, column = key 16 kt + r
        {
            bf16x8 anh[TW][4], anl[TW][4];
#pragma unroll
            for (int t = 0; t < TW; ++t)
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) split_bf16x8(prn[t][ks], anh[t][ks], anl[t][ks]);
            f32x4 vacc[TW][4];
#pragma unroll
            for (int t = 0; t < TW; ++t)
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) vacc[t][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) {
                    const bf16x8 bh_ = img_row(LKH, 16 * kt + r, ks, g), bl = img_row(LKL, 16 * kt + r, ks, g);
#pragma unroll
                    for (int t = 0; t < TW; ++t) {
                        mma(vacc[t][kt], anl[t][ks], bh_);
                        mma(vacc[t][kt], anh[t][ks], bl);
                        mma(vacc[t][kt], anh[t][ks], bh_);
                    }
                }
#pragma unroll
            for (int tk = 0; tk < 2; ++tk) {
                bf16x8 agh[TW], agl[TW];
#pragma unroll
                for (int t = 0; t < TW; ++t) {
                    agh[t] = img_tr(LGH, TW * w + t, tk, lane);
                    agl[t] = img_tr(LGL, TW * w + t, tk, lane);
                }
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) {
                    if (tk == 0 && kt >= 2) continue;   // queries 0 .. 31 see no key of these tiles
                    const bf16x8 bh_ = img_tr(LMH, kt, tk, lane), bl = img_tr(LML, kt, tk, lane);
#pragma unroll
                    for (int t = 0; t < TW; ++t) {
                        mma(vacc[t][kt], agl[t], bh_);
                        mma(vacc[t][kt], agh[t], bl);
                        mma(vacc[t][kt], agh[t], bh_);
                    }
                }
            }
            uint16_t* dvh = reinterpret_cast<uint16_t*>(dv) + (bh * N + n0) * VC;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                const int key = 16 * kt + r;
                if (key >= nv) continue;
#pragma unroll
                for (int t = 0; t < TW; ++t)
                    *reinterpret_cast<bf16x4*>(dvh + (int64_t)key * VC + 16 * (TW * w + t) + 4 * g) = pack4(vacc[t][kt]);
            }
        }
        lds_barrier();   // ac no longer read

        // ---- mt^T = [V | 1] [g | h]^T, q tile qw, key tiles kp (mod QW), into the block image (rows q)
        {
            const int q = 16 * qw + r;
            const float hq = s_h[q];
            f32x4 macc[4];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) macc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8 bh_ = img_row(LGH, q, ks, g), bl = img_row(LGL, q, ks, g);
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) {
                    if (kt % QW != kp || kt > qw) continue;
                    const bf16x8 av = img_row(LV, 16 * kt + r, ks, g);
                    mma(macc[kt], av, bl);
                    mma(macc[kt], av, bh_);
                }
            }
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                if (kt % QW != kp) continue;
                f32x4 val;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = 16 * kt + 4 * g + i;
                    val[i] = (kt <= qw && key <= q && key < nv) ? macc[kt][i] + hq : 0.f;
                }
                bf16x4 hi, lo;
                split4(val, hi, lo);
                lds_st<bf16x4>(LMH + img_slot(q, 4 * kt + g), hi);
                lds_st<bf16x4>(LML + img_slot(q, 4 * kt + g), lo);
            }
        }
        lds_barrier();

        // ---- dGamma_K^T = R [V | 1]^T + Gamma_Q^T mt: kacc[t][kt] rows = components 16 (TW w + t) + 4 g + i,
        // column = key 16 kt + r
        {
            bf16x8 adh[TW][4], adl[TW][4];
#pragma unroll
            for (int t = 0; t < TW; ++t)
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    float b[8];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        b[e] = prd[t][ks][0][e];
                        b[4 + e] = prd[t][ks][1][e];
                    }
                    split_bf16x8(b, adh[t][ks], adl[t][ks]);
                }
            f32x4 kacc[TW][4];
#pragma unroll
            for (int t = 0; t < TW; ++t)
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) kacc[t][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) {
                    const bf16x8 bv = img_row(LV, 16 * kt + r, ks, g);
#pragma unroll
                    for (int t = 0; t < TW; ++t) {
                        mma(kacc[t][kt], adl[t][ks], bv);
                        mma(kacc[t][kt], adh[t][ks], bv);
                    }
                }
#pragma unroll
            for (int tk = 0; tk < 2; ++tk) {
                bf16x8 aqh[TW], aql[TW];
#pragma unroll
                for (int t = 0; t < TW; ++t) {
                    aqh[t] = img_tr(LQH, TW * w + t, tk, lane);
                    aql[t] = img_tr(LQL, TW * w + t, tk, lane);
                }
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) {
                    if (tk == 0 && kt >= 2) continue;   // queries 0 .. 31 see no key of these tiles
                    const bf16x8 bh_ = img_tr(LMH, kt, tk, lane), bl = img_tr(LML, kt, tk, lane);
#pragma unroll
                    for (int t = 0; t < TW; ++t) {
                        mma(kacc[t][kt], aql[t], bh_);
                        mma(kacc[t][kt], aqh[t], bl);
                        mma(kacc[t][kt], aqh[t], bh_);
                    }
                }
            }
            // the r column of R: keys past N get none (their [V | 1] row is zero)
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                const bool valid = 16 * kt + r < nv;
#pragma unroll
                for (int t = 0; t < TW; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) kacc[t][kt][i] += valid ? prr[t][i] : 0.f;
            }
            finish_dgamma<TW, W>(kacc, LKH, LKL, s_part, dgk + (bh * N + n0) * KC, nv, w, lane, emit_dl);
        }
    }
}

// ---------------------------------------------------------------------------------- scans
// In place over the n chunk entries of each (batch, head), entry stride rec floats: mode 0 exclusive
// prefix, mode 1 exclusive suffix, mode 2 total (into entry 0).  A thread owns four consecutive state
// elements (one 16-byte access per entry; rec is a multiple of four) and walks the entries
// sequentially, in groups of 16 independent loads followed by the group's running sums, so that
// loads are in flight back to back.  Each element is summed in entry order.
__global__ void __launch_bounds__(64) bwd_scan_kernel(float* st, int64_t n, int64_t rec, int mode) {
    const int64_t rec4 = rec / 4;
    const int64_t per = (rec4 + 63) / 64;   // workgroups per (batch, head)
    const int64_t e = ((int64_t)blockIdx.x % per) * 64 + threadIdx.x;
    if (e >= rec4) return;
    f32x4* base = reinterpret_cast<f32x4*>(st + ((int64_t)blockIdx.x / per) * n * rec) + e;
    f32x4 run = {0.f, 0.f, 0.f, 0.f};
    for (int64_t c0 = 0; c0 < n; c0 += 16) {
        f32x4 x[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int64_t c = mode == 1 ? n - 1 - (c0 + j) : c0 + j;   // suffix: entries from the end
            x[j] = (c0 + j < n) ? base[c * rec4] : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        if (mode == 2) {
#pragma unroll
            for (int j = 0; j < 16; ++j) run += x[j];
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int64_t c = mode == 1 ? n - 1 - (c0 + j) : c0 + j;
                if (c0 + j < n) base[c * rec4] = run;
                run += x[j];
            }
        }
    }
    if (mode == 2) base[0] = run;
}

// ---------------------------------------------------------------------------------- parameters
// gp [2][B * H][n_seg][K][dxa]: the partial records of a head, nt = 2 B n_seg of them, summed per
// element into gs [H][K][dxa]:
//   G1 = sum dl x_d, G2 = sum dl x_d^2, G0 = sum dl
//   dmu = (G1 - mu G0) / s, ds = ((G2 - 2 mu G1 + mu^2 G0) / s^2 - G0 / s) / 2, draw_var = ds sigmoid(rho)
constexpr int kParamBatch = 16;  // partial loads in flight per thread in the parameter reductions

// Workgroup: 64 consecutive elements of one head; wave s sums records s nt / 4 .. (s + 1) nt / 4 - 1
// in order (kParamBatch loads in flight), then the four slices are added in order.
__global__ void __launch_bounds__(256) bwd_param_sum_kernel(const float* gp, float* gs, int64_t B, int H,
                                                            int64_t part, int64_t n_seg) {
    __shared__ float s_acc[4][64];
    const int64_t per = (part + 63) / 64;   // element blocks per head
    const int h = (int)(blockIdx.x / per);
    const int l = threadIdx.x & 63, sl = threadIdx.x >> 6;
    const int64_t e = (blockIdx.x % per) * 64 + l;
    const int64_t nt = 2 * B * n_seg;
    const int64_t a = nt * sl / 4, z = nt * (sl + 1) / 4;
    float acc = 0.f;
    if (e < part) {
        for (int64_t t0 = a; t0 < z; t0 += kParamBatch) {
            float v[kParamBatch];
#pragma unroll
            for (int j = 0; j < kParamBatch; ++j) {
                const int64_t t = t0 + j < z ? t0 + j : z - 1;
                const int64_t q = t / n_seg;
                v[j] = gp[((q * H + h) * n_seg + (t - q * n_seg)) * part + e];
            }
#pragma unroll
            for (int j = 0; j < kParamBatch; ++j)
                if (t0 + j < z) acc += v[j];
        }
    }
    s_acc[sl][l] = acc;
    __syncthreads();
    if (sl == 0 && e < part) gs[(int64_t)h * part + e] = ((s_acc[0][l] + s_acc[1][l]) + s_acc[2][l]) + s_acc[3][l];
}

__global__ void __launch_bounds__(256) bwd_param_kernel(const float* gs, const float* mu, const float* raw_var,
                                                        float* dmu, float* draw_var, int H, int K, int d_r, int dxa) {
    const int per = (K * d_r + 255) / 256;   // workgroups per head
    const int h = blockIdx.x / per;
    const int e = (blockIdx.x % per) * 256 + threadIdx.x;
    if (e >= K * d_r) return;
    const int k = e / d_r, d = e % d_r;
    const float* p = gs + ((int64_t)h * K + k) * dxa;
    const float g1 = p[d], g2 = p[d_r + d], g0 = p[2 * d_r];
    const int64_t pe = (int64_t)h * K * d_r + e;
    const float m = mu[pe], rv = raw_var[pe];
    const float s = fmaxf(rv, 0.f) + log1pf(expf(-fabsf(rv)));
    const float wv = 1.f / s;
    dmu[pe] = (g1 - m * g0) * wv;
    const float ds = 0.5f * ((g2 - 2.f * m * g1 + m * m * g0) * wv * wv - g0 * wv);
    draw_var[pe] = ds / (1.f + expf(-rv));
}

// dlog pi_k = G0_k; dprior_logits_k = G0_k - pi_k sum_j G0_j
__global__ void __launch_bounds__(256) bwd_prior_kernel(const float* gs, const float* prior, float* dprior, int H,
                                                        int K, int d_r, int dxa) {
    const int h = blockIdx.x, tid = threadIdx.x;
    __shared__ float s_g[256];
    __shared__ float s_p[256];
    if (tid < K) {
        s_g[tid] = gs[((int64_t)h * K + tid) * dxa + 2 * d_r];
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

template <int KT>
void gamma_mfma_dispatch(const void* x, bool f32, const float* bf, const double* cq, float* gamma, int64_t BH,
                         int64_t N, int H, int K, int d_r, hipStream_t s) {
    // row groups per wave (fp64 accumulators: 8 G KT registers); at KT = 8 one group measured faster than
    // two (816 -> 806 us at B1 H16 N65536 K128: twice the workgroups, half the accumulators)
    constexpr int G = KT <= 4 ? 2 : 1;
    const dim3 grid((unsigned)((N + 64 * G - 1) / (64 * G) * BH));
    const int vecx = (reinterpret_cast<uintptr_t>(x) % 16 == 0 && d_r % 4 == 0) ? 1 : 0;
    if (f32) bwd_gamma_mfma_kernel<KT, G, true><<<grid, dim3(256), 0, s>>>(x, bf, cq, gamma, N, H, K, d_r, vecx);
    else bwd_gamma_mfma_kernel<KT, G, false><<<grid, dim3(256), 0, s>>>(x, bf, cq, gamma, N, H, K, d_r, vecx);
}

}  // namespace

bool launch_bwd_gemm(const BwdGemm& g0, bool ta, bool tb, bool out_bf16, hipStream_t s) {
    const int64_t tiles = (int64_t)((g0.M + GM - 1) / GM) * ((g0.N + GN - 1) / GN);
    const int64_t grid = tiles * g0.n_inner * g0.n_outer;
    if (grid <= 0) return true;
    BwdGemm g = g0;
    auto vec_ok = [](const float* p, int ld, int64_t s0, int64_t s1, int64_t mod) {
        return reinterpret_cast<uintptr_t>(p) % 16 == 0 && ld % 4 == 0 && s0 % 4 == 0 && s1 % 4 == 0 && mod >= 0;
    };
    // a generated operand's rows start at multiples of d elements: 16-byte loads need d % 8 == 0 (bf16: 8
    // elements, fp32: two loads of 4) and an aligned base
    auto gen_vec = [](const BwdGen& q) { return reinterpret_cast<uintptr_t>(q.src) % 16 == 0 && q.d % 8 == 0; };
    g.vecA = g.ga.kind ? gen_vec(g.ga) : vec_ok(g.A, g.lda, g.sA0, g.sA1, 0);
    g.vecB = g.gb.kind ? gen_vec(g.gb) : vec_ok(g.B, g.ldb, g.sB0, g.sB1, g.modB);
    const dim3 gr((unsigned)grid), bl(256);
    const int ga = g.ga.kind, gb = g.gb.kind;
    if (g.dx_x) {
        if (ta || tb || ga || gb) return false;
        if (out_bf16) bwd_gemm_kernel<false, false, true, GEN_NONE, GEN_NONE, true><<<gr, bl, 0, s>>>(g);
        else bwd_gemm_kernel<false, false, false, GEN_NONE, GEN_NONE, true><<<gr, bl, 0, s>>>(g);
        return true;
    }
    if (ga || gb) {
        if (out_bf16) return false;
        if (ta && !tb && !ga && gb == GEN_XAUG) bwd_gemm_kernel<true, false, false, GEN_NONE, GEN_XAUG><<<gr, bl, 0, s>>>(g);
        else if (ta && !tb && !ga && gb == GEN_VAUG) bwd_gemm_kernel<true, false, false, GEN_NONE, GEN_VAUG><<<gr, bl, 0, s>>>(g);
        else if (ta && !tb && !ga && gb == GEN_GH) bwd_gemm_kernel<true, false, false, GEN_NONE, GEN_GH><<<gr, bl, 0, s>>>(g);
        else if (!ta && !tb && !ga && gb == GEN_VAUG) bwd_gemm_kernel<false, false, false, GEN_NONE, GEN_VAUG><<<gr, bl, 0, s>>>(g);
        else if (!ta && tb && ga == GEN_GH && gb == GEN_VAUG) bwd_gemm_kernel<false, true, false, GEN_GH, GEN_VAUG><<<gr, bl, 0, s>>>(g);
        else if (!ta && tb && ga == GEN_GH && !gb) bwd_gemm_kernel<false, true, false, GEN_GH, GEN_NONE><<<gr, bl, 0, s>>>(g);
        else if (!ta && tb && ga == GEN_VAUG && !gb) bwd_gemm_kernel<false, true, false, GEN_VAUG, GEN_NONE><<<gr, bl, 0, s>>>(g);
        else return false;
        return true;
    }
    if (!ta && !tb) gemm_dispatch<false, false>(g, out_bf16, grid, s);
    else if (!ta && tb) gemm_dispatch<false, true>(g, out_bf16, grid, s);
    else if (ta && !tb) gemm_dispatch<true, false>(g, out_bf16, grid, s);
    else gemm_dispatch<true, true>(g, out_bf16, grid, s);
    return true;
}

void launch_bwd_prep(const float* mu, const float* raw_var, float* mw, int H, int K, int d_r, hipStream_t s) {
    // the backward plan bounds H * ceil(K d_r / 256) by INT32_MAX (this grid and the parameter kernel's)
    bwd_prep_kernel<<<dim3((unsigned)((K * d_r + 255) / 256 * H)), dim3(256), 0, s>>>(mu, raw_var, mw, K, d_r);
}

int bwd_gamma_tiles(int K) {
    const int kt = (K + 15) / 16;
    return kt <= 1 ? 1 : kt <= 2 ? 2 : kt <= 4 ? 4 : kt <= 8 ? 8 : 16;
}

void launch_bwd_frag(const float* mu, const float* raw_var, const float* prior, float* bf, double* cq, int H, int K,
                     int d_r, bool split, hipStream_t s) {
    // H * KT <= 16 H fits the 32-bit grid (the backward plan bounds B * H * 16 by INT32_MAX)
    const int KT = bwd_gamma_tiles(K);
    bwd_frag_kernel<<<dim3((unsigned)(H * KT)), dim3(256), 0, s>>>(mu, raw_var, prior, bf, cq, K, d_r, KT,
                                                                   split ? 1 : 0);
}

bool bwd_gamma_split_supported(int K, int d_r, bool f32) {
    return !f32 && d_r % 32 == 0 && bwd_gamma_tiles(K) * (d_r / 32) <= 32;
}

void launch_bwd_gamma_split(const void* x, const float* bf, const double* cq, float* gamma, int64_t BH, int64_t N,
                            int H, int K, int d_r, hipStream_t s) {
    const int KT = bwd_gamma_tiles(K);
    // two 16-row groups per wave: every fragment read from LDS serves both (four measured slower at KT = 8,
    // 275 -> 289 us at B1 H16 N65536)
    const int rows = 1024;   // a multiple of 64 G
    const dim3 grid((unsigned)((N + rows - 1) / rows * BH)), block(256);
    const uint16_t* xp = reinterpret_cast<const uint16_t*>(x);
    const bf16x8* fr = reinterpret_cast<const bf16x8*>(bf);
    switch (KT) {
        case 1: bwd_gamma_split_kernel<1, 8, 2><<<grid, block, 0, s>>>(xp, fr, cq, gamma, N, H, K, d_r, rows); break;
        case 2: bwd_gamma_split_kernel<2, 8, 2><<<grid, block, 0, s>>>(xp, fr, cq, gamma, N, H, K, d_r, rows); break;
        case 4: bwd_gamma_split_kernel<4, 8, 2><<<grid, block, 0, s>>>(xp, fr, cq, gamma, N, H, K, d_r, rows); break;
        case 8: bwd_gamma_split_kernel<8, 4, 2><<<grid, block, 0, s>>>(xp, fr, cq, gamma, N, H, K, d_r, rows); break;
        // K = 256: one row group per wave (two leave too few registers for the 16 accumulator tiles each)
        default: bwd_gamma_split_kernel<16, 2, 1><<<grid, block, 0, s>>>(xp, fr, cq, gamma, N, H, K, d_r, rows); break;
    }
}

void launch_bwd_gamma_mfma(const void* x, bool f32, const float* bf, const double* cq, float* gamma, int64_t BH,
                           int64_t N, int H, int K, int d_r, hipStream_t s) {
    switch (bwd_gamma_tiles(K)) {
        case 1: gamma_mfma_dispatch<1>(x, f32, bf, cq, gamma, BH, N, H, K, d_r, s); break;
        case 2: gamma_mfma_dispatch<2>(x, f32, bf, cq, gamma, BH, N, H, K, d_r, s); break;
        case 4: gamma_mfma_dispatch<4>(x, f32, bf, cq, gamma, BH, N, H, K, d_r, s); break;
        case 8: gamma_mfma_dispatch<8>(x, f32, bf, cq, gamma, BH, N, H, K, d_r, s); break;
        default: gamma_mfma_dispatch<16>(x, f32, bf, cq, gamma, BH, N, H, K, d_r, s); break;
    }
}

void launch_bwd_gh(const float* p, const void* dout, bool f32, float* rs, int64_t rows, int d_v, int dva, float eps,
                   hipStream_t s) {
    const dim3 grid((unsigned)((rows + 4 * kRowsPerWave - 1) / (4 * kRowsPerWave)));
    if (f32) bwd_gh_kernel<true><<<grid, dim3(256), 0, s>>>(p, dout, rs, rows, d_v, dva, eps);
    else bwd_gh_kernel<false><<<grid, dim3(256), 0, s>>>(p, dout, rs, rows, d_v, dva, eps);
}

void launch_bwd_dl(const float* gamma, float* dg, int64_t rows, int K, hipStream_t s) {
    if (K <= 64)
        bwd_dl_kernel<4><<<dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, s>>>(gamma, dg, rows, K);
    else
        bwd_dl_kernel<1><<<dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s>>>(gamma, dg, rows, K);
}

bool bwd_chunk_q_supported(int K, int d_v, bool f32) { return !f32 && K == 128 && d_v == 128; }

bool launch_bwd_chunk_q(const float* gq, const float* gk, const void* v, const void* dout, const float* stt, float* rs,
                        float* rt, int seg_per, float* ac, float* mt, float* dgq, int64_t BH, int64_t N, int64_t n_st,
                        int K, int d_v, int dva, float eps, bool emit_dl, hipStream_t s) {
    if (!bwd_chunk_q_supported(K, d_v, false) || dva != d_v + 4 || (rt && seg_per < 1)) return false;
    // chunks per workgroup: enough workgroups for every compute unit several times over.  Longer walks
    // amortise the first chunk's unhidden loads: 16 chunks measured 1306 -> 1290 us per launch against 4
    // at B1 H16 N65536 (the key side 1078 -> 1057 us)
    int per = 16;
    while (per > 1 && BH * ((n_st + per - 1) / per) < 1024) per /= 2;
    if (rt) per = seg_per;   // each walk is one state segment, whose total it forms
    const int64_t groups = (n_st + per - 1) / per;
    const dim3 grid((unsigned)(BH * groups));
    // four wavefronts: eight (two per SIMD, half the tiles each) measured no faster (936 vs 944 us per
    // launch at B1 H16 N65536) and spill
    bwd_chunk_q_kernel<128, 128, 4><<<grid, dim3(256), 0, s>>>(gq, gk, v, dout, stt, rs, rt, ac, mt, dgq, N, n_st, per,
                                                                dva, eps, emit_dl ? 1 : 0);
    return true;
}

namespace {
// Calls f(KC, DC) with the padded class of (K, d), d = d_v or d_r, as integral constants.
template <class F>
void bidir_class(int K, int d_v, F&& f) {
    using I32 = std::integral_constant<int, 32>;
    using I64 = std::integral_constant<int, 64>;
    using I128 = std::integral_constant<int, 128>;
    if (K <= 32 && d_v <= 64) f(I32{}, I64{});
    else if (K <= 32) f(I32{}, I128{});
    else if (d_v <= 64) f(I64{}, I64{});
    else f(I64{}, I128{});
}
}  // namespace

namespace {
bool fused_rows_small(int K, int d_r) { return K <= 64 && d_r <= 128 && K % 4 == 0 && d_r % 4 == 0; }
}  // namespace

bool bwd_fused_rows_supported(int K, int d_r, bool f32) {
    return !f32 && ((K == 128 && d_r == 128) || fused_rows_small(K, d_r));
}

int bwd_fused_rows_seg(int64_t BH, int64_t N, int K, int d_r, int min_seg) {
    // the K = d_r = 128 kernel holds one workgroup per compute unit; the small classes' hold three or
    // more (their loads wait in registers), so they take shorter segments for more workgroups
    const int64_t target = (K == 128 && d_r == 128) ? 256 : 1024;
    int seg = 4096;
    while (seg / 2 >= min_seg && BH * ((N + seg - 1) / seg) < target) seg /= 2;
    return seg < min_seg ? min_seg : seg;
}

int bwd_state_segment(int64_t BH, int64_t n_st) {
    int per = 16;
    while (per > 1 && BH * ((n_st + per - 1) / per) < 512) per /= 2;
    return per;
}

bool launch_bwd_chunk_state(const float* gk, const void* v, float* stt, float* seg, int per, bool totals, int64_t BH,
                            int64_t N, int64_t n_st, int K, int d_v, int dva, hipStream_t s) {
    if (!bwd_chunk_q_supported(K, d_v, false) || dva != d_v + 4 || per < 1) return false;
    const int64_t groups = (n_st + per - 1) / per;
    bwd_chunk_state_kernel<128, 128><<<dim3((unsigned)(BH * groups)), dim3(256), 0, s>>>(gk, v, stt, seg, N, n_st, per,
                                                                                        dva, totals ? 1 : 0);
    return true;
}

bool launch_bwd_suffix_state(const float* gq, const void* dout, const float* rs, float* rt, const float* seg, int per,
                             int64_t BH, int64_t N, int64_t n_st, int K, int d_v, int dva, hipStream_t s) {
    if (!bwd_chunk_q_supported(K, d_v, false) || dva != d_v + 4 || per < 1) return false;
    const int64_t groups = (n_st + per - 1) / per;
    bwd_suffix_state_kernel<128, 128><<<dim3((unsigned)(BH * groups)), dim3(256), 0, s>>>(gq, dout, rs, rt, seg, N, n_st,
                                                                                         per, dva);
    return true;
}

bool launch_bwd_chunk_k(const float* gq, const float* gk, const void* v, const void* dout, const float* rs,
                        const float* rt, float* dgk, void* dv, int64_t BH, int64_t N, int64_t n_st, int K, int d_v,
                        int dva, bool emit_dl, hipStream_t s) {
    if (!bwd_chunk_q_supported(K, d_v, false) || dva != d_v + 4) return false;
    int per = 16;   // as the query side
    while (per > 1 && BH * ((n_st + per - 1) / per) < 1024) per /= 2;
    const int64_t groups = (n_st + per - 1) / per;
    const dim3 grid((unsigned)(BH * groups));
    bwd_chunk_k_kernel<128, 128, 4><<<grid, dim3(256), 0, s>>>(gq, gk, v, dout, rs, rt, dgk, dv, N, n_st, per, dva,
                                                                emit_dl ? 1 : 0);
    return true;
}

bool launch_bwd_fused_rows(const float* gamma, const float* dgamma, const void* x, const float* mw, void* dx, float* gp,
                           int64_t BH, int64_t N, int H, int K, int d_r, int dxa, int seg, bool dl_in, hipStream_t s) {
    if (!bwd_fused_rows_supported(K, d_r, false) || seg % kFusedChunk != 0 || dxa < 2 * d_r + 1) return false;
    const int64_t n_seg = (N + seg - 1) / seg;
    const dim3 grid((unsigned)(BH * n_seg));
    if (!(K == 128 && d_r == 128)) {
        // the small classes: (K, d_r) padded as the bidirectional kernels pad (K, d_v)
        bidir_class(K, d_r, [&](auto kc, auto dc) {
            constexpr int KC = decltype(kc)::value, DRC = decltype(dc)::value;
            if (dl_in)
                bwd_rows_small_kernel<KC, DRC, true><<<grid, dim3(256), 0, s>>>(gamma, dgamma, x, mw, dx, gp, N, H, K,
                                                                               d_r, seg, n_seg, dxa);
            else
                bwd_rows_small_kernel<KC, DRC, false><<<grid, dim3(256), 0, s>>>(gamma, dgamma, x, mw, dx, gp, N, H, K,
                                                                                d_r, seg, n_seg, dxa);
        });
        return true;
    }
    if (dl_in)
        bwd_fused_rows_kernel<128, 128, true><<<grid, dim3(256), 0, s>>>(gamma, dgamma, x, mw, dx, gp, N, H, seg, n_seg,
                                                                          dxa);
    else
        bwd_fused_rows_kernel<128, 128, false><<<grid, dim3(256), 0, s>>>(gamma, dgamma, x, mw, dx, gp, N, H, seg, n_seg,
                                                                           dxa);
    return true;
}

bool bwd_bidir_small_supported(int K, int d_v, bool f32) {
    return !f32 && K <= 64 && d_v <= 128 && K % 4 == 0 && d_v % 4 == 0;
}


bool launch_bwd_bidir_state(const float* gk, const void* v, float* st, int64_t BH, int64_t N, int K, int d_v, int dva,
                            int seg, hipStream_t s) {
    if (!bwd_bidir_small_supported(K, d_v, false) || dva != d_v + 4 || seg % kFusedChunk != 0) return false;
    const int64_t n_seg = (N + seg - 1) / seg;
    bidir_class(K, d_v, [&](auto kc, auto vc) {
        bwd_bidir_state_kernel<decltype(kc)::value, decltype(vc)::value>
            <<<dim3((unsigned)(BH * n_seg)), dim3(256), 0, s>>>(gk, v, st, N, K, d_v, dva, seg, n_seg);
    });
    return true;
}

bool launch_bwd_bidir_q(const float* gq, const void* dout, const float* st, float* dgq, float* r_seg, int64_t BH,
                        int64_t N, int K, int d_v, int dva, int seg, float eps, bool emit_dl, hipStream_t s) {
    if (!bwd_bidir_small_supported(K, d_v, false) || dva != d_v + 4 || seg % kFusedChunk != 0) return false;
    const int64_t n_seg = (N + seg - 1) / seg;
    const dim3 grid((unsigned)(BH * n_seg));
    bidir_class(K, d_v, [&](auto kc, auto vc) {
        constexpr int KC = decltype(kc)::value, VC = decltype(vc)::value;
        if (emit_dl)
            bwd_bidir_q_kernel<KC, VC, true><<<grid, dim3(256), 0, s>>>(gq, dout, st, dgq, r_seg, N, K, d_v, dva, seg,
                                                                       n_seg, eps);
        else
            bwd_bidir_q_kernel<KC, VC, false><<<grid, dim3(256), 0, s>>>(gq, dout, st, dgq, r_seg, N, K, d_v, dva, seg,
                                                                        n_seg, eps);
    });
    return true;
}

bool launch_bwd_bidir_k(const float* gk, const void* v, const float* r_seg, float* dgk, void* dv, int64_t BH, int64_t N,
                        int K, int d_v, int dva, int seg, bool emit_dl, hipStream_t s) {
    if (!bwd_bidir_small_supported(K, d_v, false) || dva != d_v + 4 || seg % kFusedChunk != 0) return false;
    const int64_t n_seg = (N + seg - 1) / seg;
    const dim3 grid((unsigned)(BH * n_seg));
    bidir_class(K, d_v, [&](auto kc, auto vc) {
        constexpr int KC = decltype(kc)::value, VC = decltype(vc)::value;
        if (emit_dl)
            bwd_bidir_k_kernel<KC, VC, true><<<grid, dim3(256), 0, s>>>(gk, v, r_seg, dgk, dv, N, K, d_v, dva, seg, n_seg);
        else
            bwd_bidir_k_kernel<KC, VC, false><<<grid, dim3(256), 0, s>>>(gk, v, r_seg, dgk, dv, N, K, d_v, dva, seg,
                                                                        n_seg);
    });
    return true;
}

void launch_bwd_scan(float* st, int64_t n_outer, int64_t n, int64_t rec, int mode, hipStream_t s) {
    bwd_scan_kernel<<<dim3((unsigned)((rec / 4 + 63) / 64 * n_outer)), dim3(64), 0, s>>>(st, n, rec, mode);
}

void launch_bwd_param(const float* gp, float* gs, const float* mu, const float* raw_var, const float* prior,
                      float* dmu, float* draw_var, float* dprior, int64_t B, int H, int K, int d_r, int dxa,
                      int64_t n_seg, hipStream_t s) {
    const int64_t part = (int64_t)K * dxa;
    bwd_param_sum_kernel<<<dim3((unsigned)((part + 63) / 64 * H)), dim3(256), 0, s>>>(gp, gs, B, H, part, n_seg);
    bwd_param_kernel<<<dim3((unsigned)((K * d_r + 255) / 256 * H)), dim3(256), 0, s>>>(gs, mu, raw_var, dmu, draw_var,
                                                                                   H, K, d_r, dxa);
    bwd_prior_kernel<<<dim3((unsigned)H), dim3(256), 0, s>>>(gs, prior, dprior, H, K, d_r, dxa);
}

}  // namespace gma
