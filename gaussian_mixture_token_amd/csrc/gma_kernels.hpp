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
//   main_kernel<..., MODE, DMA>
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
//
// Input staging.  DMA = true (bf16 with 8-aligned widths): chunk c+1 is fetched straight from
// HBM into the second half of a double-buffered LDS area (buffer_load_dwordx4 ... lds, 1 KiB per
// instruction, bounds-checked by the buffer descriptor so rows past N read as zeros) while chunk
// c is computed.  X is laid out in MFMA-fragment order (each 1 KiB block is one operand
// fragment); V is kept row-major with a 16-byte-chunk XOR swizzle and read as transposed
// operand fragments with ds_read_b64_tr_b16.  DMA = false: synchronous staging through
// registers (fp32 path and unaligned shapes).
#pragma once
#include <type_traits>

#include "gma_device.hpp"

namespace gma {

enum { MODE_RESP = 0, MODE_AGG = 1, MODE_OUT_BIDIR = 2, MODE_OUT_CAUSAL = 3,
       // token-split kernels only: the aggregate pass also stores every chunk's Gamma_K tile, and the
       // causal output pass reads those tiles instead of recomputing the K-side responsibilities
       MODE_AGG_G = 4, MODE_OUT_CAUSAL_G = 5 };

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
    static constexpr int GES = 2;   // staged Gamma / V element in bf16
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
    void* gk;              // [BH, n_chunks, 64 * KC] bf16 Gamma_K chunk tiles (MODE_AGG_G / MODE_OUT_CAUSAL_G)
    int64_t N;
    int H;
    int P;                 // record stride per head (segments per head, or per round)
    int Pg;                // segments per head launched by this grid (P, or P - 1 for causal aggregates)
    int d_r, d_v, K;
    int seg_chunks;        // chunks of C tokens per segment
    int seg0;              // first segment index of this launch (rounds of the causal token-split pair)
    int64_t gk_ring;       // Gamma_K tiles kept per (batch, head): chunk ch lives in slot ch mod gk_ring
                           // (0: one slot per chunk).  A launch's segments lie in one ring window.
    int vec_x, vec_v, vec_o;  // 16-byte (x, v) / 4-element (o) vector access allowed (register staging)
    float* stat_usage;     // MODE_RESP diagnostics (null: write Gamma): [BH, Pg, K] per-segment usage sums
    uint32_t* stat_count;  //   and hard-assignment counts; Gamma is not written
    int* flags;            // [BH] or null (bf16): set to 1 for a (batch, head) with a row whose logits are
                           // not finite (a routing input or coefficient past the fp16 operand range)
    int has_carry;         // causal: load the carried state (P > 1)
    int bidir_segs;        // bidirectional read pass: segment records to sum in order (0 or 1: record 0
                           // already holds the total)
    float eps;
};

struct PrepArgs {
    const float* mu;        // [H, K, d_r]
    const float* raw_var;   // [H, K, d_r]
    const float* prior;     // [H, K]
    void* ab;               // out
    float* cvec;            // out [H, KC]
    int* flags;             // out [n_flags] zeroed (null: none), for the out-of-range flags of the call
    int64_t n_flags;
    int H, K, d_r;
};

// ---------------------------------------------------------------------------------------------
// prep: softplus variances, log-softmax priors, expanded-quadratic coefficients.
// Grid (H, KC / kPrepComps<DRC>): one workgroup per kPrepComps components of a head, one thread per
// (component, dim) where the padded dims allow it.  [a | b] is written in the exact
// per-lane fragment order the main kernel loads:
//   ab[h][ct][ks][lane][j] = A[comp = 16 ct + lane % 16][k = ks*KS + (lane/16)*(KS/4) + j]
// with A = [a | b] (k < DRC: a_{comp,k}; k >= DRC: b_{comp,k-DRC}).  Pad components get
// a = b = 0 and c = -inf (their posterior is exactly 0); pad dimensions get a = b = 0.
// Softplus and log in fp32 (about one ulp); a, b, the per-dimension terms of c and their sum in
// fp64 (runs of consecutive dims, then a butterfly); every reduction runs in a fixed order.
constexpr int kPrepThreads = 512;
template <int DRC>
constexpr int kPrepComps = (kPrepThreads / DRC >= 16) ? 16 : (kPrepThreads / DRC >= 1 ? kPrepThreads / DRC : 1);
template <bool F32, int KC, int DRC>
__global__ void __launch_bounds__(kPrepThreads) prep_kernel(const PrepArgs p) {
    using T = Tr<F32>;
    constexpr int KS = T::KS;
    constexpr int NKS = 2 * DRC / KS;
    constexpr int EPL = KS / 4;  // elements per lane per fragment
    constexpr int CPB = kPrepComps<DRC>;
    static_assert(KC % CPB == 0 && 16 % CPB == 0, "prep: components per workgroup");
    const int h = blockIdx.x;
    const int comp0 = blockIdx.y * CPB;
    const int tid = threadIdx.x;
    const double LOG2E = 1.4426950408889634073599246810019;
    __shared__ double s_t[CPB][DRC];
    __shared__ double s_lse;
    // clear the call's out-of-range flags (the kernels that follow set them)
    if (p.flags) {
        const int64_t nthr = (int64_t)gridDim.x * gridDim.y * kPrepThreads;
        for (int64_t i = ((int64_t)blockIdx.x * gridDim.y + blockIdx.y) * kPrepThreads + tid; i < p.n_flags; i += nthr)
            p.flags[i] = 0;
    }

    // log-sum-exp of the prior logits of this head, by wave 0 (butterfly reductions, fixed order)
    if (tid < 64) {
        double m = -INFINITY;
        for (int k = tid; k < p.K; k += 64) m = fmax(m, (double)p.prior[(int64_t)h * p.K + k]);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) m = fmax(m, __shfl_xor(m, o, 64));
        double acc = 0.0;
        for (int k = tid; k < p.K; k += 64) acc += exp((double)p.prior[(int64_t)h * p.K + k] - m);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
        if (tid == 0) s_lse = m + log(acc);
    }

    // a, b and the per-dimension terms of c for the CPB components of this workgroup
    for (int e = tid; e < CPB * DRC; e += kPrepThreads) {
        const int cl = e / DRC;
        const int d = e % DRC;
        const int comp = comp0 + cl;
        const int ct = comp / 16;
        // softplus and log in fp32 (about one ulp each); the per-dimension terms of c are summed in
        // fp64 below
        double a = 0.0, b = 0.0, t = 0.0;
        if (comp < p.K && d < p.d_r) {
            const int64_t i = ((int64_t)h * p.K + comp) * p.d_r + d;
            const float r = p.raw_var[i];
            const float varf = fmaxf(r, 0.f) + log1pf(expf(-fabsf(r)));   // softplus
            const double var = varf;
            const double mu = p.mu[i];
            const double inv = 1.0 / var;
            a = -0.5 * LOG2E * inv;
            b = LOG2E * mu * inv;
            t = (double)logf(varf) + mu * mu * inv;
        }
        s_t[cl][d] = t;
        // fragment positions of k = d (a part) and k = DRC + d (b part)
#pragma unroll
        for (int part = 0; part < 2; ++part) {
            const int kk = part * DRC + d;
            const int ks = kk / KS;
            const int lane = (comp & 15) + 16 * ((kk % KS) / EPL);
            const int j = kk % EPL;
            const int64_t idx = (((int64_t)h * (KC / 16) + ct) * NKS + ks) * 64 * EPL + lane * EPL + j;
            const double val = part ? b : a;
            if constexpr (F32) {
                reinterpret_cast<float*>(p.ab)[idx] = (float)val;
            } else {
                reinterpret_cast<_Float16*>(p.ab)[idx] = (_Float16)(float)val;
            }
        }
    }
    __syncthreads();
    // c of the workgroup's components: L threads per component each add a run of DRC / L consecutive
    // dims in order, then a fixed butterfly over the L (the terms past d_r are zero)
    constexpr int L = DRC < 32 ? DRC : 32;
    constexpr int PER = DRC / L;
    static_assert(CPB * L <= kPrepThreads && 64 % L == 0, "prep: threads per component");
    const int cl = tid / L, sub = tid % L;
    double part = 0.0;
    if (tid < CPB * L) {
#pragma unroll
        for (int j = 0; j < PER; ++j) part += s_t[cl][sub * PER + j];
    }
#pragma unroll
    for (int o = L / 2; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
    if (tid < CPB * L && sub == 0) {
        const int comp = comp0 + cl;
        float c = -INFINITY;
        if (comp < p.K) {
            const double logpi = (double)p.prior[(int64_t)h * p.K + comp] - s_lse;
            c = (float)(LOG2E * (logpi - 0.5 * part));
        }
        p.cvec[(int64_t)h * KC + comp] = c;
    }
}

// ---------------------------------------------------------------------------------------------
// Synchronous staging helpers (global -> registers -> LDS).

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
            *reinterpret_cast<f16x8*>(dst) = bf16x8_bits_to_f16x8(raw);
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
// Main kernel.  Grid: BH * Pg workgroups (segment-major inside a head); block: W wavefronts.
//
// Per chunk of C tokens:
//   B0  inputs in LDS (DMA: wait for this wave's prefetch, convert its X blocks bf16 -> fp16 in
//       place, barrier, then start the prefetch of the next chunk)
//       logits^T tiles of the wave's own components for Q and/or K (MFMA), local softmax
//   B1  combine the per-wave (max, sum) pairs -> Gamma; Gamma_Q as operand fragments and
//       Gamma_K as a row-major [token][component] bf16 tile into LDS; denominators over own
//       components; Z update
//   B2  contraction over the wave's own d_v tiles: O = (Gamma_Q Vt + tril(Gamma_Q Gamma_K^T) V) /
//       (Gamma_Q Z + rowsum tril(..) + eps); state += Gamma_K^T [V | 1]
template <bool F32, int KC, int VC, int DRC, int W, int C, int MODE, bool DMA, int WPE>
__global__ void __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(WPE)))
main_kernel(const MainArgs a) {
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
    constexpr int XS = DRC * T::XES + 16;    // register-staged X row stride (bytes)
    constexpr int VTS = C * T::GES + 16;     // register-staged V^T row stride (bytes)
    constexpr bool NEED_Q = (MODE == MODE_RESP) || (MODE == MODE_OUT_BIDIR) || (MODE == MODE_OUT_CAUSAL);
    constexpr bool NEED_K = (MODE == MODE_AGG) || (MODE == MODE_OUT_CAUSAL);
    constexpr bool NEED_V = NEED_K;
    constexpr bool HAS_STATE = (MODE != MODE_RESP);
    constexpr bool OUT = (MODE == MODE_OUT_BIDIR) || (MODE == MODE_OUT_CAUSAL);
    static_assert(NCT % W == 0, "components must split evenly across waves");
    static_assert(MODE == MODE_RESP || NVT % W == 0, "d_v must split evenly across waves");
    static_assert(KC % KS == 0 && C % KS == 0 && (2 * DRC) % KS == 0, "tile shapes");
    static_assert(!DMA || !F32, "LDS DMA staging is the bf16 path");
    static_assert(W <= 4, "the softmax combine maps one wave per lane group");

    // DMA layout of one staging buffer: [X_Q fragments][X_K fragments][V rows]
    constexpr int XFRAG_BYTES = NT * NKS2 * 1024;
    constexpr int VROW_BYTES = C * VC * 2;
    constexpr int OFF_XQ = 0;
    constexpr int OFF_XK = OFF_XQ + (NEED_Q ? XFRAG_BYTES : 0);
    constexpr int OFF_V = OFF_XK + (NEED_K ? XFRAG_BYTES : 0);
    constexpr int RAW_BYTES = OFF_V + (NEED_V ? VROW_BYTES : 0);
    constexpr int CPR = VC / 8;              // 16-byte chunks per V row
    constexpr int RPB = 1024 / (VC * 2);     // V rows per 1 KiB DMA block
    constexpr int NF_X = NT * NKS2;
    // X staging by whole 128-byte row segments (8 rows x 128 B per DMA block) when rows are at least
    // that long: every fetched line is used by one instruction.  Shorter rows (DRC = 32) keep one
    // fragment per block (16 rows x 64 B, which is then a contiguous 1 KiB).
    constexpr bool XSEG = DRC >= 64;
    constexpr int NSEG = DRC / 64;           // 128-byte segments per row
    constexpr int NF_V = VROW_BYTES / 1024;
    constexpr int NF_XALL = (NEED_Q ? NF_X : 0) + (NEED_K ? NF_X : 0);
    constexpr int NF = NF_XALL + (NEED_V ? NF_V : 0);
    // buffer stores per chunk per wave (unconditional, so the count is exact)
    constexpr int NSTORE = OUT ? VT_W * NT : 0;
    static_assert(!DMA || !NEED_V || (VROW_BYTES % 1024 == 0 && 1024 % (VC * 2) == 0), "V DMA blocks");
    // Gamma_K tile in LDS: bf16 path row-major [token][component], rows padded by 32 bytes so that
    // the 16 rows a transposed read touches fall in distinct banks within each half-wave and every
    // address is affine in the component index; fp32 path as ready operand fragments (token rows,
    // and component rows for the state update)
    constexpr int GKR = KC * 2 + 32;         // bytes per Gamma_K row (bf16 path)
    constexpr int GK_BYTES = NEED_K ? (F32 ? (NT * NKQ + NCT * NTK) * 1024 : C * GKR) : 16;

    __shared__ __attribute__((aligned(16))) char s_raw0[DMA ? RAW_BYTES : 16];
    __shared__ __attribute__((aligned(16))) char s_raw1[DMA ? RAW_BYTES : 16];
    __shared__ __attribute__((aligned(16))) char s_xq[(!DMA && NEED_Q) ? C * XS : 16];
    __shared__ __attribute__((aligned(16))) char s_xk[(!DMA && NEED_K) ? C * XS : 16];
    __shared__ __attribute__((aligned(16))) char s_vt[(!DMA && NEED_V) ? VC * VTS : 16];
    __shared__ __attribute__((aligned(16))) char s_gq[OUT ? NT * NKQ * 1024 : 16];
    __shared__ __attribute__((aligned(16))) char s_gk[GK_BYTES];
    __shared__ float s_ms[2][W][C][2];
    __shared__ float s_den[W][C];
    __shared__ __attribute__((aligned(16))) float s_c[KC];   // per-component logit constants c_k
    __shared__ __attribute__((aligned(16))) float s_z[KC];   // running Z (each wave owns its components)
    // diagnostics (MODE_RESP with stat_usage): each wave's largest gamma per row and its component, and
    // the segment's hard-assignment counts
    constexpr bool RESP = MODE == MODE_RESP;
    __shared__ float s_amv[RESP ? W : 1][RESP ? C : 1];
    __shared__ int s_ami[RESP ? W : 1][RESP ? C : 1];
    __shared__ uint32_t s_cnt[RESP ? KC : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
    const int lr = lane & 15;
    const int lg = lane >> 4;
    const int bh = blockIdx.x / a.Pg;
    const int sidx = blockIdx.x % a.Pg;
    const int h = bh % a.H;
    const int64_t N = a.N;
    const int64_t n_chunks = (N + C - 1) / C;
    const int64_t ch0 = (int64_t)sidx * a.seg_chunks;
    const int64_t ch1 = (ch0 + a.seg_chunks < n_chunks) ? ch0 + a.seg_chunks : n_chunks;

    const elem_t* qx = reinterpret_cast<const elem_t*>(a.qx) + (int64_t)bh * N * a.d_r;
    const elem_t* kx = reinterpret_cast<const elem_t*>(a.kx) + (int64_t)bh * N * a.d_r;
    const elem_t* vv = reinterpret_cast<const elem_t*>(a.v) + (int64_t)bh * N * a.d_v;
    elem_t* oo = reinterpret_cast<elem_t*>(a.o) + (int64_t)bh * N * a.d_v;

    // buffer descriptors over this (batch, head) slice.  Every offset is passed as a vector offset
    // (the range check covers only that part), so reads past the end return 0 and stores past the
    // end are dropped.
    i32x4 rs_q, rs_k, rs_v;
    __amdgpu_buffer_rsrc_t rs_o;
    if constexpr (DMA) {
        rs_q = make_rsrc_words(qx, (uint32_t)(N * a.d_r * 2));
        rs_k = make_rsrc_words(kx, (uint32_t)(N * a.d_r * 2));
        rs_v = make_rsrc_words(vv, (uint32_t)(N * a.d_v * 2));
        rs_o = make_rsrc(oo, (uint32_t)(N * a.d_v * 2));
    }
    // responsibilities through buffer stores where the (batch, head)'s Gamma rows fit 31-bit offsets
    // (bit 31 marks a dropped store); otherwise plain stores and a full wait per chunk
    [[maybe_unused]] const bool resp_exact =
        DMA && MODE == MODE_RESP && !a.stat_usage && (uint64_t)N * (uint64_t)a.K * 4u < 0x80000000ull;
    [[maybe_unused]] const bool resp_k4 = (a.K & 3) == 0;
    [[maybe_unused]] __amdgpu_buffer_rsrc_t rs_g;
    if constexpr (DMA && MODE == MODE_RESP)
        rs_g = make_rsrc(resp_exact ? a.gamma + (int64_t)bh * N * a.K : a.gamma, resp_exact ? (uint32_t)(N * a.K * 4) : 0u);

    // XOR swizzle of the 16-byte chunks of a staged X row: rows r and r + 8 of a 16-row fragment use
    // disjoint bank halves, so fragment reads are conflict-free
    auto xswz = [](int row) -> int { return (row & 7) ^ ((row >> 3) & 1); };
    // LDS byte offset, within one matrix's X area, of this lane's fragment for (tt, ks)
    const int xlane0 = ((lr >> 3) * NSEG) * 1024 + (lr & 7) * 128 +
                       (((lg ^ ((lr & 3) ^ ((lr >> 3) & 1))) | (((lr >> 2) & 1) << 2)) << 4);
    const int xlane1 = ((lr >> 3) * NSEG) * 1024 + (lr & 7) * 128 +
                       (((lg ^ ((lr & 3) ^ ((lr >> 3) & 1))) | ((((lr >> 2) & 1) ^ 1) << 2)) << 4);
    auto xfrag_off = [&](int tt, int ks) -> int {
        if constexpr (XSEG) return ((ks & 1) ? xlane1 : xlane0) + (tt * 2 * NSEG + (ks >> 1)) * 1024;
        else return ((tt * NKS2 + ks) * 64 + lane) * 16;
    };

    // ---- DMA issue of chunk ch into a staging buffer (each wave issues every W-th block)
    auto issue_dma = [&](int64_t ch, char* raw) {
        const int64_t n0 = ch * C;
        for (int f = w; f < NF; f += W) {
            if (f < NF_XALL) {
                const bool isq = NEED_Q && f < NF_X;
                const int fx = (NEED_Q && !isq) ? f - NF_X : f;
                uint32_t soff, voff;
                if constexpr (XSEG) {
                    // block fx = (8-row group rb, 128-byte segment sg); lane l -> row rb*8 + l/8, LDS
                    // chunk l%8 holding global chunk (l%8) ^ xswz(row)
                    const int rb = fx / NSEG, sg = fx % NSEG;
                    const int rl = lane >> 3;
                    const int gc = (lane & 7) ^ xswz(rb * 8 + rl);
                    soff = 0;
                    voff = (uint32_t)(((n0 + rb * 8 + rl) * a.d_r + sg * 64 + gc * 8) * 2);
                } else {
                    const int tt = fx / NKS2, ks2 = fx % NKS2;
                    soff = 0;
                    voff = (uint32_t)(((n0 + tt * 16 + lr) * a.d_r + ks2 * 32 + lg * 8) * 2);
                }
                if (isq) dma16(rs_q, raw + OFF_XQ + fx * 1024, voff, soff);
                else dma16(rs_k, raw + OFF_XK + fx * 1024, voff, soff);
            } else if constexpr (NEED_V) {
                const int fv = f - NF_XALL;
                const int r0 = fv * RPB;
                const int rl = lane / CPR;
                const int row = r0 + rl;
                const int gch = (lane % CPR) ^ (row % CPR);
                const uint32_t voff = (uint32_t)(((n0 + row) * a.d_v + gch * 8) * 2);
                dma16(rs_v, raw + OFF_V + fv * 1024, voff, 0);
            }
        }
    };
    // In-place bf16 -> fp16 conversion of the X blocks this wave fetched (same byte layout).
    auto convert_own_x = [&](char* raw) {
        for (int f = w; f < NF_XALL; f += W) {
            char* p = raw + f * 1024 + lane * 16;   // X_Q blocks then X_K blocks, contiguous
            const u32x4 r = *reinterpret_cast<const u32x4*>(p);
            *reinterpret_cast<f16x8*>(p) = bf16x8_bits_to_f16x8(r);
        }
    };

    // ---- per-wave constants: [a | b] fragments of the wave's own components (registers) and the
    // logit constants c (LDS)
    xfrag_t abf[KT_W][NKS];
    {
        const xfrag_t* abg = reinterpret_cast<const xfrag_t*>(a.ab) + (int64_t)h * NCT * NKS * 64;
#pragma unroll
        for (int kt = 0; kt < KT_W; ++kt) {
            const int ct = w * KT_W + kt;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) abf[kt][ks] = abg[((int64_t)ct * NKS + ks) * 64 + lane];
        }
        for (int k = tid; k < KC; k += NTHR) s_c[k] = a.cvec[(int64_t)h * KC + k];
        if constexpr (RESP) {
            for (int k = tid; k < KC; k += NTHR) s_cnt[k] = 0u;
        }
    }
    // diagnostics: this lane's usage sums of its components (over its rows of every chunk)
    [[maybe_unused]] float use[RESP ? KT_W : 1][4] = {};

    // ---- running state: [Vt | Z] columns owned by this wave (all components), Z of own components
    constexpr int ST_T = HAS_STATE ? NCT : 1;
    constexpr int ST_V = HAS_STATE ? VT_W : 1;
    f32x4 st[ST_T][ST_V];
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
        for (int k = tid; k < KC; k += NTHR) s_z[k] = load ? src[(int64_t)KC * VC + k] : 0.f;
        if constexpr (MODE == MODE_OUT_BIDIR) {
            // total over the segment records, added in segment order (the order of the scan kernel)
            for (int t = 1; t < a.bidir_segs; ++t) {
                const float* r = src + (int64_t)t * rec;
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int vt = 0; vt < VT_W; ++vt)
                        st[ct][vt] += *reinterpret_cast<const f32x4*>(r + ((int64_t)(ct * NVT + w * VT_W + vt) * 64 + lane) * 4);
                for (int k = tid; k < KC; k += NTHR) s_z[k] += r[(int64_t)KC * VC + k];
            }
        }
    }
    lds_barrier();   // s_c and s_z visible to every wave

    if constexpr (DMA) {
        if (ch0 < ch1) issue_dma(ch0, s_raw0);
    }

    // byte offset of (row, column) in the bf16 Gamma_K tile
    auto gk_off = [&](int row, int col) -> int { return row * GKR + col * 2; };

    // set on a lane that met a live row whose logits are not finite (bf16: a routing input or a
    // coefficient past the fp16 operand range); the (batch, head) is flagged after the chunk loop
    [[maybe_unused]] bool nonfin = false;

    // ---- one chunk; BUF selects the DMA staging buffer (compile-time, so the two buffers are
    // distinct LDS objects)
    auto body = [&](auto buf_tag, int64_t ch) {
        constexpr int BUF = decltype(buf_tag)::value;
        char* raw = BUF ? s_raw1 : s_raw0;
        char* raw_next = BUF ? s_raw0 : s_raw1;
        const int64_t n0 = ch * C;
        const int rows_valid = (int)((N - n0 < C) ? N - n0 : C);

        // ---- inputs of this chunk in LDS
        if constexpr (DMA) {
            if (ch == ch0) wait_vmcnt<0>();
            else if (RESP && resp_exact) {
                // the previous chunk's Gamma stores were issued after this chunk's DMA: wait for the DMA only
                if (resp_k4) wait_vmcnt<NT * KT_W>();
                else wait_vmcnt<4 * NT * KT_W>();
            } else wait_vmcnt<NSTORE>();
            convert_own_x(raw);
            lds_barrier();
            if (ch + 1 < ch1) issue_dma(ch + 1, raw_next);
        } else {
            if constexpr (NEED_Q) stage_x<F32, C, DRC, NTHR>(s_xq, qx + n0 * a.d_r, rows_valid, a.d_r, a.vec_x, tid);
            if constexpr (NEED_K) stage_x<F32, C, DRC, NTHR>(s_xk, kx + n0 * a.d_r, rows_valid, a.d_r, a.vec_x, tid);
            if constexpr (NEED_V) stage_vt<F32, C, VC, NTHR>(s_vt, vv + n0 * a.d_v, rows_valid, a.d_v, a.vec_v, tid);
            lds_barrier();
        }

        // ---- logits^T tiles for own components: acc[kt][tt] (rows: comps 4g+i of tile ct, col: token 16tt+r)
        // fp32 storage: the matrix cores sum each step of 16 dims (a x^2 + b x, 32 products) in fp32,
        // and the steps are added in fp64 onto c.  The expanded form's terms are large and cancel (the
        // logits of a row are around -100 in log2 units while their differences are a few units), so a
        // single fp32 running sum over 2 d_r products would put about 1e-4 of error into the
        // differences at d_r = 128, and ln 2 / 4 of that into Gamma.
        auto logits = [&](int which, f32x4 (&acc)[KT_W][NT]) {
            [[maybe_unused]] double acc64[F32 ? KT_W : 1][F32 ? NT : 1][4];
#pragma unroll
            for (int kt = 0; kt < KT_W; ++kt) {
                const f32x4 cinit = *reinterpret_cast<const f32x4*>(&s_c[(w * KT_W + kt) * 16 + lg * 4]);
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) {
                    if constexpr (F32) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc64[kt][tt][i] = (double)cinit[i];
                    } else {
                        acc[kt][tt] = cinit;
                    }
                }
            }
#pragma unroll
            for (int ks = 0; ks < NKS2; ++ks) {
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) {
                    xfrag_t xf;
                    if constexpr (DMA) {
                        xf = *reinterpret_cast<const xfrag_t*>(raw + (which ? OFF_XK : OFF_XQ) + xfrag_off(tt, ks));
                    } else {
                        xf = *reinterpret_cast<const xfrag_t*>((which ? s_xk : s_xq) + (tt * 16 + lr) * XS +
                                                               (ks * KS + lg * (KS / 4)) * T::XES);
                    }
                    const xfrag_t x2 = xf * xf;
#pragma unroll
                    for (int kt = 0; kt < KT_W; ++kt) {
                        if constexpr (F32) {
                            f32x4 part = {0.f, 0.f, 0.f, 0.f};
                            mma(part, abf[kt][ks], x2);
                            mma(part, abf[kt][ks + NKS2], xf);
#pragma unroll
                            for (int i = 0; i < 4; ++i) acc64[kt][tt][i] += (double)part[i];
                        } else {
                            mma(acc[kt][tt], abf[kt][ks], x2);
                            mma(acc[kt][tt], abf[kt][ks + NKS2], xf);
                        }
                    }
                }
            }
            if constexpr (F32) {
#pragma unroll
                for (int kt = 0; kt < KT_W; ++kt)
#pragma unroll
                    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[kt][tt][i] = (float)acc64[kt][tt][i];
            }
        };
        f32x4 lq[NEED_Q ? KT_W : 1][NT];
        f32x4 lk[NEED_K ? KT_W : 1][NT];
        if constexpr (NEED_Q) logits(0, lq);
        if constexpr (NEED_K) logits(1, lk);

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
        lds_barrier();

        // ---- softmax part 2: combine the W partial (max, sum) pairs; scale to posteriors.
        // Rows past the end of the sequence get the factor 0 (their logits are finite: the
        // staged inputs of those rows are zeros).
        auto finish_softmax = [&](f32x4 (&acc)[KT_W][NT], const float (&mloc)[NT], int which) {
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                const int tok = tt * 16 + lr;
                // lane group g combines the partial of wave g (W <= 4): M = max_g m_g,
                // S = sum_g s_g 2^(m_g - M)
                const float mg = (lg < W) ? s_ms[which][lg < W ? lg : 0][tok][0] : -INFINITY;
                const float sg = (lg < W) ? s_ms[which][lg < W ? lg : 0][tok][1] : 0.f;
                const float M = group4_max(mg);
                const float S = group4_sum(mg == -INFINITY ? 0.f : sg * fast_exp2(mg - M));
                // a row maximum of -inf or NaN, or a NaN row sum (the maximum skips NaN logits)
                if constexpr (!F32) nonfin |= (tok < rows_valid) && !(M > -INFINITY && S < INFINITY);
                const bool live = mloc[tt] != -INFINITY && tok < rows_valid;
                const float f = live ? fast_exp2(mloc[tt] - M) * fast_rcp(S) : 0.f;
#pragma unroll
                for (int kt = 0; kt < KT_W; ++kt) acc[kt][tt] *= f;
            }
        };
        if constexpr (NEED_Q) finish_softmax(lq, mq, 0);
        if constexpr (NEED_K) finish_softmax(lk, mk, 1);

        if constexpr (MODE == MODE_RESP) {
            if (a.stat_usage) {
                // diagnostics instead of Gamma rows: usage sums of own components (rows past the end and
                // pad components have gamma 0), and each row's largest gamma over own components, then
                // over the lane groups (ties to the lowest component)
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) {
                    const int tok = tt * 16 + lr;
                    float best = -1.f;
                    int bi = 0x7fffffff;
#pragma unroll
                    for (int kt = 0; kt < KT_W; ++kt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int c = (w * KT_W + kt) * 16 + lg * 4 + i;
                            const float g = lq[kt][tt][i];
                            use[kt][i] += g;
                            if (c < a.K && g > best) {
                                best = g;
                                bi = c;
                            }
                        }
#pragma unroll
                    for (int o = 16; o < 64; o <<= 1) {
                        const float ob = __shfl_xor(best, o, 64);
                        const int oi = __shfl_xor(bi, o, 64);
                        if (ob > best || (ob == best && oi < bi)) {
                            best = ob;
                            bi = oi;
                        }
                    }
                    if (lg == 0) {
                        s_amv[w][tok] = best;
                        s_ami[w][tok] = bi;
                    }
                }
                lds_barrier();
                // the row's component over the waves (in wave order: the lowest component on ties); a row
                // whose gammas are not finite (flagged, recomputed afterwards) counts nowhere
                for (int tok = tid; tok < rows_valid; tok += NTHR) {
                    float best = s_amv[0][tok];
                    int bi = s_ami[0][tok];
                    for (int v = 1; v < W; ++v) {
                        const float ob = s_amv[v][tok];
                        const int oi = s_ami[v][tok];
                        if (ob > best || (ob == best && oi < bi)) {
                            best = ob;
                            bi = oi;
                        }
                    }
                    if (bi < a.K) atomicAdd(&s_cnt[bi], 1u);
                }
                if constexpr (!DMA) lds_barrier();  // staging buffers are rewritten by the next chunk
                return;
            }
            // Gamma rows out: lane holds comps 16ct + 4g .. +3 of token 16tt + r.  DMA path: buffer stores, the
            // same number on every lane and chunk (rows past N fall past the descriptor's range, pad
            // components get bit 31 of the offset; both are dropped), so that the next chunk can wait for
            // its own DMA alone
            if constexpr (DMA) {
                if (resp_exact) {
#pragma unroll
                    for (int tt = 0; tt < NT; ++tt) {
                        const uint32_t rowb = (uint32_t)(n0 + tt * 16 + lr) * (uint32_t)a.K * 4u;
#pragma unroll
                        for (int kt = 0; kt < KT_W; ++kt) {
                            const int c0 = (w * KT_W + kt) * 16 + lg * 4;
                            if (resp_k4) {
                                const uint32_t off = (rowb + (uint32_t)c0 * 4u) | (c0 + 4 <= a.K ? 0u : 0x80000000u);
                                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, lq[kt][tt]), rs_g, off, 0, 0);
                            } else {
#pragma unroll
                                for (int i = 0; i < 4; ++i) {
                                    const uint32_t off = (rowb + (uint32_t)(c0 + i) * 4u) | (c0 + i < a.K ? 0u : 0x80000000u);
                                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lq[kt][tt][i]), rs_g, off, 0, 0);
                                }
                            }
                        }
                    }
                    return;
                }
            }
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
            if constexpr (!DMA) lds_barrier();  // staging buffers are rewritten by the next chunk
            return;
        }

        // ---- Gamma to LDS; denominators from the carried Z
        if constexpr (OUT) {
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
            f32x4 zown[KT_W];
#pragma unroll
            for (int kt = 0; kt < KT_W; ++kt)
                zown[kt] = *reinterpret_cast<const f32x4*>(&s_z[(w * KT_W + kt) * 16 + lg * 4]);
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
#pragma unroll
            for (int kt = 0; kt < KT_W; ++kt) {
                const int ct = w * KT_W + kt;
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) {
                    if constexpr (F32) {
                        // token-row fragments (for S^T) ...
                        if constexpr (MODE == MODE_OUT_CAUSAL)
                            *reinterpret_cast<f32x4*>(s_gk + ((tt * NKQ + ct) * 64 + lane) * 16) = lk[kt][tt];
                        // ... and component-row fragments (for the state update), slots matching the V
                        // fragments (4 consecutive tokens per lane group)
                        char* gkc = s_gk + NT * NKQ * 1024;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int lane2 = (lg * 4 + i) + 16 * (lr >> 2);
                            reinterpret_cast<float*>(gkc + ((ct * NTK + tt) * 64 + lane2) * 16)[lr & 3] = lk[kt][tt][i];
                        }
                    } else {
                        // row-major bf16: token 16tt + r, components 16ct + 4g .. +3
                        *reinterpret_cast<bf16x4*>(s_gk + gk_off(tt * 16 + lr, ct * 16 + lg * 4)) = pack4(lk[kt][tt]);
                    }
                }
            }
        }
        lds_barrier();

        // ---- contraction phase: this wave owns d_v tiles [w*VT_W, (w+1)*VT_W)
        gfrag_t vf[NEED_V ? VT_W : 1][NTK];
        if constexpr (NEED_V) {
#pragma unroll
            for (int vt = 0; vt < VT_W; ++vt) {
                const int gvt = w * VT_W + vt;
#pragma unroll
                for (int tk = 0; tk < NTK; ++tk) {
                    if constexpr (DMA) {
                        // transposed reads of the swizzled row-major V: lane 16g + 4i + q supplies row
                        // 4g + i of the token tile and the 4 columns 16 gvt + 4q .. +3
                        const int q = lane & 3, i4 = (lane >> 2) & 3;
                        u32x2 part[2];
#pragma unroll
                        for (int hf = 0; hf < 2; ++hf) {
                            const int row = (2 * tk + hf) * 16 + lg * 4 + i4;
                            const int chunk = (2 * gvt + (q >> 1)) ^ (row % CPR);
                            part[hf] = ds_read_tr16(raw + OFF_V + row * (VC * 2) + chunk * 16 + (q & 1) * 8);
                        }
                        vf[vt][tk] = __builtin_bit_cast(bf16x8, u32x4{part[0][0], part[0][1], part[1][0], part[1][1]});
                    } else {
                        const int row = gvt * 16 + lr;
                        if constexpr (F32) {
                            vf[vt][tk] = *reinterpret_cast<const f32x4*>(s_vt + row * VTS + (tk * 16 + lg * 4) * 4);
                        } else {
                            const u32x2 lo = *reinterpret_cast<const u32x2*>(s_vt + row * VTS + ((2 * tk) * 16 + lg * 4) * 2);
                            const u32x2 hi = *reinterpret_cast<const u32x2*>(s_vt + row * VTS + ((2 * tk + 1) * 16 + lg * 4) * 2);
                            vf[vt][tk] = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
                        }
                    }
                }
            }
        }

        // Gamma_K operand fragments
        // token rows (A of S^T = Gamma_K Gamma_Q^T): lane = token 16J + r, slots = components of step kq
        auto gk_token_frag = [&](int J, int kq) -> gfrag_t {
            if constexpr (F32) {
                return *reinterpret_cast<const gfrag_t*>(s_gk + ((J * NKQ + kq) * 64 + lane) * 16);
            } else {
                const int row = J * 16 + lr;
                const u32x2 lo = *reinterpret_cast<const u32x2*>(s_gk + gk_off(row, (2 * kq) * 16 + lg * 4));
                const u32x2 hi = *reinterpret_cast<const u32x2*>(s_gk + gk_off(row, (2 * kq + 1) * 16 + lg * 4));
                return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
            }
        };
        // component rows (A of the state update Gamma_K^T V): lane = component 16ct + r, slots =
        // tokens of step tk in the V-fragment order
        auto gk_comp_frag = [&](int ct, int tk) -> gfrag_t {
            if constexpr (F32) {
                return *reinterpret_cast<const gfrag_t*>(s_gk + NT * NKQ * 1024 + ((ct * NTK + tk) * 64 + lane) * 16);
            } else {
                const int q = lane & 3, i4 = (lane >> 2) & 3;
                u32x2 part[2];
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const int row = (2 * tk + hf) * 16 + lg * 4 + i4;
                    part[hf] = ds_read_tr16(s_gk + gk_off(row, ct * 16 + 4 * q));
                }
                return __builtin_bit_cast(bf16x8, u32x4{part[0][0], part[0][1], part[1][0], part[1][1]});
            }
        };

        if constexpr (OUT) {
            // intra-chunk affinities (causal): S^T(J, I) = Gamma_K[J] Gamma_Q[I]^T for J <= I, masked
            // j <= i, as operand fragments over the token steps; row sums go to the denominators
            constexpr int NSF = (MODE == MODE_OUT_CAUSAL) ? (F32 ? NT * NT : NT * NTK) : 1;
            gfrag_t sfr[NSF];
            float den[NT];
#pragma unroll
            for (int I = 0; I < NT; ++I) {
                float d = 0.f;
#pragma unroll
                for (int ww = 0; ww < W; ++ww) d += s_den[ww][I * 16 + lr];
                if constexpr (MODE == MODE_OUT_CAUSAL) {
                    f32x4 sacc[NT];
#pragma unroll
                    for (int J = 0; J < NT; ++J) {
                        sacc[J] = f32x4{0.f, 0.f, 0.f, 0.f};
                        if (J > I) continue;
#pragma unroll
                        for (int kq = 0; kq < NKQ; ++kq) {
                            const gfrag_t gqi = *reinterpret_cast<const gfrag_t*>(s_gq + ((I * NKQ + kq) * 64 + lane) * 16);
                            mma(sacc[J], gk_token_frag(J, kq), gqi);
                        }
                        if (J == I) {
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                if (lg * 4 + i > lr) sacc[J][i] = 0.f;
                        }
                    }
                    // operand fragments over the token steps, and their column sums (an all-ones
                    // product, so the denominator sees the same rounded weights as the numerator)
                    const gfrag_t ones = ones_frag<gfrag_t>();
                    f32x4 dacc = {0.f, 0.f, 0.f, 0.f};
                    if constexpr (F32) {
#pragma unroll
                        for (int J = 0; J < NT; ++J) {
                            sfr[I * NT + J] = sacc[J];
                            if (J <= I) mma(dacc, ones, sacc[J]);
                        }
                    } else {
#pragma unroll
                        for (int tk = 0; tk < NTK; ++tk) {
                            sfr[I * NTK + tk] = pack_pair(sacc[2 * tk], sacc[2 * tk + 1]);
                            if (2 * tk <= I) mma(dacc, ones, sfr[I * NTK + tk]);
                        }
                    }
                    d += dacc[0];
                }
                den[I] = d + a.eps;
            }

#pragma unroll
            for (int vt = 0; vt < VT_W; ++vt) {
                f32x4 oacc[NT];
#pragma unroll
                for (int I = 0; I < NT; ++I) oacc[I] = f32x4{0.f, 0.f, 0.f, 0.f};
                // inter: O^T(vt, I) += state^T . Gamma_Q^T, state operands packed on the fly
#pragma unroll
                for (int kq = 0; kq < NKQ; ++kq) {
                    gfrag_t sf;
                    if constexpr (F32) sf = st[kq][vt];
                    else sf = pack_pair(st[2 * kq][vt], st[2 * kq + 1][vt]);
#pragma unroll
                    for (int I = 0; I < NT; ++I)
                        mma(oacc[I], sf, *reinterpret_cast<const gfrag_t*>(s_gq + ((I * NKQ + kq) * 64 + lane) * 16));
                }
                // intra: O^T(vt, I) += V^T(vt, tokens) . S^T(tokens, I)
                if constexpr (MODE == MODE_OUT_CAUSAL) {
#pragma unroll
                    for (int I = 0; I < NT; ++I) {
                        if constexpr (F32) {
#pragma unroll
                            for (int J = 0; J < NT; ++J)
                                if (J <= I) mma(oacc[I], vf[vt][J], sfr[I * NT + J]);
                        } else {
#pragma unroll
                            for (int tk = 0; tk < NTK; ++tk)
                                if (2 * tk <= I) mma(oacc[I], vf[vt][tk], sfr[I * NTK + tk]);
                        }
                    }
                }
                // ---- write O: lane holds d_v 16vt' + 4g .. +3 of token 16I + r
                const int c0 = (w * VT_W + vt) * 16 + lg * 4;
#pragma unroll
                for (int I = 0; I < NT; ++I) {
                    const int tok = I * 16 + lr;
                    const f32x4 ov = oacc[I] * fast_rcp(den[I]);
                    if constexpr (DMA) {
                        // unconditional bounds-checked store: rows past N and pad columns are dropped
                        const uint32_t off = (c0 < a.d_v) ? (uint32_t)(((n0 + tok) * a.d_v + c0) * 2) : 0x80000000u;
                        store_b64(rs_o, __builtin_bit_cast(u32x2, pack4(ov)), off);
                    } else {
                        if (tok >= rows_valid) continue;
                        elem_t* orow = oo + (n0 + tok) * a.d_v;
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
        }

        // ---- advance the state: Vt += Gamma_K^T V for the wave's d_v tiles, and Z += Gamma_K^T 1 for
        // its own components (a product with an all-ones operand: lane (r, g) receives the column
        // sums for components 16ct + 4g .. +3, the same bf16 Gamma_K the state sees)
        if constexpr (NEED_K) {
            const gfrag_t ones = ones_frag<gfrag_t>();
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const bool own = (ct / KT_W) == w;
                f32x4 zi = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int tk = 0; tk < NTK; ++tk) {
                    const gfrag_t gkc = gk_comp_frag(ct, tk);
#pragma unroll
                    for (int vt = 0; vt < VT_W; ++vt) mma(st[ct][vt], gkc, vf[vt][tk]);
                    if (own) mma(zi, gkc, ones);
                }
                if (own && lr == 0) {
                    f32x4* zp = reinterpret_cast<f32x4*>(&s_z[ct * 16 + lg * 4]);
                    *zp = *zp + zi;
                }
            }
        }
        if constexpr (!DMA) lds_barrier();  // staging buffers are rewritten by the next chunk
    };

    for (int64_t ch = ch0; ch < ch1; ch += 2) {
        body(std::integral_constant<int, 0>{}, ch);
        if (ch + 1 < ch1) body(std::integral_constant<int, 1>{}, ch + 1);
    }
    if constexpr (!F32) {
        if (nonfin && a.flags) a.flags[bh] = 1;
    }

    if constexpr (RESP) {
        if (a.stat_usage) {
            // the segment's partials: usage summed over the 16 rows of each lane group (fixed butterfly
            // order), counts from LDS
#pragma unroll
            for (int kt = 0; kt < KT_W; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float u = use[kt][i];
#pragma unroll
                    for (int o = 1; o < 16; o <<= 1) u += __shfl_xor(u, o, 64);
                    use[kt][i] = u;
                }
            lds_barrier();
            const int64_t base = ((int64_t)bh * a.Pg + sidx) * a.K;
            if (lr == 0) {
#pragma unroll
                for (int kt = 0; kt < KT_W; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int c = (w * KT_W + kt) * 16 + lg * 4 + i;
                        if (c < a.K) a.stat_usage[base + c] = use[kt][i];
                    }
            }
            for (int c = tid; c < a.K; c += NTHR) a.stat_count[base + c] = s_cnt[c];
        }
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
                *reinterpret_cast<f32x4*>(segrec + (int64_t)KC * VC + ct * 16 + lg * 4) =
                    *reinterpret_cast<const f32x4*>(&s_z[ct * 16 + lg * 4]);
            }
        }
    }
}

}  // namespace gma
