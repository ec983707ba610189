// Responsibilities of every row, token-split (bf16 storage): Gamma written out in fp32, or the per-segment
// diagnostics (usage sums and hard-assignment counts) with Gamma kept on chip.
//
// Method: page "Attention par Mélange Gaussien (GMA)", section "Méthodologie", sub-section "Mécanisme
// Central", item 1 (posterior responsibilities of a diagonal GMM with softplus variances and softmax
// priors), through the expanded log-density of the forward passes: logits^T = [a | b] . [x^2 ; x] + c in
// base-2 units, one MFMA GEMM per 16 rows; the diagnostics are the sums over rows of the section
// "Résultats et Performance" (component usage, hard assignments).
//
// Work split.  Each wave takes 16-row groups of its workgroup's segment (groups w, w + 4, ...) and does
// everything for them alone: the logits of all components (the [a | b] operand fragments of every
// component stay in AGPRs for the whole kernel), the softmax over the components (inside the wave: the
// four lanes r, r + 16, r + 32, r + 48 share row r) and the row's output.  The loop has no LDS staging
// and no barrier; the next group's rows are loaded into registers while the current group's are used.
#include "gma_resp.hpp"

#include "gma_device.hpp"

namespace gma {

namespace {

constexpr int kRespWaves = 4;

template <int KC, int DRC, bool STATS>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1)))
resp_tok_kernel(const MainArgs a, int64_t rows_per_seg, int vec_gamma) {
    constexpr int W = kRespWaves;
    constexpr int NCT = KC / 16;    // component tiles
    constexpr int NKS2 = DRC / 32;  // fragment steps over d_r (x^2 part; the x part follows)
    static_assert(KC <= 256, "component index in the low 8 bits of the argmax key");
    static_assert((16 * KC / 4) % 64 == 0, "whole 16-byte units per lane in the row stores");
    __shared__ __attribute__((aligned(16))) float s_c[KC];
    __shared__ float s_use[STATS ? W : 1][STATS ? KC : 1];
    __shared__ uint32_t s_cnt[STATS ? KC : 1];
    // Gamma rows out through LDS: each wave's 16 rows (row pitch KC fp32 + 16 bytes), stored as whole rows
    constexpr int ROWB = KC * 4 + 16;
    __shared__ __attribute__((aligned(16))) char s_rows[STATS ? 16 : W * 16 * ROWB];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int64_t bh = blockIdx.x / a.Pg;
    const int sidx = (int)(blockIdx.x % a.Pg);
    const int h = (int)(bh % a.H);
    const int64_t N = a.N;
    const int64_t r0 = sidx * rows_per_seg;
    const int64_t r1 = (r0 + rows_per_seg < N) ? r0 + rows_per_seg : N;
    const int d_r = a.d_r, K = a.K;
    const uint16_t* xh = reinterpret_cast<const uint16_t*>(a.qx) + bh * N * d_r;

    // [a | b] fragments of every component (AGPRs): every load issued before the first is pinned
    f16x8 abf[NCT][2 * NKS2];
    {
        const f16x8* abg = reinterpret_cast<const f16x8*>(a.ab) + (int64_t)h * NCT * 2 * NKS2 * 64;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int ks = 0; ks < 2 * NKS2; ++ks) abf[ct][ks] = abg[((int64_t)ct * 2 * NKS2 + ks) * 64 + lane];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int ks = 0; ks < 2 * NKS2; ++ks) pin_agpr(abf[ct][ks]);
        for (int k = tid; k < KC; k += 256) s_c[k] = a.cvec[(int64_t)h * KC + k];
        if constexpr (STATS) {
            for (int k = tid; k < KC; k += 256) s_cnt[k] = 0u;
        }
    }
    __syncthreads();

    // X fragment of step ks for lane (r, g): dims 32 ks + 8 g .. + 7 of row r of the group (16 bytes;
    // d_r % 8 == 0, so a piece lies wholly inside or past the row); rows past the segment read as zeros
    auto load_x = [&](int64_t g0, u32x4 (&xr)[NKS2]) {
        const int64_t row = g0 + lr;
#pragma unroll
        for (int ks = 0; ks < NKS2; ++ks) {
            const int d0 = 32 * ks + 8 * lg;
            xr[ks] = (row < r1 && d0 < d_r) ? *reinterpret_cast<const u32x4*>(xh + row * d_r + d0)
                                            : u32x4{0u, 0u, 0u, 0u};
        }
    };

    bool nonfin = false;
    [[maybe_unused]] f32x4 use[STATS ? NCT : 1];
    if constexpr (STATS) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) use[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    int64_t g0 = r0 + 16 * w;
    u32x4 xn[NKS2];
    load_x(g0, xn);
    for (; g0 < r1; g0 += 16 * W) {
        u32x4 xr[NKS2];
#pragma unroll
        for (int ks = 0; ks < NKS2; ++ks) xr[ks] = xn[ks];
        if (g0 + 16 * W < r1) load_x(g0 + 16 * W, xn);

        // fp16 operands [x ; x^2] (bf16 -> fp16 is exact in the supported range; |x| >= 256 leaves it
        // and is flagged below through the non-finite logits)
        f16x8 xf[NKS2], x2[NKS2];
#pragma unroll
        for (int ks = 0; ks < NKS2; ++ks) {
            xf[ks] = bf16x8_bits_to_f16x8(xr[ks]);
            x2[ks] = xf[ks] * xf[ks];
        }
        // logits^T: acc[ct] rows = components 16 ct + 4 g + i, column = row r of the group
        f32x4 acc[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) acc[ct] = *reinterpret_cast<const f32x4*>(s_c + ct * 16 + lg * 4);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int ks = 0; ks < NKS2; ++ks) {
                mma(acc[ct], abf[ct][ks], x2[ks]);
                mma(acc[ct], abf[ct][ks + NKS2], xf[ks]);
            }

        // softmax over the components of row r (base 2): this lane's values, then the four lane groups
        float m = acc[0][0];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) m = fmaxf(m, acc[ct][i]);
        m = group4_max(m);
        float ssum = 0.f;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[ct][i] = fast_exp2(acc[ct][i] - m);
                ssum += acc[ct][i];
            }
        ssum = group4_sum(ssum);
        const int64_t row = g0 + lr;
        const bool valid = row < r1;
        // a row maximum of -inf or NaN (the maximum skips NaN logits), or a sum that is not finite
        const bool finite = m > -INFINITY && ssum < INFINITY;
        nonfin |= valid && !finite;
        const float rs = valid ? fast_rcp(ssum) : 0.f;

        if constexpr (STATS) {
            // usage sums of this lane's components (the normalisation folded into one multiply-add); the
            // row's largest gamma: one 32-bit key per component, the top 24 bits of the non-negative
            // 2^(l - max) (ordered as an integer, and in the same order as gamma) above 255 - k, so that an
            // unsigned maximum over the lane's components and the four lane groups picks the largest (values
            // equal in their top 24 bits, within about 2^-15 of each other, tie and go to the lowest
            // component); pad components have 2^-inf = 0.
            // A row whose gammas are not finite counts nowhere (its (batch, head) is flagged and recomputed).
            uint32_t key = 0u;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                use[ct] += acc[ct] * rs;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t kk = (__float_as_uint(acc[ct][i]) & 0xffffff00u) | (uint32_t)(255 - (16 * ct + 4 * lg + i));
                    key = key > kk ? key : kk;
                }
            }
#pragma unroll
            for (int o = 16; o < 64; o <<= 1) {
                const uint32_t ok = (uint32_t)__shfl_xor((int)key, o, 64);
                key = key > ok ? key : ok;
            }
            const int bi = 255 - (int)(key & 0xffu);
            if (lg == 0 && valid && finite && bi < K) atomicAdd(&s_cnt[bi], 1u);
        } else {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) acc[ct] *= rs;
            if (vec_gamma) {
                // lane (r, g) puts components 16 ct + 4 g .. + 3 of row r into the wave's staging area, then
                // lane l stores 16 bytes (unit (64 j + l) % (KC / 4)) of row (64 j + l) / (KC / 4): each store
                // instruction writes whole rows instead of 64-byte pieces of 16 rows.  The wave's LDS
                // operations run in order; the empty asm statements keep the compiler from moving them
                // across each other.
                lds_char* sw = (lds_char*)s_rows + w * 16 * ROWB;
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) lds_st<f32x4>(sw + lr * ROWB + (16 * ct + 4 * lg) * 4, acc[ct]);
                asm volatile("" ::: "memory");
                constexpr int UPR = KC / 4;            // 16-byte units per row
                constexpr int NU = 16 * UPR / 64;      // units per lane
#pragma unroll
                for (int j = 0; j < NU; ++j) {
                    const int e = 64 * j + lane, rr = e / UPR, cu = e % UPR;
                    const f32x4 v = lds_ld<f32x4>(sw + rr * ROWB + cu * 16);
                    if (g0 + rr < r1 && 4 * cu < K)
                        *reinterpret_cast<f32x4*>(a.gamma + (bh * N + g0 + rr) * K + 4 * cu) = v;
                }
                asm volatile("" ::: "memory");
            } else if (valid) {
                float* grow = a.gamma + (bh * N + row) * K;
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    const int c0 = 16 * ct + 4 * lg;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (c0 + i < K) grow[c0 + i] = acc[ct][i];
                }
            }
        }
    }
    if (nonfin && a.flags) a.flags[bh] = 1;

    if constexpr (STATS) {
        // the segment's partials: usage over the 16 rows of each lane group (fixed butterfly), then over
        // the waves in wave order; counts from LDS
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float u = use[ct][i];
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) u += __shfl_xor(u, o, 64);
                use[ct][i] = u;
            }
        if (lr == 0) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) s_use[w][16 * ct + 4 * lg + i] = use[ct][i];
        }
        __syncthreads();
        const int64_t base = (bh * a.Pg + sidx) * K;
        for (int c = tid; c < K; c += 256) {
            float u = s_use[0][c];
#pragma unroll
            for (int v = 1; v < W; ++v) u += s_use[v][c];
            a.stat_usage[base + c] = u;
            a.stat_count[base + c] = s_cnt[c];
        }
    }
}

template <int KC, int DRC>
void launch_kc_drc(const MainArgs& a, int64_t rows_per_seg, bool vec_gamma, int grid, hipStream_t s) {
    if (a.stat_usage)
        hipLaunchKernelGGL((resp_tok_kernel<KC, DRC, true>), dim3((unsigned)grid), dim3(256), 0, s, a, rows_per_seg,
                           vec_gamma ? 1 : 0);
    else
        hipLaunchKernelGGL((resp_tok_kernel<KC, DRC, false>), dim3((unsigned)grid), dim3(256), 0, s, a, rows_per_seg,
                           vec_gamma ? 1 : 0);
}

}  // namespace

// The padded shapes of the bf16 classes that have token-split forward passes.
bool resp_tok_supported(int kc, int drc) {
    return (kc == 32 && drc == 64) || (kc == 128 && drc == 128) || (kc == 256 && drc == 64);
}

bool launch_resp_tok(const MainArgs& a, int kc, int drc, int64_t rows_per_seg, bool vec_gamma, int grid,
                     hipStream_t s) {
    if (kc == 32 && drc == 64) launch_kc_drc<32, 64>(a, rows_per_seg, vec_gamma, grid, s);
    else if (kc == 128 && drc == 128) launch_kc_drc<128, 128>(a, rows_per_seg, vec_gamma, grid, s);
    else if (kc == 256 && drc == 64) launch_kc_drc<256, 64>(a, rows_per_seg, vec_gamma, grid, s);
    else return false;
    return true;
}

}  // namespace gma
