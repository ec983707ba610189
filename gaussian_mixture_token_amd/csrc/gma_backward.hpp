// Backward of the mixer: argument blocks and launchers of the kernels in gma_backward.hip, driven
// by the host library (gma_host.cpp), which owns validation, the workspace layout and timing.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace gma {

// Batched fp32 matrix product on the matrix cores (v_mfma_f32_16x16x4_f32):
//   C[b] = alpha op(A[b]) op(B[b]) (+ beta Cin[b]),  op(A) M x Kd, op(B) Kd x N, C M x N.
// ta: A is stored Kd x M (op(A) = A^T), else M x Kd; tb: B is stored N x Kd, else Kd x N; rows of
// every matrix are lda / ldb / ldc elements apart.  Batch b = outer * n_inner + inner; operand X
// of batch b starts at X + outer * sX0 + inner * sX1 elements (B: outer taken modulo modB when
// modB > 0).  Token axes: the bits of tok_flags mark M (1), N (2), Kd (4) as counting tokens of
// the sequence; for batch b such an axis holds min(size, ntok - inner * tok_step) entries (the
// ragged last chunk), and operand entries past it are read as zero and never stored.
// tril: entry (i, j) of the product is kept only for j <= i (chunk-local token indices).
// Cin (fp32, may be null) uses C's strides.  C is fp32, or bf16 with out_bf16.
enum { GEN_NONE = 0, GEN_XAUG = 1, GEN_VAUG = 2, GEN_GH = 3 };
// GEN_XAUG: [x | x^2 | 1 | 0 ...]; GEN_VAUG: [v | 1 | 0 ...]; GEN_GH: [v rs0 | rs1 | 0 ...] (the read-phase
// gradient [g | h]: rs0 = 1 / den, rs1 = h of the row)
struct BwdGen {
    const void* src = nullptr;
    const float* rs = nullptr;
    int kind = GEN_NONE, f32 = 0, d = 0;
};

struct BwdGemm {
    const float* A = nullptr;
    const float* B = nullptr;
    const float* Cin = nullptr;
    void* C = nullptr;
    int64_t sA0 = 0, sA1 = 0, sB0 = 0, sB1 = 0, sC0 = 0, sC1 = 0;
    int64_t modB = 0;
    int lda = 0, ldb = 0, ldc = 0;
    int M = 0, N = 0, Kd = 0;
    int n_inner = 1;
    int64_t n_outer = 1;
    int64_t ntok = 0;
    int tok_step = 0;
    int tok_flags = 0;
    float alpha = 1.f, beta = 0.f;
    int tril = 0;
    // bf16 matrix cores: each fp32 operand value split into bf16 hi + lo and the product formed as
    // hi hi + hi lo + lo hi (three v_mfma_f32_16x16x32_bf16 per 32-deep step, about 16 significant bits,
    // fp32 accumulation) instead of eight v_mfma_f32_16x16x4_f32
    int split = 0;
    // set by launch_bwd_gemm: 16-byte loads are allowed (base 16-byte aligned, leading dimension and
    // batch strides multiples of 4 elements)
    bool vecA = false, vecB = false;
    // routing-input gradient in the epilogue (A, B not transposed): the product's columns come in pairs
    // (2d, 2d + 1) = (dl . mu / s, dl . 1 / s) of dim d, and the output is dx[m][d] = C[m][2d] -
    // dx_x[m][d] C[m][2d + 1] in the storage dtype (OUT_BF16), at the C strides (ldc = d_r)
    const void* dx_x = nullptr;
    // operands generated from storage rows instead of read from a materialised fp32 matrix (kind != 0);
    // the operand's batch strides (sA0, sA1 or sB0, sB1) then count rows, and row t of the view is built
    // from the d elements at src + t d (fp32 or bf16) and, for GEN_GH, the pair rs[2 t], rs[2 t + 1]
    BwdGen ga, gb;
};
// false: no compiled kernel for this combination of transposes, generated operands and epilogue
bool launch_bwd_gemm(const BwdGemm& g, bool ta, bool tb, bool out_bf16, hipStream_t s);

// Mixture constants for the routing-input gradient: mw [H, K, 2 d_r] (row k: mu_kd / s_kd and 1 / s_kd
// interleaved, at columns 2d and 2d + 1; s = softplus(raw_var)).
void launch_bwd_prep(const float* mu, const float* raw_var, float* mw, int H, int K, int d_r, hipStream_t s);

// Responsibilities of rows x [BH, N, d_r] (bf16 or fp32) in fp32 -> gamma [BH, N, K], on the matrix
// cores from the expanded log-density: component tiles of 16 (KT tiles, a power of two covering K),
// the fragment-ordered coefficients bf [H][ceil(d_r / 16)][2][KT][64][4] fp32 and constants cq
// [H][16 KT] fp64, written by launch_bwd_frag.
int bwd_gamma_tiles(int K);
void launch_bwd_frag(const float* mu, const float* raw_var, const float* prior, float* bf, double* cq, int H, int K,
                     int d_r, bool split, hipStream_t s);
void launch_bwd_gamma_mfma(const void* x, bool f32, const float* bf, const double* cq, float* gamma, int64_t BH,
                           int64_t N, int H, int K, int d_r, hipStream_t s);
// The same for bf16 rows on the bf16 matrix cores with split operands (bwd_gamma_split_supported:
// bf16, d_r a multiple of 32, the head's fragments within 128 KiB), from the fragments that
// launch_bwd_frag writes with split = true (same bytes as the fp32 ones).  x 16-byte aligned.
bool bwd_gamma_split_supported(int K, int d_r, bool f32);
void launch_bwd_gamma_split(const void* x, const float* bf, const double* cq, float* gamma, int64_t BH, int64_t N,
                            int H, int K, int d_r, hipStream_t s);

// Read-phase gradient per row: p [rows, dva] holds (num | Gamma_Q . Z, the denominator without
// eps); rs [rows, 2] <- (1 / den, h = -(dO . O) / den), so that [g | h] = [dO rs0 | rs1] (GEN_GH).
void launch_bwd_gh(const float* p, const void* dout, bool f32, float* rs, int64_t rows, int d_v, int dva, float eps,
                   hipStream_t s);
// Softmax gradient in place: dl = gamma (dgamma - gamma . dgamma) per row of K.
void launch_bwd_dl(const float* gamma, float* dg, int64_t rows, int K, hipStream_t s);
// The query-side chunk work of the causal backward in one kernel (bf16 storage, K = d_v = 128;
// bwd_chunk_q_supported), one workgroup per (batch, head, chunk of 64 tokens): from gq, gk [BH, N, K],
// v, dout [BH, N, d_v] bf16 and the exclusive prefix states stt [BH, n_st, K, dva] it writes rs
// [BH N, 2] = (1 / den, h), rt (if not null) the segment totals of Gamma_Q^T [g | h] over segments of
// seg_per chunks [BH, ceil(n_st / seg_per), K, dva] (zero padded; the layout launch_bwd_suffix_state's
// first pass writes, so that pass can be left out), dgq = [g | h] S^T + mt Gamma_K [BH, N, K] and,
// where ac and mt are not null, ac = tril(Gamma_Q Gamma_K^T) and mt = tril([g | h] [V | 1]^T)
// [BH, n_st, 64, 64].  dva = d_v + 4; rows of v and dout 16-byte aligned.  false: no kernel for this
// shape.
bool bwd_chunk_q_supported(int K, int d_v, bool f32);
bool launch_bwd_chunk_q(const float* gq, const float* gk, const void* v, const void* dout, const float* stt, float* rs,
                        float* rt, int seg_per, float* ac, float* mt, float* dgq, int64_t BH, int64_t N, int64_t n_st,
                        int K, int d_v, int dva, float eps, bool emit_dl, hipStream_t s);
// The prefix states of the chunk terms Gamma_K^T [V | 1] (the same shapes), in segments of `per` chunks
// (bwd_state_segment), two passes: totals = true writes each segment's total into seg [BH, ceil(n_st /
// per), K, dva]; after an exclusive scan of seg, totals = false writes each chunk's exclusive prefix
// state into stt [BH, n_st, K, dva] (the segment's prefix plus the earlier chunks of the segment).
// Columns d_v .. dva - 1 = Z, 0, 0, 0.
int bwd_state_segment(int64_t BH, int64_t n_st);
bool launch_bwd_chunk_state(const float* gk, const void* v, float* stt, float* seg, int per, bool totals, int64_t BH,
                            int64_t N, int64_t n_st, int K, int d_v, int dva, hipStream_t s);
// The suffix states R_c = sum over the later chunks of Gamma_Q^T [g | h] (the same shapes), from gq, dout and
// rs: seg [BH, ceil(n_st / per), K, dva] holds each segment's exclusive suffix (the segment totals of
// launch_bwd_chunk_q after an exclusive suffix scan); every chunk's R goes into rt [BH, n_st, K, dva]
// (columns d_v .. dva - 1 = the h sums, 0, 0, 0).
bool launch_bwd_suffix_state(const float* gq, const void* dout, const float* rs, float* rt, const float* seg, int per,
                             int64_t BH, int64_t N, int64_t n_st, int K, int d_v, int dva, hipStream_t s);
// Its key-side counterpart (the same shapes): from gq, gk, v, dout, rs and the exclusive suffix states
// rt [BH, n_st, K, dva] it writes dgk = [V | 1] R^T + mt^T Gamma_Q [BH, N, K] and dv = Gamma_K Rv +
// ac^T g [BH, N, d_v] bf16, recomputing ac and mt.
bool launch_bwd_chunk_k(const float* gq, const float* gk, const void* v, const void* dout, const float* rs,
                        const float* rt, float* dgk, void* dv, int64_t BH, int64_t N, int64_t n_st, int K, int d_v,
                        int dva, bool emit_dl, hipStream_t s);
// emit_dl (both chunk kernels): write the posterior gradient dl = gamma (dGamma - gamma . dGamma) of each
// row in place of dGamma (gamma as the chunk's split image holds it, about 16 significant bits).

// Posterior gradient, routing-input gradient and parameter partials of one side in one kernel
// (bf16 storage, K = d_r = 128, or K <= 64 and d_r <= 128 with both multiples of 4;
// bwd_fused_rows_supported): from gamma and dgamma [BH, N, K] fp32, the
// routing input x [BH, N, d_r] bf16 and mw (launch_bwd_prep) it writes dx [BH, N, d_r] bf16 and the
// partials gp [BH][n_seg][K][dxa] (columns x | x^2 | 1 of dl^T [x | x^2 | 1], rows dxa >= 2 d_r + 1
// floats apart) over segments of
// `seg` tokens (n_seg = ceil(N / seg)).  dl itself is not written.  Bases 16-byte aligned,
// (N + 64) K 4 < 2^31 and N d_r 2 < 2^31.  false: no fused kernel for this shape.
// bwd_fused_rows_seg: the segment length, a power of two in [min_seg, 4096] (min_seg a power of two
// >= 64, at most 4096), long enough to keep n_seg within the partials buffer sized for min_seg.
bool bwd_fused_rows_supported(int K, int d_r, bool f32);
int bwd_fused_rows_seg(int64_t BH, int64_t N, int K, int d_r, int min_seg);
bool launch_bwd_fused_rows(const float* gamma, const float* dgamma, const void* x, const float* mw, void* dx, float* gp,
                           int64_t BH, int64_t N, int H, int K, int d_r, int dxa, int seg, bool dl_in, hipStream_t s);
// dl_in: dgamma already holds dl (from the chunk kernels with emit_dl) and gamma is not read.
// Bidirectional backward products in three fused kernels (bf16 storage, K <= 64 and d_v <= 128, both
// multiples of 4, dva = d_v + 4; bwd_bidir_small_supported), over segments of `seg` tokens (a multiple
// of 64; n_seg = ceil(N / seg) records per (batch, head), each [K][dva]):
//   state: st [BH][n_seg] <- each segment's Gamma_K^T [V | 1] (columns past d_v: Z, then zeros);
//   q: with the summed state in entry 0 of st, dGamma_Q [BH, N, K] = g S_v^T + h Z^T and r_seg [BH][n_seg]
//      <- each segment's Gamma_Q^T [g | h], where g = dO / (Gamma_Q . Z + eps) and h = -(dO . num) g's
//      scale squared per row;
//   k: with the summed R in entry 0 of r_seg, dGamma_K [BH, N, K] = V R_v^T + R_1^T and dV [BH, N, d_v]
//      = Gamma_K R_v (bf16).
// V, dO and dV rows 8-byte aligned; (N + 64) K 4 and N d_v 2 below 2^31.  false: not supported.
bool bwd_bidir_small_supported(int K, int d_v, bool f32);
bool launch_bwd_bidir_state(const float* gk, const void* v, float* st, int64_t BH, int64_t N, int K, int d_v, int dva,
                            int seg, hipStream_t s);
bool launch_bwd_bidir_q(const float* gq, const void* dout, const float* st, float* dgq, float* r_seg, int64_t BH,
                        int64_t N, int K, int d_v, int dva, int seg, float eps, bool emit_dl, hipStream_t s);
bool launch_bwd_bidir_k(const float* gk, const void* v, const float* r_seg, float* dgk, void* dv, int64_t BH, int64_t N,
                        int K, int d_v, int dva, int seg, bool emit_dl, hipStream_t s);
// emit_dl (q and k): dl = Gamma (dGamma - Gamma . dGamma) of each row in place of dGamma.
// Chunk-state scans over [n_outer][n][rec]: mode 0 exclusive prefix in place, 1 exclusive suffix in
// place, 2 the total into entry 0.  rec is a multiple of 4 (K times d_v + 1 rounded up to 4) and st
// 16-byte aligned.
void launch_bwd_scan(float* st, int64_t n_outer, int64_t n, int64_t rec, int mode, hipStream_t s);
// Mixture-parameter gradients from the partial sums gp [parts][K][dxa] (parts = 2 sides x B x
// n_seg per head; columns x | x^2 | 1 of dl^T [x | x^2 | 1]), first summed per head into gs [H][K][dxa].
void launch_bwd_param(const float* gp, float* gs, const float* mu, const float* raw_var, const float* prior,
                      float* dmu, float* draw_var, float* dprior, int64_t B, int H, int K, int d_r, int dxa,
                      int64_t n_seg, hipStream_t s);

}  // namespace gma
