// Host side of libgma.so: argument validation, shape-class selection, workspace layout,
// kernel launches and optional per-kernel event timing.  Declared in include/gma.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "gma.h"
#include "gma_backward.hpp"
#include "gma_decode.hpp"
#include "gma_fixup.hpp"
#include "gma_resp.hpp"
#include "gma_registry.hpp"

namespace gma {
namespace {

thread_local std::string g_last_error;

gma_status_t fail(gma_status_t st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
gma_status_t fail(gma_status_t st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

// The segment split aims for one full round of workgroups on a 256-CU MI355X: 256 x the
// workgroups per CU that the shape class's LDS and register budgets allow.  A fixed constant
// (not a device query) keeps the decomposition, and therefore every result bit, independent of
// the device and of the HIP runtime state.
constexpr int64_t kComputeUnits = 256;
// bidirectional passes with at most this many segments per (batch, head) skip the scan kernel: the
// read pass adds the segment records itself (in segment order, the scan's order)
constexpr int kBidirReadSum = 4;

int next_pow2(int x) {
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}

enum KernelId {
    K_PREP = 0, K_AGG, K_SCAN, K_OUT_CAUSAL, K_OUT_BIDIR, K_RESP, K_STATE, K_DECODE, K_STATS,
    K_BWD_GAMMA, K_BWD_GEMM, K_BWD_ROWS, K_BWD_SCAN, K_BWD_PARAM, K_DECODE_PREP,
    K_GEN_PREP, K_GEN_GAMMA, K_GEN_GEMM, K_GEN_SCAN, K_GEN_OUT, K_FIXUP, K_BWD_FUSED, K_BWD_CHUNK, K_COUNT
};
const char* kKernelNames[K_COUNT] = {"prep", "segment_aggregate", "segment_scan", "causal_output", "bidir_output",
                                     "responsibilities", "state_convert", "decode_step", "responsibility_stats",
                                     "backward_responsibilities", "backward_products", "backward_rows",
                                     "backward_scan", "backward_parameters", "decode_prepare",
                                     "generic_prep", "generic_responsibilities", "generic_products",
                                     "generic_scan", "generic_output", "out_of_range_fixup",
                                     "backward_route_gradients", "backward_query_chunks"};

struct Plan {
    const ShapeClass* cls = nullptr;
    int64_t B = 0, H = 0, N = 0;
    int d_r = 0, K = 0, d_v = 0;
    bool f32 = false;
    float eps = 0.f;
    int64_t n_chunks = 0;
    int P = 1;
    int seg_chunks = 1;
    bool dma = false;
    bool gtiles = false;   // causal token-split pair through stored Gamma_K tiles
    int rounds = 1;        // causal token-split pair: launches of (aggregate, scan, output) over the sequence
    int P_round = 1;       // segments per (batch, head) in one round (P = rounds * P_round)
    int64_t gk_ring = 0;   // Gamma_K tile slots per (batch, head) (one round's chunks; 0: n_chunks)
    size_t off_ab = 0, off_c = 0, off_seg = 0, off_gk = 0, off_total = 0, off_state = 0, total = 0;
    // bf16 classes: the out-of-range flags [BH] and the exact recomputation's mixture scratch
    size_t off_flags = 0, off_fix = 0;
    bool flags = false;
    int stat_segs = 0;                     // responsibility diagnostics: row segments per (batch, head)
    // responsibilities through the token-split kernel (bf16 classes with token-split passes, d_r % 8 == 0):
    // segments of resp_rows rows (whole 64-row blocks; seg_chunks chunks of the class for main_kernel)
    bool resp_tok = false;
    int64_t resp_rows = 0;
    size_t off_gamma = 0, off_part = 0;
    // Generic path (no compiled class covers the shape): fp32 responsibilities and products over
    // materialised Gamma_Q, Gamma_K.  Rows of tokens in entries of gen_step (a causal chunk or a
    // bidirectional segment); records [K, gen_dva] = [Vt | Z | 0 ..] per entry.
    bool generic = false;
    int gen_step = 0, gen_dva = 0;
    int64_t gen_nst = 0, gen_rows = 0;
    size_t off_gbf = 0, off_gcq = 0, off_gq = 0, off_ggk = 0, off_gpp = 0, off_gst = 0, off_gac = 0, off_grin = 0,
           off_grout = 0;
};

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// vc < 0: any d_v class (the responsibilities kernel does not touch V).
// The compiled class that covers the padded sizes (kc <= class K, vc <= class d_v, drc <= class d_r;
// vc < 0: any d_v) with the least padded work per token, K (2 d_r + d_v); the first such class on a
// tie.  Padding components get c = -inf (zero responsibilities), padding dims and columns zero
// coefficients, so a larger class computes the same result.
const ShapeClass* find_class(bool f32, int kc, int vc, int drc) {
    int n = 0;
    const ShapeClass* tab = f32 ? classes_f32(&n) : classes_bf16(&n);
    const ShapeClass* best = nullptr;
    int64_t best_cost = 0;
    for (int i = 0; i < n; ++i) {
        if (tab[i].kc < kc || (vc >= 0 && tab[i].vc < vc) || tab[i].drc < drc) continue;
        const int64_t cost = (int64_t)tab[i].kc * (2 * tab[i].drc + (vc >= 0 ? tab[i].vc : 0));
        if (!best || cost < best_cost) {
            best = &tab[i];
            best_cost = cost;
        }
    }
    return best;
}

// Validates sizes (pure host) and fills the plan for the register-staged kernels or, with tok, for
// the token-split LDS-DMA kernels (chunks of kTokChunk tokens; with tiles, the causal pair through
// stored Gamma_K tiles where it applies).  No HIP call.
// Sizes, dtype and eps of a problem (pure host).
gma_status_t validate_problem(const gma_problem_t* p) {
    if (!p) return fail(GMA_ERROR_INVALID_VALUE, "problem is NULL");
    if (p->batch < 1 || p->heads < 1 || p->seq_len < 1)
        return fail(GMA_ERROR_INVALID_VALUE, "batch, heads and seq_len must be >= 1 (got %lld, %lld, %lld)",
                    (long long)p->batch, (long long)p->heads, (long long)p->seq_len);
    if (p->d_route < 1 || p->n_comp < 1 || p->d_value < 1)
        return fail(GMA_ERROR_INVALID_VALUE, "d_route, n_comp and d_value must be >= 1");
    if (p->dtype != GMA_DTYPE_F32 && p->dtype != GMA_DTYPE_BF16)
        return fail(GMA_ERROR_INVALID_VALUE, "dtype must be GMA_DTYPE_F32 or GMA_DTYPE_BF16 (got %d)", p->dtype);
    if (!std::isfinite(p->eps) || p->eps < 0.f)
        return fail(GMA_ERROR_INVALID_VALUE, "eps must be finite and >= 0");
    if (p->d_route > 256 || p->n_comp > 256 || p->d_value > 256)
        return fail(GMA_ERROR_NOT_SUPPORTED, "d_route, n_comp and d_value must be <= 256");
    const int64_t maxd = std::max(std::max(p->d_route, p->d_value), p->n_comp);
    if (p->batch > (int64_t(1) << 40) / p->heads ||
        p->batch * p->heads > (int64_t(1) << 52) / p->seq_len / maxd)
        return fail(GMA_ERROR_INVALID_VALUE, "tensor sizes overflow");
    if (p->batch * p->heads > INT32_MAX / 2)
        return fail(GMA_ERROR_NOT_SUPPORTED, "batch * heads too large");
    return GMA_SUCCESS;
}

constexpr int kBwdChunk = 64;    // causal chunk (tokens) of the backward and of the generic forward
constexpr int kBwdSeg = 1024;    // bidirectional state segments and parameter-partial segments (tokens)

// Generic plan for the shapes that no compiled class covers (d_r or d_v in (128, 256]): Gamma_Q and
// Gamma_K in fp32 from the matrix-core responsibilities kernel of the backward (expanded
// log-density, fp32 steps of 16 dims added in fp64), then the write and read phases as batched fp32
// matrix-core products.  Workspace (256-byte aligned regions): coefficient fragments and constants;
// for the forward Gamma_Q, Gamma_K [BH, N, K], [num | den] [BH, N, dva], the entry records
// [BH, n_entries, K, dva], (causal) the intra-chunk blocks tril(Gamma_Q Gamma_K^T) [BH, n_chunks, 64, 64]
// and (carried state) the initial and final records [BH, K, dva].
gma_status_t make_generic_plan(const gma_problem_t* p, int op, Plan* plan) {
    const bool causal = op == GMA_OP_FORWARD_CAUSAL || op == GMA_OP_FORWARD_CAUSAL_STATE;
    const bool resp = op == GMA_OP_RESPONSIBILITIES || op == GMA_OP_RESPONSIBILITY_STATS;
    const int64_t BH = plan->B * plan->H, N = plan->N;
    const int K = plan->K;
    plan->generic = true;
    plan->gen_step = causal ? kBwdChunk : kBwdSeg;
    plan->gen_nst = (N + plan->gen_step - 1) / plan->gen_step;
    plan->gen_dva = (plan->d_v + 1 + 3) / 4 * 4;
    plan->gen_rows = BH * N;
    const int64_t rec = (int64_t)K * plan->gen_dva;
    const int64_t widest = std::max<int64_t>(std::max<int64_t>(K, plan->gen_dva), plan->gen_step);
    if (BH * plan->gen_nst * ((kBwdSeg + 63) / 64) * ((widest + 63) / 64) > INT32_MAX ||
        plan->gen_rows / 4 + 1 > INT32_MAX || BH * ((rec + 255) / 256) > INT32_MAX)
        return fail(GMA_ERROR_NOT_SUPPORTED, "problem too large for the generic path's grids");
    size_t off = 0;
    auto take = [&](size_t* o, int64_t floats) {
        *o = off;
        off = align_up(off + (size_t)floats * sizeof(float), 256);
    };
    const int KT = bwd_gamma_tiles(K);
    take(&plan->off_gbf, plan->H * ((plan->d_r + 15) / 16) * 2 * KT * 256);
    take(&plan->off_gcq, plan->H * 16 * KT * 2);   // fp64
    if (!resp) {
        take(&plan->off_gq, plan->gen_rows * K);
        take(&plan->off_ggk, plan->gen_rows * K);
        take(&plan->off_gpp, plan->gen_rows * plan->gen_dva);
        take(&plan->off_gst, BH * plan->gen_nst * rec);
        take(&plan->off_gac, causal ? BH * plan->gen_nst * kBwdChunk * kBwdChunk : 0);
        take(&plan->off_grin, op == GMA_OP_FORWARD_CAUSAL_STATE ? BH * rec : 0);
        take(&plan->off_grout, op == GMA_OP_FORWARD_CAUSAL_STATE ? BH * rec : 0);
    }
    plan->total = off;
    if (op == GMA_OP_RESPONSIBILITY_STATS) {
        // Gamma of every row, then per-segment partial usages and counts
        plan->stat_segs = (int)std::max<int64_t>(1, std::min<int64_t>((1024 + BH - 1) / BH, (N + 63) / 64));
        plan->off_gamma = plan->total;
        plan->off_part = align_up(plan->off_gamma + (size_t)BH * N * K * sizeof(float), 256);
        plan->total = align_up(plan->off_part + (size_t)BH * plan->stat_segs * K * 8, 256);
    }
    return GMA_SUCCESS;
}

gma_status_t make_plan(const gma_problem_t* p, int op, Plan* plan, bool tok = false, bool tiles = true) {
    if (!p) return fail(GMA_ERROR_INVALID_VALUE, "problem is NULL");
    if (op < GMA_OP_RESPONSIBILITIES || op > GMA_OP_RESPONSIBILITY_STATS)
        return fail(GMA_ERROR_INVALID_VALUE, "unknown op %d", op);
    gma_status_t vs = validate_problem(p);
    if (vs != GMA_SUCCESS) return vs;

    plan->f32 = p->dtype == GMA_DTYPE_F32;
    plan->B = p->batch;
    plan->H = p->heads;
    plan->N = p->seq_len;
    plan->d_r = p->d_route;
    plan->K = p->n_comp;
    plan->d_v = p->d_value;
    plan->eps = p->eps;

    const int kmin = plan->f32 ? 16 : 32;
    const int kc = std::max(kmin, next_pow2(p->n_comp));
    const int w = std::min(4, kc / 16);
    const int vc = std::max(next_pow2(p->d_value), 16 * w);
    const int drc = std::max(plan->f32 ? 16 : 32, next_pow2(p->d_route));
    const bool resp = op == GMA_OP_RESPONSIBILITIES || op == GMA_OP_RESPONSIBILITY_STATS;
    plan->cls = find_class(plan->f32, kc, resp ? -1 : vc, drc);
    if (!plan->cls) {
        if (tok) return fail(GMA_ERROR_NOT_SUPPORTED, "no token-split kernels for this shape");
        return make_generic_plan(p, op, plan);
    }
    if (tok && !plan->cls->tok_out_causal)
        return fail(GMA_ERROR_NOT_SUPPORTED, "no token-split kernels for this class");
    plan->dma = tok;
    const int C = tok ? kTokChunk : plan->cls->c;
    const int wg_per_cu = tok ? plan->cls->tok_wg_per_cu : plan->cls->wg_per_cu;
    const int64_t BH = plan->B * plan->H;
    plan->n_chunks = (plan->N + C - 1) / C;
    // Token-split responsibilities (each wave alone on 16-row groups, every component's [a | b] in AGPRs,
    // Gamma rows stored whole from a per-wave LDS staging area, no barriers) against the main_kernel walk
    // below, measured on MI355X: diagnostics 230 -> 152 us at B1 H16 N65536 d_r 128 K 128, 2.91 -> 1.87 ms
    // at B1 H8 N1M d_r 64 K 256, 153 -> 46 us at B32 H8 N4096 d_r 64 K 32 (then 126 us, 1.06 ms, 42 us with
    // the packed argmax); Gamma written out 0.22 -> 0.19 ms, 2.22 -> 2.05 ms, 0.073 -> 0.059 ms.  The walk
    // serves rows that are not 16-byte aligned.
    plan->resp_tok = resp && !tok && !plan->f32 && plan->d_r % 8 == 0 && 64 % C == 0 &&
                     resp_tok_supported(plan->cls->kc, plan->cls->drc);
    if (plan->resp_tok) {
        // one round of workgroups, one per compute unit (four at K = 32, whose fragments leave room), each
        // walking a segment of whole 64-row blocks
        const int64_t wpc = plan->cls->kc <= 32 ? 4 : 1;
        const int64_t blocks = (plan->N + 63) / 64;
        int64_t P = (kComputeUnits * wpc + BH - 1) / BH;
        if (P > blocks) P = blocks;
        if (P < 1) P = 1;
        const int64_t sb = (blocks + P - 1) / P;
        plan->resp_rows = sb * 64;
        plan->seg_chunks = (int)(sb * (64 / C));
        plan->P = (int)((blocks + sb - 1) / sb);
    } else if (op == GMA_OP_RESPONSIBILITIES) {
        // two workgroups' worth per compute unit slot, each walking consecutive chunks: a workgroup loads
        // the [a | b] fragments of its components once (32 KB per wave at K = d_r = 128) for all of its
        // chunks.  One chunk per workgroup measured 0.31 against 0.21 ms at B1 H16 N65536 K128 and 2.99
        // against 2.24 ms at B1 H8 N1M K256 (one and four slots per unit: within 5% of two).
        const int64_t target = kComputeUnits * wg_per_cu * 2;
        int64_t P = (target + BH - 1) / BH;
        if (P > plan->n_chunks) P = plan->n_chunks;
        if (P < 1) P = 1;
        const int64_t sc = (plan->n_chunks + P - 1) / P;
        plan->seg_chunks = (int)sc;
        plan->P = (int)((plan->n_chunks + sc - 1) / sc);
    } else {
        const int64_t target = kComputeUnits * wg_per_cu;
        int64_t P = (target + BH - 1) / BH;
        if (P > plan->n_chunks) P = plan->n_chunks;
        if (P < 1) P = 1;
        // Causal token-split pair: the sequence may be taken in R rounds of P segments per (batch, head),
        // each round's aggregate, scan and output launched in turn, so that the output pass re-reads
        // the K_X, V and Gamma_K tiles of its round while they may still be in the last-level cache.
        // Measured slower at every R > 1 on MI355X (the passes are bound by their own instruction
        // streams, not by HBM traffic, and each round adds a launch triple), so R = 1 unless
        // GMA_CAUSAL_ROUNDS asks for more (a measurement switch; results then differ only in the
        // summation order of the carried state).
        const bool causal_op = op == GMA_OP_FORWARD_CAUSAL || op == GMA_OP_FORWARD_CAUSAL_STATE;
        int64_t R = 1;
        if (tok && causal_op) {
            const char* env = getenv("GMA_CAUSAL_ROUNDS");
            if (env) R = std::max<int64_t>(1, std::min<int64_t>(atoi(env), 64));
            R = std::min<int64_t>(R, std::max<int64_t>(1, plan->n_chunks / P));
        }
        const int64_t sc = (plan->n_chunks + P * R - 1) / (P * R);
        plan->seg_chunks = (int)sc;
        plan->P = (int)((plan->n_chunks + sc - 1) / sc);
        plan->P_round = (int)std::min<int64_t>(P, plan->P);
        plan->rounds = (plan->P + plan->P_round - 1) / plan->P_round;
        plan->gk_ring = plan->rounds > 1 ? (int64_t)plan->P_round * sc : 0;
    }
    if (BH * plan->P > INT32_MAX)
        return fail(GMA_ERROR_NOT_SUPPORTED, "grid too large");

    // Causal token-split path through stored Gamma_K tiles.  Storing Gamma_K (K bf16 per token)
    // instead of recomputing it from K_X (d_r bf16 per token) in the output pass saves the K-side
    // logits GEMM and softmax at the price of 2 K bytes written and read per token-head.  Measured
    // on MI355X it wins at K = d_r = 128 (0.62 -> 0.55 ms per step) and at K = 4 d_r = 256 (4.01 ->
    // 3.74 ms), so it is taken up to K = 4 d_r, while the tiles of one (batch, head) stay within
    // 32-bit byte offsets.
    const int64_t tile_bytes = (int64_t)C * plan->cls->kc * 2;
    const bool causal = op == GMA_OP_FORWARD_CAUSAL || op == GMA_OP_FORWARD_CAUSAL_STATE;
    plan->gtiles = tiles && tok && causal && plan->cls->tok_out_causal_g &&
                   plan->cls->kc <= 4 * plan->cls->drc && plan->n_chunks * tile_bytes < (int64_t(1) << 31);

    // workspace: [a | b] fragments, c, segment records, Gamma_K tiles, (carried state) the
    // initial and the final state as records
    const int ks = plan->f32 ? 16 : 32;
    const int nks = 2 * plan->cls->drc / ks;
    const size_t ab_bytes = (size_t)plan->H * (plan->cls->kc / 16) * nks * 64 * 16;
    const size_t c_bytes = (size_t)plan->H * plan->cls->kc * sizeof(float);
    const size_t rec_bytes = ((size_t)plan->cls->kc * plan->cls->vc + plan->cls->kc) * sizeof(float);
    const bool stateful = op == GMA_OP_FORWARD_CAUSAL_STATE;
    size_t seg_bytes = 0;
    const bool need_seg = (op == GMA_OP_FORWARD_BIDIR) || (causal && (plan->P > 1 || plan->gtiles || stateful));
    // with rounds, the segment records and the Gamma_K tiles of one round are reused by the next, and
    // the running total of the finished rounds is kept beside them
    if (need_seg) seg_bytes = (size_t)BH * (plan->rounds > 1 ? plan->P_round : plan->P) * rec_bytes;
    const int64_t gk_slots = plan->rounds > 1 ? plan->gk_ring : plan->n_chunks;
    const size_t gk_bytes = plan->gtiles ? (size_t)BH * gk_slots * tile_bytes : 0;
    const size_t total_bytes = plan->rounds > 1 ? (size_t)BH * rec_bytes : 0;
    const size_t state_bytes = stateful ? 2 * (size_t)BH * rec_bytes : 0;
    plan->off_ab = 0;
    plan->off_c = align_up(ab_bytes, 256);
    plan->off_seg = align_up(plan->off_c + c_bytes, 256);
    plan->off_gk = align_up(plan->off_seg + seg_bytes, 256);
    plan->off_total = align_up(plan->off_gk + gk_bytes, 256);
    plan->off_state = align_up(plan->off_total + total_bytes, 256);
    plan->total = align_up(plan->off_state + state_bytes, 256);
    plan->flags = !plan->f32;
    if (plan->flags) {
        plan->off_flags = plan->total;
        plan->off_fix = align_up(plan->off_flags + (size_t)BH * sizeof(int), 256);
        plan->total = align_up(plan->off_fix + fixup_scratch_bytes((int)plan->H, plan->K, plan->d_r), 256);
    }
    if (op == GMA_OP_RESPONSIBILITY_STATS) {
        // per-segment partial usages and counts, formed by the responsibilities kernel itself (Gamma is
        // never stored): [BH, P, K] of each, independent of N
        plan->stat_segs = plan->P;
        plan->off_part = plan->total;
        plan->total = align_up(plan->off_part + (size_t)BH * plan->stat_segs * plan->K * 8, 256);
    }
    return GMA_SUCCESS;
}

// Backward workspace: fp32 intermediates of the gradient, each region 256-byte aligned.
//   bf, cq                                    matrix-core log-density operands (launch_bwd_frag)
//   mw [H, K, 2 d_r]                          mixture constants mu / s and 1 / s, interleaved by dim
//   gq, gk, dgq, dgk [BH, N, K]               responsibilities and their gradients (then dl)
//   pp [BH, N, dva]                           [num | Gamma_Q . Z]  (dva = d_v + 1 rounded up to a multiple
//                                             of 4, zero padded)
//   rs [BH, N, 2]                             1 / den and h per row ([g | h] = [dO rs0 | rs1])
//   st, rt [BH, n_st, K, dva]                 states per chunk (causal) or segment (bidirectional):
//                                             Gamma_K^T [V | 1] -> prefix, Gamma_Q^T [g | h] -> suffix
//   ac, mt [BH, n_st, C, C] (causal)          tril(Gamma_Q Gamma_K^T), tril([g | h] [V | 1]^T) per chunk
//   dvt [BH, N, d_v] (causal)                 intra-chunk part of dV
//   gp [2, BH, n_sg, K, dxa]                  per-segment dl^T [x | x^2 | 1] of both sides (dxa = 2 d_r + 1
//                                             rounded up to a multiple of 4; the product generates the
//                                             augmented rows from x)
struct BwdPlan {
    int64_t B = 0, H = 0, N = 0, BH = 0;
    int d_r = 0, K = 0, d_v = 0, dva = 0, dxa = 0;
    bool f32 = false, causal = false;
    float eps = 0.f;
    int st_step = 0;            // tokens per state entry
    int64_t n_st = 0, n_sg = 0;  // state entries and parameter segments per (batch, head)
    size_t off_bf = 0, off_cq = 0, off_mw = 0, off_gq = 0, off_gk = 0, off_dgq = 0, off_dgk = 0, off_gh = 0,
           off_pp = 0, off_st = 0, off_rt = 0, off_ac = 0, off_mt = 0, off_dvt = 0, off_gp = 0, off_sgs = 0,
           off_vs = 0, off_ds = 0, off_dvs = 0, off_gs = 0, total = 0;
    int sper = 1;   // causal: chunks per state segment (bwd_state_segment)
    // causal bf16 at K = d_v = 128: the fused chunk kernels, whose plan has no [num | den], no per-chunk
    // 64 x 64 blocks and no fp32 dV; the suffix states share the bytes of the prefix states (the query side
    // reads the last prefix before the first suffix is written), and there is room to stage V, dO and dV
    // where the caller's rows are not 16-byte aligned (dO's staging shares the bytes of the parameter
    // partials, which are written only after the last read of dO)
    bool fq = false;
};

gma_status_t make_bwd_plan(const gma_problem_t* p, bool causal, BwdPlan* b) {
    gma_status_t vs = validate_problem(p);
    if (vs != GMA_SUCCESS) return vs;
    b->B = p->batch;
    b->H = p->heads;
    b->N = p->seq_len;
    b->BH = b->B * b->H;
    b->d_r = p->d_route;
    b->K = p->n_comp;
    b->d_v = p->d_value;
    b->dva = (p->d_value + 1 + 3) / 4 * 4;
    b->dxa = (2 * p->d_route + 1 + 3) / 4 * 4;
    b->f32 = p->dtype == GMA_DTYPE_F32;
    b->causal = causal;
    b->eps = p->eps;
    b->st_step = causal ? kBwdChunk : kBwdSeg;
    b->n_st = (b->N + b->st_step - 1) / b->st_step;
    b->n_sg = (b->N + kBwdSeg - 1) / kBwdSeg;
    const int64_t rows = b->BH * b->N;
    const int64_t rec = (int64_t)b->K * b->dva;
    // one product's grid: tiles x batches must fit a 32-bit launch
    const int64_t widest = std::max<int64_t>(std::max<int64_t>(b->K, b->dva), std::max<int64_t>(2 * b->d_r, b->dxa));
    if (b->BH * std::max(b->n_st, b->n_sg) * ((kBwdSeg + 63) / 64) * ((widest + 63) / 64) > INT32_MAX ||
        rows / 4 + 1 > INT32_MAX || b->BH * ((rec + 255) / 256) > INT32_MAX ||
        b->H * (((int64_t)b->K * b->d_r + 255) / 256) > INT32_MAX || b->H * (((int64_t)b->K * b->dxa + 63) / 64) > INT32_MAX)
        return fail(GMA_ERROR_NOT_SUPPORTED, "problem too large for the backward grids");
    const int64_t C = b->st_step;
    size_t off = 0;
    auto take = [&](size_t* o, int64_t floats) {
        *o = off;
        off = align_up(off + (size_t)floats * sizeof(float), 256);
    };
    const int KT = bwd_gamma_tiles(b->K);
    b->fq = causal && bwd_chunk_q_supported(b->K, b->d_v, b->f32) && b->dva == b->d_v + 4;
    const int64_t gen = b->fq ? 0 : 1;   // arrays only the general path uses
    const int64_t stage = (rows * b->d_v * 2 + 3) / 4;   // bf16 rows of V or dO, in floats
    take(&b->off_bf, b->H * ((b->d_r + 15) / 16) * 2 * KT * 256);
    take(&b->off_cq, b->H * 16 * KT * 2);   // fp64
    take(&b->off_mw, b->H * b->K * 2 * b->d_r);
    take(&b->off_gq, rows * b->K);
    take(&b->off_gk, rows * b->K);
    take(&b->off_dgq, rows * b->K);
    take(&b->off_dgk, rows * b->K);
    take(&b->off_gh, rows * 2);
    take(&b->off_pp, gen * rows * b->dva);
    take(&b->off_st, b->BH * b->n_st * rec);
    take(&b->off_rt, gen * b->BH * b->n_st * rec);
    if (b->fq) b->off_rt = b->off_st;
    take(&b->off_ac, causal ? gen * b->BH * b->n_st * C * C : 0);
    take(&b->off_mt, causal ? gen * b->BH * b->n_st * C * C : 0);
    take(&b->off_dvt, causal ? gen * rows * b->d_v : 0);
    take(&b->off_vs, b->fq ? stage : 0);
    take(&b->off_dvs, b->fq ? stage : 0);
    take(&b->off_gp, std::max<int64_t>(2 * b->BH * b->n_sg * b->K * b->dxa, b->fq ? stage : 0));
    b->off_ds = b->off_gp;
    take(&b->off_gs, b->H * b->K * b->dxa);   // the partials summed per head
    // causal: the state segments' totals, then their exclusive prefixes
    b->sper = causal ? bwd_state_segment(b->BH, b->n_st) : 1;
    take(&b->off_sgs, causal ? b->BH * ((b->n_st + b->sper - 1) / b->sper) * rec : 0);
    b->total = off;
    return GMA_SUCCESS;
}

// Workspace bytes advertised for (problem, op): the register-staged plan or the token-split plan,
// whichever is larger (which one runs is decided per call from pointer alignment).  0 if invalid.
size_t advertised_workspace(const gma_problem_t* problem, int op) {
    if (op == GMA_OP_BACKWARD_BIDIR || op == GMA_OP_BACKWARD_CAUSAL) {
        BwdPlan b;
        return make_bwd_plan(problem, op == GMA_OP_BACKWARD_CAUSAL, &b) == GMA_SUCCESS ? b.total : 0;
    }
    Plan pl;
    if (make_plan(problem, op, &pl) != GMA_SUCCESS) return 0;
    size_t total = pl.total;
    Plan pt;
    if (op != GMA_OP_RESPONSIBILITIES && op != GMA_OP_RESPONSIBILITY_STATS && !pl.generic && pl.cls->tok_out_causal &&
        make_plan(problem, op, &pt, true) == GMA_SUCCESS)
        total = std::max(total, pt.total);
    return total;
}

bool misaligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) != 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

// ---------------------------------------------------------------------------------- timing
struct Timing {
    std::mutex mu;
    bool enabled = false;
    std::vector<std::pair<hipEvent_t, hipEvent_t>> recorded[K_COUNT];
    std::vector<hipEvent_t> pool;
} g_timing;

hipEvent_t take_event() {
    if (!g_timing.pool.empty()) {
        hipEvent_t e = g_timing.pool.back();
        g_timing.pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

template <class F>
gma_status_t timed_launch(int kid, hipStream_t s, F&& launch) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    bool timing = false;
    {
        std::lock_guard<std::mutex> lk(g_timing.mu);
        if (g_timing.enabled) {
            e0 = take_event();
            e1 = take_event();
            timing = e0 && e1;
        }
    }
    if (timing) (void)hipEventRecord(e0, s);
    launch();
    const hipError_t err = hipGetLastError();
    if (timing) {
        (void)hipEventRecord(e1, s);
        std::lock_guard<std::mutex> lk(g_timing.mu);
        g_timing.recorded[kid].emplace_back(e0, e1);
    }
    if (err != hipSuccess)
        return fail(GMA_ERROR_LAUNCH, "launch of %s failed: %s", kKernelNames[kid], hipGetErrorString(err));
    return GMA_SUCCESS;
}

// ---------------------------------------------------------------------------------- launches
// scan over the P segment aggregates of each (batch, head), fixed order (deterministic).
// causal: seg[bh][s] <- init[bh] + sum_{t < s} seg[bh][t] (exclusive prefix, in place; init = 0 if
//         NULL); n_agg = aggregates present (P, or P - 1 when the last one was not computed);
//         total[bh] <- init[bh] + sum of all P aggregates (only when n_agg = P and total != NULL)
// bidir : seg[bh][0] <- sum_{t < P} seg[bh][t]
// The P records of (batch, head) y start at record y * stride + s0 (stride = P, s0 = 0 for one pass
// over the sequence; a round of the causal pair scans its own P records with init = the total of the
// previous rounds).  init and total are [B*H, rec] and may be the same buffer (read before written).
__global__ void __launch_bounds__(256) scan_kernel(float* seg, int P, int stride, int s0, int64_t rec, int causal,
                                                   int n_agg, const float* init, float* total) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= rec) return;
    float* base = seg + ((int64_t)blockIdx.y * stride + s0) * rec + e;
    const int n = causal ? n_agg : P;
    float run = (causal && init) ? init[(int64_t)blockIdx.y * rec + e] : 0.f;
    // groups of 16 independent loads, then the sequential sum over the group
    for (int g0 = 0; g0 < P; g0 += 16) {
        float x[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) x[j] = (g0 + j < n) ? base[(int64_t)(g0 + j) * rec] : 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            if (causal && g0 + j < P) base[(int64_t)(g0 + j) * rec] = run;
            run += x[j];
        }
    }
    if (!causal) base[0] = run;
    else if (total && n_agg == P) total[(int64_t)blockIdx.y * rec + e] = run;
}

// Carried state [B*H, K, d_v + 1] (row k: Vt[k, 0 .. d_v-1], then Z[k]) <-> state record in the
// kernels' accumulator-fragment order: element (component c, column j) of Vt at
// ((c/16 * VC/16 + j/16) * 64 + (c%16)/4 * 16 + j%16) * 4 + c%4, then Z[c] at KC*VC + c.
// Padding components and columns are zero in a record.
__global__ void __launch_bounds__(256) state_to_record(const float* state, float* recs, int K, int dv, int KC,
                                                       int VC, int64_t rec) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= rec) return;
    const float* sb = state + (int64_t)blockIdx.y * K * (dv + 1);
    int c, j;
    if (e < (int64_t)KC * VC) {
        const int i = (int)(e & 3), lane = (int)((e >> 2) & 63), t = (int)(e >> 8);
        const int ct = t / (VC / 16), vt = t % (VC / 16);
        c = ct * 16 + (lane >> 4) * 4 + i;
        j = vt * 16 + (lane & 15);
    } else {
        c = (int)(e - (int64_t)KC * VC);
        j = dv;
    }
    const bool in = (e < (int64_t)KC * VC) ? (c < K && j < dv) : (c < K);
    recs[(int64_t)blockIdx.y * rec + e] = in ? sb[(int64_t)c * (dv + 1) + j] : 0.f;
}

__global__ void __launch_bounds__(256) record_to_state(const float* recs, float* state, int K, int dv, int KC,
                                                       int VC, int64_t rec) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;   // element (c, j) of the state
    if (e >= (int64_t)K * (dv + 1)) return;
    const int c = (int)(e / (dv + 1)), j = (int)(e % (dv + 1));
    const int64_t r = (j < dv) ? (((int64_t)(c / 16) * (VC / 16) + j / 16) * 64 + (c % 16) / 4 * 16 + j % 16) * 4 + c % 4
                               : (int64_t)KC * VC + c;
    state[(int64_t)blockIdx.y * K * (dv + 1) + e] = recs[(int64_t)blockIdx.y * rec + r];
}

// Responsibility diagnostics over Gamma [BH, N, K] fp32, first level: workgroup (s, bh) takes rows
// [s rows_per_seg, (s + 1) rows_per_seg) of head bh, wave w every fourth of them; lane l holds
// components l, l + 64, ...  Per row: the usage sums (sequential per lane) and the hard assignment
// (largest gamma, ties to the lowest component, by butterflies).  Partials in a fixed order.
__global__ void __launch_bounds__(256) stats_partial_kernel(const float* gamma, float* pu, uint32_t* pc, int64_t N, int K,
                                                            int S, int64_t rows_per_seg) {
    const int s = blockIdx.x;
    const int64_t bh = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t r0 = (int64_t)s * rows_per_seg, r1 = std::min<int64_t>(N, r0 + rows_per_seg);
    float use[4] = {0.f, 0.f, 0.f, 0.f};
    uint32_t cnt[4] = {0u, 0u, 0u, 0u};
    __shared__ float s_u[4][256];
    __shared__ uint32_t s_c[4][256];
    for (int64_t r = r0 + w; r < r1; r += 4) {
        const float* row = gamma + (bh * N + r) * K;
        float best = -1.f;
        int bi = K;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int k = lane + 64 * u;
            if (k < K) {
                const float g = row[k];
                use[u] += g;
                if (g > best) { best = g; bi = k; }
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const float ob = __shfl_xor(best, o, 64);
            const int oi = __shfl_xor(bi, o, 64);
            if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (bi == lane + 64 * u) ++cnt[u];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        s_u[w][lane + 64 * u] = use[u];
        s_c[w][lane + 64 * u] = cnt[u];
    }
    __syncthreads();
    for (int k = tid; k < K; k += 256) {
        pu[(bh * S + s) * K + k] = ((s_u[0][k] + s_u[1][k]) + s_u[2][k]) + s_u[3][k];
        pc[(bh * S + s) * K + k] = s_c[0][k] + s_c[1][k] + s_c[2][k] + s_c[3][k];
    }
}

// Second level: usage and counts summed over the segments in order; usage entropy of usage / N,
// normalised by ln K.
__global__ void __launch_bounds__(256) stats_final_kernel(const float* pu, const uint32_t* pc, float* usage,
                                                          uint32_t* hard, float* entropy, int64_t N, int K, int S) {
    const int64_t bh = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    __shared__ float s_e[4];
    float e = 0.f;
    for (int k = tid; k < K; k += 256) {
        float u = 0.f;
        uint32_t c = 0u;
        for (int q = 0; q < S; ++q) {
            u += pu[(bh * S + q) * K + k];
            c += pc[(bh * S + q) * K + k];
        }
        usage[bh * K + k] = u;
        hard[bh * K + k] = c;
        const float p = u / (float)N;
        if (p > 0.f) e -= p * logf(p);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) e += __shfl_xor(e, o, 64);
    if (lane == 0) s_e[w] = e;
    __syncthreads();
    // normalised by its largest value ln K (0 for K = 1)
    if (tid == 0) entropy[bh] = K > 1 ? (((s_e[0] + s_e[1]) + s_e[2]) + s_e[3]) / logf((float)K) : 0.f;
}

gma_status_t launch_prep(const Plan& pl, const float* mu, const float* rv, const float* pr, char* ws, hipStream_t s) {
    PrepArgs pa;
    pa.mu = mu;
    pa.raw_var = rv;
    pa.prior = pr;
    pa.ab = ws + pl.off_ab;
    pa.cvec = reinterpret_cast<float*>(ws + pl.off_c);
    pa.H = (int)pl.H;
    pa.K = pl.K;
    pa.d_r = pl.d_r;
    pa.flags = pl.flags ? reinterpret_cast<int*>(ws + pl.off_flags) : nullptr;
    pa.n_flags = pl.B * pl.H;
    return timed_launch(K_PREP, s, [&] { pl.cls->prep(pa, (int)pl.H, s); });
}

MainArgs base_args(const Plan& pl, char* ws) {
    MainArgs a;
    std::memset(&a, 0, sizeof(a));
    a.ab = ws + pl.off_ab;
    a.cvec = reinterpret_cast<const float*>(ws + pl.off_c);
    a.seg = reinterpret_cast<float*>(ws + pl.off_seg);
    a.gk = pl.gtiles ? ws + pl.off_gk : nullptr;
    a.N = pl.N;
    a.H = (int)pl.H;
    a.P = pl.P;
    a.Pg = pl.P;
    a.d_r = pl.d_r;
    a.d_v = pl.d_v;
    a.K = pl.K;
    a.seg_chunks = pl.seg_chunks;
    a.eps = pl.eps;
    a.flags = pl.flags ? reinterpret_cast<int*>(ws + pl.off_flags) : nullptr;
    return a;
}

// Exact recomputation of the (batch, head) slices a bf16 call flagged (rows whose logits left the
// fp16 operand range); every other slice returns at once.
FixArgs fix_args(const Plan& pl, char* ws) {
    FixArgs f;
    std::memset(&f, 0, sizeof(f));
    f.flags = reinterpret_cast<const int*>(ws + pl.off_flags);
    f.scratch = reinterpret_cast<float*>(ws + pl.off_fix);
    f.BH = pl.B * pl.H;
    f.N = pl.N;
    f.N_kv = pl.N;
    f.H = (int)pl.H;
    f.K = pl.K;
    f.d_r = pl.d_r;
    f.d_v = pl.d_v;
    f.eps = pl.eps;
    return f;
}

gma_status_t launch_fixup(const Plan& pl, FixArgs f, bool forward, bool causal, hipStream_t s) {
    bool ok = true;
    const gma_status_t st = timed_launch(K_FIXUP, s, [&] {
        ok = forward ? launch_fixup_forward(f, pl.cls->kc, pl.cls->vc, pl.B * pl.H, causal, s)
             : f.stat_usage ? launch_fixup_stats(f, pl.cls->kc, pl.B * pl.H, s)
                            : launch_fixup_resp(f, pl.cls->kc, pl.B * pl.H, s);
    });
    if (!ok) return fail(GMA_ERROR_LAUNCH, "no out-of-range recomputation kernel for class K=%d d_v=%d", pl.cls->kc,
                         pl.cls->vc);
    return st;
}

int vec_ok(const void* ptr, int d, bool f32) {
    const int vec = f32 ? 4 : 8;  // elements per 16 bytes
    return (d % vec == 0) && !misaligned(ptr, 16);
}

int vec_o_ok(const void* ptr, int d, bool f32) {
    return (d % 4 == 0) && !misaligned(ptr, f32 ? 16 : 8);
}

// size_check = false: the caller checks the workspace size against the plan it finally runs
gma_status_t check_common(const gma_problem_t* p, const void* const* ptrs, int nptrs, void* ws, size_t ws_bytes,
                          const Plan& pl, bool size_check = true) {
    for (int i = 0; i < nptrs; ++i)
        if (!ptrs[i]) return fail(GMA_ERROR_INVALID_VALUE, "pointer argument %d is NULL", i);
    if (size_check && ws_bytes < pl.total)
        return fail(GMA_ERROR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes is smaller than the %zu bytes needed",
                    ws_bytes, pl.total);
    if (pl.total > 0 && !ws) return fail(GMA_ERROR_INVALID_VALUE, "workspace is NULL");
    if (ws && misaligned(ws, 16)) return fail(GMA_ERROR_INVALID_VALUE, "workspace must be 16-byte aligned");
    (void)p;
    return GMA_SUCCESS;
}

// ---------------------------------------------------------------------------------- generic path
// Carried state [B*H, K, d_v + 1] <-> generic record [B*H, K, dva] (row k: Vt[k, :], Z[k], zeros).
__global__ void __launch_bounds__(256) state_to_genrec(const float* state, float* recs, int K, int dv, int dva) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= (int64_t)K * dva) return;
    const int k = (int)(e / dva), j = (int)(e % dva);
    recs[(int64_t)blockIdx.y * K * dva + e] = j <= dv ? state[((int64_t)blockIdx.y * K + k) * (dv + 1) + j] : 0.f;
}

__global__ void __launch_bounds__(256) genrec_to_state(const float* recs, float* state, int K, int dv, int dva) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= (int64_t)K * (dv + 1)) return;
    const int k = (int)(e / (dv + 1)), j = (int)(e % (dv + 1));
    state[(int64_t)blockIdx.y * K * (dv + 1) + e] = recs[((int64_t)blockIdx.y * K + k) * dva + j];
}

// O = num / (den + eps) per row from p [rows, dva] = [num | den | 0 ..], in the storage dtype.
__global__ void __launch_bounds__(256) generic_out_kernel(const float* p, void* o, int64_t rows, int dv, int dva,
                                                          float eps, int f32) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= rows * dv) return;
    const int64_t r = e / dv;
    const int j = (int)(e % dv);
    const float val = p[r * dva + j] / (p[r * dva + dv] + eps);
    if (f32) reinterpret_cast<float*>(o)[e] = val;
    else reinterpret_cast<uint16_t*>(o)[e] = bf16_bits(val);
}

// Responsibilities of x [BH, N, d_r] in fp32 on the generic path -> gamma [BH, N, K].
gma_status_t generic_gamma(const Plan& pl, const void* x, const float* mu, const float* rv, const float* pr,
                           float* gamma, int64_t N, char* w, hipStream_t s, bool prep) {
    float* bf = reinterpret_cast<float*>(w + pl.off_gbf);
    double* cq = reinterpret_cast<double*>(w + pl.off_gcq);
    if (prep) {
        const gma_status_t st = timed_launch(K_GEN_PREP, s, [&] {
            launch_bwd_frag(mu, rv, pr, bf, cq, (int)pl.H, pl.K, pl.d_r, false, s);
        });
        if (st != GMA_SUCCESS) return st;
    }
    return timed_launch(K_GEN_GAMMA, s, [&] {
        launch_bwd_gamma_mfma(x, pl.f32, bf, cq, gamma, pl.B * pl.H, N, (int)pl.H, pl.K, pl.d_r, s);
    });
}

// Forward on the generic path (the plan from make_generic_plan; n_q query rows, n_kv key / value rows,
// equal when causal).  Write phase: records Gamma_K^T [V | 1] per entry (a 64-token chunk when causal, a
// 1024-token segment otherwise), then the fixed-order scan of the forward (exclusive prefix from the
// initial state when causal, the total into entry 0 otherwise).  Read phase: [num | den] = Gamma_Q
// times the record each entry reads, plus (causal) tril(Gamma_Q Gamma_K^T) [V | 1] within the chunk;
// O = num / (den + eps).
gma_status_t forward_generic(const Plan& pl, bool causal, int64_t n_q, int64_t n_kv, const void* qx, const void* kx,
                             const void* v, const float* mu, const float* rv, const float* pr, const float* state_in,
                             float* state_out, void* o, char* w, hipStream_t s) {
    const int64_t BH = pl.B * pl.H;
    const int K = pl.K, d_v = pl.d_v, dva = pl.gen_dva, step = pl.gen_step;
    const int64_t rec = (int64_t)K * dva;
    const int64_t nst_k = (n_kv + step - 1) / step, nst_q = (n_q + step - 1) / step;
    auto F = [&](size_t off) { return reinterpret_cast<float*>(w + off); };
    float *gq = F(pl.off_gq), *gk = F(pl.off_ggk), *pp = F(pl.off_gpp), *st = F(pl.off_gst), *ac = F(pl.off_gac);
    float* rin = state_in ? F(pl.off_grin) : nullptr;
    float* rout = state_out ? F(pl.off_grout) : nullptr;
    gma_status_t r = generic_gamma(pl, qx, mu, rv, pr, gq, n_q, w, s, true);
    if (r != GMA_SUCCESS) return r;
    r = generic_gamma(pl, kx, mu, rv, pr, gk, n_kv, w, s, false);
    if (r != GMA_SUCCESS) return r;
    struct View { const float* p; int64_t s0, s1; int ld; };
    auto gemm = [&](View A, bool ta, View B, bool tb, View C, float* out, int M, int Nn, int Kd, int tokf, int tril,
                    const float* cin, int64_t ntok, int64_t n_inner, BwdGen gb) -> gma_status_t {
        BwdGemm g;
        g.gb = gb;
        g.A = A.p; g.sA0 = A.s0; g.sA1 = A.s1; g.lda = A.ld;
        g.B = B.p; g.sB0 = B.s0; g.sB1 = B.s1; g.ldb = B.ld;
        g.C = out; g.sC0 = C.s0; g.sC1 = C.s1; g.ldc = C.ld;
        g.Cin = cin;
        g.beta = cin ? 1.f : 0.f;
        g.M = M; g.N = Nn; g.Kd = Kd;
        g.n_outer = BH;
        g.n_inner = (int)n_inner;
        g.ntok = ntok;
        g.tok_step = step;
        g.tok_flags = tokf;
        g.tril = tril;
        g.split = pl.f32 ? 0 : 1;   // bf16 storage: split-bf16 products on the bf16 matrix cores
        bool ok = true;
        const gma_status_t ls = timed_launch(K_GEN_GEMM, s, [&] { ok = launch_bwd_gemm(g, ta, tb, false, s); });
        if (!ok) return fail(GMA_ERROR_LAUNCH, "no product kernel for this operand combination");
        return ls;
    };
    constexpr int TM = 1, TN = 2, TK = 4;   // token axes of a product
    const BwdGen gen_v{v, nullptr, GEN_VAUG, pl.f32 ? 1 : 0, d_v};
    const View v_rows{nullptr, n_kv, step, 1};   // [V | 1] generated from V (views count rows)
    // write phase
    r = gemm(View{gk, n_kv * K, (int64_t)step * K, K}, true, v_rows, false, View{st, nst_k * rec, rec, dva}, st, K, dva,
             step, TK, 0, nullptr, n_kv, nst_k, gen_v);
    if (r != GMA_SUCCESS) return r;
    if (rin) {
        r = timed_launch(K_STATE, s, [&] {
            hipLaunchKernelGGL(state_to_genrec, dim3((unsigned)((rec + 255) / 256), (unsigned)BH), dim3(256), 0, s,
                               state_in, rin, K, d_v, dva);
        });
        if (r != GMA_SUCCESS) return r;
    }
    r = timed_launch(K_GEN_SCAN, s, [&] {
        hipLaunchKernelGGL(scan_kernel, dim3((unsigned)((rec + 255) / 256), (unsigned)BH), dim3(256), 0, s, st,
                           (int)nst_k, (int)nst_k, 0, rec, causal ? 1 : 0, (int)nst_k, (const float*)rin, rout);
    });
    if (r != GMA_SUCCESS) return r;
    // read phase
    r = gemm(View{gq, n_q * K, (int64_t)step * K, K}, false, View{st, nst_k * rec, causal ? rec : 0, dva}, false,
             View{pp, n_q * dva, (int64_t)step * dva, dva}, pp, step, dva, K, TM, 0, nullptr, n_q, nst_q, BwdGen{});
    if (r != GMA_SUCCESS) return r;
    if (causal) {
        const int64_t C = step;
        r = gemm(View{gq, n_q * K, C * K, K}, false, View{gk, n_kv * K, C * K, K}, true,
                 View{ac, nst_q * C * C, C * C, (int)C}, ac, (int)C, (int)C, K, TM | TN, 1, nullptr, n_q, nst_q, BwdGen{});
        if (r != GMA_SUCCESS) return r;
        r = gemm(View{ac, nst_q * C * C, C * C, (int)C}, false, v_rows, false, View{pp, n_q * dva, C * dva, dva}, pp,
                 (int)C, dva, (int)C, TM | TK, 0, pp, n_q, nst_q, gen_v);
        if (r != GMA_SUCCESS) return r;
    }
    const int64_t n_out = BH * n_q * d_v;
    r = timed_launch(K_GEN_OUT, s, [&] {
        hipLaunchKernelGGL(generic_out_kernel, dim3((unsigned)((n_out + 255) / 256)), dim3(256), 0, s, (const float*)pp, o,
                           BH * n_q, d_v, dva, pl.eps, pl.f32 ? 1 : 0);
    });
    if (r != GMA_SUCCESS || !rout) return r;
    const int64_t nstate = (int64_t)K * (d_v + 1);
    return timed_launch(K_STATE, s, [&] {
        hipLaunchKernelGGL(genrec_to_state, dim3((unsigned)((nstate + 255) / 256), (unsigned)BH), dim3(256), 0, s,
                           (const float*)rout, state_out, K, d_v, dva);
    });
}

// op: GMA_OP_FORWARD_BIDIR, GMA_OP_FORWARD_CAUSAL or GMA_OP_FORWARD_CAUSAL_STATE (state_in /
// state_out used only by the last; either may be NULL)
gma_status_t forward(const gma_problem_t* p, int op, const void* qx, const void* kx, const void* v,
                     const float* mu, const float* rv, const float* pr, const float* state_in, float* state_out,
                     void* o, void* ws, size_t ws_bytes, void* stream) {
    g_last_error.clear();
    const bool causal = op != GMA_OP_FORWARD_BIDIR;
    const bool stateful = op == GMA_OP_FORWARD_CAUSAL_STATE;
    Plan pl;
    gma_status_t st = make_plan(p, op, &pl);
    if (st != GMA_SUCCESS) return st;
    const void* ptrs[] = {qx, kx, v, mu, rv, pr, o};
    st = check_common(p, ptrs, 7, ws, ws_bytes, pl, false);
    if (st != GMA_SUCCESS) return st;
    const size_t es = pl.f32 ? 4 : 2;
    for (const void* ptr : {qx, kx, v, (const void*)o})
        if (misaligned(ptr, es)) return fail(GMA_ERROR_INVALID_VALUE, "tensor pointers must be %zu-byte aligned", es);
    for (const void* ptr : {(const void*)mu, (const void*)rv, (const void*)pr})
        if (misaligned(ptr, 4)) return fail(GMA_ERROR_INVALID_VALUE, "parameter pointers must be 4-byte aligned");
    const size_t nx = (size_t)(pl.B * pl.H * pl.N) * pl.d_r * es;
    const size_t nv = (size_t)(pl.B * pl.H * pl.N) * pl.d_v * es;
    if (overlaps(o, nv, qx, nx) || overlaps(o, nv, kx, nx) || overlaps(o, nv, v, nv))
        return fail(GMA_ERROR_INVALID_VALUE, "o must not overlap qx, kx or v");
    const size_t ns = (size_t)(pl.B * pl.H) * pl.K * (pl.d_v + 1) * sizeof(float);
    if (stateful) {
        if (misaligned(state_in, 4) || misaligned(state_out, 4))
            return fail(GMA_ERROR_INVALID_VALUE, "state pointers must be 4-byte aligned");
        for (const void* sp : {(const void*)state_in, (const void*)state_out}) {
            if (sp && (overlaps(sp, ns, qx, nx) || overlaps(sp, ns, kx, nx) || overlaps(sp, ns, v, nv) ||
                       overlaps(sp, ns, o, nv)))
                return fail(GMA_ERROR_INVALID_VALUE, "states must not overlap qx, kx, v or o");
        }
        if (state_in && state_out && state_in != state_out && overlaps(state_in, ns, state_out, ns))
            return fail(GMA_ERROR_INVALID_VALUE, "state_in and state_out must be the same buffer or disjoint");
    }

    if (pl.generic) {
        if (ws_bytes < pl.total)
            return fail(GMA_ERROR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes is smaller than the %zu bytes needed",
                        ws_bytes, pl.total);
        if (overlaps(ws, pl.total, qx, nx) || overlaps(ws, pl.total, kx, nx) || overlaps(ws, pl.total, v, nv) ||
            overlaps(ws, pl.total, o, nv) ||
            (stateful && (overlaps(ws, pl.total, state_in, state_in ? ns : 0) ||
                          overlaps(ws, pl.total, state_out, state_out ? ns : 0))))
            return fail(GMA_ERROR_INVALID_VALUE, "workspace must not overlap the tensors");
        return forward_generic(pl, causal, pl.N, pl.N, qx, kx, v, mu, rv, pr, stateful ? state_in : nullptr,
                               stateful ? state_out : nullptr, o, reinterpret_cast<char*>(ws),
                               reinterpret_cast<hipStream_t>(stream));
    }
    // Token-split LDS-DMA kernels: bf16, rows in whole 16-byte chunks, 16-byte aligned bases, byte
    // offsets within one (batch, head) slice (one chunk past the end included) below 2^31.
    const bool dma = !pl.f32 && pl.cls->tok_out_causal && pl.d_r % 8 == 0 && pl.d_v % 8 == 0 &&
                     !misaligned(qx, 16) && !misaligned(kx, 16) && !misaligned(v, 16) && !misaligned(o, 16) &&
                     (pl.N + kTokChunk) * std::max(pl.d_r, pl.d_v) * 2 < (int64_t(1) << 31);
    if (dma) {
        st = make_plan(p, op, &pl, true);
        if (st != GMA_SUCCESS) return st;
        if (pl.gtiles && ws_bytes < advertised_workspace(p, op)) {
            // less than the advertised workspace: no stored Gamma_K tiles, the causal output pass
            // recomputes Gamma_K
            st = make_plan(p, op, &pl, true, false);
            if (st != GMA_SUCCESS) return st;
        }
    }
    // the workspace against the plan that runs
    if (ws_bytes < pl.total)
        return fail(GMA_ERROR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes is smaller than the %zu bytes needed",
                    ws_bytes, pl.total);
    if (ws && (overlaps(ws, pl.total, qx, nx) || overlaps(ws, pl.total, kx, nx) || overlaps(ws, pl.total, v, nv) ||
               overlaps(ws, pl.total, o, nv) || (stateful && (overlaps(ws, pl.total, state_in, state_in ? ns : 0) ||
                                                              overlaps(ws, pl.total, state_out, state_out ? ns : 0)))))
        return fail(GMA_ERROR_INVALID_VALUE, "workspace must not overlap the tensors");

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char* w = reinterpret_cast<char*>(ws);
    st = launch_prep(pl, mu, rv, pr, w, s);
    if (st != GMA_SUCCESS) return st;
    MainArgs a = base_args(pl, w);
    a.qx = qx;
    a.kx = kx;
    a.v = v;
    a.o = o;
    a.vec_x = vec_ok(qx, pl.d_r, pl.f32) && vec_ok(kx, pl.d_r, pl.f32);
    a.vec_v = vec_ok(v, pl.d_v, pl.f32);
    a.vec_o = vec_o_ok(o, pl.d_v, pl.f32);
    const bool gt = dma && pl.gtiles;
    const main_launch_t f_agg = gt ? pl.cls->tok_agg_g : dma ? pl.cls->tok_agg : pl.cls->agg;
    const main_launch_t f_causal = gt ? pl.cls->tok_out_causal_g : dma ? pl.cls->tok_out_causal : pl.cls->out_causal;
    const main_launch_t f_bidir = dma ? pl.cls->tok_out_bidir : pl.cls->out_bidir;
    const int grid = (int)(pl.B * pl.H * pl.P);
    const int64_t rec = (int64_t)pl.cls->kc * pl.cls->vc + pl.cls->kc;
    const unsigned BH = (unsigned)(pl.B * pl.H);
    // carried state: the initial and the final state as records in the workspace
    float* rec_in = (stateful && state_in) ? reinterpret_cast<float*>(w + pl.off_state) : nullptr;
    float* rec_out = (stateful && state_out) ? reinterpret_cast<float*>(w + pl.off_state) + BH * rec : nullptr;
    if (rec_in) {
        st = timed_launch(K_STATE, s, [&] {
            hipLaunchKernelGGL(state_to_record, dim3((unsigned)((rec + 255) / 256), BH), dim3(256), 0, s, state_in,
                               rec_in, pl.K, pl.d_v, pl.cls->kc, pl.cls->vc, rec);
        });
        if (st != GMA_SUCCESS) return st;
    }
    if (!causal) {
        const int n_agg = (int)pl.P;
        MainArgs ag = a;
        st = timed_launch(K_AGG, s, [&] { f_agg(ag, (int)(pl.B * pl.H * n_agg), s); });
        if (st != GMA_SUCCESS) return st;
        const bool read_sum = pl.P <= kBidirReadSum;
        if (pl.P > 1 && !read_sum) {
            st = timed_launch(K_SCAN, s, [&] {
                hipLaunchKernelGGL(scan_kernel, dim3((unsigned)((rec + 255) / 256), BH), dim3(256), 0, s, a.seg, pl.P,
                                   pl.P, 0, rec, 0, n_agg, (const float*)nullptr, (float*)nullptr);
            });
            if (st != GMA_SUCCESS) return st;
        }
        a.bidir_segs = read_sum ? pl.P : 1;
        st = timed_launch(K_OUT_BIDIR, s, [&] { f_bidir(a, grid, s); });
        if (st != GMA_SUCCESS || !pl.flags) return st;
        FixArgs f = fix_args(pl, w);
        f.qx = qx;
        f.kx = kx;
        f.v = v;
        f.o = o;
        f.mu = mu;
        f.raw_var = rv;
        f.prior = pr;
        return launch_fixup(pl, f, true, false, s);
    }
    // Causal: rounds r = 0 .. rounds - 1, each over P_round consecutive segments of every (batch, head)
    // (one round when the plan has none): aggregate pass, exclusive prefix of the round's aggregates
    // from the total of the earlier rounds (the initial state, or zero, in round 0), output pass.  A
    // round's records and Gamma_K tiles are reused by the next round.
    float* run_total = pl.rounds > 1 ? reinterpret_cast<float*>(w + pl.off_total) : nullptr;
    a.P = pl.rounds > 1 ? pl.P_round : pl.P;
    a.gk_ring = pl.gk_ring;
    for (int r = 0; r < pl.rounds; ++r) {
        const int s0 = r * pl.P_round;
        const int np = std::min(pl.P_round, pl.P - s0);
        const bool last = r + 1 == pl.rounds;
        // the last segment's aggregate is needed only for the final state, but with stored tiles its
        // Gamma_K tiles are
        const int n_agg = (!last || gt || rec_out) ? np : np - 1;
        MainArgs ar = a;
        ar.seg0 = s0;
        if (n_agg > 0) {
            MainArgs ag = ar;
            ag.Pg = n_agg;
            st = timed_launch(K_AGG, s, [&] { f_agg(ag, (int)(pl.B * pl.H * n_agg), s); });
            if (st != GMA_SUCCESS) return st;
        }
        const float* init = r == 0 ? (const float*)rec_in : run_total;
        float* tot = last ? rec_out : run_total;
        if (np > 1 || init || tot) {
            st = timed_launch(K_SCAN, s, [&] {
                hipLaunchKernelGGL(scan_kernel, dim3((unsigned)((rec + 255) / 256), BH), dim3(256), 0, s, a.seg, np,
                                   a.P, 0, rec, 1, n_agg, init, tot);
            });
            if (st != GMA_SUCCESS) return st;
        }
        ar.Pg = np;
        ar.has_carry = np > 1 || init;
        st = timed_launch(K_OUT_CAUSAL, s, [&] { f_causal(ar, (int)(pl.B * pl.H * np), s); });
        if (st != GMA_SUCCESS) return st;
    }
    if (rec_out) {
        const int64_t nstate = (int64_t)pl.K * (pl.d_v + 1);
        st = timed_launch(K_STATE, s, [&] {
            hipLaunchKernelGGL(record_to_state, dim3((unsigned)((nstate + 255) / 256), BH), dim3(256), 0, s,
                               (const float*)rec_out, state_out, pl.K, pl.d_v, pl.cls->kc, pl.cls->vc, rec);
        });
        if (st != GMA_SUCCESS) return st;
    }
    if (!pl.flags) return GMA_SUCCESS;
    // flagged slices are recomputed from the inputs (and the initial state's record, which no kernel
    // above has written), after the final state was written, so they overwrite O and the state
    FixArgs f = fix_args(pl, w);
    f.qx = qx;
    f.kx = kx;
    f.v = v;
    f.o = o;
    f.mu = mu;
    f.raw_var = rv;
    f.prior = pr;
    f.rec_in = rec_in;
    f.state_out = rec_out ? state_out : nullptr;
    return launch_fixup(pl, f, true, true, s);
}

// Bidirectional forward with N_q query rows (problem->seq_len) and N_kv key/value rows: the
// aggregate pass and the workspace follow the key/value sequence, the read pass the queries (its
// grid has its own segments; it reads the total [Vt | Z] at the key side's record stride).
gma_status_t forward_bidir_kv(const gma_problem_t* p, int64_t n_kv, const void* qx, const void* kx, const void* v,
                              const float* mu, const float* rv, const float* pr, void* o, void* ws, size_t ws_bytes,
                              void* stream) {
    g_last_error.clear();
    if (!p) return fail(GMA_ERROR_INVALID_VALUE, "problem is NULL");
    if (n_kv < 1) return fail(GMA_ERROR_INVALID_VALUE, "seq_len_kv must be >= 1 (got %lld)", (long long)n_kv);
    gma_problem_t pk = *p;
    pk.seq_len = n_kv;
    Plan plq, plk;
    gma_status_t st = make_plan(p, GMA_OP_FORWARD_BIDIR, &plq);
    if (st != GMA_SUCCESS) return st;
    st = make_plan(&pk, GMA_OP_FORWARD_BIDIR, &plk);
    if (st != GMA_SUCCESS) return st;
    const void* ptrs[] = {qx, kx, v, mu, rv, pr, o};
    st = check_common(p, ptrs, 7, ws, ws_bytes, plk, false);
    if (st != GMA_SUCCESS) return st;
    const size_t es = plq.f32 ? 4 : 2;
    for (const void* ptr : {qx, kx, v, (const void*)o})
        if (misaligned(ptr, es)) return fail(GMA_ERROR_INVALID_VALUE, "tensor pointers must be %zu-byte aligned", es);
    for (const void* ptr : {(const void*)mu, (const void*)rv, (const void*)pr})
        if (misaligned(ptr, 4)) return fail(GMA_ERROR_INVALID_VALUE, "parameter pointers must be 4-byte aligned");
    const int64_t BH = plq.B * plq.H;
    const size_t nq = (size_t)(BH * plq.N) * plq.d_r * es, nk = (size_t)(BH * n_kv) * plq.d_r * es;
    const size_t nv = (size_t)(BH * n_kv) * plq.d_v * es, no = (size_t)(BH * plq.N) * plq.d_v * es;
    if (overlaps(o, no, qx, nq) || overlaps(o, no, kx, nk) || overlaps(o, no, v, nv))
        return fail(GMA_ERROR_INVALID_VALUE, "o must not overlap qx, kx or v");
    if (plk.generic) {
        // one plan for both sides: its row buffers hold max(N_q, N_kv) rows per (batch, head)
        Plan pg;
        gma_problem_t pm = *p;
        pm.seq_len = std::max(plq.N, n_kv);
        st = make_plan(&pm, GMA_OP_FORWARD_BIDIR, &pg);
        if (st != GMA_SUCCESS) return st;
        if (ws_bytes < pg.total)
            return fail(GMA_ERROR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes is smaller than the %zu bytes needed",
                        ws_bytes, pg.total);
        if (overlaps(ws, pg.total, qx, nq) || overlaps(ws, pg.total, kx, nk) || overlaps(ws, pg.total, v, nv) ||
            overlaps(ws, pg.total, o, no))
            return fail(GMA_ERROR_INVALID_VALUE, "workspace must not overlap the tensors");
        return forward_generic(pg, false, plq.N, n_kv, qx, kx, v, mu, rv, pr, nullptr, nullptr, o,
                               reinterpret_cast<char*>(ws), reinterpret_cast<hipStream_t>(stream));
    }
    const bool dma = !plq.f32 && plq.cls->tok_out_causal && plq.d_r % 8 == 0 && plq.d_v % 8 == 0 &&
                     !misaligned(qx, 16) && !misaligned(kx, 16) && !misaligned(v, 16) && !misaligned(o, 16) &&
                     (std::max(plq.N, n_kv) + kTokChunk) * std::max(plq.d_r, plq.d_v) * 2 < (int64_t(1) << 31);
    if (dma) {
        st = make_plan(p, GMA_OP_FORWARD_BIDIR, &plq, true);
        if (st != GMA_SUCCESS) return st;
        st = make_plan(&pk, GMA_OP_FORWARD_BIDIR, &plk, true);
        if (st != GMA_SUCCESS) return st;
    }
    if (ws_bytes < plk.total)
        return fail(GMA_ERROR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes is smaller than the %zu bytes needed",
                    ws_bytes, plk.total);
    if (ws && (overlaps(ws, plk.total, qx, nq) || overlaps(ws, plk.total, kx, nk) || overlaps(ws, plk.total, v, nv) ||
               overlaps(ws, plk.total, o, no)))
        return fail(GMA_ERROR_INVALID_VALUE, "workspace must not overlap the tensors");

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char* w = reinterpret_cast<char*>(ws);
    st = launch_prep(plk, mu, rv, pr, w, s);
    if (st != GMA_SUCCESS) return st;
    // write phase over the key/value rows
    MainArgs ag = base_args(plk, w);
    ag.kx = kx;
    ag.v = v;
    ag.vec_x = vec_ok(kx, plk.d_r, plk.f32);
    ag.vec_v = vec_ok(v, plk.d_v, plk.f32);
    const main_launch_t f_agg = dma ? plk.cls->tok_agg : plk.cls->agg;
    st = timed_launch(K_AGG, s, [&] { f_agg(ag, (int)(BH * plk.P), s); });
    if (st != GMA_SUCCESS) return st;
    const int64_t rec = (int64_t)plk.cls->kc * plk.cls->vc + plk.cls->kc;
    const bool read_sum = plk.P <= kBidirReadSum;
    if (plk.P > 1 && !read_sum) {
        st = timed_launch(K_SCAN, s, [&] {
            hipLaunchKernelGGL(scan_kernel, dim3((unsigned)((rec + 255) / 256), (unsigned)BH), dim3(256), 0, s, ag.seg,
                               plk.P, plk.P, 0, rec, 0, plk.P, (const float*)nullptr, (float*)nullptr);
        });
        if (st != GMA_SUCCESS) return st;
    }
    // read phase over the query rows, the total at record stride P of the key side
    MainArgs a = base_args(plk, w);
    a.N = plq.N;
    a.Pg = plq.P;
    a.seg_chunks = plq.seg_chunks;
    a.bidir_segs = read_sum ? plk.P : 1;
    a.qx = qx;
    a.o = o;
    a.vec_x = vec_ok(qx, plq.d_r, plq.f32);
    a.vec_o = vec_o_ok(o, plq.d_v, plq.f32);
    const main_launch_t f_bidir = dma ? plq.cls->tok_out_bidir : plq.cls->out_bidir;
    st = timed_launch(K_OUT_BIDIR, s, [&] { f_bidir(a, (int)(BH * plq.P), s); });
    if (st != GMA_SUCCESS || !plk.flags) return st;
    FixArgs f = fix_args(plk, w);
    f.N = plq.N;
    f.N_kv = n_kv;
    f.qx = qx;
    f.kx = kx;
    f.v = v;
    f.o = o;
    f.mu = mu;
    f.raw_var = rv;
    f.prior = pr;
    return launch_fixup(plk, f, true, false, s);
}

// Backward (see gma_backward.hip for the formulas): all intermediates fp32 in the workspace.
gma_status_t backward(const gma_problem_t* p, bool causal, const void* qx, const void* kx, const void* v,
                      const float* mu, const float* rv, const float* pr, const void* dout, void* dqx, void* dkx,
                      void* dv, float* dmu, float* drv, float* dpr, void* ws, size_t ws_bytes, void* stream) {
    g_last_error.clear();
    BwdPlan b;
    gma_status_t st = make_bwd_plan(p, causal, &b);
    if (st != GMA_SUCCESS) return st;
    const void* ptrs[] = {qx, kx, v, mu, rv, pr, dout, dqx, dkx, dv, dmu, drv, dpr};
    for (int i = 0; i < 13; ++i)
        if (!ptrs[i]) return fail(GMA_ERROR_INVALID_VALUE, "pointer argument %d is NULL", i);
    if (ws_bytes < b.total)
        return fail(GMA_ERROR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes is smaller than the %zu bytes needed",
                    ws_bytes, b.total);
    if (!ws) return fail(GMA_ERROR_INVALID_VALUE, "workspace is NULL");
    if (misaligned(ws, 16)) return fail(GMA_ERROR_INVALID_VALUE, "workspace must be 16-byte aligned");
    const size_t es = b.f32 ? 4 : 2;
    for (const void* ptr : {qx, kx, v, dout, (const void*)dqx, (const void*)dkx, (const void*)dv})
        if (misaligned(ptr, es)) return fail(GMA_ERROR_INVALID_VALUE, "tensor pointers must be %zu-byte aligned", es);
    for (const void* ptr : {(const void*)mu, (const void*)rv, (const void*)pr, (const void*)dmu, (const void*)drv,
                            (const void*)dpr})
        if (misaligned(ptr, 4)) return fail(GMA_ERROR_INVALID_VALUE, "parameter pointers must be 4-byte aligned");
    const size_t nx = (size_t)(b.BH * b.N) * b.d_r * es, nv = (size_t)(b.BH * b.N) * b.d_v * es;
    const size_t np = (size_t)(b.H * b.K) * b.d_r * 4, nk = (size_t)(b.H * b.K) * 4;
    const void* ins[] = {qx, kx, v, dout, mu, rv, pr, ws};
    const size_t insz[] = {nx, nx, nv, nv, np, np, nk, b.total};
    const void* outs[] = {dqx, dkx, dv, dmu, drv, dpr};
    const size_t osz[] = {nx, nx, nv, np, np, nk};
    for (int i = 0; i < 6; ++i) {
        for (int j = 0; j < 8; ++j)
            if (overlaps(outs[i], osz[i], ins[j], insz[j]))
                return fail(GMA_ERROR_INVALID_VALUE, "gradients must not overlap the inputs or the workspace");
        for (int j = 0; j < i; ++j)
            if (overlaps(outs[i], osz[i], outs[j], osz[j]))
                return fail(GMA_ERROR_INVALID_VALUE, "gradients must not overlap each other");
    }

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char* w = reinterpret_cast<char*>(ws);
    auto F = [&](size_t off) { return reinterpret_cast<float*>(w + off); };
    float *mw = F(b.off_mw), *gq = F(b.off_gq), *gk = F(b.off_gk), *dgq = F(b.off_dgq),
          *dgk = F(b.off_dgk), *rs = F(b.off_gh), *pp = F(b.off_pp), *stt = F(b.off_st),
          *rt = F(b.off_rt), *ac = F(b.off_ac), *mt = F(b.off_mt), *dvt = F(b.off_dvt),
          *gp = F(b.off_gp), *gs = F(b.off_gs);
    const int64_t BH = b.BH, N = b.N, rows = BH * N, rec = (int64_t)b.K * b.dva;
    const int K = b.K, d_r = b.d_r, d_v = b.d_v, dva = b.dva, dxa = b.dxa, H = (int)b.H;
    const int C = b.st_step;
    const bool f32 = b.f32;

    // operand views: token rows of width wd per state entry (tok) or per parameter segment (seg); the
    // states of every entry (all_st) or the one each entry reads (cur_st: its own prefix / suffix when
    // causal, the total in entry 0 when bidirectional); per-chunk C x C blocks (sq)
    struct View { const float* p; int64_t s0, s1; int ld; int64_t mod; };
    auto tok = [&](const float* ptr, int wd) { return View{ptr, N * wd, (int64_t)C * wd, wd, 0}; };
    auto seg = [&](const float* ptr, int wd) { return View{ptr, N * wd, (int64_t)kBwdSeg * wd, wd, 0}; };
    auto all_st = [&](const float* ptr) { return View{ptr, b.n_st * rec, rec, dva, 0}; };
    auto cur_st = [&](const float* ptr) { return View{ptr, b.n_st * rec, causal ? rec : 0, dva, 0}; };
    auto sq = [&](const float* ptr) { return View{ptr, b.n_st * C * C, (int64_t)C * C, C, 0}; };
    auto gemm = [&](View A, bool ta, View Bv, bool tb, View Cv, void* out, bool out_bf16, int M, int Nn, int Kd,
                    int tokf, int tril, const float* cin, bool per_seg, BwdGen ga = BwdGen{}, BwdGen gb = BwdGen{},
                    const void* dx_x = nullptr) -> gma_status_t {
        BwdGemm g;
        g.ga = ga;       // generated operands (their views count rows)
        g.gb = gb;
        g.dx_x = dx_x;   // routing-input gradient epilogue: out = dx, from the pairs (dl . mu / s, dl . 1 / s)
        g.A = A.p;
        g.sA0 = A.s0;
        g.sA1 = A.s1;
        g.lda = A.ld;
        g.B = Bv.p;
        g.sB0 = Bv.s0;
        g.sB1 = Bv.s1;
        g.ldb = Bv.ld;
        g.modB = Bv.mod;
        g.C = out;
        g.sC0 = Cv.s0;
        g.sC1 = Cv.s1;
        g.ldc = Cv.ld;
        g.Cin = cin;
        g.beta = cin ? 1.f : 0.f;
        g.M = M;
        g.N = Nn;
        g.Kd = Kd;
        g.n_outer = BH;
        g.n_inner = (int)(per_seg ? b.n_sg : b.n_st);
        g.ntok = N;
        g.tok_step = per_seg ? kBwdSeg : C;
        g.tok_flags = tokf;
        g.tril = tril;
        g.split = f32 ? 0 : 1;   // bf16 storage: split-bf16 products on the bf16 matrix cores
        bool ok = true;
        const gma_status_t ls = timed_launch(K_BWD_GEMM, s, [&] { ok = launch_bwd_gemm(g, ta, tb, out_bf16, s); });
        if (!ok) return fail(GMA_ERROR_LAUNCH, "no backward product kernel for this operand combination");
        return ls;
    };
#define GMA_TRY(x)                        \
    do {                                  \
        st = (x);                         \
        if (st != GMA_SUCCESS) return st; \
    } while (0)
    constexpr int TM = 1, TN = 2, TK = 4;   // token axes of a product

    // mixture constants, responsibilities of both sides, [V | 1]
    GMA_TRY(timed_launch(K_BWD_ROWS, s, [&] { launch_bwd_prep(mu, rv, mw, H, K, d_r, s); }));
    const double* cq = reinterpret_cast<const double*>(w + b.off_cq);
    // bf16 rows: split-bf16 products on the bf16 matrix cores (the operand fragments then take the split
    // layout in the same bytes); fp32 rows: the fp32 matrix cores with fp64 partial sums
    const bool gsplit = bwd_gamma_split_supported(K, d_r, f32) && !misaligned(qx, 16) && !misaligned(kx, 16);
    GMA_TRY(timed_launch(K_BWD_ROWS, s, [&] {
        launch_bwd_frag(mu, rv, pr, F(b.off_bf), reinterpret_cast<double*>(w + b.off_cq), H, K, d_r, gsplit, s);
    }));
    for (int side = 0; side < 2; ++side) {
        const void* x = side ? kx : qx;
        float* gam = side ? gk : gq;
        GMA_TRY(timed_launch(K_BWD_GAMMA, s, [&] {
            if (gsplit) launch_bwd_gamma_split(x, F(b.off_bf), cq, gam, BH, N, H, K, d_r, s);
            else launch_bwd_gamma_mfma(x, f32, F(b.off_bf), cq, gam, BH, N, H, K, d_r, s);
        }));
    }
    // operands generated inside the products (views in rows): [V | 1] from V, [g | h] from dO and the row
    // pair rs = (1 / den, h), [x | x^2 | 1] from the routing input
    const View rows_tok{nullptr, N, C, 1, 0}, rows_seg{nullptr, N, kBwdSeg, 1, 0};
    const View vv = rows_tok, ghv = rows_tok;
    const BwdGen gen_v{v, nullptr, GEN_VAUG, f32 ? 1 : 0, d_v};
    const BwdGen gen_gh{dout, rs, GEN_GH, f32 ? 1 : 0, d_v};
    // Per side, the posterior gradient, the routing-input gradient and the parameter partials in one fused
    // kernel where there is one for the shape.  The partials buffer holds n_sg segments of kBwdSeg tokens
    // per side: the fused segments are no shorter, so their count fits.
    const int fseg = bwd_fused_rows_seg(BH, N, K, d_r, kBwdSeg);
    const int64_t fn = (N + fseg - 1) / fseg;
    const bool fused = bwd_fused_rows_supported(K, d_r, f32) && !misaligned(qx, 16) && !misaligned(kx, 16) &&
                       !misaligned(dqx, 16) && !misaligned(dkx, 16) && (N + 64) * K * 4 < (int64_t(1) << 31) &&
                       N * d_r * 2 < (int64_t(1) << 31) && fn <= b.n_sg;
    // Causal bf16 at K = d_v = 128: fused chunk kernels for the state terms, the query side (read phase,
    // chunk terms of the suffix sums, dGamma_Q) and the key side (dGamma_K, dV).  With the fused row kernel
    // after them they write dl in place of dGamma.
    const bool qfused = b.fq;
    const bool emit_dl = qfused && fused;
    // Bidirectional bf16 at K <= 64, d_v <= 128: fused kernels for the state, the query side (num, den, g,
    // h, dGamma_Q and the segment sums of Gamma_Q^T [g | h]) and the key side (dGamma_K, dV), over the
    // state segments of C tokens
    const bool bq = !causal && bwd_bidir_small_supported(K, d_v, f32) && dva == d_v + 4 && !misaligned(v, 8) &&
                    !misaligned(dout, 8) && !misaligned(dv, 8) && (N + 64) * K * 4 < (int64_t(1) << 31) &&
                    (N + 64) * d_v * 2 < (int64_t(1) << 31);
    // with the fused row kernel after them they too write dl in place of dGamma
    const bool bq_dl = bq && fused;
    // the chunk kernels read and write whole 16-byte pieces of bf16 rows: rows that are not 16-byte aligned
    // go through aligned copies in the workspace
    const void* vq = v;
    const void* dq = dout;
    void* dvq = dv;
    const size_t row_bytes = (size_t)rows * d_v * 2;
    if (qfused) {
        if (misaligned(v, 16)) {
            if (hipMemcpyAsync(w + b.off_vs, v, row_bytes, hipMemcpyDeviceToDevice, s) != hipSuccess)
                return fail(GMA_ERROR_LAUNCH, "staging copy of v failed");
            vq = w + b.off_vs;
        }
        if (misaligned(dout, 16)) {
            if (hipMemcpyAsync(w + b.off_ds, dout, row_bytes, hipMemcpyDeviceToDevice, s) != hipSuccess)
                return fail(GMA_ERROR_LAUNCH, "staging copy of dout failed");
            dq = w + b.off_ds;
        }
        if (misaligned(dv, 16)) dvq = w + b.off_dvs;
    }
    // write phase: Gamma_K^T [V | 1] per entry -> the state before each chunk / the total
    // (fused: the totals of state segments of b.sper chunks, their exclusive scan, then the prefixes of
    // every chunk, from the segment's prefix on)
    float* sgs = F(b.off_sgs);
    const int64_t n_sgs = (b.n_st + b.sper - 1) / b.sper;
    if (qfused) {
        bool ok = true;
        GMA_TRY(timed_launch(K_BWD_CHUNK, s, [&] {
            ok = launch_bwd_chunk_state(gk, vq, stt, sgs, b.sper, true, BH, N, b.n_st, K, d_v, dva, s);
        }));
        if (!ok) return fail(GMA_ERROR_LAUNCH, "no chunk-state kernel for this shape");
        GMA_TRY(timed_launch(K_BWD_SCAN, s, [&] { launch_bwd_scan(sgs, BH, n_sgs, rec, 0, s); }));
        GMA_TRY(timed_launch(K_BWD_CHUNK, s, [&] {
            launch_bwd_chunk_state(gk, vq, stt, sgs, b.sper, false, BH, N, b.n_st, K, d_v, dva, s);
        }));
    } else if (bq) {
        bool ok = true;
        GMA_TRY(timed_launch(K_BWD_CHUNK, s, [&] {
            ok = launch_bwd_bidir_state(gk, v, stt, BH, N, K, d_v, dva, C, s);
        }));
        if (!ok) return fail(GMA_ERROR_LAUNCH, "no bidirectional state kernel for this shape");
        GMA_TRY(timed_launch(K_BWD_SCAN, s, [&] { launch_bwd_scan(stt, BH, b.n_st, rec, 2, s); }));
        GMA_TRY(timed_launch(K_BWD_CHUNK, s, [&] {
            ok = launch_bwd_bidir_q(gq, dout, stt, dgq, rt, BH, N, K, d_v, dva, C, b.eps, bq_dl, s);
        }));
        if (!ok) return fail(GMA_ERROR_LAUNCH, "no bidirectional query-side kernel for this shape");
        GMA_TRY(timed_launch(K_BWD_SCAN, s, [&] { launch_bwd_scan(rt, BH, b.n_st, rec, 2, s); }));
        GMA_TRY(timed_launch(K_BWD_CHUNK, s, [&] {
            ok = launch_bwd_bidir_k(gk, v, rt, dgk, dv, BH, N, K, d_v, dva, C, bq_dl, s);
        }));
        if (!ok) return fail(GMA_ERROR_LAUNCH, "no bidirectional key-side kernel for this shape");
    } else {
        GMA_TRY(gemm(tok(gk, K), true, vv, false, all_st(stt), stt, false, K, dva, C, TK, 0, nullptr, false, BwdGen{},
                     gen_v));
        GMA_TRY(timed_launch(K_BWD_SCAN, s, [&] { launch_bwd_scan(stt, BH, b.n_st, rec, causal ? 0 : 2, s); }));
    }
    if (qfused) {
        bool ok = true;
        GMA_TRY(timed_launch(K_BWD_CHUNK, s, [&] {
            ok = launch_bwd_chunk_q(gq, gk, vq, dq, stt, rs, sgs, b.sper, nullptr, nullptr, dgq, BH, N, b.n_st, K,
                                    d_v, dva, b.eps, emit_dl, s);
        }));
        if (!ok) return fail(GMA_ERROR_LAUNCH, "no fused query-side chunk kernel for this shape");
        // the suffix states: the query side has left the segment totals of Gamma_Q^T [g | h] in the segment
        // array (free again); their exclusive suffix scan, then every chunk's suffix from its segment's on
        GMA_TRY(timed_launch(K_BWD_SCAN, s, [&] { launch_bwd_scan(sgs, BH, n_sgs, rec, 1, s); }));
        GMA_TRY(timed_launch(K_BWD_CHUNK, s, [&] {
            launch_bwd_suffix_state(gq, dq, rs, rt, sgs, b.sper, BH, N, b.n_st, K, d_v, dva, s);
        }));
    }
    if (!qfused && !bq) {
        // read phase: [num | Gamma_Q . Z] = Gamma_Q state (+ tril(Gamma_Q Gamma_K^T) [V | 1]), then g, h
        GMA_TRY(gemm(tok(gq, K), false, cur_st(stt), false, tok(pp, dva), pp, false, C, dva, K, TM, 0, nullptr, false));
        if (causal) {
            GMA_TRY(gemm(tok(gq, K), false, tok(gk, K), true, sq(ac), ac, false, C, C, K, TM | TN, 1, nullptr, false));
            GMA_TRY(gemm(sq(ac), false, vv, false, tok(pp, dva), pp, false, C, dva, C, TM | TK, 0, pp, false, BwdGen{}, gen_v));
        }
        GMA_TRY(timed_launch(K_BWD_ROWS, s, [&] { launch_bwd_gh(pp, dout, f32, rs, rows, d_v, dva, b.eps, s); }));
        // Gamma_Q^T [g | h] per entry -> the sums over the later chunks / the total
        GMA_TRY(gemm(tok(gq, K), true, ghv, false, all_st(rt), rt, false, K, dva, C, TK, 0, nullptr, false, BwdGen{}, gen_gh));
        GMA_TRY(timed_launch(K_BWD_SCAN, s, [&] { launch_bwd_scan(rt, BH, b.n_st, rec, causal ? 1 : 2, s); }));
        // dGamma_Q = [g | h] state^T (+ tril([g | h] [V | 1]^T) Gamma_K)
        GMA_TRY(gemm(ghv, false, cur_st(stt), true, tok(dgq, K), dgq, false, C, K, dva, TM, 0, nullptr, false, gen_gh));
        if (causal) {
            GMA_TRY(gemm(ghv, false, vv, true, sq(mt), mt, false, C, C, dva, TM | TN, 1, nullptr, false, gen_gh, gen_v));
            GMA_TRY(gemm(sq(mt), false, tok(gk, K), false, tok(dgq, K), dgq, false, C, K, C, TM | TK, 0, dgq, false));
        }
    }
    if (qfused) {
        // the key-side counterpart: dGamma_K and dV per chunk (ac and mt recomputed)
        bool ok = true;
        GMA_TRY(timed_launch(K_BWD_CHUNK, s, [&] {
            ok = launch_bwd_chunk_k(gq, gk, vq, dq, rs, rt, dgk, dvq, BH, N, b.n_st, K, d_v, dva, emit_dl, s);
        }));
        if (!ok) return fail(GMA_ERROR_LAUNCH, "no fused key-side chunk kernel for this shape");
        if (dvq != dv && hipMemcpyAsync(dv, dvq, row_bytes, hipMemcpyDeviceToDevice, s) != hipSuccess)
            return fail(GMA_ERROR_LAUNCH, "copy of the staged dv failed");
    } else if (!bq) {
        // dGamma_K = [V | 1] R^T (+ the same intra-chunk block transposed, times Gamma_Q)
        GMA_TRY(gemm(vv, false, cur_st(rt), true, tok(dgk, K), dgk, false, C, K, dva, TM, 0, nullptr, false, gen_v));
        if (causal)
            GMA_TRY(gemm(sq(mt), true, tok(gq, K), false, tok(dgk, K), dgk, false, C, K, C, TM | TK, 0, dgk, false));
        // dV = Gamma_K R (+ tril(Gamma_Q Gamma_K^T)^T g), in the storage dtype
        if (causal)
            GMA_TRY(gemm(sq(ac), true, ghv, false, tok(dvt, d_v), dvt, false, C, d_v, C, TM | TK, 0, nullptr, false,
                         BwdGen{}, gen_gh));
        GMA_TRY(gemm(tok(gk, K), false, cur_st(rt), false, tok(nullptr, d_v), dv, !f32, C, d_v, K, TM, 0,
                     causal ? dvt : nullptr, false));
    }
    // posterior gradients, then per side the routing-input gradient and the parameter partials: one
    // fused kernel per side where there is one for the shape (dl then stays on chip)
    if (fused) {
        for (int side = 0; side < 2; ++side) {
            bool ok = true;
            GMA_TRY(timed_launch(K_BWD_FUSED, s, [&] {
                ok = launch_bwd_fused_rows(side ? gk : gq, side ? dgk : dgq, side ? kx : qx, mw, side ? dkx : dqx,
                                           gp + (size_t)side * BH * fn * K * dxa, BH, N, H, K, d_r, dxa, fseg,
                                           emit_dl || bq_dl, s);
            }));
            if (!ok) return fail(GMA_ERROR_LAUNCH, "no fused backward row kernel for this shape");
        }
        return timed_launch(K_BWD_PARAM, s, [&] {
            launch_bwd_param(gp, gs, mu, rv, pr, dmu, drv, dpr, b.B, H, K, d_r, dxa, fn, s);
        });
    }
    GMA_TRY(timed_launch(K_BWD_ROWS, s, [&] { launch_bwd_dl(gq, dgq, rows, K, s); }));
    GMA_TRY(timed_launch(K_BWD_ROWS, s, [&] { launch_bwd_dl(gk, dgk, rows, K, s); }));
    for (int side = 0; side < 2; ++side) {
        const void* x = side ? kx : qx;
        const float* dl = side ? dgk : dgq;
        void* dx = side ? dkx : dqx;
        const View mwv{mw, (int64_t)K * 2 * d_r, 0, 2 * d_r, H};
        // dx = dl . mu / s - x (dl . 1 / s), formed in the product's epilogue from the interleaved columns
        GMA_TRY(gemm(seg(dl, K), false, mwv, false, View{nullptr, N * d_r, (int64_t)kBwdSeg * d_r, d_r, 0}, dx, !f32,
                     kBwdSeg, 2 * d_r, K, TM, 0, nullptr, true, BwdGen{}, BwdGen{}, x));
        float* gps = gp + (size_t)side * BH * b.n_sg * K * dxa;
        const View gpv{gps, b.n_sg * K * dxa, (int64_t)K * dxa, dxa, 0};
        // dl^T [x | x^2 | 1] per segment, the augmented rows generated from x inside the product
        GMA_TRY(gemm(seg(dl, K), true, rows_seg, false, gpv, gps, false, K, dxa, kBwdSeg, TK, 0, nullptr, true,
                     BwdGen{}, BwdGen{x, nullptr, GEN_XAUG, f32 ? 1 : 0, d_r}));
    }
#undef GMA_TRY
    return timed_launch(K_BWD_PARAM, s, [&] {
        launch_bwd_param(gp, gs, mu, rv, pr, dmu, drv, dpr, b.B, H, K, d_r, dxa, b.n_sg, s);
    });
}

// Prepared decode mixture: 1 / sigma^2 [H, K, d_r] fp32, then c [H, K] fp64 at a 256-byte boundary.
struct DecodePrepLayout {
    size_t off_c, total;
};
DecodePrepLayout decode_prep_layout(const gma_problem_t* p) {
    DecodePrepLayout l;
    l.off_c = align_up((size_t)p->heads * p->n_comp * p->d_route * sizeof(float), 256);
    l.total = align_up(l.off_c + (size_t)p->heads * p->n_comp * sizeof(double), 256);
    return l;
}

// Shared by the decode entry points: validation (host only, before any HIP call) and the launch.
// With `prepared` the mixture is mu plus the gma_decode_prepare output; raw_var and prior_logits
// are then unused (NULL).
gma_status_t decode(const gma_problem_t* p, const void* qx, const void* kx, const void* v, const float* mu,
                    const float* raw_var, const float* prior_logits, const void* prepared, size_t prepared_bytes,
                    const float* state_in, float* state_out, void* o, void* stream) {
    g_last_error.clear();
    if (!p) return fail(GMA_ERROR_INVALID_VALUE, "problem is NULL");
    if (p->batch < 1 || p->heads < 1) return fail(GMA_ERROR_INVALID_VALUE, "batch and heads must be >= 1");
    if (p->seq_len != 1)
        return fail(GMA_ERROR_INVALID_VALUE, "a decode step takes one token per (batch, head): seq_len must be 1");
    if (p->d_route < 1 || p->n_comp < 1 || p->d_value < 1)
        return fail(GMA_ERROR_INVALID_VALUE, "d_route, n_comp and d_value must be >= 1");
    if (p->d_route > 256 || p->n_comp > 256 || p->d_value > 256)
        return fail(GMA_ERROR_NOT_SUPPORTED, "d_route, n_comp and d_value must be <= 256");
    if (p->dtype != GMA_DTYPE_F32 && p->dtype != GMA_DTYPE_BF16)
        return fail(GMA_ERROR_INVALID_VALUE, "dtype must be GMA_DTYPE_F32 or GMA_DTYPE_BF16 (got %d)", p->dtype);
    if (!std::isfinite(p->eps) || p->eps < 0.f) return fail(GMA_ERROR_INVALID_VALUE, "eps must be finite and >= 0");
    if (p->batch > (int64_t(1) << 40) / p->heads || p->batch * p->heads > INT32_MAX / 2)
        return fail(GMA_ERROR_NOT_SUPPORTED, "batch * heads too large");
    const void* ptrs[] = {qx, kx, v, mu, prepared ? prepared : (const void*)raw_var,
                          prepared ? prepared : (const void*)prior_logits, o};
    for (int i = 0; i < 7; ++i)
        if (!ptrs[i]) return fail(GMA_ERROR_INVALID_VALUE, "pointer argument %d is NULL", i);
    const bool f32 = p->dtype == GMA_DTYPE_F32;
    const size_t es = f32 ? 4 : 2;
    for (const void* ptr : {qx, kx, v, (const void*)o})
        if (misaligned(ptr, es)) return fail(GMA_ERROR_INVALID_VALUE, "tensor pointers must be %zu-byte aligned", es);
    for (const void* ptr : {(const void*)mu, (const void*)raw_var, (const void*)prior_logits, (const void*)state_in,
                            (const void*)state_out})
        if (misaligned(ptr, 4)) return fail(GMA_ERROR_INVALID_VALUE, "parameter and state pointers must be 4-byte aligned");
    const DecodePrepLayout lay = decode_prep_layout(p);
    if (prepared) {
        if (misaligned(prepared, 256)) return fail(GMA_ERROR_INVALID_VALUE, "prepared must be 256-byte aligned");
        if (prepared_bytes < lay.total)
            return fail(GMA_ERROR_WORKSPACE_TOO_SMALL, "prepared holds %zu bytes, %zu needed", prepared_bytes, lay.total);
    }
    const int64_t BH = p->batch * p->heads;
    const size_t nx = (size_t)BH * p->d_route * es, nv = (size_t)BH * p->d_value * es;
    const size_t ns = (size_t)BH * p->n_comp * (p->d_value + 1) * sizeof(float);
    if (overlaps(o, nv, qx, nx) || overlaps(o, nv, kx, nx) || overlaps(o, nv, v, nv))
        return fail(GMA_ERROR_INVALID_VALUE, "o must not overlap qx, kx or v");
    for (const void* sp : {(const void*)state_in, (const void*)state_out})
        if (sp && (overlaps(sp, ns, qx, nx) || overlaps(sp, ns, kx, nx) || overlaps(sp, ns, v, nv) ||
                   overlaps(sp, ns, o, nv) || (prepared && overlaps(sp, ns, prepared, lay.total))))
            return fail(GMA_ERROR_INVALID_VALUE, "states must not overlap qx, kx, v, o or prepared");
    if (prepared && overlaps(o, nv, prepared, lay.total))
        return fail(GMA_ERROR_INVALID_VALUE, "o must not overlap prepared");
    if (state_in && state_out && state_in != state_out && overlaps(state_in, ns, state_out, ns))
        return fail(GMA_ERROR_INVALID_VALUE, "state_in and state_out must be the same buffer or disjoint");
    DecodeArgs a;
    std::memset(&a, 0, sizeof(a));
    a.qx = qx;
    a.kx = kx;
    a.v = v;
    a.o = o;
    a.mu = mu;
    a.raw_var = prepared ? nullptr : raw_var;
    a.prior = prepared ? nullptr : prior_logits;
    a.state_in = state_in;
    a.state_out = state_out;
    a.H = (int)p->heads;
    a.K = p->n_comp;
    a.d_r = p->d_route;
    a.d_v = p->d_value;
    a.eps = p->eps;
    if (prepared) {
        a.inv_var = reinterpret_cast<const float*>(prepared);
        a.cconst = reinterpret_cast<const double*>(reinterpret_cast<const char*>(prepared) + lay.off_c);
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    return timed_launch(K_DECODE, s, [&] { launch_decode(a, BH, f32, s); });
}

}  // namespace
}  // namespace gma

// Workspace of gma_forward_causal_noalloc: a fixed device array, so that the call allocates nothing.
// In host code `scratch` names a host-side stand-in, not device memory: its device address is taken
// once per device with hipGetSymbolAddress (that device current) and only that address is used.
static __device__ __align__(256) char scratch[GMA_NOALLOC_SCRATCH_BYTES];

namespace gma {
namespace {

std::mutex g_scratch_mu;
constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up on the first call per device.
gma_status_t scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(GMA_ERROR_LAUNCH, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(GMA_ERROR_NOT_SUPPORTED, "device %d out of range", dev);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(GMA_ERROR_LAUNCH, "hipGetSymbolAddress of the scratch array failed on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return GMA_SUCCESS;
}

// gma_forward_causal with the device's scratch array as its workspace: the workspace the causal pass
// needs when the Gamma_K tiles are not stored (the larger of the two stagings, since pointer alignment
// decides which runs) must fit the array; the pass stores the tiles only where they fit as well.
gma_status_t forward_causal_noalloc(const gma_problem_t* p, const void* qx, const void* kx, const void* v,
                                    const float* mu, const float* rv, const float* pr, void* o, void* stream) {
    g_last_error.clear();
    Plan pl, pt;
    gma_status_t st = make_plan(p, GMA_OP_FORWARD_CAUSAL, &pl);
    if (st != GMA_SUCCESS) return st;
    for (const void* ptr : {qx, kx, v, (const void*)mu, (const void*)rv, (const void*)pr, (const void*)o})
        if (!ptr) return fail(GMA_ERROR_INVALID_VALUE, "pointer arguments must not be NULL");
    size_t need = pl.total;
    if (!pl.generic && pl.cls->tok_out_causal && make_plan(p, GMA_OP_FORWARD_CAUSAL, &pt, true, false) == GMA_SUCCESS)
        need = std::max(need, pt.total);
    if (need > (size_t)GMA_NOALLOC_SCRATCH_BYTES)
        return fail(GMA_ERROR_WORKSPACE_TOO_SMALL,
                    "the problem needs %zu bytes of workspace; the no-allocation entry point has %zu", need,
                    (size_t)GMA_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    st = scratch_address(&ws);
    if (st != GMA_SUCCESS) return st;
    return forward(p, GMA_OP_FORWARD_CAUSAL, qx, kx, v, mu, rv, pr, nullptr, nullptr, o, ws,
                   (size_t)GMA_NOALLOC_SCRATCH_BYTES, stream);
}

}  // namespace
}  // namespace gma

using namespace gma;

extern "C" {

size_t gma_workspace_size(const gma_problem_t* problem, int op) {
    const size_t total = advertised_workspace(problem, op);
    g_last_error.clear();
    return total;
}

gma_status_t gma_responsibilities(const gma_problem_t* p, const void* x, const float* mu, const float* raw_var,
                                  const float* prior_logits, float* gamma, void* ws, size_t ws_bytes, void* stream) {
    g_last_error.clear();
    Plan pl;
    gma_status_t st = make_plan(p, GMA_OP_RESPONSIBILITIES, &pl);
    if (st != GMA_SUCCESS) return st;
    const void* ptrs[] = {x, mu, raw_var, prior_logits, gamma};
    st = check_common(p, ptrs, 5, ws, ws_bytes, pl);
    if (st != GMA_SUCCESS) return st;
    const size_t es = pl.f32 ? 4 : 2;
    if (misaligned(x, es) || misaligned(gamma, 4) || misaligned(mu, 4) || misaligned(raw_var, 4) ||
        misaligned(prior_logits, 4))
        return fail(GMA_ERROR_INVALID_VALUE, "misaligned pointer");
    const size_t nx = (size_t)(pl.B * pl.H * pl.N) * pl.d_r * es;
    const size_t ng = (size_t)(pl.B * pl.H * pl.N) * pl.K * 4;
    if (overlaps(gamma, ng, x, nx)) return fail(GMA_ERROR_INVALID_VALUE, "gamma must not overlap x");
    if (ws && (overlaps(ws, pl.total, x, nx) || overlaps(ws, pl.total, gamma, ng)))
        return fail(GMA_ERROR_INVALID_VALUE, "workspace must not overlap the tensors");
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char* w = reinterpret_cast<char*>(ws);
    if (pl.generic) return generic_gamma(pl, x, mu, raw_var, prior_logits, gamma, pl.N, w, s, true);
    st = launch_prep(pl, mu, raw_var, prior_logits, w, s);
    if (st != GMA_SUCCESS) return st;
    MainArgs a = base_args(pl, w);
    a.qx = x;
    a.gamma = gamma;
    a.vec_x = vec_ok(x, pl.d_r, pl.f32);
    const bool dma = !pl.f32 && pl.cls->dma_resp && pl.d_r % 8 == 0 && !misaligned(x, 16) &&
                     (pl.N + pl.cls->c) * pl.d_r * 2 < (int64_t(1) << 31);
    const main_launch_t f_resp = dma ? pl.cls->dma_resp : pl.cls->resp;
    const int grid = (int)(pl.B * pl.H * pl.P);
    if (pl.resp_tok && !misaligned(x, 16)) {
        const bool vecg = pl.K % 4 == 0 && !misaligned(gamma, 16);
        bool ok = false;
        st = timed_launch(K_RESP, s, [&] { ok = launch_resp_tok(a, pl.cls->kc, pl.cls->drc, pl.resp_rows, vecg, grid, s); });
        if (st == GMA_SUCCESS && !ok) return fail(GMA_ERROR_NOT_SUPPORTED, "no token-split responsibilities kernel");
    } else {
        st = timed_launch(K_RESP, s, [&] { f_resp(a, grid, s); });
    }
    if (st != GMA_SUCCESS || !pl.flags) return st;
    FixArgs f = fix_args(pl, w);
    f.qx = x;
    f.gamma = gamma;
    f.mu = mu;
    f.raw_var = raw_var;
    f.prior = prior_logits;
    return launch_fixup(pl, f, false, false, s);
}

gma_status_t gma_responsibility_stats(const gma_problem_t* p, const void* x, const float* mu, const float* raw_var,
                                      const float* prior_logits, float* usage, uint32_t* hard_counts,
                                      float* usage_entropy, void* ws, size_t ws_bytes, void* stream) {
    g_last_error.clear();
    Plan pl;
    gma_status_t st = make_plan(p, GMA_OP_RESPONSIBILITY_STATS, &pl);
    if (st != GMA_SUCCESS) return st;
    const void* ptrs[] = {x, mu, raw_var, prior_logits, usage, hard_counts, usage_entropy};
    st = check_common(p, ptrs, 7, ws, ws_bytes, pl);
    if (st != GMA_SUCCESS) return st;
    const size_t es = pl.f32 ? 4 : 2;
    if (misaligned(x, es) || misaligned(mu, 4) || misaligned(raw_var, 4) || misaligned(prior_logits, 4) ||
        misaligned(usage, 4) || misaligned(hard_counts, 4) || misaligned(usage_entropy, 4))
        return fail(GMA_ERROR_INVALID_VALUE, "misaligned pointer");
    const int64_t BH = pl.B * pl.H;
    const size_t nx = (size_t)(BH * pl.N) * pl.d_r * es, nk = (size_t)BH * pl.K * 4, nb = (size_t)BH * 4;
    const void* outs[] = {usage, hard_counts, usage_entropy};
    const size_t osz[] = {nk, nk, nb};
    for (int i = 0; i < 3; ++i) {
        if (overlaps(outs[i], osz[i], x, nx) || (ws && overlaps(outs[i], osz[i], ws, pl.total)))
            return fail(GMA_ERROR_INVALID_VALUE, "outputs must not overlap x or the workspace");
        for (int j = 0; j < i; ++j)
            if (overlaps(outs[i], osz[i], outs[j], osz[j])) return fail(GMA_ERROR_INVALID_VALUE, "outputs must not overlap");
    }
    if (ws && overlaps(ws, pl.total, x, nx)) return fail(GMA_ERROR_INVALID_VALUE, "workspace must not overlap x");
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char* w = reinterpret_cast<char*>(ws);
    float* pu = reinterpret_cast<float*>(w + pl.off_part);
    uint32_t* pc = reinterpret_cast<uint32_t*>(pu + (size_t)BH * pl.stat_segs * pl.K);
    const int S = pl.stat_segs;
    if (pl.generic) {
        // generic path: Gamma of every row into the workspace, then the per-segment reductions
        float* gam = reinterpret_cast<float*>(w + pl.off_gamma);
        st = generic_gamma(pl, x, mu, raw_var, prior_logits, gam, pl.N, w, s, true);
        if (st != GMA_SUCCESS) return st;
        const int64_t rps = (pl.N + S - 1) / S;
        st = timed_launch(K_STATS, s, [&] {
            hipLaunchKernelGGL(stats_partial_kernel, dim3((unsigned)S, (unsigned)BH), dim3(256), 0, s,
                               (const float*)gam, pu, pc, pl.N, pl.K, S, rps);
        });
        if (st != GMA_SUCCESS) return st;
    } else {
        // the responsibilities kernel forms the per-segment usage and counts itself (Gamma is not stored)
        st = launch_prep(pl, mu, raw_var, prior_logits, w, s);
        if (st != GMA_SUCCESS) return st;
        MainArgs a = base_args(pl, w);
        a.qx = x;
        a.stat_usage = pu;
        a.stat_count = pc;
        a.vec_x = vec_ok(x, pl.d_r, pl.f32);
        const bool dma = !pl.f32 && pl.cls->dma_resp && pl.d_r % 8 == 0 && !misaligned(x, 16) &&
                         (pl.N + pl.cls->c) * pl.d_r * 2 < (int64_t(1) << 31);
        const main_launch_t f_resp = dma ? pl.cls->dma_resp : pl.cls->resp;
        if (pl.resp_tok && !misaligned(x, 16)) {
            bool ok = false;
            st = timed_launch(K_STATS, s, [&] {
                ok = launch_resp_tok(a, pl.cls->kc, pl.cls->drc, pl.resp_rows, false, (int)(BH * pl.P), s);
            });
            if (st == GMA_SUCCESS && !ok) return fail(GMA_ERROR_NOT_SUPPORTED, "no token-split responsibilities kernel");
        } else {
            st = timed_launch(K_STATS, s, [&] { f_resp(a, (int)(BH * pl.P), s); });
        }
        if (st != GMA_SUCCESS) return st;
        if (pl.flags) {
            FixArgs f = fix_args(pl, w);
            f.qx = x;
            f.mu = mu;
            f.raw_var = raw_var;
            f.prior = prior_logits;
            f.stat_usage = pu;
            f.stat_count = pc;
            f.stat_segs = S;
            st = launch_fixup(pl, f, false, false, s);
            if (st != GMA_SUCCESS) return st;
        }
    }
    return timed_launch(K_STATS, s, [&] {
        hipLaunchKernelGGL(stats_final_kernel, dim3((unsigned)BH), dim3(256), 0, s, (const float*)pu,
                           (const uint32_t*)pc, usage, hard_counts, usage_entropy, pl.N, pl.K, S);
    });
}

gma_status_t gma_forward_bidir(const gma_problem_t* p, const void* qx, const void* kx, const void* v, const float* mu,
                               const float* raw_var, const float* prior_logits, void* o, void* ws, size_t ws_bytes,
                               void* stream) {
    return forward(p, GMA_OP_FORWARD_BIDIR, qx, kx, v, mu, raw_var, prior_logits, nullptr, nullptr, o, ws, ws_bytes,
                   stream);
}

gma_status_t gma_forward_causal(const gma_problem_t* p, const void* qx, const void* kx, const void* v, const float* mu,
                                const float* raw_var, const float* prior_logits, void* o, void* ws, size_t ws_bytes,
                                void* stream) {
    return forward(p, GMA_OP_FORWARD_CAUSAL, qx, kx, v, mu, raw_var, prior_logits, nullptr, nullptr, o, ws, ws_bytes,
                   stream);
}

gma_status_t gma_forward_causal_noalloc(const gma_problem_t* p, const void* qx, const void* kx, const void* v,
                                        const float* mu, const float* raw_var, const float* prior_logits, void* o,
                                        void* stream) {
    return forward_causal_noalloc(p, qx, kx, v, mu, raw_var, prior_logits, o, stream);
}

gma_status_t gma_forward_bidir_kv(const gma_problem_t* p, int64_t seq_len_kv, const void* qx, const void* kx,
                                  const void* v, const float* mu, const float* raw_var, const float* prior_logits,
                                  void* o, void* ws, size_t ws_bytes, void* stream) {
    return forward_bidir_kv(p, seq_len_kv, qx, kx, v, mu, raw_var, prior_logits, o, ws, ws_bytes, stream);
}

gma_status_t gma_decode_step(const gma_problem_t* p, const void* qx, const void* kx, const void* v, const float* mu,
                             const float* raw_var, const float* prior_logits, const float* state_in, float* state_out,
                             void* o, void* stream) {
    return decode(p, qx, kx, v, mu, raw_var, prior_logits, nullptr, 0, state_in, state_out, o, stream);
}

size_t gma_decode_params_size(const gma_problem_t* p) {
    if (!p || p->heads < 1 || p->n_comp < 1 || p->d_route < 1 || p->n_comp > 256 || p->d_route > 256) return 0;
    return decode_prep_layout(p).total;
}

gma_status_t gma_decode_prepare(const gma_problem_t* p, const float* raw_var, const float* prior_logits,
                                void* prepared, size_t prepared_bytes, void* stream) {
    g_last_error.clear();
    if (!p) return fail(GMA_ERROR_INVALID_VALUE, "problem is NULL");
    if (p->heads < 1 || p->n_comp < 1 || p->d_route < 1)
        return fail(GMA_ERROR_INVALID_VALUE, "heads, n_comp and d_route must be >= 1");
    if (p->n_comp > 256 || p->d_route > 256) return fail(GMA_ERROR_NOT_SUPPORTED, "n_comp and d_route must be <= 256");
    if (p->heads > INT32_MAX / 2) return fail(GMA_ERROR_NOT_SUPPORTED, "heads too large");
    if (!raw_var || !prior_logits || !prepared)
        return fail(GMA_ERROR_INVALID_VALUE, "raw_var, prior_logits and prepared must not be NULL");
    for (const void* ptr : {(const void*)raw_var, (const void*)prior_logits})
        if (misaligned(ptr, 4)) return fail(GMA_ERROR_INVALID_VALUE, "parameter pointers must be 4-byte aligned");
    if (misaligned(prepared, 256)) return fail(GMA_ERROR_INVALID_VALUE, "prepared must be 256-byte aligned");
    const DecodePrepLayout lay = decode_prep_layout(p);
    if (prepared_bytes < lay.total)
        return fail(GMA_ERROR_WORKSPACE_TOO_SMALL, "prepared holds %zu bytes, %zu needed", prepared_bytes, lay.total);
    const size_t np = (size_t)p->heads * p->n_comp * p->d_route * sizeof(float);
    if (overlaps(prepared, lay.total, raw_var, np))
        return fail(GMA_ERROR_INVALID_VALUE, "prepared must not overlap the parameters");
    if (overlaps(prepared, lay.total, prior_logits, (size_t)p->heads * p->n_comp * sizeof(float)))
        return fail(GMA_ERROR_INVALID_VALUE, "prepared must not overlap the parameters");
    DecodePrepArgs a;
    a.raw_var = raw_var;
    a.prior = prior_logits;
    a.inv_var = reinterpret_cast<float*>(prepared);
    a.cconst = reinterpret_cast<double*>(reinterpret_cast<char*>(prepared) + lay.off_c);
    a.K = p->n_comp;
    a.d_r = p->d_route;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    return timed_launch(K_DECODE_PREP, s, [&] { launch_decode_prepare(a, (int)p->heads, s); });
}

gma_status_t gma_decode_step_prepared(const gma_problem_t* p, const void* qx, const void* kx, const void* v,
                                      const float* mu, const void* prepared, size_t prepared_bytes,
                                      const float* state_in, float* state_out, void* o, void* stream) {
    return decode(p, qx, kx, v, mu, nullptr, nullptr, prepared, prepared_bytes, state_in, state_out, o, stream);
}

gma_status_t gma_forward_causal_state(const gma_problem_t* p, const void* qx, const void* kx, const void* v,
                                      const float* mu, const float* raw_var, const float* prior_logits,
                                      const float* state_in, float* state_out, void* o, void* ws, size_t ws_bytes,
                                      void* stream) {
    return forward(p, GMA_OP_FORWARD_CAUSAL_STATE, qx, kx, v, mu, raw_var, prior_logits, state_in, state_out, o, ws,
                   ws_bytes, stream);
}

gma_status_t gma_backward_bidir(const gma_problem_t* p, const void* qx, const void* kx, const void* v, const float* mu,
                                const float* raw_var, const float* prior_logits, const void* dout, void* dqx, void* dkx,
                                void* dv, float* dmu, float* draw_var, float* dprior_logits, void* ws, size_t ws_bytes,
                                void* stream) {
    return backward(p, false, qx, kx, v, mu, raw_var, prior_logits, dout, dqx, dkx, dv, dmu, draw_var, dprior_logits,
                    ws, ws_bytes, stream);
}

gma_status_t gma_backward_causal(const gma_problem_t* p, const void* qx, const void* kx, const void* v, const float* mu,
                                 const float* raw_var, const float* prior_logits, const void* dout, void* dqx,
                                 void* dkx, void* dv, float* dmu, float* draw_var, float* dprior_logits, void* ws,
                                 size_t ws_bytes, void* stream) {
    return backward(p, true, qx, kx, v, mu, raw_var, prior_logits, dout, dqx, dkx, dv, dmu, draw_var, dprior_logits,
                    ws, ws_bytes, stream);
}

const char* gma_status_string(gma_status_t s) {
    switch (s) {
        case GMA_SUCCESS: return "success";
        case GMA_ERROR_INVALID_VALUE: return "invalid value";
        case GMA_ERROR_NOT_SUPPORTED: return "not supported";
        case GMA_ERROR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case GMA_ERROR_LAUNCH: return "kernel launch failed";
    }
    return "unknown status";
}

const char* gma_last_error(void) { return g_last_error.c_str(); }

gma_status_t gma_timing_enable(int enabled) {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    g_timing.enabled = enabled != 0;
    return GMA_SUCCESS;
}

gma_status_t gma_timing_read(int kernel_id, double* total_ms, int64_t* launches) {
    if (kernel_id < 0 || kernel_id >= K_COUNT || !total_ms || !launches)
        return fail(GMA_ERROR_INVALID_VALUE, "bad timing query");
    std::vector<std::pair<hipEvent_t, hipEvent_t>> rec;
    {
        std::lock_guard<std::mutex> lk(g_timing.mu);
        rec.swap(g_timing.recorded[kernel_id]);
    }
    double sum = 0.0;
    gma_status_t st = GMA_SUCCESS;
    for (auto& pr : rec) {
        float ms = 0.f;
        if (hipEventSynchronize(pr.second) != hipSuccess || hipEventElapsedTime(&ms, pr.first, pr.second) != hipSuccess)
            st = fail(GMA_ERROR_LAUNCH, "event query failed");
        sum += ms;
    }
    {
        std::lock_guard<std::mutex> lk(g_timing.mu);
        for (auto& pr : rec) {
            g_timing.pool.push_back(pr.first);
            g_timing.pool.push_back(pr.second);
        }
    }
    *total_ms = sum;
    *launches = (int64_t)rec.size();
    return st;
}

int gma_kernel_count(void) { return K_COUNT; }

const char* gma_kernel_name(int kernel_id) {
    return (kernel_id >= 0 && kernel_id < K_COUNT) ? kKernelNames[kernel_id] : "";
}

}  // extern "C"
