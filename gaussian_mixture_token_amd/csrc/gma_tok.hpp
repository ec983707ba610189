// Token-split kernels of the bf16 forward path (LDS-DMA staging, one workgroup of four
// wavefronts, chunks of 64 tokens).
//
// Method: page "Attention par Mélange Gaussien (GMA)", section "Méthodologie", sub-section
// "Mécanisme Central", items 1-3 (responsibilities of a diagonal GMM, write Vt = Gamma_K^T V and
// Z = Gamma_K^T 1, read O = Gamma_Q Vt / (Gamma_Q Z + eps), causal variant by prefix sums).
//
// Work split.  Wave w owns tokens 16w .. 16w+15 of every chunk for everything that is per token:
// the logits of all K components (one MFMA GEMM [a | b] . [x^2 ; x]; the [a | b] operand
// fragments of every component stay in AGPRs for the whole kernel), the softmax over K (inside
// the wave: no exchange) and the output rows.  The state [Vt | Z] is split by components (pairs
// of 16-row tiles) and, where there are fewer pairs than waves, by d_v tiles; each wave keeps its
// share in fp32 registers and publishes it once per chunk to LDS as bf16 operand fragments.
//
// Causal chunk c:
//   B0   barrier: the previous chunk's LDS reads are done.  Start the DMA of chunk c+1 (own X
//        rows, a quarter of V).
//   P1   publish the state before chunk c (bf16 state^T fragments, Z fragments); logits and
//        softmax of own tokens for K and Q.  Gamma_K (normalised) goes to LDS as bf16 rows;
//        Gamma_Q stays in registers as operand fragments, unnormalised: the row scale cancels
//        between numerator and denominator except in eps, which gets eps * rowsum.
//   B1   barrier: Gamma_K rows, V of the chunk and the published state are visible.
//   P2   own query rows: O^T = state^T Gamma_Q^T (inter-chunk) + V^T tril(Gamma_Q Gamma_K^T)^T
//        (intra-chunk), denominators Gamma_Q . Z + rowsum(tril) + eps * rowsum(Gamma_Q); state
//        update of the owned share from Gamma_K^T [V | 1].
// The denominator Gamma_Q . Z uses Z split into two bf16 halves (hi + lo, about 16 significant
// bits) and a row of ones in one extra MFMA tile, so it sees exactly the bf16 Gamma_Q the
// numerator sees.
#pragma once
#include <type_traits>

#include "gma_kernels.hpp"

namespace gma {

template <int KC, int VC, int DRC, int MODE, int WPE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE)))
tok_kernel(const MainArgs a) {
    constexpr int W = 4;
    constexpr int C = 16 * W;
    constexpr int NCT = KC / 16;   // component tiles
    constexpr int NKQ = KC / 32;   // component fragment steps (pairs of tiles)
    constexpr int NVT = VC / 16;   // d_v tiles
    constexpr int NKS2 = DRC / 32; // fragment steps over d_r (x^2 part; the x part follows)
    constexpr int NSEG = DRC / 64; // 128-byte segments per staged X row
    constexpr bool GSTORE = MODE == MODE_AGG_G;         // aggregate pass storing the Gamma_K tiles
    constexpr bool GLOAD = MODE == MODE_OUT_CAUSAL_G;   // causal output pass reading them
    constexpr bool AGG = (MODE == MODE_AGG) || GSTORE;
    constexpr bool CAUSAL = (MODE == MODE_OUT_CAUSAL) || GLOAD;
    constexpr bool NEED_Q = (MODE == MODE_OUT_BIDIR) || CAUSAL;
    constexpr bool NEED_K = AGG || (MODE == MODE_OUT_CAUSAL);   // K_X staged, Gamma_K computed
    constexpr bool NEED_V = AGG || CAUSAL;
    constexpr bool OUT = NEED_Q;
    // The aggregate passes (a plain sum over the segment's chunks) walk their chunks last to first,
    // so that the chunks they touch last are the ones the causal output pass reads first.
    constexpr bool REV = AGG;
    static_assert(MODE != MODE_RESP, "responsibilities use main_kernel");
    static_assert(DRC >= 64 && DRC % 64 == 0 && NSEG <= 2, "X rows are staged in one or two 128-byte segments");
    static_assert(KC % 32 == 0 && VC % 16 == 0, "tile shapes");
    // state ownership: wave w owns component pairs kq0 .. kq0+KQW-1 and d_v tiles vt0 .. vt0+VTW-1
    constexpr int KQW = (NKQ >= W) ? NKQ / W : 1;
    constexpr int WPK = (NKQ >= W) ? 1 : W / NKQ;   // waves sharing one component pair
    constexpr int VTW = NVT / WPK;
    static_assert((NKQ >= W) ? (NKQ % W == 0) : (W % NKQ == 0), "component pairs must split across waves");
    static_assert(NVT % WPK == 0 && VTW >= 1, "d_v tiles must split across the waves of a pair");

    // ---- LDS
    constexpr int NSIDE = (NEED_Q ? 1 : 0) + (NEED_K ? 1 : 0);
    constexpr int XSIDE = 16 * DRC * 2;            // one wave's 16 rows of Q_X or K_X
    constexpr int XWAVE = NSIDE * XSIDE;
    constexpr int XBUF = W * XWAVE;
    constexpr int VBUF = C * VC * 2;
    constexpr int NXB = 2 * NSEG;                  // X DMA blocks per wave, side and chunk
    constexpr int NXD = NSIDE * NXB;               // X DMA blocks per wave and chunk
    constexpr int NVB = NEED_V ? VBUF / 1024 : 0;  // V DMA blocks per chunk
    constexpr int NVD = NVB / W;                   // ... per wave
    // Gamma_K tile of a chunk: C rows x KC components bf16, stored and staged as one image
    constexpr int GKR = KC * 2;                    // bytes per Gamma_K row
    constexpr int GKBUF = C * GKR;                 // bytes per tile
    constexpr int GKWAVE = GKBUF / W;              // one wave's share (its own 16 rows)
    constexpr int NGD = GLOAD ? GKWAVE / 1024 : 0; // Gamma_K DMA blocks per wave and chunk
    constexpr int NGS = GSTORE ? GKWAVE / 1024 : 0;   // Gamma_K tile stores per wave and chunk
    // vector-memory stores per wave and chunk, issued after the DMA of the next chunk
    constexpr int NST = OUT ? NVT : NGS;
    // d_v tiles per output stage of the causal passes.  With an even count and no d_v padding the
    // tiles go out in pairs, 16 bytes per lane: NSTP stores per wave and chunk instead of NST.
    constexpr int VPS = (NKQ >= 8) ? 1 : ((8 / NKQ < NVT) ? 8 / NKQ : NVT);
    constexpr bool PAIRS = CAUSAL && VPS % 2 == 0;
    constexpr int NSTP = PAIRS ? NST / 2 : NST;
    // bidirectional read pass with d_v = VC: the wave's output rows go out as whole rows (16 bytes per
    // lane) from an LDS staging area, NSTF stores per chunk instead of NVT
    constexpr bool OROWS = MODE == MODE_OUT_BIDIR;
    constexpr int OROW = VC * 2 + 16;               // staging row pitch (bytes), 16 bytes of padding
    constexpr int NSTF = 16 * VC * 2 / 1024;        // 1 KiB row stores per wave and chunk
    static_assert(!OROWS || (16 * VC * 2) % 1024 == 0, "output row stores");
    static_assert(NVB % W == 0 && (NVD == 0 || NVD == 2 || NVD == 4), "V blocks must split across waves");
    static_assert(GKWAVE % 1024 == 0, "Gamma_K tile blocks");
    static_assert(NXD + NVD + NGD + NST < 64, "vmcnt range");
    constexpr int CPR = VC / 8;                    // 16-byte chunks per V row
    constexpr int RPB = 1024 / (VC * 2);           // V rows per DMA block
    static_assert((RPB == 4 || RPB == 8) && RPB * CPR == 64, "V DMA blocks");
    constexpr int OFF_XQ = 0;
    constexpr int OFF_XK = NEED_Q ? XSIDE : 0;

    __shared__ __attribute__((aligned(16))) char s_x[2 * XBUF];
    __shared__ __attribute__((aligned(16))) char s_v[NEED_V ? 2 * VBUF : 16];
    __shared__ __attribute__((aligned(16))) char s_gk[GLOAD ? 2 * GKBUF : (NEED_K ? GKBUF : 16)];
    __shared__ __attribute__((aligned(16))) char s_st[OUT ? NVT * NKQ * 1024 : 16];   // state^T fragments
    __shared__ __attribute__((aligned(16))) char s_zx[OUT ? NKQ * 1024 : 16];         // [Z_hi; Z_lo; 1; 0] fragments
    __shared__ __attribute__((aligned(16))) float s_c[KC];
    __shared__ __attribute__((aligned(16))) char s_o[OROWS ? W * 16 * OROW : 16];
    // Z of the state before the current chunk: in registers of the owning wave, except in the pass
    // that computes both the K and the Q side (its registers are full), which keeps Z in LDS
    constexpr bool ZREG = MODE != MODE_OUT_CAUSAL;
    __shared__ __attribute__((aligned(16))) float s_z[ZREG ? 4 : KC];
    lds_char* const LX = (lds_char*)s_x;
    lds_char* const LV = (lds_char*)s_v;
    lds_char* const LGK = (lds_char*)s_gk;
    lds_char* const LST = (lds_char*)s_st;
    lds_char* const LZX = (lds_char*)s_zx;
    lds_char* const LZ = (lds_char*)s_z;
    lds_char* const LC = (lds_char*)s_c;
    lds_char* const LO = (lds_char*)s_o;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    [[maybe_unused]] const int lr = lane & 15;
    [[maybe_unused]] const int lg = lane >> 4;
    const int bh = blockIdx.x / a.Pg;
    const int sidx = a.seg0 + (int)(blockIdx.x % a.Pg);
    const int h = bh % a.H;
    const int64_t N = a.N;
    const int64_t n_chunks = (N + C - 1) / C;
    const int64_t ch0 = (int64_t)sidx * a.seg_chunks;
    const int64_t ch1 = (ch0 + a.seg_chunks < n_chunks) ? ch0 + a.seg_chunks : n_chunks;
    const int kq0 = (NKQ >= W) ? w * KQW : w / WPK;
    const int vt0 = (NKQ >= W) ? 0 : (w % WPK) * VTW;
    const bool zown = (NKQ >= W) || (w % WPK == 0);   // this wave keeps Z of its components
    const uint32_t d_r = (uint32_t)a.d_r, d_v = (uint32_t)a.d_v;
    const bool pair_st = PAIRS && d_v == VC;

    const uint16_t* qx = reinterpret_cast<const uint16_t*>(a.qx) + (int64_t)bh * N * a.d_r;
    const uint16_t* kx = reinterpret_cast<const uint16_t*>(a.kx) + (int64_t)bh * N * a.d_r;
    const uint16_t* vv = reinterpret_cast<const uint16_t*>(a.v) + (int64_t)bh * N * a.d_v;
    uint16_t* oo = reinterpret_cast<uint16_t*>(a.o) + (int64_t)bh * N * a.d_v;
    // buffer descriptors over this (batch, head) slice.  Every byte offset is a vector offset (the
    // range check covers only that part), so rows past N read as zeros and their stores are dropped.
    i32x4 rs_q, rs_k, rs_v;
    __amdgpu_buffer_rsrc_t rs_o;
    if constexpr (NEED_Q) rs_q = uniform_rsrc(make_rsrc_words(qx, (uint32_t)(N * a.d_r * 2)));
    if constexpr (NEED_K) rs_k = uniform_rsrc(make_rsrc_words(kx, (uint32_t)(N * a.d_r * 2)));
    if constexpr (NEED_V) rs_v = uniform_rsrc(make_rsrc_words(vv, (uint32_t)(N * a.d_v * 2)));
    if constexpr (OUT) rs_o = make_rsrc(oo, (uint32_t)(N * a.d_v * 2));
    // Gamma_K tiles of this (batch, head): a ring of `ring` images of GKBUF bytes; chunk ch of this
    // segment sits in slot ch - gwin (the segment lies inside one ring window)
    const int64_t ring = a.gk_ring ? a.gk_ring : n_chunks;
    const int64_t gwin = (ch0 / ring) * ring;
    char* gkt = reinterpret_cast<char*>(a.gk) + (int64_t)bh * ring * GKBUF;
    i32x4 rs_g;
    __amdgpu_buffer_rsrc_t rs_gs;
    if constexpr (GLOAD) rs_g = uniform_rsrc(make_rsrc_words(gkt, (uint32_t)(ring * GKBUF)));
    if constexpr (GSTORE) rs_gs = make_rsrc(gkt, (uint32_t)(ring * GKBUF));

    // Lane id as seen inside the chunk loop: reassigned (opaque to the optimiser) at the start of every
    // chunk, so that lane-dependent offsets are recomputed there rather than held in registers
    // across the loop.  Every lambda below derives its lane quantities from it.
    int lane_v = lane;

    // ---- staged X: per wave and side, 16 rows in blocks of 8 rows x 128 bytes (block rb * NSEG + sg
    // = rows 8 rb .. 8 rb + 7, dims 64 sg .. 64 sg + 63).  The 16-byte chunks of row r are
    // XOR-swizzled by (r & 7) ^ (r >> 3) so that fragment reads are conflict-free.  Fragment step ks
    // (32 dims) of row lr for lane group lg is chunk 4 (ks & 1) + lg of segment ks / 2.
    auto xoff = [&](int ks) -> int {
        [[maybe_unused]] const int lane = lane_v, lr = lane & 15, lg = lane >> 4;
        const int xsw = lg ^ ((lr & 3) ^ ((lr >> 3) & 1));
        const int hi = (((lr >> 2) & 1) ^ (ks & 1)) << 2;
        return ((lr >> 3) * NSEG) * 1024 + (lr & 7) * 128 + ((xsw | hi) << 4) + (ks >> 1) * 1024;
    };
    // DMA: lane l of block (rb, sg) fetches row 8 rb + l/8, global chunk (l % 8) ^ (l/8) ^ rb of
    // segment sg; the vector part of its byte offset below, the rest is per block and chunk
    // V: block fv holds rows RPB fv .. RPB fv + RPB - 1 chunk-major: 16-byte chunk c of row r of the
    // block at (c RPB + r) 16 (with RPB = 4, odd blocks hold chunk c ^ 2 there).  Lane l fetches row
    // l % RPB of its block.
    const uint32_t lx_base = lds_addr(LX), lv_base = lds_addr(LV), lg_base = lds_addr(LGK);

    // DMA of chunk ch into staging buffer buf, in parts: part sd < NSIDE = own X rows of one side,
    // part NSIDE = this wave's quarter of V, part NSIDE + 1 = this wave's quarter of the Gamma_K tile
    // (a verbatim copy of the stored image)
    auto issue_part = [&](int64_t ch, int buf, int part) {
        const uint32_t lane = (uint32_t)lane_v, rl = lane >> 3;
        const uint32_t n0 = (uint32_t)(ch * C);
        if (part < NSIDE) {
            const int sd = part;
            const uint32_t xl0 = (rl * d_r + (((lane & 7) ^ rl) * 8)) * 2, xl1 = (rl * d_r + (((lane & 7) ^ rl ^ 1) * 8)) * 2;
            const uint32_t xrow = (n0 + 16 * w) * d_r * 2;   // byte offset of the wave's first row
            const uint32_t m0 = lx_base + buf * XBUF + w * XWAVE + sd * XSIDE;
            const uint32_t x0 = xl0 + xrow, x1 = xl1 + xrow + 16 * d_r;
            const i32x4& rs = (NEED_Q && sd == 0) ? rs_q : rs_k;
            if constexpr (NSEG == 2) dma16x4(rs, m0, m0 + 1024, m0 + 2048, m0 + 3072, x0, x0 + 128, x1, x1 + 128);
            else dma16x2(rs, m0, m0 + 1024, x0, x1);
        } else if (part == NSIDE) {
            if constexpr (NEED_V) {
                // with four rows per block, the blocks of odd waves (odd blocks) are rotated by 128
                // bytes (chunk index ^ 2) so that the transposed reads of two adjacent blocks do not
                // share banks
                const uint32_t vch = (lane / RPB) ^ ((RPB == 4 && (w & 1)) ? 2u : 0u);
                const uint32_t vl = ((lane % RPB) * d_v + vch * 8) * 2;
                const uint32_t vstep = W * RPB * d_v * 2;
                const uint32_t v0 = vl + (n0 + w * RPB) * d_v * 2;
                const uint32_t m0 = lv_base + buf * VBUF + w * 1024;
                if constexpr (NVD == 4)
                    dma16x4(rs_v, m0, m0 + W * 1024, m0 + 2 * W * 1024, m0 + 3 * W * 1024, v0, v0 + vstep,
                            v0 + 2 * vstep, v0 + 3 * vstep);
                else dma16x2(rs_v, m0, m0 + W * 1024, v0, v0 + vstep);
            }
        } else {
            if constexpr (GLOAD) {
                const uint32_t g0 = (uint32_t)((ch - gwin) * GKBUF) + w * GKWAVE + lane * 16;
                const uint32_t m0 = lg_base + buf * GKBUF + w * GKWAVE;
#pragma unroll
                for (int j = 0; j < NGD; j += 4) {
                    if constexpr (NGD % 4 == 0)
                        dma16x4(rs_g, m0 + j * 1024, m0 + (j + 1) * 1024, m0 + (j + 2) * 1024, m0 + (j + 3) * 1024,
                                g0 + j * 1024, g0 + (j + 1) * 1024, g0 + (j + 2) * 1024, g0 + (j + 3) * 1024);
                    else if constexpr (NGD == 2) dma16x2(rs_g, m0, m0 + 1024, g0, g0 + 1024);
                    else dma16x1(rs_g, m0, g0);
                }
            }
        }
    };
    constexpr int NPARTS = NSIDE + (NEED_V ? 1 : 0) + (GLOAD ? 1 : 0);
    static_assert(!GLOAD || NGD % 4 == 0 || NGD <= 2, "Gamma_K DMA parts");
    auto issue = [&](int64_t ch, int buf) {
#pragma unroll
        for (int part = 0; part < NPARTS; ++part) issue_part(ch, buf, part);
    };
    // the first chunk's DMA goes out before the fragment and state loads below, so that its latency
    // overlaps theirs (the waits further down then also cover those loads, which are issued after it)
    if (ch0 < ch1) issue(REV ? ch1 - 1 : ch0, 0);

    // ---- [a | b] operand fragments of every component (AGPRs), logit constants c (LDS).  Every load is
    // issued before the first is pinned, so that their latencies overlap (pinned one by one, each load
    // waited for the previous: about 16 us per workgroup at 64 fragments)
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
    }

    // ---- state share: st[kqi][hh][vti] = rows (components) of tile 2(kq0+kqi)+hh, columns of d_v
    // tile vt0+vti, in accumulator layout; Z of the owned components (zst[kqi][hh], every column of
    // the accumulator tile holds Z of its rows) in the wave that owns them
    constexpr bool HAS_STATE = AGG || OUT;
    f32x4 st[HAS_STATE ? KQW : 1][2][HAS_STATE ? VTW : 1];
    f32x4 zst[(HAS_STATE && ZREG) ? KQW : 1][2];
    const int64_t rec = (int64_t)KC * VC + KC;
    // record of this segment: index sidx - seg0 among the launch's segments (a round reuses the
    // records of the previous one; a.P is the record stride per (batch, head))
    float* segrec = a.seg + ((int64_t)bh * a.P + (sidx - a.seg0)) * rec;
    if constexpr (HAS_STATE) {
        const bool load = (MODE == MODE_OUT_BIDIR) || (CAUSAL && a.has_carry);
        const float* src = (MODE == MODE_OUT_BIDIR) ? a.seg + (int64_t)bh * a.P * rec : segrec;
#pragma unroll
        for (int kqi = 0; kqi < KQW; ++kqi)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int ct = 2 * (kq0 + kqi) + hh;
#pragma unroll
                for (int vti = 0; vti < VTW; ++vti) {
                    const int vt = vt0 + vti;
                    st[kqi][hh][vti] = load ? *reinterpret_cast<const f32x4*>(src + ((int64_t)(ct * NVT + vt) * 64 + lane) * 4)
                                            : f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
        if constexpr (ZREG) {
#pragma unroll
            for (int kqi = 0; kqi < KQW; ++kqi)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int ct = 2 * (kq0 + kqi) + hh;
                    zst[kqi][hh] = (load && zown) ? *reinterpret_cast<const f32x4*>(src + (int64_t)KC * VC + ct * 16 + lg * 4)
                                                  : f32x4{0.f, 0.f, 0.f, 0.f};
                }
        } else {
            for (int k = tid; k < KC; k += 256) s_z[k] = load ? src[(int64_t)KC * VC + k] : 0.f;
        }
        if constexpr (MODE == MODE_OUT_BIDIR) {
            // total over the segment records, added in segment order (the order of the scan kernel)
            for (int t = 1; t < a.bidir_segs; ++t) {
                const float* r = src + (int64_t)t * rec;
#pragma unroll
                for (int kqi = 0; kqi < KQW; ++kqi)
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int ct = 2 * (kq0 + kqi) + hh;
#pragma unroll
                        for (int vti = 0; vti < VTW; ++vti)
                            st[kqi][hh][vti] += *reinterpret_cast<const f32x4*>(r + ((int64_t)(ct * NVT + vt0 + vti) * 64 + lane) * 4);
                        if constexpr (ZREG) {
                            if (zown) zst[kqi][hh] += *reinterpret_cast<const f32x4*>(r + (int64_t)KC * VC + ct * 16 + lg * 4);
                        }
                    }
                if constexpr (!ZREG) {
                    for (int k = tid; k < KC; k += 256) s_z[k] += r[(int64_t)KC * VC + k];
                }
            }
        }
    }
    // bf16 state^T fragments: (vt, kq) is the A operand of O^T(vt) += state^T(vt, kq) . Gamma_Q^T(kq);
    // lane (r, g) holds d_v column 16 vt + r, components 32 kq + 4g + i and 32 kq + 16 + 4g + i
    auto write_state = [&]() {
        [[maybe_unused]] const int lane = lane_v, lr = lane & 15, lg = lane >> 4;
#pragma unroll
        for (int kqi = 0; kqi < KQW; ++kqi)
#pragma unroll
            for (int vti = 0; vti < VTW; ++vti)
                lds_st<bf16x8>(LST + ((vt0 + vti) * NKQ + kq0 + kqi) * 1024 + lane * 16,
                               pack_pair(st[kqi][0][vti], st[kqi][1][vti]));
    };
    // Z fragments for the denominators: row 4m + 0 holds Z rounded to bf16, row 4m + 1 the bf16 of
    // the remainder, row 4m + 2 ones (the row sum of Gamma_Q), row 4m + 3 zeros.  Branch-free: both
    // halves are formed on every lane and the lane's row type selects by bit masks.
    auto write_z = [&]() {
        if (!zown) return;
        [[maybe_unused]] const int lane = lane_v, lr = lane & 15, lg = lane >> 4;
        const uint32_t typ = (uint32_t)lr & 3u;
        const uint32_t mh = (typ == 0u) ? 0xffffffffu : 0u;
        const uint32_t ml = (typ == 1u) ? 0xffffffffu : 0u;
        const uint32_t mo = (typ == 2u) ? 0x3f803f80u : 0u;   // two bf16 ones
#pragma unroll
        for (int kqi = 0; kqi < KQW; ++kqi) {
            u32x4 f;
            f32x4 zq[2];
            if constexpr (ZREG) {
                zq[0] = zst[kqi][0];
                zq[1] = zst[kqi][1];
            } else {
                zq[0] = lds_ld<f32x4>(LZ + ((kq0 + kqi) * 32 + lg * 4) * 4);
                zq[1] = lds_ld<f32x4>(LZ + ((kq0 + kqi) * 32 + 16 + lg * 4) * 4);
            }
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const float z0 = zq[p >> 1][2 * (p & 1)], z1 = zq[p >> 1][2 * (p & 1) + 1];
                const uint32_t hb = pack2_bf16(z0, z1);
                const uint32_t lb = pack2_bf16(z0 - __uint_as_float(hb << 16), z1 - __uint_as_float(hb & 0xffff0000u));
                f[p] = (hb & mh) | (lb & ml) | mo;
            }
            lds_st<u32x4>(LZX + (kq0 + kqi) * 1024 + lane * 16, f);
        }
    };
    // the bidirectional pass reads the fixed total state; the causal pass publishes the state before
    // each chunk at the start of that chunk (after barrier B0, read after B1)
    if constexpr (MODE == MODE_OUT_BIDIR) {
        write_state();
        write_z();
    }

    lds_barrier();   // s_c (and the bidirectional state) visible

    // Passes with one logits side (the aggregate passes: K; the stored-tile causal pass: Q) read the
    // X operand words and the logit constants of the next chunk from LDS at the end of the current
    // one (its X rows have landed by then), so that their latency overlaps the chunk boundary
    // instead of the start of the logits
    constexpr bool PIPE = AGG || GLOAD;
    constexpr int OFF_P = GLOAD ? OFF_XQ : OFF_XK;
    u32x4 xraw_n[PIPE ? NKS2 : 1];
    f32x4 acc_n[PIPE ? NCT : 1];
    auto prefetch_x = [&](const lds_char* xw) {
        [[maybe_unused]] const int lane = lane_v, lr = lane & 15, lg = lane >> 4;
#pragma unroll
        for (int ks = 0; ks < NKS2; ++ks) xraw_n[ks] = lds_ld<u32x4>(xw + OFF_P + xoff(ks));
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) acc_n[ct] = lds_ld<f32x4>(LC + (ct * 16 + lg * 4) * 4);
    };
    if constexpr (PIPE) {
        wait_vmcnt<NVD + NGD>();   // own X rows of the first chunk
        prefetch_x(LX + w * XWAVE);
    }

    // ---- Gamma_K tile: row-major [token][component] bf16 without padding; the 8-byte slots (four
    // components) of row r are XOR-swizzled by (bits of r & 15 written r3 r2 r1 r0)
    //   KC >= 128: r2 r1 r0 r3 r2      KC = 64: r2 r1 r3 r0      KC = 32: r2 r3 r1
    // LDS serves 8-byte reads 32 lanes at a time over 256 bytes of banks, and 8-byte writes 16 lanes
    // at a time over 128 bytes.  With this swizzle the row reads of S^T (one or two slots of 16
    // consecutive rows per 32 lanes), the transposed reads of the state update (four slots of eight
    // consecutive rows per 32 lanes) and the row writes (one slot of 16 rows per 16 lanes) each touch
    // every bank once.  The stored tiles use the same image, so the causal output pass copies them
    // into LDS unchanged.
    auto gk_off = [](int row, int slot) -> int {
        const int r = row & 15;
        const int sw = (KC >= 128) ? (((r & 7) << 2) | (((r >> 3) & 1) << 1) | ((r >> 2) & 1))
                     : (KC == 64)  ? ((((r >> 1) & 3) << 2) | (((r >> 3) & 1) << 1) | (r & 1))
                                   : ((((r >> 2) & 1) << 2) | (((r >> 3) & 1) << 1) | ((r >> 1) & 1));
        return row * GKR + ((slot ^ sw) << 3);
    };
    // A of S^T = Gamma_K Gamma_Q^T: lane = token 16 J + r, slots = components of pair kq
    auto gk_token_frag = [&](const lds_char* gkb, int J, int kq) -> bf16x8 {
        [[maybe_unused]] const int lane = lane_v, lr = lane & 15, lg = lane >> 4;
        const int row = J * 16 + lr;
        const u32x2 lo = lds_ld<u32x2>(gkb + gk_off(row, 8 * kq + lg));
        const u32x2 hi = lds_ld<u32x2>(gkb + gk_off(row, 8 * kq + 4 + lg));
        return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
    };
    // A of the state update Gamma_K^T V: lane = component 16 ct + r, slots = tokens of step tk
    // (tokens 32 tk + 4g + i and 32 tk + 16 + 4g + i, the order of the V fragments)
    auto gk_comp_frag = [&](const lds_char* gkb, int ct, int tk) -> bf16x8 {
        [[maybe_unused]] const int lane = lane_v, lr = lane & 15, lg = lane >> 4;
        const int q = lane & 3, i4 = (lane >> 2) & 3;
        u32x2 part[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int row = (2 * tk + hf) * 16 + lg * 4 + i4;
            part[hf] = ds_read_tr16_at(gkb + gk_off(row, 4 * ct + q));
        }
        return __builtin_bit_cast(bf16x8, u32x4{part[0][0], part[0][1], part[1][0], part[1][1]});
    };
    // V^T fragment (d_v tile vt, token step tk) from the chunk-major V blocks: A of O^T += V^T S^T
    // and, with the same contents, B of the state update.  Lane 16g + 4 i4 + q reads row
    // 32 tk + 16 hf + 4g + i4, chunk 2 vt + q/2, half q % 2; a 16-lane group covers 128 contiguous
    // bytes (conflict-free) and the address is affine in vt and tk.
    auto v_frag = [&](const lds_char* vb, int vt, int tk) -> bf16x8 {
        [[maybe_unused]] const int lane = lane_v, lr = lane & 15, lg = lane >> 4;
        // odd blocks (four rows per block: lane group lg reads block lg of its token step) are
        // rotated by 128 bytes: there d_v tile vt sits where tile vt ^ 1 sits in even blocks
        const int rot = (RPB == 4) ? (lg & 1) * ((vt & 1) ? -128 : 128) : 0;
        const int v_lane_off = (((lg * 4 + ((lane >> 2) & 3)) / RPB) * 1024) +
                               ((((lane & 3) >> 1) * RPB + (lg * 4 + ((lane >> 2) & 3)) % RPB) * 16) + (lane & 1) * 8 + rot;
        u32x2 part[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
            part[hf] = ds_read_tr16_at(vb + v_lane_off + ((2 * tk + hf) * (16 / RPB)) * 1024 + (2 * vt) * RPB * 16);
        return __builtin_bit_cast(bf16x8, u32x4{part[0][0], part[0][1], part[1][0], part[1][1]});
    };

    // fp16 operand fragments [x ; x^2] of own tokens (bf16 -> fp16 is exact in the supported range)
    auto x_frags = [&](const lds_char* xs, f16x8 (&xf)[NKS2], f16x8 (&x2)[NKS2]) {
        u32x4 raw[NKS2];
#pragma unroll
        for (int ks = 0; ks < NKS2; ++ks) raw[ks] = lds_ld<u32x4>(xs + xoff(ks));
#pragma unroll
        for (int ks = 0; ks < NKS2; ++ks) {
            xf[ks] = bf16x8_bits_to_f16x8(raw[ks]);
            x2[ks] = xf[ks] * xf[ks];
        }
    };
    // logits^T of own tokens: acc[ct] rows = components 16 ct + 4g + i, column = token 16 w + r
    auto logits = [&](const f16x8 (&xf)[NKS2], const f16x8 (&x2)[NKS2], f32x4 (&acc)[NCT]) {
        [[maybe_unused]] const int lane = lane_v, lr = lane & 15, lg = lane >> 4;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) acc[ct] = lds_ld<f32x4>(LC + (ct * 16 + lg * 4) * 4);
#pragma unroll
        for (int ks = 0; ks < NKS2; ++ks) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                pin_agpr(abf[ct][ks]);
                mma(acc[ct], abf[ct][ks], x2[ks]);
            }
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                pin_agpr(abf[ct][ks + NKS2]);
                mma(acc[ct], abf[ct][ks + NKS2], xf[ks]);
            }
        }
    };
    // set on a lane that met a row whose logits are not finite (a routing input or a coefficient past
    // the fp16 operand range): a row maximum of -inf or NaN, or (output passes) a denominator that is
    // NaN or inf, which a NaN logit of the row or of any key it reads makes it (the maximum skips NaN).
    // The (batch, head) is flagged after the chunk loop.  Rows past N have zero inputs and finite logits.
    bool nonfin = false;
    // 2^(l - max_k l) in place (base-2 logits)
    auto exp_rows = [&](f32x4 (&acc)[NCT]) {
        float m = acc[0][0];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) m = fmaxf(m, acc[ct][i]);
        m = group4_max(m);
        nonfin |= !(m > -INFINITY);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[ct][i] = fast_exp2(acc[ct][i] - m);
    };
    // own Gamma_K rows (normalised; rows past N are zero) into LDS
    auto write_gk = [&](f32x4 (&acc)[NCT], bool valid) {
        [[maybe_unused]] const int lane = lane_v, lr = lane & 15, lg = lane >> 4;
        float s = 0.f;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) s += acc[ct][i];
        s = group4_sum(s);
        const float r = valid ? fast_rcp(s) : 0.f;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) lds_st<bf16x4>(LGK + gk_off(16 * w + lr, 4 * ct + lg), pack4(acc[ct] * r));
    };
    // own output rows: lane (r, g) holds d_v 16 vt + 4g .. +3 of token 16 w + r.  Without d_v padding
    // the column offsets are instruction immediates; with padding, pad columns get an offset past
    // the end of the buffer (dropped), computed without compares.
    auto store_tile = [&](const f32x4& o, float inv, uint32_t base, int vt) {
        [[maybe_unused]] const int lane = lane_v, lr = lane & 15, lg = lane >> 4;
        const u32x2 v = __builtin_bit_cast(u32x2, pack4(o * inv));
        if (d_v == VC) {
            __builtin_amdgcn_raw_buffer_store_b64(v, rs_o, base, vt * 32, 0);
        } else {
            const int spare = (int)d_v - 1 - (lg * 4) - vt * 16;   // < 0 for pad columns
            store_b64(rs_o, v, (base + vt * 32) | ((uint32_t)(spare >> 31) & 0x80000000u));
        }
    };
    auto row_base = [&](uint32_t tok) -> uint32_t { return (tok * d_v + (lane_v >> 4) * 4) * 2; };
    // Two d_v tiles 2p, 2p + 1 stored as 16 bytes per lane: one lane-row exchange (rows of 16 lanes
    // g = 1, 3 of tile 2p trade places with rows g = 0, 2 of tile 2p + 1) leaves lane (r, g) with d_v
    // columns 32p + pcol(g) .. +7 of token 16 w + r, pcol = 0, 16, 8, 24 for g = 0 .. 3: 64 contiguous
    // bytes of each token row per store instruction instead of two 32-byte pieces.
    auto pair_base = [&](uint32_t tok) -> uint32_t {
        const int g = lane_v >> 4;
        return (tok * d_v + 16 * (g & 1) + 8 * (g >> 1)) * 2;
    };
    auto store_pair = [&](const f32x4& o0, const f32x4& o1, float inv, uint32_t base, int p) {
        const u32x2 x = __builtin_bit_cast(u32x2, pack4(o0 * inv));
        const u32x2 y = __builtin_bit_cast(u32x2, pack4(o1 * inv));
        const auto s0 = __builtin_amdgcn_permlane16_swap(x[0], y[0], false, false);
        const auto s1 = __builtin_amdgcn_permlane16_swap(x[1], y[1], false, false);
        const u32x4 v = {s0[0], s1[0], s0[1], s1[1]};
        __builtin_amdgcn_raw_buffer_store_b128(v, rs_o, base, p * 64, 0);
    };

    // causal mask of the intra-chunk tiles: key 16 J + 4g + i is kept for query 16 w + r when
    // 16 J + i <= 16 w + r - 4g; as a factor 0 / 1 from a clamped difference (no per-element compare)
    auto keep_base = [&]() -> float {
        [[maybe_unused]] const int lane = lane_v, lr = lane & 15, lg = lane >> 4;
        return (float)(16 * w + lr - 4 * lg + 1);
    };
    const uint32_t N32 = (uint32_t)N;

    auto body = [&](auto buf_tag, int64_t ch) {
        constexpr int BUF = decltype(buf_tag)::value;
        lane_v = opaque_v(lane);
        [[maybe_unused]] const int lane = lane_v, lr = lane & 15, lg = lane >> 4;
        const uint32_t n0 = (uint32_t)(ch * C);
        const bool first = REV ? ch == ch1 - 1 : ch == ch0;
        const bool has_next = REV ? ch > ch0 : ch + 1 < ch1;
        const int64_t nxt = REV ? ch - 1 : ch + 1;
        const lds_char* xw = LX + BUF * XBUF + w * XWAVE;
        const lds_char* vb = LV + (NEED_V ? BUF * VBUF : 0);
        const uint32_t tok = n0 + 16 * w + lr;

        // own X rows of this chunk landed (V and the Gamma_K tile of the chunk and the previous
        // chunk's stores may still be in flight)
        if constexpr (PIPE) {
            // own X rows waited for and read at the end of the previous chunk.  B0 needs no LDS
            // wait: every read of the previous chunk's shared buffers has been consumed.
            block_barrier();   // B0
        } else {
            if (first) wait_vmcnt<NVD + NGD>();
            else if (OROWS && d_v == VC) wait_vmcnt<NVD + NGD + NSTF>();
            else if (pair_st) wait_vmcnt<NVD + NGD + NSTP>();
            else wait_vmcnt<NVD + NGD + NST>();
            if constexpr (NEED_V) lds_barrier();   // B0
        }
        if constexpr (!CAUSAL && !AGG) {
            if (has_next) issue(nxt, BUF ^ 1);
        }

        if constexpr (MODE == MODE_OUT_BIDIR) {
            // Gamma_Q of own tokens, then O^T = state^T Gamma_Q^T with the fixed total state
            f16x8 xf[NKS2], x2[NKS2];
            x_frags(xw + OFF_XQ, xf, x2);
            f32x4 acc[NCT];
            logits(xf, x2, acc);
            exp_rows(acc);
            bf16x8 pq[NKQ];
#pragma unroll
            for (int kq = 0; kq < NKQ; ++kq) pq[kq] = pack_pair(acc[2 * kq], acc[2 * kq + 1]);
            f32x4 oacc[NVT];
            f32x4 dx = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt) oacc[vt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kq = 0; kq < NKQ; ++kq) {
#pragma unroll
                for (int vt = 0; vt < NVT; ++vt)
                    mma(oacc[vt], lds_ld<bf16x8>(LST + (vt * NKQ + kq) * 1024 + lane * 16), pq[kq]);
                mma(dx, lds_ld<bf16x8>(LZX + kq * 1024 + lane * 16), pq[kq]);
            }
            const float den = dx[0] + dx[1] + a.eps * dx[2];
            nonfin |= !(den < INFINITY);   // NaN or inf: a logit of this row or a key's was not finite
            const float inv = fast_rcp(den);
            if (d_v == VC) {
                // rows through LDS: lane (r, g) puts d_v 16 vt + 4g .. +3 of row r, then lane l takes
                // 16 bytes (chunk l % (VC / 8)) of row i (64 / (VC / 8)) + l / (VC / 8) per store
                lds_char* ow = LO + w * 16 * OROW;
#pragma unroll
                for (int vt = 0; vt < NVT; ++vt)
                    lds_st<u32x2>(ow + lr * OROW + (16 * vt + 4 * lg) * 2, __builtin_bit_cast(u32x2, pack4(oacc[vt] * inv)));
                asm volatile("" ::: "memory");
                constexpr int CPR2 = VC / 8;        // 16-byte chunks per row
                constexpr int RPS = 64 / CPR2;      // rows per store
#pragma unroll
                for (int i = 0; i < NSTF; ++i) {
                    const int row = i * RPS + lane / CPR2, chunk = lane % CPR2;
                    const u32x4 v = lds_ld<u32x4>(ow + row * OROW + chunk * 16);
                    __builtin_amdgcn_raw_buffer_store_b128(v, rs_o, ((n0 + 16 * w + row) * d_v) * 2 + chunk * 16, 0, 0);
                }
            } else {
                const uint32_t base = row_base(tok);
#pragma unroll
                for (int vt = 0; vt < NVT; ++vt) store_tile(oacc[vt], inv, base, vt);
            }
            return;
        } else {
            // ---- P1
            bf16x8 pq[CAUSAL ? NKQ : 1];
            // one 32-bit word (two bf16) of staged X to fp16 x and x^2 (exact in the supported range)
            auto cvt_word = [](const u32x4& raw, int e, f16x8& xf, f16x8& x2) {
                const auto h = __builtin_amdgcn_cvt_pkrtz(__uint_as_float(raw[e] << 16), __uint_as_float(raw[e] & 0xffff0000u));
                xf[2 * e] = h[0];
                xf[2 * e + 1] = h[1];
                x2[2 * e] = h[0] * h[0];
                x2[2 * e + 1] = h[1] * h[1];
            };
            constexpr int NPUB = KQW * VTW;   // state fragments to publish
            if constexpr (PIPE) {
                // One logits side (stored-tile causal pass: Q, Gamma_K of the chunk arrives as a stored
                // tile; aggregate passes: K).  The logits MFMAs, each pair followed by one small piece
                // of independent vector work: one 32-bit word of the fp16 conversion of the next X
                // step, (causal) one fragment of the state publication or the Z fragments, a part of
                // the next chunk's DMA.
                u32x4 xraw[NKS2];
                f32x4 acc[NCT];
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) acc[ct] = acc_n[ct];
#pragma unroll
                for (int ks = 0; ks < NKS2; ++ks) xraw[ks] = xraw_n[ks];
                f16x8 xf[NKS2], x2[NKS2];
#pragma unroll
                for (int e = 0; e < 4; ++e) cvt_word(xraw[0], e, xf[0], x2[0]);
                fence();
                constexpr int NPUBP = GLOAD ? NPUB : 0;
                auto piece = [&](int ks, int p) {
                    const int nq = (ks + 1 < NKS2) ? 4 : 0;
                    if (p < nq) { cvt_word(xraw[ks + 1], p, xf[ks + 1], x2[ks + 1]); return; }
                    p -= nq;
                    if constexpr (GLOAD) {
                        const int npub = (NPUBP - ks + NKS2 - 1) / NKS2;   // j = ks, ks + NKS2, ...
                        if (p < npub) {
                            const int jj = ks + p * NKS2;
                            const int kqi = jj / VTW, vti = jj % VTW;
                            lds_st<bf16x8>(LST + ((vt0 + vti) * NKQ + kq0 + kqi) * 1024 + lane * 16,
                                           pack_pair(st[kqi][0][vti], st[kqi][1][vti]));
                            return;
                        }
                        p -= npub;
                        if (ks == NKS2 - 1) {
                            if (p == 0) { write_z(); return; }
                            p -= 1;
                        }
                    }
                    const int d0 = ks * NPARTS / NKS2, d1 = (ks + 1) * NPARTS / NKS2;
                    if (p < d1 - d0 && has_next) issue_part(nxt, BUF ^ 1, d0 + p);
                };
                if constexpr (AGG) {
                    // Aggregate passes: tile order.  Component tile ct's chain of 2 NKS2 MFMAs accumulates
                    // in place (measured faster here; the step order below is faster in the causal pass);
                    // the fp16 conversion of the next X steps rides on tile 0, the DMA parts on tiles >= 1.
                    constexpr int NXS = (NCT - 1) * NKS2;
                    constexpr int EPS = (NPARTS + NXS - 1) / NXS;   // DMA parts per slot
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
                        for (int ks = 0; ks < NKS2; ++ks) {
                            mma(acc[ct], abf[ct][ks], x2[ks]);
                            mma(acc[ct], abf[ct][ks + NKS2], xf[ks]);
                            if (ct == 0) {
                                if (ks + 1 < NKS2) {
#pragma unroll
                                    for (int e = 0; e < 4; ++e) cvt_word(xraw[ks + 1], e, xf[ks + 1], x2[ks + 1]);
                                }
                            } else {
                                const int sl = (ct - 1) * NKS2 + ks;
#pragma unroll
                                for (int t = 0; t < EPS; ++t)
                                    if (sl * EPS + t < NPARTS && has_next) issue_part(nxt, BUF ^ 1, sl * EPS + t);
                            }
                            fence();
                        }
                    }
                } else {
                    constexpr int NPQ = 4 + (NPUBP + NKS2 - 1) / NKS2 + (GLOAD ? 1 : 0) + (NPARTS + NKS2 - 1) / NKS2;
                    constexpr int PPQ = (NPQ + NCT - 1) / NCT;   // pieces per MFMA pair
#pragma unroll
                    for (int ks = 0; ks < NKS2; ++ks) {
#pragma unroll
                        for (int ct = 0; ct < NCT; ++ct) {
                            mma(acc[ct], abf[ct][ks], x2[ks]);
                            mma(acc[ct], abf[ct][ks + NKS2], xf[ks]);
#pragma unroll
                            for (int t = 0; t < PPQ; ++t) piece(ks, ct * PPQ + t);
                            fence();
                        }
                }
                }
                exp_rows(acc);
                if constexpr (GLOAD) {
#pragma unroll
                    for (int kq = 0; kq < NKQ; ++kq) pq[kq] = pack_pair(acc[2 * kq], acc[2 * kq + 1]);
                } else {
                    write_gk(acc, tok < N32);
                }
            } else if constexpr (CAUSAL) {
                // Region A: the K-side logits MFMAs, each pair followed by one small piece of independent
                // vector work: one 32-bit word of the fp16 conversion of the next K_X step or of a Q_X
                // step, one fragment of the state publication, a part of the next chunk's DMA.  Region B:
                // the Q-side logits MFMAs, each pair followed by a piece of the K-side softmax (running
                // max, exp per tile, sum per tile, normalisation and the Gamma_K row per tile).  The
                // pieces are fenced one by one so that the issue order stays interleaved.
                u32x4 kraw[NKS2], qraw[NKS2];
                f32x4 acck[NCT], accq[NCT];
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) acck[ct] = lds_ld<f32x4>(LC + (ct * 16 + lg * 4) * 4);
#pragma unroll
                for (int ks = 0; ks < NKS2; ++ks) kraw[ks] = lds_ld<u32x4>(xw + OFF_XK + xoff(ks));
#pragma unroll
                for (int ks = 0; ks < NKS2; ++ks) qraw[ks] = lds_ld<u32x4>(xw + OFF_XQ + xoff(ks));
                f16x8 kxf[NKS2], kx2[NKS2], qxf[NKS2], qx2[NKS2];
#pragma unroll
                for (int e = 0; e < 4; ++e) cvt_word(kraw[0], e, kxf[0], kx2[0]);
                fence();
                // pieces of step ks, in order: K_X words of step ks+1, Q_X words of step ks, state
                // fragments j = ks (mod NKS2), the Z fragments (last step), the DMA parts (steps 0..)
                auto piece_a = [&](int ks, int p) {
                    const int nk = (ks + 1 < NKS2) ? 4 : 0;
                    if (p < nk) { cvt_word(kraw[ks + 1], p, kxf[ks + 1], kx2[ks + 1]); return; }
                    p -= nk;
                    if (p < 4) { cvt_word(qraw[ks], p, qxf[ks], qx2[ks]); return; }
                    p -= 4;
                    const int npub = (NPUB - ks + NKS2 - 1) / NKS2;   // j = ks, ks + NKS2, ...
                    if (p < npub) {
                        const int jj = ks + p * NKS2;
                        const int kqi = jj / VTW, vti = jj % VTW;
                        lds_st<bf16x8>(LST + ((vt0 + vti) * NKQ + kq0 + kqi) * 1024 + lane * 16,
                                       pack_pair(st[kqi][0][vti], st[kqi][1][vti]));
                        return;
                    }
                    p -= npub;
                    if (ks == NKS2 - 1) {
                        if (p == 0) { write_z(); return; }
                        p -= 1;
                    }
                    // DMA parts: step ks issues the parts ks * NPARTS / NKS2 .. (ks + 1) * NPARTS / NKS2 - 1
                    const int d0 = ks * NPARTS / NKS2, d1 = (ks + 1) * NPARTS / NKS2;
                    if (p < d1 - d0 && has_next) issue_part(nxt, BUF ^ 1, d0 + p);
                };
                // most pieces in one step: K and Q words, state fragments, Z, DMA parts
                constexpr int NPA = 4 + 4 + (NPUB + NKS2 - 1) / NKS2 + 1 + (NPARTS + NKS2 - 1) / NKS2;
                constexpr int PPA = (NPA + NCT - 1) / NCT;   // pieces per MFMA pair
#pragma unroll
                for (int ks = 0; ks < NKS2; ++ks) {
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) {
                        mma(acck[ct], abf[ct][ks], kx2[ks]);
                        mma(acck[ct], abf[ct][ks + NKS2], kxf[ks]);
#pragma unroll
                        for (int t = 0; t < PPA; ++t) piece_a(ks, ct * PPA + t);
                        fence();
                    }
                }
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) accq[ct] = lds_ld<f32x4>(LC + (ct * 16 + lg * 4) * 4);
                fence();
                // K-side softmax pieces: 0: running max over tiles 0..NCT-1 (one piece per two tiles),
                // then the cross-lane max; exp per tile; row-sum per two tiles, cross-lane sum and
                // reciprocal; normalisation, bf16 pack and LDS row write per tile
                float mk = -INFINITY, sk = 0.f, rk = 0.f;
                constexpr int NMAXP = NCT / 2, NSUMP = NCT / 2;
                constexpr int NKSOFT = NMAXP + 1 + NCT + NSUMP + 1 + NCT;
                auto piece_b = [&](int p) {
                    if (p < NMAXP) {
#pragma unroll
                        for (int c = 2 * p; c < 2 * p + 2; ++c)
                            mk = fmaxf(mk, fmaxf(fmaxf(acck[c][0], acck[c][1]), fmaxf(acck[c][2], acck[c][3])));
                        return;
                    }
                    p -= NMAXP;
                    if (p == 0) {
                        mk = group4_max(mk);
                        nonfin |= !(mk > -INFINITY);
                        return;
                    }
                    p -= 1;
                    if (p < NCT) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) acck[p][i] = fast_exp2(acck[p][i] - mk);
                        return;
                    }
                    p -= NCT;
                    if (p < NSUMP) {
#pragma unroll
                        for (int c = 2 * p; c < 2 * p + 2; ++c) sk += (acck[c][0] + acck[c][1]) + (acck[c][2] + acck[c][3]);
                        return;
                    }
                    p -= NSUMP;
                    if (p == 0) { sk = group4_sum(sk); rk = (tok < N32) ? fast_rcp(sk) : 0.f; return; }
                    p -= 1;
                    if (p < NCT) lds_st<bf16x4>(LGK + gk_off(16 * w + lr, 4 * p + lg), pack4(acck[p] * rk));
                };
                constexpr int PPB = (NKSOFT + NCT * NKS2 - 1) / (NCT * NKS2);   // pieces per MFMA pair
#pragma unroll
                for (int ks = 0; ks < NKS2; ++ks) {
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) {
                        mma(accq[ct], abf[ct][ks], qx2[ks]);
                        mma(accq[ct], abf[ct][ks + NKS2], qxf[ks]);
#pragma unroll
                        for (int t = 0; t < PPB; ++t) piece_b((ks * NCT + ct) * PPB + t);
                        fence();
                    }
                }
                exp_rows(accq);
#pragma unroll
                for (int kq = 0; kq < NKQ; ++kq) pq[kq] = pack_pair(accq[2 * kq], accq[2 * kq + 1]);
            }

            // own V blocks (and Gamma_K blocks) of this chunk landed, then B1
            if (first) {
                if (has_next) wait_vmcnt<NXD + NVD + NGD>();
                else wait_vmcnt<0>();
            } else {
                if (pair_st) {
                    if (has_next) wait_vmcnt<NSTP + NXD + NVD + NGD>();
                    else wait_vmcnt<NSTP>();
                } else {
                    if (has_next) wait_vmcnt<NST + NXD + NVD + NGD>();
                    else wait_vmcnt<NST>();
                }
            }
            lds_barrier();   // B1
            const lds_char* gkb = LGK + (GLOAD ? BUF * GKBUF : 0);
            if constexpr (GSTORE) {
                // this wave's quarter of the chunk's Gamma_K tile to HBM, verbatim
#pragma unroll
                for (int j = 0; j < NGS; ++j) {
                    const int off = w * GKWAVE + j * 1024 + lane * 16;
                    __builtin_amdgcn_raw_buffer_store_b128(lds_ld<u32x4>(LGK + off), rs_gs, (uint32_t)((ch - gwin) * GKBUF) + off, 0, 0);
                }
            }

            // ---- P2
            constexpr bool ALL_VT = (VTW == NVT);
            bf16x8 gkc[KQW][2][2];
#pragma unroll
            for (int kqi = 0; kqi < KQW; ++kqi)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int tk = 0; tk < 2; ++tk) gkc[kqi][hh][tk] = gk_comp_frag(gkb, 2 * (kq0 + kqi) + hh, tk);

            // Software pipeline over stages: each stage first issues the LDS reads of the next stage,
            // then the matrix work of the current one (fences keep the order), so that LDS latency
            // is covered by MFMAs.
            constexpr int VP = VPS;   // d_v tiles per stage
            static_assert(NVT % VP == 0, "d_v tile stages");
            bf16x8 vfr[2][VP][2];
            bf16x8 sst[2][VP][CAUSAL ? NKQ : 1];
            auto load_vstage = [&](int buf, int vs) {
#pragma unroll
                for (int j = 0; j < VP; ++j) {
                    const int vt = vs * VP + j;
                    if constexpr (CAUSAL || ALL_VT) {
                        vfr[buf][j][0] = v_frag(vb, vt, 0);
                        vfr[buf][j][1] = v_frag(vb, vt, 1);
                    }
                    if constexpr (CAUSAL) {
#pragma unroll
                        for (int kq = 0; kq < NKQ; ++kq) sst[buf][j][kq] = lds_ld<bf16x8>(LST + (vt * NKQ + kq) * 1024 + lane * 16);
                    }
                }
            };

            bf16x8 sfr[2];
            float inv = 0.f;
            if constexpr (CAUSAL) {
                // intra-chunk affinities of own queries S^T(J, w) = Gamma_K[J] Gamma_Q[w]^T for all four
                // key blocks (the same work on every wave), causally masked; operand fragments over
                // the two token steps and their column sums.  Denominators: Gamma_Q . Z (hi + lo) and
                // eps * rowsum(Gamma_Q) from the Z fragments.
                constexpr int SKQ = (NKQ >= 2) ? 2 : 1;   // component steps per stage
                bf16x8 gt[2][SKQ][4];
                bf16x8 zx[2][SKQ];
                auto load_sstage = [&](int buf, int k0) {
#pragma unroll
                    for (int sq = 0; sq < SKQ; ++sq) {
#pragma unroll
                        for (int J = 0; J < 4; ++J) gt[buf][sq][J] = gk_token_frag(gkb, J, k0 + sq);
                        zx[buf][sq] = lds_ld<bf16x8>(LZX + (k0 + sq) * 1024 + lane * 16);
                    }
                };
                f32x4 sacc[4];
                f32x4 dx = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int J = 0; J < 4; ++J) sacc[J] = f32x4{0.f, 0.f, 0.f, 0.f};
                load_sstage(0, 0);
                fence();
#pragma unroll
                for (int k0 = 0; k0 < NKQ; k0 += SKQ) {
                    const int cb = (k0 / SKQ) & 1;
                    if (k0 + SKQ < NKQ) load_sstage(cb ^ 1, k0 + SKQ);
                    else load_vstage(0, 0);
#pragma unroll
                    for (int sq = 0; sq < SKQ; ++sq) {
#pragma unroll
                        for (int J = 0; J < 4; ++J) mma(sacc[J], gt[cb][sq][J], pq[k0 + sq]);
                        mma(dx, zx[cb][sq], pq[k0 + sq]);
                    }
                    fence();
                }
                const float kb = keep_base();
#pragma unroll
                for (int J = 0; J < 4; ++J)
#pragma unroll
                    for (int i = 0; i < 4; ++i) sacc[J][i] *= __builtin_amdgcn_fmed3f(kb - (float)(16 * J + i), 0.f, 1.f);
                const bf16x8 ones = ones_frag<bf16x8>();
                f32x4 dacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    sfr[t] = pack_pair(sacc[2 * t], sacc[2 * t + 1]);
                    mma(dacc, ones, sfr[t]);
                }
                const float den = dx[0] + dx[1] + a.eps * dx[2] + dacc[0];
                nonfin |= !(den < INFINITY);   // NaN or inf: a logit of this row or an earlier key's was not finite
                inv = fast_rcp(den);
            } else {
                if constexpr (ALL_VT) load_vstage(0, 0);
            }
            const uint32_t obase = pair_st ? pair_base(tok) : row_base(tok);
            auto store_stage = [&](const f32x4 (&ot)[VP], int vs) {
                if constexpr (PAIRS) {
                    if (pair_st) {
#pragma unroll
                        for (int j = 0; j < VP; j += 2) store_pair(ot[j], ot[j + 1], inv, obase, (vs * VP + j) / 2);
                        return;
                    }
                }
#pragma unroll
                for (int j = 0; j < VP; ++j) store_tile(ot[j], inv, obase, vs * VP + j);
            };
            fence();

            // stages of VP d_v tiles: inter (state before the chunk) and intra output of own queries,
            // state update of the owned share; each stage's output tiles are stored during the next
            if constexpr (CAUSAL || ALL_VT) {
                f32x4 oprev[VP];
#pragma unroll
                for (int vs = 0; vs < NVT / VP; ++vs) {
                    const int cb = vs & 1;
                    if (vs + 1 < NVT / VP) load_vstage(cb ^ 1, vs + 1);
                    f32x4 o[VP];
                    if constexpr (CAUSAL) {
#pragma unroll
                        for (int j = 0; j < VP; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int kq = 0; kq < NKQ; ++kq)
#pragma unroll
                            for (int j = 0; j < VP; ++j) mma(o[j], sst[cb][j][kq], pq[kq]);
#pragma unroll
                        for (int t = 0; t < 2; ++t)
#pragma unroll
                            for (int j = 0; j < VP; ++j) mma(o[j], vfr[cb][j][t], sfr[t]);
                    }
                    if constexpr (ALL_VT) {
#pragma unroll
                        for (int tk = 0; tk < 2; ++tk)
#pragma unroll
                            for (int j = 0; j < VP; ++j)
#pragma unroll
                                for (int kqi = 0; kqi < KQW; ++kqi)
#pragma unroll
                                    for (int hh = 0; hh < 2; ++hh)
                                        mma(st[kqi][hh][vs * VP + j], gkc[kqi][hh][tk], vfr[cb][j][tk]);
                    }
                    if constexpr (CAUSAL) {
                        if (vs > 0) store_stage(oprev, vs - 1);
#pragma unroll
                        for (int j = 0; j < VP; ++j) oprev[j] = o[j];
                    }
                    fence();
                }
                if constexpr (CAUSAL) store_stage(oprev, NVT / VP - 1);
            }
            if constexpr (!ALL_VT) {
                // the owned d_v tiles are a slice: fetch their V fragments again
#pragma unroll
                for (int vti = 0; vti < VTW; ++vti) {
                    const bf16x8 vf0 = v_frag(vb, vt0 + vti, 0);
                    const bf16x8 vf1 = v_frag(vb, vt0 + vti, 1);
#pragma unroll
                    for (int kqi = 0; kqi < KQW; ++kqi)
#pragma unroll
                        for (int hh = 0; hh < 2; ++hh) {
                            mma(st[kqi][hh][vti], gkc[kqi][hh][0], vf0);
                            mma(st[kqi][hh][vti], gkc[kqi][hh][1], vf1);
                        }
                }
            }
            // Z of the owned components: column sums of the same bf16 Gamma_K (all-ones operand)
            if (zown) {
                const bf16x8 ones = ones_frag<bf16x8>();
#pragma unroll
                for (int kqi = 0; kqi < KQW; ++kqi)
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        if constexpr (ZREG) {
                            mma(zst[kqi][hh], gkc[kqi][hh][0], ones);
                            mma(zst[kqi][hh], gkc[kqi][hh][1], ones);
                        } else {
                            f32x4 zi = {0.f, 0.f, 0.f, 0.f};
                            mma(zi, gkc[kqi][hh][0], ones);
                            mma(zi, gkc[kqi][hh][1], ones);
                            const int zo = ((2 * (kq0 + kqi) + hh) * 16 + lg * 4) * 4;
                            const f32x4 z = lds_ld<f32x4>(LZ + zo) + zi;
                            if (lr == 0) lds_st<f32x4>(LZ + zo, z);
                        }
                    }
            }
            if constexpr (PIPE) {
                // own X rows of the next chunk: after them only its V (and Gamma_K) blocks and this
                // chunk's stores were issued.  Done after the last chunk too (the reads then see
                // stale LDS and are never used): an unconditional update keeps the carried
                // registers dead through the chunk.
                if (pair_st) wait_vmcnt<NVD + NGD + NSTP>();
                else wait_vmcnt<NVD + NGD + NST>();
                prefetch_x(LX + (BUF ^ 1) * XBUF + w * XWAVE);
            }
        }
    };

    if constexpr (REV) {
        for (int64_t ch = ch1 - 1; ch >= ch0; ch -= 2) {
            body(std::integral_constant<int, 0>{}, ch);
            if (ch - 1 >= ch0) body(std::integral_constant<int, 1>{}, ch - 1);
        }
    } else {
        for (int64_t ch = ch0; ch < ch1; ch += 2) {
            body(std::integral_constant<int, 0>{}, ch);
            if (ch + 1 < ch1) body(std::integral_constant<int, 1>{}, ch + 1);
        }
    }
    if (nonfin && a.flags) a.flags[bh] = 1;

    if constexpr (AGG) {
#pragma unroll
        for (int kqi = 0; kqi < KQW; ++kqi)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int ct = 2 * (kq0 + kqi) + hh;
#pragma unroll
                for (int vti = 0; vti < VTW; ++vti)
                    *reinterpret_cast<f32x4*>(segrec + ((int64_t)(ct * NVT + vt0 + vti) * 64 + lane) * 4) = st[kqi][hh][vti];
            }
        if (zown && lr == 0) {
#pragma unroll
            for (int kqi = 0; kqi < KQW; ++kqi)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
                    *reinterpret_cast<f32x4*>(segrec + (int64_t)KC * VC + (2 * (kq0 + kqi) + hh) * 16 + lg * 4) = zst[kqi][hh];
        }
    }
}

}  // namespace gma
