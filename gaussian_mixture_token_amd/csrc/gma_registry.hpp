// Registry of compiled kernel shape classes (host side, shared by the host library and the
// per-dtype instantiation units).
#pragma once
#include <hip/hip_runtime.h>
#include "gma_kernels.hpp"
#include "gma_tok.hpp"

namespace gma {

using prep_launch_t = void (*)(const PrepArgs&, int heads, hipStream_t);
using main_launch_t = void (*)(const MainArgs&, int grid, hipStream_t);

// One compiled shape class: padded components KC, padded d_v VC, padded d_r DRC,
// W wavefronts per workgroup, C tokens per chunk.
struct ShapeClass {
    int f32, kc, vc, drc, w, c;
    int wg_per_cu;   // workgroups per compute unit the LDS and register budgets allow
    prep_launch_t prep;
    main_launch_t resp, agg, out_bidir, out_causal;   // main_kernel, register-staged inputs
    main_launch_t dma_resp;                           // main_kernel, LDS-DMA staged (bf16 only)
    // token-split kernels (bf16, LDS-DMA staged, 4 wavefronts, chunks of 64 tokens); null where the
    // class has none
    int tok_wg_per_cu;
    main_launch_t tok_agg, tok_out_bidir, tok_out_causal;
    // causal pair through stored Gamma_K tiles: aggregate pass that also writes the tiles, output
    // pass that reads them
    main_launch_t tok_agg_g, tok_out_causal_g;
};

constexpr int kTokChunk = 64;

const ShapeClass* classes_f32(int* count);
const ShapeClass* classes_bf16(int* count);

template <bool F32, int KC, int DRC>
void launch_prep(const PrepArgs& p, int heads, hipStream_t s) {
    hipLaunchKernelGGL((prep_kernel<F32, KC, DRC>), dim3(heads, KC / kPrepComps<DRC>), dim3(kPrepThreads), 0, s, p);
}

// WPE: wavefronts per SIMD the register allocation must allow (2 lets two workgroups share a CU).
template <bool F32, int KC, int VC, int DRC, int W, int C, int MODE, bool DMA, int WPE>
void launch_main(const MainArgs& a, int grid, hipStream_t s) {
    hipLaunchKernelGGL((main_kernel<F32, KC, VC, DRC, W, C, MODE, DMA, WPE>), dim3(grid), dim3(W * 64), 0, s, a);
}

template <int KC, int VC, int DRC, int MODE, int WPE>
void launch_tok(const MainArgs& a, int grid, hipStream_t s) {
    hipLaunchKernelGGL((tok_kernel<KC, VC, DRC, MODE, WPE>), dim3(grid), dim3(256), 0, s, a);
}

#define GMA_MAIN_SET(F32, KC, VC, DRC, W, C, DMA, WPE)                                        \
    &launch_main<F32, KC, 16 * W, DRC, W, C, MODE_RESP, DMA, WPE>,                            \
        &launch_main<F32, KC, VC, DRC, W, C, MODE_AGG, DMA, WPE>,                             \
        &launch_main<F32, KC, VC, DRC, W, C, MODE_OUT_BIDIR, DMA, WPE>,                       \
        &launch_main<F32, KC, VC, DRC, W, C, MODE_OUT_CAUSAL, DMA, WPE>

// WPC: workgroups per compute unit the segment split aims at (the aggregate pass's occupancy)
#define GMA_SHAPE_CLASS_F32(KC, VC, DRC, W, C, WPC)                                           \
    ShapeClass {                                                                              \
        1, KC, VC, DRC, W, C, WPC, &launch_prep<true, KC, DRC>, GMA_MAIN_SET(true, KC, VC, DRC, W, C, false, 1), \
            nullptr, 0, nullptr, nullptr, nullptr, nullptr, nullptr                           \
    }

// WPE: wavefronts per SIMD of the LDS-DMA responsibilities kernel; TWPE: of the token-split kernels
#define GMA_SHAPE_CLASS_BF16(KC, VC, DRC, W, C, WPE, TWPE)                                    \
    ShapeClass {                                                                              \
        0, KC, VC, DRC, W, C, WPE, &launch_prep<false, KC, DRC>,                              \
            GMA_MAIN_SET(false, KC, VC, DRC, W, C, false, 1),                                 \
            &launch_main<false, KC, 16 * W, DRC, W, C, MODE_RESP, true, WPE>, TWPE,           \
            &launch_tok<KC, VC, DRC, MODE_AGG, TWPE>, &launch_tok<KC, VC, DRC, MODE_OUT_BIDIR, TWPE>, \
            &launch_tok<KC, VC, DRC, MODE_OUT_CAUSAL, TWPE>,                                  \
            &launch_tok<KC, VC, DRC, MODE_AGG_G, TWPE>, &launch_tok<KC, VC, DRC, MODE_OUT_CAUSAL_G, TWPE> \
    }

// the same without token-split kernels
#define GMA_SHAPE_CLASS_BF16_NOTOK(KC, VC, DRC, W, C, WPE)                                    \
    ShapeClass {                                                                              \
        0, KC, VC, DRC, W, C, WPE, &launch_prep<false, KC, DRC>,                              \
            GMA_MAIN_SET(false, KC, VC, DRC, W, C, false, 1),                                 \
            &launch_main<false, KC, 16 * W, DRC, W, C, MODE_RESP, true, WPE>, 0, nullptr, nullptr, nullptr, \
            nullptr, nullptr                                                                  \
    }

}  // namespace gma
