// Registry of compiled kernel shape classes (host side, shared by the host library and the
// per-dtype instantiation units).
#pragma once
#include <hip/hip_runtime.h>
#include "gma_kernels.hpp"

namespace gma {

using prep_launch_t = void (*)(const PrepArgs&, int heads, hipStream_t);
using main_launch_t = void (*)(const MainArgs&, int grid, hipStream_t);

// One compiled shape class: padded components KC, padded d_v VC, padded d_r DRC,
// W wavefronts per workgroup, C tokens per chunk.
struct ShapeClass {
    int f32, kc, vc, drc, w, c;
    int wg_per_cu;   // workgroups per compute unit the LDS and register budgets allow
    prep_launch_t prep;
    main_launch_t resp, agg, out_bidir, out_causal;              // register-staged inputs
    main_launch_t dma_resp, dma_agg, dma_out_bidir, dma_out_causal;  // LDS-DMA staged (bf16 only)
};

const ShapeClass* classes_f32(int* count);
const ShapeClass* classes_bf16(int* count);

template <bool F32, int KC, int DRC>
void launch_prep(const PrepArgs& p, int heads, hipStream_t s) {
    hipLaunchKernelGGL((prep_kernel<F32, KC, DRC>), dim3(heads, KC / 16), dim3(256), 0, s, p);
}

// WPE: wavefronts per SIMD the register allocation must allow (2 lets two workgroups share a CU).
template <bool F32, int KC, int VC, int DRC, int W, int C, int MODE, bool DMA, int WPE>
void launch_main(const MainArgs& a, int grid, hipStream_t s) {
    hipLaunchKernelGGL((main_kernel<F32, KC, VC, DRC, W, C, MODE, DMA, WPE>), dim3(grid), dim3(W * 64), 0, s, a);
}

#define GMA_MAIN_SET(F32, KC, VC, DRC, W, C, DMA, WPE)                                        \
    &launch_main<F32, KC, 16 * W, DRC, W, C, MODE_RESP, DMA, WPE>,                            \
        &launch_main<F32, KC, VC, DRC, W, C, MODE_AGG, DMA, WPE>,                             \
        &launch_main<F32, KC, VC, DRC, W, C, MODE_OUT_BIDIR, DMA, WPE>,                       \
        &launch_main<F32, KC, VC, DRC, W, C, MODE_OUT_CAUSAL, DMA, WPE>

#define GMA_SHAPE_CLASS_F32(KC, VC, DRC, W, C)                                                \
    ShapeClass {                                                                              \
        1, KC, VC, DRC, W, C, 1, &launch_prep<true, KC, DRC>, GMA_MAIN_SET(true, KC, VC, DRC, W, C, false, 1), \
            nullptr, nullptr, nullptr, nullptr                                                \
    }

#define GMA_SHAPE_CLASS_BF16(KC, VC, DRC, W, C, WPE)                                          \
    ShapeClass {                                                                              \
        0, KC, VC, DRC, W, C, WPE, &launch_prep<false, KC, DRC>,                              \
            GMA_MAIN_SET(false, KC, VC, DRC, W, C, false, 1), GMA_MAIN_SET(false, KC, VC, DRC, W, C, true, WPE) \
    }

}  // namespace gma
