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
    prep_launch_t prep;
    main_launch_t resp, agg, out_bidir, out_causal;
};

const ShapeClass* classes_f32(int* count);
const ShapeClass* classes_bf16(int* count);

template <bool F32, int KC, int DRC>
void launch_prep(const PrepArgs& p, int heads, hipStream_t s) {
    hipLaunchKernelGGL((prep_kernel<F32, KC, DRC>), dim3(heads), dim3(256), 0, s, p);
}

template <bool F32, int KC, int VC, int DRC, int W, int C, int MODE>
void launch_main(const MainArgs& a, int grid, hipStream_t s) {
    hipLaunchKernelGGL((main_kernel<F32, KC, VC, DRC, W, C, MODE>), dim3(grid), dim3(W * 64), 0, s, a);
}

#define GMA_SHAPE_CLASS(F32, KC, VC, DRC, W, C)                                               \
    ShapeClass {                                                                              \
        F32, KC, VC, DRC, W, C, &launch_prep<F32, KC, DRC>,                                   \
            &launch_main<F32, KC, 16 * W, DRC, W, C, MODE_RESP>,                              \
            &launch_main<F32, KC, VC, DRC, W, C, MODE_AGG>,                                   \
            &launch_main<F32, KC, VC, DRC, W, C, MODE_OUT_BIDIR>,                             \
            &launch_main<F32, KC, VC, DRC, W, C, MODE_OUT_CAUSAL>                             \
    }

}  // namespace gma
