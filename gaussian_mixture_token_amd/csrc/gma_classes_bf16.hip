// Compiled shape classes for bf16 storage (fp16 logits operands, bf16 contraction operands).
// Columns: padded K, padded d_v, padded d_r, wavefronts per workgroup and tokens per chunk of the
// register-staged kernels, wavefronts per SIMD of the LDS-DMA responsibilities kernel and of the
// token-split kernels.
#include "gma_registry.hpp"

namespace gma {

static const ShapeClass kClassesBf16[] = {
    GMA_SHAPE_CLASS_BF16(32, 64, 64, 2, 32, 2, 2),
    GMA_SHAPE_CLASS_BF16(128, 128, 128, 4, 32, 2, 1),
    GMA_SHAPE_CLASS_BF16(256, 64, 64, 4, 32, 1, 1),
    GMA_SHAPE_CLASS_BF16_NOTOK(256, 128, 128, 4, 32, 1),
};

const ShapeClass* classes_bf16(int* count) {
    *count = (int)(sizeof(kClassesBf16) / sizeof(kClassesBf16[0]));
    return kClassesBf16;
}

}  // namespace gma
