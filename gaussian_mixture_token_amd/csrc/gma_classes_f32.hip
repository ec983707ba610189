// Compiled shape classes for fp32 storage and arithmetic.
// Columns: padded K, padded d_v, padded d_r, wavefronts per workgroup, tokens per chunk.
#include "gma_registry.hpp"

namespace gma {

static const ShapeClass kClassesF32[] = {
    GMA_SHAPE_CLASS_F32(16, 16, 16, 1, 64),
    GMA_SHAPE_CLASS_F32(64, 64, 64, 4, 64),
    GMA_SHAPE_CLASS_F32(128, 128, 128, 4, 32),
};

const ShapeClass* classes_f32(int* count) {
    *count = (int)(sizeof(kClassesF32) / sizeof(kClassesF32[0]));
    return kClassesF32;
}

}  // namespace gma
