// Compiled shape classes for fp32 storage and arithmetic.
// Columns: padded K, padded d_v, padded d_r, wavefronts per workgroup, tokens per chunk, workgroups per
// compute unit that the segment split aims at.  The last is the aggregate pass's occupancy (the output
// passes hold fewer and take the segments in more than one round).  Measured on MI355X (forward, B4 H8
// N4096): d = K = 16, whose workgroups are single waves, 125 -> 48 us causal and 70 -> 28 us bidirectional
// at 8 (B32: 629 -> 259 and 570 -> 109 us) against 1; d = K = 64 240 -> 221 us causal and 139 -> 104 us
// bidirectional at 2 (4 and 8 slower); at K = 128 every pass holds one workgroup per unit.
#include "gma_registry.hpp"

namespace gma {

static const ShapeClass kClassesF32[] = {
    GMA_SHAPE_CLASS_F32(16, 16, 16, 1, 64, 8),
    GMA_SHAPE_CLASS_F32(64, 64, 64, 4, 64, 2),
    GMA_SHAPE_CLASS_F32(128, 128, 128, 4, 32, 1),
};

const ShapeClass* classes_f32(int* count) {
    *count = (int)(sizeof(kClassesF32) / sizeof(kClassesF32[0]));
    return kClassesF32;
}

}  // namespace gma
