// Device-side building blocks for the GMA kernels on gfx950 (CDNA4).
//
// Fragment conventions (one 64-lane wavefront; lane = 16*g + r, r = lane % 16, g = lane / 16):
//   * 16x16 accumulator tile D (f32x4 per lane): lane holds D[4*g + i][r] for i = 0..3.
//   * bf16/fp16 operands of v_mfma_f32_16x16x32_{bf16,f16}: A lane holds A[r][8*g + j],
//     B lane holds B[8*g + j][r], j = 0..7 (16 bytes per lane).
//   * fp32 operands: one "fragment step" is four v_mfma_f32_16x16x4_f32; A lane holds
//     A[r][4*g + j], B lane holds B[4*g + j][r], j = 0..3, and MFMA j consumes element j.
// A contraction index may be permuted freely as long as both operands use the same
// permutation; the kernels use that to feed accumulator tiles straight back into the
// matrix cores without moving data between lanes (see the "pair" helpers below).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gma {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void mma(f32x4& c, const f16x8& a, const f16x8& b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& c, const bf16x8& a, const bf16x8& b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& c, const f32x4& a, const f32x4& b) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round-to-nearest-even fp32 -> bf16 (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ __bf16 to_bf16(float x) { return (__bf16)x; }

__device__ __forceinline__ uint16_t bf16_bits(float x) {
    __bf16 b = (__bf16)x;
    return __builtin_bit_cast(uint16_t, b);
}

// Two accumulator tiles -> one bf16 operand fragment whose contraction slots are
// (tile lo rows 4g..4g+3, tile hi rows 4g..4g+3).
__device__ __forceinline__ bf16x8 pack_pair(const f32x4& lo, const f32x4& hi) {
    bf16x8 r;
    r[0] = to_bf16(lo[0]); r[1] = to_bf16(lo[1]); r[2] = to_bf16(lo[2]); r[3] = to_bf16(lo[3]);
    r[4] = to_bf16(hi[0]); r[5] = to_bf16(hi[1]); r[6] = to_bf16(hi[2]); r[7] = to_bf16(hi[3]);
    return r;
}

__device__ __forceinline__ bf16x4 pack4(const f32x4& v) {
    bf16x4 r;
    r[0] = to_bf16(v[0]); r[1] = to_bf16(v[1]); r[2] = to_bf16(v[2]); r[3] = to_bf16(v[3]);
    return r;
}

__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

// Sum / max over the four lane groups g (lanes r, r+16, r+32, r+48).
__device__ __forceinline__ float group4_sum(float v) {
    v += shfl_xor(v, 16);
    v += shfl_xor(v, 32);
    return v;
}
__device__ __forceinline__ float group4_max(float v) {
    v = fmaxf(v, shfl_xor(v, 16));
    v = fmaxf(v, shfl_xor(v, 32));
    return v;
}
// Sum over the 16 lanes of one row group (lanes 16g .. 16g+15).
__device__ __forceinline__ float row16_sum(float v) {
    v += shfl_xor(v, 1);
    v += shfl_xor(v, 2);
    v += shfl_xor(v, 4);
    v += shfl_xor(v, 8);
    return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace gma
