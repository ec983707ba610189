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

// Keeps an MFMA operand in accumulation registers (AGPRs): with one wavefront per SIMD a wave has
// 256 VGPRs and 256 AGPRs, and matrix-core operands may be read from either file.
template <class T>
__device__ __forceinline__ void pin_agpr(T& v) {
    asm volatile("" : "+a"(v));
}

// Scheduling hints for one scheduling region (the code since the last sched_barrier): interleave
// N matrix-core instructions with V vector-ALU instructions after each, so that the ALU work
// issues while the matrix cores are busy.  fence() ends a region.
template <int N, int V>
__device__ __forceinline__ void interleave_mfma_valu() {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, V, 0);
    }
}
__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

// Makes v opaque to the optimiser at this point, so that values computed from it inside a loop are
// recomputed there instead of being hoisted out and held in registers across the loop.
template <class T>
__device__ __forceinline__ T opaque_v(T v) {
    asm volatile("" : "+v"(v));
    return v;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round-to-nearest-even fp32 -> bf16 (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ __bf16 to_bf16(float x) { return (__bf16)x; }

__device__ __forceinline__ uint16_t bf16_bits(float x) {
    __bf16 b = (__bf16)x;
    return __builtin_bit_cast(uint16_t, b);
}

// Two fp32 values rounded to bf16 (nearest even), packed: a in the low half, b in the high half.
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 t = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, t);
}

// x rounded to the nearest bf16 value, returned as fp32
__device__ __forceinline__ float round_bf16(float x) { return __uint_as_float((uint32_t)bf16_bits(x) << 16); }

// Two accumulator tiles -> one bf16 operand fragment whose contraction slots are
// (tile lo rows 4g..4g+3, tile hi rows 4g..4g+3).
__device__ __forceinline__ bf16x8 pack_pair(const f32x4& lo, const f32x4& hi) {
    bf16x8 r;
    r[0] = to_bf16(lo[0]); r[1] = to_bf16(lo[1]); r[2] = to_bf16(lo[2]); r[3] = to_bf16(lo[3]);
    r[4] = to_bf16(hi[0]); r[5] = to_bf16(hi[1]); r[6] = to_bf16(hi[2]); r[7] = to_bf16(hi[3]);
    return r;
}

template <class F> __device__ __forceinline__ F ones_frag();
template <> __device__ __forceinline__ f32x4 ones_frag<f32x4>() { return f32x4{1.f, 1.f, 1.f, 1.f}; }
template <> __device__ __forceinline__ bf16x8 ones_frag<bf16x8>() {
    const __bf16 o = (__bf16)1.0f;
    return bf16x8{o, o, o, o, o, o, o, o};
}

__device__ __forceinline__ bf16x4 pack4(const f32x4& v) {
    bf16x4 r;
    r[0] = to_bf16(v[0]); r[1] = to_bf16(v[1]); r[2] = to_bf16(v[2]); r[3] = to_bf16(v[3]);
    return r;
}

__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

// Sum / max over the four 16-lane rows (lanes r, r+16, r+32, r+48), in VALU: with both operands
// equal, v_permlane16_swap returns rows (0,0,2,2) and (1,1,3,3) and v_permlane32_swap returns rows
// (0,1,0,1) and (2,3,2,3).
__device__ __forceinline__ float group4_sum(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float group4_max(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
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
// v_rcp_f32 (about 1 ulp)
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// ---- bf16 -> fp16 (8 values).  Exact for every bf16 value whose magnitude lies in the fp16
// normal range: bf16 carries 8 significant bits, fp16 11, so the round-toward-zero pack
// conversion never rounds there.
__device__ __forceinline__ f16x8 bf16x8_bits_to_f16x8(const u32x4& r) {
    f16x8 h;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const auto p = __builtin_amdgcn_cvt_pkrtz(__uint_as_float(r[e] << 16), __uint_as_float(r[e] & 0xffff0000u));
        h[2 * e] = p[0];
        h[2 * e + 1] = p[1];
    }
    return h;
}

// ---- buffer descriptors, LDS DMA, transposed LDS reads, bounds-checked stores
typedef short i16x4 __attribute__((ext_vector_type(4)));
#define GMA_LDS(p) ((__attribute__((address_space(3))) void*)(p))

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor over [base, base + bytes): loads past the end return 0, stores are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// The same descriptor as four scalar dwords (base, stride 0, byte count, gfx9 format word), for
// the inline-assembly DMA below.
__device__ __forceinline__ i32x4 make_rsrc_words(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = 0x00020000;
    return r;
}

// 16 bytes per lane from global (base + soff + voff) into LDS at lds + 16 * lane (1 KiB per
// wave): buffer_load_dwordx4 ... lds.  Issued from inline assembly so that the compiler does not
// track the LDS write: the kernels wait for it explicitly (wait_vmcnt + barrier) before reading
// the buffer, and an implicit wait would otherwise serialise the prefetch with the compute of
// the current chunk.  M0 (the LDS destination) is saved and restored around the load; an SALU
// write of M0 needs one wait state before an LDS-DMA load reads it (s_nop 0).
__device__ __forceinline__ void dma16(const i32x4& rs, char* lds, uint32_t voff, uint32_t soff) {
    const uint32_t dst = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)GMA_LDS(lds)));
    i32x4 srs;
    srs[0] = __builtin_amdgcn_readfirstlane(rs[0]);
    srs[1] = __builtin_amdgcn_readfirstlane(rs[1]);
    srs[2] = __builtin_amdgcn_readfirstlane(rs[2]);
    srs[3] = __builtin_amdgcn_readfirstlane(rs[3]);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(dst), "v"(voff), "s"(srs), "s"(__builtin_amdgcn_readfirstlane(soff))
        : "memory");
}

// LDS (address space 3) byte pointers and their 32-bit addresses.
typedef __attribute__((address_space(3))) char lds_char;
__device__ __forceinline__ uint32_t lds_addr(const lds_char* p) { return (uint32_t)(uintptr_t)p; }

// Four LDS-DMA loads of 16 bytes per lane: global (rsrc, voff[i]) -> LDS at m0[i] + 16 * lane.
// rs and the LDS addresses must be wave-uniform (SGPRs).  One M0 save / restore for the four.
__device__ __forceinline__ void dma16x4(const i32x4& rs, uint32_t m0a, uint32_t m0b, uint32_t m0c, uint32_t m0d,
                                        uint32_t va, uint32_t vb, uint32_t vc, uint32_t vd) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %5, %9, 0 offen lds\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %6, %9, 0 offen lds\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %7, %9, 0 offen lds\n\t"
        "s_mov_b32 m0, %4\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %8, %9, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(m0a), "s"(m0b), "s"(m0c), "s"(m0d), "v"(va), "v"(vb), "v"(vc), "v"(vd), "s"(rs)
        : "memory");
}
__device__ __forceinline__ void dma16x1(const i32x4& rs, uint32_t m0a, uint32_t va) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(m0a), "v"(va), "s"(rs)
        : "memory");
}
__device__ __forceinline__ void dma16x2(const i32x4& rs, uint32_t m0a, uint32_t m0b, uint32_t va, uint32_t vb) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %3, %5, 0 offen lds\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %4, %5, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(m0a), "s"(m0b), "v"(va), "v"(vb), "s"(rs)
        : "memory");
}

// Uniform (SGPR) copy of a buffer descriptor.
__device__ __forceinline__ i32x4 uniform_rsrc(const i32x4& rs) {
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane(rs[0]);
    r[1] = __builtin_amdgcn_readfirstlane(rs[1]);
    r[2] = __builtin_amdgcn_readfirstlane(rs[2]);
    r[3] = __builtin_amdgcn_readfirstlane(rs[3]);
    return r;
}

// Typed accesses through LDS (address space 3) pointers.
template <class T>
__device__ __forceinline__ T lds_ld(const lds_char* p) {
    return *reinterpret_cast<const __attribute__((address_space(3))) T*>(p);
}
template <class T>
__device__ __forceinline__ void lds_st(lds_char* p, const T& v) {
    *reinterpret_cast<__attribute__((address_space(3))) T*>(p) = v;
}
__device__ __forceinline__ u32x2 ds_read_tr16_at(const lds_char* p) {
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<__attribute__((address_space(3))) i16x4*>(const_cast<lds_char*>(p)));
    return __builtin_bit_cast(u32x2, v);
}

// ds_read_b64_tr_b16: within each 16-lane group, lane r receives element (r % 4) of the 8-byte
// rows addressed by lanes 4i + r/4 of its group, i = 0..3 (a 4 x 16 transpose).
__device__ __forceinline__ u32x2 ds_read_tr16(const char* lds) {
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(GMA_LDS(lds)));
    return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ void store_b64(__amdgpu_buffer_rsrc_t rs, u32x2 v, uint32_t voff) {
    __builtin_amdgcn_raw_buffer_store_b64(v, rs, voff, 0, 0);
}

// ---- explicit waits and barriers.  A plain __syncthreads() would also wait for the LDS DMA
// prefetch in flight; these wait only for what they name.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]; lgkmcnt 0
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | (((N >> 4) & 3) << 14));
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ void block_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// LDS writes of this wave complete, then barrier.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
    block_barrier();
}

}  // namespace gma
