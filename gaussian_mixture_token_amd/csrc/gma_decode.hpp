// One-token causal decode step: launcher shared by the host library and gma_decode.hip.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace gma {

struct DecodeArgs {
    const void* qx;            // [BH, d_r] (bf16 bits or fp32): the new token's query row
    const void* kx;            // [BH, d_r]: its key row
    const void* v;             // [BH, d_v]: its value row
    void* o;                   // [BH, d_v]: its output row
    const float* mu;           // [H, K, d_r]
    const float* raw_var;      // [H, K, d_r]
    const float* prior;        // [H, K]
    const float* state_in;     // [BH, K, d_v + 1] or null (zero state)
    float* state_out;          // [BH, K, d_v + 1] or null (not written); may equal state_in
    int H, K, d_r, d_v;
    float eps;
    // prepared mixture (gma_decode_prepare) or null: then raw_var and prior are not read
    const float* inv_var;      // [H, K, d_r]: 1 / softplus(raw_var), fp32
    const double* cconst;      // [H, K]: log pi_k - 1/2 sum_d log sigma^2_kd, fp64
};

struct DecodePrepArgs {
    const float* raw_var;      // [H, K, d_r]
    const float* prior;        // [H, K]
    float* inv_var;            // [H, K, d_r]
    double* cconst;            // [H, K]
    int K, d_r;
};

// grid: one workgroup of 1024 threads per head
void launch_decode_prepare(const DecodePrepArgs& a, int heads, hipStream_t s);

// grid: one workgroup of 1024 threads per (batch, head)
void launch_decode(const DecodeArgs& a, int64_t bh, bool f32, hipStream_t s);

}  // namespace gma
