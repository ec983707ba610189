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
};

// grid: one workgroup of 1024 threads per (batch, head)
void launch_decode(const DecodeArgs& a, int64_t bh, bool f32, hipStream_t s);

}  // namespace gma
