// Exact recomputation of the (batch, head) slices whose bf16 logits left the fp16 operand range
// (launchers of gma_fixup.hip, driven by the host library).
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace gma {

struct FixArgs {
    const int* flags;       // [BH]: nonzero where a bf16 kernel met a row with non-finite logits
    const void* qx;         // [BH, N, d_r] bf16 (the rows of gamma for the responsibilities)
    const void* kx;         // [BH, N, d_r] bf16
    const void* v;          // [BH, N, d_v] bf16
    void* o;                // [BH, N, d_v] bf16
    float* gamma;           // [BH, N, K] fp32 (responsibilities)
    const float* mu;        // [H, K, d_r]
    const float* raw_var;   // [H, K, d_r]
    const float* prior;     // [H, K]
    float* scratch;         // fixup_scratch_bytes(H, K, d_r): per head, mu and 1 / sigma^2 as [d_r][K]
    const float* rec_in;    // causal, or null: the memory before the first token as the forward's state
                            // records [BH, KC VC + KC] (the copy the forward made of state_in)
    float* state_out;       // [BH, K, d_v + 1] or null (causal: the memory after the last token)
    float* stat_usage;      // diagnostics: per-segment partials [BH, stat_segs, K] (usage, then counts);
    uint32_t* stat_count;   //   a flagged slice gets its totals in segment 0 and zeros elsewhere
    int stat_segs;
    int64_t BH;             // (batch, head) slices
    int64_t N;              // rows of qx / o (and of kx / v when causal)
    int64_t N_kv;           // rows of kx / v
    int H, K, d_r, d_v;
    float eps;
};

size_t fixup_scratch_bytes(int H, int K, int d_r);
// kc, vc: the padded K and d_v of the bf16 class that ran the call (its LDS sizes); false if none
bool launch_fixup_forward(const FixArgs& a, int kc, int vc, int64_t BH, bool causal, hipStream_t s);
bool launch_fixup_resp(const FixArgs& a, int kc, int64_t BH, hipStream_t s);
bool launch_fixup_stats(const FixArgs& a, int kc, int64_t BH, hipStream_t s);

}  // namespace gma
