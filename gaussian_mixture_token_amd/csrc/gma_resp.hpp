// Token-split responsibilities kernel (bf16 storage): launchers shared by the host library and
// gma_resp.hip.
#pragma once
#include <hip/hip_runtime.h>

#include "gma_kernels.hpp"

namespace gma {

// A compiled instantiation exists for this (padded K, padded d_r)
bool resp_tok_supported(int kc, int drc);

// Gamma of every row of a.qx [BH, N, d_r] (bf16, rows 16-byte aligned, d_r % 8 == 0) into a.gamma
// [BH, N, K] fp32, or, with a.stat_usage set, each segment's usage sums and hard-assignment counts
// [BH, a.Pg, K] (Gamma not written).  Grid: BH * a.Pg workgroups of 256 threads, segment s of a
// (batch, head) = rows s * rows_per_seg .. (s + 1) * rows_per_seg - 1 (rows_per_seg a multiple of 64).
// vec_gamma: K % 4 == 0 and a.gamma 16-byte aligned (16-byte row stores).  Sets a.flags[bh] for a
// (batch, head) with a row whose logits are not finite.  False if no instantiation serves (kc, drc).
bool launch_resp_tok(const MainArgs& a, int kc, int drc, int64_t rows_per_seg, bool vec_gamma, int grid,
                     hipStream_t s);

}  // namespace gma
