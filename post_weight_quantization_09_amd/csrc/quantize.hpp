// Host interface of the column loop (see quantize.hip).
#pragma once

#include "gptq_common.hpp"

namespace gptq {

struct QuantizeArgs {
    const void* W = nullptr; gptq_dtype_t w_dtype = GPTQ_DTYPE_F32;
    int64_t K = 0, N = 0, w_rs = 0, w_cs = 0;
    const float* U = nullptr; const uint8_t* dead = nullptr; const float* P1 = nullptr;
    int bits = 4;
    bool scales_given = false;
    bool cae = false;               // compensation-aware error term (P2 = P1 + I - diag(U)^-1 U)
    const int32_t* perm = nullptr;  // act-order: processing position j handles original row perm[j]
    int64_t groupsize = 0;          // 0: one scale per channel; 32, 64, 128: group-wise scales
    bool static_groups = false;     // group scales from W before the loop (groups of original rows)
    bool mse = false;               // weight-MSE clipping of the scales taken from W before the loop
    int32_t* g_idx = nullptr;       // optional output: group of each original row
    int64_t groups = 1;             // output-channel groups: channel n uses U, P1, dead, perm (and g_idx) of group
    int64_t u_stride = 0;           //   g = n / (N / groups); U, P1 of group g at + g u_stride, the rest at + g K
    uint8_t* codes = nullptr; int64_t c_rs = 0, c_cs = 0;
    float* scales = nullptr; void* W_hat = nullptr; float* losses = nullptr; float* pre_round = nullptr;
};

size_t quantize_workspace_bytes(int64_t K, int64_t N, bool asym, bool cae, int64_t groups = 1);

// Enqueues the whole loop on `stream`; rejected inputs latch kDevNonFinite in the workspace status word.
gptq_status_t quantize_layer(const QuantizeArgs& a, void* workspace, hipStream_t stream);

}  // namespace gptq
