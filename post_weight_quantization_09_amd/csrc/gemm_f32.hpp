// Host interface of the fp32 MFMA GEMM (see gemm_f32.hip).
#pragma once

#include "gptq_common.hpp"

namespace gptq {

// Structure of the operands, used to skip k-ranges and tiles that are known to be zero.
enum : unsigned {
    kGemmAUpper = 1u << 0,            // A(m,k) == 0 for k < m (stored zeros)
    kGemmAStrictUpperMask = 1u << 1,  // treat A(m,k) as 0 for k <= m (applied when loading)
    kGemmBUpper = 1u << 2,            // B(k,n) == 0 for k > n (stored zeros)
    kGemmBLower = 1u << 3,            // B(k,n) == 0 for k < n (stored zeros)
    kGemmCUpper = 1u << 4,            // only tiles touching the upper triangle (m <= n) are computed
};

// C (M x N, ldc) = beta * C + alpha * (A1 B1 + a2_scale * A2 B2).
//   A(m,k) = transA ? A[k*lda + m] : A[m*lda + k];  B(k,n) = transB ? B[n*ldb + k] : B[k*ldb + n].
//   Pair 2 is optional (A2 == nullptr); structure flags apply to pair 1 only.
//   Batched: operand pointers advance by their stride per batch index.
struct GemmArgs {
    int64_t M = 0, N = 0, K1 = 0, K2 = 0;
    const float* A1 = nullptr; int64_t lda1 = 0;
    const float* B1 = nullptr; int64_t ldb1 = 0;
    const float* A2 = nullptr; int64_t lda2 = 0;
    const float* B2 = nullptr; int64_t ldb2 = 0;
    float* C = nullptr; int64_t ldc = 0;
    float alpha = 1.f, beta = 0.f, a2_scale = 1.f;
    int64_t strideA1 = 0, strideB1 = 0, strideA2 = 0, strideB2 = 0, strideC = 0;
    unsigned flags = 0;
    bool transA = false, transB = false;
    // set by gemm_f32()
    bool vecA1 = false, vecB1 = false, vecA2 = false, vecB2 = false;
};

hipError_t gemm_f32(GemmArgs p, int64_t batch, hipStream_t stream);

// Two independent products, each exactly as gemm_f32 computes it: one launch when both run on the 64 x 64 fp32
// kernel with B transposed in `a` only (the recursion's SYRK and its X = R12 U22), otherwise two launches.
hipError_t gemm_f32_pair(GemmArgs a, GemmArgs b, int64_t batch, hipStream_t stream);

}  // namespace gptq
