// Host interface of the bf16 MFMA Gram (see gram.hip).
#pragma once

#include "gptq_common.hpp"

namespace gptq {

struct GramArgs {
    const uint16_t* X = nullptr; int64_t ldx = 0;     // bf16 bits, M x K
    const uint16_t* Xf = nullptr; int64_t ldxf = 0;   // float stream (cross term), or null
    const uint16_t* XA = nullptr; int64_t ldxa = 0;   // staged A-side operand of the fast path, or null
    const float* rho = nullptr;                       // per-token weight (group Hessians), or null
    int64_t M = 0, K = 0;
    int nb = 0, ntiles = 0, splits = 1;
    int64_t tokens_per_split = 0;
    float* partial = nullptr;
    bool vec = false;
};

struct GramPlan {
    bool cross = false;          // plan for the cross term (all tiles) or the symmetric Gram (upper tiles)
    int nb = 0;                  // 256-column blocks
    int ntiles = 0;              // upper-triangular (or all, for the cross term) 256 x 256 tiles
    int splits = 1;              // token splits
    int64_t tokens_per_split = 0;
    size_t partial_floats = 0;   // scratch for the split partials
};

GramPlan gram_plan(int64_t K, int64_t M, bool cross);

// bf16 elements of scratch the fast path needs to stage a transformed operand (0 if it is not used).
size_t gram_staging_elems(int64_t K, int64_t M, bool transformed);

// Out += 2 * Xs^T Xs (symmetric, both triangles), or Out += 2 * bf16(Xf - X)^T X when Xf is given.
// `staging` (gram_staging_elems elements, or null) enables the fast path for the transformed operands.
hipError_t gram_bf16(const GramPlan& pl, const uint16_t* X, int64_t ldx, const uint16_t* Xf, int64_t ldxf,
                     const float* rho, int64_t M, int64_t K, float* partial, uint16_t* staging, float* Out,
                     hipStream_t stream);

}  // namespace gptq
