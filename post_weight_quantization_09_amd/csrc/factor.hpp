// Host interface of the Hessian preparation (see factor.hip).
#pragma once

#include "gptq_common.hpp"

namespace gptq {

size_t prepare_workspace_bytes(int64_t K);

// In place H -> U (upper, H_d^{-1} = U^T U, strictly lower part zero); writes dead[K]; synchronises.
gptq_status_t prepare(float* H, int64_t K, float percdamp, uint8_t* dead, float* damp_out, int64_t* n_dead_out,
                      void* workspace, hipStream_t stream);

}  // namespace gptq
