// Host interface of the Hessian preparation (see factor.hip).
#pragma once

#include "gptq_common.hpp"

namespace gptq {

size_t prepare_workspace_bytes(int64_t K, int64_t batch = 1);

// In place on `batch` Hessians H + b strideH: H -> U (upper, H_d^{-1} = U^T U, strictly lower part zero);
// writes dead[b K .. b K + K); with damp_out or n_dead_out (host, nullable) given it synchronises, fills them and
// returns the device-side status, else it returns after enqueueing.  The status words of the batch are the first
// `batch` 256-byte headers of the workspace; the first also collects every Hessian's error bits.
gptq_status_t prepare(float* H, int64_t K, int64_t batch, int64_t strideH, float percdamp, uint8_t* dead,
                      float* damp_out, int64_t* n_dead_out, void* workspace, hipStream_t stream);

}  // namespace gptq
