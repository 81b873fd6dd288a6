// Host interface of act-order (see act_order.hip).
#pragma once

#include "gptq_common.hpp"

namespace gptq {

size_t act_order_workspace_bytes(int64_t K);

// perm (device int32[K]) = coordinates by descending diagonal of H (zero diagonal counted as 1, stable); H and,
// if not null, A are permuted in place to H[perm][:, perm].
hipError_t act_order(float* H, float* A, int64_t K, int32_t* perm, void* workspace, hipStream_t stream);

}  // namespace gptq
