// Host interface of the Hadamard row rotation (see hadamard.hip).
#pragma once

#include "gptq_common.hpp"

namespace gptq {

// Rows of length K = 2^n (4 <= n <= 14): out = (in * signs) H_K / sqrt(K); in == out allowed (same ld).
hipError_t hadamard_rows(const void* in, int64_t ld_in, void* out, int64_t ld_out, bool bf16, int64_t rows, int n,
                         const int8_t* signs, hipStream_t stream);

}  // namespace gptq
