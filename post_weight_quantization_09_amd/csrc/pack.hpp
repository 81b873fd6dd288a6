// Host interface of code packing (see pack.hip).
#pragma once

#include "gptq_common.hpp"

namespace gptq {

int64_t packed_words(int64_t K, int bits);

hipError_t pack_codes(const uint8_t* codes, int64_t c_rs, int64_t c_cs, int64_t K, int64_t N, int bits,
                      uint32_t* packed, int64_t ldp, hipStream_t stream);

hipError_t unpack_codes(const uint32_t* packed, int64_t ldp, int64_t K, int64_t N, int bits, const float* scales,
                        uint8_t* codes, int64_t c_rs, int64_t c_cs, void* W_hat, bool bf16, int64_t w_rs,
                        int64_t w_cs, hipStream_t stream);

}  // namespace gptq
