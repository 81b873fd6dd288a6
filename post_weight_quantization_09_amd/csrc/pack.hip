// Code packing on gfx950: integer codes -> 32-bit words, and packed words -> codes and dequantised values.
//
// [T] section 9: the loop's results are grid values s (c - z); storing a quantised layer means the integer
// codes packed into a wider container together with the scale, zero point and layout.  Layout used here:
// each output channel's K codes form one little-endian bitstream, code k in stream bits [b k, b k + b), stored
// as 32-bit words along K (bit i of the stream is bit i % 32 of word i / 32).  For b = 3, 32 codes fill three
// words and one code in ten straddles a word boundary.
//
// Both kernels are HBM-bound elementwise passes: one thread per (word, channel) for packing and per (code,
// channel) for unpacking, channels fastest so that the uint8 codes, the words and the values are all read and
// written by consecutive lanes at consecutive addresses in the common K x N row-major layouts.  Where channels
// are contiguous and aligned, a thread takes four consecutive channels (4-byte code, 16-byte word and 8- or
// 16-byte value accesses instead of one element per lane and access).
#include "pack.hpp"

#include <algorithm>

namespace gptq {

namespace {

__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* codes, int64_t c_rs, int64_t c_cs, int64_t K,
                                                   int64_t N, int bits, uint32_t* packed, int64_t ldp, int64_t nw) {
    const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (n >= N) return;
    for (int64_t w = blockIdx.y; w < nw; w += gridDim.y) {
        const int64_t bit0 = 32 * w;                   // first stream bit of this word
        const int64_t k0 = bit0 / bits;                // first code overlapping the word
        const int64_t k1 = min<int64_t>(K, (bit0 + 32 + bits - 1) / bits);
        const uint32_t mask = (1u << bits) - 1u;
        uint32_t word = 0;
        for (int64_t k = k0; k < k1; ++k) {
            const uint32_t c = codes[k * c_rs + n * c_cs] & mask;
            const int64_t sh = k * bits - bit0;        // in (-bits, 32)
            if (sh >= 0) word |= c << sh;
            else word |= c >> (-sh);
        }
        packed[w * ldp + n] = word;
    }
}

// Four consecutive channels per thread: codes (K x N, channel stride 1, row stride and base 4-aligned) and
// packed words (ldp and base 16-byte aligned), N a multiple of 4.
__global__ __launch_bounds__(256) void pack4_kernel(const uint8_t* codes, int64_t c_rs, int64_t K, int64_t N,
                                                    int bits, uint32_t* packed, int64_t ldp, int64_t nw) {
    const int64_t n = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (n >= N) return;
    for (int64_t w = blockIdx.y; w < nw; w += gridDim.y) {
        const int64_t bit0 = 32 * w;
        const int64_t k0 = bit0 / bits;
        const int64_t k1 = min<int64_t>(K, (bit0 + 32 + bits - 1) / bits);
        const uint32_t mask = (1u << bits) - 1u;
        u32x4 word = {0u, 0u, 0u, 0u};
        for (int64_t k = k0; k < k1; ++k) {
            const uint32_t c4 = *reinterpret_cast<const uint32_t*>(codes + k * c_rs + n);
            const int64_t sh = k * bits - bit0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t c = (c4 >> (8 * j)) & mask;
                word[j] |= sh >= 0 ? c << sh : c >> (-sh);
            }
        }
        *reinterpret_cast<u32x4*>(packed + w * ldp + n) = word;
    }
}

// Four consecutive channels per thread (the alignment of pack4_kernel; W_hat with channel stride 1, its row
// stride and base aligned to the 4 values).
template <bool BF16>
__global__ __launch_bounds__(256) void unpack4_kernel(const uint32_t* packed, int64_t ldp, int64_t K, int64_t N,
                                                      int bits, const float* scales, uint8_t* codes, int64_t c_rs,
                                                      void* W_hat, int64_t w_rs) {
    const int64_t n = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (n >= N) return;
    const f32x4 s = W_hat ? *reinterpret_cast<const f32x4*>(scales + n) : f32x4{0.f, 0.f, 0.f, 0.f};
    const float z = (float)(1 << (bits - 1));
    const uint32_t mask = (1u << bits) - 1u;
    for (int64_t k = blockIdx.y; k < K; k += gridDim.y) {
        const int64_t bit = k * bits, w = bit >> 5;
        const int o = (int)(bit & 31);
        u32x4 v = *reinterpret_cast<const u32x4*>(packed + w * ldp + n);
        u32x4 c;
#pragma unroll
        for (int j = 0; j < 4; ++j) c[j] = v[j] >> o;
        if (o + bits > 32) {
            const u32x4 v2 = *reinterpret_cast<const u32x4*>(packed + (w + 1) * ldp + n);
#pragma unroll
            for (int j = 0; j < 4; ++j) c[j] |= v2[j] << (32 - o);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) c[j] &= mask;
        if (codes)
            *reinterpret_cast<uint32_t*>(codes + k * c_rs + n) = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
        if (W_hat) {
            f32x4 x;
#pragma unroll
            for (int j = 0; j < 4; ++j) x[j] = ((float)c[j] - z) * s[j];
            if (BF16) {
                u32x2 h;
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    h[j] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x[2 * j]) |
                           ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x[2 * j + 1]) << 16);
                *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(W_hat) + k * w_rs + n) = h;
            } else {
                *reinterpret_cast<f32x4*>(static_cast<float*>(W_hat) + k * w_rs + n) = x;
            }
        }
    }
}

template <bool BF16>
__global__ __launch_bounds__(256) void unpack_kernel(const uint32_t* packed, int64_t ldp, int64_t K, int64_t N,
                                                     int bits, const float* scales, uint8_t* codes, int64_t c_rs,
                                                     int64_t c_cs, void* W_hat, int64_t w_rs, int64_t w_cs) {
    const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (n >= N) return;
    for (int64_t k = blockIdx.y; k < K; k += gridDim.y) {
        const int64_t bit = k * bits, w = bit >> 5;
        const int o = (int)(bit & 31);
        uint32_t v = packed[w * ldp + n] >> o;
        if (o + bits > 32) v |= packed[(w + 1) * ldp + n] << (32 - o);
        const uint32_t c = v & ((1u << bits) - 1u);
        if (codes) codes[k * c_rs + n * c_cs] = (uint8_t)c;
        if (W_hat) {
            const float z = (float)(1 << (bits - 1));
            const float x = ((float)c - z) * scales[n];
            if (BF16) static_cast<__bf16*>(W_hat)[k * w_rs + n * w_cs] = (__bf16)x;
            else static_cast<float*>(W_hat)[k * w_rs + n * w_cs] = x;
        }
    }
}

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace

int64_t packed_words(int64_t K, int bits) { return (K * bits + 31) / 32; }

hipError_t pack_codes(const uint8_t* codes, int64_t c_rs, int64_t c_cs, int64_t K, int64_t N, int bits,
                      uint32_t* packed, int64_t ldp, hipStream_t stream) {
    const int64_t nw = packed_words(K, bits);
    if (c_cs == 1 && N % 4 == 0 && c_rs % 4 == 0 && ldp % 4 == 0 && aligned(codes, 4) && aligned(packed, 16)) {
        dim3 grid((unsigned)ceil_div(N / 4, 256), (unsigned)std::min<int64_t>(nw, 65535));
        hipLaunchKernelGGL(pack4_kernel, grid, dim3(256), 0, stream, codes, c_rs, K, N, bits, packed, ldp, nw);
        return hipGetLastError();
    }
    dim3 grid((unsigned)ceil_div(N, 256), (unsigned)std::min<int64_t>(nw, 65535));
    hipLaunchKernelGGL(pack_kernel, grid, dim3(256), 0, stream, codes, c_rs, c_cs, K, N, bits, packed, ldp, nw);
    return hipGetLastError();
}

hipError_t unpack_codes(const uint32_t* packed, int64_t ldp, int64_t K, int64_t N, int bits, const float* scales,
                        uint8_t* codes, int64_t c_rs, int64_t c_cs, void* W_hat, bool bf16, int64_t w_rs,
                        int64_t w_cs, hipStream_t stream) {
    const bool vec = N % 4 == 0 && ldp % 4 == 0 && aligned(packed, 16) &&
                     (!codes || (c_cs == 1 && c_rs % 4 == 0 && aligned(codes, 4))) &&
                     (!W_hat || (w_cs == 1 && w_rs % 4 == 0 && aligned(W_hat, bf16 ? 8 : 16) && aligned(scales, 16)));
    if (vec) {
        dim3 grid((unsigned)ceil_div(N / 4, 256), (unsigned)std::min<int64_t>(K, 65535));
        if (bf16)
            hipLaunchKernelGGL((unpack4_kernel<true>), grid, dim3(256), 0, stream, packed, ldp, K, N, bits, scales,
                               codes, c_rs, W_hat, w_rs);
        else
            hipLaunchKernelGGL((unpack4_kernel<false>), grid, dim3(256), 0, stream, packed, ldp, K, N, bits, scales,
                               codes, c_rs, W_hat, w_rs);
        return hipGetLastError();
    }
    dim3 grid((unsigned)ceil_div(N, 256), (unsigned)std::min<int64_t>(K, 65535));
    if (bf16)
        hipLaunchKernelGGL((unpack_kernel<true>), grid, dim3(256), 0, stream, packed, ldp, K, N, bits, scales, codes,
                           c_rs, c_cs, W_hat, w_rs, w_cs);
    else
        hipLaunchKernelGGL((unpack_kernel<false>), grid, dim3(256), 0, stream, packed, ldp, K, N, bits, scales, codes,
                           c_rs, c_cs, W_hat, w_rs, w_cs);
    return hipGetLastError();
}

}  // namespace gptq
