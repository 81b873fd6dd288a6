// Randomised Hadamard rotation of rows on gfx950: x <- (x * d) H_K / sqrt(K), K = 2^n, 16 <= K <= 16384.
//
// [G] (setup paragraph): a Hadamard rotation is applied before quantisation.  The same row transform rotates
// the activations (rows of X) and the weights in the nn.Linear N x K layout, so X W^T is unchanged; H_K is the
// Sylvester matrix (H_2m = [[H_m, H_m], [H_m, -H_m]]) and d a +-1 vector.
//
// One workgroup per row, K / 16 threads, 16 elements per thread in registers.  The fast Walsh-Hadamard
// transform is a butterfly on every one of the n index bits; it runs in passes of 4 bits: in a pass, thread t
// holds the 16 elements whose index differs only in the pass's 4-bit field (index = low bits of t | field |
// high bits of t) and applies those 4 butterfly stages in registers.  Between passes the row goes through LDS
// (K fp32 plus one float of padding after every 32: with it every layout used here is a per-thread base plus
// compile-time offsets, and a wave's 64 accesses fall two to a bank).  n is a template parameter, so the
// passes unroll and no index arithmetic is left in the row loop.  The first pass reads each thread's 16
// contiguous elements with vector loads (for bf16 rows, the next row's are issued before this row is
// transformed); the last pass writes with lanes on consecutive indices.  The signs and 1/sqrt(K) are applied
// together when the row is read.  One HBM read and one write per element.
#include "hadamard.hpp"

#include <algorithm>
#include <cmath>
#include <type_traits>

namespace gptq {

namespace {

// LDS position of row index k (one float of padding after every 32).  For k = a | b with disjoint bits,
// lds_pos(k) = lds_pos(a) + lds_pos(b), which makes the register-field offsets compile-time constants.
__host__ __device__ constexpr int lds_pos(int k) { return k + (k >> 5); }

// Index of element j of thread t when the register field starts at bit f.
__device__ __forceinline__ int field_index(int t, int j, int f) {
    const int low = t & ((1 << f) - 1);
    const int high = t >> f;
    return low | (j << f) | (high << (f + 4));
}

// Butterflies on bits [first, 4) of the 4-bit register index.
__device__ __forceinline__ void butterflies(float (&v)[16], int first) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        if (b < first) continue;
        const int h = 1 << b;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            if (j & h) continue;
            const float a = v[j], c = v[j | h];
            v[j] = a + c;
            v[j | h] = a - c;
        }
    }
}

template <int N, bool BF16, bool VEC>
__global__ __launch_bounds__(1024) void fwht_rows_kernel(const void* in, int64_t ld_in, void* out, int64_t ld_out,
                                                         int64_t rows, const int8_t* signs, float scale) {
    __shared__ float lds[N > 4 ? lds_pos(1 << N) : 1];
    const int t = threadIdx.x;
    float d[16];                      // this thread's signs times 1/sqrt(K), the same for every row
#pragma unroll
    for (int j = 0; j < 16; ++j) d[j] = signs ? (float)signs[16 * t + j] * scale : scale;
    // bf16 rows with 16-byte aligned rows: the next row's raw data is loaded while this one is transformed
    constexpr bool kPrefetch = BF16 && VEC;
    u32x4 pa = {0u, 0u, 0u, 0u}, pb = {0u, 0u, 0u, 0u};
    if (kPrefetch && blockIdx.x < rows) {
        const uint16_t* src = static_cast<const uint16_t*>(in) + (int64_t)blockIdx.x * ld_in + 16 * t;
        pa = reinterpret_cast<const u32x4*>(src)[0];
        pb = reinterpret_cast<const u32x4*>(src)[1];
    }
    for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
        float v[16];
        // pass 0: field at bit 0, the thread's 16 contiguous elements 16 t .. 16 t + 15
        if (BF16) {
            const uint16_t* src = static_cast<const uint16_t*>(in) + row * ld_in + 16 * t;
            if (VEC) {
                const u32x4 a = pa, b = pb;
                const int64_t nrow = row + gridDim.x;
                if (nrow < rows) {
                    const uint16_t* nsrc = static_cast<const uint16_t*>(in) + nrow * ld_in + 16 * t;
                    pa = reinterpret_cast<const u32x4*>(nsrc)[0];
                    pb = reinterpret_cast<const u32x4*>(nsrc)[1];
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v[2 * i] = bf16lo_to_f32(a[i]);
                    v[2 * i + 1] = bf16hi_to_f32(a[i]);
                    v[8 + 2 * i] = bf16lo_to_f32(b[i]);
                    v[8 + 2 * i + 1] = bf16hi_to_f32(b[i]);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 16; ++j) v[j] = __uint_as_float((uint32_t)src[j] << 16);
            }
        } else {
            const float* src = static_cast<const float*>(in) + row * ld_in + 16 * t;
            if (VEC) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const f32x4 a = reinterpret_cast<const f32x4*>(src)[i];
                    v[4 * i] = a.x; v[4 * i + 1] = a.y; v[4 * i + 2] = a.z; v[4 * i + 3] = a.w;
                }
            } else {
#pragma unroll
                for (int j = 0; j < 16; ++j) v[j] = src[j];
            }
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] *= d[j];
        butterflies(v, 0);
        int f = 0;
#pragma unroll
        for (int done = 4; done < N; done += 4) {
            const int nf = done < N - 4 ? done : N - 4;   // next field; overlaps the previous one when 4 does not divide n
            const int wbase = lds_pos(field_index(t, 0, f)), rbase = lds_pos(field_index(t, 0, nf));
            __syncthreads();                           // every thread is past the previous pass's LDS reads
#pragma unroll
            for (int j = 0; j < 16; ++j) lds[wbase + lds_pos(j << f)] = v[j];
            __syncthreads();
#pragma unroll
            for (int j = 0; j < 16; ++j) v[j] = lds[rbase + lds_pos(j << nf)];
            butterflies(v, done - nf);
            f = nf;
        }
        const int64_t obase = row * ld_out + field_index(t, 0, f);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            if (BF16) static_cast<__bf16*>(out)[obase + (j << f)] = (__bf16)v[j];
            else static_cast<float*>(out)[obase + (j << f)] = v[j];
        }
    }
}

}  // namespace

hipError_t hadamard_rows(const void* in, int64_t ld_in, void* out, int64_t ld_out, bool bf16, int64_t rows, int n,
                         const int8_t* signs, hipStream_t stream) {
    if (n < 4 || n > 14) return hipErrorInvalidValue;
    const int K = 1 << n;
    const int threads = K / 16;
    const float scale = (float)(1.0 / std::sqrt((double)K));
    const bool vec = (reinterpret_cast<uintptr_t>(in) & 15) == 0 && (ld_in % (bf16 ? 8 : 4)) == 0;
    // Up to 128k workgroups, each looping over rows with the next row's load in flight (measured on
    // 2M x 4096 bf16: 6.5 ms at 128k, 6.7-6.8 ms at 8k-64k, 7.8 ms with one workgroup per two rows).
    const dim3 grid((unsigned)std::min<int64_t>(rows, 1 << 17));
    auto launch = [&](auto nc) {
        constexpr int N = decltype(nc)::value;
#define GPTQ_FWHT(B, V)                                                                                        \
    hipLaunchKernelGGL((fwht_rows_kernel<N, B, V>), grid, dim3(threads), 0, stream, in, ld_in, out, ld_out, rows, \
                       signs, scale)
        if (bf16) {
            if (vec) GPTQ_FWHT(true, true);
            else GPTQ_FWHT(true, false);
        } else {
            if (vec) GPTQ_FWHT(false, true);
            else GPTQ_FWHT(false, false);
        }
#undef GPTQ_FWHT
    };
    switch (n) {
        case 4: launch(std::integral_constant<int, 4>{}); break;
        case 5: launch(std::integral_constant<int, 5>{}); break;
        case 6: launch(std::integral_constant<int, 6>{}); break;
        case 7: launch(std::integral_constant<int, 7>{}); break;
        case 8: launch(std::integral_constant<int, 8>{}); break;
        case 9: launch(std::integral_constant<int, 9>{}); break;
        case 10: launch(std::integral_constant<int, 10>{}); break;
        case 11: launch(std::integral_constant<int, 11>{}); break;
        case 12: launch(std::integral_constant<int, 12>{}); break;
        case 13: launch(std::integral_constant<int, 13>{}); break;
        default: launch(std::integral_constant<int, 14>{}); break;
    }
    return hipGetLastError();
}

}  // namespace gptq
