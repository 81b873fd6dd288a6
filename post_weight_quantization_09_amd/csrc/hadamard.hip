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
// (K fp32, index k stored at k ^ ((k >> 5) & 31), which spreads every access pattern used here evenly over the
// 32 banks).  The first pass reads each thread's 16 contiguous elements with vector loads; the last pass writes
// with lanes on consecutive indices.  One HBM read and one write per element: the kernel is HBM-bound.
#include "hadamard.hpp"

#include <algorithm>
#include <cmath>

namespace gptq {

namespace {

__device__ __forceinline__ int lds_idx(int k) { return k ^ ((k >> 5) & 31); }

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

template <bool BF16, bool VEC>
__global__ __launch_bounds__(1024) void fwht_rows_kernel(const void* in, int64_t ld_in, void* out, int64_t ld_out,
                                                         int64_t rows, int n, const int8_t* signs, float scale) {
    extern __shared__ float lds[];
    const int t = threadIdx.x;
    float d[16];                      // this thread's signs, the same for every row
#pragma unroll
    for (int j = 0; j < 16; ++j) d[j] = signs ? (float)signs[16 * t + j] : 1.0f;
    for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
        float v[16];
        // pass 0: field at bit 0, the thread's 16 contiguous elements 16 t .. 16 t + 15
        if (BF16) {
            const uint16_t* src = static_cast<const uint16_t*>(in) + row * ld_in + 16 * t;
            if (VEC) {
                const u32x4 a = reinterpret_cast<const u32x4*>(src)[0], b = reinterpret_cast<const u32x4*>(src)[1];
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
        for (int done = 4; done < n; done += 4) {
            const int nf = min(done, n - 4);           // next field; overlaps the previous one when 4 does not divide n
            __syncthreads();                           // every thread is past the previous pass's LDS reads
#pragma unroll
            for (int j = 0; j < 16; ++j) lds[lds_idx(field_index(t, j, f))] = v[j];
            __syncthreads();
#pragma unroll
            for (int j = 0; j < 16; ++j) v[j] = lds[lds_idx(field_index(t, j, nf))];
            butterflies(v, done - nf);
            f = nf;
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int64_t k = field_index(t, j, f);
            const float x = v[j] * scale;
            if (BF16) static_cast<__bf16*>(out)[row * ld_out + k] = (__bf16)x;
            else static_cast<float*>(out)[row * ld_out + k] = x;
        }
    }
}

}  // namespace

hipError_t hadamard_rows(const void* in, int64_t ld_in, void* out, int64_t ld_out, bool bf16, int64_t rows, int n,
                         const int8_t* signs, hipStream_t stream) {
    const int K = 1 << n;
    const int threads = K / 16;
    const size_t lds = sizeof(float) * (size_t)K;
    const float scale = (float)(1.0 / std::sqrt((double)K));
    const bool vec = (reinterpret_cast<uintptr_t>(in) & 15) == 0 && (ld_in % (bf16 ? 8 : 4)) == 0;
    const dim3 grid((unsigned)std::min<int64_t>(rows, 1 << 20));
#define GPTQ_FWHT(B, V)                                                                                    \
    hipLaunchKernelGGL((fwht_rows_kernel<B, V>), grid, dim3(threads), lds, stream, in, ld_in, out, ld_out, \
                       rows, n, signs, scale)
    if (bf16) {
        if (vec) GPTQ_FWHT(true, true);
        else GPTQ_FWHT(true, false);
    } else {
        if (vec) GPTQ_FWHT(false, true);
        else GPTQ_FWHT(false, false);
    }
#undef GPTQ_FWHT
    return hipGetLastError();
}

}  // namespace gptq
