// Act-order on gfx950 ([T] section 6): the input coordinates ordered by descending Hessian diagonal.
//
// Order: the dead fix first (a zero diagonal counts as 1), then a stable descending sort: coordinate k goes to
// position rank(k) = #{i : d_i > d_k} + #{i < k : d_i == d_k}.  The ranks are computed directly, one thread
// per coordinate comparing against all K keys staged through LDS (K^2 comparisons, ~1e9 at K = 28672: far below
// the cost of the factorisation that follows), which makes the order deterministic.  The Hessian (and the
// cross Gram of asymmetric calibration) is then permuted symmetrically, H'[i][j] = H[perm[i]][perm[j]], through
// a K x K scratch copy.
#include "act_order.hpp"

#include <algorithm>

namespace gptq {

namespace {

// A NaN diagonal sorts last (as -inf) so that the comparison stays a total order and perm a permutation; such an
// H is refused by the factorisation that follows.
__device__ __forceinline__ float order_key(const float* H, int64_t K, int64_t k) {
    const float d = H[k * K + k];
    return d != d ? -INFINITY : (d == 0.0f ? 1.0f : d);
}

__global__ __launch_bounds__(256) void rank_kernel(const float* H, int64_t K, int32_t* perm) {
    __shared__ float keys[2048];
    const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const float mine = k < K ? order_key(H, K, k) : 0.f;
    int64_t rank = 0;
    for (int64_t c0 = 0; c0 < K; c0 += 2048) {
        const int64_t cn = std::min<int64_t>(2048, K - c0);
        __syncthreads();
        for (int64_t i = threadIdx.x; i < cn; i += 256) keys[i] = order_key(H, K, c0 + i);
        __syncthreads();
        if (k < K) {
            for (int64_t i = 0; i < cn; ++i) {
                const float d = keys[i];
                rank += (d > mine) || (d == mine && c0 + i < k);
            }
        }
    }
    if (k < K) perm[rank] = (int32_t)k;
}

// dst[i][j] = src[perm[i]][perm[j]] for rows i = r0 + blockIdx.y
__global__ __launch_bounds__(256) void permute_kernel(const float* src, float* dst, int64_t K, const int32_t* perm,
                                                      int64_t r0) {
    const int64_t i = r0 + blockIdx.y;
    const int64_t pi = perm[i];
    for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < K; j += (int64_t)gridDim.x * 256)
        dst[i * K + j] = src[pi * K + perm[j]];
}

}  // namespace

size_t act_order_workspace_bytes(int64_t K) { return sizeof(float) * (size_t)K * (size_t)K; }

hipError_t act_order(float* H, float* A, int64_t K, int32_t* perm, void* workspace, hipStream_t stream) {
    hipLaunchKernelGGL(rank_kernel, dim3((unsigned)ceil_div(K, 256)), dim3(256), 0, stream, H, K, perm);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    float* tmp = static_cast<float*>(workspace);
    for (float* M : {H, A}) {
        if (!M) continue;
        for (int64_t r0 = 0; r0 < K; r0 += 65535) {      // grid.y limit
            const int64_t rows = std::min<int64_t>(65535, K - r0);
            hipLaunchKernelGGL(permute_kernel, dim3((unsigned)std::min<int64_t>(ceil_div(K, 256), 64), (unsigned)rows),
                               dim3(256), 0, stream, M, tmp, K, perm, r0);
        }
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        e = hipMemcpyAsync(M, tmp, sizeof(float) * (size_t)K * (size_t)K, hipMemcpyDeviceToDevice, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace gptq
