// Preparation of the Hessian on gfx950: dead coordinates, damping, and U with H_d^{-1} = U^T U.
//
// [T] section 6: coordinates whose Hessian diagonal is zero are "dead": their diagonal is set (here to 1)
// and their weights to zero; then percdamp * mean(diag H) is added to the diagonal.
// [T] section 4: the compensation reads rows of the upper factor U of the inverse, U_qq^2 being the inverse
// of the Hessian left when q is the first free coordinate.
//
// U is computed without forming H_d^{-1}: H_d = R R^T with R upper triangular (the Cholesky factorisation
// taken from the bottom-right corner), then U = R^{-1}, since H_d^{-1} = R^{-T} R^{-1} = U^T U with U upper.
// Both steps are blocked with nb = 128:
//   * per diagonal block (bottom-up): an LDS kernel factors the 128 x 128 block and inverts it in place
//     (the diagonal block of U is the inverse of the diagonal block of R); the panel above becomes
//     R12 = H12 U22^T and the trailing upper triangle is updated H11 -= R12 R12^T, both on fp32 MFMA.
//   * the off-diagonal blocks of U follow by recursive doubling: for adjacent blocks a (upper left) and
//     c, U_ac = -U_aa R_ac U_cc, merged for block sizes 128, 256, ... as two batched triangular GEMMs.
#include <algorithm>
#include <vector>

#include "factor.hpp"
#include "gemm_f32.hpp"

namespace gptq {

namespace {

constexpr int kNB = 128;

__global__ __launch_bounds__(1024) void dead_damp_kernel(float* H, int64_t K, float percdamp, uint8_t* dead,
                                                         DevStatus* st) {
    __shared__ double ssum[1024];
    __shared__ unsigned scnt[1024];
    __shared__ unsigned sbad[1024];
    const int tid = threadIdx.x;
    double sum = 0.0;
    unsigned nd = 0, bad = 0;
    for (int64_t k = tid; k < K; k += 1024) {
        float d = H[k * K + k];
        if (!isfinite(d)) bad = 1;
        if (d == 0.0f) {
            dead[k] = 1;
            d = 1.0f;
            H[k * K + k] = d;
            ++nd;
        } else {
            dead[k] = 0;
        }
        sum += (double)d;
    }
    ssum[tid] = sum;
    scnt[tid] = nd;
    sbad[tid] = bad;
    __syncthreads();
    for (int w = 512; w > 0; w >>= 1) {
        if (tid < w) {
            ssum[tid] += ssum[tid + w];
            scnt[tid] += scnt[tid + w];
            sbad[tid] |= sbad[tid + w];
        }
        __syncthreads();
    }
    const float damp = (float)((double)percdamp * (ssum[0] / (double)K));
    for (int64_t k = tid; k < K; k += 1024) H[k * K + k] += damp;
    if (tid == 0) {
        st->damp = damp;
        st->n_dead = scnt[0];
        if (sbad[0]) st->flags |= kDevNonFinite;
    }
}

// In place on the n x n diagonal block D (ld): reads its upper triangle (a symmetric block S), factors
// S = R R^T with R upper, and writes U22 = R^{-1} (upper, strictly lower part zeroed).
__global__ __launch_bounds__(1024) void chol_ul_inv_kernel(float* D, int64_t ld, int n, DevStatus* st) {
    __shared__ float S[kNB][kNB + 1];
    __shared__ float R[kNB][kNB + 1];
    const int tid = threadIdx.x;
    for (int idx = tid; idx < n * n; idx += 1024) {
        const int i = idx / n, k = idx % n;
        if (i <= k) S[i][k] = D[(int64_t)i * ld + k];
    }
    __syncthreads();
    unsigned bad = 0;
    // Factorisation from the last coordinate backwards: column j of R is the current column j of the
    // Schur complement divided by the square root of its pivot; the rest of the upper-left block is updated.
    for (int j = n - 1; j >= 0; --j) {
        float d = S[j][j];
        if (!(d > 0.0f)) {
            bad |= isfinite(d) ? kDevNotPD : kDevNonFinite;
            d = 1.0f;
        }
        const float invd = 1.0f / d;
        const float r = sqrtf(d);
        if (tid <= j) R[tid][j] = (tid == j) ? r : S[tid][j] / r;
        for (int m = 0; m < (kNB * kNB) / 1024; ++m) {
            const int idx = tid + 1024 * m;
            const int i = idx >> 7, k = idx & (kNB - 1);
            if (i <= k && k < j) S[i][k] = fmaf(-S[i][j] * invd, S[k][j], S[i][k]);
        }
        __syncthreads();
    }
    // Inverse of the upper-triangular R, row by row from the bottom:
    //   U_ii = 1 / R_ii;  U_ik = -U_ii * sum_{i<m<=k} R_im U_mk   (k > i).
    // 8 threads share one output column k and combine their partial sums with lane shuffles.
    const int kk = tid >> 3, part = tid & 7;
    for (int i = n - 1; i >= 0; --i) {
        const float uii = 1.0f / R[i][i];
        float acc = 0.0f;
        if (kk > i && kk < n)
            for (int m = i + 1 + part; m <= kk; m += 8) acc = fmaf(R[i][m], S[m][kk], acc);
        acc += __shfl_xor(acc, 1, 8);
        acc += __shfl_xor(acc, 2, 8);
        acc += __shfl_xor(acc, 4, 8);
        if (part == 0 && kk < n) {
            if (kk == i) S[i][i] = uii;
            else if (kk > i) S[i][kk] = -uii * acc;
        }
        __syncthreads();
    }
    for (int idx = tid; idx < n * n; idx += 1024) {
        const int i = idx / n, k = idx % n;
        D[(int64_t)i * ld + k] = (i <= k) ? S[i][k] : 0.0f;
    }
    if (bad && tid == 0) atomicOr(&st->flags, bad);
}

__global__ void zero_lower_kernel(float* U, int64_t K) {
    const int64_t row = blockIdx.x;
    for (int64_t c = threadIdx.x; c < row && c < K; c += blockDim.x) U[row * K + c] = 0.0f;
}

__global__ void clear_status_kernel(DevStatus* st) {
    if (threadIdx.x == 0) {
        st->flags = 0;
        st->n_dead = 0;
        st->damp = 0.f;
    }
}

}  // namespace

// Scratch of the inverse merges: at block size s at most (K + 128) / (2 s) pairs of s x s products with
// 2 s <= K + 128, i.e. at most (K + 128)^2 / 4 floats.
static size_t merge_scratch_floats(int64_t K) { return (size_t)(K + kNB) * (size_t)(K + kNB) / 4 + kNB * kNB; }

size_t prepare_workspace_bytes(int64_t K) {
    Carver c(nullptr);
    c.take<DevStatus>(1);
    c.take<float>(merge_scratch_floats(K));
    return c.bytes();
}

gptq_status_t prepare(float* H, int64_t K, float percdamp, uint8_t* dead, float* damp_out, int64_t* n_dead_out,
                      void* workspace, hipStream_t stream) {
    Carver c(workspace);
    DevStatus* st = c.take<DevStatus>(1);
    float* T = c.take<float>(merge_scratch_floats(K));

    hipLaunchKernelGGL(clear_status_kernel, dim3(1), dim3(64), 0, stream, st);
    hipLaunchKernelGGL(dead_damp_kernel, dim3(1), dim3(1024), 0, stream, H, K, percdamp, dead, st);
    GPTQ_LAUNCH_CHECK();

    // Blocked factorisation H_d = R R^T from the bottom-right; diagonal blocks become U_ii = R_ii^{-1}.
    for (int64_t p1 = K; p1 > 0;) {
        const int64_t p0 = std::max<int64_t>(0, p1 - kNB);
        const int n = (int)(p1 - p0);
        hipLaunchKernelGGL(chol_ul_inv_kernel, dim3(1), dim3(1024), 0, stream, H + p0 * K + p0, K, n, st);
        GPTQ_LAUNCH_CHECK();
        if (p0 > 0) {
            // R12 = H12 U22^T  (in place; one workgroup owns all n <= 128 columns of each row tile)
            GemmArgs g;
            g.M = p0; g.N = n; g.K1 = n;
            g.A1 = H + p0; g.lda1 = K;
            g.B1 = H + p0 * K + p0; g.ldb1 = K; g.transB = true;   // B(k, c) = U22[c][k]
            g.C = H + p0; g.ldc = K;
            g.alpha = 1.f; g.beta = 0.f;
            g.flags = kGemmBLower;
            if (gemm_f32(g, 1, stream) != hipSuccess) return GPTQ_ERR_HIP;
            // H11 -= R12 R12^T on the upper triangle
            GemmArgs s;
            s.M = p0; s.N = p0; s.K1 = n;
            s.A1 = H + p0; s.lda1 = K;
            s.B1 = H + p0; s.ldb1 = K; s.transB = true;            // B(k, c) = R12[c][k]
            s.C = H; s.ldc = K;
            s.alpha = -1.f; s.beta = 1.f;
            s.flags = kGemmCUpper;
            if (gemm_f32(s, 1, stream) != hipSuccess) return GPTQ_ERR_HIP;
        }
        p1 = p0;
    }

    // The merges read whole square blocks of U as triangular operands: clear the stale lower triangle.
    hipLaunchKernelGGL(zero_lower_kernel, dim3((unsigned)K), dim3(256), 0, stream, H, K);
    GPTQ_LAUNCH_CHECK();

    // Off-diagonal blocks of U = R^{-1} by recursive doubling.  The blocks are aligned to the top-left
    // corner in steps of 128 starting from the factorisation's top block, which may be shorter.
    const int64_t first = K - ((K - 1) / kNB) * kNB;   // size of the top (ragged) block, in 1..128
    // Offsets of block boundaries measured from the top: 0, first, first+128, ...
    // Merging uses "virtual" coordinates v = x + (128 - first) so that blocks are 128-aligned.
    const int64_t shift = kNB - first;
    for (int64_t s = kNB; s < K + shift; s *= 2) {
        // pairs (a, c): a = [i*2s, i*2s+s), c = [i*2s+s, i*2s+2s) in virtual coordinates
        std::vector<int64_t> full, partial_pairs;
        for (int64_t v0 = 0; v0 + s < K + shift; v0 += 2 * s) {
            const int64_t a0 = std::max<int64_t>(0, v0 - shift), a1 = v0 + s - shift;
            const int64_t c0 = a1, c1 = std::min<int64_t>(K, v0 + 2 * s - shift);
            if (a1 - a0 == s && c1 - c0 == s) full.push_back(a0);
            else partial_pairs.push_back(v0);
        }
        auto merge = [&](int64_t a0, int64_t sa, int64_t c0, int64_t sc, int64_t batch, int64_t bstride)
            -> gptq_status_t {
            // T = R_ac U_cc   (sa x sc) ;  U_ac = -U_aa T
            GemmArgs g1;
            g1.M = sa; g1.N = sc; g1.K1 = sc;
            g1.A1 = H + a0 * K + c0; g1.lda1 = K; g1.strideA1 = bstride;
            g1.B1 = H + c0 * K + c0; g1.ldb1 = K; g1.strideB1 = bstride;
            g1.C = T; g1.ldc = sc; g1.strideC = sa * sc;
            g1.flags = kGemmBUpper;
            if (gemm_f32(g1, batch, stream) != hipSuccess) return GPTQ_ERR_HIP;
            GemmArgs g2;
            g2.M = sa; g2.N = sc; g2.K1 = sa;
            g2.A1 = H + a0 * K + a0; g2.lda1 = K; g2.strideA1 = bstride;
            g2.B1 = T; g2.ldb1 = sc; g2.strideB1 = sa * sc;
            g2.C = H + a0 * K + c0; g2.ldc = K; g2.strideC = bstride;
            g2.alpha = -1.f; g2.beta = 0.f;
            g2.flags = kGemmAUpper;
            if (gemm_f32(g2, batch, stream) != hipSuccess) return GPTQ_ERR_HIP;
            return GPTQ_OK;
        };
        if (!full.empty()) {
            // full pairs are equally spaced by 2s along the diagonal
            const int64_t a0 = full.front();
            const int64_t bstride = 2 * s * (K + 1);
            gptq_status_t r = merge(a0, s, a0 + s, s, (int64_t)full.size(), bstride);
            if (r != GPTQ_OK) return r;
        }
        for (int64_t v0 : partial_pairs) {
            const int64_t a0 = std::max<int64_t>(0, v0 - shift), a1 = v0 + s - shift;
            const int64_t c0 = a1, c1 = std::min<int64_t>(K, v0 + 2 * s - shift);
            gptq_status_t r = merge(a0, a1 - a0, c0, c1 - c0, 1, 0);
            if (r != GPTQ_OK) return r;
        }
    }
    DevStatus hst;
    GPTQ_HIP_CHECK(hipMemcpyAsync(&hst, st, sizeof(DevStatus), hipMemcpyDeviceToHost, stream));
    GPTQ_HIP_CHECK(hipStreamSynchronize(stream));
    if (damp_out) *damp_out = hst.damp;
    if (n_dead_out) *n_dead_out = hst.n_dead;
    if (hst.flags & kDevNonFinite) return GPTQ_ERR_NONFINITE;
    if (hst.flags & kDevNotPD) return GPTQ_ERR_NOT_PD;
    return GPTQ_OK;
}

}  // namespace gptq
