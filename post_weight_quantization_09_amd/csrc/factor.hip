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

__device__ __forceinline__ float readlane_f(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// In place on the n x n diagonal block D (ld, n <= 128): reads its upper triangle (a symmetric block S),
// factors S = R R^T with R upper and writes U22 = R^{-1} (upper, strictly lower part zeroed).
//   Factorisation from the last coordinate backwards in panels of 16 columns: wave 0 factors a panel with the
//   panel held in registers (rows lane and lane + 64; pivots and column entries broadcast with readlane), then
//   all threads apply the rank-16 update to the remaining upper-left block (4 x 4 register tiles).
//   Inverse by recursive doubling: the eight 16 x 16 diagonal blocks are inverted by back substitution (one
//   wave each), then adjacent blocks are merged, U_ac = -U_aa (R_ac U_cc), for block sizes 16, 32 and 64.
//   Rows and columns n..127 are padded with the identity, which leaves the leading n x n result unchanged.
__global__ __launch_bounds__(1024) void chol_ul_inv_kernel(float* D, int64_t ld, int n, DevStatus* st) {
    __shared__ float S[kNB][kNB + 1];
    __shared__ float R[kNB][kNB + 1];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    for (int idx = tid; idx < kNB * kNB; idx += 1024) {
        const int i = idx >> 7, k = idx & (kNB - 1);
        float v = 0.f;
        if (i < n && k < n && i <= k) v = D[(int64_t)i * ld + k];
        S[i][k] = v;
        R[i][k] = (i == k && i >= n) ? 1.0f : 0.0f;
    }
    __syncthreads();
    unsigned bad = 0;

    for (int p1 = n; p1 > 0; p1 -= 16) {
        const int p0 = p1 > 16 ? p1 - 16 : 0;
        const int pw = p1 - p0;
        if (wave == 0) {
            float pn[2][16];
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                for (int c = 0; c < 16; ++c) pn[s2][c] = (c < pw) ? S[lane + 64 * s2][p0 + c] : 0.f;
#pragma unroll
            for (int c = 15; c >= 0; --c) {
                if (c < pw) {
                    const int j = p0 + c;
                    float d = j < 64 ? readlane_f(pn[0][c], j) : readlane_f(pn[1][c], j - 64);
                    if (!(d > 0.0f)) {
                        bad |= isfinite(d) ? kDevNotPD : kDevNonFinite;
                        d = 1.0f;
                    }
                    const float r = sqrtf(d);
                    float cj[2];
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) {
                        const int row = lane + 64 * s2;
                        cj[s2] = row < j ? pn[s2][c] / r : (row == j ? r : 0.f);
                        if (row < n) R[row][j] = cj[s2];
                    }
#pragma unroll
                    for (int cc = 0; cc < c; ++cc) {
                        const int k = p0 + cc;
                        const float ck = k < 64 ? readlane_f(cj[0], k) : readlane_f(cj[1], k - 64);
#pragma unroll
                        for (int s2 = 0; s2 < 2; ++s2) pn[s2][cc] = fmaf(-cj[s2], ck, pn[s2][cc]);
                    }
                }
            }
        }
        __syncthreads();
        if (p0 > 0) {
            const int i0 = (tid >> 5) * 4, k0 = (tid & 31) * 4;
            if (i0 < p0 && k0 < p0 && i0 <= k0 + 3) {
                float acc[4][4] = {};
                for (int c = 0; c < pw; ++c) {
                    float a4[4], b4[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        a4[u] = R[i0 + u][p0 + c];
                        b4[u] = R[k0 + u][p0 + c];
                    }
#pragma unroll
                    for (int u = 0; u < 4; ++u)
#pragma unroll
                        for (int v = 0; v < 4; ++v) acc[u][v] = fmaf(a4[u], b4[v], acc[u][v]);
                }
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        if (i0 + u < p0 && k0 + v < p0 && i0 + u <= k0 + v) S[i0 + u][k0 + v] -= acc[u][v];
            }
        }
        __syncthreads();
    }

    // Inverse of the (padded) 128 x 128 upper-triangular R, written into S.
    // Level 0: 16 x 16 diagonal blocks, column j = lane of block `wave` (lanes 0..15), back substitution.
    if (wave < 8 && lane < 16) {
        const int b0 = 16 * wave, j = lane;
        float u[16];
#pragma unroll
        for (int i = 15; i >= 0; --i) {
            const float rii = R[b0 + i][b0 + i];
            float acc = 0.f;
#pragma unroll
            for (int m = i + 1; m < 16; ++m) acc = fmaf(R[b0 + i][b0 + m], (m <= j) ? u[m] : 0.f, acc);
            u[i] = (i == j) ? 1.0f / rii : (i < j ? -acc / rii : 0.f);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) S[b0 + i][b0 + j] = u[i];
    }
    __syncthreads();
    // Levels: merge pairs (a, c) of size s: T = R_ac U_cc (kept in registers, then stored over R_ac);
    // U_ac = -U_aa T.  Each level has 64 s outputs per product, spread over the 1024 threads.
    for (int s = 16; s < kNB; s *= 2) {
        const int per = (64 * s) / 1024;                 // outputs per thread: 1, 2, 4
        float t[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            t[e] = 0.f;
            if (e < per) {
                const int o = tid * per + e;               // output index
                const int pair = o / (s * s), w = o % (s * s);
                const int i = w / s, k = w % s;
                const int a0 = 2 * s * pair, c0 = a0 + s;
                float acc = 0.f;
                for (int m = 0; m <= k; ++m) acc = fmaf(R[a0 + i][c0 + m], S[c0 + m][c0 + k], acc);
                t[e] = acc;
            }
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (e < per) {
                const int o = tid * per + e;
                const int pair = o / (s * s), w = o % (s * s);
                const int i = w / s, k = w % s;
                const int a0 = 2 * s * pair, c0 = a0 + s;
                R[a0 + i][c0 + k] = t[e];
            }
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (e < per) {
                const int o = tid * per + e;
                const int pair = o / (s * s), w = o % (s * s);
                const int i = w / s, k = w % s;
                const int a0 = 2 * s * pair, c0 = a0 + s;
                float acc = 0.f;
                for (int m = i; m < s; ++m) acc = fmaf(S[a0 + i][a0 + m], R[a0 + m][c0 + k], acc);
                S[a0 + i][c0 + k] = -acc;
            }
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
