// Preparation of the Hessian on gfx950: dead coordinates, damping, and U with H_d^{-1} = U^T U.
//
// [T] section 6: coordinates whose Hessian diagonal is zero are "dead": their diagonal is set (here to 1)
// and their weights to zero; then percdamp * mean(diag H) is added to the diagonal.
// [T] section 4: the compensation reads rows of the upper factor U of the inverse, U_qq^2 being the inverse
// of the Hessian left when q is the first free coordinate.
//
// U is computed without forming H_d^{-1}: H_d = R R^T with R upper triangular (the Cholesky factorisation
// taken from the bottom-right corner), then U = R^{-1}, since H_d^{-1} = R^{-T} R^{-1} = U^T U with U upper.
// Factor and inverse run as one recursion over a 2 x 2 split of the block (top part n1 a multiple of 128):
//     H = [H11 H12; . H22],  R = [R11 R12; 0 R22],  U = [U11 U12; 0 U22]
//   1. recurse on H22 -> U22                      (H22 = R22 R22^T)
//   2. R12 = H12 U22^T                             (from H12 = R12 R22^T)
//   3. H11 <- H11 - R12 R12^T  (upper triangle)    (H11 = R11 R11^T + R12 R12^T)
//   4. X = R12 U22
//   5. recurse on H11 -> U11
//   6. U12 = -U11 X                                (U R = I gives U11 R12 + U12 R22 = 0)
// Steps 2, 3, 4 and 6 are fp32 MFMA GEMMs; the recursion ends in 128 x 128 (or smaller) diagonal blocks that
// one LDS kernel factors and inverts.  Since the split points are multiples of 128 from the top, every
// GEMM tile is aligned with the diagonal blocks.  A batch of Hessians ([G]: one per output-channel group)
// runs the same recursion with every GEMM batched and every diagonal block one launch over the batch.
#include <algorithm>
#include <type_traits>
#include <vector>

#include "factor.hpp"

#include "gemm_f32.hpp"
#include "timer.hpp"

namespace gptq {

namespace {

constexpr int kNB = 128;

__global__ __launch_bounds__(1024) void dead_damp_kernel(float* H, int64_t K, int64_t strideH, float percdamp,
                                                         uint8_t* dead, DevStatus* st) {
    H += (int64_t)blockIdx.x * strideH;   // one workgroup per Hessian of the batch
    dead += (int64_t)blockIdx.x * K;
    st += blockIdx.x;
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

// Wave 0's factorisation of the 16-column panel p0 .. p0 + 15 of chol_ul_inv_kernel.  Lane l holds rows l and
// l + 64 of the panel in two register halves.  HI (p0 >= 64): every row of half 0 lies above the panel, so its
// entries are only scaled; otherwise every row of half 1 lies below the panel, is zero in R and is not held.
template <bool HI>
__device__ __forceinline__ void factor_panel(float (*S)[kNB + 1], float (*R)[kNB + 1], float* Rinv, int p0,
                                             int lane, unsigned& bad) {
    constexpr int NH = HI ? 2 : 1;   // register halves holding rows at or above the panel
    float pn[NH][16];
#pragma unroll
    for (int s2 = 0; s2 < NH; ++s2)
#pragma unroll
        for (int c = 0; c < 16; ++c) pn[s2][c] = S[lane + 64 * s2][p0 + c];
#pragma unroll
    for (int c = 15; c >= 0; --c) {
        const int j = p0 + c;
        float d = readlane_f(pn[NH - 1][c], j & 63);
        if (!(d > 0.0f)) {
            bad |= isfinite(d) ? kDevNotPD : kDevNonFinite;
            d = 1.0f;
        }
        float rinv = __builtin_amdgcn_rsqf(d);
        rinv = rinv * fmaf(-0.5f * d * rinv, rinv, 1.5f);   // one Newton step on 1/sqrt(d)
        const float r = d * rinv;
        float cj[NH];
#pragma unroll
        for (int s2 = 0; s2 < NH; ++s2) {
            const int row = lane + 64 * s2;
            if (HI && s2 == 0) cj[s2] = pn[s2][c] * rinv;   // row < 64 <= j
            else cj[s2] = row < j ? pn[s2][c] * rinv : (row == j ? r : 0.f);
            R[row][j] = cj[s2];
        }
        if (!HI) R[lane + 64][j] = 0.f;
        if (lane == 0) Rinv[j] = rinv;
#pragma unroll
        for (int cc = 0; cc < c; ++cc) {
            const float ck = readlane_f(cj[NH - 1], (p0 + cc) & 63);
#pragma unroll
            for (int s2 = 0; s2 < NH; ++s2) pn[s2][cc] = fmaf(-cj[s2], ck, pn[s2][cc]);
        }
    }
}

// In place on the n x n diagonal block D (ld, n <= 128): reads its upper triangle (a symmetric block S),
// factors S = R R^T with R upper and writes U = R^{-1} (upper, strictly lower part zeroed).
//   The block sits in the bottom-right corner of a 128 x 128 frame whose top-left is the identity, so every
//   loop below has a fixed trip count; the identity factors and inverts to itself.
//   Factorisation from the last coordinate backwards in panels of 16 columns: wave 0 factors a panel held in
//   registers (rows lane and lane + 64; pivot and column entries broadcast with readlane; the column is
//   scaled by the reciprocal square root of the pivot), then the rank-16 update of the remaining upper-left
//   block runs on v_mfma_f32_32x32x2_f32, one 32 x 32 tile per wave.
//   Inverse by recursive doubling: the eight 16 x 16 diagonal blocks are inverted by back substitution, then
//   adjacent blocks a (upper) and c are merged, U_ac = -U_aa (R_ac U_cc), for block sizes 16, 32 and 64,
//   each product on v_mfma_f32_16x16x4_f32, one 16 x 16 tile per wave.
__global__ __launch_bounds__(1024) void chol_ul_inv_kernel(float* D, int64_t ld, int n, DevStatus* st,
                                                           int64_t strideD) {
    D += (int64_t)blockIdx.x * strideD;   // one workgroup per Hessian of the batch
    st += blockIdx.x;
    __shared__ float S[kNB][kNB + 1];
    __shared__ float R[kNB][kNB + 1];
    __shared__ float Rinv[kNB];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int o = kNB - n;
    // a whole 128-block with 16-byte rows: thread t takes 16 consecutive entries of row t / 8 (four 16-byte loads
    // in flight at once instead of sixteen dependent scalar rounds)
    const bool vec = o == 0 && (ld & 3) == 0 && (reinterpret_cast<uintptr_t>(D) & 15) == 0;
    if (vec) {
        const int i = tid >> 3, k0 = (tid & 7) * 16;
        f32x4 v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = *reinterpret_cast<const f32x4*>(D + (int64_t)i * ld + k0 + 4 * q);
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) S[i][k0 + 4 * q + e] = (i <= k0 + 4 * q + e) ? v[q][e] : 0.0f;
    } else {
        for (int idx = tid; idx < kNB * kNB; idx += 1024) {
            const int i = idx >> 7, k = idx & (kNB - 1);
            float v = (i == k) ? 1.0f : 0.0f;
            if (i >= o && i <= k) v = D[(int64_t)(i - o) * ld + (k - o)];
            S[i][k] = v;
        }
    }
    __syncthreads();
    unsigned bad = 0;

    for (int P = kNB / 16 - 1; P >= 0; --P) {
        const int p0 = 16 * P;
        if (wave == 0) {
            if (p0 >= 64) factor_panel<true>(S, R, Rinv, p0, lane, bad);
            else factor_panel<false>(S, R, Rinv, p0, lane, bad);
        }
        __syncthreads();
        if (p0 > 0) {
            // S[i][k] -= sum_c R[i][p0+c] R[k][p0+c] for i <= k < p0, over the upper 32 x 32 tiles.
            const int T = (p0 + 31) >> 5;
            int bi = 0, bk = wave, cnt = T;
            while (bk >= cnt && cnt > 0) { bk -= cnt; ++bi; --cnt; }   // wave -> (bi, bi + bk)
            if (bi < T) {
                bk += bi;
                f32x16 acc;
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
                for (int s2 = 0; s2 < 8; ++s2) {
                    const int c = p0 + 2 * s2 + (lane >> 5);
                    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(R[32 * bi + (lane & 31)][c],
                                                               R[32 * bk + (lane & 31)][c], acc, 0, 0, 0);
                }
                const int col = 32 * bk + (lane & 31);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = 32 * bi + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    if (row <= col && col < p0) S[row][col] -= acc[r];
                }
            }
        }
        __syncthreads();
    }

    // Inverse of the upper-triangular R (128 x 128), written into S (whose strictly lower part is zero).
    // Level 0: 16 x 16 diagonal blocks, column j = lane of block `wave` (lanes 0..15), back substitution.
    if (wave < 8 && lane < 16) {
        const int b0 = 16 * wave, j = lane;
        float u[16];
#pragma unroll
        for (int i = 15; i >= 0; --i) {
            float acc = 0.f;
#pragma unroll
            for (int m = i + 1; m < 16; ++m) acc = fmaf(R[b0 + i][b0 + m], u[m], acc);
            const float ri = Rinv[b0 + i];
            u[i] = (i == j) ? ri : (i < j ? -acc * ri : 0.f);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) S[b0 + i][b0 + j] = u[i];
    }
    __syncthreads();
    // Merges of pairs (a, c) of size s: T = R_ac U_cc (then stored over R_ac), U_ac = -U_aa T.  The size is a
    // template constant so that each product's LDS operand reads are unrolled and issued ahead of its MFMA chain.
    auto merge = [&](auto sc) {
        constexpr int s = decltype(sc)::value;
        constexpr int per_side = s >> 4, tpp = per_side * per_side;
        constexpr int ntile = (kNB / (2 * s)) * tpp;   // 4, 8, 16 tiles of 16 x 16
        const int pair = wave / tpp, w = wave % tpp;
        const int ti = w / per_side, tk = w % per_side;
        const int a0 = 2 * s * pair, c0 = a0 + s;
        const int ar = 16 * ti + (lane & 15), kq = lane >> 4, oc = 16 * tk + (lane & 15);
        f32x4 t = {0.f, 0.f, 0.f, 0.f};
        if (wave < ntile) {
            float x[s / 4], y[s / 4];
#pragma unroll
            for (int m = 0; m < s / 4; ++m) { x[m] = R[a0 + ar][c0 + 4 * m + kq]; y[m] = S[c0 + 4 * m + kq][c0 + oc]; }
#pragma unroll
            for (int m = 0; m < s / 4; ++m) t = __builtin_amdgcn_mfma_f32_16x16x4f32(x[m], y[m], t, 0, 0, 0);
        }
        __syncthreads();
        if (wave < ntile) {
#pragma unroll
            for (int r = 0; r < 4; ++r) R[a0 + 16 * ti + 4 * kq + r][c0 + oc] = t[r];
        }
        __syncthreads();
        if (wave < ntile) {
            f32x4 u = {0.f, 0.f, 0.f, 0.f};
            float x[s / 4], y[s / 4];
#pragma unroll
            for (int m = 0; m < s / 4; ++m) { x[m] = S[a0 + ar][a0 + 4 * m + kq]; y[m] = R[a0 + 4 * m + kq][c0 + oc]; }
#pragma unroll
            for (int m = 0; m < s / 4; ++m) u = __builtin_amdgcn_mfma_f32_16x16x4f32(x[m], y[m], u, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) S[a0 + 16 * ti + 4 * kq + r][c0 + oc] = -u[r];
        }
        __syncthreads();
    };
    merge(std::integral_constant<int, 16>{});
    merge(std::integral_constant<int, 32>{});
    merge(std::integral_constant<int, 64>{});
    if (vec) {
        const int i = tid >> 3, k0 = (tid & 7) * 16;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (i <= k0 + 4 * q + e) ? S[i][k0 + 4 * q + e] : 0.0f;
            *reinterpret_cast<f32x4*>(D + (int64_t)i * ld + k0 + 4 * q) = v;
        }
    } else {
        for (int idx = tid; idx < kNB * kNB; idx += 1024) {
            const int i = idx >> 7, k = idx & (kNB - 1);
            if (i >= o && k >= o) D[(int64_t)(i - o) * ld + (k - o)] = (i <= k) ? S[i][k] : 0.0f;
        }
    }
    if (bad && tid == 0) atomicOr(&st->flags, bad);
}

__global__ void zero_lower_kernel(float* U, int64_t K, int64_t strideU) {
    U += (int64_t)blockIdx.y * strideU;
    const int64_t row = blockIdx.x;
    for (int64_t c = threadIdx.x; c < row && c < K; c += blockDim.x) U[row * K + c] = 0.0f;
}

__global__ void clear_status_kernel(DevStatus* st, int64_t n) {
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
        st[i].flags = 0;
        st[i].n_dead = 0;
        st[i].damp = 0.f;
    }
}

// st[0].flags |= st[b].flags for every b: the first status word then reports the whole batch.
__global__ void merge_status_kernel(DevStatus* st, int64_t n) {
    uint32_t f = 0;
    for (int64_t i = 1 + threadIdx.x; i < n; i += blockDim.x) f |= st[i].flags;
    if (f) atomicOr(&st[0].flags, f);
}

}  // namespace

// Split of an n-block (n > 128): the top part n1 is a multiple of 128, the bottom part n2 = n - n1 > 0.
static inline int64_t split_top(int64_t n) { return ((n + kNB - 1) / kNB / 2) * kNB; }

// Scratch floats of the recursion on an n-block: X (n1 x n2) lives across the recursion on H11, the
// temporary R12 (n1 x n2) only before it.
static size_t recursion_scratch_floats(int64_t n) {
    if (n <= kNB) return 0;
    const int64_t n1 = split_top(n), n2 = n - n1;
    const size_t x = (size_t)n1 * (size_t)n2;
    return std::max(recursion_scratch_floats(n2), x + std::max(x, recursion_scratch_floats(n1)));
}

// Per-Hessian scratch of a batch, rounded to 64 floats so that every batch element's operands stay 256-byte
// aligned.
static size_t batch_scratch_floats(int64_t K) {
    return (std::max<size_t>(recursion_scratch_floats(K), 1) + 63) / 64 * 64;
}

size_t prepare_workspace_bytes(int64_t K, int64_t batch) {
    batch = std::max<int64_t>(batch, 1);
    Carver c(nullptr);
    c.take<DevStatus>((size_t)batch);
    c.take<float>(batch_scratch_floats(K) * (size_t)batch);
    return c.bytes();
}

namespace {

// The recursion on `batch` Hessians at once (H + b strideH, scratch T + b Ts): the same splits for all, every
// GEMM one batched launch and every diagonal block one launch with a workgroup per Hessian.
struct Recursion {
    float* H;
    int64_t K;
    DevStatus* st;
    hipStream_t stream;
    int64_t batch = 1, strideH = 0, Ts = 0;

    hipError_t gemm(GemmArgs g, int64_t sa, int64_t sb, int64_t sc) const {
        g.strideA1 = sa; g.strideB1 = sb; g.strideC = sc;
        TimerScope ts(stream, GPTQ_TIMER_FACTOR_GEMM);
        return gemm_f32(g, batch, stream);
    }

    gptq_status_t run(int64_t o, int64_t n, float* T) {
        float* D = H + o * K + o;
        if (n <= kNB) {
            TimerScope ts(stream, GPTQ_TIMER_FACTOR_DIAG);
            hipLaunchKernelGGL(chol_ul_inv_kernel, dim3((unsigned)batch), dim3(1024), 0, stream, D, K, (int)n, st,
                               strideH);
            return hipGetLastError() == hipSuccess ? GPTQ_OK : GPTQ_ERR_HIP;
        }
        const int64_t n1 = split_top(n), n2 = n - n1;
        float* H12 = D + n1;
        float* D22 = D + n1 * K + n1;
        float* X = T;
        float* R12 = T + n1 * n2;
        gptq_status_t r = run(o + n1, n2, T);
        if (r != GPTQ_OK) return r;
        {   // R12 = H12 U22^T
            GemmArgs g;
            g.M = n1; g.N = n2; g.K1 = n2;
            g.A1 = H12; g.lda1 = K;
            g.B1 = D22; g.ldb1 = K; g.transB = true;   // B(k, c) = U22[c][k], zero for k < c
            g.C = R12; g.ldc = n2;
            g.flags = kGemmBLower;
            if (gemm(g, strideH, strideH, Ts) != hipSuccess) return GPTQ_ERR_HIP;
        }
        {   // H11 -= R12 R12^T on the upper triangle, and X = R12 U22: independent, one launch where both fit it
            GemmArgs s;
            s.M = n1; s.N = n1; s.K1 = n2;
            s.A1 = R12; s.lda1 = n2;
            s.B1 = R12; s.ldb1 = n2; s.transB = true;
            s.C = D; s.ldc = K;
            s.alpha = -1.f; s.beta = 1.f;
            s.flags = kGemmCUpper;
            s.strideA1 = Ts; s.strideB1 = Ts; s.strideC = strideH;
            GemmArgs x;
            x.M = n1; x.N = n2; x.K1 = n2;
            x.A1 = R12; x.lda1 = n2;
            x.B1 = D22; x.ldb1 = K;
            x.C = X; x.ldc = n2;
            x.flags = kGemmBUpper;
            x.strideA1 = Ts; x.strideB1 = strideH; x.strideC = Ts;
            TimerScope ts(stream, GPTQ_TIMER_FACTOR_GEMM);
            if (gemm_f32_pair(s, x, batch, stream) != hipSuccess) return GPTQ_ERR_HIP;
        }
        r = run(o, n1, T + n1 * n2);
        if (r != GPTQ_OK) return r;
        {   // U12 = -U11 X
            GemmArgs g;
            g.M = n1; g.N = n2; g.K1 = n1;
            g.A1 = D; g.lda1 = K;
            g.B1 = X; g.ldb1 = n2;
            g.C = H12; g.ldc = K;
            g.alpha = -1.f; g.beta = 0.f;
            g.flags = kGemmAUpper;
            if (gemm(g, strideH, Ts, strideH) != hipSuccess) return GPTQ_ERR_HIP;
        }
        return GPTQ_OK;
    }
};

}  // namespace

gptq_status_t prepare(float* H, int64_t K, int64_t batch, int64_t strideH, float percdamp, uint8_t* dead,
                      float* damp_out, int64_t* n_dead_out, void* workspace, hipStream_t stream) {
    Carver c(workspace);
    DevStatus* st = c.take<DevStatus>((size_t)batch);
    const int64_t Ts = (int64_t)batch_scratch_floats(K);
    float* T = c.take<float>((size_t)Ts * (size_t)batch);

    {
    TimerScope ts(stream, GPTQ_TIMER_OTHER);
    hipLaunchKernelGGL(clear_status_kernel, dim3(1), dim3(256), 0, stream, st, batch);
    hipLaunchKernelGGL(dead_damp_kernel, dim3((unsigned)batch), dim3(1024), 0, stream, H, K, strideH, percdamp, dead,
                       st);
    GPTQ_LAUNCH_CHECK();
    // Only the upper triangle of H is read.  The GEMMs treat the strictly lower parts of U blocks as stored
    // zeros, and no step writes below the diagonal outside the diagonal blocks (which the block kernel
    // clears), so clearing the lower triangle once keeps it zero throughout.
    hipLaunchKernelGGL(zero_lower_kernel, dim3((unsigned)K, (unsigned)batch), dim3(256), 0, stream, H, K, strideH);
    GPTQ_LAUNCH_CHECK();
    }

    Recursion rec{H, K, st, stream, batch, strideH, Ts};
    gptq_status_t r = rec.run(0, K, T);
    if (r != GPTQ_OK) return r;
    if (batch > 1) {   // the first status word reports every Hessian's errors (what gptq_device_status reads)
        TimerScope ts(stream, GPTQ_TIMER_OTHER);
        hipLaunchKernelGGL(merge_status_kernel, dim3(1), dim3(64), 0, stream, st, batch);
        GPTQ_LAUNCH_CHECK();
    }
    if (!damp_out && !n_dead_out) return GPTQ_OK;   // stream-ordered: errors stay latched for gptq_device_status

    std::vector<DevStatus> hst((size_t)batch);
    GPTQ_HIP_CHECK(hipMemcpyAsync(hst.data(), st, sizeof(DevStatus) * (size_t)batch, hipMemcpyDeviceToHost, stream));
    GPTQ_HIP_CHECK(hipStreamSynchronize(stream));
    uint32_t flags = 0;
    for (int64_t b = 0; b < batch; ++b) {
        if (damp_out) damp_out[b] = hst[b].damp;
        if (n_dead_out) n_dead_out[b] = hst[b].n_dead;
        flags |= hst[b].flags;
    }
    if (flags & kDevNonFinite) return GPTQ_ERR_NONFINITE;
    if (flags & kDevNotPD) return GPTQ_ERR_NOT_PD;
    return GPTQ_OK;
}

}  // namespace gptq
