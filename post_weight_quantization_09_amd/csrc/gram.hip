// Calibration Gram on gfx950 bf16 MFMA:  H += 2 Xs^T Xs  (and the asymmetric cross term A += 2 dX^T X).
//
// [T] section 1: the layer objective splits into one quadratic per output channel whose Hessian
// H = 2 X^T X is shared by all channels and accumulated batch by batch.  [R] item 3: asymmetric
// calibration reuses X^T X and adds the cross Gram (X~ - X)^T X.  [G]: each output-channel group owns a
// Hessian built from its own token weighting (row_scale).
//
// Design (256 threads, 4 waves, one 256 x 256 output tile per workgroup, 128 x 128 per wave):
//   * X is row-major (tokens x features), so both MFMA operands have the reduction index (tokens) as the
//     slow dimension.  A 32-token x 256-column slab of each operand is staged in LDS in its natural row
//     layout with 16-byte global loads (coalesced: 32 lanes read one 512-byte token row).
//   * Each lane reads 8 token rows x 4 columns (ds_read_b64) and transposes them in registers with
//     v_perm_b32 into four 8-token operand vectors, one per column.  Lane l of MFMA "a" then holds column
//     4*(l%32)+a over tokens 8*(l/32)..+7; A and B use the same token <-> (lane group, slot) map, so each
//     v_mfma_f32_32x32x16_bf16 sums over the same 16 tokens on both sides.  The column permutation is
//     undone when the result is written.
//   * Only tiles on or above the diagonal are computed (H is symmetric); the cross term computes all.
//   * The token range is split across workgroups when there are too few tiles to fill 256 CUs.  Splits are
//     assigned XCD by XCD (workgroup id mod 8) so that the workgroups sharing an XCD's L2 stream the same
//     tokens.  Each split writes its fp32 partial tile in register order (coalesced); a second kernel sums
//     the partials in a fixed order (deterministic, no float atomics), scales by 2, adds into H and writes
//     the mirrored lower triangle.
#include "gram.hpp"

#include <algorithm>

namespace gptq {

namespace {

constexpr int kGT = 256;      // output tile edge
constexpr int kGK = 32;       // tokens per LDS stage
constexpr int kGPitch = kGT;  // LDS row pitch in bf16 elements (512 B; all reads are row-contiguous)

__device__ inline int mfma32_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// Tile t -> (row block, column block): row-major over all nb x nb blocks (cross term) or over the upper
// triangle.  Out-of-range t gives bi = nb (callers return early).
__device__ inline void tile_coords(int t, int nb, bool full, int& bi, int& bj) {
    if (full) { bi = t / nb; bj = t % nb; return; }
    int b = 0, rem = t;
    while (b < nb && rem >= nb - b) { rem -= nb - b; ++b; }
    bi = b; bj = b + rem;
}

// Loads 8 consecutive bf16 (16 bytes) of row `tok`, columns [col, col+8), zero outside [0,M) x [0,K).
__device__ inline u32x4 load8(const uint16_t* X, int64_t ldx, int64_t tok, int64_t tokEnd, int64_t col, int64_t K,
                              bool vec) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (tok >= tokEnd || col >= K) return v;
    const uint16_t* p = X + tok * ldx + col;
    if (vec && col + 8 <= K) return *reinterpret_cast<const u32x4*>(p);
    uint16_t e[8];
    for (int i = 0; i < 8; ++i) e[i] = (col + i < K) ? p[i] : (uint16_t)0;
    for (int i = 0; i < 4; ++i) v[i] = (uint32_t)e[2 * i] | ((uint32_t)e[2 * i + 1] << 16);
    return v;
}

__device__ inline u32x4 scale_row_bf16(u32x4 v, float s) {
    u32x4 o;
    for (int i = 0; i < 4; ++i)
        o[i] = pack_bf16x2_rne(bf16lo_to_f32(v[i]) * s, bf16hi_to_f32(v[i]) * s);
    return o;
}

__device__ inline u32x4 diff_bf16(u32x4 xf, u32x4 x) {
    u32x4 o;
    for (int i = 0; i < 4; ++i)
        o[i] = pack_bf16x2_rne(bf16lo_to_f32(xf[i]) - bf16lo_to_f32(x[i]), bf16hi_to_f32(xf[i]) - bf16hi_to_f32(x[i]));
    return o;
}

// 8 rows (tokens) x 4 bf16 columns -> 4 column vectors of 8 tokens.
__device__ inline void transpose8x4(const u32x2 (&raw)[8], u32x4 (&out)[4]) {
    for (int s = 0; s < 4; ++s) {
        const uint32_t lo0 = raw[2 * s].x, lo1 = raw[2 * s + 1].x;   // columns 0,1
        const uint32_t hi0 = raw[2 * s].y, hi1 = raw[2 * s + 1].y;   // columns 2,3
        out[0][s] = __builtin_amdgcn_perm(lo1, lo0, 0x05040100u);
        out[1][s] = __builtin_amdgcn_perm(lo1, lo0, 0x07060302u);
        out[2][s] = __builtin_amdgcn_perm(hi1, hi0, 0x05040100u);
        out[3][s] = __builtin_amdgcn_perm(hi1, hi0, 0x07060302u);
    }
}

template <bool CROSS, bool SCALED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gram_bf16_kernel(GramArgs p) {
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][kGK][kGPitch];
    __shared__ __attribute__((aligned(16))) uint16_t sB[2][kGK][kGPitch];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wi = wave >> 1, wj = wave & 1;

    int split, tile;
    const int bid = blockIdx.x;
    if (p.splits % 8 == 0) {
        const int x = bid & 7, q = bid >> 3, per = p.splits / 8;
        split = x * per + q / p.ntiles;
        tile = q % p.ntiles;
    } else {
        split = bid / p.ntiles;
        tile = bid % p.ntiles;
    }
    int bi, bj;
    tile_coords(tile, p.nb, CROSS, bi, bj);
    if (bi >= p.nb || bj >= p.nb || split >= p.splits) return;   // whole workgroup, before any barrier
    const bool same = !CROSS && bi == bj;       // diagonal tile: quadrant (1,0) mirrors (0,1)
    const bool active = !(same && wi == 1 && wj == 0);
    const int64_t colA = (int64_t)bi * kGT, colB = (int64_t)bj * kGT;
    const int64_t t0 = (int64_t)split * p.tokens_per_split;
    const int64_t t1 = min<int64_t>(p.M, t0 + p.tokens_per_split);
    const int64_t nst = t1 > t0 ? ceil_div(t1 - t0, kGK) : 0;

    f32x16 acc[4][4];
    for (int a = 0; a < 4; ++a)
        for (int b = 0; b < 4; ++b)
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

    // Prefetch registers: 4 chunks of 16 bytes per side per thread.
    u32x4 ra[4], rb[4];
    auto gload = [&](int64_t st) {
        const int64_t tb = t0 + st * kGK;
        for (int i = 0; i < 4; ++i) {
            const int c = tid + 256 * i;
            const int tr = c >> 5, cc = c & 31;
            const int64_t tok = tb + tr;
            u32x4 x = load8(p.X, p.ldx, tok, t1, colA + cc * 8, p.K, p.vec);
            if (CROSS) {
                u32x4 xf = load8(p.Xf, p.ldxf, tok, t1, colA + cc * 8, p.K, p.vec);
                ra[i] = diff_bf16(xf, x);
                rb[i] = load8(p.X, p.ldx, tok, t1, colB + cc * 8, p.K, p.vec);
            } else {
                if (SCALED) {
                    const float s = tok < t1 ? p.rho[tok] : 0.f;
                    x = scale_row_bf16(x, s);
                }
                ra[i] = x;
                u32x4 y = load8(p.X, p.ldx, tok, t1, colB + cc * 8, p.K, p.vec);
                if (SCALED) {
                    const float s = tok < t1 ? p.rho[tok] : 0.f;
                    y = scale_row_bf16(y, s);
                }
                rb[i] = y;
            }
        }
    };
    auto lstore = [&](int buf) {
        for (int i = 0; i < 4; ++i) {
            const int c = tid + 256 * i;
            const int tr = c >> 5, cc = c & 31;
            *reinterpret_cast<u32x4*>(&sA[buf][tr][cc * 8]) = ra[i];
            *reinterpret_cast<u32x4*>(&sB[buf][tr][cc * 8]) = rb[i];
        }
    };

    if (nst > 0) {
        gload(0);
        lstore(0);
    }
    __syncthreads();
    const int g = lane >> 5, r32 = lane & 31;
    for (int64_t st = 0; st < nst; ++st) {
        const int buf = (int)(st & 1);
        if (st + 1 < nst) gload(st + 1);
        {
            const uint16_t(*pA)[kGPitch] = sA[buf];
            const uint16_t(*pB)[kGPitch] = sB[buf];
#pragma unroll
            for (int ks = 0; ks < kGK / 16; ++ks) {
                u32x2 rawA[8], rawB[8];
                const int trow = ks * 16 + 8 * g;
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    rawA[s] = *reinterpret_cast<const u32x2*>(&pA[trow + s][wi * 128 + 4 * r32]);
                    rawB[s] = *reinterpret_cast<const u32x2*>(&pB[trow + s][wj * 128 + 4 * r32]);
                }
                u32x4 va[4], vb[4];
                transpose8x4(rawA, va);
                transpose8x4(rawB, vb);
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const bf16x8 av = __builtin_bit_cast(bf16x8, va[a]);
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const bf16x8 bv = __builtin_bit_cast(bf16x8, vb[b]);
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[a][b], 0, 0, 0);
                    }
                }
            }
        }
        if (st + 1 < nst) lstore(buf ^ 1);
        __syncthreads();
    }

    if (!active) return;
    float* out = p.partial + (((int64_t)split * p.ntiles + tile) * 4 + wave) * (256 * 64);
    for (int a = 0; a < 4; ++a)
        for (int b = 0; b < 4; ++b)
            for (int r = 0; r < 16; ++r) out[((a * 4 + b) * 16 + r) * 64 + lane] = acc[a][b][r];
}

// Sums the split partials of one 128 x 128 quadrant in split order, scales by 2 and adds into the output
// (H, mirrored for off-diagonal quadrants; or the cross Gram, not mirrored).
template <bool CROSS>
__global__ __launch_bounds__(256) void gram_reduce_kernel(GramArgs p, float* Out) {
    __shared__ float T[128][129];
    const int tid = threadIdx.x;
    const int tile = blockIdx.x >> 2, wave = blockIdx.x & 3;
    const int wi = wave >> 1, wj = wave & 1;
    int bi, bj;
    tile_coords(tile, p.nb, CROSS, bi, bj);
    if (bi >= p.nb || bj >= p.nb) return;
    const bool same = !CROSS && bi == bj;
    if (same && wi == 1 && wj == 0) return;
    const bool mirror = !CROSS && !(same && wi == wj);
    const int64_t R0 = (int64_t)bi * kGT + wi * 128, C0 = (int64_t)bj * kGT + wj * 128;

    const int lane = tid & 63, rg = tid >> 6;
    const int64_t qstride = (int64_t)p.ntiles * 4 * 256 * 64;
    const float* base = p.partial + ((int64_t)tile * 4 + wave) * (256 * 64);
    for (int k = 0; k < 64; ++k) {
        const int ri = rg * 64 + k;
        float s = 0.f;
        for (int sp = 0; sp < p.splits; ++sp) s += base[sp * qstride + ri * 64 + lane];
        const int a = ri >> 6, b = (ri >> 4) & 3, r = ri & 15;
        const int row = 4 * mfma32_row(r, lane) + a;
        const int col = 4 * (lane & 31) + b;
        T[row][col] = 2.0f * s;
    }
    __syncthreads();
    for (int i = 0; i < 64; ++i) {
        const int idx = tid + 256 * i;
        const int row = idx >> 7, col = idx & 127;
        if (R0 + row < p.K && C0 + col < p.K) {
            float* o = Out + (R0 + row) * p.K + C0 + col;
            *o += T[row][col];
        }
        if (mirror && C0 + row < p.K && R0 + col < p.K) {
            float* o = Out + (C0 + row) * p.K + R0 + col;
            *o += T[col][row];
        }
    }
}

}  // namespace

GramPlan gram_plan(int64_t K, int64_t M, bool cross) {
    GramPlan pl;
    pl.cross = cross;
    pl.nb = (int)ceil_div(K, kGT);
    pl.ntiles = cross ? pl.nb * pl.nb : pl.nb * (pl.nb + 1) / 2;
    // Enough workgroups for ~8 rounds over 256 CUs, with at least 4096 tokens per split.
    int64_t s = 1;
    if (pl.ntiles < 2048) {
        s = ceil_div(2048, pl.ntiles);
        if (s >= 8) s = ceil_div(s, 8) * 8;
        const int64_t cap = std::max<int64_t>(1, M / 4096);
        if (s > cap) s = cap >= 8 ? (cap / 8) * 8 : cap;
    }
    pl.splits = (int)std::max<int64_t>(1, s);
    pl.tokens_per_split = ceil_div(ceil_div(std::max<int64_t>(M, 1), pl.splits), kGK) * kGK;
    pl.partial_floats = (size_t)pl.splits * pl.ntiles * 4 * 256 * 64;
    return pl;
}

hipError_t gram_bf16(const GramPlan& pl, const uint16_t* X, int64_t ldx, const uint16_t* Xf, int64_t ldxf,
                     const float* rho, int64_t M, int64_t K, float* partial, float* Out, hipStream_t stream) {
    if (M <= 0) return hipSuccess;
    const bool cross = Xf != nullptr;
    if (pl.cross != cross) return hipErrorInvalidValue;     // the plan's tile count is mode specific
    GramArgs p;
    p.X = X; p.ldx = ldx; p.Xf = Xf; p.ldxf = ldxf; p.rho = rho; p.M = M; p.K = K;
    p.nb = pl.nb; p.ntiles = pl.ntiles; p.splits = pl.splits; p.tokens_per_split = pl.tokens_per_split;
    p.partial = partial;
    auto al16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
    p.vec = al16(X) && ldx % 8 == 0 && (!cross || (al16(Xf) && ldxf % 8 == 0));
    const unsigned nblk = (unsigned)((int64_t)pl.ntiles * pl.splits);
    if (cross) hipLaunchKernelGGL((gram_bf16_kernel<true, false>), dim3(nblk), dim3(256), 0, stream, p);
    else if (rho) hipLaunchKernelGGL((gram_bf16_kernel<false, true>), dim3(nblk), dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((gram_bf16_kernel<false, false>), dim3(nblk), dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned nred = (unsigned)(pl.ntiles * 4);
    if (cross) hipLaunchKernelGGL((gram_reduce_kernel<true>), dim3(nred), dim3(256), 0, stream, p, Out);
    else hipLaunchKernelGGL((gram_reduce_kernel<false>), dim3(nred), dim3(256), 0, stream, p, Out);
    return hipGetLastError();
}

}  // namespace gptq
