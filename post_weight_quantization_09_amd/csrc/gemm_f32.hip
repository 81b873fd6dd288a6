// fp32 MFMA GEMM for gfx950: C = beta*C + alpha*(A1 B1 + a2_scale * A2 B2), optionally batched.
//
// Every dense contraction of the path runs here: the trailing updates of the blocked factorisation, the
// merges of the triangular inverse, the lazy-batch trailing update of the column loop ([T] section 5:
// after a block, the far weights are updated with one matrix product) and the two products of the GPTAQ
// correction ([R] item 3).
//
// Tiling: 256 threads = 4 waves in 2 x 2, a 64 x 64 tile of C per workgroup, each wave 32 x 32 as a
// v_mfma_f32_32x32x2_f32 accumulator.  k advances TK = 16 at a time through double-buffered LDS tiles stored
// k-major (As[k][m], Bs[k][n]) so that every MFMA operand read is a conflict-free ds_read_b32.  Large products
// with a long reduction take the split-bf16 kernel below (128 x 128 tiles, same structure flags and epilogue).
#include "gemm_f32.hpp"

#include <type_traits>

namespace gptq {

namespace {

constexpr int kPad = 4;

// MFMA 32x32x2 f32 output layout: lane l, accumulator register r -> (row, col) inside the 32 x 32 block.
__device__ inline int mfma32_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// Tile configuration: TM x TN outputs per workgroup (4 waves in 2 x 2, each (TM/2) x (TN/2) as 32 x 32 MFMA
// blocks), TK reduction steps per LDS stage.
template <int TM, int TN, int TK>
struct Tile {
    static constexpr int MA = TM / 64, NB = TN / 64;       // 32 x 32 blocks per wave along m and n
    static constexpr int NVA = TM * TK / 1024;             // f32x4 loads per thread for the A tile
    static constexpr int NVB = TN * TK / 1024;
    static_assert(TM % 64 == 0 && TN % 64 == 0 && TK % 4 == 0 && NVA >= 1 && NVB >= 1, "tile shape");
};

template <int TM, int TN, int TK, bool TA, bool TB, bool FULL>
struct TileIO {
    using T = Tile<TM, TN, TK>;
    // A(m,k): TA ? A[k*lda + m] : A[m*lda + k].   B(k,n): TB ? B[n*ldb + k] : B[k*ldb + n].
    // Raw values only: the scale and the triangular mask are applied when the tile is written to LDS, so no
    // arithmetic waits on an outstanding load.  FULL: the tile is entirely in range and 16-byte aligned.
    f32x4 a[T::NVA], b[T::NVB];
    float a_scale;
    bool a_mask;
    int64_t am0, ak0;   // A tile origin (for the mask)

    // Element (m, k) of the i-th A vector of thread tid (relative to the tile origin); the vector runs along
    // k (not TA) or along m (TA).
    __device__ static inline void a_pos(int i, int tid, int& m, int& k) {
        if (!TA) { constexpr int C = TK / 4; m = tid / C + (256 / C) * i; k = (tid % C) * 4; }
        else     { constexpr int C = TM / 4; k = tid / C + (256 / C) * i; m = (tid % C) * 4; }
    }
    __device__ static inline void b_pos(int i, int tid, int& n, int& k) {
        if (!TB) { constexpr int C = TN / 4; k = tid / C + (256 / C) * i; n = (tid % C) * 4; }
        else     { constexpr int C = TK / 4; n = tid / C + (256 / C) * i; k = (tid % C) * 4; }
    }

    __device__ static inline f32x4 load4(const float* base, int64_t idx0, int valid, bool vec) {
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (valid >= 4 && vec) {
            v = *reinterpret_cast<const f32x4*>(base + idx0);
        } else {
            for (int e = 0; e < 4; ++e)
                if (e < valid) v[e] = base[idx0 + e];
        }
        return v;
    }

    __device__ inline void load_a(const float* A, int64_t lda, int64_t M, int64_t kEnd, int64_t m0, int64_t k0,
                                  bool vec, float scale, bool strict_upper_mask, int tid) {
        a_scale = scale;
        a_mask = strict_upper_mask;
        am0 = m0;
        ak0 = k0;
#pragma unroll
        for (int i = 0; i < T::NVA; ++i) {
            int mi, ki;
            a_pos(i, tid, mi, ki);
            const int64_t m = m0 + mi, k = k0 + ki;
            if (FULL) {
                a[i] = *reinterpret_cast<const f32x4*>(A + (TA ? k * lda + m : m * lda + k));
                continue;
            }
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (!TA) {
                if (m < M && k < kEnd) v = load4(A, m * lda + k, (int)min<int64_t>(4, kEnd - k), vec);
            } else {
                if (k < kEnd && m < M) v = load4(A, k * lda + m, (int)min<int64_t>(4, M - m), vec);
            }
            a[i] = v;
        }
    }

    __device__ inline void load_b(const float* B, int64_t ldb, int64_t N, int64_t kEnd, int64_t n0, int64_t k0,
                                  bool vec, int tid) {
#pragma unroll
        for (int i = 0; i < T::NVB; ++i) {
            int ni, ki;
            b_pos(i, tid, ni, ki);
            const int64_t n = n0 + ni, k = k0 + ki;
            if (FULL) {
                b[i] = *reinterpret_cast<const f32x4*>(B + (TB ? n * ldb + k : k * ldb + n));
                continue;
            }
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (!TB) {
                if (k < kEnd && n < N) v = load4(B, k * ldb + n, (int)min<int64_t>(4, N - n), vec);
            } else {
                if (n < N && k < kEnd) v = load4(B, n * ldb + k, (int)min<int64_t>(4, kEnd - k), vec);
            }
            b[i] = v;
        }
    }

    __device__ inline void store(float (*As)[TM + kPad], float (*Bs)[TN + kPad], int tid) const {
#pragma unroll
        for (int i = 0; i < T::NVA; ++i) {
            int mi, ki;
            a_pos(i, tid, mi, ki);
            f32x4 va = a[i] * a_scale;
            if (a_mask) {
                for (int e = 0; e < 4; ++e) {
                    const int64_t me = am0 + mi + (TA ? e : 0), ke = ak0 + ki + (TA ? 0 : e);
                    if (ke <= me) va[e] = 0.f;
                }
            }
            if (!TA) {
                for (int e = 0; e < 4; ++e) As[ki + e][mi] = va[e];
            } else {
                *reinterpret_cast<f32x4*>(&As[ki][mi]) = va;
            }
        }
#pragma unroll
        for (int i = 0; i < T::NVB; ++i) {
            int ni, ki;
            b_pos(i, tid, ni, ki);
            if (!TB) {
                *reinterpret_cast<f32x4*>(&Bs[ki][ni]) = b[i];
            } else {
                for (int e = 0; e < 4; ++e) Bs[ki + e][ni] = b[i][e];
            }
        }
    }
};

// One output tile of a product: block (bx, by) of a gx x gy tile grid, batch element bz, with the workgroup's
// LDS tiles passed in.
template <int TM, int TN, int TK, bool TA, bool TB, bool FULL>
__device__ __forceinline__ void gemm_f32_tile(const GemmArgs& p, int64_t bx, int64_t by, int64_t gx, int64_t gy,
                                              int64_t bz, float (*As)[TK][TM + kPad], float (*Bs)[TK][TN + kPad]) {
    using T = Tile<TM, TN, TK>;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    // Tile order.  With a triangular B the work of a tile depends on its column only (k from n0 for B lower, up
    // to n0 + TN for B upper): tiles are dispatched column by column, heaviest column first, so that the last
    // workgroups to start are the shortest (25-35% faster than row order on these products).
    int64_t tx = bx, ty = by;
    if (p.flags & (kGemmBLower | kGemmBUpper)) {
        const int64_t id = by * gx + bx;
        tx = id / gy;
        ty = id % gy;
        if (p.flags & kGemmBUpper) tx = gx - 1 - tx;
    }
    const int64_t m0 = ty * TM;
    const int64_t n0 = tx * TN;
    if (m0 >= p.M || n0 >= p.N) return;
    if ((p.flags & kGemmCUpper) && m0 >= n0 + TN) return;

    const float* A1 = p.A1 + bz * p.strideA1;
    const float* B1 = p.B1 + bz * p.strideB1;
    const float* A2 = p.A2 ? p.A2 + bz * p.strideA2 : nullptr;
    const float* B2 = p.B2 ? p.B2 + bz * p.strideB2 : nullptr;
    float* C = p.C + bz * p.strideC;

    int64_t klo = 0, khi = p.K1;
    if (p.flags & (kGemmAUpper | kGemmAStrictUpperMask)) klo = max<int64_t>(klo, m0);
    if (p.flags & kGemmBLower) klo = max<int64_t>(klo, n0);
    if (p.flags & kGemmBUpper) khi = min<int64_t>(khi, n0 + TN);
    klo = (klo / TK) * TK;
    const int64_t nt1 = khi > klo ? ceil_div(khi - klo, TK) : 0;
    const int64_t nt2 = (A2 && p.K2 > 0) ? ceil_div(p.K2, TK) : 0;
    const int64_t nt = nt1 + nt2;
    const bool mask = (p.flags & kGemmAStrictUpperMask) != 0;

    f32x16 acc[T::MA][T::NB];
    for (int a = 0; a < T::MA; ++a)
        for (int b = 0; b < T::NB; ++b)
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

    // Stage t (TK values of k) is loaded into registers kD - 1 stages ahead of its product, written to the LDS
    // buffer t & 1 one stage ahead, and multiplied after a barrier.  The loop is unrolled by kD so that every
    // register slot index is a constant; loads past the last stage re-read it (never stored), which keeps the
    // loop free of branches around loads.
    constexpr int kD = 4;
    using IO = TileIO<TM, TN, TK, TA, TB, FULL>;
    IO io[kD];
    auto load = [&](IO& x, int64_t t) {
        if (t < nt1) {
            int64_t k0 = klo + t * TK;
            x.load_a(A1, p.lda1, p.M, p.K1, m0, k0, p.vecA1, 1.0f, mask, tid);
            x.load_b(B1, p.ldb1, p.N, p.K1, n0, k0, p.vecB1, tid);
        } else {
            int64_t k0 = (t - nt1) * TK;
            x.load_a(A2, p.lda2, p.M, p.K2, m0, k0, p.vecA2, p.a2_scale, false, tid);
            x.load_b(B2, p.ldb2, p.N, p.K2, n0, k0, p.vecB2, tid);
        }
    };

    if (nt > 0) {
#pragma unroll
        for (int s = 0; s < kD - 1; ++s) load(io[s], min<int64_t>(s, nt - 1));
        io[0].store(As[0], Bs[0], tid);
    }
    __syncthreads();
    for (int64_t t0 = 0; t0 < nt; t0 += kD) {
#pragma unroll
        for (int u = 0; u < kD; ++u) {
            const int64_t t = t0 + u;
            if (t >= nt) break;
            const int buf = u & 1;   // t0 is even
            load(io[(u + kD - 1) % kD], min<int64_t>(t + kD - 1, nt - 1));
#pragma unroll
            for (int kk = 0; kk < TK / 2; ++kk) {
                const int k = 2 * kk + (lane >> 5);
                float av[T::MA], bv[T::NB];
                for (int a = 0; a < T::MA; ++a) av[a] = As[buf][k][wm * (TM / 2) + 32 * a + (lane & 31)];
                for (int b = 0; b < T::NB; ++b) bv[b] = Bs[buf][k][wn * (TN / 2) + 32 * b + (lane & 31)];
                for (int a = 0; a < T::MA; ++a)
                    for (int b = 0; b < T::NB; ++b)
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[a], bv[b], acc[a][b], 0, 0, 0);
            }
            if (t + 1 < nt) io[(u + 1) % kD].store(As[buf ^ 1], Bs[buf ^ 1], tid);
            __syncthreads();
        }
    }

    // Epilogue: C = alpha * acc + beta * C.
    for (int a = 0; a < T::MA; ++a) {
        for (int b = 0; b < T::NB; ++b) {
            const int64_t col = n0 + wn * (TN / 2) + 32 * b + (lane & 31);
            if (col >= p.N) continue;
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + wm * (TM / 2) + 32 * a + mfma32_row(r, lane);
                if (row >= p.M) continue;
                float* cp = C + row * p.ldc + col;
                float v = p.alpha * acc[a][b][r];
                if (p.beta != 0.f) v += p.beta * *cp;
                *cp = v;
            }
        }
    }
}

template <int TM, int TN, int TK, bool TA, bool TB, bool FULL>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs p) {
    __shared__ __attribute__((aligned(16))) float As[2][TK][TM + kPad];
    __shared__ __attribute__((aligned(16))) float Bs[2][TK][TN + kPad];
    gemm_f32_tile<TM, TN, TK, TA, TB, FULL>(p, blockIdx.x, blockIdx.y, gridDim.x, gridDim.y, blockIdx.z, As, Bs);
}

// Two independent products in one launch (64 x 64 tiles): the first gx1 * gy1 workgroups of each batch element
// take the tiles of p1 (B transposed), the rest those of p2 (neither transposed).  Each tile is computed
// exactly as by gemm_f32_kernel.
template <bool FULL1, bool FULL2>
__global__ __launch_bounds__(256) void gemm_f32_pair_kernel(GemmArgs p1, GemmArgs p2, int gx1, int gy1, int gx2,
                                                            int gy2) {
    __shared__ __attribute__((aligned(16))) float As[2][16][64 + kPad];
    __shared__ __attribute__((aligned(16))) float Bs[2][16][64 + kPad];
    const int64_t id = blockIdx.x, n1 = (int64_t)gx1 * gy1;
    if (id < n1) {
        gemm_f32_tile<64, 64, 16, false, true, FULL1>(p1, id % gx1, id / gx1, gx1, gy1, blockIdx.z, As, Bs);
    } else {
        const int64_t j = id - n1;
        gemm_f32_tile<64, 64, 16, false, false, FULL2>(p2, j % gx2, j / gx2, gx2, gy2, blockIdx.z, As, Bs);
    }
}

// ---- fp32-accurate products on the bf16 MFMA: every fp32 operand is split into three bf16 parts
// (v = h0 + h1 + h2 + O(2^-24 |v|), each part the round-to-nearest-even bf16 of the remainder), and the six
// part products of order <= 2 are accumulated in fp32 by v_mfma_f32_32x32x16_bf16.  Part planes are stored
// k-contiguous (row pitch 24 bf16 = 48 bytes), so a lane's 8 k-values are one conflict-free 16-byte LDS read.
constexpr int kXP = 24;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
// The parts of two consecutive k-values at once (one packed conversion per part); word q holds part q of
// `lo` in its low half and of `hi` in its high half.
__device__ inline void split3x2(float lo, float hi, uint32_t& w0, uint32_t& w1, uint32_t& w2) {
    const f32x2_t v = {lo, hi};
    const bf16x2_t b0 = __builtin_convertvector(v, bf16x2_t);
    const f32x2_t r1 = v - __builtin_convertvector(b0, f32x2_t);
    const bf16x2_t b1 = __builtin_convertvector(r1, bf16x2_t);
    const f32x2_t r2 = r1 - __builtin_convertvector(b1, f32x2_t);
    const bf16x2_t b2 = __builtin_convertvector(r2, bf16x2_t);
    w0 = __builtin_bit_cast(uint32_t, b0);
    w1 = __builtin_bit_cast(uint32_t, b1);
    w2 = __builtin_bit_cast(uint32_t, b2);
}

template <int TM, int TN, int TK, bool TA, bool TB, bool FULL>
__global__ __launch_bounds__(256) void gemm_x6_kernel(GemmArgs p) {
    using T = Tile<TM, TN, TK>;
    static_assert(TK == 16, "one 32x32x16 MFMA k-step per stage");
    static_assert(TM % 128 == 0 && TN % 128 == 0, "strided operands are loaded 128 rows per pass");
    __shared__ __attribute__((aligned(16))) uint16_t As[2][3][TM][kXP];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][3][TN][kXP];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    int64_t tx = blockIdx.x, ty = blockIdx.y;
    if (p.flags & (kGemmBLower | kGemmBUpper)) {
        const int64_t id = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
        tx = id / gridDim.y;
        ty = id % gridDim.y;
        if (p.flags & kGemmBUpper) tx = gridDim.x - 1 - tx;
    }
    const int64_t m0 = ty * TM;
    const int64_t n0 = tx * TN;
    const int64_t bz = blockIdx.z;
    if (m0 >= p.M || n0 >= p.N) return;
    if ((p.flags & kGemmCUpper) && m0 >= n0 + TN) return;

    const float* A1 = p.A1 + bz * p.strideA1;
    const float* B1 = p.B1 + bz * p.strideB1;
    const float* A2 = p.A2 ? p.A2 + bz * p.strideA2 : nullptr;
    const float* B2 = p.B2 ? p.B2 + bz * p.strideB2 : nullptr;
    float* C = p.C + bz * p.strideC;

    int64_t klo = 0, khi = p.K1;
    if (p.flags & (kGemmAUpper | kGemmAStrictUpperMask)) klo = max<int64_t>(klo, m0);
    if (p.flags & kGemmBLower) klo = max<int64_t>(klo, n0);
    if (p.flags & kGemmBUpper) khi = min<int64_t>(khi, n0 + TN);
    klo = (klo / TK) * TK;
    const int64_t nt1 = khi > klo ? ceil_div(khi - klo, TK) : 0;
    const int64_t nt2 = (A2 && p.K2 > 0) ? ceil_div(p.K2, TK) : 0;
    const int64_t nt = nt1 + nt2;
    const bool mask = (p.flags & kGemmAStrictUpperMask) != 0;

    f32x16 acc[T::MA][T::NB];
#pragma unroll
    for (int a = 0; a < T::MA; ++a)
#pragma unroll
        for (int b = 0; b < T::NB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

    // Raw global data of one stage, held in registers from its load to its split-and-store two stages later; two
    // such sets (stages of even and odd index).  Operands whose k index is strided in memory (A with TA, B without
    // TB) are loaded as single floats: thread t takes row/column t % 128 and the 8 consecutive k of group t / 128
    // (a 256-row tile takes two such passes), so each load instruction is coalesced along the contiguous index and
    // each thread ends with k-contiguous values for its planes.
    constexpr int SA = TA ? TM / 128 : 1, SB = TB ? 1 : TN / 128;
    struct Staged {
        TileIO<TM, TN, TK, TA, TB, FULL> io;
        float sa[SA][8], sb[SB][8];
        float sa_scale;
    };
    Staged S0, S1;
    auto load_strided = [&](const float* X, int64_t ldx, int64_t rows, int64_t kEnd, int64_t r0, int64_t k0,
                            bool strict_upper, float (*dst)[8], int passes) {
        const int r = tid & 127, kq = tid >> 7;
#pragma unroll
        for (int ps = 0; ps < passes; ++ps) {
            const int64_t row = r0 + 128 * ps + r;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int64_t kk = k0 + 8 * kq + e;
                float v = (FULL || (row < rows && kk < kEnd)) ? X[kk * ldx + row] : 0.f;
                if (strict_upper && kk <= row) v = 0.f;
                dst[ps][e] = v;
            }
        }
    };
    auto load = [&](int64_t t, Staged& S) {
        const bool second = t >= nt1;
        const int64_t k0 = second ? (t - nt1) * TK : klo + t * TK;
        const float* Ap = second ? A2 : A1; const float* Bp = second ? B2 : B1;
        const int64_t ldA = second ? p.lda2 : p.lda1, ldB = second ? p.ldb2 : p.ldb1;
        const int64_t kEnd = second ? p.K2 : p.K1;
        if constexpr (TA) {
            load_strided(Ap, ldA, p.M, kEnd, m0, k0, second ? false : mask, S.sa, SA);
            S.sa_scale = second ? p.a2_scale : 1.f;
        } else {
            S.io.load_a(Ap, ldA, p.M, kEnd, m0, k0, second ? p.vecA2 : p.vecA1, second ? p.a2_scale : 1.0f,
                        second ? false : mask, tid);
        }
        if constexpr (TB) S.io.load_b(Bp, ldB, p.N, kEnd, n0, k0, second ? p.vecB2 : p.vecB1, tid);
        else load_strided(Bp, ldB, p.N, kEnd, n0, k0, false, S.sb, SB);
    };
    // Split-and-store pieces of a staged stage into LDS buffer `buf`: first the A pieces (one per 16-byte vector,
    // or one per 128-row pass of a strided A), then the B pieces likewise.
    constexpr int kPA = TA ? SA : T::NVA, kPB = TB ? T::NVB : SB, kPieces = kPA + kPB;
    auto store_piece = [&](const Staged& S, int buf, int piece) {
        if (piece < kPA) {
            if constexpr (TA) {
                const int r = tid & 127, kq = tid >> 7, ps = piece;
                uint32_t w[3][4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    split3x2(S.sa[ps][2 * e] * S.sa_scale, S.sa[ps][2 * e + 1] * S.sa_scale, w[0][e], w[1][e], w[2][e]);
#pragma unroll
                for (int q = 0; q < 3; ++q)
                    *reinterpret_cast<u32x4*>(&As[buf][q][128 * ps + r][8 * kq]) = u32x4{w[q][0], w[q][1], w[q][2], w[q][3]};
            } else {
                const int i = piece;
                int mi, ki;
                S.io.a_pos(i, tid, mi, ki);
                f32x4 va = S.io.a[i] * S.io.a_scale;
                {   // strict-upper mask as selects (no branch inside the pinned schedule)
                    const int d = (int)(S.io.ak0 - S.io.am0) + ki - mi;   // k - m of element 0 (|k - m| < 2^31)
#pragma unroll
                    for (int e = 0; e < 4; ++e) va[e] = (S.io.a_mask && d + e <= 0) ? 0.f : va[e];
                }
                uint32_t w[3][2];
#pragma unroll
                for (int e = 0; e < 2; ++e) split3x2(va[2 * e], va[2 * e + 1], w[0][e], w[1][e], w[2][e]);
#pragma unroll
                for (int q = 0; q < 3; ++q) *reinterpret_cast<u32x2*>(&As[buf][q][mi][ki]) = u32x2{w[q][0], w[q][1]};
            }
        } else {
            const int pb = piece - kPA;
            if constexpr (TB) {
                int ni, ki;
                S.io.b_pos(pb, tid, ni, ki);
                const f32x4 vb = S.io.b[pb];
                uint32_t w[3][2];
#pragma unroll
                for (int e = 0; e < 2; ++e) split3x2(vb[2 * e], vb[2 * e + 1], w[0][e], w[1][e], w[2][e]);
#pragma unroll
                for (int q = 0; q < 3; ++q) *reinterpret_cast<u32x2*>(&Bs[buf][q][ni][ki]) = u32x2{w[q][0], w[q][1]};
            } else {
                const int r = tid & 127, kq = tid >> 7, ps = pb;
                uint32_t w[3][4];
#pragma unroll
                for (int e = 0; e < 4; ++e) split3x2(S.sb[ps][2 * e], S.sb[ps][2 * e + 1], w[0][e], w[1][e], w[2][e]);
#pragma unroll
                for (int q = 0; q < 3; ++q)
                    *reinterpret_cast<u32x4*>(&Bs[buf][q][128 * ps + r][8 * kq]) = u32x4{w[q][0], w[q][1], w[q][2], w[q][3]};
            }
        }
    };
    auto store_all = [&](const Staged& S, int buf) {
#pragma unroll
        for (int pc = 0; pc < kPieces; ++pc) store_piece(S, buf, pc);
    };
    // Fragments of one stage: plane q of A block a and of B block b (a lane's 8 k-values, one 16-byte read each).
    constexpr int kFrag = 3 * (T::MA + T::NB);
    struct Frags { u32x4 a[3][T::MA], b[3][T::NB]; };
    const int kk = 8 * (lane >> 5);
    auto read_frag = [&](Frags& F, int buf, int f) {
        const int q = f / (T::MA + T::NB), j = f % (T::MA + T::NB);
        if (j < T::MA)
            F.a[q][j] = *reinterpret_cast<const u32x4*>(&As[buf][q][wm * (TM / 2) + 32 * j + (lane & 31)][kk]);
        else
            F.b[q][j - T::MA] = *reinterpret_cast<const u32x4*>(&Bs[buf][q][wn * (TN / 2) + 32 * (j - T::MA) + (lane & 31)][kk]);
    };
    auto read_all = [&](Frags& F, int buf) {
#pragma unroll
        for (int f = 0; f < kFrag; ++f) read_frag(F, buf, f);
    };
    // MFMA i of a stage: block (a, b) = (i / 6) / NB, (i / 6) % NB; part products small parts first.
    constexpr int kMfma = 6 * T::MA * T::NB;
    auto mfma = [&](const Frags& F, int i) {
        const int blk = i / 6, part = i % 6, a = blk / T::NB, b = blk % T::NB;
        constexpr int qa[6] = {2, 1, 0, 1, 0, 0}, qb[6] = {0, 1, 2, 0, 1, 0};
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, F.a[qa[part]][a]),
                                                           __builtin_bit_cast(bf16x8, F.b[qb[part]][b]), acc[a][b], 0, 0, 0);
    };

    // Software pipeline over stages t (LDS buffer t & 1, staging set t & 1):
    //   stage t is loaded from global in iteration t-4 (prologue for t < 4), split and stored to LDS in iteration
    //   t-2, read into fragments in iteration t-1 and multiplied in iteration t; one barrier per iteration.
    //   Iteration t: [MFMAs of stage t || stores of stage t+2 (staged in set t & 1) into buffer t & 1, then the
    //   loads of stage t+4 into that set; fragment reads of stage t+1 from buffer (t+1) & 1]  barrier
    // Each MFMA is followed by a fixed share of that work, pinned with scheduling barriers: the split-and-store
    // pieces after the first MFMAs, the 12 fragment reads after MFMAs 4-15, the loads after MFMA 16.  Against the
    // previous loop (one stage loaded, split and stored per iteration around a block of 24 MFMAs, results
    // bit-identical) the far trailing products of the 28672 x 8192 layer take 44.5 instead of 47.0 ms.
    Frags F0, F1;
    auto iter_steady = [&](auto Qc, int64_t t) {
        constexpr int Q = decltype(Qc)::value;
        Frags& Fc = Q ? F1 : F0;
        Frags& Fn = Q ? F0 : F1;
        Staged& Sq = Q ? S1 : S0;
#pragma unroll
        for (int i = 0; i < kMfma; ++i) {
            mfma(Fc, i);
            if (i < kPieces) store_piece(Sq, Q, i);
            if (i >= 4 && i < 4 + kFrag) read_frag(Fn, Q ^ 1, i - 4);
            if (i == 4 + kFrag) load(t + 4, Sq);
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
    };
    auto iter_drain = [&](auto Qc, int64_t t) {
        constexpr int Q = decltype(Qc)::value;
        Frags& Fc = Q ? F1 : F0;
        Frags& Fn = Q ? F0 : F1;
        Staged& Sq = Q ? S1 : S0;
#pragma unroll
        for (int i = 0; i < kMfma; ++i) mfma(Fc, i);
        if (t + 2 < nt) store_all(Sq, Q);
        if (t + 4 < nt) load(t + 4, Sq);
        if (t + 1 < nt) read_all(Fn, Q ^ 1);
        __syncthreads();
    };
    if (nt > 5) {
        // unconditional prologue, so that the order of the loads in flight is known at the loop entry
        load(0, S0);
        load(1, S1);
        store_all(S0, 0);
        load(2, S0);
        __syncthreads();
        read_all(F0, 0);
        store_all(S1, 1);
        load(3, S1);
        __syncthreads();
        int64_t t = 0;
#pragma clang loop unroll(disable)
        for (; t + 5 < nt; t += 2) {
            iter_steady(std::integral_constant<int, 0>{}, t);
            iter_steady(std::integral_constant<int, 1>{}, t + 1);
        }
#pragma clang loop unroll(disable)
        for (; t < nt; t += 2) {
            iter_drain(std::integral_constant<int, 0>{}, t);
            if (t + 1 < nt) iter_drain(std::integral_constant<int, 1>{}, t + 1);
        }
    } else {
        // short reductions: one stage at a time
        for (int64_t t = 0; t < nt; ++t) {
            load(t, S0);
            __syncthreads();
            store_all(S0, 0);
            __syncthreads();
            read_all(F0, 0);
#pragma unroll
            for (int i = 0; i < kMfma; ++i) mfma(F0, i);
        }
    }

#pragma unroll
    for (int a = 0; a < T::MA; ++a) {
#pragma unroll
        for (int b = 0; b < T::NB; ++b) {
            const int64_t col = n0 + wn * (TN / 2) + 32 * b + (lane & 31);
            if (col >= p.N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + wm * (TM / 2) + 32 * a + mfma32_row(r, lane);
                if (row >= p.M) continue;
                float* cp = C + row * p.ldc + col;
                float v = p.alpha * acc[a][b][r];
                if (p.beta != 0.f) v += p.beta * *cp;
                *cp = v;
            }
        }
    }
}

template <int TM, int TN>
hipError_t launch_x6(const GemmArgs& p, int64_t batch, hipStream_t stream) {
    constexpr int TK = 16;
    dim3 grid((unsigned)ceil_div(p.N, TN), (unsigned)ceil_div(p.M, TM), (unsigned)batch);
    if (grid.y > 65535u || grid.z > 65535u) return hipErrorInvalidValue;
    const bool full = p.M % TM == 0 && p.N % TN == 0 && p.K1 % TK == 0 && p.vecA1 && p.vecB1 &&
                      (!p.A2 || (p.K2 % TK == 0 && p.vecA2 && p.vecB2));
#define GPTQ_X6_LAUNCH(TA_, TB_)                                                                              \
    if (full) hipLaunchKernelGGL((gemm_x6_kernel<TM, TN, TK, TA_, TB_, true>), grid, dim3(256), 0, stream, p);  \
    else hipLaunchKernelGGL((gemm_x6_kernel<TM, TN, TK, TA_, TB_, false>), grid, dim3(256), 0, stream, p);
    if (!p.transA && !p.transB) { GPTQ_X6_LAUNCH(false, false) }
    else if (!p.transA && p.transB) { GPTQ_X6_LAUNCH(false, true) }
    else if (p.transA && !p.transB) { GPTQ_X6_LAUNCH(true, false) }
    else { GPTQ_X6_LAUNCH(true, true) }
#undef GPTQ_X6_LAUNCH
    return hipGetLastError();
}

inline bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; }


// Whole tiles only, every operand 16-byte vectorisable: no per-element guards in the k-loop.
bool full_tiles(const GemmArgs& p, int TM, int TN, int TK) {
    return p.M % TM == 0 && p.N % TN == 0 && p.K1 % TK == 0 && p.vecA1 && p.vecB1 &&
           (!p.A2 || (p.K2 % TK == 0 && p.vecA2 && p.vecB2));
}

template <int TM, int TN, int TK>
hipError_t launch(const GemmArgs& p, int64_t batch, hipStream_t stream) {
    dim3 grid((unsigned)ceil_div(p.N, TN), (unsigned)ceil_div(p.M, TM), (unsigned)batch);
    if (grid.y > 65535u || grid.z > 65535u) return hipErrorInvalidValue;
    const bool full = full_tiles(p, TM, TN, TK);
#define GPTQ_GEMM_LAUNCH(TA_, TB_)                                                                          \
    if (full) hipLaunchKernelGGL((gemm_f32_kernel<TM, TN, TK, TA_, TB_, true>), grid, dim3(256), 0, stream, p); \
    else hipLaunchKernelGGL((gemm_f32_kernel<TM, TN, TK, TA_, TB_, false>), grid, dim3(256), 0, stream, p);
    if (!p.transA && !p.transB) { GPTQ_GEMM_LAUNCH(false, false) }
    else if (!p.transA && p.transB) { GPTQ_GEMM_LAUNCH(false, true) }
    else if (p.transA && !p.transB) { GPTQ_GEMM_LAUNCH(true, false) }
    else { GPTQ_GEMM_LAUNCH(true, true) }
#undef GPTQ_GEMM_LAUNCH
    return hipGetLastError();
}

// 16-byte vector loads need an aligned base, a leading dimension (and batch stride) that is a multiple of 4
// floats; otherwise the tile loads fall back to scalar accesses.
void set_vector_flags(GemmArgs& p, int64_t batch) {
    auto vec_ok = [&](const float* ptr, int64_t ld, int64_t stride) {
        return ptr && aligned16(ptr) && ld % 4 == 0 && (batch == 1 || stride % 4 == 0);
    };
    p.vecA1 = vec_ok(p.A1, p.lda1, p.strideA1);
    p.vecB1 = vec_ok(p.B1, p.ldb1, p.strideB1);
    p.vecA2 = vec_ok(p.A2, p.lda2, p.strideA2);
    p.vecB2 = vec_ok(p.B2, p.ldb2, p.strideB2);
}

bool use_split_bf16(const GemmArgs& p) {
    const int64_t tiles128 = ceil_div(p.M, 128) * ceil_div(p.N, 128);
    return p.K1 >= 1024 && p.M >= 1024 && p.N >= 1024 && tiles128 >= 512;
}

}  // namespace

hipError_t gemm_f32(GemmArgs p, int64_t batch, hipStream_t stream) {
    if (p.M <= 0 || p.N <= 0 || batch <= 0) return hipSuccess;
    set_vector_flags(p, batch);
    // Tile shape, measured on gfx950 (random data): 64 x 64 matches 128 x 128 on general products up to ~7k and
    // beats it on the depth-128 trailing updates and on small products (more workgroups in flight); from about
    // 12k x 12k outputs on, 128 x 128 is faster (half the L2 traffic per flop: +20% at 14336).  Triangular
    // products (the factorisation's) switch at 7168, where 128 x 128 is 2-8% faster and at 3584 up to 30% slower.
    // Products with a long reduction and enough 128 x 128 tiles run on the bf16 MFMA with three-part operand
    // splits (fp32 accuracy).  Measured at depth >= 1024: 156-167 TFLOP/s against 87-122 for the fp32 MFMA on
    // 3584-14336 squares (the fp32 MFMA peak is 157.3), 118-136 against 87-106 on the 1024-3072-wide trailing
    // updates; equal at 256 tiles, slower on the 2048 squares and at depth <= 512 (per-stage overhead).  The choice
    // depends on one batch element's shape only, so a batched call (all output-channel groups at once) does the
    // same arithmetic as one call per element, bit for bit.
    if (use_split_bf16(p)) return launch_x6<128, 128>(p, batch, stream);
    return launch<64, 64, 16>(p, batch, stream);
}

hipError_t gemm_f32_pair(GemmArgs a, GemmArgs b, int64_t batch, hipStream_t stream) {
    if (batch <= 0) return hipSuccess;
    const bool pairable = a.M > 0 && a.N > 0 && b.M > 0 && b.N > 0 && !use_split_bf16(a) && !use_split_bf16(b) &&
                          !a.transA && a.transB && !b.transA && !b.transB && batch <= 65535;
    const int64_t gx1 = ceil_div(a.N, 64), gy1 = ceil_div(a.M, 64), gx2 = ceil_div(b.N, 64), gy2 = ceil_div(b.M, 64);
    const int64_t n = gx1 * gy1 + gx2 * gy2;
    if (!pairable || n > 0x7fffffff) {
        const hipError_t e = gemm_f32(a, batch, stream);
        return e != hipSuccess ? e : gemm_f32(b, batch, stream);
    }
    set_vector_flags(a, batch);
    set_vector_flags(b, batch);
    const bool f1 = full_tiles(a, 64, 64, 16), f2 = full_tiles(b, 64, 64, 16);
    const dim3 grid((unsigned)n, 1, (unsigned)batch);
    const int g[4] = {(int)gx1, (int)gy1, (int)gx2, (int)gy2};
    if (f1 && f2) hipLaunchKernelGGL((gemm_f32_pair_kernel<true, true>), grid, dim3(256), 0, stream, a, b, g[0], g[1], g[2], g[3]);
    else if (f1) hipLaunchKernelGGL((gemm_f32_pair_kernel<true, false>), grid, dim3(256), 0, stream, a, b, g[0], g[1], g[2], g[3]);
    else if (f2) hipLaunchKernelGGL((gemm_f32_pair_kernel<false, true>), grid, dim3(256), 0, stream, a, b, g[0], g[1], g[2], g[3]);
    else hipLaunchKernelGGL((gemm_f32_pair_kernel<false, false>), grid, dim3(256), 0, stream, a, b, g[0], g[1], g[2], g[3]);
    return hipGetLastError();
}

}  // namespace gptq
