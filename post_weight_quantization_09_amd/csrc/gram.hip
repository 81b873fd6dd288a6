// Calibration Gram on gfx950 bf16 MFMA:  H += 2 Xs^T Xs  (and the asymmetric cross term A += 2 dX^T X).
//
// [T] section 1: the layer objective splits into one quadratic per output channel whose Hessian
// H = 2 X^T X is shared by all channels and accumulated batch by batch.  [R] item 3: asymmetric
// calibration reuses X^T X and adds the cross Gram (X~ - X)^T X.  [G]: each output-channel group owns a
// Hessian built from its own token weighting (row_scale).
//
// Design (256 threads, 4 waves, one 256 x 256 output tile per workgroup, 128 x 128 per wave):
//   * X is row-major (tokens x features), so both MFMA operands have the reduction index (tokens) as the
//     slow dimension.  32-token x 256-column slabs of the two operands are staged in LDS in their natural
//     row layout.
//   * Operands are read with ds_read_b64 (each lane 4 columns of one token row; lanes on consecutive
//     columns, so the reads are conflict-free) and regrouped with v_perm into v_mfma_f32_32x32x16_bf16
//     fragments: lane l gets 4 columns x 8 tokens and accumulates the 4 x 4 interleaved sub-blocks
//     (row 4 r + a, column 4 c + b) of its wave's 128 x 128 quadrant.  A and B use the same token <->
//     (lane half, slot) map.
//   * Only tiles on or above the diagonal are computed (H is symmetric); the cross term computes all.
//   * The token range is split across workgroups: enough ways to fill whole rounds of 256 CUs when there
//     are few tiles, 8 ways (one range per XCD) when there are many; work_item maps workgroups to (split,
//     tile) so that the workgroups sharing an XCD's L2 stream the same tokens in step.  Each split writes its
//     fp32 partial tile in register order (coalesced); a second kernel sums the partials in a fixed order
//     (deterministic, no float atomics), scales by 2, adds into H and writes the mirrored lower triangle.
#include "gram.hpp"

#include <algorithm>

#include "timer.hpp"

namespace gptq {

namespace {

constexpr int kGT = 256;      // output tile edge
constexpr int kGK = 32;       // tokens per LDS stage
constexpr int kGPitch = kGT;  // LDS row pitch in bf16 elements (512 B; all reads are row-contiguous)

__device__ inline int mfma32_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

#ifndef GPTQ_GRAM_GROUP
#define GPTQ_GRAM_GROUP 8       // tiles are enumerated in G x G groups (see tile_coords)
#endif

// Tile t -> (row block, column block) over all nb x nb blocks (cross term) or over the upper triangle.
// Tiles are enumerated group by group, G x G blocks at a time (groups row-major; inside a group row-major,
// upper part only on diagonal groups of the symmetric case).  The workgroups that run together on one XCD
// take consecutive tiles of one token split, so a compact group makes them share the same few column slabs
// in that XCD's L2.  Out-of-range t gives bi = nb (callers return early).
__device__ inline void tile_coords(int t, int nb, bool full, int& bi, int& bj) {
    constexpr int G = GPTQ_GRAM_GROUP;
    const int ng = (nb + G - 1) / G;
    int rem = t;
    for (int I = 0; I < ng; ++I) {
        const int gi = min(G, nb - I * G);
        for (int J = full ? 0 : I; J < ng; ++J) {
            const int gj = min(G, nb - J * G);
            const bool diag = !full && I == J;
            const int cnt = diag ? gi * (gi + 1) / 2 : gi * gj;
            if (rem < cnt) {
                if (diag) {
                    int b = 0;
                    while (rem >= gi - b) { rem -= gi - b; ++b; }
                    bi = I * G + b;
                    bj = I * G + b + rem;
                } else {
                    bi = I * G + rem / gj;
                    bj = J * G + rem % gj;
                }
                return;
            }
            rem -= cnt;
        }
    }
    bi = nb;
    bj = nb;
}

// Workgroup -> (token split, tile).  Workgroup b runs on XCD b % 8, and each XCD runs its workgroups in rounds
// of 32 (one per CU), in order.  8 splits (many tiles): XCD x streams split x, consecutive tiles at a time, so
// the co-resident workgroups of an XCD read the same tokens and share column slabs in its L2.  Fewer splits
// (short token ranges): split-major order.
// More splits (few tiles, short token ranges): the 256 co-resident workgroups of the chip take 256 consecutive
// (split, tile) items, XCD x the x-th 32 of them, so that all XCDs sweep the same few splits together and the
// slabs one XCD misses in its L2 have mostly just been fetched by another (hits in the memory-side cache):
// 2.5% faster at 2M tokens x 4096 features, but 7% slower at 8 splits of 28672 features, hence the rule.
// The last partial round (fewer than 256 workgroups) keeps the identity order.
__device__ inline void work_item(int bid, const GramArgs& p, int& split, int& tile) {
    if (p.splits > 8) {
        const int full = (p.ntiles * p.splits) & ~255;
        int idx = bid;
        if (bid < full) {
            const int x = bid & 7, q = bid >> 3;
            idx = 256 * (q >> 5) + 32 * x + (q & 31);
        }
        split = idx / p.ntiles;
        tile = idx % p.ntiles;
    } else if (p.splits == 8) {
        split = bid & 7;
        tile = bid >> 3;
    } else {
        split = bid / p.ntiles;
        tile = bid % p.ntiles;
    }
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


// Short offset of (row, col) in a 32 x 256 bf16 slab (rows contiguous, 512 bytes each).  Written as chunk
// base + chunk offset rather than plain `col`: the compiler then schedules the operand addresses of the
// streaming kernel in a way measured about 2% faster (2M tokens x 4096 features).
__device__ __forceinline__ int slab_off(int row, int col) { return row * kGT + (col & ~7) + (col & 7); }

// MFMA fragments of one 16-token k-step for 4 x 32 columns starting at column `base` of a slab: b64 reads of
// 4 columns x 8 token rows, regrouped by v_perm so that frag[a] holds column base + 4 (l % 32) + a over tokens
// 16 ks + 8 (l / 32) + 0..7 (lane l).  The reads are row-contiguous across lanes (conflict-free).
__device__ __forceinline__ u32x2 frag_row(const uint16_t* slab, int base, int ks, int lane, int s8) {
    const int row = ks * 16 + 8 * (lane >> 5) + s8;
    return *reinterpret_cast<const u32x2*>(slab + slab_off(row, base + 4 * (lane & 31)));
}
// Token rows 2s and 2s+1 of the 8 read rows -> element s of the 4 column fragments.
__device__ __forceinline__ void frag_regroup(const u32x2 (&raw)[8], int s, u32x4 (&frag)[4]) {
    const uint32_t lo0 = raw[2 * s].x, lo1 = raw[2 * s + 1].x;
    const uint32_t hi0 = raw[2 * s].y, hi1 = raw[2 * s + 1].y;
    frag[0][s] = __builtin_amdgcn_perm(lo1, lo0, 0x05040100u);
    frag[1][s] = __builtin_amdgcn_perm(lo1, lo0, 0x07060302u);
    frag[2][s] = __builtin_amdgcn_perm(hi1, hi0, 0x05040100u);
    frag[3][s] = __builtin_amdgcn_perm(hi1, hi0, 0x07060302u);
}
__device__ __forceinline__ void load_frags(const uint16_t* slab, int base, int ks, int lane, u32x4 (&frag)[4]) {
    u32x2 raw[8];
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) raw[s8] = frag_row(slab, base, ks, lane, s8);
#pragma unroll
    for (int s = 0; s < 4; ++s) frag_regroup(raw, s, frag);
}

// (row, col) of accumulator element r of MFMA block (a, b) for `lane` inside a wave's 128 x 128 quadrant.
__device__ __forceinline__ int acc_row(int a, int r, int lane) { return 4 * mfma32_row(r, lane) + a; }
__device__ __forceinline__ int acc_col(int b, int lane) { return 4 * (lane & 31) + b; }

// Raw global data of one 32-token stage held in registers while it is in flight; the per-token weight and
// the float-stream mismatch are applied when the stage is written to LDS, so that no arithmetic waits on
// an outstanding load.
template <bool CROSS, bool SCALED>
struct StageRegs {
    u32x4 a[4], b[4];
    u32x4 f[CROSS ? 4 : 1];
    float s[SCALED ? 4 : 1];
};

// Scheduling hint (gfx9 sched_group_barrier masks): spread the 16 LDS reads and the v_perm regrouping of one
// k-step over the 16 MFMAs of the other, so the matrix core keeps a queue while operands are fetched.
__device__ __forceinline__ void interleave_kstep() {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // VALU (v_perm)
    }
}

template <bool CROSS, bool SCALED, bool FAST>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gram_bf16_kernel(GramArgs p) {
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][kGK][kGPitch];
    __shared__ __attribute__((aligned(16))) uint16_t sB[2][kGK][kGPitch];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wi = wave >> 1, wj = wave & 1;

    int split, tile;
    const int bid = blockIdx.x;
    work_item(bid, p, split, tile);
    int bi, bj;
    tile_coords(tile, p.nb, CROSS, bi, bj);
    if (bi >= p.nb || bj >= p.nb || split >= p.splits) return;   // whole workgroup, before any barrier
    const bool same = !CROSS && bi == bj;       // diagonal tile: quadrant (1,0) mirrors (0,1)
    const bool active = !(same && wi == 1 && wj == 0);
    const int64_t colA = (int64_t)bi * kGT, colB = (int64_t)bj * kGT;
    const int64_t t0 = (int64_t)split * p.tokens_per_split;
    const int64_t t1 = min<int64_t>(p.M, t0 + p.tokens_per_split);
    // Stage count rounded up to even (the pipeline handles stages in pairs); a padding stage holds only
    // tokens >= t1, which are written to LDS as zeros.
    const int64_t nst = t1 > t0 ? (ceil_div(t1 - t0, kGK) + 1) & ~(int64_t)1 : 0;

    f32x16 acc[4][4];
    for (int a = 0; a < 4; ++a)
        for (int b = 0; b < 4; ++b)
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

    typedef StageRegs<CROSS, SCALED> Regs;
    // thread -> (token row, 8-column chunk) of a stage: chunk c = tid + 256 i, row c / 32, chunk c % 32
    auto ld = [&](const uint16_t* base, int64_t ldb, int64_t tok, int64_t col) -> u32x4 {
        if (FAST) return *reinterpret_cast<const u32x4*>(base + (tok < t1 ? tok : t1 - 1) * ldb + col);
        return load8(base, ldb, tok, t1, col, p.K, p.vec);
    };
    auto gload = [&](int64_t st, Regs& R) {
        const int64_t tb = t0 + st * kGK;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + 256 * i;
            const int64_t tok = tb + (c >> 5);
            const int64_t col = (c & 31) * 8;
            R.a[i] = ld(p.X, p.ldx, tok, colA + col);
            R.b[i] = ld(p.X, p.ldx, tok, colB + col);
            if constexpr (CROSS) R.f[i] = ld(p.Xf, p.ldxf, tok, colA + col);
            if constexpr (SCALED) R.s[i] = p.rho[tok < t1 ? tok : t1 - 1];
        }
    };
    auto lstore = [&](int64_t st, const Regs& R, int buf) {
        const int64_t tb = t0 + st * kGK;
        const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + 256 * i;
            const int tr = c >> 5, cc = c & 31;
            const bool ok = tb + tr < t1;
            u32x4 va = R.a[i], vb = R.b[i];
            if constexpr (CROSS) va = diff_bf16(R.f[i], R.a[i]);
            if constexpr (SCALED) {
                va = scale_row_bf16(va, R.s[i]);
                vb = scale_row_bf16(vb, R.s[i]);
            }
            *reinterpret_cast<u32x4*>(&sA[buf][0][0] + slab_off(tr, cc * 8)) = ok ? va : zero;
            *reinterpret_cast<u32x4*>(&sB[buf][0][0] + slab_off(tr, cc * 8)) = ok ? vb : zero;
        }
    };
    auto prep = [&](int buf, int ks, u32x4 (&va)[4], u32x4 (&vb)[4]) {
        load_frags(&sA[buf][0][0], wi * 128, ks, lane, va);
        load_frags(&sB[buf][0][0], wj * 128, ks, lane, vb);
    };
    auto mfma = [&](const u32x4 (&va)[4], const u32x4 (&vb)[4]) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const bf16x8 av = __builtin_bit_cast(bf16x8, va[a]);
#pragma unroll
            for (int b = 0; b < 4; ++b)
                acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8, vb[b]), acc[a][b],
                                                                   0, 0, 0);
        }
    };

    // Software pipeline over stages st (LDS buffer st & 1):
    //   stage s is read from global at iteration s-3, written to LDS at iteration s-1;
    //   iteration st: [MFMA (st, k0) || LDS reads of (st, k1)]  [LDS write of st+1; loads of st+3]  barrier
    //                 [MFMA (st, k1) || LDS reads of (st+1, k0)]
    Regs R0, R1;
    u32x4 k0a[4], k0b[4], k1a[4], k1b[4];
    if (nst > 0) gload(0, R0);
    if (nst > 1) gload(1, R1);
    if (nst > 0) lstore(0, R0, 0);
    if (nst > 2) gload(2, R0);
    __syncthreads();
    if (nst > 0) prep(0, 0, k0a, k0b);

    auto body = [&](int64_t st, Regs& Rn) {
        const int buf = (int)(st & 1);
        prep(buf, 1, k1a, k1b);
        mfma(k0a, k0b);
        interleave_kstep();
        if (st + 1 < nst) lstore(st + 1, Rn, buf ^ 1);
        if (st + 3 < nst) gload(st + 3, Rn);
        __syncthreads();
        if (st + 1 < nst) prep(buf ^ 1, 0, k0a, k0b);
        mfma(k1a, k1b);
        interleave_kstep();
    };
#pragma clang loop unroll(disable)
    for (int64_t st = 0; st < nst; st += 2) {
        body(st, R1);
        body(st + 1, R0);
    }

    if (!active) return;
    float* out = p.partial + (((int64_t)split * p.ntiles + tile) * 4 + wave) * (256 * 64);
    for (int a = 0; a < 4; ++a)
        for (int b = 0; b < 4; ++b)
            for (int r = 0; r < 16; ++r) out[((a * 4 + b) * 16 + r) * 64 + lane] = acc[a][b][r];
}

// Plain symmetric Gram, fast layout (K a multiple of 256, 16-byte aligned rows, every split a whole number
// of 32-token stages): activations go straight from global memory into a RING-slot LDS ring (32 KB per
// slot) with global_load_lds_dwordx4 (no register staging), so RING-1 stages are in flight while one is
// consumed.  Wait counts and barriers are explicit: the compiler cannot see that a DMA'd stage belongs to a
// different ring slot than the one being read and would otherwise drain all loads at every barrier.
// Per stage st:  [MFMA (st, k-step 0) || LDS reads + v_perm of (st, k-step 1)]
//                [wait for this wave's loads of st+1; barrier]
//                [MFMA (st, k-step 1) || loads of st+RING-1 into the freed slot, LDS reads + v_perm of
//                 (st+1, k-step 0)]
// Ring depth, measured on MI355X with this schedule (2M tokens x 4096 / 524288 x 28672 features): 4 slots
// 30.8 / 373 ms, 3 slots 33.6 / 444 ms, 5 slots 34.4 / 416 ms (the extra requests only queue in the L2).
// The launch is power-bound on random bf16 data: the shader clock runs at about 1.5-1.6 GHz with loads and
// MFMAs overlapped, 1.9 GHz for the MFMA work alone (operands resident in LDS) and 2.4 GHz for the loads
// alone.
typedef __attribute__((address_space(3))) void lds_void_t;

// Wait until at most `later` stages (8 DMA instructions each) of this wave are still in flight, then
// synchronise the workgroup.
__device__ __forceinline__ void wait_vm_and_barrier(int later) {
    if (later >= 3) asm volatile("s_waitcnt vmcnt(24) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else if (later == 2) asm volatile("s_waitcnt vmcnt(16) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else if (later == 1) asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <bool CROSS, int RING>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gram_bf16_lds_kernel(GramArgs p) {
    constexpr int kRing = RING;
    static_assert(kRing >= 3 && kRing <= 5, "ring slots: 3..5 (32 KB each, 160 KB of LDS)");
    __shared__ __attribute__((aligned(1024))) uint16_t ring[kRing][2][kGK][kGT];

    // the wave index is uniform: keep it (and the LDS addresses derived from it) in scalar registers
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int wi = wave >> 1, wj = wave & 1;
    int split, tile;
    const int bid = blockIdx.x;
    work_item(bid, p, split, tile);
    int bi, bj;
    tile_coords(tile, p.nb, CROSS, bi, bj);
    if (bi >= p.nb || bj >= p.nb || split >= p.splits) return;
    const bool active = CROSS || !(bi == bj && wi == 1 && wj == 0);
    const int64_t t0 = (int64_t)split * p.tokens_per_split;
    const int64_t t1 = min<int64_t>(p.M, t0 + p.tokens_per_split);
    const int64_t nst = t1 > t0 ? (t1 - t0) / kGK : 0;       // whole stages (checked on the host)

    f32x16 acc[4][4];
    for (int a = 0; a < 4; ++a)
        for (int b = 0; b < 4; ++b)
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

    // This wave DMAs token rows 8*wave .. 8*wave+7 of both slabs: 8 instructions of 1 KB (two 512-byte
    // rows each: lanes 0-31 the first row, lanes 32-63 the second; lane l lands in, and fetches, 16-byte
    // chunk l % 32 of its row).  Instruction j: rows 8*wave + 2*(j/2) + 0..1 of operand j % 2.
    const int lrow = 8 * wave + (lane >> 5);
    const uint16_t* XA = p.XA ? p.XA : p.X;          // A-side operand (the mismatch for the cross term)
    const int64_t lda = p.XA ? p.ldxa : p.ldx;
    const uint16_t* srcA = XA + (int64_t)bi * kGT + (lane & 31) * 8;
    const uint16_t* srcB = p.X + (int64_t)bj * kGT + (lane & 31) * 8;
    auto slot_of = [](int64_t st) { return (int)((uint32_t)st % (uint32_t)kRing); };
    auto issue_one = [&](int64_t st, int j) {
        const int slot = slot_of(st);
        const int64_t tok = t0 + st * kGK + lrow + 2 * (j >> 1);
        if (j & 1)
            __builtin_amdgcn_global_load_lds((const void*)(srcB + tok * p.ldx),
                                             (lds_void_t*)&ring[slot][1][8 * wave + 2 * (j >> 1)][0], 16, 0, 0);
        else
            __builtin_amdgcn_global_load_lds((const void*)(srcA + tok * lda),
                                             (lds_void_t*)&ring[slot][0][8 * wave + 2 * (j >> 1)][0], 16, 0, 0);
    };
    auto issue = [&](int64_t st) {
#pragma unroll
        for (int j = 0; j < 8; ++j) issue_one(st, j);
    };
    auto prep = [&](int64_t st, int ks, u32x4 (&va)[4], u32x4 (&vb)[4]) {
        const int slot = slot_of(st);
        load_frags(&ring[slot][0][0][0], wi * 128, ks, lane, va);
        load_frags(&ring[slot][1][0][0], wj * 128, ks, lane, vb);
    };
    auto mfma1 = [&](int i, const u32x4 (&va)[4], const u32x4 (&vb)[4]) {
        const int a = i >> 2, b = i & 3;
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va[a]),
                                                           __builtin_bit_cast(bf16x8, vb[b]), acc[a][b], 0, 0, 0);
    };
    // One k-step: the 16 MFMAs on (va, vb), each followed by a fixed share of the next k-step's operand work,
    // pinned in place with scheduling barriers (the scheduler otherwise groups all MFMAs together and leaves
    // the LDS reads and the regrouping to run on their own): after MFMA i < 8 the LDS reads of token row i of
    // (st_n, ks_n) for A and B; after every even MFMA, if `dma`, one of the 8 DMA instructions of stage
    // `st_dma`; after MFMAs 8-15 the regrouping of one fragment element (A for 8-11, B for 12-15).  Measured
    // against other placements (2M tokens x 4096 / 524288 x 28672 features): the reads packed into MFMAs 0-3
    // 31.7 / 418 ms, this 30.8 / 373 ms, the regrouping started at MFMA 6 37.2 / 452 ms, one DMA instruction
    // after each of MFMAs 0-7 30.9 / 380 ms.
    auto kstep = [&](const u32x4 (&va)[4], const u32x4 (&vb)[4], int64_t st_n, int ks_n, u32x4 (&na)[4],
                     u32x4 (&nb)[4], bool dma, int64_t st_dma) {
        const int sl = slot_of(st_n);
        const uint16_t* slabA = &ring[sl][0][0][0];
        const uint16_t* slabB = &ring[sl][1][0][0];
        u32x2 ra[8], rb[8];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            mfma1(i, va, vb);
            if (dma && (i & 1) == 0) issue_one(st_dma, i >> 1);
            if (i < 8) {
                ra[i] = frag_row(slabA, wi * 128, ks_n, lane, i);
                rb[i] = frag_row(slabB, wj * 128, ks_n, lane, i);
            } else if (i < 12) {
                frag_regroup(ra, i - 8, na);
            } else {
                frag_regroup(rb, i - 12, nb);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto mfma = [&](const u32x4 (&va)[4], const u32x4 (&vb)[4]) {
#pragma unroll
        for (int i = 0; i < 16; ++i) mfma1(i, va, vb);
    };

    // Stage s is DMA'd kRing-1 stages ahead of its use: issued after the barrier of iteration s-kRing+1,
    // waited for before the barrier of iteration s-1.
    u32x4 k0a[4], k0b[4], k1a[4], k1b[4];
    if (nst > 0) {
        const int64_t pre = nst < kRing - 1 ? nst : kRing - 1;
        for (int64_t s0 = 0; s0 < pre; ++s0) issue(s0);
        wait_vm_and_barrier((int)pre - 1);           // stage 0 landed for every wave
        prep(0, 0, k0a, k0b);
    }
    // Steady state (stage st+kRing-1 exists): [k-step 0 of st || operands of (st, 1)] barrier
    // [k-step 1 of st || DMA of st+kRing-1, operands of (st+1, 0)].  The iteration has no branch.
    const int64_t nsteady = nst > kRing - 1 ? nst - (kRing - 1) : 0;
#pragma clang loop unroll(disable)
    for (int64_t st = 0; st < nsteady; ++st) {
        kstep(k0a, k0b, st, 1, k1a, k1b, false, 0);
        // own loads of st+1 landed (stages st+2 .. st+kRing-2 may be pending); everyone is past st-1
        wait_vm_and_barrier(kRing - 3);
        kstep(k1a, k1b, st + 1, 0, k0a, k0b, true, st + kRing - 1);
    }
    // Drain: the last kRing-1 stages, nothing left to issue.
#pragma clang loop unroll(disable)
    for (int64_t st = nsteady; st < nst; ++st) {
        prep(st, 1, k1a, k1b);
        mfma(k0a, k0b);
        if (st + 1 < nst) {
            wait_vm_and_barrier((int)(nst - 1 - (st + 1)));
            prep(st + 1, 0, k0a, k0b);
        }
        mfma(k1a, k1b);
    }

    if (!active) return;
    float* out = p.partial + (((int64_t)split * p.ntiles + tile) * 4 + wave) * (256 * 64);
    for (int a = 0; a < 4; ++a)
        for (int b = 0; b < 4; ++b)
            for (int r = 0; r < 16; ++r) out[((a * 4 + b) * 16 + r) * 64 + lane] = acc[a][b][r];
}

// Elementwise operand preparation for the fast Gram path: Xs = bf16(rho_t * x) (group weights) or
// dX = bf16(X~ - X) (asymmetric cross term), written densely (ld = K).  HBM-bound, 8 elements per thread.
template <bool DIFF>
__global__ __launch_bounds__(256) void gram_operand_kernel(const uint16_t* X, int64_t ldx, const uint16_t* Xf,
                                                           int64_t ldxf, const float* rho, int64_t M, int64_t K,
                                                           uint16_t* out) {
    const int64_t chunks_per_row = K / 8;
    const int64_t total = M * chunks_per_row;
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total; c += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = c / chunks_per_row, k = (c % chunks_per_row) * 8;
        const u32x4 x = *reinterpret_cast<const u32x4*>(X + t * ldx + k);
        u32x4 o;
        if (DIFF) o = diff_bf16(*reinterpret_cast<const u32x4*>(Xf + t * ldxf + k), x);
        else o = scale_row_bf16(x, rho[t]);
        *reinterpret_cast<u32x4*>(out + t * K + k) = o;
    }
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

    // The partial of (split, tile, wave) is 256 registers x 64 lanes, contiguous.  Thread t sums elements
    // 4 (t + 256 i) .. +3 over the splits in split order (the order of the original sequential sum), two
    // element groups at a time with eight splits each: sixteen 16-byte loads in flight per thread.
    const int64_t qstride = (int64_t)p.ntiles * 4 * 256 * 64;
    const float* base = p.partial + ((int64_t)tile * 4 + wave) * (256 * 64);
    constexpr int kInFlight = 8;
    for (int i = 0; i < 16; i += 2) {
        const int e0 = (tid + 256 * i) * 4, e1 = e0 + 256 * 4;   // elements (ri, lane0 .. lane0+3)
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0;
        int sp = 0;
        for (; sp + kInFlight <= p.splits; sp += kInFlight) {
            f32x4 v0[kInFlight], v1[kInFlight];
#pragma unroll
            for (int u = 0; u < kInFlight; ++u) {
                const float* q = base + (int64_t)(sp + u) * qstride;
                v0[u] = *reinterpret_cast<const f32x4*>(q + e0);
                v1[u] = *reinterpret_cast<const f32x4*>(q + e1);
            }
#pragma unroll
            for (int u = 0; u < kInFlight; ++u) { s0 += v0[u]; s1 += v1[u]; }
        }
        for (; sp < p.splits; ++sp) {
            const float* q = base + (int64_t)sp * qstride;
            s0 += *reinterpret_cast<const f32x4*>(q + e0);
            s1 += *reinterpret_cast<const f32x4*>(q + e1);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int e = h ? e1 : e0;
            const f32x4 s = h ? s1 : s0;
            const int ri = e >> 6, lane0 = e & 63;
            const int a = ri >> 6, b = (ri >> 4) & 3, r = ri & 15;
#pragma unroll
            for (int q = 0; q < 4; ++q) T[acc_row(a, r, lane0 + q)][acc_col(b, lane0 + q)] = 2.0f * s[q];
        }
    }
    __syncthreads();
    // Out += the quadrant (and its mirror).  The two blocks a workgroup updates are disjoint, and disjoint from
    // every other workgroup's, so sixteen rows' reads are issued before their writes instead of one
    // read-modify-write round trip at a time.
    constexpr int kRows = 16;
    for (int i0 = 0; i0 < 64; i0 += kRows) {
        float dv[kRows], mv[kRows];
#pragma unroll
        for (int u = 0; u < kRows; ++u) {
            const int idx = tid + 256 * (i0 + u);
            const int row = idx >> 7, col = idx & 127;
            dv[u] = (R0 + row < p.K && C0 + col < p.K) ? Out[(R0 + row) * p.K + C0 + col] : 0.f;
            mv[u] = (mirror && C0 + row < p.K && R0 + col < p.K) ? Out[(C0 + row) * p.K + R0 + col] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kRows; ++u) {
            const int idx = tid + 256 * (i0 + u);
            const int row = idx >> 7, col = idx & 127;
            if (R0 + row < p.K && C0 + col < p.K) Out[(R0 + row) * p.K + C0 + col] = dv[u] + T[row][col];
            if (mirror && C0 + row < p.K && R0 + col < p.K) Out[(C0 + row) * p.K + R0 + col] = mv[u] + T[col][row];
        }
    }
}

}  // namespace

GramPlan gram_plan(int64_t K, int64_t M, bool cross) {
    GramPlan pl;
    pl.cross = cross;
    pl.nb = (int)ceil_div(K, kGT);
    pl.ntiles = cross ? pl.nb * pl.nb : pl.nb * (pl.nb + 1) / 2;
    // One workgroup per CU (256 CUs).  With few tiles the token range is split so that the workgroup
    // count fills whole rounds of 256: the split count (a multiple of 8, so that splits map to XCDs)
    // minimising the idle fraction of the last round, keeping >= 8192 tokens per split.  With many tiles the
    // range is still split 8 ways, one range per XCD: a workgroup then streams 1/8 of the tokens, and the 32
    // co-resident workgroups of an XCD, which run consecutive tiles of the same range, stay close enough in
    // step for their shared column slabs to hit in the XCD's L2 (unsplit, they drift apart over the whole
    // range: 29% L2 hits and 79x the activation bytes fetched at 28672 features).  Measured: 488 -> 467 ms at
    // 524288 x 28672, 66.4 -> 58.5 ms at 262144 x 14336, for 8 partial tile sums more.
    int64_t best = 1;
    if (pl.ntiles < 1024) {
        double best_eff = -1.0;
        for (int64_t s = 8; s <= 64; s += 8) {
            if (s > 8 && M / s < 8192) break;
            const double wgs = (double)pl.ntiles * s;
            const double eff = wgs / (ceil_div((int64_t)wgs, 256) * 256.0);
            if (eff > best_eff + 1e-9) { best_eff = eff; best = s; }
        }
        if (M < 8 * 4096) best = std::max<int64_t>(1, std::min<int64_t>(8, M / 4096));
    } else if (M >= 8 * 8192) {
        best = 8;
    }
    pl.splits = (int)best;
    pl.tokens_per_split = ceil_div(ceil_div(std::max<int64_t>(M, 1), pl.splits), kGK) * kGK;
    pl.partial_floats = (size_t)pl.splits * pl.ntiles * 4 * 256 * 64;
    return pl;
}

size_t gram_staging_elems(int64_t K, int64_t M, bool transformed) {
    // The fast path stages a transformed operand (group-weighted X or the cross mismatch) densely in bf16.
    return transformed && K % kGT == 0 && M % kGK == 0 ? (size_t)M * (size_t)K : 0;
}

hipError_t gram_bf16(const GramPlan& pl, const uint16_t* X, int64_t ldx, const uint16_t* Xf, int64_t ldxf,
                     const float* rho, int64_t M, int64_t K, float* partial, uint16_t* staging, float* Out,
                     hipStream_t stream) {
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
    // Fast path: whole 256-column tiles, 16-byte aligned rows, whole 32-token stages in every split.
    const bool fast = p.vec && K % kGT == 0;
    const bool whole_stages = p.tokens_per_split % kGK == 0 && M % kGK == 0;
    const bool transformed = cross || rho != nullptr;
    {
    TimerScope ts(stream, GPTQ_TIMER_GRAM);
    if (fast && whole_stages && (!transformed || staging)) {
        // stage indices are taken modulo the ring in 32 bits
        if (p.tokens_per_split / kGK >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
        if (transformed) {
            // stage bf16(rho * X) or bf16(X~ - X) once, then run the plain streaming kernel on it
            const int64_t chunks = M * (K / 8);
            const unsigned g = (unsigned)std::min<int64_t>(ceil_div(chunks, 256), 256 * 64);
            if (cross)
                hipLaunchKernelGGL((gram_operand_kernel<true>), dim3(g), dim3(256), 0, stream, X, ldx, Xf, ldxf,
                                   nullptr, M, K, staging);
            else
                hipLaunchKernelGGL((gram_operand_kernel<false>), dim3(g), dim3(256), 0, stream, X, ldx, nullptr,
                                   (int64_t)0, rho, M, K, staging);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            if (cross) { p.XA = staging; p.ldxa = K; }
            else { p.X = staging; p.ldx = K; }
        }
        if (cross) hipLaunchKernelGGL((gram_bf16_lds_kernel<true, 4>), dim3(nblk), dim3(256), 0, stream, p);
        else hipLaunchKernelGGL((gram_bf16_lds_kernel<false, 4>), dim3(nblk), dim3(256), 0, stream, p);
    } else if (fast) {
        if (cross) hipLaunchKernelGGL((gram_bf16_kernel<true, false, true>), dim3(nblk), dim3(256), 0, stream, p);
        else if (rho) hipLaunchKernelGGL((gram_bf16_kernel<false, true, true>), dim3(nblk), dim3(256), 0, stream, p);
        else hipLaunchKernelGGL((gram_bf16_kernel<false, false, true>), dim3(nblk), dim3(256), 0, stream, p);
    } else {
        if (cross) hipLaunchKernelGGL((gram_bf16_kernel<true, false, false>), dim3(nblk), dim3(256), 0, stream, p);
        else if (rho) hipLaunchKernelGGL((gram_bf16_kernel<false, true, false>), dim3(nblk), dim3(256), 0, stream, p);
        else hipLaunchKernelGGL((gram_bf16_kernel<false, false, false>), dim3(nblk), dim3(256), 0, stream, p);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    }
    TimerScope ts(stream, GPTQ_TIMER_GRAM_REDUCE);
    const unsigned nred = (unsigned)(pl.ntiles * 4);
    if (cross) hipLaunchKernelGGL((gram_reduce_kernel<true>), dim3(nred), dim3(256), 0, stream, p, Out);
    else hipLaunchKernelGGL((gram_reduce_kernel<false>), dim3(nred), dim3(256), 0, stream, p, Out);
    return hipGetLastError();
}

}  // namespace gptq
