// Shared-order column loop with lazy block updates on gfx950.
//
// [T] section 3: fixing coordinate q to its grid value moves the still-free weights along the OBS direction.
// [T] section 4: with U the upper factor of H_d^{-1}, that move is w_k -= U_qk E_q with E_q = (w_q - Q(w_q)) / U_qq.
// [T] section 5: every output channel uses the same coordinate order, so all channels share U; inside a
// block of 128 coordinates the updates are applied at once, the rest of the matrix is updated by matrix
// products (W[b1:] -= U[B, b1:]^T E_B), here fp32-accurate MFMA GEMMs.  The products are applied in two
// levels: after each block only the rows of its 1024-coordinate super-block, and once per super-block the far
// rows with the errors of all its blocks (depth 1024), so the far part of W is read and written once per
// super-block instead of once per block, and the far product is deep enough for the split-bf16 GEMM.  The sums
// are the same; only their grouping differs.
// [R] item 3 / [A]: the asymmetric variant adds w_k += P1_qk * w_q(before rounding), in block and in the
// lazy product (a second operand pair of the same GEMM).
// [G] / [T] section 2: symmetric per-channel grid, codes 0..2^b-1, zero point 2^(b-1), value s (c - z).
//
// Data layout: the working weights are kept transposed, Wt[n][k] (fp32, N x ldt, ldt = K rounded up to
// 128), so that one channel's block of 128 coordinates is contiguous.  Both loop kernels give each channel
// 16 lanes (one DPP row); lane l holds coordinates 16 m + l, m = 0..7, of the current block in registers,
// so that the coordinates still free after step j = 16 m + l0 are exactly the slots >= m and the
// triangular work shrinks with m.  The U panel (and P1 panel) of the block sits in LDS, permuted so that a
// lane's coefficients of row j for its still-free slots are at most two 16-byte reads; both kernels copy it there by
// DMA from a copy prepared once per super-block by strip_prep_kernel.  At step j the value w_j is broadcast from its
// owner lane to the row with DPP row_newbcast; every lane of the row then evaluates the same rounding and
// error (no further communication), updates its own slots, and the owner keeps the code.
// Two kernels run these steps: quant_strip_kernel (no asymmetric term, at most 512 workgroups) does a whole
// 1024-coordinate super-block per launch with the channels' weights in LDS and the near updates in-kernel;
// quant_block_kernel does one 128-block per launch, the near updates left to a product after each block.
#include <algorithm>
#include <utility>

#include "gemm_f32.hpp"
#include "quantize.hpp"
#include "timer.hpp"

namespace gptq {

namespace {

constexpr int kB = 128;          // block (lazy batch) width
constexpr int kSB = 8 * kB;      // super-block: far rows are updated once per kSB coordinates
constexpr int kChPerWG = 16;     // channels per workgroup of the block kernel

__global__ void quant_init_kernel(DevStatus* st, uint32_t* amax_bits, float* loss_acc, int64_t N) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i == 0) { st->flags = 0; st->n_dead = 0; st->damp = 0.f; }
    if (i < N) { amax_bits[i] = 0u; loss_acc[i] = 0.f; }
}

// W (K x N view with strides) -> Wt (N x ldt fp32, dead rows zeroed, padding zero) and per-channel max |w|
// taken before dead rows are zeroed.  64 x 64 tiles transposed through LDS.
// With act-order, processing position k reads original row perm[k]; `dead` is indexed by processing position.
// Output-channel groups of gs channels: channel n uses the dead flags and permutation of group n / gs
// (dead + g K, perm + g K).
template <bool BF16>
__global__ __launch_bounds__(256) void convert_kernel(const void* Wv, int64_t K, int64_t N, int64_t w_rs,
                                                     int64_t w_cs, const uint8_t* dead, float* Wt, int64_t ldt,
                                                     uint32_t* amax_bits, DevStatus* st, const int32_t* perm,
                                                     int64_t gs) {
    __shared__ float tile[64][65];
    const int tid = threadIdx.x;
    const int64_t k0 = (int64_t)blockIdx.y * 64, n0 = (int64_t)blockIdx.x * 64;
    const bool n_fast = (w_cs == 1) || (w_rs != 1 && w_cs <= w_rs);
    // Whole tile, channels contiguous in 16-byte rows, natural order: 16-byte loads along n and 16-byte stores
    // along k (the general path moves one element per lane and access).
    constexpr int V = BF16 ? 8 : 4;                  // elements per 16-byte load
    const bool fast = !perm && w_cs == 1 && k0 + 64 <= K && n0 + 64 <= N && w_rs % V == 0 &&
                      (reinterpret_cast<uintptr_t>(Wv) & 15) == 0 &&
                      (!dead || ((reinterpret_cast<uintptr_t>(dead) & 3) == 0 && K % 4 == 0));
    unsigned bad = 0;
    if (fast) {
#pragma unroll
        for (int i = 0; i < 64 * (64 / V) / 256; ++i) {
            const int idx = tid + 256 * i;
            const int kk = idx / (64 / V), nv = (idx % (64 / V)) * V;
            const int64_t off = (k0 + kk) * w_rs + n0 + nv;
            float v[V];
            if constexpr (BF16) {
                const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(Wv) + off);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[2 * e] = __uint_as_float(w[e] << 16);
                    v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
                }
            } else {
                const f32x4 w = *reinterpret_cast<const f32x4*>(static_cast<const float*>(Wv) + off);
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = w[e];
            }
#pragma unroll
            for (int e = 0; e < V; ++e) {
                if (!isfinite(v[e])) bad = 1;
                tile[kk][nv + e] = v[e];
            }
        }
    } else {
        for (int i = 0; i < 16; ++i) {
            const int idx = tid + 256 * i;
            const int a = idx >> 6, b = idx & 63;         // (slow, fast)
            const int kk = n_fast ? a : b, nn = n_fast ? b : a;
            const int64_t k = k0 + kk, n = n0 + nn;
            float v = 0.f;
            if (k < K && n < N) {
                const int64_t gK = (int64_t)((uint32_t)n / (uint32_t)gs) * K;
                const int64_t off = (perm ? (int64_t)perm[gK + k] : k) * w_rs + n * w_cs;
                if (BF16) v = __uint_as_float((uint32_t)(static_cast<const uint16_t*>(Wv)[off]) << 16);
                else v = static_cast<const float*>(Wv)[off];
                if (!isfinite(v)) bad = 1;
            }
            tile[kk][nn] = v;
        }
    }
    __syncthreads();
    // column max over this tile's 64 rows, 4 threads per channel
    {
        const int nn = tid >> 2, part = tid & 3;
        float m = 0.f;
        for (int kk = part; kk < 64; kk += 4) m = fmaxf(m, fabsf(tile[kk][nn]));
        m = fmaxf(m, __shfl_xor(m, 1, 4));
        m = fmaxf(m, __shfl_xor(m, 2, 4));
        if (part == 0 && n0 + nn < N && m > 0.f) atomicMax(&amax_bits[n0 + nn], __float_as_uint(m));
    }
    if (fast) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = tid + 256 * i;
            const int nn = idx >> 4, kq = (idx & 15) * 4;
            const int64_t n = n0 + nn;
            f32x4 v = {tile[kq][nn], tile[kq + 1][nn], tile[kq + 2][nn], tile[kq + 3][nn]};
            if (dead) {
                const uint32_t d4 = *reinterpret_cast<const uint32_t*>(
                    dead + (int64_t)((uint32_t)n / (uint32_t)gs) * K + k0 + kq);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if ((d4 >> (8 * e)) & 0xffu) v[e] = 0.f;
            }
            *reinterpret_cast<f32x4*>(Wt + n * ldt + k0 + kq) = v;
        }
    } else {
        for (int i = 0; i < 16; ++i) {
            const int idx = tid + 256 * i;
            const int nn = idx >> 6, kk = idx & 63;
            const int64_t k = k0 + kk, n = n0 + nn;
            if (n < N && k < ldt) {
                float v = (k < K) ? tile[kk][nn] : 0.f;
                if (k < K && dead && dead[(int64_t)((uint32_t)n / (uint32_t)gs) * K + k]) v = 0.f;
                Wt[n * ldt + k] = v;
            }
        }
    }
    if (bad) atomicOr(&st->flags, (uint32_t)kDevNonFinite);
}

__global__ void scales_kernel(const uint32_t* amax_bits, float* scales, float* rscale, int64_t N, int bits,
                              bool given, DevStatus* st) {
    const int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= N) return;
    float s;
    if (given) {
        s = scales[n];
        if (!(isfinite(s) && s > 0.f)) {
            atomicOr(&st->flags, (uint32_t)kDevNonFinite);
            s = 1.f;
        }
    } else {
        const float amax = __uint_as_float(amax_bits[n]);
        const float qmax = (float)((1 << bits) - 1);
        s = amax > 0.f ? (2.0f * amax) / qmax : 1.0f;   // IEEE division, round to nearest even
        scales[n] = s;
    }
    rscale[n] = 1.0f / s;
}

// Scales from W before the loop, one per (group of G original rows, channel): static groups, and the
// weight-MSE clipping of [G]'s main experiments (also for per-channel scales, G = K).  s = fp32(2 max|w| / qmax),
// or with clipping the candidate fp32(fp32(2 max|w| alpha_i) / qmax), alpha_i = 1.00, 0.99, .., 0.80, with the
// least sum of squared rounding errors over the group (first on ties).  A workgroup takes 16 channels of one
// group; 16 threads per channel split its rows and combine their maxima and error sums through LDS in a fixed
// order; the rows are read twice (max, then all 21 candidate errors at once).
constexpr int kShrink = 21;

template <bool BF16>
__global__ __launch_bounds__(256) void group_scales_kernel(const void* Wv, int64_t K, int64_t N, int64_t w_rs,
                                                          int64_t w_cs, int64_t G, int bits, bool mse,
                                                          float* scales) {
    __shared__ float part[16][kShrink][17];
    const int c = threadIdx.x & 15, r = threadIdx.x >> 4;            // channel in the workgroup, row part
    const int64_t n = (int64_t)blockIdx.x * 16 + c;
    const int64_t g = blockIdx.y;
    const int64_t k0 = g * G, k1 = min<int64_t>(K, k0 + G);
    const bool live = n < N;
    auto ld = [&](int64_t k) -> float {
        const int64_t off = k * w_rs + n * w_cs;
        return BF16 ? __uint_as_float((uint32_t)(static_cast<const uint16_t*>(Wv)[off]) << 16)
                    : static_cast<const float*>(Wv)[off];
    };
    float amax = 0.f;
    if (live)
        for (int64_t k = k0 + r; k < k1; k += 16) amax = fmaxf(amax, fabsf(ld(k)));
    part[r][0][c] = amax;
    __syncthreads();
    amax = 0.f;
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, part[i][0][c]);
    __syncthreads();
    const float qmax = (float)((1 << bits) - 1), z = (float)(1 << (bits - 1));
    const float base = 2.0f * amax;
    float s = base / qmax;
    if (mse && amax > 0.f) {   // the same for a channel's 16 threads; the barrier below is outside it
        float cand[kShrink], rcand[kShrink], err[kShrink];
#pragma unroll
        for (int i = 0; i < kShrink; ++i) {
            const float alpha = (float)(1.0 - i / 100.0);
            cand[i] = (base * alpha) / qmax;
            rcand[i] = 1.0f / cand[i];
            err[i] = 0.f;
        }
        for (int64_t k = k0 + r; k < k1; k += 16) {
            const float w = ld(k);
#pragma unroll
            for (int i = 0; i < kShrink; ++i) {
                const float cc = fminf(fmaxf(rintf(w * rcand[i]) + z, 0.f), qmax);
                const float d = w - (cc - z) * cand[i];
                err[i] = fmaf(d, d, err[i]);
            }
        }
#pragma unroll
        for (int i = 0; i < kShrink; ++i) part[r][i][c] = err[i];
    }
    __syncthreads();
    if (mse && amax > 0.f && r == 0) {
        float best_e = 0.f;
        int best = 0;
        for (int i = 0; i < kShrink; ++i) {
            float e = 0.f;
            for (int j = 0; j < 16; ++j) e += part[j][i][c];
            if (i == 0 || e < best_e) {
                best_e = e;
                best = i;
            }
        }
        s = ((base * (float)(1.0 - best / 100.0)) / qmax);
    }
    if (r == 0 && live) scales[g * N + n] = amax > 0.f ? s : 1.0f;
}

// Broadcast lane SRC of each 16-lane row to the whole row (DPP row_newbcast, gfx90a+).  Every lane reads a lane
// of its own row, so the destination's previous value does not matter.
template <int SRC>
__device__ __forceinline__ float row_bcast(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x150 + SRC, 0xF, 0xF, true));
}

struct BlockArgs {
    float* Wt; int64_t ldt;         // working weights, transposed
    const float* U; const float* P1; int64_t K;
    int64_t N;
    int64_t b0; int bs;             // block start and size (<= 128)
    const float* scales; const float* rscale;
    int bits;
    uint8_t* codes_t;               // N x ldt
    float* E;                       // this block's errors: N rows, stride lde
    float* Wpre;                    // this block's weights before rounding (asymmetric without CAE), stride lde
    int64_t lde;                    // row stride of E and Wpre
    const float* W0t;               // N x ldt original weights (CAE only)
    float* loss_acc;                // N
    float* pre_round;               // optional, K x N
    const DevStatus* st;
    int64_t G;                      // group size (group modes)
    int64_t gs, u_stride;           // output-channel groups: gs channels each, U and P1 of group g at + g u_stride
    const int32_t* perm;            // act-order (static groups look up the original row's group)
    float* gscales;                 // ng x N: written at group starts (re-estimated) or read (static)
    const float* Pnl;               // the super-block's block panels of U as staged in LDS (strip_prep_kernel), group 0
    const float* Ppn;               // the same for P1 (asymmetric term)
};

// Scale modes of the block kernel: one scale per channel; groups re-estimated from the current weights at each
// group start (processing order); static groups whose scales were computed from W before the loop.
enum : int { kScalePerChannel = 0, kScaleDynamic = 1, kScaleStatic = 2 };

// With one scale per channel the loop runs on the weights divided by the scale, v = w / s: the code is then
// rint(v) clamped, the step's error term v_j - c needs no multiply, and the slot updates v_k -= (U_jk / U_jj)(v_j - c)
// are those of the weights divided by s.  The errors E_j = (v_j - c) s / U_jj and the outputs are in weight units.
template <int SM>
constexpr bool kScaled = SM == kScalePerChannel;

// Per-lane state of the block kernel: 8 strided coordinates of one channel.  A coordinate's slot keeps its value
// just before rounding: the step that fixes coordinate j leaves slot j alone (the panel's entry (j, j) is zero), and
// later steps add zero to it (U is upper triangular), so codes, errors and losses are evaluated once at the end of
// the block from the kept values, with the same arithmetic as inside the step.
struct LaneState {
    float w[8], w0[8];
    float s, rs;                    // scale in force (and its reciprocal)
    float qs[4], qrs[4];            // re-estimated groups: the scale of each 32-coordinate quarter of the block
    float dp, wup;                  // the previous step's d and update value (its deferred slot updates use them)
};

struct StepConst {
    const float* Up; const float* Pp;
    const float* Ts; const float* Trs;   // static groups: per-step scales of this workgroup's 16 channels
    float clo, chi, qmax;                // signed code range -z .. qmax - z
    int l, ch;
    int64_t G, b0;
    float* gscales;
    int64_t N, n; bool live;
};

// Per-step operands read from LDS: this lane's 8 entries of row J of the scaled panel U_Jk / U_JJ (and of P1).
// Row J is read kAhead steps ahead into a ring of kRing entries, so no LDS latency sits on the chain of dependent
// steps; the ring also keeps row J - 1, whose update of most slots is applied during step J (see loop_step).
struct StepOps {
    f32x4 u0, u1, p0, p1;
    float s, rs;
};
constexpr int kAhead = 3;
constexpr int kRing = kAhead + 2;

template <int J, bool ASYM, int SM>
__device__ __forceinline__ void load_ops(StepOps& o, const StepConst& k) {
    if constexpr (J < kB) {
        if constexpr (SM == kScaleStatic) {
            o.s = k.Ts[J * 16 + k.ch];
            o.rs = k.Trs[J * 16 + k.ch];
        }
        // step J updates slots m..7 only (m = J / 16): entries below m are not read from LDS
        constexpr int m = J >> 4;
        // row J: entries 0-3 of the 16 lanes, then entries 4-7 (16 consecutive bytes per lane: conflict-free reads)
        const float* urow = k.Up + J * 128 + k.l * 4;
        if constexpr (m < 4) o.u0 = *reinterpret_cast<const f32x4*>(urow);
        if constexpr (m < 6) {
            o.u1 = *reinterpret_cast<const f32x4*>(urow + 64);
        } else {
            const f32x2 t = *reinterpret_cast<const f32x2*>(urow + 66);
            o.u1[2] = t[0];
            o.u1[3] = t[1];
        }
        if constexpr (ASYM) {
            const float* prow = k.Pp + J * 128 + k.l * 4;
            if constexpr (m < 4) o.p0 = *reinterpret_cast<const f32x4*>(prow);
            if constexpr (m < 6) {
                o.p1 = *reinterpret_cast<const f32x4*>(prow + 64);
            } else {
                const f32x2 t = *reinterpret_cast<const f32x2*>(prow + 66);
                o.p1[2] = t[0];
                o.p1[3] = t[1];
            }
        }
    }
}

// Re-estimated groups: at a group's first coordinate J the scale becomes 2 max|w| / qmax over the group's
// rows J .. J+G-1 of the current weights (registers m in [J/16, (J+G)/16) of the channel's 16 lanes).
template <int J>
__device__ __forceinline__ void regroup(LaneState& st, const StepConst& k) {
    if ((J & (k.G - 1)) != 0) return;
    constexpr int m0 = J >> 4;
    const int m1 = m0 + (int)(k.G >> 4);
    float mx = 0.f;
#pragma unroll
    for (int m = m0; m < 8; ++m)
        if (m < m1) mx = fmaxf(mx, fabsf(st.w[m]));
    mx = fmaxf(mx, __shfl_xor(mx, 8, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 4, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 2, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 1, 16));
    st.s = mx > 0.f ? (2.0f * mx) / k.qmax : 1.0f;
    st.rs = 1.0f / st.s;
    if (k.l == 0 && k.live) k.gscales[((k.b0 + J) / k.G) * k.N + k.n] = st.s;
}

// Signed code of v: round half to even, clamp to -z .. qmax - z.
__device__ __forceinline__ float signed_code(float v, const StepConst& k) {
    return __builtin_amdgcn_fmed3f(rintf(v), k.clo, k.chi);
}

// Entry MM of a lane's 8 panel entries (a, b: entries 0-3 and 4-7).
template <int MM>
__device__ __forceinline__ float entry(const f32x4& a, const f32x4& b) {
    if constexpr (MM < 4) return a[MM];
    else return b[MM - 4];
}

// The update of slot MM by a step with error term d: w -= (U_jk / U_jj) d, and with the asymmetric term
// w += P1_jk wu (o: that step's panel entries).
template <int MM, bool ASYM>
__device__ __forceinline__ void slot_update(LaneState& st, const StepOps& o, float d, float wu) {
    if constexpr (ASYM) st.w[MM] = fmaf(entry<MM>(o.p0, o.p1), wu, fmaf(-entry<MM>(o.u0, o.u1), d, st.w[MM]));
    else st.w[MM] = fmaf(-entry<MM>(o.u0, o.u1), d, st.w[MM]);
}

// Step P updates slots P/16 .. 7 (the slots holding coordinates after P).  Of these, the slot holding coordinate
// P + 1 is updated within step P (the next step broadcasts from it); the others, its "tail", are updated during step
// P + 1.  tail_slot(P, i) is the i-th slot of that tail, or -1.
constexpr int tail_slot(int P, int i) {
    if (P < 0) return -1;
    int cnt = 0;
    for (int mm = P >> 4; mm < 8; ++mm) {
        if (mm == ((P + 1) >> 4)) continue;
        if (cnt == i) return mm;
        ++cnt;
    }
    return -1;
}

template <int P, int I, bool ASYM>
__device__ __forceinline__ void tail_update(LaneState& st, const StepOps& op) {
    constexpr int mm = tail_slot(P, I);
    if constexpr (mm >= 0) slot_update<mm, ASYM>(st, op, st.dp, st.wup);
}

template <int P, bool ASYM>
__device__ __forceinline__ void tail_all(LaneState& st, const StepOps& op) {
    tail_update<P, 0, ASYM>(st, op);
    tail_update<P, 1, ASYM>(st, op);
    tail_update<P, 2, ASYM>(st, op);
    tail_update<P, 3, ASYM>(st, op);
    tail_update<P, 4, ASYM>(st, op);
    tail_update<P, 5, ASYM>(st, op);
    tail_update<P, 6, ASYM>(st, op);
}

#define GPTQ_SB() __builtin_amdgcn_sched_barrier(0)

// One step j of the loop (j compile-time so that slots, DPP lane and LDS offsets are immediates).  The chain
// from one step to the next is: broadcast w_j, scale, round, clamp, d = w_j - c s, then the update of the slot
// holding coordinate j + 1.  With the panel holding U_jk / U_jj, w_k -= (U_jk / U_jj) d is the update
// w_k -= U_jk E_j with E_j = d / U_jj; slot j itself has a zero entry and keeps its pre-rounding value.
// CAE: the update is taken from the original weight, d = w0_j - c s (the P2 = P1 + I - diag(U)^-1 U form), and the
// P1 coefficient is w0_j.
// DEFER (whole blocks): only the slot of coordinate j + 1 is updated on the chain; the other slots of step j - 1 are
// updated here, one between each pair of dependent chain instructions, where the wave would otherwise wait.  Every
// slot still receives the steps' updates in step order, so the results are those of updating all slots at once.
// The instruction order is fixed by scheduling barriers (the scheduler would otherwise sink the look-ahead reads to
// their uses and group the slot updates together).
template <int J, bool ASYM, bool CAE, int SM, bool DEFER>
__device__ __forceinline__ void loop_step(LaneState& st, const StepConst& k, StepOps (&ops)[kRing]) {
    constexpr int m = J >> 4, lj = J & 15, mn = (J + 1) >> 4, P = J - 1;
    const StepOps& o = ops[J % kRing];
    const StepOps& op = ops[(J + kRing - 1) % kRing];
    GPTQ_SB();
    constexpr bool kRegroup = SM == kScaleDynamic && (J & 31) == 0;
    if constexpr (kRegroup) {
        if constexpr (DEFER) tail_all<P, ASYM>(st, op);   // the group maximum reads the current weights
        regroup<J>(st, k);
        st.qs[J >> 5] = st.s;
        st.qrs[J >> 5] = st.rs;
    }
    if constexpr (SM == kScaleStatic) {
        st.s = o.s;
        st.rs = o.rs;
    }
    load_ops<J + kAhead, ASYM, SM>(ops[(J + kAhead) % kRing], k);
    if constexpr (DEFER) {
        constexpr int T0 = kRegroup ? 8 : 0;   // tail of step J - 1 already applied
        const float wj = row_bcast<lj>(st.w[m]);
        const float wu = CAE ? row_bcast<lj>(st.w0[m]) : wj;
        GPTQ_SB();
        tail_update<P, T0 + 0, ASYM>(st, op);
        GPTQ_SB();
        const float x = kScaled<SM> ? wj : wj * st.rs;
        GPTQ_SB();
        tail_update<P, T0 + 1, ASYM>(st, op);
        GPTQ_SB();
        const float r = rintf(x);
        GPTQ_SB();
        tail_update<P, T0 + 2, ASYM>(st, op);
        GPTQ_SB();
        const float c = __builtin_amdgcn_fmed3f(r, k.clo, k.chi);
        GPTQ_SB();
        tail_update<P, T0 + 3, ASYM>(st, op);
        GPTQ_SB();
        const float d = kScaled<SM> ? wu - c : fmaf(-c, st.s, wu);
        GPTQ_SB();
        tail_update<P, T0 + 4, ASYM>(st, op);
        GPTQ_SB();
        if constexpr (mn < 8) slot_update<mn, ASYM>(st, o, d, wu);
        GPTQ_SB();
        tail_update<P, T0 + 5, ASYM>(st, op);
        tail_update<P, T0 + 6, ASYM>(st, op);
        st.dp = d;
        st.wup = wu;
        // Row J - 1's registers are read for the last time here; keeping all of them live until here stops the
        // allocator from giving one to another value while the read of row J + kAhead into them is outstanding.
        asm volatile("" ::"v"(op.u0), "v"(op.u1));
        if constexpr (ASYM) asm volatile("" ::"v"(op.p0), "v"(op.p1));
    } else {
        const float wj = row_bcast<lj>(st.w[m]);
        const float c = signed_code(kScaled<SM> ? wj : wj * st.rs, k);
        const float wu = CAE ? row_bcast<lj>(st.w0[m]) : wj;     // value the update is taken from
        const float d = kScaled<SM> ? wu - c : fmaf(-c, st.s, wu);
#pragma unroll
        for (int mm = m; mm < 8; ++mm) {
            if constexpr (ASYM) {
                const float pp = mm < 4 ? o.p0[mm & 3] : o.p1[mm & 3];
                const float uu = mm < 4 ? o.u0[mm & 3] : o.u1[mm & 3];
                st.w[mm] = fmaf(pp, wu, fmaf(-uu, d, st.w[mm]));
            } else {
                const float uu = mm < 4 ? o.u0[mm & 3] : o.u1[mm & 3];
                st.w[mm] = fmaf(-uu, d, st.w[mm]);
            }
        }
        // The entries of slots below m are not needed, but their registers are the destinations of this step's LDS
        // read; keeping them live until here stops the allocator from reusing one while the read is in flight.
        asm volatile("" ::"v"(o.u0), "v"(o.u1));
        if constexpr (ASYM) asm volatile("" ::"v"(o.p0), "v"(o.p1));
    }
}

// The steps of one block.  WHOLE (all 128 coordinates): deferred slot updates, the last step's tail applied at the
// end; a ragged block (the last of a layer whose K is not a multiple of 128) updates every slot within its step.
template <bool ASYM, bool CAE, int SM, bool WHOLE, int... Js>
__device__ __forceinline__ void run_steps(LaneState& st, const StepConst& k, int bs,
                                          std::integer_sequence<int, Js...>) {
    StepOps ops[kRing];
    static_assert(kAhead == 3, "the prologue loads kAhead rows");
    load_ops<0, ASYM, SM>(ops[0], k);
    load_ops<1, ASYM, SM>(ops[1], k);
    load_ops<2, ASYM, SM>(ops[2], k);
    st.dp = 0.f;
    st.wup = 0.f;
    ((WHOLE || Js < bs ? loop_step<Js, ASYM, CAE, SM, WHOLE>(st, k, ops) : (void)0), ...);
    if constexpr (WHOLE) {
        GPTQ_SB();
        tail_all<kB - 1, ASYM>(st, ops[(kB - 1) % kRing]);
        asm volatile("" ::"v"(ops[(kB - 1) % kRing].u0), "v"(ops[(kB - 1) % kRing].u1));
    }
}

// Static groups: the scale (and reciprocal) of every step of the block for the workgroup's 16 channels, [step][channel].
__device__ __forceinline__ void stage_static_scales(float* Ts, float* Trs, const BlockArgs& p, int64_t b0, int bs,
                                                    int tid) {
    for (int idx = tid; idx < kB * kChPerWG; idx += 256) {
        const int j = idx >> 4;
        const int64_t nc = (int64_t)blockIdx.x * kChPerWG + (idx & 15);
        float sc = 1.0f;
        if (j < bs && nc < p.N) {
            const int64_t ko = p.perm ? (int64_t)p.perm[b0 + j] : b0 + j;
            sc = p.gscales[(ko / p.G) * p.N + nc];
        }
        Ts[idx] = sc;
        Trs[idx] = 1.0f / sc;
    }
}

// Per-lane set-up of the loop state for the block at b0 (slots from `wsrc`, coordinate 16 m + l at wsrc[16 m + l]).
template <bool CAE, int SM>
__device__ __forceinline__ void init_lane(LaneState& st, StepConst& k, const BlockArgs& p, const float* wsrc,
                                          const float* Up, const float* Pp, const float* Ts, const float* Trs,
                                          int64_t b0, int tid) {
    const int l = tid & 15;
    const int64_t n = (int64_t)blockIdx.x * kChPerWG + (tid >> 4);
    const bool live = n < p.N;
    const int64_t nn = live ? n : 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        st.qs[q] = 1.0f;
        st.qrs[q] = 1.0f;
    }
    if constexpr (SM == kScalePerChannel) {
        st.s = p.scales[nn];
        st.rs = p.rscale[nn];
    } else {
        st.s = 1.0f;
        st.rs = 1.0f;
    }
    const float* w0row = CAE ? p.W0t + nn * p.ldt + b0 : nullptr;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        st.w[m] = wsrc[16 * m + l];
        if constexpr (CAE) st.w0[m] = w0row[16 * m + l];
        if constexpr (kScaled<SM>) {
            st.w[m] *= st.rs;
            if constexpr (CAE) st.w0[m] *= st.rs;
        }
    }
    k.Up = Up; k.Pp = Pp; k.Ts = Ts; k.Trs = Trs;
    const float z = (float)(1 << (p.bits - 1));
    k.qmax = (float)((1 << p.bits) - 1);
    k.clo = -z;
    k.chi = k.qmax - z;
    k.l = l;
    k.ch = tid >> 4;
    k.G = p.G; k.b0 = b0; k.gscales = p.gscales;
    k.N = p.N; k.n = n; k.live = live;
}

// End of a block: codes, errors, pre-rounding values and the loss from the kept pre-rounding values, with the step's
// arithmetic.  Es (optional): the block's errors are also written to LDS as Es[channel][j] (row pitch kEsPitch).
constexpr int kEsPitch = kB + 1;
template <bool ASYM, bool CAE, int SM, bool WHOLE>
__device__ __forceinline__ void block_epilogue(const LaneState& st, const StepConst& k, const BlockArgs& p,
                                               const float* rdiag, const float* Ts, const float* Trs, int64_t b0,
                                               int bs, float* Es) {
    const int l = k.l;
    const int64_t n = k.n;
    const bool live = k.live;
    const int64_t nn = live ? n : 0;
    const float z = -k.clo;
    float loss = 0.f;
    uint8_t* crow = p.codes_t + nn * p.ldt + b0;
    float* erow = p.E + nn * p.lde;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int j = 16 * m + l;
        float s = st.s, rs = st.rs;
        if constexpr (SM == kScaleDynamic) {
            s = st.qs[m >> 1];
            rs = st.qrs[m >> 1];
        }
        if constexpr (SM == kScaleStatic) {
            s = Ts[j * 16 + k.ch];
            rs = Trs[j * 16 + k.ch];
        }
        float eo = 0.f;   // the error the trailing updates use
        if (WHOLE || j < bs) {
            const float v = kScaled<SM> ? st.w[m] : st.w[m] * rs;
            const float c = signed_code(v, k);
            const float r = rdiag[j];
            const float e = (kScaled<SM> ? (v - c) * s : fmaf(-c, s, st.w[m])) * r;
            loss = fmaf(e, e, loss);
            eo = CAE ? (kScaled<SM> ? (st.w0[m] - c) * s : fmaf(-c, s, st.w0[m])) * r : e;
            if (live) {
                crow[j] = (uint8_t)(uint32_t)(c + z);
                if (ASYM && !CAE) p.Wpre[n * p.lde + j] = kScaled<SM> ? st.w[m] * s : st.w[m];
                if (p.pre_round) p.pre_round[(b0 + j) * p.N + n] = v;
            }
        } else if (live && ASYM && !CAE) {
            p.Wpre[n * p.lde + j] = 0.f;
        }
        if (live) erow[j] = eo;
        if (Es) Es[k.ch * kEsPitch + j] = eo;
    }
    // the channel's loss: sum over its 16 lanes
    loss += __shfl_xor(loss, 8, 16);
    loss += __shfl_xor(loss, 4, 16);
    loss += __shfl_xor(loss, 2, 16);
    loss += __shfl_xor(loss, 1, 16);
    if (l == 0 && live) p.loss_acc[n] += 0.5f * loss;
}

// A block's panel as the loop kernels hold it in LDS: the scaled U rows in the step layout, then rdiag, then padding
// to a whole number of 1 KB DMA transfers (65 of them, one per wave instruction); a P1 panel likewise (unscaled, the
// rdiag part zero).  Prepared once per super-block by strip_prep_kernel.
constexpr int kPnl = kB * kB + 256;
static_assert(kPnl % 256 == 0, "whole 1 KB transfers");

typedef __attribute__((address_space(3))) void lds_void_t;

// The prepared panel `src` (kPnl floats in HBM) into LDS `dst` by LDS DMA (no registers): wave w issues transfers
// w, w + 4, ...; transfer i moves floats 256 i .. 256 i + 255, lane l's 16 bytes to dst + 256 i + 4 l.  The caller
// waits for them (vmcnt) before the barrier after which they are read.
__device__ __forceinline__ void panel_dma(float* dst, const float* src, int wave, int lane) {
    for (int i = wave; i < kPnl / 256; i += 4)
        __builtin_amdgcn_global_load_lds((const void*)(src + 256 * i + 4 * lane), (lds_void_t*)(dst + 256 * i), 16, 0,
                                         0);
}

// One block of 128 coordinates per launch (the asymmetric variants).  WHOLE: the block has all 128 coordinates
// (every block but a ragged last one), so the steps carry no bounds test.
template <bool ASYM, bool CAE, int SM, bool WHOLE>
__global__ __launch_bounds__(256) void quant_block_kernel(BlockArgs p) {
    __shared__ __attribute__((aligned(16))) float Upr[kPnl];                 // [row j][slots 0-3, 4-7][16 lanes][4], then rdiag
    __shared__ __attribute__((aligned(16))) float Ppr[ASYM ? kPnl : 4];      // same layout (asymmetric)
    float* const Up = Upr;
    float* const Pp = Ppr;
    float* const rdiag = Upr + kB * kB;
    __shared__ float Ts[SM == kScaleStatic ? kB * kChPerWG : 1];           // [step][channel] static scales
    __shared__ float Trs[SM == kScaleStatic ? kB * kChPerWG : 1];

    if (p.st->flags) return;   // an input was rejected earlier in this call
    {   // output-channel groups: the workgroup's channels all belong to one group (gs is a multiple of 16)
        const int64_t g = (int64_t)blockIdx.x * kChPerWG / p.gs;
        p.U += g * p.u_stride;
        if (p.P1) p.P1 += g * p.u_stride;
        if (p.perm) p.perm += g * p.K;
        p.Pnl += g * (int64_t)(kSB / kB) * kPnl;
        if (ASYM) p.Ppn += g * (int64_t)(kSB / kB) * kPnl;
    }
    const int tid = threadIdx.x;
    const int64_t b0 = p.b0;
    const int bs = WHOLE ? kB : p.bs;
    {   // the block's prepared panels by DMA (super-blocks start at multiples of kSB)
        const int64_t bi = (b0 % kSB) / kB;
        panel_dma(Upr, p.Pnl + bi * kPnl, tid >> 6, tid & 63);
        if constexpr (ASYM) panel_dma(Ppr, p.Ppn + bi * kPnl, tid >> 6, tid & 63);
    }
    if constexpr (SM == kScaleStatic) stage_static_scales(Ts, Trs, p, b0, bs, tid);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the panels' DMA transfers have landed
    __syncthreads();

    const int64_t n = (int64_t)blockIdx.x * kChPerWG + (tid >> 4);
    LaneState st;
    StepConst k;
    init_lane<CAE, SM>(st, k, p, p.Wt + (n < p.N ? n : 0) * p.ldt + b0, Up, Pp, Ts, Trs, b0, tid);
    run_steps<ASYM, CAE, SM, WHOLE>(st, k, bs, std::make_integer_sequence<int, kB>{});
    block_epilogue<ASYM, CAE, SM, WHOLE>(st, k, p, rdiag, Ts, Trs, b0, bs, nullptr);
}

// One super-block of up to kSBS coordinates per launch for 16 channels (the variants without the asymmetric term):
// the channels' weights of the super-block stay in LDS (Ws, 16 x kSBS fp32), the blocks run one after the other,
// and after each block the rows of the super-block still to come get its update W -= E_B U[B, rows] right here,
// 16 channels x 16 rows per MFMA tile with fp32 accuracy: -E and the U rows each split into three bf16 parts (U's
// parts prepared once per super-block by strip_prep_kernel), the six part products of order <= 2 accumulated by
// v_mfma_f32_16x16x32_bf16 from zero and the sum added to Ws once.  No separate product runs between the blocks;
// only the rows after the super-block are left to the trailing product that follows the launch.
constexpr int kSBS = 8 * kB;          // super-block of the strip kernel (its near rows are updated in-kernel)
static_assert(kSBS == kSB, "both loop kernels take their panels from one per-super-block preparation");
constexpr int kWsPitch = kSBS + 12;   // the near update's accesses of one instruction (channels 4 g + q, g = 0..3) hit disjoint banks
constexpr int64_t kStripMaxWG = 512;   // up to two rounds of one workgroup per CU

struct StripArgs {
    BlockArgs p;
    int64_t sb0, sb1;      // super-block [sb0, sb1)
    const uint16_t* Usp;   // the super-block's diagonal block of U in three bf16 parts (strip_prep_kernel), per group
};

// fp32-accurate products on the bf16 MFMA: v = h0 + h1 + h2 + O(2^-24 |v|), each part the round-to-nearest-even bf16
// of the remainder; the six part products of order <= 2 summed in fp32 equal the fp32 product to that order.  Two
// values at once, one packed conversion per part; word q holds part q of `lo` (low half) and of `hi` (high half).
typedef __attribute__((ext_vector_type(2))) float f32x2_q;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_q;
__device__ __forceinline__ void split3_pair(float lo, float hi, uint32_t& w0, uint32_t& w1, uint32_t& w2) {
    const f32x2_q v = {lo, hi};
    const bf16x2_q b0 = __builtin_convertvector(v, bf16x2_q);
    const f32x2_q r1 = v - __builtin_convertvector(b0, f32x2_q);
    const bf16x2_q b1 = __builtin_convertvector(r1, bf16x2_q);
    const f32x2_q r2 = r1 - __builtin_convertvector(b1, f32x2_q);
    const bf16x2_q b2 = __builtin_convertvector(r2, bf16x2_q);
    w0 = __builtin_bit_cast(uint32_t, b0);
    w1 = __builtin_bit_cast(uint32_t, b1);
    w2 = __builtin_bit_cast(uint32_t, b2);
}

// Eight values -> their three parts, each as 8 bf16 in 16 bytes (element i = value i).
__device__ __forceinline__ void split3_oct(const float (&v)[8], u32x4 (&w)[3]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        uint32_t x0, x1, x2;
        split3_pair(v[2 * e], v[2 * e + 1], x0, x1, x2);
        w[0][e] = x0;
        w[1][e] = x1;
        w[2][e] = x2;
    }
}

// Per super-block set-up of the loop kernels, for every group's U (blockIdx.y), in one launch:
// - blocks [0, nsplit): the diagonal block [sb0, sb0 + kSBS)^2 split into three bf16 parts, in the layout of the near
//   update's MFMA B operand: part q, row octet o (rows sb0 + 8 o .. + 7), column sb0 + r as 8 bf16 at
//   Usp[((q * kSBS / 8 + o) * kSBS + r) * 8] (group g at + g 3 kSBS^2).  Zero beyond K.  One thread per (o, r).
// - the next npanel = nblk * kPnl / 256 blocks: the panels of the super-block's blocks as the loop kernels hold them
//   in LDS: Pnl[bi kPnl + 128 j + 64 (m / 4) + 4 l + m % 4] = U_jc * rcp(U_jj) for c = 16 m + l > j (0 otherwise
//   and beyond the block), rdiag[j] = rcp(U_jj) at Pnl[bi kPnl + kB kB + j]; group g at + g 8 kPnl.
// - with P1, the next npanel blocks: its panels in the same layout, P1_jc as it is (strictly upper), at Ppn.
__global__ __launch_bounds__(256) void strip_prep_kernel(const float* U, const float* P1, int64_t K, int64_t u_stride,
                                                         int64_t sb0, int64_t sb1, int nsplit, int npanel,
                                                         uint16_t* Usp, float* Pnl, float* Ppn) {
    const int64_t g = blockIdx.y;
    U += g * u_stride;
    if ((int)blockIdx.x < nsplit) {
        Usp += g * (int64_t)3 * kSBS * kSBS;
        const int idx = blockIdx.x * 256 + threadIdx.x;
        const int o = idx / kSBS, r = idx % kSBS;
        const int64_t c = sb0 + r;
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t j = sb0 + 8 * o + i;
            v[i] = (j < K && c < K) ? U[j * K + c] : 0.f;
        }
        u32x4 w[3];
        split3_oct(v, w);
#pragma unroll
        for (int q = 0; q < 3; ++q)
            *reinterpret_cast<u32x4*>(Usp + (((int64_t)q * (kSBS / 8) + o) * kSBS + r) * 8) = w[q];
        return;
    }
    const bool p1 = (int)blockIdx.x >= nsplit + npanel;   // P1 panels: unscaled, no rdiag
    const int idx = ((int)blockIdx.x - nsplit - (p1 ? npanel : 0)) * 256 + threadIdx.x;
    const int bi = idx / kPnl, e = idx % kPnl;
    const int64_t b0 = sb0 + (int64_t)bi * kB;
    if (b0 >= sb1) return;
    const int bs = (int)min<int64_t>(kB, K - b0);
    float* out = (p1 ? Ppn : Pnl) + g * (int64_t)(kSBS / kB) * kPnl + (int64_t)bi * kPnl;
    if (p1) {
        P1 += g * u_stride;
        const int j = e >> 7, l = (e >> 2) & 15, m = ((e >> 6) & 1) * 4 + (e & 3), c = 16 * m + l;
        out[e] = (e < kB * kB && j < bs && c < bs) ? P1[(b0 + j) * K + b0 + c] : 0.f;
        return;
    }
    if (e < kB * kB) {
        const int j = e >> 7, l = (e >> 2) & 15, m = ((e >> 6) & 1) * 4 + (e & 3), c = 16 * m + l;
        const float r = j < bs ? __builtin_amdgcn_rcpf(U[(b0 + j) * K + b0 + j]) : 0.f;
        const float u = (j < bs && c < bs) ? U[(b0 + j) * K + b0 + c] : 0.f;
        out[e] = c > j ? u * r : 0.f;
    } else {
        const int j = e - kB * kB;
        out[e] = j < bs ? __builtin_amdgcn_rcpf(U[(b0 + j) * K + b0 + j]) : 0.f;
    }
}

template <bool CAE, int SM>
__global__ __launch_bounds__(256) void quant_strip_kernel(StripArgs a) {
    __shared__ __attribute__((aligned(16))) float Ws[kChPerWG * kWsPitch];   // [channel][coordinate - sb0]
    __shared__ __attribute__((aligned(16))) float Upr[kPnl];   // the block's panel (kB x kB), then rdiag
    float* const Up = Upr;
    float* const rdiag = Upr + kB * kB;
    __shared__ float Es[kChPerWG * kEsPitch];                                // [channel][j] this block's errors
    __shared__ float Ts[SM == kScaleStatic ? kB * kChPerWG : 1];
    __shared__ float Trs[SM == kScaleStatic ? kB * kChPerWG : 1];

    BlockArgs& p = a.p;
    if (p.st->flags) return;
    {
        const int64_t g = (int64_t)blockIdx.x * kChPerWG / p.gs;
        p.U += g * p.u_stride;
        if (p.perm) p.perm += g * p.K;
        a.Usp += g * (int64_t)3 * kSBS * kSBS;
        p.Pnl += g * (int64_t)(kSBS / kB) * kPnl;
    }
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t sb0 = a.sb0, sb1 = a.sb1;
    const int64_t nbase = (int64_t)blockIdx.x * kChPerWG;
    // the super-block's weights of the 16 channels (zero for channels beyond N; Wt is zero-padded up to ldt): every
    // load issued before the LDS stores
    const int64_t width = ((sb1 - sb0) + kB - 1) / kB * kB;
    panel_dma(Upr, p.Pnl, wave, lane);   // the first block's panel
    {
        constexpr int kWV = kChPerWG * kSBS / 4 / 256;   // 16-byte vectors per thread for a full super-block
        f32x4 wv[kWV];
#pragma unroll
        for (int i = 0; i < kWV; ++i) {
            const int idx = tid + 256 * i, ch = idx / (kSBS / 4);
            const int64_t c4 = (int64_t)(idx % (kSBS / 4)) * 4;
            wv[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (c4 < width && nbase + ch < p.N) wv[i] = *reinterpret_cast<const f32x4*>(p.Wt + (nbase + ch) * p.ldt + sb0 + c4);
        }
#pragma unroll
        for (int i = 0; i < kWV; ++i) {
            const int idx = tid + 256 * i, ch = idx / (kSBS / 4);
            const int c4 = (idx % (kSBS / 4)) * 4;
            *reinterpret_cast<f32x4*>(&Ws[ch * kWsPitch + c4]) = wv[i];
        }
    }
    if constexpr (SM == kScaleStatic) stage_static_scales(Ts, Trs, p, sb0, (int)min<int64_t>(kB, p.K - sb0), tid);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the panel's DMA transfers have landed
    __syncthreads();

    for (int64_t b0 = sb0; b0 < sb1; b0 += kB) {
        const int bs = (int)min<int64_t>(kB, p.K - b0);
        // here: this block's panel is staged and Ws holds its compensated weights
        BlockArgs pb = p;
        pb.E = p.E + (b0 - sb0);
        LaneState st;
        StepConst k;
        init_lane<CAE, SM>(st, k, pb, &Ws[(tid >> 4) * kWsPitch + (b0 - sb0)], Up, nullptr, Ts, Trs, b0, tid);
        const int64_t bn = b0 + kB;
        const bool next = bn < sb1;
        const int bsn = next ? (int)min<int64_t>(kB, p.K - bn) : 0;
        if (bs == kB) {
            run_steps<false, CAE, SM, true>(st, k, bs, std::make_integer_sequence<int, kB>{});
            block_epilogue<false, CAE, SM, true>(st, k, pb, rdiag, Ts, Trs, b0, bs, Es);
        } else {
            run_steps<false, CAE, SM, false>(st, k, bs, std::make_integer_sequence<int, kB>{});
            block_epilogue<false, CAE, SM, false>(st, k, pb, rdiag, Ts, Trs, b0, bs, Es);
        }
        __syncthreads();   // Es complete; the panel and this block's slots of Ws are no longer read


        // rows b1..sb1-1 of the super-block: Ws[ch][r] -= sum_j Es[ch][j] U[b0 + j][r]  (whole blocks only: a ragged
        // block is the last of the layer)
        const int64_t b1 = b0 + bs;
        if (b1 < sb1) {
            // A operand of 32-coordinate chunk c: parts of -E[channel lane % 16][32 c + 8 (lane / 16) + i], i = 0..7
            u32x4 ea[kB / 32][3];
#pragma unroll
            for (int c = 0; c < kB / 32; ++c) {
                float v[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) v[i] = -Es[(lane & 15) * kEsPitch + 32 * c + 8 * (lane >> 4) + i];
                split3_oct(v, ea[c]);
            }
            const int64_t ntile = (sb1 - b1 + 15) / 16;
            const int oct0 = (int)((b0 - sb0) / 8) + (lane >> 4);
            // B operand of chunk c for tile t: parts of U[b0 + 32 c + 8 (lane / 16) + i][b1 + 16 t + lane % 16]
            auto load_b = [&](int64_t t, u32x4 (&bq)[kB / 32][3]) {
                const int64_t rl = b1 - sb0 + 16 * t + (lane & 15);
#pragma unroll
                for (int c = 0; c < kB / 32; ++c)
#pragma unroll
                    for (int q = 0; q < 3; ++q)
                        bq[c][q] = *reinterpret_cast<const u32x4*>(
                            a.Usp + (((int64_t)q * (kSBS / 8) + oct0 + 4 * c) * kSBS + rl) * 8);
            };
            // Ws[channels][tile t] += -E U over the 128 coordinates of the block: per chunk the six part products
            // (small parts first) on v_mfma_f32_16x16x32_bf16, two accumulators, summed and added to the weights once
            // (one rounding of the weights per block, as by a separate product with beta = 1)
            auto update = [&](int64_t t, const u32x4 (&bq)[kB / 32][3]) {
                f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
                for (int c = 0; c < kB / 32; ++c) {
                    f32x4& ac = acc[c & 1];
                    auto mm = [&](const u32x4& x, const u32x4& y) {
                        ac = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x),
                                                                     __builtin_bit_cast(bf16x8, y), ac, 0, 0, 0);
                    };
                    mm(ea[c][2], bq[c][0]);
                    mm(ea[c][1], bq[c][1]);
                    mm(ea[c][0], bq[c][2]);
                    mm(ea[c][1], bq[c][0]);
                    mm(ea[c][0], bq[c][1]);
                    mm(ea[c][0], bq[c][0]);
                }
                const f32x4 sum = acc[0] + acc[1];
                float* wc = &Ws[(4 * (lane >> 4)) * kWsPitch + (b1 + 16 * t + (lane & 15) - sb0)];
                float cur[4];   // the four reads issued together, then the sums written
#pragma unroll
                for (int q = 0; q < 4; ++q) cur[q] = wc[q * kWsPitch];
#pragma unroll
                for (int q = 0; q < 4; ++q) wc[q * kWsPitch] = cur[q] + sum[q];
            };
            // tiles wave, wave + 4, ... (a quarter of the block's at most (kSBS - kB) / 16 tiles per wave) in a loop
            // of two tiles on two operand buffers: the B operands of the next tile are loaded while a tile is
            // computed.  That load is issued on every path (past the wave's last tile it repeats tile ntile - 1, which
            // is in bounds), so the wait before a tile's products is for that tile's loads alone and never for the
            // ones just issued.
            if (wave < ntile) {
                u32x4 ub0[kB / 32][3], ub1[kB / 32][3];
                int64_t t = wave;
                load_b(t, ub0);
                // scheduling barriers keep each prefetch ahead of the products (the scheduler would otherwise sink
                // the loads to their uses to save registers)
                for (;;) {
                    load_b(min<int64_t>(t + 4, ntile - 1), ub1);
                    __builtin_amdgcn_sched_barrier(0);
                    update(t, ub0);
                    __builtin_amdgcn_sched_barrier(0);
                    t += 4;
                    if (t >= ntile) break;
                    load_b(min<int64_t>(t + 4, ntile - 1), ub0);
                    __builtin_amdgcn_sched_barrier(0);
                    update(t, ub1);
                    __builtin_amdgcn_sched_barrier(0);
                    t += 4;
                    if (t >= ntile) break;
                }
            }
        }
        // the next block's panel by DMA after the near update (DMA transfers in flight during the near update's
        // loop make the compiler wait for every outstanding load there, the tile prefetch included)
        if (next) panel_dma(Upr, p.Pnl + (int64_t)((bn - sb0) / kB) * kPnl, wave, lane);
        if (next && SM == kScaleStatic) stage_static_scales(Ts, Trs, p, bn, bsn, tid);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the next panel's DMA transfers have landed
        __syncthreads();   // Ws updated and the next panel staged before the next block reads them
    }
}

// codes_t (N x ldt) -> codes (K x N view with strides); W_hat = s (c - z) in the weight dtype; losses copy.
// Processing position k is written to original row perm[k]; its scale is scales[n] (per channel) or
// scales[g N + n] with g = k / G (groups re-estimated in processing order) or perm[k] / G (static groups).
template <bool BF16>
__global__ __launch_bounds__(256) void finalize_kernel(const uint8_t* codes_t, int64_t ldt, int64_t K, int64_t N,
                                                      uint8_t* codes, int64_t c_rs, int64_t c_cs, void* W_hat,
                                                      int64_t w_rs, int64_t w_cs, const float* scales, int bits,
                                                      const int32_t* perm, int64_t G, bool static_groups,
                                                      int64_t gs) {
    __shared__ uint8_t tile[64][65];
    const int tid = threadIdx.x;
    const int64_t k0 = (int64_t)blockIdx.y * 64, n0 = (int64_t)blockIdx.x * 64;
    // Whole tile, codes only, natural order, channels contiguous in 16-byte rows: one 16-byte load of codes_t and
    // one 16-byte store of codes per thread (the general path moves a byte per lane and access).
    const bool fast = !W_hat && !perm && c_cs == 1 && k0 + 64 <= K && n0 + 64 <= N && c_rs % 16 == 0 &&
                      (reinterpret_cast<uintptr_t>(codes) & 15) == 0;
    if (fast) {
        {
            const int nn = tid >> 2, kq = (tid & 3) * 16;
            const u32x4 c = *reinterpret_cast<const u32x4*>(codes_t + (n0 + nn) * ldt + k0 + kq);
#pragma unroll
            for (int e = 0; e < 16; ++e) tile[kq + e][nn] = (uint8_t)(c[e >> 2] >> (8 * (e & 3)));
        }
        __syncthreads();
        const int kk = tid >> 2, nq = (tid & 3) * 16;
        u32x4 o;
#pragma unroll
        for (int w = 0; w < 4; ++w)
            o[w] = (uint32_t)tile[kk][nq + 4 * w] | ((uint32_t)tile[kk][nq + 4 * w + 1] << 8) |
                   ((uint32_t)tile[kk][nq + 4 * w + 2] << 16) | ((uint32_t)tile[kk][nq + 4 * w + 3] << 24);
        *reinterpret_cast<u32x4*>(codes + (k0 + kk) * c_rs + n0 + nq) = o;
        return;
    }
    for (int i = 0; i < 16; ++i) {
        const int idx = tid + 256 * i;
        const int nn = idx >> 6, kk = idx & 63;
        const int64_t k = k0 + kk, n = n0 + nn;
        tile[kk][nn] = (k < K && n < N) ? codes_t[n * ldt + k] : (uint8_t)0;
    }
    __syncthreads();
    const bool n_fast_c = (c_cs == 1) || (c_rs != 1 && c_cs <= c_rs);
    const bool n_fast_w = (w_cs == 1) || (w_rs != 1 && w_cs <= w_rs);
    const float z = (float)(1 << (bits - 1));
    for (int i = 0; i < 16; ++i) {
        const int idx = tid + 256 * i;
        const int a = idx >> 6, b = idx & 63;
        {
            const int kk = n_fast_c ? a : b, nn = n_fast_c ? b : a;
            const int64_t k = k0 + kk, n = n0 + nn;
            if (k < K && n < N) {
                const int64_t gK = (int64_t)((uint32_t)n / (uint32_t)gs) * K;
                codes[(perm ? (int64_t)perm[gK + k] : k) * c_rs + n * c_cs] = tile[kk][nn];
            }
        }
        if (W_hat) {
            const int kk = n_fast_w ? a : b, nn = n_fast_w ? b : a;
            const int64_t k = k0 + kk, n = n0 + nn;
            if (k < K && n < N) {
                const int64_t gK = (int64_t)((uint32_t)n / (uint32_t)gs) * K;
                const int64_t ko = perm ? (int64_t)perm[gK + k] : k;
                const float s = G > 0 ? scales[((static_groups ? ko : k) / G) * N + n] : scales[n];
                const float v = ((float)tile[kk][nn] - z) * s;
                if (BF16) static_cast<__bf16*>(W_hat)[ko * w_rs + n * w_cs] = (__bf16)v;
                else static_cast<float*>(W_hat)[ko * w_rs + n * w_cs] = v;
            }
        }
    }
}

__global__ void copy_losses_kernel(const float* src, float* dst, int64_t N) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < N) dst[i] = src[i];
}

// Group of every original row: processing position j (original row perm[j]) is in group j / G (re-estimated
// groups) or perm[j] / G (static groups); 0 with one scale per channel.
__global__ void g_idx_kernel(int32_t* g_idx, int64_t K, const int32_t* perm, int64_t G, bool static_groups) {
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= K) return;
    g_idx += (int64_t)blockIdx.y * K;   // one row of K per output-channel group
    if (perm) perm += (int64_t)blockIdx.y * K;
    const int64_t ko = perm ? (int64_t)perm[j] : j;
    g_idx[ko] = G > 0 ? (int32_t)((static_groups ? ko : j) / G) : 0;
}

struct QuantLayout {
    DevStatus* st;
    uint32_t* amax;
    float* rscale;
    float* loss_acc;
    float* Wt;
    uint8_t* codes_t;
    float* E;
    float* Wpre;
    float* W0t;
    uint16_t* Usp;
    float* Pnl;
    float* Ppn;
    size_t bytes;
};

// The column loop of N channels in `groups` output-channel groups runs on the strip kernel when it has no asymmetric
// term and one workgroup per CU covers every channel.
bool strip_path(int64_t N, bool asym) { return !asym && ceil_div(N, kChPerWG) <= kStripMaxWG; }

QuantLayout carve(void* ws, int64_t K, int64_t N, bool asym, bool cae, int64_t groups) {
    const int64_t ldt = ceil_div(std::max<int64_t>(K, 1), kB) * kB;
    Carver c(ws);
    QuantLayout L;
    L.st = c.take<DevStatus>(1);
    L.amax = c.take<uint32_t>((size_t)N);
    L.rscale = c.take<float>((size_t)N);
    L.loss_acc = c.take<float>((size_t)N);
    L.Wt = c.take<float>((size_t)N * ldt);
    L.codes_t = c.take<uint8_t>((size_t)N * ldt);
    L.E = c.take<float>((size_t)N * kSB);
    L.Wpre = asym && !cae ? c.take<float>((size_t)N * kSB) : nullptr;
    L.W0t = cae ? c.take<float>((size_t)N * ldt) : nullptr;
    L.Usp = strip_path(N, asym) ? c.take<uint16_t>((size_t)std::max<int64_t>(groups, 1) * 3 * kSBS * kSBS) : nullptr;
    L.Pnl = c.take<float>((size_t)std::max<int64_t>(groups, 1) * (kSBS / kB) * kPnl);
    L.Ppn = asym ? c.take<float>((size_t)std::max<int64_t>(groups, 1) * (kSBS / kB) * kPnl) : nullptr;
    L.bytes = c.bytes();
    return L;
}

}  // namespace

size_t quantize_workspace_bytes(int64_t K, int64_t N, bool asym, bool cae, int64_t groups) {
    return carve(nullptr, K, N, asym, cae, groups).bytes;
}

gptq_status_t quantize_layer(const QuantizeArgs& a, void* workspace, hipStream_t stream) {
    const bool asym = a.P1 != nullptr;
    const int64_t K = a.K, N = a.N;
    const int64_t ldt = ceil_div(std::max<int64_t>(K, 1), kB) * kB;
    const bool cae = a.cae;
    const int64_t groups = std::max<int64_t>(a.groups, 1), gs = N / groups;   // output-channel groups
    QuantLayout L = carve(workspace, K, N, asym, cae, groups);

    const int64_t G = a.groupsize;
    const int sm = G == 0 ? kScalePerChannel : (a.static_groups ? kScaleStatic : kScaleDynamic);
    {
    TimerScope ts(stream, GPTQ_TIMER_OTHER);
    hipLaunchKernelGGL(quant_init_kernel, grid1d(std::max<int64_t>(N, 1), 256), dim3(256), 0, stream, L.st, L.amax,
                       L.loss_acc, N);
    GPTQ_LAUNCH_CHECK();
    {
        dim3 grid((unsigned)ceil_div(N, 64), (unsigned)ceil_div(ldt, 64));
        if (a.w_dtype == GPTQ_DTYPE_BF16)
            hipLaunchKernelGGL((convert_kernel<true>), grid, dim3(256), 0, stream, a.W, K, N, a.w_rs, a.w_cs, a.dead,
                               L.Wt, ldt, L.amax, L.st, a.perm, gs);
        else
            hipLaunchKernelGGL((convert_kernel<false>), grid, dim3(256), 0, stream, a.W, K, N, a.w_rs, a.w_cs, a.dead,
                               L.Wt, ldt, L.amax, L.st, a.perm, gs);
        GPTQ_LAUNCH_CHECK();
    }
    if (G == 0 && !a.mse) {
        hipLaunchKernelGGL(scales_kernel, grid1d(N, 256), dim3(256), 0, stream, L.amax, a.scales, L.rscale, N, a.bits,
                           a.scales_given, L.st);
        GPTQ_LAUNCH_CHECK();
    } else if (sm != kScaleDynamic) {
        // scales from W before the loop: MSE-clipped per channel (one group of K rows) or static groups
        const int64_t gsz = G == 0 ? K : G;
        dim3 grid((unsigned)ceil_div(N, 16), (unsigned)ceil_div(K, gsz));
        if (a.w_dtype == GPTQ_DTYPE_BF16)
            hipLaunchKernelGGL((group_scales_kernel<true>), grid, dim3(256), 0, stream, a.W, K, N, a.w_rs, a.w_cs, gsz,
                               a.bits, a.mse, a.scales);
        else
            hipLaunchKernelGGL((group_scales_kernel<false>), grid, dim3(256), 0, stream, a.W, K, N, a.w_rs, a.w_cs, gsz,
                               a.bits, a.mse, a.scales);
        GPTQ_LAUNCH_CHECK();
        if (G == 0) {   // reciprocals for the per-channel loop
            hipLaunchKernelGGL(scales_kernel, grid1d(N, 256), dim3(256), 0, stream, L.amax, a.scales, L.rscale, N,
                               a.bits, true, L.st);
            GPTQ_LAUNCH_CHECK();
        }
    }
    if (cae)   // the original weights (dead rows zeroed), read by every step and by the trailing updates
        GPTQ_HIP_CHECK(hipMemcpyAsync(L.W0t, L.Wt, sizeof(float) * (size_t)N * (size_t)ldt, hipMemcpyDeviceToDevice,
                                      stream));
    }

    // Wt[:, r0:r1] -= E U[k0:k0+depth, r0:r1] (+ Wpre P1[k0:k0+depth, r0:r1] for the asymmetric term; with CAE,
    // E holds (w0 - q) / U_jj and the P1 term takes the original weights W0[:, k0:k0+depth]).  E and Wpre point
    // at the errors / pre-rounding weights of coordinate k0 (row stride kSB).
    // With output-channel groups the product runs batched over the groups: group g's gs channels (rows of E, Wt)
    // with its own U and P1.
    auto trailing = [&](int64_t r0, int64_t r1, int64_t k0, int64_t depth, const float* Ek, const float* Wpk) {
        GemmArgs g;
        g.M = gs; g.N = r1 - r0; g.K1 = depth;
        g.A1 = Ek; g.lda1 = kSB; g.strideA1 = gs * kSB;
        g.B1 = a.U + k0 * K + r0; g.ldb1 = K; g.strideB1 = a.u_stride;
        if (asym) {
            g.K2 = depth;
            g.A2 = cae ? L.W0t + k0 : Wpk;
            g.lda2 = cae ? ldt : kSB;
            g.strideA2 = gs * (cae ? ldt : kSB);
            g.B2 = a.P1 + k0 * K + r0; g.ldb2 = K; g.strideB2 = a.u_stride;
            g.a2_scale = -1.f;
        }
        g.C = L.Wt + r0; g.ldc = ldt; g.strideC = gs * ldt;
        g.alpha = -1.f; g.beta = 1.f;
        TimerScope ts(stream, GPTQ_TIMER_TRAILING);
        return gemm_f32(g, groups, stream) == hipSuccess;
    };

    // Without the asymmetric term, and when one workgroup per CU covers every channel (the strip kernel's LDS
    // allows one per CU): each super-block of kSBS coordinates in one launch, its near rows updated inside.
    const bool strip = strip_path(N, asym);
    const int64_t sbw = strip ? kSBS : kSB;
    for (int64_t sb0 = 0; sb0 < K; sb0 += sbw) {
        const int64_t sb1 = std::min<int64_t>(K, sb0 + sbw);
        if (strip) {
            StripArgs sa;
            BlockArgs& p = sa.p;
            p.Wt = L.Wt; p.ldt = ldt; p.U = a.U; p.P1 = nullptr; p.K = K; p.N = N; p.b0 = sb0; p.bs = 0;
            p.scales = a.scales; p.rscale = L.rscale; p.bits = a.bits; p.codes_t = L.codes_t;
            p.E = L.E; p.Wpre = nullptr; p.lde = kSB;
            p.W0t = L.W0t; p.loss_acc = L.loss_acc; p.pre_round = a.pre_round; p.st = L.st;
            p.G = G; p.perm = a.perm; p.gscales = a.scales;
            p.gs = gs; p.u_stride = a.u_stride;
            p.Pnl = L.Pnl; p.Ppn = nullptr;
            sa.sb0 = sb0; sa.sb1 = sb1; sa.Usp = L.Usp;
            dim3 grid((unsigned)ceil_div(N, kChPerWG));
            {
                TimerScope ts(stream, GPTQ_TIMER_LOOP);
                {   // every group's block panels, and the split diagonal block when near updates happen
                    const int nsplit = sb0 + kB < sb1 ? kSBS / 8 * kSBS / 256 : 0;
                    const int npanel = (int)ceil_div((sb1 - sb0), kB) * kPnl / 256;
                    hipLaunchKernelGGL(strip_prep_kernel, dim3((unsigned)(nsplit + npanel), (unsigned)groups),
                                       dim3(256), 0, stream, a.U, nullptr, K, a.u_stride, sb0, sb1, nsplit, npanel,
                                       L.Usp, L.Pnl, nullptr);
                    GPTQ_LAUNCH_CHECK();
                }
#define GPTQ_STRIP(C_)                                                                                               \
    if (sm == kScaleDynamic) hipLaunchKernelGGL((quant_strip_kernel<C_, kScaleDynamic>), grid, dim3(256), 0, stream, sa); \
    else if (sm == kScaleStatic) hipLaunchKernelGGL((quant_strip_kernel<C_, kScaleStatic>), grid, dim3(256), 0, stream, sa); \
    else hipLaunchKernelGGL((quant_strip_kernel<C_, kScalePerChannel>), grid, dim3(256), 0, stream, sa);
                if (cae) { GPTQ_STRIP(true) } else { GPTQ_STRIP(false) }
#undef GPTQ_STRIP
                GPTQ_LAUNCH_CHECK();
            }
            if (sb1 < K && !trailing(sb1, K, sb0, sb1 - sb0, L.E, nullptr)) return GPTQ_ERR_HIP;
            continue;
        }
        {   // every group's block panels of U (and P1) for this super-block
            TimerScope ts(stream, GPTQ_TIMER_LOOP);
            const int npanel = (int)ceil_div((sb1 - sb0), kB) * kPnl / 256;
            hipLaunchKernelGGL(strip_prep_kernel, dim3((unsigned)(npanel * (asym ? 2 : 1)), (unsigned)groups), dim3(256),
                               0, stream, a.U, a.P1, K, a.u_stride, sb0, sb1, 0, npanel, nullptr, L.Pnl, L.Ppn);
            GPTQ_LAUNCH_CHECK();
        }
        for (int64_t b0 = sb0; b0 < sb1; b0 += kB) {
            const int bs = (int)std::min<int64_t>(kB, K - b0);
            float* Eb = L.E + (b0 - sb0);
            float* Wpb = L.Wpre ? L.Wpre + (b0 - sb0) : nullptr;
            BlockArgs p;
            p.Wt = L.Wt; p.ldt = ldt; p.U = a.U; p.P1 = a.P1; p.K = K; p.N = N; p.b0 = b0; p.bs = bs;
            p.scales = a.scales; p.rscale = L.rscale; p.bits = a.bits; p.codes_t = L.codes_t;
            p.E = Eb; p.Wpre = Wpb; p.lde = kSB;
            p.W0t = L.W0t; p.loss_acc = L.loss_acc; p.pre_round = a.pre_round; p.st = L.st;
            p.G = G; p.perm = a.perm; p.gscales = a.scales;
            p.gs = gs; p.u_stride = a.u_stride;
            p.Pnl = L.Pnl; p.Ppn = L.Ppn;
            dim3 grid((unsigned)ceil_div(N, kChPerWG));
            {
            TimerScope ts(stream, GPTQ_TIMER_LOOP);
#define GPTQ_BLOCK_W(A_, C_, W_)                                                                                  \
    if (sm == kScaleDynamic) hipLaunchKernelGGL((quant_block_kernel<A_, C_, kScaleDynamic, W_>), grid, dim3(256), 0, stream, p); \
    else if (sm == kScaleStatic) hipLaunchKernelGGL((quant_block_kernel<A_, C_, kScaleStatic, W_>), grid, dim3(256), 0, stream, p); \
    else hipLaunchKernelGGL((quant_block_kernel<A_, C_, kScalePerChannel, W_>), grid, dim3(256), 0, stream, p);
#define GPTQ_BLOCK(A_, C_)                                                                                        \
    if (bs == kB) { GPTQ_BLOCK_W(A_, C_, true) } else { GPTQ_BLOCK_W(A_, C_, false) }
            if (asym && cae) { GPTQ_BLOCK(true, true) }
            else if (asym) { GPTQ_BLOCK(true, false) }
            else if (cae) { GPTQ_BLOCK(false, true) }
            else { GPTQ_BLOCK(false, false) }
#undef GPTQ_BLOCK
#undef GPTQ_BLOCK_W
            GPTQ_LAUNCH_CHECK();
            }
            // near rows: the rest of this super-block
            const int64_t b1 = b0 + bs;
            if (b1 < sb1 && !trailing(b1, sb1, b0, bs, Eb, Wpb)) return GPTQ_ERR_HIP;
        }
        // far rows: everything after the super-block, with the errors of all its blocks
        if (sb1 < K && !trailing(sb1, K, sb0, sb1 - sb0, L.E, L.Wpre)) return GPTQ_ERR_HIP;
    }
    TimerScope ts(stream, GPTQ_TIMER_OTHER);
    {
        dim3 grid((unsigned)ceil_div(N, 64), (unsigned)ceil_div(K, 64));
        if (a.w_dtype == GPTQ_DTYPE_BF16)
            hipLaunchKernelGGL((finalize_kernel<true>), grid, dim3(256), 0, stream, L.codes_t, ldt, K, N, a.codes, a.c_rs,
                               a.c_cs, a.W_hat, a.w_rs, a.w_cs, a.scales, a.bits, a.perm, G, a.static_groups, gs);
        else
            hipLaunchKernelGGL((finalize_kernel<false>), grid, dim3(256), 0, stream, L.codes_t, ldt, K, N, a.codes, a.c_rs,
                               a.c_cs, a.W_hat, a.w_rs, a.w_cs, a.scales, a.bits, a.perm, G, a.static_groups, gs);
        GPTQ_LAUNCH_CHECK();
    }
    if (a.g_idx) {
        dim3 gi = grid1d(K, 256);
        gi.y = (unsigned)groups;
        hipLaunchKernelGGL(g_idx_kernel, gi, dim3(256), 0, stream, a.g_idx, K, a.perm, G, a.static_groups);
        GPTQ_LAUNCH_CHECK();
    }
    if (a.losses) {
        hipLaunchKernelGGL(copy_losses_kernel, grid1d(N, 256), dim3(256), 0, stream, L.loss_acc, a.losses, N);
        GPTQ_LAUNCH_CHECK();
    }
    return GPTQ_OK;
}

}  // namespace gptq
