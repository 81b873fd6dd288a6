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
// 128), so that one channel's block of 128 coordinates is contiguous.  The block kernel gives each
// channel 16 lanes (one DPP row); lane l holds coordinates 16 m + l, m = 0..7, of the current block in
// registers, so that the coordinates still free after step j = 16 m + l0 are exactly the slots >= m and
// the triangular work shrinks with m.  The U panel (and P1 panel) of the block sits in LDS, permuted so
// that a lane's eight coefficients of row j are two 16-byte reads.  At step j the value w_j is broadcast
// from its owner lane to the row with DPP row_newbcast; every lane of the row then evaluates the same
// rounding and error (no further communication), updates its own slots, and the owner keeps the code.
#include <algorithm>
#include <utility>

#include "gemm_f32.hpp"
#include "quantize.hpp"

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
    unsigned bad = 0;
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

// Broadcast lane `src` of each 16-lane row to the whole row (DPP row_newbcast, gfx90a+).
__device__ inline float row_bcast(float x, int src) {
    const int xi = __float_as_int(x);
    int r;
    switch (src) {
#define GPTQ_BC(i) case i: r = __builtin_amdgcn_update_dpp(0, xi, 0x150 + i, 0xF, 0xF, false); break;
        GPTQ_BC(0) GPTQ_BC(1) GPTQ_BC(2) GPTQ_BC(3) GPTQ_BC(4) GPTQ_BC(5) GPTQ_BC(6) GPTQ_BC(7)
        GPTQ_BC(8) GPTQ_BC(9) GPTQ_BC(10) GPTQ_BC(11) GPTQ_BC(12) GPTQ_BC(13) GPTQ_BC(14) GPTQ_BC(15)
#undef GPTQ_BC
        default: r = xi;
    }
    return __int_as_float(r);
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
};

// Scale modes of the block kernel: one scale per channel; groups re-estimated from the current weights at each
// group start (processing order); static groups whose scales were computed from W before the loop.
enum : int { kScalePerChannel = 0, kScaleDynamic = 1, kScaleStatic = 2 };

// Per-lane state of the block kernel: 8 strided coordinates of one channel.
struct LaneState {
    float w[8], e[8], pre[8], w0[8];
    uint32_t code[8];
    float loss;
    float s, rs;                    // scale in force (and its reciprocal)
};

struct StepConst {
    const float* Up; const float* Pp; const float* rdiag;
    const float* Ts; const float* Trs;   // static groups: per-step scales of this workgroup's 16 channels
    float z, qmax;
    int l, ch;
    int64_t G, b0;
    float* gscales;
    float* pre_round; int64_t prow_off; int64_t N; bool live;
};

// Per-step operands read from LDS: this lane's 8 entries of U row J (and of P1 row J), 1 / U_JJ.  Step J
// reads the operands of step J + 1 while it runs, so no LDS latency sits on the chain of dependent steps.
struct StepOps {
    f32x4 u0, u1, p0, p1;
    float rd, s, rs;
};

template <int J, bool ASYM, int SM>
__device__ __forceinline__ void load_ops(StepOps& o, const StepConst& k) {
    if constexpr (J < kB) {
        if constexpr (SM == kScaleStatic) {
            o.s = k.Ts[J * 16 + k.ch];
            o.rs = k.Trs[J * 16 + k.ch];
        }
        const f32x4* urow = reinterpret_cast<const f32x4*>(k.Up + (J * 16 + k.l) * 8);
        o.u0 = urow[0];
        o.u1 = urow[1];
        if constexpr (ASYM) {
            const f32x4* prow = reinterpret_cast<const f32x4*>(k.Pp + (J * 16 + k.l) * 8);
            o.p0 = prow[0];
            o.p1 = prow[1];
        }
        o.rd = k.rdiag[J];
    }
}

// One step j of the loop (j compile-time so that slots, DPP lane and LDS offsets are immediates).
// CAE: the step's update uses the original weight w0_j in place of the pre-rounding value, both in the
// error that multiplies U (w0_j - q) / U_jj and in the P1 coefficient; the step error E_j itself still feeds
// the loss.  This is the P2 = P1 + I - diag(U)^-1 U form of the CAE term.
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
    if (k.l == 0 && k.live) k.gscales[((k.b0 + J) / k.G) * k.N + k.prow_off] = st.s;
}

template <int J, bool ASYM, bool CAE, bool PRE, int SM>
__device__ __forceinline__ void loop_step(LaneState& st, const StepConst& k, StepOps (&ops)[2]) {
    constexpr int m = J >> 4, lj = J & 15;
    const StepOps& o = ops[J & 1];
    if constexpr (SM == kScaleDynamic) regroup<J>(st, k);
    if constexpr (SM == kScaleStatic) {
        st.s = o.s;
        st.rs = o.rs;
    }
    load_ops<J + 1, ASYM, SM>(ops[(J + 1) & 1], k);
    const float wj = row_bcast(st.w[m], lj);
    const float v = wj * st.rs;
    const float c = fminf(fmaxf(rintf(v) + k.z, 0.f), k.qmax);
    const float q = (c - k.z) * st.s;
    const float e = (wj - q) * o.rd;
    const float wu = CAE ? row_bcast(st.w0[m], lj) : wj;      // value the update is taken from
    const float eu = CAE ? (wu - q) * o.rd : e;
    const float uu[8] = {o.u0.x, o.u0.y, o.u0.z, o.u0.w, o.u1.x, o.u1.y, o.u1.z, o.u1.w};
    const bool owner = (k.l == lj);
    if constexpr (ASYM) {
        const float pp[8] = {o.p0.x, o.p0.y, o.p0.z, o.p0.w, o.p1.x, o.p1.y, o.p1.z, o.p1.w};
        st.w[m] = owner ? q : fmaf(pp[m], wu, fmaf(-uu[m], eu, st.w[m]));
#pragma unroll
        for (int mm = m + 1; mm < 8; ++mm) st.w[mm] = fmaf(pp[mm], wu, fmaf(-uu[mm], eu, st.w[mm]));
    } else {
        st.w[m] = owner ? q : fmaf(-uu[m], eu, st.w[m]);
#pragma unroll
        for (int mm = m + 1; mm < 8; ++mm) st.w[mm] = fmaf(-uu[mm], eu, st.w[mm]);
    }
    st.loss = fmaf(e, e, st.loss);
    st.code[m] = owner ? (uint32_t)c : st.code[m];
    st.e[m] = owner ? eu : st.e[m];
    if constexpr (ASYM) st.pre[m] = owner ? wj : st.pre[m];
    if constexpr (PRE) {
        if (owner && k.live) k.pre_round[(int64_t)J * k.N + k.prow_off] = v;
    }
}

template <bool ASYM, bool CAE, bool PRE, int SM, int... Js>
__device__ __forceinline__ void run_steps(LaneState& st, const StepConst& k, int bs,
                                          std::integer_sequence<int, Js...>) {
    StepOps ops[2];
    load_ops<0, ASYM, SM>(ops[0], k);
    ((Js < bs ? loop_step<Js, ASYM, CAE, PRE, SM>(st, k, ops) : (void)0), ...);
}

template <bool ASYM, bool CAE, int SM>
__global__ __launch_bounds__(256) void quant_block_kernel(BlockArgs p) {
    __shared__ __attribute__((aligned(16))) float Up[kB * kB];               // [row j][16 lanes][8 slots]
    __shared__ __attribute__((aligned(16))) float Pp[ASYM ? kB * kB : 4];    // same layout (asymmetric)
    __shared__ float rdiag[kB];
    __shared__ float Ts[SM == kScaleStatic ? kB * kChPerWG : 1];           // [step][channel] static scales
    __shared__ float Trs[SM == kScaleStatic ? kB * kChPerWG : 1];

    if (p.st->flags) return;   // an input was rejected earlier in this call
    {   // output-channel groups: the workgroup's channels all belong to one group (gs is a multiple of 16)
        const int64_t g = (int64_t)blockIdx.x * kChPerWG / p.gs;
        p.U += g * p.u_stride;
        if (p.P1) p.P1 += g * p.u_stride;
        if (p.perm) p.perm += g * p.K;
    }
    const int tid = threadIdx.x;
    const int64_t b0 = p.b0;
    const int bs = p.bs;
    // Stage the U (and P1) panel rows b0..b0+bs-1, columns b0..b0+127 (zero beyond the block) as
    // [row j][lane l][slot m] for column 16 m + l.  All global loads are issued before the LDS stores.
    {
        constexpr int kV = kB * kB / 4 / 256;     // 16-byte vectors per thread
        const bool vec = p.bs == kB && (p.K % 4) == 0 && (b0 % 4) == 0;
        f32x4 uv[kV], pv[ASYM ? kV : 1];
#pragma unroll
        for (int i = 0; i < kV; ++i) {
            const int idx = tid + 256 * i, j = idx >> 5, c = (idx & 31) * 4;
            const int64_t off = (b0 + j) * p.K + b0 + c;
            f32x4 u = {0.f, 0.f, 0.f, 0.f}, q = {0.f, 0.f, 0.f, 0.f};
            if (vec) {
                u = *reinterpret_cast<const f32x4*>(p.U + off);
                if constexpr (ASYM) q = *reinterpret_cast<const f32x4*>(p.P1 + off);
            } else if (j < bs) {
                for (int e = 0; e < 4; ++e)
                    if (c + e < bs) {
                        u[e] = p.U[off + e];
                        if constexpr (ASYM) q[e] = p.P1[off + e];
                    }
            }
            uv[i] = u;
            if constexpr (ASYM) pv[i] = q;
        }
#pragma unroll
        for (int i = 0; i < kV; ++i) {
            const int idx = tid + 256 * i, j = idx >> 5, c = (idx & 31) * 4;
            for (int e = 0; e < 4; ++e) {
                const int l = (c + e) & 15, m = (c + e) >> 4;
                Up[(j * 16 + l) * 8 + m] = uv[i][e];
                if constexpr (ASYM) Pp[(j * 16 + l) * 8 + m] = pv[i][e];
            }
        }
    }
    for (int j = tid; j < kB; j += 256) rdiag[j] = (j < bs) ? 1.0f / p.U[(b0 + j) * p.K + b0 + j] : 0.f;
    if constexpr (SM == kScaleStatic) {
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
    __syncthreads();

    const int lane = tid & 63, l = lane & 15;
    const int64_t n = (int64_t)blockIdx.x * kChPerWG + (tid >> 4);
    const bool live = n < p.N;
    const int64_t nn = live ? n : 0;

    LaneState st;
    const float* wrow = p.Wt + nn * p.ldt + b0;
    const float* w0row = CAE ? p.W0t + nn * p.ldt + b0 : nullptr;
    for (int m = 0; m < 8; ++m) {
        st.w[m] = wrow[16 * m + l];
        if constexpr (CAE) st.w0[m] = w0row[16 * m + l];
        st.e[m] = 0.f;
        st.pre[m] = 0.f;
        st.code[m] = 0;
    }
    st.loss = 0.f;
    StepConst k;
    k.Up = Up; k.Pp = Pp; k.rdiag = rdiag; k.Ts = Ts; k.Trs = Trs;
    if constexpr (SM == kScalePerChannel) {
        st.s = p.scales[nn];
        st.rs = p.rscale[nn];
    } else {
        st.s = 1.0f;
        st.rs = 1.0f;
    }
    k.z = (float)(1 << (p.bits - 1));
    k.qmax = (float)((1 << p.bits) - 1);
    k.l = l;
    k.ch = tid >> 4;
    k.G = p.G; k.b0 = b0; k.gscales = p.gscales;
    k.pre_round = p.pre_round ? p.pre_round + b0 * p.N : nullptr;
    k.prow_off = n; k.N = p.N; k.live = live;
    if (k.pre_round) run_steps<ASYM, CAE, true, SM>(st, k, bs, std::make_integer_sequence<int, kB>{});
    else run_steps<ASYM, CAE, false, SM>(st, k, bs, std::make_integer_sequence<int, kB>{});

    if (!live) return;
    uint8_t* crow = p.codes_t + n * p.ldt + b0;
    float* erow = p.E + n * p.lde;
    for (int m = 0; m < 8; ++m) {
        const int c = 16 * m + l;
        if (c < bs) crow[c] = (uint8_t)st.code[m];
        erow[c] = st.e[m];
        if (ASYM && !CAE) p.Wpre[n * p.lde + c] = st.pre[m];
    }
    if (l == 0) p.loss_acc[n] += 0.5f * st.loss;
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
    size_t bytes;
};

QuantLayout carve(void* ws, int64_t K, int64_t N, bool asym, bool cae) {
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
    L.bytes = c.bytes();
    return L;
}

}  // namespace

size_t quantize_workspace_bytes(int64_t K, int64_t N, bool asym, bool cae) {
    return carve(nullptr, K, N, asym, cae).bytes;
}

gptq_status_t quantize_layer(const QuantizeArgs& a, void* workspace, hipStream_t stream) {
    const bool asym = a.P1 != nullptr;
    const int64_t K = a.K, N = a.N;
    const int64_t ldt = ceil_div(std::max<int64_t>(K, 1), kB) * kB;
    const bool cae = a.cae;
    QuantLayout L = carve(workspace, K, N, asym, cae);
    const int64_t groups = std::max<int64_t>(a.groups, 1), gs = N / groups;   // output-channel groups

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
    const int64_t G = a.groupsize;
    const int sm = G == 0 ? kScalePerChannel : (a.static_groups ? kScaleStatic : kScaleDynamic);
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
        return gemm_f32(g, groups, stream) == hipSuccess;
    };

    for (int64_t sb0 = 0; sb0 < K; sb0 += kSB) {
        const int64_t sb1 = std::min<int64_t>(K, sb0 + kSB);
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
            dim3 grid((unsigned)ceil_div(N, kChPerWG));
#define GPTQ_BLOCK(A_, C_)                                                                                        \
    if (sm == kScaleDynamic) hipLaunchKernelGGL((quant_block_kernel<A_, C_, kScaleDynamic>), grid, dim3(256), 0, stream, p); \
    else if (sm == kScaleStatic) hipLaunchKernelGGL((quant_block_kernel<A_, C_, kScaleStatic>), grid, dim3(256), 0, stream, p); \
    else hipLaunchKernelGGL((quant_block_kernel<A_, C_, kScalePerChannel>), grid, dim3(256), 0, stream, p);
            if (asym && cae) { GPTQ_BLOCK(true, true) }
            else if (asym) { GPTQ_BLOCK(true, false) }
            else if (cae) { GPTQ_BLOCK(false, true) }
            else { GPTQ_BLOCK(false, false) }
#undef GPTQ_BLOCK
            GPTQ_LAUNCH_CHECK();
            // near rows: the rest of this super-block
            const int64_t b1 = b0 + bs;
            if (b1 < sb1 && !trailing(b1, sb1, b0, bs, Eb, Wpb)) return GPTQ_ERR_HIP;
        }
        // far rows: everything after the super-block, with the errors of all its blocks
        if (sb1 < K && !trailing(sb1, K, sb0, sb1 - sb0, L.E, L.Wpre)) return GPTQ_ERR_HIP;
    }
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
    DevStatus hst;
    GPTQ_HIP_CHECK(hipMemcpyAsync(&hst, L.st, sizeof(DevStatus), hipMemcpyDeviceToHost, stream));
    GPTQ_HIP_CHECK(hipStreamSynchronize(stream));
    if (hst.flags & kDevNonFinite) return GPTQ_ERR_NONFINITE;
    return GPTQ_OK;
}

}  // namespace gptq
