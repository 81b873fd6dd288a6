// Shared-order column loop with lazy block updates on gfx950.
//
// [T] section 3: fixing coordinate q to its grid value moves the still-free weights along the OBS direction.
// [T] section 4: with U the upper factor of H_d^{-1}, that move is w_k -= U_qk E_q with E_q = (w_q - Q(w_q)) / U_qq.
// [T] section 5: every output channel uses the same coordinate order, so all channels share U; inside a
// block of 128 coordinates the updates are applied at once, the rest of the matrix is updated once per
// block by one matrix product (W[b1:] -= U[B, b1:]^T E_B), here an fp32 MFMA GEMM.
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
constexpr int kChPerWG = 16;     // channels per workgroup of the block kernel

__global__ void quant_init_kernel(DevStatus* st, uint32_t* amax_bits, float* loss_acc, int64_t N) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i == 0) { st->flags = 0; st->n_dead = 0; st->damp = 0.f; }
    if (i < N) { amax_bits[i] = 0u; loss_acc[i] = 0.f; }
}

// W (K x N view with strides) -> Wt (N x ldt fp32, dead rows zeroed, padding zero) and per-channel max |w|
// taken before dead rows are zeroed.  64 x 64 tiles transposed through LDS.
template <bool BF16>
__global__ __launch_bounds__(256) void convert_kernel(const void* Wv, int64_t K, int64_t N, int64_t w_rs,
                                                     int64_t w_cs, const uint8_t* dead, float* Wt, int64_t ldt,
                                                     uint32_t* amax_bits, DevStatus* st) {
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
            const int64_t off = k * w_rs + n * w_cs;
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
            if (k < K && dead && dead[k]) v = 0.f;
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
    float* E;                       // N x 128
    float* Wpre;                    // N x 128 (asymmetric without CAE)
    const float* W0t;               // N x ldt original weights (CAE only)
    float* loss_acc;                // N
    float* pre_round;               // optional, K x N
    const DevStatus* st;
};

// Per-lane state of the block kernel: 8 strided coordinates of one channel.
struct LaneState {
    float w[8], e[8], pre[8], w0[8];
    uint32_t code[8];
    float loss;
};

struct StepConst {
    const float* Up; const float* Pp; const float* rdiag;
    float s, rs, z, qmax;
    int l;
    float* pre_round; int64_t prow_off; int64_t N; bool live;
};

// Per-step operands read from LDS: this lane's 8 entries of U row J (and of P1 row J), 1 / U_JJ.  Step J
// reads the operands of step J + 1 while it runs, so no LDS latency sits on the chain of dependent steps.
struct StepOps {
    f32x4 u0, u1, p0, p1;
    float rd;
};

template <int J, bool ASYM>
__device__ __forceinline__ void load_ops(StepOps& o, const StepConst& k) {
    if constexpr (J < kB) {
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
template <int J, bool ASYM, bool CAE, bool PRE>
__device__ __forceinline__ void loop_step(LaneState& st, const StepConst& k, StepOps (&ops)[2]) {
    constexpr int m = J >> 4, lj = J & 15;
    const StepOps& o = ops[J & 1];
    load_ops<J + 1, ASYM>(ops[(J + 1) & 1], k);
    const float wj = row_bcast(st.w[m], lj);
    const float v = wj * k.rs;
    const float c = fminf(fmaxf(rintf(v) + k.z, 0.f), k.qmax);
    const float q = (c - k.z) * k.s;
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

template <bool ASYM, bool CAE, bool PRE, int... Js>
__device__ __forceinline__ void run_steps(LaneState& st, const StepConst& k, int bs,
                                          std::integer_sequence<int, Js...>) {
    StepOps ops[2];
    load_ops<0, ASYM>(ops[0], k);
    ((Js < bs ? loop_step<Js, ASYM, CAE, PRE>(st, k, ops) : (void)0), ...);
}

template <bool ASYM, bool CAE>
__global__ __launch_bounds__(256) void quant_block_kernel(BlockArgs p) {
    __shared__ __attribute__((aligned(16))) float Up[kB * kB];               // [row j][16 lanes][8 slots]
    __shared__ __attribute__((aligned(16))) float Pp[ASYM ? kB * kB : 4];    // same layout (asymmetric)
    __shared__ float rdiag[kB];

    if (p.st->flags) return;   // an input was rejected earlier in this call
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
    k.Up = Up; k.Pp = Pp; k.rdiag = rdiag;
    k.s = p.scales[nn]; k.rs = p.rscale[nn];
    k.z = (float)(1 << (p.bits - 1));
    k.qmax = (float)((1 << p.bits) - 1);
    k.l = l;
    k.pre_round = p.pre_round ? p.pre_round + b0 * p.N : nullptr;
    k.prow_off = n; k.N = p.N; k.live = live;
    if (k.pre_round) run_steps<ASYM, CAE, true>(st, k, bs, std::make_integer_sequence<int, kB>{});
    else run_steps<ASYM, CAE, false>(st, k, bs, std::make_integer_sequence<int, kB>{});

    if (!live) return;
    uint8_t* crow = p.codes_t + n * p.ldt + b0;
    float* erow = p.E + n * kB;
    for (int m = 0; m < 8; ++m) {
        const int c = 16 * m + l;
        if (c < bs) crow[c] = (uint8_t)st.code[m];
        erow[c] = st.e[m];
        if (ASYM && !CAE) p.Wpre[n * kB + c] = st.pre[m];
    }
    if (l == 0) p.loss_acc[n] += 0.5f * st.loss;
}

// codes_t (N x ldt) -> codes (K x N view with strides); W_hat = s (c - z) in the weight dtype; losses copy.
template <bool BF16>
__global__ __launch_bounds__(256) void finalize_kernel(const uint8_t* codes_t, int64_t ldt, int64_t K, int64_t N,
                                                      uint8_t* codes, int64_t c_rs, int64_t c_cs, void* W_hat,
                                                      int64_t w_rs, int64_t w_cs, const float* scales, int bits) {
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
            if (k < K && n < N) codes[k * c_rs + n * c_cs] = tile[kk][nn];
        }
        if (W_hat) {
            const int kk = n_fast_w ? a : b, nn = n_fast_w ? b : a;
            const int64_t k = k0 + kk, n = n0 + nn;
            if (k < K && n < N) {
                const float v = ((float)tile[kk][nn] - z) * scales[n];
                if (BF16) static_cast<__bf16*>(W_hat)[k * w_rs + n * w_cs] = (__bf16)v;
                else static_cast<float*>(W_hat)[k * w_rs + n * w_cs] = v;
            }
        }
    }
}

__global__ void copy_losses_kernel(const float* src, float* dst, int64_t N) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < N) dst[i] = src[i];
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
    L.E = c.take<float>((size_t)N * kB);
    L.Wpre = asym && !cae ? c.take<float>((size_t)N * kB) : nullptr;
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

    hipLaunchKernelGGL(quant_init_kernel, grid1d(std::max<int64_t>(N, 1), 256), dim3(256), 0, stream, L.st, L.amax,
                       L.loss_acc, N);
    GPTQ_LAUNCH_CHECK();
    {
        dim3 grid((unsigned)ceil_div(N, 64), (unsigned)ceil_div(ldt, 64));
        if (a.w_dtype == GPTQ_DTYPE_BF16)
            hipLaunchKernelGGL((convert_kernel<true>), grid, dim3(256), 0, stream, a.W, K, N, a.w_rs, a.w_cs, a.dead,
                               L.Wt, ldt, L.amax, L.st);
        else
            hipLaunchKernelGGL((convert_kernel<false>), grid, dim3(256), 0, stream, a.W, K, N, a.w_rs, a.w_cs, a.dead,
                               L.Wt, ldt, L.amax, L.st);
        GPTQ_LAUNCH_CHECK();
    }
    hipLaunchKernelGGL(scales_kernel, grid1d(N, 256), dim3(256), 0, stream, L.amax, a.scales, L.rscale, N, a.bits,
                       a.scales_given, L.st);
    GPTQ_LAUNCH_CHECK();
    if (cae)   // the original weights (dead rows zeroed), read by every step and by the trailing updates
        GPTQ_HIP_CHECK(hipMemcpyAsync(L.W0t, L.Wt, sizeof(float) * (size_t)N * (size_t)ldt, hipMemcpyDeviceToDevice,
                                      stream));

    for (int64_t b0 = 0; b0 < K; b0 += kB) {
        const int bs = (int)std::min<int64_t>(kB, K - b0);
        BlockArgs p;
        p.Wt = L.Wt; p.ldt = ldt; p.U = a.U; p.P1 = a.P1; p.K = K; p.N = N; p.b0 = b0; p.bs = bs;
        p.scales = a.scales; p.rscale = L.rscale; p.bits = a.bits; p.codes_t = L.codes_t; p.E = L.E;
        p.Wpre = L.Wpre; p.W0t = L.W0t; p.loss_acc = L.loss_acc; p.pre_round = a.pre_round; p.st = L.st;
        dim3 grid((unsigned)ceil_div(N, kChPerWG));
        if (asym && cae) hipLaunchKernelGGL((quant_block_kernel<true, true>), grid, dim3(256), 0, stream, p);
        else if (asym) hipLaunchKernelGGL((quant_block_kernel<true, false>), grid, dim3(256), 0, stream, p);
        else if (cae) hipLaunchKernelGGL((quant_block_kernel<false, true>), grid, dim3(256), 0, stream, p);
        else hipLaunchKernelGGL((quant_block_kernel<false, false>), grid, dim3(256), 0, stream, p);
        GPTQ_LAUNCH_CHECK();
        const int64_t b1 = b0 + bs;
        if (b1 < K) {
            // Lazy batch: Wt[:, b1:] -= E_B U[B, b1:]  (+ Wpre_B P1[B, b1:] for the asymmetric term; with CAE,
            // E holds (w0 - q) / U_jj and the P1 term takes the original weights W0_B)
            GemmArgs g;
            g.M = N; g.N = K - b1; g.K1 = bs;
            g.A1 = L.E; g.lda1 = kB;
            g.B1 = a.U + b0 * K + b1; g.ldb1 = K;
            if (asym) {
                g.K2 = bs;
                g.A2 = cae ? L.W0t + b0 : L.Wpre;
                g.lda2 = cae ? ldt : kB;
                g.B2 = a.P1 + b0 * K + b1; g.ldb2 = K;
                g.a2_scale = -1.f;
            }
            g.C = L.Wt + b1; g.ldc = ldt;
            g.alpha = -1.f; g.beta = 1.f;
            if (gemm_f32(g, 1, stream) != hipSuccess) return GPTQ_ERR_HIP;
        }
    }
    {
        dim3 grid((unsigned)ceil_div(N, 64), (unsigned)ceil_div(K, 64));
        if (a.w_dtype == GPTQ_DTYPE_BF16)
            hipLaunchKernelGGL((finalize_kernel<true>), grid, dim3(256), 0, stream, L.codes_t, ldt, K, N, a.codes, a.c_rs,
                               a.c_cs, a.W_hat, a.w_rs, a.w_cs, a.scales, a.bits);
        else
            hipLaunchKernelGGL((finalize_kernel<false>), grid, dim3(256), 0, stream, L.codes_t, ldt, K, N, a.codes, a.c_rs,
                               a.c_cs, a.W_hat, a.w_rs, a.w_cs, a.scales, a.bits);
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
