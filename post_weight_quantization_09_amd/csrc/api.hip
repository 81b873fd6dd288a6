// C ABI of libgptq_hip.so: argument validation, workspace sizing and launch order (see include/gptq.h).
#include <algorithm>
#include <cmath>
#include <mutex>

#include "factor.hpp"
#include "gemm_f32.hpp"
#include "gram.hpp"
#include "quantize.hpp"
#include "pack.hpp"
#include "hadamard.hpp"
#include "act_order.hpp"
#include "timer.hpp"

using namespace gptq;

namespace {

bool ws_ok(const void* ws, size_t have, size_t need) {
    if (need == 0) return true;
    return ws != nullptr && (reinterpret_cast<uintptr_t>(ws) % kAlign) == 0 && have >= need;
}

// Split partials are reused by the symmetric Gram and then the cross term: size for the larger plan.
size_t accumulate_partial_floats(int64_t K, int64_t M, bool cross) {
    size_t f = gram_plan(K, M, false).partial_floats;
    if (cross) f = std::max(f, gram_plan(K, M, true).partial_floats);
    return f;
}

size_t accumulate_ws(int64_t K, int64_t M, bool cross, bool scaled) {
    Carver c(nullptr);
    c.take<DevStatus>(1);
    c.take<float>(accumulate_partial_floats(K, M, cross));
    c.take<uint16_t>(gram_staging_elems(K, M, cross || scaled));
    return c.bytes();
}

size_t asym_ws(int64_t K) {
    Carver c(nullptr);
    c.take<DevStatus>(1);
    c.take<float>((size_t)K * (size_t)K);
    return c.bytes();
}

gptq_status_t quantize_common(const void* W, gptq_dtype_t w_dtype, int64_t K, int64_t N, int64_t w_rs, int64_t w_cs,
                              int64_t groups, const float* U, int64_t u_stride, const uint8_t* dead, const float* P1,
                              int bits, int blocksize, unsigned flags, uint8_t* codes, int64_t c_rs, int64_t c_cs,
                              float* scales, void* W_hat, float* losses, float* pre_round, const int32_t* perm,
                              int64_t groupsize, int32_t* g_idx, void* workspace, size_t workspace_bytes,
                              void* stream) {
    if (!W || !U || !codes || !scales || K < 1 || N < 1) return GPTQ_ERR_ARG;
    if (w_dtype != GPTQ_DTYPE_F32 && w_dtype != GPTQ_DTYPE_BF16) return GPTQ_ERR_ARG;
    // bits 2..6: wider grids put |w / s| up to 2^(bits-1), and at 7-8 bits the fp32 working weights drift past the
    // 1e-4 s tie band of the codes over a few thousand coordinates (measured 2.6e-4 at 8 bits, K = 4096)
    if (bits < 2 || bits > 6 || blocksize != 128) return GPTQ_ERR_ARG;
    const unsigned known = GPTQ_FLAG_SCALES_GIVEN | GPTQ_FLAG_CAE | GPTQ_FLAG_STATIC_GROUPS | GPTQ_FLAG_MSE;
    if ((flags & ~known) != 0) return GPTQ_ERR_ARG;
    if (groupsize != 0 && groupsize != 32 && groupsize != 64 && groupsize != 128) return GPTQ_ERR_ARG;
    const bool stat = (flags & GPTQ_FLAG_STATIC_GROUPS) != 0, mse = (flags & GPTQ_FLAG_MSE) != 0;
    if (stat && groupsize == 0) return GPTQ_ERR_ARG;
    if (mse && groupsize != 0 && !stat) return GPTQ_ERR_ARG;
    if ((flags & GPTQ_FLAG_SCALES_GIVEN) && (groupsize != 0 || mse)) return GPTQ_ERR_ARG;
    if (w_rs < 1 || w_cs < 1 || c_rs < 1 || c_cs < 1) return GPTQ_ERR_ARG;
    if (K > (int64_t)1 << 24 || N > (int64_t)1 << 28) return GPTQ_ERR_ARG;
    if (groups < 1 || groups > 65535 || N % groups != 0) return GPTQ_ERR_ARG;
    if (groups > 1 && ((N / groups) % 16 != 0 || u_stride < K * K)) return GPTQ_ERR_ARG;
    if (!ws_ok(workspace, workspace_bytes,
               quantize_workspace_bytes(K, N, P1 != nullptr, (flags & GPTQ_FLAG_CAE) != 0, groups)))
        return GPTQ_ERR_WORKSPACE;
    QuantizeArgs a;
    a.W = W; a.w_dtype = w_dtype; a.K = K; a.N = N; a.w_rs = w_rs; a.w_cs = w_cs;
    a.U = U; a.dead = dead; a.P1 = P1; a.bits = bits; a.scales_given = (flags & GPTQ_FLAG_SCALES_GIVEN) != 0;
    a.cae = (flags & GPTQ_FLAG_CAE) != 0;
    a.perm = perm; a.groupsize = groupsize; a.static_groups = stat; a.mse = mse; a.g_idx = g_idx;
    a.groups = groups; a.u_stride = groups > 1 ? u_stride : 0;
    a.codes = codes; a.c_rs = c_rs; a.c_cs = c_cs; a.scales = scales; a.W_hat = W_hat; a.losses = losses;
    a.pre_round = pre_round;
    return quantize_layer(a, workspace, static_cast<hipStream_t>(stream));
}

// Scratch of gptq_quantize_layer_noalloc: a static device array, one copy per device, kept until the process ends.
// Host code uses it only through the device address hipGetSymbolAddress returns for the current device (the array's
// name is a host-side stand-in, not a device address).
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's scratch address, looked up on the first call on the device (with it current) and cached.
// lookup = false only reads the cache (null if no call has run on the current device).
gptq_status_t static_scratch(void** out, bool lookup) {
    *out = nullptr;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return lookup ? GPTQ_ERR_HIP : GPTQ_ERR_ARG;
    std::lock_guard<std::mutex> g(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        if (!lookup) return GPTQ_ERR_ARG;
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GPTQ_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return GPTQ_OK;
}

}  // namespace

extern "C" {

const char* gptq_version(void) { return "0.1.0"; }

const char* gptq_status_string(gptq_status_t s) {
    switch (s) {
        case GPTQ_OK: return "ok";
        case GPTQ_ERR_ARG: return "invalid argument";
        case GPTQ_ERR_NONFINITE: return "non-finite input";
        case GPTQ_ERR_NOT_PD: return "damped Hessian not positive definite";
        case GPTQ_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case GPTQ_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

gptq_status_t gptq_device_status(const void* workspace, void* stream) {
    if (!workspace) {   // the static scratch of gptq_quantize_layer_noalloc on the current device
        void* p = nullptr;
        const gptq_status_t r = static_scratch(&p, false);
        if (r != GPTQ_OK) return r;
        workspace = p;
    }
    if ((reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0) return GPTQ_ERR_ARG;
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint32_t flags = 0;
    // the read is ordered after the stream's work; the copy into pageable memory returns once it is done
    if (hipMemcpyAsync(&flags, workspace, sizeof(flags), hipMemcpyDeviceToHost, st) != hipSuccess) return GPTQ_ERR_HIP;
    if (hipStreamSynchronize(st) != hipSuccess) return GPTQ_ERR_HIP;
    if (flags & kDevNonFinite) return GPTQ_ERR_NONFINITE;
    if (flags & kDevNotPD) return GPTQ_ERR_NOT_PD;
    return GPTQ_OK;
}

size_t gptq_workspace_bytes(gptq_call_t call, int64_t K, int64_t N, int64_t M, unsigned flags) {
    if (K < 1) K = 1;
    if (N < 1) N = 1;
    if (M < 0) M = 0;
    switch (call) {
        case GPTQ_CALL_ACCUMULATE_HESSIAN: return accumulate_ws(K, M, (flags & 1u) != 0, (flags & 2u) != 0);
        case GPTQ_CALL_PREPARE: return prepare_workspace_bytes(K, N);   // N: Hessians of gptq_prepare_groups
        case GPTQ_CALL_ASYM_CORRECTION: return asym_ws(K);
        case GPTQ_CALL_ACT_ORDER: return K > 0 ? act_order_workspace_bytes(K) : 0;
        case GPTQ_CALL_QUANTIZE_LAYER:
            // M: the output-channel groups of gptq_quantize_layer_groups (0 or 1: one)
            return quantize_workspace_bytes(K, N, (flags & 2u) != 0, (flags & GPTQ_FLAG_CAE) != 0, std::max<int64_t>(M, 1));
    }
    return 0;
}

gptq_status_t gptq_gram_plan(int64_t K, int64_t M, int cross, int transformed, int64_t* out) {
    if (K < 1 || M < 0 || !out) return GPTQ_ERR_ARG;
    const GramPlan pl = gram_plan(K, M, cross != 0);
    out[0] = pl.nb;
    out[1] = pl.ntiles;
    out[2] = pl.splits;
    out[3] = pl.tokens_per_split;
    out[4] = (int64_t)pl.partial_floats;
    out[5] = (int64_t)gram_staging_elems(K, M, transformed != 0);
    return GPTQ_OK;
}

gptq_status_t gptq_accumulate_hessian(float* H, int64_t K, const void* X, gptq_dtype_t x_dtype, int64_t M,
                                      int64_t ldx, const float* row_scale, const void* X_float, int64_t ldxf,
                                      float* A, void* workspace, size_t workspace_bytes, void* stream) {
    if (!H || K < 1 || M < 0 || (M > 0 && !X) || ldx < K) return GPTQ_ERR_ARG;
    if (x_dtype != GPTQ_DTYPE_F32 && x_dtype != GPTQ_DTYPE_BF16) return GPTQ_ERR_ARG;
    if (row_scale && x_dtype != GPTQ_DTYPE_BF16) return GPTQ_ERR_ARG;
    const bool cross = X_float != nullptr;
    if (cross && (x_dtype != GPTQ_DTYPE_BF16 || !A || ldxf < K || row_scale)) return GPTQ_ERR_ARG;
    if (!cross && A) return GPTQ_ERR_ARG;
    const size_t need = x_dtype == GPTQ_DTYPE_BF16 ? accumulate_ws(K, M, cross, row_scale != nullptr) : 0;
    if (!ws_ok(workspace, workspace_bytes, need)) return GPTQ_ERR_WORKSPACE;
    if (M == 0) return GPTQ_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (x_dtype == GPTQ_DTYPE_F32) {
        // fp32 activations: H += 2 X^T X on fp32 MFMA (A(m,k) = X[k][m], B(k,n) = X[k][n]).
        GemmArgs g;
        g.M = K; g.N = K; g.K1 = M;
        g.A1 = static_cast<const float*>(X); g.lda1 = ldx; g.transA = true;
        g.B1 = static_cast<const float*>(X); g.ldb1 = ldx;
        g.C = H; g.ldc = K;
        g.alpha = 2.f; g.beta = 1.f;
        TimerScope ts(st, GPTQ_TIMER_GRAM);
        return gemm_f32(g, 1, st) == hipSuccess ? GPTQ_OK : GPTQ_ERR_HIP;
    }
    Carver c(workspace);
    c.take<DevStatus>(1);
    const GramPlan pl = gram_plan(K, M, false);
    float* partial = c.take<float>(accumulate_partial_floats(K, M, cross));
    const size_t nstage = gram_staging_elems(K, M, cross || row_scale != nullptr);
    uint16_t* staging = nstage ? c.take<uint16_t>(nstage) : nullptr;
    hipError_t e = gram_bf16(pl, static_cast<const uint16_t*>(X), ldx, nullptr, 0, row_scale, M, K, partial, staging,
                             H, st);
    if (e != hipSuccess) return GPTQ_ERR_HIP;
    if (cross) {
        const GramPlan px = gram_plan(K, M, true);
        e = gram_bf16(px, static_cast<const uint16_t*>(X), ldx, static_cast<const uint16_t*>(X_float), ldxf, nullptr,
                      M, K, partial, staging, A, st);
        if (e != hipSuccess) return GPTQ_ERR_HIP;
    }
    return GPTQ_OK;
}

gptq_status_t gptq_prepare(float* H_to_U, int64_t K, float percdamp, uint8_t* dead, float* damp_out,
                           int64_t* n_dead_out, void* workspace, size_t workspace_bytes, void* stream) {
    if (!H_to_U || K < 1 || !dead || !std::isfinite(percdamp) || percdamp < 0.f) return GPTQ_ERR_ARG;
    if (K > (int64_t)1 << 20) return GPTQ_ERR_ARG;
    if (!ws_ok(workspace, workspace_bytes, prepare_workspace_bytes(K))) return GPTQ_ERR_WORKSPACE;
    return prepare(H_to_U, K, 1, K * K, percdamp, dead, damp_out, n_dead_out, workspace,
                   static_cast<hipStream_t>(stream));
}

gptq_status_t gptq_prepare_groups(float* H_to_U, int64_t K, int64_t groups, int64_t group_stride, float percdamp,
                                  uint8_t* dead, float* damp_out, int64_t* n_dead_out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    if (!H_to_U || K < 1 || !dead || !std::isfinite(percdamp) || percdamp < 0.f) return GPTQ_ERR_ARG;
    if (K > (int64_t)1 << 20 || groups < 1 || groups > 65535 || group_stride < K * K) return GPTQ_ERR_ARG;
    if (!ws_ok(workspace, workspace_bytes, prepare_workspace_bytes(K, groups))) return GPTQ_ERR_WORKSPACE;
    return prepare(H_to_U, K, groups, group_stride, percdamp, dead, damp_out, n_dead_out, workspace,
                   static_cast<hipStream_t>(stream));
}

gptq_status_t gptq_asym_correction(const float* U, const float* A, float* P1, int64_t K, void* workspace,
                                   size_t workspace_bytes, void* stream) {
    if (!U || !A || !P1 || K < 1) return GPTQ_ERR_ARG;
    if (!ws_ok(workspace, workspace_bytes, asym_ws(K))) return GPTQ_ERR_WORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    Carver c(workspace);
    c.take<DevStatus>(1);
    float* T = c.take<float>((size_t)K * (size_t)K);
    TimerScope ts(st, GPTQ_TIMER_FACTOR_GEMM);
    // T = A U^T  (only the part on or above the diagonal is used)
    GemmArgs g1;
    g1.M = K; g1.N = K; g1.K1 = K;
    g1.A1 = A; g1.lda1 = K;
    g1.B1 = U; g1.ldb1 = K; g1.transB = true;       // B(k, n) = U[n][k], zero for k < n
    g1.C = T; g1.ldc = K;
    g1.flags = kGemmBLower | kGemmCUpper;
    if (gemm_f32(g1, 1, st) != hipSuccess) return GPTQ_ERR_HIP;
    // P1 = (T masked to k > m) U
    GemmArgs g2;
    g2.M = K; g2.N = K; g2.K1 = K;
    g2.A1 = T; g2.lda1 = K;
    g2.B1 = U; g2.ldb1 = K;                          // upper: zero for k > n
    g2.C = P1; g2.ldc = K;
    g2.flags = kGemmAStrictUpperMask | kGemmBUpper;
    if (gemm_f32(g2, 1, st) != hipSuccess) return GPTQ_ERR_HIP;
    return GPTQ_OK;
}

gptq_status_t gptq_quantize_layer(const void* W, gptq_dtype_t w_dtype, int64_t K, int64_t N, int64_t w_rs,
                                  int64_t w_cs, const float* U, const uint8_t* dead, const float* P1, int bits,
                                  int blocksize, unsigned flags, uint8_t* codes, int64_t c_rs, int64_t c_cs,
                                  float* scales, void* W_hat, float* losses, float* pre_round, const int32_t* perm,
                                  int64_t groupsize, int32_t* g_idx, void* workspace, size_t workspace_bytes,
                                  void* stream) {
    return quantize_common(W, w_dtype, K, N, w_rs, w_cs, 1, U, 0, dead, P1, bits, blocksize, flags, codes, c_rs, c_cs,
                           scales, W_hat, losses, pre_round, perm, groupsize, g_idx, workspace, workspace_bytes,
                           stream);
}

gptq_status_t gptq_quantize_layer_noalloc(const void* W, gptq_dtype_t w_dtype, int64_t K, int64_t N, int64_t w_rs,
                                          int64_t w_cs, const float* U, const uint8_t* dead, const float* P1, int bits,
                                          int blocksize, unsigned flags, uint8_t* codes, int64_t c_rs, int64_t c_cs,
                                          float* scales, void* W_hat, float* losses, float* pre_round,
                                          const int32_t* perm, int64_t groupsize, int32_t* g_idx, void* stream) {
    // The size check comes before any HIP call; the argument checks are those of gptq_quantize_layer, which runs
    // unchanged on the static scratch (the kernel timer is kept off so that no event is created).
    if (K < 1 || N < 1 || K > (int64_t)1 << 24 || N > (int64_t)1 << 28) return GPTQ_ERR_ARG;
    if (quantize_workspace_bytes(K, N, P1 != nullptr, (flags & GPTQ_FLAG_CAE) != 0) > kStaticScratchBytes)
        return GPTQ_ERR_WORKSPACE;
    void* ws = nullptr;
    const gptq_status_t r = static_scratch(&ws, true);
    if (r != GPTQ_OK) return r;
    TimerSuppress quiet;
    return quantize_common(W, w_dtype, K, N, w_rs, w_cs, 1, U, 0, dead, P1, bits, blocksize, flags, codes, c_rs, c_cs,
                           scales, W_hat, losses, pre_round, perm, groupsize, g_idx, ws, kStaticScratchBytes, stream);
}

gptq_status_t gptq_quantize_layer_groups(const void* W, gptq_dtype_t w_dtype, int64_t K, int64_t N, int64_t w_rs,
                                         int64_t w_cs, int64_t groups, const float* U, int64_t u_stride,
                                         const uint8_t* dead, const float* P1, int bits, int blocksize,
                                         unsigned flags, uint8_t* codes, int64_t c_rs, int64_t c_cs, float* scales,
                                         void* W_hat, float* losses, float* pre_round, const int32_t* perm,
                                         int64_t groupsize, int32_t* g_idx, void* workspace, size_t workspace_bytes,
                                         void* stream) {
    return quantize_common(W, w_dtype, K, N, w_rs, w_cs, groups, U, u_stride, dead, P1, bits, blocksize, flags, codes,
                           c_rs, c_cs, scales, W_hat, losses, pre_round, perm, groupsize, g_idx, workspace,
                           workspace_bytes, stream);
}

gptq_status_t gptq_act_order(float* H, float* A, int64_t K, int32_t* perm, void* workspace, size_t workspace_bytes,
                             void* stream) {
    if (!H || !perm || K < 1 || K > (int64_t)1 << 24) return GPTQ_ERR_ARG;
    if (!ws_ok(workspace, workspace_bytes, act_order_workspace_bytes(K))) return GPTQ_ERR_WORKSPACE;
    TimerScope ts(static_cast<hipStream_t>(stream), GPTQ_TIMER_OTHER);
    return act_order(H, A, K, perm, workspace, static_cast<hipStream_t>(stream)) == hipSuccess ? GPTQ_OK
                                                                                                : GPTQ_ERR_HIP;
}

gptq_status_t gptq_hadamard_rotate(const void* in, int64_t ld_in, void* out, int64_t ld_out, gptq_dtype_t dtype,
                                   int64_t rows, int64_t K, const int8_t* signs, void* stream) {
    if (!in || !out || rows < 0 || K < 16 || K > 16384 || (K & (K - 1)) != 0) return GPTQ_ERR_ARG;
    if (dtype != GPTQ_DTYPE_F32 && dtype != GPTQ_DTYPE_BF16) return GPTQ_ERR_ARG;
    if (ld_in < K || ld_out < K || (in == out && ld_in != ld_out)) return GPTQ_ERR_ARG;
    if (rows == 0) return GPTQ_OK;
    int n = 0;
    while ((int64_t(1) << n) < K) ++n;
    TimerScope ts(static_cast<hipStream_t>(stream), GPTQ_TIMER_OTHER);
    return hadamard_rows(in, ld_in, out, ld_out, dtype == GPTQ_DTYPE_BF16, rows, n, signs,
                         static_cast<hipStream_t>(stream)) == hipSuccess
               ? GPTQ_OK
               : GPTQ_ERR_HIP;
}

int64_t gptq_packed_words(int64_t K, int bits) {
    if (K < 0 || bits < 1 || bits > 8) return -1;
    return packed_words(K, bits);
}

gptq_status_t gptq_pack_codes(const uint8_t* codes, int64_t c_rs, int64_t c_cs, int64_t K, int64_t N, int bits,
                              uint32_t* packed, int64_t ldp, void* stream) {
    if (!codes || !packed || K < 1 || N < 1 || bits < 1 || bits > 8) return GPTQ_ERR_ARG;
    if (c_rs < 1 || c_cs < 1 || ldp < N) return GPTQ_ERR_ARG;
    TimerScope ts(static_cast<hipStream_t>(stream), GPTQ_TIMER_OTHER);
    return pack_codes(codes, c_rs, c_cs, K, N, bits, packed, ldp, static_cast<hipStream_t>(stream)) == hipSuccess
               ? GPTQ_OK
               : GPTQ_ERR_HIP;
}

gptq_status_t gptq_unpack_codes(const uint32_t* packed, int64_t ldp, int64_t K, int64_t N, int bits,
                                const float* scales, uint8_t* codes, int64_t c_rs, int64_t c_cs, void* W_hat,
                                gptq_dtype_t w_dtype, int64_t w_rs, int64_t w_cs, void* stream) {
    if (!packed || K < 1 || N < 1 || bits < 1 || bits > 8 || ldp < N) return GPTQ_ERR_ARG;
    if (codes && (c_rs < 1 || c_cs < 1)) return GPTQ_ERR_ARG;
    if (W_hat && (!scales || w_rs < 1 || w_cs < 1)) return GPTQ_ERR_ARG;
    if (W_hat && w_dtype != GPTQ_DTYPE_F32 && w_dtype != GPTQ_DTYPE_BF16) return GPTQ_ERR_ARG;
    TimerScope ts(static_cast<hipStream_t>(stream), GPTQ_TIMER_OTHER);
    return unpack_codes(packed, ldp, K, N, bits, scales, codes, c_rs, c_cs, W_hat, w_dtype == GPTQ_DTYPE_BF16, w_rs,
                        w_cs, static_cast<hipStream_t>(stream)) == hipSuccess
               ? GPTQ_OK
               : GPTQ_ERR_HIP;
}

}  // extern "C"
