// Shared definitions of the gfx950 kernels: vector types, MFMA wrappers, status word, workspace carving.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/gptq.h"

namespace gptq {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

// Status word kept at the head of every workspace (device-side error latch).
enum : uint32_t {
    kDevOk = 0,
    kDevNonFinite = 1u << 0,
    kDevNotPD = 1u << 1,
};

struct DevStatus {
    uint32_t flags;       // OR of kDev* bits
    uint32_t n_dead;
    float damp;
    float pad[61];        // keeps the header 256 bytes
};
static_assert(sizeof(DevStatus) == 256, "status header is 256 bytes");

constexpr size_t kAlign = 256;

__host__ __device__ inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Sequential carving of one workspace buffer into 256-byte aligned regions.
struct Carver {
    char* base;
    size_t off;
    explicit Carver(void* p) : base(static_cast<char*>(p)), off(0) {}
    template <typename T>
    T* take(size_t count) {
        off = align_up(off, kAlign);
        T* p = reinterpret_cast<T*>(base ? base + off : nullptr);
        off += count * sizeof(T);
        return p;
    }
    size_t bytes() const { return align_up(off, kAlign); }
};

// bf16 <-> fp32 bit helpers (bf16 is the upper half of binary32).
__device__ inline float bf16lo_to_f32(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ inline float bf16hi_to_f32(uint32_t packed) { return __uint_as_float(packed & 0xFFFF0000u); }

// Round-to-nearest-even fp32 -> bf16 of two values packed as (lo | hi << 16).
__device__ inline uint32_t pack_bf16x2_rne(float lo, float hi) {
    __bf16 a = (__bf16)lo;
    __bf16 b = (__bf16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// Grid of blocks for a 1-D launch, clamped to what hardware accepts in x.
inline dim3 grid1d(int64_t n, int threads) { return dim3((unsigned)ceil_div(n, threads)); }

}  // namespace gptq

#define GPTQ_HIP_CHECK(expr)                                          \
    do {                                                              \
        hipError_t _e = (expr);                                       \
        if (_e != hipSuccess) return GPTQ_ERR_HIP;                    \
    } while (0)

#define GPTQ_LAUNCH_CHECK()                                           \
    do {                                                              \
        hipError_t _e = hipGetLastError();                            \
        if (_e != hipSuccess) return GPTQ_ERR_HIP;                    \
    } while (0)
