// Shared device/host helpers of the gfx950 MoE library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

typedef uint16_t bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int WAVE = 64;

// A value every lane of the wave holds alike, made visibly uniform to the compiler (kept in
// a scalar register), so that address math and buffer descriptors built from it stay scalar.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even (inputs are finite).
__device__ __forceinline__ bf16_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
    return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}

__device__ __forceinline__ float lo_bf(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float hi_bf(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
// Non-temporal forms, for rows that a kernel reads or writes exactly once: they neither
// allocate in nor evict from the caches, so a stream over hundreds of MB does not first have
// to push other kernels' dirty lines out to HBM.
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16_nt(void* p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}


// Wave-level inclusive scan (sum) of an int over 64 lanes, fixed order.
__device__ __forceinline__ int wave_incl_scan(int v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int o = __shfl_up(v, d, 64);
        if (lane >= d) v += o;
    }
    return v;
}

}  // namespace moe

// Host-side argument checks.
#define MOE_REQUIRE(cond)                 \
    do {                                  \
        if (!(cond)) return MOE_EINVAL;   \
    } while (0)

#define MOE_LAUNCH_CHECK()                                      \
    do {                                                        \
        if (hipGetLastError() != hipSuccess) return MOE_EHIP;   \
    } while (0)

// Rows the weight-gradient products of the backward reduce over: the routed rows of every
// pass of a macrobatch (pass p's rows start at row p * pass_rows; offsets [P][E+1] are
// pass-local), or of one pass (P = 1, offsets [E+1]), or all R rows (offsets null: shared
// experts).
struct MoeWgradSpan {
    const moe::bf16_t* xp;
    const moe::bf16_t* h;
    const moe::bf16_t* dy;
    const moe::bf16_t* dgu;
    const int32_t* offsets;
    int P, pass_rows, R;
    moe::bf16_t* dw1;
    moe::bf16_t* dw2;
};

// dy rows formed where they are consumed, instead of read from a stored copy: routed row p is
// bf16(w * dout[s / k]) for (s, w) = src[p] when 0 <= s < T k and pos[s] == p, and zeros
// otherwise -- the combine backward's dy; that kernel then writes src (the weight's bits in
// .y) instead of dy.
struct MoeTokPull {
    const moe::bf16_t* dout;  // [T, C]
    const int2* src;          // [R]: routed row -> (t k + j, bits of w[t, j])
    const int32_t* pos;       // [T, k]
    int T, k;
};

// Returns MOE_OK when the current device is gfx950 (cached per device).
int moe_check_device();

// Optional launch tracing (moe_trace_begin in moe.h): with tracing armed on the calling
// thread, each launch is bracketed by two event records on its stream.
void moe_trace_pre(hipStream_t st);
void moe_trace_post(const char* name, hipStream_t st);
#define MOE_TRACED(name, st, ...)       \
    do {                                \
        moe_trace_pre(st);              \
        __VA_ARGS__;                    \
        moe_trace_post(name, st);       \
    } while (0)

static inline size_t moe_align256(size_t n) { return (n + 255) & ~(size_t)255; }
