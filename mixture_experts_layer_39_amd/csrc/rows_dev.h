// Device bodies of the token-row steps shared by the kernels of rows.hip and the
// single-launch layer: the token-driven dispatch and the fixed-order combine.  See rows.hip
// for the access pattern and the reduction orders.
#pragma once

#include "common.h"

namespace moe {

constexpr int ROW_UN = 8;  // 16-byte loads a thread issues before its first store
constexpr int MAXK = 64;   // largest k the row kernels stage in LDS
constexpr int RG = 2;      // 16-byte chunks per thread per pass in the gather-reduce kernels

// Token-driven dispatch of token t by NTHR threads (the whole block): the token's k
// destination rows (pos[t,j]) are filled from one read of its source row.  sp: k ints of LDS.
template <int NTHR>
__device__ __forceinline__ void dispatch_token(const bf16_t* __restrict__ x, int H, int k,
                                               const int32_t* __restrict__ pos, int R,
                                               bf16_t* __restrict__ xp, const int t, int* sp) {
    const bf16_t* in = x + (size_t)t * H;
    if (threadIdx.x < k) sp[threadIdx.x] = pos[(size_t)t * k + threadIdx.x];
    const int nc = H / 8;
    // the loop bound is block-uniform, so the barrier (pos staged) in its first pass is too
    for (int c0 = 0; c0 < nc; c0 += NTHR * ROW_UN) {
        u32x4 v[ROW_UN];
#pragma unroll
        for (int u = 0; u < ROW_UN; ++u) {
            const int c = c0 + threadIdx.x + u * NTHR;
            v[u] = c < nc ? ld16(in + c * 8) : u32x4{0, 0, 0, 0};
        }
        if (c0 == 0) __syncthreads();
        for (int j = 0; j < k; ++j) {
            const int r = sp[j];
            if (r < 0 || r >= R) continue;
            bf16_t* out = xp + (size_t)r * H;
#pragma unroll
            for (int u = 0; u < ROW_UN; ++u) {
                const int c = c0 + threadIdx.x + u * NTHR;
                if (c < nc) st16(out + c * 8, v[u]);
            }
        }
    }
    __syncthreads();  // sp may be reused
}

// Combine of token t by NTHR threads (the whole block).  Per element, fp32: acc = 0;
// acc += w[t,j]*y[pos[t,j]] for j = 0..k-1; acc += ys[s,t] for s = 0..S-1; one rounding to
// bf16.  sp, sw: k ints and k floats of LDS.  Every routed row and the output row are touched
// once, so they move with non-temporal loads and stores (measured 49 against 56 us at the
// EP-64 share with cold caches, and 50 against 99 us when the caches hold other dirty data).
template <int NTHR>
__device__ __forceinline__ void combine_token(const bf16_t* __restrict__ y,
                                              const int32_t* __restrict__ pos,
                                              const float* __restrict__ w, int T, int k, int H,
                                              int R, const bf16_t* __restrict__ ys, int S,
                                              bf16_t* __restrict__ out, const int t, int* sp,
                                              float* sw) {
    if (threadIdx.x < k) {
        int p = pos[(size_t)t * k + threadIdx.x];
        sp[threadIdx.x] = (p >= 0 && p < R) ? p : -1;
        sw[threadIdx.x] = w[(size_t)t * k + threadIdx.x];
    }
    __syncthreads();
    const int nc = H / 8;
    // each thread takes RG chunks per pass and loads every slot's rows of them before
    // summing any (the summation order per element is unchanged)
    for (int c0 = threadIdx.x; c0 < nc; c0 += NTHR * RG) {
        float acc[RG][8];
#pragma unroll
        for (int g = 0; g < RG; ++g)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[g][i] = 0.0f;
        for (int j0 = 0; j0 < k; j0 += 8) {
            u32x4 v[RG][8];
#pragma unroll
            for (int g = 0; g < RG; ++g)
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int j = j0 + u, c = c0 + g * NTHR;
                    const int p = j < k ? sp[j] : -1;
                    v[g][u] = (p >= 0 && c < nc) ? ld16_nt(y + (size_t)p * H + c * 8) : u32x4{0, 0, 0, 0};
                }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int j = j0 + u;
                if (j >= k || sp[j] < 0) continue;
                const float wj = sw[j];
#pragma unroll
                for (int g = 0; g < RG; ++g)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        acc[g][2 * q] = __fadd_rn(acc[g][2 * q], __fmul_rn(wj, lo_bf(v[g][u][q])));
                        acc[g][2 * q + 1] = __fadd_rn(acc[g][2 * q + 1], __fmul_rn(wj, hi_bf(v[g][u][q])));
                    }
            }
        }
#pragma unroll
        for (int g = 0; g < RG; ++g) {
            const int c = c0 + g * NTHR;
            if (c >= nc) continue;
            for (int s = 0; s < S; ++s) {
                u32x4 v = ld16_nt(ys + ((size_t)s * T + t) * H + c * 8);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[g][2 * q] = __fadd_rn(acc[g][2 * q], lo_bf(v[q]));
                    acc[g][2 * q + 1] = __fadd_rn(acc[g][2 * q + 1], hi_bf(v[q]));
                }
            }
            u32x4 o;
#pragma unroll
            for (int q = 0; q < 4; ++q) o[q] = pack_bf2(acc[g][2 * q], acc[g][2 * q + 1]);
            st16_nt(out + (size_t)t * H + c * 8, o);
        }
    }
    __syncthreads();  // sp, sw may be reused
}

// The combine of one token by one wave (no LDS, no block barrier), for a kernel that keeps one
// block per CU: each wave of the block works on its own token, so that a CU has several
// tokens' loads in flight.  Same results, bit for bit, as combine_token (same order per
// element), and the same non-temporal accesses.  pos / w of slot j are held by lane j and
// broadcast with a lane read.
template <int G>
__device__ __forceinline__ void combine_token_wave(const bf16_t* __restrict__ y,
                                                   const int32_t* __restrict__ pos,
                                                   const float* __restrict__ w, int T, int k,
                                                   int H, int R, const bf16_t* __restrict__ ys,
                                                   int S, bf16_t* __restrict__ out, const int t,
                                                   const int lane) {
    int myp = -1;
    float myw = 0.0f;
    if (lane < k) {
        const int p = pos[(size_t)t * k + lane];
        myp = (p >= 0 && p < R) ? p : -1;
        myw = w[(size_t)t * k + lane];
    }
    const int nc = H / 8;
    for (int c0 = lane; c0 < nc; c0 += 64 * G) {
        float acc[G][8];
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[g][i] = 0.0f;
        for (int j0 = 0; j0 < k; j0 += 8) {
            u32x4 v[G][8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int p = __shfl(myp, (j0 + u) & 63, 64);
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const int c = c0 + g * 64;
                    v[g][u] = (j0 + u < k && p >= 0 && c < nc) ? ld16_nt(y + (size_t)p * H + c * 8)
                                                               : u32x4{0, 0, 0, 0};
                }
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int j = j0 + u;
                const int p = __shfl(myp, j & 63, 64);
                const float wj = __shfl(myw, j & 63, 64);
                if (j >= k || p < 0) continue;
#pragma unroll
                for (int g = 0; g < G; ++g)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        acc[g][2 * q] = __fadd_rn(acc[g][2 * q], __fmul_rn(wj, lo_bf(v[g][u][q])));
                        acc[g][2 * q + 1] = __fadd_rn(acc[g][2 * q + 1], __fmul_rn(wj, hi_bf(v[g][u][q])));
                    }
            }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int c = c0 + g * 64;
            if (c >= nc) continue;
            for (int s = 0; s < S; ++s) {
                u32x4 v = ld16_nt(ys + ((size_t)s * T + t) * H + c * 8);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[g][2 * q] = __fadd_rn(acc[g][2 * q], lo_bf(v[q]));
                    acc[g][2 * q + 1] = __fadd_rn(acc[g][2 * q + 1], hi_bf(v[q]));
                }
            }
            u32x4 o;
#pragma unroll
            for (int q = 0; q < 4; ++q) o[q] = pack_bf2(acc[g][2 * q], acc[g][2 * q + 1]);
            st16_nt(out + (size_t)t * H + c * 8, o);
        }
    }
}

}  // namespace moe
