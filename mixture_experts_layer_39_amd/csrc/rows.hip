// Row-wise, HBM-bound kernels: dispatch (gather, optionally MX-quantising), combine, the
// combine backward, the un-permute reduce of dX, the router backward and MX quantisation.
//
// Each token row is moved with 16-byte vector accesses by consecutive lanes, so every wave
// access is a contiguous, fully coalesced 1 KB segment; a row gather needs no LDS staging
// because source and destination rows are both contiguous.  Every reduction runs in a fixed
// order (slots, then shared experts; fixed butterfly trees), so results are bit-identical
// from run to run (pulsen.vercel.app, "Cursor åpner megakernelen…", ¶3-¶4).
#include "mx_dev.h"
#include "rows_dev.h"

namespace moe {

// Quantise 32 fp32 values (one block) held in v[]; returns the scale code, codes packed
// little-endian into q[8].
__device__ __forceinline__ int mx_block(const float* v, int mode, uint32_t* q) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    int sc = mx_scale_code(amax, mode);
    int sh = 127 - sc;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        q[i] = e4m3x4(ldexpf(v[4 * i], sh), ldexpf(v[4 * i + 1], sh), ldexpf(v[4 * i + 2], sh),
                      ldexpf(v[4 * i + 3], sh));
    return sc;
}

// ------------------------------------------------------------------ dispatch
// One block per destination row: xp[r,:] = x[src[r]/k,:].  Each thread issues all of its
// 16-byte loads (up to UN) before any store, so a CU keeps enough bytes in flight to cover
// the memory latency.

__global__ __launch_bounds__(128) void dispatch_kernel(const bf16_t* __restrict__ x, int64_t n_pairs,
                                                       int H, int k, const int32_t* __restrict__ src,
                                                       bf16_t* __restrict__ xp) {
    const int r = blockIdx.x;
    const int s = src[r];
    const bool ok = s >= 0 && s < n_pairs;
    const bf16_t* in = x + (size_t)(ok ? s / k : 0) * H;
    bf16_t* out = xp + (size_t)r * H;
    const int nc = H / 8;
    for (int c0 = threadIdx.x; c0 < nc; c0 += 128 * ROW_UN) {
        u32x4 v[ROW_UN];
#pragma unroll
        for (int u = 0; u < ROW_UN; ++u) {
            const int c = c0 + u * 128;
            v[u] = (ok && c < nc) ? ld16(in + c * 8) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < ROW_UN; ++u) {
            const int c = c0 + u * 128;
            if (c < nc) st16(out + c * 8, v[u]);
        }
    }
}

__global__ __launch_bounds__(128) void dispatch_tok_kernel(const bf16_t* __restrict__ x, int H,
                                                           int k, const int32_t* __restrict__ pos,
                                                           int R, bf16_t* __restrict__ xp) {
    __shared__ int sp[MAXK];
    dispatch_token<128>(x, H, k, pos, R, xp, blockIdx.x, sp);
}

// Dispatch with MX quantisation: one thread per 32-value block of the destination row.
__global__ __launch_bounds__(256) void dispatch_mx_kernel(const bf16_t* __restrict__ x, int64_t n_pairs,
                                                          int H, int k, const int32_t* __restrict__ src,
                                                          bf16_t* __restrict__ xp,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
    const int r = blockIdx.y;
    const int nb = H / 32;
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= nb) return;
    const int s = src[r];
    const bool ok = s >= 0 && s < n_pairs;
    const bf16_t* in = x + (size_t)(ok ? s / k : 0) * H + b * 32;
    float v[32];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        u32x4 q = ok ? ld16(in + c * 8) : u32x4{0, 0, 0, 0};
        if (xp) st16(xp + (size_t)r * H + b * 32 + c * 8, q);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[c * 8 + 2 * j] = lo_bf(q[j]);
            v[c * 8 + 2 * j + 1] = hi_bf(q[j]);
        }
    }
    uint32_t q[8];
    int sc = mx_block(v, MOE_MX_FLOOR, q);
    uint8_t* co = codes + (size_t)r * H + b * 32;
    st16(co, u32x4{q[0], q[1], q[2], q[3]});
    st16(co + 16, u32x4{q[4], q[5], q[6], q[7]});
    scales[(size_t)r * nb + b] = (uint8_t)sc;
}

// Token-driven dispatch with MX quantisation: one thread per 8 values (a 16-byte chunk) of a
// source row, four consecutive lanes per 32-value block, so a wave reads 1 KB of the row and
// writes 512 bytes of codes in one piece.  The block maximum takes two exchanges between the
// four lanes; the codes and scale are those of mx_block (same maximum, scale rule and
// encoder).  Each chunk's codes and its bf16 copy (xp, optional) go to all k rows.
__global__ __launch_bounds__(256) void dispatch_mx_tok_kernel(const bf16_t* __restrict__ x, int H,
                                                              int k, const int32_t* __restrict__ pos,
                                                              int R, bf16_t* __restrict__ xp,
                                                              uint8_t* __restrict__ codes,
                                                              uint8_t* __restrict__ scales) {
    __shared__ int sp[MAXK];
    const int t = blockIdx.y;
    const int nc = H / 8, nb = H / 32;
    const int c = blockIdx.x * blockDim.x + threadIdx.x;  // chunk; block c / 4
    const bool live = c < nc;  // H % 32 == 0: a block's four lanes are all live or all not
    const u32x4 raw = live ? ld16(x + (size_t)t * H + c * 8) : u32x4{0, 0, 0, 0};
    if (threadIdx.x < k) sp[threadIdx.x] = pos[(size_t)t * k + threadIdx.x];
    float v[8];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[2 * j] = lo_bf(raw[j]);
        v[2 * j + 1] = hi_bf(raw[j]);
        amax = fmaxf(amax, fmaxf(fabsf(v[2 * j]), fabsf(v[2 * j + 1])));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    const int sc = mx_scale_code(amax, MOE_MX_FLOOR);
    const int sh = 127 - sc;
    const uint2 q = make_uint2(e4m3x4(ldexpf(v[0], sh), ldexpf(v[1], sh), ldexpf(v[2], sh),
                                      ldexpf(v[3], sh)),
                               e4m3x4(ldexpf(v[4], sh), ldexpf(v[5], sh), ldexpf(v[6], sh),
                                      ldexpf(v[7], sh)));
    __syncthreads();
    if (!live) return;
    for (int j = 0; j < k; ++j) {
        const int r = sp[j];
        if (r < 0 || r >= R) continue;
        if (xp) st16(xp + (size_t)r * H + c * 8, raw);
        *reinterpret_cast<uint2*>(codes + (size_t)r * H + c * 8) = q;
        if ((c & 3) == 0) scales[(size_t)r * nb + c / 4] = (uint8_t)sc;
    }
}

// ------------------------------------------------------------------ mx_quantize
// One thread per 32-value block of a bf16 or fp32 input: the block's E8M0 scale and codes.
template <bool F32>
__global__ __launch_bounds__(256) void mx_quantize_kernel(const void* __restrict__ in, int64_t nblocks,
                                                          int mode, uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
    int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= nblocks) return;
    float v[32];
    if (F32) {
        const float* p = (const float*)in + b * 32;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            u32x4 q = ld16(p + c * 4);
#pragma unroll
            for (int j = 0; j < 4; ++j) v[c * 4 + j] = __uint_as_float(q[j]);
        }
    } else {
        const bf16_t* p = (const bf16_t*)in + b * 32;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            u32x4 q = ld16(p + c * 8);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[c * 8 + 2 * j] = lo_bf(q[j]);
                v[c * 8 + 2 * j + 1] = hi_bf(q[j]);
            }
        }
    }
    uint32_t q[8];
    int sc = mx_block(v, mode, q);
    st16(codes + b * 32, u32x4{q[0], q[1], q[2], q[3]});
    st16(codes + b * 32 + 16, u32x4{q[4], q[5], q[6], q[7]});
    scales[b] = (uint8_t)sc;
}

// ------------------------------------------------------------------ combine
// One block per token.  Per element, fp32: acc = 0; acc += w[t,j]*y[pos[t,j]] for j = 0..k-1;
// acc += ys[s,t] for s = 0..S-1; one rounding to bf16.

// The block size is the smallest multiple of 64 threads (at most 512) that covers the row in
// one pass of RG chunks per thread: 448 for H = 7168, 128 for H = 2048.
template <int NTHR>
__global__ __launch_bounds__(NTHR) void combine_kernel(const bf16_t* __restrict__ y,
                                                       const int32_t* __restrict__ pos,
                                                       const float* __restrict__ w, int T, int k,
                                                       int H, int R, const bf16_t* __restrict__ ys,
                                                       int S, bf16_t* __restrict__ out) {
    __shared__ int sp[MAXK];
    __shared__ float sw[MAXK];
    combine_token<NTHR>(y, pos, w, T, k, H, R, ys, S, out, blockIdx.x, sp, sw);
}

static int combine_threads(int H) {
    const int per_pass = (H / 8 + RG - 1) / RG;
    return std::min(512, std::max(64, (per_pass + 63) / 64 * 64));
}

// ------------------------------------------------------------------ combine backward
// One block per token: dy[pos[t,j],:] = bf16(w[t,j] * dout[t,:]) and
// dw[t,j] = <dout[t,:], y[pos[t,j],:]> in fp32 with a fixed reduction tree: each thread sums
// its chunks in ascending order, then a butterfly over the wave and the four waves in order.
// dy null: no dy rows; src (if given) receives src[pos[t,j]] = (t k + j, bits of w[t,j])
// instead, so that the consumer of dy forms its rows itself (MoeTokPull).
constexpr int CB_UN = 4;

__global__ __launch_bounds__(256) void combine_bwd_kernel(const bf16_t* __restrict__ dout,
                                                          const bf16_t* __restrict__ y,
                                                          const int32_t* __restrict__ pos,
                                                          const float* __restrict__ w, int k,
                                                          int H, int R, bf16_t* __restrict__ dy,
                                                          int2* __restrict__ src,
                                                          float* __restrict__ dw) {
    const int t = blockIdx.x;
    __shared__ float red[4][MAXK];
    const int nc = H / 8;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const bf16_t* g_row = dout + (size_t)t * H;
    if (src && threadIdx.x < k) {
        const int s = t * k + (int)threadIdx.x;
        const int pp = pos[s];
        if (pp >= 0 && pp < R) src[pp] = make_int2(s, __float_as_int(w[s]));
    }
    if (nc <= 256 * CB_UN) {
        // The row in one pass: the thread's dout chunks are loaded once for all slots, slot
        // j's position and weight come from lane j of every wave (k <= 64), and slot j+1's
        // y chunks are loaded before slot j is summed.  Per slot and element the arithmetic
        // and its order are those of the general loop below.
        int myp = -1;
        float myw = 0.0f;
        if (lane < k) {
            const int pp = pos[(size_t)t * k + lane];
            myp = (pp >= 0 && pp < R) ? pp : -1;
            myw = w[(size_t)t * k + lane];
        }
        u32x4 g[CB_UN], v[CB_UN], vn[CB_UN];
#pragma unroll
        for (int u = 0; u < CB_UN; ++u) {
            const int c = threadIdx.x + u * 256;
            g[u] = c < nc ? ld16(g_row + c * 8) : u32x4{0, 0, 0, 0};
        }
        auto load_y = [&](int p, u32x4* dst) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < CB_UN; ++u) {
                const int c = threadIdx.x + u * 256;
                dst[u] = (p >= 0 && c < nc) ? ld16_nt(y + (size_t)p * H + c * 8)
                                            : u32x4{0, 0, 0, 0};
            }
        };
        int p = __builtin_amdgcn_readlane(myp, 0);
        load_y(p, v);
        for (int j = 0; j < k; ++j) {
            const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(myw), j));
            const int pnext = j + 1 < k ? __builtin_amdgcn_readlane(myp, j + 1) : -1;
            load_y(pnext, vn);
            float part = 0.0f;
            if (p >= 0) {
#pragma unroll
                for (int u = 0; u < CB_UN; ++u) {
                    const int c = threadIdx.x + u * 256;
                    if (c >= nc) continue;
                    u32x4 o;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float g0 = lo_bf(g[u][q]), g1 = hi_bf(g[u][q]);
                        part = __fadd_rn(part, __fmul_rn(g0, lo_bf(v[u][q])));
                        part = __fadd_rn(part, __fmul_rn(g1, hi_bf(v[u][q])));
                        o[q] = pack_bf2(__fmul_rn(wj, g0), __fmul_rn(wj, g1));
                    }
                    if (dy) st16(dy + (size_t)p * H + c * 8, o);
                }
            }
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) part = __fadd_rn(part, __shfl_xor(part, d, 64));
            if (lane == 0) red[wid][j] = part;
#pragma unroll
            for (int u = 0; u < CB_UN; ++u) v[u] = vn[u];
            p = pnext;
        }
    } else {
        for (int j = 0; j < k; ++j) {
            const int p = pos[(size_t)t * k + j];
            const bool ok = p >= 0 && p < R;
            const float wj = w[(size_t)t * k + j];
            float part = 0.0f;
            if (ok) {
                const bf16_t* y_row = y + (size_t)p * H;
                for (int c0 = threadIdx.x; c0 < nc; c0 += 256 * CB_UN) {
                    u32x4 g[CB_UN], v[CB_UN];
#pragma unroll
                    for (int u = 0; u < CB_UN; ++u) {
                        const int c = c0 + u * 256;
                        g[u] = c < nc ? ld16(g_row + c * 8) : u32x4{0, 0, 0, 0};
                        v[u] = c < nc ? ld16_nt(y_row + c * 8) : u32x4{0, 0, 0, 0};
                    }
#pragma unroll
                    for (int u = 0; u < CB_UN; ++u) {
                        const int c = c0 + u * 256;
                        if (c >= nc) continue;
                        u32x4 o;
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const float g0 = lo_bf(g[u][q]), g1 = hi_bf(g[u][q]);
                            part = __fadd_rn(part, __fmul_rn(g0, lo_bf(v[u][q])));
                            part = __fadd_rn(part, __fmul_rn(g1, hi_bf(v[u][q])));
                            o[q] = pack_bf2(__fmul_rn(wj, g0), __fmul_rn(wj, g1));
                        }
                        if (dy) st16(dy + (size_t)p * H + c * 8, o);
                    }
                }
            }
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) part = __fadd_rn(part, __shfl_xor(part, d, 64));
            if (lane == 0) red[wid][j] = part;
        }
    }
    __syncthreads();
    if (threadIdx.x < k) {
        int j = threadIdx.x;
        float s = __fadd_rn(__fadd_rn(red[0][j], red[1][j]), __fadd_rn(red[2][j], red[3][j]));
        dw[(size_t)t * k + j] = s;
    }
}

// ------------------------------------------------------------------ un-permute reduce
// dx[t,:] = sum_j dxp[pos[t,j],:] + sum_s dxs[s,t,:], fp32 in that order, one rounding.  As
// the combine: block size from H, rows read and written once with non-temporal accesses.
template <int NTHR>
__global__ __launch_bounds__(NTHR) void unpermute_kernel(const bf16_t* __restrict__ dxp,
                                                        const int32_t* __restrict__ pos, int T,
                                                        int k, int H, int R,
                                                        const bf16_t* __restrict__ dxs, int S,
                                                        int ldT, bf16_t* __restrict__ dx) {
    const int t = blockIdx.x;
    __shared__ int sp[MAXK];
    if (threadIdx.x < k) {
        int p = pos[(size_t)t * k + threadIdx.x];
        sp[threadIdx.x] = (p >= 0 && p < R) ? p : -1;
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
                    v[g][u] = (p >= 0 && c < nc) ? ld16_nt(dxp + (size_t)p * H + c * 8) : u32x4{0, 0, 0, 0};
                }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int j = j0 + u;
                if (j >= k || sp[j] < 0) continue;
#pragma unroll
                for (int g = 0; g < RG; ++g)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        acc[g][2 * q] = __fadd_rn(acc[g][2 * q], lo_bf(v[g][u][q]));
                        acc[g][2 * q + 1] = __fadd_rn(acc[g][2 * q + 1], hi_bf(v[g][u][q]));
                    }
            }
        }
#pragma unroll
        for (int g = 0; g < RG; ++g) {
            const int c = c0 + g * NTHR;
            if (c >= nc) continue;
            for (int s = 0; s < S; ++s) {
                u32x4 v = ld16_nt(dxs + ((size_t)s * ldT + t) * H + c * 8);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[g][2 * q] = __fadd_rn(acc[g][2 * q], lo_bf(v[q]));
                    acc[g][2 * q + 1] = __fadd_rn(acc[g][2 * q + 1], hi_bf(v[q]));
                }
            }
            u32x4 o;
#pragma unroll
            for (int q = 0; q < 4; ++q) o[q] = pack_bf2(acc[g][2 * q], acc[g][2 * q + 1]);
            st16_nt(dx + (size_t)t * H + c * 8, o);
        }
    }
}

// ------------------------------------------------------------------ router backward
// One wave per token; lane l owns logits e = l + 64*i.  Derivative of the weight formulas
// (selection passes no gradient):
//   softmax renorm:    dL[i_j] = w_j (dw_j - sum w dw)
//   softmax full:      dL[e]   = p_e (dw at e - sum w dw)
//   sigmoid renorm:    dL[i_j] = s_j(1-s_j) (c/S)(dw_j - sum (w/c) dw),  S = sum s
//   sigmoid plain:     dL[i_j] = c dw_j s_j (1-s_j)
__global__ __launch_bounds__(256) void router_bwd_kernel(const int32_t* __restrict__ idx,
                                                         const float* __restrict__ w,
                                                         const float* __restrict__ s_sel,
                                                         const float* __restrict__ dw,
                                                         const float* __restrict__ logits, int T,
                                                         int E, int k, int score, int renorm,
                                                         float c, float* __restrict__ dL) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const bool act = lane < k;
    const size_t o = (size_t)t * k + lane;
    int id = act ? idx[o] : -1;
    float wj = act ? w[o] : 0.0f, gj = act ? dw[o] : 0.0f, sj = act ? s_sel[o] : 0.0f;
    float wg = wj * gj;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) wg = __fadd_rn(wg, __shfl_xor(wg, d, 64));
    float ssum = sj;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) ssum = __fadd_rn(ssum, __shfl_xor(ssum, d, 64));
    float contrib = 0.0f;  // this slot's gradient at its expert
    if (score == MOE_SCORE_SOFTMAX) {
        contrib = renorm ? wj * (gj - wg) : wj * gj;
    } else {
        float ds = renorm ? (c / ssum) * (gj - wg / c) : c * gj;
        contrib = ds * sj * (1.0f - sj);
    }
    float m = 0.0f, se = 1.0f;
    const bool full = score == MOE_SCORE_SOFTMAX && !renorm;
    if (full) {
        const float* L = logits + (size_t)t * E;
        m = -INFINITY;
        for (int e = lane; e < E; e += 64) m = fmaxf(m, L[e]);
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
        se = 0.0f;
        for (int e = lane; e < E; e += 64) se += expf(L[e] - m);
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) se = __fadd_rn(se, __shfl_xor(se, d, 64));
    }
    for (int e0 = 0; e0 < E; e0 += 64) {
        int e = e0 + lane;
        float v = 0.0f;
        if (full && e < E) v = -(expf(logits[(size_t)t * E + e] - m) / se) * wg;
        for (int j = 0; j < k; ++j) {
            int idj = __shfl(id, j, 64);
            float cj = __shfl(contrib, j, 64);
            if (idj == e) v += cj;
        }
        if (e < E) dL[(size_t)t * E + e] = v;
    }
}

// ------------------------------------------------------------------ mx_quantize_t
// Quantisation along the first dimension of each [A, B] matrix of a batch, written transposed:
// codes [batch][B][A], scales [batch][B][A/32].  One thread per (column, 32-row block): it
// reads its column's 32 values (consecutive threads read consecutive columns, so every row
// access is coalesced) and writes the block's 32 codes as two 16-byte stores.
__global__ __launch_bounds__(256) void mx_quantize_t_kernel(const bf16_t* __restrict__ in, int A,
                                                            int B, int mode,
                                                            uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales) {
    const int col = blockIdx.x * blockDim.x + threadIdx.x;
    const int ab = blockIdx.y;            // 32-row block
    const int64_t m = blockIdx.z;         // matrix of the batch
    if (col >= B) return;
    const bf16_t* p = in + (m * A + (int64_t)ab * 32) * B + col;
    float v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = __uint_as_float((uint32_t)p[(int64_t)i * B] << 16);
    uint32_t q[8];
    const int sc = mx_block(v, mode, q);
    uint8_t* out = codes + (m * B + col) * A + ab * 32;
    st16(out, u32x4{q[0], q[1], q[2], q[3]});
    st16(out + 16, u32x4{q[4], q[5], q[6], q[7]});
    scales[(m * B + col) * (A / 32) + ab] = (uint8_t)sc;
}

// ------------------------------------------------------------------ mx_dequantize
// value = E4M3(code) * 2^(scale - 127) in fp32, rounded to bf16 (exact for every normal bf16
// value: a code has 3 mantissa bits).  One thread per 16 codes (half a block): 16-byte code
// loads, so a wave reads 1 KB in one piece.  The codes decode with the hardware fp8 -> fp32
// conversion, exact for every finite E4M3FN code (the quantisers here never emit the NaN
// code).
__global__ __launch_bounds__(256) void mx_dequantize_kernel(const uint8_t* __restrict__ codes,
                                                            const uint8_t* __restrict__ scales,
                                                            int64_t nblocks,
                                                            bf16_t* __restrict__ out) {
    const int64_t hb = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // half-block index
    if (hb >= 2 * nblocks) return;
    const u32x4 c = ld16_nt(codes + hb * 16);
    const float f = ldexpf(1.0f, (int)scales[hb >> 1] - 127);
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[i], false);  // bytes 0, 1
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[i], true);   // bytes 2, 3
        w[2 * i] = pack_bf2(lo[0] * f, lo[1] * f);
        w[2 * i + 1] = pack_bf2(hi[0] * f, hi[1] * f);
    }
    st16(out + hb * 16, u32x4{w[0], w[1], w[2], w[3]});
    st16(out + hb * 16 + 8, u32x4{w[4], w[5], w[6], w[7]});
}

// ------------------------------------------------------------------ token-axis quantisation
// The weight-gradient operands of the MXFP8 backward: X [R, C] (routed rows in expert order)
// quantised along the rows of each expert, written transposed as codes [C][Kp] and scales
// [C][Kp/32].  Expert e's rows occupy the code columns [P_e, P_e + pad(cnt_e)), where pad
// rounds up to a whole K step (128) and P_e is the sum of the padded counts before e; the
// 32-row blocks start at the expert's first row and the padding holds zero codes.  Columns
// past the last expert are zero.  Optionally (rcodes) the same rows are also quantised along
// C into rcodes [R][C], rscales [R][C/32] (the dgrad operand).  A 128-position block never
// straddles two experts.
//
// One block per (128 columns, 128 padded positions), C % 128 == 0:
//  1. the 128 x 128 tile of X is staged through LDS with 16-byte row loads (all of a
//     thread's loads issued first); X may also come as MX codes with scales along C
//     (TOK_IN_MX), decoded while staging exactly as mx_dequantize decodes them (so the staged
//     values are those a dequantised copy would hold), or as the combine backward's dy rows
//     formed from their tokens (TOK_IN_PULL, MoeTokPull: the same product and rounding);
//  2. column pass: wave w takes the rows 32w .. 32w+31, lane l the column pair 2l, 2l+1
//     (one dword LDS read per row: 64 consecutive dwords, conflict-free); row pass: items
//     (row r, 32-column block b), four lanes per row, 64 contiguous LDS bytes each;
//  3. the codes and scales go back into LDS as byte images of their output lines
//     (a column's 128 token codes, a row's 128 column codes, four scale bytes each), and
//  4. leave as whole 128-byte lines, eight lanes per line, and 4-byte scale words.
// The element order of every 32-value block, and so every code and scale, is unchanged.
constexpr int TOK_PAD = 128, TOK_COLS = 128;
constexpr int TOK_LD = TOK_COLS * 2 + 16;  // bytes per staged input row (16-byte aligned)
constexpr int TOK_OL = 128 + 16;           // bytes per staged output line
constexpr int TOK_LDS = 2 * TOK_PAD * TOK_OL + 2 * 128 * 4;  // >= TOK_PAD * TOK_LD

constexpr int TOK_IN_BF16 = 0, TOK_IN_MX = 1, TOK_IN_PULL = 2;

template <int IN>
__global__ __launch_bounds__(256) void mx_quantize_tok_kernel(const bf16_t* __restrict__ X,
                                                              const uint8_t* __restrict__ Xq,
                                                              const uint8_t* __restrict__ Xs,
                                                              int R, int C,
                                                              const int32_t* __restrict__ offsets,
                                                              int E, int Kp,
                                                              uint8_t* __restrict__ codes,
                                                              uint8_t* __restrict__ scales,
                                                              uint8_t* __restrict__ rcodes,
                                                              uint8_t* __restrict__ rscales,
                                                              uint8_t* __restrict__ cpanel,
                                                              uint8_t* __restrict__ rpanel,
                                                              MoeTokPull pull) {
    static_assert(TOK_LDS >= TOK_PAD * TOK_LD, "output images reuse the input tile");
    __shared__ __attribute__((aligned(16))) uint8_t lds[TOK_LDS];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int p = blockIdx.y * TOK_PAD;  // padded position of this block's first row
    const int c0 = blockIdx.x * TOK_COLS;
    // the block's expert e, its first padded position P and (for rpanel) its first 256-row
    // block MT among all experts' row blocks
    int e = -1, P = 0, MT = 0, run = 0, run2 = 0;
    for (int base = 0; base < E && e < 0; base += 64) {
        const int x = base + lane;
        int v = 0, v2 = 0;
        if (x < E) {
            const int lo = min(max(offsets[x], 0), R);
            const int hi = min(max(offsets[x + 1], lo), R);
            v = (hi - lo + TOK_PAD - 1) / TOK_PAD * TOK_PAD;
            v2 = (hi - lo + 255) / 256;
        }
        const int inc = wave_incl_scan(v) + run;
        const int inc2 = wave_incl_scan(v2) + run2;
        const uint64_t m = __ballot(x < E && inc > p);
        if (m) {
            const int l = __ffsll((unsigned long long)m) - 1;
            e = base + l;
            P = __shfl(inc - v, l, 64);
            MT = __shfl(inc2 - v2, l, 64);
        }
        run = __shfl(inc, 63, 64);
        run2 = __shfl(inc2, 63, 64);
    }
    int lo = 0, cnt = 0;
    if (e >= 0) {
        lo = min(max(offsets[e], 0), R);
        cnt = min(max(offsets[e + 1], lo), R) - lo;
    }
    const int t0 = p - P;  // the block's first row within the expert
    if (IN == TOK_IN_BF16) {
        // 1. stage 128 rows x 128 columns: 16 chunks of 8 values per row, 8 per thread
        constexpr int NLD = TOK_PAD * (TOK_COLS / 8) / 256;
        u32x4 v4[NLD];
#pragma unroll
        for (int u = 0; u < NLD; ++u) {
            const int i = tid + 256 * u;
            const int r = i / (TOK_COLS / 8), col = c0 + (i % (TOK_COLS / 8)) * 8;
            v4[u] = (e >= 0 && t0 + r < cnt) ? ld16_nt(X + (int64_t)(lo + t0 + r) * C + col)
                                             : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < NLD; ++u) {
            const int i = tid + 256 * u;
            const int r = i / (TOK_COLS / 8), ch = i % (TOK_COLS / 8);
            *reinterpret_cast<u32x4*>(lds + r * TOK_LD + ch * 16) = v4[u];
        }
    } else if (IN == TOK_IN_PULL) {
        // 1. (dy rows formed here) row lo + t0 + r is bf16(w * dout[s / k]) for its source
        //    (s, w), or zeros: 16 chunks of 8 values per row, 8 per thread.  The row's dout
        //    chunk and the check of s against pos are loaded together, after src.
        constexpr int NLD = TOK_PAD * (TOK_COLS / 8) / 256;
        int2 sw[NLD];
#pragma unroll
        for (int u = 0; u < NLD; ++u) {
            const int i = tid + 256 * u;
            const int r = i / (TOK_COLS / 8);
            sw[u] = (e >= 0 && t0 + r < cnt) ? pull.src[lo + t0 + r] : make_int2(-1, 0);
        }
        int back[NLD];
        u32x4 v4[NLD];
#pragma unroll
        for (int u = 0; u < NLD; ++u) {
            const int i = tid + 256 * u;
            const int col = c0 + (i % (TOK_COLS / 8)) * 8;
            const int sl = sw[u].x;
            const bool in = sl >= 0 && sl < pull.T * pull.k;
            back[u] = in ? pull.pos[sl] : -1;
            v4[u] = in ? ld16(pull.dout + (int64_t)(sl / pull.k) * C + col)
                       : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < NLD; ++u) {
            const int i = tid + 256 * u;
            const int r = i / (TOK_COLS / 8), ch = i % (TOK_COLS / 8);
            const bool ok = back[u] == lo + t0 + r;
            const float wv = ok ? __int_as_float(sw[u].y) : 0.0f;
            u32x4 o;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                o[q] = ok ? pack_bf2(__fmul_rn(wv, lo_bf(v4[u][q])),
                                     __fmul_rn(wv, hi_bf(v4[u][q])))
                          : 0u;
            *reinterpret_cast<u32x4*>(lds + r * TOK_LD + ch * 16) = o;
        }
    } else {
        // 1. (MX input) 128 rows x 128 codes: 8 chunks of 16 codes per row, 4 per thread;
        //    chunk ch of a row lies in the row's 32-code block c0/32 + ch/2
        constexpr int NLD = TOK_PAD * (TOK_COLS / 16) / 256;
        u32x4 q4[NLD];
        int sc4[NLD];
#pragma unroll
        for (int u = 0; u < NLD; ++u) {
            const int i = tid + 256 * u;
            const int r = i / (TOK_COLS / 16), ch = i % (TOK_COLS / 16);
            const bool ok = e >= 0 && t0 + r < cnt;
            const int64_t row = lo + t0 + r;
            q4[u] = ok ? ld16_nt(Xq + row * C + c0 + ch * 16) : u32x4{0u, 0u, 0u, 0u};
            sc4[u] = ok ? (int)Xs[row * (C / 32) + c0 / 32 + ch / 2] : 127;
        }
#pragma unroll
        for (int u = 0; u < NLD; ++u) {
            const int i = tid + 256 * u;
            const int r = i / (TOK_COLS / 16), ch = i % (TOK_COLS / 16);
            const float f = ldexpf(1.0f, sc4[u] - 127);
            uint32_t w8[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)q4[u][q], false);
                const auto b = __builtin_amdgcn_cvt_pk_f32_fp8((int)q4[u][q], true);
                w8[2 * q] = pack_bf2(a[0] * f, a[1] * f);
                w8[2 * q + 1] = pack_bf2(b[0] * f, b[1] * f);
            }
            uint8_t* d = lds + r * TOK_LD + ch * 32;
            *reinterpret_cast<u32x4*>(d) = u32x4{w8[0], w8[1], w8[2], w8[3]};
            *reinterpret_cast<u32x4*>(d + 16) = u32x4{w8[4], w8[5], w8[6], w8[7]};
        }
    }
    __syncthreads();
    // 2a. column pass: rows 32 wid .. +31, columns 2 lane and 2 lane + 1
    uint32_t cq[2][8];
    int csc[2];
    {
        uint32_t pr[32];
#pragma unroll
        for (int i = 0; i < 32; ++i)
            pr[i] = *reinterpret_cast<const uint32_t*>(lds + (wid * 32 + i) * TOK_LD + lane * 4);
        float v[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = lo_bf(pr[i]);
        csc[0] = mx_block(v, MOE_MX_FLOOR, cq[0]);
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = hi_bf(pr[i]);
        csc[1] = mx_block(v, MOE_MX_FLOOR, cq[1]);
    }
    // 2b. row pass: items tid and tid + 256 -> (row it / 4, 32-column block it % 4)
    uint32_t rq[2][8];
    int rsc[2] = {0, 0};
    if (rcodes) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int it = tid + 256 * h, r = it >> 2, b = it & 3;
            float v[32];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const u32x4 w = *reinterpret_cast<const u32x4*>(lds + r * TOK_LD + b * 64 + c * 16);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    v[8 * c + 2 * q] = lo_bf(w[q]);
                    v[8 * c + 2 * q + 1] = hi_bf(w[q]);
                }
            }
            rsc[h] = mx_block(v, MOE_MX_FLOOR, rq[h]);
        }
    }
    __syncthreads();  // every read of the input tile is done: its LDS takes the output images
    // 3. output images: column lines [128][TOK_OL], row lines [128][TOK_OL], column scale
    //    words [128], row scale words [128]
    uint8_t* const col_img = lds;
    uint8_t* const row_img = lds + TOK_PAD * TOK_OL;
    uint8_t* const col_sc = lds + 2 * TOK_PAD * TOK_OL;
    uint8_t* const row_sc = col_sc + 128 * 4;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        uint8_t* d = col_img + (2 * lane + h) * TOK_OL + wid * 32;
        *reinterpret_cast<u32x4*>(d) = u32x4{cq[h][0], cq[h][1], cq[h][2], cq[h][3]};
        *reinterpret_cast<u32x4*>(d + 16) = u32x4{cq[h][4], cq[h][5], cq[h][6], cq[h][7]};
        col_sc[(2 * lane + h) * 4 + wid] = (uint8_t)csc[h];
    }
    if (rcodes) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int it = tid + 256 * h, r = it >> 2, b = it & 3;
            uint8_t* d = row_img + r * TOK_OL + b * 32;
            *reinterpret_cast<u32x4*>(d) = u32x4{rq[h][0], rq[h][1], rq[h][2], rq[h][3]};
            *reinterpret_cast<u32x4*>(d + 16) = u32x4{rq[h][4], rq[h][5], rq[h][6], rq[h][7]};
            row_sc[r * 4 + b] = (uint8_t)rsc[h];
        }
    }
    __syncthreads();
    // 4. whole lines: column c's 128 codes at codes[(c0 + c) Kp + p], row r's 128 codes at
    //    rcodes[(lo + t0 + r) C + c0]; scale words likewise (4-byte aligned: C, Kp and c0, p
    //    are multiples of 128)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int i = tid + 256 * u, ln = i >> 3, ch = i & 7;
        st16(codes + (int64_t)(c0 + ln) * Kp + p + ch * 16,
             *reinterpret_cast<const u32x4*>(col_img + ln * TOK_OL + ch * 16));
    }
    if (tid < 128)
        *reinterpret_cast<uint32_t*>(scales + (int64_t)(c0 + tid) * (Kp / 32) + p / 32) =
            *reinterpret_cast<const uint32_t*>(col_sc + tid * 4);
    if (rcodes) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = tid + 256 * u, ln = i >> 3, ch = i & 7;
            if (e >= 0 && t0 + ln < cnt)
                st16(rcodes + (int64_t)(lo + t0 + ln) * C + c0 + ch * 16,
                     *reinterpret_cast<const u32x4*>(row_img + ln * TOK_OL + ch * 16));
        }
        if (tid < 128 && e >= 0 && t0 + tid < cnt)
            *reinterpret_cast<uint32_t*>(rscales + (int64_t)(lo + t0 + tid) * (C / 32) + c0 / 32) =
                *reinterpret_cast<const uint32_t*>(row_sc + tid * 4);
    }
    // 5. the same scales in the MX GEMMs' panel layout (a run of 512 bytes per 128-row panel
    //    and K step of 128 codes; byte 8 (32 g + l) + 2 t + kk holds the scale of panel row
    //    32 t + l in the step's 32-code block 2 kk + g), gathered from the scale images in LDS
    //    and written as whole words, so that no separate pass lays them out.  A panel whose
    //    256-row block has no rows past this block's gets zeros, as the panels built from
    //    stored scales do for rows outside the operand.
    auto gather4 = [&](const uint8_t* img) {  // run bytes 4 tid .. 4 tid + 3 from [row][blk]
        uint32_t wv = 0;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int j = 4 * tid + x, L = j >> 3, t = (j & 7) >> 1, kk = j & 1;
            wv |= (uint32_t)img[(32 * t + (L & 31)) * 4 + 2 * kk + (L >> 5)] << (8 * x);
        }
        return wv;
    };
    if (cpanel && tid < 128) {
        // token-axis operand: panel row = column c0 + row, K step = position p / 128, block =
        // the 32 positions of wave blk
        uint8_t* run_ = cpanel + ((int64_t)(c0 / 128) * (Kp / 128) + p / 128) * 512;
        *reinterpret_cast<uint32_t*>(run_ + 4 * tid) = gather4(col_sc);
        if (C % 256 == 128 && c0 == C - 128)
            *reinterpret_cast<uint32_t*>(run_ + (int64_t)(Kp / 128) * 512 + 4 * tid) = 0u;
    }
    if (rpanel && rcodes && e >= 0 && tid < 128) {
        // row-wise operand of the dgrad product: panel row = row t0 % 128 + r of the expert's
        // 256-row block MT + t0 / 256, K step = c0 / 128, block = 32-column block b
        const int q = 2 * (MT + t0 / 256) + ((t0 / 128) & 1);
        uint8_t* run_ = rpanel + ((int64_t)q * (C / 128) + c0 / 128) * 512;
        *reinterpret_cast<uint32_t*>(run_ + 4 * tid) = gather4(row_sc);
        if (((t0 / 128) & 1) == 0 && t0 + 128 >= cnt)
            *reinterpret_cast<uint32_t*>(run_ + (int64_t)(C / 128) * 512 + 4 * tid) = 0u;
    }
}

}  // namespace moe

using namespace moe;

// ------------------------------------------------------------------ C ABI
extern "C" int moe_dispatch(const void* x, int T, int H, int k, const int32_t* src,
                            const int32_t* pos, int R, void* xp, uint8_t* xp_codes,
                            uint8_t* xp_scales, void* stream) {
    MOE_REQUIRE(T >= 0 && H >= 8 && H % 8 == 0 && k >= 1 && R >= 0);
    MOE_REQUIRE((xp_codes == nullptr) == (xp_scales == nullptr));
    MOE_REQUIRE(xp || xp_codes);
    if (xp_codes) MOE_REQUIRE(H % 32 == 0);
    MOE_REQUIRE(R == 0 || (x && (src || pos)));
    MOE_REQUIRE(!pos || k <= MAXK);
    if (R == 0 || (pos && T == 0)) return MOE_OK;
    int rc = moe_check_device();
    if (rc) return rc;
    hipStream_t st = (hipStream_t)stream;
    int64_t n_pairs = (int64_t)T * k;
    if (pos) {
        if (xp_codes) {
            const int nc = H / 8;  // 16-byte chunks of a row, one per thread
            dim3 grid((nc + 255) / 256, T);
            MOE_TRACED("dispatch_mx", st,
                       dispatch_mx_tok_kernel<<<grid, 256, 0, st>>>((const bf16_t*)x, H, k, pos, R,
                                                                    (bf16_t*)xp, xp_codes,
                                                                    xp_scales));
        } else {
            MOE_TRACED("dispatch", st,
                       dispatch_tok_kernel<<<T, 128, 0, st>>>((const bf16_t*)x, H, k, pos, R,
                                                              (bf16_t*)xp));
        }
    } else if (xp_codes) {
        int nb = H / 32;
        dim3 grid((nb + 255) / 256, R);
        MOE_TRACED("dispatch_mx", st,
                   dispatch_mx_kernel<<<grid, 256, 0, st>>>((const bf16_t*)x, n_pairs, H, k, src,
                                                             (bf16_t*)xp, xp_codes, xp_scales));
    } else {
        MOE_TRACED("dispatch", st,
                   dispatch_kernel<<<R, 128, 0, st>>>((const bf16_t*)x, n_pairs, H, k, src,
                                                      (bf16_t*)xp));
    }
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

extern "C" int moe_combine(const void* y, const int32_t* pos, const float* w, int T, int k, int H,
                           int R, const void* ys, int S, void* out, void* stream) {
    MOE_REQUIRE(T >= 0 && k >= 1 && k <= MAXK && H >= 8 && H % 8 == 0 && R >= 0 && S >= 0);
    MOE_REQUIRE((S == 0) == (ys == nullptr));
    MOE_REQUIRE(T == 0 || (y && pos && w && out));
    if (T == 0) return MOE_OK;
    int rc = moe_check_device();
    if (rc) return rc;
    hipStream_t st = (hipStream_t)stream;
    const bf16_t *yb = (const bf16_t*)y, *ysb = (const bf16_t*)ys;
    bf16_t* ob = (bf16_t*)out;
#define MOE_COMBINE_CASE(N)                                                                  \
    case N:                                                                                  \
        MOE_TRACED("combine", st,                                                            \
                   combine_kernel<N><<<T, N, 0, st>>>(yb, pos, w, T, k, H, R, ysb, S, ob)); \
        break;
    switch (combine_threads(H)) {
        MOE_COMBINE_CASE(64) MOE_COMBINE_CASE(128) MOE_COMBINE_CASE(192) MOE_COMBINE_CASE(256)
        MOE_COMBINE_CASE(320) MOE_COMBINE_CASE(384) MOE_COMBINE_CASE(448) MOE_COMBINE_CASE(512)
        default: return MOE_EINVAL;
    }
#undef MOE_COMBINE_CASE
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

extern "C" int mx_quantize(const void* in, int in_dtype, int rows, int K, uint8_t* codes,
                           uint8_t* scales, int scale_mode, void* stream) {
    MOE_REQUIRE(rows >= 0 && K >= 32 && K % 32 == 0);
    MOE_REQUIRE(in_dtype == MOE_BF16 || in_dtype == MOE_F32);
    MOE_REQUIRE(scale_mode == MOE_MX_FLOOR || scale_mode == MOE_MX_CEIL);
    MOE_REQUIRE(rows == 0 || (in && codes && scales));
    if (rows == 0) return MOE_OK;
    int rc = moe_check_device();
    if (rc) return rc;
    int64_t nb = (int64_t)rows * (K / 32);
    dim3 grid((unsigned)((nb + 255) / 256));
    hipStream_t st = (hipStream_t)stream;
    MOE_TRACED("mx_quantize", st,
               if (in_dtype == MOE_F32)
                   mx_quantize_kernel<true><<<grid, 256, 0, st>>>(in, nb, scale_mode, codes, scales);
               else
                   mx_quantize_kernel<false><<<grid, 256, 0, st>>>(in, nb, scale_mode, codes, scales));
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

int moe_launch_mx_quantize_tok(const bf16_t* X, const uint8_t* Xq, const uint8_t* Xs,
                               const MoeTokPull* pull, int R, int C, const int32_t* offsets,
                               int E, int Kp, uint8_t* codes, uint8_t* scales, uint8_t* rcodes,
                               uint8_t* rscales, uint8_t* cpanel, uint8_t* rpanel,
                               const char* name, hipStream_t st) {
    if (Kp == 0 || C == 0) return MOE_OK;
    if (C % TOK_COLS != 0 || Kp % TOK_PAD != 0) return MOE_EINVAL;
    const dim3 grid((unsigned)(C / TOK_COLS), (unsigned)(Kp / TOK_PAD));
    const MoeTokPull none{};
    if (Xq) {  // MX codes and scales along C (X unused)
        if (!Xs) return MOE_EINVAL;
        MOE_TRACED(name, st,
                   mx_quantize_tok_kernel<TOK_IN_MX><<<grid, 256, 0, st>>>(
                       nullptr, Xq, Xs, R, C, offsets, E, Kp, codes, scales, rcodes, rscales,
                       cpanel, rpanel, none));
    } else if (pull) {  // dy rows formed from dout and the rows' sources (X unused)
        if (!pull->dout || !pull->src || !pull->pos || pull->k < 1) return MOE_EINVAL;
        MOE_TRACED(name, st,
                   mx_quantize_tok_kernel<TOK_IN_PULL><<<grid, 256, 0, st>>>(
                       nullptr, nullptr, nullptr, R, C, offsets, E, Kp, codes, scales, rcodes,
                       rscales, cpanel, rpanel, *pull));
    } else {
        MOE_TRACED(name, st,
                   mx_quantize_tok_kernel<TOK_IN_BF16><<<grid, 256, 0, st>>>(
                       X, nullptr, nullptr, R, C, offsets, E, Kp, codes, scales, rcodes,
                       rscales, cpanel, rpanel, none));
    }
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

extern "C" int mx_quantize_t(const void* in, int batch, int A, int B, uint8_t* codes,
                             uint8_t* scales, int scale_mode, void* stream) {
    MOE_REQUIRE(batch >= 0 && A >= 32 && A % 32 == 0 && B >= 1 && batch <= 65535);
    MOE_REQUIRE(scale_mode == MOE_MX_FLOOR || scale_mode == MOE_MX_CEIL);
    MOE_REQUIRE(batch == 0 || (in && codes && scales));
    if (batch == 0) return MOE_OK;
    int rc = moe_check_device();
    if (rc) return rc;
    hipStream_t st = (hipStream_t)stream;
    const dim3 grid((unsigned)((B + 255) / 256), (unsigned)(A / 32), (unsigned)batch);
    MOE_TRACED("mx_quantize_t", st,
               mx_quantize_t_kernel<<<grid, 256, 0, st>>>((const bf16_t*)in, A, B, scale_mode,
                                                          codes, scales));
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

int moe_launch_mx_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int K,
                             bf16_t* out, hipStream_t st) {
    const int64_t nb = rows * (K / 32);
    if (nb == 0) return MOE_OK;
    MOE_TRACED("mx_dequantize", st,
               mx_dequantize_kernel<<<(unsigned)((2 * nb + 255) / 256), 256, 0, st>>>(
                   codes, scales, nb, out));
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

extern "C" int mx_dequantize(const uint8_t* codes, const uint8_t* scales, int rows, int K,
                             void* out, void* stream) {
    MOE_REQUIRE(rows >= 0 && K >= 32 && K % 32 == 0);
    MOE_REQUIRE(rows == 0 || (codes && scales && out));
    if (rows == 0) return MOE_OK;
    int rc = moe_check_device();
    if (rc) return rc;
    return moe_launch_mx_dequantize(codes, scales, rows, K, (bf16_t*)out, (hipStream_t)stream);
}

// Internal launchers used by the backward orchestration.
int moe_launch_combine_bwd(const bf16_t* dout, const bf16_t* y, const int32_t* pos, const float* w,
                           int T, int k, int H, int R, bf16_t* dy, int2* src, float* dw,
                           hipStream_t st) {
    if (T == 0) return MOE_OK;
    MOE_TRACED("combine_bwd", st,
               combine_bwd_kernel<<<T, 256, 0, st>>>(dout, y, pos, w, k, H, R, dy, src, dw));
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

// dxs: S arrays of ldT token rows (the caller may point into the middle of them).
int moe_launch_unpermute(const bf16_t* dxp, const int32_t* pos, int T, int k, int H, int R,
                         const bf16_t* dxs, int S, int ldT, bf16_t* dx, hipStream_t st) {
    if (T == 0) return MOE_OK;
#define MOE_UNPERMUTE_CASE(N)                                                               \
    case N:                                                                                 \
        MOE_TRACED("unpermute", st,                                                         \
                   unpermute_kernel<N><<<T, N, 0, st>>>(dxp, pos, T, k, H, R, dxs, S, ldT, dx)); \
        break;
    switch (combine_threads(H)) {
        MOE_UNPERMUTE_CASE(64) MOE_UNPERMUTE_CASE(128) MOE_UNPERMUTE_CASE(192)
        MOE_UNPERMUTE_CASE(256) MOE_UNPERMUTE_CASE(320) MOE_UNPERMUTE_CASE(384)
        MOE_UNPERMUTE_CASE(448) MOE_UNPERMUTE_CASE(512)
        default: return MOE_EINVAL;
    }
#undef MOE_UNPERMUTE_CASE
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

int moe_launch_router_bwd(const int32_t* idx, const float* w, const float* s_sel, const float* dw,
                          const float* logits, int T, int E, int k, int score, int renorm, float c,
                          float* dL, hipStream_t st) {
    if (T == 0) return MOE_OK;
    MOE_TRACED("router_bwd", st,
               router_bwd_kernel<<<(T + 3) / 4, 256, 0, st>>>(idx, w, s_sel, dw, logits, T, E, k,
                                                              score, renorm, c, dL));
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

int moe_launch_mx_quantize_bf16(const bf16_t* in, int64_t rows, int K, uint8_t* codes,
                                uint8_t* scales, const char* name, hipStream_t st) {
    int64_t nb = rows * (K / 32);
    if (nb == 0) return MOE_OK;
    MOE_TRACED(name, st,
               mx_quantize_kernel<false><<<(unsigned)((nb + 255) / 256), 256, 0, st>>>(
                   in, nb, MOE_MX_FLOOR, codes, scales));
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

