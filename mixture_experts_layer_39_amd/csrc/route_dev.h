// Device bodies of the routing steps (top-k selection and weights, and the expert-contiguous
// permutation), shared by the per-step kernels of route.hip and the single-launch layer.
// See route.hip for what each step computes and why it is bit-exact.
#pragma once

#include "common.h"

namespace moe {

// This wave's LDS operations complete (s_waitcnt lgkmcnt(0)) before it goes on.
__device__ __forceinline__ void lds_wave_sync() {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_wave_barrier();
}

// ------------------------------------------------------------------ sigmoid key
// Fixed fp32 recipe (IEEE operations rounded to nearest even, no contraction), so keys are
// reproducible on any IEEE machine:  clamp x to [-40,40], z = -x;  n = rint(z*log2 e);
// r = (z - n*C1) - n*C2 with C1 = ln 2 cut to 12 significant bits (n*C1 exact) and
// C2 = fp32(ln 2 - C1) (Cody & Waite reduction);  p = degree-7 Taylor polynomial of e^r in
// Horner form with fp32(1/j!) coefficients;  s = 1 / (1 + p*2^n).
__device__ __forceinline__ float rsig(float x) {
    const float C1 = 0x1.62ep-1f;          // floor(ln2 * 2^12) / 2^12
    const float C2 = 0x1.0bfbe8p-15f;      // fp32(ln2 - C1)
    const float L2E = 0x1.715476p+0f;      // fp32(log2 e)
    float xc = fminf(fmaxf(x, -40.0f), 40.0f);
    float z = -xc;
    float n = rintf(__fmul_rn(z, L2E));
    float r = __fsub_rn(__fsub_rn(z, __fmul_rn(n, C1)), __fmul_rn(n, C2));
    float p = 0x1.a01a02p-13f;                        // fp32(1/5040)
    p = __fadd_rn(0x1.6c16c2p-10f, __fmul_rn(r, p));  // fp32(1/720)
    p = __fadd_rn(0x1.111112p-7f, __fmul_rn(r, p));   // fp32(1/120)
    p = __fadd_rn(0x1.555556p-5f, __fmul_rn(r, p));   // fp32(1/24)
    p = __fadd_rn(0x1.555556p-3f, __fmul_rn(r, p));   // fp32(1/6)
    p = __fadd_rn(0.5f, __fmul_rn(r, p));
    p = __fadd_rn(1.0f, __fmul_rn(r, p));
    p = __fadd_rn(1.0f, __fmul_rn(r, p));
    float eps = ldexpf(p, (int)n);
    return __fdiv_rn(1.0f, __fadd_rn(1.0f, eps));
}

// Total order on (key desc, id asc) packed in 64 bits; 0 = "no candidate".
__device__ __forceinline__ uint64_t pack_key(float k, int id) {
    uint32_t u = __float_as_uint(__fadd_rn(k, 0.0f));  // -0 -> +0
    uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)o << 32) | (uint32_t)(0xFFFFu - (uint32_t)id);
}
__device__ __forceinline__ int key_id(uint64_t p) { return (int)(0xFFFFu - (uint32_t)(p & 0xFFFFu)); }

// Maximum over the wave's 64 lanes (every lane active), returned wave-uniform.  Within each
// row of 16 lanes by DPP moves (quad swaps of 1 and 2 lanes, then the half-row and row
// mirrors: each step pairs groups that already hold their own maxima), then the four rows'
// maxima through readlane.  DPP moves take a few cycles where the LDS permutes of a shuffle
// butterfly take about a hundred each, and the top-k chains dozens of these reductions.
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
    return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}
__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t lane_u64(uint64_t v, int l) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    v = max_u64(v, dpp_u64<0xB1>(v));   // quad_perm [1,0,3,2]
    v = max_u64(v, dpp_u64<0x4E>(v));   // quad_perm [2,3,0,1]
    v = max_u64(v, dpp_u64<0x141>(v));  // row_half_mirror
    v = max_u64(v, dpp_u64<0x140>(v));  // row_mirror
    return max_u64(max_u64(lane_u64(v, 0), lane_u64(v, 16)),
                   max_u64(lane_u64(v, 32), lane_u64(v, 48)));
}

// Fixed-order wave sum (butterfly): every lane ends with the same bits.
__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) v = __fadd_rn(v, __shfl_xor(v, d, 64));
    return v;
}
__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) v = fmaxf(v, __shfl_xor(v, d, 64));
    return v;
}

// Router logit `id` = t*E + e: sum_h x[t,h] * w[e,h] in fp32, ascending h, from +0.  The
// bf16 x bf16 products are exact in fp32, so the sequential order fixes the value bit for bit.
// With 16-byte aligned rows (H % 8 == 0) the operands come 8 values per load, four loads of
// each row in flight, and are summed in the same ascending order.
__device__ __forceinline__ void router_logit(const bf16_t* __restrict__ x,
                                             const bf16_t* __restrict__ wr, int H, int E, int id,
                                             float* __restrict__ logits) {
    const int t = id / E, e = id % E;
    const bf16_t* xr = x + (size_t)t * H;
    const bf16_t* wrow = wr + (size_t)e * H;
    float acc = 0.0f;
    int h = 0;
    if (H % 8 == 0 && ((reinterpret_cast<uintptr_t>(xr) | reinterpret_cast<uintptr_t>(wrow)) & 15) == 0) {
        constexpr int U = 4;  // 16-byte chunks of each row per batch
        for (; h + 8 * U <= H; h += 8 * U) {
            u32x4 xv[U], wv[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                xv[u] = ld16(xr + h + 8 * u);
                wv[u] = ld16(wrow + h + 8 * u);
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc = __fadd_rn(acc, __fmul_rn(lo_bf(xv[u][q]), lo_bf(wv[u][q])));
                    acc = __fadd_rn(acc, __fmul_rn(hi_bf(xv[u][q]), hi_bf(wv[u][q])));
                }
        }
    }
    for (; h < H; ++h) acc = __fadd_rn(acc, __fmul_rn(bf2f(xr[h]), bf2f(wrow[h])));
    logits[id] = acc;
}

constexpr int MAX_NV = 16;  // experts per lane: E <= 1024

struct TopkParams {
    const float* logits;
    const float* bias;
    int T, E, k, score, n_groups, topk_groups, per_group, renorm;
    float route_scale;
    int32_t* idx;
    float* w;
    float* s_sel;
};

// One wave per token.  Lane l holds experts e = l + 64*i.
template <int NV>
__device__ __forceinline__ void topk_token(const TopkParams& p, const int t, const int lane) {
    const float* L = p.logits + (size_t)t * p.E;
    float lg[NV];
    uint64_t key[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        int e = lane + 64 * i;
        key[i] = 0;
        lg[i] = 0.0f;
        if (e < p.E) {
            lg[i] = L[e];
            float kk = lg[i];
            if (p.score == MOE_SCORE_SIGMOID) {
                kk = rsig(lg[i]);
                if (p.bias) kk = __fadd_rn(kk, p.bias[e]);
            }
            key[i] = pack_key(kk, e);
        }
    }
    if (p.n_groups > 1) {
        const int gs = p.E / p.n_groups;
        int grp[NV];  // group of each of the lane's experts (-1: none)
#pragma unroll
        for (int i = 0; i < NV; ++i) grp[i] = lane + 64 * i < p.E ? (lane + 64 * i) / gs : -1;
        // group scores: fp32 sum, largest first, of the top per_group keys of each group
        float gscore_mine = 0.0f;  // lane g holds group g's score (n_groups <= 64)
        for (int g = 0; g < p.n_groups; ++g) {
            uint64_t taken_bits[NV];
#pragma unroll
            for (int i = 0; i < NV; ++i) taken_bits[i] = 0;
            float s = 0.0f;
            for (int q = 0; q < p.per_group; ++q) {
                uint64_t best = 0;
#pragma unroll
                for (int i = 0; i < NV; ++i) {
                    bool in = grp[i] == g && !taken_bits[i];
                    uint64_t c = in ? key[i] : 0;
                    best = c > best ? c : best;
                }
                best = wave_max_u64(best);
                int eb = key_id(best);
#pragma unroll
                for (int i = 0; i < NV; ++i)
                    if (lane + 64 * i == eb) taken_bits[i] = 1;
                // recover the key value of the winner
                uint32_t o = (uint32_t)(best >> 32);
                uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
                s = __fadd_rn(s, __uint_as_float(u));
            }
            if (lane == g) gscore_mine = __fadd_rn(s, 0.0f);
        }
        // keep the topk_groups best groups (score desc, group asc)
        uint64_t gk = lane < p.n_groups ? pack_key(gscore_mine, lane) : 0;
        bool keep = false;
        for (int q = 0; q < p.topk_groups; ++q) {
            uint64_t best = wave_max_u64(keep ? 0 : gk);
            if (lane < p.n_groups && key_id(best) == lane) keep = true;
        }
        uint64_t keepmask = __ballot(keep);
#pragma unroll
        for (int i = 0; i < NV; ++i)
            if (grp[i] >= 0 && !((keepmask >> grp[i]) & 1)) key[i] = 0;
    }
    // top-k: k rounds of wave argmax; lane j keeps slot j
    int my_id = 0;
    float my_logit = 0.0f;
    for (int j = 0; j < p.k; ++j) {
        uint64_t best = 0;
#pragma unroll
        for (int i = 0; i < NV; ++i) best = key[i] > best ? key[i] : best;
        best = wave_max_u64(best);
        int eb = key_id(best);
#pragma unroll
        for (int i = 0; i < NV; ++i)
            if (lane + 64 * i == eb) key[i] = 0;
        // the winner's logit, fetched from the owning lane
        float lv = 0.0f;
#pragma unroll
        for (int i = 0; i < NV; ++i)
            if (lane + 64 * i == eb) lv = lg[i];
        lv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lv), eb & 63));
        if (lane == j) { my_id = eb; my_logit = lv; }
    }
    // weights
    const bool act = lane < p.k;
    float s_val, wv;
    if (p.score == MOE_SCORE_SIGMOID) {
        s_val = act ? rsig(my_logit) : 0.0f;
        float tot = wave_sum_f32(s_val);
        wv = p.renorm ? __fdiv_rn(__fmul_rn(p.route_scale, s_val), tot)
                      : __fmul_rn(p.route_scale, s_val);
    } else {
        s_val = my_logit;
        if (p.renorm) {
            float l0 = __shfl(my_logit, 0, 64);  // slot 0 holds the largest logit
            float ex = act ? expf(my_logit - l0) : 0.0f;
            float tot = wave_sum_f32(ex);
            wv = ex / tot;
        } else {
            float m = -INFINITY;
#pragma unroll
            for (int i = 0; i < NV; ++i)
                if (lane + 64 * i < p.E) m = fmaxf(m, lg[i]);
            m = wave_max_f32(m);
            float se = 0.0f;
#pragma unroll
            for (int i = 0; i < NV; ++i)
                if (lane + 64 * i < p.E) se += expf(lg[i] - m);
            se = wave_sum_f32(se);
            wv = expf(my_logit - m) / se;
        }
    }
    if (act) {
        size_t o = (size_t)t * p.k + lane;
        p.idx[o] = my_id;
        p.w[o] = wv;
        p.s_sel[o] = s_val;
    }
}

// ------------------------------------------------------------------ permutation
// Pairs are processed in chunks of CHUNK consecutive (t,j) in token-major order.
constexpr int CHUNK = 256;

// Expert histogram of chunk `c` (integer LDS atomics: the counts do not depend on order).
// The whole block (blockDim.x >= CHUNK threads) works on one chunk; hist holds E ints.
__device__ __forceinline__ void count_chunk(const int32_t* __restrict__ idx, int64_t n, int E,
                                            int32_t* __restrict__ blk, int c, int* hist) {
    for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
    __syncthreads();
    int64_t i = (int64_t)c * CHUNK + threadIdx.x;
    if (threadIdx.x < CHUNK && i < n) {
        int e = idx[i];
        if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) blk[(size_t)c * E + e] = hist[e];
    __syncthreads();  // hist may be reused
}

// One block: counts[e] = sum over chunks; offsets = exclusive scan over e; blk[c][e]
// becomes the first row of expert e owned by chunk c.  The chunk histograms are staged
// through LDS with coalesced loads when they fit (SCAN_LDS ints), so that the per-expert
// running sums walk LDS instead of a chain of dependent global loads and stores.
constexpr int SCAN_LDS = 32768;  // 128 KB

// One block of any size: hs holds SCAN_LDS ints, exo 1024.
__device__ __forceinline__ void scan_body(int32_t* __restrict__ blk, int nchunks, int E,
                                          int32_t* __restrict__ counts,
                                          int32_t* __restrict__ offsets, int* hs, int* exo) {
    const int nt = blockDim.x;
    const int64_t tot = (int64_t)nchunks * E;
    const bool staged = tot <= SCAN_LDS;
    if (staged) {
        for (int i = threadIdx.x; i < (int)tot; i += nt) hs[i] = blk[i];
        __syncthreads();
    }
    // per-expert running sums over the chunks (chunk c's entry becomes its chunk-local base)
    for (int e = threadIdx.x; e < E; e += nt) {
        int run = 0;
        if (staged) {
            for (int c = 0; c < nchunks; ++c) {
                const int v = hs[c * E + e];
                hs[c * E + e] = run;
                run += v;
            }
        } else {
            // 16 chunks' counts are loaded before any is rewritten (independent loads in
            // flight instead of one load-store round trip per chunk)
            for (int c0 = 0; c0 < nchunks; c0 += 16) {
                int v[16];
#pragma unroll
                for (int u = 0; u < 16; ++u)
                    v[u] = c0 + u < nchunks ? blk[(size_t)(c0 + u) * E + e] : 0;
#pragma unroll
                for (int u = 0; u < 16; ++u)
                    if (c0 + u < nchunks) {
                        blk[(size_t)(c0 + u) * E + e] = run;
                        run += v[u];
                    }
            }
        }
        counts[e] = run;
        exo[e] = run;
    }
    __syncthreads();
    // exclusive scan of the totals over e, by the first wave, 64 experts at a time
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        int carry = 0;
        for (int base = 0; base < E; base += 64) {
            const int e = base + lane;
            const int v = e < E ? exo[e] : 0;
            const int inc = wave_incl_scan(v) + carry;
            if (e < E) exo[e] = inc - v;
            carry = __shfl(inc, 63, 64);
        }
        if (lane == 0) offsets[E] = carry;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += nt) offsets[e] = exo[e];
    if (staged) {
        for (int i = threadIdx.x; i < (int)tot; i += nt) blk[i] = hs[i] + exo[i % E];
    } else {  // every entry independently: consecutive threads take consecutive entries
        for (int64_t i = threadIdx.x; i < tot; i += nt) blk[i] += exo[i % E];
    }
    __syncthreads();  // hs / exo may be reused
}

// One wave ranks chunk `c`'s pairs in order.  Pairs with equal expert among 64 lanes are
// found by matching the expert id bit by bit with ballots.  cnt: E ints of this wave's own.
// Only this wave touches cnt, so waiting for its own LDS operations (no block barrier) orders
// the counter updates between groups.
__device__ __forceinline__ void rank_chunk(const int32_t* __restrict__ idx, int64_t n, int E,
                                           int nbits, const int32_t* __restrict__ blk,
                                           int32_t* __restrict__ pos, int32_t* __restrict__ src,
                                           int c, int* cnt) {
    const int lane = threadIdx.x & 63;
    for (int e = lane; e < E; e += 64) cnt[e] = blk[(size_t)c * E + e];
    lds_wave_sync();
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int g = 0; g < CHUNK / 64; ++g) {
        int64_t i = (int64_t)c * CHUNK + g * 64 + lane;
        int e = (i < n) ? idx[i] : -1;
        bool valid = e >= 0 && e < E;
        uint64_t peers = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
            bool bit = valid && ((e >> b) & 1);
            uint64_t bal = __ballot(bit);
            peers &= bit ? bal : ~bal;
        }
        int before = __popcll(peers & lt);
        int base = valid ? cnt[e] : 0;
        lds_wave_sync();
        if (valid) {
            int r = base + before;
            pos[i] = r;
            src[r] = (int32_t)i;
            // the highest lane of each peer group advances the counter
            if ((peers >> lane) == 1ull) cnt[e] = base + __popcll(peers);
        } else if (i < n) {
            pos[i] = -1;
        }
        lds_wave_sync();
    }
}

}  // namespace moe
