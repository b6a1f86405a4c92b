// Routing: router projection, top-k selection (softmax / sigmoid / group-limited), routing
// weights, and the deterministic expert-contiguous permutation (counts, offsets, pos, src).
//
// The pages only name the layer type (pulsen.vercel.app, "Cursor åpner megakernelen…", ¶6:
// DeepSeek-V3-type MoE layers); the routing below is that layer's top-k router.  Every
// integer output is a bit-exact function of the inputs: selection keys are fp32 values
// computed by a fixed recipe and compared as totally ordered keys (ties: lower id first),
// and row positions come from an ordered ballot ranking, never from atomic fetch-add.
#include "common.h"

namespace moe {

// ------------------------------------------------------------------ router projection
// logits[t,e] = sum_h x[t,h] * w[e,h] in fp32, ascending h, from +0.  The bf16 x bf16
// products are exact in fp32, so the sequential order fixes the value bit for bit.
__global__ void router_proj_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ wr,
                                   int T, int H, int E, float* __restrict__ logits) {
    int id = blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= T * E) return;
    int t = id / E, e = id % E;
    const bf16_t* xr = x + (size_t)t * H;
    const bf16_t* wrow = wr + (size_t)e * H;
    float acc = 0.0f;
    for (int h = 0; h < H; ++h) acc = __fadd_rn(acc, __fmul_rn(bf2f(xr[h]), bf2f(wrow[h])));
    logits[id] = acc;
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

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        uint64_t o = __shfl_xor(v, d, 64);
        v = o > v ? o : v;
    }
    return v;
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
__global__ __launch_bounds__(256) void topk_kernel(TopkParams p) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
    if (t >= p.T) return;
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
                    int e = lane + 64 * i;
                    bool in = e < p.E && e / gs == g && !taken_bits[i];
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
        for (int i = 0; i < NV; ++i) {
            int e = lane + 64 * i;
            if (e < p.E && !((keepmask >> (e / gs)) & 1)) key[i] = 0;
        }
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
        lv = __shfl(lv, eb & 63, 64);
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

// Per-chunk expert histogram (integer LDS atomics: the counts do not depend on order).
__global__ __launch_bounds__(256) void count_kernel(const int32_t* __restrict__ idx, int64_t n,
                                                    int E, int32_t* __restrict__ blk) {
    extern __shared__ int hist[];
    for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
    __syncthreads();
    int64_t i = (int64_t)blockIdx.x * CHUNK + threadIdx.x;
    if (threadIdx.x < CHUNK && i < n) {
        int e = idx[i];
        if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) blk[(size_t)blockIdx.x * E + e] = hist[e];
}

// One block: counts[e] = sum over chunks; offsets = exclusive scan over e; blk[c][e]
// becomes the first row of expert e owned by chunk c.  The chunk histograms are staged
// through LDS with coalesced loads when they fit (SCAN_LDS ints), so that the per-expert
// running sums walk LDS instead of a chain of dependent global loads and stores.
constexpr int SCAN_LDS = 32768;  // 128 KB

__global__ __launch_bounds__(1024) void scan_kernel(int32_t* __restrict__ blk, int nchunks, int E,
                                                    int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets) {
    __shared__ int wsum[16];
    __shared__ int exo[1024];    // offsets[e], for the write-back
    __shared__ int hs[SCAN_LDS];  // [nchunks][E] when staged
    const int e = threadIdx.x;
    const int64_t tot = (int64_t)nchunks * E;
    const bool staged = tot <= SCAN_LDS;
    int run = 0;
    if (staged) {
        for (int i = threadIdx.x; i < (int)tot; i += 1024) hs[i] = blk[i];
        __syncthreads();
        if (e < E) {
            for (int c = 0; c < nchunks; ++c) {
                const int v = hs[c * E + e];
                hs[c * E + e] = run;
                run += v;
            }
        }
    } else if (e < E) {
        for (int c = 0; c < nchunks; ++c) {
            const int v = blk[(size_t)c * E + e];
            blk[(size_t)c * E + e] = run;
            run += v;
        }
    }
    if (e < E) counts[e] = run;
    // exclusive scan of run over e (block of 1024 = 16 waves)
    int incl = wave_incl_scan(e < E ? run : 0);
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane == 63) wsum[wid] = incl;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wid; ++w) base += wsum[w];
    const int excl = base + incl - (e < E ? run : 0);
    if (e < E) offsets[e] = excl;
    if (e == E - 1) offsets[E] = excl + run;
    if (E == 0 && e == 0) offsets[0] = 0;
    if (staged) {
        // every thread writes back entries of every expert: publish the offsets in LDS
        if (e < E) exo[e] = excl;
        __syncthreads();
        for (int i = threadIdx.x; i < (int)tot; i += 1024) blk[i] = hs[i] + exo[i % E];
    } else if (e < E) {
        for (int c = 0; c < nchunks; ++c) blk[(size_t)c * E + e] += excl;
    }
}

// One wave per chunk: ranks the chunk's pairs in order.  Pairs with equal expert among
// 64 lanes are found by matching the expert id bit by bit with ballots.
__global__ __launch_bounds__(64) void rank_kernel(const int32_t* __restrict__ idx, int64_t n,
                                                  int E, int nbits,
                                                  const int32_t* __restrict__ blk,
                                                  int32_t* __restrict__ pos,
                                                  int32_t* __restrict__ src) {
    extern __shared__ int cnt[];
    const int lane = threadIdx.x;
    for (int e = lane; e < E; e += 64) cnt[e] = blk[(size_t)blockIdx.x * E + e];
    __syncthreads();
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int g = 0; g < CHUNK / 64; ++g) {
        int64_t i = (int64_t)blockIdx.x * CHUNK + g * 64 + lane;
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
        __syncthreads();
        if (valid) {
            int r = base + before;
            pos[i] = r;
            src[r] = (int32_t)i;
            // the highest lane of each peer group advances the counter
            if ((peers >> lane) == 1ull) cnt[e] = base + __popcll(peers);
        } else if (i < n) {
            pos[i] = -1;
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------ load balancing
// One block: total = sum of counts (integer, so any order gives the same value), then each
// expert's bias moves by gamma against its load (counts[e] * E against total, exact).
__global__ __launch_bounds__(1024) void bias_update_kernel(const int32_t* __restrict__ counts,
                                                           int E, float gamma,
                                                           float* __restrict__ bias) {
    __shared__ long long part[16];
    const int e = threadIdx.x;
    const long long c = e < E ? (long long)counts[e] : 0;
    long long v = c;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
    __syncthreads();
    long long total = 0;
    for (int w = 0; w < 16; ++w) total += part[w];
    if (e < E) {
        const long long scaled = c * E;
        float b = bias[e];
        if (scaled > total) b = __fsub_rn(b, gamma);
        else if (scaled < total) b = __fadd_rn(b, gamma);
        bias[e] = b;
    }
}

}  // namespace moe

using namespace moe;

extern "C" int moe_update_bias(const int32_t* counts, int E, float gamma, float* bias,
                               void* stream) {
    MOE_REQUIRE(E >= 1 && E <= 1024 && counts && bias);
    int rc = moe_check_device();
    if (rc) return rc;
    hipStream_t st = (hipStream_t)stream;
    MOE_TRACED("bias_update", st, bias_update_kernel<<<1, 1024, 0, st>>>(counts, E, gamma, bias));
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

extern "C" size_t moe_route_workspace_size(int T, int k, int E) {
    if (T < 0 || k < 1 || E < 1) return 0;
    int64_t n = (int64_t)T * k;
    int64_t nch = (n + CHUNK - 1) / CHUNK;
    return moe_align256((size_t)nch * E * sizeof(int32_t)) + 256;
}

extern "C" int moe_route(const float* logits, const void* x, const void* w_router, int T, int H,
                         int E, int k, const moe_route_cfg* cfg, const int32_t* idx_in,
                         int32_t* idx, float* w, float* s_sel, int32_t* counts, int32_t* offsets,
                         int32_t* pos, int32_t* src, void* ws, size_t ws_bytes, void* stream) {
    MOE_REQUIRE(T >= 0 && E >= 1 && E <= 1024 && k >= 1 && k <= 64);
    MOE_REQUIRE(counts && offsets && (T == 0 || (pos && src)));
    MOE_REQUIRE((x == nullptr) == (w_router == nullptr));
    int n_groups = 1, topk_groups = 1, per_group = 1;
    if (!idx_in) {
        MOE_REQUIRE(cfg && k <= E);
        MOE_REQUIRE(cfg->score == MOE_SCORE_SOFTMAX || cfg->score == MOE_SCORE_SIGMOID);
        MOE_REQUIRE(T == 0 || (logits && idx && w && s_sel));
        if (w_router) MOE_REQUIRE(H >= 1 && H % 8 == 0);
        n_groups = cfg->n_groups < 1 ? 1 : cfg->n_groups;
        topk_groups = (cfg->topk_groups < 1 || n_groups == 1) ? n_groups : cfg->topk_groups;
        MOE_REQUIRE(n_groups <= 64 && E % n_groups == 0 && topk_groups <= n_groups);
        int gs = E / n_groups;
        per_group = k / topk_groups < 1 ? 1 : k / topk_groups;
        MOE_REQUIRE(per_group <= gs && k <= topk_groups * gs);
    } else {
        MOE_REQUIRE(T == 0 || idx_in);
    }
    int64_t n = (int64_t)T * k;
    MOE_REQUIRE(n <= 0x7FFFFFFF);
    size_t need = moe_route_workspace_size(T, k, E);
    if (!ws || ws_bytes < need) return MOE_EWORKSPACE;
    int rc = moe_check_device();
    if (rc) return rc;
    hipStream_t st = (hipStream_t)stream;
    if (T > 0 && !idx_in) {
        if (w_router) {
            int tot = T * E;
            MOE_TRACED("router_proj", st,
                       router_proj_kernel<<<(tot + 255) / 256, 256, 0, st>>>(
                           (const bf16_t*)x, (const bf16_t*)w_router, T, H, E, (float*)logits));
            MOE_LAUNCH_CHECK();
        }
        TopkParams p{logits, cfg->sel_bias, T, E, k, cfg->score, n_groups, topk_groups,
                     per_group, cfg->renorm, cfg->route_scale, idx, w, s_sel};
        int nv = (E + 63) / 64;
        dim3 grid((T + 3) / 4), block(256);
        MOE_TRACED("topk", st,
                   if (nv <= 1) topk_kernel<1><<<grid, block, 0, st>>>(p);
                   else if (nv <= 2) topk_kernel<2><<<grid, block, 0, st>>>(p);
                   else if (nv <= 4) topk_kernel<4><<<grid, block, 0, st>>>(p);
                   else if (nv <= 8) topk_kernel<8><<<grid, block, 0, st>>>(p);
                   else topk_kernel<16><<<grid, block, 0, st>>>(p));
        MOE_LAUNCH_CHECK();
    }
    const int32_t* ids = idx_in ? idx_in : idx;
    int nch = (int)((n + CHUNK - 1) / CHUNK);
    int32_t* blk = (int32_t*)ws;
    if (nch > 0) {
        MOE_TRACED("perm_count", st,
                   count_kernel<<<nch, 256, E * sizeof(int), st>>>(ids, n, E, blk));
        MOE_LAUNCH_CHECK();
    }
    MOE_TRACED("perm_scan", st, scan_kernel<<<1, 1024, 0, st>>>(blk, nch, E, counts, offsets));
    MOE_LAUNCH_CHECK();
    if (nch > 0) {
        int nbits = 0;
        while ((1 << nbits) < E) ++nbits;
        MOE_TRACED("perm_rank", st,
                   rank_kernel<<<nch, 64, E * sizeof(int), st>>>(ids, n, E, nbits, blk, pos, src));
        MOE_LAUNCH_CHECK();
    }
    return MOE_OK;
}
