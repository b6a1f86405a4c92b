// Routing: router projection, top-k selection (softmax / sigmoid / group-limited), routing
// weights, and the deterministic expert-contiguous permutation (counts, offsets, pos, src).
//
// The pages only name the layer type (pulsen.vercel.app, "Cursor åpner megakernelen…", ¶6:
// DeepSeek-V3-type MoE layers); the routing below is that layer's top-k router.  Every
// integer output is a bit-exact function of the inputs: selection keys are fp32 values
// computed by a fixed recipe and compared as totally ordered keys (ties: lower id first),
// and row positions come from an ordered ballot ranking, never from atomic fetch-add.
#include <mutex>

#include "route_dev.h"

namespace moe {

// Scratch of moe_route_noalloc: the chunk histograms of the permutation, in a file-scope
// device array instead of a caller's workspace.  Each device the library runs on holds its
// own copy until the process ends.  Host code never passes the array's name to a kernel
// (on the host it is only a stand-in for the symbol): it uses the device address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[MOE_ROUTE_NOALLOC_SCRATCH_BYTES];

// ------------------------------------------------------------------ router projection
__global__ void router_proj_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ wr,
                                   int T, int H, int E, float* __restrict__ logits) {
    int id = blockIdx.x * blockDim.x + threadIdx.x;
    if (id < T * E) router_logit(x, wr, H, E, id, logits);
}

// ------------------------------------------------------------------ kernels of the steps
template <int NV>
__global__ __launch_bounds__(256) void topk_kernel(TopkParams p) {
    const int t = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
    if (t < p.T) topk_token<NV>(p, t, threadIdx.x & 63);
}

__global__ __launch_bounds__(256) void count_kernel(const int32_t* __restrict__ idx, int64_t n,
                                                    int E, int32_t* __restrict__ blk) {
    extern __shared__ int hist[];
    count_chunk(idx, n, E, blk, blockIdx.x, hist);
}

__global__ __launch_bounds__(1024) void scan_kernel(int32_t* __restrict__ blk, int nchunks, int E,
                                                    int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets) {
    __shared__ int exo[1024];
    __shared__ int hs[SCAN_LDS];
    scan_body(blk, nchunks, E, counts, offsets, hs, exo);
}

__global__ __launch_bounds__(64) void rank_kernel(const int32_t* __restrict__ idx, int64_t n,
                                                  int E, int nbits,
                                                  const int32_t* __restrict__ blk,
                                                  int32_t* __restrict__ pos,
                                                  int32_t* __restrict__ src) {
    extern __shared__ int cnt[];
    rank_chunk(idx, n, E, nbits, blk, pos, src, blockIdx.x, cnt);
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

// Argument checks of moe_route (host only, no HIP call); fills the group configuration.
static int route_validate(const float* logits, const void* x, const void* w_router, int T, int H,
                          int E, int k, const moe_route_cfg* cfg, const int32_t* idx_in,
                          const int32_t* idx, const float* w, const float* s_sel,
                          const int32_t* counts, const int32_t* offsets, const int32_t* pos,
                          const int32_t* src, int* n_groups_out, int* topk_groups_out,
                          int* per_group_out) {
    MOE_REQUIRE(T >= 0 && E >= 1 && E <= 1024 && k >= 1 && k <= 64);
    // permutation outputs: none (selection only), counts + offsets (the loads), or all four
    MOE_REQUIRE((counts == nullptr) == (offsets == nullptr) && (pos == nullptr) == (src == nullptr));
    MOE_REQUIRE(!pos || counts);
    MOE_REQUIRE(counts || !idx_in);                       // given ids: nothing but permuting
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
    MOE_REQUIRE((int64_t)T * k <= 0x7FFFFFFF);
    *n_groups_out = n_groups;
    *topk_groups_out = topk_groups;
    *per_group_out = per_group;
    return MOE_OK;
}

// The launches of moe_route, after validation, with a workspace of the needed size.
static int route_launch(const float* logits, const void* x, const void* w_router, int T, int H,
                        int E, int k, const moe_route_cfg* cfg, int n_groups, int topk_groups,
                        int per_group, const int32_t* idx_in, int32_t* idx, float* w,
                        float* s_sel, int32_t* counts, int32_t* offsets, int32_t* pos,
                        int32_t* src, void* ws, hipStream_t st) {
    const int64_t n = (int64_t)T * k;
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
    if (!counts) return MOE_OK;  // selection only
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
    if (nch > 0 && pos) {
        int nbits = 0;
        while ((1 << nbits) < E) ++nbits;
        MOE_TRACED("perm_rank", st,
                   rank_kernel<<<nch, 64, E * sizeof(int), st>>>(ids, n, E, nbits, blk, pos, src));
        MOE_LAUNCH_CHECK();
    }
    return MOE_OK;
}

extern "C" int moe_route(const float* logits, const void* x, const void* w_router, int T, int H,
                         int E, int k, const moe_route_cfg* cfg, const int32_t* idx_in,
                         int32_t* idx, float* w, float* s_sel, int32_t* counts, int32_t* offsets,
                         int32_t* pos, int32_t* src, void* ws, size_t ws_bytes, void* stream) {
    int n_groups, topk_groups, per_group;
    int rc = route_validate(logits, x, w_router, T, H, E, k, cfg, idx_in, idx, w, s_sel, counts,
                            offsets, pos, src, &n_groups, &topk_groups, &per_group);
    if (rc) return rc;
    size_t need = moe_route_workspace_size(T, k, E);
    if (!ws || ws_bytes < need) return MOE_EWORKSPACE;
    rc = moe_check_device();
    if (rc) return rc;
    return route_launch(logits, x, w_router, T, H, E, k, cfg, n_groups, topk_groups, per_group,
                        idx_in, idx, w, s_sel, counts, offsets, pos, src, ws,
                        (hipStream_t)stream);
}

// ------------------------------------------------------------------ no-allocation variant
namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES];  // device address of `scratch` per device (null: not yet)
}  // namespace

// The device address of the current device's `scratch`, looked up once per device (with
// that device current) and kept; null if the lookup fails.
static void* route_scratch_ptr() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

extern "C" int moe_route_noalloc(const float* logits, const void* x, const void* w_router, int T,
                                 int H, int E, int k, const moe_route_cfg* cfg,
                                 const int32_t* idx_in, int32_t* idx, float* w, float* s_sel,
                                 int32_t* counts, int32_t* offsets, int32_t* pos, int32_t* src,
                                 void* stream) {
    // the argument checks of moe_route (no HIP call), then the size limit of the scratch
    int n_groups, topk_groups, per_group;
    int rc = route_validate(logits, x, w_router, T, H, E, k, cfg, idx_in, idx, w, s_sel, counts,
                            offsets, pos, src, &n_groups, &topk_groups, &per_group);
    if (rc) return rc;
    if (moe_route_workspace_size(T, k, E) > (size_t)MOE_ROUTE_NOALLOC_SCRATCH_BYTES)
        return MOE_EWORKSPACE;
    rc = moe_check_device();
    if (rc) return rc;
    void* ws = route_scratch_ptr();
    if (!ws) return MOE_EHIP;
    // Every histogram entry a call reads is written by the same call before (count_kernel
    // writes all [chunks][E] of them): nothing has to start at zero.
    return route_launch(logits, x, w_router, T, H, E, k, cfg, n_groups, topk_groups, per_group,
                        idx_in, idx, w, s_sel, counts, offsets, pos, src, ws,
                        (hipStream_t)stream);
}
