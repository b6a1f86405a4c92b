// Host side of the C ABI: validation, workspace layout and the call sequences of
// moe_expert_ffn and moe_backward.  Every call only enqueues kernels on the caller's stream.
#include <string.h>

#include <vector>

#include "common.h"

using moe::bf16_t;

int moe_ffn_bf16(const bf16_t* xp, const int32_t* offsets, int E, int R, int H, int I,
                 const bf16_t* w1, const bf16_t* w2, bf16_t* gu, bf16_t* h, bf16_t* y,
                 hipStream_t st);
int64_t moe_ffn_row_blocks(int E, int R, bool shared);
size_t moe_ffn_sync_bytes(int E, int R, bool shared);
size_t moe_ffn_error_word();
int moe_ffn_bf16_queue(const bf16_t* xp, const int32_t* offsets, int E, int R, int H, int I,
                       const bf16_t* w1, const bf16_t* w2, bf16_t* gu, bf16_t* h, bf16_t* y,
                       unsigned* sy, hipStream_t st);
int moe_ffn_bwd_bf16(const bf16_t* xp, const int32_t* offsets, int E, int R, int H, int I,
                     const bf16_t* w1, const bf16_t* w2, const bf16_t* gu, const bf16_t* h,
                     const bf16_t* dy, bf16_t* dgu, bf16_t* dxp, const MoeWgradSpan* wg,
                     hipStream_t st);
int moe_ffn_mx(const uint8_t* xq, const uint8_t* xs, const int32_t* offsets, int E, int R, int H,
               int I, const uint8_t* w1q, const uint8_t* w1s, const uint8_t* w2q,
               const uint8_t* w2s, uint8_t* hq, uint8_t* hs, uint8_t* panels,
               bf16_t* gu_save, bf16_t* h_save, bf16_t* y, hipStream_t st);
size_t moe_ffn_bwd_mx_bytes(int E, int R, int H, int I, bool wgrad);
int moe_ffn_bwd_mx(const int32_t* offsets, int E, int R, int H, int I, const uint8_t* w1tq,
                   const uint8_t* w1ts, const uint8_t* w2tq, const uint8_t* w2ts,
                   const bf16_t* gu, const bf16_t* dy, const MoeTokPull* dy_pull, bf16_t* dgu,
                   bf16_t* dxp, const bf16_t* h, const bf16_t* xp, const uint8_t* xq,
                   const uint8_t* xs, bf16_t* dw1, bf16_t* dw2, uint8_t* ws, hipStream_t st);
int moe_ffn_wgrad_bf16(const MoeWgradSpan* wg, int E, int H, int I, hipStream_t st);
size_t moe_mx_panel_bytes(int E, int R, int H, int I, bool shared);
int moe_launch_combine_bwd(const bf16_t* dout, const bf16_t* y, const int32_t* pos, const float* w,
                           int T, int k, int H, int R, bf16_t* dy, int2* src, float* dw,
                           hipStream_t st);
int moe_launch_unpermute(const bf16_t* dxp, const int32_t* pos, int T, int k, int H, int R,
                         const bf16_t* dxs, int S, int ldT, bf16_t* dx, hipStream_t st);
int moe_launch_router_bwd(const int32_t* idx, const float* w, const float* s_sel, const float* dw,
                          const float* logits, int T, int E, int k, int score, int renorm, float c,
                          float* dL, hipStream_t st);

int moe_check_device() {
    static int cached[64];  // 0 unknown, 1 ok, 2 unsupported
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_EHIP;
    if (dev < 0 || dev >= 64) return MOE_EUNSUPPORTED;
    if (cached[dev] == 0) {
        hipDeviceProp_t p;
        if (hipGetDeviceProperties(&p, dev) != hipSuccess) return MOE_EHIP;
        cached[dev] = strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    }
    return cached[dev] == 1 ? MOE_OK : MOE_EUNSUPPORTED;
}

extern "C" int moe_abi_version(void) { return MOE_ABI_VERSION; }

// ---------------------------------------------------------------------- launch tracing
// Per host thread: a pool of event pairs (created once, reused), the number of launches
// recorded since moe_trace_begin, and whether tracing is armed.  Off by default, so the
// calls cost one thread-local flag test when nobody traces.
namespace {
struct TraceRec {
    const char* name;
    hipEvent_t a, b;
};
struct TraceState {
    std::vector<TraceRec> recs;
    int cap = 0, n = 0;
    bool on = false, pending = false;
};
thread_local TraceState g_trace;
}  // namespace

void moe_trace_pre(hipStream_t st) {
    TraceState& t = g_trace;
    t.pending = false;
    if (!t.on || t.n >= t.cap) return;
    if (hipEventRecord(t.recs[t.n].a, st) == hipSuccess) t.pending = true;
}

void moe_trace_post(const char* name, hipStream_t st) {
    TraceState& t = g_trace;
    if (!t.pending) return;
    t.pending = false;
    if (hipEventRecord(t.recs[t.n].b, st) != hipSuccess) return;
    t.recs[t.n].name = name;
    ++t.n;
}

extern "C" int moe_trace_begin(int cap) {
    if (cap < 1 || cap > (1 << 20)) return MOE_EINVAL;
    TraceState& t = g_trace;
    while ((int)t.recs.size() < cap) {
        TraceRec r{"", nullptr, nullptr};
        if (hipEventCreate(&r.a) != hipSuccess) return MOE_EHIP;
        if (hipEventCreate(&r.b) != hipSuccess) {
            (void)hipEventDestroy(r.a);
            return MOE_EHIP;
        }
        t.recs.push_back(r);
    }
    t.cap = cap;
    t.n = 0;
    t.on = true;
    return MOE_OK;
}

extern "C" int moe_trace_end(void) {
    g_trace.on = false;
    return g_trace.n;
}

extern "C" int moe_trace_get(int i, const char** name, float* ms) {
    TraceState& t = g_trace;
    if (i < 0 || i >= t.n || !name || !ms) return MOE_EINVAL;
    if (hipEventSynchronize(t.recs[i].b) != hipSuccess) return MOE_EHIP;
    if (hipEventElapsedTime(ms, t.recs[i].a, t.recs[i].b) != hipSuccess) return MOE_EHIP;
    *name = t.recs[i].name;
    return MOE_OK;
}

extern "C" const char* moe_strerror(int code) {
    switch (code) {
        case MOE_OK: return "ok";
        case MOE_EINVAL: return "invalid argument";
        case MOE_EWORKSPACE: return "workspace missing or too small";
        case MOE_EHIP: return "HIP launch failed";
        case MOE_EUNSUPPORTED: return "device is not gfx950";
        default: return "unknown error";
    }
}

// ---------------------------------------------------------------------- expert FFN
extern "C" size_t moe_ffn_workspace_size(int dtype, int E, int R, int H, int I, int shared) {
    if (E < 1 || R < 0 || H < 1 || I < 1) return 0;
    size_t rows = shared ? (size_t)E * R : (size_t)R;
    if (dtype == MOE_MXFP8)
        return moe_align256(rows * I) + moe_align256(rows * (I / 32)) +
               moe_mx_panel_bytes(E, R, H, I, shared != 0) + 256;
    // BF16: the synchronisation words of the one-launch queue, then room for h
    return moe_ffn_sync_bytes(E, R, shared != 0) + moe_align256(rows * I * 2) + 256;
}

extern "C" size_t moe_ffn_error_offset(void) { return moe_ffn_error_word(); }

extern "C" int moe_expert_ffn(int dtype, const void* xp, const uint8_t* xp_scales,
                              const int32_t* offsets, int E, int R, int H, int I, const void* w1,
                              const uint8_t* w1_scales, const void* w2, const uint8_t* w2_scales,
                              void* gu_save, void* h_save, void* y, void* ws, size_t ws_bytes,
                              void* stream) {
    MOE_REQUIRE(dtype == MOE_BF16 || dtype == MOE_MXFP8);
    MOE_REQUIRE(E >= 1 && R >= 0 && H >= 64 && H % 64 == 0 && I >= 64 && I % 64 == 0);
    MOE_REQUIRE(E <= 1024);
    MOE_REQUIRE((int64_t)R * H < (1ll << 31) && (int64_t)R * 2 * I < (1ll << 31));
    MOE_REQUIRE(xp && w1 && w2 && y);
    if (dtype == MOE_MXFP8) {
        MOE_REQUIRE(xp_scales && w1_scales && w2_scales && H % 128 == 0 && I % 128 == 0);
    } else {
        MOE_REQUIRE(!xp_scales && !w1_scales && !w2_scales);
    }
    size_t need = moe_ffn_workspace_size(dtype, E, R, H, I, offsets == nullptr);
    const bool have_ws = ws && ws_bytes >= need;
    const bool need_ws = dtype == MOE_MXFP8 || h_save == nullptr;
    if (need_ws && !have_ws) return MOE_EWORKSPACE;
    if (R == 0) return MOE_OK;
    int rc = moe_check_device();
    if (rc) return rc;
    hipStream_t st = (hipStream_t)stream;
    size_t rows = offsets ? (size_t)R : (size_t)E * R;
    if (dtype == MOE_BF16) {
        // With a workspace both products run as one launch (the tile queue): GEMM2 tiles
        // fill the last round of GEMM1 tiles.  Every GEMM1 tile writes its XCD's L2 back
        // before it counts itself done; the g|u save goes out with whole-line non-temporal
        // stores, so that flush carries only h (1.28 against 1.32 ms for two launches at
        // the EP-64 share, with the save).  Without a workspace (h_save given): two launches.
        // h: the caller's save, else the workspace after the synchronisation words (a
        // workspace is there whenever h_save is not: checked above)
        const size_t sync = moe_ffn_sync_bytes(E, R, offsets == nullptr);
        bf16_t* h = h_save ? (bf16_t*)h_save : (bf16_t*)((char*)ws + sync);
        if (!have_ws)
            return moe_ffn_bf16((const bf16_t*)xp, offsets, E, R, H, I, (const bf16_t*)w1,
                                (const bf16_t*)w2, (bf16_t*)gu_save, h, (bf16_t*)y, st);
        return moe_ffn_bf16_queue((const bf16_t*)xp, offsets, E, R, H, I, (const bf16_t*)w1,
                                  (const bf16_t*)w2, (bf16_t*)gu_save, h, (bf16_t*)y,
                                  (unsigned*)ws, st);
    }
    char* p = (char*)ws;
    uint8_t* hq = (uint8_t*)p;
    p += moe_align256(rows * I);
    uint8_t* hs = (uint8_t*)p;
    p += moe_align256(rows * (I / 32));
    uint8_t* panels = (uint8_t*)p;
    return moe_ffn_mx((const uint8_t*)xp, xp_scales, offsets, E, R, H, I, (const uint8_t*)w1,
                      w1_scales, (const uint8_t*)w2, w2_scales, hq, hs, panels,
                      (bf16_t*)gu_save, (bf16_t*)h_save, (bf16_t*)y, st);
}

// ---------------------------------------------------------------------- backward
namespace {
struct BwdLayout {
    size_t dy, dgu, dxp, dgus, dxs, mx, total;
};
BwdLayout bwd_layout(const moe_bwd_args* a) {
    BwdLayout L;
    size_t o = 0;
    L.dy = o;   o += moe_align256((size_t)a->R * a->H * 2);
    L.dgu = o;  o += moe_align256((size_t)a->R * 2 * a->I * 2);
    L.dxp = o;  o += moe_align256((size_t)a->R * a->H * 2);
    L.dgus = o; o += moe_align256((size_t)a->S * a->T * 2 * a->Is * 2);
    L.dxs = o;  o += moe_align256((size_t)a->S * a->T * a->H * 2);
    L.mx = o;
    if (a->mx) o += moe_align256(moe_ffn_bwd_mx_bytes(a->E, a->R, a->H, a->I, a->mx == 2));
    L.total = o + 256;
    return L;
}
}  // namespace

extern "C" size_t moe_backward_workspace_size(const moe_bwd_args* a) {
    if (!a || a->R < 0 || a->T < 0 || a->H < 1 || a->I < 1 || a->S < 0) return 0;
    return bwd_layout(a).total;
}

extern "C" int moe_backward(const moe_bwd_args* a, void* ws, size_t ws_bytes, void* stream) {
    MOE_REQUIRE(a);
    MOE_REQUIRE(a->T >= 0 && a->R >= 0 && a->E >= 1 && a->E <= 1024 && a->k >= 1 && a->k <= 64);
    MOE_REQUIRE(a->H >= 64 && a->H % 64 == 0 && a->I >= 64 && a->I % 64 == 0);
    MOE_REQUIRE(a->S >= 0 && (a->S == 0 || (a->Is >= 64 && a->Is % 64 == 0)));
    MOE_REQUIRE(a->E_router >= 1 && a->E_router <= 1024);
    MOE_REQUIRE(a->score == MOE_SCORE_SOFTMAX || a->score == MOE_SCORE_SIGMOID);
    MOE_REQUIRE((int64_t)a->R * a->H < (1ll << 31) && (int64_t)a->T * a->H < (1ll << 31));
    const int passes = a->passes < 1 ? 1 : a->passes;
    if (passes > 1) {
        // every pass but the last holds exactly pass_tokens tokens; R spans all pass regions
        MOE_REQUIRE(a->pass_tokens >= 1 && a->pass_rows >= 0 && passes <= 4096);
        MOE_REQUIRE((int64_t)passes * a->pass_rows == a->R);
        MOE_REQUIRE((int64_t)(passes - 1) * a->pass_tokens < a->T &&
                    a->T <= (int64_t)passes * a->pass_tokens);
        MOE_REQUIRE((int64_t)a->pass_tokens * a->k <= a->pass_rows);
    }
    MOE_REQUIRE(a->mx >= 0 && a->mx <= 2);
    if (a->mx) {  // MXFP8 products: one pass, K steps of 128 codes
        MOE_REQUIRE(passes == 1 && a->H % 128 == 0 && a->I % 128 == 0);
        MOE_REQUIRE(a->T == 0 || (a->w1t_codes && a->w1t_scales && a->w2t_codes && a->w2t_scales));
    }
    const bool xp_as_codes = a->mx == 2 && a->xp_codes && a->xp_scales;
    if (a->T > 0) {
        MOE_REQUIRE((a->xp || xp_as_codes) && a->gu && a->h && a->y && a->offsets && a->pos && a->idx && a->w &&
                    a->s_sel && a->w1 && a->w2 && a->dout && a->dx && a->dw1 && a->dw2 &&
                    a->dw_route && a->dlogits);
        if (a->score == MOE_SCORE_SOFTMAX && !a->renorm) MOE_REQUIRE(a->logits);
        if (a->S > 0)
            MOE_REQUIRE(a->x && a->gus && a->hs && a->ws1 && a->ws2 && a->dws1 && a->dws2);
    }
    BwdLayout L = bwd_layout(a);
    if (!ws || ws_bytes < L.total) return MOE_EWORKSPACE;
    if (a->T == 0) return MOE_OK;
    int rc = moe_check_device();
    if (rc) return rc;
    hipStream_t st = (hipStream_t)stream;
    char* base = (char*)ws;
    bf16_t* dy = (bf16_t*)(base + L.dy);
    bf16_t* dgu = (bf16_t*)(base + L.dgu);
    bf16_t* dxp = (bf16_t*)(base + L.dxp);
    bf16_t* dgus = (bf16_t*)(base + L.dgus);
    bf16_t* dxs = (bf16_t*)(base + L.dxs);
    const int H = a->H, I = a->I, k = a->k, E = a->E;
    // shared experts: gradient dout with weight one, input x, every expert takes all T rows
    if (a->S > 0) {
        MoeWgradSpan sw{(const bf16_t*)a->x, (const bf16_t*)a->hs, (const bf16_t*)a->dout, dgus,
                        nullptr, 1, 0, a->T, (bf16_t*)a->dws1, (bf16_t*)a->dws2};
        rc = moe_ffn_bwd_bf16((const bf16_t*)a->x, nullptr, a->S, a->T, H, a->Is,
                              (const bf16_t*)a->ws1, (const bf16_t*)a->ws2, (const bf16_t*)a->gus,
                              (const bf16_t*)a->hs, (const bf16_t*)a->dout, dgus, dxs, &sw, st);
        if (rc) return rc;
    }
    // routed experts, one pass at a time (a macrobatch walked in passes keeps each pass's
    // rows in its own region); the weight gradients over every pass run with the last pass
    const int prow = passes > 1 ? a->pass_rows : a->R;
    const int ptok = passes > 1 ? a->pass_tokens : a->T;
    MoeWgradSpan wg{(const bf16_t*)a->xp, (const bf16_t*)a->h, dy, dgu, a->offsets, passes,
                    passes > 1 ? a->pass_rows : 0, a->R, (bf16_t*)a->dw1, (bf16_t*)a->dw2};
    for (int p = 0; p < passes; ++p) {
        const int t0 = p * ptok, Tp = min(ptok, a->T - t0);
        const size_t r0 = (size_t)p * prow;
        const bf16_t* dout_p = (const bf16_t*)a->dout + (size_t)t0 * H;
        const int32_t* pos_p = a->pos + (size_t)t0 * k;
        // combine backward: dy rows of the pass and the routing-weight gradient of its tokens.
        // With MXFP8 weight gradients (one pass) dy is only ever read by its quantiser, which
        // then forms the rows itself from dout and each row's source slot and weight (written
        // in dy's place).
        const bool mxw = a->mx == 2;
        int2* src = mxw ? (int2*)dy : nullptr;
        const MoeTokPull pull{dout_p, src, pos_p, Tp, k};
        rc = moe_launch_combine_bwd(dout_p, (const bf16_t*)a->y + r0 * H, pos_p,
                                    a->w + (size_t)t0 * k, Tp, k, H, prow,
                                    mxw ? nullptr : dy + r0 * H, src,
                                    a->dw_route + (size_t)t0 * k, st);
        if (rc) return rc;
        if (prow > 0 && a->mx) {
            rc = moe_ffn_bwd_mx(a->offsets, E, prow, H, I, a->w1t_codes, a->w1t_scales,
                                a->w2t_codes, a->w2t_scales, (const bf16_t*)a->gu,
                                mxw ? nullptr : dy, mxw ? &pull : nullptr, dgu, dxp,
                                (const bf16_t*)a->h, (const bf16_t*)a->xp,
                                xp_as_codes ? a->xp_codes : nullptr,
                                xp_as_codes ? a->xp_scales : nullptr,
                                mxw ? (bf16_t*)a->dw1 : nullptr, mxw ? (bf16_t*)a->dw2 : nullptr,
                                (uint8_t*)(base + L.mx), st);
            if (rc) return rc;
            if (!mxw) {
                rc = moe_ffn_wgrad_bf16(&wg, E, H, I, st);
                if (rc) return rc;
            }
        } else if (prow > 0) {
            rc = moe_ffn_bwd_bf16((const bf16_t*)a->xp + r0 * H, a->offsets + (size_t)p * (E + 1),
                                  E, prow, H, I, (const bf16_t*)a->w1, (const bf16_t*)a->w2,
                                  (const bf16_t*)a->gu + r0 * 2 * I, (const bf16_t*)a->h + r0 * I,
                                  dy + r0 * H, dgu + r0 * 2 * I, dxp + r0 * H,
                                  p == passes - 1 ? &wg : nullptr, st);
            if (rc) return rc;
        }
        rc = moe_launch_unpermute(dxp + r0 * H, pos_p, Tp, k, H, prow,
                                  a->S ? dxs + (size_t)t0 * H : nullptr, a->S, a->T,
                                  (bf16_t*)a->dx + (size_t)t0 * H, st);
        if (rc) return rc;
    }
    return moe_launch_router_bwd(a->idx, a->w, a->s_sel, a->dw_route, a->logits, a->T, a->E_router,
                                 a->k, a->score, a->renorm, a->route_scale, a->dlogits, st);
}
