/*
 * moe.h -- C ABI of the MI355X (gfx950) deterministic mixture-of-experts layer library.
 *
 * The layer is one GPU's share of a DeepSeek-V3-type MoE layer, the layer type the pages
 * name (pulsen.vercel.app, "Cursor åpner megakernelen som ga 41 prosent flere tokens i
 * sekundet", ¶6), run forward in BF16 or MXFP8 and backward in BF16 (same page, ¶3;
 * aiexpert.news, "Megakernels are dead and back", ¶4), fully deterministic (pulsen ¶3-¶4;
 * ki-pruefstand.de, "Cursor veröffentlicht MoE-Megakernel Mixture-of-Kittens als Open
 * Source", ¶3): repeated calls with the same inputs give bit-identical outputs.  No kernel
 * uses floating-point atomics; every sum runs in one fixed order.
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers owned by the caller unless marked "host".  The library
 *    never allocates, frees or synchronises; scratch memory comes in through `ws`.
 *  - bf16 tensors are raw 16-bit patterns (uint16_t storage), row-major, rows contiguous.
 *  - `stream` is a hipStream_t (NULL: the null stream).  Calls only enqueue work on it and
 *    never read device data back to the host (no CPU-GPU synchronisation; aiexpert.news ¶3,
 *    ki-pruefstand.de "Kommunikation im Kernel" ¶2).  A kernel fault surfaces at the
 *    caller's next synchronisation.
 *  - Arguments are validated on the host before any HIP call; an invalid call returns a
 *    negative code and enqueues nothing.  Device-resident indices (src, pos, offsets) are
 *    clamped by the kernels, so that corrupt indices cannot access memory out of bounds.
 *  - Calls on distinct streams with distinct workspaces may run concurrently; the library
 *    holds no mutable global state apart from the optional, per-thread launch trace below.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 8

/* return codes */
#define MOE_OK 0
#define MOE_EINVAL (-1)        /* invalid argument (null pointer, size, configuration) */
#define MOE_EWORKSPACE (-2)    /* workspace missing or smaller than *_workspace_size() */
#define MOE_EHIP (-3)          /* a HIP launch failed */
#define MOE_EUNSUPPORTED (-4)  /* current device is not gfx950 */

/* router score functions */
#define MOE_SCORE_SOFTMAX 0
#define MOE_SCORE_SIGMOID 1

/* data types */
#define MOE_BF16 0
#define MOE_MXFP8 1   /* E4M3 codes with one E8M0 scale per 32 values along K */
#define MOE_F32 2

/* MX shared-scale rules */
#define MOE_MX_FLOOR 0  /* 2^(floor(log2 amax) - 8); elements above 448 saturate */
#define MOE_MX_CEIL 1   /* smallest power of two keeping amax within 448 */

int moe_abi_version(void);
const char *moe_strerror(int code);

/* ------------------------------------------------------------------ routing
 * Router configuration (host struct, read during the call).
 *   score:        MOE_SCORE_SOFTMAX (selection key = logit) or MOE_SCORE_SIGMOID (key =
 *                 sigmoid(logit) + sel_bias[e]; the sigmoid is a fixed fp32 recipe, see the
 *                 routing kernel, so keys are reproducible bit for bit);
 *   n_groups:     >1: experts form n_groups contiguous groups; a group's score is the sum of
 *                 its top k/topk_groups keys; only the topk_groups best groups stay;
 *   renorm:       softmax: weights renormalised over the k selected experts (else the full
 *                 softmax); sigmoid: w = route_scale * s / sum(selected s) (else route_scale*s);
 *   sel_bias:     DEVICE [E] fp32 added to sigmoid keys for selection only, or NULL.
 * Ties rank the lower expert (group) id first; slot j holds the j-th best expert. */
typedef struct moe_route_cfg {
    int score;
    int n_groups;
    int topk_groups;
    int renorm;
    float route_scale;
    const float *sel_bias;
} moe_route_cfg;

size_t moe_route_workspace_size(int T, int k, int E);

/* moe_route: top-k routing plus the expert-contiguous permutation -- the router of the
 * DeepSeek-V3-type layer the pages name (pulsen.vercel.app, "Cursor åpner megakernelen…",
 * ¶6: sigmoid or softmax scores, optionally group-limited) and the per-expert row order its
 * dispatch needs ("pull": the expert-side rows fetch their tokens, same page ¶5), computed
 * with no host readback (aiexpert.news ¶3) and bit for bit reproducibly (pulsen ¶3-¶4).
 *   logits   [T,E] fp32.  Read; or, when w_router != NULL, first WRITTEN with the router
 *            projection logits[t,e] = sum_h x[t,h]*w_router[e,h], accumulated in fp32 in
 *            ascending h (exact products, so the result is fixed bit for bit).
 *   x        [T,H] bf16 and w_router [E,H] bf16: both NULL, or both given.
 *   idx_in   [T,k] int32 or NULL.  Given: the expert of every routed pair is taken from it
 *            (one GPU's share of a larger layer); selection is skipped and logits, idx, w,
 *            s_sel are not touched (may be NULL).
 *   idx      [T,k] int32  selected experts, slot order = rank order.
 *   w        [T,k] fp32   routing weights.
 *   s_sel    [T,k] fp32   selected scores (sigmoid value, or the logit for softmax).
 *   counts   [E]   int32  routed rows per expert.
 *   offsets  [E+1] int32  exclusive prefix sum of counts (offsets[E] = T*k).
 *   pos      [T,k] int32  row of pair (t,j) in expert-contiguous order; rows of one expert are
 *            in ascending (t,j) order.
 *   src      [T*k] int32  inverse of pos: src[pos[t,j]] = t*k + j.
 *   counts/offsets and pos/src are optional in pairs: all four NULL computes the selection
 *   alone (idx, w, s_sel; not with idx_in); counts and offsets without pos and src compute
 *   the loads but no permutation; pos and src need counts and offsets.
 * Limits: 1 <= k <= min(E, 64), E <= 1024, T >= 0, H % 8 == 0 when projecting.
 * Outputs are bit-exact functions of the inputs. */
int moe_route(const float *logits, const void *x, const void *w_router, int T, int H, int E,
              int k, const moe_route_cfg *cfg, const int32_t *idx_in, int32_t *idx, float *w,
              float *s_sel, int32_t *counts, int32_t *offsets, int32_t *pos, int32_t *src,
              void *ws, size_t ws_bytes, void *stream);

/* moe_route_noalloc: moe_route for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation): the same
 * arguments without ws / ws_bytes, the same kernels and bit-identical outputs.  Its scratch
 * (the permutation's chunk histograms) is a static device array of
 * MOE_ROUTE_NOALLOC_SCRATCH_BYTES that the library holds on each device it runs on until the
 * process ends; the call itself allocates and frees nothing.  Calls whose scratch would not
 * fit -- moe_route_workspace_size(T, k, E) > MOE_ROUTE_NOALLOC_SCRATCH_BYTES, i.e. about
 * ceil(T*k / 256) * E * 4 bytes -- return MOE_EWORKSPACE and enqueue nothing (1 MiB covers,
 * e.g., T*k = 65536 routed pairs over E = 512 experts).  Every call on one device shares
 * that device's array: calls that may overlap on one device (different streams, or different
 * host threads without ordering) race and must be serialised by the caller; stream-ordered
 * calls are safe, since each call writes all the scratch it reads before reading it.
 * Other errors as moe_route; MOE_EHIP if the array's device address cannot be looked up. */
#define MOE_ROUTE_NOALLOC_SCRATCH_BYTES (1u << 20)
int moe_route_noalloc(const float *logits, const void *x, const void *w_router, int T, int H,
                      int E, int k, const moe_route_cfg *cfg, const int32_t *idx_in,
                      int32_t *idx, float *w, float *s_sel, int32_t *counts, int32_t *offsets,
                      int32_t *pos, int32_t *src, void *stream);

/* ------------------------------------------------------------------ load balancing
 * moe_update_bias: the auxiliary-loss-free load balancing of a DeepSeek-V3-type layer
 * (layer type: pulsen.vercel.app ¶6; rule: DeepSeek-V3 Technical Report, arXiv:2412.19437,
 * §2.1.2).  After a step, with load counts[e] (e.g. the counts of moe_route) and the mean
 * load (sum of counts) / E:  bias[e] -= gamma where counts[e] is above the mean,
 * bias[e] += gamma where it is below, unchanged where equal (compared exactly, as
 * counts[e] * E against the sum); each update is one fp32 rounding.
 *   counts  DEVICE [E] int32 (non-negative), bias DEVICE [E] fp32, updated in place (the
 *           sel_bias of moe_route_cfg).  1 <= E <= 1024.  Bit-exact. */
int moe_update_bias(const int32_t *counts, int E, float gamma, float *bias, void *stream);

/* ------------------------------------------------------------------ dispatch
 * moe_dispatch: gather token rows into expert-contiguous order ("pull": the expert-side rows
 * fetch their source, pulsen.vercel.app ¶5): xp[r,:] = x[src[r]/k,:], r in [0,R).
 *   src       [R] (the permutation of moe_route), or NULL when pos is given.
 *   pos       [T,k] (the inverse permutation of moe_route), or NULL.  When given, each token's
 *             k destination rows are filled together from one read of its source row (the
 *             source is read once instead of k times): xp[pos[t,j],:] = x[t,:] for every
 *             pos[t,j] in [0,R); rows that no pos entry names are left unwritten.  When NULL,
 *             every row r in [0,R) is written from src, and src values outside [0, T*k)
 *             produce zero rows.
 *   xp        [R,H] bf16 or NULL: bf16 copy (bit-exact).
 *   xp_codes  [R,H] E4M3 and xp_scales [R,H/32] E8M0, or both NULL: the rows MX-quantised
 *             (MOE_MX_FLOOR) in the same pass.  At least one output must be given.
 * H % 8 == 0 (H % 32 == 0 for MX); k <= 64 when pos is given. */
int moe_dispatch(const void *x, int T, int H, int k, const int32_t *src, const int32_t *pos,
                 int R, void *xp, uint8_t *xp_codes, uint8_t *xp_scales, void *stream);

/* ------------------------------------------------------------------ expert FFN
 * moe_expert_ffn: the experts of the DeepSeek-V3-type layer (pulsen.vercel.app ¶6) as
 * grouped GEMMs, in BF16 or MXFP8 (the two forward precisions the pages report: pulsen ¶3,
 * aiexpert.news ¶4).  Per expert e, for its rows r in [offsets[e], offsets[e+1]):
 *   [g | u] = xp_r . w1[e]^T  (w1[e] is [2I,H]: gate rows 0..I-1 over up rows I..2I-1),
 *   h = silu(g) * u,  y_r = h . w2[e]^T  (w2[e] is [H,I]);  fp32 accumulation.
 * The offsets are read on the device (no host readback); each expert's tile list is derived
 * from them inside the kernels.  offsets == NULL: every one of the E experts takes all R rows
 * (shared experts) and the outputs are stacked per expert: y [E,R,H], gu [E,R,2I], h [E,R,I].
 *   dtype = MOE_BF16:  xp [R,H] bf16, w1/w2 bf16, *_scales NULL.  gu_save [R,2I] bf16 and
 *            h_save [R,I] bf16 are optional saves for the backward (NULL: not written).
 *   dtype = MOE_MXFP8: xp/w1/w2 are E4M3 codes with E8M0 scales per 32 values along their
 *            last (K) dimension: xp_scales [R,H/32], w1_scales [E,2I,H/32], w2_scales
 *            [E,H,I/32].  h is MX-quantised along I from fp32 before the down projection.
 *            Optional saves for the backward: gu_save [R,2I] bf16 (the fp32 pre-activations,
 *            rounded) and h_save [R,I] bf16 (h as the down projection consumes it: the
 *            MX-quantised values, which bf16 holds exactly).  H % 128 == 0, I % 128 == 0.
 *   y [R,H] bf16 (routed rows, expert order).
 * Limits: H % 64 == 0, I % 64 == 0 (both % 128 for MOE_MXFP8), offsets non-decreasing with
 * offsets[E] <= R.
 * Workspace: moe_ffn_workspace_size().  MOE_MXFP8 always needs it.  MOE_BF16 with a workspace
 *   of that size runs both products as ONE launch: a queue of GEMM1 and GEMM2 tiles in which
 *   a GEMM2 tile waits only for the GEMM1 tiles of its own rows (per-row-block counters in
 *   the workspace, cleared by a small kernel before the launch), so the second product
 *   fills the first one's last, partial round.  Without a workspace (h_save given) the two
 *   products run as two launches.  Both forms give bit-identical outputs.  The queue form clears its counters and the uint32 at byte
 *   moe_ffn_error_offset() of the workspace before it starts; a queue wait is bounded (2 s),
 *   and past it that word becomes nonzero and the outputs are not valid.  The two-launch form
 *   does not touch the word.  Calls that share a workspace must be stream-ordered. */
size_t moe_ffn_workspace_size(int dtype, int E, int R, int H, int I, int shared);
size_t moe_ffn_error_offset(void);
int moe_expert_ffn(int dtype, const void *xp, const uint8_t *xp_scales, const int32_t *offsets,
                   int E, int R, int H, int I, const void *w1, const uint8_t *w1_scales,
                   const void *w2, const uint8_t *w2_scales, void *gu_save, void *h_save,
                   void *y, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------ combine
 * moe_combine: out[t,:] = sum_{j<k} w[t,j] * y[pos[t,j],:] + sum_{s<S} ys[s,t,:], summed in
 * fp32 in exactly that order (slots, then shared experts), rounded once to bf16 ("push" of
 * each routed result to its token, pulsen.vercel.app ¶5; weighted combine, no atomics).
 *   y [R,H] bf16, pos [T,k], w [T,k] fp32, ys [S,T,H] bf16 or NULL (S = 0), out [T,H] bf16.
 * pos values outside [0,R) contribute nothing.  H % 8 == 0. */
int moe_combine(const void *y, const int32_t *pos, const float *w, int T, int k, int H, int R,
                const void *ys, int S, void *out, void *stream);

/* ------------------------------------------------------------------ the forward in one launch
 * moe_layer_forward: the whole BF16 forward of the layer -- router projection (optional),
 * top-k routing, the expert-contiguous permutation, dispatch, the routed and shared experts'
 * GEMM1 + SwiGLU and GEMM2, and the weighted combine -- as ONE persistent kernel
 * launch (the single MoE kernel of pulsen.vercel.app ¶3 and ki-pruefstand.de "Kommunikation
 * im Kernel" ¶2, at one GPU): one block per compute unit walks each step's work and
 * device-wide barriers separate the steps, so no host round trip or launch gap sits between
 * them.  Every output is bit-identical to the one the per-step calls give (moe_route with the
 * same cfg, moe_dispatch with pos, moe_expert_ffn in BF16 for the routed experts and for the
 * shared experts with offsets NULL, moe_combine).
 * Fields (DEVICE pointers unless noted; R = T*k routed rows):
 *   T, H, E, k, I      tokens, hidden size, routed experts on this GPU, slots, intermediate;
 *   S, Is              shared experts (S = 0: none) and their intermediate size;
 *   E_router           experts the router scores;  cfg: router configuration (as moe_route);
 *   x [T,H] bf16;  w_router [E_router,H] bf16 or NULL;
 *   logits [T,E_router] fp32: read, or first WRITTEN with the projection when w_router given;
 *   idx_in [T,k] int32 local expert ids in [0,E), or NULL (then E must equal E_router and the
 *          router's own choice is permuted).  Given: one GPU's share of a larger layer -- the
 *          router still selects over E_router experts and its weights w scale the combine,
 *          while the rows are permuted by idx_in;
 *   w1 [E,2I,H], w2 [E,H,I], ws1 [S,2Is,H], ws2 [S,H,Is] bf16;
 *   idx, w, s_sel [T,k];  counts [E], offsets [E+1], pos [T,k], src [R] (as moe_route);
 *   xp [R,H], h [R,I], y [R,H] bf16;  gu [R,2I] bf16 or NULL (the backward's save);
 *   hs [S,T,Is], ys [S,T,H] bf16;  gus [S,T,2Is] bf16 or NULL;  out [T,H] bf16.
 * Limits: 1 <= E <= 256, 1 <= E_router <= 256, 1 <= k <= min(E_router, 64), T >= 1,
 * 0 <= S <= 64, H % 64 == 0, I % 64 == 0 (Is too when S > 0), R*max(H,2I) < 2^31.
 * Execution: a one-block clear of the workspace's synchronisation words, then the kernel as an
 * ordinary launch of one block per CU (a block takes 160 KB of LDS, so no CU holds two; the
 * device-wide barriers need every block resident, which an otherwise idle device gives at
 * once, and work of other streams holding CUs only delays the start).  Inside, the routing
 * steps, the dispatch and the combine are separated by device-wide barriers; the two expert
 * products form one queue of tiles (GEMM1 tiles, then GEMM2 tiles) claimed in order, where a
 * GEMM2 tile waits only for the GEMM1 tiles of its own rows (per-row-block completion
 * counters).  Every wait is bounded (2 s): one that runs out (for instance on a device that
 * can never hold all the blocks at once) sets the 32-bit word at byte offset
 * moe_layer_forward_error_offset() of ws to nonzero and the outputs are then undefined; the
 * word is 0 after a call that completed normally.
 * Concurrent calls need distinct workspaces.
 * Workspace: moe_layer_forward_workspace_size(). */
typedef struct moe_fwd_args {
    int T, H, E, k, I;
    int S, Is;
    int E_router;
    moe_route_cfg cfg;
    const void *x;
    const void *w_router;
    float *logits;
    const int32_t *idx_in;
    const void *w1, *w2, *ws1, *ws2;
    int32_t *idx;
    float *w, *s_sel;
    int32_t *counts, *offsets, *pos, *src;
    void *xp, *gu, *h, *y;
    void *gus, *hs, *ys;
    void *out;
} moe_fwd_args;

size_t moe_layer_forward_workspace_size(const moe_fwd_args *a);
size_t moe_layer_forward_error_offset(const moe_fwd_args *a);
int moe_layer_forward(const moe_fwd_args *a, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------ backward
 * BF16 backward of the whole layer (pulsen.vercel.app ¶3) given the upstream gradient dout
 * and the forward's saved tensors.  Gradients flow to x (through the routed and the shared
 * experts), to every expert weight, to the routing weights and through them to the logits;
 * no gradient flows through the selection itself.  Weight gradients are full reductions
 * over each expert's rows in a fixed order (no split-K, no atomics). */
typedef struct moe_bwd_args {
    int T, H, E, k, I, R;       /* routed part (R = rows = offsets[E]) */
    int S, Is;                  /* shared experts (S = 0: none) */
    int E_router;               /* width of the logits (experts the router scores) */
    int score, renorm;
    float route_scale;
    /* saved forward state */
    const void *x;              /* [T,H] bf16 (input of the shared experts) */
    const void *xp;             /* [R,H] bf16 dispatched rows */
    const void *gu;             /* [R,2I] bf16 saved gate/up pre-activations */
    const void *h;              /* [R,I] bf16 saved SwiGLU outputs */
    const void *y;              /* [R,H] bf16 expert outputs */
    const int32_t *offsets;     /* [E+1] */
    const int32_t *pos;         /* [T,k] */
    const int32_t *idx;         /* [T,k] router expert ids, in [0, E_router) */
    const float *w;             /* [T,k] routing weights */
    const float *s_sel;         /* [T,k] selected scores */
    const float *logits;        /* [T,E_router]; read only for softmax without renorm */
    const void *w1, *w2;        /* [E,2I,H], [E,H,I] bf16 */
    const void *gus, *hs;       /* [S,T,2Is], [S,T,Is] bf16 (shared experts' saves) */
    const void *ws1, *ws2;      /* [S,2Is,H], [S,H,Is] bf16 */
    const void *dout;           /* [T,H] bf16 upstream gradient */
    /* outputs */
    void *dx;                   /* [T,H] bf16 */
    void *dw1, *dw2;            /* [E,2I,H], [E,H,I] bf16 */
    void *dws1, *dws2;          /* [S,2Is,H], [S,H,Is] bf16 (NULL when S = 0) */
    float *dw_route;            /* [T,k] fp32: dL/dw[t,j] = <dout[t], y[pos[t,j]]> */
    float *dlogits;             /* [T,E_router] fp32 */
    /* Macrobatch walked in passes (aiexpert.news ¶4: a fixed ring buffer walked at minibatch
     * granularity).  passes <= 1: one pass, offsets [E+1], pos rows in [0,R).  passes > 1: the
     * tokens form consecutive passes of pass_tokens tokens (the last may hold fewer); pass p's
     * routed rows occupy rows [p*pass_rows, (p+1)*pass_rows) of xp, gu, h and y, offsets is
     * [passes][E+1] and pos holds rows local to the token's pass.  Weight gradients reduce
     * over the rows of every pass, in pass order.  R must equal passes * pass_rows. */
    int passes, pass_tokens, pass_rows;
    /* MXFP8 backward after an MXFP8 forward (mx = 1 or 2; one pass, H % 128 == 0,
     * I % 128 == 0).  The products take MX-quantised operands (MOE_MX_FLOOR) along their
     * contraction dimension and run on the scaled FP8 MFMA:
     *   dgrad (mx >= 1): dh = Q(dy) Q(W2_e^T)^T (with the SwiGLU backward) and
     *     dXp = Q(dGU) Q(W1_e^T)^T; dy and dGU are quantised on the fly, the weights come
     *     quantised along the contraction dimension, as mx_quantize_t writes them;
     *   weight gradients (mx == 2): dW2_e = Qt(dy_e)^T Qt(h_e), dW1_e = Qt(dGU_e)^T Qt(xp_e),
     *     every operand quantised along the expert's rows (32-row blocks from the expert's
     *     first row, the last one zero-padded); with mx == 1 they stay BF16 products.
     * xp and h must hold what the MX forward's GEMMs consumed -- the dequantised xp codes
     * (mx_dequantize) and the h_save of moe_expert_ffn -- and gu its gu_save.  With mx == 2,
     * xp may instead be given as the forward's codes and scales (xp_codes, xp_scales, from
     * moe_dispatch): xp is then not read and may be NULL, and the weight-gradient quantiser
     * decodes the codes itself (the same values, so the same results). */
    int mx;
    const uint8_t *w2t_codes;   /* [E,I,H]  W2_e^T codes, scales [E,I,H/32] (along H) */
    const uint8_t *w2t_scales;
    const uint8_t *w1t_codes;   /* [E,H,2I] W1_e^T codes, scales [E,H,2I/32] (along 2I) */
    const uint8_t *w1t_scales;
    const uint8_t *xp_codes;    /* mx == 2, optional: [R,H] xp codes, scales [R,H/32] */
    const uint8_t *xp_scales;
} moe_bwd_args;

size_t moe_backward_workspace_size(const moe_bwd_args *a);
int moe_backward(const moe_bwd_args *a, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------ MX quantisation
 * The operands of the MXFP8 forward (pulsen.vercel.app ¶3; aiexpert.news ¶4, whose headline
 * speed-up is for that precision), in the OCP Microscaling (MX) v1.0 format.
 * mx_quantize: OCP microscaling, one E8M0 scale per 32 consecutive values along K and E4M3
 * ("FN": bias 7, no infinity, max 448) codes, rounded to nearest even and saturating.
 * MOE_MX_FLOOR: scale 2^(floor(log2 amax) - 8); MOE_MX_CEIL: smallest power of two with
 * amax/scale <= 448.  An all-zero block gets scale code 0.  Bit-exact.
 *   in [rows,K] (in_dtype MOE_BF16 or MOE_F32), codes [rows,K] u8, scales [rows,K/32] u8.
 * K % 32 == 0. */
int mx_quantize(const void *in, int in_dtype, int rows, int K, uint8_t *codes, uint8_t *scales,
                int scale_mode, void *stream);

/* mx_quantize_t: the same quantisation along the FIRST dimension of each [A,B] bf16 matrix of a
 * batch, written transposed: codes [batch,B,A], scales [batch,B,A/32] (so that the codes of
 * a column of the input are contiguous: the layout a product contracting over A reads).  For
 * the MXFP8 backward: W2 [E,H,I] -> W2^T along H, W1 [E,2I,H] -> W1^T along 2I.
 * A % 32 == 0, batch <= 65535.  Bit-exact. */
int mx_quantize_t(const void *in, int batch, int A, int B, uint8_t *codes, uint8_t *scales,
                  int scale_mode, void *stream);

/* mx_dequantize: out [rows,K] bf16 = E4M3(code) * 2^(scale - 127), rounded to nearest even
 * (exact for every value in bf16's normal range).  K % 32 == 0.  Bit-exact. */
int mx_dequantize(const uint8_t *codes, const uint8_t *scales, int rows, int K, void *out,
                  void *stream);

/* ------------------------------------------------------------------ launch tracing
 * Optional timing of the library's own kernels, for profiling (the layer needs none of it).
 * moe_trace_begin(cap) arms tracing on the calling host thread: every kernel the library
 * then launches from this thread is bracketed by two hipEvent records on its stream, for the
 * first cap launches (later launches run untraced).  The events are created on the first
 * call (hipEventCreate; no device memory is allocated) and reused afterwards.  Returns
 * MOE_EINVAL unless 1 <= cap <= 2^20, MOE_EHIP if an event cannot be created.
 * moe_trace_end() disarms tracing and returns the number of launches recorded since
 * moe_trace_begin.  moe_trace_get(i, &name, &ms), for 0 <= i < that number, waits for
 * launch i to finish and returns its role name (a static string such as "gemm1_swiglu" or
 * "dispatch") and its duration in milliseconds; MOE_EINVAL for i out of range, MOE_EHIP on
 * an event error.  Records stay readable until the next moe_trace_begin on the thread. */
int moe_trace_begin(int cap);
int moe_trace_end(void);
int moe_trace_get(int i, const char **name, float *ms);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
