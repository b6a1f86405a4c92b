/*
 * moe_oracle.c -- plain, slow CPU oracle of the deterministic mixture-of-experts layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark load this library.  It shares no code, header, table or constant
 * generator with the GPU library, and the GPU library never calls it.
 *
 * What it computes: one GPU's share of a DeepSeek-V3-type MoE layer (pulsen.vercel.app,
 * "Cursor åpner megakernelen som ga 41 prosent flere tokens i sekundet", ¶6): router top-k,
 * dispatch into expert-contiguous rows, a SwiGLU FFN per expert, a weighted combine back to
 * token order, the BF16 backward of all of it (same page, ¶3), and the MXFP8 forward with
 * E8M0-scaled E4M3 operands (same page ¶3; aiexpert.news, "Megakernels are dead and back",
 * ¶4).  The pages print no formulas; every step below is the textbook definition of that
 * layer, written as plain loops.
 *
 * Precision: every floating-point value of the layer is computed in fp64 from the exact
 * bf16 inputs, with no intermediate rounding.  The one exception is where a float decides
 * an integer: the routing keys and group scores that pick experts are computed in fp32,
 * the precision the GPU kernels take that decision in, so that the choice is comparable
 * bit for bit.
 *
 * Parallelism: OpenMP only across independent outputs, never across a reduction, so every
 * sum here has one fixed sequential order and the oracle is itself deterministic.
 * Build: gcc -O2 -std=c99 -fopenmp -ffp-contract=off -fno-fast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_SOFTMAX 0
#define ORC_SIGMOID 1

static double bf(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static float bff(uint16_t b) { return (float)bf(b); }

int orc_version(void) { return 1; }

/* Threads the OpenMP loops of this library use (1 when built without OpenMP). */
#ifdef _OPENMP
#include <omp.h>
int orc_threads(void) { return omp_get_max_threads(); }
#else
int orc_threads(void) { return 1; }
#endif

/* bf16 bit patterns -> fp64 (exact). */
void orc_bf16_to_f64(const uint16_t *in, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; i++) out[i] = bf(in[i]);
}

/* ------------------------------------------------------------------ router projection
 * logits[t,e] = sum_h x[t,h] * w_router[e,h], accumulated in fp32 in ascending h starting
 * from +0.  A bf16 x bf16 product is exact in fp32, so this order fixes the result bit
 * for bit (reading of the router input for the tiny workload; the pages are silent). */
void orc_router_logits(const uint16_t *x, const uint16_t *wr, int T, int H, int E,
                       float *logits)
{
    for (int t = 0; t < T; t++)
        for (int e = 0; e < E; e++) {
            float acc = 0.0f;
            for (int h = 0; h < H; h++) {
                float p = bff(x[(size_t)t * H + h]) * bff(wr[(size_t)e * H + h]);
                acc = acc + p;
            }
            logits[(size_t)t * E + e] = acc;
        }
}

/* ------------------------------------------------------------------ sigmoid key
 * Reading: sigmoid scores that decide routing are computed with a fixed recipe of IEEE fp32
 * operations (each rounded to nearest even, no fused multiply-add), so that CPU and GPU keys
 * agree bit for bit:
 *   clamp x to [-40, 40]; z = -x;
 *   n = rint(z * log2(e));  r = (z - n*C1) - n*C2  (Cody & Waite additive range reduction,
 *       C1 = ln 2 truncated to 12 significant bits so n*C1 is exact, C2 = fp32(ln 2 - C1));
 *   p = 1 + r(1 + r(1/2 + r(1/6 + r(1/24 + r(1/120 + r(1/720 + r/5040))))))  (Taylor series
 *       of exp to degree 7, Horner form, coefficients fp32(1/j!));
 *   eps = p * 2^n;  s = 1 / (1 + eps). */
float orc_rsig(float x)
{
    const double ln2 = 0.69314718055994530942;
    const float C1 = (float)(floor(ln2 * 4096.0) / 4096.0);
    const float C2 = (float)(ln2 - (double)C1);
    const float L2E = (float)1.44269504088896340736;
    float xc = x < -40.0f ? -40.0f : (x > 40.0f ? 40.0f : x);
    float z = -xc;
    float n = rintf(z * L2E);
    float r = (z - n * C1) - n * C2;
    float p = 1.0f / 5040.0f;
    p = (float)(1.0 / 720.0) + r * p;
    p = (float)(1.0 / 120.0) + r * p;
    p = (float)(1.0 / 24.0) + r * p;
    p = (float)(1.0 / 6.0) + r * p;
    p = 0.5f + r * p;
    p = 1.0f + r * p;
    p = 1.0f + r * p;
    float eps = ldexpf(p, (int)n);
    return 1.0f / (1.0f + eps);
}

static float sel_key(float logit, int score, const float *bias, int e)
{
    float k;
    if (score == ORC_SIGMOID) {
        k = orc_rsig(logit);
        if (bias) k = k + bias[e];
    } else {
        k = logit;
    }
    return k + 0.0f; /* -0 -> +0: equal keys compare equal */
}

/* a ranks before b: larger key, then lower index. */
static int ranks_before(float ka, int a, float kb, int b)
{
    return ka > kb || (ka == kb && a < b);
}

/* ------------------------------------------------------------------ top-k selection
 * For every token: selection keys (softmax: the logit, since softmax is monotone; sigmoid:
 * sigmoid(logit) + bias).  With n_groups > 1 the experts are split into n_groups contiguous
 * groups; a group's score is the fp32 sum, largest first, of its top k/topk_groups keys; the
 * topk_groups best groups (score desc, then lower group id) stay and the other groups'
 * experts are masked (DeepSeek-V3 group-limited routing; the pages only name the layer
 * type).  Then the k unmasked experts of largest key are taken, slot j being the j-th in
 * (key desc, expert id asc) order.
 * idx [T,k] int32; s_sel [T,k] fp32 = the selected score (sigmoid value, or the logit). */
int orc_route_select(const float *logits, int T, int E, int k, int score, int n_groups,
                     int topk_groups, const float *bias, int32_t *idx, float *s_sel)
{
    if (n_groups < 1) n_groups = 1;
    if (topk_groups < 1 || n_groups == 1) topk_groups = n_groups;
    if (E % n_groups || k > E || topk_groups > n_groups) return -1;
    int gs = E / n_groups;
    int per_group = k / topk_groups;
    if (per_group < 1) per_group = 1;
    if (per_group > gs || k > topk_groups * gs) return -1;
    float *key = malloc(sizeof(float) * E);
    char *avail = malloc(E);
    float *gscore = malloc(sizeof(float) * n_groups);
    char *gkeep = malloc(n_groups);
    char *gtaken = malloc(gs);
    for (int t = 0; t < T; t++) {
        const float *L = logits + (size_t)t * E;
        for (int e = 0; e < E; e++) key[e] = sel_key(L[e], score, bias, e);
        for (int e = 0; e < E; e++) avail[e] = 1;
        if (n_groups > 1) {
            for (int g = 0; g < n_groups; g++) {
                /* top per_group keys of the group, summed largest first */
                memset(gtaken, 0, gs);
                float s = 0.0f;
                for (int q = 0; q < per_group; q++) {
                    int best = -1;
                    for (int i = 0; i < gs; i++) {
                        if (gtaken[i]) continue;
                        int e = g * gs + i;
                        if (best < 0 || ranks_before(key[e], e, key[g * gs + best], g * gs + best))
                            best = i;
                    }
                    gtaken[best] = 1;
                    s = s + key[g * gs + best];
                }
                gscore[g] = s + 0.0f;
                gkeep[g] = 0;
            }
            for (int q = 0; q < topk_groups; q++) {
                int best = -1;
                for (int g = 0; g < n_groups; g++) {
                    if (gkeep[g]) continue;
                    if (best < 0 || ranks_before(gscore[g], g, gscore[best], best)) best = g;
                }
                gkeep[best] = 1;
            }
            for (int e = 0; e < E; e++) avail[e] = gkeep[e / gs];
        }
        for (int j = 0; j < k; j++) {
            int best = -1;
            for (int e = 0; e < E; e++) {
                if (!avail[e]) continue;
                if (best < 0 || ranks_before(key[e], e, key[best], best)) best = e;
            }
            avail[best] = 0;
            idx[(size_t)t * k + j] = best;
            s_sel[(size_t)t * k + j] = score == ORC_SIGMOID ? orc_rsig(L[best]) : L[best];
        }
    }
    free(key); free(avail); free(gscore); free(gkeep); free(gtaken);
    return 0;
}

/* ------------------------------------------------------------------ routing weights (fp64)
 * softmax, renorm:    w_j = exp(L_j) / sum_j' exp(L_j') over the k selected logits (equal to
 *                     the full softmax renormalised over the selection);
 * softmax, no renorm: w_j = full softmax over all E logits, at the selected expert;
 * sigmoid, renorm:    w_j = route_scale * s_j / sum_j' s_j', s = 1/(1+exp(-L));
 * sigmoid, no renorm: w_j = route_scale * s_j. */
void orc_route_weights(const double *L, const int32_t *idx, int T, int E, int k, int score,
                       int renorm, double route_scale, double *w)
{
    for (int t = 0; t < T; t++) {
        const double *l = L + (size_t)t * E;
        const int32_t *id = idx + (size_t)t * k;
        double *wt = w + (size_t)t * k;
        if (score == ORC_SOFTMAX) {
            if (renorm) {
                double m = l[id[0]];
                for (int j = 1; j < k; j++) if (l[id[j]] > m) m = l[id[j]];
                double s = 0.0;
                for (int j = 0; j < k; j++) s += exp(l[id[j]] - m);
                for (int j = 0; j < k; j++) wt[j] = exp(l[id[j]] - m) / s;
            } else {
                double m = l[0];
                for (int e = 1; e < E; e++) if (l[e] > m) m = l[e];
                double s = 0.0;
                for (int e = 0; e < E; e++) s += exp(l[e] - m);
                for (int j = 0; j < k; j++) wt[j] = exp(l[id[j]] - m) / s;
            }
        } else {
            double s = 0.0;
            for (int j = 0; j < k; j++) s += 1.0 / (1.0 + exp(-l[id[j]]));
            for (int j = 0; j < k; j++) {
                double sj = 1.0 / (1.0 + exp(-l[id[j]]));
                wt[j] = renorm ? route_scale * sj / s : route_scale * sj;
            }
        }
    }
}

/* ------------------------------------------------------------------ permutation
 * counts[e] = number of (t,j) with idx[t,j] = e;  offsets = exclusive prefix sum (E+1);
 * pos[t,j] = offsets[e] + number of pairs (t',j') before (t,j) in token-major order with the
 * same expert (reading: rows of one expert in ascending (t,j));  src[pos[t,j]] = t*k + j. */
void orc_permute(const int32_t *idx, int T, int k, int E, int32_t *counts, int32_t *offsets,
                 int32_t *pos, int32_t *src)
{
    for (int e = 0; e < E; e++) counts[e] = 0;
    for (int64_t p = 0; p < (int64_t)T * k; p++) counts[idx[p]]++;
    offsets[0] = 0;
    for (int e = 0; e < E; e++) offsets[e + 1] = offsets[e] + counts[e];
    int32_t *fill = calloc((size_t)(E > 0 ? E : 1), sizeof(int32_t));
    for (int64_t p = 0; p < (int64_t)T * k; p++) {
        int e = idx[p];
        int32_t r = offsets[e] + fill[e]++;
        pos[p] = r;
        src[r] = (int32_t)p;
    }
    free(fill);
}

/* ------------------------------------------------------------------ load-balancing bias
 * Auxiliary-loss-free balancing of DeepSeek-V3 (the layer type of pulsen.vercel.app ¶6; the
 * rule itself is from the DeepSeek-V3 Technical Report, arXiv:2412.19437, §2.1.2): after a
 * step, each expert's selection bias moves by gamma against its load -- down when the expert
 * received more than the mean load, up when it received less, unchanged at the mean.
 * Reading: load = counts[e], mean = (sum of counts) / E, compared exactly as
 * counts[e] * E against the sum; the new bias is the fp32 sum bias + (+-gamma), one rounding. */
void orc_update_bias(const int32_t *counts, int E, float gamma, float *bias)
{
    int64_t total = 0;
    for (int e = 0; e < E; e++) total += counts[e];
    for (int e = 0; e < E; e++) {
        int64_t scaled = (int64_t)counts[e] * E;
        if (scaled > total) bias[e] = bias[e] - gamma;
        else if (scaled < total) bias[e] = bias[e] + gamma;
    }
}

/* ------------------------------------------------------------------ dispatch
 * xp[r,:] = x[src[r] / k, :]  (byte copy). */
void orc_dispatch(const uint16_t *x, int T, int H, int k, const int32_t *src, int R,
                  uint16_t *xp)
{
    (void)T;
    for (int r = 0; r < R; r++)
        memcpy(xp + (size_t)r * H, x + (size_t)(src[r] / k) * H, sizeof(uint16_t) * H);
}

/* ------------------------------------------------------------------ MX (OCP microscaling)
 * E4M3 ("FN" variant): 1 sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0
 * is subnormal (m/8 * 2^-6); 0x7F / 0xFF are NaN; no infinity; largest finite 448. */
double orc_e4m3_decode(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    double v = e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* Round to the nearest E4M3 value, ties to the even mantissa, saturating at +-448. */
uint8_t orc_e4m3_encode(double v)
{
    uint8_t s = (v < 0 || (v == 0 && signbit(v))) ? 0x80 : 0;
    double a = fabs(v);
    if (a >= 448.0) return s | 0x7E;
    int ex;
    frexp(a, &ex);            /* a = f * 2^ex, f in [0.5, 1) */
    int e = ex - 1;           /* floor(log2 a) for a > 0 */
    if (a == 0.0 || e < -6) e = -6;
    double quantum = ldexp(1.0, e - 3);
    double q = rint(a / quantum);   /* exact division (power of two); rint: ties to even */
    double r = q * quantum;
    if (r >= 448.0) return s | 0x7E;
    /* encode r exactly */
    if (r < ldexp(1.0, -6)) return s | (uint8_t)(int)(r / ldexp(1.0, -9));
    frexp(r, &ex);
    e = ex - 1;
    int m = (int)((r / ldexp(1.0, e) - 1.0) * 8.0);
    return s | (uint8_t)(((e + 7) << 3) | m);
}

/* E8M0 shared scale of one block of n values (OCP MX: X = 2^(floor(log2 amax) - 8), 8 being
 * the largest E4M3 exponent), returned as the biased code (exponent + 127), clamped to
 * [0, 254].  An all-zero block takes code 0.  mode 1 (option): the smallest power of two
 * with amax / X <= 448, so that no element saturates. */
static int mx_scale_code(const double *v, int n, int mode)
{
    double amax = 0.0;
    for (int i = 0; i < n; i++) if (fabs(v[i]) > amax) amax = fabs(v[i]);
    if (amax == 0.0) return 0;
    int ex;
    frexp(amax, &ex);
    int e = ex - 1 - 8;
    if (mode == 1) {
        e = ex - 1 - 8;
        while (amax / ldexp(1.0, e) > 448.0) e++;
        while (e > -127 && amax / ldexp(1.0, e - 1) <= 448.0) e--;
    }
    int code = e + 127;
    if (code < 0) code = 0;
    if (code > 254) code = 254;
    return code;
}

/* codes [rows, K] E4M3, scales [rows, K/32] E8M0: blocks of 32 consecutive values along K. */
void orc_mx_quantize(const double *in, int64_t rows, int K, int mode, uint8_t *codes,
                     uint8_t *scales)
{
    int nb = K / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++)
        for (int b = 0; b < nb; b++) {
            const double *v = in + r * K + b * 32;
            int sc = mx_scale_code(v, 32, mode);
            scales[r * nb + b] = (uint8_t)sc;
            double X = ldexp(1.0, sc - 127);
            for (int i = 0; i < 32; i++) codes[r * K + b * 32 + i] = orc_e4m3_encode(v[i] / X);
        }
}

void orc_mx_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t rows, int K,
                       double *out)
{
    int nb = K / 32;
    for (int64_t r = 0; r < rows; r++)
        for (int i = 0; i < K; i++)
            out[r * K + i] = orc_e4m3_decode(codes[r * K + i]) *
                             ldexp(1.0, (int)scales[r * nb + i / 32] - 127);
}

/* ------------------------------------------------------------------ expert FFN (fp64)
 * Per expert e and routed row r of it (SwiGLU, no biases; w1 stacks the gate rows 0..I-1
 * over the up rows I..2I-1):
 *   g_i = sum_h xp[r,h] w1[e][i,h];  u_i = sum_h xp[r,h] w1[e][I+i,h];
 *   h_i = g_i * sigmoid(g_i) * u_i;  y[r,c] = sum_i h_i w2[e][c,i].
 * offsets [E+1] give each expert's rows; offsets == NULL means every expert takes all R
 * rows (shared experts), writing y[e*R + r].  gu [R,2I] and h [R,I] are optional saves.
 * h_mx != 0: h is MX-quantised along I (blocks of 32) and dequantised before the second
 * product, as the MXFP8 forward feeds the down projection. */
static double dot(const double *a, const double *b, int n)
{
    double s = 0.0;
    for (int i = 0; i < n; i++) s += a[i] * b[i];
    return s;
}

static double sigm(double g) { return 1.0 / (1.0 + exp(-g)); }

void orc_ffn_fwd(const double *xp, const int32_t *offsets, int E, int R, int H, int I,
                 const double *w1, const double *w2, int h_mx, double *gu, double *hout,
                 double *y)
{
    for (int e = 0; e < E; e++) {
        int r0 = offsets ? offsets[e] : 0, r1 = offsets ? offsets[e + 1] : R;
        const double *W1 = w1 + (size_t)e * 2 * I * H;
        const double *W2 = w2 + (size_t)e * H * I;
#pragma omp parallel for schedule(dynamic, 1)
        for (int r = r0; r < r1; r++) {
            const double *row = xp + (size_t)r * H;
            size_t orow = offsets ? (size_t)r : (size_t)e * R + r;
            double *hv = malloc(sizeof(double) * I);
            for (int i = 0; i < I; i++) {
                double g = dot(row, W1 + (size_t)i * H, H);
                double u = dot(row, W1 + (size_t)(I + i) * H, H);
                if (gu) { gu[orow * 2 * I + i] = g; gu[orow * 2 * I + I + i] = u; }
                hv[i] = g * sigm(g) * u;
            }
            if (h_mx) {
                uint8_t cb[32], sb;
                for (int b = 0; b < I / 32; b++) {
                    orc_mx_quantize(hv + b * 32, 1, 32, 0, cb, &sb);
                    orc_mx_dequantize(cb, &sb, 1, 32, hv + b * 32);
                }
            }
            if (hout) memcpy(hout + orow * I, hv, sizeof(double) * I);
            for (int c = 0; c < H; c++) y[orow * H + c] = dot(hv, W2 + (size_t)c * I, I);
            free(hv);
        }
    }
}

/* ------------------------------------------------------------------ combine
 * out[t,:] = sum_{j=0..k-1} w[t,j] * y[pos[t,j],:]  +  sum_{s=0..S-1} ys[s,t,:]. */
void orc_combine(const double *y, const int32_t *pos, const double *w, int T, int k, int H,
                 const double *ys, int S, double *out)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; t++)
        for (int c = 0; c < H; c++) {
            double acc = 0.0;
            for (int j = 0; j < k; j++)
                acc += w[(size_t)t * k + j] * y[(size_t)pos[(size_t)t * k + j] * H + c];
            for (int s = 0; s < S; s++) acc += ys[((size_t)s * T + t) * H + c];
            out[(size_t)t * H + c] = acc;
        }
}

/* ------------------------------------------------------------------ backward (fp64)
 * Combine:  dy[pos[t,j],:] = w[t,j] * dout[t,:];  dw[t,j] = <dout[t,:], y[pos[t,j],:]>. */
void orc_combine_bwd(const double *dout, const double *y, const int32_t *pos,
                     const double *w, int T, int k, int H, double *dy, double *dw)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; t++)
        for (int j = 0; j < k; j++) {
            size_t r = (size_t)pos[(size_t)t * k + j];
            double wt = w[(size_t)t * k + j];
            for (int c = 0; c < H; c++) dy[r * H + c] = wt * dout[(size_t)t * H + c];
            dw[(size_t)t * k + j] = dot(dout + (size_t)t * H, y + r * H, H);
        }
}

/* FFN backward given dy (gradient at the FFN output rows):
 *   dh_i = sum_c dy[r,c] w2[e][c,i];
 *   dg_i = dh_i * u_i * sig(g_i) * (1 + g_i (1 - sig(g_i)));  du_i = dh_i * g_i * sig(g_i);
 *   dxp[r,h] = sum_i dg_i w1[e][i,h] + du_i w1[e][I+i,h];
 *   dw2[e][c,i] = sum_{r in e} dy[r,c] h[r,i];
 *   dw1[e][i,h] = sum_{r in e} dg[r,i] xp[r,h];  dw1[e][I+i,h] = sum_{r in e} du[r,i] xp[r,h].
 * Token sums run over the expert's rows in ascending order.  offsets == NULL: every expert
 * takes all R rows (shared experts), dy and dxp indexed [e*R + r]. */
void orc_ffn_bwd(const double *xp, const int32_t *offsets, int E, int R, int H, int I,
                 const double *w1, const double *w2, const double *dy, double *dxp,
                 double *dw1, double *dw2)
{
    for (int e = 0; e < E; e++) {
        int r0 = offsets ? offsets[e] : 0, r1 = offsets ? offsets[e + 1] : R;
        int M = r1 - r0;
        size_t ob = offsets ? 0 : (size_t)e * R;
        const double *W1 = w1 + (size_t)e * 2 * I * H;
        const double *W2 = w2 + (size_t)e * H * I;
        double *dW1 = dw1 + (size_t)e * 2 * I * H;
        double *dW2 = dw2 + (size_t)e * H * I;
        double *hv = malloc(sizeof(double) * ((size_t)M * I + 1));
        double *dg = malloc(sizeof(double) * ((size_t)M * I + 1));
        double *du = malloc(sizeof(double) * ((size_t)M * I + 1));
#pragma omp parallel for schedule(dynamic, 1)
        for (int m = 0; m < M; m++) {
            size_t r = (size_t)(r0 + m);
            const double *row = xp + r * H;
            const double *dyr = dy + (ob + r) * H;
            for (int i = 0; i < I; i++) {
                double g = dot(row, W1 + (size_t)i * H, H);
                double u = dot(row, W1 + (size_t)(I + i) * H, H);
                double sg = sigm(g);
                double dh = 0.0;
                for (int c = 0; c < H; c++) dh += dyr[c] * W2[(size_t)c * I + i];
                hv[(size_t)m * I + i] = g * sg * u;
                dg[(size_t)m * I + i] = dh * u * sg * (1.0 + g * (1.0 - sg));
                du[(size_t)m * I + i] = dh * g * sg;
            }
            for (int c = 0; c < H; c++) {
                double acc = 0.0;
                for (int i = 0; i < I; i++)
                    acc += dg[(size_t)m * I + i] * W1[(size_t)i * H + c] +
                           du[(size_t)m * I + i] * W1[(size_t)(I + i) * H + c];
                dxp[(ob + r) * H + c] = acc;
            }
        }
#pragma omp parallel for schedule(static)
        for (int c = 0; c < H; c++)
            for (int i = 0; i < I; i++) {
                double acc = 0.0;
                for (int m = 0; m < M; m++)
                    acc += dy[(ob + r0 + m) * H + c] * hv[(size_t)m * I + i];
                dW2[(size_t)c * I + i] = acc;
            }
#pragma omp parallel for schedule(static)
        for (int i = 0; i < I; i++)
            for (int c = 0; c < H; c++) {
                double ag = 0.0, au = 0.0;
                for (int m = 0; m < M; m++) {
                    double xv = xp[(size_t)(r0 + m) * H + c];
                    ag += dg[(size_t)m * I + i] * xv;
                    au += du[(size_t)m * I + i] * xv;
                }
                dW1[(size_t)i * H + c] = ag;
                dW1[(size_t)(I + i) * H + c] = au;
            }
        free(hv); free(dg); free(du);
    }
}

/* Un-permute:  dx[t,:] = sum_{j} dxp[pos[t,j],:] + sum_s dxs[s,t,:]. */
void orc_unpermute(const double *dxp, const int32_t *pos, int T, int k, int H,
                   const double *dxs, int S, double *dx)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; t++)
        for (int c = 0; c < H; c++) {
            double acc = 0.0;
            for (int j = 0; j < k; j++) acc += dxp[(size_t)pos[(size_t)t * k + j] * H + c];
            for (int s = 0; s < S; s++) acc += dxs[((size_t)s * T + t) * H + c];
            dx[(size_t)t * H + c] = acc;
        }
}

/* Router backward: gradient of the loss with respect to the logits, given dw = dL/dw.
 * Selection (top-k, group mask, bias) passes no gradient; the derivative is that of the
 * weight formulas of orc_route_weights:
 *   softmax renorm:    dL[i_j] = w_j (dw_j - sum_j' w_j' dw_j');
 *   softmax no renorm: dL[e] = p_e (dw at e if selected, else 0  -  sum_j w_j dw_j);
 *   sigmoid renorm:    dL[i_j] = s_j(1-s_j) (c/S) (dw_j - sum_j' (w_j'/c) dw_j'),
 *                      S = sum of the selected s, c = route_scale;
 *   sigmoid no renorm: dL[i_j] = c dw_j s_j (1 - s_j).
 * dL [T,E] is written in full (zeros where no gradient flows). */
void orc_router_bwd(const double *L, const int32_t *idx, const double *dw, int T, int E,
                    int k, int score, int renorm, double route_scale, double *dL)
{
    double *w = malloc(sizeof(double) * k);
    for (int t = 0; t < T; t++) {
        const double *l = L + (size_t)t * E;
        const int32_t *id = idx + (size_t)t * k;
        const double *g = dw + (size_t)t * k;
        double *d = dL + (size_t)t * E;
        for (int e = 0; e < E; e++) d[e] = 0.0;
        orc_route_weights(l, id, 1, E, k, score, renorm, route_scale, w);
        double wg = 0.0;
        for (int j = 0; j < k; j++) wg += w[j] * g[j];
        if (score == ORC_SOFTMAX) {
            if (renorm) {
                for (int j = 0; j < k; j++) d[id[j]] += w[j] * (g[j] - wg);
            } else {
                double m = l[0];
                for (int e = 1; e < E; e++) if (l[e] > m) m = l[e];
                double s = 0.0;
                for (int e = 0; e < E; e++) s += exp(l[e] - m);
                for (int e = 0; e < E; e++) d[e] = -(exp(l[e] - m) / s) * wg;
                for (int j = 0; j < k; j++) d[id[j]] += w[j] * g[j];
            }
        } else {
            double S = 0.0;
            for (int j = 0; j < k; j++) S += sigm(l[id[j]]);
            for (int j = 0; j < k; j++) {
                double s = sigm(l[id[j]]);
                double ds = renorm ? (route_scale / S) * (g[j] - wg / route_scale)
                                   : route_scale * g[j];
                d[id[j]] += ds * s * (1.0 - s);
            }
        }
    }
    free(w);
}
