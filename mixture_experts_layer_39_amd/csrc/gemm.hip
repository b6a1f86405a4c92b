// Grouped GEMMs of the expert FFN on gfx950 MFMA, forward and backward.
//
// One kernel template covers every product of the layer:
//   forward   GEMM1  [g|u] = Xp_e W1_e^T  with the SwiGLU epilogue (h, optional saved g/u)
//             GEMM2  y = h_e W2_e^T
//   backward  dgrad  dh = dy_e W2_e  with the SwiGLU-backward epilogue (dg, du)
//             dgrad  dXp = dGU_e W1_e
//             wgrad  dW2_e = dy_e^T h_e,  dW1_e = dGU_e^T Xp_e   (full reduction over the
//                    expert's rows inside one tile: no split-K, no atomics)
// (the layer is the DeepSeek-V3-type MoE layer of pulsen.vercel.app, "Cursor åpner
// megakernelen…", ¶6, trained with a BF16 backward, same page ¶3).
//
// Design (CDNA4, wave64):
//  - 256x256 output tile per 256-thread block, 4 waves in 2x2, each wave a 128x128 sub-tile
//    of 4x4 v_mfma_f32_32x32x16_bf16 accumulators (256 fp32 per lane, one wave per SIMD).
//  - K steps of 64; operands staged global -> registers -> LDS, LDS double-buffered so one
//    barrier per K step suffices; loads of step k+1 are in flight during the MFMAs of step k.
//  - LDS rows are K-contiguous (16-byte chunks XOR-swizzled by row) so every MFMA operand is
//    one conflict-free ds_read_b128.  Operands that are M- or N-contiguous in memory (the
//    weights in dgrad, both operands in wgrad) are transposed 8x8 in registers on the way.
//  - Global loads are raw buffer loads whose range check returns zeros past the end of an
//    expert's rows, which pads ragged M tails and ragged K (wgrad) tails for free.
//  - Expert tile lists are derived on the device from the offsets (no host readback): each
//    block scans the per-expert tile counts in a wave and finds its tile.  Block b runs on
//    XCD b % 8; tiles are renumbered so each XCD works on a contiguous range of the tile
//    order, which is grouped 4 M-tiles at a time so concurrent tiles share A and B panels in
//    that XCD's L2.
#include "common.h"

namespace moe {

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                             0x00020000);
}
__device__ __forceinline__ u32x4 bload(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

constexpr int BM = 256, BN = 256, BK = 64, NTH = 256;
constexpr int GM = 4;  // M tiles per L2 group

enum { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_DSWIGLU = 2 };

struct GemmArgs {
    const bf16_t* A;
    int64_t a_es;  // per-expert element stride of A
    int lda;
    const bf16_t* B;
    int64_t b_es;
    int ldb;
    bf16_t* C;
    int64_t c_es;
    int ldc;
    bf16_t* C2;  // SwiGLU: saved g|u (may be null); SwiGLU-backward: the saved g|u (read)
    int64_t c2_es;
    int ldc2;
    const int32_t* offsets;  // ragged rows per expert, or null: every expert has R rows
    int E, R;
    int M, N, K;  // static extents (ragged-M mode: N, K; ragged-K mode: M, N)
    int I;        // SwiGLU channels
    int b_rows;   // rows of B per expert (K-contiguous B) or K (N-contiguous B)
    int total;    // tile count when it is static (ragged-K or shared mode)
};

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ uint32_t lds_off(int buf, int row, int chunk) {
    return (uint32_t)((buf * 256 + row) * 128 + ((chunk ^ swz(row)) << 4));
}
__host__ __device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

// 8x8 transpose of bf16: in[kk] holds 8 m-values at k = kk; out[mm] holds 8 k-values at m = mm.
__device__ __forceinline__ void transpose8x8(const u32x4* in, u32x4* out) {
#pragma unroll
    for (int mm = 0; mm < 8; ++mm) {
        const uint32_t sel = (mm & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            out[mm][j] = __builtin_amdgcn_perm(in[2 * j + 1][mm >> 1], in[2 * j][mm >> 1], sel);
    }
}

template <bool A_K, bool B_K, int EPI, bool GK>
__device__ __forceinline__ void gemm_body(const GemmArgs& g) {
    __shared__ __attribute__((aligned(16))) char smem[4 * 256 * 128];
    __shared__ int s_tp[1024];
    __shared__ int s_total;

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid >> 1, wn = wid & 1;
    const int NT = (EPI == EPI_SWIGLU) ? cdiv(g.I, 128) : cdiv(g.N, BN);

    // ---------------------------------------------------------------- locate the tile
    int total;
    const bool ragged_m = !GK && g.offsets != nullptr;
    if (ragged_m) {
        if (wid == 0) {
            int run = 0;
            for (int base = 0; base < g.E; base += 64) {
                int e = base + lane, tiles = 0;
                if (e < g.E) {
                    int lo = min(max(g.offsets[e], 0), g.R);
                    int hi = min(max(g.offsets[e + 1], lo), g.R);
                    tiles = cdiv(hi - lo, BM) * NT;
                }
                int inc = wave_incl_scan(tiles) + run;
                if (e < g.E) s_tp[e] = inc;
                run = __shfl(inc, 63, 64);
            }
            if (lane == 0) s_total = run;
        }
        __syncthreads();
        total = s_total;
    } else {
        total = g.total;
    }
    const int bid = blockIdx.x;
    if (bid >= total) return;
    // XCD-aware renumbering: XCD x = bid % 8 takes a contiguous range of tile ids.
    int logical;
    {
        int q = total >> 3, r = total & 7, x = bid & 7;
        logical = x * q + min(x, r) + (bid >> 3);
    }
    int e, t_local, Mrows, row0;
    if (ragged_m) {
        int lo = 0, hi = g.E - 1;
        while (lo < hi) {
            int mid = (lo + hi) >> 1;
            if (s_tp[mid] > logical) hi = mid; else lo = mid + 1;
        }
        e = lo;
        t_local = logical - (e ? s_tp[e - 1] : 0);
        int a = min(max(g.offsets[e], 0), g.R);
        int b = min(max(g.offsets[e + 1], a), g.R);
        row0 = a;
        Mrows = b - a;
    } else {
        int per = GK ? cdiv(g.M, BM) * NT : cdiv(g.R, BM) * NT;
        e = logical / per;
        t_local = logical - e * per;
        if (GK) {
            if (g.offsets) {
                int a = min(max(g.offsets[e], 0), g.R);
                int b = min(max(g.offsets[e + 1], a), g.R);
                row0 = a;
                Mrows = b - a;  // here: the K extent (rows of the expert)
            } else {
                row0 = 0;
                Mrows = g.R;
            }
        } else {
            row0 = 0;
            Mrows = g.R;
        }
    }
    const int MT = GK ? cdiv(g.M, BM) : cdiv(Mrows, BM);
    int tm, tn;
    {
        int grp = t_local / (GM * NT);
        int first = grp * GM;
        int gsz = min(MT - first, GM);
        int rr = t_local - grp * GM * NT;
        tm = first + rr % gsz;
        tn = rr / gsz;
    }
    const int m0 = tm * BM;
    const int Kdim = GK ? Mrows : g.K;
    const int Mvalid = GK ? g.M : Mrows;

    // ---------------------------------------------------------------- operand setup
    // A: K-contiguous (row m at A_e + (row0 + m)*lda)  or  M-contiguous (wgrad: element
    // (m,k) at A_e + (row0 + k)*lda + m).
    rsrc_t ra, rb;
    uint32_t va[8], vb[8];
    uint32_t a_kstep, b_kstep;
    if (A_K) {
        const bf16_t* base = g.A + e * g.a_es + (int64_t)(row0 + m0) * g.lda;
        ra = make_rsrc(base, (uint32_t)max(Mrows - m0, 0) * (uint32_t)g.lda * 2u);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            va[i] = (uint32_t)((tid >> 3) + 32 * i) * (uint32_t)g.lda * 2u + (uint32_t)(tid & 7) * 16u;
        a_kstep = BK * 2;
    } else {
        const bf16_t* base = g.A + e * g.a_es + (int64_t)row0 * g.lda + m0;
        ra = make_rsrc(base, (uint32_t)Kdim * (uint32_t)g.lda * 2u - (uint32_t)m0 * 2u);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
            va[kk] = (uint32_t)((tid >> 5) * 8 + kk) * (uint32_t)g.lda * 2u + (uint32_t)(tid & 31) * 16u;
        a_kstep = (uint32_t)BK * (uint32_t)g.lda * 2u;
    }
    const int n0 = tn * BN;
    const int ch0 = tn * 128;  // SwiGLU channel base
    if (B_K) {
        const bf16_t* base = g.B + e * g.b_es;
        rb = make_rsrc(base, (uint32_t)g.b_rows * (uint32_t)g.ldb * 2u);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            int nn = (tid >> 3) + 32 * i;
            int row;
            if (EPI == EPI_SWIGLU) {
                int q = nn & 127;
                row = (q >> 6) * g.I + ch0 + (nn >> 7) * 64 + (q & 63);
            } else {
                row = n0 + nn;
            }
            vb[i] = (uint32_t)row * (uint32_t)g.ldb * 2u + (uint32_t)(tid & 7) * 16u;
        }
        b_kstep = BK * 2;
    } else {
        // N-contiguous: element (n,k) at B_e + (row0_k + k)*ldb + n; in ragged-M mode B is a
        // weight with K rows (row0_k = 0); in ragged-K mode the rows are the expert's tokens.
        const int64_t kbase = GK ? row0 : 0;
        const bf16_t* base = g.B + e * g.b_es + kbase * g.ldb + n0;
        rb = make_rsrc(base, (uint32_t)Kdim * (uint32_t)g.ldb * 2u - (uint32_t)n0 * 2u);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
            vb[kk] = (uint32_t)((tid >> 5) * 8 + kk) * (uint32_t)g.ldb * 2u + (uint32_t)(tid & 31) * 16u;
        b_kstep = (uint32_t)BK * (uint32_t)g.ldb * 2u;
    }

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    u32x4 ra_reg[8], rb_reg[8];
    auto gload = [&](int ks) {
        const uint32_t ao = (uint32_t)ks * a_kstep, bo = (uint32_t)ks * b_kstep;
#pragma unroll
        for (int i = 0; i < 8; ++i) ra_reg[i] = bload(ra, va[i] + ao);
#pragma unroll
        for (int i = 0; i < 8; ++i) rb_reg[i] = bload(rb, vb[i] + bo);
    };
    auto lstore = [&](int buf) {
        char* sA = smem + (2 * buf) * 256 * 128;
        char* sB = smem + (2 * buf + 1) * 256 * 128;
        if (A_K) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                st16(sA + lds_off(0, (tid >> 3) + 32 * i, tid & 7), ra_reg[i]);
        } else {
            u32x4 t[8];
            transpose8x8(ra_reg, t);
#pragma unroll
            for (int mm = 0; mm < 8; ++mm) st16(sA + lds_off(0, (tid & 31) * 8 + mm, tid >> 5), t[mm]);
        }
        if (B_K) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                st16(sB + lds_off(0, (tid >> 3) + 32 * i, tid & 7), rb_reg[i]);
        } else {
            u32x4 t[8];
            transpose8x8(rb_reg, t);
#pragma unroll
            for (int mm = 0; mm < 8; ++mm) st16(sB + lds_off(0, (tid & 31) * 8 + mm, tid >> 5), t[mm]);
        }
    };

    const int nk = cdiv(Kdim, BK);
    if (nk > 0) {
        gload(0);
        lstore(0);
    }
    __syncthreads();
    for (int ks = 0; ks < nk; ++ks) {
        const int buf = ks & 1;
        if (ks + 1 < nk) gload(ks + 1);
        const char* sA = smem + (2 * buf) * 256 * 128;
        const char* sB = smem + (2 * buf + 1) * 256 * 128;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            bf16x8 af[4], bfr[4];
            const int chunk = kk * 2 + (lane >> 5);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = *reinterpret_cast<const bf16x8*>(sA + lds_off(0, wm * 128 + i * 32 + (lane & 31), chunk));
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8*>(sB + lds_off(0, wn * 128 + j * 32 + (lane & 31), chunk));
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if (ks + 1 < nk) lstore(buf ^ 1);
        __syncthreads();
    }

    // ---------------------------------------------------------------- epilogue
    // Accumulator layout of v_mfma_f32_32x32x16: lane l holds column l%32 and rows
    // 8*(v/4) + 4*(l/32) + v%4 of its 32x32 tile, v = 0..15.
    const int lc = lane & 31, lr = (lane >> 5) * 4;
    if (EPI == EPI_STORE) {
        bf16_t* C = g.C + e * g.c_es + (GK ? 0 : (int64_t)row0 * g.ldc);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = n0 + wn * 128 + j * 32 + lc;
                const bool cok = col < g.N;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int row = m0 + wm * 128 + i * 32 + (v >> 2) * 8 + lr + (v & 3);
                    const float val = acc[i][j][v];
                    if (cok && row < Mvalid) C[(int64_t)row * g.ldc + col] = f2bf(val);
                }
            }
    } else if (EPI == EPI_SWIGLU) {
        bf16_t* C = g.C + e * g.c_es + (int64_t)row0 * g.ldc;
        bf16_t* C2 = g.C2 ? g.C2 + e * g.c2_es + (int64_t)row0 * g.ldc2 : nullptr;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int ch = ch0 + wn * 64 + j * 32 + lc;
                const bool cok = ch < g.I;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int row = m0 + wm * 128 + i * 32 + (v >> 2) * 8 + lr + (v & 3);
                    const float gv = acc[i][j][v], uv = acc[i][j + 2][v];
                    const float hv = gv / (1.0f + __expf(-gv)) * uv;
                    if (cok && row < Mvalid) {
                        C[(int64_t)row * g.ldc + ch] = f2bf(hv);
                        if (C2) {
                            C2[(int64_t)row * g.ldc2 + ch] = f2bf(gv);
                            C2[(int64_t)row * g.ldc2 + g.I + ch] = f2bf(uv);
                        }
                    }
                }
            }
    } else {  // EPI_DSWIGLU: acc = dh; read saved g|u, write dg|du
        bf16_t* C = g.C + e * g.c_es + (int64_t)row0 * g.ldc;
        const bf16_t* GU = g.C2 + e * g.c2_es + (int64_t)row0 * g.ldc2;
#pragma clang loop unroll(full)
        for (int i = 0; i < 4; ++i)
#pragma clang loop unroll(full)
            for (int j = 0; j < 4; ++j) {
                const int ch = n0 + wn * 128 + j * 32 + lc;
                const bool cok = ch < g.N;
#pragma clang loop unroll(full)
                for (int v = 0; v < 16; ++v) {
                    const int row = m0 + wm * 128 + i * 32 + (v >> 2) * 8 + lr + (v & 3);
                    const float dh = acc[i][j][v];
                    const bool ok = cok && row < Mvalid;
                    // clamped (always in-bounds) reads keep the loop branch-free
                    const int64_t gro = (int64_t)(ok ? row : 0) * g.ldc2 + (cok ? ch : 0);
                    const float gv = bf2f(GU[gro]);
                    const float uv = bf2f(GU[gro + g.I]);
                    const float sg = 1.0f / (1.0f + __expf(-gv));
                    const float dg = dh * uv * sg * (1.0f + gv * (1.0f - sg));
                    const float du = dh * gv * sg;
                    if (ok) {
                        C[(int64_t)row * g.ldc + ch] = f2bf(dg);
                        C[(int64_t)row * g.ldc + g.I + ch] = f2bf(du);
                    }
                }
            }
    }
}

// One kernel symbol per product of the layer, so that profiles name each role.
#define MOE_GEMM_KERNEL(NAME, AK, BK, EPI, GK)                                         \
    __global__ __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(1, 1))) void \
    NAME(GemmArgs g) {                                                                 \
        gemm_body<AK, BK, EPI, GK>(g);                                                 \
    }
MOE_GEMM_KERNEL(gemm1_swiglu, true, true, EPI_SWIGLU, false)     // [g|u] = Xp W1^T, h
MOE_GEMM_KERNEL(gemm2_down, true, true, EPI_STORE, false)        // y = h W2^T
MOE_GEMM_KERNEL(dgrad_down_dswiglu, true, false, EPI_DSWIGLU, false)  // dh = dy W2 -> dg|du
MOE_GEMM_KERNEL(dgrad_gate_up, true, false, EPI_STORE, false)    // dXp = dGU W1
MOE_GEMM_KERNEL(wgrad_down, false, false, EPI_STORE, true)       // dW2 = dy^T h
MOE_GEMM_KERNEL(wgrad_gate_up, false, false, EPI_STORE, true)    // dW1 = dGU^T Xp
#undef MOE_GEMM_KERNEL

// Upper bound on the tile count of a ragged-M product (host side, no device data).
static int ragged_tiles_bound(int R, int E, int NT) {
    int64_t mt = ((int64_t)R + (int64_t)E * (BM - 1)) / BM;
    return (int)(mt * NT);
}

template <int EPI, bool GK>
static int launch(void (*kern)(GemmArgs), const char* name, const GemmArgs& g, hipStream_t st) {
    int NT = (EPI == EPI_SWIGLU) ? cdiv(g.I, 128) : cdiv(g.N, BN);
    int grid;
    if (GK) grid = g.total;
    else if (g.offsets) grid = ragged_tiles_bound(g.R, g.E, NT);
    else grid = g.total;
    if (grid <= 0) return MOE_OK;
    MOE_TRACED(name, st, kern<<<grid, NTH, 0, st>>>(g));
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

static GemmArgs blank() {
    GemmArgs g{};
    return g;
}

}  // namespace moe

using namespace moe;

// ---------------------------------------------------------------------- internal API
// Forward FFN in BF16.  offsets == null: shared mode (every expert takes all R rows).
int moe_ffn_bf16(const bf16_t* xp, const int32_t* offsets, int E, int R, int H, int I,
                 const bf16_t* w1, const bf16_t* w2, bf16_t* gu, bf16_t* h, bf16_t* y,
                 hipStream_t st) {
    const bool shared = offsets == nullptr;
    GemmArgs g = blank();
    g.A = xp; g.a_es = 0; g.lda = H;
    g.B = w1; g.b_es = (int64_t)2 * I * H; g.ldb = H; g.b_rows = 2 * I;
    g.C = h; g.c_es = shared ? (int64_t)R * I : 0; g.ldc = I;
    g.C2 = gu; g.c2_es = shared ? (int64_t)R * 2 * I : 0; g.ldc2 = 2 * I;
    g.offsets = offsets; g.E = E; g.R = R; g.N = 2 * I; g.K = H; g.I = I;
    g.total = shared ? E * cdiv(R, BM) * cdiv(I, 128) : 0;
    int rc = launch<EPI_SWIGLU, false>(gemm1_swiglu, "gemm1_swiglu", g, st);
    if (rc) return rc;
    GemmArgs g2 = blank();
    g2.A = h; g2.a_es = shared ? (int64_t)R * I : 0; g2.lda = I;
    g2.B = w2; g2.b_es = (int64_t)H * I; g2.ldb = I; g2.b_rows = H;
    g2.C = y; g2.c_es = shared ? (int64_t)R * H : 0; g2.ldc = H;
    g2.offsets = offsets; g2.E = E; g2.R = R; g2.N = H; g2.K = I; g2.I = I;
    g2.total = shared ? E * cdiv(R, BM) * cdiv(H, BN) : 0;
    return launch<EPI_STORE, false>(gemm2_down, "gemm2_down", g2, st);
}

// Backward of the FFN for one group of experts.
//   dy [rows,H] (shared mode: one [R,H] gradient used by every expert, dy_shared = true)
//   gu, h: saved forward values; xp: forward input rows (shared mode: one [R,H] input).
//   Outputs dgu (workspace) [rows,2I], dxp [rows,H], dw1 [E,2I,H], dw2 [E,H,I].
int moe_ffn_bwd_bf16(const bf16_t* xp, const int32_t* offsets, int E, int R, int H, int I,
                     const bf16_t* w1, const bf16_t* w2, const bf16_t* gu, const bf16_t* h,
                     const bf16_t* dy, bf16_t* dgu, bf16_t* dxp, bf16_t* dw1, bf16_t* dw2,
                     hipStream_t st) {
    const bool shared = offsets == nullptr;
    int rc;
    {   // dh = dy_e W2_e (W2_e is [H,I]: N-contiguous in I), SwiGLU backward -> dgu
        GemmArgs g = blank();
        g.A = dy; g.a_es = 0; g.lda = H;
        g.B = w2; g.b_es = (int64_t)H * I; g.ldb = I; g.b_rows = H;
        g.C = dgu; g.c_es = shared ? (int64_t)R * 2 * I : 0; g.ldc = 2 * I;
        g.C2 = const_cast<bf16_t*>(gu); g.c2_es = shared ? (int64_t)R * 2 * I : 0; g.ldc2 = 2 * I;
        g.offsets = offsets; g.E = E; g.R = R; g.N = I; g.K = H; g.I = I;
        g.total = shared ? E * cdiv(R, BM) * cdiv(I, BN) : 0;
        rc = launch<EPI_DSWIGLU, false>(dgrad_down_dswiglu, "dgrad_down_dswiglu", g, st);
        if (rc) return rc;
    }
    {   // dXp = dGU_e W1_e (W1_e is [2I,H]: N-contiguous in H)
        GemmArgs g = blank();
        g.A = dgu; g.a_es = shared ? (int64_t)R * 2 * I : 0; g.lda = 2 * I;
        g.B = w1; g.b_es = (int64_t)2 * I * H; g.ldb = H; g.b_rows = 2 * I;
        g.C = dxp; g.c_es = shared ? (int64_t)R * H : 0; g.ldc = H;
        g.offsets = offsets; g.E = E; g.R = R; g.N = H; g.K = 2 * I; g.I = I;
        g.total = shared ? E * cdiv(R, BM) * cdiv(H, BN) : 0;
        rc = launch<EPI_STORE, false>(dgrad_gate_up, "dgrad_gate_up", g, st);
        if (rc) return rc;
    }
    {   // dW2_e = dy_e^T h_e: M = H, N = I, K = the expert's rows
        GemmArgs g = blank();
        g.A = dy; g.a_es = 0; g.lda = H;
        g.B = h; g.b_es = shared ? (int64_t)R * I : 0; g.ldb = I;
        g.C = dw2; g.c_es = (int64_t)H * I; g.ldc = I;
        g.offsets = offsets; g.E = E; g.R = R; g.M = H; g.N = I; g.I = I;
        g.total = E * cdiv(H, BM) * cdiv(I, BN);
        rc = launch<EPI_STORE, true>(wgrad_down, "wgrad_down", g, st);
        if (rc) return rc;
    }
    {   // dW1_e = dGU_e^T Xp_e: M = 2I, N = H
        GemmArgs g = blank();
        g.A = dgu; g.a_es = shared ? (int64_t)R * 2 * I : 0; g.lda = 2 * I;
        g.B = xp; g.b_es = 0; g.ldb = H;
        g.C = dw1; g.c_es = (int64_t)2 * I * H; g.ldc = H;
        g.offsets = offsets; g.E = E; g.R = R; g.M = 2 * I; g.N = H; g.I = I;
        g.total = E * cdiv(2 * I, BM) * cdiv(H, BN);
        rc = launch<EPI_STORE, true>(wgrad_gate_up, "wgrad_gate_up", g, st);
        if (rc) return rc;
    }
    return MOE_OK;
}
