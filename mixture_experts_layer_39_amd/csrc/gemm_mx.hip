// MXFP8 grouped GEMMs of the expert FFN forward (E4M3 codes, one E8M0 scale per 32 values
// along K) on gfx950's scaled MFMA, v_mfma_scale_f32_32x32x64_f8f6f4.  The MXFP8 forward is
// the path the pages report the largest gain on (pulsen.vercel.app, "Cursor åpner
// megakernelen…", ¶3; aiexpert.news, "Megakernels are dead and back", ¶4).
//   GEMM1: [g|u] = Xq_e W1q_e^T, epilogue h = silu(g)*u in fp32.
//   GEMM2: y = hq_e W2q_e^T, bf16 output (h MX-quantised along I in between).
//
// The pipeline of the BF16 kernels for byte codes: 256x256 tiles, 4 waves of 128x128, K steps
// of 128 codes (a 128-byte LDS row per operand row: the bytes, swizzle and load map of a
// 64-wide BF16 step) in the ring of five 32 KB operand slots, filled by direct global-to-LDS
// loads spread over the step; buffer loads that zero-fill past an expert's rows;
// device-side expert tile lists; tiles in launch order.
//
// Scales.  The five slots take all 160 KB of LDS, so the E8M0 scales go straight to
// registers.  Per K step and sub-tile a lane needs the scales of one row in two of the step's
// four 32-code blocks; read from the [rows, K/32] layout those bytes are scattered over 32
// rows per instruction.  A pre-pass therefore lays the scales of every 128-row operand panel
// out per K step in the order the 64 lanes consume them (8 bytes per lane, one 512-byte run
// per panel and step), and the K loop fetches them with one 8-byte load per lane and operand
// per step, two steps ahead.  GEMM1's epilogue writes the panels of h for GEMM2 directly.
#include "mx_dev.h"
#include "pipe.h"

namespace moe {

constexpr int XBM = 256, XBN = 256, XNTH = 256;
constexpr int XBK = 128;                 // codes (bytes) per K step
constexpr int XGM = 2;                   // M tiles per group of the launch order (as the
                                         // BF16 products: fewer panels per XCD than 4)
typedef Pipe<64> XP;                     // 128-byte rows: the LDS layout of a 64-wide BF16 step
constexpr int XOPB = XP::OPB;            // bytes of one operand step (one slot)
constexpr int XLPW = XP::LPW;            // direct loads per operand per wave per step
constexpr int SPAN = 512;                // bytes of one panel's scales for one K step

enum { XEPI_SWIGLU_MX = 0, XEPI_STORE_BF16 = 1, XEPI_DSWIGLU = 2 };

struct MxArgs {
    const uint8_t* A;    // codes [rows, K]
    const uint8_t* At;   // panel scales of A: [A panels][K/128][512]
    int64_t a_es;        // per-expert row stride (shared mode), in rows
    const uint8_t* B;    // codes [E, b_rows, K]
    const uint8_t* Bt;   // panel scales of B: [E][NT][2][K/128][512]
    int b_rows;
    void* C;             // store: bf16 y [rows, N];  SwiGLU backward: bf16 dg|du [rows, 2I]
    uint8_t* Cq;         // SwiGLU: h's E4M3 codes [rows, I] (MX-quantised along I in the epilogue)
    uint8_t* Cs;         // SwiGLU: h's E8M0 scales [rows, I/32]
    bf16_t* Ch;          // SwiGLU: h as the codes hold it, bf16 [rows, I], or null
    int64_t c_es;        // per-expert row stride of C / Cq / Ch (shared mode), in rows
    int ldc;
    bf16_t* C2;          // SwiGLU: bf16 g|u save [rows, 2I] or null;  SwiGLU backward: the
                         // saved g|u (read)
    int ldc2;
    const int32_t* offsets;
    int E, R, N, K, I;
    int total;           // tile count when static (shared mode, weight gradients)
    int M;               // weight gradients: rows of A (static); K is then the row stride of
                         // the token-axis operands and each expert takes its own code columns
    int bound;           // blocks a pair launch gives this product (dgrad: the host's upper
                         // bound of its tiles; the blocks past the device count exit)
    uint8_t* Ph;         // SwiGLU: the down projection's panel scales of h [A panels][I/128]
                         // [512], written by the epilogue, or null
};

struct alignas(1024) MxSmem {
    char st[5 * XOPB];   // the five operand slots
};

template <int EPI>
__host__ __device__ __forceinline__ int mx_n_tiles(int N, int I) {
    return (EPI == XEPI_SWIGLU_MX) ? cdiv(I, 128) : cdiv(N, XBN);
}

// tile row nn -> B row.  SwiGLU: a tile holds gate and up rows of 128 channels; each
// 32-column MFMA block takes 16 channels, gate in its columns 0-15 and up in 16-31.
template <int EPI>
__device__ __forceinline__ int mx_brow(int nn, int n0, int ch0, int I) {
    if (EPI == XEPI_SWIGLU_MX)
        return ((nn >> 4) & 1) * I + ch0 + (nn >> 7) * 64 + ((nn & 127) >> 5) * 16 + (nn & 15);
    return n0 + nn;
}

// Ragged-M products: every wave scans the per-expert tile counts (NT tiles per 256-row M
// tile) itself, 64 experts at a time.  Returns the tile count; with `logical` >= 0 it finds
// the expert owning tile `logical` and that expert's first tile instead.
__device__ __forceinline__ int mx_ragged_scan(const int32_t* offsets, int E, int R, int NT,
                                              int logical, int* e_out, int* first_out) {
    const int lane = threadIdx.x & 63;
    int run = 0;
    for (int base = 0; base < E; base += 64) {
        const int e = base + lane;
        int tiles = 0;
        if (e < E) {
            const int lo = min(max(offsets[e], 0), R);
            const int hi = min(max(offsets[e + 1], lo), R);
            tiles = cdiv(hi - lo, XBM) * NT;
        }
        const int inc = wave_incl_scan(tiles) + run;
        if (logical >= 0) {
            const uint64_t m = __ballot(e < E && inc > logical);
            if (m) {
                const int l = __ffsll((unsigned long long)m) - 1;
                *e_out = base + l;
                *first_out = __shfl(inc - tiles, l, 64);
                return -1;
            }
        }
        run = __shfl(inc, 63, 64);
    }
    return run;
}

// ---------------------------------------------------------------- panel scales
// For the panel rows prow(32 t + l) (t = 0..3, l = 0..31) and K step s, byte 8 L + 2 t + kk of
// the step's 512-byte run (lane L = 32 g + l) holds the scale of row prow(32 t + l) in the
// 32-code block 4 s + 2 kk + g; rows outside the operand give 0.  In the scaled MFMA, lane
// group g supplies the scale of block g of its 64-code sub-step.

// One block per 256-row tile of an operand (both of its 128-row panels) and 64 scale
// columns (16 K steps): the tile's scale rows pass through LDS, loaded with dword loads along
// the rows, so that the gather of single bytes into lane order runs on LDS.
constexpr int PS_COLS = 64;  // scale columns (bytes) staged per pass

__device__ __forceinline__ void panel_tile(const uint8_t* __restrict__ sc, int KB, int nsteps,
                                           const int* srow, uint8_t* __restrict__ out,
                                           uint8_t (*stg)[PS_COLS + 4]) {
    const int tid = threadIdx.x;
    {
        const int c0 = (int)blockIdx.y * PS_COLS;
        __syncthreads();  // srow written
        // 256 rows x 16 dwords: thread i loads dword i % 16 of row i / 16 (+16 rows per pass);
        // all 16 loads of a thread are issued before its first LDS store
        constexpr int NLD = PS_COLS / 4;
        uint32_t v[NLD];
#pragma unroll
        for (int u = 0; u < NLD; ++u) {
            const int i = tid + 256 * u;
            const int row = i / (PS_COLS / 4), col = c0 + 4 * (i % (PS_COLS / 4));
            const int rr = srow[row];
            v[u] = (rr >= 0 && col < KB) ? *reinterpret_cast<const uint32_t*>(sc + (int64_t)rr * KB + col)
                                         : 0u;
        }
#pragma unroll
        for (int u = 0; u < NLD; ++u) {
            const int i = tid + 256 * u;
            const int row = i / (PS_COLS / 4), col = 4 * (i % (PS_COLS / 4));
            *reinterpret_cast<uint32_t*>(&stg[row][col]) = v[u];
        }
        __syncthreads();
        // entries (half w, step s, lane L): 2 x 16 x 64 per pass, 8 per thread
        const int s0 = c0 / 4;
        for (int i = tid; i < 2 * (PS_COLS / 4) * 64; i += 256) {
            const int L = i & 63, ds = (i >> 6) % (PS_COLS / 4), w = i / (64 * (PS_COLS / 4));
            const int s = s0 + ds;
            if (s >= nsteps) continue;
            const int l = L & 31, g = L >> 5;
            uint32_t wd[2] = {0u, 0u};
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const int col = 4 * ds + 2 * kk + g;
                    const uint32_t v = (c0 + col < KB) ? stg[w * 128 + 32 * t + l][col] : 0u;
                    wd[t >> 1] |= v << (8 * (2 * (t & 1) + kk));
                }
            *reinterpret_cast<uint2*>(out + ((int64_t)w * nsteps + s) * SPAN + 8 * L) =
                make_uint2(wd[0], wd[1]);
        }
    }
}

// A operand: tile `bx` (a 256-row M tile), panels 2 bx + half.
__device__ __forceinline__ void panel_a(int bx, const uint8_t* __restrict__ sc,
                                        const int32_t* __restrict__ offsets, int E, int R,
                                        int64_t a_es, int KB, int nsteps, int total_static,
                                        uint8_t* __restrict__ out, uint8_t (*stg)[PS_COLS + 4],
                                        int* srow) {
    int e, tm, row0, M;
    if (offsets) {
        const int total = uni(mx_ragged_scan(offsets, E, R, 1, -1, nullptr, nullptr));
        if (bx >= total) return;
        int ee = 0, first = 0;
        mx_ragged_scan(offsets, E, R, 1, bx, &ee, &first);
        e = uni(ee);
        tm = uni(bx - first);
        const int a = min(max(offsets[e], 0), R);
        const int b = min(max(offsets[e + 1], a), R);
        row0 = a;
        M = b - a;
    } else {
        if (bx >= total_static) return;
        const int MT = cdiv(R, XBM);
        e = bx / MT;
        tm = bx % MT;
        row0 = 0;
        M = R;
    }
    const int rr = tm * XBM + (int)threadIdx.x;
    srow[threadIdx.x] = rr < M ? (int)((int64_t)e * a_es + row0 + rr) : -1;
    panel_tile(sc, KB, nsteps, srow, out + (int64_t)(2 * bx) * nsteps * SPAN, stg);
}

// B operand: tile `bx` = e NT + tn, panels 2 bx + half.
template <int EPI>
__device__ __forceinline__ void panel_b(int bx, const uint8_t* __restrict__ sc, int b_rows, int N,
                                        int I, int KB, int nsteps, uint8_t* __restrict__ out,
                                        uint8_t (*stg)[PS_COLS + 4], int* srow) {
    const int NT = mx_n_tiles<EPI>(N, I);
    const int e = bx / NT, tn = bx % NT;
    const int rr = mx_brow<EPI>((int)threadIdx.x, tn * XBN, tn * 128, I);
    srow[threadIdx.x] = rr < b_rows ? (int)((int64_t)e * b_rows + rr) : -1;
    panel_tile(sc, KB, nsteps, srow, out + (int64_t)(2 * bx) * nsteps * SPAN, stg);
}

struct PanelJobs {
    // A panels of GEMM1 (xp scales), B panels of both GEMMs (weight scales)
    const uint8_t* xs; const int32_t* offsets; int E, R, H, I, na, total_static;
    const uint8_t* w1s; const uint8_t* w2s;
    uint8_t* pa1; uint8_t* pb1; uint8_t* pb2;
};

// One launch for the panels known before GEMM1: x blocks [0, na) A panels of xp, then E NT1
// B panels of W1, then E NT2 B panels of W2; y blocks: 64-column chunks of each operand's
// scales (blocks past an operand's chunks exit).  GEMM2's A panels (h's scales) come from
// GEMM1's epilogue.
__global__ __launch_bounds__(256) void mx_panel_scales_pre(PanelJobs j) {
    __shared__ uint8_t stg[256][PS_COLS + 4];
    __shared__ int srow[256];
    const int nb1 = j.E * mx_n_tiles<XEPI_SWIGLU_MX>(2 * j.I, j.I);
    const int bx = blockIdx.x;
    const int KBh = j.H / 32, KBi = j.I / 32;
    if (bx < j.na) {
        if ((int)blockIdx.y * PS_COLS >= KBh) return;
        panel_a(bx, j.xs, j.offsets, j.E, j.R, 0, KBh, j.H / XBK, j.total_static, j.pa1, stg, srow);
    } else if (bx < j.na + nb1) {
        if ((int)blockIdx.y * PS_COLS >= KBh) return;
        panel_b<XEPI_SWIGLU_MX>(bx - j.na, j.w1s, 2 * j.I, 2 * j.I, j.I, KBh, j.H / XBK, j.pb1,
                                 stg, srow);
    } else {
        if ((int)blockIdx.y * PS_COLS >= KBi) return;
        panel_b<XEPI_STORE_BF16>(bx - j.na - nb1, j.w2s, j.H, j.H, j.I, KBi, j.I / XBK, j.pb2,
                                 stg, srow);
    }
}

// The panels of one product of the backward: x blocks [0, na) the A panels -- ragged rows
// from the offsets, or (offsets null) R static rows -- then EB * b_rows/256 B panels of
// operands with plain rows; y blocks: 64-column chunks of the scales.
__global__ __launch_bounds__(256) void mx_panel_scales_ab(const uint8_t* __restrict__ as,
                                                          const int32_t* __restrict__ offsets,
                                                          int E, int R, int na,
                                                          const uint8_t* __restrict__ bs,
                                                          int b_rows, int K,
                                                          uint8_t* __restrict__ pa,
                                                          uint8_t* __restrict__ pb) {
    __shared__ uint8_t stg[256][PS_COLS + 4];
    __shared__ int srow[256];
    if ((int)blockIdx.y * PS_COLS >= K / 32) return;
    const int bx = blockIdx.x;
    if (bx < na)
        panel_a(bx, as, offsets, offsets ? E : 1, R, 0, K / 32, K / XBK, offsets ? 0 : na, pa,
                stg, srow);
    else
        panel_b<XEPI_STORE_BF16>(bx - na, bs, b_rows, b_rows, 0, K / 32, K / XBK, pb, stg, srow);
}

// 8 bytes per lane straight to registers, issued through inline asm like the LDS loads so that
// the pipeline's explicit wait counts cover both.  The registers are read only after a wait
// that covers the load, followed by `settle`, which redefines the value for the compiler.
// Like lds_load16, the asm carries the wait states after a VALU write of an SGPR it reads.
__device__ __forceinline__ void vgpr_load8(uint2& dst, rsrc_t r, uint32_t voff, uint32_t soff) {
    asm volatile("s_nop 4\n\tbuffer_load_dwordx2 %0, %1, %2, %3 offen"
                 : "=v"(dst)
                 : "v"(voff), "s"(r), "s"(soff)
                 : "memory");
}
__device__ __forceinline__ void settle(uint2& v) { asm volatile("" : "+v"(v)); }

// Token-axis operands of the weight gradients: expert e's code columns start at P_e, the sum
// of the padded (whole K step) row counts of the experts before it, and span pad(cnt_e).
__device__ __forceinline__ void mx_token_range(const int32_t* offsets, int E, int R, int e,
                                               int* P, int* span) {
    const int lane = threadIdx.x & 63;
    int run = 0;
    for (int base = 0; base < e; base += 64) {
        const int x = base + lane;
        int v = 0;
        if (x < e) {
            const int lo = min(max(offsets[x], 0), R);
            const int hi = min(max(offsets[x + 1], lo), R);
            v = cdiv(hi - lo, XBK) * XBK;
        }
        run += __shfl(wave_incl_scan(v), 63, 64);
    }
    const int lo = min(max(offsets[e], 0), R);
    const int hi = min(max(offsets[e + 1], lo), R);
    *P = run;
    *span = cdiv(hi - lo, XBK) * XBK;
}

// ---------------------------------------------------------------- one output tile
// GK: a weight-gradient tile (expert e, static M x N, K = the expert's token columns).
template <int EPI, bool GK = false>
__device__ __forceinline__ void mx_tile(const MxArgs& g, MxSmem& sm, const int logical) {
    const int tid = threadIdx.x, lane = tid & 63, wid = uni(tid >> 6);
    const int wm = wid >> 1, wn = wid & 1;
    const int NT = mx_n_tiles<EPI>(g.N, g.I);
    const int K = g.K;  // row stride of the codes
    int nk = K / XBK, kbase = 0;

    int e, t_local, Mrows, row0, mt_first;
    if (GK) {
        const int per = cdiv(g.M, XBM) * NT;
        e = logical / per;
        t_local = logical - e * per;
        mt_first = 0;
        row0 = 0;
        Mrows = g.M;
        int P = 0, span = 0;
        mx_token_range(g.offsets, g.E, g.R, e, &P, &span);
        kbase = uni(P);
        nk = uni(span / XBK);
    } else if (g.offsets) {
        int ee = 0, first = 0;
        mx_ragged_scan(g.offsets, g.E, g.R, NT, logical, &ee, &first);
        e = uni(ee);
        t_local = uni(logical - first);
        mt_first = uni(first / NT);  // M tiles of the experts before e
        int a = min(max(g.offsets[e], 0), g.R);
        int b = min(max(g.offsets[e + 1], a), g.R);
        row0 = uni(a);
        Mrows = uni(b - a);
    } else {
        int per = cdiv(g.R, XBM) * NT;
        e = logical / per;
        t_local = logical - e * per;
        mt_first = e * cdiv(g.R, XBM);
        row0 = 0;
        Mrows = g.R;
    }
    const int MT = cdiv(Mrows, XBM);
    int tm, tn;
    {
        int grp = t_local / (XGM * NT);
        int first = grp * XGM;
        int gsz = min(MT - first, XGM);
        int rr = t_local - grp * XGM * NT;
        tm = first + rr % gsz;
        tn = rr / gsz;
    }
    const int m0 = tm * XBM, n0 = tn * XBN, ch0 = tn * 128;
    // the row block's index among all 256-row blocks of the call (its panels)
    const int mblock = mt_first + tm;

    // ---------------------------------------------------------------- operands
    // codes: the K-major load map of a 64-wide BF16 step (128-byte rows; ld in 2-byte units)
    const int64_t arow = GK ? (int64_t)m0 : (int64_t)e * g.a_es + row0 + m0;
    const uint32_t arows = (uint32_t)max(Mrows - m0, 0);
    // GK: the operands start at the expert's first code column of their shared rows
    const uint32_t aspan = arows ? arows * (uint32_t)K - (uint32_t)kbase : 0u;
    Operand oa, ob;
    setup_kmajor<64>(oa, g.A + arow * K + kbase, aspan, K / 2, wid, lane, wm * 128,
                     [](int r) { return r; }, 2 * XP::RPI, 4 * XP::RPI);
    const int I = g.I;
    setup_kmajor<64>(ob, GK ? g.B + kbase : g.B + (int64_t)e * g.b_rows * K,
                     (uint32_t)g.b_rows * (uint32_t)K - (uint32_t)kbase, K / 2,
                     wid, lane, wn * 128, [=](int nn) { return mx_brow<EPI>(nn, n0, ch0, I); },
                     EPI == XEPI_SWIGLU_MX ? I : 2 * XP::RPI,
                     EPI == XEPI_SWIGLU_MX ? 16 : 4 * XP::RPI);
    // panel scales of this wave's A rows and B rows
    const uint32_t pbytes = (uint32_t)nk * SPAN;
    // GK: panels over the whole token axis (K / 128 steps each); the expert's steps start at
    // its first code column
    const int64_t pstride = GK ? (int64_t)(K / XBK) * SPAN : (int64_t)pbytes;
    const int64_t pfirst = GK ? (int64_t)(kbase / XBK) * SPAN : 0;
    const rsrc_t rsa =
        make_rsrc(g.At + (int64_t)(2 * (mt_first + tm) + wm) * pstride + pfirst, pbytes);
    const rsrc_t rsb = make_rsrc(
        g.Bt + (int64_t)(2 * ((GK ? 0 : e * NT) + tn) + wn) * pstride + pfirst, pbytes);
    const uint32_t lso = (uint32_t)lane * 8u;
    const rsrc_t rnull = make_rsrc(nullptr, 0);

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    // ---------------------------------------------------------------- main loop
    // Slots as in the BF16 kernel: A of step s in slot 2s mod 5, B in slot 2s+1 mod 5; A(s+2)
    // goes into the slot B(s-1) left at the previous step's barrier, B(s+2) into the slot A(s)
    // leaves at this step's barrier.  A step is two sub-steps of 16 scaled MFMAs (64 codes
    // each).  Loads of step s:
    //   sub-step 0: A(s+2), then the scales of step s+2
    //   barrier (A(s+1), B(s+1) and the scales of s+1 landed; every read of step s done)
    //   sub-step 1: B(s+2)
    // so every load has at least one whole sub-step to land before the barrier that waits for
    // it (splitting B over two steps, as the four-sub-step BF16 step does, left the second
    // half of B(s+1) only the rest of the sub-step it was issued in).
    // The scales of steps s, s+1, s+2 live in three register sets, so the loop is unrolled
    // over lcm(5, 3) = 15 steps; at its back edge the set in flight is waited for, so that no
    // register still being written crosses it.
    i32x8 fa[2][4], fb[2][4];
    uint2 sca[3], scb[3];
    // fragment r (0..7) of sub-step kk, in MFMA consumption order a0 b0 b1 b2 b3 a1 a2 a3:
    // 32 codes per lane, chunks 4 kk + g and 4 kk + 2 + g of the row (g = lane / 32)
    auto read_ab = [&](const char* sa_, const char* sb_, int kk, int f, int r) __attribute__((always_inline)) {
        const bool isa = (r == 0 || r >= 5);
        const int t = r == 0 ? 0 : (r <= 4 ? r - 1 : r - 4);
        const Operand& o = isa ? oa : ob;
        const char* base = (isa ? sa_ : sb_) + t * 32 * XP::KROW;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(base + o.rd[2 * kk]);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(base + o.rd[2 * kk + 1]);
        const i32x8 v = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                         (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        if (isa) fa[f][t] = v;
        else fb[f][t] = v;
    };
    // MFMA n of sub-step kk with fragment set f and scale set c: the scale of sub-tile t is
    // byte 2 (t % 2) + kk of dword t / 2 (the MFMA's opsel operand picks the byte)
    auto mfma_one = [&](int f, int kk, int c, int n) __attribute__((always_inline)) {
        const int i = n >> 2, j = n & 3;
        const int sa_w = (i >> 1) ? (int)sca[c].y : (int)sca[c].x;
        const int sb_w = (j >> 1) ? (int)scb[c].y : (int)scb[c].x;
        const int pa = 2 * (i & 1) + kk, pb = 2 * (j & 1) + kk;
#define MX_MFMA(PA, PB)                                                                       \
    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[f][j], fa[f][i], acc[i][j], \
                                                               0, 0, PB, sb_w, PA, sa_w)
#define MX_ROW(PA)                         \
    if (pb == 0) MX_MFMA(PA, 0);           \
    else if (pb == 1) MX_MFMA(PA, 1);      \
    else if (pb == 2) MX_MFMA(PA, 2);      \
    else MX_MFMA(PA, 3);
        if (pa == 0) { MX_ROW(0) }
        else if (pa == 1) { MX_ROW(1) }
        else if (pa == 2) { MX_ROW(2) }
        else { MX_ROW(3) }
#undef MX_ROW
#undef MX_MFMA
    };
    auto codes_src = [&](int ks, rsrc_t& ra_, rsrc_t& rb_, uint32_t& so) __attribute__((always_inline)) {
        const bool live = ks < nk;
        ra_ = live ? oa.r : rnull;
        rb_ = live ? ob.r : rnull;
        so = live ? (uint32_t)ks * XBK : 0u;
    };
    auto load_scales = [&](int ks, int c) __attribute__((always_inline)) {
        const bool live = ks < nk;
        const uint32_t so = live ? (uint32_t)ks * SPAN : 0u;
        vgpr_load8(sca[c], live ? rsa : rnull, lso, so);
        vgpr_load8(scb[c], live ? rsb : rnull, lso, so);
    };
    auto kstep = [&](int u, int ks) __attribute__((always_inline)) {
        const int su = u % 5, c = u % 3;
        char* const cA = sm.st + ((2 * su) % 5) * XOPB;
        char* const cB = sm.st + ((2 * su + 1) % 5) * XOPB;
        char* const nA = sm.st + ((2 * su + 2) % 5) * XOPB;
        char* const nB = sm.st + ((2 * su + 3) % 5) * XOPB;
        const uint32_t base32 = lds_addr(sm.st);
        const uint32_t lA = base32 + ((2 * su + 4) % 5) * XOPB;   // A(ks+2): slot of B(ks-1)
        const uint32_t lB = base32 + ((2 * su) % 5) * XOPB;       // B(ks+2): slot of A(ks)
        rsrc_t ra_, rb_;
        uint32_t so;
        codes_src(ks + 2, ra_, rb_, so);
        __builtin_amdgcn_sched_barrier(0);
        // sub-step 0: fragment reads of sub-step 1; the 8 code loads of A(ks+2), then the
        // scales of ks+2
#pragma unroll
        for (int n = 0; n < 16; ++n) {
            mfma_one(0, 0, c, n);
            if ((n & 1) == 0) read_ab(cA, cB, 1, 1, n / 2);
            else issue_load<64>(oa, lA, wid, n / 2, ra_, so);
            if (n == 15) load_scales(ks + 2, (u + 2) % 3);
            __builtin_amdgcn_sched_barrier(0);
        }
        wait_vm_lgkm0<XLPW + 2>();  // all but A(ks+2) and its scales
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        settle(sca[(u + 1) % 3]);
        settle(scb[(u + 1) % 3]);
        // sub-step 1: fragment reads of the next step's sub-step 0; the 8 code loads of B(ks+2).
        // The reads run in the last step too (of slots inside LDS, values unused): a read
        // under a condition makes the compiler carry each fragment's old value through
        // register copies into MFMA source registers.
#pragma unroll
        for (int n = 0; n < 16; ++n) {
            mfma_one(1, 1, c, n);
            if ((n & 1) == 0) {
                read_ab(nA, nB, 0, 0, n / 2);
            } else {
                issue_load<64>(ob, lB, wid, n / 2, rb_, so);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if (nk > 0) {
        const uint32_t base32 = lds_addr(sm.st);
        // scales of steps 0 and 1; A(0), B(0), A(1), B(1)
        load_scales(0, 0);
        load_scales(1, 1);
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            rsrc_t ra_, rb_;
            uint32_t so;
            codes_src(p, ra_, rb_, so);
#pragma unroll
            for (int i = 0; i < XLPW; ++i) {
                issue_load<64>(oa, base32 + (2 * p) * XOPB, wid, i, ra_, so);
                issue_load<64>(ob, base32 + (2 * p + 1) * XOPB, wid, i, rb_, so);
            }
        }
        wait_vm_lgkm0<2 * XLPW>();  // the scales of steps 0, 1 and step 0 landed
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        settle(sca[0]);
        settle(scb[0]);
        settle(sca[1]);
        settle(scb[1]);
#pragma unroll
        for (int r = 0; r < 8; ++r) read_ab(sm.st, sm.st + XOPB, 0, 0, r);
        for (int ks = 0; ks < nk; ks += 15) {
#pragma unroll
            for (int u = 0; u < 15; ++u)
                if (ks + u < nk) kstep(u, ks + u);
            if (ks + 15 < nk) {
                // back edge: the scales of ks+16 (set 1) were issued before the last 8 loads
                wait_vm_lgkm0<XLPW>();
                settle(sca[1]);
                settle(scb[1]);
            }
        }
        wait_vm_lgkm0<0>();  // no load may still be writing LDS when the block ends
        // The last steps issued scale loads past the end of K whose values no MFMA reads:
        // redefine every set after the wait, so that each register a load writes stays
        // allocated to it until the load has landed.
#pragma unroll
        for (int c = 0; c < 3; ++c) {
            settle(sca[c]);
            settle(scb[c]);
        }
    }

    // ---------------------------------------------------------------- epilogue
    // B fragment first: lane l holds row l % 32 of its 32x32 block and columns
    // 8 (v/4) + 4 (l/32) + v%4, v = 0..15: four runs of 4 consecutive columns.  Stores go
    // through LDS (staged epilogues, pipe.h): each wave stages its 128 x 128 sub-tile in its
    // quarter of the (now free) operand slots and stores whole rows.
    const int lrow = lane & 31, lcol = (lane >> 5) * 4;
    __syncthreads();                                  // every wave is done reading the slots
    char* const stg = sm.st + wid * (5 * XOPB / 4);
    const int wrow = m0 + wm * 128;                   // the wave's first row (of the tile's rows)
    if (EPI == XEPI_SWIGLU_MX) {
        // block (i, j): channels ch0 + 64 wn + 16 j + 8 hf + lcol .. +3; gate at accumulators
        // 4 hf .. +3, up at 8 + 4 hf .. +3.  h = silu(g) u in fp32 is MX-quantised here, along
        // I in blocks of 32 channels: block b of the wave's 64 channels (j = 2b, 2b + 1) of a
        // row sits in lanes l and l ^ 32 (16 values each), so its maximum takes one exchange
        // between the two halves of the wave.  Same values, same encoder and same order-free
        // maximum as quantising a stored fp32 h: the same codes and scales.
        const int ch_w = ch0 + wn * 64;  // the wave's 64 channels exist all or none (I % 64)
        if (ch_w < g.I) {
            const int64_t rb = (int64_t)e * g.c_es + row0;  // row base of the outputs
            if (g.C2) {
                // saved g|u: staged rows hold g (channels 0-63, bytes 0-127) then u (128-255)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int hf = 0; hf < 2; ++hf) {
                            const f32x16& a = acc[i][j];
                            char* rp = stg + (i * 32 + lrow) * STG_RS + (j * 16 + 8 * hf + lcol) * 2;
                            *reinterpret_cast<uint2*>(rp) =
                                make_uint2(pack_bf2(a[4 * hf], a[4 * hf + 1]),
                                           pack_bf2(a[4 * hf + 2], a[4 * hf + 3]));
                            *reinterpret_cast<uint2*>(rp + 128) =
                                make_uint2(pack_bf2(a[8 + 4 * hf], a[8 + 4 * hf + 1]),
                                           pack_bf2(a[8 + 4 * hf + 2], a[8 + 4 * hf + 3]));
                        }
                lds_wait();
                const int rr = lane >> 4, ck = lane & 15;
                const int gcol = (ck < 8 ? 0 : g.I) + ch_w + (ck & 7) * 8;
#pragma unroll 8
                for (int p = 0; p < 32; ++p) {
                    const int r = 4 * p + rr, row = wrow + r;
                    const u32x4 v = *reinterpret_cast<const u32x4*>(stg + r * STG_RS + ck * 16);
                    // non-temporal: only the backward reads the save, much later
                    if (row < Mrows) st16_nt(g.C2 + (rb + row) * g.ldc2 + gcol, v);
                }
                lds_wait();  // the reads are done before the codes overwrite the rows
            }
            // codes (rows of 64 bytes, stride 80) and the bf16 save of the quantised values
            // (rows of 128 bytes, stride 144, after the codes)
            constexpr int CRS = 80, HRS = 144, HOFF = 128 * CRS;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = i * 32 + lrow, row = wrow + r;
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    float hv[2][2][4];
                    float amax = 0.0f;
#pragma unroll
                    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                            for (int c = 0; c < 4; ++c) {
                                const f32x16& a = acc[i][2 * b + jj];
                                const float gv = a[4 * hf + c], uv = a[8 + 4 * hf + c];
                                const float h = gv / (1.0f + __expf(-gv)) * uv;
                                hv[jj][hf][c] = h;
                                amax = fmaxf(amax, fabsf(h));
                            }
                    amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
                    const int sc = mx_scale_code(amax, MOE_MX_FLOOR);
                    const int sh = 127 - sc;
                    const float f = ldexpf(1.0f, sc - 127);
#pragma unroll
                    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                        for (int hf = 0; hf < 2; ++hf) {
                            const int cw = b * 32 + 16 * jj + 8 * hf + lcol;  // channel in the wave
                            const float* h4 = hv[jj][hf];
                            const uint32_t w = e4m3x4(ldexpf(h4[0], sh), ldexpf(h4[1], sh),
                                                      ldexpf(h4[2], sh), ldexpf(h4[3], sh));
                            *reinterpret_cast<uint32_t*>(stg + r * CRS + cw) = w;
                            if (g.Ch) {  // the quantised values (exact in bf16)
                                const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
                                const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
                                *reinterpret_cast<uint2*>(stg + HOFF + r * HRS + cw * 2) =
                                    make_uint2(pack_bf2(lo[0] * f, lo[1] * f),
                                               pack_bf2(hi[0] * f, hi[1] * f));
                            }
                        }
                    if (lane < 32 && row < Mrows)
                        g.Cs[(rb + row) * (g.ldc / 32) + (ch_w + b * 32) / 32] = (uint8_t)sc;
                    // the down projection's panel scales of h: its K step tn holds these 128
                    // channels; the row is row 32 i + lrow of panel wm and this is its scale
                    // column 2 wn + b of the step, so byte 8 (32 b + lrow) + 2 i + wn of the
                    // step's run.  Rows past the expert's get the scale of zeros (code 0), as
                    // the panels built from stored scales do.
                    if (g.Ph && lane < 32)
                        g.Ph[((int64_t)(2 * mblock + wm) * (g.I / XBK) + tn) * SPAN +
                             8 * (32 * b + lrow) + 2 * i + wn] = (uint8_t)sc;
                }
            }
            lds_wait();
            {   // codes: 4 lanes per 64-byte row, 16 rows per instruction
                const int r4 = lane >> 2, c4 = lane & 3;
#pragma unroll
                for (int p = 0; p < 8; ++p) {
                    const int r = 16 * p + r4, row = wrow + r;
                    const u32x4 v = *reinterpret_cast<const u32x4*>(stg + r * CRS + c4 * 16);
                    if (row < Mrows) st16(g.Cq + (rb + row) * g.ldc + ch_w + c4 * 16, v);
                }
            }
            if (g.Ch) {  // h save: 8 lanes per 128-byte row, 8 rows per instruction
                const int r8 = lane >> 3, c8 = lane & 7;
#pragma unroll 8
                for (int p = 0; p < 16; ++p) {
                    const int r = 8 * p + r8, row = wrow + r;
                    const u32x4 v = *reinterpret_cast<const u32x4*>(stg + HOFF + r * HRS + c8 * 16);
                    if (row < Mrows) st16(g.Ch + (rb + row) * g.ldc + ch_w + c8 * 8, v);
                }
            }
        }
    } else if (EPI == XEPI_DSWIGLU) {
        // acc = dh at the wave's 128 channels; the saved g|u of the rows give dg|du
        const int chw = n0 + wn * 128;
        bf16_t* C = (bf16_t*)g.C + ((int64_t)e * g.c_es + row0) * g.ldc;
        const bf16_t* GU = g.C2 + ((int64_t)e * g.c_es + row0) * g.ldc2;
        dswiglu_staged(stg, acc, GU + (int64_t)wrow * g.ldc2 + chw, g.ldc2,
                       C + (int64_t)wrow * g.ldc + chw, g.ldc, g.I, Mrows - wrow, g.N - chw, lane);
    } else {
        bf16_t* C = (bf16_t*)g.C + ((int64_t)e * g.c_es + row0) * g.ldc;
        const int col = n0 + wn * 128;
        stage_bf16(stg, acc, lane);
        lds_wait();
        store_staged<4>(stg, C + (int64_t)wrow * g.ldc + col, g.ldc, Mrows - wrow, g.N - col, lane);
    }
}

// A dgrad product and an independent weight-gradient product in one launch, the dgrad tiles
// first: the weight-gradient tiles (E static grids of M x N tiles, each over its expert's
// token columns) fill the dgrad's last, partial round of 256 CUs.
template <int EPI>
__device__ __forceinline__ void mx_pair(const MxArgs& gd, const MxArgs& gw, MxSmem& sm) {
    const int b = blockIdx.x;
    if (b < gd.bound) {
        // the dgrad tiles: the device count of the experts' tiles (blocks past it exit)
        const int td = uni(mx_ragged_scan(gd.offsets, gd.E, gd.R, mx_n_tiles<EPI>(gd.N, gd.I), -1,
                                          nullptr, nullptr));
        if (b < td) mx_tile<EPI>(gd, sm, b);
    } else if (b - gd.bound < gw.total) {
        mx_tile<XEPI_STORE_BF16, true>(gw, sm, b - gd.bound);
    }
}
__global__ __launch_bounds__(XNTH) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mx_bwd_down_pair(MxArgs gd, MxArgs gw) {
    __shared__ MxSmem sm;
    mx_pair<XEPI_DSWIGLU>(gd, gw, sm);
}
__global__ __launch_bounds__(XNTH) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mx_bwd_gate_up_pair(MxArgs gd, MxArgs gw) {
    __shared__ MxSmem sm;
    mx_pair<XEPI_STORE_BF16>(gd, gw, sm);
}

// ---------------------------------------------------------------- the forward products
// One block per tile (blocks past the device count of the experts' tiles exit).  GEMM1 writes
// h's codes and, through Ph, GEMM2's panel scales of h, so GEMM2 follows it directly.
#define MOE_MX_KERNEL(NAME, EPI)                                                          \
    __global__ __launch_bounds__(XNTH) __attribute__((amdgpu_waves_per_eu(1, 1))) void    \
    NAME(MxArgs g) {                                                                      \
        __shared__ MxSmem sm;                                                             \
        const int total = g.offsets ? uni(mx_ragged_scan(g.offsets, g.E, g.R,              \
                                                         mx_n_tiles<EPI>(g.N, g.I), -1,   \
                                                         nullptr, nullptr))               \
                                    : g.total;                                            \
        if ((int)blockIdx.x < total) mx_tile<EPI>(g, sm, blockIdx.x);                     \
    }
MOE_MX_KERNEL(mx_gemm1_swiglu, XEPI_SWIGLU_MX)
MOE_MX_KERNEL(mx_gemm2_down, XEPI_STORE_BF16)
#undef MOE_MX_KERNEL

// Upper bound on the 256-row M tiles of an operand (host side, no device data).
static int mx_mtiles_bound(int R, int E, bool shared) {
    if (shared) return E * cdiv(R, XBM);
    return (int)(((int64_t)R + (int64_t)E * (XBM - 1)) / XBM);
}

static int mx_panels_pre(const PanelJobs& j, hipStream_t st) {
    const int nb = j.na + j.E * mx_n_tiles<XEPI_SWIGLU_MX>(2 * j.I, j.I) +
                   j.E * mx_n_tiles<XEPI_STORE_BF16>(j.H, j.I);
    const dim3 grid(nb, cdiv(max(j.H, j.I) / 32, PS_COLS));
    MOE_TRACED("mx_panel_scales", st, mx_panel_scales_pre<<<grid, 256, 0, st>>>(j));
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

static size_t mx_panel_a_bytes(int E, int R, int K, bool shared) {
    return moe_align256(2 * (size_t)mx_mtiles_bound(R, E, shared) * (size_t)(K / XBK) * SPAN);
}
template <int EPI>
static size_t mx_panel_b_bytes(int E, int N, int I, int K) {
    return moe_align256(2 * (size_t)E * (size_t)mx_n_tiles<EPI>(N, I) * (size_t)(K / XBK) * SPAN);
}

}  // namespace moe

using namespace moe;

// Workspace bytes of the panel scales of both MXFP8 GEMMs (A and B operands).
size_t moe_mx_panel_bytes(int E, int R, int H, int I, bool shared) {
    return mx_panel_a_bytes(E, R, H, shared) + mx_panel_a_bytes(E, R, I, shared) +
           mx_panel_b_bytes<XEPI_SWIGLU_MX>(E, 2 * I, I, H) +
           mx_panel_b_bytes<XEPI_STORE_BF16>(E, H, I, I);
}

int moe_launch_mx_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int K,
                             bf16_t* out, hipStream_t st);
int moe_launch_mx_quantize_bf16(const bf16_t* in, int64_t rows, int K, uint8_t* codes,
                                uint8_t* scales, const char* name, hipStream_t st);

// gu_save [rows, 2I] bf16 (the fp32 pre-activations, rounded) and h_save [rows, I] bf16 (h as
// GEMM2 consumes it: the MX-quantised values, exact in bf16) are optional saves for the
// backward.
int moe_ffn_mx(const uint8_t* xq, const uint8_t* xs, const int32_t* offsets, int E, int R, int H,
               int I, const uint8_t* w1q, const uint8_t* w1s, const uint8_t* w2q,
               const uint8_t* w2s, uint8_t* hq, uint8_t* hs, uint8_t* panels,
               bf16_t* gu_save, bf16_t* h_save, bf16_t* y, hipStream_t st) {
    // K steps of 128 codes: H and I multiples of 128
    if (H % XBK || I % XBK) return MOE_EINVAL;
    const bool shared = offsets == nullptr;
    const int mtiles = mx_mtiles_bound(R, E, shared);
    const int nt1 = mx_n_tiles<XEPI_SWIGLU_MX>(2 * I, I), nt2 = mx_n_tiles<XEPI_STORE_BF16>(H, I);
    if (mtiles <= 0) return MOE_OK;
    uint8_t* pa1 = panels;
    uint8_t* pa2 = pa1 + mx_panel_a_bytes(E, R, H, shared);
    uint8_t* pb1 = pa2 + mx_panel_a_bytes(E, R, I, shared);
    uint8_t* pb2 = pb1 + mx_panel_b_bytes<XEPI_SWIGLU_MX>(E, 2 * I, I, H);
    PanelJobs pj{xs, offsets, E, R, H, I, mtiles, shared ? mtiles : 0, w1s, w2s, pa1, pb1, pb2};
    int rc = mx_panels_pre(pj, st);
    if (rc) return rc;
    MxArgs g{};
    g.A = xq; g.At = pa1; g.a_es = 0;
    g.B = w1q; g.Bt = pb1; g.b_rows = 2 * I;
    g.Cq = hq; g.Cs = hs; g.Ch = h_save; g.c_es = shared ? R : 0; g.ldc = I;
    g.C2 = gu_save; g.ldc2 = 2 * I;
    g.offsets = offsets; g.E = E; g.R = R; g.N = 2 * I; g.K = H; g.I = I;
    g.total = shared ? mtiles * nt1 : 0;
    g.Ph = pa2;
    MOE_TRACED("mx_gemm1_swiglu", st, mx_gemm1_swiglu<<<mtiles * nt1, XNTH, 0, st>>>(g));
    MOE_LAUNCH_CHECK();
    MxArgs g2{};
    g2.A = hq; g2.At = pa2; g2.a_es = shared ? R : 0;
    g2.B = w2q; g2.Bt = pb2; g2.b_rows = H;
    g2.C = y; g2.c_es = shared ? R : 0; g2.ldc = H;
    g2.offsets = offsets; g2.E = E; g2.R = R; g2.N = H; g2.K = I; g2.I = I;
    g2.total = shared ? mtiles * nt2 : 0;
    MOE_TRACED("mx_gemm2_down", st, mx_gemm2_down<<<mtiles * nt2, XNTH, 0, st>>>(g2));
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

// ---------------------------------------------------------------- backward, MXFP8 dgrad
// Code columns of the token-axis operands: every expert's rows padded to a whole K step.
static int mx_tok_cols(int E, int R) { return cdiv(R + E * (XBK - 1), XBK) * XBK; }

// Token-axis codes, scales and panel scales of one [R, C] operand.
static size_t mx_tok_bytes(int C, int Kp) {
    return moe_align256((size_t)C * Kp) + moe_align256((size_t)C * Kp / 32) +
           moe_align256(2 * (size_t)cdiv(C, XBM) * (size_t)(Kp / XBK) * SPAN);
}

// Workspace of moe_ffn_bwd_mx: MX codes and scales of dy [R,H] and dGU [R,2I], the panel
// scales of both dgrad products' operands and, with MXFP8 weight gradients, the token-axis
// operands dy, h, dGU and xp.
size_t moe_ffn_bwd_mx_bytes(int E, int R, int H, int I, bool wgrad) {
    size_t n = moe_align256((size_t)R * H) + moe_align256((size_t)R * H / 32) +
               moe_align256((size_t)R * 2 * I) + moe_align256((size_t)R * 2 * I / 32) +
               mx_panel_a_bytes(E, R, H, false) + mx_panel_a_bytes(E, R, 2 * I, false) +
               mx_panel_b_bytes<XEPI_STORE_BF16>(E, I, I, H) +
               mx_panel_b_bytes<XEPI_STORE_BF16>(E, H, I, 2 * I);
    if (wgrad) {
        const int Kp = mx_tok_cols(E, R);
        n += 2 * mx_tok_bytes(H, Kp) + mx_tok_bytes(I, Kp) + mx_tok_bytes(2 * I, Kp);
    }
    return n;
}

int moe_launch_mx_quantize_tok(const bf16_t* X, const uint8_t* Xq, const uint8_t* Xs,
                               const MoeTokPull* pull, int R, int C, const int32_t* offsets,
                               int E, int Kp, uint8_t* codes, uint8_t* scales, uint8_t* rcodes,
                               uint8_t* rscales, uint8_t* cpanel, uint8_t* rpanel,
                               const char* name, hipStream_t st);

// A: ragged rows (offsets) or R static rows (offsets null); B: EB operands of b_rows rows.
// as null: the B panels only (the A panels come from the operand's quantiser).
static int mx_panels_ab(const uint8_t* as, const int32_t* offsets, int E, int R,
                        const uint8_t* bs, int EB, int b_rows, int K, uint8_t* pa, uint8_t* pb,
                        hipStream_t st) {
    const int na = !as ? 0 : offsets ? mx_mtiles_bound(R, E, false) : cdiv(R, XBM);
    const dim3 grid(na + EB * cdiv(b_rows, XBN), cdiv(K / 32, PS_COLS));
    MOE_TRACED("mx_panel_scales", st,
               mx_panel_scales_ab<<<grid, 256, 0, st>>>(as, offsets, E, R, na, bs, b_rows, K, pa,
                                                        pb));
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}


// One MXFP8 weight-gradient product, prepared: dW_e [M,N] = Qt(A_e)^T Qt(B_e) over expert e's
// rows, with A [R,M] and B [R,N] in expert order; quantises both operands along the tokens into
// ws (advanced past them), with their panel scales, and returns the product's arguments.  The
// pass over A also writes A quantised along its rows (arq, ars, and the panels arp: the
// operand of the dgrad product that shares A).  B may come as MX codes and scales along its
// columns (Bq, Bs; B unused), which the pass decodes.
static int mx_wgrad_prepare(const bf16_t* A, const MoeTokPull* Ap, int M, const bf16_t* B,
                            const uint8_t* Bq,
                            const uint8_t* Bs, int N,
                            const int32_t* offsets, int E, int R, bf16_t* dw, uint8_t*& ws,
                            uint8_t* arq, uint8_t* ars, uint8_t* arp, const char* qa,
                            const char* qb, MxArgs& g, hipStream_t st) {
    const int Kp = mx_tok_cols(E, R);
    uint8_t* ac = ws;
    uint8_t* as = ac + moe_align256((size_t)M * Kp);
    uint8_t* ap = as + moe_align256((size_t)M * Kp / 32);
    uint8_t* bc = ws + mx_tok_bytes(M, Kp);
    uint8_t* bsc = bc + moe_align256((size_t)N * Kp);
    uint8_t* bp = bsc + moe_align256((size_t)N * Kp / 32);
    ws += mx_tok_bytes(M, Kp) + mx_tok_bytes(N, Kp);
    int rc = moe_launch_mx_quantize_tok(A, nullptr, nullptr, Ap, R, M, offsets, E, Kp, ac, as,
                                        arq, ars, ap, arp, qa, st);
    if (rc) return rc;
    rc = moe_launch_mx_quantize_tok(B, Bq, Bs, nullptr, R, N, offsets, E, Kp, bc, bsc, nullptr,
                                    nullptr, bp, nullptr, qb, st);
    if (rc) return rc;
    g = MxArgs{};
    g.A = ac; g.At = ap; g.a_es = 0;
    g.B = bc; g.Bt = bp; g.b_rows = N;
    g.C = dw; g.c_es = M; g.ldc = N;
    g.offsets = offsets; g.E = E; g.R = R; g.N = N; g.K = Kp; g.I = 0; g.M = M;
    g.total = E * cdiv(M, XBM) * cdiv(N, XBN);
    return MOE_OK;
}

template <int EPI>
static int mx_launch_pair(const MxArgs& gd_, const MxArgs& gw, const char* name, hipStream_t st) {
    MxArgs gd = gd_;
    gd.bound = mx_mtiles_bound(gd.R, gd.E, false) * mx_n_tiles<EPI>(gd.N, gd.I);
    const int grid = gd.bound + gw.total;
    if (grid <= 0) return MOE_OK;
    if (EPI == XEPI_DSWIGLU)
        MOE_TRACED(name, st, mx_bwd_down_pair<<<grid, XNTH, 0, st>>>(gd, gw));
    else
        MOE_TRACED(name, st, mx_bwd_gate_up_pair<<<grid, XNTH, 0, st>>>(gd, gw));
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

// The routed experts' backward products in MXFP8, each operand MX-quantised along the
// product's contraction dimension:
//   dh = Q(dy) Q(W2_e^T)^T with the SwiGLU backward in the epilogue -> dgu [R,2I] bf16,
//   dXp = Q(dGU) Q(W1_e^T)^T -> dxp [R,H] bf16,
// and with wgrad (dw1, dw2 given) the weight gradients dW2_e = Qt(dy_e)^T Qt(h_e) and
// dW1_e = Qt(dGU_e)^T Qt(xp_e) in the same launches as the dgrad products.
// w2t: W2_e^T codes [E][I][H] and scales [E][I][H/32] (along H); w1t: W1_e^T codes [E][H][2I]
// and scales [E][H][2I/32] (along 2I) -- mx_quantize_t of the weights.  gu: the forward's g|u;
// h, xp: the forward's GEMM inputs (bf16); xp may instead come as its MX codes and scales
// (xq, xs: then xp is not read; weight gradients only).  With the weight gradients, dy may
// instead come as dy_pull (its rows formed from dout where they are quantised; dy unused).
int moe_ffn_bwd_mx(const int32_t* offsets, int E, int R, int H, int I, const uint8_t* w1tq,
                   const uint8_t* w1ts, const uint8_t* w2tq, const uint8_t* w2ts,
                   const bf16_t* gu, const bf16_t* dy, const MoeTokPull* dy_pull, bf16_t* dgu,
                   bf16_t* dxp, const bf16_t* h, const bf16_t* xp, const uint8_t* xq,
                   const uint8_t* xs, bf16_t* dw1, bf16_t* dw2, uint8_t* ws, hipStream_t st) {
    if (H % XBK || I % XBK) return MOE_EINVAL;
    const bool wgrad = dw1 && dw2;
    if (!wgrad && !dy) return MOE_EINVAL;
    uint8_t* dyq = ws;
    uint8_t* dys = dyq + moe_align256((size_t)R * H);
    uint8_t* gq = dys + moe_align256((size_t)R * H / 32);
    uint8_t* gs = gq + moe_align256((size_t)R * 2 * I);
    uint8_t* pa1 = gs + moe_align256((size_t)R * 2 * I / 32);
    uint8_t* pa2 = pa1 + mx_panel_a_bytes(E, R, H, false);
    uint8_t* pb1 = pa2 + mx_panel_a_bytes(E, R, 2 * I, false);
    uint8_t* pb2 = pb1 + mx_panel_b_bytes<XEPI_STORE_BF16>(E, I, I, H);
    uint8_t* wsw = ws + moe_ffn_bwd_mx_bytes(E, R, H, I, false);
    MxArgs gw{}, gw2{};  // total 0: no weight-gradient tiles
    // dy quantised along H for dh and, with the weight gradients, along the tokens for dW2 in
    // the same pass
    int rc = wgrad ? mx_wgrad_prepare(dy, dy_pull, H, h, nullptr, nullptr, I, offsets, E, R, dw2,
                                      wsw, dyq, dys, pa1, "mx_quantize_tok_dy",
                                      "mx_quantize_tok_h", gw, st)
                   : moe_launch_mx_quantize_bf16(dy, R, H, dyq, dys, "mx_quantize_dy", st);
    if (rc) return rc;
    rc = mx_panels_ab(wgrad ? nullptr : dys, offsets, E, R, w2ts, E, I, H, pa1, pb1, st);
    if (rc) return rc;
    MxArgs g{};
    g.A = dyq; g.At = pa1; g.a_es = 0;
    g.B = w2tq; g.Bt = pb1; g.b_rows = I;
    g.C = dgu; g.c_es = 0; g.ldc = 2 * I;
    g.C2 = const_cast<bf16_t*>(gu); g.ldc2 = 2 * I;
    g.offsets = offsets; g.E = E; g.R = R; g.N = I; g.K = H; g.I = I;
    rc = mx_launch_pair<XEPI_DSWIGLU>(g, gw, wgrad ? "mx_bwd_down_wgrad" : "mx_bwd_down", st);
    if (rc) return rc;
    rc = wgrad ? mx_wgrad_prepare(dgu, nullptr, 2 * I, xp, xq, xs, H, offsets, E, R, dw1, wsw, gq,
                                  gs, pa2, "mx_quantize_tok_dgu", "mx_quantize_tok_xp", gw2, st)
               : moe_launch_mx_quantize_bf16(dgu, R, 2 * I, gq, gs, "mx_quantize_dgu", st);
    if (rc) return rc;
    rc = mx_panels_ab(wgrad ? nullptr : gs, offsets, E, R, w1ts, E, H, 2 * I, pa2, pb2, st);
    if (rc) return rc;
    MxArgs g2{};
    g2.A = gq; g2.At = pa2; g2.a_es = 0;
    g2.B = w1tq; g2.Bt = pb2; g2.b_rows = H;
    g2.C = dxp; g2.c_es = 0; g2.ldc = H;
    g2.offsets = offsets; g2.E = E; g2.R = R; g2.N = H; g2.K = 2 * I; g2.I = I;
    return mx_launch_pair<XEPI_STORE_BF16>(g2, gw2,
                                           wgrad ? "mx_bwd_gate_up_wgrad" : "mx_bwd_gate_up", st);
}
