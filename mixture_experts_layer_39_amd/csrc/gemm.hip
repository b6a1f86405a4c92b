// Grouped GEMMs of the expert FFN on gfx950 MFMA, forward and backward.
//
// One tile routine covers every product of the layer:
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
//  - 256x256 output tile per block of v_mfma_f32_32x32x16_bf16 accumulators: 4 waves in 2x2,
//    each a 128x128 sub-tile (256 fp32 per lane, one wave per SIMD), or 8 waves in 4x2, each
//    a 64x128 sub-tile (128 fp32 per lane, two waves per SIMD: one can issue while the other
//    waits).  The operand ring and its loads are the same; each wave issues its share.
//  - K steps of 64: a K-major tile row is then 128 contiguous bytes per step (a whole L2
//    line per request).  At this tile size the chip's L2 can just about feed the MFMAs
//    (both need about a tile's K loop worth of 229K cycles), so the loads must stream
//    evenly: the operands of a step sit in a ring of five 32 KB LDS slots, filled by direct
//    global-to-LDS buffer loads one to two steps ahead, four loads per 16-MFMA sub-step;
//    one barrier per step.
//  - Operands contiguous along K are read from LDS with ds_read_b128; operands contiguous
//    along M or N (the weights in dgrad, both operands in wgrad) are stored as loaded and
//    read with the transposing ds_read_b64_tr_b16.  Both LDS layouts are swizzled so that
//    every read is free of bank conflicts.
//  - Loads and LDS reads are interleaved one per MFMA.
//  - Buffer loads return zeros past the end of an expert's rows, which pads ragged M tails
//    and ragged K (wgrad) tails for free.
//  - Expert tile lists are derived on the device from the offsets (no host readback): each
//    block scans the per-expert tile counts in a wave and finds its tile.
//  - The backward's independent dgrad/wgrad pairs share one launch each (bwd_down,
//    bwd_gate_up), so that one fills the other's last partial round of tiles.
#include <algorithm>

#include "pipe.h"
#include "route_dev.h"
#include "rows_dev.h"

namespace moe {

constexpr int BM = 256, BN = 256, NTH = 256;
// M tiles per group of the launch order (tm fastest within a group).  Blocks go to the 8 XCDs
// round-robin, so an XCD's resident tiles are every eighth of the order: with 2, about 5.5 A
// and 10 B operand panels per XCD at a time at the EP-64 share's shapes, against 3.6 and 18.5
// with 4 (and 10.6 and 24.3 with 3), and about 1% faster than 4 there.
constexpr int GM = 2;

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
    // wgrad over a macrobatch walked in P passes: offsets is [P][E+1] (pass-local rows) and
    // pass p's rows start at row p * pass_rows of A and B; the K loop of a tile walks the
    // expert's rows of every pass in pass order.  P = 1: one pass, offsets [E+1].
    int P;
    int pass_rows;
    int bound;  // blocks a pair launch gives this product: its tile count, or for ragged rows
                // the host's upper bound of it (the blocks past the device count exit)
};

// ---------------------------------------------------------------- LDS tiles
// (layouts, load maps and operand set-up: pipe.h)
#ifndef MOE_GEMM_SLOTS5
#define MOE_GEMM_SLOTS5 1
#endif
// LDS of one block: the stage ring (128 KB), or for BK = 64 five operand slots (160 KB).
constexpr int LDS_BYTES = MOE_GEMM_SLOTS5 ? 160 * 1024 : LDS_STAGES_BYTES;
// LDS each wave stages its output sub-tile in after the K loop (its share of the block's)
template <int NW>
constexpr int epi_wave_bytes() { return LDS_BYTES / NW; }
static_assert(STG_BYTES <= epi_wave_bytes<4>(), "staged 128-row sub-tile");
static_assert(STG_BYTES / 2 <= epi_wave_bytes<8>(), "staged 64-row sub-tile");

typedef short i16x4 __attribute__((ext_vector_type(4)));

// Transposed 8-byte LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes, lane i
// receives element i % 4 of the 8-byte chunks addressed by lanes i/4 + 4j, j = 0..3.
__device__ __forceinline__ i16x4 lds_read_tr(const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(p));
}

// Bytes of an MN-major operand range: `rows` k-rows of `ld` elements from column offset m0.
__device__ __forceinline__ uint32_t mn_bytes(int rows, int ld, int m0) {
    return (uint32_t)max((int64_t)rows * ld * 2 - (int64_t)m0 * 2, (int64_t)0);
}

// The 32x32x16 MFMA fragment of sub-tile t at k sub-step kk: 8 bf16 (k = 8 (lane/32) .. +7 of
// the sub-step) of row (or column) lane % 32.
template <int BK, bool KMAJ>
__device__ __forceinline__ bf16x8 read_frag(const Operand& o, const char* stage_op, int t, int kk) {
    if (KMAJ) {
        return *reinterpret_cast<const bf16x8*>(stage_op + o.rd[kk] + t * 32 * Pipe<BK>::KROW);
    } else {
        const char* p = stage_op + o.rd[t] + 16 * kk * 512;
        i16x4 lo = lds_read_tr(p);
        i16x4 hi = lds_read_tr(p + 4 * 512);
        typedef short i16x8 __attribute__((ext_vector_type(8)));
        i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return __builtin_bit_cast(bf16x8, v);
    }
}

// Shared memory of one GEMM block: the pipeline stages.
struct alignas(1024) GemmSmem {
    char st[LDS_BYTES];
};

template <int EPI>
__device__ __forceinline__ int n_tiles(const GemmArgs& g) {
    return (EPI == EPI_SWIGLU) ? cdiv(g.I, 128) : cdiv(g.N, BN);
}

// Ragged-M products (expert rows from device offsets) find their tiles on the device: every
// wave scans the per-expert tile counts itself, 64 experts at a time (no LDS, no barrier).
// ragged_scan returns the tile count; with `logical` >= 0 it also finds the expert owning
// tile `logical` and that expert's first tile.
__device__ __forceinline__ int ragged_scan(const GemmArgs& g, int NT, int logical, int* e_out,
                                           int* first_out) {
    const int lane = threadIdx.x & 63;
    int run = 0;
    for (int base = 0; base < g.E; base += 64) {
        const int e = base + lane;
        int tiles = 0;
        if (e < g.E) {
            const int lo = min(max(g.offsets[e], 0), g.R);
            const int hi = min(max(g.offsets[e + 1], lo), g.R);
            tiles = cdiv(hi - lo, BM) * NT;
        }
        const int inc = wave_incl_scan(tiles) + run;
        if (logical >= 0) {
            const uint64_t m = __ballot(e < g.E && inc > logical);
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

template <int EPI, bool GK>
__device__ __forceinline__ int tile_total(const GemmArgs& g) {
    if (GK || g.offsets == nullptr) return g.total;
    return uni(ragged_scan(g, n_tiles<EPI>(g), -1, nullptr, nullptr));
}

// Where tile `logical` of a product sits: its expert, the expert's rows [row0, row0+Mrows)
// (ragged-M products: from the device offsets), its M and N tile within the expert, and its
// row block: the index of (expert, M tile) among the row blocks of all experts in order.
struct TileAt {
    int e, row0, Mrows, tm, tn, mblock;
};

template <int EPI, bool GK>
__device__ __forceinline__ TileAt tile_at(const GemmArgs& g, const int logical) {
    const int NT = n_tiles<EPI>(g);
    const bool ragged_m = !GK && g.offsets != nullptr;
    TileAt t;
    int t_local, mbase;
    if (ragged_m) {
        int ee = 0, first = 0;
        ragged_scan(g, NT, logical, &ee, &first);
        t.e = uni(ee);
        t_local = uni(logical - first);
        mbase = uni(first / NT);
        int a = min(max(g.offsets[t.e], 0), g.R);
        int b = min(max(g.offsets[t.e + 1], a), g.R);
        t.row0 = uni(a);
        t.Mrows = uni(b - a);
    } else {
        int per = GK ? cdiv(g.M, BM) * NT : cdiv(g.R, BM) * NT;
        t.e = logical / per;
        t_local = logical - t.e * per;
        mbase = GK ? 0 : t.e * cdiv(g.R, BM);
        if (GK) {
            if (g.offsets) {
                // K extent: the expert's rows (of the first pass when P > 1)
                const int lim = g.P > 1 ? g.pass_rows : g.R;
                int a = min(max(g.offsets[t.e], 0), lim);
                int b = min(max(g.offsets[t.e + 1], a), lim);
                t.row0 = uni(a);
                t.Mrows = uni(b - a);
            } else {
                t.row0 = 0;
                t.Mrows = g.R;
            }
        } else {
            t.row0 = 0;
            t.Mrows = g.R;
        }
    }
    const int MT = GK ? cdiv(g.M, BM) : cdiv(t.Mrows, BM);
    {
        int grp = t_local / (GM * NT);
        int first = grp * GM;
        int gsz = min(MT - first, GM);
        int rr = t_local - grp * GM * NT;
        t.tm = first + rr % gsz;
        t.tn = rr / gsz;
    }
    t.mblock = mbase + t.tm;
    return t;
}

// One TM x 256 output tile at M tile `at.tm` of the product (tiles run in launch order: the
// blocks in flight at once, spread over all XCDs, work on neighbouring tiles whose operand
// panels meet in the shared last-level cache, which measured faster than giving each XCD
// its own compact block of tiles).  TM = 256, or 128 / 64 for the last, partial M tile of an
// expert (K-major A only; 64 with 4 waves only): the tile covers the first TM of the M tile's
// 256 rows, each wave TM / (NW / 2) of them, and every output element takes exactly the same
// MFMAs in the same order as in a 256-row tile, so the results depend neither on TM nor on NW.
template <int BK, int TM, bool A_K, bool B_K, int EPI, bool GK, int NW>
__device__ __forceinline__ void gemm_tile(const GemmArgs& g, GemmSmem& sm, const TileAt& at) {
    typedef Pipe<BK> PP;
    constexpr int KK = PP::KK, NST = PP::NST, OPB = PP::OPB;
    constexpr bool SLOTS5 = (BK == 64) && MOE_GEMM_SLOTS5;
    static_assert(TM == 256 || (TM == 128 || TM == 64) && A_K && SLOTS5, "tile heights");
    static_assert(NW == 4 || (NW == 8 && SLOTS5 && TM >= 128), "eight waves: five slots");
    constexpr int WM = NW / 2;       // waves along M (two along N)
    constexpr int WR = TM / WM;      // rows of a wave's sub-tile
    constexpr int MI = WR / 32;      // 32-row accumulator blocks per wave
    static_assert(MI >= 1 && WR % 32 == 0, "wave rows");
    constexpr int LPW = OPB / 1024 / NW;    // B loads per wave per K step
    constexpr int LPS = 2 * LPW;
    constexpr int WBB = OPB / NW;           // bytes of B a wave loads per K step
    constexpr int LPA = TM * BK * 2 / 1024 / NW;  // A loads per wave per K step
    constexpr int WBA = TM * BK * 2 / NW;   // bytes of A a wave loads per K step
    const int tid = threadIdx.x, lane = tid & 63, wid = uni(tid >> 6);
    const int wm = wid >> 1, wn = wid & 1;
    const int e = at.e, row0 = at.row0, Mrows = at.Mrows, tm = at.tm, tn = at.tn;
    const int m0 = tm * BM;
    const int Kdim = GK ? Mrows : g.K;
    const int Mvalid = GK ? g.M : Mrows;
    const int n0 = tn * BN;
    const int ch0 = tn * 128;  // SwiGLU channel base

    // ---------------------------------------------------------------- operands
    // A: K-major rows m at A_e + (row0 + m)*lda; or MN-major (wgrad): (m, k) at
    //    A_e + (row0 + k)*lda + m.
    // B: K-major rows n at B_e + n*ldb; or MN-major: (n, k) at B_e + (kbase + k)*ldb + n,
    //    kbase = row0 for wgrad (the expert's tokens), else 0 (a weight with K rows).
    //    SwiGLU: a tile holds gate and up rows of 128 channels.  Each 32-column MFMA block
    //    takes 16 channels, gate in its columns 0-15 and up in 16-31, so that every lane
    //    holds the gate and up values of the same channels in one accumulator block.
    Operand oa, ob;
    if (A_K) {
        const bf16_t* base = g.A + e * g.a_es + (int64_t)(row0 + m0) * g.lda;
        auto ident = [](int r) { return r; };
        setup_kmajor<BK, decltype(ident), TM / NW>(
            oa, base, (uint32_t)max(Mrows - m0, 0) * (uint32_t)g.lda * 2u, g.lda, wid, lane,
            wm * WR, ident, 2 * PP::RPI, 4 * PP::RPI);
    } else {
        const bf16_t* base = g.A + e * g.a_es + (int64_t)row0 * g.lda + m0;
        setup_mnmajor<BK, BK / NW>(oa, base, mn_bytes(Kdim, g.lda, m0), g.lda, wid, lane, wm * WR);
    }
    if (B_K) {
        const bf16_t* base = g.B + e * g.b_es;
        const int I = g.I;
        auto swiglu_rows = [=](int nn) {
            return ((nn >> 4) & 1) * I + ch0 + (nn >> 7) * 64 + ((nn & 127) >> 5) * 16 + (nn & 15);
        };
        auto plain_rows = [=](int nn) { return n0 + nn; };
        if (EPI == EPI_SWIGLU)
            setup_kmajor<BK, decltype(swiglu_rows), 256 / NW>(
                ob, base, (uint32_t)g.b_rows * (uint32_t)g.ldb * 2u, g.ldb, wid, lane, wn * 128,
                swiglu_rows, PP::RPI == 8 ? I : 16, PP::RPI == 8 ? 16 : 32);
        else
            setup_kmajor<BK, decltype(plain_rows), 256 / NW>(
                ob, base, (uint32_t)g.b_rows * (uint32_t)g.ldb * 2u, g.ldb, wid, lane, wn * 128,
                plain_rows, 2 * PP::RPI, 4 * PP::RPI);
    } else {
        const int64_t kbase = GK ? row0 : 0;
        const bf16_t* base = g.B + e * g.b_es + kbase * g.ldb + n0;
        setup_mnmajor<BK, BK / NW>(ob, base, mn_bytes(Kdim, g.ldb, n0), g.ldb, wid, lane, wn * 128);
    }

    f32x16 acc[MI][4];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
    // The accumulators live in the AGPRs across the K loop (they fill them exactly).  With
    // the SwiGLU epilogue the register allocator otherwise splits them over both register
    // files and spills inside the loop; pinning them there at the start prevents that (the
    // other products allocate better without it).
    auto pin_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) asm volatile("" : "+a"(acc[i][j]));
    };
    if (EPI == EPI_SWIGLU && NW == 4) pin_acc();

    // ---------------------------------------------------------------- main loop
    // NST stages in a ring: at the end of K step ks the stage it used is refilled with step
    // ks + NST.  A step is KK sub-steps of 16 k (16 MFMAs each).  The LDS reads of the next
    // sub-step's fragments and the global->LDS loads are interleaved with the MFMAs, so they
    // issue while the MFMA pipe is busy.  The step barrier (all waves done reading this
    // stage; step ks+1 landed) sits before the last sub-step, whose fragments were read
    // during the one before; the last sub-step then refills the stage and reads the next
    // step's first fragments.  Fragment reads follow the order the MFMAs consume them.
    // The MFMA takes the B fragment as its first operand, so each lane's accumulators hold
    // one output row (m) and 4-column runs (n): the epilogue stores 8-byte vectors.
    static_assert(KK >= 2 && LPS <= 16 && NST >= 2, "the step below is written for these");
    // K segments: one, except for wgrad over P > 1 passes (the expert's rows of each pass)
    const int P = (GK && g.offsets) ? max(g.P, 1) : 1;
    auto seg = [&](int p, int& first, int& len) __attribute__((always_inline)) {
        const int32_t* off = g.offsets + (int64_t)p * (g.E + 1);
        const int a = min(max(off[e], 0), g.pass_rows);
        const int b = min(max(off[e + 1], a), g.pass_rows);
        first = uni(p * g.pass_rows + a);
        len = uni(b - a);
    };
    int nk = cdiv(Kdim, BK);
    if (P > 1) {
        for (int p = 1; p < P; ++p) {
            int f, l;
            seg(p, f, l);
            nk += cdiv(l, BK);
        }
    }
    // The load cursor: the segment holding the K step being loaded (steps are loaded in
    // increasing order).  Each segment has its own buffer descriptors, so the K tail of
    // every segment reads zeros.
    int cur_p = 0, cur_start = 0, cur_steps = cdiv(Kdim, BK);
    const rsrc_t rnull = make_rsrc(nullptr, 0);
    auto load_src = [&](int ks, rsrc_t& ra_, rsrc_t& rb_, uint32_t& sa, uint32_t& sb) __attribute__((always_inline)) {
        if (ks >= nk) {  // past the end: empty descriptors (the load writes zeros)
            ra_ = rnull;
            rb_ = rnull;
            sa = sb = 0;
            return;
        }
        if (P > 1 && ks >= cur_start + cur_steps) {
            int p = cur_p, start = cur_start + cur_steps, f = 0, l = 0;
            for (;;) {
                ++p;
                seg(p, f, l);
                const int st = cdiv(l, BK);
                if (ks < start + st) {
                    cur_steps = st;
                    break;
                }
                start += st;
            }
            cur_p = p;
            cur_start = start;
            oa.r = make_rsrc(g.A + e * g.a_es + (int64_t)f * g.lda + m0, mn_bytes(l, g.lda, m0));
            ob.r = make_rsrc(g.B + e * g.b_es + (int64_t)f * g.ldb + n0, mn_bytes(l, g.ldb, n0));
        }
        ra_ = oa.r;
        rb_ = ob.r;
        sa = (uint32_t)(ks - cur_start) * oa.kstep;
        sb = (uint32_t)(ks - cur_start) * ob.kstep;
    };
    bf16x8 fa[2][MI], fb[2][4];
    // read number r (0 .. NR - 1) of a sub-step, in MFMA consumption order: a0 b0 b1 b2 b3
    // a1 .. a(MI - 1)
    auto read_ab = [&](const char* sa_, const char* sb_, int kk, int f, int r) __attribute__((always_inline)) {
        if (r == 0) fa[f][0] = read_frag<BK, A_K>(oa, sa_, 0, kk);
        else if (r <= 4) fb[f][r - 1] = read_frag<BK, B_K>(ob, sb_, r - 1, kk);
        else fa[f][r - 4] = read_frag<BK, A_K>(oa, sa_, r - 4, kk);
    };
    auto read_one = [&](const char* st, int kk, int f, int r) __attribute__((always_inline)) {
        read_ab(st, st + OPB, kk, f, r);
    };
    auto mfma_one = [&](int f, int n) __attribute__((always_inline)) {
        const int i = n >> 2, j = n & 3;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[f][j], fa[f][i], acc[i][j], 0, 0, 0);
    };
    // Schedule of a sub-step (NM MFMAs): fragment read r after MFMA rslot(r); the sub-step's
    // ql loads (4 of B, or LPA / 2 of A) at lslot(q).  For TM = 256: reads at the even MFMAs,
    // loads at every fourth odd one.
    constexpr int NM = 4 * MI, NR = 4 + MI;
    auto rslot = [](int r) constexpr { return r * NM / NR; };
    auto lslot = [](int q, int ql) constexpr { return q * NM / ql + (NM / ql > 1 ? 1 : 0); };
    auto kstep = [&](char* cur, char* nxt, uint32_t cur32, int ks) __attribute__((always_inline)) {
        // sub-steps 0 .. KK-2 (fragments kk % 2), each with the reads of the next one
#pragma unroll
        for (int kk = 0; kk < KK - 1; ++kk) {
#pragma unroll
            for (int n = 0; n < 16; ++n) {
                mfma_one(kk & 1, n);
                if (n < NR) read_one(cur, kk + 1, (kk + 1) & 1, n);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        wait_vm_lgkm0<(NST - 2) * LPS>();  // step ks+1 landed (later steps may be in flight)
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        // last sub-step with the loads of step ks+NST into this stage and the reads of the
        // next step's sub-step 0
        const bool more = ks + 1 < nk;
        rsrc_t ra_, rb_;
        uint32_t sa, sb;
        load_src(ks + NST, ra_, rb_, sa, sb);
        __builtin_amdgcn_sched_barrier(0);
        constexpr int fl = (KK - 1) & 1;
#pragma unroll
        for (int n = 0; n < 16; ++n) {
            mfma_one(fl, n);
            if (n < LPW) issue_load<BK, WBB>(oa, cur32, wid, n, ra_, sa);
            else if (n < LPS) issue_load<BK, WBB>(ob, cur32 + OPB, wid, n - LPW, rb_, sb);
            if (n >= 8 && n - 8 < NR && more) read_one(nxt, 0, 0, n - 8);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // Five operand slots (BK = 64): operand slots of OPB bytes in a ring of five, A of step s
    // in slot 2s mod 5 and B in slot 2s+1 mod 5.  Slots free up at the step barriers (which
    // follow the last LDS reads of a step): A(s+2) goes into the slot B(s-1) left, B(s+2)
    // into the slot A(s) leaves.  Four loads are issued per sub-step: in step s, the second
    // half of B(s+1) (sub-step 0), A(s+2) (sub-steps 1, 2) and after the barrier the first
    // half of B(s+2) (sub-step 3).  A gets two steps to land, B more than one, and the load
    // path sees an even stream instead of bursts after each barrier.  Within a sub-step the
    // 8 fragment reads take the even MFMA slots and the 4 loads every fourth odd one.
    rsrc_t pend_rb = make_rsrc(nullptr, 0);  // descriptor and offset of B(s+1)'s second half
    uint32_t pend_sb = 0;
    constexpr int QB = LPW / 2;  // B loads per sub-step (sub-steps 0 and 3)
    auto kstep5 = [&](int u, int ks) __attribute__((always_inline)) {
        char* const cA = sm.st + ((2 * u) % 5) * OPB;
        char* const cB = sm.st + ((2 * u + 1) % 5) * OPB;
        char* const nA = sm.st + ((2 * u + 2) % 5) * OPB;
        char* const nB = sm.st + ((2 * u + 3) % 5) * OPB;
        const uint32_t base32 = lds_addr(sm.st);
        const uint32_t lB1 = base32 + ((2 * u + 3) % 5) * OPB;  // B(ks+1): slot of A(ks-1)
        const uint32_t lA = base32 + ((2 * u + 4) % 5) * OPB;   // A(ks+2): slot of B(ks-1)
        const uint32_t lB = base32 + ((2 * u) % 5) * OPB;       // B(ks+2): slot of A(ks)
        const rsrc_t rb1 = pend_rb;
        const uint32_t sb1 = pend_sb;
        rsrc_t ra_, rb_;
        uint32_t sa, sb;
        load_src(ks + 2, ra_, rb_, sa, sb);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kk = 0; kk < KK - 1; ++kk) {
            constexpr int QA = LPA / 2;  // A loads per sub-step (sub-steps 1, 2)
            static_assert(QA >= 1 && 2 * QA == LPA, "A loads per sub-step");
#pragma unroll
            for (int n = 0; n < NM; ++n) {
                mfma_one(kk & 1, n);
#pragma unroll
                for (int r = 0; r < NR; ++r)
                    if (rslot(r) == n) read_ab(cA, cB, kk + 1, (kk + 1) & 1, r);
                if (kk == 0) {
#pragma unroll
                    for (int q = 0; q < QB; ++q)
                        if (lslot(q, QB) == n) issue_load<BK, WBB>(ob, lB1, wid, QB + q, rb1, sb1);
                } else {
#pragma unroll
                    for (int q = 0; q < QA; ++q)
                        if (lslot(q, QA) == n)
                            issue_load<BK, WBA>(oa, lA, wid, QA * (kk - 1) + q, ra_, sa);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        wait_vm_lgkm0<LPA>();  // A(ks+1), B(ks+1) landed; A(ks+2) may be in flight
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        const bool more = ks + 1 < nk;
        constexpr int fl = (KK - 1) & 1;
#pragma unroll
        for (int n = 0; n < NM; ++n) {
            mfma_one(fl, n);
#pragma unroll
            for (int q = 0; q < QB; ++q)
                if (lslot(q, QB) == n) issue_load<BK, WBB>(ob, lB, wid, q, rb_, sb);
#pragma unroll
            for (int r = 0; r < NR; ++r)
                if (rslot(r) == n && more) read_ab(nA, nB, 0, 0, r);
            __builtin_amdgcn_sched_barrier(0);
        }
        pend_rb = rb_;
        pend_sb = sb;
    };
    // 64-row tiles (an expert's last tile of at most 64 rows) stream their weight panel from
    // HBM with few MFMAs per byte, so the loads decide their time.  They use a deeper ring:
    // four 32 KB slots for B and the fifth split into four 8 KB parts for A, step s in slot
    // s mod 4 of each; step s issues the loads of step s+3 (into the slots step s-1 left at its
    // barrier) in its first three sub-steps, so three steps of operands are in flight where the
    // five-slot ring keeps about one and a half.
    auto kstep4 = [&](int u, int ks) __attribute__((always_inline)) {
        char* const cA = sm.st + 4 * OPB + u * (OPB / 4);
        char* const cB = sm.st + u * OPB;
        char* const nA = sm.st + 4 * OPB + ((u + 1) & 3) * (OPB / 4);
        char* const nB = sm.st + ((u + 1) & 3) * OPB;
        const uint32_t base32 = lds_addr(sm.st);
        const uint32_t lA = base32 + 4 * OPB + ((u + 3) & 3) * (OPB / 4);  // A(ks+3): A(ks-1)'s part
        const uint32_t lB = base32 + ((u + 3) & 3) * OPB;                  // B(ks+3): B(ks-1)'s slot
        rsrc_t ra_, rb_;
        uint32_t sa, sb;
        load_src(ks + 3, ra_, rb_, sa, sb);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kk = 0; kk < KK - 1; ++kk) {
#pragma unroll
            for (int n = 0; n < NM; ++n) {
                mfma_one(kk & 1, n);
#pragma unroll
                for (int r = 0; r < NR; ++r)
                    if (rslot(r) == n) read_ab(cA, cB, kk + 1, (kk + 1) & 1, r);
                if (kk < 2) {  // B(ks+3): half in sub-step 0, half in sub-step 1
#pragma unroll
                    for (int q = 0; q < LPW / 2; ++q)
                        if (lslot(q, LPW / 2) == n)
                            issue_load<BK, WBB>(ob, lB, wid, (LPW / 2) * kk + q, rb_, sb);
                } else {       // A(ks+3) in sub-step 2
#pragma unroll
                    for (int q = 0; q < LPA; ++q)
                        if (lslot(q, LPA) == n) issue_load<BK, WBA>(oa, lA, wid, q, ra_, sa);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        wait_vm_lgkm0<2 * (LPA + LPW)>();  // step ks+1 landed; ks+2 and ks+3 may be in flight
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        constexpr int fl = (KK - 1) & 1;
        // last sub-step, with the reads of the next step's first fragments (they run after the
        // last step too, of slots inside LDS with values unused: a read under a condition
        // would make the compiler copy the fragments)
#pragma unroll
        for (int n = 0; n < NM; ++n) {
            mfma_one(fl, n);
#pragma unroll
            for (int r = 0; r < NR; ++r)
                if (rslot(r) == n) read_ab(nA, nB, 0, 0, r);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if (TM == 64 && nk > 0 && SLOTS5) {
        static_assert(TM != 64 || (KK == 4 && 4 * OPB + 4 * (OPB / 4) <= (int)sizeof(GemmSmem) &&
                                   WBA * 4 == OPB / 4), "deep ring layout");
        const uint32_t base32 = lds_addr(sm.st);
        // steps 0, 1, 2
#pragma unroll
        for (int p = 0; p < 3; ++p) {
            rsrc_t ra_, rb_;
            uint32_t sa, sb;
            load_src(p, ra_, rb_, sa, sb);
#pragma unroll
            for (int i = 0; i < LPW; ++i) {
                if (i < LPA) issue_load<BK, WBA>(oa, base32 + 4 * OPB + p * (OPB / 4), wid, i, ra_, sa);
                issue_load<BK, WBB>(ob, base32 + p * OPB, wid, i, rb_, sb);
            }
        }
        wait_vm_lgkm0<2 * (LPA + LPW)>();  // step 0 landed
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < NR; ++r) read_ab(sm.st + 4 * OPB, sm.st, 0, 0, r);
        for (int ks = 0; ks < nk; ks += 4) {
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (ks + u < nk) kstep4(u, ks + u);
        }
        wait_vm_lgkm0<0>();  // no load may still be writing LDS when the block ends
    } else if (nk > 0 && SLOTS5) {
        static_assert(!SLOTS5 || (KK == 4 && LPW * NW == 32 && 5 * OPB <= (int)sizeof(GemmSmem)),
                      "five-slot ring layout");
        const uint32_t base32 = lds_addr(sm.st);
        // A(0), B(0), A(1) and the first half of B(1); step 0 issues B(1)'s second half
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            rsrc_t ra_, rb_;
            uint32_t sa, sb;
            load_src(p, ra_, rb_, sa, sb);
#pragma unroll
            for (int i = 0; i < LPW; ++i) {
                if (i < LPA) issue_load<BK, WBA>(oa, base32 + (2 * p) * OPB, wid, i, ra_, sa);
                if (p == 0 || i < LPW / 2)
                    issue_load<BK, WBB>(ob, base32 + (2 * p + 1) * OPB, wid, i, rb_, sb);
            }
            pend_rb = rb_;
            pend_sb = sb;
        }
        wait_vm_lgkm0<LPA + LPW / 2>();  // step 0 landed
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < NR; ++r) read_ab(sm.st, sm.st + OPB, 0, 0, r);
        for (int ks = 0; ks < nk; ks += 5) {
#pragma unroll
            for (int u = 0; u < 5; ++u)
                if (ks + u < nk) kstep5(u, ks + u);
        }
        wait_vm_lgkm0<0>();  // no load may still be writing LDS when the block ends
    } else if (nk > 0) {
        static_assert(SLOTS5 || (TM == 256 && NW == 4), "the stage ring takes 256-row tiles");
        const uint32_t st_base = lds_addr(sm.st);  // stage p at st_base + p * 2 * OPB
#pragma unroll
        for (int p = 0; p < NST; ++p) {
            rsrc_t ra_, rb_;
            uint32_t sa, sb;
            load_src(p, ra_, rb_, sa, sb);
#pragma unroll
            for (int i = 0; i < LPW; ++i) {
                issue_load<BK, WBB>(oa, st_base + p * 2 * OPB, wid, i, ra_, sa);
                issue_load<BK, WBB>(ob, st_base + p * 2 * OPB + OPB, wid, i, rb_, sb);
            }
        }
        wait_vm_lgkm0<(NST - 1) * LPS>();  // step 0 landed
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < NR; ++r) read_one(sm.st, 0, 0, r);
        for (int ks = 0; ks < nk; ks += NST) {
#pragma unroll
            for (int u = 0; u < NST; ++u)
                if (ks + u < nk)
                    kstep(sm.st + u * 2 * OPB, sm.st + ((u + 1) % NST) * 2 * OPB, st_base + u * 2 * OPB, ks + u);
        }
        wait_vm_lgkm0<0>();  // no load may still be writing LDS when the block ends
    }

    // ---------------------------------------------------------------- epilogue
    // Through LDS (staged epilogues, pipe.h): each wave stages its WR x 128 sub-tile in its
    // share (a quarter or an eighth) of the (now free) operand slots and stores whole rows.
    const int lrow = lane & 31, lcol = (lane >> 5) * 4;
    __syncthreads();                                  // every wave is done reading the slots
    static_assert(MI * 32 * STG_RS <= epi_wave_bytes<NW>(), "staging area of a wave");
    char* const stg = sm.st + wid * epi_wave_bytes<NW>();
    const int wrow = m0 + wm * WR;                    // the wave's first row (of the tile's rows)
    const int wrows = min(Mvalid - wrow, WR);          // its rows that exist
    if (EPI == EPI_STORE) {
        bf16_t* C = g.C + e * g.c_es + (GK ? 0 : (int64_t)row0 * g.ldc);
        const int col = n0 + wn * 128;
        stage_bf16<MI>(stg, acc, lane);
        lds_wait();
        // weight gradients (GK): written once per step and read by nothing in it
        store_staged<MI, GK>(stg, C + (int64_t)wrow * g.ldc + col, g.ldc, wrows, g.N - col, lane);
    } else if (EPI == EPI_SWIGLU) {
        // block (i, j) of a lane: channels 16 j + 8 hf + lcol .. +3 (hf = 0, 1) of the wave's
        // 64 (ch_w ..), gate at accumulators 4 hf .. +3, up at 8 + 4 hf .. +3; the wave's 64
        // channels exist all or none (I % 64 == 0)
        const int ch_w = ch0 + wn * 64;
        if (ch_w < g.I) {
            if (g.C2) {
                // saved g|u: staged rows hold g (channels 0-63, bytes 0-127) then u (128-255)
                bf16_t* C2 = g.C2 + e * g.c2_es + (int64_t)row0 * g.ldc2;
#pragma unroll
                for (int i = 0; i < MI; ++i)
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
                for (int p = 0; p < 8 * MI; ++p) {
                    const int r = 4 * p + rr, row = wrow + r;
                    const u32x4 v = *reinterpret_cast<const u32x4*>(stg + r * STG_RS + ck * 16);
                    // non-temporal: only the backward reads the save, much later
                    if (r < wrows) st16_nt(C2 + (int64_t)row * g.ldc2 + gcol, v);
                }
                lds_wait();  // the reads are done before h overwrites the rows
            }
            // h = silu(g) u: staged rows of 64 channels (128 bytes), read back by 8 lanes
            bf16_t* C = g.C + e * g.c_es + (int64_t)row0 * g.ldc;
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf) {
                        const f32x16& a = acc[i][j];
                        float hv[4];
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const float gv = a[4 * hf + c], uv = a[8 + 4 * hf + c];
                            hv[c] = gv / (1.0f + __expf(-gv)) * uv;
                        }
                        *reinterpret_cast<uint2*>(stg + (i * 32 + lrow) * STG_RS +
                                                  (j * 16 + 8 * hf + lcol) * 2) =
                            make_uint2(pack_bf2(hv[0], hv[1]), pack_bf2(hv[2], hv[3]));
                    }
            lds_wait();
            const int r8 = lane >> 3, c8 = lane & 7;
#pragma unroll 8
            for (int p = 0; p < 4 * MI; ++p) {
                const int r = 8 * p + r8, row = wrow + r;
                const u32x4 v = *reinterpret_cast<const u32x4*>(stg + r * STG_RS + c8 * 16);
                if (r < wrows) st16(C + (int64_t)row * g.ldc + ch_w + c8 * 8, v);
            }
        }
    } else {  // EPI_DSWIGLU: acc = dh; the saved g|u give dg|du
        const int chw = n0 + wn * 128;
        bf16_t* C = g.C + e * g.c_es + (int64_t)row0 * g.ldc;
        const bf16_t* GU = g.C2 + e * g.c2_es + (int64_t)row0 * g.ldc2;
        dswiglu_staged<MI, NW == 4 ? 2 : 1>(stg, acc, GU + (int64_t)wrow * g.ldc2 + chw, g.ldc2,
                           C + (int64_t)wrow * g.ldc + chw, g.ldc, g.I, wrows, g.N - chw, lane);
    }
}

// A tile of a product: the products with ragged, K-major A (rows of experts) run each
// expert's last M tile, when it holds at most 128 (64) rows, as a 128-row (64-row) tile: less
// MFMA work on padding rows, bit-identical results.
template <int BK, bool A_K, bool B_K, int EPI, bool GK, int NW>
__device__ __forceinline__ void run_tile(const GemmArgs& g, GemmSmem& sm, const TileAt& at) {
    if (A_K && !GK) {
        const int rem = at.Mrows - at.tm * BM;
        if (NW == 4 && rem <= 64) {
            gemm_tile<BK, (A_K && !GK && NW == 4) ? 64 : 256, A_K, B_K, EPI, GK, NW>(g, sm, at);
            return;
        }
        if (rem <= 128) {
            gemm_tile<BK, (A_K && !GK) ? 128 : 256, A_K, B_K, EPI, GK, NW>(g, sm, at);
            return;
        }
    }
    gemm_tile<BK, 256, A_K, B_K, EPI, GK, NW>(g, sm, at);
}

// One kernel symbol per product of the layer, so that profiles name each role.
// K step per product.  Every product measures fastest with 64-wide steps in the five-slot
// ring (the 32-wide ring of four stages stays available to the tile routine).
constexpr int BK_FWD = 64, BK_DGRAD = 64, BK_WGRAD = 64;
// Waves per block: 4 (one per SIMD, each a 128 x 128 sub-tile) for the forward products, 8
// (two per SIMD, 64 x 128 each) for the backward pairs.  Same-box measurements: the backward
// pairs of the weight-streaming layers (many small experts, weight-gradient tiles of a few K
// steps) ran 5-8% faster with eight waves and the EP-64 share's pairs the same or 1% faster;
// the forward products ran 1-2% slower (and their experts' last tiles of at most 64 rows lose
// the deep ring, which needs four waves).  The single launch keeps 4: its other steps are
// written for 256-thread blocks.
#ifndef MOE_FWD_NW
#define MOE_FWD_NW 4
#endif
#ifndef MOE_BWD_NW
#define MOE_BWD_NW 8
#endif
constexpr int FWD_NW = MOE_FWD_NW, BWD_NW = MOE_BWD_NW;
#define MOE_GEMM_ATTRS(NW) \
    __launch_bounds__(64 * (NW)) __attribute__((amdgpu_waves_per_eu((NW) / 4, (NW) / 4)))

#define MOE_GEMM_KERNEL(NAME, AKM, BKM, EPI, GK)                                          \
    __global__ MOE_GEMM_ATTRS(FWD_NW) void NAME(GemmArgs g) {                             \
        __shared__ GemmSmem sm;                                                            \
        const int total = tile_total<EPI, GK>(g);                                          \
        if ((int)blockIdx.x < total)                                                        \
            run_tile<BK_FWD, AKM, BKM, EPI, GK, FWD_NW>(g, sm, tile_at<EPI, GK>(g, blockIdx.x)); \
    }
MOE_GEMM_KERNEL(gemm1_swiglu, true, true, EPI_SWIGLU, false)     // [g|u] = Xp W1^T, h
MOE_GEMM_KERNEL(gemm2_down, true, true, EPI_STORE, false)        // y = h W2^T
#undef MOE_GEMM_KERNEL

// The backward's two pairs of independent products run as one launch each, the dgrad tiles
// first and the wgrad tiles after them, so that the second product fills the last,
// partly empty round of the first (256 CUs, one tile each at a time).  The dgrad product
// gets the first gd.bound blocks (for ragged rows the host's upper bound of its tiles: the
// blocks past the device count exit at once), so that a weight-gradient block knows its tile
// without the scan of the experts' row counts, which costs a block a few microseconds and
// weighs on weight-gradient tiles of one or two K steps.
//   bwd_down:     dh = dy W2 -> dg|du (SwiGLU backward)   and   dW2 = dy^T h
//   bwd_gate_up:  dXp = dGU W1                           and   dW1 = dGU^T Xp
__global__ MOE_GEMM_ATTRS(BWD_NW) void bwd_down(GemmArgs gd, GemmArgs gw) {
    __shared__ GemmSmem sm;
    const int b = blockIdx.x;
    if (b < gd.bound) {
        if (b < tile_total<EPI_DSWIGLU, false>(gd))
            run_tile<BK_DGRAD, true, false, EPI_DSWIGLU, false, BWD_NW>(gd, sm, tile_at<EPI_DSWIGLU, false>(gd, b));
    } else if (b - gd.bound < gw.total) {
        run_tile<BK_WGRAD, false, false, EPI_STORE, true, BWD_NW>(gw, sm, tile_at<EPI_STORE, true>(gw, b - gd.bound));
    }
}

__global__ MOE_GEMM_ATTRS(BWD_NW) void bwd_gate_up(GemmArgs gd, GemmArgs gw) {
    __shared__ GemmSmem sm;
    const int b = blockIdx.x;
    if (b < gd.bound) {
        if (b < tile_total<EPI_STORE, false>(gd))
            run_tile<BK_DGRAD, true, false, EPI_STORE, false, BWD_NW>(gd, sm, tile_at<EPI_STORE, false>(gd, b));
    } else if (b - gd.bound < gw.total) {
        run_tile<BK_WGRAD, false, false, EPI_STORE, true, BWD_NW>(gw, sm, tile_at<EPI_STORE, true>(gw, b - gd.bound));
    }
}

// Upper bound on the tile count of a ragged-M product (host side, no device data).
static int ragged_tiles_bound(int R, int E, int NT) {
    int64_t mt = ((int64_t)R + (int64_t)E * (BM - 1)) / BM;
    return (int)(mt * NT);
}

// Blocks to launch for a product: its tile count, or for ragged-M products an upper bound
// (surplus blocks exit at once).
static int grid_of(const GemmArgs& g, int NT, bool GK) {
    if (GK || !g.offsets) return g.total;
    return ragged_tiles_bound(g.R, g.E, NT);
}

static int launch(void (*kern)(GemmArgs), const char* name, const GemmArgs& g, int NT,
                  hipStream_t st) {
    const int grid = grid_of(g, NT, false);
    if (grid <= 0) return MOE_OK;
    MOE_TRACED(name, st, kern<<<grid, 64 * FWD_NW, 0, st>>>(g));
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

static int launch_pair(void (*kern)(GemmArgs, GemmArgs), const char* name, const GemmArgs& gd_,
                       const GemmArgs& gw, hipStream_t st) {
    GemmArgs gd = gd_;
    gd.bound = grid_of(gd, cdiv(gd.N, BN), false);
    const int grid = gd.bound + gw.total;
    if (grid <= 0) return MOE_OK;
    MOE_TRACED(name, st, kern<<<grid, 64 * BWD_NW, 0, st>>>(gd, gw));
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

// ---------------------------------------------------------------- the layer in one launch
// The forward of the layer -- router projection, top-k routing, the expert-contiguous
// permutation, dispatch, GEMM1 + SwiGLU, GEMM2 and the combine -- as one persistent kernel
// with every block resident at once (the single fused MoE kernel of pulsen.vercel.app, "Cursor åpner
// megakernelen…", ¶3, and ki-pruefstand.de, "Cursor veröffentlicht MoE-Megakernel…",
// "Kommunikation im Kernel" ¶2, on one GPU): one block per CU.  The routing steps, the
// dispatch and the combine are separated by device-wide barriers.  The two expert products
// run as one queue of tiles that blocks claim in order -- GEMM1 tiles, then GEMM2 tiles --
// where a GEMM2 tile waits only for the GEMM1 tiles of its own row block, through per-row-
// block completion counters (a tile-level dependency in place of a barrier between the
// products, the idea of the tile-level triggers aiexpert.news, "Megakernels are dead and
// back", ¶2, describes for kernel launches), so the last, partial round of GEMM1 tiles fills
// with GEMM2 tiles.  Every item runs the same device code as its own kernel, so the outputs
// are bit-identical to the step-by-step launches.  Claiming in order makes the queue
// deadlock-free: a tile only waits for tiles claimed before it, which run on blocks that are
// resident (they claimed it) and never wait for later tiles.
// Visibility across XCDs: each XCD has its own L2, so a finished GEMM1 tile writes its L2
// back (device-scope release) before it counts itself done; a GEMM2 tile drops stale lines
// (acquire) before reading.  GEMM2 tiles do not signal: a write-back per tile of the second
// product measured more costly than the barrier before the combine.
struct FusedFwd {
    const bf16_t* wr;         // router weights [E_router,H], or null: the logits are given
    float* proj;              // logits written by the projection (tp.logits), or null
    TopkParams tp;            // top-k over the router logits (tp.T tokens)
    const int32_t* perm_ids;  // expert ids to permute: tp.idx, or the given local ids
    int64_t n;                // pairs T * k
    int E, nbits, nch;
    int32_t* blk;             // [nch][E] chunk histograms (workspace)
    int32_t *counts, *offsets, *pos, *src;
    const bf16_t* x;
    int T, H, k, R, S;
    bf16_t* xp;
    GemmArgs g1, g2;          // routed experts: GEMM1 + SwiGLU, GEMM2
    GemmArgs s1, s2;          // shared experts (total 0 when there are none)
    const bf16_t* ys;
    bf16_t* out;
    unsigned* sy;             // synchronisation words (workspace, cleared before the launch)
    int mbr;                  // row blocks reserved for the routed experts (upper bound)
    int mbs;                  // row blocks per shared expert: cdiv(T, BM)
};

constexpr int FUSED_NV = 4;      // router experts per lane: E_router <= 256
constexpr int RG_WAVE = 4;       // 16-byte row chunks a lane sums per pass (combine)
// synchronisation words (4-byte units): barrier count and generation, the queue's claim
// counter and the error flag on their own 128-byte lines; then the per-row-block counters of
// finished GEMM1 tiles
constexpr int SY_COUNT = 0, SY_GEN = 32, SY_CLAIM = 64, SY_ERR = 96, SY_READY = 128;
constexpr uint64_t SPIN_TICKS = 200000000ull;  // 2 s of the 100 MHz clock: wait limit

// Every thread's global stores are acknowledged (vmcnt(0)), so that after the block barrier
// that follows, one thread's device-scope release covers the whole block's writes.
__device__ __forceinline__ void stores_done() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ unsigned ld_relaxed(const unsigned* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Spins (one thread) until *p >= need.  Bounded: past SPIN_TICKS it raises the error flag and
// returns, so that a broken invariant ends the kernel instead of hanging the GPU.
__device__ __forceinline__ void spin_until(const unsigned* p, unsigned need, unsigned* sy) {
    if (ld_relaxed(p) >= need) return;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (ld_relaxed(p) < need) {
        if (ld_relaxed(sy + SY_ERR)) return;  // an earlier wait ran out: do not wait again
        __builtin_amdgcn_s_sleep(1);
        if (__builtin_amdgcn_s_memrealtime() - t0 > SPIN_TICKS) {
            __hip_atomic_fetch_or(sy + SY_ERR, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
    }
}

// Device-wide barrier: every block's writes before it are visible to every block after it.
// The arriving block makes its writes visible at device scope (L2 write-back), counts itself
// in, and the last one to arrive resets the count and advances the generation the others
// wait on; each then drops stale cached lines (acquire).
__device__ __forceinline__ void grid_barrier(unsigned* sy) {
    stores_done();
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned gen = ld_relaxed(sy + SY_GEN);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        const unsigned old =
            __hip_atomic_fetch_add(sy + SY_COUNT, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (old == gridDim.x - 1) {
            __hip_atomic_exchange(sy + SY_COUNT, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_fetch_add(sy + SY_GEN, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
            while (ld_relaxed(sy + SY_GEN) == gen) {
                if (ld_relaxed(sy + SY_ERR)) break;
                __builtin_amdgcn_s_sleep(1);
                if (__builtin_amdgcn_s_memrealtime() - t0 > SPIN_TICKS) {
                    __hip_atomic_fetch_or(sy + SY_ERR, 2u, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
}

// Marks one more tile of row block `mb` done, after every thread's stores of the tile are
// acknowledged and made visible device-wide (L2 write-back).
__device__ __forceinline__ void tile_done(unsigned* ready, int mb) {
    stores_done();
    __syncthreads();
    if (threadIdx.x == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __hip_atomic_fetch_add(ready + mb, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

__global__ void fused_clear(unsigned* sy, int words) {
    for (int i = threadIdx.x; i < words; i += blockDim.x) sy[i] = 0;
}

__global__ __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(1, 1)))
void layer_forward_fused(FusedFwd a) {
    __shared__ GemmSmem sm;
    const int nb = gridDim.x, wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
    int* lds_i = reinterpret_cast<int*>(sm.st);
    unsigned* const ready1 = a.sy + SY_READY;
    const bool local = a.perm_ids != a.tp.idx;
    // 0. router projection (when the logits are not given): one thread per logit
    if (a.wr) {
        const int nl = a.tp.T * a.tp.E;
        for (int id = blockIdx.x * NTH + threadIdx.x; id < nl; id += nb * NTH)
            router_logit(a.x, a.wr, a.H, a.tp.E, id, a.proj);
        grid_barrier(a.sy);
    }
    // 1. top-k and weights: one wave per token; 2. chunk histograms of the expert ids: one
    // block per chunk (in the same step when the ids are given, not selected)
    for (int t = blockIdx.x * 4 + wid; t < a.tp.T; t += nb * 4)
        topk_token<FUSED_NV>(a.tp, t, lane);
    if (!local) grid_barrier(a.sy);
    for (int c = blockIdx.x; c < a.nch; c += nb) count_chunk(a.perm_ids, a.n, a.E, a.blk, c, lds_i);
    grid_barrier(a.sy);
    // 3. counts, offsets and chunk bases: one block
    if (blockIdx.x == 0)
        scan_body(a.blk, a.nch, a.E, a.counts, a.offsets, lds_i, lds_i + SCAN_LDS);
    grid_barrier(a.sy);
    // 4. ranks: one wave per chunk, each with its own counters
    for (int c = blockIdx.x * 4 + wid; c < a.nch; c += nb * 4)
        rank_chunk(a.perm_ids, a.n, a.E, a.nbits, a.blk, a.pos, a.src, c, lds_i + wid * a.E);
    grid_barrier(a.sy);
    // 5. dispatch: one block per source token (measured faster here than a wave per token
    // for wide rows; the gather-reduce of the combine is the other way round)
    for (int t = blockIdx.x; t < a.T; t += nb) dispatch_token<NTH>(a.x, a.H, a.k, a.pos, a.R, a.xp, t, lds_i);
    grid_barrier(a.sy);
    // 6. the queue: GEMM1 tiles (routed, shared), then GEMM2 tiles (routed, shared)
    const int n1r = tile_total<EPI_SWIGLU, false>(a.g1), n1 = n1r + a.s1.total;
    const int n2r = tile_total<EPI_STORE, false>(a.g2), total = n1 + n2r + a.s2.total;
    const unsigned nt1 = (unsigned)n_tiles<EPI_SWIGLU>(a.g1);
    const unsigned nt1s = a.S ? (unsigned)n_tiles<EPI_SWIGLU>(a.s1) : 0u;
    int* const bcast = reinterpret_cast<int*>(sm.st + LDS_BYTES - 16);
    int item = blockIdx.x;
    while (item < total) {
        int next = 0;
        if (threadIdx.x == 0)
            next = nb + (int)__hip_atomic_fetch_add(a.sy + SY_CLAIM, 1u, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT);
        if (item < n1) {
            const bool r = item < n1r;
            const GemmArgs& g = r ? a.g1 : a.s1;
            const TileAt at = tile_at<EPI_SWIGLU, false>(g, r ? item : item - n1r);
            run_tile<BK_FWD, true, true, EPI_SWIGLU, false, 4>(g, sm, at);
            tile_done(ready1, r ? at.mblock : a.mbr + at.mblock);
        } else {
            const int i2 = item - n1;
            const bool r = i2 < n2r;
            const GemmArgs& g = r ? a.g2 : a.s2;
            const TileAt at = tile_at<EPI_STORE, false>(g, r ? i2 : i2 - n2r);
            if (threadIdx.x == 0) {
                spin_until(ready1 + (r ? at.mblock : a.mbr + at.mblock), r ? nt1 : nt1s, a.sy);
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            }
            __syncthreads();
            run_tile<BK_FWD, true, true, EPI_STORE, false, 4>(g, sm, at);
        }
        __syncthreads();
        if (threadIdx.x == 0) *bcast = next;
        __syncthreads();
        item = *bcast;
        __syncthreads();
    }
    grid_barrier(a.sy);
    // 7. combine: one wave per token
    for (int t = blockIdx.x * 4 + wid; t < a.T; t += nb * 4)
        combine_token_wave<RG_WAVE>(a.g2.C, a.pos, a.tp.w, a.T, a.k, a.H, a.R, a.ys, a.S, a.out,
                                    t, lane);
}

// ---------------------------------------------------------------- the FFN in one launch
// GEMM1 + SwiGLU and GEMM2 of one moe_expert_ffn call (BF16) as one queue of tiles, the
// product queue of layer_forward_fused on its own: a GEMM2 tile waits only for the GEMM1
// tiles of its row block (per-row-block counters), so GEMM2 tiles fill the last, partial
// round of GEMM1 tiles instead of waiting for a second launch.  Every item is claimed from a
// counter, the first one included: a tile is then only ever held by a running block, and a
// GEMM2 tile waits only for GEMM1 tiles claimed before it, which never wait themselves.  The
// queue cannot deadlock however many of the blocks are resident, so an ordinary launch of
// one block per CU serves.  Same tile code as gemm1_swiglu / gemm2_down: bit-identical
// outputs.  The synchronisation words (sy) are cleared by ffn_queue_clear just before.
struct FfnQueue {
    GemmArgs g1, g2;
    unsigned* sy;
};

__global__ void ffn_queue_clear(unsigned* sy, int words) {
    for (int i = threadIdx.x; i < words; i += blockDim.x) sy[i] = 0;
}

__global__ MOE_GEMM_ATTRS(FWD_NW) void ffn_queue(FfnQueue q) {
    __shared__ GemmSmem sm;
    unsigned* const ready = q.sy + SY_READY;
    const int n1 = tile_total<EPI_SWIGLU, false>(q.g1);
    const int total = n1 + tile_total<EPI_STORE, false>(q.g2);
    const unsigned nt1 = (unsigned)n_tiles<EPI_SWIGLU>(q.g1);
    int* const bcast = reinterpret_cast<int*>(sm.st + LDS_BYTES - 16);
    for (;;) {
        if (threadIdx.x == 0)
            *bcast = (int)__hip_atomic_fetch_add(q.sy + SY_CLAIM, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const int item = *bcast;
        __syncthreads();
        if (item >= total) break;
        if (item < n1) {
            const TileAt at = tile_at<EPI_SWIGLU, false>(q.g1, item);
            run_tile<BK_FWD, true, true, EPI_SWIGLU, false, FWD_NW>(q.g1, sm, at);
            tile_done(ready, at.mblock);
        } else {
            const TileAt at = tile_at<EPI_STORE, false>(q.g2, item - n1);
            if (threadIdx.x == 0) {
                spin_until(ready + at.mblock, nt1, q.sy);
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            }
            __syncthreads();
            run_tile<BK_FWD, true, true, EPI_STORE, false, FWD_NW>(q.g2, sm, at);
        }
        __syncthreads();
    }
}

static GemmArgs blank() {
    GemmArgs g{};
    return g;
}

}  // namespace moe

using namespace moe;

// ---------------------------------------------------------------------- internal API
// Forward FFN in BF16.  offsets == null: shared mode (every expert takes all R rows).
// Arguments of the forward GEMMs (GEMM1 + SwiGLU, GEMM2) of one FFN call.
static void ffn_args(const bf16_t* xp, const int32_t* offsets, int E, int R, int H, int I,
                     const bf16_t* w1, const bf16_t* w2, bf16_t* gu, bf16_t* h, bf16_t* y,
                     GemmArgs& g, GemmArgs& g2) {
    const bool shared = offsets == nullptr;
    g = blank();
    g.A = xp; g.a_es = 0; g.lda = H;
    g.B = w1; g.b_es = (int64_t)2 * I * H; g.ldb = H; g.b_rows = 2 * I;
    g.C = h; g.c_es = shared ? (int64_t)R * I : 0; g.ldc = I;
    g.C2 = gu; g.c2_es = shared ? (int64_t)R * 2 * I : 0; g.ldc2 = 2 * I;
    g.offsets = offsets; g.E = E; g.R = R; g.N = 2 * I; g.K = H; g.I = I;
    g.total = shared ? E * cdiv(R, BM) * cdiv(I, 128) : 0;
    g2 = blank();
    g2.A = h; g2.a_es = shared ? (int64_t)R * I : 0; g2.lda = I;
    g2.B = w2; g2.b_es = (int64_t)H * I; g2.ldb = I; g2.b_rows = H;
    g2.C = y; g2.c_es = shared ? (int64_t)R * H : 0; g2.ldc = H;
    g2.offsets = offsets; g2.E = E; g2.R = R; g2.N = H; g2.K = I; g2.I = I;
    g2.total = shared ? E * cdiv(R, BM) * cdiv(H, BN) : 0;
}

int moe_ffn_bf16(const bf16_t* xp, const int32_t* offsets, int E, int R, int H, int I,
                 const bf16_t* w1, const bf16_t* w2, bf16_t* gu, bf16_t* h, bf16_t* y,
                 hipStream_t st) {
    GemmArgs g, g2;
    ffn_args(xp, offsets, E, R, H, I, w1, w2, gu, h, y, g, g2);
    int rc = launch(gemm1_swiglu, "gemm1_swiglu", g, cdiv(I, 128), st);
    if (rc) return rc;
    return launch(gemm2_down, "gemm2_down", g2, cdiv(H, BN), st);
}

// Row blocks of one FFN call (the per-row-block counters of ffn_queue): an upper bound for
// ragged experts, E * cdiv(R, BM) for shared ones.
int64_t moe_ffn_row_blocks(int E, int R, bool shared) {
    return shared ? (int64_t)E * cdiv(R, BM) : ((int64_t)R + (int64_t)E * (BM - 1)) / BM;
}

size_t moe_ffn_sync_bytes(int E, int R, bool shared) {
    return moe_align256((size_t)(SY_READY + moe_ffn_row_blocks(E, R, shared)) * 4);
}

size_t moe_ffn_error_word() { return SY_ERR * 4; }

// The same products as moe_ffn_bf16 as one launch (ffn_queue); sy: moe_ffn_sync_bytes().
int moe_ffn_bf16_queue(const bf16_t* xp, const int32_t* offsets, int E, int R, int H, int I,
                       const bf16_t* w1, const bf16_t* w2, bf16_t* gu, bf16_t* h, bf16_t* y,
                       unsigned* sy, hipStream_t st) {
    FfnQueue q{};
    ffn_args(xp, offsets, E, R, H, I, w1, w2, gu, h, y, q.g1, q.g2);
    q.sy = sy;
    const int64_t tiles = (int64_t)grid_of(q.g1, cdiv(I, 128), false) +
                          grid_of(q.g2, cdiv(H, BN), false);
    if (tiles <= 0) return MOE_OK;
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        ncu < 1)
        return MOE_EHIP;
    const int grid = (int)std::min<int64_t>(tiles, ncu);  // one block per CU (LDS)
    const int words = (int)(SY_READY + moe_ffn_row_blocks(E, R, offsets == nullptr));
    MOE_TRACED("ffn_queue_clear", st, ffn_queue_clear<<<1, 1024, 0, st>>>(sy, words));
    MOE_LAUNCH_CHECK();
    MOE_TRACED("ffn_queue", st, ffn_queue<<<grid, 64 * FWD_NW, 0, st>>>(q));
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

// Synchronisation words of the single launch: the fixed words and the GEMM1 counter of every
// row block (routed: an upper bound; shared: S * cdiv(T, BM)).
static int64_t fused_sync_words(const moe_fwd_args& f, int64_t* mbr, int64_t* mbs) {
    const int64_t R = (int64_t)f.T * f.k;
    *mbr = (R + (int64_t)f.E * (BM - 1)) / BM;
    *mbs = cdiv(f.T, BM);
    return SY_READY + *mbr + (int64_t)f.S * *mbs;
}

extern "C" size_t moe_layer_forward_workspace_size(const moe_fwd_args* a) {
    if (!a || a->T < 1 || a->k < 1 || a->E < 1 || a->S < 0) return 0;
    int64_t mbr, mbs;
    const int64_t words = fused_sync_words(*a, &mbr, &mbs);
    return moe_align256(moe_route_workspace_size(a->T, a->k, a->E)) +
           moe_align256((size_t)words * 4);
}

extern "C" size_t moe_layer_forward_error_offset(const moe_fwd_args* a) {
    if (!a || a->T < 1 || a->k < 1 || a->E < 1) return 0;
    return moe_align256(moe_route_workspace_size(a->T, a->k, a->E)) + SY_ERR * 4;
}

extern "C" int moe_layer_forward(const moe_fwd_args* p, void* ws, size_t ws_bytes, void* stream) {
    MOE_REQUIRE(p);
    const moe_fwd_args& f = *p;
    const moe_route_cfg& cfg = f.cfg;
    MOE_REQUIRE(f.T >= 1 && f.k >= 1 && f.k <= MAXK && f.E >= 1 && f.E <= 256);
    MOE_REQUIRE(f.E_router >= 1 && f.E_router <= 64 * FUSED_NV && f.k <= f.E_router);
    MOE_REQUIRE(f.idx_in || f.E == f.E_router);
    MOE_REQUIRE(f.H >= 64 && f.H % 64 == 0 && f.I >= 64 && f.I % 64 == 0);
    MOE_REQUIRE(f.S >= 0 && f.S <= 64 && (f.S == 0 || (f.Is >= 64 && f.Is % 64 == 0)));
    const int64_t R = (int64_t)f.T * f.k;
    MOE_REQUIRE(R * f.H < (1ll << 31) && R * 2 * f.I < (1ll << 31));
    MOE_REQUIRE((int64_t)f.S * f.T * f.H < (1ll << 31) && (int64_t)f.S * f.T * 2 * f.Is < (1ll << 31));
    MOE_REQUIRE(f.x && f.logits && f.w1 && f.w2 && f.idx && f.w && f.s_sel && f.counts &&
                f.offsets && f.pos && f.src && f.xp && f.h && f.y && f.out);
    MOE_REQUIRE(f.S == 0 || (f.ws1 && f.ws2 && f.hs && f.ys));
    MOE_REQUIRE(cfg.score == MOE_SCORE_SOFTMAX || cfg.score == MOE_SCORE_SIGMOID);
    const int n_groups = cfg.n_groups < 1 ? 1 : cfg.n_groups;
    const int topk_groups = (cfg.topk_groups < 1 || n_groups == 1) ? n_groups : cfg.topk_groups;
    MOE_REQUIRE(n_groups <= 64 && f.E_router % n_groups == 0 && topk_groups <= n_groups);
    const int per_group = f.k / topk_groups < 1 ? 1 : f.k / topk_groups;
    MOE_REQUIRE(per_group <= f.E_router / n_groups && f.k <= topk_groups * (f.E_router / n_groups));
    const size_t need = moe_layer_forward_workspace_size(p);
    if (!ws || ws_bytes < need) return MOE_EWORKSPACE;
    int rc = moe_check_device();
    if (rc) return rc;
    hipStream_t st = (hipStream_t)stream;
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        ncu < 1)
        return MOE_EHIP;
    // One block per CU, as an ordinary launch.  The device-wide barriers need every block
    // resident at once: a block needs 160 KB of LDS, so no CU holds two, and the ncu blocks
    // of an otherwise idle device all start together.  Work of other streams that holds CUs
    // only delays the late blocks until it ends (the resident blocks wait at the first
    // barrier); a device that can never hold them all runs into the bounded waits, which set
    // the error word instead of hanging.  (A cooperative launch would guarantee residency up
    // front, at about 16 us more per launch, through a runtime path whose teardown faulted
    // at process exit under rocprofv3.)
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, layer_forward_fused, NTH, 0) !=
            hipSuccess || per_cu < 1)
        return MOE_EHIP;
    FusedFwd a{};
    a.wr = (const bf16_t*)f.w_router;
    a.proj = f.w_router ? f.logits : nullptr;
    a.tp = TopkParams{f.logits, cfg.sel_bias, f.T, f.E_router, f.k, cfg.score, n_groups,
                      topk_groups, per_group, cfg.renorm, cfg.route_scale, f.idx, f.w, f.s_sel};
    a.perm_ids = f.idx_in ? f.idx_in : f.idx;
    a.n = R;
    a.E = f.E;
    int nbits = 0;
    while ((1 << nbits) < f.E) ++nbits;
    a.nbits = nbits;
    a.nch = (int)((R + CHUNK - 1) / CHUNK);
    a.blk = (int32_t*)ws;
    a.counts = f.counts; a.offsets = f.offsets; a.pos = f.pos; a.src = f.src;
    a.x = (const bf16_t*)f.x;
    a.T = f.T; a.H = f.H; a.k = f.k; a.R = (int)R; a.S = f.S;
    a.xp = (bf16_t*)f.xp;
    ffn_args((const bf16_t*)f.xp, f.offsets, f.E, a.R, f.H, f.I, (const bf16_t*)f.w1,
             (const bf16_t*)f.w2, (bf16_t*)f.gu, (bf16_t*)f.h, (bf16_t*)f.y, a.g1, a.g2);
    if (f.S > 0)
        ffn_args((const bf16_t*)f.x, nullptr, f.S, f.T, f.H, f.Is, (const bf16_t*)f.ws1,
                 (const bf16_t*)f.ws2, (bf16_t*)f.gus, (bf16_t*)f.hs, (bf16_t*)f.ys, a.s1, a.s2);
    a.ys = (const bf16_t*)f.ys;
    a.out = (bf16_t*)f.out;
    int64_t mbr, mbs;
    const int64_t words = fused_sync_words(f, &mbr, &mbs);
    a.sy = (unsigned*)((char*)ws + moe_align256(moe_route_workspace_size(f.T, f.k, f.E)));
    a.mbr = (int)mbr;
    a.mbs = (int)mbs;
    // Blocks: one per CU, or fewer when no step has work for that many (every step strides
    // over the blocks, so any count gives the same outputs): the device-wide barriers then
    // have fewer blocks to gather.  The widest steps: the product queue's tiles (an upper
    // bound), four tokens per block (top-k, combine), one chunk per block (histograms), the
    // router projection's logits (256 per block).
    const int64_t tiles = mbr * (cdiv(f.I, 128) + cdiv(f.H, BN)) +
                          (f.S > 0 ? (int64_t)f.S * mbs * (cdiv(f.Is, 128) + cdiv(f.H, BN)) : 0);
    const int64_t widest = std::max<int64_t>(
        std::max<int64_t>(tiles, cdiv(f.T, 4)),
        std::max<int64_t>(a.nch, f.w_router ? ((int64_t)f.T * f.E_router + 255) / 256 : 1));
    const int grid = (int)std::min<int64_t>(ncu, std::max<int64_t>(widest, 1));
    MOE_TRACED("fused_clear", st, fused_clear<<<1, 1024, 0, st>>>(a.sy, (int)words));
    MOE_LAUNCH_CHECK();
    MOE_TRACED("layer_forward_fused", st, layer_forward_fused<<<grid, NTH, 0, st>>>(a));
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

// Backward of the FFN for one group of experts, over the rows of one pass (pointers already
// at the pass's rows; offsets [E+1] pass-local, or null in shared mode: every expert takes
// all R rows and dy / xp are one [R,H] array used by every expert).
//   dgrad: dgu [rows,2I] (dh = dy W2 with the SwiGLU backward, from the saved g|u) and
//          dxp [rows,H] = dGU W1.
//   wgrad: when wg is given, dW2 = dy^T h and dW1 = dGU^T Xp over every pass it spans, in the
//          same launches as the dgrad products (the caller passes it with the last pass, once
//          dy and dGU of all passes exist).
// The weight-gradient products over an expert's rows (of every pass): dW2_e = dy_e^T h_e
// (M = H, N = I) and dW1_e = dGU_e^T Xp_e (M = 2I, N = H).
static void wgrad_args(const MoeWgradSpan& wg, bool shared, int E, int H, int I, GemmArgs& gw,
                       GemmArgs& gw2) {
    gw = blank();
    gw.A = wg.dy; gw.a_es = 0; gw.lda = H;
    gw.B = wg.h; gw.b_es = shared ? (int64_t)wg.R * I : 0; gw.ldb = I;
    gw.C = wg.dw2; gw.c_es = (int64_t)H * I; gw.ldc = I;
    gw.offsets = wg.offsets; gw.E = E; gw.R = wg.R; gw.M = H; gw.N = I; gw.I = I;
    gw.P = wg.P; gw.pass_rows = wg.pass_rows;
    gw.total = E * cdiv(H, BM) * cdiv(I, BN);
    gw2 = blank();
    gw2.A = wg.dgu; gw2.a_es = shared ? (int64_t)wg.R * 2 * I : 0; gw2.lda = 2 * I;
    gw2.B = wg.xp; gw2.b_es = 0; gw2.ldb = H;
    gw2.C = wg.dw1; gw2.c_es = (int64_t)2 * I * H; gw2.ldc = H;
    gw2.offsets = wg.offsets; gw2.E = E; gw2.R = wg.R; gw2.M = 2 * I; gw2.N = H; gw2.I = I;
    gw2.P = wg.P; gw2.pass_rows = wg.pass_rows;
    gw2.total = E * cdiv(2 * I, BM) * cdiv(H, BN);
}

// The two weight-gradient products alone (BF16), for the backward whose dgrad products run
// in MXFP8: the launches of the BF16 backward with no dgrad tiles.
int moe_ffn_wgrad_bf16(const MoeWgradSpan* wg, int E, int H, int I, hipStream_t st) {
    GemmArgs none = blank(), gw, gw2;
    wgrad_args(*wg, false, E, H, I, gw, gw2);
    int rc = launch_pair(bwd_down, "wgrad_down", none, gw, st);
    if (rc) return rc;
    return launch_pair(bwd_gate_up, "wgrad_gate_up", none, gw2, st);
}

int moe_ffn_bwd_bf16(const bf16_t* xp, const int32_t* offsets, int E, int R, int H, int I,
                     const bf16_t* w1, const bf16_t* w2, const bf16_t* gu, const bf16_t* h,
                     const bf16_t* dy, bf16_t* dgu, bf16_t* dxp, const MoeWgradSpan* wg,
                     hipStream_t st) {
    (void)xp;
    const bool shared = offsets == nullptr;
    int rc;
    // dh = dy_e W2_e (W2_e is [H,I]: N-contiguous in I), SwiGLU backward -> dgu
    GemmArgs gd = blank();
    gd.A = dy; gd.a_es = 0; gd.lda = H;
    gd.B = w2; gd.b_es = (int64_t)H * I; gd.ldb = I; gd.b_rows = H;
    gd.C = dgu; gd.c_es = shared ? (int64_t)R * 2 * I : 0; gd.ldc = 2 * I;
    gd.C2 = const_cast<bf16_t*>(gu); gd.c2_es = shared ? (int64_t)R * 2 * I : 0; gd.ldc2 = 2 * I;
    gd.offsets = offsets; gd.E = E; gd.R = R; gd.N = I; gd.K = H; gd.I = I;
    gd.total = shared ? E * cdiv(R, BM) * cdiv(I, BN) : 0;
    GemmArgs gw = blank(), gw2 = blank();
    if (wg) wgrad_args(*wg, shared, E, H, I, gw, gw2);
    rc = launch_pair(bwd_down, "bwd_down", gd, gw, st);
    if (rc) return rc;
    // dXp = dGU_e W1_e (W1_e is [2I,H]: N-contiguous in H)
    GemmArgs gd2 = blank();
    gd2.A = dgu; gd2.a_es = shared ? (int64_t)R * 2 * I : 0; gd2.lda = 2 * I;
    gd2.B = w1; gd2.b_es = (int64_t)2 * I * H; gd2.ldb = H; gd2.b_rows = 2 * I;
    gd2.C = dxp; gd2.c_es = shared ? (int64_t)R * H : 0; gd2.ldc = H;
    gd2.offsets = offsets; gd2.E = E; gd2.R = R; gd2.N = H; gd2.K = 2 * I; gd2.I = I;
    gd2.total = shared ? E * cdiv(R, BM) * cdiv(H, BN) : 0;
    rc = launch_pair(bwd_gate_up, "bwd_gate_up", gd2, gw2, st);
    if (rc) return rc;
    return MOE_OK;
}
