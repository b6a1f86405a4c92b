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
//  - 256x256 output tile per 256-thread block, 4 waves in 2x2, each wave a 128x128 sub-tile
//    of 4x4 v_mfma_f32_32x32x16_bf16 accumulators (256 fp32 per lane, one wave per SIMD).
//  - K steps of 32 through a ring of 4 LDS stages (128 KB), filled by direct global-to-LDS
//    buffer loads three steps ahead of their use; one barrier per step.
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
#include "pipe.h"

namespace moe {

constexpr int BM = 256, BN = 256, BK = 32, NTH = 256;
constexpr int KK = BK / 16;   // 32x32x16 MFMA sub-steps per K step
constexpr int NST = 4;        // pipeline stages (K steps resident or in flight)
constexpr int GM = 4;         // M tiles per L2 group

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
};

// ---------------------------------------------------------------- LDS tiles
// One pipeline stage holds one K step (BK = 32) of both operands, 16 KB each.  Two layouts:
//  K-major   (operand contiguous along K in memory): tile row r (an M or N index) is 64 bytes,
//            four 16-byte chunks of 8 k values; chunk c is stored at chunk c ^ kswz(r).  The
//            rows read by one 128-byte (8-lane) or 256-byte (16-lane) phase of a fragment read
//            then hit distinct bank groups.
//  MN-major  (operand contiguous along M or N): k-row kr is 512 bytes, 32 chunks of 8 m (n)
//            values; chunk c is stored at chunk c ^ mswz(kr % 4), mswz = {0, 6, 10, 12}, so
//            the k-rows and columns read by one 16-lane (128-byte) or 32-lane (256-byte) phase
//            of a transpose read hit distinct banks.
// Both are filled by direct global-to-LDS loads (buffer_load ... lds): lane L of a wave
// writes 16 bytes at LDS base + 16 L, so each lane fetches the global chunk that belongs at
// its LDS position and the swizzle lives entirely in the global offsets.
constexpr int KROW = BK * 2;          // bytes of one K-major tile row
constexpr int OPB = 256 * BK * 2;     // bytes of one operand in one stage
constexpr int LPW = OPB / 1024 / 4;   // direct-load instructions per operand per wave per step
constexpr int LPS = 2 * LPW;          // ... for both operands

__device__ __forceinline__ int mswz(int kr) { return (0xCA60 >> (4 * (kr & 3))) & 15; }

typedef short i16x4 __attribute__((ext_vector_type(4)));

// Transposed 8-byte LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes, lane i
// receives element i % 4 of the 8-byte chunks addressed by lanes i/4 + 4j, j = 0..3.
__device__ __forceinline__ i16x4 lds_read_tr(const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(p));
}

// Per-lane description of one operand's global->LDS loads (LPW per wave per K step) and of
// its MFMA fragment reads (4 sub-tiles of 32 rows per wave).
struct Operand {
    rsrc_t r;
    uint32_t voff[LPW];  // byte offset of this lane's 16-byte chunk, per load instruction
    uint32_t kstep;      // byte advance of the global offset per K step
    int ldsrow[LPW];     // LDS byte offset (within the operand's stage area) per instruction
    uint32_t rd[4];      // fragment-read base offset per sub-tile
    int rs[4];           // K-major: swizzle bit 1 of the sub-tile's row
};

// K-major operand.  rowmap(nn) gives the global row (relative to the descriptor base) of
// tile row nn.  Each wave loads 64 tile rows, 16 rows per instruction.
template <typename RowMap>
__device__ __forceinline__ void setup_kmajor(Operand& o, const void* base, uint32_t bytes, int ld,
                                             int wid, int lane, int wsub, RowMap rowmap) {
    o.r = make_rsrc(base, bytes);
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int r = 64 * wid + 16 * i + (lane >> 2);
        const int c = (lane & 3) ^ kswz(r);
        o.voff[i] = (uint32_t)rowmap(r) * (uint32_t)ld * 2u + (uint32_t)c * 16u;
        o.ldsrow[i] = (64 * wid + 16 * i) * KROW;
    }
    o.kstep = BK * 2;
    // fragment reads: lane reads row rb + lane%32, logical chunk 2 kk + lane/32
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int r = wsub + 32 * t + (lane & 31);
        const int s = kswz(r);
        o.rd[t] = (uint32_t)(r * KROW) | ((uint32_t)(((lane >> 5) ^ s) & 1) << 4);
        o.rs[t] = s & 2;
    }
}

// MN-major operand: element (mn, k) at base + k*ld + mn (bytes x2).  Each wave loads
// BK/4 k-rows of the step, 2 per instruction.
__device__ __forceinline__ void setup_mnmajor(Operand& o, const void* base, uint32_t bytes, int ld,
                                              int wid, int lane, int wsub) {
    o.r = make_rsrc(base, bytes);
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int kr = (BK / 4) * wid + 2 * i + (lane >> 5);
        const int c = (lane & 31) ^ mswz(kr);
        o.voff[i] = (uint32_t)kr * (uint32_t)ld * 2u + (uint32_t)c * 16u;
        o.ldsrow[i] = ((BK / 4) * wid + 2 * i) * 512;
    }
    o.kstep = (uint32_t)BK * (uint32_t)ld * 2u;
    // transpose reads: lane group g = lane/16, q = lane%4, j = (lane%16)/4 reads k-row
    // 16 kk + 8 (g/2) + 4 h + j at columns mnb + 16 (g%2) + 4 q .. +3
    const int gq = lane >> 4, q = lane & 3, j = (lane >> 2) & 3;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int mn = wsub + 32 * t + 16 * (gq & 1) + 4 * q;
        const int kr = 8 * (gq >> 1) + j;
        const int pc = (mn >> 3) ^ mswz(j);
        o.rd[t] = (uint32_t)(kr * 512 + pc * 16 + 8 * (q & 1));
        o.rs[t] = 0;
    }
}

// Load instruction i of K step ks into the operand's area of a stage.  Steps past the end
// of K use an empty descriptor: the load still issues (so every step issues the same number
// of loads and the wait counts are constants) but fetches nothing and writes zeros.
__device__ __forceinline__ void issue_load(const Operand& o, uint32_t stage_op, int i, rsrc_t r,
                                           uint32_t soff) {
    lds_load16(r, stage_op + (uint32_t)o.ldsrow[i], o.voff[i], soff);
}

// Bytes of an MN-major operand range: `rows` k-rows of `ld` elements from column offset m0.
__device__ __forceinline__ uint32_t mn_bytes(int rows, int ld, int m0) {
    return (uint32_t)max((int64_t)rows * ld * 2 - (int64_t)m0 * 2, (int64_t)0);
}

// The 32x32x16 MFMA fragment of sub-tile t at k sub-step kk: 8 bf16 (k = 8 (lane/32) .. +7 of
// the sub-step) of row (or column) lane % 32.
template <bool KMAJ>
__device__ __forceinline__ bf16x8 read_frag(const Operand& o, const char* stage_op, int t, int kk) {
    if (KMAJ) {
        const uint32_t off = o.rd[t] + ((uint32_t)((2 * kk) ^ o.rs[t]) << 4);
        return *reinterpret_cast<const bf16x8*>(stage_op + off);
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
    char st[NST][2 * OPB];
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

// One 256 x 256 output tile, number `logical` of the product (tiles run in launch order: the
// blocks in flight at once, spread over all XCDs, work on neighbouring tiles whose operand
// panels meet in the shared last-level cache, which measured faster than giving each XCD
// its own compact block of tiles).
template <bool A_K, bool B_K, int EPI, bool GK>
__device__ __forceinline__ void gemm_tile(const GemmArgs& g, GemmSmem& sm, const int logical) {
    const int tid = threadIdx.x, lane = tid & 63, wid = uni(tid >> 6);
    const int wm = wid >> 1, wn = wid & 1;
    const int NT = n_tiles<EPI>(g);
    const bool ragged_m = !GK && g.offsets != nullptr;
    int e, t_local, Mrows, row0;
    if (ragged_m) {
        int ee = 0, first = 0;
        ragged_scan(g, NT, logical, &ee, &first);
        e = uni(ee);
        t_local = uni(logical - first);
        int a = min(max(g.offsets[e], 0), g.R);
        int b = min(max(g.offsets[e + 1], a), g.R);
        row0 = uni(a);
        Mrows = uni(b - a);
    } else {
        int per = GK ? cdiv(g.M, BM) * NT : cdiv(g.R, BM) * NT;
        e = logical / per;
        t_local = logical - e * per;
        if (GK) {
            if (g.offsets) {
                // K extent: the expert's rows (of the first pass when P > 1)
                const int lim = g.P > 1 ? g.pass_rows : g.R;
                int a = min(max(g.offsets[e], 0), lim);
                int b = min(max(g.offsets[e + 1], a), lim);
                row0 = uni(a);
                Mrows = uni(b - a);
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
    const int n0 = tn * BN;
    const int ch0 = tn * 128;  // SwiGLU channel base

    // ---------------------------------------------------------------- operands
    // A: K-major rows m at A_e + (row0 + m)*lda; or MN-major (wgrad): (m, k) at
    //    A_e + (row0 + k)*lda + m.
    // B: K-major rows n at B_e + n*ldb (SwiGLU: gate and up rows interleaved so a tile holds
    //    128 channels of each); or MN-major: (n, k) at B_e + (kbase + k)*ldb + n, kbase = row0
    //    for wgrad (the expert's tokens), else 0 (a weight with K rows).
    Operand oa, ob;
    if (A_K) {
        const bf16_t* base = g.A + e * g.a_es + (int64_t)(row0 + m0) * g.lda;
        setup_kmajor(oa, base, (uint32_t)max(Mrows - m0, 0) * (uint32_t)g.lda * 2u, g.lda, wid,
                     lane, wm * 128, [](int r) { return r; });
    } else {
        const bf16_t* base = g.A + e * g.a_es + (int64_t)row0 * g.lda + m0;
        setup_mnmajor(oa, base, mn_bytes(Kdim, g.lda, m0), g.lda, wid, lane, wm * 128);
    }
    if (B_K) {
        const bf16_t* base = g.B + e * g.b_es;
        const int I = g.I;
        if (EPI == EPI_SWIGLU)
            setup_kmajor(ob, base, (uint32_t)g.b_rows * (uint32_t)g.ldb * 2u, g.ldb, wid, lane,
                         wn * 128, [=](int nn) {
                             int q = nn & 127;
                             return (q >> 6) * I + ch0 + (nn >> 7) * 64 + (q & 63);
                         });
        else
            setup_kmajor(ob, base, (uint32_t)g.b_rows * (uint32_t)g.ldb * 2u, g.ldb, wid, lane,
                         wn * 128, [=](int nn) { return n0 + nn; });
    } else {
        const int64_t kbase = GK ? row0 : 0;
        const bf16_t* base = g.B + e * g.b_es + kbase * g.ldb + n0;
        setup_mnmajor(ob, base, mn_bytes(Kdim, g.ldb, n0), g.ldb, wid, lane, wn * 128);
    }

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    // ---------------------------------------------------------------- main loop
    // NST stages in a ring: at the end of K step ks the stage it used is refilled with step
    // ks + NST, so every load has NST - 1 steps to land.  A step is two sub-steps of 16 k
    // (16 MFMAs each).  The LDS reads of the next sub-step's fragments and the global->LDS
    // loads are interleaved one per MFMA, so they issue while the MFMA pipe is busy; the step
    // barrier (all waves done reading this stage; step ks+1 landed) sits between the two
    // sub-steps.  Fragment reads follow the order the MFMAs consume them.
    // The MFMA takes the B fragment as its first operand, so each lane's accumulators hold
    // one output row (m) and 4-column runs (n): the epilogue stores 8-byte vectors.
    static_assert(KK == 2 && LPW == 4 && NST >= 3, "the step below is written for these");
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
    bf16x8 fa[2][4], fb[2][4];
    // read number r (0..7) of a sub-step, in MFMA consumption order: a0 b0 b1 b2 b3 a1 a2 a3
    auto read_one = [&](const char* st, int kk, int f, int r) __attribute__((always_inline)) {
        if (r == 0) fa[f][0] = read_frag<A_K>(oa, st, 0, kk);
        else if (r <= 4) fb[f][r - 1] = read_frag<B_K>(ob, st + OPB, r - 1, kk);
        else fa[f][r - 4] = read_frag<A_K>(oa, st, r - 4, kk);
    };
    auto mfma_one = [&](int f, int n) __attribute__((always_inline)) {
        const int i = n >> 2, j = n & 3;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[f][j], fa[f][i], acc[i][j], 0, 0, 0);
    };
    auto kstep = [&](char* cur, char* nxt, uint32_t cur32, int ks) __attribute__((always_inline)) {
        // sub-step 0 (fragments f = 0) with the reads of sub-step 1
#pragma unroll
        for (int n = 0; n < 16; ++n) {
            mfma_one(0, n);
            if (n < 8) read_one(cur, 1, 1, n);
            __builtin_amdgcn_sched_barrier(0);
        }
        wait_vm_lgkm0<(NST - 2) * LPS>();  // step ks+1 landed (later steps may be in flight)
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        // sub-step 1 (f = 1) with the loads of step ks+NST into this stage and the reads of
        // the next step's sub-step 0
        const bool more = ks + 1 < nk;
        rsrc_t ra_, rb_;
        uint32_t sa, sb;
        load_src(ks + NST, ra_, rb_, sa, sb);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int n = 0; n < 16; ++n) {
            mfma_one(1, n);
            if (n < 4) issue_load(oa, cur32, n, ra_, sa);
            else if (n < 8) issue_load(ob, cur32 + OPB, n - 4, rb_, sb);
            else if (more) read_one(nxt, 0, 0, n - 8);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if (nk > 0) {
        const uint32_t st_base = lds_addr(sm.st[0]);  // stage p at st_base + p * 2 * OPB
#pragma unroll
        for (int p = 0; p < NST; ++p) {
            rsrc_t ra_, rb_;
            uint32_t sa, sb;
            load_src(p, ra_, rb_, sa, sb);
#pragma unroll
            for (int i = 0; i < LPW; ++i) {
                issue_load(oa, st_base + p * 2 * OPB, i, ra_, sa);
                issue_load(ob, st_base + p * 2 * OPB + OPB, i, rb_, sb);
            }
        }
        wait_vm_lgkm0<(NST - 1) * LPS>();  // step 0 landed
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < 8; ++r) read_one(sm.st[0], 0, 0, r);
        for (int ks = 0; ks < nk; ks += NST) {
#pragma unroll
            for (int u = 0; u < NST; ++u)
                if (ks + u < nk)
                    kstep(sm.st[u], sm.st[(u + 1) % NST], st_base + u * 2 * OPB, ks + u);
        }
        wait_vm_lgkm0<0>();  // no load may still be writing LDS when the block ends
    }

    // ---------------------------------------------------------------- epilogue
    // Accumulator layout (B fragment first): lane l holds row l % 32 of its 32x32 block and
    // columns 8 (v/4) + 4 (l/32) + v%4, v = 0..15: four runs of 4 consecutive columns.
    const int lrow = lane & 31, lcol = (lane >> 5) * 4;
    if (EPI == EPI_STORE) {
        bf16_t* C = g.C + e * g.c_es + (GK ? 0 : (int64_t)row0 * g.ldc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = m0 + wm * 128 + i * 32 + lrow;
            if (row >= Mvalid) continue;
            bf16_t* Crow = C + (int64_t)row * g.ldc;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int col = n0 + wn * 128 + j * 32 + 8 * q + lcol;
                    if (col < g.N) {
                        uint2 v = make_uint2(pack_bf2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                                             pack_bf2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]));
                        *reinterpret_cast<uint2*>(Crow + col) = v;
                    }
                }
        }
    } else if (EPI == EPI_SWIGLU) {
        bf16_t* C = g.C + e * g.c_es + (int64_t)row0 * g.ldc;
        bf16_t* C2 = g.C2 ? g.C2 + e * g.c2_es + (int64_t)row0 * g.ldc2 : nullptr;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = m0 + wm * 128 + i * 32 + lrow;
            if (row >= Mvalid) continue;
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int ch = ch0 + wn * 64 + j * 32 + 8 * q + lcol;
                    if (ch >= g.I) continue;
                    float hv[4];
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const float gv = acc[i][j][4 * q + c], uv = acc[i][j + 2][4 * q + c];
                        hv[c] = gv / (1.0f + __expf(-gv)) * uv;
                    }
                    *reinterpret_cast<uint2*>(C + (int64_t)row * g.ldc + ch) =
                        make_uint2(pack_bf2(hv[0], hv[1]), pack_bf2(hv[2], hv[3]));
                    if (C2) {
                        bf16_t* gr = C2 + (int64_t)row * g.ldc2;
                        *reinterpret_cast<uint2*>(gr + ch) =
                            make_uint2(pack_bf2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                                       pack_bf2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]));
                        *reinterpret_cast<uint2*>(gr + g.I + ch) =
                            make_uint2(pack_bf2(acc[i][j + 2][4 * q], acc[i][j + 2][4 * q + 1]),
                                       pack_bf2(acc[i][j + 2][4 * q + 2], acc[i][j + 2][4 * q + 3]));
                    }
                }
        }
    } else {  // EPI_DSWIGLU: acc = dh; read saved g|u, write dg|du
        bf16_t* C = g.C + e * g.c_es + (int64_t)row0 * g.ldc;
        const bf16_t* GU = g.C2 + e * g.c2_es + (int64_t)row0 * g.ldc2;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = m0 + wm * 128 + i * 32 + lrow;
            if (row >= Mvalid) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int ch = n0 + wn * 128 + j * 32 + 8 * q + lcol;
                    if (ch >= g.N) continue;
                    const uint2 gg = *reinterpret_cast<const uint2*>(GU + (int64_t)row * g.ldc2 + ch);
                    const uint2 uu = *reinterpret_cast<const uint2*>(GU + (int64_t)row * g.ldc2 + g.I + ch);
                    const float gv[4] = {lo_bf(gg.x), hi_bf(gg.x), lo_bf(gg.y), hi_bf(gg.y)};
                    const float uv[4] = {lo_bf(uu.x), hi_bf(uu.x), lo_bf(uu.y), hi_bf(uu.y)};
                    float dg[4], du[4];
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const float dh = acc[i][j][4 * q + c];
                        const float sg = 1.0f / (1.0f + __expf(-gv[c]));
                        dg[c] = dh * uv[c] * sg * (1.0f + gv[c] * (1.0f - sg));
                        du[c] = dh * gv[c] * sg;
                    }
                    bf16_t* cr = C + (int64_t)row * g.ldc;
                    *reinterpret_cast<uint2*>(cr + ch) =
                        make_uint2(pack_bf2(dg[0], dg[1]), pack_bf2(dg[2], dg[3]));
                    *reinterpret_cast<uint2*>(cr + g.I + ch) =
                        make_uint2(pack_bf2(du[0], du[1]), pack_bf2(du[2], du[3]));
                }
        }
    }
}

// One kernel symbol per product of the layer, so that profiles name each role.
#define MOE_GEMM_KERNEL(NAME, AKM, BKM, EPI, GK)                                       \
    __global__ __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(1, 1))) void \
    NAME(GemmArgs g) {                                                                 \
        __shared__ GemmSmem sm;                                                        \
        const int total = tile_total<EPI, GK>(g);                                      \
        if ((int)blockIdx.x < total) gemm_tile<AKM, BKM, EPI, GK>(g, sm, blockIdx.x);  \
    }
MOE_GEMM_KERNEL(gemm1_swiglu, true, true, EPI_SWIGLU, false)     // [g|u] = Xp W1^T, h
MOE_GEMM_KERNEL(gemm2_down, true, true, EPI_STORE, false)        // y = h W2^T
#undef MOE_GEMM_KERNEL

// The backward's two pairs of independent products run as one launch each, the dgrad tiles
// first and the wgrad tiles after them, so that the second product fills the last,
// partly empty round of the first (256 CUs, one tile each at a time).
//   bwd_down:     dh = dy W2 -> dg|du (SwiGLU backward)   and   dW2 = dy^T h
//   bwd_gate_up:  dXp = dGU W1                           and   dW1 = dGU^T Xp
__global__ __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_down(GemmArgs gd, GemmArgs gw) {
    __shared__ GemmSmem sm;
    const int td = tile_total<EPI_DSWIGLU, false>(gd);
    const int b = blockIdx.x;
    if (b < td) gemm_tile<true, false, EPI_DSWIGLU, false>(gd, sm, b);
    else if (b - td < gw.total) gemm_tile<false, false, EPI_STORE, true>(gw, sm, b - td);
}

__global__ __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_gate_up(GemmArgs gd, GemmArgs gw) {
    __shared__ GemmSmem sm;
    const int td = tile_total<EPI_STORE, false>(gd);
    const int b = blockIdx.x;
    if (b < td) gemm_tile<true, false, EPI_STORE, false>(gd, sm, b);
    else if (b - td < gw.total) gemm_tile<false, false, EPI_STORE, true>(gw, sm, b - td);
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
    MOE_TRACED(name, st, kern<<<grid, NTH, 0, st>>>(g));
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

static int launch_pair(void (*kern)(GemmArgs, GemmArgs), const char* name, const GemmArgs& gd,
                       const GemmArgs& gw, hipStream_t st) {
    const int grid = grid_of(gd, cdiv(gd.N, BN), false) + gw.total;
    if (grid <= 0) return MOE_OK;
    MOE_TRACED(name, st, kern<<<grid, NTH, 0, st>>>(gd, gw));
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
    int rc = launch(gemm1_swiglu, "gemm1_swiglu", g, cdiv(I, 128), st);
    if (rc) return rc;
    GemmArgs g2 = blank();
    g2.A = h; g2.a_es = shared ? (int64_t)R * I : 0; g2.lda = I;
    g2.B = w2; g2.b_es = (int64_t)H * I; g2.ldb = I; g2.b_rows = H;
    g2.C = y; g2.c_es = shared ? (int64_t)R * H : 0; g2.ldc = H;
    g2.offsets = offsets; g2.E = E; g2.R = R; g2.N = H; g2.K = I; g2.I = I;
    g2.total = shared ? E * cdiv(R, BM) * cdiv(H, BN) : 0;
    return launch(gemm2_down, "gemm2_down", g2, cdiv(H, BN), st);
}

// Backward of the FFN for one group of experts, over the rows of one pass (pointers already
// at the pass's rows; offsets [E+1] pass-local, or null in shared mode: every expert takes
// all R rows and dy / xp are one [R,H] array used by every expert).
//   dgrad: dgu [rows,2I] (dh = dy W2 with the SwiGLU backward, from the saved g|u) and
//          dxp [rows,H] = dGU W1.
//   wgrad: when wg is given, dW2 = dy^T h and dW1 = dGU^T Xp over every pass it spans, in the
//          same launches as the dgrad products (the caller passes it with the last pass, once
//          dy and dGU of all passes exist).
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
    // dW2_e = dy_e^T h_e: M = H, N = I, K = the expert's rows (of every pass)
    GemmArgs gw = blank();
    if (wg) {
        gw.A = wg->dy; gw.a_es = 0; gw.lda = H;
        gw.B = wg->h; gw.b_es = shared ? (int64_t)wg->R * I : 0; gw.ldb = I;
        gw.C = wg->dw2; gw.c_es = (int64_t)H * I; gw.ldc = I;
        gw.offsets = wg->offsets; gw.E = E; gw.R = wg->R; gw.M = H; gw.N = I; gw.I = I;
        gw.P = wg->P; gw.pass_rows = wg->pass_rows;
        gw.total = E * cdiv(H, BM) * cdiv(I, BN);
    }
    rc = launch_pair(bwd_down, "bwd_down", gd, gw, st);
    if (rc) return rc;
    // dXp = dGU_e W1_e (W1_e is [2I,H]: N-contiguous in H)
    GemmArgs gd2 = blank();
    gd2.A = dgu; gd2.a_es = shared ? (int64_t)R * 2 * I : 0; gd2.lda = 2 * I;
    gd2.B = w1; gd2.b_es = (int64_t)2 * I * H; gd2.ldb = H; gd2.b_rows = 2 * I;
    gd2.C = dxp; gd2.c_es = shared ? (int64_t)R * H : 0; gd2.ldc = H;
    gd2.offsets = offsets; gd2.E = E; gd2.R = R; gd2.N = H; gd2.K = 2 * I; gd2.I = I;
    gd2.total = shared ? E * cdiv(R, BM) * cdiv(H, BN) : 0;
    // dW1_e = dGU_e^T Xp_e: M = 2I, N = H
    GemmArgs gw2 = blank();
    if (wg) {
        gw2.A = wg->dgu; gw2.a_es = shared ? (int64_t)wg->R * 2 * I : 0; gw2.lda = 2 * I;
        gw2.B = wg->xp; gw2.b_es = 0; gw2.ldb = H;
        gw2.C = wg->dw1; gw2.c_es = (int64_t)2 * I * H; gw2.ldc = H;
        gw2.offsets = wg->offsets; gw2.E = E; gw2.R = wg->R; gw2.M = 2 * I; gw2.N = H; gw2.I = I;
        gw2.P = wg->P; gw2.pass_rows = wg->pass_rows;
        gw2.total = E * cdiv(2 * I, BM) * cdiv(H, BN);
    }
    rc = launch_pair(bwd_gate_up, "bwd_gate_up", gd2, gw2, st);
    if (rc) return rc;
    return MOE_OK;
}
