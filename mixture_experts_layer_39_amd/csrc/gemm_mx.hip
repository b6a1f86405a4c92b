// MXFP8 grouped GEMMs of the expert FFN forward (E4M3 codes, one E8M0 scale per 32 values
// along K) on gfx950's scaled MFMA, v_mfma_scale_f32_32x32x64_f8f6f4.  The MXFP8 forward is
// the path the pages report the largest gain on (pulsen.vercel.app, "Cursor åpner
// megakernelen…", ¶3; aiexpert.news, "Megakernels are dead and back", ¶4).
//   GEMM1: [g|u] = Xq_e W1q_e^T, epilogue h = silu(g)*u in fp32.
//   GEMM2: y = hq_e W2q_e^T, bf16 output (h MX-quantised along I in between).
//
// The pipeline of the BF16 kernels, for byte codes: 256x256 tiles, 4 waves of 128x128, K steps
// of 64 codes (one 64-byte swizzled LDS row per operand row) through a ring of 4 LDS stages
// filled by direct global-to-LDS loads three steps ahead, loads and LDS reads interleaved one
// per MFMA, buffer loads that zero-fill past an expert's rows, device-side expert tile lists,
// tiles in launch order.  The E8M0 scales travel through LDS in groups of 8 K steps (16 bytes
// per row), double-buffered; each lane hands the MFMA the scale of its row in the 32-code
// block its lane group stands for.
#include "pipe.h"

namespace moe {

constexpr int XBM = 256, XBN = 256, XBK = 64, XNTH = 256;  // XBK: codes (bytes) per K step
constexpr int XNST = 4;                  // pipeline stages
constexpr int XGM = 4;                   // M tiles per L2 group
constexpr int XOPB = 256 * XBK;          // bytes of one operand in one stage
constexpr int XLPW = XOPB / 1024 / 4;    // direct loads per operand per wave per step
constexpr int XLPS = 2 * XLPW;           // ... for both operands
constexpr int SGRP = 8;                  // K steps per scale group (16 E8M0 bytes per row)
constexpr int SOPB = 256 * 16;           // bytes of one operand's scale group

enum { XEPI_SWIGLU_F32 = 0, XEPI_STORE_BF16 = 1 };

struct MxArgs {
    const uint8_t* A;   // codes [rows, K]
    const uint8_t* As;  // scales [rows, K/32]
    int64_t a_es;       // per-expert row stride (shared mode), in rows
    const uint8_t* B;   // codes [E, b_rows, K]
    const uint8_t* Bs;  // scales [E, b_rows, K/32]
    int b_rows;
    void* C;            // SwiGLU: fp32 h [rows, I];  store: bf16 y [rows, N]
    int64_t c_es;       // per-expert row stride of C (shared mode), in rows
    int ldc;
    const int32_t* offsets;
    int E, R, N, K, I;
    int total;
};

struct alignas(1024) MxSmem {
    char st[XNST][2 * XOPB];  // code stages: A then B
    char sc[2][2 * SOPB];     // scale groups: A then B, 16 bytes per tile row
    int tp[1024];
    int total;
};

typedef int i32x8 __attribute__((ext_vector_type(8)));

template <int EPI>
__device__ __forceinline__ int mx_n_tiles(const MxArgs& g) {
    return (EPI == XEPI_SWIGLU_F32) ? cdiv(g.I, 128) : cdiv(g.N, XBN);
}

template <int EPI>
__device__ __forceinline__ int mx_tile_total(const MxArgs& g, MxSmem& sm) {
    if (g.offsets == nullptr) return g.total;
    const int lane = threadIdx.x & 63;
    const int NT = mx_n_tiles<EPI>(g);
    if (threadIdx.x < 64) {
        int run = 0;
        for (int base = 0; base < g.E; base += 64) {
            int e = base + lane, tiles = 0;
            if (e < g.E) {
                int lo = min(max(g.offsets[e], 0), g.R);
                int hi = min(max(g.offsets[e + 1], lo), g.R);
                tiles = cdiv(hi - lo, XBM) * NT;
            }
            int inc = wave_incl_scan(tiles) + run;
            if (e < g.E) sm.tp[e] = inc;
            run = __shfl(inc, 63, 64);
        }
        if (lane == 0) sm.total = run;
    }
    __syncthreads();
    return uni(sm.total);
}

template <int EPI>
__device__ __forceinline__ void mx_tile(const MxArgs& g, MxSmem& sm, const int logical) {
    const int tid = threadIdx.x, lane = tid & 63, wid = uni(tid >> 6);
    const int wm = wid >> 1, wn = wid & 1;
    const int NT = mx_n_tiles<EPI>(g);
    const int K = g.K, KB = g.K / 32;

    int e, t_local, Mrows, row0;
    if (g.offsets) {
        int lo = 0, hi = g.E - 1;
        while (lo < hi) {
            int mid = (lo + hi) >> 1;
            if (sm.tp[mid] > logical) hi = mid; else lo = mid + 1;
        }
        e = uni(lo);
        t_local = uni(logical - (e ? sm.tp[e - 1] : 0));
        int a = min(max(g.offsets[e], 0), g.R);
        int b = min(max(g.offsets[e + 1], a), g.R);
        row0 = uni(a);
        Mrows = uni(b - a);
    } else {
        int per = cdiv(g.R, XBM) * NT;
        e = logical / per;
        t_local = logical - e * per;
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

    // tile row -> B row (SwiGLU: 128 gate rows and the matching 128 up rows per tile)
    auto brow = [&](int nn) __attribute__((always_inline)) {
        if (EPI == XEPI_SWIGLU_F32) {
            int q = nn & 127;
            return (q >> 6) * g.I + ch0 + (nn >> 7) * 64 + (q & 63);
        }
        return n0 + nn;
    };
    // ---------------------------------------------------------------- operands
    const int64_t arow = (int64_t)e * g.a_es + row0 + m0;
    const uint32_t arows = (uint32_t)max(Mrows - m0, 0);
    const rsrc_t ra = make_rsrc(g.A + arow * K, arows * (uint32_t)K);
    const rsrc_t ras = make_rsrc(g.As + arow * KB, arows * (uint32_t)KB);
    const rsrc_t rb = make_rsrc(g.B + (int64_t)e * g.b_rows * K, (uint32_t)g.b_rows * (uint32_t)K);
    const rsrc_t rbs = make_rsrc(g.Bs + (int64_t)e * g.b_rows * KB, (uint32_t)g.b_rows * (uint32_t)KB);
    // code loads: wave w loads tile rows 64w .. 64w+63, 16 rows per instruction; lane L of an
    // instruction writes LDS row base + L/4, chunk L%4, which holds logical chunk
    // (L%4) ^ kswz(row)
    uint32_t va[XLPW], vb[XLPW];
    int ldsrow[XLPW];
#pragma unroll
    for (int i = 0; i < XLPW; ++i) {
        const int r = 64 * wid + 16 * i + (lane >> 2);
        const int c = (lane & 3) ^ kswz(r);
        va[i] = (uint32_t)r * (uint32_t)K + (uint32_t)c * 16u;
        vb[i] = (uint32_t)brow(r) * (uint32_t)K + (uint32_t)c * 16u;
        ldsrow[i] = (64 * wid + 16 * i) * XBK;
    }
    // scale loads: wave w loads the 16-byte group entries of tile rows 64w .. 64w+63
    const uint32_t vas = (uint32_t)(64 * wid + lane) * (uint32_t)KB;
    const uint32_t vbs = (uint32_t)brow(64 * wid + lane) * (uint32_t)KB;
    // fragment reads: lane reads row (sub-tile base) + lane%32, logical chunks g and g+2
    // (g = lane/32).  Sub-tile bases are multiples of 32, so the row swizzle is the lane's.
    const int gsel = lane >> 5;
    const uint32_t rowa = (uint32_t)(wm * 128 + (lane & 31)), rowb = (uint32_t)(wn * 128 + (lane & 31));
    const uint32_t clo = (uint32_t)((gsel ^ kswz(lane & 31)) << 4);
    const uint32_t chi = (uint32_t)(((gsel + 2) ^ kswz(lane & 31)) << 4);

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    // ---------------------------------------------------------------- main loop
    // One K step = 64 codes = one scaled MFMA per sub-tile pair (16 per wave).  At the top of
    // each step one barrier certifies that step ks+1 has landed and that every wave has read
    // step ks; the step's MFMAs then interleave the loads of step ks+4 into the stage just
    // freed and the reads of step ks+1's fragments and scales.
    //
    // Operand layout of the 32x32x64 scaled MFMA: lane group g = lane/32 holds codes
    // [16g, 16g+16) of each of the instruction's two 32-code blocks (first block in bytes
    // 0-15, second in 16-31), and the scale of lane l is that of row l%32 in block g.
    const int nk = cdiv(K, XBK);
    const int ngrp = cdiv(nk, SGRP);
    const rsrc_t rnull = make_rsrc(nullptr, 0);
    const uint32_t sa0 = lds_addr(sm.st[0]), sa1 = lds_addr(sm.st[1]), sa2 = lds_addr(sm.st[2]),
                   sa3 = lds_addr(sm.st[3]);
    const uint32_t stg[XNST] = {sa0, sa1, sa2, sa3};
    const uint32_t sc0 = lds_addr(sm.sc[0]);
    i32x8 fa[2][4], fb[2][4];
    int xa[2][4], xb[2][4];

    auto load_step = [&](uint32_t st, int ks, int i) __attribute__((always_inline)) {  // instruction i of step ks (0..7)
        const bool live = ks < nk;
        const uint32_t so = live ? (uint32_t)ks * XBK : 0u;
        if (i < XLPW) lds_load16(live ? ra : rnull, st + ldsrow[i], va[i], so);
        else lds_load16(live ? rb : rnull, st + XOPB + ldsrow[i - XLPW], vb[i - XLPW], so);
    };
    auto load_scales = [&](int grp) __attribute__((always_inline)) {
        const uint32_t dst = sc0 + (uint32_t)(grp & 1) * (2u * SOPB);  // sm.sc[grp & 1]
        lds_load16(ras, dst + 64 * 16 * wid, vas, (uint32_t)grp * 16u);
        lds_load16(rbs, dst + SOPB + 64 * 16 * wid, vbs, (uint32_t)grp * 16u);
    };
    // read number r (0..11) of step ks into set f: fragments a0 b0 b1 b2 b3 a1 a2 a3 (the
    // order the MFMAs consume them), then the scale bytes of sub-tile r-8 of A and of B
    auto read_one = [&](const char* st, int ks, int f, int r) __attribute__((always_inline)) {
        if (r < 8) {
            const bool isa = (r == 0 || r >= 5);
            const int t = r == 0 ? 0 : (r <= 4 ? r - 1 : r - 4);
            const char* base = st + (isa ? 0 : XOPB) + ((isa ? rowa : rowb) + 32 * t) * XBK;
            const u32x4 lo = *reinterpret_cast<const u32x4*>(base + clo);
            const u32x4 hi = *reinterpret_cast<const u32x4*>(base + chi);
            const i32x8 v = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                             (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            if (isa) fa[f][t] = v;
            else fb[f][t] = v;
        } else {
            const char* sc = sm.sc[(ks / SGRP) & 1];
            const int byte = 2 * (ks % SGRP) + gsel;
            const int t = r - 8;
            xa[f][t] = (int)(uint8_t)sc[(rowa + 32 * t) * 16 + byte];
            xb[f][t] = (int)(uint8_t)sc[SOPB + (rowb + 32 * t) * 16 + byte];
        }
    };
    auto mfma_one = [&](int f, int n) __attribute__((always_inline)) {
        const int i = n >> 2, j = n & 3;
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            fb[f][j], fa[f][i], acc[i][j], 0, 0, 0, xb[f][j], 0, xa[f][i]);
    };
    // f: the fragment set step ks reads from (ks & 1, passed as a literal)
    auto kstep = [&](int ks, int f, uint32_t cur32, const char* nxt) __attribute__((always_inline)) {
        wait_vm_lgkm0<2 * XLPS>();  // step ks+1 (and the scale group it needs) landed
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (ks % SGRP == 0 && ks / SGRP + 1 < ngrp) load_scales(ks / SGRP + 1);
        const bool more = ks + 1 < nk;
#pragma unroll
        for (int n = 0; n < 16; ++n) {
            mfma_one(f, n);
            if (n < 8) {
                load_step(cur32, ks + XNST, n);
            } else if (more) {
                read_one(nxt, ks + 1, f ^ 1, n - 8);
                if (n >= 12) read_one(nxt, ks + 1, f ^ 1, n - 4);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if (nk > 0) {
        load_scales(0);
        if (ngrp > 1) load_scales(1);
#pragma unroll
        for (int p = 0; p < XNST; ++p)
#pragma unroll
            for (int i = 0; i < XLPS; ++i) load_step(stg[p], p, i);
        wait_vm_lgkm0<3 * XLPS>();  // scales and step 0 landed
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < 12; ++r) read_one(sm.st[0], 0, 0, r);
        for (int ks = 0; ks < nk; ks += XNST) {
            kstep(ks, 0, sa0, sm.st[1]);
            if (ks + 1 < nk) kstep(ks + 1, 1, sa1, sm.st[2]);
            if (ks + 2 < nk) kstep(ks + 2, 0, sa2, sm.st[3]);
            if (ks + 3 < nk) kstep(ks + 3, 1, sa3, sm.st[0]);
        }
        wait_vm_lgkm0<0>();  // no load may still be writing LDS when the block ends
    }

    // ---------------------------------------------------------------- epilogue
    // B fragment first: lane l holds row l % 32 of its 32x32 block and columns
    // 8 (v/4) + 4 (l/32) + v%4, v = 0..15: four runs of 4 consecutive columns.
    const int lrow = lane & 31, lcol = (lane >> 5) * 4;
    if (EPI == XEPI_SWIGLU_F32) {
        float* C = (float*)g.C + ((int64_t)e * g.c_es + row0) * g.ldc;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = m0 + wm * 128 + i * 32 + lrow;
            if (row >= Mrows) continue;
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int ch = ch0 + wn * 64 + j * 32 + 8 * q + lcol;
                    if (ch >= g.I) continue;
                    f32x4 hv;
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const float gv = acc[i][j][4 * q + c], uv = acc[i][j + 2][4 * q + c];
                        hv[c] = gv / (1.0f + __expf(-gv)) * uv;
                    }
                    *reinterpret_cast<f32x4*>(C + (int64_t)row * g.ldc + ch) = hv;
                }
        }
    } else {
        bf16_t* C = (bf16_t*)g.C + ((int64_t)e * g.c_es + row0) * g.ldc;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = m0 + wm * 128 + i * 32 + lrow;
            if (row >= Mrows) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int col = n0 + wn * 128 + j * 32 + 8 * q + lcol;
                    if (col >= g.N) continue;
                    *reinterpret_cast<uint2*>(C + (int64_t)row * g.ldc + col) =
                        make_uint2(pack_bf2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                                   pack_bf2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]));
                }
        }
    }
}

#define MOE_MX_KERNEL(NAME, EPI)                                                       \
    __global__ __launch_bounds__(XNTH) __attribute__((amdgpu_waves_per_eu(1, 1))) void \
    NAME(MxArgs g) {                                                                   \
        __shared__ MxSmem sm;                                                          \
        const int total = mx_tile_total<EPI>(g, sm);                                   \
        if ((int)blockIdx.x < total) mx_tile<EPI>(g, sm, blockIdx.x);                  \
    }
MOE_MX_KERNEL(mx_gemm1_swiglu, XEPI_SWIGLU_F32)
MOE_MX_KERNEL(mx_gemm2_down, XEPI_STORE_BF16)
#undef MOE_MX_KERNEL

template <int EPI>
static int mx_launch(const MxArgs& g, hipStream_t st) {
    int NT = (EPI == XEPI_SWIGLU_F32) ? cdiv(g.I, 128) : cdiv(g.N, XBN);
    int grid;
    if (g.offsets) {
        int64_t mt = ((int64_t)g.R + (int64_t)g.E * (XBM - 1)) / XBM;
        grid = (int)(mt * NT);
    } else {
        grid = g.total;
    }
    if (grid <= 0) return MOE_OK;
    if (EPI == XEPI_SWIGLU_F32)
        MOE_TRACED("mx_gemm1_swiglu", st, mx_gemm1_swiglu<<<grid, XNTH, 0, st>>>(g));
    else
        MOE_TRACED("mx_gemm2_down", st, mx_gemm2_down<<<grid, XNTH, 0, st>>>(g));
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

}  // namespace moe

using namespace moe;

int moe_launch_mx_quantize_f32(const float* in, int64_t rows, int K, uint8_t* codes, uint8_t* scales,
                               hipStream_t st);

int moe_ffn_mx(const uint8_t* xq, const uint8_t* xs, const int32_t* offsets, int E, int R, int H,
               int I, const uint8_t* w1q, const uint8_t* w1s, const uint8_t* w2q,
               const uint8_t* w2s, float* hf, uint8_t* hq, uint8_t* hs, bf16_t* y, hipStream_t st) {
    // scale groups are 16-byte chunks of each row's K/32 scales: K a multiple of 128 keeps
    // every chunk start 4-byte aligned
    if (H % 128 || I % 128) return MOE_EINVAL;
    const bool shared = offsets == nullptr;
    MxArgs g{};
    g.A = xq; g.As = xs; g.a_es = 0;
    g.B = w1q; g.Bs = w1s; g.b_rows = 2 * I;
    g.C = hf; g.c_es = shared ? R : 0; g.ldc = I;
    g.offsets = offsets; g.E = E; g.R = R; g.N = 2 * I; g.K = H; g.I = I;
    g.total = shared ? E * cdiv(R, XBM) * cdiv(I, 128) : 0;
    int rc = mx_launch<XEPI_SWIGLU_F32>(g, st);
    if (rc) return rc;
    int64_t rows = shared ? (int64_t)E * R : R;
    rc = moe_launch_mx_quantize_f32(hf, rows, I, hq, hs, st);
    if (rc) return rc;
    MxArgs g2{};
    g2.A = hq; g2.As = hs; g2.a_es = shared ? R : 0;
    g2.B = w2q; g2.Bs = w2s; g2.b_rows = H;
    g2.C = y; g2.c_es = shared ? R : 0; g2.ldc = H;
    g2.offsets = offsets; g2.E = E; g2.R = R; g2.N = H; g2.K = I; g2.I = I;
    g2.total = shared ? E * cdiv(R, XBM) * cdiv(H, XBN) : 0;
    return mx_launch<XEPI_STORE_BF16>(g2, st);
}
