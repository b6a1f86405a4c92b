// MXFP8 grouped GEMMs of the expert FFN forward (E4M3 codes, one E8M0 scale per 32 values
// along K) on gfx950's scaled MFMA, v_mfma_scale_f32_32x32x64_f8f6f4.  The MXFP8 forward is
// the path the pages report the largest gain on (pulsen.vercel.app, "Cursor åpner
// megakernelen…", ¶3; aiexpert.news, "Megakernels are dead and back", ¶4).
//
// Same tiling as the BF16 kernels: 256x256 tiles, 4 waves of 128x128, K steps of 128 codes
// (one 128-byte LDS row per operand row, XOR-swizzled 16-byte chunks), double-buffered LDS,
// buffer loads that zero-fill past an expert's rows, device-side expert tile lists and the
// XCD-aware tile order.  The E8M0 scales of a K step (4 per row) travel as one dword per
// row through LDS; each lane hands the MFMA the scale of its row in the 32-code block that
// its lane group stands for.
//   GEMM1: [g|u] = Xq_e W1q_e^T, epilogue h = silu(g)*u in fp32.
//   GEMM2: y = hq_e W2q_e^T, bf16 output (h MX-quantised along I in between).
#include "common.h"

namespace moe {

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Buffer descriptor of a block-uniform range, kept in scalar registers (see make_rsrc).
__device__ __forceinline__ rsrc_t mx_rsrc(const void* p, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = (uint32_t)uni((int)(uint32_t)a);
    const uint32_t hi = (uint32_t)uni((int)(uint32_t)(a >> 32));
    void* q = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(q, (short)0, uni((int)bytes), 0x00020000);
}
__device__ __forceinline__ u32x4 mx_bload16(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ uint32_t mx_bload4(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}

constexpr int XBM = 256, XBN = 256, XBK = 128, XNTH = 256, XGM = 4;

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

__device__ __forceinline__ int xswz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ uint32_t xlds(int row, int chunk) {
    return (uint32_t)(row * 128 + ((chunk ^ xswz(row)) << 4));
}
__host__ __device__ __forceinline__ int xcdiv(int a, int b) { return (a + b - 1) / b; }

template <int EPI>
__device__ __forceinline__ void mx_gemm_body(const MxArgs& g) {
    __shared__ __attribute__((aligned(16))) char smem[4 * 256 * 128];
    __shared__ uint32_t s_sc[2][2][256];
    __shared__ int s_tp[1024];
    __shared__ int s_total;

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid >> 1, wn = wid & 1;
    const int NT = (EPI == XEPI_SWIGLU_F32) ? xcdiv(g.I, 128) : xcdiv(g.N, XBN);
    const int KB = g.K / 32;

    int total;
    if (g.offsets) {
        if (wid == 0) {
            int run = 0;
            for (int base = 0; base < g.E; base += 64) {
                int e = base + lane, tiles = 0;
                if (e < g.E) {
                    int lo = min(max(g.offsets[e], 0), g.R);
                    int hi = min(max(g.offsets[e + 1], lo), g.R);
                    tiles = xcdiv(hi - lo, XBM) * NT;
                }
                int inc = wave_incl_scan(tiles) + run;
                if (e < g.E) s_tp[e] = inc;
                run = __shfl(inc, 63, 64);
            }
            if (lane == 0) s_total = run;
        }
        __syncthreads();
        total = uni(s_total);
    } else {
        total = g.total;
    }
    const int bid = blockIdx.x;
    if (bid >= total) return;
    int logical;
    {
        int q = total >> 3, r = total & 7, x = bid & 7;
        logical = x * q + min(x, r) + (bid >> 3);
    }
    int e, t_local, Mrows, row0;
    if (g.offsets) {
        int lo = 0, hi = g.E - 1;
        while (lo < hi) {
            int mid = (lo + hi) >> 1;
            if (s_tp[mid] > logical) hi = mid; else lo = mid + 1;
        }
        e = uni(lo);
        t_local = uni(logical - (e ? s_tp[e - 1] : 0));
        int a = min(max(g.offsets[e], 0), g.R);
        int b = min(max(g.offsets[e + 1], a), g.R);
        row0 = uni(a);
        Mrows = uni(b - a);
    } else {
        int per = xcdiv(g.R, XBM) * NT;
        e = logical / per;
        t_local = logical - e * per;
        row0 = 0;
        Mrows = g.R;
    }
    const int MT = xcdiv(Mrows, XBM);
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

    // operands (codes are bytes: one row of a K step is 128 bytes = 8 chunks of 16)
    const int64_t arow = (int64_t)e * g.a_es + row0 + m0;
    const uint32_t arows = (uint32_t)max(Mrows - m0, 0);
    rsrc_t ra = mx_rsrc(g.A + arow * g.K, arows * (uint32_t)g.K);
    rsrc_t ras = mx_rsrc(g.As + arow * KB, arows * (uint32_t)KB);
    rsrc_t rb = mx_rsrc(g.B + (int64_t)e * g.b_rows * g.K, (uint32_t)g.b_rows * (uint32_t)g.K);
    rsrc_t rbs = mx_rsrc(g.Bs + (int64_t)e * g.b_rows * KB, (uint32_t)g.b_rows * (uint32_t)KB);
    uint32_t va[8], vb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        int rr = (tid >> 3) + 32 * i;
        va[i] = (uint32_t)rr * (uint32_t)g.K + (uint32_t)(tid & 7) * 16u;
        int brow;
        if (EPI == XEPI_SWIGLU_F32) {
            int q = rr & 127;
            brow = (q >> 6) * g.I + ch0 + (rr >> 7) * 64 + (q & 63);
        } else {
            brow = n0 + rr;
        }
        vb[i] = (uint32_t)brow * (uint32_t)g.K + (uint32_t)(tid & 7) * 16u;
    }
    // scale dword of row `tid` (4 blocks of one K step)
    const uint32_t vas = (uint32_t)tid * (uint32_t)KB;
    uint32_t vbs;
    {
        int brow;
        if (EPI == XEPI_SWIGLU_F32) {
            int q = tid & 127;
            brow = (q >> 6) * g.I + ch0 + (tid >> 7) * 64 + (q & 63);
        } else {
            brow = n0 + tid;
        }
        vbs = (uint32_t)brow * (uint32_t)KB;
    }

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    u32x4 ar[8], br[8];
    uint32_t asr, bsr;
    auto gload = [&](int ks) {
        const uint32_t o = (uint32_t)ks * XBK;
#pragma unroll
        for (int i = 0; i < 8; ++i) ar[i] = mx_bload16(ra, va[i] + o);
#pragma unroll
        for (int i = 0; i < 8; ++i) br[i] = mx_bload16(rb, vb[i] + o);
        asr = mx_bload4(ras, vas + (uint32_t)ks * 4u);
        bsr = mx_bload4(rbs, vbs + (uint32_t)ks * 4u);
    };
    auto lstore = [&](int buf) {
        char* sA = smem + (2 * buf) * 256 * 128;
        char* sB = smem + (2 * buf + 1) * 256 * 128;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            st16(sA + xlds((tid >> 3) + 32 * i, tid & 7), ar[i]);
            st16(sB + xlds((tid >> 3) + 32 * i, tid & 7), br[i]);
        }
        s_sc[buf][0][tid] = asr;
        s_sc[buf][1][tid] = bsr;
    };

    const int nk = g.K / XBK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int ks = 0; ks < nk; ++ks) {
        const int buf = ks & 1;
        if (ks + 1 < nk) gload(ks + 1);
        const char* sA = smem + (2 * buf) * 256 * 128;
        const char* sB = smem + (2 * buf + 1) * 256 * 128;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            // Operand layout of the 32x32x64 scaled MFMA: lane group g = lane/32 holds codes
            // [16g, 16g+16) of each of the instruction's two 32-code blocks (first block in
            // bytes 0-15, second in bytes 16-31), and the scale of lane l is that of row l%32
            // in block g.  In LDS a K step row is 8 chunks of 16 codes: chunks 4kk+g and
            // 4kk+g+2 for this lane; its scale byte is block kb = 2kk+g of the step.
            const int kb = kk * 2 + (lane >> 5);
            const int c0 = kk * 4 + (lane >> 5);
            i32x8 af[4], bfr[4];
            int asc[4], bsc[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                int row = wm * 128 + i * 32 + (lane & 31);
                u32x4 lo = *reinterpret_cast<const u32x4*>(sA + xlds(row, c0));
                u32x4 hi = *reinterpret_cast<const u32x4*>(sA + xlds(row, c0 + 2));
                af[i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                              (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                asc[i] = (int)((s_sc[buf][0][row] >> (8 * kb)) & 0xFFu);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                int row = wn * 128 + j * 32 + (lane & 31);
                u32x4 lo = *reinterpret_cast<const u32x4*>(sB + xlds(row, c0));
                u32x4 hi = *reinterpret_cast<const u32x4*>(sB + xlds(row, c0 + 2));
                bfr[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                               (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                bsc[j] = (int)((s_sc[buf][1][row] >> (8 * kb)) & 0xFFu);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        af[i], bfr[j], acc[i][j], 0, 0, 0, asc[i], 0, bsc[j]);
        }
        if (ks + 1 < nk) lstore(buf ^ 1);
        __syncthreads();
    }

    const int lc = lane & 31, lr = (lane >> 5) * 4;
    if (EPI == XEPI_SWIGLU_F32) {
        float* C = (float*)g.C + ((int64_t)e * g.c_es + row0) * g.ldc;
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
                    if (cok && row < Mrows) C[(int64_t)row * g.ldc + ch] = hv;
                }
            }
    } else {
        bf16_t* C = (bf16_t*)g.C + ((int64_t)e * g.c_es + row0) * g.ldc;
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
                    if (cok && row < Mrows) C[(int64_t)row * g.ldc + col] = f2bf(val);
                }
            }
    }
}

__global__ __launch_bounds__(XNTH) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mx_gemm1_swiglu(MxArgs g) { mx_gemm_body<XEPI_SWIGLU_F32>(g); }
__global__ __launch_bounds__(XNTH) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mx_gemm2_down(MxArgs g) { mx_gemm_body<XEPI_STORE_BF16>(g); }

template <int EPI>
static int mx_launch(const MxArgs& g, hipStream_t st) {
    int NT = (EPI == XEPI_SWIGLU_F32) ? xcdiv(g.I, 128) : xcdiv(g.N, XBN);
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
    if (H % XBK || I % XBK) return MOE_EINVAL;
    const bool shared = offsets == nullptr;
    MxArgs g{};
    g.A = xq; g.As = xs; g.a_es = 0;
    g.B = w1q; g.Bs = w1s; g.b_rows = 2 * I;
    g.C = hf; g.c_es = shared ? R : 0; g.ldc = I;
    g.offsets = offsets; g.E = E; g.R = R; g.N = 2 * I; g.K = H; g.I = I;
    g.total = shared ? E * xcdiv(R, XBM) * xcdiv(I, 128) : 0;
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
    g2.total = shared ? E * xcdiv(R, XBM) * xcdiv(H, XBN) : 0;
    return mx_launch<XEPI_STORE_BF16>(g2, st);
}
