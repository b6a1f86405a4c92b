// Pieces shared by the grouped-GEMM kernels (BF16 and MXFP8): scalar buffer descriptors,
// direct global-to-LDS loads, explicit wait counts, and the LDS tile layouts, load maps and
// operand set-up of the pipelined tiles.
#pragma once

#include "common.h"

namespace moe {

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void* lds_ptr;

// Buffer descriptor of a block-uniform range: base and size pass through readfirstlane so that
// the descriptor lives in scalar registers (a descriptor the compiler sees as divergent costs
// a waterfall loop around every load).  Accesses past `bytes` return zeros.
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = (uint32_t)uni((int)(uint32_t)a);
    const uint32_t hi = (uint32_t)uni((int)(uint32_t)(a >> 32));
    void* q = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(q, (short)0, uni((int)bytes), 0x00020000);
}

// Direct load of 16 bytes per lane into LDS at M0 + 16 * lane.  Issued through inline asm:
// the compiler's own wait-count tracking of such loads cannot tell pipeline stages apart and
// would drain every stage in flight before each LDS read; the main loops wait for exactly
// the stage they need instead (wait_vm_lgkm0).  The loads are ordered like any volatile asm.
// The LDS address is an operand bound to M0 ("{m0}"), so the compiler itself sets M0 and
// knows the instruction reads it (M0 is never written behind its back).  The compiler does
// not see into the asm, so it does not insert the wait states a vector memory instruction
// needs after a VALU write of an SGPR it reads (its descriptor or offset: e.g. an SGPR
// reloaded from a spill lane by v_readlane just before) or after an SALU write of M0; the
// asm carries them itself (s_nop 4: five wait states).
__device__ __forceinline__ void lds_load16(rsrc_t r, uint32_t lds_dst, uint32_t voff, uint32_t soff) {
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(voff), "s"(r), "s"(soff), "{m0}"(lds_dst)
                 : "memory");
}

// 32-bit LDS address of a __shared__ object (wave-uniform).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)uni((int)(uint32_t)(uintptr_t)(lds_ptr)p);
}

// s_waitcnt: at most N vector-memory operations outstanding, no LDS operation outstanding.
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
}

__host__ __device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------- LDS tiles (both GEMM files)
// The K step is BK = 32 or 64 (a template parameter of the tile); the stages fill 128 KB of
// LDS, 4 of BK = 32 or 2 of BK = 64.  A 64-wide step makes each K-major tile row 128
// contiguous bytes (a whole L2 line per request, half the requests of 64-byte rows); a 32-wide
// step keeps three steps in flight instead of one, which pays where the rows are long
// already (MN-major operands).  One stage holds one K step of both operands.  Two layouts:
//  K-major   (operand contiguous along K in memory): tile row r (an M or N index) is BK * 2
//            bytes of 16-byte chunks of 8 k values; chunk c is stored at chunk c ^ swz(r),
//            swz = kswz4 (BK = 32) or kswz8 (BK = 64).  The rows read by one 128-byte (8-lane)
//            or 256-byte (16-lane) phase of a fragment read then hit distinct bank groups.
//  MN-major  (operand contiguous along M or N): k-row kr is 512 bytes, 32 chunks of 8 m (n)
//            values; chunk c is stored at chunk c ^ mswz(kr % 4), mswz = {0, 6, 10, 12}, so
//            the k-rows and columns read by one 16-lane (128-byte) or 32-lane (256-byte) phase
//            of a transpose read hit distinct banks.
// Both are filled by direct global-to-LDS loads (buffer_load ... lds): lane L of a wave
// writes 16 bytes at LDS base + 16 L, so each lane fetches the global chunk that belongs at
// its LDS position and the swizzle lives entirely in the global offsets.
constexpr int LDS_STAGES_BYTES = 128 * 1024;

template <int BK_>
struct Pipe {
    static constexpr int BK = BK_;
    static constexpr int KK = BK / 16;              // 32x32x16 MFMA sub-steps per K step
    static constexpr int KROW = BK * 2;             // bytes of one K-major tile row
    static constexpr int OPB = 256 * BK * 2;        // bytes of one operand in one stage
    static constexpr int NST = LDS_STAGES_BYTES / (2 * OPB);  // pipeline stages
    static constexpr int LPW = OPB / 1024 / 4;      // direct loads per operand per wave per step
    static constexpr int LPS = 2 * LPW;             // ... for both operands
    static constexpr int RPI = 1024 / KROW;         // K-major tile rows per load instruction
    static_assert(BK == 32 || BK == 64, "K step");
};

__device__ __forceinline__ int mswz(int kr) { return (0xCA60 >> (4 * (kr & 3))) & 15; }
// K-major row swizzles, chosen so that the rows read by one 128-byte (8-lane) or 256-byte
// (16-lane) phase of a 16-byte-per-lane fragment read hit distinct bank groups: kswz4 for
// rows of four chunks, kswz8 for rows of eight (distinct over any 8 consecutive rows, and
// over the even (odd) rows of any 16 consecutive rows).
__device__ __forceinline__ int kswz4(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }
__device__ __forceinline__ int kswz8(int r) { return (r & 7) ^ ((r >> 3) & 1); }
template <int BK>
__device__ __forceinline__ int kswz_of(int r) { return BK == 64 ? kswz8(r) : kswz4(r); }

// Per-lane description of one operand's global->LDS loads (LPW per wave per K step) and of
// its MFMA fragment reads (up to 4 sub-tiles of 32 rows per wave).  Of NW waves, wave w fills
// the NW-th of the operand's stage area at w OPB/NW, 1 KB per instruction.  The global offset of load i
// is voff[i % 2] + ((i / 2) % 2) ist1 + (i / 4) ist2: the swizzled chunk depends only on the
// parity of i, and the rows of one wave's loads advance by two scalar strides.
struct Operand {
    rsrc_t r;
    uint32_t voff[2];  // byte offset of this lane's 16-byte chunk, even / odd instructions
    uint32_t ist1, ist2;  // byte advances of instructions 2, 3 and 4-7 (see above)
    uint32_t kstep;    // byte advance of the global offset per K step
    // fragment-read offsets: K-major, per sub-step kk (sub-tile t adds 32 t KROW, an
    // immediate); MN-major, per sub-tile t (sub-step kk adds 8192 kk)
    uint32_t rd[4];
};

// K-major operand.  rowmap(nn) gives the global row (relative to the descriptor base) of
// tile row nn.  Each wave loads RW tile rows (64 of a 256-row operand; 32 or 16 of a 128- or
// 64-row one), RPI rows of BK * 2 bytes per instruction: tile rows RW w + RPI i + L / (64 / RPI)
// for instruction i, whose global rows must be those of instruction i % 2 plus
// ((i / 2) % 2) rs1 + (i / 4) rs2.
template <int BK, typename RowMap, int RW = 64>
__device__ __forceinline__ void setup_kmajor(Operand& o, const void* base, uint32_t bytes, int ld,
                                             int wid, int lane, int wsub, RowMap rowmap,
                                             int rs1, int rs2) {
    typedef Pipe<BK> PP;
    constexpr int CPR = PP::KROW / 16;  // 16-byte chunks per row
    o.r = make_rsrc(base, bytes);
#pragma unroll
    for (int par = 0; par < 2; ++par) {
        const int r = RW * wid + PP::RPI * par + lane / CPR;
        const int c = (lane % CPR) ^ kswz_of<BK>(r);
        o.voff[par] = (uint32_t)rowmap(r) * (uint32_t)ld * 2u + (uint32_t)c * 16u;
    }
    o.ist1 = (uint32_t)rs1 * (uint32_t)ld * 2u;
    o.ist2 = (uint32_t)rs2 * (uint32_t)ld * 2u;
    o.kstep = BK * 2;
    // fragment reads: lane reads row wsub + 32 t + lane%32, logical chunk 2 kk + lane/32,
    // stored at chunk (2 kk + lane/32) ^ swz(row); swz does not depend on t
    const int r = wsub + (lane & 31);
    const int x = (lane >> 5) ^ kswz_of<BK>(r);
#pragma unroll
    for (int kk = 0; kk < PP::KK; ++kk)
        o.rd[kk] = (uint32_t)(r * PP::KROW) + ((uint32_t)((2 * kk) ^ x) << 4);
}

// MN-major operand: element (mn, k) at base + k*ld + mn (bytes x2).  Each wave loads
// KPW k-rows of the step (BK/4 with four waves, BK/8 with eight), 2 per instruction.
template <int BK, int KPW = BK / 4>
__device__ __forceinline__ void setup_mnmajor(Operand& o, const void* base, uint32_t bytes, int ld,
                                              int wid, int lane, int wsub) {
    o.r = make_rsrc(base, bytes);
#pragma unroll
    for (int par = 0; par < 2; ++par) {
        const int kr = KPW * wid + 2 * par + (lane >> 5);
        const int c = (lane & 31) ^ mswz(kr);
        o.voff[par] = (uint32_t)kr * (uint32_t)ld * 2u + (uint32_t)c * 16u;
    }
    o.ist1 = 4u * (uint32_t)ld * 2u;
    o.ist2 = 8u * (uint32_t)ld * 2u;
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
    }
}

// Load instruction i of K step ks into the operand's area of a stage (wave w fills the WB
// bytes from w WB: its share of the operand's rows).  Steps past the end of K use an empty
// descriptor: the load still issues (so every step issues the same number of loads and the
// wait counts are constants) but fetches nothing and writes zeros.
template <int BK, int WB = Pipe<BK>::OPB / 4>
__device__ __forceinline__ void issue_load(const Operand& o, uint32_t stage_op, int wid, int i,
                                           rsrc_t r, uint32_t soff) {
    lds_load16(r, stage_op + (uint32_t)(wid * WB + i * 1024), o.voff[i & 1],
               soff + (uint32_t)((i >> 1) & 1) * o.ist1 + (uint32_t)(i >> 2) * o.ist2);
}

// ---------------------------------------------------------------- staged epilogues
// After the K loop each wave owns a 32 MI x 128 output sub-tile in accumulators: MI x 4 blocks
// of 32 x 32, B fragment first, so lane l holds row l % 32 of a block and columns
// 8 (v / 4) + 4 (l / 32) + v % 4, v = 0..15.  Stores go through LDS: the wave writes its
// sub-tile into a private staging area (row-major, rows STG_RS bytes apart: 256 bytes plus a
// 16-byte pad that spreads the 32 rows of one accumulator write over the banks) and reads it
// back as 16-byte chunks of whole rows, 16 lanes per 256-byte row, so that each global store
// instruction writes complete 128-byte lines.
constexpr int STG_RS = 272;
constexpr int STG_BYTES = 128 * STG_RS;  // one wave's staging area

__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// The sub-tile's values (MI blocks of 32 rows) as bf16 rows of the staging area.
template <int MI>
__device__ __forceinline__ void stage_bf16(char* stg, const f32x16 (&acc)[MI][4], int lane) {
    const int lrow = lane & 31, lcol = (lane >> 5) * 4;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<uint2*>(stg + (i * 32 + lrow) * STG_RS + (j * 32 + 8 * q + lcol) * 2) =
                    make_uint2(pack_bf2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                               pack_bf2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]));
}

// Staged rows 0 .. 32 MI - 1 (256 bytes each) to C + r * ldc for r < nrows; the 8-column
// chunk at column c is written when c < ncols.  Non-temporal (NT) stores neither allocate in
// nor evict from the caches: for results that nothing reads again soon (weight gradients).
template <int MI, bool NT = false>
__device__ __forceinline__ void store_staged(const char* stg, bf16_t* C, int64_t ldc, int nrows,
                                             int ncols, int lane) {
    const int rr = lane >> 4, ck = lane & 15;
    const bool colok = ck * 8 < ncols;
#pragma unroll 8
    for (int p = 0; p < 8 * MI; ++p) {
        const int r = 4 * p + rr;
        const u32x4 v = *reinterpret_cast<const u32x4*>(stg + r * STG_RS + ck * 16);
        if (r < nrows && colok) {
            if (NT) st16_nt(C + (int64_t)r * ldc + ck * 8, v);
            else st16(C + (int64_t)r * ldc + ck * 8, v);
        }
    }
}

// The SwiGLU backward of a dgrad sub-tile (acc = dh at 32 MI rows x 128 channels): with the
// saved g at GU + r * ldgu + c (u at + I) it writes dg at C + r * ldc + c and du at + I, for
// rows r < nrows and 8-channel chunks with c < ncols.  In parts of up to 32 PBMAX rows (PBMAX
// blocks of 32): the g and u rows of the part are loaded as whole-row 16-byte chunks into the
// staging area (g rows first, then u rows), each lane turns its own g, u elements into dg, du
// in place (one lane owns each element), and the rows go back out whole.  The staging area
// takes 64 PB rows.
template <int MI, int PBMAX = 2>
__device__ __forceinline__ void dswiglu_staged(char* stg, const f32x16 (&acc)[MI][4],
                                               const bf16_t* GU, int64_t ldgu, bf16_t* C,
                                               int64_t ldc, int I, int nrows, int ncols,
                                               int lane) {
    constexpr int PB = MI < PBMAX ? MI : PBMAX;  // 32-row blocks per part
    constexpr int UR = 32 * PB;                  // first staged row of u
    const int lrow = lane & 31, lcol = (lane >> 5) * 4;
    const int rr = lane >> 4, ck = lane & 15;
    const bool colok = ck * 8 < ncols;
#pragma unroll
    for (int half = 0; half < MI / PB; ++half) {
        const int rb = half * PB * 32;
#pragma unroll 4
        for (int p = 0; p < 8 * PB; ++p) {
            const int r = 4 * p + rr;
            u32x4 gv = {0u, 0u, 0u, 0u}, uv = {0u, 0u, 0u, 0u};
            if (rb + r < nrows && colok) {
                const bf16_t* src = GU + (int64_t)(rb + r) * ldgu + ck * 8;
                gv = ld16(src);
                uv = ld16(src + I);
            }
            *reinterpret_cast<u32x4*>(stg + r * STG_RS + ck * 16) = gv;
            *reinterpret_cast<u32x4*>(stg + (UR + r) * STG_RS + ck * 16) = uv;
        }
        lds_wait();
#pragma unroll
        for (int ih = 0; ih < PB; ++ih) {
            const int i = PB * half + ih;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    char* pg = stg + (ih * 32 + lrow) * STG_RS + (j * 32 + 8 * q + lcol) * 2;
                    char* pu = pg + UR * STG_RS;
                    const uint2 gg = *reinterpret_cast<const uint2*>(pg);
                    const uint2 uu = *reinterpret_cast<const uint2*>(pu);
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
                    *reinterpret_cast<uint2*>(pg) =
                        make_uint2(pack_bf2(dg[0], dg[1]), pack_bf2(dg[2], dg[3]));
                    *reinterpret_cast<uint2*>(pu) =
                        make_uint2(pack_bf2(du[0], du[1]), pack_bf2(du[2], du[3]));
                }
        }
        lds_wait();
#pragma unroll 4
        for (int p = 0; p < 8 * PB; ++p) {
            const int r = 4 * p + rr;
            const u32x4 dgv = *reinterpret_cast<const u32x4*>(stg + r * STG_RS + ck * 16);
            const u32x4 duv = *reinterpret_cast<const u32x4*>(stg + (UR + r) * STG_RS + ck * 16);
            if (rb + r < nrows && colok) {
                bf16_t* dst = C + (int64_t)(rb + r) * ldc + ck * 8;
                st16(dst, dgv);
                st16(dst + I, duv);
            }
        }
        lds_wait();  // the read-back is done before the next half overwrites the rows
    }
}

}  // namespace moe
