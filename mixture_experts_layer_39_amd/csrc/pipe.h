// Pieces shared by the grouped-GEMM kernels (BF16 and MXFP8): scalar buffer descriptors,
// direct global-to-LDS loads, explicit wait counts and the K-major LDS row swizzle.
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
__device__ __forceinline__ void lds_load16(rsrc_t r, uint32_t lds_dst, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(lds_dst), "v"(voff), "s"(r), "s"(soff)
                 : "memory", "m0");
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

// Swizzle of 64-byte K-major LDS rows (four 16-byte chunks): chunk c of row r is stored at
// chunk c ^ kswz(r), which keeps the rows read by one 128-byte (8-lane) or 256-byte
// (16-lane) phase of a 16-byte-per-lane read on distinct banks.
__device__ __forceinline__ int kswz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

__host__ __device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

}  // namespace moe
