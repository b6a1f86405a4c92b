// E4M3 / E8M0 encoding shared by the MX quantisers (rows.hip) and the MX GEMM1 epilogue
// (gemm_mx.hip): OCP Microscaling E4M3 ("FN") codes with one E8M0 scale per 32 values.
#pragma once

#include "common.h"

namespace moe {

// ------------------------------------------------------------------ E4M3 / E8M0
// Round a finite fp32 value to E4M3 ("FN": bias 7, max 448, no infinity), nearest even,
// saturating at +-448.  Pure integer work on the fp32 bit pattern.
__device__ __forceinline__ uint32_t e4m3_rne(float a) {
    uint32_t u = __float_as_uint(a);
    uint32_t s = (u >> 24) & 0x80u;
    u &= 0x7FFFFFFFu;
    if (u >= 0x43E00000u) return s | 0x7Eu;            // |a| >= 448
    int ex = (int)(u >> 23) - 127;
    uint32_t code;
    if (ex < -6) {
        // subnormal range: multiples of 2^-9 (scaling by 2^9 is exact)
        code = (uint32_t)rintf(__uint_as_float(u) * 512.0f);
    } else {
        uint32_t c = ((uint32_t)(ex + 7) << 23) | (u & 0x7FFFFFu);
        c = c + 0x7FFFFu + ((c >> 20) & 1u);
        code = c >> 20;
        if (code > 0x7Eu) code = 0x7Eu;
    }
    return s | code;
}

// Four values to E4M3 codes packed little-endian (first value in the low byte), by the
// hardware conversion v_cvt_pk_fp8_f32 (round to nearest even, OCP E4M3FN) after a clamp to
// +-448: an exhaustive run over every finite fp32 bit pattern on gfx950 gave the same code as
// e4m3_rne above for each one.  Without the clamp the conversion turns values beyond 448 into
// NaN codes instead of saturating.  Two instructions per four values instead of about 25 per
// value: the quantisers become bound by memory rather than by the vector ALU.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
    const auto cl = [](float x) { return fmaxf(-448.0f, fminf(x, 448.0f)); };
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(a), cl(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(c), cl(d), w, true);
    return (uint32_t)w;
}

// E8M0 code of a block maximum: floor(log2 amax) - 8 + 127 (MOE_MX_FLOOR) or the smallest
// exponent keeping amax/2^e <= 448 (MOE_MX_CEIL); clamped to [0,254]; zero block -> 0.
__device__ __forceinline__ int mx_scale_code(float amax, int mode) {
    if (!(amax > 0.0f)) return 0;
    int e = ilogbf(amax) - 8;
    if (mode == MOE_MX_CEIL && ldexpf(amax, -e) > 448.0f) e += 1;
    int code = e + 127;
    return code < 0 ? 0 : (code > 254 ? 254 : code);
}

}  // namespace moe
