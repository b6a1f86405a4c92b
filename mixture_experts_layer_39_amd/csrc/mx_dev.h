// E4M3 / E8M0 encoding shared by the MX quantisers (rows.hip) and the MX GEMM1 epilogue
// (gemm_mx.hip): OCP Microscaling E4M3 ("FN") codes with one E8M0 scale per 32 values.
#pragma once

#include "common.h"

namespace moe {

// Four finite values to E4M3 ("FN": bias 7, max 448, no infinity) codes, rounded to nearest
// even and saturating at +-448, packed little-endian (first value in the low byte).  The
// hardware conversion v_cvt_pk_fp8_f32 rounds to nearest even in OCP E4M3FN; clamping the
// input to +-448 first makes it saturate (without the clamp it turns values beyond 448 into
// NaN codes).  A probe over every finite fp32 bit pattern on gfx950 found this equal to an
// integer encoder written from the format definition, for each one; the GPU tests compare it
// with the CPU oracle on every rounding case.  Two instructions per four values, where the
// integer encoder took about 25 per value and left the quantisers bound by the vector ALU.
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
