// quant_dev.h -- E4M3 scale and encode helpers (quant.hip, prologue.hip).
#pragma once

#include "common.h"

namespace moe {
namespace quant_dev {

__device__ __forceinline__ void scales_from_amax(uint32_t bits, float *scale, float *inv) {
    const float amax = __uint_as_float(bits);
    if (amax == 0.0f) {
        *scale = 1.0f;
        *inv = 1.0f;
    } else {
        *scale = amax / 448.0f;   // IEEE division: the same rounding on every side
        *inv = 448.0f / amax;
    }
}

__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d, float inv) {
    const float lim = 448.0f;
    a = fminf(fmaxf(a * inv, -lim), lim);
    b = fminf(fmaxf(b * inv, -lim), lim);
    c = fminf(fmaxf(c * inv, -lim), lim);
    d = fminf(fmaxf(d * inv, -lim), lim);
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

}  // namespace quant_dev
}  // namespace moe
