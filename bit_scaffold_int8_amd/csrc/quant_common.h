// quant_common.h -- the per-token int8 code of one activation, shared by the
// quantizer kernels and the fused decode kernel so that every path produces the same
// bytes.  Private to the library.
//
// DF-SSM technical summary (gist.science), section 2C: activations enter the int8
// product as per-token absmax codes: s = absmax / 127 (IEEE division), q = rint(x / s)
// with ties to even, clamped to [-127, 127]; an all-zero token has s = 0, q = 0.
#pragma once

#include "device_common.h"

namespace dfssm {

// Code of one element: rint(fl(v / s)) clamped to [-127, 127] (round half to even).
__device__ __forceinline__ int8_t exact_code(float v, float s) {
    float r = rintf(v / s);  // IEEE division (correctly rounded), ties to even
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int8_t)(int)r;
}

// The same code from a multiply: with inv = fl(1 / s) and |v / s| <= 127 (+ rounding),
// |fl(v * inv) - fl(v / s)| is at most 0.5 ulp(v/s) + 127 * 2^-24 + 0.5 ulp(v*inv)
// < 1.6e-5.  The two can only round to different integers if a half-integer lies
// between them, i.e. within 1.6e-5 of fl(v * inv).  Such elements are flagged in
// `near` (margin 2^-15 = 3.05e-5) and must be redone with exact_code; all others
// are bit-identical to the IEEE quotient's code.
__device__ __forceinline__ uint32_t fast_code(float v, float inv, bool& near) {
    const float r = v * inv;
    const float f = r - floorf(r);  // exact: the fraction bits of r
    near = fabsf(f - 0.5f) <= 0x1p-15f;
    const float q = fminf(fmaxf(rintf(r), -127.0f), 127.0f);
    return (uint32_t)(uint8_t)(int8_t)(int)q;
}

// Four codes packed little-endian; bit c of `near4` flags element c.
__device__ __forceinline__ uint32_t fast_code4(float4 v, float inv, uint32_t& near4) {
    bool n0, n1, n2, n3;
    const uint32_t b0 = fast_code(v.x, inv, n0), b1 = fast_code(v.y, inv, n1);
    const uint32_t b2 = fast_code(v.z, inv, n2), b3 = fast_code(v.w, inv, n3);
    near4 = (uint32_t)n0 | ((uint32_t)n1 << 1) | ((uint32_t)n2 << 2) | ((uint32_t)n3 << 3);
    return b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
}

__device__ __forceinline__ uint32_t exact_code4(float4 v, float s) {
    return (uint32_t)(uint8_t)exact_code(v.x, s) | ((uint32_t)(uint8_t)exact_code(v.y, s) << 8) |
           ((uint32_t)(uint8_t)exact_code(v.z, s) << 16) | ((uint32_t)(uint8_t)exact_code(v.w, s) << 24);
}

// Row scale, its reciprocal, and whether the multiply path is usable for the row.
struct RowScale {
    float s, inv;
    bool fast;
};

__device__ __forceinline__ RowScale row_scale(float amax) {
    RowScale r;
    r.s = amax / 127.0f;  // one IEEE division
    r.inv = 1.0f / r.s;
    r.fast = isfinite(r.inv);
    return r;
}

__device__ __forceinline__ float absmax4(float4 v) {
    return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

}  // namespace dfssm
