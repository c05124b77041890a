// quantize.hip -- per-token absmax int8 activation quantizer (gfx950).
//
// DF-SSM technical summary (gist.science), section 2C: the scaffold product is an
// int8 x int8 contraction, so each token's fp32 activations are quantized to int8
// with one fp32 scale:  s = absmax / 127 (IEEE division), q = rint(x / s) with ties
// to even, clamped to [-127, 127]; an all-zero token gets s = 0 and q = 0.
//
// One workgroup per token.  The row is read once with 16-byte loads and held in
// registers (up to kVecPerThread float4 per lane); the absmax is reduced with
// cross-lane shuffles within each wave and through LDS across waves; the codes are
// written as packed char4.  Rows longer than the register budget take a second
// pass over global memory.  This pass is HBM-bound (4 bytes in, 1 byte out per
// element): nothing here is a contraction, so it stays on the vector ALUs.
#include "device_common.h"

namespace dfssm {

constexpr int kQuantThreads = 256;
constexpr int kVecPerThread = 4;  // K <= 4096 stays in registers

__device__ __forceinline__ int8_t quantize_one(float v, float s) {
    float r = rintf(v / s);  // IEEE division (correctly rounded), round half to even
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int8_t)(int)r;
}

__device__ __forceinline__ uint32_t quantize4(float4 v, float s) {
    uint32_t b0 = (uint8_t)quantize_one(v.x, s);
    uint32_t b1 = (uint8_t)quantize_one(v.y, s);
    uint32_t b2 = (uint8_t)quantize_one(v.z, s);
    uint32_t b3 = (uint8_t)quantize_one(v.w, s);
    return b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
}

// Block-wide max over kQuantThreads lanes; every lane gets the result.
__device__ __forceinline__ float block_max(float v, float* red) {
    v = wave_max(v);
    const int wave = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) red[wave] = v;
    __syncthreads();
    float m = red[0];
#pragma unroll
    for (int w = 1; w < kQuantThreads / kWave; ++w) m = fmaxf(m, red[w]);
    return m;
}

// vec4: K % 4 == 0 and x, x_q rows 16-/4-byte aligned.
template <bool kVec4>
__global__ __launch_bounds__(kQuantThreads) void quantize_act_kernel(
    const float* __restrict__ x, int64_t K, int8_t* __restrict__ x_q, float* __restrict__ s_x) {
    __shared__ float red[kQuantThreads / kWave];
    const int64_t m = blockIdx.x;
    const float* row = x + m * K;
    int8_t* qrow = x_q + m * K;
    const int tid = threadIdx.x;

    if constexpr (kVec4) {
        const int64_t K4 = K / 4;
        const float4* row4 = reinterpret_cast<const float4*>(row);
        uint32_t* q4 = reinterpret_cast<uint32_t*>(qrow);
        float4 v[kVecPerThread];
        float amax = 0.0f;
        const bool in_regs = K4 <= (int64_t)kQuantThreads * kVecPerThread;
        if (in_regs) {
#pragma unroll
            for (int i = 0; i < kVecPerThread; ++i) {
                const int64_t idx = tid + (int64_t)i * kQuantThreads;
                v[i] = idx < K4 ? row4[idx] : make_float4(0.f, 0.f, 0.f, 0.f);
                amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)),
                                         fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
            }
        } else {
            for (int64_t idx = tid; idx < K4; idx += kQuantThreads) {
                const float4 t = row4[idx];
                amax = fmaxf(amax, fmaxf(fmaxf(fabsf(t.x), fabsf(t.y)), fmaxf(fabsf(t.z), fabsf(t.w))));
            }
        }
        amax = block_max(amax, red);
        if (amax == 0.0f) {
            for (int64_t idx = tid; idx < K4; idx += kQuantThreads) q4[idx] = 0u;
            if (tid == 0) s_x[m] = 0.0f;
            return;
        }
        const float s = amax / 127.0f;
        if (tid == 0) s_x[m] = s;
        if (in_regs) {
#pragma unroll
            for (int i = 0; i < kVecPerThread; ++i) {
                const int64_t idx = tid + (int64_t)i * kQuantThreads;
                if (idx < K4) q4[idx] = quantize4(v[i], s);
            }
        } else {
            for (int64_t idx = tid; idx < K4; idx += kQuantThreads) q4[idx] = quantize4(row4[idx], s);
        }
    } else {
        float amax = 0.0f;
        for (int64_t k = tid; k < K; k += kQuantThreads) amax = fmaxf(amax, fabsf(row[k]));
        amax = block_max(amax, red);
        if (amax == 0.0f) {
            for (int64_t k = tid; k < K; k += kQuantThreads) qrow[k] = 0;
            if (tid == 0) s_x[m] = 0.0f;
            return;
        }
        const float s = amax / 127.0f;
        if (tid == 0) s_x[m] = s;
        for (int64_t k = tid; k < K; k += kQuantThreads) qrow[k] = quantize_one(row[k], s);
    }
}

hipError_t launch_quantize_act(const float* x, int64_t M, int64_t K, int8_t* x_q, float* s_x,
                               hipStream_t stream) {
    const bool vec4 = (K % 4 == 0) && ((uintptr_t)x % 16 == 0) && ((uintptr_t)x_q % 4 == 0);
    if (vec4) {
        quantize_act_kernel<true><<<dim3((unsigned)M), dim3(kQuantThreads), 0, stream>>>(x, K, x_q, s_x);
    } else {
        quantize_act_kernel<false><<<dim3((unsigned)M), dim3(kQuantThreads), 0, stream>>>(x, K, x_q, s_x);
    }
    return hipGetLastError();
}

}  // namespace dfssm
