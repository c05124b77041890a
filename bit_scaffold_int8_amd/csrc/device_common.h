// device_common.h -- small gfx950 device helpers shared by the projection kernels.
// Private to the library (not installed, not included by the public header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dfssm {

typedef int32_t v4i __attribute__((ext_vector_type(4)));
typedef int32_t v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;
constexpr int kRank = 16;

// v_perm_b32: byte i of the result is byte sel.byte[i] of the 64-bit value {hi, lo}
// (selector 0..3 pick lo's bytes, 4..7 pick hi's bytes).
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// 4x4 byte transpose: out[j] = (s0.byte j, s1.byte j, s2.byte j, s3.byte j).
__device__ __forceinline__ void transpose4x4(uint32_t s0, uint32_t s1, uint32_t s2, uint32_t s3,
                                             uint32_t& o0, uint32_t& o1, uint32_t& o2, uint32_t& o3) {
    const uint32_t a_lo = perm(s1, s0, 0x05010400u);  // s0.0 s1.0 s0.1 s1.1
    const uint32_t a_hi = perm(s1, s0, 0x07030602u);  // s0.2 s1.2 s0.3 s1.3
    const uint32_t b_lo = perm(s3, s2, 0x05010400u);  // s2.0 s3.0 s2.1 s3.1
    const uint32_t b_hi = perm(s3, s2, 0x07030602u);  // s2.2 s3.2 s2.3 s3.3
    o0 = perm(b_lo, a_lo, 0x05040100u);
    o1 = perm(b_lo, a_lo, 0x07060302u);
    o2 = perm(b_hi, a_hi, 0x05040100u);
    o3 = perm(b_hi, a_hi, 0x07060302u);
}

// Sum of the four signed bytes of a word (v_dot4 against all-ones).
__device__ __forceinline__ int32_t byte_sum(uint32_t w, int32_t acc) {
    return __builtin_amdgcn_sdot4((int)w, 0x01010101, acc, false);
}

// 16-byte load of bytes [off, off+16) of a buffer of `limit` bytes; bytes past the
// limit read as zero.  `fast` promises 16-byte alignment of base+off whenever the
// whole chunk is in range.
__device__ __forceinline__ uint4 load16_guarded(const uint8_t* base, int64_t off, int64_t limit,
                                                bool fast) {
    if (off + 16 <= limit && fast) {
        return *reinterpret_cast<const uint4*>(base + off);
    }
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    for (int b = 0; b < 16; ++b) {
        if (off + b < limit) w[b >> 2] |= uint32_t(base[off + b]) << (8 * (b & 3));
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// 4-byte load of bytes [off, off+4) with the same zero-fill rule.
__device__ __forceinline__ uint32_t load4_guarded(const uint8_t* base, int64_t off, int64_t limit,
                                                  bool fast) {
    if (off + 4 <= limit && fast) {
        return *reinterpret_cast<const uint32_t*>(base + off);
    }
    uint32_t w = 0u;
    for (int b = 0; b < 4; ++b) {
        if (off + b < limit) w |= uint32_t(base[off + b]) << (8 * b);
    }
    return w;
}

__device__ __forceinline__ float wave_max(float v) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

__device__ __forceinline__ int32_t wave_sum(int32_t v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

}  // namespace dfssm
