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
// limit read as zero.  kFast: the caller guarantees base+off is 16-byte aligned and
// limit a multiple of 16, so a chunk is either wholly inside or wholly outside and a
// single masked vector load suffices.  Otherwise bytes are gathered one by one.
template <bool kFast>
__device__ __forceinline__ uint4 load16_guarded(const uint8_t* base, int64_t off, int64_t limit) {
    if constexpr (kFast) {
        return off < limit ? *reinterpret_cast<const uint4*>(base + off) : make_uint4(0u, 0u, 0u, 0u);
    } else {
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        for (int b = 0; b < 16; ++b) {
            if (off + b < limit) w[b >> 2] |= uint32_t(base[off + b]) << (8 * (b & 3));
        }
        return make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// 4-byte load of bytes [off, off+4) with the same rule (kFast: 4-byte aligned, limit
// a multiple of 4).
template <bool kFast>
__device__ __forceinline__ uint32_t load4_guarded(const uint8_t* base, int64_t off, int64_t limit) {
    if constexpr (kFast) {
        return off < limit ? *reinterpret_cast<const uint32_t*>(base + off) : 0u;
    } else {
        uint32_t w = 0u;
        for (int b = 0; b < 4; ++b) {
            if (off + b < limit) w |= uint32_t(base[off + b]) << (8 * b);
        }
        return w;
    }
}

// 16-byte load that never branches: `base` must point at 16 readable bytes; the
// value is returned when `live`, zero otherwise (dead lanes read base itself).
// The zeroing is an AND with a mask the optimizer cannot see through (an empty asm
// statement with a register operand emits no instruction); a plain select lets it
// sink the load into a branch, which costs a wait per load.
__device__ __forceinline__ uint32_t opaque_mask(bool live) {
    uint32_t m = live ? 0xFFFFFFFFu : 0u;
    asm volatile("" : "+v"(m));
    return m;
}

__device__ __forceinline__ uint4 load16_select(const uint8_t* base, int64_t off, bool live) {
    const uint4 v = *reinterpret_cast<const uint4*>(base + (live ? off : 0));
    const uint32_t m = opaque_mask(live);
    return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
}

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also orders
// global memory, which makes every wave wait for all of its outstanding global
// loads (s_waitcnt vmcnt(0)) and so drains a software prefetch pipeline; this one
// lets prefetched loads stay in flight across the barrier.  Only for barriers that
// publish LDS data, never for global-memory hand-offs between threads.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Raw buffer resource over [base, base + bytes).  A buffer access past `bytes` is
// dropped (store) or reads zero (load) by the hardware range check, so an offset of
// kOffDead predicates a store without a branch -- and without the control flow that
// makes the compiler wait for every outstanding load at the join.  Word 3 is the
// gfx9-family raw-buffer default.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
constexpr int kOffDead = 0x7fffffff;

__device__ __forceinline__ void store_f32(float v, __amdgpu_buffer_rsrc_t r, int byte_off) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, byte_off, 0, 0);
}

__device__ __forceinline__ void store_i32(int32_t v, __amdgpu_buffer_rsrc_t r, int byte_off) {
    __builtin_amdgcn_raw_buffer_store_b32((uint32_t)v, r, byte_off, 0, 0);
}

// Device-scope stores (cache-policy bit SC1 of the buffer instruction's aux operand on
// gfx950).  Such a store is written through the XCD's L2 rather than left dirty in it,
// so a large output that every workgroup writes at the end of its tile drains while
// the stores are issued, instead of in a write-back of the L2s when the kernel ends.
// Measured on the prefill projections (64 MB and 16 MB of fp32 output) only; the
// Mamba-2 state update, which rewrites what it reads, runs slower with it.
constexpr int kAuxDeviceScope = 16;
__device__ __forceinline__ void store_f32_dev(float v, __amdgpu_buffer_rsrc_t r, int byte_off) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, byte_off, 0, kAuxDeviceScope);
}
__device__ __forceinline__ void store_i32_dev(int32_t v, __amdgpu_buffer_rsrc_t r, int byte_off) {
    __builtin_amdgcn_raw_buffer_store_b32((uint32_t)v, r, byte_off, 0, kAuxDeviceScope);
}

// A shift amount of 1 the optimizer cannot see (an empty asm statement with a scalar
// register operand emits no instruction).  With a constant shift, InstCombine
// re-associates a Horner chain (((a << 1) + b) << 1) + c into separate shifts and
// adds; with this one every step stays a single v_lshl_add_u32.  No instruction is
// written by hand, so the compiler still inserts the MFMA-to-VALU wait states.
__device__ __forceinline__ int32_t opaque_one() {
    int32_t one = 1;
    asm volatile("" : "+s"(one));
    return one;
}

// ---- cross-lane steps on the DPP paths: each reads another lane's register inside a
// VALU instruction (a shuffle through ds_bpermute is an LDS round trip, ~100 cycles).
// Every lane of the wave must be active.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppRowRor8 = 0x128;    // row_ror:8 (lane i <- lane i ^ 8 within a row of 16)
constexpr int kDppMirror = 0x140;     // row_mirror (lane i <- lane 15 - i)
constexpr int kDppHalfMirror = 0x141; // row_half_mirror (lane i <- lane 7 - i within 8)
constexpr int kDppBcast15 = 0x142;    // row_bcast:15 (rows 1, 3 <- lane 15 of the row before)
constexpr int kDppBcast31 = 0x143;    // row_bcast:31 (rows 2, 3 <- lane 31)

// Another lane's value; rows outside kRowMask get `identity`.
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ int dpp_i(int v, int identity = 0) {
    return __builtin_amdgcn_update_dpp(identity, v, kCtrl, kRowMask, 0xF, false);
}
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ float dpp_f(float v, float identity = 0.0f) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(__float_as_int(identity), __float_as_int(v), kCtrl, kRowMask, 0xF, false));
}

// The wave's maximum, in every lane (exact: any order gives the same value).
__device__ __forceinline__ float wave_max(float v) {
    const float lo = -__builtin_inff();
    v = fmaxf(v, dpp_f<kDppXor1>(v));
    v = fmaxf(v, dpp_f<kDppXor2>(v));
    v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
    v = fmaxf(v, dpp_f<kDppMirror>(v));
    v = fmaxf(v, dpp_f<kDppBcast15, 0xA>(v, lo));
    v = fmaxf(v, dpp_f<kDppBcast31, 0xC>(v, lo));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// The wave's integer sum, in every lane.
__device__ __forceinline__ int32_t wave_sum(int32_t v) {
    v += dpp_i<kDppXor1>(v);
    v += dpp_i<kDppXor2>(v);
    v += dpp_i<kDppHalfMirror>(v);
    v += dpp_i<kDppMirror>(v);
    v += dpp_i<kDppBcast15, 0xA>(v);
    v += dpp_i<kDppBcast31, 0xC>(v);
    return __builtin_amdgcn_readlane(v, 63);
}

}  // namespace dfssm
