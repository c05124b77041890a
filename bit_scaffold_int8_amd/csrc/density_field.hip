// density_field.hip -- the density-field state codec (gfx950).
//
// DF-SSM technical summary (gist.science), section 2D "Density Field State
// Representation": the SSM state is held as a binary field per state element, with
// about 4 d_state cells, through normalization, sigma-delta injection (error feedback),
// binarization and a popcount readout, at chunk boundaries.  Here a state element is
// one row of d_state values (one channel of one head), and:
//   s     = max_n |v_n|                               (the row's scale, fp32)
//   u_n   = (v_n / s + 1) / 2                          (density in [0, 1]; 1/2 if s = 0)
//   cells: a first-order modulator over the row's 4 d_state cells in order, value n
//          owning cells 4 n .. 4 n + 3: w = u_n + e; cell = (w >= 1/2); e = w - cell
//   v'_n  = s (2 popcount(cells of n) / 4 - 1)          (readout: s times -1 .. 1 in halves)
// Storage: 32 cells per uint32 (cell c in bit c % 32 of word c / 32: value n is nibble
// n % 8 of word n / 8), d_state / 8 words and one fp32 scale per row -- 68 bytes for a
// 512-byte row of 128 fp32 values.
//
// The modulator is a chain over a row's cells, so a thread takes a whole row, held in
// registers: a group of 64 threads stages its 64 rows through LDS 32 values at a time
// with coalesced 16-byte loads (chunk stride 33 words, so each thread's copy of its own
// row falls in distinct banks), computes the densities (independent quotients by one
// scale, ahead of the chain), then runs the chain and writes its words.  A small tile keeps several
// groups resident per SIMD, so their chains overlap.  The
// readout is one thread per word (eight popcounts, two 16-byte stores).  Both passes
// are bound by HBM traffic (the state) at the sizes a decode batch holds.
#include "device_common.h"

namespace dfssm {

namespace {

constexpr int kDfRows = 64;       // rows per encode group, one per thread
constexpr int kDfDecThreads = 256;

// Rows of up to 128 values: three waves per SIMD (at most 168 registers, a few values
// spilled outside the chain) hide the chain's dependent steps and hazard waits better
// than two: encode 47.3 -> 46.3 us, round trip 65.0 -> 61.0 us for 262144 rows of 128.
template <int D>
__global__ __launch_bounds__(kDfRows) __attribute__((amdgpu_waves_per_eu(D <= 128 ? 3 : 1, D <= 128 ? 3 : 8))) void density_encode_kernel(const float* __restrict__ state, int64_t R,
                                                                  uint32_t* __restrict__ field,
                                                                  float* __restrict__ scale,
                                                                  float* __restrict__ state_out) {
    constexpr int W = D / 8;                 // field words per row
    constexpr int kChunk = 32;               // values per staged chunk of the group's rows
    constexpr int LD = kChunk + 1;           // LDS row stride of a chunk (words)
    __shared__ float tile[kDfRows * LD];
    const int64_t r0 = (int64_t)blockIdx.x * kDfRows;
    const int rows = (int)(R - r0 < kDfRows ? R - r0 : kDfRows);
    const int tid = threadIdx.x;

    // the thread's row in registers, chunk by chunk: coalesced 16-byte loads of the
    // group's rows into LDS (eight threads per 128-byte piece of a row), then each
    // thread copies its own row's chunk out (stride 33: distinct banks)
    // every load of the group's tile is issued first (their registers then become the
    // row's values chunk by chunk, so the peak stays near one row per thread)
    float4 raw[D / kChunk][kChunk / 4];
#pragma unroll
    for (int q = 0; q < D / kChunk; ++q) {
#pragma unroll
        for (int i = 0; i < kChunk / 4; ++i) {
            const int idx = tid + kDfRows * i;               // float4 piece of the chunk
            const int row = idx / (kChunk / 4), c4 = idx % (kChunk / 4);
            raw[q][i] = row < rows ? *reinterpret_cast<const float4*>(state + (r0 + row) * D + kChunk * q + 4 * c4)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    float v[D];
#pragma unroll
    for (int q = 0; q < D / kChunk; ++q) {
#pragma unroll
        for (int i = 0; i < kChunk / 4; ++i) {
            const int idx = tid + kDfRows * i;
            const int row = idx / (kChunk / 4), c4 = idx % (kChunk / 4);
            float* dst = tile + row * LD + 4 * c4;
            dst[0] = raw[q][i].x;
            dst[1] = raw[q][i].y;
            dst[2] = raw[q][i].z;
            dst[3] = raw[q][i].w;
        }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < kChunk; ++c) v[kChunk * q + c] = tile[tid * LD + c];
        __syncthreads();
    }

    const bool live = tid < rows;
    float s = 0.0f;
#pragma unroll
    for (int n = 0; n < D; ++n) s = fmaxf(s, fabsf(v[n]));
    // densities, in place: independent quotients, ahead of the chain.  Every value of
    // the row is divided by the same s, so the correctly rounded quotient v / s costs
    // one IEEE reciprocal per row and four operations per value (Markstein's
    // correction on operands scaled by a power of two):
    //   k = 1 - exponent(s), s' = s 2^k in [1, 2), v' = v 2^k  (exact scalings),
    //   y = RN(1 / s'), q0 = RN(v' y), r = v' - q0 s' (exact, one FMA), q = RN(q0 + r y).
    // With y within half an ulp of 1/s' and q0 within an ulp of v'/s' = v/s, q is
    // RN(v / s) (Markstein's theorem).  Only where v' falls below the normal range can
    // the scaling round, and there |v / s| < 2^-126, far below what moves (q + 1) / 2.
    // s = 0 (an all-zero row) takes s' = 1 and k = 0 (q = 0); s = inf takes s' = 1 and
    // k = -300, sending finite values to zero (v / inf = 0) and infinite ones to NaN.
    {
        const bool fin = s > 0.0f && s <= 0x1.fffffep127f;
        const int k = fin ? 1 - __builtin_amdgcn_frexp_expf(s) : (s > 0.0f ? -300 : 0);
        const float sp = fin ? __builtin_ldexpf(s, k) : 1.0f;
        const float y = 1.0f / sp;  // IEEE division
#pragma unroll
        for (int n = 0; n < D; ++n) {
            const float vp = __builtin_ldexpf(v[n], k);
            const float q0 = vp * y;
            const float rr = __builtin_fmaf(-q0, sp, vp);
            const float a = __builtin_fmaf(rr, y, q0);
            v[n] = (a + 1.0f) * 0.5f;  // the halving is exact
        }
    }
    // the modulator over the row's cells, 32 cells (8 values) per field word
    const int64_t r = r0 + (live ? tid : 0);
    float e = 0.0f;
    uint32_t words[W];
#pragma unroll
    for (int w = 0; w < W; ++w) {
        uint32_t bits = 0u;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float u = v[8 * w + j];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float wv = u + e;            // inject the carried error
                const bool b = wv >= 0.5f;         // binarize
                e = b ? wv - 1.0f : wv;            // the residual (exact)
                bits |= (uint32_t)b << (4 * j + k);
            }
        }
        words[w] = bits;
    }
    if (live) {
        if (field) {
            uint4* dst = reinterpret_cast<uint4*>(field + r * W);
#pragma unroll
            for (int q = 0; q < W / 4; ++q)
                dst[q] = make_uint4(words[4 * q], words[4 * q + 1], words[4 * q + 2], words[4 * q + 3]);
        }
        if (scale) scale[r] = s;
    }
    if (state_out) {
        // the readout, written back through the same chunked transposition
#pragma unroll
        for (int q = 0; q < D / kChunk; ++q) {
#pragma unroll
            for (int c = 0; c < kChunk; ++c) {
                const int n = kChunk * q + c;
                const int pc = __builtin_popcount((words[n >> 3] >> (4 * (n & 7))) & 0xFu);
                tile[tid * LD + c] = s * ((float)pc * 0.5f - 1.0f);
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < kChunk / 4; ++i) {
                const int idx = tid + kDfRows * i;
                const int row = idx / (kChunk / 4), c4 = idx % (kChunk / 4);
                if (row < rows) {
                    const float* p = tile + row * LD + 4 * c4;
                    *reinterpret_cast<float4*>(state_out + (r0 + row) * D + kChunk * q + 4 * c4) =
                        make_float4(p[0], p[1], p[2], p[3]);
                }
            }
            __syncthreads();
        }
    }
}

// One thread per field word: its eight values.
template <int D>
__global__ __launch_bounds__(kDfDecThreads) void density_decode_kernel(const uint32_t* __restrict__ field,
                                                                        const float* __restrict__ scale, int64_t R,
                                                                        float* __restrict__ state) {
    constexpr int W = D / 8;
    const int64_t i = (int64_t)blockIdx.x * kDfDecThreads + threadIdx.x;
    if (i >= R * W) return;
    const uint32_t w = field[i];
    const float s = scale[i / W];
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int pc = __builtin_popcount((w >> (4 * j)) & 0xFu);
        v[j] = s * ((float)pc * 0.5f - 1.0f);
    }
    float4* dst = reinterpret_cast<float4*>(state + i * 8);
    dst[0] = make_float4(v[0], v[1], v[2], v[3]);
    dst[1] = make_float4(v[4], v[5], v[6], v[7]);
}

template <int D>
hipError_t launch_encode_d(const float* state, int64_t R, uint32_t* field, float* scale, float* state_out,
                           hipStream_t stream) {
    const int64_t groups = (R + kDfRows - 1) / kDfRows;
    if (groups > 0x7fffffffLL) return hipErrorInvalidValue;
    density_encode_kernel<D><<<dim3((unsigned)groups), kDfRows, 0, stream>>>(state, R, field, scale, state_out);
    return hipGetLastError();
}

template <int D>
hipError_t launch_decode_d(const uint32_t* field, const float* scale, int64_t R, float* state, hipStream_t stream) {
    const int64_t groups = (R * (D / 8) + kDfDecThreads - 1) / kDfDecThreads;
    if (groups > 0x7fffffffLL) return hipErrorInvalidValue;
    density_decode_kernel<D><<<dim3((unsigned)groups), kDfDecThreads, 0, stream>>>(field, scale, R, state);
    return hipGetLastError();
}

}  // namespace

bool density_field_supported(int64_t d_state) { return d_state == 64 || d_state == 128 || d_state == 256; }

// encode (state_out == NULL) or the in-place round trip (state_out == state; field and
// scale optional)
hipError_t launch_density_encode(const float* state, int64_t R, int64_t D, uint32_t* field, float* scale,
                                 float* state_out, hipStream_t stream) {
    switch (D) {
        case 64: return launch_encode_d<64>(state, R, field, scale, state_out, stream);
        case 128: return launch_encode_d<128>(state, R, field, scale, state_out, stream);
        case 256: return launch_encode_d<256>(state, R, field, scale, state_out, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_density_decode(const uint32_t* field, const float* scale, int64_t R, int64_t D, float* state,
                                 hipStream_t stream) {
    switch (D) {
        case 64: return launch_decode_d<64>(field, scale, R, state, stream);
        case 128: return launch_decode_d<128>(field, scale, R, state, stream);
        case 256: return launch_decode_d<256>(field, scale, R, state, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace dfssm
