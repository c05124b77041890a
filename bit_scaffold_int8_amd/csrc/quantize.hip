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
#include "quant_common.h"

namespace dfssm {

constexpr int kQuantThreads = 256;
constexpr int kVecPerThread = 4;  // K <= 4096 stays in registers

// Block-wide max over kQuantThreads lanes; every lane gets the result.
__device__ __forceinline__ float block_max(float v, float* red) {
    v = wave_max(v);
    const int wave = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) red[wave] = v;
    lds_barrier();
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
        const RowScale rs = row_scale(amax);
        if (tid == 0) s_x[m] = rs.s;
        if (in_regs) {
            uint32_t near = 0;  // bit 4i+c: element c of float4 i needs the exact quotient
#pragma unroll
            for (int i = 0; i < kVecPerThread; ++i) {
                const int64_t idx = tid + (int64_t)i * kQuantThreads;
                if (idx < K4) {
                    uint32_t n4;
                    q4[idx] = fast_code4(v[i], rs.inv, n4);
                    near |= (rs.fast ? n4 : 0xFu) << (4 * i);
                }
            }
            while (near) {  // rare: redo flagged elements exactly (same thread, same bytes)
                const int bit = __builtin_ctz(near);
                near &= near - 1;
                const int64_t k = 4 * (tid + (int64_t)(bit >> 2) * kQuantThreads) + (bit & 3);
                qrow[k] = exact_code(row[k], rs.s);
            }
        } else {
            for (int64_t idx = tid; idx < K4; idx += kQuantThreads) {
                const float4 xv = row4[idx];
                uint32_t n4;
                uint32_t q = fast_code4(xv, rs.inv, n4);
                if (!rs.fast || n4) q = exact_code4(xv, rs.s);
                q4[idx] = q;
            }
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
        for (int64_t k = tid; k < K; k += kQuantThreads) qrow[k] = exact_code(row[k], s);
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

// ---------------------------------------------------------------------------------
// Fused quantizer + LoRA down-projection: one kernel writes x_q, s_x and
// t[m][r] = sum_k W_B[r][k] x_q[m][k] (technical summary section 2B: the int8 rank-16
// correction acts on the same int8 activations).  Each workgroup takes up to 16
// tokens; each wave quantizes whole token rows on its own (wave-level absmax, no
// block barrier per token, all of a row's loads in flight at once) and also keeps
// the codes in LDS; then the 16-token x 16-rank tile of t is one
// v_mfma_i32_16x16x64_i8 accumulator per wave over a K slice, summed through LDS.
// Requires K % 4 == 0 (16-byte aligned fp32 rows); a group takes as many tokens
// (at most 16) as fit 63 KiB of LDS, so rows up to 64512 elements.
namespace dfssm {

constexpr int kQLWaves = 8;
constexpr int kQLThreads = kQLWaves * kWave;
constexpr int64_t kQLLdsBytes = 65536 - 1024;  // codes; the rest of 64 KiB holds the t tile
// Template parameters: NV float4 of a row per lane kept in registers (a row longer than
// the waves sharing it hold is read twice), NP W_B fragments per wave fetched ahead.
// The launch picks the smallest that cover the row, so short rows leave registers for
// more resident groups.

// kRows16: K % 16 == 0, so a 16-byte W_B chunk lies wholly inside its row or wholly
// past it, and every global load of the kernel is a branch-free buffer load.
template <int kQLRegVec, int kQLPre, bool kRows16>
__global__ __launch_bounds__(kQLThreads) void quantize_lora_down_kernel(
    const float* __restrict__ x, int64_t M, int64_t K, const int8_t* __restrict__ w_b, int rank,
    int8_t* __restrict__ x_q, float* __restrict__ s_x, int32_t* __restrict__ t, int tokens_per_group) {
    extern __shared__ __align__(16) uint8_t lds_q[];  // [tokens_per_group][K] codes
    __shared__ int32_t tsum[16][16];                   // t tile [token][rank], summed over waves
    __shared__ float amax_part[kQLWaves];

    const int64_t p = blockIdx.y;  // problem of a dense batch
    x += p * M * K;
    x_q += p * M * K;
    s_x += p * M;
    if (rank != 0) {
        w_b += p * kRank * K;
        t += p * M * kRank;
    }

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));  // uniform
    const int64_t m0 = (int64_t)blockIdx.x * tokens_per_group;
    const int rows = (int)((M - m0) < tokens_per_group ? (M - m0) : tokens_per_group);
    const int64_t K4 = K / 4;
    if (threadIdx.x < 256) tsum[threadIdx.x >> 4][threadIdx.x & 15] = 0;
    // loads past a buffer's range read zero; a dead offset lies past every range
    constexpr int kLoadDead = 0x7ff00000;

    // W_B does not depend on x: its first fragments are fetched right after the row
    // loads, so the absmax waits for the row only and the W_B stream overlaps the
    // quantization
    const int i = lane & 15, g = lane >> 4;
    const uint8_t* brow = reinterpret_cast<const uint8_t*>(w_b) + (int64_t)i * K;
    const int64_t steps = (K + 63) / 64;
    const bool rows16 = (K % 16) == 0;  // 16-byte aligned rows in LDS and in W_B
    // the problem's W_B (rank 0: an empty range, so every load reads zero)
    const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc(w_b, rank != 0 ? (uint32_t)(kRank * K) : 0u);
    auto load_b = [&](int64_t st) -> uint4 {
        const int64_t off = st * 64 + 16 * g;
        if constexpr (kRows16) {
            const int o = off < K ? (int)(i * K + off) : kLoadDead;
            const v4i v = __builtin_amdgcn_raw_buffer_load_b128(b_rsrc, o, 0, 0);
            return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
        } else {
            if (rank == 0 || st >= steps || off >= K) return make_uint4(0u, 0u, 0u, 0u);
            uint32_t bw[4] = {0u, 0u, 0u, 0u};
            for (int e = 0; e < 4; ++e)
                if (off + 4 * e < K) bw[e] = *reinterpret_cast<const uint32_t*>(brow + off + 4 * e);
            return make_uint4(bw[0], bw[1], bw[2], bw[3]);
        }
    };
    uint4 bpre[kQLPre];
    auto prefetch_b = [&]() {
#pragma unroll
        for (int u = 0; u < kQLPre; ++u) bpre[u] = load_b(wave + (int64_t)u * kQLWaves);
    };

    // ---- phase 1: quantize the group's rows.  Few rows (decode): several waves
    // share a row and combine their absmax through LDS; many rows: a wave per row.
    const int wpr = rows >= 8 ? 1 : (rows >= 4 ? 2 : (rows >= 2 ? 4 : 8));  // waves per row
    const int rpp = kQLWaves / wpr;                                           // rows per pass
    const int sub = wave % wpr;
    const int64_t lstride = (int64_t)wpr * kWave;  // float4 stride of one lane within its row
    const bool in_regs = K4 <= lstride * kQLRegVec;
    for (int r0 = 0; r0 < rows; r0 += rpp) {
        const int r = r0 + wave / wpr;
        const bool live = r < rows;
        const int64_t m = m0 + (live ? r : 0);
        const float4* row4 = reinterpret_cast<const float4*>(x + m * K);
        uint32_t* q4 = reinterpret_cast<uint32_t*>(x_q + m * K);
        uint32_t* l4 = reinterpret_cast<uint32_t*>(lds_q + (int64_t)(live ? r : 0) * K);
        const int64_t lbase = (int64_t)sub * kWave + lane;
        float4 v[kQLRegVec];
        float amax = 0.0f;
        if (in_regs) {
            // the row through a buffer resource (a dead row has an empty range): no
            // branch around the loads, so the absmax below waits for them alone
            const __amdgpu_buffer_rsrc_t x_rsrc = make_rsrc(x + m * K, live ? (uint32_t)(K * 4) : 0u);
#pragma unroll
            for (int e = 0; e < kQLRegVec; ++e) {
                const v4f t4 = __builtin_bit_cast(
                    v4f, __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, (int)((lbase + (int64_t)e * lstride) * 16), 0, 0));
                v[e] = make_float4(t4[0], t4[1], t4[2], t4[3]);
            }
        } else if (live) {
            for (int64_t idx = lbase; idx < K4; idx += lstride) amax = fmaxf(amax, absmax4(row4[idx]));
        }
        // (re-issued on every pass: identical values, L2 hits after the first, and a
        // load on every path keeps the wait below partial)
        prefetch_b();
        if (in_regs) {
#pragma unroll
            for (int e = 0; e < kQLRegVec; ++e) amax = fmaxf(amax, absmax4(v[e]));
        }
        amax = wave_max(amax);
        if (lane == 0) amax_part[wave] = amax;
        lds_barrier();
        const int w0 = (wave / wpr) * wpr;
        for (int w = 0; w < wpr; ++w) amax = fmaxf(amax, amax_part[w0 + w]);
        lds_barrier();  // amax_part is rewritten by the next pass
        if (live) {
            const RowScale rs = row_scale(amax);
            if (lane == 0 && sub == 0) s_x[m] = amax == 0.0f ? 0.0f : rs.s;
            if (in_regs) {
#pragma unroll
                for (int e = 0; e < kQLRegVec; ++e) {
                    const int64_t idx = lbase + (int64_t)e * lstride;
                    if (idx < K4) {
                        uint32_t n4 = 0;
                        uint32_t q = amax == 0.0f ? 0u : fast_code4(v[e], rs.inv, n4);
                        // rare: a code within reach of a rounding tie is redone with the
                        // IEEE quotient, from the values still in registers
                        if (amax != 0.0f && (!rs.fast || n4)) q = exact_code4(v[e], rs.s);
                        q4[idx] = q;
                        l4[idx] = q;
                    }
                }
            } else {
                for (int64_t idx = lbase; idx < K4; idx += lstride) {
                    const float4 xv = row4[idx];
                    uint32_t n4 = 0;
                    uint32_t q = amax == 0.0f ? 0u : fast_code4(xv, rs.inv, n4);
                    if (amax != 0.0f && (!rs.fast || n4)) q = exact_code4(xv, rs.s);
                    q4[idx] = q;
                    l4[idx] = q;
                }
            }
        }
    }
    if (rank == 0) return;
    lds_barrier();

    // ---- phase 2: t tile = codes (16 tokens, LDS) x W_B^T (16 ranks, global)
    const uint8_t* arow = lds_q + (int64_t)i * K;
    const bool arow_live = i < rows;
    auto load_a = [&](int64_t st) -> uint4 {
        const int64_t off = st * 64 + 16 * g;
        if (!arow_live || st >= steps || off >= K) return make_uint4(0u, 0u, 0u, 0u);
        if (rows16 && off + 16 <= K) return *reinterpret_cast<const uint4*>(arow + off);
        uint32_t aw[4] = {0u, 0u, 0u, 0u};
        for (int e = 0; e < 4; ++e)
            if (off + 4 * e < K) aw[e] = *reinterpret_cast<const uint32_t*>(arow + off + 4 * e);
        return make_uint4(aw[0], aw[1], aw[2], aw[3]);
    };
    auto mfma = [](uint4 a, uint4 b, v4i acc) {
        const v4i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w};
        const v4i bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w};
        return __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv, acc, 0, 0, 0);
    };
    v4i acc = {0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < kQLPre; ++u) acc = mfma(load_a(wave + (int64_t)u * kQLWaves), bpre[u], acc);
    for (int64_t st = wave + (int64_t)kQLPre * kQLWaves; st < steps; st += kQLWaves)
        acc = mfma(load_a(st), load_b(st), acc);
    // D[4g + v][i] = t[token 4g+v][rank i]; integer adds commute, so LDS atomics
    // give the exact sum in any order
#pragma unroll
    for (int v = 0; v < 4; ++v) atomicAdd(&tsum[4 * g + v][i], acc[v]);
    lds_barrier();
    if (threadIdx.x < 256) {
        const int tok = threadIdx.x >> 4, r = threadIdx.x & 15;
        if (tok < rows) t[(m0 + tok) * kRank + r] = tsum[tok][r];
    }
}

// Tokens per group so that the codes fit the LDS budget; 0 when one row does not fit.
int quantize_lora_tokens_per_group(int64_t K) {
    const int64_t n = kQLLdsBytes / K;
    return (int)(n >= 16 ? 16 : n);
}

hipError_t launch_quantize_lora_down(const float* x, int64_t M, int64_t K, const int8_t* w_b, int rank,
                                     int8_t* x_q, float* s_x, int32_t* t, int64_t batch, hipStream_t stream) {
    int tpg = quantize_lora_tokens_per_group(K);
    if (tpg <= 0 || K % 4 != 0) return hipErrorInvalidValue;
    // Many tokens: fewer per group, so that there are about two groups per CU (each
    // group's rows are one latency-bound pass; W_B, read by every group, stays in L2).
    const int64_t want = (M * batch + 511) / 512;
    if (want < tpg) tpg = (int)(want < 1 ? 1 : want);
    // registers: the float4 per lane of a full group's rows (waves per row as the
    // kernel picks them), and W_B steps per wave
    auto wpr_of = [](int64_t rows) -> int64_t { return rows >= 8 ? 1 : (rows >= 4 ? 2 : (rows >= 2 ? 4 : 8)); };
    auto nv_of = [&](int64_t g) -> int64_t {
        const int64_t rows = M < g ? M : g, wpr = wpr_of(rows);
        return (K / 4 + wpr * kWave - 1) / (wpr * kWave);
    };
    // rows that need more than 4 float4 per lane cost the second resident group per
    // CU anyway: then take twice the rows per group (one wave per row, all rows' loads
    // in flight at once, one group per CU)
    if (M * batch >= 1024 && nv_of(tpg) > 4 && 2 * tpg <= quantize_lora_tokens_per_group(K)) tpg = 2 * tpg;
    const int64_t nv = nv_of(tpg);
    const int64_t np = ((K + 63) / 64 + kQLWaves - 1) / kQLWaves;
    const dim3 grid((unsigned)((M + tpg - 1) / tpg), (unsigned)batch);
    const size_t lds = (size_t)tpg * (size_t)K;
#define DFSSM_QL(NV, NP)                                                                                         \
    do {                                                                                                         \
        if (K % 16 == 0)                                                                                         \
            quantize_lora_down_kernel<NV, NP, true><<<grid, kQLThreads, lds, stream>>>(x, M, K, w_b, rank, x_q,  \
                                                                                       s_x, t, tpg);             \
        else                                                                                                     \
            quantize_lora_down_kernel<NV, NP, false><<<grid, kQLThreads, lds, stream>>>(x, M, K, w_b, rank, x_q, \
                                                                                        s_x, t, tpg);            \
    } while (0)
    if (nv <= 4 && np <= 4) DFSSM_QL(4, 4);
    else if (nv <= 4) DFSSM_QL(4, 8);
    else if (nv <= 8 && np <= 4) DFSSM_QL(8, 4);
    else if (nv <= 8) DFSSM_QL(8, 8);
    else DFSSM_QL(16, 8);
#undef DFSSM_QL
    return hipGetLastError();
}

}  // namespace dfssm
