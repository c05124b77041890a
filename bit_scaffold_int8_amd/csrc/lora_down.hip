// lora_down.hip -- LoRA down-projection t[m][r] = sum_k W_B[r][k] * x_q[m][k] (gfx950).
//
// DF-SSM technical summary (gist.science), section 2B: the rank-16 int8 correction
// W_A (d_out x r) . W_B (r x d_in) is applied to the same int8 activations as the
// scaffold; t stays an exact int32 and is scaled in the epilogue.
//
// A 16-token x 16-rank output tile is one v_mfma_i32_16x16x64_i8 accumulator:
// A = 16 token rows of x_q, B = the 16 rows of W_B, both read straight from global
// memory in natural k order (each lane loads the same 16 k-values of its token and
// of its rank, which is all the MFMA needs: A and B share the per-lane k set).
// The K range is split across the workgroup's waves (64 k per wave per step) and
// the partial tiles are summed through LDS.  One workgroup per 16 tokens.
#include "device_common.h"

namespace dfssm {

constexpr int kLoraWaves = 8;

template <bool kFast>
__global__ __launch_bounds__(kLoraWaves * kWave) void lora_down_kernel(
    const int8_t* __restrict__ x_q, int64_t M, int64_t K, const int8_t* __restrict__ w_b,
    int32_t* __restrict__ t) {
    // problem blockIdx.y of a dense batch: x_q [M][K], W_B [16][K], t [M][16] each
    const int64_t p = blockIdx.y;
    x_q += p * M * K;
    w_b += p * kRank * K;
    t += p * M * kRank;
    __shared__ int32_t part[kLoraWaves][16][16];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int i = lane & 15;   // token row (A) / rank column (B)
    const int g = lane >> 4;   // 16-byte k group
    const int64_t m0 = (int64_t)blockIdx.x * 16;
    const int64_t m = m0 + i;
    const uint8_t* xrow = reinterpret_cast<const uint8_t*>(x_q) + (m < M ? m : 0) * K;
    const uint8_t* brow = reinterpret_cast<const uint8_t*>(w_b) + (int64_t)i * K;
    const int64_t xlimit = m < M ? K : 0;

    v4i acc = {0, 0, 0, 0};
    const int64_t steps = (K + 63) / 64;
    for (int64_t s = wave; s < steps; s += kLoraWaves) {
        const int64_t off = s * 64 + 16 * g;
        const uint4 a = load16_guarded<kFast>(xrow, off, xlimit);
        const uint4 b = load16_guarded<kFast>(brow, off, K);
        const v4i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w};
        const v4i bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w};
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv, acc, 0, 0, 0);
    }
    // D[4g + v][i]: token 4g+v, rank i
#pragma unroll
    for (int v = 0; v < 4; ++v) part[wave][4 * g + v][i] = acc[v];
    lds_barrier();
    if (threadIdx.x < 256) {
        const int tok = threadIdx.x >> 4, r = threadIdx.x & 15;
        int32_t s = 0;
#pragma unroll
        for (int w = 0; w < kLoraWaves; ++w) s += part[w][tok][r];
        if (m0 + tok < M) t[(m0 + tok) * kRank + r] = s;
    }
}

hipError_t launch_lora_down(const int8_t* x_q, int64_t M, int64_t K, const int8_t* w_b, int32_t* t,
                            int64_t batch, hipStream_t stream) {
    const bool fast = (K % 16 == 0) && ((uintptr_t)x_q % 16 == 0) && ((uintptr_t)w_b % 16 == 0);
    const dim3 grid((unsigned)((M + 15) / 16), (unsigned)batch);
    if (fast) {
        lora_down_kernel<true><<<grid, kLoraWaves * kWave, 0, stream>>>(x_q, M, K, w_b, t);
    } else {
        lora_down_kernel<false><<<grid, kLoraWaves * kWave, 0, stream>>>(x_q, M, K, w_b, t);
    }
    return hipGetLastError();
}

}  // namespace dfssm
