// gemm_mfma.hip -- prefill-shaped scaffold + LoRA projection on the int8 MFMA pipe (gfx950).
//
// DF-SSM technical summary (gist.science), section 2C: packed 1-bit scaffold
// weights are expanded to int8 and multiplied with int8 activations on the matrix
// cores.  At many tokens this is a dense int8 contraction, so it belongs on
// v_mfma_i32_32x32x32_i8.  Unlike the pages' flow (expand to a dense int8 copy in
// memory, then a library GEMM), nothing is materialized: each wave expands its
// B-fragments from the packed bits in registers, K-step by K-step.
//
// Tiling: 128 x 128 output tile per 256-thread workgroup, 2 x 2 waves of 64 x 64,
// each a 2 x 2 grid of 32 x 32 MFMA accumulators; K-step 64.
//  * A (x_q, natural k order) is staged through LDS with 16-byte loads/stores;
//    rows are padded to 80 bytes against bank conflicts.  The staging threads also
//    accumulate each token row's sum of codes (needed below) with v_dot4.
//  * B: each lane owns one scaffold row of a 32-column block and 32 consecutive k
//    (one 4-byte load), expands them nibble by nibble to 0/1 bytes
//    ((nib * 0x00204081) & 0x01010101), and feeds two MFMAs.  The A-fragment read
//    for the same lane covers the same 16 k values, which is all the MFMA needs.
//  * 0/1 weights give S = sum_{bit=1} x_q; the +-1 result is exact as acc = 2 S - rowsum.
//  * Epilogue: y = s_x * (s_w * acc + s_A * sum_r W_A[n][r] * (s_B[r] t[m][r])), with
//    s_B * t and W_A staged in LDS as fp32.
//  * kTin: t = W_B x_q is computed here too, one v_mfma_i32_16x16x64_i8 per 16 token
//    rows per K-step (A = the staged codes, B = the 16 rows of W_B); each wave owns 32
//    of the tile's rows.
#include "device_common.h"

namespace dfssm {

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kLdA = kBK + 16;  // LDS row stride (bytes)

__device__ __forceinline__ uint32_t spread_nibble(uint32_t w, int shift) {
    return (((w >> shift) & 0xFu) * 0x00204081u) & 0x01010101u;
}

template <bool kFast, bool kTin>
__global__ __launch_bounds__(256) void gemm_mfma_kernel(
    const int8_t* __restrict__ x_q, const float* __restrict__ s_x, int64_t M, int64_t N, int64_t K,
    const uint8_t* __restrict__ w_bits, const float* __restrict__ s_w,
    const int8_t* __restrict__ w_a, const float* __restrict__ s_a, const float* __restrict__ s_b,
    const int32_t* __restrict__ t, int rank, float* __restrict__ y, int32_t* __restrict__ acc_dbg,
    int64_t tiles_n, const int8_t* __restrict__ w_b, int32_t* __restrict__ t_out) {
    __shared__ __align__(16) uint8_t As[kBM * kLdA];
    __shared__ int32_t rowsum[kBM];
    __shared__ float uS[kBM][kRank + 1];
    __shared__ float waS[kBN][kRank + 1];
    __shared__ int32_t tS[kTin ? kBM : 1][kRank];

    // problem blockIdx.y of a dense batch (every operand advanced by its own size)
    {
        const int64_t p = blockIdx.y;
        x_q += p * M * K;
        s_x += p * M;
        w_bits += p * N * (K / 8);
        s_w += p * N;
        y += p * M * N;
        if (acc_dbg) acc_dbg += p * M * N;
        if (rank != 0) {
            w_a += p * N * kRank;
            s_a += p * N;
            s_b += p * kRank;
            if (kTin) {
                w_b += p * kRank * K;
                if (t_out) t_out += p * M * kRank;
            } else {
                t += p * M * kRank;
            }
        }
    }

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int wm = wave & 1, wn = wave >> 1;
    const int64_t tile_m = blockIdx.x / tiles_n, tile_n = blockIdx.x % tiles_n;
    const int64_t m0 = tile_m * kBM, n0 = tile_n * kBN;
    const int64_t RB = K / 8;

    // A staging: thread -> (row, 32-byte half of the K-step)
    const int srow = tid >> 1, shalf = tid & 1;
    const int64_t gm = m0 + srow;
    const uint8_t* xrow = reinterpret_cast<const uint8_t*>(x_q) + (gm < M ? gm * K : 0);
    const int64_t xlimit = gm < M ? K : 0;
    int32_t rs = 0;

    // B: lane -> scaffold row of each 32-column block, 32-k group
    const int g = lane >> 5;
    const uint8_t* brow[2];
    int64_t blimit[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const int64_t n = n0 + wn * 64 + nb * 32 + (lane & 31);
        brow[nb] = w_bits + (n < N ? n * RB : 0);
        blimit[nb] = n < N ? RB : 0;
    }

    v16i acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = (v16i){};
    // kTin: W_B row (lane & 15), k-slice 16 (lane >> 4) of each K-step; rows
    // 32 wave + 16 j + (lane & 15) of the tile
    const uint8_t* wbrow = reinterpret_cast<const uint8_t*>(kTin ? w_b : x_q) + (kTin ? (int64_t)(lane & 15) * K : 0);
    v4i tacc[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};

    for (int64_t k0 = 0; k0 < K; k0 += kBK) {
        const uint4 a0 = load16_guarded<kFast>(xrow, k0 + 32 * shalf, xlimit);
        const uint4 a1 = load16_guarded<kFast>(xrow, k0 + 32 * shalf + 16, xlimit);
        uint32_t bw[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) bw[nb] = load4_guarded<kFast>(brow[nb], k0 / 8 + 4 * g, blimit[nb]);
        rs = byte_sum(a0.x, rs); rs = byte_sum(a0.y, rs); rs = byte_sum(a0.z, rs); rs = byte_sum(a0.w, rs);
        rs = byte_sum(a1.x, rs); rs = byte_sum(a1.y, rs); rs = byte_sum(a1.z, rs); rs = byte_sum(a1.w, rs);
        __syncthreads();  // previous K-step's fragment reads are done
        *reinterpret_cast<uint4*>(As + srow * kLdA + 32 * shalf) = a0;
        *reinterpret_cast<uint4*>(As + srow * kLdA + 32 * shalf + 16) = a1;
        __syncthreads();
        if constexpr (kTin) {
            const uint4 wv = load16_guarded<kFast>(wbrow, k0 + 16 * (lane >> 4), K);
            const v4i bt = {(int)wv.x, (int)wv.y, (int)wv.z, (int)wv.w};
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const v4i at = *reinterpret_cast<const v4i*>(As + (32 * wave + 16 * j + (lane & 15)) * kLdA +
                                                             16 * (lane >> 4));
                tacc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(at, bt, tacc[j], 0, 0, 0);
            }
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            v4i af[2];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
                af[mb] = *reinterpret_cast<const v4i*>(As + (wm * 64 + mb * 32 + (lane & 31)) * kLdA + 32 * g + 16 * s);
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                const v4i bf = {(int)spread_nibble(bw[nb], 16 * s + 0), (int)spread_nibble(bw[nb], 16 * s + 4),
                                (int)spread_nibble(bw[nb], 16 * s + 8), (int)spread_nibble(bw[nb], 16 * s + 12)};
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[mb], bf, acc[mb][nb], 0, 0, 0);
            }
        }
    }

    // row sums of the codes, LoRA operands for this tile
    rs += __shfl_xor(rs, 1, kWave);
    if (shalf == 0) rowsum[srow] = rs;
    if constexpr (kTin) {
        // D[4 (lane >> 4) + v][lane & 15] = t[row 32 wave + 16 j + 4 (lane >> 4) + v][rank lane & 15]
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) tS[32 * wave + 16 * j + 4 * (lane >> 4) + v][lane & 15] = tacc[j][v];
        __syncthreads();
        if (t_out && rank != 0 && tile_n == 0) {
            for (int e = tid; e < kBM * kRank; e += 256) {
                const int64_t m = m0 + e / kRank;
                if (m < M) t_out[m * kRank + e % kRank] = tS[e / kRank][e % kRank];
            }
        }
    }
    for (int e = tid; e < kBM * kRank; e += 256) {
        const int r = e % kRank, row = e / kRank;
        const int64_t m = m0 + row;
        const float tv = kTin ? (float)tS[row][r] : (rank != 0 && m < M) ? (float)t[m * kRank + r] : 0.0f;
        uS[row][r] = (rank != 0 && m < M) ? s_b[r] * tv : 0.0f;
        const int64_t n = n0 + row;
        waS[row][r] = (rank != 0 && n < N) ? (float)w_a[n * kRank + r] : 0.0f;
    }
    __syncthreads();

#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const int col = wn * 64 + nb * 32 + (lane & 31);
            const int64_t n = n0 + col;
            if (n >= N) continue;
            const float sw = s_w[n];
            const float sa = rank != 0 ? s_a[n] : 0.0f;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = wm * 64 + mb * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                const int64_t m = m0 + row;
                if (m >= M) continue;
                const int32_t acc_pm = 2 * acc[mb][nb][v] - rowsum[row];
                if (acc_dbg) acc_dbg[m * N + n] = acc_pm;
                float lora = 0.0f;
#pragma unroll
                for (int r = 0; r < kRank; ++r) lora = fmaf(waS[col][r], uS[row][r], lora);
                const float inner = rank != 0 ? fmaf(sa, lora, sw * (float)acc_pm) : sw * (float)acc_pm;
                y[m * N + n] = s_x[m] * inner;
            }
        }
    }
}

// t given (w_b == NULL), or computed here from W_B (t_out, when not NULL, receives it).
hipError_t launch_gemm_mfma(const int8_t* x_q, const float* s_x, int64_t M, int64_t N, int64_t K,
                            const uint8_t* w_bits, const float* s_w, const int8_t* w_a, const float* s_a,
                            const int8_t* w_b, const float* s_b, const int32_t* t, int32_t* t_out, int rank,
                            float* y, int32_t* acc_dbg, int64_t batch, hipStream_t stream) {
    const int64_t tiles_m = (M + kBM - 1) / kBM, tiles_n = (N + kBN - 1) / kBN;
    const int64_t grid = tiles_m * tiles_n;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    const bool tin = rank != 0 && w_b != nullptr;
    const bool fast = (K % 64 == 0) && ((uintptr_t)x_q % 16 == 0) && ((uintptr_t)w_bits % 16 == 0) &&
                      (!tin || (uintptr_t)w_b % 16 == 0);
    const dim3 g3((unsigned)grid, (unsigned)batch);
#define DFSSM_MFMA_LAUNCH(FAST, TIN)                                                                          \
    gemm_mfma_kernel<FAST, TIN><<<g3, 256, 0, stream>>>(x_q, s_x, M, N, K, w_bits, s_w, w_a, s_a, s_b, t, rank, \
                                                        y, acc_dbg, tiles_n, w_b, t_out)
    if (fast) {
        if (tin) {
            DFSSM_MFMA_LAUNCH(true, true);
        } else {
            DFSSM_MFMA_LAUNCH(true, false);
        }
    } else if (tin) {
        DFSSM_MFMA_LAUNCH(false, true);
    } else {
        DFSSM_MFMA_LAUNCH(false, false);
    }
#undef DFSSM_MFMA_LAUNCH
    return hipGetLastError();
}

}  // namespace dfssm
