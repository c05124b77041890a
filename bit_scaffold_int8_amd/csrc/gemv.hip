// gemv.hip -- decode-shaped scaffold + LoRA projection for M <= 16 tokens (gfx950).
//
// DF-SSM technical summary (gist.science), section 2C: the 1-bit scaffold weights are
// stored packed and expanded to int8 on the fly for an int8 x int8 product, which
// cuts the weight traffic eightfold against int8 weights.  At M <= 16 that packed
// weight stream is the whole cost: the kernel must run at HBM rate.
//
// Design (MI355X-first, not the pages' expand-then-cuBLAS flow):
//  * Tokens ride the 16 columns of one v_mfma_i32_16x16x64_i8; 16 scaffold rows are
//    its 16 A rows.  Padding M up to 16 costs the matrix pipe only, which has ~2.5x
//    headroom over the packed-bit stream, so M = 1, 4 and 16 cost the same ALU work.
//  * Bit-plane expansion: a 32-bit word of packed signs covers k = 8b + j (byte b,
//    bit j).  AND with (0x01010101 << j) yields four bytes 2^j * bit for k = j, j+8,
//    j+16, j+24 -- one VALU op per four expanded weights, half the cost of any
//    in-order expansion.  Each plane j feeds its own accumulator; the planes are
//    recombined exactly at the end (acc_j is a multiple of 2^j; plane 7 reads as
//    -128 in signed int8 and is negated).
//  * The activations are permuted once per workgroup into the same plane order
//    (byte transposes with v_perm_b32) and stay in VGPRs for every row tile.
//  * 0/1 weights give S = sum_{bit=1} x_q; the +-1 product follows exactly as
//    acc = 2 S - sum_k x_q.
//  * K is split across the workgroup's waves (16-byte chunks, 4 lane groups per
//    wave); the per-wave partial tiles are summed through LDS, then the fused
//    epilogue applies s_w, the LoRA up-projection and s_x and writes fp32 y.
//  * Packed weight loads are 16 bytes per lane, 64-byte contiguous runs per row per
//    instruction, and the next tile's loads are issued before the current tile's
//    MFMAs.
#include "device_common.h"

namespace dfssm {

// One lane group = 16 lanes; one chunk = 16 packed bytes = 128 k of one row.
template <int W, int C, bool kFast>
__global__ __launch_bounds__(W * kWave) void gemv_kernel(
    const int8_t* __restrict__ x_q, const float* __restrict__ s_x, int M, int64_t N, int64_t K,
    const uint8_t* __restrict__ w_bits, const float* __restrict__ s_w,
    const int8_t* __restrict__ w_a, const float* __restrict__ s_a, const float* __restrict__ s_b,
    const int32_t* __restrict__ t, int rank, float* __restrict__ y, int32_t* __restrict__ acc_dbg,
    int64_t num_tiles, int tiles_per_wg) {
    __shared__ int32_t red[W][16][17];
    __shared__ int32_t xs_part[W][kWave];
    __shared__ int32_t xsum[16];
    __shared__ float u[16][kRank];

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
            t += p * M * kRank;
        }
    }

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int i = lane & 15;
    const int g = lane >> 4;
    const int64_t RB = K / 8;

    // LoRA: u[tok][r] = s_B[r] * t[tok][r] (fp32), shared by every output row.
    for (int e = threadIdx.x; e < 16 * kRank; e += W * kWave) {
        const int tok = e / kRank, r = e % kRank;
        u[tok][r] = (rank != 0 && tok < M) ? s_b[r] * (float)t[tok * kRank + r] : 0.0f;
    }

    // Activations of token i in bit-plane order, for this lane's chunks.
    v4i X[C][8];
    int32_t xpart = 0;
    const uint8_t* xrow = reinterpret_cast<const uint8_t*>(x_q) + (i < M ? (int64_t)i * K : 0);
    const int64_t xlimit = i < M ? K : 0;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int64_t q = ((int64_t)c * W + wave) * 4 + g;
        const int64_t kb = 128 * q;
        uint32_t nat[32];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint4 v = load16_guarded(xrow, kb + 16 * e, xlimit, kFast);
            nat[4 * e + 0] = v.x;
            nat[4 * e + 1] = v.y;
            nat[4 * e + 2] = v.z;
            nat[4 * e + 3] = v.w;
        }
#pragma unroll
        for (int e = 0; e < 32; ++e) xpart = byte_sum(nat[e], xpart);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
#pragma unroll
            for (int jh = 0; jh < 2; ++jh) {
                uint32_t o0, o1, o2, o3;
                transpose4x4(nat[8 * qq + 0 + jh], nat[8 * qq + 2 + jh], nat[8 * qq + 4 + jh],
                             nat[8 * qq + 6 + jh], o0, o1, o2, o3);
                X[c][4 * jh + 0][qq] = (int)o0;
                X[c][4 * jh + 1][qq] = (int)o1;
                X[c][4 * jh + 2][qq] = (int)o2;
                X[c][4 * jh + 3][qq] = (int)o3;
            }
        }
    }
    xs_part[wave][lane] = xpart;
    __syncthreads();
    if (threadIdx.x < 16) {
        int32_t s = 0;
        for (int w = 0; w < W; ++w)
            for (int gg = 0; gg < 4; ++gg) s += xs_part[w][16 * gg + threadIdx.x];
        xsum[threadIdx.x] = s;
    }
    // (xsum is read after the first tile's barrier below)

    const int64_t tile_begin = (int64_t)blockIdx.x * tiles_per_wg;
    const int64_t tile_end = tile_begin + tiles_per_wg < num_tiles ? tile_begin + tiles_per_wg : num_tiles;

    auto load_tile = [&](int64_t tile, uint4 (&wv)[C]) {
        const int64_t n = tile * 16 + i;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int64_t q = ((int64_t)c * W + wave) * 4 + g;
            wv[c] = (n < N) ? load16_guarded(w_bits + n * RB, 16 * q, RB, kFast) : make_uint4(0u, 0u, 0u, 0u);
        }
    };

    uint4 wcur[C];
    if (tile_begin < tile_end) load_tile(tile_begin, wcur);
    for (int64_t tile = tile_begin; tile < tile_end; ++tile) {
        uint4 wnext[C];
        if (tile + 1 < tile_end) load_tile(tile + 1, wnext);

        v4i acc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = (v4i){0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < C; ++c) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t msk = 0x01010101u << j;
                const v4i a = {(int)(wcur[c].x & msk), (int)(wcur[c].y & msk),
                               (int)(wcur[c].z & msk), (int)(wcur[c].w & msk)};
                acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, X[c][j], acc[j], 0, 0, 0);
            }
        }
        // D[4g + v][i]: scaffold row 4g+v of the tile, token i.
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            int32_t s = -(acc[7][v] >> 7);
#pragma unroll
            for (int j = 0; j < 7; ++j) s += acc[j][v] >> j;
            red[wave][4 * g + v][i] = s;
        }
        __syncthreads();
        for (int e = threadIdx.x; e < 16 * M; e += W * kWave) {
            const int row = e & 15, tok = e >> 4;
            const int64_t n = tile * 16 + row;
            if (n < N) {
                int32_t s1 = 0;
#pragma unroll
                for (int w = 0; w < W; ++w) s1 += red[w][row][tok];
                const int32_t acc_pm = 2 * s1 - xsum[tok];
                if (acc_dbg) acc_dbg[(int64_t)tok * N + n] = acc_pm;
                float lora = 0.0f;
                if (rank != 0) {
                    const uint4 wa = *reinterpret_cast<const uint4*>(w_a + n * kRank);
                    const uint32_t words[4] = {wa.x, wa.y, wa.z, wa.w};
#pragma unroll
                    for (int r = 0; r < kRank; ++r) {
                        const float a = (float)(int8_t)(words[r >> 2] >> (8 * (r & 3)));
                        lora = fmaf(a, u[tok][r], lora);
                    }
                }
                const float inner = rank != 0 ? fmaf(s_a[n], lora, s_w[n] * (float)acc_pm)
                                              : s_w[n] * (float)acc_pm;
                y[(int64_t)tok * N + n] = s_x[tok] * inner;
            }
        }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < C; ++c) wcur[c] = wnext[c];
    }
}

template <int W, int C>
static hipError_t launch_gemv_wc(bool fast, const int8_t* x_q, const float* s_x, int M, int64_t N,
                                 int64_t K, const uint8_t* w_bits, const float* s_w, const int8_t* w_a,
                                 const float* s_a, const float* s_b, const int32_t* t, int rank,
                                 float* y, int32_t* acc_dbg, int64_t batch, hipStream_t stream) {
    // Enough workgroups to fill 256 CUs several times over; beyond that each group
    // takes more row tiles, which amortizes its activation setup.
    const int64_t num_tiles = (N + 15) / 16;
    const int64_t target_wgs = 2048;
    const int64_t per_problem = (target_wgs + batch - 1) / batch;
    const int tiles_per_wg = (int)((num_tiles + per_problem - 1) / per_problem);
    const dim3 grid((unsigned)((num_tiles + tiles_per_wg - 1) / tiles_per_wg), (unsigned)batch);
    if (fast) {
        gemv_kernel<W, C, true><<<grid, W * kWave, 0, stream>>>(x_q, s_x, M, N, K, w_bits, s_w, w_a, s_a, s_b,
                                                                t, rank, y, acc_dbg, num_tiles, tiles_per_wg);
    } else {
        gemv_kernel<W, C, false><<<grid, W * kWave, 0, stream>>>(x_q, s_x, M, N, K, w_bits, s_w, w_a, s_a, s_b,
                                                                 t, rank, y, acc_dbg, num_tiles, tiles_per_wg);
    }
    return hipGetLastError();
}


hipError_t launch_gemv(const int8_t* x_q, const float* s_x, int M, int64_t N, int64_t K,
                       const uint8_t* w_bits, const float* s_w, const int8_t* w_a, const float* s_a,
                       const float* s_b, const int32_t* t, int rank, float* y, int32_t* acc_dbg,
                       int64_t batch, hipStream_t stream) {
    const int64_t RB = K / 8;
    const int64_t NC = (RB + 15) / 16;  // 16-byte chunks per row
    const bool fast = (RB % 16 == 0) && ((uintptr_t)w_bits % 16 == 0) && ((uintptr_t)x_q % 16 == 0);
#define DFSSM_GEMV(Wv, Cv) \
    return launch_gemv_wc<Wv, Cv>(fast, x_q, s_x, M, N, K, w_bits, s_w, w_a, s_a, s_b, t, rank, y, acc_dbg, batch, \
                                  stream)
    if (NC <= 4) DFSSM_GEMV(1, 1);
    if (NC <= 8) DFSSM_GEMV(2, 1);
    if (NC <= 16) DFSSM_GEMV(4, 1);
    if (NC <= 32) DFSSM_GEMV(8, 1);
    // 512-thread groups keep the full 256-VGPR budget for the wider activation slices
    if (NC <= 64) DFSSM_GEMV(8, 2);
    if (NC <= 128) DFSSM_GEMV(8, 4);
#undef DFSSM_GEMV
    return hipErrorInvalidValue;
}

}  // namespace dfssm
