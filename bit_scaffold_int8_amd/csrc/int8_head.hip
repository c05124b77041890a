// int8_head.hip -- the int8 embedding / LM head of the model (gfx950).
//
// DF-SSM technical summary (gist.science): besides the 1-bit scaffold and the int8
// LoRA, the embedding and LM-head matrix is int8 with a per-row scale (one tied matrix,
// 37 % of the model's bytes).  Two operations use it:
//  * the LM head, an int8 x int8 product of the tokens' int8 codes (the same per-token
//    absmax codes as the projections) with every row:
//        acc[m][n] = sum_k E[n][k] x_q[m][k]   (exact int32)
//        y[m][n]   = s_x[m] * (s_e[n] * acc[m][n])   (fp32)
//  * the embedding lookup, a dequantized row: out[t][k] = s_e[id] * E[id][k].
//
// The head at decode (M <= 16 tokens) streams N x K bytes once: HBM-bound.  Its kernel
// has the decode scaffold kernel's shape with int8 operands straight from memory:
//  * 16 rows of E are the A rows of v_mfma_i32_16x16x64_i8 and the tokens its 16 B
//    columns, so M = 1 .. 16 cost the same;
//  * K is split over the 8 waves of a group in 16-byte pieces (lane group g of wave w
//    takes pieces (c W + w) 4 + g, c < C), each lane's A operand is 16 bytes of one
//    row and its B operand the token's 16 codes of the same piece (held in registers
//    for the whole group), so any piece order is consistent;
//  * rows go in stages of T tiles, loaded through a buffer resource two stages ahead
//    into three register buffers that rotate by name; the waves' partial sums meet in
//    LDS (atomics from the token lanes), double-buffered by stage parity so one
//    barrier per stage suffices; the epilogue scales each stage's outputs into LDS,
//    and the group writes its whole [M][rows] block of y once, after its last stage
//    (small stores mixed into the weight stream slow the stream down).
#include "device_common.h"

namespace dfssm {

constexpr int kHeadWaves = 8;
constexpr int kHeadThreads = kHeadWaves * kWave;
constexpr int kHeadRowsCap = 512;  // rows one group owns at most (their scales and y live in LDS)

// C 16-byte pieces per lane per row, T 16-row tiles per stage.
template <int C, int T>
__global__ __launch_bounds__(kHeadThreads) void int8_gemv_kernel(
    const int8_t* __restrict__ x_q, const float* __restrict__ s_x, int M, int64_t N, int64_t K,
    const int8_t* __restrict__ e, const float* __restrict__ s_e, float* __restrict__ y,
    int32_t* __restrict__ acc_dbg, int64_t num_tiles, int stages_per_wg) {
    constexpr int W = kHeadWaves, NT = kHeadThreads;
    static_assert(NT % (T * 16) == 0, "a stage's rows must divide the group size");
    constexpr int kTokStride = NT / (T * 16);
    constexpr int E = (16 + kTokStride - 1) / kTokStride;  // tokens per epilogue thread

    __shared__ float se_lds[kHeadRowsCap];
    __shared__ float y_lds[16][kHeadRowsCap];  // [token][row of the group]
    // row stride 20 words: the adds of one instruction (rows 4g+v, tokens i) hit
    // distinct banks
    __shared__ int32_t red[2][T * 16][20];
    __shared__ float sxs[kHeadThreads];  // token scales in the first M slots (one slot per thread)

    {
        const int64_t p = blockIdx.y;  // problem of a dense batch
        x_q += p * M * K;
        s_x += p * M;
        e += p * N * K;
        s_e += p * N;
        y += p * M * N;
        if (acc_dbg) acc_dbg += p * M * N;
    }
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const int i = lane & 15, g = lane >> 4;
    const int64_t num_stages = (num_tiles + T - 1) / T;
    const int64_t st_begin = (int64_t)blockIdx.x * stages_per_wg;
    const int64_t st_end = st_begin + stages_per_wg < num_stages ? st_begin + stages_per_wg : num_stages;

    // weights through a buffer resource over this problem's matrix: rows past N read
    // zero; a piece past K reads the row's first piece and meets zero codes
    const __amdgpu_buffer_rsrc_t e_rsrc = make_rsrc(e, (uint32_t)(N * K));
    int lane_off[C];
    bool piece_live[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int64_t piece = ((int64_t)c * W + wave) * 4 + g;
        piece_live[c] = 16 * piece < K;
        lane_off[c] = (int)((int64_t)i * K + (piece_live[c] ? 16 * piece : 0));
    }
    const int tile_bytes = (int)(16 * K);
    struct Stage {
        v4i w[T][C];
    };
    auto load_stage = [&](int64_t st, Stage& b) {
#pragma unroll
        for (int tt = 0; tt < T; ++tt) {
            const int base = (int)((st * T + tt) * tile_bytes);
#pragma unroll
            for (int c = 0; c < C; ++c) b.w[tt][c] = __builtin_amdgcn_raw_buffer_load_b128(e_rsrc, base + lane_off[c], 0, 0);
        }
    };
    // The small setup loads go out first, into registers: waits count loads in issue
    // order, so the wait for them (before their LDS stores and the setup barrier) then
    // leaves the first two weight stages in flight, instead of waiting for both to land
    // and only then issuing the third.
    // The group's row scales: one per thread (kHeadRowsCap == NT), rows clamped below N
    // (clamped rows are never stored).
    static_assert(kHeadRowsCap <= NT, "one row scale per thread");
    const int64_t row0 = st_begin * T * 16;
    const int nrows = (int)((st_end - st_begin) * T * 16);
    const float sev = s_e[row0 + threadIdx.x < N ? row0 + threadIdx.x : N - 1];
    // token i's codes for this lane's pieces (tokens past M and pieces past K: zero)
    v4i X[C];
    const uint8_t* xrow = reinterpret_cast<const uint8_t*>(x_q) + (i < M ? (int64_t)i * K : 0);
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int64_t piece = ((int64_t)c * W + wave) * 4 + g;
        const uint4 v = load16_select(xrow, piece_live[c] ? 16 * piece : 0, i < M && piece_live[c]);
        X[c] = (v4i){(int)v.x, (int)v.y, (int)v.z, (int)v.w};
    }
    const float sxv = __uint_as_float(__float_as_uint(s_x[threadIdx.x < M ? threadIdx.x : 0]) &
                                      opaque_mask(threadIdx.x < M));

    Stage s0, s1, s2;
    load_stage(st_begin, s0);  // every group has at least one stage
    load_stage(st_begin + 1 < st_end ? st_begin + 1 : st_end - 1, s1);

    // (every thread stores its slot, so neither load has a branch to sink into, where
    // the wait for it would also wait for the stages; slots past the group's rows and
    // past M tokens are never read)
    se_lds[threadIdx.x] = sev;
    sxs[threadIdx.x] = sxv;
    for (int q = threadIdx.x; q < 2 * T * 16 * 20; q += NT) (&red[0][0][0])[q] = 0;
    lds_barrier();

    const __amdgpu_buffer_rsrc_t acc_rsrc = make_rsrc(acc_dbg, acc_dbg ? (uint32_t)(M * N * 4) : 0u);
    const int erow = threadIdx.x % (T * 16);
    const int etok0 = threadIdx.x / (T * 16);

    // One stage: prefetch two ahead (a clamped index past the range re-reads the last
    // stage, so the load is unconditional), then consume `cur`.  Branches hold no
    // global loads, so the compiler's waits stay partial and prefetches stay in flight.
    auto run_stage = [&](int64_t st, Stage& cur, Stage& nxt2, int rb) {
        load_stage(st + 2 < st_end ? st + 2 : st_end - 1, nxt2);
        if (st >= st_end) return;  // uniform
#pragma unroll
        for (int tt = 0; tt < T; ++tt) {
            v4i acc = {0, 0, 0, 0};
#pragma unroll
            for (int c = 0; c < C; ++c) acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(cur.w[tt][c], X[c], acc, 0, 0, 0);
            // D[4g + v][i]: row 4g+v of tile tt, token i
            if (i < M) {
#pragma unroll
                for (int v = 0; v < 4; ++v) atomicAdd(&red[rb][tt * 16 + 4 * g + v][i], acc[v]);
            }
        }
        lds_barrier();
        const int64_t n = st * T * 16 + erow;
        const float se = se_lds[n - row0];
#pragma unroll
        for (int q = 0; q < E; ++q) {
            const int tok = etok0 + q * kTokStride;
            if (tok < M) {
                const int32_t a = red[rb][erow][tok];
                red[rb][erow][tok] = 0;  // ready for the stage after next
                y_lds[tok][n - row0] = sxs[tok] * (se * (float)a);
                if (acc_dbg) store_i32(a, acc_rsrc, n < N ? (int)(((int64_t)tok * N + n) * 4) : kOffDead);
            }
        }
        // no second barrier: the next stage adds into the other buffer, and this one is
        // added into again only after the next stage's barrier
    };
    for (int64_t st = st_begin; st < st_end; st += 3) {
        const int rb = (int)((st - st_begin) & 1);
        run_stage(st, s0, s2, rb);
        run_stage(st + 1, s1, s0, rb ^ 1);
        run_stage(st + 2, s2, s1, rb);
    }
    // the group's y: token by token, its rows below N, consecutive threads on
    // consecutive rows (one coalesced run per token)
    lds_barrier();
    const int live_rows = (int)(N - row0 < nrows ? N - row0 : nrows);
    const __amdgpu_buffer_rsrc_t y_rsrc = make_rsrc(y + row0, (uint32_t)((M - 1) * N * 4 + live_rows * 4));
    for (int q = threadIdx.x; q < M * live_rows; q += NT) {
        const int tok = q / live_rows, r = q - tok * live_rows;
        store_f32(y_lds[tok][r], y_rsrc, (int)(((int64_t)tok * N + r) * 4));
    }
}

template <int C, int T>
static hipError_t launch_int8_gemv_ct(const int8_t* x_q, const float* s_x, int M, int64_t N, int64_t K,
                                      const int8_t* e, const float* s_e, float* y, int32_t* acc_dbg, int64_t batch,
                                      hipStream_t stream) {
    const int64_t num_tiles = (N + 15) / 16;
    const int64_t num_stages = (num_tiles + T - 1) / T;
    // large total work: one group per CU, each over a long run of stages (measured on
    // the 50280 x 2048 head: 242 groups of 13 stages 22.7 us, 449 groups of 7 stages
    // 25.9 us, 1572 groups of 2 stages 36 us -- with one MFMA per 16 weight bytes there
    // is little work for a second group per CU to hide); otherwise ~8 groups per CU
    const int64_t resident_wgs = 256;
    const int64_t target_wgs = batch * num_stages >= 4 * resident_wgs ? resident_wgs : 2048;
    const int64_t per_problem = (target_wgs + batch - 1) / batch;
    int stages_per_wg = (int)((num_stages + per_problem - 1) / per_problem);
    if (stages_per_wg * T * 16 > kHeadRowsCap) stages_per_wg = kHeadRowsCap / (T * 16);
    const dim3 grid((unsigned)((num_stages + stages_per_wg - 1) / stages_per_wg), (unsigned)batch);
    int8_gemv_kernel<C, T><<<grid, kHeadThreads, 0, stream>>>(x_q, s_x, M, N, K, e, s_e, y, acc_dbg, num_tiles,
                                                              stages_per_wg);
    return hipGetLastError();
}

// Whether the head kernel takes the shape: M <= 16 tokens, K % 16 == 0, K <= 4096.
bool int8_head_supported(int64_t M, int64_t K) { return M >= 1 && M <= 16 && K % 16 == 0 && K >= 16 && K <= 4096; }

hipError_t launch_int8_head(const int8_t* x_q, const float* s_x, int M, int64_t N, int64_t K, const int8_t* e,
                            const float* s_e, float* y, int32_t* acc_dbg, int64_t batch, hipStream_t stream) {
    if (!int8_head_supported(M, K)) return hipErrorInvalidValue;
    // pieces per lane: ceil(K / 16 / (4 lane groups x 8 waves)); stages of ~4 KB per wave
    const int64_t pieces = K / 16;
    if (pieces <= 32) return launch_int8_gemv_ct<1, 4>(x_q, s_x, M, N, K, e, s_e, y, acc_dbg, batch, stream);
    if (pieces <= 64) return launch_int8_gemv_ct<2, 2>(x_q, s_x, M, N, K, e, s_e, y, acc_dbg, batch, stream);
    if (pieces <= 128) return launch_int8_gemv_ct<4, 1>(x_q, s_x, M, N, K, e, s_e, y, acc_dbg, batch, stream);
    return launch_int8_gemv_ct<8, 1>(x_q, s_x, M, N, K, e, s_e, y, acc_dbg, batch, stream);
}

// ---------------------------------------------------------------- embedding lookup

// out[t][k] = s_e[id] * E[id][k] for id = tokens[t]; ids outside [0, V) give zeros.
// One thread per output element (grid-stride); a tiny, latency-bound kernel.
__global__ __launch_bounds__(256) void embedding_lookup_kernel(const int32_t* __restrict__ tokens, int64_t T,
                                                               const int8_t* __restrict__ e,
                                                               const float* __restrict__ s_e, int64_t V, int64_t K,
                                                               float* __restrict__ out) {
    const int64_t total = T * K;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = idx / K, k = idx - t * K;
        const int64_t id = tokens[t];
        float v = 0.0f;
        if (id >= 0 && id < V) v = s_e[id] * (float)e[id * K + k];
        out[idx] = v;
    }
}

hipError_t launch_embedding_lookup(const int32_t* tokens, int64_t T, const int8_t* e, const float* s_e, int64_t V,
                                   int64_t K, float* out, hipStream_t stream) {
    const int64_t total = T * K;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    embedding_lookup_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(tokens, T, e, s_e, V, K, out);
    return hipGetLastError();
}

}  // namespace dfssm
