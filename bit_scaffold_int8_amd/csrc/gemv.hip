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
//    j+16, j+24 -- one VALU op per four expanded weights.  Planes 4..7 come from the
//    word shifted right by 4 under the same four masks, so planes j and j+4 share
//    accumulator j (weights 2^j, never the int8 sign bit); the four accumulators are
//    recombined exactly once per tile as (8 acc0 + 4 acc1 + 2 acc2 + acc3) / 8.
//  * The activations are permuted once per workgroup into the same plane order
//    (byte transposes with v_perm_b32) and stay in VGPRs for every row tile.
//  * 0/1 weights give S = sum_{bit=1} x_q; the +-1 product follows exactly as
//    acc = 2 S - sum_k x_q.
//  * K is split across the workgroup's waves (16-byte chunks, 4 lane groups per
//    wave); the per-wave partial tiles are summed through LDS, then the fused
//    epilogue applies s_w, the LoRA up-projection and s_x and writes fp32 y.
//  * Epilogue operands: the group's rows of W_A, s_A and s_w are copied into LDS at the
//    start by buffer loads with an LDS destination (no registers held).  For up to 4
//    tokens, the LoRA up-projection of every row is formed once after the setup and y
//    is held in LDS, written after the last stage: small scattered stores interleaved
//    with the packed-sign stream slow the stream far beyond their bytes.
//  * Memory pipeline: rows go in stages of T 16-row tiles.  Packed-sign loads are
//    16 bytes per lane (64-byte runs per row per instruction), issued two stages
//    ahead of their use from clamped always-valid addresses (never masked, so never
//    waited for early), and the barriers between stages order LDS only, so the
//    prefetched loads stay in flight across them.
#include "device_common.h"
#include "quant_common.h"

namespace dfssm {

// A workgroup barrier for the setup's LDS exchanges only: this wave's LDS operations
// complete (lgkmcnt), then the barrier, with the compiler kept from moving memory
// operations across it.  Unlike lds_barrier's release fence it does not wait for the
// rows' LDS-destination loads still in flight (they are waited for by the lds_barrier
// ahead of their first use), so the setup's steps overlap their arrival.
__device__ __forceinline__ void setup_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt left alone
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Where a group's setup takes the tokens' codes and the LoRA down-projection from:
//  kGivenT   x_q and t = W_B x_q are inputs (t from a LoRA-down call);
//  kQuantize x is the input: the setup quantizes the tokens and computes t itself (the
//            one-call form; x_q, s_x and t are outputs);
//  kCodes    x_q is the input: the setup computes t = W_B x_q itself (t an optional
//            output).
// Outputs of the setup are written by the first group of each problem; every group
// computes them alike.
enum : int { kGivenT = 0, kQuantize = 1, kCodes = 2 };

// Operands of the kQuantize and kCodes setups.
struct FusedIO {
    const float* x;     // fp32 [M][K] (kQuantize)
    const int8_t* w_b;  // int8 [16][K] (rank 16) or unused
    int8_t* x_q;        // int8 [M][K]  (out, kQuantize)
    float* s_x;         // fp32 [M]     (out, kQuantize)
    int32_t* t;         // int32 [M][16] (out, rank 16; may be NULL with kCodes)
};

// Rows one workgroup owns at most (their epilogue operands live in LDS): 2048 for the
// 8-wave, 4-tile-stage shape that large batches run (one group per 2048-row problem),
// 1088 (17 stages of 64 rows) otherwise, which keeps four 4-wave groups resident per CU
// and splits a 8512-row problem into 8 groups (two resident rounds over 256 problems).
// A multiple of 64: the row loads fill whole 64-row slots.
constexpr int gemv_rows_cap(int W, int T) { return (W >= 8 && T >= 4) ? 2048 : 1088; }

// One lane group = 16 lanes; one chunk = 16 packed bytes = 128 k of one row.
// W waves split K; C chunks per lane; T row tiles (16 rows each) per stage.
// kSetup: kQuantize needs the 16-byte path, one chunk per lane, M <= 4 and
// M K <= 1024 W; kCodes and kGivenT take any decode shape.
template <int W, int C, int T, bool kFast, int kSetup>
// One chunk per lane with 8 waves, or with 4 (except the fused 4-tile shape, which
// needs more): held to 128 registers per lane, so that four waves share each SIMD (two
// 8-wave groups, or four 4-wave groups, per CU); wider variants take what they need.
__global__ __launch_bounds__(W * kWave)
__attribute__((amdgpu_waves_per_eu(C == 1 && (W == 8 || (W == 4 && (T == 1 || kSetup != kQuantize))) ? 4 : 1))) void gemv_kernel(
    const int8_t* __restrict__ x_q, const float* __restrict__ s_x, int M, int64_t N, int64_t K,
    const uint8_t* __restrict__ w_bits, const float* __restrict__ s_w,
    const int8_t* __restrict__ w_a, const float* __restrict__ s_a, const float* __restrict__ s_b,
    const int32_t* __restrict__ t, int rank, float* __restrict__ y, int32_t* __restrict__ acc_dbg,
    int64_t num_tiles, FusedIO fio) {
    constexpr bool kFused = kSetup == kQuantize;
    static_assert(!kFused || (kFast && C == 1), "the fused setup needs whole 128-k chunks, one per lane");
    constexpr int kSubThreads = W * kWave;
    const int tid = (int)threadIdx.x;
    // Workgroups go to the 8 XCDs round-robin by linear id.  With 4 or more groups per
    // problem and a batch that is a multiple of 8, a problem's groups are placed on one
    // XCD (group g of problem p at linear id 8 (gx (p / 8) + g) + p % 8), so that the
    // setup data they all read (tokens, W_B, t) comes into one L2: 48 out_proj problems
    // of 5 groups 22.2 -> 20.6 us in one launch.  With 2 groups per problem the same
    // placement measured slower (96 problems 35.1 -> 37.0 us), so fewer keep the identity.
    int64_t prob = blockIdx.y, grp = blockIdx.x;
    if (gridDim.x >= 4 && gridDim.y % 8 == 0) {  // uniform
        const int64_t lin = (int64_t)blockIdx.y * gridDim.x + blockIdx.x, slot = lin / 8;
        prob = (slot / gridDim.x) * 8 + lin % 8;
        grp = slot % gridDim.x;
    }
    // epilogue: thread -> one row of the stage (its W_A row, s_A, s_w are loaded once per
    // stage) and E of that row's tokens
    static_assert((W * kWave) % (T * 16) == 0, "a stage's rows must divide the group size");
    constexpr int E = (T * 16 * 16 + W * kWave - 1) / (W * kWave);
    constexpr int kTokStride = W * kWave / (T * 16);

    // per-row epilogue operands of every row this group owns, staged once at setup
    constexpr int kRowsCap = gemv_rows_cap(W, T);
    __shared__ uint4 wa_lds[kRowsCap];
    __shared__ float sa_lds[kRowsCap];
    __shared__ float sw_lds[kRowsCap];
    // the stage's scaffold sums, added into by every wave (exact integer adds commute),
    // double-buffered by stage parity so one barrier per stage suffices.  Row stride 20
    // words keeps the adds of one instruction (rows 4g+v, tokens i) on distinct banks.
    __shared__ int32_t red[2][T * 16][20];
    __shared__ int32_t xs_part[W][kWave];
    __shared__ int32_t xsum[16];
    // u[tok][r] = s_B[r] t[tok][r], flat, plus one slot that absorbs the writes of
    // threads past the 16 x 16 tile (a branch-free write keeps the compiler from sinking
    // the t and s_B loads into a branch, where their use would wait for every load)
    __shared__ float u[16 * kRank + 1];
    __shared__ float sxs[17];  // slot 16 takes the discarded writes of lanes past 16
    // fused setup only: the tokens' codes, per-wave absmax partials, the t tile
    constexpr int kFusedMK = 1024 * W;  // largest M K the fused setup takes
    __shared__ __align__(16) uint32_t codes_lds[kFused ? kFusedMK / 4 : 1];
    __shared__ float amax_part[kFused ? W : 1][4];
    __shared__ int32_t tsum[kSetup != kGivenT ? 16 : 1][kRank];

    // problem `prob` of a dense batch (every operand advanced by its own size)
    {
        const int64_t p = prob;
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

    // Issue priority.  A SIMD issues from its highest-priority wave first, then the
    // oldest, so of two groups sharing a CU the younger one falls behind from its setup
    // on and ends its stream alone.  The setup runs at the top priority, and in the
    // stream a group's priority steps down with each quarter of its stages, so the group
    // that lags issues first until the two are level.
    __builtin_amdgcn_s_setprio(3);
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int i = lane & 15;
    const int g = lane >> 4;
    const int64_t RB = K / 8;
    const int64_t num_stages = (num_tiles + T - 1) / T;
    // the problem's stages split evenly over its gridDim.x groups (counts differ by one at
    // most; the host keeps every group within its rows cap and at least one stage)
    const int64_t st_begin = grp * num_stages / gridDim.x;
    const int64_t st_end = (grp + 1) * num_stages / gridDim.x;

    // packed-sign loads of one stage: T tiles x C chunks, 16 bytes per lane.  The fast
    // path loads through a buffer resource over this problem's signs: offsets advance
    // by a constant per stage, rows past N read zero from the range check, and the
    // values are never masked or used early, so prefetched stages stay in flight.
    // Chunks past K (lane groups with no chunk) read a valid chunk of the row and meet
    // all-zero activations.
    const __amdgpu_buffer_rsrc_t w_rsrc = make_rsrc(w_bits, (uint32_t)(N * RB));
    int lane_off[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int64_t q = ((int64_t)c * W + wave) * 4 + g;
        lane_off[c] = (int)((int64_t)i * RB + (16 * q < RB ? 16 * q : 0));
    }
    const int stage_bytes = (int)(T * 16 * RB);
    auto load_stage = [&](int64_t st, uint4 (&wv)[T][C]) __attribute__((always_inline)) {
#pragma unroll
        for (int tt = 0; tt < T; ++tt) {
            if constexpr (kFast) {
                const int base = (int)(st * stage_bytes) + (int)(tt * 16 * RB);
#pragma unroll
                for (int c = 0; c < C; ++c) {
                    const v4i v = __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, base + lane_off[c], 0, 0);
                    wv[tt][c] = make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
                }
            } else {
                const int64_t n = (st * T + tt) * 16 + i;
                const uint8_t* row = w_bits + (n < N ? n : N - 1) * RB;
#pragma unroll
                for (int c = 0; c < C; ++c) {
                    const int64_t q = ((int64_t)c * W + wave) * 4 + g;
                    wv[tt][c] = (n < N) ? load16_guarded<false>(row, 16 * q, RB) : make_uint4(0u, 0u, 0u, 0u);
                }
            }
        }
    };

    // Stages hold packed signs only; they are prefetched two ahead into three named
    // buffers that rotate by name, never by copy (a copy of an in-flight register
    // would wait for its load).  The first two are in flight during the setup.
    struct Stage {
        uint4 w[T][C];
    };
    auto prefetch = [&](int64_t st, Stage& b) __attribute__((always_inline)) { load_stage(st, b.w); };
    Stage s0, s1, s2;
    auto prefetch_first_stages = [&]() __attribute__((always_inline)) {
        prefetch(st_begin, s0);  // every group has at least one stage
        prefetch(st_begin + 1 < st_end ? st_begin + 1 : st_end - 1, s1);
    };

    // The group's rows: W_A row, s_A and s_w go straight into LDS -- buffer loads with an
    // LDS destination, so they hold no registers and nothing waits for them until the
    // first stage's epilogue.  They are issued ahead of the first stages' signs: loads
    // complete in issue order, so a wave that has its first stage's signs has its rows
    // in LDS too, and that stage's barrier makes every wave's rows visible.  Lane l of a
    // wave's load lands at the wave's LDS address + l times the size; slots past the
    // group's rows (short of the next multiple of 64, inside the arrays) take clamped
    // rows.  Rank 0 gives the LoRA operands an empty range: they read zero.
    const int64_t row0 = st_begin * T * 16;
    const int nrows = (int)((st_end - st_begin) * T * 16);
    const __amdgpu_buffer_rsrc_t sw_rsrc = make_rsrc(s_w, (uint32_t)(N * 4));
    const __amdgpu_buffer_rsrc_t wa_rsrc = make_rsrc(w_a, rank != 0 ? (uint32_t)(N * kRank) : 0u);
    const __amdgpu_buffer_rsrc_t sa_rsrc = make_rsrc(s_a, rank != 0 ? (uint32_t)(N * 4) : 0u);
    auto issue_rows = [&]() __attribute__((always_inline)) {
        const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
        for (int rw = wv * kWave; rw < nrows; rw += kSubThreads) {  // uniform per wave
            const int64_t n = row0 + rw + lane;
            const int nc = (int)(n < N ? n : N - 1);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wa_rsrc, (__attribute__((address_space(3))) void*)&wa_lds[rw],
                                                     16, kRank * nc, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(sw_rsrc, (__attribute__((address_space(3))) void*)&sw_lds[rw],
                                                     4, 4 * nc, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(sa_rsrc, (__attribute__((address_space(3))) void*)&sa_lds[rw],
                                                     4, 4 * nc, 0, 0, 0);
        }
    };

    constexpr int U = (16 * kRank + W * kWave - 1) / (W * kWave);
    v4i X[C][8];
    if constexpr (kFused) {
        // ---- fused setup: quantize the tokens (every group alike), build the
        // plane-ordered activations from the codes, and t = W_B x_q as one more 16-row
        // MFMA tile whose rows are W_B's ranks.
        constexpr int NT = W * kWave;
        constexpr int kXV = kFusedMK / 4 / NT;  // float4 of the rows per thread (4)
        const int64_t p = prob;
        const bool writer = grp == 0;
        const int64_t MK4 = (int64_t)M * K / 4;
        for (int e = tid; e < 16 * kRank; e += NT) (&tsum[0][0])[e] = 0;
        for (int e = tid; e < 2 * T * 16 * 20; e += NT) (&red[0][0][0])[e] = 0;

        // loads: the rows (float4 f = e NT + tid of the dense [M][K] block), this lane's
        // 128-k chunk of W_B row i as eight 16-byte pieces, and s_B
        const __amdgpu_buffer_rsrc_t x_rsrc = make_rsrc(fio.x + p * M * K, (uint32_t)(M * K * 4));
        float4 xv[kXV];
#pragma unroll
        for (int e = 0; e < kXV; ++e) {
            const v4f v = __builtin_bit_cast(
                v4f, __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, (e * NT + tid) * 16, 0, 0));
            xv[e] = make_float4(v[0], v[1], v[2], v[3]);
        }
        const int qch = wave * 4 + g;            // this lane's chunk (C == 1)
        const bool chunk_live = 128 * qch < K;   // K % 128 == 0: whole chunks only
        const __amdgpu_buffer_rsrc_t wb_rsrc =
            make_rsrc(rank != 0 ? fio.w_b + p * kRank * K : fio.w_b, rank != 0 ? (uint32_t)(kRank * K) : 0u);
        // W_B for t: the contraction's k order is free (the codes are read from LDS in
        // the same order), so piece e of lane group g is bytes 512 wave + 64 e + 16 g of
        // row i -- each instruction reads 64 contiguous bytes of every row, not sixteen
        // scattered pieces per 128-byte line; pieces past K read zero
        auto t_k = [&](int e) __attribute__((always_inline)) { return 512 * wave + 64 * e + 16 * g; };
        v4i wbv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            wbv[e] = __builtin_amdgcn_raw_buffer_load_b128(
                wb_rsrc, t_k(e) < K ? (int)(i * K + t_k(e)) : kOffDead - 64, 0, 0);
        const __amdgpu_buffer_rsrc_t sb_rsrc = make_rsrc(s_b, rank != 0 ? (uint32_t)(kRank * 4) : 0u);
        float sbv[U];
#pragma unroll
        for (int q = 0; q < U; ++q) {
            const int e = tid + q * NT;
            sbv[q] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(sb_rsrc, 4 * (e % kRank), 0, 0));
        }
        issue_rows();
        prefetch_first_stages();
        // every load above is issued before any of the work below waits on one
        __builtin_amdgcn_sched_barrier(0);

        // per-token absmax: per thread, per wave, then across waves through LDS.  The
        // token of float4 f is (4 f) / K, found by comparisons (M <= 4); past the rows
        // the values are zero, so any token will do.
        const int K32 = (int)K;
        auto token_of = [&](int e) __attribute__((always_inline)) {
            const int k4 = 4 * (e * NT + tid);
            return (k4 >= K32 ? 1 : 0) + (k4 >= 2 * K32 ? 1 : 0) + (k4 >= 3 * K32 ? 1 : 0);
        };
        float am[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int e = 0; e < kXV; ++e) {
            const int m = token_of(e);
            const float a = absmax4(xv[e]);
#pragma unroll
            for (int mm = 0; mm < 4; ++mm)
                if (m == mm) am[mm] = fmaxf(am[mm], a);
        }
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) {
            if (mm < M) {
                const float w = wave_max(am[mm]);
                if (lane == 0) amax_part[wave][mm] = w;
            }
        }
        setup_barrier();
        float sc[4] = {0.0f, 0.0f, 0.0f, 0.0f}, inv[4] = {0.0f, 0.0f, 0.0f, 0.0f}, amx[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        bool fast[4] = {false, false, false, false};
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) {
            if (mm < M) {  // uniform: two IEEE divisions per live token only
                float a = 0.0f;
                for (int w = 0; w < W; ++w) a = fmaxf(a, amax_part[w][mm]);
                const RowScale rs = row_scale(a);
                amx[mm] = a;
                sc[mm] = a == 0.0f ? 0.0f : rs.s;
                inv[mm] = rs.inv;
                fast[mm] = rs.fast;
            }
        }

        // codes into LDS (and x_q, s_x from the problem's first group)
        const __amdgpu_buffer_rsrc_t xq_rsrc = make_rsrc(fio.x_q + p * M * K, writer ? (uint32_t)(M * K) : 0u);
#pragma unroll
        for (int e = 0; e < kXV; ++e) {
            const int f = e * NT + tid;
            const int m = token_of(e);
            float a = amx[0], s = sc[0], iv = inv[0];
            bool fs = fast[0];
#pragma unroll
            for (int mm = 1; mm < 4; ++mm)
                if (m == mm) { a = amx[mm]; s = sc[mm]; iv = inv[mm]; fs = fast[mm]; }
            uint32_t n4 = 0;
            uint32_t q = a == 0.0f ? 0u : fast_code4(xv[e], iv, n4);
            // rare: a code within reach of a rounding tie is redone with the IEEE quotient
            if (a != 0.0f && (!fs || n4)) q = exact_code4(xv[e], s);
            if (f < MK4) codes_lds[f] = q;
            __builtin_amdgcn_raw_buffer_store_b32(q, xq_rsrc, f < MK4 ? 4 * f : kOffDead, 0, 0);
        }
        if (tid < 16) {
            float s = 0.0f;
#pragma unroll
            for (int mm = 0; mm < 4; ++mm)
                if (tid == mm && mm < M) s = sc[mm];
            sxs[tid] = s;
            if (writer && tid < M) fio.s_x[p * M + tid] = s;
        }
        setup_barrier();

        // token i's codes: t's pieces (in W_B's order above), and this lane's chunk two
        // 16-byte pieces at a time for the scaffold operand (bit-plane order)
        const uint8_t* crow = reinterpret_cast<const uint8_t*>(codes_lds) + (i < M ? i * K : 0);
        const bool xlive = i < M && chunk_live;
        int32_t xpart = 0;
        v4i acc_t = {0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint4 v = (i < M && t_k(e) < K) ? *reinterpret_cast<const uint4*>(crow + t_k(e))
                                                  : make_uint4(0u, 0u, 0u, 0u);
            const v4i bv = {(int)v.x, (int)v.y, (int)v.z, (int)v.w};
            acc_t = __builtin_amdgcn_mfma_i32_16x16x64_i8(wbv[e], bv, acc_t, 0, 0, 0);
        }
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            uint32_t nat[8];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int e = 2 * qq + h;
                const uint4 v = xlive ? *reinterpret_cast<const uint4*>(crow + 128 * qch + 16 * e)
                                      : make_uint4(0u, 0u, 0u, 0u);
                nat[4 * h + 0] = v.x;
                nat[4 * h + 1] = v.y;
                nat[4 * h + 2] = v.z;
                nat[4 * h + 3] = v.w;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) xpart = byte_sum(nat[e], xpart);
#pragma unroll
            for (int jh = 0; jh < 2; ++jh) {
                uint32_t o0, o1, o2, o3;
                transpose4x4(nat[0 + jh], nat[2 + jh], nat[4 + jh], nat[6 + jh], o0, o1, o2, o3);
                X[0][4 * jh + 0][qq] = (int)o0;
                X[0][4 * jh + 1][qq] = (int)o1;
                X[0][4 * jh + 2][qq] = (int)o2;
                X[0][4 * jh + 3][qq] = (int)o3;
            }
        }
        // D[4g + v][i] = t[token i][rank 4g + v]: the waves' partial sums meet in LDS
        if (i < M) {
#pragma unroll
            for (int v = 0; v < 4; ++v) atomicAdd(&tsum[i][4 * g + v], acc_t[v]);
        }
        xs_part[wave][lane] = xpart;
        setup_barrier();
#pragma unroll
        for (int q = 0; q < U; ++q) {
            const int e = tid + q * NT;
            if (e < 16 * kRank) {
                const int tok = e / kRank, r = e % kRank;
                const int32_t tt = tsum[tok][r];
                u[tok * kRank + r] = tok < M ? sbv[q] * (float)tt : 0.0f;
                if (writer && rank != 0 && tok < M) fio.t[(p * M + tok) * kRank + r] = tt;
            }
        }
        if (tid < 16) {
            int32_t s = 0;
            for (int w = 0; w < W; ++w)
                for (int gg = 0; gg < 4; ++gg) s += xs_part[w][16 * gg + tid];
            xsum[tid] = s;
        }
        // (u and xsum are read after the first stage's barrier below)
    } else {
        // kCodes: t = W_B x_q is summed into LDS by every wave; zero it first
        if constexpr (kSetup == kCodes) {
            for (int e = tid; e < 16 * kRank; e += W * kWave) (&tsum[0][0])[e] = 0;
            setup_barrier();
        }
        // token scales and the LoRA down-projection: loaded now, stored to LDS after the
        // activation loads below have been issued too
        // (buffer loads: t past M tokens and every LoRA operand at rank 0 read zero)
        const __amdgpu_buffer_rsrc_t t_rsrc =
            make_rsrc(t, (kSetup == kGivenT && rank != 0) ? (uint32_t)(M * kRank * 4) : 0u);
        const __amdgpu_buffer_rsrc_t sb_rsrc = make_rsrc(s_b, rank != 0 ? (uint32_t)(kRank * 4) : 0u);
        float tv[U], sbv[U];
#pragma unroll
        for (int q = 0; q < U; ++q) {
            const int e = tid + q * W * kWave;
            const int tok = e / kRank, r = e % kRank;
            const bool live = e < 16 * kRank;  // tokens past M fall past t's range
            tv[q] = kSetup == kGivenT ? (float)(int32_t)__builtin_amdgcn_raw_buffer_load_b32(
                                            t_rsrc, live ? 4 * (tok * kRank + r) : kOffDead, 0, 0)
                                      : 0.0f;
            sbv[q] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(sb_rsrc, 4 * r, 0, 0));
        }
        // token scales past M read zero (buffer range of M floats)
        const float sxv = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            make_rsrc(s_x, (uint32_t)(M * 4)), 4 * (tid < 16 ? tid : 16), 0, 0));

        // Activations of token i in bit-plane order, for this lane's chunks.  With one
        // chunk per lane its loads go out ahead of the first row's epilogue operands and
        // the stage prefetches (32 registers); wider rows issue those first.
        int32_t xpart = 0;
        const uint8_t* xrow = reinterpret_cast<const uint8_t*>(x_q) + (i < M ? (int64_t)i * K : 0);
        const int64_t xlimit = i < M ? K : 0;
        // One resource over all M rows (uniform, so it stays in scalar registers); lanes of
        // tokens past M fall past its range and read zero, and so do chunks past the row's
        // end (a far offset: they would otherwise read the next token's row).  K is a
        // multiple of 128 on the 16-byte path, so a chunk is wholly in or out of the row.
        const __amdgpu_buffer_rsrc_t x_rsrc = make_rsrc(x_q, kFast ? (uint32_t)(M * K) : 0u);
        const int xoff = kFast ? i * (int)K : 0;
        // kCodes: W_B row i (rank i) over the same k as token i's codes, the A operand of
        // the t MFMAs (B = the codes in natural order): D[4g + v][i] = t[token i][rank 4g + v]
        const int8_t* wb_p = kSetup == kCodes ? fio.w_b + prob * kRank * K : x_q;
        const __amdgpu_buffer_rsrc_t wb_rsrc =
            make_rsrc(wb_p, (kSetup == kCodes && kFast) ? (uint32_t)(kRank * K) : 0u);
        const uint8_t* wbrow = reinterpret_cast<const uint8_t*>(wb_p) + (int64_t)i * K;
        v4i acc_t = {0, 0, 0, 0};
        if constexpr (kSetup == kCodes && !kFast) {
            // byte-gathering path (ragged K or unaligned rows): t in a pass of its own over
            // this lane's chunks, so its registers are not held beside the activations'
#pragma unroll 1
            for (int c = 0; c < C; ++c) {
                const int64_t kb = 128 * (((int64_t)c * W + wave) * 4 + g);
#pragma unroll 1
                for (int e = 0; e < 8; ++e) {
                    const uint4 av = load16_guarded<false>(wbrow, kb + 16 * e, K);
                    const uint4 bv = load16_guarded<false>(xrow, kb + 16 * e, xlimit);
                    acc_t = __builtin_amdgcn_mfma_i32_16x16x64_i8((v4i){(int)av.x, (int)av.y, (int)av.z, (int)av.w},
                                                                  (v4i){(int)bv.x, (int)bv.y, (int)bv.z, (int)bv.w},
                                                                  acc_t, 0, 0, 0);
                }
            }
        }
        if constexpr (C > 1) {
            issue_rows();
            prefetch_first_stages();
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int64_t q = ((int64_t)c * W + wave) * 4 + g;
            const int64_t kb = 128 * q;
            const int xb = kb < K ? xoff + (int)kb : 0x40000000;
            uint32_t nat[32];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                uint4 v;
                if constexpr (kFast) {
                    const v4i b = __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, xb + 16 * e, 0, 0);
                    v = make_uint4((uint32_t)b[0], (uint32_t)b[1], (uint32_t)b[2], (uint32_t)b[3]);
                } else {
                    v = load16_guarded<false>(xrow, kb + 16 * e, xlimit);
                }
                nat[4 * e + 0] = v.x;
                nat[4 * e + 1] = v.y;
                nat[4 * e + 2] = v.z;
                nat[4 * e + 3] = v.w;
            }
            // (the fast path issues all eight W_B pieces now, beside the activations)
            v4i wbv[(kSetup == kCodes && kFast) ? 8 : 1];
            if constexpr (kSetup == kCodes && kFast) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    wbv[e] = __builtin_amdgcn_raw_buffer_load_b128(
                        wb_rsrc, kb < K ? (int)(i * K + kb + 16 * e) : kOffDead - 64, 0, 0);
            }
            if constexpr (C == 1) {
                __builtin_amdgcn_sched_barrier(0);  // the activation loads go out first
                issue_rows();
                prefetch_first_stages();
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int e = 0; e < 32; ++e) xpart = byte_sum(nat[e], xpart);
            if constexpr (kSetup == kCodes && kFast) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const v4i bv = {(int)nat[4 * e], (int)nat[4 * e + 1], (int)nat[4 * e + 2], (int)nat[4 * e + 3]};
                    acc_t = __builtin_amdgcn_mfma_i32_16x16x64_i8(wbv[e], bv, acc_t, 0, 0, 0);
                }
            }
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
        if constexpr (kSetup == kCodes) {
            // the waves' partial t tiles meet in LDS (token lanes only)
            if (i < M) {
#pragma unroll
                for (int v = 0; v < 4; ++v) atomicAdd(&tsum[i][4 * g + v], acc_t[v]);
            }
        } else {
            // LoRA: u[tok][r] = s_B[r] * t[tok][r] (fp32), shared by every output row.
#pragma unroll
            for (int q = 0; q < U; ++q) {
                const int e = tid + q * W * kWave;
                u[e < 16 * kRank ? e : 16 * kRank] = sbv[q] * tv[q];
            }
        }
        sxs[tid < 16 ? tid : 16] = sxv;
        xs_part[wave][lane] = xpart;
        for (int e = tid; e < 2 * T * 16 * 20; e += W * kWave) (&red[0][0][0])[e] = 0;
        setup_barrier();
        if constexpr (kSetup == kCodes) {
            // u from the summed t; the problem's first group also writes t when asked to
            const bool writer = grp == 0 && fio.t != nullptr && rank != 0;
#pragma unroll
            for (int q = 0; q < U; ++q) {
                const int e = tid + q * W * kWave;
                if (e < 16 * kRank) {
                    const int tok = e / kRank, r = e % kRank;
                    const int32_t tt = tsum[tok][r];
                    u[e] = tok < M ? sbv[q] * (float)tt : 0.0f;
                    if (writer && tok < M) fio.t[(prob * M + tok) * kRank + r] = tt;
                }
            }
        }
        if (tid < 16) {
            int32_t s = 0;
            for (int w = 0; w < W; ++w)
                for (int gg = 0; gg < 4; ++gg) s += xs_part[w][16 * gg + tid];
            xsum[tid] = s;
        }
        // (xsum is read after the first stage's barrier below)
    }

    // The LoRA up-projection of every row the group owns, once, for up to 4 tokens:
    // lora[n][tok] = sum_r W_A[n][r] u[tok][r] -- the fmaf chain the per-element form
    // runs, in the same order -- written over the row's W_A in LDS (16 bytes either
    // way), so that each stage's epilogue reads one value instead of running the
    // 16-term chain (with more tokens the epilogue still runs it).  The barrier makes u
    // and every wave's row operands (their LDS loads waited for by its fence) visible.
    const bool lora_pre = M <= 4;
    if (lora_pre) {
        lds_barrier();
        for (int r = tid; r < nrows; r += kSubThreads) {
            // (u is re-read per row: hoisted out of the loop, 4 x 16 values would stay
            // live across it and push the kernel's registers past its budget)
            asm volatile("" ::: "memory");
            const uint4 wa = wa_lds[r];
            const uint32_t words[4] = {wa.x, wa.y, wa.z, wa.w};
            float l[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int tok = 0; tok < 4; ++tok) {
                if (tok < M) {  // uniform
                    float acc = 0.0f;
#pragma unroll
                    for (int q = 0; q < kRank; ++q) {
                        const float a = (float)(int8_t)(words[q >> 2] >> (8 * (q & 3)));
                        acc = fmaf(a, u[tok * kRank + q], acc);
                    }
                    l[tok] = acc;
                }
            }
            wa_lds[r] = make_uint4(__float_as_uint(l[0]), __float_as_uint(l[1]), __float_as_uint(l[2]),
                                   __float_as_uint(l[3]));
        }
        // (read by the epilogues after the first stage's barrier)
    }

    // Outputs through buffer resources: dead elements store to an out-of-range offset.
    const __amdgpu_buffer_rsrc_t y_rsrc = make_rsrc(y, (uint32_t)(M * N * 4));
    const __amdgpu_buffer_rsrc_t acc_rsrc = make_rsrc(acc_dbg, acc_dbg ? (uint32_t)(M * N * 4) : 0u);

    // One stage: issue the prefetch two ahead into `nxt2` (a clamped stage index past
    // the group's range re-reads its last stage, so the load is unconditional), then
    // consume `cur`.  Branches below hold no global loads -- only LDS traffic, ALU work
    // and buffer stores -- so the compiler's waits stay partial across them and the
    // prefetched stages remain in flight.
    auto run_stage = [&](int64_t st, Stage& cur, Stage& nxt2, int rb) __attribute__((always_inline)) {
        prefetch(st + 2 < st_end ? st + 2 : st_end - 1, nxt2);
        if (st >= st_end) return;  // uniform: stage past the group's range

        const int32_t one = opaque_one();
#pragma unroll
        for (int tt = 0; tt < T; ++tt) {
            // planes j and j+4 share accumulator j (weight bytes 2^j * bit):
            // low planes from w, high planes from w >> 4 under the same masks
            v4i acc[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = (v4i){0, 0, 0, 0};
#pragma unroll
            for (int c = 0; c < C; ++c) {
                const uint4 lo = cur.w[tt][c];
                const uint4 hi = make_uint4(lo.x >> 4, lo.y >> 4, lo.z >> 4, lo.w >> 4);
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const uint4 wv = half ? hi : lo;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t msk = 0x01010101u << j;
                        const v4i a = {(int)(wv.x & msk), (int)(wv.y & msk), (int)(wv.z & msk), (int)(wv.w & msk)};
                        acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, X[c][j + 4 * half], acc[j], 0, 0, 0);
                    }
                }
            }
            // D[4g + v][i]: row 4g+v of tile tt, token i; sum_j acc_j / 2^j, exactly.
            // Only token lanes (i < M) add; the branch holds no global load.
            if (i < M) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    // Horner form, three v_lshl_add_u32 per value: 8 acc0 + 4 acc1 + 2 acc2 + acc3
                    const int32_t s8b = (((((acc[0][v] << one) + acc[1][v]) << one) + acc[2][v]) << one) + acc[3][v];
                    atomicAdd(&red[rb][tt * 16 + 4 * g + v][i], s8b >> 3);
                }
            }
        }
        lds_barrier();
        // Epilogue element (row erow of the stage, tokens etok0 + q kTokStride): the
        // thread-to-element map rotates by one wave per stage, so with few tokens the
        // waves (and SIMDs) that carry the epilogue change from stage to stage.
        const int rtid = (int)((tid + (st % W) * kWave) % (W * kWave));
        const int erow = rtid % (T * 16), etok0 = rtid / (T * 16);
        const int64_t n = st * T * 16 + erow;
        const int lrow = (int)(n - row0);
        const uint4 wa = wa_lds[lrow];
        const float sa = sa_lds[lrow], sw = sw_lds[lrow];
        const uint32_t words[4] = {wa.x, wa.y, wa.z, wa.w};
#pragma unroll
        for (int q = 0; q < E; ++q) {
            const int tok = etok0 + q * kTokStride;  // uniform per wave when a stage is 64 rows
            if (tok < M) {
                const int32_t s1 = red[rb][erow][tok];
                red[rb][erow][tok] = 0;  // ready for the stage after next
                const int32_t acc_pm = 2 * s1 - xsum[tok];
                // LoRA up (u and W_A are zero at rank 0, leaving the scaffold term exact):
                // precomputed per row for up to 4 tokens, else the chain here
                float lora = 0.0f;
                if (lora_pre) {
                    lora = __uint_as_float(words[tok & 3]);
                } else {
#pragma unroll
                    for (int r = 0; r < kRank; ++r) {
                        const float a = (float)(int8_t)(words[r >> 2] >> (8 * (r & 3)));
                        lora = fmaf(a, u[tok * kRank + r], lora);
                    }
                }
                const float inner = fmaf(sa, lora, sw * (float)acc_pm);
                const int off = n < N ? (int)(((int64_t)tok * N + n) * 4) : kOffDead;
                store_i32(acc_pm, acc_rsrc, off);
                if (lora_pre) {
                    // y waits in the row's slot, in place of the LoRA value just read
                    // (each slot word is one element's), until the group's last stage
                    reinterpret_cast<float*>(&wa_lds[lrow])[tok & 3] = sxs[tok] * inner;
                } else {
                    store_f32(sxs[tok] * inner, y_rsrc, off);
                }
            }
        }
        // No second barrier: the next stage adds into the other buffer, and this one is
        // added into again only after the next stage's barrier, which every wave reaches
        // after finishing this epilogue.
    };

    // three stages per trip so the register buffers rotate by name
    for (int64_t st = st_begin; st < st_end; st += 3) {
        {
            const int64_t done4 = 4 * (st - st_begin), n = st_end - st_begin;  // uniform
            if (done4 < n) __builtin_amdgcn_s_setprio(3);
            else if (done4 < 2 * n) __builtin_amdgcn_s_setprio(2);
            else if (done4 < 3 * n) __builtin_amdgcn_s_setprio(1);
            else __builtin_amdgcn_s_setprio(0);
        }
        const int rb = (int)((st - st_begin) & 1);
        run_stage(st, s0, s2, rb);
        run_stage(st + 1, s1, s0, rb ^ 1);
        run_stage(st + 2, s2, s1, rb);
    }
    // y of the group's rows, held in LDS by the epilogues, leaves in one pass:
    // interleaved with the packed-sign stream, the small scattered stores cost the
    // stream far more than their bytes (the HBM turns between reads and writes)
    if (lora_pre) {
        lds_barrier();
        for (int tok = 0; tok < M; ++tok) {  // uniform
            for (int r = tid; r < nrows; r += kSubThreads) {
                const int64_t n = row0 + r;
                store_f32(reinterpret_cast<const float*>(&wa_lds[r])[tok], y_rsrc,
                          n < N ? (int)(((int64_t)tok * N + n) * 4) : kOffDead);
            }
        }
    }
}

// Groups of one kernel instance that the GPU holds at once: the per-CU occupancy its
// registers and LDS allow, times the CU count.  Taken once per instance.
template <typename Kernel>
static int64_t resident_groups(Kernel kernel, int threads) {
    int per_cu = 0, dev = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess || per_cu < 1)
        per_cu = 1;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        cus = 256;
    return (int64_t)per_cu * cus;
}

template <int W, int C, int T, bool kFast, int kSetup>
static int64_t gemv_resident() {
    static const int64_t n = resident_groups(gemv_kernel<W, C, T, kFast, kSetup>, W * kWave);
    return n;
}

template <int W, int C, int T>
static hipError_t launch_gemv_wct(bool fast, int setup, const int8_t* x_q, const float* s_x, int M, int64_t N,
                                  int64_t K, const uint8_t* w_bits, const float* s_w, const int8_t* w_a,
                                  const float* s_a, const float* s_b, const int32_t* t, int rank, float* y,
                                  int32_t* acc_dbg, int64_t batch, const FusedIO& fio, hipStream_t stream) {
    const int64_t num_tiles = (N + 15) / 16;
    const int64_t num_stages = (num_tiles + T - 1) / T;
    // Large batches: one resident round of groups, each over as many rows as it can
    // hold, so the setup is paid once per group and no second round trails.  Otherwise
    // ~8 groups per CU, or ~1 per CU for the setups that compute t, whose every group
    // reads all of W_B (and, in the one-call form, quantizes the tokens).
    int64_t resident_wgs;
    if (setup == kQuantize) {
        if constexpr (C == 1) {
            resident_wgs = gemv_resident<W, C, T, true, kQuantize>();
        } else {
            return hipErrorNotSupported;
        }
    } else if (setup == kCodes) {
        resident_wgs = fast ? gemv_resident<W, C, T, true, kCodes>() : gemv_resident<W, C, T, false, kCodes>();
    } else {
        resident_wgs = fast ? gemv_resident<W, C, T, true, kGivenT>() : gemv_resident<W, C, T, false, kGivenT>();
    }
    const bool throughput = batch * num_stages >= 4 * resident_wgs;
    constexpr int kRowsCap = gemv_rows_cap(W, T);
    constexpr int64_t kMaxStages = kRowsCap / (T * 16);
    // Groups per problem round down, so a launch never spills a few groups into a
    // partial second round, nor puts a second group on a few CUs while the rest hold one
    // (batch 48: in_proj 1056 groups for 1024 resident, out_proj one-call 288 groups on
    // 256 CUs, when rounded up).
    int64_t per_problem;
    if (throughput) {
        // whole resident rounds: as few as the rows cap allows, their groups spread
        // evenly over the problems (and a problem's stages evenly over its groups)
        const int64_t rounds = (batch * num_stages + resident_wgs * kMaxStages - 1) / (resident_wgs * kMaxStages);
        per_problem = (rounds * resident_wgs) / batch;
    } else {
        // t given: ~8 groups per CU for one problem, ~2 per CU over a batch (at 2048 a
        // batch of 48 out_proj problems got single-stage groups, whose loads never
        // pipeline: 38.9 against 24.8 us; batch 8 in_proj 20.5 against 15.2 us)
        const int64_t target_wgs = setup != kGivenT ? 256 : (batch > 1 ? 512 : 2048);
        per_problem = target_wgs / batch;
    }
    if (per_problem < 1) per_problem = 1;
    const int64_t min_groups = (num_stages + kMaxStages - 1) / kMaxStages;  // the rows cap
    if (per_problem < min_groups) per_problem = min_groups;
    if (per_problem > num_stages) per_problem = num_stages;
    const dim3 grid((unsigned)per_problem, (unsigned)batch);
    // In the throughput regime the one-call form pays off only with one group per
    // problem: every further group would quantize the tokens and read W_B again.
    if (setup == kQuantize && throughput && grid.x > 1) return hipErrorNotSupported;
#define DFSSM_GEMV_LAUNCH(FAST, SETUP)                                                                        \
    gemv_kernel<W, C, T, FAST, SETUP><<<grid, W * kWave, 0, stream>>>(x_q, s_x, M, N, K, w_bits, s_w, w_a, s_a, \
                                                                      s_b, t, rank, y, acc_dbg, num_tiles, fio)
    if (setup == kQuantize) {
        if constexpr (C == 1) DFSSM_GEMV_LAUNCH(true, kQuantize);
    } else if (setup == kCodes) {
        if (fast) {
            DFSSM_GEMV_LAUNCH(true, kCodes);
        } else {
            DFSSM_GEMV_LAUNCH(false, kCodes);
        }
    } else if (fast) {
        DFSSM_GEMV_LAUNCH(true, kGivenT);
    } else {
        DFSSM_GEMV_LAUNCH(false, kGivenT);
    }
#undef DFSSM_GEMV_LAUNCH
    return hipGetLastError();
}

template <int W, int C>
static hipError_t launch_gemv_wc(bool fast, int setup, const int8_t* x_q, const float* s_x, int M, int64_t N,
                                 int64_t K, const uint8_t* w_bits, const float* s_w, const int8_t* w_a,
                                 const float* s_a, const float* s_b, const int32_t* t, int rank, float* y,
                                 int32_t* acc_dbg, int64_t batch, const FusedIO& fio, hipStream_t stream) {
    // Few tiles overall (one decode call): one tile per stage spreads the rows over
    // the most CUs.  Many tiles (batched calls): four tiles per stage keep more
    // packed-sign loads in flight per wave.
    constexpr int kTBig = (W >= 4 && C <= 2) ? 4 : 1;
    const int64_t total_tiles = batch * ((N + 15) / 16);
    if (total_tiles <= 4096)
        return launch_gemv_wct<W, C, 1>(fast, setup, x_q, s_x, M, N, K, w_bits, s_w, w_a, s_a, s_b, t, rank, y,
                                        acc_dbg, batch, fio, stream);
    return launch_gemv_wct<W, C, kTBig>(fast, setup, x_q, s_x, M, N, K, w_bits, s_w, w_a, s_a, s_b, t, rank, y,
                                        acc_dbg, batch, fio, stream);
}

// Waves per group for rows of NC 16-byte chunks (zero: too long for the decode kernel).
static int gemv_waves(int64_t NC) { return NC <= 4 ? 1 : NC <= 8 ? 2 : NC <= 16 ? 4 : NC <= 128 ? 8 : 0; }

static hipError_t launch_gemv_any(bool fast, int setup, const int8_t* x_q, const float* s_x, int M, int64_t N,
                                  int64_t K, const uint8_t* w_bits, const float* s_w, const int8_t* w_a,
                                  const float* s_a, const float* s_b, const int32_t* t, int rank, float* y,
                                  int32_t* acc_dbg, int64_t batch, const FusedIO& fio, hipStream_t stream) {
    const int64_t NC = (K / 8 + 15) / 16;  // 16-byte chunks per row
#define DFSSM_GEMV(Wv, Cv)                                                                                       \
    return launch_gemv_wc<Wv, Cv>(fast, setup, x_q, s_x, M, N, K, w_bits, s_w, w_a, s_a, s_b, t, rank, y, acc_dbg, \
                                  batch, fio, stream)
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

// The decode kernel with t given (w_b == NULL) or, with rank 16 and w_b given, with
// t = W_B x_q computed by every group (t_out, when not NULL, receives it).
hipError_t launch_gemv(const int8_t* x_q, const float* s_x, int M, int64_t N, int64_t K,
                       const uint8_t* w_bits, const float* s_w, const int8_t* w_a, const float* s_a,
                       const int8_t* w_b, const float* s_b, const int32_t* t, int32_t* t_out, int rank, float* y,
                       int32_t* acc_dbg, int64_t batch, hipStream_t stream) {
    const int64_t RB = K / 8;
    const bool codes = rank != 0 && w_b != nullptr;
    const bool fast = (RB % 16 == 0) && ((uintptr_t)w_bits % 16 == 0) && ((uintptr_t)x_q % 16 == 0) &&
                      (!codes || (uintptr_t)w_b % 16 == 0);
    const FusedIO fio{nullptr, w_b, nullptr, nullptr, t_out};
    return launch_gemv_any(fast, codes ? kCodes : kGivenT, x_q, s_x, M, N, K, w_bits, s_w, w_a, s_a, s_b, t, rank,
                           y, acc_dbg, batch, fio, stream);
}

// Whether one launch can quantize, project down and run the scaffold product: whole
// 128-k chunks, one chunk per lane (K <= 4096), at most 4 tokens, and the tokens'
// codes within the group's LDS (M K <= 1024 x waves per group).
bool decode_fused_supported(int64_t M, int64_t K) {
    if (K % 128 != 0 || K > 4096 || M < 1 || M > 4) return false;
    return M * K <= 1024 * gemv_waves(K / 128);
}

// hipErrorNotSupported (nothing launched) when the shape or the launch plan does not
// suit the fused variant: the caller then takes the two-kernel form.
hipError_t launch_decode_fused(const float* x, int M, int64_t N, int64_t K, const uint8_t* w_bits,
                               const float* s_w, const int8_t* w_a, const float* s_a, const int8_t* w_b,
                               const float* s_b, int rank, int8_t* x_q, float* s_x, int32_t* t, float* y,
                               int32_t* acc_dbg, int64_t batch, hipStream_t stream) {
    if (!decode_fused_supported(M, K) || (uintptr_t)w_bits % 16 != 0 || (uintptr_t)x % 16 != 0)
        return hipErrorNotSupported;
    const FusedIO fio{x, w_b, x_q, s_x, t};
    return launch_gemv_any(true, kQuantize, x_q, s_x, M, N, K, w_bits, s_w, w_a, s_a, s_b, t, rank, y, acc_dbg,
                           batch, fio, stream);
}

}  // namespace dfssm
