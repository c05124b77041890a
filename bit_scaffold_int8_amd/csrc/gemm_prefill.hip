// gemm_prefill.hip -- prefill-shaped scaffold + LoRA projection on the int8 MFMA pipe (gfx950).
//
// DF-SSM technical summary (gist.science), section 2C: packed 1-bit scaffold
// weights are expanded to int8 on the fly and multiplied with int8 activations on the
// matrix cores; section 2B: the rank-16 int8 LoRA correction W_A (W_B x) with
// per-channel/row scales.  At many tokens the scaffold product is a dense int8
// contraction, so it runs on v_mfma_i32_32x32x32_i8; nothing is materialized in memory.
//
// Work split.  A workgroup is NW = 4 or 8 waves (one or two per SIMD) and owns a
// (32 MB) x (32 NB WNW) output tile: WNW = NW / KS waves side by side along N and KS
// groups along K (split-K inside the workgroup, summed through LDS at the end).  Each
// wave keeps its (32 MB) x (32 NB) partial tile in MB x NB accumulators of 16
// registers (AGPRs).  Some 4-wave configurations run two workgroups per CU, each with
// half the register and LDS budget: the two drift apart, so one's epilogue stores and
// the narrow tail groups overlap the other's MFMA work.
//
// Weights as 0/1.  A sign w = 2 b - 1 with bit b, so sum_k w x = 2 S - R with
// S = sum_k b x (the MFMA product with 0/1 bytes) and R = sum_k x (the token's code
// sum).  0/1 operand bytes switch far fewer bits than 0x01/0xFF, which lets the
// matrix cores run measurably faster under the same power limit, and the expansion
// is one VALU op shorter per word: nibble * 0x00204081 & 0x01010101 spreads four
// sign bits to four bytes.  R is summed by the threads that stage the codes.
//
// Data flow per K group, in 128-k chunks:
//  * A (codes): staged through LDS, 8 threads per 128-byte row segment (whole cache
//    lines), rows padded to 144 bytes so the 16 rows one 16-lane group reads land in
//    distinct banks.  In a chunk, lane group g = lane / 32 takes k in [64 g, 64 g + 64)
//    and MFMA step s its 16 bytes [64 g + 16 s, +16); any per-lane k order is valid as
//    long as A and B agree.  Double-buffered, one barrier per chunk.
//  * B (sign bits, [N][K/8] rows): staged through LDS four chunks at a time, so each
//    column contributes a 64-byte run (4 threads, 16 bytes each) instead of 16 bytes
//    per chunk; rows of the LDS copy are padded to 72 bytes (conflict-free 8-byte
//    reads).  Double-buffered per 4-chunk block, written two chunks before use.
//  * Operands one step ahead: A fragments are read and B operands expanded for step
//    s + 1 while step s's MFMAs run; loads run one to two chunks ahead.
//  * Tails: every global access goes through a buffer resource; rows past M, columns
//    past the tile and chunks past K or past the group's range read zero.
//
// Epilogue.  y = s_x (s_w acc + s_A sum_r W_A[n][r] s_B[r] t[m][r]), stored at device
// scope (written through the L2, so the output drains while tiles still finish).
// The LoRA-up product is a second, tiny contraction (rank 16) and runs on
// v_mfma_f32_32x32x16_bf16: W_A is exact in bf16, and u = s_B t (fp32) is split
// exactly into three bf16 parts (h + m + l, each the truncation of the remainder), so
// the products are exact and only fp32 accumulation rounds.  Its output layout equals the int32 accumulator's,
// so the scale epilogue combines them register by register.
//
// One launch can carry two tile configurations over two column ranges (a main part
// and a narrow tail), so that a width like 8512 = 32 x 256 + 320 takes one round of
// main tiles plus tail groups that run beside them, instead of two full rounds.
#include "device_common.h"

namespace dfssm {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

namespace prefill {
constexpr int kChunk = 128;            // k per main-loop chunk (64 per lane group)
constexpr int kBlk = 4;                // chunks per staged block of sign bits
constexpr int kLdA = kChunk + 16;      // LDS row stride of a code chunk (bytes)
constexpr int kLdB = kBlk * 16 + 8;    // LDS row stride of a column's block of sign bits (bytes)
constexpr int kLoadDead = 0x7ff00000;  // a load offset past every resource used here: reads zero
constexpr int kRedBlocks = 8;          // accumulator blocks per split-K reduction phase
constexpr int kColDead = 0x40000000;   // store offset added for columns past the range: past the y resource

// OCC_ workgroups of the configuration share a CU (its register and LDS budgets are
// split between them).
template <int MB_, int NB_, int KS_, int NW_ = 4, int OCC_ = 1>
struct Cfg {
    static constexpr int MB = MB_, NB = NB_, KS = KS_, NW = NW_, OCC = OCC_;
    static constexpr int WNW = NW / KS;                      // waves along N
    static constexpr int BM = 32 * MB, WN = 32 * NB, BN = WN * WNW;
    static constexpr int GS = kWave * WNW;                   // threads of one K group
    static constexpr int P = BM * 8 / GS;                    // code pieces per thread per chunk
    static constexpr int JB = BN * kBlk / GS;                // sign pieces per thread per block
    // The narrow configurations (at most 2 accumulator blocks per wave) stage W_B with
    // the codes in the instances that compute t; a code chunk buffer then holds BM token
    // rows and after them the chunk's kRank rows of W_B.  (The wider ones lack the
    // registers, or, at 4 blocks, measured slower with the extra LDS traffic.)
    static constexpr bool kStageWb = MB * NB <= 2;
    static constexpr int kABytes = (BM + (kStageWb ? kRank : 0)) * kLdA, kBBytes = BN * kLdB;
    static constexpr int kGroupBytes = 2 * kABytes + 2 * kBBytes;
    static constexpr int RBLK = MB * NB < kRedBlocks ? MB * NB : kRedBlocks;  // blocks per hand-over phase
    static constexpr int kRedBytes = KS > 1 ? WNW * RBLK * KS * 4 * kWave * 16 : 0;
    // int32 [KS][BM] code sums, after both the chunk buffers and the split-K hand-over
    // area that reuses them
    static constexpr int kRowSumOff = KS * kGroupBytes > kRedBytes ? KS * kGroupBytes : kRedBytes;
    static constexpr int kLdsBytes = kRowSumOff + KS * BM * 4;
    static_assert((NW == 4 || NW == 8) && NW * OCC <= 8, "one or two waves per SIMD");
    static_assert(KS == 1 || KS == 2 || KS == 4, "waves split over K and N");
    static_assert(P * GS == BM * 8 && (P % 4 == 0 || 4 % P == 0), "code pieces split evenly over steps");
    static_assert(JB * GS == BN * kBlk, "sign pieces split evenly over threads");
    static_assert(!kStageWb || GS >= 8 * kRank, "a K group has a thread for each W_B piece of a chunk");
    static_assert(kLdsBytes * OCC <= 160 * 1024, "LDS");
};

// One part of a launch: a column range [n_begin, n_end) tiled by one configuration.
struct Seg {
    int tiles_m, tiles_n, n_begin, n_end;
};

struct Args {
    const int8_t* x_q;
    const float* s_x;
    const uint8_t* w_bits;
    const float* s_w;
    const int8_t* w_a;
    const float* s_a;
    const float* s_b;
    const int32_t* t;     // given t (kTin = false)
    const int8_t* w_b;    // W_B (kTin = true: t = W_B x_q computed in the K loop)
    int32_t* t_out;       // kTin: optional copy of t (written by the first column tile)
    float* y;
    int32_t* acc_dbg;
    int M, N, K, rank;
};
}  // namespace prefill

// 4 sign bits -> 4 bytes of 0/1 (bit i -> byte i).
__device__ __forceinline__ uint32_t bits4(uint32_t nib) { return (nib * 0x00204081u) & 0x01010101u; }

// Low 16 bits of w -> a 16-byte B operand of 0/1 (bit i -> byte i).
__device__ __forceinline__ v4i bits16(uint32_t w) {
    return (v4i){(int)bits4(w & 0xFu), (int)bits4((w >> 4) & 0xFu), (int)bits4((w >> 8) & 0xFu),
                 (int)bits4((w >> 12) & 0xFu)};
}

// Exact split of a finite fp32 value into three bf16 values, u = h + m + l: h keeps
// the top 8 significant bits (truncation), the remainder u - h is exact in fp32 and
// holds at most 16 significant bits, m keeps its top 8, and l = (u - h) - m is exact
// and has at most 8 significant bits.  Returned as bf16 bit patterns.
__device__ __forceinline__ void split3_bf16(float u, uint32_t& h, uint32_t& m, uint32_t& l) {
    const uint32_t hb = __float_as_uint(u) & 0xFFFF0000u;
    const float r = u - __uint_as_float(hb);
    const uint32_t mb = __float_as_uint(r) & 0xFFFF0000u;
    const float q = r - __uint_as_float(mb);
    h = hb >> 16;
    m = mb >> 16;
    l = __float_as_uint(q) >> 16;
}

__device__ __forceinline__ v8bf pack_bf16(const uint32_t (&b)[8]) {
    const v4u w = {b[0] | (b[1] << 16), b[2] | (b[3] << 16), b[4] | (b[5] << 16), b[6] | (b[7] << 16)};
    return __builtin_bit_cast(v8bf, w);
}

// One output tile of configuration C over the column range of `seg`.  kTin: the LoRA
// down-projection t = W_B x_q is computed here, from the code chunks already in LDS, on
// v_mfma_i32_16x16x64_i8 (A = 16 token rows, B = the 16 rows of W_B):
// the waves of a K group share the tile's 16-row blocks, and the K groups' partial t
// meet in LDS after the main loop.
template <class C, bool kDebug, bool kTin>
__device__ __forceinline__ void prefill_tile(const prefill::Args& a, uint8_t* __restrict__ lds, int tile,
                                             const prefill::Seg& seg) {
    using namespace prefill;
    constexpr int MB = C::MB, NB = C::NB, KS = C::KS, WNW = C::WNW, BM = C::BM, WN = C::WN, BN = C::BN;
    constexpr int GS = C::GS, P = C::P, JB = C::JB, RBLK = C::RBLK;
    // 16-row blocks of t per wave (every block once per K group)
    constexpr int TB = (BM / 16 + WNW - 1) / WNW;
    static_assert(TB * WNW == BM / 16, "t row blocks split evenly over a K group's waves");
    static_assert(!kTin || KS * BM * kRank * 4 <= C::kABytes * 2, "t hand-over fits the chunk buffers");
    // code piece j is staged in step st_step(j) of a chunk
    auto st_step = [](int j) { return j * 4 / P; };
    const int M = a.M, N = a.N, K = a.K;

    const int tm = tile / seg.tiles_n, tn = tile % seg.tiles_n;
    // wave index made visibly wave-uniform, so the per-wave buffer resources are scalar
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const int lane = threadIdx.x % kWave;
    const int wn = wave % WNW, kq = wave / WNW;
    const int g = lane >> 5, l32 = lane & 31;
    const int tg = wn * kWave + lane;  // thread index within the K group
    const int m0 = tm * BM;
    const int n0g = seg.n_begin + tn * BN;  // first column of the workgroup
    const int n0 = n0g + wn * WN;           // first column of this wave
    const int RB = K / 8;
    // (readfirstlane: the clamps compile to VALU min/max, whose results the resource
    // builder would otherwise treat as per-lane)
    const int rows = __builtin_amdgcn_readfirstlane(min(M - m0, BM));
    const int cols_g = __builtin_amdgcn_readfirstlane(max(0, min(seg.n_end - n0g, BN)));
    const int cols = __builtin_amdgcn_readfirstlane(max(0, min(seg.n_end - n0, WN)));

    const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(a.x_q + (int64_t)m0 * K, (uint32_t)(rows * K));
    const __amdgpu_buffer_rsrc_t b_rsrc =
        make_rsrc(a.w_bits + (int64_t)min(n0g, N) * RB, (uint32_t)(cols_g * RB));

    // every wave runs the same number of chunks (the barriers pair up), a multiple of
    // the sign-bit block; chunks past its K range read zeros
    const int nch = (K + kChunk - 1) / kChunk;
    const int per = ((nch + KS - 1) / KS + kBlk - 1) / kBlk * kBlk;
    const int c_begin = kq * per, c_end = min(nch, c_begin + per);
    const int nblk = per / kBlk;

    uint8_t* const abuf = lds + kq * C::kGroupBytes;  // 2 x kABytes, this K group's
    uint8_t* const bbuf = abuf + 2 * C::kABytes;       // 2 x kBBytes
    int32_t* const rowsum = reinterpret_cast<int32_t*>(lds + C::kRowSumOff);

    // code staging: piece j -> row j GS / 8 + tg / 8, bytes [16 p, +16).  One base
    // offset per lane (piece j adds a uniform j GS / 8 rows): rows past `rows` lie past
    // the end of a_rsrc and read zero, so no per-piece offsets stay live in registers.
    const int p16 = 16 * (tg & 7);
    const int st_gbase = (tg >> 3) * K + p16;
    const int st_lbase = (tg >> 3) * kLdA + p16;
    // sign staging: slot i -> group column (tg / 4) + (GS / 4) i, chunk (tg & 3) of the
    // block (columns past cols_g lie past the end of b_rsrc)
    const int bs_gbase = (tg >> 2) * RB + 16 * (tg & 3);
    const int bs_lbase = (tg >> 2) * kLdB + 16 * (tg & 3);
    auto st_loff = [&](int j) { return st_lbase + j * (GS / 8) * kLdA; };
    auto bs_loff = [&](int i) { return bs_lbase + i * (GS / 4) * kLdB; };

    auto st_load = [&](int c, int j) -> v4i {
        const int k = c * kChunk;
        const bool live = c < c_end && k + p16 < K;
        return __builtin_bit_cast(
            v4i, __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, live ? st_gbase + (j * (GS / 8) * K + k) : kLoadDead,
                                                       0, 0));
    };
    // sign bits of block b (chunks c_begin + 4 b .. + 3), slot i: 16 bytes of its chunk
    auto bs_load = [&](int b, int i) -> v4i {
        const int c0 = c_begin + kBlk * b;
        const bool live = b < nblk && c0 + (tg & 3) < c_end;
        return __builtin_bit_cast(
            v4i, __builtin_amdgcn_raw_buffer_load_b128(
                     b_rsrc, live ? bs_gbase + (i * (GS / 4) * RB + 16 * c0) : kLoadDead, 0, 0));
    };
    // A operand of step s, row block mb: row 32 mb + l32, bytes [64 g + 16 s, +16)
    auto a_frag = [&](int buf, int s, int mb) -> v4i {
        return *reinterpret_cast<const v4i*>(abuf + buf * C::kABytes + (32 * mb + l32) * kLdA + 64 * g + 16 * s);
    };
    // this lane's 64 sign bits of column block nb, chunk q of block buffer bb: k in
    // [c kChunk + 64 g, +64)
    auto b_bits = [&](int bb, int q, int nb) -> v2u {
        return *reinterpret_cast<const v2u*>(bbuf + bb * C::kBBytes + (wn * WN + 32 * nb + l32) * kLdB + 16 * q +
                                             8 * g);
    };
    auto b_op = [](const v2u& bits, int s) -> v4i { return bits16((s < 2 ? bits.x : bits.y) >> (16 * (s & 1))); };

    // kTin: W_B, the B operand of the t MFMAs (row lane & 15 over k = c kChunk + 64 h +
    // 16 (lane >> 4) in k-step h = 0, 1).  Chunks past the group's range or past K read
    // zero.  Two ways in:
    //  * staged (kWbLds): the chunk's kRank rows (kRank x 128 bytes) travel with its
    //    codes, two chunks ahead, by the K group's first 8 kRank threads (whole waves):
    //    piece tg -> row tg / 8, bytes [p16, +16), after the buffer's BM code rows (the
    //    code staging's base offsets serve).  The t MFMAs read them from LDS;
    //  * loaded (the widest configurations, whose registers are spent): each k-step's
    //    piece straight from memory a step or two ahead, one register set.  A wait for
    //    it also waits for the staging loads issued before it, cutting their slack.
    constexpr bool kWbLds = kTin && C::kStageWb;
    const bool lora = a.rank != 0;
    const __amdgpu_buffer_rsrc_t wb_rsrc = make_rsrc(a.w_b, (kTin && lora) ? (uint32_t)(kRank * K) : 0u);
    const int wb_lane = (lane & 15) * K + 16 * (lane >> 4);
    auto wb_load = [&](int c, int h) -> v4i {
        const int k = c * kChunk + 64 * h;
        const bool live = kTin && c < c_end && k < K;
        return __builtin_bit_cast(
            v4i, __builtin_amdgcn_raw_buffer_load_b128(wb_rsrc, live ? wb_lane + k : kLoadDead, 0, 0));
    };
    const bool wb_stager = tg < 8 * kRank;  // wave-uniform: whole waves
    const int wb_loff = st_lbase + BM * kLdA;
    auto wb_stage_load = [&](int c) -> v4i {
        const int k = c * kChunk;
        const bool live = kTin && wb_stager && c < c_end && k + p16 < K;
        return __builtin_bit_cast(
            v4i, __builtin_amdgcn_raw_buffer_load_b128(wb_rsrc, live ? st_gbase + k : kLoadDead, 0, 0));
    };
    auto wb_frag = [&](int buf, int h) -> v4i {
        return *reinterpret_cast<const v4i*>(abuf + buf * C::kABytes + (BM + (lane & 15)) * kLdA + 64 * h +
                                             16 * (lane >> 4));
    };
    // A operand of the t MFMAs: token rows 16 rb + (lane & 15) of block j, k-step h
    auto ta_frag = [&](int buf, int j, int h) -> v4i {
        const int rb = wn + WNW * j;
        return *reinterpret_cast<const v4i*>(abuf + buf * C::kABytes + (16 * rb + (lane & 15)) * kLdA + 64 * h +
                                             16 * (lane >> 4));
    };
    v4i tacc[kTin ? TB : 1];
#pragma unroll
    for (int j = 0; j < (kTin ? TB : 1); ++j) tacc[j] = (v4i){0, 0, 0, 0};
    v4i wbv;  // loaded: the W_B piece of the next t k-step; staged: this thread's piece of the next chunk

    v16i acc[MB][NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = (v16i){};
    int rsum[P];
#pragma unroll
    for (int j = 0; j < P; ++j) rsum[j] = 0;

    // ---- prologue: chunk 0 and sign block 0 into LDS; chunk 1 in flight ----
    v4i stage[P], bst[JB];
#pragma unroll
    for (int j = 0; j < P; ++j) stage[j] = st_load(c_begin, j);
#pragma unroll
    for (int i = 0; i < JB; ++i) bst[i] = bs_load(0, i);
    if constexpr (kWbLds) wbv = wb_stage_load(c_begin);
    else if constexpr (kTin) wbv = wb_load(c_begin, 0);
#pragma unroll
    for (int j = 0; j < P; ++j) {
        *reinterpret_cast<v4i*>(abuf + st_loff(j)) = stage[j];
#pragma unroll
        for (int w = 0; w < 4; ++w) rsum[j] = byte_sum((uint32_t)stage[j][w], rsum[j]);
        stage[j] = st_load(c_begin + 1, j);
    }
#pragma unroll
    for (int i = 0; i < JB; ++i) *reinterpret_cast<v4i*>(bbuf + bs_loff(i)) = bst[i];
    if constexpr (kWbLds) {
        if (wb_stager) *reinterpret_cast<v4i*>(abuf + wb_loff) = wbv;
        wbv = wb_stage_load(c_begin + 1);
    }
    lds_barrier();
    v4i afr[2][MB], bop[2][NB];
    v2u bits0[NB], bits1[NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) afr[0][mb] = a_frag(0, 0, mb);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        bits0[nb] = b_bits(0, 0, nb);
        bop[0][nb] = b_op(bits0[nb], 0);
    }
    // Drain the prologue's loads here, once: the wait the loop header needs is the
    // worst case over its entry and back edge, and an entry with loads still in
    // flight would make every iteration wait for nearly all of its own loads.
    __builtin_amdgcn_s_waitcnt(0);

    // One chunk: the q-th of sign block b, code buffer q & 1, sign bits bc (the next
    // chunk's go to bn).  Per step s: store staged piece s of the next chunk into the
    // other code buffer and reload it two chunks ahead; fetch the next step's A
    // operands; run this step's MFMAs while expanding the next B operands.  Step 1
    // reads the next chunk's sign bits.  Chunk 0 of block b loads block b + 1's sign
    // bits and chunk 2 stores them, a chunk before chunk 3 first reads them.  The one
    // barrier per chunk sits in step 3, after the last store and before the first read
    // of the next chunk; every read of the current buffers was issued before it.
    // kTin: the t MFMAs of k-step h run in step h, beside the main MFMAs, on the current
    // code buffer.  Staged W_B: step 0 stores the next chunk's piece and loads the one two
    // chunks ahead, like a code piece.  Loaded W_B: the piece of k-step 1 is loaded in
    // step 0, and the next chunk's first piece in step 2.
    auto chunk = [&](int b, int q, const v2u (&bc)[NB], v2u (&bn)[NB]) {
        const int c = c_begin + kBlk * b + q;
        const int cur = q & 1, nxt = cur ^ 1;
        const int bb_cur = b & 1;
        if (q == 0) {
#pragma unroll
            for (int i = 0; i < JB; ++i) bst[i] = bs_load(b + 1, i);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int j = 0; j < P; ++j) {
                if (st_step(j) != s) continue;
                *reinterpret_cast<v4i*>(abuf + nxt * C::kABytes + st_loff(j)) = stage[j];
#pragma unroll
                for (int w = 0; w < 4; ++w) rsum[j] = byte_sum((uint32_t)stage[j][w], rsum[j]);
                stage[j] = st_load(c + 2, j);
            }
            if (s == 1) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) bn[nb] = q < 3 ? b_bits(bb_cur, q + 1, nb) : b_bits(bb_cur ^ 1, 0, nb);
            }
            if constexpr (kTin) {
                if (s < 2) {
                    const v4i wb = kWbLds ? wb_frag(cur, s) : wbv;
#pragma unroll
                    for (int j = 0; j < TB; ++j)
                        tacc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ta_frag(cur, j, s), wb, tacc[j], 0, 0, 0);
                }
                if constexpr (kWbLds) {
                    if (s == 0) {
                        if (wb_stager) *reinterpret_cast<v4i*>(abuf + nxt * C::kABytes + wb_loff) = wbv;
                        wbv = wb_stage_load(c + 2);
                    }
                } else {
                    if (s == 0) wbv = wb_load(c, 1);
                    if (s == 2) wbv = wb_load(c + 1, 0);
                }
            }
            if (s == 3) {
                if (q == 2) {
#pragma unroll
                    for (int i = 0; i < JB; ++i)
                        *reinterpret_cast<v4i*>(bbuf + (bb_cur ^ 1) * C::kBBytes + bs_loff(i)) = bst[i];
                }
                lds_barrier();
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) afr[(s + 1) & 1][mb] = s < 3 ? a_frag(cur, s + 1, mb) : a_frag(nxt, 0, mb);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    acc[mb][nb] =
                        __builtin_amdgcn_mfma_i32_32x32x32_i8(afr[s & 1][mb], bop[s & 1][nb], acc[mb][nb], 0, 0, 0);
                bop[(s + 1) & 1][nb] = s < 3 ? b_op(bc[nb], s + 1) : b_op(bn[nb], 0);
            }
            // one scheduling region per step, so loads stay where they are issued
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    for (int b = 0; b < nblk; ++b) {
        chunk(b, 0, bits0, bits1);
        chunk(b, 1, bits1, bits0);
        chunk(b, 2, bits0, bits1);
        chunk(b, 3, bits1, bits0);
    }

    // token code sums of this K group: the 8 threads of a row hold one 16-byte column
    // of it each
#pragma unroll
    for (int j = 0; j < P; ++j) {
        int v = rsum[j];
        v += __shfl_xor(v, 1, kWave);
        v += __shfl_xor(v, 2, kWave);
        v += __shfl_xor(v, 4, kWave);
        if ((tg & 7) == 0) rowsum[kq * BM + j * (GS / 8) + (tg >> 3)] = v;
    }
    lds_barrier();  // row sums published; the reduction below reuses the chunk buffers

    // Split-K: the KS groups of one column group hold partial sums of the same tile.
    // Block b = nb * MB + mb belongs to group kq = b % KS; the others hand theirs over
    // through LDS, RBLK blocks per phase.  Every wave runs every barrier.
    constexpr int NBLK = MB * NB;
    if constexpr (KS > 1) {
        v4i* const red = reinterpret_cast<v4i*>(lds);
#pragma unroll
        for (int p0 = 0; p0 < NBLK; p0 += RBLK) {
#pragma unroll
            for (int bI = p0; bI < NBLK && bI < p0 + RBLK; ++bI) {
                const int mb = bI % MB, nb = bI / MB;
                if (kq != bI % KS) {
                    const int slot = ((wn * RBLK + (bI - p0)) * KS + kq) * 4;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        red[(slot + j) * kWave + lane] = (v4i){acc[mb][nb][4 * j], acc[mb][nb][4 * j + 1],
                                                               acc[mb][nb][4 * j + 2], acc[mb][nb][4 * j + 3]};
                }
            }
            lds_barrier();
#pragma unroll
            for (int bI = p0; bI < NBLK && bI < p0 + RBLK; ++bI) {
                const int mb = bI % MB, nb = bI / MB;
                if (kq == bI % KS) {
#pragma unroll
                    for (int q = 0; q < KS; ++q) {
                        if (q == bI % KS) continue;
                        const int slot = ((wn * RBLK + (bI - p0)) * KS + q) * 4;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const v4i v = red[(slot + j) * kWave + lane];
#pragma unroll
                            for (int i = 0; i < 4; ++i) acc[mb][nb][4 * j + i] += v[i];
                        }
                    }
                }
            }
            lds_barrier();
        }
    }

    // kTin: the K groups' partial t tiles, tl[kq][row][rank], in the chunk buffers (free
    // now: their last reads came before the barriers above); D[4 (lane >> 4) + v][lane & 15]
    // of block j is t[row 16 rb + 4 (lane >> 4) + v][rank lane & 15].
    int32_t* const tl = reinterpret_cast<int32_t*>(lds);
    if constexpr (kTin) {
#pragma unroll
        for (int j = 0; j < TB; ++j) {
            const int rb = wn + WNW * j;
#pragma unroll
            for (int v = 0; v < 4; ++v)
                tl[(kq * BM + 16 * rb + 4 * (lane >> 4) + v) * kRank + (lane & 15)] = tacc[j][v];
        }
        lds_barrier();
        // the first column tile of each row block also writes t
        if (a.t_out != nullptr && lora && seg.n_begin == 0 && tn == 0) {
            for (int e = threadIdx.x; e < BM * kRank; e += C::NW * kWave) {
                int32_t v = 0;
#pragma unroll
                for (int q = 0; q < KS; ++q) v += tl[q * BM * kRank + e];
                if (e / kRank < rows) a.t_out[(int64_t)m0 * kRank + e] = v;
            }
        }
    }

    // ---- epilogue: LoRA-up on bf16 MFMA, scales, stores ----
    // Every load and store below goes through a resource sized to this tile, so no
    // element needs a branch: rows past M fall past the y resource by construction,
    // columns past the range get kColDead added, and a missing LoRA reads as zeros.
    const int N4 = N * 4;
    const __amdgpu_buffer_rsrc_t y_rsrc = make_rsrc(a.y + (int64_t)m0 * N, (uint32_t)(rows * N4));
    const __amdgpu_buffer_rsrc_t d_rsrc =
        make_rsrc(kDebug ? a.acc_dbg + (int64_t)m0 * N : a.acc_dbg, kDebug ? (uint32_t)(rows * N4) : 0u);
    const __amdgpu_buffer_rsrc_t sx_rsrc = make_rsrc(a.s_x + m0, (uint32_t)(rows * 4));
    const int ncl = min(n0, N);
    const __amdgpu_buffer_rsrc_t sw_rsrc = make_rsrc(a.s_w + ncl, (uint32_t)(cols * 4));
    const __amdgpu_buffer_rsrc_t sa_rsrc = make_rsrc(lora ? a.s_a + ncl : a.s_a, lora ? (uint32_t)(cols * 4) : 0u);
    const __amdgpu_buffer_rsrc_t wa_rsrc =
        make_rsrc(lora ? a.w_a + (int64_t)ncl * kRank : a.w_a, lora ? (uint32_t)(cols * kRank) : 0u);
    const __amdgpu_buffer_rsrc_t t_rsrc =
        make_rsrc(lora && !kTin ? static_cast<const void*>(a.t + (int64_t)m0 * kRank) : static_cast<const void*>(a.s_x),
                  lora && !kTin ? (uint32_t)(rows * kRank * 4) : 0u);
    const __amdgpu_buffer_rsrc_t sb_rsrc = make_rsrc(a.s_b, lora ? (uint32_t)(kRank * 4) : 0u);

    // per column block: this lane's column n0 + 32 nb + l32
    float sw[NB], sa[NB];
    int col_off[NB];
    v8bf wa[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int c = 32 * nb + l32;
        const bool live = c < cols;
        col_off[nb] = live ? (n0 + c) * 4 : kColDead;
        sw[nb] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(sw_rsrc, live ? c * 4 : kLoadDead, 0, 0));
        sa[nb] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(sa_rsrc, live ? c * 4 : kLoadDead, 0, 0));
        // W_A[n][8 g .. 8 g + 7] -> bf16 (exact: |W_A| <= 127)
        const v2u wr = __builtin_bit_cast(
            v2u, __builtin_amdgcn_raw_buffer_load_b64(wa_rsrc, live ? c * kRank + 8 * g : kLoadDead, 0, 0));
        uint32_t bits[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int v = (int)(int8_t)(((e < 4 ? wr.x : wr.y) >> (8 * (e & 3))) & 0xFFu);
            bits[e] = __float_as_uint((float)v) >> 16;
        }
        wa[nb] = pack_bf16(bits);
    }
    float sbv[8];
    {
        const v4u s0 = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(sb_rsrc, 32 * g, 0, 0));
        const v4u s1 = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(sb_rsrc, 32 * g + 16, 0, 0));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sbv[e] = __uint_as_float(s0[e]);
            sbv[4 + e] = __uint_as_float(s1[e]);
        }
    }

#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        bool any = KS == 1;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) any = any || kq == (nb * MB + mb) % KS;
        if (!any) continue;

        // s_x and the code sum R of this lane's 16 output rows 32 mb + 8 (v / 4) + 4 g + v % 4
        float sx[16];
        int rs[16];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 32 * mb + 8 * j + 4 * g;
            const v4u v = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(sx_rsrc, r * 4, 0, 0));
            v4i rt = *reinterpret_cast<const v4i*>(rowsum + r);
#pragma unroll
            for (int q = 1; q < KS; ++q) rt += *reinterpret_cast<const v4i*>(rowsum + q * BM + r);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sx[4 * j + i] = __uint_as_float(v[i]);
                rs[4 * j + i] = rt[i];
            }
        }
        // u = s_B t for token row 32 mb + l32, ranks 8 g .. 8 g + 7, as three bf16 parts
        v8bf uh, um, ul;
        if (lora) {
            const int off = ((32 * mb + l32) * kRank + 8 * g) * 4;
            v4u t0, t1;
            if constexpr (kTin) {
                // rows past M hold codes of zero, so their t is zero like a missing row's
                t0 = *reinterpret_cast<const v4u*>(tl + (32 * mb + l32) * kRank + 8 * g);
                t1 = *reinterpret_cast<const v4u*>(tl + (32 * mb + l32) * kRank + 8 * g + 4);
#pragma unroll
                for (int q = 1; q < KS; ++q) {
                    t0 += *reinterpret_cast<const v4u*>(tl + (q * BM + 32 * mb + l32) * kRank + 8 * g);
                    t1 += *reinterpret_cast<const v4u*>(tl + (q * BM + 32 * mb + l32) * kRank + 8 * g + 4);
                }
            } else {
                t0 = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(t_rsrc, off, 0, 0));
                t1 = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(t_rsrc, off + 16, 0, 0));
            }
            uint32_t h[8], m[8], l[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float u = sbv[e] * (float)(int32_t)(e < 4 ? t0[e] : t1[e - 4]);
                split3_bf16(u, h[e], m[e], l[e]);
            }
            uh = pack_bf16(h);
            um = pack_bf16(m);
            ul = pack_bf16(l);
        }
        const int row_base = (32 * mb + 4 * g) * N4;

#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            if (kq != (nb * MB + mb) % KS) continue;
            v16f lo = (v16f){};
            if (lora) {
                lo = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ul, wa[nb], lo, 0, 0, 0);
                lo = __builtin_amdgcn_mfma_f32_32x32x16_bf16(um, wa[nb], lo, 0, 0, 0);
                lo = __builtin_amdgcn_mfma_f32_32x32x16_bf16(uh, wa[nb], lo, 0, 0, 0);
            }
            const int base = row_base + col_off[nb];
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                // row 32 mb + 8 (v / 4) + 4 g + v % 4 (past `rows`: past the resource)
                const int off = base + (8 * (v / 4) + (v % 4)) * N4;
                const int32_t acc_pm = 2 * acc[mb][nb][v] - rs[v];  // the +-1 sum
                // without LoRA, sa = lo = 0 and the fma returns s_w acc unchanged
                const float inner = fmaf(sa[nb], lo[v], sw[nb] * (float)acc_pm);
                store_f32_dev(sx[v] * inner, y_rsrc, off);
                if constexpr (kDebug) store_i32_dev(acc_pm, d_rsrc, off);
            }
            // Two groups per CU: let each column block's stores complete before the next
            // block's go out (vmcnt(0) alone).  The row blocks already drain this way (their
            // loads follow the previous block's stores); draining per column block as well
            // paces the output of groups that all finish together (measured: in_proj M2048
            // 0.7 us faster; the one-group-per-CU configurations measured slower with it).
            if constexpr (C::OCC > 1) __builtin_amdgcn_s_waitcnt(0x0F70);
        }
    }
}

// Problem blockIdx.y of a dense batch; blocks [0, T0) run configuration C0 over seg0,
// the rest C1 over seg1.  Segment 0's tiles are dealt to the 8 XCDs in contiguous runs
// (workgroups go to XCDs round-robin), so the code rows and sign columns one XCD reads
// stay in its L2.
template <class C0, class C1, bool kDebug, bool kTin>
__global__ __launch_bounds__(C0::NW * kWave) __attribute__((amdgpu_waves_per_eu(C0::NW / 4 * C0::OCC, C0::NW / 4 * C0::OCC))) void
gemm_prefill_kernel(prefill::Args a, prefill::Seg seg0, prefill::Seg seg1) {
    static_assert(C0::NW == C1::NW && C0::OCC == C1::OCC, "both parts of a launch use the same workgroup shape");
    constexpr int kLds = C0::kLdsBytes > C1::kLdsBytes ? C0::kLdsBytes : C1::kLdsBytes;
    __shared__ __align__(16) uint8_t lds[kLds];
    {
        const int64_t p = blockIdx.y;
        const int64_t M = a.M, N = a.N, K = a.K;
        a.x_q += p * M * K;
        a.s_x += p * M;
        a.w_bits += p * N * (K / 8);
        a.s_w += p * N;
        a.y += p * M * N;
        if (kDebug) a.acc_dbg += p * M * N;
        if (a.rank != 0) {
            a.w_a += p * N * kRank;
            a.s_a += p * N;
            a.s_b += p * kRank;
            if (kTin) {
                a.w_b += p * kRank * K;
                if (a.t_out) a.t_out += p * M * kRank;
            } else {
                a.t += p * M * kRank;
            }
        }
    }
    const int T0 = seg0.tiles_m * seg0.tiles_n;
    const int b = blockIdx.x;
    if (b < T0) {
        const int xcd = b % 8, q8 = T0 / 8, r8 = T0 % 8;
        const int tile = xcd * q8 + min(xcd, r8) + b / 8;
        prefill_tile<C0, kDebug, kTin>(a, lds, tile, seg0);
    } else {
        prefill_tile<C1, kDebug, kTin>(a, lds, b - T0, seg1);
    }
}

namespace {

using prefill::Cfg;
using prefill::Seg;

// Tile configurations (row blocks, column blocks per wave, K groups, waves):
using C441 = Cfg<4, 4, 1>;     // 128 x 512, wide N
using C422 = Cfg<4, 2, 2>;     // 128 x 128, split-K by 2
using C412 = Cfg<4, 1, 2>;     // 128 x 64, split-K by 2 (narrow parts)
using C4218 = Cfg<4, 2, 1, 8>;  // 128 x 512, two waves per SIMD
using C4128 = Cfg<4, 1, 2, 8>;  // 128 x 128, split-K by 2, two waves per SIMD
using C2128 = Cfg<2, 1, 2, 8>;  // 64 x 128, split-K by 2, two waves per SIMD (narrow parts)
using C2148 = Cfg<2, 1, 4, 8>;  // 64 x 64, split-K by 4, two waves per SIMD (narrow parts)
using C4214 = Cfg<4, 2, 1, 4, 2>;  // 128 x 256, two 4-wave groups per CU
using C2124 = Cfg<2, 1, 2, 4, 2>;  // 64 x 64, split-K by 2, two 4-wave groups per CU (narrow parts)

struct CfgInfo {
    int bm, bn, ks, nw, wave_cols, occ;
};
constexpr CfgInfo kCfgs[] = {{128, 512, 1, 4, 128, 1}, {128, 128, 2, 4, 64, 1}, {128, 64, 2, 4, 32, 1},
                             {128, 512, 1, 8, 64, 1},  {128, 128, 2, 8, 32, 1}, {64, 128, 2, 8, 32, 1},
                             {64, 64, 4, 8, 32, 1},    {128, 256, 1, 4, 64, 2}, {64, 64, 2, 4, 32, 2}};
constexpr int kNumCfgs = 9;
// The narrower configurations each one is instantiated with for a tail (-1: none).
constexpr int kTails[kNumCfgs][2] = {{1, 2}, {2, -1}, {-1, -1}, {5, 6}, {5, 6}, {6, -1}, {-1, -1}, {8, -1}, {-1, -1}};
constexpr int kNumCUs = 256;

struct Plan {
    int main_cfg, tail_cfg;  // indices into kCfgs; tail_cfg < 0: no tail
    int n_split;             // columns [0, n_split) main, [n_split, N) tail
};

int64_t tiles_of(int cfg, int64_t M, int64_t n_cols) {
    const CfgInfo& c = kCfgs[cfg];
    return ((M + c.bm - 1) / c.bm) * ((n_cols + c.bn - 1) / c.bn);
}

// Workgroups of configuration cfg the GPU holds at once.
int64_t slots_of(int cfg) { return (int64_t)kNumCUs * kCfgs[cfg].occ; }

// Modelled time of one part, in units of a 128 x 128 x 128 MFMA step of one SIMD:
// rounds of resident workgroups, each costing a fixed latency (prologue, epilogue,
// launch: ~2.3 units, fitted to the measured cost of a short second round) plus the
// steps of one SIMD (a chunk count rounded up to the 4-chunk sign block; the SIMD
// serves one wave of each co-resident group), 10 % extra for the split-K hand-over,
// 15 % less with two waves per SIMD (measured: their stalls overlap), 1 % more with
// two groups per CU (measured on one round of 128 x 256 tiles against 128 x 512), and
// 60 % more for 64-row tiles (half the MFMAs per expanded sign operand).
constexpr double kRoundLatency = 2.3;
double part_cost(int cfg, int64_t M, int64_t n_cols, int64_t K, int64_t batch, int64_t* wgs_out) {
    const CfgInfo& c = kCfgs[cfg];
    const int64_t wgs = tiles_of(cfg, M, n_cols) * batch;
    if (wgs_out) *wgs_out = wgs;
    const int64_t rounds = (wgs + slots_of(cfg) - 1) / slots_of(cfg);
    const int64_t nch = (K + 127) / 128;
    const int64_t per = ((nch + c.ks - 1) / c.ks + 3) / 4 * 4;
    const int waves_per_simd = c.nw * c.occ / 4;
    return (double)rounds * (kRoundLatency + (double)per * (c.wave_cols * waves_per_simd / 128.0) * (c.bm / 128.0) *
                                                 (c.ks > 1 ? 1.1 : 1.0) * (waves_per_simd == 2 ? 0.85 : 1.0) *
                                                 (c.occ > 1 ? 1.01 : 1.0) * (c.bm < 128 ? 1.6 : 1.0));
}

// Column counts [0, n) that configuration cfg can take in whole tiles, leaving the
// rest to a narrower configuration: every whole tile, or the widest part that fills
// whole rounds of resident workgroups (so that a few main tiles do not spill into a
// round of their own).  Returns how many of the two exist.
int main_splits(int cfg, int64_t M, int64_t N, int64_t batch, int64_t (&n)[2]) {
    const int64_t bn = kCfgs[cfg].bn;
    const int64_t whole = N / bn * bn;
    int cnt = 0;
    if (whole > 0 && whole < N) n[cnt++] = whole;
    const int64_t tiles_m = (M + kCfgs[cfg].bm - 1) / kCfgs[cfg].bm * batch;
    const int64_t per_round = slots_of(cfg) / tiles_m;  // column tiles per round
    if (per_round >= 1) {
        const int64_t fill = N / bn / per_round * per_round * bn;
        if (fill > 0 && fill < N && (cnt == 0 || fill != n[0])) n[cnt++] = fill;
    }
    return cnt;
}

// Modelled time of main configuration mc over [0, n_main) plus tc over the rest, in
// one launch: the tail's workgroups take the slots the main part leaves free, then the
// ones that free up first.  With two groups per CU and a main part of one round, a
// tail group runs beside a main group that is still busy, which hides about half of
// its cost (measured; behind two or more main rounds it hid nothing measurable).
double split_cost(int mc, int tc, int64_t n_main, int64_t M, int64_t N, int64_t K, int64_t batch) {
    int64_t wm = 0, wt = 0;
    const double cm = part_cost(mc, M, n_main, K, batch, &wm);
    const bool beside = kCfgs[mc].occ > 1 && wm <= slots_of(mc);
    const double ct = part_cost(tc, M, N - n_main, K, batch, &wt) * (beside ? 0.5 : 1.0);
    const int64_t free_slots = (slots_of(mc) - wm % slots_of(mc)) % slots_of(mc);
    return wt <= free_slots ? (cm > ct ? cm : ct) : cm + ct;
}

bool tail_fits(int mc, int tc) { return tc >= 0 && (kTails[mc][0] == tc || kTails[mc][1] == tc); }

Plan plan_for(int64_t M, int64_t N, int64_t K, int64_t batch, int force, int force_tail) {
    if (force >= 0 && force < kNumCfgs) {
        // pinned: `force`, with the columns past its main part (the cheaper of its
        // splits) on `force_tail` when `force` has an instance with that tail
        int64_t n[2];
        const int cnt = force_tail < kNumCfgs && tail_fits(force, force_tail)
                            ? main_splits(force, M, N, batch, n)
                            : 0;
        if (cnt == 0) return Plan{force, -1, (int)N};
        int64_t pick = n[0];
        if (cnt == 2 && split_cost(force, force_tail, n[1], M, N, K, batch) <
                            split_cost(force, force_tail, n[0], M, N, K, batch))
            pick = n[1];
        return Plan{force, force_tail, (int)pick};
    }
    Plan best{0, -1, (int)N};
    double best_cost = 1e300;
    for (int mc = 0; mc < kNumCfgs; ++mc) {
        const double whole = part_cost(mc, M, N, K, batch, nullptr);
        if (whole < best_cost) {
            best_cost = whole;
            best = Plan{mc, -1, (int)N};
        }
        int64_t n[2];
        const int cnt = main_splits(mc, M, N, batch, n);
        for (int s = 0; s < cnt; ++s) {
            for (int tc = 0; tc < kNumCfgs; ++tc) {
                if (!tail_fits(mc, tc)) continue;
                const double cost = split_cost(mc, tc, n[s], M, N, K, batch);
                if (cost < best_cost) {
                    best_cost = cost;
                    best = Plan{mc, tc, (int)n[s]};
                }
            }
        }
    }
    return best;
}

template <class C0, class C1>
hipError_t launch2(const prefill::Args& a, const Seg& s0, const Seg& s1, int64_t batch, hipStream_t stream) {
    const int64_t blocks = (int64_t)s0.tiles_m * s0.tiles_n + (int64_t)s1.tiles_m * s1.tiles_n;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks, (unsigned)batch);
    const bool tin = a.rank != 0 && a.w_b != nullptr;
    if (a.acc_dbg) {
        if (tin) {
            gemm_prefill_kernel<C0, C1, true, true><<<grid, C0::NW * kWave, 0, stream>>>(a, s0, s1);
        } else {
            gemm_prefill_kernel<C0, C1, true, false><<<grid, C0::NW * kWave, 0, stream>>>(a, s0, s1);
        }
    } else if (tin) {
        gemm_prefill_kernel<C0, C1, false, true><<<grid, C0::NW * kWave, 0, stream>>>(a, s0, s1);
    } else {
        gemm_prefill_kernel<C0, C1, false, false><<<grid, C0::NW * kWave, 0, stream>>>(a, s0, s1);
    }
    return hipGetLastError();
}

template <class C>
Seg make_seg(int64_t M, int n_begin, int n_end) {
    return Seg{(int)((M + C::BM - 1) / C::BM), (n_end - n_begin + C::BN - 1) / C::BN, n_begin, n_end};
}

// T0 and T1 are the configurations kTails lists for C0 (a repeat where it has fewer).
template <class C0, class T0, class T1>
hipError_t launch_main(const prefill::Args& a, const Plan& p, int64_t batch, hipStream_t stream) {
    const Seg s0 = make_seg<C0>(a.M, 0, p.n_split);
    const Seg none{0, 0, a.N, a.N};
    const int* const tails = kTails[p.main_cfg];
    if (p.tail_cfg >= 0 && p.tail_cfg == tails[0])
        return launch2<C0, T0>(a, s0, make_seg<T0>(a.M, p.n_split, a.N), batch, stream);
    if (p.tail_cfg >= 0 && p.tail_cfg == tails[1])
        return launch2<C0, T1>(a, s0, make_seg<T1>(a.M, p.n_split, a.N), batch, stream);
    // no tail: every column on the main configuration
    return launch2<C0, C0>(a, make_seg<C0>(a.M, 0, a.N), none, batch, stream);
}

}  // namespace

// The cost model's plan for a shape (host only, no launch): the main configuration, the
// tail configuration (-1: none) and the first column of the tail.
void prefill_plan_query(int64_t M, int64_t N, int64_t K, int64_t batch, int* main_cfg, int* tail_cfg,
                        int64_t* n_split) {
    const Plan p = plan_for(M, N, K, batch, -1, -1);
    *main_cfg = p.main_cfg;
    *tail_cfg = p.tail_cfg;
    *n_split = p.tail_cfg >= 0 ? p.n_split : N;
}

// Tile configurations the prefill kernel can be pinned to by tests (index; -1 = pick
// by the cost model; a tail configuration applies to the columns past the last whole
// main tile).
int prefill_num_cfgs() { return kNumCfgs; }

// The prefill kernel needs K % 64 == 0 (whole 64-k lane-group slices) and per-tile
// byte offsets of y below 2^30 (128 rows x N x 4 bytes, plus kColDead below 2^31).
bool prefill_supported(int64_t M, int64_t N, int64_t K) {
    return K % 64 == 0 && K <= 131072 && M < ((int64_t)1 << 30) && N < ((int64_t)1 << 20) &&
           M * N < ((int64_t)1 << 40);
}

// t given (w_b == NULL), or computed in the K loop from W_B (t_out, when not NULL,
// receives it).
hipError_t launch_gemm_prefill(const int8_t* x_q, const float* s_x, int64_t M, int64_t N, int64_t K,
                               const uint8_t* w_bits, const float* s_w, const int8_t* w_a, const float* s_a,
                               const int8_t* w_b, const float* s_b, const int32_t* t, int32_t* t_out, int rank,
                               float* y, int32_t* acc_dbg, int64_t batch, int force_cfg, int force_tail,
                               hipStream_t stream) {
    const prefill::Args a{x_q, s_x, w_bits, s_w, w_a, s_a, s_b, t, w_b, t_out, y, acc_dbg,
                          (int)M, (int)N, (int)K, rank};
    const Plan p = plan_for(M, N, K, batch, force_cfg, force_tail);
    switch (p.main_cfg) {
        case 0: return launch_main<C441, C422, C412>(a, p, batch, stream);
        case 1: return launch_main<C422, C412, C412>(a, p, batch, stream);
        case 2: return launch_main<C412, C412, C412>(a, p, batch, stream);
        case 3: return launch_main<C4218, C2128, C2148>(a, p, batch, stream);
        case 4: return launch_main<C4128, C2128, C2148>(a, p, batch, stream);
        case 5: return launch_main<C2128, C2148, C2148>(a, p, batch, stream);
        case 6: return launch_main<C2148, C2148, C2148>(a, p, batch, stream);
        case 7: return launch_main<C4214, C2124, C2124>(a, p, batch, stream);
        default: return launch_main<C2124, C2124, C2124>(a, p, batch, stream);
    }
}

}  // namespace dfssm
