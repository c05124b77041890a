// gemm_prefill.hip -- prefill-shaped scaffold + LoRA projection on the int8 MFMA pipe (gfx950).
//
// DF-SSM technical summary (gist.science), section 2C: packed 1-bit scaffold
// weights are expanded to int8 on the fly and multiplied with int8 activations on the
// matrix cores; section 2B: the rank-16 int8 LoRA correction W_A (W_B x) with
// per-channel/row scales.  At many tokens the scaffold product is a dense int8
// contraction, so it runs on v_mfma_i32_32x32x32_i8; nothing is materialized in memory.
//
// Work split.  A workgroup is 4 waves (one per SIMD) and owns a (32 MB) x (32 NB WNW)
// output tile; WNW = 4 / KS waves side by side along N, KS waves along K (split-K
// inside the workgroup, reduced through LDS at the end).  Each wave keeps its
// (32 MB) x (32 NB) partial tile in MB x NB accumulators of 16 registers (AGPRs).
//
// Operands, straight from memory into registers (no LDS in the main loop):
//  * A (x_q rows): in a 128-k chunk, lane group g = lane / 32 takes k in
//    [64 g, 64 g + 64) and MFMA step s its 16 bytes [64 g + 16 s, +16) -- one 16-byte
//    load per row per step.  Any per-lane k order is valid as long as A and B agree.
//  * B (signs): the same lane's 64 sign bits of a column are 8 contiguous bytes (one
//    8-byte load per column per chunk).  Step s takes 16 of them and expands them to
//    16 bytes of +-1: each nibble is spread to one bit per byte ((nib * 0x00204081)
//    & 0x01010101) and a byte permute maps 0/1 to 0xFF/0x01.  With +-1 weights the
//    accumulator is the scaffold sum itself, no row-sum correction.
//  * 4-deep step rotation: the A registers of step s are reloaded with the next
//    chunk's step s right after their MFMAs, so loads run one chunk ahead.
//  * Tails: every load goes through a buffer resource; rows past M, columns past N
//    and k past K use an offset beyond the resource, which reads zero.
//
// Epilogue.  y = s_x (s_w acc + s_A sum_r W_A[n][r] s_B[r] t[m][r]).  The LoRA-up
// product is a second, tiny contraction (rank 16) and runs on v_mfma_f32_32x32x16_bf16:
// W_A is exact in bf16, and u = s_B t (fp32) is split exactly into three bf16 parts
// (h + m + l, each the truncation of the remainder), so the products are exact and
// only fp32 accumulation rounds.  Its output layout equals the int32 accumulator's,
// so the scale epilogue combines them register by register.
#include "device_common.h"

namespace dfssm {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

namespace prefill {
constexpr int kChunk = 128;            // k per main-loop chunk (64 per lane group)
constexpr int kLoadDead = 0x7ff00000;  // a load offset past every resource used here: reads zero
constexpr int kRedBlocks = 8;          // accumulator blocks per split-K reduction phase
constexpr int kColDead = 0x40000000;   // store offset added for columns past N: past the y resource
}  // namespace prefill

// 4 sign bits -> 4 bytes of +-1 (bit i -> byte i).
__device__ __forceinline__ uint32_t signs4(uint32_t nib) {
    return perm(0u, 0x000001FFu, (nib * 0x00204081u) & 0x01010101u);
}

// Low 16 bits of w -> a 16-byte B operand of +-1 (bit i -> byte i).
__device__ __forceinline__ v4i signs16(uint32_t w) {
    return (v4i){(int)signs4(w & 0xFu), (int)signs4((w >> 4) & 0xFu), (int)signs4((w >> 8) & 0xFu),
                 (int)signs4((w >> 12) & 0xFu)};
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

template <int MB, int NB, int KS, bool kDebug>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_prefill_kernel(
    const int8_t* __restrict__ x_q, const float* __restrict__ s_x, int M, int N, int K,
    const uint8_t* __restrict__ w_bits, const float* __restrict__ s_w, const int8_t* __restrict__ w_a,
    const float* __restrict__ s_a, const float* __restrict__ s_b, const int32_t* __restrict__ t, int rank,
    float* __restrict__ y, int32_t* __restrict__ acc_dbg, int tiles_m, int tiles_n) {
    using namespace prefill;
    constexpr int WNW = 4 / KS;
    constexpr int BM = 32 * MB, WN = 32 * NB, BN = WN * WNW;
    static_assert(KS == 1 || KS == 2 || KS == 4, "4 waves split over K and N");
    // LDS: per K group two chunk buffers of BM rows (row stride kLdA, padded so the
    // 16 rows a 16-lane group reads land in distinct banks); the split-K reduction
    // reuses the same bytes after the main loop.
    constexpr int kLdA = kChunk + 16;
    constexpr int kBufBytes = BM * kLdA;
    constexpr int kMainBytes = KS * 2 * kBufBytes;
    constexpr int kRedBytes = KS > 1 ? WNW * kRedBlocks * KS * 4 * kWave * 16 : 0;
    __shared__ __align__(16) uint8_t lds[kMainBytes > kRedBytes ? kMainBytes : kRedBytes];
    v4i* const red = reinterpret_cast<v4i*>(lds);
    // staging: the WNW waves of a K group load its chunk, 16-byte pieces, 8 threads
    // per 128-byte row segment (whole cache lines); J pieces per thread per step
    constexpr int GS = kWave * WNW;
    constexpr int J = BM * 8 / (4 * GS);
    static_assert(J * 4 * GS == BM * 8, "chunk pieces split evenly over steps");

    // problem blockIdx.y of a dense batch
    {
        const int64_t p = blockIdx.y;
        x_q += p * M * K;
        s_x += p * M;
        w_bits += p * N * (int64_t)(K / 8);
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

    // Workgroups are dealt to the 8 XCDs round-robin; give each XCD a contiguous run
    // of tiles (row-major), so the x_q rows and sign columns it reads stay in its L2.
    const int T = tiles_m * tiles_n;
    const int xcd = blockIdx.x % 8, q8 = T / 8, r8 = T % 8;
    const int tile = xcd * q8 + min(xcd, r8) + (int)(blockIdx.x / 8);
    const int tm = tile / tiles_n, tn = tile % tiles_n;

    // wave index made visibly wave-uniform, so the per-wave buffer resources are scalar
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const int lane = threadIdx.x % kWave;
    const int wn = wave % WNW, kq = wave / WNW;
    const int g = lane >> 5, l32 = lane & 31;
    const int m0 = tm * BM, n0 = tn * BN + wn * WN;
    const int RB = K / 8;
    // (readfirstlane: the clamps compile to VALU min/max, whose results the resource
    // builder would otherwise treat as per-lane)
    const int rows = __builtin_amdgcn_readfirstlane(min(M - m0, BM));
    const int cols = __builtin_amdgcn_readfirstlane(max(0, min(N - n0, WN)));

    const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(x_q + (int64_t)m0 * K, (uint32_t)(rows * K));
    const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc(w_bits + (int64_t)min(n0, N) * RB, (uint32_t)(cols * RB));
    int b_off[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) b_off[nb] = 32 * nb + l32 < cols ? (32 * nb + l32) * RB : kLoadDead;

    // every wave runs the same number of chunks (the barriers pair up); chunks past
    // its K range read zeros
    const int nch = (K + kChunk - 1) / kChunk;
    const int per = (nch + KS - 1) / KS;
    const int c_begin = kq * per, c_end = min(nch, c_begin + per);

    // staging pieces of this thread: step s, slot j -> row (s J + j) GS / 8 + tg / 8,
    // bytes [16 p, 16 p + 16) of the row's chunk segment
    const int tg = wn * kWave + lane, p16 = 16 * (tg & 7);
    int st_goff[4][J], st_loff[4][J];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int r = (s * J + j) * (GS / 8) + (tg >> 3);
            st_goff[s][j] = r < rows ? r * K + p16 : kLoadDead;
            st_loff[s][j] = r * kLdA + p16;
        }
    uint8_t* const abase = lds + kq * 2 * kBufBytes;

    // piece (s, j) of chunk c (zero past the wave's chunk range or past K)
    auto st_load = [&](int c, int s, int j) -> v4i {
        const int k = c * kChunk;
        const bool live = c < c_end && k + p16 < K;
        return __builtin_bit_cast(
            v4i, __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, live ? st_goff[s][j] + k : kLoadDead, 0, 0));
    };
    // A operand of step s, row block mb: row 32 mb + l32, bytes [64 g + 16 s, +16)
    auto a_frag = [&](int buf, int s, int mb) -> v4i {
        return *reinterpret_cast<const v4i*>(abase + buf * kBufBytes + (32 * mb + l32) * kLdA + 64 * g + 16 * s);
    };
    // 64 sign bits of column nb for chunk c: k in [c kChunk + 64 g, +64)
    auto b_load = [&](int c, int nb) -> v2u {
        const int k = c * kChunk + 64 * g;
        const bool live = c < c_end && k < K;
        return __builtin_bit_cast(
            v2u, __builtin_amdgcn_raw_buffer_load_b64(b_rsrc, live ? b_off[nb] + k / 8 : kLoadDead, 0, 0));
    };
    // B operand of step s from a chunk's 64 sign bits
    auto b_op = [](const v2u& bits, int s) -> v4i {
        return signs16((s < 2 ? bits.x : bits.y) >> (16 * (s & 1)));
    };

    v16i acc[MB][NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = (v16i){};

    // prologue: chunk c_begin into LDS buffer 0, chunk c_begin + 1 into the staging
    // registers, sign bits of both chunks, the first A and B operands
    v4i stage[4][J];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int j = 0; j < J; ++j) stage[s][j] = st_load(c_begin, s, j);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int j = 0; j < J; ++j) *reinterpret_cast<v4i*>(abase + st_loff[s][j]) = stage[s][j];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int j = 0; j < J; ++j) stage[s][j] = st_load(c_begin + 1, s, j);
    v2u bb0[NB], bb1[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        bb0[nb] = b_load(c_begin, nb);
        bb1[nb] = b_load(c_begin + 1, nb);
    }
    lds_barrier();
    // A and B operands are fetched / expanded one step ahead (double buffers), so each
    // step's LDS reads and VALU work are independent of its MFMAs and interleave.
    v4i afr[2][MB], bop[2][NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) afr[0][mb] = a_frag(0, 0, mb);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) bop[0][nb] = b_op(bb0[nb], 0);
    // Drain the prologue's loads here, once: the wait the loop header needs is the
    // worst case over its entry and back edge, and an entry with loads still in
    // flight would make every iteration wait for nearly all of its own loads.
    __builtin_amdgcn_s_waitcnt(0);

    // One chunk c, read from LDS buffer `cur`: per step s, store staged piece s of
    // chunk c + 1 into the other buffer and reload it with chunk c + 2, fetch the next
    // step's A operands, run the step's MFMAs while expanding the next B operands.
    // The one barrier per chunk sits in step 3, after the last store of chunk c + 1
    // and before its first operand read; every read of `cur` was issued before it.
    auto chunk = [&](int c, int cur, v2u (&bb)[NB], const v2u (&bn)[NB]) {
        const int nxt = cur ^ 1;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int j = 0; j < J; ++j) {
                *reinterpret_cast<v4i*>(abase + nxt * kBufBytes + st_loff[s][j]) = stage[s][j];
                stage[s][j] = st_load(c + 2, s, j);
            }
            if (s == 3) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) bb[nb] = b_load(c + 2, nb);
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
                bop[(s + 1) & 1][nb] = s < 3 ? b_op(bb[nb], s + 1) : b_op(bn[nb], 0);
            }
            // one scheduling region per step, so loads stay where they are issued
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    for (int i = 0; i < per; i += 2) {
        chunk(c_begin + i, 0, bb0, bb1);
        chunk(c_begin + i + 1, 1, bb1, bb0);
    }
    lds_barrier();  // the reduction below reuses the chunk buffers

    // Split-K: the KS waves of one column group hold partial sums of the same tile.
    // Block b = nb * MB + mb belongs to wave kq = b % KS; the others hand theirs over
    // through LDS, kRedBlocks blocks per phase.  Every wave runs every barrier.
    constexpr int NBLK = MB * NB;
    if constexpr (KS > 1) {
#pragma unroll
        for (int p0 = 0; p0 < NBLK; p0 += kRedBlocks) {
#pragma unroll
            for (int b = p0; b < NBLK && b < p0 + kRedBlocks; ++b) {
                const int mb = b % MB, nb = b / MB;
                if (kq != b % KS) {
                    const int slot = ((wn * kRedBlocks + (b - p0)) * KS + kq) * 4;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        red[(slot + j) * kWave + lane] = (v4i){acc[mb][nb][4 * j], acc[mb][nb][4 * j + 1],
                                                               acc[mb][nb][4 * j + 2], acc[mb][nb][4 * j + 3]};
                }
            }
            lds_barrier();
#pragma unroll
            for (int b = p0; b < NBLK && b < p0 + kRedBlocks; ++b) {
                const int mb = b % MB, nb = b / MB;
                if (kq == b % KS) {
#pragma unroll
                    for (int q = 0; q < KS; ++q) {
                        if (q == b % KS) continue;
                        const int slot = ((wn * kRedBlocks + (b - p0)) * KS + q) * 4;
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

    // ---- epilogue: LoRA-up on bf16 MFMA, scales, stores ----
    // Every load and store below goes through a resource sized to this tile, so no
    // element needs a branch: rows past M fall past the y resource by construction,
    // columns past N get kColDead added, and a missing LoRA reads as zeros.
    const bool lora = rank != 0;
    const int N4 = N * 4;
    const __amdgpu_buffer_rsrc_t y_rsrc = make_rsrc(y + (int64_t)m0 * N, (uint32_t)(rows * N4));
    const __amdgpu_buffer_rsrc_t d_rsrc =
        make_rsrc(kDebug ? acc_dbg + (int64_t)m0 * N : acc_dbg, kDebug ? (uint32_t)(rows * N4) : 0u);
    const __amdgpu_buffer_rsrc_t sx_rsrc = make_rsrc(s_x + m0, (uint32_t)(rows * 4));
    const int ncl = min(n0, N);
    const __amdgpu_buffer_rsrc_t sw_rsrc = make_rsrc(s_w + ncl, (uint32_t)(cols * 4));
    const __amdgpu_buffer_rsrc_t sa_rsrc = make_rsrc(lora ? s_a + ncl : s_a, lora ? (uint32_t)(cols * 4) : 0u);
    const __amdgpu_buffer_rsrc_t wa_rsrc =
        make_rsrc(lora ? w_a + (int64_t)ncl * kRank : w_a, lora ? (uint32_t)(cols * kRank) : 0u);
    const __amdgpu_buffer_rsrc_t t_rsrc =
        make_rsrc(lora ? t + (int64_t)m0 * kRank : t, lora ? (uint32_t)(rows * kRank * 4) : 0u);
    const __amdgpu_buffer_rsrc_t sb_rsrc = make_rsrc(s_b, lora ? (uint32_t)(kRank * 4) : 0u);

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

        // s_x of this lane's 16 output rows 32 mb + 8 (v / 4) + 4 g + v % 4
        float sx[16];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 32 * mb + 8 * j + 4 * g;
            const v4u v = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(sx_rsrc, r * 4, 0, 0));
#pragma unroll
            for (int i = 0; i < 4; ++i) sx[4 * j + i] = __uint_as_float(v[i]);
        }
        // u = s_B t for token row 32 mb + l32, ranks 8 g .. 8 g + 7, as three bf16 parts
        v8bf uh, um, ul;
        if (lora) {
            const int off = ((32 * mb + l32) * kRank + 8 * g) * 4;
            const v4u t0 = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(t_rsrc, off, 0, 0));
            const v4u t1 = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(t_rsrc, off + 16, 0, 0));
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
                const int32_t a = acc[mb][nb][v];
                // without LoRA, sa = lo = 0 and the fma returns s_w acc unchanged
                const float inner = fmaf(sa[nb], lo[v], sw[nb] * (float)a);
                store_f32(sx[v] * inner, y_rsrc, off);
                if constexpr (kDebug) store_i32(a, d_rsrc, off);
            }
        }
    }
}

namespace {

struct PrefillCfg {
    int mb, nb, ks;
};

constexpr PrefillCfg kPrefillCfgs[] = {{4, 4, 1}, {4, 4, 2}, {4, 4, 4}};
constexpr int kNumCUs = 256;

template <int MB, int NB, int KS>
hipError_t launch_cfg(const int8_t* x_q, const float* s_x, int M, int N, int K, const uint8_t* w_bits,
                      const float* s_w, const int8_t* w_a, const float* s_a, const float* s_b, const int32_t* t,
                      int rank, float* y, int32_t* acc_dbg, int64_t batch, hipStream_t stream) {
    const int BM = 32 * MB, BN = 32 * NB * (4 / KS);
    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const dim3 grid((unsigned)(tiles_m * tiles_n), (unsigned)batch);
    if (acc_dbg) {
        gemm_prefill_kernel<MB, NB, KS, true><<<grid, 256, 0, stream>>>(x_q, s_x, M, N, K, w_bits, s_w, w_a, s_a,
                                                                        s_b, t, rank, y, acc_dbg, tiles_m, tiles_n);
    } else {
        gemm_prefill_kernel<MB, NB, KS, false><<<grid, 256, 0, stream>>>(x_q, s_x, M, N, K, w_bits, s_w, w_a, s_a,
                                                                         s_b, t, rank, y, acc_dbg, tiles_m, tiles_n);
    }
    return hipGetLastError();
}

// Modelled time of a configuration: whole rounds of 256 one-workgroup-per-CU tiles,
// times the MFMA steps per wave, plus the split-K hand-over.
double cfg_cost(const PrefillCfg& c, int64_t M, int64_t N, int64_t K, int64_t batch) {
    const int64_t BM = 32 * c.mb, BN = 32 * c.nb * (4 / c.ks);
    const int64_t wgs = ((M + BM - 1) / BM) * ((N + BN - 1) / BN) * batch;
    const int64_t rounds = (wgs + kNumCUs - 1) / kNumCUs;
    const int64_t nch = (K + 127) / 128;
    const int64_t steps = (int64_t)c.mb * c.nb * ((nch + c.ks - 1) / c.ks);
    return (double)rounds * (double)steps * (c.ks > 1 ? 1.15 : 1.0);
}

}  // namespace

// Tile configurations the prefill kernel can take, for tests that pin one
// (index into kPrefillCfgs; -1 = pick by the cost model).
int prefill_num_cfgs() { return (int)(sizeof(kPrefillCfgs) / sizeof(kPrefillCfgs[0])); }

// The prefill kernel needs K % 64 == 0 (whole 64-k lane-group slices) and per-tile
// byte offsets of y below 2^30 (128 rows x N x 4 bytes, plus kColDead below 2^31).
bool prefill_supported(int64_t M, int64_t N, int64_t K) {
    return K % 64 == 0 && K <= 131072 && M < ((int64_t)1 << 30) && N < ((int64_t)1 << 20) &&
           M * N < ((int64_t)1 << 40);
}

hipError_t launch_gemm_prefill(const int8_t* x_q, const float* s_x, int64_t M, int64_t N, int64_t K,
                               const uint8_t* w_bits, const float* s_w, const int8_t* w_a, const float* s_a,
                               const float* s_b, const int32_t* t, int rank, float* y, int32_t* acc_dbg,
                               int64_t batch, int force_cfg, hipStream_t stream) {
    int best = 0;
    if (force_cfg >= 0 && force_cfg < prefill_num_cfgs()) {
        best = force_cfg;
    } else {
        double best_cost = 0.0;
        for (int i = 0; i < prefill_num_cfgs(); ++i) {
            const double c = cfg_cost(kPrefillCfgs[i], M, N, K, batch);
            if (i == 0 || c < best_cost) {
                best = i;
                best_cost = c;
            }
        }
    }
    const PrefillCfg c = kPrefillCfgs[best];
    const int64_t BM = 32 * c.mb, BN = 32 * c.nb * (4 / c.ks);
    if (((M + BM - 1) / BM) * ((N + BN - 1) / BN) > 0x7fffffffLL) return hipErrorInvalidValue;
    const int m = (int)M, n = (int)N, k = (int)K;
    switch (best) {
        case 0: return launch_cfg<4, 4, 1>(x_q, s_x, m, n, k, w_bits, s_w, w_a, s_a, s_b, t, rank, y, acc_dbg, batch, stream);
        case 1: return launch_cfg<4, 4, 2>(x_q, s_x, m, n, k, w_bits, s_w, w_a, s_a, s_b, t, rank, y, acc_dbg, batch, stream);
        default: return launch_cfg<4, 4, 4>(x_q, s_x, m, n, k, w_bits, s_w, w_a, s_a, s_b, t, rank, y, acc_dbg, batch, stream);
    }
}

}  // namespace dfssm
