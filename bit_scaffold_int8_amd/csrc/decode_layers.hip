// decode_layers.hip -- the whole per-token decode of a stack of DF-SSM layers for one
// sequence in ONE kernel launch (gfx950).
//
// DF-SSM technical summary (gist.science), section 2C "Optimized Inference Pipeline":
// the entire 48-layer forward pass is captured as one CUDA graph because launch overhead
// decides batch-1 speed; the layer is in_proj (1-bit scaffold + int8 LoRA) -> the
// stateful convolution and SSM recurrence -> out_proj.  Here the launches go away
// altogether: one persistent grid (one 512-thread group per CU, co-resident by a
// cooperative launch) walks all layers, and the dependencies between the three steps
// of a layer become device-wide counters:
//
//   phase A (in_proj, K 2048 -> N 8512): every group quantizes the layer's input x
//     (absmax / 127, ties to even), computes t = W_B x_q for itself, and produces its
//     33 or 34 rows of zxbcdt; then it counts itself in A[l].
//   phase B (Mamba-2 step): group g owns 16 channels of head g / 4; once A[l] reaches
//     the group count it reads its z, x, dt and the shared B, C, runs the convolution,
//     the state update and the gate, g = y silu(z), for its channels; counts in B[l].
//   phase C (gated RMS norm + out_proj, K 4096 -> N 2048): once B[l] is full, every
//     group reads all of g, forms the norm (the mean square in one fixed order, so all
//     groups get the same bits), quantizes the result, computes t, and produces its 8
//     rows of the next layer's input; counts in C[l], which phase A of layer l + 1
//     waits for.
//
// Weights do not depend on activations, so each group issues the loads of its next
// phase's packed signs, W_B slice, epilogue operands and state slice before it waits:
// the HBM stream overlaps the wait.  Exchanged activations are written with
// device-scope (write-through) stores and read with device-scope loads, so they are
// coherent across the XCDs' L2s without cache-maintenance fences; a group counts
// itself only after its stores have completed.  Every wait is bounded: past the
// poll limit, or once any group has reported a failure, it gives up and ORs a bit
// into the caller's status word; the kernel always runs to the end.  The last group
// to finish resets the counters, so the workspace is ready for the next call.
//
// At M = 1 the products are latency-bound, so they run on the vector ALUs: the packed
// signs are expanded by bit plane (w & (0x01010101 << j) holds four weights of plane
// j) against the codes stored in plane order in LDS, four products per v_dot4.
#include "decode_args.h"
#include "device_common.h"
#include "quant_common.h"

#include <mutex>

namespace dfssm {

namespace decode {

constexpr int kDModel = 2048, kDInner = 4096, kDState = 128, kNHeads = 64, kHeadDim = 64;
constexpr int kConvDim = kDInner + 2 * kDState;            // 4352
constexpr int kNIn = kDInner + kConvDim + kNHeads;          // 8512
constexpr int kGroups = 256, kThreads = 512, kWaves = kThreads / kWave;
constexpr int kCtrStride = 16;                               // words between counters (64 B)
constexpr int kMaxLayers = 64;
constexpr int kStatusTimeout = 1, kStatusGaveUp = 2;

// workspace layout (4-byte words)
constexpr int kWsCounters = 0;                               // (3 kMaxLayers + 1) counters
constexpr int kWsX = (3 * kMaxLayers + 1) * kCtrStride;      // x [2][2048]
constexpr int kWsZx = kWsX + 2 * kDModel;                    // zxbcdt [2][8512]
constexpr int kWsG = kWsZx + 2 * kNIn;                       // g [2][4096]
constexpr int kWsWords = kWsG + 2 * kDInner;

// trace layout per layer (4-byte words)
constexpr int kTrZx = 0, kTrOut = kTrZx + kNIn, kTrXn = kTrOut + kDInner, kTrAccIn = kTrXn + kDModel,
              kTrAccOut = kTrAccIn + kNIn, kTrXqIn = kTrAccOut + kDModel, kTrXqOut = kTrXqIn + kDModel / 4,
              kTrTIn = kTrXqOut + kDInner / 4, kTrTOut = kTrTIn + kRank, kTrSx = kTrTOut + kRank,
              kTrWords = kTrSx + 16;


__device__ __forceinline__ float silu(float v) { return v / (1.0f + expf(-v)); }
__device__ __forceinline__ float softplus(float v) { return v > 20.0f ? v : log1pf(expf(v)); }

// device-scope (coherent across XCDs) exchange loads and stores
__device__ __forceinline__ float4 ld4_dev(const float* base, uint32_t bytes, int byte_off) {
    const v4f v = __builtin_bit_cast(
        v4f, __builtin_amdgcn_raw_buffer_load_b128(make_rsrc(base, bytes), byte_off, 0, kAuxDeviceScope));
    return make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ float ld_dev(const float* base, uint32_t bytes, int byte_off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(make_rsrc(base, bytes), byte_off, 0, kAuxDeviceScope));
}

// Every store of this thread has completed (stores count in vmcnt on gfx9-family parts;
// device-scope stores complete once written through).
__device__ __forceinline__ void wait_stores() {
    __builtin_amdgcn_s_waitcnt(0);
    asm volatile("" ::: "memory");
}

// Bounded wait of the whole group until *ctr >= target (thread 0 polls).  Returns false
// once the group has failed (then it no longer waits).
__device__ bool group_wait(const Args& a, uint32_t* ctr, uint32_t target, bool ok, int* sflag) {
    if (threadIdx.x == 0) {
        int fail = ok ? 0 : 1;
        if (ok) {
            const uint32_t want = target + a.target_bias;
            for (int64_t n = 0;; ++n) {
                const uint32_t v = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (v >= want) break;
                if (n >= a.spin_limit) {
                    __hip_atomic_fetch_or(a.status, kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    fail = 1;
                    break;
                }
                if ((n & 15) == 15 &&
                    __hip_atomic_load(a.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
                    __hip_atomic_fetch_or(a.status, kStatusGaveUp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    fail = 1;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        }
        *sflag = fail;
    }
    lds_barrier();
    const bool r = *sflag == 0;
    lds_barrier();  // the flag slot is reused by the next wait
    return r;
}

// Count the group in *ctr once every thread's stores have completed.
__device__ __forceinline__ void group_signal(uint32_t* ctr) {
    wait_stores();
    lds_barrier();
    if (threadIdx.x == 0) __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Maximum over the group (every thread gets it): one barrier; `red` is not reused
// before a later barrier.
__device__ __forceinline__ float group_max(float v, float* red) {
    v = wave_max(v);
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = v;
    lds_barrier();
    float m = red[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m = fmaxf(m, red[w]);
    return m;
}

// Sum over the group in one fixed order (a butterfly within each wave, then the waves
// in order), so every group that sums the same values gets the same bits.
__device__ __forceinline__ float group_sum_fixed(float v, float* red) {
    for (int o = 1; o < kWave; o <<= 1) v += __shfl_xor(v, o, kWave);
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = v;
    lds_barrier();
    float s = red[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) s += red[w];
    return s;
}

// Plane order of 32 codes (one 32-k block, natural words n[0..7] = codes k..k+31):
// p[j] = (x[j], x[8 + j], x[16 + j], x[24 + j]), the four codes that bit j of the four
// bytes of a packed-sign word weights.
__device__ __forceinline__ void to_planes(const uint32_t (&n)[8], uint32_t (&p)[8]) {
#pragma unroll
    for (int jh = 0; jh < 2; ++jh) {
        uint32_t o0, o1, o2, o3;
        // bytes j and j + 4 of each pair of words: transpose the 4x4 byte blocks
        transpose4x4(n[0 + jh], n[2 + jh], n[4 + jh], n[6 + jh], o0, o1, o2, o3);
        p[4 * jh + 0] = o0;
        p[4 * jh + 1] = o1;
        p[4 * jh + 2] = o2;
        p[4 * jh + 3] = o3;
    }
}

// Sum of the codes whose sign bit is 1 over one packed-sign word w (32 k) against its
// plane-ordered codes p[0..7]: planes j and j + 4 share mask j (w and w >> 4), and the
// four partial sums, weighted 2^j by the mask, recombine exactly.
__device__ __forceinline__ void plane_dot(uint32_t w, const uint32_t* p, int32_t (&a)[4]) {
    const uint32_t hi = w >> 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t m = 0x01010101u << j;
        a[j] = __builtin_amdgcn_sdot4((int)(w & m), (int)p[j], a[j], false);
        a[j] = __builtin_amdgcn_sdot4((int)(hi & m), (int)p[j + 4], a[j], false);
    }
}
__device__ __forceinline__ int32_t plane_combine(const int32_t (&a)[4]) {
    return (8 * a[0] + 4 * a[1] + 2 * a[2] + a[3]) >> 3;
}

// Plane-ordered codes in LDS: block m (32 k) takes 8 words; every 8 blocks are followed
// by 8 words of padding, so that the 8 blocks that one read instruction's threads take
// (8 consecutive k-slices, or blocks 2 kc and 2 kc + 1 of 8 consecutive slices) fall in
// distinct LDS banks.
constexpr int kPlaneRow = 72;
__device__ __forceinline__ int plane_addr(int m) { return (m >> 3) * kPlaneRow + (m & 7) * 8; }

struct Lds {
    uint32_t nat[kDInner / 4];                                         // the codes, natural order
    __attribute__((aligned(16))) uint32_t planes[kDInner / 32 / 8 * kPlaneRow];  // plane order
    float red_max[kWaves], red_ss[kWaves];
    int32_t red_xsum[4];
    int32_t rowred[kWaves][8];      // out_proj: per-wave partial sums of the group's 8 rows
    int32_t tsl[kRank];             // t
    float xs[16], ys[16], Bs[kDState], Cs[kDState];
    float dt_h;
    int flag;
};

// The codes of V float4 pieces per thread (absmax / 127, ties to even), with the
// quantizer's own arithmetic: a reciprocal multiply, the IEEE quotient redone next to
// a tie.
template <int V>
__device__ __forceinline__ void codes_of(const float4 (&v)[V], float amax, uint32_t (&q)[V]) {
    const RowScale rs = row_scale(amax);
#pragma unroll
    for (int i = 0; i < V; ++i) {
        uint32_t n4 = 0;
        q[i] = amax == 0.0f ? 0u : fast_code4(v[i], rs.inv, n4);
        if (amax != 0.0f && (!rs.fast || n4)) q[i] = exact_code4(v[i], rs.s);
    }
}

// Thread t < n_blocks: plane order of block t of the natural codes, and (waves holding
// such threads) the code sum of those blocks into red_xsum[wave].
__device__ __forceinline__ void build_planes(Lds& s, int n_blocks) {
    if ((int)threadIdx.x < n_blocks) {
        uint32_t nw[8], pw[8];
        const uint4 a0 = *reinterpret_cast<const uint4*>(s.nat + 8 * threadIdx.x);
        const uint4 a1 = *reinterpret_cast<const uint4*>(s.nat + 8 * threadIdx.x + 4);
        nw[0] = a0.x; nw[1] = a0.y; nw[2] = a0.z; nw[3] = a0.w;
        nw[4] = a1.x; nw[5] = a1.y; nw[6] = a1.z; nw[7] = a1.w;
        to_planes(nw, pw);
        uint32_t* dst = s.planes + plane_addr(threadIdx.x);
        *reinterpret_cast<uint4*>(dst) = make_uint4(pw[0], pw[1], pw[2], pw[3]);
        *reinterpret_cast<uint4*>(dst + 4) = make_uint4(pw[4], pw[5], pw[6], pw[7]);
        int32_t part = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) part = byte_sum(nw[e], part);
        part = wave_sum(part);
        if ((threadIdx.x & (kWave - 1)) == 0) s.red_xsum[threadIdx.x / kWave] = part;
    }
}

// plane_dot over block m read from LDS (two 16-byte reads)
__device__ __forceinline__ void plane_dot_lds(uint32_t w, const Lds& s, int m, int32_t (&a)[4]) {
    const uint32_t* src = s.planes + plane_addr(m);
    const uint4 p0 = *reinterpret_cast<const uint4*>(src);
    const uint4 p1 = *reinterpret_cast<const uint4*>(src + 4);
    const uint32_t p[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    plane_dot(w, p, a);
}

__global__ __launch_bounds__(kThreads) void decode_layers_kernel(Args a) {
    __shared__ Lds s;
    const int g = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    uint32_t* const ctr = a.ws + kWsCounters;
    float* const xbuf = reinterpret_cast<float*>(a.ws + kWsX);
    float* const zxbuf = reinterpret_cast<float*>(a.ws + kWsZx);
    float* const gbuf = reinterpret_cast<float*>(a.ws + kWsG);
    bool ok = true;

    // ---- this group's fixed roles
    // phase A: rows [ra0, ra1) of in_proj; thread (rr = tid / 8, kc = tid % 8) takes row
    // ra0 + rr, bytes [32 kc, 32 kc + 32) of its packed signs (blocks 8 kc .. 8 kc + 7)
    const int ra0 = (int)(((int64_t)g * kNIn) / kGroups), ra1 = (int)(((int64_t)(g + 1) * kNIn) / kGroups);
    const int rr = tid >> 3, kc = tid & 7;
    const int na = ra0 + rr;
    const bool a_live = na < ra1;
    const int na_c = a_live ? na : ra0;
    // t: thread (r = tid / 32, slice ks = tid % 32): W_B row r, the 16-byte pieces at
    // k = 16 ks + 512 e (e < 4 for in_proj, < 8 for out_proj; interleaved so that the
    // threads of a wave read the codes from distinct LDS banks)
    const int tr = tid >> 5, ks = tid & 31;
    // phase B: head h, channels [16 pb, 16 pb + 16) of it; state thread (p = tid / 32,
    // q = tid % 32) holds values [4 q, 4 q + 4) of channel p
    const int h = g >> 2, pb = g & 3;
    const int sp = tid >> 5, sq = tid & 31;
    const int ch0 = h * kHeadDim + pb * 16;
    // conv thread c < 272: channel ch0 + c (c < 16) or B / C channel c - 16
    const bool conv_live = tid < 16 + 2 * kDState;
    const int conv_c = tid < 16 ? ch0 + tid : kDInner + (tid - 16);  // index into xBC
    // phase C: the group's rows 8 g .. 8 g + 7 of out_proj; thread (crow = tid % 8,
    // cks = tid / 8) takes row 8 g + crow, bytes [8 cks, 8 cks + 8) (blocks 2 cks, 2 cks + 1)
    const int crow = tid & 7, cks = tid >> 3;
    const int nc = 8 * g + crow;

    for (int l = 0; l < a.L; ++l) {
        // ======================= phase A: in_proj =======================
        // weights first (they do not depend on the layer's input)
        const uint8_t* const bitsA = a.in_bits + (int64_t)l * kNIn * (kDModel / 8);
        uint4 wbitsA[2];
#pragma unroll
        for (int e = 0; e < 2; ++e)
            wbitsA[e] = *reinterpret_cast<const uint4*>(bitsA + (int64_t)na_c * (kDModel / 8) + 32 * kc + 16 * e);
        uint4 wbA[4];
        const int8_t* const wbrowA = a.in_wb + ((int64_t)l * kRank + tr) * kDModel + 16 * ks;
#pragma unroll
        for (int e = 0; e < 4; ++e) wbA[e] = *reinterpret_cast<const uint4*>(wbrowA + 512 * e);
        const uint4 waA = *reinterpret_cast<const uint4*>(a.in_wa + ((int64_t)l * kNIn + na_c) * kRank);
        const float saA = a.in_sa[(int64_t)l * kNIn + na_c], swA = a.in_sw[(int64_t)l * kNIn + na_c];
        float sbA[kRank];
#pragma unroll
        for (int r = 0; r < kRank; ++r) sbA[r] = a.in_sb[(int64_t)l * kRank + r];

        // the layer's input: x_in, or the previous layer's out_proj rows
        float4 xv[1];
        if (l == 0) {
            xv[0] = reinterpret_cast<const float4*>(a.x_in)[tid];
        } else {
            ok = group_wait(a, ctr + (3 * (l - 1) + 2) * kCtrStride, kGroups, ok, &s.flag);
            xv[0] = ld4_dev(xbuf + (l & 1) * kDModel, kDModel * 4, 16 * tid);
        }
        // quantize: the absmax, then the codes in natural order
        const float amaxA = group_max(absmax4(xv[0]), s.red_max);
        const float sxA = amaxA == 0.0f ? 0.0f : row_scale(amaxA).s;
        {
            uint32_t q[1];
            codes_of<1>(xv, amaxA, q);
            s.nat[tid] = q[0];
        }
        lds_barrier();
        // t = W_B x_q (16 sdot4 per thread over 64 k, summed over the 32 slices), and the
        // plane order with the code sum (threads of wave 0: 64 blocks)
        {
            int32_t acc = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint4 c = *reinterpret_cast<const uint4*>(s.nat + 4 * ks + 128 * e);
                acc = __builtin_amdgcn_sdot4((int)wbA[e].x, (int)c.x, acc, false);
                acc = __builtin_amdgcn_sdot4((int)wbA[e].y, (int)c.y, acc, false);
                acc = __builtin_amdgcn_sdot4((int)wbA[e].z, (int)c.z, acc, false);
                acc = __builtin_amdgcn_sdot4((int)wbA[e].w, (int)c.w, acc, false);
            }
#pragma unroll
            for (int o = 16; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 32);
            if (ks == 0) s.tsl[tr] = acc;
        }
        build_planes(s, kDModel / 32);
        if (a.trace && g == 0) {
            uint32_t* tr_l = a.trace + (int64_t)l * kTrWords;
            tr_l[kTrXqIn + tid] = s.nat[tid];
            if (tid == 0) tr_l[kTrSx] = __float_as_uint(sxA);
        }
        lds_barrier();
        if (a.trace && g == 0 && tid < kRank) a.trace[(int64_t)l * kTrWords + kTrTIn + tid] = (uint32_t)s.tsl[tid];
        // the group's rows: S = sum of codes under 1 bits over 256 k per thread, summed
        // over the 8 slices
        {
            int32_t pa[4] = {0, 0, 0, 0};
            const uint32_t wsA[8] = {wbitsA[0].x, wbitsA[0].y, wbitsA[0].z, wbitsA[0].w,
                                     wbitsA[1].x, wbitsA[1].y, wbitsA[1].z, wbitsA[1].w};
#pragma unroll
            for (int i = 0; i < 8; ++i) plane_dot_lds(wsA[i], s, 8 * kc + i, pa);
            int32_t S = plane_combine(pa);
#pragma unroll
            for (int o = 4; o > 0; o >>= 1) S += __shfl_xor(S, o, 8);
            if (kc == 0 && a_live) {
                const int32_t acc = 2 * S - s.red_xsum[0];
                float lora = 0.0f;
                const uint32_t words[4] = {waA.x, waA.y, waA.z, waA.w};
#pragma unroll
                for (int r = 0; r < kRank; ++r)
                    lora = fmaf((float)(int8_t)(words[r >> 2] >> (8 * (r & 3))), sbA[r] * (float)s.tsl[r], lora);
                const float y = sxA * fmaf(saA, lora, swA * (float)acc);
                store_f32_dev(y, make_rsrc(zxbuf + (l & 1) * kNIn, kNIn * 4), 4 * na);
                if (a.trace) {
                    a.trace[(int64_t)l * kTrWords + kTrZx + na] = __float_as_uint(y);
                    a.trace[(int64_t)l * kTrWords + kTrAccIn + na] = (uint32_t)acc;
                }
            }
        }
        group_signal(ctr + (3 * l + 0) * kCtrStride);

        // ======================= phase B: Mamba-2 step =======================
        float4* const stp = reinterpret_cast<float4*>(
            a.ssm_state + ((((int64_t)l * kNHeads + h) * kHeadDim + pb * 16 + sp) * kDState + 4 * sq));
        float4 hv = *stp;
        float4 win = make_float4(0.f, 0.f, 0.f, 0.f), cw = win;
        float cb = 0.0f;
        if (conv_live) {
            const int64_t ci = (int64_t)l * kConvDim + conv_c;
            win = reinterpret_cast<const float4*>(a.conv_in)[ci];
            cw = reinterpret_cast<const float4*>(a.conv_w)[ci];
            cb = a.conv_b[ci];
        }
        const float dtb = a.dt_bias[(int64_t)l * kNHeads + h], alog = a.A_log[(int64_t)l * kNHeads + h];
        const float dph = a.Dp[(int64_t)l * kNHeads + h];
        ok = group_wait(a, ctr + (3 * l + 0) * kCtrStride, kGroups, ok, &s.flag);
        {
            const float* zx = zxbuf + (l & 1) * kNIn;
            float xn = 0.0f, zv = 0.0f;
            if (conv_live) xn = ld_dev(zx, kNIn * 4, 4 * (kDInner + conv_c));
            if (tid < 16) zv = ld_dev(zx, kNIn * 4, 4 * (ch0 + tid));
            if (tid == 0) s.dt_h = ld_dev(zx, kNIn * 4, 4 * (kDInner + kConvDim + h));
            if (conv_live) {
                float acc = cb;
                acc = fmaf(cw.x, win.y, acc);
                acc = fmaf(cw.y, win.z, acc);
                acc = fmaf(cw.z, win.w, acc);
                acc = fmaf(cw.w, xn, acc);
                const float act = silu(acc);
                if (tid < 16) {
                    s.xs[tid] = act;
                } else if (tid < 16 + kDState) {
                    s.Bs[tid - 16] = act;
                } else {
                    s.Cs[tid - 16 - kDState] = act;
                }
                if (tid < 16 || g == 0)
                    reinterpret_cast<float4*>(a.conv_out)[(int64_t)l * kConvDim + conv_c] =
                        make_float4(win.y, win.z, win.w, xn);
            }
            lds_barrier();
            const float dt = softplus(s.dt_h + dtb);
            const float dA = expf(-dt * expf(alog));
            const float xp = s.xs[sp];
            const float dtx = dt * xp;
            const float* b = s.Bs + 4 * sq;
            const float* cc = s.Cs + 4 * sq;
            hv.x = fmaf(hv.x, dA, dtx * b[0]);
            hv.y = fmaf(hv.y, dA, dtx * b[1]);
            hv.z = fmaf(hv.z, dA, dtx * b[2]);
            hv.w = fmaf(hv.w, dA, dtx * b[3]);
            *stp = hv;
            float acc = hv.x * cc[0];
            acc = fmaf(hv.y, cc[1], acc);
            acc = fmaf(hv.z, cc[2], acc);
            acc = fmaf(hv.w, cc[3], acc);
#pragma unroll
            for (int o = 16; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 32);
            // y of channel sp goes through LDS to thread sp, which holds its z, gates it
            // and stores g
            if (sq == 0) s.ys[sp] = fmaf(dph, xp, acc);
            lds_barrier();
            if (tid < 16) {
                const float gv = s.ys[tid] * silu(zv);
                store_f32_dev(gv, make_rsrc(gbuf + (l & 1) * kDInner, kDInner * 4), 4 * (ch0 + tid));
            }
        }
        group_signal(ctr + (3 * l + 1) * kCtrStride);

        // ======================= phase C: norm + out_proj =======================
        const float4* const nw4 = reinterpret_cast<const float4*>(a.norm_w + (int64_t)l * kDInner);
        const float4 nwv0 = nw4[2 * tid], nwv1 = nw4[2 * tid + 1];
        uint4 wbC[8];
        const int8_t* const wbrowC = a.out_wb + ((int64_t)l * kRank + tr) * kDInner + 16 * ks;
#pragma unroll
        for (int e = 0; e < 8; ++e) wbC[e] = *reinterpret_cast<const uint4*>(wbrowC + 512 * e);
        const uint2 wbitsC =
            *reinterpret_cast<const uint2*>(a.out_bits + ((int64_t)l * kDModel + nc) * (kDInner / 8) + 8 * cks);
        const uint4 waC = *reinterpret_cast<const uint4*>(a.out_wa + ((int64_t)l * kDModel + nc) * kRank);
        const float saC = a.out_sa[(int64_t)l * kDModel + nc], swC = a.out_sw[(int64_t)l * kDModel + nc];
        float sbC[kRank];
#pragma unroll
        for (int r = 0; r < kRank; ++r) sbC[r] = a.out_sb[(int64_t)l * kRank + r];
        ok = group_wait(a, ctr + (3 * l + 1) * kCtrStride, kGroups, ok, &s.flag);
        float4 ov[2];
        {
            const float* gb = gbuf + (l & 1) * kDInner;
            ov[0] = ld4_dev(gb, kDInner * 4, 32 * tid);
            ov[1] = ld4_dev(gb, kDInner * 4, 32 * tid + 16);
            float ss = 0.0f;
            ss = fmaf(ov[0].x, ov[0].x, ss);
            ss = fmaf(ov[0].y, ov[0].y, ss);
            ss = fmaf(ov[0].z, ov[0].z, ss);
            ss = fmaf(ov[0].w, ov[0].w, ss);
            ss = fmaf(ov[1].x, ov[1].x, ss);
            ss = fmaf(ov[1].y, ov[1].y, ss);
            ss = fmaf(ov[1].z, ov[1].z, ss);
            ss = fmaf(ov[1].w, ov[1].w, ss);
            const float tot = group_sum_fixed(ss, s.red_ss);
            const float r = 1.0f / sqrtf(tot / (float)kDInner + a.eps);
            ov[0] = make_float4(ov[0].x * r * nwv0.x, ov[0].y * r * nwv0.y, ov[0].z * r * nwv0.z,
                                ov[0].w * r * nwv0.w);
            ov[1] = make_float4(ov[1].x * r * nwv1.x, ov[1].y * r * nwv1.y, ov[1].z * r * nwv1.z,
                                ov[1].w * r * nwv1.w);
            if (a.trace && (tid >> 1) == g) {
                uint32_t* tr_o = a.trace + (int64_t)l * kTrWords + kTrOut + 8 * tid;
                tr_o[0] = __float_as_uint(ov[0].x);
                tr_o[1] = __float_as_uint(ov[0].y);
                tr_o[2] = __float_as_uint(ov[0].z);
                tr_o[3] = __float_as_uint(ov[0].w);
                tr_o[4] = __float_as_uint(ov[1].x);
                tr_o[5] = __float_as_uint(ov[1].y);
                tr_o[6] = __float_as_uint(ov[1].z);
                tr_o[7] = __float_as_uint(ov[1].w);
            }
        }
        // quantize the 4096 values (thread tid holds elements 8 tid .. 8 tid + 7)
        const float amaxC = group_max(fmaxf(absmax4(ov[0]), absmax4(ov[1])), s.red_max);
        const float sxC = amaxC == 0.0f ? 0.0f : row_scale(amaxC).s;
        {
            uint32_t q[2];
            codes_of<2>(ov, amaxC, q);
            *reinterpret_cast<uint2*>(s.nat + 2 * tid) = make_uint2(q[0], q[1]);
        }
        lds_barrier();
        // t = W_B x_q over 4096 k (128 k per thread), and the plane order with the code
        // sum (threads of waves 0 and 1: 128 blocks)
        {
            int32_t acc = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint4 c = *reinterpret_cast<const uint4*>(s.nat + 4 * ks + 128 * e);
                acc = __builtin_amdgcn_sdot4((int)wbC[e].x, (int)c.x, acc, false);
                acc = __builtin_amdgcn_sdot4((int)wbC[e].y, (int)c.y, acc, false);
                acc = __builtin_amdgcn_sdot4((int)wbC[e].z, (int)c.z, acc, false);
                acc = __builtin_amdgcn_sdot4((int)wbC[e].w, (int)c.w, acc, false);
            }
#pragma unroll
            for (int o = 16; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 32);
            if (ks == 0) s.tsl[tr] = acc;
        }
        build_planes(s, kDInner / 32);
        if (a.trace && g == 0) {
            uint32_t* tr_l = a.trace + (int64_t)l * kTrWords;
            tr_l[kTrXqOut + 2 * tid] = s.nat[2 * tid];
            tr_l[kTrXqOut + 2 * tid + 1] = s.nat[2 * tid + 1];
            if (tid == 0) tr_l[kTrSx + 1] = __float_as_uint(sxC);
        }
        lds_barrier();
        if (a.trace && g == 0 && tid < kRank) a.trace[(int64_t)l * kTrWords + kTrTOut + tid] = (uint32_t)s.tsl[tid];
        // row 8 g + crow: 64 k per thread (blocks 2 cks, 2 cks + 1), summed over the 8
        // slices of the wave (lanes crow + 8 i) and then over the 8 waves
        {
            int32_t pa[4] = {0, 0, 0, 0};
            plane_dot_lds(wbitsC.x, s, 2 * cks, pa);
            plane_dot_lds(wbitsC.y, s, 2 * cks + 1, pa);
            int32_t S = plane_combine(pa);
            S += __shfl_xor(S, 8, kWave);
            S += __shfl_xor(S, 16, kWave);
            S += __shfl_xor(S, 32, kWave);
            if (lane < 8) s.rowred[wave][lane] = S;
        }
        lds_barrier();
        if (tid < 8) {
            int32_t S = 0;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) S += s.rowred[w][tid];
            const int32_t acc = 2 * S - (s.red_xsum[0] + s.red_xsum[1]);
            float lora = 0.0f;
            const uint32_t words[4] = {waC.x, waC.y, waC.z, waC.w};
#pragma unroll
            for (int r = 0; r < kRank; ++r)
                lora = fmaf((float)(int8_t)(words[r >> 2] >> (8 * (r & 3))), sbC[r] * (float)s.tsl[r], lora);
            const float y = sxC * fmaf(saC, lora, swC * (float)acc);
            if (l + 1 < a.L) {
                store_f32_dev(y, make_rsrc(xbuf + ((l + 1) & 1) * kDModel, kDModel * 4), 4 * nc);
            } else {
                a.x_out[nc] = y;
            }
            if (a.trace) {
                a.trace[(int64_t)l * kTrWords + kTrXn + nc] = __float_as_uint(y);
                a.trace[(int64_t)l * kTrWords + kTrAccOut + nc] = (uint32_t)acc;
            }
        }
        group_signal(ctr + (3 * l + 2) * kCtrStride);
    }

    // the last group to finish clears the counters for the next call
    if (tid == 0) {
        uint32_t* const done = ctr + 3 * kMaxLayers * kCtrStride;
        const uint32_t prev = __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (prev == kGroups - 1) {
            for (int i = 0; i < 3 * a.L; ++i)
                __hip_atomic_store(ctr + i * kCtrStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

}  // namespace decode

}  // namespace dfssm

namespace dfssm {

namespace {

// The no-allocation entry point's workspace: one array per GPU, held until the process
// ends.  In host code `scratch` only names the variable; its device address comes from
// hipGetSymbolAddress, once per device.
__device__ __align__(256) uint32_t scratch[decode::kWsWords];

__global__ void zero_words_kernel(uint32_t* p, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
uint32_t* scratch_ptr[kMaxDevices];

}  // namespace

// The current device's scratch array: its address is taken (and its counters cleared on
// `stream`) the first time a device is seen.  nullptr on a HIP error.
uint32_t* decode_layers_scratch(hipStream_t stream) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
        // the counters must start at zero (every call leaves them so)
        zero_words_kernel<<<16, 256, 0, stream>>>(static_cast<uint32_t*>(ptr), decode::kWsX);
        if (hipGetLastError() != hipSuccess) return nullptr;
        scratch_ptr[dev] = static_cast<uint32_t*>(ptr);
    }
    return scratch_ptr[dev];
}

size_t decode_layers_workspace_bytes() { return (size_t)decode::kWsWords * 4; }
int64_t decode_layers_trace_words() { return decode::kTrWords; }
int64_t decode_layers_max_layers() { return decode::kMaxLayers; }

// One cooperative launch of the persistent grid: one 512-thread group per CU, all 256
// co-resident (the runtime refuses a cooperative launch that does not fit).
// hipErrorNotSupported: this device cannot hold the grid.
hipError_t launch_decode_layers(const decode::Args& a, hipStream_t stream) {
    int dev = 0, cus = 0, coop = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorNoDevice;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess)
        return hipErrorNotSupported;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode::decode_layers_kernel, decode::kThreads, 0) !=
        hipSuccess)
        return hipErrorNotSupported;
    if (!coop || (int64_t)cus * per_cu < decode::kGroups) return hipErrorNotSupported;
    decode::Args args = a;
    void* params[] = {&args};
    const hipError_t e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(decode::decode_layers_kernel),
                                                    dim3(decode::kGroups), dim3(decode::kThreads), params, 0, stream);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

}  // namespace dfssm
