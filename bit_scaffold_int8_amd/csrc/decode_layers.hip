// decode_layers.hip -- the whole per-token decode of a stack of DF-SSM layers for one
// sequence in ONE kernel launch (gfx950).
//
// DF-SSM technical summary (gist.science), section 2C "Optimized Inference Pipeline":
// the entire 48-layer forward pass is captured as one CUDA graph because launch overhead
// decides batch-1 speed; the layer is in_proj (1-bit scaffold + int8 LoRA) -> the
// stateful convolution and SSM recurrence -> out_proj.  Here the launches go away
// altogether: one persistent grid (one 512-thread group per CU, co-resident by a
// cooperative launch) walks all layers, and the dependencies between the three steps
// of a layer become tagged exchanges (below):
//
//   phase A (in_proj, K 2048 -> N 8512): every group quantizes the layer's input x
//     (absmax / 127, ties to even), computes t = W_B x_q for itself, and produces its
//     33 or 34 rows of zxbcdt.
//   phase B (Mamba-2 step): group g owns 16 channels of head g / 4; it reads its z, x,
//     dt and the shared B, C, runs the convolution, the state update and the gate,
//     g = y silu(z), for its channels.
//   phase C (gated RMS norm + out_proj, K 4096 -> N 2048): every group reads all of g,
//     forms the norm (the mean square in one fixed order, so all groups get the same
//     bits), quantizes the result, computes t, and produces its 8 rows of the next
//     layer's input.
//
// Exchanges: each produced value travels with a tag in one 8-byte device-scope store
// (write-through, coherent across the XCDs' L2s without cache-maintenance fences; an
// aligned 8-byte store is one access, so a reader that sees the tag sees the value
// stored with it).  The tag names the call, the layer and the phase; readers poll the
// pairs they need until the tags are current -- no counters, no waiting for store
// completions.  The slots are double-buffered by layer parity: a slot is written again
// two layers later, which the data dependencies order after every read of it.  Every
// wait is bounded: past the poll limit, or once any group has reported a failure, it
// gives up and ORs a bit into the caller's status word; the kernel always runs to the
// end.  The last group to finish advances the call counter that the tags carry.
//
// Weights do not depend on activations, so each group issues the loads of its next
// phase's packed signs, W_B slice, epilogue operands and state slice before it waits:
// the HBM stream overlaps the wait.
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
constexpr int kCtrStride = 16;                               // words per counter slot (64 B)
constexpr int kMaxLayers = 64;
constexpr int kStatusTimeout = 1, kStatusGaveUp = 2;

// workspace layout (4-byte words): the count of groups done (the last one resets it),
// the call counter (it tags every exchanged value), then the exchange slots as
// (value, tag) pairs, double-buffered by layer parity
constexpr int kWsDone = 0;
constexpr int kWsGen = kCtrStride;
constexpr int kWsX = 2 * kCtrStride;                         // x      [2][2048] pairs
constexpr int kWsZx = kWsX + 2 * 2 * kDModel;                // zxbcdt [2][8512] pairs
constexpr int kWsG = kWsZx + 2 * 2 * kNIn;                   // g      [2][4096] pairs
constexpr int kWsWords = kWsG + 2 * 2 * kDInner;

// trace layout per layer (4-byte words)
constexpr int kTrZx = 0, kTrOut = kTrZx + kNIn, kTrXn = kTrOut + kDInner, kTrAccIn = kTrXn + kDModel,
              kTrAccOut = kTrAccIn + kNIn, kTrXqIn = kTrAccOut + kDModel, kTrXqOut = kTrXqIn + kDModel / 4,
              kTrTIn = kTrXqOut + kDInner / 4, kTrTOut = kTrTIn + kRank, kTrSx = kTrTOut + kRank,
              kTrWords = kTrSx + 16;


__device__ __forceinline__ float silu(float v) { return v / (1.0f + expf(-v)); }
__device__ __forceinline__ float softplus(float v) { return v > 20.0f ? v : log1pf(expf(v)); }

// ---- tagged exchanges (device scope: coherent across the XCDs' L2s)
typedef int v2i_t __attribute__((ext_vector_type(2)));

// The tag of the values phase `phase` of layer l writes in call `gen` (never 0, so a
// zeroed slot never passes; L <= 64 keeps the layers of one call apart).
__device__ __forceinline__ uint32_t xtag(uint32_t gen, int l, int phase) {
    return ((gen + 1u) << 8) + 4u * (uint32_t)l + (uint32_t)phase;
}

// One value and its tag, in one 8-byte store.
__device__ __forceinline__ void store_pair(float v, uint32_t tag, __amdgpu_buffer_rsrc_t r, int byte_off) {
    const v2i_t q = {(int)__float_as_uint(v), (int)tag};
    __builtin_amdgcn_raw_buffer_store_b64(q, r, byte_off, 0, kAuxDeviceScope);
}

// One round of a bounded wait: counts it, gives up past the poll limit or once the
// status word shows a failure elsewhere (checked every 16 rounds; either way this
// thread ORs its reason into the status word), else sleeps briefly.  False: give up.
__device__ __forceinline__ bool poll_round(const Args& a, int64_t& n) {
    ++n;
    if (n >= a.spin_limit) {
        __hip_atomic_fetch_or(a.status, kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return false;
    }
    if ((n & 15) == 15 && __hip_atomic_load(a.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
        __hip_atomic_fetch_or(a.status, kStatusGaveUp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return false;
    }
    __builtin_amdgcn_s_sleep(1);
    return true;
}

// P consecutive 16-byte pieces (two pairs each) from byte offset `off`, all written by
// one producer at one moment: the first piece is polled until both its tags equal
// `want`, then the rest are read together (and any still stale is polled alone).
// Returns false once this thread has given up (its later waits then only read).
template <int P>
__device__ bool read_pieces(const Args& a, __amdgpu_buffer_rsrc_t r, int off, uint32_t want, float (&v)[2 * P],
                            bool ok) {
    int64_t n = 0;
    for (;;) {
        const v4i q = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAuxDeviceScope);
        v[0] = __int_as_float(q[0]);
        v[1] = __int_as_float(q[2]);
        if (((uint32_t)q[1] == want && (uint32_t)q[3] == want) || !ok) break;
        ok = poll_round(a, n);
    }
    v4i q[P > 1 ? P - 1 : 1];
#pragma unroll
    for (int p = 1; p < P; ++p) q[p - 1] = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * p, 0, kAuxDeviceScope);
#pragma unroll
    for (int p = 1; p < P; ++p) {
        for (;;) {
            v[2 * p] = __int_as_float(q[p - 1][0]);
            v[2 * p + 1] = __int_as_float(q[p - 1][2]);
            if (((uint32_t)q[p - 1][1] == want && (uint32_t)q[p - 1][3] == want) || !ok) break;
            ok = poll_round(a, n);
            q[p - 1] = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * p, 0, kAuxDeviceScope);
        }
    }
    return ok;
}

// One pair, polled until its tag equals `want`.
__device__ bool read_pair(const Args& a, __amdgpu_buffer_rsrc_t r, int off, uint32_t want, float& v, bool ok) {
    int64_t n = 0;
    for (;;) {
        const v2i_t q = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kAuxDeviceScope);
        v = __int_as_float(q[0]);
        if ((uint32_t)q[1] == want || !ok) break;
        ok = poll_round(a, n);
    }
    return ok;
}

// ---- cross-lane sums on the DPP paths (the helpers in device_common.h): the kernel's
// critical path runs ~45 such steps a layer.  The patterns are fixed, so every group
// forms the same float sums bit for bit.

// Sum over each group of 8 lanes (every lane of the 8 gets it).
__device__ __forceinline__ int32_t sum8(int32_t v) {
    v += dpp_i<kDppXor1>(v);
    v += dpp_i<kDppXor2>(v);
    v += dpp_i<kDppHalfMirror>(v);
    return v;
}
// Sums over each half-wave of 32 lanes: lanes 16..31 get lanes 0..31's, 48..63 get
// 32..63's (T: int32_t or float; float sums in one fixed order).
__device__ __forceinline__ int32_t sum32_hi(int32_t v) {
    v = sum8(v);
    v += dpp_i<kDppMirror>(v);
    v += dpp_i<kDppBcast15, 0xA>(v);
    return v;
}
__device__ __forceinline__ float sum32_hi(float v) {
    v += dpp_f<kDppXor1>(v);
    v += dpp_f<kDppXor2>(v);
    v += dpp_f<kDppHalfMirror>(v);
    v += dpp_f<kDppMirror>(v);
    v += dpp_f<kDppBcast15, 0xA>(v);
    return v;
}
// The wave's float sum in one fixed order, uniform.
__device__ __forceinline__ float wave_sum_fixed(float v) {
    v = sum32_hi(v);
    v += dpp_f<kDppBcast31, 0xC>(v);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
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
    v = wave_sum_fixed(v);
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
    int32_t rowred[kWaves][4][8];   // out_proj: per-(wave, 16-lane row) sums of the group's 8 rows
    int32_t tsl[kRank];             // t
    float xs[16], ys[16], Bs[kDState], Cs[kDState];
    float dt_h;
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
    // the exchange slots, (value, tag) pairs; slot parity p of each at p * (its pairs)
    const __amdgpu_buffer_rsrc_t x_rsrc = make_rsrc(a.ws + kWsX, 2 * 2 * kDModel * 4);
    const __amdgpu_buffer_rsrc_t zx_rsrc = make_rsrc(a.ws + kWsZx, 2 * 2 * kNIn * 4);
    const __amdgpu_buffer_rsrc_t g_rsrc = make_rsrc(a.ws + kWsG, 2 * 2 * kDInner * 4);
    // this call's number (every group reads it before any group can advance it)
    const uint32_t gen = __hip_atomic_load(a.ws + kWsGen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
            // x[4 tid .. 4 tid + 3], from the group that wrote rows 8 (tid / 2) ..
            float v[4];
            ok = read_pieces<2>(a, x_rsrc, 8 * ((l & 1) * kDModel + 4 * tid), xtag(gen, l - 1, 2) + a.target_bias,
                                v, ok);
            xv[0] = make_float4(v[0], v[1], v[2], v[3]);
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
            acc = sum32_hi(acc);
            if (ks == 31) s.tsl[tr] = acc;
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
            S = sum8(S);
            if (kc == 0 && a_live) {
                const int32_t acc = 2 * S - s.red_xsum[0];
                float lora = 0.0f;
                const uint32_t words[4] = {waA.x, waA.y, waA.z, waA.w};
#pragma unroll
                for (int r = 0; r < kRank; ++r)
                    lora = fmaf((float)(int8_t)(words[r >> 2] >> (8 * (r & 3))), sbA[r] * (float)s.tsl[r], lora);
                const float y = sxA * fmaf(saA, lora, swA * (float)acc);
                store_pair(y, xtag(gen, l, 0), zx_rsrc, 8 * ((l & 1) * kNIn + na));
                if (a.trace) {
                    a.trace[(int64_t)l * kTrWords + kTrZx + na] = __float_as_uint(y);
                    a.trace[(int64_t)l * kTrWords + kTrAccIn + na] = (uint32_t)acc;
                }
            }
        }
        lds_barrier();  // the phase's LDS is free for the next

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
        {
            // this group's rows of zxbcdt, each polled until phase A of this layer wrote it
            const uint32_t want = xtag(gen, l, 0) + a.target_bias;
            const int zx0 = (l & 1) * kNIn;
            float xn = 0.0f, zv = 0.0f;
            if (conv_live) ok = read_pair(a, zx_rsrc, 8 * (zx0 + kDInner + conv_c), want, xn, ok);
            if (tid < 16) ok = read_pair(a, zx_rsrc, 8 * (zx0 + ch0 + tid), want, zv, ok);
            if (tid == 0) {
                float dtv = 0.0f;
                ok = read_pair(a, zx_rsrc, 8 * (zx0 + kDInner + kConvDim + h), want, dtv, ok);
                s.dt_h = dtv;
            }
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
            acc = sum32_hi(acc);
            // y of channel sp goes through LDS to thread sp, which holds its z, gates it
            // and stores g
            if (sq == 31) s.ys[sp] = fmaf(dph, xp, acc);
            lds_barrier();
            if (tid < 16) {
                const float gv = s.ys[tid] * silu(zv);
                store_pair(gv, xtag(gen, l, 1), g_rsrc, 8 * ((l & 1) * kDInner + ch0 + tid));
            }
        }
        lds_barrier();  // the phase's LDS is free for the next

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
        float4 ov[2];
        {
            // g[8 tid .. 8 tid + 7], from the group that owns channels 16 (tid / 2) ..
            float v[8];
            ok = read_pieces<4>(a, g_rsrc, 8 * ((l & 1) * kDInner + 8 * tid), xtag(gen, l, 1) + a.target_bias, v,
                                ok);
            ov[0] = make_float4(v[0], v[1], v[2], v[3]);
            ov[1] = make_float4(v[4], v[5], v[6], v[7]);
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
            acc = sum32_hi(acc);
            if (ks == 31) s.tsl[tr] = acc;
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
        // row 8 g + crow: 64 k per thread (blocks 2 cks, 2 cks + 1), summed over the 2
        // slices of each 16-lane row (lanes crow, crow + 8), then through LDS over the
        // 4 rows of each of the 8 waves
        {
            int32_t pa[4] = {0, 0, 0, 0};
            plane_dot_lds(wbitsC.x, s, 2 * cks, pa);
            plane_dot_lds(wbitsC.y, s, 2 * cks + 1, pa);
            int32_t S = plane_combine(pa);
            S += dpp_i<kDppRowRor8>(S);
            if ((lane & 15) < 8) s.rowred[wave][lane >> 4][lane & 7] = S;
        }
        lds_barrier();
        if (tid < 8) {
            int32_t S = 0;
#pragma unroll
            for (int w = 0; w < kWaves; ++w)
#pragma unroll
                for (int q = 0; q < 4; ++q) S += s.rowred[w][q][tid];
            const int32_t acc = 2 * S - (s.red_xsum[0] + s.red_xsum[1]);
            float lora = 0.0f;
            const uint32_t words[4] = {waC.x, waC.y, waC.z, waC.w};
#pragma unroll
            for (int r = 0; r < kRank; ++r)
                lora = fmaf((float)(int8_t)(words[r >> 2] >> (8 * (r & 3))), sbC[r] * (float)s.tsl[r], lora);
            const float y = sxC * fmaf(saC, lora, swC * (float)acc);
            if (l + 1 < a.L) {
                store_pair(y, xtag(gen, l, 2), x_rsrc, 8 * (((l + 1) & 1) * kDModel + nc));
            } else {
                a.x_out[nc] = y;
            }
            if (a.trace) {
                a.trace[(int64_t)l * kTrWords + kTrXn + nc] = __float_as_uint(y);
                a.trace[(int64_t)l * kTrWords + kTrAccOut + nc] = (uint32_t)acc;
            }
        }
        lds_barrier();  // the phase's LDS is free for the next
    }

    // the last group to finish advances the call counter (every group has read all it
    // needs by then) and clears the done count for the next call
    if (tid == 0) {
        uint32_t* const done = a.ws + kWsDone;
        const uint32_t prev = __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (prev == kGroups - 1) {
            __hip_atomic_store(a.ws + kWsGen, gen + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
        // the array starts zeroed (the done count, the call counter, no current tags)
        zero_words_kernel<<<64, 256, 0, stream>>>(static_cast<uint32_t*>(ptr), decode::kWsWords);
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
