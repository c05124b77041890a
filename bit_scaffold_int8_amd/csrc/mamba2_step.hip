// mamba2_step.hip -- the Mamba-2 decode step between in_proj and out_proj (gfx950).
//
// DF-SSM technical summary (gist.science), section 2C "Optimized Inference Pipeline",
// Stateful Ops: the stateful shift register (the causal convolution) and the SSM
// recurrence with a reduction over the state.  The arithmetic is the published
// Mamba-2 single-token step (Mamba-2 1.3B: 64 heads of 64 channels, state size 128,
// one group, convolution width 4), for S independent sequences:
//   in_proj output row = [z (d_inner) | xBC (d_inner + 2 d_state) | dt (nheads)]
//   window <- [window[1..3], xBC];  xBC' = silu(sum_j w[c, j] window[c, j] + b[c])
//   x | B | C = xBC';  dt = softplus(dt + dt_bias);  dA = exp(-dt exp(A_log))
//   state[h, p, n] <- state dA + (dt x[h, p]) B[n];  y = sum_n state C[n] + D[h] x
//   out = g / sqrt(mean(g^2) + eps) w,  g = y silu(z)        (out_proj's input)
//
// Two launches, both HBM-bound at batch (the state is 2 MB of fp32 per sequence and
// layer, read and written once):
//  * mamba2_ssm_kernel: one 256-thread group per (16 channels of a head, sequence).
//    It runs the convolution for its 16 x channels and for B and C (every group of
//    the sequence needs them; one group writes their new windows), then updates its
//    16 x 128 slice of the state: each thread owns 8 consecutive state values of one
//    channel (two 16-byte loads and stores; a wave covers 2 KB contiguously), and the
//    16 threads of a channel sum their C-weighted parts with lane shuffles.  The
//    gated value g is written to `out`.
//  * mamba2_gated_norm_kernel: one group per sequence: the mean square of g in a
//    fixed order (per thread, then a tree in LDS), then out = g r w in place.
// The convolution windows are double-buffered (in and out), because every group of
// a sequence reads the B and C windows that one of them rewrites; the SSM state is
// updated in place, each value by the one thread that reads it.
#include "device_common.h"

namespace dfssm {

namespace {

constexpr int kHeadDim = 64, kDState = 128, kDConv = 4;
static_assert(kDConv == 4, "a convolution window is one float4");
constexpr int kSsmThreads = 256;
constexpr int kNormThreads = 256;

__device__ __forceinline__ float silu(float v) { return v / (1.0f + expf(-v)); }

// softplus with the usual identity above 20
__device__ __forceinline__ float softplus(float v) { return v > 20.0f ? v : log1pf(expf(v)); }

// kPBlock channels of a head per group; each channel's 128 state values are split over
// kTPC = 256 / kPBlock consecutive lanes, kV = 128 / kTPC values (kV / 4 16-byte pieces)
// each.
template <int kPBlock>
__global__ __launch_bounds__(kSsmThreads) void mamba2_ssm_kernel(
    const float* __restrict__ zxbcdt, int nheads, const float* __restrict__ conv_in, float* __restrict__ conv_out,
    float* __restrict__ ssm_state, const float* __restrict__ conv_w, const float* __restrict__ conv_b,
    const float* __restrict__ dt_bias, const float* __restrict__ A_log, const float* __restrict__ Dp,
    float* __restrict__ out) {
    constexpr int kTPC = kSsmThreads / kPBlock, kV = kDState / kTPC, kV4 = kV / 4;
    static_assert(kTPC * kPBlock == kSsmThreads && kV * kTPC == kDState && kV % 4 == 0, "state split");
    const int d_inner = nheads * kHeadDim;
    const int conv_dim = d_inner + 2 * kDState;
    const int64_t width = (int64_t)d_inner + conv_dim + nheads;
    constexpr int blocks_per_head = kHeadDim / kPBlock;
    const int h = blockIdx.x / blocks_per_head, pb = blockIdx.x % blocks_per_head;
    const int64_t s = blockIdx.y;
    const float* const row = zxbcdt + s * width;
    const int tid = threadIdx.x;

    __shared__ float xs[kPBlock], Bs[kDState], Cs[kDState];

    // this thread's kV state values (channel p of the block, values [kV q, kV q + kV))
    // and the head's dt go out first: they do not depend on the convolution, so their
    // latency overlaps its loads
    const int p = tid / kTPC, q = tid % kTPC;
    float4* const st = reinterpret_cast<float4*>(
        ssm_state + ((s * nheads + h) * kHeadDim + pb * kPBlock + p) * (int64_t)kDState + kV * q);
    float4 hv[kV4];
#pragma unroll
    for (int i = 0; i < kV4; ++i) hv[i] = st[i];
    const float dt_raw = row[d_inner + conv_dim + h] + dt_bias[h];
    const float a_log = A_log[h];

    // convolution: this group's kPBlock x channels, then B and C
    for (int idx = tid; idx < kPBlock + 2 * kDState; idx += kSsmThreads) {
        const int c = idx < kPBlock ? h * kHeadDim + pb * kPBlock + idx : d_inner + (idx - kPBlock);
        const int64_t sc = s * conv_dim + c;
        const float4 win = reinterpret_cast<const float4*>(conv_in)[sc];
        const float xn = row[d_inner + c];
        const float4 w = reinterpret_cast<const float4*>(conv_w)[c];
        float acc = conv_b[c];
        acc = fmaf(w.x, win.y, acc);
        acc = fmaf(w.y, win.z, acc);
        acc = fmaf(w.z, win.w, acc);
        acc = fmaf(w.w, xn, acc);
        const float act = silu(acc);
        if (idx < kPBlock) {
            xs[idx] = act;
        } else if (idx < kPBlock + kDState) {
            Bs[idx - kPBlock] = act;
        } else {
            Cs[idx - kPBlock - kDState] = act;
        }
        if (idx < kPBlock || blockIdx.x == 0) reinterpret_cast<float4*>(conv_out)[sc] = make_float4(win.y, win.z, win.w, xn);
    }

    const float dt = softplus(dt_raw);
    const float dA = expf(-dt * expf(a_log));
    __syncthreads();

    const float xp = xs[p];
    const float dtx = dt * xp;
    const float* const b = Bs + kV * q;
    const float* const cc = Cs + kV * q;
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < kV4; ++i) {
        float4 v = hv[i];
        v.x = fmaf(v.x, dA, dtx * b[4 * i + 0]);
        v.y = fmaf(v.y, dA, dtx * b[4 * i + 1]);
        v.z = fmaf(v.z, dA, dtx * b[4 * i + 2]);
        v.w = fmaf(v.w, dA, dtx * b[4 * i + 3]);
        st[i] = v;
        acc = i == 0 ? v.x * cc[0] : fmaf(v.x, cc[4 * i], acc);
        acc = fmaf(v.y, cc[4 * i + 1], acc);
        acc = fmaf(v.z, cc[4 * i + 2], acc);
        acc = fmaf(v.w, cc[4 * i + 3], acc);
    }
    // the kTPC threads of channel p are kTPC consecutive lanes
#pragma unroll
    for (int off = kTPC / 2; off > 0; off /= 2) acc += __shfl_xor(acc, off, kTPC);
    if (q == 0) {
        const int ch = h * kHeadDim + pb * kPBlock + p;
        const float y = fmaf(Dp[h], xp, acc);
        out[s * d_inner + ch] = y * silu(row[ch]);
    }
}

__global__ __launch_bounds__(kNormThreads) void mamba2_gated_norm_kernel(float* __restrict__ out, int d_inner,
                                                                          const float* __restrict__ w, float eps) {
    __shared__ float part[kNormThreads];
    float4* const g = reinterpret_cast<float4*>(out + (int64_t)blockIdx.x * d_inner);
    const float4* const w4 = reinterpret_cast<const float4*>(w);
    const int n4 = d_inner / 4;
    float ss = 0.0f;
    for (int i = threadIdx.x; i < n4; i += kNormThreads) {
        const float4 v = g[i];
        ss = fmaf(v.x, v.x, ss);
        ss = fmaf(v.y, v.y, ss);
        ss = fmaf(v.z, v.z, ss);
        ss = fmaf(v.w, v.w, ss);
    }
    part[threadIdx.x] = ss;
    __syncthreads();
    for (int half = kNormThreads / 2; half > 0; half /= 2) {
        if ((int)threadIdx.x < half) part[threadIdx.x] += part[threadIdx.x + half];
        __syncthreads();
    }
    const float r = 1.0f / sqrtf(part[0] / (float)d_inner + eps);
    for (int i = threadIdx.x; i < n4; i += kNormThreads) {
        float4 v = g[i];
        const float4 ww = w4[i];
        v.x = v.x * r * ww.x;
        v.y = v.y * r * ww.y;
        v.z = v.z * r * ww.z;
        v.w = v.w * r * ww.w;
        g[i] = v;
    }
}

}  // namespace

bool mamba2_step_supported(int64_t nheads, int64_t headdim, int64_t d_state) {
    return headdim == kHeadDim && d_state == kDState && nheads >= 1 && nheads <= 1024;
}

hipError_t launch_mamba2_step(const float* zxbcdt, int64_t S, int nheads, const float* conv_in, float* conv_out,
                              float* ssm_state, const float* conv_w, const float* conv_b, const float* dt_bias,
                              const float* A_log, const float* D, const float* norm_w, float eps, float* out,
                              hipStream_t stream) {
    // 16 channels per group (4 groups per head): measured against a whole head (64) and
    // 8 channels per group, it streams the state fastest at 1, 64 and 512 sequences
    const dim3 grid((unsigned)(nheads * (kHeadDim / 16)), (unsigned)S);
    mamba2_ssm_kernel<16><<<grid, kSsmThreads, 0, stream>>>(zxbcdt, nheads, conv_in, conv_out, ssm_state, conv_w,
                                                           conv_b, dt_bias, A_log, D, out);
    mamba2_gated_norm_kernel<<<dim3((unsigned)S), kNormThreads, 0, stream>>>(out, nheads * kHeadDim, norm_w, eps);
    return hipGetLastError();
}

}  // namespace dfssm
