// api.hip -- the C ABI (include/dfssm.h): host-side validation and kernel dispatch.
//
// Every entry point validates its arguments before enqueuing anything, launches on
// the caller's stream, never synchronizes and allocates nothing.
#include "dfssm.h"

#include <hip/hip_runtime.h>
#include <stdlib.h>

namespace dfssm {
hipError_t launch_quantize_act(const float* x, int64_t M, int64_t K, int8_t* x_q, float* s_x,
                               hipStream_t stream);
int quantize_lora_tokens_per_group(int64_t K);
hipError_t launch_quantize_lora_down(const float* x, int64_t M, int64_t K, const int8_t* w_b, int rank,
                                     int8_t* x_q, float* s_x, int32_t* t, int64_t batch, hipStream_t stream);
hipError_t launch_lora_down(const int8_t* x_q, int64_t M, int64_t K, const int8_t* w_b, int32_t* t,
                            int64_t batch, hipStream_t stream);
hipError_t launch_gemv(const int8_t* x_q, const float* s_x, int M, int64_t N, int64_t K,
                       const uint8_t* w_bits, const float* s_w, const int8_t* w_a, const float* s_a,
                       const int8_t* w_b, const float* s_b, const int32_t* t, int32_t* t_out, int rank, float* y,
                       int32_t* acc_dbg, int64_t batch, hipStream_t stream);
hipError_t launch_gemm_mfma(const int8_t* x_q, const float* s_x, int64_t M, int64_t N, int64_t K,
                            const uint8_t* w_bits, const float* s_w, const int8_t* w_a, const float* s_a,
                            const int8_t* w_b, const float* s_b, const int32_t* t, int32_t* t_out, int rank,
                            float* y, int32_t* acc_dbg, int64_t batch, hipStream_t stream);
bool decode_fused_supported(int64_t M, int64_t K);
hipError_t launch_decode_fused(const float* x, int M, int64_t N, int64_t K, const uint8_t* w_bits,
                               const float* s_w, const int8_t* w_a, const float* s_a, const int8_t* w_b,
                               const float* s_b, int rank, int8_t* x_q, float* s_x, int32_t* t, float* y,
                               int32_t* acc_dbg, int64_t batch, hipStream_t stream);
bool int8_head_supported(int64_t M, int64_t K);
hipError_t launch_int8_head(const int8_t* x_q, const float* s_x, int M, int64_t N, int64_t K, const int8_t* e,
                            const float* s_e, float* y, int32_t* acc_dbg, int64_t batch, hipStream_t stream);
hipError_t launch_embedding_lookup(const int32_t* tokens, int64_t T, const int8_t* e, const float* s_e, int64_t V,
                                   int64_t K, float* out, hipStream_t stream);
bool mamba2_step_supported(int64_t nheads, int64_t headdim, int64_t d_state);
hipError_t launch_mamba2_step(const float* zxbcdt, int64_t S, int nheads, const float* conv_in, float* conv_out,
                              float* ssm_state, const float* conv_w, const float* conv_b, const float* dt_bias,
                              const float* A_log, const float* D, const float* norm_w, float eps, float* out,
                              hipStream_t stream);
bool density_field_supported(int64_t d_state);
hipError_t launch_density_encode(const float* state, int64_t R, int64_t D, uint32_t* field, float* scale,
                                 float* state_out, hipStream_t stream);
hipError_t launch_density_decode(const uint32_t* field, const float* scale, int64_t R, int64_t D, float* state,
                                 hipStream_t stream);
size_t decode_layers_workspace_bytes();
uint32_t* decode_layers_scratch(hipStream_t stream);
int64_t decode_layers_trace_words();
int64_t decode_layers_max_layers();
bool prefill_supported(int64_t M, int64_t N, int64_t K);
int prefill_num_cfgs();
void prefill_plan_query(int64_t M, int64_t N, int64_t K, int64_t batch, int* main_cfg, int* tail_cfg,
                        int64_t* n_split);
hipError_t launch_gemm_prefill(const int8_t* x_q, const float* s_x, int64_t M, int64_t N, int64_t K,
                               const uint8_t* w_bits, const float* s_w, const int8_t* w_a, const float* s_a,
                               const int8_t* w_b, const float* s_b, const int32_t* t, int32_t* t_out, int rank,
                               float* y, int32_t* acc_dbg, int64_t batch, int force_cfg, int force_tail,
                               hipStream_t stream);
}  // namespace dfssm

#include "decode_args.h"

namespace {

constexpr int64_t kMaxDecodeM = 16;
constexpr int64_t kGemvMaxK = 8 * 4 * 4 * 128;  // decode kernel: 8 waves x 4 lane groups x 4 chunks x 128 k
// |t| <= 127 * 127 * K must fit int32 (and |acc| <= 127 * K with it)
constexpr int64_t kMaxK = 131072;
constexpr int64_t kMaxRows = (int64_t)1 << 31;
constexpr int64_t kMaxBatch = 65535;  // problems ride gridDim.y
constexpr int64_t kRankBytes = 16;     // one row of W_A (int8, rank 16)

// Operands read with 16-byte vector loads (x, x_q, w_bits, w_a, w_b) must be 16-byte
// aligned; scale vectors, t, y and acc_dbg only need their element alignment.
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }
bool aligned4_or_null(const void* p) { return p == nullptr || aligned4(p); }

dfssm_status check_rank(int32_t rank) {
    return (rank == 0 || rank == 16) ? DFSSM_OK : DFSSM_ERR_UNSUPPORTED;
}

dfssm_status check_sizes(int64_t M, int64_t K, int64_t batch) {
    if (M <= 0 || K <= 0 || batch <= 0 || M >= kMaxRows) return DFSSM_ERR_INVALID_ARG;
    if (batch > kMaxBatch) return DFSSM_ERR_UNSUPPORTED;
    return DFSSM_OK;
}

dfssm_status lora_down_impl(const int8_t* x_q, int64_t M, int64_t K, const int8_t* w_b, int32_t rank, int32_t* t,
                            int64_t batch, hipStream_t stream) {
    if (!x_q || !w_b || !t) return DFSSM_ERR_INVALID_ARG;
    if (dfssm_status st = check_sizes(M, K, batch)) return st;
    if (!aligned16(x_q) || !aligned16(w_b) || !aligned4(t)) return DFSSM_ERR_INVALID_ARG;
    if (rank != 16) return DFSSM_ERR_UNSUPPORTED;
    if (K > kMaxK) return DFSSM_ERR_UNSUPPORTED;
    return dfssm::launch_lora_down(x_q, M, K, w_b, t, batch, stream) == hipSuccess ? DFSSM_OK : DFSSM_ERR_HIP;
}

dfssm_status quantize_lora_down_impl(const float* x, int64_t M, int64_t K, const int8_t* w_b, int32_t rank,
                                     int8_t* x_q, float* s_x, int32_t* t, int64_t batch, hipStream_t stream) {
    if (!x || !x_q || !s_x) return DFSSM_ERR_INVALID_ARG;
    if (dfssm_status st = check_sizes(M, K, batch)) return st;
    if (!aligned16(x) || !aligned16(x_q) || !aligned4(s_x)) return DFSSM_ERR_INVALID_ARG;
    if (dfssm_status st = check_rank(rank)) return st;
    if (rank == 16) {
        if (!w_b || !t) return DFSSM_ERR_INVALID_ARG;
        if (!aligned16(w_b) || !aligned4(t)) return DFSSM_ERR_INVALID_ARG;
        if (K > kMaxK) return DFSSM_ERR_UNSUPPORTED;
    }
    if (M * batch >= kMaxRows) return DFSSM_ERR_INVALID_ARG;
    hipError_t e;
    if (K % 4 == 0 && dfssm::quantize_lora_tokens_per_group(K) > 0) {
        e = dfssm::launch_quantize_lora_down(x, M, K, w_b, rank, x_q, s_x, t, batch, stream);
    } else {
        // rows not 16-byte aligned, or longer than the fused kernel's LDS holds: two kernels
        e = dfssm::launch_quantize_act(x, M * batch, K, x_q, s_x, stream);
        if (e == hipSuccess && rank == 16) e = dfssm::launch_lora_down(x_q, M, K, w_b, t, batch, stream);
    }
    return e == hipSuccess ? DFSSM_OK : DFSSM_ERR_HIP;
}

// The scaffold product with the scale + LoRA-up epilogue.  Exactly one of t (given,
// from a LoRA-down call) and w_b (t = W_B x_q computed by the kernel; t_out, when not
// NULL, receives it) is used at rank 16.
dfssm_status gemm_impl(const int8_t* x_q, const float* s_x, int64_t M, int64_t N, int64_t K,
                       const uint8_t* w_bits, const float* s_w, const int8_t* w_a, const float* s_a,
                       const int8_t* w_b, const float* s_b, const int32_t* t, int32_t* t_out, int32_t rank, float* y,
                       int32_t* acc_dbg, int64_t batch, hipStream_t stream) {
    if (!x_q || !s_x || !w_bits || !s_w || !y) return DFSSM_ERR_INVALID_ARG;
    if (dfssm_status st = check_sizes(M, K, batch)) return st;
    if (N <= 0 || N >= kMaxRows || (K % 8) != 0) return DFSSM_ERR_INVALID_ARG;
    if (!aligned16(x_q) || !aligned4(s_x) || !aligned16(w_bits) || !aligned4(s_w) || !aligned4(y) ||
        !aligned4_or_null(acc_dbg) || !aligned4_or_null(t_out))
        return DFSSM_ERR_INVALID_ARG;
    if (dfssm_status st = check_rank(rank)) return st;
    if (rank == 16) {
        if (!w_a || !s_a || !s_b || (!t && !w_b)) return DFSSM_ERR_INVALID_ARG;
        if (!aligned16(w_a) || !aligned4(s_a) || !aligned4(s_b)) return DFSSM_ERR_INVALID_ARG;
        if ((t && !aligned4(t)) || (w_b && !aligned16(w_b))) return DFSSM_ERR_INVALID_ARG;
    }
    if (K > kMaxK) return DFSSM_ERR_UNSUPPORTED;
    if (rank == 0) {
        w_b = nullptr;
        t = nullptr;
        t_out = nullptr;
    } else if (t) {
        w_b = nullptr;  // the given-t form
        t_out = nullptr;
    }
    hipError_t e;
    // the decode kernel addresses one problem's signs, LoRA rows and outputs with 32-bit
    // offsets
    const bool gemv_fits = N * (K / 8) < ((int64_t)1 << 31) && M * N * 4 < ((int64_t)1 << 31) &&
                           N * kRankBytes < ((int64_t)1 << 31);
    if (M <= kMaxDecodeM && K <= kGemvMaxK && gemv_fits) {
        e = dfssm::launch_gemv(x_q, s_x, (int)M, N, K, w_bits, s_w, w_a, s_a, w_b, s_b, t, t_out, rank, y, acc_dbg,
                               batch, stream);
    } else {
        // DFSSM_PREFILL_CFG pins the many-token kernel's tile configuration (0 ..
        // prefill_num_cfgs() - 1) or, with -2, the generic fallback kernel; unset or -1
        // lets the cost model choose.  DFSSM_PREFILL_TAIL adds a narrower configuration
        // for the columns past the pinned one's main part, where the pinned one is built
        // with that tail.  Testing and tuning knobs.
        int force = -1, force_tail = -1;
        if (const char* f = getenv("DFSSM_PREFILL_CFG")) force = atoi(f);
        if (const char* f = getenv("DFSSM_PREFILL_TAIL")) force_tail = atoi(f);
        const bool prefill = force != -2 && dfssm::prefill_supported(M, N, K) && aligned16(w_bits) &&
                             (rank == 0 || aligned16(w_a));
        if (prefill) {
            e = dfssm::launch_gemm_prefill(x_q, s_x, M, N, K, w_bits, s_w, w_a, s_a, w_b, s_b, t, t_out, rank, y,
                                           acc_dbg, batch, force, force_tail, stream);
        } else {
            e = dfssm::launch_gemm_mfma(x_q, s_x, M, N, K, w_bits, s_w, w_a, s_a, w_b, s_b, t, t_out, rank, y,
                                        acc_dbg, batch, stream);
        }
    }
    return e == hipSuccess ? DFSSM_OK : DFSSM_ERR_HIP;
}

dfssm_status forward_impl(const float* x, int64_t M, int64_t N, int64_t K, const uint8_t* w_bits,
                          const float* s_w, const int8_t* w_a, const float* s_a, const int8_t* w_b,
                          const float* s_b, int32_t rank, int8_t* x_q, float* s_x, int32_t* t, float* y,
                          int32_t* acc_dbg, int64_t batch, hipStream_t stream) {
    // the two calls' checks, in full, before anything is launched
    if (!x || !x_q || !s_x || !w_bits || !s_w || !y) return DFSSM_ERR_INVALID_ARG;
    if (dfssm_status st = check_sizes(M, K, batch)) return st;
    if (N <= 0 || N >= kMaxRows || (K % 8) != 0) return DFSSM_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(x_q) || !aligned4(s_x) || !aligned16(w_bits) || !aligned4(s_w) ||
        !aligned4(y) || !aligned4_or_null(acc_dbg))
        return DFSSM_ERR_INVALID_ARG;
    if (dfssm_status st = check_rank(rank)) return st;
    if (rank == 16) {
        if (!w_a || !s_a || !w_b || !s_b || !t) return DFSSM_ERR_INVALID_ARG;
        if (!aligned16(w_a) || !aligned4(s_a) || !aligned16(w_b) || !aligned4(s_b) || !aligned4(t))
            return DFSSM_ERR_INVALID_ARG;
    }
    if (K > kMaxK) return DFSSM_ERR_UNSUPPORTED;
    if (M * batch >= kMaxRows) return DFSSM_ERR_INVALID_ARG;
    const bool gemv_fits = N * (K / 8) < ((int64_t)1 << 31) && M * N * 4 < ((int64_t)1 << 31) &&
                           N * kRankBytes < ((int64_t)1 << 31);
    if (gemv_fits && dfssm::decode_fused_supported(M, K)) {
        const hipError_t e = dfssm::launch_decode_fused(x, (int)M, N, K, w_bits, s_w, w_a, s_a, w_b, s_b, rank, x_q,
                                                        s_x, t, y, acc_dbg, batch, stream);
        if (e != hipErrorNotSupported) return e == hipSuccess ? DFSSM_OK : DFSSM_ERR_HIP;
        // the launch plan has several groups per problem at a throughput batch: two kernels
    }
    // Many-token projections with under 2^24 outputs per launch: the plain quantizer, then
    // the MFMA kernel computing t from the code chunks it already stages (its first column
    // tile writes t out).  Against quantize + LoRA-down followed by the product given t it
    // measured 1.2-2 us faster from 17 to 2048 tokens for N = 2048, K = 4096, and level or
    // up to 2.9 us faster from 17 to 1536 tokens for N = 8512, K = 2048.  At 2048 tokens of
    // the latter (2^24 outputs and more) the product is MFMA-bound and the W_B chunks every
    // column tile recomputes cost more than the separate LoRA-down pass (1.1 us slower).
    // The bytes written are the same either way.
    const bool decode_kernel = M <= kMaxDecodeM && K <= kGemvMaxK && gemv_fits;
    if (rank == 16 && !decode_kernel && M * N * batch < ((int64_t)1 << 24) && dfssm::prefill_supported(M, N, K)) {
        if (dfssm::launch_quantize_act(x, M * batch, K, x_q, s_x, stream) != hipSuccess) return DFSSM_ERR_HIP;
        return gemm_impl(x_q, s_x, M, N, K, w_bits, s_w, w_a, s_a, w_b, s_b, nullptr, t, rank, y, acc_dbg, batch,
                         stream);
    }
    if (dfssm_status st = quantize_lora_down_impl(x, M, K, w_b, rank, x_q, s_x, t, batch, stream)) return st;
    return gemm_impl(x_q, s_x, M, N, K, w_bits, s_w, w_a, s_a, nullptr, s_b, t, nullptr, rank, y, acc_dbg, batch,
                     stream);
}

dfssm_status int8_head_impl(const int8_t* x_q, const float* s_x, int64_t M, int64_t N, int64_t K, const int8_t* e,
                           const float* s_e, float* y, int32_t* acc_dbg, int64_t batch, hipStream_t stream) {
    if (!x_q || !s_x || !e || !s_e || !y) return DFSSM_ERR_INVALID_ARG;
    if (dfssm_status st = check_sizes(M, K, batch)) return st;
    if (N <= 0 || N >= kMaxRows || (K % 16) != 0) return DFSSM_ERR_INVALID_ARG;
    if (!aligned16(x_q) || !aligned4(s_x) || !aligned16(e) || !aligned4(s_e) || !aligned4(y) ||
        !aligned4_or_null(acc_dbg))
        return DFSSM_ERR_INVALID_ARG;
    // one problem's matrix and outputs are addressed with 32-bit offsets (plus one
    // stage of rows past N)
    if ((N + 128) * K >= ((int64_t)1 << 31) || M * N * 4 >= ((int64_t)1 << 31)) return DFSSM_ERR_UNSUPPORTED;
    if (!dfssm::int8_head_supported(M, K)) return DFSSM_ERR_UNSUPPORTED;
    return dfssm::launch_int8_head(x_q, s_x, (int)M, N, K, e, s_e, y, acc_dbg, batch, stream) == hipSuccess
               ? DFSSM_OK
               : DFSSM_ERR_HIP;
}

dfssm_status decode_layers_impl(const dfssm_decode_layer_weights* w, int64_t n_layers, const float* x_in,
                                float* x_out, const float* conv_in, float* conv_out, float* ssm_state, float eps,
                                void* workspace, size_t workspace_bytes, int32_t* status, uint32_t* trace,
                                int64_t spin_limit, uint32_t flags, hipStream_t stream, bool validate_only = false) {
    if (!w || !x_in || !x_out || !conv_in || !conv_out || !ssm_state || !workspace || !status)
        return DFSSM_ERR_INVALID_ARG;
    if (!w->in_w_bits || !w->in_s_w || !w->in_w_a || !w->in_s_a || !w->in_w_b || !w->in_s_b || !w->conv_w ||
        !w->conv_b || !w->dt_bias || !w->A_log || !w->D || !w->norm_w || !w->out_w_bits || !w->out_s_w ||
        !w->out_w_a || !w->out_s_a || !w->out_w_b || !w->out_s_b)
        return DFSSM_ERR_INVALID_ARG;
    if (n_layers < 1 || n_layers > dfssm::decode_layers_max_layers()) return DFSSM_ERR_INVALID_ARG;
    if (!(eps >= 0.0f) || eps > 1e30f) return DFSSM_ERR_INVALID_ARG;
    if (workspace_bytes < dfssm::decode_layers_workspace_bytes()) return DFSSM_ERR_INVALID_ARG;
    if (flags & ~DFSSM_DECODE_UNREACHABLE_WAITS) return DFSSM_ERR_INVALID_ARG;
    if (!aligned16(w->in_w_bits) || !aligned16(w->in_w_a) || !aligned16(w->in_w_b) || !aligned16(w->conv_w) ||
        !aligned16(w->norm_w) || !aligned16(w->out_w_bits) || !aligned16(w->out_w_a) || !aligned16(w->out_w_b) ||
        !aligned4(w->in_s_w) || !aligned4(w->in_s_a) || !aligned4(w->in_s_b) || !aligned4(w->conv_b) ||
        !aligned4(w->dt_bias) || !aligned4(w->A_log) || !aligned4(w->D) || !aligned4(w->out_s_w) ||
        !aligned4(w->out_s_a) || !aligned4(w->out_s_b) || !aligned16(x_in) || !aligned4(x_out) ||
        !aligned16(conv_in) || !aligned16(conv_out) || !aligned16(ssm_state) || !aligned16(workspace) ||
        !aligned4(status) || !aligned4_or_null(trace))
        return DFSSM_ERR_INVALID_ARG;
    const int64_t conv_bytes = n_layers * 4352 * 16;
    const uintptr_t ci = (uintptr_t)conv_in, co = (uintptr_t)conv_out;
    if (ci < co + (uintptr_t)conv_bytes && co < ci + (uintptr_t)conv_bytes) return DFSSM_ERR_INVALID_ARG;
    if (validate_only) return DFSSM_OK;
    const dfssm::decode::Args a{w->in_w_bits, w->in_s_w, w->in_w_a, w->in_s_a, w->in_w_b, w->in_s_b,
                                w->conv_w, w->conv_b, w->dt_bias, w->A_log, w->D, w->norm_w,
                                w->out_w_bits, w->out_s_w, w->out_w_a, w->out_s_a, w->out_w_b, w->out_s_b,
                                conv_in, conv_out, ssm_state, x_in, x_out, trace,
                                static_cast<uint32_t*>(workspace), status, (int)n_layers, eps,
                                spin_limit > 0 ? spin_limit : ((int64_t)1 << 22),
                                (flags & DFSSM_DECODE_UNREACHABLE_WAITS) ? (1u << 30) : 0u};
    const hipError_t e = dfssm::launch_decode_layers(a, stream);
    if (e == hipErrorNotSupported) return DFSSM_ERR_UNSUPPORTED;
    return e == hipSuccess ? DFSSM_OK : DFSSM_ERR_HIP;
}

dfssm_status density_checks(int64_t rows, int64_t d_state) {
    if (rows <= 0 || d_state <= 0) return DFSSM_ERR_INVALID_ARG;
    if (!dfssm::density_field_supported(d_state)) return DFSSM_ERR_UNSUPPORTED;
    if (rows >= ((int64_t)1 << 40) / d_state) return DFSSM_ERR_INVALID_ARG;
    return DFSSM_OK;
}

}  // namespace

extern "C" {

const char* dfssm_status_string(dfssm_status status) {
    switch (status) {
        case DFSSM_OK: return "DFSSM_OK";
        case DFSSM_ERR_INVALID_ARG: return "DFSSM_ERR_INVALID_ARG";
        case DFSSM_ERR_UNSUPPORTED: return "DFSSM_ERR_UNSUPPORTED";
        case DFSSM_ERR_HIP: return "DFSSM_ERR_HIP";
    }
    return "DFSSM_ERR_UNKNOWN";
}

int32_t dfssm_version(void) { return 400; }

dfssm_status dfssm_prefill_plan(int64_t M, int64_t N, int64_t K, int64_t batch, int32_t* main_cfg,
                                int32_t* tail_cfg, int64_t* n_split) {
    if (!main_cfg || !tail_cfg || !n_split) return DFSSM_ERR_INVALID_ARG;
    if (dfssm_status st = check_sizes(M, K, batch)) return st;
    if (N <= 0 || N >= kMaxRows || (K % 8) != 0) return DFSSM_ERR_INVALID_ARG;
    if (K > kMaxK) return DFSSM_ERR_UNSUPPORTED;
    // the same tests as dfssm_scaffold_lora_gemm[_strided_batched]: the decode kernel, or
    // the generic kernel, takes the shape
    const bool gemv_fits = N * (K / 8) < ((int64_t)1 << 31) && M * N * 4 < ((int64_t)1 << 31) &&
                           N * kRankBytes < ((int64_t)1 << 31);
    if (M <= kMaxDecodeM && K <= kGemvMaxK && gemv_fits) return DFSSM_ERR_UNSUPPORTED;
    if (!dfssm::prefill_supported(M, N, K)) return DFSSM_ERR_UNSUPPORTED;
    int mc = 0, tc = -1;
    int64_t ns = N;
    dfssm::prefill_plan_query(M, N, K, batch, &mc, &tc, &ns);
    *main_cfg = mc;
    *tail_cfg = tc;
    *n_split = ns;
    return DFSSM_OK;
}

dfssm_status dfssm_quantize_act(const float* x, int64_t M, int64_t K, int8_t* x_q, float* s_x,
                                hipStream_t stream) {
    if (!x || !x_q || !s_x) return DFSSM_ERR_INVALID_ARG;
    if (M <= 0 || K <= 0 || M >= kMaxRows) return DFSSM_ERR_INVALID_ARG;
    if (!aligned4(x) || !aligned4(s_x)) return DFSSM_ERR_INVALID_ARG;
    return dfssm::launch_quantize_act(x, M, K, x_q, s_x, stream) == hipSuccess ? DFSSM_OK : DFSSM_ERR_HIP;
}

dfssm_status dfssm_lora_down(const int8_t* x_q, int64_t M, int64_t K, const int8_t* w_b, int32_t rank, int32_t* t,
                             hipStream_t stream) {
    return lora_down_impl(x_q, M, K, w_b, rank, t, 1, stream);
}

dfssm_status dfssm_lora_down_strided_batched(const int8_t* x_q, int64_t M, int64_t K, const int8_t* w_b,
                                             int32_t rank, int32_t* t, int64_t batch, hipStream_t stream) {
    return lora_down_impl(x_q, M, K, w_b, rank, t, batch, stream);
}

dfssm_status dfssm_quantize_lora_down(const float* x, int64_t M, int64_t K, const int8_t* w_b, int32_t rank,
                                      int8_t* x_q, float* s_x, int32_t* t, hipStream_t stream) {
    return quantize_lora_down_impl(x, M, K, w_b, rank, x_q, s_x, t, 1, stream);
}

dfssm_status dfssm_quantize_lora_down_strided_batched(const float* x, int64_t M, int64_t K, const int8_t* w_b,
                                                      int32_t rank, int8_t* x_q, float* s_x, int32_t* t,
                                                      int64_t batch, hipStream_t stream) {
    return quantize_lora_down_impl(x, M, K, w_b, rank, x_q, s_x, t, batch, stream);
}

dfssm_status dfssm_scaffold_lora_gemm(const int8_t* x_q, const float* s_x, int64_t M, int64_t N, int64_t K,
                                      const uint8_t* w_bits, const float* s_w, const int8_t* w_a,
                                      const float* s_a, const int8_t* w_b, const float* s_b, int32_t rank,
                                      float* y, int32_t* acc_dbg, int32_t* t_dbg, hipStream_t stream) {
    if (rank != 0 && !w_b) return DFSSM_ERR_INVALID_ARG;
    return gemm_impl(x_q, s_x, M, N, K, w_bits, s_w, w_a, s_a, w_b, s_b, nullptr, t_dbg, rank, y, acc_dbg, 1,
                     stream);
}

dfssm_status dfssm_scaffold_lora_gemm_strided_batched(const int8_t* x_q, const float* s_x, int64_t M, int64_t N,
                                                      int64_t K, const uint8_t* w_bits, const float* s_w,
                                                      const int8_t* w_a, const float* s_a, const int8_t* w_b,
                                                      const float* s_b, int32_t rank, float* y, int32_t* acc_dbg,
                                                      int32_t* t_dbg, int64_t batch, hipStream_t stream) {
    if (rank != 0 && !w_b) return DFSSM_ERR_INVALID_ARG;
    return gemm_impl(x_q, s_x, M, N, K, w_bits, s_w, w_a, s_a, w_b, s_b, nullptr, t_dbg, rank, y, acc_dbg, batch,
                     stream);
}

dfssm_status dfssm_scaffold_lora_gemm_given_t(const int8_t* x_q, const float* s_x, int64_t M, int64_t N, int64_t K,
                                              const uint8_t* w_bits, const float* s_w, const int8_t* w_a,
                                              const float* s_a, const float* s_b, const int32_t* t, int32_t rank,
                                              float* y, int32_t* acc_dbg, hipStream_t stream) {
    if (rank != 0 && !t) return DFSSM_ERR_INVALID_ARG;
    return gemm_impl(x_q, s_x, M, N, K, w_bits, s_w, w_a, s_a, nullptr, s_b, t, nullptr, rank, y, acc_dbg, 1,
                     stream);
}

dfssm_status dfssm_scaffold_lora_gemm_given_t_strided_batched(const int8_t* x_q, const float* s_x, int64_t M,
                                                              int64_t N, int64_t K, const uint8_t* w_bits,
                                                              const float* s_w, const int8_t* w_a, const float* s_a,
                                                              const float* s_b, const int32_t* t, int32_t rank,
                                                              float* y, int32_t* acc_dbg, int64_t batch,
                                                              hipStream_t stream) {
    if (rank != 0 && !t) return DFSSM_ERR_INVALID_ARG;
    return gemm_impl(x_q, s_x, M, N, K, w_bits, s_w, w_a, s_a, nullptr, s_b, t, nullptr, rank, y, acc_dbg, batch,
                     stream);
}

dfssm_status dfssm_scaffold_lora_forward(const float* x, int64_t M, int64_t N, int64_t K, const uint8_t* w_bits,
                                         const float* s_w, const int8_t* w_a, const float* s_a, const int8_t* w_b,
                                         const float* s_b, int32_t rank, int8_t* x_q, float* s_x, int32_t* t,
                                         float* y, int32_t* acc_dbg, hipStream_t stream) {
    return forward_impl(x, M, N, K, w_bits, s_w, w_a, s_a, w_b, s_b, rank, x_q, s_x, t, y, acc_dbg, 1, stream);
}

dfssm_status dfssm_scaffold_lora_forward_strided_batched(const float* x, int64_t M, int64_t N, int64_t K,
                                                         const uint8_t* w_bits, const float* s_w, const int8_t* w_a,
                                                         const float* s_a, const int8_t* w_b, const float* s_b,
                                                         int32_t rank, int8_t* x_q, float* s_x, int32_t* t,
                                                         float* y, int32_t* acc_dbg, int64_t batch,
                                                         hipStream_t stream) {
    return forward_impl(x, M, N, K, w_bits, s_w, w_a, s_a, w_b, s_b, rank, x_q, s_x, t, y, acc_dbg, batch, stream);
}

dfssm_status dfssm_int8_rowscale_gemm(const int8_t* x_q, const float* s_x, int64_t M, int64_t N, int64_t K,
                                      const int8_t* e, const float* s_e, float* y, int32_t* acc_dbg,
                                      hipStream_t stream) {
    return int8_head_impl(x_q, s_x, M, N, K, e, s_e, y, acc_dbg, 1, stream);
}

dfssm_status dfssm_int8_rowscale_gemm_strided_batched(const int8_t* x_q, const float* s_x, int64_t M, int64_t N,
                                                      int64_t K, const int8_t* e, const float* s_e, float* y,
                                                      int32_t* acc_dbg, int64_t batch, hipStream_t stream) {
    return int8_head_impl(x_q, s_x, M, N, K, e, s_e, y, acc_dbg, batch, stream);
}

dfssm_status dfssm_embedding_lookup(const int32_t* tokens, int64_t T, const int8_t* e, const float* s_e, int64_t V,
                                    int64_t K, float* out, hipStream_t stream) {
    if (!tokens || !e || !s_e || !out) return DFSSM_ERR_INVALID_ARG;
    if (T <= 0 || V <= 0 || K <= 0 || T >= kMaxRows) return DFSSM_ERR_INVALID_ARG;
    if (!aligned4(tokens) || !aligned4(s_e) || !aligned4(out)) return DFSSM_ERR_INVALID_ARG;
    if (V * K >= ((int64_t)1 << 40) || T * K >= ((int64_t)1 << 40)) return DFSSM_ERR_UNSUPPORTED;
    return dfssm::launch_embedding_lookup(tokens, T, e, s_e, V, K, out, stream) == hipSuccess ? DFSSM_OK
                                                                                            : DFSSM_ERR_HIP;
}

dfssm_status dfssm_density_field_encode(const float* state, int64_t rows, int64_t d_state, uint32_t* field,
                                        float* scale, hipStream_t stream) {
    if (!state || !field || !scale) return DFSSM_ERR_INVALID_ARG;
    if (dfssm_status st = density_checks(rows, d_state)) return st;
    if (!aligned16(state) || !aligned16(field) || !aligned4(scale)) return DFSSM_ERR_INVALID_ARG;
    return dfssm::launch_density_encode(state, rows, d_state, field, scale, nullptr, stream) == hipSuccess
               ? DFSSM_OK
               : DFSSM_ERR_HIP;
}

dfssm_status dfssm_density_field_decode(const uint32_t* field, const float* scale, int64_t rows, int64_t d_state,
                                        float* state, hipStream_t stream) {
    if (!state || !field || !scale) return DFSSM_ERR_INVALID_ARG;
    if (dfssm_status st = density_checks(rows, d_state)) return st;
    if (!aligned16(state) || !aligned4(field) || !aligned4(scale)) return DFSSM_ERR_INVALID_ARG;
    return dfssm::launch_density_decode(field, scale, rows, d_state, state, stream) == hipSuccess ? DFSSM_OK
                                                                                                 : DFSSM_ERR_HIP;
}

dfssm_status dfssm_density_field_requantize(float* state, int64_t rows, int64_t d_state, uint32_t* field,
                                            float* scale, hipStream_t stream) {
    if (!state) return DFSSM_ERR_INVALID_ARG;
    if (dfssm_status st = density_checks(rows, d_state)) return st;
    if (!aligned16(state) || !aligned4_or_null(field) || !aligned4_or_null(scale)) return DFSSM_ERR_INVALID_ARG;
    return dfssm::launch_density_encode(state, rows, d_state, field, scale, state, stream) == hipSuccess
               ? DFSSM_OK
               : DFSSM_ERR_HIP;
}

size_t dfssm_decode_layers_workspace_bytes(void) { return dfssm::decode_layers_workspace_bytes(); }

int64_t dfssm_decode_layers_trace_words(void) { return dfssm::decode_layers_trace_words(); }

dfssm_status dfssm_decode_layers_noalloc(const dfssm_decode_layer_weights* w, int64_t n_layers, const float* x_in,
                                         float* x_out, const float* conv_state_in, float* conv_state_out,
                                         float* ssm_state, float eps, int32_t* status, uint32_t* trace,
                                         int64_t spin_limit, uint32_t flags, hipStream_t stream) {
    // the same checks as dfssm_decode_layers, with the library's array standing in for
    // the workspace (a stand-in address passes them; the real one is fetched after)
    alignas(16) static char probe[16];
    if (dfssm_status st = decode_layers_impl(w, n_layers, x_in, x_out, conv_state_in, conv_state_out, ssm_state, eps,
                                             probe, dfssm::decode_layers_workspace_bytes(), status, trace, spin_limit,
                                             flags, stream, /*validate_only=*/true))
        return st;
    uint32_t* ws = dfssm::decode_layers_scratch(stream);
    if (ws == nullptr) return DFSSM_ERR_HIP;
    return decode_layers_impl(w, n_layers, x_in, x_out, conv_state_in, conv_state_out, ssm_state, eps, ws,
                              dfssm::decode_layers_workspace_bytes(), status, trace, spin_limit, flags, stream, false);
}

dfssm_status dfssm_decode_layers(const dfssm_decode_layer_weights* w, int64_t n_layers, const float* x_in,
                                 float* x_out, const float* conv_state_in, float* conv_state_out, float* ssm_state,
                                 float eps, void* workspace, size_t workspace_bytes, int32_t* status, uint32_t* trace,
                                 int64_t spin_limit, uint32_t flags, hipStream_t stream) {
    return decode_layers_impl(w, n_layers, x_in, x_out, conv_state_in, conv_state_out, ssm_state, eps, workspace,
                              workspace_bytes, status, trace, spin_limit, flags, stream);
}

dfssm_status dfssm_mamba2_decode_step(const float* zxbcdt, int64_t S, int64_t nheads, int64_t headdim,
                                      int64_t d_state, const float* conv_state_in, float* conv_state_out,
                                      float* ssm_state, const float* conv_w, const float* conv_b,
                                      const float* dt_bias, const float* A_log, const float* D,
                                      const float* norm_w, float eps, float* out, hipStream_t stream) {
    if (!zxbcdt || !conv_state_in || !conv_state_out || !ssm_state || !conv_w || !conv_b || !dt_bias || !A_log ||
        !D || !norm_w || !out)
        return DFSSM_ERR_INVALID_ARG;
    if (S <= 0 || S > kMaxBatch || nheads <= 0 || headdim <= 0 || d_state <= 0) return DFSSM_ERR_INVALID_ARG;
    if (!(eps >= 0.0f) || eps > 1e30f) return DFSSM_ERR_INVALID_ARG;
    if (!aligned16(conv_state_in) || !aligned16(conv_state_out) || !aligned16(ssm_state) || !aligned16(conv_w) ||
        !aligned16(norm_w) || !aligned16(out) || !aligned4(zxbcdt) || !aligned4(conv_b) || !aligned4(dt_bias) ||
        !aligned4(A_log) || !aligned4(D))
        return DFSSM_ERR_INVALID_ARG;
    if (!dfssm::mamba2_step_supported(nheads, headdim, d_state)) return DFSSM_ERR_UNSUPPORTED;
    const int64_t d_inner = nheads * headdim, conv_dim = d_inner + 2 * d_state;
    auto overlap = [](const void* a, int64_t na, const void* b, int64_t nb) {
        const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
        return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
    };
    if (overlap(conv_state_in, S * conv_dim * 16, conv_state_out, S * conv_dim * 16) ||
        overlap(out, S * d_inner * 4, zxbcdt, S * (d_inner + conv_dim + nheads) * 4))
        return DFSSM_ERR_INVALID_ARG;
    return dfssm::launch_mamba2_step(zxbcdt, S, (int)nheads, conv_state_in, conv_state_out, ssm_state, conv_w, conv_b,
                                     dt_bias, A_log, D, norm_w, eps, out, stream) == hipSuccess
               ? DFSSM_OK
               : DFSSM_ERR_HIP;
}

}  // extern "C"
