// api.hip -- the C ABI (include/dfssm.h): host-side validation and kernel dispatch.
//
// Every entry point validates its arguments before enqueuing anything, launches on
// the caller's stream, never synchronizes and allocates nothing.
#include "dfssm.h"

#include <hip/hip_runtime.h>

namespace dfssm {
hipError_t launch_quantize_act(const float* x, int64_t M, int64_t K, int8_t* x_q, float* s_x,
                               hipStream_t stream);
hipError_t launch_lora_down(const int8_t* x_q, int64_t M, int64_t K, const int8_t* w_b, int32_t* t,
                            hipStream_t stream);
hipError_t launch_gemv(const int8_t* x_q, const float* s_x, int M, int64_t N, int64_t K,
                       const uint8_t* w_bits, const float* s_w, const int8_t* w_a, const float* s_a,
                       const float* s_b, const int32_t* t, int rank, float* y, int32_t* acc_dbg,
                       hipStream_t stream);
hipError_t launch_gemm_mfma(const int8_t* x_q, const float* s_x, int64_t M, int64_t N, int64_t K,
                            const uint8_t* w_bits, const float* s_w, const int8_t* w_a, const float* s_a,
                            const float* s_b, const int32_t* t, int rank, float* y, int32_t* acc_dbg,
                            hipStream_t stream);
}  // namespace dfssm

namespace {

constexpr int64_t kMaxDecodeM = 16;
constexpr int64_t kGemvMaxK = 8 * 4 * 4 * 128;  // decode kernel's largest K (8 waves x 4 lane groups x 4 chunks)
// |t| <= 127 * 127 * K must fit int32, and |acc| <= 127 * K with it.
constexpr int64_t kMaxK = 131072;
constexpr int64_t kMaxRows = (int64_t)1 << 31;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool aligned_or_null(const void* p) { return p == nullptr || aligned16(p); }

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

int32_t dfssm_version(void) { return 100; }

dfssm_status dfssm_quantize_act(const float* x, int64_t M, int64_t K, int8_t* x_q, float* s_x,
                                hipStream_t stream) {
    if (!x || !x_q || !s_x) return DFSSM_ERR_INVALID_ARG;
    if (M <= 0 || K <= 0 || M >= kMaxRows) return DFSSM_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(x_q) || !aligned16(s_x)) return DFSSM_ERR_INVALID_ARG;
    if (dfssm::launch_quantize_act(x, M, K, x_q, s_x, stream) != hipSuccess) return DFSSM_ERR_HIP;
    return DFSSM_OK;
}

dfssm_status dfssm_scaffold_lora_gemm(const int8_t* x_q, const float* s_x, int64_t M, int64_t N, int64_t K,
                                      const uint8_t* w_bits, const float* s_w, const int8_t* w_a,
                                      const float* s_a, const int8_t* w_b, const float* s_b, int32_t rank,
                                      float* y, int32_t* t, int32_t* acc_dbg, hipStream_t stream) {
    if (!x_q || !s_x || !w_bits || !s_w || !y) return DFSSM_ERR_INVALID_ARG;
    if (M <= 0 || N <= 0 || K <= 0 || (K % 8) != 0) return DFSSM_ERR_INVALID_ARG;
    if (M >= kMaxRows || N >= kMaxRows) return DFSSM_ERR_INVALID_ARG;
    if (!aligned16(x_q) || !aligned16(s_x) || !aligned16(w_bits) || !aligned16(s_w) || !aligned16(y) ||
        !aligned_or_null(acc_dbg))
        return DFSSM_ERR_INVALID_ARG;
    if (rank != 0 && rank != 16) return DFSSM_ERR_UNSUPPORTED;
    if (rank == 16) {
        if (!w_a || !s_a || !w_b || !s_b || !t) return DFSSM_ERR_INVALID_ARG;
        if (!aligned16(w_a) || !aligned16(s_a) || !aligned16(w_b) || !aligned16(s_b) || !aligned16(t))
            return DFSSM_ERR_INVALID_ARG;
    }
    if (K > kMaxK) return DFSSM_ERR_UNSUPPORTED;

    if (rank == 16) {
        if (dfssm::launch_lora_down(x_q, M, K, w_b, t, stream) != hipSuccess) return DFSSM_ERR_HIP;
    }
    hipError_t e;
    if (M <= kMaxDecodeM && K <= kGemvMaxK) {
        e = dfssm::launch_gemv(x_q, s_x, (int)M, N, K, w_bits, s_w, w_a, s_a, s_b, t, rank, y, acc_dbg, stream);
    } else {
        e = dfssm::launch_gemm_mfma(x_q, s_x, M, N, K, w_bits, s_w, w_a, s_a, s_b, t, rank, y, acc_dbg, stream);
    }
    return e == hipSuccess ? DFSSM_OK : DFSSM_ERR_HIP;
}

}  // extern "C"
