/*
 * dfssm.h -- C ABI of the DF-SSM scaffold projection for AMD Instinct MI355X (gfx950).
 *
 * The operation (DF-SSM, "Density Field State Space Models"; technical summary on
 * gist.science, section 2B "Frozen Scaffold with LoRA Correction" and section 2C
 * "Optimized Inference Pipeline"): every in_proj / out_proj of the 48-layer
 * Mamba-2 1.3B model is a frozen 1-bit scaffold W (signs, d_out x d_in) plus an
 * int8 rank-16 LoRA correction W_A (d_out x 16) . W_B (16 x d_in) with
 * per-row scales; the scaffold's packed bits are expanded to int8 on the fly and
 * multiplied with int8 activations.  With M tokens, K = d_in, N = d_out, r = 16:
 *
 *   s_x[m]    = absmax_k |x[m][k]| / 127                  (fp32, IEEE division; 0 if absmax = 0)
 *   x_q[m][k] = clamp(rint(x[m][k] / s_x[m]), -127, 127)  (IEEE division, ties to even)
 *   acc[m][n] = sum_k w[n][k] * x_q[m][k]                  (exact int32, w in {-1, +1})
 *   t[m][r]   = sum_k W_B[r][k] * x_q[m][k]                (exact int32)
 *   y[m][n]   = s_x[m] * ( s_w[n] * acc[m][n]
 *                          + s_A[n] * sum_r W_A[n][r] * s_B[r] * t[m][r] )   (fp32)
 *
 * Data layout (all row-major, contiguous, device memory unless stated):
 *   x      fp32  [M][K]
 *   x_q    int8  [M][K]          s_x  fp32 [M]
 *   w_bits uint8 [N][K/8]        bit b of byte j of row n is the sign of w[n][8j+b]:
 *                                1 = +1, 0 = -1 (eight signs per byte, lowest k in the LSB)
 *   s_w    fp32  [N]             per-output-channel scaffold scale
 *   w_a    int8  [N][rank]       s_a fp32 [N]      (LoRA up, per-row scale)
 *   w_b    int8  [rank][K]       s_b fp32 [rank]   (LoRA down, per-row scale)
 *   t      int32 [M][rank]       LoRA down-projection (written by the library)
 *   y      fp32  [M][N]
 *
 * Ownership and threading: the caller owns every buffer; the library keeps
 * pointers only for the duration of a call, allocates no device memory on
 * these entry points, never synchronizes the stream, and enqueues all work on
 * `stream` (0 = the default stream), so the calls may be captured in a HIP
 * graph.  Calls on different streams are independent as long as their output
 * buffers do not overlap.
 *
 * Errors: arguments are validated on the host before anything is enqueued; on
 * a validation error nothing is launched.  DFSSM_ERR_HIP reports a launch
 * failure (hipGetLastError after the launch).  Non-finite x is a documented
 * precondition violation: results are then unspecified.
 */
#ifndef DFSSM_H
#define DFSSM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DFSSM_OK = 0,
    DFSSM_ERR_INVALID_ARG = 1,   /* NULL required pointer, M/N/K <= 0, K % 8 != 0, misaligned pointer */
    DFSSM_ERR_UNSUPPORTED = 2,   /* rank other than 0 or 16 */
    DFSSM_ERR_HIP = 3            /* the HIP runtime reported an error for a launch */
} dfssm_status;

/* Human-readable name of a status code (static storage, never NULL). */
const char* dfssm_status_string(dfssm_status status);

/* Library version as major*10000 + minor*100 + patch. */
int32_t dfssm_version(void);

/*
 * Per-token absmax int8 quantization of activations (the int8 operand of the
 * scaffold product; technical summary section 2C).
 *   x    fp32 [M][K], read only, 4-byte aligned
 *   x_q  int8 [M][K], written
 *   s_x  fp32 [M],    written (0 for an all-zero token, whose codes are all 0)
 * Requires M >= 1, K >= 1.  Bit-exact with the IEEE definition above.
 */
dfssm_status dfssm_quantize_act(const float* x, int64_t M, int64_t K,
                                int8_t* x_q, float* s_x, hipStream_t stream);

/*
 * Scaffold + LoRA projection y = s_x . (s_w . (W x_q) + s_A . W_A (s_B . W_B x_q))
 * (technical summary sections 2B and 2C).
 *   x_q, s_x     the quantized activations (as written by dfssm_quantize_act)
 *   w_bits, s_w  the 1-bit scaffold and its per-output-channel scale
 *   w_a, s_a, w_b, s_b, rank   the int8 LoRA pair; rank must be 16, or 0 for no
 *                correction (then w_a, s_a, w_b, s_b may be NULL)
 *   y            fp32 [M][N], written
 *   t            int32 [M][rank], written when rank == 16 (may be NULL when
 *                rank == 0); it carries W_B x_q from the LoRA-down kernel to
 *                the epilogue, and its values are exact
 *   acc_dbg      optional int32 [M][N]: when not NULL, also receives the exact
 *                scaffold accumulators sum_k w x_q (for verification; slower)
 * Requires M, N >= 1, K >= 8, K % 8 == 0, w_bits 4-byte aligned.
 * M <= 16 runs the bandwidth-bound decode kernel; larger M the int8 MFMA kernel.
 */
dfssm_status dfssm_scaffold_lora_gemm(const int8_t* x_q, const float* s_x,
                                      int64_t M, int64_t N, int64_t K,
                                      const uint8_t* w_bits, const float* s_w,
                                      const int8_t* w_a, const float* s_a,
                                      const int8_t* w_b, const float* s_b, int32_t rank,
                                      float* y, int32_t* t, int32_t* acc_dbg,
                                      hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DFSSM_H */
