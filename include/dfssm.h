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
 * A forward step is dfssm_quantize_act (x -> x_q, s_x) followed by
 * dfssm_scaffold_lora_gemm (x_q, s_x, W, W_A, W_B -> y, t computed inside), or one
 * call, dfssm_scaffold_lora_forward (x -> x_q, s_x, t, y), or the split form
 * dfssm_quantize_lora_down (x -> x_q, s_x, t) then dfssm_scaffold_lora_gemm_given_t
 * (x_q, s_x, t -> y).  The LoRA down-projection t is a reduction over all of K that
 * every output needs: dfssm_scaffold_lora_gemm has every workgroup compute the part of
 * it that its outputs need (no cross-workgroup dependency, no scratch memory), and the
 * split form produces it before the main kernel.
 *
 * Data layout (all row-major, contiguous, device memory):
 *   x      fp32  [M][K]
 *   x_q    int8  [M][K]          s_x  fp32 [M]
 *   w_bits uint8 [N][K/8]        bit b of byte j of row n is the sign of w[n][8j+b]:
 *                                1 = +1, 0 = -1 (eight signs per byte, lowest k in the LSB)
 *   s_w    fp32  [N]             per-output-channel scaffold scale
 *   w_a    int8  [N][rank]       s_a fp32 [N]      (LoRA up, per-row scale)
 *   w_b    int8  [rank][K]       s_b fp32 [rank]   (LoRA down, per-row scale)
 *   t      int32 [M][rank]       LoRA down-projection
 *   y      fp32  [M][N]
 * Alignment: x_q, w_bits, w_a, w_b (and x, except in dfssm_quantize_act) must be
 * 16-byte aligned; s_x, s_w, s_a, s_b, t, y, acc_dbg need 4-byte alignment.
 * Allocator-returned buffers satisfy both.
 *
 * Ownership and threading: the caller owns every buffer; the library keeps
 * pointers only for the duration of a call, allocates no memory, never
 * synchronizes the stream, and enqueues all work on `stream` (0 = the default
 * stream), so calls may be captured in a HIP graph.  Calls on different streams
 * are independent as long as their output buffers do not overlap.
 *
 * Errors: arguments are validated on the host before anything is enqueued; on a
 * validation error nothing is launched.  DFSSM_ERR_HIP reports a launch failure
 * (hipGetLastError after the launch).  Non-finite x is a documented precondition
 * violation: results are then unspecified.
 *
 * Batched forms: `batch` independent problems of identical shape in one launch
 * (each layer's projection has its own scaffold and LoRA pair; independent
 * inputs -- rotated weight copies, layers fed independent activations -- can
 * share the launch cost).  Operands of problem p follow those of problem p-1
 * densely in every buffer: x + p*M*K, x_q + p*M*K, s_x + p*M, w_bits + p*N*K/8,
 * s_w + p*N, w_a + p*N*16, s_a + p*N, w_b + p*16*K, s_b + p*16, t + p*M*16,
 * y + p*M*N, acc_dbg + p*M*N.  1 <= batch <= 65535.
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
    DFSSM_ERR_INVALID_ARG = 1,   /* NULL required pointer, size <= 0, K % 8 != 0 (gemm), misaligned pointer */
    DFSSM_ERR_UNSUPPORTED = 2,   /* rank other than 0 or 16, K > 131072, batch > 65535 */
    DFSSM_ERR_HIP = 3            /* the HIP runtime reported an error for a launch */
} dfssm_status;

/* Human-readable name of a status code (static storage, never NULL). */
const char* dfssm_status_string(dfssm_status status);

/* Library version as major*100 + minor. */
int32_t dfssm_version(void);

/* The tile plan the int8 MFMA kernel takes for a dfssm_scaffold_lora_gemm[_strided_batched]
 * call of this shape, as its cost model picks it (the DFSSM_PREFILL_CFG / _TAIL pins are
 * not applied).  Host only: launches nothing and needs no GPU.  A testing and tuning
 * aid.  Outputs (host pointers, written on DFSSM_OK):
 *   main_cfg  the configuration of columns [0, n_split) (0, 1, ...)
 *   tail_cfg  the configuration of columns [n_split, N), or -1 (then n_split = N)
 * Configurations: 0 128x512 (4 waves), 1 128x128 split-K 2, 2 128x64 split-K 2,
 * 3 128x512 (8 waves), 4 128x128 split-K 2 (8 waves), 5 64x128 split-K 2 (8 waves),
 * 6 64x64 split-K 4 (8 waves), 7 128x256 (4 waves, two groups per CU), 8 64x64
 * split-K 2 (4 waves, two groups per CU).
 * Returns DFSSM_ERR_INVALID_ARG for NULL outputs or sizes the call would reject, and
 * DFSSM_ERR_UNSUPPORTED when the call would take another kernel: the decode kernel
 * (M <= 16) or the generic one (K % 64 != 0), or K > 131072. */
dfssm_status dfssm_prefill_plan(int64_t M, int64_t N, int64_t K, int64_t batch, int32_t* main_cfg,
                                int32_t* tail_cfg, int64_t* n_split);

/*
 * Per-token absmax int8 quantization of activations, the int8 operand of the
 * scaffold product (technical summary section 2C).
 *   x    fp32 [M][K], read
 *   x_q  int8 [M][K], written
 *   s_x  fp32 [M],    written (0 for an all-zero token, whose codes are all 0)
 * Requires M >= 1, K >= 1.  Bit-exact with the IEEE definition above.
 */
dfssm_status dfssm_quantize_act(const float* x, int64_t M, int64_t K,
                                int8_t* x_q, float* s_x, hipStream_t stream);

/*
 * LoRA down-projection t = W_B x_q in exact int32 (technical summary section 2B).
 *   x_q int8 [M][K], w_b int8 [rank][K], t int32 [M][rank] (written).
 * rank must be 16 (DFSSM_ERR_UNSUPPORTED otherwise); K <= 131072 keeps
 * |t| <= 127*127*K within int32.
 */
dfssm_status dfssm_lora_down(const int8_t* x_q, int64_t M, int64_t K, const int8_t* w_b, int32_t rank,
                             int32_t* t, hipStream_t stream);
dfssm_status dfssm_lora_down_strided_batched(const int8_t* x_q, int64_t M, int64_t K, const int8_t* w_b,
                                             int32_t rank, int32_t* t, int64_t batch, hipStream_t stream);

/*
 * dfssm_quantize_act and dfssm_lora_down fused into one kernel: writes x_q, s_x and
 * (rank 16) t.  With rank 0, w_b and t may be NULL and only x_q, s_x are written.
 * Results are identical to the two separate calls.
 */
dfssm_status dfssm_quantize_lora_down(const float* x, int64_t M, int64_t K, const int8_t* w_b, int32_t rank,
                                      int8_t* x_q, float* s_x, int32_t* t, hipStream_t stream);
dfssm_status dfssm_quantize_lora_down_strided_batched(const float* x, int64_t M, int64_t K,
                                                      const int8_t* w_b, int32_t rank, int8_t* x_q,
                                                      float* s_x, int32_t* t, int64_t batch,
                                                      hipStream_t stream);

/*
 * Scaffold product with the fused LoRA + scale epilogue (technical summary section 2B,
 * "Frozen Scaffold with LoRA Correction": W_A d_out x r, W_B r x d_in, r = 16, int8 with
 * per-row scales; section 2C, "Optimized Inference Pipeline": packed 1-bit weights
 * expanded on the fly to int8 for an int8 x int8 product):
 *   t   = W_B x_q                                       (exact int32, computed here)
 *   y   = s_x . (s_w . (W x_q) + s_A . W_A (s_B . t))
 *   x_q, s_x     int8 [M][K] and fp32 [M]: quantized activations (dfssm_quantize_act)
 *   w_bits, s_w  the 1-bit scaffold [N][K/8] and its per-output-channel scale [N]
 *   w_a, s_a     LoRA up, int8 [N][rank] and fp32 [N]
 *   w_b, s_b     LoRA down, int8 [rank][K] and fp32 [rank]
 *   rank         16, or 0 for no correction (then w_a, s_a, w_b, s_b may be NULL)
 *   y            fp32 [M][N], written
 *   acc_dbg      optional int32 [M][N]: when not NULL, also receives the exact scaffold
 *                accumulators sum_k w x_q (verification aid; NULL in timed runs)
 *   t_dbg        optional int32 [M][rank]: when not NULL (rank 16), also receives t
 *                (verification aid; NULL in timed runs)
 * Requires M, N >= 1, K >= 8, K % 8 == 0, K <= 131072.  M <= 16 (with K <= 16384)
 * runs the bandwidth-bound decode kernel, whose every workgroup computes t for the
 * tokens from W_B (16 K bytes, L2-resident) before streaming its rows; otherwise an int8
 * MFMA kernel (tile configuration chosen by a cost model of the shape; K % 64 != 0
 * takes a generic fallback kernel) computes each tile's rows of t inside its K loop,
 * from the code chunks it already stages.  Either way one kernel launch and no scratch
 * memory.  For tests and tuning, the environment variable DFSSM_PREFILL_CFG pins the
 * MFMA kernel's tile configuration (0, 1, ...; -2 = the generic kernel) and
 * DFSSM_PREFILL_TAIL a narrower one for the columns past the pinned one's main part,
 * where the pinned configuration is built with that tail (otherwise every column runs
 * on the pinned one); results are the same either way.
 * Errors: DFSSM_ERR_INVALID_ARG for a NULL x_q, s_x, w_bits, s_w or y, for a NULL w_a,
 * s_a, w_b or s_b at rank 16, for sizes out of range or K % 8 != 0, and for
 * misaligned pointers; DFSSM_ERR_UNSUPPORTED for rank other than 0 and 16 or
 * K > 131072; DFSSM_ERR_HIP for a failed launch.  Nothing is launched on an error.
 */
dfssm_status dfssm_scaffold_lora_gemm(const int8_t* x_q, const float* s_x, int64_t M, int64_t N, int64_t K,
                                      const uint8_t* w_bits, const float* s_w,
                                      const int8_t* w_a, const float* s_a,
                                      const int8_t* w_b, const float* s_b, int32_t rank,
                                      float* y, int32_t* acc_dbg, int32_t* t_dbg, hipStream_t stream);
dfssm_status dfssm_scaffold_lora_gemm_strided_batched(const int8_t* x_q, const float* s_x,
                                                      int64_t M, int64_t N, int64_t K,
                                                      const uint8_t* w_bits, const float* s_w,
                                                      const int8_t* w_a, const float* s_a,
                                                      const int8_t* w_b, const float* s_b, int32_t rank,
                                                      float* y, int32_t* acc_dbg, int32_t* t_dbg,
                                                      int64_t batch, hipStream_t stream);

/*
 * The same product with t given (technical summary sections 2B and 2C): t = W_B x_q
 * from dfssm_lora_down or dfssm_quantize_lora_down, so the kernel reads t instead of
 * W_B.  Results are bit-identical to dfssm_scaffold_lora_gemm on the same x_q.
 *   w_a, s_a, s_b, t, rank  the LoRA up factor, its scales and t int32 [M][rank];
 *                rank 16, or 0 for no correction (then w_a, s_a, s_b, t may be NULL)
 * Other arguments, requirements and errors as dfssm_scaffold_lora_gemm (a NULL t at
 * rank 16 is DFSSM_ERR_INVALID_ARG).
 */
dfssm_status dfssm_scaffold_lora_gemm_given_t(const int8_t* x_q, const float* s_x,
                                              int64_t M, int64_t N, int64_t K,
                                              const uint8_t* w_bits, const float* s_w,
                                              const int8_t* w_a, const float* s_a, const float* s_b,
                                              const int32_t* t, int32_t rank,
                                              float* y, int32_t* acc_dbg, hipStream_t stream);
dfssm_status dfssm_scaffold_lora_gemm_given_t_strided_batched(const int8_t* x_q, const float* s_x,
                                                              int64_t M, int64_t N, int64_t K,
                                                              const uint8_t* w_bits, const float* s_w,
                                                              const int8_t* w_a, const float* s_a,
                                                              const float* s_b, const int32_t* t, int32_t rank,
                                                              float* y, int32_t* acc_dbg,
                                                              int64_t batch, hipStream_t stream);

/*
 * The whole projection in one call (technical summary sections 2B and 2C; the
 * formulas above): x -> x_q, s_x, t and y, with the same results, bit for bit, as
 * dfssm_quantize_lora_down followed by dfssm_scaffold_lora_gemm_given_t.
 *   x                      fp32 [M][K], read
 *   w_bits, s_w            the scaffold and its scale
 *   w_a, s_a, w_b, s_b     the LoRA pair and its scales (rank 16), or rank 0 with
 *                          all four (and t) NULL
 *   x_q, s_x, t            written (the quantized tokens, their scales, t = W_B x_q)
 *   y                      fp32 [M][N], written
 *   acc_dbg                optional int32 [M][N] scaffold accumulators
 * Decode shapes run as ONE kernel launch: K % 128 == 0, K <= 4096, M <= 4 and
 * M*K <= 1024 * (waves per group: 1 for K <= 512, 2 for K <= 1024, 4 for K <= 2048,
 * 8 up to 4096) -- e.g. M = 1, 2 at K = 4096 and K = 2048.  Every workgroup then
 * quantizes the tokens and computes t itself; the first workgroup of each problem
 * writes x_q, s_x and t.  Large batches that would spread one problem over several
 * workgroups (which would each redo that work), and all other shapes, take two
 * kernels: at rank 16, shapes past the decode kernel (M > 16 or K > 16384) with
 * M*N*batch < 2^24 and K % 64 == 0 the quantizer, then the product computing t in its
 * K loop (the form dfssm_scaffold_lora_gemm runs), which writes t out as well; the
 * rest those of the two-call form.
 * Requirements and errors are the union of the two calls'.
 */
dfssm_status dfssm_scaffold_lora_forward(const float* x, int64_t M, int64_t N, int64_t K,
                                         const uint8_t* w_bits, const float* s_w,
                                         const int8_t* w_a, const float* s_a,
                                         const int8_t* w_b, const float* s_b, int32_t rank,
                                         int8_t* x_q, float* s_x, int32_t* t,
                                         float* y, int32_t* acc_dbg, hipStream_t stream);
dfssm_status dfssm_scaffold_lora_forward_strided_batched(const float* x, int64_t M, int64_t N, int64_t K,
                                                         const uint8_t* w_bits, const float* s_w,
                                                         const int8_t* w_a, const float* s_a,
                                                         const int8_t* w_b, const float* s_b, int32_t rank,
                                                         int8_t* x_q, float* s_x, int32_t* t,
                                                         float* y, int32_t* acc_dbg,
                                                         int64_t batch, hipStream_t stream);

/*
 * int8 LM head: the model's int8 embedding / LM-head matrix E [N][K] (N = vocabulary,
 * K = model width) with one fp32 scale per row (technical summary: embedding and LM
 * head quantized to int8 with per-row scaling), applied to M tokens' int8 codes:
 *   acc[m][n] = sum_k E[n][k] * x_q[m][k]        (exact int32)
 *   y[m][n]   = s_x[m] * (s_e[n] * acc[m][n])    (fp32)
 * x_q, s_x are the tokens' per-token absmax codes (dfssm_quantize_act), the same as
 * the projections take.  The pages leave the head's activation precision open; this
 * int8 x int8 reading matches the rest of the int8 path.
 *   x_q  int8 [M][K] (16-byte aligned), s_x fp32 [M]
 *   e    int8 [N][K] (16-byte aligned), s_e fp32 [N]
 *   y    fp32 [M][N], written; acc_dbg optional int32 [M][N] (verification aid)
 * Requires K % 16 == 0 (DFSSM_ERR_INVALID_ARG otherwise); DFSSM_ERR_UNSUPPORTED for
 * M > 16, K > 4096, or (N + 128) * K >= 2^31.  One kernel launch, bandwidth-bound
 * (N K bytes per problem).  Batched form: operands of problem p at x_q + p*M*K,
 * s_x + p*M, e + p*N*K, s_e + p*N, y + p*M*N, acc_dbg + p*M*N.
 */
dfssm_status dfssm_int8_rowscale_gemm(const int8_t* x_q, const float* s_x, int64_t M, int64_t N, int64_t K,
                                      const int8_t* e, const float* s_e, float* y, int32_t* acc_dbg,
                                      hipStream_t stream);
dfssm_status dfssm_int8_rowscale_gemm_strided_batched(const int8_t* x_q, const float* s_x, int64_t M, int64_t N,
                                                      int64_t K, const int8_t* e, const float* s_e, float* y,
                                                      int32_t* acc_dbg, int64_t batch, hipStream_t stream);

/*
 * Embedding lookup from the same int8 matrix: out[t][k] = s_e[id] * E[id][k] (one fp32
 * product) for id = tokens[t].  An id outside [0, V) gives a row of zeros (ids live in
 * device memory, so they are not checked on the host).
 *   tokens int32 [T], e int8 [V][K], s_e fp32 [V], out fp32 [T][K] (written)
 * Requires T, V, K >= 1; V*K and T*K below 2^40.
 */
dfssm_status dfssm_embedding_lookup(const int32_t* tokens, int64_t T, const int8_t* e, const float* s_e,
                                    int64_t V, int64_t K, float* out, hipStream_t stream);

/*
 * Mamba-2 decode step between in_proj and out_proj, for S sequences (technical
 * summary, section 2C, Stateful Ops: the stateful shift register -- the causal
 * convolution -- and the SSM recurrence; the arithmetic is the published Mamba-2
 * single-token step, one group):
 *   in_proj row = [z (d_inner) | xBC (conv_dim) | dt (nheads)],
 *       d_inner = nheads * headdim, conv_dim = d_inner + 2 * d_state
 *   window[c] <- [window[c][1..3], xBC[c]];  a = silu(sum_j conv_w[c][j] window[c][j] + conv_b[c])
 *   x (nheads x headdim) | B (d_state) | C (d_state) = a
 *   dt = softplus(dt + dt_bias) (identity above 20), dA = exp(-dt * exp(A_log))
 *   state[h][p][n] = state[h][p][n] * dA[h] + (dt[h] * x[h][p]) * B[n]
 *   y[h][p] = sum_n state[h][p][n] * C[n] + D[h] * x[h][p]
 *   out = g / sqrt(mean(g^2) + eps) * norm_w,  g = y * silu(z)   (out_proj's input)
 * Arguments (fp32, device memory; per sequence s the rows below are offset by s):
 *   zxbcdt         [S][d_inner + conv_dim + nheads]   the in_proj output (read)
 *   conv_state_in  [S][conv_dim][4]  the windows, oldest first (read; 16-byte aligned)
 *   conv_state_out [S][conv_dim][4]  the advanced windows (written; 16-byte aligned;
 *                  must not overlap conv_state_in: every group of a sequence reads the
 *                  B and C windows that one of them rewrites)
 *   ssm_state      [S][nheads][headdim][d_state]  updated in place (16-byte aligned)
 *   conv_w [conv_dim][4] (16-byte aligned), conv_b [conv_dim], dt_bias, A_log, D [nheads],
 *   norm_w [d_inner] (16-byte aligned), eps >= 0
 *   out            [S][d_inner] (written; 16-byte aligned; must not overlap zxbcdt)
 * Requires 1 <= S <= 65535; DFSSM_ERR_UNSUPPORTED unless headdim == 64, d_state == 128
 * and 1 <= nheads <= 1024 (Mamba-2 1.3B: nheads 64).  Two kernel launches on `stream`.
 * Non-finite inputs are a precondition violation (outputs undefined).
 */
dfssm_status dfssm_mamba2_decode_step(const float* zxbcdt, int64_t S, int64_t nheads, int64_t headdim,
                                      int64_t d_state, const float* conv_state_in, float* conv_state_out,
                                      float* ssm_state, const float* conv_w, const float* conv_b,
                                      const float* dt_bias, const float* A_log, const float* D,
                                      const float* norm_w, float eps, float* out, hipStream_t stream);

/*
 * The decode step of a stack of n_layers DF-SSM layers for one sequence (one token), in
 * ONE kernel launch (technical summary section 2C, "Optimized Inference Pipeline": the
 * whole 48-layer forward is captured as one graph because launch overhead decides
 * batch-1 speed).  Per layer l, with the layer's input x (fp32 [2048]):
 *   zxbcdt = scaffold_lora(quantize(x); in_proj weights of l)       (K 2048 -> N 8512)
 *   out    = Mamba-2 step of dfssm_mamba2_decode_step (64 heads x 64 channels,
 *            d_state 128, eps) on zxbcdt, with layer l's windows and state
 *   x'     = scaffold_lora(quantize(out); out_proj weights of l)    (K 4096 -> N 2048)
 * and x' is layer l + 1's input; x_out receives the last layer's x'.  Every arithmetic
 * step is the one the single-projection entry points and dfssm_mamba2_decode_step
 * define (the same quantizer, exact int32 products, the same fp32 epilogue and step).
 * Model sizes are fixed to Mamba-2 1.3B's: d_model 2048, d_inner 4096, 64 heads,
 * d_state 128, convolution width 4, in_proj width 8512.
 *
 * Weights (device memory, densely stacked over the layers; layer l's block follows
 * layer l - 1's; 16-byte aligned where a row is read as a vector: the bits, W_A, W_B,
 * conv_w, norm_w):
 *   in_w_bits uint8 [L][8512][256]  in_s_w fp32 [L][8512]  in_w_a int8 [L][8512][16]
 *   in_s_a fp32 [L][8512]  in_w_b int8 [L][16][2048]  in_s_b fp32 [L][16]
 *   conv_w fp32 [L][4352][4]  conv_b, dt_bias, A_log, D fp32 [L][4352], [L][64] x 3
 *   norm_w fp32 [L][4096]
 *   out_w_bits uint8 [L][2048][512]  out_s_w fp32 [L][2048]  out_w_a int8 [L][2048][16]
 *   out_s_a fp32 [L][2048]  out_w_b int8 [L][16][4096]  out_s_b fp32 [L][16]
 * State and activations (device memory):
 *   x_in  fp32 [2048] (16-byte aligned), read;  x_out fp32 [2048], written (may alias x_in)
 *   conv_state_in [L][4352][4] read, conv_state_out [L][4352][4] written (16-byte
 *     aligned, must not overlap: the caller swaps them between tokens)
 *   ssm_state fp32 [L][64][64][128], updated in place (16-byte aligned)
 *   trace  optional uint32 [L][dfssm_decode_layers_trace_words()]: when not NULL, each
 *     layer's intermediates, at these word offsets: zxbcdt fp32 [8512] at 0, out fp32
 *     [4096] at 8512, x' fp32 [2048] at 12608, in_proj accumulators int32 [8512] at
 *     14656, out_proj accumulators int32 [2048] at 23168, x_q of x int8 [2048] at 25216,
 *     x_q of out int8 [4096] at 25728, t of in_proj int32 [16] at 26752, t of out_proj
 *     int32 [16] at 26768, s_x of x and of out fp32 at 26784 and 26785 (verification aid)
 * The layer's three steps exchange their outputs through `workspace` (>=
 * dfssm_decode_layers_workspace_bytes() bytes, 16-byte aligned): each value is stored
 * with a tag naming the call, the layer and the step, and its readers wait for the tag.
 * The caller zeroes the workspace once before its first use and then leaves it to the
 * library between calls (it holds a call counter that the tags carry; re-zeroing it is
 * allowed only together with all of it).  Calls that share a workspace must not overlap
 * (the same stream serializes them).
 *   status     int32 in device memory: each wait that gives up ORs a bit in --
 *              DFSSM_DECODE_STATUS_TIMEOUT (its poll limit passed) or
 *              DFSSM_DECODE_STATUS_GAVE_UP (another group had failed); outputs are
 *              then unspecified.  The kernel never hangs: every wait is bounded.  The
 *              caller clears it; the library only ORs into it.
 *   spin_limit polls per wait before it gives up (<= 0: 1 << 22, far beyond any wait
 *              of a healthy run)
 *   flags      0, or DFSSM_DECODE_UNREACHABLE_WAITS (a test aid: every wait's target is
 *              unreachable, so every wait times out and the kernel still ends)
 * Requires 1 <= n_layers <= 64 and eps >= 0.  DFSSM_ERR_UNSUPPORTED when the device
 * cannot hold the persistent grid (256 co-resident 512-thread groups in a cooperative
 * launch: MI355X's 256 CUs); DFSSM_ERR_INVALID_ARG for a NULL or misaligned pointer, a
 * short workspace, overlapping windows or sizes out of range.  One launch on `stream`,
 * nothing allocated; not for HIP graph capture (a cooperative launch).
 */
typedef struct dfssm_decode_layer_weights {
    const uint8_t* in_w_bits;
    const float* in_s_w;
    const int8_t* in_w_a;
    const float* in_s_a;
    const int8_t* in_w_b;
    const float* in_s_b;
    const float* conv_w;
    const float* conv_b;
    const float* dt_bias;
    const float* A_log;
    const float* D;
    const float* norm_w;
    const uint8_t* out_w_bits;
    const float* out_s_w;
    const int8_t* out_w_a;
    const float* out_s_a;
    const int8_t* out_w_b;
    const float* out_s_b;
} dfssm_decode_layer_weights;

#define DFSSM_DECODE_STATUS_TIMEOUT 1
#define DFSSM_DECODE_STATUS_GAVE_UP 2
#define DFSSM_DECODE_UNREACHABLE_WAITS 1u

size_t dfssm_decode_layers_workspace_bytes(void);
int64_t dfssm_decode_layers_trace_words(void);
dfssm_status dfssm_decode_layers(const dfssm_decode_layer_weights* w, int64_t n_layers,
                                 const float* x_in, float* x_out,
                                 const float* conv_state_in, float* conv_state_out, float* ssm_state,
                                 float eps, void* workspace, size_t workspace_bytes, int32_t* status,
                                 uint32_t* trace, int64_t spin_limit, uint32_t flags, hipStream_t stream);

/*
 * dfssm_decode_layers for callers that cannot allocate device memory (code that must
 * not call hipMalloc: tight serving loops, harnesses that forbid it).  Same arguments,
 * results and errors, minus the workspace: the library's own array of
 * dfssm_decode_layers_workspace_bytes() bytes per GPU (a file-scope device array, held
 * until the process ends; zeroed on `stream` the first time a device is used) serves
 * instead, so nothing is allocated or freed.  The array's size covers the largest stack
 * the call accepts (n_layers <= 64; larger is DFSSM_ERR_INVALID_ARG).  Every call on one
 * GPU shares that GPU's array: calls that overlap on one GPU (other streams, other
 * threads) race, so the caller serializes them (one stream does).  DFSSM_ERR_HIP if the array's device
 * address cannot be obtained.
 */
dfssm_status dfssm_decode_layers_noalloc(const dfssm_decode_layer_weights* w, int64_t n_layers,
                                         const float* x_in, float* x_out,
                                         const float* conv_state_in, float* conv_state_out, float* ssm_state,
                                         float eps, int32_t* status, uint32_t* trace, int64_t spin_limit,
                                         uint32_t flags, hipStream_t stream);

/*
 * The density-field state codec (technical summary section 2D, "Density Field State
 * Representation": a binary field of about 4 d_state cells per state element, through
 * normalization, sigma-delta injection with error feedback, binarization and a
 * popcount readout, applied at chunk boundaries).  A state element is one row of
 * d_state fp32 values (one channel of one head of the SSM state, e.g. [S][64][64][128]
 * is 4096 S rows of 128).  Per row, with value n owning cells 4n .. 4n + 3:
 *   s   = max_n |v_n|                       (scale, fp32)
 *   u_n = (v_n / s + 1) / 2                 (IEEE division; 1/2 when s = 0)
 *   cells in order, e = 0 at the row's start: w = u_n + e; cell = (w >= 1/2); e = w - cell
 *   readout v'_n = s * (popcount(cells of n) * 0.5 - 1)   (s times -1, -1/2, 0, 1/2 or 1)
 * Field layout: uint32 [rows][d_state / 8]; cell c is bit c % 32 of word c / 32, so value
 * n is nibble n % 8 of word n / 8 (the notional K x K field, K = ceil(sqrt(4 d_state)),
 * keeps its remaining K^2 - 4 d_state cells at 0; they are not stored).
 *   state  fp32 [rows][d_state] (16-byte aligned)
 *   field  uint32 [rows][d_state / 8] (16-byte aligned)   scale fp32 [rows]
 * d_state must be 64, 128 or 256 (DFSSM_ERR_UNSUPPORTED otherwise); rows >= 1 and
 * rows * d_state < 2^40.  Non-finite state values are a precondition violation.
 *   encode:      state -> field, scale
 *   decode:      field, scale -> state (the readout)
 *   requantize:  the round trip at a chunk boundary, in place: state <- readout of its
 *                own field; field and scale are also written when not NULL
 * One kernel launch each on `stream`; nothing is allocated.
 */
dfssm_status dfssm_density_field_encode(const float* state, int64_t rows, int64_t d_state, uint32_t* field,
                                        float* scale, hipStream_t stream);
dfssm_status dfssm_density_field_decode(const uint32_t* field, const float* scale, int64_t rows, int64_t d_state,
                                        float* state, hipStream_t stream);
dfssm_status dfssm_density_field_requantize(float* state, int64_t rows, int64_t d_state, uint32_t* field,
                                            float* scale, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DFSSM_H */
