/*
 * dfssm_oracle.c -- plain, slow CPU oracle for the DF-SSM scaffold projection.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or load
 * this file: only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark use it.  It shares no code, header, table or helper with the HIP
 * library.
 *
 * What it computes (DF-SSM, "Density Field State Space Models", technical
 * summary on gist.science, section 2B "Frozen Scaffold with LoRA Correction"
 * and section 2C "Optimized Inference Pipeline"):
 *   - a 1-bit scaffold weight w[n][k] in {-1,+1}, stored as sign bits, eight to
 *     a byte, lowest input index in the least significant bit, bit 1 = +1
 *     (section 2C: packed weights expanded on the fly to int8);
 *   - per-token int8 activations with an fp32 scale (absmax / 127, round half
 *     to even), since the scaffold product is an int8 x int8 contraction
 *     (section 2C: INT8 tensor cores; the CPU path's int8 dot products);
 *   - an int8 rank-16 LoRA pair W_A [d_out x r], W_B [r x d_in] with
 *     per-row scales (section 2B: LoRA module, rank 16, int8 with
 *     per-channel/row scaling).
 *
 * Arithmetic rules (each one written out where it happens below):
 *   amax[m]   = max_k |x[m][k]|
 *   s_x[m]    = fl32(amax / 127)              (0 when amax == 0)
 *   x_q[m][k] = clamp(rint(fl32(x / s_x)), -127, 127) under round-to-nearest-even
 *   acc[m][n] = sum_k w[n][k] * x_q[m][k]     (exact, int64, must fit int32)
 *   t[m][r]   = sum_k W_B[r][k] * x_q[m][k]   (exact, int64, must fit int32)
 *   y[m][n]   = fl32( s_x * ( s_w[n]*acc + s_A[n] * sum_r W_A[n][r]*s_B[r]*t[m][r] ) )
 *               evaluated in fp64 in exactly that order and rounded once.
 *
 * Built with gcc -O1 -ffp-contract=off (no fused multiply-add, no fast-math),
 * so every float operation above is the IEEE operation it says it is.
 */
#include <fenv.h>
#include <math.h>
#include <stdint.h>
#include <stddef.h>

#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1
#define ORACLE_ERR_OVERFLOW 2

/* Per-token absmax int8 quantizer.  Returns ORACLE_OK or ORACLE_ERR_ARG. */
int oracle_quantize_act(const float* x, int64_t M, int64_t K, int8_t* x_q, float* s_x)
{
    if (M < 0 || K < 0) return ORACLE_ERR_ARG;
    if (fegetround() != FE_TONEAREST) fesetround(FE_TONEAREST);
    for (int64_t m = 0; m < M; ++m) {
        const float* row = x + m * K;
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(row[k]);
            if (a > amax) amax = a;
        }
        if (amax == 0.0f) {
            /* all-zero token: scale 0, codes 0, no division */
            s_x[m] = 0.0f;
            for (int64_t k = 0; k < K; ++k) x_q[m * K + k] = 0;
            continue;
        }
        float s = amax / 127.0f;            /* one IEEE fp32 division */
        s_x[m] = s;
        for (int64_t k = 0; k < K; ++k) {
            float v = row[k] / s;            /* IEEE fp32 division */
            float r = rintf(v);              /* round half to even */
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            x_q[m * K + k] = (int8_t)r;
        }
    }
    return ORACLE_OK;
}

/* Sign of scaffold weight (n, k) from the packed bits: bit 1 -> +1, bit 0 -> -1. */
static int sign_at(const uint8_t* w_bits, int64_t K, int64_t n, int64_t k)
{
    uint8_t byte = w_bits[n * (K / 8) + k / 8];
    int bit = (byte >> (k % 8)) & 1;
    return bit ? +1 : -1;
}

/* acc[m][n] = sum_k w[n][k] * x_q[m][k], exact. */
int oracle_scaffold_acc(const int8_t* x_q, int64_t M, int64_t N, int64_t K,
                        const uint8_t* w_bits, int32_t* acc)
{
    if (M < 0 || N < 0 || K < 0 || (K % 8) != 0) return ORACLE_ERR_ARG;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k)
                s += (int64_t)sign_at(w_bits, K, n, k) * (int64_t)x_q[m * K + k];
            if (s > INT32_MAX || s < INT32_MIN) return ORACLE_ERR_OVERFLOW;
            acc[m * N + n] = (int32_t)s;
        }
    return ORACLE_OK;
}

/* t[m][r] = sum_k W_B[r][k] * x_q[m][k], exact (LoRA down-projection). */
int oracle_lora_down(const int8_t* x_q, int64_t M, int64_t K,
                     const int8_t* w_b, int32_t rank, int32_t* t)
{
    if (M < 0 || K < 0 || rank < 0) return ORACLE_ERR_ARG;
    for (int64_t m = 0; m < M; ++m)
        for (int32_t r = 0; r < rank; ++r) {
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k)
                s += (int64_t)w_b[(int64_t)r * K + k] * (int64_t)x_q[m * K + k];
            if (s > INT32_MAX || s < INT32_MIN) return ORACLE_ERR_OVERFLOW;
            t[m * rank + r] = (int32_t)s;
        }
    return ORACLE_OK;
}

/* y for one (m, n) from its integer accumulators, in fp64, rounded once. */
static float y_at(float s_x, float s_w, int32_t acc, float s_a,
                  const int8_t* w_a_row, const float* s_b, const int32_t* t_row, int32_t rank)
{
    double lora = 0.0;
    for (int32_t r = 0; r < rank; ++r)
        lora += (double)w_a_row[r] * (double)s_b[r] * (double)t_row[r];
    double inner = (double)s_w * (double)acc + (double)s_a * lora;
    return (float)((double)s_x * inner);
}

/*
 * Full projection: acc, t and y for all (m, n).  acc and t may be NULL when
 * the caller does not want them.  nthreads > 1 splits the independent output
 * rows n across OpenMP threads; the arithmetic per output is unchanged.
 */
int oracle_scaffold_lora_gemm(const int8_t* x_q, const float* s_x,
                              int64_t M, int64_t N, int64_t K,
                              const uint8_t* w_bits, const float* s_w,
                              const int8_t* w_a, const float* s_a,
                              const int8_t* w_b, const float* s_b, int32_t rank,
                              float* y, int32_t* acc_out, int32_t* t_out, int32_t nthreads)
{
    if (M < 0 || N < 0 || K < 0 || (K % 8) != 0 || rank < 0 || rank > 64) return ORACLE_ERR_ARG;
    int32_t t_local[64];
    int status = ORACLE_OK;
    for (int64_t m = 0; m < M; ++m) {
        /* LoRA down for this token */
        for (int32_t r = 0; r < rank; ++r) {
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k)
                s += (int64_t)w_b[(int64_t)r * K + k] * (int64_t)x_q[m * K + k];
            if (s > INT32_MAX || s < INT32_MIN) return ORACLE_ERR_OVERFLOW;
            t_local[r] = (int32_t)s;
            if (t_out) t_out[m * rank + r] = (int32_t)s;
        }
        int overflow = 0;
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1) reduction(| : overflow)
        for (int64_t n = 0; n < N; ++n) {
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k)
                s += (int64_t)sign_at(w_bits, K, n, k) * (int64_t)x_q[m * K + k];
            if (s > INT32_MAX || s < INT32_MIN) { overflow = 1; continue; }
            if (acc_out) acc_out[m * N + n] = (int32_t)s;
            y[m * N + n] = y_at(s_x[m], s_w[n], (int32_t)s, rank ? s_a[n] : 0.0f,
                                rank ? w_a + n * rank : NULL, s_b, t_local, rank);
        }
        if (overflow) status = ORACLE_ERR_OVERFLOW;
    }
    return status;
}

/*
 * The same projection at an explicit list of output positions (m_idx[i], n_idx[i]),
 * for checks at sizes where the full product would take too long.  Writes y,
 * and acc / t rows when the pointers are not NULL (t is [count][rank]).
 */
int oracle_scaffold_lora_at(const int8_t* x_q, const float* s_x,
                            int64_t M, int64_t N, int64_t K,
                            const uint8_t* w_bits, const float* s_w,
                            const int8_t* w_a, const float* s_a,
                            const int8_t* w_b, const float* s_b, int32_t rank,
                            const int64_t* m_idx, const int64_t* n_idx, int64_t count,
                            float* y, int32_t* acc_out, int32_t* t_out)
{
    if (M < 0 || N < 0 || K < 0 || (K % 8) != 0 || rank < 0 || rank > 64) return ORACLE_ERR_ARG;
    int32_t t_local[64];
    for (int64_t i = 0; i < count; ++i) {
        int64_t m = m_idx[i], n = n_idx[i];
        if (m < 0 || m >= M || n < 0 || n >= N) return ORACLE_ERR_ARG;
        for (int32_t r = 0; r < rank; ++r) {
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k)
                s += (int64_t)w_b[(int64_t)r * K + k] * (int64_t)x_q[m * K + k];
            if (s > INT32_MAX || s < INT32_MIN) return ORACLE_ERR_OVERFLOW;
            t_local[r] = (int32_t)s;
            if (t_out) t_out[i * rank + r] = (int32_t)s;
        }
        int64_t s = 0;
        for (int64_t k = 0; k < K; ++k)
            s += (int64_t)sign_at(w_bits, K, n, k) * (int64_t)x_q[m * K + k];
        if (s > INT32_MAX || s < INT32_MIN) return ORACLE_ERR_OVERFLOW;
        if (acc_out) acc_out[i] = (int32_t)s;
        y[i] = y_at(s_x[m], s_w[n], (int32_t)s, rank ? s_a[n] : 0.0f,
                    rank ? w_a + n * rank : NULL, s_b, t_local, rank);
    }
    return ORACLE_OK;
}

/*
 * int8 embedding / LM head (technical summary: the embedding and LM-head matrices
 * are int8 with per-row scales; one tied matrix E [V][d] serves both).
 *
 * LM head, for M tokens against the V rows of E (here N = V, K = d):
 *   acc[m][n] = sum_k E[n][k] * x_q[m][k]     (exact, int64, must fit int32)
 *   y[m][n]   = fl32( s_x[m] * ( s_e[n] * acc[m][n] ) )   in fp64, rounded once
 * with x_q, s_x the same per-token codes as above (oracle_quantize_act).
 */
int oracle_int8_rowscale_gemm(const int8_t* x_q, const float* s_x, int64_t M, int64_t N, int64_t K,
                              const int8_t* e, const float* s_e, float* y, int32_t* acc_out, int32_t nthreads)
{
    if (M < 0 || N < 0 || K < 0) return ORACLE_ERR_ARG;
    int status = ORACLE_OK;
    for (int64_t m = 0; m < M; ++m) {
        int overflow = 0;
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1) reduction(| : overflow)
        for (int64_t n = 0; n < N; ++n) {
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k)
                s += (int64_t)e[n * K + k] * (int64_t)x_q[m * K + k];
            if (s > INT32_MAX || s < INT32_MIN) { overflow = 1; continue; }
            if (acc_out) acc_out[m * N + n] = (int32_t)s;
            y[m * N + n] = (float)((double)s_x[m] * ((double)s_e[n] * (double)s));
        }
        if (overflow) status = ORACLE_ERR_OVERFLOW;
    }
    return status;
}

/*
 * Embedding lookup: out[t][k] = fl32( s_e[id] * E[id][k] ) for id = tokens[t]; an id
 * outside [0, V) gives a row of zeros.  (The product of an fp32 scale and an int8
 * value is exact in fp64, so rounding it once to fp32 is the fp32 product.)
 */
int oracle_embedding_lookup(const int32_t* tokens, int64_t T, const int8_t* e, const float* s_e,
                            int64_t V, int64_t K, float* out)
{
    if (T < 0 || V < 0 || K < 0) return ORACLE_ERR_ARG;
    for (int64_t t = 0; t < T; ++t) {
        const int64_t id = tokens[t];
        for (int64_t k = 0; k < K; ++k) {
            if (id < 0 || id >= V) {
                out[t * K + k] = 0.0f;
            } else {
                out[t * K + k] = (float)((double)s_e[id] * (double)e[id * K + k]);
            }
        }
    }
    return ORACLE_OK;
}
