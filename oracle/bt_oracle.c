/*
 * bt_oracle.c -- plain, slow CPU oracle for the BitNet b1.58 W1.58A8 ternary
 * linear layer.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg load this code. The product (the HIP library) never calls it,
 * shares no source, header, table or helper with it, and does not fall back to
 * it. It is compiled with gcc -O2 -fno-fast-math -ffp-contract=off so every
 * floating-point step below is one IEEE-754 operation in the stated precision
 * (x86-64 SSE: float math is evaluated in float, double in double, RNE).
 *
 * What is computed, and where the pages define it:
 *  - absmean weight scale and ternarization to {-1,0,+1}: "bit-floor" page,
 *    "What's inside" table (pack.rs: a mean-abs threshold picks which weights
 *    become zero), with the per-tensor absmean of the BitNet b1.58 method.
 *  - per-token absmax int8 activations: BitNet GPU guide ("How to Run BitNet
 *    Inference on GPU Using CUDA Kernels"), section "Understanding the
 *    Two-Phase Architecture" (BitLinearKernel quantizes inputs to INT8 with
 *    their own scales), and the "bit-floor" page, "What's inside" (scale.rs:
 *    absmax, activations quantized on the fly before each GEMV).
 *  - integer-only ternary product: "BitCompute" page, section "Features"
 *    (multiplying by -1, 0 or 1 is an add, a subtract or a skip) and the
 *    "bit-floor" page, section "The core math" (no floating point until the
 *    final scale multiply: y = scale_w * scale_x * integer dot).
 *
 * Readings taken where the pages are silent or ambiguous:
 *  R1  one scale gamma per weight matrix;
 *  R2  gamma = mean |W| summed in fp64, each row summed k = 0..K-1, then the
 *      row sums summed n = 0..N-1, divided once by N*K and rounded once to fp32;
 *  R3  t = RoundClip(W / gamma, -1, 1) with round-half-to-even, evaluated as
 *      the exact compare |w| > gamma/2 (gamma/2 is an exact fp32 halving), so
 *      |w| == gamma/2 gives 0; gamma == 0 gives threshold 0;
 *  R4  per-token absmax a = max_k |x|, inv = 127.0f / a (fp32, correctly
 *      rounded), q = clamp(rint(x * inv), -127, 127) with rint half-to-even,
 *      s_x = a / 127.0f; a zero row gives q = 0 and s_x = 0;
 *  R5  y = acc * gamma * s_x evaluated in fp64 and rounded once to fp32;
 *  R6  non-finite inputs are outside the contract: the oracle rejects them;
 *  R12 row-group scales (the "_rows" functions): the rows of W are cut, in order,
 *      into groups that are separate matrices stored one above the other (the Q,
 *      K and V blocks of a fused projection; one row per group at the finest);
 *      each group gets the R2 scale of its own rows, its codes use that scale
 *      (R3), and y uses the scale of its output row (R5 with gamma_n).
 *  R13 1-bit operands (the binary W1A1 and the ternary-weight W1.58A1 products):
 *      a value binarizes to +1 when v >= 0 and to -1 when v < 0; the scale of a
 *      binarized weight matrix is its absmax, that of a binarized token its
 *      absmax; y = acc * scale_w * scale_x as in R5 (scale_w = gamma for
 *      ternary weights).
 *
 * Every entry point returns 0 on success and 1 when an input is not finite
 * (2 when the row groups do not cover the N rows exactly).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* gamma = mean |W| over the whole [N,K] matrix (readings R1, R2).
 * Follows the "bit-floor" page, "What's inside" (pack.rs, mean-abs scale for
 * ternary weights) and the absmean named by the BitNet b1.58 method. */
int oracle_absmean(const float *W, int64_t N, int64_t K, float *gamma_out)
{
    if (N <= 0 || K <= 0) {
        /* An empty matrix has no weights; its scale is defined as 0. */
        *gamma_out = 0.0f;
        return 0;
    }
    double total = 0.0;
    for (int64_t n = 0; n < N; ++n) {
        double row = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            float w = W[n * K + k];
            if (!isfinite(w))
                return 1;
            row += fabs((double)w);
        }
        total += row;
    }
    *gamma_out = (float)(total / (double)(N * K));
    return 0;
}

/* t[n,k] = RoundClip(W[n,k] / gamma, -1, 1) as an exact compare (R3).
 * Follows the "bit-floor" page, "What's inside" (pack.rs: the mean-abs
 * threshold suppresses small weights to zero; the rest keep their sign). */
int oracle_ternarize(const float *W, int64_t N, int64_t K, float gamma, int8_t *T)
{
    const float half = gamma * 0.5f;
    for (int64_t i = 0; i < N * K; ++i) {
        float w = W[i];
        if (!isfinite(w))
            return 1;
        if (w > half)
            T[i] = 1;
        else if (w < -half)
            T[i] = -1;
        else
            T[i] = 0;
    }
    return 0;
}

/* Per-token absmax int8 quantization of X [M,K] (R4). Writes Q [M,K],
 * s_x [M] (the dequantization factor a/127) and qsum [M] = sum_k Q[m,k].
 * Follows the BitNet GPU guide, "Understanding the Two-Phase Architecture"
 * (inputs quantized to INT8 with per-row scales before the kernel call) and
 * the "bit-floor" page, "What's inside" (scale.rs: absmax scale, activations
 * quantized before each GEMV). */
int oracle_quant_act(const float *X, int64_t M, int64_t K, int8_t *Q, float *s_x,
                     int32_t *qsum)
{
    for (int64_t m = 0; m < M; ++m) {
        const float *x = X + m * K;
        float a = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            if (!isfinite(x[k]))
                return 1;
            float v = fabsf(x[k]);
            if (v > a)
                a = v;
        }
        if (a == 0.0f) {
            memset(Q + m * K, 0, (size_t)K);
            s_x[m] = 0.0f;
            qsum[m] = 0;
            continue;
        }
        const float inv = 127.0f / a;
        int32_t sum = 0;
        for (int64_t k = 0; k < K; ++k) {
            float r = rintf(x[k] * inv);
            if (r > 127.0f)
                r = 127.0f;
            if (r < -127.0f)
                r = -127.0f;
            Q[m * K + k] = (int8_t)r;
            sum += (int32_t)r;
        }
        s_x[m] = a / 127.0f;
        qsum[m] = sum;
    }
    return 0;
}

/* acc[m,n] = sum_k T[n,k] * Q[m,k] in int32: the naive triple loop.
 * Follows the "BitCompute" page, "Features" (a ternary weight turns the
 * product into add / subtract / skip) and the "bit-floor" page, "The core
 * math" (integer inner loop). |acc| <= 127*K, so int32 cannot overflow for
 * K < 2^24. */
int oracle_ternary_matmul(const int8_t *T, const int8_t *Q, int64_t M, int64_t N,
                          int64_t K, int32_t *acc)
{
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int32_t s = 0;
            for (int64_t k = 0; k < K; ++k)
                s += (int32_t)T[n * K + k] * (int32_t)Q[m * K + k];
            acc[m * N + n] = s;
        }
    }
    return 0;
}

/* y[m,n] = acc[m,n] * gamma * s_x[m], in fp64, rounded once to fp32 (R5).
 * Follows the "bit-floor" page, "The core math" (the output is the weight
 * scale times the activation scale times the integer dot product). */
int oracle_scale_epilogue(const int32_t *acc, float gamma, const float *s_x,
                          int64_t M, int64_t N, float *Y)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            Y[m * N + n] = (float)((double)acc[m * N + n] * (double)gamma * (double)s_x[m]);
    return 0;
}

/* Row-group weight scales (R12): the rows are cut, in order, into nseg groups of
 * seg_rows[s] >= 1 rows (seg_rows == NULL: each of the N rows is its own group);
 * row_scale[n] receives the mean |W| of row n's group alone, summed as in R2.
 * Follows the BitNet GPU guide, "Frequently Asked Questions" (the kernel wrapper
 * assumes model-specific quantization scales and group dimensions). */
int oracle_absmean_rows(const float *W, int64_t N, int64_t K, const int64_t *seg_rows,
                        int64_t nseg, float *row_scale)
{
    const int64_t groups = seg_rows ? nseg : N;
    int64_t n0 = 0;
    for (int64_t s = 0; s < groups; ++s) {
        const int64_t rows = seg_rows ? seg_rows[s] : 1;
        if (rows < 1 || n0 + rows > N)
            return 2;
        float g;
        if (oracle_absmean(W + n0 * K, rows, K, &g))
            return 1;
        for (int64_t n = n0; n < n0 + rows; ++n)
            row_scale[n] = g;
        n0 += rows;
    }
    return n0 == N ? 0 : 2;
}

/* Codes of every row against its own scale (R3 with gamma_n, R12). */
int oracle_ternarize_rows(const float *W, int64_t N, int64_t K, const float *row_scale,
                          int8_t *T)
{
    for (int64_t n = 0; n < N; ++n)
        if (oracle_ternarize(W + n * K, 1, K, row_scale[n], T + n * K))
            return 1;
    return 0;
}

/* y[m,n] = acc[m,n] * gamma_n * s_x[m], in fp64, rounded once to fp32 (R5, R12).
 * Follows the "bit-floor" page, "The core math" (weight scale times activation
 * scale times the integer dot), with the weight scale of output row n. */
int oracle_scale_epilogue_rows(const int32_t *acc, const float *row_scale, const float *s_x,
                               int64_t M, int64_t N, float *Y)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            Y[m * N + n] = (float)((double)acc[m * N + n] * (double)row_scale[n] * (double)s_x[m]);
    return 0;
}

/* max |V[r, :]| of every row of V [R,C] (R13; an empty row gives 0). A matrix's absmax
 * is this with R = 1 over all its entries. Follows the "bit-floor" page, "What's
 * inside" (pack.rs: absmax scale for binary weights; scale.rs: absmax scales). */
int oracle_absmax_rows(const float *V, int64_t R, int64_t C, float *amax)
{
    for (int64_t r = 0; r < R; ++r) {
        float a = 0.0f;
        for (int64_t c = 0; c < C; ++c) {
            const float v = V[r * C + c];
            if (!isfinite(v))
                return 1;
            if (fabsf(v) > a)
                a = fabsf(v);
        }
        amax[r] = a;
    }
    return 0;
}

/* B = +1 where V >= 0, -1 where V < 0 (R13): one bit per value. Follows the
 * "bit-floor" page, "The core math" (binary weights are +1 or -1) and "What's
 * inside" (scale.rs: activations quantized to packed bits before each GEMV). */
int oracle_binarize(const float *V, int64_t R, int64_t C, int8_t *B)
{
    for (int64_t i = 0; i < R * C; ++i) {
        if (!isfinite(V[i]))
            return 1;
        B[i] = V[i] >= 0.0f ? 1 : -1;
    }
    return 0;
}
