/*
 * oracle_driver.c -- runs the CPU oracle's functions on cases read from a file, so that
 * the oracle can be built with AddressSanitizer and UndefinedBehaviorSanitizer as a plain
 * executable (tests/test_oracle_sanitized.py). Every array of a case lives in its own
 * heap block of exactly the size the call is documented to use, so any access outside it
 * is reported. Test infrastructure only.
 *
 * Case file: a sequence of records, each
 *   int32 fn, int64 d0, d1, d2, float f, then the inputs of fn (raw, row-major);
 * results file: per record, int32 return code, then the outputs of fn.
 *   fn 1 absmean          W f32[d0*d1]                         -> gamma f32
 *   fn 2 ternarize        W f32[d0*d1], gamma = f              -> T i8[d0*d1]
 *   fn 3 quant_act        X f32[d0*d1]                         -> Q i8[d0*d1], s f32[d0], qsum i32[d0]
 *   fn 4 ternary_matmul   T i8[d1*d2], Q i8[d0*d2] (M=d0,N=d1,K=d2) -> acc i32[d0*d1]
 *   fn 5 scale_epilogue   acc i32[d0*d1], s f32[d0], gamma = f -> Y f32[d0*d1]
 *   fn 6 absmean_rows     W f32[d0*d1], d2 groups, seg i64[d2] (d2 == 0: one per row) -> scale f32[d0]
 *   fn 7 ternarize_rows   W f32[d0*d1], scale f32[d0]          -> T i8[d0*d1]
 *   fn 8 epilogue_rows    acc i32[d0*d1], scale f32[d1], s f32[d0] -> Y f32[d0*d1]
 *   fn 9 absmax_rows      V f32[d0*d1]                         -> amax f32[d0]
 *   fn 10 binarize        V f32[d0*d1]                         -> B i8[d0*d1]
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_absmean(const float *W, int64_t N, int64_t K, float *gamma_out);
int oracle_ternarize(const float *W, int64_t N, int64_t K, float gamma, int8_t *T);
int oracle_quant_act(const float *X, int64_t M, int64_t K, int8_t *Q, float *s_x, int32_t *qsum);
int oracle_ternary_matmul(const int8_t *T, const int8_t *Q, int64_t M, int64_t N, int64_t K, int32_t *acc);
int oracle_scale_epilogue(const int32_t *acc, float gamma, const float *s_x, int64_t M, int64_t N, float *Y);
int oracle_absmean_rows(const float *W, int64_t N, int64_t K, const int64_t *seg_rows, int64_t nseg,
                        float *row_scale);
int oracle_ternarize_rows(const float *W, int64_t N, int64_t K, const float *row_scale, int8_t *T);
int oracle_scale_epilogue_rows(const int32_t *acc, const float *row_scale, const float *s_x, int64_t M, int64_t N,
                               float *Y);
int oracle_absmax_rows(const float *V, int64_t R, int64_t C, float *amax);
int oracle_binarize(const float *V, int64_t R, int64_t C, int8_t *B);

static FILE *in, *out;

static void *take(size_t bytes)
{
    /* an exact-size block (malloc(0) may return NULL: use a 1-byte block the call never reads) */
    void *p = malloc(bytes ? bytes : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(3);
    }
    if (bytes && fread(p, 1, bytes, in) != bytes) {
        fprintf(stderr, "short case file\n");
        exit(3);
    }
    return p;
}

static void *room(size_t bytes)
{
    void *p = malloc(bytes ? bytes : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(3);
    }
    return p;
}

static void put(const void *p, size_t bytes)
{
    if (bytes && fwrite(p, 1, bytes, out) != bytes)
        exit(4);
}

int main(int argc, char **argv)
{
    if (argc != 3) {
        fprintf(stderr, "usage: %s CASES RESULTS\n", argv[0]);
        return 2;
    }
    in = fopen(argv[1], "rb");
    out = fopen(argv[2], "wb");
    if (!in || !out)
        return 2;
    int32_t fn;
    while (fread(&fn, 4, 1, in) == 1) {
        int64_t d[3];
        float f;
        if (fread(d, 8, 3, in) != 3 || fread(&f, 4, 1, in) != 1)
            return 3;
        const size_t a = (size_t)d[0], b = (size_t)d[1], c = (size_t)d[2];
        int32_t rc = 0;
        switch (fn) {
        case 1: {
            float *W = take(4 * a * b), g = -1.0f;
            rc = oracle_absmean(W, d[0], d[1], &g);
            put(&rc, 4), put(&g, 4);
            free(W);
            break;
        }
        case 2: {
            float *W = take(4 * a * b);
            int8_t *T = room(a * b);
            rc = oracle_ternarize(W, d[0], d[1], f, T);
            put(&rc, 4), put(T, a * b);
            free(W), free(T);
            break;
        }
        case 3: {
            float *X = take(4 * a * b), *s = room(4 * a);
            int8_t *Q = room(a * b);
            int32_t *qs = room(4 * a);
            rc = oracle_quant_act(X, d[0], d[1], Q, s, qs);
            put(&rc, 4), put(Q, a * b), put(s, 4 * a), put(qs, 4 * a);
            free(X), free(s), free(Q), free(qs);
            break;
        }
        case 4: {
            int8_t *T = take(b * c), *Q = take(a * c);
            int32_t *acc = room(4 * a * b);
            rc = oracle_ternary_matmul(T, Q, d[0], d[1], d[2], acc);
            put(&rc, 4), put(acc, 4 * a * b);
            free(T), free(Q), free(acc);
            break;
        }
        case 5: {
            int32_t *acc = take(4 * a * b);
            float *s = take(4 * a), *Y = room(4 * a * b);
            rc = oracle_scale_epilogue(acc, f, s, d[0], d[1], Y);
            put(&rc, 4), put(Y, 4 * a * b);
            free(acc), free(s), free(Y);
            break;
        }
        case 6: {
            float *W = take(4 * a * b), *sc = room(4 * a);
            int64_t *seg = c ? take(8 * c) : NULL;
            rc = oracle_absmean_rows(W, d[0], d[1], seg, d[2], sc);
            put(&rc, 4), put(sc, 4 * a);
            free(W), free(sc), free(seg);
            break;
        }
        case 7: {
            float *W = take(4 * a * b), *sc = take(4 * a);
            int8_t *T = room(a * b);
            rc = oracle_ternarize_rows(W, d[0], d[1], sc, T);
            put(&rc, 4), put(T, a * b);
            free(W), free(sc), free(T);
            break;
        }
        case 8: {
            int32_t *acc = take(4 * a * b);
            float *sc = take(4 * b), *s = take(4 * a), *Y = room(4 * a * b);
            rc = oracle_scale_epilogue_rows(acc, sc, s, d[0], d[1], Y);
            put(&rc, 4), put(Y, 4 * a * b);
            free(acc), free(sc), free(s), free(Y);
            break;
        }
        case 9: {
            float *V = take(4 * a * b), *m = room(4 * a);
            rc = oracle_absmax_rows(V, d[0], d[1], m);
            put(&rc, 4), put(m, 4 * a);
            free(V), free(m);
            break;
        }
        case 10: {
            float *V = take(4 * a * b);
            int8_t *B = room(a * b);
            rc = oracle_binarize(V, d[0], d[1], B);
            put(&rc, 4), put(B, a * b);
            free(V), free(B);
            break;
        }
        default:
            fprintf(stderr, "unknown fn %d\n", fn);
            return 3;
        }
    }
    fclose(out);
    fclose(in);
    return 0;
}
