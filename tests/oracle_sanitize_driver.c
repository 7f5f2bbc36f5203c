/*
 * Runs every entry point of the fp64 oracle (oracle/oracle.c) once on small
 * inputs, for a build with AddressSanitizer and UndefinedBehaviorSanitizer.
 * Test infrastructure only: tests/test_oracle_sanitizers.py compiles this file
 * together with oracle.c and runs it; any out-of-bounds access, use of freed
 * memory or undefined operation aborts the program with a report.  Shapes are
 * ragged on purpose (rows past a tile, a partial last page, an empty sequence,
 * a chunk with no visible key).  Prints "ok" and the sum of the outputs.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_prefill(const double *, const double *, const double *, double *, double *, int, int, int, int, int,
                   int, double, int);
int oracle_prefill_ext(const double *, const double *, const double *, double *, double *, int, int, int, int,
                       int, int, double, int, double, int);
int oracle_prefill_tiled(const double *, const double *, const double *, double *, double *, int, int, int, int,
                         int, int, double, int, int);
int oracle_decode(const double *, const double *, const double *, const int32_t *, const int32_t *, double *,
                  double *, int, int, int, int, int, int, double);
int oracle_decode_ext(const double *, const double *, const double *, const int32_t *, const int32_t *, double *,
                      double *, int, int, int, int, int, int, double, int, double);
int oracle_split_decode(const double *, const double *, const double *, const int32_t *, const int32_t *,
                        double *, double *, int, int, int, int, int, int, double, int, int, double *, double *);
int oracle_lse_combine(const double *, const double *, const int32_t *, int, int, int, double *, double *);
int oracle_online_trace(const double *, const double *, int, int, double *, double *, double *, double *,
                        double *, double *);
int oracle_e4m3_decode(const uint8_t *, double *, int64_t);
int oracle_set_num_threads(int);

static uint64_t state = 0x9e3779b97f4a7c15ull;
static double rnd(void) /* splitmix64 -> uniform in [-1, 1) */
{
    uint64_t z = (state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    z ^= z >> 31;
    return (double)(z >> 11) / 4503599627370496.0 - 1.0;
}

static double *arr(size_t n) /* exactly n doubles, filled: ASan sees any overrun */
{
    double *p = malloc(n * sizeof(double));
    if (!p) exit(2);
    for (size_t i = 0; i < n; ++i) p[i] = 2.0 * rnd();
    return p;
}

static double sum(const double *p, size_t n)
{
    double s = 0;
    for (size_t i = 0; i < n; ++i)
        if (isfinite(p[i])) s += p[i];
    return s;
}

#define CHECK(x)                                                   \
    do {                                                           \
        if ((x) < 0) {                                             \
            fprintf(stderr, "%s returned an error\n", #x);        \
            return 1;                                              \
        }                                                          \
    } while (0)

int main(void)
{
    double total = 0;
    oracle_set_num_threads(2);
    /* prefill: B=2, Hq=4, Hkv=2, N=37, d=16 */
    {
        const int B = 2, Hq = 4, Hkv = 2, N = 37, d = 16;
        const size_t nq = (size_t)B * Hq * N * d, nk = (size_t)B * Hkv * N * d, nl = (size_t)B * Hq * N;
        double *q = arr(nq), *k = arr(nk), *v = arr(nk), *o = arr(nq), *l = arr(nl);
        CHECK(oracle_prefill(q, k, v, o, l, B, Hq, Hkv, N, d, 1, 0.25, 1));
        total += sum(o, nq) + sum(l, nl);
        CHECK(oracle_prefill(q, k, v, o, l, B, Hq, Hkv, N, d, 0, 0.25, 3));
        CHECK(oracle_prefill_ext(q, k, v, o, l, B, Hq, Hkv, N, d, 1, 0.25, 5, 7.5, 1));
        total += sum(o, nq) + sum(l, nl);
        CHECK(oracle_prefill_tiled(q, k, v, o, l, B, Hq, Hkv, N, d, 1, 0.25, 5, 7));
        CHECK(oracle_prefill_tiled(q, k, v, o, l, B, Hq, Hkv, N, d, 0, 0.25, 64, 3));
        total += sum(o, nq) + sum(l, nl);
        free(q); free(k); free(v); free(o); free(l);
    }
    /* paged decode: B=3 (lengths 45, 0, 16), Hq=4, Hkv=2, d=8, pages of 16, 4 slots per row */
    {
        const int B = 3, Hq = 4, Hkv = 2, d = 8, P = 16, MB = 4, NB = 6;
        int32_t lens[3] = {45, 0, 16};
        int32_t bt[12] = {5, 0, 3, -1, -1, -1, -1, -1, 2, -1, -1, -1};
        const size_t nq = (size_t)B * Hq * d, nc = (size_t)NB * P * Hkv * d, nl = (size_t)B * Hq;
        double *q = arr(nq), *kc = arr(nc), *vc = arr(nc), *o = arr(nq), *l = arr(nl);
        CHECK(oracle_decode(q, kc, vc, bt, lens, o, l, B, Hq, Hkv, d, P, MB, 0.3));
        total += sum(o, nq) + sum(l, nl);
        CHECK(oracle_decode_ext(q, kc, vc, bt, lens, o, l, B, Hq, Hkv, d, P, MB, 0.3, 9, 5.0));
        total += sum(o, nq) + sum(l, nl);
        const int chunk = 32, max_chunks = (MB * P + chunk - 1) / chunk;
        double *op = arr((size_t)B * Hq * max_chunks * d), *lp = arr((size_t)B * Hq * max_chunks);
        CHECK(oracle_split_decode(q, kc, vc, bt, lens, o, l, B, Hq, Hkv, d, P, MB, 0.3, chunk, 8, op, lp));
        total += sum(o, nq) + sum(l, nl);
        CHECK(oracle_lse_combine(op, lp, NULL, B * Hq, max_chunks, d, o, l));
        total += sum(o, nq) + sum(l, nl);
        free(op); free(lp);
        /* contiguous cache: [B][S][Hkv][d] with S = MB * P */
        double *kk = arr((size_t)B * MB * P * Hkv * d), *vv = arr((size_t)B * MB * P * Hkv * d);
        CHECK(oracle_decode(q, kk, vv, NULL, lens, o, l, B, Hq, Hkv, d, P, MB, 0.3));
        total += sum(o, nq) + sum(l, nl);
        free(kk); free(vv);
        free(q); free(kc); free(vc); free(o); free(l);
    }
    /* the worked example's online trace with blocks of 2, and a ragged block */
    {
        double s[5] = {2, 1, 4, 3, 0.5}, v[5] = {1, 0, 2, -1, 3};
        double m[3], l[3], ot[3], c[3], o, lse;
        CHECK(oracle_online_trace(s, v, 4, 2, m, l, ot, c, &o, &lse));
        total += o + lse;
        CHECK(oracle_online_trace(s, v, 5, 2, m, l, ot, c, &o, &lse));
        total += o + lse;
    }
    /* every E4M3 code */
    {
        uint8_t codes[256];
        double out[256];
        for (int i = 0; i < 256; ++i) codes[i] = (uint8_t)i;
        CHECK(oracle_e4m3_decode(codes, out, 256));
        total += sum(out, 256);
    }
    printf("ok %.6f\n", total);
    return 0;
}
