/*
 * Driver for the address- and undefined-behaviour-sanitised build of the C
 * oracle (TEST INFRASTRUCTURE ONLY, built and run by the CPU tests).  Every
 * exported routine runs on small shapes with buffers malloc'ed at exactly the
 * size its contract states, so any read or write past a stated extent stops
 * the run; the optional arguments are exercised both given and NULL.  A few
 * closed-form checks make sure the calls really computed something.
 * Exit status 0 on success, 1 on a failed check.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void dpo_partition_rows(int64_t H, int64_t N, int64_t r, int64_t* row0, int64_t* row1);
void dpo_linear(const double* x, const double* w, const double* bias, double* y, int64_t M, int64_t Cin,
                int64_t Cout);
void dpo_attention(const double* q, const double* k, const double* v, double* o, int64_t B, int64_t H,
                   int64_t Tq, int64_t Tkv, int64_t d, double scale);
void dpo_conv3x3_halo(const double* x, const double* halo_top, const double* halo_bot, const double* w,
                      const double* bias, double* y, int64_t B, int64_t h, int64_t W, int64_t Cin, int64_t Cout);
void dpo_group_sums(const double* x, int64_t B, int64_t T, int64_t C, int64_t G, double* sums);
void dpo_groupnorm_stale(const double* x, const double* stale, int64_t n_patches, int64_t rank, int64_t T_total,
                         const double* gamma, const double* beta, double eps, int silu, double* y, double* fresh,
                         int64_t B, int64_t T, int64_t C, int64_t G);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static double uniform(void) { /* xorshift64*, in [-1, 1) */
    g_state ^= g_state >> 12;
    g_state ^= g_state << 25;
    g_state ^= g_state >> 27;
    return (double)((g_state * 0x2545F4914F6CDD1Dull) >> 11) / 4503599627370496.0 - 1.0;
}
static double* filled(size_t n) {
    double* p = (double*)malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) p[i] = uniform();
    return p;
}
static int g_fail = 0;
static void expect(int ok, const char* what) {
    if (!ok) {
        fprintf(stderr, "check failed: %s\n", what);
        g_fail = 1;
    }
}

int main(void) {
    /* row bands cover [0, H) without gaps */
    int64_t prev = 0;
    for (int64_t r = 0; r < 3; ++r) {
        int64_t a, b;
        dpo_partition_rows(10, 3, r, &a, &b);
        expect(a == prev && b >= a, "partition contiguous");
        prev = b;
    }
    expect(prev == 10, "partition covers H");

    /* linear, with and without bias */
    {
        const int64_t M = 3, Cin = 5, Cout = 7;
        double *x = filled(M * Cin), *w = filled(Cout * Cin), *bias = filled(Cout);
        double *y = malloc(M * Cout * sizeof(double)), *y0 = malloc(M * Cout * sizeof(double));
        dpo_linear(x, w, bias, y, M, Cin, Cout);
        dpo_linear(x, w, NULL, y0, M, Cin, Cout);
        for (int64_t i = 0; i < M * Cout; ++i) expect(fabs(y[i] - y0[i] - bias[i % Cout]) < 1e-12, "linear bias");
        free(x), free(w), free(bias), free(y), free(y0);
    }

    /* attention: one key gives its value exactly; odd sizes otherwise */
    {
        const int64_t B = 2, H = 3, Tq = 5, d = 4, C = H * d;
        for (int64_t Tkv = 1; Tkv <= 7; Tkv += 6) {
            double *q = filled(B * Tq * C), *k = filled(B * Tkv * C), *v = filled(B * Tkv * C);
            double* o = malloc(B * Tq * C * sizeof(double));
            dpo_attention(q, k, v, o, B, H, Tq, Tkv, d, 0.5);
            if (Tkv == 1)
                for (int64_t b = 0; b < B; ++b)
                    for (int64_t t = 0; t < Tq; ++t)
                        for (int64_t c = 0; c < C; ++c)
                            expect(fabs(o[(b * Tq + t) * C + c] - v[b * C + c]) < 1e-12, "attention one key");
            free(q), free(k), free(v), free(o);
        }
    }

    /* conv: halos given and NULL, bias given and NULL; a centre-only identity
     * kernel returns its input */
    {
        const int64_t B = 2, h = 3, W = 4, Cin = 3, Cout = 5;
        double *x = filled(B * h * W * Cin), *ht = filled(B * W * Cin), *hb = filled(B * W * Cin);
        double *w = filled(Cout * 9 * Cin), *bias = filled(Cout), *y = malloc(B * h * W * Cout * sizeof(double));
        dpo_conv3x3_halo(x, ht, hb, w, bias, y, B, h, W, Cin, Cout);
        dpo_conv3x3_halo(x, NULL, NULL, w, NULL, y, B, h, W, Cin, Cout);
        dpo_conv3x3_halo(x, ht, NULL, w, bias, y, B, h, W, Cin, Cout);
        double* id = calloc(Cin * 9 * Cin, sizeof(double));
        double* yi = malloc(B * h * W * Cin * sizeof(double));
        for (int64_t o = 0; o < Cin; ++o) id[(o * 9 + 4) * Cin + o] = 1.0;
        dpo_conv3x3_halo(x, ht, hb, id, NULL, yi, B, h, W, Cin, Cin);
        for (int64_t i = 0; i < B * h * W * Cin; ++i) expect(yi[i] == x[i], "conv identity");
        free(x), free(ht), free(hb), free(w), free(bias), free(y), free(id), free(yi);
    }

    /* group sums and the stale GroupNorm: several patches, and a single patch
     * with NULL stale sums, gamma and beta (then every group has mean 0) */
    {
        const int64_t B = 2, T = 5, C = 6, G = 3, N = 3;
        double *x = filled(B * T * C), *sums = malloc(B * G * 2 * sizeof(double));
        dpo_group_sums(x, B, T, C, G, sums);
        double s = 0.0;
        for (int64_t t = 0; t < T; ++t)
            for (int64_t c = 0; c < 2; ++c) s += x[t * C + c];
        expect(fabs(sums[0] - s) < 1e-12, "group sum");
        double *stale = filled(N * B * G * 2), *gamma = filled(C), *beta = filled(C);
        for (int64_t i = 0; i < N * B * G; ++i) stale[2 * i + 1] = 10.0 + fabs(stale[2 * i + 1]);
        double *y = malloc(B * T * C * sizeof(double)), *fresh = malloc(B * G * 2 * sizeof(double));
        dpo_groupnorm_stale(x, stale, N, 1, N * T, gamma, beta, 1e-5, 1, y, fresh, B, T, C, G);
        for (int64_t i = 0; i < B * G * 2; ++i) expect(fresh[i] == sums[i], "fresh sums");
        dpo_groupnorm_stale(x, NULL, 1, 0, T, NULL, NULL, 1e-5, 0, y, NULL, B, T, C, G);
        for (int64_t b = 0; b < B; ++b)
            for (int64_t g = 0; g < G; ++g) {
                double m = 0.0;
                for (int64_t t = 0; t < T; ++t)
                    for (int64_t c = 2 * g; c < 2 * g + 2; ++c) m += y[(b * T + t) * C + c];
                expect(fabs(m) < 1e-9, "normalised group mean");
            }
        free(x), free(sums), free(stale), free(gamma), free(beta), free(y), free(fresh);
    }
    if (!g_fail) printf("asan driver: all oracle routines ran clean\n");
    return g_fail;
}
