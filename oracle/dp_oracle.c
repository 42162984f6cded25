/*
 * CPU oracle for one rank's share of a displaced-patch (DistriFusion-style)
 * diffusion step.  TEST INFRASTRUCTURE ONLY: it is linked by the tests, by the
 * smoke check and by the benchmark's CPU-baseline leg, never by the product
 * path.  It shares no code, header or constant with the HIP library.
 *
 * Every routine is the plain definition of what the method computes, in
 * float64, with straightforward loops and no blocking, fusion or reordering.
 * Inputs arrive widened to float64 (exact for float32 and bfloat16 storage).
 * The outermost independent index is spread over OpenMP threads; each output
 * element is still produced by one sequential loop.
 *
 * Sources (the web pages this build works from):
 *  - DistriFusion project summary, "How It Works": the image is partitioned
 *    across devices and later steps reuse activations from the previous step.
 *  - "OTIL for SDXL on 4x L40S", "What is implemented where": the three
 *    displaced layer kinds (self-attention, 3x3 conv, GroupNorm) and the two
 *    scalars per group that GroupNorm combines across slices.
 *  - same page, "Read this before interpreting the numbers", item 3: the stale
 *    state is the attention K/V buffers and the conv halo buffers.
 *  - "Tensor Parallelism with Stale Activations ..." (xDiT issue thread),
 *    maintainer's replies: stale K/V buffers have the full spatial shape, and a
 *    feature may mix fresh (local) and stale (remote) partial values.
 *  - "Benchmarking DistVAE", "Glossary": a halo is the neighbouring rows a
 *    sharded convolution needs; patchify splits into rank-local row bands.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define EXPORT __attribute__((visibility("default")))

/* Row band of rank r when H rows are split over N ranks (DistVAE "Glossary",
 * patchify into row bands): [floor(r*H/N), floor((r+1)*H/N)). */
EXPORT void dpo_partition_rows(int64_t H, int64_t N, int64_t r, int64_t* row0, int64_t* row1) {
    *row0 = (r * H) / N;
    *row1 = ((r + 1) * H) / N;
}

/* Dense projection y[m,o] = sum_c x[m,c] * w[o,c] (+ bias[o]).
 * x [M,Cin], w [Cout,Cin], bias [Cout] or NULL, y [M,Cout].
 * The Q/K/V/output projections of the displaced self-attention layer
 * ("OTIL ...", "What is implemented where") are this map applied to the
 * rank's own rows only. */
EXPORT void dpo_linear(const double* x, const double* w, const double* bias, double* y,
                       int64_t M, int64_t Cin, int64_t Cout) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t o = 0; o < Cout; ++o) {
            double acc = bias ? bias[o] : 0.0;
            for (int64_t c = 0; c < Cin; ++c) acc += x[m * Cin + c] * w[o * Cin + c];
            y[m * Cout + o] = acc;
        }
    }
}

/* Softmax attention of the local queries over every key of the full-image
 * buffer, no mask:  o = sum_j p_j v_j / sum_j p_j,  p_j = exp(s_j - max s),
 * s_j = scale * <q, k_j>.  Head h uses channels [h*d, (h+1)*d).
 * q [B,Tq,H*d], k,v [B,Tkv,H*d] (the spliced buffers), o [B,Tq,H*d].
 * The full-spatial K/V buffer is the one the xDiT issue thread describes; the
 * local rows in it are fresh and the others stale (issue thread, partial stale
 * values). */
EXPORT void dpo_attention(const double* q, const double* k, const double* v, double* o,
                          int64_t B, int64_t H, int64_t Tq, int64_t Tkv, int64_t d,
                          double scale) {
    const int64_t C = H * d;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(Tkv > 0 ? Tkv : 1));
#pragma omp for schedule(static) collapse(3)
        for (int64_t b = 0; b < B; ++b)
            for (int64_t h = 0; h < H; ++h)
                for (int64_t i = 0; i < Tq; ++i) {
                    const double* qi = q + (b * Tq + i) * C + h * d;
                    double mx = -INFINITY;
                    for (int64_t j = 0; j < Tkv; ++j) {
                        const double* kj = k + (b * Tkv + j) * C + h * d;
                        double dot = 0.0;
                        for (int64_t e = 0; e < d; ++e) dot += qi[e] * kj[e];
                        s[j] = scale * dot;
                        if (s[j] > mx) mx = s[j];
                    }
                    double Z = 0.0;
                    for (int64_t j = 0; j < Tkv; ++j) {
                        s[j] = exp(s[j] - mx);
                        Z += s[j];
                    }
                    double* oi = o + (b * Tq + i) * C + h * d;
                    for (int64_t e = 0; e < d; ++e) {
                        double acc = 0.0;
                        for (int64_t j = 0; j < Tkv; ++j) acc += s[j] * v[(b * Tkv + j) * C + h * d + e];
                        oi[e] = acc / Z;
                    }
                }
        free(s);
    }
}

/* Source pixel of the 3x3 window: row -1 is the stale row above the band
 * (halo_top), row h the stale row below (halo_bot), a NULL halo and any
 * column outside [0,W) read as zero (DistVAE "Glossary": halo). */
static double conv_src(const double* x, const double* halo_top, const double* halo_bot,
                       int64_t b, int64_t row, int64_t col, int64_t c,
                       int64_t h, int64_t W, int64_t Cin) {
    if (col < 0 || col >= W) return 0.0;
    if (row < 0) return halo_top ? halo_top[(b * W + col) * Cin + c] : 0.0;
    if (row >= h) return halo_bot ? halo_bot[(b * W + col) * Cin + c] : 0.0;
    return x[((b * h + row) * W + col) * Cin + c];
}

/* 3x3, stride 1, pad 1 cross-correlation over the rank's rows with stale halo
 * rows ("OTIL ...", "What is implemented where": the displaced conv;
 * "Read this ...", item 3: conv halo buffers):
 *   y[b,i,x,o] = bias[o] + sum_{dy,dx in {-1,0,1}} sum_c w[o,dy+1,dx+1,c] * src(b,i+dy,x+dx,c).
 * x [B,h,W,Cin], halos [B,W,Cin] or NULL, w [Cout,3,3,Cin], bias [Cout] or
 * NULL, y [B,h,W,Cout]. */
EXPORT void dpo_conv3x3_halo(const double* x, const double* halo_top, const double* halo_bot,
                             const double* w, const double* bias, double* y,
                             int64_t B, int64_t h, int64_t W, int64_t Cin, int64_t Cout) {
#pragma omp parallel for schedule(static) collapse(3)
    for (int64_t b = 0; b < B; ++b)
        for (int64_t i = 0; i < h; ++i)
            for (int64_t xc = 0; xc < W; ++xc)
                for (int64_t o = 0; o < Cout; ++o) {
                    double acc = bias ? bias[o] : 0.0;
                    for (int64_t dy = -1; dy <= 1; ++dy)
                        for (int64_t dx = -1; dx <= 1; ++dx) {
                            const double* wt = w + ((o * 3 + (dy + 1)) * 3 + (dx + 1)) * Cin;
                            for (int64_t c = 0; c < Cin; ++c)
                                acc += wt[c] * conv_src(x, halo_top, halo_bot, b, i + dy, xc + dx,
                                                        c, h, W, Cin);
                        }
                    y[((b * h + i) * W + xc) * Cout + o] = acc;
                }
}

/* The two scalars per group ("OTIL ...", "What is implemented where", GroupNorm
 * sync): sums[b,g,0] = sum of x, sums[b,g,1] = sum of x^2, over every token of
 * x and the group's contiguous channels [g*C/G, (g+1)*C/G).
 * x [B,T,C], sums [B,G,2]. */
EXPORT void dpo_group_sums(const double* x, int64_t B, int64_t T, int64_t C, int64_t G,
                           double* sums) {
    const int64_t Cg = C / G;
#pragma omp parallel for schedule(static) collapse(2)
    for (int64_t b = 0; b < B; ++b)
        for (int64_t g = 0; g < G; ++g) {
            double s1 = 0.0, s2 = 0.0;
            for (int64_t t = 0; t < T; ++t)
                for (int64_t c = g * Cg; c < (g + 1) * Cg; ++c) {
                    double v = x[(b * T + t) * C + c];
                    s1 += v;
                    s2 += v * v;
                }
            sums[(b * G + g) * 2 + 0] = s1;
            sums[(b * G + g) * 2 + 1] = s2;
        }
}

/* GroupNorm over the full image from fresh local sums plus the stale sums of
 * the other patches (xDiT issue thread: partial stale values; "OTIL ...",
 * "What is implemented where": the per-group scalars decide slice brightness
 * and contrast):
 *   S = local sums + sum_{p != rank} stale[p,b,g,:];  n = T_total * C/G;
 *   mean = S1/n;  var = max(S2/n - mean^2, 0);
 *   y = (x - mean) / sqrt(var + eps) * gamma[c] + beta[c],  then y*sigmoid(y) if silu.
 * x [B,T,C]; stale [N,B,G,2] (entry [rank] never read); gamma/beta [C] or NULL
 * (=1/0); y [B,T,C]; fresh [B,G,2] receives the local sums (may be NULL). */
EXPORT void dpo_groupnorm_stale(const double* x, const double* stale, int64_t n_patches,
                                int64_t rank, int64_t T_total, const double* gamma,
                                const double* beta, double eps, int silu, double* y,
                                double* fresh, int64_t B, int64_t T, int64_t C, int64_t G) {
    const int64_t Cg = C / G;
    double* loc = (double*)malloc(sizeof(double) * (size_t)(B * G * 2));
    dpo_group_sums(x, B, T, C, G, loc);
#pragma omp parallel for schedule(static) collapse(2)
    for (int64_t b = 0; b < B; ++b)
        for (int64_t g = 0; g < G; ++g) {
            double s1 = loc[(b * G + g) * 2 + 0];
            double s2 = loc[(b * G + g) * 2 + 1];
            for (int64_t p = 0; p < n_patches; ++p) {
                if (p == rank) continue;
                s1 += stale[((p * B + b) * G + g) * 2 + 0];
                s2 += stale[((p * B + b) * G + g) * 2 + 1];
            }
            const double n = (double)T_total * (double)Cg;
            const double mean = s1 / n;
            double var = s2 / n - mean * mean;
            if (var < 0.0) var = 0.0;
            const double inv = 1.0 / sqrt(var + eps);
            for (int64_t t = 0; t < T; ++t)
                for (int64_t c = g * Cg; c < (g + 1) * Cg; ++c) {
                    const int64_t idx = (b * T + t) * C + c;
                    double v = (x[idx] - mean) * inv;
                    v = v * (gamma ? gamma[c] : 1.0) + (beta ? beta[c] : 0.0);
                    if (silu) v = v / (1.0 + exp(-v));
                    y[idx] = v;
                }
        }
    if (fresh) memcpy(fresh, loc, sizeof(double) * (size_t)(B * G * 2));
    free(loc);
}
