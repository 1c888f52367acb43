/*
 * oracle.c -- plain, slow CPU definition of the per-token sparse MoE block.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load or call this library.  It shares no code, header,
 * table or helper with the GPU library; both read the same canonical expert
 * blobs and the same seeded inputs, nothing else.
 *
 * Every quantity is accumulated in fp64 from the exact fp32 / bf16 input
 * values, in plain index order, with no blocking or reordering beyond what
 * the definitions below state.  Sources (the pages describing the Flash-MoE
 * "streaming experts" engine):
 *   - toolarium.ru, "Mixture of Experts и почему SSD достаточно": the router
 *     picks 4 of 512 experts per token per layer.
 *   - hakusoku.com, "モデルアーキテクチャ": K=4 active experts per token plus
 *     a shared expert, hidden size 4096.
 *   - hakusoku.com, "パイプライン概要": softmax / top-K routing step.
 *   - toolarium.ru, "Оптимизации, которые сработали": the dequantised weight
 *     is nibble*scale + bias; the FMA rewrite fma(nibble, scale*x, bias*x);
 *     combine + residual + normalisation fused.
 *   - hakusoku.com, "主要技術": 4/2-bit dequant matvec, SwiGLU, RMS norm and
 *     MoE combine kernels; combine and norm hand their result to the next
 *     layer.
 * Readings where the pages are silent (layout, group size, tie order,
 * shared-expert weight, eps placement) are listed in the design notes and
 * restated at each function below.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#include "oracle.h"

void orc_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int orc_get_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------------------
 * Canonical expert blob (one contiguous byte range per expert):
 *   [gate.q | up.q | down.q | gate.sb | up.sb | down.sb]
 * gate and up are [I rows][D cols]; down is [D rows][I cols]; all row-major.
 * q: element (row, col) of a matrix with `cols` columns sits at bit offset
 *    (row*cols + col)*bits of that matrix's q region, read as little-endian
 *    32-bit words, lowest bits first; value in [0, 2^bits).
 * sb: one 32-bit word per group of `group` consecutive columns of a row,
 *    word index row*(cols/group) + col/group; low 16 bits = bf16 scale,
 *    high 16 bits = bf16 bias.
 * Size: the pages give about 6.75 MB per expert (toolarium.ru, "Flash-MoE:
 * чистый C, Metal и никакого Python"); D=4096, I=1024, 4-bit, group 64 with a
 * 16-bit scale and a 16-bit bias gives 7,077,888 B = 6.75 MiB.
 * ------------------------------------------------------------------------- */
uint64_t orc_blob_bytes(int D, int I, int bits, int group)
{
    uint64_t elems = (uint64_t)D * (uint64_t)I;          /* per matrix */
    uint64_t q_bytes = 3 * elems * (uint64_t)bits / 8;   /* three matrices */
    uint64_t sb_bytes = 3 * (elems / (uint64_t)group) * 4;
    return q_bytes + sb_bytes;
}

static double bf16_to_double(uint32_t h16)
{
    uint32_t u = h16 << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static uint32_t read_u32(const uint8_t *p)
{
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}

/* Rows and columns of matrix `mat` (0 gate, 1 up, 2 down). */
static void mat_dims(int D, int I, int mat, int *rows, int *cols)
{
    if (mat == 2) { *rows = D; *cols = I; }
    else { *rows = I; *cols = D; }
}

/* Quantised code q(row, col) of matrix `mat`. */
int orc_q(const uint8_t *blob, int D, int I, int bits, int mat, int row, int col)
{
    int rows, cols;
    mat_dims(D, I, mat, &rows, &cols);
    uint64_t region = (uint64_t)mat * ((uint64_t)D * (uint64_t)I * (uint64_t)bits / 8);
    uint64_t bit = ((uint64_t)row * (uint64_t)cols + (uint64_t)col) * (uint64_t)bits;
    uint32_t word = read_u32(blob + region + (bit / 32) * 4);
    return (int)((word >> (bit % 32)) & ((1u << bits) - 1u));
}

/* Scale and bias of the group holding (row, col) of matrix `mat`. */
void orc_sb(const uint8_t *blob, int D, int I, int bits, int group, int mat, int row, int col,
            double *scale, double *bias)
{
    int rows, cols;
    mat_dims(D, I, mat, &rows, &cols);
    uint64_t elems = (uint64_t)D * (uint64_t)I;
    uint64_t sb0 = 3 * elems * (uint64_t)bits / 8 + (uint64_t)mat * (elems / (uint64_t)group) * 4;
    uint64_t g = (uint64_t)row * (uint64_t)(cols / group) + (uint64_t)(col / group);
    uint32_t word = read_u32(blob + sb0 + g * 4);
    *scale = bf16_to_double(word & 0xFFFFu);
    *bias = bf16_to_double(word >> 16);
}

/* Dequantised weight: unsigned affine, w = q*scale + bias (toolarium.ru,
 * "Оптимизации, которые сработали": nibble x scale + bias).  Exact in fp64:
 * q has at most 4 bits and scale/bias are bf16. */
double orc_w(const uint8_t *blob, int D, int I, int bits, int group, int mat, int row, int col)
{
    double s, b;
    orc_sb(blob, D, I, bits, group, mat, row, col, &s, &b);
    return (double)orc_q(blob, D, I, bits, mat, row, col) * s + b;
}

/* One row of a dequantised matrix times x, in one of three algebraically
 * equal forms (the FMA rewrite on toolarium.ru, "Оптимизации, которые
 * сработали"):
 *   form 0: sum_j (q*s + b) * x_j                 (the basic kernel)
 *   form 1: sum_j fma(q, s*x_j, b*x_j)            (the FMA kernel)
 *   form 2: sum_groups s * sum_j q*x_j + b * sum_j x_j
 * Terms are added in ascending column order. */
double orc_row_dot(const uint8_t *blob, int D, int I, int bits, int group, int mat, int row,
                   const double *x, int form)
{
    int rows, cols;
    mat_dims(D, I, mat, &rows, &cols);
    double acc = 0.0;
    if (form == 2) {
        for (int g0 = 0; g0 < cols; g0 += group) {
            double s, b, qx = 0.0, xs = 0.0;
            orc_sb(blob, D, I, bits, group, mat, row, g0, &s, &b);
            for (int j = g0; j < g0 + group; ++j) {
                qx += (double)orc_q(blob, D, I, bits, mat, row, j) * x[j];
                xs += x[j];
            }
            acc += s * qx + b * xs;
        }
        return acc;
    }
    for (int j = 0; j < cols; ++j) {
        double s, b;
        orc_sb(blob, D, I, bits, group, mat, row, j, &s, &b);
        double q = (double)orc_q(blob, D, I, bits, mat, row, j);
        if (form == 1) acc += fma(q, s * x[j], b * x[j]);
        else acc += (q * s + b) * x[j];
    }
    return acc;
}

/* Router projection: logits[e] = sum_d Wr[e][d] * x[d], Wr fp32 row-major
 * [E][D] (toolarium.ru: the router chooses 4 of 512 experts; the projection
 * runs with the shared expert in one GPU command, hakusoku.com,
 * "パイプライン概要"). */
void orc_router(const float *Wr, int E, int D, const double *x, double *logits)
{
#pragma omp parallel for schedule(static)
    for (int e = 0; e < E; ++e) {
        double acc = 0.0;
        for (int d = 0; d < D; ++d) acc += (double)Wr[(size_t)e * (size_t)D + (size_t)d] * x[d];
        logits[e] = acc;
    }
}

/* Top-K selection in rank order: repeatedly take the largest remaining logit,
 * the lower index winning an exact tie.  gap = (K-th selected logit) -
 * (largest unselected logit), +inf when K == E.  Returns 0, or -1 on bad K. */
int orc_topk(const double *logits, int E, int K, int32_t *sel, double *gap)
{
    if (K < 1 || K > E) return -1;
    unsigned char taken[4096];
    if (E > 4096) return -1;
    memset(taken, 0, (size_t)E);
    for (int k = 0; k < K; ++k) {
        int best = -1;
        for (int e = 0; e < E; ++e)
            if (!taken[e] && (best < 0 || logits[e] > logits[best])) best = e;
        taken[best] = 1;
        sel[k] = best;
    }
    double next = -INFINITY;
    for (int e = 0; e < E; ++e)
        if (!taken[e] && logits[e] > next) next = logits[e];
    *gap = (K < E) ? logits[sel[K - 1]] - next : INFINITY;
    return 0;
}

/* Routing weights: softmax over all E logits, then renormalised over the K
 * selected ones (hakusoku.com, "パイプライン概要": softmax/topK).  The
 * normaliser over all E cancels, so w_k = exp(l_k - m) / sum_j exp(l_j - m)
 * over the selected j, m = the largest selected logit. */
void orc_route_weights(const double *logits, const int32_t *sel, int K, double *w)
{
    double m = logits[sel[0]];
    for (int k = 1; k < K; ++k)
        if (logits[sel[k]] > m) m = logits[sel[k]];
    double z = 0.0;
    for (int k = 0; k < K; ++k) z += exp(logits[sel[k]] - m);
    for (int k = 0; k < K; ++k) w[k] = exp(logits[sel[k]] - m) / z;
}

/* One expert FFN with SwiGLU (hakusoku.com, "主要技術"):
 *   g_i = sum_j Wg[i][j] x_j,  u_i = sum_j Wu[i][j] x_j,
 *   h_i = silu(g_i) * u_i = g_i / (1 + exp(-g_i)) * u_i,
 *   y_o = sum_i Wd[o][i] h_i.
 * h (length I) may be NULL. */
void orc_expert(const uint8_t *blob, int D, int I, int bits, int group, const double *x, double *h,
                double *y)
{
    double *hh = h;
    double hbuf[16384];
    if (!hh) hh = hbuf; /* I <= 16384 checked by the caller */
#pragma omp parallel for schedule(static)
    for (int i = 0; i < I; ++i) {
        double g = 0.0, u = 0.0;
        for (int j = 0; j < D; ++j) {
            g += orc_w(blob, D, I, bits, group, 0, i, j) * x[j];
            u += orc_w(blob, D, I, bits, group, 1, i, j) * x[j];
        }
        hh[i] = g / (1.0 + exp(-g)) * u;
    }
#pragma omp parallel for schedule(static)
    for (int o = 0; o < D; ++o) {
        double acc = 0.0;
        for (int i = 0; i < I; ++i) acc += orc_w(blob, D, I, bits, group, 2, o, i) * hh[i];
        y[o] = acc;
    }
}

/* Residual add and RMSNorm (toolarium.ru: combine + residual + normalisation
 * in one kernel): r' = r + c; x' = r' / sqrt(mean(r'^2) + eps) * gamma. */
void orc_resnorm(const double *r, const double *c, const float *gamma, int D, double eps, double *r_out,
                 double *x_out)
{
    double ss = 0.0;
    for (int o = 0; o < D; ++o) {
        r_out[o] = r[o] + c[o];
        ss += r_out[o] * r_out[o];
    }
    double inv = 1.0 / sqrt(ss / (double)D + eps);
    for (int o = 0; o < D; ++o) x_out[o] = r_out[o] * inv * (double)gamma[o];
}

/* One MoE layer for one token.
 *   1. logits = router(x)                                      (fp64)
 *   2. sel = top-K(logits) unless forced_sel is given; gap recorded
 *   3. w = softmax over the selected logits
 *   4. y_e = expert_e(x) for e in sel, and y_s = shared(x) when present
 *   5. c = sum_k w_k y_sel[k] + y_s   (shared expert added with weight 1)
 *   6. r' = r + c; x' = RMSNorm(r') * gamma
 * Inputs r, x are fp32 [D]; blobs[e] points at expert e's canonical blob;
 * shared is NULL when there is no shared expert.  Outputs are fp64.
 * Returns 0, or -1 on a bad argument. */
int orc_layer(const orc_layer_args *a, const float *r_in, const float *x_in, const int32_t *forced_sel,
              double *logits, int32_t *sel, double *w, double *gap, double *c, double *r_out,
              double *x_out)
{
    const int D = a->D, E = a->E, K = a->K, I = a->I;
    if (D <= 0 || D > 16384 || I <= 0 || I > 16384 || E <= 0 || E > 4096 || K < 1 || K > E) return -1;
    if (a->bits != 2 && a->bits != 4) return -1;
    if (a->group <= 0 || D % a->group || I % a->group) return -1;
    double x[16384], r[16384], y[16384];
    for (int d = 0; d < D; ++d) { x[d] = (double)x_in[d]; r[d] = (double)r_in[d]; }

    orc_router(a->router, E, D, x, logits);
    if (forced_sel) {
        for (int k = 0; k < K; ++k) {
            if (forced_sel[k] < 0 || forced_sel[k] >= E) return -1;
            sel[k] = forced_sel[k];
        }
        *gap = NAN;
    } else if (orc_topk(logits, E, K, sel, gap)) {
        return -1;
    }
    orc_route_weights(logits, sel, K, w);

    for (int o = 0; o < D; ++o) c[o] = 0.0;
    for (int k = 0; k < K; ++k) {
        orc_expert(a->blobs[sel[k]], D, I, a->bits, a->group, x, NULL, y);
        for (int o = 0; o < D; ++o) c[o] += w[k] * y[o];
    }
    if (a->shared) {
        orc_expert(a->shared, D, I, a->bits, a->group, x, NULL, y);
        for (int o = 0; o < D; ++o) c[o] += y[o];
    }
    orc_resnorm(r, c, a->gamma, D, a->eps, r_out, x_out);
    return 0;
}

/* Token -> expert grouping for a batch (integer): count[e] = number of
 * (token, slot) pairs routed to e; offset = exclusive prefix sum of count
 * (E+1 entries); perm lists the pair indices p = t*K + k grouped by expert
 * in ascending e, ascending p inside a group. */
void orc_group(const int32_t *topk_idx, int T, int K, int E, int32_t *count, int32_t *offset, int32_t *perm)
{
    int pos = 0;
    offset[0] = 0;
    for (int e = 0; e < E; ++e) {
        int n = 0;
        for (int p = 0; p < T * K; ++p)
            if (topk_idx[p] == e) { perm[pos++] = p; ++n; }
        count[e] = n;
        offset[e + 1] = offset[e] + n;
    }
}
