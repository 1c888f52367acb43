/*
 * oracle.h -- declarations of the CPU oracle (oracle.c).
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may include, load or call this.  The GPU library neither
 * includes this header nor links this code.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

typedef struct {
    int32_t D, E, K, I, bits, group;
    double eps;
    const float *router;            /* [E][D] fp32 row-major          */
    const float *gamma;             /* [D] fp32                        */
    const uint8_t *const *blobs;    /* E pointers to canonical blobs   */
    const uint8_t *shared;          /* shared expert's blob, or NULL   */
} orc_layer_args;

void orc_set_threads(int n);
int orc_get_threads(void);
uint64_t orc_blob_bytes(int D, int I, int bits, int group);
int orc_q(const uint8_t *blob, int D, int I, int bits, int mat, int row, int col);
void orc_sb(const uint8_t *blob, int D, int I, int bits, int group, int mat, int row, int col,
            double *scale, double *bias);
double orc_w(const uint8_t *blob, int D, int I, int bits, int group, int mat, int row, int col);
double orc_row_dot(const uint8_t *blob, int D, int I, int bits, int group, int mat, int row,
                   const double *x, int form);
void orc_router(const float *Wr, int E, int D, const double *x, double *logits);
int orc_topk(const double *logits, int E, int K, int32_t *sel, double *gap);
void orc_route_weights(const double *logits, const int32_t *sel, int K, double *w);
void orc_expert(const uint8_t *blob, int D, int I, int bits, int group, const double *x, double *h,
                double *y);
void orc_resnorm(const double *r, const double *c, const float *gamma, int D, double eps, double *r_out,
                 double *x_out);
int orc_layer(const orc_layer_args *a, const float *r_in, const float *x_in, const int32_t *forced_sel,
              double *logits, int32_t *sel, double *w, double *gap, double *c, double *r_out,
              double *x_out);
void orc_group(const int32_t *topk_idx, int T, int K, int E, int32_t *count, int32_t *offset,
               int32_t *perm);

#endif
