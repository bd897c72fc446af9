/*
 * gdn_oracle.h -- plain, slow, single-threaded CPU oracle for the Gated
 * DeltaNet (GDN) gated delta-rule recurrent decode step and its front end.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this code: only the test-suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no source, header, table or helper with
 * the HIP library.
 *
 * Source: "Kestrel_VLLM #24: GDN linear attention on GPU" (wsisp.com), Fig. 1
 * caption and sections 3-4 (the beta/g, conv+SiLU and delta-recurrence
 * kernels); "Kestrel_VLLM #27: register residency and fused launch"
 * (juejin.cn), section 3.1 (same recurrence, state column in registers) and
 * section 4.2 (paired GEMV); "Kestrel_VLLM #34: batched M rows" (juejin.cn),
 * sections 3.6 (M sequential steps) and 3.7 (mark / rollback).
 *
 * Precision: the pages fix fp32 state and activations, so the fp32 oracle
 * (ref_*) works in fp32 with every multiply and add rounded separately
 * (built with -ffp-contract=off, no fast-math), in the pages' loop order.
 * ref64_* are double-precision brute-force twins for tiny shapes that use a
 * deliberately different (matrix) formulation; they exist only to pin the
 * fp32 oracle.
 *
 * Layouts (all row-major, contiguous, "unit" = one independent state, i.e.
 * one (sequence, layer) pair):
 *   S     [N][vh][kd][vd]      state, dv fastest (#24 section 4)
 *   q, k  [M][N][kh][kd]       M = 1 for a single step
 *   v, o  [M][N][vh][vd]
 *   g, beta [M][N][vh]         g is the log-domain gate, alpha = exp(g)
 *   value head i reads key head i / (vh / kh)   (#24 section 4)
 *
 * Return values: 0 on success, -1 on a bad argument (NULL pointer, a
 * non-positive size, vh not a multiple of kh, accepted[] out of range, a
 * rollback with no armed snapshot).
 */
#ifndef GDN_ORACLE_H
#define GDN_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* One decode step for every unit; S advances in place, o = S'^T q. */
int ref_gdn_step(float *S, const float *q, const float *k, const float *v,
                 const float *g, const float *beta, float *o,
                 int64_t n_units, int vh, int kh, int kd, int vd);

/* M sequential steps, row m of every input feeding step m (#34 section 3.6).
 * o is [M][N][vh][vd]. */
int ref_gdn_step_m(float *S, const float *q, const float *k, const float *v,
                   const float *g, const float *beta, float *o,
                   int64_t n_units, int M, int vh, int kh, int kd, int vd);

/* Snapshot slab of the oracle: host copies of S and the conv history plus
 * the one-shot "armed" flag (#34 section 3.7). */
typedef struct {
    float *S_snap;        /* n_units*vh*kd*vd floats, owned by the caller */
    float *hist_snap;     /* n_units*hist_floats floats or NULL */
    int64_t n_units;
    int64_t hist_floats;  /* per unit: (ck-1)*conv_dim, 0 = no history */
    int vh, kh, kd, vd;
    int armed;
} ref_slab;

/* Copy S (and hist when both hist and the slab's history area are non-NULL)
 * into the slab and arm it. */
int ref_gdn_mark(ref_slab *slab, const float *S, const float *hist);

/* Restore S (and hist) from the slab, then replay, for every unit u, the
 * first accepted[u] rows of the inputs that were given to step_m (q, k, v, g,
 * beta laid out [M][N][...]); the conv history replays the raw conv inputs
 * xc_raw [M][N][conv_dim] (needed only when hist is restored).  Disarms the
 * slab.  Returns -1 (and changes nothing) when the slab is not armed or an
 * accepted[u] lies outside 0..M. */
int ref_gdn_rollback(ref_slab *slab, float *S, float *hist,
                     const float *q, const float *k, const float *v,
                     const float *g, const float *beta,
                     const float *xc_raw, int conv_dim, int ck,
                     int M, const int32_t *accepted);

/* Push one raw conv input frame into a history [ck-1][conv_dim]:
 * frames shift one place towards the oldest slot, the newest slot gets raw. */
void ref_conv_push(float *hist, const float *raw, int conv_dim, int ck);

/* Front end for B independent rows (one layer):
 *   a = Wa x, b = Wb x                      (paired GEMV, #27 section 4.2)
 *   g = -exp(A_log) * softplus(a + dt_bias), beta = sigmoid(b)  (#24 sec. 3)
 *   conv: out = silu(sum_j w[ch][j] hist[j][ch] + w[ch][ck-1] raw[ch]),
 *         history advances by one raw frame                      (#24 sec. 3)
 *   split out into q | k | v                                     (#34 sec. 3.6)
 *   q, k: per key head x / sqrt(sum x^2 + 1e-6); q also * 1/sqrt(kd)
 * x [B][dim]; Wa, Wb [vh][dim]; A_log, dt_bias [vh]; xc_raw [B][conv_dim];
 * hist [B][ck-1][conv_dim] (in/out); conv_w [conv_dim][ck];
 * q, k [B][kh][kd]; v [B][vh][vd]; g, beta [B][vh].  conv_dim must equal
 * 2*kh*kd + vh*vd. */
int ref_gdn_frontend(const float *x, const float *Wa, const float *Wb,
                     const float *A_log, const float *dt_bias,
                     const float *xc_raw, float *hist, const float *conv_w,
                     float *q, float *k, float *v, float *g, float *beta,
                     int B, int dim, int conv_dim, int ck,
                     int vh, int kh, int kd, int vd);

/* M draft rows of the front end: M successive ref_gdn_frontend calls, row m
 * taking x [M][B][dim] and xc_raw [M][B][conv_dim] row m, the history
 * advancing once per row; outputs [M][B][...]. */
int ref_gdn_frontend_m(const float *x, const float *Wa, const float *Wb,
                       const float *A_log, const float *dt_bias,
                       const float *xc_raw, float *hist, const float *conv_w,
                       float *q, float *k, float *v, float *g, float *beta,
                       int B, int M, int dim, int conv_dim, int ck,
                       int vh, int kh, int kd, int vd);

/* Gated RMSNorm of the output, per row of vd values:
 * out = (o / sqrt(mean(o^2) + eps)) * w * silu(z).  o, z, out [rows][vd];
 * w [vd]. */
int ref_gdn_gated_norm(const float *o, const float *z, const float *w, float eps,
                       float *out, int64_t rows, int vd);

/* Dense projection of the layer (the in_proj and out_proj products):
 * y[r][o] = sum over c of W[o][c] * x[r][c], a strict left fold over
 * c = 0..C-1 with every product and sum rounded to fp32 on its own.
 * x [rows][C], W [R][C] (row-major, one output per row), y [rows][R].
 * Each row is computed on its own, so M rows in one call equal M one-row
 * calls. */
int ref_gdn_proj(const float *x, const float *W, float *y, int64_t rows, int R, int C);

/* IEEE 754 binary16 -> binary32 of n values (bit patterns in h). */
void ref_half_to_float(const uint16_t *h, float *f, int64_t n);

/* The projection with 4-bit weights: W[o][c] = n * s, n the signed
 * (two's complement) 4-bit value of element c of row o, s the binary16 scale
 * shared by the 32 elements of its block.  q [R][C/2] bytes: element 2i in
 * the low nibble of byte i, element 2i+1 in the high nibble; scale [R][C/32]
 * binary16 bit patterns.  Every W[o][c] is exact in fp32; then y is the
 * strict left fold of ref_gdn_proj.  C must be a multiple of 32. */
int ref_gdn_proj_q4(const float *x, const uint8_t *q, const uint16_t *scale, float *y,
                    int64_t rows, int R, int C);

/* Double-precision brute force of one step for tiny shapes, in the
 * re-associated matrix form S' = alpha (I - beta k k^T) S + beta k v^T,
 * o = S'^T q, built from explicit kd x kd and kd x vd matrices.  Same
 * layouts as ref_gdn_step (double instead of float).  kd, vd <= 16. */
int ref64_gdn_step(double *S, const double *q, const double *k,
                   const double *v, const double *g, const double *beta,
                   double *o, int64_t n_units, int vh, int kh, int kd, int vd);

#ifdef __cplusplus
}
#endif

#endif /* GDN_ORACLE_H */
