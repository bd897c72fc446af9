/*
 * gdn_oracle.c -- plain CPU oracle for the GDN recurrent decode step.
 *
 * TEST INFRASTRUCTURE ONLY (see gdn_oracle.h).  Build with
 *   gcc -std=c99 -O2 -ffp-contract=off -fno-fast-math
 * so that every fp32 multiply and add is rounded on its own and no reduction
 * is re-associated (the compiler may still process independent columns side
 * by side, which changes no rounding).  The passes follow the order in which
 * the operator is stated: decay, key read-out, delta, rank-1 update, query
 * read-out with the updated state.
 */
#include "gdn_oracle.h"

#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

static int dims_ok(int64_t n, int vh, int kh, int kd, int vd)
{
    return n >= 0 && vh > 0 && kh > 0 && kd > 0 && vd > 0 && vh % kh == 0;
}

/*
 * The operator on one (unit, value head) tile, stated as whole-tile passes
 * ("Kestrel_VLLM #24", Fig. 1 caption, step 5: alpha scale, then S.k, then
 * (v - .) beta, then the rank-1 add, then S.q on the updated state; section 4
 * fixes the tile layout st[r][c], r over kd, c over vd):
 *   1. st      <- decay * st                       (every element)
 *   2. kread   <- st^T kvec                        (decayed tile)
 *   3. delta   <- (vvec - kread) * b
 *   4. st      <- st + kvec delta^T                (rank-1 update)
 *   5. out     <- st^T qvec                        (updated tile)
 * Each read-out element is a strict left fold over r = 0..kd-1, and every
 * multiply and add is rounded to fp32 on its own.  out may be NULL (no
 * read-out wanted).
 */
static void tile_update(float *st, const float *qvec, const float *kvec,
                        const float *vvec, float decay, float b, float *out,
                        int kd, int vd)
{
    float kread[vd], delta[vd];

    for (int r = 0; r < kd; r++)
        for (int c = 0; c < vd; c++)
            st[(size_t)r * vd + c] = st[(size_t)r * vd + c] * decay;

    for (int c = 0; c < vd; c++)
        kread[c] = 0.0f;
    for (int r = 0; r < kd; r++)
        for (int c = 0; c < vd; c++)
            kread[c] = kread[c] + st[(size_t)r * vd + c] * kvec[r];

    for (int c = 0; c < vd; c++)
        delta[c] = (vvec[c] - kread[c]) * b;

    for (int r = 0; r < kd; r++)
        for (int c = 0; c < vd; c++)
            st[(size_t)r * vd + c] = st[(size_t)r * vd + c] + kvec[r] * delta[c];

    if (!out)
        return;
    for (int c = 0; c < vd; c++)
        out[c] = 0.0f;
    for (int r = 0; r < kd; r++)
        for (int c = 0; c < vd; c++)
            out[c] = out[c] + st[(size_t)r * vd + c] * qvec[r];
}

/* One unit: every value head i of the unit, with its key head
 * i / (vh / kh) ("Kestrel_VLLM #24", section 4: three value heads share each
 * key head, value head i taking key head i / rep). */
static void unit_update(float *Su, const float *qu, const float *ku,
                        const float *vu, const float *gu, const float *bu,
                        float *ou, int vh, int kh, int kd, int vd)
{
    const int group = vh / kh;
    for (int i = 0; i < vh; i++) {
        const int key = i / group;
        tile_update(Su + (size_t)i * kd * vd, qu + (size_t)key * kd,
                    ku + (size_t)key * kd, vu + (size_t)i * vd, expf(gu[i]), bu[i],
                    ou ? ou + (size_t)i * vd : NULL, kd, vd);
    }
}

int ref_gdn_step(float *S, const float *q, const float *k, const float *v,
                 const float *g, const float *beta, float *o,
                 int64_t n_units, int vh, int kh, int kd, int vd)
{
    if (!dims_ok(n_units, vh, kh, kd, vd))
        return -1;
    if (n_units == 0)
        return 0;
    if (!S || !q || !k || !v || !g || !beta || !o)
        return -1;
    for (int64_t u = 0; u < n_units; u++)
        unit_update(S + (size_t)u * vh * kd * vd, q + (size_t)u * kh * kd,
                    k + (size_t)u * kh * kd, v + (size_t)u * vh * vd,
                    g + (size_t)u * vh, beta + (size_t)u * vh,
                    o + (size_t)u * vh * vd, vh, kh, kd, vd);
    return 0;
}

/* "Kestrel_VLLM #34", section 3.6: the recurrence is serial in time; M rows
 * are M single steps in order, each with row m's inputs, the state advancing
 * in place.  No chunked scan. */
int ref_gdn_step_m(float *S, const float *q, const float *k, const float *v,
                   const float *g, const float *beta, float *o,
                   int64_t n_units, int M, int vh, int kh, int kd, int vd)
{
    if (!dims_ok(n_units, vh, kh, kd, vd) || M < 0)
        return -1;
    if (n_units == 0 || M == 0)
        return 0;
    const size_t nqk = (size_t)n_units * kh * kd;
    const size_t nv = (size_t)n_units * vh * vd;
    const size_t ng = (size_t)n_units * vh;
    for (int m = 0; m < M; m++) {
        int rc = ref_gdn_step(S, q + m * nqk, k + m * nqk, v + m * nv,
                              g + m * ng, beta + m * ng, o + m * nv,
                              n_units, vh, kh, kd, vd);
        if (rc)
            return rc;
    }
    return 0;
}

/* The conv history is a queue of the last ck - 1 raw conv INPUT frames,
 * oldest first ("Kestrel_VLLM #24", section 3): a new frame enters at the
 * back and the oldest leaves at the front. */
void ref_conv_push(float *hist, const float *raw, int conv_dim, int ck)
{
    const int frames = ck - 1;
    if (frames < 1)
        return;
    const size_t fb = (size_t)conv_dim * sizeof(float);
    memmove(hist, hist + conv_dim, (size_t)(frames - 1) * fb);
    memcpy(hist + (size_t)(frames - 1) * conv_dim, raw, fb);
}

/* "Kestrel_VLLM #34", section 3.7: mark is a plain copy of S and the conv
 * history; the snapshot is one-shot. */
int ref_gdn_mark(ref_slab *slab, const float *S, const float *hist)
{
    if (!slab || !S || !slab->S_snap)
        return -1;
    if (!dims_ok(slab->n_units, slab->vh, slab->kh, slab->kd, slab->vd))
        return -1;
    const size_t ns = (size_t)slab->n_units * slab->vh * slab->kd * slab->vd;
    memcpy(slab->S_snap, S, ns * sizeof(float));
    if (hist && slab->hist_snap && slab->hist_floats > 0)
        memcpy(slab->hist_snap, hist,
               (size_t)slab->n_units * slab->hist_floats * sizeof(float));
    slab->armed = 1;
    return 0;
}

/* Rollback to an accepted length: restore the marked bytes, then re-run the
 * first accepted[u] single steps of unit u from the rows given to step_m;
 * the conv history re-receives the same raw frames.  One-shot: disarms.
 * ("Kestrel_VLLM #34", section 3.7: restore, then the caller replays single
 * steps; here the replay is folded into the call.) */
int ref_gdn_rollback(ref_slab *slab, float *S, float *hist,
                     const float *q, const float *k, const float *v,
                     const float *g, const float *beta,
                     const float *xc_raw, int conv_dim, int ck,
                     int M, const int32_t *accepted)
{
    if (!slab || !S || !accepted || !slab->armed || M < 0)
        return -1;
    const int64_t N = slab->n_units;
    const int vh = slab->vh, kh = slab->kh, kd = slab->kd, vd = slab->vd;
    for (int64_t u = 0; u < N; u++)
        if (accepted[u] < 0 || accepted[u] > M)
            return -1;
    int any = 0;
    for (int64_t u = 0; u < N; u++)
        any |= accepted[u] > 0;
    if (any && (!q || !k || !v || !g || !beta))
        return -1;
    const int with_hist = hist && slab->hist_snap && slab->hist_floats > 0;
    if (with_hist && (ck < 2 || (int64_t)(ck - 1) * conv_dim != slab->hist_floats))
        return -1;
    if (with_hist && any && !xc_raw)
        return -1;

    const size_t per_s = (size_t)vh * kd * vd;
    memcpy(S, slab->S_snap, (size_t)N * per_s * sizeof(float));
    if (with_hist)
        memcpy(hist, slab->hist_snap, (size_t)N * slab->hist_floats * sizeof(float));

    /* row m of an input laid out [M][N][w] starts at (m * N + u) * w for unit u */
    for (int64_t u = 0; u < N; u++) {
        for (int m = 0; m < accepted[u]; m++) {
            const size_t row = (size_t)m * N + (size_t)u;
            unit_update(S + (size_t)u * per_s, q + row * kh * kd, k + row * kh * kd,
                        v + row * vh * vd, g + row * vh, beta + row * vh, NULL,
                        vh, kh, kd, vd);
            if (with_hist)
                ref_conv_push(hist + (size_t)u * slab->hist_floats,
                              xc_raw + row * conv_dim, conv_dim, ck);
        }
    }
    slab->armed = 0;
    return 0;
}

/* The log-domain gate from the a projection ("Kestrel_VLLM #24", section 3
 * and Fig. 1 caption): g = -exp(A_log) * softplus(a + dt_bias), with
 * softplus(z) = log(1 + e^z) taken as z itself for z > 20 and as e^z for
 * z < -20, where the dropped term lies below fp32 resolution. */
static float log_gate(float a, float A_log, float dt_bias)
{
    const float z = a + dt_bias;
    float softplus;
    if (z > 20.0f)
        softplus = z;
    else if (z < -20.0f)
        softplus = expf(z);
    else
        softplus = log1pf(expf(z));
    return -expf(A_log) * softplus;
}

int ref_gdn_frontend(const float *x, const float *Wa, const float *Wb,
                     const float *A_log, const float *dt_bias,
                     const float *xc_raw, float *hist, const float *conv_w,
                     float *q, float *k, float *v, float *g, float *beta,
                     int B, int dim, int conv_dim, int ck,
                     int vh, int kh, int kd, int vd)
{
    if (B < 0 || dim <= 0 || ck < 1 || !dims_ok(1, vh, kh, kd, vd))
        return -1;
    if (conv_dim != 2 * kh * kd + vh * vd)
        return -1;
    if (B == 0)
        return 0;
    if (!x || !Wa || !Wb || !A_log || !dt_bias || !xc_raw || !conv_w ||
        !q || !k || !v || !g || !beta || (ck > 1 && !hist))
        return -1;

    const int qk_w = kh * kd;
    float *out = (float *)malloc((size_t)conv_dim * sizeof(float)); /* one row's conv output */
    if (!out)
        return -1;
    const float q_scale = 1.0f / sqrtf((float)kd);

    for (int b = 0; b < B; b++) {
        const float *xb = x + (size_t)b * dim;
        /* (i) paired GEMV ("Kestrel_VLLM #27", section 4.2): two same-shape
         * row-times-vector products, a from Wa, b from Wb; left folds. */
        for (int r = 0; r < vh; r++) {
            float acc_a = 0.0f, acc_b = 0.0f;
            for (int c = 0; c < dim; c++) {
                acc_a = acc_a + Wa[(size_t)r * dim + c] * xb[c];
                acc_b = acc_b + Wb[(size_t)r * dim + c] * xb[c];
            }
            /* (ii) gate and beta ("Kestrel_VLLM #24", section 3 and Fig. 1
             * caption): the gate comes from a, in the log domain and
             * negative; beta comes from b. */
            g[(size_t)b * vh + r] = log_gate(acc_a, A_log[r], dt_bias[r]);
            beta[(size_t)b * vh + r] = 1.0f / (1.0f + expf(-acc_b));
        }

        /* (iii) depthwise causal conv + SiLU per channel ("Kestrel_VLLM
         * #24", section 3): taps 0..ck-2 over the history frames (oldest
         * first), the last tap over the current raw input; then the history
         * advances by the raw input; then silu(acc) = acc / (1 + exp(-acc)). */
        const float *frames[ck];                 /* the window, oldest first */
        float *queue = hist ? hist + (size_t)b * (ck - 1) * conv_dim : NULL;
        for (int j = 0; j + 1 < ck; j++)
            frames[j] = queue + (size_t)j * conv_dim;
        frames[ck - 1] = xc_raw + (size_t)b * conv_dim;
        for (int ch = 0; ch < conv_dim; ch++) {
            float y = 0.0f;
            for (int j = 0; j < ck; j++)
                y = y + conv_w[(size_t)ch * ck + j] * frames[j][ch];
            out[ch] = y / (1.0f + expf(-y));
        }
        if (queue)
            ref_conv_push(queue, frames[ck - 1], conv_dim, ck);

        /* (iv) split into q | k | v ("Kestrel_VLLM #34", section 3.6: the
         * step receives the conv output at offsets 0, kh*kd, 2*kh*kd). */
        float *qb = q + (size_t)b * qk_w, *kb = k + (size_t)b * qk_w;
        memcpy(qb, out, (size_t)qk_w * sizeof(float));
        memcpy(kb, out + qk_w, (size_t)qk_w * sizeof(float));
        memcpy(v + (size_t)b * vh * vd, out + 2 * qk_w, (size_t)vh * vd * sizeof(float));

        /* (v) per key head L2 normalisation ("Kestrel_VLLM #24", Fig. 1
         * caption and section 4 name the step without a formula):
         * x * (1/sqrt(sum x^2 + 1e-6)); q additionally * 1/sqrt(kd). */
        for (int h = 0; h < kh; h++) {
            float *qh = qb + (size_t)h * kd, *kk = kb + (size_t)h * kd;
            float ssq = 0.0f, ssk = 0.0f;
            for (int j = 0; j < kd; j++) {
                ssq = ssq + qh[j] * qh[j];
                ssk = ssk + kk[j] * kk[j];
            }
            const float iq = 1.0f / sqrtf(ssq + 1e-6f);
            const float ik = 1.0f / sqrtf(ssk + 1e-6f);
            for (int j = 0; j < kd; j++) {
                qh[j] = (qh[j] * iq) * q_scale;
                kk[j] = kk[j] * ik;
            }
        }
    }
    free(out);
    return 0;
}

/* "Kestrel_VLLM #34", section 3.6: the M draft rows run the per-row front end
 * serially, the conv history advancing in place; inputs and outputs are
 * [M][B][...]. */
int ref_gdn_frontend_m(const float *x, const float *Wa, const float *Wb,
                       const float *A_log, const float *dt_bias,
                       const float *xc_raw, float *hist, const float *conv_w,
                       float *q, float *k, float *v, float *g, float *beta,
                       int B, int M, int dim, int conv_dim, int ck,
                       int vh, int kh, int kd, int vd)
{
    if (M < 0 || B < 0)
        return -1;
    for (int m = 0; m < M; m++) {
        const size_t r = (size_t)m * B;
        int rc = ref_gdn_frontend(x + r * dim, Wa, Wb, A_log, dt_bias, xc_raw + r * conv_dim,
                                  hist, conv_w, q + r * kh * kd, k + r * kh * kd,
                                  v + r * vh * vd, g + r * vh, beta + r * vh,
                                  B, dim, conv_dim, ck, vh, kh, kd, vd);
        if (rc)
            return rc;
    }
    return 0;
}

/* Gated RMSNorm of the layer output ("Kestrel_VLLM #24", Fig. 1 caption,
 * step 6, after the recurrence; one group per value head; no formula on the
 * pages, the model family's definition is used): per row of vd outputs,
 * ms = (sum o^2) / vd, r = 1/sqrt(ms + eps),
 * out = ((o * r) * w) * silu(z), silu(z) = z / (1 + exp(-z)). */
int ref_gdn_gated_norm(const float *o, const float *z, const float *w, float eps,
                       float *out, int64_t rows, int vd)
{
    if (rows < 0 || vd <= 0 || !(eps >= 0.0f))
        return -1;
    if (rows == 0)
        return 0;
    if (!o || !z || !w || !out)
        return -1;
    for (int64_t r = 0; r < rows; r++) {
        const float *orow = o + (size_t)r * vd, *zrow = z + (size_t)r * vd;
        float ss = 0.0f;
        for (int c = 0; c < vd; c++)
            ss = ss + orow[c] * orow[c];
        const float rinv = 1.0f / sqrtf(ss / (float)vd + eps);
        for (int c = 0; c < vd; c++) {
            const float sz = zrow[c] / (1.0f + expf(-zrow[c]));
            out[(size_t)r * vd + c] = ((orow[c] * rinv) * w[c]) * sz;
        }
    }
    return 0;
}

/* The layer's dense projections ("Kestrel_VLLM #24", Fig. 1 caption, steps
 * 1 and 7: in_proj_qkv feeding the conv, in_proj_z feeding the output gate,
 * out_proj after the gated norm; "Kestrel_VLLM #34", section 3.6: for M
 * draft rows the projections take all rows at once so that the weights are
 * read once, each row giving what a one-row call gives).  Per row r and
 * output o: acc = 0; acc = acc + W[o][c] * x[r][c] for c = 0..C-1. */
int ref_gdn_proj(const float *x, const float *W, float *y, int64_t rows, int R, int C)
{
    if (rows < 0 || R <= 0 || C <= 0)
        return -1;
    if (rows == 0)
        return 0;
    if (!x || !W || !y)
        return -1;
    for (int64_t r = 0; r < rows; r++) {
        const float *xr = x + (size_t)r * C;
        for (int o = 0; o < R; o++) {
            const float *wo = W + (size_t)o * C;
            float acc = 0.0f;
            for (int c = 0; c < C; c++)
                acc = acc + wo[c] * xr[c];
            y[(size_t)r * R + o] = acc;
        }
    }
    return 0;
}

/* binary16: sign bit, 5-bit exponent e (bias 15), 10-bit fraction f.
 * e = 0: zero or subnormal, f * 2^-24; 0 < e < 31: (1024 + f) * 2^(e - 25);
 * e = 31: infinity (f = 0) or NaN.  Every finite value is exact in binary32.
 * (The half-precision block scales of "Kestrel_VLLM #24", section 12, whose
 * conversion the page states is exact and unique for every non-NaN input.) */
static float half_to_float(uint16_t h)
{
    const int e = (h >> 10) & 0x1f;
    const int f = h & 0x3ff;
    float mag;
    if (e == 0)
        mag = ldexpf((float)f, -24);
    else if (e == 31)
        mag = f ? NAN : INFINITY;
    else
        mag = ldexpf((float)(1024 + f), e - 25);
    return (h & 0x8000) ? -mag : mag;
}

void ref_half_to_float(const uint16_t *h, float *f, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        f[i] = half_to_float(h[i]);
}

/* The 4-bit projection of the q4 tier ("Kestrel_VLLM #24", section 8: the
 * three large projections read 4-bit weights with f32 activations; section
 * 12: signed 4-bit values times a half-precision block scale; the 63.9 MB of
 * weights it reads per layer fixes 32 weights per scale).  The weight is
 * formed exactly, then the strict left fold of ref_gdn_proj. */
int ref_gdn_proj_q4(const float *x, const uint8_t *q, const uint16_t *scale, float *y,
                    int64_t rows, int R, int C)
{
    if (rows < 0 || R <= 0 || C <= 0 || C % 32 != 0)
        return -1;
    if (rows == 0)
        return 0;
    if (!x || !q || !scale || !y)
        return -1;
    for (int64_t r = 0; r < rows; r++) {
        const float *xr = x + (size_t)r * C;
        for (int o = 0; o < R; o++) {
            const uint8_t *qo = q + (size_t)o * (C / 2);
            const uint16_t *so = scale + (size_t)o * (C / 32);
            float acc = 0.0f;
            for (int c = 0; c < C; c++) {
                const int nib = (c & 1) ? (qo[c / 2] >> 4) : (qo[c / 2] & 0x0f);
                const int n = (nib ^ 8) - 8;
                const float w = (float)n * half_to_float(so[c / 32]);
                acc = acc + w * xr[c];
            }
            y[(size_t)r * R + o] = acc;
        }
    }
    return 0;
}

/*
 * Double-precision brute force, re-associated: S' = alpha (I - beta k k^T) S
 * + beta k v^T and o = S'^T q, with the kd x kd matrix P = alpha (I - beta k
 * k^T) formed explicitly and multiplied into S.  Algebraically equal to the
 * whole-tile passes of tile_update: S'^T k-term expands as alpha S - alpha beta
 * k (k^T S) + beta k v^T.
 */
int ref64_gdn_step(double *S, const double *q, const double *k,
                   const double *v, const double *g, const double *beta,
                   double *o, int64_t n_units, int vh, int kh, int kd, int vd)
{
    if (!dims_ok(n_units, vh, kh, kd, vd) || kd > 16 || vd > 16)
        return -1;
    if (!S || !q || !k || !v || !g || !beta || !o)
        return -1;
    const int rep = vh / kh;
    for (int64_t u = 0; u < n_units; u++) {
        for (int i = 0; i < vh; i++) {
            const int hh = i / rep;
            double *Sh = S + ((size_t)u * vh + i) * kd * vd;
            const double *kk = k + ((size_t)u * kh + hh) * kd;
            const double *qq = q + ((size_t)u * kh + hh) * kd;
            const double *vv = v + ((size_t)u * vh + i) * vd;
            const double alpha = exp(g[(size_t)u * vh + i]);
            const double bt = beta[(size_t)u * vh + i];
            double P[16][16], R[16][16];
            for (int a = 0; a < kd; a++)
                for (int c = 0; c < kd; c++)
                    P[a][c] = alpha * ((a == c ? 1.0 : 0.0) - bt * kk[a] * kk[c]);
            for (int a = 0; a < kd; a++)
                for (int c = 0; c < vd; c++) {
                    double s = 0.0;
                    for (int e = 0; e < kd; e++)
                        s += P[a][e] * Sh[(size_t)e * vd + c];
                    R[a][c] = s + bt * kk[a] * vv[c];
                }
            for (int a = 0; a < kd; a++)
                for (int c = 0; c < vd; c++)
                    Sh[(size_t)a * vd + c] = R[a][c];
            double *oo = o + ((size_t)u * vh + i) * vd;
            for (int c = 0; c < vd; c++) {
                double s = 0.0;
                for (int a = 0; a < kd; a++)
                    s += R[a][c] * qq[a];
                oo[c] = s;
            }
        }
    }
    return 0;
}
