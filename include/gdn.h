/*
 * gdn.h -- C ABI of the MI355X (gfx950) Gated DeltaNet recurrent decode step.
 *
 * Operator ("Kestrel_VLLM #24: GDN linear attention on GPU", section 4 and
 * Fig. 1 caption; "Kestrel_VLLM #27: register residency and fused launch",
 * section 3.1).  For every unit u (one sequence x layer state) and value head
 * i, with key head h = i / (vh / kh):
 *     alpha = exp(g[u][i])
 *     S     = alpha * S                          (S = S[u][i], kd x vd, fp32)
 *     kv    = S^T k[u][h]                        (decayed state)
 *     tmp   = (v[u][i] - kv) * beta[u][i]
 *     S     = S + k[u][h] tmp^T                  (rank-1 update, in place)
 *     o[u][i] = S^T q[u][h]                      (updated state)
 *
 * Conventions shared by every call:
 *  - Every pointer named as device memory is a device pointer (e.g. a torch
 *    tensor's data_ptr) owned by the caller, fp32 unless stated, contiguous,
 *    and 16-byte aligned.  The library allocates nothing and keeps no global
 *    mutable state other than gdn_rollback_static's count area.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  A
 *    call validates its arguments on the host, enqueues its kernels on the
 *    stream and returns without synchronising, except where noted.
 *  - Return: GDN_OK (0) once enqueued, or a negative error code.  On a
 *    refusal (GDN_EINVAL, GDN_EUNSUPPORTED, GDN_ESTATE) nothing has been
 *    enqueued and nothing has changed; GDN_EDEVICE reports a runtime failure,
 *    possibly after part of the call's work was enqueued.  Shapes the kernels
 *    were not built for are refused, never served by a slower fallback
 *    ("Kestrel_VLLM #34", section 3.5: a path that was not validated is
 *    refused rather than taken silently).
 *  - Layouts (row-major; N = n_units; M = draft rows, 1 for a single step):
 *      S        [N][vh][kd][vd]   dv fastest
 *      q, k     [M][N][kh][kd]
 *      v, o     [M][N][vh][vd]
 *      g, beta  [M][N][vh]        g is the log-domain gate (<= 0 in use)
 *    The unit order inside N is the caller's (sequence-major in the tests).
 *  - Supported: kd == vd in {64, 128}, vh % kh == 0, vh <= 4096.  A launch
 *    stays below 2^32 work-items: n_units * vh * 1024 (kd = 128) or
 *    n_units * vh * 256 (kd = 64), plus any history replay; larger calls
 *    return GDN_EUNSUPPORTED.
 *  - S must not overlap q, k, v, g, beta or o.
 */
#ifndef GDN_H
#define GDN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_OK 0
#define GDN_EINVAL (-1)       /* NULL/misaligned pointer, bad size, aliasing, bad M or accepted[] */
#define GDN_EUNSUPPORTED (-2) /* a shape the kernels are not built for */
#define GDN_ESTATE (-3)       /* slab not armed, too small, or mismatched */
#define GDN_EDEVICE (-4)      /* the HIP runtime reported a launch or copy error */

/* Text for an error code (static storage). */
const char *gdn_strerror(int rc);

/*
 * One decode step for N units.  S is read and written in place; o receives
 * S'^T q.  n_units == 0 is a no-op.
 * ("Kestrel_VLLM #24", section 4: one state update per token per head.)
 */
int gdn_step(float *S, const float *q, const float *k, const float *v,
             const float *g, const float *beta, float *o, int64_t n_units,
             int32_t vh, int32_t kh, int32_t kd, int32_t vd, void *stream);

/*
 * M sequential steps for N units (speculative verify): step m uses row m of
 * q, k, v, g, beta and writes row m of o; S advances in place through all M
 * steps.  Bit-identical to M calls of gdn_step with the same rows.
 * 1 <= M <= 64.  ("Kestrel_VLLM #34: batched M rows", section 3.6: the
 * recurrence is serial in time, rows are M single steps.)
 */
int gdn_step_m(float *S, const float *q, const float *k, const float *v,
               const float *g, const float *beta, float *o, int64_t n_units,
               int32_t M, int32_t vh, int32_t kh, int32_t kd, int32_t vd,
               void *stream);

/*
 * M sequential steps (1 <= M <= 64; M = 1 is a single step) whose output goes
 * through the layer's gated RMSNorm in the same launch, so the raw read-out
 * never reaches memory ("Kestrel_VLLM #24", Fig. 1 caption, step 6: gated
 * RMSNorm after the recurrence, one group per value head; the pages give no
 * formula, this is the model family's definition):
 *   out[m][u][i][:] = (o / sqrt(mean(o^2) + eps)) * norm_w * silu(z[m][u][i][:])
 * with o = S'^T q of that step and silu(z) = z / (1 + exp(-z)).
 * z, out [M][N][vh][vd]; norm_w [vd]; 0 <= eps <= 1.  S advances exactly as
 * in gdn_step_m (same bits).
 */
int gdn_step_gated(float *S, const float *q, const float *k, const float *v,
                   const float *g, const float *beta, const float *z,
                   const float *norm_w, float eps, float *out, int64_t n_units,
                   int32_t M, int32_t vh, int32_t kh, int32_t kd, int32_t vd,
                   void *stream);

/*
 * Snapshot slab for mark / rollback ("Kestrel_VLLM #34", section 3.7: the
 * recurrent state and the conv history can only be restored from a copy; the
 * snapshot is one-shot).  The struct lives in caller host memory; `dev`
 * points at caller device memory of at least gdn_slab_bytes() bytes.  Fields
 * are managed by the library; treat them as read-only.
 */
typedef struct gdn_slab {
    void *dev;            /* device memory: S snapshot | hist snapshot | accepted[] */
    int64_t bytes;        /* size of dev */
    int64_t n_units;
    int64_t hist_floats;  /* conv-history floats per unit, (ck-1)*conv_dim, or 0 */
    int32_t vh, kh, kd, vd;
    int32_t armed;        /* bit 0: state marked; bit 1: history marked */
    int32_t magic;        /* set by gdn_slab_init */
} gdn_slab;

/* Device bytes a slab for n_units units needs: the state snapshot, the
 * conv-history snapshot (hist_floats_per_unit floats per unit, 0 for none,
 * a multiple of 4) and the per-unit count area, each 256-byte aligned.  The
 * caller sizes the slab for the largest call it will make, not the current
 * one ("Kestrel_VLLM #34", section 3.5: the draft-row buffer is allocated for
 * the maximum row count), and queries the size before allocating
 * ("Kestrel_VLLM #24", section 10: a size query before the copy, a refusal
 * rather than a truncation).  Returns the byte count, or GDN_EINVAL for bad
 * dims, n_units < 1 or a hist size that is negative or not a multiple of 4;
 * GDN_EUNSUPPORTED for an unsupported kd / vd, more units than one
 * recurrence launch takes (n_units * vh tiles within the grid limit of
 * gdn_step), or more than 2^24 history floats per unit. */
int64_t gdn_slab_bytes(int64_t n_units, int32_t vh, int32_t kh, int32_t kd,
                       int32_t vd, int64_t hist_floats_per_unit);

/* Bind a slab to caller device memory `dev` (256-byte aligned) of `bytes`
 * bytes ("Kestrel_VLLM #34", section 3.7: the snapshot of the state and of
 * the conv history).  Host only, enqueues nothing; leaves the slab disarmed.
 * Errors: GDN_EINVAL for a null slab or dev, a misaligned dev or bad sizes;
 * GDN_ESTATE when bytes < gdn_slab_bytes(...). */
int gdn_slab_init(gdn_slab *slab, void *dev, int64_t bytes, int64_t n_units,
                  int32_t vh, int32_t kh, int32_t kd, int32_t vd,
                  int64_t hist_floats_per_unit);

/* Copy S (and hist [N][hist_floats] unless NULL) into the slab and arm it
 * ("Kestrel_VLLM #34", section 3.7: the recurrent state and the conv history
 * cannot be recomputed backwards, so a copy is taken before the draft rows
 * run).  Re-marking an armed slab overwrites the snapshot.  Errors:
 * GDN_ESTATE for an uninitialised slab or a hist on a slab without a history
 * area; GDN_EINVAL for a bad pointer or S / hist overlapping the slab. */
int gdn_mark(gdn_slab *slab, const float *S, const float *hist, void *stream);

/*
 * gdn_mark(slab, S, hist) followed by gdn_step_m(S, ..., M), with the state
 * read from memory once: each tile is written to the snapshot as loaded and
 * then advanced.  Same results, bit for bit, as the two calls; arms the slab
 * like gdn_mark.  n_units and the dims must equal the slab's (else
 * GDN_ESTATE).  ("Kestrel_VLLM #34", section 3.7: mark before the M-row
 * verify.)  hist is copied as it stands at this call, so it must still be
 * the history the draft rows were computed from: pair this call with
 * gdn_frontend_verify_m, which leaves the history as it was.  After
 * gdn_frontend_m the history already holds the draft rows' frames, and a
 * rollback would push the accepted frames a second time (mark with gdn_mark
 * before gdn_frontend_m instead).
 */
int gdn_mark_step_m(gdn_slab *slab, float *S, const float *hist, const float *q,
                    const float *k, const float *v, const float *g,
                    const float *beta, float *o, int64_t n_units, int32_t M,
                    int32_t vh, int32_t kh, int32_t kd, int32_t vd, void *stream);

/*
 * Roll back to an accepted length: for every unit u, S (and hist, unless
 * NULL) become the marked bytes advanced by accepted[u] single steps that use
 * rows 0..accepted[u]-1 of the inputs given to gdn_step_m (q, k, v, g, beta,
 * [M][N][...]); no o is written ("Kestrel_VLLM #34", section 3.7: restore the
 * snapshot, then re-run the accepted rows; the snapshot is one-shot).  The
 * history replays the raw conv input frames xc_raw [M][N][conv_dim] (needed
 * only with hist): ck is the conv kernel width, which must be 4 (else
 * GDN_EUNSUPPORTED), and conv_dim * (ck - 1) must equal the slab's
 * hist_floats (else GDN_EINVAL); both are ignored when hist is NULL.
 * accepted is a HOST array of N int32 in 0..M (else GDN_EINVAL).  The counts
 * reach the device inside the arguments of the call's launches, so the array
 * is no longer read once the call returns, whatever memory holds it.
 * accepted[u] == 0 restores the marked bytes exactly; accepted[u] == M
 * reproduces gdn_step_m bit for bit.  The slab is disarmed afterwards: a
 * rollback on a disarmed slab, or with hist when the history was not marked,
 * returns GDN_ESTATE and changes nothing.  A launch that would pass the grid
 * limit (the units' tiles plus their history replay: fewer than 2^32
 * work-items) returns GDN_EUNSUPPORTED.
 */
int gdn_rollback(gdn_slab *slab, float *S, float *hist, const float *q,
                 const float *k, const float *v, const float *g,
                 const float *beta, const float *xc_raw, int32_t conv_dim,
                 int32_t ck, int32_t M, const int32_t *accepted, void *stream);

/*
 * gdn_rollback for callers that cannot allocate device memory (code under
 * graph capture, serving loops, harnesses that forbid allocation): the same
 * arguments, refusals and results, bit for bit, but the per-unit counts are
 * staged in a count area the library owns instead of the slab's: one static
 * device array of 65536 int32 (256 KiB) per GPU, held until the process
 * ends.  The call allocates nothing.  More than 65536 units (the slab's
 * n_units) are refused with GDN_EUNSUPPORTED before anything is enqueued.
 * Every call on one GPU shares that GPU's area and overwrites the counts of
 * its own units before reading them; calls that overlap on one GPU (on
 * different streams, or from different threads) race and must be ordered by
 * the caller.
 */
int gdn_rollback_static(gdn_slab *slab, float *S, float *hist, const float *q,
                        const float *k, const float *v, const float *g,
                        const float *beta, const float *xc_raw, int32_t conv_dim,
                        int32_t ck, int32_t M, const int32_t *accepted, void *stream);

/*
 * Speculative verify without a snapshot.  The M draft rows are evaluated
 * against the state, which is left untouched; the accepted prefix is
 * applied afterwards by gdn_commit.  A verify + commit cycle reads the state
 * twice and writes it once, against five state passes for mark + step_m +
 * rollback (snapshot copy, M-step read/write, restore read/write), and needs
 * no slab.  Same results, bit for bit, as gdn_mark + gdn_step_m +
 * gdn_rollback with the same rows and accepted lengths.
 *
 * gdn_verify_m: o [M][N][vh][vd] as gdn_step_m would produce them; S is read
 * only.  1 <= M <= 64.
 */
int gdn_verify_m(const float *S, const float *q, const float *k,
                 const float *v, const float *g, const float *beta, float *o,
                 int64_t n_units, int32_t M, int32_t vh, int32_t kh, int32_t kd,
                 int32_t vd, void *stream);

/*
 * gdn_verify_m_gated: the outputs gdn_step_gated would produce for the M
 * draft rows (each head's read-out through the gated RMSNorm,
 * "Kestrel_VLLM #24", Fig. 1 caption, step 6), S read only, bit for bit.
 * z [M][N][vh][vd] (the gate), norm_w [vd], 0 <= eps <= 1, out
 * [M][N][vh][vd].  The accepted prefix is then applied by gdn_commit as for
 * gdn_verify_m.  Errors as gdn_step_gated.
 */
int gdn_verify_m_gated(const float *S, const float *q, const float *k,
                       const float *v, const float *g, const float *beta,
                       const float *z, const float *norm_w, float eps, float *out,
                       int64_t n_units, int32_t M, int32_t vh, int32_t kh, int32_t kd,
                       int32_t vd, void *stream);

/*
 * gdn_commit: advance every unit u by accepted[u] single steps using rows
 * 0..accepted[u]-1 of the inputs given to gdn_verify_m, in place; with hist
 * (nullable) the conv history [N][ck-1][conv_dim] receives the raw conv input
 * frames xc_raw [M][N][conv_dim] of those rows (ck must be 4, else
 * GDN_EUNSUPPORTED; ignored when hist is NULL).  accepted is a DEVICE array
 * of N int32, read by the kernels (so the whole cycle can be captured into a
 * graph).  An entry outside 0..M leaves that unit's state and history
 * unchanged and sets *status = 1 (status: device int32, nullable; never
 * cleared by the library).  Units with accepted[u] == 0 are not touched.
 * ("Kestrel_VLLM #34", section 3.7: after verification only the accepted
 * prefix may remain applied to the state and the history.)
 * Errors: GDN_EINVAL for M outside 1..64, n_units < 0, a null or misaligned
 * pointer, or S, hist or status overlapping another array of the call;
 * GDN_EUNSUPPORTED for the shapes gdn_step refuses, ck != 4 with a history,
 * or a history replay that takes the launch past the grid limit (fewer than
 * 2^32 work-items with the tiles).  n_units == 0 is a no-op.
 */
int gdn_commit(float *S, float *hist, const float *q, const float *k,
               const float *v, const float *g, const float *beta,
               const float *xc_raw, int32_t conv_dim, int32_t ck, int64_t n_units,
               int32_t M, int32_t vh, int32_t kh, int32_t kd, int32_t vd,
               const int32_t *accepted, int32_t *status, void *stream);

/*
 * gdn_commit followed by gdn_verify_m, in one pass over the state: each unit
 * applies accepted[u] rows of the first set (q, k, v, g, beta [M][N][...],
 * the rows of the previous verify; hist and xc_raw as in gdn_commit), the
 * committed state is stored, and the M2 rows of the second set (q2, k2, v2,
 * g2, beta2 [M2][N][...], the next draft rows) run from it, writing o
 * [M2][N][vh][vd] as gdn_verify_m does; the state is not advanced by them.
 * Same results, bit for bit, as the two calls, with one read of the state
 * instead of two per speculative cycle ("Kestrel_VLLM #34", section 3.7:
 * only the accepted prefix remains applied; section 3.6: the draft rows are
 * serial steps from the current state).  1 <= M, M2 <= 64; ungated outputs.
 * Errors: those of gdn_commit and gdn_verify_m, and GDN_EINVAL when o or
 * the history overlaps another array of the call.
 */
int gdn_commit_verify_m(float *S, float *hist, const float *q, const float *k,
                        const float *v, const float *g, const float *beta,
                        const float *xc_raw, int32_t conv_dim, int32_t ck,
                        int64_t n_units, int32_t M, const int32_t *accepted,
                        int32_t *status, const float *q2, const float *k2,
                        const float *v2, const float *g2, const float *beta2, float *o,
                        int32_t M2, int32_t vh, int32_t kh, int32_t kd, int32_t vd,
                        void *stream);

/*
 * Front end of one GDN layer for B rows ("Kestrel_VLLM #27", section 4.2:
 * the beta and a projections as one paired launch; "Kestrel_VLLM #24",
 * section 3 and Fig. 1 caption: gate/beta transform, depthwise causal conv +
 * SiLU with the history of raw conv inputs, split, per key-head norm):
 *   a = Wa x_b, b = Wb x_b                     Wa, Wb [vh][dim]
 *   g = -exp(A_log) * softplus(a + dt_bias)    softplus(z) = z above 20,
 *                                              exp(z) below -20
 *   beta = 1 / (1 + exp(-b))
 *   c[ch] = silu(sum_{j<ck-1} conv_w[ch][j] hist[b][j][ch]
 *                + conv_w[ch][ck-1] xc_raw[b][ch])
 *   hist[b] shifts one frame towards the oldest slot; the newest gets xc_raw[b]
 *   q = c[0 : kh*kd], k = c[kh*kd : 2*kh*kd], v = c[2*kh*kd : conv_dim]
 *   per key head: q *= 1/sqrt(sum q^2 + 1e-6) * 1/sqrt(kd);
 *                 k *= 1/sqrt(sum k^2 + 1e-6)
 * x [B][dim] (dim % 4 == 0); A_log, dt_bias [vh]; xc_raw [B][conv_dim];
 * hist [B][ck-1][conv_dim] in/out; conv_w [conv_dim][ck]; outputs q, k
 * [B][kh][kd], v [B][vh][vd], g, beta [B][vh] feed gdn_step with N = B.
 * conv_dim must equal 2*kh*kd + vh*vd; ck must be 4.
 * Errors: GDN_EINVAL for a null or misaligned pointer, B < 0, dim not a
 * positive multiple of 4, a conv_dim other than the one above, or an output
 * (q, k, v, g, beta, hist) overlapping another array of the call;
 * GDN_EUNSUPPORTED for the kd / vd gdn_step refuses, ck != 4, or a launch
 * beyond the grid limit.  B == 0 is a no-op.
 */
int gdn_frontend(const float *x, const float *Wa, const float *Wb,
                 const float *A_log, const float *dt_bias, const float *xc_raw,
                 float *hist, const float *conv_w, float *q, float *k, float *v,
                 float *g, float *beta, int32_t B, int32_t dim, int32_t conv_dim,
                 int32_t ck, int32_t vh, int32_t kh, int32_t kd, int32_t vd,
                 void *stream);

/*
 * Front end for M draft rows of B units in one call (speculative verify):
 * equivalent, bit for bit, to M successive gdn_frontend calls where call m
 * takes row m of x [M][B][dim] and xc_raw [M][B][conv_dim] and the history
 * advances one frame per row; outputs q, k [M][B][kh][kd], v [M][B][vh][vd],
 * g, beta [M][B][vh] are exactly the rows gdn_step_m takes (N = B).
 * 1 <= M <= 64; other arguments as gdn_frontend.  ("Kestrel_VLLM #34",
 * section 3.6: the per-row conv/norm/step chain runs serially over the M rows
 * with the history advancing in place.)
 */
int gdn_frontend_m(const float *x, const float *Wa, const float *Wb,
                   const float *A_log, const float *dt_bias, const float *xc_raw,
                   float *hist, const float *conv_w, float *q, float *k, float *v,
                   float *g, float *beta, int32_t B, int32_t M, int32_t dim,
                   int32_t conv_dim, int32_t ck, int32_t vh, int32_t kh, int32_t kd,
                   int32_t vd, void *stream);

/*
 * gdn_frontend_m without advancing the history: the M draft rows see the
 * history as gdn_frontend_m would, but hist is only read.  Pair with
 * gdn_commit, which pushes the accepted rows' raw frames into the history.
 */
int gdn_frontend_verify_m(const float *x, const float *Wa, const float *Wb,
                          const float *A_log, const float *dt_bias,
                          const float *xc_raw, const float *hist,
                          const float *conv_w, float *q, float *k, float *v,
                          float *g, float *beta, int32_t B, int32_t M,
                          int32_t dim, int32_t conv_dim, int32_t ck, int32_t vh,
                          int32_t kh, int32_t kd, int32_t vd, void *stream);

/*
 * Measurement aid: stream n_floats floats from src to dst with the same
 * 128-bit non-temporal access pattern as the state stream (the read+write
 * floor against which the step is read).  src == dst is allowed (read and
 * write back in place).  Used by gdn_mark for its copy.
 */
int gdn_stream_copy(float *dst, const float *src, int64_t n_floats, void *stream);

/*
 * Measurement aid: the read-only floor ("Kestrel_VLLM #27", section 3.2: a
 * read-only floor and a read+write floor bracket what a state stream can
 * reach).  Streams n_floats floats of src with 128-bit non-temporal loads and
 * writes words[c] = the XOR of the 32-bit words of floats
 * [32768 c, min(32768 (c + 1), n_floats)) for c < gdn_stream_read_words(n),
 * so that no load can be dropped and the result is checkable.  src, words:
 * device memory (src 16-byte, words 4-byte aligned, not overlapping).
 * n_floats == 0 is a no-op.  Errors: GDN_EINVAL.
 */
int64_t gdn_stream_read_words(int64_t n_floats);   /* < 0: n_floats < 1 */
int gdn_stream_read(const float *src, int64_t n_floats, uint32_t *words, void *stream);

/*
 * Weight packing for gdn_proj: copies a row-major weight matrix W [R][C] into
 * the matrix-core operand order that gdn_proj streams.  Packed slab s of 16
 * rows, 16-column block kb and lane l = 0..63 hold
 *   Wp[((s * (C / 16) + kb) * 64 + l) * 4 + i] = W[16 s + l % 16][16 kb + 4 (l / 16) + i]
 * for i = 0..3 (same size as W; a pure permutation, bit-exact).  Done once
 * per weight matrix, when the weights are loaded.
 *   W, Wp: fp32 device arrays, 16-byte aligned, not overlapping.
 * Errors: GDN_EINVAL for a null or misaligned pointer, R <= 0, C <= 0 or
 * overlapping arrays; GDN_EUNSUPPORTED when C is not a multiple of 128, R not
 * a multiple of 16, C > 2^22 or R * C > 2^40.
 */
int gdn_proj_pack(const float *W, float *Wp, int32_t R, int32_t C, void *stream);

/*
 * Dense projections of the layer: y0[r][o] = sum over c of W0[o][c] * x[r][c]
 * for r < rows, o < R0 and, when W1 is non-null, y1 likewise from W1 [R1][C]
 * in the same launch (the two input projections share x).
 * ("Kestrel_VLLM #24", Fig. 1 caption, steps 1 and 7: in_proj_qkv gives the
 * conv input, in_proj_z the output gate, out_proj maps the gated output back
 * to the model width; "Kestrel_VLLM #34", section 3.6: the projections take
 * all draft rows at once and read the weights once.)
 *   x  [rows][C] row-major; y0 [rows][R0]; y1 [rows][R1];
 *   W0, W1: R x C weights in the packed order of gdn_proj_pack
 *   (fp32 device arrays, 16-byte aligned; W1 == NULL requires R1 == 0 and
 *   y1 == NULL).
 * Each row's result is independent of the other rows in the call and of the
 * row count, bit for bit: one call over M rows equals M one-row calls.  The
 * sum over c runs in a fixed order of fp32 operations (8 equal segments of C,
 * each an ascending chain of matrix-core steps; segments 0..3 folded left to
 * right, so are 4..7, and the two sums added), so it differs from a left
 * fold by rounding only.  Launches of 2 to 16 rows with few output tiles
 * first zero y0 (and y1), then add two partial folds into each element, so
 * y0 and y1 hold intermediate values until the call's work completes on the
 * stream.
 * Ownership: every buffer belongs to the caller; nothing is allocated.
 * Errors: GDN_EINVAL for a null or misaligned pointer, rows < 0, C <= 0,
 * R <= 0, or an output overlapping an input or the other output;
 * GDN_EUNSUPPORTED when C is not a multiple of 128, R not a multiple of 16,
 * C > 2^22, R * C > 2^40, rows > 2^31, or the launch would exceed the grid
 * limit.  rows == 0 is a no-op.
 */
int gdn_proj(const float *x, int64_t rows, int32_t C,
             const float *W0, int32_t R0, float *y0,
             const float *W1, int32_t R1, float *y1, void *stream);

/*
 * Bytes of a 4-bit weight matrix [R][C] packed by gdn_proj_q4_pack: 9 C / 16
 * per row (C / 2 bytes of 4-bit values and C / 32 binary16 scales).
 * Returns -1 when R or C is not positive, R is not a multiple of 64 or C not a
 * multiple of 1024.
 */
int64_t gdn_proj_q4_bytes(int32_t R, int32_t C);

/*
 * Packing of 4-bit weights for gdn_proj_q4 ("Kestrel_VLLM #24", section 8:
 * the large projections read 4-bit weights with f32 activations; section 12:
 * each weight is a signed 4-bit value times a binary16 scale shared by its
 * block; the per-layer weight size fixes a block of 32).  The source format:
 *   q [R][C / 2] bytes, element 2 i of a row in the low nibble of byte i and
 *     element 2 i + 1 in the high nibble, each a two's-complement value -8..7;
 *   scale [R][C / 32] finite binary16 bit patterns, scale b covering elements
 *     32 b .. 32 b + 31 of its row.
 * The packed order, per tile t of 16 rows and chunk m of 256 columns (2304
 * bytes, t-major): 32-bit word 8 (16 d + o) + i holds the biased values
 * u = n + 8 of row 16 t + o, columns 256 m + 32 i + 8 d + k (k = 0..7), value
 * k at bit 4 (k >> 1) + 16 (k & 1); then at offset 2048 + 16 o the 8 scales of
 * row 16 t + o for the chunk's blocks i = 0..7.  No value is rounded: the
 * packing is a re-arrangement plus the fixed offset of 8.
 *   q, scale, Wq: device arrays, 16-byte aligned, Wq of gdn_proj_q4_bytes(R, C)
 *   bytes, not overlapping the sources.
 * Errors: GDN_EINVAL for a null or misaligned pointer, R <= 0, C <= 0 or
 * overlapping arrays; GDN_EUNSUPPORTED when C is not a multiple of 1024, R not
 * a multiple of 64, C > 2^22 or R * C > 2^40.
 */
int gdn_proj_q4_pack(const uint8_t *q, const uint16_t *scale, void *Wq, int32_t R, int32_t C,
                     void *stream);

/*
 * gdn_proj with 4-bit weights packed by gdn_proj_q4_pack, for 1 to 16 rows
 * (the decode and draft-verify sizes): y0[r][o] = sum over c of W0[o][c] *
 * x[r][c], with W0[o][c] = n * s formed exactly in fp32 from the 4-bit value n
 * and its block's scale s, and y1 likewise from Wq1 in the same launch
 * ("Kestrel_VLLM #24", section 8 and Fig. 1 caption, steps 1 and 7).
 * The sum runs in a fixed order: for each row and 256-column chunk, x is
 * scaled by a power of two 2^k (its largest magnitude in [2^14, 2^15)) and
 * split into three binary16 parts x1 = rn(2^k x), x2 = rn(2^k x - x1),
 * x3 = rn(2^k x - x1 - x2), which add up to 2^k x exactly (for elements of at
 * least 2^-15 of the chunk's largest magnitude; smaller ones to within 2^-39
 * of it); the fp16 matrix cores form each 32-column block's sums of n x1,
 * n x2 and n x3 (exact products, fp32 accumulation), their fp32 sum T is
 * scaled by s in one fused multiply-add per block, chained over the chunk's 8
 * blocks from +0 and scaled back by 2^-k; C is cut into 4 quarters whose
 * chunk results are added in order, and y = (q0 + q1) + (q2 + q3).  So the
 * result differs from a left fold of the fp32 products by rounding only; an
 * infinite x makes every output of its row +inf, -inf or NaN, the class the
 * left fold gives (the chunk's scale 2^k then comes from its largest finite
 * magnitude).  A row's result does not depend on the other rows of the
 * call, on their number, or on whether the matrix shares the launch with a
 * second one.
 *   x [rows][C] fp32; y0 [rows][R0], y1 [rows][R1] fp32; Wq0, Wq1 packed
 *   (16-byte aligned; Wq1 == NULL requires R1 == 0 and y1 == NULL).
 * Ownership: every buffer belongs to the caller; nothing is allocated.
 * Errors: GDN_EINVAL for a null or misaligned pointer, rows < 0, C <= 0,
 * R <= 0, or an output overlapping an input or the other output;
 * GDN_EUNSUPPORTED when C is not a multiple of 1024, R not a multiple of 64,
 * C > 2^22, R * C > 2^40 or rows > 16.  rows == 0 is a no-op.
 */
int gdn_proj_q4(const float *x, int64_t rows, int32_t C,
                const void *Wq0, int32_t R0, float *y0,
                const void *Wq1, int32_t R1, float *y1, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
