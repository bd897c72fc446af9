// gdn_api.cpp -- the C ABI declared in include/gdn.h: argument validation on
// the host, launch-shape choice, enqueue on the caller's stream.  Every check
// happens before anything is enqueued, so a refused call changes nothing and
// needs no device (the validation runs on machines without a GPU).
#include "gdn.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "gdn_launch.h"

namespace {

constexpr int32_t kMaxM = 64;
constexpr int32_t kMaxHeads = 4096;
constexpr int32_t kSlabMagic = 0x47444e53;  // "GDNS"
constexpr int64_t kAlign = 256;
constexpr int32_t kConvK = 4;       // conv kernel width the kernels are built for
constexpr int64_t kMaxHistFloats = (int64_t)1 << 24;   // per unit: (ck - 1) x conv_dim

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Pointer p must be non-null and 16-byte aligned.
bool ptr_ok(const void *p) { return p != nullptr && aligned16(p); }

int check_dims(int32_t vh, int32_t kh, int32_t kd, int32_t vd) {
  if (vh <= 0 || kh <= 0 || kd <= 0 || vd <= 0 || vh % kh != 0 || vh > kMaxHeads) return GDN_EINVAL;
  if (kd != vd || (kd != 128 && kd != 64)) return GDN_EUNSUPPORTED;
  return GDN_OK;
}

bool overlaps(const void *a, int64_t abytes, const void *b, int64_t bbytes) {
  if (!a || !b || abytes <= 0 || bbytes <= 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

int64_t align_up(int64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Launch-size limit: the grid of a recurrence launch must stay below 2^32
// work-items.  No geometry gives a tile more lanes than recur_lanes(kd), and
// a history replay appends, per unit, conv_dim / 4 lanes rounded up to a
// workgroup of at most 1024 lanes.
bool grid_fits(int64_t n_units, int32_t vh, int32_t kd, int32_t conv_dim = 0) {
  const int64_t lim = 0xFFFFFFFF;
  if (n_units > lim / vh) return false;
  int64_t items = n_units * vh * gdn::recur_lanes(kd);
  if (conv_dim > 0) items += n_units * ((int64_t)conv_dim / 4 + 1023);
  return items <= lim;
}

int enq(int hip_rc) { return hip_rc == 0 ? GDN_OK : GDN_EDEVICE; }

// Validation shared by gdn_step / gdn_step_m.  rows = M.
int check_step(const float *S, const float *q, const float *k, const float *v, const float *g,
               const float *beta, const float *o, int64_t n_units, int32_t rows, int32_t vh,
               int32_t kh, int32_t kd, int32_t vd) {
  int rc = check_dims(vh, kh, kd, vd);
  if (rc) return rc;
  if (n_units < 0) return GDN_EINVAL;
  if (n_units == 0) return GDN_OK;
  if (!grid_fits(n_units, vh, kd)) return GDN_EUNSUPPORTED;
  if (!ptr_ok(S) || !ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !ptr_ok(o)) return GDN_EINVAL;
  if (g == nullptr || beta == nullptr) return GDN_EINVAL;
  const int64_t sb = n_units * vh * (int64_t)kd * vd * 4;
  const int64_t qkb = (int64_t)rows * n_units * kh * kd * 4;
  const int64_t vb = (int64_t)rows * n_units * vh * vd * 4;
  const int64_t gb = (int64_t)rows * n_units * vh * 4;
  if (overlaps(S, sb, q, qkb) || overlaps(S, sb, k, qkb) || overlaps(S, sb, v, vb) ||
      overlaps(S, sb, o, vb) || overlaps(S, sb, g, gb) || overlaps(S, sb, beta, gb))
    return GDN_EINVAL;
  if (overlaps(o, vb, q, qkb) || overlaps(o, vb, k, qkb) || overlaps(o, vb, v, vb) ||
      overlaps(o, vb, g, gb) || overlaps(o, vb, beta, gb))
    return GDN_EINVAL;
  return GDN_OK;
}

}  // namespace

extern "C" {

const char *gdn_strerror(int rc) {
  switch (rc) {
    case GDN_OK: return "ok";
    case GDN_EINVAL: return "invalid argument (NULL or misaligned pointer, bad size, aliasing, M or accepted out of range)";
    case GDN_EUNSUPPORTED:
      return "unsupported shape (recurrence: kd == vd must be 64 or 128; projection: C a multiple "
             "of 128, R of 16; conv width other than 4; a launch too large; or more than 65536 "
             "units for gdn_rollback_static)";
    case GDN_ESTATE: return "slab state error (not armed, history not marked, too small, or mismatched)";
    case GDN_EDEVICE: return "HIP runtime error while enqueuing";
    default: return "unknown error code";
  }
}

int gdn_step(float *S, const float *q, const float *k, const float *v, const float *g,
             const float *beta, float *o, int64_t n_units, int32_t vh, int32_t kh, int32_t kd,
             int32_t vd, void *stream) {
  int rc = check_step(S, q, k, v, g, beta, o, n_units, 1, vh, kh, kd, vd);
  if (rc || n_units == 0) return rc;
  return enq(gdn::launch_recur(kd, S, S, q, k, v, g, beta, o, nullptr, n_units, vh, kh, 1,
                               (hipStream_t)stream));
}

int gdn_step_m(float *S, const float *q, const float *k, const float *v, const float *g,
               const float *beta, float *o, int64_t n_units, int32_t M, int32_t vh, int32_t kh,
               int32_t kd, int32_t vd, void *stream) {
  if (M < 1 || M > kMaxM) return GDN_EINVAL;
  int rc = check_step(S, q, k, v, g, beta, o, n_units, M, vh, kh, kd, vd);
  if (rc || n_units == 0) return rc;
  return enq(gdn::launch_recur(kd, S, S, q, k, v, g, beta, o, nullptr, n_units, vh, kh, M,
                               (hipStream_t)stream));
}

int gdn_step_gated(float *S, const float *q, const float *k, const float *v, const float *g,
                   const float *beta, const float *z, const float *norm_w, float eps, float *out,
                   int64_t n_units, int32_t M, int32_t vh, int32_t kh, int32_t kd, int32_t vd,
                   void *stream) {
  if (M < 1 || M > kMaxM) return GDN_EINVAL;
  if (!(eps >= 0.0f) || eps > 1.0f) return GDN_EINVAL;   // also refuses NaN
  int rc = check_step(S, q, k, v, g, beta, out, n_units, M, vh, kh, kd, vd);
  if (rc || n_units == 0) return rc;
  if (!ptr_ok(z) || !ptr_ok(norm_w)) return GDN_EINVAL;
  const int64_t sb = n_units * vh * (int64_t)kd * vd * 4;
  const int64_t zb = (int64_t)M * n_units * vh * vd * 4;
  if (overlaps(S, sb, z, zb) || overlaps(out, zb, z, zb) || overlaps(S, sb, norm_w, vd * 4) ||
      overlaps(out, zb, norm_w, vd * 4))
    return GDN_EINVAL;
  return enq(gdn::launch_recur(kd, S, S, q, k, v, g, beta, out, nullptr, n_units, vh, kh, M,
                               (hipStream_t)stream, z, norm_w, eps));
}

int64_t gdn_slab_bytes(int64_t n_units, int32_t vh, int32_t kh, int32_t kd, int32_t vd,
                       int64_t hist_floats_per_unit) {
  int rc = check_dims(vh, kh, kd, vd);
  if (rc) return rc;
  if (n_units < 1 || hist_floats_per_unit < 0 || hist_floats_per_unit % 4 != 0) return GDN_EINVAL;
  // a slab's units are replayed in one recurrence launch, so they obey its
  // grid limit; both bounds also keep the byte counts below far from 2^63
  if (!grid_fits(n_units, vh, kd) || hist_floats_per_unit > kMaxHistFloats)
    return GDN_EUNSUPPORTED;
  const int64_t s_bytes = align_up(n_units * vh * (int64_t)kd * vd * 4);
  const int64_t h_bytes = align_up(n_units * hist_floats_per_unit * 4);
  const int64_t a_bytes = align_up(n_units * 4);
  return s_bytes + h_bytes + a_bytes;
}

int gdn_slab_init(gdn_slab *slab, void *dev, int64_t bytes, int64_t n_units, int32_t vh,
                  int32_t kh, int32_t kd, int32_t vd, int64_t hist_floats_per_unit) {
  if (slab == nullptr || dev == nullptr || (reinterpret_cast<uintptr_t>(dev) % kAlign) != 0)
    return GDN_EINVAL;
  const int64_t need = gdn_slab_bytes(n_units, vh, kh, kd, vd, hist_floats_per_unit);
  if (need < 0) return (int)need;
  if (bytes < need) return GDN_ESTATE;
  memset(slab, 0, sizeof(*slab));
  slab->dev = dev;
  slab->bytes = bytes;
  slab->n_units = n_units;
  slab->hist_floats = hist_floats_per_unit;
  slab->vh = vh;
  slab->kh = kh;
  slab->kd = kd;
  slab->vd = vd;
  slab->armed = 0;
  slab->magic = kSlabMagic;
  return GDN_OK;
}

namespace {

bool slab_valid(const gdn_slab *sl) {
  if (sl == nullptr || sl->magic != kSlabMagic || sl->dev == nullptr) return false;
  const int64_t need = gdn_slab_bytes(sl->n_units, sl->vh, sl->kh, sl->kd, sl->vd, sl->hist_floats);
  return need > 0 && sl->bytes >= need;
}

float *slab_S(const gdn_slab *sl) { return static_cast<float *>(sl->dev); }
float *slab_hist(const gdn_slab *sl) {
  return reinterpret_cast<float *>(static_cast<char *>(sl->dev) +
                                   align_up(sl->n_units * sl->vh * (int64_t)sl->kd * sl->vd * 4));
}
int32_t *slab_accepted(const gdn_slab *sl) {
  return reinterpret_cast<int32_t *>(reinterpret_cast<char *>(slab_hist(sl)) +
                                     align_up(sl->n_units * sl->hist_floats * 4));
}

}  // namespace

int gdn_mark(gdn_slab *slab, const float *S, const float *hist, void *stream) {
  if (!slab_valid(slab)) return GDN_ESTATE;
  if (!ptr_ok(S) || (hist != nullptr && !aligned16(hist))) return GDN_EINVAL;
  if (hist != nullptr && slab->hist_floats == 0) return GDN_ESTATE;
  const int64_t ns = slab->n_units * slab->vh * (int64_t)slab->kd * slab->vd;
  const int64_t nh = slab->n_units * slab->hist_floats;
  if (overlaps(S, ns * 4, slab->dev, slab->bytes) ||
      (hist && overlaps(hist, nh * 4, slab->dev, slab->bytes)))
    return GDN_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  int rc = enq(gdn::launch_copy(slab_S(slab), S, ns, s));
  if (rc) return rc;
  if (hist != nullptr) {
    rc = enq(gdn::launch_copy(slab_hist(slab), hist, nh, s));
    if (rc) return rc;
  }
  slab->armed = 1 | (hist != nullptr ? 2 : 0);
  return GDN_OK;
}

int gdn_mark_step_m(gdn_slab *slab, float *S, const float *hist, const float *q, const float *k,
                    const float *v, const float *g, const float *beta, float *o, int64_t n_units,
                    int32_t M, int32_t vh, int32_t kh, int32_t kd, int32_t vd, void *stream) {
  if (!slab_valid(slab)) return GDN_ESTATE;
  if (n_units != slab->n_units || vh != slab->vh || kh != slab->kh || kd != slab->kd ||
      vd != slab->vd)
    return GDN_ESTATE;
  if (M < 1 || M > kMaxM) return GDN_EINVAL;
  int rc = check_step(S, q, k, v, g, beta, o, n_units, M, vh, kh, kd, vd);
  if (rc) return rc;
  if (hist != nullptr && !aligned16(hist)) return GDN_EINVAL;
  if (hist != nullptr && slab->hist_floats == 0) return GDN_ESTATE;
  const int64_t ns = slab->n_units * slab->vh * (int64_t)slab->kd * slab->vd;
  const int64_t nh = slab->n_units * slab->hist_floats;
  const int64_t qkb = (int64_t)M * n_units * kh * kd * 4, vb = (int64_t)M * n_units * vh * vd * 4,
                gb = (int64_t)M * n_units * vh * 4;
  const void *ins[6] = {q, k, v, g, beta, o};
  const int64_t ib[6] = {qkb, qkb, vb, gb, gb, vb};
  if (overlaps(S, ns * 4, slab->dev, slab->bytes) ||
      (hist && overlaps(hist, nh * 4, slab->dev, slab->bytes)))
    return GDN_EINVAL;
  for (int i = 0; i < 6; i++)
    if (overlaps(ins[i], ib[i], slab->dev, slab->bytes)) return GDN_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  if (hist != nullptr) {
    rc = enq(gdn::launch_copy(slab_hist(slab), hist, nh, s));
    if (rc) return rc;
  }
  rc = enq(gdn::launch_recur(kd, S, S, q, k, v, g, beta, o, nullptr, n_units, vh, kh, M, s,
                             nullptr, nullptr, 0.0f, slab_S(slab)));
  if (rc) return rc;
  slab->armed = 1 | (hist != nullptr ? 2 : 0);
  return GDN_OK;
}

namespace {

// gdn_rollback with the per-unit counts staged in `counts` (device, N int32):
// the slab's count area, or the library's static one (counts == nullptr:
// looked up after validation).
int rollback_impl(gdn_slab *slab, float *S, float *hist, const float *q, const float *k,
                  const float *v, const float *g, const float *beta, const float *xc_raw,
                  int32_t conv_dim, int32_t ck, int32_t M, const int32_t *accepted,
                  bool static_counts, void *stream) {
  if (!slab_valid(slab)) return GDN_ESTATE;
  if (!(slab->armed & 1)) return GDN_ESTATE;
  if (hist != nullptr && !(slab->armed & 2)) return GDN_ESTATE;
  if (M < 1 || M > kMaxM || accepted == nullptr || !ptr_ok(S)) return GDN_EINVAL;
  const int64_t N = slab->n_units;
  bool any = false;
  for (int64_t u = 0; u < N; u++) {
    if (accepted[u] < 0 || accepted[u] > M) return GDN_EINVAL;
    any |= accepted[u] > 0;
  }
  const int vh = slab->vh, kh = slab->kh, kd = slab->kd, vd = slab->vd;
  const int64_t ns = N * vh * (int64_t)kd * vd;
  if (overlaps(S, ns * 4, slab->dev, slab->bytes)) return GDN_EINVAL;
  if (any) {
    if (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || g == nullptr || beta == nullptr)
      return GDN_EINVAL;
    const int64_t qkb = (int64_t)M * N * kh * kd * 4, vb = (int64_t)M * N * vh * vd * 4,
                  gb = (int64_t)M * N * vh * 4;
    if (overlaps(S, ns * 4, q, qkb) || overlaps(S, ns * 4, k, qkb) || overlaps(S, ns * 4, v, vb) ||
        overlaps(S, ns * 4, g, gb) || overlaps(S, ns * 4, beta, gb))
      return GDN_EINVAL;
  }
  if (hist != nullptr) {
    if (ck != kConvK) return GDN_EUNSUPPORTED;
    if (!aligned16(hist) || conv_dim <= 0 || conv_dim % 4 != 0 ||
        (int64_t)(ck - 1) * conv_dim != slab->hist_floats)
      return GDN_EINVAL;
    if (overlaps(hist, N * slab->hist_floats * 4, slab->dev, slab->bytes)) return GDN_EINVAL;
    if (any && !ptr_ok(xc_raw)) return GDN_EINVAL;
  }
  if (!grid_fits(N, vh, kd, hist != nullptr ? conv_dim : 0)) return GDN_EUNSUPPORTED;
  if (static_counts && N > gdn::kStaticCountsMax) return GDN_EUNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  // accepted[] reaches the count area through kernel arguments, so the host
  // array is consumed before return and the counts are ordered on the stream
  // before the kernels that read them.
  int32_t *d_acc = slab_accepted(slab);
  if (static_counts && gdn::static_counts_area(&d_acc) != 0) return GDN_EDEVICE;
  int rc0 = enq(gdn::launch_stage_counts(d_acc, accepted, N, s));
  if (rc0) return rc0;
  // the history replay runs in the same launch as the state replay
  int rc = enq(gdn::launch_recur(kd, slab_S(slab), S, q, k, v, g, beta, nullptr, d_acc, N, vh, kh,
                                 M, s, nullptr, nullptr, 0.0f, nullptr, nullptr, hist,
                                 slab_hist(slab), xc_raw, conv_dim));
  if (rc) return rc;
  slab->armed = 0;
  return GDN_OK;
}

}  // namespace

int gdn_rollback(gdn_slab *slab, float *S, float *hist, const float *q, const float *k,
                 const float *v, const float *g, const float *beta, const float *xc_raw,
                 int32_t conv_dim, int32_t ck, int32_t M, const int32_t *accepted,
                 void *stream) {
  return rollback_impl(slab, S, hist, q, k, v, g, beta, xc_raw, conv_dim, ck, M, accepted,
                       false, stream);
}

int gdn_rollback_static(gdn_slab *slab, float *S, float *hist, const float *q, const float *k,
                        const float *v, const float *g, const float *beta, const float *xc_raw,
                        int32_t conv_dim, int32_t ck, int32_t M, const int32_t *accepted,
                        void *stream) {
  return rollback_impl(slab, S, hist, q, k, v, g, beta, xc_raw, conv_dim, ck, M, accepted,
                       true, stream);
}

namespace {

int frontend_impl(const float *x, const float *Wa, const float *Wb, const float *A_log,
                  const float *dt_bias, const float *xc_raw, float *hist, const float *conv_w,
                  float *q, float *k, float *v, float *g, float *beta, int32_t B, int32_t M,
                  int32_t dim, int32_t conv_dim, int32_t ck, int32_t vh, int32_t kh, int32_t kd,
                  int32_t vd, bool write_hist, void *stream) {
  int rc = check_dims(vh, kh, kd, vd);
  if (rc) return rc;
  if (ck != kConvK) return GDN_EUNSUPPORTED;
  if (B < 0 || M < 1 || M > kMaxM || dim <= 0 || dim % 4 != 0 ||
      conv_dim != 2 * kh * kd + vh * vd)
    return GDN_EINVAL;
  if (B == 0) return GDN_OK;
  if (gdn::frontend_workitems(B, M, conv_dim, vh) > (int64_t)0xFFFFFFFF) return GDN_EUNSUPPORTED;
  if (!ptr_ok(x) || !ptr_ok(Wa) || !ptr_ok(Wb) || !A_log || !dt_bias || !ptr_ok(xc_raw) ||
      !ptr_ok(hist) || !ptr_ok(conv_w) || !ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !g || !beta)
    return GDN_EINVAL;
  const int64_t rows = (int64_t)M * B;
  const int64_t hb = (int64_t)B * (ck - 1) * conv_dim * 4;
  const int64_t rawb = rows * conv_dim * 4, xb = rows * dim * 4;
  const int64_t qkb = rows * kh * kd * 4, vb = rows * vh * vd * 4, gb = rows * vh * 4;
  const void *outs[5] = {q, k, v, g, beta};
  const int64_t ob[5] = {qkb, qkb, vb, gb, gb};
  const int64_t wb = (int64_t)vh * dim * 4, cwb = (int64_t)conv_dim * ck * 4, hb1 = vh * 4;
  const void *ins[7] = {x, xc_raw, Wa, Wb, conv_w, A_log, dt_bias};
  const int64_t ib[7] = {xb, rawb, wb, wb, cwb, hb1, hb1};
  for (int i = 0; i < 5; i++) {
    if (overlaps(outs[i], ob[i], hist, hb)) return GDN_EINVAL;
    for (int j = 0; j < 7; j++)
      if (overlaps(outs[i], ob[i], ins[j], ib[j])) return GDN_EINVAL;
    for (int j = i + 1; j < 5; j++)
      if (overlaps(outs[i], ob[i], outs[j], ob[j])) return GDN_EINVAL;
  }
  for (int j = 0; j < 7; j++)
    if (overlaps(hist, hb, ins[j], ib[j])) return GDN_EINVAL;
  return enq(gdn::launch_frontend(x, Wa, Wb, A_log, dt_bias, xc_raw, hist, conv_w, q, k, v, g,
                                  beta, B, M, dim, conv_dim, vh, kh, kd, write_hist,
                                  (hipStream_t)stream));
}

}  // namespace

int gdn_frontend(const float *x, const float *Wa, const float *Wb, const float *A_log,
                 const float *dt_bias, const float *xc_raw, float *hist, const float *conv_w,
                 float *q, float *k, float *v, float *g, float *beta, int32_t B, int32_t dim,
                 int32_t conv_dim, int32_t ck, int32_t vh, int32_t kh, int32_t kd, int32_t vd,
                 void *stream) {
  return frontend_impl(x, Wa, Wb, A_log, dt_bias, xc_raw, hist, conv_w, q, k, v, g, beta, B, 1,
                       dim, conv_dim, ck, vh, kh, kd, vd, true, stream);
}

int gdn_frontend_m(const float *x, const float *Wa, const float *Wb, const float *A_log,
                   const float *dt_bias, const float *xc_raw, float *hist, const float *conv_w,
                   float *q, float *k, float *v, float *g, float *beta, int32_t B, int32_t M,
                   int32_t dim, int32_t conv_dim, int32_t ck, int32_t vh, int32_t kh, int32_t kd,
                   int32_t vd, void *stream) {
  return frontend_impl(x, Wa, Wb, A_log, dt_bias, xc_raw, hist, conv_w, q, k, v, g, beta, B, M,
                       dim, conv_dim, ck, vh, kh, kd, vd, true, stream);
}

int gdn_frontend_verify_m(const float *x, const float *Wa, const float *Wb, const float *A_log,
                          const float *dt_bias, const float *xc_raw, const float *hist,
                          const float *conv_w, float *q, float *k, float *v, float *g,
                          float *beta, int32_t B, int32_t M, int32_t dim, int32_t conv_dim,
                          int32_t ck, int32_t vh, int32_t kh, int32_t kd, int32_t vd,
                          void *stream) {
  return frontend_impl(x, Wa, Wb, A_log, dt_bias, xc_raw, const_cast<float *>(hist), conv_w, q,
                       k, v, g, beta, B, M, dim, conv_dim, ck, vh, kh, kd, vd, false, stream);
}

int gdn_verify_m(const float *S, const float *q, const float *k, const float *v, const float *g,
                 const float *beta, float *o, int64_t n_units, int32_t M, int32_t vh, int32_t kh,
                 int32_t kd, int32_t vd, void *stream) {
  if (M < 1 || M > kMaxM) return GDN_EINVAL;
  int rc = check_step(S, q, k, v, g, beta, o, n_units, M, vh, kh, kd, vd);
  if (rc || n_units == 0) return rc;
  return enq(gdn::launch_recur(kd, S, nullptr, q, k, v, g, beta, o, nullptr, n_units, vh, kh, M,
                               (hipStream_t)stream));
}

int gdn_verify_m_gated(const float *S, const float *q, const float *k, const float *v,
                       const float *g, const float *beta, const float *z, const float *norm_w,
                       float eps, float *out, int64_t n_units, int32_t M, int32_t vh,
                       int32_t kh, int32_t kd, int32_t vd, void *stream) {
  if (M < 1 || M > kMaxM) return GDN_EINVAL;
  if (!(eps >= 0.0f) || eps > 1.0f) return GDN_EINVAL;   // also refuses NaN
  int rc = check_step(S, q, k, v, g, beta, out, n_units, M, vh, kh, kd, vd);
  if (rc || n_units == 0) return rc;
  if (!ptr_ok(z) || !ptr_ok(norm_w)) return GDN_EINVAL;
  const int64_t sb = n_units * vh * (int64_t)kd * vd * 4;
  const int64_t zb = (int64_t)M * n_units * vh * vd * 4;
  if (overlaps(out, zb, z, zb) || overlaps(out, zb, norm_w, vd * 4) || overlaps(S, sb, out, zb))
    return GDN_EINVAL;
  return enq(gdn::launch_recur(kd, S, nullptr, q, k, v, g, beta, out, nullptr, n_units, vh, kh,
                               M, (hipStream_t)stream, z, norm_w, eps));
}

}  // extern "C"

namespace {

// The arguments of gdn_commit (also the first half of gdn_commit_verify_m).
// n_units == 0 passes; the caller then launches nothing.
int check_commit(const float *S, const float *hist, const float *q, const float *k,
                 const float *v, const float *g, const float *beta, const float *xc_raw,
                 int32_t conv_dim, int32_t ck, int64_t n_units, int32_t M, int32_t vh,
                 int32_t kh, int32_t kd, int32_t vd, const int32_t *accepted,
                 const int32_t *status) {
  if (M < 1 || M > kMaxM) return GDN_EINVAL;
  int rc = check_dims(vh, kh, kd, vd);
  if (rc) return rc;
  if (n_units < 0) return GDN_EINVAL;
  if (n_units == 0) return GDN_OK;
  if (!grid_fits(n_units, vh, kd)) return GDN_EUNSUPPORTED;
  const uintptr_t amask = 3u;
  if (accepted == nullptr || (reinterpret_cast<uintptr_t>(accepted) & amask) ||
      (status != nullptr && (reinterpret_cast<uintptr_t>(status) & amask)))
    return GDN_EINVAL;
  if (!ptr_ok(S) || !ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || g == nullptr || beta == nullptr)
    return GDN_EINVAL;
  const int64_t sb = n_units * vh * (int64_t)kd * vd * 4;
  const int64_t qkb = (int64_t)M * n_units * kh * kd * 4, vb = (int64_t)M * n_units * vh * vd * 4,
                gb = (int64_t)M * n_units * vh * 4;
  const void *ins[6] = {q, k, v, g, beta, accepted};
  const int64_t ib[6] = {qkb, qkb, vb, gb, gb, n_units * 4};
  for (int i = 0; i < 6; i++)
    if (overlaps(S, sb, ins[i], ib[i])) return GDN_EINVAL;
  if (status != nullptr && overlaps(S, sb, status, 4)) return GDN_EINVAL;
  if (hist != nullptr && ck != kConvK) return GDN_EUNSUPPORTED;
  const int64_t hb = n_units * (kConvK - 1) * (int64_t)conv_dim * 4;
  if (hist != nullptr) {
    if (!aligned16(hist) || !ptr_ok(xc_raw) || conv_dim <= 0 || conv_dim % 4 != 0)
      return GDN_EINVAL;
    if (!grid_fits(n_units, vh, kd, conv_dim)) return GDN_EUNSUPPORTED;
    if (overlaps(hist, hb, S, sb) || overlaps(hist, hb, xc_raw, (int64_t)M * n_units * conv_dim * 4))
      return GDN_EINVAL;
    for (int i = 0; i < 6; i++)
      if (overlaps(hist, hb, ins[i], ib[i])) return GDN_EINVAL;
    if (status != nullptr && overlaps(status, 4, hist, hb)) return GDN_EINVAL;
  }
  if (status != nullptr && overlaps(status, 4, accepted, n_units * 4)) return GDN_EINVAL;
  return GDN_OK;
}

}  // namespace

extern "C" {

int gdn_commit(float *S, float *hist, const float *q, const float *k, const float *v,
               const float *g, const float *beta, const float *xc_raw, int32_t conv_dim,
               int32_t ck, int64_t n_units, int32_t M, int32_t vh, int32_t kh, int32_t kd,
               int32_t vd, const int32_t *accepted, int32_t *status, void *stream) {
  const int rc = check_commit(S, hist, q, k, v, g, beta, xc_raw, conv_dim, ck, n_units, M, vh, kh,
                              kd, vd, accepted, status);
  if (rc || n_units == 0) return rc;
  hipStream_t s = (hipStream_t)stream;
  // the history replay runs in the same launch as the state replay
  return enq(gdn::launch_recur(kd, S, S, q, k, v, g, beta, nullptr, accepted, n_units, vh, kh, M, s,
                               nullptr, nullptr, 0.0f, nullptr, status, hist, hist, xc_raw,
                               conv_dim));
}

int gdn_commit_verify_m(float *S, float *hist, const float *q, const float *k, const float *v,
                        const float *g, const float *beta, const float *xc_raw, int32_t conv_dim,
                        int32_t ck, int64_t n_units, int32_t M, const int32_t *accepted,
                        int32_t *status, const float *q2, const float *k2, const float *v2,
                        const float *g2, const float *beta2, float *o, int32_t M2, int32_t vh,
                        int32_t kh, int32_t kd, int32_t vd, void *stream) {
  int rc = check_commit(S, hist, q, k, v, g, beta, xc_raw, conv_dim, ck, n_units, M, vh, kh, kd,
                        vd, accepted, status);
  if (rc) return rc;
  if (M2 < 1 || M2 > kMaxM) return GDN_EINVAL;
  rc = check_step(S, q2, k2, v2, g2, beta2, o, n_units, M2, vh, kh, kd, vd);
  if (rc || n_units == 0) return rc;
  // the verify's outputs against everything else the call reads or writes,
  // and the written history against the verify's rows
  const int64_t qkb = (int64_t)M * n_units * kh * kd * 4, vb = (int64_t)M * n_units * vh * vd * 4,
                gb = (int64_t)M * n_units * vh * 4;
  const int64_t qkb2 = (int64_t)M2 * n_units * kh * kd * 4,
                vb2 = (int64_t)M2 * n_units * vh * vd * 4, gb2 = (int64_t)M2 * n_units * vh * 4;
  const int64_t hb = n_units * (kConvK - 1) * (int64_t)conv_dim * 4;
  const void *first[7] = {q, k, v, g, beta, accepted, hist ? xc_raw : nullptr};
  const int64_t fb[7] = {qkb, qkb, vb, gb, gb, n_units * 4, (int64_t)M * n_units * conv_dim * 4};
  for (int i = 0; i < 7; i++)
    if (overlaps(o, vb2, first[i], fb[i])) return GDN_EINVAL;
  if (status != nullptr && overlaps(o, vb2, status, 4)) return GDN_EINVAL;
  if (hist != nullptr) {
    const void *second[6] = {q2, k2, v2, g2, beta2, o};
    const int64_t sb2[6] = {qkb2, qkb2, vb2, gb2, gb2, vb2};
    for (int i = 0; i < 6; i++)
      if (overlaps(hist, hb, second[i], sb2[i])) return GDN_EINVAL;
  }
  return enq(gdn::launch_commit_verify(kd, S, q, k, v, g, beta, accepted, status, hist, xc_raw,
                                       conv_dim, n_units, vh, kh, M, q2, k2, v2, g2, beta2, o, M2,
                                       (hipStream_t)stream));
}

int gdn_stream_copy(float *dst, const float *src, int64_t n_floats, void *stream) {
  if (n_floats < 0) return GDN_EINVAL;
  if (n_floats == 0) return GDN_OK;
  if (!ptr_ok(dst) || !ptr_ok(src)) return GDN_EINVAL;
  if (dst != src && overlaps(dst, n_floats * 4, src, n_floats * 4)) return GDN_EINVAL;
  return enq(gdn::launch_copy(dst, src, n_floats, (hipStream_t)stream));
}

int64_t gdn_stream_read_words(int64_t n_floats) {
  if (n_floats < 1) return GDN_EINVAL;
  return gdn::read_chunks(n_floats);
}

int gdn_stream_read(const float *src, int64_t n_floats, uint32_t *words, void *stream) {
  if (n_floats < 0) return GDN_EINVAL;
  if (n_floats == 0) return GDN_OK;
  if (!ptr_ok(src) || words == nullptr || (reinterpret_cast<uintptr_t>(words) & 3u))
    return GDN_EINVAL;
  if (overlaps(src, n_floats * 4, words, gdn::read_chunks(n_floats) * 4)) return GDN_EINVAL;
  return enq(gdn::launch_read(src, n_floats, words, (hipStream_t)stream));
}

// Projection size limits: a workgroup addresses its (at most 64) packed
// weight rows with 32-bit byte offsets (64 * C * 4 < 2^31), and the packing
// grid (R * C / 4 lanes) stays below 2^32.
constexpr int32_t kProjMaxC = 1 << 22;
constexpr int64_t kProjMaxRC = (int64_t)1 << 40;
constexpr int64_t kProjMaxRows = (int64_t)1 << 31;
constexpr int64_t kProjQ4MaxRows = 16;   // the 4-bit path: one row block (decode, verify)

int gdn_proj_pack(const float *W, float *Wp, int32_t R, int32_t C, void *stream) {
  if (R <= 0 || C <= 0) return GDN_EINVAL;
  if (C % 128 != 0 || R % 16 != 0) return GDN_EUNSUPPORTED;
  if (C > kProjMaxC || (int64_t)R * C > kProjMaxRC) return GDN_EUNSUPPORTED;
  if (!ptr_ok(W) || !ptr_ok(Wp)) return GDN_EINVAL;
  const int64_t wb = (int64_t)R * C * 4;
  if (overlaps(W, wb, Wp, wb)) return GDN_EINVAL;
  return enq(gdn::launch_proj_pack(W, Wp, R, C, (hipStream_t)stream));
}

int gdn_proj(const float *x, int64_t rows, int32_t C, const float *W0, int32_t R0, float *y0,
             const float *W1, int32_t R1, float *y1, void *stream) {
  if (rows < 0 || C <= 0 || R0 <= 0) return GDN_EINVAL;
  if (W1 == nullptr) {
    if (R1 != 0 || y1 != nullptr) return GDN_EINVAL;
  } else if (R1 <= 0) {
    return GDN_EINVAL;
  }
  if (C % 128 != 0 || R0 % 16 != 0 || (W1 != nullptr && R1 % 16 != 0)) return GDN_EUNSUPPORTED;
  if (C > kProjMaxC || rows > kProjMaxRows || (int64_t)R0 * C > kProjMaxRC ||
      (int64_t)R1 * C > kProjMaxRC)
    return GDN_EUNSUPPORTED;
  if (rows == 0) return GDN_OK;
  if (!ptr_ok(x) || !ptr_ok(W0) || !ptr_ok(y0)) return GDN_EINVAL;
  if (W1 != nullptr && (!ptr_ok(W1) || !ptr_ok(y1))) return GDN_EINVAL;
  if (gdn::proj_workgroups(rows, R0, R1) > (int64_t)0xFFFFFFFF / 512) return GDN_EUNSUPPORTED;
  const int64_t xb = rows * C * 4, w0b = (int64_t)R0 * C * 4, y0b = rows * R0 * 4;
  const int64_t w1b = (int64_t)R1 * C * 4, y1b = rows * R1 * 4;
  if (overlaps(y0, y0b, x, xb) || overlaps(y0, y0b, W0, w0b) || overlaps(y0, y0b, W1, w1b))
    return GDN_EINVAL;
  if (W1 != nullptr && (overlaps(y1, y1b, x, xb) || overlaps(y1, y1b, W0, w0b) ||
                        overlaps(y1, y1b, W1, w1b) || overlaps(y1, y1b, y0, y0b)))
    return GDN_EINVAL;
  return enq(gdn::launch_proj(x, rows, C, W0, R0, y0, W1, R1, y1, (hipStream_t)stream));
}

int64_t gdn_proj_q4_bytes(int32_t R, int32_t C) {
  if (R <= 0 || C <= 0 || R % 64 != 0 || C % 1024 != 0) return -1;
  return (int64_t)R * C / 16 * 9;
}

int gdn_proj_q4_pack(const uint8_t *q, const uint16_t *scale, void *Wq, int32_t R, int32_t C,
                     void *stream) {
  if (R <= 0 || C <= 0) return GDN_EINVAL;
  if (C % 1024 != 0 || R % 64 != 0) return GDN_EUNSUPPORTED;
  if (C > kProjMaxC || (int64_t)R * C > kProjMaxRC) return GDN_EUNSUPPORTED;
  if (!ptr_ok(q) || !ptr_ok(scale) || !ptr_ok(Wq)) return GDN_EINVAL;
  const int64_t qb = (int64_t)R * C / 2, sb = (int64_t)R * C / 16, wb = qb + sb;
  if (overlaps(q, qb, Wq, wb) || overlaps(scale, sb, Wq, wb)) return GDN_EINVAL;
  return enq(gdn::launch_proj_q4_pack(q, scale, Wq, R, C, (hipStream_t)stream));
}

int gdn_proj_q4(const float *x, int64_t rows, int32_t C, const void *Wq0, int32_t R0, float *y0,
                const void *Wq1, int32_t R1, float *y1, void *stream) {
  if (rows < 0 || C <= 0 || R0 <= 0) return GDN_EINVAL;
  if (Wq1 == nullptr) {
    if (R1 != 0 || y1 != nullptr) return GDN_EINVAL;
  } else if (R1 <= 0) {
    return GDN_EINVAL;
  }
  if (C % 1024 != 0 || R0 % 64 != 0 || (Wq1 != nullptr && R1 % 64 != 0)) return GDN_EUNSUPPORTED;
  if (C > kProjMaxC || rows > kProjQ4MaxRows || (int64_t)R0 * C > kProjMaxRC ||
      (int64_t)R1 * C > kProjMaxRC)
    return GDN_EUNSUPPORTED;
  if (rows == 0) return GDN_OK;
  if (!ptr_ok(x) || !ptr_ok(Wq0) || !ptr_ok(y0)) return GDN_EINVAL;
  if (Wq1 != nullptr && (!ptr_ok(Wq1) || !ptr_ok(y1))) return GDN_EINVAL;
  const int64_t xb = rows * C * 4, w0b = (int64_t)R0 * C / 16 * 9, y0b = rows * R0 * 4;
  const int64_t w1b = (int64_t)R1 * C / 16 * 9, y1b = rows * R1 * 4;
  if (overlaps(y0, y0b, x, xb) || overlaps(y0, y0b, Wq0, w0b) || overlaps(y0, y0b, Wq1, w1b))
    return GDN_EINVAL;
  if (Wq1 != nullptr && (overlaps(y1, y1b, x, xb) || overlaps(y1, y1b, Wq0, w0b) ||
                         overlaps(y1, y1b, Wq1, w1b) || overlaps(y1, y1b, y0, y0b)))
    return GDN_EINVAL;
  return enq(gdn::launch_proj_q4(x, rows, C, Wq0, R0, y0, Wq1, R1, y1, (hipStream_t)stream));
}

}  // extern "C"
