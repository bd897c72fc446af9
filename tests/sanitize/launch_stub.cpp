// Test-only stand-ins for the launchers of gdn_launch.h, linked with
// gdn_api.cpp into a host-only library built with AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_sanitized_builds.py).  Every
// launcher only counts its call and reports success; nothing touches the
// pointers it receives.  The sizing helpers return what the library's own
// ones return for the same shapes (the grid-size refusals depend on them).
#include <stdint.h>

#include "gdn_launch.h"

namespace {
int64_t g_launches = 0;
int32_t g_counts[gdn::kStaticCountsMax];
int launched() {
  ++g_launches;
  return 0;
}
}  // namespace

extern "C" int64_t gdn_stub_launches() { return g_launches; }

namespace gdn {

int recur_lanes(int kd) { return kd == 128 ? 1024 : 256; }

int launch_recur(int, const float *, float *, const float *, const float *, const float *,
                 const float *, const float *, float *, const int32_t *, int64_t, int, int, int,
                 hipStream_t, const float *, const float *, float, float *, int32_t *, float *,
                 const float *, const float *, int) {
  return launched();
}

int launch_commit_verify(int, float *, const float *, const float *, const float *,
                         const float *, const float *, const int32_t *, int32_t *, float *,
                         const float *, int, int64_t, int, int, int, const float *,
                         const float *, const float *, const float *, const float *, float *,
                         int, hipStream_t) {
  return launched();
}

int launch_copy(float *, const float *, int64_t, hipStream_t) { return launched(); }

int64_t read_chunks(int64_t n) {
  const int64_t c = (n + 32767) / 32768;
  return c < 1 ? 1 : c;
}

int launch_read(const float *, int64_t, uint32_t *, hipStream_t) { return launched(); }

int launch_stage_counts(int32_t *, const int32_t *host, int64_t n, hipStream_t) {
  int64_t sum = 0;   // reads the whole host array, as the real launcher does
  for (int64_t i = 0; i < n; i++) sum += host[i];
  (void)sum;
  return launched();
}

int static_counts_area(int32_t **area) {
  *area = g_counts;
  return 0;
}

int launch_hist_replay(float *, const float *, const float *, const int32_t *, int64_t, int, int,
                       int32_t *, hipStream_t) {
  return launched();
}

int64_t frontend_workitems(int64_t B, int64_t M, int64_t conv_dim, int64_t vh) {
  const int64_t n_gemv = M * B <= 8 ? 2 * vh : ((M * B + 7) / 8) * ((2 * vh + 3) / 4);
  const int64_t n_conv = M >= 2 && B <= 8 ? ((conv_dim + 255) / 256) * B
                                          : ((conv_dim + 1023) / 1024) * ((B + 1) / 2);
  return (n_gemv + n_conv) * 512;
}

int launch_frontend(const float *, const float *, const float *, const float *, const float *,
                    const float *, float *, const float *, float *, float *, float *, float *,
                    float *, int, int, int, int, int, int, int, bool, hipStream_t) {
  return launched();
}

int launch_proj_pack(const float *, float *, int, int, hipStream_t) { return launched(); }

int launch_proj_q4_pack(const uint8_t *, const uint16_t *, void *, int, int, hipStream_t) {
  return launched();
}

int launch_proj_q4(const float *, int64_t, int, const void *, int, float *, const void *, int,
                   float *, hipStream_t) {
  return launched();
}

int64_t proj_workgroups(int64_t rows, int R0, int R1) {
  // an upper bound of the library's tile count (its smallest tiles: 16 rows
  // x 16 outputs), so a call refused there is refused here too
  return ((int64_t)R0 / 16 + (int64_t)R1 / 16) * ((rows + 15) / 16);
}

int launch_proj(const float *, int64_t, int, const float *, int, float *, const float *, int,
                float *, hipStream_t) {
  return launched();
}

}  // namespace gdn
