// gdn_launch.h -- internal launchers of the gfx950 kernels (not part of the
// C ABI).  Every launcher assumes its arguments were validated by the caller
// in gdn_api.cpp and returns a hipError_t cast to int (0 = enqueued).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// Lanes per workgroup of the recurrence kernel for a square head of size kd.
int recur_lanes(int kd);

// Recurrence over tiles (unit, value head).  Reads the state from S_src,
// writes it to S_dst (may equal S_src).  Runs `M` steps per unit, or
// steps[u] steps when `steps` (device int32 [n_units]) is non-null.  Inputs
// are [rows][n_units][...]; o (nullable) is [rows][n_units][vh][kd].  With a
// non-null z ([rows][n_units][vh][kd]) the output goes through the gated
// RMSNorm with weight norm_w [kd] and eps.  With a non-null snap (same
// layout as the state) every tile is also written there as loaded, before
// its first step (a mark fused into the step).  A null S_dst computes the
// outputs only and leaves the state untouched.  Step counts read from
// `steps` outside 0..M run no step for that unit and set *status = 1
// (status nullable); with S_src == S_dst such a unit is left as it was.
int launch_recur(int kd, const float *S_src, float *S_dst, const float *q,
                 const float *k, const float *v, const float *g,
                 const float *beta, float *o, const int32_t *steps,
                 int64_t n_units, int vh, int kh, int M, hipStream_t s,
                 const float *z = nullptr, const float *norm_w = nullptr, float eps = 0.0f,
                 float *snap = nullptr, int32_t *status = nullptr, float *hist = nullptr,
                 const float *hist_src = nullptr, const float *xc_raw = nullptr,
                 int conv_dim = 0);

// gdn_commit then gdn_verify_m (ungated) in one pass over the state.
int launch_commit_verify(int kd, float *S, const float *q, const float *k, const float *v,
                         const float *g, const float *beta, const int32_t *steps,
                         int32_t *status, float *hist, const float *xc_raw, int conv_dim,
                         int64_t n_units, int vh, int kh, int M, const float *q2,
                         const float *k2, const float *v2, const float *g2,
                         const float *beta2, float *o2, int M2, hipStream_t s);

// 128-bit streaming copy of n floats (src == dst allowed).
int launch_copy(float *dst, const float *src, int64_t n, hipStream_t s);

// Read-only stream of n floats; words[c] = XOR of the 32-bit words of chunk
// c (read_chunks(n) chunks of 128 KiB, the last one ragged).
int64_t read_chunks(int64_t n);
int launch_read(const float *src, int64_t n, uint32_t *words, hipStream_t s);

// dst[u] = host[u] for u < n (each 0..255), through kernel arguments: the host
// array is not read after the call returns.
int launch_stage_counts(int32_t *dst, const int32_t *host, int64_t n, hipStream_t s);

// Units whose counts the library-owned count area holds (256 KiB).
constexpr int64_t kStaticCountsMax = 1 << 16;

// Device address of the library-owned count area of kStaticCountsMax int32
// on the current device (looked up once per device, then cached); 0 on
// success, else a HIP error code or -1.
int static_counts_area(int32_t **area);

// Conv-history replay (ck = 4): hist[u] = last 3 frames of
// [src[u] frames..., xc_raw[0][u], ..., xc_raw[a-1][u]], a = accepted[u];
// src may be hist itself.  a outside 0..M: the unit gets a = 0 and *status
// is set to 1 (status nullable).
int launch_hist_replay(float *hist, const float *src, const float *xc_raw,
                       const int32_t *accepted, int64_t n_units, int conv_dim, int M,
                       int32_t *status, hipStream_t s);

// Front end for M rows of B units: paired GEMV + gate/beta over all M*B
// rows, and conv + SiLU + history + split + per key-head norm with the
// history advancing one frame per row.  x [M][B][dim], xc_raw [M][B][...],
// outputs [M][B][...].
// Work-items the front-end launch needs (its grid must stay below 2^32).
int64_t frontend_workitems(int64_t B, int64_t M, int64_t conv_dim, int64_t vh);

int launch_frontend(const float *x, const float *Wa, const float *Wb,
                    const float *A_log, const float *dt_bias,
                    const float *xc_raw, float *hist, const float *conv_w,
                    float *q, float *k, float *v, float *g, float *beta, int B, int M,
                    int dim, int conv_dim, int vh, int kh, int kd, bool write_hist,
                    hipStream_t s);

// Dense projection y[r][o] = sum_c W[o][c] x[r][c] for rows r of x
// [rows][C]; W0 (R0 x C, packed by launch_proj_pack) -> y0 [rows][R0] and,
// when W1 is non-null, W1 -> y1 [rows][R1] in the same launch.
// C % 128 == 0, R % 16 == 0.
int launch_proj_pack(const float *W, float *Wp, int R, int C, hipStream_t s);

// The same projection with 4-bit weights packed by launch_proj_q4_pack from
// q [R][C/2] bytes and binary16 scales [R][C/32] (9 C / 16 bytes per row);
// 1 to 16 rows, R % 64 == 0, C % 1024 == 0.
int launch_proj_q4_pack(const uint8_t *q, const uint16_t *scale, void *Wq, int R, int C,
                        hipStream_t s);
int launch_proj_q4(const float *x, int64_t rows, int C, const void *Wq0, int R0, float *y0,
                   const void *Wq1, int R1, float *y1, hipStream_t s);
int64_t proj_workgroups(int64_t rows, int R0, int R1);
int launch_proj(const float *x, int64_t rows, int C, const float *W0, int R0, float *y0,
                const float *W1, int R1, float *y1, hipStream_t s);

}  // namespace gdn
