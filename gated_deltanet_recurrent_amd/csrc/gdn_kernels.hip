// gdn_kernels.hip -- gfx950 (MI355X, CDNA4) kernels of the Gated DeltaNet
// recurrent decode step, its M-step / rollback forms and its front end.
//
// The step ("Kestrel_VLLM #24: GDN linear attention on GPU", section 4 and
// Fig. 1 caption) is a GEMV plus a rank-1 update per (unit, value head) over
// a kd x vd fp32 state: 0.87 flop per byte, so it is bound by HBM bandwidth,
// not by arithmetic, and uses no MFMA.  The design streams each 64 KiB state
// tile through VGPRs exactly once per call:
//
//  * one workgroup per tile (unit, value head); 256 lanes (4 wave64) for
//    kd = 128, 64 lanes for kd = 64.  Lane t owns 4 adjacent columns
//    (dv = 4*(t % (kd/4)) .. +3) of the rows dk = rg + RG*j, j = 0..15,
//    rg = t / (kd/4), RG = row groups.  One wave-wide 128-bit load therefore
//    covers RG*... contiguous 512 B rows: every access is a fully coalesced
//    global_load_dwordx4, issued all at once before any arithmetic.
//  * the key/query read-outs (sums over dk) are done per lane over its 16
//    rows, then across the RG row groups through LDS with one barrier each.
//  * q and k of the tile's key head are staged in LDS once per step.
//  * the state is loaded and stored with non-temporal hints: it is touched
//    once per call and would only evict useful lines from L2 / MALL.
//  * the M-step form keeps the tile in VGPRs across all M steps (read once,
//    written once); rollback is the same kernel reading the snapshot and
//    running accepted[u] steps.  gdn_step, gdn_step_m and gdn_rollback thus
//    execute the identical per-step instruction sequence (bit-identical
//    results), with FMA use fixed explicitly: this file is compiled with
//    -ffp-contract=off and fuses only where __builtin_elementwise_fma says so.
#include "gdn_launch.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace gdn {

typedef float f4 __attribute__((ext_vector_type(4)));

static __device__ __forceinline__ f4 fma4(f4 a, f4 b, f4 c) {
  return __builtin_elementwise_fma(a, b, c);
}
static __device__ __forceinline__ f4 splat(float x) { return f4{x, x, x, x}; }

static __device__ __forceinline__ f4 ld_nt(const float *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f4 *>(p));
}
static __device__ __forceinline__ void st_nt(float *p, f4 x) {
  __builtin_nontemporal_store(x, reinterpret_cast<f4 *>(p));
}
static __device__ __forceinline__ f4 ld4(const float *p) {
  return *reinterpret_cast<const f4 *>(p);
}
static __device__ __forceinline__ void st4(float *p, f4 x) {
  *reinterpret_cast<f4 *>(p) = x;
}

// ---------------------------------------------------------------------------
// Recurrence
// ---------------------------------------------------------------------------

template <int KD, int NW>
struct Geo {
  static constexpr int LANES = 64 * NW;
  static constexpr int CG = KD / 4;          // column groups (4 columns each)
  static constexpr int RG = LANES / CG;      // row groups
  static constexpr int R = KD / RG;          // rows per lane
  static constexpr int QK = 2 * KD / LANES;  // q/k elements staged per lane
  static_assert(LANES % CG == 0 && KD % RG == 0 && (2 * KD) % LANES == 0, "tile");
};

struct RecurArgs {
  const float *S_src;
  float *S_dst;
  const float *q, *k, *v, *g, *beta;
  float *o;              // nullable: rollback writes no output
  const int32_t *steps;  // nullable: per-unit step counts
  int64_t n_units;
  int vh, kh, M;
};

template <int KD, int NW>
__global__ __launch_bounds__(64 * NW) void recur_kernel(RecurArgs a) {
  using G = Geo<KD, NW>;
  __shared__ float s_qk[2 * KD];              // q | k of the current step
  __shared__ f4 s_red_k[G::RG][G::CG];        // per row-group partials of S^T k
  __shared__ f4 s_red_o[G::RG][G::CG];        // per row-group partials of S^T q

  const int t = threadIdx.x;
  const int cg = t % G::CG;
  const int rg = t / G::CG;
  const int64_t tile = blockIdx.x;
  const int64_t unit = tile / a.vh;
  const int head = (int)(tile - unit * a.vh);
  const int hh = head / (a.vh / a.kh);
  const int steps = a.steps ? a.steps[unit] : a.M;
  const int64_t tile_off = tile * (int64_t)(KD * KD);
  const float *src = a.S_src + tile_off + rg * KD + 4 * cg;
  float *dst = a.S_dst + tile_off + rg * KD + 4 * cg;

  // Inputs of step 0, fetched before the state so that their latency hides
  // under the state stream.
  float qk_reg[G::QK];
  f4 vv = splat(0.0f);
  float gg = 0.0f, bt = 0.0f;
  auto fetch = [&](int m) {
    const int64_t urow = (int64_t)m * a.n_units + unit;
    const float *qrow = a.q + (urow * a.kh + hh) * KD;
    const float *krow = a.k + (urow * a.kh + hh) * KD;
#pragma unroll
    for (int i = 0; i < G::QK; i++) {
      const int e = t + i * G::LANES;
      qk_reg[i] = e < KD ? qrow[e] : krow[e - KD];
    }
    vv = ld4(a.v + (urow * a.vh + head) * KD + 4 * cg);
    gg = a.g[urow * a.vh + head];
    bt = a.beta[urow * a.vh + head];
  };
  if (steps > 0) fetch(0);

  f4 s[G::R];
#pragma unroll
  for (int j = 0; j < G::R; j++) s[j] = ld_nt(src + j * (G::RG * KD));

  for (int m = 0; m < steps; m++) {
#pragma unroll
    for (int i = 0; i < G::QK; i++) s_qk[t + i * G::LANES] = qk_reg[i];
    const float alpha = expf(gg);
    const float beta = bt;
    const f4 vcur = vv;
    __syncthreads();
    if (m + 1 < steps) fetch(m + 1);

    // decay, then partial S^T k over this lane's rows (decayed state)
    f4 kvp = splat(0.0f);
#pragma unroll
    for (int j = 0; j < G::R; j++) {
      s[j] = s[j] * alpha;
      kvp = fma4(s[j], splat(s_qk[KD + rg + G::RG * j]), kvp);
    }
    s_red_k[rg][cg] = kvp;
    __syncthreads();
    f4 kv = s_red_k[0][cg];
#pragma unroll
    for (int r = 1; r < G::RG; r++) kv = kv + s_red_k[r][cg];
    const f4 tmp = (vcur - kv) * beta;

    // rank-1 update, then partial S^T q with the updated state
    f4 op = splat(0.0f);
#pragma unroll
    for (int j = 0; j < G::R; j++) {
      const int row = rg + G::RG * j;
      s[j] = fma4(splat(s_qk[KD + row]), tmp, s[j]);
      op = fma4(s[j], splat(s_qk[row]), op);
    }
    s_red_o[rg][cg] = op;
    __syncthreads();
    if (a.o != nullptr && rg == 0) {
      f4 ov = s_red_o[0][cg];
#pragma unroll
      for (int r = 1; r < G::RG; r++) ov = ov + s_red_o[r][cg];
      const int64_t urow = (int64_t)m * a.n_units + unit;
      st4(a.o + (urow * a.vh + head) * KD + 4 * cg, ov);
    }
  }

#pragma unroll
  for (int j = 0; j < G::R; j++) st_nt(dst + j * (G::RG * KD), s[j]);
}

int recur_lanes(int kd) { return kd == 128 ? 256 : 64; }

int launch_recur(int kd, const float *S_src, float *S_dst, const float *q,
                 const float *k, const float *v, const float *g,
                 const float *beta, float *o, const int32_t *steps,
                 int64_t n_units, int vh, int kh, int M, hipStream_t s) {
  RecurArgs a{S_src, S_dst, q, k, v, g, beta, o, steps, n_units, vh, kh, M};
  const int64_t tiles = n_units * vh;
  if (tiles <= 0) return 0;
  if (kd == 128)
    hipLaunchKernelGGL((recur_kernel<128, 4>), dim3((unsigned)tiles), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((recur_kernel<64, 1>), dim3((unsigned)tiles), dim3(64), 0, s, a);
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------
// Streaming copy (mark, and the read+write floor)
// ---------------------------------------------------------------------------

constexpr int COPY_LANES = 256;
constexpr int COPY_UNROLL = 4;

__global__ __launch_bounds__(COPY_LANES) void copy_kernel(float *dst, const float *src,
                                                          int64_t n4, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * COPY_LANES;
  int64_t i = (int64_t)blockIdx.x * COPY_LANES + threadIdx.x;
  for (; i + (COPY_UNROLL - 1) * stride < n4; i += COPY_UNROLL * stride) {
    f4 x[COPY_UNROLL];
#pragma unroll
    for (int u = 0; u < COPY_UNROLL; u++) x[u] = ld_nt(src + 4 * (i + u * stride));
#pragma unroll
    for (int u = 0; u < COPY_UNROLL; u++) st_nt(dst + 4 * (i + u * stride), x[u]);
  }
  for (; i < n4; i += stride) st_nt(dst + 4 * i, ld_nt(src + 4 * i));
  if (blockIdx.x == 0 && threadIdx.x < (n - 4 * n4)) dst[4 * n4 + threadIdx.x] = src[4 * n4 + threadIdx.x];
}

int launch_copy(float *dst, const float *src, int64_t n, hipStream_t s) {
  if (n <= 0) return 0;
  const int64_t n4 = n / 4;
  int64_t blocks = (n4 + (int64_t)COPY_LANES * COPY_UNROLL - 1) / ((int64_t)COPY_LANES * COPY_UNROLL);
  if (blocks > 256 * 64) blocks = 256 * 64;   // 64 workgroups per CU, grid-stride beyond
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(COPY_LANES), 0, s, dst, src, n4, n);
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------
// Conv-history rollback: pure data movement, bit-exact.
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void hist_replay_kernel(float *hist, const float *snap,
                                                          const float *xc_raw,
                                                          const int32_t *accepted,
                                                          int64_t n_units, int conv_dim,
                                                          int nprev) {
  const int64_t u = blockIdx.y;
  const int c4 = blockIdx.x * 256 + threadIdx.x;
  if (4 * c4 >= conv_dim) return;
  const int acc = accepted[u];
  const int64_t hbase = u * (int64_t)nprev * conv_dim + 4 * c4;
  for (int j = 0; j < nprev; j++) {
    // frame j of the history after acc pushes is element acc + j of the
    // sequence [old frames 0..nprev-1, raw 0..acc-1]
    const int idx = acc + j;
    const float *from = idx < nprev ? snap + u * (int64_t)nprev * conv_dim + (int64_t)idx * conv_dim + 4 * c4
                                    : xc_raw + ((int64_t)(idx - nprev) * n_units + u) * conv_dim + 4 * c4;
    st4(hist + hbase + (int64_t)j * conv_dim, ld4(from));
  }
}

int launch_hist_replay(float *hist, const float *snap, const float *xc_raw,
                       const int32_t *accepted, int64_t n_units, int conv_dim,
                       int ck, hipStream_t s) {
  if (n_units <= 0) return 0;
  dim3 grid((unsigned)((conv_dim / 4 + 255) / 256), (unsigned)n_units);
  hipLaunchKernelGGL(hist_replay_kernel, grid, dim3(256), 0, s, hist, snap, xc_raw, accepted,
                     n_units, conv_dim, ck - 1);
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------
// Front end, kernel A: paired GEMV (a = Wa x, b = Wb x) with the gate / beta
// transform in the epilogue ("Kestrel_VLLM #27", section 4.2: both
// projections in one launch; "Kestrel_VLLM #24", section 3: g from a, beta
// from b).  A workgroup owns FB batch rows x FR rows of the stacked [Wa; Wb]
// and splits the dot products across its 256 lanes (128-bit loads, lane
// stride 1024 floats); the 32 partial sums per lane are reduced with a
// transposing butterfly (32 shuffles per lane) and then across the 4 waves.
// ---------------------------------------------------------------------------

constexpr int FB = 8;   // batch rows per workgroup
constexpr int FR = 4;   // stacked weight rows per workgroup

static __device__ __forceinline__ float softplus_guarded(float z) {
  if (z > 20.0f) return z;
  if (z < -20.0f) return expf(z);
  return log1pf(expf(z));
}

__global__ __launch_bounds__(256) void fe_gemv_kernel(const float *x, const float *Wa,
                                                      const float *Wb, const float *A_log,
                                                      const float *dt_bias, float *g,
                                                      float *beta, int B, int dim, int vh) {
  __shared__ float s_w[4][FB * FR];
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int b0 = blockIdx.x * FB;
  const int r0 = blockIdx.y * FR;

  const float *wrow[FR];
#pragma unroll
  for (int r = 0; r < FR; r++) {
    int R = r0 + r;
    if (R >= 2 * vh) R = 2 * vh - 1;                 // clamped rows are never written
    wrow[r] = R < vh ? Wa + (int64_t)R * dim : Wb + (int64_t)(R - vh) * dim;
  }
  const float *xrow[FB];
#pragma unroll
  for (int b = 0; b < FB; b++) {
    int bb = b0 + b;
    if (bb >= B) bb = B - 1;
    xrow[b] = x + (int64_t)bb * dim;
  }

  float acc[FB * FR];
#pragma unroll
  for (int i = 0; i < FB * FR; i++) acc[i] = 0.0f;
  for (int c = 4 * t; c < dim; c += 4 * 256) {
    f4 w[FR];
#pragma unroll
    for (int r = 0; r < FR; r++) w[r] = ld4(wrow[r] + c);
#pragma unroll
    for (int b = 0; b < FB; b++) {
      const f4 xv = ld4(xrow[b] + c);
#pragma unroll
      for (int r = 0; r < FR; r++) {
        float s = acc[b * FR + r];
        s = __builtin_fmaf(w[r].x, xv.x, s);
        s = __builtin_fmaf(w[r].y, xv.y, s);
        s = __builtin_fmaf(w[r].z, xv.z, s);
        s = __builtin_fmaf(w[r].w, xv.w, s);
        acc[b * FR + r] = s;
      }
    }
  }

  // Transposing butterfly over the 64 lanes: after the step with offset 2^p
  // (p = 5..1) each lane keeps half of its values, summed with its partner's
  // matching half; finally lane pairs (offset 1) add up.  Lane l then holds
  // the wave sum of output (l >> 1).
  static_assert(FB * FR == 32, "butterfly is written for 32 outputs");
  float v16[16];
  {
    const bool up = lane & 32;
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const float send = up ? acc[i] : acc[16 + i];
      const float keep = up ? acc[16 + i] : acc[i];
      v16[i] = keep + __shfl_xor(send, 32);
    }
  }
  float v8[8];
  {
    const bool up = lane & 16;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const float send = up ? v16[i] : v16[8 + i];
      const float keep = up ? v16[8 + i] : v16[i];
      v8[i] = keep + __shfl_xor(send, 16);
    }
  }
  float v4[4];
  {
    const bool up = lane & 8;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const float send = up ? v8[i] : v8[4 + i];
      const float keep = up ? v8[4 + i] : v8[i];
      v4[i] = keep + __shfl_xor(send, 8);
    }
  }
  float v2[2];
  {
    const bool up = lane & 4;
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const float send = up ? v4[i] : v4[2 + i];
      const float keep = up ? v4[2 + i] : v4[i];
      v2[i] = keep + __shfl_xor(send, 4);
    }
  }
  float v1;
  {
    const bool up = lane & 2;
    const float send = up ? v2[0] : v2[1];
    const float keep = up ? v2[1] : v2[0];
    v1 = keep + __shfl_xor(send, 2);
  }
  v1 = v1 + __shfl_xor(v1, 1);
  if ((lane & 1) == 0) s_w[wave][lane >> 1] = v1;
  __syncthreads();
  if (t < FB * FR) {
    const float sum = ((s_w[0][t] + s_w[1][t]) + s_w[2][t]) + s_w[3][t];
    const int b = b0 + t / FR;
    const int R = r0 + t % FR;
    if (b < B && R < 2 * vh) {
      if (R < vh) {
        const float sp = softplus_guarded(sum + dt_bias[R]);
        g[(int64_t)b * vh + R] = -expf(A_log[R]) * sp;
      } else {
        beta[(int64_t)b * vh + (R - vh)] = 1.0f / (1.0f + expf(-sum));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Front end, kernel B: depthwise causal conv (4 taps) + SiLU + history
// advance + split + per key-head L2 norm ("Kestrel_VLLM #24", section 3 and
// Fig. 1 caption).  One workgroup per (row, block of 1024 channels); each
// lane owns 4 adjacent channels, whose 4 taps are one 16-float run of conv_w.
// A key head (KD channels) is KD/4 adjacent lanes of one wave, so its sum of
// squares is a shuffle reduction.  Head boundaries are multiples of KD and
// blocks are multiples of 1024, so no head straddles two workgroups.
// ---------------------------------------------------------------------------

template <int KD>
__global__ __launch_bounds__(256) void fe_conv_kernel(const float *xc_raw, float *hist,
                                                      const float *conv_w, float *q, float *k,
                                                      float *v, int conv_dim, int kh, int vh) {
  const int t = threadIdx.x;
  const int64_t b = blockIdx.y;
  const int ch = blockIdx.x * 1024 + 4 * t;
  const bool valid = ch < conv_dim;
  const int qk_w = kh * KD;
  float out[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (valid) {
    const f4 raw = ld4(xc_raw + b * conv_dim + ch);
    float *hb = hist + b * 3 * (int64_t)conv_dim + ch;
    const f4 h0 = ld4(hb), h1 = ld4(hb + conv_dim), h2 = ld4(hb + 2 * (int64_t)conv_dim);
    const float *w = conv_w + (int64_t)ch * 4;
    const f4 w0 = ld4(w), w1 = ld4(w + 4), w2 = ld4(w + 8), w3 = ld4(w + 12);
    const f4 wc[4] = {w0, w1, w2, w3};
    const float hr0[4] = {h0.x, h0.y, h0.z, h0.w};
    const float hr1[4] = {h1.x, h1.y, h1.z, h1.w};
    const float hr2[4] = {h2.x, h2.y, h2.z, h2.w};
    const float rr[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int c = 0; c < 4; c++) {
      float acc = wc[c].x * hr0[c];
      acc = __builtin_fmaf(wc[c].y, hr1[c], acc);
      acc = __builtin_fmaf(wc[c].z, hr2[c], acc);
      acc = __builtin_fmaf(wc[c].w, rr[c], acc);
      out[c] = acc / (1.0f + expf(-acc));
    }
    st4(hb, h1);
    st4(hb + conv_dim, h2);
    st4(hb + 2 * (int64_t)conv_dim, raw);
  }
  // per key-head sum of squares over KD/4 lanes (every lane takes part)
  float ss = out[0] * out[0];
  ss = __builtin_fmaf(out[1], out[1], ss);
  ss = __builtin_fmaf(out[2], out[2], ss);
  ss = __builtin_fmaf(out[3], out[3], ss);
#pragma unroll
  for (int off = 1; off < KD / 4; off <<= 1) ss = ss + __shfl_xor(ss, off);
  if (!valid) return;
  const f4 o4 = {out[0], out[1], out[2], out[3]};
  if (ch < 2 * qk_w) {
    const float inv = 1.0f / sqrtf(ss + 1e-6f);
    if (ch < qk_w) {
      const float qs = inv * (1.0f / sqrtf((float)KD));
      st4(q + b * qk_w + ch, (o4 * inv) * (1.0f / sqrtf((float)KD)));
      (void)qs;
    } else {
      st4(k + b * qk_w + (ch - qk_w), o4 * inv);
    }
  } else {
    st4(v + b * (int64_t)vh * KD + (ch - 2 * qk_w), o4);
  }
}

int launch_frontend(const float *x, const float *Wa, const float *Wb,
                    const float *A_log, const float *dt_bias,
                    const float *xc_raw, float *hist, const float *conv_w,
                    float *q, float *k, float *v, float *g, float *beta, int B,
                    int dim, int conv_dim, int vh, int kh, int kd,
                    hipStream_t s) {
  if (B <= 0) return 0;
  dim3 ga((unsigned)((B + FB - 1) / FB), (unsigned)((2 * vh + FR - 1) / FR));
  hipLaunchKernelGGL(fe_gemv_kernel, ga, dim3(256), 0, s, x, Wa, Wb, A_log, dt_bias, g, beta,
                     B, dim, vh);
  dim3 gb((unsigned)((conv_dim + 1023) / 1024), (unsigned)B);
  if (kd == 128)
    hipLaunchKernelGGL(fe_conv_kernel<128>, gb, dim3(256), 0, s, xc_raw, hist, conv_w, q, k, v,
                       conv_dim, kh, vh);
  else
    hipLaunchKernelGGL(fe_conv_kernel<64>, gb, dim3(256), 0, s, xc_raw, hist, conv_w, q, k, v,
                       conv_dim, kh, vh);
  return (int)hipGetLastError();
}

}  // namespace gdn
