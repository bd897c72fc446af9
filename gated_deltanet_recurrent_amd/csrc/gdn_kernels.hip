// gdn_kernels.hip -- gfx950 (MI355X, CDNA4) kernels of the Gated DeltaNet
// recurrent decode step, its M-step / rollback / verify forms, its front end
// and the layer's dense projections.
//
// Recurrence.  The step ("Kestrel_VLLM #24: GDN linear attention on GPU",
// section 4 and Fig. 1 caption) is a GEMV plus a rank-1 update per (unit,
// value head) over a kd x vd fp32 state: 0.87 flop per byte, so it is bound
// by HBM bandwidth, not by arithmetic, and uses no MFMA.  Each 64 KiB state
// tile streams through VGPRs exactly once per call:
//  * wide geometry (single steps; also M <= 8 steps for launches of few
//    tiles): 16 floats per lane, 4 adjacent columns of the rows rg + RG*j;
//    kd = 128 on 1024 lanes per tile, kd = 64 on 256 lanes with four tiles of
//    one unit per workgroup.  A wave-wide 128-bit load covers 1 KiB of
//    consecutive rows, all issued before any arithmetic.
//  * deep geometry (M steps): 64 floats per lane, more tiles per CU and fewer
//    cross-lane exchanges per element; the tile stays in VGPRs across all M
//    steps (read once, written once).
//  * split geometry (ungated calls on a few tiles, kd = 128): the wide lane
//    layout over a quarter of a tile's columns, four workgroups per tile, one
//    barrier per step; for the latency-bound single-sequence case.
//  * all geometries compute one canonical summation tree for the read-outs,
//    so step, step_m, rollback, verify and commit agree bit for bit whichever
//    geometry serves them; FMA use is explicit (this file is compiled with
//    -ffp-contract=off and fuses only where an fma builtin says so).
//  * workgroups are remapped so that each XCD streams a contiguous range of
//    tiles; the state is streamed with raw buffer loads (nt) and stores
//    (sc0 sc1 nt); per-step inputs are staged in LDS in chunks of 8 rows.
// Front end (section 3 and Fig. 1 caption): the paired beta / a GEMV with the
// gate transform and the causal conv + SiLU + q/k normalisation in one launch
// (M draft rows of a few sequences run their conv rows in parallel).
// Projections (Fig. 1 caption, steps 1 and 7): f32 weights on the fp32
// matrix cores in packed operand order, and 4-bit weights with binary16 block
// scales (section 8 and 12) on the fp16 matrix cores, the values decoded
// exactly and x split exactly into three binary16 parts; each with a fixed
// summation order independent of the row count.
#include "gdn_launch.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

namespace gdn {

typedef float f4 __attribute__((ext_vector_type(4)));

static __device__ __forceinline__ f4 fma4(f4 a, f4 b, f4 c) {
  return __builtin_elementwise_fma(a, b, c);
}
static __device__ __forceinline__ f4 splat(float x) { return f4{x, x, x, x}; }

typedef unsigned u4 __attribute__((ext_vector_type(4)));

// The state stream goes through raw buffer loads/stores so that its cache
// policy can be set per instruction.  A state larger than the caches
// (RESIDENT = false) is streamed with non-temporal loads (nt) and stores
// carrying sc0 sc1 nt: on a 50/50 read/write stream of 64 KiB tiles that
// store policy measured 1.4% above nt alone.  A state that fits in half the
// 256 MiB MALL (RESIDENT = true) keeps the default policy, so that it can
// stay cached between calls (one unit of 48 heads: 5.9 -> 5.2 us per step).
// A buffer resource covers one tile (bounds = its size in bytes), so
// offsets are 32-bit.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int POL_STREAM_LOAD = 2;                 // nt
constexpr int POL_STREAM_STORE = 1 | 2 | 16;       // sc0 | nt | sc1
constexpr int RSRC_FLAGS = 0x00020000;             // raw 32-bit buffer, gfx9 family
constexpr int64_t RESIDENT_MAX_BYTES = 128ll << 20;

static __device__ __forceinline__ rsrc_t buf_rsrc(const float *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), 0, bytes, RSRC_FLAGS);
}
// voff: per-lane byte offset (VGPR); soff: wave-uniform byte offset (SGPR),
// so that one VGPR addresses all of a lane's rows.
template <bool RESIDENT = false>
static __device__ __forceinline__ f4 ld_stream(rsrc_t r, int voff, int soff = 0) {
  return __builtin_bit_cast(
      f4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, RESIDENT ? 0 : POL_STREAM_LOAD));
}
template <bool RESIDENT = false>
static __device__ __forceinline__ void st_stream(rsrc_t r, int voff, int soff, f4 x) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, x), r, voff, soff,
                                         RESIDENT ? 0 : POL_STREAM_STORE);
}
static __device__ __forceinline__ f4 ld4(const float *p) {
  return *reinterpret_cast<const f4 *>(p);
}
static __device__ __forceinline__ void st4(float *p, f4 x) {
  *reinterpret_cast<f4 *>(p) = x;
}

// The value of lane (lane ^ OFF) of the wave, without the LDS crossbar:
// v_permlane32_swap / v_permlane16_swap (gfx950) for 32 and 16, DPP row_ror:8
// and quad_perm for 8, 2 and 1, ds_swizzle's bitmask mode for 4.  Every lane
// of the wave must be active.
template <int OFF>
static __device__ __forceinline__ float lane_xor(float v) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  unsigned r;
  if constexpr (OFF == 32) {
    const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    r = (threadIdx.x & 32) ? p[0] : p[1];
  } else if constexpr (OFF == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    r = (threadIdx.x & 16) ? p[0] : p[1];
  } else if constexpr (OFF == 8) {
    r = __builtin_amdgcn_update_dpp(0u, u, 0x128, 0xf, 0xf, false);   // row_ror:8
  } else if constexpr (OFF == 4) {
    r = __builtin_amdgcn_ds_swizzle(u, 0x1f | (4 << 10));              // xor 4 in 32 lanes
  } else if constexpr (OFF == 2) {
    r = __builtin_amdgcn_update_dpp(0u, u, 0x4e, 0xf, 0xf, false);    // quad_perm [2,3,0,1]
  } else {
    static_assert(OFF == 1, "lane_xor: offsets 1, 2, 4, 8, 16, 32");
    r = __builtin_amdgcn_update_dpp(0u, u, 0xb1, 0xf, 0xf, false);    // quad_perm [1,0,3,2]
  }
  return __builtin_bit_cast(float, r);
}

// v + v of lane (lane ^ OFF), for OFF = FROM, 2 FROM, ... up to TO - 1.
// XB: through the LDS crossbar (ds_bpermute) instead, which costs the
// bandwidth-bound single-step kernel less issue time (0.25% in a same-box
// A/B); both move the same values, so the sums are the same bits.
template <int FROM, int TO, bool XB = false>
static __device__ __forceinline__ float xor_fold(float v) {
  if constexpr (FROM < TO) {
    v = v + (XB ? __shfl_xor(v, FROM) : lane_xor<FROM>(v));
    return xor_fold<2 * FROM, TO, XB>(v);
  } else {
    return v;
  }
}

// ---------------------------------------------------------------------------
// Workgroup -> tile mapping
// ---------------------------------------------------------------------------

// The dispatcher hands workgroup b to XCD b % 8.  Remap so that each XCD
// streams one contiguous range of tiles (large sequential runs per XCD measure
// 6-8% faster on a 50/50 read/write stream than tiles interleaved across
// XCDs) and so that the value heads sharing a key head meet in one L2.
// Bijective for any grid size: the first `full` XCDs get `per` blocks, the
// others per - 1.
static __device__ __forceinline__ int64_t xcd_contiguous(int64_t b, int64_t nb) {
  const int64_t per = (nb + 7) >> 3;
  const int64_t x = b & 7, i = b >> 3;
  const int64_t full = nb - 8 * (per - 1);
  return x < full ? x * per + i : full * per + (x - full) * (per - 1) + i;
}

// ---------------------------------------------------------------------------
// Recurrence
// ---------------------------------------------------------------------------
//
// Canonical summation order of the read-outs S^T k and S^T q for one column.
// Rows are grouped as rg + RG*j (RG = kd/4 row groups, j = 0..3):
//   p[rg]  = fma chain over j = 0..3 of S[rg + RG*j] * x[rg + RG*j]
//   kd = 128: W[w] = p[2w] + p[2w+1] (w < 16);
//             H0 = W0 + W1 + ... + W7, H1 = W8 + ... + W15 (left folds);
//             sum = H0 + H1
//   kd = 64:  W[w] = (p[4w] + p[4w+1]) + (p[4w+2] + p[4w+3]) (w < 4);
//             sum = (W0 + W1) + (W2 + W3)
// Three tile geometries compute exactly this tree, so every entry point gives
// the same bits whichever geometry serves it:
//   wide (single steps, bandwidth bound): 16 floats per lane, kd = 128 on
//     1024 lanes, kd = 64 on 256 lanes; lane = (column group, row group);
//   deep (several steps per call, arithmetic bound): 64 floats per lane,
//     kd = 128 on 256 lanes, kd = 64 on one wave; lane = (column group,
//     4 consecutive row groups), which keeps more tiles resident per CU and
//     needs fewer cross-lane exchanges per element;
//   split (few tiles, latency bound, kd = 128): the wide lane layout over a
//     quarter of the columns, four workgroups per tile.

template <int KD>
struct Canon {
  static constexpr int RG = KD / 4;              // row groups (rows rg + RG*j)
  static constexpr int CG = KD / 4;              // column groups of 4 columns
  static constexpr int NWP = KD == 128 ? 16 : 4; // W partials
};

// Wide geometry.
template <int KD>
struct Geo {
  static constexpr int NW = KD * KD / (16 * 64);  // waves per tile
  static constexpr int LANES = 64 * NW;
  static constexpr int CG = Canon<KD>::CG;
  static constexpr int RG = LANES / CG;           // row groups, one per lane row
  static constexpr int R = KD / RG;               // rows per lane
  static constexpr int GPW = 64 / CG;             // row groups per wave
  static constexpr int PER = NW / GPW;            // W partials per final-sum lane group
  static_assert(R == 4 && RG == Canon<KD>::RG && NW == Canon<KD>::NWP, "wide geometry");
};

// Deep geometry.
template <int KD>
struct Deep {
  static constexpr int LANES = KD * KD / 64;      // 64 floats per lane
  static constexpr int CG = Canon<KD>::CG;
  static constexpr int LG = LANES / CG;           // lane rows; each holds 4 row groups
  static_assert(LG * 4 == Canon<KD>::RG, "deep geometry");
};

// Fold over the row groups that share this lane's columns inside one wave
// (lanes t, t ^ CG, ...).  Every add is commutative, so all those lanes end
// up with the same bits.
template <int KD, bool XB = false>
static __device__ __forceinline__ f4 wave_fold(f4 p) {
  p.x = xor_fold<Canon<KD>::CG, 64, XB>(p.x);
  p.y = xor_fold<Canon<KD>::CG, 64, XB>(p.y);
  p.z = xor_fold<Canon<KD>::CG, 64, XB>(p.z);
  p.w = xor_fold<Canon<KD>::CG, 64, XB>(p.w);
  return p;
}

// Final sum over the W partials red[NWP][CG] by one wave: lane group
// h = lane / CG left-folds partials h*PER .. h*PER + PER - 1, then the groups
// are folded.  Valid in every lane of the wave for column group lane % CG.
template <int KD, bool XB = false>
static __device__ __forceinline__ f4 tile_sum(const f4 (*red)[Canon<KD>::CG], int lane) {
  constexpr int CG = Canon<KD>::CG;
  constexpr int PER = Canon<KD>::NWP / (64 / CG);
  const int cg = lane % CG, h = lane / CG;
  f4 acc = red[h * PER][cg];
#pragma unroll
  for (int i = 1; i < PER; i++) acc = acc + red[h * PER + i][cg];
  return wave_fold<KD, XB>(acc);
}

struct RecurArgs {
  const float *S_src;
  float *S_dst;
  const float *q, *k, *v, *g, *beta;
  float *o;              // nullable: rollback writes no output
  const int32_t *steps;  // nullable: per-unit step counts
  const float *z;        // gated output only: gate z [rows][N][vh][vd]
  const float *norm_w;   // gated output only: RMSNorm weight [vd]
  float eps;             // gated output only
  float *snap;           // nullable: the loaded state is also written here (mark)
  int32_t *status;       // nullable: set to 1 when a per-unit step count is out of range
  int64_t n_units;
  int vh, kh, M;
  // nullable: the conv history replayed in the same launch (M-step kernels):
  // workgroups past the tiles' push steps[u] raw rows into hist[u]
  float *hist;
  const float *hist_src; // hist itself (commit) or its snapshot (rollback)
  const float *xc_raw;   // [M][N][conv_dim]
  int conv_dim;
  int64_t tile_wgs;      // workgroups of the tiles; the rest replay history
  // commit + verify in one pass (M-step kernel only; q2 == nullptr otherwise):
  // after the steps[u] rows above are applied and the state stored, M2 rows
  // of these inputs run from the stored state, outputs to o2, state not stored
  const float *q2 = nullptr, *k2 = nullptr, *v2 = nullptr, *g2 = nullptr, *beta2 = nullptr;
  float *o2 = nullptr;
  int M2 = 0;
};

// Per-step inputs are staged through LDS in chunks of MC rows.  q and k are
// stored permuted, element rg*4 + j holding row rg + RG*j, so that a lane
// reads the 4 values of one row group with a single 128-bit LDS load.  For
// calls of more than MC rows the registers of each lane prefetch the next
// chunk while the current one runs (double-buffered stage).
constexpr int MC = 8;

template <int KD, bool GATED>
struct Stage {
  float q[MC][KD];
  float k[MC][KD];
  float v[MC][KD];
  float z[GATED ? MC : 1][GATED ? KD : 1];   // gate of the fused RMSNorm
  float alpha[MC];       // exp(g)
  float beta[MC];
};

template <int KD, int LANES, bool GATED>
struct ChunkRegs {
  static constexpr int E = MC * KD;                   // floats of q (or k, v) per chunk
  static constexpr int P = (E + LANES - 1) / LANES;   // per lane
  float q[P], k[P], v[P];
  float z[GATED ? P : 1];
  float gb;  // g (lanes < MC) or beta (lanes MC .. 2*MC-1)
};

template <int KD, int LANES, bool GATED>
static __device__ __forceinline__ void chunk_load(ChunkRegs<KD, LANES, GATED> &c,
                                                  const RecurArgs &a, int t, int64_t unit,
                                                  int head, int hh, int m0, int nr) {
  using C = ChunkRegs<KD, LANES, GATED>;
  if constexpr (LANES % KD == 0) {
    // element i of this lane is row t / KD + i LANES / KD, column t % KD:
    // one base address per array and a uniform row stride
    constexpr int RPI = LANES / KD;
    const int col = t % KD, r0 = t / KD;
    const int64_t urow = (int64_t)(m0 + r0) * a.n_units + unit;
    const float *qp = a.q + (urow * a.kh + hh) * KD + col;
    const float *kp = a.k + (urow * a.kh + hh) * KD + col;
    const float *vp = a.v + (urow * a.vh + head) * KD + col;
    const float *zp = GATED ? a.z + (urow * a.vh + head) * KD + col : nullptr;
    const int64_t sqk = (int64_t)RPI * a.n_units * a.kh * KD;
    const int64_t sv = (int64_t)RPI * a.n_units * a.vh * KD;
#pragma unroll
    for (int i = 0; i < C::P; i++) {
      if (t + i * LANES < C::E && r0 + RPI * i < nr) {
        c.q[i] = qp[i * sqk];
        c.k[i] = kp[i * sqk];
        c.v[i] = vp[i * sv];
        if constexpr (GATED) c.z[i] = zp[i * sv];
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < C::P; i++) {
      const int e = t + i * LANES;
      const int r = e / KD, col = e % KD;
      if (e < C::E && r < nr) {
        const int64_t urow = (int64_t)(m0 + r) * a.n_units + unit;
        c.q[i] = a.q[(urow * a.kh + hh) * KD + col];
        c.k[i] = a.k[(urow * a.kh + hh) * KD + col];
        c.v[i] = a.v[(urow * a.vh + head) * KD + col];
        if constexpr (GATED) c.z[i] = a.z[(urow * a.vh + head) * KD + col];
      }
    }
  }
  if (t < 2 * MC) {
    const int r = t % MC;
    if (r < nr) {
      const int64_t urow = (int64_t)(m0 + r) * a.n_units + unit;
      c.gb = t < MC ? a.g[urow * a.vh + head] : a.beta[urow * a.vh + head];
    }
  }
}

template <int KD, int LANES, bool GATED>
static __device__ __forceinline__ void chunk_store(Stage<KD, GATED> &st,
                                                   const ChunkRegs<KD, LANES, GATED> &c, int t,
                                                   int nr) {
  using C = ChunkRegs<KD, LANES, GATED>;
  constexpr int RG = Canon<KD>::RG;
#pragma unroll
  for (int i = 0; i < C::P; i++) {
    const int e = t + i * LANES;
    const int r = e / KD, col = e % KD;
    if (e < C::E && r < nr) {
      const int pc = (col % RG) * 4 + col / RG;
      st.q[r][pc] = c.q[i];
      st.k[r][pc] = c.k[i];
      st.v[r][col] = c.v[i];
      if constexpr (GATED) st.z[r][col] = c.z[i];
    }
  }
  if (t < 2 * MC && t % MC < nr) {
    if (t < MC)
      st.alpha[t] = expf(c.gb);
    else
      st.beta[t - MC] = c.gb;
  }
}

static __device__ __forceinline__ f4 lds4(const float *p) {
  return *reinterpret_cast<const f4 *>(p);
}

// Writes one head's output for columns 4*cg .. 4*cg+3.  Called by every lane
// of a wave whose lane groups of CG lanes all hold the full output row (the
// fold below reduces across the CG lanes of a group); lanes with `write` set
// store.  GATED applies the gated RMSNorm of the layer's output step
// ("Kestrel_VLLM #24", Fig. 1 caption, step 6; the pages give no formula, the
// model family's definition is used): out = (o * 1/sqrt(mean(o^2) + eps)) *
// w * silu(z), per value head over its vd outputs.
template <int KD, bool GATED, bool XB = false>
static __device__ __forceinline__ void emit_o(const RecurArgs &a, int64_t urow, int head, int cg,
                                              bool write, f4 ov, const float *zrow) {
  if constexpr (GATED) {
    const f4 wn = ld4(a.norm_w + 4 * cg);   // 512 B shared by all tiles: an L2 hit
    float ss = ov.x * ov.x;
    ss = __builtin_fmaf(ov.y, ov.y, ss);
    ss = __builtin_fmaf(ov.z, ov.z, ss);
    ss = __builtin_fmaf(ov.w, ov.w, ss);
    ss = xor_fold<1, Canon<KD>::CG, XB>(ss);
    const float rinv = 1.0f / sqrtf(ss / (float)KD + a.eps);
    const f4 z = lds4(zrow + 4 * cg);
    f4 sz;
    sz.x = z.x / (1.0f + expf(-z.x));
    sz.y = z.y / (1.0f + expf(-z.y));
    sz.z = z.z / (1.0f + expf(-z.z));
    sz.w = z.w / (1.0f + expf(-z.w));
    ov = ((ov * rinv) * wn) * sz;
  }
  if (write) st4(a.o + (urow * a.vh + head) * KD + 4 * cg, ov);
}

struct TileIdx {
  int64_t unit, tile_off;
  int head, hh, steps;
};

static __device__ __forceinline__ TileIdx tile_index(const RecurArgs &a, int kdkd, int tpw = 1,
                                                     int sub = 0) {
  TileIdx x;
  // 32-bit: a launch has fewer than 2^32 work-items and at least 64 per
  // tile, so tile indices stay below 2^26
  const uint32_t tile = (uint32_t)(xcd_contiguous(blockIdx.x, gridDim.x) * tpw + sub);
  const uint32_t unit = tile / (uint32_t)a.vh;
  x.unit = unit;
  x.head = (int)(tile - unit * (uint32_t)a.vh);
  x.hh = (int)((uint32_t)x.head / (uint32_t)(a.vh / a.kh));
  x.steps = a.steps ? a.steps[x.unit] : a.M;
  if (x.steps < 0 || x.steps > a.M) {   // device-supplied counts: refuse the unit
    if (a.status != nullptr && threadIdx.x == 0) a.status[0] = 1;
    x.steps = 0;
  }
  x.tile_off = tile * (int64_t)kdkd;
  return x;
}

// ----- wide geometry -------------------------------------------------------
//
// Serves single-step calls (M = 1; rollback with M = 1 runs 0 or 1 step per
// unit).  Decay and S^T k partials; barrier; wave 0 of each tile finishes
// S^T k and forms tmp = (v - kv) beta; barrier; rank-1 update and S^T q
// partials; barrier; wave 0 of each tile finishes the output.  TPW tiles of
// one unit share a workgroup (lane group t / Geo::LANES owns tile TPW*b + that
// index), so every lane group takes the same branches and barriers.
// kd = 128: at most 64 VGPRs (8 waves per SIMD), so two 16-wave workgroups
// share a CU.
template <int KD, bool RESIDENT, bool GATED, int TPW>
__global__ __launch_bounds__(Geo<KD>::LANES * TPW) __attribute__((amdgpu_waves_per_eu(KD == 128 ? 8 : 6)))
void recur_wide_kernel(RecurArgs a) {
  using G = Geo<KD>;
  constexpr int LANES = G::LANES;
  __shared__ Stage<KD, GATED> sb_all[TPW];
  __shared__ f4 s_red_k_all[TPW][G::NW][G::CG];
  __shared__ f4 s_red_o_all[TPW][G::NW][G::CG];
  __shared__ f4 s_tmp_all[TPW][G::CG];

  const int sub = TPW == 1 ? 0 : (int)threadIdx.x / LANES;   // tile of this lane group
  const int t = TPW == 1 ? (int)threadIdx.x : (int)threadIdx.x % LANES;
  Stage<KD, GATED> &sb = sb_all[sub];
  f4 (*s_red_k)[G::CG] = s_red_k_all[sub];
  f4 (*s_red_o)[G::CG] = s_red_o_all[sub];
  f4 *s_tmp = s_tmp_all[sub];
  const int lane = t & 63, wave = t >> 6;
  const int cg = t % G::CG, rg = t / G::CG;
  const TileIdx ti = tile_index(a, KD * KD, TPW, sub);
  const bool run = ti.steps > 0;       // uniform per workgroup (its tiles share a unit)
  // an in-place update with nothing to run leaves the tile as it is
  if (!run && a.S_src == a.S_dst && a.snap == nullptr) return;
  const rsrc_t src = buf_rsrc(a.S_src + ti.tile_off, KD * KD * 4);
  const int lane_off = (rg * KD + 4 * cg) * 4;

  // the inputs are requested before the state, so that their latency hides
  // under the state stream
  ChunkRegs<KD, LANES, GATED> cr;
  if (run) chunk_load<KD, LANES, GATED>(cr, a, t, ti.unit, ti.head, ti.hh, 0, 1);

  f4 s[G::R];
#pragma unroll
  for (int j = 0; j < G::R; j++) s[j] = ld_stream<RESIDENT>(src, lane_off, j * (G::RG * KD * 4));
  if (a.snap != nullptr) {            // fused mark: the tile as loaded, before the step
    const rsrc_t snp = buf_rsrc(a.snap + ti.tile_off, KD * KD * 4);
#pragma unroll
    for (int j = 0; j < G::R; j++) st_stream<false>(snp, lane_off, j * (G::RG * KD * 4), s[j]);
  }

  if (run) {
    chunk_store<KD, LANES, GATED>(sb, cr, t, 1);
    __syncthreads();
    const float alpha = sb.alpha[0];
    const f4 kk = lds4(&sb.k[0][rg * 4]);
    // decay, then S^T k over the decayed state
    f4 p = splat(0.0f);
#pragma unroll
    for (int j = 0; j < G::R; j++) {
      s[j] = s[j] * alpha;
      p = fma4(s[j], splat(kk[j]), p);
    }
    p = wave_fold<KD, true>(p);
    if (lane < G::CG) s_red_k[wave][lane] = p;
    __syncthreads();
    if (wave == 0) {
      const f4 kv = tile_sum<KD, true>(s_red_k, lane);
      if (lane < G::CG) s_tmp[lane] = (lds4(&sb.v[0][4 * lane]) - kv) * sb.beta[0];
    }
    __syncthreads();
    const f4 tmp = s_tmp[cg];
    const f4 qq = lds4(&sb.q[0][rg * 4]);
    // rank-1 update, then S^T q with the updated state
    p = splat(0.0f);
#pragma unroll
    for (int j = 0; j < G::R; j++) {
      s[j] = fma4(splat(kk[j]), tmp, s[j]);
      p = fma4(s[j], splat(qq[j]), p);
    }
    p = wave_fold<KD, true>(p);
    if (lane < G::CG) s_red_o[wave][lane] = p;
  }

  if (a.S_dst != nullptr) {            // null: outputs only, the state is left as it was
    const rsrc_t dst = buf_rsrc(a.S_dst + ti.tile_off, KD * KD * 4);
#pragma unroll
    for (int j = 0; j < G::R; j++) st_stream<RESIDENT>(dst, lane_off, j * (G::RG * KD * 4), s[j]);
  }

  if (run) {
    __syncthreads();
    if (wave == 0 && a.o != nullptr) {
      const f4 ov = tile_sum<KD, true>(s_red_o, lane);
      emit_o<KD, GATED, true>(a, ti.unit, ti.head, lane % G::CG, lane < G::CG, ov,
                        &sb.z[0][0]);
    }
  }
}

// Conv-history replay of unit u, float4 channels c4 (pure data movement,
// bit-exact): frame j after acc pushes is element acc + j of the sequence
// [old frames 0..2, raw rows 0..acc-1]; all frames are read before any is
// written, so src may be hist itself.  A count outside 0..M leaves the unit
// as it was and sets status.
static __device__ __forceinline__ void hist_replay_at(float *hist, const float *src,
                                                      const float *xc_raw,
                                                      const int32_t *accepted, int64_t n_units,
                                                      int conv_dim, int M, int32_t *status,
                                                      int64_t u, int c4, bool report) {
  constexpr int NPREV = 3;             // ck = 4
  int acc = accepted[u];
  if (acc < 0 || acc > M) {            // device-supplied counts: refuse the unit
    if (status != nullptr && report) status[0] = 1;
    acc = 0;
  }
  if (4 * c4 >= conv_dim) return;
  if (acc == 0 && src == hist) return; // in place, nothing accepted: unchanged
  const int64_t hbase = u * (int64_t)NPREV * conv_dim + 4 * c4;
  f4 fr[NPREV];
#pragma unroll
  for (int j = 0; j < NPREV; j++) {
    const int idx = acc + j;
    const float *from = idx < NPREV ? src + hbase + (int64_t)idx * conv_dim
                                    : xc_raw + ((int64_t)(idx - NPREV) * n_units + u) * conv_dim + 4 * c4;
    fr[j] = ld4(from);
  }
#pragma unroll
  for (int j = 0; j < NPREV; j++) st4(hist + hbase + (int64_t)j * conv_dim, fr[j]);
}

// History work of an M-step launch: item i of LANES float4 channels.
template <int LANES>
static __device__ __forceinline__ void hist_item(const RecurArgs &a, int64_t item) {
  const int64_t per_unit = (a.conv_dim / 4 + LANES - 1) / LANES;
  const int64_t u = item / per_unit;
  const int c4 = (int)(item - u * per_unit) * LANES + (int)threadIdx.x;
  hist_replay_at(a.hist, a.hist_src, a.xc_raw, a.steps, a.n_units, a.conv_dim, a.M, a.status, u,
                 c4, threadIdx.x == 0);
}

// ----- wide geometry, several steps ---------------------------------------
//
// Up to MC steps per call for launches with few tiles (a handful of units,
// where the deep geometry leaves most CUs idle and each step waits on a
// 256-lane tile): the wide lane layout, four times the lanes per tile, with
// the deep kernel's step loop (all rows staged at once; the output of step
// m - 1 is completed by wave 1 in parallel with wave 0's S^T k of step m).
// Same canonical tree, so the same bits as the deep and single-step kernels.
// Serves the gated calls and kd = 64; ungated kd = 128 calls on few tiles
// take the split geometry below.
template <int KD, bool GATED>
__global__ __launch_bounds__(Geo<KD>::LANES) void recur_widem_kernel(RecurArgs a) {
  using G = Geo<KD>;
  constexpr int LANES = G::LANES;
  __shared__ Stage<KD, GATED> sb;
  __shared__ f4 s_red_k[G::NW][G::CG];
  __shared__ f4 s_red_o[G::NW][G::CG];
  __shared__ f4 s_tmp[G::CG];
  // gated: the folded output rows, normalised after the last step (the
  // RMSNorm of each row then runs on its own wave, off the step chain)
  __shared__ f4 s_orow[GATED ? MC : 1][G::CG];

  if (a.hist != nullptr) {             // uniform per workgroup
    const int64_t bid = xcd_contiguous(blockIdx.x, gridDim.x);
    if (bid >= a.tile_wgs) {
      hist_item<LANES>(a, bid - a.tile_wgs);
      return;
    }
  }
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int cg = t % G::CG, rg = t / G::CG;
  const TileIdx ti = tile_index(a, KD * KD);
  const int steps = ti.steps;          // 0 .. M <= MC
  // an in-place update with nothing to run leaves the tile as it is
  if (steps == 0 && a.S_src == a.S_dst && a.snap == nullptr) return;
  const rsrc_t src = buf_rsrc(a.S_src + ti.tile_off, KD * KD * 4);
  const int lane_off = (rg * KD + 4 * cg) * 4;

  ChunkRegs<KD, LANES, GATED> cr;
  if (steps > 0) chunk_load<KD, LANES, GATED>(cr, a, t, ti.unit, ti.head, ti.hh, 0, steps);

  // few tiles: the state stays cache-resident between calls (default policy)
  f4 s[G::R];
#pragma unroll
  for (int j = 0; j < G::R; j++) s[j] = ld_stream<true>(src, lane_off, j * (G::RG * KD * 4));
  if (a.snap != nullptr) {            // fused mark: the tile as loaded, before the steps
    const rsrc_t snp = buf_rsrc(a.snap + ti.tile_off, KD * KD * 4);
#pragma unroll
    for (int j = 0; j < G::R; j++) st_stream<false>(snp, lane_off, j * (G::RG * KD * 4), s[j]);
  }

  const float *zprev = nullptr;
  if (steps > 0) {
    chunk_store<KD, LANES, GATED>(sb, cr, t, steps);
    __syncthreads();
    for (int r = 0; r < steps; r++) {
      const float alpha = sb.alpha[r];
      const f4 kk = lds4(&sb.k[r][rg * 4]);
      // decay, then S^T k over the decayed state
      f4 p = splat(0.0f);
#pragma unroll
      for (int j = 0; j < G::R; j++) {
        s[j] = s[j] * alpha;
        p = fma4(s[j], splat(kk[j]), p);
      }
      p = wave_fold<KD>(p);
      if (lane < G::CG) s_red_k[wave][lane] = p;
      __syncthreads();
      if (wave == 0) {
        const f4 kv = tile_sum<KD>(s_red_k, lane);
        if (lane < G::CG) s_tmp[lane] = (lds4(&sb.v[r][4 * lane]) - kv) * sb.beta[r];
      } else if (wave == 1 && r > 0 && a.o != nullptr) {
        // the previous step's output, in parallel with wave 0's S^T k
        const f4 ov = tile_sum<KD>(s_red_o, lane);
        if constexpr (GATED) {
          if (lane < G::CG) s_orow[r - 1][lane] = ov;
        } else {
          const int64_t prow = (int64_t)(r - 1) * a.n_units + ti.unit;
          emit_o<KD, GATED>(a, prow, ti.head, lane % G::CG, lane < G::CG, ov, zprev);
        }
      }
      __syncthreads();
      const f4 tmp = s_tmp[cg];
      const f4 qq = lds4(&sb.q[r][rg * 4]);
      // rank-1 update, then S^T q with the updated state
      p = splat(0.0f);
#pragma unroll
      for (int j = 0; j < G::R; j++) {
        s[j] = fma4(splat(kk[j]), tmp, s[j]);
        p = fma4(s[j], splat(qq[j]), p);
      }
      p = wave_fold<KD>(p);
      if (lane < G::CG) s_red_o[wave][lane] = p;
      if constexpr (GATED) zprev = &sb.z[r][0];
    }
  }

  if (a.S_dst != nullptr) {            // null: outputs only, the state is left as it was
    const rsrc_t dst = buf_rsrc(a.S_dst + ti.tile_off, KD * KD * 4);
#pragma unroll
    for (int j = 0; j < G::R; j++) st_stream<true>(dst, lane_off, j * (G::RG * KD * 4), s[j]);
  }

  if (steps > 0) {
    __syncthreads();
    if (wave == 0 && a.o != nullptr) {
      const f4 ov = tile_sum<KD>(s_red_o, lane);
      if constexpr (GATED) {
        if (lane < G::CG) s_orow[steps - 1][lane] = ov;
      } else {
        const int64_t urow = (int64_t)(steps - 1) * a.n_units + ti.unit;
        emit_o<KD, GATED>(a, urow, ti.head, lane % G::CG, lane < G::CG, ov, zprev);
      }
    }
    if constexpr (GATED) {
      __syncthreads();
      if (a.o != nullptr) {
        for (int r = wave; r < steps; r += G::NW) {
          const int64_t urow = (int64_t)r * a.n_units + ti.unit;
          emit_o<KD, GATED>(a, urow, ti.head, lane % G::CG, lane < G::CG,
                            s_orow[r][lane % G::CG], &sb.z[r][0]);
        }
      }
    }
  }
}

// ----- deep geometry -------------------------------------------------------
//
// Lane (cg, L) holds row groups 4L .. 4L+3 (16 rows x 4 columns) and forms
// their p's itself.  kd = 128: the W partials go through LDS to wave 0 as in
// the wide kernel (2 barriers per step); kd = 64: the whole tile is one wave
// and both read-outs finish with in-wave shuffles (no barrier per step).
template <int KD>
static __device__ __forceinline__ void deep_partials(const f4 (&p)[4], f4 &w0, f4 &w1) {
  if (KD == 128) {
    w0 = p[0] + p[1];
    w1 = p[2] + p[3];
  } else {
    w0 = (p[0] + p[1]) + (p[2] + p[3]);
  }
}

template <int KD, bool MULTI, bool GATED, bool FUSED = false>
__global__ __launch_bounds__(Deep<KD>::LANES) void recur_deep_kernel(RecurArgs a) {
  using D = Deep<KD>;
  constexpr int LANES = D::LANES, RG = Canon<KD>::RG, CG = D::CG;
  constexpr bool XWAVE = KD == 128;             // partials cross waves
  __shared__ Stage<KD, GATED> st[MULTI ? 2 : 1];
  __shared__ f4 s_red_k[XWAVE ? Canon<KD>::NWP : 1][CG];
  __shared__ f4 s_red_o[XWAVE ? Canon<KD>::NWP : 1][CG];
  __shared__ f4 s_tmp[CG];

  if (a.hist != nullptr) {             // uniform per workgroup
    const int64_t bid = xcd_contiguous(blockIdx.x, gridDim.x);
    if (bid >= a.tile_wgs) {
      hist_item<LANES>(a, bid - a.tile_wgs);
      return;
    }
  }
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int cg = t % CG, L = t / CG;
  const TileIdx ti = tile_index(a, KD * KD);
  const int steps = ti.steps;
  // an in-place update with nothing to run leaves the tile as it is (a fused
  // call still runs the next verify's rows)
  if (!FUSED && steps == 0 && a.S_src == a.S_dst && a.snap == nullptr) return;
  // element (i, j) of this lane: row 4L + i + RG*j
  const rsrc_t src = buf_rsrc(a.S_src + ti.tile_off, KD * KD * 4);
  const int lane_off = ((4 * L) * KD + 4 * cg) * 4;

  ChunkRegs<KD, LANES, GATED> cr;
  if (steps > 0) chunk_load<KD, LANES, GATED>(cr, a, t, ti.unit, ti.head, ti.hh, 0, steps < MC ? steps : MC);

  f4 s[4][4];
#pragma unroll
  for (int j = 0; j < 4; j++)
#pragma unroll
    for (int i = 0; i < 4; i++) s[i][j] = ld_stream(src, lane_off, (i + RG * j) * KD * 4);
  if (a.snap != nullptr) {            // fused mark: the tile as loaded, before the steps
    const rsrc_t snp = buf_rsrc(a.snap + ti.tile_off, KD * KD * 4);
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int i = 0; i < 4; i++) st_stream(snp, lane_off, (i + RG * j) * KD * 4, s[i][j]);
  }

  // the step loop over nst rows of ra's inputs, outputs to ra.o when it is
  // non-null (the first chunk already in cr); emit_last then writes the last
  // row's output, which the cross-wave kernel holds back one step
  const float *zprev = nullptr;
  auto run = [&](const RecurArgs &ra, int nst) {
    int buf = 0;
    for (int m0 = 0; m0 < nst; m0 += MC) {
      const int nr = nst - m0 < MC ? nst - m0 : MC;
      Stage<KD, GATED> &sb = st[MULTI ? buf : 0];
      chunk_store<KD, LANES, GATED>(sb, cr, t, nr);
      __syncthreads();
      if (MULTI && m0 + MC < nst) {
        const int nn = nst - m0 - MC;
        chunk_load<KD, LANES, GATED>(cr, ra, t, ti.unit, ti.head, ti.hh, m0 + MC, nn < MC ? nn : MC);
      }
      for (int r = 0; r < nr; r++) {
        const int m = m0 + r;
        const int64_t urow = (int64_t)m * ra.n_units + ti.unit;
        const float alpha = sb.alpha[r];
        f4 p[4], w0, w1 = splat(0.0f);
        f4 kkr[4];
#pragma unroll
        for (int i = 0; i < 4; i++) kkr[i] = lds4(&sb.k[r][(4 * L + i) * 4]);
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const f4 kk = kkr[i];
          p[i] = splat(0.0f);
#pragma unroll
          for (int j = 0; j < 4; j++) {
            s[i][j] = s[i][j] * alpha;
            p[i] = fma4(s[i][j], splat(kk[j]), p[i]);
          }
        }
        deep_partials<KD>(p, w0, w1);
        f4 tmp;
        if (XWAVE) {
          s_red_k[2 * L][cg] = w0;
          s_red_k[2 * L + 1][cg] = w1;
          __syncthreads();
          if (wave == 0) {
            const f4 kv = tile_sum<KD>(s_red_k, lane);
            if (lane < CG) s_tmp[lane] = (lds4(&sb.v[r][4 * lane]) - kv) * sb.beta[r];
          } else if (wave == 1 && m > 0 && ra.o != nullptr) {
            // the previous step's output, in parallel with wave 0's S^T k
            const f4 ov = tile_sum<KD>(s_red_o, lane);
            const int64_t prow = (int64_t)(m - 1) * ra.n_units + ti.unit;
            emit_o<KD, GATED>(ra, prow, ti.head, lane % CG, lane < CG, ov, zprev);
          }
          __syncthreads();
          tmp = s_tmp[cg];
        } else {
          const f4 kv = wave_fold<KD>(w0);
          tmp = (lds4(&sb.v[r][4 * cg]) - kv) * sb.beta[r];
        }
        // rank-1 update, then S^T q with the updated state
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const f4 kk = kkr[i];
          const f4 qq = lds4(&sb.q[r][(4 * L + i) * 4]);
          p[i] = splat(0.0f);
#pragma unroll
          for (int j = 0; j < 4; j++) {
            s[i][j] = fma4(splat(kk[j]), tmp, s[i][j]);
            p[i] = fma4(s[i][j], splat(qq[j]), p[i]);
          }
        }
        deep_partials<KD>(p, w0, w1);
        if (XWAVE) {
          s_red_o[2 * L][cg] = w0;
          s_red_o[2 * L + 1][cg] = w1;
        } else if (ra.o != nullptr) {
          const f4 ov = wave_fold<KD>(w0);
          emit_o<KD, GATED>(ra, urow, ti.head, cg, L == 0, ov, &sb.z[GATED ? r : 0][0]);
        }
        if constexpr (GATED) zprev = &sb.z[r][0];
      }
      buf ^= 1;
    }
  };
  auto emit_last = [&](const RecurArgs &ra, int nst) {
    if (XWAVE && nst > 0) {
      __syncthreads();
      if (wave == 0 && ra.o != nullptr) {
        const f4 ov = tile_sum<KD>(s_red_o, lane);
        const int64_t urow = (int64_t)(nst - 1) * ra.n_units + ti.unit;
        emit_o<KD, GATED>(ra, urow, ti.head, lane % CG, lane < CG, ov, zprev);
      }
    }
  };

  run(a, steps);
  // null: outputs only, the state is left as it was; a fused call with no
  // accepted rows leaves it too
  if (a.S_dst != nullptr && (!FUSED || steps > 0)) {
    const rsrc_t dst = buf_rsrc(a.S_dst + ti.tile_off, KD * KD * 4);
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int i = 0; i < 4; i++) st_stream(dst, lane_off, (i + RG * j) * KD * 4, s[i][j]);
  }
  emit_last(a, steps);

  if constexpr (FUSED) {
    // the draft rows of the next verify, from the committed state in registers
    RecurArgs b = a;
    b.q = a.q2;
    b.k = a.k2;
    b.v = a.v2;
    b.g = a.g2;
    b.beta = a.beta2;
    b.o = a.o2;
    b.M = a.M2;
    b.steps = nullptr;
    __syncthreads();                   // the stage and fold buffers are reused
    chunk_load<KD, LANES, GATED>(cr, b, t, ti.unit, ti.head, ti.hh, 0, b.M < MC ? b.M : MC);
    zprev = nullptr;
    run(b, b.M);
    emit_last(b, b.M);
  }
}

// ----- split geometry, several steps (kd = 128, few tiles) ----------------
//
// With a sequence or two per launch, the wide M-step kernel runs one
// 1024-lane workgroup per tile: four waves per SIMD on a few dozen CUs, and
// each step waits on two barriers and one wave's fold.  Here SPLIT_NS
// workgroups serve a tile, one per KD / SPLIT_NS columns.  The columns of S
// are independent (S^T k and S^T q reduce over rows only), so a workgroup
// holds every row of its columns and needs no other.  Lane t is (row group
// t / SPLIT_CG, column group t % SPLIT_CG): the W partial of row groups 2w
// and 2w + 1 pairs lanes t and t ^ SPLIT_CG; the 16 W partials go through LDS
// (double-buffered by step parity), and every lane folds them for its own
// column group (H0, H1, H0 + H1).  That is the canonical tree, so the bits
// are those of the other geometries, with one barrier per step.  Ungated
// calls only: the gated RMSNorm needs the whole head's output in one
// workgroup (a second pass over the raw outputs cost more than it saved).
constexpr int SPLIT_NS = 4;                                  // workgroups per tile
constexpr int SPLIT_CG = Canon<128>::CG / SPLIT_NS;          // column groups per workgroup
constexpr int SPLIT_LANES = Canon<128>::RG * SPLIT_CG;       // 256

// Left folds of W partials 0..7 and 8..15 for column group lane % SPLIT_CG,
// then their sum (lanes l and l ^ SPLIT_CG hold the two folds).
static __device__ __forceinline__ f4 split_sum(const f4 (*red)[SPLIT_CG], int lane) {
  constexpr int PER = Canon<128>::NWP / 2;
  const int h = (lane / SPLIT_CG) & 1, c = lane % SPLIT_CG;
  f4 acc = red[h * PER][c];
#pragma unroll
  for (int i = 1; i < PER; i++) acc = acc + red[h * PER + i][c];
  acc.x = acc.x + lane_xor<SPLIT_CG>(acc.x);
  acc.y = acc.y + lane_xor<SPLIT_CG>(acc.y);
  acc.z = acc.z + lane_xor<SPLIT_CG>(acc.z);
  acc.w = acc.w + lane_xor<SPLIT_CG>(acc.w);
  return acc;
}

// p[rg] + p[rg ^ 1]: the partner row group sits SPLIT_CG lanes away
static __device__ __forceinline__ f4 split_pair(f4 p) {
  p.x = p.x + lane_xor<SPLIT_CG>(p.x);
  p.y = p.y + lane_xor<SPLIT_CG>(p.y);
  p.z = p.z + lane_xor<SPLIT_CG>(p.z);
  p.w = p.w + lane_xor<SPLIT_CG>(p.w);
  return p;
}

__global__ __launch_bounds__(SPLIT_LANES) void recur_split_kernel(RecurArgs a) {
  constexpr int KD = 128, RG = Canon<KD>::RG, NWP = Canon<KD>::NWP;
  __shared__ Stage<KD, false> sb;
  __shared__ f4 s_red_k[2][NWP][SPLIT_CG];
  __shared__ f4 s_red_o[2][NWP][SPLIT_CG];

  const int64_t bid = xcd_contiguous(blockIdx.x, gridDim.x);
  if (a.hist != nullptr && bid >= a.tile_wgs) {   // uniform per workgroup
    hist_item<SPLIT_LANES>(a, bid - a.tile_wgs);
    return;
  }
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int cg = t % SPLIT_CG, rg = t / SPLIT_CG;
  // the tile and this workgroup's columns (the SPLIT_NS workgroups of a tile
  // are adjacent, so they share an XCD and its L2 copy of q, k, v)
  const int64_t tile = bid / SPLIT_NS;
  const int col0 = 4 * ((int)(bid - tile * SPLIT_NS) * SPLIT_CG + cg);
  const int64_t unit = tile / a.vh;
  const int head = (int)(tile - unit * a.vh);
  const int hh = head / (a.vh / a.kh);
  int steps = a.steps ? a.steps[unit] : a.M;
  if (steps < 0 || steps > a.M) {      // device-supplied counts: refuse the unit
    if (a.status != nullptr && t == 0) a.status[0] = 1;
    steps = 0;
  }
  if (steps == 0 && a.S_src == a.S_dst && a.snap == nullptr) return;
  const int64_t tile_off = tile * (int64_t)(KD * KD);
  const rsrc_t src = buf_rsrc(a.S_src + tile_off, KD * KD * 4);
  const int lane_off = (rg * KD + col0) * 4;

  ChunkRegs<KD, SPLIT_LANES, false> cr;
  if (steps > 0) chunk_load<KD, SPLIT_LANES, false>(cr, a, t, unit, head, hh, 0, steps);
  f4 s[4];
#pragma unroll
  for (int j = 0; j < 4; j++) s[j] = ld_stream<true>(src, lane_off, j * (RG * KD * 4));
  if (a.snap != nullptr) {            // fused mark: the tile as loaded, before the steps
    const rsrc_t snp = buf_rsrc(a.snap + tile_off, KD * KD * 4);
#pragma unroll
    for (int j = 0; j < 4; j++) st_stream<false>(snp, lane_off, j * (RG * KD * 4), s[j]);
  }
  // the output of row r for this workgroup's columns
  auto emit = [&](int r, int par) {
    const f4 ov = split_sum(s_red_o[par], lane);
    if (lane < SPLIT_CG) {
      const int64_t urow = (int64_t)r * a.n_units + unit;
      st4(a.o + (urow * a.vh + head) * KD + 4 * ((col0 / 4 - cg) + lane), ov);
    }
  };

  if (steps > 0) {
    chunk_store<KD, SPLIT_LANES, false>(sb, cr, t, steps);
    __syncthreads();
    for (int r = 0; r < steps; r++) {
      const int par = r & 1;
      const float alpha = sb.alpha[r];
      const f4 kk = lds4(&sb.k[r][rg * 4]);
      // decay, then S^T k partials over the decayed state
      f4 p = splat(0.0f);
#pragma unroll
      for (int j = 0; j < 4; j++) {
        s[j] = s[j] * alpha;
        p = fma4(s[j], splat(kk[j]), p);
      }
      p = split_pair(p);
      if ((rg & 1) == 0) s_red_k[par][rg >> 1][cg] = p;
      __syncthreads();
      // the previous row's output, beside every wave's fold of S^T k
      if (wave == 1 && r > 0 && a.o != nullptr) emit(r - 1, par ^ 1);
      const f4 kv = split_sum(s_red_k[par], lane);
      const f4 tmp = (lds4(&sb.v[r][col0]) - kv) * sb.beta[r];
      const f4 qq = lds4(&sb.q[r][rg * 4]);
      // rank-1 update, then S^T q partials with the updated state
      p = splat(0.0f);
#pragma unroll
      for (int j = 0; j < 4; j++) {
        s[j] = fma4(splat(kk[j]), tmp, s[j]);
        p = fma4(s[j], splat(qq[j]), p);
      }
      p = split_pair(p);
      if ((rg & 1) == 0) s_red_o[par][rg >> 1][cg] = p;
    }
  }

  if (a.S_dst != nullptr) {            // null: outputs only, the state is left as it was
    const rsrc_t dst = buf_rsrc(a.S_dst + tile_off, KD * KD * 4);
#pragma unroll
    for (int j = 0; j < 4; j++) st_stream<true>(dst, lane_off, j * (RG * KD * 4), s[j]);
  }
  if (steps > 0) {
    __syncthreads();
    if (wave == 0 && a.o != nullptr) emit(steps - 1, (steps - 1) & 1);
  }
}

// Launches of fewer than kWidemBelow tiles with M <= MC rows per unit and
// at most kFewTileRows tile-rows (tiles x M) run the split geometry (kd =
// 128, ungated); otherwise single steps run the wide geometry, and M >= 2 rows
// the wide one step after step (the same few-tile bound) or the deep
// geometry.  The same bits whichever serves a call.  The bound is where the
// deep kernel's throughput overtakes the few-tile kernels' latency (step_m at
// M = 8: split 13.4 against 14.8 us at 192 tiles, 20.6 against 18.0 at 384;
// at M = 2 split is ahead up to 1008 tiles).
constexpr int64_t kWidemBelow = 1024;
constexpr int64_t kFewTileRows = 2048;

int recur_lanes(int kd) { return kd == 128 ? Geo<128>::LANES : Geo<64>::LANES; }

// Workgroups that replay the history after the tiles' workgroups.
static int64_t hist_wgs(const RecurArgs &a, int lanes) {
  return a.hist == nullptr ? 0 : a.n_units * ((a.conv_dim / 4 + lanes - 1) / lanes);
}

template <int KD, bool GATED>
static void launch_recur_kd(RecurArgs a, int64_t tiles, hipStream_t s) {
  const dim3 grid((unsigned)tiles);
  a.tile_wgs = tiles;
  const bool few = a.M <= MC && tiles < kWidemBelow && tiles * a.M <= kFewTileRows;
  if (KD == 128 && !GATED && few) {
    a.tile_wgs = tiles * SPLIT_NS;
    const dim3 g2((unsigned)(a.tile_wgs + hist_wgs(a, SPLIT_LANES)));
    hipLaunchKernelGGL(recur_split_kernel, g2, dim3(SPLIT_LANES), 0, s, a);
  } else if (a.M == 1) {
    // kd = 64: four adjacent heads of one unit per workgroup, so that a
    // workgroup streams 64 KiB of consecutive state like a kd = 128 one
    constexpr int TPW = KD == 64 ? 4 : 1;
    if (TPW > 1 && a.vh % TPW == 0) {
      const dim3 g4((unsigned)(tiles / TPW));
      if (tiles * KD * KD * 4 <= RESIDENT_MAX_BYTES)
        hipLaunchKernelGGL((recur_wide_kernel<KD, true, GATED, TPW>), g4,
                           dim3(Geo<KD>::LANES * TPW), 0, s, a);
      else
        hipLaunchKernelGGL((recur_wide_kernel<KD, false, GATED, TPW>), g4,
                           dim3(Geo<KD>::LANES * TPW), 0, s, a);
    } else if (tiles * KD * KD * 4 <= RESIDENT_MAX_BYTES) {
      hipLaunchKernelGGL((recur_wide_kernel<KD, true, GATED, 1>), grid, dim3(Geo<KD>::LANES), 0,
                         s, a);
    } else {
      hipLaunchKernelGGL((recur_wide_kernel<KD, false, GATED, 1>), grid, dim3(Geo<KD>::LANES), 0,
                         s, a);
    }
  } else if (few) {
    const dim3 g2((unsigned)(tiles + hist_wgs(a, Geo<KD>::LANES)));
    hipLaunchKernelGGL((recur_widem_kernel<KD, GATED>), g2, dim3(Geo<KD>::LANES), 0, s, a);
  } else {
    const dim3 g2((unsigned)(tiles + hist_wgs(a, Deep<KD>::LANES)));
    if (a.M <= MC)
      hipLaunchKernelGGL((recur_deep_kernel<KD, false, GATED>), g2, dim3(Deep<KD>::LANES), 0, s, a);
    else
      hipLaunchKernelGGL((recur_deep_kernel<KD, true, GATED>), g2, dim3(Deep<KD>::LANES), 0, s, a);
  }
}

int launch_recur(int kd, const float *S_src, float *S_dst, const float *q,
                 const float *k, const float *v, const float *g,
                 const float *beta, float *o, const int32_t *steps,
                 int64_t n_units, int vh, int kh, int M, hipStream_t s,
                 const float *z, const float *norm_w, float eps, float *snap,
                 int32_t *status, float *hist, const float *hist_src, const float *xc_raw,
                 int conv_dim) {
  RecurArgs a{S_src, S_dst, q, k, v, g, beta, o, steps, z, norm_w, eps, snap, status,
              n_units, vh, kh, M, nullptr, nullptr, nullptr, 0, 0};
  const int64_t tiles = n_units * vh;
  if (tiles <= 0) return 0;
  if (hist != nullptr) {
    if (M == 1) {
      // single steps run the wide kernel, which has no history part: the
      // replay is its own launch
      const int rc = launch_hist_replay(hist, hist_src, xc_raw, steps, n_units, conv_dim, M,
                                        status, s);
      if (rc) return rc;
    } else {
      a.hist = hist;
      a.hist_src = hist_src;
      a.xc_raw = xc_raw;
      a.conv_dim = conv_dim;
    }
  }
  const bool gated = z != nullptr;
  if (kd == 128) {
    if (gated)
      launch_recur_kd<128, true>(a, tiles, s);
    else
      launch_recur_kd<128, false>(a, tiles, s);
  } else {
    if (gated)
      launch_recur_kd<64, true>(a, tiles, s);
    else
      launch_recur_kd<64, false>(a, tiles, s);
  }
  return (int)hipGetLastError();
}

// gdn_commit followed by gdn_verify_m, ungated, in one pass over the state:
// the M-step kernel applies steps[u] rows of the first set, stores the tile,
// and runs the M2 rows of the second set from the registers (outputs only).
// Launches the few-tile kernels would serve run as those two launches
// instead (the same bits).
int launch_commit_verify(int kd, float *S, const float *q, const float *k, const float *v,
                         const float *g, const float *beta, const int32_t *steps,
                         int32_t *status, float *hist, const float *xc_raw, int conv_dim,
                         int64_t n_units, int vh, int kh, int M, const float *q2,
                         const float *k2, const float *v2, const float *g2,
                         const float *beta2, float *o2, int M2, hipStream_t s) {
  const int64_t tiles = n_units * vh;
  if (tiles <= 0) return 0;
  const bool few = tiles < kWidemBelow && (int64_t)(M > M2 ? M : M2) * tiles <= kFewTileRows;
  if (few) {
    int rc = launch_recur(kd, S, S, q, k, v, g, beta, nullptr, steps, n_units, vh, kh, M, s,
                          nullptr, nullptr, 0.0f, nullptr, status, hist, hist, xc_raw, conv_dim);
    if (rc) return rc;
    return launch_recur(kd, S, nullptr, q2, k2, v2, g2, beta2, o2, nullptr, n_units, vh, kh, M2,
                        s);
  }
  RecurArgs a{S, S, q, k, v, g, beta, nullptr, steps, nullptr, nullptr, 0.0f, nullptr, status,
              n_units, vh, kh, M, hist, hist, xc_raw, conv_dim, tiles};
  a.q2 = q2;
  a.k2 = k2;
  a.v2 = v2;
  a.g2 = g2;
  a.beta2 = beta2;
  a.o2 = o2;
  a.M2 = M2;
  const bool multi = M > MC || M2 > MC;
  if (kd == 128) {
    const dim3 grid((unsigned)(tiles + hist_wgs(a, Deep<128>::LANES)));
    if (multi)
      hipLaunchKernelGGL((recur_deep_kernel<128, true, false, true>), grid,
                         dim3(Deep<128>::LANES), 0, s, a);
    else
      hipLaunchKernelGGL((recur_deep_kernel<128, false, false, true>), grid,
                         dim3(Deep<128>::LANES), 0, s, a);
  } else {
    const dim3 grid((unsigned)(tiles + hist_wgs(a, Deep<64>::LANES)));
    if (multi)
      hipLaunchKernelGGL((recur_deep_kernel<64, true, false, true>), grid, dim3(Deep<64>::LANES),
                         0, s, a);
    else
      hipLaunchKernelGGL((recur_deep_kernel<64, false, false, true>), grid,
                         dim3(Deep<64>::LANES), 0, s, a);
  }
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------
// Streaming copy (mark, and the read+write floor): one workgroup per 64 KiB
// chunk, 1024 lanes x 4 x 128-bit, chunks laid out contiguously per XCD.
// ---------------------------------------------------------------------------

constexpr int COPY_LANES = 1024;
constexpr int COPY_F4 = 4;                          // float4 per lane per chunk
constexpr int64_t COPY_CHUNK4 = COPY_LANES * COPY_F4;  // float4 per chunk

__global__ __launch_bounds__(COPY_LANES) void copy_kernel(float *dst, const float *src,
                                                          int64_t n4, int64_t n) {
  const int64_t c = xcd_contiguous(blockIdx.x, gridDim.x);
  // this chunk's float4 range [c*COPY_CHUNK4, end); buffer bounds = its bytes
  const int64_t first = c * COPY_CHUNK4;
  const int64_t cnt = n4 - first < COPY_CHUNK4 ? n4 - first : COPY_CHUNK4;
  const rsrc_t rs = buf_rsrc(src + 4 * first, (int)(cnt * 16));
  const rsrc_t rd = buf_rsrc(dst + 4 * first, (int)(cnt * 16));
  f4 x[COPY_F4];
#pragma unroll
  for (int u = 0; u < COPY_F4; u++) {
    const int i = threadIdx.x + u * COPY_LANES;
    if (i < cnt) x[u] = ld_stream(rs, threadIdx.x * 16, u * COPY_LANES * 16);
  }
#pragma unroll
  for (int u = 0; u < COPY_F4; u++) {
    const int i = threadIdx.x + u * COPY_LANES;
    if (i < cnt) st_stream(rd, threadIdx.x * 16, u * COPY_LANES * 16, x[u]);
  }
  if (c == 0 && threadIdx.x < (n - 4 * n4)) dst[4 * n4 + threadIdx.x] = src[4 * n4 + threadIdx.x];
}

int launch_copy(float *dst, const float *src, int64_t n, hipStream_t s) {
  if (n <= 0) return 0;
  const int64_t n4 = n / 4;
  int64_t blocks = (n4 + COPY_CHUNK4 - 1) / COPY_CHUNK4;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(COPY_LANES), 0, s, dst, src, n4, n);
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------
// Read-only floor: stream n floats with 128-bit non-temporal loads, 256 lanes
// x 32 loads per workgroup (the shape that reads fastest), and write one
// 32-bit word per 128 KiB chunk, the XOR of the chunk's words, so that the
// loads cannot be dropped and the result can be checked.
// ---------------------------------------------------------------------------

constexpr int READ_LANES = 256;
constexpr int READ_F4 = 32;
constexpr int64_t READ_CHUNK4 = READ_LANES * READ_F4;   // float4 per chunk

__global__ __launch_bounds__(READ_LANES) void read_kernel(const float *src, int64_t n4,
                                                          int64_t n, uint32_t *words) {
  __shared__ uint32_t s_x[READ_LANES / 64];
  const int64_t c = xcd_contiguous(blockIdx.x, gridDim.x);
  const int64_t first = c * READ_CHUNK4;
  const int64_t cnt = n4 - first < READ_CHUNK4 ? n4 - first : READ_CHUNK4;
  // loads past cnt are outside the buffer's bounds and return zeros
  const rsrc_t rs = buf_rsrc(src + 4 * first, (int)(cnt > 0 ? cnt * 16 : 0));
  f4 x[READ_F4];
#pragma unroll
  for (int u = 0; u < READ_F4; u++) x[u] = ld_stream(rs, threadIdx.x * 16, u * READ_LANES * 16);
  uint32_t h = 0;
#pragma unroll
  for (int u = 0; u < READ_F4; u++)
    h ^= __float_as_uint(x[u].x) ^ __float_as_uint(x[u].y) ^ __float_as_uint(x[u].z) ^
         __float_as_uint(x[u].w);
  // the last chunk also takes the 0..3 floats past the last whole float4
  if (c == gridDim.x - 1 && threadIdx.x < n - 4 * n4) h ^= __float_as_uint(src[4 * n4 + threadIdx.x]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) h ^= (uint32_t)__shfl_xor((int)h, off);
  if ((threadIdx.x & 63) == 0) s_x[threadIdx.x >> 6] = h;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < READ_LANES / 64; i++) w ^= s_x[i];
    words[c] = w;
  }
}

// chunk c holds floats [4 READ_CHUNK4 c, 4 READ_CHUNK4 (c + 1)); the last one
// may hold no whole float4, only the 1..3 floats past the last one
int64_t read_chunks(int64_t n) {
  const int64_t c = (n + 4 * READ_CHUNK4 - 1) / (4 * READ_CHUNK4);
  return c < 1 ? 1 : c;
}

int launch_read(const float *src, int64_t n, uint32_t *words, hipStream_t s) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(read_kernel, dim3((unsigned)read_chunks(n)), dim3(READ_LANES), 0, s, src,
                     n / 4, n, words);
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------
// Per-unit step counts from a host array, handed to the device by value: the
// counts of up to COUNT_CHUNK units travel in one launch's kernel arguments,
// which the runtime copies when the launch is enqueued, so the host array is
// no longer read once the call returns (no host-memory copy is left pending).
// ---------------------------------------------------------------------------

constexpr int COUNT_CHUNK = 1024;
struct CountChunk {
  uint8_t c[COUNT_CHUNK];   // counts 0..64
};

__global__ __launch_bounds__(256) void count_stage_kernel(int32_t *dst, int n, CountChunk ch) {
  for (int i = threadIdx.x; i < n; i += 256) dst[i] = ch.c[i];
}

int launch_stage_counts(int32_t *dst, const int32_t *host, int64_t n, hipStream_t s) {
  for (int64_t base = 0; base < n; base += COUNT_CHUNK) {
    const int len = (int)(n - base < COUNT_CHUNK ? n - base : COUNT_CHUNK);
    CountChunk ch;
    for (int i = 0; i < COUNT_CHUNK; i++) ch.c[i] = i < len ? (uint8_t)host[base + i] : 0;
    hipLaunchKernelGGL(count_stage_kernel, dim3(1), dim3(256), 0, s, dst + base, len, ch);
    const int rc = (int)hipGetLastError();
    if (rc) return rc;
  }
  return 0;
}

// ---------------------------------------------------------------------------
// Library-owned count area for callers that cannot allocate: a file-scope
// device array, one copy per GPU, whose device address is looked up once per
// device (the array's name is a host-side stand-in in host code and must not
// be passed to a kernel).  Every call on a GPU shares that GPU's copy.
// ---------------------------------------------------------------------------

static __device__ __align__(256) int32_t scratch[kStaticCountsMax];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t *g_scratch_ptr[kMaxDevices];
}  // namespace

int static_counts_area(int32_t **area) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return e != hipSuccess ? (int)e : -1;
    g_scratch_ptr[dev] = static_cast<int32_t *>(p);
  }
  *area = g_scratch_ptr[dev];
  return 0;
}

// ---------------------------------------------------------------------------
// Conv-history rollback: pure data movement, bit-exact.
// ---------------------------------------------------------------------------

// One-dimensional grid, `chunks` workgroups of 256 float4 channels per unit
// (a second grid dimension would cap the unit count at 65536).
__global__ __launch_bounds__(256) void hist_replay_kernel(float *hist, const float *src,
                                                          const float *xc_raw,
                                                          const int32_t *accepted,
                                                          int64_t n_units, int conv_dim, int M,
                                                          int32_t *status, uint32_t chunks) {
  const uint32_t u = blockIdx.x / chunks, c = blockIdx.x - u * chunks;
  hist_replay_at(hist, src, xc_raw, accepted, n_units, conv_dim, M, status, u,
                 (int)(c * 256 + threadIdx.x), threadIdx.x == 0 && c == 0);
}

int launch_hist_replay(float *hist, const float *src, const float *xc_raw,
                       const int32_t *accepted, int64_t n_units, int conv_dim, int M,
                       int32_t *status, hipStream_t s) {
  if (n_units <= 0) return 0;
  const uint32_t chunks = (uint32_t)((conv_dim / 4 + 255) / 256);
  const dim3 grid((unsigned)(n_units * chunks));
  hipLaunchKernelGGL(hist_replay_kernel, grid, dim3(256), 0, s, hist, src, xc_raw, accepted,
                     n_units, conv_dim, M, status, chunks);
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------
// Front end, kernel A: paired GEMV (a = Wa x, b = Wb x) with the gate / beta
// transform in the epilogue ("Kestrel_VLLM #27", section 4.2: both
// projections in one launch; "Kestrel_VLLM #24", section 3: g from a, beta
// from b).  A workgroup owns FB batch rows x FR rows of the stacked [Wa; Wb]
// and splits the dot products across FE_LANES lanes (128-bit loads, two
// chunks in flight per lane); the 32 partial sums per lane are reduced with a
// transposing butterfly (32 shuffles per lane) and then across the waves in
// a fixed order.
// ---------------------------------------------------------------------------

constexpr int FB = 8;   // batch rows per workgroup
constexpr int FR = 4;   // stacked weight rows per workgroup
constexpr int FE_LANES = 512;
constexpr int FE_WAVES = FE_LANES / 64;

// The log-domain gate g = -exp(A_log) softplus(a + dt_bias) ("Kestrel_VLLM
// #24", section 3).  softplus(z) = log(1 + e^z) is z itself to fp32 precision
// above 20 and e^z below -20; one exp serves all three ranges (its argument
// is capped at 20 by a compare, so a NaN z stays NaN).
static __device__ __forceinline__ float log_gate(float a, float A_log, float dt_bias) {
  const float z = a + dt_bias;
  const float e = expf(z > 20.0f ? 20.0f : z);
  const float sp = z > 20.0f ? z : z < -20.0f ? e : log1pf(e);
  return -expf(A_log) * sp;
}

static __device__ __forceinline__ void fe_accumulate(float (&acc)[FB * FR], const f4 (&w)[FR],
                                                     const f4 (&xv)[FB]) {
#pragma unroll
  for (int b = 0; b < FB; b++)
#pragma unroll
    for (int r = 0; r < FR; r++) {
      float s = acc[b * FR + r];
      s = __builtin_fmaf(w[r].x, xv[b].x, s);
      s = __builtin_fmaf(w[r].y, xv[b].y, s);
      s = __builtin_fmaf(w[r].z, xv[b].z, s);
      s = __builtin_fmaf(w[r].w, xv[b].w, s);
      acc[b * FR + r] = s;
    }
}

static __device__ __forceinline__ void fe_gemv_block(int bx, int by, const float *x,
                                                     const float *Wa, const float *Wb,
                                                     const float *A_log, const float *dt_bias,
                                                     float *g, float *beta, int B, int dim,
                                                     int vh) {
  __shared__ float s_w[FE_WAVES][FB * FR];
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int b0 = bx * FB;
  const int r0 = by * FR;

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
  constexpr int STRIDE = 4 * FE_LANES;
  int c = 4 * t;
  for (; c + STRIDE < dim; c += 2 * STRIDE) {
    f4 w0[FR], w1[FR], x0[FB], x1[FB];
#pragma unroll
    for (int r = 0; r < FR; r++) {
      w0[r] = ld4(wrow[r] + c);
      w1[r] = ld4(wrow[r] + c + STRIDE);
    }
#pragma unroll
    for (int b = 0; b < FB; b++) {
      x0[b] = ld4(xrow[b] + c);
      x1[b] = ld4(xrow[b] + c + STRIDE);
    }
    fe_accumulate(acc, w0, x0);
    fe_accumulate(acc, w1, x1);
  }
  if (c < dim) {
    f4 w0[FR], x0[FB];
#pragma unroll
    for (int r = 0; r < FR; r++) w0[r] = ld4(wrow[r] + c);
#pragma unroll
    for (int b = 0; b < FB; b++) x0[b] = ld4(xrow[b] + c);
    fe_accumulate(acc, w0, x0);
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
      v16[i] = keep + lane_xor<32>(send);
    }
  }
  float v8[8];
  {
    const bool up = lane & 16;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const float send = up ? v16[i] : v16[8 + i];
      const float keep = up ? v16[8 + i] : v16[i];
      v8[i] = keep + lane_xor<16>(send);
    }
  }
  float v4[4];
  {
    const bool up = lane & 8;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const float send = up ? v8[i] : v8[4 + i];
      const float keep = up ? v8[4 + i] : v8[i];
      v4[i] = keep + lane_xor<8>(send);
    }
  }
  float v2[2];
  {
    const bool up = lane & 4;
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const float send = up ? v4[i] : v4[2 + i];
      const float keep = up ? v4[2 + i] : v4[i];
      v2[i] = keep + lane_xor<4>(send);
    }
  }
  float v1;
  {
    const bool up = lane & 2;
    const float send = up ? v2[0] : v2[1];
    const float keep = up ? v2[1] : v2[0];
    v1 = keep + lane_xor<2>(send);
  }
  v1 = v1 + lane_xor<1>(v1);
  if ((lane & 1) == 0) s_w[wave][lane >> 1] = v1;
  __syncthreads();
  if (t < FB * FR) {
    float sum = s_w[0][t];
#pragma unroll
    for (int w = 1; w < FE_WAVES; w++) sum = sum + s_w[w][t];
    const int b = b0 + t / FR;
    const int R = r0 + t % FR;
    if (b < B && R < 2 * vh) {
      if (R < vh) {
        g[(int64_t)b * vh + R] = log_gate(sum, A_log[R], dt_bias[R]);
      } else {
        beta[(int64_t)b * vh + (R - vh)] = 1.0f / (1.0f + expf(-sum));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Front end, conv part: depthwise causal conv (4 taps) + SiLU + history
// advance + split + per key-head L2 norm ("Kestrel_VLLM #24", section 3 and
// Fig. 1 caption).  Each half of a FE_LANES workgroup handles one batch row
// and a block of 1024 channels; a lane owns 4 adjacent channels, whose 4
// taps are one 16-float run of conv_w.  A key head (KD channels) is KD/4
// adjacent lanes of one wave, so its sum of squares is a shuffle reduction.
// Head boundaries are multiples of KD and blocks are multiples of 1024, so no
// head straddles two blocks.
// ---------------------------------------------------------------------------

constexpr int CONV_ROWS = FE_LANES / 256;   // units per conv block

// M rows of one unit: the 4-frame window [h0, h1, h2, raw_m] slides across
// the rows (h0 <- h1, h1 <- h2, h2 <- raw_m), which is what M successive
// single-row calls do to the history; every row uses the same arithmetic as a
// single-row call, so the results are bit-identical to M such calls.  The
// history is written once, after the last row.
template <int KD>
static __device__ __forceinline__ void fe_conv_block(int bx, int by, const float *xc_raw,
                                                     float *hist, const float *conv_w, float *q,
                                                     float *k, float *v, int B, int M,
                                                     int conv_dim, int kh, int vh,
                                                     bool write_hist) {
  const int t = threadIdx.x % 256;
  const int64_t b = (int64_t)by * CONV_ROWS + threadIdx.x / 256;
  const int ch = bx * 1024 + 4 * t;
  const bool valid = ch < conv_dim && b < B;     // b is uniform per wave
  const int qk_w = kh * KD;
  f4 h0 = splat(0.0f), h1 = splat(0.0f), h2 = splat(0.0f);
  f4 wc[4] = {splat(0.0f), splat(0.0f), splat(0.0f), splat(0.0f)};
  float *hb = hist + b * 3 * (int64_t)conv_dim + ch;
  if (valid) {
    h0 = ld4(hb);
    h1 = ld4(hb + conv_dim);
    h2 = ld4(hb + 2 * (int64_t)conv_dim);
    const float *w = conv_w + (int64_t)ch * 4;
#pragma unroll
    for (int c = 0; c < 4; c++) wc[c] = ld4(w + 4 * c);
  }
  for (int m = 0; m < M; m++) {
    const int64_t row = (int64_t)m * B + b;      // [M][B] row
    float out[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (valid) {
      const f4 raw = ld4(xc_raw + row * conv_dim + ch);
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
      h0 = h1;
      h1 = h2;
      h2 = raw;
    }
    // per key-head sum of squares over KD/4 lanes (every lane takes part)
    float ss = out[0] * out[0];
    ss = __builtin_fmaf(out[1], out[1], ss);
    ss = __builtin_fmaf(out[2], out[2], ss);
    ss = __builtin_fmaf(out[3], out[3], ss);
    ss = xor_fold<1, KD / 4>(ss);
    if (valid) {
      const f4 o4 = {out[0], out[1], out[2], out[3]};
      if (ch < 2 * qk_w) {
        const float inv = 1.0f / sqrtf(ss + 1e-6f);
        if (ch < qk_w)
          st4(q + row * qk_w + ch, (o4 * inv) * (1.0f / sqrtf((float)KD)));
        else
          st4(k + row * qk_w + (ch - qk_w), o4 * inv);
      } else {
        st4(v + row * (int64_t)vh * KD + (ch - 2 * qk_w), o4);
      }
    }
  }
  if (valid && write_hist) {
    st4(hb, h0);
    st4(hb + conv_dim, h1);
    st4(hb + 2 * (int64_t)conv_dim, h2);
  }
}

// M draft rows at once (M >= 2): wave m of a workgroup takes row m (and m +
// FE_WAVES, ...) of one sequence over CONV_RCH channels.  Row m's taps are
// raw rows m - 3 .. m, those before row 0 from the history, so the rows need
// not wait on each other as the sliding window above does; each row uses that
// window's arithmetic on the same frames, so the bits are the same.  The new
// history (the last three frames) is read before a barrier and written after
// it, once every row of the workgroup has read the old one.
constexpr int CONV_RCH = 256;   // channels per row-parallel workgroup
// up to this many sequences (frontend_m at M = 8: 1 sequence 7.1 -> 4.6 us,
// 8 sequences 9.3 -> 7.2; from 16 the window's single read of each frame
// wins, 10.9 against 11.2 us, and 54 against 62 at 128)
constexpr int kConvRowsMaxB = 8;

template <int KD>
static __device__ __forceinline__ void fe_conv_rows(int bx, int b, const float *xc_raw, float *hist,
                                                    const float *conv_w, float *q, float *k,
                                                    float *v, int B, int M, int conv_dim, int kh,
                                                    int vh, bool write_hist) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ch = bx * CONV_RCH + 4 * lane;
  const bool valid = ch < conv_dim;
  const int qk_w = kh * KD;
  float *hb = hist + (int64_t)b * 3 * conv_dim + ch;
  // raw frame f of sequence b; f < 0: history frame 3 + f (oldest first)
  auto frame = [&](int f) -> f4 {
    return f < 0 ? ld4(hb + (int64_t)(3 + f) * conv_dim)
                 : ld4(xc_raw + ((int64_t)f * B + b) * conv_dim + ch);
  };
  f4 wc[4] = {splat(0.0f), splat(0.0f), splat(0.0f), splat(0.0f)};
  if (valid) {
    const float *w = conv_w + (int64_t)ch * 4;
#pragma unroll
    for (int c = 0; c < 4; c++) wc[c] = ld4(w + 4 * c);
  }
  for (int m = wave; m < M; m += FE_WAVES) {    // uniform per wave
    const int64_t row = (int64_t)m * B + b;      // [M][B] row
    float out[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (valid) {
      const f4 h0 = frame(m - 3), h1 = frame(m - 2), h2 = frame(m - 1), raw = frame(m);
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
    }
    // per key-head sum of squares over KD/4 lanes (every lane takes part)
    float ss = out[0] * out[0];
    ss = __builtin_fmaf(out[1], out[1], ss);
    ss = __builtin_fmaf(out[2], out[2], ss);
    ss = __builtin_fmaf(out[3], out[3], ss);
    ss = xor_fold<1, KD / 4>(ss);
    if (valid) {
      const f4 o4 = {out[0], out[1], out[2], out[3]};
      if (ch < 2 * qk_w) {
        const float inv = 1.0f / sqrtf(ss + 1e-6f);
        if (ch < qk_w)
          st4(q + row * qk_w + ch, (o4 * inv) * (1.0f / sqrtf((float)KD)));
        else
          st4(k + row * qk_w + (ch - qk_w), o4 * inv);
      } else {
        st4(v + row * (int64_t)vh * KD + (ch - 2 * qk_w), o4);
      }
    }
  }
  if (write_hist) {                               // uniform
    f4 hn = splat(0.0f);
    if (valid && wave < 3) hn = frame(M - 3 + wave);
    __syncthreads();
    if (valid && wave < 3) st4(hb + (int64_t)wave * conv_dim, hn);
  }
}

// One GEMV row per call (one sequence, one draft row): a workgroup per
// stacked weight row (2 vh of them instead of 2 vh / FR), every lane's chunks
// requested at once.  Each lane's chain over its columns and the lane pairing
// of the butterfly (offsets 32, 16, 8, 4, 2, 1) are those of fe_gemv_block,
// and every add is commutative, so the results are the same bits.
static __device__ __forceinline__ void fe_gemv_row(int R, const float *x, const float *Wa,
                                                   const float *Wb, const float *A_log,
                                                   const float *dt_bias, float *g, float *beta,
                                                   int dim, int vh) {
  __shared__ float s_w1[FE_WAVES];
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const float *wrow = R < vh ? Wa + (int64_t)R * dim : Wb + (int64_t)(R - vh) * dim;
  constexpr int STRIDE = 4 * FE_LANES;
  constexpr int DEPTH = 4;                      // chunks per lane in flight
  float acc = 0.0f;
  for (int c0 = 4 * t; c0 < dim; c0 += DEPTH * STRIDE) {
    f4 w[DEPTH], xv[DEPTH];
#pragma unroll
    for (int k = 0; k < DEPTH; k++) {
      const int c = c0 + k * STRIDE;
      if (c < dim) {
        w[k] = ld4(wrow + c);
        xv[k] = ld4(x + c);
      }
    }
#pragma unroll
    for (int k = 0; k < DEPTH; k++) {
      if (c0 + k * STRIDE < dim) {
        acc = __builtin_fmaf(w[k].x, xv[k].x, acc);
        acc = __builtin_fmaf(w[k].y, xv[k].y, acc);
        acc = __builtin_fmaf(w[k].z, xv[k].z, acc);
        acc = __builtin_fmaf(w[k].w, xv[k].w, acc);
      }
    }
  }
  acc = acc + lane_xor<32>(acc);
  acc = acc + lane_xor<16>(acc);
  acc = acc + lane_xor<8>(acc);
  acc = acc + lane_xor<4>(acc);
  acc = acc + lane_xor<2>(acc);
  acc = acc + lane_xor<1>(acc);
  if (lane == 0) s_w1[wave] = acc;
  __syncthreads();
  if (t == 0) {
    float sum = s_w1[0];
#pragma unroll
    for (int w = 1; w < FE_WAVES; w++) sum = sum + s_w1[w];
    if (R < vh) {
      g[R] = log_gate(sum, A_log[R], dt_bias[R]);
    } else {
      beta[R - vh] = 1.0f / (1.0f + expf(-sum));
    }
  }
}

// 2 to 8 GEMV rows (a few sequences, or one sequence's draft rows): a
// workgroup per stacked weight row and all 8 batch slots (4 times the
// workgroups of fe_gemv_block), three chunks per lane in flight.  Each slot's
// chain and the butterfly's lane pairing (offsets 32, 16, 8, then 4, 2, 1)
// are those of fe_gemv_block, so the results are the same bits.
static __device__ __forceinline__ void fe_gemv_col8(int bx, int R, const float *x,
                                                    const float *Wa, const float *Wb,
                                                    const float *A_log, const float *dt_bias,
                                                    float *g, float *beta, int B, int dim,
                                                    int vh) {
  __shared__ float s_w8[FE_WAVES][FB];
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int b0 = bx * FB;
  const float *wrow = R < vh ? Wa + (int64_t)R * dim : Wb + (int64_t)(R - vh) * dim;
  const float *xrow[FB];
#pragma unroll
  for (int b = 0; b < FB; b++) {
    int bb = b0 + b;
    if (bb >= B) bb = B - 1;                       // clamped rows are never written
    xrow[b] = x + (int64_t)bb * dim;
  }
  constexpr int STRIDE = 4 * FE_LANES;
  constexpr int DEPTH = 3;                         // chunks per lane in flight
  float acc[FB];
#pragma unroll
  for (int b = 0; b < FB; b++) acc[b] = 0.0f;
  for (int c0 = 4 * t; c0 < dim; c0 += DEPTH * STRIDE) {
    f4 w[DEPTH], xv[DEPTH][FB];
#pragma unroll
    for (int k = 0; k < DEPTH; k++) {
      const int c = c0 + k * STRIDE;
      if (c < dim) {
        w[k] = ld4(wrow + c);
#pragma unroll
        for (int b = 0; b < FB; b++) xv[k][b] = ld4(xrow[b] + c);
      }
    }
#pragma unroll
    for (int k = 0; k < DEPTH; k++) {
      if (c0 + k * STRIDE < dim) {
#pragma unroll
        for (int b = 0; b < FB; b++) {
          float s = acc[b];
          s = __builtin_fmaf(w[k].x, xv[k][b].x, s);
          s = __builtin_fmaf(w[k].y, xv[k][b].y, s);
          s = __builtin_fmaf(w[k].z, xv[k][b].z, s);
          s = __builtin_fmaf(w[k].w, xv[k][b].w, s);
          acc[b] = s;
        }
      }
    }
  }
  // transposing butterfly over 8 slots (offsets 32, 16, 8), then plain adds
  float v4[4], v2[2], v1;
  {
    const bool up = lane & 32;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const float send = up ? acc[i] : acc[4 + i];
      const float keep = up ? acc[4 + i] : acc[i];
      v4[i] = keep + lane_xor<32>(send);
    }
  }
  {
    const bool up = lane & 16;
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const float send = up ? v4[i] : v4[2 + i];
      const float keep = up ? v4[2 + i] : v4[i];
      v2[i] = keep + lane_xor<16>(send);
    }
  }
  {
    const bool up = lane & 8;
    const float send = up ? v2[0] : v2[1];
    const float keep = up ? v2[1] : v2[0];
    v1 = keep + lane_xor<8>(send);
  }
  v1 = v1 + lane_xor<4>(v1);
  v1 = v1 + lane_xor<2>(v1);
  v1 = v1 + lane_xor<1>(v1);
  if ((lane & 7) == 0) s_w8[wave][lane >> 3] = v1;   // slot 4 b5 + 2 b4 + b3
  __syncthreads();
  if (t < FB) {
    float sum = s_w8[0][t];
#pragma unroll
    for (int w = 1; w < FE_WAVES; w++) sum = sum + s_w8[w][t];
    const int b = b0 + t;
    if (b < B) {
      if (R < vh) {
        g[(int64_t)b * vh + R] = log_gate(sum, A_log[R], dt_bias[R]);
      } else {
        beta[(int64_t)b * vh + (R - vh)] = 1.0f / (1.0f + expf(-sum));
      }
    }
  }
}

// One launch for the whole front end: the first n_conv workgroups run the
// conv, the rest the paired GEMV; the two parts are independent, so their
// latency-bound and bandwidth-bound phases overlap on the device (the conv
// workgroups are dispatched first).  GS picks the GEMV shape (0: one row, 1:
// 2..8 rows, 2: more) and CR the conv (0: a sliding window per sequence for
// single rows, 1: M >= 2 rows in parallel), one instance each so that each
// keeps its own register budget.
struct FeArgs {
  const float *x, *Wa, *Wb, *A_log, *dt_bias, *xc_raw;
  float *hist;
  const float *conv_w;
  float *q, *k, *v, *g, *beta;
  int B, M, dim, conv_dim, vh, kh;
  int write_hist;         // 0: the history is read but left as it was
  int gemv_bx, conv_bx;   // x extents of the two parts
  int n_gemv;             // workgroups of the GEMV part
  int n_conv;             // workgroups of the conv part
};

template <int KD, int GS, bool CR>
__global__ __launch_bounds__(FE_LANES) void fe_kernel(FeArgs a) {
  if ((int)blockIdx.x >= a.n_conv) {
    const int id = (int)blockIdx.x - a.n_conv;
    // Each XCD takes a contiguous, batch-major range of GEMV blocks, so its
    // L2 holds a few batch rows of x and the weights once, instead of every
    // L2 pulling in all of x and all of W.  The GEMV rows of all M draft rows
    // are independent: [M][B] = M*B rows.
    const int g = (int)xcd_contiguous(id, a.n_gemv);
    if constexpr (GS == 0) {
      fe_gemv_row(g, a.x, a.Wa, a.Wb, a.A_log, a.dt_bias, a.g, a.beta, a.dim, a.vh);
    } else if constexpr (GS == 1) {
      fe_gemv_col8(0, g, a.x, a.Wa, a.Wb, a.A_log, a.dt_bias, a.g, a.beta, a.M * a.B, a.dim,
                   a.vh);
    } else {
      const int r_tiles = a.n_gemv / a.gemv_bx;
      fe_gemv_block(g / r_tiles, g % r_tiles, a.x, a.Wa, a.Wb, a.A_log, a.dt_bias, a.g,
                    a.beta, a.M * a.B, a.dim, a.vh);
    }
  } else {
    const int c = (int)blockIdx.x;
    if constexpr (CR)
      fe_conv_rows<KD>(c % a.conv_bx, c / a.conv_bx, a.xc_raw, a.hist, a.conv_w, a.q, a.k, a.v,
                       a.B, a.M, a.conv_dim, a.kh, a.vh, a.write_hist != 0);
    else
      fe_conv_block<KD>(c % a.conv_bx, c / a.conv_bx, a.xc_raw, a.hist, a.conv_w, a.q, a.k,
                        a.v, a.B, a.M, a.conv_dim, a.kh, a.vh, a.write_hist != 0);
  }
}

int64_t frontend_workitems(int64_t B, int64_t M, int64_t conv_dim, int64_t vh) {
  const int64_t n_gemv = M * B <= FB ? 2 * vh : ((M * B + FB - 1) / FB) * ((2 * vh + FR - 1) / FR);
  const int64_t n_conv = M >= 2 && B <= kConvRowsMaxB
                             ? ((conv_dim + CONV_RCH - 1) / CONV_RCH) * B
                                : ((conv_dim + 1023) / 1024) * ((B + CONV_ROWS - 1) / CONV_ROWS);
  return (n_gemv + n_conv) * FE_LANES;
}

int launch_frontend(const float *x, const float *Wa, const float *Wb,
                    const float *A_log, const float *dt_bias,
                    const float *xc_raw, float *hist, const float *conv_w,
                    float *q, float *k, float *v, float *g, float *beta, int B, int M,
                    int dim, int conv_dim, int vh, int kh, int kd, bool write_hist,
                    hipStream_t s) {
  if (B <= 0 || M <= 0) return 0;
  FeArgs a{x, Wa, Wb, A_log, dt_bias, xc_raw, hist, conv_w, q, k, v, g, beta,
           B, M, dim, conv_dim, vh, kh, write_hist ? 1 : 0, 0, 0, 0, 0};
  a.gemv_bx = (M * B + FB - 1) / FB;
  a.n_gemv = M * B <= FB ? 2 * vh : a.gemv_bx * ((2 * vh + FR - 1) / FR);
  const bool cr = M >= 2 && B <= kConvRowsMaxB;
  a.conv_bx = cr ? (conv_dim + CONV_RCH - 1) / CONV_RCH : (conv_dim + 1023) / 1024;
  a.n_conv = cr ? a.conv_bx * B : a.conv_bx * ((B + CONV_ROWS - 1) / CONV_ROWS);
  const dim3 grid((unsigned)(a.n_gemv + a.n_conv));
  const int gs = M * B == 1 ? 0 : M * B <= FB ? 1 : 2;
  auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, grid, dim3(FE_LANES), 0, s, a); };
  if (kd == 128) {
    if (cr)
      gs == 1 ? go(fe_kernel<128, 1, true>) : go(fe_kernel<128, 2, true>);
    else
      gs == 0 ? go(fe_kernel<128, 0, false>) : gs == 1 ? go(fe_kernel<128, 1, false>)
              : go(fe_kernel<128, 2, false>);
  } else {
    if (cr)
      gs == 1 ? go(fe_kernel<64, 1, true>) : go(fe_kernel<64, 2, true>);
    else
      gs == 0 ? go(fe_kernel<64, 0, false>) : gs == 1 ? go(fe_kernel<64, 1, false>)
              : go(fe_kernel<64, 2, false>);
  }
  return (int)hipGetLastError();
}

// y0[0..n0) = 0 and y1[0..n1) = 0: the fill before a launch whose two
// half-workgroups add their folds into y with atomics.
__global__ __launch_bounds__(256) void zero2_kernel(float *y0, int64_t n0, float *y1, int64_t n1) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n0)
    y0[i] = 0.f;
  else if (i - n0 < n1)
    y1[i - n0] = 0.f;
}

// ---------------------------------------------------------------------------
// Dense layer projections on the matrix cores: y[r][o] = sum_c W[o][c] x[r][c]
// ("Kestrel_VLLM #24", Fig. 1 caption, steps 1 and 7: in_proj_qkv, in_proj_z
// and out_proj; "Kestrel_VLLM #34", section 3.6: all draft rows in one pass
// over the weights, each row giving what a one-row call gives).
//
// With 1-16 rows the product streams the weights once and is bound by HBM;
// with 64 and more rows it is a dense fp32 contraction (32 flop per weight
// byte at 64 rows, above the ridge), so it runs on v_mfma_f32_16x16x4_f32
// throughout.  Operand layout of that instruction (checked on gfx950): lane
// l supplies A[l % 16][l / 16] and B[l / 16][l % 16] and receives
// D[4 (l / 16) + t][l % 16] in accumulator register t.  Here A is a block of
// 16 rows of x, B a block of 16 weight rows (transposed), so one lane loads
// the 4 consecutive columns 4 (l / 16) .. +3 of one x row and of one weight
// row with a 128-bit load and feeds them to 4 successive MFMAs.
//
// The weights are stored once, at load time, in that operand order
// (gdn_proj_pack): slab s of 16 weight rows, 16-column block kb, lane l hold
// W[16 s + l % 16][16 kb + 4 (l / 16) .. +3] as the 1 KiB block
// Wp[(s (C / 16) + kb) 256 + 4 l ..].  A wave then streams its weights as
// contiguous 1 KiB loads; read row-major, every load touched 16 rows in
// 64-byte pieces and the call ran 25-30% slower at 1 row.
//
// Canonical summation, independent of the row count and of the tiling: C is
// cut into PJ_SEG = 8 equal segments; each segment is summed by one MFMA
// chain over its 16-column blocks in ascending order (block kb, MFMA step s
// adds the terms of columns kb + 4 i + s, i = 0..3); segments 0..3 are
// folded left to right, so are segments 4..7, and the two sums are added.  A
// row's result therefore does not depend on which other rows share the call,
// and every tile shape gives the same bits.
//
// A workgroup is PJ_SEG waves, wave w owning segment w for a tile of 16 RB
// rows x 16 OJ outputs; the segment sums meet in LDS and are folded there.
// When a launch of 2 to 16 rows has fewer tiles than twice the CUs (out_proj:
// 320), each tile takes two workgroups of 4 waves instead, one per half of
// the segments, and each adds its half's fold into y, which a fill kernel set
// to zero.  Every segment sum is a chain started at +0, so no
// fold is -0 and +0 + h = h exactly; with exactly two addends the result is
// h0 + h1 whichever arrives first (fp addition is commutative), so both
// shapes give the same bits, and out_proj's 640 half-tiles spread over the
// CUs (8 rows: 27.8 -> 23.5 us).  At one row the fill kernel's launch costs
// what the split gains, so one-row launches keep whole tiles.
// Workgroups are ordered output-slab major, row-group minor, and laid out
// contiguously per XCD, so the row groups sharing a weight slab run on one
// L2.  Two products over the same x (in_proj_qkv and in_proj_z) share one
// launch.
// ---------------------------------------------------------------------------

constexpr int PJ_SEG = 8;                 // segments of C, one wave each
constexpr int PJ_LANES = 64 * PJ_SEG;
constexpr int64_t kPjSplitBelow = 512;    // few-row launches of fewer tiles: two halves each
constexpr int64_t kPjMinWg = 128;
constexpr int64_t kPjMinWg1 = 256;
constexpr int64_t kPjU2Rows = 8;        // few rows: up to this many
constexpr int64_t kPjMinWgFew = 1024;
constexpr int64_t kPjStagedMin = 256;   // 4 x 4 tiles: staged fold from this many

struct ProjProblem {
  const float *W;
  float *y;
  int R;
  int blocks;       // workgroups: (R / (16 OJ)) * row_groups, twice that when split
};

struct ProjArgs {
  const float *x;
  int64_t rows;
  int C;
  int row_groups;
  ProjProblem p[2];
};

typedef float pj_acc __attribute__((ext_vector_type(4)));

// Weight loads: with a single row group each weight is read exactly once, so
// it is streamed past the caches (nt) and leaves L2 to x.  Tiles of 4 row
// blocks over several row groups use the default policy, so that the groups
// sharing a slab hit in L2; tiles of 1 or 2 row blocks (at most two row
// groups by the shape rule below) measured faster streaming.
template <bool STREAM>
static __device__ __forceinline__ f4 ld_w(rsrc_t r, int voff) {
  return __builtin_bit_cast(
      f4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, STREAM ? POL_STREAM_LOAD : 0));
}

// RB row blocks x OJ output slabs per wave, U 16-column blocks per trip; NW
// waves per workgroup (PJ_SEG: a whole tile; PJ_SEG / 2: half a tile, the
// two halves of a tile in adjacent workgroups).  STAGED (whole tiles only)
// folds the segment sums through two LDS buffers instead of one block per
// segment: 32 KiB instead of 128 KiB for a 4 x 4 tile.
template <int RB, int OJ, int U, bool STREAM, int NW, bool STAGED = false>
__global__ __launch_bounds__(64 * NW) void proj_kernel(ProjArgs a) {
  constexpr bool SPLIT = NW < PJ_SEG;
  static_assert(!(SPLIT && STAGED), "a half tile folds in one buffer");
  __shared__ pj_acc red[STAGED ? 2 : NW][RB * OJ][64];
  const int b = (int)xcd_contiguous(blockIdx.x, gridDim.x);
  const bool second = b >= a.p[0].blocks;
  const float *W = second ? a.p[1].W : a.p[0].W;
  float *y = second ? a.p[1].y : a.p[0].y;
  const int R = second ? a.p[1].R : a.p[0].R;
  const int lbh = second ? b - a.p[0].blocks : b;
  const int lb = SPLIT ? lbh >> 1 : lbh;            // the tile
  const int half = SPLIT ? lbh & 1 : 0;
  const int slab = lb / a.row_groups, rgp = lb - slab * a.row_groups;
  const int o0 = slab * 16 * OJ;
  const int64_t r0 = (int64_t)rgp * 16 * RB;
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int sgm = NW * half + wave;                 // this wave's segment
  const int j = l & 15, kq = l >> 4;
  const int C = a.C;
  const int seg = C / PJ_SEG;
  const int k0 = sgm * seg + 4 * kq;

  // one buffer resource over the workgroup's OJ packed slabs (< 2 GiB); the
  // 16-column block at column c of slab oj starts at float oj 16 C + 16 c
  const rsrc_t wr = buf_rsrc(W + (int64_t)o0 * C, 16 * OJ * C * 4);
  int wo[OJ];
#pragma unroll
  for (int oj = 0; oj < OJ; oj++) wo[oj] = (16 * oj * C + 16 * sgm * seg + 4 * l) * 4;
  const float *xp[RB];
  bool xon[RB];
#pragma unroll
  for (int rb = 0; rb < RB; rb++) {
    const int64_t row = r0 + 16 * rb + j;
    xon[rb] = row < a.rows;
    xp[rb] = a.x + (xon[rb] ? row : 0) * C + k0;
  }

  pj_acc acc[RB][OJ];
#pragma unroll
  for (int rb = 0; rb < RB; rb++)
#pragma unroll
    for (int oj = 0; oj < OJ; oj++) acc[rb][oj] = pj_acc{0.f, 0.f, 0.f, 0.f};

  int kb = 0;
  if constexpr (RB == 1 || (RB * OJ >= 8 && U == 1)) {
    // software-pipelined: the loads of trip i + 1 are issued before the
    // MFMAs of trip i (same MFMA order as the plain loop below).  Measured
    // 3-17% faster up to 16 rows (weights streamed at 6.6 TB/s).  The 2 x 4
    // and 4 x 4 tiles take it with one column block per trip (103 and 162
    // VGPRs) when the launch is one round of workgroups, whose load latency
    // nothing else on the CU hides; with more rounds the plain loop with two
    // blocks per trip measured faster.
    f4 wn[U][OJ], xn[U][RB];
    auto issue = [&](int k) {
#pragma unroll
      for (int u = 0; u < U; u++)
#pragma unroll
        for (int oj = 0; oj < OJ; oj++) wn[u][oj] = ld_w<STREAM>(wr, wo[oj] + (k + 16 * u) * 64);
#pragma unroll
      for (int u = 0; u < U; u++)
#pragma unroll
        for (int rb = 0; rb < RB; rb++)
          xn[u][rb] = xon[rb] ? ld4(xp[rb] + k + 16 * u) : splat(0.f);
    };
    if (16 * U <= seg) issue(0);
    for (; kb + 16 * U <= seg; kb += 16 * U) {
      f4 w[U][OJ], xv[U][RB];
#pragma unroll
      for (int u = 0; u < U; u++) {
#pragma unroll
        for (int oj = 0; oj < OJ; oj++) w[u][oj] = wn[u][oj];
#pragma unroll
        for (int rb = 0; rb < RB; rb++) xv[u][rb] = xn[u][rb];
      }
      if (kb + 32 * U <= seg) issue(kb + 16 * U);
#pragma unroll
      for (int u = 0; u < U; u++)
#pragma unroll
        for (int s = 0; s < 4; s++)
#pragma unroll
          for (int rb = 0; rb < RB; rb++)
#pragma unroll
            for (int oj = 0; oj < OJ; oj++)
              acc[rb][oj] = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[u][rb][s], w[u][oj][s],
                                                                 acc[rb][oj], 0, 0, 0);
    }
  } else {
    for (; kb + 16 * U <= seg; kb += 16 * U) {
      f4 w[U][OJ], xv[U][RB];
#pragma unroll
      for (int u = 0; u < U; u++)
#pragma unroll
        for (int oj = 0; oj < OJ; oj++) w[u][oj] = ld_w<STREAM>(wr, wo[oj] + (kb + 16 * u) * 64);
#pragma unroll
      for (int u = 0; u < U; u++)
#pragma unroll
        for (int rb = 0; rb < RB; rb++)
          xv[u][rb] = xon[rb] ? ld4(xp[rb] + kb + 16 * u) : splat(0.f);
#pragma unroll
      for (int u = 0; u < U; u++)
#pragma unroll
        for (int s = 0; s < 4; s++)
#pragma unroll
          for (int rb = 0; rb < RB; rb++)
#pragma unroll
            for (int oj = 0; oj < OJ; oj++)
              acc[rb][oj] = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[u][rb][s], w[u][oj][s],
                                                                 acc[rb][oj], 0, 0, 0);
    }
  }
  for (; kb < seg; kb += 16) {             // the rest of a segment, one block at a time
    f4 w[OJ], xv[RB];
#pragma unroll
    for (int oj = 0; oj < OJ; oj++) w[oj] = ld_w<STREAM>(wr, wo[oj] + kb * 64);
#pragma unroll
    for (int rb = 0; rb < RB; rb++) xv[rb] = xon[rb] ? ld4(xp[rb] + kb) : splat(0.f);
#pragma unroll
    for (int s = 0; s < 4; s++)
#pragma unroll
      for (int rb = 0; rb < RB; rb++)
#pragma unroll
        for (int oj = 0; oj < OJ; oj++)
          acc[rb][oj] = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[rb][s], w[oj][s], acc[rb][oj],
                                                             0, 0, 0);
  }

  if constexpr (STAGED) {
    // wave 0 left-folds segments 1..3 into its own sum, wave PJ_SEG / 2
    // segments 5..7 into its own, one segment per round through buffer 0 or
    // 1; then wave 0 adds the second fold and stores (the same operations, in
    // the same order, as the one-buffer fold below)
    constexpr int H = PJ_SEG / 2;
#pragma unroll
    for (int jj = 1; jj < H; jj++) {
      if (wave == jj || wave == H + jj) {
        const int bsel = wave == jj ? 0 : 1;
#pragma unroll
        for (int rb = 0; rb < RB; rb++)
#pragma unroll
          for (int oj = 0; oj < OJ; oj++) red[bsel][rb * OJ + oj][l] = acc[rb][oj];
      }
      __syncthreads();
      if (wave == 0 || wave == H) {
        const int bsel = wave == 0 ? 0 : 1;
#pragma unroll
        for (int rb = 0; rb < RB; rb++)
#pragma unroll
          for (int oj = 0; oj < OJ; oj++) acc[rb][oj] = acc[rb][oj] + red[bsel][rb * OJ + oj][l];
      }
      __syncthreads();
    }
    if (wave == H) {
#pragma unroll
      for (int rb = 0; rb < RB; rb++)
#pragma unroll
        for (int oj = 0; oj < OJ; oj++) red[1][rb * OJ + oj][l] = acc[rb][oj];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int rb = 0; rb < RB; rb++)
#pragma unroll
        for (int oj = 0; oj < OJ; oj++) {
          const pj_acc sum = acc[rb][oj] + red[1][rb * OJ + oj][l];
#pragma unroll
          for (int t = 0; t < 4; t++) {
            const int64_t row = r0 + 16 * rb + 4 * (l >> 4) + t;
            if (row < a.rows) y[row * R + o0 + 16 * oj + (l & 15)] = sum[t];
          }
        }
    }
    return;
  }
#pragma unroll
  for (int rb = 0; rb < RB; rb++)
#pragma unroll
    for (int oj = 0; oj < OJ; oj++) red[wave][rb * OJ + oj][l] = acc[rb][oj];
  __syncthreads();
  // fold the segment sums: segments 0..3 left to right, 4..7 likewise, then
  // their sum (or this half's fold added into y); element e = (tile, lane,
  // register t) is float e of every segment's block of LDS
  constexpr int ELEMS = RB * OJ * 256;
  const float *redf = reinterpret_cast<const float *>(red);
  for (int e = threadIdx.x; e < ELEMS; e += 64 * NW) {
    const int tile = e >> 8, ll = (e >> 2) & 63, t = e & 3;
    float h0 = redf[e];
#pragma unroll
    for (int w = 1; w < PJ_SEG / 2; w++) h0 = h0 + redf[w * ELEMS + e];
    float sum = h0;
    if constexpr (!SPLIT) {
      float h1 = redf[(PJ_SEG / 2) * ELEMS + e];
#pragma unroll
      for (int w = PJ_SEG / 2 + 1; w < PJ_SEG; w++) h1 = h1 + redf[w * ELEMS + e];
      sum = h0 + h1;
    }
    const int rb = tile / OJ, oj = tile - rb * OJ;
    const int64_t row = r0 + 16 * rb + 4 * (ll >> 4) + t;
    if (row < a.rows) {
      float *dst = &y[row * R + o0 + 16 * oj + (ll & 15)];
      if constexpr (SPLIT)
        atomicAdd(dst, sum);               // the other half adds the other fold
      else
        *dst = sum;
    }
  }
}

// Tile shape of a call.  Up to 16 rows (one row block) the call streams the
// weights: the widest output slab group (1, 2 or 4 slabs of 16) dividing
// R / 16 that still leaves >= kPjMinWg1 workgroups (kPjMinWgFew up
// to 8 rows), to spread the stream over every CU: in_proj at 1 to 4 rows
// takes 52 us with 1024 one-slab workgroups against 55 us with 256 four-slab
// ones, but 66 against 54 us at 16 rows.  Beyond 16 rows it is bound by the matrix cores and by x
// traffic: the widest slab group dividing R / 16 (each x load then serves
// more outputs), then the most row blocks per tile (up to the rows present)
// that still leave >= kPjMinWg workgroups.  Measured at 64 rows:
// out_proj (R = 5120) 2 row blocks x 4 slabs 70 us, 4 x 2 96 us, 4 x 4
// 128 us; in_proj 4 x 4 128 us.
// That whole-tile choice is kept beyond 16 rows only while it fills the chip
// evenly with little padding.  If it leaves CUs idle (fewer than
// kPjFullTiles tiles), ends on a last round of workgroups that is mostly
// empty (under 80% of its rounds' slots used), or, from 40 rows, pads the
// rows by more than a quarter, the call runs split halves of one-row-block
// tiles instead, with the widest slab group that still gives
// kPjSplitTilesMin tiles.  Measured (8 weight sets from HBM) against the
// whole-tile choice: out_proj at 17-32 rows 45 -> 39-42 us, 40-64 rows
// 68 -> 42-59 us, 80-128 rows 119-123 -> 72-91 us, 256 rows 230 -> 175 us;
// in_proj at 80 rows 197 -> 157 us, 96 rows 199 -> 183 us.  No choice
// changes a result (canonical summation above).
constexpr int64_t kPjFullTiles = 224;
constexpr int64_t kPjSplitTilesMin = 192;
constexpr int64_t kPjCUs = 256;

struct ProjShape {
  int rb, oj, row_groups;
  bool split;   // two half-tile workgroups per tile (one row block)
};

static int64_t proj_tiles(int64_t rows, int R0, int R1, int rb, int oj) {
  const int64_t groups = (rows + 16 * rb - 1) / (16 * rb);
  return ((int64_t)R0 / (16 * oj) + (int64_t)R1 / (16 * oj)) * groups;
}

static ProjShape proj_shape(int64_t rows, int R0, int R1) {
  ProjShape sh;
  const int rb_max = rows <= 16 ? 1 : rows <= 32 ? 2 : 4;
  const int64_t min_wg1 = rows <= kPjU2Rows ? kPjMinWgFew : kPjMinWg1;
  sh.oj = 1;
  for (int oj = 4; oj > 1; oj >>= 1) {
    const bool divides = (R0 / 16) % oj == 0 && (R1 / 16) % oj == 0;
    if (divides && (rb_max > 1 || proj_tiles(rows, R0, R1, 1, oj) >= min_wg1)) {
      sh.oj = oj;
      break;
    }
  }
  sh.rb = rb_max;
  while (sh.rb > 1 && proj_tiles(rows, R0, R1, sh.rb, sh.oj) < kPjMinWg) sh.rb >>= 1;
  sh.row_groups = (int)((rows + 16 * sh.rb - 1) / (16 * sh.rb));
  sh.split = false;
  if (rows > 16) {
    const int64_t t = proj_tiles(rows, R0, R1, sh.rb, sh.oj);
    const int64_t rounds = (t + kPjCUs - 1) / kPjCUs;
    const int64_t padded = (int64_t)sh.row_groups * 16 * sh.rb;
    if (t < kPjFullTiles || 5 * t < 4 * rounds * kPjCUs || (rows >= 40 && 4 * padded > 5 * rows)) {
      sh.rb = 1;
      sh.oj = 1;
      for (int oj = 4; oj > 1; oj >>= 1) {
        const bool divides = (R0 / 16) % oj == 0 && (R1 / 16) % oj == 0;
        if (divides && proj_tiles(rows, R0, R1, 1, oj) >= kPjSplitTilesMin) {
          sh.oj = oj;
          break;
        }
      }
      sh.row_groups = (int)((rows + 15) / 16);
      sh.split = true;
    }
  }
  return sh;
}

static bool proj_split(const ProjShape &sh, int64_t rows, int64_t tiles) {
  return sh.split || (rows >= 2 && sh.rb == 1 && sh.oj == 1 && tiles < kPjSplitBelow);
}

int64_t proj_workgroups(int64_t rows, int R0, int R1) {
  const ProjShape sh = proj_shape(rows, R0, R1);
  const int64_t tiles = proj_tiles(rows, R0, R1, sh.rb, sh.oj);
  return proj_split(sh, rows, tiles) ? 2 * tiles : tiles;
}

template <int RB, int OJ, int U, bool STAGED = false>
static void launch_proj_t(const ProjArgs &a, bool stream, hipStream_t s) {
  const dim3 grid((unsigned)(a.p[0].blocks + a.p[1].blocks));
  if (RB < 4 || stream)       // see ld_w
    hipLaunchKernelGGL((proj_kernel<RB, OJ, U, true, PJ_SEG, STAGED>), grid, dim3(PJ_LANES), 0,
                       s, a);
  else
    hipLaunchKernelGGL((proj_kernel<RB, OJ, U, RB < 4, PJ_SEG, STAGED>), grid, dim3(PJ_LANES), 0,
                       s, a);
}

// The split shape (one row block): two half-tile workgroups of PJ_SEG / 2
// waves per tile, after a fill kernel zeroed y.  The weights are streamed
// past the caches when one row group reads them once, as in ld_w.
template <int OJ, int U>
static void launch_proj_split(const ProjArgs &a, bool stream, hipStream_t s) {
  const int64_t n0 = a.rows * a.p[0].R, n1 = a.p[1].W ? a.rows * a.p[1].R : 0;
  hipLaunchKernelGGL(zero2_kernel, dim3((unsigned)((n0 + n1 + 255) / 256)), dim3(256), 0, s,
                     a.p[0].y, n0, a.p[1].y, n1);
  const dim3 grid((unsigned)(a.p[0].blocks + a.p[1].blocks));
  if (stream)
    hipLaunchKernelGGL((proj_kernel<1, OJ, U, true, PJ_SEG / 2>), grid, dim3(PJ_LANES / 2), 0,
                       s, a);
  else
    hipLaunchKernelGGL((proj_kernel<1, OJ, U, false, PJ_SEG / 2>), grid, dim3(PJ_LANES / 2), 0,
                       s, a);
}

// Weight packing (one launch per matrix, pure data movement): thread i
// writes packed float4 i, gathered from its row-major place.
__global__ __launch_bounds__(256) void proj_pack_kernel(const float *W, float *Wp, int C,
                                                        int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const int l = (int)(i & 63);
  const int64_t blk = i >> 6;                      // s (C / 16) + kb
  const int64_t s = blk / (C / 16), kb = blk - s * (C / 16);
  const int64_t row = 16 * s + (l & 15), col = 16 * kb + 4 * (l >> 4);
  st4(Wp + 4 * i, ld4(W + row * C + col));
}

int launch_proj_pack(const float *W, float *Wp, int R, int C, hipStream_t s) {
  const int64_t n4 = (int64_t)R * C / 4;
  if (n4 <= 0) return 0;
  hipLaunchKernelGGL(proj_pack_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, W,
                     Wp, C, n4);
  return (int)hipGetLastError();
}

int launch_proj(const float *x, int64_t rows, int C, const float *W0, int R0, float *y0,
                const float *W1, int R1, float *y1, hipStream_t s) {
  if (rows <= 0) return 0;
  const ProjShape sh = proj_shape(rows, R0, W1 ? R1 : 0);
  ProjArgs a{};
  a.x = x;
  a.rows = rows;
  a.C = C;
  a.row_groups = sh.row_groups;
  a.p[0] = ProjProblem{W0, y0, R0, R0 / (16 * sh.oj) * sh.row_groups};
  a.p[1] = ProjProblem{W1, y1, R1, W1 ? R1 / (16 * sh.oj) * sh.row_groups : 0};
  const bool stream = sh.row_groups == 1;
  if (proj_split(sh, rows, a.p[0].blocks + a.p[1].blocks)) {
    a.p[0].blocks *= 2;
    a.p[1].blocks *= 2;
    if (sh.oj == 4)
      launch_proj_split<4, 2>(a, stream, s);
    else if (sh.oj == 2)
      launch_proj_split<2, 4>(a, stream, s);
    else if (rows <= kPjU2Rows)
      launch_proj_split<1, 2>(a, stream, s);
    else
      launch_proj_split<1, 4>(a, stream, s);
    return (int)hipGetLastError();
  }
  switch (sh.rb * 8 + sh.oj) {
    // one row block: up to 8 rows, 2 blocks per trip unless the grid has
    // >= kPjMinWgFew workgroups (out_proj at one row 28.7 -> 24.4 us;
    // in_proj keeps 4), 4 beyond; the MFMA order is the same either way
    case 1 * 8 + 1:
      if (rows <= kPjU2Rows && a.p[0].blocks + a.p[1].blocks < kPjMinWgFew)
        launch_proj_t<1, 1, 2>(a, true, s);
      else
        launch_proj_t<1, 1, 4>(a, true, s);
      break;
    case 1 * 8 + 2:
      if (rows <= kPjU2Rows && a.p[0].blocks + a.p[1].blocks < kPjMinWgFew)
        launch_proj_t<1, 2, 2>(a, true, s);
      else
        launch_proj_t<1, 2, 4>(a, true, s);
      break;
    case 1 * 8 + 4: launch_proj_t<1, 4, 2>(a, true, s); break;
    case 2 * 8 + 1: launch_proj_t<2, 1, 4>(a, true, s); break;
    case 2 * 8 + 2: launch_proj_t<2, 2, 4>(a, true, s); break;
    case 2 * 8 + 4:   // one round: pipelined (in_proj at 17 rows 61.6 -> 57.5 us)
      if (a.p[0].blocks + a.p[1].blocks <= kPjCUs)
        launch_proj_t<2, 4, 1>(a, true, s);
      else
        launch_proj_t<2, 4, 2>(a, true, s);
      break;
    case 4 * 8 + 1: launch_proj_t<4, 1, 4>(a, stream, s); break;
    case 4 * 8 + 2: launch_proj_t<4, 2, 4>(a, stream, s); break;
    // 4 x 4: the staged fold measured faster with a workgroup or more per CU
    // (in_proj at 64 rows, 256 tiles: 119.7 -> 114.3 us; 128 rows: 206.6 ->
    // 203.6), slower below (out_proj at 128 rows, 160 tiles: 116.6 -> 117.2).
    // A staged launch of one round takes the pipelined loop (in_proj at 33
    // and 64 rows: 102.9 -> 97.1 and 114.3 -> 107.9 us); with the one-buffer
    // fold it measured slower (out_proj at 192 rows, 240 tiles: 117.9 ->
    // 122.9 us), and so did launches of several rounds.
    default:
      if (a.p[0].blocks + a.p[1].blocks >= kPjStagedMin) {
        if (a.p[0].blocks + a.p[1].blocks <= kPjCUs)
          launch_proj_t<4, 4, 1, true>(a, stream, s);
        else
          launch_proj_t<4, 4, 2, true>(a, stream, s);
      } else {
        launch_proj_t<4, 4, 2>(a, stream, s);
      }
      break;
  }
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------
// Dense layer projections with 4-bit weights
// ---------------------------------------------------------------------------
//
// Up to 16 rows the product streams 0.56 bytes per weight.  A VALU kernel that
// forms each weight n s in fp32 and runs an fma chain per row spends about
// 1.75 + rows instructions per weight and is instruction-bound from 2 rows
// on.  Here the products run on the fp16 matrix cores
// (v_mfma_f32_16x16x32_f16, 16 row slots x 16 outputs x 32 columns, fp32
// accumulation), with every operand exact:
//  - the 4-bit value n is exact in binary16: two biased values u = n + 8 are
//    masked into the mantissas of a binary16 pair, (w & m) | 0x6400 6400,
//    giving 1024 + u or 1024 + 16 u, and one packed fp16 add or fma gives n
//    (1024 + u - 1032, or (1024 + 16 u) / 16 - 72): nine instructions per 8
//    weights;
//  - x is scaled by a power of two 2^k per row and 256-column chunk (the
//    chunk's largest magnitude lands in [2^14, 2^15)) and split into three
//    binary16 parts, x1 = rn(2^k x), x2 = rn(2^k x - x1) and x3 =
//    rn(2^k x - x1 - x2), whose sum is 2^k x exactly for every element of at
//    least 2^-15 of the chunk's largest magnitude (11 + 11 + 11 bits hold its
//    24; a smaller one is off by under 2^-39 of that magnitude); the parts of
//    a row take three of the four row slots one lane of the product holds,
//    so one instruction covers 4 rows;
//  - the block's binary16 scale s multiplies the fp32 sum of the block in a
//    mixed-precision fma (exact conversion, one rounding).
// The MFMA's result for one output does not depend on the other slots or on
// its own slot position, so a row's bits do not depend on the row count.
//
// Summation order of y[r][o], fixed and independent of the row count: C is cut
// into 4 quarters; in quarter q, for each chunk of 8 blocks of 32 columns,
// cacc = +0 and for each block j in order cacc = fma(T_j, s[o][j], cacc) with
// T_j = (D1_j + D2_j) + D3_j (the MFMA dot products of the block's n with x1,
// x2 and x3);
// the chunk's cacc, scaled back by 2^-k, is added to acc_q (+0 first);
// y = (acc_0 + acc_1) + (acc_2 + acc_3).  The launch shapes all compute
// exactly that:
//  - one 16-wave workgroup per group of 4 column tiles (64 outputs; wave =
//    column tile x quarter), the quarter sums folded in LDS, for launches of
//    up to 4 rows with enough groups to fill the chip;
//  - two workgroups per group of 4 column tiles (quarters 0-1 and 2-3),
//    each adding its half into y, which a fill kernel zeroed first.  With
//    exactly two addends on +0 the result does not depend on their arrival
//    order (fp addition is commutative, and none of these sums is -0), so the
//    shapes give the same bits.  Used for launches with fewer groups than the
//    chip has CUs (out_proj: 80 groups) and for 5 to 16 rows; at 5 to 8 rows
//    each wave takes two column tiles, which share every x operand read.
// Each row's x is split once per workgroup.  For 1 to 3 rows all of it is
// staged up front, compactly (only the live row slots; a slot past the rows
// reads a live slot's x, and its result is never stored), and the K loop runs
// without a barrier (proj_q4_pre_kernel).  For more rows it is staged chunk by
// chunk into two alternating LDS buffers, one barrier per chunk, its loads
// issued two chunks ahead (proj_q4_kernel).  Either way each lane converts 8
// columns of a row, and the 32 lanes of a row's chunk reduce its largest
// magnitude with lane exchanges.  The weights stream two chunks ahead of use.
//
// Packed layout, per 16-output column tile t and chunk m of 8 blocks of 32
// columns (2304 bytes, t-major): dword 8 (16 d + o) + i holds output
// 16 t + o's biased values u = n + 8 of columns 256 m + 32 i + 8 d + k,
// k = 0..7, value k at bit 4 (k >> 1) + 16 (k & 1), so that lane 16 d + o
// reads its 8 blocks of the chunk as 32 contiguous bytes; then at 2048 + 16 o
// the 8 binary16 scales of output 16 t + o for the chunk's blocks.

// launches that one workgroup per 4 column tiles would give fewer workgroups
// than this take two workgroups per group
constexpr int kQ4SplitBelow = 256;
constexpr int Q4_CH = 8;                       // blocks per quarter per chunk
constexpr int Q4_TC = 2304;                    // bytes per column tile and chunk
// a buffer offset beyond every resource's range: the load returns zeros and
// touches no memory (prefetch of the chunk after the last)
constexpr int Q4_OOB = (int)0x80000000u;

struct Q4Problem {
  const uint8_t *W;
  float *y;
  int R;
  int wgs;                                     // workgroups: R / 64, x 2 when split
};
struct Q4Args {
  const float *x;
  int rows;
  int C;
  Q4Problem p[2];
};

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

// (x & m) | c: one v_and_or_b32.  No inline assembly may write a vector
// register in these kernels: the compiler's hazard checks do not see its
// writes, and a result lane that no code reads (the pad slot of the matrix
// product) is written late by the matrix core, over whatever the compiler
// placed in that register meanwhile.
static __device__ __forceinline__ unsigned and_or(unsigned x, unsigned m, unsigned c) {
  return (x & m) | c;
}

// 8 biased 4-bit values of one output (one packed dword) -> the binary16
// values n, exact, in column order
static __device__ __forceinline__ h8 q4_decode(unsigned w, unsigned magic) {
  const h2 m1032 = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const h2 r16 = {(_Float16)0.0625f, (_Float16)0.0625f};
  const h2 m72 = {(_Float16)-72.0f, (_Float16)-72.0f};
  const unsigned w8 = w >> 8;
  const h2 a = __builtin_bit_cast(h2, and_or(w, 0x000f000fu, magic)) + m1032;
  const h2 b = __builtin_elementwise_fma(__builtin_bit_cast(h2, and_or(w, 0x00f000f0u, magic)),
                                         r16, m72);
  const h2 c = __builtin_bit_cast(h2, and_or(w8, 0x000f000fu, magic)) + m1032;
  const h2 d = __builtin_elementwise_fma(__builtin_bit_cast(h2, and_or(w8, 0x00f000f0u, magic)),
                                         r16, m72);
  return h8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// v - (float)h (h the low or high binary16 of p): exact, since h is v
// rounded to binary16.  m1 is -1 held in a register the compiler cannot see
// through, so the fma stays one mixed-precision instruction reading the
// binary16 half directly (with a literal -1 it becomes a conversion and a
// subtraction).
template <bool HI>
static __device__ __forceinline__ float minus_half(unsigned p, float v, float m1) {
  const float h = (float)__builtin_bit_cast(_Float16, (unsigned short)(HI ? p >> 16 : p & 0xffffu));
  return __builtin_fmaf(h, m1, v);
}

static __device__ __forceinline__ unsigned pk_half(float a, float b) {
  typedef float f2v __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(unsigned, __builtin_convertvector((f2v){a, b}, h2));
}

// 8 consecutive x of one row -> the chunk's exponent k (shared by the 32 lanes
// of the row's chunk, which hold its 256 columns) and the three binary16 parts
// of 2^k x, each as 4 packed pairs.  An infinite x: k comes from the chunk's
// largest finite magnitude (an infinite one would leave k = 15 and overflow
// the chunk's other values to infinities), the infinity reaches the sum
// through the first part, and its NaN residuals are replaced by finite values
// with a packed max (which passes over NaN); waves without an infinite x skip
// both.  m1: -1 (minus_half).  Every lane of the wave calls this together.
static __device__ __forceinline__ int x_split(const f4 &x0, const f4 &x1, unsigned (&p1)[4],
                                              unsigned (&p2)[4], unsigned (&p3)[4], float m1) {
  const float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < 8; e++) m = fmaxf(m, fabsf(v[e]));     // NaN is passed over
  auto half_wave_max = [](float mm) {
    mm = fmaxf(mm, lane_xor<16>(mm));
    mm = fmaxf(mm, lane_xor<8>(mm));
    mm = fmaxf(mm, lane_xor<4>(mm));
    mm = fmaxf(mm, lane_xor<2>(mm));
    return fmaxf(mm, lane_xor<1>(mm));
  };
  m = half_wave_max(m);
  const bool inf = __builtin_amdgcn_ballot_w64(m > 3.4028235e38f) != 0;   // wave-uniform
  if (inf) {
    m = 0.f;
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const float a = fabsf(v[e]);
      m = fmaxf(m, a <= 3.4028235e38f ? a : 0.f);
    }
    m = half_wave_max(m);
  }
  // largest finite magnitude in [2^14, 2^15) after scaling (m = 0: any k)
  const int k = 15 - __builtin_amdgcn_frexp_expf(m);
#pragma unroll
  for (int e = 0; e < 4; e++) {
    const float s0 = __builtin_amdgcn_ldexpf(v[2 * e], k);
    const float s1 = __builtin_amdgcn_ldexpf(v[2 * e + 1], k);
    p1[e] = pk_half(s0, s1);
    const float r0 = minus_half<false>(p1[e], s0, m1), r1 = minus_half<true>(p1[e], s1, m1);
    p2[e] = pk_half(r0, r1);
    const float t0 = minus_half<false>(p2[e], r0, m1), t1 = minus_half<true>(p2[e], r1, m1);
    p3[e] = pk_half(t0, t1);
  }
  if (inf) {
    const h2 lo = {(_Float16)-65504.0f, (_Float16)-65504.0f};
#pragma unroll
    for (int e = 0; e < 4; e++) {
      p2[e] = __builtin_bit_cast(unsigned,
                                 __builtin_elementwise_max(__builtin_bit_cast(h2, p2[e]), lo));
      p3[e] = __builtin_bit_cast(unsigned,
                                 __builtin_elementwise_max(__builtin_bit_cast(h2, p3[e]), lo));
    }
  }
  return k;
}

// NT: row tiles of 4 rows (rows <= 4 NT); SPLIT: two workgroups per group of
// CT TW column tiles (quarters 0-1 and 2-3), else one (all four quarters); TW:
// column tiles per wave, which share each x operand read
template <int NT, bool SPLIT, int CT, int TW>
__global__ __launch_bounds__(64 * CT * (SPLIT ? 2 : 4)) void proj_q4_kernel(Q4Args a) {
  static_assert(CT == 2 || CT == 4, "4 or 2 wave columns per workgroup");
  static_assert(TW == 1 || TW == 2, "1 or 2 column tiles per wave");
  constexpr int NQ = SPLIT ? 2 : 4;            // quarters per workgroup
  constexpr int NTHR = 64 * CT * NQ;
  constexpr int STAGE = NQ * Q4_CH * NT * 1024;
  __shared__ __align__(16) unsigned char xs[2][STAGE];
  __shared__ int kexp[2][NQ][4 * NT];
  const int bid = (int)xcd_contiguous(blockIdx.x, gridDim.x);
  const bool second = bid >= a.p[0].wgs;
  const uint8_t *W = second ? a.p[1].W : a.p[0].W;
  float *y = second ? a.p[1].y : a.p[0].y;
  const int R = second ? a.p[1].R : a.p[0].R;
  const int gh = second ? bid - a.p[0].wgs : bid;
  const int g = SPLIT ? gh >> 1 : gh;
  const int q0 = SPLIT ? 2 * (gh & 1) : 0;     // first quarter of this workgroup
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  float m1 = -1.0f;                            // x_split's -1, kept in a register
  __asm__("" : "+v"(m1));                      // (no instruction; defined before any product)
  const int ct = wave % CT, qw = wave / CT;
  const int q = q0 + qw;
  const int C = a.C, rows = a.rows, nblk = C / 32, Q = nblk / 4, nch = Q / Q4_CH;
  const int tile = (CT * g + ct) * TW;         // the wave's first column tile
  const int tbytes = nblk / Q4_CH * Q4_TC;     // packed bytes of one column tile
  const rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(W + (int64_t)tile * tbytes), 0, TW * tbytes, RSRC_FLAGS);

  // zero both stage buffers: the pad slot of every row and the slots past
  // `rows` stay zero
  for (int i = tid; i < 2 * STAGE / 16; i += NTHR)
    reinterpret_cast<u4 *>(&xs[0][0])[i] = u4{0, 0, 0, 0};

  // x staging: item = (quarter slot, row, block in chunk, d) with d, then the
  // block, fastest, so the 32 lanes of a row's chunk are one half-wave; at
  // most NQ 4 NT 32 items, ITEMS per lane.  Stage layout: per quarter slot,
  // block and row tile a 1 KiB operand tile, row slot s of column group d at
  // 16 (16 d + (s ^ i ^ 8 (d & 1))) for block i of the chunk (row r, part p:
  // slot 4 (r % 4) + p).
  constexpr int ITEMS = (2 * NT + CT - 1) / CT;
  const int nitems = NQ * rows * Q4_CH * 4;
  // the lane's items, the same in every chunk: x element offset in chunk 0
  // (-1: no item), LDS byte offset, exponent slot
  int xoff[ITEMS], xdst[ITEMS], xkix[ITEMS];
#pragma unroll
  for (int it = 0; it < ITEMS; it++) {
    const int idx = tid + it * NTHR;
    const bool ok = idx < nitems;
    const int d = idx & 3, i = (idx >> 2) & 7, rest = idx >> 5;
    const int bb = ok ? rest % rows : 0, qi = ok ? rest / rows : 0;
    xoff[it] = ok ? bb * C + ((q0 + qi) * Q + i) * 32 + 8 * d : -1;
    xdst[it] = ((qi * Q4_CH + i) * NT + bb / 4) * 1024 +
               16 * (16 * d + ((4 * (bb % 4)) ^ i ^ (8 * (d & 1))));
    xkix[it] = qi * 4 * NT + bb;
  }
  // x of a chunk, in three register sets rotating with the weight sets
  struct XSet {
    f4 v[ITEMS][2];
  };
  // buffer loads with an out-of-range offset for a missing item: no branch,
  // so the wait counts stay exact
  const rsrc_t xr = buf_rsrc(a.x, rows * C * 4);
  auto x_issue = [&](XSet &xv, int ch) {
#pragma unroll
    for (int it = 0; it < ITEMS; it++) {
      const bool ok = xoff[it] >= 0 && ch < nch;
      const int vo = ok ? 4 * (xoff[it] + ch * Q4_CH * 32) : Q4_OOB;
      xv.v[it][0] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(xr, vo, 0, 0));
      xv.v[it][1] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(xr, vo, 16, 0));
    }
  };
  auto x_stage = [&](const XSet &xv, int ch) {
    unsigned char *buf = xs[ch & 1];
#pragma unroll
    for (int it = 0; it < ITEMS; it++) {
      unsigned p1[4], p2[4], p3[4];
      const int k = x_split(xv.v[it][0], xv.v[it][1], p1, p2, p3, m1);
      if (xoff[it] >= 0) {
        *reinterpret_cast<u4 *>(buf + xdst[it]) = u4{p1[0], p1[1], p1[2], p1[3]};
        *reinterpret_cast<u4 *>(buf + (xdst[it] ^ 16)) = u4{p2[0], p2[1], p2[2], p2[3]};
        *reinterpret_cast<u4 *>(buf + (xdst[it] ^ 32)) = u4{p3[0], p3[1], p3[2], p3[3]};
        if ((l & 31) == 0) (&kexp[ch & 1][0][0])[xkix[it]] = k;
      }
    }
  };

  // weights of chunk ch, per column tile of the wave: the lane's 8 dwords
  // (blocks q Q + ch CH + 0..7) and its output's 8 scales, three 128-bit loads
  struct WSet {
    u4 w0[TW], w1[TW], s[TW];
  };
  auto w_issue = [&](WSet &ws, int ch) {
    const bool ok = ch < nch;
    const int so = __builtin_amdgcn_readfirstlane((ok ? q * nch + ch : 0) * Q4_TC);
#pragma unroll
    for (int tw = 0; tw < TW; tw++) {
      ws.w0[tw] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(
                                             wr, ok ? 32 * l : Q4_OOB, so + tw * tbytes,
                                             POL_STREAM_LOAD));
      ws.w1[tw] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(
                                             wr, ok ? 32 * l + 16 : Q4_OOB, so + tw * tbytes,
                                             POL_STREAM_LOAD));
      ws.s[tw] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(
                                            wr, ok ? 2048 + 16 * (l & 15) : Q4_OOB,
                                            so + tw * tbytes, POL_STREAM_LOAD));
    }
  };

  // Loads return in order, so a chunk's x is requested two chunks ahead,
  // before the weights it would otherwise wait behind.
  WSet S0, S1, S2;
  XSet X0, X1, X2;
  x_issue(X0, 0);
  w_issue(S0, 0);
  x_issue(X1, 1);
  w_issue(S1, 1);
  __syncthreads();                             // zeroed buffers before staging
  x_stage(X0, 0);
  __syncthreads();

  unsigned magic = 0x64006400u;                // binary16 1024 in both halves
  __asm__("" : "+v"(magic));                   // kept in a vector register
  float acc[TW][NT];
#pragma unroll
  for (int tw = 0; tw < TW; tw++)
#pragma unroll
    for (int t = 0; t < NT; t++) acc[tw][t] = 0.f;
  // blocks whose products are in flight together
  constexpr int GB = TW == 1 ? (NT == 1 ? 4 : 2) : (NT <= 2 ? 2 : 1);

  // one chunk: issue chunk ch + 2's x and weights, compute chunk ch, stage
  // chunk ch + 1's x, one barrier
  auto chunk = [&](const WSet &cur, WSet &pf, const XSet &xn, XSet &xf, int ch) {
    x_issue(xf, ch + 2);
    w_issue(pf, ch + 2);
    if (ch < nch) {
      // lane l reads slot l % 16 of column group l / 16, at the writers'
      // swizzled place
      const unsigned char *buf = xs[ch & 1] + (qw * Q4_CH) * NT * 1024;
      const int lx = 16 * (l ^ ((l >> 1) & 8));
      float cacc[TW][NT];
#pragma unroll
      for (int tw = 0; tw < TW; tw++)
#pragma unroll
        for (int t = 0; t < NT; t++) cacc[tw][t] = 0.f;
#pragma unroll
      for (int h = 0; h < Q4_CH / GB; h++) {
        f4 D[GB][NT][TW];
        float sv[GB][TW];
#pragma unroll
        for (int j = 0; j < GB; j++) {
          const int i = GB * h + j;
          h8 B[TW];
#pragma unroll
          for (int tw = 0; tw < TW; tw++) {
            B[tw] = q4_decode(i < 4 ? cur.w0[tw][i] : cur.w1[tw][i - 4], magic);
            const unsigned sw = cur.s[tw][i >> 1];
            sv[j][tw] = (float)__builtin_bit_cast(
                _Float16, (unsigned short)((i & 1) ? sw >> 16 : sw & 0xffffu));
          }
#pragma unroll
          for (int t = 0; t < NT; t++) {
            const h8 A =
                *reinterpret_cast<const h8 *>(buf + (i * NT + t) * 1024 + (lx ^ (16 * i)));
#pragma unroll
            for (int tw = 0; tw < TW; tw++)
              D[j][t][tw] =
                  __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B[tw], f4{0, 0, 0, 0}, 0, 0, 0);
          }
        }
        // the lane's row of each tile: its three parts' sums
#pragma unroll
        for (int j = 0; j < GB; j++)
#pragma unroll
          for (int t = 0; t < NT; t++)
#pragma unroll
            for (int tw = 0; tw < TW; tw++)
              cacc[tw][t] = __builtin_fmaf((D[j][t][tw].x + D[j][t][tw].y) + D[j][t][tw].z,
                                           sv[j][tw], cacc[tw][t]);
      }
#pragma unroll
      for (int t = 0; t < NT; t++) {
        const int k = kexp[ch & 1][qw][4 * t + (l >> 4)];
#pragma unroll
        for (int tw = 0; tw < TW; tw++)
          acc[tw][t] = acc[tw][t] + __builtin_amdgcn_ldexpf(cacc[tw][t], -k);
      }
    }
    if (ch + 1 < nch) x_stage(xn, ch + 1);
    __syncthreads();
  };
  for (int ch = 0; ch < nch; ch += 3) {
    chunk(S0, S2, X1, X2, ch);
    chunk(S1, S0, X2, X0, ch + 1);
    chunk(S2, S1, X0, X1, ch + 2);
  }

  // fold the quarters: wave (ct, qw) -> LDS; the first quarter's waves add
  float *fold = reinterpret_cast<float *>(&xs[0][0]);   // [ct][qw][tw][t][64]
  static_assert(CT * NQ * TW * NT * 256 <= 2 * STAGE, "fold fits the stage buffers");
#pragma unroll
  for (int tw = 0; tw < TW; tw++)
#pragma unroll
    for (int t = 0; t < NT; t++) fold[(((ct * NQ + qw) * TW + tw) * NT + t) * 64 + l] = acc[tw][t];
  __syncthreads();
  if (qw == 0) {
#pragma unroll
    for (int tw = 0; tw < TW; tw++)
#pragma unroll
      for (int t = 0; t < NT; t++) {
        auto at = [&](int qq) { return fold[(((ct * NQ + qq) * TW + tw) * NT + t) * 64 + l]; };
        const int row = 4 * t + (l >> 4);
        float v = acc[tw][t] + at(1);
        if constexpr (!SPLIT) v = v + (at(2) + at(3));
        if (row < rows) {
          float *dst = y + (int64_t)row * R + 16 * (tile + tw) + (l & 15);
          if constexpr (SPLIT)
            atomicAdd(dst, v);                 // two addends on +0: order-free
          else
            *dst = v;
        }
      }
  }
}

// Launches of few rows stage all of their x once, compactly (the three parts
// of each live row), and then run the K loop without barriers: LDS bytes for
// the x parts of a workgroup's column range (half of C when split: two such
// workgroups fit a CU; one row of C <= 6826 for one column tile per
// workgroup: four fit), and ints for its chunk exponents.
constexpr int q4_pre_bytes(bool split, int ct) {
  return split ? 57344 : ct == 1 ? 40960 : 98304;
}
constexpr int Q4_PRE_K = 256;

// The same order as proj_q4_kernel for NR rows (1..3), every x chunk staged
// in the prologue.
template <bool SPLIT, int CT, int NR>
__global__ __launch_bounds__(64 * CT * (SPLIT ? 2 : 4)) void proj_q4_pre_kernel(Q4Args a) {
  static_assert(CT == 1 || CT == 2 || CT == 4, "4, 2 or 1 column tiles per workgroup");
  constexpr int NQ = SPLIT ? 2 : 4;            // quarters per workgroup
  constexpr int NTHR = 64 * CT * NQ;
  // x parts [block of the range][d][row][part][16 bytes]
  __shared__ __align__(16) unsigned char xp[q4_pre_bytes(SPLIT, CT)];
  __shared__ int kp[Q4_PRE_K];                 // [row][chunk of the range]
  const int bid = (int)xcd_contiguous(blockIdx.x, gridDim.x);
  const bool second = bid >= a.p[0].wgs;
  const uint8_t *W = second ? a.p[1].W : a.p[0].W;
  float *y = second ? a.p[1].y : a.p[0].y;
  const int R = second ? a.p[1].R : a.p[0].R;
  const int gh = second ? bid - a.p[0].wgs : bid;
  const int g = SPLIT ? gh >> 1 : gh;
  const int q0 = SPLIT ? 2 * (gh & 1) : 0;     // first quarter of this workgroup
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  float m1 = -1.0f;                            // x_split's -1, kept in a register
  __asm__("" : "+v"(m1));                      // (no instruction; defined before any product)
  const int ct = wave % CT, qw = wave / CT;
  const int q = q0 + qw;
  constexpr int rows = NR, S3 = 3 * NR;        // live row slots (three parts per row)
  const int C = a.C, nblk = C / 32, Q = nblk / 4, nch = Q / Q4_CH;
  const int ncw = NQ * nch;                    // chunks of the workgroup's range
  const int tile = CT * g + ct;
  const rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(W + (int64_t)tile * (nblk / Q4_CH) * Q4_TC), 0,
      nblk / Q4_CH * Q4_TC, RSRC_FLAGS);

  struct WSet {
    u4 w0, w1, s;
  };
  auto w_issue = [&](WSet &ws, int ch) {
    const bool ok = ch < nch;
    const int so = __builtin_amdgcn_readfirstlane((ok ? q * nch + ch : 0) * Q4_TC);
    ws.w0 = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(
                                       wr, ok ? 32 * l : Q4_OOB, so, POL_STREAM_LOAD));
    ws.w1 = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(
                                       wr, ok ? 32 * l + 16 : Q4_OOB, so, POL_STREAM_LOAD));
    ws.s = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(
                                      wr, ok ? 2048 + 16 * (l & 15) : Q4_OOB, so,
                                      POL_STREAM_LOAD));
  };

  // stage every chunk: item = (row, chunk, block in chunk, d) with d, then the
  // block, fastest (the 32 lanes of a row's chunk are one half-wave); the
  // trip count is uniform, so every exchange has its partner lane active.
  // The first trip's x is requested before the first weights (loads return
  // in order), so staging does not wait for the weight stream.
  const int nitems = rows * ncw * 32;
  const rsrc_t xr = buf_rsrc(a.x, rows * C * 4);
  auto x_load = [&](int base, f4 &x0, f4 &x1) {
    const int idx = base + tid;
    const bool ok = idx < nitems;
    const int d = idx & 3, i = (idx >> 2) & 7, rest = idx >> 5;
    const int c = ok ? rest % ncw : 0, bb = ok ? rest / ncw : 0;
    const int vo = ok ? 4 * (bb * C + (q0 * Q + c * Q4_CH + i) * 32 + 8 * d) : Q4_OOB;
    x0 = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(xr, vo, 0, 0));
    x1 = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(xr, vo, 16, 0));
  };
  f4 xn0, xn1;
  x_load(0, xn0, xn1);
  WSet S0, S1, S2w;
  w_issue(S0, 0);
  w_issue(S1, 1);
  for (int base = 0; base < nitems; base += NTHR) {
    const int idx = base + tid;
    const bool ok = idx < nitems;
    const int d = idx & 3, i = (idx >> 2) & 7, rest = idx >> 5;
    const int c = ok ? rest % ncw : 0, bb = ok ? rest / ncw : 0;
    f4 x0 = xn0, x1 = xn1;
    if (base > 0) x_load(base, x0, x1);
    unsigned p1[4], p2[4], p3[4];
    const int k = x_split(x0, x1, p1, p2, p3, m1);
    if (ok) {
      unsigned char *dst = xp + (((c * Q4_CH + i) * 4 + d) * S3 + 3 * bb) * 16;
      *reinterpret_cast<u4 *>(dst) = u4{p1[0], p1[1], p1[2], p1[3]};
      *reinterpret_cast<u4 *>(dst + 16) = u4{p2[0], p2[1], p2[2], p2[3]};
      *reinterpret_cast<u4 *>(dst + 32) = u4{p3[0], p3[1], p3[2], p3[3]};
      if ((l & 31) == 0) kp[bb * ncw + c] = k;
    }
  }
  __syncthreads();

  unsigned magic = 0x64006400u;                // binary16 1024 in both halves
  __asm__("" : "+v"(magic));                   // kept in a vector register
  // lane l supplies row slot l % 16 (row (l % 16) / 4, part l % 4) of column
  // group l / 16; a row past `rows` and the pad part read a live slot's x:
  // their results belong to no row and are never stored (a slot's result
  // does not depend on the others)
  const int sl = l & 15, dl = l >> 4;
  const int lrow = (sl >> 2) % rows, lpart = (sl & 3) == 3 ? 0 : (sl & 3);
  const unsigned char *xl = xp + (dl * S3 + 3 * lrow + lpart) * 16;
  const int row = l >> 4;                      // the lane's result row
  const int krow = (row < rows ? row : 0) * ncw + qw * nch;
  float acc = 0.f;
  auto chunk = [&](const WSet &cur, WSet &pf, int ch) {
    w_issue(pf, ch + 2);
    if (ch < nch) {
      const int jr0 = qw * Q + ch * Q4_CH;     // first block of the chunk in the range
      float cacc = 0.f;
#pragma unroll
      for (int h = 0; h < 2; h++) {
        f4 D[4];
        float sv[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const int i = 4 * h + j;
          const h8 B = q4_decode(h ? cur.w1[j] : cur.w0[j], magic);
          const unsigned sw = cur.s[i >> 1];
          sv[j] = (float)__builtin_bit_cast(_Float16,
                                            (unsigned short)((i & 1) ? sw >> 16 : sw & 0xffffu));
          const h8 A = *reinterpret_cast<const h8 *>(xl + (jr0 + i) * 64 * S3);
          D[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B, f4{0, 0, 0, 0}, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 4; j++)
          cacc = __builtin_fmaf((D[j].x + D[j].y) + D[j].z, sv[j], cacc);
      }
      acc = acc + __builtin_amdgcn_ldexpf(cacc, -kp[krow + ch]);
    }
  };
  for (int ch = 0; ch < nch; ch += 3) {
    chunk(S0, S2w, ch);
    chunk(S1, S0, ch + 1);
    chunk(S2w, S1, ch + 2);
  }

  // fold the quarters (as proj_q4_kernel)
  __syncthreads();                             // every x read before the fold writes
  float *fold = reinterpret_cast<float *>(xp);   // [ct][qw][64]
  fold[(ct * NQ + qw) * 64 + l] = acc;
  __syncthreads();
  if (qw == 0) {
    auto at = [&](int qq) { return fold[(ct * NQ + qq) * 64 + l]; };
    float v = acc + at(1);
    if constexpr (!SPLIT) v = v + (at(2) + at(3));
    if (row < rows) {
      float *dst = y + (int64_t)row * R + 16 * tile + sl;
      if constexpr (SPLIT)
        atomicAdd(dst, v);                     // two addends on +0: order-free
      else
        *dst = v;
    }
  }
}

// 4-bit packing: thread (output o, block b) writes o's four dwords of block b
// and its scale.
__global__ __launch_bounds__(256) void proj_q4_pack_kernel(const uint8_t *q, const uint16_t *scale,
                                                           uint8_t *Wq, int C, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int nblk = C / 32;
  const int64_t o = i / nblk;
  const int bb = (int)(i - o * nblk);
  const int64_t t = o >> 4;
  const int oi = (int)(o & 15), m = bb / Q4_CH, i8 = bb % Q4_CH;
  const uint8_t *src = q + o * (C / 2) + 16 * bb;
  auto u = [&](int c) -> unsigned {            // biased value of column c of the block
    const unsigned by = src[c >> 1];
    return (((c & 1) ? by >> 4 : by) & 15u) ^ 8u;
  };
  unsigned *dst = reinterpret_cast<unsigned *>(Wq + (t * (nblk / Q4_CH) + m) * Q4_TC);
#pragma unroll
  for (int d = 0; d < 4; d++) {
    unsigned wd = 0;
#pragma unroll
    for (int k = 0; k < 8; k++) wd |= u(8 * d + k) << (4 * (k >> 1) + 16 * (k & 1));
    dst[8 * (16 * d + oi) + i8] = wd;
  }
  reinterpret_cast<uint16_t *>(dst + 512 + 4 * oi)[i8] = scale[o * nblk + bb];
}

int launch_proj_q4_pack(const uint8_t *q, const uint16_t *scale, void *Wq, int R, int C,
                        hipStream_t s) {
  const int64_t n = (int64_t)R * (C / 32);
  if (n <= 0) return 0;
  hipLaunchKernelGGL(proj_q4_pack_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, q,
                     scale, static_cast<uint8_t *>(Wq), C, n);
  return (int)hipGetLastError();
}

template <int NT, bool SPLIT, int CT, int TW = 1>
static void launch_q4(const Q4Args &a, hipStream_t s) {
  hipLaunchKernelGGL((proj_q4_kernel<NT, SPLIT, CT, TW>), dim3((unsigned)(a.p[0].wgs + a.p[1].wgs)),
                     dim3(64 * CT * (SPLIT ? 2 : 4)), 0, s, a);
}
template <bool SPLIT, int CT>
static void launch_q4_pre(const Q4Args &a, hipStream_t s) {
  const dim3 grid((unsigned)(a.p[0].wgs + a.p[1].wgs)), block(64 * CT * (SPLIT ? 2 : 4));
  if (a.rows == 1)
    hipLaunchKernelGGL((proj_q4_pre_kernel<SPLIT, CT, 1>), grid, block, 0, s, a);
  else if (a.rows == 2)
    hipLaunchKernelGGL((proj_q4_pre_kernel<SPLIT, CT, 2>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((proj_q4_pre_kernel<SPLIT, CT, 3>), grid, block, 0, s, a);
}

int launch_proj_q4(const float *x, int64_t rows, int C, const void *Wq0, int R0, float *y0,
                   const void *Wq1, int R1, float *y1, hipStream_t s) {
  if (rows <= 0) return 0;
  if (rows > 16 || C % 1024 != 0) return (int)hipErrorInvalidValue;
  // Launch shape (every shape gives the same bits): one 16-wave workgroup per
  // 4 column tiles when that fills the chip and rows <= 4; else two
  // workgroups per group of 4 TW tiles (the 5-16 row instances of one
  // workgroup per group would be held to 128 VGPRs), TW = 2 for 5-8 rows when
  // the groups of 8 tiles still fill the chip (at 9-16 rows the pair of tiles
  // would spill).  Fewer, fuller workgroups beat more of 2 tiles each: with 4
  // wave columns the split of x is shared by twice the waves.
  const int tiles = R0 / 16 + (Wq1 ? R1 / 16 : 0);
  // one row, too few groups of 4 tiles, enough single tiles: one workgroup
  // per tile, the up-front stage of x small enough for four per CU
  const bool tile1 = rows == 1 && tiles / 4 < kQ4SplitBelow && tiles >= kQ4SplitBelow &&
                     C / 32 * 192 <= q4_pre_bytes(false, 1);
  // 5-8 rows: two column tiles per wave (one x operand read serves both)
  // when two workgroups per group of 8 tiles still fill the chip
  const bool pair = rows > 4 && rows <= 8 && R0 % 128 == 0 && (!Wq1 || R1 % 128 == 0) &&
                    tiles / 8 * 2 >= kQ4SplitBelow;
  const bool split = (tiles / 4 < kQ4SplitBelow || rows > 4) && !tile1;
  const int ct = tile1 ? 1 : 4;
  const int f = split ? 2 : 1;
  const int tw = pair ? 2 : 1;
  Q4Args a{};
  a.x = x;
  a.rows = (int)rows;
  a.C = C;
  a.p[0] = Q4Problem{static_cast<const uint8_t *>(Wq0), y0, R0, R0 / 16 / (ct * tw) * f};
  a.p[1] = Q4Problem{static_cast<const uint8_t *>(Wq1), y1, R1, Wq1 ? R1 / 16 / (ct * tw) * f : 0};
  if (split) {
    const int64_t n0 = rows * R0, n1 = Wq1 ? rows * R1 : 0;
    hipLaunchKernelGGL(zero2_kernel, dim3((unsigned)((n0 + n1 + 255) / 256)), dim3(256), 0, s,
                       y0, n0, y1, n1);
  }
  // all of a workgroup's x staged up front when it fits
  const int range = split ? C / 2 : C;
  const bool pre = rows <= 3 && (int64_t)range / 32 * 192 * rows <= q4_pre_bytes(split, ct) &&
                   (int64_t)range / 256 * rows <= Q4_PRE_K;
  if (tile1)
    hipLaunchKernelGGL((proj_q4_pre_kernel<false, 1, 1>), dim3((unsigned)(a.p[0].wgs + a.p[1].wgs)),
                       dim3(256), 0, s, a);
  else if (pre)
    !split ? launch_q4_pre<false, 4>(a, s) : launch_q4_pre<true, 4>(a, s);
  else if (!split)
    launch_q4<1, false, 4>(a, s);
  else if (rows <= 4)
    launch_q4<1, true, 4>(a, s);
  else if (rows <= 8)
    tw == 2 ? launch_q4<2, true, 4, 2>(a, s) : launch_q4<2, true, 4>(a, s);
  else
    launch_q4<4, true, 4>(a, s);
  return (int)hipGetLastError();
}

}  // namespace gdn
