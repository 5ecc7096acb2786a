// encode: query-aware (H-weighted) nearest-centroid assignment of keys, uint16 codes.
// "veloxquant_mlx.quantizers.a2ats module", a2ats_h_weighted_assignment (Eq. 14 through the
// Eq. 15-17 Cholesky identity):
//     code(k) = argmin_j (k - c_j) H (k - c_j)^T = argmin_j ||k L - c_j L||^2,   H = L L^T.
// With w_j = c_j L, v_j = w_j L^T (= c_j H) and b_j = ||w_j||^2, all exact in fp64,
//     ||kL - c_jL||^2 = ||kL||^2 - 2 (k . v_j - b_j / 2),
// so the code maximises the score s_j = k . v_j - b_j / 2: a dense contraction of the keys
// against the transformed codebook plus a row argmax.  Without L, H = I (plain nearest
// centroid, the bulk path of the first docs page's "How it works").
//
// Exactness.  The contraction runs on fp16 MFMA (bf16 keys are exact in fp16; the codebook
// side is rounded after a power-of-two scale S).  For each key the error of every MFMA score
// is bounded rigorously,
//     |acc_j - S s_j| <= E = |k| rho + |k - k16| nu + gamma (B + |k16| nu) + u B,
// (rho = max_j |S v_j - v16_j|, nu = max_j |v16_j|, B = max_j S b_j / 2, gamma covers the
// fp32 accumulation of 129 terms).  The MFMA winner is accepted only when the bound proves
// it; close calls are settled by fp32 scores of the two leading candidates under a rigorous
// error bound, and whatever is still open is rescanned and decided in fp64.
//
// Kernels (in launch order)
//   enc_prep_gram       M = L L^T in fp64 (H-weighted only).
//   enc_prep_rows       v = c M, b = v . c in fp64 (fp64 MFMA), ||fp32(v)|| per centroid,
//                       per-workgroup maxima.
//   enc_prep_frag       fp16 fragments of S v in MFMA A-operand order, fp32 bias -S b / 2 per
//                       accumulator slot, per-workgroup rho / nu; optional fp16 hi/lo
//                       fragments of L^T for ||kL||^2; clears the run state (list lengths,
//                       decision counters, candidate counts).
//   enc_znorm64         ||kL||^2 in fp64 (fp32 keys with distances and L only).
//   enc_coarse          the MFMA pass (with ||kL||^2 from L^T fragments when distances are
//                       wanted); writes directly certified codes; in its tail, fp32 scores of
//                       the two leading candidates of the other keys, formed from the exact
//                       key fragments in registers, settle most of them and list the rest
//                       for the rescan.
//   enc_rescan_collect  second MFMA pass over the keys still open: collects every centroid
//                       whose score could reach the best exact score (per wave in LDS, then
//                       one global atomic per key and work item to append them).
//   enc_rescan_decide   fp64 over the collected candidates; fp64 over the whole codebook for
//                       the keys listed for it (fp16 overflow, list overflow).
#include "common.hpp"

namespace a2ats {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef __fp16 h2rtz __attribute__((ext_vector_type(2)));

constexpr int kD = A2ATS_HEAD_DIM;
constexpr int kLd = kD + 1;               // padded LDS row of L (conflict-free column reads)
constexpr int kRows = 32;                 // centroids per MFMA tile
constexpr int kSteps = kD / 16;           // k-steps per tile (v_mfma_f32_32x32x16_f16)
constexpr int kFragPerTile = kSteps * 64; // half8 fragments per tile (8 KiB)
constexpr int kTPS = 4;                   // tiles per LDS stage of the coarse pass
constexpr int kKeysPerWG = 256;           // 4 waves x 64 keys
constexpr int kCandCap = 32;              // rescan candidates per key
constexpr int kDecideWgs = 1024;          // workgroups of the rescan decide pass (a multiple of 8)
constexpr float kPadBias = -1.0e38f;      // bias of padding rows: finite, never competitive

struct Counters {
  unsigned stat_x[8][16];    // keys, direct decisions, reranks per XCD (statistics only)
  unsigned full;             // full-scan list entries
  unsigned stats[8];         // [3] rescanned, [4] full scan
  unsigned done_grp[8][64];  // rescan-decide workgroups finished, per group blockIdx % 8 (256 B apart)
  unsigned done;             // groups finished (the last workgroup clears the run state)
  unsigned unc[1];           // per-head rescan list lengths follow (heads entries)
};

struct UncEntry {       // a key left open by the coarse pass
  int32_t row;
  int32_t jbest;        // the leading candidate
  double sbest;         // a lower bound of the best score (of jbest's at least)
  double e_unscaled;
  float z2;
  int32_t pad;
};

struct FullEntry {
  int32_t head, row;
  float z2;
  int32_t pad;
};

__device__ __forceinline__ float round_up_f(double x) {
  float f = (float)x;
  if ((double)f < x) f = __uint_as_float(__float_as_uint(f) + (f >= 0.f ? 1u : 0xFFFFFFFFu));
  return f;
}

__device__ __forceinline__ int ilog2_floor(float x) {  // x > 0, normal
  return (int)((__float_as_uint(x) >> 23) & 0xFF) - 127;
}

__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((unsigned)(e + 127) << 23); }

__device__ __forceinline__ float scale_for(float maxabs) {  // max |S x| in [2^14, 2^15)
  return maxabs > 0.f ? pow2f(14 - ilog2_floor(maxabs)) : 1.f;
}

// Accumulator slot r of a lane in half hh holds MFMA output row 8(r/4) + 4hh + (r%4).
__device__ __forceinline__ int slot_row(int r, int hh) { return 8 * (r >> 2) + 4 * hh + (r & 3); }

// Workgroup-aggregated list append: every thread of the workgroup calls it (uniform control
// flow); threads with want == true receive distinct slots of `*counter`.  One global atomic
// per workgroup instead of one per entry (same-address atomics serialise at the L2).
__device__ __forceinline__ unsigned block_append(unsigned* counter, bool want, unsigned* s_cnt,
                                                 unsigned* s_base) {
  __syncthreads();
  if (threadIdx.x == 0) *s_cnt = 0u;
  __syncthreads();
  const unsigned local = want ? atomicAdd(s_cnt, 1u) : 0u;
  __syncthreads();
  if (threadIdx.x == 0) *s_base = *s_cnt ? atomicAdd(counter, *s_cnt) : 0u;
  __syncthreads();
  return *s_base + local;
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// ------------------------------------------------------------------ prep
typedef double d4 __attribute__((ext_vector_type(4)));

// M = L L^T (fp64, symmetric) of one head, 8 rows of M per workgroup; workgroup 0 of a head
// also records max |L| in the head's first prep_rows partial.
__global__ __launch_bounds__(256) void enc_prep_gram(const float* __restrict__ chol,
                                                     double* __restrict__ gram,
                                                     float* __restrict__ part_a, int nwg) {
  __shared__ float Ls[kD * kLd];
  __shared__ float red[4];
  const int head = blockIdx.y, rb = blockIdx.x, t = threadIdx.x;
  const float* L = chol + (int64_t)head * kD * kD;
  float lmax = 0.f;
#pragma unroll 16
  for (int e = t; e < kD * kD; e += 256) {
    const float x = L[e];
    Ls[(e / kD) * kLd + e % kD] = x;
    lmax = fmaxf(lmax, fabsf(x));
  }
  __syncthreads();
  const int bcol = t % kD;          // column b of M
  const int a0 = rb * 8 + (t / kD) * 4;  // rows a0 .. a0+3
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  for (int k = 0; k < kD; ++k) {
    const double lb = (double)Ls[bcol * kLd + k];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += (double)Ls[(a0 + i) * kLd + k] * lb;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) gram[((int64_t)head * kD + a0 + i) * kD + bcol] = acc[i];
  if (rb == 0) {
    for (int o = 32; o > 0; o >>= 1) lmax = fmaxf(lmax, __shfl_xor(lmax, o));
    if ((t & 63) == 0) red[t >> 6] = lmax;
    __syncthreads();
    if (t == 0) part_a[((int64_t)head * nwg) * 4 + 2] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  }
}

// 32 codebook rows per workgroup: v = c M (fp64 MFMA, M = L L^T; v = c without L) and
// b = v . c (= ||c L||^2), written as fp64 and fp32, plus this workgroup's max |v| and
// max b.  Wave w computes columns 32w .. 32w+31 as 2 x 2 tiles of 16 x 16.
__global__ __launch_bounds__(256) void enc_prep_rows(const float* __restrict__ cb, int64_t c,
                                                     const double* __restrict__ gram,
                                                     double* __restrict__ v64,
                                                     float* __restrict__ v32,
                                                     double* __restrict__ b64,
                                                     float* __restrict__ vnorm,
                                                     float* __restrict__ part_a, int nwg) {
  __shared__ float cr[32 * kD];
  __shared__ double bsum[4][32];
  __shared__ double nsum[4][32];
  __shared__ float red[2][4];
  const int head = blockIdx.y;
  const int64_t j0 = (int64_t)blockIdx.x * 32;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const float* cbh = cb + (int64_t)head * c * kD;
#pragma unroll
  for (int e = t; e < 32 * kD; e += 256) {
    const int r = e / kD, a = e % kD;
    cr[e] = (j0 + r < c) ? cbh[(j0 + r) * kD + a] : 0.f;
  }
  __syncthreads();
  // acc[rt][ct][r]: row 16 rt + 4 r + lane / 16, column 32 wave + 16 ct + lane % 16
  d4 acc[2][2];
  if (gram) {
    const double* M = gram + (int64_t)head * kD * kD;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) acc[rt][ct] = d4{0.0, 0.0, 0.0, 0.0};
    const int li = lane % 16, lk = lane / 16;
    // every M element this lane needs is loaded before the first MFMA (one memory round
    // trip instead of one per k-step)
    double mb0[kD / 4], mb1[kD / 4];
#pragma unroll
    for (int q = 0; q < kD / 4; ++q) {
      mb0[q] = M[(4 * q + lk) * kD + 32 * wave + li];
      mb1[q] = M[(4 * q + lk) * kD + 32 * wave + 16 + li];
    }
#pragma unroll
    for (int k0 = 0; k0 < kD; k0 += 4) {
      const double a0 = (double)cr[li * kD + k0 + lk];
      const double a1 = (double)cr[(16 + li) * kD + k0 + lk];
      const double b0 = mb0[k0 / 4];
      const double b1 = mb1[k0 / 4];
      acc[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b1, acc[1][1], 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc[rt][ct][r] = (double)cr[(16 * rt + 4 * r + lane / 16) * kD + 32 * wave + 16 * ct + lane % 16];
  }
  float vmax = 0.f;
  double bp[2][4], np_[2][4];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * rt + 4 * r + lane / 16;
      const int64_t j = j0 + row;
      double p = 0.0, q = 0.0;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const int col = 32 * wave + 16 * ct + lane % 16;
        const double x = acc[rt][ct][r];
        const double x32 = (double)(float)x;
        p += x * (double)cr[row * kD + col];
        q += x32 * x32;
        if (j < c) {
          v64[((int64_t)head * c + j) * kD + col] = x;
          v32[((int64_t)head * c + j) * kD + col] = (float)x;
          vmax = fmaxf(vmax, round_up_f(fabs(x)));
        }
      }
      bp[rt][r] = p;
      np_[rt][r] = q;
    }
  // b and ||v32||^2: sums over the 16 lanes of a row, then over the four waves
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      double p = bp[rt][r], q = np_[rt][r];
      for (int o = 8; o > 0; o >>= 1) {
        p += __shfl_xor(p, o);
        q += __shfl_xor(q, o);
      }
      if (lane % 16 == 0) {
        bsum[wave][16 * rt + 4 * r + lane / 16] = p;
        nsum[wave][16 * rt + 4 * r + lane / 16] = q;
      }
    }
  for (int o = 32; o > 0; o >>= 1) vmax = fmaxf(vmax, __shfl_xor(vmax, o));
  if (lane == 0) red[0][wave] = vmax;
  __syncthreads();
  float bmax = 0.f;
  if (t < 32) {
    const double bj = ((bsum[0][t] + bsum[1][t]) + bsum[2][t]) + bsum[3][t];
    if (j0 + t < c) {
      b64[(int64_t)head * c + j0 + t] = bj;
      bmax = round_up_f(bj);
      // ||v32_j|| rounded up (the fp64 sum of 128 squares is within 2^-45 of exact)
      const double nj = ((nsum[0][t] + nsum[1][t]) + nsum[2][t]) + nsum[3][t];
      vnorm[(int64_t)head * c + j0 + t] = round_up_f(sqrt(nj) * (1.0 + 0x1p-40));
    }
    for (int o = 16; o > 0; o >>= 1) bmax = fmaxf(bmax, __shfl_xor(bmax, o));
  }
  if (t == 0) {
    float* pa = part_a + ((int64_t)head * nwg + blockIdx.x) * 4;
    pa[0] = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
    pa[1] = bmax;
    if (!gram) pa[2] = 0.f;  // no L: max |L| unused
  }
}

// Head constants from the prep_rows partials.
struct HeadScale {
  float S;      // codebook-side scale
  float maxb;   // max b_j (rounded up)
  float SL;     // L-side scale
};

// Scales of one head from the prep_rows partial maxima; every thread of the workgroup calls
// it (a workgroup reduction).
__device__ HeadScale head_scale_wg(const float* part_a, int64_t head, int nwg) {
  __shared__ float red[2][4];
  const int t = threadIdx.x;
  float a = 0.f, b = 0.f;
  for (int i = t; i < nwg; i += blockDim.x) {
    a = fmaxf(a, part_a[(head * nwg + i) * 4 + 0]);
    b = fmaxf(b, part_a[(head * nwg + i) * 4 + 1]);
  }
  for (int o = 32; o > 0; o >>= 1) {
    a = fmaxf(a, __shfl_xor(a, o));
    b = fmaxf(b, __shfl_xor(b, o));
  }
  __syncthreads();
  if ((t & 63) == 0) {
    red[0][t >> 6] = a;
    red[1][t >> 6] = b;
  }
  __syncthreads();
  const int nw = (int)(blockDim.x + 63) / 64;
  for (int w = 0; w < nw; ++w) {
    a = fmaxf(a, red[0][w]);
    b = fmaxf(b, red[1][w]);
  }
  HeadScale h;
  h.S = scale_for(a);
  h.maxb = b;
  h.SL = scale_for(part_a[(head * nwg) * 4 + 2]);
  return h;
}

// 16 threads per padded row (each one k-chunk of 8): fp16 fragments of S v, the bias slot,
// and this workgroup's max residual / max fragment norm.  Threads past the rows build the
// L^T hi/lo fragments; workgroup (0, 0) clears the list counters.
__global__ __launch_bounds__(256) void enc_prep_frag(const double* __restrict__ v64,
                                                     const double* __restrict__ b64, int64_t c,
                                                     int T, const float* __restrict__ chol,
                                                     int want_l, const float* __restrict__ part_a,
                                                     int nwg_a, float* __restrict__ part_b,
                                                     half8* __restrict__ v16,
                                                     float* __restrict__ bias,
                                                     half8* __restrict__ lfrag,
                                                     HeadScale* __restrict__ hsc,
                                                     unsigned* __restrict__ clr0, int nclr0,
                                                     unsigned* __restrict__ clr1, int64_t nclr1) {
  const int head = blockIdx.y;
  const int t = threadIdx.x;
  {  // the run state (list lengths, decision counters, candidate counts) starts at zero
    const int64_t g = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * 256 + t;
    const int64_t stride = (int64_t)gridDim.x * gridDim.y * 256;
    for (int64_t k = g; k < nclr0; k += stride) clr0[k] = 0u;
    for (int64_t k = g; k < nclr1; k += stride) clr1[k] = 0u;
  }
  const int64_t rows = (int64_t)T * kRows;
  const int64_t rid = (int64_t)blockIdx.x * 16 + t / 16;  // padded row (or L^T row after rows)
  const int chunk = t % 16;                                // k = 8 chunk .. 8 chunk + 7
  const int s = chunk / 2, hh = chunk % 2;
  const bool is_row = rid < rows;
  const bool is_l = !is_row && want_l && rid < rows + kD;
  // this thread's inputs are read before the head's scales are reduced, so that both reads
  // are in flight together (the scales only multiply them)
  double vin[8];
  double bin = 0.0;
  if (is_row) {
    const int64_t j = rid;
#pragma unroll
    for (int e = 0; e < 8; ++e) vin[e] = (j < c) ? v64[((int64_t)head * c + j) * kD + 8 * chunk + e] : 0.0;
    if (chunk == 0 && j < c) bin = b64[(int64_t)head * c + j];
  } else if (is_l) {
    const int a = (int)(rid - rows);
    const float* L = chol + (int64_t)head * kD * kD;
#pragma unroll
    for (int e = 0; e < 8; ++e) vin[e] = (double)L[(8 * chunk + e) * kD + a];
  }
  const HeadScale hs = head_scale_wg(part_a, head, nwg_a);
  if (blockIdx.x == 0 && t == 0) hsc[head] = hs;  // for the later passes
  double rho2 = 0.0, nu2 = 0.0;
  if (is_row) {
    const int64_t j = rid;
    const int64_t tile = j / kRows;
    const int i = (int)(j % kRows);
    half8 f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double sv = (j < c) ? (double)hs.S * vin[e] : 0.0;
      const _Float16 q = (_Float16)sv;  // fp64 -> fp16, round to nearest even
      const double dq = (double)q;
      rho2 += (sv - dq) * (sv - dq);
      nu2 += dq * dq;
      f[e] = q;
    }
    v16[((int64_t)head * T + tile) * kFragPerTile + s * 64 + i + 32 * hh] = f;
    if (chunk == 0) {
      const int bh = (i >> 2) & 1;
      const int r = (i >> 3) * 4 + (i & 3);
      bias[((int64_t)head * T + tile) * 32 + bh * 16 + r] =
          (j < c) ? (float)(-0.5 * (double)hs.S * bin) : kPadBias;
    }
  } else if (is_l) {
    // Row a of L^T (output z_a = sum_b k_b L_ba) as A-operand fragments: 4 output tiles of
    // 32 rows, each as two tiles, the fp16 high parts (tile 2 tz) and the residuals (2 tz + 1),
    // so that the coarse pass streams them as two stages of four tiles.
    const int a = (int)(rid - rows);
    const int tile = a / kRows, i = a % kRows;
    half8 fh, fl;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double x = (double)hs.SL * vin[e];
      const _Float16 qh = (_Float16)x;
      fh[e] = qh;
      fl[e] = (_Float16)(x - (double)qh);
    }
    half8* lt = lfrag + (int64_t)head * 8 * kFragPerTile;
    lt[(int64_t)(2 * tile) * kFragPerTile + s * 64 + i + 32 * hh] = fh;
    lt[(int64_t)(2 * tile + 1) * kFragPerTile + s * 64 + i + 32 * hh] = fl;
  }
  // row norms over the 16 threads of the row, then the workgroup maxima
  for (int o = 8; o > 0; o >>= 1) {
    rho2 += __shfl_xor(rho2, o);
    nu2 += __shfl_xor(nu2, o);
  }
  float rr = round_up_f(sqrt(rho2)), nn = round_up_f(sqrt(nu2));
  for (int o = 32; o > 0; o >>= 1) {
    rr = fmaxf(rr, __shfl_xor(rr, o));
    nn = fmaxf(nn, __shfl_xor(nn, o));
  }
  __shared__ float red[2][4];
  if ((t & 63) == 0) {
    red[0][t >> 6] = rr;
    red[1][t >> 6] = nn;
  }
  __syncthreads();
  if (t < 2)
    part_b[((int64_t)head * gridDim.x + blockIdx.x) * 2 + t] =
        fmaxf(fmaxf(red[t][0], red[t][1]), fmaxf(red[t][2], red[t][3]));
}

// ------------------------------------------------------------------ shared helpers
template <int NB>
struct KeyFrags {
  half8 f[NB][kSteps];  // 32-key blocks (MFMA B operand: key = lane % 32, k = 16s+8hh+e)
  float n2[NB];         // ||k||^2 (fp32 of the exact values)
  float e2[NB];         // ||k - k16||^2
  bool bad[NB];         // an element outside the fp16 range
};

// Converts one step (8 elements) of a key to fp16 and accumulates its norm terms.
__device__ __forceinline__ void key_step(const float (&x)[8], half8& v, float& n2, float& e2,
                                         bool& bad) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const bool ok = fabsf(x[e]) < 65504.0f;
    const _Float16 q = ok ? (_Float16)x[e] : (_Float16)0.0f;
    bad |= !ok;
    const float d = x[e] - (float)q;  // exact
    n2 += x[e] * x[e];
    e2 += d * d;
    v[e] = q;
  }
}

// Every load is issued without a branch before any of them is used (a skipped key reads row 0
// of its head and is zeroed afterwards): the lane's loads are then in flight together instead
// of costing one memory round trip each.  bf16 keys: all blocks' loads at once (4 VGPRs per
// step); f32 keys: one block at a time.
template <int DT, int NB>
__device__ __forceinline__ void load_key_frags(const void* keys, int64_t head, int64_t n,
                                               const int64_t* row, int hh, KeyFrags<NB>& kf) {
  if constexpr (DT == A2ATS_BF16) {
    // bf16 -> fp16 is exact for 2^-14 <= |x| <= 65280 (and zero); such a key needs none of
    // key_step's per-element work: two fp16 conversions per instruction (toward zero, exact
    // here), ||k||^2 from fp16 dot products (the products are exact), and one running
    // maximum and minimum of the 15-bit magnitudes (two per instruction) to find the rare
    // key that is not.  Beyond 65280 (bf16's next value is 65536) a key is outside the fp16
    // range (scanned in fp64 instead); below 2^-14 its fp16 value is |q| <= |x| with
    // |x - q| < 2^-24, so at most 64 such elements in a lane add less than 64 * 2^-28 to
    // ||k||^2 and to ||k - k16||^2, the bounds added below.
    uint4 raw[NB][kSteps];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      const int64_t off = (head * n + (row[blk] >= 0 ? row[blk] : 0)) * kD + 8 * hh;
#pragma unroll
      for (int s = 0; s < kSteps; ++s)
      {
        // non-temporal: the keys are read once, and should not evict the codebook tables
        // that the tail reads from L2
        typedef unsigned u4x __attribute__((ext_vector_type(4)));
        const u4x r = __builtin_nontemporal_load(
            reinterpret_cast<const u4x*>(static_cast<const uint16_t*>(keys) + off + 16 * s));
        raw[blk][s] = uint4{r.x, r.y, r.z, r.w};
      }
    }
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      const unsigned live = row[blk] >= 0 ? 0xFFFFFFFFu : 0u;
      float n2 = 0.f;
      unsigned mx = 0u, mn = 0xFFFFFFFFu;  // per 16-bit half: max |x| bits, min |x| bits - 1
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        const unsigned wv[4] = {raw[blk][s].x & live, raw[blk][s].y & live, raw[blk][s].z & live,
                                raw[blk][s].w & live};
        unsigned qw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const h2rtz q2 = __builtin_amdgcn_cvt_pkrtz(__uint_as_float(wv[e] << 16),
                                                       __uint_as_float(wv[e] & 0xFFFF0000u));
          n2 = __builtin_amdgcn_fdot2(q2, q2, n2, false);
          qw[e] = __builtin_bit_cast(unsigned, q2);
          // packed 16-bit integer ops (the same in vector-of-u16 C lets the register allocator
          // spill around the MFMA loop); m - 1 wraps for a zero, which drops out of the minimum
          const unsigned m = wv[e] & 0x7FFF7FFFu;
          unsigned m1;
          asm("v_pk_sub_u16 %0, %1, 1 op_sel_hi:[1,0]" : "=v"(m1) : "v"(m));
          asm("v_pk_max_u16 %0, %1, %2" : "=v"(mx) : "v"(mx), "v"(m));
          asm("v_pk_min_u16 %0, %1, %2" : "=v"(mn) : "v"(mn), "v"(m1));
        }
        kf.f[blk][s] = __builtin_bit_cast(half8, (uint4){qw[0], qw[1], qw[2], qw[3]});
      }
      const bool tiny = (mn & 0xFFFFu) < 0x387Fu || (mn >> 16) < 0x387Fu;  // 0 < |x| < 2^-14
      kf.bad[blk] = (mx & 0xFFFFu) > 0x477Fu || (mx >> 16) > 0x477Fu;
      kf.n2[blk] = tiny ? n2 + 0x1p-22f : n2;
      kf.e2[blk] = tiny ? 0x1p-22f : 0.f;
    }
  } else {
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      const int64_t off = (head * n + (row[blk] >= 0 ? row[blk] : 0)) * kD + 8 * hh;
      float4 raw[kSteps][2];
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(keys) + off + 16 * s);
        raw[s][0] = p[0];
        raw[s][1] = p[1];
      }
      const bool live = row[blk] >= 0;
      kf.n2[blk] = 0.f;
      kf.e2[blk] = 0.f;
      kf.bad[blk] = false;
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        const float4 a = raw[s][0], b = raw[s][1];
        float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = live ? x[e] : 0.f;
        key_step(x, kf.f[blk][s], kf.n2[blk], kf.e2[blk], kf.bad[blk]);
      }
    }
  }
#pragma unroll
  for (int blk = 0; blk < NB; ++blk) {
    kf.n2[blk] += __shfl_xor(kf.n2[blk], 32);
    kf.e2[blk] += __shfl_xor(kf.e2[blk], 32);
    // the shuffle runs in every lane (under a short-circuit it would skip the lanes that
    // already know, and their partners would read nothing from them)
    const int partner_bad = __shfl_xor((int)kf.bad[blk], 32);
    kf.bad[blk] = kf.bad[blk] || partner_bad != 0;
  }
}

// Error bound E (scaled units) of a key's MFMA scores, evaluated with upward margins.
__device__ __forceinline__ double score_bound(float n2, float e2, double rho, double nu, double B) {
  const double kn = sqrt((double)n2) * (1.0 + 0x1p-18);
  const double ke = sqrt((double)e2) * (1.0 + 0x1p-18);
  const double gamma = 130.0 * 0x1p-23;
  return (kn * rho + ke * nu + gamma * (B + (kn + ke) * nu) + 0x1p-23 * B) * (1.0 + 0x1p-16) + 1e-30;
}

// Largest possible change of a value by overwriting its low `tbits` bits.
__device__ __forceinline__ double pack_slack(float p, int tbits) {
  return fabs((double)p) * ldexp(1.0, tbits - 22) + ldexp(1.0, tbits - 140);
}

// Replace the low bits of x with the tile index.  Written in C so the compiler inserts the
// wait states between the MFMA that produced x and this read; with the tile index held in
// a VGPR (see vgpr_of) it becomes one v_and_or_b32 (mask in an SGPR).
__device__ __forceinline__ float pack_tile(float x, unsigned keep, unsigned tile_v) {
  return __uint_as_float((__float_as_uint(x) & keep) | tile_v);
}

// Largest of three with IEEE-754 maximum semantics (one v_maximum3_f32; the operands are
// never NaN, and unlike fmaxf it needs no canonicalising of integer-packed inputs).
__device__ __forceinline__ float fmax3(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// Element h of a two-element register array without dynamic indexing (which would move
// the array, and everything that shares its storage, to scratch memory).
template <class T>
__device__ __forceinline__ T sel2(const T (&a)[2], int h) {
  return h ? a[1] : a[0];
}

// A uniform value copied into a VGPR, opaque to the optimiser (GFX9 VALU instructions may
// read only one scalar operand).
__device__ __forceinline__ unsigned vgpr_of(unsigned s) {
  unsigned v;
  asm("v_mov_b32 %0, %1" : "=v"(v) : "s"(s));
  return v;
}

// ------------------------------------------------------------------ exact fp64 scores
// Exact fp64 score of one candidate, G lanes cooperating (lane g of the group owns dims
// (128/G)g .. (128/G)(g+1)-1).  Returns the score (valid in every lane of the group) and, in
// z2, ||k||^2.
template <int DT, int G, typename VT>
__device__ __forceinline__ double coop_score_g(const void* keys, int64_t off_key, const VT* vrow,
                                               double bj, int g, double* z2) {
  constexpr int DIM = kD / G;
  double x[DIM];
  if (DT == A2ATS_BF16) {
    const uint4* kp = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(keys) + off_key + DIM * g);
#pragma unroll
    for (int q = 0; q < DIM / 8; ++q) {
      const uint4 r = kp[q];
      const unsigned wv[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[8 * q + 2 * e] = (double)__uint_as_float(wv[e] << 16);
        x[8 * q + 2 * e + 1] = (double)__uint_as_float(wv[e] & 0xFFFF0000u);
      }
    }
  } else {
    const float4* kp = reinterpret_cast<const float4*>(static_cast<const float*>(keys) + off_key + DIM * g);
#pragma unroll
    for (int q = 0; q < DIM / 4; ++q) {
      const float4 a = kp[q];
      x[4 * q] = a.x; x[4 * q + 1] = a.y; x[4 * q + 2] = a.z; x[4 * q + 3] = a.w;
    }
  }
  double v[DIM];
  if (sizeof(VT) == 8) {
    const double2* v2 = reinterpret_cast<const double2*>(vrow + DIM * g);
#pragma unroll
    for (int e = 0; e < DIM / 2; ++e) {
      const double2 vv = v2[e];
      v[2 * e] = vv.x;
      v[2 * e + 1] = vv.y;
    }
  } else {
    const float4* v4 = reinterpret_cast<const float4*>(vrow + DIM * g);
#pragma unroll
    for (int e = 0; e < DIM / 4; ++e) {
      const float4 vv = v4[e];
      v[4 * e] = vv.x; v[4 * e + 1] = vv.y; v[4 * e + 2] = vv.z; v[4 * e + 3] = vv.w;
    }
  }
  double s = 0.0, k2 = 0.0;
#pragma unroll
  for (int e = 0; e < DIM; ++e) {
    s += x[e] * v[e];
    k2 += x[e] * x[e];
  }
  for (int o = G / 2; o > 0; o >>= 1) {
    s += __shfl_xor(s, o);
    k2 += __shfl_xor(k2, o);
  }
  *z2 = k2;
  return s - 0.5 * bj;
}

// Lists a key for the fp64 scan of the whole codebook.
__device__ __forceinline__ void full_append(FullEntry* full, Counters* cnt, int32_t head,
                                            int32_t row, float z2) {
  FullEntry fe;
  fe.head = head;
  fe.row = row;
  fe.z2 = z2;
  fe.pad = 0;
  full[atomicAdd(&cnt->full, 1u)] = fe;
}

// Number of listed open keys of a head (capped to the list capacity).
__device__ __forceinline__ int64_t open_count(const Counters* cnt, int64_t head, int64_t cap) {
  const unsigned u = __hip_atomic_load(&cnt->unc[head], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return (int64_t)u < cap ? (int64_t)u : cap;
}

constexpr int kMaxHeadsLds = 1024;

// The heads a workgroup of the rescan kernels serves (all of them: binding heads to XCDs
// measured slower, the heads' open counts differ too much) and its rank among the
// workgroups serving them.
struct HeadSet {
  int64_t count;
  int64_t rank, ranks;
  __device__ int64_t head(int64_t v) const { return v; }
};

__device__ __forceinline__ HeadSet all_heads(int64_t heads) {
  HeadSet hs;
  hs.count = heads;
  hs.rank = blockIdx.x;
  hs.ranks = gridDim.x;
  return hs;
}

// Exclusive prefix over the set's heads of `per(open count)`, built once per workgroup in
// LDS (up to kMaxHeadsLds heads; beyond that the global counters are scanned).  The first
// wave reads 64 heads' counters at once and scans them with shuffles.
template <typename F>
__device__ int64_t head_prefix(const Counters* cnt, const HeadSet& hs, int64_t cap, int64_t* pre,
                               F per) {
  __syncthreads();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int64_t hn = hs.count < kMaxHeadsLds ? hs.count : kMaxHeadsLds;
    int64_t run = 0;
    for (int64_t h0 = 0; h0 < hn; h0 += 64) {
      const int64_t h = h0 + lane;
      const int64_t v = h < hn ? per(open_count(cnt, hs.head(h), cap)) : 0;
      int64_t incl = v;
      for (int o = 1; o < 64; o <<= 1) {
        const int64_t u = __shfl_up(incl, o);
        if (lane >= o) incl += u;
      }
      if (h < hn) pre[h] = run + incl - v;
      run += __shfl(incl, 63);
    }
    if (lane == 0) {
      for (int64_t h = hn; h < hs.count; ++h) run += per(open_count(cnt, hs.head(h), cap));
      pre[kMaxHeadsLds] = run;
    }
  }
  __syncthreads();
  return pre[kMaxHeadsLds];
}

// Head (real index) owning item `it` of the set (prefix from head_prefix).
template <typename F>
__device__ int64_t find_head(const Counters* cnt, const HeadSet& hs, int64_t cap, const int64_t* pre,
                             int64_t it, F per, int64_t* rest) {
  const int64_t hn = hs.count < kMaxHeadsLds ? hs.count : kMaxHeadsLds;
  int64_t lo = 0, hi = hn - 1;
  if (hn > 0 && it < (hn < hs.count ? pre[hn - 1] + per(open_count(cnt, hs.head(hn - 1), cap))
                                    : pre[kMaxHeadsLds])) {
    while (lo < hi) {  // last head with pre[h] <= it
      const int64_t mid = (lo + hi + 1) / 2;
      if (pre[mid] <= it) lo = mid;
      else hi = mid - 1;
    }
    *rest = it - pre[lo];
    return hs.head(lo);
  }
  int64_t run = hn > 0 ? pre[hn - 1] + per(open_count(cnt, hs.head(hn - 1), cap)) : 0;
  for (int64_t h = hn; h < hs.count; ++h) {
    const int64_t m = per(open_count(cnt, hs.head(h), cap));
    if (it < run + m) {
      *rest = it - run;
      return hs.head(h);
    }
    run += m;
  }
  *rest = 0;
  return hs.head(hs.count - 1);
}

// Half of a key's dot with a row of v: the lane's 64 dims (8 per k-step, its exact fp16
// fragments, parked in LDS at kp[256 s]) against the fp32 row, one fp32 multiply-add chain.
__device__ __forceinline__ float half_dot_lds(const half8* kp, const float* v) {
  f4 va[kSteps], vb[kSteps];
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    va[s] = *reinterpret_cast<const f4*>(v + 16 * s);
    vb[s] = *reinterpret_cast<const f4*>(v + 16 * s + 4);
  }
  float acc = 0.f;
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    const half8 k = kp[256 * s];
    acc = fmaf((float)k[0], va[s].x, acc);
    acc = fmaf((float)k[1], va[s].y, acc);
    acc = fmaf((float)k[2], va[s].z, acc);
    acc = fmaf((float)k[3], va[s].w, acc);
    acc = fmaf((float)k[4], vb[s].x, acc);
    acc = fmaf((float)k[5], vb[s].y, acc);
    acc = fmaf((float)k[6], vb[s].z, acc);
    acc = fmaf((float)k[7], vb[s].w, acc);
  }
  return acc;
}

// ------------------------------------------------------------------ the MFMA pass
// Workgroup: 256 keys of one head (4 waves x two 32-key column blocks).  Lane l serves key
// column l % 32 of both blocks and, in every 32-centroid tile, the 16 rows
// 8(r/4) + 4(l/32) + (r%4).  Codebook tiles stream through LDS in double-buffered stages of
// four tiles, loads issued a stage ahead, one LDS-only barrier per stage; each tile costs 8
// MFMAs per block with the bias as the first accumulator input, and its VALU fold overlaps
// the next tile's MFMAs.
// Each lane keeps 8 slot maxima per block (a slot pairs two of its rows), the tile index and
// row parity packed into the low bits, plus one value U bounding every score that is not a
// slot maximum.  At the end each key has 16 slot maxima and U:
//   direct  t1 - max(t2, U) > 2E (+ packing slack)  -> code j(t1)
//   else    fp32 scores of j(t1), j(t2) (error e << E) against max(t3, U) + E: the better
//           one when the bounds prove it, else the key is listed for the rescan.
// Workgroups are dealt to XCDs round-robin; the mapping gives each XCD a contiguous range of
// (head, key block) pairs so a head's codebook stays in one L2.
template <int DT, bool ZNORM, bool DIST>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void enc_coarse(
    const void* __restrict__ keys, int64_t n, const int32_t* __restrict__ idx, int64_t n_sel,
    int64_t heads, int nkb, int T, int tbits, const half8* __restrict__ v16,
    const float* __restrict__ bias, const float* __restrict__ v32,
    const double* __restrict__ b64, int64_t c, const half8* __restrict__ lfrag,
    const HeadScale* __restrict__ hsc, const float* __restrict__ part_b, int nwg_b,
    float* __restrict__ znorm, uint16_t* __restrict__ codes, float* __restrict__ dist,
    const float* __restrict__ vnorm, UncEntry* __restrict__ unc, int64_t unc_cap,
    FullEntry* __restrict__ full, Counters* __restrict__ cnt, int want_stats) {
  // two stage buffers as separate arrays: the compiler then sees that the loads streaming
  // into one buffer cannot alias the LDS reads of the other, and does not wait for them
  __shared__ half8 sv0[kTPS][kFragPerTile], sv1[kTPS][kFragPerTile];
  __shared__ __attribute__((aligned(16))) float sb0[kTPS][32], sb1[kTPS][32];
  __shared__ float s_red[2][4];
  const int64_t G = gridDim.x;
  const int64_t per_xcd = G / 8;
  const int64_t wk = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (wk >= heads * nkb) return;
  const int64_t head = wk / nkb;
  const int64_t kb = wk % nkb;
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63, col = lane & 31, hh = lane >> 5;
  const HeadScale hs = hsc[head];
  // Every prologue load is issued before any result is needed, so they share one memory round
  // trip: the first partials of rho and nu (clamped rather than skipped: a repeated entry
  // leaves a maximum unchanged), the rows (a key past the end reads the last entry and is then
  // dropped), the first codebook stage and the keys.
  const int ib = t < nwg_b ? t : nwg_b - 1;
  const float rr0 = part_b[(head * nwg_b + ib) * 2 + 0];
  const float nn0 = part_b[(head * nwg_b + ib) * 2 + 1];
  int64_t row[2], sel[2], sc[2];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    sel[blk] = kb * kKeysPerWG + wave * 64 + blk * 32 + col;
    sc[blk] = sel[blk] < n_sel ? sel[blk] : n_sel - 1;
    row[blk] = sc[blk];
  }
  if (idx) {
    row[0] = (int64_t)idx[head * n_sel + sc[0]];
    row[1] = (int64_t)idx[head * n_sel + sc[1]];
  }
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)  // out-of-range index entries are skipped
    row[blk] = (sel[blk] < n_sel && row[blk] >= 0 && row[blk] < n) ? row[blk] : -1;
  const half8* vh = v16 + head * (int64_t)T * kFragPerTile;
  const float* bh = bias + head * (int64_t)T * 32;
  // stage loader: a stage is kTPS tiles (32 KiB of fragments, 512 B of bias), loaded straight
  // into LDS (global_load_lds_dwordx4: lane l of a wave writes 16 B at the wave's LDS base +
  // 16 l); 256 threads x 8 fragments, 32 threads x 4 bias floats.  Stage s+1 is loaded while
  // stage s is computed: its loads go out at the start of stage s, right after the barrier
  // that freed its buffer, so no load is in flight across the loop's back edge.
  const int nst = (T + kTPS - 1) / kTPS;
  const unsigned lds_sv[2] = {lds_offset(&sv0[0][0]), lds_offset(&sv1[0][0])};
  const unsigned lds_sb[2] = {lds_offset(&sb0[0][0]), lds_offset(&sb1[0][0])};
  auto load_frags = [&](const half8* src, int buf) {  // kTPS tiles of fragments
    const unsigned dst = lds_sv[buf] + (unsigned)(wave * 64 * sizeof(half8));
#pragma unroll
    for (int q = 0; q < kTPS; ++q) {
      lds_dma16(src + q * kFragPerTile + t, dst + q * kFragPerTile * sizeof(half8));
      lds_dma16(src + q * kFragPerTile + 256 + t, dst + (q * kFragPerTile + 256) * sizeof(half8));
    }
  };
  auto load_stage = [&](int st, int buf) {
    load_frags(vh + (int64_t)st * kTPS * kFragPerTile, buf);
    if (t < 8 * kTPS) lds_dma16(bh + (int64_t)st * kTPS * 32 + t * 4, lds_sb[buf]);
  };
  // With ||kL||^2 the stream starts with two stages of L^T fragments (z stages), then the
  // codebook; without, with the codebook.
  const half8* lt = lfrag + head * 8 * kFragPerTile;
  if (ZNORM) load_frags(lt, 0);
  else load_stage(0, 0);

  KeyFrags<2> kf;
  load_key_frags<DT, 2>(keys, head, n, row, hh, kf);
  {  // rho and nu: maxima over the prep_frag partials of this head
    float rr = fmaxf(0.f, rr0), nn = fmaxf(0.f, nn0);
    for (int i = t + 256; i < nwg_b; i += 256) {
      rr = fmaxf(rr, part_b[(head * nwg_b + i) * 2 + 0]);
      nn = fmaxf(nn, part_b[(head * nwg_b + i) * 2 + 1]);
    }
    for (int o = 32; o > 0; o >>= 1) {
      rr = fmaxf(rr, __shfl_xor(rr, o));
      nn = fmaxf(nn, __shfl_xor(nn, o));
    }
    if (lane == 0) {
      s_red[0][wave] = rr;
      s_red[1][wave] = nn;
    }
  }

  // ||k L||^2 from fp16 hi/lo fragments of L^T (bf16 keys are exact in fp16), on the MFMA
  // with the fragments streamed through the stage buffers like codebook tiles: z stage zs
  // holds [hi, lo] of output tiles 2 zs and 2 zs + 1; each output tile's hi and lo products
  // accumulate into one fp32 result, whose squares are summed.  The second z stage issues
  // the loads of codebook stage 0 into buffer 0.
  float zn[2] = {0.f, 0.f};
  if (ZNORM) {
    lds_dma_barrier();  // z stage 0 in LDS, s_red visible
    auto zstage = [&](half8 (&svb)[kTPS][kFragPerTile], int zs) {
      if (zs == 0) load_frags(lt + kTPS * kFragPerTile, 1);
      else load_stage(0, 0);
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        f16v z0 = {}, z1 = {};
#pragma unroll
        for (int part = 0; part < 2; ++part) {
#pragma unroll
          for (int s = 0; s < kSteps; ++s) {
            const half8 a = svb[2 * p + part][s * 64 + lane];
            z0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, kf.f[0][s], z0, 0, 0, 0);
            z1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, kf.f[1][s], z1, 0, 0, 0);
          }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          zn[0] += z0[r] * z0[r];
          zn[1] += z1[r] * z1[r];
        }
      }
      lds_dma_barrier();  // the next stage landed; this buffer free everywhere
    };
    zstage(sv0, 0);
    zstage(sv1, 1);
    const float inv = 1.f / (hs.SL * hs.SL);
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) zn[blk] = (zn[blk] + __shfl_xor(zn[blk], 32)) * inv;
  }

  // Per lane and 32-key block: 8 slot maxima (slot i = the lane's tile rows of registers 2i
  // and 2i+1, over all tiles), each packed with (tile << 1 | register parity) in its low
  // bits, and one running value U at least as large as every score that is not a slot
  // maximum.  Per pair of scores: two packs, a med3 (the middle of slot max and the pair,
  // which is the largest value the slot drops) and a max3; U absorbs two dropped values per
  // max3: 2.25 VALU ops per score.
  float m1[2][8], U[2];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    U[blk] = -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i) m1[blk][i] = -INFINITY;
  }
  const unsigned keep = ~((1u << tbits) - 1u);
  lds_dma_barrier();  // stage 0 in LDS, s_red visible

  // Fold pair i (registers 2i, 2i+1) of one tile's scores into the slot maxima and U.
  float dr[2][8];
  auto fold_pair = [&](const f16v& a0, const f16v& a1, int i, unsigned te, unsigned to) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const f16v& acc = blk ? a1 : a0;
      const float p = pack_tile(acc[2 * i], keep, te);
      const float q = pack_tile(acc[2 * i + 1], keep, to);
      dr[blk][i] = __builtin_amdgcn_fmed3f(m1[blk][i], p, q);
      m1[blk][i] = fmax3(m1[blk][i], p, q);
      if (i & 1) U[blk] = fmax3(U[blk], dr[blk][i - 1], dr[blk][i]);
    }
    // an empty use pins the fold here (it would otherwise sink to the end of the stage,
    // keeping every tile's accumulators live at once)
    asm volatile("" ::"v"(m1[0][i]), "v"(m1[1][i]));
    if (i & 1) asm volatile("" ::"v"(U[0]), "v"(U[1]));
  };
  auto load_bias = [&](float (&sbb)[kTPS][32], int q) {
    const f4* bl = reinterpret_cast<const f4*>(&sbb[q][hh * 16]);
    f16v bv;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f4 b4 = bl[k];
      bv[4 * k + 0] = b4.x; bv[4 * k + 1] = b4.y; bv[4 * k + 2] = b4.z; bv[4 * k + 3] = b4.w;
    }
    return bv;
  };

  // Software pipeline: tile q of a stage runs its 8 MFMA steps into (a0, a1) while the VALU
  // folds the previous tile (p0, p1) one register pair per step; scheduling barriers keep
  // that interleave.  Fragments are read from LDS kAhead steps before their MFMAs, the bias
  // of the next tile two steps before it starts.  Stages always hold kTPS tiles (tiles past
  // the codebook carry the padding bias), so the accumulator pairs x and y simply
  // alternate; y starts as a fold-neutral stand-in for the tile before the first.
  constexpr int kAhead = 3;
  constexpr int kStageSteps = kTPS * kSteps;
  f16v x0, x1, y0, y1;
#pragma unroll
  for (int r = 0; r < 16; ++r) y0[r] = y1[r] = kPadBias;
  auto stage = [&](int st, half8 (&svb)[kTPS][kFragPerTile], float (&sbb)[kTPS][32], int nbuf) {
    const int base = st * kTPS;
    half8 fr[kStageSteps];
#pragma unroll
    for (int g = 0; g < kAhead; ++g) fr[g] = svb[g / kSteps][(g % kSteps) * 64 + lane];
    f16v bv = load_bias(sbb, 0);
    if (st + 1 < nst) load_stage(st + 1, nbuf);
#pragma unroll
    for (int q = 0; q < kTPS; ++q) {
      f16v& a0 = (q & 1) ? y0 : x0;
      f16v& a1 = (q & 1) ? y1 : x1;
      const f16v& p0 = (q & 1) ? x0 : y0;
      const f16v& p1 = (q & 1) ? x1 : y1;
      const int ptile = base + q - 1 < 0 ? 0 : base + q - 1;
      const unsigned te = vgpr_of((unsigned)ptile << 1);
      const unsigned to = te | 1u;
      f16v bn;
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        const int g = q * kSteps + s;
        if (g + kAhead < kStageSteps)
          fr[g + kAhead] = svb[(g + kAhead) / kSteps][((g + kAhead) % kSteps) * 64 + lane];
        if (s == kSteps - 2 && q + 1 < kTPS) bn = load_bias(sbb, q + 1);
        a0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(fr[g], kf.f[0][s], s == 0 ? bv : a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(fr[g], kf.f[1][s], s == 0 ? bv : a1, 0, 0, 0);
        fold_pair(p0, p1, s, te, to);
        __builtin_amdgcn_sched_barrier(0);
      }
      bv = bn;
    }
    lds_dma_barrier();  // this wave's loads of stage st+1 landed; this buffer free everywhere
  };
  for (int st = 0; st < nst; st += 2) {
    stage(st, sv0, sb0, 1);
    if (st + 1 < nst) stage(st + 1, sv1, sb1, 0);
  }
  {
    const unsigned te = vgpr_of((unsigned)(nst * kTPS - 1) << 1);
    const unsigned to = te | 1u;
#pragma unroll
    for (int i = 0; i < 8; ++i) fold_pair(y0, y1, i, te, to);
  }
  __syncthreads();

  // ---- per-key certificate.  Lane (col, hh) finalises key col of block hh: it keeps its own
  // 8 slot maxima of that block and takes the partner lane's 8 (the other 16 rows).
  const unsigned tmask = ~keep;
  float v[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = hh ? m1[1][i] : m1[0][i];
    v[8 + i] = __shfl_xor(hh ? m1[0][i] : m1[1][i], 32);
  }
  const float um = fmaxf(hh ? U[1] : U[0], __shfl_xor(hh ? U[0] : U[1], 32));
  // top three values: a0 >= a1 >= a2 (med3 insertion, three ops per value)
  float a0 = -INFINITY, a1 = -INFINITY, a2 = -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float n2 = __builtin_amdgcn_fmed3f(a1, a2, v[i]);
    const float n1 = __builtin_amdgcn_fmed3f(a0, a1, v[i]);
    a0 = __builtin_elementwise_maximum(a0, v[i]);
    a1 = n1;
    a2 = n2;
  }
  // the slots holding a0 and (another) a1.  Equal packed values break ties arbitrarily: they
  // never certify directly, and the rerank and rescan resolve them exactly.
  int i0 = 0, i1 = 0;
#pragma unroll
  for (int i = 15; i >= 0; --i) i0 = v[i] == a0 ? i : i0;
#pragma unroll
  for (int i = 15; i >= 0; --i) i1 = (v[i] == a1 && i != i0) ? i : i1;
  // centroid index of slot i: tile and parity from the packed bits, row from the slot
  auto jdec = [&](float x, int i) {
    const unsigned low = __float_as_uint(x) & tmask;
    const int h = i < 8 ? hh : 1 - hh;
    const int ii = i & 7;
    return (int)(low >> 1) * kRows + 8 * (ii >> 1) + 4 * h + 2 * (ii & 1) + (int)(low & 1u);
  };
  const int j0 = jdec(a0, i0), j1 = jdec(a1, i1);
  const int64_t myrow = hh ? row[1] : row[0];
  const bool mybad = hh ? kf.bad[1] : kf.bad[0];
  // The fragments hold the key exactly (a bf16 key within fp16's normal range): its scores
  // can then be formed from them below.
  const bool exact_k = DT == A2ATS_BF16 && !mybad && (hh ? kf.e2[1] : kf.e2[0]) == 0.f;
  int outcome = 0;  // 1 direct, 2 scored from the fragments, 3 open, 4 full scan
  float z2 = -1.f;
  const double S = (double)hs.S;
  double E = 0.0, thr = 0.0, lb3 = 0.0;
  if (myrow >= 0) {
    const double rho = (double)fmaxf(fmaxf(s_red[0][0], s_red[0][1]), fmaxf(s_red[0][2], s_red[0][3]));
    const double nu = (double)fmaxf(fmaxf(s_red[1][0], s_red[1][1]), fmaxf(s_red[1][2], s_red[1][3]));
    const double B = 0.5 * S * (double)hs.maxb;
    E = score_bound(hh ? kf.n2[1] : kf.n2[0], hh ? kf.e2[1] : kf.e2[0], rho, nu, B);
    const float t1u = fmaxf(a1, um);  // bound on every score but the best
    const double s0 = pack_slack(a0, tbits), s1 = pack_slack(t1u, tbits);
    if (ZNORM) z2 = hh ? zn[1] : zn[0];
    else if (znorm) z2 = znorm[head * n + myrow];
    if (mybad || j0 >= c) {
      outcome = 4;
      if (ZNORM) z2 = -2.f;  // the fp16 fragments do not hold this key: ||kL||^2 in the scan
    } else if ((double)a0 - s0 - E > (double)t1u + s1 + E) {
      outcome = 1;
      codes[head * n + myrow] = (uint16_t)j0;
    } else {
      outcome = exact_k ? 2 : 3;
      // every score but those of j0 and j1 lies below thr; s_j0 >= lb3
      const double Ub = fmax((double)a2, (double)um);
      thr = (Ub + pack_slack((float)Ub, tbits) + E) / S;
      lb3 = ((double)a0 - s0 - E) / S;
    }
  }
  // fp32 scores of the leading candidates from the key fragments: j0 for a key decided
  // directly whose distance is wanted, j0 and j1 for a key not decided.  Lane (col, hh) holds
  // dims 16s + 8hh .. 16s + 8hh + 7 of key col of both blocks, so each lane forms half of
  // every dot and the halves are added across the lane pair.  Bound of a score's error:
  // 70 u ||k|| ||v32_j|| (a 65-term fp32 dot, the fp32 copy of v) plus the fp64 subtraction.
  const bool w0 = (outcome == 1 && DIST && exact_k) || outcome == 2;
  const bool w1 = outcome == 2 && j1 < c;
  const int jj0 = w0 ? j0 : 0, jj1 = w1 ? j1 : 0;
  const int pj0 = __shfl_xor(jj0, 32), pj1 = __shfl_xor(jj1, 32);
  const int pw = __shfl_xor((w0 ? 1 : 0) | (w1 ? 2 : 0), 32);
  const double bq0 = w0 ? b64[head * c + jj0] : 0.0, bq1 = w1 ? b64[head * c + jj1] : 0.0;
  const float vn0 = w0 ? vnorm[head * c + jj0] : 0.f, vn1 = w1 ? vnorm[head * c + jj1] : 0.f;
  float hd0[2] = {0.f, 0.f}, hd1[2] = {0.f, 0.f};
  if constexpr (DT == A2ATS_BF16) {
    // The key fragments move to the stage buffers (free after the loop; each lane reads back
    // only its own), so that a round of row loads (both blocks' rows, 512 bytes a lane) fits
    // in registers: two rounds, j0 then j1, where row 0 stands in for a row not needed.
    half8* kst0 = &sv0[0][0] + t;
    half8* kst1 = &sv1[0][0] + t;
#pragma unroll
    for (int q = 0; q < kSteps; ++q) {
      kst0[q * 256] = kf.f[0][q];
      kst1[q * 256] = kf.f[1][q];
    }
    const float* v32h = v32 + head * c * kD + 8 * hh;
    {
      const int r0 = hh ? ((pw & 1) ? pj0 : 0) : (w0 ? jj0 : 0);   // block 0's key's j0
      const int r1 = hh ? (w0 ? jj0 : 0) : ((pw & 1) ? pj0 : 0);   // block 1's
      hd0[0] = half_dot_lds(kst0, v32h + (int64_t)r0 * kD);
      hd0[1] = half_dot_lds(kst1, v32h + (int64_t)r1 * kD);
    }
    if (__ballot(w1)) {  // wave-uniform
      int r0 = hh ? ((pw & 2) ? pj1 : 0) : (w1 ? jj1 : 0);
      int r1 = hh ? (w1 ? jj1 : 0) : ((pw & 2) ? pj1 : 0);
      // the rows of this round depend (opaquely) on the first round's products, so that
      // the compiler does not issue both rounds' loads at once (their registers would spill)
      asm volatile("" : "+v"(r0), "+v"(r1) : "v"(hd0[0]), "v"(hd0[1]));
      hd1[0] = half_dot_lds(kst0, v32h + (int64_t)r0 * kD);
      hd1[1] = half_dot_lds(kst1, v32h + (int64_t)r1 * kD);
    }
  }
  float q0, q1;
  {
    const float f00 = hd0[0] + __shfl_xor(hd0[0], 32), f01 = hd0[1] + __shfl_xor(hd0[1], 32);
    const float f10 = hd1[0] + __shfl_xor(hd1[0], 32), f11 = hd1[1] + __shfl_xor(hd1[1], 32);
    q0 = hh ? f01 : f00;
    q1 = hh ? f11 : f10;
  }
  const double kn = sqrt((double)(hh ? kf.n2[1] : kf.n2[0])) * (1.0 + 0x1p-16);
  const double zz = (ZNORM || znorm) ? (double)z2 : (double)(hh ? kf.n2[1] : kf.n2[0]);
  bool open = outcome == 3;
  int jbest = j0;
  double sbest = lb3;
  unsigned reranked = 0;
  if (outcome == 1 && DIST) {
    if (exact_k) {
      const double sc = (double)q0 - 0.5 * bq0;
      dist[head * n + myrow] = (float)fmax(zz - 2.0 * sc, 0.0);
    } else {
      // a key the fragments do not hold exactly: fp32 dot with the key read again, in two
      // halves whose loads are all issued before their products
      const float* vr = v32 + (head * c + j0) * kD;
      const int64_t off = (head * n + myrow) * kD;
      float sdot = 0.f, k2 = 0.f;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        f4 vv[16];
        float x[64];
#pragma unroll
        for (int q = 0; q < 16; ++q) vv[q] = *reinterpret_cast<const f4*>(vr + 64 * half + 4 * q);
        if constexpr (DT == A2ATS_BF16) {
          const uint4* kp = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(keys) + off + 64 * half);
          uint4 raw[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) raw[q] = kp[q];
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const unsigned wv[4] = {raw[q].x, raw[q].y, raw[q].z, raw[q].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              x[8 * q + 2 * e] = __uint_as_float(wv[e] << 16);
              x[8 * q + 2 * e + 1] = __uint_as_float(wv[e] & 0xFFFF0000u);
            }
          }
        } else {
          const f4* kp = reinterpret_cast<const f4*>(static_cast<const float*>(keys) + off + 64 * half);
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const f4 a = kp[q];
            x[4 * q] = a.x; x[4 * q + 1] = a.y; x[4 * q + 2] = a.z; x[4 * q + 3] = a.w;
          }
        }
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          sdot += x[4 * q] * vv[q].x + x[4 * q + 1] * vv[q].y + x[4 * q + 2] * vv[q].z +
                  x[4 * q + 3] * vv[q].w;
#pragma unroll
          for (int e = 0; e < 4; ++e) k2 += x[4 * q + e] * x[4 * q + e];
        }
      }
      const double zk = (ZNORM || znorm) ? (double)z2 : (double)k2;
      const double sc = (double)sdot - 0.5 * b64[head * c + j0];
      dist[head * n + myrow] = (float)fmax(zk - 2.0 * sc, 0.0);
    }
  } else if (outcome == 2) {
    constexpr double kU70 = 70.0 * 0x1p-24;
    const double sa = (double)q0 - 0.5 * bq0;
    const double ea = kU70 * kn * (double)vn0 + 0x1p-52 * (fabs((double)q0) + 0.5 * bq0);
    double sb = -INFINITY, eb = 0.0;
    if (w1) {
      sb = (double)q1 - 0.5 * bq1;
      eb = kU70 * kn * (double)vn1 + 0x1p-52 * (fabs((double)q1) + 0.5 * bq1);
    }
    // the better of the two, when the bounds order them; then certified when its lower
    // bound clears every other score
    const bool b_wins = sb > sa;
    jbest = b_wins ? j1 : j0;
    const double s_hi = b_wins ? sb : sa, e_hi = b_wins ? eb : ea;
    const bool ordered = !w1 || fabs(sa - sb) > ea + eb;
    if (ordered && s_hi - e_hi > thr) {
      codes[head * n + myrow] = (uint16_t)jbest;
      if (DIST) dist[head * n + myrow] = (float)fmax(zz - 2.0 * s_hi, 0.0);
      reranked = 1;
    } else {
      open = true;
      sbest = fmax(sa - ea, sb - eb);  // a lower bound of the larger of s_j0, s_j1
      jbest = (sa - ea >= sb - eb) ? j0 : j1;
    }
  }
  // Open keys go to the rescan list: one list append per wave (the keys of a workgroup are
  // one head's, and device-scope atomics on one address serialise at the memory side).  The
  // entry's score is a lower bound of the best score, which is all the rescan needs.
  {
    const unsigned long long m = __ballot(open);
    if (m) {  // wave-uniform
      unsigned base = 0u;
      if (lane == __builtin_ctzll(m)) base = atomicAdd(&cnt->unc[head], (unsigned)__popcll(m));
      base = __shfl(base, __builtin_ctzll(m));
      if (open) {
        const unsigned slot = base + (unsigned)__builtin_amdgcn_mbcnt_hi(
                                         (unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
        if (slot < unc_cap) {
          UncEntry ue;
          ue.row = (int32_t)myrow;
          ue.jbest = jbest;
          ue.sbest = sbest;
          ue.e_unscaled = E / S;
          ue.z2 = z2;
          ue.pad = 0;
          unc[head * unc_cap + slot] = ue;
        } else {
          full_append(full, cnt, (int32_t)head, (int32_t)myrow, z2);
        }
      }
    }
  }
  __shared__ unsigned s_cnt, s_base, s_stat[3];
  const unsigned xcd = blockIdx.x % 8;
  const unsigned fslot = block_append(&cnt->full, outcome == 4, &s_cnt, &s_base);
  if (outcome == 4) {
    FullEntry fe;
    fe.head = (int32_t)head;
    fe.row = (int32_t)myrow;
    fe.z2 = z2;
    fe.pad = 0;
    full[fslot] = fe;
  }
  if (want_stats) {  // keys, direct decisions and reranks, per XCD
    if (t == 0) s_stat[0] = s_stat[1] = s_stat[2] = 0u;
    __syncthreads();
    const unsigned long long valid = __ballot(myrow >= 0);
    const unsigned long long dmask = __ballot(outcome == 1);
    for (int o = 32; o > 0; o >>= 1) reranked += __shfl_xor(reranked, o);
    if (lane == 0) {
      atomicAdd(&s_stat[0], (unsigned)__popcll(valid));
      atomicAdd(&s_stat[1], (unsigned)__popcll(dmask));
      atomicAdd(&s_stat[2], reranked);
    }
    __syncthreads();
    if (t == 0) {
      if (s_stat[0]) atomicAdd(&cnt->stat_x[xcd][0], s_stat[0]);
      if (s_stat[1]) atomicAdd(&cnt->stat_x[xcd][1], s_stat[1]);
      if (s_stat[2]) atomicAdd(&cnt->stat_x[xcd][2], s_stat[2]);
    }
  }
}

// ------------------------------------------------------------------ rescan of open keys
// Work item = (head, group of 32 listed keys, chunk of tiles).  One wave per item: the keys
// are loaded once, then the chunk's tiles are scored on MFMA (fragments straight from L2,
// the next tile's fragments and bias loaded while the current tile runs); every centroid
// whose score reaches S * sbest - E is appended to the key's candidate list.  The chunk
// length adapts to the number of groups: about two items per wave of the grid (short
// chunks when few keys are open, long ones when many are).
template <int DT>
__global__ __launch_bounds__(256) void enc_rescan_collect(
    const void* __restrict__ keys, int64_t n, int64_t heads, int T, int64_t c,
    const half8* __restrict__ v16, const float* __restrict__ bias,
    const HeadScale* __restrict__ hsc, const UncEntry* __restrict__ unc,
    int64_t unc_cap, const Counters* __restrict__ cnt, unsigned* __restrict__ cand_n,
    int32_t* __restrict__ cand) {
  const int t = threadIdx.x, lane = t & 63, col = lane & 31, hh = lane >> 5;
  const HeadSet hsx = all_heads(heads);
  __shared__ int64_t pre[kMaxHeadsLds + 1];
  auto groups = [](int64_t m) { return (m + 31) / 32; };
  const int64_t ngroups = head_prefix(cnt, hsx, unc_cap, pre, groups);
  const int64_t waves = hsx.ranks * 4;
  int64_t chunks = ngroups > 0 ? (2 * waves + ngroups - 1) / ngroups : 1;
  if (chunks > T / 2) chunks = T / 2;
  if (chunks < 1) chunks = 1;
  int tpi = (int)((T + chunks - 1) / chunks);
  tpi = (tpi + 1) & ~1;  // whole tile pairs (T is a multiple of kTPS)
  chunks = (T + tpi - 1) / tpi;
  const int64_t items = ngroups * chunks;
  // candidates gathered per wave in LDS (one slot list per key column) and appended to the
  // key's global list with one atomic per key and item, after the item's tiles
  __shared__ int s_cand[4][32][kCandCap];
  __shared__ unsigned s_cn[4][32];
  const int wv = t >> 6;
  for (int64_t it = hsx.rank * 4 + (t >> 6); it < items; it += hsx.ranks * 4) {
    if (lane < 32) s_cn[wv][lane] = 0u;
    __builtin_amdgcn_wave_barrier();
    int64_t rest = 0;
    const int64_t head = find_head(cnt, hsx, unc_cap, pre, it / chunks, groups, &rest);
    const int chunk = (int)(it % chunks);
    const int64_t m = open_count(cnt, head, unc_cap);
    const int64_t slot = rest * 32 + col;
    const bool live = slot < m;
    UncEntry ue;
    ue.row = -1;
    ue.sbest = 0.0;
    ue.e_unscaled = 0.0;
    if (live) ue = unc[head * unc_cap + slot];
    const HeadScale hs = hsc[head];
    const int64_t row[1] = {live ? (int64_t)ue.row : -1};
    KeyFrags<1> kf;
    load_key_frags<DT, 1>(keys, head, n, row, hh, kf);
    const double th = (ue.sbest - ue.e_unscaled) * (double)hs.S;
    const float thr = live ? (float)(th - fabs(th) * 0x1p-20 - 1e-30) : INFINITY;
    const half8* vh = v16 + head * (int64_t)T * kFragPerTile;
    const float* bh = bias + head * (int64_t)T * 32;
    const int tb = chunk * tpi;
    const int nt = T - tb < tpi ? T - tb : tpi;  // even
    auto load_tile = [&](int tile, half8 (&fa)[kSteps], f16v& acc) {
      const f4* bl = reinterpret_cast<const f4*>(bh + (int64_t)tile * 32 + hh * 16);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const f4 b4 = bl[k];
        acc[4 * k + 0] = b4.x; acc[4 * k + 1] = b4.y; acc[4 * k + 2] = b4.z; acc[4 * k + 3] = b4.w;
      }
#pragma unroll
      for (int st = 0; st < kSteps; ++st) fa[st] = vh[(int64_t)tile * kFragPerTile + st * 64 + lane];
    };
    auto score_tile = [&](int tile, const half8 (&fa)[kSteps], f16v& acc) {
#pragma unroll
      for (int st = 0; st < kSteps; ++st)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[st], kf.f[0][st], acc, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (acc[r] >= thr) {
          const int j = tile * kRows + slot_row(r, hh);
          if (j < c) {
            const unsigned pos = atomicAdd(&s_cn[wv][col], 1u);
            if (pos < (unsigned)kCandCap) s_cand[wv][col][pos] = j;
          }
        }
      }
    };
    half8 fa0[kSteps], fa1[kSteps];
    f16v acc0, acc1;
    load_tile(tb, fa0, acc0);
    for (int q = 0; q < nt; q += 2) {
      load_tile(tb + q + 1, fa1, acc1);
      score_tile(tb + q, fa0, acc0);
      if (q + 2 < nt) load_tile(tb + q + 2, fa0, acc0);
      score_tile(tb + q + 1, fa1, acc1);
    }
    __builtin_amdgcn_wave_barrier();
    if (live && hh == 0) {
      const unsigned nl = s_cn[wv][col];
      if (nl != 0u) {
        const unsigned base = atomicAdd(&cand_n[head * unc_cap + slot], nl);
        for (unsigned i = 0; i < nl && i < (unsigned)kCandCap && base + i < (unsigned)kCandCap;
             ++i)
          cand[(head * unc_cap + slot) * kCandCap + base + i] = s_cand[wv][col][i];
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// fp64 scan of the whole codebook for one key by one wave (kx: this wave's LDS row of 128).
// z2f: ||kL||^2 for the distance, -1 for ||k||^2 (no L), -2 for ||kL||^2 computed here in
// fp64 from chol (a bf16 key outside the fp16 range, whose fp16 fragments do not hold it).
template <int DT>
__device__ void full_scan_wave(const void* keys, int64_t n, int64_t c, const double* v64,
                               const double* b64, const float* chol, int64_t head, int64_t row,
                               float z2f, uint16_t* codes, float* dist, double* kx, int lane) {
  const int64_t off = (head * n + row) * kD;
  wave_sync();
  kx[lane] = (double)load_elem(keys, DT, off + lane);
  kx[lane + 64] = (double)load_elem(keys, DT, off + lane + 64);
  wave_sync();
  double best = -INFINITY;
  int bj = 0x7FFFFFFF;
  for (int64_t j = lane; j < c; j += 64) {
    const double* v = v64 + (head * c + j) * kD;
    double sj = 0.0;
    for (int a = 0; a < kD; ++a) sj += kx[a] * v[a];
    sj -= 0.5 * b64[head * c + j];
    if (sj > best || (sj == best && j < bj)) {
      best = sj;
      bj = (int)j;
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    const double ob = __shfl_xor(best, o);
    const int oj = __shfl_xor(bj, o);
    if (ob > best || (ob == best && oj < bj)) {
      best = ob;
      bj = oj;
    }
  }
  double zl = 0.0;
  if (dist && z2f < -1.5f) {  // one key per wave: uniform
    const float* L = chol + head * kD * kD;
    for (int a = lane; a < kD; a += 64) {
      double z = 0.0;
      for (int b = a; b < kD; ++b) z += kx[b] * (double)L[b * kD + a];  // L lower
      zl += z * z;
    }
    for (int o = 32; o > 0; o >>= 1) zl += __shfl_xor(zl, o);
  }
  if (lane == 0) {
    codes[head * n + row] = (uint16_t)bj;
    if (dist) {
      double z2 = z2f < -1.5f ? zl : (double)z2f;
      if (z2f < 0.f && z2f > -1.5f) {
        z2 = 0.0;
        for (int a = 0; a < kD; ++a) z2 += kx[a] * kx[a];
      }
      dist[head * n + row] = (float)fmax(z2 - 2.0 * best, 0.0);
    }
  }
}

// Four open keys a wave: fp64 over each key's candidates (4 lanes per candidate, 4 candidates
// of each key at a time), so that the keys' chains of dependent reads overlap (one key a wave
// took 55 us on the large-codebook workload, four take 32 us); a key whose candidate list
// overflowed gets the full scan, by the whole wave.  Then the keys the coarse pass listed for
// the full scan (fp16-range keys, rescan list overflow).  Decision counts
// are gathered per workgroup and added once, and only when statistics were asked for (a
// same-address atomic per wave would serialise at the end of the pass).
template <int DT>
__global__ __launch_bounds__(256) void enc_rescan_decide(
    const void* __restrict__ keys, int64_t n, int64_t heads, int64_t c,
    const double* __restrict__ v64, const float* __restrict__ v32, int plain,
    const double* __restrict__ b64,
    const UncEntry* __restrict__ unc, int64_t unc_cap, unsigned* __restrict__ cand_n,
    const int32_t* __restrict__ cand, uint16_t* __restrict__ codes, float* __restrict__ dist,
    FullEntry* __restrict__ full, Counters* __restrict__ cnt, int want_stats,
    const float* __restrict__ chol, int clear_words) {
  const int t = threadIdx.x, lane = t & 63, g = lane & 3, q16 = lane >> 2;
  const HeadSet hsx = all_heads(heads);
  __shared__ int64_t pre[kMaxHeadsLds + 1];
  __shared__ double kx[4][kD];
  auto per = [](int64_t m) { return m; };
  const int64_t total = head_prefix(cnt, hsx, unc_cap, pre, per);
  unsigned decided = 0, full_scans = 0;
  // Four keys a wave, sixteen lanes a key (lanes 16 kq ..): four candidates a round, four
  // lanes a candidate (lane quarter g of the dimensions), so that the four keys' chains of
  // dependent reads (entry, candidate list, rows) overlap.
  const int kq = lane >> 4, sub = (lane >> 2) & 3;
  for (int64_t e0 = (hsx.rank * 4 + (t >> 6)) * 4; e0 < total; e0 += hsx.ranks * 16) {
    const int64_t e = e0 + kq;
    const bool valid = e < total;
    int64_t rest = 0, head = 0, slot = 0;
    UncEntry ue;
    ue.row = 0;
    ue.jbest = 0;
    ue.z2 = 0.f;
    unsigned nc = 0u;
    if (valid) {
      head = find_head(cnt, hsx, unc_cap, pre, e, per, &rest);
      slot = head * unc_cap + rest;
      ue = unc[slot];
      nc = cand_n[slot];
    }
    if (valid && (lane & 15) == 0) cand_n[slot] = 0u;  // left cleared for the next run
    const bool full_key = valid && nc > (unsigned)kCandCap;
    const bool dec = valid && !full_key;
    const int64_t off = ((int64_t)head * n + ue.row) * kD;
    // exact fp64 scores of the collected candidates and of jbest (the entry's score is only a
    // lower bound of the best score, so jbest is scored here too); candidate nc is jbest
    double best = -INFINITY, k2 = 0.0;
    int bj = 0x7FFFFFFF;
    for (unsigned q0 = 0;; q0 += 4) {
      if (!__builtin_amdgcn_ballot_w64(dec && q0 <= nc)) break;
      const unsigned q = q0 + sub;
      const bool live = dec && q <= nc;
      const int jj = dec && q < nc ? cand[slot * kCandCap + q] : ue.jbest;
      const int64_t vo = ((int64_t)head * c + jj) * kD;
      const double bjj = b64[(int64_t)head * c + jj];
      double kk = 0.0;
      const double sj = plain ? coop_score_g<DT, 4>(keys, off, v32 + vo, bjj, g, &kk)
                              : coop_score_g<DT, 4>(keys, off, v64 + vo, bjj, g, &kk);
      double s = live ? sj : -INFINITY;
      int j = live ? jj : 0x7FFFFFFF;
      if (q0 == 0) k2 = kk;  // ||k||^2, for distances without a precomputed ||kL||^2
      for (int o = 4; o < 16; o <<= 1) {  // within the key's sixteen lanes
        const double os = __shfl_xor(s, o);
        const int oj = __shfl_xor(j, o);
        if (os > s || (os == s && oj < j)) {
          s = os;
          j = oj;
        }
      }
      if (s > best || (s == best && j < bj)) {
        best = s;
        bj = j;
      }
    }
    if (dec && (lane & 15) == 0) {
      codes[(int64_t)head * n + ue.row] = (uint16_t)bj;
      if (dist) {
        const double z2 = ue.z2 >= 0.f ? (double)ue.z2 : k2;
        dist[(int64_t)head * n + ue.row] = (float)fmax(z2 - 2.0 * best, 0.0);
      }
    }
    const unsigned long long dm = __builtin_amdgcn_ballot_w64(dec && (lane & 15) == 0);
    if (lane == 0) decided += (unsigned)__popcll(dm);
    // a key whose candidate list overflowed gets the full scan, by the whole wave
    unsigned long long fm = __builtin_amdgcn_ballot_w64(full_key && (lane & 15) == 0);
    while (fm) {
      const int src = __ffsll((long long)fm) - 1;
      fm &= fm - 1;
      const int64_t fh = __shfl((int)head, src);
      const int64_t frow = __shfl(ue.row, src);
      const float fz2 = __shfl(ue.z2, src);
      full_scan_wave<DT>(keys, n, c, v64, b64, chol, fh, frow, fz2, codes, dist, kx[t >> 6],
                         lane);
      if (lane == 0) full_scans += 1;
    }
  }
  const unsigned nfull = __hip_atomic_load(&cnt->full, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int64_t e = (int64_t)blockIdx.x * 4 + (t >> 6); e < (int64_t)nfull; e += (int64_t)gridDim.x * 4) {
    const FullEntry fe = full[e];
    full_scan_wave<DT>(keys, n, c, v64, b64, chol, fe.head, fe.row, fe.z2, codes, dist, kx[t >> 6],
                       lane);
    if (lane == 0) full_scans += 1;
  }
  if (want_stats) {
    __shared__ unsigned s_dec, s_full;
    if (t == 0) s_dec = s_full = 0u;
    __syncthreads();
    if (lane == 0 && decided) atomicAdd(&s_dec, decided);
    if (lane == 0 && full_scans) atomicAdd(&s_full, full_scans);
    __syncthreads();
    if (t == 0 && s_dec) atomicAdd(&cnt->stats[3], s_dec);
    if (t == 0 && s_full) atomicAdd(&cnt->stats[4], s_full);
  }
  if (clear_words > 0) {  // the last workgroup to finish leaves the run counters cleared
    // Without statistics this pass changes no counter; it only reads them, and every read
    // has returned (its value was used) before the workgroup takes its ticket, so no
    // device-scope fence is needed (one costs an L2 write-back per workgroup); the clearing
    // stores are device-scope atomics, visible to every XCD.  Tickets are taken in two
    // levels, per group of workgroups (blockIdx % 8) and then per group: same-address
    // device-scope atomics serialise at the memory side, 256 of them on one address cost
    // about 6 us.
    __shared__ unsigned s_last;
    __syncthreads();
    if (t == 0) {
      const unsigned grp = blockIdx.x % 8u;
      const unsigned members = gridDim.x / 8u + (grp < gridDim.x % 8u ? 1u : 0u);
      const bool last_of_grp = atomicAdd(&cnt->done_grp[grp][0], 1u) == members - 1u;
      const unsigned groups = gridDim.x < 8u ? gridDim.x : 8u;
      s_last = last_of_grp && atomicAdd(&cnt->done, 1u) == groups - 1u;
    }
    __syncthreads();
    if (s_last) {
      unsigned* w = reinterpret_cast<unsigned*>(cnt);
      for (int i = t; i < clear_words; i += 256)
        __hip_atomic_store(&w[i], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}


// ||k L||^2 in fp64, one wave per selected key (fp32 keys with distances and L).
__global__ __launch_bounds__(256) void enc_znorm64(const float* __restrict__ keys, int64_t n,
                                                   const int32_t* __restrict__ idx,
                                                   int64_t n_sel, int64_t heads,
                                                   const float* __restrict__ chol,
                                                   float* __restrict__ znorm) {
  __shared__ double kx[4][kD];
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int64_t total = heads * n_sel;
  for (int64_t e = (int64_t)blockIdx.x * 4 + wave; e < total; e += (int64_t)gridDim.x * 4) {
    const int64_t head = e / n_sel, sel = e % n_sel;
    const int64_t row = idx ? (int64_t)idx[head * n_sel + sel] : sel;
    if (row < 0 || row >= n) continue;  // uniform per wave: one key per wave
    const float* k = keys + (head * n + row) * kD;
    wave_sync();
    kx[wave][lane] = (double)k[lane];
    kx[wave][lane + 64] = (double)k[lane + 64];
    wave_sync();
    const float* L = chol + head * kD * kD;
    double part = 0.0;
    for (int a = lane; a < kD; a += 64) {
      double z = 0.0;
      for (int b = a; b < kD; ++b) z += kx[wave][b] * (double)L[b * kD + a];  // L lower
      part += z * z;
    }
    for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o);
    if (lane == 0) znorm[head * n + row] = (float)part;
  }
}

// Copies the run's decision counts out, then leaves the run counters cleared.
__global__ void enc_stats_out(Counters* __restrict__ cnt, a2ats_encode_stats* out, int clear_words) {
  if (threadIdx.x == 0) {
    unsigned keys = 0, direct = 0;
    for (int x = 0; x < 8; ++x) {
      keys += cnt->stat_x[x][0];
      direct += cnt->stat_x[x][1];
    }
    out->keys = keys;
    out->direct = direct;
    unsigned reranked = 0;
    for (int x = 0; x < 8; ++x) reranked += cnt->stat_x[x][2];
    out->reranked = reranked;
    out->rescanned = cnt->stats[3];
    out->full_scan = cnt->stats[4];
    out->reserved[0] = 0;
    out->reserved[1] = cnt->full;
    out->reserved[2] = 0;
  }
  __syncthreads();
  unsigned* w = reinterpret_cast<unsigned*>(cnt);
  for (int i = threadIdx.x; i < clear_words; i += blockDim.x) w[i] = 0u;
}

// ------------------------------------------------------------------ host side
inline int64_t unc_capacity(int64_t n) {
  const int64_t cap = n / 8;
  return cap < 1024 ? (n < 1024 ? n : 1024) : cap;
}

struct EncLayout {
  double* v64;
  float* v32;
  double* b64;
  half8* v16;
  float* bias;
  half8* lfrag;
  float* part_a;
  float* part_b;
  unsigned* cnt;
  UncEntry* unc;
  FullEntry* full;
  unsigned* cand_n;
  int32_t* cand;
  float* znorm;
  float* vnorm;
  HeadScale* hsc;
  double* gram;
  int nwg_a, nwg_b, ncnt;
  int64_t unc_cap;
  size_t bytes;
};

// Codebook tiles of 32 centroids, padded to whole coarse-pass stages; the padding tiles hold
// zero fragments and the padding bias.
int64_t tiles_of(int64_t c) { return ((c + kRows - 1) / kRows + kTPS - 1) / kTPS * kTPS; }

EncLayout carve(void* ws, int64_t heads, int64_t n, int64_t c) {
  const int64_t T = tiles_of(c);
  Carver cv(ws);
  EncLayout L;
  L.nwg_a = (int)((c + 31) / 32);
  L.nwg_b = (int)((T * kRows + kD + 15) / 16);
  L.ncnt = (int)(offsetof(Counters, unc) / 4 + heads);
  L.unc_cap = unc_capacity(n);
  L.v64 = cv.take<double>((size_t)heads * c * kD);
  L.v32 = cv.take<float>((size_t)heads * c * kD);
  L.b64 = cv.take<double>((size_t)heads * c);
  L.vnorm = cv.take<float>((size_t)heads * c);
  L.v16 = cv.take<half8>((size_t)heads * T * kFragPerTile);
  L.bias = cv.take<float>((size_t)heads * T * 32);
  L.lfrag = cv.take<half8>((size_t)heads * 8 * kFragPerTile);
  L.part_a = cv.take<float>((size_t)heads * L.nwg_a * 4);
  L.part_b = cv.take<float>((size_t)heads * L.nwg_b * 2);
  L.hsc = cv.take<HeadScale>((size_t)heads);
  L.gram = cv.take<double>((size_t)heads * kD * kD);
  L.cnt = cv.take<unsigned>((size_t)L.ncnt);
  L.unc = cv.take<UncEntry>((size_t)heads * L.unc_cap);
  L.full = cv.take<FullEntry>((size_t)heads * n);
  L.cand_n = cv.take<unsigned>((size_t)heads * L.unc_cap);
  L.cand = cv.take<int32_t>((size_t)heads * L.unc_cap * kCandCap);
  L.znorm = cv.take<float>((size_t)heads * n);
  L.bytes = cv.used;
  return L;
}

// Codebook-side preparation: M = L L^T (with L), v, b, the fp16 fragments, the bias and the
// per-head scales.  Depends on the codebook and L only.
int encode_prepare(int64_t heads, const float* codebook, int64_t c, const float* chol,
                   const EncLayout& L, hipStream_t s) {
  const int T = (int)tiles_of(c);
  const bool plain = chol == nullptr;
  const int64_t ncand = heads * L.unc_cap;
  if (!plain)
    A2ATS_TRY(launch("encode_prep_gram", enc_prep_gram, dim3(kD / 8, (unsigned)heads), dim3(256), 0, s,
                     chol, L.gram, L.part_a, L.nwg_a));
  A2ATS_TRY(launch("encode_prep_rows", enc_prep_rows, dim3((unsigned)L.nwg_a, (unsigned)heads),
                   dim3(256), 0, s, codebook, c, plain ? nullptr : L.gram, L.v64, L.v32, L.b64,
                   L.vnorm, L.part_a, L.nwg_a));
  return launch("encode_prep_frag", enc_prep_frag, dim3((unsigned)L.nwg_b, (unsigned)heads),
                dim3(256), 0, s, L.v64, L.b64, c, T, chol, (int)!plain, L.part_a, L.nwg_a,
                L.part_b, L.v16, L.bias, L.lfrag, L.hsc, L.cnt, L.ncnt, L.cand_n, ncand);
}

// Key-side pass over a prepared workspace.
template <int DT>
int encode_run(const void* keys, int64_t heads, int64_t n, const int32_t* idx, int64_t n_sel,
               int64_t c, const float* chol, uint16_t* codes, float* dist,
               a2ats_encode_stats* stats, const EncLayout& L, hipStream_t s) {
  const int T = (int)tiles_of(c);
  // packed into the low bits of the coarse pass: (tile << 1 | parity)
  int tbits = 1;
  while ((1 << (tbits - 1)) < T) ++tbits;
  const bool plain = chol == nullptr;
  Counters* cnt = reinterpret_cast<Counters*>(L.cnt);
  const bool znorm_mfma = dist && !plain && DT == A2ATS_BF16;
  float* znorm = nullptr;
  if (dist && !plain) {
    znorm = L.znorm;
    if (DT == A2ATS_F32)
      A2ATS_TRY(launch("encode_znorm64", enc_znorm64, dim3(grid_for(heads * n_sel, 4, 65536)),
                       dim3(256), 0, s, static_cast<const float*>(keys), n, idx, n_sel, heads, chol,
                       L.znorm));
  }
  const int nkb = (int)((n_sel + kKeysPerWG - 1) / kKeysPerWG);
  const int64_t G = (heads * nkb + 7) / 8 * 8;
  const char* name = plain ? "encode_coarse_plain" : "encode_coarse_h";
#define A2ATS_COARSE(Z, DI)                                                                       \
  launch(name, enc_coarse<DT, Z, DI>, dim3((unsigned)G), dim3(256), 0, s, keys, n, idx, n_sel,   \
         heads, nkb, T, tbits, L.v16, L.bias, L.v32, L.b64, c, L.lfrag, L.hsc,                    \
         L.part_b, L.nwg_b, znorm, codes, dist, L.vnorm, L.unc, L.unc_cap, L.full,                   \
         cnt, stats ? 1 : 0)
  if (znorm_mfma) A2ATS_TRY(A2ATS_COARSE(true, true));
  else if (dist) A2ATS_TRY(A2ATS_COARSE(false, true));
  else A2ATS_TRY(A2ATS_COARSE(false, false));
#undef A2ATS_COARSE
  A2ATS_TRY(launch("encode_rescan_collect", enc_rescan_collect<DT>, dim3(512), dim3(256), 0, s, keys,
                   n, heads, T, c, L.v16, L.bias, L.hsc, L.unc, L.unc_cap, cnt,
                   L.cand_n, L.cand));
  A2ATS_TRY(launch("encode_rescan_decide", enc_rescan_decide<DT>, dim3(kDecideWgs), dim3(256), 0, s, keys, n,
                   heads, c, L.v64, L.v32, plain ? 1 : 0, L.b64, L.unc, L.unc_cap, L.cand_n, L.cand, codes, dist, L.full,
                   cnt, stats ? 1 : 0, chol, stats ? 0 : L.ncnt));
  if (stats)
    A2ATS_TRY(launch("encode_stats", enc_stats_out, dim3(1), dim3(64), 0, s, cnt, stats, L.ncnt));
  return A2ATS_OK;
}

}  // namespace
}  // namespace a2ats

using namespace a2ats;

extern "C" size_t a2ats_encode_workspace(int64_t heads, int64_t n, int64_t d, int64_t c) {
  if (heads < 1 || n < 0 || d != kD || c < 1 || c > 65536) return 0;
  return carve(nullptr, heads, n, c).bytes;
}

static int encode_check_keys(const void* keys, int keys_dtype, int64_t heads, int64_t n, int64_t d,
                             const int32_t* idx, int64_t n_idx, int64_t c, uint16_t* codes,
                             int64_t* n_sel) {
  if (keys_dtype != A2ATS_F32 && keys_dtype != A2ATS_BF16) return A2ATS_EDTYPE;
  if (d != kD || heads < 1 || n < 0 || c < 1 || c > 65536) return A2ATS_EINVAL;
  if (n > 0x7FFFFFFF || heads > 65535) return A2ATS_EINVAL;
  *n_sel = idx ? n_idx : n;
  if (*n_sel < 0 || *n_sel > n) return A2ATS_EINVAL;
  if (*n_sel == 0) return A2ATS_OK;
  if (!keys || !codes) return A2ATS_EINVAL;
  if ((reinterpret_cast<uintptr_t>(keys) & 15) != 0) return A2ATS_EINVAL;
  return A2ATS_OK;
}

static int encode_dispatch(const void* keys, int keys_dtype, int64_t heads, int64_t n,
                           const int32_t* idx, int64_t n_sel, int64_t c, const float* chol,
                           uint16_t* codes, float* dist, a2ats_encode_stats* stats,
                           const EncLayout& L, hipStream_t s) {
  if (keys_dtype == A2ATS_BF16)
    return encode_run<A2ATS_BF16>(keys, heads, n, idx, n_sel, c, chol, codes, dist, stats, L, s);
  return encode_run<A2ATS_F32>(keys, heads, n, idx, n_sel, c, chol, codes, dist, stats, L, s);
}

extern "C" int a2ats_encode(const void* keys, int keys_dtype, int64_t heads, int64_t n, int64_t d,
                            const int32_t* idx, int64_t n_idx, const float* codebook, int64_t c,
                            const float* chol, uint16_t* codes, float* dist,
                            a2ats_encode_stats* stats, void* workspace, size_t workspace_bytes,
                            void* stream) {
  int64_t n_sel = 0;
  A2ATS_TRY(encode_check_keys(keys, keys_dtype, heads, n, d, idx, n_idx, c, codes, &n_sel));
  if (n_sel == 0) return A2ATS_OK;
  if (!codebook) return A2ATS_EINVAL;
  const size_t need = a2ats_encode_workspace(heads, n, d, c);
  if (!ws_ok(workspace, workspace_bytes, need)) return A2ATS_EWORKSPACE;
  EncLayout L = carve(workspace, heads, n, c);
  hipStream_t s = static_cast<hipStream_t>(stream);
  A2ATS_TRY(encode_prepare(heads, codebook, c, chol, L, s));
  return encode_dispatch(keys, keys_dtype, heads, n, idx, n_sel, c, chol, codes, dist, stats, L, s);
}

// codes[h, idx[h, i]] = src[h, idx[h, i]]: the retrieval keys take the query-aware codes.
__global__ __launch_bounds__(256) void enc_merge(const uint16_t* __restrict__ src,
                                                 const int32_t* __restrict__ idx, int64_t heads,
                                                 int64_t n, int64_t n_idx,
                                                 uint16_t* __restrict__ codes) {
  const int64_t total = heads * n_idx;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * 256) {
    const int64_t h = e / n_idx;
    const int64_t r = idx[e];
    if (r >= 0 && r < n) codes[h * n + r] = src[h * n + r];
  }
}

extern "C" int a2ats_merge_codes(const uint16_t* src, const int32_t* idx, int64_t heads,
                                 int64_t n, int64_t n_idx, uint16_t* codes, void* stream) {
  if (heads < 1 || heads > 65535 || n < 0 || n > 0x7FFFFFFF || n_idx < 0 || n_idx > n)
    return A2ATS_EINVAL;
  if (n_idx == 0) return A2ATS_OK;
  if (!src || !idx || !codes) return A2ATS_EINVAL;
  if (src == codes) return A2ATS_OK;
  return launch("encode_merge", enc_merge, dim3(grid_for(heads * n_idx, 256, 4096)), dim3(256), 0,
                static_cast<hipStream_t>(stream), src, idx, heads, n, n_idx, codes);
}

extern "C" int a2ats_encode_prepare(const float* codebook, int64_t c, const float* chol,
                                    int64_t heads, int64_t n, int64_t d, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  if (d != kD || heads < 1 || heads > 65535 || n < 0 || n > 0x7FFFFFFF || c < 1 || c > 65536)
    return A2ATS_EINVAL;
  if (!codebook) return A2ATS_EINVAL;
  const size_t need = a2ats_encode_workspace(heads, n, d, c);
  if (!ws_ok(workspace, workspace_bytes, need)) return A2ATS_EWORKSPACE;
  return encode_prepare(heads, codebook, c, chol, carve(workspace, heads, n, c),
                        static_cast<hipStream_t>(stream));
}

extern "C" int a2ats_encode_prepared(const void* keys, int keys_dtype, int64_t heads, int64_t n,
                                     int64_t d, const int32_t* idx, int64_t n_idx, int64_t c,
                                     const float* chol, uint16_t* codes, float* dist,
                                     a2ats_encode_stats* stats, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  int64_t n_sel = 0;
  A2ATS_TRY(encode_check_keys(keys, keys_dtype, heads, n, d, idx, n_idx, c, codes, &n_sel));
  if (n_sel == 0) return A2ATS_OK;
  const size_t need = a2ats_encode_workspace(heads, n, d, c);
  if (!ws_ok(workspace, workspace_bytes, need)) return A2ATS_EWORKSPACE;
  return encode_dispatch(keys, keys_dtype, heads, n, idx, n_sel, c, chol, codes, dist, stats,
                         carve(workspace, heads, n, c), static_cast<hipStream_t>(stream));
}
