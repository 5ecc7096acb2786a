// Sub-vector (product) VQ: the pages' default configuration.  The "A2ATS-adapted" docs
// ("Configuration reference", "What you get with the defaults", the calibration example of
// "How it works") bundle sub_dim consecutive numbers of a head vector into one lookup: a
// single codebook of 2^bits sub-centroids of width sub_dim, trained on the pooled
// sub-vectors of every head, and one optional sub_dim x sub_dim query second moment H.
// Each sub-vector gets its own code (one byte):
//   H-weighted  argmin_j (x_s - c_j) H (x_s - c_j)^T            ("veloxquant_mlx.quantizers.
//                                                                 a2ats module",
//                                                                 a2ats_h_weighted_assignment)
//   blend       argmax_j beta (-e_j / max e) + (1 - beta) cos(q_s, c_j)
//                                                                (a2ats_query_aware_assignment,
//                                                                 q_s the same slice of the query)
//   plain       argmin_j ||x_s - c_j||^2                         (bulk rows and values)
// Ties go to the lowest index.
//
// Encode on the matrix cores.  With v_j = c_j H (c_j itself without H), b_j = c_j H c_j^T,
//     argmin_j (x_s - c_j) H (x_s - c_j)^T = argmax_j s_j,   s_j = x_s . v_j - b_j / 2,
// so the code is a contraction of every sub-vector against the (at most 256-row) table plus a
// row argmax.  A wave takes 64 sub-vectors, two blocks of 32 MFMA columns, against the whole
// table, 8 tiles of 32 rows, on v_mfma_f32_32x32x16_f16.  The table side is scaled by a
// power of two S and split into fp16 hi + lo parts; the sub-vectors are exact in fp16 (bf16
// inputs in fp16's range) or split the same way (fp32 inputs); the bias -S b_j / 2 enters as
// fp16 hi + lo parts times a power of two (sub_dim 8: a small MFMA per tile whose result seeds
// both blocks' accumulators; sub_dim 4: spare K slots of the same MFMA).  The table operands
// live in LDS, prepared by each workgroup.
//   Fold: each accumulator register keeps its maximum over the 8 tiles (v_maximum3, half an
// operation per score, no index).  A sub-vector's 32 register maxima ("slots", 16 in each
// lane of a lane pair, exchanged with v_permlane32_swap) are packed with their slot number
// and the largest two taken: the winning slot and a bound on every other slot.  The winning
// slot's 8 centroids are scored again in fp64, and the best of them is the code when its
// score beats the second slot's maximum by more than a rigorous bound on an MFMA score's
// error (hi/lo residuals, the bias residual, fp32 accumulation of up to 25 terms, the packed
// low bits), taken only over the rows that could reach that score at all: s_j <= ||z|| n_j -
// n_j^2 / 2 with n_j = ||c_j L|| (z = x L) limits them to n_j <= R = ||z|| + sqrt(||z||^2 -
// 2 s_a), and every error term of a row grows with n_j (a table with a few far-out rows would
// otherwise set the bound for all).  The rest, about 1 in 10^4 on the workloads, is decided by
// the whole wave in fp64 over the whole table.
//   Blend: e_j = ||x - c_j||^2 = ||x||^2 - 2 s_j (plain s_j), so max_j e_j comes from a first
// pass folding the smallest s_j the same way (the farthest slot rescored in fp64, exactly as
// the definition sums).  Up to a constant per sub-vector the blended score is
//     (2 beta / max e) s_j + ((1 - beta) / ||q_s||) (q_s . c_j / ||c_j||),
// formed in fp32 from two accumulators (the second against the unit-norm table) and folded as
// above; the winning slot is rescored in fp64 by the blend's own formula (reciprocals of
// max e, ||q_s|| and ||c_j|| taken once: a few ulps from the divided form).
#include "common.hpp"

namespace a2ats {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef __fp16 h2rtz __attribute__((ext_vector_type(2)));
typedef unsigned u4v __attribute__((ext_vector_type(4)));

constexpr int kD = A2ATS_HEAD_DIM;
constexpr int kPqMaxK = 256;
constexpr int kPqTiles = kPqMaxK / 32;
constexpr int kPqWaves = 4;
constexpr int kPqThreads = 64 * kPqWaves;  // one table row per thread in the preparation
constexpr int kPqWgPerCu = 2;
constexpr int kPqCus = 256;
constexpr float kPadMark = 65504.f;        // the largest fp16: x 2^15, a pad row's bias
constexpr double kRnd = 0x1p-23;           // one fp32 rounding, doubled (truncation allowed)
constexpr double kHalfMin = 0x1p-14;       // smallest normal fp16

enum PqMode { kPlain = 0, kHWeighted = 1, kBlend = 2 };

// Two floats to packed fp16, rounded toward zero (exact for values fp16 holds).
__device__ __forceinline__ unsigned pk16(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(a, b));
}
__device__ __forceinline__ float lo16(unsigned p) { return (float)__builtin_bit_cast(h2rtz, p)[0]; }
__device__ __forceinline__ float hi16(unsigned p) { return (float)__builtin_bit_cast(h2rtz, p)[1]; }
__device__ __forceinline__ half8 h8(unsigned a, unsigned b, unsigned c, unsigned d) {
  const u4v v = {a, b, c, d};
  return __builtin_bit_cast(half8, v);
}
__device__ __forceinline__ unsigned pkh(_Float16 a, _Float16 b) {
  return (unsigned)__builtin_bit_cast(unsigned short, a) |
         ((unsigned)__builtin_bit_cast(unsigned short, b) << 16);
}
__device__ __forceinline__ float fmax3(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}
__device__ __forceinline__ double up(double x) { return x * (1.0 + 0x1p-40); }  // x >= 0

// fp16 nearest to x, with values below fp16's normal range flushed to zero (the residual is
// then carried by the next part or the error bound; no subnormal reaches the matrix cores
// from the table side).
__device__ __forceinline__ _Float16 half_of(double x) {
  const _Float16 h = (_Float16)(float)x;
  return fabs((double)h) < kHalfMin ? (_Float16)0.f : h;
}

// Workgroup-wide maxima of N doubles (every thread receives them).
template <int N>
__device__ __forceinline__ void block_max(double (&v)[N], double (*red)[kPqWaves]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < N; ++i)
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v[i] = fmax(v[i], __shfl_xor(v[i], o));
  if (lane == 0)
#pragma unroll
    for (int i = 0; i < N; ++i) red[i][wave] = v[i];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = fmax(fmax(red[i][0], red[i][1]), fmax(red[i][2], red[i][3]));
  __syncthreads();
}

// Workgroup-wide maxima of N floats (every thread receives them).
template <int N>
__device__ __forceinline__ void block_maxf(float (&v)[N], float (*red)[kPqWaves]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < N; ++i)
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v[i] = fmaxf(v[i], __shfl_xor(v[i], o));
  if (lane == 0)
#pragma unroll
    for (int i = 0; i < N; ++i) red[i][wave] = v[i];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = fmaxf(fmaxf(red[i][0], red[i][1]), fmaxf(red[i][2], red[i][3]));
  __syncthreads();
}

// x rounded to fp32 upward / downward (x >= 0).
__device__ __forceinline__ float round_up_f(double x) {
  float f = (float)x;
  if ((double)f < x) f = __uint_as_float(__float_as_uint(f) + 1u);
  return f;
}
__device__ __forceinline__ float round_down_f(double x) {
  float f = (float)x;
  if ((double)f > x) f = __uint_as_float(__float_as_uint(f) - 1u);
  return f;
}

template <int SUB, bool BLEND>
struct PqShared {
  half8 fa[kPqTiles][64];            // table operand, MFMA A order
  unsigned fb[kPqTiles][64][4];      // bias operand (sub_dim 8; zero in lanes 32-63 and in
                                     // dwords 2-3, so one 16-byte read is the operand)
  half8 fq[BLEND ? kPqTiles : 1][64];  // unit-norm table operand (blend)
  // per row in fp64: v_j (c_j for the blend), then b_j / 2 and 1 / ||c_j|| (0 for a zero row;
  // blend).  The row stride (80 or 48 bytes) puts 8 consecutive rows' 16-byte reads in 8
  // different LDS bank groups (a 64-byte stride would use 2).
  double v64[kPqMaxK][SUB + 2];
  double lsh[SUB][SUB];
  float l32[SUB][SUB];               // the fp32 factor (H-weighted)
  double red[4][kPqWaves];
  float redf[9][kPqWaves];
};

// Per-call constants of the preparation (identical in every thread).
struct PqConsts {
  int se, eb, sq;      // S = 2^se (table), bias parts x 2^eb, Sq = 2^sq (unit-norm table)
  bool finite;         // every table entry finite (else every sub-vector takes the fp64 scan)
  double rho, nu, nul, B, betab, Mv, Shb;  // bound terms of the table side (S units)
  double kv, kr, kl, kb, kbeta;            // the same per row, over ||w_j|| or ||w_j||^2
  double lf;                               // ||L||_F rounded up (H-weighted)
  double c_rr, c_x, c_d, c_l;              // E(R) = R (c_rr R + c_x ||x|| + c_d ||x - x'|| + c_l ||lo||)
  double rhoq, nuq, nulq;                  // the same for the unit-norm table (Sq units)
};

// The table operands and bound terms.  Thread t handles row t (rows >= k are pads: zero
// operand, bias -65504 x 2^15).
template <int SUB, int MODE, int DT>
__device__ __forceinline__ PqConsts pq_prep(const float* __restrict__ cb, int k,
                                            const float* __restrict__ chol,
                                            PqShared<SUB, MODE == kBlend>& sh) {
  const int t = threadIdx.x;
  if (MODE == kHWeighted && t < SUB * SUB) {
    sh.lsh[t / SUB][t % SUB] = (double)chol[t];
    sh.l32[t / SUB][t % SUB] = chol[t];
  }
  __syncthreads();
  double lf2 = 0.0;
  if constexpr (MODE == kHWeighted) {
#pragma unroll 1
    for (int i = 0; i < SUB * SUB; ++i) lf2 += sh.lsh[i / SUB][i % SUB] * sh.lsh[i / SUB][i % SUB];
  }
  const bool real = t < k;
  double c[SUB], v[SUB], hb;
#pragma unroll
  for (int e = 0; e < SUB; ++e) c[e] = real ? (double)cb[(int64_t)t * SUB + e] : 0.0;
  if constexpr (MODE == kHWeighted) {
    double w[SUB], b2 = 0.0;
#pragma unroll
    for (int a = 0; a < SUB; ++a) {
      double s = 0.0;
#pragma unroll
      for (int b = 0; b < SUB; ++b) s += c[b] * sh.lsh[b][a];  // (c L)_a
      w[a] = s;
      b2 += s * s;
    }
    hb = 0.5 * b2;
#pragma unroll
    for (int e = 0; e < SUB; ++e) {
      double s = 0.0;
#pragma unroll
      for (int a = 0; a < SUB; ++a) s += w[a] * sh.lsh[e][a];  // (w L^T)_e = (c H)_e
      v[e] = s;
    }
  } else {
    double b2 = 0.0;
#pragma unroll
    for (int e = 0; e < SUB; ++e) {
      v[e] = c[e];
      b2 += c[e] * c[e];
    }
    hb = 0.5 * b2;
  }
  double mv = 0.0, ic = 0.0, mq = 0.0, fin = 0.0;
#pragma unroll
  for (int e = 0; e < SUB; ++e) {
    sh.v64[t][e] = v[e];
    mv = fmax(mv, fabs(v[e]));
    fin += 0.0 * v[e];
  }
  sh.v64[t][SUB] = real ? hb : 0x1p1000;  // a pad row scores about -2^1000 in fp64
  sh.v64[t][SUB + 1] = 0.0;
  fin += 0.0 * hb;
  if constexpr (MODE == kBlend) {
    double cn2 = 0.0;
#pragma unroll
    for (int e = 0; e < SUB; ++e) cn2 += c[e] * c[e];
    const double cn = sqrt(cn2);
    ic = cn > 0.0 ? 1.0 / cn : 0.0;
    sh.v64[t][SUB + 1] = ic;
#pragma unroll
    for (int e = 0; e < SUB; ++e) mq = fmax(mq, fabs(c[e] * ic));
  }
  double r1[4] = {mv, hb, mq, fin == 0.0 ? 0.0 : 1.0};  // fin: NaN for a non-finite row
  block_max(r1, sh.red);
  PqConsts pc;
  pc.finite = r1[3] == 0.0;
  pc.lf = up(sqrt(lf2)) * (1.0 + 0x1p-30);
  int se = 0;
  if (r1[0] > 0.0) se = 14 - ilogb(r1[0]);
  if (r1[1] > 0.0) se = min(se, 28 - ilogb(r1[1]));
  se = max(-900, min(900, se));
  const double S = ldexp(1.0, se);
  int eb = r1[1] > 0.0 ? ilogb(S * r1[1]) - 14 : -14;
  eb = max(-14, min(15, eb));
  const int sq = r1[2] > 0.0 ? 14 - ilogb(r1[2]) : 0;
  pc.se = se;
  pc.eb = eb;
  pc.sq = sq;

  // fp16 parts of S v_j and their residuals
  _Float16 vh[SUB], vl[SUB];
  double rr = 0.0, nh2 = 0.0, nl2 = 0.0, nv2 = 0.0;
#pragma unroll
  for (int e = 0; e < SUB; ++e) {
    const double sv = S * v[e];
    vh[e] = half_of(sv);
    const double d1 = sv - (double)vh[e];
    vl[e] = half_of(d1);
    const double d2 = d1 - (double)vl[e];
    rr += d2 * d2;
    nh2 += (double)vh[e] * (double)vh[e];
    nl2 += (double)vl[e] * (double)vl[e];
    nv2 += sv * sv;
  }
  // the bias -S b_j / 2 as (h1 + h2) 2^eb
  const double bias = -S * hb;
  const double bs = ldexp(bias, -eb);
  const _Float16 h1 = half_of(bs);
  const _Float16 h2 = half_of(bs - (double)h1);
  const double cbm = ldexp(fabs((double)h1) + fabs((double)h2), eb);
  const double cbx = ldexp((double)h1 + (double)h2, eb);
  const _Float16 pm = real ? (_Float16)0.f : (_Float16)(-kPadMark);
  const _Float16 z16 = (_Float16)0.f;
  const int tile = t >> 5, r = t & 31;
  if constexpr (SUB == 8) {
    sh.fa[tile][r] = h8(pkh(vh[0], vh[1]), pkh(vh[2], vh[3]), pkh(vh[4], vh[5]), pkh(vh[6], vh[7]));
    sh.fa[tile][r + 32] = h8(pkh(vl[0], vl[1]), pkh(vl[2], vl[3]), pkh(vl[4], vl[5]), pkh(vl[6], vl[7]));
    sh.fb[tile][r][0] = pkh(h1, h2);
    sh.fb[tile][r][1] = pkh(pm, z16);
    sh.fb[tile][r][2] = 0u;
    sh.fb[tile][r][3] = 0u;
    sh.fb[tile][r + 32][0] = 0u;
    sh.fb[tile][r + 32][1] = 0u;
    sh.fb[tile][r + 32][2] = 0u;
    sh.fb[tile][r + 32][3] = 0u;
  } else {
    // K slots, lanes 0-31: vh vl; lanes 32-63: h1 h2 pad-mark, then (fp32 inputs) vh again
    // against the inputs' lo parts
    sh.fa[tile][r] = h8(pkh(vh[0], vh[1]), pkh(vh[2], vh[3]), pkh(vl[0], vl[1]), pkh(vl[2], vl[3]));
    if (DT == A2ATS_F32)
      sh.fa[tile][r + 32] = h8(pkh(h1, h2), pkh(pm, vh[0]), pkh(vh[1], vh[2]), pkh(vh[3], z16));
    else
      sh.fa[tile][r + 32] = h8(pkh(h1, h2), pkh(pm, z16), 0u, 0u);
  }
  // Row terms in fp32 rounded up; the blend keeps their maxima, the plain and H-weighted codes
  // the maxima of the same divided by the row's size n_j = ||w_j|| (||c_j|| without H, so
  // b_j / 2 = n_j^2 / 2; a zero row has no error terms at all).  n_j below 2^-60 counts as
  // 2^-60 (R is never smaller).
  auto sq_up = [](double s2) { return sqrtf(round_up_f(s2)) * (1.f + 0x1p-20f); };
  const float rho_j = sq_up(rr), nul_j = sq_up(nl2);
  const float nu_j = (sq_up(nh2) + nul_j) * (1.f + 0x1p-22f);
  const float cb_j = round_up_f(cbm * (1.0 + 0x1p-22));
  const float beta_j = round_up_f(fabs(cbx - bias) + kRnd * cbm);
  constexpr int NR = MODE == kBlend ? 9 : 5;
  float r2[NR];
  if constexpr (MODE == kBlend) {
    const double Sq = ldexp(1.0, sq);
    _Float16 ch[SUB], cl[SUB];
    double rq = 0.0, qh2 = 0.0, ql2 = 0.0;
#pragma unroll
    for (int e = 0; e < SUB; ++e) {
      const double u = Sq * (c[e] * ic);
      ch[e] = half_of(u);
      const double d1 = u - (double)ch[e];
      cl[e] = half_of(d1);
      const double d2 = d1 - (double)cl[e];
      rq += d2 * d2;
      qh2 += (double)ch[e] * (double)ch[e];
      ql2 += (double)cl[e] * (double)cl[e];
    }
    if constexpr (SUB == 8) {
      sh.fq[tile][r] = h8(pkh(ch[0], ch[1]), pkh(ch[2], ch[3]), pkh(ch[4], ch[5]), pkh(ch[6], ch[7]));
      sh.fq[tile][r + 32] = h8(pkh(cl[0], cl[1]), pkh(cl[2], cl[3]), pkh(cl[4], cl[5]), pkh(cl[6], cl[7]));
    } else {
      sh.fq[tile][r] = h8(pkh(ch[0], ch[1]), pkh(ch[2], ch[3]), pkh(cl[0], cl[1]), pkh(cl[2], cl[3]));
      if (DT == A2ATS_F32)
        sh.fq[tile][r + 32] = h8(0u, pkh(z16, ch[0]), pkh(ch[1], ch[2]), pkh(ch[3], z16));
      else
        sh.fq[tile][r + 32] = h8(0u, 0u, 0u, 0u);
    }
    const float nulq = sq_up(ql2);
    const float vals[9] = {rho_j, nu_j, nul_j, sq_up(nv2), cb_j, beta_j, sq_up(rq),
                           (sq_up(qh2) + nulq) * (1.f + 0x1p-22f), nulq};
#pragma unroll
    for (int q = 0; q < 9; ++q) r2[q] = vals[q];
  } else {
    const double n2 = 2.0 * hb;
    float inj = 0.f;  // 1 / max(n_j, 2^-60), rounded up
    if (n2 > 0.0) {
      float nlo = sqrtf(round_down_f(n2)) * (1.f - 0x1p-20f);
      nlo = fmaxf(nlo, 0x1p-60f);
      inj = n2 < 3.0e38 ? (1.f / nlo) * (1.f + 0x1p-20f) : INFINITY;
    }
    const float inj2 = inj * inj * (1.f + 0x1p-20f), f = 1.f + 0x1p-20f;
    const float vals[5] = {nu_j * inj * f, rho_j * inj * f, nul_j * inj * f, cb_j * inj2 * f,
                           beta_j * inj2 * f};
#pragma unroll
    for (int q = 0; q < 5; ++q) r2[q] = n2 > 0.0 ? vals[q] : 0.f;
  }
  block_maxf(r2, sh.redf);  // also publishes the operands written above
  pc.Shb = up(ldexp(r1[1], se));
  if constexpr (MODE == kBlend) {
    pc.rho = r2[0];
    pc.nu = r2[1];
    pc.nul = r2[2];
    pc.Mv = r2[3];
    pc.B = r2[4];
    pc.betab = r2[5];
    pc.rhoq = r2[6];
    pc.nuq = r2[7];
    pc.nulq = r2[8];
  } else {
    pc.kv = r2[0];
    pc.kr = r2[1];
    pc.kl = r2[2];
    pc.kb = r2[3];
    pc.kbeta = r2[4];
  }
  {
    // the bound for rows of size at most R (score_bound_r), its terms collected
    constexpr int terms = (SUB == 8 ? 2 * SUB + 1 : 2 * SUB + 3) + (DT == A2ATS_F32 ? SUB : 0);
    const double g = (terms + 2) * kRnd, f = (1.0 + 0x1p-16) * (1.0 + 0x1p-30);
    pc.c_rr = (g * pc.kb + pc.kbeta) * f + 0x1p-40 * pc.kb;
    pc.c_x = (g * pc.kv + pc.kr) * f + 0x1p-40 * pc.kv;
    pc.c_d = (g * pc.kv + pc.kr + pc.kv + pc.kr) * f;
    pc.c_l = (2.0 * g * pc.kv + pc.kl) * f;
  }
  return pc;
}

// The raw dwords of one sub-vector: SUB bf16 (SUB / 2 dwords) or SUB fp32.
template <int DT, int SUB>
struct Raw {
  static constexpr int W = DT == A2ATS_BF16 ? SUB / 2 : SUB;
  unsigned w[W];
};

template <int DT, int SUB>
__device__ __forceinline__ Raw<DT, SUB> load_raw(const void* base, int64_t elem, bool ok) {
  Raw<DT, SUB> r;
  constexpr int W = Raw<DT, SUB>::W;
  const unsigned* p = reinterpret_cast<const unsigned*>(
      static_cast<const char*>(base) + (ok ? elem : 0) * (DT == A2ATS_BF16 ? 2 : 4));
  if constexpr (W == 2) {
    const uint2 a = ok ? *reinterpret_cast<const uint2*>(p) : make_uint2(0u, 0u);
    r.w[0] = a.x;
    r.w[1] = a.y;
  } else {
#pragma unroll
    for (int q = 0; q < W / 4; ++q) {
      const uint4 a = ok ? reinterpret_cast<const uint4*>(p)[q] : make_uint4(0u, 0u, 0u, 0u);
      r.w[4 * q] = a.x;
      r.w[4 * q + 1] = a.y;
      r.w[4 * q + 2] = a.z;
      r.w[4 * q + 3] = a.w;
    }
  }
  return r;
}

template <int DT, int SUB>
__device__ __forceinline__ void raw_floats(const Raw<DT, SUB>& r, float (&x)[SUB]) {
  if constexpr (DT == A2ATS_BF16) {
#pragma unroll
    for (int i = 0; i < SUB / 2; ++i) {
      x[2 * i] = __uint_as_float(r.w[i] << 16);
      x[2 * i + 1] = __uint_as_float(r.w[i] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < SUB; ++i) x[i] = __uint_as_float(r.w[i]);
  }
}

template <int DT, int SUB>
__device__ __forceinline__ Raw<DT, SUB> raw_sel(const Raw<DT, SUB>& a, const Raw<DT, SUB>& b, bool second) {
  Raw<DT, SUB> r;
#pragma unroll
  for (int i = 0; i < Raw<DT, SUB>::W; ++i) r.w[i] = second ? b.w[i] : a.w[i];
  return r;
}

// B operands of one block column.  hi: the fp16 parts (x itself for bf16); lo: fp32 inputs'
// second parts.  sub_dim 8: B1 = [hi | hi], B2 = [lo | 0].  sub_dim 4: lanes 0-31 [hi hi],
// lanes 32-63 [2^eb 2^eb 2^15 lo 0] (the bias and pad-mark slots; `tail` for a table without
// bias, the unit-norm one, has zeros there).
template <int DT, int SUB>
__device__ __forceinline__ void make_b(const Raw<DT, SUB>& r, int hh, unsigned bias_pk,
                                       unsigned mark_pk, half8& B1, half8& B2) {
  float x[SUB];
  raw_floats<DT, SUB>(r, x);
  unsigned p[SUB / 2], l[SUB / 2];
#pragma unroll
  for (int i = 0; i < SUB / 2; ++i) {
    p[i] = pk16(x[2 * i], x[2 * i + 1]);
    if (DT == A2ATS_F32) l[i] = pk16(x[2 * i] - lo16(p[i]), x[2 * i + 1] - hi16(p[i]));
  }
  if constexpr (SUB == 8) {
    B1 = h8(p[0], p[1], p[2], p[3]);
    if (DT == A2ATS_F32) B2 = hh ? h8(0u, 0u, 0u, 0u) : h8(l[0], l[1], l[2], l[3]);
  } else {
    if (DT == A2ATS_F32) {
      const unsigned mk = mark_pk & 0xFFFFu;  // 2^15 in the low half
      B1 = hh ? h8(bias_pk, mk | (l[0] << 16), (l[0] >> 16) | (l[1] << 16), l[1] >> 16)
              : h8(p[0], p[1], p[0], p[1]);
    } else {
      B1 = hh ? h8(bias_pk, mark_pk, 0u, 0u) : h8(p[0], p[1], p[0], p[1]);
    }
  }
}

// An upper bound of sqrt(s) for s >= 0: the hardware square root (within an ulp), a relative
// margin, and 2^-60 for an input the hardware flushes (below 2^-126).
__device__ __forceinline__ float sqrt_up(float s) {
  return __builtin_amdgcn_sqrtf(s * (1.f + 0x1p-18f)) * (1.f + 0x1p-20f) + 0x1p-60f;
}

// Maximum of two finite fp64 values (a single v_max_f64: the operands are bit-packed
// scores, never NaN, so no canonicalising is needed).
__device__ __forceinline__ double max_f64(double a, double b) {
  double r;
  asm("v_max_f64 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Norm terms of one sub-vector against what the matrix cores see of it, in fp32 rounded
// up: ||x||, ||x - x'|| (x' = the fp16 parts, a subnormal part possibly flushed) and ||lo||
// (fp32 inputs' second parts).  x - hi - lo is exact in fp32 (each part is the other's
// truncation).  A square that overflows makes the bound infinite (the fp64 scan decides).
template <int DT, int SUB>
__device__ __forceinline__ void norms(const Raw<DT, SUB>& r, float& nx, float& nd, float& nl) {
  float x[SUB];
  raw_floats<DT, SUB>(r, x);
  if constexpr (DT == A2ATS_BF16) {
    // a bf16 value is exact in fp16 when 2^-14 <= |x| <= 65504 (its 8 significant bits fit);
    // otherwise x' is 0, a subnormal or 65504 and |x - x'| <= |x|
    float sx = 0.f, sd = 0.f;
#pragma unroll
    for (int e = 0; e < SUB; ++e) {
      const float ax = fabsf(x[e]);
      const float d = __builtin_amdgcn_fmed3f(ax, (float)kHalfMin, 65504.f) == ax ? 0.f : x[e];
      sx = __fmaf_rn(x[e], x[e], sx);
      sd = __fmaf_rn(d, d, sd);
    }
    nx = sqrt_up(sx);
    nd = sd > 0.f ? sqrt_up(sd) : 0.f;
    nl = 0.f;
    return;
  }
  float sx = 0.f, sd = 0.f, sl = 0.f;
#pragma unroll
  for (int i = 0; i < SUB / 2; ++i) {
    const unsigned p = pk16(x[2 * i], x[2 * i + 1]);
    const float h[2] = {lo16(p), hi16(p)};
    float lw[2] = {0.f, 0.f};
    if (DT == A2ATS_F32) {
      const unsigned q = pk16(x[2 * i] - h[0], x[2 * i + 1] - h[1]);
      lw[0] = lo16(q);
      lw[1] = hi16(q);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float xe = x[2 * i + u], he = h[u], le = lw[u];
      float d = fabsf(xe - he - le);
      if (fabsf(he) < (float)kHalfMin) d += fabsf(he);
      if (DT == A2ATS_F32 && fabsf(le) < (float)kHalfMin) d += fabsf(le);
      sx = __fmaf_rn(xe, xe, sx);
      sd = __fmaf_rn(d, d, sd);
      sl = __fmaf_rn(le, le, sl);
    }
  }
  // SUB-term fp32 sums: within 2^-20 relative; sqrt within an ulp
  nx = sqrt_up(sx);
  nd = sd > 0.f ? sqrt_up(sd) : 0.f;
  nl = sl > 0.f ? sqrt_up(sl) : 0.f;
}

// Rigorous bound on |acc_j - S s_j| for every row j (S units).
template <int DT, int SUB>
__device__ __forceinline__ double score_bound(double nx, double nd, double nl, double rho,
                                              double nu, double nul, double B, double betab) {
  constexpr int terms = (SUB == 8 ? 2 * SUB + 1 : 2 * SUB + 3) + (DT == A2ATS_F32 ? SUB : 0);
  const double g = (terms + 2) * kRnd;
  const double nxh = nx + nl + nd;
  return (g * (B + (nxh + nl) * nu) + (nx + nd) * rho + nd * (nu + rho) + nl * nul + betab) *
             (1.0 + 0x1p-16) +
         0x1p-40 * (B + nx * nu) + 0x1p-120;
}

// An empty use that pins a fold's result where it is written (the compiler would otherwise
// sink the fold below later tiles' MFMAs, keeping every tile's accumulators live).
__device__ __forceinline__ void pin(const f16v& a, const f16v& b) {
#pragma unroll
  for (int r = 0; r < 16; ++r) asm volatile("" ::"v"(a[r]), "v"(b[r]));
}

// The bound for the rows that can reach a score s (the certificate of the plain and
// H-weighted codes): only rows with n_j <= R do (s_j <= ||z|| n_j - n_j^2 / 2 in the metric of
// H, z = x L), and every term of a row's bound grows with n_j, so the per-row ratios times R
// (or R^2) bound it; the preparation collects the terms into E(R) = R (c_rr R + c_x ||x|| +
// c_d ||x - x'|| + c_l ||lo||).

// Largest change of a slot value by its packed low bits.
__device__ __forceinline__ double pack_slack(float a) { return fabs((double)a) * 0x1p-18 + 0x1p-140; }

// Exchange the lane pair's slot maxima (block hh's 32 slots end in lane (col, hh)), pack the
// slot number into the low 5 bits and return the largest two values.
__device__ __forceinline__ void top2_slots(const f16v& m0, const f16v& m1, float& a0, float& a1) {
  float v[32];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(m0[r]), __float_as_uint(m1[r]),
                                                     false, false);
    v[r] = __uint_as_float((pr[0] & 0xFFFFFFE0u) | (unsigned)r);            // rows of half 0
    v[16 + r] = __uint_as_float((pr[1] & 0xFFFFFFE0u) | (unsigned)(16 + r));  // half 1
  }
  float b0 = -INFINITY, b1 = -INFINITY;
#pragma unroll
  for (int i = 0; i < 32; i += 2) {
    const float md = __builtin_amdgcn_fmed3f(b0, v[i], v[i + 1]);
    b0 = fmax3(b0, v[i], v[i + 1]);
    b1 = __builtin_elementwise_maximum(b1, md);
  }
  a0 = b0;
  a1 = b1;
}

// Row (within a tile) of slot i: accumulator register r = i & 15 of lane half i >> 4.
__device__ __forceinline__ int slot_row(unsigned i) {
  return 8 * ((i & 15u) >> 2) + 4 * (i >> 4) + (i & 3u);
}

// Wave-wide argmax of (s, j): larger s, then smaller j; lanes with j < 0 hold nothing.
__device__ __forceinline__ void wave_argmax(double& s, int& j) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const double so = __shfl_xor(s, o);
    const int jo = __shfl_xor(j, o);
    if (jo >= 0 && (j < 0 || so > s || (so == s && jo < j))) {
      s = so;
      j = jo;
    }
  }
}

// ||x - c||^2 summed in the definition's order, without fused multiply-adds.
template <int SUB>
__device__ __forceinline__ double sq_dist(const double (&x)[SUB], const double* c) {
#pragma clang fp contract(off)
  double s = 0.0;
#pragma unroll
  for (int e = 0; e < SUB; ++e) {
    const double df = x[e] - c[e];
    s += df * df;
  }
  return s;
}

// The blended score of one row in fp64: beta (-e_j / max e) + (1 - beta) cos(q, c_j), the
// divisions replaced by the reciprocals iem = 1 / max e, iqn = 1 / ||q||, icn = 1 / ||c_j||;
// zero norms and a zero maximum error as the definition has them.
template <int SUB>
__device__ __forceinline__ double blend_score(const double (&x)[SUB], const double (&q)[SUB],
                                              const double* c, double icn, double iem, double qn,
                                              double iqn, double beta) {
#pragma clang fp contract(off)
  double e2 = 0.0, dot = 0.0;
#pragma unroll
  for (int e = 0; e < SUB; ++e) {
    const double df = x[e] - c[e];
    e2 += df * df;
    dot += q[e] * c[e];
  }
  const double cosv = (qn > 0.0 && icn > 0.0) ? dot * (iqn * icn) : 0.0;
  const double err = iem > 0.0 ? e2 * iem : 0.0;
  return beta * (-err) + (1.0 - beta) * cosv;
}

// The blend.  Each wave iteration: pass 1 (the smallest s_j, folded and certified like the
// codes, for max e), pass 2 (the blended fp32 scores folded), the winning slot rescored by the
// blend's formula in fp64, the certificate, the rare fp64 scans and the stores.  The table
// operands are read from LDS at each tile.
template <int DT, int SUB>
__global__ __launch_bounds__(kPqThreads, kPqWgPerCu) void pq_encode_blend(
    const void* __restrict__ x, int64_t n, const int32_t* __restrict__ idx, int64_t n_sel,
    int64_t heads, const float* __restrict__ cb, int k, const void* __restrict__ query,
    int64_t nq, double beta, uint8_t* __restrict__ codes) {
  constexpr int M = kD / SUB;   // sub-spaces per row
  constexpr int RPI = 64 / M;   // rows per wave iteration
  __shared__ PqShared<SUB, true> sh;
  const int lane = threadIdx.x & 63, col = lane & 31, hh = lane >> 5;

  // this lane's column in each block: row offset within the iteration and sub-space
  int lr[2], ss[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    lr[b] = (32 * b + col) / M;
    ss[b] = (32 * b + col) % M;
  }
  const int lr_own = lane / M, ss_own = lane % M;  // the sub-vector this lane decides

  // Iterations: (head, group of RPI selected rows), wave-uniform (scalar registers); a wave
  // takes every stride-th one, advanced without a division per step.
  const int64_t G = (n_sel + RPI - 1) / RPI;
  const int64_t stride = (int64_t)gridDim.x * kPqWaves;
  const int64_t st_h = stride / G, st_g = stride % G;
  const int64_t it0 = (int64_t)blockIdx.x * kPqWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int64_t h_cur = it0 / G, g_cur = it0 % G;
  auto advance = [&](int64_t& h, int64_t& g) {
    h += st_h;
    g += st_g;
    if (g >= G) {
      g -= G;
      ++h;
    }
  };
  // the row of this lane's column in block row l_r of iteration (h, g); false when none
  auto locate = [&](int64_t h, int64_t g, int l_r, int64_t& row) {
    const int64_t sel = g * RPI + l_r;
    row = -1;
    if (h < heads && sel < n_sel) row = idx ? (int64_t)idx[h * n_sel + sel] : sel;
    return row >= 0 && row < n;
  };

  Raw<DT, SUB> nx_raw[2], nq_raw[2];
  auto fetch = [&](int64_t h, int64_t g, Raw<DT, SUB> (&xr)[2], Raw<DT, SUB> (&qr)[2]) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      int64_t row = 0;
      const bool ok = locate(h, g, lr[b], row);
      xr[b] = load_raw<DT, SUB>(x, ((h * n + row) * kD + ss[b] * SUB), ok);
      qr[b] = load_raw<DT, SUB>(query, ((h * nq + (nq == 1 ? 0 : row)) * kD + ss[b] * SUB), ok);
    }
  };
  fetch(h_cur, g_cur, nx_raw, nq_raw);  // in flight during the preparation

  const PqConsts pc = pq_prep<SUB, kBlend, DT>(cb, k, nullptr, sh);
  // (lds_lane: the lane index plus an opaque zero set in each iteration, so that the
  // loop-invariant table reads are not hoisted out of the loop into registers)
  int lds_lane = lane;
  auto a_op = [&](int tt) { return sh.fa[tt][lds_lane]; };
  auto fb_op = [&](int tt, int w) { return sh.fb[tt][lds_lane][w]; };
  const unsigned e2 = pk16(ldexpf(1.f, pc.eb), ldexpf(1.f, pc.eb));
  const unsigned mk = pk16(32768.f, 0.f);
  const half8 Bb = hh ? h8(0u, 0u, 0u, 0u) : h8(e2, mk, 0u, 0u);  // bias operand, sub_dim 8
  const f16v zero = {};


  for (; h_cur < heads; advance(h_cur, g_cur)) {
    {
      int z = 0;
      asm volatile("" : "+v"(z));
      lds_lane = lane + z;
    }
    const Raw<DT, SUB> xr[2] = {nx_raw[0], nx_raw[1]};
    const Raw<DT, SUB> qr[2] = {nq_raw[0], nq_raw[1]};
    {
      int64_t h_nx = h_cur, g_nx = g_cur;
      advance(h_nx, g_nx);
      fetch(h_nx, g_nx, nx_raw, nq_raw);  // the next iteration's inputs stay in flight
    }

    int64_t orow;
    const int64_t ohead = h_cur;
    const bool own_ok = locate(h_cur, g_cur, lr_own, orow);
    const Raw<DT, SUB> xo = raw_sel<DT, SUB>(xr[0], xr[1], hh);

    half8 B1[2], B2[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) make_b<DT, SUB>(xr[b], hh, e2, mk, B1[b], B2[b]);

    // scores of tile tt for both blocks (S units, bias included)
    auto tile_scores = [&](int tt, const half8 (&b1)[2], const half8 (&b2)[2], unsigned mark_flip,
                           f16v& s0, f16v& s1) {
      const half8 at0 = a_op(tt);
      if constexpr (SUB == 8) {
        const f16v cbias = __builtin_amdgcn_mfma_f32_32x32x16_f16(
            h8(fb_op(tt, 0), fb_op(tt, 1) ^ (hh ? 0u : mark_flip), 0u, 0u), Bb, zero, 0, 0, 0);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(at0, b1[0], cbias, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(at0, b1[1], cbias, 0, 0, 0);
        if constexpr (DT == A2ATS_F32) {
          s0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(at0, b2[0], s0, 0, 0, 0);
          s1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(at0, b2[1], s1, 0, 0, 0);
        }
      } else {
        u4v a = __builtin_bit_cast(u4v, at0);
        a[1] ^= hh ? mark_flip : 0u;  // the pad mark: lanes 32-63, low half of dword 1
        const half8 at = __builtin_bit_cast(half8, a);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(at, b1[0], zero, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(at, b1[1], zero, 0, 0, 0);
      }
    };

    int code = 0;
    bool open = false;
    // this lane's sub-vector, exact, and the bound E on its MFMA scores' error (formed after
    // the fold, which needs the registers)
    double xs[SUB], nx, E, xnd, xnl;
    auto finals = [&]() {
      Raw<DT, SUB> xw = xo;
#pragma unroll
      for (int i = 0; i < Raw<DT, SUB>::W; ++i) asm volatile("" : "+v"(xw.w[i]));
      float xf[SUB];
      raw_floats<DT, SUB>(xw, xf);
#pragma unroll
      for (int e = 0; e < SUB; ++e) xs[e] = xf[e];
      float fx, fd, fl;
      norms<DT, SUB>(xw, fx, fd, fl);
      nx = fx;
      xnd = fd;
      xnl = fl;
      E = score_bound<DT, SUB>(nx, xnd, xnl, pc.rho, pc.nu, pc.nul, pc.B, pc.betab);
    };
    // all of a broadcast sub-vector finite (a non-finite one has code 0: every distance is
    // inf or NaN)
    auto all_finite = [](const double (&v)[SUB]) {
      bool f = true;
#pragma unroll
      for (int e = 0; e < SUB; ++e) f = f && (v[e] - v[e] == 0.0);
      return f;
    };

    // ---- pass 1: max_j e_j through the smallest s_j (pad rows' mark flipped to +)
    const unsigned flip = 0x8000u;  // sign of the pad mark's fp16
    f16v m0, m1;
#pragma unroll
    for (int tp = 0; tp < kPqTiles / 2; ++tp) {
      f16v a0, a1, c0, c1;
      tile_scores(2 * tp, B1, B2, flip, a0, a1);
      tile_scores(2 * tp + 1, B1, B2, flip, c0, c1);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        m0[r] = tp ? fmax3(m0[r], -a0[r], -c0[r]) : __builtin_elementwise_maximum(-a0[r], -c0[r]);
        m1[r] = tp ? fmax3(m1[r], -a1[r], -c1[r]) : __builtin_elementwise_maximum(-a1[r], -c1[r]);
      }
      pin(m0, m1);
      __builtin_amdgcn_sched_barrier(0);
    }
    double emax;
    {
      float t0, t1;
      top2_slots(m0, m1, t0, t1);
      finals();
      double nx2 = 0.0;
#pragma unroll
      for (int e = 0; e < SUB; ++e) nx2 = fma(xs[e], xs[e], nx2);
      const int row = slot_row(__float_as_uint(t0) & 31u);
      double em = -INFINITY;
      int je = -1;
#pragma unroll 2
      for (int tt = 0; tt < kPqTiles; ++tt) {
        const int j = 32 * tt + row;
        if (j < k) {
          const double e2v = sq_dist<SUB>(xs, sh.v64[j]);
          if (e2v > em) {
            em = e2v;
            je = j;
          }
        }
      }
      const double tb = 2.0 * ldexp((double)t1 + pack_slack(t1) + E, -pc.se);
      const double ub = nx2 + tb;
      const double margin = 0x1p-44 * (nx2 + fabs(tb) + fabs(em));
      emax = em;
      bool open1 = own_ok && !(pc.finite && je >= 0 && em - margin > ub);
      unsigned long long todo = __ballot(open1);
      while (todo) {
        const int src = __ffsll((long long)todo) - 1;
        todo &= todo - 1;
        double xb[SUB];
#pragma unroll
        for (int e = 0; e < SUB; ++e) xb[e] = __shfl(xs[e], src);
        double mx = -INFINITY;
        for (int j = lane; j < k; j += 64) mx = fmax(mx, sq_dist<SUB>(xb, sh.v64[j]));
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o));
        if (lane == src) emax = mx;
      }
    }
    // ---- pass 2: the blend, up to the constant beta ||x||^2 / max e
    const Raw<DT, SUB> qo = raw_sel<DT, SUB>(qr[0], qr[1], hh);
    double qn;
    {
      float qf[SUB];
      raw_floats<DT, SUB>(qo, qf);
      double qn2 = 0.0;
#pragma unroll
      for (int e = 0; e < SUB; ++e) qn2 += (double)qf[e] * (double)qf[e];
      qn = sqrt(qn2);
    }
    const double iqn = qn > 0.0 ? 1.0 / qn : 0.0;
    const double iem = emax > 0.0 ? 1.0 / emax : 0.0;
    const float al_own = (float)(2.0 * beta * ldexp(iem, -pc.se));
    const float ga_own = (float)((1.0 - beta) * ldexp(iqn, -pc.sq));
    float al[2], ga[2];
    {
      const float alp = __shfl_xor(al_own, 32), gap = __shfl_xor(ga_own, 32);
      al[0] = hh ? alp : al_own;
      al[1] = hh ? al_own : alp;
      ga[0] = hh ? gap : ga_own;
      ga[1] = hh ? ga_own : gap;
    }
    half8 Q1[2], Q2[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) make_b<DT, SUB>(qr[b], hh, 0u, 0u, Q1[b], Q2[b]);
    // the blended fold value of tile tt, one block's q-accumulator at a time
    auto blended = [&](int tt, f16v& s0, f16v& s1) {
      tile_scores(tt, B1, B2, 0u, s0, s1);
      const half8 fq = sh.fq[tt][lds_lane];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        f16v q = __builtin_amdgcn_mfma_f32_32x32x16_f16(fq, Q1[b], zero, 0, 0, 0);
        if constexpr (SUB == 8 && DT == A2ATS_F32)
          q = __builtin_amdgcn_mfma_f32_32x32x16_f16(fq, Q2[b], q, 0, 0, 0);
        f16v& sb = b ? s1 : s0;
#pragma unroll
        for (int r = 0; r < 16; ++r) sb[r] = __fmaf_rn(al[b], sb[r], ga[b] * q[r]);
      }
    };
#pragma unroll
    for (int tt = 0; tt < kPqTiles; ++tt) {
      f16v a0, a1;
      blended(tt, a0, a1);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        m0[r] = tt ? __builtin_elementwise_maximum(m0[r], a0[r]) : a0[r];
        m1[r] = tt ? __builtin_elementwise_maximum(m1[r], a1[r]) : a1[r];
      }
      pin(m0, m1);
      __builtin_amdgcn_sched_barrier(0);  // one tile's accumulators live at a time
    }
    finals();  // x and its bound again (not kept across the fold)
    double qs[SUB];
    {
      float qf[SUB];
      raw_floats<DT, SUB>(qo, qf);
#pragma unroll
      for (int e = 0; e < SUB; ++e) qs[e] = qf[e];
    }
    float t0, t1;
    top2_slots(m0, m1, t0, t1);
    const int row = slot_row(__float_as_uint(t0) & 31u);
    double sa = -INFINITY;
    int ja = -1;
#pragma unroll 2
    for (int tt = 0; tt < kPqTiles; ++tt) {
      const int j = 32 * tt + row;
      if (j < k) {
        const double sc = blend_score<SUB>(xs, qs, sh.v64[j], sh.v64[j][SUB + 1], iem, qn, iqn, beta);
        if (sc > sa) {
          sa = sc;
          ja = j;
        }
      }
    }
    // the fp32 fold value of row j approximates score_j + K0; its error bound
    double nx2 = 0.0;
#pragma unroll
    for (int e = 0; e < SUB; ++e) nx2 = fma(xs[e], xs[e], nx2);
    const double K0 = beta * nx2 * iem;
    const double Ms = nx * pc.Mv + pc.Shb;
    const double Mq = ldexp(qn, pc.sq) * (1.0 + 0x1p-40);
    float qnf, qd, ql;
    norms<DT, SUB>(qo, qnf, qd, ql);
    const double Eq = score_bound<DT, SUB>(qnf, qd, ql, pc.rhoq, pc.nuq, pc.nulq, 0.0, 0.0) +
                      0x1p-40 * Mq;
    const double aa = fabs((double)al_own), gg = fabs((double)ga_own);
    const double E2 = (aa * (E * (1.0 + kRnd) + 3.0 * kRnd * Ms) +
                       gg * (Eq * (1.0 + 2.0 * kRnd) + 4.0 * kRnd * Mq)) * (1.0 + 0x1p-16) +
                      0x1p-120;
    const double lhs = sa + K0 - 0x1p-44 * (fabs(sa) + K0 + 1.0);
    const double rhs = (double)t1 + pack_slack(t1) + E2;
    code = ja;
    open = own_ok && !(pc.finite && ja >= 0 && emax > 0.0 && lhs > rhs);
    unsigned long long todo = __ballot(open);
    while (todo) {
      const int src = __ffsll((long long)todo) - 1;
      todo &= todo - 1;
      double xb[SUB], qb[SUB];
#pragma unroll
      for (int e = 0; e < SUB; ++e) {
        xb[e] = __shfl(xs[e], src);
        qb[e] = __shfl(qs[e], src);
      }
      const bool fin = all_finite(xb);
      double mx = -INFINITY;
      for (int j = lane; j < k; j += 64) mx = fmax(mx, sq_dist<SUB>(xb, sh.v64[j]));
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o));
      double qq = 0.0;
#pragma unroll
      for (int e = 0; e < SUB; ++e) qq += qb[e] * qb[e];
      const double qnb = sqrt(qq);
      const double iqb = qnb > 0.0 ? 1.0 / qnb : 0.0;
      const double ieb = mx > 0.0 ? 1.0 / mx : 0.0;
      double bs = -INFINITY;
      int bj = -1;
      for (int j = lane; j < k; j += 64) {
        const double sc = blend_score<SUB>(xb, qb, sh.v64[j], sh.v64[j][SUB + 1], ieb, qnb, iqb, beta);
        if (sc > bs) {
          bs = sc;
          bj = j;
        }
      }
      wave_argmax(bs, bj);
      if (lane == src) code = fin && bj >= 0 ? bj : 0;
    }
    if (own_ok) codes[(ohead * n + orow) * M + ss_own] = (uint8_t)code;
  }
}

// Plain and H-weighted codes.  Each wave iteration: the 8 tiles' MFMAs folded into the slot
// maxima (the table operand read from LDS at each tile pair), then the finalisation in
// parts: the top two slots, the fp64 rescoring of the winning slot, the certificate, the rare
// fp64 scans and the stores.  The inputs are fetched one iteration ahead; bf16 plain codes
// run three workgroups per CU (their registers fit).
template <int DT, int SUB, int MODE>
constexpr int pq_wg_per_cu() {
  return (DT == A2ATS_BF16 && MODE == kPlain) ? 3 : kPqWgPerCu;
}

template <int DT, int SUB, int MODE>
__global__ __launch_bounds__(kPqThreads, (pq_wg_per_cu<DT, SUB, MODE>())) void pq_encode_codes(
    const void* __restrict__ x, int64_t n, const int32_t* __restrict__ idx, int64_t n_sel,
    int64_t heads, const float* __restrict__ cb, int k, const float* __restrict__ chol,
    uint8_t* __restrict__ codes) {
  constexpr int M = kD / SUB;   // sub-spaces per row
  constexpr int RPI = 64 / M;   // rows per wave iteration
  __shared__ PqShared<SUB, false> sh;
  const int lane = threadIdx.x & 63, col = lane & 31, hh = lane >> 5;
  int lr[2], ss[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    lr[b] = (32 * b + col) / M;
    ss[b] = (32 * b + col) % M;
  }
  const int lr_own = lane / M, ss_own = lane % M;  // the sub-vector this lane decides

  // iterations (head, group of RPI selected rows), wave-uniform, every stride-th one
  const int64_t G = (n_sel + RPI - 1) / RPI;
  const int64_t stride = (int64_t)gridDim.x * kPqWaves;
  const int64_t st_h = stride / G, st_g = stride % G;
  const int64_t it0 = (int64_t)blockIdx.x * kPqWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int64_t h_cur = it0 / G, g_cur = it0 % G;
  auto advance = [&](int64_t& h, int64_t& g) {
    h += st_h;
    g += st_g;
    if (g >= G) {
      g -= G;
      ++h;
    }
  };
  auto locate = [&](int64_t h, int64_t g, int l_r, int64_t& row) {
    const int64_t sel = g * RPI + l_r;
    row = -1;
    if (h < heads && sel < n_sel) row = idx ? (int64_t)idx[h * n_sel + sel] : sel;
    return row >= 0 && row < n;
  };
  Raw<DT, SUB> nx_raw[2];
  auto fetch = [&](int64_t h, int64_t g, Raw<DT, SUB> (&dst)[2]) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      int64_t row = 0;
      const bool ok = locate(h, g, lr[b], row);
      dst[b] = load_raw<DT, SUB>(x, ((h * n + row) * kD + ss[b] * SUB), ok);
    }
  };
  int64_t h_nx = h_cur, g_nx = g_cur;  // the iteration after the current one
  advance(h_nx, g_nx);
  fetch(h_cur, g_cur, nx_raw);  // in flight during the preparation

  const PqConsts pc = pq_prep<SUB, MODE, DT>(cb, k, chol, sh);
  if (h_cur >= heads) return;  // no iteration for this wave (the preparation's barriers are past)

  const unsigned e2 = pk16(ldexpf(1.f, pc.eb), ldexpf(1.f, pc.eb));
  const unsigned mk = pk16(32768.f, 0.f);
  const half8 Bb = hh ? h8(0u, 0u, 0u, 0u) : h8(e2, mk, 0u, 0u);  // bias operand, sub_dim 8
  const f16v zero = {};
  int lds_lane = lane, lds_zero = 0;

  // The table operand of a tile pair, read from LDS.
  struct PairOps {
    half8 a[2];
    half8 bb[2];
  };
  auto load_ops = [&](int tp) {
    PairOps o;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      o.a[q] = sh.fa[2 * tp + q][lds_lane];
      if constexpr (SUB == 8) {
        o.bb[q] = *reinterpret_cast<const half8*>(&sh.fb[2 * tp + q][lds_lane][0]);
      }
    }
    return o;
  };
  // scores of tile tt for both blocks (S units, bias included)
  auto tile_scores = [&](const PairOps& o, int q, const half8 (&b1)[2], const half8 (&b2)[2],
                         f16v& s0, f16v& s1) {
    const half8 at = o.a[q];
    if constexpr (SUB == 8) {
      const f16v cbias = __builtin_amdgcn_mfma_f32_32x32x16_f16(o.bb[q], Bb, zero, 0, 0, 0);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(at, b1[0], cbias, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(at, b1[1], cbias, 0, 0, 0);
      if constexpr (DT == A2ATS_F32) {
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(at, b2[0], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(at, b2[1], s1, 0, 0, 0);
      }
    } else {
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(at, b1[0], zero, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(at, b1[1], zero, 0, 0, 0);
    }
  };
  // tile pair tp of one iteration folded into the slot maxima (n0, n1)
  auto fold_pair = [&](int tp, const PairOps& o, const half8 (&b1)[2], const half8 (&b2)[2],
                       f16v& n0, f16v& n1) {
    f16v a0, a1, c0, c1;
    tile_scores(o, 0, b1, b2, a0, a1);
    tile_scores(o, 1, b1, b2, c0, c1);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      n0[r] = tp ? fmax3(n0[r], a0[r], c0[r]) : __builtin_elementwise_maximum(a0[r], c0[r]);
      n1[r] = tp ? fmax3(n1[r], a1[r], c1[r]) : __builtin_elementwise_maximum(a1[r], c1[r]);
    }
    pin(n0, n1);
  };

  // ---- an iteration's state and its finalisation, in parts
  f16v m0, m1;          // its slot maxima
  Raw<DT, SUB> xo_p;    // this lane's sub-vector of it
  int64_t orow_p = -1, ohead_p = 0;
  bool ok_p = false;
  float t0, t1;         // its top two slot values (packed)
  int row;              // the winning slot's row within a tile
  double xs[SUB];       // the sub-vector, exact
  double sa = 0.0;      // the best packed fp64 score of the winning slot
  float fx, fd, fl;     // ||x||, ||x - x'||, ||lo||
  int code = 0;
  bool open = false;
  auto fin_a = [&]() {
    top2_slots(m0, m1, t0, t1);
    row = slot_row(__float_as_uint(t0) & 31u);
    asm volatile("" ::"v"(t1), "v"(row));
  };
  // rows tt0 .. tt0 + 3 of the winning slot in fp64 (a pad row scores about -2^1000); each
  // score carries its tile in its lowest 3 bits, ordered so that the larger packed value is
  // the lower tile between equal scores, and the best is a plain maximum
  auto fin_rows = [&](int tt0) {
#pragma unroll
    for (int tt = tt0; tt < tt0 + 4; ++tt) {
      const int j = 32 * tt + row;
      double s = -sh.v64[j][SUB];
#pragma unroll
      for (int e = 0; e < SUB; ++e) s = fma(xs[e], sh.v64[j][e], s);
      const int hi = __double2hiint(s);
      const unsigned c3 = (unsigned)(7 - tt) ^ ((unsigned)(hi >> 31) & 7u);
      s = __hiloint2double(hi, (int)(((unsigned)__double2loint(s) & ~7u) | c3));
      sa = tt ? max_f64(sa, s) : s;
    }
    asm volatile("" ::"v"(sa));
  };
  auto fin_b = [&]() {
    float xf[SUB];
    raw_floats<DT, SUB>(xo_p, xf);
#pragma unroll
    for (int e = 0; e < SUB; ++e) xs[e] = xf[e];
    fin_rows(0);
  };
  auto fin_c = [&]() {
    fin_rows(4);
    norms<DT, SUB>(xo_p, fx, fd, fl);
    asm volatile("" ::"v"(fx), "v"(fd), "v"(fl));
  };
  auto fin_d = [&]() {
    const int hia = __double2hiint(sa);
    const int tta = 7 - (int)(((unsigned)__double2loint(sa) & 7u) ^ ((unsigned)(hia >> 31) & 7u));
    const int ja = sa > -0x1p999 ? 32 * tta + row : -1;
    // every row outside the winning slot: its MFMA score is at most t1 (plus the packing), its
    // error, when it could reach s_a at all, at most the bound for rows of size R
    const double nx = fx;
    double Z = nx;  // ||z|| (z = x L; x itself without L), rounded up
    if constexpr (MODE == kHWeighted) {
      // z in fp32: each element within 2^-21 sum_b |x_b L_ba|, so ||z|| within
      // 2^-21 ||x|| ||L||_F of the fp32 vector's norm
      float xf[SUB];
      raw_floats<DT, SUB>(xo_p, xf);
      float z2 = 0.f;
#pragma unroll
      for (int a = 0; a < SUB; ++a) {
        float za = 0.f;
#pragma unroll
        for (int b = 0; b < SUB; ++b) za = __fmaf_rn(xf[b], sh.l32[b][a + lds_zero], za);
        z2 = __fmaf_rn(za, za, z2);
      }
      Z = (double)sqrt_up(z2) + 0x1p-21 * nx * pc.lf;
    }
    const float disc = (float)fmax(0.0, Z * Z - 2.0 * sa) * (1.f + 0x1p-18f);
    const double R = (Z + (double)sqrt_up(disc)) * (1.0 + 0x1p-20) + 0x1p-60;
    const double Ec = R * (pc.c_rr * R + pc.c_x * nx + pc.c_d * (double)fd + pc.c_l * (double)fl) + 0x1p-120;
    const double lhs = ldexp(sa, pc.se) * (1.0 - 0x1p-47 * (sa < 0.0 ? -1.0 : 1.0));  // the packed bits
    const double rhs = (double)t1 + pack_slack(t1) + Ec;
    code = ja;
    open = ok_p && !(pc.finite && ja >= 0 && lhs > rhs);
    asm volatile("" ::"v"(code), "v"(open ? 1 : 0));
  };
  // the rest (rare): the whole wave scores the whole table in fp64 for one sub-vector at a
  // time; then the codes are stored
  auto fin_tail = [&]() {
    unsigned long long todo = __ballot(open);
    while (todo) {
      const int src = __ffsll((long long)todo) - 1;
      todo &= todo - 1;
      double xb[SUB];
      bool fin = true;
#pragma unroll
      for (int e = 0; e < SUB; ++e) {
        xb[e] = __shfl(xs[e], src);
        fin = fin && (xb[e] - xb[e] == 0.0);
      }
      double bs = -INFINITY;
      int bj = -1;
      for (int j = lane; j < k; j += 64) {
        double s = -sh.v64[j][SUB];
#pragma unroll
        for (int e = 0; e < SUB; ++e) s = fma(xb[e], sh.v64[j][e], s);
        if (s > bs) {  // a NaN score (a non-finite table row) never wins
          bs = s;
          bj = j;
        }
      }
      wave_argmax(bs, bj);
      // a non-finite input: every distance is inf or NaN, code 0
      if (lane == src) code = fin && bj >= 0 ? bj : 0;
    }
    if (ok_p) codes[(ohead_p * n + orow_p) * M + ss_own] = (uint8_t)code;
  };

  // ---- each iteration: the fold of all tiles, then the finalisation
  for (;;) {
    {
      int z = 0;
      asm volatile("" : "+v"(z));
      lds_zero = z;
      lds_lane = lane + z;
    }
    const Raw<DT, SUB> xr[2] = {nx_raw[0], nx_raw[1]};
    half8 B1[2], B2[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) make_b<DT, SUB>(xr[b], hh, e2, mk, B1[b], B2[b]);
    xo_p = raw_sel<DT, SUB>(xr[0], xr[1], hh);
    fetch(h_nx, g_nx, nx_raw);  // the next iteration's inputs stay in flight through this one
#pragma unroll
    for (int tp = 0; tp < kPqTiles / 2; ++tp) {
      fold_pair(tp, load_ops(tp), B1, B2, m0, m1);
      __builtin_amdgcn_sched_barrier(0);  // one tile pair's accumulators live at a time
    }
    ohead_p = h_cur;
    ok_p = locate(h_cur, g_cur, lr_own, orow_p);
    fin_a();
    fin_b();
    fin_c();
    fin_d();
    fin_tail();
    h_cur = h_nx;
    g_cur = g_nx;
    advance(h_nx, g_nx);
    if (h_cur >= heads) break;
  }
}

template <int DT, int SUB>
int launch_pq(int mode, const void* x, int64_t n, const int32_t* idx, int64_t n_sel,
              int64_t heads, const float* cb, int k, const float* chol, const void* query,
              int64_t nq, double beta, uint8_t* codes, hipStream_t s) {
  const int64_t rpi = 64 / (kD / SUB);
  const int64_t waves = heads * ((n_sel + rpi - 1) / rpi);  // one wave iteration each
  int64_t g = (waves + kPqWaves - 1) / kPqWaves;
  const int per_cu = mode == kPlain ? pq_wg_per_cu<DT, SUB, kPlain>()
                                    : (mode == kHWeighted ? pq_wg_per_cu<DT, SUB, kHWeighted>()
                                                          : kPqWgPerCu);
  if (g > (int64_t)kPqCus * per_cu) g = (int64_t)kPqCus * per_cu;
  const dim3 grid((unsigned)g), block(kPqThreads);
  if (mode == kHWeighted)
    return launch("pq_encode_h", pq_encode_codes<DT, SUB, kHWeighted>, grid, block, 0, s, x, n,
                  idx, n_sel, heads, cb, k, chol, codes);
  if (mode == kBlend)
    return launch("pq_encode_blend", pq_encode_blend<DT, SUB>, grid, block, 0, s, x, n, idx,
                  n_sel, heads, cb, k, query, nq, beta, codes);
  return launch("pq_encode_plain", pq_encode_codes<DT, SUB, kPlain>, grid, block, 0, s, x, n, idx,
                n_sel, heads, cb, k, chol, codes);
}

template <int DT>
int dispatch_sub(int64_t sub, int mode, const void* x, int64_t n, const int32_t* idx,
                 int64_t n_sel, int64_t heads, const float* cb, int k, const float* chol,
                 const void* query, int64_t nq, double beta, uint8_t* codes, hipStream_t s) {
  if (sub == 4)
    return launch_pq<DT, 4>(mode, x, n, idx, n_sel, heads, cb, k, chol, query, nq, beta, codes, s);
  return launch_pq<DT, 8>(mode, x, n, idx, n_sel, heads, cb, k, chol, query, nq, beta, codes, s);
}

}  // namespace
}  // namespace a2ats

using namespace a2ats;

extern "C" int a2ats_pq_encode(const void* x, int x_dtype, int64_t heads, int64_t n, int64_t d,
                               int64_t sub_dim, const int32_t* idx, int64_t n_idx,
                               const float* codebook, int64_t k, const float* chol,
                               const void* query, int64_t nq, double beta, uint8_t* codes,
                               void* stream) {
  if (x_dtype != A2ATS_F32 && x_dtype != A2ATS_BF16) return A2ATS_EDTYPE;
  if (d != kD || heads < 1 || n < 0) return A2ATS_EINVAL;
  if (sub_dim != 4 && sub_dim != 8) return A2ATS_EINVAL;  // the pages' table rows
  if (k < 1 || k > kPqMaxK) return A2ATS_EINVAL;
  const int64_t n_sel = idx ? n_idx : n;
  if (n_sel < 0 || n > 0x7FFFFFFF) return A2ATS_EINVAL;
  int mode = kPlain;
  if (chol) {
    mode = kHWeighted;
  } else if (query) {
    mode = kBlend;
    if (!(beta >= 0.0 && beta <= 1.0)) return A2ATS_EINVAL;
    if (!(nq == 1 || nq == n)) return A2ATS_EINVAL;
  }
  if (n == 0 || n_sel == 0) return A2ATS_OK;
  if (!x || !codebook || !codes) return A2ATS_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (x_dtype == A2ATS_BF16)
    return dispatch_sub<A2ATS_BF16>(sub_dim, mode, x, n, idx, n_sel, heads, codebook, (int)k, chol,
                                    query, nq, beta, codes, s);
  return dispatch_sub<A2ATS_F32>(sub_dim, mode, x, n, idx, n_sel, heads, codebook, (int)k, chol,
                                 query, nq, beta, codes, s);
}

// The compression the settings alone decide ("A2ATS-adapted" docs, "What you get with the
// defaults"): bits / sub_dim bits per number, 16 / that against fp16, and a table of
// 2^bits x sub_dim entries stored as fp16.  The stored-bytes figures count packed codes
// (bits per sub-vector), as the docs' byte accounting does; this library stores one byte
// per code.
extern "C" int a2ats_pq_accounting(int64_t tokens, int64_t heads, int64_t d, int64_t sub_dim,
                                   int bits, double* bits_per_number, double* ratio_vs_fp16,
                                   int64_t* table_bytes, int64_t* compressed_bytes,
                                   int64_t* fp16_bytes) {
  if (tokens < 0 || heads < 1 || d < 1 || sub_dim < 1 || d % sub_dim != 0 || bits < 1 ||
      bits > 16)
    return A2ATS_EINVAL;
  const double bpn = (double)bits / (double)sub_dim;
  if (bits_per_number) *bits_per_number = bpn;
  if (ratio_vs_fp16) *ratio_vs_fp16 = 16.0 / bpn;
  if (table_bytes) *table_bytes = ((int64_t)1 << bits) * sub_dim * 2;
  if (compressed_bytes) *compressed_bytes = (tokens * heads * (d / sub_dim) * bits + 7) / 8;
  if (fp16_bytes) *fp16_bytes = tokens * heads * d * 2;
  return A2ATS_OK;
}
