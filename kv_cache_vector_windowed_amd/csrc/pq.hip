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
// Kernel pq_encode: one thread per (row, group of four consecutive sub-spaces), groups of a
// row on consecutive lanes (coalesced loads of whole rows); the four sub-vectors share every
// centroid read from LDS.  Each workgroup first stages the transformed codebook in LDS: w_j = c_j L and b_j = ||w_j||^2 in fp64 (w_j = c_j without L), plus fp32
// copies and, per centroid, the terms of its error bound.  A thread forms z = x_s L in fp64
// and scans the K scores s_j = z . w_j - b_j / 2 in fp32.  Each fp32 score is within
// E_j = c (||z|| ||w_j|| + b_j) of the exact one (c = 18 u, u = 2^-24: the roundings of z, w
// and b to fp32 and the (sub_dim + 1)-term fp32 sum, with room to spare), so the thread
// keeps the two largest t_j = s_j + E_j and the winner a is certain when s_a - E_a exceeds
// the other t; otherwise it rescans the K scores in fp64 (about 3 in 10^5 sub-vectors on
// the workloads; a single codebook-wide bound sent 2% there).  The blend is evaluated in
// fp64 throughout (two passes: max e, then the blended argmax, with the per-centroid and
// per-row reciprocals taken once), as the whole-vector blend is.
#include "common.hpp"

namespace a2ats {
namespace {

constexpr int kD = A2ATS_HEAD_DIM;
constexpr int kPqThreads = 256;
constexpr int kPqMaxK = 256;
// fp32 score bound factor (sub_dim + 10) u, u = 2^-24: the roundings of z and w to fp32
// (2u ||z|| ||w||), the (sub_dim + 1)-term fp32 sum ((sub_dim + 1) u of the magnitudes),
// b_j's rounding (u b_j) and the rounding of t_j itself (u |t_j|), with room to spare
constexpr double kBoundC = 18.0 * 0x1p-24;
constexpr int kPqRows = 4;  // sub-vectors per thread: each LDS centroid read serves four

enum PqMode { kPlain = 0, kHWeighted = 1, kBlend = 2 };

// x rounded to fp32 towards +infinity.
__device__ __forceinline__ float round_up_f(double x) {
  float f = (float)x;
  if ((double)f < x) f = __uint_as_float(__float_as_uint(f) + (f >= 0.f ? 1u : 0xFFFFFFFFu));
  return f;
}

__device__ __forceinline__ bool better(double s, int j, double bs, int bj) {
  return s > bs || (s == bs && j < bj);
}

template <int DT, int MODE, int SUB, int R>
__global__ __launch_bounds__(kPqThreads) void pq_encode(
    const void* __restrict__ x, int64_t n, const int32_t* __restrict__ idx, int64_t n_sel,
    int64_t heads, const float* __restrict__ cb, int k, const float* __restrict__ chol,
    const void* __restrict__ query, int64_t nq, double beta, uint8_t* __restrict__ codes) {
  constexpr int M = kD / SUB;  // sub-spaces per row
  __shared__ double w64[kPqMaxK][SUB];
  __shared__ float w32[kPqMaxK][SUB];
  __shared__ double b64[kPqMaxK];
  __shared__ float b32[kPqMaxK];
  __shared__ float wn32[kPqMaxK];   // ||w_j|| rounded up (bound term)
  __shared__ float eb32[kPqMaxK];   // c b_j rounded up (bound term)
  __shared__ double icn[kPqMaxK];   // 1 / ||c_j|| (0 for a zero centroid; blend)
  __shared__ double lsh[SUB][SUB];
  const int t = threadIdx.x;
  // ---- the transformed codebook (or, for the blend, the codebook and its norms)
  if (MODE == kHWeighted && t < SUB * SUB) lsh[t / SUB][t % SUB] = (double)chol[t];
  __syncthreads();
  for (int j = t; j < k; j += kPqThreads) {
    double c[SUB];
#pragma unroll
    for (int e = 0; e < SUB; ++e) c[e] = (double)cb[(int64_t)j * SUB + e];
    double w[SUB];
#pragma unroll
    for (int e = 0; e < SUB; ++e) {
      if (MODE == kHWeighted) {
        double s = 0.0;
#pragma unroll
        for (int a = 0; a < SUB; ++a) s += c[a] * lsh[a][e];  // (c L)_e
        w[e] = s;
      } else {
        w[e] = c[e];
      }
    }
    double b = 0.0;
#pragma unroll
    for (int e = 0; e < SUB; ++e) {
      b += w[e] * w[e];
      w64[j][e] = w[e];
      w32[j][e] = (float)w[e];
    }
    b64[j] = b;  // ||w_j||^2 (for the blend: ||c_j||^2)
    b32[j] = (float)b;
    const double wn = sqrt(b);
    wn32[j] = round_up_f(wn * (1.0 + 0x1p-40));
    eb32[j] = round_up_f(kBoundC * b * (1.0 + 0x1p-40));
    icn[j] = wn > 0.0 ? 1.0 / wn : 0.0;
  }
  __syncthreads();

  // items: (head, selected row, group of R consecutive sub-spaces); every centroid read from
  // LDS serves the thread's R sub-vectors
  constexpr int G = M / R;  // groups per row
  const int64_t items = heads * n_sel * G;
  for (int64_t it = (int64_t)blockIdx.x * kPqThreads + t; it < items;
       it += (int64_t)gridDim.x * kPqThreads) {
    const int grp = (int)(it % G);
    const int64_t hi = it / G;  // head * n_sel + selected row
    const int64_t head = hi / n_sel;
    const int64_t sel = hi % n_sel;
    const int64_t row = idx ? (int64_t)idx[head * n_sel + sel] : sel;
    if (row < 0 || row >= n) continue;  // out-of-range index entries are skipped
    const int64_t xoff = (head * n + row) * kD + (int64_t)grp * R * SUB;
    float xs[R][SUB];  // exact: the inputs are fp32 or bf16
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int e = 0; e < SUB; ++e) xs[r][e] = load_elem(x, DT, xoff + r * SUB + e);
    if (MODE == kBlend) {
      const int64_t qoff = (head * nq + (nq == 1 ? 0 : row)) * kD + (int64_t)grp * R * SUB;
      double qs[R][SUB], qn[R], emax[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        double qn2 = 0.0;
#pragma unroll
        for (int e = 0; e < SUB; ++e) {
          qs[r][e] = (double)load_elem(query, DT, qoff + r * SUB + e);
          qn2 += qs[r][e] * qs[r][e];
        }
        const double qnr = sqrt(qn2);
        qn[r] = qnr > 0.0 ? 1.0 / qnr : 0.0;  // held as 1 / ||q_s|| (0: cosine 0)
        emax[r] = 0.0;
      }
      for (int j = 0; j < k; ++j) {
        double cv[SUB];
#pragma unroll
        for (int a = 0; a < SUB; ++a) cv[a] = w64[j][a];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          double e2 = 0.0;
#pragma unroll
          for (int a = 0; a < SUB; ++a) {
            const double df = (double)xs[r][a] - cv[a];
            e2 += df * df;
          }
          emax[r] = fmax(emax[r], e2);
        }
      }
      double bs[R];
      int bj[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        bs[r] = -INFINITY;
        bj[r] = 0x7FFFFFFF;
        emax[r] = emax[r] > 0.0 ? 1.0 / emax[r] : 0.0;  // held as 1 / max e (0: no error term)
      }
      for (int j = 0; j < k; ++j) {
        double cv[SUB];
#pragma unroll
        for (int a = 0; a < SUB; ++a) cv[a] = w64[j][a];
        const double ic = icn[j];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          double e2 = 0.0, dot = 0.0;
#pragma unroll
          for (int a = 0; a < SUB; ++a) {
            const double df = (double)xs[r][a] - cv[a];
            e2 += df * df;
            dot += qs[r][a] * cv[a];
          }
          // the blend with reciprocals (fp64 throughout; rounding differs from the divided
          // form by a few ulps, far inside any decided margin)
          const double cosv = dot * qn[r] * ic;
          const double err = e2 * emax[r];
          const double sc = beta * (-err) + (1.0 - beta) * cosv;
          if (better(sc, j, bs[r], bj[r])) {
            bs[r] = sc;
            bj[r] = j;
          }
        }
      }
      uint8_t* cp = codes + (head * n + row) * M + grp * R;
#pragma unroll
      for (int r = 0; r < R; ++r) cp[r] = (uint8_t)bj[r];
    } else {
      // z = x_s L in fp64 (x_s itself without L); the fp64 values are formed again for a
      // close call rather than kept, which keeps the register count down
      // (L is read from LDS at each use: an opaque zero offset keeps the compiler from
      // hoisting all SUB x SUB fp64 entries into registers for the whole loop)
      int opq = 0;
      asm volatile("" : "+v"(opq));
      const double* lp = &lsh[0][0] + opq;
      auto z_of = [&](int r, double (&z)[SUB]) {
#pragma unroll
        for (int e = 0; e < SUB; ++e) {
          if (MODE == kHWeighted) {
            double sacc = 0.0;
#pragma unroll
            for (int a = 0; a < SUB; ++a) sacc += (double)xs[r][a] * lp[a * SUB + e];
            z[e] = sacc;
          } else {
            z[e] = (double)xs[r][e];
          }
        }
      };
      double zn[R];
      float zf[R][SUB];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        double z[SUB];
        z_of(r, z);
        double zn2 = 0.0;
#pragma unroll
        for (int e = 0; e < SUB; ++e) {
          zn2 += z[e] * z[e];
          zf[r][e] = (float)z[e];
        }
        zn[r] = sqrt(zn2);
      }
      // t_j = s~_j + E_j with E_j = c (||z|| ||w_j|| + b_j): the best a by t is certain when
      // s~_a - E_a exceeds every other t_j (the second largest t)
      float cz[R], t1[R], t2[R];
      int ja[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        cz[r] = round_up_f(kBoundC * zn[r] * (1.0 + 0x1p-40));
        t1[r] = -INFINITY;
        t2[r] = -INFINITY;
        ja[r] = 0;
      }
      for (int j = 0; j < k; ++j) {
        float wv[SUB];
#pragma unroll
        for (int e = 0; e < SUB; ++e) wv[e] = w32[j][e];
        const float hb = -0.5f * b32[j];
        const float wn = wn32[j], eb = eb32[j];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float sc = 0.f;
#pragma unroll
          for (int e = 0; e < SUB; ++e) sc = __fmaf_rn(zf[r][e], wv[e], sc);
          sc += hb;  // -b/2 is exact in fp32 (a power-of-two scale of b32)
          const float tj = sc + __fmaf_rn(cz[r], wn, eb);
          t2[r] = fmaxf(t2[r], fminf(t1[r], tj));
          if (tj > t1[r]) {
            t1[r] = tj;
            ja[r] = j;
          }
        }
      }
      int best[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int a = ja[r];
        float sa = 0.f;  // the candidate's fp32 score, formed exactly as in the scan
#pragma unroll
        for (int e = 0; e < SUB; ++e) sa = __fmaf_rn(zf[r][e], w32[a][e], sa);
        sa += -0.5f * b32[a];
        const float ea = __fmaf_rn(cz[r], wn32[a], eb32[a]);
        if ((double)sa - (double)ea > (double)t2[r]) {
          best[r] = a;
        } else {  // close call: every score in fp64
          double z[SUB];
          z_of(r, z);
          double bs = -INFINITY;
          int bj = 0x7FFFFFFF;
          for (int j = 0; j < k; ++j) {
            double sc = 0.0;
#pragma unroll
            for (int e = 0; e < SUB; ++e) sc += z[e] * w64[j][e];
            sc -= 0.5 * b64[j];
            if (better(sc, j, bs, bj)) {
              bs = sc;
              bj = j;
            }
          }
          best[r] = bj;
        }
      }
      uint8_t* cp = codes + (head * n + row) * M + grp * R;
#pragma unroll
      for (int r = 0; r < R; ++r) cp[r] = (uint8_t)best[r];
      continue;
    }
  }
}

template <int DT, int SUB>
int launch_pq(int mode, const void* x, int64_t n, const int32_t* idx, int64_t n_sel,
              int64_t heads, const float* cb, int k, const float* chol, const void* query,
              int64_t nq, double beta, uint8_t* codes, hipStream_t s) {
  constexpr int R = kPqRows;
  const int64_t items = heads * n_sel * (kD / SUB / R);
  int64_t g = (items + kPqThreads - 1) / kPqThreads;
  if (g > 4096) g = 4096;
  if (g < 1) g = 1;
  const dim3 grid((unsigned)g), block(kPqThreads);
  if (mode == kHWeighted)
    return launch("pq_encode_h", pq_encode<DT, kHWeighted, SUB, R>, grid, block, 0, s, x, n, idx,
                  n_sel, heads, cb, k, chol, query, nq, beta, codes);
  if (mode == kBlend)
    return launch("pq_encode_blend", pq_encode<DT, kBlend, SUB, R>, grid, block, 0, s, x, n, idx,
                  n_sel, heads, cb, k, chol, query, nq, beta, codes);
  return launch("pq_encode_plain", pq_encode<DT, kPlain, SUB, R>, grid, block, 0, s, x, n, idx, n_sel,
                heads, cb, k, chol, query, nq, beta, codes);
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
