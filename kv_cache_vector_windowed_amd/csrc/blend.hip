// assign_cosine: the cosine-blend assignment of the decode path.
// "veloxquant_mlx.quantizers.a2ats module", a2ats_query_aware_assignment:
//   score_j = beta * (-e_j / max_i e_i) + (1 - beta) * cos(q, c_j),  e_j = ||x - c_j||^2,
//   code = argmax_j score_j  (lowest index on ties).
// The error term is 0 when the row's maximum error is 0; a zero-norm query or centroid
// has cosine 0.
//
// Two kernels, rows in batches that keep the workspace under a fixed size:
//   blend_dots  workgroup = (head, 4 rows, 256 centroids): 32-dimension slices of the
//               centroids go through LDS transposed (thread j reads its centroid's value of
//               a dimension with a conflict-free load), the rows' x and q values are read
//               from LDS as fp64 broadcasts; per (row, centroid) it writes e_j = ||x - c_j||^2
//               (fp64 sum of squared fp64 differences in dimension order) and
//               g_j = (q . c_j) / ||c_j|| (0 when ||c_j|| = 0).
//   blend_pick  workgroup = (head, row): max_j e_j, then the blended scores
//               beta (-e_j / max e) + (1 - beta) g_j / ||q|| and their argmax (lowest index on
//               ties), all in fp64.
// The workspace holds e and g for the rows of one batch: the codebook is read once per four
// rows instead of once per row, with coalesced loads.
#include "common.hpp"

namespace a2ats {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ double block_max(double v, double* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  v = red[0];
  for (int i = 1; i < kThreads / 64; ++i) v = fmax(v, red[i]);
  return v;
}

__device__ __forceinline__ double block_sum(double v, double* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  v = red[0];
  for (int i = 1; i < kThreads / 64; ++i) v += red[i];
  return v;
}

// (score, index): larger score wins, equal scores keep the lower index.
__device__ __forceinline__ bool better(double s, int j, double bs, int bj) {
  return s > bs || (s == bs && j < bj);
}

constexpr int kBlRows = 4;     // rows per dot workgroup
constexpr int kBlTile = 256;   // centroids per dot workgroup (one per thread)
constexpr int kBlDims = 32;    // dimensions per codebook slice
constexpr size_t kBlWsCap = (size_t)64 << 20;  // workspace bound (e and g of one batch)
constexpr int kPickPre = 8;    // e and g entries a blend_pick thread reads up front

__global__ __launch_bounds__(kThreads) void blend_dots(
    const void* __restrict__ x, int xdt, int64_t n, int d, const void* __restrict__ query,
    int64_t nq, const float* __restrict__ cb, int64_t c, int64_t rb0, int64_t nrb,
    double* __restrict__ e_out, double* __restrict__ g_out) {
  __shared__ __align__(16) double xq[256][2 * kBlRows];   // [dim][x of 4 rows, q of 4 rows]
  __shared__ float ct[kBlDims][kBlTile + 1];              // codebook slice, transposed
  const int t = threadIdx.x;
  const int64_t item = rb0 + blockIdx.y;                  // (head, row block), flattened
  const int64_t head = item / nrb, r0 = (item % nrb) * kBlRows;
  const int64_t j0 = (int64_t)blockIdx.x * kBlTile;
  {  // the rows' x and q, all loads issued before the LDS stores (d <= 256: 8 per thread)
    constexpr int kXq = 256 * 2 * kBlRows / kThreads;
    float v[kXq];
#pragma unroll
    for (int u = 0; u < kXq; ++u) {
      const int i = t + kThreads * u;
      const int a = i / (2 * kBlRows), k = i % (2 * kBlRows), r = k % kBlRows;
      const int64_t row = r0 + r;
      v[u] = 0.f;
      if (a < d && row < n)
        v[u] = k < kBlRows ? load_elem(x, xdt, (head * n + row) * d + a)
                           : load_elem(query, xdt, (head * nq + (nq == 1 ? 0 : row)) * d + a);
    }
#pragma unroll
    for (int u = 0; u < kXq; ++u) {
      const int i = t + kThreads * u;
      xq[i / (2 * kBlRows)][i % (2 * kBlRows)] = (double)v[u];
    }
  }
  const float* cbh = cb + head * c * d;
  const int64_t j = j0 + t;
  double e[kBlRows], g[kBlRows], cn2 = 0.0;
#pragma unroll
  for (int r = 0; r < kBlRows; ++r) e[r] = g[r] = 0.0;
  // slice staging: thread t loads dimension t % 32 of centroids t / 32 + 8 i (32 consecutive
  // threads read one centroid row segment); all of a slice's loads are issued together, and
  // the next slice's while the current one is computed
  constexpr int kPer = kBlTile * kBlDims / kThreads;
  const int sa = t % kBlDims, sj = t / kBlDims;
  float pre[kPer];
  auto load_slice = [&](int a0) {
    const int da = d - a0 < kBlDims ? d - a0 : kBlDims;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int64_t jg = j0 + sj + (kThreads / kBlDims) * i;
      pre[i] = (jg < c && sa < da) ? cbh[jg * d + a0 + sa] : 0.f;
    }
  };
  load_slice(0);
  for (int a0 = 0; a0 < d; a0 += kBlDims) {
    const int da = d - a0 < kBlDims ? d - a0 : kBlDims;
    __syncthreads();  // the previous slice's readers are done (and xq is written)
#pragma unroll
    for (int i = 0; i < kPer; ++i) ct[sa][sj + (kThreads / kBlDims) * i] = pre[i];
    __syncthreads();
    if (a0 + kBlDims < d) load_slice(a0 + kBlDims);
    auto dim_step = [&](int aa) {
      const double cv = (double)ct[aa][t];
      const double* p = &xq[a0 + aa][0];
      double xs[kBlRows], qs[kBlRows];
#pragma unroll
      for (int r = 0; r < kBlRows; ++r) {
        xs[r] = p[r];
        qs[r] = p[kBlRows + r];
      }
      cn2 = __fma_rn(cv, cv, cn2);
#pragma unroll
      for (int r = 0; r < kBlRows; ++r) {
        const double df = xs[r] - cv;
        e[r] = __fma_rn(df, df, e[r]);
        g[r] = __fma_rn(qs[r], cv, g[r]);
      }
    };
    if (da == kBlDims) {  // a whole slice: a fixed trip count lets the loads run ahead
#pragma unroll 8
      for (int aa = 0; aa < kBlDims; ++aa) dim_step(aa);
    } else {
      for (int aa = 0; aa < da; ++aa) dim_step(aa);
    }
  }
  if (j < c) {
    const double cn = sqrt(cn2);
#pragma unroll
    for (int r = 0; r < kBlRows; ++r) {
      if (r0 + r >= n) break;
      const int64_t o = ((item - rb0) * kBlRows + r) * c + j;
      e_out[o] = e[r];
      g_out[o] = cn > 0.0 ? g[r] / cn : 0.0;
    }
  }
}

__global__ __launch_bounds__(kThreads) void blend_pick(
    const void* __restrict__ query, int xdt, int64_t n, int d, int64_t nq, int64_t c,
    double beta, int64_t rb0, int64_t nrb, const double* __restrict__ e_in,
    const double* __restrict__ g_in, uint16_t* __restrict__ codes) {
  __shared__ double red[kThreads / 64];
  __shared__ double rs[kThreads / 64];
  __shared__ int rj[kThreads / 64];
  const int t = threadIdx.x;
  const int64_t item = rb0 + blockIdx.y;
  const int r = blockIdx.x;  // row within the block
  const int64_t head = item / nrb, row = (item % nrb) * kBlRows + r;
  if (row >= n) return;      // uniform per workgroup
  const int64_t qoff = (head * nq + (nq == 1 ? 0 : row)) * d;
  const double* er = e_in + ((item - rb0) * kBlRows + r) * c;
  const double* gr = g_in + ((item - rb0) * kBlRows + r) * c;
  // the row's first kPickPre * kThreads entries are read with the query, before the
  // reductions, so that the reads are in flight together (the rest, for larger codebooks,
  // in the loops below)
  double ev[kPickPre], gv[kPickPre];
#pragma unroll
  for (int i = 0; i < kPickPre; ++i) {
    const int64_t j = t + (int64_t)kThreads * i;
    ev[i] = j < c ? er[j] : 0.0;
    gv[i] = j < c ? gr[j] : 0.0;
  }
  double qv = 0.0;
  if (t < d) qv = (double)load_elem(query, xdt, qoff + t);
  const double qn = sqrt(block_sum(qv * qv, red));
  constexpr int64_t kHeld = (int64_t)kPickPre * kThreads;
  double emax = 0.0;
#pragma unroll
  for (int i = 0; i < kPickPre; ++i)
    if (t + (int64_t)kThreads * i < c) emax = fmax(emax, ev[i]);
  for (int64_t j = kHeld + t; j < c; j += kThreads) emax = fmax(emax, er[j]);
  emax = block_max(emax, red);
  double bs = -INFINITY;
  int bj = 0x7FFFFFFF;
  auto consider = [&](int64_t j, double e, double gq) {
    const double cosv = qn > 0.0 ? gq / qn : 0.0;
    const double err = emax > 0.0 ? e / emax : 0.0;
    const double s = beta * (-err) + (1.0 - beta) * cosv;
    if (better(s, (int)j, bs, bj)) {
      bs = s;
      bj = (int)j;
    }
  };
#pragma unroll
  for (int i = 0; i < kPickPre; ++i) {
    const int64_t j = t + (int64_t)kThreads * i;
    if (j < c) consider(j, ev[i], gv[i]);
  }
  for (int64_t j = kHeld + t; j < c; j += kThreads) consider(j, er[j], gr[j]);
  for (int o = 32; o > 0; o >>= 1) {
    const double os = __shfl_xor(bs, o);
    const int oj = __shfl_xor(bj, o);
    if (better(os, oj, bs, bj)) {
      bs = os;
      bj = oj;
    }
  }
  const int lane = t & 63, w = t >> 6;
  if (lane == 0) {
    rs[w] = bs;
    rj[w] = bj;
  }
  __syncthreads();
  if (t == 0) {
    for (int i = 1; i < kThreads / 64; ++i)
      if (better(rs[i], rj[i], bs, bj)) {
        bs = rs[i];
        bj = rj[i];
      }
    codes[head * n + row] = (uint16_t)bj;
  }
}

// Row blocks per batch: as many as fit the workspace bound (at least one).
inline int64_t blend_batch(int64_t heads, int64_t n, int64_t c) {
  const int64_t nrb = (n + kBlRows - 1) / kBlRows;
  const size_t per = (size_t)kBlRows * c * 2 * sizeof(double);
  int64_t b = (int64_t)(kBlWsCap / per);
  if (b < 1) b = 1;
  if (b > 65535) b = 65535;  // second grid dimension
  return b < heads * nrb ? b : heads * nrb;
}

}  // namespace
}  // namespace a2ats

using namespace a2ats;

extern "C" size_t a2ats_assign_cosine_workspace(int64_t heads, int64_t n, int64_t c) {
  if (heads < 1 || n < 1 || c < 1) return 0;
  const size_t rows = (size_t)blend_batch(heads, n, c) * kBlRows;
  return 2 * align_up(rows * c * sizeof(double));
}

extern "C" int a2ats_assign_cosine(const void* x, int x_dtype, int64_t heads, int64_t n,
                                   int64_t d, const void* query, int64_t nq,
                                   const float* codebook, int64_t c, double beta,
                                   uint16_t* codes, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  if (x_dtype != A2ATS_F32 && x_dtype != A2ATS_BF16) return A2ATS_EDTYPE;
  if (heads < 1 || n < 0 || d < 1 || d > 256 || c < 1 || c > 65536) return A2ATS_EINVAL;
  if (!(beta >= 0.0 && beta <= 1.0)) return A2ATS_EINVAL;
  if (n == 0) return A2ATS_OK;
  if (!(nq == 1 || nq == n)) return A2ATS_EINVAL;
  if (!x || !query || !codebook || !codes) return A2ATS_EINVAL;
  if (heads > 65535 || n > 0x7FFFFFFF) return A2ATS_EINVAL;
  if (!ws_ok(workspace, workspace_bytes, a2ats_assign_cosine_workspace(heads, n, c)))
    return A2ATS_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t nrb = (n + kBlRows - 1) / kBlRows;
  const int64_t batch = blend_batch(heads, n, c);
  const size_t half = align_up((size_t)batch * kBlRows * c * sizeof(double));
  double* e = static_cast<double*>(workspace);
  double* g = reinterpret_cast<double*>(static_cast<char*>(workspace) + half);
  for (int64_t rb0 = 0; rb0 < heads * nrb; rb0 += batch) {
    const int64_t m = heads * nrb - rb0 < batch ? heads * nrb - rb0 : batch;
    A2ATS_TRY(launch("assign_cosine_dots", blend_dots,
                     dim3((unsigned)((c + kBlTile - 1) / kBlTile), (unsigned)m), dim3(kThreads), 0,
                     s, x, x_dtype, n, (int)d, query, nq, codebook, c, rb0, nrb, e, g));
    A2ATS_TRY(launch("assign_cosine", blend_pick, dim3(kBlRows, (unsigned)m), dim3(kThreads), 0,
                     s, query, x_dtype, n, (int)d, nq, c, beta, rb0, nrb, e, g, codes));
  }
  return A2ATS_OK;
}
