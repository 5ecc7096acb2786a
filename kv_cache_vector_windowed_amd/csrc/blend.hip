// assign_cosine: the cosine-blend assignment of the decode path.
// "veloxquant_mlx.quantizers.a2ats module", a2ats_query_aware_assignment:
//   score_j = beta * (-e_j / max_i e_i) + (1 - beta) * cos(q, c_j),  e_j = ||x - c_j||^2,
//   code = argmax_j score_j  (lowest index on ties).
// The error term is 0 when the row's maximum error is 0; a zero-norm query or centroid
// has cosine 0.
//
// One workgroup per (head, row).  The row and its query are staged in LDS as fp64; each
// thread owns centroids j = tid, tid + 256, ...  Pass 1 finds max_j e_j, pass 2 scores and
// takes the argmax.  Everything is fp64: the work is tiny (latency-bound) and fp64 keeps the
// decision identical to an exact evaluation except at true ties.
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

__global__ __launch_bounds__(kThreads) void blend_assign(
    const void* __restrict__ x, int xdt, int64_t n, int d, const void* __restrict__ query,
    int64_t nq, const float* __restrict__ cb, int64_t c, double beta,
    uint16_t* __restrict__ codes) {
  const int64_t head = blockIdx.y;
  const int64_t row = blockIdx.x;
  __shared__ double xs[256];
  __shared__ double qs[256];
  __shared__ double red[kThreads / 64];
  __shared__ double rs[kThreads / 64];
  __shared__ int rj[kThreads / 64];
  const int t = threadIdx.x;
  const int64_t xoff = (head * n + row) * d;
  const int64_t qoff = (head * nq + (nq == 1 ? 0 : row)) * d;
  if (t < d) {
    xs[t] = (double)load_elem(x, xdt, xoff + t);
    qs[t] = (double)load_elem(query, xdt, qoff + t);
  }
  __syncthreads();
  const double qn2 = block_sum(t < d ? qs[t] * qs[t] : 0.0, red);
  const double qn = sqrt(qn2);
  const float* cbh = cb + head * c * d;

  double emax = 0.0;
  for (int64_t j = t; j < c; j += kThreads) {
    const float* cr = cbh + j * d;
    double e = 0.0;
    for (int a = 0; a < d; ++a) {
      double df = xs[a] - (double)cr[a];
      e += df * df;
    }
    emax = fmax(emax, e);
  }
  emax = block_max(emax, red);

  double bs = -INFINITY;
  int bj = 0x7FFFFFFF;
  for (int64_t j = t; j < c; j += kThreads) {
    const float* cr = cbh + j * d;
    double e = 0.0, dot = 0.0, cn2 = 0.0;
    for (int a = 0; a < d; ++a) {
      double cv = (double)cr[a];
      double df = xs[a] - cv;
      e += df * df;
      dot += qs[a] * cv;
      cn2 += cv * cv;
    }
    const double cn = sqrt(cn2);
    const double cosv = (qn > 0.0 && cn > 0.0) ? dot / (qn * cn) : 0.0;
    const double err = emax > 0.0 ? e / emax : 0.0;
    const double s = beta * (-err) + (1.0 - beta) * cosv;
    if (better(s, (int)j, bs, bj)) {
      bs = s;
      bj = (int)j;
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    double os = __shfl_xor(bs, o);
    int oj = __shfl_xor(bj, o);
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

}  // namespace
}  // namespace a2ats

using namespace a2ats;

extern "C" int a2ats_assign_cosine(const void* x, int x_dtype, int64_t heads, int64_t n,
                                   int64_t d, const void* query, int64_t nq,
                                   const float* codebook, int64_t c, double beta,
                                   uint16_t* codes, void* stream) {
  if (x_dtype != A2ATS_F32 && x_dtype != A2ATS_BF16) return A2ATS_EDTYPE;
  if (heads < 1 || n < 0 || d < 1 || d > 256 || c < 1 || c > 65536) return A2ATS_EINVAL;
  if (!(beta >= 0.0 && beta <= 1.0)) return A2ATS_EINVAL;
  if (n == 0) return A2ATS_OK;
  if (!(nq == 1 || nq == n)) return A2ATS_EINVAL;
  if (!x || !query || !codebook || !codes) return A2ATS_EINVAL;
  if (heads > 65535 || n > 0x7FFFFFFF) return A2ATS_EINVAL;
  return launch("assign_cosine", blend_assign, dim3((unsigned)n, (unsigned)heads), dim3(kThreads),
                0, static_cast<hipStream_t>(stream), x, x_dtype, n, (int)d, query, nq, codebook,
                c, beta, codes);
}
