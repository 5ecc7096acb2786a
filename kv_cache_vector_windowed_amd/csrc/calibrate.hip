// calibrate: the query second moment H = E[q^T q] + ridge I and its Cholesky factor L.
// "veloxquant_mlx.quantizers.a2ats module": a2ats_query_second_moment (Eq. 10) and
// a2ats_cholesky_factor (Eq. 15).
//
// Kernels
//   cal_moment_partial  per (head, 64x64 output tile, chunk of 512 query rows): fp64 partial
//                       sums of q_a q_b (the fp32 products are exact in fp64).
//   cal_moment_reduce   per H element: sums the chunk partials in chunk order, divides by m,
//                       adds the ridge on the diagonal, rounds once to fp32.
//   cal_cholesky        one workgroup per head, the whole matrix in LDS as fp64: right-
//                       looking elimination.  Each entry receives its updates in the same
//                       order as the row-by-row (Cholesky-Banachiewicz) recurrence, with
//                       separately rounded multiply and subtract, so the factor of a given
//                       fp32 H does not depend on the thread schedule.
#include "common.hpp"

namespace a2ats {
namespace {

constexpr int kTile = 64;      // H tile edge per workgroup
constexpr int kChunk = 512;    // query rows per partial sum
constexpr int kStage = 64;     // query rows staged in LDS at a time

__global__ __launch_bounds__(256) void cal_moment_partial(const float* __restrict__ q, int64_t m,
                                                          int d, int tiles_1d, int chunks,
                                                          double* __restrict__ part) {
  const int head = blockIdx.z;
  const int chunk = blockIdx.y;
  const int a0 = (blockIdx.x / tiles_1d) * kTile;
  const int b0 = (blockIdx.x % tiles_1d) * kTile;
  const int t = threadIdx.x;
  const int ty = t / 16, tx = t % 16;
  __shared__ float qa[kStage][kTile + 1];
  __shared__ float qb[kStage][kTile + 1];
  double acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;

  const float* qh = q + (int64_t)head * m * d;
  const int64_t r_begin = (int64_t)chunk * kChunk;
  const int64_t r_end = r_begin + kChunk < m ? r_begin + kChunk : m;
  for (int64_t r0 = r_begin; r0 < r_end; r0 += kStage) {
    __syncthreads();
    for (int e = t; e < kStage * kTile; e += 256) {
      int rr = e / kTile, cc = e % kTile;
      int64_t r = r0 + rr;
      bool ok_r = r < r_end;
      qa[rr][cc] = (ok_r && a0 + cc < d) ? qh[r * d + a0 + cc] : 0.f;
      qb[rr][cc] = (ok_r && b0 + cc < d) ? qh[r * d + b0 + cc] : 0.f;
    }
    __syncthreads();
    for (int rr = 0; rr < kStage; ++rr) {
      double va[4], vb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        va[i] = (double)qa[rr][ty * 4 + i];
        vb[i] = (double)qb[rr][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += va[i] * vb[j];  // exact products
    }
  }
  double* out = part + ((int64_t)head * chunks + chunk) * d * d;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int a = a0 + ty * 4 + i, b = b0 + tx * 4 + j;
      if (a < d && b < d) out[a * d + b] = acc[i][j];
    }
}

__global__ __launch_bounds__(256) void cal_moment_reduce(const double* __restrict__ part,
                                                         int64_t m, int d, int chunks,
                                                         int64_t heads, double ridge,
                                                         float* __restrict__ h_out) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = heads * d * d;
  if (e >= total) return;
  const int64_t head = e / ((int64_t)d * d);
  const int64_t ab = e % ((int64_t)d * d);
  const double* p = part + head * chunks * d * d + ab;
  double s = 0.0;
  for (int c = 0; c < chunks; ++c) s += p[(int64_t)c * d * d];
  s = s / (double)m;
  if (ab / d == ab % d) s += ridge;
  h_out[e] = (float)s;
}

// One workgroup per head; LDS holds the (d x d) working matrix in fp64 with a padded row.
__global__ __launch_bounds__(256) void cal_cholesky(const float* __restrict__ h, int d,
                                                    float* __restrict__ l_out,
                                                    int* __restrict__ status) {
  extern __shared__ double A[];  // [d][d + 1]
  const int ld = d + 1;
  const int head = blockIdx.x;
  const int t = threadIdx.x;
  const float* hh = h + (int64_t)head * d * d;
#pragma unroll 8
  for (int e = t; e < d * d; e += 256) {
    int i = e / d, k = e % d;
    A[i * ld + k] = (double)hh[e];
  }
  __shared__ int failed;
  if (t == 0) failed = 0;
  __syncthreads();
  for (int j = 0; j < d; ++j) {
    const double piv = A[j * ld + j];
    if (!(piv > 0.0)) {
      if (t == 0) failed = 1;
      break;  // uniform: every thread read the same pivot
    }
    const double ljj = sqrt(piv);
    __syncthreads();
    if (t == 0) A[j * ld + j] = ljj;
    for (int i = j + 1 + t; i < d; i += 256) A[i * ld + j] = A[i * ld + j] / ljj;
    __syncthreads();
    const int ty = t / 16, tx = t % 16;
    for (int i = j + 1 + ty; i < d; i += 16) {
      const double lij = A[i * ld + j];
      for (int k = j + 1 + tx; k <= i; k += 16) {
        double prod = __dmul_rn(lij, A[k * ld + j]);
        A[i * ld + k] = __dsub_rn(A[i * ld + k], prod);
      }
    }
    __syncthreads();
  }
  __syncthreads();
  float* lo = l_out + (int64_t)head * d * d;
  for (int e = t; e < d * d; e += 256) {
    int i = e / d, k = e % d;
    lo[e] = (k <= i && !failed) ? (float)A[i * ld + k] : 0.f;
  }
  if (t == 0) status[head] = failed ? A2ATS_ENOTSPD : A2ATS_OK;
}

inline int chunks_for(int64_t m) { return (int)((m + kChunk - 1) / kChunk); }

}  // namespace
}  // namespace a2ats

using namespace a2ats;

extern "C" size_t a2ats_calibrate_workspace(int64_t heads, int64_t m, int64_t d) {
  if (heads < 1 || m < 1 || d < 1 || d > 128) return 0;
  Carver c(nullptr);
  c.take<double>((size_t)heads * chunks_for(m) * d * d);
  c.take<int>((size_t)heads);
  return c.used;
}

extern "C" int a2ats_calibrate(const float* queries, int64_t heads, int64_t m, int64_t d,
                               double ridge, float* h_out, float* l_out, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (heads < 1 || m < 1 || d < 1 || d > 128) return A2ATS_EINVAL;
  if (!(ridge >= 0.0) || !std::isfinite(ridge)) return A2ATS_EINVAL;
  if (!queries || !h_out || !l_out) return A2ATS_EINVAL;
  if (heads > 65535 || chunks_for(m) > 65535) return A2ATS_EINVAL;
  const size_t need = a2ats_calibrate_workspace(heads, m, d);
  if (!ws_ok(workspace, workspace_bytes, need)) return A2ATS_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Carver c(workspace);
  const int chunks = chunks_for(m);
  double* part = c.take<double>((size_t)heads * chunks * d * d);
  int* status = c.take<int>((size_t)heads);
  const int tiles_1d = (int)((d + kTile - 1) / kTile);
  A2ATS_TRY(launch("calibrate_moment_partial", cal_moment_partial,
                   dim3(tiles_1d * tiles_1d, chunks, (unsigned)heads), dim3(256), 0, s, queries,
                   m, (int)d, tiles_1d, chunks, part));
  A2ATS_TRY(launch("calibrate_moment_reduce", cal_moment_reduce,
                   dim3(grid_for(heads * d * d, 256)), dim3(256), 0, s, part, m, (int)d, chunks,
                   heads, ridge, h_out));
  const size_t shmem = (size_t)d * (d + 1) * sizeof(double);
  A2ATS_TRY(set_dynamic_lds(cal_cholesky, shmem));
  A2ATS_TRY(launch("calibrate_cholesky", cal_cholesky, dim3((unsigned)heads), dim3(256), shmem, s,
                   h_out, (int)d, l_out, status));
  int host_status[64];
  for (int64_t h0 = 0; h0 < heads; h0 += 64) {
    int64_t cnt = heads - h0 < 64 ? heads - h0 : 64;
    if (hipMemcpyAsync(host_status, status + h0, cnt * sizeof(int), hipMemcpyDeviceToHost, s) !=
        hipSuccess)
      return A2ATS_EHIP;
    if (hipStreamSynchronize(s) != hipSuccess) return A2ATS_EHIP;
    for (int64_t i = 0; i < cnt; ++i)
      if (host_status[i] != A2ATS_OK) return A2ATS_ENOTSPD;
  }
  return A2ATS_OK;
}
