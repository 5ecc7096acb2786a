// k-means++ seeding of a codebook in z-space.  "veloxquant_mlx.quantizers.a2ats module",
// a2ats_cholesky_factor: Eq. 16-18 turn the H-weighted objective into a plain Euclidean one
// on z = x L, which is what lets conventional k-means++ build the codebook (the docs'
// calibration trains it with a seed).  k-means++ (Arthur and Vassilvitskii): the first
// center is a uniformly drawn row; every next center is a row drawn with probability
// proportional to D^2, its squared distance to the nearest center chosen so far.
//
// The draws are inputs, r[t] uniform over [0, 2^64) for center t, and the weighting is made
// exact so the result does not depend on how the rows are split over workgroups:
//   z_i = x_i L, each z_ia the fp64 sum over b in order of x_ib L_ba, rounded to fp32 (x_i
//         itself without L); Z = max_i ||z_i||^2
//   c_0 = floor(r_0 n / 2^64)
//   D2_i = min over chosen c of ||z_i - z_c||^2 (fp64, dimensions in order, no fused
//          multiply-add), w_i = floor(D2_i 2^e) as a 64-bit integer with the fixed
//          e = 60 - ceil(log2 n) - ceil(log2 4Z), W = sum w_i (exact: integers)
//   c_t = the first row whose running sum of w exceeds floor(r_t W / 2^64)
//         (floor(r_t n / 2^64) when W = 0).
// Every floating-point operation is the same sequence, in the same order, as in a plain
// sequential loop, so the centers are those of such a loop bit for bit.
//
// Kernels
//   kmpp_clear   Z of every head to 0
//   kmpp_z       thread (row, dim): z in fp64 then fp32, stored dimension-major [d][n] so
//                that a thread per row reads a coalesced column per dimension; per row
//                ||z||^2 (in order) folded into Z by an integer maximum of its bits
//   kmpp_round   one launch per center t = 1 .. k-1: every workgroup first locates center
//                t-1 itself (from the previous launch's block sums and D2, the same exact
//                integer search in every workgroup, so no workgroup waits for another),
//                then updates D2 of its rows against it and writes its block sum of w.
//                D2 and the block sums are double-buffered across launches.
//   kmpp_final   the last center, then the rows gathered into the codebook.
#include "common.hpp"

namespace a2ats {
namespace {

constexpr int kKmppBlk = 1024;   // rows per workgroup of a round (4 per thread)
constexpr int kKmppMaxD = 128;

__device__ __forceinline__ uint64_t mulhi64(uint64_t a, uint64_t b) { return __umul64hi(a, b); }

// ceil(log2(x)) for x > 0, exactly.
__device__ __forceinline__ int clog2_exact(double x) {
  int p = 0;
  const double m = frexp(x, &p);
  return m == 0.5 ? p - 1 : p;
}

__device__ __forceinline__ int weight_exp(int64_t n, const uint64_t* zmax_bits) {
  const double z = __longlong_as_double((long long)*zmax_bits);
  int e = 60 - clog2_exact((double)n);
  if (z > 0.0) e -= clog2_exact(4.0 * z);
  return e;
}

__device__ __forceinline__ uint64_t weight_of(double d2, int e) {
  return (uint64_t)floor(ldexp(d2, e));
}

// Exclusive prefix over the 256 threads of a workgroup of 64-bit values (thread order);
// *total receives the sum.  Every thread must call it.
__device__ uint64_t block_scan_u64(uint64_t v, uint64_t* total) {
  __shared__ uint64_t wsum[4];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  uint64_t incl = v;
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t u = __shfl_up(incl, o);
    if (lane >= o) incl += u;
  }
  __syncthreads();
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint64_t before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  *total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  return before + incl - v;
}

// The center drawn with r from the weights of (d2, n rows) whose block sums are bsum (nblk
// blocks of kKmppBlk rows).  Every thread of the workgroup calls it and gets the row.
__device__ int64_t kmpp_select(const uint64_t* __restrict__ bsum, const double* __restrict__ d2,
                               int64_t n, int nblk, int e, uint64_t r) {
  __shared__ int64_t s_pick;
  __shared__ uint64_t s_rest;
  const int t = threadIdx.x;
  // blocks: a contiguous chunk per thread
  const int chunk = (nblk + 255) / 256;
  const int b0 = t * chunk, b1 = min(nblk, b0 + chunk);
  uint64_t mine = 0;
  for (int b = b0; b < b1; ++b) mine += bsum[b];
  uint64_t W = 0;
  const uint64_t before = block_scan_u64(mine, &W);
  if (W == 0) return (int64_t)mulhi64(r, (uint64_t)n);
  const uint64_t T = mulhi64(r, W);
  if (T >= before && T < before + mine) {  // exactly one thread
    uint64_t run = before;
    for (int b = b0; b < b1; ++b) {
      if (T < run + bsum[b]) {
        s_pick = b;
        s_rest = T - run;
        break;
      }
      run += bsum[b];
    }
  }
  __syncthreads();
  const int64_t bstar = s_pick;
  const uint64_t rest = s_rest;
  // rows of block b*: 4 consecutive rows per thread, in row order
  const int64_t r0 = bstar * kKmppBlk + (int64_t)t * 4;
  uint64_t w[4], wm = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    w[q] = (r0 + q < n) ? weight_of(d2[r0 + q], e) : 0;
    wm += w[q];
  }
  uint64_t tot = 0;
  const uint64_t bef = block_scan_u64(wm, &tot);
  __syncthreads();
  if (rest >= bef && rest < bef + wm) {
    uint64_t run = bef;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      run += w[q];
      if (rest < run) {
        s_pick = r0 + q;
        break;
      }
    }
  }
  __syncthreads();
  return s_pick;
}

__global__ void kmpp_clear(uint64_t* __restrict__ zmax, int64_t heads) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < heads) zmax[i] = 0;
}

// z = x L (fp64 sums in order, rounded to fp32), dimension-major; Z = max ||z||^2.
template <int DT>
__global__ __launch_bounds__(256) void kmpp_z(const void* __restrict__ x, int64_t n, int d,
                                              const float* __restrict__ chol,
                                              float* __restrict__ z, uint64_t* __restrict__ zmax) {
#pragma clang fp contract(off)
  __shared__ float Ls[kKmppMaxD * kKmppMaxD];
  __shared__ double xr[256];
  __shared__ float zr[256];
  const int64_t head = blockIdx.y;
  const int t = threadIdx.x;
  if (chol) {
    const float* L = chol + head * (int64_t)d * d;
    for (int e = t; e < d * d; e += 256) Ls[e] = L[e];
  }
  const int ppb = 256 / d;  // rows per pass
  const int p = t / d, a = t % d;
  double zloc = 0.0;  // largest ||z||^2 of the rows this thread summed
  for (int64_t r0 = (int64_t)blockIdx.x * ppb; r0 < n; r0 += (int64_t)gridDim.x * ppb) {
    const int64_t row = r0 + p;
    __syncthreads();
    xr[t] = row < n ? (double)load_elem(x, DT, (head * n + row) * d + a) : 0.0;
    __syncthreads();
    float zv;
    if (chol) {
      double s = 0.0;
      for (int b = 0; b < d; ++b) s = s + xr[p * d + b] * (double)Ls[b * d + a];
      zv = (float)s;
    } else {
      zv = (float)xr[t];
    }
    zr[t] = zv;
    if (row < n) z[(head * d + a) * n + row] = zv;
    __syncthreads();
    if (a == 0 && row < n) {
      double s = 0.0;
      for (int b = 0; b < d; ++b) {
        const double v = (double)zr[p * d + b];
        s = s + v * v;
      }
      zloc = fmax(zloc, s);
    }
  }
  // non-negative doubles order as their bit patterns
  for (int o = 32; o > 0; o >>= 1) zloc = fmax(zloc, __shfl_xor(zloc, o));
  if ((t & 63) == 0 && zloc > 0.0)
    atomicMax(reinterpret_cast<unsigned long long*>(zmax + head),
              (unsigned long long)__double_as_longlong(zloc));
}

// Round t (1 .. k-1): center t-1, then D2 and the block sums for round t.
template <int D>
__global__ __launch_bounds__(256) void kmpp_round(const float* __restrict__ z, int64_t n,
                                                  int nblk, int64_t k, int64_t t,
                                                  const uint64_t* __restrict__ draws,
                                                  const uint64_t* __restrict__ zmax,
                                                  double* __restrict__ d2buf,
                                                  uint64_t* __restrict__ bsbuf,
                                                  int32_t* __restrict__ sel) {
#pragma clang fp contract(off)
  __shared__ float zc[D];
  const int64_t head = blockIdx.y;
  const int tid = threadIdx.x;
  const int e = weight_exp(n, zmax + head);
  const int cur = (int)(t & 1), prev = cur ^ 1;
  double* d2c = d2buf + ((int64_t)cur * gridDim.y + head) * n;
  const double* d2p = d2buf + ((int64_t)prev * gridDim.y + head) * n;
  const uint64_t* bsp = bsbuf + ((int64_t)prev * gridDim.y + head) * nblk;
  uint64_t* bsc = bsbuf + ((int64_t)cur * gridDim.y + head) * nblk;
  int64_t c;
  if (t == 1) c = (int64_t)mulhi64(draws[head * k], (uint64_t)n);
  else c = kmpp_select(bsp, d2p, n, nblk, e, draws[head * k + t - 1]);
  if (blockIdx.x == 0 && tid == 0) sel[head * k + t - 1] = (int32_t)c;
  const float* zh = z + head * (int64_t)D * n;
  if (tid < D) zc[tid] = zh[(int64_t)tid * n + c];
  __syncthreads();
  uint64_t wsum = 0;
#pragma unroll
  for (int q = 0; q < kKmppBlk / 256; ++q) {
    const int64_t row = (int64_t)blockIdx.x * kKmppBlk + q * 256 + tid;
    if (row < n) {
      double s = 0.0;
#pragma unroll 8
      for (int a = 0; a < D; ++a) {
        const double df = (double)zh[(int64_t)a * n + row] - (double)zc[a];
        s = s + df * df;
      }
      double v = s;
      if (t > 1 && !(s < d2p[row])) v = d2p[row];
      d2c[row] = v;
      wsum += weight_of(v, e);
    }
  }
  uint64_t tot = 0;
  (void)block_scan_u64(wsum, &tot);
  if (tid == 0) bsc[blockIdx.x] = tot;
}

// The last center (k >= 2: from round k-1's weights; k = 1: the uniform first draw), then
// the rows of all k centers gathered into the codebook (fp32) and idx.
__global__ __launch_bounds__(256) void kmpp_final(const uint64_t* __restrict__ draws, int64_t n,
                                                  int nblk, int64_t k,
                                                  const uint64_t* __restrict__ zmax,
                                                  const double* __restrict__ d2buf,
                                                  const uint64_t* __restrict__ bsbuf,
                                                  int32_t* __restrict__ sel) {
  const int64_t head = blockIdx.x;
  int64_t c;
  if (k == 1) {
    c = (int64_t)mulhi64(draws[head * k], (uint64_t)n);
  } else {
    const int last = (int)((k - 1) & 1);
    const int e = weight_exp(n, zmax + head);
    c = kmpp_select(bsbuf + ((int64_t)last * gridDim.x + head) * nblk,
                    d2buf + ((int64_t)last * gridDim.x + head) * n, n, nblk, e,
                    draws[head * k + k - 1]);
  }
  if (threadIdx.x == 0) sel[head * k + k - 1] = (int32_t)c;
}

template <int DT>
__global__ __launch_bounds__(256) void kmpp_gather(const void* __restrict__ x, int64_t n, int d,
                                                   int64_t k, int64_t heads,
                                                   const int32_t* __restrict__ sel,
                                                   float* __restrict__ codebook,
                                                   int32_t* __restrict__ idx) {
  const int64_t total = heads * k * d;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * 256) {
    const int64_t a = e % d, j = (e / d) % k, h = e / (d * k);
    const int64_t row = sel[h * k + j];
    codebook[e] = load_elem(x, DT, (h * n + row) * d + a);
    if (idx && a == 0) idx[h * k + j] = (int32_t)row;
  }
}

struct KmppLayout {
  float* z;
  double* d2;
  uint64_t* bsum;
  uint64_t* zmax;
  int32_t* sel;
  int nblk;
  size_t bytes;
};

KmppLayout kmpp_carve(void* ws, int64_t heads, int64_t n, int64_t d, int64_t k) {
  Carver cv(ws);
  KmppLayout L;
  L.nblk = (int)((n + kKmppBlk - 1) / kKmppBlk);
  L.z = cv.take<float>((size_t)(heads * n * d));
  L.d2 = cv.take<double>((size_t)(2 * heads * n));
  L.bsum = cv.take<uint64_t>((size_t)(2 * heads * L.nblk));
  L.zmax = cv.take<uint64_t>((size_t)heads);
  L.sel = cv.take<int32_t>((size_t)(heads * k));
  L.bytes = cv.used;
  return L;
}

bool kmpp_shape_ok(int64_t heads, int64_t n, int64_t d, int64_t k) {
  if (heads < 1 || heads > 65535 || n < 1 || n > 0x7FFFFFFF || k < 1 || k > n) return false;
  return d == 4 || d == 8 || d == 16 || d == 32 || d == 64 || d == 128;
}

template <int D>
int kmpp_rounds(const KmppLayout& L, int64_t heads, int64_t n, int64_t k, const uint64_t* draws,
                hipStream_t s) {
  for (int64_t t = 1; t < k; ++t)
    A2ATS_TRY(launch("kmeans_init_round", kmpp_round<D>, dim3((unsigned)L.nblk, (unsigned)heads),
                     dim3(256), 0, s, L.z, n, L.nblk, k, t, draws, L.zmax, L.d2, L.bsum, L.sel));
  return A2ATS_OK;
}

}  // namespace
}  // namespace a2ats

using namespace a2ats;

extern "C" size_t a2ats_kmeans_init_workspace(int64_t heads, int64_t n, int64_t d, int64_t k) {
  if (!kmpp_shape_ok(heads, n, d, k)) return 0;
  return kmpp_carve(nullptr, heads, n, d, k).bytes;
}

extern "C" int a2ats_kmeans_init(const void* x, int x_dtype, int64_t heads, int64_t n, int64_t d,
                                 int64_t k, const float* chol, const uint64_t* draws,
                                 float* codebook, int32_t* idx, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (x_dtype != A2ATS_F32 && x_dtype != A2ATS_BF16) return A2ATS_EDTYPE;
  if (!kmpp_shape_ok(heads, n, d, k)) return A2ATS_EINVAL;
  if (!x || !draws || !codebook) return A2ATS_EINVAL;
  const size_t need = a2ats_kmeans_init_workspace(heads, n, d, k);
  if (!ws_ok(workspace, workspace_bytes, need)) return A2ATS_EWORKSPACE;
  const KmppLayout L = kmpp_carve(workspace, heads, n, d, k);
  hipStream_t s = static_cast<hipStream_t>(stream);
  A2ATS_TRY(launch("kmeans_init_clear", kmpp_clear, dim3(grid_for(heads, 256)), dim3(256), 0, s,
                   L.zmax, heads));
  const int64_t ppb = 256 / d;
  const unsigned gz = grid_for(n, (int)ppb, 4096);
  if (x_dtype == A2ATS_BF16)
    A2ATS_TRY(launch("kmeans_init_z", kmpp_z<A2ATS_BF16>, dim3(gz, (unsigned)heads), dim3(256), 0,
                     s, x, n, (int)d, chol, L.z, L.zmax));
  else
    A2ATS_TRY(launch("kmeans_init_z", kmpp_z<A2ATS_F32>, dim3(gz, (unsigned)heads), dim3(256), 0,
                     s, x, n, (int)d, chol, L.z, L.zmax));
  switch (d) {
    case 4: A2ATS_TRY(kmpp_rounds<4>(L, heads, n, k, draws, s)); break;
    case 8: A2ATS_TRY(kmpp_rounds<8>(L, heads, n, k, draws, s)); break;
    case 16: A2ATS_TRY(kmpp_rounds<16>(L, heads, n, k, draws, s)); break;
    case 32: A2ATS_TRY(kmpp_rounds<32>(L, heads, n, k, draws, s)); break;
    case 64: A2ATS_TRY(kmpp_rounds<64>(L, heads, n, k, draws, s)); break;
    default: A2ATS_TRY(kmpp_rounds<128>(L, heads, n, k, draws, s)); break;
  }
  A2ATS_TRY(launch("kmeans_init_final", kmpp_final, dim3((unsigned)heads), dim3(256), 0, s, draws,
                   n, L.nblk, k, L.zmax, L.d2, L.bsum, L.sel));
  const unsigned gg = grid_for(heads * k * d, 256, 8192);
  if (x_dtype == A2ATS_BF16)
    return launch("kmeans_init_gather", kmpp_gather<A2ATS_BF16>, dim3(gg), dim3(256), 0, s, x, n,
                  (int)d, k, heads, L.sel, codebook, idx);
  return launch("kmeans_init_gather", kmpp_gather<A2ATS_F32>, dim3(gg), dim3(256), 0, s, x, n,
                (int)d, k, heads, L.sel, codebook, idx);
}
