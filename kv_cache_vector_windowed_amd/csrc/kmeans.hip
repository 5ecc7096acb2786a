// Codebook training: Lloyd's k-means with the H-weighted assignment.  "veloxquant_mlx.
// quantizers.a2ats module", a2ats_cholesky_factor: Eq. 16-18 map the H-weighted objective to
// a plain Euclidean one on z = xL, where conventional k-means applies.  Because z = xL is
// linear and L invertible, the z-space update (the mean of a cluster's z rows) mapped back
// by L^-1 is the mean of the cluster's x rows: the original-space centroid is the plain
// member mean, with or without H.  The assignment step is the library's exact encode (whole
// head vectors, uint16 codes) or its sub-vector encode (the pages train one codebook on the
// pooled sub-vectors, uint8 codes).
//
// The update is deterministic (no floating-point atomics): the rows are grouped by code with
// a stable counting sort, and each centroid's members are summed in fp64 in a fixed order.
//   km_hist     per block of rows: code counts (LDS histogram)
//   km_offsets  one 1024-thread workgroup per head: per code, the exclusive offsets of the
//               blocks and, over codes, the start of each code's run (prefix sums over 16
//               block groups and 64-code tiles)
//   km_scatter  per block: the block's rows written into their code's run in row order; the
//               16 waves of a 1024-row chunk take turns, each ranking its lanes among equal
//               codes with ballots over the code bits (stable), then advancing the per-code
//               running counts in LDS
//   km_mean     one workgroup per centroid: members summed in fp64 (lanes over dimensions
//               and, for narrow rows, over interleaved member subsets combined by a fixed
//               shuffle tree; a large cluster in up to 16 ordered segments), divided by the
//               count, rounded once; an empty cluster keeps its row.
#include "common.hpp"

namespace a2ats {
namespace {

constexpr int kKmMaxK = 4096;   // centroids (LDS histogram of ints)
constexpr int kKmMaxBlocks = 256;  // row blocks per head

template <typename CT>
__global__ __launch_bounds__(256) void km_hist(const CT* __restrict__ codes, int64_t n, int k,
                                               int64_t rows_per_blk, int nblk,
                                               int* __restrict__ cnt) {
  __shared__ int h[kKmMaxK];
  const int64_t head = blockIdx.y;
  const int blk = blockIdx.x;
  const int t = threadIdx.x;
  for (int j = t; j < k; j += 256) h[j] = 0;
  __syncthreads();
  const int64_t r0 = (int64_t)blk * rows_per_blk;
  const int64_t r1 = r0 + rows_per_blk < n ? r0 + rows_per_blk : n;
  for (int64_t r = r0 + t; r < r1; r += 256) {
    const int c = (int)codes[head * n + r];
    if (c < k) atomicAdd(&h[c], 1);
  }
  __syncthreads();
  int* out = cnt + (head * nblk + blk) * (int64_t)k;
  for (int j = t; j < k; j += 256) out[j] = h[j];
}

// Codes are taken 64 at a time; thread (bg, cl) owns code j = tile + cl over the blocks
// [bg * per, (bg + 1) * per) (16 block groups), so the per-code prefix over blocks is a
// short serial run per thread plus a 16-way combine in LDS, and the prefix over codes a
// wave scan plus a running carry.
__global__ __launch_bounds__(1024) void km_offsets(const int* __restrict__ cnt, int nblk, int k,
                                                   int* __restrict__ off, int* __restrict__ base,
                                                   int* __restrict__ counts,
                                                   int32_t* __restrict__ user_counts) {
  __shared__ int s_part[16][64];
  const int64_t head = blockIdx.x;
  const int t = threadIdx.x, cl = t & 63, bg = t >> 6;
  const int per = (nblk + 15) / 16;
  const int b0 = bg * per < nblk ? bg * per : nblk;
  const int b1 = b0 + per < nblk ? b0 + per : nblk;
  int carry = 0;
  for (int j0 = 0; j0 < k; j0 += 64) {
    const int j = j0 + cl;
    int run = 0;
    if (j < k) {
#pragma unroll 8
      for (int b = b0; b < b1; ++b) {
        const int64_t e = (head * nblk + b) * (int64_t)k + j;
        const int c = cnt[e];
        off[e] = run;
        run += c;
      }
    }
    s_part[bg][cl] = run;
    __syncthreads();
    int pre = 0, tot = 0;
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      const int v = s_part[g][cl];
      pre += g < bg ? v : 0;
      tot += v;
    }
    int incl = tot;  // prefix over the tile's 64 codes (every wave holds all of them)
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl, o);
      if (cl >= o) incl += u;
    }
    const int basej = carry + incl - tot;
    if (j < k) {
#pragma unroll 8
      for (int b = b0; b < b1; ++b) off[(head * nblk + b) * (int64_t)k + j] += basej + pre;
      if (bg == 0) {
        base[head * k + j] = basej;
        counts[head * k + j] = tot;
        if (user_counts) user_counts[head * k + j] = tot;
      }
    }
    carry += __shfl(incl, 63);
    __syncthreads();  // s_part is reused by the next tile
  }
}

template <typename CT>
__global__ __launch_bounds__(1024) void km_scatter(const CT* __restrict__ codes, int64_t n, int k,
                                                   int64_t rows_per_blk, int nblk,
                                                   const int* __restrict__ off,
                                                   int* __restrict__ sorted) {
  __shared__ int run[kKmMaxK];
  const int64_t head = blockIdx.y;
  const int blk = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  for (int j = t; j < k; j += 1024) run[j] = 0;
  __syncthreads();
  const int64_t r0 = (int64_t)blk * rows_per_blk;
  const int64_t r1 = r0 + rows_per_blk < n ? r0 + rows_per_blk : n;
  const int* offb = off + (head * nblk + blk) * (int64_t)k;
  int* sh = sorted + head * n;
  const unsigned long long lt = (1ull << lane) - 1ull;
  for (int64_t c0 = r0; c0 < r1; c0 += 1024) {
    const int64_t r = c0 + t;
    const int code = r < r1 ? (int)codes[head * n + r] : k;  // k: not counted
    const bool live = code < k;
    // lanes of this wave holding the same code (ballot per code bit), live lanes only
    unsigned long long same = __ballot(live);
    for (int bit = 0; bit < 16; ++bit) {
      const unsigned long long ones = __ballot(live && ((code >> bit) & 1));
      same &= ((code >> bit) & 1) ? ones : ~ones;
    }
    const int rank = __popcll(same & lt);
    const bool leader = live && rank == 0;
    for (int w = 0; w < 16; ++w) {  // waves in order: a stable ranking across the chunk
      if (wave == w && live) {
        sh[offb[code] + run[code] + rank] = (int)r;
      }
      __syncthreads();
      if (wave == w && leader) run[code] += __popcll(same);
      __syncthreads();
    }
  }
}

// One workgroup of WAVES waves per centroid.  A cluster of m members is cut into
// S = min(WAVES, ceil(m / 256)) contiguous segments, one per wave; each wave sums its segment
// (members in sorted order, four loads in flight), and wave 0 adds the segment sums in
// segment order.  Clusters of at most 256 members are thus summed in plain ascending row
// order.
template <int DT, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void km_mean(const void* __restrict__ x, int64_t n, int d,
                                                      int k, const int* __restrict__ sorted,
                                                      const int* __restrict__ base,
                                                      const int* __restrict__ counts,
                                                      const float* __restrict__ cb_in,
                                                      float* __restrict__ cb_out) {
  __shared__ double part[WAVES][2][64];
  const int64_t head = blockIdx.y;
  const int j = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int dpl = d > 64 ? d / 64 : 1;  // dimensions per lane (1 or 2)
  const int lanes_per_row = d / dpl;    // 64 for d >= 64
  const int groups = 64 / lanes_per_row;
  const int g = lane / lanes_per_row;
  const int a0 = (lane % lanes_per_row) * dpl;
  const int m = counts[head * k + j];
  int nseg = (m + 255) / 256;
  if (nseg > WAVES) nseg = WAVES;
  if (nseg < 1) nseg = 1;
  const int seg_len = (m + nseg - 1) / nseg;
  const int i0 = wave * seg_len;
  const int i1 = i0 + seg_len < m ? i0 + seg_len : m;
  const int* mem = sorted + head * n + base[head * k + j];
  double acc0 = 0.0, acc1 = 0.0;
  if (wave < nseg) {
    int i = i0 + g;
    for (; i + 3 * groups < i1; i += 4 * groups) {
      int64_t rows[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) rows[u] = mem[i + u * groups];
      double v0[4], v1[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t xo = (head * n + rows[u]) * d + a0;
        v0[u] = (double)load_elem(x, DT, xo);
        v1[u] = dpl == 2 ? (double)load_elem(x, DT, xo + 1) : 0.0;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {  // added in member order
        acc0 += v0[u];
        acc1 += v1[u];
      }
    }
    for (; i < i1; i += groups) {
      const int64_t xo = (head * n + mem[i]) * d + a0;
      acc0 += (double)load_elem(x, DT, xo);
      if (dpl == 2) acc1 += (double)load_elem(x, DT, xo + 1);
    }
    for (int o = lanes_per_row; o < 64; o <<= 1) {  // the member subsets, in a fixed tree
      acc0 += __shfl_xor(acc0, o);
      acc1 += __shfl_xor(acc1, o);
    }
  }
  part[wave][0][lane] = acc0;
  part[wave][1][lane] = acc1;
  __syncthreads();
  if (wave == 0 && g == 0) {
    double s0 = part[0][0][lane], s1 = part[0][1][lane];
    for (int w = 1; w < nseg; ++w) {
      s0 += part[w][0][lane];
      s1 += part[w][1][lane];
    }
    float* out = cb_out + (head * k + j) * (int64_t)d + a0;
    const float* in = cb_in + (head * k + j) * (int64_t)d + a0;
    if (m > 0) {
      out[0] = (float)(s0 / (double)m);
      if (dpl == 2) out[1] = (float)(s1 / (double)m);
    } else {
      out[0] = in[0];
      if (dpl == 2) out[1] = in[1];
    }
  }
}

struct KmLayout {
  int* cnt;
  int* off;
  int* base;
  int* counts;
  int* sorted;
  size_t bytes;
};

void km_blocks(int64_t n, int64_t* rows_per_blk, int* nblk) {
  int64_t r = 1024;
  while ((n + r - 1) / r > kKmMaxBlocks) r *= 2;
  *rows_per_blk = r;
  *nblk = (int)std::max<int64_t>(1, (n + r - 1) / r);
}

KmLayout km_carve(void* ws, int64_t heads, int64_t n, int64_t k) {
  int64_t rpb;
  int nblk;
  km_blocks(n, &rpb, &nblk);
  Carver c(ws);
  KmLayout L;
  L.cnt = c.take<int>((size_t)(heads * nblk * k));
  L.off = c.take<int>((size_t)(heads * nblk * k));
  L.base = c.take<int>((size_t)(heads * k));
  L.counts = c.take<int>((size_t)(heads * k));
  L.sorted = c.take<int>((size_t)(heads * n));
  L.bytes = c.used;
  return L;
}

template <typename CT>
int km_update_impl(const void* x, int x_dtype, int64_t heads, int64_t n, int64_t d,
                   const CT* codes, int64_t k, const float* cb_in, float* cb_out,
                   int32_t* counts, const KmLayout& L, hipStream_t s) {
  int64_t rpb;
  int nblk;
  km_blocks(n, &rpb, &nblk);
  A2ATS_TRY(launch("kmeans_hist", km_hist<CT>, dim3((unsigned)nblk, (unsigned)heads), dim3(256), 0,
                   s, codes, n, (int)k, rpb, nblk, L.cnt));
  A2ATS_TRY(launch("kmeans_offsets", km_offsets, dim3((unsigned)heads), dim3(1024), 0, s, L.cnt,
                   nblk, (int)k, L.off, L.base, L.counts, counts));
  A2ATS_TRY(launch("kmeans_scatter", km_scatter<CT>, dim3((unsigned)nblk, (unsigned)heads),
                   dim3(1024), 0, s, codes, n, (int)k, rpb, nblk, L.off, L.sorted));
  const dim3 g((unsigned)k, (unsigned)heads);
  // large clusters (the pooled sub-vector codebooks: thousands of members each) get 16
  // segment waves per centroid, small ones 4
  const bool big = n / k >= 1024;
#define A2ATS_KM_MEAN(DTV, WV)                                                                   \
  launch("kmeans_mean", km_mean<DTV, WV>, g, dim3(WV * 64), 0, s, x, n, (int)d, (int)k, L.sorted, \
         L.base, L.counts, cb_in, cb_out)
  if (x_dtype == A2ATS_BF16)
    A2ATS_TRY(big ? A2ATS_KM_MEAN(A2ATS_BF16, 16) : A2ATS_KM_MEAN(A2ATS_BF16, 4));
  else
    A2ATS_TRY(big ? A2ATS_KM_MEAN(A2ATS_F32, 16) : A2ATS_KM_MEAN(A2ATS_F32, 4));
#undef A2ATS_KM_MEAN
  return A2ATS_OK;
}

bool km_shape_ok(int64_t heads, int64_t n, int64_t d, int64_t k) {
  if (heads < 1 || heads > 65535 || n < 0 || n > 0x7FFFFFFF || k < 1 || k > kKmMaxK) return false;
  return d == 4 || d == 8 || d == 16 || d == 32 || d == 64 || d == 128;
}

}  // namespace
}  // namespace a2ats

using namespace a2ats;

extern "C" size_t a2ats_kmeans_update_workspace(int64_t heads, int64_t n, int64_t k) {
  if (heads < 1 || n < 0 || k < 1) return 0;
  return km_carve(nullptr, heads, n, k).bytes;
}

extern "C" int a2ats_kmeans_update(const void* x, int x_dtype, int64_t heads, int64_t n,
                                   int64_t d, const void* codes, int codes_bytes, int64_t k,
                                   const float* codebook_in, float* codebook_out,
                                   int32_t* counts, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  if (x_dtype != A2ATS_F32 && x_dtype != A2ATS_BF16) return A2ATS_EDTYPE;
  if (codes_bytes != 1 && codes_bytes != 2) return A2ATS_EDTYPE;
  if (!km_shape_ok(heads, n, d, k)) return A2ATS_EINVAL;
  if (codes_bytes == 1 && k > 256) return A2ATS_EINVAL;
  if (!x || !codes || !codebook_in || !codebook_out) return A2ATS_EINVAL;
  const size_t need = a2ats_kmeans_update_workspace(heads, n, k);
  if (!ws_ok(workspace, workspace_bytes, need)) return A2ATS_EWORKSPACE;
  const KmLayout L = km_carve(workspace, heads, n, k);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (codes_bytes == 2)
    return km_update_impl<uint16_t>(x, x_dtype, heads, n, d, static_cast<const uint16_t*>(codes),
                                    k, codebook_in, codebook_out, counts, L, s);
  return km_update_impl<uint8_t>(x, x_dtype, heads, n, d, static_cast<const uint8_t*>(codes), k,
                                 codebook_in, codebook_out, counts, L, s);
}

// Lloyd's iterations on the device: `iters` rounds of (exact assignment, member-mean update),
// then the final assignment.  d = 128: whole head vectors of `heads` heads, per-head codebooks
// and L (a2ats_encode; codes uint16 [heads, n]).  d = 4 or 8: one shared codebook over pooled
// sub-vectors (heads must be 1, n a multiple of 128 / d; a2ats_pq_encode on the rows viewed
// as [n d / 128, 128]; codes uint8 [n]).
extern "C" size_t a2ats_kmeans_workspace(int64_t heads, int64_t n, int64_t d, int64_t k) {
  if (heads < 1 || n < 0 || k < 1) return 0;
  size_t enc = 0;
  if (d == A2ATS_HEAD_DIM) enc = align_up(a2ats_encode_workspace(heads, n, d, k));
  return enc + a2ats_kmeans_update_workspace(heads, n, k);
}

extern "C" int a2ats_kmeans(const void* x, int x_dtype, int64_t heads, int64_t n, int64_t d,
                            int64_t k, const float* chol, int iters, float* codebook, void* codes,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (x_dtype != A2ATS_F32 && x_dtype != A2ATS_BF16) return A2ATS_EDTYPE;
  const bool whole = d == A2ATS_HEAD_DIM;
  if (!whole && !(d == 4 || d == 8)) return A2ATS_EINVAL;
  if (!km_shape_ok(heads, n, d, k) || iters < 0) return A2ATS_EINVAL;
  if (!whole && (heads != 1 || k > 256 || n % (A2ATS_HEAD_DIM / d) != 0)) return A2ATS_EINVAL;
  if (!x || !codebook || !codes) return A2ATS_EINVAL;
  if (n == 0) return A2ATS_OK;
  const size_t need = a2ats_kmeans_workspace(heads, n, d, k);
  if (!ws_ok(workspace, workspace_bytes, need)) return A2ATS_EWORKSPACE;
  const size_t enc = whole ? align_up(a2ats_encode_workspace(heads, n, d, k)) : 0;
  void* ws_km = static_cast<char*>(workspace) + enc;
  const size_t wsb_km = workspace_bytes - enc;
  const int64_t rows128 = whole ? n : n * d / A2ATS_HEAD_DIM;
  auto assign = [&]() -> int {
    if (whole)
      return a2ats_encode(x, x_dtype, heads, n, d, nullptr, 0, codebook, k, chol,
                          static_cast<uint16_t*>(codes), nullptr, nullptr, workspace, enc, stream);
    return a2ats_pq_encode(x, x_dtype, 1, rows128, A2ATS_HEAD_DIM, d, nullptr, 0, codebook, k,
                           chol, nullptr, 0, 0.0, static_cast<uint8_t*>(codes), stream);
  };
  for (int it = 0; it < iters; ++it) {
    A2ATS_TRY(assign());
    A2ATS_TRY(a2ats_kmeans_update(x, x_dtype, heads, n, d, codes, whole ? 2 : 1, k, codebook,
                                  codebook, nullptr, ws_km, wsb_km, stream));
  }
  return assign();
}
