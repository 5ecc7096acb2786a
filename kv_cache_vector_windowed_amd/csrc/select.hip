// select_retrieval: per head, the ceil(f * n) keys with the largest cosine to the proxy
// query form the retrieval set, the rest the bulk; both outputs ascending.
// "veloxquant_mlx.quantizers.a2ats module", a2ats_select_retrieval_set.
//
// Ranking score: s = k.q / ||k|| in fp32 (||q|| is constant per head).  Each score is
// mapped to an order-preserving 32-bit key u; the selection order is the 64-bit key
// (u << 32) | (0xffffffff - index), so equal scores keep the lower index first and every
// element has a distinct key.
//
// Kernels (6 launches, no host round trip, no workgroup waits for another):
//   sel_init     per head: ||q|| and the binning scale; zeroes histograms and counters.
//   sel_score    HBM-bound pass over the keys (8 lanes per key, 4 keys in flight per lane
//                group): writes u.
//   sel_hist     1024-bin histogram of a monotone binning of s/||q|| in [-1, 1] from the
//                L2/MALL-resident scores (LDS histograms, one global atomic per non-empty
//                bin and workgroup); the last workgroup of each head (fenced atomic counter,
//                no waiting) finds, with a parallel prefix sum, the bin b* that holds the
//                n_r-th largest score.
//   sel_collect  pass over u: per block of 1024 scores, the count above b* and the keys in
//                b* (into the block's own region of the candidate array).
//   sel_thresh   one workgroup per head: the exact n_r-th largest 64-bit key among the
//                candidates, the selected candidates per block, and every block's output
//                offset (parallel prefix sums).
//   sel_scatter  pass over u: ordered compaction of the predicate key64 >= threshold into
//                the retrieval and bulk index arrays.
#include "common.hpp"

namespace a2ats {
namespace {

typedef unsigned u4v __attribute__((ext_vector_type(4)));
typedef float f4v __attribute__((ext_vector_type(4)));

constexpr int kD = A2ATS_HEAD_DIM;
constexpr int kBins = 1024;
constexpr float kHalfBins = 512.0f;
constexpr int kHistScores = 16384;  // scores per sel_hist workgroup (at most 64 per head)
constexpr int kScoreChunk = 512;    // keys per sel_score workgroup
constexpr int kScoreUnroll = 4;     // keys in flight per 8-lane group
constexpr int kBlock = 1024;        // scores per sel_collect / sel_scatter workgroup
constexpr int kSortCap = 4096;      // candidates sorted in LDS; more take the radix path

struct HeadInfo {
  float inv_scale;       // (kBins / 2) / ||q||, or 0 when q == 0
  int n_r;               // retrieval-set size
  int bstar;             // bin holding the n_r-th largest score (kBins: nothing selected)
  int count_above;       // keys in bins above bstar
  int n_cand;            // unused
  unsigned done_score;   // workgroups of sel_hist finished
  unsigned done_collect; // unused
  int pad;
  unsigned long long thr; // 64-bit key of the n_r-th largest element
};

__device__ __forceinline__ unsigned order_key(float s) {
  if (s == 0.0f) s = 0.0f;  // -0 and +0 rank equal
  unsigned b = __float_as_uint(s);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float key_value(unsigned u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// Monotone non-decreasing in s: a positive scale, an add and floor all preserve order.
__device__ __forceinline__ int bin_of(unsigned u, float inv_scale) {
  float s = key_value(u);
  float v = floorf(__fmaf_rn(s, inv_scale, kHalfBins));  // one rounding, identical everywhere
  v = fminf(fmaxf(v, 0.0f), (float)(kBins - 1));
  return (int)v;
}

__device__ __forceinline__ unsigned long long key64(unsigned u, int64_t idx) {
  return ((unsigned long long)u << 32) | (unsigned long long)(0xFFFFFFFFu - (unsigned)idx);
}

__device__ __forceinline__ unsigned atomic_load_u32(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(256) void sel_init(const void* __restrict__ query, int dt, int64_t n,
                                                double fraction, HeadInfo* __restrict__ info,
                                                unsigned* __restrict__ hist,
                                                unsigned* __restrict__ sel_extra, int nblk) {
  const int head = blockIdx.x;
  const int t = threadIdx.x;
  __shared__ float red[4];
  float v = 0.f;
  if (t < kD) {
    float x = load_elem(query, dt, (int64_t)head * kD + t);
    v = x * x;
  }
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if ((t & 63) == 0) red[t >> 6] = v;
  __syncthreads();
  for (int i = t; i < kBins; i += 256) hist[(int64_t)head * kBins + i] = 0u;
  for (int i = t; i < nblk; i += 256) sel_extra[(int64_t)head * nblk + i] = 0u;
  if (t == 0) {
    float qn = sqrtf(red[0] + red[1] + red[2] + red[3]);
    HeadInfo h;
    h.inv_scale = qn > 0.f ? kHalfBins / qn : 0.f;
    h.n_r = (int)ceil(fraction * (double)n);
    h.bstar = kBins;
    h.count_above = 0;
    h.n_cand = 0;
    h.done_score = 0u;
    h.done_collect = 0u;
    h.pad = 0;
    h.thr = ~0ull;
    info[head] = h;
  }
}

// Exclusive prefix sum over the 256 threads of a workgroup (thread order); returns the sum of
// the threads before this one and, in *total, the workgroup sum.
__device__ __forceinline__ unsigned block_exclusive_scan(unsigned v, unsigned* total) {
  __shared__ unsigned wsum[4];
  const int t = threadIdx.x, lane = t & 63;
  unsigned incl = v;
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned u = __shfl_up(incl, o);
    if (lane >= o) incl += u;
  }
  __syncthreads();
  if (lane == 63) wsum[t >> 6] = incl;
  __syncthreads();
  unsigned before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    before += w < (t >> 6) ? wsum[w] : 0u;
    all += wsum[w];
  }
  *total = all;
  return before + incl - v;
}

// 8 lanes per key; each lane covers 16 consecutive elements of the 128.
template <int DT>
__global__ __launch_bounds__(256) void sel_score(const void* __restrict__ keys,
                                                 const void* __restrict__ query, int64_t n,
                                                 int wg_per_head, unsigned* __restrict__ scores) {
  const int head = blockIdx.x / wg_per_head;
  const int wg = blockIdx.x % wg_per_head;
  const int t = threadIdx.x;
  const int sub = t & 7;
  float qv[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) qv[e] = load_elem(query, DT, (int64_t)head * kD + sub * 16 + e);
  const int64_t k_begin = (int64_t)wg * kScoreChunk;
  const int64_t k_end = k_begin + kScoreChunk < n ? k_begin + kScoreChunk : n;
  const int64_t hoff = (int64_t)head * n;
  for (int64_t k0 = k_begin; k0 < k_end; k0 += 32 * kScoreUnroll) {
    float x[kScoreUnroll][16];
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u) {  // issue every load first
      const int64_t key = k0 + u * 32 + (t >> 3);
      if (key < k_end) {
        if (DT == A2ATS_BF16) {
          const u4v* p = reinterpret_cast<const u4v*>(static_cast<const uint16_t*>(keys) +
                                                      (hoff + key) * kD + sub * 16);
          const u4v r0 = p[0], r1 = p[1];
          const unsigned w[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            x[u][2 * e] = __uint_as_float(w[e] << 16);
            x[u][2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
          }
        } else {
          const f4v* p = reinterpret_cast<const f4v*>(static_cast<const float*>(keys) +
                                                      (hoff + key) * kD + sub * 16);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f4v a = p[q];
            x[u][4 * q] = a.x; x[u][4 * q + 1] = a.y; x[u][4 * q + 2] = a.z; x[u][4 * q + 3] = a.w;
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) x[u][e] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u) {
      float dot = 0.f, nrm = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        dot += x[u][e] * qv[e];
        nrm += x[u][e] * x[u][e];
      }
#pragma unroll
      for (int o = 4; o > 0; o >>= 1) {
        dot += __shfl_xor(dot, o);
        nrm += __shfl_xor(nrm, o);
      }
      const int64_t key = k0 + u * 32 + (t >> 3);
      if (sub == 0 && key < k_end) {
        const float sc = nrm > 0.f ? dot / sqrtf(nrm) : 0.f;
        scores[hoff + key] = order_key(sc);
      }
    }
  }
}

// Histogram of the binned scores from the L2/MALL-resident score array: kHistScores
// scores per workgroup into an LDS histogram, one global atomic per non-empty bin (the
// scores of a head fall into a few hundred bins); the last workgroup of each head (fenced
// counter, no waiting) finds, with a parallel prefix sum, the bin b* holding the n_r-th
// largest score.
__global__ __launch_bounds__(256) void sel_hist(const unsigned* __restrict__ scores, int64_t n,
                                                int wg_per_head, HeadInfo* __restrict__ info,
                                                unsigned* __restrict__ hist) {
  const int head = blockIdx.x / wg_per_head;
  const int wg = blockIdx.x % wg_per_head;
  const int t = threadIdx.x;
  __shared__ unsigned lh[kBins];
  __shared__ int is_last;
  for (int i = t; i < kBins; i += 256) lh[i] = 0u;
  const float inv = info[head].inv_scale;
  unsigned* hh = hist + (int64_t)head * kBins;
  __syncthreads();
  const int64_t per = ((n + wg_per_head - 1) / wg_per_head + 3) / 4 * 4;
  const int64_t i_begin = (int64_t)wg * per;
  const int64_t i_end = i_begin + per < n ? i_begin + per : n;
  const int64_t hoff = (int64_t)head * n;
  for (int64_t i0 = i_begin + 4 * t; i0 < i_end; i0 += 1024) {
    if (i0 + 3 < i_end && ((hoff + i0) & 3) == 0) {
      const uint4 q = *reinterpret_cast<const uint4*>(scores + hoff + i0);
      atomicAdd(&lh[bin_of(q.x, inv)], 1u);
      atomicAdd(&lh[bin_of(q.y, inv)], 1u);
      atomicAdd(&lh[bin_of(q.z, inv)], 1u);
      atomicAdd(&lh[bin_of(q.w, inv)], 1u);
    } else {
      for (int k = 0; k < 4 && i0 + k < i_end; ++k)
        atomicAdd(&lh[bin_of(scores[hoff + i0 + k], inv)], 1u);
    }
  }
  __syncthreads();
  for (int i = t; i < kBins; i += 256)
    if (lh[i]) atomicAdd(&hh[i], lh[i]);
  __threadfence();
  __syncthreads();
  if (t == 0) is_last = (atomicAdd(&info[head].done_score, 1u) == (unsigned)wg_per_head - 1);
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  // Last workgroup of this head: thread t owns the 4 bins kBins-4(t+1) .. kBins-4t-1, taken
  // in descending order; a prefix sum over the threads finds the bin of the n_r-th largest.
  const int n_r = info[head].n_r;
  const uint4 v = *reinterpret_cast<const uint4*>(hh + kBins - 4 * (t + 1));  // plain load: fenced
  const unsigned c4[4] = {v.w, v.z, v.y, v.x};
  const unsigned s4 = c4[0] + c4[1] + c4[2] + c4[3];
  unsigned total;
  unsigned cum = block_exclusive_scan(s4, &total);
  if (n_r > 0 && cum < (unsigned)n_r && cum + s4 >= (unsigned)n_r) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (cum < (unsigned)n_r && cum + c4[i] >= (unsigned)n_r) {
        info[head].bstar = kBins - 1 - 4 * t - i;
        info[head].count_above = (int)cum;
      }
      cum += c4[i];
    }
  }
}

// Per block of kBlock scores: the count above b* and the keys in b*, appended to the
// block's own region of the candidate array (no global atomics).
__global__ __launch_bounds__(256) void sel_collect(const unsigned* __restrict__ scores, int64_t n,
                                                   int nblk, const HeadInfo* __restrict__ info,
                                                   unsigned* __restrict__ above_blk,
                                                   unsigned* __restrict__ cand_blk,
                                                   unsigned long long* __restrict__ cand) {
  const int head = blockIdx.x / nblk;
  const int blk = blockIdx.x % nblk;
  const int t = threadIdx.x;
  const int bstar = info[head].bstar;
  const float inv = info[head].inv_scale;
  const int64_t hoff = (int64_t)head * n;
  const int64_t i_begin = (int64_t)blk * kBlock;
  const int64_t i_end = i_begin + kBlock < n ? i_begin + kBlock : n;
  unsigned above = 0;
  __shared__ unsigned s_cnt;
  __shared__ unsigned red[4];
  if (t == 0) s_cnt = 0u;
  __syncthreads();
  const int64_t i0 = i_begin + 4 * t;  // 4 consecutive scores per thread
  unsigned uv[4];
  if (i0 + 3 < i_end && ((hoff + i0) & 3) == 0) {
    const uint4 q = *reinterpret_cast<const uint4*>(scores + hoff + i0);
    uv[0] = q.x; uv[1] = q.y; uv[2] = q.z; uv[3] = q.w;
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) uv[k] = (i0 + k < i_end) ? scores[hoff + i0 + k] : 0u;
  }
  unsigned mine = 0, local = 0;  // candidates of this thread, and their slot base
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (i0 + k < i_end) {
      const int b = bin_of(uv[k], inv);
      if (b > bstar) above += 1;
      if (b == bstar) mine |= 1u << k;
    }
  }
  if (mine) local = atomicAdd(&s_cnt, (unsigned)__popc(mine));
  for (int k = 0; k < 4; ++k)
    if (mine & (1u << k)) cand[hoff + i_begin + local++] = key64(uv[k], i0 + k);
  for (int o = 32; o > 0; o >>= 1) above += __shfl_xor(above, o);
  if ((t & 63) == 0) red[t >> 6] = above;
  __syncthreads();
  if (t == 0) {
    above_blk[(int64_t)head * nblk + blk] = red[0] + red[1] + red[2] + red[3];
    cand_blk[(int64_t)head * nblk + blk] = s_cnt;
  }
}

// One workgroup per head: the exact n_r-th largest 64-bit key among the candidates of bin
// b* (LDS bitonic sort, radix select beyond kSortCap), the selected candidates per block,
// and the exclusive output offset of every block (parallel prefix sums).
__global__ __launch_bounds__(256) void sel_thresh(int64_t n, int nblk, HeadInfo* __restrict__ info,
                                                  const unsigned* __restrict__ above_blk,
                                                  const unsigned* __restrict__ cand_blk,
                                                  const unsigned long long* __restrict__ cand,
                                                  unsigned* __restrict__ sel_extra) {
  const int head = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t hoff = (int64_t)head * n;
  const int r = info[head].n_r - info[head].count_above;  // 1-based rank inside bin b*
  __shared__ unsigned long long sk[kSortCap];
  // candidate count, and (when they fit) the candidates packed into LDS in block order
  unsigned n_cand = 0;
  for (int b0 = 0; b0 < nblk; b0 += 256) {
    const int b = b0 + t;
    const unsigned cb = b < nblk ? cand_blk[(int64_t)head * nblk + b] : 0u;
    unsigned chunk;
    const unsigned ex = block_exclusive_scan(cb, &chunk);
    if (n_cand + ex + cb <= (unsigned)kSortCap)
      for (unsigned i = 0; i < cb; ++i) sk[n_cand + ex + i] = cand[hoff + (int64_t)b * kBlock + i];
    n_cand += chunk;
  }
  __syncthreads();
  __shared__ unsigned dh[256];
  __shared__ unsigned long long s_prefix;
  __shared__ unsigned s_remaining;
  unsigned long long prefix = 0ull, mask = 0ull;
  if (t == 0) s_remaining = (unsigned)(r > 0 ? r : 0);
  __syncthreads();
  const bool fits = n_cand <= (unsigned)kSortCap;
  if (r > 0 && fits) {
    // bitonic sort of the candidate keys, descending; the r-th is the threshold
    int P = 1;
    while (P < (int)n_cand) P <<= 1;
    for (int i = (int)n_cand + t; i < P; i += 256) sk[i] = 0ull;
    __syncthreads();
    for (int k = 2; k <= P; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = t; i < P; i += 256) {
          const int l = i ^ j;
          if (l > i) {
            const unsigned long long a = sk[i], b = sk[l];
            const bool desc = (i & k) == 0;
            if (desc ? (a < b) : (a > b)) {
              sk[i] = b;
              sk[l] = a;
            }
          }
        }
        __syncthreads();
      }
    }
    prefix = sk[r - 1];
  } else if (r > 0) {
    // radix select over the per-block candidate regions, 8 bits at a time
    for (int shift = 56; shift >= 0; shift -= 8) {
      dh[t] = 0u;
      __syncthreads();
      for (int b = t; b < nblk; b += 256) {
        const unsigned cb = cand_blk[(int64_t)head * nblk + b];
        for (unsigned i = 0; i < cb; ++i) {
          const unsigned long long kv = cand[hoff + (int64_t)b * kBlock + i];
          if ((kv & mask) == prefix) atomicAdd(&dh[(kv >> shift) & 0xFF], 1u);
        }
      }
      __syncthreads();
      {  // digit holding the rem-th largest: thread t takes digit 255 - t (descending)
        const unsigned rem = s_remaining;
        const unsigned cdg = dh[255 - t];
        unsigned all;
        const unsigned cum = block_exclusive_scan(cdg, &all);
        if (cum < rem && cum + cdg >= rem) {
          s_remaining = rem - cum;
          s_prefix = prefix | ((unsigned long long)(255 - t) << shift);
        }
      }
      __syncthreads();
      prefix = s_prefix;
      mask |= 0xFFull << shift;
      __syncthreads();
    }
  }
  const unsigned long long thr = r > 0 ? prefix : ~0ull;
  if (t == 0) info[head].thr = thr;
  // selected candidates per block
  if (r > 0) {
    if (fits) {
      for (int i = t; i < (int)n_cand; i += 256) {
        const unsigned long long kv = sk[i];
        if (kv >= thr) {
          const int64_t idx = (int64_t)(0xFFFFFFFFu - (unsigned)(kv & 0xFFFFFFFFull));
          atomicAdd(&sel_extra[(int64_t)head * nblk + idx / kBlock], 1u);
        }
      }
    } else {
      for (int b = t; b < nblk; b += 256) {
        const unsigned cb = cand_blk[(int64_t)head * nblk + b];
        unsigned sel = 0;
        for (unsigned i = 0; i < cb; ++i) sel += cand[hoff + (int64_t)b * kBlock + i] >= thr ? 1u : 0u;
        if (sel) atomicAdd(&sel_extra[(int64_t)head * nblk + b], sel);
      }
    }
  }
  __threadfence();
  __syncthreads();
  // exclusive offsets over the blocks, 256 at a time (atomic loads for the counters this
  // workgroup just incremented)
  unsigned run = 0;
  for (int b0 = 0; b0 < nblk; b0 += 256) {
    const int b = b0 + t;
    const unsigned cntb = b < nblk ? above_blk[(int64_t)head * nblk + b] +
                                         atomic_load_u32(&sel_extra[(int64_t)head * nblk + b])
                                   : 0u;
    unsigned chunk;
    const unsigned ex = block_exclusive_scan(cntb, &chunk);
    if (b < nblk) sel_extra[(int64_t)head * nblk + b] = run + ex;  // the exclusive offset
    run += chunk;
  }
}

__global__ __launch_bounds__(256) void sel_scatter(const unsigned* __restrict__ scores, int64_t n,
                                                   int nblk, const HeadInfo* __restrict__ info,
                                                   const unsigned* __restrict__ offsets,
                                                   int32_t* __restrict__ ret,
                                                   int32_t* __restrict__ bulk) {
  const int head = blockIdx.x / nblk;
  const int blk = blockIdx.x % nblk;
  const int t = threadIdx.x;
  const int bstar = info[head].bstar;
  const float inv = info[head].inv_scale;
  const unsigned long long thr = info[head].thr;
  const int n_r = info[head].n_r;
  const int64_t hoff = (int64_t)head * n;
  const int64_t i_begin = (int64_t)blk * kBlock;
  constexpr int kPer = kBlock / 256;  // consecutive elements per thread
  const int64_t my0 = i_begin + (int64_t)t * kPer;
  unsigned flags = 0;
  int cnt = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int64_t i = my0 + k;
    if (i < n) {
      const unsigned u = scores[hoff + i];
      const int b = bin_of(u, inv);
      const bool sel = b > bstar || (b == bstar && key64(u, i) >= thr);
      if (sel) {
        flags |= 1u << k;
        ++cnt;
      }
    }
  }
  // exclusive scan of cnt over the workgroup (thread order = index order)
  __shared__ int wsum[4];
  int incl = cnt;
  const int lane = t & 63;
  for (int o = 1; o < 64; o <<= 1) {
    int v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wsum[t >> 6] = incl;
  __syncthreads();
  int wbase = 0;
  for (int w = 0; w < (t >> 6); ++w) wbase += wsum[w];
  const int64_t sel_before = (int64_t)offsets[(int64_t)head * nblk + blk] + wbase + incl - cnt;
  int64_t rpos = sel_before;
  int64_t bpos = my0 - sel_before;  // non-selected before my0
  int32_t* rh = ret + (int64_t)head * n_r;
  int32_t* bh = bulk + (int64_t)head * (n - n_r);
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int64_t i = my0 + k;
    if (i < n) {
      // bounds guards: the counts are consistent by construction, the guards keep any
      // inconsistency a wrong answer instead of an out-of-bounds store
      if (flags & (1u << k)) {
        if (rpos < n_r) rh[rpos] = (int32_t)i;
        ++rpos;
      } else {
        if (bpos < n - n_r) bh[bpos] = (int32_t)i;
        ++bpos;
      }
    }
  }
}

struct SelLayout {
  HeadInfo* info;
  unsigned* hist;
  unsigned* scores;
  unsigned long long* cand;
  unsigned* above_blk;
  unsigned* cand_blk;
  unsigned* sel_extra;
  size_t bytes;
};

SelLayout carve(void* ws, int64_t heads, int64_t n) {
  const int64_t nblk = (n + kBlock - 1) / kBlock;
  Carver c(ws);
  SelLayout L;
  L.info = c.take<HeadInfo>((size_t)heads);
  L.hist = c.take<unsigned>((size_t)heads * kBins);
  L.scores = c.take<unsigned>((size_t)heads * n);
  L.cand = c.take<unsigned long long>((size_t)heads * n);
  L.above_blk = c.take<unsigned>((size_t)heads * nblk);
  L.cand_blk = c.take<unsigned>((size_t)heads * nblk);
  L.sel_extra = c.take<unsigned>((size_t)heads * nblk);
  L.bytes = c.used;
  return L;
}

}  // namespace
}  // namespace a2ats

using namespace a2ats;

extern "C" size_t a2ats_select_retrieval_workspace(int64_t heads, int64_t n) {
  if (heads < 1 || n < 0) return 0;
  return carve(nullptr, heads, n).bytes;
}

extern "C" int a2ats_select_retrieval(const void* keys, int keys_dtype, int64_t heads, int64_t n,
                                      int64_t d, const void* query, double fraction,
                                      int32_t* retrieval_idx, int32_t* bulk_idx, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  if (keys_dtype != A2ATS_F32 && keys_dtype != A2ATS_BF16) return A2ATS_EDTYPE;
  if (d != kD || heads < 1 || n < 0 || n > 0x7FFFFFFF) return A2ATS_EINVAL;
  const int64_t n_r = a2ats_retrieval_count(n, fraction);
  if (n_r < 0) return A2ATS_EINVAL;
  if (n == 0) return A2ATS_OK;
  if (!keys || !query) return A2ATS_EINVAL;
  if ((n_r > 0 && !retrieval_idx) || (n_r < n && !bulk_idx)) return A2ATS_EINVAL;
  const int64_t wg_per_head = (n + kScoreChunk - 1) / kScoreChunk;
  const int64_t nblk = (n + kBlock - 1) / kBlock;
  if (heads * wg_per_head > 0x7FFFFFFF || heads > 65535) return A2ATS_EINVAL;
  const size_t need = a2ats_select_retrieval_workspace(heads, n);
  if (!ws_ok(workspace, workspace_bytes, need)) return A2ATS_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  SelLayout L = carve(workspace, heads, n);
  A2ATS_TRY(launch("select_init", sel_init, dim3((unsigned)heads), dim3(256), 0, s, query,
                   keys_dtype, n, fraction, L.info, L.hist, L.sel_extra, (int)nblk));
  if (keys_dtype == A2ATS_BF16)
    A2ATS_TRY(launch("select_score", sel_score<A2ATS_BF16>, dim3((unsigned)(heads * wg_per_head)),
                     dim3(256), 0, s, keys, query, n, (int)wg_per_head, L.scores));
  else
    A2ATS_TRY(launch("select_score", sel_score<A2ATS_F32>, dim3((unsigned)(heads * wg_per_head)),
                     dim3(256), 0, s, keys, query, n, (int)wg_per_head, L.scores));
  const int64_t hist_wg = std::min<int64_t>(64, std::max<int64_t>(1, (n + kHistScores - 1) / kHistScores));
  A2ATS_TRY(launch("select_hist", sel_hist, dim3((unsigned)(heads * hist_wg)), dim3(256), 0, s,
                   L.scores, n, (int)hist_wg, L.info, L.hist));
  A2ATS_TRY(launch("select_collect", sel_collect, dim3((unsigned)(heads * nblk)), dim3(256), 0, s,
                   L.scores, n, (int)nblk, L.info, L.above_blk, L.cand_blk, L.cand));
  A2ATS_TRY(launch("select_thresh", sel_thresh, dim3((unsigned)heads), dim3(256), 0, s, n, (int)nblk,
                   L.info, L.above_blk, L.cand_blk, L.cand, L.sel_extra));
  return launch("select_scatter", sel_scatter, dim3((unsigned)(heads * nblk)), dim3(256), 0, s,
                L.scores, n, (int)nblk, L.info, L.sel_extra, retrieval_idx, bulk_idx);
}
