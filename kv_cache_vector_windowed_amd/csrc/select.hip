// select_retrieval: per head, the ceil(f * n) keys with the largest cosine to the proxy
// query form the retrieval set, the rest the bulk; both outputs ascending.
// "veloxquant_mlx.quantizers.a2ats module", a2ats_select_retrieval_set.
//
// Ranking score: s = k.q / ||k|| in fp32 (||q|| is constant per head).  Each score is
// mapped to an order-preserving 32-bit key u; the selection order is the 64-bit key
// (u << 32) | (0xffffffff - index), so equal scores keep the lower index first and every
// element has a distinct key.
//
// Kernels (4 launches, no host round trip, no workgroup waits for another, no global atomics):
//   sel_score    HBM-bound pass over the keys (8 lanes per key, 2 keys in flight per lane
//                group): writes u, and the workgroup's 1024-bin histogram of a monotone
//                binning of s/||q|| in [-1, 1] (LDS counts, written out whole; at most 64
//                workgroups per head), with its 32 coarse counts of 32 bins each.
//   sel_collect  pass over u: every workgroup first finds the bin b* that holds the n_r-th
//                largest score from the partial histograms (coarse counts, then the fine
//                counts of one coarse bin: 16 KB of reads), then, per block of 1024 scores,
//                counts the keys above b* and writes those in b* (into the block's own
//                region of the candidate array).
//   sel_thresh   one workgroup per head: the exact n_r-th largest 64-bit key among the
//                candidates (gathered into LDS in parallel; rank counting, a bitonic sort,
//                or a radix select when they do not fit), the selected count of every block
//                from the block-ordered copy, and every block's output offset (parallel
//                prefix sums).
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
constexpr int kScoreWgPerHead = 64; // at most this many sel_score workgroups (partial histograms) per head
constexpr int kScoreMinKeys = 512;  // and at least this many keys per workgroup
constexpr int kScoreUnroll = 2;     // keys in flight per 8-lane group
constexpr int kScoreThreads = 512;  // sel_score workgroup size
constexpr int kBlock = 1024;        // scores per sel_collect / sel_scatter workgroup
constexpr int kSortCap = 4096;      // candidates sorted in LDS; more take the radix path
constexpr int kOffCap = 4096;       // blocks whose candidate offsets fit in LDS (n <= 4M)
constexpr int kRankCap = 1024;      // up to this many candidates: rank counting instead of a sort
constexpr int kCoarse = 32;         // coarse bins (of kBins / kCoarse bins each) for the b* search

struct HeadInfo {
  float inv_scale;        // (kBins / 2) / ||q||, or 0 when q == 0
  int n_r;                // retrieval-set size
  int bstar;              // bin holding the n_r-th largest score (kBins: nothing selected)
  int count_above;        // keys in bins above bstar
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

// Exclusive prefix sum over the NT threads of a workgroup (thread order); returns the sum of
// the threads before this one and, in *total, the workgroup sum.  Every thread must call it.
template <int NT = 256>
__device__ __forceinline__ unsigned block_exclusive_scan(unsigned v, unsigned* total) {
  constexpr int kW = NT / 64;
  __shared__ unsigned wsum[kW];
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
  for (int w = 0; w < kW; ++w) {
    before += w < (t >> 6) ? wsum[w] : 0u;
    all += wsum[w];
  }
  *total = all;
  return before + incl - v;
}

// 8 lanes per key; each lane covers 16 consecutive elements of the 128.  Workgroup wg of a
// head scores keys [wg * per_wg, (wg + 1) * per_wg) and writes their histogram (all kBins
// counts) to part[head][wg].  ||q|| is formed identically in every workgroup (the same
// sums in the same order), and workgroup 0 of the head publishes the binning scale.  The
// raw key words are held until every load of a round is issued (bf16: 8 registers a key
// per lane), so that kScoreUnroll keys per lane group are in flight.
template <int DT>
__global__ __launch_bounds__(kScoreThreads) void sel_score(const void* __restrict__ keys,
                                                           const void* __restrict__ query,
                                                           int64_t n, int wg_per_head,
                                                           int64_t per_wg,
                                                           unsigned* __restrict__ scores,
                                                           unsigned* __restrict__ part,
                                                           unsigned* __restrict__ coarse,
                                                           HeadInfo* __restrict__ info) {
  constexpr int kKeysPerRound = kScoreThreads / 8;
  constexpr int kWords = DT == A2ATS_BF16 ? 2 : 4;  // 16-byte words per lane and key
  const int head = blockIdx.x / wg_per_head;
  const int wg = blockIdx.x % wg_per_head;
  const int t = threadIdx.x;
  const int sub = t & 7;
  __shared__ unsigned lh[kBins];
  for (int i = t; i < kBins; i += kScoreThreads) lh[i] = 0u;
  float qv[16];
  float qq = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    qv[e] = load_elem(query, DT, (int64_t)head * kD + sub * 16 + e);
    qq += qv[e] * qv[e];
  }
  // butterfly sums are commutative pairwise, so every lane ends with the same value
#pragma unroll
  for (int o = 4; o > 0; o >>= 1) qq += __shfl_xor(qq, o);
  const float qn = sqrtf(qq);
  const float inv = qn > 0.f ? kHalfBins / qn : 0.f;
  if (wg == 0 && t == 0) info[head].inv_scale = inv;
  __syncthreads();
  const int64_t k_begin = (int64_t)wg * per_wg;
  const int64_t k_end = k_begin + per_wg < n ? k_begin + per_wg : n;
  const int64_t hoff = (int64_t)head * n;
  const char* kbase = static_cast<const char*>(keys) + sub * 16 * (DT == A2ATS_BF16 ? 2 : 4);
  constexpr int kRowBytes = kD * (DT == A2ATS_BF16 ? 2 : 4);
  for (int64_t k0 = k_begin; k0 < k_end; k0 += kKeysPerRound * kScoreUnroll) {
    u4v raw[kScoreUnroll][kWords];
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u) {  // issue every load first
      const int64_t key = k0 + u * kKeysPerRound + (t >> 3);
      const u4v* p = reinterpret_cast<const u4v*>(kbase + (hoff + key) * kRowBytes);
#pragma unroll
      for (int q = 0; q < kWords; ++q) raw[u][q] = key < k_end ? p[q] : u4v{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u) {
      float x[16];
#pragma unroll
      for (int q = 0; q < kWords; ++q) {
        const unsigned w[4] = {raw[u][q].x, raw[u][q].y, raw[u][q].z, raw[u][q].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (DT == A2ATS_BF16) {
            x[8 * q + 2 * e] = __uint_as_float(w[e] << 16);
            x[8 * q + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
          } else {
            x[4 * q + e] = __uint_as_float(w[e]);
          }
        }
      }
      float dot = 0.f, nrm = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        dot += x[e] * qv[e];
        nrm += x[e] * x[e];
      }
#pragma unroll
      for (int o = 4; o > 0; o >>= 1) {
        dot += __shfl_xor(dot, o);
        nrm += __shfl_xor(nrm, o);
      }
      const int64_t key = k0 + u * kKeysPerRound + (t >> 3);
      if (sub == 0 && key < k_end) {
        const float sc = nrm > 0.f ? dot / sqrtf(nrm) : 0.f;
        const unsigned uk = order_key(sc);
        scores[hoff + key] = uk;
        atomicAdd(&lh[bin_of(uk, inv)], 1u);
      }
    }
  }
  __syncthreads();
  uint4* dst = reinterpret_cast<uint4*>(part + ((int64_t)head * wg_per_head + wg) * kBins);
  const uint4* src = reinterpret_cast<const uint4*>(lh);
  for (int i = t; i < kBins / 4; i += kScoreThreads) dst[i] = src[i];
  if (t < kBins / 4) {  // coarse counts: 8 lanes sum the 32 bins of one coarse bin
    unsigned c = lh[4 * t] + lh[4 * t + 1] + lh[4 * t + 2] + lh[4 * t + 3];
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) c += __shfl_xor(c, o);
    if ((t & 7) == 0) coarse[((int64_t)head * wg_per_head + wg) * kCoarse + (t >> 3)] = c;
  }
}

// Sum over the `rows` partial rows (stride `stride` words) of the 32 consecutive counts at
// `base`, into s_out[32], by a workgroup of 256 threads: thread t loads the 4 counts 4 (t % 8)
// .. of rows t / 8, t / 8 + 32, ... (all its loads in flight), lanes with the same t % 8 meet
// by butterfly shuffles, the four waves in LDS.  Every thread must call it.
__device__ __forceinline__ void sum_rows32(const unsigned* __restrict__ base, int64_t stride, int rows,
                                           unsigned* s_out) {
  constexpr int kRowsPerThread = (kScoreWgPerHead + 31) / 32;
  __shared__ uint4 s_q[4][8];
  const int t = threadIdx.x, lane = t & 63, q = t & 7, rw = t >> 3;
  uint4 x[kRowsPerThread];
#pragma unroll
  for (int k = 0; k < kRowsPerThread; ++k) {
    const int r = rw + 32 * k;
    x[k] = r < rows ? *reinterpret_cast<const uint4*>(base + (int64_t)r * stride + 4 * q)
                    : make_uint4(0u, 0u, 0u, 0u);
  }
  uint4 a = x[0];
#pragma unroll
  for (int k = 1; k < kRowsPerThread; ++k) {
    a.x += x[k].x; a.y += x[k].y; a.z += x[k].z; a.w += x[k].w;
  }
#pragma unroll
  for (int o = 8; o < 64; o <<= 1) {
    a.x += __shfl_xor(a.x, o);
    a.y += __shfl_xor(a.y, o);
    a.z += __shfl_xor(a.z, o);
    a.w += __shfl_xor(a.w, o);
  }
  if (lane < 8) s_q[t >> 6][lane] = a;
  __syncthreads();
  if (t < 8) {
    uint4 m = s_q[0][t];
#pragma unroll
    for (int wv = 1; wv < 4; ++wv) {
      const uint4 o = s_q[wv][t];
      m.x += o.x; m.y += o.y; m.z += o.z; m.w += o.w;
    }
    s_out[4 * t] = m.x;
    s_out[4 * t + 1] = m.y;
    s_out[4 * t + 2] = m.z;
    s_out[4 * t + 3] = m.w;
  }
  __syncthreads();
}

// In wave 0: the slot i of counts[32] (taken in descending order from slot 31) at which the
// running sum, starting at `from`, reaches `need`; *pick = i and *before = the sum of the
// slots above it.  Counts must reach need.
__device__ __forceinline__ void pick_desc32(const unsigned* counts, unsigned from, unsigned need,
                                            int* pick, unsigned* before) {
  const int lane = threadIdx.x & 63;
  const unsigned c = lane < 32 ? counts[31 - lane] : 0u;
  unsigned incl = c;
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) {
    const unsigned u = __shfl_up(incl, o);
    if (lane >= o) incl += u;
  }
  const unsigned cum = from + incl - c;
  if (lane < 32 && cum < need && cum + c >= need) {
    *pick = 31 - lane;
    *before = cum;
  }
}

// b* of a head and the count above it, in every workgroup that needs them: the 32 coarse
// counts (32 bins each) summed over the head's sel_score partials give the coarse bin of the
// n_r-th largest, then its 32 fine counts the bin.  Two rounds of 8 KB of reads in place of
// the whole 1024-bin partials.  b* = kBins (nothing selected) when n_r is 0.
__device__ void bstar_two_level(const unsigned* __restrict__ part_head,
                                const unsigned* __restrict__ coarse_head, int wg_per_head,
                                int64_t n_r, int* bstar, int* count_above) {
  __shared__ unsigned s_cnt[kCoarse];
  __shared__ int s_pick;
  __shared__ unsigned s_before;
  const int t = threadIdx.x;
  if (n_r == 0) {
    *bstar = kBins;
    *count_above = 0;
    return;
  }
  sum_rows32(coarse_head, kCoarse, wg_per_head, s_cnt);
  if (t < 64) pick_desc32(s_cnt, 0u, (unsigned)n_r, &s_pick, &s_before);
  __syncthreads();
  const int cbin = s_pick;
  const unsigned above_c = s_before;
  sum_rows32(part_head + cbin * (kBins / kCoarse), kBins, wg_per_head, s_cnt);
  if (t < 64) pick_desc32(s_cnt, above_c, (unsigned)n_r, &s_pick, &s_before);
  __syncthreads();
  *bstar = cbin * (kBins / kCoarse) + s_pick;
  *count_above = (int)s_before;
}

// Per block of kBlock scores: b* (every workgroup finds it from the partial histograms, its
// scores' reads already in flight; block 0 of the head records it), then the count above b*
// and the keys in b*, appended to the block's own region of the candidate array (no global
// atomics).
__global__ __launch_bounds__(256) void sel_collect(const unsigned* __restrict__ scores, int64_t n,
                                                   int nblk, const unsigned* __restrict__ part,
                                                   const unsigned* __restrict__ coarse,
                                                   int wg_per_head, int64_t n_r,
                                                   HeadInfo* __restrict__ info,
                                                   unsigned* __restrict__ above_blk,
                                                   unsigned* __restrict__ cand_blk,
                                                   unsigned long long* __restrict__ cand) {
  const int head = blockIdx.x / nblk;
  const int blk = blockIdx.x % nblk;
  const int t = threadIdx.x;
  const int64_t hoff = (int64_t)head * n;
  const int64_t i_begin = (int64_t)blk * kBlock;
  const int64_t i_end = i_begin + kBlock < n ? i_begin + kBlock : n;
  const int64_t i0 = i_begin + 4 * t;  // 4 consecutive scores per thread, read before b* is known
  unsigned uv[4];
  if (i0 + 3 < i_end && ((hoff + i0) & 3) == 0) {
    const uint4 q = *reinterpret_cast<const uint4*>(scores + hoff + i0);
    uv[0] = q.x; uv[1] = q.y; uv[2] = q.z; uv[3] = q.w;
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) uv[k] = (i0 + k < i_end) ? scores[hoff + i0 + k] : 0u;
  }
  const float inv = info[head].inv_scale;
  int bstar, count_above;
  bstar_two_level(part + (int64_t)head * wg_per_head * kBins,
                  coarse + (int64_t)head * wg_per_head * kCoarse, wg_per_head, n_r, &bstar,
                  &count_above);
  if (blk == 0 && t == 0) {  // every block of the head finds the same; block 0 records it
    info[head].n_r = (int)n_r;
    info[head].thr = ~0ull;
    info[head].bstar = bstar;
    info[head].count_above = count_above;
  }
  unsigned above = 0;
  __shared__ unsigned s_cnt;
  __shared__ unsigned red[4];
  if (t == 0) s_cnt = 0u;
  __syncthreads();
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

// One workgroup of 1024 threads per head: the exact n_r-th largest 64-bit key among the
// candidates of bin b*, the selected candidates per block, and the exclusive output offset of
// every block.  When the candidates fit (at most kSortCap of them, at most kOffCap blocks)
// they are gathered into LDS in parallel (each thread finds the block of its slot by binary
// search over the block offsets), kept in block order in `su`; up to kRankCap of them each
// candidate counts the larger ones (pairs of candidates, up to 8 threads a pair, each over its
// part of the list), more are sorted descending (bitonic) in `sk`.  Otherwise a radix select runs over
// the candidate regions in global memory.
constexpr int kThreshThreads = 1024;
__global__ __launch_bounds__(kThreshThreads) void sel_thresh(int64_t n, int nblk,
                                                             HeadInfo* __restrict__ info,
                                                             const unsigned* __restrict__ above_blk,
                                                             const unsigned* __restrict__ cand_blk,
                                                             const unsigned long long* __restrict__ cand,
                                                             unsigned* __restrict__ blk_off) {
  constexpr int NT = kThreshThreads;
  const int head = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t hoff = (int64_t)head * n;
  const int64_t cbase = (int64_t)head * nblk;
  // the first NT blocks' above-b* counts are fetched up front, beside the head's record
  const unsigned above0 = t < nblk ? above_blk[cbase + t] : 0u;
  const int r = info[head].n_r - info[head].count_above;  // 1-based rank inside bin b*
  __shared__ unsigned long long sk[kSortCap];
  __shared__ unsigned long long su[kSortCap];
  __shared__ unsigned s_off[kOffCap + 1];
  // candidate count and per-block candidate offsets
  unsigned n_cand = 0;
  for (int b0 = 0; b0 < nblk; b0 += NT) {
    const int b = b0 + t;
    const unsigned cb = b < nblk ? cand_blk[cbase + b] : 0u;
    unsigned chunk;
    const unsigned ex = block_exclusive_scan<NT>(cb, &chunk);
    if (b < nblk && b < kOffCap) s_off[b] = n_cand + ex;
    n_cand += chunk;
  }
  if (t == 0 && nblk <= kOffCap) s_off[nblk] = n_cand;
  __syncthreads();
  const bool fits = n_cand <= (unsigned)kSortCap && nblk <= kOffCap;
  __shared__ unsigned dh[256];
  __shared__ unsigned long long s_prefix;
  __shared__ unsigned s_remaining;
  unsigned long long prefix = 0ull, mask = 0ull;
  if (t == 0) s_remaining = (unsigned)(r > 0 ? r : 0);
  if (r > 0 && fits) {
    const bool by_rank = n_cand <= (unsigned)kRankCap;
    for (int j = t; j < (int)n_cand; j += NT) {
      int lo = 0, hi = nblk - 1;  // the last block whose offset is <= j holds slot j
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_off[mid] <= (unsigned)j) lo = mid;
        else hi = mid - 1;
      }
      const unsigned long long v = cand[hoff + (int64_t)lo * kBlock + (j - (int)s_off[lo])];
      su[j] = v;
      if (!by_rank) sk[j] = v;
    }
    if (by_rank) {
      // Candidates in pairs (2c, 2c + 1), P threads a pair (at most 8), each counting the
      // larger keys (all distinct) in its part of the list for both; the candidate with r - 1
      // larger ones is it.  Part q holds every P-th slot from q, so the P parts a wave reads
      // at once are adjacent slots (distinct banks); slots past n_cand hold 0, which counts
      // nothing.
      const unsigned pairs = (n_cand + 1u) / 2u;
      int lp = 0;
      while (lp < 3 && (pairs << (lp + 1)) <= (unsigned)NT) ++lp;
      const int P = 1 << lp;
      const int L = (((int)n_cand + P - 1) / P + 7) & ~7;
      for (int i = (int)n_cand + t; i < P * L; i += NT) su[i] = 0ull;
      __syncthreads();
      const int c = t >> lp, q = t & (P - 1);
      const bool two = 2 * c + 1 < (int)n_cand;
      unsigned long long m0 = ~0ull, m1 = ~0ull;
      unsigned r0 = 0, r1 = 0;
      if (c < (int)pairs) {  // waves past the last pair skip the loop
        m0 = su[2 * c];
        m1 = two ? su[2 * c + 1] : ~0ull;
        for (int i = 0; i < L; i += 8) {  // part q: slots q, q + P, q + 2P, ...
          unsigned long long x[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = su[(i + e) * P + q];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            r0 += x[e] > m0 ? 1u : 0u;
            r1 += x[e] > m1 ? 1u : 0u;
          }
        }
      }
#pragma unroll
      for (int o = 1; o < 8; o <<= 1)
        if (o < P) {
          r0 += __shfl_xor(r0, o);
          r1 += __shfl_xor(r1, o);
        }
      if (c < (int)pairs && q == 0) {
        if (r0 == (unsigned)(r - 1)) s_prefix = m0;
        if (two && r1 == (unsigned)(r - 1)) s_prefix = m1;
      }
      __syncthreads();
      prefix = s_prefix;
    } else {
      int P = 1;
      while (P < (int)n_cand) P <<= 1;
      for (int i = (int)n_cand + t; i < P; i += NT) sk[i] = 0ull;
      __syncthreads();
      // bitonic sort, descending; every thread takes whole compare-exchange pairs
      for (int k = 2; k <= P; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
          for (int q = t; q < P / 2; q += NT) {
            const int i = (q / j) * 2 * j + (q % j);
            const int l = i + j;
            const unsigned long long a = sk[i], b = sk[l];
            const bool desc = (i & k) == 0;
            if (desc ? (a < b) : (a > b)) {
              sk[i] = b;
              sk[l] = a;
            }
          }
          __syncthreads();
        }
      }
      prefix = sk[r - 1];
    }
  } else if (r > 0) {
    __syncthreads();
    // radix select over the per-block candidate regions, 8 bits at a time
    for (int shift = 56; shift >= 0; shift -= 8) {
      if (t < 256) dh[t] = 0u;
      __syncthreads();
      for (int b = t; b < nblk; b += NT) {
        const unsigned cb = cand_blk[cbase + b];
        for (unsigned i = 0; i < cb; ++i) {
          const unsigned long long kv = cand[hoff + (int64_t)b * kBlock + i];
          if ((kv & mask) == prefix) atomicAdd(&dh[(kv >> shift) & 0xFF], 1u);
        }
      }
      __syncthreads();
      {  // digit holding the rem-th largest: thread t < 256 takes digit 255 - t (descending)
        const unsigned rem = s_remaining;
        const unsigned cdg = t < 256 ? dh[255 - t] : 0u;
        unsigned all;
        const unsigned cum = block_exclusive_scan<NT>(cdg, &all);
        if (t < 256 && cum < rem && cum + cdg >= rem) {
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
  // per block: keys above b* plus its selected candidates, then exclusive offsets
  unsigned run = 0;
  for (int b0 = 0; b0 < nblk; b0 += NT) {
    const int b = b0 + t;
    unsigned cnt = 0;
    if (b < nblk) {
      cnt = b0 == 0 ? above0 : above_blk[cbase + b];
      if (r > 0 && fits) {
        for (unsigned i = s_off[b]; i < s_off[b + 1]; ++i) cnt += su[i] >= thr ? 1u : 0u;
      } else if (r > 0) {
        const unsigned cb = cand_blk[cbase + b];
        for (unsigned i = 0; i < cb; ++i)
          cnt += cand[hoff + (int64_t)b * kBlock + i] >= thr ? 1u : 0u;
      }
    }
    unsigned chunk;
    const unsigned ex = block_exclusive_scan<NT>(cnt, &chunk);
    if (b < nblk) blk_off[cbase + b] = run + ex;
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
  const unsigned blk_base = offsets[(int64_t)head * nblk + blk];  // read up front, beside the record
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
  const int64_t sel_before = (int64_t)blk_base + wbase + incl - cnt;
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
  unsigned* part;
  unsigned* coarse;
  unsigned* scores;
  unsigned long long* cand;
  unsigned* above_blk;
  unsigned* cand_blk;
  unsigned* blk_off;
  size_t bytes;
};

// sel_score workgroups per head and keys per workgroup
inline void score_split(int64_t n, int64_t* wg_per_head, int64_t* per_wg) {
  int64_t w = (n + kScoreMinKeys - 1) / kScoreMinKeys;
  if (w > kScoreWgPerHead) w = kScoreWgPerHead;
  if (w < 1) w = 1;
  *wg_per_head = w;
  *per_wg = (n + w - 1) / w;
}

SelLayout carve(void* ws, int64_t heads, int64_t n) {
  const int64_t nblk = (n + kBlock - 1) / kBlock;
  Carver c(ws);
  SelLayout L;
  L.info = c.take<HeadInfo>((size_t)heads);
  int64_t wgph, per;
  score_split(n, &wgph, &per);
  L.part = c.take<unsigned>((size_t)(heads * wgph * kBins));
  L.coarse = c.take<unsigned>((size_t)(heads * wgph * kCoarse));
  L.scores = c.take<unsigned>((size_t)heads * n);
  L.cand = c.take<unsigned long long>((size_t)heads * n);
  L.above_blk = c.take<unsigned>((size_t)heads * nblk);
  L.cand_blk = c.take<unsigned>((size_t)heads * nblk);
  L.blk_off = c.take<unsigned>((size_t)heads * nblk);
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
  int64_t wg_per_head, per_wg;
  score_split(n, &wg_per_head, &per_wg);
  const int64_t nblk = (n + kBlock - 1) / kBlock;
  if (heads * nblk > 0x7FFFFFFF || heads > 65535) return A2ATS_EINVAL;
  const size_t need = a2ats_select_retrieval_workspace(heads, n);
  if (!ws_ok(workspace, workspace_bytes, need)) return A2ATS_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  SelLayout L = carve(workspace, heads, n);
  if (keys_dtype == A2ATS_BF16)
    A2ATS_TRY(launch("select_score", sel_score<A2ATS_BF16>, dim3((unsigned)(heads * wg_per_head)),
                     dim3(kScoreThreads), 0, s, keys, query, n, (int)wg_per_head, per_wg, L.scores, L.part,
                     L.coarse, L.info));
  else
    A2ATS_TRY(launch("select_score", sel_score<A2ATS_F32>, dim3((unsigned)(heads * wg_per_head)),
                     dim3(kScoreThreads), 0, s, keys, query, n, (int)wg_per_head, per_wg, L.scores, L.part,
                     L.coarse, L.info));
  A2ATS_TRY(launch("select_collect", sel_collect, dim3((unsigned)(heads * nblk)), dim3(256), 0, s,
                   L.scores, n, (int)nblk, L.part, L.coarse, (int)wg_per_head, n_r, L.info,
                   L.above_blk, L.cand_blk, L.cand));
  A2ATS_TRY(launch("select_thresh", sel_thresh, dim3((unsigned)heads), dim3(kThreshThreads), 0, s, n,
                   (int)nblk, L.info, L.above_blk, L.cand_blk, L.cand, L.blk_off));
  return launch("select_scatter", sel_scatter, dim3((unsigned)(heads * nblk)), dim3(256), 0, s,
                L.scores, n, (int)nblk, L.info, L.blk_off, retrieval_idx, bulk_idx);
}
