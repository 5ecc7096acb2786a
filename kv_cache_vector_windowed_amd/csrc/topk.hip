// Approximate attention-score top-K over codes.  The A2ATS paper page ("Abstract (arXiv)")
// retrieves the top-K tokens by attention scores approximated with the vector-quantised keys;
// with far keys kept unrotated and the far rotation R_b moved onto the query ("A2ATS-adapted"
// docs, "paper fidelity" section, Eq. 11-12) the approximate logit of token t is
// (q R_b) . c_{code_t}: one table of C values per query, gathered by code.
//
// Kernel topk_codes_rows: one 1024-thread workgroup per (sequence, key/value head, group of up
// to four of the query heads that share that key/value head).  The codes and the codebook are
// read once for the whole group.
//   1. table: lut_gj = fp32(sum_a qb_ga * c_ja) with the sum taken in fp64 in dimension order
//      and rounded to fp32 once.  Both factors have at most 24 significant bits, so each fp64
//      product is exact and fma(q, c, acc) equals acc + q*c rounded once: the fma loop is the
//      plain product-then-add sum.  The codebook streams through LDS in 1024-centroid x
//      8-dimension tiles, double-buffered and stored transposed by eight loader waves while
//      four table waves compute; each table thread owns four adjacent centroids (one 16-byte
//      LDS read a dimension) and reads the query values with wave-uniform scalar loads, so
//      one codebook read serves every query of the group.
//   2. the code row goes to LDS (rows up to 32768 tokens; longer rows are read from global
//      memory in each pass) and its histogram over the C codes (+1 bin for codes >= C) is taken.
//   3. for all queries of the group at once: the K-th largest score T_g by a radix select
//      (8 bits a pass, four passes) over the C + 1 table entries weighted by their counts, not
//      over the n tokens; r_g = how many of the tokens scoring exactly T_g are taken (the
//      lowest indices among them).  Then one class byte per code: bit 2g = above T_g, bit
//      2g+1 = equal to T_g.
//   4. ordered compaction.  Each wave owns a contiguous token range, 256 tokens a step (four
//      a lane, slot-major so that one ballot per slot orders them); a first pass counts every
//      query's tokens above and at T_g per wave, a second writes every query's taken indices
//      (and scores) in ascending order.
// Scores compare through the order-preserving map of fp32 onto u32 (-0 and +0 equal); a code
// >= C scores -inf.
#include "common.hpp"

namespace a2ats {
namespace {

constexpr int kD = A2ATS_HEAD_DIM;
constexpr int kTkThreads = 1024;
constexpr int kTkMaxC = 4096;                        // table entries per query in LDS
constexpr int kTkEnt = (kTkMaxC + 1 + kTkThreads - 1) / kTkThreads;  // table entries per thread
constexpr int kTkTile = 1024;                        // centroids per codebook tile
constexpr int kTkDims = 8;                           // dimensions per codebook tile
// A tile is stored transposed, one row of 1024 centroids per dimension.  The pitch makes the
// transposing scalar writes conflict-free (the two half-rows a wave writes land 32 banks
// apart) and keeps rows 16-byte aligned for the four-centroid reads.
constexpr int kTkPitch = kTkTile + 8;
constexpr int kTkR = 4;                              // centroids per table thread
constexpr int kTkStage = 2 * kTkDims * kTkPitch;     // floats: two tiles; also the code row
constexpr int kTkLdsCodes = 32768;                   // longest code row kept in LDS
static_assert(kTkLdsCodes * 2 <= kTkStage * 4, "code row must fit the staging area");
static_assert(kTkTile == kTkR * 256, "256 table threads");

__device__ __forceinline__ unsigned tk_order_key(float s) {
  if (s == 0.0f) s = 0.0f;  // -0 and +0 rank equal
  const unsigned b = __float_as_uint(s);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ int tk_wave_sum(int v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

constexpr int kTkLoaders = 512;  // threads 512 .. 1023 stage the codebook tiles

// Codebook tile [cb0, cb0 + 1024) x [8 ch, 8 ch + 8) into a loader thread's registers (u =
// its index among the loaders): four float4, two loaders a centroid row segment (32 bytes).
__device__ __forceinline__ void tk_load_tile(float4 (&pre)[4], const float* __restrict__ cbh,
                                             int c, int cb0, int ch, int u) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = u + kTkLoaders * i, j = cb0 + (q >> 1);
    pre[i] = j < c ? *reinterpret_cast<const float4*>(cbh + (int64_t)j * kD + ch * kTkDims +
                                                      (q & 1) * 4)
                   : make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// Transposed store: dimension 4h + e of centroid j goes to buf[(4h + e) * pitch + j].
__device__ __forceinline__ void tk_store_tile(float* buf, const float4 (&pre)[4], int u) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = u + kTkLoaders * i, j = q >> 1;
    float* s = buf + (q & 1) * 4 * kTkPitch + j;
    s[0] = pre[i].x;
    s[kTkPitch] = pre[i].y;
    s[2 * kTkPitch] = pre[i].z;
    s[3 * kTkPitch] = pre[i].w;
  }
}

template <int QDT, int GN, bool CLDS>
__global__ __launch_bounds__(kTkThreads) void topk_codes_rows(
    const void* __restrict__ qb, int64_t hq, int64_t hkv, int group, int nchunk,
    const uint16_t* __restrict__ codes, int64_t n, const float* __restrict__ cb, int c,
    int64_t k, int32_t* __restrict__ idx, float* __restrict__ score) {
  constexpr int kWaves = kTkThreads / 64;
  __shared__ float lut[GN][kTkMaxC + 1];
  __shared__ __align__(16) float stage[kTkStage];
  __shared__ unsigned cnt[kTkMaxC + 1];  // code histogram; then the class bytes
  __shared__ unsigned hist[GN][256];
  __shared__ unsigned s_prefix[GN], s_rem[GN];
  __shared__ int wcnt[kWaves][2 * GN];   // per wave and query: tokens above, tokens equal

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t wg = blockIdx.x;
  const int chunk = (int)(wg % nchunk);
  const int64_t bk = wg / nchunk;  // sequence * hkv + key/value head
  const int64_t b = bk / hkv, kvh = bk % hkv;
  const int g0 = chunk * GN;
  const int gv = group - g0 < GN ? group - g0 : GN;  // query heads of this group in use
  const int64_t row0 = b * hq + kvh * group + g0;    // their first output row

  int64_t qoff[GN];  // query rows (a slot past the group's last query repeats it)
#pragma unroll
  for (int g = 0; g < GN; ++g) qoff[g] = (row0 + (g < gv ? g : gv - 1)) * kD;

  // ---- 1. score table
  const float* cbh = cb + kvh * (int64_t)c * kD;
  // Warp-specialised and double-buffered: the table threads (waves 0-3; thread t owns
  // centroids 4t .. 4t + 3) work on one tile while the loader threads (waves 8-15) store the
  // next into the other buffer; each tile is loaded two steps before it is stored.
  constexpr int kChunks = kD / kTkDims;
  const bool table_thread = t < kTkTile / kTkR, loader = t >= kTkThreads - kTkLoaders;
  const int u = t - (kTkThreads - kTkLoaders);
  for (int cb0 = 0; cb0 < c; cb0 += kTkTile) {
    float4 pre[2][4];
    double acc[kTkR][GN];
#pragma unroll
    for (int r = 0; r < kTkR; ++r)
#pragma unroll
      for (int g = 0; g < GN; ++g) acc[r][g] = 0.0;
    if (loader) {
      tk_load_tile(pre[0], cbh, c, cb0, 0, u);
      tk_load_tile(pre[1], cbh, c, cb0, 1, u);
    }
    __syncthreads();  // the previous tile's readers are done with both buffers
    if (loader) {
      tk_store_tile(stage, pre[0], u);
      tk_load_tile(pre[0], cbh, c, cb0, 2, u);
    }
    __syncthreads();
#pragma unroll
    for (int ch = 0; ch < kChunks; ++ch) {
      if (loader && ch + 1 < kChunks) {
        tk_store_tile(stage + ((ch + 1) & 1) * kTkDims * kTkPitch, pre[(ch + 1) & 1], u);
        if (ch + 3 < kChunks) tk_load_tile(pre[(ch + 1) & 1], cbh, c, cb0, ch + 3, u);
      }
      if (table_thread) {
        const float* sb = stage + (ch & 1) * kTkDims * kTkPitch + 4 * t;
#pragma unroll
        for (int a = 0; a < kTkDims; ++a) {
          const float4 xv = *reinterpret_cast<const float4*>(sb + a * kTkPitch);
          const double x[kTkR] = {(double)xv.x, (double)xv.y, (double)xv.z, (double)xv.w};
#pragma unroll
          for (int g = 0; g < GN; ++g) {
            const double qv = (double)load_elem(qb, QDT, qoff[g] + ch * kTkDims + a);
#pragma unroll
            for (int r = 0; r < kTkR; ++r) acc[r][g] = __fma_rn(qv, x[r], acc[r][g]);
          }
        }
      }
      __syncthreads();
    }
    if (table_thread) {
#pragma unroll
      for (int r = 0; r < kTkR; ++r) {
        const int j = cb0 + 4 * t + r;
        if (j < c)
#pragma unroll
          for (int g = 0; g < GN; ++g) lut[g][j] = (float)acc[r][g];
      }
    }
  }
  if (t < GN) lut[t][c] = -INFINITY;  // the score of every code >= c
  __syncthreads();

  // ---- 2. code row and its histogram
  for (int j = t; j <= c; j += kTkThreads) cnt[j] = 0u;
  __syncthreads();
  const uint16_t* cg = codes + bk * n;
  uint16_t* cl = reinterpret_cast<uint16_t*>(stage);
  const unsigned cu = (unsigned)c;
  if (CLDS && (n & 7) == 0) {  // 16-byte rows: eight codes a load
    const uint4* src = reinterpret_cast<const uint4*>(cg);
    uint4* dst = reinterpret_cast<uint4*>(cl);
    const int n8 = (int)(n >> 3);
    for (int i = t; i < n8; i += 2 * kTkThreads) {
      const bool two = i + kTkThreads < n8;
      const uint4 v0 = src[i];
      const uint4 v1 = two ? src[i + kTkThreads] : make_uint4(0u, 0u, 0u, 0u);
      dst[i] = v0;
      if (two) dst[i + kTkThreads] = v1;
      const unsigned w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (q >= 4 && !two) break;
        const unsigned lo = w[q] & 0xFFFFu, hi = w[q] >> 16;
        atomicAdd(&cnt[lo < cu ? lo : cu], 1u);
        atomicAdd(&cnt[hi < cu ? hi : cu], 1u);
      }
    }
  } else {
    for (int64_t i = t; i < n; i += kTkThreads) {
      const unsigned v = cg[i];
      if (CLDS) cl[i] = (uint16_t)v;
      atomicAdd(&cnt[v < cu ? v : cu], 1u);
    }
  }
  __syncthreads();

  // ---- 3. weighted radix select over the table entries, every query at once
  const unsigned neg_inf_key = tk_order_key(-INFINITY);
  unsigned ek[GN][kTkEnt], ec[kTkEnt];
#pragma unroll
  for (int e = 0; e < kTkEnt; ++e) {
    const int j = t + kTkThreads * e;
    ec[e] = j <= c ? cnt[j] : 0u;
#pragma unroll
    for (int g = 0; g < GN; ++g) ek[g][e] = j < c ? tk_order_key(lut[g][j]) : neg_inf_key;
  }
  if (t < GN) s_rem[t] = (unsigned)k;
  unsigned prefix[GN], mask = 0u;
#pragma unroll
  for (int g = 0; g < GN; ++g) prefix[g] = 0u;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = t; i < GN * 256; i += kTkThreads) (&hist[0][0])[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kTkEnt; ++e) {
      if (ec[e] == 0u) continue;
#pragma unroll
      for (int g = 0; g < GN; ++g)
        if ((ek[g][e] & mask) == prefix[g]) atomicAdd(&hist[g][(ek[g][e] >> shift) & 0xFFu], ec[e]);
    }
    __syncthreads();
    if (wave < GN) {  // wave g: the digit holding query g's remaining rank
      const int g = wave;
      unsigned h[4], sum = 0u;
#pragma unroll
      for (int q = 0; q < 4; ++q) {  // lane l: digits 255 - 4l .. 252 - 4l (descending)
        h[q] = hist[g][255 - 4 * lane - q];
        sum += h[q];
      }
      unsigned incl = sum;
      for (int o = 1; o < 64; o <<= 1) {
        const unsigned u = __shfl_up(incl, o);
        if (lane >= o) incl += u;
      }
      unsigned cum = incl - sum;
      const unsigned rem = s_rem[g];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (cum < rem && cum + h[q] >= rem) {
          s_rem[g] = rem - cum;
          s_prefix[g] = prefix[g] | ((unsigned)(255 - 4 * lane - q) << shift);
        }
        cum += h[q];
      }
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < GN; ++g) prefix[g] = s_prefix[g];
    mask |= 0xFFu << shift;
  }
  // prefix[g] is now T_g, the K-th largest score key; s_rem[g] of the tokens at T_g are taken

  // class byte per code (the histogram is no longer needed)
  uint8_t* cls = reinterpret_cast<uint8_t*>(cnt);
  for (int j = t; j <= c; j += kTkThreads) {
    unsigned v = 0u;
#pragma unroll
    for (int g = 0; g < GN; ++g) {
      const unsigned u = j < c ? tk_order_key(lut[g][j]) : neg_inf_key;
      v |= (u > prefix[g] ? 1u : 0u) << (2 * g);
      v |= (u == prefix[g] ? 1u : 0u) << (2 * g + 1);
    }
    cls[j] = (uint8_t)v;
  }
  __syncthreads();

  // ---- 4. ordered compaction: wave ranges of whole 256-token steps; in a step, slot e of
  // lane l is token base + 64 e + l, so a ballot per slot orders the wave's tokens
  const int64_t per = ((n + kWaves - 1) / kWaves + 255) / 256 * 256;
  const int64_t w0 = (int64_t)wave * per < n ? (int64_t)wave * per : n;
  const int64_t w1 = w0 + per < n ? w0 + per : n;
  const unsigned long long lt = (1ull << lane) - 1ull;
  // codes (clamped to c) and class bytes of the lane's four tokens; class 0 past the range
  auto step = [&](int64_t base, unsigned (&cc)[4], unsigned (&v)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t i = base + 64 * e + lane;
      const unsigned code = i < w1 ? (CLDS ? (unsigned)cl[i] : (unsigned)cg[i]) : cu;
      cc[e] = code < cu ? code : cu;
      v[e] = i < w1 ? (unsigned)cls[cc[e]] : 0u;
    }
  };
  {
    int na[GN], ne[GN];
#pragma unroll
    for (int g = 0; g < GN; ++g) na[g] = ne[g] = 0;
    for (int64_t base = w0; base < w1; base += 256) {
      unsigned cc[4], v[4];
      step(base, cc, v);
      const unsigned x = v[0] | (v[1] << 8) | (v[2] << 16) | (v[3] << 24);
#pragma unroll
      for (int g = 0; g < GN; ++g) {
        na[g] += __popc(x & (0x01010101u << (2 * g)));
        ne[g] += __popc(x & (0x02020202u << (2 * g)));
      }
    }
#pragma unroll
    for (int g = 0; g < GN; ++g) {
      const int a = tk_wave_sum(na[g]), e = tk_wave_sum(ne[g]);
      if (lane == 0) {
        wcnt[wave][2 * g] = a;
        wcnt[wave][2 * g + 1] = e;
      }
    }
  }
  __syncthreads();

  // per query: this wave's first output slot and its share of the tokens at T_g
  int out[GN], eq_take[GN], eq_seen[GN];
#pragma unroll
  for (int g = 0; g < GN; ++g) {
    const int r_eq = (int)s_rem[g];
    int o = 0, eq_before = 0;
    for (int w = 0; w < wave; ++w) {
      const int e = wcnt[w][2 * g + 1];
      int take = r_eq - eq_before;
      take = take < 0 ? 0 : (take > e ? e : take);
      o += wcnt[w][2 * g] + take;
      eq_before += e;
    }
    const int mine = wcnt[wave][2 * g + 1];
    const int et = r_eq - eq_before;
    out[g] = o;
    eq_take[g] = et < 0 ? 0 : (et > mine ? mine : et);
    eq_seen[g] = 0;
  }
  auto below = [](unsigned long long m) {  // set bits of m in the lanes below this one
    return (int)__builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32),
                                          __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
  };
  const unsigned ku = (unsigned)k;
  for (int64_t base = w0; base < w1; base += 256) {
    unsigned cc[4], v[4];
    step(base, cc, v);
    const unsigned vor = v[0] | v[1] | v[2] | v[3];
#pragma unroll
    for (int g = 0; g < GN; ++g) {
      if (g >= gv) break;
      bool take[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) take[e] = (v[e] >> (2 * g)) & 1u;
      if (__ballot((vor >> (2 * g + 1)) & 1u)) {  // tokens at T_g: the first eq_take of the range
        int seen = eq_seen[g];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool eq = (v[e] >> (2 * g + 1)) & 1u;
          const unsigned long long m = __ballot(eq);
          take[e] = take[e] || (eq && seen + below(m) < eq_take[g]);
          seen += __popcll(m);
        }
        eq_seen[g] = seen;
      }
      int32_t* orow = idx + (row0 + g) * k;
      float* srow = score ? score + (row0 + g) * k : nullptr;
      float sv[4];  // read ahead: one LDS wait for the four stores
#pragma unroll
      for (int e = 0; e < 4; ++e) sv[e] = lut[g][cc[e]];
      int o = out[g];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const unsigned long long m = __ballot(take[e]);
        const unsigned pos = (unsigned)(o + below(m));
        if (take[e] && pos < ku) {  // the bound turns any inconsistency into a wrong answer
          orow[pos] = (int32_t)(base + 64 * e + lane);
          if (srow) srow[pos] = sv[e];
        }
        o += __popcll(m);
      }
      out[g] = o;
    }
  }
}

template <int QDT, int GN>
int topk_launch(bool clds, dim3 grid, hipStream_t s, const void* qb, int64_t hq, int64_t hkv,
                int group, int nchunk, const uint16_t* codes, int64_t n, const float* cb, int c,
                int64_t k, int32_t* idx, float* score) {
  if (clds)
    return launch("topk_codes", topk_codes_rows<QDT, GN, true>, grid, dim3(kTkThreads), 0, s, qb,
                  hq, hkv, group, nchunk, codes, n, cb, c, k, idx, score);
  return launch("topk_codes", topk_codes_rows<QDT, GN, false>, grid, dim3(kTkThreads), 0, s, qb,
                hq, hkv, group, nchunk, codes, n, cb, c, k, idx, score);
}

template <int QDT>
int topk_dispatch(int gn, bool clds, dim3 grid, hipStream_t s, const void* qb, int64_t hq,
                  int64_t hkv, int group, int nchunk, const uint16_t* codes, int64_t n,
                  const float* cb, int c, int64_t k, int32_t* idx, float* score) {
  switch (gn) {
    case 1:
      return topk_launch<QDT, 1>(clds, grid, s, qb, hq, hkv, group, nchunk, codes, n, cb, c, k,
                                 idx, score);
    case 2:
      return topk_launch<QDT, 2>(clds, grid, s, qb, hq, hkv, group, nchunk, codes, n, cb, c, k,
                                 idx, score);
    case 3:
      return topk_launch<QDT, 3>(clds, grid, s, qb, hq, hkv, group, nchunk, codes, n, cb, c, k,
                                 idx, score);
    default:
      return topk_launch<QDT, 4>(clds, grid, s, qb, hq, hkv, group, nchunk, codes, n, cb, c, k,
                                 idx, score);
  }
}

}  // namespace
}  // namespace a2ats

using namespace a2ats;

extern "C" int a2ats_topk_codes(const void* qb, int q_dtype, int64_t batch, int64_t hq,
                                int64_t hkv, int64_t d, const uint16_t* codes, int64_t n,
                                const float* codebook, int64_t c, int64_t k, int32_t* idx,
                                float* score, void* stream) {
  if (q_dtype != A2ATS_F32 && q_dtype != A2ATS_BF16) return A2ATS_EDTYPE;
  if (d != kD || batch < 1 || hq < 1 || hkv < 1 || hq % hkv != 0) return A2ATS_EINVAL;
  if (n < 0 || n > 0x7FFFFFFF || c < 1 || c > kTkMaxC || k < 0 || k > n) return A2ATS_EINVAL;
  const int group = (int)(hq / hkv);
  const int gn = group < 4 ? group : 4;
  const int nchunk = (group + gn - 1) / gn;
  if (batch * hkv * nchunk > 0x7FFFFFFF) return A2ATS_EINVAL;
  if (n == 0 || k == 0) return A2ATS_OK;
  if (!qb || !codes || !codebook || !idx) return A2ATS_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)(batch * hkv * nchunk));
  const bool clds = n <= kTkLdsCodes;
  if (q_dtype == A2ATS_F32)
    return topk_dispatch<A2ATS_F32>(gn, clds, grid, s, qb, hq, hkv, group, nchunk, codes, n,
                                    codebook, (int)c, k, idx, score);
  return topk_dispatch<A2ATS_BF16>(gn, clds, grid, s, qb, hq, hkv, group, nchunk, codes, n,
                                   codebook, (int)c, k, idx, score);
}
