// Approximate attention-score top-K over codes.  The A2ATS paper page ("Abstract (arXiv)")
// retrieves the top-K tokens by attention scores approximated with the vector-quantised keys;
// with far keys kept unrotated and the far rotation R_b moved onto the query ("A2ATS-adapted"
// docs, "paper fidelity" section, Eq. 11-12) the approximate logit of token t is
// (q R_b) . c_{code_t}: one table of C values per query, gathered by code.
//
// Two kernels (their own comments say more):
//   topk_table       every query's table, lut_gj = fp32(sum_a qb_ga * c_ja) with the sum taken
//                    in fp64 in dimension order and rounded to fp32 once (both factors have at
//                    most 24 significant bits, so each fp64 product is exact and fma(q, c, acc)
//                    equals acc + q*c rounded once: the fma chain is the plain product-then-add
//                    sum), on the fp64 matrix cores, into the workspace.
//   topk_codes_rows  per (sequence, key/value head, up to four query heads): the tables in
//                    LDS, the histogram of the code row, the K-th largest score by monotone-bin
//                    histogram passes over the C + 1 weighted table entries (not over the n
//                    tokens), and the taken tokens in token order.
// Scores compare through the order-preserving map of fp32 onto u32 (-0 and +0 equal); a code
// >= C scores -inf.
#include "common.hpp"

namespace a2ats {
namespace {

constexpr int kD = A2ATS_HEAD_DIM;
constexpr int kTkThreads = 1024;
constexpr int kTkMaxC = 4096;                        // table entries per query in LDS
constexpr int kTkLdsCodes = 16384;                   // longest code row kept in LDS
typedef unsigned tk_u4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ unsigned tk_order_key(float s) {
  if (s == 0.0f) s = 0.0f;  // -0 and +0 rank equal
  const unsigned b = __float_as_uint(s);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Kernel topk_table, on the fp64 matrix cores.  v_mfma_f64_16x16x4f64 adds its four products to
// C in k order with one rounding each (an fma chain), so a chain of 32 of them over the
// dimensions in order forms exactly the dimension-ordered fp64 sum.  One 768-thread workgroup per
// (key/value head, strip of 32 centroids, chunk of up to 96 of that head's batch * group queries,
// taken in (sequence, query head) order).  The strip and the chunk's queries are staged in LDS
// as fp32 (exact for fp32 and bf16 queries), rows padded to 132 floats so that the 16 rows x 4
// dimensions a wave reads at once fall in distinct banks.  Wave w (of 12, three a SIMD) runs one
// chain: centroid tile w & 1 (16 centroids) against query tile w >> 1 (16 queries; a tile past
// the chunk multiplies zero rows and is never stored).  Operands: A lane l = query l % 16 of the
// tile, dimension 4 s + l / 16; B lane l = centroid l % 16, same dimension; result register r of
// lane l = query 4 r + l / 16, centroid l % 16, stored rounded to fp32 at
// lut[(sequence * hq + query head) * c + j].
typedef double tb_d4 __attribute__((ext_vector_type(4)));
typedef float tb_f4 __attribute__((ext_vector_type(4)));
constexpr int kTbPitch = kD + 4;
constexpr int kTbStrip = 32;        // centroids a workgroup (two tiles)
constexpr int kTbChunk = 96;        // queries a workgroup (six tiles)
constexpr int kTbThreads = 64 * (kTbStrip / 16) * (kTbChunk / 16);

template <int QDT>
__global__ __launch_bounds__(kTbThreads) void topk_table(const void* __restrict__ qb,
                                                         const float* __restrict__ cb,
                                                         int64_t batch, int64_t hq, int group,
                                                         int c, int nstrip, int nchunk,
                                                         float* __restrict__ lut) {
  __shared__ __align__(16) float cs[kTbStrip * kTbPitch];  // [centroid of the strip][dimension]
  __shared__ __align__(16) float qs[kTbChunk * kTbPitch];  // [query of the chunk][dimension]
  constexpr int kCv = (kTbStrip * 32 + kTbThreads - 1) / kTbThreads;  // strip float4 a thread
  constexpr int kQv = kTbChunk * 32 / kTbThreads;                     // query float4 a thread
  static_assert(kTbChunk * 32 % kTbThreads == 0, "query staging");
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  unsigned w = blockIdx.x;
  const int qc = (int)(w % (unsigned)nchunk);
  w /= (unsigned)nchunk;
  const int strip = (int)(w % (unsigned)nstrip);
  const int64_t kvh = w / (unsigned)nstrip;
  const int j0 = strip * kTbStrip, q0 = qc * kTbChunk;
  const int nq = (int)(batch * group);  // this head's queries (batch * hq < 2^31)
  const int nqc = nq - q0 < kTbChunk ? nq - q0 : kTbChunk;
  auto qrow = [&](int qi) {  // row of query qi of this head in qb and lut
    const int sq = qi / group;
    return (int64_t)sq * hq + kvh * group + (qi - sq * group);
  };
  {
    // every load in flight before the LDS writes; rows past c or past the chunk are zero
    const float* src = cb + kvh * c * kD;
    tb_f4 cv[kCv];
#pragma unroll
    for (int i = 0; i < kCv; ++i) {
      const int f = t + kTbThreads * i, r = j0 + (f >> 5);
      if (f < kTbStrip * 32)
        cv[i] = reinterpret_cast<const tb_f4*>(src + (int64_t)(r < c ? r : c - 1) * kD)[f & 31];
    }
    tb_f4 qv[kQv];
#pragma unroll
    for (int i = 0; i < kQv; ++i) {
      const int f = t + kTbThreads * i, r = f >> 5;
      const int64_t row = qrow(q0 + (r < nqc ? r : nqc - 1));  // past the chunk: zeroed below
      if (QDT == A2ATS_F32) {
        qv[i] = reinterpret_cast<const tb_f4*>(qb)[row * (kD / 4) + (f & 31)];
      } else {
        const uint2 x = reinterpret_cast<const uint2*>(qb)[row * (kD / 4) + (f & 31)];
        qv[i] = (tb_f4){__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xFFFF0000u),
                        __uint_as_float(x.y << 16), __uint_as_float(x.y & 0xFFFF0000u)};
      }
    }
    const tb_f4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kCv; ++i) {
      const int f = t + kTbThreads * i, r = f >> 5;
      if (f < kTbStrip * 32)
        *reinterpret_cast<tb_f4*>(cs + r * kTbPitch + 4 * (f & 31)) = j0 + r < c ? cv[i] : z;
    }
#pragma unroll
    for (int i = 0; i < kQv; ++i) {
      const int f = t + kTbThreads * i, r = f >> 5;
      *reinterpret_cast<tb_f4*>(qs + r * kTbPitch + 4 * (f & 31)) = r < nqc ? qv[i] : z;
    }
  }
  __syncthreads();
  const int li = lane & 15, lk = lane >> 4, ct = wave & 1, qt = wave >> 1;
  const float* bp = cs + (16 * ct + li) * kTbPitch + lk;
  const float* ap = qs + (16 * qt + li) * kTbPitch + lk;
  // every operand read into registers first, so that the chain runs without LDS waits
  float bv[kD / 4], av[kD / 4];
#pragma unroll
  for (int s = 0; s < kD / 4; ++s) {
    bv[s] = bp[4 * s];
    av[s] = ap[4 * s];
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the chain
  tb_d4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int s = 0; s < kD / 4; ++s)
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)av[s], (double)bv[s], acc, 0, 0, 0);
  const int j = j0 + 16 * ct + li;
  if (j < c)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int qi = 16 * qt + 4 * r + lk;
      if (qi < nqc) lut[qrow(q0 + qi) * c + j] = (float)acc[r];
    }
}

// Kernel topk_codes_rows: one 1024-thread workgroup per (sequence, key/value head, group of up
// to four query heads sharing it).  LDS is laid out per call (TkLayout): the group's tables,
// the select histograms (later the output lists), the code histogram (then the class bytes)
// and the code row when it fits.
//   1. the group's tables, read from the workspace (their key ranges reduced on the way); the
//      code row and its histogram over the C codes (+1 bin for codes >= C): the weight of
//      table entry j is the number of tokens holding it.
//   2. for all queries at once, the K-th largest score T_g over the C + 1 weighted entries
//      (thread t holds entries t, t + 1024, ... < C in registers, thread 0 also the -inf entry
//      of the codes >= C) and r_g = how many of the tokens scoring exactly T_g are taken (the
//      lowest indices).  A pass bins the live entries into 1024 bins by a monotone map of the
//      score (linear in the fp32 value while the range is finite, else a shift of the order
//      key), wave g finds the bin holding the remaining rank, and that bin's entries stay
//      live.  A pass over keys closer than 1024 units is exact; a bin of at most 64 entries is
//      settled by wave g comparing them pairwise.
//   3. one class byte per code: bit 2g = above T_g, bit 2g+1 = equal to T_g.
//   4. rounds of 16384 tokens, 16 contiguous tokens a lane: per query, lane counts by bit
//      counts and wave scans, one barrier for the counts across waves, then each wave lists
//      its taken tokens (ascending) in LDS and copies the list out whole.
struct TkLayout {
  unsigned lut, hist, cnt, cl, total;
  int scap;  // output staging slots per (wave, query)
};

constexpr unsigned kTkLdsMax = 156 * 1024;  // dynamic LDS; the static arrays take the rest
constexpr int kNb = 1024;                   // bins of a select pass
constexpr int kNbPad = kNb + kNb / 16;      // a pad slot after every 16 bins
constexpr int kCand = 64;                   // largest bin settled pairwise
constexpr int kTkRound = kTkThreads * 16;   // tokens of an output round (16 a thread)

inline unsigned tk_al16(unsigned x) { return (x + 15u) & ~15u; }

// The LDS layout of a call; cl is 0xFFFFFFFF when the code row does not fit.  The select
// histograms' region later holds each wave's output list per query (scap slots, as many as fit
// up to 256) and a trash slot per thread.
inline TkLayout tk_layout(int gn, int c, int64_t n) {
  const int waves = kTkThreads / 64;
  const unsigned lutb = tk_al16((unsigned)(gn * (c + 1)) * 4u);
  const unsigned histb = tk_al16((unsigned)(gn * kNbPad) * 8u);
  const unsigned cntb = tk_al16((unsigned)(c + 1) * 4u);
  unsigned clb = 0;
  if (n <= kTkLdsCodes && lutb + histb + cntb + (unsigned)n * 2u <= kTkLdsMax)
    clb = tk_al16((unsigned)n * 2u);
  const unsigned room = kTkLdsMax - lutb - cntb - clb;  // >= histb
  const int scap0 = (int)((room / 4u - (unsigned)kTkThreads) / (unsigned)(waves * gn));
  TkLayout L;
  L.scap = scap0 < 256 ? scap0 : 256;
  const unsigned stageb = tk_al16((unsigned)(waves * gn * L.scap + kTkThreads) * 4u);
  L.lut = 0;
  L.hist = lutb;
  L.cnt = L.hist + (histb > stageb ? histb : stageb);
  L.cl = clb ? L.cnt + cntb : 0xFFFFFFFFu;
  L.total = L.cnt + cntb + clb;
  return L;
}

// the histogram slot of bin b: a pad after every 16 bins, so that lanes reading 16 bins each
// (a stride of 17 eight-byte slots) hit distinct banks
__device__ __forceinline__ int tk_hslot(unsigned b) { return (int)(b + (b >> 4)); }

template <int CTRL, int ROWS = 0xF, bool BOUND = false>
__device__ __forceinline__ unsigned tk_dpp(unsigned x) {
  return (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROWS, 0xF, BOUND);
}
// minimum / maximum over each row of 16 lanes, in every lane of the row
__device__ __forceinline__ unsigned row_min(unsigned x) {
  x = min(x, tk_dpp<0xB1>(x));   // quad_perm 1,0,3,2
  x = min(x, tk_dpp<0x4E>(x));   // quad_perm 2,3,0,1
  x = min(x, tk_dpp<0x141>(x));  // row_half_mirror
  return min(x, tk_dpp<0x140>(x));  // row_mirror
}
__device__ __forceinline__ unsigned row_max(unsigned x) {
  x = max(x, tk_dpp<0xB1>(x));
  x = max(x, tk_dpp<0x4E>(x));
  x = max(x, tk_dpp<0x141>(x));
  return max(x, tk_dpp<0x140>(x));
}
__device__ __forceinline__ unsigned rdlane(unsigned x, int l) {
  return (unsigned)__builtin_amdgcn_readlane((int)x, l);
}
__device__ __forceinline__ unsigned wave_min(unsigned x) {
  x = row_min(x);
  return min(min(rdlane(x, 0), rdlane(x, 16)), min(rdlane(x, 32), rdlane(x, 48)));
}
__device__ __forceinline__ unsigned wave_max(unsigned x) {
  x = row_max(x);
  return max(max(rdlane(x, 0), rdlane(x, 16)), max(rdlane(x, 32), rdlane(x, 48)));
}
// inclusive sum over each row of 16 lanes
__device__ __forceinline__ unsigned row_incl_sum(unsigned x) {
  x += tk_dpp<0x111, 0xF, true>(x);  // row_shr 1, 0 past the row start
  x += tk_dpp<0x112, 0xF, true>(x);
  x += tk_dpp<0x114, 0xF, true>(x);
  return x + tk_dpp<0x118, 0xF, true>(x);
}
// inclusive sum over the wave
__device__ __forceinline__ unsigned wave_incl_sum(unsigned x) {
  x = row_incl_sum(x);
  x += tk_dpp<0x142, 0xA>(x);  // row_bcast15: row 0's total into row 1, row 2's into row 3
  return x + tk_dpp<0x143, 0xC>(x);  // row_bcast31: rows 0-1's total into rows 2 and 3
}
// bit count of the lanes below this one in m, plus base
__device__ __forceinline__ unsigned lanes_below(unsigned long long m, unsigned base) {
  return __builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, base));
}
__device__ __forceinline__ unsigned long long tk_ballot(bool p) {
  return __builtin_amdgcn_ballot_w64(p);
}
// the fp32 value of an order key (the inverse of tk_order_key; +0 for the zero key)
__device__ __forceinline__ float tk_key_value(unsigned u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// One select pass's monotone bin map: linear in the fp32 value, or the order key shifted right.
struct TkBins {
  bool lin;
  float lo, scale;
  unsigned kmin, sh;
  __device__ __forceinline__ unsigned operator()(unsigned key) const {
    if (lin) {
      const float d = (tk_key_value(key) - lo) * scale;
      return d >= (float)(kNb - 1) ? (unsigned)(kNb - 1) : (unsigned)d;
    }
    return (key - kmin) >> sh;
  }
};

// The bin map of a pass over keys [lo, hi], lo < hi: linear bins while both ends are finite
// (keys strictly between those of -inf and +inf) and the scale is finite, for the first two
// passes only, so that the shift passes (each narrowing the key range at least 512-fold) bound
// the pass count.  Both maps send lo to bin 0 and hi to a bin >= 511, so every pass drops
// entries.
__device__ __forceinline__ TkBins tk_bin_map(unsigned lo, unsigned hi, int pass) {
  TkBins B;
  B.kmin = lo;
  B.sh = 0u;
  B.lin = false;
  B.lo = 0.0f;
  B.scale = 0.0f;
  if (pass < 2 && lo > 0x007FFFFFu && hi < 0xFF800000u) {
    const float vlo = tk_key_value(lo), span = tk_key_value(hi) - vlo;
    const float scale = (float)kNb / span;
    if (span > 0.0f && span <= 3.0e38f && scale > 0.0f && scale <= 3.0e38f) {
      B.lin = true;
      B.lo = vlo;
      B.scale = scale;
      return B;
    }
  }
  const int bits = 32 - __clz((int)(hi - lo));
  B.sh = bits > 10 ? (unsigned)(bits - 10) : 0u;
  return B;
}

template <int GN, int E, bool CLDS>
__global__ __launch_bounds__(kTkThreads) void topk_codes_rows(
    const float* __restrict__ tab, int64_t hq, int64_t hkv,
    int group, int nchunk, const uint16_t* __restrict__ codes, int64_t n, int c, int64_t k,
    int32_t* __restrict__ idx, float* __restrict__ score, TkLayout ly) {
  constexpr int kWaves = kTkThreads / 64;
  constexpr unsigned kNegInfKey = 0x007FFFFFu;  // the order key of -inf
  extern __shared__ __align__(16) unsigned char tk_smem[];
  float* lut = reinterpret_cast<float*>(tk_smem + ly.lut);  // [GN][c + 1]
  unsigned long long* hist =
      reinterpret_cast<unsigned long long*>(tk_smem + ly.hist);  // [GN][kNbPad]
  unsigned* cnt = reinterpret_cast<unsigned*>(tk_smem + ly.cnt);  // [c + 1]
  uint16_t* cl = reinterpret_cast<uint16_t*>(tk_smem + (CLDS ? ly.cl : 0u));
  __shared__ unsigned rng[GN][2];                 // a live set's key range (atomic min / max)
  __shared__ unsigned sel[GN][4];                 // a pass's bin, remaining rank, its entries
  __shared__ unsigned long long cand[GN][kCand];  // (weight << 32) | key of a small bin
  __shared__ unsigned ccnt[GN], s_tr[GN][2];
  __shared__ unsigned wsum[2][kWaves][2 * GN];    // per round parity and wave: above, equal
  const int cp = c + 1;  // table row pitch

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t wg = blockIdx.x;
  const int chunk = (int)(wg % nchunk);
  const int64_t bk = wg / nchunk;  // sequence * hkv + key/value head
  const int64_t b = bk / hkv, kvh = bk % hkv;
  const int g0 = chunk * GN;
  const int gv = group - g0 < GN ? group - g0 : GN;  // query heads of this group in use
  const int64_t row0 = b * hq + kvh * group + g0;    // their first output row

  // ---- 1. the group's tables from the table kernel (a slot past the group's last query
  // repeats it); their key ranges are reduced on the way.  A code row kept in LDS in 16-byte
  // pieces (at most two a thread) is loaded first, so that both loads are in flight together.
  const uint16_t* cg = codes + bk * n;
  const unsigned cu = (unsigned)c;
  const bool rows16 = CLDS && (n & 7) == 0;
  const int n8 = (int)(n >> 3);
  tk_u4 pre[kTkLdsCodes / 8 / kTkThreads];
  if (rows16)
#pragma unroll
    for (int q = 0; q < kTkLdsCodes / 8 / kTkThreads; ++q)
      if (t + kTkThreads * q < n8) pre[q] = reinterpret_cast<const tk_u4*>(cg)[t + kTkThreads * q];
  for (int j = t; j < GN * kNbPad; j += kTkThreads) hist[j] = 0ull;
  for (int j = t; j <= c; j += kTkThreads) cnt[j] = 0u;
  if (t < GN) {
    rng[t][0] = 0xFFFFFFFFu;
    rng[t][1] = 0u;
    ccnt[t] = 0u;
  }
  unsigned key[GN][E], klo[GN], khi[GN];
  {
    float acc[E][GN];
#pragma unroll
    for (int g = 0; g < GN; ++g) {
      const float* tr = tab + (row0 + (g < gv ? g : gv - 1)) * c;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int j = t + kTkThreads * e;
        acc[e][g] = tr[j < c ? j : c - 1];
      }
    }
#pragma unroll
    for (int g = 0; g < GN; ++g) {
      klo[g] = 0xFFFFFFFFu;
      khi[g] = 0u;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int j = t + kTkThreads * e;
        const float v = acc[e][g];
        key[g][e] = tk_order_key(v);
        if (j < c) {
          lut[g * cp + j] = v;
          klo[g] = min(klo[g], key[g][e]);
          khi[g] = max(khi[g], key[g][e]);
        }
      }
      if (t == 0) lut[g * cp + c] = -INFINITY;  // the score of every code >= c
      klo[g] = wave_min(klo[g]);
      khi[g] = wave_max(khi[g]);
    }
  }
  __syncthreads();
  if (lane == 0)
#pragma unroll
    for (int g = 0; g < GN; ++g) {
      atomicMin(&rng[g][0], klo[g]);
      atomicMax(&rng[g][1], khi[g]);
    }
  if (rows16) {  // eight codes a piece
#pragma unroll
    for (int q = 0; q < kTkLdsCodes / 8 / kTkThreads; ++q) {
      const int i = t + kTkThreads * q;
      if (i >= n8) break;
      const tk_u4 v = pre[q];
      reinterpret_cast<tk_u4*>(cl)[i] = v;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const unsigned lo = v[h] & 0xFFFFu, hi = v[h] >> 16;
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

  // ---- 2. select.  The live set of a query is the weighted entries with keys in [plo, phi]:
  // a bin of a monotone map holds a key interval.
  unsigned wgt[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = t + kTkThreads * e;
    wgt[e] = j < c ? cnt[j] : 0u;
  }
  const unsigned wneg = t == 0 ? cnt[c] : 0u;  // the -inf entry's weight, held by thread 0
  unsigned act = (1u << gv) - 1u;  // queries still selecting (uniform)
  unsigned plo[GN], phi[GN], rem[GN], bsel[GN], T[GN], R[GN];
  TkBins mp[GN];
  {
    const bool inv = cnt[c] != 0u;  // a code >= c occurs: -inf is a weighted score
#pragma unroll
    for (int g = 0; g < GN; ++g) {
      plo[g] = inv ? kNegInfKey : rng[g][0];
      phi[g] = rng[g][1];
      rem[g] = (unsigned)k;
      bsel[g] = 0u;
      T[g] = R[g] = 0u;
    }
  }
  for (int pass = 0; act != 0u; ++pass) {
    if (pass > 0) {  // the range of what the last pass kept
#pragma unroll
      for (int g = 0; g < GN; ++g) {
        if (!((act >> g) & 1u)) continue;
        unsigned lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
        for (int e = 0; e <= E; ++e) {
          const unsigned x = e < E ? key[g][e] : kNegInfKey, w = e < E ? wgt[e] : wneg;
          if (w != 0u && x >= plo[g] && x <= phi[g] && mp[g](x) == bsel[g]) {
            lo = min(lo, x);
            hi = max(hi, x);
          }
        }
        lo = wave_min(lo);
        hi = wave_max(hi);
        if (lane == 0) {
          atomicMin(&rng[g][0], lo);
          atomicMax(&rng[g][1], hi);
        }
      }
      __syncthreads();
#pragma unroll
      for (int g = 0; g < GN; ++g) {
        if (!((act >> g) & 1u)) continue;
        plo[g] = rng[g][0];
        phi[g] = rng[g][1];
      }
    }
    // one score left is T_g; else the weighted histogram of the live entries over the bins
#pragma unroll
    for (int g = 0; g < GN; ++g) {
      if (!((act >> g) & 1u)) continue;
      if (plo[g] == phi[g]) {
        T[g] = plo[g];
        R[g] = rem[g];
        act &= ~(1u << g);
        continue;
      }
      mp[g] = tk_bin_map(plo[g], phi[g], pass);
#pragma unroll
      for (int e = 0; e <= E; ++e) {
        const unsigned x = e < E ? key[g][e] : kNegInfKey, w = e < E ? wgt[e] : wneg;
        if (w != 0u && x >= plo[g] && x <= phi[g])
          atomicAdd(&hist[g * kNbPad + tk_hslot(mp[g](x))], (1ull << 32) | (unsigned long long)w);
      }
    }
    if (act == 0u) break;  // uniform
    __syncthreads();
    // wave g: the bin holding rank rem_g from the top.  Lane l holds bins 1023 - 16 l down to
    // 1008 - 16 l, and clears them for the next pass.
    if (wave < GN && ((act >> wave) & 1u)) {
      const int g = wave;
      unsigned long long* hg = hist + g * kNbPad + tk_hslot(kNb - 16 - 16 * lane);
      unsigned long long h[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) h[q] = hg[15 - q];
#pragma unroll
      for (int q = 0; q < 16; ++q) hg[q] = 0ull;
      unsigned sum = 0u;
#pragma unroll
      for (int q = 0; q < 16; ++q) sum += (unsigned)h[q];
      unsigned r = 0u;
#pragma unroll
      for (int q = 0; q < GN; ++q)
        if (q == g) r = rem[q];
      unsigned cum = wave_incl_sum(sum) - sum;
      int hit = -1;
      unsigned nrem = 0u, ne = 0u;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const unsigned w = (unsigned)h[q];
        if (hit < 0 && cum < r && cum + w >= r) {
          hit = kNb - 1 - 16 * lane - q;
          nrem = r - cum;
          ne = (unsigned)(h[q] >> 32);
        }
        cum += w;
      }
      // one lane holds the bin (the live weights add up to at least rem_g >= 1)
      if (hit >= 0) {
        sel[g][0] = (unsigned)hit;
        sel[g][1] = nrem;
        sel[g][2] = ne;
      }
      if (lane == 0) {  // the next pass's range reduction starts empty
        rng[g][0] = 0xFFFFFFFFu;
        rng[g][1] = 0u;
      }
    }
    __syncthreads();
    unsigned settle = 0u;
#pragma unroll
    for (int g = 0; g < GN; ++g) {
      if (!((act >> g) & 1u)) continue;
      bsel[g] = sel[g][0];
      rem[g] = sel[g][1];
      if (!mp[g].lin && mp[g].sh == 0u) {  // the bin is one key
        T[g] = mp[g].kmin + bsel[g];
        R[g] = rem[g];
        act &= ~(1u << g);
      } else if (sel[g][2] <= (unsigned)kCand) {
#pragma unroll
        for (int e = 0; e <= E; ++e) {
          const unsigned x = e < E ? key[g][e] : kNegInfKey, w = e < E ? wgt[e] : wneg;
          if (w != 0u && x >= plo[g] && x <= phi[g] && mp[g](x) == bsel[g])
            cand[g][atomicAdd(&ccnt[g], 1u)] = ((unsigned long long)w << 32) | (unsigned long long)x;
        }
        settle |= 1u << g;
      }
    }
    if (settle == 0u) continue;  // uniform
    __syncthreads();
    // wave g settles a small bin: the key with less than rem_g weight above it and at least
    // rem_g at or above it
    if (wave < GN && ((settle >> wave) & 1u)) {
      const int g = wave;
      unsigned r = 0u;
#pragma unroll
      for (int q = 0; q < GN; ++q)
        if (q == g) r = rem[q];
      const unsigned m = ccnt[g];
      const unsigned long long me = lane < (int)m ? cand[g][lane] : 0ull;
      const unsigned mk = (unsigned)me;
      unsigned above = 0u, eq = 0u;
      for (unsigned j = 0; j < m; ++j) {
        const unsigned long long o = cand[g][j];
        const unsigned ok = (unsigned)o, ow = (unsigned)(o >> 32);
        above += ok > mk ? ow : 0u;
        eq += ok == mk ? ow : 0u;
      }
      if (lane < (int)m && above < r && r <= above + eq) {  // equal keys write equal values
        s_tr[g][0] = mk;
        s_tr[g][1] = r - above;
      }
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < GN; ++g)
      if ((settle >> g) & 1u) {
        T[g] = s_tr[g][0];
        R[g] = s_tr[g][1];
      }
    act &= ~settle;
  }

  // ---- 3. class byte per code (the code histogram is no longer needed)
  uint8_t* cls = reinterpret_cast<uint8_t*>(cnt);
  __syncthreads();  // every thread has read the code histogram
  for (int j = t; j <= c; j += kTkThreads) {
    unsigned v = 0u;
#pragma unroll
    for (int g = 0; g < GN; ++g) {
      const unsigned u = tk_order_key(lut[g * cp + j]);
      v |= (u > T[g] ? 1u : 0u) << (2 * g);
      v |= (u == T[g] ? 1u : 0u) << (2 * g + 1);
    }
    cls[j] = (uint8_t)v;
  }
  __syncthreads();

  // ---- 4. output.  Rounds of 16384 tokens; lane l of wave w takes tokens r0 + 1024 w + 16 l
  // + b (b < 16), their class bytes packed four to a register.  Per query: lane counts by bit
  // counts, wave scans by DPP, one barrier for the counts across waves, then each wave lists its
  // taken tokens in LDS (a token not taken goes to the thread's trash slot) and copies the list
  // out whole.
  unsigned* stage = reinterpret_cast<unsigned*>(tk_smem + ly.hist);  // [kWaves][GN][scap]
  unsigned* trash = stage + kWaves * GN * ly.scap + t;
  unsigned run_a[GN], run_e[GN];  // tokens above / at T_g in the rounds before
#pragma unroll
  for (int g = 0; g < GN; ++g) run_a[g] = run_e[g] = 0u;
  auto token_code = [&](int64_t i) -> unsigned {
    const unsigned x = CLDS ? (unsigned)cl[i] : (unsigned)cg[i];
    return x < cu ? x : cu;
  };
  for (int64_t r0 = 0, par = 0; r0 < n; r0 += kTkRound, par ^= 1) {
    const int64_t tb = r0 + (int64_t)wave * (kTkRound / kWaves) + 16 * lane;
    unsigned V[4];
    {
      unsigned cc[16];
      if (CLDS && tb + 16 <= n) {
        const uint4 x0 = *reinterpret_cast<const uint4*>(cl + tb);
        const uint4 x1 = *reinterpret_cast<const uint4*>(cl + tb + 8);
        const unsigned w[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int h = 0; h < 8; ++h) {
          cc[2 * h] = min(w[h] & 0xFFFFu, cu);
          cc[2 * h + 1] = min(w[h] >> 16, cu);
        }
      } else {
#pragma unroll
        for (int b = 0; b < 16; ++b) cc[b] = tb + b < n ? token_code(tb + b) : cu;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        unsigned v = 0u;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const int b = 4 * q + h;
          v |= (tb + b < n ? (unsigned)cls[cc[b]] : 0u) << (8 * h);
        }
        V[q] = v;
      }
    }
    unsigned xa[GN], xe[GN], ta[GN], te[GN];  // lane-exclusive and wave counts: above, at T_g
#pragma unroll
    for (int g = 0; g < GN; ++g) {
      const unsigned sa = 0x01010101u << (2 * g), se = sa << 1;
      unsigned na = 0u, ne = 0u;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        na += __popc(V[q] & sa);
        ne += __popc(V[q] & se);
      }
      const unsigned ia = wave_incl_sum(na), ie = wave_incl_sum(ne);
      xa[g] = ia - na;
      xe[g] = ie - ne;
      ta[g] = rdlane(ia, 63);
      te[g] = rdlane(ie, 63);
    }
    if (lane == 0)
#pragma unroll
      for (int g = 0; g < GN; ++g) {
        wsum[par][wave][2 * g] = ta[g];
        wsum[par][wave][2 * g + 1] = te[g];
      }
    __syncthreads();  // wsum[par] is rewritten two rounds on, after the next round's barrier
#pragma unroll
    for (int g = 0; g < GN; ++g) {
      const unsigned wa = lane < kWaves ? wsum[par][lane][2 * g] : 0u;
      const unsigned we = lane < kWaves ? wsum[par][lane][2 * g + 1] : 0u;
      const unsigned iwa = row_incl_sum(wa), iwe = row_incl_sum(we);
      const unsigned pe = run_e[g] + rdlane(iwe, wave) - rdlane(we, wave);  // at T_g before
      const unsigned pa = run_a[g] + rdlane(iwa, wave) - rdlane(wa, wave) + min(pe, R[g]);
      run_a[g] += rdlane(iwa, kWaves - 1);
      run_e[g] += rdlane(iwe, kWaves - 1);
      if (g >= gv) continue;
      // the taken bit of each token, at bit 8 h of T[q] for token 4 q + h
      const unsigned ab = 0x01010101u;
      unsigned T[4], excl, cnt_w;
      if (pe + te[g] <= R[g]) {  // every token at T_g in this wave is taken (uniform)
#pragma unroll
        for (int q = 0; q < 4; ++q) T[q] = ((V[q] >> (2 * g)) | (V[q] >> (2 * g + 1))) & ab;
        excl = xa[g] + xe[g];
        cnt_w = ta[g] + te[g];
      } else if (pe >= R[g]) {  // none is
#pragma unroll
        for (int q = 0; q < 4; ++q) T[q] = (V[q] >> (2 * g)) & ab;
        excl = xa[g];
        cnt_w = ta[g];
      } else {  // the wave holding the R_g-th: each lane takes its first m tokens at T_g
        const unsigned before = pe + xe[g];
        unsigned m = before < R[g] ? R[g] - before : 0u;
        unsigned ct = 0u;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          unsigned tq = 0u;
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const unsigned byte = V[q] >> (8 * h + 2 * g);
            unsigned tk = byte & 1u;
            if ((byte & 2u) && m != 0u) {
              tk = 1u;
              --m;
            }
            tq |= tk << (8 * h);
            ct += tk;
          }
          T[q] = tq;
        }
        const unsigned ic = wave_incl_sum(ct);
        excl = ic - ct;
        cnt_w = rdlane(ic, 63);
      }
      int32_t* orow = idx + (row0 + g) * k;
      float* srow = score ? score + (row0 + g) * k : nullptr;
      if (cnt_w <= (unsigned)ly.scap) {  // uniform
        unsigned* sg = stage + (wave * GN + g) * ly.scap;
        unsigned p = excl;
#pragma unroll
        for (int b = 0; b < 16; ++b) {
          const unsigned bit = (T[b >> 2] >> (8 * (b & 3))) & 1u;
          *(bit ? sg + p : trash) = (unsigned)(tb + b);
          p += bit;
        }
        // the wave's list (its own LDS operations complete in order)
        for (unsigned i = lane; i < cnt_w; i += 64) {
          const unsigned tok = sg[i], pos = pa + i;
          if (pos < (unsigned)k) {  // the bound turns any inconsistency into a wrong answer
            orow[pos] = (int32_t)tok;
            if (srow) srow[pos] = lut[g * cp + token_code(tok)];
          }
        }
      } else {  // longer than the staging slots: straight to global memory
        unsigned p = pa + excl;
#pragma unroll
        for (int b = 0; b < 16; ++b) {
          const unsigned bit = (T[b >> 2] >> (8 * (b & 3))) & 1u;
          if (bit && p < (unsigned)k) {
            orow[p] = (int32_t)(tb + b);
            if (srow) srow[p] = lut[g * cp + token_code(tb + b)];
          }
          p += bit;
        }
      }
    }
  }
}

template <int GN, int E, bool CLDS>
int topk_launch3(dim3 grid, hipStream_t s, const float* cb, int64_t hq,
                 int64_t hkv, int group, int nchunk, const uint16_t* codes, int64_t n, int c,
                 int64_t k, int32_t* idx, float* score, const TkLayout& ly) {
  auto kern = topk_codes_rows<GN, E, CLDS>;
  A2ATS_TRY(set_dynamic_lds(kern, ly.total));
  return launch("topk_codes", kern, grid, dim3(kTkThreads), ly.total, s, cb, hq, hkv, group,
                nchunk, codes, n, c, k, idx, score, ly);
}

template <int GN, int E>
int topk_launch2(dim3 grid, hipStream_t s, const float* cb, int64_t hq,
                 int64_t hkv, int group, int nchunk, const uint16_t* codes, int64_t n, int c,
                 int64_t k, int32_t* idx, float* score) {
  const TkLayout ly = tk_layout(GN, c, n);
  if (ly.cl != 0xFFFFFFFFu)
    return topk_launch3<GN, E, true>(grid, s, cb, hq, hkv, group, nchunk, codes, n, c, k,
                                     idx, score, ly);
  return topk_launch3<GN, E, false>(grid, s, cb, hq, hkv, group, nchunk, codes, n, c, k,
                                    idx, score, ly);
}

// table entries a thread holds: C <= 1024, 2048, 4096
template <int GN>
int topk_launch(dim3 grid, hipStream_t s, const float* cb, int64_t hq,
                int64_t hkv, int group, int nchunk, const uint16_t* codes, int64_t n, int c,
                int64_t k, int32_t* idx, float* score) {
  if (c <= kTkThreads)
    return topk_launch2<GN, 1>(grid, s, cb, hq, hkv, group, nchunk, codes, n, c, k, idx,
                               score);
  if (c <= 2 * kTkThreads)
    return topk_launch2<GN, 2>(grid, s, cb, hq, hkv, group, nchunk, codes, n, c, k, idx,
                               score);
  return topk_launch2<GN, 4>(grid, s, cb, hq, hkv, group, nchunk, codes, n, c, k, idx,
                             score);
}

int topk_dispatch(int gn, dim3 grid, hipStream_t s, const float* cb,
                  int64_t hq, int64_t hkv, int group, int nchunk, const uint16_t* codes,
                  int64_t n, int c, int64_t k, int32_t* idx, float* score) {
  switch (gn) {
    case 1:
      return topk_launch<1>(grid, s, cb, hq, hkv, group, nchunk, codes, n, c, k, idx, score);
    case 2:
      return topk_launch<2>(grid, s, cb, hq, hkv, group, nchunk, codes, n, c, k, idx, score);
    case 3:
      return topk_launch<3>(grid, s, cb, hq, hkv, group, nchunk, codes, n, c, k, idx, score);
    default:
      return topk_launch<4>(grid, s, cb, hq, hkv, group, nchunk, codes, n, c, k, idx, score);
  }
}

}  // namespace
}  // namespace a2ats

using namespace a2ats;

// The workspace: the queries' tables [batch * hq][c] in fp32.

extern "C" size_t a2ats_topk_workspace(int64_t batch, int64_t hq, int64_t c) {
  if (batch < 1 || hq < 1 || c < 1 || c > kTkMaxC) return 0;
  return align_up((size_t)(batch * hq * c) * sizeof(float));
}

extern "C" int a2ats_topk_codes(const void* qb, int q_dtype, int64_t batch, int64_t hq,
                                int64_t hkv, int64_t d, const uint16_t* codes, int64_t n,
                                const float* codebook, int64_t c, int64_t k, int32_t* idx,
                                float* score, void* workspace, size_t workspace_bytes,
                                void* stream) {
  if (q_dtype != A2ATS_F32 && q_dtype != A2ATS_BF16) return A2ATS_EDTYPE;
  if (d != kD || batch < 1 || hq < 1 || hkv < 1 || hq % hkv != 0) return A2ATS_EINVAL;
  if (n < 0 || n > 0x7FFFFFFF || c < 1 || c > kTkMaxC || k < 0 || k > n) return A2ATS_EINVAL;
  const int group = (int)(hq / hkv);
  const int gn = group < 4 ? group : 4;
  const int nchunk = (group + gn - 1) / gn;
  if (batch * hkv * nchunk > 0x7FFFFFFF || batch * hq > 0x7FFFFFFF) return A2ATS_EINVAL;
  if (hkv * ((c + kTbStrip - 1) / kTbStrip) * ((batch * group + kTbChunk - 1) / kTbChunk) >
      0x7FFFFFFF)
    return A2ATS_EINVAL;
  if (n == 0 || k == 0) return A2ATS_OK;
  if (!qb || !codes || !codebook || !idx) return A2ATS_EINVAL;
  if ((reinterpret_cast<uintptr_t>(qb) & 15) != 0) return A2ATS_EINVAL;
  if (!ws_ok(workspace, workspace_bytes, a2ats_topk_workspace(batch, hq, c)))
    return A2ATS_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* tab = static_cast<float*>(workspace);
  const int nstrip = (int)((c + kTbStrip - 1) / kTbStrip);
  const int64_t nqch = (batch * group + kTbChunk - 1) / kTbChunk;
  const dim3 tgrid((unsigned)(hkv * nstrip * nqch));
  const dim3 tblock(kTbThreads);
  if (q_dtype == A2ATS_F32)
    A2ATS_TRY(launch("topk_table", topk_table<A2ATS_F32>, tgrid, tblock, 0, s, qb, codebook, batch,
                     hq, group, (int)c, nstrip, (int)nqch, tab));
  else
    A2ATS_TRY(launch("topk_table", topk_table<A2ATS_BF16>, tgrid, tblock, 0, s, qb, codebook, batch,
                     hq, group, (int)c, nstrip, (int)nqch, tab));
  const dim3 grid((unsigned)(batch * hkv * nchunk));
  return topk_dispatch(gn, grid, s, tab, hq, hkv, group, nchunk, codes, n, (int)c, k, idx,
                       score);
}
