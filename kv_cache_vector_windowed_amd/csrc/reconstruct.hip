// reconstruct: centroid gather + windowed RoPE of every cached token, each decode step.
// "A2ATS-adapted -- Windowed RoPE + Query-Aware Retrieval VQ", How it works steps 3-4, and
// the "paper fidelity" section of the later docs (Eq. 11-12, a2ats_b).
//
//   x = codebook[h, code]                 the pre-RoPE key (dequantisation)
//   near (0 <= cur - pos < W):            RoPE(x, pos)
//   far, fixed offset:                    RoPE(x, cur - b)   -- the key-side image of Eq. 11:
//                                         RoPE(q, cur) . RoPE(k, cur - b) = RoPE(q, b) . k
//   far, unrotated:                       x                  -- Eq. 12 literally
// RoPE rotates half-split pairs (i, i + d/2) by pos * base^(-2i/d).
//
// Kernels
//   rope_table   (R + 1) rows of fp64 (cos, sin): row r < R is position cur - r,
//                R = min(max(W, 0), cur + 1); row R is the far rotation (identity when far
//                keys stay unrotated).  With a workspace that has room for them
//                (rope_prep), the same launch also writes every centroid's far row, rotated
//                and rounded once: all far tokens of a head share the rotation, so a far
//                token's row is a copy of its centroid's far row.
//   rope_gather  HBM-write-bound stream: each thread owns a fixed group of P pairs of the
//                head dimension (P = 4 for fp32 output, 8 for bf16, so every store is 16 B),
//                takes the far row's cos/sin for its pairs from a copy the workgroup stages
//                in LDS (with the codes and positions of all its work items), gathers the
//                centroid from L2, rotates in fp64, rounds once to the output type, and
//                writes with non-temporal stores (a far token with far rows prepared: its
//                centroid's far row copied).  Work
//                items are (batch, head, 64-token chunk); item k has head k % heads and the
//                grid is a multiple of 8 * heads, so a workgroup always serves one head and,
//                with 8 heads, each XCD (workgroups are dealt round-robin over the 8 XCDs)
//                keeps a single head's codebook in its L2.
#include <mutex>

#include "common.hpp"

namespace a2ats {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));
typedef double d2 __attribute__((ext_vector_type(2)));

constexpr int kD = A2ATS_HEAD_DIM;
constexpr int kHalf = kD / 2;
constexpr int kChunkF32 = 64;   // tokens per work item, fp32 output
constexpr int kChunkBf16 = 64;  // tokens per work item, bf16 output
// Work items per workgroup (the grid is rounded to a multiple of 8 * heads and is at least
// kGridMin).  rope_gather stages the codes and positions of all of a workgroup's items in LDS
// first, so that their reads, which miss every cache in a decode step, are in flight
// together; four items a workgroup, measured on the decode and long-context workloads after
// a cache-evicting read (0.48-0.51 -> 0.62-0.66 and 0.36-0.41 -> 0.50 of HBM; back to back
// within about 7% of the one-item grid either way; two and eight items measured lower).
// pq_gather reads each item's code rows in
// its loop (staging them the same way measured no faster on the sub-vector layer workload):
// one fp32 and four bf16 items a workgroup.  A later item's loads wait, in order, behind the
// earlier item's stores (one vector memory counter); a software-pipelined variant that
// issues the next item's row loads before the current item's stores needs more registers and
// measured slower.
constexpr int kGatherItems = 4;
constexpr int kItemsPerWgF32 = 1;
constexpr int kItemsPerWgBf16 = 4;
constexpr int kGridMin = 256;

// (cos, sin) of the rotation of pair i at position p: angle p * base^(-2i/d), fp64.  The
// table, the incremental update and the query-side rotation all take their angles from here,
// so equal positions give bitwise equal rotations in every kernel.
__device__ __forceinline__ d2 rope_cs(double p, int i, int d, double base) {
  const double theta = pow(base, -2.0 * (double)i / (double)d);
  const double phi = p * theta;
  d2 v;
  v.x = cos(phi);
  v.y = sin(phi);
  return v;
}

__global__ __launch_bounds__(256) void rope_table(int64_t rows_near, int64_t cur, int64_t far_pos,
                                                  int far_identity, double base, int d,
                                                  d2* __restrict__ table) {
  const int half = d / 2;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (rows_near + 1) * half) return;
  const int64_t r = e / half;
  const int i = (int)(e % half);
  d2 v;
  if (r == rows_near && far_identity) {
    v.x = 1.0;
    v.y = 0.0;
  } else {
    v = rope_cs((r == rows_near) ? (double)far_pos : (double)(cur - r), i, d, base);
  }
  table[e] = v;
}

typedef __bf16 bf2 __attribute__((ext_vector_type(2)));

// Two fp32 values to a packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  bf2 v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(unsigned, v);
}

__device__ __forceinline__ bool in_window(int64_t cur, int64_t pos, int64_t window) {
  const int64_t delta = cur - pos;
  return delta >= 0 && delta < window;
}

// The rotation of P pairs, (lo, hi) = (xl c - xh s, xh c + xl s), as one product and one
// fused multiply-add each; every kernel that writes reconstructed rows uses it.
template <typename real, int P>
__device__ __forceinline__ void rotate_pairs(const float (&xl)[P], const float (&xh)[P],
                                             const real (&cs)[P], const real (&sn)[P],
                                             real (&lo)[P], real (&hi)[P]) {
#pragma unroll
  for (int k = 0; k < P; ++k) {
    lo[k] = fma((real)xl[k], cs[k], -((real)xh[k] * sn[k]));
    hi[k] = fma((real)xh[k], cs[k], (real)xl[k] * sn[k]);
  }
}

// Moves y = fp32(x) one fp32 unit toward x when y lies exactly halfway between two bf16
// values while x does not.  Only there can the nearest-even rounding of y to bf16 differ
// from that of x: a bf16 midpoint is itself an fp32 value, so x below (above) a midpoint
// gives y at or below (above) it, and y equal to the midpoint only in this case.
__device__ __forceinline__ float bf16_tie_fix(double x, float y) {
  const unsigned b = __float_as_uint(y);
  if ((b & 0xFFFFu) != 0x8000u || (double)y == x) return y;
  return __uint_as_float(fabs(x) > fabs((double)y) ? b + 1u : b - 1u);
}

// P pairs of one row rounded once to the output type, as the two 16-byte words of the row
// (low half at pair i0, high half at i0 + d/2).  bf16: the fp32 roundings of the fp64
// values are rounded to bf16 (nearest even); the rare fp32 value on a bf16 midpoint is
// corrected first (one branch per thread for all 2P values), so the result is the single
// nearest-even rounding of the fp64 value.
template <bool BF16, int P>
__device__ __forceinline__ void round_pairs(const double (&lo)[P], const double (&hi)[P], u4& a,
                                            u4& bb) {
  if constexpr (BF16) {
    static_assert(P == 8, "bf16 rows: 8 pairs per thread");
    float fl[P], fh[P];
    bool tie = false;
#pragma unroll
    for (int k = 0; k < P; ++k) {
      fl[k] = (float)lo[k];
      fh[k] = (float)hi[k];
      tie |= (__float_as_uint(fl[k]) & 0xFFFFu) == 0x8000u;
      tie |= (__float_as_uint(fh[k]) & 0xFFFFu) == 0x8000u;
    }
    if (__builtin_expect(tie, 0)) {
#pragma unroll
      for (int k = 0; k < P; ++k) {
        fl[k] = bf16_tie_fix(lo[k], fl[k]);
        fh[k] = bf16_tie_fix(hi[k], fh[k]);
      }
    }
    a.x = pack_bf16x2(fl[0], fl[1]);
    a.y = pack_bf16x2(fl[2], fl[3]);
    a.z = pack_bf16x2(fl[4], fl[5]);
    a.w = pack_bf16x2(fl[6], fl[7]);
    bb.x = pack_bf16x2(fh[0], fh[1]);
    bb.y = pack_bf16x2(fh[2], fh[3]);
    bb.z = pack_bf16x2(fh[4], fh[5]);
    bb.w = pack_bf16x2(fh[6], fh[7]);
  } else {
    static_assert(P == 4, "fp32 rows: 4 pairs per thread");
    a.x = __float_as_uint((float)lo[0]); a.y = __float_as_uint((float)lo[1]);
    a.z = __float_as_uint((float)lo[2]); a.w = __float_as_uint((float)lo[3]);
    bb.x = __float_as_uint((float)hi[0]); bb.y = __float_as_uint((float)hi[1]);
    bb.z = __float_as_uint((float)hi[2]); bb.w = __float_as_uint((float)hi[3]);
  }
}

// The two words of P pairs written with non-temporal stores at element offset ooff.
template <bool BF16>
__device__ __forceinline__ void store_words(void* out, int64_t ooff, const u4& a, const u4& bb) {
  if constexpr (BF16) {
    uint16_t* o = static_cast<uint16_t*>(out) + ooff;
    __builtin_nontemporal_store(a, reinterpret_cast<u4*>(o));
    __builtin_nontemporal_store(bb, reinterpret_cast<u4*>(o + kHalf));
  } else {
    float* o = static_cast<float*>(out) + ooff;
    __builtin_nontemporal_store(a, reinterpret_cast<u4*>(o));
    __builtin_nontemporal_store(bb, reinterpret_cast<u4*>(o + kHalf));
  }
}

template <bool BF16, int P>
__device__ __forceinline__ void store_pairs(void* out, int64_t ooff, const double (&lo)[P],
                                            const double (&hi)[P]) {
  u4 a, bb;
  round_pairs<BF16, P>(lo, hi, a, bb);
  store_words<BF16>(out, ooff, a, bb);
}

// The two words of P pairs at element offset off of a row store (for copying).
template <bool BF16>
__device__ __forceinline__ void load_words(const void* src, int64_t off, u4& a, u4& bb) {
  if constexpr (BF16) {
    const uint16_t* p = static_cast<const uint16_t*>(src) + off;
    a = *reinterpret_cast<const u4*>(p);
    bb = *reinterpret_cast<const u4*>(p + kHalf);
  } else {
    const float* p = static_cast<const float*>(src) + off;
    a = *reinterpret_cast<const u4*>(p);
    bb = *reinterpret_cast<const u4*>(p + kHalf);
  }
}

// Centroid halves of P pairs starting at pair i0 (row x of the codebook).
template <int P>
__device__ __forceinline__ void load_pairs(const float* x, float (&xl)[P], float (&xh)[P]) {
#pragma unroll
  for (int k = 0; k < P; k += 4) {
    const f4 a = *reinterpret_cast<const f4*>(x + k);
    const f4 bb = *reinterpret_cast<const f4*>(x + kHalf + k);
    xl[k] = a.x; xl[k + 1] = a.y; xl[k + 2] = a.z; xl[k + 3] = a.w;
    xh[k] = bb.x; xh[k + 1] = bb.y; xh[k + 2] = bb.z; xh[k + 3] = bb.w;
  }
}

// The rope table (as rope_table, blocks [0, tab_blocks)) and, in the blocks after it, the far
// rotation of every codebook row, rounded once to the output type: farcb [heads][c][d].  A far
// token's reconstructed row is then a copy of its centroid's far row, bit for bit what
// rope_gather computes for it (the same fp64 angles from rope_cs, rotation and rounding).
// Far rows: 256 / (d/2 / P) rows per workgroup; the workgroup first forms the 64 far
// (cos, sin) in LDS.
template <bool BF16>
__global__ __launch_bounds__(256) void rope_prep(int64_t rows_near, int64_t cur, int64_t far_pos,
                                                 int far_identity, double base, d2* __restrict__ table,
                                                 int64_t tab_blocks, const float* __restrict__ cb,
                                                 int64_t rows_far, void* __restrict__ farcb) {
  constexpr int P = BF16 ? 8 : 4;
  constexpr int TPT = kHalf / P;          // threads per row
  constexpr int RPW = 256 / TPT;          // rows per workgroup
  const int t = threadIdx.x;
  if ((int64_t)blockIdx.x < tab_blocks) {
    const int64_t e = (int64_t)blockIdx.x * 256 + t;
    if (e >= (rows_near + 1) * kHalf) return;
    const int64_t r = e / kHalf;
    const int i = (int)(e % kHalf);
    d2 v;
    if (r == rows_near && far_identity) {
      v.x = 1.0;
      v.y = 0.0;
    } else {
      v = rope_cs((r == rows_near) ? (double)far_pos : (double)(cur - r), i, kD, base);
    }
    table[e] = v;
    return;
  }
  __shared__ d2 s_far[kHalf];
  if (t < kHalf) {
    d2 v;
    if (far_identity) {
      v.x = 1.0;
      v.y = 0.0;
    } else {
      v = rope_cs((double)far_pos, t, kD, base);
    }
    s_far[t] = v;
  }
  __syncthreads();
  const int64_t row = ((int64_t)blockIdx.x - tab_blocks) * RPW + t / TPT;
  if (row >= rows_far) return;
  const int i0 = (t % TPT) * P;
  float xl[P], xh[P];
  load_pairs<P>(cb + row * kD + i0, xl, xh);
  double cs[P], sn[P], lo[P], hi[P];
#pragma unroll
  for (int k = 0; k < P; ++k) {
    cs[k] = s_far[i0 + k].x;
    sn[k] = s_far[i0 + k].y;
  }
  rotate_pairs<double, P>(xl, xh, cs, sn, lo, hi);
  u4 a, bb;
  round_pairs<BF16, P>(lo, hi, a, bb);
  if constexpr (BF16) {
    uint16_t* o = static_cast<uint16_t*>(farcb) + row * kD + i0;
    *reinterpret_cast<u4*>(o) = a;
    *reinterpret_cast<u4*>(o + kHalf) = bb;
  } else {
    float* o = static_cast<float*>(farcb) + row * kD + i0;
    *reinterpret_cast<u4*>(o) = a;
    *reinterpret_cast<u4*>(o + kHalf) = bb;
  }
}

// fp32 output: 4 pairs per thread; bf16 output: 8 pairs per thread (16-byte stores).  The
// rotation is fp64 for both, written as one product and one fused multiply-add (so the
// rounding steps do not depend on how the compiler contracts the expression), and rounded
// once to the output type.
// Each thread handles U tokens of a chunk at once.  The codes and positions of the
// workgroup's next chunk are fetched before the current chunk's centroids are gathered,
// rotated and stored, so the dependent loads of one chunk overlap the work of the previous.
template <bool BF16>
__global__ __launch_bounds__(256) void rope_gather(
    const uint16_t* __restrict__ codes, const int32_t* __restrict__ positions, int64_t heads,
    int64_t n, const float* __restrict__ cb, int64_t c, int64_t cur, int64_t window,
    int64_t rows_near, const d2* __restrict__ table, const void* __restrict__ farcb,
    void* __restrict__ out, int64_t items) {
  constexpr int P = BF16 ? 8 : 4;        // pairs per thread
  constexpr int TPT = kHalf / P;         // threads per token
  constexpr int TOK = 256 / TPT;         // tokens per pass of the workgroup
  constexpr int CH = BF16 ? kChunkBf16 : kChunkF32;
  constexpr int U = CH / TOK;            // tokens per thread per chunk
  using real = double;
  const int t = threadIdx.x;
  const int g = t % TPT;                 // pair group: pairs [g*P, g*P + P)
  const int tk = t / TPT;
  const int i0 = g * P;
  // the far rotation, read once per workgroup (one 16-byte load per pair) and shared in LDS
  __shared__ d2 s_far[kHalf];
  if (t < kHalf) s_far[t] = table[rows_near * kHalf + t];
  __syncthreads();
  real fc[P], fs[P];
#pragma unroll
  for (int k = 0; k < P; ++k) {
    const d2 v = s_far[i0 + k];
    fc[k] = (real)v.x;
    fs[k] = (real)v.y;
  }
  const int64_t chunks = (n + CH - 1) / CH;
  int code[U], pos[U];
  auto fetch = [&](int64_t item, int* cd, int* ps) {
    const int64_t h = item % heads;
    const int64_t rest = item / heads;
    const int64_t b = rest / chunks;
    const int64_t t0 = (rest % chunks) * CH;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t tok = t0 + u * TOK + tk;
      cd[u] = 0;
      ps[u] = -1;
      if (item < items && tok < n) {
        cd[u] = codes[(b * heads + h) * n + tok];
        ps[u] = positions[b * n + tok];
      }
    }
  };
  // the codes and positions of this workgroup's items (at most kGatherItems; more would be
  // read in the loop), staged in LDS
  __shared__ int s_code[kGatherItems][CH], s_pos[kGatherItems][CH];
  for (int f = t; f < kGatherItems * CH; f += 256) {
    const int k = f / CH, j = f % CH;
    const int64_t item = (int64_t)blockIdx.x + (int64_t)k * gridDim.x;
    const int64_t h = item % heads;
    const int64_t rest = item / heads;
    const int64_t b = rest / chunks;
    const int64_t tok = (rest % chunks) * CH + j;
    int cd = 0, ps = -1;
    if (item < items && tok < n) {
      cd = codes[(b * heads + h) * n + tok];
      ps = positions[b * n + tok];
    }
    s_code[k][j] = cd;
    s_pos[k][j] = ps;
  }
  __syncthreads();
  auto take = [&](int k, int64_t item, int* cd, int* ps) {
    if (k < kGatherItems) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        cd[u] = s_code[k][u * TOK + tk];
        ps[u] = s_pos[k][u * TOK + tk];
      }
    } else {
      fetch(item, cd, ps);
    }
  };
  take(0, blockIdx.x, code, pos);
  int kn = 0;  // the next item's slot
  for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
    int ncode[U], npos[U];
    take(++kn, item + gridDim.x, ncode, npos);
    const int64_t h = item % heads;
    const int64_t rest = item / heads;
    const int64_t b = rest / chunks;
    const int64_t t0 = (rest % chunks) * CH;
    const float* cbh = cb + h * c * kD;
    float xl[U][P], xh[U][P];
    u4 wa[U], wb[U];
    bool copy[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t tok = t0 + u * TOK + tk;
      const bool ok = tok < n && code[u] < c && pos[u] >= 0;
      // a far token with pre-rotated far rows: its row is copied
      copy[u] = ok && farcb != nullptr && !in_window(cur, pos[u], window);
      if (copy[u]) load_words<BF16>(farcb, (h * c + code[u]) * kD + i0, wa[u], wb[u]);
      else load_pairs<P>(cbh + (int64_t)(ok ? code[u] : 0) * kD + i0, xl[u], xh[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t tok = t0 + u * TOK + tk;
      if (tok >= n) continue;
      const int64_t ooff = ((b * heads + h) * n + tok) * kD + i0;
      if (copy[u]) {
        store_words<BF16>(out, ooff, wa[u], wb[u]);
        continue;
      }
      real lo[P], hi[P];
      if ((int64_t)code[u] >= c || pos[u] < 0) {
#pragma unroll
        for (int k = 0; k < P; ++k) lo[k] = hi[k] = (real)NAN;
      } else {
        real cs[P], sn[P];
        const int64_t delta = cur - (int64_t)pos[u];
        if (in_window(cur, pos[u], window)) {
          const d2* row = table + delta * kHalf + i0;  // delta < rows_near since pos >= 0
#pragma unroll
          for (int k = 0; k < P; ++k) {
            const d2 v = row[k];
            cs[k] = (real)v.x;
            sn[k] = (real)v.y;
          }
        } else {
#pragma unroll
          for (int k = 0; k < P; ++k) {
            cs[k] = fc[k];
            sn[k] = fs[k];
          }
        }
        rotate_pairs<real, P>(xl[u], xh[u], cs, sn, lo, hi);
      }
      store_pairs<BF16, P>(out, ooff, lo, hi);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      code[u] = ncode[u];
      pos[u] = npos[u];
    }
  }
}

// Sub-vector (product) codes: a token's key is the concatenation of d / SUB sub-centroids
// of one shared codebook [k, SUB] ("A2ATS-adapted" docs, "What you get with the
// defaults").  Same work items and arithmetic as rope_gather; each thread reads the
// token's whole code row (d / SUB bytes), takes for each 4-dimension group of its pairs the
// sub-centroid slice that covers it, and rotates and stores exactly as rope_gather does.  A
// token with any code >= k, or a negative position, gets a row of NaN.
template <bool BF16, int SUB>
__global__ __launch_bounds__(256) void pq_gather(
    const uint8_t* __restrict__ codes, const int32_t* __restrict__ positions, int64_t heads,
    int64_t n, const float* __restrict__ cb, int64_t k, int64_t cur, int64_t window,
    int64_t rows_near, const d2* __restrict__ table, void* __restrict__ out, int64_t items) {
  constexpr int P = BF16 ? 8 : 4;
  constexpr int TPT = kHalf / P;
  constexpr int TOK = 256 / TPT;
  constexpr int CH = BF16 ? kChunkBf16 : kChunkF32;
  constexpr int U = CH / TOK;
  constexpr int M = kD / SUB;   // codes per token
  constexpr int NW = M / 4;     // 32-bit words of a code row (4 for SUB 8, 8 for SUB 4)
  static_assert(SUB % 4 == 0 && M % 16 == 0, "code rows of whole 16-byte vectors");
  using real = double;
  const int t = threadIdx.x;
  const int g = t % TPT;
  const int tk = t / TPT;
  const int i0 = g * P;
  __shared__ d2 s_far[kHalf];
  if (t < kHalf) s_far[t] = table[rows_near * kHalf + t];
  __syncthreads();
  real fc[P], fs[P];
#pragma unroll
  for (int kk = 0; kk < P; ++kk) {
    const d2 v = s_far[i0 + kk];
    fc[kk] = (real)v.x;
    fs[kk] = (real)v.y;
  }
  const int64_t chunks = (n + CH - 1) / CH;
  for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
    const int64_t h = item % heads;
    const int64_t rest = item / heads;
    const int64_t b = rest / chunks;
    const int64_t t0 = (rest % chunks) * CH;
    unsigned cw[U][NW];
    int pos[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t tok = t0 + u * TOK + tk;
      pos[u] = -1;
#pragma unroll
      for (int q = 0; q < NW; ++q) cw[u][q] = 0u;
      if (tok < n) {
        const uint4* cr = reinterpret_cast<const uint4*>(codes + ((b * heads + h) * n + tok) * M);
#pragma unroll
        for (int q = 0; q < NW / 4; ++q) {
          const uint4 v = cr[q];
          cw[u][4 * q] = v.x; cw[u][4 * q + 1] = v.y; cw[u][4 * q + 2] = v.z; cw[u][4 * q + 3] = v.w;
        }
        pos[u] = positions[b * n + tok];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t tok = t0 + u * TOK + tk;
      if (tok >= n) continue;
      bool ok = pos[u] >= 0;
#pragma unroll
      for (int q = 0; q < NW; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) ok = ok && (int64_t)((cw[u][q] >> (8 * e)) & 0xFFu) < k;
      // the code of sub-space sidx (a runtime byte of the row held in registers)
      auto code_of = [&](int sidx) {
        unsigned w = 0u;
#pragma unroll
        for (int q = 0; q < NW; ++q) w = (sidx >> 2) == q ? cw[u][q] : w;
        return (int64_t)((w >> (8 * (sidx & 3))) & 0xFFu);
      };
      float xl[P], xh[P];
#pragma unroll
      for (int kk = 0; kk < P; kk += 4) {
        const int dl = i0 + kk, dh = kHalf + i0 + kk;
        const int64_t cl = ok ? code_of(dl / SUB) : 0, chh = ok ? code_of(dh / SUB) : 0;
        const f4 a = *reinterpret_cast<const f4*>(cb + cl * SUB + dl % SUB);
        const f4 bb = *reinterpret_cast<const f4*>(cb + chh * SUB + dh % SUB);
        xl[kk] = a.x; xl[kk + 1] = a.y; xl[kk + 2] = a.z; xl[kk + 3] = a.w;
        xh[kk] = bb.x; xh[kk + 1] = bb.y; xh[kk + 2] = bb.z; xh[kk + 3] = bb.w;
      }
      const int64_t ooff = ((b * heads + h) * n + tok) * kD + i0;
      real lo[P], hi[P];
      if (!ok) {
#pragma unroll
        for (int kk = 0; kk < P; ++kk) lo[kk] = hi[kk] = (real)NAN;
      } else {
        real cs[P], sn[P];
        if (in_window(cur, pos[u], window)) {
          const d2* row = table + (cur - (int64_t)pos[u]) * kHalf + i0;
#pragma unroll
          for (int kk = 0; kk < P; ++kk) {
            const d2 v = row[kk];
            cs[kk] = (real)v.x;
            sn[kk] = (real)v.y;
          }
        } else {
#pragma unroll
          for (int kk = 0; kk < P; ++kk) {
            cs[kk] = fc[kk];
            sn[kk] = fs[kk];
          }
        }
        rotate_pairs<real, P>(xl, xh, cs, sn, lo, hi);
      }
      store_pairs<BF16, P>(out, ooff, lo, hi);
    }
  }
}

// Incremental update for far keys left unrotated (Eq. 12): a token's reconstructed row then
// depends on the current position only through its near/far status, so moving from cur_prev
// to cur rewrites only the tokens whose status changed, plus the tokens appended since
// (index >= n_prev).  Work item = (sequence, 256 tokens): each thread tests one token, the
// changed ones are listed in LDS, and the workgroup then writes their rows for every head
// (all (head, token) rows spread over the workgroup at once) with the gather's own arithmetic (near: the rotation at the token's position from
// rope_cs; far: identity), so the rows are bitwise those of a full reconstruct at cur.
template <bool BF16>
__global__ __launch_bounds__(256) void rope_update(
    const uint16_t* __restrict__ codes, const int32_t* __restrict__ positions, int64_t heads,
    int64_t n, const float* __restrict__ cb, int64_t c, int64_t n_prev, int64_t cur_prev,
    int64_t cur, int64_t window, double base, void* __restrict__ out, int64_t chunks) {
  constexpr int P = BF16 ? 8 : 4;
  constexpr int TPT = kHalf / P;
  constexpr int TOK = 256 / TPT;
  using real = double;
  __shared__ int s_tok[256];
  __shared__ int s_pos[256];
  __shared__ unsigned s_n;
  const int t = threadIdx.x, lane = t & 63;
  const int64_t b = blockIdx.x / chunks;
  const int64_t t0 = (blockIdx.x % chunks) * 256;
  if (t == 0) s_n = 0u;
  __syncthreads();
  const int64_t tok = t0 + t;
  bool changed = false;
  int p = -1;
  if (tok < n) {
    p = positions[b * n + tok];
    changed = tok >= n_prev ||
              (p >= 0 && in_window(cur_prev, p, window) != in_window(cur, p, window));
  }
  const unsigned long long m = __ballot(changed);
  unsigned wbase = 0u;
  if (lane == 0 && m) wbase = atomicAdd(&s_n, (unsigned)__popcll(m));
  wbase = __shfl(wbase, 0);
  if (changed) {
    const unsigned slot = wbase + (unsigned)__popcll(m & ((1ull << lane) - 1ull));
    s_tok[slot] = t;
    s_pos[slot] = p;
  }
  __syncthreads();
  const int cnt = (int)s_n;
  if (cnt == 0) return;
  const int g = t % TPT, tk = t / TPT;
  const int i0 = g * P;
  // (head, listed token) pairs, all heads at once, so every row's loads are in flight together
  const int64_t rows_total = heads * (int64_t)cnt;
  for (int64_t e2 = tk; e2 < rows_total; e2 += TOK) {
    const int64_t h = e2 / cnt;
    const int e = (int)(e2 % cnt);
    const float* cbh = cb + h * c * kD;
    const int64_t row = t0 + s_tok[e];
    const int pp = s_pos[e];
    const int code = codes[(b * heads + h) * n + row];
    const int64_t ooff = ((b * heads + h) * n + row) * kD + i0;
    real lo[P], hi[P];
    if ((int64_t)code >= c || pp < 0) {
#pragma unroll
      for (int k = 0; k < P; ++k) lo[k] = hi[k] = (real)NAN;
    } else {
      float xl[P], xh[P];
      load_pairs<P>(cbh + (int64_t)code * kD + i0, xl, xh);
      real cs[P], sn[P];
      if (in_window(cur, pp, window)) {
#pragma unroll
        for (int k = 0; k < P; ++k) {
          const d2 v = rope_cs((double)pp, i0 + k, kD, base);
          cs[k] = (real)v.x;
          sn[k] = (real)v.y;
        }
      } else {
#pragma unroll
        for (int k = 0; k < P; ++k) {
          cs[k] = (real)1.0;
          sn[k] = (real)0.0;
        }
      }
      rotate_pairs<real, P>(xl, xh, cs, sn, lo, hi);
    }
    store_pairs<BF16, P>(out, ooff, lo, hi);
  }
}

// The query-side half of Eq. 11: every row rotated as a token at position b, in fp64, then
// rounded once to the output type.  The 64 (cos, sin) pairs are formed once per workgroup in
// LDS; thread t handles pair t % 64 of rows t / 64, t / 64 + 4, ...  Each thread reads both
// elements of its pair before writing them, so the output may be the input itself.
template <int DIN, int DOUT>
__global__ __launch_bounds__(256) void rope_query(const void* __restrict__ q, int64_t rows,
                                                  double position, double base, void* out) {
  __shared__ d2 s_cs[kHalf];
  const int t = threadIdx.x;
  if (t < kHalf) s_cs[t] = rope_cs(position, t, kD, base);
  __syncthreads();
  const int i = t % kHalf;
  const d2 v = s_cs[i];
  for (int64_t r = (int64_t)blockIdx.x * 4 + t / kHalf; r < rows; r += (int64_t)gridDim.x * 4) {
    const double xl = (double)load_elem(q, DIN, r * kD + i);
    const double xh = (double)load_elem(q, DIN, r * kD + kHalf + i);
    const double lo = fma(xl, v.x, -(xh * v.y));
    const double hi = fma(xh, v.x, xl * v.y);
    if (DOUT == A2ATS_F32) {
      static_cast<float*>(out)[r * kD + i] = (float)lo;
      static_cast<float*>(out)[r * kD + kHalf + i] = (float)hi;
    } else {
      static_cast<uint16_t*>(out)[r * kD + i] = f64_to_bf16(lo);
      static_cast<uint16_t*>(out)[r * kD + kHalf + i] = f64_to_bf16(hi);
    }
  }
}

inline int64_t near_rows(int64_t cur, int64_t window) {
  int64_t w = window > 0 ? window : 0;
  return w < cur + 1 ? w : cur + 1;
}

}  // namespace
}  // namespace a2ats

using namespace a2ats;

namespace a2ats {
namespace {
size_t table_bytes(int64_t cur_pos, int64_t window) {
  return align_up((size_t)(near_rows(cur_pos, window) + 1) * kHalf * sizeof(d2));
}
}  // namespace
}  // namespace a2ats

extern "C" size_t a2ats_reconstruct_workspace(int64_t heads, int64_t c, int64_t d,
                                              int64_t cur_pos, int64_t window, int out_dtype) {
  if (d != kD || cur_pos < 0 || heads < 1 || c < 1 || c > 65536) return 0;
  if (out_dtype != A2ATS_F32 && out_dtype != A2ATS_BF16) return 0;
  const size_t far_rows = align_up((size_t)(heads * c * kD) * (out_dtype == A2ATS_F32 ? 4 : 2));
  return table_bytes(cur_pos, window) + far_rows;
}

extern "C" size_t a2ats_pq_reconstruct_workspace(int64_t d, int64_t cur_pos, int64_t window) {
  if (d != kD || cur_pos < 0) return 0;
  return table_bytes(cur_pos, window);
}

namespace a2ats {
namespace {

// Argument checks shared by a2ats_reconstruct and a2ats_reconstruct_noalloc (A2ATS_OK with
// *empty set when there is nothing to do).
int reconstruct_check(const uint16_t* codes, const int32_t* positions, int64_t batch,
                      int64_t heads, int64_t n, int64_t d, const float* codebook, int64_t c,
                      int64_t cur_pos, int far_mode, double rope_base, const void* out,
                      int out_dtype, bool* empty) {
  *empty = false;
  if (out_dtype != A2ATS_F32 && out_dtype != A2ATS_BF16) return A2ATS_EDTYPE;
  if (d != kD || batch < 1 || heads < 1 || n < 0 || c < 1 || c > 65536) return A2ATS_EINVAL;
  if (cur_pos < 0 || !(rope_base > 0.0) || !std::isfinite(rope_base)) return A2ATS_EINVAL;
  if (far_mode != A2ATS_FAR_FIXED_OFFSET && far_mode != A2ATS_FAR_UNROTATED) return A2ATS_EINVAL;
  if (n == 0) {
    *empty = true;
    return A2ATS_OK;
  }
  if (!codes || !positions || !codebook || !out) return A2ATS_EINVAL;
  return A2ATS_OK;
}

// The table and gather launches of a reconstruct, the table in `table` (rows + 1 rows); with
// farcb (room for [heads][c][d] in the output type) the same launch as the table also
// writes every centroid's far row, which far tokens then copy.
int reconstruct_launch(const uint16_t* codes, const int32_t* positions, int64_t batch,
                       int64_t heads, int64_t n, const float* codebook, int64_t c,
                       int64_t cur_pos, int64_t window, int64_t far_offset, int far_mode,
                       double rope_base, void* out, int out_dtype, d2* table, void* farcb,
                       hipStream_t s) {
  const int64_t rows = near_rows(cur_pos, window);
  const int far_identity = (int)(far_mode == A2ATS_FAR_UNROTATED);
  if (farcb) {
    const int64_t tab_blocks = ((rows + 1) * kHalf + 255) / 256;
    const int64_t rows_far = heads * c;
    const int rpw = out_dtype == A2ATS_F32 ? 16 : 32;  // 256 / (64 / P)
    const int64_t far_blocks = (rows_far + rpw - 1) / rpw;
    if (tab_blocks + far_blocks > 0x7FFFFFFF) return A2ATS_EINVAL;
    const dim3 g((unsigned)(tab_blocks + far_blocks));
    if (out_dtype == A2ATS_F32)
      A2ATS_TRY(launch("rope_table", rope_prep<false>, g, dim3(256), 0, s, rows, cur_pos,
                       cur_pos - far_offset, far_identity, rope_base, table, tab_blocks, codebook,
                       rows_far, farcb));
    else
      A2ATS_TRY(launch("rope_table", rope_prep<true>, g, dim3(256), 0, s, rows, cur_pos,
                       cur_pos - far_offset, far_identity, rope_base, table, tab_blocks, codebook,
                       rows_far, farcb));
  } else {
    A2ATS_TRY(launch("rope_table", rope_table, dim3(grid_for((rows + 1) * kHalf, 256)), dim3(256), 0,
                     s, rows, cur_pos, cur_pos - far_offset, far_identity, rope_base, (int)kD, table));
  }
  const int64_t chunk = out_dtype == A2ATS_F32 ? kChunkF32 : kChunkBf16;
  const int64_t items = batch * heads * ((n + chunk - 1) / chunk);
  // A multiple of 8 * heads workgroups, enough to fill the chip several times over.
  int64_t per = 8 * heads;
  int64_t g = items / kGatherItems;
  if (g < kGridMin) g = kGridMin;
  g = (g + per - 1) / per * per;
  if (g > items) g = items;
  if (g > (int64_t)1 << 30) g = (int64_t)1 << 30;
  if (out_dtype == A2ATS_F32)
    return launch("reconstruct", rope_gather<false>, dim3((unsigned)g), dim3(256), 0, s, codes,
                  positions, heads, n, codebook, c, cur_pos, window, rows, table, farcb, out, items);
  return launch("reconstruct", rope_gather<true>, dim3((unsigned)g), dim3(256), 0, s, codes,
                positions, heads, n, codebook, c, cur_pos, window, rows, table, farcb, out, items);
}

}  // namespace
}  // namespace a2ats

extern "C" int a2ats_reconstruct(const uint16_t* codes, const int32_t* positions, int64_t batch,
                                 int64_t heads, int64_t n, int64_t d, const float* codebook,
                                 int64_t c, int64_t cur_pos, int64_t window, int64_t far_offset,
                                 int far_mode, double rope_base, void* out, int out_dtype,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  bool empty = false;
  A2ATS_TRY(reconstruct_check(codes, positions, batch, heads, n, d, codebook, c, cur_pos,
                              far_mode, rope_base, out, out_dtype, &empty));
  if (empty) return A2ATS_OK;
  const size_t need = a2ats_reconstruct_workspace(heads, c, d, cur_pos, window, out_dtype);
  if (!ws_ok(workspace, workspace_bytes, need)) return A2ATS_EWORKSPACE;
  char* ws = static_cast<char*>(workspace);
  return reconstruct_launch(codes, positions, batch, heads, n, codebook, c, cur_pos, window,
                            far_offset, far_mode, rope_base, out, out_dtype,
                            reinterpret_cast<d2*>(ws), ws + table_bytes(cur_pos, window),
                            static_cast<hipStream_t>(stream));
}

// ------------------------------------------------------------------ allocation-free variant
// The rope table of a2ats_reconstruct_noalloc: (cos, sin) of the 64 pairs, A2ATS_NOALLOC_TABLE_ROWS
// rows, in a fixed device array (one per GPU, held until the process ends).  In host code the
// name `scratch` stands for the host-side shadow of the symbol; the device address of each
// GPU's copy is looked up once per device (with that device current) and kept in
// g_scratch_dev, which is what the kernels receive.
static __device__ __align__(256) double scratch[A2ATS_NOALLOC_TABLE_ROWS * kD];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];

// Device address of the current device's table (looked up on the device's first call).
int scratch_table(d2** table) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return A2ATS_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return A2ATS_EHIP;
    g_scratch_dev[dev] = p;
  }
  *table = static_cast<d2*>(g_scratch_dev[dev]);
  return A2ATS_OK;
}
}  // namespace

extern "C" int a2ats_reconstruct_noalloc(const uint16_t* codes, const int32_t* positions,
                                         int64_t batch, int64_t heads, int64_t n, int64_t d,
                                         const float* codebook, int64_t c, int64_t cur_pos,
                                         int64_t window, int64_t far_offset, int far_mode,
                                         double rope_base, void* out, int out_dtype,
                                         void* stream) {
  bool empty = false;
  A2ATS_TRY(reconstruct_check(codes, positions, batch, heads, n, d, codebook, c, cur_pos,
                              far_mode, rope_base, out, out_dtype, &empty));
  if (empty) return A2ATS_OK;
  if (near_rows(cur_pos, window) + 1 > A2ATS_NOALLOC_TABLE_ROWS) return A2ATS_ESCRATCH;
  d2* table = nullptr;
  A2ATS_TRY(scratch_table(&table));
  return reconstruct_launch(codes, positions, batch, heads, n, codebook, c, cur_pos, window,
                            far_offset, far_mode, rope_base, out, out_dtype, table, nullptr,
                            static_cast<hipStream_t>(stream));
}

extern "C" int a2ats_reconstruct_update(const uint16_t* codes, const int32_t* positions,
                                        int64_t batch, int64_t heads, int64_t n, int64_t d,
                                        const float* codebook, int64_t c, int64_t n_prev,
                                        int64_t cur_prev, int64_t cur_pos, int64_t window,
                                        double rope_base, void* out, int out_dtype, void* stream) {
  if (out_dtype != A2ATS_F32 && out_dtype != A2ATS_BF16) return A2ATS_EDTYPE;
  if (d != kD || batch < 1 || heads < 1 || n < 0 || c < 1 || c > 65536) return A2ATS_EINVAL;
  if (n_prev < 0 || n_prev > n || cur_prev < 0 || cur_pos < 0) return A2ATS_EINVAL;
  if (!(rope_base > 0.0) || !std::isfinite(rope_base)) return A2ATS_EINVAL;
  if (n == 0) return A2ATS_OK;
  if (!codes || !positions || !codebook || !out) return A2ATS_EINVAL;
  const int64_t chunks = (n + 255) / 256;
  if (batch * chunks > 0x7FFFFFFF) return A2ATS_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (out_dtype == A2ATS_F32)
    return launch("reconstruct_update", rope_update<false>, dim3((unsigned)(batch * chunks)),
                  dim3(256), 0, s, codes, positions, heads, n, codebook, c, n_prev, cur_prev,
                  cur_pos, window, rope_base, out, chunks);
  return launch("reconstruct_update", rope_update<true>, dim3((unsigned)(batch * chunks)),
                dim3(256), 0, s, codes, positions, heads, n, codebook, c, n_prev, cur_prev,
                cur_pos, window, rope_base, out, chunks);
}

extern "C" int a2ats_far_query_rope(const void* q, int q_dtype, int64_t rows, int64_t d,
                                    int64_t far_offset, double rope_base, void* out,
                                    int out_dtype, void* stream) {
  if ((q_dtype != A2ATS_F32 && q_dtype != A2ATS_BF16) ||
      (out_dtype != A2ATS_F32 && out_dtype != A2ATS_BF16))
    return A2ATS_EDTYPE;
  if (d != kD || rows < 0) return A2ATS_EINVAL;
  if (!(rope_base > 0.0) || !std::isfinite(rope_base)) return A2ATS_EINVAL;
  if (rows == 0) return A2ATS_OK;
  if (!q || !out) return A2ATS_EINVAL;
  // the output may be the input itself (same dtype), but may not overlap it otherwise
  const size_t in_bytes = (size_t)rows * kD * (q_dtype == A2ATS_F32 ? 4 : 2);
  const size_t out_bytes = (size_t)rows * kD * (out_dtype == A2ATS_F32 ? 4 : 2);
  const char* qa = static_cast<const char*>(q);
  const char* oa = static_cast<const char*>(out);
  const bool overlap = qa < oa + out_bytes && oa < qa + in_bytes;
  if (overlap && (qa != oa || q_dtype != out_dtype)) return A2ATS_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int64_t g = (rows + 3) / 4;
  if (g > 1024) g = 1024;
  const double pos = (double)far_offset;
#define A2ATS_QROPE(I, O)                                                                        \
  launch("far_query_rope", rope_query<I, O>, dim3((unsigned)g), dim3(256), 0, s, q, rows, pos, \
         rope_base, out)
  if (q_dtype == A2ATS_F32)
    return out_dtype == A2ATS_F32 ? A2ATS_QROPE(A2ATS_F32, A2ATS_F32) : A2ATS_QROPE(A2ATS_F32, A2ATS_BF16);
  return out_dtype == A2ATS_F32 ? A2ATS_QROPE(A2ATS_BF16, A2ATS_F32) : A2ATS_QROPE(A2ATS_BF16, A2ATS_BF16);
#undef A2ATS_QROPE
}

extern "C" int a2ats_pq_reconstruct(const uint8_t* codes, const int32_t* positions, int64_t batch,
                                    int64_t heads, int64_t n, int64_t d, int64_t sub_dim,
                                    const float* codebook, int64_t k, int64_t cur_pos,
                                    int64_t window, int64_t far_offset, int far_mode,
                                    double rope_base, void* out, int out_dtype, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  if (out_dtype != A2ATS_F32 && out_dtype != A2ATS_BF16) return A2ATS_EDTYPE;
  if (d != kD || batch < 1 || heads < 1 || n < 0 || k < 1 || k > 256) return A2ATS_EINVAL;
  if (sub_dim != 4 && sub_dim != 8) return A2ATS_EINVAL;
  if (cur_pos < 0 || !(rope_base > 0.0) || !std::isfinite(rope_base)) return A2ATS_EINVAL;
  if (far_mode != A2ATS_FAR_FIXED_OFFSET && far_mode != A2ATS_FAR_UNROTATED) return A2ATS_EINVAL;
  if (n == 0) return A2ATS_OK;
  if (!codes || !positions || !codebook || !out) return A2ATS_EINVAL;
  const int64_t rows = near_rows(cur_pos, window);
  const size_t need = a2ats_pq_reconstruct_workspace(d, cur_pos, window);
  if (!ws_ok(workspace, workspace_bytes, need)) return A2ATS_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  d2* table = static_cast<d2*>(workspace);
  A2ATS_TRY(launch("rope_table", rope_table, dim3(grid_for((rows + 1) * kHalf, 256)), dim3(256), 0,
                   s, rows, cur_pos, cur_pos - far_offset, (int)(far_mode == A2ATS_FAR_UNROTATED),
                   rope_base, (int)kD, table));
  const int64_t chunk = out_dtype == A2ATS_F32 ? kChunkF32 : kChunkBf16;
  const int64_t items = batch * heads * ((n + chunk - 1) / chunk);
  int64_t per = 8 * heads;
  int64_t g = items / (out_dtype == A2ATS_F32 ? kItemsPerWgF32 : kItemsPerWgBf16);
  if (g < kGridMin) g = kGridMin;
  g = (g + per - 1) / per * per;
  if (g > items) g = items;
  if (g > (int64_t)1 << 30) g = (int64_t)1 << 30;
#define A2ATS_PQG(B, S)                                                                          \
  launch("pq_reconstruct", pq_gather<B, S>, dim3((unsigned)g), dim3(256), 0, s, codes, positions, \
         heads, n, codebook, k, cur_pos, window, rows, table, out, items)
  if (out_dtype == A2ATS_F32)
    return sub_dim == 8 ? A2ATS_PQG(false, 8) : A2ATS_PQG(false, 4);
  return sub_dim == 8 ? A2ATS_PQG(true, 8) : A2ATS_PQG(true, 4);
#undef A2ATS_PQG
}
