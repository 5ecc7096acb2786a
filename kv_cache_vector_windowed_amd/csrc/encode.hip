// encode: query-aware (H-weighted) nearest-centroid assignment of keys, uint16 codes.
// "veloxquant_mlx.quantizers.a2ats module", a2ats_h_weighted_assignment (Eq. 14 through the
// Eq. 15-17 Cholesky identity):
//     code(k) = argmin_j (k - c_j) H (k - c_j)^T = argmin_j ||k L - c_j L||^2,   H = L L^T.
// Expanding the square, with v_j = c_j H and b_j = c_j H c_j^T (exact in fp64),
//     ||kL - c_jL||^2 = ||kL||^2 - 2 (k . v_j - b_j / 2),
// so the code maximises the score s_j = k . v_j - b_j / 2: a dense contraction of the keys
// against the transformed codebook plus a row argmax.  Without L, H = I (plain nearest
// centroid, the bulk path).
//
// Exactness.  The contraction runs on fp16 MFMA (bf16 keys are exact in fp16; the codebook
// side is rounded after a power-of-two scale S).  For each key the kernel bounds the
// MFMA error rigorously,
//     |acc_j - S s_j| <= E = |k| rho + |k - k16| nu + gamma (B + |k16| nu) + u B,
// (rho = max_j |S v_j - v16_j|, nu = max_j |v16_j|, B = max_j S b_j / 2, gamma covers the
// fp32 accumulation of 129 terms) and only accepts the MFMA winner when the bound proves it.
// Close calls are settled by exact fp64 scores; what remains is rescanned.
//
// Kernels
//   enc_gram        H = L L^T in fp64 (skipped without L); zeroes per-call counters.
//   enc_prep_rows   v_j = c_j H and b_j in fp64; per-head max |v| and max b.
//   enc_prep_frag   fp16 operand fragments of S v (MFMA A-operand order), the fp32 bias
//                   -S b_j / 2 per accumulator slot, rho and nu; optionally fp16 hi/lo
//                   fragments of L^T for ||kL||^2.
//   enc_coarse      the MFMA pass (see the kernel comment) with certification and fp64
//                   rerank of the two leading candidates.
//   enc_rescan      keys left uncertified: a second MFMA pass that collects every centroid
//                   whose score could reach the best exact score, then fp64 decides.
//   enc_fullscan    keys that overflow fp16 or overflow the candidate list: fp64 scan.
//   enc_znorm64     ||kL||^2 in fp64 for fp32 keys when distances are requested with L.
#include "common.hpp"

namespace a2ats {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kD = A2ATS_HEAD_DIM;
constexpr int kRows = 32;                 // centroids per MFMA tile
constexpr int kSteps = kD / 16;           // k-steps of 16 per tile (v_mfma_f32_32x32x16_f16)
constexpr int kFragPerTile = kSteps * 64; // half8 fragments per tile
constexpr int kTPS = 4;                   // tiles per LDS stage
constexpr int kKeysPerWG = 256;           // 4 waves x 64 keys
constexpr int kCandCap = 32;              // rescan candidates per key
constexpr float kPadBias = -1.0e38f;      // bias of padding rows: finite, never competitive

struct EncHead {
  unsigned maxabs_v;  // float bits, max |v_ja| rounded up
  unsigned maxb;      // float bits, max b_j rounded up
  unsigned rho;       // float bits, max_j ||S v_j - v16_j|| rounded up (scaled units)
  unsigned nu;        // float bits, max_j ||v16_j|| rounded up (scaled units)
  unsigned maxabs_l;  // float bits, max |L_ab| rounded up
  unsigned pad[3];
};

struct Counters {
  unsigned unc;        // entries in the rescan list
  unsigned full;       // entries in the full-scan list
  unsigned stats[8];   // keys, direct, reranked, rescanned, full_scan
};

struct UncEntry {
  int32_t head;
  int32_t row;
  double sbest;        // exact score of the best reranked candidate (a lower bound of the max)
  int32_t jbest;       // its index
  int32_t pad;
};

__device__ __forceinline__ float round_up_f(double x) {
  float f = (float)x;
  if ((double)f < x) f = __uint_as_float(__float_as_uint(f) + (f >= 0.f ? 1u : -1u));
  return f;
}

__device__ __forceinline__ int ilog2_floor(float x) {  // x > 0, normal
  return (int)((__float_as_uint(x) >> 23) & 0xFF) - 127;
}

__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((unsigned)(e + 127) << 23); }

// Accumulator slot r of a lane in half hh holds MFMA output row 8(r/4) + 4hh + (r%4).
__device__ __forceinline__ int slot_row(int r, int hh) { return 8 * (r >> 2) + 4 * hh + (r & 3); }

// ------------------------------------------------------------------ prep
__global__ __launch_bounds__(256) void enc_gram(const float* __restrict__ chol,
                                                double* __restrict__ h64,
                                                EncHead* __restrict__ info,
                                                Counters* __restrict__ cnt) {
  const int head = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;  // element of the 128 x 128 matrix
  if (blockIdx.x == 0 && threadIdx.x < sizeof(EncHead) / 4)
    reinterpret_cast<unsigned*>(&info[head])[threadIdx.x] = 0u;
  if (head == 0 && blockIdx.x == 0 && threadIdx.x < sizeof(Counters) / 4)
    reinterpret_cast<unsigned*>(cnt)[threadIdx.x] = 0u;
  if (!chol) return;
  const float* L = chol + (int64_t)head * kD * kD;
  const int i = e / kD, j = e % kD;
  const int kmax = i < j ? i : j;
  double s = 0.0;
  for (int k = 0; k <= kmax; ++k) s += (double)L[i * kD + k] * (double)L[j * kD + k];
  h64[(int64_t)head * kD * kD + e] = s;
}

// v_j = c_j H, b_j = c_j . v_j (fp64).  32 rows per workgroup; H and the rows in LDS.
__global__ __launch_bounds__(256) void enc_prep_rows(const float* __restrict__ cb, int64_t c,
                                                     const double* __restrict__ h64,
                                                     const float* __restrict__ chol,
                                                     double* __restrict__ v64,
                                                     double* __restrict__ b64,
                                                     EncHead* __restrict__ info) {
  const int plain = chol == nullptr;
  extern __shared__ double sm[];
  double* H = sm;                                  // [128][128] (unused when plain)
  float* cr = reinterpret_cast<float*>(sm + (plain ? 0 : kD * kD));  // [32][128]
  const int head = blockIdx.y;
  const int64_t j0 = (int64_t)blockIdx.x * 32;
  const int t = threadIdx.x;
  const float* cbh = cb + (int64_t)head * c * kD;
  if (!plain)
    for (int e = t; e < kD * kD; e += 256) H[e] = h64[(int64_t)head * kD * kD + e];
  for (int e = t; e < 32 * kD; e += 256) {
    int r = e / kD, a = e % kD;
    cr[e] = (j0 + r < c) ? cbh[(j0 + r) * kD + a] : 0.f;
  }
  __syncthreads();
  const int rg = t / 32;  // rows rg*4 .. rg*4+3
  const int cg = t % 32;  // columns cg + 32m
  double acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[i][m] = 0.0;
  if (plain) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int m = 0; m < 4; ++m) acc[i][m] = (double)cr[(rg * 4 + i) * kD + cg + 32 * m];
  } else {
    for (int b = 0; b < kD; ++b) {
      double cv[4], hv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) cv[i] = (double)cr[(rg * 4 + i) * kD + b];
#pragma unroll
      for (int m = 0; m < 4; ++m) hv[m] = H[b * kD + cg + 32 * m];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[i][m] += cv[i] * hv[m];
    }
  }
  float vmax = 0.f, bmax = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t j = j0 + rg * 4 + i;
    double bp = 0.0;
#pragma unroll
    for (int m = 0; m < 4; ++m) bp += (double)cr[(rg * 4 + i) * kD + cg + 32 * m] * acc[i][m];
    for (int o = 16; o > 0; o >>= 1) bp += __shfl_xor(bp, o);  // 32 lanes of this row group
    if (j < c) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        v64[((int64_t)head * c + j) * kD + cg + 32 * m] = acc[i][m];
        vmax = fmaxf(vmax, round_up_f(fabs(acc[i][m])));
      }
      if (cg == 0) b64[(int64_t)head * c + j] = bp;
      bmax = fmaxf(bmax, round_up_f(bp));
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    vmax = fmaxf(vmax, __shfl_xor(vmax, o));
    bmax = fmaxf(bmax, __shfl_xor(bmax, o));
  }
  if ((t & 63) == 0) {
    atomicMax(&info[head].maxabs_v, __float_as_uint(vmax));
    atomicMax(&info[head].maxb, __float_as_uint(bmax));
  }
  if (!plain && blockIdx.x == 0) {  // max |L| for the z-norm fragments
    const float* L = chol + (int64_t)head * kD * kD;
    float a = 0.f;
    for (int e = t; e < kD * kD; e += 256) a = fmaxf(a, fabsf(L[e]));
    for (int o = 32; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o));
    if ((t & 63) == 0) atomicMax(&info[head].maxabs_l, __float_as_uint(a));
  }
}

__device__ __forceinline__ float head_scale(const EncHead& h) {
  float m = __uint_as_float(h.maxabs_v);
  if (!(m > 0.f)) return 1.f;
  return pow2f(14 - ilog2_floor(m));  // max |S v| in [2^14, 2^15)
}

// One thread per padded row j in [0, T*32): fp16 fragments of S v_j, the bias slot, rho, nu.
// Threads past the rows build the L^T hi/lo fragments when requested.
__global__ __launch_bounds__(256) void enc_prep_frag(const double* __restrict__ v64,
                                                     const double* __restrict__ b64, int64_t c,
                                                     int T, const float* __restrict__ chol,
                                                     int want_l, EncHead* __restrict__ info,
                                                     half8* __restrict__ v16,
                                                     float* __restrict__ bias,
                                                     half8* __restrict__ lfrag) {
  const int head = blockIdx.y;
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rows = (int64_t)T * kRows;
  EncHead hi = info[head];
  float rr = 0.f, nn = 0.f;
  if (j < rows) {
    const float S = head_scale(hi);
    const int64_t tile = j / kRows;
    const int i = (int)(j % kRows);
    half8* vt = v16 + ((int64_t)head * T + tile) * kFragPerTile;
    double rho2 = 0.0, nu2 = 0.0;
    for (int s = 0; s < kSteps; ++s) {
      for (int hh = 0; hh < 2; ++hh) {
        half8 f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int a = 16 * s + 8 * hh + e;
          double sv = (j < c) ? (double)S * v64[((int64_t)head * c + j) * kD + a] : 0.0;
          _Float16 q = (_Float16)sv;  // fp64 -> fp16, round to nearest even
          double dq = (double)q;
          rho2 += (sv - dq) * (sv - dq);
          nu2 += dq * dq;
          f[e] = q;
        }
        vt[s * 64 + i + 32 * hh] = f;
      }
    }
    const int hh = (i >> 2) & 1;
    const int r = (i >> 3) * 4 + (i & 3);
    bias[((int64_t)head * T + tile) * 32 + hh * 16 + r] =
        (j < c) ? (float)(-0.5 * (double)S * b64[(int64_t)head * c + j]) : kPadBias;
    rr = round_up_f(sqrt(rho2));
    nn = round_up_f(sqrt(nu2));
  } else if (want_l && j < rows + kD) {
    // Row a of L^T (output component z_a = sum_b k_b L_ba) as MFMA A-operand fragments:
    // 4 tiles of 32 rows; tiles 0..3 hold the fp16 high parts, 4..7 the residuals.
    const int a = (int)(j - rows);
    const float* L = chol + (int64_t)head * kD * kD;
    float ml = __uint_as_float(hi.maxabs_l);
    const float SL = ml > 0.f ? pow2f(14 - ilog2_floor(ml)) : 1.f;
    const int tile = a / kRows, i = a % kRows;
    half8* lt = lfrag + (int64_t)head * 8 * kFragPerTile;
    for (int s = 0; s < kSteps; ++s) {
      for (int hh = 0; hh < 2; ++hh) {
        half8 fh, fl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int b = 16 * s + 8 * hh + e;
          double x = (double)SL * (double)L[b * kD + a];
          _Float16 qh = (_Float16)x;
          fh[e] = qh;
          fl[e] = (_Float16)(x - (double)qh);
        }
        lt[(int64_t)tile * kFragPerTile + s * 64 + i + 32 * hh] = fh;
        lt[(int64_t)(tile + 4) * kFragPerTile + s * 64 + i + 32 * hh] = fl;
      }
    }
  }
  for (int o = 32; o > 0; o >>= 1) {  // every lane of the wave takes part
    rr = fmaxf(rr, __shfl_xor(rr, o));
    nn = fmaxf(nn, __shfl_xor(nn, o));
  }
  if ((threadIdx.x & 63) == 0) {
    atomicMax(&info[head].rho, __float_as_uint(rr));
    atomicMax(&info[head].nu, __float_as_uint(nn));
  }
}

// ------------------------------------------------------------------ key fragments
struct KeyFrags {
  half8 f[2][kSteps];  // two 32-key blocks (MFMA B operand: key = lane % 32, k = 16s+8hh+e)
  float n2[2];         // ||k||^2 of this lane's 64 elements (fp32, exact values)
  float e2[2];         // ||k - k16||^2 partial
  bool bad[2];         // an element outside the fp16 range
};

template <int DT>
__device__ __forceinline__ void load_key_frags(const void* keys, int64_t head, int64_t n,
                                               const int64_t row[2], int hh, KeyFrags& kf) {
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    kf.n2[blk] = 0.f;
    kf.e2[blk] = 0.f;
    kf.bad[blk] = false;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      float x[8];
      if (row[blk] >= 0) {
        const int64_t off = (head * n + row[blk]) * kD + 16 * s + 8 * hh;
        if (DT == A2ATS_BF16) {
          const uint4 raw = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(keys) + off);
          const unsigned w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[2 * e] = __uint_as_float(w[e] << 16);
            x[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
          }
        } else {
          const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(keys) + off);
          const float4 a = p[0], b = p[1];
          x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
          x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool ok = fabsf(x[e]) < 65504.0f;
        const _Float16 q = ok ? (_Float16)x[e] : (_Float16)0.0f;
        kf.bad[blk] |= !ok;
        const float d = x[e] - (float)q;  // exact: q is x rounded to 11 significant bits
        kf.n2[blk] += x[e] * x[e];
        kf.e2[blk] += d * d;
        kf.f[blk][s][e] = q;
      }
    }
  }
}

// Exact score s_j = k . v_j - b_j / 2 in fp64, key row read from global.
template <int DT>
__device__ double exact_score(const void* keys, int64_t head, int64_t n, int64_t row,
                              const double* v64, const double* b64, int64_t c, int64_t j) {
  const double* v = v64 + (head * c + j) * kD;
  const int64_t off = (head * n + row) * kD;
  double s = 0.0;
  for (int a = 0; a < kD; a += 2) {
    const double2 vv = *reinterpret_cast<const double2*>(v + a);
    s += (double)load_elem(keys, DT, off + a) * vv.x;
    s += (double)load_elem(keys, DT, off + a + 1) * vv.y;
  }
  return s - 0.5 * b64[head * c + j];
}

// (value, index) order: larger value first, equal values keep the lower index first.
__device__ __forceinline__ bool before(float v1, int j1, float v2, int j2) {
  return v1 > v2 || (v1 == v2 && j1 < j2);
}

struct Top3 {
  float v[3];
  int j[3];
  __device__ __forceinline__ void init() {
    v[0] = v[1] = v[2] = -INFINITY;
    j[0] = j[1] = j[2] = 0x7FFFFFFF;
  }
  __device__ __forceinline__ void push(float x, int jx) {
    if (before(x, jx, v[2], j[2])) {
      if (before(x, jx, v[1], j[1])) {
        v[2] = v[1]; j[2] = j[1];
        if (before(x, jx, v[0], j[0])) {
          v[1] = v[0]; j[1] = j[0];
          v[0] = x; j[0] = jx;
        } else {
          v[1] = x; j[1] = jx;
        }
      } else {
        v[2] = x; j[2] = jx;
      }
    }
  }
};

// Error bound E (scaled units) of a key's MFMA scores, evaluated with upward margins.
__device__ __forceinline__ double score_bound(float n2, float e2, const EncHead& h, float S) {
  const double kn = sqrt((double)n2) * (1.0 + 0x1p-18);
  const double ke = sqrt((double)e2) * (1.0 + 0x1p-18);
  const double rho = (double)__uint_as_float(h.rho);
  const double nu = (double)__uint_as_float(h.nu);
  const double B = 0.5 * (double)S * (double)__uint_as_float(h.maxb);
  const double gamma = 130.0 * 0x1p-23;
  return (kn * rho + ke * nu + gamma * (B + (kn + ke) * nu) + 0x1p-23 * B) * (1.0 + 0x1p-16) + 1e-30;
}

// Largest possible change of a value by overwriting its low `tbits` bits.
__device__ __forceinline__ double pack_slack(float p, int tbits) {
  return fabs((double)p) * ldexp(1.0, tbits - 22) + ldexp(1.0, tbits - 140);
}

// ------------------------------------------------------------------ the MFMA pass
// Workgroup: 256 keys of one head (4 waves x two 32-key column blocks).  Lane l serves key
// column l % 32 of both blocks and, within every 32-centroid tile, the 16 rows
// 8(r/4) + 4(l/32) + (r%4).  The codebook streams through LDS in stages of 4 tiles,
// double-buffered; each tile costs 8 MFMAs per block with the bias preloaded as the
// accumulator.  Every accumulator slot r keeps its own running top-2 over the tiles (the
// tile index packed into the low bits): 3 VALU ops per score (pack, med3, max).  At the end
// each key has 32 (max, second) pairs; the top three of those and the largest second give
// the certificate:
//   direct    t1 - t2 > 2E (+ packing slack)                  -> code = j(t1)
//   reranked  exact fp64 scores of j(t1), j(t2) beat max(t3, every list's second) + E
//   otherwise the key goes to the rescan list with its best exact score.
// Workgroups are mapped so that each XCD serves a contiguous range of (head, block) pairs.
template <int DT, bool ZNORM>
__global__ __launch_bounds__(256, 2) void enc_coarse(
    const void* __restrict__ keys, int64_t n, const int32_t* __restrict__ idx, int64_t n_sel,
    int64_t heads, int nkb, int T, int tbits, const half8* __restrict__ v16,
    const float* __restrict__ bias, const double* __restrict__ v64,
    const double* __restrict__ b64, int64_t c, const half8* __restrict__ lfrag,
    const EncHead* __restrict__ info, float* __restrict__ znorm,
    uint16_t* __restrict__ codes, float* __restrict__ dist, UncEntry* __restrict__ unc,
    UncEntry* __restrict__ full, Counters* __restrict__ cnt) {
  __shared__ half8 sv[2][kTPS][kFragPerTile];
  __shared__ __attribute__((aligned(16))) float sb[2][kTPS][32];
  const int64_t G = gridDim.x;
  const int64_t per_xcd = G / 8;
  const int64_t w = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (w >= heads * nkb) return;
  const int64_t head = w / nkb;
  const int64_t kb = w % nkb;
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63, col = lane & 31, hh = lane >> 5;
  const EncHead hinfo = info[head];
  const float S = head_scale(hinfo);

  int64_t row[2];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const int64_t sel = kb * kKeysPerWG + wave * 64 + blk * 32 + col;
    int64_t r = sel < n_sel ? (idx ? (int64_t)idx[head * n_sel + sel] : sel) : -1;
    row[blk] = (r >= 0 && r < n) ? r : -1;  // out-of-range index entries are skipped
  }
  KeyFrags kf;
  load_key_frags<DT>(keys, head, n, row, hh, kf);
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    kf.n2[blk] += __shfl_xor(kf.n2[blk], 32);
    kf.e2[blk] += __shfl_xor(kf.e2[blk], 32);
    kf.bad[blk] = kf.bad[blk] || __shfl_xor((int)kf.bad[blk], 32);
  }

  // ||k L||^2 from fp16 hi/lo fragments of L^T (bf16 keys are exact in fp16).
  float zn[2] = {0.f, 0.f};
  if (ZNORM) {
    const half8* lt = lfrag + head * 8 * kFragPerTile;
    float ml = __uint_as_float(hinfo.maxabs_l);
    const float SL = ml > 0.f ? pow2f(14 - ilog2_floor(ml)) : 1.f;
    for (int tz = 0; tz < 4; ++tz) {
      f16v z0 = {}, z1 = {};
#pragma unroll
      for (int part = 0; part < 2; ++part) {
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
          const half8 a = lt[(int64_t)(tz + 4 * part) * kFragPerTile + s * 64 + lane];
          z0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, kf.f[0][s], z0, 0, 0, 0);
          z1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, kf.f[1][s], z1, 0, 0, 0);
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        zn[0] += z0[r] * z0[r];
        zn[1] += z1[r] * z1[r];
      }
    }
    const float inv = 1.f / (SL * SL);
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) zn[blk] = (zn[blk] + __shfl_xor(zn[blk], 32)) * inv;
  }

  float m1[2][16], m2[2][16];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int r = 0; r < 16; ++r) m1[blk][r] = m2[blk][r] = -INFINITY;
  const unsigned tmask = (1u << tbits) - 1u;

  const half8* vh = v16 + head * (int64_t)T * kFragPerTile;
  const float* bh = bias + head * (int64_t)T * 32;
  const int nst = (T + kTPS - 1) / kTPS;
  // stage loader: 256 threads x 8 fragments = 4 tiles; 32 threads x 4 bias floats
  half8 pf[8];
  f4 pb;
  auto fetch = [&](int st) {
    const int t0 = st * kTPS;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int e = q * 256 + t;               // fragment within the stage
      const int tt = e / kFragPerTile;
      pf[q] = (t0 + tt < T) ? vh[(int64_t)t0 * kFragPerTile + e] : half8{};
    }
    if (t < 32) {
      const int tt = t / 8;
      pb = (t0 + tt < T) ? *reinterpret_cast<const f4*>(bh + (int64_t)t0 * 32 + t * 4) : f4{};
    }
  };
  auto commit = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int e = q * 256 + t;
      sv[buf][e / kFragPerTile][e % kFragPerTile] = pf[q];
    }
    if (t < 32) *reinterpret_cast<f4*>(&sb[buf][t / 8][(t % 8) * 4]) = pb;
  };
  fetch(0);
  commit(0);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    if (st + 1 < nst) fetch(st + 1);
    const int tiles = (T - st * kTPS) < kTPS ? (T - st * kTPS) : kTPS;
    for (int tt = 0; tt < tiles; ++tt) {
      const unsigned tile = (unsigned)(st * kTPS + tt);
      f16v acc0, acc1;
      const f4* bl = reinterpret_cast<const f4*>(&sb[buf][tt][hh * 16]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f4 b4 = bl[q];
        acc0[4 * q + 0] = b4.x; acc0[4 * q + 1] = b4.y; acc0[4 * q + 2] = b4.z; acc0[4 * q + 3] = b4.w;
      }
      acc1 = acc0;
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        const half8 a = sv[buf][tt][s * 64 + lane];
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, kf.f[0][s], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, kf.f[1][s], acc1, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p0 = __uint_as_float((__float_as_uint(acc0[r]) & ~tmask) | tile);
        const float p1 = __uint_as_float((__float_as_uint(acc1[r]) & ~tmask) | tile);
        m2[0][r] = __builtin_amdgcn_fmed3f(m1[0][r], m2[0][r], p0);
        m1[0][r] = fmaxf(m1[0][r], p0);
        m2[1][r] = __builtin_amdgcn_fmed3f(m1[1][r], m2[1][r], p1);
        m1[1][r] = fmaxf(m1[1][r], p1);
      }
    }
    if (st + 1 < nst) {
      commit(buf ^ 1);
    }
    __syncthreads();
  }

  // ---- per-key certificate.  Both lanes of a key merge the same 32 lists; lane half hh
  // finalises block hh.
  Top3 top[2];
  float useg[2];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    top[blk].init();
    useg[blk] = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rowi = slot_row(r, hh);
      const float a = m1[blk][r], b = m2[blk][r];
      if (a > -INFINITY) top[blk].push(a, (int)((__float_as_uint(a) & tmask) * kRows + rowi));
      if (b > -INFINITY) top[blk].push(b, (int)((__float_as_uint(b) & tmask) * kRows + rowi));
      useg[blk] = fmaxf(useg[blk], b);
    }
  }
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    float pv[3];
    int pj[3];
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      pv[q] = __shfl_xor(top[blk].v[q], 32);
      pj[q] = __shfl_xor(top[blk].j[q], 32);
    }
#pragma unroll
    for (int q = 0; q < 3; ++q)
      if (pv[q] > -INFINITY) top[blk].push(pv[q], pj[q]);
    useg[blk] = fmaxf(useg[blk], __shfl_xor(useg[blk], 32));
  }
  const int blk = hh;
  const int64_t myrow = row[blk];
  const Top3 tp = top[blk];
  int outcome = 0;  // 1 direct, 2 reranked, 3 rescan list, 4 full-scan list
  if (myrow >= 0) {
    const double E = score_bound(kf.n2[blk], kf.e2[blk], hinfo, S);
    const double s1 = pack_slack(tp.v[0], tbits), s2 = pack_slack(tp.v[1], tbits);
    int code = tp.j[0];
    double sbest = 0.0;
    bool have_exact = false;
    if (kf.bad[blk]) {
      outcome = 4;
    } else if ((double)tp.v[0] - s1 - E > (double)tp.v[1] + s2 + E) {
      outcome = 1;
    } else {
      // exact scores of the two leading candidates
      double ex[2];
      int ej[2];
      int ne = 0;
      for (int q = 0; q < 2; ++q) {
        if (tp.j[q] < c && tp.v[q] > -INFINITY) {
          ex[ne] = exact_score<DT>(keys, head, n, myrow, v64, b64, c, tp.j[q]);
          ej[ne] = tp.j[q];
          ++ne;
        }
      }
      int bi = 0;
      if (ne == 2 && (ex[1] > ex[0] || (ex[1] == ex[0] && ej[1] < ej[0]))) bi = 1;
      sbest = ex[bi];
      code = ej[bi];
      have_exact = true;
      const double U = fmax((double)tp.v[2], (double)useg[blk]);
      const double su = pack_slack((float)U, tbits);
      const double nuraw = (double)__uint_as_float(hinfo.nu) / (double)S;
      const double eps = ldexp(1.0, -40) * (sqrt((double)kf.n2[blk]) * nuraw * 2.0 +
                                           (double)__uint_as_float(hinfo.maxb));
      outcome = ((sbest - eps) * (double)S > U + su + E) ? 2 : 3;
    }
    if (ZNORM && dist) znorm[head * n + myrow] = zn[blk];
    if (outcome <= 2) {
      codes[head * n + myrow] = (uint16_t)code;
      if (dist) {
        if (!have_exact) sbest = exact_score<DT>(keys, head, n, myrow, v64, b64, c, code);
        double z2;
        if (ZNORM) {
          z2 = (double)zn[blk];
        } else if (znorm) {
          z2 = (double)znorm[head * n + myrow];  // fp64 ||kL||^2 computed beforehand
        } else {
          z2 = 0.0;  // plain: ||k||^2 exactly
          const int64_t off = (head * n + myrow) * kD;
          for (int a = 0; a < kD; ++a) {
            const double x = (double)load_elem(keys, DT, off + a);
            z2 += x * x;
          }
        }
        dist[head * n + myrow] = (float)fmax(z2 - 2.0 * sbest, 0.0);
      }
    } else {
      UncEntry ue;
      ue.head = (int32_t)head;
      ue.row = (int32_t)myrow;
      ue.sbest = have_exact ? sbest : -INFINITY;
      ue.jbest = have_exact ? code : -1;
      ue.pad = 0;
      if (outcome == 3) unc[atomicAdd(&cnt->unc, 1u)] = ue;
      else full[atomicAdd(&cnt->full, 1u)] = ue;
    }
  }
  // statistics (per wave)
  const unsigned long long valid = __ballot(myrow >= 0);
#pragma unroll
  for (int o = 1; o <= 4; ++o) {
    const unsigned long long m = __ballot(outcome == o);
    if (lane == 0 && m) atomicAdd(&cnt->stats[o], (unsigned)__popcll(m));
  }
  if (lane == 0 && valid) atomicAdd(&cnt->stats[0], (unsigned)__popcll(valid));
}

// ------------------------------------------------------------------ rescan of uncertified keys
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Squared norm used for distances of keys decided outside the MFMA pass.
template <int DT>
__device__ double key_z2(const void* keys, int64_t head, int64_t n, int64_t row,
                         const float* znorm) {
  if (znorm) return (double)znorm[head * n + row];
  double z2 = 0.0;
  const int64_t off = (head * n + row) * kD;
  for (int a = 0; a < kD; ++a) {
    const double x = (double)load_elem(keys, DT, off + a);
    z2 += x * x;
  }
  return z2;
}

// Each wave takes 32 listed keys of one head at a time (MFMA column block 0; lanes 32-63
// hold the other half of the k dimension).  Every centroid whose MFMA score reaches
// S * sbest - E could be the maximiser (sbest is an exact score, so the maximum is at least
// that); those are collected in the wave's LDS slice (kCandCap per key) and decided in
// fp64.  A key with more candidates is forwarded to the full scan.  Waves synchronise only
// with themselves: the loop trip count differs between waves.
template <int DT>
__global__ __launch_bounds__(256) void enc_rescan(
    const void* __restrict__ keys, int64_t n, int T, int64_t c, const half8* __restrict__ v16,
    const float* __restrict__ bias, const double* __restrict__ v64,
    const double* __restrict__ b64, const EncHead* __restrict__ info,
    const float* __restrict__ znorm, uint16_t* __restrict__ codes, float* __restrict__ dist,
    const UncEntry* __restrict__ unc, UncEntry* __restrict__ full, Counters* __restrict__ cnt) {
  __shared__ int cand[4][32][kCandCap];
  __shared__ int ncand[4][32];
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63, col = lane & 31, hh = lane >> 5;
  const unsigned total = __hip_atomic_load(&cnt->unc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int64_t groups = ((int64_t)total + 31) / 32;
  for (int64_t g = (int64_t)blockIdx.x * 4 + wave; g < groups; g += (int64_t)gridDim.x * 4) {
    const int64_t e = g * 32 + col;
    const bool live = e < (int64_t)total;
    UncEntry ue;
    ue.head = -1;
    ue.row = -1;
    ue.sbest = -INFINITY;
    ue.jbest = -1;
    ue.pad = 0;
    if (live) ue = unc[e];
    int pending = live ? ue.head : 0x7FFFFFFF;
    for (;;) {
      int hmin = pending;  // smallest head still pending in this wave
      for (int o = 32; o > 0; o >>= 1) hmin = min(hmin, __shfl_xor(hmin, o));
      if (hmin == 0x7FFFFFFF) break;
      const bool mine = live && ue.head == hmin;
      if (lane < 32) ncand[wave][col] = 0;
      wave_sync();
      const EncHead hinfo = info[hmin];
      const float S = head_scale(hinfo);
      const int64_t row[2] = {mine ? (int64_t)ue.row : -1, -1};
      KeyFrags kf;
      load_key_frags<DT>(keys, hmin, n, row, hh, kf);
      kf.n2[0] += __shfl_xor(kf.n2[0], 32);
      kf.e2[0] += __shfl_xor(kf.e2[0], 32);
      const double E = score_bound(kf.n2[0], kf.e2[0], hinfo, S);
      const double th = ue.sbest * (double)S - E;
      const float thr = mine ? (float)(th - fabs(th) * 0x1p-20 - 1e-30) : INFINITY;
      const half8* vh = v16 + (int64_t)hmin * T * kFragPerTile;
      const float* bh = bias + (int64_t)hmin * T * 32;
      for (int tile = 0; tile < T; ++tile) {
        f16v acc;
        const f4* bl = reinterpret_cast<const f4*>(bh + (int64_t)tile * 32 + hh * 16);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f4 b4 = bl[q];
          acc[4 * q + 0] = b4.x; acc[4 * q + 1] = b4.y; acc[4 * q + 2] = b4.z; acc[4 * q + 3] = b4.w;
        }
#pragma unroll
        for (int s2 = 0; s2 < kSteps; ++s2) {
          const half8 a = vh[(int64_t)tile * kFragPerTile + s2 * 64 + lane];
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, kf.f[0][s2], acc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (acc[r] >= thr) {
            const int j = tile * kRows + slot_row(r, hh);
            if (j < c) {
              const int pos = atomicAdd(&ncand[wave][col], 1);
              if (pos < kCandCap) cand[wave][col][pos] = j;
            }
          }
        }
      }
      wave_sync();
      if (mine && hh == 0) {
        const int nc = ncand[wave][col];
        if (nc > kCandCap) {
          full[atomicAdd(&cnt->full, 1u)] = ue;
        } else {
          double best = ue.sbest;
          int bj = ue.jbest >= 0 ? ue.jbest : 0x7FFFFFFF;
          for (int q = 0; q < nc; ++q) {
            const int j = cand[wave][col][q];
            const double sj = exact_score<DT>(keys, hmin, n, ue.row, v64, b64, c, j);
            if (sj > best || (sj == best && j < bj)) {
              best = sj;
              bj = j;
            }
          }
          codes[(int64_t)hmin * n + ue.row] = (uint16_t)bj;
          if (dist)
            dist[(int64_t)hmin * n + ue.row] =
                (float)fmax(key_z2<DT>(keys, hmin, n, ue.row, znorm) - 2.0 * best, 0.0);
          atomicAdd(&cnt->stats[5], 1u);
        }
      }
      wave_sync();
      if (mine) pending = 0x7FFFFFFF;
    }
  }
}

// fp64 scan of the whole codebook, one wave per listed key.  Runs after the rescan, which
// may append to the list.
template <int DT>
__global__ __launch_bounds__(256) void enc_fullscan(
    const void* __restrict__ keys, int64_t n, int64_t c, const double* __restrict__ v64,
    const double* __restrict__ b64, const float* __restrict__ znorm, uint16_t* __restrict__ codes,
    float* __restrict__ dist, const UncEntry* __restrict__ full, Counters* __restrict__ cnt) {
  __shared__ double kx[4][kD];
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const unsigned total = __hip_atomic_load(&cnt->full, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int64_t e = (int64_t)blockIdx.x * 4 + wave; e < (int64_t)total; e += (int64_t)gridDim.x * 4) {
    const UncEntry ue = full[e];
    const int64_t off = ((int64_t)ue.head * n + ue.row) * kD;
    wave_sync();
    kx[wave][lane] = (double)load_elem(keys, DT, off + lane);
    kx[wave][lane + 64] = (double)load_elem(keys, DT, off + lane + 64);
    wave_sync();
    double best = -INFINITY;
    int bj = 0x7FFFFFFF;
    for (int64_t j = lane; j < c; j += 64) {
      const double* v = v64 + ((int64_t)ue.head * c + j) * kD;
      double sj = 0.0;
      for (int a = 0; a < kD; ++a) sj += kx[wave][a] * v[a];
      sj -= 0.5 * b64[(int64_t)ue.head * c + j];
      if (sj > best || (sj == best && j < bj)) {
        best = sj;
        bj = (int)j;
      }
    }
    for (int o = 32; o > 0; o >>= 1) {
      const double ob = __shfl_xor(best, o);
      const int oj = __shfl_xor(bj, o);
      if (ob > best || (ob == best && oj < bj)) {
        best = ob;
        bj = oj;
      }
    }
    if (lane == 0) {
      codes[(int64_t)ue.head * n + ue.row] = (uint16_t)bj;
      if (dist)
        dist[(int64_t)ue.head * n + ue.row] =
            (float)fmax(key_z2<DT>(keys, ue.head, n, ue.row, znorm) - 2.0 * best, 0.0);
      atomicAdd(&cnt->stats[6], 1u);
    }
  }
}

// ||k L||^2 in fp64, one wave per selected key (fp32 keys with distances and L).
__global__ __launch_bounds__(256) void enc_znorm64(const float* __restrict__ keys, int64_t n,
                                                   const int32_t* __restrict__ idx,
                                                   int64_t n_sel, int64_t heads,
                                                   const float* __restrict__ chol,
                                                   float* __restrict__ znorm) {
  __shared__ double kx[4][kD];
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int64_t total = heads * n_sel;
  for (int64_t e = (int64_t)blockIdx.x * 4 + wave; e < total; e += (int64_t)gridDim.x * 4) {
    const int64_t head = e / n_sel, sel = e % n_sel;
    const int64_t row = idx ? (int64_t)idx[head * n_sel + sel] : sel;
    if (row < 0 || row >= n) continue;  // uniform per wave: one key per wave
    const float* k = keys + (head * n + row) * kD;
    wave_sync();
    kx[wave][lane] = (double)k[lane];
    kx[wave][lane + 64] = (double)k[lane + 64];
    wave_sync();
    const float* L = chol + head * kD * kD;
    double part = 0.0;
    for (int a = lane; a < kD; a += 64) {
      double z = 0.0;
      for (int b = a; b < kD; ++b) z += kx[wave][b] * (double)L[b * kD + a];  // L lower
      part += z * z;
    }
    for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o);
    if (lane == 0) znorm[head * n + row] = (float)part;
  }
}

__global__ void enc_stats_out(const Counters* __restrict__ cnt, a2ats_encode_stats* out) {
  if (threadIdx.x == 0) {
    out->keys = cnt->stats[0];
    out->direct = cnt->stats[1];
    out->reranked = cnt->stats[2];
    out->rescanned = cnt->stats[5];
    out->full_scan = cnt->stats[6];
    out->reserved[0] = cnt->stats[3];
    out->reserved[1] = cnt->stats[4];
    out->reserved[2] = 0;
  }
}

struct EncLayout {
  double* h64;
  double* v64;
  double* b64;
  half8* v16;
  float* bias;
  half8* lfrag;
  EncHead* info;
  Counters* cnt;
  UncEntry* unc;
  UncEntry* full;
  float* znorm;
  size_t bytes;
};

EncLayout carve(void* ws, int64_t heads, int64_t n, int64_t c) {
  const int64_t T = (c + kRows - 1) / kRows;
  Carver cv(ws);
  EncLayout L;
  L.h64 = cv.take<double>((size_t)heads * kD * kD);
  L.v64 = cv.take<double>((size_t)heads * c * kD);
  L.b64 = cv.take<double>((size_t)heads * c);
  L.v16 = cv.take<half8>((size_t)heads * T * kFragPerTile);
  L.bias = cv.take<float>((size_t)heads * T * 32);
  L.lfrag = cv.take<half8>((size_t)heads * 8 * kFragPerTile);
  L.info = cv.take<EncHead>((size_t)heads);
  L.cnt = cv.take<Counters>(1);
  L.unc = cv.take<UncEntry>((size_t)heads * n);
  L.full = cv.take<UncEntry>((size_t)heads * n);
  L.znorm = cv.take<float>((size_t)heads * n);
  L.bytes = cv.used;
  return L;
}

template <int DT>
int encode_typed(const void* keys, int64_t heads, int64_t n, const int32_t* idx, int64_t n_sel,
                 const float* codebook, int64_t c, const float* chol, uint16_t* codes,
                 float* dist, a2ats_encode_stats* stats, const EncLayout& L, hipStream_t s) {
  const int T = (int)((c + kRows - 1) / kRows);
  int tbits = 0;
  while ((1 << tbits) < T) ++tbits;
  const int plain = chol == nullptr;
  A2ATS_TRY(launch("encode_gram", enc_gram, dim3(kD * kD / 256, (unsigned)heads), dim3(256), 0, s,
                   chol, L.h64, L.info, L.cnt));
  const size_t sm_rows = (plain ? 0 : kD * kD * sizeof(double)) + 32 * kD * sizeof(float);
  A2ATS_TRY(set_dynamic_lds(enc_prep_rows, sm_rows));
  A2ATS_TRY(launch("encode_prep_rows", enc_prep_rows, dim3((unsigned)((c + 31) / 32), (unsigned)heads),
                   dim3(256), sm_rows, s, codebook, c, L.h64, chol, L.v64, L.b64, L.info));
  const bool znorm_mfma = dist && !plain && DT == A2ATS_BF16;
  const int64_t frag_threads = (int64_t)T * kRows + (znorm_mfma ? kD : 0);
  A2ATS_TRY(launch("encode_prep_frag", enc_prep_frag, dim3(grid_for(frag_threads, 256), (unsigned)heads),
                   dim3(256), 0, s, L.v64, L.b64, c, T, chol, (int)znorm_mfma, L.info, L.v16,
                   L.bias, L.lfrag));
  // ||kL||^2 for distances with L: MFMA prologue of the coarse pass for bf16 keys (it also
  // stores the value for keys decided later), an fp64 pass for fp32 keys.
  float* znorm = nullptr;
  if (dist && !plain) {
    znorm = L.znorm;
    if (DT == A2ATS_F32)
      A2ATS_TRY(launch("encode_znorm64", enc_znorm64, dim3(grid_for(heads * n_sel, 4, 65536)),
                       dim3(256), 0, s, static_cast<const float*>(keys), n, idx, n_sel, heads, chol,
                       L.znorm));
  }
  const int nkb = (int)((n_sel + kKeysPerWG - 1) / kKeysPerWG);
  const int64_t work = heads * nkb;
  const int64_t G = (work + 7) / 8 * 8;
  if (znorm_mfma)
    A2ATS_TRY(launch("encode_coarse", enc_coarse<DT, true>, dim3((unsigned)G), dim3(256), 0, s, keys, n,
                     idx, n_sel, heads, nkb, T, tbits, L.v16, L.bias, L.v64, L.b64, c, L.lfrag, L.info,
                     znorm, codes, dist, L.unc, L.full, L.cnt));
  else
    A2ATS_TRY(launch("encode_coarse", enc_coarse<DT, false>, dim3((unsigned)G), dim3(256), 0, s, keys, n,
                     idx, n_sel, heads, nkb, T, tbits, L.v16, L.bias, L.v64, L.b64, c, L.lfrag, L.info,
                     znorm, codes, dist, L.unc, L.full, L.cnt));
  A2ATS_TRY(launch("encode_rescan", enc_rescan<DT>, dim3(256), dim3(256), 0, s, keys, n, T, c, L.v16,
                   L.bias, L.v64, L.b64, L.info, znorm, codes, dist, L.unc, L.full, L.cnt));
  A2ATS_TRY(launch("encode_fullscan", enc_fullscan<DT>, dim3(256), dim3(256), 0, s, keys, n, c, L.v64,
                   L.b64, znorm, codes, dist, L.full, L.cnt));
  if (stats)
    A2ATS_TRY(launch("encode_stats", enc_stats_out, dim3(1), dim3(64), 0, s, L.cnt, stats));
  return A2ATS_OK;
}

}  // namespace
}  // namespace a2ats

using namespace a2ats;

extern "C" size_t a2ats_encode_workspace(int64_t heads, int64_t n, int64_t d, int64_t c) {
  if (heads < 1 || n < 0 || d != kD || c < 1 || c > 65536) return 0;
  return carve(nullptr, heads, n, c).bytes;
}

extern "C" int a2ats_encode(const void* keys, int keys_dtype, int64_t heads, int64_t n, int64_t d,
                            const int32_t* idx, int64_t n_idx, const float* codebook, int64_t c,
                            const float* chol, uint16_t* codes, float* dist,
                            a2ats_encode_stats* stats, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (keys_dtype != A2ATS_F32 && keys_dtype != A2ATS_BF16) return A2ATS_EDTYPE;
  if (d != kD || heads < 1 || n < 0 || c < 1 || c > 65536) return A2ATS_EINVAL;
  if (n > 0x7FFFFFFF || heads > 65535) return A2ATS_EINVAL;
  const int64_t n_sel = idx ? n_idx : n;
  if (n_sel < 0 || n_sel > n) return A2ATS_EINVAL;
  if (n_sel == 0) return A2ATS_OK;
  if (!keys || !codebook || !codes) return A2ATS_EINVAL;
  if ((reinterpret_cast<uintptr_t>(keys) & 15) != 0) return A2ATS_EINVAL;
  const size_t need = a2ats_encode_workspace(heads, n, d, c);
  if (!ws_ok(workspace, workspace_bytes, need)) return A2ATS_EWORKSPACE;
  EncLayout L = carve(workspace, heads, n, c);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (keys_dtype == A2ATS_BF16)
    return encode_typed<A2ATS_BF16>(keys, heads, n, idx, n_sel, codebook, c, chol, codes, dist,
                                    stats, L, s);
  return encode_typed<A2ATS_F32>(keys, heads, n, idx, n_sel, codebook, c, chol, codes, dist, stats,
                                 L, s);
}
