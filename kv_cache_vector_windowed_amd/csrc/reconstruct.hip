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
//                keys stay unrotated).
//   rope_gather  HBM-write-bound stream: each thread owns a fixed group of P pairs of the
//                head dimension (P = 4 for fp32 output, 8 for bf16, so every store is 16 B),
//                keeps the far row's cos/sin for its pairs in registers, gathers the
//                centroid from L2, rotates in fp64, rounds once, and writes with
//                non-temporal stores.  Work items are (batch, head, 64-token chunk); item k
//                has head k % heads and the grid is a multiple of 8 * heads, so a workgroup
//                always serves one head and, with 8 heads, each XCD (workgroups are dealt
//                round-robin over the 8 XCDs) keeps a single head's codebook in its L2.
#include "common.hpp"

namespace a2ats {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));
typedef double d2 __attribute__((ext_vector_type(2)));

constexpr int kD = A2ATS_HEAD_DIM;
constexpr int kHalf = kD / 2;
constexpr int kChunk = 64;  // tokens per work item

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
    const double p = (r == rows_near) ? (double)far_pos : (double)(cur - r);
    const double theta = pow(base, -2.0 * (double)i / (double)d);
    const double phi = p * theta;
    v.x = cos(phi);
    v.y = sin(phi);
  }
  table[e] = v;
}

template <int P>
struct OutT;
template <>
struct OutT<4> {  // fp32 output: 4 pairs -> two 16-byte stores
  static __device__ __forceinline__ void store(void* out, int64_t off, const double* lo,
                                               const double* hi) {
    f4 a, b;
    a.x = (float)lo[0]; a.y = (float)lo[1]; a.z = (float)lo[2]; a.w = (float)lo[3];
    b.x = (float)hi[0]; b.y = (float)hi[1]; b.z = (float)hi[2]; b.w = (float)hi[3];
    float* o = static_cast<float*>(out) + off;
    __builtin_nontemporal_store(a, reinterpret_cast<f4*>(o));
    __builtin_nontemporal_store(b, reinterpret_cast<f4*>(o + kHalf));
  }
};
template <>
struct OutT<8> {  // bf16 output: 8 pairs -> two 16-byte stores
  static __device__ __forceinline__ void store(void* out, int64_t off, const double* lo,
                                               const double* hi) {
    u4 a, b;
    unsigned la[4], lb[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      la[k] = (unsigned)f64_to_bf16(lo[2 * k]) | ((unsigned)f64_to_bf16(lo[2 * k + 1]) << 16);
      lb[k] = (unsigned)f64_to_bf16(hi[2 * k]) | ((unsigned)f64_to_bf16(hi[2 * k + 1]) << 16);
    }
    a.x = la[0]; a.y = la[1]; a.z = la[2]; a.w = la[3];
    b.x = lb[0]; b.y = lb[1]; b.z = lb[2]; b.w = lb[3];
    uint16_t* o = static_cast<uint16_t*>(out) + off;
    __builtin_nontemporal_store(a, reinterpret_cast<u4*>(o));
    __builtin_nontemporal_store(b, reinterpret_cast<u4*>(o + kHalf));
  }
};

template <int P>
__global__ __launch_bounds__(256) void rope_gather(
    const uint16_t* __restrict__ codes, const int32_t* __restrict__ positions, int64_t heads,
    int64_t n, const float* __restrict__ cb, int64_t c, int64_t cur, int64_t window,
    int64_t rows_near, const d2* __restrict__ table, void* __restrict__ out, int64_t items) {
  constexpr int TPT = kHalf / P;          // threads per token
  constexpr int TOK = 256 / TPT;          // tokens per pass of the workgroup
  const int t = threadIdx.x;
  const int g = t % TPT;                  // pair group: pairs [g*P, g*P + P)
  const int tk = t / TPT;
  const int i0 = g * P;
  double fc[P], fs[P];
  const d2* far_row = table + rows_near * kHalf;
#pragma unroll
  for (int k = 0; k < P; ++k) {
    d2 v = far_row[i0 + k];
    fc[k] = v.x;
    fs[k] = v.y;
  }
  const int64_t chunks = (n + kChunk - 1) / kChunk;
  for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
    const int64_t h = item % heads;
    const int64_t rest = item / heads;
    const int64_t b = rest / chunks;
    const int64_t t0 = (rest % chunks) * kChunk;
    const float* cbh = cb + h * c * kD;
    for (int base = 0; base < kChunk; base += TOK) {
      const int64_t tok = t0 + base + tk;
      if (tok >= n) break;
      const uint16_t code = codes[(b * heads + h) * n + tok];
      const int32_t pos = positions[b * n + tok];
      const int64_t ooff = ((b * heads + h) * n + tok) * kD + i0;
      double lo[P], hi[P];
      if ((int64_t)code >= c || pos < 0) {
#pragma unroll
        for (int k = 0; k < P; ++k) lo[k] = hi[k] = __longlong_as_double(0x7FF8000000000000ll);
        OutT<P>::store(out, ooff, lo, hi);
        continue;
      }
      const float* x = cbh + (int64_t)code * kD + i0;
      float xl[P], xh[P];
#pragma unroll
      for (int k = 0; k < P; k += 4) {
        f4 a = *reinterpret_cast<const f4*>(x + k);
        f4 bb = *reinterpret_cast<const f4*>(x + kHalf + k);
        xl[k] = a.x; xl[k + 1] = a.y; xl[k + 2] = a.z; xl[k + 3] = a.w;
        xh[k] = bb.x; xh[k + 1] = bb.y; xh[k + 2] = bb.z; xh[k + 3] = bb.w;
      }
      const int64_t delta = cur - (int64_t)pos;
      if (delta >= 0 && delta < window) {
        const d2* row = table + delta * kHalf + i0;  // delta < rows_near since pos >= 0
#pragma unroll
        for (int k = 0; k < P; ++k) {
          d2 v = row[k];
          lo[k] = (double)xl[k] * v.x - (double)xh[k] * v.y;
          hi[k] = (double)xh[k] * v.x + (double)xl[k] * v.y;
        }
      } else {
#pragma unroll
        for (int k = 0; k < P; ++k) {
          lo[k] = (double)xl[k] * fc[k] - (double)xh[k] * fs[k];
          hi[k] = (double)xh[k] * fc[k] + (double)xl[k] * fs[k];
        }
      }
      OutT<P>::store(out, ooff, lo, hi);
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

extern "C" size_t a2ats_reconstruct_workspace(int64_t d, int64_t cur_pos, int64_t window) {
  if (d != kD || cur_pos < 0) return 0;
  return align_up((size_t)(near_rows(cur_pos, window) + 1) * kHalf * sizeof(d2));
}

extern "C" int a2ats_reconstruct(const uint16_t* codes, const int32_t* positions, int64_t batch,
                                 int64_t heads, int64_t n, int64_t d, const float* codebook,
                                 int64_t c, int64_t cur_pos, int64_t window, int64_t far_offset,
                                 int far_mode, double rope_base, void* out, int out_dtype,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  if (out_dtype != A2ATS_F32 && out_dtype != A2ATS_BF16) return A2ATS_EDTYPE;
  if (d != kD || batch < 1 || heads < 1 || n < 0 || c < 1 || c > 65536) return A2ATS_EINVAL;
  if (cur_pos < 0 || !(rope_base > 0.0) || !std::isfinite(rope_base)) return A2ATS_EINVAL;
  if (far_mode != A2ATS_FAR_FIXED_OFFSET && far_mode != A2ATS_FAR_UNROTATED) return A2ATS_EINVAL;
  if (n == 0) return A2ATS_OK;
  if (!codes || !positions || !codebook || !out) return A2ATS_EINVAL;
  const int64_t rows = near_rows(cur_pos, window);
  const size_t need = a2ats_reconstruct_workspace(d, cur_pos, window);
  if (!ws_ok(workspace, workspace_bytes, need)) return A2ATS_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  d2* table = static_cast<d2*>(workspace);
  A2ATS_TRY(launch("rope_table", rope_table, dim3(grid_for((rows + 1) * kHalf, 256)), dim3(256), 0,
                   s, rows, cur_pos, cur_pos - far_offset, (int)(far_mode == A2ATS_FAR_UNROTATED),
                   rope_base, (int)kD, table));
  const int64_t items = batch * heads * ((n + kChunk - 1) / kChunk);
  // A multiple of 8 * heads workgroups, enough to fill the chip several times over.
  int64_t per = 8 * heads;
  int64_t g = (2048 + per - 1) / per * per;
  if (g > items) g = items;
  if (g > (int64_t)1 << 30) g = (int64_t)1 << 30;
  if (out_dtype == A2ATS_F32)
    return launch("reconstruct", rope_gather<4>, dim3((unsigned)g), dim3(256), 0, s, codes,
                  positions, heads, n, codebook, c, cur_pos, window, rows, table, out, items);
  return launch("reconstruct", rope_gather<8>, dim3((unsigned)g), dim3(256), 0, s, codes, positions,
                heads, n, codebook, c, cur_pos, window, rows, table, out, items);
}
