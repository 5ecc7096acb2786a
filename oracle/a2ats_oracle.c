/* CPU oracle for the A2ATS key-cache hot path -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain fp64 loops that restate, step by step, what the pages define.  No
 * blocking, no fusion, no reordering beyond the definitions.  OpenMP only
 * splits independent rows (keys, tokens) across threads; every per-row
 * computation is sequential and identical to the single-threaded one.
 *
 * Sources (web pages, cited by title and section):
 *  [API]  "veloxquant_mlx.quantizers.a2ats module" (API reference): the five
 *         public functions and their docstrings.
 *  [DOC1] "A2ATS-adapted -- Windowed RoPE + Query-Aware Retrieval VQ", section
 *         "How it works".
 *  [DOC2] "A2ATS-adapted" docs, sections "Configuration reference",
 *         "The one setting worth tuning: a2ats_window", "How it works" and
 *         "For contributors -- paper fidelity".
 *  [LOG]  veloxquant-mlx changelog, entry "A2ATS-adapted paper-fidelity fixes (#29)".
 *  RoPE frequencies follow RoFormer (the paper's cited rotary embedding).
 */
#include "a2ats_oracle.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ calibrate */

/* [API] a2ats_query_second_moment, Eq. 10: H = E[q^T q] over the M query rows
 * (a plain, uncentred sample mean), then ridge added to the diagonal. */
int orc_second_moment(const double* q, int64_t m, int64_t d, double ridge, double* h) {
  if (m <= 0 || d <= 0 || !(ridge >= 0.0)) return ORC_EINVAL;
  for (int64_t a = 0; a < d; ++a) {
    for (int64_t b = 0; b < d; ++b) {
      double s = 0.0;
      for (int64_t r = 0; r < m; ++r) s += q[r * d + a] * q[r * d + b];
      h[a * d + b] = s / (double)m;
    }
  }
  for (int64_t a = 0; a < d; ++a) h[a * d + a] += ridge;
  return ORC_OK;
}

/* [API] a2ats_cholesky_factor, Eq. 15: H = L L^T with L lower triangular.
 * Cholesky-Banachiewicz, row by row:
 *   L_jj = sqrt(H_jj - sum_{k<j} L_jk^2),  L_ij = (H_ij - sum_{k<j} L_ik L_jk) / L_jj. */
int orc_cholesky(const double* h, int64_t d, double* l) {
  if (d <= 0) return ORC_EINVAL;
  memset(l, 0, sizeof(double) * (size_t)(d * d));
  for (int64_t i = 0; i < d; ++i) {
    for (int64_t j = 0; j <= i; ++j) {
      double s = h[i * d + j];
      for (int64_t k = 0; k < j; ++k) s -= l[i * d + k] * l[j * d + k];
      if (i == j) {
        if (!(s > 0.0)) return ORC_ENOTSPD;
        l[i * d + i] = sqrt(s);
      } else {
        l[i * d + j] = s / l[j * d + j];
      }
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------ encode */

/* [API] a2ats_h_weighted_assignment, Eq. 14 evaluated through the Eq. 17 identity:
 * (x - c_j) H (x - c_j)^T = ||x L - c_j L||^2 with z = x L and w_j = c_j L (row vectors).
 * With l == NULL the weighting is the identity: plain nearest centroid (the bulk path of
 * [DOC1] step 2). */
int orc_assign_h(const double* x, int64_t n, int64_t d, const double* cb, int64_t c,
                 const double* l, int32_t* code, double* d1, double* d2) {
  if (n < 0 || d <= 0 || c <= 0) return ORC_EINVAL;
  double* w = (double*)malloc(sizeof(double) * (size_t)(c * d));
  if (!w) return ORC_EINVAL;
  /* w_j = c_j L */
  for (int64_t j = 0; j < c; ++j) {
    for (int64_t a = 0; a < d; ++a) {
      if (!l) { w[j * d + a] = cb[j * d + a]; continue; }
      double s = 0.0;
      for (int64_t b = 0; b < d; ++b) s += cb[j * d + b] * l[b * d + a];
      w[j * d + a] = s;
    }
  }
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < n; ++t) {
    double z[1024];
    double* zz = d <= 1024 ? z : (double*)malloc(sizeof(double) * (size_t)d);
    /* z = x_t L */
    for (int64_t a = 0; a < d; ++a) {
      if (!l) { zz[a] = x[t * d + a]; continue; }
      double s = 0.0;
      for (int64_t b = 0; b < d; ++b) s += x[t * d + b] * l[b * d + a];
      zz[a] = s;
    }
    double best = INFINITY, second = INFINITY;
    int32_t arg = 0;
    for (int64_t j = 0; j < c; ++j) {
      double s = 0.0;
      for (int64_t a = 0; a < d; ++a) {
        double e = zz[a] - w[j * d + a];
        s += e * e;
      }
      if (s < best) { second = best; best = s; arg = (int32_t)j; }
      else if (s < second) second = s;
    }
    code[t] = arg;
    if (d1) d1[t] = best;
    if (d2) d2[t] = second;
    if (zz != z) free(zz);
  }
  free(w);
  return ORC_OK;
}

/* [API] a2ats_query_aware_assignment (the cosine-blend substitute used on the decode path):
 *   score_j = beta * (-e_j / max_k e_k) + (1 - beta) * cos(q, c_j),  e_j = ||x - c_j||^2,
 * code = argmax_j score_j.  The reconstruction term is normalised by the per-row maximum
 * error; when that maximum is 0 the term is 0.  A zero-norm query or centroid has cosine 0. */
int orc_assign_cosine(const double* x, int64_t n, int64_t d, const double* q, int64_t nq,
                      const double* cb, int64_t c, double beta, int32_t* code, double* s1,
                      double* s2) {
  if (n < 0 || d <= 0 || c <= 0 || !(beta >= 0.0 && beta <= 1.0)) return ORC_EINVAL;
  if (!(nq == 1 || nq == n)) return ORC_EINVAL;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t t = 0; t < n; ++t) {
    const double* xr = x + t * d;
    const double* qr = q + (nq == 1 ? 0 : t) * d;
    double* e = (double*)malloc(sizeof(double) * (size_t)c);
    double emax = 0.0;
    for (int64_t j = 0; j < c; ++j) {
      double s = 0.0;
      for (int64_t a = 0; a < d; ++a) {
        double df = xr[a] - cb[j * d + a];
        s += df * df;
      }
      e[j] = s;
      if (j == 0 || s > emax) emax = s;
    }
    double qn = 0.0;
    for (int64_t a = 0; a < d; ++a) qn += qr[a] * qr[a];
    qn = sqrt(qn);
    double best = -INFINITY, second = -INFINITY;
    int32_t arg = 0;
    for (int64_t j = 0; j < c; ++j) {
      double dot = 0.0, cn = 0.0;
      for (int64_t a = 0; a < d; ++a) {
        dot += qr[a] * cb[j * d + a];
        cn += cb[j * d + a] * cb[j * d + a];
      }
      cn = sqrt(cn);
      double cosv = (qn > 0.0 && cn > 0.0) ? dot / (qn * cn) : 0.0;
      double err = emax > 0.0 ? e[j] / emax : 0.0;
      double s = beta * (-err) + (1.0 - beta) * cosv;
      if (s > best) { second = best; best = s; arg = (int32_t)j; }
      else if (s > second) second = s;
    }
    code[t] = arg;
    if (s1) s1[t] = best;
    if (s2) s2[t] = second;
    free(e);
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------ retrieval split */

/* [API] a2ats_select_retrieval_set: the retrieval set has ceil(retrieval_fraction * N)
 * members, evaluated literally in fp64. */
int64_t orc_retrieval_count(int64_t n, double fraction) {
  if (n < 0 || !(fraction >= 0.0 && fraction <= 1.0)) return -1;
  return (int64_t)ceil(fraction * (double)n);
}

typedef struct { double cosv; int32_t idx; } orc_scored;

/* Descending cosine; equal cosines keep the lower index first. */
static int orc_cmp_desc(const void* pa, const void* pb) {
  const orc_scored* a = (const orc_scored*)pa;
  const orc_scored* b = (const orc_scored*)pb;
  if (a->cosv > b->cosv) return -1;
  if (a->cosv < b->cosv) return 1;
  return (a->idx > b->idx) - (a->idx < b->idx);
}

static int orc_cmp_i32(const void* pa, const void* pb) {
  int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
  return (a > b) - (a < b);
}

/* [API] a2ats_select_retrieval_set: rank the N keys by cosine similarity to the query,
 * take the top ceil(f*N) as the retrieval set and the rest as the bulk; the two index
 * sets are disjoint and together cover 0..N-1 once.  A zero-norm key or query has
 * cosine 0.  The full sort gives the same set as the pages' heap top-k. */
int orc_select_retrieval(const double* keys, int64_t n, int64_t d, const double* q,
                         double fraction, int32_t* ret, int32_t* bulk, double* cosine) {
  int64_t nr = orc_retrieval_count(n, fraction);
  if (nr < 0 || d <= 0) return ORC_EINVAL;
  orc_scored* s = (orc_scored*)malloc(sizeof(orc_scored) * (size_t)(n > 0 ? n : 1));
  double qn = 0.0;
  for (int64_t a = 0; a < d; ++a) qn += q[a] * q[a];
  qn = sqrt(qn);
  for (int64_t i = 0; i < n; ++i) {
    double dot = 0.0, kn = 0.0;
    for (int64_t a = 0; a < d; ++a) {
      dot += keys[i * d + a] * q[a];
      kn += keys[i * d + a] * keys[i * d + a];
    }
    kn = sqrt(kn);
    s[i].cosv = (kn > 0.0 && qn > 0.0) ? dot / (kn * qn) : 0.0;
    s[i].idx = (int32_t)i;
    if (cosine) cosine[i] = s[i].cosv;
  }
  qsort(s, (size_t)n, sizeof(orc_scored), orc_cmp_desc);
  for (int64_t i = 0; i < nr; ++i) ret[i] = s[i].idx;
  for (int64_t i = nr; i < n; ++i) bulk[i - nr] = s[i].idx;
  qsort(ret, (size_t)nr, sizeof(int32_t), orc_cmp_i32);
  qsort(bulk, (size_t)(n - nr), sizeof(int32_t), orc_cmp_i32);
  free(s);
  return ORC_OK;
}

/* ------------------------------------------------------------------ reconstruct */

/* Dequantise and apply windowed RoPE.
 * [DOC1] steps 3-4: the pre-RoPE key is the assigned centroid; a token within `window`
 * positions of the current decode position gets exact RoPE at its own position (near iff
 * 0 <= cur - pos < window, so window <= 0 makes every token far and window beyond the
 * sequence length makes every token exact, [DOC2] window table).  Far tokens share one
 * fixed-offset rotation: [DOC2] "paper fidelity" puts R_b (Eq. 11) on the query and leaves
 * far keys unrotated (Eq. 12); rotating every far key at the absolute position cur - b
 * is the key-side image of the same score, since RoPE(q, cur) . RoPE(k, cur - b) =
 * RoPE(q, b) . k.  b is the a2ats_b knob ([DOC2] configuration reference, default 2048);
 * ORC_FAR_UNROTATED returns far keys unrotated (literal Eq. 12).
 * Rotation: half-split pairs (i, i + d/2), theta_i = base^(-2i/d) (RoFormer), angle
 * phi = P * theta_i:  o_i = x_i cos phi - x_{i+d/2} sin phi,
 *                     o_{i+d/2} = x_{i+d/2} cos phi + x_i sin phi. */
int orc_reconstruct(const uint16_t* codes, const int32_t* pos, int64_t n, int64_t d,
                    const double* cb, int64_t c, int64_t cur, int64_t window, int64_t far_b,
                    int far_mode, double base, double* out, int64_t* far_count) {
  if (n < 0 || d <= 0 || (d % 2) != 0 || c <= 0) return ORC_EINVAL;
  if (far_mode != ORC_FAR_FIXED_OFFSET && far_mode != ORC_FAR_UNROTATED) return ORC_EINVAL;
  const int64_t half = d / 2;
  int64_t nfar = 0;
#pragma omp parallel for schedule(static) reduction(+ : nfar)
  for (int64_t t = 0; t < n; ++t) {
    double* o = out + t * d;
    if ((int64_t)codes[t] >= c || pos[t] < 0) {
      for (int64_t a = 0; a < d; ++a) o[a] = NAN;
      continue;
    }
    const double* x = cb + (int64_t)codes[t] * d;
    int64_t delta = cur - (int64_t)pos[t];
    int near = (delta >= 0 && delta < window);
    if (!near) nfar += 1;
    if (!near && far_mode == ORC_FAR_UNROTATED) {
      for (int64_t a = 0; a < d; ++a) o[a] = x[a];
      continue;
    }
    double p = near ? (double)pos[t] : (double)(cur - far_b);
    for (int64_t i = 0; i < half; ++i) {
      double theta = pow(base, -2.0 * (double)i / (double)d);
      double phi = p * theta;
      double cs = cos(phi), sn = sin(phi);
      o[i] = x[i] * cs - x[i + half] * sn;
      o[i + half] = x[i + half] * cs + x[i] * sn;
    }
  }
  if (far_count) *far_count = nfar;
  return ORC_OK;
}

/* ------------------------------------------------------------------ query-side far rotation */

/* The query-side half of Eq. 11: [DOC2] "paper fidelity" keeps far keys unrotated (Eq. 12)
 * and puts the constant far rotation R_b on the query, so the far attention logit is
 * (q R_b) . k; [LOG] adds this half as a2ats_apply_far_query_rope.  Each row of x is
 * rotated as a token at position `position` (= b): the same half-split pairs and RoFormer
 * frequencies as orc_reconstruct, in fp64. */
int orc_rope_at(const double* x, int64_t rows, int64_t d, double position, double base,
                double* out) {
  if (rows < 0 || d <= 0 || (d % 2) != 0 || !(base > 0.0)) return ORC_EINVAL;
  const int64_t half = d / 2;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const double* q = x + r * d;
    double* o = out + r * d;
    for (int64_t i = 0; i < half; ++i) {
      double theta = pow(base, -2.0 * (double)i / (double)d);
      double phi = position * theta;
      double cs = cos(phi), sn = sin(phi);
      o[i] = q[i] * cs - q[i + half] * sn;
      o[i + half] = q[i + half] * cs + q[i] * sn;
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------ codebook training */

/* The update step of k-means in z-space ([API] a2ats_cholesky_factor: Eq. 16-18 make the
 * H-weighted objective a plain Euclidean one on z = xL, so conventional k-means applies).
 * The Euclidean k-means update in z-space is the mean of the cluster's z rows; since
 * z = xL is linear and L is invertible, mapping that mean back (w L^-1) gives the mean of
 * the cluster's x rows: the original-space centroid is the plain member mean, with or
 * without H.  Members are summed in ascending row order in fp64, then divided by the count;
 * a cluster with no member keeps its previous centroid.  counts (optional) gets the sizes. */
int orc_kmeans_update(const double* x, int64_t n, int64_t d, const int32_t* code, int64_t k,
                      const double* cb_in, double* cb_out, int64_t* counts) {
  if (n < 0 || d <= 0 || k <= 0) return ORC_EINVAL;
  double* sum = (double*)calloc((size_t)(k * d), sizeof(double));
  int64_t* cnt = (int64_t*)calloc((size_t)k, sizeof(int64_t));
  if (!sum || !cnt) { free(sum); free(cnt); return ORC_EINVAL; }
  for (int64_t t = 0; t < n; ++t) {
    const int64_t j = code[t];
    if (j < 0 || j >= k) continue;
    cnt[j] += 1;
    for (int64_t a = 0; a < d; ++a) sum[j * d + a] += x[t * d + a];
  }
  for (int64_t j = 0; j < k; ++j) {
    for (int64_t a = 0; a < d; ++a)
      cb_out[j * d + a] = cnt[j] > 0 ? sum[j * d + a] / (double)cnt[j] : cb_in[j * d + a];
    if (counts) counts[j] = cnt[j];
  }
  free(sum);
  free(cnt);
  return ORC_OK;
}

/* Lloyd's iteration with the H-weighted assignment: `iters` rounds of (orc_assign_h with L,
 * or plain without, then orc_kmeans_update), cb updated in place, then the final assignment
 * into code.  Each round's new centroids are rounded to fp32 before the next assignment, as
 * a codebook stored in fp32 would be. */
int orc_kmeans(const double* x, int64_t n, int64_t d, int64_t k, const double* l, int iters,
               double* cb, int32_t* code) {
  if (n < 0 || d <= 0 || k <= 0 || iters < 0) return ORC_EINVAL;
  double* nxt = (double*)malloc(sizeof(double) * (size_t)(k * d));
  if (!nxt) return ORC_EINVAL;
  int st = ORC_OK;
  for (int it = 0; it < iters && st == ORC_OK; ++it) {
    st = orc_assign_h(x, n, d, cb, k, l, code, NULL, NULL);
    if (st == ORC_OK) st = orc_kmeans_update(x, n, d, code, k, cb, nxt, NULL);
    for (int64_t e = 0; e < k * d; ++e) cb[e] = (double)(float)nxt[e];
  }
  if (st == ORC_OK) st = orc_assign_h(x, n, d, cb, k, l, code, NULL, NULL);
  free(nxt);
  return st;
}

/* ------------------------------------------------------------------ k-means++ seeding */

/* ceil(log2(x)) for x > 0, exactly (frexp: x = m 2^p with m in [0.5, 1)). */
static int orc_clog2(double x) {
  int p = 0;
  const double m = frexp(x, &p);
  return m == 0.5 ? p - 1 : p;
}

/* floor(a * b / 2^64) for unsigned 64-bit a, b: the draw r (uniform over [0, 2^64)) scaled
 * to [0, b). */
static uint64_t orc_mulhi(uint64_t a, uint64_t b) {
  return (uint64_t)(((unsigned __int128)a * (unsigned __int128)b) >> 64);
}

/* k-means++ seeding in z-space ([API] a2ats_cholesky_factor: Eq. 16-18 turn the H-weighted
 * objective into a plain Euclidean one on z = x L, "what lets conventional k-means++ build
 * the codebook"; the docs' calibration trains with a seed).  The random draws are inputs:
 * r[t], uniform over [0, 2^64), for center t.  Steps, k-means++ as Arthur and Vassilvitskii
 * define it:
 *   z_i = x_i L (each z_ia the fp64 sum over b in order of x_ib L_ba, rounded to fp32; x_i
 *         itself without L), Z = max_i ||z_i||^2;
 *   c_0 = floor(r_0 n / 2^64)  (uniform over the rows);
 *   for t = 1 .. k-1:  D2_i = min over s < t of ||z_i - z_{c_s}||^2  (fp64, dimensions in
 *         order), each D2_i taken as the integer w_i = floor(D2_i 2^e) with the fixed
 *         e = 60 - ceil(log2 n) - ceil(log2 4Z) (so the sum cannot overflow; D2 <= 4Z), and
 *         c_t = the first row i whose running integer sum w_0 + .. + w_i exceeds
 *         floor(r_t W / 2^64), W = sum of all w (row i is drawn with probability w_i / W,
 *         the D^2 weighting); c_t = floor(r_t n / 2^64) when W = 0.
 * A chosen row has D2 = 0 and is never drawn again while W > 0.  idx[t] = c_t. */
int orc_kmeans_init(const double* x, int64_t n, int64_t d, int64_t k, const double* l,
                    const uint64_t* r, int32_t* idx) {
  if (n <= 0 || d <= 0 || k <= 0) return ORC_EINVAL;
  double* z = (double*)malloc(sizeof(double) * (size_t)(n * d));
  double* d2 = (double*)malloc(sizeof(double) * (size_t)n);
  uint64_t* w = (uint64_t*)malloc(sizeof(uint64_t) * (size_t)n);
  if (!z || !d2 || !w) { free(z); free(d2); free(w); return ORC_EINVAL; }
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    for (int64_t a = 0; a < d; ++a) {
      double s = 0.0;
      if (l) {
        for (int64_t b = 0; b < d; ++b) s += x[i * d + b] * l[b * d + a];
      } else {
        s = x[i * d + a];
      }
      z[i * d + a] = (double)(float)s;
    }
  }
  double zmax = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    double s = 0.0;
    for (int64_t a = 0; a < d; ++a) s += z[i * d + a] * z[i * d + a];
    if (s > zmax) zmax = s;
  }
  int e = 60 - orc_clog2((double)n);
  if (zmax > 0.0) e -= orc_clog2(4.0 * zmax);
  int64_t c = (int64_t)orc_mulhi(r[0], (uint64_t)n);
  idx[0] = (int32_t)c;
  for (int64_t t = 1; t < k; ++t) {
    const double* zc = z + c * d;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
      double s = 0.0;
      for (int64_t a = 0; a < d; ++a) {
        const double df = z[i * d + a] - zc[a];
        s += df * df;
      }
      if (t == 1 || s < d2[i]) d2[i] = s;
      w[i] = (uint64_t)floor(ldexp(d2[i], e));
    }
    uint64_t tot = 0;
    for (int64_t i = 0; i < n; ++i) tot += w[i];
    if (tot == 0) {
      c = (int64_t)orc_mulhi(r[t], (uint64_t)n);
    } else {
      const uint64_t target = orc_mulhi(r[t], tot);
      uint64_t run = 0;
      c = n - 1;
      for (int64_t i = 0; i < n; ++i) {
        run += w[i];
        if (run > target) { c = i; break; }
      }
    }
    idx[t] = (int32_t)c;
  }
  free(z);
  free(d2);
  free(w);
  return ORC_OK;
}

/* ------------------------------------------------------------------ top-K over codes */

static int orc_cmp_score_desc(const void* a, const void* b) {
  const orc_scored* x = (const orc_scored*)a;
  const orc_scored* y = (const orc_scored*)b;
  if (x->cosv > y->cosv) return -1;
  if (x->cosv < y->cosv) return 1;
  return (x->idx > y->idx) - (x->idx < y->idx);
}

/* [ABS] A2ATS approximates attention scores with the quantised keys to retrieve the top-K
 * tokens.  With far keys unrotated (Eq. 12) and R_b on the query (Eq. 11), the approximate
 * logit of token t is (q R_b) . c_{code_t}: one table of C values per query, gathered by
 * code.  qb is q R_b.  The table entries are the fp64 dot products (each product, then the
 * running sum, in dimension order) rounded once to fp32.  A token whose code is >= C scores
 * -inf.  The K tokens with the largest scores (equal scores: lower index first) are returned
 * in ascending index order with their scores. */
int orc_topk_codes(const double* qb, int64_t d, const uint16_t* codes, int64_t n,
                   const double* cb, int64_t c, int64_t k, int32_t* idx, double* score) {
  if (d <= 0 || n < 0 || c <= 0 || k < 0 || k > n) return ORC_EINVAL;
  double* lut = (double*)malloc(sizeof(double) * (size_t)c);
  orc_scored* s = (orc_scored*)malloc(sizeof(orc_scored) * (size_t)(n > 0 ? n : 1));
  if (!lut || !s) { free(lut); free(s); return ORC_EINVAL; }
  for (int64_t j = 0; j < c; ++j) {
    double acc = 0.0;
    for (int64_t a = 0; a < d; ++a) acc += qb[a] * cb[j * d + a];
    lut[j] = (double)(float)acc;
  }
  for (int64_t t = 0; t < n; ++t) {
    s[t].cosv = codes[t] < c ? lut[codes[t]] : -INFINITY;  /* the record's score field */
    s[t].idx = (int32_t)t;
  }
  qsort(s, (size_t)n, sizeof(orc_scored), orc_cmp_score_desc);
  /* the first k, back in index order */
  int32_t* pick = (int32_t*)malloc(sizeof(int32_t) * (size_t)(k > 0 ? k : 1));
  if (!pick) { free(lut); free(s); return ORC_EINVAL; }
  for (int64_t i = 0; i < k; ++i) pick[i] = s[i].idx;
  qsort(pick, (size_t)k, sizeof(int32_t), orc_cmp_i32);
  for (int64_t i = 0; i < k; ++i) {
    idx[i] = pick[i];
    if (score) score[i] = codes[pick[i]] < c ? lut[codes[pick[i]]] : -INFINITY;
  }
  free(pick);
  free(lut);
  free(s);
  return ORC_OK;
}

/* ------------------------------------------------------------------ output rounding */

/* Nearest bf16 (8 significant bits, fp32 exponent range), ties to even, computed from
 * the fp64 value directly so no intermediate fp32 rounding occurs. */
void orc_round_bf16(const double* x, int64_t n, uint16_t* out) {
  for (int64_t t = 0; t < n; ++t) {
    double v = x[t];
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    if (isnan(v)) { out[t] = 0x7FC0u; continue; }
    if (a == 0.0) { out[t] = sign; continue; }
    int e;
    frexp(a, &e);                       /* a = m * 2^e, m in [0.5, 1) */
    int q = e - 8;                      /* spacing of 8-significant-bit values near a */
    if (q < -133) q = -133;             /* bf16 subnormal spacing is 2^-133 */
    double scaled = ldexp(a, -q);       /* exact: a power-of-two scale */
    double fl = floor(scaled);
    double rem = scaled - fl;
    double r = fl;
    if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0)) r = fl + 1.0;
    double rv = ldexp(r, q);
    if (rv >= ldexp(1.0, 128)) { out[t] = sign | 0x7F80u; continue; } /* overflow to inf */
    float f = (float)rv;                /* exact: rv has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    out[t] = (uint16_t)(u >> 16) | sign;
  }
}

/* Threads OpenMP uses for the parallel loops above. */
int orc_threads(void) { return omp_get_max_threads(); }
