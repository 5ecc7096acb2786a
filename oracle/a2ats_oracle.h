/* CPU oracle for the A2ATS key-cache hot path -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 restatement of what each step computes, used to check
 * the GPU library.  It shares no source, header, table or helper with the GPU
 * library, and nothing in the product path may link or call it.  Only the
 * tests, the smoke check and the benchmark's CPU-baseline leg use it.
 *
 * Every array is a plain host array, row-major and contiguous.  Inputs are
 * widened to fp64 by the caller (bf16 and fp32 widen exactly); every function
 * computes in fp64 and returns fp64 unless stated otherwise.
 */
#ifndef A2ATS_ORACLE_H
#define A2ATS_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORC_OK 0
#define ORC_EINVAL (-1)
#define ORC_ENOTSPD (-4)

#define ORC_FAR_FIXED_OFFSET 0
#define ORC_FAR_UNROTATED 1

/* H = (1/M) sum_m q_m^T q_m + ridge I   (q: [m,d]; h: [d,d]). */
int orc_second_moment(const double* q, int64_t m, int64_t d, double ridge, double* h);

/* Lower-triangular L with L L^T = H (h, l: [d,d]); ORC_ENOTSPD if a pivot is <= 0. */
int orc_cholesky(const double* h, int64_t d, double* l);

/* code[n] = argmin_j (x_n - c_j) L L^T (x_n - c_j)^T evaluated as ||x_n L - c_j L||^2.
 * l == NULL means L = I (plain nearest centroid).  d1/d2: best and second-best
 * distance (d2 = +inf when c == 1).  Ties go to the lowest index. */
int orc_assign_h(const double* x, int64_t n, int64_t d, const double* cb, int64_t c,
                 const double* l, int32_t* code, double* d1, double* d2);

/* Cosine blend: score_j = -beta * e_j / max_j e_j + (1 - beta) * cos(q, c_j),
 * e_j = ||x - c_j||^2, code = argmax (lowest index on ties).  q: [nq,d], nq in {1,n}.
 * s1/s2: best and second-best score (s2 = -inf when c == 1). */
int orc_assign_cosine(const double* x, int64_t n, int64_t d, const double* q, int64_t nq,
                      const double* cb, int64_t c, double beta, int32_t* code, double* s1,
                      double* s2);

/* ceil(fraction * n) evaluated in fp64; -1 if fraction is NaN or outside [0,1] or n < 0. */
int64_t orc_retrieval_count(int64_t n, double fraction);

/* Retrieval split: the ceil(f*n) keys with the largest cosine to q (ties: lower index
 * first) form ret[], the others bulk[]; both ascending.  cosine[n] receives the cosines. */
int orc_select_retrieval(const double* keys, int64_t n, int64_t d, const double* q,
                         double fraction, int32_t* ret, int32_t* bulk, double* cosine);

/* Windowed-RoPE reconstruction of n tokens: x = cb[codes[t]], rotated at the token's own
 * position if 0 <= cur - pos[t] < window, else at cur - far_b (ORC_FAR_FIXED_OFFSET) or
 * not at all (ORC_FAR_UNROTATED).  A token with codes[t] >= c or pos[t] < 0 gets a NaN row.
 * far_count (optional) receives the number of far tokens. */
int orc_reconstruct(const uint16_t* codes, const int32_t* pos, int64_t n, int64_t d,
                    const double* cb, int64_t c, int64_t cur, int64_t window, int64_t far_b,
                    int far_mode, double base, double* out, int64_t* far_count);

/* Query-side far rotation (Eq. 11, R_b on the query): every row of x [rows, d] rotated as a
 * token at `position`, same pairs and frequencies as orc_reconstruct. */
int orc_rope_at(const double* x, int64_t rows, int64_t d, double position, double base,
                double* out);

/* k-means update: each cluster's centroid becomes the fp64 mean of its member rows (ascending
 * row order), an empty cluster keeps cb_in's row; counts (optional) receives the sizes. */
int orc_kmeans_update(const double* x, int64_t n, int64_t d, const int32_t* code, int64_t k,
                      const double* cb_in, double* cb_out, int64_t* counts);

/* Lloyd's iterations with the H-weighted (L) or plain (L == NULL) assignment; cb in place,
 * rounded to fp32 after each update; code receives the final assignment. */
int orc_kmeans(const double* x, int64_t n, int64_t d, int64_t k, const double* l, int iters,
               double* cb, int32_t* code);

/* k-means++ seeding in z-space: z = fp32(x L) (x without L), c_0 = floor(r_0 n / 2^64), then
 * each next center drawn with probability D^2 / sum D^2 (D^2: squared z-space distance to the
 * nearest chosen center, fp64), the weights taken as integers floor(D^2 2^e) with
 * e = 60 - ceil(log2 n) - ceil(log2 (4 max ||z||^2)) and the draw floor(r_t W / 2^64) located
 * in their running sum.  idx[t] = the row chosen as center t. */
int orc_kmeans_init(const double* x, int64_t n, int64_t d, int64_t k, const double* l,
                    const uint64_t* r, int32_t* idx);

/* Approximate-score top-K over codes: table lut_j = fl32(qb . c_j) (fp64 products and sum in
 * dimension order), score_t = lut[codes[t]] (-inf for codes >= c); the k largest (equal
 * scores: lower index first) in ascending index order, with their scores. */
int orc_topk_codes(const double* qb, int64_t d, const uint16_t* codes, int64_t n,
                   const double* cb, int64_t c, int64_t k, int32_t* idx, double* score);

/* Threads the OpenMP loops use. */
int orc_threads(void);

/* Round fp64 values to bf16 (nearest, ties to even), raw bits. */
void orc_round_bf16(const double* x, int64_t n, uint16_t* out);

#ifdef __cplusplus
}
#endif
#endif
