/* a2ats.h -- C ABI of the A2ATS key-cache hot path on gfx950 (MI355X).
 *
 * The operations of the A2ATS method ("A2ATS: Retrieval-Based KV Cache Reduction via
 * Windowed Rotary Position Embedding and Query-Aware Vector Quantization", as adapted and
 * documented by the "A2ATS-adapted" VeloxQuant-MLX pages):
 *   calibrate          H = E[q^T q] + ridge I and its Cholesky factor L
 *   encode             H-weighted (or plain) nearest-centroid codes, uint16
 *   assign_cosine      the cosine-blend assignment of the decode path
 *   select_retrieval   top-fraction cosine split of token indices
 *   reconstruct        centroid gather + windowed RoPE (and its incremental update for far
 *                      keys left unrotated)
 *   far_query_rope     the query-side far rotation R_b of Eq. 11
 *   pq_*               the sub-vector (product) codes of the pages' default configuration
 *   kmeans*            codebook training: Lloyd's k-means with the H-weighted assignment
 *
 * Conventions shared by every call:
 *  - All array pointers are DEVICE pointers owned by the caller, row-major, contiguous,
 *    and must not alias one another unless stated.  The library never allocates device
 *    memory and keeps no state between calls (apart from optional profiling, below).
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Every call
 *    enqueues its kernels on that stream and returns without waiting, except
 *    a2ats_calibrate, which waits for its own work so it can report a non-positive-definite
 *    input.
 *  - Scratch memory is passed in as `workspace` (device, 256-byte aligned) of at least the
 *    size returned by the matching *_workspace() query; its contents on entry are ignored.
 *  - Arguments are validated on the host before anything is launched; an invalid call
 *    returns a negative status and launches nothing.  Conditions that only the data can
 *    reveal (an out-of-range code or position) do not fault: they produce NaN outputs as
 *    documented per call.
 *  - Results are deterministic: the same inputs give bitwise identical outputs.
 *  - This header needs no HIP headers.
 */
#ifndef A2ATS_H
#define A2ATS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define A2ATS_VERSION 1

/* Status codes. */
#define A2ATS_OK 0
#define A2ATS_EINVAL (-1)     /* a size, pointer or parameter is invalid */
#define A2ATS_EDTYPE (-2)     /* unsupported dtype */
#define A2ATS_EWORKSPACE (-3) /* workspace missing, too small or misaligned */
#define A2ATS_ENOTSPD (-4)    /* calibrate: H is not positive definite */
#define A2ATS_EHIP (-5)       /* the HIP runtime reported an error */
#define A2ATS_ESCRATCH (-6)   /* larger than the fixed scratch of an allocation-free call */

/* Element types of key / query / output arrays. */
#define A2ATS_F32 0
#define A2ATS_BF16 1

/* Far-token treatment in reconstruct. */
#define A2ATS_FAR_FIXED_OFFSET 0 /* rotate far keys at position cur_pos - far_offset */
#define A2ATS_FAR_UNROTATED 1    /* leave far keys unrotated */

/* Head dimension supported by encode, select_retrieval and reconstruct. */
#define A2ATS_HEAD_DIM 128

/* Human-readable text for a status code (static storage). */
const char* a2ats_strerror(int status);

/* A2ATS_VERSION of the library actually loaded. */
int a2ats_version(void);

/* ---------------------------------------------------------------------------------------
 * Retrieval-set size: ceil(fraction * n) evaluated as an fp64 product, as the API page
 * "veloxquant_mlx.quantizers.a2ats module" defines for a2ats_select_retrieval_set.
 * Returns -1 if n < 0 or fraction is NaN or outside [0, 1].  Host only.
 */
int64_t a2ats_retrieval_count(int64_t n, double fraction);

/* ---------------------------------------------------------------------------------------
 * calibrate -- "veloxquant_mlx.quantizers.a2ats module", a2ats_query_second_moment (Eq. 10)
 * and a2ats_cholesky_factor (Eq. 15).
 *
 *   queries  [heads, m, d] fp32   post-position-embedding query states
 *   h_out    [heads, d, d] fp32   H = (1/m) sum_r q_r^T q_r + ridge I   (uncentred mean)
 *   l_out    [heads, d, d] fp32   lower-triangular L with L L^T = H, upper triangle zero;
 *                                 factored in fp64 from the fp32 H written to h_out
 * Accumulation is fp64; each output is rounded once to fp32.
 * Requires 1 <= d <= 128, m >= 1, heads >= 1, ridge >= 0.  Waits for completion.
 * Returns A2ATS_ENOTSPD (h_out still written, l_out undefined) if a pivot is <= 0.
 */
size_t a2ats_calibrate_workspace(int64_t heads, int64_t m, int64_t d);
int a2ats_calibrate(const float* queries, int64_t heads, int64_t m, int64_t d, double ridge,
                    float* h_out, float* l_out, void* workspace, size_t workspace_bytes,
                    void* stream);

/* ---------------------------------------------------------------------------------------
 * encode -- "veloxquant_mlx.quantizers.a2ats module", a2ats_h_weighted_assignment
 * (Eq. 14 through the Eq. 17 identity): for every selected key k of head h,
 *     codes[h, row] = argmin_j (k - c_j) H (k - c_j)^T,   H = L L^T,
 * with chol == NULL meaning H = I (plain nearest centroid, the bulk path).  Ties go to the
 * lowest centroid index.  The minimiser is exact: a fp16 MFMA pass proposes candidates
 * under a rigorous error bound and fp64 arithmetic decides every close call.
 *
 *   keys      [heads, n, d]  fp32 or bf16 (keys_dtype); d must be 128
 *   idx       [heads, n_idx] int32 row indices in [0, n) to encode, or NULL for all rows
 *             (then n_idx is ignored); only the listed rows of codes/dist are written;
 *             entries outside [0, n) are skipped
 *   codebook  [heads, c, d]  fp32 centroids in the original (un-transformed) space
 *   chol      [heads, d, d]  fp32 lower-triangular L, or NULL
 *   codes     [heads, n]     uint16 output; 1 <= c <= 65536
 *   dist      [heads, n]     fp32 output (k - c_code) H (k - c_code)^T, or NULL
 *   stats     device a2ats_encode_stats, or NULL: counters of how each key was decided
 * Keys with an element of magnitude >= 65504 (outside fp16) are decided entirely in fp64.
 * Returns without waiting.
 */
typedef struct a2ats_encode_stats {
  uint32_t keys;        /* keys encoded */
  uint32_t direct;      /* decided by the MFMA pass alone */
  uint32_t reranked;    /* decided after an fp64 rerank of the leading candidates */
  uint32_t rescanned;   /* decided by a second candidate pass over the codebook */
  uint32_t full_scan;   /* decided by an fp64 scan of the whole codebook */
  uint32_t reserved[3];
} a2ats_encode_stats;

size_t a2ats_encode_workspace(int64_t heads, int64_t n, int64_t d, int64_t c);
int a2ats_encode(const void* keys, int keys_dtype, int64_t heads, int64_t n, int64_t d,
                 const int32_t* idx, int64_t n_idx, const float* codebook, int64_t c,
                 const float* chol, uint16_t* codes, float* dist, a2ats_encode_stats* stats,
                 void* workspace, size_t workspace_bytes, void* stream);

/* encode in two calls -- the same computation as a2ats_encode, split at the boundary between
 * its codebook side and its key side, so that the codebook side (which depends on the
 * codebook and L only) can run once for several key sets, or on another stream while the
 * keys are still being produced.
 *
 * a2ats_encode_prepare writes the prepared codebook (fp64 rows v = c L L^T, b = ||c L||^2,
 * the fp16 MFMA fragments, the bias and the per-head scales) into a workspace of
 * a2ats_encode_workspace(heads, n, d, c) bytes; n is the largest key count the workspace will
 * serve.  codebook and chol as for a2ats_encode (chol NULL: plain nearest centroid).
 *
 * a2ats_encode_prepared encodes keys with a workspace that a2ats_encode_prepare filled for the
 * same heads, n, c and chol-or-NULL; the other arguments are as for a2ats_encode.  It does not
 * read the codebook or L again (chol only selects the H-weighted rule, and with fp32 keys and
 * dist != NULL it is read for ||k L||^2).  Any number of runs may follow one prepare:
 * a2ats_encode_prepare also clears the run state kept in the workspace (list lengths,
 * decision counters), and every run leaves it cleared when its last kernel ends.  Runs on one
 * workspace must be ordered on one stream (they share that state and the list buffers); the
 * workspace must not be written between prepare and the runs; after a run that returned an
 * error, prepare again.  Both return without waiting; errors as for a2ats_encode.
 */
int a2ats_encode_prepare(const float* codebook, int64_t c, const float* chol, int64_t heads,
                         int64_t n, int64_t d, void* workspace, size_t workspace_bytes,
                         void* stream);
int a2ats_encode_prepared(const void* keys, int keys_dtype, int64_t heads, int64_t n, int64_t d,
                          const int32_t* idx, int64_t n_idx, int64_t c, const float* chol,
                          uint16_t* codes, float* dist, a2ats_encode_stats* stats,
                          void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * assign_cosine -- "veloxquant_mlx.quantizers.a2ats module", a2ats_query_aware_assignment:
 *     score_j = beta * (-e_j / max_i e_i) + (1 - beta) * cos(q, c_j),  e_j = ||x - c_j||^2,
 *     codes[h, r] = argmax_j score_j  (lowest index on ties).
 * The error term is 0 when max_i e_i == 0; a zero-norm q or c_j has cosine 0.  beta = 1 is
 * plain nearest centroid.  Computed in fp64.
 *
 *   x         [heads, n, d]   fp32 or bf16 (x_dtype)
 *   query     [heads, nq, d]  same dtype as x; nq == 1 (one query per head) or nq == n
 *   codebook  [heads, c, d]   fp32
 *   codes     [heads, n]      uint16 output
 * Requires 1 <= d <= 256 and 1 <= c <= 65536, beta in [0, 1].  Workspace:
 * a2ats_assign_cosine_workspace(heads, n, c) bytes (per-centroid errors and cosine numerators
 * of a batch of rows, at most 128 MiB; larger inputs run in several batches).
 */
size_t a2ats_assign_cosine_workspace(int64_t heads, int64_t n, int64_t c);
int a2ats_assign_cosine(const void* x, int x_dtype, int64_t heads, int64_t n, int64_t d,
                        const void* query, int64_t nq, const float* codebook, int64_t c,
                        double beta, uint16_t* codes, void* workspace, size_t workspace_bytes,
                        void* stream);

/* ---------------------------------------------------------------------------------------
 * merge_codes -- the last step of the encode pipeline in "A2ATS-adapted -- Windowed RoPE +
 * Query-Aware Retrieval VQ", How it works: every key first takes its plain code, and the
 * keys of the retrieval set then take the query-aware (H-weighted or blended) code.  With
 * both passes run over separate code arrays (so that they can run at the same time), this
 * writes the second array's codes at the retrieval indices into the first:
 *     codes[h, idx[h, i]] = src[h, idx[h, i]]   for i < n_idx
 *
 *   src    [heads, n]      uint16 codes of the query-aware pass (only the listed rows read)
 *   idx    [heads, n_idx]  int32 row indices; entries outside [0, n) are skipped
 *   codes  [heads, n]      uint16, updated in place at the listed rows only
 * Requires 0 <= n_idx <= n <= 2^31 - 1; src and codes may be the same array (no change).
 * Returns without waiting.
 */
int a2ats_merge_codes(const uint16_t* src, const int32_t* idx, int64_t heads, int64_t n,
                      int64_t n_idx, uint16_t* codes, void* stream);

/* ---------------------------------------------------------------------------------------
 * select_retrieval -- "veloxquant_mlx.quantizers.a2ats module", a2ats_select_retrieval_set:
 * per head, the n_r = a2ats_retrieval_count(n, fraction) keys with the largest cosine to
 * the query form the retrieval set, the other n - n_r the bulk.  Equal scores keep the
 * lower index first.  Both outputs are ascending and together cover 0..n-1 exactly once.
 * A zero-norm key scores 0.  The ranking score is k.q / ||k|| in fp32 (||q|| is a per-head
 * constant and does not change the order).
 *
 *   keys           [heads, n, d] fp32 or bf16; d must be 128
 *   query          [heads, d]    same dtype as keys (the proxy query)
 *   retrieval_idx  [heads, n_r]      int32 output
 *   bulk_idx       [heads, n - n_r]  int32 output
 * Requires n <= 2^31 - 1.
 */
size_t a2ats_select_retrieval_workspace(int64_t heads, int64_t n);
int a2ats_select_retrieval(const void* keys, int keys_dtype, int64_t heads, int64_t n,
                           int64_t d, const void* query, double fraction,
                           int32_t* retrieval_idx, int32_t* bulk_idx, void* workspace,
                           size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * reconstruct -- "A2ATS-adapted -- Windowed RoPE + Query-Aware Retrieval VQ", How it works
 * steps 3-4, with the far-token rule of the "paper fidelity" section (Eq. 11-12):
 *   x = codebook[h, codes[b, h, t]]                      (the pre-RoPE key)
 *   near  <=>  0 <= cur_pos - positions[b, t] < window:  RoPE(x, positions[b, t])
 *   far, A2ATS_FAR_FIXED_OFFSET:                          RoPE(x, cur_pos - far_offset)
 *   far, A2ATS_FAR_UNROTATED:                             x
 * RoPE rotates the half-split pairs (i, i + d/2) by pos * rope_base^(-2i/d); angles, sines
 * and the rotation are evaluated in fp64 and rounded once to out_dtype.
 * window <= 0 makes every token far; window > cur_pos makes every valid token near.
 *
 *   codes      [batch, heads, n] uint16
 *   positions  [batch, n]        int32 absolute positions, shared by the heads
 *   codebook   [heads, c, d]     fp32; d must be 128
 *   out        [batch, heads, n, d]  fp32 or bf16 (out_dtype)
 * A token whose code is >= c or whose position is negative gets a row of NaN.
 * Requires cur_pos >= 0 and rope_base > 0.
 */
/* Workspace: a2ats_reconstruct_workspace(heads, c, d, cur_pos, window, out_dtype) bytes: the
 * rope table and, for the far tokens (which all share one rotation), every centroid's far row
 * rotated and rounded once, which far tokens copy (the same values, bit for bit). */
size_t a2ats_reconstruct_workspace(int64_t heads, int64_t c, int64_t d, int64_t cur_pos,
                                   int64_t window, int out_dtype);
int a2ats_reconstruct(const uint16_t* codes, const int32_t* positions, int64_t batch,
                      int64_t heads, int64_t n, int64_t d, const float* codebook, int64_t c,
                      int64_t cur_pos, int64_t window, int64_t far_offset, int far_mode,
                      double rope_base, void* out, int out_dtype, void* workspace,
                      size_t workspace_bytes, void* stream);

/* reconstruct_noalloc -- a2ats_reconstruct for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * arguments, results and arithmetic are those of a2ats_reconstruct (same kernels); instead
 * of a caller workspace the rope table lives in a fixed device array of the library,
 * A2ATS_NOALLOC_TABLE_ROWS rows, one per GPU the library runs on, held until the process
 * ends.  The call allocates nothing.  Requires min(max(window, 0), cur_pos + 1) + 1 <=
 * A2ATS_NOALLOC_TABLE_ROWS (windows up to 8191 tokens), else returns A2ATS_ESCRATCH before
 * launching anything.  The array belongs to the device that is current when the call is made
 * (the device of `stream`); its address is looked up on that device's first call.  Every call
 * on one GPU uses the same array: calls whose work overlaps on one GPU (concurrent streams,
 * or host threads sharing a device) race on it and must be ordered by the caller.
 */
#define A2ATS_NOALLOC_TABLE_ROWS 8192
int a2ats_reconstruct_noalloc(const uint16_t* codes, const int32_t* positions, int64_t batch,
                              int64_t heads, int64_t n, int64_t d, const float* codebook,
                              int64_t c, int64_t cur_pos, int64_t window, int64_t far_offset,
                              int far_mode, double rope_base, void* out, int out_dtype,
                              void* stream);

/* reconstruct_update -- the decode-time use of far keys left unrotated ("A2ATS-adapted"
 * docs, "paper fidelity" section, Eq. 12: far keys are returned as the centroid itself).  With
 * A2ATS_FAR_UNROTATED a row depends on cur_pos only through the token's near/far status, so
 * advancing the decode position rewrites only the tokens that crossed the window edge:
 * given `out` holding a2ats_reconstruct(..., cur_prev, window, A2ATS_FAR_UNROTATED) of the
 * first n_prev tokens (same codes, positions, codebook and rope_base), this call makes `out`
 * equal, bit for bit, to a2ats_reconstruct(..., cur_pos, window, A2ATS_FAR_UNROTATED) of all
 * n tokens.  It writes exactly the rows of tokens t >= n_prev (appended since) and of tokens
 * t < n_prev with positions[b, t] >= 0 whose status (0 <= cur - pos < window) differs
 * between cur_prev and cur_pos; every other row is left untouched.  Arguments as for
 * a2ats_reconstruct; requires 0 <= n_prev <= n, cur_prev >= 0, cur_pos >= 0.  No workspace.
 * The far keys' position (R_b) then belongs on the query: see a2ats_far_query_rope.
 */
int a2ats_reconstruct_update(const uint16_t* codes, const int32_t* positions, int64_t batch,
                             int64_t heads, int64_t n, int64_t d, const float* codebook,
                             int64_t c, int64_t n_prev, int64_t cur_prev, int64_t cur_pos,
                             int64_t window, double rope_base, void* out, int out_dtype,
                             void* stream);

/* far_query_rope -- the query-side half of Eq. 11 ("A2ATS-adapted" docs, "paper fidelity"
 * section; a2ats_apply_far_query_rope of the changelog entry "A2ATS-adapted paper-fidelity
 * fixes"): every row of q is rotated as a token at position far_offset (= b), so that
 * (q R_b) . k is the far-token logit against keys left unrotated.  With the same far_offset,
 * RoPE(q, cur) . RoPE(k, cur - b) = RoPE(q, b) . k, which is what A2ATS_FAR_FIXED_OFFSET
 * bakes into the keys instead.  Same pairs (i, i + d/2) and frequencies as reconstruct;
 * rotation in fp64, one rounding to out_dtype.
 *
 *   q    [rows, d]  fp32 or bf16 (q_dtype), d must be 128
 *   out  [rows, d]  fp32 or bf16 (out_dtype); may be q itself when the dtypes agree, and may
 *                   not overlap q otherwise (A2ATS_EINVAL)
 */
int a2ats_far_query_rope(const void* q, int q_dtype, int64_t rows, int64_t d, int64_t far_offset,
                         double rope_base, void* out, int out_dtype, void* stream);

/* ---------------------------------------------------------------------------------------
 * Sub-vector (product) VQ -- the pages' default configuration ("A2ATS-adapted" docs,
 * "Configuration reference" and "What you get with the defaults"; the calibration example in
 * "How it works" trains one codebook on the pooled sub-vectors of every head).  A head vector
 * of d = 128 numbers is cut into d / sub_dim sub-vectors, each coded by one byte against a
 * single shared codebook [k, sub_dim] (k = 2^bits <= 256).  sub_dim is 4 or 8 (the table's
 * rows).
 *
 * pq_encode: for every selected row of x [heads, n, d] (idx as for a2ats_encode) and every
 * sub-space s, codes[h, row, s] (uint8, [heads, n, d / sub_dim]) =
 *   chol != NULL   argmin_j (x_s - c_j) H (x_s - c_j)^T, H = L L^T, chol = L [sub_dim,
 *                  sub_dim] fp32 lower-triangular (one H for every sub-space, from the
 *                  query sub-vectors: a2ats_calibrate with d = sub_dim on the queries viewed
 *                  as [m * d / sub_dim, sub_dim])     -- a2ats_h_weighted_assignment
 *   chol == NULL, query != NULL
 *                  argmax_j beta (-e_j / max_i e_i) + (1 - beta) cos(q_s, c_j), q_s the same
 *                  slice of query [heads, nq, d] (nq 1 or n, dtype of x), rules as for
 *                  a2ats_assign_cosine            -- a2ats_query_aware_assignment
 *   both NULL      argmin_j ||x_s - c_j||^2 (bulk rows; values)
 * Ties go to the lowest index; the decision is exact: fp16 matrix-core scores (table split
 * hi + lo) folded per accumulator slot, the winning slot rescored in fp64 and accepted under
 * a proven error bound, the rare rest decided in fp64 over the whole table (the blend the
 * same way, its maximum error from a first pass).  A sub-vector with a non-finite element
 * gets code 0 (all its distances are inf or NaN).  No workspace; returns without waiting.
 */
int a2ats_pq_encode(const void* x, int x_dtype, int64_t heads, int64_t n, int64_t d,
                    int64_t sub_dim, const int32_t* idx, int64_t n_idx, const float* codebook,
                    int64_t k, const float* chol, const void* query, int64_t nq, double beta,
                    uint8_t* codes, void* stream);

/* pq_reconstruct: as a2ats_reconstruct, with x = the concatenation of the token's sub-centroids
 * codebook[codes[b, h, t, s]] (codes uint8 [batch, heads, n, d / sub_dim]).  The value path of
 * the pages (values are never rotated) is this call with window <= 0 and A2ATS_FAR_UNROTATED:
 * a plain gather.  A token with any code >= k, or a negative position, gets a row of NaN.
 * Workspace: a2ats_pq_reconstruct_workspace(d, cur_pos, window) bytes.
 */
size_t a2ats_pq_reconstruct_workspace(int64_t d, int64_t cur_pos, int64_t window);
int a2ats_pq_reconstruct(const uint8_t* codes, const int32_t* positions, int64_t batch,
                         int64_t heads, int64_t n, int64_t d, int64_t sub_dim,
                         const float* codebook, int64_t k, int64_t cur_pos, int64_t window,
                         int64_t far_offset, int far_mode, double rope_base, void* out,
                         int out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/* pq_accounting (host only): what the settings alone decide ("What you get with the
 * defaults"): bits / sub_dim bits per number, 16 / that as the ratio against fp16, a table of
 * 2^bits x sub_dim fp16 entries; for `tokens` tokens of `heads` heads, the packed code bytes
 * and the fp16 bytes of the same keys.  Any output pointer may be NULL.  Returns A2ATS_EINVAL
 * unless d % sub_dim == 0 and 1 <= bits <= 16.
 */
int a2ats_pq_accounting(int64_t tokens, int64_t heads, int64_t d, int64_t sub_dim, int bits,
                        double* bits_per_number, double* ratio_vs_fp16, int64_t* table_bytes,
                        int64_t* compressed_bytes, int64_t* fp16_bytes);

/* ---------------------------------------------------------------------------------------
 * Codebook training -- "veloxquant_mlx.quantizers.a2ats module", a2ats_cholesky_factor:
 * Eq. 16-18 map the H-weighted objective to plain k-means on z = xL.  The z-space update
 * (the cluster mean of z) mapped back through L^-1 is the cluster mean of x, so Lloyd's
 * iteration here alternates the exact H-weighted (or plain) assignment with the member mean.
 *
 * kmeans_update: codebook_out[h, j] = fp64 mean of the rows x[h, r] with codes[h, r] == j,
 * rounded once to fp32; a code with no member keeps codebook_in[h, j]; codes >= k are
 * ignored.  counts (optional) [heads, k] int32 receives the cluster sizes.
 *   x         [heads, n, d] fp32 or bf16, d in {4, 8, 16, 32, 64, 128}
 *   codes     [heads, n] uint16 (codes_bytes 2) or uint8 (codes_bytes 1, k <= 256)
 *   codebook  [heads, k] x d fp32, 1 <= k <= 4096; codebook_out may be codebook_in
 * Deterministic: the members are grouped by a stable sort and summed in a fixed order (no
 * floating-point atomics).  Workspace: a2ats_kmeans_update_workspace(heads, n, k) bytes.
 */
size_t a2ats_kmeans_update_workspace(int64_t heads, int64_t n, int64_t k);
int a2ats_kmeans_update(const void* x, int x_dtype, int64_t heads, int64_t n, int64_t d,
                        const void* codes, int codes_bytes, int64_t k, const float* codebook_in,
                        float* codebook_out, int32_t* counts, void* workspace,
                        size_t workspace_bytes, void* stream);

/* kmeans_init: k-means++ seeding in z-space -- the pages' "conventional k-means++" on
 * z = x L (a2ats_cholesky_factor, Eq. 16-18; the docs' calibration trains with a seed).  The
 * random draws are inputs: draws[h, t] uniform over [0, 2^64) for center t of head h.
 *   z_i = x_i L (each component the fp64 sum over b in order of x_ib L_ba, rounded to fp32;
 *         x_i itself when chol is NULL), Z = max_i ||z_i||^2 per head
 *   c_0 = floor(draws[h, 0] n / 2^64)
 *   c_t = the first row whose running sum of w exceeds floor(draws[h, t] W / 2^64), where
 *         w_i = floor(D2_i 2^e), D2_i = min over chosen c of ||z_i - z_c||^2 (fp64, in
 *         dimension order), e = 60 - ceil(log2 n) - ceil(log2 4Z), W = sum of w
 *         (floor(draws[h, t] n / 2^64) when W = 0): each row is drawn with probability
 *         D2 / sum D2, and the integer weights make the choice independent of how the
 *         rows are split over workgroups.
 *   x         [heads, n, d] fp32 or bf16, d in {4, 8, 16, 32, 64, 128}; 1 <= k <= n
 *   chol      [heads, d, d] fp32 lower-triangular L, or NULL (plain k-means++)
 *   draws     [heads, k] uint64 (device)
 *   codebook  [heads, k, d] fp32 output: the chosen rows, in order
 *   idx       [heads, k] int32 output (may be NULL): the chosen row indices
 * Pooled sub-vectors (one shared codebook) are heads = 1 with x viewed as [1, n, sub_dim].
 * One launch per center; returns without waiting.  Workspace:
 * a2ats_kmeans_init_workspace(heads, n, d, k) bytes.
 */
size_t a2ats_kmeans_init_workspace(int64_t heads, int64_t n, int64_t d, int64_t k);
int a2ats_kmeans_init(const void* x, int x_dtype, int64_t heads, int64_t n, int64_t d,
                      int64_t k, const float* chol, const uint64_t* draws, float* codebook,
                      int32_t* idx, void* workspace, size_t workspace_bytes, void* stream);

/* kmeans: `iters` Lloyd rounds on the device from the initial codebook (updated in place),
 * then the final assignment into codes.  chol (optional) is L for the H-weighted assignment.
 *   d = 128   x [heads, n, 128], per-head codebooks [heads, k, 128] and L [heads, 128, 128]
 *             (a2ats_encode); codes uint16 [heads, n]
 *   d = 4, 8  one codebook [k, d] (k <= 256) over the pooled sub-vectors x [n, d] (heads must
 *             be 1, n a multiple of 128 / d), L [d, d] (a2ats_pq_encode); codes uint8 [n] --
 *             the pages' calibration trains this codebook on the keys viewed as [-1, sub_dim]
 * Workspace: a2ats_kmeans_workspace(heads, n, d, k) bytes.  Returns without waiting.
 */
size_t a2ats_kmeans_workspace(int64_t heads, int64_t n, int64_t d, int64_t k);
int a2ats_kmeans(const void* x, int x_dtype, int64_t heads, int64_t n, int64_t d, int64_t k,
                 const float* chol, int iters, float* codebook, void* codes, void* workspace,
                 size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * Approximate attention-score top-K over codes -- the A2ATS paper page ("Abstract (arXiv)")
 * retrieves the tokens with the top-K attention scores approximated from the quantised keys.
 * With far keys unrotated, the far logit of token t is (q R_b) . c_{code_t} ("A2ATS-adapted"
 * docs, "paper fidelity" section, Eq. 11-12), so one table of C values per query, gathered by
 * code, scores every token.
 *
 * topk_codes: for every sequence b and query head h (key/value head h / (hq / hkv)):
 *   lut_j     = fp32( sum_a qb[b, h, a] * codebook[kvh, j, a] ), the products formed in fp64
 *               and added in dimension order, rounded to fp32 once
 *   score_t   = lut[codes[b, kvh, t]], or -inf for a code >= c
 *   idx[b, h] = the k tokens with the largest scores (equal scores: lower index first; -0 and
 *               +0 are equal), in ascending index order; score[b, h] (optional) their scores
 *   qb        [batch, hq, d] fp32 or bf16 (q_dtype), 16-byte aligned: the query already
 *               rotated by R_b (a2ats_far_query_rope)
 *   codes     [batch, hkv, n] uint16; codebook [hkv, c, d] fp32, 1 <= c <= 4096, d = 128
 *   idx       [batch, hq, k] int32; score [batch, hq, k] fp32 or NULL; 0 <= k <= n
 * hq must be a multiple of hkv and batch * hq < 2^31.  Nothing is written when n or k is 0.
 * Two launches: every query's table into the workspace (fp64 matrix cores, whose fma-chain
 * accumulation in k order gives the dimension-ordered sum exactly), then one workgroup per
 * code row and up to four query heads of a group: their tables in LDS, the K-th largest
 * score by passes of monotone 1024-bin histograms over the C + 1 table entries weighted by
 * their token counts, then the taken tokens in token order.  Workspace:
 * a2ats_topk_workspace(batch, hq, c) bytes (256-byte aligned), A2ATS_EWORKSPACE when missing
 * or short; A2ATS_EINVAL for misaligned queries.  Returns without waiting.
 */
size_t a2ats_topk_workspace(int64_t batch, int64_t hq, int64_t c);
int a2ats_topk_codes(const void* qb, int q_dtype, int64_t batch, int64_t hq, int64_t hkv,
                     int64_t d, const uint16_t* codes, int64_t n, const float* codebook,
                     int64_t c, int64_t k, int32_t* idx, float* score, void* workspace,
                     size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * Kernel timing (diagnostics).  While enabled, every kernel the library launches is
 * bracketed by HIP events recorded on its stream.  a2ats_profile_read waits for those
 * events and writes one line per kernel name, "name<TAB>launches<TAB>total_ms\n", into
 * buf (NUL-terminated, truncated to len); it returns the number of bytes needed.
 * Not thread-safe; intended for benchmarks.
 */
int a2ats_profile_enable(int on);
int a2ats_profile_reset(void);
int64_t a2ats_profile_read(char* buf, size_t len);

#ifdef __cplusplus
}
#endif
#endif /* A2ATS_H */
