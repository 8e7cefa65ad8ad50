/*
 * tq.h -- C ABI of libtq, the TurboQuant online vector quantiser for AMD
 * Instinct MI355X (gfx950).
 *
 * What the calls compute (sources are cited by title and section):
 *   "TurboQuant: Online Vector Quantization" paper summary (Jump2Paper
 *   Archive, arXiv 2504.19874) -- definitions table: a quantiser
 *   Q : R^d -> {0,1}^(b*d) with a dequantiser Q^-1; Lemma 1 (the Beta-type
 *   marginal of a rotated unit vector); the MSE decomposition into a 1-D
 *   k-means problem solved by Lloyd-Max; Definition 1 (QJL map sign(S x))
 *   and its dequantiser sqrt(pi/2)/d * S^T z (Lemma 4); Theorem D_prod
 *   (TurboQuant_prod = (b-1)-bit TurboQuant_mse + 1-bit QJL of the residual,
 *   unbiased inner products).
 *   AI Trends summary of the TurboQuant video -- chapter 04:24 (L2 normalise,
 *   then multiply by the randomised Hadamard matrix), 06:06 (quantise in the
 *   rotated domain; undo by the transpose and the stored norm).
 *
 * Conventions used by every call
 *   - d is the padded dimension: a power of two with 32 <= d <= 4096.
 *     Inputs have d_in <= d coordinates and are zero-padded to d.
 *   - The rotation is Pi = (1/sqrt d) * H * diag(signs), H the natural-order
 *     Sylvester Hadamard matrix (H[i][j] = (-1)^popcount(i & j)).
 *   - A vector x is stored as its norm n = ||x||_2 (float32) and the code of
 *     y = Pi (x / n) (y = 0 when n = 0).
 *   - Scalar code, m bits per coordinate: with K = 2^m and L the number of
 *     positive thresholds t with |y_j| >= t, idx_j = K/2 + L if y_j >= 0 and
 *     K/2 - 1 - L otherwise (nearest centroid; exact ties go to the centroid
 *     of larger magnitude; y_j = 0 goes to the positive side).  Decided in
 *     float32.
 *   - Record layout ("codes"): per vector m*d/8 bytes, dense m-bit codes:
 *     idx_j occupies bits [m*j, m*j + m) of a little-endian bit stream (bit s
 *     is bit s%8 of byte s/8; bit p of idx_j is stream bit m*j + p).
 *     Vector v's record starts at codes + v * m*d/8.
 *   - QJL plane ("qjl", TurboQuant_prod only): per vector d/8 bytes, bit i at
 *     stream position i equals [(S r)_i >= 0] where r = y - c[idx] is the
 *     residual in the rotated domain; "rnorms" holds gamma = ||r||_2.
 *     Dequantised residual: gamma * sqrt(pi/2)/d * S^T z with z_i = 2 bit - 1.
 *   - Pointers are device pointers unless marked [host].  All buffers are
 *     owned by the caller; the library never allocates, frees or keeps
 *     memory.  Calls are stateless and re-entrant; kernels are launched
 *     asynchronously on `stream` (a hipStream_t, NULL = default stream) and
 *     their outputs are valid once the caller synchronises that stream.
 *   - Arguments are checked before any launch; on error nothing is launched
 *     and nothing is written.  n = 0 is a no-op returning TQ_OK.  No
 *     exception or abort crosses this interface.
 *   - Non-finite input: a row whose float32 sum of squares is not finite (it
 *     holds a NaN or an infinity, or its squares overflow float32) is
 *     encoded exactly as the zero row (every code idx = 2^m / 2, the code of
 *     y = 0; for TurboQuant_prod the zero row's QJL plane and gamma) and its
 *     norm is stored as NaN, so it decodes to NaN and scores NaN (top-k never
 *     selects it).  The other rows are unaffected.  Queries are not checked.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TQ_VERSION 2

typedef enum {
  TQ_OK = 0,
  TQ_ERR_ARG = -1,       /* NULL required pointer, negative count, bad enum,
                            unsupported combination */
  TQ_ERR_DIM = -2,       /* d not a power of two in [32, 4096], or d_in outside [1, d] */
  TQ_ERR_BITS = -3,      /* m outside the range the call accepts */
  TQ_ERR_ALIGN = -4,     /* a pointer not aligned as documented, or a row stride too small */
  TQ_ERR_WORKSPACE = -5, /* workspace NULL or smaller than tq_score_workspace() */
  TQ_ERR_HIP = -6,       /* the HIP runtime reported an error at launch */
  TQ_ERR_NOCONV = -7     /* tq_make_codebook did not converge */
} tq_status;

typedef enum { TQ_F32 = 0, TQ_F16 = 1, TQ_BF16 = 2 } tq_dtype;
typedef enum { TQ_MSE = 0, TQ_PROD = 1 } tq_mode;

/* The random rotation Pi applied to x / ||x|| before quantisation.
 *   TQ_ROT_RHT: Pi = (1/sqrt d) H diag(signs) (the default; see above).
 *   TQ_ROT_GIVENS: block diagonal, one 2-D Givens rotation per coordinate
 *     pair (2i, 2i+1): (v0, v1) -> (c v0 - s v1, s v0 + c v1).
 *   TQ_ROT_QUAT: block diagonal, one unit quaternion p = (w, x, y, z) per
 *     coordinate quad 4i..4i+3, applied as the left product p * v of the quad
 *     read as a quaternion (v0 + v1 i + v2 j + v3 k).
 * The block-diagonal variants are the 2-D Givens / 4-D quaternion rotations
 * the RotorQuant forum post describes as cheaper than the Hadamard
 * butterflies; they keep the same Lemma 1 codebook.  Pi^-1 = Pi^T in every
 * case.  Block rotations are supported for d = d_in = 128 by the encode,
 * decode, score, top-k and rotation calls (not by tq_attend). */
typedef enum { TQ_ROT_RHT = 0, TQ_ROT_GIVENS = 1, TQ_ROT_QUAT = 2 } tq_rotation;

/* Parameters of one quantiser.  The random parameters (signs, S) are inputs
 * drawn by the caller; the codebook comes from tq_make_codebook rounded to
 * float32. */
typedef struct {
  int32_t d_in;              /* input dimension, 1 <= d_in <= d */
  int32_t d;                 /* padded dimension, power of two, 32..4096 */
  int32_t m;                 /* bits of the scalar code per coordinate:
                                TurboQuant_mse with b bits: m = b (1..8);
                                TurboQuant_prod with b bits: m = b - 1 (0..7,
                                0 = pure QJL) */
  int32_t rotation;          /* tq_rotation; TQ_ROT_RHT unless stated */
  const float *centroids;    /* [2^m] ascending, exactly odd-symmetric; NULL if m == 0 */
  const float *thresholds;   /* [2^m - 1] midpoints, thresholds[2^(m-1) - 1] == 0; NULL if m == 0 */
  const int8_t *signs;       /* [d] entries -1 or +1: the RHT diagonal
                                (TQ_ROT_RHT only) */
  const uint16_t *qjl_s;     /* [d][d] bfloat16 bit patterns, row-major: the QJL
                                matrix S (i.i.d. N(0,1) draws rounded to bfloat16);
                                required by TQ_PROD calls, ignored otherwise.
                                Entries must be finite with |S_ij| <= 65504: the
                                d = 128 encoder multiplies in float16, where
                                entries below 2^-14 in magnitude keep only the
                                bits down to 2^-24 (rounded toward zero), which
                                moves (S r)_i by at most 2^-24 sum_j |r_j| <=
                                2^-24 sqrt(d) gamma; every other path uses S as
                                given */
  const float *rot;          /* block rotation parameters, 16-byte aligned:
                                TQ_ROT_GIVENS [d/2][2] (cos, sin) of pair i;
                                TQ_ROT_QUAT [d/4][4] unit quaternion (w, x, y, z)
                                of quad i; ignored for TQ_ROT_RHT */
} tq_params;

/* One batch of encoded vectors (structure of arrays). */
typedef struct {
  uint8_t *codes;            /* [n][m*d/8], 4-byte aligned; NULL allowed when m == 0 */
  uint8_t *qjl;              /* [n][d/8], 4-byte aligned (TQ_PROD), else ignored */
  float *norms;              /* [n] ||x||_2 */
  float *rnorms;             /* [n] gamma = ||r||_2 (TQ_PROD), else ignored */
} tq_codes;

/* Lloyd-Max codebook of 2^m levels for the Lemma 1 density at dimension d
 * (setup table: codebooks precomputed for b = 1..8 by numerical Max-Lloyd;
 * MSE decomposition: D_mse = d * C(f_X, b)).  Runs on the host in float64:
 * Lloyd iterations to a near fixed point, then Newton steps on the
 * optimality conditions.  Output is exactly odd-symmetric.
 *   d: 3..65536 (any integer; the kernels use the padded power of two)
 *   m: 1..8
 *   centroids  [host] out, 2^m values ascending
 *   thresholds [host] out, 2^m - 1 midpoints
 *   dmse       [host] out, nullable: d * sum_k int (x - c_k)^2 f_X
 * Returns TQ_OK, TQ_ERR_ARG, TQ_ERR_DIM, TQ_ERR_BITS or TQ_ERR_NOCONV. */
int tq_make_codebook(int32_t d, int32_t m, double *centroids, double *thresholds,
                     double *dmse);

/* TurboQuant_mse encode (the mse variant of the paper summary): for each row
 * of x, n = ||x||, y = Pi (x/n), idx = bucket(y), packed into out->codes;
 * out->norms = n.
 *   p: m in 1..8; centroids, thresholds, signs required
 *   x: [n][ld_x] elements of `dtype`, first d_in used; 16-byte aligned
 *   ld_x: row stride in elements, >= d_in (block rotations: also <= 2^24,
 *         else TQ_ERR_ALIGN)
 *   out: codes and norms required
 * Returns TQ_OK, TQ_ERR_ARG, TQ_ERR_DIM, TQ_ERR_BITS, TQ_ERR_ALIGN or TQ_ERR_HIP. */
int tq_encode_mse(const tq_params *p, const void *x, int32_t dtype, int64_t ld_x, int64_t n,
                  const tq_codes *out, void *stream);

/* TurboQuant_prod encode (Theorem D_prod): the m-bit mse code of y as above
 * (m = b - 1, may be 0), then r = y - c[idx], gamma = ||r||, and the QJL
 * plane sign(S r) (Definition 1 applied to the residual in the rotated
 * domain; sign(0) = +1).
 *   p: m in 0..7; signs and qjl_s required, codebook required when m > 0
 *   out: qjl, norms and rnorms required; codes required when m > 0
 * Returns as tq_encode_mse. */
int tq_encode_prod(const tq_params *p, const void *x, int32_t dtype, int64_t ld_x, int64_t n,
                   const tq_codes *out, void *stream);

/* Dequantise (Q^-1): y~ = c[idx] (+ gamma * sqrt(pi/2)/d * S^T z for
 * TQ_PROD), x~ = n * Pi^T y~, first d_in coordinates written.
 *   mode: TQ_MSE (m in 1..8) or TQ_PROD (m in 0..7)
 *   in: the arrays written by the matching encode call
 *   out: [n][ld_out] float32, 16-byte aligned, ld_out >= d_in
 * Returns TQ_OK, TQ_ERR_ARG, TQ_ERR_DIM, TQ_ERR_BITS, TQ_ERR_ALIGN or TQ_ERR_HIP. */
int tq_decode(const tq_params *p, int32_t mode, const tq_codes *in, int64_t n, float *out,
              int64_t ld_out, void *stream);

/* Bytes of device workspace tq_score needs for nq queries: the rotated
 * queries and, for TQ_PROD, S times them; for TQ_MSE, their float16 split
 * and per-row scales (used when 16 or more queries per group go to the
 * matrix cores).  0 on bad arguments. */
size_t tq_score_workspace(const tq_params *p, int32_t mode, int64_t nq);

/* Inner-product estimates <q, Q^-1(Q(x))> of every query with every key,
 * computed from the packed codes without decoding:
 *   est = n * ( sum_j q'_j c[idx_j] + gamma * sqrt(pi/2)/d * sum_i (S q')_i z_i )
 * with q' = Pi q (the query is rotated once instead of un-rotating keys).
 *   q: [nq][ldq] float32, ldq >= d_in
 *   keys: codes and norms (+ qjl, rnorms for TQ_PROD) of n keys
 *   scores: [nq][ld_scores] float32, ld_scores >= n; scores[i*ld_scores + k]
 *   workspace: device, >= tq_score_workspace(p, mode, nq) bytes, 256-byte
 *              aligned; scratch for the rotated queries (at d = 128 with
 *              1..4 code bits the kernels keep them on chip and leave it
 *              untouched)
 * Returns TQ_OK, TQ_ERR_ARG, TQ_ERR_DIM, TQ_ERR_BITS, TQ_ERR_ALIGN,
 * TQ_ERR_WORKSPACE or TQ_ERR_HIP. */
int tq_score(const tq_params *p, int32_t mode, const float *q, int64_t ldq, int64_t nq,
             const tq_codes *keys, int64_t n, float *scores, int64_t ld_scores,
             void *workspace, size_t ws_bytes, void *stream);

/* Grouped form of tq_score for attention-style layouts (grouped-query
 * attention: each KV head's keys scored only against its own query heads).
 * Queries are `groups` consecutive blocks of nq_per_group rows, keys are
 * `groups` consecutive blocks of n_per_group records; query row
 * g*nq_per_group + i is scored against keys g*n_per_group .. + n_per_group - 1
 * into scores[(g*nq_per_group + i)*ld_scores + k], k < n_per_group.
 * groups * nq_per_group <= 65535; workspace as tq_score_workspace(p, mode,
 * groups * nq_per_group).  tq_score(..., nq, keys, n, ...) is this call with
 * groups = 1.  Returns as tq_score. */
int tq_score_grouped(const tq_params *p, int32_t mode, const float *q, int64_t ldq, int64_t groups,
                     int64_t nq_per_group, const tq_codes *keys, int64_t n_per_group, float *scores,
                     int64_t ld_scores, void *workspace, size_t ws_bytes, void *stream);

/* As tq_score_grouped, but adds each estimate to what `scores` holds
 * instead of overwriting it.
 *
 * This serves the outlier-channel split of the paper summary's KV-cache
 * experiments (a set of high-variance channels quantised at more bits than
 * the rest, each set by its own TurboQuant instance): store the channels of
 * each set contiguously (a fixed channel order, e.g. outliers first), then
 *   encode: one tq_encode_* call per set on the column range
 *           (x + first column, row stride ld_x, its own d_in and d);
 *   decode: one tq_decode per set into the matching output columns;
 *   score:  tq_score_grouped for the first set, tq_score_accumulate for the
 *           others, each on its column range of the queries.
 * The estimate is the sum of the sets' estimates; each set keeps its own
 * norm.  Returns as tq_score_grouped. */
int tq_score_accumulate(const tq_params *p, int32_t mode, const float *q, int64_t ldq, int64_t groups,
                        int64_t nq_per_group, const tq_codes *keys, int64_t n_per_group, float *scores,
                        int64_t ld_scores, void *workspace, size_t ws_bytes, void *stream);

/* Bytes of device workspace tq_topk needs: the score workspace and a score
 * buffer for up to 64 query rows at a time, and the top-k candidate lists of
 * the segments the rows are cut into; for the filtered search (below) also
 * the query set-up of up to 1,024 queries, their estimates of a 16,384-key
 * sample and a 4,096-entry candidate list each.  0 on bad arguments. */
size_t tq_topk_workspace(const tq_params *p, int32_t mode, int64_t nq, int64_t n, int32_t k);

/* Nearest-neighbour search on quantised keys (the search application of the
 * paper summary): for each query, the k keys with the largest estimate
 * <q, Q^-1(Q(x))> (as tq_score), best first; equal estimates are ordered by
 * smaller key index, NaN estimates are never selected.
 *   q: [nq][ldq] float32; keys: n records (n < 2^31)
 *   k: 1..32
 *   idx: [nq][k] int64, 8-byte aligned; vals: [nq][k] float32 estimates.
 *   When n < k the tail of a row is idx -1, value -inf.
 *   workspace: device, >= tq_topk_workspace(p, mode, nq, n, k) bytes,
 *   256-byte aligned.
 * With 16 or more TurboQuant_mse queries (1..4 code bits, d >= 128) and at
 * least 2^17 keys the search is filtered: the estimates of an evenly spread
 * sample of 16,384 keys give tau, the k-th largest of them (at most the k-th
 * largest over all keys); the full pass keeps only estimates >= tau, no score
 * matrix is written, and a query whose candidates exceed 4,096 takes the
 * full score row instead.  The result is the same either way.
 * Returns TQ_OK, TQ_ERR_ARG, TQ_ERR_DIM, TQ_ERR_BITS, TQ_ERR_ALIGN,
 * TQ_ERR_WORKSPACE or TQ_ERR_HIP. */
int tq_topk(const tq_params *p, int32_t mode, const float *q, int64_t ldq, int64_t nq, const tq_codes *keys,
            int64_t n, int32_t k, int64_t *idx, float *vals, void *workspace, size_t ws_bytes, void *stream);

/* Bytes of device workspace tq_attend needs: the per-chunk partial softmax
 * sums (132 floats per query row and chunk of 256 tokens).  0 on bad
 * arguments (the keys' d must be 128). */
size_t tq_attend_workspace(const tq_params *pk, int32_t kmode, int64_t groups, int64_t nq_per_group,
                           int64_t n_per_group);

/* Decode attention on quantised keys and values (PolarQuant paper review,
 * step 9: the reconstructed K^ and V^ enter softmax(K^ q / sqrt d) V^).  For
 * query row g*nq_per_group + i, against the n_per_group tokens of KV group g
 * (grouped-query attention):
 *   s_t = scale * <q, Q^-1(key_t)>  (the tq_score estimate),
 *   out = sum_t softmax(s)_t * Q^-1(value_t),
 * computed without materialising K^ or V^: the values are summed in the
 * rotated domain and rotated back once per query row.
 *   pk, kmode: key quantiser; TQ_MSE with m 1..4 or TQ_PROD with m 0..3
 *   keys: codes/norms (+ qjl/rnorms for TQ_PROD) of groups*n_per_group keys
 *   pv, values: TurboQuant_mse value quantiser (m 1..4) and records
 *   Both quantisers need d = 128 and the same d_in (their rotations may
 *   differ).
 *   q: [groups*nq_per_group][ldq] float32, ldq >= d_in
 *   scale: multiplies the estimates before the softmax (1/sqrt(d) for
 *          standard scaled attention)
 *   out: [groups*nq_per_group][ld_out] float32, first d_in written
 *   workspace: device, >= tq_attend_workspace(...) bytes, 256-byte aligned
 *   groups * ceil(nq_per_group / 4) <= 65535.  n_per_group = 0 (or no
 *   queries) is a no-op that writes nothing.
 * Returns TQ_OK, TQ_ERR_ARG, TQ_ERR_DIM, TQ_ERR_BITS, TQ_ERR_ALIGN,
 * TQ_ERR_WORKSPACE or TQ_ERR_HIP. */
int tq_attend(const tq_params *pk, int32_t kmode, const tq_codes *keys, const tq_params *pv,
              const tq_codes *values, const float *q, int64_t ldq, int64_t groups, int64_t nq_per_group,
              int64_t n_per_group, float scale, float *out, int64_t ld_out, void *workspace,
              size_t ws_bytes, void *stream);

/* tq_attend without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops that must not
 * call hipMalloc, harnesses that forbid it).  Same arguments, checks and
 * results as tq_attend; the per-chunk partials go to a fixed 16 MiB device
 * array inside the library instead (one per GPU, looked up on the first call
 * on that device with it current, and held until the process ends).  The
 * call allocates nothing.  Limit: tq_attend_workspace(pk, kmode, groups,
 * nq_per_group, n_per_group) <= 16 MiB (e.g. 32 query rows over 32,768
 * tokens per group need 2.1 MiB), else TQ_ERR_WORKSPACE before any launch.
 * Calls on one GPU share the array: calls that overlap in time on that GPU
 * (other streams, other threads) race and must be serialised by the caller;
 * the array keeps the last call's partials (every entry a call reads is
 * written by that call first).  `stream` must belong to the current device.
 * Returns as tq_attend (TQ_ERR_HIP also when the array cannot be found). */
int tq_attend_noalloc(const tq_params *pk, int32_t kmode, const tq_codes *keys, const tq_params *pv,
                      const tq_codes *values, const float *q, int64_t ldq, int64_t groups,
                      int64_t nq_per_group, int64_t n_per_group, float scale, float *out, int64_t ld_out,
                      void *stream);

/* The rotation alone, on float32 rows: out = Pi in_pad (inverse = 0) or
 * out = (Pi^T in)[0:d_in] (inverse != 0).  Forward reads d_in columns and
 * writes d; inverse reads d and writes d_in.
 *   in: [n][ld_in] float32; out: [n][ld_out] float32
 * Returns TQ_OK, TQ_ERR_ARG, TQ_ERR_DIM, TQ_ERR_ALIGN or TQ_ERR_HIP. */
int tq_rht(const tq_params *p, const float *in, int64_t ld_in, float *out, int64_t ld_out,
           int64_t n, int32_t inverse, void *stream);

/* Static description of a status code (never NULL). */
const char *tq_status_string(int32_t status);

/* TQ_VERSION of the built library. */
int32_t tq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
