// C-ABI entry points of libtq: argument checks, then one launch (or two for
// tq_score) on the caller's stream.  Nothing is allocated or kept, except
// the fixed device array behind tq_attend_noalloc (below).

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "tq_internal.h"

using namespace tq;

namespace {

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int log2i(int v) {
  int r = 0;
  while ((1 << r) < v) ++r;
  return r;
}

int check_dims(const tq_params *p) {
  if (!p) return TQ_ERR_ARG;
  if (p->rotation != TQ_ROT_RHT && p->rotation != TQ_ROT_GIVENS && p->rotation != TQ_ROT_QUAT) return TQ_ERR_ARG;
  if (!is_pow2(p->d) || p->d < kMinD || p->d > kMaxD) return TQ_ERR_DIM;
  if (p->d_in < 1 || p->d_in > p->d) return TQ_ERR_DIM;
  return TQ_OK;
}

// The rotation's parameters: RHT signs, or a block rotation's table (only
// for d = d_in = 128).
int check_rotation(const tq_params *p) {
  if (p->rotation == TQ_ROT_RHT) return p->signs ? TQ_OK : TQ_ERR_ARG;
  if (p->d != 128 || p->d_in != 128) return TQ_ERR_DIM;
  if (!p->rot) return TQ_ERR_ARG;
  if (!aligned(p->rot, 16)) return TQ_ERR_ALIGN;
  return TQ_OK;
}

// Common checks of the quantiser parameters for `prod` calls or not.
int check_params(const tq_params *p, bool prod) {
  int st = check_dims(p);
  if (st != TQ_OK) return st;
  if (prod) {
    if (p->m < 0 || p->m > 7) return TQ_ERR_BITS;
    if (!p->qjl_s) return TQ_ERR_ARG;
    if (!aligned(p->qjl_s, 16)) return TQ_ERR_ALIGN;
  } else {
    if (p->m < 1 || p->m > 8) return TQ_ERR_BITS;
  }
  st = check_rotation(p);
  if (st != TQ_OK) return st;
  if (p->m > 0 && (!p->centroids || !p->thresholds)) return TQ_ERR_ARG;
  return TQ_OK;
}

int hip_status(int err) { return err == 0 ? TQ_OK : TQ_ERR_HIP; }

// Rotates the queries into the workspace (and S q' for prod), then scores.
// Where the score kernels prepare their queries themselves (d = 128 with 1..4
// code bits) the workspace is left untouched.
int score_launch(const tq_params *p, bool prod, const float *q, int64_t ldq, int64_t groups, int64_t nq,
                 const tq_codes *keys, int64_t n, float *scores, int64_t ld_scores, void *workspace,
                 size_t need, void *stream, bool accumulate = false);

// Argument checks of tq_score_grouped / tq_score_accumulate, then the launches.
int score_checked(const tq_params *p, int32_t mode, const float *q, int64_t ldq, int64_t groups, int64_t nq,
                  const tq_codes *keys, int64_t n, float *scores, int64_t ld_scores, void *workspace,
                  size_t ws_bytes, void *stream, bool accumulate);

// tq_topk scores at most kTopkChunk query rows at a time into a workspace
// buffer of rows padded to a multiple of 4 floats.
constexpr int64_t kTopkChunk = 64;
constexpr int32_t kTopkMaxK = 32;
int64_t topk_ld(int64_t n) { return (n + 3) & ~int64_t{3}; }
// segment candidate lists: at most max(2048, rows) (value, index) lists of k
size_t topk_cand_bytes(int64_t qc, int32_t k) {
  const int64_t lists = qc > 2048 ? qc : 2048;
  return static_cast<size_t>(lists) * k * (sizeof(float) + sizeof(int32_t));
}
size_t round256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

// Filtered search (TurboQuant_mse keys on the matrix cores, n >= kFuseMinN):
// an evenly spread sample of kSampleBlocks blocks of kScoreMKeys keys is
// scored and its top k taken; the k-th of those estimates, tau, is at most the k-th
// largest estimate over all keys, so every key of the final top k has an
// estimate >= tau.  The full pass then keeps only the estimates >= tau (in a
// list of kListCap per query, no score matrix), and the top k of the list is
// the answer.  A query whose list overflows takes the full score matrix.
constexpr int64_t kFuseMinN = int64_t{1} << 17;
constexpr int64_t kFilterChunk = 1024;        // queries filtered together
constexpr int64_t kSampleBlocks = 32;
constexpr int64_t kSampleCols = kSampleBlocks * kScoreMKeys;
constexpr int32_t kListCap = 4096;
bool topk_filtered(const tq_params *p, bool prod, int64_t qc, int64_t n) {
  return n >= kFuseMinN && score_on_mfma(p->d, p->m, prod, qc);
}
// the filtered search's extra workspace for qf queries: sample scores, the
// sample's top k (index, value), tau, counts and the lists
size_t topk_filter_bytes(int64_t qc, int32_t k) {
  return round256(static_cast<size_t>(qc) * kSampleCols * sizeof(float)) +
         round256(static_cast<size_t>(qc) * k * sizeof(int64_t)) + round256(static_cast<size_t>(qc) * k * sizeof(float)) +
         round256(static_cast<size_t>(qc) * sizeof(float)) + round256(static_cast<size_t>(qc) * sizeof(int32_t)) +
         round256(static_cast<size_t>(qc) * kListCap * sizeof(float)) +
         round256(static_cast<size_t>(qc) * kListCap * sizeof(int32_t));
}

// Rotated, split queries for the matrix-core score kernel in the workspace;
// returns the kernel's arguments with the score matrix fields unset.
int scorem_prepare(const tq_params *p, const float *q, int64_t ldq, int64_t nq, const tq_codes *keys, int64_t n,
                   void *workspace, void *stream, ScoreMArgs &sm);

int encode_common(const tq_params *p, const void *x, int32_t dtype, int64_t ld_x, int64_t n,
                  const tq_codes *out, void *stream, bool prod) {
  int st = check_params(p, prod);
  if (st != TQ_OK) return st;
  if (n < 0 || !out) return TQ_ERR_ARG;
  if (dtype != TQ_F32 && dtype != TQ_F16 && dtype != TQ_BF16) return TQ_ERR_ARG;
  if (n == 0) return TQ_OK;
  if (!x || !out->norms) return TQ_ERR_ARG;
  if (p->m > 0 && !out->codes) return TQ_ERR_ARG;
  if (prod && (!out->qjl || !out->rnorms)) return TQ_ERR_ARG;
  const int esize = dtype == TQ_F32 ? 4 : 2;
  if (!aligned(x, 16)) return TQ_ERR_ALIGN;
  if (ld_x < p->d_in) return TQ_ERR_ALIGN;
  if (p->m > 0 && !aligned(out->codes, 4)) return TQ_ERR_ALIGN;
  if (prod && !aligned(out->qjl, 4)) return TQ_ERR_ALIGN;
  if (!aligned(out->norms, 4) || (prod && !aligned(out->rnorms, 4))) return TQ_ERR_ALIGN;
  EncodeArgs a{};
  a.x = x;
  a.ld_x = ld_x;
  a.n = n;
  a.d_in = p->d_in;
  a.d = p->d;
  a.log_lpv = log2i(p->d / kEPL);
  a.dtype = dtype;
  a.m = p->m;
  a.vec_loads = ((static_cast<int64_t>(p->d_in) * esize) % 16 == 0) && ((ld_x * esize) % 16 == 0);
  if (p->rotation != TQ_ROT_RHT) {
    // block rotations run in the d = 128 kernel only
    if ((prod && p->m > 3) || (!prod && p->m > 4)) return TQ_ERR_BITS;
    if (!a.vec_loads || ld_x > (int64_t(1) << 24)) return TQ_ERR_ALIGN;
  }
  a.rot_kind = p->rotation;
  a.rot = p->rot;
  a.centroids = p->centroids;
  a.thresholds = p->thresholds;
  a.signs = p->signs;
  a.qjl_s = p->qjl_s;
  a.codes = out->codes;
  a.qjl = out->qjl;
  a.norms = out->norms;
  a.rnorms = out->rnorms;
  return hip_status(launch_encode(a, prod, stream));
}

}  // namespace

extern "C" {

int tq_make_codebook(int32_t d, int32_t m, double *centroids, double *thresholds, double *dmse) {
  if (!centroids || !thresholds) return TQ_ERR_ARG;
  if (d < 3 || d > 65536) return TQ_ERR_DIM;
  if (m < 1 || m > 8) return TQ_ERR_BITS;
  try {
    return make_codebook(d, m, centroids, thresholds, dmse);
  } catch (...) {
    return TQ_ERR_NOCONV;
  }
}

int tq_encode_mse(const tq_params *p, const void *x, int32_t dtype, int64_t ld_x, int64_t n,
                  const tq_codes *out, void *stream) {
  return encode_common(p, x, dtype, ld_x, n, out, stream, false);
}

int tq_encode_prod(const tq_params *p, const void *x, int32_t dtype, int64_t ld_x, int64_t n,
                   const tq_codes *out, void *stream) {
  return encode_common(p, x, dtype, ld_x, n, out, stream, true);
}

int tq_decode(const tq_params *p, int32_t mode, const tq_codes *in, int64_t n, float *out,
              int64_t ld_out, void *stream) {
  if (mode != TQ_MSE && mode != TQ_PROD) return TQ_ERR_ARG;
  const bool prod = mode == TQ_PROD;
  int st = check_params(p, prod);
  if (st != TQ_OK) return st;
  if (n < 0 || !in) return TQ_ERR_ARG;
  if (n == 0) return TQ_OK;
  if (!out || !in->norms) return TQ_ERR_ARG;
  if (p->m > 0 && !in->codes) return TQ_ERR_ARG;
  if (prod && (!in->qjl || !in->rnorms)) return TQ_ERR_ARG;
  if (!aligned(out, 16) || ld_out < p->d_in) return TQ_ERR_ALIGN;
  if ((p->m > 0 && !aligned(in->codes, 4)) || (prod && !aligned(in->qjl, 4))) return TQ_ERR_ALIGN;
  DecodeArgs a{};
  a.n = n;
  a.d_in = p->d_in;
  a.d = p->d;
  a.log_lpv = log2i(p->d / kEPL);
  a.m = p->m;
  a.prod = prod ? 1 : 0;
  a.centroids = p->centroids;
  a.signs = p->signs;
  a.qjl_s = p->qjl_s;
  a.rot_kind = p->rotation;
  a.rot = p->rot;
  if (p->rotation != TQ_ROT_RHT) {
    // block rotations run in the d = 128 kernel only
    if (p->m > 4) return TQ_ERR_BITS;
    if ((ld_out & 3) != 0) return TQ_ERR_ALIGN;
  }
  a.codes = in->codes;
  a.qjl = in->qjl;
  a.norms = in->norms;
  a.rnorms = in->rnorms;
  a.out = out;
  a.ld_out = ld_out;
  return hip_status(launch_decode(a, stream));
}

size_t tq_score_workspace(const tq_params *p, int32_t mode, int64_t nq) {
  if (check_dims(p) != TQ_OK || nq < 0 || (mode != TQ_MSE && mode != TQ_PROD)) return 0;
  const size_t per = static_cast<size_t>(nq) * p->d * sizeof(float);
  const size_t rounded = (per + 255) & ~static_cast<size_t>(255);
  // TurboQuant_prod: rotated queries and S q'.  TurboQuant_mse: rotated
  // queries, their float16 (hi, lo) split and one scale per row.
  const size_t scales = (static_cast<size_t>(nq) * sizeof(float) + 255) & ~static_cast<size_t>(255);
  return mode == TQ_PROD ? 2 * rounded : 2 * rounded + scales;
}

int tq_score_grouped(const tq_params *p, int32_t mode, const float *q, int64_t ldq, int64_t groups,
                     int64_t nq, const tq_codes *keys, int64_t n, float *scores, int64_t ld_scores,
                     void *workspace, size_t ws_bytes, void *stream) {
  return score_checked(p, mode, q, ldq, groups, nq, keys, n, scores, ld_scores, workspace, ws_bytes, stream,
                       false);
}

int tq_score_accumulate(const tq_params *p, int32_t mode, const float *q, int64_t ldq, int64_t groups,
                        int64_t nq, const tq_codes *keys, int64_t n, float *scores, int64_t ld_scores,
                        void *workspace, size_t ws_bytes, void *stream) {
  return score_checked(p, mode, q, ldq, groups, nq, keys, n, scores, ld_scores, workspace, ws_bytes, stream,
                       true);
}

}  // extern "C"

namespace {

int score_checked(const tq_params *p, int32_t mode, const float *q, int64_t ldq, int64_t groups, int64_t nq,
                  const tq_codes *keys, int64_t n, float *scores, int64_t ld_scores, void *workspace,
                  size_t ws_bytes, void *stream, bool accumulate) {
  if (mode != TQ_MSE && mode != TQ_PROD) return TQ_ERR_ARG;
  const bool prod = mode == TQ_PROD;
  int st = check_params(p, prod);
  if (st != TQ_OK) return st;
  if (n < 0 || nq < 0 || groups < 0 || !keys) return TQ_ERR_ARG;
  if (n == 0 || nq == 0 || groups == 0) return TQ_OK;
  if (groups * nq > 65535) return TQ_ERR_ARG;
  if (!q || !scores || !keys->norms) return TQ_ERR_ARG;
  if (p->m > 0 && !keys->codes) return TQ_ERR_ARG;
  if (prod && (!keys->qjl || !keys->rnorms)) return TQ_ERR_ARG;
  if (ldq < p->d_in || ld_scores < n) return TQ_ERR_ALIGN;
  if (!aligned(q, 4) || !aligned(scores, 4)) return TQ_ERR_ALIGN;
  if ((p->m > 0 && !aligned(keys->codes, 16)) || (prod && !aligned(keys->qjl, 16))) return TQ_ERR_ALIGN;
  const int64_t nq_all = groups * nq;
  const size_t need = tq_score_workspace(p, mode, nq_all);
  if (!workspace || ws_bytes < need) return TQ_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return TQ_ERR_ALIGN;
  return score_launch(p, prod, q, ldq, groups, nq, keys, n, scores, ld_scores, workspace, need, stream,
                      accumulate);
}

}  // namespace

extern "C" {

int tq_score(const tq_params *p, int32_t mode, const float *q, int64_t ldq, int64_t nq,
             const tq_codes *keys, int64_t n, float *scores, int64_t ld_scores, void *workspace,
             size_t ws_bytes, void *stream) {
  return tq_score_grouped(p, mode, q, ldq, 1, nq, keys, n, scores, ld_scores, workspace, ws_bytes, stream);
}

size_t tq_topk_workspace(const tq_params *p, int32_t mode, int64_t nq, int64_t n, int32_t k) {
  if (check_dims(p) != TQ_OK || nq < 0 || n < 0 || k < 1 || k > kTopkMaxK) return 0;
  if (mode != TQ_MSE && mode != TQ_PROD) return 0;
  const int64_t qc = nq < kTopkChunk ? nq : kTopkChunk;
  const int64_t qf = nq < kFilterChunk ? nq : kFilterChunk;
  const bool filt = topk_filtered(p, mode == TQ_PROD, qf, n);
  const size_t rot = tq_score_workspace(p, mode, filt ? qf : qc);
  const size_t buf = static_cast<size_t>(qc) * topk_ld(n) * sizeof(float);
  return rot + round256(buf) + round256(topk_cand_bytes(qc, k)) + (filt ? topk_filter_bytes(qf, k) : 0);
}

int tq_topk(const tq_params *p, int32_t mode, const float *q, int64_t ldq, int64_t nq, const tq_codes *keys,
            int64_t n, int32_t k, int64_t *idx, float *vals, void *workspace, size_t ws_bytes, void *stream) {
  if (mode != TQ_MSE && mode != TQ_PROD) return TQ_ERR_ARG;
  const bool prod = mode == TQ_PROD;
  int st = check_params(p, prod);
  if (st != TQ_OK) return st;
  if (n < 0 || nq < 0 || !keys || k < 1 || k > kTopkMaxK || n >= (int64_t{1} << 31)) return TQ_ERR_ARG;
  if (nq == 0) return TQ_OK;
  if (!q || !idx || !vals) return TQ_ERR_ARG;
  if (n > 0) {                          // no key arrays are read when there are no keys
    if (!keys->norms || (p->m > 0 && !keys->codes)) return TQ_ERR_ARG;
    if (prod && (!keys->qjl || !keys->rnorms)) return TQ_ERR_ARG;
  }
  if (ldq < p->d_in) return TQ_ERR_ALIGN;
  if (!aligned(q, 4) || !aligned(idx, 8) || !aligned(vals, 4)) return TQ_ERR_ALIGN;
  if ((p->m > 0 && !aligned(keys->codes, 16)) || (prod && !aligned(keys->qjl, 16))) return TQ_ERR_ALIGN;
  const size_t need = tq_topk_workspace(p, mode, nq, n, k);
  if (!workspace || ws_bytes < need) return TQ_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return TQ_ERR_ALIGN;
  const int64_t qc = nq < kTopkChunk ? nq : kTopkChunk;
  const int64_t qf = nq < kFilterChunk ? nq : kFilterChunk;
  const bool filt = topk_filtered(p, prod, qf, n);
  const size_t rot = tq_score_workspace(p, mode, filt ? qf : qc);
  char *wsb = static_cast<char *>(workspace);
  float *buf = reinterpret_cast<float *>(wsb + rot);
  const int64_t ld = topk_ld(n);
  const size_t buf_bytes = round256(static_cast<size_t>(qc) * ld * sizeof(float));
  const int64_t lists = qc > 2048 ? qc : 2048;
  float *cand_vals = reinterpret_cast<float *>(wsb + rot + buf_bytes);
  int32_t *cand_idx = reinterpret_cast<int32_t *>(cand_vals + lists * k);

  // the top k of rows [r0, r0 + rows) from their score rows in buf, or only
  // the rows whose list count exceeds kListCap (over != nullptr)
  auto select = [&](int64_t r0, int64_t rows, const int32_t *over) {
    TopkArgs t{};
    t.scores = buf;
    t.ld = ld;
    t.n = n;
    t.rows = rows;
    t.k = k;
    t.idx = idx + r0 * k;
    t.vals = vals + r0 * k;
    t.segs = static_cast<int32_t>(topk_segments(rows, n));
    t.seg_len = ((n + t.segs - 1) / t.segs + 3) & ~int64_t{3};
    t.cand_vals = cand_vals;
    t.cand_idx = cand_idx;
    t.only_over = over;
    t.over_cap = kListCap;
    return launch_topk(t, stream) ? TQ_ERR_HIP : TQ_OK;
  };

  int64_t q0 = 0;
  if (filt) {
    // the filtered search's arrays
    char *fx = wsb + rot + buf_bytes + round256(topk_cand_bytes(qc, k));
    float *sample = reinterpret_cast<float *>(fx);
    fx += round256(static_cast<size_t>(qf) * kSampleCols * sizeof(float));
    int64_t *s_idx = reinterpret_cast<int64_t *>(fx);
    fx += round256(static_cast<size_t>(qf) * k * sizeof(int64_t));
    float *s_vals = reinterpret_cast<float *>(fx);
    fx += round256(static_cast<size_t>(qf) * k * sizeof(float));
    float *tau = reinterpret_cast<float *>(fx);
    fx += round256(static_cast<size_t>(qf) * sizeof(float));
    int32_t *cnt = reinterpret_cast<int32_t *>(fx);
    fx += round256(static_cast<size_t>(qf) * sizeof(int32_t));
    float *list_v = reinterpret_cast<float *>(fx);
    fx += round256(static_cast<size_t>(qf) * kListCap * sizeof(float));
    int32_t *list_i = reinterpret_cast<int32_t *>(fx);
    for (; q0 < nq; q0 += qf) {
      const int64_t rows = nq - q0 < qf ? nq - q0 : qf;
      if (!topk_filtered(p, prod, rows, n)) break;          // a short remainder: the plain path
      // 1. the sample's estimates and their top k -> tau, counts zeroed
      ScoreMArgs sm{};
      st = scorem_prepare(p, q + q0 * ldq, ldq, rows, keys, n, workspace, stream, sm);
      if (st != TQ_OK) return st;
      ScoreMArgs ss = sm;
      ss.kb_stride = (n / kScoreMKeys) / kSampleBlocks;
      ss.n_cols = kSampleCols;
      ss.scores = sample;
      ss.ld_scores = kSampleCols;
      if (launch_scorem(ss, stream)) return TQ_ERR_HIP;
      TopkArgs ts{};
      ts.scores = sample;
      ts.ld = kSampleCols;
      ts.n = kSampleCols;
      ts.rows = rows;
      ts.k = k;
      ts.idx = s_idx;
      ts.vals = s_vals;
      ts.segs = static_cast<int32_t>(topk_segments(rows, kSampleCols));
      ts.seg_len = ((kSampleCols + ts.segs - 1) / ts.segs + 3) & ~int64_t{3};
      ts.cand_vals = cand_vals;
      ts.cand_idx = cand_idx;
      if (launch_topk(ts, stream)) return TQ_ERR_HIP;
      TauArgs ta{rows, k, s_idx, s_vals, tau, cnt};
      if (launch_tau(ta, stream)) return TQ_ERR_HIP;
      // 2. every key against tau, into the lists, and their top k
      ScoreMArgs sf = sm;
      sf.tau = tau;
      sf.cnt = cnt;
      sf.list_v = list_v;
      sf.list_i = list_i;
      sf.list_cap = kListCap;
      if (launch_scorem(sf, stream)) return TQ_ERR_HIP;
      TopkListArgs tl{rows, k, list_v, list_i, cnt, kListCap, idx + q0 * k, vals + q0 * k};
      if (launch_topk_lists(tl, stream)) return TQ_ERR_HIP;
      // 3. rows whose list overflowed: the full score rows and their top k,
      // qc rows at a time (the launches find nothing to do when no list did)
      for (int64_t f0 = 0; f0 < rows; f0 += qc) {
        const int64_t fr = rows - f0 < qc ? rows - f0 : qc;
        ScoreMArgs so = sm;
        so.nq = static_cast<int32_t>(fr);
        so.qh = sm.qh + f0 * p->d;
        so.ql = sm.ql + f0 * p->d;
        so.qinv = sm.qinv + f0;
        so.scores = buf;
        so.ld_scores = ld;
        so.only_over = cnt + f0;
        so.list_cap = kListCap;
        if (launch_scorem(so, stream)) return TQ_ERR_HIP;
        st = select(q0 + f0, fr, cnt + f0);
        if (st != TQ_OK) return st;
      }
    }
  }
  for (; q0 < nq; q0 += qc) {
    const int64_t rows = nq - q0 < qc ? nq - q0 : qc;
    if (n > 0) {
      st = score_launch(p, prod, q + q0 * ldq, ldq, 1, rows, keys, n, buf, ld, workspace, rot, stream);
      if (st != TQ_OK) return st;
    }
    st = select(q0, rows, nullptr);
    if (st != TQ_OK) return st;
  }
  return TQ_OK;
}

}  // extern "C"

namespace {

// The float16 (hi, lo) split of the rotated queries in the workspace (which
// holds them first) for the matrix-core kernel; fills sm's query fields.
int scorem_split(const tq_params *p, int64_t nq_all, void *workspace, void *stream, ScoreMArgs &sm) {
  const size_t per = ((static_cast<size_t>(nq_all) * p->d * sizeof(float)) + 255) & ~static_cast<size_t>(255);
  QSplitArgs qs{};
  qs.rows = nq_all;
  qs.d = p->d;
  qs.qrot = static_cast<float *>(workspace);
  qs.qh = reinterpret_cast<uint16_t *>(static_cast<char *>(workspace) + per);
  qs.ql = qs.qh + static_cast<size_t>(nq_all) * p->d;
  qs.qinv = reinterpret_cast<float *>(static_cast<char *>(workspace) + 2 * per);
  const int err = launch_qsplit(qs, stream);
  sm.d = p->d;
  sm.m = p->m;
  sm.centroids = p->centroids;
  sm.qh = qs.qh;
  sm.ql = qs.ql;
  sm.qinv = qs.qinv;
  return err;
}

int scorem_prepare(const tq_params *p, const float *q, int64_t ldq, int64_t nq, const tq_codes *keys, int64_t n,
                   void *workspace, void *stream, ScoreMArgs &sm) {
  RhtArgs r{};
  r.n = nq;
  r.d_in = p->d_in;
  r.d = p->d;
  r.log_lpv = log2i(p->d / kEPL);
  r.inverse = 0;
  r.signs = p->signs;
  r.rot_kind = p->rotation;
  r.rot = p->rot;
  r.in = q;
  r.ld_in = ldq;
  r.out = static_cast<float *>(workspace);
  r.ld_out = p->d;
  if (launch_rht(r, stream)) return TQ_ERR_HIP;
  if (scorem_split(p, nq, workspace, stream, sm)) return TQ_ERR_HIP;
  sm.n = n;
  sm.nq = static_cast<int32_t>(nq);
  sm.groups = 1;
  sm.codes = keys->codes;
  sm.norms = keys->norms;
  sm.kb_stride = 1;
  sm.n_cols = n;
  return TQ_OK;
}

int score_launch(const tq_params *p, bool prod, const float *q, int64_t ldq, int64_t groups, int64_t nq,
                 const tq_codes *keys, int64_t n, float *scores, int64_t ld_scores, void *workspace,
                 size_t need, void *stream, bool accumulate) {
  const int64_t nq_all = groups * nq;
  (void)need;
  float *qrot = static_cast<float *>(workspace);
  const size_t per = ((static_cast<size_t>(nq_all) * p->d * sizeof(float)) + 255) & ~static_cast<size_t>(255);
  float *sq = prod ? reinterpret_cast<float *>(static_cast<char *>(workspace) + per) : nullptr;
  const bool mfma = score_on_mfma(p->d, p->m, prod, nq);
  const bool in_kernel = !mfma && score_prep_in_kernel(p->d, p->m);
  if (!in_kernel) {   // rotate the queries (and form S q') into the workspace
    RhtArgs r{};
    r.n = nq_all;
    r.d_in = p->d_in;
    r.d = p->d;
    r.log_lpv = log2i(p->d / kEPL);
    r.inverse = 0;
    r.signs = p->signs;
    r.rot_kind = p->rotation;
    r.rot = p->rot;
    r.in = q;
    r.ld_in = ldq;
    r.out = qrot;
    r.ld_out = p->d;
    int err = launch_rht(r, stream);
    if (err) return TQ_ERR_HIP;
    if (prod) {
      SqArgs sa{};
      sa.nq = static_cast<int32_t>(nq_all);
      sa.d = p->d;
      sa.qjl_s = p->qjl_s;
      sa.qrot = qrot;
      sa.sq = sq;
      err = launch_sq(sa, stream);
      if (err) return TQ_ERR_HIP;
    }
  }
  if (mfma) {
    // split the rotated queries for the matrix cores, then score
    ScoreMArgs sm{};
    if (scorem_split(p, nq_all, workspace, stream, sm)) return TQ_ERR_HIP;
    sm.n = n;
    sm.nq = static_cast<int32_t>(nq);
    sm.groups = static_cast<int32_t>(groups);
    sm.codes = keys->codes;
    sm.norms = keys->norms;
    sm.scores = scores;
    sm.ld_scores = ld_scores;
    sm.accumulate = accumulate ? 1 : 0;
    sm.kb_stride = 1;
    sm.n_cols = n;
    return hip_status(launch_scorem(sm, stream));
  }
  ScoreArgs a{};
  a.n = n;
  a.nq = static_cast<int32_t>(nq);
  a.groups = static_cast<int32_t>(groups);
  a.d = p->d;
  a.m = p->m;
  a.prod = prod ? 1 : 0;
  a.centroids = p->centroids;
  a.qrot = qrot;
  a.sq = sq;
  a.codes = keys->codes;
  a.qjl = keys->qjl;
  a.norms = keys->norms;
  a.rnorms = keys->rnorms;
  a.scores = scores;
  a.ld_scores = ld_scores;
  a.accumulate = accumulate ? 1 : 0;
  a.q = q;
  a.ldq = ldq;
  a.d_in = p->d_in;
  a.rot_kind = p->rotation;
  a.signs = p->signs;
  a.rot = p->rot;
  a.qjl_s = p->qjl_s;
  return hip_status(launch_score(a, stream));
}

}  // namespace

extern "C" {

int tq_rht(const tq_params *p, const float *in, int64_t ld_in, float *out, int64_t ld_out, int64_t n,
           int32_t inverse, void *stream) {
  int st = check_dims(p);
  if (st != TQ_OK) return st;
  st = check_rotation(p);
  if (st != TQ_OK) return st;
  if (n < 0) return TQ_ERR_ARG;
  if (n == 0) return TQ_OK;
  if (!in || !out) return TQ_ERR_ARG;
  const int in_cols = inverse ? p->d : p->d_in;
  const int out_cols = inverse ? p->d_in : p->d;
  if (ld_in < in_cols || ld_out < out_cols) return TQ_ERR_ALIGN;
  if (!aligned(in, 4) || !aligned(out, 4)) return TQ_ERR_ALIGN;
  RhtArgs r{};
  r.n = n;
  r.d_in = p->d_in;
  r.d = p->d;
  r.log_lpv = log2i(p->d / kEPL);
  r.inverse = inverse ? 1 : 0;
  r.signs = p->signs;
  r.rot_kind = p->rotation;
  r.rot = p->rot;
  r.in = in;
  r.ld_in = ld_in;
  r.out = out;
  r.ld_out = ld_out;
  return hip_status(launch_rht(r, stream));
}

size_t tq_attend_workspace(const tq_params *pk, int32_t kmode, int64_t groups, int64_t nq_per_group,
                           int64_t n_per_group) {
  if (check_dims(pk) != TQ_OK || pk->d != 128) return 0;
  if (kmode != TQ_MSE && kmode != TQ_PROD) return 0;
  if (groups < 0 || nq_per_group < 0 || n_per_group < 0) return 0;
  const int64_t nq_all = groups * nq_per_group;
  return static_cast<size_t>(nq_all) * attend_chunks(n_per_group) * kAttnPart * sizeof(float);
}

}  // extern "C"

namespace {

// Argument checks of tq_attend except the workspace: TQ_OK, a negative
// status, or 1 when the call has no work (nothing to launch).
int attend_check(const tq_params *pk, int32_t kmode, const tq_codes *keys, const tq_params *pv,
                 const tq_codes *values, const float *q, int64_t ldq, int64_t groups, int64_t nq_per_group,
                 int64_t n_per_group, float *out, int64_t ld_out) {
  if (kmode != TQ_MSE && kmode != TQ_PROD) return TQ_ERR_ARG;
  const bool prodk = kmode == TQ_PROD;
  int st = check_params(pk, prodk);
  if (st != TQ_OK) return st;
  st = check_params(pv, false);
  if (st != TQ_OK) return st;
  if (pk->d != 128 || pv->d != 128 || pv->d_in != pk->d_in) return TQ_ERR_DIM;
  if (pk->rotation != TQ_ROT_RHT || pv->rotation != TQ_ROT_RHT) return TQ_ERR_ARG;
  if ((prodk && pk->m > 3) || (!prodk && pk->m > 4) || pv->m > 4) return TQ_ERR_BITS;
  if (!keys || !values || groups < 0 || nq_per_group < 0 || n_per_group < 0) return TQ_ERR_ARG;
  if (groups == 0 || nq_per_group == 0 || n_per_group == 0) return 1;
  const int64_t qblocks = (nq_per_group + 3) / 4;
  if (groups * qblocks > 65535 || attend_chunks(n_per_group) > 0x7FFFFFFF) return TQ_ERR_ARG;
  if (!q || !out || !keys->norms || !values->codes || !values->norms) return TQ_ERR_ARG;
  if (pk->m > 0 && !keys->codes) return TQ_ERR_ARG;
  if (prodk && (!keys->qjl || !keys->rnorms)) return TQ_ERR_ARG;
  if (ldq < pk->d_in || ld_out < pv->d_in) return TQ_ERR_ALIGN;
  if (!aligned(q, 4) || !aligned(out, 4) || !aligned(values->codes, 4)) return TQ_ERR_ALIGN;
  if ((pk->m > 0 && !aligned(keys->codes, 16)) || (prodk && !aligned(keys->qjl, 16))) return TQ_ERR_ALIGN;
  return TQ_OK;
}

// The launches of tq_attend with the partials in `part` (checked arguments).
int attend_launch(const tq_params *pk, int32_t kmode, const tq_codes *keys, const tq_params *pv,
                  const tq_codes *values, const float *q, int64_t ldq, int64_t groups, int64_t nq_per_group,
                  int64_t n_per_group, float scale, float *out, int64_t ld_out, float *part, void *stream) {
  const bool prodk = kmode == TQ_PROD;
  const int64_t nq_all = groups * nq_per_group;
  AttnArgs a{};
  a.n = n_per_group;
  a.nq_all = nq_all;
  a.nq = static_cast<int32_t>(nq_per_group);
  a.groups = static_cast<int32_t>(groups);
  a.d_in = pv->d_in;
  a.mk = pk->m;
  a.prodk = prodk ? 1 : 0;
  a.mv = pv->m;
  a.scale = scale;
  a.k_centroids = pk->centroids;
  a.v_centroids = pv->centroids;
  a.v_signs = pv->signs;
  a.q = q;
  a.ldq = ldq;
  a.k_signs = pk->signs;
  a.qjl_s = prodk ? pk->qjl_s : nullptr;
  a.k_codes = keys->codes;
  a.k_qjl = keys->qjl;
  a.k_norms = keys->norms;
  a.k_rnorms = keys->rnorms;
  a.v_codes = values->codes;
  a.v_norms = values->norms;
  a.part = part;
  a.out = out;
  a.ld_out = ld_out;
  return hip_status(launch_attend(a, stream));
}

}  // namespace

// Fixed scratch of tq_attend_noalloc: one copy per GPU, held until the
// process ends.  Host code never passes `scratch` itself to a kernel or a
// copy (on the host the name is a stand-in, not device memory): each
// device's address is looked up once, with that device current, and kept.
static constexpr size_t kAttendScratchBytes = size_t{16} << 20;
static __device__ __align__(256) uint8_t scratch[kAttendScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void *> g_attend_scratch[kMaxDevices];
std::mutex g_attend_scratch_mu;

int attend_scratch_ptr(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TQ_ERR_HIP;
  void *p = g_attend_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_attend_scratch_mu);
    p = g_attend_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TQ_ERR_HIP;
      g_attend_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return TQ_OK;
}

}  // namespace

extern "C" {

int tq_attend(const tq_params *pk, int32_t kmode, const tq_codes *keys, const tq_params *pv,
              const tq_codes *values, const float *q, int64_t ldq, int64_t groups, int64_t nq_per_group,
              int64_t n_per_group, float scale, float *out, int64_t ld_out, void *workspace,
              size_t ws_bytes, void *stream) {
  const int st = attend_check(pk, kmode, keys, pv, values, q, ldq, groups, nq_per_group, n_per_group, out, ld_out);
  if (st != TQ_OK) return st < 0 ? st : TQ_OK;
  const size_t need = tq_attend_workspace(pk, kmode, groups, nq_per_group, n_per_group);
  if (!workspace || ws_bytes < need) return TQ_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return TQ_ERR_ALIGN;
  return attend_launch(pk, kmode, keys, pv, values, q, ldq, groups, nq_per_group, n_per_group, scale, out,
                       ld_out, static_cast<float *>(workspace), stream);
}

int tq_attend_noalloc(const tq_params *pk, int32_t kmode, const tq_codes *keys, const tq_params *pv,
                      const tq_codes *values, const float *q, int64_t ldq, int64_t groups, int64_t nq_per_group,
                      int64_t n_per_group, float scale, float *out, int64_t ld_out, void *stream) {
  const int st = attend_check(pk, kmode, keys, pv, values, q, ldq, groups, nq_per_group, n_per_group, out, ld_out);
  if (st != TQ_OK) return st < 0 ? st : TQ_OK;
  if (tq_attend_workspace(pk, kmode, groups, nq_per_group, n_per_group) > kAttendScratchBytes)
    return TQ_ERR_WORKSPACE;
  void *part = nullptr;
  const int sp = attend_scratch_ptr(&part);
  if (sp != TQ_OK) return sp;
  return attend_launch(pk, kmode, keys, pv, values, q, ldq, groups, nq_per_group, n_per_group, scale, out,
                       ld_out, static_cast<float *>(part), stream);
}

const char *tq_status_string(int32_t status) {
  switch (status) {
    case TQ_OK: return "ok";
    case TQ_ERR_ARG: return "invalid argument (NULL pointer, negative count or unknown enum)";
    case TQ_ERR_DIM: return "invalid dimension (d must be a power of two in [32, 4096], 1 <= d_in <= d)";
    case TQ_ERR_BITS: return "invalid bit width m for this call";
    case TQ_ERR_ALIGN: return "misaligned pointer or row stride too small";
    case TQ_ERR_WORKSPACE: return "workspace missing or smaller than tq_score_workspace()";
    case TQ_ERR_HIP: return "HIP runtime error at launch";
    case TQ_ERR_NOCONV: return "codebook iteration did not converge";
    default: return "unknown status";
  }
}

int32_t tq_version(void) { return TQ_VERSION; }

}  // extern "C"
