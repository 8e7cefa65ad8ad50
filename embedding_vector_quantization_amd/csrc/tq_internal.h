// Internal declarations shared by the host entry points and the kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/tq.h"

namespace tq {

// Register-resident layout used by every kernel: a vector of d coordinates
// is held by LPV = d / 32 consecutive lanes, lane `sub` owning the 32
// contiguous coordinates [32 sub, 32 sub + 32); a wave holds 64 / LPV
// vectors, and at d = 4096 a vector spans two waves (sub = 64 h + lane for
// wave h of the pair).  A lane's m-bit codes are then exactly m dwords of
// the record.
constexpr int kEPL = 32;
constexpr int kMinD = 32;
constexpr int kMaxD = 4096;
constexpr int kPairLogLpv = 7;     // log2(4096 / 32): the paired-wave layout
constexpr int kScoreMKeys = 512;   // keys per workgroup of the many-query score kernel

struct EncodeArgs {
  const void *x;
  int64_t ld_x;         // elements
  int64_t n;
  int32_t d_in, d, log_lpv, dtype;
  int32_t m;
  int32_t vec_loads;    // 1: rows are 16-byte aligned and d_in*esize % 16 == 0
  const float *centroids;
  const float *thresholds;
  const int8_t *signs;
  const uint16_t *qjl_s;
  int32_t rot_kind;     // TQ_ROT_*
  const float *rot;     // block rotation parameters
  uint8_t *codes;
  uint8_t *qjl;
  float *norms;
  float *rnorms;
};

struct DecodeArgs {
  int64_t n;
  int32_t d_in, d, log_lpv, m;
  int32_t prod;
  const float *centroids;
  const int8_t *signs;
  const uint16_t *qjl_s;
  int32_t rot_kind;     // TQ_ROT_*
  const float *rot;     // block rotation parameters
  const uint8_t *codes;
  const uint8_t *qjl;
  const float *norms;
  const float *rnorms;
  float *out;
  int64_t ld_out;
};

struct RhtArgs {
  int64_t n;
  int32_t d_in, d, log_lpv, inverse;
  const int8_t *signs;
  int32_t rot_kind;     // TQ_ROT_*
  const float *rot;     // block rotation parameters
  const float *in;
  int64_t ld_in;
  float *out;
  int64_t ld_out;
};

struct ScoreArgs {
  int64_t n;            // keys per group
  int32_t nq;           // queries per group
  int32_t groups;       // query group g is scored against key group g only
  int32_t d, m, prod;
  const float *centroids;
  const float *qrot;    // [nq][d] rotated queries (workspace)
  const float *sq;      // [nq][d] S * rotated queries (workspace, prod)
  const uint8_t *codes;
  const uint8_t *qjl;
  const float *norms;
  const float *rnorms;
  float *scores;
  int64_t ld_scores;
  int32_t accumulate;   // 1: add the estimates to scores
  // Raw queries and rotation, read when the kernel prepares its own queries
  // (score_prep_in_kernel(d, m)): then qrot and sq are not used.
  const float *q;       // [groups * nq][ldq]
  int64_t ldq;
  int32_t d_in, rot_kind;
  const int8_t *signs;
  const float *rot;
  const uint16_t *qjl_s;
};

// Many queries against TurboQuant_mse keys on the matrix cores: the rotated
// queries are first split into float16 (hi, lo) parts, scaled by a power of
// two per row (qinv = the inverse scale).
struct QSplitArgs {
  int64_t rows;
  int32_t d;
  const float *qrot;    // [rows][d]
  uint16_t *qh;         // [rows][d] float16 bits
  uint16_t *ql;         // [rows][d] float16 bits
  float *qinv;          // [rows]
};

struct ScoreMArgs {
  int64_t n;            // keys per group
  int32_t nq;           // queries per group
  int32_t groups;
  int32_t d, m;
  const float *centroids;
  const uint16_t *qh, *ql;
  const float *qinv;
  const uint8_t *codes;
  const float *norms;
  float *scores;
  int64_t ld_scores;
  int32_t accumulate;
  // Key blocks of kScoreMKeys: block kb reads the keys from
  // kb * kb_stride * kScoreMKeys on (kb_stride > 1: an evenly spread sample)
  // and its estimates go to columns kb * kScoreMKeys .. of scores; n_cols
  // columns (n when kb_stride == 1).
  int64_t kb_stride;
  int64_t n_cols;
  // Filtered (tau != nullptr): no score matrix; an estimate >= tau[row] is
  // appended to the row's list (list_v / list_i + row * list_cap) at the
  // slot an atomic count cnt[row] hands out (slots past list_cap are
  // dropped, the count still grows).
  const float *tau;
  int32_t *cnt;
  float *list_v;
  int32_t *list_i;
  int32_t list_cap;
  // only_over != nullptr: only workgroups with a query row whose count
  // only_over[row] exceeds list_cap do any work.
  const int32_t *only_over;
};

// True when the matrix-core path scores (TurboQuant_mse, 1 <= m <= 4, at
// least 16 queries per group).
bool score_on_mfma(int d, int m, bool prod, int64_t nq);

// True when the score kernels for (d, m) rotate their queries (and form
// S q') themselves, so no separate query launches are needed.
bool score_prep_in_kernel(int d, int m);

struct SqArgs {
  int32_t nq, d;
  const uint16_t *qjl_s;
  const float *qrot;
  float *sq;
};

// Decode attention (d = 128): per (query row, token chunk) partial
// m, l, two pad floats, acc[128].
constexpr int kAttnPart = 132;

struct AttnArgs {
  int64_t n;            // tokens per group
  int64_t nq_all;       // query rows over all groups
  int32_t nq;           // query rows per group
  int32_t groups;
  int32_t d_in;
  int32_t mk, prodk, mv;
  float scale;
  const float *k_centroids;
  const float *v_centroids;
  const int8_t *v_signs;
  const float *q;       // [nq_all][ldq] queries (d_in used)
  int64_t ldq;
  const int8_t *k_signs;
  const uint16_t *qjl_s;  // S of prod keys (bfloat16, [128][128])
  const uint8_t *k_codes;
  const uint8_t *k_qjl;
  const float *k_norms;
  const float *k_rnorms;
  const uint8_t *v_codes;
  const float *v_norms;
  float *part;          // [nq_all][chunks][kAttnPart] (workspace)
  float *out;
  int64_t ld_out;
};

int64_t attend_chunks(int64_t n);

struct TopkArgs {
  const float *scores;  // [rows][ld] estimates
  int64_t ld;
  int64_t n;            // keys per row, < 2^31
  int64_t rows;
  int32_t k;            // 1..32
  int64_t *idx;         // [rows][k]
  float *vals;          // [rows][k]
  // Rows are cut into `segs` segments of seg_len keys (a multiple of 4); with
  // more than one, each segment's top k go to the candidate lists first.
  int32_t segs;
  int64_t seg_len;
  float *cand_vals;     // [rows][segs][k] (workspace)
  int32_t *cand_idx;    // [rows][segs][k] (workspace)
  // only_over != nullptr: only rows whose only_over[row] exceeds over_cap.
  const int32_t *only_over;
  int32_t over_cap;
};

// Final top k of counted candidate lists: row r's input is the first
// min(cnt[r], cap) entries of list_v / list_i + r * cap; a row whose count
// exceeds cap is left alone.
struct TopkListArgs {
  int64_t rows;
  int32_t k;
  const float *list_v;
  const int32_t *list_i;
  const int32_t *cnt;
  int32_t cap;
  int64_t *idx;
  float *vals;
};

// tau[r] = row r's k-th value of a finished top k (idx, vals [rows][k]), or
// -inf when the row has fewer than k entries; cnt[r] = 0.
struct TauArgs {
  int64_t rows;
  int32_t k;
  const int64_t *idx;
  const float *vals;
  float *tau;
  int32_t *cnt;
};

// Segments per row for `rows` rows of n keys (rows * segments <= max(2048, rows)).
int64_t topk_segments(int64_t rows, int64_t n);

int make_codebook(int d, int m, double *centroids, double *thresholds, double *dmse);

// Launchers: return 0 or a hipError_t value.
int launch_encode(const EncodeArgs &a, bool prod, void *stream);
int launch_decode(const DecodeArgs &a, void *stream);
int launch_rht(const RhtArgs &a, void *stream);
int launch_score(const ScoreArgs &a, void *stream);
int launch_sq(const SqArgs &a, void *stream);
int launch_attend(const AttnArgs &a, void *stream);
int launch_topk(const TopkArgs &a, void *stream);
int launch_topk_lists(const TopkListArgs &a, void *stream);
int launch_tau(const TauArgs &a, void *stream);
int launch_qsplit(const QSplitArgs &a, void *stream);
int launch_scorem(const ScoreMArgs &a, void *stream);

}  // namespace tq
