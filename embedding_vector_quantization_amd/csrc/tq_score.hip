// Inner-product estimator on packed codes for gfx950.
//
// Sources: "TurboQuant: Online Vector Quantization" paper summary (Jump2Paper
// Archive) -- the estimator <y, Q^-1(Q(x))> of the definitions table, the
// QJL dequantiser sqrt(pi/2)/d * S^T z (Definition 1, Lemma 4) and Theorem
// D_prod (unbiased inner products for TurboQuant_prod); GeekNews Hacker News
// thread (queries are rotated once instead of un-rotating every key).
//
// For a key with norm n, codes idx and (prod) gamma, z:
//   est = n * ( sum_j q'_j c[idx_j] + gamma sqrt(pi/2)/d sum_i s_i z_i ),
//   q' = Pi q, s = S q'.
// Keys and queries come in `groups`: query group g is scored against key
// group g (one KV head and its query heads, or G = 1 for all pairs).
//
// Streaming kernels (d >= 128), one lane per key, coordinates in chunks of
// 128.  For each chunk the workgroup builds tables in LDS whose entry for a
// group of G coordinates and their G*m code bits is sum_j q'_j c[code_j]:
//   * one query: groups of up to 8 code bits, one float per entry, so a key
//     costs one bit-field extract, one LDS read and one add per group;
//   * up to four queries: smaller groups (tables <= 64 KiB) whose entries
//     hold the four queries' sums as one float4, so one 16-byte LDS read
//     serves all of them;
//   * prod adds a table over the QJL plane with entry (k, v) =
//     sum_t (bit t of v ? s : -s)_{8k+t} (bytes for one query, nibbles for
//     four).
// Small d (< 128) uses a plain per-coordinate loop.

#include <hip/hip_runtime.h>

#include "tq_device.h"
#include "tq_internal.h"
#include "tq_lut.h"

namespace tq {
namespace {

constexpr int kThreads = 256;

// Writes an estimate, or adds it to what is there (scores of one channel
// range added to those of the others).
__device__ __forceinline__ void put_score(const ScoreArgs &a, int64_t i, float v) {
  a.scores[i] = a.accumulate ? a.scores[i] + v : v;
}


// ------------------------------------------------------------ one query

template <int M>
struct Shape1 {
  // 16-entry tables for 1, 2 and 4 code bits (conflict-free lookups, see
  // kZ1Bits); 3 bits keep two coordinates (64 entries: single coordinates
  // double the lookups and measured slower, 185 against 161 us over 2^24 keys)
  static constexpr int G = (M == 1) ? 4 : (M == 2) ? 2 : (M == 3) ? 2 : 1;   // coordinates per group
  static constexpr int W = G * M;                                             // bits per group
  static constexpr int NG = kChunk / G;                                       // groups per chunk
  static constexpr int ENTRIES = NG << W;
};
template <>
struct Shape1<0> {
  static constexpr int G = 1, W = 0, NG = 0, ENTRIES = 0;
};
// QJL bits per lookup: 16-entry tables, like the 2-bit codes' (2 coordinates
// per lookup): a table of 16 floats spans 16 distinct LDS banks, so the 64
// lanes' random lookups never conflict.  Tables of 256 entries (8 bits per
// lookup) take half the lookups, but their conflicts cost more: the one-query
// prod b = 3 score over 2^24 keys took 209 us with 8-bit code and QJL
// lookups, 187 us with 4-bit code lookups, 186.5 us with both 4-bit.
constexpr int kZ1Bits = 4;
constexpr int kZ1Entries = (128 / kZ1Bits) << kZ1Bits;          // QJL tables per chunk

template <int M, bool PROD>
constexpr int floats1() { return Shape1<M>::ENTRIES + (PROD ? kZ1Entries : 0); }

// Largest table kept in static LDS for the d = 128 path: a static array has a
// compile-time address, so each lookup's table offset folds into the LDS
// instruction instead of costing an add.
constexpr int kStaticLutBytes = 48 * 1024;

// acc[T & 3] += table entry of group T (four partial sums for ILP).
template <int M, int T>
__device__ __forceinline__ void groups1(const uint32_t *w, const float *lut, float (&acc)[4]) {
  using S = Shape1<M>;
  if constexpr (T < S::NG) {
    const uint32_t f4 = field_at<S::W, T * S::W, 2>(w);
    acc[T & 3] += *reinterpret_cast<const float *>(reinterpret_cast<const char *>(lut) + (T << S::W) * 4 + f4);
    groups1<M, T + 1>(w, lut, acc);
  }
}


// blockIdx.y = query index over all groups (g = y / nq).
template <int M, bool PROD>
constexpr bool static_lut1() { return RecStage<M>::kOn && floats1<M, PROD>() * 4 <= kStaticLutBytes; }

template <int M, bool PROD, int NT>
__global__ void __launch_bounds__(NT) score1_kernel(ScoreArgs a) {
  extern __shared__ __attribute__((aligned(16))) float dyn_lut[];
  constexpr bool kStatic = static_lut1<M, PROD>();
  __shared__ __attribute__((aligned(16))) float st_lut[kStatic ? floats1<M, PROD>() : 1];
  using S = Shape1<M>;
  constexpr int K = 1 << M;
  __shared__ float cb[K > 1 ? K : 2];
  if constexpr (M >= 1) {
    for (int k = threadIdx.x; k < K; k += NT) cb[k] = a.centroids[k];
  }
  const int qg = blockIdx.y;                     // query row over all groups
  const int64_t grp = qg / a.nq;
  const int nchunks = a.d / kChunk;
  const int64_t tiles = (a.n + NT - 1) / NT;
  const float zs = kQjlScale / static_cast<float>(a.d);
  const size_t rec_words = static_cast<size_t>(M) * a.d / 32;
  const size_t z_words = static_cast<size_t>(a.d) / 32;
  const int64_t key0 = grp * a.n;

  // qb, sb: the query's rotated coordinates and S q' (row starts)
  auto build = [&](int c, float *lut, const float *qb, const float *sb) {
    __syncthreads();
    for (int i = threadIdx.x; i < floats1<M, PROD>(); i += NT) {
      float val = 0.0f;
      if (i < S::ENTRIES) {
        if constexpr (M >= 1) {
          const int t = i >> S::W;
          const int v = i & ((1 << S::W) - 1);
          const float *qr = qb + c * kChunk + t * S::G;
#pragma unroll
          for (int u = 0; u < S::G; ++u) val = fmaf(qr[u], cb[(v >> (M * u)) & (K - 1)], val);
        }
      } else {
        const int rz = i - S::ENTRIES;
        const int k = rz >> kZ1Bits;
        const int v = rz & ((1 << kZ1Bits) - 1);
        const float *sq = sb + c * kChunk + kZ1Bits * k;
#pragma unroll
        for (int t = 0; t < kZ1Bits; ++t) val += ((v >> t) & 1) ? sq[t] : -sq[t];
      }
      lut[i] = val;
    }
    __syncthreads();
  };

  using RS = RecStage<M>;
  if constexpr (RS::kOn) {
    if (nchunks == 1) {
      // d = 128: the block rotates its query itself; each wave's records
      // go straight from HBM into its LDS stage, next tile in flight
      using RD = RecDma<M>;
      float *lut = kStatic ? st_lut : dyn_lut;
      __shared__ __attribute__((aligned(16))) float qr_lds[1][128];
      __shared__ __attribute__((aligned(16))) float sq_lds[1][PROD ? 128 : 1];
      __shared__ __attribute__((aligned(16))) uint32_t rstage[(NT / 64) * RD::kWaveDwords];
      const int lane = threadIdx.x & 63;
      const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: so is the stage base
      uint32_t *ws = rstage + wv * RD::kWaveDwords;
      uint4 nz = make_uint4(0, 0, 0, 0);
      float nn = 0.0f, ng = 0.0f;
      auto issue = [&](int64_t t) {
        const int64_t k0 = t * NT + wv * 64;             // wave's first key in the group
        RD::issue(a.codes, key0 + k0, a.n - k0, lane, ws);
        const int64_t kl = t * NT + threadIdx.x;
        const int64_t kk = key0 + (kl < a.n ? kl : 0);
        nn = a.norms[kk];
        if constexpr (PROD) {
          ng = a.rnorms[kk];
          nz = load_nt16(a.qjl + kk * 16);
        }
      };
      int64_t tile = blockIdx.x;
      if (tile < tiles) issue(tile);                 // in flight during the query set-up
      if (wv == 0) rotate_query128(a.q + static_cast<int64_t>(qg) * a.ldq, a.d_in, a.rot_kind, a.signs, a.rot,
                                   qr_lds[0], lane);
      if constexpr (PROD) {
        __shared__ __attribute__((aligned(16))) float sq_part[NT / 128][128];
        __syncthreads();
        sq_rows128<NT, 1>(a.qjl_s, qr_lds, reinterpret_cast<float (*)[128]>(&sq_lds[0][0]), sq_part, 1);
      }
      build(0, lut, qr_lds[0], &sq_lds[0][0]);
      for (; tile < tiles; tile += gridDim.x) {
        // this tile's records have landed; the previous tile's score store,
        // the one access issued after them, may still be in flight.  The
        // stage is read, then refilled.
        asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
        uint32_t w[4 * M];
        RD::get(ws, lane, w);
        const float nrm = nn;
        const float g = PROD ? ng * zs : 0.0f;
        const uint4 zv = nz;
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (tile + gridDim.x < tiles) issue(tile + gridDim.x);
        float accz = 0.0f;
        if constexpr (PROD) {
          const uint32_t zw[4] = {zv.x, zv.y, zv.z, zv.w};
          const float *lz = lut + S::ENTRIES;
          float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
          for (int k = 0; k < 128 / kZ1Bits; k += 2) {
            constexpr int per = 32 / kZ1Bits;
            p0 += lz[(k << kZ1Bits) + ((zw[k / per] >> (kZ1Bits * (k % per))) & ((1u << kZ1Bits) - 1u))];
            p1 += lz[((k + 1) << kZ1Bits) + ((zw[(k + 1) / per] >> (kZ1Bits * ((k + 1) % per))) & ((1u << kZ1Bits) - 1u))];
          }
          accz = p0 + p1;
        }
        float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        groups1<M, 0>(w, lut, part);
        const float acc = (part[0] + part[1]) + (part[2] + part[3]);
        // the tile's scores as a ranged buffer: every lane stores, keys past
        // n are dropped (a store under a branch would make the next wait
        // cover it)
        const int64_t t0k = tile * NT;
        const int rows = a.n - t0k < NT ? static_cast<int>(a.n - t0k) : NT;
        const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.scores + static_cast<int64_t>(qg) * a.ld_scores + t0k, rows * 4);
        float v = nrm * fmaf(g, accz, acc);
        if (a.accumulate) v += load_f32_rsrc(sr, 4 * threadIdx.x);
        store_f32_rsrc(v, sr, 4 * threadIdx.x);
      }
      return;
    }
  }
  float *lut = dyn_lut;
  const float *qb = a.qrot + static_cast<int64_t>(qg) * a.d;
  const float *sb = PROD ? a.sq + static_cast<int64_t>(qg) * a.d : nullptr;
  if (nchunks == 1) build(0, lut, qb, sb);
  for (int64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
    const int64_t kl = tile * NT + threadIdx.x;       // key within the group
    const bool live = kl < a.n;
    const int64_t kk = key0 + (live ? kl : 0);
    float acc = 0.0f, accz = 0.0f;
    for (int c = 0; c < nchunks; ++c) {
      if (nchunks > 1) build(c, lut, qb, sb);
      if constexpr (M >= 1) {
        uint32_t w[4 * M];
        const uint4 *src = reinterpret_cast<const uint4 *>(a.codes) + (kk * rec_words + 4 * M * c) / 4;
#pragma unroll
        for (int i = 0; i < M; ++i) {
          const uint4 v = src[i];
          w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
        }
        float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        groups1<M, 0>(w, lut, part);
        acc += (part[0] + part[1]) + (part[2] + part[3]);
      }
      if constexpr (PROD) {
        const uint4 zv = reinterpret_cast<const uint4 *>(a.qjl)[(kk * z_words + 4 * c) / 4];
        const uint32_t zw[4] = {zv.x, zv.y, zv.z, zv.w};
        const float *lz = lut + S::ENTRIES;
        float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
        for (int k = 0; k < 128 / kZ1Bits; k += 2) {
          constexpr int per = 32 / kZ1Bits;
          p0 += lz[(k << kZ1Bits) + ((zw[k / per] >> (kZ1Bits * (k % per))) & ((1u << kZ1Bits) - 1u))];
          p1 += lz[((k + 1) << kZ1Bits) + ((zw[(k + 1) / per] >> (kZ1Bits * ((k + 1) % per))) & ((1u << kZ1Bits) - 1u))];
        }
        accz += p0 + p1;
      }
    }
    if (live) {
      const float nrm = a.norms[kk];
      const float g = PROD ? a.rnorms[kk] * zs : 0.0f;
      put_score(a, static_cast<int64_t>(qg) * a.ld_scores + kl, nrm * fmaf(g, accz, acc));
    }
  }
}

// ------------------------------------------------------------ four queries

template <int M, bool PROD>
constexpr bool static_lut4() { return RecStage<M>::kOn && entries4<M, PROD>() * 16 <= kStaticLutBytes; }

// blockIdx.y = g * qblocks + qb: queries qb*4 .. qb*4+3 of group g.
template <int M, bool PROD, int NT>
__global__ void __launch_bounds__(NT) score4_kernel(ScoreArgs a) {
  extern __shared__ __attribute__((aligned(16))) float4 dyn_lut4[];
  constexpr bool kStatic = static_lut4<M, PROD>();
  __shared__ __attribute__((aligned(16))) float4 st_lut4[kStatic ? entries4<M, PROD>() : 1];
  using S = Shape4<M>;
  constexpr int K = 1 << M;
  constexpr int E = entries4<M, PROD>();
  __shared__ float cb[K > 1 ? K : 2];
  if constexpr (M >= 1) {
    for (int k = threadIdx.x; k < K; k += NT) cb[k] = a.centroids[k];
  }
  const int qblocks = (a.nq + 3) / 4;
  const int64_t grp = blockIdx.y / qblocks;
  const int qb = blockIdx.y - static_cast<int>(grp) * qblocks;
  const int q0 = qb * 4;                              // within the group
  const int nchunks = a.d / kChunk;
  const int64_t tiles = (a.n + NT - 1) / NT;
  const float zs = kQjlScale / static_cast<float>(a.d);
  const size_t rec_words = static_cast<size_t>(M) * a.d / 32;
  const size_t z_words = static_cast<size_t>(a.d) / 32;
  const int64_t key0 = grp * a.n;
  const int64_t qrow0 = grp * a.nq + q0;              // query row over all groups

  // qb: rotated coordinates of query q0 (row stride qs), sb: its S q'
  auto build = [&](int c, float4 *lut4, const float *qb, int64_t qs, const float *sb) {
    __syncthreads();
    for (int i = threadIdx.x; i < E; i += NT) {
      float v4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (q0 + q >= a.nq) continue;
        float val = 0.0f;
        if (i < S::ENTRIES) {
          if constexpr (M >= 1) {
            const int t = i >> S::W;
            const int v = i & ((1 << S::W) - 1);
            const float *qp = qb + q * qs + c * kChunk + t * S::G;
#pragma unroll
            for (int u = 0; u < S::G; ++u) val = fmaf(qp[u], cb[(v >> (M * u)) & (K - 1)], val);
          }
        } else {
          const int rz = i - S::ENTRIES;
          const int k = rz >> 4;
          const int v = rz & 15;
          const float *sq = sb + q * qs + c * kChunk + 4 * k;
#pragma unroll
          for (int t = 0; t < 4; ++t) val += ((v >> t) & 1) ? sq[t] : -sq[t];
        }
        v4[q] = val;
      }
      lut4[i] = make_float4(v4[0], v4[1], v4[2], v4[3]);
    }
    __syncthreads();
  };

  using RS = RecStage<M>;
  if constexpr (RS::kOn) {
    if (nchunks == 1) {
      // d = 128: the block rotates its queries itself; each wave's records
      // go straight from HBM into its LDS stage, next tile in flight
      using RD = RecDma<M>;
      float4 *lut4 = kStatic ? st_lut4 : dyn_lut4;
      __shared__ __attribute__((aligned(16))) float qr_lds[4][128];
      __shared__ __attribute__((aligned(16))) float sq_lds[PROD ? 4 : 1][128];
      __shared__ __attribute__((aligned(16))) uint32_t rstage[(NT / 64) * RD::kWaveDwords];
      const int lane = threadIdx.x & 63;
      const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: so is the stage base
      uint32_t *ws = rstage + wv * RD::kWaveDwords;
      uint4 nz = make_uint4(0, 0, 0, 0);
      float nn = 0.0f, ng = 0.0f;
      auto issue = [&](int64_t t) {
        const int64_t k0 = t * NT + wv * 64;
        RD::issue(a.codes, key0 + k0, a.n - k0, lane, ws);
        const int64_t kl = t * NT + threadIdx.x;
        const int64_t kk = key0 + (kl < a.n ? kl : 0);
        nn = a.norms[kk];
        if constexpr (PROD) {
          ng = a.rnorms[kk];
          nz = load_nt16(a.qjl + kk * 16);
        }
      };
      int64_t tile = blockIdx.x;
      if (tile < tiles) issue(tile);                 // in flight during the query set-up
      const int nqb = a.nq - q0 < 4 ? a.nq - q0 : 4;
      if (wv < nqb) rotate_query128(a.q + (qrow0 + wv) * a.ldq, a.d_in, a.rot_kind, a.signs, a.rot, qr_lds[wv], lane);
      if constexpr (PROD) {
        __shared__ __attribute__((aligned(16))) float sq_part[(NT / 128) * 4][128];
        __syncthreads();
        sq_rows128<NT, 4>(a.qjl_s, qr_lds, sq_lds, sq_part, nqb);
      }
      build(0, lut4, &qr_lds[0][0], 128, &sq_lds[0][0]);
      for (; tile < tiles; tile += gridDim.x) {
        // this tile's records have landed; with four live queries the
        // previous tile's four score stores, the accesses issued after them,
        // may still be in flight.  The stage is read, then refilled.
        if (nqb == 4) {
          asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
        } else {
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        uint32_t w[4 * M];
        RD::get(ws, lane, w);
        const float nrm = nn;
        const float g = PROD ? ng * zs : 0.0f;
        const uint4 zv = nz;
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (tile + gridDim.x < tiles) issue(tile + gridDim.x);
        float4 accz = make_float4(0.f, 0.f, 0.f, 0.f);
        if constexpr (PROD) {
          const uint32_t zw[4] = {zv.x, zv.y, zv.z, zv.w};
          float4 part[2] = {make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)};
          nibbles4<0>(zw, lut4 + S::ENTRIES, part);
          add4(accz, part[0]);
          add4(accz, part[1]);
        }
        float4 part[2] = {make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)};
        groups4<M, 0>(w, lut4, part);
        float4 acc = part[0];
        add4(acc, part[1]);
        // each query's scores of the tile as a ranged buffer (keys past n
        // dropped), so every lane stores without a branch
        const int64_t t0k = tile * NT;
        const int rows = a.n - t0k < NT ? static_cast<int>(a.n - t0k) : NT;
        const float r[4] = {nrm * fmaf(g, accz.x, acc.x), nrm * fmaf(g, accz.y, acc.y),
                            nrm * fmaf(g, accz.z, acc.z), nrm * fmaf(g, accz.w, acc.w)};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (q < nqb) {
            const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.scores + (qrow0 + q) * a.ld_scores + t0k, rows * 4);
            float v = r[q];
            if (a.accumulate) v += load_f32_rsrc(sr, 4 * threadIdx.x);
            store_f32_rsrc(v, sr, 4 * threadIdx.x);
          }
        }
      }
      return;
    }
  }
  float4 *lut4 = dyn_lut4;
  const float *qw = a.qrot + qrow0 * a.d;
  const float *sw = PROD ? a.sq + qrow0 * a.d : nullptr;
  if (nchunks == 1) build(0, lut4, qw, a.d, sw);
  for (int64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
    const int64_t kl = tile * NT + threadIdx.x;
    const bool live = kl < a.n;
    const int64_t kk = key0 + (live ? kl : 0);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f), accz = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int c = 0; c < nchunks; ++c) {
      if (nchunks > 1) build(c, lut4, qw, a.d, sw);
      if constexpr (M >= 1) {
        uint32_t w[4 * M];
        const uint4 *src = reinterpret_cast<const uint4 *>(a.codes) + (kk * rec_words + 4 * M * c) / 4;
#pragma unroll
        for (int i = 0; i < M; ++i) {
          const uint4 v = src[i];
          w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
        }
        float4 part[2] = {make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)};
        groups4<M, 0>(w, lut4, part);
        add4(acc, part[0]);
        add4(acc, part[1]);
      }
      if constexpr (PROD) {
        const uint4 zv = reinterpret_cast<const uint4 *>(a.qjl)[(kk * z_words + 4 * c) / 4];
        const uint32_t zw[4] = {zv.x, zv.y, zv.z, zv.w};
        float4 part[2] = {make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)};
        nibbles4<0>(zw, lut4 + S::ENTRIES, part);
        add4(accz, part[0]);
        add4(accz, part[1]);
      }
    }
    if (live) {
      const float nrm = a.norms[kk];
      const float g = PROD ? a.rnorms[kk] * zs : 0.0f;
      const float r[4] = {nrm * fmaf(g, accz.x, acc.x), nrm * fmaf(g, accz.y, acc.y),
                          nrm * fmaf(g, accz.z, acc.z), nrm * fmaf(g, accz.w, acc.w)};
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (q0 + q < a.nq) put_score(a, (qrow0 + q) * a.ld_scores + kl, r[q]);
    }
  }
}

// ------------------------------------------------------------ up to four queries on the int8 matrix cores

// Two or more queries against keys with 0..2 code bits: the estimate on the
// int8 matrix cores (the fixed-point form described with i8_query_operands).

constexpr int kThreadsI = 1024;
constexpr int kTileI = 4;                      // key groups of 16 per wave step (a tile)

template <int M, bool PROD>
__global__ void __launch_bounds__(kThreadsI) score4i_kernel(ScoreArgs a) {
  static_assert(M <= 2 && (M >= 1 || PROD), "0..2 code bits");
  constexpr int NW = kThreadsI / 64;
  // A operands in lane order: [operand][lane][16 bytes]: operands 0..3 the
  // mse weights (m = 2: L of code word 0, L of word 1, M of word 0, M of
  // word 1; m = 1: even and odd plane bits), 4, 5 the QJL weights (even and
  // odd plane bits)
  constexpr int kOps = kI8Ops;
  __shared__ __attribute__((aligned(16))) float qr_lds[4][128];
  __shared__ __attribute__((aligned(16))) float sq_lds[PROD ? 4 : 1][128];
  __shared__ __attribute__((aligned(16))) float sq_part[PROD ? (kThreadsI / 128) * 4 : 1][128];
  __shared__ __attribute__((aligned(16))) uint32_t a_lds[kOps][64][4];
  __shared__ float vmax[8];
  __shared__ float vsum[8];
  static_assert(kThreadsI == 1024, "S q' takes one thread per (row, column part)");

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kb = lane >> 4;                  // B operand: coordinates 32 kb .. ; output: query kb
  const int key = lane & 15;
  const int qblocks = (a.nq + 3) / 4;
  const int64_t grp = blockIdx.y / qblocks;
  const int q0 = (blockIdx.y - static_cast<int>(grp) * qblocks) * 4;
  const int nqb = a.nq - q0 < 4 ? a.nq - q0 : 4;
  const int64_t qrow0 = grp * a.nq + q0;
  const int64_t key0 = grp * a.n;
  constexpr int kRec = M * 16;               // record bytes

  // ---- the wave's first two tiles in flight during the query set-up.
  // Register slots form a ring of three: while one tile is computed the next
  // two are in flight (each wave has only a few tiles, so one tile ahead
  // would leave a full memory latency per tile).
  constexpr int kSlots = 3;
  const int64_t tiles = (a.n + 16 * kTileI - 1) / (16 * kTileI);
  const int64_t tstride = static_cast<int64_t>(gridDim.x) * NW;
  int64_t tile = static_cast<int64_t>(blockIdx.x) * NW + wv;
  uint32_t cw[kSlots][kTileI][M == 2 ? 2 : 1], zw[kSlots][kTileI];
  float nv[kSlots], gv[kSlots];              // lane l: key l of the tile
  auto issue = [&](int64_t t, int slot) {
    // ranged buffers over the tile: keys past n read as zero; a tile past
    // the end is an empty buffer (no memory traffic)
    const int64_t k0 = t * 16 * kTileI;
    const int64_t left = a.n - k0;
    const int live = left <= 0 ? 0 : left < 16 * kTileI ? static_cast<int>(left) : 16 * kTileI;
    const int64_t kk = key0 + (live > 0 ? k0 : 0);
#pragma unroll
    for (int gi = 0; gi < kTileI; ++gi) {
      const int kr = 16 * gi + key;
      if constexpr (M == 2) {
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(a.codes + kk * kRec, live * kRec);
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rc, kr * kRec + 8 * kb, 0, 2);
        cw[slot][gi][0] = v.x;
        cw[slot][gi][1] = v.y;
      } else if constexpr (M == 1) {
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(a.codes + kk * kRec, live * kRec);
        cw[slot][gi][0] = __builtin_amdgcn_raw_buffer_load_b32(rc, kr * kRec + 4 * kb, 0, 2);
      }
      if constexpr (PROD) {
        const __amdgpu_buffer_rsrc_t rz = make_rsrc(a.qjl + kk * 16, live * 16);
        zw[slot][gi] = __builtin_amdgcn_raw_buffer_load_b32(rz, kr * 16 + 4 * kb, 0, 2);
      }
    }
    nv[slot] = load_f32_rsrc(make_rsrc(a.norms + kk, live * 4), 4 * lane);
    if constexpr (PROD) gv[slot] = load_f32_rsrc(make_rsrc(a.rnorms + kk, live * 4), 4 * lane);
  };
  // the set-up's own loads (a query row per wave, the thread's words of S)
  // go first, so they are not queued behind the key stream
  QueryLanes ql;
  if (wv < nqb) ql = load_query128(a.q + (qrow0 + wv) * a.ldq, a.d_in, a.rot_kind, a.signs, a.rot, lane);
  uint4 sw[2];
  if constexpr (PROD) sq_words1024(a.qjl_s, sw);
  issue(tile, 0);
  issue(tile + tstride, 1);

  // ---- q' = Pi q (one wave per query) and S q'
  if (wv < nqb) rotate_loaded128(ql, a.rot_kind, qr_lds[wv], lane);
  __syncthreads();
  if constexpr (PROD) {
    sq_rows1024_from(sw, qr_lds, sq_lds, sq_part, nqb);
    __syncthreads();
  }

  // ---- fixed-point weights of the block's queries
  float cA = 0.0f, cB = 0.0f;
  i8_coefs<M>(a.centroids, cA, cB);
  i8_query_operands<M, PROD, kThreadsI>(qr_lds, sq_lds, nqb, cA, cB, a_lds, vmax, vsum);
  uint32_t aop[kOps][4];
#pragma unroll
  for (int o = 0; o < kOps; ++o)
#pragma unroll
    for (int i = 0; i < 4; ++i) aop[o][i] = a_lds[o][lane][i];
  // constants of query kb: est = n (cm D_mse + cc + g zs (cz D_z + cz0))
  const float cm = i8_scale(vmax[kb]);
  const float cc = i8_offset<M>(a.centroids, vsum[kb]);
  const float cz = 2.0f * i8_scale(vmax[4 + kb]), cz0 = -vsum[4 + kb];
  const float zs = kQjlScale / 128.0f;

  // ---- stream the keys, tile by tile; the tile two ahead is issued before
  // this one is computed
  auto step = [&](const int slot) {
    const int64_t k0 = tile * 16 * kTileI;
    issue(tile + 2 * tstride, (slot + 2) % kSlots);
    float out[kTileI];
#pragma unroll
    for (int gi = 0; gi < kTileI; ++gi) {
      float est = cc;
      if constexpr (M >= 1) {
        i32x4 dm = {0, 0, 0, 0};
        uint32_t bt[4];
        if constexpr (M == 2) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            bytes_of<false>(cw[slot][gi][h], bt);
            dm = mfma_i8(aop[h], bt, dm);
            bytes_of<true>(cw[slot][gi][h], bt);
            dm = mfma_i8(aop[2 + h], bt, dm);
          }
        } else {
          bytes_of<false>(cw[slot][gi][0], bt);
          dm = mfma_i8(aop[0], bt, dm);
          bytes_of<true>(cw[slot][gi][0], bt);
          dm = mfma_i8(aop[1], bt, dm);
        }
        est = fmaf(cm, digits(dm), est);
      }
      if constexpr (PROD) {
        i32x4 dz = {0, 0, 0, 0};
        uint32_t bt[4];
        bytes_of<false>(zw[slot][gi], bt);
        dz = mfma_i8(aop[4], bt, dz);
        bytes_of<true>(zw[slot][gi], bt);
        dz = mfma_i8(aop[5], bt, dz);
        est = fmaf(__shfl(gv[slot], 16 * gi + key) * zs, fmaf(cz, digits(dz), cz0), est);
      }
      out[gi] = __shfl(nv[slot], 16 * gi + key) * est;
    }
    // query kb's scores of the tile through one ranged buffer over the
    // block's rows from this tile on; keys past n and absent queries get an
    // offset past its end (dropped), so no lane branches
    const int64_t left = a.n - k0;
    const int live = left < 16 * kTileI ? static_cast<int>(left) : 16 * kTileI;
    const int64_t span = static_cast<int64_t>(nqb - 1) * a.ld_scores + live;
    const __amdgpu_buffer_rsrc_t so = make_rsrc(a.scores + qrow0 * a.ld_scores + k0, static_cast<int>(span * 4));
#pragma unroll
    for (int gi = 0; gi < kTileI; ++gi) {
      const int kr = 16 * gi + key;
      const int off = (kb < nqb && kr < live) ? static_cast<int>((kb * a.ld_scores + kr) * 4) : 0x7FFFFFF0;
      float val = out[gi];
      if (a.accumulate) val += load_f32_rsrc(so, off);
      store_f32_rsrc(val, so, off);
    }
    tile += tstride;
  };
  while (tile < tiles) {
    step(0);
    if (tile >= tiles) break;
    step(1);
    if (tile >= tiles) break;
    step(2);
  }
}

// ------------------------------------------------------------ small d

// d < 128: one lane per key, a loop over coordinates; blockIdx.y = group.
__global__ void __launch_bounds__(kThreads) score_small_kernel(ScoreArgs a) {
  __shared__ float cb[256];
  __shared__ float qs[2 * 64];
  const int K = a.m > 0 ? (1 << a.m) : 0;
  for (int k = threadIdx.x; k < K; k += kThreads) cb[k] = a.centroids[k];
  const float zs = kQjlScale / static_cast<float>(a.d);
  const size_t rec_bytes = static_cast<size_t>(a.m) * a.d / 8;
  const int64_t grp = blockIdx.y;
  for (int qi = 0; qi < a.nq; ++qi) {
    const int64_t qr = grp * a.nq + qi;
    __syncthreads();
    for (int j = threadIdx.x; j < a.d; j += kThreads) {
      qs[j] = a.qrot[qr * a.d + j];
      qs[64 + j] = a.prod ? a.sq[qr * a.d + j] : 0.0f;
    }
    __syncthreads();
    for (int64_t kl = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; kl < a.n;
         kl += static_cast<int64_t>(gridDim.x) * kThreads) {
      const int64_t key = grp * a.n + kl;
      float acc = 0.0f, accz = 0.0f;
      if (a.m > 0) {
        const uint8_t *rec = a.codes + key * rec_bytes;
        for (int j = 0; j < a.d; ++j) {
          int idx = 0;
          for (int p = 0; p < a.m; ++p) {
            const int s = a.m * j + p;
            idx |= ((rec[s >> 3] >> (s & 7)) & 1) << p;
          }
          acc = fmaf(qs[j], cb[idx], acc);
        }
      }
      if (a.prod) {
        const uint8_t *zr = a.qjl + key * (a.d / 8);
        for (int i = 0; i < a.d; ++i) accz += ((zr[i >> 3] >> (i & 7)) & 1) ? qs[64 + i] : -qs[64 + i];
      }
      const float g = a.prod ? a.rnorms[key] * zs : 0.0f;
      put_score(a, qr * a.ld_scores + kl, a.norms[key] * fmaf(g, accz, acc));
    }
  }
}

// s = S q' for every query: one wave per (query, output row), lanes over the
// row, then a wave sum.
__global__ void __launch_bounds__(kThreads) sq_kernel(SqArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t item = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  if (item >= static_cast<int64_t>(a.nq) * a.d) return;
  const int qi = static_cast<int>(item / a.d);
  const int o = static_cast<int>(item - static_cast<int64_t>(qi) * a.d);
  const uint16_t *srow = a.qjl_s + static_cast<int64_t>(o) * a.d;
  const float *q = a.qrot + static_cast<int64_t>(qi) * a.d;
  float acc = 0.0f;
  for (int j = lane; j < a.d; j += 64) acc = fmaf(__uint_as_float(static_cast<uint32_t>(srow[j]) << 16), q[j], acc);
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) a.sq[item] = acc;
}

hipError_t set_lds(const void *fn, size_t bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
}

// Key tiles per workgroup of nt threads: about `target` workgroups over the
// whole grid, so that each one's set-up (tables, and at d = 128 the query
// rotation) is spread over several tiles.
unsigned key_blocks(const ScoreArgs &a, int64_t ysize, int nt, int64_t target) {
  const int64_t tiles = (a.n + nt - 1) / nt;
  int64_t gx = (target + ysize - 1) / ysize;
  if (gx < 1) gx = 1;
  if (gx > tiles) gx = tiles;
  return static_cast<unsigned>(gx);
}

// d = 128 with 1..4 code bits: the kernels rotate their own queries, with
// larger workgroups that share one set-up -- 512 threads for one query (about
// twelve workgroups per CU on MI355X's 256 CUs: a sweep of 768..8,192 put
// 3,072 about 3 % ahead of 1,536), 1024 for four (one per CU, the best of
// 128..2,048).
constexpr int kThreads1 = 512, kBlocks1 = 3072;
constexpr int kThreads4 = 1024, kBlocks4 = 256;

template <int M, bool PROD>
int launch1(const ScoreArgs &a, hipStream_t s) {
  const int64_t ys = static_cast<int64_t>(a.nq) * a.groups;
  if constexpr (M >= 1 && M <= 4) {
    if (score_prep_in_kernel(a.d, a.m)) {
      const size_t lds = static_lut1<M, PROD>() ? 0 : static_cast<size_t>(floats1<M, PROD>()) * sizeof(float);
      const void *fn = reinterpret_cast<const void *>(&score1_kernel<M, PROD, kThreads1>);
      const hipError_t e = set_lds(fn, lds);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((score1_kernel<M, PROD, kThreads1>),
                         dim3(key_blocks(a, ys, kThreads1, kBlocks1), static_cast<unsigned>(ys)), dim3(kThreads1),
                         lds, s, a);
      return hipGetLastError();
    }
  }
  const size_t lds = static_cast<size_t>(floats1<M, PROD>()) * sizeof(float);
  const void *fn = reinterpret_cast<const void *>(&score1_kernel<M, PROD, kThreads>);
  const hipError_t e = set_lds(fn, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((score1_kernel<M, PROD, kThreads>),
                     dim3(key_blocks(a, ys, kThreads, 2048), static_cast<unsigned>(ys)), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <int M, bool PROD>
int launch4(const ScoreArgs &a, hipStream_t s) {
  const int64_t ys = static_cast<int64_t>((a.nq + 3) / 4) * a.groups;
  if constexpr (M <= 2 && (M >= 1 || PROD)) {
    // (its score stores address four rows with 32-bit byte offsets)
    if (a.d == kChunk && a.ld_scores < (int64_t{1} << 26)) {
      // 0..2 code bits at d = 128: the digit sums on the int8 matrix cores,
      // one 16-wave workgroup per CU over all query blocks
      const int64_t tiles = (a.n + 16 * kTileI - 1) / (16 * kTileI);
      const unsigned gx = key_blocks(a, ys, kThreadsI, 256);
      const unsigned gxw = static_cast<unsigned>((tiles + kThreadsI / 64 - 1) / (kThreadsI / 64));
      hipLaunchKernelGGL((score4i_kernel<M, PROD>), dim3(gx < gxw ? gx : gxw, static_cast<unsigned>(ys)),
                         dim3(kThreadsI), 0, s, a);
      return hipGetLastError();
    }
  }
  if constexpr (M >= 1 && M <= 4) {
    if (score_prep_in_kernel(a.d, a.m)) {
      const size_t lds = static_lut4<M, PROD>() ? 0 : static_cast<size_t>(entries4<M, PROD>()) * sizeof(float4);
      const void *fn = reinterpret_cast<const void *>(&score4_kernel<M, PROD, kThreads4>);
      const hipError_t e = set_lds(fn, lds);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((score4_kernel<M, PROD, kThreads4>),
                         dim3(key_blocks(a, ys, kThreads4, kBlocks4), static_cast<unsigned>(ys)), dim3(kThreads4),
                         lds, s, a);
      return hipGetLastError();
    }
  }
  const size_t lds = static_cast<size_t>(entries4<M, PROD>()) * sizeof(float4);
  const void *fn = reinterpret_cast<const void *>(&score4_kernel<M, PROD, kThreads>);
  const hipError_t e = set_lds(fn, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((score4_kernel<M, PROD, kThreads>),
                     dim3(key_blocks(a, ys, kThreads, 2048), static_cast<unsigned>(ys)), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <int M, bool PROD>
int launch_m(const ScoreArgs &a, hipStream_t s) {
  if constexpr (M <= 5) {
    if (a.nq >= 2) return launch4<M, PROD>(a, s);
  }
  return launch1<M, PROD>(a, s);
}

}  // namespace

int launch_score(const ScoreArgs &a, void *stream) {
  (void)hipGetLastError();   // report only errors of this launch
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (a.d < kChunk) {
    int64_t blocks = (a.n + kThreads - 1) / kThreads;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(score_small_kernel, dim3(static_cast<unsigned>(blocks), static_cast<unsigned>(a.groups)),
                       dim3(kThreads), 0, s, a);
    return hipGetLastError();
  }
  if (a.prod) {
    switch (a.m) {
      case 0: return launch_m<0, true>(a, s);
      case 1: return launch_m<1, true>(a, s);
      case 2: return launch_m<2, true>(a, s);
      case 3: return launch_m<3, true>(a, s);
      case 4: return launch_m<4, true>(a, s);
      case 5: return launch_m<5, true>(a, s);
      case 6: return launch_m<6, true>(a, s);
      case 7: return launch_m<7, true>(a, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (a.m) {
    case 1: return launch_m<1, false>(a, s);
    case 2: return launch_m<2, false>(a, s);
    case 3: return launch_m<3, false>(a, s);
    case 4: return launch_m<4, false>(a, s);
    case 5: return launch_m<5, false>(a, s);
    case 6: return launch_m<6, false>(a, s);
    case 7: return launch_m<7, false>(a, s);
    case 8: return launch_m<8, false>(a, s);
    default: return hipErrorInvalidValue;
  }
}

int launch_sq(const SqArgs &a, void *stream) {
  (void)hipGetLastError();   // report only errors of this launch
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t items = static_cast<int64_t>(a.nq) * a.d;
  const int64_t blocks = (items + 3) / 4;
  hipLaunchKernelGGL(sq_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace tq

namespace tq {

bool score_prep_in_kernel(int d, int m) { return d == kChunk && m >= 1 && m <= 4; }

}  // namespace tq
