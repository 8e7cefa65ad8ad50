// Inner-product estimator for many queries on the matrix cores (gfx950).
//
// Sources: "TurboQuant: Online Vector Quantization" paper summary (Jump2Paper
// Archive) -- the estimator <y, Q^-1(Q(x))> of the definitions table for
// TurboQuant_mse keys, and the nearest-neighbour search application, where a
// batch of queries is scored against the whole quantised database.
//
// For Q queries against n keys the estimates form the product
//   est[q][k] = n_k * sum_j q'_j c[idx_kj],
// a dense contraction over the d rotated coordinates, which runs here on
// v_mfma_f32_16x16x32_f16.  Float16 alone is too coarse for a float32-level
// estimate, so both operands are split exactly enough: each query row and the
// codebook are scaled by a power of two into [0.5, 1) and written as hi + lo
// float16 parts, and three products hi*hi + hi*lo + lo*hi are accumulated in
// float32 (the dropped lo*lo term is about 2^-22 of the product).
//
// Tile: 16 QT queries (QT = 2 or 4 tiles of 16) x 512 keys, eight waves of
// 16 QT x 64.  Per chunk of 128 coordinates the workgroup loads the queries'
// hi and lo parts straight into LDS, and each wave its 64 key records (direct
// loads, the next chunk in flight while this one is multiplied).  The
// workgroups are persistent, one per resident slot, and stream their tiles
// chunk after chunk.  Query and key loads keep the normal cache policy: every
// key block serves all the query blocks (those on one XCD share its L2), and
// the query rows serve every key block.
//
// Within a chunk, k-step s of lane group g takes coordinates 32 g + 8 s ..
// 32 g + 8 s + 7 (the A and B operands agree on it, and the contraction does
// not care about the order), so a lane reads its key's 32 coordinates of
// codes once per chunk.  The key operand is built from small tables of the
// codes' float16 (hi, lo) values, laid out so that each lane reads its own
// LDS bank whatever the code: an entry is repeated once per lane (m <= 2:
// entries of 4 / m coordinates, hi and lo tables; m >= 3: one code's
// (hi | lo << 16) dword, and the two halves of a coordinate pair are put
// together with v_perm_b32).  The next k-step's key operands are looked up
// while the current one multiplies.

#include <hip/hip_runtime.h>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kKT = kScoreMKeys;   // keys per workgroup: 64 per wave, four 16-column tiles
constexpr int kCC = 128;           // coordinates per staged chunk (four k-steps of 32)
static_assert(kKT == 64 * kWaves, "a wave per 64 keys");

__device__ __forceinline__ uint32_t f16_bits(_Float16 h) {
  uint16_t b;
  __builtin_memcpy(&b, &h, 2);
  return b;
}

// One wave per query row: max |q'_j| -> scale 2^-e putting it in [0.5, 1),
// then hi = f16(q' 2^-e), lo = f16(q' 2^-e - hi).
__global__ void __launch_bounds__(kThreads) qsplit_kernel(QSplitArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  const float *q = a.qrot + row * a.d;
  float mx = 0.0f;
  for (int j = lane; j < a.d; j += 64) mx = fmaxf(mx, fabsf(q[j]));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  int e = 0;
  if (mx > 0.0f) (void)frexpf(mx, &e);
  const float s = ldexpf(1.0f, -e);
  for (int j = lane; j < a.d; j += 64) {
    const float v = q[j] * s;
    const _Float16 h = static_cast<_Float16>(v);
    const _Float16 l = static_cast<_Float16>(v - static_cast<float>(h));
    a.qh[row * a.d + j] = static_cast<uint16_t>(f16_bits(h));
    a.ql[row * a.d + j] = static_cast<uint16_t>(f16_bits(l));
  }
  if (lane == 0) a.qinv[row] = ldexpf(1.0f, e);
}

// 16 bytes from p straight into LDS with the normal cache policy (lane l at
// lds_base + 16 l; lds_base the same on every lane; counted in vmcnt).
__device__ __forceinline__ void load_lds16(const void *p, void *lds_base) {
  __builtin_amdgcn_global_load_lds((glb_void_t *)p, (lds_void_t *)lds_base, 16, 0, 0);
}
// 4 bytes from p straight into LDS (lane l at lds_base + 4 l).
__device__ __forceinline__ void load_lds4(const void *p, void *lds_base) {
  __builtin_amdgcn_global_load_lds((glb_void_t *)p, (lds_void_t *)lds_base, 4, 0, 0);
}

// A tile's scales in LDS: its keys' norms (64 per wave), then 64 query
// rows' 2^e and 64 rows' tau.
constexpr int kScaleFloats = kKT + 64 + 64;
constexpr int kScaleBytes = kScaleFloats * 4;
// A wave's stage for score rows: 8 rows of its 64 keys (rows of 68 floats:
// the lanes' 4-byte writes and 16-byte reads fall in distinct banks).
constexpr int kOutRow = 64 + 4;
constexpr int kOutStageBytes = 8 * kOutRow * 4;

// The per-lane code tables.  Entry e sits at e * 256 + lane slot, so the
// lanes of one read hit distinct banks whatever entries they ask for.
//   m = 1: e = 4 codes (4 coordinates), 8 bytes of float16 per part, 32 slots
//   m = 2: e = 2 codes, 4 bytes per part, 64 slots
//   m >= 3: e = 1 code, (hi | lo << 16), 64 slots
// The lo table (m <= 2) starts 4096 + one slot after the hi table: the
// same lane then reads bank l + 1, and the distance is no multiple that lets
// the compiler pair a hi and a lo read into one instruction (which would
// land them in neighbouring registers instead of the operands' own).
template <int M>
struct KeyTab {
  static constexpr int kE = M <= 2 ? 16 : (1 << M);
  static constexpr int kSlot = M == 1 ? 8 : 4;
  static constexpr int kSlots = 256 / kSlot;
  static constexpr int kLo = M <= 2 ? 4096 + kSlot : 0;
  static constexpr int kBytes = M <= 2 ? kLo + kE * 256 : kE * 256;
};

// s_waitcnt vmcnt(N) lgkmcnt(0): at most N vector memory operations of the
// wave still in flight (they complete in issue order), none of LDS
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// (byte k of x) * 256 + base for base < 256: one v_perm_b32 (selector bytes:
// base's byte 0, x's byte k, zero, zero)
__device__ __forceinline__ uint32_t entry_addr(uint32_t x, int k, uint32_t base) {
  return __builtin_amdgcn_perm(x, base, 0x0C0C0400u | (static_cast<uint32_t>(k) << 8));
}

// code of coordinate u (0 .. 31) of a lane's 4 M bytes of codes
template <int M>
__device__ __forceinline__ uint32_t code_at(const uint32_t (&w)[M], int u) {
  const int bit = M * u, i = bit >> 5, sh = bit & 31;
  if (sh + M <= 32 || i + 1 >= M) return (w[i] >> sh) & ((1u << M) - 1);
  return __builtin_amdgcn_alignbit(w[i + 1], w[i], sh) & ((1u << M) - 1);
}

// a lane's 4 M bytes of codes (4 M-byte aligned in LDS) as M words
template <int M>
__device__ __forceinline__ void lane_codes(const uint8_t *p, uint32_t (&w)[M]) {
  if constexpr (M == 1) {
    w[0] = *reinterpret_cast<const uint32_t *>(p);
  } else if constexpr (M == 2) {
    const uint2 v = *reinterpret_cast<const uint2 *>(p);
    w[0] = v.x; w[1] = v.y;
  } else if constexpr (M == 4) {
    const uint4 v = *reinterpret_cast<const uint4 *>(p);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else {
#pragma unroll
    for (int i = 0; i < M; ++i) w[i] = reinterpret_cast<const uint32_t *>(p)[i];
  }
}

// Exact key values for 1 or 2 code bits.  With an odd-symmetric codebook
// there are one or two magnitudes, b (outer) >= a (inner) >= 0.  Values
// v = c / u that are exact in float16 for one float32 unit u make the key
// operand exact, so an estimate needs only the query's (hi, lo) parts times
// v: two products instead of three.  m = 1: v = +-1024.  m = 2: v_outer = P
// in [1024, 2047] and v_inner = q 2^-k with q <= 2047 the largest such
// multiple, over the P that minimises |v_inner / P - a / b| (one candidate P
// per thread, a block minimum in LDS), u = b / P.  The fit is taken only
// when delta = max_c |v_c u - c| satisfies delta sqrt(d) <= b / 150000: an
// estimate n sum_j q'_j c_j then moves by at most n delta sum_j |q'_j| <=
// n delta sqrt(d) |q'| <= n b |q'| / 150000, which for the codebooks of the
// Lemma 1 density (b sqrt(d) about 1.5 at 1 and 2 bits) is a tenth of the
// 1e-4 of n |q'| / sqrt(d) the float32 result is held to, and scales with
// the codebook otherwise.  Else (and for any codebook that is not exactly
// odd-symmetric) the caller keeps the three-product path.  Every thread of the block calls this (it holds a
// barrier); all read the same codebook, so the early returns are uniform.
template <int M>
__device__ bool exact_values(const float *c, int d, float &unit, float (&v)[1 << M]) {
  constexpr int K = 1 << M;
  __shared__ unsigned long long best;
  bool sym = true;
#pragma unroll
  for (int k = 0; k < K / 2; ++k) sym = sym && c[k] == -c[K - 1 - k];
  const double b = c[K - 1], a = M == 2 ? static_cast<double>(c[K / 2]) : 0.0;
  if (!sym || !(b >= a && a >= 0.0 && b < 1e30)) return false;
  if (b == 0.0) {
    unit = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) v[k] = 0.0f;
    return true;
  }
  int P = 1024, k2 = 0;
  double qv = 0.0;
  const double alpha = a / b;
  if constexpr (M == 2) {
    if (threadIdx.x == 0) best = ~0ull;
    __syncthreads();
    for (int p = 1024 + static_cast<int>(threadIdx.x); p < 2048; p += blockDim.x) {
      const double x = alpha * p;
      int k = 0;
      while (k < 24 && rint(ldexp(x, k + 1)) <= 2047.0) ++k;
      const double err = fabs(ldexp(rint(ldexp(x, k)), -k) / p - alpha);
      const unsigned long long key = (static_cast<unsigned long long>(__float_as_uint(static_cast<float>(err))) << 32) |
                                     (static_cast<unsigned long long>(p) << 5) | static_cast<unsigned long long>(k);
      atomicMin(&best, key);
    }
    __syncthreads();
    const unsigned long long kb = best;
    P = static_cast<int>((kb >> 5) & 2047);
    k2 = static_cast<int>(kb & 31);
    qv = ldexp(rint(ldexp(alpha * P, k2)), -k2);
  }
  unit = static_cast<float>(b / P);
  const double u = unit;
  double delta = fabs(P * u - b);
  if constexpr (M == 2) delta = fmax(delta, fabs(qv * u - a));
  if (!(delta * sqrt(static_cast<double>(d)) * 150000.0 <= b)) return false;
  v[K - 1] = static_cast<float>(P);
  v[0] = -static_cast<float>(P);
  if constexpr (M == 2) {
    v[2] = static_cast<float>(qv);
    v[1] = -static_cast<float>(qv);
  }
  return true;
}

template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

// FILT: the filtered pass (candidate lists against tau), else score rows.
template <int M, int QT, bool FILT>
__global__ void __launch_bounds__(kThreads) scorem_kernel(ScoreMArgs a) {
  constexpr int K = 1 << M;
  constexpr int CB = 16 * M;             // bytes of one key's 128-coordinate chunk
  constexpr int SB = 64 * CB;            // bytes of a wave's staged chunk
  constexpr int NQ = 16 * QT;            // queries per workgroup
  constexpr int QB = NQ * kCC * 2;       // bytes of one part (hi or lo) of a query chunk
  constexpr int RPW = NQ / kWaves;       // query rows each wave loads (2 or 8)
  using T = KeyTab<M>;
  constexpr int kTabBytes = (T::kBytes + 255) & ~255;
  // One LDS block: the code tables first, at address 0, so that a table
  // read's constant part (the lo table's distance) fits the instruction's
  // 16-bit offset; then the key stage, kWaves x two buffers; then the query
  // chunks, two buffers x (hi, lo): row r's 16-byte slot c at
  // r * 256 + 16 (c ^ (r & 15)), so a wave's operand reads hit distinct
  // banks; then the scales of three tiles (see load_scales); then each
  // wave's stage for writing score rows (see finish).
  __shared__ __attribute__((aligned(256))) uint8_t smem[kTabBytes + kWaves * 2 * SB + 2 * 2 * QB + 3 * kScaleBytes +
                                                        (FILT ? 1 : kWaves) * kOutStageBytes];
  uint8_t *const tab = smem;
  uint8_t *const stage = smem + kTabBytes;
  uint8_t *const qstage = stage + kWaves * 2 * SB;
  float *const scl = reinterpret_cast<float *>(qstage + 2 * 2 * QB);

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 15;
  const int g = lane >> 4;
  float *const ostage = scl + 3 * kScaleFloats + wv * (kOutStageBytes / 4);
  const int qblocks = (a.nq + NQ - 1) / NQ;
  const int64_t ntiles = static_cast<int64_t>(qblocks) * ((a.n_cols + kKT - 1) / kKT);
  const int64_t grp = blockIdx.y;
  const int64_t key0 = grp * a.n;                       // group's first key
  const int64_t rec_bytes = static_cast<int64_t>(M) * a.d / 8;
  const int nchunk = a.d / kCC;

  // A tile is 16 QT queries x 512 keys: tile i has query block i % qblocks
  // and key block i / qblocks.  The workgroup takes tiles blockIdx.x,
  // blockIdx.x + gridDim.x, ... (a multiple of 8 apart, so the tiles of one
  // XCD share their query blocks), streaming chunk after chunk across tile
  // boundaries: the loads of a tile's first chunk overlap the previous
  // tile's last, and the previous tile's estimates are written while the
  // next tile's first chunk is multiplied.
  struct Tile {
    int64_t kw;      // wave's first key in the group
    int64_t cw;      // its first score column
    int64_t qrow0;   // block's first query row
    int nqb;         // live queries of the block
  };
  auto tile_of = [&](int64_t i) {
    const int qb = static_cast<int>(i % qblocks);
    const int64_t kb = i / qblocks;
    Tile t;
    t.kw = kb * a.kb_stride * kKT + 64 * wv;
    t.cw = kb * kKT + 64 * wv;
    t.qrow0 = grp * a.nq + static_cast<int64_t>(qb) * NQ;
    t.nqb = a.nq - qb * NQ < NQ ? a.nq - qb * NQ : NQ;
    return t;
  };
  // the next tile from i on (stepping gridDim.x) with work to do: with
  // only_over set, the pass for rows whose candidate lists overflowed, a
  // tile works only if one of its rows did (every thread reads the same)
  auto next_tile = [&](int64_t i) {
    if (a.only_over) {
      for (; i < ntiles; i += gridDim.x) {
        const Tile t = tile_of(i);
        bool any = false;
        for (int qi = 0; qi < t.nqb; ++qi) any = any || a.only_over[t.qrow0 + qi] > a.list_cap;
        if (any) break;
      }
    }
    return i;
  };
  if (a.only_over) {
    // nothing to do unless some row of the group overflowed (one vote of
    // the block, so that passes with nothing to do end at once)
    int over = 0;
    for (int r = threadIdx.x; r < a.nq; r += kThreads) over |= a.only_over[grp * a.nq + r] > a.list_cap;
    if (!__syncthreads_or(over)) return;
  }
  int64_t cur = next_tile(blockIdx.x);
  if (cur >= ntiles || a.n <= 0) return;                 // uniform over the block

  // the code values: exact float16 multiples of one unit (m <= 2, see
  // exact_values; the lo parts are then zero), else the codebook scaled by
  // 2^-ec into [0.5, 1) as (hi, lo) float16 parts
  float xv[M <= 2 ? K : 1];
  float unit = 0.0f;
  bool exact = false;
  if constexpr (M <= 2) exact = exact_values<M>(a.centroids, a.d, unit, xv);
  float cmax = 0.0f;
#pragma unroll
  for (int k = 0; k < K; ++k) cmax = fmaxf(cmax, fabsf(a.centroids[k]));
  int ec = 0;
  if (cmax > 0.0f) (void)frexpf(cmax, &ec);
  const float cs = ldexpf(1.0f, -ec);
  auto split = [&](int code, uint32_t &h, uint32_t &l) {
    if constexpr (M <= 2) {
      if (exact) {
        h = f16_bits(static_cast<_Float16>(xv[code]));
        l = 0u;
        return;
      }
    }
    const float c = a.centroids[code] * cs;
    const _Float16 hh = static_cast<_Float16>(c);
    h = f16_bits(hh);
    l = f16_bits(static_cast<_Float16>(c - static_cast<float>(hh)));
  };
  for (int i = threadIdx.x; i < T::kE * T::kSlots; i += kThreads) {
    const int e = i / T::kSlots, at = e * 256 + (i % T::kSlots) * T::kSlot;
    if constexpr (M <= 2) {
      constexpr int CPE = 4 / M;           // coordinates per entry
      uint32_t hw[2] = {0, 0}, lw[2] = {0, 0};
#pragma unroll
      for (int u = 0; u < CPE; ++u) {
        uint32_t h, l;
        split((e >> (M * u)) & (K - 1), h, l);
        hw[u >> 1] |= h << (16 * (u & 1));
        lw[u >> 1] |= l << (16 * (u & 1));
      }
      __builtin_memcpy(tab + at, hw, T::kSlot);
      __builtin_memcpy(tab + T::kLo + at, lw, T::kSlot);
    } else {
      uint32_t h, l;
      split(e, h, l);
      *reinterpret_cast<uint32_t *>(tab + at) = h | (l << 16);
    }
  }
  const uint32_t slot_off = static_cast<uint32_t>(M == 1 ? (lane & 31) * 8 : lane * 4);

  uint8_t *st0 = stage + wv * 2 * SB;
  // chunk c of the wave's 64 records of tile t into stage buffer b, key k's
  // piece at k * CB; keys past the group's end fetch its last key
  auto issue = [&](const Tile &t, int c, int b) {
    const int64_t nlive = a.n - t.kw;                      // live keys from the wave's first on
    if (nlive <= 0) return;                                // uniform over the wave
    const uint8_t *base = a.codes + (key0 + t.kw) * rec_bytes + static_cast<int64_t>(c) * CB;
#pragma unroll
    for (int i = 0; i < M; ++i) {
      const int f = i * 64 + lane;
      const int64_t k = f / M;
      const int64_t kk = k < nlive ? k : nlive - 1;
      load_lds16(base + kk * rec_bytes + (f % M) * 16, st0 + b * SB + 1024 * i);
    }
  };
  // chunk c of query rows RPW wv .. RPW wv + RPW - 1 (hi and lo) of tile t
  // into query buffer b: a load covers 4 rows, lane l row + l / 16, slot
  // l % 16, fetching the column chunk that the slot swizzle puts there
  auto issue_q = [&](const Tile &t, int c, int b) {
#pragma unroll
    for (int h = 0; h < RPW / 4; ++h) {
      const int r = RPW * wv + 4 * h + (lane >> 4);
      const int rr = r < t.nqb ? r : t.nqb - 1;           // rows past the block's queries: a copy
      const int col = (lane & 15) ^ (r & 15);
      const int64_t off = (t.qrow0 + rr) * a.d + static_cast<int64_t>(c) * kCC + 8 * col;
      uint8_t *dst = qstage + b * 2 * QB + (RPW * wv + 4 * h) * 256;
      load_lds16(a.qh + off, dst);
      load_lds16(a.ql + off, dst + QB);
    }
  };
  static_assert(RPW % 4 == 0, "query rows per wave: whole 4-row loads");

  // the scales the estimates of tile t take, loaded into scale buffer sb
  // with its first chunk: each wave its 64 keys' norms, wave 0 the block's
  // query rows' 2^e, wave 1 their tau when filtering; indexes past the live
  // keys and rows read the last live one (never stored).  Three buffers: a
  // tile's scales are read while the next tile's first chunk runs, and the
  // buffer is loaded again only two tiles later, after a barrier.
  auto load_scales = [&](const Tile &t, int sb) {
    float *dst = scl + sb * kScaleFloats;
    const int64_t kl = t.kw + lane;
    load_lds4(a.norms + key0 + (kl < a.n ? kl : a.n - 1), dst + 64 * wv);
    const int64_t row = t.qrow0 + (lane < t.nqb ? lane : t.nqb - 1);
    if (wv == 0) load_lds4(a.qinv + row, dst + kKT);
    if (FILT && wv == 1) load_lds4(a.tau + row, dst + kKT + 64);
  };

  // this lane's query operand rows (tile qt, row j)
  int qoff[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) qoff[qt] = (16 * qt + j) * 256;

  f32x4 acc[QT][4];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[qt][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // acc[qt][t][r] = estimate of query 16 qt + 4 g + r and key 16 t + j of
  // tile tl: to the score matrix, or (filtering) to the candidate lists
  const float cinv = exact ? unit : ldexpf(1.0f, ec);
  bool ranged = false;         // the last finish left exactly its stores in flight
  auto finish = [&](const Tile &tl, int sb) {
    ranged = false;
    const float *sc = scl + sb * kScaleFloats;
    float pq[QT][4], pt[QT][4];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float4 v = *reinterpret_cast<const float4 *>(sc + kKT + 16 * qt + 4 * g);
      pq[qt][0] = v.x; pq[qt][1] = v.y; pq[qt][2] = v.z; pq[qt][3] = v.w;
      if constexpr (FILT) {
        const float4 u = *reinterpret_cast<const float4 *>(sc + kKT + 64 + 16 * qt + 4 * g);
        pt[qt][0] = u.x; pt[qt][1] = u.y; pt[qt][2] = u.z; pt[qt][3] = u.w;
      }
    }
    float nk[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) nk[t] = sc[64 * wv + 16 * t + j] * cinv;
    if constexpr (FILT) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int64_t kl = tl.kw + 16 * t + j;             // key within the group
        const int64_t col = tl.cw + 16 * t + j;            // its score column
        if (kl >= a.n || col >= a.n_cols) continue;
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int qi = 16 * qt + 4 * g + r;
            if (qi >= tl.nqb) continue;
            const int64_t row = tl.qrow0 + qi;
            const float v = acc[qt][t][r] * nk[t] * pq[qt][r];
            // a candidate (NaN never is)
            if (v >= pt[qt][r]) {
              const int slot = atomicAdd(a.cnt + row, 1);
              if (slot < a.list_cap) {
                a.list_v[row * a.list_cap + slot] = v;
                a.list_i[row * a.list_cap + slot] = static_cast<int32_t>(kl);
              }
            }
          }
      }
    } else {
      // score rows through the wave's stage, 8 rows at a time (rows 16 qt +
      // 4 g + 2 h + r', staged as row 2 g + r'), so that a lane stores 16
      // bytes of one row and an instruction writes four rows' 256-byte pieces
      // of the wave's 64 keys (whole lines), not 64 bytes of 16 rows.  When
      // the wave's 64 columns are all live and its rows fit one ranged
      // buffer, every store is issued by the whole wave (rows past the
      // block's queries get an offset past the buffer's end and are dropped),
      // so the wave knows how many stores it left in flight.
      const int c4 = 4 * (lane & 15);
      const int64_t kl0 = tl.kw + c4, col0 = tl.cw + c4;  // the lane's first key and column
      const int64_t span = (static_cast<int64_t>(tl.nqb) - 1) * a.ld_scores + 64;
      ranged = tl.kw + 64 <= a.n && tl.cw + 64 <= a.n_cols && span * 4 < (int64_t{1} << 31);
      const __amdgpu_buffer_rsrc_t so =
          make_rsrc(a.scores + tl.qrow0 * a.ld_scores + tl.cw, ranged ? static_cast<int>(span * 4) : 0);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
          for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int rr = 0; rr < 2; ++rr)
              ostage[(2 * g + rr) * kOutRow + 16 * t + j] = acc[qt][t][2 * hh + rr] * nk[t] * pq[qt][2 * hh + rr];
          wave_lds_sync();
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const int rho = 4 * i + (lane >> 4);               // staged row
            const int qi = 16 * qt + 4 * (rho >> 1) + 2 * hh + (rho & 1);
            const float4 v = *reinterpret_cast<const float4 *>(ostage + rho * kOutRow + c4);
            uint32_t w[4] = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)};
            if (ranged) {
              const int off = qi < tl.nqb ? static_cast<int>((qi * a.ld_scores + c4) * 4) : 0x7FFFFFF0;
              if (a.accumulate) {
                const u32x4 p = __builtin_amdgcn_raw_buffer_load_b128(so, off, 0, 0);
                w[0] = __float_as_uint(v.x + __uint_as_float(p.x));
                w[1] = __float_as_uint(v.y + __uint_as_float(p.y));
                w[2] = __float_as_uint(v.z + __uint_as_float(p.z));
                w[3] = __float_as_uint(v.w + __uint_as_float(p.w));
              }
              store_words_rsrc<4>(w, so, off);
            } else if (qi < tl.nqb) {
              float *dst = a.scores + (tl.qrow0 + qi) * a.ld_scores + col0;
              const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
              for (int u = 0; u < 4; ++u) {
                if (kl0 + u >= a.n || col0 + u >= a.n_cols) continue;
                dst[u] = a.accumulate ? dst[u] + vv[u] : vv[u];
              }
            }
          }
          wave_lds_sync();
        }
    }
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[qt][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  };

  // the chunk loop, with the key operand's lo part (EX = false) or without
  // it (EX = true: exact code values)
  auto run = [&](auto ex) {
    constexpr bool EX = decltype(ex)::value;
    Tile tc = tile_of(cur);
    issue_q(tc, 0, 0);
    issue(tc, 0, 0);
    int sb = 0;                  // this tile's scale buffer
    load_scales(tc, sb);
    int64_t done = -1;           // the tile whose estimates wait to be written
    for (int c = 0, b = 0;; b ^= 1) {
      // this wave's loads of this chunk have landed; after the barrier every
      // wave's have, and every wave is done with the previous chunk, whose
      // buffers then take the next (the barrier also publishes the code
      // tables)
      // (after a ranged finish, its 4 QT stores -- 8 QT operations with the
      // accumulating loads -- were issued after this chunk's loads and
      // complete after them, so they may stay in flight)
      if (!FILT && ranged) {
        if (a.accumulate) wait_vm_lgkm0<8 * QT>();
        else wait_vm_lgkm0<4 * QT>();
      } else {
        wait_vm_lgkm0<0>();
      }
      ranged = false;
      // a bare barrier: __syncthreads() would also wait for the stores (its
      // workgroup fence); LDS is ordered by the waits above, and the compiler
      // keeps memory accesses on their side of it
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      int cn = c + 1;
      int64_t nxt = cur;
      if (cn == nchunk) {
        nxt = next_tile(cur + gridDim.x);
        cn = 0;
      }
      if (nxt < ntiles) {
        const Tile tn = nxt == cur ? tc : tile_of(nxt);
        issue_q(tn, cn, b ^ 1);
        issue(tn, cn, b ^ 1);
        if (cn == 0) load_scales(tn, sb == 2 ? 0 : sb + 1);
      }
      if (done >= 0) {
        // the previous tile's estimates (issued after the loads above: the
        // count the next wait relies on)
        asm volatile("" ::: "memory");
        finish(tile_of(done), sb == 0 ? 2 : sb - 1);
        done = -1;
      }
      const uint8_t *st = st0 + b * SB;
      const uint8_t *qs = qstage + b * 2 * QB;
      // codes of this lane's 32 coordinates of keys 16 t + j
      uint32_t kc[4][M];
  #pragma unroll
      for (int t = 0; t < 4; ++t) lane_codes<M>(st + (16 * t + j) * CB + 4 * M * g, kc[t]);
      // the key operands of k-step s, hi and lo parts, for keys 16 t + j
      auto key_operands = [&](int s, f16x8 (&bh)[4], f16x8 (&bl)[4]) {
  #pragma unroll
      for (int t = 0; t < 4; ++t) {
        uint32_t hw[4], lw[4];
        if constexpr (M == 1) {
          // byte s = coordinates 8 s .. 8 s + 7: its low and high nibbles
          const uint32_t w = kc[t][0];
          const uint32_t x = w & 0x0F0F0F0Fu, y = (w >> 4) & 0x0F0F0F0Fu;
          const uint32_t e0 = entry_addr(x, s, slot_off), e1 = entry_addr(y, s, slot_off);
          const uint2 h0 = *reinterpret_cast<const uint2 *>(tab + e0);
          const uint2 h1 = *reinterpret_cast<const uint2 *>(tab + e1);
          hw[0] = h0.x; hw[1] = h0.y; hw[2] = h1.x; hw[3] = h1.y;
          if constexpr (!EX) {
            const uint2 l0 = *reinterpret_cast<const uint2 *>(tab + T::kLo + e0);
            const uint2 l1 = *reinterpret_cast<const uint2 *>(tab + T::kLo + e1);
            lw[0] = l0.x; lw[1] = l0.y; lw[2] = l1.x; lw[3] = l1.y;
          }
        } else if constexpr (M == 2) {
          // nibbles 4 (s & 1) + p of word s >> 1: coordinate pairs p
          const uint32_t w = kc[t][s >> 1];
          const uint32_t x = w & 0x0F0F0F0Fu, y = (w >> 4) & 0x0F0F0F0Fu;
  #pragma unroll
          for (int p = 0; p < 4; ++p) {
            const int k = 4 * (s & 1) + p;
            const uint32_t e = entry_addr((k & 1) ? y : x, k >> 1, slot_off);
            hw[p] = *reinterpret_cast<const uint32_t *>(tab + e);
            if constexpr (!EX) lw[p] = *reinterpret_cast<const uint32_t *>(tab + T::kLo + e);
          }
        } else {
          uint32_t ev[8];
  #pragma unroll
          for (int u = 0; u < 8; ++u) {
            uint32_t e;
            if constexpr (M == 4) {
              // nibble u of word s
              const uint32_t w = kc[t][s];
              e = entry_addr((u & 1) ? (w >> 4) & 0x0F0F0F0Fu : w & 0x0F0F0F0Fu, u >> 1, slot_off);
            } else {
              e = (code_at<M>(kc[t], 8 * s + u) << 8) | slot_off;
            }
            ev[u] = *reinterpret_cast<const uint32_t *>(tab + e);
          }
  #pragma unroll
          for (int p = 0; p < 4; ++p) {
            hw[p] = __builtin_amdgcn_perm(ev[2 * p + 1], ev[2 * p], 0x05040100u);
            lw[p] = __builtin_amdgcn_perm(ev[2 * p + 1], ev[2 * p], 0x07060302u);
          }
        }
        __builtin_memcpy(&bh[t], hw, 16);
        if constexpr (!EX) __builtin_memcpy(&bl[t], lw, 16);
      }
      };
      // k-step s + 1's key operands are looked up while k-step s multiplies
      f16x8 bh[2][4], bl[2][4];
      key_operands(0, bh[0], bl[0]);
  #pragma unroll
      for (int s = 0; s < 4; ++s) {
        f16x8 ah[QT], al[QT];
  #pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          const int slot = (4 * g + s) ^ j;                 // (16 qt + j) & 15 == j
          ah[qt] = *reinterpret_cast<const f16x8 *>(qs + qoff[qt] + 16 * slot);
          al[qt] = *reinterpret_cast<const f16x8 *>(qs + QB + qoff[qt] + 16 * slot);
        }
        if (s + 1 < 4) key_operands(s + 1, bh[(s + 1) & 1], bl[(s + 1) & 1]);
  #pragma unroll
        for (int qt = 0; qt < QT; ++qt)
  #pragma unroll
          for (int t = 0; t < 4; ++t) {
            acc[qt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[qt], bh[s & 1][t], acc[qt][t], 0, 0, 0);
            if constexpr (!EX) acc[qt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[qt], bl[s & 1][t], acc[qt][t], 0, 0, 0);
            acc[qt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[qt], bh[s & 1][t], acc[qt][t], 0, 0, 0);
          }
      }
      if (cn == 0) {
        // the tile's last chunk: its estimates are written during the next
        // tile's first chunk
        if (nxt >= ntiles) break;
        done = cur;
        cur = nxt;
        tc = tile_of(cur);
        sb = sb == 2 ? 0 : sb + 1;
      }
      c = cn;
    }
    // the last tile's scales: each wave waits for its own loads, and the
    // barrier publishes the query scales that waves 0 and 1 loaded
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    finish(tc, sb);
  };
  if constexpr (M <= 2) {
    if (exact) run(BoolC<true>{});
    else run(BoolC<false>{});
  } else {
    run(BoolC<false>{});
  }
}

// One resident workgroup per slot the device holds (a multiple of 8, one
// XCD's share each), or one per tile when there are fewer tiles.
template <int M, int QT, bool FILT>
int launch_mq(const ScoreMArgs &a, hipStream_t s) {
  static const int64_t slots = [] {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(&scorem_kernel<M, QT, FILT>),
                                                     kThreads, 0) != hipSuccess)
      return int64_t{0};
    const int64_t n = static_cast<int64_t>(cus) * (per_cu > 0 ? per_cu : 1);
    return n >= 8 ? n / 8 * 8 : n;
  }();
  if (slots <= 0) return hipErrorInvalidDevice;
  const int64_t qblocks = (a.nq + 16 * QT - 1) / (16 * QT);
  const int64_t kblocks = (a.n_cols + kKT - 1) / kKT;
  const int64_t tiles = qblocks * kblocks;
  const dim3 grid(static_cast<unsigned>(tiles < slots ? tiles : slots), static_cast<unsigned>(a.groups));
  hipLaunchKernelGGL((scorem_kernel<M, QT, FILT>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

// 64-query blocks, or 32 when a group has no more than 32 queries; the
// filtered pass (tau set) or score rows
template <int M>
int launch_m(const ScoreMArgs &a, hipStream_t s) {
  if (a.tau) return a.nq <= 32 ? launch_mq<M, 2, true>(a, s) : launch_mq<M, 4, true>(a, s);
  return a.nq <= 32 ? launch_mq<M, 2, false>(a, s) : launch_mq<M, 4, false>(a, s);
}

}  // namespace

bool score_on_mfma(int d, int m, bool prod, int64_t nq) {
  return !prod && m >= 1 && m <= 4 && d >= kCC && nq >= 16;
}

int launch_qsplit(const QSplitArgs &a, void *stream) {
  (void)hipGetLastError();   // report only errors of this launch
  const int64_t blocks = (a.rows + kWaves - 1) / kWaves;
  hipLaunchKernelGGL(qsplit_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), a);
  return hipGetLastError();
}

int launch_scorem(const ScoreMArgs &a, void *stream) {
  (void)hipGetLastError();   // report only errors of this launch
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (a.m) {
    case 1: return launch_m<1>(a, s);
    case 2: return launch_m<2>(a, s);
    case 3: return launch_m<3>(a, s);
    case 4: return launch_m<4>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tq
