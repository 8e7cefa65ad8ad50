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
// Workgroup: 32 queries x 256 keys, four waves of 32 x 64.  Per chunk of 128
// coordinates the workgroup loads the 32 queries' hi and lo parts straight
// into LDS (each wave 8 rows), and each wave its 64 key records (direct
// loads, the next chunk in flight while this one is multiplied).  A wave
// builds its key operand from pairs of codes with a small table of (hi, hi)
// and (lo, lo) float16 pairs, and reads the query operand from LDS.

#include <hip/hip_runtime.h>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kQT = 32;            // queries per workgroup: two 16-row tiles
constexpr int kKT = 64 * kWaves;   // keys per workgroup: 64 per wave, four 16-column tiles
constexpr int kCC = 128;           // coordinates per staged chunk (four k-steps of 32)

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

// 8 codes of m bits (coordinates 8 g' .. 8 g' + 7 of a k-step) from the
// staged record chunk at byte p.
template <int M>
__device__ __forceinline__ uint32_t codes8(const uint8_t *p) {
  if constexpr (M == 1) {
    return p[0];
  } else if constexpr (M == 2) {
    return *reinterpret_cast<const uint16_t *>(p);
  } else if constexpr (M == 3) {
    return static_cast<uint32_t>(p[0]) | (static_cast<uint32_t>(p[1]) << 8) | (static_cast<uint32_t>(p[2]) << 16);
  } else {
    return *reinterpret_cast<const uint32_t *>(p);
  }
}

template <int M>
__global__ void __launch_bounds__(kThreads) scorem_kernel(ScoreMArgs a) {
  constexpr int K = 1 << M;
  constexpr int PE = K * K;              // pair-table entries
  constexpr int CB = 16 * M;             // bytes of one key's 128-coordinate chunk
  constexpr int SB = 64 * CB;            // bytes of a wave's staged chunk
  constexpr int QB = kQT * kCC * 2;      // bytes of one part (hi or lo) of a query chunk
  // m <= 2: one byte of codes (8 / m coordinates) indexes a table of their
  // float16 values, hi parts and lo parts in two tables (TW bytes per entry),
  // so a lookup lands in the operand's registers as they are; m >= 3: pairs
  // of codes index (hi, hi | lo, lo) pairs
  constexpr bool kByte = M <= 2;
  constexpr int TW = kByte ? 16 / M : 8;
  __shared__ __attribute__((aligned(16))) uint8_t tab_lds[kByte ? 2 * 256 * TW : 16];
  __shared__ uint2 pair_lds[kByte ? 1 : PE];   // (hi of c0 | hi of c1 << 16, lo ... )
  __shared__ __attribute__((aligned(16))) uint8_t stage[kWaves * 2 * SB];
  // query chunks, two buffers x (hi, lo): row r's 16-byte slot c at
  // r * 256 + 16 (c ^ (r & 15)), so a wave's operand reads hit distinct banks
  __shared__ __attribute__((aligned(16))) uint8_t qstage[2 * 2 * QB];

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 15;
  const int g = lane >> 4;
  const int qblocks = (a.nq + kQT - 1) / kQT;
  const int qb = static_cast<int>(blockIdx.x % qblocks);
  const int64_t kb = blockIdx.x / qblocks;
  const int64_t grp = blockIdx.y;
  const int64_t key0 = grp * a.n;                       // group's first key
  const int64_t kw = kb * a.kb_stride * kKT + 64 * wv;  // wave's first key in the group
  const int64_t nlive = a.n - kw;                       // live keys from there on
  const int64_t cw = kb * kKT + 64 * wv;                // its first score column
  const int64_t qrow0 = grp * a.nq + static_cast<int64_t>(qb) * kQT;
  const int nqb = a.nq - qb * kQT < kQT ? a.nq - qb * kQT : kQT;
  if (a.only_over) {
    // the pass for rows whose candidate lists overflowed: nothing to do
    // unless one of this block's rows did (every thread reads the same)
    bool any = false;
    for (int qi = 0; qi < nqb; ++qi) any = any || a.only_over[qrow0 + qi] > a.list_cap;
    if (!any) return;
  }

  // codebook scaled by 2^-ec into [0.5, 1), as (hi, lo) float16 pairs
  float cmax = 0.0f;
#pragma unroll
  for (int k = 0; k < K; ++k) cmax = fmaxf(cmax, fabsf(a.centroids[k]));
  int ec = 0;
  if (cmax > 0.0f) (void)frexpf(cmax, &ec);
  const float cs = ldexpf(1.0f, -ec);
  if constexpr (kByte) {
    // entry e: coordinate u of the byte has code (e >> M u) & (K - 1)
    constexpr int CPE = 8 / M;           // coordinates per entry
    for (int i = threadIdx.x; i < 256 * CPE; i += kThreads) {
      const int e = i / CPE, u = i - e * CPE;
      const float c = a.centroids[(e >> (M * u)) & (K - 1)] * cs;
      const _Float16 h = static_cast<_Float16>(c);
      const _Float16 l = static_cast<_Float16>(c - static_cast<float>(h));
      reinterpret_cast<uint16_t *>(tab_lds)[e * CPE + u] = static_cast<uint16_t>(f16_bits(h));
      reinterpret_cast<uint16_t *>(tab_lds + 256 * TW)[e * CPE + u] = static_cast<uint16_t>(f16_bits(l));
    }
  } else {
    for (int i = threadIdx.x; i < PE; i += kThreads) {
      const float c0 = a.centroids[i & (K - 1)] * cs, c1 = a.centroids[i >> M] * cs;
      const _Float16 h0 = static_cast<_Float16>(c0), h1 = static_cast<_Float16>(c1);
      const _Float16 l0 = static_cast<_Float16>(c0 - static_cast<float>(h0));
      const _Float16 l1 = static_cast<_Float16>(c1 - static_cast<float>(h1));
      pair_lds[i] = make_uint2(f16_bits(h0) | (f16_bits(h1) << 16), f16_bits(l0) | (f16_bits(l1) << 16));
    }
  }

  const int64_t rec_bytes = static_cast<int64_t>(M) * a.d / 8;
  uint8_t *st0 = stage + wv * 2 * SB;
  // chunk c of the wave's 64 records into stage buffer b, key k's piece at
  // k * CB; keys past the group's end fetch its last key
  auto issue = [&](int c, int b) {
    if (nlive <= 0) return;                                // uniform over the wave
    const uint8_t *base = a.codes + (key0 + kw) * rec_bytes + static_cast<int64_t>(c) * CB;
#pragma unroll
    for (int i = 0; i < M; ++i) {
      const int f = i * 64 + lane;
      const int64_t k = f / M;
      const int64_t kk = k < nlive ? k : nlive - 1;
      load_lds16_nt(base + kk * rec_bytes + (f % M) * 16, st0 + b * SB + 1024 * i);
    }
  };
  // chunk c of query rows 8 wv .. 8 wv + 7 (hi and lo) into query buffer b:
  // load h covers rows 8 wv + 4 h .. + 3, lane l row + l / 16, slot l % 16,
  // fetching the column chunk that the slot swizzle puts there
  const int qr_l = 8 * wv + (lane >> 4);                  // + 4 h
  auto issue_q = [&](int c, int b) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = qr_l + 4 * h;
      const int rr = r < nqb ? r : nqb - 1;               // rows past the block's queries: a copy
      const int col = (lane & 15) ^ (r & 15);
      const int64_t off = (qrow0 + rr) * a.d + static_cast<int64_t>(c) * kCC + 8 * col;
      uint8_t *dst = qstage + b * 2 * QB + (8 * wv + 4 * h) * 256;
      load_lds16_nt(a.qh + off, dst);
      load_lds16_nt(a.ql + off, dst + QB);
    }
  };
  issue_q(0, 0);
  issue(0, 0);

  // The lo table at an offset the compiler cannot see as a constant: it then
  // reads each part into the operand's own registers instead of pairing the
  // hi and lo reads and moving the results apart.
  uint32_t lo_off = 256 * TW;
  asm volatile("" : "+v"(lo_off));

  // this lane's query operand rows (tile qt, row j) and their swizzle
  int qoff[2];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) qoff[qt] = (16 * qt + j) * 256;

  f32x4 acc[2][4];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[qt][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const int nchunk = a.d / kCC;
  for (int c = 0; c < nchunk; ++c) {
    const int b = c & 1;
    // this wave's loads of chunk c have landed; after the barrier every
    // wave's have, and every wave is done with chunk c - 1, whose buffers
    // then take chunk c + 1 (the barrier also publishes the pair table)
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __syncthreads();
    if (c + 1 < nchunk) {
      issue_q(c + 1, b ^ 1);
      issue(c + 1, b ^ 1);
    }
    const uint8_t *st = st0 + b * SB;
    const uint8_t *qs = qstage + b * 2 * QB;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      f16x8 ah[2], al[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const int slot = (4 * s + g) ^ j;                 // (16 qt + j) & 15 == j
        ah[qt] = *reinterpret_cast<const f16x8 *>(qs + qoff[qt] + 16 * slot);
        al[qt] = *reinterpret_cast<const f16x8 *>(qs + QB + qoff[qt] + 16 * slot);
      }
      f16x8 bh[4], bl[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t bits = codes8<M>(st + (16 * t + j) * CB + (4 * s + g) * M);
        if constexpr (M == 1) {
          // one byte = the 8 coordinates: one 16-byte entry per part
          const uint8_t *e = tab_lds + 16 * bits;
          bh[t] = *reinterpret_cast<const f16x8 *>(e);
          bl[t] = *reinterpret_cast<const f16x8 *>(tab_lds + (lo_off + 16 * bits));
        } else if constexpr (M == 2) {
          // two bytes of 4 coordinates: two 8-byte entries per part
          const uint32_t o0 = 8 * (bits & 0xFFu), o1 = 8 * (bits >> 8);
          const uint2 h0 = *reinterpret_cast<const uint2 *>(tab_lds + o0);
          const uint2 h1 = *reinterpret_cast<const uint2 *>(tab_lds + o1);
          const uint2 l0 = *reinterpret_cast<const uint2 *>(tab_lds + (lo_off + o0));
          const uint2 l1 = *reinterpret_cast<const uint2 *>(tab_lds + (lo_off + o1));
          const uint32_t hw[4] = {h0.x, h0.y, h1.x, h1.y}, lw[4] = {l0.x, l0.y, l1.x, l1.y};
          __builtin_memcpy(&bh[t], hw, 16);
          __builtin_memcpy(&bl[t], lw, 16);
        } else {
          uint32_t hw[4], lw[4];
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const uint2 e = pair_lds[(bits >> (2 * M * p)) & (PE - 1)];
            hw[p] = e.x;
            lw[p] = e.y;
          }
          __builtin_memcpy(&bh[t], hw, 16);
          __builtin_memcpy(&bl[t], lw, 16);
        }
      }
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          acc[qt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[qt], bh[t], acc[qt][t], 0, 0, 0);
          acc[qt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[qt], bl[t], acc[qt][t], 0, 0, 0);
          acc[qt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[qt], bh[t], acc[qt][t], 0, 0, 0);
        }
    }
  }

  // acc[qt][t][r] = estimate of query 16 qt + 4 g + r and key 16 t + j
  const float cinv = ldexpf(1.0f, ec);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int64_t kl = kw + 16 * t + j;                    // key within the group
    const int64_t col = cw + 16 * t + j;                   // its score column
    if (kl >= a.n || col >= a.n_cols) continue;
    const float nk = a.norms[key0 + kl] * cinv;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int qi = 16 * qt + 4 * g + r;
        if (qi >= nqb) continue;
        const int64_t row = qrow0 + qi;
        const float v = acc[qt][t][r] * nk * a.qinv[row];
        if (a.tau) {
          // a candidate (NaN never is)
          if (v >= a.tau[row]) {
            const int slot = atomicAdd(a.cnt + row, 1);
            if (slot < a.list_cap) {
              a.list_v[row * a.list_cap + slot] = v;
              a.list_i[row * a.list_cap + slot] = static_cast<int32_t>(kl);
            }
          }
        } else {
          float *dst = a.scores + row * a.ld_scores + col;
          *dst = a.accumulate ? *dst + v : v;
        }
      }
  }
}

template <int M>
int launch_m(const ScoreMArgs &a, hipStream_t s) {
  const int64_t qblocks = (a.nq + kQT - 1) / kQT;
  const int64_t kblocks = (a.n_cols + kKT - 1) / kKT;
  const dim3 grid(static_cast<unsigned>(qblocks * kblocks), static_cast<unsigned>(a.groups));
  hipLaunchKernelGGL((scorem_kernel<M>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
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
