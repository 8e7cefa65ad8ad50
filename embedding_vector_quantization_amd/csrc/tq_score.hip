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
// Streaming kernel (d >= 128): one lane per key.  The coordinates are
// processed in chunks of 128; for each chunk and query the workgroup builds a
// table in LDS whose entry for a group of G coordinates and their G*m code
// bits is sum_{j in group} q'_j c[code_j] (G*m <= 8 bits), and, for prod, a
// byte table over the QJL plane: entry (k, v) = sum_{t<8} +-s_{8k+t}.  A key
// then costs one bit-field extract, one LDS read and one add per group.
// Small d (< 128) uses a plain per-coordinate loop.

#include <hip/hip_runtime.h>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 128;
constexpr float kQjlScale = 1.2533141373155003f;   // sqrt(pi/2)

template <int M>
struct LutShape {
  static constexpr int G = (M == 1) ? 8 : (M == 2) ? 4 : (M <= 4) ? 2 : 1;   // coordinates per group
  static constexpr int W = G * M;                                             // bits per group
  static constexpr int NG = kChunk / G;                                       // groups per chunk
  static constexpr int ENTRIES = NG << W;                                     // mse entries per chunk
};
template <>
struct LutShape<0> {
  static constexpr int G = 1, W = 0, NG = 0, ENTRIES = 0;
};
constexpr int kZEntries = 16 * 256;                 // QJL byte table per chunk

template <int M, bool PROD>
constexpr int lut_floats_per_query() {
  return LutShape<M>::ENTRIES + (PROD ? kZEntries : 0);
}

// Field of W bits at bit offset POS of the chunk's words, times 4 (a byte
// offset into a float table).
template <int W, int POS>
__device__ __forceinline__ uint32_t field_x4(const uint32_t *w) {
  constexpr int wi = POS >> 5, off = POS & 31;
  constexpr uint32_t mask = ((1u << W) - 1u) << 2;
  if constexpr (off >= 2) {
    if constexpr (off + W <= 32) {
      return (w[wi] >> (off - 2)) & mask;
    } else {
      return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], off - 2) & mask;
    }
  } else {
    return (w[wi] << (2 - off)) & mask;
  }
}

// acc[T & 3] += table entry of group T (four partial sums for ILP).
template <int M, int T>
__device__ __forceinline__ void mse_groups(const uint32_t *w, const float *lut, float (&acc)[4]) {
  using S = LutShape<M>;
  if constexpr (T < S::NG) {
    const uint32_t f4 = field_x4<S::W, T * S::W>(w);
    acc[T & 3] += *reinterpret_cast<const float *>(reinterpret_cast<const char *>(lut) + (T << S::W) * 4 + f4);
    mse_groups<M, T + 1>(w, lut, acc);
  }
}

template <int M, bool PROD, int QB>
__global__ void __launch_bounds__(kThreads) score_kernel(ScoreArgs a) {
  extern __shared__ __attribute__((aligned(16))) float lut[];
  using S = LutShape<M>;
  constexpr int kPerQ = lut_floats_per_query<M, PROD>();
  constexpr int K = 1 << M;
  __shared__ float cb[K > 1 ? K : 2];
  if constexpr (M >= 1) {
    for (int k = threadIdx.x; k < K; k += kThreads) cb[k] = a.centroids[k];
  }
  const int q0 = blockIdx.y * QB;
  const int nchunks = a.d / kChunk;
  const int64_t tiles = (a.n + kThreads - 1) / kThreads;
  const float zs = kQjlScale / static_cast<float>(a.d);
  const size_t rec_words = static_cast<size_t>(M) * a.d / 32;
  const size_t z_words = static_cast<size_t>(a.d) / 32;

  auto build = [&](int c) {
    __syncthreads();
    for (int i = threadIdx.x; i < QB * kPerQ; i += kThreads) {
      const int q = i / kPerQ;
      const int r = i - q * kPerQ;
      const int qi = q0 + q;
      float val = 0.0f;
      if (qi < a.nq) {
        if (r < S::ENTRIES) {
          if constexpr (M >= 1) {
            const int t = r >> S::W;
            const int v = r & ((1 << S::W) - 1);
            const float *qr = a.qrot + static_cast<int64_t>(qi) * a.d + c * kChunk + t * S::G;
#pragma unroll
            for (int u = 0; u < S::G; ++u) val = fmaf(qr[u], cb[(v >> (M * u)) & (K - 1)], val);
          }
        } else {
          const int rz = r - S::ENTRIES;
          const int k = rz >> 8;
          const int v = rz & 255;
          const float *sq = a.sq + static_cast<int64_t>(qi) * a.d + c * kChunk + 8 * k;
#pragma unroll
          for (int t = 0; t < 8; ++t) val += ((v >> t) & 1) ? sq[t] : -sq[t];
        }
      }
      lut[i] = val;
    }
    __syncthreads();
  };

  if (nchunks == 1) build(0);
  for (int64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
    const int64_t key = tile * kThreads + threadIdx.x;
    const bool live = key < a.n;
    const int64_t kk = live ? key : 0;
    float acc[QB], accz[QB];
#pragma unroll
    for (int q = 0; q < QB; ++q) acc[q] = accz[q] = 0.0f;
    for (int c = 0; c < nchunks; ++c) {
      if (nchunks > 1) build(c);
      if constexpr (M >= 1) {
        uint32_t w[4 * M];
        const uint4 *src = reinterpret_cast<const uint4 *>(a.codes) + (kk * rec_words + 4 * M * c) / 4;
#pragma unroll
        for (int i = 0; i < M; ++i) {
          const uint4 v = src[i];
          w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
        }
#pragma unroll
        for (int q = 0; q < QB; ++q) {
          float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
          mse_groups<M, 0>(w, lut + q * kPerQ, part);
          acc[q] += (part[0] + part[1]) + (part[2] + part[3]);
        }
      }
      if constexpr (PROD) {
        const uint4 zv = reinterpret_cast<const uint4 *>(a.qjl)[(kk * z_words + 4 * c) / 4];
        const uint32_t zw[4] = {zv.x, zv.y, zv.z, zv.w};
#pragma unroll
        for (int q = 0; q < QB; ++q) {
          const float *lz = lut + q * kPerQ + S::ENTRIES;
          float part = 0.0f;
#pragma unroll
          for (int k = 0; k < 16; ++k) part += lz[k * 256 + ((zw[k >> 2] >> (8 * (k & 3))) & 255u)];
          accz[q] += part;
        }
      }
    }
    if (live) {
      const float nrm = a.norms[key];
      const float g = PROD ? a.rnorms[key] * zs : 0.0f;
#pragma unroll
      for (int q = 0; q < QB; ++q) {
        const int qi = q0 + q;
        if (qi < a.nq) a.scores[static_cast<int64_t>(qi) * a.ld_scores + key] = nrm * fmaf(g, accz[q], acc[q]);
      }
    }
  }
}

// d < 128: one lane per key, a loop over coordinates.
__global__ void __launch_bounds__(kThreads) score_small_kernel(ScoreArgs a) {
  __shared__ float cb[256];
  __shared__ float qs[2 * 64];
  const int K = a.m > 0 ? (1 << a.m) : 0;
  for (int k = threadIdx.x; k < K; k += kThreads) cb[k] = a.centroids[k];
  const float zs = kQjlScale / static_cast<float>(a.d);
  const size_t rec_bytes = static_cast<size_t>(a.m) * a.d / 8;
  for (int qi = 0; qi < a.nq; ++qi) {
    __syncthreads();
    for (int j = threadIdx.x; j < a.d; j += kThreads) {
      qs[j] = a.qrot[static_cast<int64_t>(qi) * a.d + j];
      qs[64 + j] = a.prod ? a.sq[static_cast<int64_t>(qi) * a.d + j] : 0.0f;
    }
    __syncthreads();
    for (int64_t key = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; key < a.n;
         key += static_cast<int64_t>(gridDim.x) * kThreads) {
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
      a.scores[static_cast<int64_t>(qi) * a.ld_scores + key] = a.norms[key] * fmaf(g, accz, acc);
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

template <int M, bool PROD, int QB>
int launch_mq(const ScoreArgs &a, hipStream_t s) {
  constexpr int kPerQ = lut_floats_per_query<M, PROD>();
  const size_t lds = static_cast<size_t>(QB) * kPerQ * sizeof(float);
  const int64_t tiles = (a.n + kThreads - 1) / kThreads;
  const int qblocks = (a.nq + QB - 1) / QB;
  int64_t gx = 2048 / qblocks;
  if (gx < 64) gx = 64;
  if (gx > tiles) gx = tiles;
  if (a.d > kChunk && gx > 1024) gx = 1024;
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&score_kernel<M, PROD, QB>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((score_kernel<M, PROD, QB>), dim3(static_cast<unsigned>(gx), qblocks), dim3(kThreads),
                     lds, s, a);
  return hipGetLastError();
}

template <int M, bool PROD>
int launch_m(const ScoreArgs &a, hipStream_t s) {
  constexpr size_t per_q = static_cast<size_t>(lut_floats_per_query<M, PROD>()) * sizeof(float);
  if (a.nq >= 4 && 4 * per_q <= 64 * 1024) return launch_mq<M, PROD, 4>(a, s);
  if (a.nq >= 2 && 2 * per_q <= 64 * 1024) return launch_mq<M, PROD, 2>(a, s);
  return launch_mq<M, PROD, 1>(a, s);
}

}  // namespace

int launch_score(const ScoreArgs &a, void *stream) {
  (void)hipGetLastError();   // report only errors of this launch
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (a.d < kChunk) {
    int64_t blocks = (a.n + kThreads - 1) / kThreads;
    if (blocks > 2048) blocks = 2048;
    hipLaunchKernelGGL(score_small_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, s, a);
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
