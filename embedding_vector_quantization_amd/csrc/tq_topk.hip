// Top-k selection over estimated inner products for gfx950.
//
// Sources: "TurboQuant: Online Vector Quantization" paper summary (Jump2Paper
// Archive) -- the nearest-neighbour search application (the database is
// quantised once, queries are scored against the codes, and recall of the
// top results is what the experiments report).
//
// Rows of a float32 score matrix (16-byte aligned, fewer than 2^31 keys) are
// cut into segments, one workgroup per (segment, row): each thread keeps a
// sorted list of its best k candidates while it streams its share of the
// segment (16-byte loads), the lists go to LDS, and k rounds of a block-wide
// argmax pick the segment's top k.  With several segments per row a second
// pass does the same over the rows' segment candidates.  Order: larger
// estimate first, equal estimates by smaller key index; NaN estimates are
// never selected.  When a row has fewer than k keys the tail is index -1,
// value -inf.

#include <hip/hip_runtime.h>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// (v, i) ranks before (w, j)?
__device__ __forceinline__ bool better(float v, int i, float w, int j) {
  return v > w || (v == w && i < j);
}

// FROM_CAND: the input is candidate lists (value, key index; index < 0 =
// empty) of t.segs segments per row; otherwise a segment of a score row.
// TO_CAND: the output is this segment's candidate list; otherwise the row's
// final top k.  LISTS: the input is the row's counted list (TopkListArgs).
template <int KMAX, bool FROM_CAND, bool TO_CAND, bool LISTS = false>
__global__ void __launch_bounds__(kThreads) topk_kernel(TopkArgs a, TopkListArgs la) {
  __shared__ float lv[KMAX][kThreads];
  __shared__ int li[KMAX][kThreads];
  __shared__ float wv[kWaves];
  __shared__ int wi[kWaves];
  __shared__ int wt[kWaves];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int k = LISTS ? la.k : a.k;
  const int64_t row = blockIdx.y;
  const int seg = blockIdx.x;
  const float ninf = -__builtin_inff();
  // (every thread reads the same count, so whole workgroups leave together)
  if constexpr (LISTS) {
    if (la.cnt[row] > la.cap) return;
  } else {
    if (a.only_over && a.only_over[row] <= a.over_cap) return;
  }

  float tv[KMAX];
  int ti[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    tv[j] = ninf;
    ti[j] = -1;
  }
  auto offer = [&](float v, int i) {
    // insert (v, i) if it beats the current k-th entry; NaN never does
    if (!(v == v)) return;
    if (!better(v, i, tv[KMAX - 1], ti[KMAX - 1]) && ti[KMAX - 1] >= 0) return;
#pragma unroll
    for (int j = KMAX - 1; j >= 0; --j) {
      const bool above = j > 0 && (ti[j - 1] < 0 || better(v, i, tv[j - 1], ti[j - 1]));
      if (above) {
        tv[j] = tv[j - 1];
        ti[j] = ti[j - 1];
      } else {
        const bool here = ti[j] < 0 || better(v, i, tv[j], ti[j]);
        if (here) {
          tv[j] = v;
          ti[j] = i;
        }
        break;
      }
    }
  };
  // Lists keep KMAX entries; only the first k matter, since a thread's k
  // best are a prefix of its KMAX best.
  if constexpr (LISTS) {
    const int cnt = la.cnt[row];
    const float *cv = la.list_v + row * la.cap;
    const int *ci = la.list_i + row * la.cap;
    for (int t = tid; t < cnt; t += kThreads) offer(cv[t], ci[t]);
  } else if constexpr (FROM_CAND) {
    const int cnt = a.segs * k;
    const float *cv = a.cand_vals + row * cnt;
    const int *ci = a.cand_idx + row * cnt;
    for (int t = tid; t < cnt; t += kThreads) {
      const int i = ci[t];
      if (i >= 0) offer(cv[t], i);
    }
  } else {
    const float *s = a.scores + row * a.ld;
    const int t0 = static_cast<int>(static_cast<int64_t>(seg) * a.seg_len);   // multiple of 4
    const int64_t t1l = t0 + a.seg_len < a.n ? t0 + a.seg_len : a.n;
    const int t1 = static_cast<int>(t1l);                                      // < 2^31, checked by the caller
    const int t4 = t0 + ((t1 - t0) & ~3);
    // Pass 1: each thread's largest estimate; tau = the k-th largest of
    // those maxima is at most the segment's k-th largest estimate, so every
    // member of the top k is >= tau, and few others are.
    float mx = ninf;
    for (int t = t0 + 4 * tid; t < t4; t += 4 * kThreads) {
      const float4 v = *reinterpret_cast<const float4 *>(s + t);
      mx = fmaxf(mx, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));       // fmaxf ignores NaN
    }
    for (int t = t4 + tid; t < t1; t += kThreads) mx = fmaxf(mx, s[t]);
    lv[0][tid] = mx;
    __syncthreads();
    int above = 0;                                   // maxima ranked before this thread's
    for (int u = 0; u < kThreads; ++u) {
      const float o = lv[0][u];
      above += (o > mx || (o == mx && u < tid)) ? 1 : 0;
    }
    __shared__ float tau_s;
    if (above == k - 1) tau_s = mx;
    __syncthreads();
    const float tau = tau_s;
    __syncthreads();
    // Pass 2: only estimates >= tau compete
    for (int t = t0 + 4 * tid; t < t4; t += 4 * kThreads) {
      const float4 v = *reinterpret_cast<const float4 *>(s + t);
      if (v.x >= tau) offer(v.x, t);
      if (v.y >= tau) offer(v.y, t + 1);
      if (v.z >= tau) offer(v.z, t + 2);
      if (v.w >= tau) offer(v.w, t + 3);
    }
    for (int t = t4 + tid; t < t1; t += kThreads)
      if (s[t] >= tau) offer(s[t], t);
  }
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    lv[j][tid] = tv[j];
    li[j][tid] = ti[j];
  }
  __syncthreads();

  int ptr = 0;                                  // this thread's next candidate
  for (int r = 0; r < k; ++r) {
    float hv = ninf;
    int hi = -1;
    if (ptr < KMAX) {
      hv = lv[ptr][tid];
      hi = li[ptr][tid];
    }
    float bv = hv;
    int bi = hi;
    int bt = tid;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      const int ot = __shfl_xor(bt, off);
      const bool take = oi >= 0 && (bi < 0 || better(ov, oi, bv, bi));
      if (take) {
        bv = ov;
        bi = oi;
        bt = ot;
      }
    }
    if (lane == 0) {
      wv[wave] = bv;
      wi[wave] = bi;
      wt[wave] = bt;
    }
    __syncthreads();
    float fv = wv[0];
    int fi = wi[0];
    int ft = wt[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      if (wi[w] >= 0 && (fi < 0 || better(wv[w], wi[w], fv, fi))) {
        fv = wv[w];
        fi = wi[w];
        ft = wt[w];
      }
    }
    if (tid == 0) {
      if constexpr (TO_CAND) {
        const int64_t o = (row * a.segs + seg) * k + r;
        a.cand_vals[o] = fv;
        a.cand_idx[o] = fi;
      } else if constexpr (LISTS) {
        la.idx[row * k + r] = fi;
        la.vals[row * k + r] = fi >= 0 ? fv : ninf;
      } else {
        a.idx[row * a.k + r] = fi;
        a.vals[row * a.k + r] = fi >= 0 ? fv : ninf;
      }
    }
    if (tid == ft && fi >= 0) ++ptr;
    __syncthreads();
  }
}

template <int KMAX>
void launch_k(const TopkArgs &a, hipStream_t s) {
  const unsigned rows = static_cast<unsigned>(a.rows);
  const TopkListArgs none{};
  if (a.segs <= 1) {
    hipLaunchKernelGGL((topk_kernel<KMAX, false, false>), dim3(1, rows), dim3(kThreads), 0, s, a, none);
  } else {
    hipLaunchKernelGGL((topk_kernel<KMAX, false, true>), dim3(static_cast<unsigned>(a.segs), rows), dim3(kThreads), 0,
                       s, a, none);
    hipLaunchKernelGGL((topk_kernel<KMAX, true, false>), dim3(1, rows), dim3(kThreads), 0, s, a, none);
  }
}

__global__ void __launch_bounds__(kThreads) tau_kernel(TauArgs a) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (r >= a.rows) return;
  const int64_t last = r * a.k + a.k - 1;
  a.tau[r] = a.idx[last] >= 0 ? a.vals[last] : -__builtin_inff();
  a.cnt[r] = 0;
}

}  // namespace

int launch_topk_lists(const TopkListArgs &a, void *stream) {
  (void)hipGetLastError();   // report only errors of this launch
  hipStream_t s = static_cast<hipStream_t>(stream);
  const TopkArgs none{};
  const dim3 grid(1, static_cast<unsigned>(a.rows));
  if (a.k <= 16) {
    hipLaunchKernelGGL((topk_kernel<16, true, false, true>), grid, dim3(kThreads), 0, s, none, a);
  } else {
    hipLaunchKernelGGL((topk_kernel<32, true, false, true>), grid, dim3(kThreads), 0, s, none, a);
  }
  return hipGetLastError();
}

int launch_tau(const TauArgs &a, void *stream) {
  (void)hipGetLastError();   // report only errors of this launch
  const unsigned blocks = static_cast<unsigned>((a.rows + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(tau_kernel, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream), a);
  return hipGetLastError();
}

int64_t topk_segments(int64_t rows, int64_t n) {
  // about 2048 workgroups over the rows, each segment at least 4096 keys
  int64_t segs = rows > 0 ? 2048 / rows : 1;
  const int64_t by_len = (n + 4095) / 4096;
  if (segs > by_len) segs = by_len;
  return segs < 1 ? 1 : segs;
}

int launch_topk(const TopkArgs &a, void *stream) {
  (void)hipGetLastError();   // report only errors of this launch
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (a.k <= 16) {
    launch_k<16>(a, s);
  } else {
    launch_k<32>(a, s);
  }
  return hipGetLastError();
}

}  // namespace tq
