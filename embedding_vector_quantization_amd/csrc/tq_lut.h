// Packed-code table machinery shared by the score and attention kernels:
// bit-field extraction from a key's record words, the LDS staging of a
// wave's records, and the four-query lookup tables (float4 entries).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_device.h"

namespace tq {
namespace {

constexpr int kChunk = 128;
constexpr float kQjlScale = 1.2533141373155003f;   // sqrt(pi/2)

// Field of W bits at bit offset POS of the chunk's words, shifted left by SH
// (a byte offset into a table of 2^SH-byte entries).
template <int W, int POS, int SH>
__device__ __forceinline__ uint32_t field_at(const uint32_t *w) {
  constexpr int wi = POS >> 5, off = POS & 31;
  constexpr uint32_t mask = ((1u << W) - 1u) << SH;
  if constexpr (off >= SH) {
    if constexpr (off + W <= 32) {
      return (w[wi] >> (off - SH)) & mask;
    } else {
      return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], off - SH) & mask;
    }
  } else {
    if constexpr (off + W <= 32) {
      return (w[wi] << (SH - off)) & mask;
    } else {
      return ((w[wi] >> off) | (w[wi + 1] << (32 - off))) << SH & mask;
    }
  }
}

// Records of a wave's 64 keys staged in LDS (d = 128, 1 <= M <= 4): the wave
// reads them as 64 * M fully coalesced non-temporal 16-byte loads, then each
// lane reads its own key's M chunks.  Key pitch 4M dwords, plus 4 when M is
// even, so that 16 consecutive lanes hit 64 distinct banks.
template <int M>
struct RecStage {
  static constexpr bool kOn = (M >= 1 && M <= 4);
  static constexpr int kPitch = kOn ? 4 * M + ((M & 1) ? 0 : 4) : 4;   // dwords per key
  static constexpr int kWaveDwords = 64 * kPitch;

  // The wave's flat chunk i * 64 + lane of the records starting at key kb
  // (live keys < nlive) into regs.
  __device__ __forceinline__ static void issue(const uint8_t *codes, int64_t kb, int64_t nlive, int lane,
                                               uint4 (&r)[kOn ? M : 1]) {
    const uint8_t *src = codes + kb * (16 * M);
#pragma unroll
    for (int i = 0; i < M; ++i) {
      const int f = i * 64 + lane;
      r[i] = (f / M < nlive) ? load_nt16(src + 16 * f) : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ static void put(uint32_t *ws, int lane, const uint4 (&r)[kOn ? M : 1]) {
#pragma unroll
    for (int i = 0; i < M; ++i) {
      const int f = i * 64 + lane;
      *reinterpret_cast<uint4 *>(ws + (f / M) * kPitch + (f % M) * 4) = r[i];
    }
  }
  __device__ __forceinline__ static void get(const uint32_t *ws, int lane, uint32_t (&w)[4 * M]) {
#pragma unroll
    for (int i = 0; i < M; ++i) {
      const uint4 v = *reinterpret_cast<const uint4 *>(ws + lane * kPitch + 4 * i);
      w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
    }
  }
};

// Records of a wave's 64 keys loaded straight from HBM into LDS (d = 128,
// 1 <= M <= 4), no registers in between: load i of the M 16-byte loads per
// lane fills 1 KiB in lane order, so the 64 records lie back to back (key k's
// chunk c at 16 (M k + c) bytes).  Lanes past the group's last key fetch that
// key again (its estimate is never stored); a wave with no live key loads
// nothing.  The loads count as vector memory (vmcnt), not LDS.
template <int M>
struct RecDma {
  static constexpr int kWaveDwords = 64 * 4 * M;

  __device__ __forceinline__ static void issue(const uint8_t *codes, int64_t kb, int64_t nlive, int lane,
                                               uint32_t *ws) {
    if (nlive <= 0) return;                        // uniform over the wave
    const uint8_t *src = codes + kb * (16 * M);
#pragma unroll
    for (int i = 0; i < M; ++i) {
      const int f = i * 64 + lane;
      const int64_t k = f / M;
      const int64_t g = k < nlive ? f : (nlive - 1) * M + f % M;
      load_lds16_nt(src + 16 * g, ws + 256 * i);
    }
  }
  __device__ __forceinline__ static void get(const uint32_t *ws, int lane, uint32_t (&w)[4 * M]) {
#pragma unroll
    for (int i = 0; i < M; ++i) {
      const uint4 v = *reinterpret_cast<const uint4 *>(ws + lane * 4 * M + 4 * i);
      w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
    }
  }
};

// ------------------------------------------------------------ four queries

template <int M>
struct Shape4 {
  static constexpr int G = (M == 1) ? 4 : (M <= 3) ? 2 : 1;
  static constexpr int W = G * M;
  static constexpr int NG = kChunk / G;
  static constexpr int ENTRIES = NG << W;      // float4 entries
};
template <>
struct Shape4<0> {
  static constexpr int G = 1, W = 0, NG = 0, ENTRIES = 0;
};
constexpr int kZ4Entries = 32 * 16;            // QJL nibble table per chunk (float4)

template <int M, bool PROD>
constexpr int entries4() { return Shape4<M>::ENTRIES + (PROD ? kZ4Entries : 0); }

__device__ __forceinline__ void add4(float4 &acc, const float4 v) {
  acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
}

// An empty asm statement that reads and writes the accumulators and clobbers
// memory: table reads after it cannot be moved above it, and the sums before
// it must be complete, which bounds the number of reads in flight.
__device__ __forceinline__ void settle4(float4 (&acc)[2]) {
  asm volatile("" : "+v"(acc[0].x), "+v"(acc[0].y), "+v"(acc[0].z), "+v"(acc[0].w),
                    "+v"(acc[1].x), "+v"(acc[1].y), "+v"(acc[1].z), "+v"(acc[1].w) : : "memory");
}

template <int M, int T>
__device__ __forceinline__ void groups4(const uint32_t *w, const float4 *lut, float4 (&acc)[2]) {
  using S = Shape4<M>;
  if constexpr (T < S::NG) {
    const uint32_t f16 = field_at<S::W, T * S::W, 4>(w);
    add4(acc[T & 1], *reinterpret_cast<const float4 *>(reinterpret_cast<const char *>(lut) + (T << S::W) * 16 + f16));
    // keep at most 8 groups' table reads in flight (otherwise all of them
    // are hoisted, 4 registers each, and occupancy collapses)
    if constexpr ((T & 7) == 7) settle4(acc);
    groups4<M, T + 1>(w, lut, acc);
  }
}

template <int T>
__device__ __forceinline__ void nibbles4(const uint32_t *zw, const float4 *lz, float4 (&acc)[2]) {
  if constexpr (T < 32) {
    const uint32_t f16 = field_at<4, T * 4, 4>(zw);
    add4(acc[T & 1], *reinterpret_cast<const float4 *>(reinterpret_cast<const char *>(lz) + T * 256 + f16));
    if constexpr ((T & 7) == 7) settle4(acc);
    nibbles4<T + 1>(zw, lz, acc);
  }
}


// ------------------------------------------------------------ queries at d = 128

// Walsh-Hadamard transform of 128 values held two per lane (coordinate
// 2 lane + e in v[e]): bit 0 inside the lane, bits 1..6 across lanes.
__device__ __forceinline__ void fwht128_wave(float &v0, float &v1, int lane) {
  const float s0 = v0 + v1, s1 = v0 - v1;
  v0 = s0;
  v1 = s1;
#pragma unroll
  for (int b = 0; b < 6; ++b) {
    const float eps = (lane >> b) & 1 ? -1.0f : 1.0f;
    const float p0 = __shfl_xor(v0, 1 << b), p1 = __shfl_xor(v1, 1 << b);
    v0 = fmaf(eps, v0, p0);
    v1 = fmaf(eps, v1, p1);
  }
}

// q' = Pi q for one query row (d_in columns, zero padded to d = 128), by one
// whole wave: lane l holds coordinates 2 l and 2 l + 1.  Rotation as the
// encoder's: TQ_ROT_RHT (1/sqrt 128) H diag(signs); TQ_ROT_GIVENS one 2-D
// rotation per coordinate pair (lane-local); TQ_ROT_QUAT the left product
// with a unit quaternion per coordinate quad (lanes 2 i and 2 i + 1).
// load_query128 issues the lane's loads (the two coordinates and the
// rotation parameters they need), rotate_loaded128 does the arithmetic, so a
// caller can put other loads in flight between the two.
struct QueryLanes {
  float v0, v1;         // coordinates 2 l, 2 l + 1
  float r[4];           // RHT: the two signs; Givens: c, s; quaternion: w, x, y, z
};

__device__ __forceinline__ QueryLanes load_query128(const float *q, int d_in, int rot_kind, const int8_t *signs,
                                                    const float *rot, int lane) {
  const int j0 = 2 * lane, j1 = 2 * lane + 1;
  QueryLanes t;
  t.v0 = j0 < d_in ? q[j0] : 0.0f;
  t.v1 = j1 < d_in ? q[j1] : 0.0f;
  t.r[2] = t.r[3] = 0.0f;
  if (rot_kind == TQ_ROT_GIVENS) {
    t.r[0] = rot[j0];
    t.r[1] = rot[j1];
  } else if (rot_kind == TQ_ROT_QUAT) {
    const float *p = rot + 4 * (lane >> 1);
#pragma unroll
    for (int k = 0; k < 4; ++k) t.r[k] = p[k];
  } else {
    t.r[0] = signs[j0] < 0 ? -1.0f : 1.0f;
    t.r[1] = signs[j1] < 0 ? -1.0f : 1.0f;
  }
  return t;
}

__device__ __forceinline__ void rotate_loaded128(const QueryLanes &t, int rot_kind, float *dst, int lane) {
  const int j0 = 2 * lane, j1 = 2 * lane + 1;
  float v0 = t.v0, v1 = t.v1;
  if (rot_kind == TQ_ROT_GIVENS) {
    const float c = t.r[0], s = t.r[1];
    const float y0 = fmaf(c, v0, -s * v1), y1 = fmaf(s, v0, c * v1);
    v0 = y0;
    v1 = y1;
  } else if (rot_kind == TQ_ROT_QUAT) {
    const float o0 = __shfl_xor(v0, 1), o1 = __shfl_xor(v1, 1);
    const bool hi = lane & 1;                         // this lane holds coordinates 2, 3 of the quad
    const float a = hi ? o0 : v0, b = hi ? o1 : v1, c = hi ? v0 : o0, d = hi ? v1 : o1;
    const float w = t.r[0], x = t.r[1], y = t.r[2], z = t.r[3];
    if (hi) {
      v0 = y * a + z * b + w * c - x * d;
      v1 = z * a - y * b + x * c + w * d;
    } else {
      v0 = w * a - x * b - y * c - z * d;
      v1 = x * a + w * b - z * c + y * d;
    }
  } else {
    v0 = t.r[0] < 0.0f ? -v0 : v0;
    v1 = t.r[1] < 0.0f ? -v1 : v1;
    fwht128_wave(v0, v1, lane);
    const float rsd = 0.08838834764831845f;          // 1 / sqrt(128)
    v0 *= rsd;
    v1 *= rsd;
  }
  dst[j0] = v0;
  dst[j1] = v1;
}

__device__ __forceinline__ void rotate_query128(const float *q, int d_in, int rot_kind, const int8_t *signs,
                                                const float *rot, float *dst, int lane) {
  rotate_loaded128(load_query128(q, d_in, rot_kind, signs, rot, lane), rot_kind, dst, lane);
}

// s = S q' for rows 0 .. nq-1 (nq <= NQ) of qr (LDS, [.][128]) into sq, S
// bfloat16 [128][128] row-major, by all NT threads of the block: thread t
// takes row t % 128 and a contiguous 1/(NT/128) of its columns, with up to
// two 16-byte loads of S in flight, and leaves one partial sum per query in part
// ([NT/128 * NQ][128], LDS); the partials are then added in a fixed order.
// qr must be complete before the call; sq is complete after the next
// barrier.
// S q' for four queries by 1024 threads whose S words were loaded ahead
// (sq_words1024): thread t holds row t & 127, columns 16 (t >> 7) .. + 15.
// The same products in the same order as sq_rows128<1024, 4>.
__device__ __forceinline__ void sq_words1024(const uint16_t *s_mat, uint4 (&w)[2]) {
  const uint4 *src = reinterpret_cast<const uint4 *>(s_mat + (threadIdx.x & 127) * 128 + (threadIdx.x >> 7) * 16);
  w[0] = src[0];
  w[1] = src[1];
}

__device__ __forceinline__ void sq_rows1024_from(const uint4 (&w)[2], const float (*qr)[128], float (*sq)[128],
                                                 float (*part)[128], int nq) {
  const int i = threadIdx.x & 127, h = threadIdx.x >> 7;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (q < nq) {
      const float *qq = qr[q] + h * 16;
      float acc = 0.0f;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        acc = fmaf(bf16_lo(w[k].x), qq[8 * k + 0], acc);
        acc = fmaf(bf16_hi(w[k].x), qq[8 * k + 1], acc);
        acc = fmaf(bf16_lo(w[k].y), qq[8 * k + 2], acc);
        acc = fmaf(bf16_hi(w[k].y), qq[8 * k + 3], acc);
        acc = fmaf(bf16_lo(w[k].z), qq[8 * k + 4], acc);
        acc = fmaf(bf16_hi(w[k].z), qq[8 * k + 5], acc);
        acc = fmaf(bf16_lo(w[k].w), qq[8 * k + 6], acc);
        acc = fmaf(bf16_hi(w[k].w), qq[8 * k + 7], acc);
      }
      part[h * 4 + q][i] = acc;
    }
  }
  __syncthreads();
  for (int o = threadIdx.x; o < nq * 128; o += 1024) {
    const int q = o >> 7, r = o & 127;
    float acc = 0.0f;
#pragma unroll
    for (int hh = 0; hh < 8; ++hh) acc += part[hh * 4 + q][r];
    sq[q][r] = acc;
  }
}

template <int NT, int NQ>
__device__ __forceinline__ void sq_rows128(const uint16_t *s_mat, const float (*qr)[128], float (*sq)[128],
                                           float (*part)[128], int nq) {
  constexpr int P = NT / 128;                       // column parts
  constexpr int C = 128 / P;                        // columns per part
  const int i = threadIdx.x & 127, h = threadIdx.x >> 7;
  constexpr int KB = C / 8 < 2 ? C / 8 : 2;          // 16-byte loads in flight
  const uint4 *src = reinterpret_cast<const uint4 *>(s_mat + i * 128 + h * C);
  float acc[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) acc[q] = 0.0f;
#pragma unroll
  for (int k0 = 0; k0 < C / 8; k0 += KB) {
    // at most KB loads in flight: the sums so far are complete here, and
    // later loads may not move above this point
    if constexpr (NQ == 1) {
      asm volatile("" : "+v"(acc[0]) : : "memory");
    } else {
      static_assert(NQ == 4, "one or four queries");
      asm volatile("" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]) : : "memory");
    }
    uint4 w[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) w[k] = src[k0 + k];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      if (q < nq) {
        const float *qq = qr[q] + h * C + 8 * k0;
#pragma unroll
        for (int k = 0; k < KB; ++k) {
          acc[q] = fmaf(bf16_lo(w[k].x), qq[8 * k + 0], acc[q]);
          acc[q] = fmaf(bf16_hi(w[k].x), qq[8 * k + 1], acc[q]);
          acc[q] = fmaf(bf16_lo(w[k].y), qq[8 * k + 2], acc[q]);
          acc[q] = fmaf(bf16_hi(w[k].y), qq[8 * k + 3], acc[q]);
          acc[q] = fmaf(bf16_lo(w[k].z), qq[8 * k + 4], acc[q]);
          acc[q] = fmaf(bf16_hi(w[k].z), qq[8 * k + 5], acc[q]);
          acc[q] = fmaf(bf16_lo(w[k].w), qq[8 * k + 6], acc[q]);
          acc[q] = fmaf(bf16_hi(w[k].w), qq[8 * k + 7], acc[q]);
        }
      }
    }
  }
#pragma unroll
  for (int q = 0; q < NQ; ++q)
    if (q < nq) part[h * NQ + q][i] = acc[q];
  __syncthreads();
  for (int o = threadIdx.x; o < nq * 128; o += NT) {
    const int q = o >> 7, r = o & 127;
    float acc = 0.0f;
#pragma unroll
    for (int hh = 0; hh < P; ++hh) acc += part[hh * NQ + q][r];
    sq[q][r] = acc;
  }
}

// ---------------------------------------------------------------- int8 estimate

// With at most two code bits the estimate is linear in the raw bits of a
// key's record.  For m = 2 and the symmetric centroids (-c1, -c0, c0, c1),
// idx = 2 M + L (M the top, L the bottom code bit):
//   c[idx] = -c1 + (c0 + c1) M + (c1 - c0) L;
// for m = 1, c[idx] = -c0 + 2 c0 b; and a QJL sign is z = 2 b - 1.  So
//   sum_j q'_j c[idx_j] = -c1 sum q' + sum_j ((c0 + c1) q'_j M_j + (c1 - c0) q'_j L_j)
// (m = 1: -c0 sum q' + sum_j 2 c0 q'_j b_j) and sum_i (S q')_i z_i =
// 2 sum_i (S q')_i b_i - sum S q': sums of query weights over the set bits.
// They run exactly on v_mfma_i32_16x16x64_i8.  A bit becomes a byte by one
// AND per four: w & (0x01010101 << 2 t) keeps bits 8 b + 2 t (b = 0..3) with
// byte values 4^t, (w >> 1) & (0x01010101 << 2 t) bits 8 b + 2 t + 1.  Each
// bit's weight -- coefficient times query coordinate, divided by its byte
// value 4^t -- is put in fixed point, w -> round(w 2^e) with |w 2^e| < 2^30,
// as four signed base-256 digits, one per row of the A operand (row 4 q + l:
// query q, digit l); all the mse bits of a key accumulate into one sum and
// the QJL bits into another.  Lane (k, key) of the output holds query k's
// four digit sums for that key, recombined in float32.  (Rounding a weight
// moves a sum by at most 2^-24 of the largest weight per bit, far inside
// the 1e-4 bar.)  A 2-bit code word (16
// coordinates) gives its coordinates 4 b + t; a 1-bit plane word (32
// coordinates) its bits 8 b + 2 t (even) and 8 b + 2 t + 1 (odd).  Lane
// (k, key) of the B operand takes coordinates 32 k .. 32 k + 31 of its key:
// 2-bit code words 2 k and 2 k + 1, plane word k.

typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4 mfma_i8(const uint32_t (&a)[4], const uint32_t (&b)[4], i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(i32x4{(int)a[0], (int)a[1], (int)a[2], (int)a[3]},
                                               i32x4{(int)b[0], (int)b[1], (int)b[2], (int)b[3]}, c, 0, 0, 0);
}

// float of the four digit sums d[l] (weights 256^l).  With at most 256
// bits per sum and byte values up to 64, d0 + 256 d1 is an exact int32
// below 2^30 whose conversion loses at most 2^-24 of the largest weight,
// and d2 + 256 d3 stays below 2^24 (the whole sum is below 2^38 units), so
// it converts exactly: two conversions and one FMA
__device__ __forceinline__ float digits(const i32x4 &d) {
  const float lo = static_cast<float>(d[0] + (d[1] << 8));
  const float hi = static_cast<float>(d[2] + (d[3] << 8));
  return fmaf(65536.0f, hi, lo);
}

// the bytes of a word: plane[t] = bits 8 b + 2 t (+1 for ODD), value 4^t
template <bool ODD>
__device__ __forceinline__ void bytes_of(uint32_t w, uint32_t (&bt)[4]) {
  const uint32_t v = ODD ? w >> 1 : w;
#pragma unroll
  for (int t = 0; t < 4; ++t) bt[t] = v & (0x01010101u << (2 * t));
}

constexpr int kI8Ops = 6;   // A operands: 0..3 code bits (m = 2: L and M of words 0, 1; m = 1: even, odd), 4, 5 QJL

// The mse coefficients of the bits: m = 2: c1 - c0 for L, c0 + c1 for M;
// m = 1: 2 c0 for both; m = 0: none.
template <int M>
__device__ __forceinline__ void i8_coefs(const float *centroids, float &cA, float &cB) {
  if constexpr (M == 2) {
    cA = centroids[3] - centroids[2];
    cB = centroids[3] + centroids[2];
  } else if constexpr (M == 1) {
    cA = cB = 2.0f * centroids[1];
  } else {
    cA = cB = 0.0f;
  }
}

// The estimate's constant term: -c1 sum q' (m = 2), -c0 sum q' (m = 1).
template <int M>
__device__ __forceinline__ float i8_offset(const float *centroids, float qsum) {
  return M == 2 ? -centroids[3] * qsum : M == 1 ? -centroids[1] * qsum : 0.0f;
}

// 2^-e of a vector whose largest weight is mx (weights times 2^e below 2^30).
__device__ __forceinline__ int i8_exp(float mx) { return mx > 0.0f ? 29 - ilogbf(mx) : 0; }
__device__ __forceinline__ float i8_scale(float mx) { return mx > 0.0f ? ldexpf(1.0f, ilogbf(mx) - 29) : 0.0f; }

// Fixed-point A operands of up to four queries (q' rows in qr, S q' rows in
// sq for prod; nqb live) into a_lds ([operand][lane][16 bytes], lane order),
// and for each vector v = 4 p + q (p = 0: q', p = 1: S q') its largest
// weight vmax[v] and its coordinate sum vsum[v].  Every thread of the
// NT-thread block calls it; the results are complete when it returns (it
// ends with a barrier), and qr / sq must be complete when it is called.
template <int M, bool PROD, int NT>
__device__ __forceinline__ void i8_query_operands(const float (*qr)[128], const float (*sq)[128], int nqb,
                                                  float cA, float cB, uint32_t (*a_lds)[64][4], float *vmax,
                                                  float *vsum) {
  static_assert(NT % 64 == 0, "whole waves");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // largest weight and sum of each vector, one wave per vector
  for (int v = wave; v < 8; v += NT / 64) {
    const int p = v >> 2, q = v & 3;
    const bool have = q < nqb && (p == 0 ? M >= 1 : PROD);
    const float *src = p == 0 ? qr[q] : sq[PROD ? q : 0];
    const float x0 = have ? src[lane] : 0.0f, x1 = have ? src[64 + lane] : 0.0f;
    float mx = fmaxf(fabsf(x0), fabsf(x1)) * (p == 0 ? fmaxf(cA, cB) : 1.0f);
    float sm = x0 + x1;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      mx = fmaxf(mx, __shfl_xor(mx, off));
      sm += __shfl_xor(sm, off);
    }
    if (lane == 0) {
      vmax[v] = mx;
      vsum[v] = sm;
    }
  }
  __syncthreads();
  // balanced base-256 digits of round(weight 2^e), written where lane
  // (k, 4 q + l) of operand op reads byte `byte`
  for (int it = threadIdx.x; it < 1024; it += NT) {
    const int pv = it >> 9, qv = (it >> 7) & 3, jv = it & 127;
    const bool have = qv < nqb && (pv == 0 ? M >= 1 : PROD);
    const float v = have ? (pv == 0 ? qr[qv][jv] : sq[PROD ? qv : 0][jv]) : 0.0f;
    const int e = i8_exp(vmax[4 * pv + qv]);
    auto put = [&](float wgt, int op, int byte) {
      int r = __float2int_rn(ldexpf(wgt, e));
      uint8_t *dst = reinterpret_cast<uint8_t *>(&a_lds[op][16 * (jv >> 5) + 4 * qv][0]) + byte;
#pragma unroll
      for (int l = 0; l < 4; ++l) {
        const int dl = l < 3 ? ((r + 128) & 255) - 128 : r;
        r = (r - dl) >> 8;
        dst[16 * l] = static_cast<uint8_t>(dl);
      }
    };
    if (pv == 0 && M == 2) {
      // code word (jv >> 4) & 1, coordinate 4 b + t of it: byte 4 t + b, value 4^t
      const int h = (jv >> 4) & 1, b = (jv >> 2) & 3, t = jv & 3;
      const float inv4t = 1.0f / static_cast<float>(1 << (2 * t));
      put(cA * v * inv4t, h, 4 * t + b);        // L
      put(cB * v * inv4t, 2 + h, 4 * t + b);    // M
    } else {
      // plane bit 8 b + 2 t + odd of word jv >> 5: byte 4 t + b, value 4^t
      const int odd = jv & 1, b = (jv >> 3) & 3, t = (jv >> 1) & 3;
      const float inv4t = 1.0f / static_cast<float>(1 << (2 * t));
      put((pv == 0 ? cA : 1.0f) * v * inv4t, (pv == 0 ? 0 : 4) + odd, 4 * t + b);
    }
  }
  __syncthreads();
}

}  // namespace
}  // namespace tq
