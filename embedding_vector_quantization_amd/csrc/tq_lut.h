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
__device__ __forceinline__ void rotate_query128(const float *q, int d_in, int rot_kind, const int8_t *signs,
                                                const float *rot, float *dst, int lane) {
  const int j0 = 2 * lane, j1 = 2 * lane + 1;
  float v0 = j0 < d_in ? q[j0] : 0.0f;
  float v1 = j1 < d_in ? q[j1] : 0.0f;
  if (rot_kind == TQ_ROT_GIVENS) {
    const float c = rot[j0], s = rot[j1];
    const float y0 = fmaf(c, v0, -s * v1), y1 = fmaf(s, v0, c * v1);
    v0 = y0;
    v1 = y1;
  } else if (rot_kind == TQ_ROT_QUAT) {
    const float o0 = __shfl_xor(v0, 1), o1 = __shfl_xor(v1, 1);
    const bool hi = lane & 1;                         // this lane holds coordinates 2, 3 of the quad
    const float a = hi ? o0 : v0, b = hi ? o1 : v1, c = hi ? v0 : o0, d = hi ? v1 : o1;
    const float *p = rot + 4 * (lane >> 1);
    const float w = p[0], x = p[1], y = p[2], z = p[3];
    if (hi) {
      v0 = y * a + z * b + w * c - x * d;
      v1 = z * a - y * b + x * c + w * d;
    } else {
      v0 = w * a - x * b - y * c - z * d;
      v1 = x * a + w * b - z * c + y * d;
    }
  } else {
    v0 = signs[j0] < 0 ? -v0 : v0;
    v1 = signs[j1] < 0 ? -v1 : v1;
    fwht128_wave(v0, v1, lane);
    const float rsd = 0.08838834764831845f;          // 1 / sqrt(128)
    v0 *= rsd;
    v1 *= rsd;
  }
  dst[j0] = v0;
  dst[j1] = v1;
}

// s = S q' for rows 0 .. nq-1 (nq <= NQ) of qr (LDS, [.][128]) into sq, S
// bfloat16 [128][128] row-major, by all NT threads of the block: thread t
// takes row t % 128 and a contiguous 1/(NT/128) of its columns, with up to
// two 16-byte loads of S in flight, and leaves one partial sum per query in part
// ([NT/128 * NQ][128], LDS); the partials are then added in a fixed order.
// qr must be complete before the call; sq is complete after the next
// barrier.
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

}  // namespace
}  // namespace tq
