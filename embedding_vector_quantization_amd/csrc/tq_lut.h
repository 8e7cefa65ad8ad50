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

}  // namespace
}  // namespace tq
