// TurboQuant_mse / TurboQuant_prod encode for gfx950.
//
// Sources: "TurboQuant: Online Vector Quantization" paper summary (Jump2Paper
// Archive) -- the mse variant (random rotation, then the Lloyd-Max scalar
// quantiser of the Lemma 1 density per coordinate), the definitions table
// (b*d bits per vector), Definition 1 (QJL map sign(S x)) and Theorem D_prod
// ((b-1)-bit mse code plus one QJL bit of the residual); AI Trends video
// summary chapter 04:24 (L2 normalise, multiply by the randomised Hadamard
// matrix); GeekNews Hacker News thread (the Hadamard rotation in
// O(d log d)).
//
// One wave encodes 64/LPV vectors at a time, LPV = d/32 lanes per vector,
// 32 contiguous coordinates per lane:
//   1. coalesced 16-byte global loads of the wave's rows, staged through a
//      wave-private LDS region so each lane gets its 32 coordinates;
//   2. n^2 = sum x^2 (lane FMAs, then a butterfly sum over the LPV lanes);
//   3. sign flip (XOR of the float sign bit), Walsh-Hadamard transform: 5
//      butterfly stages inside the lane, log2(LPV) across lanes (DPP /
//      ds_swizzle);
//   4. y = h * sign / (n sqrt d); the m-bit code is decided in float32:
//      MSB = [y >= 0], magnitude level by a binary search of |y| over the
//      positive thresholds (registers for m <= 4, LDS above);
//   5. the lane's 32 codes are appended bit by bit into exactly m dwords of
//      the dense record, which the lane stores directly.
// TurboQuant_prod then forms r = y - c[idx] and gamma = ||r||, writes r to
// LDS split into three bfloat16 parts (hi + mid + lo == r exactly), and
// computes S r for 16 vectors at a time with v_mfma_f32_16x16x32_bf16 (S is
// stored in bfloat16, so every product is exact and accumulation is fp32).
// Lane (g, c) of the MFMA output owns outputs [c d/16, (c+1) d/16) of rows
// 4g..4g+3, i.e. whole bytes of the QJL plane.

#include <hip/hip_runtime.h>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
// Per-wave LDS: staging of 64 lanes x (128 B + 16 B pad) for float32 input;
// the prod path reuses it for the three bfloat16 residual tiles.
constexpr int kStageBytes = 64 * (kEPL * 4 + 16);                  // 9216
constexpr int kTilePad = 8;                                         // bf16 elements per tile row
// three bfloat16 tiles of vpw rows x (d + pad), vpw * d == 2048, vpw <= 16
constexpr int kProdTileBytes = 3 * (2048 + 16 * kTilePad) * 2;      // 13056
constexpr int kWaveLds = kStageBytes > kProdTileBytes ? kStageBytes : kProdTileBytes;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int M>
struct PosThr {
  static constexpr int kCount = (M >= 2 && M <= 4) ? (1 << (M - 1)) - 1 : 0;
  float t[kCount > 0 ? kCount : 1];
};

// Magnitude level L = #{positive thresholds t : a >= t}, m - 1 bits, found by
// binary search; bits[k] is bit k of L.
template <int M>
__device__ __forceinline__ int mag_level(float a, const PosThr<M> &tp, const float *tp_lds) {
  if constexpr (M <= 1) {
    return 0;
  } else if constexpr (M == 2) {
    return a >= tp.t[0] ? 1 : 0;
  } else if constexpr (M == 3) {
    const bool l1 = a >= tp.t[1];
    const float t = l1 ? tp.t[2] : tp.t[0];
    const bool l0 = a >= t;
    return (l1 ? 2 : 0) | (l0 ? 1 : 0);
  } else if constexpr (M == 4) {
    const bool l2 = a >= tp.t[3];
    const float t1 = l2 ? tp.t[5] : tp.t[1];
    const bool l1 = a >= t1;
    const float t0 = l2 ? (l1 ? tp.t[6] : tp.t[4]) : (l1 ? tp.t[2] : tp.t[0]);
    const bool l0 = a >= t0;
    return (l2 ? 4 : 0) | (l1 ? 2 : 0) | (l0 ? 1 : 0);
  } else {
    int level = 0;
#pragma unroll
    for (int bit = M - 2; bit >= 0; --bit) {
      const int probe = level + (1 << bit) - 1;
      if (a >= tp_lds[probe]) level += 1 << bit;
    }
    return level;
  }
}

// r -> (hi, mid, lo) bfloat16 with hi + mid + lo == r exactly: each part
// keeps the top 8 significant bits of what is left (truncation), and the
// remainders are exact float32 differences.
__device__ __forceinline__ void split3(float r, uint16_t &hi, uint16_t &mid, uint16_t &lo) {
  const uint32_t b0 = __float_as_uint(r);
  const float h = __uint_as_float(b0 & 0xFFFF0000u);
  const float r1 = r - h;
  const uint32_t b1 = __float_as_uint(r1);
  const float md = __uint_as_float(b1 & 0xFFFF0000u);
  const float r2 = r1 - md;
  hi = static_cast<uint16_t>(b0 >> 16);
  mid = static_cast<uint16_t>(b1 >> 16);
  lo = static_cast<uint16_t>(__float_as_uint(r2) >> 16);
}

template <int M, bool PROD>
__global__ void __launch_bounds__(kThreads) encode_kernel(EncodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kWaves * kWaveLds];
  __shared__ float tp_lds[128];
  __shared__ float cb_lds[256];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int log_lpv = a.log_lpv;
  const int sub = lane & ((1 << log_lpv) - 1);
  const int vslot = lane >> log_lpv;
  const int vpw = 64 >> log_lpv;
  uint8_t *stage = lds + wave * kWaveLds;

  constexpr int K = 1 << M;
  constexpr int H = K >> 1;
  PosThr<M> tp;
  if constexpr (M >= 2 && M <= 4) {
#pragma unroll
    for (int k = 0; k < PosThr<M>::kCount; ++k) tp.t[k] = a.thresholds[H + k];
  }
  if constexpr (M >= 5) {
    for (int k = threadIdx.x; k < H - 1; k += kThreads) tp_lds[k] = a.thresholds[H + k];
  }
  if constexpr (PROD && M >= 1) {
    for (int k = threadIdx.x; k < K; k += kThreads) cb_lds[k] = a.centroids[k];
  }
  __syncthreads();

  // XOR masks of the sign vector for this lane's coordinates.
  uint32_t smask[kEPL];
#pragma unroll
  for (int e = 0; e < kEPL; ++e) smask[e] = a.signs[sub * kEPL + e] < 0 ? 0x80000000u : 0u;

  const float inv_sqrt_d = 1.0f / sqrtf(static_cast<float>(a.d));
  const float sigma = cross_sign(sub);
  const int64_t groups = (a.n + vpw - 1) / vpw;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kWaves;
  const size_t rec_bytes = static_cast<size_t>(M) * a.d / 8;

  for (int64_t grp = static_cast<int64_t>(blockIdx.x) * kWaves + wave; grp < groups; grp += stride) {
    const int64_t base_row = grp * vpw;
    const int64_t row = base_row + vslot;
    float xv[kEPL];
    RowSpan src{a.x, a.ld_x, a.n, a.d_in, a.dtype};
    if (a.vec_loads) {
      load_rows_staged(src, base_row, a.log_lpv, lane, stage, xv);
      if (a.d_in < a.d) {
#pragma unroll
        for (int e = 0; e < kEPL; ++e)
          if (sub * kEPL + e >= a.d_in) xv[e] = 0.0f;
      }
    } else {
      load_rows_direct(src, row, sub, xv);
    }

    // 2. squared norm
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
    for (int e = 0; e < kEPL; e += 4) {
      s0 = fmaf(xv[e], xv[e], s0);
      s1 = fmaf(xv[e + 1], xv[e + 1], s1);
      s2 = fmaf(xv[e + 2], xv[e + 2], s2);
      s3 = fmaf(xv[e + 3], xv[e + 3], s3);
    }
    const float ss = group_sum((s0 + s1) + (s2 + s3), log_lpv);

    // 3. rotation
#pragma unroll
    for (int e = 0; e < kEPL; ++e) xv[e] = __uint_as_float(__float_as_uint(xv[e]) ^ smask[e]);
    fwht_lane(xv);
    fwht_cross(xv, log_lpv, lane);
    const float nrm = sqrtf(ss);
    const float scale = ss > 0.0f ? sigma * inv_sqrt_d / nrm : 0.0f;
#pragma unroll
    for (int e = 0; e < kEPL; ++e) xv[e] *= scale;   // xv now holds y

    // 4-5. codes
    float rr = 0.0f;
    if constexpr (M >= 1) {
      uint32_t words[M];
#pragma unroll
      for (int w = 0; w < M; ++w) words[w] = 0u;
#pragma unroll
      for (int e = kEPL - 1; e >= 0; --e) {
        const float y = xv[e];
        const bool pos = y >= 0.0f;
        const int level = mag_level<M>(fabsf(y), tp, tp_lds);
        // stream bits M*e + M-1 .. M*e, appended from the top
#pragma unroll
        for (int p = M - 1; p >= 0; --p) {
          const int s = M * e + p;
          bool bit;
          if (p == M - 1) bit = pos;
          else bit = (((level >> p) & 1) != 0) != !pos;
          words[s >> 5] = append_bit(words[s >> 5], bit);
        }
        if constexpr (PROD) {
          const int idx = pos ? (H + level) : (H - 1 - level);
          const float r = y - cb_lds[idx];
          xv[e] = r;
          rr = fmaf(r, r, rr);
        }
      }
      if (row < a.n) {
        uint32_t *dst = reinterpret_cast<uint32_t *>(a.codes + row * rec_bytes) + sub * M;
#pragma unroll
        for (int w = 0; w < M; ++w) dst[w] = words[w];
      }
    } else {
#pragma unroll
      for (int e = 0; e < kEPL; ++e) rr = fmaf(xv[e], xv[e], rr);
    }
    if (sub == 0 && row < a.n) a.norms[row] = nrm;

    if constexpr (PROD) {
      const float g2 = group_sum(rr, log_lpv);
      if (sub == 0 && row < a.n) a.rnorms[row] = sqrtf(g2);

      if (a.d < 128) {
        // Small d: S r on the vector ALU in float32 from an LDS copy of r.
        float *rt = reinterpret_cast<float *>(stage);    // [vpw][d]
#pragma unroll
        for (int e = 0; e < kEPL; ++e) rt[vslot * a.d + sub * kEPL + e] = xv[e];
        wave_lds_sync();
        uint32_t bits = 0u;
        for (int o = kEPL - 1; o >= 0; --o) {
          const int out = sub * kEPL + o;
          const uint16_t *srow = a.qjl_s + static_cast<int64_t>(out) * a.d;
          float acc = 0.0f;
          for (int j = 0; j < a.d; ++j)
            acc = fmaf(__uint_as_float(static_cast<uint32_t>(srow[j]) << 16), rt[vslot * a.d + j], acc);
          bits = append_bit(bits, acc >= 0.0f);
        }
        if (row < a.n) reinterpret_cast<uint32_t *>(a.qjl + row * (a.d / 8))[sub] = bits;
        wave_lds_sync();
      } else {
        // d >= 128: vpw <= 16 rows, one MFMA row tile.
        const int dpad = a.d + kTilePad;                 // bf16 elements per tile row
        uint16_t *th = reinterpret_cast<uint16_t *>(stage);
        uint16_t *tm = th + vpw * dpad;
        uint16_t *tl = tm + vpw * dpad;
#pragma unroll
        for (int e = 0; e < kEPL; ++e) {
          uint16_t h, md, lo;
          split3(xv[e], h, md, lo);
          const int off = vslot * dpad + sub * kEPL + e;
          th[off] = h;
          tm[off] = md;
          tl[off] = lo;
        }
        wave_lds_sync();
        const int fr = lane & 15;                 // MFMA row (A) / column (B)
        const int fk = (lane >> 4) * 8;           // k offset inside a 32-wide chunk
        const bool row_ok = fr < vpw;
        const int ntiles = a.d >> 4;
        const int kchunks = a.d >> 5;
        const int bits_per = ntiles;              // output bits per (lane, row)
        // outputs of this lane: [fr * ntiles, fr * ntiles + ntiles) ; tile nt
        // holds output fr * ntiles + nt.
        uint32_t qb[4][4];                        // up to 128 bits per row (d <= 2048)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int w = 0; w < 4; ++w) qb[i][w] = 0u;
        for (int nt = ntiles - 1; nt >= 0; --nt) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          const uint16_t *srow = a.qjl_s + static_cast<int64_t>(fr * ntiles + nt) * a.d + fk;
          for (int kc = 0; kc < kchunks; ++kc) {
            const bf16x8 b = *reinterpret_cast<const bf16x8 *>(srow + kc * 32);
            bf16x8 ah, am, al;
            if (row_ok) {
              const int off = fr * dpad + kc * 32 + fk;
              ah = *reinterpret_cast<const bf16x8 *>(th + off);
              am = *reinterpret_cast<const bf16x8 *>(tm + off);
              al = *reinterpret_cast<const bf16x8 *>(tl + off);
            } else {
              ah = am = al = bf16x8{};
            }
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, b, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am, b, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, b, acc, 0, 0, 0);
          }
          const int w = nt >> 5;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool bit = acc[i] >= 0.0f;
            // append into word w of row i (bits arrive from nt high to low)
            if (w == 0) qb[i][0] = append_bit(qb[i][0], bit);
            else if (w == 1) qb[i][1] = append_bit(qb[i][1], bit);
            else if (w == 2) qb[i][2] = append_bit(qb[i][2], bit);
            else qb[i][3] = append_bit(qb[i][3], bit);
          }
        }
        // Row 4g + i, bits [fr * ntiles, fr * ntiles + ntiles) of the plane.
        const int g = lane >> 4;
        const int nbytes = bits_per >> 3;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * g + i;
          const int64_t orow = base_row + r;
          if (r < vpw && orow < a.n) {
            uint8_t *dst = a.qjl + orow * (a.d / 8) + fr * nbytes;
            for (int bb = 0; bb < nbytes; ++bb) dst[bb] = static_cast<uint8_t>(qb[i][bb >> 2] >> (8 * (bb & 3)));
          }
        }
        wave_lds_sync();
      }
    }
  }
}

template <bool PROD>
int launch_m(const EncodeArgs &a, hipStream_t s, dim3 grid) {
  switch (a.m) {
#define TQ_CASE(MM)                                                              \
  case MM:                                                                       \
    hipLaunchKernelGGL((encode_kernel<MM, PROD>), grid, dim3(kThreads), 0, s, a); \
    break;
    TQ_CASE(1) TQ_CASE(2) TQ_CASE(3) TQ_CASE(4) TQ_CASE(5) TQ_CASE(6) TQ_CASE(7)
    case 8:
      if constexpr (!PROD) {
        hipLaunchKernelGGL((encode_kernel<8, false>), grid, dim3(kThreads), 0, s, a);
        break;
      }
      return hipErrorInvalidValue;
    case 0:
      if constexpr (PROD) {
        hipLaunchKernelGGL((encode_kernel<0, true>), grid, dim3(kThreads), 0, s, a);
        break;
      }
      return hipErrorInvalidValue;
#undef TQ_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int launch_encode(const EncodeArgs &a, bool prod, void *stream) {
  (void)hipGetLastError();   // report only errors of this launch
  const int vpw = 64 >> a.log_lpv;
  const int64_t groups = (a.n + vpw - 1) / vpw;
  const int64_t blocks_needed = (groups + kWaves - 1) / kWaves;
  const int64_t max_blocks = 256 * 8;
  const dim3 grid(static_cast<unsigned>(blocks_needed < max_blocks ? blocks_needed : max_blocks));
  hipStream_t s = static_cast<hipStream_t>(stream);
  return prod ? launch_m<true>(a, s, grid) : launch_m<false>(a, s, grid);
}

}  // namespace tq
