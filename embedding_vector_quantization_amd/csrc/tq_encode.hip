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
//      ds_swizzle); 16-bit input at d = 128 is never widened element by
//      element: packed dot products of each element pair with its signs give
//      the first two stages, and the squares for n^2;
//   4. y = h * sign / (n sqrt d); the m-bit code is decided in float32:
//      MSB = [y >= 0], magnitude level by a binary search of |y| over the
//      positive thresholds (registers for m <= 4, LDS above);
//   5. the lane's 32 codes are appended bit by bit into exactly m dwords of
//      the dense record (one v_addc per bit, the wave mask of the compare as
//      carry-in), which the lane stores directly.
// TurboQuant_prod then forms r = y - c[idx] and gamma = ||r||, and computes
// S r on the matrix cores for 16 vectors at a time: at d = 128 with
// v_mfma_f32_16x16x32_f16 on a two-part float16 split of 2^14 r against an
// LDS float16 copy of S; otherwise with v_mfma_f32_16x16x32_bf16 on an exact
// three-part bfloat16 split of r against S (bfloat16 in memory: every product
// exact, fp32 accumulation).  Lane (g, c) of the MFMA output owns outputs
// [c d/16, (c+1) d/16) of rows 4g..4g+3, i.e. whole bytes of the QJL plane
// (at d = 128 built from the sign bits of S r, one v_alignbit per bit).
//
// Two kernels share these steps: a specialised one for d = d_in = 128 with
// aligned rows (compile-time lane layout and input type, precomputed staging
// addresses, the next group's loads in flight while the current group is
// computed), and a general one for any d in [32, 2048], d_in <= d, any row
// stride.

#include <hip/hip_runtime.h>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
// The d = 128 TurboQuant_prod kernel runs 12 waves per workgroup: one copy
// of S (32 KiB) then serves 12 wave stages, and three waves fit per SIMD.
constexpr int kWaves128P = 12;
// Per-wave LDS: staging of 64 lanes x (128 B + 16 B pad) for float32 input;
// the prod path reuses it for the three bfloat16 residual tiles.
constexpr int kStageBytes = 64 * (kEPL * 4 + 16);                  // 9216
constexpr int kTilePad = 8;                                         // bf16 elements per tile row
// three bfloat16 tiles of vpw rows x (d + pad), vpw * d == 2048, vpw <= 16
constexpr int kProdTileBytes = 3 * (2048 + 16 * kTilePad) * 2;      // 13056
constexpr int kProdWaveLds = kStageBytes > kProdTileBytes ? kStageBytes : kProdTileBytes;
// d = 4096: the three tiles of one row span the two stages of a wave pair
static_assert(2 * kProdWaveLds >= 3 * (4096 + kTilePad) * 2, "paired prod tiles");

template <bool PROD>
constexpr int wave_lds() { return PROD ? kProdWaveLds : kStageBytes; }

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int M>
struct PosThr {
  static constexpr int kCount = (M >= 2 && M <= 4) ? (1 << (M - 1)) - 1 : 0;
  float t[kCount > 0 ? kCount : 1];
};

template <int M>
struct PosCent {                     // positive centroids c[H..K-1], m <= 4
  static constexpr int kCount = (M >= 1 && M <= 4) ? (1 << (M - 1)) : 0;
  float c[kCount > 0 ? kCount : 1];
};

// Magnitude level L = #{positive thresholds t : a >= t} by binary search over
// the LDS copy of the positive thresholds (m >= 5).
template <int M>
__device__ __forceinline__ int mag_level_lds(float a, const float *tp_lds) {
  int level = 0;
#pragma unroll
  for (int bit = M - 2; bit >= 0; --bit) {
    const int probe = level + (1 << bit) - 1;
    if (a >= tp_lds[probe]) level += 1 << bit;
  }
  return level;
}

// Codes of the lane's 32 rotated coordinates y (in xv) into M words: for
// coordinate e, stream bits M e + M-1 .. M e are appended from the top, so
// the words come out in the record's little-endian order.  Code bits: MSB =
// [y >= 0]; low bits = L xor (y < 0 ? all ones : 0).  For prod, xv is
// replaced by the residual and rr accumulates its square.
// SCALED (m <= 4): xv holds h = y / s for a per-vector s > 0 (or a zero
// row), tp and pc are the thresholds and centroids in h's units resp. times
// rscale / s, and the residual is formed as h * rscale - c in one FMA
// (rscale = s times a power of two); otherwise y - c.
template <int M, bool PROD, bool SCALED = false>
__device__ __forceinline__ void quantize_lane(float (&xv)[kEPL], const PosThr<M> &tp,
                                              const PosCent<M> &pc, const float *tp_lds,
                                              const float *cb_lds, uint32_t (&words)[M > 0 ? M : 1],
                                              float &rr, float rscale = 1.0f) {
  static_assert(!SCALED || M <= 4, "scaled thresholds live in registers");
  constexpr int H = (1 << M) >> 1;
#pragma unroll
  for (int w = 0; w < (M > 0 ? M : 1); ++w) words[w] = 0u;
  rr = 0.0f;
#pragma unroll
  for (int e = kEPL - 1; e >= 0; --e) {
    float y = xv[e];
    if constexpr (PROD) {
      // The centroid select reuses the compare masks; without this the
      // compiler hoists every element's compares and spills their masks.
      // Making each fourth element's input depend on the running residual
      // sum keeps at most four elements' masks live.
      if ((e & 3) == 3 && e != kEPL - 1) asm volatile("" : "+v"(y) : "v"(rr));
    }
    const float a = fabsf(y);
    const bool pos = y >= 0.0f;
    const uint64_t ms = __builtin_amdgcn_ballot_w64(pos);
    float c = 0.0f;
    if constexpr (M == 1) {
      words[e >> 5] = append_mask(words[e >> 5], ms);
      if constexpr (PROD) c = pos ? pc.c[0] : -pc.c[0];
    } else if constexpr (M == 2) {
      const bool l0 = a >= tp.t[0];
      const uint64_t m0 = __builtin_amdgcn_ballot_w64(l0);
      words[(2 * e + 1) >> 5] = append_mask(words[(2 * e + 1) >> 5], ms);
      words[(2 * e) >> 5] = append_mask(words[(2 * e) >> 5], ~(m0 ^ ms));
      if constexpr (PROD) {
        const float mag = l0 ? pc.c[1] : pc.c[0];
        c = pos ? mag : -mag;
      }
    } else if constexpr (M == 3) {
      const bool l1 = a >= tp.t[1];
      const float t = l1 ? tp.t[2] : tp.t[0];
      const bool l0 = a >= t;
      const uint64_t m1 = __builtin_amdgcn_ballot_w64(l1);
      const uint64_t m0 = __builtin_amdgcn_ballot_w64(l0);
      words[(3 * e + 2) >> 5] = append_mask(words[(3 * e + 2) >> 5], ms);
      words[(3 * e + 1) >> 5] = append_mask(words[(3 * e + 1) >> 5], ~(m1 ^ ms));
      words[(3 * e) >> 5] = append_mask(words[(3 * e) >> 5], ~(m0 ^ ms));
      if constexpr (PROD) {
        const float mag = l1 ? (l0 ? pc.c[3] : pc.c[2]) : (l0 ? pc.c[1] : pc.c[0]);
        c = pos ? mag : -mag;
      }
    } else if constexpr (M == 4) {
      const bool l2 = a >= tp.t[3];
      const float t1 = l2 ? tp.t[5] : tp.t[1];
      const bool l1 = a >= t1;
      const float t0 = l2 ? (l1 ? tp.t[6] : tp.t[4]) : (l1 ? tp.t[2] : tp.t[0]);
      const bool l0 = a >= t0;
      const uint64_t m2 = __builtin_amdgcn_ballot_w64(l2);
      const uint64_t m1 = __builtin_amdgcn_ballot_w64(l1);
      const uint64_t m0 = __builtin_amdgcn_ballot_w64(l0);
      words[(4 * e + 3) >> 5] = append_mask(words[(4 * e + 3) >> 5], ms);
      words[(4 * e + 2) >> 5] = append_mask(words[(4 * e + 2) >> 5], ~(m2 ^ ms));
      words[(4 * e + 1) >> 5] = append_mask(words[(4 * e + 1) >> 5], ~(m1 ^ ms));
      words[(4 * e) >> 5] = append_mask(words[(4 * e) >> 5], ~(m0 ^ ms));
      if constexpr (PROD) {
        const float mag = l2 ? (l1 ? (l0 ? pc.c[7] : pc.c[6]) : (l0 ? pc.c[5] : pc.c[4]))
                             : (l1 ? (l0 ? pc.c[3] : pc.c[2]) : (l0 ? pc.c[1] : pc.c[0]));
        c = pos ? mag : -mag;
      }
    } else if constexpr (M >= 5) {
      const int level = mag_level_lds<M>(a, tp_lds);
#pragma unroll
      for (int p = M - 1; p >= 0; --p) {
        const int s = M * e + p;
        const bool bit = (p == M - 1) ? pos : ((((level >> p) & 1) != 0) != !pos);
        words[s >> 5] = append_bit(words[s >> 5], bit);
      }
      if constexpr (PROD) c = cb_lds[pos ? (H + level) : (H - 1 - level)];
    }
    if constexpr (PROD) {
      const float r = SCALED ? fmaf(y, rscale, -c) : y - c;
      xv[e] = r;
      rr = fmaf(r, r, rr);
    }
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

// QJL plane of the wave's vectors from their residuals (xv of every lane).
__device__ __forceinline__ void qjl_plane(const EncodeArgs &a, int d, int log_lpv, int lane,
                                          int64_t base_row, uint8_t *stage, const float (&xv)[kEPL]) {
  const int sub = lane & ((1 << log_lpv) - 1);
  const int vslot = lane >> log_lpv;
  const int vpw = 64 >> log_lpv;
  const int64_t row = base_row + vslot;
  if (d < 128) {
    // Small d: S r on the vector ALU in float32 from an LDS copy of r.
    float *rt = reinterpret_cast<float *>(stage);    // [vpw][d]
#pragma unroll
    for (int e = 0; e < kEPL; ++e) rt[vslot * d + sub * kEPL + e] = xv[e];
    wave_lds_sync();
    uint32_t bits = 0u;
    for (int o = kEPL - 1; o >= 0; --o) {
      const int out = sub * kEPL + o;
      const uint16_t *srow = a.qjl_s + static_cast<int64_t>(out) * d;
      float acc = 0.0f;
      for (int j = 0; j < d; ++j)
        acc = fmaf(__uint_as_float(static_cast<uint32_t>(srow[j]) << 16), rt[vslot * d + j], acc);
      bits = append_bit(bits, acc >= 0.0f);
    }
    if (row < a.n) reinterpret_cast<uint32_t *>(a.qjl + row * (d / 8))[sub] = bits;
    wave_lds_sync();
    return;
  }
  // d >= 128: vpw <= 16 rows, one MFMA row tile.
  const int dpad = d + kTilePad;                   // bf16 elements per tile row
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
  const int ntiles = d >> 4;
  const int kchunks = d >> 5;
  // Tile nt column fr holds output fr * ntiles + nt: this lane collects the
  // bits of outputs [fr * ntiles, fr * ntiles + ntiles) for rows 4g..4g+3.
  uint32_t qb[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int w = 0; w < 4; ++w) qb[i][w] = 0u;
  for (int nt = ntiles - 1; nt >= 0; --nt) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const uint16_t *srow = a.qjl_s + static_cast<int64_t>(fr * ntiles + nt) * d + fk;
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
      if (w == 0) qb[i][0] = append_bit(qb[i][0], bit);
      else if (w == 1) qb[i][1] = append_bit(qb[i][1], bit);
      else if (w == 2) qb[i][2] = append_bit(qb[i][2], bit);
      else qb[i][3] = append_bit(qb[i][3], bit);
    }
  }
  const int g = lane >> 4;
  const int nbytes = ntiles >> 3;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * g + i;
    const int64_t orow = base_row + r;
    if (r < vpw && orow < a.n) {
      uint8_t *dst = a.qjl + orow * (d / 8) + fr * nbytes;
      for (int bb = 0; bb < nbytes; ++bb) dst[bb] = static_cast<uint8_t>(qb[i][bb >> 2] >> (8 * (bb & 3)));
    }
  }
  wave_lds_sync();
}

// QJL plane at d = 4096 (a vector over the two waves of a pair, wave h
// holding coordinates 2048 h + 32 lane + e): both waves write their
// residual's exact three-part bfloat16 split into one row of the pair's
// tiles (its two wave stages, 3 x 4104 elements), then wave h forms outputs
// [2048 h, 2048 h + 2048) as in qjl_plane (output 2048 h + 128 fr + nt in
// tile nt, column fr; only MFMA row 0 is a vector).
__device__ __forceinline__ void qjl_plane_pair(const EncodeArgs &a, int lane, int h, int64_t row, uint8_t *tiles,
                                               const float (&xv)[kEPL]) {
  constexpr int kD = 4096, kPad = kD + kTilePad;
  uint16_t *th = reinterpret_cast<uint16_t *>(tiles);
  uint16_t *tm = th + kPad;
  uint16_t *tl = tm + kPad;
  const int sub = 64 * h + lane;
#pragma unroll
  for (int e = 0; e < kEPL; ++e) {
    uint16_t hi, md, lo;
    split3(xv[e], hi, md, lo);
    th[sub * kEPL + e] = hi;
    tm[sub * kEPL + e] = md;
    tl[sub * kEPL + e] = lo;
  }
  __syncthreads();
  const int fr = lane & 15;
  const int fk = (lane >> 4) * 8;
  uint32_t qb[4] = {0u, 0u, 0u, 0u};
  for (int nt = 127; nt >= 0; --nt) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const uint16_t *srow = a.qjl_s + static_cast<int64_t>(2048 * h + fr * 128 + nt) * kD + fk;
    for (int kc = 0; kc < kD / 32; ++kc) {
      const bf16x8 b = *reinterpret_cast<const bf16x8 *>(srow + kc * 32);
      bf16x8 ah = bf16x8{}, am = bf16x8{}, al = bf16x8{};
      if (fr == 0) {
        ah = *reinterpret_cast<const bf16x8 *>(th + kc * 32 + fk);
        am = *reinterpret_cast<const bf16x8 *>(tm + kc * 32 + fk);
        al = *reinterpret_cast<const bf16x8 *>(tl + kc * 32 + fk);
      }
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, b, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am, b, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, b, acc, 0, 0, 0);
    }
    const bool bit = acc[0] >= 0.0f;      // row 0 of the tile (lanes 0..15)
    const int w = nt >> 5;
    if (w == 0) qb[0] = append_bit(qb[0], bit);
    else if (w == 1) qb[1] = append_bit(qb[1], bit);
    else if (w == 2) qb[2] = append_bit(qb[2], bit);
    else qb[3] = append_bit(qb[3], bit);
  }
  if (lane < 16 && row < a.n) {
    uint32_t *dst = reinterpret_cast<uint32_t *>(a.qjl + row * (kD / 8) + 256 * h + 16 * fr);
#pragma unroll
    for (int w = 0; w < 4; ++w) dst[w] = qb[w];
  }
  __syncthreads();
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// S for d = 128 as float16 in LDS, 256 bytes per row o, 16-byte chunk c
// stored at chunk c ^ ((o >> 3) & 15): the 16 lanes fr = 0..15 that read
// rows 8 fr + nt of one chunk together then cover all 64 banks once.  A
// bfloat16 value converts exactly unless its magnitude is below 2^-17 (a
// float16 subnormal step of 2^-24) or above 65504 (the conversion rounds
// toward zero, so such a value becomes 65504).
constexpr int kS16Bytes = 128 * 256;

__device__ __forceinline__ int s16_offset(int o, int chunk) {
  return o * 256 + ((chunk ^ ((o >> 3) & 15)) << 4);
}

// The layout the matrix-core transform kernel reads S in: 16-byte chunk c
// of row o at chunk c ^ ((o & 3) | ((o >> 5) & 3) << 2), so that the 16
// lanes reading rows 32 (r >> 2) + 4 nt + (r & 3), r = 0..15, of one chunk
// cover all 64 banks once.
__device__ __forceinline__ int s16h_offset(int o, int chunk) {
  return o * 256 + ((chunk ^ ((o & 3) | (((o >> 5) & 3) << 2))) << 4);
}

template <int NT, bool HLAYOUT = false>
__device__ __forceinline__ void load_s16(const uint16_t *s_bf16, uint8_t *s16) {
  for (int ch = threadIdx.x; ch < 128 * 16; ch += NT) {
    const int o = ch >> 4, c = ch & 15;
    const uint4 v = *reinterpret_cast<const uint4 *>(s_bf16 + o * 128 + c * 8);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t outw[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const auto pk = __builtin_amdgcn_cvt_pkrtz(bf16_lo(w[p]), bf16_hi(w[p]));
      __builtin_memcpy(&outw[p], &pk, 4);
    }
    *reinterpret_cast<uint4 *>(s16 + (HLAYOUT ? s16h_offset(o, c) : s16_offset(o, c))) =
        make_uint4(outw[0], outw[1], outw[2], outw[3]);
  }
}

// r - h, h the float16 in half HALF (0 = low) of the packed pair hp, in one
// v_fma_mix_f32 (the float16 operand is widened inside the instruction).
// Exact: h is r rounded toward zero, so r - h is a float32.
template <int HALF>
__device__ __forceinline__ float sub_f16_half(float r, uint32_t hp) {
  float out;
  if constexpr (HALF == 0) {
    asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel:[0,0,0] op_sel_hi:[1,0,0]" : "=v"(out) : "v"(hp), "v"(r));
  } else {
    asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(out) : "v"(hp), "v"(r));
  }
  return out;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// acc + x0 y0 + x1 y1 for packed pairs of 16-bit elements (bfloat16 or
// float16, low half first).  The products of 16-bit values are exact in
// float32; the sum comes out truncated (within one ulp of a float32 add).
template <int DT>
__device__ __forceinline__ float dot2(uint32_t x, uint32_t y, float acc) {
  if constexpr (DT == TQ_BF16) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), __builtin_bit_cast(bf16x2, y), acc, false);
  } else {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, x), __builtin_bit_cast(f16x2, y), acc, false);
  }
}

// Eight 16-bit elements x[0..7] (packed words w[0..3], low half first) with
// their RHT signs s[0..7], through the first two butterfly stages, in 12
// packed dot products.  For the word pair (w0, w1) with g_j = (s_2j, s_2j+1):
//   u0 = (s0, s1).w0, u1 = (s0, -s1).w0          (stage 1 of elements 0, 1)
//   out0 = u0 + (s2, s3).w1, out2 = u0 + (-s2, -s3).w1,
//   out1 = u1 + (s2, -s3).w1, out3 = u1 + (-s2, s3).w1
// (stage 1 of elements 2, 3 inside the stage-2 sums).  Every sign pattern is
// g_j with the neg_lo / neg_hi operand modifiers.  The compiler's own dot2
// form ties the accumulator to the result, which costs a move per output, and
// it does not fold negations, hence the asm.  A dot result read by another vector
// instruction needs three wait states first, which the compiler cannot see
// inside asm: each u is read at least three instructions after it is
// written, and the block ends with s_nop 2 before any output is read.
#define TQ_PAIR_STAGES(OP)                                                          \
  asm(OP " %8, %12, %16, 0\n\t"                                                  \
      OP " %9, %12, %16, 0 neg_hi:[0,1,0]\n\t"                                   \
      OP " %10, %14, %18, 0\n\t"                                                 \
      OP " %11, %14, %18, 0 neg_hi:[0,1,0]\n\t"                                  \
      OP " %0, %13, %17, %8\n\t"                                                 \
      OP " %2, %13, %17, %8 neg_lo:[0,1,0] neg_hi:[0,1,0]\n\t"                   \
      OP " %1, %13, %17, %9 neg_hi:[0,1,0]\n\t"                                  \
      OP " %3, %13, %17, %9 neg_lo:[0,1,0]\n\t"                                  \
      OP " %4, %15, %19, %10\n\t"                                                \
      OP " %6, %15, %19, %10 neg_lo:[0,1,0] neg_hi:[0,1,0]\n\t"                  \
      OP " %5, %15, %19, %11 neg_hi:[0,1,0]\n\t"                                 \
      OP " %7, %15, %19, %11 neg_lo:[0,1,0]\n\t"                                 \
      "s_nop 2"                                                                     \
      : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]), \
        "=&v"(x[6]), "=&v"(x[7]), "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3])  \
      : "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]), "v"(g[0]), "v"(g[1]), "v"(g[2]), "v"(g[3]))

template <int DT>
__device__ __forceinline__ void pair_stages(const uint32_t (&w)[4], const uint32_t *g, float *x) {
  float t[4];
  if constexpr (DT == TQ_BF16) {
    TQ_PAIR_STAGES("v_dot2_f32_bf16");
  } else {
    TQ_PAIR_STAGES("v_dot2_f32_f16");
  }
}
#undef TQ_PAIR_STAGES

// QJL plane for d = 128 (16 vectors per wave): S r with
// v_mfma_f32_16x16x32_f16 on r' = 2^14 r (xv holds r') split as hi + lo
// float16 (the scale keeps hi and lo normal; the sign of S r' is the sign of
// S r).  The
// rounding of the split leaves |r' - hi - lo| <= 2^-21 |r'|, far below the
// decision band of the sign.  Output tile nt, column fr is output 8 fr + nt,
// so lane (g, fr) ends with byte fr of the planes of rows 4g..4g+3.
__device__ __forceinline__ void qjl_plane128(int lane, __amdgpu_buffer_rsrc_t qjl_rows, uint8_t *stage,
                                             const uint8_t *s16, const float (&xv)[kEPL]) {
  constexpr int kRow = 136;                        // float16 elements per tile row
  const int sub = lane & 3;
  const int vslot = lane >> 2;
  uint8_t *thi = stage;                            // [16][kRow] float16
  uint8_t *tlo = stage + 16 * kRow * 2;
  uint32_t hw[16], lw[16];
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    const float r0 = xv[2 * p], r1 = xv[2 * p + 1];
    const auto h = __builtin_amdgcn_cvt_pkrtz(r0, r1);
    __builtin_memcpy(&hw[p], &h, 4);
    const auto l = __builtin_amdgcn_cvt_pkrtz(sub_f16_half<0>(r0, hw[p]), sub_f16_half<1>(r1, hw[p]));
    __builtin_memcpy(&lw[p], &l, 4);
  }
  const int woff = (vslot * kRow + sub * kEPL) * 2;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    *reinterpret_cast<uint4 *>(thi + woff + 16 * q) = make_uint4(hw[4 * q], hw[4 * q + 1], hw[4 * q + 2], hw[4 * q + 3]);
    *reinterpret_cast<uint4 *>(tlo + woff + 16 * q) = make_uint4(lw[4 * q], lw[4 * q + 1], lw[4 * q + 2], lw[4 * q + 3]);
  }
  wave_lds_sync();
  const int fr = lane & 15;
  const int g = lane >> 4;
  f16x8 ahi[4], alo[4];
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) {
    const int roff = (fr * kRow + 32 * kc + 8 * g) * 2;
    ahi[kc] = *reinterpret_cast<const f16x8 *>(thi + roff);
    alo[kc] = *reinterpret_cast<const f16x8 *>(tlo + roff);
  }
  // The sign bits of (S r)_o are shifted in from the top (one v_alignbit
  // each); the plane bit [S r >= 0] is their complement.  S r is never -0:
  // the accumulation starts from +0.
  uint32_t qn[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int nt = 7; nt >= 0; --nt) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int o = 8 * fr + nt;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const f16x8 b = *reinterpret_cast<const f16x8 *>(s16 + s16_offset(o, 4 * kc + g));
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[kc], b, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[kc], b, acc, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) qn[i] = __builtin_amdgcn_alignbit(qn[i], __float_as_uint(acc[i]), 31);
  }
  // byte fr of the planes of rows 4g + i, through the group's ranged buffer
#pragma unroll
  for (int i = 0; i < 4; ++i)
    __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(~qn[i]), qjl_rows, (4 * g + i) * 16 + fr, 0, 0);
  wave_lds_sync();
}

// Loads the per-block constants: positive thresholds and centroids.
template <int M, bool PROD>
__device__ __forceinline__ void load_consts(const EncodeArgs &a, PosThr<M> &tp, PosCent<M> &pc,
                                            float *tp_lds, float *cb_lds) {
  constexpr int K = 1 << M;
  constexpr int H = K >> 1;
  if constexpr (M >= 2 && M <= 4) {
#pragma unroll
    for (int k = 0; k < PosThr<M>::kCount; ++k) tp.t[k] = a.thresholds[H + k];
  }
  if constexpr (PROD && M >= 1 && M <= 4) {
#pragma unroll
    for (int k = 0; k < PosCent<M>::kCount; ++k) pc.c[k] = a.centroids[H + k];
  }
  if constexpr (M >= 5) {
    for (int k = threadIdx.x; k < H - 1; k += kThreads) tp_lds[k] = a.thresholds[H + k];
    if constexpr (PROD) {
      for (int k = threadIdx.x; k < K; k += kThreads) cb_lds[k] = a.centroids[k];
    }
  }
}

// ------------------------------------------------------------ general kernel

template <int M, bool PROD>
__global__ void __launch_bounds__(kThreads) encode_kernel(EncodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kWaves * wave_lds<PROD>()];
  __shared__ float tp_lds[128];
  __shared__ float cb_lds[256];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const Layout L = layout_of(a.log_lpv, kWaves, wave, lane);
  const bool paired = L.paired;
  const int h = L.h, wlog = L.wlog, sub = L.sub, vslot = L.vslot, vpw = L.vpw;
  uint8_t *stage = lds + wave * wave_lds<PROD>();
  uint8_t *partner = lds + (wave ^ 1) * wave_lds<PROD>();

  PosThr<M> tp;
  PosCent<M> pc;
  load_consts<M, PROD>(a, tp, pc, tp_lds, cb_lds);
  __syncthreads();

  // XOR masks of the sign vector for this lane's coordinates.
  uint32_t smask[kEPL];
#pragma unroll
  for (int e = 0; e < kEPL; ++e) smask[e] = a.signs[sub * kEPL + e] < 0 ? 0x80000000u : 0u;

  const float inv_sqrt_d = 1.0f / sqrtf(static_cast<float>(a.d));
  const float sigma = cross_sign(sub & 63);
  const int units = L.units, unit = L.unit;
  const int64_t groups = (a.n + vpw - 1) / vpw;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * units;
  const size_t rec_bytes = static_cast<size_t>(M) * a.d / 8;
  const int esize = a.dtype == TQ_F32 ? 4 : 2;
  const int cols_h = half_cols(L, a.d_in);
  const void *xh = static_cast<const uint8_t *>(a.x) + (paired ? 2048 * h * esize : 0);

  // Every wave of a block makes the same number of passes, so that the
  // block barriers of the paired layout line up (an idle pair computes on
  // row n and stores nothing).
  for (int64_t g0 = static_cast<int64_t>(blockIdx.x) * units; g0 < groups; g0 += stride) {
    const int64_t grp = g0 + unit;
    if (!paired && grp >= groups) break;
    const int64_t base_row = grp * vpw;
    const int64_t row = base_row + vslot;
    float xv[kEPL];
    RowSpan src{xh, a.ld_x, a.n, cols_h, a.dtype};
    if (a.vec_loads) {
      load_rows_staged(src, base_row, wlog, lane, stage, xv);
      if (a.d_in < a.d) {
#pragma unroll
        for (int e = 0; e < kEPL; ++e)
          if (sub * kEPL + e >= a.d_in) xv[e] = 0.0f;
      }
    } else {
      load_rows_direct(src, row, paired ? lane : sub, xv);
    }

    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
    for (int e = 0; e < kEPL; e += 4) {
      s0 = fmaf(xv[e], xv[e], s0);
      s1 = fmaf(xv[e + 1], xv[e + 1], s1);
      s2 = fmaf(xv[e + 2], xv[e + 2], s2);
      s3 = fmaf(xv[e + 3], xv[e + 3], s3);
    }
    float ss = group_sum((s0 + s1) + (s2 + s3), wlog);
#pragma unroll
    for (int e = 0; e < kEPL; ++e) xv[e] = __uint_as_float(__float_as_uint(xv[e]) ^ smask[e]);
    fwht_lane(xv);
    fwht_cross(xv, wlog, lane);
    if (paired) pair_stage(xv, ss, stage, partner, h, lane);
    // (a non-finite row is zeroed after the transform, which is linear)
    const bool bad = zero_if_nonfinite(xv, ss);
    const float nrm = sqrtf(ss);
    const float scale = ss > 0.0f ? sigma * inv_sqrt_d / nrm : 0.0f;
#pragma unroll
    for (int e = 0; e < kEPL; ++e) xv[e] *= scale;   // xv now holds y

    uint32_t words[M > 0 ? M : 1];
    float rr = 0.0f;
    if constexpr (M >= 1) {
      quantize_lane<M, PROD>(xv, tp, pc, tp_lds, cb_lds, words, rr);
      if (row < a.n) {
        uint32_t *dst = reinterpret_cast<uint32_t *>(a.codes + row * rec_bytes) + sub * M;
#pragma unroll
        for (int w = 0; w < M; ++w) dst[w] = words[w];
      }
    } else {
#pragma unroll
      for (int e = 0; e < kEPL; ++e) rr = fmaf(xv[e], xv[e], rr);
    }
    if (sub == 0 && row < a.n) a.norms[row] = bad ? __builtin_nanf("") : nrm;

    if constexpr (PROD) {
      float g2 = group_sum(rr, wlog);
      if (paired) {
        g2 = pair_sum(g2, stage, partner, lane);
        if (sub == 0 && row < a.n) a.rnorms[row] = sqrtf(g2);
        qjl_plane_pair(a, lane, h, row, lds + (wave & ~1) * wave_lds<PROD>(), xv);
      } else {
        if (sub == 0 && row < a.n) a.rnorms[row] = sqrtf(g2);
        qjl_plane(a, a.d, wlog, lane, base_row, stage, xv);
      }
    }
  }
}

// ------------------------------------------------------------ d = 128 kernel

// d = d_in = 128 (4 lanes per vector, 16 vectors per wave), element type DT
// known at compile time, rows 16-byte aligned with a stride that keeps them
// so.  Group g's 16 rows arrive as 2*esize 16-byte loads per lane (flat chunk
// f = 64 k + lane -> row f / CPR, chunk f % CPR); the next group's loads are
// issued before the current group is staged out of LDS and computed.
template <int M, bool PROD, int DT, int ROT>
__global__ void __launch_bounds__((PROD ? kWaves128P : kWaves) * 64) encode128_kernel(EncodeArgs a) {
  constexpr int NW = PROD ? kWaves128P : kWaves;
  constexpr int LOG_LPV = 2;
  constexpr int VPW = 16;
  constexpr int ES = (DT == TQ_F32) ? 4 : 2;
  constexpr int SEG = kEPL * ES + 16;        // LDS bytes per lane segment
  constexpr int NL = 2 * ES;                 // 16-byte loads per lane per group
  constexpr int CPR = 128 * ES / 16;         // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;              // rows per load instruction
  constexpr int SEG_CH = kEPL * ES / 16;     // chunks per lane segment
  // The float16 residual tiles of qjl_plane128 (2 x 16 x 136 x 2 bytes) fit
  // in the float32 staging region.
  __shared__ __attribute__((aligned(16))) uint8_t lds[NW * kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s16[PROD ? kS16Bytes : 16];
  __shared__ float tp_lds[128];
  __shared__ float cb_lds[256];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: the stage base is too
  const int sub = lane & 3;
  const int vslot = lane >> 2;
  uint8_t *stage = lds + wave * kStageBytes;

  PosThr<M> tp;
  PosCent<M> pc;
  load_consts<M, PROD>(a, tp, pc, tp_lds, cb_lds);
  if constexpr (PROD) load_s16<NW * 64>(a.qjl_s, s16);
  __syncthreads();

  // Lane sub transforms the coordinates of lane sub ^ 3.  The cross-lane
  // butterflies leave lane sub's outputs multiplied by (-1)^popcount(sub),
  // which is H[j][96] for every coordinate j of the lane; with P the
  // permutation j -> j ^ 96, H P = diag(H[j][96]) H, so feeding P D u gives
  // H D u itself.
  // Block rotations keep the lane's own coordinates and load their 32
  // parameters (pairs or quads of this lane's coordinates).
  constexpr bool kRht = ROT == TQ_ROT_RHT;
  const int src_sub = kRht ? (sub ^ 3) : sub;
  // 16-bit inputs with the RHT are never widened on their own: packed
  // element pair (x0, x1) = elements (2i, 2i+1) meets its signs (s0, s1) as
  // +-1.0 of the input type (psg) in the packed dot products of pair_stages,
  // which also make the first two butterfly stages; one more per pair gives
  // x0^2 + x1^2 for n^2.
  constexpr bool kPairSigns = kRht && ES == 2;
  uint32_t smask[kRht && !kPairSigns ? kEPL : 1];
  uint32_t psg[kPairSigns ? kEPL / 2 : 1];
  float rc[kRht ? 1 : kEPL];
  if constexpr (kPairSigns) {
    constexpr uint32_t kOne = DT == TQ_BF16 ? 0x3F80u : 0x3C00u;   // 1.0
#pragma unroll
    for (int i = 0; i < kEPL / 2; ++i)
      psg[i] = (kOne | (a.signs[src_sub * kEPL + 2 * i] < 0 ? 0x8000u : 0u)) |
               ((kOne | (a.signs[src_sub * kEPL + 2 * i + 1] < 0 ? 0x8000u : 0u)) << 16);
  } else if constexpr (kRht) {
#pragma unroll
    for (int e = 0; e < kEPL; ++e) smask[e] = a.signs[src_sub * kEPL + e] < 0 ? 0x80000000u : 0u;
  } else {
#pragma unroll
    for (int e = 0; e < kEPL; ++e) rc[e] = a.rot[sub * kEPL + e];
  }

  // This lane's chunk: row lane / CPR (+ RPI per load), column lane % CPR.
  const int lrow = lane / CPR;
  const int lcol = lane % CPR;
  const int lds_w = (lrow * 4 + lcol / SEG_CH) * SEG + (lcol % SEG_CH) * 16;   // + k * RPI * 4 * SEG
  const int64_t row_bytes = a.ld_x * ES;
  const int xoff = lrow * static_cast<int>(row_bytes) + lcol * 16;   // + k * RPI * row_bytes

  const float rsd = 0.08838834764831845f;     // 1 / sqrt(128)
  const float sqd = 11.313708498984761f;      // sqrt(128)
  // residuals are formed as r' = 2^14 r (see qjl_plane128)
  PosCent<M> pcs;
  if constexpr (PROD && M >= 1) {
#pragma unroll
    for (int k = 0; k < PosCent<M>::kCount; ++k) pcs.c[k] = pc.c[k] * 16384.0f;
  }
  const int64_t groups = (a.n + VPW - 1) / VPW;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * NW;
  constexpr size_t rec_bytes = static_cast<size_t>(M) * 16;

  // TurboQuant_mse loads the rows straight into the wave's LDS stage (no
  // registers held for the next group).  Load k fills a 1 KiB block at
  // kbase(k) in lane order; the chunk a lane fetches is chosen so that when
  // the lanes later read their own 32 coordinates, 16-byte chunk q of every
  // lane of a row pair sits in a different bank group: the slot of chunk q of
  // segment `seg` of a load's row `srow` is q ^ swz(srow, seg) (float32
  // blocks are 1152 bytes apart for the same reason across row pairs).
  constexpr bool kDirect = !PROD;
  auto kbase = [](int k) { return k * (ES == 4 ? 1152 : 1024); };
  auto swz = [](int srow, int seg) { return ES == 4 ? ((4 * (srow & 1) + seg) & 7) : ((srow + 2 * (seg >> 1)) & 3); };
  const int dl_sl = lane % CPR;
  const int dl_seg = dl_sl / SEG_CH;
  const int dl_col = dl_seg * SEG_CH + ((dl_sl % SEG_CH) ^ swz(lrow, dl_seg));
  const uint8_t *xd = static_cast<const uint8_t *>(a.x) + lrow * row_bytes + dl_col * 16;
  const int rd_seg = kRht ? (sub ^ 3) : sub;
  const int rd_k = vslot / RPI, rd_srow = vslot % RPI;
  const int rd_base = kbase(rd_k) + (CPR * rd_srow + SEG_CH * rd_seg) * 16 + (swz(rd_srow, rd_seg) << 4);

  // Packed chunk c (8 elements of a 16-bit type) into xv[8c .. 8c+7]: with
  // the RHT signed and through the first two butterfly stages, with the
  // squares added to sq; otherwise widened as they are.
  auto take16 = [&](const uint4 &w, int c, float (&xv)[kEPL], float (&sq)[4]) {
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
    if constexpr (kPairSigns) {
      pair_stages<DT>(wd, &psg[4 * c], &xv[8 * c]);
#pragma unroll
      for (int j = 0; j < 4; ++j) sq[j] = dot2<DT>(wd[j], wd[j], sq[j]);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (DT == TQ_BF16) {
          xv[8 * c + 2 * j] = bf16_lo(wd[j]); xv[8 * c + 2 * j + 1] = bf16_hi(wd[j]);
        } else {
          xv[8 * c + 2 * j] = f16_lo(wd[j]); xv[8 * c + 2 * j + 1] = f16_hi(wd[j]);
        }
      }
    }
  };
  uint4 buf[kDirect ? 1 : NL];
  auto issue = [&](int64_t g) {
    const int64_t base = g * VPW;
    if constexpr (kDirect) {
      const uint8_t *p = xd + base * row_bytes;
      if (base + VPW <= a.n) {
#pragma unroll
        for (int k = 0; k < NL; ++k) load_lds16_nt(p + k * RPI * row_bytes, stage + kbase(k));
      } else {
        // rows past n fetch row n - 1 instead; their results are never stored
#pragma unroll
        for (int k = 0; k < NL; ++k) {
          const int64_t r = base + lrow + k * RPI < a.n ? lrow + k * RPI : a.n - 1 - base;
          load_lds16_nt(xd + (base + r - lrow) * row_bytes, stage + kbase(k));
        }
      }
    } else {
      // the group's rows as one ranged buffer: rows past n read as zero (a
      // group past the end, g >= groups, is an empty buffer: its loads read
      // nothing from memory)
      const int64_t left = a.n - base;
      const int rows = left <= 0 ? 0 : left < VPW ? static_cast<int>(left) : VPW;
      const __amdgpu_buffer_rsrc_t xr = make_rsrc(static_cast<const uint8_t *>(a.x) + (rows > 0 ? base * row_bytes : 0),
                                                  rows * static_cast<int>(row_bytes));
#pragma unroll
      for (int k = 0; k < NL; ++k) buf[k] = load16_rsrc_nt(xr, xoff + k * RPI * static_cast<int>(row_bytes));
    }
  };

  // Staged (register) loads: group g's rows are written to the stage at the
  // end of the step before (so the wait for them sits behind that step's
  // stores, which may stay in flight), and the loads of the next group are
  // issued right after the stage has been read.
  auto stage_rows = [&]() {
#pragma unroll
    for (int k = 0; k < NL; ++k) *reinterpret_cast<uint4 *>(stage + lds_w + k * RPI * 4 * SEG) = buf[k];
  };
  int64_t grp = static_cast<int64_t>(blockIdx.x) * NW + wave;
  if (grp < groups) {
    issue(grp);
    if constexpr (!kDirect) stage_rows();
  }
  for (; grp < groups; grp += stride) {
    const int64_t base_row = grp * VPW;
    // this group's outputs as ranged buffers: rows past n are not written,
    // so every lane stores without a branch
    const int rows = a.n - base_row < VPW ? static_cast<int>(a.n - base_row) : VPW;
    float xv[kEPL];
    float sq[4] = {0.f, 0.f, 0.f, 0.f};      // squares of packed pairs (kPairSigns)
    if constexpr (kDirect) {
      // this group's rows have landed (the wait also covers the previous
      // group's stores); the stage is read, then refilled with the next group
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
      for (int q = 0; q < SEG_CH; q += 2) {
        const uint4 w[2] = {*reinterpret_cast<const uint4 *>(stage + (rd_base ^ (q << 4))),
                            *reinterpret_cast<const uint4 *>(stage + (rd_base ^ ((q + 1) << 4)))};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if constexpr (DT == TQ_F32) {
            xv[4 * (q + h) + 0] = __uint_as_float(w[h].x);
            xv[4 * (q + h) + 1] = __uint_as_float(w[h].y);
            xv[4 * (q + h) + 2] = __uint_as_float(w[h].z);
            xv[4 * (q + h) + 3] = __uint_as_float(w[h].w);
          } else {
            take16(w[h], q + h, xv, sq);
          }
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (grp + stride < groups) issue(grp + stride);
    } else {
    wave_lds_sync();
    const uint4 *src = reinterpret_cast<const uint4 *>(stage + (kRht ? (lane ^ 3) : lane) * SEG);
    if constexpr (DT == TQ_F32) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint4 w = src[q];
        xv[4 * q + 0] = __uint_as_float(w.x);
        xv[4 * q + 1] = __uint_as_float(w.y);
        xv[4 * q + 2] = __uint_as_float(w.z);
        xv[4 * q + 3] = __uint_as_float(w.w);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) take16(src[q], q, xv, sq);
    }
    wave_lds_sync();
    issue(grp + stride);   // past the last group: an empty buffer, no memory traffic
    }

    if constexpr (!kPairSigns) {
#pragma unroll
      for (int e = 0; e < kEPL; e += 4) {
        sq[0] = fmaf(xv[e], xv[e], sq[0]);
        sq[1] = fmaf(xv[e + 1], xv[e + 1], sq[1]);
        sq[2] = fmaf(xv[e + 2], xv[e + 2], sq[2]);
        sq[3] = fmaf(xv[e + 3], xv[e + 3], sq[3]);
      }
    }
    float ss = (sq[0] + sq[1]) + (sq[2] + sq[3]);
    ss += xor_partner<0>(ss);
    ss += xor_partner<1>(ss);
    const bool bad = zero_if_nonfinite(xv, ss);
    if constexpr (kRht) {
      if constexpr (!kPairSigns) {
#pragma unroll
        for (int e = 0; e < kEPL; ++e) xv[e] = __uint_as_float(__float_as_uint(xv[e]) ^ smask[e]);
      }
      fwht_lane<kPairSigns ? 4 : 1>(xv);     // take16 made the first two stages
      cross_stage<0>(xv, (lane & 1) ? -1.0f : 1.0f);
      cross_stage<1>(xv, (lane & 2) ? -1.0f : 1.0f);
    } else {
      rotate_blocks<ROT, false>(xv, rc);
    }
    // 1/n from the hardware reciprocal square root (about 1 ulp); n = ss/n.
    // y = h / (n sqrt d) (RHT; h / n for a block rotation); instead of
    // scaling the 32 coordinates, the thresholds move to h's scale.  A zero
    // row (y = 0) gets infinite thresholds: level 0 on the positive side, as
    // for y = 0.
    const float rn = __builtin_amdgcn_rsqf(ss);
    const float nrm = ss > 0.0f ? ss * rn : 0.0f;
    const float tscale = ss > 0.0f ? (kRht ? nrm * sqd : nrm) : __builtin_inff();
    const float r14 = ss > 0.0f ? 16384.0f * (kRht ? rsd : 1.0f) * rn : 0.0f;     // h -> 2^14 y
    PosThr<M> ts;
#pragma unroll
    for (int k = 0; k < PosThr<M>::kCount; ++k) ts.t[k] = tp.t[k] * tscale;

    uint32_t words[M > 0 ? M : 1];
    float rr = 0.0f;
    if constexpr (M >= 1) {
      quantize_lane<M, PROD, true>(xv, ts, pcs, tp_lds, cb_lds, words, rr, r14);
      store_words_rsrc<M>(words, make_rsrc(a.codes + base_row * rec_bytes, rows * static_cast<int>(rec_bytes)),
                          static_cast<int>(vslot * rec_bytes) + 4 * M * sub);
    } else {
#pragma unroll
      for (int e = 0; e < kEPL; ++e) {
        xv[e] *= r14;
        rr = fmaf(xv[e], xv[e], rr);
      }
    }
    // the four lanes of a row hold the same norms and all store them
    const uint32_t nw[1] = {__float_as_uint(bad ? __builtin_nanf("") : nrm)};
    store_words_rsrc<1>(nw, make_rsrc(a.norms + base_row, rows * 4), 4 * vslot);
    if constexpr (PROD) {
      float g2 = rr;
      g2 += xor_partner<0>(g2);
      g2 += xor_partner<1>(g2);
      const uint32_t gw[1] = {__float_as_uint(sqrtf(g2) * 6.103515625e-05f)};   // 2^-14
      store_words_rsrc<1>(gw, make_rsrc(a.rnorms + base_row, rows * 4), 4 * vslot);
      qjl_plane128(lane, make_rsrc(a.qjl + base_row * 16, rows * 16), stage, s16, xv);
    }
    if constexpr (!kDirect) stage_rows();
  }
}

// ------------------------------------------------------------ d = 128 TurboQuant_prod, 16-bit rows

// The Walsh-Hadamard transform of 16-bit rows on the matrix cores.  Sylvester
// H_128 factors over the bits of the coordinate index: writing
// j = 32 g + 8 c + 4 h + i (g, c two bits; h one; i two),
//   H_128[j][j'] = H_4[c][c'] * (-1)^(popcount(g & g') + popcount((4h + i) & t'))
// for j' = 32 g' + 8 c' + t'.  For each chunk c' (the 32 inputs whose index
// bits 3..4 equal c') one v_mfma_f32_16x16x32 (bf16 or f16 inputs, exact
// +-1 products, float32 sums) forms the inner 32-point transform of 16 rows
// with the RHT signs folded into its constant operand, and two butterfly
// stages inside the lane then apply H_4 across the four chunks.  In MFMA
// terms lane (g, k) (g = lane / 16, k = lane % 16) supplies row k's inputs
// 32 g + 8 c' .. + 7 for chunk c' and receives row k's outputs
// 32 g + 8 c + 4 h + i -- it ends up owning coordinates 32 g .. 32 g + 31
// of row k, whose codes are whole words of the record.  The residual then
// stays in the lane as the B operand of S r (no LDS transpose), and the
// lane's S r outputs are the bits 32 g .. 32 g + 31 of row k's QJL plane.

constexpr int kWavesH = 8;
constexpr int kStageH = 16 * 256;    // one group: 16 rows of 128 16-bit elements

template <int DT>
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (DT == TQ_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                  0, 0, 0);
  }
}

// Bits of word w (of the lane's 32 M-bit codes) that hold the top bit of a
// code: stream positions M e + M - 1.
template <int M>
constexpr uint32_t top_bits(int w) {
  uint32_t m = 0;
  for (int b = 0; b < 32; ++b)
    if ((32 * w + b) % M == M - 1) m |= 1u << b;
  return m;
}

// The words are built with [h < 0] at each code's top bit and the level
// bits L below it uncorrected; the code is (1, L) for h >= 0 and
// (0, ~L) for h < 0: xor each level bit with its code's top bit, then
// invert the top bits.
template <int M>
__device__ __forceinline__ void fix_codes(uint32_t (&w)[M > 0 ? M : 1]) {
  if constexpr (M == 1) {
    w[0] = ~w[0];
  } else if constexpr (M == 2) {
#pragma unroll
    for (int i = 0; i < 2; ++i) w[i] ^= ((w[i] >> 1) & 0x55555555u) | 0xAAAAAAAAu;
  } else if constexpr (M >= 3) {
    uint32_t top[M];
#pragma unroll
    for (int i = 0; i < M; ++i) top[i] = w[i] & top_bits<M>(i);
#pragma unroll
    for (int k = 1; k < M; ++k)
#pragma unroll
      for (int i = 0; i < M; ++i) w[i] ^= __builtin_amdgcn_alignbit(i + 1 < M ? top[i + 1] : 0u, top[i], k);
#pragma unroll
    for (int i = 0; i < M; ++i) w[i] ^= top_bits<M>(i);
  }
}

// Codes of the lane's 32 coordinates h (unnormalised: y = h / s, s > 0,
// with ts the positive thresholds times s), appended into the M words of the
// lane's part of the record, and the residuals r' = h r14 - c' (c' the
// centroids times 2^14, r14 = 2^14 / s) in place of h with their squares
// summed into rr.  A code's top bit is h's float sign bit (one v_alignbit,
// no compare); fix_codes turns the raw words into codes.  h is never -0 here
// (sums of products started from +0), so the sign bit is [h < 0].
template <int M>
__device__ __forceinline__ void quantize_h(float (&xv)[kEPL], const PosThr<M> &ts, const PosCent<M> &pcs, float r14,
                                           uint32_t (&words)[M > 0 ? M : 1], float &rr) {
#pragma unroll
  for (int w = 0; w < (M > 0 ? M : 1); ++w) words[w] = 0u;
  rr = 0.0f;
#pragma unroll
  for (int e = kEPL - 1; e >= 0; --e) {
    float h = xv[e];
    // keep at most four elements' compare masks live (see quantize_lane)
    if ((e & 3) == 3 && e != kEPL - 1) asm volatile("" : "+v"(h) : "v"(rr));
    const float a = fabsf(h);
    float mag;
    if constexpr (M == 1) {
      words[e >> 5] = __builtin_amdgcn_alignbit(words[e >> 5], __float_as_uint(h), 31);
      mag = pcs.c[0];
    } else if constexpr (M == 2) {
      words[(2 * e + 1) >> 5] = __builtin_amdgcn_alignbit(words[(2 * e + 1) >> 5], __float_as_uint(h), 31);
      const bool l0 = a >= ts.t[0];
      words[(2 * e) >> 5] = append_mask(words[(2 * e) >> 5], __builtin_amdgcn_ballot_w64(l0));
      mag = l0 ? pcs.c[1] : pcs.c[0];
    } else {
      static_assert(M == 3, "1..3 code bits");
      words[(3 * e + 2) >> 5] = __builtin_amdgcn_alignbit(words[(3 * e + 2) >> 5], __float_as_uint(h), 31);
      const bool l1 = a >= ts.t[1];
      const float t = l1 ? ts.t[2] : ts.t[0];
      const bool l0 = a >= t;
      words[(3 * e + 1) >> 5] = append_mask(words[(3 * e + 1) >> 5], __builtin_amdgcn_ballot_w64(l1));
      words[(3 * e) >> 5] = append_mask(words[(3 * e) >> 5], __builtin_amdgcn_ballot_w64(l0));
      mag = l1 ? (l0 ? pcs.c[3] : pcs.c[2]) : (l0 ? pcs.c[1] : pcs.c[0]);
    }
    // the centroid has h's sign, so r' = sign(h) (|h| r14 - |c'|): one FMA
    // with operand modifiers, then h's sign bit xor-ed in (v_bitop3)
    const float ra = fmaf(a, r14, -mag);
    xv[e] = __uint_as_float(__float_as_uint(ra) ^ (__float_as_uint(h) & 0x80000000u));
    rr = fmaf(ra, ra, rr);
  }
  fix_codes<M>(words);
}

// d = d_in = 128, 16-bit rows (DT = TQ_BF16 or TQ_F16), RHT, TurboQuant_prod
// with M = 0..3 code bits, rows 16-byte aligned with a stride that keeps them
// so.  One wave encodes 16 rows (a group) at a time.  A group's rows come
// straight from HBM into the wave's LDS stage, four whole rows per load; the
// next group's loads are issued as soon as the stage has been read.
template <int M, int DT>
__global__ void __launch_bounds__(kWavesH * 64) encode128h_kernel(EncodeArgs a) {
  static_assert(DT == TQ_BF16 || DT == TQ_F16, "16-bit rows");
  __shared__ __attribute__((aligned(16))) uint8_t lds[kWavesH * kStageH];
  __shared__ __attribute__((aligned(16))) uint8_t s16[kS16Bytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int key = lane & 15;
  uint8_t *stage = lds + wave * kStageH;

  PosThr<M> tp;
  PosCent<M> pc;
  load_consts<M, true>(a, tp, pc, nullptr, nullptr);
  load_s16<kWavesH * 64, true>(a.qjl_s, s16);

  // Constant operand of the transform for chunk c' and output half h: as an
  // A-operand lane, (g, key) holds row key = 4 g_out + i (output coordinate
  // 32 g_out + 8 c + 4 h + i) and K block g (inputs 32 g + 8 c' + t, t < 8).
  constexpr uint32_t kOne = DT == TQ_BF16 ? 0x3F80u : 0x3C00u;
  u32x4 ha[4][2];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t v[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        uint32_t pair = 0;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int t = 2 * p + q;
          const int par = __builtin_popcount((key >> 2) & g) + __builtin_popcount((4 * h + (key & 3)) & t) +
                          (a.signs[32 * g + 8 * c + t] < 0 ? 1 : 0);
          pair |= (kOne | ((par & 1) ? 0x8000u : 0u)) << (16 * q);
        }
        v[p] = pair;
      }
      ha[c][h] = u32x4{v[0], v[1], v[2], v[3]};
    }
  }
  PosCent<M> pcs;                       // centroids times 2^14 (r' = 2^14 r)
#pragma unroll
  for (int k = 0; k < PosCent<M>::kCount; ++k) pcs.c[k] = pc.c[k] * 16384.0f;
  __syncthreads();

  // Stage layout: 16-byte slot s of the stage holds chunk (row s / 16,
  // column ((s % 16) - s / 16) % 16) of the group, so load kk (slots
  // 64 kk + lane) reads rows 4 kk .. 4 kk + 3 whole, and the reads of chunk
  // (row key, column 4 g + q) by 16 lanes fall in 16 distinct bank groups.
  const int64_t row_bytes = a.ld_x * 2;
  const uint8_t *xb = static_cast<const uint8_t *>(a.x);
  int loff[4];                          // lane's byte offset in the group, load kk
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int r = 4 * kk + (lane >> 4);
    loff[kk] = r * static_cast<int>(row_bytes) + (((lane & 15) - r) & 15) * 16;
  }
  auto issue = [&](int64_t grp) {
    const int64_t base = grp * 16;
    const uint8_t *gb = xb + base * row_bytes;     // wave-uniform
    if (base + 16 <= a.n) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) load_lds16_nt(gb + loff[kk], stage + kk * 1024);
    } else {
      // rows past n fetch row n - 1 instead; their results are never stored
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int r = 4 * kk + (lane >> 4);
        const int64_t row = base + r < a.n ? base + r : a.n - 1;
        load_lds16_nt(xb + row * row_bytes + (((lane & 15) - r) & 15) * 16, stage + kk * 1024);
      }
    }
  };
  int rd[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) rd[q] = (16 * key + ((4 * g + q + key) & 15)) * 16;

  const float rsd = 0.08838834764831845f;     // 1 / sqrt(128)
  const float sqd = 11.313708498984761f;      // sqrt(128)
  constexpr int kRec = M * 16;                // record bytes
  const int64_t groups = (a.n + 15) / 16;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kWavesH;
  int64_t grp = static_cast<int64_t>(blockIdx.x) * kWavesH + wave;
  if (grp < groups) issue(grp);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  for (; grp < groups; grp += stride) {
    const int64_t base_row = grp * 16;
    const int rows = a.n - base_row < 16 ? static_cast<int>(a.n - base_row) : 16;
    u32x4 w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = *reinterpret_cast<const u32x4 *>(stage + rd[q]);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (grp + stride < groups) issue(grp + stride);

    // n^2 from packed dot products of the element pairs
    float sq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      sq[0] = dot2<DT>(w[q].x, w[q].x, sq[0]);
      sq[1] = dot2<DT>(w[q].y, w[q].y, sq[1]);
      sq[2] = dot2<DT>(w[q].z, w[q].z, sq[2]);
      sq[3] = dot2<DT>(w[q].w, w[q].w, sq[3]);
    }
    float ss = (sq[0] + sq[1]) + (sq[2] + sq[3]);
    ss += xor_partner<4>(ss);
    ss += xor_partner<5>(ss);
    // a row with a NaN or an infinity: encoded as the zero row, norm NaN
    const bool bad = !(ss <= 3.402823466e38f);
    if (__builtin_amdgcn_ballot_w64(bad) != 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) w[q] = bad ? u32x4{0u, 0u, 0u, 0u} : w[q];
      ss = bad ? 0.0f : ss;
    }

    // h = H D x: one MFMA per (chunk, output half), then H_4 across chunks
    f32x4 acc[4][2];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int h = 0; h < 2; ++h) acc[c][h] = mfma16x16x32<DT>(ha[c][h], w[c], f32x4{0.f, 0.f, 0.f, 0.f});
    float xv[kEPL];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float t0 = acc[0][h][i] + acc[1][h][i], t1 = acc[0][h][i] - acc[1][h][i];
        const float t2 = acc[2][h][i] + acc[3][h][i], t3 = acc[2][h][i] - acc[3][h][i];
        xv[4 * h + i] = t0 + t2;           // c = 0
        xv[8 + 4 * h + i] = t1 + t3;       // c = 1
        xv[16 + 4 * h + i] = t0 - t2;      // c = 2
        xv[24 + 4 * h + i] = t1 - t3;      // c = 3
      }
    }

    // y = h / (n sqrt d): thresholds move to h's scale instead; a zero row
    // gets infinite thresholds (level 0 on the positive side, as y = 0)
    const float rn = __builtin_amdgcn_rsqf(ss);
    const float nrm = ss > 0.0f ? ss * rn : 0.0f;
    const float tscale = ss > 0.0f ? nrm * sqd : __builtin_inff();
    const float r14 = ss > 0.0f ? 16384.0f * rsd * rn : 0.0f;     // h -> 2^14 y
    PosThr<M> ts;
#pragma unroll
    for (int k = 0; k < PosThr<M>::kCount; ++k) ts.t[k] = tp.t[k] * tscale;

    uint32_t words[M > 0 ? M : 1];
    float rr = 0.0f;
    if constexpr (M >= 1) {
      quantize_h<M>(xv, ts, pcs, r14, words, rr);
      store_words_rsrc<M>(words, make_rsrc(a.codes + base_row * kRec, rows * kRec), key * kRec + 4 * M * g);
    } else {
#pragma unroll
      for (int e = 0; e < kEPL; ++e) {
        xv[e] *= r14;
        rr = fmaf(xv[e], xv[e], rr);
      }
    }
    const uint32_t nw[1] = {__float_as_uint(bad ? __builtin_nanf("") : nrm)};
    store_words_rsrc<1>(nw, make_rsrc(a.norms + base_row, rows * 4), 4 * key);
    float g2 = rr;
    g2 += xor_partner<4>(g2);
    g2 += xor_partner<5>(g2);
    const uint32_t gw[1] = {__float_as_uint(sqrtf(g2) * 6.103515625e-05f)};   // 2^-14
    store_words_rsrc<1>(gw, make_rsrc(a.rnorms + base_row, rows * 4), 4 * key);

    // S r' on r' = hi + lo (float16, hi = r' rounded toward zero)
    uint32_t hw[16], lw[16];
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const float r0 = xv[2 * p], r1 = xv[2 * p + 1];
      const auto hp = __builtin_amdgcn_cvt_pkrtz(r0, r1);
      __builtin_memcpy(&hw[p], &hp, 4);
      const auto lp = __builtin_amdgcn_cvt_pkrtz(sub_f16_half<0>(r0, hw[p]), sub_f16_half<1>(r1, hw[p]));
      __builtin_memcpy(&lw[p], &lp, 4);
    }
    // output o = 32 g + 4 nt + i lands in this lane as bit 4 nt + i of word g
    // of row key's plane; the sign bits are shifted in from the top
    uint32_t qn = 0u;
    const int orow = 32 * (key >> 2) + (key & 3);     // + 4 nt: the S row this lane reads as A operand
#pragma unroll
    for (int nt = 7; nt >= 0; --nt) {
      f32x4 sr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const u32x4 sa = *reinterpret_cast<const u32x4 *>(s16 + s16h_offset(orow + 4 * nt, 4 * g + kc));
        sr = mfma16x16x32<TQ_F16>(sa, u32x4{hw[4 * kc], hw[4 * kc + 1], hw[4 * kc + 2], hw[4 * kc + 3]}, sr);
        sr = mfma16x16x32<TQ_F16>(sa, u32x4{lw[4 * kc], lw[4 * kc + 1], lw[4 * kc + 2], lw[4 * kc + 3]}, sr);
      }
#pragma unroll
      for (int i = 3; i >= 0; --i) qn = __builtin_amdgcn_alignbit(qn, __float_as_uint(sr[i]), 31);
    }
    const uint32_t qw[1] = {~qn};
    store_words_rsrc<1>(qw, make_rsrc(a.qjl + base_row * 16, rows * 16), key * 16 + 4 * g);
    // the next group's rows have landed once at most this group's stores are
    // still in flight (loads and stores complete in issue order)
    if constexpr (M >= 1) {
      asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
    }
  }
}

dim3 grid_for(int64_t n, int vpw, int64_t max_blocks = 256 * 8, int waves = kWaves) {
  const int64_t groups = (n + vpw - 1) / vpw;
  const int64_t blocks_needed = (groups + waves - 1) / waves;
  return dim3(static_cast<unsigned>(blocks_needed < max_blocks ? blocks_needed : max_blocks));
}

template <int M, bool PROD, int ROT>
void launch_128(const EncodeArgs &a, hipStream_t s) {
  // Measured sweeps (1M bf16 prod keys, 4M float32 mse rows): TurboQuant_prod
  // is fastest persistent, one 12-wave workgroup per CU; TurboQuant_mse with
  // about 128 workgroups per CU queued, i.e. each wave taking two groups
  // (about 6 % ahead of 16 per CU)
  constexpr int nw = PROD ? kWaves128P : kWaves;
  const dim3 grid = grid_for(a.n, 16, PROD ? 256 : 256 * 128, nw);
  if (a.dtype == TQ_F32) hipLaunchKernelGGL((encode128_kernel<M, PROD, TQ_F32, ROT>), grid, dim3(nw * 64), 0, s, a);
  else if (a.dtype == TQ_BF16) hipLaunchKernelGGL((encode128_kernel<M, PROD, TQ_BF16, ROT>), grid, dim3(nw * 64), 0, s, a);
  else hipLaunchKernelGGL((encode128_kernel<M, PROD, TQ_F16, ROT>), grid, dim3(nw * 64), 0, s, a);
}

// Workgroups of the general kernel: one vector per pair of waves at d = 4096.
dim3 grid_general(const EncodeArgs &a) {
  if (a.log_lpv == kPairLogLpv) {
    const int64_t blocks = (a.n + kWaves / 2 - 1) / (kWaves / 2);
    return dim3(static_cast<unsigned>(blocks < 2048 ? blocks : 2048));
  }
  return grid_for(a.n, 64 >> a.log_lpv);
}

template <int M>
void launch_128h(const EncodeArgs &a, hipStream_t s) {
  const dim3 grid = grid_for(a.n, 16, 256 * 2, kWavesH);
  if (a.dtype == TQ_BF16) hipLaunchKernelGGL((encode128h_kernel<M, TQ_BF16>), grid, dim3(kWavesH * 64), 0, s, a);
  else hipLaunchKernelGGL((encode128h_kernel<M, TQ_F16>), grid, dim3(kWavesH * 64), 0, s, a);
}

template <int M, bool PROD>
void launch_one(const EncodeArgs &a, hipStream_t s, bool fast) {
  if constexpr (PROD && M <= 3) {
    // 16-bit rows with the RHT: the transform on the matrix cores
    if (fast && a.rot_kind == TQ_ROT_RHT && a.dtype != TQ_F32) {
      launch_128h<M>(a, s);
      return;
    }
  }
  if (a.rot_kind == TQ_ROT_GIVENS) {
    launch_128<M, PROD, TQ_ROT_GIVENS>(a, s);
  } else if (a.rot_kind == TQ_ROT_QUAT) {
    launch_128<M, PROD, TQ_ROT_QUAT>(a, s);
  } else if (fast) {
    launch_128<M, PROD, TQ_ROT_RHT>(a, s);
  } else {
    hipLaunchKernelGGL((encode_kernel<M, PROD>), grid_general(a), dim3(kThreads), 0, s, a);
  }
}

template <int M, bool PROD>
void launch_general(const EncodeArgs &a, hipStream_t s) {
  hipLaunchKernelGGL((encode_kernel<M, PROD>), grid_general(a), dim3(kThreads), 0, s, a);
}

}  // namespace

int launch_encode(const EncodeArgs &a, bool prod, void *stream) {
  (void)hipGetLastError();   // report only errors of this launch
  hipStream_t s = static_cast<hipStream_t>(stream);
  // (the d = 128 kernel addresses a group of 16 rows with 32-bit offsets)
  const bool fast = a.d == 128 && a.d_in == 128 && a.vec_loads && a.ld_x <= (1 << 24);
  if (prod) {
    switch (a.m) {
      case 0: launch_one<0, true>(a, s, fast); break;
      case 1: launch_one<1, true>(a, s, fast); break;
      case 2: launch_one<2, true>(a, s, fast); break;
      case 3: launch_one<3, true>(a, s, fast); break;
      case 4: launch_general<4, true>(a, s); break;
      case 5: launch_general<5, true>(a, s); break;
      case 6: launch_general<6, true>(a, s); break;
      case 7: launch_general<7, true>(a, s); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (a.m) {
      case 1: launch_one<1, false>(a, s, fast); break;
      case 2: launch_one<2, false>(a, s, fast); break;
      case 3: launch_one<3, false>(a, s, fast); break;
      case 4: launch_one<4, false>(a, s, fast); break;
      case 5: launch_general<5, false>(a, s); break;
      case 6: launch_general<6, false>(a, s); break;
      case 7: launch_general<7, false>(a, s); break;
      case 8: launch_general<8, false>(a, s); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

}  // namespace tq
