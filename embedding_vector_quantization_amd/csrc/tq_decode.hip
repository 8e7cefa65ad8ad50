// Dequantiser Q^-1 and the bare rotation for gfx950.
//
// Sources: "TurboQuant: Online Vector Quantization" paper summary (Jump2Paper
// Archive) -- Q^-1 of the definitions table (centroid lookup, inverse
// rotation) and the QJL dequantiser sqrt(pi/2)/d * S^T z of Definition 1 /
// Lemma 4, used on the residual in Theorem D_prod; AI Trends video summary
// chapter 06:06 (the rotation is orthogonal, so its transpose undoes it, and
// the stored norm restores the scale).
//
// Same register layout as the encoder: LPV = d/32 lanes per vector, 32
// contiguous coordinates per lane.  Decode reads the lane's m dwords of the
// record, looks up centroids in LDS, adds the QJL term for TurboQuant_prod,
// runs the Walsh-Hadamard transform (H is symmetric, so Pi^T = D H / sqrt d)
// and writes n * D (H y~) / sqrt d through a wave-private LDS stage so that
// global stores are coalesced.

#include <hip/hip_runtime.h>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kStageBytes = 64 * (kEPL * 4 + 16);
// d = 128 prod: S^T in LDS with rows padded to 136 bf16 (272 bytes, so the
// 16-byte fragment reads of 8 consecutive rows hit distinct banks).
constexpr int kStRow = 128 + 8;
constexpr int kStBytes = 128 * kStRow * 2;
constexpr int kCRow = 128 + 4;                // float32 MFMA output tile row

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Eight QJL bits (bit t of `byte`) as bfloat16 +1 / -1 values, bit t in
// element t.
__device__ __forceinline__ bf16x8 signs_bf16x8(uint32_t byte) {
  uint32_t w[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t lo = ((~byte >> (2 * p)) & 1u) << 15;
    const uint32_t hi = ((~byte >> (2 * p + 1)) & 1u) << 31;
    w[p] = 0x3F803F80u | lo | hi;
  }
  bf16x8 r;
  __builtin_memcpy(&r, w, sizeof(r));
  return r;
}

// Bits [M e, M e + M) of the lane's M-word segment.
template <int M>
__device__ __forceinline__ int code_at(const uint32_t (&w)[M > 0 ? M : 1], int e) {
  const int s = M * e;
  const int wi = s >> 5, off = s & 31;
  uint32_t v = w[wi] >> off;
  if (off + M > 32) v |= w[wi + 1] << (32 - off);
  return static_cast<int>(v & ((1u << M) - 1u));
}

template <int M, bool PROD>
__global__ void __launch_bounds__(kThreads) decode_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kWaves * kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t st_lds[PROD ? kStBytes : 16];
  __shared__ float cb_lds[256];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // d = 4096: a vector over a pair of waves (the last butterfly stage
  // through LDS); the loop is then the same for every wave of the block
  const Layout L = layout_of(a.log_lpv, kWaves, wave, lane);
  const int sub = L.sub, vslot = L.vslot, vpw = L.vpw;
  uint8_t *stage = lds + wave * kStageBytes;
  uint8_t *partner = lds + (wave ^ 1) * kStageBytes;
  if constexpr (M >= 1) {
    for (int k = threadIdx.x; k < (1 << M); k += kThreads) cb_lds[k] = a.centroids[k];
  }
  const bool mfma_qjl = PROD && a.d == 128;
  if (mfma_qjl) {
    // S^T into LDS: st[j][i] = S[i][j].
    uint16_t *st = reinterpret_cast<uint16_t *>(st_lds);
    for (int idx = threadIdx.x; idx < 128 * 128; idx += kThreads)
      st[(idx & 127) * kStRow + (idx >> 7)] = a.qjl_s[idx];
  }
  __syncthreads();

  uint32_t smask[kEPL];
#pragma unroll
  for (int e = 0; e < kEPL; ++e) smask[e] = a.signs[sub * kEPL + e] < 0 ? 0x80000000u : 0u;
  const float inv_sqrt_d = 1.0f / sqrtf(static_cast<float>(a.d));
  const float sigma = cross_sign(sub & 63);
  const float qjl_scale = 1.2533141373155003f / static_cast<float>(a.d);   // sqrt(pi/2) / d
  const int64_t groups = (a.n + vpw - 1) / vpw;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * L.units;
  const size_t rec_bytes = static_cast<size_t>(M) * a.d / 8;
  const bool staged_out = ((a.d_in & 3) == 0) && ((a.ld_out & 3) == 0) &&
                          ((reinterpret_cast<uintptr_t>(a.out) & 15) == 0);
  // this wave's columns of the output rows
  const int cols_h = half_cols(L, a.d_in);
  float *out_h = a.out + 2048 * L.h;

  // The next group's record (codes, QJL bytes of the MFMA rows, norms) is
  // loaded into registers while the current group is computed.
  constexpr int MW = M > 0 ? M : 1;
  uint32_t cw[MW], nw[MW], cz[4], nz[4];
  float cn = 0.0f, cg = 0.0f, nn = 0.0f, ng = 0.0f;
  auto fetch = [&](int64_t g, uint32_t (&w)[MW], uint32_t (&z)[4], float &nr, float &gm) {
    const int64_t rw = g * vpw + vslot;
    const bool lv = rw < a.n;
    if constexpr (M >= 1) {
#pragma unroll
      for (int k = 0; k < M; ++k)
        w[k] = lv ? reinterpret_cast<const uint32_t *>(a.codes + rw * rec_bytes)[sub * M + k] : 0u;
    }
    if constexpr (PROD) {
      const int64_t zrow = g * vpw + (lane & 15);
      const bool zl = mfma_qjl && zrow < a.n;
#pragma unroll
      for (int k = 0; k < 4; ++k) z[k] = zl ? reinterpret_cast<const uint32_t *>(a.qjl + zrow * 16)[k] : 0u;
      gm = lv ? a.rnorms[rw] : 0.0f;
    }
    nr = lv ? a.norms[rw] : 0.0f;
  };
  // (paired: a unit past the end fetches zeros and stores nothing)
  int64_t g0 = static_cast<int64_t>(blockIdx.x) * L.units;
  if (g0 + L.unit < groups || L.paired) fetch(g0 + L.unit, cw, cz, cn, cg);
  for (; g0 < groups; g0 += stride) {
    const int64_t grp = g0 + L.unit;
    if (!L.paired && grp >= groups) break;
    if (grp + stride < groups || L.paired) fetch(grp + stride, nw, nz, nn, ng);
    const int64_t base_row = grp * vpw;
    const int64_t row = base_row + vslot;
    const bool live = row < a.n;
    float yv[kEPL];
    if constexpr (M >= 1) {
#pragma unroll
      for (int e = 0; e < kEPL; ++e) yv[e] = cb_lds[code_at<M>(cw, e)];
    } else {
#pragma unroll
      for (int e = 0; e < kEPL; ++e) yv[e] = 0.0f;
    }
    if constexpr (PROD) {
     if (mfma_qjl) {
      // T = Z S for the wave's 16 vectors with v_mfma_f32_16x16x32_bf16:
      // A[v][i] = z_v[i] (+-1, exact in bf16), B[i][j] = S[i][j] read from
      // the S^T rows in LDS; 8 column tiles x 4 k-chunks, one exact pass.
      // The output tile goes through LDS back to the lane layout.
      const int fr = lane & 15, g = lane >> 4;
      bf16x8 af[4];
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) af[kc] = signs_bf16x8((cz[kc] >> (8 * g)) & 0xFFu);
      float *ct = reinterpret_cast<float *>(stage);        // [16][kCRow]
      const uint16_t *st = reinterpret_cast<const uint16_t *>(st_lds);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          const bf16x8 b = *reinterpret_cast<const bf16x8 *>(st + (16 * nt + fr) * kStRow + 32 * kc + 8 * g);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[kc], b, acc, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) ct[(4 * g + i) * kCRow + 16 * nt + fr] = acc[i];
      }
      wave_lds_sync();
      const float gam = cg * qjl_scale;
      const float4 *tv = reinterpret_cast<const float4 *>(ct + vslot * kCRow + sub * kEPL);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float4 t4 = tv[q];
        yv[4 * q + 0] = fmaf(gam, t4.x, yv[4 * q + 0]);
        yv[4 * q + 1] = fmaf(gam, t4.y, yv[4 * q + 1]);
        yv[4 * q + 2] = fmaf(gam, t4.z, yv[4 * q + 2]);
        yv[4 * q + 3] = fmaf(gam, t4.w, yv[4 * q + 3]);
      }
      wave_lds_sync();
     } else {
      // y~_j += gamma * sqrt(pi/2)/d * sum_i z_i S[i][j] over this lane's 32
      // coordinates j; z = +-1 from the QJL plane.
      const float gam = cg * qjl_scale;
      const uint32_t *zq = reinterpret_cast<const uint32_t *>(a.qjl + (live ? row : 0) * (a.d / 8));
      float acc[kEPL];
#pragma unroll
      for (int e = 0; e < kEPL; ++e) acc[e] = 0.0f;
      for (int iw = 0; iw < (a.d >> 5); ++iw) {
        const uint32_t zw = live ? zq[iw] : 0u;
        for (int ib = 0; ib < 32; ++ib) {
          const int i = iw * 32 + ib;
          const float z = ((zw >> ib) & 1u) ? 1.0f : -1.0f;
          const uint4 *srow = reinterpret_cast<const uint4 *>(a.qjl_s + static_cast<int64_t>(i) * a.d + sub * kEPL);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint4 sv = srow[q];
            acc[8 * q + 0] = fmaf(z, bf16_lo(sv.x), acc[8 * q + 0]);
            acc[8 * q + 1] = fmaf(z, bf16_hi(sv.x), acc[8 * q + 1]);
            acc[8 * q + 2] = fmaf(z, bf16_lo(sv.y), acc[8 * q + 2]);
            acc[8 * q + 3] = fmaf(z, bf16_hi(sv.y), acc[8 * q + 3]);
            acc[8 * q + 4] = fmaf(z, bf16_lo(sv.z), acc[8 * q + 4]);
            acc[8 * q + 5] = fmaf(z, bf16_hi(sv.z), acc[8 * q + 5]);
            acc[8 * q + 6] = fmaf(z, bf16_lo(sv.w), acc[8 * q + 6]);
            acc[8 * q + 7] = fmaf(z, bf16_hi(sv.w), acc[8 * q + 7]);
          }
        }
      }
#pragma unroll
      for (int e = 0; e < kEPL; ++e) yv[e] = fmaf(gam, acc[e], yv[e]);
     }
    }
    fwht_lane(yv);
    fwht_cross(yv, L.wlog, lane);
    if (L.paired) {
      float unused = 0.0f;
      pair_stage(yv, unused, stage, partner, L.h, lane);
    }
    const float scale = sigma * inv_sqrt_d * cn;
#pragma unroll
    for (int e = 0; e < kEPL; ++e)
      yv[e] = __uint_as_float(__float_as_uint(yv[e] * scale) ^ smask[e]);
    if (staged_out) {
      store_rows_staged(out_h, a.ld_out, a.n, cols_h, base_row, L.wlog, lane, stage, yv);
    } else {
      store_rows_direct(out_h, a.ld_out, a.n, cols_h, row, L.paired ? lane : sub, yv);
    }
#pragma unroll
    for (int k = 0; k < MW; ++k) cw[k] = nw[k];
#pragma unroll
    for (int k = 0; k < 4; ++k) cz[k] = nz[k];
    cn = nn;
    cg = ng;
  }
}

// ------------------------------------------------------------ d = 128 kernel

// The lane's 4M code bits of coordinates 16 k + 4 sub .. 16 k + 4 sub + 3
// from the row's 4M record words (bit offset M (16 k + 4 sub)).
template <int M, int K>
__device__ __forceinline__ uint32_t code_group128(const uint32_t (&w)[4 * M], int sub) {
  if constexpr (M == 1) {
    return __builtin_amdgcn_ubfe(w[K >> 1], 16 * (K & 1) + 4 * sub, 4);
  } else if constexpr (M == 2) {
    return __builtin_amdgcn_ubfe(w[K], 8 * sub, 8);
  } else if constexpr (M == 3) {
    constexpr int w0 = (48 * K) >> 5, base = (48 * K) & 31;
    const uint64_t v = (static_cast<uint64_t>(w[w0 + 1]) << 32) | w[w0];
    return static_cast<uint32_t>(v >> (base + 12 * sub)) & 0xFFFu;
  } else {
    const uint32_t v = (sub & 2) ? w[2 * K + 1] : w[2 * K];
    return __builtin_amdgcn_ubfe(v, 16 * (sub & 1), 16);
  }
}

// d = d_in = 128, 1 <= m <= 4 (or prod m = 0), float32 rows 16-byte aligned
// with ld_out % 4 == 0.  Four lanes per vector, 16 vectors per wave; lane
// (vslot, sub) holds coordinate 16 k + 4 sub + t in register 4 k + t, so the
// in-lane butterflies run over coordinate bits 0, 1, 4, 5, 6, the cross-lane
// ones over bits 2, 3.  The rows leave through a per-wave LDS stage, eight at
// a time, so that each store instruction writes two whole rows (1 KiB in
// 128-byte lines) instead of 64 bytes of each of 16 rows: the memory system
// takes the whole-line pattern about a quarter faster.  The next group's
// records are loaded while the current one is computed.
template <int M, bool PROD, int ROT>
__global__ void __launch_bounds__(kThreads) decode128_kernel(DecodeArgs a) {
  constexpr int RW = M > 0 ? 4 * M : 1;        // record words per row
  constexpr int kHalfRow = 64 + 4;             // float32 per row of a half MFMA tile
  constexpr int kOutRow = 128 + 16;            // float32 per staged output row (no bank conflicts)
  constexpr int kWaveLds = 8 * kOutRow > 16 * kHalfRow ? 8 * kOutRow : 16 * kHalfRow;
  __shared__ __attribute__((aligned(16))) uint8_t st_lds[PROD ? kStBytes : 16];
  // per wave: the Z S tiles (prod), then the output rows
  __shared__ __attribute__((aligned(16))) float ct_lds[kWaves * kWaveLds];
  __shared__ float cb_lds[M >= 1 ? (1 << M) : 1];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sub = lane & 3;
  const int vslot = lane >> 2;
  if constexpr (M >= 1) {
    for (int k = threadIdx.x; k < (1 << M); k += kThreads) cb_lds[k] = a.centroids[k];
  }
  if constexpr (PROD) {
    uint16_t *st = reinterpret_cast<uint16_t *>(st_lds);     // st[j][i] = S[i][j]
    for (int idx = threadIdx.x; idx < 128 * 128; idx += kThreads)
      st[(idx & 127) * kStRow + (idx >> 7)] = a.qjl_s[idx];
  }
  __syncthreads();

  // RHT: sign of output coordinate j = 16 k + 4 sub + t, the RHT sign
  // times the (-1)^popcount(sub) the cross-lane butterflies leave on this
  // lane.  Block rotations: the parameters of the lane's quads 4 k + sub
  // (pairs 8 k + 2 sub, 8 k + 2 sub + 1), i.e. floats 16 k + 4 sub .. + 3.
  constexpr bool kRht = ROT == TQ_ROT_RHT;
  uint32_t smask[kRht ? kEPL : 1];
  float rc[kRht ? 1 : kEPL];
  if constexpr (kRht) {
    const uint32_t lane_sign = (__builtin_popcount(sub) & 1) ? 0x80000000u : 0u;
#pragma unroll
    for (int e = 0; e < kEPL; ++e)
      smask[e] = (a.signs[16 * (e >> 2) + 4 * sub + (e & 3)] < 0 ? 0x80000000u : 0u) ^ lane_sign;
  } else {
#pragma unroll
    for (int e = 0; e < kEPL; ++e) rc[e] = a.rot[16 * (e >> 2) + 4 * sub + (e & 3)];
  }
  const float rsd = 0.08838834764831845f;                       // 1 / sqrt(128)
  const float qjl_scale = 1.2533141373155003f / 128.0f;         // sqrt(pi/2) / d
  const int64_t groups = (a.n + 15) / 16;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kWaves;

  uint32_t cw[RW], nw[RW], cz[4], nz[4];
  float cn = 0.0f, cg = 0.0f, nn = 0.0f, ng = 0.0f;
  auto fetch = [&](int64_t g, uint32_t (&w)[RW], uint32_t (&z)[4], float &nr, float &gm) {
    const int64_t rw = g * 16 + vslot;
    const bool lv = rw < a.n;
    if constexpr (M >= 1) {
      const uint8_t *rec = a.codes + (lv ? rw : 0) * (16 * M);
#pragma unroll
      for (int q = 0; q < M; ++q) {
        const uint4 v = lv ? load_nt16(rec + 16 * q) : make_uint4(0, 0, 0, 0);
        w[4 * q] = v.x; w[4 * q + 1] = v.y; w[4 * q + 2] = v.z; w[4 * q + 3] = v.w;
      }
    }
    if constexpr (PROD) {
      const int64_t zrow = g * 16 + (lane & 15);
      const uint4 v = zrow < a.n ? load_nt16(a.qjl + zrow * 16) : make_uint4(0, 0, 0, 0);
      z[0] = v.x; z[1] = v.y; z[2] = v.z; z[3] = v.w;
      gm = lv ? a.rnorms[rw] : 0.0f;
    }
    nr = lv ? a.norms[rw] : 0.0f;
  };

  int64_t grp = static_cast<int64_t>(blockIdx.x) * kWaves + wave;
  if (grp < groups) fetch(grp, cw, cz, cn, cg);
  for (; grp < groups; grp += stride) {
    if (grp + stride < groups) fetch(grp + stride, nw, nz, nn, ng);
    float yv[kEPL];
    if constexpr (M >= 1) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        uint32_t gk;
        switch (k) {
          case 0: gk = code_group128<M, 0>(cw, sub); break;
          case 1: gk = code_group128<M, 1>(cw, sub); break;
          case 2: gk = code_group128<M, 2>(cw, sub); break;
          case 3: gk = code_group128<M, 3>(cw, sub); break;
          case 4: gk = code_group128<M, 4>(cw, sub); break;
          case 5: gk = code_group128<M, 5>(cw, sub); break;
          case 6: gk = code_group128<M, 6>(cw, sub); break;
          default: gk = code_group128<M, 7>(cw, sub); break;
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) yv[4 * k + t] = cb_lds[(gk >> (M * t)) & ((1u << M) - 1u)];
      }
    } else {
#pragma unroll
      for (int e = 0; e < kEPL; ++e) yv[e] = 0.0f;
    }
    if constexpr (PROD) {
      // T = Z S for the wave's 16 vectors with v_mfma_f32_16x16x32_bf16
      // (z = +-1 and S in bfloat16: every product exact, float32 sums);
      // output tiles go through LDS to the lane layout, 4 tiles at a time.
      const int fr = lane & 15, g = lane >> 4;
      bf16x8 af[4];
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) af[kc] = signs_bf16x8((cz[kc] >> (8 * g)) & 0xFFu);
      float *ct = ct_lds + wave * kWaveLds;
      const uint16_t *st = reinterpret_cast<const uint16_t *>(st_lds);
      const float gam = cg * qjl_scale;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int n4 = 0; n4 < 4; ++n4) {
          const int nt = 4 * h + n4;
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kc = 0; kc < 4; ++kc) {
            const bf16x8 b = *reinterpret_cast<const bf16x8 *>(st + (16 * nt + fr) * kStRow + 32 * kc + 8 * g);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[kc], b, acc, 0, 0, 0);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) ct[(4 * g + i) * kHalfRow + 16 * n4 + fr] = acc[i];
        }
        wave_lds_sync();
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
          const float4 t4 = *reinterpret_cast<const float4 *>(ct + vslot * kHalfRow + 16 * k4 + 4 * sub);
          const int e = 4 * (4 * h + k4);
          yv[e + 0] = fmaf(gam, t4.x, yv[e + 0]);
          yv[e + 1] = fmaf(gam, t4.y, yv[e + 1]);
          yv[e + 2] = fmaf(gam, t4.z, yv[e + 2]);
          yv[e + 3] = fmaf(gam, t4.w, yv[e + 3]);
        }
        wave_lds_sync();
      }
    }
    if constexpr (kRht) {
      fwht_lane(yv);
      cross_stage<0>(yv, (lane & 1) ? -1.0f : 1.0f);
      cross_stage<1>(yv, (lane & 2) ? -1.0f : 1.0f);
    } else {
      rotate_blocks<ROT, true>(yv, rc);     // quads are registers 4k..4k+3
    }
    const float scale = kRht ? rsd * cn : cn;
    float4 ov[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if constexpr (kRht) {
        ov[k].x = __uint_as_float(__float_as_uint(yv[4 * k + 0] * scale) ^ smask[4 * k + 0]);
        ov[k].y = __uint_as_float(__float_as_uint(yv[4 * k + 1] * scale) ^ smask[4 * k + 1]);
        ov[k].z = __uint_as_float(__float_as_uint(yv[4 * k + 2] * scale) ^ smask[4 * k + 2]);
        ov[k].w = __uint_as_float(__float_as_uint(yv[4 * k + 3] * scale) ^ smask[4 * k + 3]);
      } else {
        ov[k] = make_float4(yv[4 * k] * scale, yv[4 * k + 1] * scale, yv[4 * k + 2] * scale, yv[4 * k + 3] * scale);
      }
    }
    // rows 8 hf .. 8 hf + 7: their lanes write them to the stage, then every
    // lane stores 16 bytes of rows 2 i and 2 i + 1 (lanes 0..31, 32..63)
    float *so = ct_lds + wave * kWaveLds;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      if ((vslot >> 3) == hf) {
#pragma unroll
        for (int k = 0; k < 8; ++k) *reinterpret_cast<float4 *>(so + (vslot & 7) * kOutRow + 16 * k + 4 * sub) = ov[k];
      }
      wave_lds_sync();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 2 * i + (lane >> 5);
        const int64_t orow = grp * 16 + 8 * hf + r;
        const float4 v = *reinterpret_cast<const float4 *>(so + r * kOutRow + 4 * (lane & 31));
        if (orow < a.n) *reinterpret_cast<float4 *>(a.out + orow * a.ld_out + 4 * (lane & 31)) = v;
      }
      wave_lds_sync();
    }
#pragma unroll
    for (int k = 0; k < RW; ++k) cw[k] = nw[k];
#pragma unroll
    for (int k = 0; k < 4; ++k) cz[k] = nz[k];
    cn = nn;
    cg = ng;
  }
}

__global__ void __launch_bounds__(kThreads) rht_kernel(RhtArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kWaves * kStageBytes];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const Layout L = layout_of(a.log_lpv, kWaves, wave, lane);
  const int sub = L.sub, vslot = L.vslot, vpw = L.vpw;
  uint8_t *stage = lds + wave * kStageBytes;
  uint8_t *partner = lds + (wave ^ 1) * kStageBytes;
  const bool rht = a.rot_kind == TQ_ROT_RHT;
  uint32_t smask[kEPL];
  float rc[kEPL];
#pragma unroll
  for (int e = 0; e < kEPL; ++e) {
    smask[e] = rht && a.signs[sub * kEPL + e] < 0 ? 0x80000000u : 0u;
    rc[e] = rht ? 0.0f : a.rot[sub * kEPL + e];
  }
  const float scale = rht ? cross_sign(sub & 63) / sqrtf(static_cast<float>(a.d)) : 1.0f;
  const int in_cols = a.inverse ? a.d : a.d_in;
  const int out_cols = a.inverse ? a.d_in : a.d;
  const bool staged_in = ((in_cols & 3) == 0) && ((a.ld_in & 3) == 0) &&
                         ((reinterpret_cast<uintptr_t>(a.in) & 15) == 0);
  const bool staged_out = ((out_cols & 3) == 0) && ((a.ld_out & 3) == 0) &&
                          ((reinterpret_cast<uintptr_t>(a.out) & 15) == 0);
  const int64_t groups = (a.n + vpw - 1) / vpw;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * L.units;
  // this wave's columns of the input and output rows
  const int in_h = half_cols(L, in_cols), out_h = half_cols(L, out_cols);
  const float *in_p = a.in + 2048 * L.h;
  float *out_p = a.out + 2048 * L.h;
  // (paired: every wave of the block makes the same passes, a unit past the
  // end loading zeros and storing nothing)
  for (int64_t g0 = static_cast<int64_t>(blockIdx.x) * L.units; g0 < groups; g0 += stride) {
    const int64_t grp = g0 + L.unit;
    if (!L.paired && grp >= groups) break;
    const int64_t base_row = grp * vpw;
    const int64_t row = base_row + vslot;
    float v[kEPL];
    RowSpan src{in_p, a.ld_in, a.n, in_h, TQ_F32};
    if (staged_in) {
      load_rows_staged(src, base_row, L.wlog, lane, stage, v);
#pragma unroll
      for (int e = 0; e < kEPL; ++e)
        if (sub * kEPL + e >= in_cols) v[e] = 0.0f;
    } else {
      load_rows_direct(src, row, L.paired ? lane : sub, v);
    }
    if (rht) {
      if (!a.inverse) {
#pragma unroll
        for (int e = 0; e < kEPL; ++e) v[e] = __uint_as_float(__float_as_uint(v[e]) ^ smask[e]);
      }
      fwht_lane(v);
      fwht_cross(v, L.wlog, lane);
      if (L.paired) {
        float unused = 0.0f;
        pair_stage(v, unused, stage, partner, L.h, lane);
      }
#pragma unroll
      for (int e = 0; e < kEPL; ++e) v[e] *= scale;
      if (a.inverse) {
#pragma unroll
        for (int e = 0; e < kEPL; ++e) v[e] = __uint_as_float(__float_as_uint(v[e]) ^ smask[e]);
      }
    } else if (a.rot_kind == TQ_ROT_GIVENS) {
      if (a.inverse) rotate_blocks<TQ_ROT_GIVENS, true>(v, rc);
      else rotate_blocks<TQ_ROT_GIVENS, false>(v, rc);
    } else {
      if (a.inverse) rotate_blocks<TQ_ROT_QUAT, true>(v, rc);
      else rotate_blocks<TQ_ROT_QUAT, false>(v, rc);
    }
    if (staged_out) {
      store_rows_staged(out_p, a.ld_out, a.n, out_h, base_row, L.wlog, lane, stage, v);
    } else {
      store_rows_direct(out_p, a.ld_out, a.n, out_h, row, L.paired ? lane : sub, v);
    }
  }
}

// cap: 2048 blocks for streaming; 512 (two resident blocks per CU) when every
// block first stages S^T in LDS.
dim3 grid_for(int64_t n, int log_lpv, int64_t cap = 256 * 8) {
  // d = 4096: one vector per pair of waves
  const bool paired = log_lpv == kPairLogLpv;
  const int vpw = paired ? 1 : 64 >> log_lpv;
  const int units = paired ? kWaves / 2 : kWaves;
  const int64_t groups = (n + vpw - 1) / vpw;
  const int64_t blocks = (groups + units - 1) / units;
  return dim3(static_cast<unsigned>(blocks < cap ? blocks : cap));
}

template <int ROT>
int launch_decode128(const DecodeArgs &a, dim3 grid, dim3 block, hipStream_t s) {
  if (a.prod) {
    switch (a.m) {
#define TQ_CASE(MM) case MM: hipLaunchKernelGGL((decode128_kernel<MM, true, ROT>), grid, block, 0, s, a); break;
      TQ_CASE(0) TQ_CASE(1) TQ_CASE(2) TQ_CASE(3) TQ_CASE(4)
#undef TQ_CASE
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (a.m) {
#define TQ_CASE(MM) case MM: hipLaunchKernelGGL((decode128_kernel<MM, false, ROT>), grid, block, 0, s, a); break;
      TQ_CASE(1) TQ_CASE(2) TQ_CASE(3) TQ_CASE(4)
#undef TQ_CASE
      default: return hipErrorInvalidValue;
    }
  }
  return 0;
}

}  // namespace

int launch_decode(const DecodeArgs &a, void *stream) {
  (void)hipGetLastError();   // report only errors of this launch
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 block(kThreads);
  const bool fast = a.d == 128 && a.d_in == 128 && a.m <= 4 && (a.m >= 1 || a.prod) &&
                    (a.ld_out & 3) == 0 && (reinterpret_cast<uintptr_t>(a.out) & 15) == 0;
  if (a.rot_kind != TQ_ROT_RHT && !fast) return hipErrorInvalidValue;
  if (fast) {
    // three workgroups per CU: a measured sweep of 256..2,048 workgroups put
    // 512, 768 and 1,536 about 6 % ahead of 1,024 and 2,048
    const dim3 grid = grid_for(a.n, 2, 768);
    int err = 0;
    if (a.rot_kind == TQ_ROT_GIVENS) err = launch_decode128<TQ_ROT_GIVENS>(a, grid, block, s);
    else if (a.rot_kind == TQ_ROT_QUAT) err = launch_decode128<TQ_ROT_QUAT>(a, grid, block, s);
    else err = launch_decode128<TQ_ROT_RHT>(a, grid, block, s);
    if (err) return err;
    return hipGetLastError();
  }
  const dim3 grid = grid_for(a.n, a.log_lpv, (a.prod && a.d == 128) ? 512 : 2048);
  if (a.prod) {
    switch (a.m) {
#define TQ_CASE(MM) case MM: hipLaunchKernelGGL((decode_kernel<MM, true>), grid, block, 0, s, a); break;
      TQ_CASE(0) TQ_CASE(1) TQ_CASE(2) TQ_CASE(3) TQ_CASE(4) TQ_CASE(5) TQ_CASE(6) TQ_CASE(7)
#undef TQ_CASE
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (a.m) {
#define TQ_CASE(MM) case MM: hipLaunchKernelGGL((decode_kernel<MM, false>), grid, block, 0, s, a); break;
      TQ_CASE(1) TQ_CASE(2) TQ_CASE(3) TQ_CASE(4) TQ_CASE(5) TQ_CASE(6) TQ_CASE(7) TQ_CASE(8)
#undef TQ_CASE
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

int launch_rht(const RhtArgs &a, void *stream) {
  (void)hipGetLastError();   // report only errors of this launch
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(rht_kernel, grid_for(a.n, a.log_lpv), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace tq
