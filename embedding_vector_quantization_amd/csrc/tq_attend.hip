// Fused decode attention on TurboQuant codes for gfx950 (d = 128).
//
// Sources: the PolarQuant paper review (모두의 AI), step 9 "into attention":
// the reconstructed keys and values enter the usual scaled attention
// softmax(K^ q / sqrt d) V^; "TurboQuant: Online Vector Quantization" paper
// summary (Jump2Paper Archive) -- the inner-product estimator of the
// definitions table (with Definition 1 / Theorem D_prod for prod keys) and
// the mse dequantiser; AI Trends video summary chapter 06:06 (the rotation
// is undone by its transpose, the norm restores the scale).
//
// For query row i of KV group g (grouped-query attention: the group's query
// heads share its keys and values):
//   s_t = scale * est(q_i, key_t),  p = softmax(s),  o_i = sum_t p_t v~_t.
// Each v~_t = n_t Pi_v^T c[idx_t], so o_i = Pi_v^T (sum_t p_t n_t c[idx_t]):
// values are summed in the rotated domain and one inverse rotation per
// query row is applied at the end.
//
// Split over tokens: block (c, g, qb) takes tokens [T c, T c + T) of group g
// (T = 256, or 512 for the larger lookup tables) and queries 4 qb .. 4 qb + 3
// of the group.  It rotates its queries
// (and forms S q' for prod keys) in LDS, scores its tokens with the
// four-query lookup tables of the score kernel (one lane per token), forms
// the chunk maximum m, l = sum exp(s - m) and acc = sum exp(s - m) n_t
// c[idx_t] (lanes over coordinates), and writes (m, l, acc).
// attend_combine_kernel merges the chunks of a query row (log-sum-exp) and
// applies Pi_v^T.

#include <hip/hip_runtime.h>

#include "tq_device.h"
#include "tq_internal.h"
#include "tq_lut.h"

namespace tq {
namespace {

// Tokens per block = threads per block = 64 * waves: 4 waves, or 8 when the
// lookup table is 16 KiB or more, so that one table serves more tokens and a
// layer's blocks still fit on the CUs together (16 waves measured slower).
constexpr int kMinTok = 256;                   // the smallest block; sizes the workspace
template <int MK, bool PRODK>
constexpr int attend_waves() { return entries4<MK, PRODK>() >= 1024 ? 8 : 4; }

// Keys with 0..2 code bits are scored on the int8 matrix cores (the
// fixed-point form of the grouped score), the others with lookup tables.
template <int MK, bool PRODK>
constexpr bool attend_i8() { return MK <= 2 && (MK >= 1 || PRODK); }

// Dynamic LDS of the partial kernel.  Tables: the lookup table (its space
// later holds the per-wave value sums).  int8: the A operands (6 KiB, in an
// 8 KiB slot), then per wave a [64 tokens][8] stage of the estimates and,
// for prod keys, a [64][4] stage of the QJL words; the value sums reuse the
// space from its start.
constexpr int kA8Bytes = 8192;
template <int MK, bool PRODK>
constexpr int attend_dyn_lds() {
  constexpr int W = attend_waves<MK, PRODK>();
  constexpr int red = W * 4 * 128 * 4;
  if constexpr (attend_i8<MK, PRODK>()) {
    constexpr int used = kA8Bytes + W * 64 * 8 * 4 + (PRODK ? W * 64 * 16 : 0);
    return used > red ? used : red;
  } else {
    return entries4<MK, PRODK>() * 16;
  }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Code bits of coordinates 2 l and 2 l + 1 (2 MV bits at bit 2 MV l) of a
// value record of 4 MV words.
template <int MV>
__device__ __forceinline__ uint32_t value_pair(const uint32_t *rec, int lane) {
  constexpr int W = 2 * MV;
  const int bit = W * lane;
  const int w0 = bit >> 5, off = bit & 31;
  if constexpr (32 % W == 0) {
    return __builtin_amdgcn_ubfe(rec[w0], off, W);
  } else {
    // a field may straddle two words; the straddling ones never start in
    // the record's last word
    const uint32_t lo = rec[w0];
    const uint32_t hi = (w0 + 1 < 4 * MV) ? rec[w0 + 1] : 0u;
    return static_cast<uint32_t>(((static_cast<uint64_t>(hi) << 32) | lo) >> off) & ((1u << W) - 1u);
  }
}

template <int MK, bool PRODK, int MV>
__global__ void __launch_bounds__((64 * attend_waves<MK, PRODK>())) attend_partial_kernel(AttnArgs a) {
  constexpr int kWaves = attend_waves<MK, PRODK>();
  constexpr int kThreads = 64 * kWaves;
  constexpr int kTok = kThreads;
  extern __shared__ __attribute__((aligned(16))) float4 lut4[];
  using S = Shape4<MK>;
  using RS = RecStage<MK>;
  constexpr int KK = 1 << MK;
  constexpr int E = entries4<MK, PRODK>();
  __shared__ float cbk[KK > 1 ? KK : 2];
  __shared__ float2 cbv2[1 << (2 * MV)];           // value centroids of a coordinate pair
  __shared__ __attribute__((aligned(16))) uint32_t rstage[RS::kOn ? kWaves * RS::kWaveDwords : 4];
  // Buffers of the later phases reuse those of the earlier ones (a barrier
  // lies between the last read of the old and the first write of the new),
  // so that all blocks of a layer fit on the CUs at once: the weights
  // p_t * n_t per query take the key-record stage (when there is one), the
  // per-wave value sums take the lookup table (at least 8 KiB).
  constexpr bool kWInStage = RS::kOn && RS::kWaveDwords * kWaves * 4 >= kTok * 16;
  __shared__ __attribute__((aligned(16))) float4 w_own[kWInStage ? 1 : kTok];
  float4 *const w_lds = kWInStage ? reinterpret_cast<float4 *>(rstage) : w_own;
  constexpr bool kI8 = attend_i8<MK, PRODK>();
  static_assert(attend_dyn_lds<MK, PRODK>() >= kWaves * 4 * 128 * 4, "value sums fit in the dynamic LDS");
  float (*const red)[4][128] = reinterpret_cast<float (*)[4][128]>(lut4);
  __shared__ float vmax[kI8 ? 8 : 1], vsum[kI8 ? 8 : 1];
  __shared__ float4 wred[kWaves];
  __shared__ __attribute__((aligned(16))) float qr_lds[4][128];             // rotated queries
  __shared__ __attribute__((aligned(16))) float sq_lds[PRODK ? 4 : 1][128]; // S q' (prod keys)

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  if constexpr (MK >= 1) {
    for (int k = threadIdx.x; k < KK; k += kThreads) cbk[k] = a.k_centroids[k];
  }
  for (int k = threadIdx.x; k < (1 << (2 * MV)); k += kThreads)
    cbv2[k] = make_float2(a.v_centroids[k & ((1 << MV) - 1)], a.v_centroids[k >> MV]);

  const int qblocks = (a.nq + 3) / 4;
  const int64_t grp = blockIdx.y / qblocks;
  const int qb = blockIdx.y - static_cast<int>(grp) * qblocks;
  const int q0 = 4 * qb;
  const int nqb = a.nq - q0 < 4 ? a.nq - q0 : 4;     // live queries of this block
  const int64_t qrow0 = grp * a.nq + q0;             // query row over all groups
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kTok;
  const int64_t key0 = grp * a.n;

  // Every global load of the block is issued first, so that its latency
  // overlaps the table build: this lane's key record (staged), norms, QJL
  // word, and the value code bits of the wave's 64 tokens.
  const int64_t tl = t0 + threadIdx.x;                // token within the group
  const bool live = tl < a.n;
  const int64_t tk = key0 + (live ? tl : 0);
  uint4 nb[RS::kOn ? MK : 1];
  if constexpr (MK >= 1) {
    const int64_t k0 = t0 + 64 * wave;
    RS::issue(a.k_codes, key0 + k0, a.n - k0, lane, nb);
  }
  uint4 zv = make_uint4(0, 0, 0, 0);
  float gk = 0.0f;
  if constexpr (PRODK) {
    zv = load_nt16(a.k_qjl + tk * 16);
    gk = a.k_rnorms[tk] * (kQjlScale / 128.0f);
  }
  const float nk = a.k_norms[tk];
  const float nv = live ? a.v_norms[tk] : 0.0f;
  const int64_t tw = t0 + 64 * wave;               // wave's first token
  const int ntok = a.n - tw < 64 ? (a.n - tw > 0 ? static_cast<int>(a.n - tw) : 0) : 64;
  constexpr int RV = 4 * MV;                        // words per value record
  uint32_t pr[64];
  if (ntok == 64) {
    // the wave's 64 records lie back to back: one base address, and record
    // j's words at a constant offset the loads carry as an immediate
    const uint32_t *recs = reinterpret_cast<const uint32_t *>(a.v_codes) + (key0 + tw) * RV;
#pragma unroll
    for (int j = 0; j < 64; ++j) pr[j] = value_pair<MV>(recs + j * RV, lane);
  } else {
#pragma unroll
    for (int j = 0; j < 64; ++j) {
      // clamped to the group's last token, so the address is always valid
      const int64_t tj = tw + j < a.n ? tw + j : a.n - 1;
      const uint32_t *rec = reinterpret_cast<const uint32_t *>(a.v_codes) + (key0 + tj) * RV;
      const uint32_t bits = value_pair<MV>(rec, lane);
      pr[j] = j < ntok ? bits : 0u;
    }
  }

  // ---- the block's queries: wave w rotates query q0 + w, q' = Pi q
  if (wave < nqb) {
    const float *qg = a.q + (qrow0 + wave) * a.ldq;
    const int j0 = 2 * lane, j1 = 2 * lane + 1;
    float v0 = j0 < a.d_in ? qg[j0] : 0.0f;
    float v1 = j1 < a.d_in ? qg[j1] : 0.0f;
    v0 = a.k_signs[j0] < 0 ? -v0 : v0;
    v1 = a.k_signs[j1] < 0 ? -v1 : v1;
    fwht128_wave(v0, v1, lane);
    const float rsd = 0.08838834764831845f;          // 1 / sqrt(128)
    qr_lds[wave][j0] = v0 * rsd;
    qr_lds[wave][j1] = v1 * rsd;
  }
  __syncthreads();
  if constexpr (PRODK) {
    // s = S q' for the block's queries: two outputs per thread, rows of S
    // (bfloat16) from global memory, q' from LDS
    for (int o = threadIdx.x; o < 4 * 128; o += kThreads) {
      const int q = o >> 7, i = o & 127;
      float acc_s = 0.0f;
      if (q < nqb) {
        const uint4 *srow = reinterpret_cast<const uint4 *>(a.qjl_s + i * 128);
#pragma unroll
        for (int c = 0; c < 16; ++c) {
          const uint4 w = srow[c];
          const float *qq = &qr_lds[q][8 * c];
          acc_s = fmaf(bf16_lo(w.x), qq[0], acc_s);
          acc_s = fmaf(bf16_hi(w.x), qq[1], acc_s);
          acc_s = fmaf(bf16_lo(w.y), qq[2], acc_s);
          acc_s = fmaf(bf16_hi(w.y), qq[3], acc_s);
          acc_s = fmaf(bf16_lo(w.z), qq[4], acc_s);
          acc_s = fmaf(bf16_hi(w.z), qq[5], acc_s);
          acc_s = fmaf(bf16_lo(w.w), qq[6], acc_s);
          acc_s = fmaf(bf16_hi(w.w), qq[7], acc_s);
        }
      }
      sq_lds[q][i] = acc_s;
    }
    __syncthreads();
  }

  // ---- lookup tables of the block's queries (as in the four-query score)
  for (int i = threadIdx.x; i < (kI8 ? 0 : E); i += kThreads) {
    float v4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (q >= nqb) continue;
      float val = 0.0f;
      if (i < S::ENTRIES) {
        if constexpr (MK >= 1) {
          const int t = i >> S::W;
          const int v = i & ((1 << S::W) - 1);
          const float *qp = &qr_lds[q][t * S::G];
#pragma unroll
          for (int u = 0; u < S::G; ++u) val = fmaf(qp[u], cbk[(v >> (MK * u)) & (KK - 1)], val);
        }
      } else if constexpr (PRODK) {
        const int rz = i - S::ENTRIES;
        const int k = rz >> 4;
        const int v = rz & 15;
        const float *sq = &sq_lds[q][4 * k];
#pragma unroll
        for (int t = 0; t < 4; ++t) val += ((v >> t) & 1) ? sq[t] : -sq[t];
      }
      v4[q] = val;
    }
    lut4[i] = make_float4(v4[0], v4[1], v4[2], v4[3]);
  }
  __syncthreads();

  // ---- scores of the block's tokens, one lane per token
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float4 accz = make_float4(0.f, 0.f, 0.f, 0.f);
  if constexpr (kI8) {
    // the int8 matrix cores: the queries in fixed point (A), the raw code and
    // QJL bits of 16 tokens (B) per product; lane (kb, key) gets query kb's
    // digit sums for token 16 gi + key, which go through a per-wave LDS
    // stage back to one lane per token
    uint8_t *dyn = reinterpret_cast<uint8_t *>(lut4);
    auto a8 = reinterpret_cast<uint32_t (*)[64][4]>(dyn);
    float (*const sst)[8] = reinterpret_cast<float (*)[8]>(dyn + kA8Bytes) + 64 * wave;
    uint4 *const zst = reinterpret_cast<uint4 *>(dyn + kA8Bytes + kWaves * 64 * 8 * 4) + 64 * wave;
    float cA = 0.0f, cB = 0.0f;
    i8_coefs<MK>(a.k_centroids, cA, cB);
    i8_query_operands<MK, PRODK, kThreads>(qr_lds, sq_lds, nqb, cA, cB, a8, vmax, vsum);
    uint32_t aop[kI8Ops][4];
#pragma unroll
    for (int o = 0; o < kI8Ops; ++o)
#pragma unroll
      for (int i = 0; i < 4; ++i) aop[o][i] = a8[o][lane][i];
    const int kb = lane >> 4, key = lane & 15;
    const float cm = i8_scale(vmax[kb]);
    const float cc = i8_offset<MK>(a.k_centroids, vsum[kb]);
    const float cz = 2.0f * i8_scale(vmax[4 + kb]), cz0 = -vsum[4 + kb];
    uint32_t *ws = rstage + wave * RS::kWaveDwords;
    if constexpr (MK >= 1) RS::put(ws, lane, nb);
    if constexpr (PRODK) zst[lane] = zv;
    wave_lds_sync();
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const int tok = 16 * gi + key;
      uint32_t bt[4];
      if constexpr (MK >= 1) {
        i32x4 dm = {0, 0, 0, 0};
        if constexpr (MK == 2) {
          const uint2 cw = *reinterpret_cast<const uint2 *>(ws + tok * RS::kPitch + 2 * kb);
          const uint32_t w2[2] = {cw.x, cw.y};
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            bytes_of<false>(w2[h], bt);
            dm = mfma_i8(aop[h], bt, dm);
            bytes_of<true>(w2[h], bt);
            dm = mfma_i8(aop[2 + h], bt, dm);
          }
        } else {
          const uint32_t cw = ws[tok * RS::kPitch + kb];
          bytes_of<false>(cw, bt);
          dm = mfma_i8(aop[0], bt, dm);
          bytes_of<true>(cw, bt);
          dm = mfma_i8(aop[1], bt, dm);
        }
        sst[tok][kb] = fmaf(cm, digits(dm), cc);
      }
      if constexpr (PRODK) {
        const uint32_t zw = reinterpret_cast<const uint32_t *>(zst + tok)[kb];
        i32x4 dz = {0, 0, 0, 0};
        bytes_of<false>(zw, bt);
        dz = mfma_i8(aop[4], bt, dz);
        bytes_of<true>(zw, bt);
        dz = mfma_i8(aop[5], bt, dz);
        sst[tok][4 + kb] = fmaf(cz, digits(dz), cz0);
      }
    }
    wave_lds_sync();
    if constexpr (MK >= 1) acc = *reinterpret_cast<const float4 *>(sst[lane]);
    if constexpr (PRODK) accz = *reinterpret_cast<const float4 *>(sst[lane] + 4);
  } else if constexpr (MK >= 1) {
    uint32_t w[4 * MK];
    uint32_t *ws = rstage + wave * RS::kWaveDwords;
    RS::put(ws, lane, nb);
    wave_lds_sync();
    RS::get(ws, lane, w);
    float4 part[2] = {make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)};
    groups4<MK, 0>(w, lut4, part);
    acc = part[0];
    add4(acc, part[1]);
  }
  if constexpr (PRODK && !kI8) {
    const uint32_t zw[4] = {zv.x, zv.y, zv.z, zv.w};
    float4 part[2] = {make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)};
    nibbles4<0>(zw, lut4 + S::ENTRIES, part);
    accz = part[0];
    add4(accz, part[1]);
  }
  const float sc[4] = {a.scale * nk * fmaf(gk, accz.x, acc.x), a.scale * nk * fmaf(gk, accz.y, acc.y),
                       a.scale * nk * fmaf(gk, accz.z, acc.z), a.scale * nk * fmaf(gk, accz.w, acc.w)};
  const float ninf = -__builtin_inff();

  // ---- chunk maximum and exponentials
  float mx[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) mx[q] = wave_max(live ? sc[q] : ninf);
  if (lane == 0) wred[wave] = make_float4(mx[0], mx[1], mx[2], mx[3]);
  __syncthreads();
  float m[4] = {ninf, ninf, ninf, ninf};
#pragma unroll
  for (int wv = 0; wv < kWaves; ++wv) {
    const float4 r = wred[wv];
    m[0] = fmaxf(m[0], r.x); m[1] = fmaxf(m[1], r.y); m[2] = fmaxf(m[2], r.z); m[3] = fmaxf(m[3], r.w);
  }
  float p[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) p[q] = live ? __expf(sc[q] - m[q]) : 0.0f;
  w_lds[threadIdx.x] = make_float4(p[0] * nv, p[1] * nv, p[2] * nv, p[3] * nv);
  float ls[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) ls[q] = wave_sum(p[q]);
  __syncthreads();                                 // everyone has read wred; w_lds complete
  if (lane == 0) wred[wave] = make_float4(ls[0], ls[1], ls[2], ls[3]);

  // ---- values: lanes over coordinates 2 l, 2 l + 1, wave over 64 tokens
  // (tokens past the end have weight 0 and code bits 0)
  float va[4][2] = {{0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}};
  if (ntok > 0) {
#pragma unroll
    for (int j = 0; j < 64; ++j) {
      const float4 wt = w_lds[64 * wave + j];
      const float2 cc = cbv2[pr[j]];
      const float c0 = cc.x, c1 = cc.y;
      va[0][0] = fmaf(wt.x, c0, va[0][0]); va[0][1] = fmaf(wt.x, c1, va[0][1]);
      va[1][0] = fmaf(wt.y, c0, va[1][0]); va[1][1] = fmaf(wt.y, c1, va[1][1]);
      va[2][0] = fmaf(wt.z, c0, va[2][0]); va[2][1] = fmaf(wt.z, c1, va[2][1]);
      va[3][0] = fmaf(wt.w, c0, va[3][0]); va[3][1] = fmaf(wt.w, c1, va[3][1]);
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    red[wave][q][2 * lane] = va[q][0];
    red[wave][q][2 * lane + 1] = va[q][1];
  }
  __syncthreads();

  // ---- partial (m, l, acc[128]) per query of the block
  const int64_t nchunks = gridDim.x;
  for (int i = threadIdx.x; i < 4 * 128; i += kThreads) {
    const int q = i >> 7, jj = i & 127;
    if (q >= nqb) continue;
    float s = 0.0f;
#pragma unroll
    for (int wv = 0; wv < kWaves; ++wv) s += red[wv][q][jj];
    a.part[((qrow0 + q) * nchunks + blockIdx.x) * kAttnPart + 4 + jj] = s;
  }
  if (threadIdx.x < 4 && static_cast<int>(threadIdx.x) < nqb) {
    const int q = threadIdx.x;
    float l = 0.0f;
#pragma unroll
    for (int wv = 0; wv < kWaves; ++wv) {
      const float4 r = wred[wv];
      l += q == 0 ? r.x : q == 1 ? r.y : q == 2 ? r.z : r.w;
    }
    float *pp = a.part + ((qrow0 + q) * nchunks + blockIdx.x) * kAttnPart;
    pp[0] = m[q];
    pp[1] = l;
  }
}

// One block of 16 waves per query row: merge the chunks, then
// o = Pi_v^T (acc / l).  Wave w loads chunks w, w + 16, ... (at most
// kCombineChunks per wave) in one round trip; the maxima, exponential sums
// and value sums are combined across the waves in LDS.
constexpr int kCombineThreads = 1024;
constexpr int kCombineWaves = kCombineThreads / 64;
constexpr int kCombineChunks = 8;

__global__ void __launch_bounds__(kCombineThreads) attend_combine_kernel(AttnArgs a, int64_t nchunks) {
  __shared__ float wm[kCombineWaves], wl[kCombineWaves];
  __shared__ __attribute__((aligned(16))) float2 wv[kCombineWaves][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t row = blockIdx.x;
  const float *pr = a.part + row * nchunks * kAttnPart;
  const float ninf = -__builtin_inff();
  float m_all = ninf, l_all = 0.0f, v0 = 0.0f, v1 = 0.0f;
  // chunks are merged in passes of kCombineWaves * kCombineChunks
  for (int64_t base = 0; base < nchunks; base += kCombineWaves * kCombineChunks) {
    float mc[kCombineChunks], lc[kCombineChunks];
    float2 xc[kCombineChunks];
#pragma unroll
    for (int u = 0; u < kCombineChunks; ++u) {
      const int64_t c = base + wave + u * kCombineWaves;
      const bool ok = c < nchunks;
      const float *pc = pr + (ok ? c : 0) * kAttnPart;
      mc[u] = ok ? pc[0] : ninf;
      lc[u] = ok ? pc[1] : 0.0f;
      xc[u] = ok ? *reinterpret_cast<const float2 *>(pc + 4 + 2 * lane) : make_float2(0.f, 0.f);
    }
    float mw = m_all;
#pragma unroll
    for (int u = 0; u < kCombineChunks; ++u) mw = fmaxf(mw, mc[u]);
    // rescale what this wave holds to the new running maximum
    const float r = m_all == ninf ? 0.0f : __expf(m_all - mw);
    l_all *= r;
    v0 *= r;
    v1 *= r;
#pragma unroll
    for (int u = 0; u < kCombineChunks; ++u) {
      const float f = mc[u] == ninf ? 0.0f : __expf(mc[u] - mw);
      l_all = fmaf(f, lc[u], l_all);
      v0 = fmaf(f, xc[u].x, v0);
      v1 = fmaf(f, xc[u].y, v1);
    }
    m_all = mw;
  }
  if (lane == 0) wm[wave] = m_all;
  __syncthreads();
  float M = ninf;
#pragma unroll
  for (int w = 0; w < kCombineWaves; ++w) M = fmaxf(M, wm[w]);
  const float r = m_all == ninf ? 0.0f : __expf(m_all - M);
  if (lane == 0) wl[wave] = l_all * r;
  wv[wave][lane] = make_float2(v0 * r, v1 * r);
  __syncthreads();
  if (wave != 0) return;
  float L = 0.0f;
  v0 = 0.0f;
  v1 = 0.0f;
#pragma unroll
  for (int w = 0; w < kCombineWaves; ++w) {
    L += wl[w];
    v0 += wv[w][lane].x;
    v1 += wv[w][lane].y;
  }
  const float inv = 1.0f / L;
  v0 *= inv;
  v1 *= inv;
  fwht128_wave(v0, v1, lane);
  const float rsd = 0.08838834764831845f;          // 1 / sqrt(128)
  const int j0 = 2 * lane, j1 = 2 * lane + 1;
  float *o = a.out + row * a.ld_out;
  if (j0 < a.d_in) o[j0] = v0 * rsd * static_cast<float>(a.v_signs[j0]);
  if (j1 < a.d_in) o[j1] = v1 * rsd * static_cast<float>(a.v_signs[j1]);
}

// Launches the partial kernel; nchunks receives its number of token chunks.
template <int MK, bool PRODK, int MV>
int launch_partial(const AttnArgs &a, int64_t &nchunks, hipStream_t s) {
  const size_t lds = static_cast<size_t>(attend_dyn_lds<MK, PRODK>());
  constexpr int threads = 64 * attend_waves<MK, PRODK>();
  nchunks = (a.n + threads - 1) / threads;
  const void *fn = reinterpret_cast<const void *>(&attend_partial_kernel<MK, PRODK, MV>);
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  const int64_t qblocks = (a.nq + 3) / 4;
  hipLaunchKernelGGL((attend_partial_kernel<MK, PRODK, MV>),
                     dim3(static_cast<unsigned>(nchunks), static_cast<unsigned>(a.groups * qblocks)),
                     dim3(threads), lds, s, a);
  return hipGetLastError();
}

template <int MK, bool PRODK>
int launch_mv(const AttnArgs &a, int64_t &nchunks, hipStream_t s) {
  switch (a.mv) {
    case 1: return launch_partial<MK, PRODK, 1>(a, nchunks, s);
    case 2: return launch_partial<MK, PRODK, 2>(a, nchunks, s);
    case 3: return launch_partial<MK, PRODK, 3>(a, nchunks, s);
    case 4: return launch_partial<MK, PRODK, 4>(a, nchunks, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int64_t attend_chunks(int64_t n) { return (n + kMinTok - 1) / kMinTok; }

int launch_attend(const AttnArgs &a, void *stream) {
  (void)hipGetLastError();   // report only errors of this launch
  hipStream_t s = static_cast<hipStream_t>(stream);
  int64_t nchunks = 0;                       // at most attend_chunks(a.n)
  int err;
  if (a.prodk) {
    switch (a.mk) {
      case 0: err = launch_mv<0, true>(a, nchunks, s); break;
      case 1: err = launch_mv<1, true>(a, nchunks, s); break;
      case 2: err = launch_mv<2, true>(a, nchunks, s); break;
      case 3: err = launch_mv<3, true>(a, nchunks, s); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (a.mk) {
      case 1: err = launch_mv<1, false>(a, nchunks, s); break;
      case 2: err = launch_mv<2, false>(a, nchunks, s); break;
      case 3: err = launch_mv<3, false>(a, nchunks, s); break;
      case 4: err = launch_mv<4, false>(a, nchunks, s); break;
      default: return hipErrorInvalidValue;
    }
  }
  if (err) return err;
  hipLaunchKernelGGL(attend_combine_kernel, dim3(static_cast<unsigned>(a.nq_all)), dim3(kCombineThreads), 0, s,
                     a, nchunks);
  return hipGetLastError();
}

}  // namespace tq
