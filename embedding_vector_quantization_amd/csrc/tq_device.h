// Device helpers shared by the gfx950 kernels: cross-lane partners, the
// fast Walsh-Hadamard butterflies, bit appends and element conversion.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_internal.h"

namespace tq {

// ---------------------------------------------------------------- lanes

// Value of `v` held by lane (lane ^ (1 << K)), K = 0..5.  DPP for the
// patterns gfx9 DPP reaches in one instruction (xor 1, xor 2 via quad_perm,
// xor 8 as a rotate by 8 within a row of 16), ds_swizzle for xor 4 and
// xor 16 (inside 32-lane halves), ds_bpermute for xor 32.
template <int K>
__device__ __forceinline__ float xor_partner(float v) {
  const int iv = __float_as_int(v);
  int r;
  if constexpr (K == 0) {
    r = __builtin_amdgcn_mov_dpp(iv, 0xB1, 0xF, 0xF, true);   // quad_perm [1,0,3,2]
  } else if constexpr (K == 1) {
    r = __builtin_amdgcn_mov_dpp(iv, 0x4E, 0xF, 0xF, true);   // quad_perm [2,3,0,1]
  } else if constexpr (K == 2) {
    r = __builtin_amdgcn_ds_swizzle(iv, (4 << 10) | 0x1F);    // xor 4
  } else if constexpr (K == 3) {
    r = __builtin_amdgcn_mov_dpp(iv, 0x128, 0xF, 0xF, true);  // row_ror:8
  } else if constexpr (K == 4) {
    r = __builtin_amdgcn_ds_swizzle(iv, (16 << 10) | 0x1F);   // xor 16
  } else {
    r = __shfl_xor(iv, 32);
  }
  return __int_as_float(r);
}

// Sum of v over the 2^log_lpv lanes of a vector group (all lanes get it).
__device__ __forceinline__ float group_sum(float v, int log_lpv) {
  if (log_lpv > 0) v += xor_partner<0>(v);
  if (log_lpv > 1) v += xor_partner<1>(v);
  if (log_lpv > 2) v += xor_partner<2>(v);
  if (log_lpv > 3) v += xor_partner<3>(v);
  if (log_lpv > 4) v += xor_partner<4>(v);
  if (log_lpv > 5) v += xor_partner<5>(v);
  return v;
}

// ---------------------------------------------------------------- FWHT

// In-lane butterflies over the 5 element-index bits: v <- H_32 v.  With
// H0 > 1 the stages below H0 have been applied already (the stages commute).
template <int H0 = 1>
__device__ __forceinline__ void fwht_lane(float (&v)[kEPL]) {
#pragma unroll
  for (int h = H0; h < kEPL; h <<= 1) {
#pragma unroll
    for (int i = 0; i < kEPL; ++i) {
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
}

// v[i] += eps * (v[i] of the partner lane) for 16 elements with
// v_fmac_f32_dpp (the partner's value arrives through the DPP source), one
// instruction per element instead of a DPP move and an FMA.  The leading
// s_nop 1 provides the two wait states a DPP read needs after a VALU write of
// its source register; within the block no instruction reads a register
// written by the one before it.
#define TQ_FMAC_DPP16(CTRL, v, o, eps)          \
  asm("s_nop 1\n\t"          \
      "v_fmac_f32_dpp %0, %0, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"   \
      "v_fmac_f32_dpp %1, %1, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"   \
      "v_fmac_f32_dpp %2, %2, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"   \
      "v_fmac_f32_dpp %3, %3, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"   \
      "v_fmac_f32_dpp %4, %4, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"   \
      "v_fmac_f32_dpp %5, %5, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"   \
      "v_fmac_f32_dpp %6, %6, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"   \
      "v_fmac_f32_dpp %7, %7, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"   \
      "v_fmac_f32_dpp %8, %8, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"   \
      "v_fmac_f32_dpp %9, %9, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"   \
      "v_fmac_f32_dpp %10, %10, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"   \
      "v_fmac_f32_dpp %11, %11, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"   \
      "v_fmac_f32_dpp %12, %12, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"   \
      "v_fmac_f32_dpp %13, %13, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"   \
      "v_fmac_f32_dpp %14, %14, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"   \
      "v_fmac_f32_dpp %15, %15, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"   \
      : "+v"(v[o + 0]), "+v"(v[o + 1]), "+v"(v[o + 2]), "+v"(v[o + 3]), "+v"(v[o + 4]),   \
        "+v"(v[o + 5]), "+v"(v[o + 6]), "+v"(v[o + 7]), "+v"(v[o + 8]), "+v"(v[o + 9]),   \
        "+v"(v[o + 10]), "+v"(v[o + 11]), "+v"(v[o + 12]), "+v"(v[o + 13]),             \
        "+v"(v[o + 14]), "+v"(v[o + 15])                                              \
      : "v"(eps))

template <int K>
__device__ __forceinline__ void cross_stage(float (&v)[kEPL], float eps) {
  static_assert(kEPL == 32, "two blocks of 16 elements");
  if constexpr (K == 0) {
    TQ_FMAC_DPP16("quad_perm:[1,0,3,2]", v, 0, eps);
    TQ_FMAC_DPP16("quad_perm:[1,0,3,2]", v, 16, eps);
  } else if constexpr (K == 1) {
    TQ_FMAC_DPP16("quad_perm:[2,3,0,1]", v, 0, eps);
    TQ_FMAC_DPP16("quad_perm:[2,3,0,1]", v, 16, eps);
  } else {
#pragma unroll
    for (int i = 0; i < kEPL; ++i) v[i] = fmaf(xor_partner<K>(v[i]), eps, v[i]);
  }
}

// Butterflies across the lanes of a vector group (lane bits 0..log_lpv-1 are
// coordinate bits 5..).  Each stage computes v + eps * partner with
// eps = -1 on lanes whose bit is set; those lanes then hold the negated
// difference.  Partners always carry the same accumulated sign, so after all
// stages lane `sub` holds (-1)^popcount(sub) * (H v); the caller folds that
// sign into its scale factor.
__device__ __forceinline__ void fwht_cross(float (&v)[kEPL], int log_lpv, int lane) {
  if (log_lpv > 0) cross_stage<0>(v, (lane & 1) ? -1.0f : 1.0f);
  if (log_lpv > 1) cross_stage<1>(v, (lane & 2) ? -1.0f : 1.0f);
  if (log_lpv > 2) cross_stage<2>(v, (lane & 4) ? -1.0f : 1.0f);
  if (log_lpv > 3) cross_stage<3>(v, (lane & 8) ? -1.0f : 1.0f);
  if (log_lpv > 4) cross_stage<4>(v, (lane & 16) ? -1.0f : 1.0f);
  if (log_lpv > 5) cross_stage<5>(v, (lane & 32) ? -1.0f : 1.0f);
}

__device__ __forceinline__ float cross_sign(int sub) {
  return (__builtin_popcount(sub) & 1) ? -1.0f : 1.0f;
}

// ---------------------------------------------------------------- paired waves (d = 4096)

// At d = 4096 a vector spans two waves of a block (128 lanes of 32
// coordinates): wave h of the pair holds coordinates 2048 h + 32 lane + e.
// The butterfly stage over coordinate bit 11 and the sums over the vector
// then go through LDS: each wave of the pair writes its values to its own
// exchange area (64 lanes x 144 bytes; the 16-byte pad keeps the lanes'
// 16-byte accesses in distinct banks) and reads its partner's.  Every wave
// of the block must make the same calls (they hold block barriers).
constexpr int kPairLaneBytes = kEPL * 4 + 16;

// v <- v + partner (h = 0) or partner - v (h = 1); x <- x + partner's x.
__device__ __forceinline__ void pair_stage(float (&v)[kEPL], float &x, uint8_t *mine, const uint8_t *other,
                                           int h, int lane) {
  float *dst = reinterpret_cast<float *>(mine + lane * kPairLaneBytes);
#pragma unroll
  for (int q = 0; q < kEPL / 4; ++q)
    reinterpret_cast<float4 *>(dst)[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
  dst[kEPL] = x;
  __syncthreads();
  const float *src = reinterpret_cast<const float *>(other + lane * kPairLaneBytes);
#pragma unroll
  for (int q = 0; q < kEPL / 4; ++q) {
    const float4 o = reinterpret_cast<const float4 *>(src)[q];
    const float ov[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) v[4 * q + t] = h == 0 ? v[4 * q + t] + ov[t] : ov[t] - v[4 * q + t];
  }
  x += src[kEPL];
  __syncthreads();
}

// A lane's place in the register layout: at d = 4096 (log_lpv ==
// kPairLogLpv) a vector over a pair of waves, wave h = wave & 1 holding
// coordinates 2048 h .., as one 64-lane vector of 2048 within the wave (wlog
// = 6); otherwise 64 / LPV vectors per wave.  Work units are vector groups
// of a wave, or the vector of a pair.
struct Layout {
  bool paired;
  int h;          // half of the vector this wave holds (paired), else 0
  int wlog;       // log2 of the vector's lanes within one wave
  int sub;        // lane's index within the vector (0 .. d/32 - 1)
  int vslot;      // vector slot within the wave
  int vpw;        // vectors per wave (1 when paired)
  int units;      // work units per workgroup
  int unit;       // this wave's unit
};

__device__ __forceinline__ Layout layout_of(int log_lpv, int waves, int wave, int lane) {
  Layout L;
  L.paired = log_lpv == kPairLogLpv;
  L.h = L.paired ? (wave & 1) : 0;
  L.wlog = L.paired ? 6 : log_lpv;
  L.sub = L.paired ? 64 * L.h + lane : lane & ((1 << L.wlog) - 1);
  L.vslot = L.paired ? 0 : lane >> L.wlog;
  L.vpw = L.paired ? 1 : 64 >> L.wlog;
  L.units = L.paired ? waves / 2 : waves;
  L.unit = L.paired ? (wave >> 1) : wave;
  return L;
}

// The columns of a row (cols of them) that fall in this wave's half.
__device__ __forceinline__ int half_cols(const Layout &L, int cols) {
  if (!L.paired) return cols;
  const int c = cols - 2048 * L.h;
  return c < 0 ? 0 : (c > 2048 ? 2048 : c);
}

// x + the partner wave's x (same lane).
__device__ __forceinline__ float pair_sum(float x, uint8_t *mine, const uint8_t *other, int lane) {
  reinterpret_cast<float *>(mine + lane * kPairLaneBytes)[kEPL] = x;
  __syncthreads();
  x += reinterpret_cast<const float *>(other + lane * kPairLaneBytes)[kEPL];
  __syncthreads();
  return x;
}

// ---------------------------------------------------------------- memory

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load marked non-temporal: data streamed once (input rows, packed
// records) need not stay in the caches, which keeps HBM reads flowing at a
// higher rate when every lane reads whole cache lines with its neighbours.
__device__ __forceinline__ uint4 load_nt16(const void *p) {
  const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4 *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Raw buffer resource over `bytes` bytes from p (no stride; word 3 selects
// 32-bit data, as buffer accesses on gfx9 require).  The hardware checks each
// access against the size: a load at an offset >= bytes returns zero and a
// store there is dropped.  The d = 128 encoder and score kernels address each
// group of rows or keys through one, so that the last, ragged group needs no
// per-lane branches: a store under a divergent branch makes the compiler wait
// for every outstanding store before the next prefetched load may be used
// (loads and stores share one completion counter).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, bytes, 0x00020000);
}

// 16 bytes at byte offset off, non-temporal.
__device__ __forceinline__ uint4 load16_rsrc_nt(__amdgpu_buffer_rsrc_t r, int off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float load_f32_rsrc(__amdgpu_buffer_rsrc_t r, int off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

__device__ __forceinline__ void store_f32_rsrc(float v, __amdgpu_buffer_rsrc_t r, int off) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
}

// W consecutive words at byte offset off (W = 1..4, one store).
template <int W>
__device__ __forceinline__ void store_words_rsrc(const uint32_t (&w)[W], __amdgpu_buffer_rsrc_t r, int off) {
  if constexpr (W == 1) {
    __builtin_amdgcn_raw_buffer_store_b32(w[0], r, off, 0, 0);
  } else if constexpr (W == 2) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{w[0], w[1]}, r, off, 0, 0);
  } else if constexpr (W == 3) {
    typedef unsigned int u32x3 __attribute__((ext_vector_type(3)));
    __builtin_amdgcn_raw_buffer_store_b96(u32x3{w[0], w[1], w[2]}, r, off, 0, 0);
  } else {
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{w[0], w[1], w[2], w[3]}, r, off, 0, 0);
  }
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// 16 bytes from p straight into LDS, non-temporal: the wave's 64 lanes fill
// the 1 KiB at lds_base in lane order (lane l at lds_base + 16 l).  lds_base
// must be the same on every lane.  Completion is tracked like a load
// (vmcnt), not like an LDS access.
__device__ __forceinline__ void load_lds16_nt(const void *p, void *lds_base) {
  __builtin_amdgcn_global_load_lds((glb_void_t *)p, (lds_void_t *)lds_base, 16, 0, 2);
}

// ---------------------------------------------------------------- block rotations

// In place on the lane's 32 contiguous coordinates, with the lane's 32
// rotation parameters rc (TQ_ROT_GIVENS: 16 pairs of (cos, sin);
// TQ_ROT_QUAT: 8 unit quaternions (w, x, y, z)).  INV applies the transpose.
template <int ROT, bool INV>
__device__ __forceinline__ void rotate_blocks(float (&v)[kEPL], const float (&rc)[kEPL]) {
  if constexpr (ROT == TQ_ROT_GIVENS) {
#pragma unroll
    for (int p = 0; p < kEPL / 2; ++p) {
      const float c = rc[2 * p], s = INV ? -rc[2 * p + 1] : rc[2 * p + 1];
      const float v0 = v[2 * p], v1 = v[2 * p + 1];
      v[2 * p] = fmaf(c, v0, -s * v1);
      v[2 * p + 1] = fmaf(s, v0, c * v1);
    }
  } else if constexpr (ROT == TQ_ROT_QUAT) {
#pragma unroll
    for (int k = 0; k < kEPL / 4; ++k) {
      // p * v with p = (w, x, y, z); the transpose is the product with the
      // conjugate (w, -x, -y, -z)
      const float w = rc[4 * k];
      const float x = INV ? -rc[4 * k + 1] : rc[4 * k + 1];
      const float y = INV ? -rc[4 * k + 2] : rc[4 * k + 2];
      const float z = INV ? -rc[4 * k + 3] : rc[4 * k + 3];
      const float a = v[4 * k], b = v[4 * k + 1], c = v[4 * k + 2], d = v[4 * k + 3];
      v[4 * k] = w * a - x * b - y * c - z * d;
      v[4 * k + 1] = x * a + w * b - z * c + y * d;
      v[4 * k + 2] = y * a + z * b + w * c - x * d;
      v[4 * k + 3] = z * a - y * b + x * c + w * d;
    }
  }
}

// ---------------------------------------------------------------- misc

// Non-finite rows: a vector whose float32 sum of squares ss is NaN or
// infinite (it holds a NaN or an infinity, or its squares overflow) is
// encoded as the zero vector, and its norm is stored as NaN.  Returns
// whether this lane's vector is such a row; when any lane of the wave has
// one (rare: one wave-uniform branch otherwise), its coordinates and ss are
// set to zero.  v may be the raw coordinates or any linear transform of them.
template <int N>
__device__ __forceinline__ bool zero_if_nonfinite(float (&v)[N], float &ss) {
  const bool bad = !(ss <= 3.402823466e38f);
  if (__builtin_amdgcn_ballot_w64(bad) != 0) {
#pragma unroll
    for (int e = 0; e < N; ++e) v[e] = bad ? 0.0f : v[e];
    ss = bad ? 0.0f : ss;
  }
  return bad;
}

// w <- 2 w + b: append one bit below the ones already present.
__device__ __forceinline__ uint32_t append_bit(uint32_t w, bool b) {
  return w + w + (b ? 1u : 0u);
}

// w <- 2 w + (bit `lane` of the wave mask m): one v_addc with the mask as
// carry-in.  Masks come from __builtin_amdgcn_ballot_w64 of compares and
// are combined with 64-bit scalar logic, so a code bit costs one VALU op.
__device__ __forceinline__ uint32_t append_mask(uint32_t w, uint64_t m) {
  uint32_t r;
  uint64_t carry_out;
  asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(r), "=s"(carry_out) : "v"(w), "s"(m));
  return r;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xFFFFu)));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
}

// Orders LDS traffic between the lanes of one wave (regions private to a
// wave need no workgroup barrier).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}


// ---------------------------------------------------------------- rows

// A row-major matrix of `n` rows, `cols` used columns, row stride `ld`
// elements of type `dtype` (TQ_F32, TQ_F16 or TQ_BF16).
struct RowSpan {
  const void *p;
  int64_t ld;
  int64_t n;
  int32_t cols;
  int32_t dtype;
};

__device__ __forceinline__ float load_elem(const RowSpan &r, int64_t off) {
  if (r.dtype == TQ_F32) return static_cast<const float *>(r.p)[off];
  const uint16_t h = static_cast<const uint16_t *>(r.p)[off];
  return (r.dtype == TQ_BF16) ? __uint_as_float(static_cast<uint32_t>(h) << 16)
                              : static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// Coordinates [32 sub, 32 sub + 32) of row `row`, zero beyond `cols` and for
// rows >= n, one element load each (any alignment).
__device__ __forceinline__ void load_rows_direct(const RowSpan &r, int64_t row, int sub,
                                                 float (&xv)[kEPL]) {
#pragma unroll
  for (int e = 0; e < kEPL; ++e) {
    const int j = sub * kEPL + e;
    xv[e] = (row < r.n && j < r.cols) ? load_elem(r, row * r.ld + j) : 0.0f;
  }
}

// Coalesced path for rows whose used part is a whole number of 16-byte
// chunks and 16-byte aligned: the wave's 64 >> log_lpv rows starting at
// base_row are read as 16-byte chunks spread over all 64 lanes, written to a
// wave-private LDS region at the owning lane's segment (32 elements + 16
// bytes of padding, so the read-back is free of bank conflicts), then each
// lane reads its 32 coordinates.  Coordinates >= cols are left unspecified;
// rows >= n read as zero.
__device__ __forceinline__ void load_rows_staged(const RowSpan &r, int64_t base_row, int log_lpv,
                                                 int lane, uint8_t *stage, float (&xv)[kEPL]) {
  const int esize = (r.dtype == TQ_F32) ? 4 : 2;
  const int seg = kEPL * esize + 16;
  const int lane_shift = (esize == 4) ? 7 : 6;          // log2(32 * esize)
  const int cpr = (r.cols * esize) >> 4;                 // 16-byte chunks per row
  const int vpw = 64 >> log_lpv;
  const int total = vpw * cpr;
  const float rcp_cpr = 1.0f / static_cast<float>(cpr);
  const uint8_t *xb = static_cast<const uint8_t *>(r.p);
  const int64_t row_bytes = r.ld * esize;
  for (int f = lane; f < total; f += 64) {
    const int v = __float2int_rz((static_cast<float>(f) + 0.5f) * rcp_cpr);
    const int c = f - v * cpr;
    const int64_t row = base_row + v;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (row < r.n) val = load_nt16(xb + row * row_bytes + (c << 4));
    const int byte = c << 4;
    const int s = byte >> lane_shift;
    const int inner = byte & ((1 << lane_shift) - 1);
    *reinterpret_cast<uint4 *>(stage + ((v << log_lpv) + s) * seg + inner) = val;
  }
  wave_lds_sync();
  const uint4 *src = reinterpret_cast<const uint4 *>(stage + lane * seg);
  if (esize == 4) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint4 w = src[q];
      xv[4 * q + 0] = __uint_as_float(w.x);
      xv[4 * q + 1] = __uint_as_float(w.y);
      xv[4 * q + 2] = __uint_as_float(w.z);
      xv[4 * q + 3] = __uint_as_float(w.w);
    }
  } else if (r.dtype == TQ_BF16) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 w = src[q];
      xv[8 * q + 0] = bf16_lo(w.x); xv[8 * q + 1] = bf16_hi(w.x);
      xv[8 * q + 2] = bf16_lo(w.y); xv[8 * q + 3] = bf16_hi(w.y);
      xv[8 * q + 4] = bf16_lo(w.z); xv[8 * q + 5] = bf16_hi(w.z);
      xv[8 * q + 6] = bf16_lo(w.w); xv[8 * q + 7] = bf16_hi(w.w);
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 w = src[q];
      xv[8 * q + 0] = f16_lo(w.x); xv[8 * q + 1] = f16_hi(w.x);
      xv[8 * q + 2] = f16_lo(w.y); xv[8 * q + 3] = f16_hi(w.y);
      xv[8 * q + 4] = f16_lo(w.z); xv[8 * q + 5] = f16_hi(w.z);
      xv[8 * q + 6] = f16_lo(w.w); xv[8 * q + 7] = f16_hi(w.w);
    }
  }
  wave_lds_sync();
}

// Stores coordinates [32 sub, 32 sub + 32) of float32 rows, first `cols`
// only, one element store each.
__device__ __forceinline__ void store_rows_direct(float *out, int64_t ld, int64_t n, int cols,
                                                  int64_t row, int sub, const float (&v)[kEPL]) {
  if (row >= n) return;
#pragma unroll
  for (int e = 0; e < kEPL; ++e) {
    const int j = sub * kEPL + e;
    if (j < cols) out[row * ld + j] = v[e];
  }
}

// Reverse of load_rows_staged for float32 output rows: lanes write their 32
// coordinates to LDS, then the wave stores whole 16-byte chunks of the used
// columns with consecutive lanes on consecutive addresses.
__device__ __forceinline__ void store_rows_staged(float *out, int64_t ld, int64_t n, int cols,
                                                  int64_t base_row, int log_lpv, int lane,
                                                  uint8_t *stage, const float (&v)[kEPL]) {
  const int seg = kEPL * 4 + 16;
  uint4 *dst = reinterpret_cast<uint4 *>(stage + lane * seg);
#pragma unroll
  for (int q = 0; q < 8; ++q)
    dst[q] = make_uint4(__float_as_uint(v[4 * q]), __float_as_uint(v[4 * q + 1]),
                        __float_as_uint(v[4 * q + 2]), __float_as_uint(v[4 * q + 3]));
  wave_lds_sync();
  const int cpr = (cols * 4) >> 4;
  const int vpw = 64 >> log_lpv;
  const int total = vpw * cpr;
  const float rcp_cpr = 1.0f / static_cast<float>(cpr);
  uint8_t *ob = reinterpret_cast<uint8_t *>(out);
  for (int f = lane; f < total; f += 64) {
    const int rv = __float2int_rz((static_cast<float>(f) + 0.5f) * rcp_cpr);
    const int c = f - rv * cpr;
    const int64_t row = base_row + rv;
    const int byte = c << 4;
    const uint4 val = *reinterpret_cast<const uint4 *>(stage + ((rv << log_lpv) + (byte >> 7)) * seg + (byte & 127));
    if (row < n) *reinterpret_cast<uint4 *>(ob + row * ld * 4 + byte) = val;
  }
  wave_lds_sync();
}

}  // namespace tq
