// HBM bandwidth probes for gfx950 (measurement only; not part of the
// quantiser's C ABI).  Three streaming patterns of known byte counts give the
// rates the memory system reaches for a pure read stream, a pure write
// stream, and a stream that reads IN and writes OUT bytes per unit -- the
// traffic mix of a decode that reads a packed record and writes a float32
// row.  Every lane moves whole 16-byte chunks, consecutive lanes on
// consecutive addresses; what is written depends on what was read, so no
// load can be dropped.  The write and mixed probes come in two launch
// shapes: persistent workgroups striding over the buffer, and one-shot
// workgroups that each move one span and exit.  A further probe measures how the SIMD overlaps
// matrix-core work with ordinary vector work.  Built into libtqprobe.so,
// loaded by the benchmark.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

__global__ void __launch_bounds__(kThreads) read_kernel(const u32x4 *p, int64_t chunks, uint32_t *sink) {
  uint32_t acc = 0;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < chunks; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // a store that never happens for the data the probes use, but that the
  // compiler cannot rule out
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

__global__ void __launch_bounds__(kThreads) write_kernel(u32x4 *p, int64_t chunks, uint32_t seed) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < chunks; i += stride) {
    const uint32_t s = seed ^ static_cast<uint32_t>(i);
    p[i] = u32x4{s, s + 1u, s + 2u, s + 3u};
  }
}

// Units in groups of 16 per wave: the group's 16 * IN input bytes are read
// as IN/64 16-byte chunks per lane and its 16 * OUT output bytes written as
// OUT/64 chunks per lane.  IN and OUT are multiples of 64.  ROWS = false:
// each store instruction writes 1 KiB of consecutive bytes (whole 128-byte
// lines); ROWS = true: 64 bytes of each of the 16 units' rows (four lanes per
// row), the pattern of a kernel that keeps four lanes per output row.
template <bool ROWS>
__global__ void __launch_bounds__(kThreads) mixed_kernel(const u32x4 *in, u32x4 *out, int64_t groups, int in_ch,
                                                         int out_ch) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  const int64_t waves = static_cast<int64_t>(gridDim.x) * (kThreads / 64);
  for (int64_t g = wave; g < groups; g += waves) {
    const u32x4 *src = in + g * 64 * in_ch;
    u32x4 *dst = out + g * 64 * out_ch;
    uint32_t acc = 0;
    for (int k = 0; k < in_ch; ++k) {
      const u32x4 v = __builtin_nontemporal_load(src + k * 64 + lane);
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    for (int k = 0; k < out_ch; ++k) {
      const int64_t at = ROWS ? (lane >> 2) * (4 * out_ch) + 4 * k + (lane & 3) : k * 64 + lane;
      dst[at] = u32x4{acc, acc ^ 1u, acc ^ 2u, static_cast<uint32_t>(k)};
    }
  }
}

// One-shot forms of the write and mixed probes: no workgroup loops.  The
// write probe has each thread store one 16-byte chunk.  The mixed probe gives
// each wave of a 16-wave workgroup one group of 16 units and deals the
// workgroup's 1 KiB pieces out in turn: piece k of wave w of workgroup b is
// piece (16 k + w) of the workgroup's span, on the input side as on the
// output side, so the k-th loads and stores of all its waves cover
// consecutive KiB.  Workgroups then retire in about the order they were
// dispatched, and the memory system sees a window of addresses that moves
// forward.
constexpr int kOneShotWaves = 16;

__global__ void __launch_bounds__(kThreads) write_once_kernel(u32x4 *p, int64_t chunks, uint32_t seed) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i < chunks) {
    const uint32_t s = seed ^ static_cast<uint32_t>(i);
    p[i] = u32x4{s, s + 1u, s + 2u, s + 3u};
  }
}

__global__ void __launch_bounds__(kOneShotWaves * 64) mixed_once_kernel(const u32x4 *in, u32x4 *out, int64_t groups,
                                                                        int in_ch, int out_ch) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int64_t g0 = static_cast<int64_t>(blockIdx.x) * kOneShotWaves;    // the workgroup's first group
  if (g0 + w >= groups) return;
  // the span's pieces past the last group are never touched: with fewer than
  // 16 groups left, piece 16 k + w of a live wave w can still lie beyond them,
  // so the last workgroup falls back to whole groups per wave
  const bool full = g0 + kOneShotWaves <= groups;
  uint32_t acc = 0;
  for (int k = 0; k < in_ch; ++k) {
    const int64_t piece = full ? g0 * in_ch + k * kOneShotWaves + w : (g0 + w) * in_ch + k;
    const u32x4 v = __builtin_nontemporal_load(in + piece * 64 + lane);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  for (int k = 0; k < out_ch; ++k) {
    const int64_t piece = full ? g0 * out_ch + k * kOneShotWaves + w : (g0 + w) * out_ch + k;
    out[piece * 64 + lane] = u32x4{acc, acc ^ 1u, acc ^ 2u, static_cast<uint32_t>(k)};
  }
}

// Issue probe: every wave loops `iters` times over a fixed body.  MODE 0:
// four independent v_mfma_f32_16x16x32_f16 chains; 1: 64 v_fma_f32 over
// eight independent registers; 2: both in every wave.  MODE 2's time
// against MODES 0 and 1 shows how much of the matrix-core work the SIMD
// overlaps with vector work of the same wave.
// out[blockIdx.x * 256 + threadIdx.x] receives each thread's sums.
template <int MODE>
__global__ void __launch_bounds__(kThreads) issue_kernel(float *out, int iters) {
  typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  f16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<_Float16>(threadIdx.x * 0.001f + i);
    b[i] = static_cast<_Float16>(i * 0.5f);
  }
  f32x4 acc[4];
  for (int k = 0; k < 4; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  float v[8];
  for (int k = 0; k < 8; ++k) v[k] = threadIdx.x * 0.01f + k;
  constexpr bool do_m = MODE == 0 || MODE == 2;
  constexpr bool do_v = MODE == 1 || MODE == 2;
  for (int it = 0; it < iters; ++it) {
    if constexpr (do_m) {
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[k], 0, 0, 0);
    }
    if constexpr (do_v) {
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = fmaf(v[k], 1.0000001f, 0.5f);
    }
  }
  float s = 0.f;
  for (int k = 0; k < 4; ++k) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
  for (int k = 0; k < 8; ++k) s += v[k];
  out[static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x] = s;
}

int64_t grid_blocks(int64_t work_items, int64_t per_block) {
  const int64_t need = (work_items + per_block - 1) / per_block;
  const int64_t cap = 256 * 16;   // 16 workgroups per CU
  return need < 1 ? 1 : (need < cap ? need : cap);
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16, 16-byte aligned) from p.  sink: device,
// >= 4096 words, written only in a case the probes never produce.
// Returns 0 or a hipError_t value.
int tqp_read(const void *p, int64_t bytes, void *sink, void *stream) {
  if (!p || !sink || bytes < 0 || (bytes & 15) || (reinterpret_cast<uintptr_t>(p) & 15)) return hipErrorInvalidValue;
  (void)hipGetLastError();
  const int64_t chunks = bytes >> 4;
  hipLaunchKernelGGL(read_kernel, dim3(grid_blocks(chunks, kThreads)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4 *>(p), chunks,
                     static_cast<uint32_t *>(sink));
  return hipGetLastError();
}

// Writes `bytes` (a multiple of 16, 16-byte aligned) to p.
int tqp_write(void *p, int64_t bytes, uint32_t seed, void *stream) {
  if (!p || bytes < 0 || (bytes & 15) || (reinterpret_cast<uintptr_t>(p) & 15)) return hipErrorInvalidValue;
  (void)hipGetLastError();
  const int64_t chunks = bytes >> 4;
  hipLaunchKernelGGL(write_kernel, dim3(grid_blocks(chunks, kThreads)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<u32x4 *>(p), chunks, seed);
  return hipGetLastError();
}

// For `units` units (a multiple of 16): reads in_bytes and writes out_bytes
// per unit (each a multiple of 64, 1..4096), from `in` [units][in_bytes]
// to `out` [units][out_bytes] (16-byte aligned).  rows = 0: whole-line
// stores; rows = 1: 64 bytes of 16 rows per store instruction.
int tqp_mixed(const void *in, int64_t in_bytes, void *out, int64_t out_bytes, int64_t units, int32_t rows,
              void *stream) {
  if (!in || !out || units < 0 || (units & 15) || in_bytes < 64 || out_bytes < 64 || in_bytes > 4096 ||
      out_bytes > 4096 || (in_bytes & 63) || (out_bytes & 63) || (reinterpret_cast<uintptr_t>(in) & 15) ||
      (reinterpret_cast<uintptr_t>(out) & 15))
    return hipErrorInvalidValue;
  (void)hipGetLastError();
  const int64_t groups = units / 16;
  const dim3 grid(grid_blocks(groups, kThreads / 64));
  const int in_ch = static_cast<int>(in_bytes / 64), out_ch = static_cast<int>(out_bytes / 64);
  if (rows) {
    hipLaunchKernelGGL(mixed_kernel<true>, grid, dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4 *>(in), static_cast<u32x4 *>(out), groups, in_ch, out_ch);
  } else {
    hipLaunchKernelGGL(mixed_kernel<false>, grid, dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4 *>(in), static_cast<u32x4 *>(out), groups, in_ch, out_ch);
  }
  return hipGetLastError();
}

// As tqp_write, one-shot: one thread per 16-byte chunk.
int tqp_write_once(void *p, int64_t bytes, uint32_t seed, void *stream) {
  if (!p || bytes < 0 || (bytes & 15) || (reinterpret_cast<uintptr_t>(p) & 15)) return hipErrorInvalidValue;
  (void)hipGetLastError();
  const int64_t chunks = bytes >> 4;
  const int64_t blocks = (chunks + kThreads - 1) / kThreads;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (blocks == 0) return 0;
  hipLaunchKernelGGL(write_once_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<u32x4 *>(p), chunks, seed);
  return hipGetLastError();
}

// As tqp_mixed with whole-line stores, one-shot: one group of 16 units per
// wave, 16-wave workgroups, pieces dealt out in turn (mixed_once_kernel).
int tqp_mixed_once(const void *in, int64_t in_bytes, void *out, int64_t out_bytes, int64_t units, void *stream) {
  if (!in || !out || units < 0 || (units & 15) || in_bytes < 64 || out_bytes < 64 || in_bytes > 4096 ||
      out_bytes > 4096 || (in_bytes & 63) || (out_bytes & 63) || (reinterpret_cast<uintptr_t>(in) & 15) ||
      (reinterpret_cast<uintptr_t>(out) & 15))
    return hipErrorInvalidValue;
  (void)hipGetLastError();
  const int64_t groups = units / 16;
  const int64_t blocks = (groups + kOneShotWaves - 1) / kOneShotWaves;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (blocks == 0) return 0;
  const int in_ch = static_cast<int>(in_bytes / 64), out_ch = static_cast<int>(out_bytes / 64);
  hipLaunchKernelGGL(mixed_once_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kOneShotWaves * 64), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4 *>(in), static_cast<u32x4 *>(out),
                     groups, in_ch, out_ch);
  return hipGetLastError();
}

// Issue probe (see issue_kernel): mode 0..2, `blocks` workgroups of 256
// threads, `iters` loop trips; out: device, blocks * 256 floats.
int tqp_issue(int32_t mode, void *out, int32_t blocks, int32_t iters, void *stream) {
  if (!out || blocks < 1 || blocks > 65536 || iters < 0 || mode < 0 || mode > 2) return hipErrorInvalidValue;
  (void)hipGetLastError();
  float *o = static_cast<float *>(out);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (mode) {
    case 0: hipLaunchKernelGGL(issue_kernel<0>, dim3(blocks), dim3(kThreads), 0, s, o, iters); break;
    case 1: hipLaunchKernelGGL(issue_kernel<1>, dim3(blocks), dim3(kThreads), 0, s, o, iters); break;
    default: hipLaunchKernelGGL(issue_kernel<2>, dim3(blocks), dim3(kThreads), 0, s, o, iters); break;
  }
  return hipGetLastError();
}

}  // extern "C"
