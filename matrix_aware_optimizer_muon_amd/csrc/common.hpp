// Shared device helpers for the Muon kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muon {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Storage type tags.  16-bit values are kept as raw uint16_t in memory.
struct BF16 {};
struct F16 {};
struct F32 {};

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// fp32 -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// fp32 -> fp16, round to nearest even (hardware conversion).
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;
  return __builtin_bit_cast(uint16_t, h);
}

template <typename T> struct Store;
template <> struct Store<BF16> {
  typedef uint16_t type;
  static __device__ __forceinline__ uint16_t from(float f) { return f32_to_bf16_bits(f); }
};
template <> struct Store<F16> {
  typedef uint16_t type;
  static __device__ __forceinline__ uint16_t from(float f) { return f32_to_f16_bits(f); }
};
template <> struct Store<F32> {
  typedef float type;
  static __device__ __forceinline__ float from(float f) { return f; }
};

// Map a linear workgroup id so that consecutive logical ids land on the same
// XCD.  The hardware dispatches workgroup w to XCD (w mod 8); tiles that share
// operand panels should share that XCD's L2.  Bijective for any total.
__host__ __device__ __forceinline__ uint32_t xcd_remap(uint32_t bid, uint32_t total) {
  const uint32_t nx = 8;
  uint32_t x = bid % nx, slot = bid / nx;
  uint32_t q = total / nx, rem = total % nx;
  return x * q + (x < rem ? x : rem) + slot;
}

// Workgroup -> tile id in runs of C per XCD: XCD x takes tiles
// [k 8C + x C, k 8C + x C + C) in its k-th run, so at any time the eight XCDs
// work inside one window of 8C consecutive tiles (operands that the shared
// last-level cache can hold) while each XCD's own workgroups still take
// consecutive tiles (operand panels shared in its L2).  Tiles past the last
// whole window are split as in xcd_remap.  A bijection on [0, total) for any
// C > 0.
__host__ __device__ __forceinline__ uint32_t xcd_remap_chunked(uint32_t bid, uint32_t total,
                                                             uint32_t C) {
  const uint32_t nx = 8;
  const uint32_t x = bid % nx, slot = bid / nx;
  const uint32_t span = nx * C, full = total / span;
  if (slot / C < full) return (slot / C) * span + x * C + slot % C;
  const uint32_t base = full * span;
  return base + xcd_remap(bid - base, total - base);
}

// Tile traversal orders.  Consecutive tile ids run concurrently on one XCD
// (after xcd_remap), so the order decides how many operand panels the ~32
// tiles in flight there share through its L2.
//
// Full grid: groups of GH tile rows (8 by default), column by column inside a
// group, so 32 consecutive tiles cover 8 rows x 4 columns (12 operand panels)
// instead of one row x 32 columns (33 panels) as in row-major order.
__host__ __device__ __forceinline__ void full_tile_grouped(int t, int tiles_m, int tiles_n, int GH, int* ti,
                                                  int* tj) {
  const int g = t / (GH * tiles_n);
  const int u = t - g * GH * tiles_n;
  const int h = GH < tiles_m - g * GH ? GH : tiles_m - g * GH;
  *ti = g * GH + u % h;
  *tj = u / h;
}

// Lower-triangular grid (T x T tiles, I >= J): super-rows of SH tile rows (4
// by default), walked column by column; the diagonal block of a super-row
// comes last.
__host__ __device__ __forceinline__ void tri_tile_grouped(int t, int T, int SH, int* ti, int* tj) {
  // tiles before super-row s: (SH s)(SH s + 1)/2
  int s = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f) / SH;
  while (s > 0 && (SH * s) * (SH * s + 1) / 2 > t) --s;
  while ((SH * (s + 1)) * (SH * (s + 1) + 1) / 2 <= t && SH * (s + 1) < T) ++s;
  int u = t - (SH * s) * (SH * s + 1) / 2;
  const int h = SH < T - SH * s ? SH : T - SH * s;
  const int r0 = SH * s;
  if (u < h * r0) {
    *tj = u / h;
    *ti = r0 + u % h;
    return;
  }
  u -= h * r0;
  int d = 0;
  while (u >= h - d) {
    u -= h - d;
    ++d;
  }
  *tj = r0 + d;
  *ti = r0 + d + u;
}

// Streaming (non-temporal) 16-byte global access for data touched once per
// step (M, G, W, the X0 copies): keeps it from displacing reusable lines.
// gfx950 transposing LDS read of 16-bit elements (ds_read_b64_tr_b16): in
// each group of 16 lanes, lane 4e + i/4 of the group supplies the 64-bit row
// whose element i % 4 lane i receives as its element e.  With lane i
// addressing row i / 4 and columns 4 (i % 4) .. +3 of a 4 x 16 block of a
// row-major (k, n) tile, lane i receives column i of the block's 4 rows:
// four consecutive k of one n.  p must point into LDS.
typedef __attribute__((__vector_size__(4 * sizeof(__fp16)))) __fp16 fp16x4_t;
__device__ __forceinline__ uint2 tr_read(const char* p) {
  typedef __attribute__((address_space(3))) fp16x4_t lds_fp16x4;
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4*)p));
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 nt_load4(const float* p) {
  const f32x4 v = __builtin_nontemporal_load((const f32x4*)p);
  return make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void nt_store4(float* p, float4 v) {
  const f32x4 x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, (f32x4*)p);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

}  // namespace muon
