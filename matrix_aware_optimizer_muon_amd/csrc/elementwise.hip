// Memory-bound kernels of the Muon and periodic-RowNorm steps.
//
// prep:       M <- mu M + G ("Infra Optimizers" eq. (1)); U = mu M + G
//             (Nesterov remark); partial sums of ||U||_F^2; U stored in the
//             Newton-Schulz operand type both as is and transposed through
//             LDS, zero padded to the GEMM tile: one copy is X0 = O(U)
//             ("Scaling Muon for DiT" 3.1), the other X0^T.  When the
//             products read X0 across K the transposed copy is left out and
//             a row-tiled variant streams U in the natural layout only.  One
//             read of M and G, one write of M and of the copies.
// finalize:   deterministic (fixed order, fp64) reduction of the partial sums
//             to 1/||U||_F per matrix (0 when the norm is 0, NaN when the sum
//             is NaN or infinite).
// rownorm:    the same M update and U, then R_eps over the r oriented rows
//             ("Scaling Muon for DiT" 3.1) and the decayed, scaled update of W
//             ("Infra Optimizers" eq. (4)).  m <= n: one workgroup per row,
//             one pass.  m > n: the rows of O(U) are columns of U, so a column
//             sum-of-squares pass, a fixed-order finalize and an apply pass.
#include "common.hpp"
#include "kernels.h"

namespace muon {

// ---------------------------------------------------------------------------
// Four consecutive elements of M (fp32) and G (fp32 or bf16), vector or
// bounds-checked scalar access.
template <bool GBF16>
__device__ __forceinline__ float4 load_g4(const void* G, size_t idx, bool vec, int valid) {
  float4 g = make_float4(0.f, 0.f, 0.f, 0.f);
  if (GBF16) {
    const uint16_t* g16 = (const uint16_t*)G + idx;
    if (vec) {
      const uint2 u = *(const uint2*)g16;
      g.x = __uint_as_float(u.x << 16);
      g.y = __uint_as_float(u.x & 0xffff0000u);
      g.z = __uint_as_float(u.y << 16);
      g.w = __uint_as_float(u.y & 0xffff0000u);
    } else {
      if (valid > 0) g.x = bf16_bits_to_f32(g16[0]);
      if (valid > 1) g.y = bf16_bits_to_f32(g16[1]);
      if (valid > 2) g.z = bf16_bits_to_f32(g16[2]);
      if (valid > 3) g.w = bf16_bits_to_f32(g16[3]);
    }
  } else {
    const float* g32 = (const float*)G + idx;
    if (vec) {
      g = *(const float4*)g32;
    } else {
      if (valid > 0) g.x = g32[0];
      if (valid > 1) g.y = g32[1];
      if (valid > 2) g.z = g32[2];
      if (valid > 3) g.w = g32[3];
    }
  }
  return g;
}

__device__ __forceinline__ float4 load_f4(const float* p, bool vec, int valid) {
  if (vec) return nt_load4(p);
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (valid > 0) v.x = p[0];
  if (valid > 1) v.y = p[1];
  if (valid > 2) v.z = p[2];
  if (valid > 3) v.w = p[3];
  return v;
}

__device__ __forceinline__ void store_f4(float* p, float4 v, bool vec, int valid) {
  if (vec) {
    nt_store4(p, v);
    return;
  }
  if (valid > 0) p[0] = v.x;
  if (valid > 1) p[1] = v.y;
  if (valid > 2) p[2] = v.z;
  if (valid > 3) p[3] = v.w;
}

// M' = mu M + G (stored), returns U = mu M' + G (or M' without Nesterov).
__device__ __forceinline__ float4 momentum4(float4 m, float4 g, float mu, int nesterov,
                                            float4* mnew) {
  float4 mn;
  mn.x = mu * m.x + g.x;
  mn.y = mu * m.y + g.y;
  mn.z = mu * m.z + g.z;
  mn.w = mu * m.w + g.w;
  *mnew = mn;
  if (!nesterov) return mn;
  return make_float4(mu * mn.x + g.x, mu * mn.y + g.y, mu * mn.z + g.z, mu * mn.w + g.w);
}

template <int BS>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < BS / 64; ++w) s += red[w];
  return s;
}

// ---------------------------------------------------------------------------
// prep: one 64 x 64 tile of U (rows i < m, cols j < n; zero in the padding)
// per workgroup.  U is written twice in the operand type: in its natural
// layout (m_pad x n_pad) and transposed through LDS (n_pad x m_pad), so that
// X0 = O(U) and X0^T are both available K-contiguous to the GEMMs.  Tiles
// are walked down the columns (ti fastest), so that neighbouring workgroups
// extend the same rows of the transposed copy (measured 2-4 % faster than
// the row-major walk).
template <bool GBF16, bool XF32>
__global__ void __launch_bounds__(256) prep_tile_kernel(const PrepParams p, int vec) {
  __shared__ float tile[64][65];
  __shared__ float red[4];
  const int ib = p.m_pad / 64, jb = p.n_pad / 64;
  const int per_mat = ib * jb;
  const int mat = blockIdx.x / per_mat;
  const int bl = blockIdx.x - mat * per_mat;
  const int tj = bl / ib, ti = bl - tj * ib;
  const MatPtrs mp = p.table[mat];
  const int t = threadIdx.x;
  const size_t xbase = (size_t)mat * p.x_stride;
  float ss = 0.f;
  {
    const int c4 = (t & 15) * 4;
    const int j = tj * 64 + c4;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int rl = (t >> 4) + 16 * q;
      const int i = ti * 64 + rl;
      float4 u = make_float4(0.f, 0.f, 0.f, 0.f);
      if (i < p.m && j < p.n) {
        const int valid = p.n - j;
        const size_t idx = (size_t)i * p.n + j;
        const bool v4 = vec && valid >= 4;
        const float4 m = load_f4(mp.M + idx, v4, valid);
        const float4 g = load_g4<GBF16>(mp.G, idx, v4, valid);
        float4 mn;
        u = momentum4(m, g, p.mu, p.nesterov, &mn);
        store_f4(mp.M + idx, mn, v4, valid);
        if (valid < 4) {  // keep the padding exactly zero
          if (valid < 2) u.y = 0.f;
          if (valid < 3) u.z = 0.f;
          u.w = 0.f;
        }
        ss += u.x * u.x + u.y * u.y + u.z * u.z + u.w * u.w;
      }
      const size_t xo = xbase + (size_t)i * p.n_pad + j;
      if (XF32) {
        nt_store4((float*)p.X + xo, u);
      } else {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 pk = {(uint32_t)f32_to_bf16_bits(u.x) | ((uint32_t)f32_to_bf16_bits(u.y) << 16),
                          (uint32_t)f32_to_bf16_bits(u.z) | ((uint32_t)f32_to_bf16_bits(u.w) << 16)};
        __builtin_nontemporal_store(pk, (u32x2*)((uint16_t*)p.X + xo));
      }
      if (p.XT) {
        tile[rl][c4 + 0] = u.x;
        tile[rl][c4 + 1] = u.y;
        tile[rl][c4 + 2] = u.z;
        tile[rl][c4 + 3] = u.w;
      }
    }
  }
  if (p.XT) {  // (uniform) the transposed copy, unless the products read U across K
    __syncthreads();
    {
      const int jl = t >> 2;        // transposed row within the tile
      const int i0 = (t & 3) * 16;  // 16 consecutive transposed columns
      const size_t xo = xbase + (size_t)(tj * 64 + jl) * p.m_pad + ti * 64 + i0;
      if (XF32) {
        float* xp = (float*)p.XT + xo;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          nt_store4(xp + 4 * q, make_float4(tile[i0 + 4 * q][jl], tile[i0 + 4 * q + 1][jl],
                                            tile[i0 + 4 * q + 2][jl], tile[i0 + 4 * q + 3][jl]));
      } else {
        uint32_t w[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
          w[q] = (uint32_t)f32_to_bf16_bits(tile[i0 + 2 * q][jl]) |
                 ((uint32_t)f32_to_bf16_bits(tile[i0 + 2 * q + 1][jl]) << 16);
        u32x4* xp = (u32x4*)((uint16_t*)p.XT + xo);
        __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]}, xp);
        __builtin_nontemporal_store(u32x4{w[4], w[5], w[6], w[7]}, xp + 1);
      }
    }
  }
  const float tot = block_sum<256>(ss, red);
  if (threadIdx.x == 0) p.partials[(size_t)mat * p.blocks_per_mat + bl] = tot;
}

__global__ void __launch_bounds__(256) norm_finalize_kernel(const PrepParams p) {
  __shared__ double red[4];
  const int mat = blockIdx.x;
  const float* part = p.partials + (size_t)mat * p.blocks_per_mat;
  double s = 0.0;
  for (int i = threadIdx.x; i < p.blocks_per_mat; i += 256) s += (double)part[i];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    const double tot = red[0] + red[1] + red[2] + red[3];
    // ||U|| = 0: no direction (pure decay).  A NaN or an infinite sum (a
    // NaN or Inf in U, or squares past fp32's range) gives NaN, so the
    // matrix's direction and weights become NaN as the plain formula's
    // X / ||X|| does, instead of a silently wrong finite step.
    p.inv_norm[mat] = tot == 0.0 ? 0.0f : (tot < INFINITY ? (float)(1.0 / sqrt(tot)) : NAN);
  }
}

// prep with one layout (the products read X0 across K, no transposed copy):
// 8 rows x 512 columns of U per workgroup, each half of the workgroup one row
// segment (2 KB of M, 1 KB of X, 1 or 2 KB of G, all contiguous), the
// workgroups walking along the rows; the four rows of a thread are loaded
// before any is stored.
template <bool GBF16>
__global__ void __launch_bounds__(256) prep_rows_kernel(const PrepParams p, int vec) {
  __shared__ float red[4];
  const int cb = (p.n_pad + 511) / 512;
  const int per_mat = (p.m_pad / 8) * cb;
  const int mat = blockIdx.x / per_mat;
  const int bl = blockIdx.x - mat * per_mat;
  const int rb = bl / cb, c = bl - rb * cb;
  const MatPtrs mp = p.table[mat];
  const int t = threadIdx.x;
  const int j = c * 512 + (t & 127) * 4;
  const size_t xbase = (size_t)mat * p.x_stride;
  const int valid = p.n - j;
  const bool v4 = vec && valid >= 4;
  float ss = 0.f;
  if (j < p.n_pad) {
    float4 m[4], g[4];
    bool in[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = rb * 8 + 2 * q + (t >> 7);
      in[q] = i < p.m && valid > 0;
      const size_t idx = (size_t)i * p.n + j;
      m[q] = in[q] ? load_f4(mp.M + idx, v4, valid) : make_float4(0.f, 0.f, 0.f, 0.f);
      g[q] = in[q] ? load_g4<GBF16>(mp.G, idx, v4, valid) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = rb * 8 + 2 * q + (t >> 7);
      float4 u = make_float4(0.f, 0.f, 0.f, 0.f);
      if (in[q]) {
        float4 mn;
        u = momentum4(m[q], g[q], p.mu, p.nesterov, &mn);
        store_f4(mp.M + (size_t)i * p.n + j, mn, v4, valid);
        if (valid < 4) {  // keep the padding exactly zero
          if (valid < 2) u.y = 0.f;
          if (valid < 3) u.z = 0.f;
          u.w = 0.f;
        }
        ss += u.x * u.x + u.y * u.y + u.z * u.z + u.w * u.w;
      }
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      const u32x2 pk = {(uint32_t)f32_to_bf16_bits(u.x) | ((uint32_t)f32_to_bf16_bits(u.y) << 16),
                        (uint32_t)f32_to_bf16_bits(u.z) | ((uint32_t)f32_to_bf16_bits(u.w) << 16)};
      __builtin_nontemporal_store(pk, (u32x2*)((uint16_t*)p.X + xbase + (size_t)i * p.n_pad + j));
    }
  }
  const float tot = block_sum<256>(ss, red);
  if (t == 0) p.partials[(size_t)mat * p.blocks_per_mat + bl] = tot;
}

int prep_blocks_per_mat(int m_pad, int n_pad, bool rows) {
  return rows ? (m_pad / 8) * ((n_pad + 511) / 512) : (m_pad / 64) * (n_pad / 64);
}

hipError_t launch_prep(const PrepParams& p, int grad_bf16, int x_f32, int nmat, int vec,
                       hipStream_t s) {
  const uint64_t blocks = (uint64_t)nmat * p.blocks_per_mat;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffull || p.m_pad % 64 || p.n_pad % 64) return hipErrorInvalidValue;
  const dim3 g((uint32_t)blocks), b(256);
  if (!p.XT && !x_f32) {
    if (p.blocks_per_mat != prep_blocks_per_mat(p.m_pad, p.n_pad, true)) return hipErrorInvalidValue;
    if (grad_bf16) hipLaunchKernelGGL((prep_rows_kernel<true>), g, b, 0, s, p, vec);
    else hipLaunchKernelGGL((prep_rows_kernel<false>), g, b, 0, s, p, vec);
    return hipGetLastError();
  }
  if (p.blocks_per_mat != prep_blocks_per_mat(p.m_pad, p.n_pad, false)) return hipErrorInvalidValue;
  if (grad_bf16) {
    if (x_f32) hipLaunchKernelGGL((prep_tile_kernel<true, true>), g, b, 0, s, p, vec);
    else hipLaunchKernelGGL((prep_tile_kernel<true, false>), g, b, 0, s, p, vec);
  } else {
    if (x_f32) hipLaunchKernelGGL((prep_tile_kernel<false, true>), g, b, 0, s, p, vec);
    else hipLaunchKernelGGL((prep_tile_kernel<false, false>), g, b, 0, s, p, vec);
  }
  return hipGetLastError();
}

hipError_t launch_norm_finalize(const PrepParams& p, int nmat, hipStream_t s) {
  hipLaunchKernelGGL(norm_finalize_kernel, dim3(nmat), dim3(256), 0, s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// RowNorm, m <= n: one workgroup of NT threads per row.  Every load of the
// row (M, G and W) is issued before the row reduction, so its latency is not
// paid twice; U stays in registers (CH float4 chunks per thread).  Rows wider
// than NT*CH*4 take the generic path that re-reads M' and G (CH == 0).
// max(||row||, eps) of R_eps that keeps a NaN norm (fmaxf would return eps
// and scale the rest of a NaN row by 1/eps).
__device__ __forceinline__ float max_eps(float nrm, float eps) { return nrm < eps ? eps : nrm; }

template <int BS>
__device__ __forceinline__ float block_sum_n(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < BS / 64; ++w) s += red[w];
  return s;
}

template <bool GBF16, int CH, int NT>
__global__ void __launch_bounds__(NT) rownorm_rows_kernel(const RowNormParams p, int vec) {
  __shared__ float red[NT / 64];
  const int mat = blockIdx.x / p.m;
  const int row = blockIdx.x - mat * p.m;
  const MatPtrs mp = p.table[mat];
  const size_t base = (size_t)row * p.n;
  const int nc = (p.n + 3) / 4;
  float ss = 0.f;
  if constexpr (CH > 0) {
    float4 mm[CH], gg[CH], ww[CH];
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int c = threadIdx.x + NT * k;
      if (c < nc) {
        const int col = c * 4, valid = p.n - col;
        const bool v4 = vec && valid >= 4;
        mm[k] = load_f4(mp.M + base + col, v4, valid);
        gg[k] = load_g4<GBF16>(mp.G, base + col, v4, valid);
        ww[k] = load_f4(mp.W + base + col, v4, valid);
      }
    }
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int c = threadIdx.x + NT * k;
      if (c < nc) {
        const int col = c * 4, valid = p.n - col;
        const bool v4 = vec && valid >= 4;
        float4 mn;
        mm[k] = momentum4(mm[k], gg[k], p.mu, p.nesterov, &mn);  // mm now holds U
        store_f4(mp.M + base + col, mn, v4, valid);
        ss += mm[k].x * mm[k].x + mm[k].y * mm[k].y + mm[k].z * mm[k].z + mm[k].w * mm[k].w;
      }
    }
    const float inv = 1.0f / max_eps(sqrtf(block_sum_n<NT>(ss, red)), p.eps);
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int c = threadIdx.x + NT * k;
      if (c < nc) {
        const int col = c * 4, valid = p.n - col;
        const bool v4 = vec && valid >= 4;
        const float4 u = mm[k];
        const float4 r = make_float4(u.x * inv, u.y * inv, u.z * inv, u.w * inv);
        float4 w = ww[k];
        w.x = p.decay * w.x - p.step * r.x;
        w.y = p.decay * w.y - p.step * r.y;
        w.z = p.decay * w.z - p.step * r.z;
        w.w = p.decay * w.w - p.step * r.w;
        store_f4(mp.W + base + col, w, v4, valid);
        if (mp.O) store_f4(mp.O + base + col, r, v4, valid);
      }
    }
  } else {
    for (int c = threadIdx.x; c < nc; c += NT) {
      const int col = c * 4, valid = p.n - col;
      const bool v4 = vec && valid >= 4;
      const float4 m = load_f4(mp.M + base + col, v4, valid);
      const float4 g = load_g4<GBF16>(mp.G, base + col, v4, valid);
      float4 mn;
      const float4 u = momentum4(m, g, p.mu, p.nesterov, &mn);
      store_f4(mp.M + base + col, mn, v4, valid);
      ss += u.x * u.x + u.y * u.y + u.z * u.z + u.w * u.w;
    }
    const float inv = 1.0f / max_eps(sqrtf(block_sum_n<NT>(ss, red)), p.eps);
    // each thread re-reads exactly the chunks it wrote above
    for (int c = threadIdx.x; c < nc; c += NT) {
      const int col = c * 4, valid = p.n - col;
      const bool v4 = vec && valid >= 4;
      const float4 mn = load_f4(mp.M + base + col, v4, valid);
      const float4 g = load_g4<GBF16>(mp.G, base + col, v4, valid);
      const float4 u = p.nesterov ? make_float4(p.mu * mn.x + g.x, p.mu * mn.y + g.y,
                                                p.mu * mn.z + g.z, p.mu * mn.w + g.w)
                                  : mn;
      const float4 r = make_float4(u.x * inv, u.y * inv, u.z * inv, u.w * inv);
      float4 w = load_f4(mp.W + base + col, v4, valid);
      w.x = p.decay * w.x - p.step * r.x;
      w.y = p.decay * w.y - p.step * r.y;
      w.z = p.decay * w.z - p.step * r.z;
      w.w = p.decay * w.w - p.step * r.w;
      store_f4(mp.W + base + col, w, v4, valid);
      if (mp.O) store_f4(mp.O + base + col, r, v4, valid);
    }
  }
}

// RowNorm, m > n.  Pass A: M update and column sums of U^2 over a block of
// RN_ROWS rows (fixed-order partials).  Each thread owns 4 columns.
constexpr int RN_ROWS = 256;

template <bool GBF16>
__global__ void __launch_bounds__(256) rownorm_colsum_kernel(const RowNormParams p, int vec) {
  const int cblocks = (p.n + 1023) / 1024;
  const int per_mat = cblocks * p.row_blocks;
  const int mat = blockIdx.x / per_mat;
  const int bl = blockIdx.x - mat * per_mat;
  const int rb = bl / cblocks, cb = bl - rb * cblocks;
  const MatPtrs mp = p.table[mat];
  const int col = cb * 1024 + threadIdx.x * 4;
  if (col >= p.n) return;
  const int valid = p.n - col;
  const bool v4 = vec && valid >= 4;
  float4 ss = make_float4(0.f, 0.f, 0.f, 0.f);
  const int r0 = rb * RN_ROWS, r1 = min(p.m, r0 + RN_ROWS);
  constexpr int UR = 4;  // rows per iteration (loads in flight)
  int row = r0;
  for (; row + UR <= r1; row += UR) {
    float4 m[UR], g[UR];
#pragma unroll
    for (int q = 0; q < UR; ++q) {
      const size_t idx = (size_t)(row + q) * p.n + col;
      m[q] = load_f4(mp.M + idx, v4, valid);
      g[q] = load_g4<GBF16>(mp.G, idx, v4, valid);
    }
#pragma unroll
    for (int q = 0; q < UR; ++q) {
      float4 mn;
      const float4 u = momentum4(m[q], g[q], p.mu, p.nesterov, &mn);
      store_f4(mp.M + (size_t)(row + q) * p.n + col, mn, v4, valid);
      ss.x += u.x * u.x;
      ss.y += u.y * u.y;
      ss.z += u.z * u.z;
      ss.w += u.w * u.w;
    }
  }
  for (; row < r1; ++row) {
    const size_t idx = (size_t)row * p.n + col;
    const float4 m = load_f4(mp.M + idx, v4, valid);
    const float4 g = load_g4<GBF16>(mp.G, idx, v4, valid);
    float4 mn;
    const float4 u = momentum4(m, g, p.mu, p.nesterov, &mn);
    store_f4(mp.M + idx, mn, v4, valid);
    ss.x += u.x * u.x;
    ss.y += u.y * u.y;
    ss.z += u.z * u.z;
    ss.w += u.w * u.w;
  }
  float* dst = p.partials + ((size_t)mat * p.row_blocks + rb) * p.n + col;
  store_f4(dst, ss, v4, valid);
}

__global__ void __launch_bounds__(256) rownorm_colfinal_kernel(const RowNormParams p) {
  const int cb = (p.n + 255) / 256;
  const int mat = blockIdx.x / cb;
  const int col = (blockIdx.x - mat * cb) * 256 + threadIdx.x;
  if (col >= p.n) return;
  const float* part = p.partials + (size_t)mat * p.row_blocks * p.n + col;
  double s = 0.0;
  for (int rb = 0; rb < p.row_blocks; ++rb) s += (double)part[(size_t)rb * p.n];
  const float nrm = (float)sqrt(s);
  p.colscale[(size_t)mat * p.n + col] = 1.0f / max_eps(nrm, p.eps);
}

template <bool GBF16>
__global__ void __launch_bounds__(256) rownorm_colapply_kernel(const RowNormParams p, int vec) {
  const int cblocks = (p.n + 1023) / 1024;
  const int per_mat = cblocks * p.row_blocks;
  const int mat = blockIdx.x / per_mat;
  const int bl = blockIdx.x - mat * per_mat;
  const int rb = bl / cblocks, cb = bl - rb * cblocks;
  const MatPtrs mp = p.table[mat];
  const int col = cb * 1024 + threadIdx.x * 4;
  if (col >= p.n) return;
  const int valid = p.n - col;
  const bool v4 = vec && valid >= 4;
  const float4 sc = load_f4(p.colscale + (size_t)mat * p.n + col, v4, valid);
  const int r0 = rb * RN_ROWS, r1 = min(p.m, r0 + RN_ROWS);
  auto apply = [&](size_t idx, float4 mn, float4 g, float4 w) {
    const float4 u = p.nesterov ? make_float4(p.mu * mn.x + g.x, p.mu * mn.y + g.y,
                                              p.mu * mn.z + g.z, p.mu * mn.w + g.w)
                                : mn;
    const float4 r = make_float4(u.x * sc.x, u.y * sc.y, u.z * sc.z, u.w * sc.w);
    w.x = p.decay * w.x - p.step * r.x;
    w.y = p.decay * w.y - p.step * r.y;
    w.z = p.decay * w.z - p.step * r.z;
    w.w = p.decay * w.w - p.step * r.w;
    store_f4(mp.W + idx, w, v4, valid);
    if (mp.O) store_f4(mp.O + idx, r, v4, valid);
  };
  constexpr int UR = 4;  // rows per iteration (loads in flight)
  int row = r0;
  for (; row + UR <= r1; row += UR) {
    float4 mn[UR], g[UR], w[UR];
#pragma unroll
    for (int q = 0; q < UR; ++q) {
      const size_t idx = (size_t)(row + q) * p.n + col;
      mn[q] = load_f4(mp.M + idx, v4, valid);
      g[q] = load_g4<GBF16>(mp.G, idx, v4, valid);
      w[q] = load_f4(mp.W + idx, v4, valid);
    }
#pragma unroll
    for (int q = 0; q < UR; ++q) apply((size_t)(row + q) * p.n + col, mn[q], g[q], w[q]);
  }
  for (; row < r1; ++row) {
    const size_t idx = (size_t)row * p.n + col;
    apply(idx, load_f4(mp.M + idx, v4, valid), load_g4<GBF16>(mp.G, idx, v4, valid),
          load_f4(mp.W + idx, v4, valid));
  }
}

int rownorm_row_blocks(int m, int n) {
  (void)n;
  return (m + RN_ROWS - 1) / RN_ROWS;
}

hipError_t launch_rownorm(const RowNormParams& p, int grad_bf16, int nmat, int vec, int phase,
                          hipStream_t s) {
  if (nmat == 0) return hipSuccess;
  const dim3 b(256);
  if (phase == RN_PHASE_ROWS) {
    const uint64_t blocks = (uint64_t)nmat * p.m;
    if (blocks > 0x7fffffffull) return hipErrorInvalidValue;
    const int nc = (p.n + 3) / 4;
    const dim3 g((uint32_t)blocks);
#define RN_ROWS_LAUNCH(GB)                                                                      \
  do {                                                                                          \
    if (nc <= 256) hipLaunchKernelGGL((rownorm_rows_kernel<GB, 1, 256>), g, dim3(256), 0, s, p, vec);  \
    else if (nc <= 1024) hipLaunchKernelGGL((rownorm_rows_kernel<GB, 4, 256>), g, dim3(256), 0, s, p, vec); \
    else if (nc <= 2048) hipLaunchKernelGGL((rownorm_rows_kernel<GB, 4, 512>), g, dim3(512), 0, s, p, vec); \
    else if (nc <= 4096) hipLaunchKernelGGL((rownorm_rows_kernel<GB, 4, 1024>), g, dim3(1024), 0, s, p, vec); \
    else hipLaunchKernelGGL((rownorm_rows_kernel<GB, 0, 1024>), g, dim3(1024), 0, s, p, vec);  \
  } while (0)
    if (grad_bf16) RN_ROWS_LAUNCH(true); else RN_ROWS_LAUNCH(false);
#undef RN_ROWS_LAUNCH
    return hipGetLastError();
  }
  if (phase == RN_PHASE_COLFINAL) {
    hipLaunchKernelGGL(rownorm_colfinal_kernel, dim3((uint32_t)(nmat * ((p.n + 255) / 256))), b,
                       0, s, p);
    return hipGetLastError();
  }
  const uint64_t blocks = (uint64_t)nmat * p.row_blocks * ((p.n + 1023) / 1024);
  if (blocks > 0x7fffffffull) return hipErrorInvalidValue;
  const dim3 g((uint32_t)blocks);
  if (phase == RN_PHASE_COLSUM) {
    if (grad_bf16) hipLaunchKernelGGL((rownorm_colsum_kernel<true>), g, b, 0, s, p, vec);
    else hipLaunchKernelGGL((rownorm_colsum_kernel<false>), g, b, 0, s, p, vec);
  } else {
    if (grad_bf16) hipLaunchKernelGGL((rownorm_colapply_kernel<true>), g, b, 0, s, p, vec);
    else hipLaunchKernelGGL((rownorm_colapply_kernel<false>), g, b, 0, s, p, vec);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Pointer-table upload from kernel arguments (one thread per entry).
constexpr int kTableThreads = (kTableChunk + 63) / 64 * 64;
static_assert(sizeof(TableChunk) + sizeof(MatPtrs*) <= 4096, "kernel argument block over 4 KB");

__global__ void __launch_bounds__(kTableThreads) write_table_kernel(const TableChunk t, MatPtrs* dst) {
  const int i = threadIdx.x;
  if (i < t.count) dst[i] = t.e[i];
}

hipError_t launch_write_table(const TableChunk& t, MatPtrs* dst, hipStream_t s) {
  if (t.count < 1 || t.count > kTableChunk) return hipErrorInvalidValue;
  hipLaunchKernelGGL(write_table_kernel, dim3(1), dim3(kTableThreads), 0, s, t, dst);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Direct form.  X0 cast: each thread converts 8 consecutive elements (one
// 16-byte load, one 16-byte store) of one of the two layouts in place.
__global__ void __launch_bounds__(256) xcast_kernel(const XcastParams p) {
  const int64_t per_buf = p.elems / 8;
  const int64_t blocks_per_buf = (per_buf + 255) / 256;
  const int nbuf = p.Xt ? 2 : 1;
  const int64_t b = blockIdx.x;
  const int mat = (int)(b / (nbuf * blocks_per_buf));
  const int64_t rem = b - (int64_t)mat * nbuf * blocks_per_buf;
  const int which = rem >= blocks_per_buf ? 1 : 0;
  const int64_t chunk = (rem - which * blocks_per_buf) * 256 + threadIdx.x;
  if (chunk >= per_buf) return;
  uint16_t* base = (uint16_t*)(which ? p.Xt : p.Xn) + (size_t)mat * p.x_stride + (size_t)chunk * 8;
  const float sc = p.inv_norm[mat] * p.sx;
  const u32x4 in = *(const u32x4*)base;
  u32x4 out;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float lo = __uint_as_float(in[k] << 16), hi = __uint_as_float(in[k] & 0xffff0000u);
    out[k] = (uint32_t)f32_to_f16_bits(lo * sc) | ((uint32_t)f32_to_f16_bits(hi * sc) << 16);
  }
  *(u32x4*)base = out;
}

hipError_t launch_xcast(const XcastParams& p, int nmat, hipStream_t s) {
  if (p.elems % 8) return hipErrorInvalidValue;
  const uint64_t blocks = (uint64_t)nmat * (p.Xt ? 2 : 1) * (uint64_t)((p.elems / 8 + 255) / 256);
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffull) return hipErrorInvalidValue;
  hipLaunchKernelGGL(xcast_kernel, dim3((uint32_t)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

// Weight update from X_N: 4 columns per thread, a 1024-column strip of one
// row per workgroup.
__global__ void __launch_bounds__(256) wupd_kernel(const WupdParams p, int vec) {
  const int cblocks = (p.n + 1023) / 1024;
  const int per_mat = cblocks * p.m;
  const int mat = blockIdx.x / per_mat;
  const int bl = blockIdx.x - mat * per_mat;
  const int row = bl / cblocks, cb = bl - row * cblocks;
  const int col = cb * 1024 + threadIdx.x * 4;
  if (col >= p.n) return;
  const int valid = p.n - col;
  const bool v4 = vec && valid >= 4;
  const MatPtrs mp = p.table[mat];
  const uint16_t* xr = (const uint16_t*)p.X + (size_t)mat * p.x_stride + (size_t)row * p.n_pad + col;
  // the X row is padded to n_pad (a multiple of 256): 4 elements always readable
  const uint2 xv = *(const uint2*)xr;
  const _Float16* xh = (const _Float16*)&xv;
  const float4 o = make_float4((float)xh[0] * p.inv_sx, (float)xh[1] * p.inv_sx,
                               (float)xh[2] * p.inv_sx, (float)xh[3] * p.inv_sx);
  const size_t idx = (size_t)row * p.n + col;
  float4 w = load_f4(mp.W + idx, v4, valid);
  w.x = p.decay * w.x - p.step * o.x;
  w.y = p.decay * w.y - p.step * o.y;
  w.z = p.decay * w.z - p.step * o.z;
  w.w = p.decay * w.w - p.step * o.w;
  store_f4(mp.W + idx, w, v4, valid);
  if (mp.O) store_f4(mp.O + idx, o, v4, valid);
}

hipError_t launch_wupd(const WupdParams& p, int nmat, int vec, hipStream_t s) {
  const uint64_t blocks = (uint64_t)nmat * (uint64_t)p.m * (uint64_t)((p.n + 1023) / 1024);
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffull || p.n_pad % 4 || p.n > p.n_pad) return hipErrorInvalidValue;
  hipLaunchKernelGGL(wupd_kernel, dim3((uint32_t)blocks), dim3(256), 0, s, p, vec);
  return hipGetLastError();
}

}  // namespace muon
