// Fused epilogues shared by the GEMM kernels (see gemm.hip for the list).
#pragma once

#include "common.hpp"
#include "kernels.h"

namespace muon {

template <bool F32PATH>
__device__ __forceinline__ void store_hat(void* base, size_t o, float v) {
  if constexpr (F32PATH) {
    ((float*)base)[o] = v;
  } else {
    ((uint16_t*)base)[o] = f32_to_f16_bits(v);
  }
}

// Epilogue value for one accumulator element at global (gi, gj) of matrix
// `mat`; it also performs the stores for the element itself.  The mirrored
// element (gj, gi) of a symmetric result is stored by a second call with the
// indices swapped, which recomputes the identical value from the transposed
// read (all r x r inputs are stored exactly symmetric).
template <int EPI, bool F32PATH>
__device__ __forceinline__ void epilogue(const GemmParams& p, int mat, int prod, int gi, int gj,
                                         float acc) {
  if constexpr (EPI == EPI_FINAL) {
    if (gi < p.out_rows && gj < p.out_cols) {
      const MatPtrs mp = p.table[mat];
      const float o = acc * p.inv_norm[mat];
      const size_t idx = (size_t)gi * p.out_cols + gj;
      mp.W[idx] = p.decay * mp.W[idx] - p.step * o;
      if (mp.O) mp.O[idx] = o;
    }
    return;
  } else {
    const size_t o1 = (size_t)mat * p.rr_stride + (size_t)gi * p.ldr + gj;
    float v;
    if constexpr (EPI == EPI_SYRK) {
      const float inv = p.inv_norm[mat];
      v = acc * inv * inv;
      p.Gf[o1] = v;
      if constexpr (!F32PATH) store_hat<false>(p.Gh, o1, v * p.sG);
      return;
    } else if constexpr (EPI == EPI_POLY) {
      const float g = p.Gf[o1];
      const float s2 = acc * (1.0f / (p.sG * p.sG));
      const float pt = p.b * g + p.c * s2;
      store_hat<F32PATH>(p.Ph, o1, pt * p.sP);
      if (!p.first) return;
      v = pt + (gi == gj ? p.a : 0.0f);  // Q1 = P1 = a I + P~
    } else if constexpr (EPI == EPI_PQPG) {
      if (prod == 1) {
        const float hv = p.a * p.Gf[o1] + acc * (1.0f / (p.sP * p.sG));
        p.Hf[o1] = hv;
        if constexpr (!F32PATH) store_hat<false>(p.Hh, o1, hv * p.sH);
        return;
      }
      v = p.a * p.Qf_src[o1] + acc * (1.0f / (p.sP * p.sQ));
    } else {  // EPI_PH
      const float g = p.a * p.Hf[o1] + acc * (1.0f / (p.sP * p.sH));
      p.Gf[o1] = g;
      if constexpr (!F32PATH) store_hat<false>(p.Gh, o1, g * p.sG);
      return;
    }
    // Q output (POLY on the first iteration, or the PQ product)
    if constexpr (F32PATH) {
      p.Qf_dst[o1] = v;
    } else {
      if (p.last) {  // operand of the final bf16 product, unscaled
        ((uint16_t*)p.Qh_dst)[o1] = f32_to_bf16_bits(v);
      } else {
        p.Qf_dst[o1] = v;
        store_hat<false>(p.Qh_dst, o1, v * p.sQ);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp16-only epilogues of the 256-tile path: the r x r inputs of the identity
// terms are read from the fp16 operand copies (no fp32 master copies), four
// consecutive elements per call.  `prim` receives the value the mirrored
// stores are derived from.

__device__ __forceinline__ float4 ld_h4(const void* base, size_t o, float inv_scale) {
  const uint2 u = *(const uint2*)((const uint16_t*)base + o);
  const _Float16* h = (const _Float16*)&u;
  return make_float4((float)h[0] * inv_scale, (float)h[1] * inv_scale, (float)h[2] * inv_scale,
                     (float)h[3] * inv_scale);
}

__device__ __forceinline__ void st_h4(void* base, size_t o, float4 v, float scale) {
  uint2 u;
  u.x = (uint32_t)f32_to_f16_bits(v.x * scale) | ((uint32_t)f32_to_f16_bits(v.y * scale) << 16);
  u.y = (uint32_t)f32_to_f16_bits(v.z * scale) | ((uint32_t)f32_to_f16_bits(v.w * scale) << 16);
  *(uint2*)((uint16_t*)base + o) = u;
}

__device__ __forceinline__ void st_b4(void* base, size_t o, float4 v) {
  uint2 u;
  u.x = (uint32_t)f32_to_bf16_bits(v.x) | ((uint32_t)f32_to_bf16_bits(v.y) << 16);
  u.y = (uint32_t)f32_to_bf16_bits(v.z) | ((uint32_t)f32_to_bf16_bits(v.w) << 16);
  *(uint2*)((uint16_t*)base + o) = u;
}

__device__ __forceinline__ float4 f4_axpy(float a, float4 x, float b, float4 y) {
  return make_float4(a * x.x + b * y.x, a * x.y + b * y.y, a * x.z + b * y.z, a * x.w + b * y.w);
}

// Store the outputs that derive from `v` at (gi, gj..gj+3) of an r x r
// result; `diag` adds a*I to the Q output of the first iteration.
template <int EPI>
__device__ __forceinline__ void store_rr4(const GemmParams& p, size_t o, int prod, float4 v,
                                          float4 q) {
  if constexpr (EPI == EPI_SYRK || EPI == EPI_PH) {
    st_h4(p.Gh, o, v, p.sG);
  } else if constexpr (EPI == EPI_POLY) {
    st_h4(p.Ph, o, v, p.sP);
    if (p.first) {
      if (p.last) st_b4(p.Qh_dst, o, q);
      else st_h4(p.Qh_dst, o, q, p.sQ);
    }
  } else {  // EPI_PQPG
    if (prod == 1) {
      st_h4(p.Hh, o, v, p.sH);
    } else {
      if (p.last) st_b4(p.Qh_dst, o, v);
      else st_h4(p.Qh_dst, o, v, p.sQ);
    }
  }
}

// Scalar forms for the diagonal tiles (lower-triangle masking per element).
__device__ __forceinline__ float ld_h1(const void* base, size_t o, float inv_scale) {
  return (float)__builtin_bit_cast(_Float16, ((const uint16_t*)base)[o]) * inv_scale;
}

template <int EPI>
__device__ __forceinline__ void store_rr1(const GemmParams& p, size_t o, int prod, float v,
                                          float q) {
  if constexpr (EPI == EPI_SYRK || EPI == EPI_PH) {
    ((uint16_t*)p.Gh)[o] = f32_to_f16_bits(v * p.sG);
  } else if constexpr (EPI == EPI_POLY) {
    ((uint16_t*)p.Ph)[o] = f32_to_f16_bits(v * p.sP);
    if (p.first)
      ((uint16_t*)p.Qh_dst)[o] = p.last ? f32_to_bf16_bits(q) : f32_to_f16_bits(q * p.sQ);
  } else {
    if (prod == 1) ((uint16_t*)p.Hh)[o] = f32_to_f16_bits(v * p.sH);
    else ((uint16_t*)p.Qh_dst)[o] = p.last ? f32_to_bf16_bits(v) : f32_to_f16_bits(v * p.sQ);
  }
}

template <int EPI>
__device__ __forceinline__ void store_rr1(const GemmParams& p, size_t o, int prod, float v) {
  store_rr1<EPI>(p, o, prod, v, v);
}

template <int EPI>
__device__ __forceinline__ float epilogue_rr1(const GemmParams& p, int mat, int prod, int gi,
                                              int gj, float acc) {
  const size_t o = (size_t)mat * p.rr_stride + (size_t)gi * p.ldr + gj;
  float v, q;
  if constexpr (EPI == EPI_SYRK) {
    const float inv = p.inv_norm[mat];
    v = acc * inv * inv;
    q = v;
  } else if constexpr (EPI == EPI_POLY) {
    v = p.b * ld_h1(p.Gh, o, 1.0f / p.sG) + p.c * (1.0f / (p.sG * p.sG)) * acc;
    q = v + ((p.first && gi == gj) ? p.a : 0.0f);
  } else if constexpr (EPI == EPI_PQPG) {
    if (prod == 1) v = p.a * ld_h1(p.Gh, o, 1.0f / p.sG) + (1.0f / (p.sP * p.sG)) * acc;
    else v = p.a * ld_h1(p.Qh_src, o, 1.0f / p.sQ) + (1.0f / (p.sP * p.sQ)) * acc;
    q = v;
  } else {
    v = p.a * ld_h1(p.Hh, o, 1.0f / p.sH) + (1.0f / (p.sP * p.sH)) * acc;
    q = v;
  }
  store_rr1<EPI>(p, o, prod, v, q);
  return v;
}

// Row pass: compute from the accumulators at (gi, gj..gj+3), store, return
// the primary value.
template <int EPI>
__device__ __forceinline__ float4 epilogue_rr4(const GemmParams& p, int mat, int prod, int gi,
                                               int gj, float4 acc) {
  const size_t o = (size_t)mat * p.rr_stride + (size_t)gi * p.ldr + gj;
  float4 v, q;
  if constexpr (EPI == EPI_SYRK) {
    const float inv = p.inv_norm[mat];
    v = f4_axpy(inv * inv, acc, 0.0f, acc);
    q = v;
  } else if constexpr (EPI == EPI_POLY) {
    const float4 g = ld_h4(p.Gh, o, 1.0f / p.sG);
    v = f4_axpy(p.b, g, p.c * (1.0f / (p.sG * p.sG)), acc);
    q = v;
    if (p.first) {
      if (gi == gj + 0) q.x += p.a;
      if (gi == gj + 1) q.y += p.a;
      if (gi == gj + 2) q.z += p.a;
      if (gi == gj + 3) q.w += p.a;
    }
  } else if constexpr (EPI == EPI_PQPG) {
    if (prod == 1) {
      const float4 g = ld_h4(p.Gh, o, 1.0f / p.sG);
      v = f4_axpy(p.a, g, 1.0f / (p.sP * p.sG), acc);
    } else {
      const float4 qs = ld_h4(p.Qh_src, o, 1.0f / p.sQ);
      v = f4_axpy(p.a, qs, 1.0f / (p.sP * p.sQ), acc);
    }
    q = v;
  } else {  // EPI_PH
    const float4 hh = ld_h4(p.Hh, o, 1.0f / p.sH);
    v = f4_axpy(p.a, hh, 1.0f / (p.sP * p.sH), acc);
    q = v;
  }
  store_rr4<EPI>(p, o, prod, v, q);
  return v;
}

// Row pass with the identity-term input already loaded (4 raw fp16 values).
__device__ __forceinline__ float4 h4_from_raw(uint2 u, float inv_scale) {
  const _Float16* h = (const _Float16*)&u;
  return make_float4((float)h[0] * inv_scale, (float)h[1] * inv_scale, (float)h[2] * inv_scale,
                     (float)h[3] * inv_scale);
}

template <int EPI>
__device__ __forceinline__ const void* rr_input(const GemmParams& p, int prod, float* inv_scale) {
  if constexpr (EPI == EPI_POLY) {
    *inv_scale = 1.0f / p.sG;
    return p.Gh;
  } else if constexpr (EPI == EPI_PQPG) {
    *inv_scale = prod == 1 ? 1.0f / p.sG : 1.0f / p.sQ;
    return prod == 1 ? p.Gh : p.Qh_src;
  } else {  // EPI_PH
    *inv_scale = 1.0f / p.sH;
    return p.Hh;
  }
}

template <int EPI>
__device__ __forceinline__ float4 epilogue_rr4_pre(const GemmParams& p, int mat, int prod, int gi,
                                                   int gj, float4 acc, uint2 raw) {
  const size_t o = (size_t)mat * p.rr_stride + (size_t)gi * p.ldr + gj;
  float4 v, q;
  if constexpr (EPI == EPI_SYRK) {
    const float inv = p.inv_norm[mat];
    v = f4_axpy(inv * inv, acc, 0.0f, acc);
    q = v;
  } else if constexpr (EPI == EPI_POLY) {
    v = f4_axpy(p.b, h4_from_raw(raw, 1.0f / p.sG), p.c * (1.0f / (p.sG * p.sG)), acc);
    q = v;
    if (p.first) {  // off-diagonal tile: Q1 = P~ there
    }
  } else if constexpr (EPI == EPI_PQPG) {
    if (prod == 1) v = f4_axpy(p.a, h4_from_raw(raw, 1.0f / p.sG), 1.0f / (p.sP * p.sG), acc);
    else v = f4_axpy(p.a, h4_from_raw(raw, 1.0f / p.sQ), 1.0f / (p.sP * p.sQ), acc);
    q = v;
  } else {  // EPI_PH
    v = f4_axpy(p.a, h4_from_raw(raw, 1.0f / p.sH), 1.0f / (p.sP * p.sH), acc);
    q = v;
  }
  store_rr4<EPI>(p, o, prod, v, q);
  return v;
}

// Final product: O = acc / ||U||, W <- decay W - step O at (gi, gj..gj+3).
__device__ __forceinline__ void epilogue_final4(const GemmParams& p, int mat, int gi, int gj,
                                                float4 acc) {
  if (gi >= p.out_rows || gj >= p.out_cols) return;
  const MatPtrs mp = p.table[mat];
  const float inv = p.inv_norm[mat];
  const float4 o = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  const size_t idx = (size_t)gi * p.out_cols + gj;
  if (p.vec && gj + 4 <= p.out_cols) {
    float4 w = *(const float4*)(mp.W + idx);
    w = f4_axpy(p.decay, w, -p.step, o);
    *(float4*)(mp.W + idx) = w;
    if (mp.O) *(float4*)(mp.O + idx) = o;
  } else {
    const float ov[4] = {o.x, o.y, o.z, o.w};
    for (int k = 0; k < 4 && gj + k < p.out_cols; ++k) {
      mp.W[idx + k] = p.decay * mp.W[idx + k] - p.step * ov[k];
      if (mp.O) mp.O[idx + k] = ov[k];
    }
  }
}

}  // namespace muon
