// Fused epilogues shared by the GEMM kernels (see gemm.hip for the list).
#pragma once

#include "common.hpp"
#include "kernels.h"

namespace muon {

// a x + b y, elementwise
__device__ __forceinline__ float4 f4_axpy(float a, float4 x, float b, float4 y) {
  return make_float4(a * x.x + b * y.x, a * x.y + b * y.y, a * x.z + b * y.z, a * x.w + b * y.w);
}

// ---------------------------------------------------------------------------
// Epilogues of the small-tile kernel's r x r products, four columns at a
// time: accumulators of (row, col0 + k), k = 0..3, stored for k in
// [klo, khi) (the rest lies on the other side of the diagonal).  The mirror
// pass calls it with row and column swapped and recomputes the identical
// value from the transposed read (every r x r input is stored exactly
// symmetric).  col0 is a multiple of 4 and the padded r x r buffers have a
// multiple of 4 columns, so every input is one 16-byte load; whole groups
// store fp32 as 16 bytes and 16-bit copies as 8 bytes.
//   SYRK  G0 = acc / ||U||^2                      fp32 G, fp16 G^ = G sG
//   POLY  P~ = b G + c acc / sG^2                 fp16 P^ = P~ sP; first: Q = a I + P~
//   PQPG  H = a G + acc / (sP sG)   (product 1)   fp32 H, fp16 H^ = H sH
//         Q = a Q + acc / (sP sQ)   (product 0)   fp32 Q, fp16 Q^ = Q sQ (bf16 Q when last)
//   PH    G = a H + acc / (sP sH)                 fp32 G, fp16 G^
// (the fp32 path keeps fp32 operand copies: every scale is 1)
__device__ __forceinline__ float4 ld4(const float* b, size_t o) { return *(const float4*)(b + o); }
__device__ __forceinline__ float f4at(const float4& v, int k) {
  return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
}
__device__ __forceinline__ void st4f(float* b, size_t o, float4 v, int klo, int khi) {
  if (klo == 0 && khi == 4) {
    *(float4*)(b + o) = v;
    return;
  }
  for (int k = klo; k < khi; ++k) b[o + k] = f4at(v, k);
}
// 16-bit copy of four values (scaled fp16, or bf16 when bf is set)
__device__ __forceinline__ void st4h(void* base, size_t o, float4 v, float scale, bool bf, int klo,
                                     int khi) {
  uint16_t e[4];
  for (int k = 0; k < 4; ++k)
    e[k] = bf ? f32_to_bf16_bits(f4at(v, k)) : f32_to_f16_bits(f4at(v, k) * scale);
  uint16_t* b = (uint16_t*)base;
  if (klo == 0 && khi == 4) {
    *(uint2*)(b + o) = make_uint2((uint32_t)e[0] | ((uint32_t)e[1] << 16),
                                  (uint32_t)e[2] | ((uint32_t)e[3] << 16));
    return;
  }
  for (int k = klo; k < khi; ++k) b[o + k] = e[k];
}

template <int EPI, bool F32PATH>
__device__ __forceinline__ void epilogue4(const GemmParams& p, int mat, int prod, int row, int col0,
                                          float4 acc, int klo, int khi) {
  static_assert(EPI != EPI_FINAL && EPI != EPI_XUPD && EPI != EPI_XFINAL,
                "the final and X' products have their own epilogues");
  const size_t o1 = (size_t)mat * p.rr_stride + (size_t)row * p.ldr + col0;
  auto scale4 = [](float4 a, float s) { return make_float4(a.x * s, a.y * s, a.z * s, a.w * s); };
  float4 v;
  if constexpr (EPI == EPI_SYRK) {
    // Gram form: G0 = acc / ||U||^2; direct form (fp16 X scaled by sX):
    // A = acc * syrk_scale
    const float inv = p.inv_norm[mat];
    const float sc = p.syrk_scale > 0.0f ? p.syrk_scale : inv * inv;
    v = make_float4(acc.x * sc, acc.y * sc, acc.z * sc, acc.w * sc);
    st4f(p.Gf, o1, v, klo, khi);
    if constexpr (!F32PATH) st4h(p.Gh, o1, v, p.sG, false, klo, khi);
    return;
  } else if constexpr (EPI == EPI_POLY) {
    const float4 g = ld4(p.Gf, o1);
    const float4 s2 = scale4(acc, 1.0f / (p.sG * p.sG));
    const float4 pt = f4_axpy(p.b, g, p.c, s2);
    if constexpr (F32PATH) st4f((float*)p.Ph, o1, scale4(pt, p.sP), klo, khi);
    else st4h(p.Ph, o1, pt, p.sP, false, klo, khi);
    if (!p.first) return;
    v = pt;  // Q1 = P1 = a I + P~
    if (row == col0) v.x += p.a;
    if (row == col0 + 1) v.y += p.a;
    if (row == col0 + 2) v.z += p.a;
    if (row == col0 + 3) v.w += p.a;
  } else if constexpr (EPI == EPI_PQPG) {
    if (prod == 1) {
      const float4 hv = f4_axpy(p.a, ld4(p.Gf, o1), 1.0f, scale4(acc, 1.0f / (p.sP * p.sG)));
      st4f(p.Hf, o1, hv, klo, khi);
      if constexpr (!F32PATH) st4h(p.Hh, o1, hv, p.sH, false, klo, khi);
      return;
    }
    v = f4_axpy(p.a, ld4(p.Qf_src, o1), 1.0f, scale4(acc, 1.0f / (p.sP * p.sQ)));
  } else {  // EPI_PH
    const float4 g = f4_axpy(p.a, ld4(p.Hf, o1), 1.0f, scale4(acc, 1.0f / (p.sP * p.sH)));
    st4f(p.Gf, o1, g, klo, khi);
    if constexpr (!F32PATH) st4h(p.Gh, o1, g, p.sG, false, klo, khi);
    return;
  }
  // Q output (POLY on the first iteration, or the PQ product)
  if constexpr (F32PATH) {
    st4f(p.Qf_dst, o1, v, klo, khi);
  } else {
    if (p.last) {  // operand of the final bf16 product, unscaled
      st4h(p.Qh_dst, o1, v, 1.0f, true, klo, khi);
    } else {
      st4f(p.Qf_dst, o1, v, klo, khi);
      st4h(p.Qh_dst, o1, v, p.sQ, false, klo, khi);
    }
  }
}

// ---------------------------------------------------------------------------
// Helpers of the 256-tile path (gemm_dma.hip), which keeps no fp32 master
// copies of the r x r results.
//
// The 256-tile kernels fold the identity term of each r x r product into
// the accumulators while the product runs (acc += gamma * X, X the raw fp16
// identity-term operand), so the epilogue only scales: v = beta * acc.
//   SYRK  G0 = X0 X0^T / ||U||^2                 beta = 1/||U||^2
//   POLY  P~ = b G + c G^2,  acc = sG^2 G^2       beta = c/sG^2,       gamma = b sG / c
//   PQPG  H  = a G + P~ G,   acc = sP sG P~ G     beta = 1/(sP sG),    gamma = a sP
//         Q' = a Q + P~ Q,   acc = sP sQ P~ Q     beta = 1/(sP sQ),    gamma = a sP
//   PH    G' = a H + P~ H,   acc = sP sH P~ H     beta = 1/(sP sH),    gamma = a sP
//   XUPD  X' = a X + P~ X,   acc = sP sX P~ X     beta = 1/(sP sX),    gamma = a sP
//         (direct form; SYRK there runs on fp16 X: beta = 1/sX^2; XFINAL is
//         the last XUPD applied to W by the final product's epilogue)
template <int EPI>
__device__ __forceinline__ float rr_beta(const GemmParams& p, int mat, int prod) {
  if constexpr (EPI == EPI_SYRK) {
    if (p.syrk_scale > 0.0f) return p.syrk_scale;
    const float inv = p.inv_norm[mat];
    return inv * inv;
  } else if constexpr (EPI == EPI_XUPD || EPI == EPI_XFINAL) {
    return 1.0f / (p.sP * p.sX);
  } else if constexpr (EPI == EPI_POLY) {
    return p.c * (1.0f / (p.sG * p.sG));
  } else if constexpr (EPI == EPI_PQPG) {
    return prod == 1 ? 1.0f / (p.sP * p.sG) : 1.0f / (p.sP * p.sQ);
  } else {
    return 1.0f / (p.sP * p.sH);
  }
}
template <int EPI>
__device__ __forceinline__ float rr_gamma(const GemmParams& p) {
  if constexpr (EPI == EPI_POLY) return p.b * p.sG / p.c;
  else return p.a * p.sP;
}

// Four fp16 values (scaled X of the direct form) as floats.
__device__ __forceinline__ float4 ld4h(const void* base, size_t o) {
  const uint2 u = *(const uint2*)((const uint16_t*)base + o);
  const _Float16* h = (const _Float16*)&u;
  return make_float4((float)h[0], (float)h[1], (float)h[2], (float)h[3]);
}

// Final product: O = inv * acc (inv = 1/||U||, or the direct form's 1/(sP sX)),
// W <- decay W - step O at (gi, gj..gj+3).
__device__ __forceinline__ void epilogue_final4(const GemmParams& p, int mat, int gi, int gj,
                                                float4 acc, float inv) {
  if (gi >= p.out_rows || gj >= p.out_cols) return;
  const MatPtrs mp = p.table[mat];
  const float4 o = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  const size_t idx = (size_t)gi * p.out_cols + gj;
  if (p.vec && gj + 4 <= p.out_cols) {
    nt_store4(mp.W + idx, f4_axpy(p.decay, nt_load4(mp.W + idx), -p.step, o));
    if (mp.O) nt_store4(mp.O + idx, o);
  } else {
    const float ov[4] = {o.x, o.y, o.z, o.w};
    for (int k = 0; k < 4 && gj + k < p.out_cols; ++k) {
      mp.W[idx + k] = p.decay * mp.W[idx + k] - p.step * ov[k];
      if (mp.O) mp.O[idx + k] = ov[k];
    }
  }
}

}  // namespace muon
