// Batched MFMA GEMM C = A * B^T for the Gram-space Newton-Schulz step, with
// the fused epilogues of every product on the path:
//   EPI_SYRK  G0 = X X^T / ||U||^2, lower-triangle tiles only, mirrored
//             ("DMuon" 2.2: symmetric SYRK-style Gram product)
//   EPI_POLY  S = G G, then P~ = b G + c S   (P = a I + P~, eq. (2) polynomial)
//             and, on the first iteration, Q = P
//   EPI_PQPG  Q' = a Q + P~ Q  and  H = a G + P~ G  in one launch
//   EPI_PH    G' = a H + P~ H   (so G' = P G P)
//   EPI_FINAL O = Q X0 / ||U||, then W <- (1 - lr wd) W - lr s O
//             ("Infra Optimizers" eq. (4); "Scaling Muon for DiT" 2.1)
// Every r x r matrix of the recursion is a polynomial in G0, hence symmetric
// and commuting, so each product needs only its lower-triangle tiles and
// B^T == B for the K-contiguous operand layout.
//
// CDNA4 mapping: 256 threads = 4 wave64 in a 2 x 2 grid, each wave owns a
// (BT/2) x (BT/2) sub-tile built from 32x32x16 MFMAs (bf16 or fp16 operands,
// fp32 accumulate) or 32x32x2 fp32 MFMAs.  Operand tiles are staged through
// LDS in a K-contiguous layout with an XOR swizzle on 16-byte chunks (bank
// conflict free for both the MFMA fragment reads and the global->LDS
// writes), double buffered with one barrier per K step.  A K-strided
// operand (X0 in the final product) is transposed in registers, 8x8 (or
// 4x4) at a time, on its way into LDS.  Workgroup ids are remapped so that
// consecutive tiles share an XCD's L2.
#include "common.hpp"
#include "kernels.h"

namespace muon {

enum Kind { K_BF16 = 0, K_F16 = 1, K_F32 = 2 };

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

template <int KIND>
__device__ __forceinline__ void mfma16B(const u32x4& a, const u32x4& b, f32x16& c) {
  if constexpr (KIND == K_BF16) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else if constexpr (KIND == K_F16) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                               __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  } else {
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[0]), __uint_as_float(b[0]), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[1]), __uint_as_float(b[1]), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[2]), __uint_as_float(b[2]), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[3]), __uint_as_float(b[3]), c, 0, 0, 0);
  }
}


// Transpose an E x E block held as E rows of 16 bytes (row kk = one k,
// E consecutive "rows" of the operand) into E rows of E consecutive k.
template <int ES>
__device__ __forceinline__ void transpose_block(const u32x4* in, u32x4* out) {
  if constexpr (ES == 2) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t d[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = in[2 * q][j >> 1];
        const uint32_t hi = in[2 * q + 1][j >> 1];
        d[q] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
      }
      out[j] = u32x4{d[0], d[1], d[2], d[3]};
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      out[j] = u32x4{in[0][j], in[1][j], in[2][j], in[3][j]};
  }
}

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

// Global -> register stage of one operand tile (BT rows x KT k).
template <int ES, int BT, bool KS>
__device__ __forceinline__ void load_tile(const char* __restrict__ base, int ld, int row0, int k0,
                                          int tid, u32x4* r) {
  constexpr int E = 16 / ES, KT = 128 / ES;
  if constexpr (!KS) {
    constexpr int LOADS = BT * 8 / 256;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int q = tid + 256 * i;
      const int row = q >> 3, ch = q & 7;
      r[i] = *(const u32x4*)(base + ((size_t)(row0 + row) * ld + k0) * ES + ch * 16);
    }
  } else {
    constexpr int NBLK = (KT / E) * (BT / E), BPT = (NBLK + 255) / 256;
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
      const int blk = tid + 256 * b;
      if (NBLK % 256 == 0 || blk < NBLK) {
        const int nc = blk % (BT / E), kg = blk / (BT / E);
#pragma unroll
        for (int kk = 0; kk < E; ++kk)
          r[b * E + kk] =
              *(const u32x4*)(base + ((size_t)(k0 + kg * E + kk) * ld + row0 + nc * E) * ES);
      }
    }
  }
}

// Register -> LDS stage (K-contiguous, swizzled).  A K-strided tile is
// transposed E x E in registers first.
template <int ES, int BT, bool KS>
__device__ __forceinline__ void store_tile(u32x4* s, const u32x4* r, int tid) {
  constexpr int E = 16 / ES, KT = 128 / ES;
  if constexpr (!KS) {
    constexpr int LOADS = BT * 8 / 256;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int q = tid + 256 * i;
      const int row = q >> 3, ch = q & 7;
      s[row * 8 + (ch ^ swz(row))] = r[i];
    }
  } else {
    constexpr int NBLK = (KT / E) * (BT / E), BPT = (NBLK + 255) / 256;
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
      const int blk = tid + 256 * b;
      if (NBLK % 256 == 0 || blk < NBLK) {
        const int nc = blk % (BT / E), kg = blk / (BT / E);
        u32x4 tr[E];
        transpose_block<ES>(r + b * E, tr);
#pragma unroll
        for (int j = 0; j < E; ++j) {
          const int row = nc * E + j;
          s[row * 8 + (kg ^ swz(row))] = tr[j];
        }
      }
    }
  }
}

template <int KIND, int BT, int EPI, bool AKS, bool BKS, bool F32PATH>
__global__ void __launch_bounds__(256) gemm_kernel(const GemmParams p) {
  constexpr int ES = (KIND == K_F32) ? 4 : 2;
  constexpr int E = 16 / ES;           // elements per 16-byte chunk
  constexpr int KT = 128 / ES;         // K elements per step (8 chunks per row)
  constexpr int WT = BT / 2;           // wave sub-tile
  constexpr int F = WT / 32;           // 32x32 MFMA blocks per wave dimension
  constexpr int LOADS = BT * 8 / 256;  // 16-byte chunks per thread (K-contiguous)
  constexpr int NBLK = (KT / E) * (BT / E);  // E x E blocks (K-strided)
  constexpr int BPT = (NBLK + 255) / 256;
  static_assert(F >= 1 && LOADS >= 1, "tile too small");
  (void)E;

  constexpr int RR = BT < 128 ? BT : 128;  // epilogue rows staged per round
  constexpr int EPI_LD = BT + 1;            // padded fp32 row (bank spread)
  constexpr int SMEM_OPS = 2 * 2 * BT * 8 * 16;
  constexpr int SMEM_EPI = RR * EPI_LD * 4;
  constexpr int SMEM_BYTES = SMEM_OPS > SMEM_EPI ? SMEM_OPS : SMEM_EPI;
  __shared__ __attribute__((aligned(16))) char smem_raw[SMEM_BYTES];
  u32x4(*smem)[2][BT * 8] = reinterpret_cast<u32x4(*)[2][BT * 8]>(smem_raw);
  float* stile = reinterpret_cast<float*>(smem_raw);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, l32 = lane & 31;

  const uint32_t bid = xcd_remap(blockIdx.x, gridDim.x);
  const int per_mat = p.tiles_per_prod * p.products;
  const int mat = bid / per_mat;
  int t = bid - mat * per_mat;
  const int pi = t / p.tiles_per_prod;  // operand set of this tile
  t -= pi * p.tiles_per_prod;
  const int prod = pi + p.prod_base;      // epilogue selector
  int ti, tj;
  if (p.triangular) {
    ti = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
    while ((ti + 1) * (ti + 2) / 2 <= t) ++ti;
    while (ti * (ti + 1) / 2 > t) --ti;
    tj = t - ti * (ti + 1) / 2;
  } else {
    ti = t / p.tiles_n;
    tj = t - ti * p.tiles_n;
  }
  const int row0A = ti * BT, row0B = tj * BT;
  const char* Ab = (const char*)p.A + (size_t)mat * p.a_stride * ES;
  const char* Bb = pi ? (const char*)p.B2 + (size_t)mat * p.b2_stride * ES
                        : (const char*)p.B + (size_t)mat * p.b_stride * ES;

  u32x4 ra[AKS ? BPT * E : LOADS];
  u32x4 rb[BKS ? BPT * E : LOADS];

  f32x16 acc[F][F];
#pragma unroll
  for (int i = 0; i < F; ++i)
#pragma unroll
    for (int j = 0; j < F; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int nk = p.Kdim / KT;
  load_tile<ES, BT, AKS>(Ab, p.lda, row0A, 0, tid, ra);
  load_tile<ES, BT, BKS>(Bb, p.ldb, row0B, 0, tid, rb);
  store_tile<ES, BT, AKS>(smem[0][0], ra, tid);
  store_tile<ES, BT, BKS>(smem[0][1], rb, tid);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      load_tile<ES, BT, AKS>(Ab, p.lda, row0A, (kt + 1) * KT, tid, ra);
      load_tile<ES, BT, BKS>(Bb, p.ldb, row0B, (kt + 1) * KT, tid, rb);
    }
    const u32x4* sA = smem[cur][0];
    const u32x4* sB = smem[cur][1];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int ch = 2 * s + h;
      u32x4 af[F], bfr[F];
#pragma unroll
      for (int f = 0; f < F; ++f) {
        const int ra_ = wm * WT + f * 32 + l32;
        af[f] = sA[ra_ * 8 + (ch ^ swz(ra_))];
        const int rb_ = wn * WT + f * 32 + l32;
        bfr[f] = sB[rb_ * 8 + (ch ^ swz(rb_))];
      }
#pragma unroll
      for (int i = 0; i < F; ++i)
#pragma unroll
        for (int j = 0; j < F; ++j) mfma16B<KIND>(af[i], bfr[j], acc[i][j]);
    }
    if (more) {
      store_tile<ES, BT, AKS>(smem[cur ^ 1][0], ra, tid);
      store_tile<ES, BT, BKS>(smem[cur ^ 1][1], rb, tid);
    }
    __syncthreads();
  }

  // Epilogue: stage RR rows of the fp32 tile through LDS per round, then let
  // all 256 threads walk it row-major (coalesced stores of (gi, gj)) and, for
  // symmetric results, column-major (coalesced stores of the mirror (gj, gi)).
#pragma unroll
  for (int round = 0; round < BT / RR; ++round) {
    if ((wm * WT) / RR == round) {
#pragma unroll
      for (int i = 0; i < F; ++i)
#pragma unroll
        for (int j = 0; j < F; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int il = wm * WT + i * 32 + 8 * (v >> 2) + 4 * h + (v & 3) - round * RR;
            const int jl = wn * WT + j * 32 + l32;
            stile[il * EPI_LD + jl] = acc[i][j][v];
          }
    }
    __syncthreads();
    const int gr0 = row0A + round * RR;
    constexpr int PER = RR * BT / 256;
    if constexpr (BT >= 256) {
      // row pass: one full tile row per iteration
#pragma unroll 4
      for (int e = 0; e < PER; ++e) {
        const int il = e * (256 / BT), jl = tid % BT;
        const int gi = gr0 + il, gj = row0B + jl;
        if (EPI == EPI_FINAL || gi >= gj)
          epilogue<EPI, F32PATH>(p, mat, prod, gi, gj, stile[il * EPI_LD + jl]);
      }
    } else {
#pragma unroll 4
      for (int e = 0; e < PER; ++e) {
        const int il = e * (256 / BT) + tid / BT, jl = tid % BT;
        const int gi = gr0 + il, gj = row0B + jl;
        if (EPI == EPI_FINAL || gi >= gj)
          epilogue<EPI, F32PATH>(p, mat, prod, gi, gj, stile[il * EPI_LD + jl]);
      }
    }
    if constexpr (EPI != EPI_FINAL) {
      // mirror pass: consecutive threads take consecutive tile rows il, so the
      // stores to (gj, gi) are contiguous in gi
#pragma unroll 4
      for (int e = 0; e < PER; ++e) {
        const int il = tid % RR, jl = e * (256 / RR) + tid / RR;
        const int gi = gr0 + il, gj = row0B + jl;
        if (gi > gj) epilogue<EPI, F32PATH>(p, mat, prod, gj, gi, stile[il * EPI_LD + jl]);
      }
    }
    __syncthreads();
  }
}

template <int KIND, int BT, int EPI, bool AKS, bool BKS, bool F32PATH>
static hipError_t launch_one(const GemmParams& p, int nmat, hipStream_t s) {
  const uint64_t blocks = (uint64_t)nmat * p.tiles_per_prod * p.products;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffull) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_kernel<KIND, BT, EPI, AKS, BKS, F32PATH>), dim3((uint32_t)blocks),
                     dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int BT, bool F32PATH>
static hipError_t launch_bt(const GemmParams& p, int epi, int aks, int bks, int nmat,
                            hipStream_t s) {
  constexpr int KX = F32PATH ? K_F32 : K_BF16;  // X0 / final operands
  constexpr int KR = F32PATH ? K_F32 : K_F16;   // r x r recursion operands
  switch (epi) {
    case EPI_SYRK: return launch_one<KX, BT, EPI_SYRK, false, false, F32PATH>(p, nmat, s);
    case EPI_POLY: return launch_one<KR, BT, EPI_POLY, false, false, F32PATH>(p, nmat, s);
    case EPI_PQPG: return launch_one<KR, BT, EPI_PQPG, false, false, F32PATH>(p, nmat, s);
    case EPI_PH: return launch_one<KR, BT, EPI_PH, false, false, F32PATH>(p, nmat, s);
    case EPI_FINAL:
      if (aks && !bks) return launch_one<KX, BT, EPI_FINAL, true, false, F32PATH>(p, nmat, s);
      if (!aks && bks) return launch_one<KX, BT, EPI_FINAL, false, true, F32PATH>(p, nmat, s);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm(const GemmParams& p, int epi, int op, int bt, int aks, int bks, int nmat,
                       hipStream_t s) {
  if (op == OP_BF16) {
    switch (bt) {
      case 64: return launch_bt<64, false>(p, epi, aks, bks, nmat, s);
      case 128: return launch_bt<128, false>(p, epi, aks, bks, nmat, s);
      case 256: return launch_bt<256, false>(p, epi, aks, bks, nmat, s);
    }
  } else if (op == OP_F32) {
    switch (bt) {
      case 64: return launch_bt<64, true>(p, epi, aks, bks, nmat, s);
      case 128: return launch_bt<128, true>(p, epi, aks, bks, nmat, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace muon
