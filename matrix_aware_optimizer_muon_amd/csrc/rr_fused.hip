// The whole r x r Newton-Schulz recursion of the Gram form ("DMuon" 2.2,
// "Infra Optimizers" eq. (2)) in one launch for buckets with r_pad <= 128,
// one workgroup per matrix.  At that size every product is a few dozen MFMAs
// per wave and the launch-by-launch sequence (up to 17 dependent launches)
// is bound by launch latency, not by work.
//
// Same arithmetic as the small-tile kernels' epilogues (gemm_epilogue.hpp),
// same operand formats and power-of-two scales: per iteration k
//   POLY  S = G G                 P~ = b G + c S, P^ = fp16(P~ sP)
//                                 (k = 0: Q = a I + P~)
//   PQ    (k > 0)                 Q  = a Q + P~ Q
//   PG    (k < N-1)               H  = a G + P~ G
//   PH    (k < N-1)               G  = a H + P~ H
// with fp32 masters of G, Q, H and fp16 MFMA operands G^ = fp16(G sG),
// Q^ = fp16(Q sQ), H^ = fp16(H sH); the last Q is written as bf16, the
// operand of the final product.
//
// Layout: one wave64 per 32 x 32 block of the r_pad x r_pad matrices (4
// waves for r_pad = 64, 16 for 128: four per SIMD, so one wave's LDS and
// barrier waits overlap the others' MFMAs; with 4 waves of 64 x 64 each the
// r = 128 recursion kept the MFMAs busy ~10 % of the time), 32x32x16 fp16
// MFMAs.  The fp32 masters stay in registers in the accumulator layout (lane
// (h, l32) holds rows 8(v>>2) + 4h + (v&3), column l32 of the wave's
// block).  The four fp16 operands live in LDS, row-major with the 16-byte
// chunk index XOR-swizzled by the row; a lane writes its four consecutive
// rows of column l32 as four consecutive elements of LDS row l32, i.e. the
// LDS copy holds the transpose, which is the same matrix (every matrix of
// the recursion is symmetric up to rounding).  Exact symmetry is restored
// after every update: the Gram recursion G <- P G P amplifies an
// antisymmetric rounding component by about a^2 per iteration (simulated on
// a 3 x 5 input: 0.74 relative error after N = 5 without, 1.4e-3 with), so
// each new fp32 master is replaced by the mean of itself and its transpose
// through an fp32 LDS exchange (the tile kernels get exact symmetry by
// storing lower tiles and their mirror).
// LDS: three fp16 operands (G^ and H^ share a buffer: G^ is dead once PQ and
// PG have read it) and a half-matrix fp32 exchange, RP = 128: 96 + 33 KB.
#include "common.hpp"
#include "kernels.h"

namespace muon {

namespace {

template <int RP>
struct RrLds {
  static constexpr int NCH = RP / 8;  // 16-byte chunks per row
  // byte offset of chunk ch of row r
  __device__ static __forceinline__ int off(int r, int ch) { return r * RP * 2 + ((ch ^ (r & (NCH - 1))) << 4); }
};

__device__ __forceinline__ uint32_t pk_h2(float a, float b) {
  return (uint32_t)f32_to_f16_bits(a) | ((uint32_t)f32_to_f16_bits(b) << 16);
}
__device__ __forceinline__ uint32_t pk_b2(float a, float b) {
  return (uint32_t)f32_to_bf16_bits(a) | ((uint32_t)f32_to_bf16_bits(b) << 16);
}

}  // namespace

template <int RP>
__global__ void __launch_bounds__((RP / 32) * (RP / 32) * 64, 1) rr_fused_kernel(const RrFusedParams p) {
  constexpr int NB = RP / 32;         // 32 x 32 blocks per matrix dimension, one wave each
  constexpr int HB = NB / 2;          // block rows per exchange half
  constexpr int MB = RP * RP * 2;     // bytes of one fp16 matrix
  constexpr int XP = RP + 1;          // fp32 exchange pitch (bank spread)
  __shared__ __attribute__((aligned(16))) char smem[3 * MB + (RP / 2) * XP * 4];
  char* bG = smem;                    // G^, or H^ between PG and PH
  char* bP = smem + MB;
  char* bQ = smem + 2 * MB;
  float* xch = (float*)(smem + 3 * MB);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / NB, wn = wave % NB;  // the wave's block row and column
  const int h = lane >> 5, l32 = lane & 31;
  const int mat = blockIdx.x;

  // element (row, col) of accumulator value v of the wave's block
  auto row_of = [&](int v) { return wm * 32 + 8 * (v >> 2) + 4 * h + (v & 3); };
  const int col = wn * 32 + l32;

  // exact symmetry: every element becomes the mean of itself and its mirror
  // (fp32 addition commutes and halving is exact, so (r, c) and (c, r) get
  // the same value).  The exchange holds RP / 2 rows at a time (pitch
  // RP + 1: a row write and a column read by 32 lanes both touch 32 banks):
  // in half hf the waves of block rows [hf HB, hf HB + HB) write their rows,
  // and the waves whose block column lies in that range read their mirrors.
  // A block and its mirror in the same half average together; otherwise the
  // lower one (block row in the later half) reads first, in its column's
  // half, and writes its averaged values in the later half, where the upper
  // one takes them as they are instead of averaging a second time.
  const bool upper_later = (wm / HB) < (wn / HB);
  const float keep = upper_later ? 0.0f : 0.5f;  // m <- keep m + take mirror
  const float take = upper_later ? 1.0f : 0.5f;
  auto symm = [&](f32x16& m) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      if (wm / HB == hf) {
#pragma unroll
        for (int v = 0; v < 16; ++v) xch[(row_of(v) - hf * (RP / 2)) * XP + col] = m[v];
      }
      __syncthreads();
      if (wn / HB == hf) {
#pragma unroll
        for (int v = 0; v < 16; ++v) m[v] = keep * m[v] + take * xch[(col - hf * (RP / 2)) * XP + row_of(v)];
      }
      __syncthreads();
    }
  };

  // fp16 copy of a (symmetric) master into an LDS matrix: lane's rows
  // r0..r0+3 of column col become elements r0..r0+3 of LDS row col (one
  // 8-byte write per group)
  auto put = [&](char* buf, const f32x16& m, float scale) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int r0 = wm * 32 + 8 * g + 4 * h;
      const uint2 v = make_uint2(pk_h2(m[4 * g] * scale, m[4 * g + 1] * scale),
                                 pk_h2(m[4 * g + 2] * scale, m[4 * g + 3] * scale));
      *(uint2*)(buf + RrLds<RP>::off(col, r0 >> 3) + ((r0 & 7) << 1)) = v;
    }
  };

  // acc = A * B^T over K = RP, both operands in LDS
  auto mm = [&](const char* A, const char* B, f32x16& acc) {
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
    // RP = 128 (16 waves, 128 VGPRs each): two K steps' fragments in flight
    constexpr int UNR = RP == 64 ? RP / 16 : 2;
#pragma unroll UNR
    for (int ks = 0; ks < RP / 16; ++ks) {
      const u32x4 af = *(const u32x4*)(A + RrLds<RP>::off(wm * 32 + l32, 2 * ks + h));
      const u32x4 bf = *(const u32x4*)(B + RrLds<RP>::off(wn * 32 + l32, 2 * ks + h));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, af),
                                                   __builtin_bit_cast(f16x8, bf), acc, 0, 0, 0);
    }
  };

  // bf16 Q (the final product's operand) to global memory
  auto put_q_out = [&](const f32x16& m) {
    uint16_t* q = (uint16_t*)p.Qout + (size_t)mat * p.rr_stride;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int r0 = wm * 32 + 8 * g + 4 * h;
      *(uint2*)(q + (size_t)col * RP + r0) =
          make_uint2(pk_b2(m[4 * g], m[4 * g + 1]), pk_b2(m[4 * g + 2], m[4 * g + 3]));
    }
  };

  // fp32 masters: G (H between PG and PH, which replaces it) and Q; P~ is
  // formed in place in the accumulators
  f32x16 Gm, Qm, acc;
  {
    const float* g0 = p.Gf + (size_t)mat * p.rr_stride;
#pragma unroll
    for (int v = 0; v < 16; ++v) Gm[v] = g0[(size_t)row_of(v) * RP + col];
  }
  put(bG, Gm, p.sG);  // G0 from the SYRK is stored exactly symmetric
  __syncthreads();

  const float inv_gg = 1.0f / (p.sG * p.sG);
  const float inv_pq = 1.0f / (p.sP * p.sQ);
  const float inv_pg = 1.0f / (p.sP * p.sG);
  const float inv_ph = 1.0f / (p.sP * p.sH);
  for (int k = 0; k < p.N; ++k) {
    const bool first = k == 0, last = k == p.N - 1;
    // POLY: P~ = b G + c G^2, and Q1 = a I + P~
    mm(bG, bG, acc);
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = p.b * Gm[v] + p.c * (acc[v] * inv_gg);
    symm(acc);
    put(bP, acc, p.sP);
    if (first) {
      Qm = acc;
      // the diagonal: in a diagonal block, lane (h, l32) holds element
      // (l32, l32) as value 4 (l32 >> 3) + (l32 & 3) when bit 2 of l32 is h
      if (wm == wn && ((l32 >> 2) & 1) == h) Qm[4 * (l32 >> 3) + (l32 & 3)] += p.a;
      if (last) put_q_out(Qm);
      else put(bQ, Qm, p.sQ);
    }
    __syncthreads();
    if (!first) {
      // PQ: Q = a Q + P~ Q
      mm(bP, bQ, acc);
      __syncthreads();  // every read of Q^ is done before it is replaced
#pragma unroll
      for (int v = 0; v < 16; ++v) Qm[v] = p.a * Qm[v] + acc[v] * inv_pq;
      symm(Qm);
      if (last) put_q_out(Qm);
      else put(bQ, Qm, p.sQ);
    }
    if (!last) {
      // PG: H = a G + P~ G (in Gm), then PH: G = a H + P~ H
      mm(bP, bG, acc);
      __syncthreads();  // every read of G^ is done before H^ replaces it
#pragma unroll
      for (int v = 0; v < 16; ++v) Gm[v] = p.a * Gm[v] + acc[v] * inv_pg;
      symm(Gm);
      put(bG, Gm, p.sH);
      __syncthreads();
      mm(bP, bG, acc);
      __syncthreads();  // every read of H^ is done before G^ replaces it
#pragma unroll
      for (int v = 0; v < 16; ++v) Gm[v] = p.a * Gm[v] + acc[v] * inv_ph;
      symm(Gm);
      put(bG, Gm, p.sG);
      __syncthreads();
    }
  }
}

hipError_t launch_rr_fused(const RrFusedParams& p, int nmat, hipStream_t s) {
  if (nmat <= 0) return hipSuccess;
  if (p.N < 1) return hipErrorInvalidValue;
  switch (p.r_pad) {
    case 64:
      hipLaunchKernelGGL((rr_fused_kernel<64>), dim3((uint32_t)nmat), dim3(4 * 64), 0, s, p);
      break;
    case 128:
      hipLaunchKernelGGL((rr_fused_kernel<128>), dim3((uint32_t)nmat), dim3(16 * 64), 0, s, p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace muon
