// The whole direct-form Newton-Schulz iteration ("Infra Optimizers" eq. (2)
// iterated on X: A = X X^T, P~ = b A + c A^2, X' = a X + P~ X) and the weight
// update ("Infra Optimizers" eq. (4); "Scaling Muon for Diffusion
// Transformers" 2.1) in one launch, one workgroup per matrix, for buckets of
// padded squares with r_pad = c_pad in {128, 256} on the 16-bit path.  With
// small tiles each of the 3 N products of such a bucket is a short launch
// bound by latency (64 x 256^2: ~20 us per launch, 15 launches); here they
// run back to back inside the workgroup and the r x r intermediates never
// leave LDS.
//
// Arithmetic (the small-tile kernels' direct-form epilogues, gemm.hip, with
// the same operand formats and power-of-two scales; X^ = X sX in fp16, both
// layouts, cast by the workgroup itself from the prep pass's bf16 U and the
// norm), per iteration
//   SYRK  A^ = fp16(acc sG / sX^2)                    (A = X X^T)
//   POLY  P~ = b A^ / sG + c acc / sG^2,  P^ = fp16(P~ sP)
//   XUPD  X'^ = fp16(a X^ + acc / sP), both layouts
// and for the last iteration, in place of XUPD's stores,
//   O = (acc + a sP X^) / (sP sX),  W <- decay W - step O   (O_out too if set).
// One difference from the launch sequence: POLY's b A term takes A from its
// fp16 copy A^ (resident in LDS) instead of an fp32 copy; that adds a
// rounding of 2^-11 relative to A, the order of P^'s own fp16 rounding.
//
// Layout: 16 wave64 in 4 x 4, wave (wr, wc) owning the BS x BS output block
// (BS = r_pad / 4) of every product as (BS / 16)^2 blocks of 16x16x32 fp16
// MFMAs (four waves per SIMD hide each other's LDS and barrier waits).
// LDS holds one full r_pad x r_pad fp16 matrix (A^, then P^ in place; 128 KB
// for r_pad = 256) in the 256-tile kernel's operand format (32-K sub-blocks
// of 64-byte rows, 16-byte chunks swizzled by row bit 2, conflict free for
// the fragment reads) and two 16-KB stages through which X^ (SYRK) and X^T
// (XUPD's B operand) stream from global memory by direct global -> LDS
// loads.  Lane (q4, c16) of an MFMA block holds four consecutive rows of one
// column, so A^ and P^ are stored as their transposes (the same matrices,
// symmetric) with 8-byte writes; X'^ goes to global memory through LDS in
// the natural layout (16-byte rows) and straight from the accumulators in
// the transposed one, and the W update through LDS in two rounds of fp32.
#include "common.hpp"
#include "kernels.h"

namespace muon {

namespace {

constexpr int DF_ROWB = 64;  // bytes of one row of a 32-K sub-block

typedef __attribute__((address_space(3))) void df_lds_ptr_t;
typedef const __attribute__((address_space(1))) void df_gbl_ptr_t;

// s_waitcnt immediate (gfx9 encoding): vmcnt in [3:0] and [15:14], expcnt
// [6:4] left at its maximum, lgkmcnt [11:8].
constexpr int df_wait_imm(int vm, int lgkm) {
  return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 15) << 8);
}

// 16-byte chunk swizzle of a 64-byte row: conflict free for the 16x16x32
// fragment reads (16 rows x 4 chunks per instruction), as in gemm_dma.hip
__device__ __forceinline__ int df_swz(int row) { return ((row >> 2) & 1) << 1; }

__device__ __forceinline__ void df_mfma(const u32x4& a, const u32x4& b, f32x4& c) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                             0, 0, 0);
}

__device__ __forceinline__ uint32_t df_h2(float a, float b) {
  return (uint32_t)f32_to_f16_bits(a) | ((uint32_t)f32_to_f16_bits(b) << 16);
}

__device__ __forceinline__ float df_h(uint32_t w, int hi) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(hi ? (w >> 16) : w));
}

// A copy of v that the compiler cannot see through: addresses derived from
// it are computed where they are used instead of being hoisted out of the
// iteration loop (one address per output block and buffer would otherwise
// stay live across every product).
__device__ __forceinline__ int df_fresh(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

}  // namespace

template <int RP>
__global__ void __launch_bounds__(1024, 1) direct_fused_kernel(const DirectFusedParams p) {
  constexpr int BS = RP / 4;              // wave block
  constexpr int FB = BS / 16;             // 16 x 16 MFMA blocks per wave dimension
  constexpr int SUB = RP * DF_ROWB;       // one 32-K sub-block of an RP-row operand
  constexpr int FULL = (RP / 32) * SUB;   // a whole RP x RP fp16 matrix
  constexpr int SPS = 256 / RP;           // sub-blocks per stage: 16 KB, one DMA per wave
  constexpr int STG = SPS * SUB;
  constexpr int NST = RP / 32 / SPS;      // stages per streamed product
  static_assert(STG == 16384 && FULL + 2 * STG <= 163840, "LDS budget");
  __shared__ __attribute__((aligned(1024))) char smem[FULL + 2 * STG];
  char* full = smem;
  char* stg = smem + FULL;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 2, wc = wave & 3;
  const int q4 = lane >> 4, c16 = lane & 15;
  const int mat = blockIdx.x;
  const size_t xo = (size_t)mat * p.x_stride;

  // byte offset of element (row, k) of an RP-row operand in the sub-block
  // format (k a multiple of 4 for the 8-byte accesses below)
  auto el = [](int row, int k) {
    return (k >> 5) * SUB + row * DF_ROWB + ((((k & 31) >> 3) ^ df_swz(row)) << 4) + ((k & 7) << 1);
  };
  // fragment offset in a sub-block: the row's swizzle depends only on its
  // low 4 bits (block rows start at multiples of 16), so block i / j adds a
  // constant 16 rows
  const int offA = (wr * BS + c16) * DF_ROWB + ((q4 ^ df_swz(c16)) << 4);
  const int offB = (wc * BS + c16) * DF_ROWB + ((q4 ^ df_swz(c16)) << 4);

  f32x4 acc[FB][FB];
  auto zero = [&]() {
#pragma unroll
    for (int i = 0; i < FB; ++i)
#pragma unroll
      for (int j = 0; j < FB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  // MFMAs of one 32-K sub-block: A fragments at a + i 16 rows, B at b + j 16
  auto mma = [&](const char* a, const char* b) {
    u32x4 bf[FB];
#pragma unroll
    for (int j = 0; j < FB; ++j) bf[j] = *(const u32x4*)(b + j * 16 * DF_ROWB);
#pragma unroll
    for (int i = 0; i < FB; ++i) {
      const u32x4 af = *(const u32x4*)(a + i * 16 * DF_ROWB);
#pragma unroll
      for (int j = 0; j < FB; ++j) df_mfma(af, bf[j], acc[i][j]);
    }
  };
  // Stream operand S (RP x RP, K-contiguous, ld RP) through the two stages:
  // each stage is one 1-KB DMA per wave (16 rows of one sub-block).  afull:
  // the A operand is the resident full matrix; else both operands are S.
  auto stream = [&](const uint16_t* S, bool afull) {
    auto issue = [&](int st) {
      const int sub = wave / (RP / 16), rg = wave % (RP / 16);
      const int row = rg * 16 + (lane >> 2);
      const int e = df_fresh(row * RP + (st * SPS + sub) * 32 + (((lane & 3) ^ df_swz(row)) << 3));
      char* dst = stg + (st & 1) * STG + sub * SUB + rg * 1024;
      __builtin_amdgcn_global_load_lds((df_gbl_ptr_t*)(S + e), (df_lds_ptr_t*)dst, 16, 0, 0);
    };
    zero();
    issue(0);
    if (NST > 1) issue(1);
#pragma unroll 1
    for (int st = 0; st < NST; ++st) {
      if (st + 1 < NST) __builtin_amdgcn_s_waitcnt(df_wait_imm(1, 15));
      else __builtin_amdgcn_s_waitcnt(df_wait_imm(0, 15));
      __syncthreads();
      const char* sb = stg + (st & 1) * STG;
#pragma unroll
      for (int s = 0; s < SPS; ++s) {
        const char* bop = sb + s * SUB + offB;
        const char* aop = afull ? full + (st * SPS + s) * SUB + offA : sb + s * SUB + offA;
        mma(aop, bop);
      }
      __syncthreads();  // every read of this stage's buffer is done
      if (st + 2 < NST) issue(st + 2);
    }
  };

  // 1 / ||U|| from the prep pass's partial sums, reduced exactly as the
  // finalize kernel does (threads 0..255 in fp64, a wave-level butterfly,
  // then the four wave sums in order), so that the value agrees bit for bit
  // and the launch sequence needs no finalize launch for these buckets;
  // the LDS it uses is not touched again before the cast's closing barrier
  float inv_norm;
  {
    double* red = reinterpret_cast<double*>(smem);
    if (tid < 256) {  // waves 0..3, whole
      const float* part = p.partials + (size_t)mat * p.blocks_per_mat;
      double s = 0.0;
      for (int i = tid; i < p.blocks_per_mat; i += 256) s += (double)part[i];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
      if (lane == 0) red[wave] = s;
    }
    __syncthreads();
    const double tot = red[0] + red[1] + red[2] + red[3];
    inv_norm = tot == 0.0 ? 0.0f : (tot < INFINITY ? (float)(1.0 / sqrt(tot)) : NAN);
  }

  // X^ = fp16(U sX / ||U||) in place over both layouts of U (bf16 from the
  // prep pass; the cast pass of the launch sequence, done here by the
  // matrix's own workgroup)
  {
    // every load of both layouts in flight at once: U was written by the
    // prep pass well before and comes from memory, and one chunk at a time
    // paid that latency 2 RP^2 / 8192 times per thread
    constexpr int CPT = RP * RP / 8 / 1024;  // 16-byte chunks per thread per layout
    const float sc = inv_norm * p.sX;
    uint32_t* bl[2] = {(uint32_t*)((uint16_t*)p.Xn[0] + xo), (uint32_t*)((uint16_t*)p.Xt[0] + xo)};
    u32x4 v[2][CPT];
#pragma unroll
    for (int lay = 0; lay < 2; ++lay)
#pragma unroll
      for (int t = 0; t < CPT; ++t) v[lay][t] = *(const u32x4*)(bl[lay] + 4 * (tid + 1024 * t));
#pragma unroll
    for (int lay = 0; lay < 2; ++lay)
#pragma unroll
      for (int t = 0; t < CPT; ++t) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          v[lay][t][q] = df_h2(__uint_as_float(v[lay][t][q] << 16) * sc,
                               __uint_as_float(v[lay][t][q] & 0xffff0000u) * sc);
        *(u32x4*)(bl[lay] + 4 * (tid + 1024 * t)) = v[lay][t];
      }
    __syncthreads();
  }

  // accumulator element e of block (i, j): row wr*BS + i*16 + 4*q4 + e,
  // column wc*BS + j*16 + c16
  for (int k = 0; k < p.N; ++k) {
    const int cur = k & 1, nx = cur ^ 1;
    const uint16_t* Xn = (const uint16_t*)p.Xn[cur] + xo;  // X^, RP x RP
    const uint16_t* Xt = (const uint16_t*)p.Xt[cur] + xo;  // X^T

    // SYRK: A^ = fp16(X^ X^T sG / sX^2), stored as its transpose: lane's
    // rows r0..r0+3 of column c are elements r0..r0+3 of LDS row c
    stream(Xn, false);
    {
      const float sc = p.syrk_scale * p.sG;
      const int rb = df_fresh(wr * BS + 4 * q4), cb = df_fresh(wc * BS + c16);
#pragma unroll
      for (int i = 0; i < FB; ++i)
#pragma unroll
        for (int j = 0; j < FB; ++j) {
          const f32x4 a = acc[i][j];
          *(uint2*)(full + el(cb + j * 16, rb + i * 16)) =
              make_uint2(df_h2(a[0] * sc, a[1] * sc), df_h2(a[2] * sc, a[3] * sc));
        }
    }
    __syncthreads();

    // POLY: P~ = b A + c A^2, both operands A^ from LDS; written in place
    // (each lane rewrites the A^ values it reads for the b A term)
    zero();
#pragma unroll 1
    for (int s = 0; s < RP / 32; ++s) mma(full + s * SUB + offA, full + s * SUB + offB);
    __syncthreads();  // every fragment read of A^ is done
    {
      const float inv_g = 1.0f / p.sG, inv_gg = inv_g * inv_g;
      const int rb = df_fresh(wr * BS + 4 * q4), cb = df_fresh(wc * BS + c16);
#pragma unroll
      for (int i = 0; i < FB; ++i)
#pragma unroll
        for (int j = 0; j < FB; ++j) {
          uint2* q = (uint2*)(full + el(cb + j * 16, rb + i * 16));
          const uint2 g = *q;
          float pt[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            pt[e] = p.b * (df_h(e < 2 ? g.x : g.y, e & 1) * inv_g) + p.c * (acc[i][j][e] * inv_gg);
          *q = make_uint2(df_h2(pt[0] * p.sP, pt[1] * p.sP), df_h2(pt[2] * p.sP, pt[3] * p.sP));
        }
    }
    __syncthreads();

    // X' = a X + P~ X: A = P^ (resident), B = X^T streamed (row c of X^T is
    // column c of X)
    stream(Xt, true);
    const int rb = df_fresh(wr * BS + 4 * q4), cb = df_fresh(wc * BS + c16);
    if (k < p.N - 1) {
      // X'^ = a X^ + acc / sP: the transposed layout straight from the
      // accumulators (8 bytes per lane and block), the natural one through
      // LDS (free after the product) as 16-byte rows
      uint16_t* Yn = (uint16_t*)p.Xn[nx] + xo;
      uint16_t* Yt = (uint16_t*)p.Xt[nx] + xo;
      uint16_t* nat = (uint16_t*)smem;  // RP x RP, row-major, pitch NP
      constexpr int NP = RP + 8;
      static_assert(RP * NP * 2 <= FULL + 2 * STG, "natural staging fits");
      const float inv_sp = 1.0f / p.sP;
#pragma unroll
      for (int i = 0; i < FB; ++i)
#pragma unroll
        for (int j = 0; j < FB; ++j) {
          const int r0 = rb + i * 16, c = cb + j * 16;
          const uint2 xw = *(const uint2*)(Xt + c * RP + r0);  // X^(r0..r0+3, c)
          uint16_t hv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            hv[e] = f32_to_f16_bits(p.a * df_h(e < 2 ? xw.x : xw.y, e & 1) + acc[i][j][e] * inv_sp);
          *(uint2*)(Yt + c * RP + r0) =
              make_uint2((uint32_t)hv[0] | ((uint32_t)hv[1] << 16), (uint32_t)hv[2] | ((uint32_t)hv[3] << 16));
#pragma unroll
          for (int e = 0; e < 4; ++e) nat[(r0 + e) * NP + c] = hv[e];
        }
      __syncthreads();
      // rows of X'^: RP / 8 16-byte chunks per row, 1024 threads
      for (int t = tid; t < RP * (RP / 8); t += 1024) {
        const int r = t / (RP / 8), ch = t % (RP / 8);
        *(uint4*)(Yn + r * RP + ch * 8) = *(const uint4*)(nat + r * NP + ch * 8);
      }
      __syncthreads();
    } else {
      // X_N's block is W's block: O = (acc + a sP X^) / (sP sX) staged as
      // fp32 through LDS in two rounds of RP / 2 rows, then W <- decay W -
      // step O on the true m x n extent, four columns per thread
      const MatPtrs mp = p.table[mat];
      const float inv = 1.0f / (p.sP * p.sX);
      const float asp = p.a * p.sP;
      float* ost = (float*)smem;  // (RP / 2) x RP fp32, pitch OP
      constexpr int OP = RP + 4;
      static_assert((RP / 2) * OP * 4 <= FULL + 2 * STG, "O staging fits");
#pragma unroll
      for (int round = 0; round < 2; ++round) {
        if (wr / 2 == round) {
#pragma unroll
          for (int i = 0; i < FB; ++i)
#pragma unroll
            for (int j = 0; j < FB; ++j) {
              const int r0 = rb + i * 16, c = cb + j * 16;
              const uint2 xw = *(const uint2*)(Xt + c * RP + r0);
#pragma unroll
              for (int e = 0; e < 4; ++e)
                ost[(r0 + e - round * (RP / 2)) * OP + c] =
                    (acc[i][j][e] + asp * df_h(e < 2 ? xw.x : xw.y, e & 1)) * inv;
            }
        }
        __syncthreads();
        for (int t = tid; t < (RP / 2) * (RP / 4); t += 1024) {
          const int rl = t / (RP / 4), c = (t % (RP / 4)) * 4;
          const int r = round * (RP / 2) + rl;
          if (r >= p.m || c >= p.n) continue;
          const float4 o = *(const float4*)(ost + rl * OP + c);
          const size_t idx = (size_t)r * p.n + c;
          if (p.vec && c + 4 <= p.n) {
            const float4 w = *(const float4*)(mp.W + idx);
            *(float4*)(mp.W + idx) = make_float4(p.decay * w.x - p.step * o.x, p.decay * w.y - p.step * o.y,
                                                 p.decay * w.z - p.step * o.z, p.decay * w.w - p.step * o.w);
            if (mp.O) *(float4*)(mp.O + idx) = o;
          } else {
            const float ov[4] = {o.x, o.y, o.z, o.w};
            for (int e = 0; e < 4 && c + e < p.n; ++e) {
              mp.W[idx + e] = p.decay * mp.W[idx + e] - p.step * ov[e];
              if (mp.O) mp.O[idx + e] = ov[e];
            }
          }
        }
        __syncthreads();
      }
    }
  }
}

hipError_t launch_direct_fused(const DirectFusedParams& p, int nmat, hipStream_t s) {
  if (nmat <= 0) return hipSuccess;
  if (p.N < 1 || p.m > p.rp || p.n > p.rp) return hipErrorInvalidValue;
  switch (p.rp) {
    case 128:
      hipLaunchKernelGGL((direct_fused_kernel<128>), dim3((uint32_t)nmat), dim3(1024), 0, s, p);
      break;
    case 256:
      hipLaunchKernelGGL((direct_fused_kernel<256>), dim3((uint32_t)nmat), dim3(1024), 0, s, p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace muon
