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
//   direct form (eq. (2) iterated on X, scaled fp16 X): EPI_SYRK on X,
//   EPI_POLY, EPI_XUPD X' = a X + P~ X written in both layouts, EPI_XFINAL
//   the last X' applied to W as EPI_FINAL does
// Every r x r matrix of the recursion is a polynomial in G0, hence symmetric
// and commuting, so each product needs only its lower-triangle tiles and
// B^T == B for the K-contiguous operand layout.
//
// CDNA4 mapping: 256 threads = 4 wave64 in a 2 x 2 grid, each wave owns a
// (BT/2) x (BT/2) sub-tile built from 32x32x16 MFMAs (bf16 or fp16 operands,
// fp32 accumulate) or 32x32x2 fp32 MFMAs.  Operand tiles (both K-contiguous)
// are staged global -> registers -> LDS with an XOR swizzle on 16-byte chunks
// (bank conflict free for both the MFMA fragment reads and the LDS writes),
// double buffered in LDS with one barrier per K step, and up to 4 K steps
// in flight in registers.  The final product can instead take X0 itself as
// its B operand, K-major (rows of k, n contiguous; BKN): the tile is staged
// as it lies, 64-byte segments of a row XOR-swizzled by the row's low bits,
// and each 32x32x16 B fragment (eight consecutive k of one n) is two
// transposing LDS reads, so that no transposed copy of X0 is needed.  Workgroup ids are remapped so
// that consecutive tiles share an XCD's L2.  This kernel serves the fp32 path
// and tiles below 256; 256-tile 16-bit products use gemm_dma.hip.
#include "common.hpp"
#include "gemm_epilogue.hpp"
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


// Global -> register stage of one operand tile (BT rows x KT k, K-contiguous).
template <int ES, int BT>
__device__ __forceinline__ void load_tile(const char* __restrict__ base, int ld, int row0, int k0,
                                          int tid, u32x4* r) {
  constexpr int LOADS = BT * 8 / 256;
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int q = tid + 256 * i;
    const int row = q >> 3, ch = q & 7;
    r[i] = *(const u32x4*)(base + ((size_t)(row0 + row) * ld + k0) * ES + ch * 16);
  }
}

// Register -> LDS stage (K-contiguous, 16-byte chunks swizzled).
template <int BT>
__device__ __forceinline__ void store_tile(u32x4* s, const u32x4* r, int tid) {
  constexpr int LOADS = BT * 8 / 256;
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int q = tid + 256 * i;
    const int row = q >> 3, ch = q & 7;
    s[row * 8 + (ch ^ swz(row))] = r[i];
  }
}

// K-major operand tile (KT = 64 rows of k, BT elements of n each, 16-bit):
// the 64-byte segments of row k are permuted by segk(k), so that the four
// consecutive rows one transposing read touches (same columns) fall in four
// different 64-byte bank groups.
template <int BT>
__device__ __forceinline__ int segk(int k) {
  static_assert(BT == 64 || BT == 128, "K-major tiles are 64 or 128 wide");
  return BT == 64 ? ((k >> 1) & 1) : (k & 3);
}

template <int BT>
__device__ __forceinline__ void load_tile_kn(const char* __restrict__ base, int ld, int col0, int k0,
                                             int tid, u32x4* r) {
  constexpr int LOADS = BT * 8 / 256;
  constexpr int CPR = BT / 8;  // 16-byte chunks per row of k
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int q = tid + 256 * i;
    const int row = q / CPR, ch = q % CPR;
    r[i] = *(const u32x4*)(base + ((size_t)(k0 + row) * ld + col0) * 2 + ch * 16);
  }
}

template <int BT>
__device__ __forceinline__ void store_tile_kn(u32x4* s, const u32x4* r, int tid) {
  constexpr int LOADS = BT * 8 / 256;
  constexpr int CPR = BT / 8;
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int q = tid + 256 * i;
    const int row = q / CPR, ch = q % CPR;
    s[row * CPR + (ch ^ (segk<BT>(row) << 2))] = r[i];
  }
}

// B fragments of 32x32x16 MFMAs (lane: n = l32, k = 16 s + 8 h .. +7) from a
// K-major tile: lane i of each 16-lane group addresses row k + i / 4 and
// columns 4 (i % 4) .. +3 of its 16-column half; two reads give k .. k+3 and
// k+4 .. k+7.  A lane reads rows kl + 16 s + 4 e (kl = 8 h + i / 4, e = 0, 1):
// adding multiples of 4 leaves segk unchanged, so each lane's byte offset
// for the block of columns n0 is fixed (kn_lane_offset) and the step s and
// the half e are immediates.  n0 is a multiple of 32 (its chunk index a
// multiple of 4), so the segment permutation and the lane's chunk within the
// segment (0..3) combine by addition.
template <int BT>
__device__ __forceinline__ int kn_lane_offset(int n0, int lane) {
  const int h = lane >> 5, g = (lane >> 4) & 1, i = lane & 15;
  const int kl = 8 * h + (i >> 2);
  const int ch = (((n0 >> 3) ^ (segk<BT>(kl) << 2)) + 2 * g + ((i & 3) >> 1));
  return kl * 2 * BT + ch * 16 + 8 * (i & 1);
}

template <int BT>
__device__ __forceinline__ u32x4 frag_kn(const char* lp, int s) {
  const uint2 lo = tr_read(lp + s * 32 * BT);
  const uint2 hi = tr_read(lp + s * 32 * BT + 8 * BT);
  u32x4 f;
  f[0] = lo.x;
  f[1] = lo.y;
  f[2] = hi.x;
  f[3] = hi.y;
  return f;
}

// (the K-major 128-wide final product is held to two waves per SIMD, which
// the other 128-wide 16-bit variants reach by themselves)
template <int KIND, int BT, int EPI, bool F32PATH, bool BKN = false>
__global__ void __launch_bounds__(256, (BKN && BT == 128) ? 2 : 1) gemm_kernel(const GemmParams p) {
  static_assert(!BKN || (EPI == EPI_FINAL && KIND == K_BF16), "K-major B: bf16 final product only");
  constexpr int ES = (KIND == K_F32) ? 4 : 2;
  constexpr int E = 16 / ES;           // elements per 16-byte chunk
  constexpr int KT = 128 / ES;         // K elements per step (8 chunks per row)
  constexpr int WT = BT / 2;           // wave sub-tile
  constexpr int F = WT / 32;           // 32x32 MFMA blocks per wave dimension
  constexpr int LOADS = BT * 8 / 256;  // 16-byte chunks per thread
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

  // K steps in flight: a ring of D register stages ahead of the LDS double
  // buffer (long-K products on few tiles, e.g. a 128 x 3584 SYRK: 336
  // workgroups over 56 K steps, otherwise pay one memory latency per step)
  constexpr int D = BT == 64 ? 4 : (BT == 128 ? 2 : 1);
  u32x4 ra[D][LOADS];
  u32x4 rb[D][LOADS];

  f32x16 acc[F][F];
#pragma unroll
  for (int i = 0; i < F; ++i)
#pragma unroll
    for (int j = 0; j < F; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int nk = p.Kdim / KT;
#pragma unroll
  for (int u = 0; u < D; ++u)
    if (u < nk) {
      load_tile<ES, BT>(Ab, p.lda, row0A, u * KT, tid, ra[u]);
      if constexpr (BKN) load_tile_kn<BT>(Bb, p.ldb, row0B, u * KT, tid, rb[u]);
      else load_tile<ES, BT>(Bb, p.ldb, row0B, u * KT, tid, rb[u]);
    }

  // Final product (and the direct form's last X') on 64-wide 16-bit tiles: the
  // W values (and the a X term of XFINAL) that this thread updates in the
  // epilogue's row pass, four groups of four, are requested before the K
  // loop, so their memory latency overlaps the loop instead of following it
  // (the small buckets that take this tile run a few K steps, and the tile's
  // time was mostly these loads' latency).
  constexpr bool FIN = EPI == EPI_FINAL || EPI == EPI_XFINAL;
  constexpr bool PRE = FIN && BT == 64 && !F32PATH;
  constexpr int FTPR = BT / 4;       // threads per tile row in the row pass
  constexpr int FRPI = 256 / FTPR;   // tile rows per row-pass iteration
  constexpr int FNE = PRE ? RR / FRPI : 1;
  float4 wpre[FNE], xpre[FNE];
  bool wok[FNE];
  if constexpr (PRE) {
    const MatPtrs mp = p.table[mat];
#pragma unroll
    for (int e = 0; e < FNE; ++e) {
      const int gi = row0A + e * FRPI + tid / FTPR, gj = row0B + (tid % FTPR) * 4;
      wok[e] = p.vec && gi < p.out_rows && gj + 4 <= p.out_cols;
      wpre[e] = wok[e] ? nt_load4(mp.W + (size_t)gi * p.out_cols + gj) : make_float4(0.f, 0.f, 0.f, 0.f);
      if constexpr (EPI == EPI_XFINAL)
        xpre[e] = ld4h(p.Xid, (size_t)mat * p.y_stride + (size_t)gi * p.ldyn + gj);
    }
  }
  int kn_off[F];
#pragma unroll
  for (int f = 0; f < F; ++f) {
    if constexpr (BKN) kn_off[f] = kn_lane_offset<BT>(wn * WT + f * 32, lane);
    else kn_off[f] = 0;
  }
  store_tile<BT>(smem[0][0], ra[0], tid);
  if constexpr (BKN) store_tile_kn<BT>(smem[0][1], rb[0], tid);
  else store_tile<BT>(smem[0][1], rb[0], tid);
  __syncthreads();

  // ring slot u holds K step k0 + u; unrolled by D so that every step's
  // register slot is static
#pragma unroll 1
  for (int k0 = 0; k0 < nk; k0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int kt = k0 + u;
      if (kt < nk) {
        // step kt is in LDS: its slot takes step kt + D
        if (kt + D < nk) {
          load_tile<ES, BT>(Ab, p.lda, row0A, (kt + D) * KT, tid, ra[u]);
          if constexpr (BKN) load_tile_kn<BT>(Bb, p.ldb, row0B, (kt + D) * KT, tid, rb[u]);
          else load_tile<ES, BT>(Bb, p.ldb, row0B, (kt + D) * KT, tid, rb[u]);
        }
        const u32x4* sA = smem[kt & 1][0];
        const u32x4* sB = smem[kt & 1][1];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int ch = 2 * s + h;
          u32x4 af[F], bfr[F];
#pragma unroll
          for (int f = 0; f < F; ++f) {
            const int ra_ = wm * WT + f * 32 + l32;
            af[f] = sA[ra_ * 8 + (ch ^ swz(ra_))];
            if constexpr (BKN) {
              bfr[f] = frag_kn<BT>((const char*)sB + kn_off[f], s);
            } else {
              const int rb_ = wn * WT + f * 32 + l32;
              bfr[f] = sB[rb_ * 8 + (ch ^ swz(rb_))];
            }
          }
#pragma unroll
          for (int i = 0; i < F; ++i)
#pragma unroll
            for (int j = 0; j < F; ++j) mfma16B<KIND>(af[i], bfr[j], acc[i][j]);
        }
        if (kt + 1 < nk) {
          store_tile<BT>(smem[(kt + 1) & 1][0], ra[(u + 1) % D], tid);
          if constexpr (BKN) store_tile_kn<BT>(smem[(kt + 1) & 1][1], rb[(u + 1) % D], tid);
          else store_tile<BT>(smem[(kt + 1) & 1][1], rb[(u + 1) % D], tid);
        }
        __syncthreads();
      }
    }
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
    if constexpr (EPI == EPI_FINAL || EPI == EPI_XFINAL) {
      // four consecutive columns per thread: one 16-byte W load and store
      // (W is touched once; the fp32 tile row is read from LDS as scalars).
      // XFINAL (the direct form's last X' = a X + P~ X, X and P~ scaled
      // fp16): acc + a sP X^ is sP sX X', so O = (acc + a sP X^) / (sP sX)
      constexpr int TPR = FTPR;          // threads per tile row
      constexpr int RPI = FRPI;          // tile rows per iteration
      const float inv = EPI == EPI_FINAL ? p.inv_norm[mat] : 1.0f / (p.sP * p.sX);
#pragma unroll 4
      for (int e = 0; e < RR / RPI; ++e) {
        const int il = e * RPI + tid / TPR, jl = (tid % TPR) * 4;
        const float* sr = stile + il * EPI_LD + jl;
        float4 acc4 = make_float4(sr[0], sr[1], sr[2], sr[3]);
        if constexpr (PRE) {
          // W (and X) were requested before the K loop
          if constexpr (EPI == EPI_XFINAL) acc4 = f4_axpy(1.0f, acc4, p.a * p.sP, xpre[e]);
          if (wok[e]) {
            const MatPtrs mp = p.table[mat];
            const float4 o = make_float4(acc4.x * inv, acc4.y * inv, acc4.z * inv, acc4.w * inv);
            const size_t idx = (size_t)(gr0 + il) * p.out_cols + row0B + jl;
            nt_store4(mp.W + idx, f4_axpy(p.decay, wpre[e], -p.step, o));
            if (mp.O) nt_store4(mp.O + idx, o);
          } else {
            epilogue_final4(p, mat, gr0 + il, row0B + jl, acc4, inv);
          }
        } else {
          if constexpr (EPI == EPI_XFINAL) {
            const float4 x = ld4h(p.Xid, (size_t)mat * p.y_stride + (size_t)(gr0 + il) * p.ldyn + row0B + jl);
            acc4 = f4_axpy(1.0f, acc4, p.a * p.sP, x);
          }
          epilogue_final4(p, mat, gr0 + il, row0B + jl, acc4, inv);
        }
      }
    } else if constexpr (EPI == EPI_XUPD) {
      // X'^ = a X^ + acc / sP in the scaled fp16 units of X^ (acc = sP sX P~ X):
      // the row pass writes the natural layout Yn (X^ from Xid), the column
      // pass the transposed Yt (X^ from the B operand, X^T), four
      // consecutive elements per thread in both
      const size_t yb = (size_t)mat * p.y_stride;
      const float inv_sp = 1.0f / p.sP;
      constexpr int TPR = BT / 4;     // threads per tile row
      constexpr int RPI = 256 / TPR;  // tile rows per iteration
#pragma unroll 2
      for (int e = 0; e < RR / RPI; ++e) {
        const int il = e * RPI + tid / TPR, jl = (tid % TPR) * 4;
        const float* sr = stile + il * EPI_LD + jl;
        const size_t o = yb + (size_t)(gr0 + il) * p.ldyn + row0B + jl;
        const float4 v = f4_axpy(p.a, ld4h(p.Xid, o), inv_sp, make_float4(sr[0], sr[1], sr[2], sr[3]));
        st4h(p.Yn, o, v, 1.0f, false, 0, 4);
      }
      constexpr int TPC = RR / 4;     // threads per tile column
      constexpr int CPI = 256 / TPC;  // tile columns per iteration
#pragma unroll 2
      for (int e = 0; e < BT / CPI; ++e) {
        const int il = (tid % TPC) * 4, jl = e * CPI + tid / TPC;
        const float* sc = stile + il * EPI_LD + jl;
        const size_t o = yb + (size_t)(row0B + jl) * p.ldyt + gr0 + il;
        const float4 xt = ld4h(p.B, (size_t)mat * p.b_stride + (size_t)(row0B + jl) * p.ldb + gr0 + il);
        const float4 v = f4_axpy(p.a, xt, inv_sp, make_float4(sc[0], sc[EPI_LD], sc[2 * EPI_LD], sc[3 * EPI_LD]));
        st4h(p.Yt, o, v, 1.0f, false, 0, 4);
      }
    } else {
      // row pass (lower triangle incl. the diagonal): four consecutive
      // columns of a tile row per thread
      constexpr int TPR = BT / 4;     // threads per tile row
      constexpr int RPI = 256 / TPR;  // tile rows per iteration
#pragma unroll 2
      for (int e = 0; e < RR / RPI; ++e) {
        const int il = e * RPI + tid / TPR, jl = (tid % TPR) * 4;
        const int gi = gr0 + il, gj = row0B + jl;
        const int khi = min(max(gi - gj + 1, 0), 4);
        if (khi > 0) {
          const float* sr = stile + il * EPI_LD + jl;
          epilogue4<EPI, F32PATH>(p, mat, prod, gi, gj, make_float4(sr[0], sr[1], sr[2], sr[3]), 0,
                                  khi);
        }
      }
      // mirror pass (strictly lower part, stored at (gj, gi)): four
      // consecutive tile rows of one tile column per thread, so the stores
      // run along the mirrored row
      constexpr int TPC = RR / 4;     // threads per tile column
      constexpr int CPI = 256 / TPC;  // tile columns per iteration
#pragma unroll 2
      for (int e = 0; e < BT / CPI; ++e) {
        const int il = (tid % TPC) * 4, jl = e * CPI + tid / TPC;
        const int gi = gr0 + il, gj = row0B + jl;
        const int klo = min(max(gj - gi + 1, 0), 4);
        if (klo < 4) {
          const float* sc = stile + il * EPI_LD + jl;
          epilogue4<EPI, F32PATH>(p, mat, prod, gj, gi,
                                  make_float4(sc[0], sc[EPI_LD], sc[2 * EPI_LD], sc[3 * EPI_LD]), klo,
                                  4);
        }
      }
    }
    __syncthreads();
  }
}

template <int KIND, int BT, int EPI, bool F32PATH, bool BKN = false>
static hipError_t launch_one(const GemmParams& p, int nmat, hipStream_t s) {
  const uint64_t blocks = (uint64_t)nmat * p.tiles_per_prod * p.products;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffull) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_kernel<KIND, BT, EPI, F32PATH, BKN>), dim3((uint32_t)blocks), dim3(256), 0,
                     s, p);
  return hipGetLastError();
}

template <int BT, bool F32PATH>
static hipError_t launch_bt(const GemmParams& p, int epi, int nmat, hipStream_t s) {
  constexpr int KX = F32PATH ? K_F32 : K_BF16;  // X0 / final operands
  constexpr int KR = F32PATH ? K_F32 : K_F16;   // r x r recursion operands
  if constexpr (!F32PATH) {
    // direct form: scaled fp16 X in every product
    switch (epi) {
      case EPI_SYRK:
        if (p.xkind) return launch_one<K_F16, BT, EPI_SYRK, false>(p, nmat, s);
        break;
      case EPI_XUPD: return launch_one<K_F16, BT, EPI_XUPD, false>(p, nmat, s);
      case EPI_XFINAL: return launch_one<K_F16, BT, EPI_XFINAL, false>(p, nmat, s);
      default: break;
    }
  }
  if (p.b_kn) {
    // K-major B: the 16-bit final product on 64- and 128-wide tiles only
    if constexpr (!F32PATH && BT <= 128)
      if (epi == EPI_FINAL) return launch_one<K_BF16, BT, EPI_FINAL, false, true>(p, nmat, s);
    return hipErrorInvalidValue;
  }
  switch (epi) {
    case EPI_SYRK: return launch_one<KX, BT, EPI_SYRK, F32PATH>(p, nmat, s);
    case EPI_POLY: return launch_one<KR, BT, EPI_POLY, F32PATH>(p, nmat, s);
    case EPI_PQPG: return launch_one<KR, BT, EPI_PQPG, F32PATH>(p, nmat, s);
    case EPI_PH: return launch_one<KR, BT, EPI_PH, F32PATH>(p, nmat, s);
    case EPI_FINAL: return launch_one<KX, BT, EPI_FINAL, F32PATH>(p, nmat, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm(const GemmParams& p, int epi, int op, int bt, int nmat, hipStream_t s) {
  if (op == OP_BF16) {
    switch (bt) {
      case 64: return launch_bt<64, false>(p, epi, nmat, s);
      case 128: return launch_bt<128, false>(p, epi, nmat, s);
      case 256: return launch_bt<256, false>(p, epi, nmat, s);
    }
  } else if (op == OP_F32) {
    switch (bt) {
      case 64: return launch_bt<64, true>(p, epi, nmat, s);
      case 128: return launch_bt<128, true>(p, epi, nmat, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace muon
