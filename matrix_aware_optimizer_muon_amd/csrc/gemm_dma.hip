// 256 x 256 MFMA GEMM C = A * B^T with a four-stage LDS ring filled by
// direct global->LDS loads (gfx950 global_load_lds_dwordx4), for the large
// products of the Newton-Schulz step: SYRK, the r x r recursion and the final
// product of the Gram form, and the direct form's X' = a X + P~ X (XUPD).
//
// Both operands are K-contiguous (the prep kernel writes X0 and X0^T), or,
// for the final product and X' of buckets kept in one layout, B is X0 (X)
// itself, K-major, read through gfx950's transposing LDS loads (BKN).
// 8 wave64 (two per SIMD) in 2 x 4, each owning 128 x 64 = 8 x 4 blocks of
// 16x16x32 MFMAs (128 fp32 accumulators), so one wave's barrier, DMA-issue
// and LDS waits overlap the other's MFMAs (a 4-wave 128 x 128 variant serves
// SYRK and the final product when a tuning hint asks for it).  A stage holds
// 32 K elements of both 256-row operand tiles (2 x 16 KB), one MFMA K step;
// every 1-KB DMA instruction lands lane L at LDS offset 16*L of its block, so
// the 16-byte chunk swizzle is applied on the global side.  Up to four stages
// are in flight; each K step has one barrier, placed so that it both
// publishes the next stage and retires the reads of the current one.  The
// stage's MFMAs run in two halves by block row: the fragments of the second
// half are read from LDS while the first half's MFMAs run, and the next
// stage's first-half fragments while the second half's run.
//
// 16x16x32 rather than 32x32x16 MFMAs: the same issue rate per flop with half
// the accumulator traffic per instruction; measured on the final product
// (same box, sustained): 1046 -> 1084 TFLOP/s over eight 3584 x 18944
// products, 970 -> 1028 over one.
#include "common.hpp"
#include "gemm_epilogue.hpp"
#include "kernels.h"

namespace muon {

namespace {

constexpr int DT = 256;                        // tile rows / cols
constexpr int DBK = 32;                        // K elements per stage
constexpr int DSTAGES = 4;
constexpr int ROWB = DBK * 2;                  // bytes of one tile row per stage
constexpr int OPB = DT * ROWB;                 // one operand per stage: 16 KB
constexpr int STAGEB = 2 * OPB;                // 32 KB

// s_waitcnt immediate (gfx9 encoding): vmcnt in [3:0] and [15:14], expcnt
// [6:4] left at its maximum, lgkmcnt [11:8].
constexpr int wait_imm(int vm, int lgkm) {
  return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 15) << 8);
}

typedef __attribute__((address_space(3))) void lds_ptr_t;
typedef const __attribute__((address_space(1))) void gbl_ptr_t;

// 16-byte chunk swizzle of a 64-byte row for the MFMA fragment reads (lane
// l reads row base + (l & 15), chunk l >> 4).  Chosen by measurement on
// gfx950 (bank-conflict counter of a one-wave ds_read_b128 probe over all
// 1024 GF(2)-linear 2-bit functions of the row's low five bits): flipping
// chunk bit 1 with row bit 2 is conflict free, while (r ^ (r >> 3)) & 3,
// (r >> 2) & 3 and (r ^ (r >> 2)) & 3 cost four conflict cycles per read.
__device__ __forceinline__ int swz4(int row) { return ((row >> 2) & 1) << 1; }

// Slot of 8-byte chunk q (tile rows 4q..4q+3) in staged column c of the
// 16-bit epilogue (64 slots per 512-byte column): a bijection per column,
// conflict free for the staging writes (16 columns x 4 chunks per
// instruction), the row reads (columns 4L + k of one chunk) and the mirror
// reads (one whole column per half wave, as aligned 16-byte pairs).
__device__ __forceinline__ int slot16(int c, int q) {
  const int h = ((((c >> 2) & 3) << 2) | ((c & 3) << 4)) ^ ((c >> 4) & 3) ^ (((c >> 6) & 3) << 4);
  return q ^ h;
}

__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// K-major operand stages (32 rows of k, 512 bytes = the tile's 256 columns
// each): 16-byte chunk c of row k is stored at chunk c ^ swzk(k), an even
// XOR (aligned chunk pairs stay pairs) from row bits 0, 1 and 3.  A
// transposing read instruction reads 16 rows (bits 0-1 and 3-4 vary) of 32
// bytes each: eight distinct pair positions, so two rows per bank group.
__device__ __forceinline__ int swzk(int k) { return ((k & 3) | (((k >> 3) & 1) << 2)) << 1; }

// (tr_read, the transposing LDS read, is in common.hpp: with lane i of a
// 16-lane group addressing row i / 4 and columns 4 (i % 4) .. +3 of a 4 x 16
// block, lane i receives four consecutive k of one n, half a 16x16x32 MFMA
// operand fragment.)

template <int KIND>
__device__ __forceinline__ void mfma(const u32x4& a, const u32x4& b, f32x4& c) {
  if constexpr (KIND == 0) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                               __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

// Four fp32 values to packed 16-bit, round to nearest even: one
// v_cvt_pk_f16_f32 / v_cvt_pk_bf16_f32 per pair (gfx950).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_h2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}
__device__ __forceinline__ uint32_t cvt_b2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint2 pack_h4(float4 v, float scale) {
  return make_uint2(cvt_h2(v.x * scale, v.y * scale), cvt_h2(v.z * scale, v.w * scale));
}
__device__ __forceinline__ uint2 pack_b4(float4 v) {
  return make_uint2(cvt_b2(v.x, v.y), cvt_b2(v.z, v.w));
}

// Store elements [lo, hi) of four packed 16-bit values at base + o (one
// 8-byte store when all four go).  The whole-chunk stores are non-temporal:
// a launch's outputs (over 1 GB for the large buckets) are read only by the
// next launch and would otherwise push the operand panels that the resident
// tiles still share out of L2 (measured 0.4-1.6 % faster per product class).
__device__ __forceinline__ void store16x4(uint16_t* base, size_t o, uint2 v, int lo, int hi) {
  if (lo == 0 && hi == 4) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 x = {v.x, v.y};
    __builtin_nontemporal_store(x, (u32x2*)(base + o));
    return;
  }
  const uint16_t e[4] = {(uint16_t)v.x, (uint16_t)(v.x >> 16), (uint16_t)v.y, (uint16_t)(v.y >> 16)};
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (k >= lo && k < hi) base[o + k] = e[k];
}

// Store elements [lo, 8) of eight packed 16-bit values (v0: 0..3, v1: 4..7)
// at base + o: one non-temporal 16-byte store when all eight go.
__device__ __forceinline__ void store16x8(uint16_t* base, size_t o, uint2 v0, uint2 v1, int lo) {
  if (lo == 0) {
    const u32x4 x = {v0.x, v0.y, v1.x, v1.y};
    __builtin_nontemporal_store(x, (u32x4*)(base + o));
    return;
  }
  store16x4(base, o, v0, min(lo, 4), 4);
  store16x4(base, o + 4, v1, max(lo - 4, 0), 4);
}

// Q1 = a I + P~ from four staged P~ values (fp16, scaled by 1/inv_sp):
// element `dk` (if 0..3) lies on the diagonal.  Output in Q's format.
__device__ __forceinline__ uint2 q_from_p(uint2 pv, float inv_sp, const GemmParams& p, int dk) {
  const _Float16* hp = (const _Float16*)&pv;
  float4 qv = make_float4((float)hp[0] * inv_sp, (float)hp[1] * inv_sp, (float)hp[2] * inv_sp,
                          (float)hp[3] * inv_sp);
  if (dk == 0) qv.x += p.a;
  if (dk == 1) qv.y += p.a;
  if (dk == 2) qv.z += p.a;
  if (dk == 3) qv.w += p.a;
  return p.last ? pack_b4(qv) : pack_h4(qv, p.sQ);
}

}  // namespace

// NW = 4: waves in 2 x 2, each 128 x 128 (8 x 8 MFMA blocks, one wave per SIMD)
// NW = 8: waves in 2 x 4, each 128 x 64 (8 x 4 MFMA blocks, two waves per SIMD)
// BKN: the B operand is stored K-major (rows of k, ld ldb, the tile's n
// contiguous: X itself instead of a transposed copy); its stages hold 32
// rows of 512 bytes and its fragments come from transposing reads.
template <int KIND, int EPI, int NW, bool BKN = false>
__global__ void __launch_bounds__(64 * NW, 1) gemm_dma_kernel(const GemmParams p) {
  constexpr int NT = 64 * NW;                    // threads
  constexpr int WGN = NW / 2;                    // waves along N
  constexpr int WTN = DT / WGN;                  // wave tile N (128 or 64)
  constexpr int FM = 8, FN = WTN / 16;           // 16 x 16 MFMA blocks per wave
  constexpr int DMA_PER_OP = OPB / 1024 / NW;    // 1-KB DMA instructions per wave per operand
  constexpr int DPS = 2 * DMA_PER_OP;            // per wave per stage (vmcnt units)
  // MFMAs between the refill DMAs: the first half-stage carries DPS / 2 of
  // them after its first block row, the second half-stage the other DPS / 2
  constexpr int I1 = 3 * FN / (DPS / 2), I2 = 4 * FN / (DPS / 2);
  static_assert(I1 * (DPS / 2) == 3 * FN && I2 * (DPS / 2) == 4 * FN, "even DMA spacing");
  constexpr int RR = 128;
  constexpr int SMEM_OPS = DSTAGES * STAGEB;
  constexpr int SMEM_EPI = RR * DT * 4;
  constexpr int SMEM_BYTES = SMEM_OPS > SMEM_EPI ? SMEM_OPS : SMEM_EPI;
  __shared__ __attribute__((aligned(1024))) char smem[SMEM_BYTES];
  float* stile = reinterpret_cast<float*>(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wave / WGN, wn = wave % WGN;
  const int q4 = lane >> 4, c16 = lane & 15;  // MFMA lane: K chunk / output row group, row / column

  const uint32_t bid = p.xcd_chunk > 0 ? xcd_remap_chunked(blockIdx.x, gridDim.x, (uint32_t)p.xcd_chunk)
                                       : xcd_remap(blockIdx.x, gridDim.x);
  const int per_mat = p.tiles_per_prod * p.products;
  const int mat = bid / per_mat;
  int t = bid - mat * per_mat;
  const int pi = t / p.tiles_per_prod;
  t -= pi * p.tiles_per_prod;
  const int prod = pi + p.prod_base;
  int ti, tj;
  if (p.triangular) tri_tile_grouped(t, p.tiles_m, p.group > 0 ? p.group : 4, &ti, &tj);
  else full_tile_grouped(t, p.tiles_m, p.tiles_n, p.group > 0 ? p.group : 8, &ti, &tj);
  const int row0A = ti * DT, row0B = tj * DT;
  const char* Ab = (const char*)p.A + (size_t)mat * p.a_stride * 2;
  const char* Bb = pi ? (const char*)p.B2 + (size_t)mat * p.b2_stride * 2
                      : (const char*)p.B + (size_t)mat * p.b_stride * 2;

  // DMA sources: instruction i of this wave fills LDS rows
  // [(wave*DMA_PER_OP + i)*16, +16) of an operand; lane L -> row (L>>2),
  // physical chunk (L&3), which holds logical chunk (L&3) ^ swz4(row).
  const char* srcA[DMA_PER_OP];
  const char* srcB[DMA_PER_OP];
#pragma unroll
  for (int i = 0; i < DMA_PER_OP; ++i) {
    const int row = (wave * DMA_PER_OP + i) * 16 + (lane >> 2);
    const int ch = (lane & 3) ^ swz4(row);
    srcA[i] = Ab + ((size_t)(row0A + row) * p.lda + ch * 8) * 2;
    if constexpr (BKN) {
      // two 512-byte rows of k per instruction; lane L -> row L >> 5,
      // physical chunk L & 31, which holds logical chunk (L & 31) ^ swzk
      const int krow = (wave * DMA_PER_OP + i) * 2 + (lane >> 5);
      srcB[i] = Bb + ((size_t)krow * p.ldb + row0B + (((lane & 31) ^ swzk(krow)) << 3)) * 2;
    } else {
      srcB[i] = Bb + ((size_t)(row0B + row) * p.ldb + ch * 8) * 2;
    }
  }
  // One 1-KB DMA instruction (q = 0..DPS-1: A blocks, then B blocks) of
  // stage ks into ring buffer `buf`.  Stages past the last one re-read the
  // last stage (in bounds; their buffer is never read), so every K step
  // issues the same number of DMAs and the vmcnt bookkeeping is constant.
  const int nk = p.Kdim / DBK;
  auto dma = [&](int q, int buf, int ks) {
    const int kc = ks < nk ? ks : nk - 1;
    char* sb = smem + buf * STAGEB + (q >= DMA_PER_OP ? OPB : 0) +
               (wave * DMA_PER_OP + (q % DMA_PER_OP)) * 1024;
    const char* src = q < DMA_PER_OP ? srcA[q] + kc * ROWB
                                     : srcB[q - DMA_PER_OP] + (BKN ? (size_t)kc * DBK * p.ldb * 2 : (size_t)kc * ROWB);
    __builtin_amdgcn_global_load_lds((gbl_ptr_t*)src, (lds_ptr_t*)sb, 16, 0, 0);
  };

  // fragment addresses (byte offsets within a stage): block f of A / B
  // starts 16 rows (1 KB) after block f - 1, and the swizzle depends only on
  // the row's low bits, so one base per operand serves every block
  const int ra0 = wm * 128 + c16, rb0 = wn * WTN + c16;
  const int offA = ra0 * ROWB + ((q4 ^ swz4(ra0)) << 4);
  const int offB = OPB + rb0 * ROWB + ((q4 ^ swz4(rb0)) << 4);
  auto frag = [&](const char* sb, int off, int f) { return *(const u32x4*)(sb + off + f * 16 * ROWB); };
  // K-major B: block f's fragment is two transposing reads (k 8 q4 .. +3 and
  // +4 .. +7); lane (q4, c16) addresses row 8 q4 + c16 / 4 (+ 4) and
  // columns wn WTN + 16 f + 4 (c16 % 4) .. +3.  swzk is the same for both
  // rows (bit 2 does not enter it)
  const int kb0 = 8 * q4 + (c16 >> 2);
  const int offBK = OPB + kb0 * 512 + ((c16 & 3) >> 1) * 16 + (c16 & 1) * 8;
  const int swB = swzk(kb0) << 4;
  auto fragB = [&](const char* sb, int f) -> u32x4 {
    if constexpr (BKN) {
      const int co = (((wn * WTN) >> 3) + 2 * f) << 4;
      const char* a = sb + offBK + (co ^ swB);
      const uint2 lo = tr_read(a), hi = tr_read(a + 4 * 512);
      return u32x4{lo.x, lo.y, hi.x, hi.y};
    } else {
      return frag(sb, offB, f);
    }
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  u32x4 fa[FM], fb0[FN], fb1[FN];

  // Identity-term harvest (POLY, PQPG, PH, XUPD, XFINAL).  The term X(m, n)
  // that the epilogue adds is symmetric, and X(n, m) is this tile's own B
  // operand at K = m: stages hk0 .. hk0+3 hold the wave's 128 rows m, stage
  // hk0 + s the 32 rows of MFMA block rows 2s and 2s + 1.  While such a stage
  // is resident each lane reads, for each of its FN block columns n and both
  // block rows, the 16-byte chunk holding its 4 consecutive m (half q4 & 1 of
  // chunk 2 (i & 1) + (q4 >> 1)) and adds gamma * X to the accumulators, so
  // the epilogue reads no r x r input.  With a K-major B (X' only) the stage
  // rows are the m themselves, and one transposing read per block returns
  // exactly the lane's 4 values.
  constexpr bool HARVEST =
      EPI == EPI_POLY || EPI == EPI_PQPG || EPI == EPI_PH || EPI == EPI_XUPD || EPI == EPI_XFINAL;
  float gam = 0.0f;
  if constexpr (HARVEST) gam = rr_gamma<EPI>(p);
  const int hk0 = row0A / DBK + wm * 4;

  // Refill schedule: the DMAs of a stage go out in two halves, so that
  // every MFMA run of an iteration carries the same share of them.  Stage
  // kt+4's first DPS/2 instructions (A blocks) are issued in the second half
  // of iteration kt, into the buffer released by that iteration's barrier;
  // its other DPS/2 (B blocks) in the first half of iteration kt+1.  Issued
  // all at once, the 8 waves' refills queued at the CU's address unit and
  // held up the MFMAs behind them in each wave.
  // prologue: stages 0..2 and the first half of stage 3 in flight, wait for
  // stage 0
#pragma unroll
  for (int st = 0; st < DSTAGES; ++st)
#pragma unroll
    for (int q = 0; q < DPS; ++q)
      if (st < DSTAGES - 1 || q < DPS / 2) dma(q, st, st);
  __builtin_amdgcn_s_waitcnt(wait_imm(2 * DPS + DPS / 2, 15));
  barrier();
#pragma unroll
  for (int f = 0; f < FM / 2; ++f) fa[f] = frag(smem, offA, f);
#pragma unroll
  for (int f = 0; f < FN; ++f) fb0[f] = fragB(smem, f);

  // one K step; fb holds this stage's B fragments, fbn receives the next's
  auto step = [&](int kt, u32x4* fb, u32x4* fbn) {
    const int buf = kt & (DSTAGES - 1);
    const char* sb = smem + buf * STAGEB;
    // first half (block rows 0..3): one block row of MFMAs, then this
    // stage's second-half A fragments (and harvest chunks), then the other
    // three block rows
#pragma unroll
    for (int j = 0; j < FN; ++j) mfma<KIND>(fa[0], fb[j], acc[0][j]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int f = FM / 2; f < FM; ++f) fa[f] = frag(sb, offA, f);
    const int hs = kt - hk0;
    u32x4 hv[FN][2];  // whole 16-byte chunks; this lane's 4 values are half q4 & 1
    if (HARVEST && (unsigned)hs < 4u) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int rb = wn * WTN + j * 16 + c16;
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
          if constexpr (BKN) {
            // rows 16 ii + 4 q4 + c16 / 4 of the stage: lane c16 receives
            // X(m .. m + 3, n) for its own 4 rows m and column n (half 0)
            const int kr = 16 * ii + 4 * q4 + (c16 >> 2);
            const int co = (((wn * WTN) >> 3) + 2 * j) << 4;
            const uint2 t = tr_read(sb + OPB + kr * 512 + ((c16 & 3) >> 1) * 16 + (c16 & 1) * 8 +
                                    (co ^ (swzk(kr) << 4)));
            hv[j][ii] = u32x4{t.x, t.y, 0u, 0u};
          } else {
            hv[j][ii] = *(const u32x4*)(sb + OPB + rb * ROWB + (((2 * ii + (q4 >> 1)) ^ swz4(rb)) << 4));
          }
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // the other three block rows of the first half, with the second half of
    // stage kt+3's DMAs (its buffer was released at the previous iteration's
    // barrier)
#pragma unroll
    for (int n = 0; n < 3 * FN; ++n) {
      mfma<KIND>(fa[1 + n / FN], fb[n % FN], acc[1 + n / FN][n % FN]);
      if (n % I1 == I1 - 1) {
        dma(DPS / 2 + n / I1, (kt + DSTAGES - 1) & (DSTAGES - 1), kt + DSTAGES - 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // stage kt+1 landed for this wave (the later DMAs, 2 * DPS of them, may
    // still fly) and this wave's reads of stage kt are done; then publish /
    // retire
    __builtin_amdgcn_s_waitcnt(wait_imm(2 * DPS, 0));
    if (HARVEST && (unsigned)hs < 4u) {
      // every block row takes gamma X or 0 by a select on the wave-uniform
      // stage index: branching to the two block rows of stage hs lets the
      // compiler merge the four branches into one dynamically indexed add,
      // which moves the accumulators to scratch memory
      float gx[2][FN][4];
#pragma unroll
      for (int ii = 0; ii < 2; ++ii)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const u32x4 h = hv[j][ii];
          const uint32_t w0 = (!BKN && (q4 & 1)) ? h[2] : h[0];
          const uint32_t w1 = (!BKN && (q4 & 1)) ? h[3] : h[1];
          gx[ii][j][0] = gam * (float)__builtin_bit_cast(_Float16, (uint16_t)w0);
          gx[ii][j][1] = gam * (float)__builtin_bit_cast(_Float16, (uint16_t)(w0 >> 16));
          gx[ii][j][2] = gam * (float)__builtin_bit_cast(_Float16, (uint16_t)w1);
          gx[ii][j][3] = gam * (float)__builtin_bit_cast(_Float16, (uint16_t)(w1 >> 16));
        }
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const bool on = (i >> 1) == hs;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][j][e] += on ? gx[i & 1][j][e] : 0.0f;
      }
    }
    barrier();
    {  // next stage's first half (unused after the last step; in LDS bounds)
      const char* sn = smem + ((kt + 1) & (DSTAGES - 1)) * STAGEB;
#pragma unroll
      for (int f = 0; f < FM / 2; ++f) fa[f] = frag(sn, offA, f);
#pragma unroll
      for (int f = 0; f < FN; ++f) fbn[f] = fragB(sn, f);
    }
    __builtin_amdgcn_sched_barrier(0);
    // second half (block rows 4..7), with the first half of the refill of
    // this stage's buffer (stage kt+4)
#pragma unroll
    for (int n = 0; n < 4 * FN; ++n) {
      mfma<KIND>(fa[FM / 2 + n / FN], fb[n % FN], acc[FM / 2 + n / FN][n % FN]);
      if (n % I2 == I2 - 1) dma(n / I2, buf, kt + DSTAGES);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // two K steps per trip, so that the B fragments alternate between two
  // register sets without copies
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    step(kt, fb0, fb1);
    step(kt + 1, fb1, fb0);
  }
  if (kt < nk) step(kt, fb0, fb1);
  __builtin_amdgcn_s_waitcnt(wait_imm(0, 0));
  __syncthreads();

  // accumulator element e of block (i, j) is tile row wm*128 + i*16 + 4*q4 + e,
  // tile column wn*WTN + j*16 + c16
  if constexpr (EPI == EPI_FINAL || EPI == EPI_XFINAL) {
    // Final product (and the direct form's last X', whose identity term the
    // loop has harvested): the fp32 tile goes through LDS in two rounds of 128
    // rows, its 16-column groups XOR-swizzled by bits 2-3 of the row
    // (epi_off) so that the staging writes (16 columns of 4 rows 4 apart per
    // instruction) and the row reads are conflict free.  All of a round's W
    // rows are requested before the staging, so their latency overlaps it;
    // each thread then updates four consecutive columns of a row (64 threads
    // per tile row).
    auto epi_off = [](int il, int jc) { return il * DT + (jc ^ (((il >> 2) & 3) << 4)); };
    const int jl = (tid & 63) * 4;
    const int gj = row0B + jl;
    constexpr int RPI = NT / 64;   // tile rows per row-pass iteration
    constexpr int PER = RR / RPI;  // row-pass iterations per round
    const MatPtrs mp = p.table[mat];
    const float inv = EPI == EPI_FINAL ? p.inv_norm[mat] : rr_beta<EPI_XFINAL>(p, mat, 0);
    const bool wvec = p.vec && gj + 4 <= p.out_cols;
#pragma unroll
    for (int round = 0; round < 2; ++round) {
      const int gr0 = row0A + round * RR;
      float4 win[PER];
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const int gi = gr0 + e * RPI + (tid >> 6);
        win[e] = (wvec && gi < p.out_rows) ? nt_load4(mp.W + (size_t)gi * p.out_cols + gj)
                                           : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      if (wm == round) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v)
              stile[epi_off(i * 16 + 4 * q4 + v, wn * WTN + j * 16 + c16)] = acc[i][j][v];
      }
      __syncthreads();
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const int il = e * RPI + (tid >> 6);
        const float4 av = *(const float4*)(stile + epi_off(il, jl));
        const int gi = gr0 + il;
        if (wvec) {
          if (gi < p.out_rows) {
            const float4 o = make_float4(av.x * inv, av.y * inv, av.z * inv, av.w * inv);
            const size_t idx = (size_t)gi * p.out_cols + gj;
            nt_store4(mp.W + idx, f4_axpy(p.decay, win[e], -p.step, o));
            if (mp.O) nt_store4(mp.O + idx, o);
          }
        } else {
          epilogue_final4(p, mat, gi, gj, av, inv);
        }
      }
      __syncthreads();
    }
  } else {
    // Symmetric r x r results (and the direct form's X' = a X + P~ X, whose
    // transposed block goes to the X'^T buffer).  Every wave converts its accumulators to the
    // 16-bit output format (v = beta * acc, scaled fp16 or bf16) and stages
    // the whole tile once, column-major, in the freed operand ring: T[c] holds
    // column c of the tile as 64 chunks of 4 rows (8 bytes), chunk q stored at
    // slot slot16(c, q), which keeps the staging writes and both read passes
    // below free of bank conflicts.  After one barrier:
    //   rows:    lane L of an iteration reads the 4 x 4 block of columns
    //            4L..4L+3 x rows 4q..4q+3, transposes it in registers and
    //            writes 4 rows (each store instruction is one 512-byte row)
    //   mirror:  T[c] is row c of the mirrored block, copied out as is
    // Diagonal tiles store the lower triangle directly and mirror the strictly
    // lower part; POLY on the first iteration also writes Q1 = a I + P~,
    // derived from the staged P~ (power-of-two rescale).
    auto t_off = [](int c, int q) { return c * 512 + (slot16(c, q) << 3); };
    const bool diag = p.triangular && ti == tj;
    const float beta = rr_beta<EPI>(p, mat, prod);
    uint16_t* out1;
    float sc1;
    bool bf1 = false;
    if constexpr (EPI == EPI_XUPD) {
      out1 = (uint16_t*)p.Yn;
      sc1 = p.sX;
    } else if constexpr (EPI == EPI_SYRK || EPI == EPI_PH) {
      out1 = (uint16_t*)p.Gh;
      sc1 = p.sG;
    } else if constexpr (EPI == EPI_POLY) {
      out1 = (uint16_t*)p.Ph;
      sc1 = p.sP;
    } else if (prod == 1) {
      out1 = (uint16_t*)p.Hh;
      sc1 = p.sH;
    } else {
      out1 = (uint16_t*)p.Qh_dst;
      sc1 = p.sQ;
      bf1 = p.last;
    }
    // beta and the power-of-two fp16 scale fold into one factor: the product
    // rounds once to fp32 exactly as beta * acc does, then once to 16 bits
    const float bsc = bf1 ? beta : beta * sc1;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const f32x4 v = acc[i][j];
        *(uint2*)(smem + t_off(wn * WTN + 16 * j + c16, wm * 32 + 4 * i + q4)) =
            bf1 ? pack_b4(make_float4(v[0] * bsc, v[1] * bsc, v[2] * bsc, v[3] * bsc))
                : pack_h4(make_float4(v[0], v[1], v[2], v[3]), bsc);
      }
    __syncthreads();
    const bool qout = EPI == EPI_POLY && p.first;
    uint16_t* out2 = (uint16_t*)p.Qh_dst;
    const float inv_s1 = 1.0f / sc1;
    // rows go to out1 (ld ldp), the transposed block to outm (ld ldm): the
    // same symmetric buffer for r x r results, X' and X'^T for XUPD
    uint16_t* outm = out1;
    int ldp = p.ldr, ldm = p.ldr;
    size_t mb = (size_t)mat * p.rr_stride;
    if constexpr (EPI == EPI_XUPD) {
      outm = (uint16_t*)p.Yt;
      ldp = p.ldyn;
      ldm = p.ldyt;
      mb = (size_t)mat * p.y_stride;
    }
    constexpr int QPW = 64 / NW;  // row-chunk iterations per wave
#pragma unroll 2
    for (int it = 0; it < QPW; ++it) {
      const int q = wave * QPW + it;
      uint2 b[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) b[k] = *(const uint2*)(smem + t_off(4 * lane + k, q));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        const uint2 row =
            e < 2 ? make_uint2(__builtin_amdgcn_perm(b[1].x, b[0].x, sel),
                               __builtin_amdgcn_perm(b[3].x, b[2].x, sel))
                  : make_uint2(__builtin_amdgcn_perm(b[1].y, b[0].y, sel),
                               __builtin_amdgcn_perm(b[3].y, b[2].y, sel));
        const int il = 4 * q + e, jc = 4 * lane;
        const size_t o = mb + (size_t)(row0A + il) * ldp + (row0B + jc);
        // diagonal tile: columns jc + k with k <= il - jc are on or below it
        const int n = diag ? min(max(il - jc + 1, 0), 4) : 4;
        store16x4(out1, o, row, 0, n);
        if (qout) store16x4(out2, o, q_from_p(row, inv_s1, p, diag ? il - jc : -1), 0, n);
      }
    }
    // mirror pass: two staged columns per iteration, half a wave each; lane
    // k of a half takes chunks 2k and 2k + 1 (tile rows 8k..8k+7), which sit
    // in slots s and s ^ 1 (s = slot16(c, 2k)) of one aligned 16-byte pair,
    // and stores them as eight consecutive elements of mirrored row c
    // (X' kept in one layout: no transposed block)
    constexpr int CPW = 256 / NW;  // mirrored rows per wave
#pragma unroll 4
    for (int it = 0; it < ((EPI != EPI_XUPD || p.Yt) ? CPW / 2 : 0); ++it) {
      const int jc = wave * CPW + 2 * it + (lane >> 5);
      const int k = lane & 31;
      const int sl = slot16(jc, 2 * k);
      const uint4 w = *(const uint4*)(smem + jc * 512 + ((sl & ~1) << 3));
      const bool sw = sl & 1;
      const uint2 v0 = sw ? make_uint2(w.z, w.w) : make_uint2(w.x, w.y);  // rows 8k..8k+3
      const uint2 v1 = sw ? make_uint2(w.x, w.y) : make_uint2(w.z, w.w);  // rows 8k+4..8k+7
      const int il0 = 8 * k;
      const size_t o = mb + (size_t)(row0B + jc) * ldm + (row0A + il0);
      // diagonal tile: rows il0 + e > jc only (strictly lower in the tile)
      const int s0 = diag ? min(max(jc - il0 + 1, 0), 8) : 0;
      store16x8(outm, o, v0, v1, s0);
      if (qout) store16x8(out2, o, q_from_p(v0, inv_s1, p, -1), q_from_p(v1, inv_s1, p, -1), s0);
    }
  }
}

template <int KIND, int EPI, int NW, bool BKN = false>
static hipError_t launch_dma_one(const GemmParams& p, int nmat, hipStream_t s) {
  const uint64_t blocks = (uint64_t)nmat * p.tiles_per_prod * p.products;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffull) return hipErrorInvalidValue;
  if (p.Kdim % DBK != 0 || p.Mdim % DT != 0 || p.Ndim % DT != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_dma_kernel<KIND, EPI, NW, BKN>), dim3((uint32_t)blocks), dim3(64 * NW), 0, s,
                     p);
  return hipGetLastError();
}

// Eight waves (two per SIMD) everywhere; four (one per SIMD, 128 x 128 each,
// 256 accumulators per lane) for the products without an identity term to
// harvest (SYRK and the final product), where they fit the register file.
hipError_t launch_gemm_dma(const GemmParams& p, int epi, int nmat, hipStream_t s) {
  const bool w4 = p.waves == 4;
  if (p.waves != 0 && p.waves != 4 && p.waves != 8) return hipErrorInvalidValue;
  if (w4 && epi != EPI_SYRK && epi != EPI_FINAL) return hipErrorInvalidValue;
  if (p.b_kn) {  // K-major B operand: the final product and the direct form's X'
    switch (epi) {
      case EPI_XUPD: return launch_dma_one<1, EPI_XUPD, 8, true>(p, nmat, s);
      case EPI_XFINAL: return launch_dma_one<1, EPI_XFINAL, 8, true>(p, nmat, s);
      case EPI_FINAL: return launch_dma_one<0, EPI_FINAL, 8, true>(p, nmat, s);  // (8 waves)
    }
    return hipErrorInvalidValue;
  }
  switch (epi) {
    case EPI_SYRK:
      if (p.xkind) return w4 ? launch_dma_one<1, EPI_SYRK, 4>(p, nmat, s) : launch_dma_one<1, EPI_SYRK, 8>(p, nmat, s);
      return w4 ? launch_dma_one<0, EPI_SYRK, 4>(p, nmat, s) : launch_dma_one<0, EPI_SYRK, 8>(p, nmat, s);
    case EPI_XUPD: return launch_dma_one<1, EPI_XUPD, 8>(p, nmat, s);
    case EPI_XFINAL: return launch_dma_one<1, EPI_XFINAL, 8>(p, nmat, s);
    case EPI_POLY: return launch_dma_one<1, EPI_POLY, 8>(p, nmat, s);
    case EPI_PQPG: return launch_dma_one<1, EPI_PQPG, 8>(p, nmat, s);
    case EPI_PH: return launch_dma_one<1, EPI_PH, 8>(p, nmat, s);
    case EPI_FINAL:
      return w4 ? launch_dma_one<0, EPI_FINAL, 4>(p, nmat, s) : launch_dma_one<0, EPI_FINAL, 8>(p, nmat, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace muon
