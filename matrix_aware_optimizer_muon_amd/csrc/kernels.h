// Internal launch interface between the C-ABI host code and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muon {

// One entry per matrix, in plan order (device-resident table).
struct MatPtrs {
  float* W;
  float* M;
  const void* G;
  float* O;  // nullable direction output
};

// EPI_XFINAL: the direct form's last X' = a X + P~ X, applied to W as the
// final product does (X' is O; non-transposed buckets).
enum Epi : int { EPI_SYRK = 0, EPI_POLY = 1, EPI_PQPG = 2, EPI_PH = 3, EPI_FINAL = 4, EPI_XUPD = 5,
                 EPI_XFINAL = 6 };
enum OpType : int { OP_BF16 = 0, OP_F32 = 1 };

// Parameters of one batched GEMM launch C = A * B^T over a chunk of
// same-shape matrices, plus its fused epilogue.  All matrices of the chunk
// use the same strides; matrix `mat` of the chunk adds mat*stride.
struct GemmParams {
  const void* A;
  const void* B;
  const void* B2;          // second B operand of a two-product launch
  int64_t a_stride, b_stride, b2_stride;  // elements between matrices
  int lda, ldb;            // leading dimensions (elements)
  int Mdim, Ndim, Kdim;    // padded sizes (multiples of the tile / K step)
  int tiles_m, tiles_n;
  int triangular;          // lower-triangle tiles only (symmetric result)
  int tiles_per_prod;      // tiles of one product of one matrix
  int products;            // 1 or 2
  int xcd_chunk;           // 0: each XCD takes one contiguous range of the
                           // launch's tiles; > 0: runs of this many (xcd_remap_chunked)
  int group;               // 256-wide kernels: tile rows per tile-order group
                           // (0: 8 for full grids, 4 for triangular ones)
  int waves;               // 256-wide kernels: 8, or 4 (SYRK and the final product)
  int prod_base;           // epilogue product index of the first product
  int b_kn;                // B stored K-major (rows of k, ld ldb, the tile's n
                           // contiguous): 256-wide kernels' final product and
                           // EPI_XUPD / EPI_XFINAL; the 64- and 128-wide 16-bit
                           // final product
  // r x r recursion buffers (fp32 master copies and MFMA operand copies)
  float* Gf;
  float* Qf_src;
  float* Qf_dst;
  float* Hf;
  void* Gh;
  void* Ph;
  void* Qh_dst;
  const void* Qh_src;      // fp16 copy of the previous Q (fp16-only epilogues)
  void* Hh;
  int64_t rr_stride;       // elements between matrices in r x r buffers
  int ldr;                 // r_pad
  float a, b, c;           // quintic coefficients
  float sG, sP, sQ, sH;    // power-of-two operand scales
  int first, last;
  // final update
  const MatPtrs* table;    // chunk's first entry
  const float* inv_norm;   // per matrix of the chunk
  int out_rows, out_cols;  // m, n of the parameter
  float decay;             // 1 - lr*wd
  float step;              // lr * scale_coeff * sqrt(max(m, n))
  int vec;                 // W / O rows allow 16-byte access
  // direct form
  int xkind;               // SYRK operand type: 0 bf16, 1 fp16
  float syrk_scale;        // SYRK result scale; 0: 1/||U||^2
  float sX;                // fp16 scale of X
  void* Yn;                // EPI_XUPD: X' natural layout (r_pad x c_pad, ld ldyn)
  void* Yt;                // EPI_XUPD: X' transposed (c_pad x r_pad, ld ldyt); null on
                           // the 256-wide kernels: X' in the natural layout only
  int ldyn, ldyt;
  int64_t y_stride;        // elements between matrices (both)
  const void* Xid;         // small-tile EPI_XUPD / EPI_XFINAL: X in the layout
                           // of Yn (ld ldyn, stride y_stride), for the a X term
};

hipError_t launch_gemm(const GemmParams& p, int epi, int op, int bt, int nmat, hipStream_t s);
// 256-tile 16-bit products with the direct-to-LDS pipeline (gemm_dma.hip)
hipError_t launch_gemm_dma(const GemmParams& p, int epi, int nmat, hipStream_t s);

// The whole r x r recursion in one launch for r_pad <= 128 (rr_fused.hip):
// reads G0 (fp32, from the SYRK), writes the last Q as bf16.
struct RrFusedParams {
  const float* Gf;         // G0 per matrix, r_pad x r_pad fp32
  int64_t rr_stride;       // elements between matrices (Gf and Qout)
  int r_pad;               // 64 or 128
  void* Qout;              // bf16 Q_N per matrix, r_pad x r_pad
  float a, b, c;           // quintic coefficients
  float sG, sP, sQ, sH;    // power-of-two operand scales
  int N;                   // iterations
};
hipError_t launch_rr_fused(const RrFusedParams& p, int nmat, hipStream_t s);

// The whole direct-form iteration and the weight update in one launch for
// buckets of padded squares, r_pad = c_pad in {128, 256}, on the 16-bit path
// (direct_fused.hip): U (bf16, both layouts, from the prep pass) is cast to
// X^ (fp16, scaled by sX / ||U||) in place; the pair buffers alternate per
// iteration (the r x r intermediates stay in LDS).
struct DirectFusedParams {
  const MatPtrs* table;    // chunk's first entry (W, O)
  const float* partials;   // the prep pass's ||U||^2 partial sums, [nmat][blocks_per_mat]
  int blocks_per_mat;      // (each workgroup forms its matrix's 1 / ||U|| from them)
  void* Xn[2];             // natural layout, per iteration parity (Xn[0]: U
  void* Xt[2];             // in bf16 on entry, cast in place); transposed
  int64_t x_stride;        // elements between matrices in Xn / Xt
  int rp;                  // r_pad = c_pad
  int m, n;                // true sizes (m <= n)
  float a, b, c;
  float sX, sG, sP;
  float syrk_scale;        // 1 / sX^2
  int N;
  float decay, step;
  int vec;                 // W / O rows allow 16-byte access
};
hipError_t launch_direct_fused(const DirectFusedParams& p, int nmat, hipStream_t s);

// Write up to kTableChunk pointer-table entries, passed by value as kernel
// arguments, to dst[0 .. count) (no staging buffer and no host-memory copy;
// 120 entries keep the argument block under 4 KB).
constexpr int kTableChunk = 120;
struct TableChunk {
  MatPtrs e[kTableChunk];
  int count;
};
hipError_t launch_write_table(const TableChunk& t, MatPtrs* dst, hipStream_t s);

// ---- memory-bound kernels ------------------------------------------------
struct PrepParams {
  const MatPtrs* table;
  int m, n;                // parameter shape
  int m_pad, n_pad;        // padded natural shape (multiples of 64)
  float mu;
  int nesterov;
  void* X;                 // U, natural layout m_pad x n_pad (matrix 0 of the chunk)
  void* XT;                // U^T, n_pad x m_pad (null: not written; the 16-bit path
                           // then runs the row-tiled kernel)
  int64_t x_stride;        // elements between matrices (both copies)
  float* partials;         // [nmat][blocks_per_mat]
  int blocks_per_mat;
  float* inv_norm;         // [nmat]
};

hipError_t launch_prep(const PrepParams& p, int grad_bf16, int x_f32, int nmat, int vec,
                       hipStream_t s);
hipError_t launch_norm_finalize(const PrepParams& p, int nmat, hipStream_t s);
// partial sums per matrix: 64 x 64 tiles, or 8 x 512 row tiles when rows
// (one layout: XT null on the 16-bit path)
int prep_blocks_per_mat(int m_pad, int n_pad, bool rows);

struct RowNormParams {
  const MatPtrs* table;
  int m, n;
  float mu;
  int nesterov;
  float eps;
  float decay, step;
  float* partials;         // tall case: [nmat][row_blocks][n]
  float* colscale;         // tall case: [nmat][n]
  int row_blocks;
};

// ---- direct form ("Infra Optimizers" eq. (2) iterated on X) --------------
// X0 = U / ||U|| as fp16 scaled by sx, in place over both U layouts of the
// chunk (natural m_pad x n_pad and transposed n_pad x m_pad, bf16 on entry).
struct XcastParams {
  void* Xn;                // natural layout, matrix 0 of the chunk
  void* Xt;                // transposed layout (null: one layout)
  int64_t x_stride;        // elements between matrices (both buffers)
  int64_t elems;           // m_pad * n_pad (a multiple of 8)
  const float* inv_norm;   // [nmat]
  float sx;
};
hipError_t launch_xcast(const XcastParams& p, int nmat, hipStream_t s);

// W <- decay W - step O with O = X_N / sx read from the natural-layout
// buffer (m_pad x n_pad, fp16); O_out receives O when non-null.
struct WupdParams {
  const MatPtrs* table;
  const void* X;           // natural layout of X_N, matrix 0 of the chunk
  int64_t x_stride;
  int m, n, n_pad;
  float inv_sx, decay, step;
};
hipError_t launch_wupd(const WupdParams& p, int nmat, int vec, hipStream_t s);

enum RowNormPhase : int { RN_PHASE_ROWS = 0, RN_PHASE_COLSUM = 1, RN_PHASE_COLFINAL = 2, RN_PHASE_COLAPPLY = 3 };
hipError_t launch_rownorm(const RowNormParams& p, int grad_bf16, int nmat, int vec, int phase,
                          hipStream_t s);
int rownorm_row_blocks(int m, int n);

}  // namespace muon
