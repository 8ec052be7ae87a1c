// kda_record.h -- per-chunk records passed from the parallel first pass of the two-pass
// chunk forward to the state pass.
//
// RecordLayout<T, DK> (fp32 inputs, d_k = d_v = 64): the byte image of the LDS tiles the
// fp32 state pass reads, padded rows included, so that it moves with plain 16-byte DMA:
//   WW  [64][DK]  -W           (W = M diag(beta) (K o gamma)),  rows of DK*ES + 16 bytes
//   QG  [64][DK]  Q o gamma,                                    rows of DK*ES + 16 bytes
//   KRT [DK][64]  (K o rho)^T,                                  rows of 64*ES + 16 bytes
//   AT  [64][64]  A, zero above the diagonal,                   rows of 64*ES + 16 bytes
//   MT  [64][64]  M diag(beta), zero above the diagonal,        rows of 64*ES + 16 bytes
//   GC  [DK]      gamma of the chunk's last row, fp32
// (element type T unless noted; the 16 pad bytes of a row hold no data).
//
// WalkRecord<DK> (bf16 inputs): only what the key and query sides cannot rebuild cheaply.
// The state pass re-reads q, k and alpha and forms Q o gamma, K o gamma and K o rho itself
// (the gate products are running products of alpha inside the chunk), so the record
// carries the two 64 x 64 chunk matrices:
//   A    lower 64 x 64, bf16      A_ij = sum_c q_ic k_jc r_ijc (j <= i)
//   MH   lower 64 x 64, bf16      M~ = (I + T)^-1 diag(beta) rounded to bf16
//   ML   lower 64 x 64, bf16      M~ - MH rounded to bf16 (MH + ML carries M~ to ~2^-17)
// A lower matrix is stored as two row-major blocks: rows 0..31 with columns 0..31 (rows of
// 64 bytes) and rows 32..63 with columns 0..63 (rows of 128 bytes); the upper-right 32 x 32
// block, all zeros, is not stored.  There is no padding: the 16-byte units of a row are
// permuted instead (unit u of row i sits at u ^ ((i >> 2) & 3) in the top block and at
// u ^ ((i >> 1) & 7) in the bottom one), so that the sixteen rows a matrix-core fragment
// read touches land on distinct LDS banks.  The state pass moves the whole record into LDS
// as one image.
#pragma once
#include <stddef.h>

#include "kda_common.h"

namespace kda {

template <typename T, int DK>
struct RecordLayout {
  static constexpr int ES = Elem<T>::kBytes;
  static constexpr int RS_DK = DK * ES + 16;  // [pos][channel] row stride
  static constexpr int RS_C = 64 * ES + 16;   // [channel][pos] and [pos][pos] row stride
  static constexpr int WW = 0;
  static constexpr int QG = WW + 64 * RS_DK;
  static constexpr int KRT = QG + 64 * RS_DK;
  static constexpr int AT = KRT + DK * RS_C;
  static constexpr int MT = AT + 64 * RS_C;
  static constexpr int GC = MT + 64 * RS_C;
  static constexpr int IMG = GC + DK * 4;                       // bytes that carry the image
  static constexpr size_t BYTES = ((size_t)IMG + 255) / 256 * 256;  // stride between records
  static_assert(IMG % 16 == 0, "16-byte units");
};

template <int DK>
struct WalkRecord {
  static constexpr int RS_TOP = 32 * 2;  // rows 0..31, columns 0..31
  static constexpr int RS_BOT = 64 * 2;  // rows 32..63, columns 0..63
  static constexpr int BOT = 32 * RS_TOP;
  static constexpr int MAT = BOT + 32 * RS_BOT;  // one lower matrix
  static constexpr int A = 0;
  static constexpr int MH = MAT;
  static constexpr int ML = 2 * MAT;
  static constexpr int DMA = 3 * MAT;  // moved into LDS by the state pass
  static constexpr size_t BYTES = ((size_t)DMA + 255) / 256 * 256;
  static_assert(DMA % 1024 == 0, "whole 1 KiB transfer units");
  // the stored position of 16-byte unit u of row i
  __host__ __device__ static constexpr int unit(int i, int u) { return i < 32 ? u ^ ((i >> 2) & 3) : u ^ ((i >> 1) & 7); }
  // byte offset of element (i, j), j <= 31 for i <= 31, of a lower matrix image
  __host__ __device__ static constexpr int at(int i, int j) {
    return (i < 32 ? i * RS_TOP : BOT + (i - 32) * RS_BOT) + 16 * unit(i, j >> 3) + 2 * (j & 7);
  }
};

}  // namespace kda
