// kda_record.h -- per-chunk record passed from the parallel first pass of the two-pass
// chunk forward to the state pass.  A record is the byte image of the LDS tiles the
// state pass reads, padded rows included, so that the state pass moves it into LDS with
// plain 16-byte DMA and reads it there without bank conflicts:
//   WW  [64][DK]  -W           (W = M diag(beta) (K o gamma)),  rows of DK*ES + 16 bytes
//   QG  [64][DK]  Q o gamma,                                    rows of DK*ES + 16 bytes
//   KRT [DK][64]  (K o rho)^T,                                  rows of 64*ES + 16 bytes
//   AT  [64][64]  A, zero above the diagonal,                   rows of 64*ES + 16 bytes
//   MT  [64][64]  M diag(beta), zero above the diagonal,        rows of 64*ES + 16 bytes
//   GC  [DK]      gamma of the chunk's last row, fp32
// (element type T unless noted; the 16 pad bytes of a row hold no data).
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

}  // namespace kda
