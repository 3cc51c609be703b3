// Workgroup order and LDS tile layouts of the gfx950 kernels: integer
// functions only, compiled both for the device (the kernels) and for the
// host (the CPU tests check the bijection of the workgroup order and the
// bank-conflict freedom of the LDS reads on these very functions).
#pragma once

#include <stdint.h>

#include "cowa_internal.h"
#include "cowa_pattern.h"

#if defined(__HIPCC__)
#define COWA_UNROLL _Pragma("unroll")
#else
#define COWA_UNROLL
#endif

namespace cowa {

// Logical index of workgroup i under the chunked XCD order (see kXcds), or
// -1 for a padding workgroup past total.  Round j deals chunks 8j .. 8j+7 to
// the XCDs in alternating directions, so with heavy-first work the XCD that
// takes a round's heaviest chunk takes the next round's lightest.
COWA_HD int32_t xcd_logical(int32_t i, int32_t chunk, int32_t total) {
  const int32_t xcd = i % kXcds;
  const int32_t r = i / kXcds;
  const int32_t j = r / chunk;
  const int32_t c = (j & 1) ? kXcds - 1 - xcd : xcd;
  const int32_t l = (j * kXcds + c) * chunk + (r - j * chunk);
  return l < total ? l : -1;
}

// ---- LDS tiles: row-major [rows x D] bf16, 16-byte chunks XOR-swizzled ----
//
// Reads of an MFMA A operand (v_mfma_f32_32x32x16_bf16: lane l supplies
// A[l % 32][8 (l / 32) .. +7]) come in two kinds:
//  - plain: 16-byte reads, lane l takes row r0 + (l % 32), chunk 2 ks + l / 32
//    (k runs over the head dimension);
//  - transposing (ds_read_b64_tr_b16): within each group of 16 lanes, lane i
//    receives element i % 4 of the 8-byte pieces addressed by lanes
//    4 e + i / 4; a lane addresses row 8 ri + 4 (l / 32) + (l % 16) / 4 at
//    dims 32 db + 16 ((l / 16) % 2) + 4 (l % 4) .. +3 (k runs over rows).

// Swizzle for tiles read both ways: [0, 6, 12, 10][row % 4] ^ ((row / 4) % 4),
// written with bit operations so that the compiler can bound it.  Free of
// bank conflicts for both kinds of read at D = 128, and its low three bits at
// D = 64 (8 chunks per row).
COWA_HD int32_t swz_both_d128(int32_t row) {
  const int32_t a = row & 3;
  return (((a << 2) ^ (a << 1)) & 14) ^ ((row >> 2) & 3);
}

template <int D>
COWA_HD int32_t swz_both(int32_t row) {
  static_assert(D == 64 || D == 128, "head dimension");
  return swz_both_d128(row) & (D / 8 - 1);
}

// Element offset of a plain read: row `row` of the tile, chunk `chunk`.
template <int D>
COWA_HD int32_t plain_offset(int32_t row, int32_t chunk) {
  return row * D + ((chunk ^ swz_both<D>(row)) * 8);
}

// Plain-read offsets of a lane (l32 = lane % 32, hl = lane / 32) for row
// blocks blk = 0, 1 (rows 32 blk + l32) and k steps ks.  The swizzle depends
// on row % 16 only, so the two blocks differ by the constant 32 D, which the
// compiler folds into the read's offset field.
template <int D>
COWA_HD void plain_offsets(int32_t l32, int32_t hl, int32_t (&off)[2][D / 16]) {
  COWA_UNROLL
  for (int blk = 0; blk < 2; ++blk)
    COWA_UNROLL
    for (int ks = 0; ks < D / 16; ++ks) off[blk][ks] = 32 * blk * D + plain_offset<D>(l32, 2 * ks + hl);
}

// Transposing-read offsets of a lane for the 16-row k step's halves ri = 0, 1
// and head-dim blocks db (add 16 D per k step).
template <int D>
COWA_HD void tr_offsets(int32_t lane, int32_t (&off)[2][D / 32]) {
  const int32_t hl = lane >> 5, r16 = lane & 15, gi = (lane >> 4) & 1;
  COWA_UNROLL
  for (int ri = 0; ri < 2; ++ri)
    COWA_UNROLL
    for (int db = 0; db < D / 32; ++db) {
      const int32_t row = 8 * ri + 4 * hl + (r16 >> 2);
      const int32_t d = 32 * db + 16 * gi + 4 * (r16 & 3);
      off[ri][db] = row * D + (((d >> 3) ^ swz_both<D>(row)) * 8) + (d & 7);
    }
}

// Head-dim-major tiles (one row per head dim, 64 positions = 8 chunks of 8):
// the MFMA operand reads take 16 consecutive rows at one chunk, which this
// swizzle spreads over all banks (whether the LDS serves 128 or 256 bytes per
// cycle).  It repeats every 64 rows.
COWA_HD int32_t swz_tr8(int32_t row) { return (row ^ (row >> 3)) & 7; }

// Storage position of key r inside its group of 16 in a head-dim-major copy:
// bits 2 and 3 swapped, so that the 8 positions a lane reads as one 16-byte
// chunk (k index 8 * (lane / 32) + m of the 32x32x16 MFMA) are the keys the
// probability accumulator gives that lane: 8 (m / 4) + 4 (lane / 32) + m % 4.
// The map is its own inverse.
COWA_HD int32_t tr16_position(int32_t r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// Operand reads from a head-dim-major tile (rows of 64 positions): for
// 16-position step st and head-dim block db, the lane reads row
// 32 db + lane % 32, chunk 2 st + lane / 32.  Element offsets off[db][st];
// the swizzle repeats every 64 rows, so blocks 2, 3 are blocks 0, 1 plus a
// constant (which the compiler folds into the read's offset field).
template <int D>
COWA_HD void hdm_read_offsets(int32_t lane, int32_t (&off)[D / 32][4]) {
  const int32_t l32 = lane & 31, hl = lane >> 5;
  COWA_UNROLL
  for (int db = 0; db < D / 32; ++db)
    COWA_UNROLL
    for (int st = 0; st < 4; ++st) {
      const int32_t row = 32 * db + l32;
      off[db][st] = db >= 2 ? off[db - 2][st] + 64 * 64
                            : row * 64 + (((2 * st + hl) ^ swz_tr8(row)) * 8);
    }
}

// Direct loads of a head-dim-major tile: LDS chunk position P holds row
// P / 8 and the tile's chunk (P % 8) ^ swz_tr8(P / 8) of that row.
COWA_HD int32_t hdm_load_row(int32_t P) { return P >> 3; }
COWA_HD int32_t hdm_load_chunk(int32_t P) { return (P & 7) ^ swz_tr8(P >> 3); }

// Direct global -> LDS loads: the loading lanes of a tile, in order, fill
// 16-byte LDS chunk positions P = 0, 1, ...; position P holds row P / (D / 8),
// column chunk (P % (D / 8)) ^ swz_both(row), i.e. the global chunk read by
// the lane for position P.
template <int D>
COWA_HD int32_t load_row(int32_t P) { return P / (D / 8); }
template <int D>
COWA_HD int32_t load_col(int32_t P) {
  return ((P % (D / 8)) ^ swz_both<D>(P / (D / 8))) * 8;
}

}  // namespace cowa
