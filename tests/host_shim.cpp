// Host build of the kernels' integer helpers, for the CPU tests: the same
// header functions the gfx950 kernels compile (tile masks, workgroup order,
// LDS layouts), exported with C linkage and plain integer arguments.  Built
// with g++ by tests/host_shim.py; nothing in the library links it.
#include "cowa_layout.h"
#include "cowa_pattern.h"

using namespace cowa;

static HeadPattern hp_of(int32_t sink, int32_t window, int32_t band, int32_t b, int32_t causal) {
  return head_pattern(sink, window, band, b, causal);
}

extern "C" {

uint64_t shim_row_visible_bits(int32_t sink, int32_t window, int32_t band, int32_t b,
                               int32_t causal, int32_t t, int32_t base) {
  return row_visible_bits(hp_of(sink, window, band, b, causal), t, base);
}

uint64_t shim_col_visible_bits(int32_t sink, int32_t window, int32_t band, int32_t b,
                               int32_t causal, int32_t base, int32_t j) {
  return col_visible_bits(hp_of(sink, window, band, b, causal), base, j);
}

void shim_row_ranges(int32_t sink, int32_t window, int32_t band, int32_t b, int32_t causal,
                     int32_t t, int32_t* lo, int32_t* hi) {
  const RowRanges r = row_ranges(hp_of(sink, window, band, b, causal), t);
  for (int i = 0; i < 3; ++i) {
    lo[i] = r.lo[i];
    hi[i] = r.hi[i];
  }
}

int32_t shim_xcd_logical(int32_t i, int32_t chunk, int32_t total) {
  return xcd_logical(i, chunk, total);
}
int32_t shim_xcd_chunk(int64_t per_unit, int64_t units, int64_t max_units) {
  return xcd_chunk(per_unit, units, max_units);
}
int64_t shim_xcd_grid(int64_t total, int32_t chunk) { return xcd_grid(total, chunk); }

int32_t shim_swz_both(int32_t d, int32_t row) {
  return d == 128 ? swz_both<128>(row) : swz_both<64>(row);
}

// Element offsets of one lane's plain reads: out[blk * (d / 16) + ks].
void shim_plain_offsets(int32_t d, int32_t lane, int32_t* out) {
  if (d == 128) {
    int32_t off[2][8];
    plain_offsets<128>(lane & 31, lane >> 5, off);
    for (int i = 0; i < 16; ++i) out[i] = off[i / 8][i % 8];
  } else {
    int32_t off[2][4];
    plain_offsets<64>(lane & 31, lane >> 5, off);
    for (int i = 0; i < 8; ++i) out[i] = off[i / 4][i % 4];
  }
}

// Element offsets of one lane's transposing reads: out[ri * (d / 32) + db].
void shim_tr_offsets(int32_t d, int32_t lane, int32_t* out) {
  if (d == 128) {
    int32_t off[2][4];
    tr_offsets<128>(lane, off);
    for (int i = 0; i < 8; ++i) out[i] = off[i / 4][i % 4];
  } else {
    int32_t off[2][2];
    tr_offsets<64>(lane, off);
    for (int i = 0; i < 4; ++i) out[i] = off[i / 2][i % 2];
  }
}

int32_t shim_load_row(int32_t d, int32_t P) { return d == 128 ? load_row<128>(P) : load_row<64>(P); }

// Head-dim-major tiles: swizzle, position order inside 16-key groups, and
// one lane's operand-read offsets out[db * 4 + st].
int32_t shim_swz_tr8(int32_t row) { return swz_tr8(row); }
int32_t shim_tr16_position(int32_t r) { return tr16_position(r); }
void shim_hdm_read_offsets(int32_t d, int32_t lane, int32_t* out) {
  if (d == 128) {
    int32_t off[4][4];
    hdm_read_offsets<128>(lane, off);
    for (int i = 0; i < 16; ++i) out[i] = off[i / 4][i % 4];
  } else {
    int32_t off[2][4];
    hdm_read_offsets<64>(lane, off);
    for (int i = 0; i < 8; ++i) out[i] = off[i / 4][i % 4];
  }
}
int32_t shim_hdm_load_row(int32_t P) { return hdm_load_row(P); }
int32_t shim_hdm_load_chunk(int32_t P) { return hdm_load_chunk(P); }
int32_t shim_load_col(int32_t d, int32_t P) { return d == 128 ? load_col<128>(P) : load_col<64>(P); }

}  // extern "C"
