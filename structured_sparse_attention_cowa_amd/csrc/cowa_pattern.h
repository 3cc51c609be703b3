// Position arithmetic of the CoWA pattern, shared by the host plan and the
// device kernels.
//
// "Splitting long-range windows across KV heads beats duplicating them at
// lower cost" (mechanism paragraph) and "CoWindow Attention: Full Causal
// Coverage Is a Collective Property" (Abstract): every KV head sees a shared
// prefix-sink window and a shared near-diagonal window; the remaining causal
// history is cut into non-overlapping long-range bands, one per global KV
// head.  The band partition used here (the pages give no formula):
//   L = ceil((n_ctx - W) / H_kv_global) if n_ctx > W else 0,
//   head g sees distances t - j in [W + b*L, W + (b+1)*L) with b = g for
//   CoWA, b = g mod m for the duplicated-window ablation with m distinct
//   windows (news page, ablation paragraph); L = 0 for sink + local only.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define COWA_HD __host__ __device__ __forceinline__
#else
#define COWA_HD inline
#endif

namespace cowa {

COWA_HD int32_t imax(int32_t a, int32_t b) { return a > b ? a : b; }
COWA_HD int32_t imin(int32_t a, int32_t b) { return a < b ? a : b; }

COWA_HD int32_t derive_band(int32_t n_ctx, int32_t window, int32_t h_kv_global) {
  if (n_ctx <= window) return 0;
  int64_t rest = (int64_t)n_ctx - window;
  return (int32_t)((rest + h_kv_global - 1) / h_kv_global);
}

// Long-range window index of global KV head g when m distinct windows are
// shared out over the heads (m = h_kv_global: CoWA, every head its own).
COWA_HD int32_t band_slot(int32_t g, int32_t m) { return m > 0 ? g % m : g; }

// Parameters of one global KV head, with the band bounds expressed as
// distances.  Band distances [band_lo, band_hi); band_hi == band_lo when L == 0.
struct HeadPattern {
  int32_t sink;
  int32_t window;
  int32_t band_lo;
  int32_t band_hi;
  int32_t causal;  // 1: dense causal mode
};

// b: the head's long-range window index (band_slot of its global index)
COWA_HD HeadPattern head_pattern(int32_t sink, int32_t window, int32_t band, int32_t b,
                                 int32_t causal) {
  HeadPattern h;
  h.sink = sink;
  h.window = window;
  // distances can exceed int32 only for absurd n_ctx; clamp in 64-bit
  int64_t lo = (int64_t)window + (int64_t)b * band;
  int64_t hi = lo + band;
  h.band_lo = lo > 0x3fffffff ? 0x3fffffff : (int32_t)lo;
  h.band_hi = hi > 0x3fffffff ? 0x3fffffff : (int32_t)hi;
  h.causal = causal;
  return h;
}

// Element predicate vis_g(t, j).
COWA_HD bool visible(const HeadPattern& h, int32_t t, int32_t j) {
  int32_t dist = t - j;
  if (j < 0 || dist < 0) return false;
  if (h.causal) return true;
  return j < h.sink || dist < h.window || (dist >= h.band_lo && dist < h.band_hi);
}

// Visible keys of query row t as three disjoint half-open ranges in
// ascending key order: sink [0, s_end), band [b_lo, b_hi), local [l_lo, t+1).
// Empty ranges have lo == hi.  In causal mode the whole prefix is returned as
// the "local" range.
struct RowRanges {
  int32_t lo[3];
  int32_t hi[3];
};

COWA_HD RowRanges row_ranges(const HeadPattern& h, int32_t t) {
  RowRanges r;
  if (h.causal) {
    r.lo[0] = r.hi[0] = 0;
    r.lo[1] = r.hi[1] = 0;
    r.lo[2] = 0;
    r.hi[2] = t + 1;
    return r;
  }
  int32_t s_end = imin(h.sink, t + 1);
  int32_t l_lo = imax(imax(t - h.window + 1, 0), s_end);
  // band keys: t - band_hi < j <= t - band_lo, kept above the sink and below
  // the local window (distances >= W never reach the local window)
  int32_t b_lo = imax(t - h.band_hi + 1, s_end);
  int32_t b_hi = imin(t - h.band_lo + 1, l_lo);
  if (b_hi < b_lo) b_hi = b_lo;
  r.lo[0] = 0;
  r.hi[0] = s_end;
  r.lo[1] = b_lo;
  r.hi[1] = b_hi;
  r.lo[2] = l_lo;
  r.hi[2] = t + 1;
  return r;
}

COWA_HD int32_t row_count(const RowRanges& r) {
  return (r.hi[0] - r.lo[0]) + (r.hi[1] - r.lo[1]) + (r.hi[2] - r.lo[2]);
}

// Masks of partial tiles.  Within a tile, the keys (or queries) one lane
// handles fall into at most three intervals of the element offset o in
// [0, 64): the sink, the local window and the band of vis_g(t, j).  The
// kernels fold them into one 64-bit mask (bit o set: visible).  Host and
// device compile the same functions.

// Bits [lo, hi) of a 64-bit mask, with lo and hi clamped to [0, 64].
COWA_HD uint64_t bit_range(int32_t lo, int32_t hi) {
  lo = imin(imax(lo, 0), 64);
  hi = imin(imax(hi, lo), 64);
  const int32_t w = hi - lo;  // lo <= 63 whenever w > 0
  return w == 0 ? 0ull : (((2ull << (w - 1)) - 1ull) << lo);
}

// Row form: query t, element o is key j = base + o.
COWA_HD uint64_t row_visible_bits(const HeadPattern& hp, int32_t t, int32_t base) {
  const int32_t d0 = t - base;  // o <= d0 is j <= t
  if (hp.causal) return bit_range(0, d0 + 1);
  // a window longer than d0 + 65 covers the same offsets (and keeps d0 - w in
  // range); the band lies at distances >= W >= 1, so it is causal by itself
  const int32_t w = imin(hp.window, imax(d0, 0) + 65);
  return bit_range(0, imin(hp.sink - base, d0 + 1)) | bit_range(d0 - w + 1, d0 + 1) |
         bit_range(d0 - hp.band_hi + 1, d0 - hp.band_lo + 1);
}

// Column form: key j, element o is query t = base + o.
COWA_HD uint64_t col_visible_bits(const HeadPattern& hp, int32_t base, int32_t j) {
  const int32_t c0 = j - base;  // o >= c0 is t >= j
  if (hp.causal || j < hp.sink) return bit_range(c0, 64);
  // offsets past 63 do not matter: the window is cut to 64 - c0 (no overflow)
  const int32_t w = imin(hp.window, 64 - c0);
  return bit_range(c0, c0 + w) | bit_range(c0 + hp.band_lo, c0 + hp.band_hi);
}

// Windowed KV cache for decode ("CoWindow Attention: Full Causal Coverage Is
// a Collective Property", Abstract: lower per-rank decode memory).  For query
// t, head g with long-range window b sees non-sink keys only at distances
// t - j < W + (b+1) L, and later queries see even newer keys, so keys at
// larger distances (other than the sink) are never read again.  A head's
// retained cache is its sink rows followed by a ring of
//   R = min(W + (b+1) L, n_max - S')     (S' = min(S, n_max))
// rows; position j >= S' lives in ring row (j - S') mod R.  Visible keys are
// closer than R to the query, so two of them never share a ring row.
COWA_HD int32_t window_sink_rows(int32_t sink, int32_t n_max) { return imin(sink, n_max); }

COWA_HD int32_t window_ring_rows(int32_t sink, int32_t window, int32_t band, int32_t b,
                                 int32_t n_max) {
  const int64_t want = (int64_t)window + ((int64_t)b + 1) * band;
  const int64_t cap = (int64_t)n_max - window_sink_rows(sink, n_max);
  return (int32_t)(want < cap ? want : cap);
}

// Largest number of keys any row can see: bounds the decode split count.
COWA_HD int32_t max_row_count(int32_t sink, int32_t window, int32_t band, int32_t causal,
                              int32_t n_keys) {
  if (causal) return n_keys;
  int64_t m = (int64_t)sink + window + band;
  return m < n_keys ? (int32_t)m : n_keys;
}

}  // namespace cowa
