// Device helpers shared by the prefill forward and backward kernels (gfx950).
//
// Frame: both passes use v_mfma_f32_32x32x16_bf16.  For D[32x32] += A[32x16]
// B[16x32], lane l holds A[l % 32][8 (l / 32) + e] and B[8 (l / 32) + e][l % 32]
// (e = 0..7), and accumulator register i of lane l holds
// D[8 (i / 4) + 4 (l / 32) + i % 4][l % 32].
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "cowa_internal.h"

namespace cowa {
namespace kern {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float NEG_INF = -__builtin_huge_valf();
constexpr float POS_INF = __builtin_huge_valf();
constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Logical index of workgroup i under the chunked XCD order (see kXcds), or
// -1 for a padding workgroup past total.  Round j deals chunks 8j .. 8j+7 to
// the XCDs in alternating directions, so with heavy-first work the XCD that
// takes a round's heaviest chunk takes the next round's lightest.
__device__ __forceinline__ int xcd_logical(int i, int chunk, int total) {
  const int xcd = i % kXcds;
  const int r = i / kXcds;
  const int j = r / chunk;
  const int c = (j & 1) ? kXcds - 1 - xcd : xcd;
  const int l = (j * kXcds + c) * chunk + (r - j * chunk);
  return l < total ? l : -1;
}

// Masking of partial tiles.  Within a tile, the keys (or queries) a lane
// sees form at most three intervals of the element offset o in [0, 64): the
// sink, the local window and the band of vis_g(t, j) (cowa_pattern.h).  Each
// lane folds them into one 64-bit mask; an element is then kept or set to
// -inf with a sign-extended bit extract and a bitfield insert.

// Bits [lo, hi) of a 64-bit mask, with lo and hi clamped to [0, 64].
__device__ __forceinline__ uint64_t bit_range(int lo, int hi) {
  lo = min(max(lo, 0), 64);
  hi = min(max(hi, lo), 64);
  const int w = hi - lo;  // lo <= 63 whenever w > 0
  return w == 0 ? 0ull : (((2ull << (w - 1)) - 1ull) << lo);
}

// Row form: the lane is query t, element o is key j = base + o.
__device__ __forceinline__ uint64_t row_visible_bits(const HeadPattern& hp, int t, int base) {
  const int d0 = t - base;  // o <= d0 is j <= t
  if (hp.causal) return bit_range(0, d0 + 1);
  // a window longer than d0 + 65 covers the same offsets (and keeps d0 - w in
  // range); the band lies at distances >= W >= 1, so it is causal by itself
  const int w = min(hp.window, max(d0, 0) + 65);
  return bit_range(0, min(hp.sink - base, d0 + 1)) | bit_range(d0 - w + 1, d0 + 1) |
         bit_range(d0 - hp.band_hi + 1, d0 - hp.band_lo + 1);
}

// Column form: the lane is key j, element o is query t = base + o.
__device__ __forceinline__ uint64_t col_visible_bits(const HeadPattern& hp, int base, int j) {
  const int c0 = j - base;  // o >= c0 is t >= j
  if (hp.causal || j < hp.sink) return bit_range(c0, 64);
  // offsets past 63 do not matter: the window is cut to 64 - c0 (no overflow)
  const int w = min(hp.window, 64 - c0);
  return bit_range(c0, c0 + w) | bit_range(c0 + hp.band_lo, c0 + hp.band_hi);
}

// s if bit o of m is set, else -inf (o is a compile-time constant).
__device__ __forceinline__ float keep_if(float s, uint64_t m, int o) {
  const int word = (int)(o < 32 ? (uint32_t)m : (uint32_t)(m >> 32));
  const unsigned keep = (unsigned)__builtin_amdgcn_sbfe(word, o & 31, 1);
  return __uint_as_float((__float_as_uint(s) & keep) | (0xff800000u & ~keep));
}

// Lane l and lane l^32 hold the two halves of one accumulator column; this
// returns (value of lane l, value of lane l^32) in some order on every lane.
__device__ __forceinline__ void pair_swap(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

__device__ __forceinline__ float pair_max(float x) {
  float a, b;
  pair_swap(x, a, b);
  return fmaxf(a, b);
}

__device__ __forceinline__ float pair_sum(float x) {
  float a, b;
  pair_swap(x, a, b);
  return a + b;
}

__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  bf16x2 r = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(unsigned, r);
}

// One 16-byte chunk per lane from global memory straight into LDS; the
// wavefront's 64 chunks land contiguously at lds_base (+16 bytes per lane).
__device__ __forceinline__ void g2lds16(const uint16_t* g, uint16_t* lds_base) {
  __builtin_amdgcn_global_load_lds((const void*)g, (lds_void*)lds_base, 16, 0, 0);
}

// One dword per lane into LDS at lds_base + 4 * lane.
__device__ __forceinline__ void g2lds4(const float* g, float* lds_base) {
  __builtin_amdgcn_global_load_lds((const void*)g, (lds_void*)lds_base, 4, 0, 0);
}

// gfx950 transposing LDS read (ds_read_b64_tr_b16): within each 16-lane
// group, lane i receives element i % 4 of the 64-bit rows addressed by lanes
// 4 e + i / 4 (e = 0..3).
__device__ __forceinline__ i16x4 lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
}

// The A operand of a 32x32x16 product whose k index runs over rows of a
// row-major LDS tile: the transposing reads at two row offsets, joined.
__device__ __forceinline__ bf16x8 lds_read_tr_pair(const uint16_t* lo, const uint16_t* hi) {
  const i16x4 a8[2] = {lds_read_tr(lo), lds_read_tr(hi)};
  return __builtin_bit_cast(bf16x8, a8);
}

// Row-major [rows x 128] bf16 LDS tiles whose 16-byte chunks are XOR-swizzled
// by this function of the row are free of bank conflicts both for 16-byte
// reads of one chunk column by 16 consecutive rows and for transposing reads
// of 4 consecutive rows x 2-4 adjacent chunks.
// The value is [0, 6, 12, 10][row % 4] ^ ((row / 4) % 4), written with bit
// operations so that the compiler can bound it (and the offsets built from it).
__device__ __forceinline__ int swz_both_d128(int row) {
  const int a = row & 3;
  return (((a << 2) ^ (a << 1)) & 14) ^ ((row >> 2) & 3);
}

// The same swizzle for [rows x D] tiles: for D = 64 (8 chunks per row) its low
// three bits keep both read patterns free of bank conflicts (checked on the
// host against a model of 128- and 256-byte LDS cycles).
template <int D>
__device__ __forceinline__ int swz_both(int row) {
  static_assert(D == 64 || D == 128, "head dimension");
  return swz_both_d128(row) & (D / 8 - 1);
}

}  // namespace kern
}  // namespace cowa
