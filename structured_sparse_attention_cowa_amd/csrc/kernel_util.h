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
#include "cowa_layout.h"

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

// Direct global -> LDS loads go through a buffer resource (buffer_load ...
// lds) rather than the FLAT-encoded global_load_lds: with a FLAT load to LDS
// in flight the compiler's wait-count pass cannot count LDS reads precisely
// and waits for every outstanding one before each use.  A resource covers
// 2^31 - 1 bytes from its base; callers keep byte offsets below that.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t lds_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff,
                                           0x00020000);
}

// One 16-byte chunk per lane at byte offset voff from the resource's base
// into LDS; the wavefront's 64 chunks land contiguously at lds_base
// (+16 bytes per lane).
__device__ __forceinline__ void buf2lds16(__amdgpu_buffer_rsrc_t rs, int voff, uint16_t* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)lds_base, 16, voff, 0, 0, 0);
}

// One dword per lane at byte offset voff into LDS at lds_base + 4 * lane.
__device__ __forceinline__ void buf2lds4(__amdgpu_buffer_rsrc_t rs, int voff, float* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)lds_base, 4, voff, 0, 0, 0);
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

}  // namespace kern
}  // namespace cowa
