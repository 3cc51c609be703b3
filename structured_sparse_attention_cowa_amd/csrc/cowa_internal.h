// Internal declarations of libcowa: validation helpers, launch parameter
// blocks and launchers.  Not part of the public ABI (include/cowa.h).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/cowa.h"
#include "cowa_pattern.h"

namespace cowa {

// Prefill kernel tile: 8 wavefronts x 32 query rows, 64 keys per K/V tile.
constexpr int kFwdBlockM = 256;
constexpr int kFwdBlockN = 64;

// Decode: largest visible-key chunk one workgroup handles, and the largest
// GQA group size compiled.
constexpr int kDecodeChunkMax = 512;
constexpr int kDecodeMaxGroup = 8;

cowa_status validate_pattern(const cowa_pattern* p, int32_t h_kv_local);
int32_t resolve_band(const cowa_pattern* p);

cowa_status plan_impl(const cowa_pattern* p, int32_t n, int32_t h_kv_local, int32_t bm,
                      int32_t bn, int32_t* row_ptr, int32_t* col, uint8_t* flags, int64_t cap,
                      int64_t* nnz_out);

struct FwdParams {
  const int32_t* row_ptr;
  const int32_t* col;
  const uint8_t* flags;
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* o;
  float* lse;
  int64_t qs_b, qs_t, qs_h;
  int64_t ks_b, ks_t, ks_h;
  int64_t vs_b, vs_t, vs_h;
  int64_t os_b, os_t, os_h;
  int32_t B, N, Hq, Hkv, G, nqt;
  int32_t sink, window, band, kv_head_offset, causal;
  float scale;       // softmax scale (natural-log domain)
  float scale_log2;  // scale * log2(e)
};

// Decode workspace: partial outputs fp32[n_splits, B, H_q, d], then partial
// LSEs fp32[n_splits, B, H_q].
struct DecodeGeometry {
  int32_t chunk;     // visible keys per split
  int32_t n_splits;  // splits per (b, KV head), upper bound
  size_t opart_offset;
  size_t lse_offset;
  size_t total_bytes;
};

DecodeGeometry decode_geometry(const cowa_pattern* p, int32_t B, int32_t H_q, int32_t H_kv_local,
                               int32_t d, int32_t n_max);

struct DecodeParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* seqlens;
  void* o;
  float* lse;
  float* opart;     // [n_splits, B, Hq, d]
  float* lsepart;   // [n_splits, B, Hq]
  int64_t qs_b, qs_h;
  int64_t ks_b, ks_t, ks_h;
  int64_t vs_b, vs_t, vs_h;
  int64_t os_b, os_h;
  int32_t B, Hq, Hkv, G, n_max;
  int32_t sink, window, band, kv_head_offset, causal;
  int32_t chunk, n_splits;
  int32_t o_f32;
  float scale;
  float scale_log2;
};

// Launchers return a hipError_t value (0 on success).
int launch_fwd(const FwdParams& p, int d, int o_f32, void* stream);
int launch_decode(const DecodeParams& p, int d, int o_f32, void* stream);

}  // namespace cowa
