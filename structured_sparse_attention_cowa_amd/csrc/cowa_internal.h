// Internal declarations of libcowa: validation helpers, launch parameter
// blocks and launchers.  Not part of the public ABI (include/cowa.h).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/cowa.h"
#include "cowa_pattern.h"

namespace cowa {

// Prefill kernel tile: 8 wavefronts x 32 query rows, 64 keys per K/V tile.
// Workgroup order dealt to the XCDs in chunks.  The dispatcher sends
// workgroup i to XCD i mod kXcds; a kernel that maps i through xcd_logical
// runs logical workgroups [c * chunk, (c + 1) * chunk) on XCD c mod kXcds, so
// neighbours in the logical order (which read the same tiles) share an L2.
constexpr int kXcds = 8;  // XCDs of an MI355X

// chunk = k units of per_unit workgroups, 1 <= k <= max_units: at least
// enough units to fill one XCD's 32 compute units (workgroups of neighbouring
// units read the same tiles, and only those running together share the L2),
// and beyond that only as many as leave every XCD 16 chunks or more, so that
// the heavy-first order evens out across the XCDs.
inline int32_t xcd_chunk(int64_t per_unit, int64_t units, int64_t max_units) {
  const int64_t fill = (32 + per_unit - 1) / per_unit;
  const int64_t spread = units / (16 * kXcds);
  int64_t k = spread < max_units ? spread : max_units;
  k = k > fill ? k : fill;
  k = k > max_units ? max_units : k;
  k = k < 1 ? 1 : k;
  return (int32_t)(per_unit * k);
}
// grid size: the logical count padded to whole rounds of kXcds chunks
inline int64_t xcd_grid(int64_t total, int32_t chunk) {
  const int64_t span = (int64_t)kXcds * chunk;
  return (total + span - 1) / span * span;
}

constexpr int kFwdBlockM = 256;
constexpr int kFwdBlockN = 64;

// Bytes of the forward's workspace: V head-dim-major for B sequences of up to
// N keys (N rounded up to kFwdBlockN), 256-byte multiple.
inline size_t fwd_workspace_bytes(int64_t B, int64_t N, int64_t H_kv, int64_t d) {
  const int64_t npad = (N + kFwdBlockN - 1) / kFwdBlockN * kFwdBlockN;
  return ((size_t)(B * H_kv * d * npad * 2) + 255) / 256 * 256;
}

// Decode: largest visible-key chunk one workgroup handles, and the largest
// GQA group size compiled.
constexpr int kDecodeChunkMax = 768;
constexpr int kDecodeMaxGroup = 8;

cowa_status validate_pattern(const cowa_pattern* p, int32_t h_kv_local);
int32_t resolve_band(const cowa_pattern* p);
int32_t resolve_n_bands(const cowa_pattern* p);

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
  int32_t n_bands;  // distinct long-range windows (head g takes g mod n_bands)
  // packed sequences (varlen): B sequences, sequence b at token rows
  // [cu_seqlens[b], cu_seqlens[b+1]) of length <= N; LSE [H_q, total_tokens].
  // NULL: the batched layout ([B, N, ...] with the b strides).
  const int32_t* cu_seqlens;
  int32_t total_tokens;
  int32_t xcd_chunk;  // workgroup order: chunks of this many go to one XCD (0: launch_fwd's default)
  // workspace: V head-dim-major, [B][H_kv][d][npad] bf16 (B = sequences when
  // packed), the keys of each 16-key group stored in the order the P operand
  // takes them (tr16_position), zero past each sequence's end; written by the
  // transpose kernel of launch_fwd before the forward kernel reads it
  uint16_t* vt;
  int32_t npad;  // N (the longest sequence when packed) rounded up to 64
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
  int32_t n_bands;  // distinct long-range windows (head g takes g mod n_bands)
  int32_t chunk, n_splits;
  int32_t o_f32;
  int32_t win;  // 1: K/V in the windowed layout (rows [B][heads x (sink + ring)][d])
  float scale;
  float scale_log2;
};

// Backward dK/dV kernel tile: 64 query rows x 128 keys (4 wavefronts x 32 keys).
constexpr int kBwdBlockM = 64;
constexpr int kBwdBlockN = 128;

cowa_status plan_kv_impl(const cowa_pattern* p, int32_t n, int32_t h_kv_local, int32_t bm,
                         int32_t bn, int32_t* row_ptr, int32_t* col, uint8_t* flags,
                         int64_t cap, int64_t* nnz_out);

struct BwdParams {
  const int32_t* row_ptr;     // query-major plan (dQ)
  const int32_t* col;
  const uint8_t* flags;
  const int32_t* row_ptr_kv;  // key-major plan (dK, dV)
  const int32_t* col_kv;
  const uint8_t* flags_kv;
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const void* o;
  const uint16_t* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* lse2;   // workspace [B, Hq, npad]: LSE * log2(e), +inf for rows >= N
  float* delta;  // workspace [B, Hq, npad]: rowsum(dO * O), 0 for rows >= N
  int64_t qs_b, qs_t, qs_h;
  int64_t ks_b, ks_t, ks_h;
  int64_t vs_b, vs_t, vs_h;
  int64_t os_b, os_t, os_h;
  int64_t dos_b, dos_t, dos_h;
  int64_t dqs_b, dqs_t, dqs_h;
  int64_t dks_b, dks_t, dks_h;
  int64_t dvs_b, dvs_t, dvs_h;
  float* part;   // workspace: fp32 dK, dV partials of the split sink key tiles
  // packed sequences (varlen): B sequences, sequence b at token rows
  // [cu_seqlens[b], cu_seqlens[b+1]) of length <= N (b strides 0); LSE
  // [H_q, total_tokens].  NULL: the batched layout.
  const int32_t* cu_seqlens;
  int32_t total_tokens;
  int32_t B, N, Hq, Hkv, G, nqt, nkt_kv, nqt_kv, npad;
  int32_t xcd_chunk_q, xcd_chunk_kv;  // workgroup chunks per XCD (0: launch_bwd's default)
  int32_t n_sink_tiles;  // leading key tiles whose step lists are split (0: none)
  int32_t nch;           // parts per split key tile
  int32_t sink, window, band, kv_head_offset, causal;
  int32_t n_bands;  // distinct long-range windows (head g takes g mod n_bands)
  int32_t o_f32, g_f32;
  float scale;
  float scale_log2;
};

// Launchers return a hipError_t value (0 on success).
int launch_fwd(const FwdParams& p, int d, int o_f32, void* stream);
int launch_decode(const DecodeParams& p, int d, int o_f32, void* stream);

// The current device's address of the library-owned decode scratch
// (COWA_DECODE_SCRATCH_BYTES, 256-byte aligned): looked up once per device.
// Returns a hipError_t value (0 on success).
int decode_scratch_address(void** ptr);

// Windowed KV cache (fill from a full cache / append one token).
struct KvWinParams {
  const uint16_t* k_src;  // fill: full cache [B, n_max, H_kv, d]; append: [B, H_kv, d]
  const uint16_t* v_src;
  const int32_t* seqlens;
  uint16_t* k_win;  // [B, rows, d], rows = heads x (sink rows + ring rows)
  uint16_t* v_win;
  int64_t ks_b, ks_t, ks_h;
  int64_t vs_b, vs_t, vs_h;
  int64_t kw_b, vw_b;
  int32_t B, Hkv, d, n_max;
  int32_t sink, window, band, kv_head_offset, n_bands;
};
int launch_kv_window_fill(const KvWinParams& p, int max_head_rows, void* stream);
int launch_kv_window_append(const KvWinParams& p, void* stream);
int launch_bwd(const BwdParams& p, int d, void* stream);

}  // namespace cowa
