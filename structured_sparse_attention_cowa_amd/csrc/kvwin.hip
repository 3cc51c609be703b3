// Windowed KV cache for decode: fill from a full cache, append one token.
//
// "CoWindow Attention: Full Causal Coverage Is a Collective Property"
// (Abstract) reports per-rank decode memory well below FullAttn's.  With the
// pattern fixed by positions, a KV head never reads a non-sink key again once
// it lies W + (b+1) L or more behind the newest query (b: the head's
// long-range window), so each head keeps only its sink rows and a ring of the
// most recent positions (ring size and mapping in cowa_pattern.h).
//
// Layout of one sequence: local KV heads stacked, each head's S' sink rows then
// its R ring rows, every row d contiguous bf16 values.
#include <hip/hip_runtime.h>

#include "cowa_internal.h"

namespace cowa {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int64_t head_first_row(const KvWinParams& p, int h) {
  const int s_rows = window_sink_rows(p.sink, p.n_max);
  int64_t r = 0;
  for (int i = 0; i < h; ++i)
    r += s_rows + window_ring_rows(p.sink, p.window, p.band,
                                   band_slot(p.kv_head_offset + i, p.n_bands), p.n_max);
  return r;
}

// Grid (ceil(max head rows / rows per block), H_kv_local, B); one 16-byte
// chunk per thread.  Ring row r holds the newest position j <= len - 1 with
// j >= S' and (j - S') mod R = r; rows that hold no position yet are zeroed.
__global__ __launch_bounds__(256) void cowa_kv_window_fill_kernel(KvWinParams p) {
  const int cpr = p.d / 8;  // chunks per row
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int s_rows = window_sink_rows(p.sink, p.n_max);
  const int ring = window_ring_rows(p.sink, p.window, p.band,
                                    band_slot(p.kv_head_offset + h, p.n_bands), p.n_max);
  const int rows_per_block = 256 / cpr;
  const int r = blockIdx.x * rows_per_block + threadIdx.x / cpr;
  const int c = threadIdx.x % cpr;
  if (r >= s_rows + ring) return;
  int len = p.seqlens[b];
  len = len < 1 ? 1 : (len > p.n_max ? p.n_max : len);
  int j = -1;
  if (r < s_rows) {
    j = r < len ? r : -1;
  } else {
    const int rr = r - s_rows;
    const int last = len - 1 - s_rows - rr;  // >= 0 iff some position maps here
    if (last >= 0) j = s_rows + rr + (last / ring) * ring;
  }
  const int64_t wrow = head_first_row(p, h) + r;
  u32x4* kd = reinterpret_cast<u32x4*>(p.k_win + (int64_t)b * p.kw_b + wrow * p.d) + c;
  u32x4* vd = reinterpret_cast<u32x4*>(p.v_win + (int64_t)b * p.vw_b + wrow * p.d) + c;
  if (j < 0) {
    *kd = u32x4{};
    *vd = u32x4{};
    return;
  }
  *kd = *(reinterpret_cast<const u32x4*>(p.k_src + (int64_t)b * p.ks_b + (int64_t)j * p.ks_t +
                                         (int64_t)h * p.ks_h) + c);
  *vd = *(reinterpret_cast<const u32x4*>(p.v_src + (int64_t)b * p.vs_b + (int64_t)j * p.vs_t +
                                         (int64_t)h * p.vs_h) + c);
}

// Grid (H_kv_local, B), 64 threads: the token at position len - 1 (its K and V
// rows in k_src/v_src at [b, h]) goes to its sink or ring row.
__global__ __launch_bounds__(64) void cowa_kv_window_append_kernel(KvWinParams p) {
  const int cpr = p.d / 8;
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int s_rows = window_sink_rows(p.sink, p.n_max);
  const int ring = window_ring_rows(p.sink, p.window, p.band,
                                    band_slot(p.kv_head_offset + h, p.n_bands), p.n_max);
  int len = p.seqlens[b];
  len = len < 1 ? 1 : (len > p.n_max ? p.n_max : len);
  const int j = len - 1;
  const int r = j < s_rows ? j : s_rows + (j - s_rows) % ring;
  const int64_t wrow = head_first_row(p, h) + r;
  for (int c = threadIdx.x; c < 2 * cpr; c += 64) {
    const bool is_v = c >= cpr;
    const int cc = is_v ? c - cpr : c;
    const uint16_t* src = is_v ? p.v_src + (int64_t)b * p.vs_b + (int64_t)h * p.vs_h
                               : p.k_src + (int64_t)b * p.ks_b + (int64_t)h * p.ks_h;
    uint16_t* dst = is_v ? p.v_win + (int64_t)b * p.vw_b + wrow * p.d
                         : p.k_win + (int64_t)b * p.kw_b + wrow * p.d;
    reinterpret_cast<u32x4*>(dst)[cc] = reinterpret_cast<const u32x4*>(src)[cc];
  }
}

}  // namespace

int launch_kv_window_fill(const KvWinParams& p, int max_head_rows, void* stream) {
  const int rows_per_block = 256 / (p.d / 8);
  const dim3 grid((unsigned)((max_head_rows + rows_per_block - 1) / rows_per_block),
                  (unsigned)p.Hkv, (unsigned)p.B);
  hipLaunchKernelGGL(cowa_kv_window_fill_kernel, grid, dim3(256), 0,
                     static_cast<hipStream_t>(stream), p);
  return (int)hipGetLastError();
}

int launch_kv_window_append(const KvWinParams& p, void* stream) {
  hipLaunchKernelGGL(cowa_kv_window_append_kernel, dim3((unsigned)p.Hkv, (unsigned)p.B), dim3(64),
                     0, static_cast<hipStream_t>(stream), p);
  return (int)hipGetLastError();
}

}  // namespace cowa
