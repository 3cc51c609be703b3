// libcowa C ABI: argument validation and dispatch to the gfx950 kernels.
// Every check runs on the host before anything is launched.
#include <math.h>

#include <vector>

#include "cowa_internal.h"

namespace cowa {

cowa_status validate_pattern(const cowa_pattern* p, int32_t h_kv_local) {
  if (!p) return COWA_ERR_INVALID_ARG;
  if (p->mode != COWA_MODE_COWA && p->mode != COWA_MODE_CAUSAL &&
      p->mode != COWA_MODE_SINK_LOCAL)
    return COWA_ERR_INVALID_ARG;
  if (p->n_ctx < 1 || p->sink < 0 || p->window < 1 || p->h_kv_global < 1 ||
      p->kv_head_offset < 0)
    return COWA_ERR_INVALID_ARG;
  if (h_kv_local < 1 || (int64_t)p->kv_head_offset + h_kv_local > p->h_kv_global)
    return COWA_ERR_INVALID_ARG;
  if (p->n_bands < 0 || p->n_bands > p->h_kv_global) return COWA_ERR_INVALID_ARG;
  return COWA_OK;
}

// Distinct long-range windows: n_bands, or one per global KV head.
int32_t resolve_n_bands(const cowa_pattern* p) {
  return p->n_bands > 0 ? p->n_bands : p->h_kv_global;
}

// A grid of `total` workgroups in the chunked XCD order (chunks of at most 8
// units of per_unit workgroups, or of at most 64 workgroups when chosen by
// balanced_chunks) is padded to whole rounds of kXcds chunks; the padded count
// must fit the 31-bit workgroup index.
bool grid_fits(int64_t total, int64_t per_unit) {
  const int64_t chunk = 8 * per_unit > 64 ? 8 * per_unit : 64;
  return total + (int64_t)kXcds * chunk <= 0x7fffffffLL;
}

int32_t resolve_band(const cowa_pattern* p) {
  if (p->mode == COWA_MODE_SINK_LOCAL) return 0;
  return p->band > 0 ? p->band : derive_band(p->n_ctx, p->window, p->h_kv_global);
}

DecodeGeometry decode_geometry(const cowa_pattern* p, int32_t B, int32_t H_q, int32_t H_kv_local,
                               int32_t d, int32_t n_max) {
  DecodeGeometry g;
  const int32_t L = resolve_band(p);
  const int32_t max_vis = max_row_count(p->sink, p->window, L, p->mode == COWA_MODE_CAUSAL, n_max);
  // aim for ~2048 workgroups (8 per compute unit) over all (b, head, split)
  const int64_t pairs = (int64_t)B * H_kv_local;
  int64_t want_splits = (2048 + pairs - 1) / pairs;
  if (want_splits < 1) want_splits = 1;
  int64_t chunk = (max_vis + want_splits - 1) / want_splits;
  chunk = (chunk + 63) / 64 * 64;
  if (chunk < 64) chunk = 64;
  if (chunk > kDecodeChunkMax) chunk = kDecodeChunkMax;
  g.chunk = (int32_t)chunk;
  g.n_splits = (int32_t)((max_vis + chunk - 1) / chunk);
  g.opart_offset = 0;
  const size_t opart_bytes = (size_t)g.n_splits * B * H_q * d * sizeof(float);
  g.lse_offset = g.opart_offset + (opart_bytes + 255) / 256 * 256;
  g.total_bytes = g.lse_offset + (size_t)g.n_splits * B * H_q * sizeof(float);
  return g;
}

}  // namespace cowa

using namespace cowa;

extern "C" const char* cowa_status_str(cowa_status s) {
  switch (s) {
    case COWA_OK: return "ok";
    case COWA_ERR_INVALID_ARG: return "invalid argument";
    case COWA_ERR_UNSUPPORTED: return "unsupported configuration";
    case COWA_ERR_WORKSPACE: return "workspace missing or too small";
    case COWA_ERR_PLAN_MISMATCH: return "plan does not match pattern, shape or tile";
    case COWA_ERR_HIP: return "HIP launch failed";
    case COWA_ERR_CAPACITY: return "plan buffers too small";
    case COWA_ERR_SCRATCH_LIMIT: return "problem needs more than the library's decode scratch";
  }
  return "unknown status";
}

extern "C" int32_t cowa_band_length(const cowa_pattern* p) {
  if (!p || validate_pattern(p, 1) != COWA_OK) return -1;
  return resolve_band(p);
}

extern "C" cowa_status cowa_fwd_block_sizes(int32_t d, int32_t* block_m, int32_t* block_n) {
  if (!block_m || !block_n) return COWA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return COWA_ERR_UNSUPPORTED;
  *block_m = kFwdBlockM;
  *block_n = kFwdBlockN;
  return COWA_OK;
}

extern "C" cowa_status cowa_visible_ranges(const cowa_pattern* p, int32_t h, int32_t t,
                                           int32_t lo[3], int32_t hi[3]) {
  if (!p || !lo || !hi || t < 0 || h < 0) return COWA_ERR_INVALID_ARG;
  cowa_status st = validate_pattern(p, h + 1);
  if (st != COWA_OK) return st;
  const HeadPattern hp = head_pattern(p->sink, p->window, resolve_band(p),
                                      band_slot(p->kv_head_offset + h, resolve_n_bands(p)),
                                      p->mode == COWA_MODE_CAUSAL);
  const RowRanges r = row_ranges(hp, t);
  for (int i = 0; i < 3; ++i) {
    lo[i] = r.lo[i];
    hi[i] = r.hi[i];
  }
  return COWA_OK;
}

// Plan sizes of recently seen shapes, per thread, so that checking a plan
// against its pattern does not rebuild it on every call.
static cowa_status plan_size_memo(const cowa_pattern* p, int32_t n, int32_t h_kv_local,
                                  int32_t bm, int32_t bn, int64_t* nnz) {
  struct Entry {
    cowa_pattern p;
    int32_t n, h, bm, bn;
    int64_t nnz;
    bool used;
  };
  thread_local Entry memo[8] = {};
  thread_local int next = 0;
  for (auto& e : memo) {
    if (e.used && e.n == n && e.h == h_kv_local && e.bm == bm && e.bn == bn &&
        e.p.n_ctx == p->n_ctx && e.p.sink == p->sink && e.p.window == p->window &&
        e.p.band == p->band && e.p.h_kv_global == p->h_kv_global &&
        e.p.kv_head_offset == p->kv_head_offset && e.p.mode == p->mode &&
        e.p.n_bands == p->n_bands) {
      *nnz = e.nnz;
      return COWA_OK;
    }
  }
  cowa_status st = plan_impl(p, n, h_kv_local, bm, bn, nullptr, nullptr, nullptr, 0, nnz);
  if (st != COWA_OK) return st;
  memo[next] = Entry{*p, n, h_kv_local, bm, bn, *nnz, true};
  next = (next + 1) & 7;
  return COWA_OK;
}

// Chunk sizes of the forward and dQ grids, chosen against the work of each
// workgroup.  Chunks are dealt to the XCDs in rounds of kXcds, alternating
// direction (xcd_logical), and the work of a workgroup is the row length of
// its (KV head, query tile) in the plan plus a fixed cost of a few steps, so
// the host can total every XCD's work for a candidate chunk size.  Sizes from
// 32 workgroups (one per compute unit of an XCD: those running together share
// its L2) to 64 are tried and the one whose busiest XCD carries the least work
// is kept (the larger on a tie).  0 asks the launcher for its default.
struct GridChoice {
  int32_t fwd, dq;
};

static double busiest_xcd(const std::vector<double>& prefix, int64_t chunk) {
  const int64_t n = (int64_t)prefix.size() - 1;
  double x[kXcds] = {};
  for (int64_t c = 0, a = 0; a < n; ++c, a += chunk) {
    const int64_t j = c / kXcds, r = c % kXcds;
    const int64_t xcd = (j & 1) ? kXcds - 1 - r : r;
    x[xcd] += prefix[a + chunk < n ? a + chunk : n] - prefix[a];
  }
  double m = 0;
  for (double v : x) m = v > m ? v : m;
  return m;
}

// Grids outside [2 * kXcds * 32, kMaxSearched] workgroups keep the default:
// too few for the search to matter, or so many that it would cost more host
// time and memory than it could save (and every XCD then gets many chunks).
constexpr int64_t kMaxSearched = 1 << 20;

static int32_t best_chunk(const std::vector<double>& work) {
  const int64_t n = (int64_t)work.size();
  std::vector<double> prefix(n + 1, 0.0);
  for (int64_t i = 0; i < n; ++i) prefix[i + 1] = prefix[i] + work[i];
  int32_t best = 0;
  double best_v = 0;
  for (int32_t c = 32; c <= 64; ++c) {
    const double v = busiest_xcd(prefix, c);
    if (best == 0 || v <= best_v * (1 + 1e-9)) {
      best = c;
      best_v = v;
    }
  }
  return best;
}

static cowa_status balanced_chunks(const cowa_pattern* p, int32_t N, int32_t H_kv_local,
                                   int32_t B, int32_t H_q, GridChoice* out) {
  struct Entry {
    cowa_pattern p;
    int32_t n, h, b, hq;
    GridChoice g;
    bool used;
  };
  thread_local Entry memo[8] = {};
  thread_local int next = 0;
  for (auto& e : memo) {
    if (e.used && e.n == N && e.h == H_kv_local && e.b == B && e.hq == H_q &&
        e.p.n_ctx == p->n_ctx && e.p.sink == p->sink && e.p.window == p->window &&
        e.p.band == p->band && e.p.h_kv_global == p->h_kv_global &&
        e.p.kv_head_offset == p->kv_head_offset && e.p.mode == p->mode &&
        e.p.n_bands == p->n_bands) {
      *out = e.g;
      return COWA_OK;
    }
  }
  const int32_t nqt = (N + kFwdBlockM - 1) / kFwdBlockM;
  const int64_t total = (int64_t)B * H_q * nqt;
  if (total < 2 * kXcds * 32 || total > kMaxSearched) {
    *out = GridChoice{0, 0};
    return COWA_OK;
  }
  std::vector<int32_t> rp((size_t)H_kv_local * nqt + 1);
  int64_t nnz = 0;
  cowa_status st = plan_impl(p, N, H_kv_local, kFwdBlockM, kFwdBlockN, rp.data(), nullptr,
                             nullptr, 0, &nnz);
  if (st != COWA_OK) return st;
  const int32_t G = H_q / H_kv_local;
  const double fixed = 4.0;  // steps' worth of set-up per workgroup
  auto work_of = [&](int32_t qi, int32_t hq) {
    const int32_t h = hq / G;
    return fixed + (rp[(size_t)h * nqt + qi + 1] - rp[(size_t)h * nqt + qi]);
  };
  std::vector<double> w(total);
  // forward order: query tiles heavy first, then (sequence, head)
  for (int64_t i = 0; i < total; ++i) {
    const int32_t qi = nqt - 1 - (int32_t)(i / ((int64_t)B * H_q));
    w[i] = work_of(qi, (int32_t)(i % ((int64_t)B * H_q)) % H_q);
  }
  GridChoice g;
  g.fwd = best_chunk(w);
  // dQ order: sequence, then query tiles heavy first, then head
  for (int64_t i = 0; i < total; ++i) {
    const int64_t rem = i % ((int64_t)nqt * H_q);
    w[i] = work_of(nqt - 1 - (int32_t)(rem / H_q), (int32_t)(rem % H_q));
  }
  g.dq = best_chunk(w);
  memo[next] = Entry{*p, N, H_kv_local, B, H_q, g, true};
  next = (next + 1) & 7;
  *out = g;
  return COWA_OK;
}

static bool strides_ok(const int64_t* s, int n) {
  for (int i = 0; i < n; ++i)
    if (s[i] < 0) return false;
  return true;
}

// The kernels move 16 bytes per lane from and to the start of every row: a
// tensor's base pointer must be 16-byte aligned and its n row strides
// (elements of elem_bytes each) multiples of 16 bytes.
static bool rows16(const void* base, const int64_t* strides, int n, int elem_bytes) {
  if (reinterpret_cast<uintptr_t>(base) & 15) return false;
  const int64_t m = 16 / elem_bytes;
  for (int i = 0; i < n; ++i)
    if (strides[i] % m) return false;
  return true;
}

// Prefill forward, batched (cu_seqlens NULL: [B, N, ...] with b strides) or
// packed (cu_seqlens: B sequences of length <= N at rows cu_seqlens[b]..).
static cowa_status fwd_impl(const cowa_pattern* p, const int32_t* d_row_ptr, const int32_t* d_col,
                            const uint8_t* d_flags, int64_t nnz, int32_t block_m,
                            int32_t block_n, const void* q, const void* k, const void* v,
                            void* o, int32_t o_dtype, float* lse, int32_t B, int32_t N,
                            int32_t H_q, int32_t H_kv_local, int32_t d,
                            const int64_t strides[12], float softmax_scale,
                            const int32_t* cu_seqlens, int32_t total_tokens, void* workspace,
                            size_t ws_bytes, void* stream) {
  cowa_status st = validate_pattern(p, H_kv_local);
  if (st != COWA_OK) return st;
  if (!d_row_ptr || !d_col || !d_flags || !q || !k || !v || !o || !lse || !strides)
    return COWA_ERR_INVALID_ARG;
  if (B < 1 || N < 1 || H_q < 1 || H_q % H_kv_local != 0) return COWA_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale)) return COWA_ERR_INVALID_ARG;
  if (o_dtype != COWA_DTYPE_BF16 && o_dtype != COWA_DTYPE_F32) return COWA_ERR_INVALID_ARG;
  if (!strides_ok(strides, 12)) return COWA_ERR_INVALID_ARG;
  if (!rows16(q, strides, 3, 2) || !rows16(k, strides + 3, 3, 2) || !rows16(v, strides + 6, 3, 2) ||
      !rows16(o, strides + 9, 3, o_dtype == COWA_DTYPE_F32 ? 4 : 2))
    return COWA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return COWA_ERR_UNSUPPORTED;
  if (block_m != kFwdBlockM || block_n != kFwdBlockN) return COWA_ERR_UNSUPPORTED;
  // per-lane byte offsets inside one K tile, and inside one tile of the
  // head-dim-major V copy (d rows of npad keys), are 31-bit (buffer loads)
  const int64_t npad = (N + (int64_t)kFwdBlockN - 1) / kFwdBlockN * kFwdBlockN;
  if ((int64_t)block_n * strides[4] >= (1LL << 30) || (int64_t)d * npad * 2 >= (1LL << 31))
    return COWA_ERR_UNSUPPORTED;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255) ||
      ws_bytes < fwd_workspace_bytes(B, N, H_kv_local, d))
    return COWA_ERR_WORKSPACE;
  const int64_t nqt = (N + block_m - 1) / block_m;
  if (!grid_fits((int64_t)B * nqt * H_q, (int64_t)B * H_q)) return COWA_ERR_UNSUPPORTED;
  int64_t want = 0;
  st = plan_size_memo(p, N, H_kv_local, block_m, block_n, &want);
  if (st != COWA_OK) return st;
  if (want != nnz) return COWA_ERR_PLAN_MISMATCH;

  FwdParams fp;
  fp.row_ptr = d_row_ptr;
  fp.col = d_col;
  fp.flags = d_flags;
  fp.q = static_cast<const uint16_t*>(q);
  fp.k = static_cast<const uint16_t*>(k);
  fp.v = static_cast<const uint16_t*>(v);
  fp.o = o;
  fp.lse = lse;
  fp.qs_b = strides[0]; fp.qs_t = strides[1]; fp.qs_h = strides[2];
  fp.ks_b = strides[3]; fp.ks_t = strides[4]; fp.ks_h = strides[5];
  fp.vs_b = strides[6]; fp.vs_t = strides[7]; fp.vs_h = strides[8];
  fp.os_b = strides[9]; fp.os_t = strides[10]; fp.os_h = strides[11];
  fp.B = B;
  fp.N = N;
  fp.Hq = H_q;
  fp.Hkv = H_kv_local;
  fp.G = H_q / H_kv_local;
  fp.nqt = (int32_t)nqt;
  fp.sink = p->sink;
  fp.window = p->window;
  fp.band = resolve_band(p);
  fp.kv_head_offset = p->kv_head_offset;
  fp.causal = p->mode == COWA_MODE_CAUSAL;
  fp.n_bands = resolve_n_bands(p);
  fp.cu_seqlens = cu_seqlens;
  fp.total_tokens = total_tokens;
  // packed sequences: lengths are on the device, so the launcher's default order
  fp.xcd_chunk = 0;
  if (!cu_seqlens) {
    GridChoice gc;
    st = balanced_chunks(p, N, H_kv_local, B, H_q, &gc);
    if (st != COWA_OK) return st;
    fp.xcd_chunk = gc.fwd;
  }
  fp.vt = static_cast<uint16_t*>(workspace);
  fp.npad = (int32_t)npad;
  fp.scale = softmax_scale;
  fp.scale_log2 = softmax_scale * 1.4426950408889634f;
  return launch_fwd(fp, d, o_dtype == COWA_DTYPE_F32, stream) == 0 ? COWA_OK : COWA_ERR_HIP;
}

extern "C" cowa_status cowa_fwd_workspace_size(int32_t B, int32_t N, int32_t H_kv_local,
                                               int32_t d, size_t* bytes) {
  if (!bytes || B < 1 || N < 1 || H_kv_local < 1) return COWA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return COWA_ERR_UNSUPPORTED;
  *bytes = fwd_workspace_bytes(B, N, H_kv_local, d);
  return COWA_OK;
}

extern "C" cowa_status cowa_fwd(const cowa_pattern* p, const int32_t* d_row_ptr,
                                const int32_t* d_col, const uint8_t* d_flags, int64_t nnz,
                                int32_t block_m, int32_t block_n, const void* q, const void* k,
                                const void* v, void* o, int32_t o_dtype, float* lse, int32_t B,
                                int32_t N, int32_t H_q, int32_t H_kv_local, int32_t d,
                                const int64_t strides[12], float softmax_scale,
                                void* workspace, size_t ws_bytes, void* stream) {
  return fwd_impl(p, d_row_ptr, d_col, d_flags, nnz, block_m, block_n, q, k, v, o, o_dtype, lse,
                  B, N, H_q, H_kv_local, d, strides, softmax_scale, nullptr, 0, workspace,
                  ws_bytes, stream);
}

extern "C" cowa_status cowa_fwd_varlen(const cowa_pattern* p, const int32_t* d_row_ptr,
                                       const int32_t* d_col, const uint8_t* d_flags, int64_t nnz,
                                       int32_t block_m, int32_t block_n, const void* q,
                                       const void* k, const void* v, void* o, int32_t o_dtype,
                                       float* lse, const int32_t* cu_seqlens, int32_t n_seqs,
                                       int32_t max_seqlen, int32_t total_tokens, int32_t H_q,
                                       int32_t H_kv_local, int32_t d, const int64_t strides[8],
                                       float softmax_scale, void* workspace, size_t ws_bytes,
                                       void* stream) {
  if (!cu_seqlens || !strides) return COWA_ERR_INVALID_ARG;
  if (n_seqs < 1 || total_tokens < 1 || max_seqlen < 1) return COWA_ERR_INVALID_ARG;
  // token rows: (t, h) strides; the per-sequence offset comes from cu_seqlens
  const int64_t full[12] = {0, strides[0], strides[1], 0, strides[2], strides[3],
                            0, strides[4], strides[5], 0, strides[6], strides[7]};
  return fwd_impl(p, d_row_ptr, d_col, d_flags, nnz, block_m, block_n, q, k, v, o, o_dtype, lse,
                  n_seqs, max_seqlen, H_q, H_kv_local, d, full, softmax_scale, cu_seqlens,
                  total_tokens, workspace, ws_bytes, stream);
}

extern "C" cowa_status cowa_decode_workspace_size(const cowa_pattern* p, int32_t B, int32_t H_q,
                                                  int32_t H_kv_local, int32_t d, int32_t n_max,
                                                  size_t* bytes) {
  cowa_status st = validate_pattern(p, H_kv_local);
  if (st != COWA_OK) return st;
  if (!bytes || B < 1 || H_q < 1 || H_q % H_kv_local != 0 || n_max < 1)
    return COWA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return COWA_ERR_UNSUPPORTED;
  *bytes = decode_geometry(p, B, H_q, H_kv_local, d, n_max).total_bytes;
  return COWA_OK;
}

// Decode against a full cache (win = 0: strides[2..7] = k b,t,h and v b,t,h)
// or against the windowed layout (win = 1: rows of d contiguous values,
// strides[2] and strides[5] = the per-sequence stride of k_win and v_win).
static cowa_status decode_impl(const cowa_pattern* p, const void* q, const void* k,
                               const void* v, const int32_t* cache_seqlens, void* o,
                               int32_t o_dtype, float* lse, int32_t B, int32_t H_q,
                               int32_t H_kv_local, int32_t d, int32_t n_max,
                               const int64_t strides[10], float softmax_scale, void* workspace,
                               size_t ws_bytes, void* stream, int win,
                               bool noalloc = false) {
  cowa_status st = validate_pattern(p, H_kv_local);
  if (st != COWA_OK) return st;
  if (!q || !k || !v || !cache_seqlens || !o || !lse || !strides) return COWA_ERR_INVALID_ARG;
  if (B < 1 || H_q < 1 || n_max < 1 || H_q % H_kv_local != 0) return COWA_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale)) return COWA_ERR_INVALID_ARG;
  if (o_dtype != COWA_DTYPE_BF16 && o_dtype != COWA_DTYPE_F32) return COWA_ERR_INVALID_ARG;
  if (!strides_ok(strides, 10)) return COWA_ERR_INVALID_ARG;
  if (!rows16(q, strides, 2, 2) || !rows16(k, strides + 2, 3, 2) || !rows16(v, strides + 5, 3, 2))
    return COWA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return COWA_ERR_UNSUPPORTED;
  if (win && p->mode == COWA_MODE_CAUSAL) return COWA_ERR_UNSUPPORTED;
  const int32_t G = H_q / H_kv_local;
  if (G > kDecodeMaxGroup) return COWA_ERR_UNSUPPORTED;
  const DecodeGeometry geo = decode_geometry(p, B, H_q, H_kv_local, d, n_max);
  // grid (splits, H_kv_local, B): splits are at most ceil(n_max / 64); the
  // other two dimensions are limited to 65535
  if (B > 65535 || H_kv_local > 65535) return COWA_ERR_UNSUPPORTED;
  if (noalloc) {
    // the library's own scratch (cowa_decode_noalloc): no caller workspace
    if (geo.total_bytes > COWA_DECODE_SCRATCH_BYTES) return COWA_ERR_SCRATCH_LIMIT;
    if (decode_scratch_address(&workspace) != 0) return COWA_ERR_HIP;
    ws_bytes = COWA_DECODE_SCRATCH_BYTES;
  }
  if (!workspace || ws_bytes < geo.total_bytes || (reinterpret_cast<uintptr_t>(workspace) & 255))
    return COWA_ERR_WORKSPACE;

  DecodeParams dp;
  dp.q = static_cast<const uint16_t*>(q);
  dp.k = static_cast<const uint16_t*>(k);
  dp.v = static_cast<const uint16_t*>(v);
  dp.seqlens = cache_seqlens;
  dp.o = o;
  dp.lse = lse;
  dp.opart = reinterpret_cast<float*>(static_cast<char*>(workspace) + geo.opart_offset);
  dp.lsepart = reinterpret_cast<float*>(static_cast<char*>(workspace) + geo.lse_offset);
  dp.qs_b = strides[0]; dp.qs_h = strides[1];
  dp.ks_b = strides[2]; dp.ks_t = strides[3]; dp.ks_h = strides[4];
  dp.vs_b = strides[5]; dp.vs_t = strides[6]; dp.vs_h = strides[7];
  dp.os_b = strides[8]; dp.os_h = strides[9];
  dp.B = B;
  dp.Hq = H_q;
  dp.Hkv = H_kv_local;
  dp.G = G;
  dp.n_max = n_max;
  dp.sink = p->sink;
  dp.window = p->window;
  dp.band = resolve_band(p);
  dp.kv_head_offset = p->kv_head_offset;
  dp.causal = p->mode == COWA_MODE_CAUSAL;
  dp.n_bands = resolve_n_bands(p);
  dp.chunk = geo.chunk;
  dp.n_splits = geo.n_splits;
  dp.o_f32 = o_dtype == COWA_DTYPE_F32;
  dp.win = win;
  dp.scale = softmax_scale;
  dp.scale_log2 = softmax_scale * 1.4426950408889634f;
  return launch_decode(dp, d, o_dtype == COWA_DTYPE_F32, stream) == 0 ? COWA_OK : COWA_ERR_HIP;
}

extern "C" cowa_status cowa_decode(const cowa_pattern* p, const void* q, const void* k_cache,
                                   const void* v_cache, const int32_t* cache_seqlens, void* o,
                                   int32_t o_dtype, float* lse, int32_t B, int32_t H_q,
                                   int32_t H_kv_local, int32_t d, int32_t n_max,
                                   const int64_t strides[10], float softmax_scale,
                                   void* workspace, size_t ws_bytes, void* stream) {
  return decode_impl(p, q, k_cache, v_cache, cache_seqlens, o, o_dtype, lse, B, H_q, H_kv_local,
                     d, n_max, strides, softmax_scale, workspace, ws_bytes, stream, 0);
}

extern "C" cowa_status cowa_decode_noalloc(const cowa_pattern* p, const void* q,
                                           const void* k_cache, const void* v_cache,
                                           const int32_t* cache_seqlens, void* o, int32_t o_dtype,
                                           float* lse, int32_t B, int32_t H_q,
                                           int32_t H_kv_local, int32_t d, int32_t n_max,
                                           const int64_t strides[10], float softmax_scale,
                                           void* stream) {
  return decode_impl(p, q, k_cache, v_cache, cache_seqlens, o, o_dtype, lse, B, H_q, H_kv_local,
                     d, n_max, strides, softmax_scale, nullptr, 0, stream, 0, true);
}

// ---- windowed KV cache ----

static cowa_status window_rows(const cowa_pattern* p, int32_t h_kv_local, int32_t n_max,
                               int32_t* head_rows, int64_t* total, int32_t* max_rows) {
  cowa_status st = validate_pattern(p, h_kv_local);
  if (st != COWA_OK) return st;
  if (n_max < 1) return COWA_ERR_INVALID_ARG;
  if (p->mode == COWA_MODE_CAUSAL) return COWA_ERR_UNSUPPORTED;
  const int32_t L = resolve_band(p);
  const int32_t m = resolve_n_bands(p);
  const int32_t s_rows = window_sink_rows(p->sink, n_max);
  int64_t sum = 0;
  int32_t mx = 0;
  for (int32_t h = 0; h < h_kv_local; ++h) {
    const int32_t r =
        s_rows + window_ring_rows(p->sink, p->window, L, band_slot(p->kv_head_offset + h, m), n_max);
    if (head_rows) head_rows[h] = r;
    sum += r;
    mx = r > mx ? r : mx;
  }
  if (total) *total = sum;
  if (max_rows) *max_rows = mx;
  return COWA_OK;
}

extern "C" cowa_status cowa_kv_window_rows(const cowa_pattern* p, int32_t h_kv_local,
                                           int32_t n_max, int32_t* head_rows,
                                           int64_t* total_rows) {
  if (!total_rows) return COWA_ERR_INVALID_ARG;
  return window_rows(p, h_kv_local, n_max, head_rows, total_rows, nullptr);
}

static cowa_status kvwin_common(const cowa_pattern* p, int32_t B, int32_t H_kv_local, int32_t d,
                                int32_t n_max, const int64_t* win_strides, KvWinParams* kp,
                                int32_t* max_rows) {
  int64_t total = 0;
  cowa_status st = window_rows(p, H_kv_local, n_max, nullptr, &total, max_rows);
  if (st != COWA_OK) return st;
  if (B < 1 || B > 65535 || H_kv_local > 65535) return COWA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return COWA_ERR_UNSUPPORTED;
  // each sequence's rows must fit its stride
  if (win_strides[0] < total * d || win_strides[1] < total * d) return COWA_ERR_INVALID_ARG;
  kp->kw_b = win_strides[0];
  kp->vw_b = win_strides[1];
  kp->B = B;
  kp->Hkv = H_kv_local;
  kp->d = d;
  kp->n_max = n_max;
  kp->sink = p->sink;
  kp->window = p->window;
  kp->band = resolve_band(p);
  kp->kv_head_offset = p->kv_head_offset;
  kp->n_bands = resolve_n_bands(p);
  return COWA_OK;
}

extern "C" cowa_status cowa_kv_window_fill(const cowa_pattern* p, const void* k_cache,
                                           const void* v_cache, const int32_t* cache_seqlens,
                                           void* k_win, void* v_win, int32_t B,
                                           int32_t H_kv_local, int32_t d, int32_t n_max,
                                           const int64_t strides[8], void* stream) {
  if (!k_cache || !v_cache || !cache_seqlens || !k_win || !v_win || !strides)
    return COWA_ERR_INVALID_ARG;
  if (!strides_ok(strides, 8)) return COWA_ERR_INVALID_ARG;
  if (!rows16(k_cache, strides, 3, 2) || !rows16(v_cache, strides + 3, 3, 2) ||
      !rows16(k_win, strides + 6, 1, 2) || !rows16(v_win, strides + 7, 1, 2))
    return COWA_ERR_INVALID_ARG;
  KvWinParams kp;
  int32_t max_rows = 0;
  cowa_status st = kvwin_common(p, B, H_kv_local, d, n_max, strides + 6, &kp, &max_rows);
  if (st != COWA_OK) return st;
  kp.k_src = static_cast<const uint16_t*>(k_cache);
  kp.v_src = static_cast<const uint16_t*>(v_cache);
  kp.seqlens = cache_seqlens;
  kp.k_win = static_cast<uint16_t*>(k_win);
  kp.v_win = static_cast<uint16_t*>(v_win);
  kp.ks_b = strides[0]; kp.ks_t = strides[1]; kp.ks_h = strides[2];
  kp.vs_b = strides[3]; kp.vs_t = strides[4]; kp.vs_h = strides[5];
  if (max_rows == 0) return COWA_OK;
  return launch_kv_window_fill(kp, max_rows, stream) == 0 ? COWA_OK : COWA_ERR_HIP;
}

extern "C" cowa_status cowa_kv_window_append(const cowa_pattern* p, const void* k_new,
                                             const void* v_new, const int32_t* cache_seqlens,
                                             void* k_win, void* v_win, int32_t B,
                                             int32_t H_kv_local, int32_t d, int32_t n_max,
                                             const int64_t strides[6], void* stream) {
  if (!k_new || !v_new || !cache_seqlens || !k_win || !v_win || !strides)
    return COWA_ERR_INVALID_ARG;
  if (!strides_ok(strides, 6)) return COWA_ERR_INVALID_ARG;
  if (!rows16(k_new, strides, 2, 2) || !rows16(v_new, strides + 2, 2, 2) ||
      !rows16(k_win, strides + 4, 1, 2) || !rows16(v_win, strides + 5, 1, 2))
    return COWA_ERR_INVALID_ARG;
  KvWinParams kp;
  cowa_status st = kvwin_common(p, B, H_kv_local, d, n_max, strides + 4, &kp, nullptr);
  if (st != COWA_OK) return st;
  kp.k_src = static_cast<const uint16_t*>(k_new);
  kp.v_src = static_cast<const uint16_t*>(v_new);
  kp.seqlens = cache_seqlens;
  kp.k_win = static_cast<uint16_t*>(k_win);
  kp.v_win = static_cast<uint16_t*>(v_win);
  kp.ks_b = strides[0]; kp.ks_t = 0; kp.ks_h = strides[1];
  kp.vs_b = strides[2]; kp.vs_t = 0; kp.vs_h = strides[3];
  return launch_kv_window_append(kp, stream) == 0 ? COWA_OK : COWA_ERR_HIP;
}

extern "C" cowa_status cowa_decode_window(const cowa_pattern* p, const void* q, const void* k_win,
                                          const void* v_win, const int32_t* cache_seqlens,
                                          void* o, int32_t o_dtype, float* lse, int32_t B,
                                          int32_t H_q, int32_t H_kv_local, int32_t d,
                                          int32_t n_max, const int64_t strides[6],
                                          float softmax_scale, void* workspace, size_t ws_bytes,
                                          void* stream) {
  if (!strides) return COWA_ERR_INVALID_ARG;
  int64_t total = 0;
  cowa_status st = window_rows(p, H_kv_local, n_max, nullptr, &total, nullptr);
  if (st != COWA_OK) return st;
  if (strides[2] < total * d || strides[3] < total * d) return COWA_ERR_INVALID_ARG;
  // windowed rows are d contiguous values; the head offset is a row offset
  const int64_t full[10] = {strides[0], strides[1], strides[2], d, 0,
                            strides[3], d, 0, strides[4], strides[5]};
  return decode_impl(p, q, k_win, v_win, cache_seqlens, o, o_dtype, lse, B, H_q, H_kv_local, d,
                     n_max, full, softmax_scale, workspace, ws_bytes, stream, 1);
}

extern "C" cowa_status cowa_bwd_block_sizes(int32_t d, int32_t* block_m, int32_t* block_n) {
  if (!block_m || !block_n) return COWA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return COWA_ERR_UNSUPPORTED;
  *block_m = kBwdBlockM;
  *block_n = kBwdBlockN;
  return COWA_OK;
}

namespace {
// Workspace of the backward: LSE2 and D, each [B, H_q, npad] fp32, then the
// fp32 dK/dV partials of the key tiles that hold sink keys.  Those tiles are
// seen by every query tile, so their step lists (query heads x query tiles)
// are cut into nch parts when they exceed twice the mean step count of a key
// tile; the parts run as separate workgroups and a reduction sums them in a
// fixed order.
struct BwdGeometry {
  int32_t npad, n_sink_tiles, nch;
  size_t delta_offset, part_offset, total_bytes;
};
cowa_status bwd_geometry(const cowa_pattern* p, int32_t B, int32_t H_q, int32_t H_kv_local,
                         int32_t N, BwdGeometry* g) {
  g->npad = (N + kBwdBlockM - 1) / kBwdBlockM * kBwdBlockM;
  const size_t one = ((size_t)B * H_q * g->npad * sizeof(float) + 255) / 256 * 256;
  g->delta_offset = one;
  g->part_offset = 2 * one;
  const int32_t nkt = (N + kBwdBlockN - 1) / kBwdBlockN;
  const int32_t nqt = (N + kBwdBlockM - 1) / kBwdBlockM;
  const int64_t G = H_q / H_kv_local;
  int64_t nnz = 0;
  cowa_status st = plan_size_memo(p, N, H_kv_local, kBwdBlockM, kBwdBlockN, &nnz);
  if (st != COWA_OK) return st;
  const int64_t mean_steps = (G * nnz + (int64_t)H_kv_local * nkt - 1) / ((int64_t)H_kv_local * nkt);
  const int64_t cap = mean_steps * 2 > 256 ? mean_steps * 2 : 256;
  const int64_t nch = (G * nqt + cap - 1) / cap;
  const int32_t sink_tiles = (int32_t)(((int64_t)p->sink + kBwdBlockN - 1) / kBwdBlockN);
  g->n_sink_tiles = nch > 1 ? (sink_tiles < nkt ? sink_tiles : nkt) : 0;
  g->nch = g->n_sink_tiles > 0 ? (int32_t)nch : 1;
  // partial rows are sized for the largest head dimension (128)
  const size_t part_bytes = (size_t)B * H_kv_local * g->n_sink_tiles * g->nch * 2 * kBwdBlockN *
                            128 * sizeof(float);
  g->total_bytes = g->part_offset + part_bytes;
  return COWA_OK;
}
}  // namespace

extern "C" cowa_status cowa_bwd_workspace_size(const cowa_pattern* p, int32_t B, int32_t H_q,
                                               int32_t H_kv_local, int32_t N, size_t* bytes) {
  cowa_status st = validate_pattern(p, H_kv_local);
  if (st != COWA_OK) return st;
  if (!bytes || B < 1 || H_q < 1 || N < 1 || H_q % H_kv_local != 0) return COWA_ERR_INVALID_ARG;
  BwdGeometry g;
  st = bwd_geometry(p, B, H_q, H_kv_local, N, &g);
  if (st != COWA_OK) return st;
  *bytes = g.total_bytes;
  return COWA_OK;
}

// The backward for the batched layout (cu_seqlens NULL) or for packed
// sequences (B = n_seqs, N = max_seqlen, b strides 0).
static cowa_status bwd_impl(const cowa_pattern* p, const int32_t* d_row_ptr,
                            const int32_t* d_col, const uint8_t* d_flags, int64_t nnz,
                            int32_t block_m, int32_t block_n, const int32_t* d_row_ptr_kv,
                            const int32_t* d_col_kv, const uint8_t* d_flags_kv, int64_t nnz_kv,
                            int32_t block_m_kv, int32_t block_n_kv, const void* q, const void* k,
                            const void* v, const void* o, int32_t o_dtype, const void* dout,
                            const float* lse, void* dq, void* dk, void* dv, int32_t g_dtype,
                            int32_t B, int32_t N, int32_t H_q, int32_t H_kv_local, int32_t d,
                            const int64_t strides[24], float softmax_scale, void* workspace,
                            size_t ws_bytes, void* stream, const int32_t* cu_seqlens,
                            int32_t total_tokens) {
  cowa_status st = validate_pattern(p, H_kv_local);
  if (st != COWA_OK) return st;
  if (!d_row_ptr || !d_col || !d_flags || !d_row_ptr_kv || !d_col_kv || !d_flags_kv || !q ||
      !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !strides)
    return COWA_ERR_INVALID_ARG;
  if (B < 1 || N < 1 || H_q < 1 || H_q % H_kv_local != 0) return COWA_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale)) return COWA_ERR_INVALID_ARG;
  if (o_dtype != COWA_DTYPE_BF16 && o_dtype != COWA_DTYPE_F32) return COWA_ERR_INVALID_ARG;
  if (g_dtype != COWA_DTYPE_BF16 && g_dtype != COWA_DTYPE_F32) return COWA_ERR_INVALID_ARG;
  if (!strides_ok(strides, 24)) return COWA_ERR_INVALID_ARG;
  {
    const int ob = o_dtype == COWA_DTYPE_F32 ? 4 : 2, gb = g_dtype == COWA_DTYPE_F32 ? 4 : 2;
    const void* bases[8] = {q, k, v, o, dout, dq, dk, dv};
    const int bytes[8] = {2, 2, 2, ob, 2, gb, gb, gb};
    for (int i = 0; i < 8; ++i)
      if (!rows16(bases[i], strides + 3 * i, 3, bytes[i])) return COWA_ERR_INVALID_ARG;
  }
  if (d != 64 && d != 128) return COWA_ERR_UNSUPPORTED;
  if (block_m != kFwdBlockM || block_n != kFwdBlockN || block_m_kv != kBwdBlockM ||
      block_n_kv != kBwdBlockN)
    return COWA_ERR_UNSUPPORTED;
  // per-lane byte offsets inside one 64-row tile are 31-bit (buffer loads)
  const int tile_strides[4] = {1, 4, 7, 13};  // q, k, v, dout row strides
  for (int i : tile_strides)
    if ((int64_t)64 * strides[i] >= (1LL << 30)) return COWA_ERR_UNSUPPORTED;
  const int64_t nqt = (N + block_m - 1) / block_m;
  const int64_t nkt_kv = (N + block_n_kv - 1) / block_n_kv;
  if (!grid_fits((int64_t)B * nqt * H_q, H_q) ||
      !grid_fits((int64_t)B * H_kv_local * nkt_kv, (int64_t)B * H_kv_local) ||
      B > 65535 || H_q > 65535)
    return COWA_ERR_UNSUPPORTED;
  int64_t want = 0;
  st = plan_size_memo(p, N, H_kv_local, block_m, block_n, &want);
  if (st != COWA_OK) return st;
  if (want != nnz) return COWA_ERR_PLAN_MISMATCH;
  // the key-major plan holds the same tiles as the query-major one of its shape
  st = plan_size_memo(p, N, H_kv_local, block_m_kv, block_n_kv, &want);
  if (st != COWA_OK) return st;
  if (want != nnz_kv) return COWA_ERR_PLAN_MISMATCH;
  BwdGeometry geo;
  st = bwd_geometry(p, B, H_q, H_kv_local, N, &geo);
  if (st != COWA_OK) return st;
  if (!workspace || ws_bytes < geo.total_bytes || (reinterpret_cast<uintptr_t>(workspace) & 255))
    return COWA_ERR_WORKSPACE;
  if (!grid_fits((int64_t)B * H_kv_local * (nkt_kv + (int64_t)geo.n_sink_tiles * (geo.nch - 1)),
                 (int64_t)B * H_kv_local))
    return COWA_ERR_UNSUPPORTED;

  BwdParams bp;
  bp.row_ptr = d_row_ptr;
  bp.col = d_col;
  bp.flags = d_flags;
  bp.row_ptr_kv = d_row_ptr_kv;
  bp.col_kv = d_col_kv;
  bp.flags_kv = d_flags_kv;
  bp.q = static_cast<const uint16_t*>(q);
  bp.k = static_cast<const uint16_t*>(k);
  bp.v = static_cast<const uint16_t*>(v);
  bp.o = o;
  bp.dout = static_cast<const uint16_t*>(dout);
  bp.lse = lse;
  bp.dq = dq;
  bp.dk = dk;
  bp.dv = dv;
  bp.lse2 = static_cast<float*>(workspace);
  bp.delta = reinterpret_cast<float*>(static_cast<char*>(workspace) + geo.delta_offset);
  bp.part = reinterpret_cast<float*>(static_cast<char*>(workspace) + geo.part_offset);
  bp.n_sink_tiles = geo.n_sink_tiles;
  bp.nch = geo.nch;
  int64_t* const dst[24] = {&bp.qs_b,  &bp.qs_t,  &bp.qs_h,  &bp.ks_b,  &bp.ks_t,  &bp.ks_h,
                            &bp.vs_b,  &bp.vs_t,  &bp.vs_h,  &bp.os_b,  &bp.os_t,  &bp.os_h,
                            &bp.dos_b, &bp.dos_t, &bp.dos_h, &bp.dqs_b, &bp.dqs_t, &bp.dqs_h,
                            &bp.dks_b, &bp.dks_t, &bp.dks_h, &bp.dvs_b, &bp.dvs_t, &bp.dvs_h};
  for (int i = 0; i < 24; ++i) *dst[i] = strides[i];
  bp.B = B;
  bp.N = N;
  bp.Hq = H_q;
  bp.Hkv = H_kv_local;
  bp.G = H_q / H_kv_local;
  bp.nqt = (int32_t)nqt;
  bp.nkt_kv = (int32_t)nkt_kv;
  bp.nqt_kv = (N + block_m_kv - 1) / block_m_kv;
  bp.npad = geo.npad;
  bp.sink = p->sink;
  bp.window = p->window;
  bp.band = resolve_band(p);
  bp.kv_head_offset = p->kv_head_offset;
  bp.causal = p->mode == COWA_MODE_CAUSAL;
  bp.n_bands = resolve_n_bands(p);
  bp.o_f32 = o_dtype == COWA_DTYPE_F32;
  bp.g_f32 = g_dtype == COWA_DTYPE_F32;
  bp.scale = softmax_scale;
  bp.scale_log2 = softmax_scale * 1.4426950408889634f;
  bp.cu_seqlens = cu_seqlens;
  bp.total_tokens = total_tokens;
  bp.xcd_chunk_q = 0;
  bp.xcd_chunk_kv = 0;
  if (!cu_seqlens) {
    GridChoice gc;
    st = balanced_chunks(p, N, H_kv_local, B, H_q, &gc);
    if (st != COWA_OK) return st;
    bp.xcd_chunk_q = gc.dq;
  }
  return launch_bwd(bp, d, stream) == 0 ? COWA_OK : COWA_ERR_HIP;
}

extern "C" cowa_status cowa_bwd(const cowa_pattern* p, const int32_t* d_row_ptr,
                                const int32_t* d_col, const uint8_t* d_flags, int64_t nnz,
                                int32_t block_m, int32_t block_n, const int32_t* d_row_ptr_kv,
                                const int32_t* d_col_kv, const uint8_t* d_flags_kv,
                                int64_t nnz_kv, int32_t block_m_kv, int32_t block_n_kv,
                                const void* q, const void* k, const void* v, const void* o,
                                int32_t o_dtype, const void* dout, const float* lse, void* dq,
                                void* dk, void* dv, int32_t g_dtype, int32_t B, int32_t N,
                                int32_t H_q, int32_t H_kv_local, int32_t d,
                                const int64_t strides[24], float softmax_scale, void* workspace,
                                size_t ws_bytes, void* stream) {
  return bwd_impl(p, d_row_ptr, d_col, d_flags, nnz, block_m, block_n, d_row_ptr_kv, d_col_kv,
                  d_flags_kv, nnz_kv, block_m_kv, block_n_kv, q, k, v, o, o_dtype, dout, lse, dq,
                  dk, dv, g_dtype, B, N, H_q, H_kv_local, d, strides, softmax_scale, workspace,
                  ws_bytes, stream, nullptr, 0);
}

extern "C" cowa_status cowa_bwd_varlen(
    const cowa_pattern* p, const int32_t* d_row_ptr, const int32_t* d_col,
    const uint8_t* d_flags, int64_t nnz, int32_t block_m, int32_t block_n,
    const int32_t* d_row_ptr_kv, const int32_t* d_col_kv, const uint8_t* d_flags_kv,
    int64_t nnz_kv, int32_t block_m_kv, int32_t block_n_kv, const void* q, const void* k,
    const void* v, const void* o, int32_t o_dtype, const void* dout, const float* lse, void* dq,
    void* dk, void* dv, int32_t g_dtype, const int32_t* cu_seqlens, int32_t n_seqs,
    int32_t max_seqlen, int32_t total_tokens, int32_t H_q, int32_t H_kv_local, int32_t d,
    const int64_t strides[16], float softmax_scale, void* workspace, size_t ws_bytes,
    void* stream) {
  if (!cu_seqlens || !strides) return COWA_ERR_INVALID_ARG;
  if (n_seqs < 1 || total_tokens < 1 || max_seqlen < 1) return COWA_ERR_INVALID_ARG;
  // token rows: (t, h) strides of q, k, v, o, dout, dq, dk, dv; the per-sequence
  // offset comes from cu_seqlens
  int64_t full[24];
  for (int i = 0; i < 8; ++i) {
    full[3 * i] = 0;
    full[3 * i + 1] = strides[2 * i];
    full[3 * i + 2] = strides[2 * i + 1];
  }
  return bwd_impl(p, d_row_ptr, d_col, d_flags, nnz, block_m, block_n, d_row_ptr_kv, d_col_kv,
                  d_flags_kv, nnz_kv, block_m_kv, block_n_kv, q, k, v, o, o_dtype, dout, lse, dq,
                  dk, dv, g_dtype, n_seqs, max_seqlen, H_q, H_kv_local, d, full, softmax_scale,
                  workspace, ws_bytes, stream, cu_seqlens, total_tokens);
}
