// cowa_plan: visible-tile lists per (global KV head, query tile), host only.
//
// The pattern is fixed by positions and the global KV-head index, so the
// lists need no router or indexer ("Splitting long-range windows across KV
// heads beats duplicating them at lower cost", efficiency paragraph).
//
// Method: for each query row t of a query tile the visible keys are at most
// three disjoint ranges (sink, band, local).  After merging adjacent ranges,
// a key tile is touched by row t iff it meets one merged range, and lies
// wholly inside row t's visible set iff it lies inside one merged range.
// Two difference arrays over key tiles count, per tile, the rows that touch
// it and the rows that cover it; a tile is listed if touched at least once
// and full if covered by all block_m rows.
#include <string.h>

#include <vector>

#include "cowa_internal.h"

namespace cowa {

cowa_status plan_impl(const cowa_pattern* p, int32_t n, int32_t h_kv_local, int32_t bm,
                      int32_t bn, int32_t* row_ptr, int32_t* col, uint8_t* flags, int64_t cap,
                      int64_t* nnz_out) {
  cowa_status st = validate_pattern(p, h_kv_local);
  if (st != COWA_OK) return st;
  if (n < 1 || bm < 1 || bn < 1 || bm > (1 << 16) || bn > (1 << 16))
    return COWA_ERR_INVALID_ARG;
  const int32_t L = resolve_band(p);
  const int32_t nqt = (n + bm - 1) / bm;
  const int32_t nkt = (n + bn - 1) / bn;
  const bool write = row_ptr != nullptr && col != nullptr;  // the whole plan
  const bool rows_only = row_ptr != nullptr && col == nullptr;  // row_ptr alone
  std::vector<int32_t> touch(nkt + 1), cover(nkt + 1);
  int64_t nnz = 0;
  if (write || rows_only) row_ptr[0] = 0;
  for (int32_t h = 0; h < h_kv_local; ++h) {
    const HeadPattern hp = head_pattern(p->sink, p->window, L,
                                        band_slot(p->kv_head_offset + h, resolve_n_bands(p)),
                                        p->mode == COWA_MODE_CAUSAL);
    for (int32_t qi = 0; qi < nqt; ++qi) {
      const int32_t r0 = qi * bm;
      const int32_t r1 = imin(r0 + bm, n);
      int32_t kmin = nkt, kmax = -1;
      for (int32_t t = r0; t < r1; ++t) {
        RowRanges rr = row_ranges(hp, t);
        // merge adjacent ranges (they are disjoint and ascending)
        int32_t mlo[3], mhi[3], m = 0;
        for (int i = 0; i < 3; ++i) {
          if (rr.hi[i] <= rr.lo[i]) continue;
          if (m > 0 && rr.lo[i] == mhi[m - 1]) {
            mhi[m - 1] = rr.hi[i];
          } else {
            mlo[m] = rr.lo[i];
            mhi[m] = rr.hi[i];
            ++m;
          }
        }
        for (int i = 0; i < m; ++i) {
          const int32_t a = mlo[i], b = mhi[i];
          const int32_t ta = a / bn, tb = (b - 1) / bn;  // touched tiles [ta, tb]
          touch[ta] += 1;
          touch[tb + 1] -= 1;
          kmin = imin(kmin, ta);
          kmax = imax(kmax, tb);
          const int32_t ca = (a + bn - 1) / bn, cb = b / bn;  // covered tiles [ca, cb)
          if (ca < cb) {
            cover[ca] += 1;
            cover[cb] -= 1;
          }
        }
      }
      const int32_t rows = r1 - r0;
      int32_t run_t = 0, run_c = 0;
      for (int32_t kj = kmin; kj <= kmax; ++kj) {
        run_t += touch[kj];
        run_c += cover[kj];
        touch[kj] = 0;
        cover[kj] = 0;
        if (run_t <= 0) continue;
        if (write) {
          if (nnz >= cap) return COWA_ERR_CAPACITY;
          col[nnz] = kj;
          flags[nnz] = (rows == bm && run_c == bm) ? 1 : 0;
        }
        ++nnz;
      }
      if (kmax >= 0) {
        touch[kmax + 1] = 0;
        cover[kmax + 1] = 0;
      }
      if (write || rows_only) {
        if (nnz > 0x7fffffff) return COWA_ERR_CAPACITY;
        row_ptr[(int64_t)h * nqt + qi + 1] = (int32_t)nnz;
      }
    }
  }
  if (nnz_out) *nnz_out = nnz;
  return COWA_OK;
}

// Key-major lists: the query-major plan transposed per head (counting sort
// over key tiles; query tiles stay ascending because they are visited in
// order).
cowa_status plan_kv_impl(const cowa_pattern* p, int32_t n, int32_t h_kv_local, int32_t bm,
                         int32_t bn, int32_t* row_ptr, int32_t* col, uint8_t* flags,
                         int64_t cap, int64_t* nnz_out) {
  int64_t nnz = 0;
  cowa_status st = plan_impl(p, n, h_kv_local, bm, bn, nullptr, nullptr, nullptr, 0, &nnz);
  if (st != COWA_OK) return st;
  if (nnz_out) *nnz_out = nnz;
  if (!row_ptr) return COWA_OK;
  if (nnz > cap) return COWA_ERR_CAPACITY;
  const int32_t nqt = (n + bm - 1) / bm;
  const int32_t nkt = (n + bn - 1) / bn;
  std::vector<int32_t> qrp((size_t)h_kv_local * nqt + 1), qcol(nnz > 0 ? nnz : 1);
  std::vector<uint8_t> qfl(nnz > 0 ? nnz : 1);
  st = plan_impl(p, n, h_kv_local, bm, bn, qrp.data(), qcol.data(), qfl.data(), nnz, nullptr);
  if (st != COWA_OK) return st;
  std::vector<int64_t> fill(nkt);
  row_ptr[0] = 0;
  int64_t base = 0;
  for (int32_t h = 0; h < h_kv_local; ++h) {
    std::vector<int64_t> cnt(nkt, 0);
    for (int64_t e = qrp[(size_t)h * nqt]; e < qrp[(size_t)(h + 1) * nqt]; ++e) ++cnt[qcol[e]];
    for (int32_t kj = 0; kj < nkt; ++kj) {
      fill[kj] = base;
      base += cnt[kj];
      row_ptr[(int64_t)h * nkt + kj + 1] = (int32_t)base;
    }
    for (int32_t qi = 0; qi < nqt; ++qi) {
      const int64_t r = (int64_t)h * nqt + qi;
      for (int64_t e = qrp[r]; e < qrp[r + 1]; ++e) {
        const int64_t pos = fill[qcol[e]]++;
        col[pos] = qi;
        flags[pos] = qfl[e];
      }
    }
  }
  return COWA_OK;
}

}  // namespace cowa

extern "C" cowa_status cowa_plan_kv_size(const cowa_pattern* p, int32_t n, int32_t h_kv_local,
                                         int32_t block_m, int32_t block_n, int64_t* nnz_out) {
  if (!p || !nnz_out) return COWA_ERR_INVALID_ARG;
  return cowa::plan_kv_impl(p, n, h_kv_local, block_m, block_n, nullptr, nullptr, nullptr, 0,
                            nnz_out);
}

extern "C" cowa_status cowa_plan_kv(const cowa_pattern* p, int32_t n, int32_t h_kv_local,
                                    int32_t block_m, int32_t block_n, int32_t* row_ptr,
                                    int32_t* col, uint8_t* flags, int64_t cap) {
  if (!p || !row_ptr || (cap > 0 && (!col || !flags)) || cap < 0) return COWA_ERR_INVALID_ARG;
  int64_t nnz = 0;
  return cowa::plan_kv_impl(p, n, h_kv_local, block_m, block_n, row_ptr, col, flags, cap, &nnz);
}

extern "C" cowa_status cowa_plan_size(const cowa_pattern* p, int32_t n, int32_t h_kv_local,
                                      int32_t block_m, int32_t block_n, int64_t* nnz_out) {
  if (!p || !nnz_out) return COWA_ERR_INVALID_ARG;
  return cowa::plan_impl(p, n, h_kv_local, block_m, block_n, nullptr, nullptr, nullptr, 0,
                         nnz_out);
}

extern "C" cowa_status cowa_plan(const cowa_pattern* p, int32_t n, int32_t h_kv_local,
                                 int32_t block_m, int32_t block_n, int32_t* row_ptr,
                                 int32_t* col, uint8_t* flags, int64_t cap) {
  if (!p || !row_ptr || (cap > 0 && (!col || !flags)) || cap < 0) return COWA_ERR_INVALID_ARG;
  int64_t nnz = 0;
  return cowa::plan_impl(p, n, h_kv_local, block_m, block_n, row_ptr, col, flags, cap, &nnz);
}
